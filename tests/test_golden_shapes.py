"""The workload shapes against the sizes the pages print."""

import synth


def test_ling_shape_matches_pages(golden):
    fx = golden("ling_shapes.json")
    s = synth.LING
    assert s.H == fx["hidden"]["value"] and s.I == fx["moe_intermediate"]["value"]
    assert s.E == fx["routed_experts"]["value"] and s.k == fx["top_k"]["value"]
    assert synth.LMHEAD_V == fx["vocab"]["value"] and synth.LMHEAD_H == fx["hidden"]["value"]
    assert synth.STACK_LAYERS == fx["layers"]["value"]


def test_parameter_count_identities(golden):
    fx = golden("ling_shapes.json")
    s = synth.LING
    per_layer = (s.E + 1) * 3 * s.I * s.H
    raw = synth.STACK_LAYERS * per_layer
    assert abs(raw / fx["total_params_raw"]["value"] - 1) < 0.002          # 127.08B vs ~127B
    assert abs((synth.STACK_LAYERS - 1) * per_layer / fx["total_params_nominal"]["value"] - 1) < 0.001
    cap16, cap8, cap4 = fx["capacity_gb_16_8_4bit"]["value"]
    nominal = fx["total_params_nominal"]["value"]
    assert (nominal * 2 / 1e9, nominal / 1e9, nominal * 0.5 / 1e9) == (cap16, cap8, cap4)


def test_verify_window_expert_bound(golden):
    fx = golden("ling_shapes.json")
    assert fx["verify_window"]["value"] * synth.LING.k == fx["max_experts_per_verify"]["value"]


def test_lmhead_fp8_halves_the_read():
    bf16_bytes = synth.LMHEAD_V * synth.LMHEAD_H * 2
    fp8_bytes = synth.LMHEAD_V * synth.LMHEAD_H * 1
    assert bf16_bytes == 804_782_080 and fp8_bytes * 2 == bf16_bytes
