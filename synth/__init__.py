"""Seeded synthetic inputs for the MoE-decode and LM-head paths.

This package is the only code that both the HIP path's tests/benchmarks and
the CPU oracle consume.  It holds no arithmetic of the method: it draws bytes
and Gaussian samples and lays them out in the canonical formats.

Two generators are used:

* Counter-based SplitMix64 for every MXFP4 byte (E2M1 code bytes and E8M0
  scale bytes).  Output n of a stream with state s is
      mix(s + (n + 1) * 0x9E3779B97F4A7C15)
  with mix the SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014; constants as in Vigna's
  public-domain splitmix64.c).  Being counter-based, any byte of any expert of
  any layer can be regenerated alone on the host, which is how the oracle
  gets the few active experts of a layer that the device generated in full.
  The device twin (synth/fill.hip) implements the same published definition.
* numpy PCG64 (SeedSequence([seed, stream])) for Gaussian tensors: activations,
  router logits, LM-head weights.  Values are drawn in float64 (float32 for the
  400M-element LM head), scaled, and rounded to bf16 by torch's RNE cast or
  kept as float32.

Stream identifiers keep every tensor independent (the sampling draws of
decode step t use stream 2^40 + t of the SplitMix64 generator):
  MXFP4 tensor (layer, expert, matrix, part):
      ((layer * 1025 + expert) * 3 + matrix) * 2 + part
  matrix 0 = gate, 1 = up, 2 = down; part 0 = codes, 1 = scales;
  expert 0..E-1 routed, E = the shared expert (E <= 1024).
"""

from dataclasses import dataclass, field

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2
PART_CODES, PART_SCALES = 0, 1


def mix64(z):
    """SplitMix64 finaliser on uint64 arrays (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix_outputs(state, idx):
    """Outputs number idx (0-based) of the SplitMix64 stream with state `state`."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(state) + (idx + np.uint64(1)) * GOLDEN)


def stream_state(seed, stream_id):
    """State of stream `stream_id`: output number stream_id of the seed's stream."""
    return int(splitmix_outputs(np.uint64(seed), np.uint64(stream_id)))


def mxfp4_stream_id(layer, expert, matrix, part):
    assert 0 <= expert <= 1024 and matrix in (0, 1, 2) and part in (0, 1)
    return ((layer * 1025 + expert) * 3 + matrix) * 2 + part


def hash_bytes(state, n_bytes, start=0):
    """Bytes start..start+n_bytes-1 of a stream: byte b is byte (b % 8),
    little-endian, of output b // 8."""
    first = start // 8
    last = (start + n_bytes + 7) // 8
    words = splitmix_outputs(state, np.arange(first, last, dtype=np.uint64))
    raw = words.astype("<u8").view(np.uint8)
    off = start - first * 8
    return raw[off:off + n_bytes].copy()


def hash_scale_codes(state, n, lo, hi, start=0):
    """Scale bytes start..start+n-1: lo + (output i) mod (hi - lo + 1)."""
    span = np.uint64(hi - lo + 1)
    words = splitmix_outputs(state, np.arange(start, start + n, dtype=np.uint64))
    return (np.uint64(lo) + words % span).astype(np.uint8)


@dataclass(frozen=True)
class MoEShape:
    H: int
    I: int
    E: int
    k: int
    scale_lo: int          # E8M0 code range (inclusive)
    scale_hi: int


def mxfp4_matrix(seed, layer, expert, matrix, n_rows, n_cols, scale_lo, scale_hi):
    """Canonical MXFP4 matrix (codes uint8 [N][K/2], scales uint8 [N][K/32])."""
    sc = stream_state(seed, mxfp4_stream_id(layer, expert, matrix, PART_CODES))
    ss = stream_state(seed, mxfp4_stream_id(layer, expert, matrix, PART_SCALES))
    codes = hash_bytes(sc, n_rows * n_cols // 2).reshape(n_rows, n_cols // 2)
    scales = hash_scale_codes(ss, n_rows * n_cols // 32, scale_lo, scale_hi)
    return codes, scales.reshape(n_rows, n_cols // 32)


def mxfp4_expert(seed, layer, expert, shape):
    """Canonical gate [I][H], up [I][H], down [H][I] MXFP4 matrices of one
    expert (expert == shape.E is the shared expert)."""
    H, I = shape.H, shape.I
    lo, hi = shape.scale_lo, shape.scale_hi
    return {
        "gate": mxfp4_matrix(seed, layer, expert, MAT_GATE, I, H, lo, hi),
        "up": mxfp4_matrix(seed, layer, expert, MAT_UP, I, H, lo, hi),
        "down": mxfp4_matrix(seed, layer, expert, MAT_DOWN, H, I, lo, hi),
    }


def mxfp4_layer(seed, layer, shape):
    """All E routed experts plus the shared expert of one layer, stacked:
    gate/up codes [E+1][I][H/2], scales [E+1][I][H/32]; down codes
    [E+1][H][I/2], scales [E+1][H][I/32].  Host generation; meant for small
    shapes (the device twin fills full Ling-sized layers)."""
    out = {name: ([], []) for name in ("gate", "up", "down")}
    for e in range(shape.E + 1):
        ex = mxfp4_expert(seed, layer, e, shape)
        for name in out:
            out[name][0].append(ex[name][0])
            out[name][1].append(ex[name][1])
    return {name: (np.stack(c), np.stack(s)) for name, (c, s) in out.items()}


def _rng(seed, stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


# Stream numbers for Gaussian tensors.
GAUSS_X, GAUSS_LOGITS, GAUSS_ROUTER, GAUSS_LMHEAD_W, GAUSS_LMHEAD_X = 1, 2, 3, 4, 5
GAUSS_ROUTER_W = 6
GAUSS_SHARED_W = 7


def bf16_bits_from_f32(v):
    """uint16 bf16 patterns of float32 values by torch's RNE cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits):
    """float32 values of uint16 bf16 patterns (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def activations_bf16(seed, layer, m_tokens, hidden, std=1.0):
    """bf16 activations ~ N(0, std^2), as uint16 bit patterns [M][H]."""
    g = _rng(seed, GAUSS_X * 1000 + layer).standard_normal((m_tokens, hidden))
    return bf16_bits_from_f32((g * std).astype(np.float32))


def logits_f32(seed, layer, m_tokens, n_experts):
    """float32 router logits ~ N(0, 1), independent per token [M][E]."""
    g = _rng(seed, GAUSS_LOGITS * 1000 + layer).standard_normal((m_tokens, n_experts))
    return g.astype(np.float32)


def router_logits_f32(seed, x_bits, n_experts):
    """Logits fl32(x . W_r) from a seeded router matrix W_r [H][E] ~ N(0, 1/H).
    The product is taken once here, in float64, and rounded to float32; both
    sides consume the same float32 logits."""
    x = bf16_values(x_bits).astype(np.float64)
    hidden = x.shape[1]
    wr = _rng(seed, GAUSS_ROUTER).standard_normal((hidden, n_experts)) / np.sqrt(hidden)
    return (x @ wr).astype(np.float32)


def router_weight_bf16(seed, layer, n_experts, hidden):
    """bf16 router matrix W_router [E][H] ~ N(0, 1/H) (uint16 patterns), so
    that with N(0,1) activations the logits are about N(0,1)."""
    g = _rng(seed, GAUSS_ROUTER_W * 1000 + layer).standard_normal((n_experts, hidden), dtype=np.float32)
    return bf16_bits_from_f32(g * np.float32(1.0 / np.sqrt(hidden)))


def shared_expert_bf16(seed, layer, hidden, inter):
    """bf16 source weights of a shared expert stored in FP8 (uint16 patterns):
    W_gate, W_up [inter][hidden] ~ N(0, 1/hidden) and W_down [hidden][inter]
    ~ N(0, 1/inter), so that with N(0,1) activations g, u and y are about
    N(0,1)."""
    rng = _rng(seed, GAUSS_SHARED_W * 1000 + layer)
    g = rng.standard_normal((inter, hidden), dtype=np.float32) * np.float32(1.0 / np.sqrt(hidden))
    u = rng.standard_normal((inter, hidden), dtype=np.float32) * np.float32(1.0 / np.sqrt(hidden))
    d = rng.standard_normal((hidden, inter), dtype=np.float32) * np.float32(1.0 / np.sqrt(inter))
    return bf16_bits_from_f32(g), bf16_bits_from_f32(u), bf16_bits_from_f32(d)


def lmhead_weight_bf16(seed, vocab, hidden, std=0.02, row_start=0, n_rows=None):
    """LM-head weights ~ N(0, std^2) as bf16 patterns [V][H] (rows
    row_start..row_start+n_rows-1; the full matrix is drawn in one pass so that
    a row block is the same slice whatever block is asked for)."""
    n_rows = vocab - row_start if n_rows is None else n_rows
    rng = _rng(seed, GAUSS_LMHEAD_W)
    out = np.empty((n_rows, hidden), dtype=np.uint16)
    chunk = 8192
    for r0 in range(0, vocab, chunk):
        r1 = min(vocab, r0 + chunk)
        g = rng.standard_normal((r1 - r0, hidden), dtype=np.float32)
        lo, hi = max(r0, row_start), min(r1, row_start + n_rows)
        if lo < hi:
            out[lo - row_start:hi - row_start] = bf16_bits_from_f32(g[lo - r0:hi - r0] * np.float32(std))
        if r1 >= row_start + n_rows:
            break
    return out


SAMPLING_STREAM_BASE = 1 << 40


def sampling_uniforms(seed, step, m_tokens):
    """float32 [m_tokens] uniforms in [0, 1) for the draw of decode step `step`:
    output m of SplitMix64 stream SAMPLING_STREAM_BASE + step, top 24 bits
    divided by 2^24 (exact in float32, never 1.0)."""
    state = stream_state(seed, SAMPLING_STREAM_BASE + step)
    words = splitmix_outputs(state, np.arange(m_tokens, dtype=np.uint64))
    return ((words >> np.uint64(40)).astype(np.float64) / float(1 << 24)).astype(np.float32)


def lmhead_x_bf16(seed, m_tokens, hidden):
    g = _rng(seed, GAUSS_LMHEAD_X).standard_normal((m_tokens, hidden))
    return bf16_bits_from_f32(g.astype(np.float32))


# ----------------------------------------------------------------------------
# Workloads.  Shapes follow the pages (hidden 2,560, 512 routed experts top-8
# plus one shared, expert intermediate 768, vocabulary 157,184, 42 layers,
# a 4-token verify window); value distributions are those stated per workload.

TINY = MoEShape(H=256, I=64, E=16, k=2, scale_lo=127 - 8, scale_hi=127 - 4)
LING = MoEShape(H=2560, I=768, E=512, k=8, scale_lo=127 - 10, scale_hi=127 - 6)
LMHEAD_V, LMHEAD_H = 157184, 2560
STACK_LAYERS = 42


@dataclass(frozen=True)
class Workload:
    name: str
    shape: MoEShape
    M: int
    seed: int = 0
    router_matrix: bool = False    # logits from x . W_r instead of N(0,1)
    notes: str = field(default="")


WORKLOADS = {
    "tiny_m1": Workload("tiny_m1", TINY, 1, router_matrix=True,
                        notes="hidden 256, 16 experts top-2 + shared, I 64, M 1"),
    "ling_m1": Workload("ling_m1", LING, 1,
                        notes="Ling-shaped layer, M 1"),
    "ling_m4": Workload("ling_m4", LING, 4,
                        notes="Ling-shaped layer, 4-token verify window"),
}


def moe_inputs(wl, layer=0):
    """(x bits [M][H], logits float32 [M][E]) of a workload."""
    x = activations_bf16(wl.seed, layer, wl.M, wl.shape.H)
    if wl.router_matrix:
        lg = router_logits_f32(wl.seed, x, wl.shape.E)
    else:
        lg = logits_f32(wl.seed, layer, wl.M, wl.shape.E)
    return x, lg
