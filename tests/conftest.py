"""Shared pytest configuration: the `gpu` marker and common helpers."""

import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def golden():
    return load_golden


def _ensure_built():
    lib = os.path.join(ROOT, "bit_moe_expert_topk_amd", "libmoedec.so")
    synth_lib = os.path.join(ROOT, "synth", "libmoedec_synth.so")
    if not (os.path.exists(lib) and os.path.exists(synth_lib)):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_moedec_build", os.path.join(ROOT, "bit_moe_expert_topk_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)          # loads no library
        mod.build()


_ensure_built()
