"""Build libmoedec.so (and the synthetic-input helper library) for gfx950.

Sources are compiled one object per file, in parallel, with hipcc, then linked
into shared libraries placed next to the Python code that loads them:
  bit_moe_expert_topk_amd/libmoedec.so   from bit_moe_expert_topk_amd/csrc
  synth/libmoedec_synth.so               from synth/fill.hip
Objects go to _build/ at the repository root.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-float32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

LIB = os.path.join(PKG, "libmoedec.so")
SYNTH_LIB = os.path.join(ROOT, "synth", "libmoedec_synth.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def _compile_all(sources, includes, out_dir, verbose):
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        for src in sources:
            obj = os.path.join(out_dir, os.path.basename(src) + ".o")
            objs.append(obj)
            cmd = [HIPCC] + COMMON + [f"-I{d}" for d in includes] + ["-c", src, "-o", obj]
            jobs.append(ex.submit(_run, cmd, verbose))
        for j in jobs:
            j.result()
    return objs


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, out)


def build(verbose=False):
    csrc = os.path.join(PKG, "csrc")
    sources = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".cpp")))
    objs = _compile_all(sources, [os.path.join(ROOT, "include"), csrc],
                        os.path.join(ROOT, "_build", "moedec"), verbose)
    _link(objs, LIB, verbose)
    sobjs = _compile_all([os.path.join(ROOT, "synth", "fill.hip")], [],
                         os.path.join(ROOT, "_build", "synth"), verbose)
    _link(sobjs, SYNTH_LIB, verbose)
    return LIB, SYNTH_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
