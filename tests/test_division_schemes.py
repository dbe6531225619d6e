"""CPU check of the division scheme the SwiGLU kernels use instead of the IEEE
fp32 division in SiLU (Markstein's theorem: with a reciprocal within half an
ulp and a quotient within one ulp, one exact-remainder FMA correction gives the
correctly rounded quotient).  The GPU kernels must return the same bits as the
oracle's plain division; this covers every bf16 gate on the fast path and each
reciprocal within 3 ulp that the hardware's approximate reciprocal may return,
so the claim does not depend on which one the GPU gives.
"""
import os
import subprocess


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_EXE = None


def _binary():
    global _EXE
    if _EXE is None:
        out = os.path.join(ROOT, "_build")
        os.makedirs(out, exist_ok=True)
        exe = os.path.join(out, "divschemes")
        subprocess.run(["gcc", "-O2", "-pthread", "-ffp-contract=off",
                        os.path.join(ROOT, "tests", "c", "divschemes.c"), "-o", exe, "-ldl",
                        "-lm"], check=True)
        _EXE = exe
    return _EXE


def _run(mode):
    from oracle import build as ob
    nth = str(min(16, os.cpu_count() or 1))
    r = subprocess.run([_binary(), ob.LIB, mode, nth], check=True, capture_output=True,
                       text=True)
    return dict(tok.split("=") for tok in r.stdout.split())


def test_silu_division_scheme_matches_ieee(orc):
    kv = _run("silu")
    assert int(kv["bad"]) == 0, kv
    assert int(kv["checked"]) >= 150000, kv
