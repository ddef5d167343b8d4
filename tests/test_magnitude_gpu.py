"""dO rows of very different magnitudes in one call, on the GPU through the C ABI.

dS = P (dP - delta) goes to fp16 scaled by a power of two. With one exponent for the whole call,
the rows whose dO is 10^4 below the largest would put dS among fp16's subnormals and lose
precision without moving the pooled NMSE. Every magnitude class of rows must therefore meet the
bar on its own (dQ rows, LSE, delta), and a KV group whose every dO row is tiny must meet it on
its own dK and dV too."""
import numpy as np
import pytest

import fa_inputs
from oracle import fa_back_oracle as O
from tests.gpu_util import compare, run_gpu, say, walk1

pytestmark = pytest.mark.gpu

DECADES = [
    dict(name="dO_5_decades", D=128, H=8, Hkv=2, N=64, M=512, mask="none", k_type="q8_0",
         v_type="q8_0", d_decades=4),
    dict(name="dO_5_decades_d256_tail", D=256, H=6, Hkv=1, N=40, M=700, mask="tail",
         k_type="q8_0", v_type="q8_0", d_decades=4),
]


@pytest.mark.parametrize("mode", ["rows", "keys", "rows_ds"])
@pytest.mark.parametrize("cfg", DECADES, ids=[c["name"] for c in DECADES])
def test_every_magnitude_class(cfg, mode):
    p = walk1(fa_inputs.make_custom(**cfg), mode)
    got, _, _ = run_gpu(p)
    ref = O.run_problem(p)
    compare(got, ref)
    cls = fa_inputs.magnitude_class(p.N, p.H, cfg["d_decades"] + 1).T      # (H, N) like dq, lse
    for c in range(cfg["d_decades"] + 1):
        sel = cls == c
        sub = lambda o: {"dq": o["dq"][sel], "lse": o["lse"][sel], "delta": o["delta"][sel]}
        errs = compare(sub(got), sub(ref), keys=("dq", "lse", "delta"))
        say(f"   rows x 1e-{c}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("mode", ["rows", "keys", "rows_ds"])
def test_tiny_kv_group(mode):
    # every dO row of KV head 1's query heads is 1e-4 of the others: its dK and dV, and its rows'
    # dQ and delta, meet the bar on their own
    p = walk1(fa_inputs.make_custom(name="tiny_group", D=128, H=8, Hkv=2, N=64, M=512, mask="tail",
                                    k_type="q8_0", v_type="q8_0", d_group_mult=(1, 1e-4)), mode)
    got, _, _ = run_gpu(p)
    ref = O.run_problem(p)
    compare(got, ref)
    G = p.H // p.Hkv
    part = lambda o: {"dq": o["dq"][G:], "lse": o["lse"][G:], "delta": o["delta"][G:],
                      "dk": o["dk"][1:], "dv": o["dv"][1:]}
    errs = compare(part(got), part(ref))
    say("   tiny group: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
