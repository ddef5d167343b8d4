"""A seeded sweep of random problems against the float64 oracle, through the C ABI (GPU only).

Each case draws a head size (64, 128, 256), a GQA shape, ragged N and M (so tiles of every
kind end part-full), K and V types from all eight, a mask (none, stored causal-tail, stored
random with one or per-head mask rows, or the implicit causal tail) and one of the walk-1 /
cache-image plans, and must meet the parity bar of every fixed case (tests.gpu_util.compare).
A second set takes F32 / F16 / BF16 caches whose K or V values share a large common part,
centred by the descriptor flags, with dO rows spread over up to four decades.
Sizes are capped so that the oracle finishes each case in a few seconds."""
import numpy as np
import pytest

import fa_inputs
from flash_attention_backward_amd import fa_back as B
from oracle import fa_back_oracle as O
from tests.gpu_util import compare, run_gpu, say
from tests.test_saved_gpu import _run_saved

pytestmark = pytest.mark.gpu

KV_TYPES = ["f32", "f16", "bf16", "q8_0", "q4_0", "q4_1", "q5_0", "q5_1"]
# with the image the plan forms dQ from the key side's stored dS unless DS_RECOMPUTE says
# otherwise, so the image plans cover both dQ paths
PLANS = [0, B.FLAG_WALK1_ROWS, B.FLAG_WALK1_KEYS, B.FLAG_WALK1_ROWS | B.FLAG_KV_IMAGE,
         B.FLAG_WALK1_KEYS | B.FLAG_KV_IMAGE | B.FLAG_DS_RECOMPUTE, B.FLAG_WALK1_ROWS | B.FLAG_KV_INLINE,
         B.FLAG_WALK1_KEYS | B.FLAG_DS_STORE]


def _cases(n=96, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        D = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2, 4]))
        H = Hkv * int(rng.choice([1, 2, 3, 6]))
        N = int(rng.integers(1, 600))
        cap = max(1, int(6e8 // (H * D * N)))            # oracle work ~ N * M * H * D
        M = int(min(rng.integers(1, 5000), cap))
        mask = str(rng.choice(["none", "tail", "random", "implicit"]))
        Hm = int(rng.choice([1, H])) if mask == "random" else 1
        kt, vt = (str(x) for x in rng.choice(KV_TYPES, 2))
        out.append(dict(name=f"sweep{c}", D=D, H=H, Hkv=Hkv, N=N, M=M, Hm=Hm, k_type=kt, v_type=vt,
                        mask=mask, flags=int(PLANS[c % len(PLANS)]), seed=100 + c))
    return out


def _cases_centred(n=32, seed=77):
    """Row-type caches whose values share a large common part (near-constant K or V), centred by
    the descriptor flags, with dO rows over several decades of magnitude."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        D = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 3, 6]))
        N = int(rng.integers(1, 400))
        cap = max(1, int(4e8 // (H * D * N)))
        M = int(min(rng.integers(1, 3000), cap))
        kt, vt = (str(x) for x in rng.choice(["f32", "f16", "bf16"], 2))
        near_k, near_v = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        flags = (B.FLAG_CENTER_K if near_k else 0) | (B.FLAG_CENTER_V if near_v else 0)
        flags |= int(PLANS[c % len(PLANS)])
        out.append(dict(name=f"centred{c}", D=D, H=H, Hkv=Hkv, N=N, M=M, k_type=kt, v_type=vt,
                        mask=str(rng.choice(["none", "tail", "implicit"])), flags=flags, seed=300 + c,
                        k_offset=2.0 if near_k else 0.0, k_spread=0.02 if near_k else 1.0,
                        v_offset=1.5 if near_v else 0.0, v_spread=0.02 if near_v else 1.0,
                        d_decades=int(rng.integers(0, 4))))
    return out


CASES = _cases() + _cases_centred()


def _problem(cfg):
    cfg = dict(cfg)
    implicit = cfg["mask"] == "implicit"
    if implicit:
        cfg["mask"] = "tail"
    p = fa_inputs.make_custom(**cfg)
    return fa_inputs.implicit_causal(p) if implicit else p


@pytest.mark.parametrize("cfg", CASES, ids=[c["name"] for c in CASES])
def test_sweep_against_oracle(cfg):
    p = _problem(cfg)
    got, _, _ = run_gpu(p)
    ref = O.run_problem(p)
    errs = compare(got, ref)
    say("   nmse " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


# every fourth case of the first set through the saved-statistics entry (the forward's LSE and
# O from the oracle)
SAVED = CASES[:96:4]


@pytest.mark.parametrize("cfg", SAVED, ids=[c["name"] + "_saved" for c in SAVED])
def test_sweep_saved_entry(cfg):
    p = _problem(cfg)
    got = _run_saved(p)[0]
    ref = O.run_problem(p)
    errs = compare(got, ref)
    say("   nmse " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
