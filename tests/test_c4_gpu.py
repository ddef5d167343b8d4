"""The long-cache causal-tail workload (N2048 / M75520, H24 / Hkv4, D256, q8_0 K/V) on the GPU.

The N=8 and N=16 pilots (last rows of the same draws, same cache) are checked against the
full oracle. The full N=2048 run, in the launch configuration the benchmark times, is checked
on sampled query rows (dQ, LSE, delta) and sampled keys (dK, dV), each computed whole by the
oracle. The q4_0 pilot (c4q4n16: the same draws with the cache encoded q4_0) is checked
against the full oracle too."""
import numpy as np
import pytest

import fa_inputs
from oracle import fa_back_oracle as O
from tests.gpu_util import compare, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c4n8", "c4n16", "c4q4n16"])
def test_pilots_full_oracle(name):
    p = fa_inputs.make(name)
    got, _, _ = run_gpu(p)
    say("   oracle ...")
    ref = O.run_problem(p)
    errs = compare(got, ref)
    say("   nmse " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_full_size_sampled():
    p = fa_inputs.make("c4")
    got, _, _ = run_gpu(p)
    rng = np.random.default_rng(123)
    rows = [(0, 0), (23, p.N - 1), (5, p.N // 2), (17, 1)]
    rows += [(int(h), int(i)) for h, i in zip(rng.integers(0, p.H, 28), rng.integers(0, p.N, 28))]
    hk = p.Hkv - 1
    keys = [(hk, 0), (hk, p.M - 1), (hk, p.M - p.N), (hk, p.M - p.N + 1), (hk, p.M // 2)]
    keys += [(hk, int(j)) for j in rng.integers(0, p.M, 11)]
    say("   oracle: sampled rows and keys ...")
    q, k, v, do, mask = O.problem_arrays(p)
    dq, lse, dl = O.query_rows(q, k, v, do, mask, p.scale, rows)
    dk, dv = O.key_rows(q, k, v, do, mask, p.scale, keys)
    ghs = {"dq": np.array([got["dq"][h, i] for h, i in rows]),
           "lse": np.array([got["lse"][h, i] for h, i in rows]),
           "delta": np.array([got["delta"][h, i] for h, i in rows]),
           "dk": np.array([got["dk"][a, j] for a, j in keys]),
           "dv": np.array([got["dv"][a, j] for a, j in keys])}
    errs = compare(ghs, {"dq": dq, "lse": lse, "delta": dl, "dk": dk, "dv": dv})
    say("   sampled nmse " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    # every output is finite (no row of this workload is fully masked) and dK/dV of the
    # last key, which only the last query row sees, is non-zero
    for key in ("dq", "dk", "dv", "lse", "delta"):
        assert np.isfinite(got[key]).all(), key
    assert np.abs(got["dv"][:, p.M - 1]).max() > 0
