"""Helpers shared by the GPU tests: run a Problem through the C ABI, compare with the oracle."""
import math
import sys

import numpy as np

import flash_attention_backward_amd as fab
from oracle import fa_back_oracle as O

KEYS = ("dq", "dk", "dv", "lse", "delta")
TOL = 1e-5   # NMSE per output


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(p, device="cuda:0", poison=True):
    import torch
    say(f"[gpu] {p.name}: D={p.D} H={p.H} Hkv={p.Hkv} N={p.N} M={p.M} "
        f"types q={p.q_type} k={p.k_type} v={p.v_type} d={p.d_type} mask={p.mask_type} "
        f"flags={getattr(p, 'flags', 0)}")
    dp = fab.DeviceProblem(p, device, poison=poison)
    dp.run()
    torch.cuda.synchronize()
    out = dp.outputs()
    raw = dp.out.cpu().numpy()
    lay = dp.layout
    dp.close()
    return out, raw, lay


def compare(got, ref, keys=KEYS, tol=TOL):
    """Per-output NMSE (finite entries) and exact agreement of the non-finite pattern."""
    errs = {}
    for k in keys:
        g = np.asarray(got[k], dtype=np.float64)
        r = np.asarray(ref[k], dtype=np.float64)
        assert g.shape == r.shape, (k, g.shape, r.shape)
        fin = np.isfinite(r)
        assert np.array_equal(np.isfinite(g), fin), f"{k}: non-finite pattern differs"
        if (~fin).any():
            assert np.array_equal(g[~fin], r[~fin]), f"{k}: -inf entries differ"
        errs[k] = O.nmse(g[fin], r[fin])
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, f"NMSE above {tol}: {bad} (all: {errs})"
    return errs
