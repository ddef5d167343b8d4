"""Helpers shared by the GPU tests: run a Problem through the C ABI, compare with the oracle."""
import dataclasses
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


def run_gpu(p, device="cuda:0", poison=True, fill=0xFF):
    """Run p through the C ABI; output and workspace are first filled with the byte `fill`
    (0xFF: NaN patterns, so that an unwritten defined byte shows up)."""
    import torch
    say(f"[gpu] {p.name}: D={p.D} H={p.H} Hkv={p.Hkv} N={p.N} M={p.M} "
        f"types q={p.q_type} k={p.k_type} v={p.v_type} d={p.d_type} mask={p.mask_type} "
        f"flags={getattr(p, 'flags', 0)}")
    dp = fab.DeviceProblem(p, device, poison=False)
    if poison:
        dp.out.fill_(fill)
        dp.ws.fill_(fill)
    dp.run()
    torch.cuda.synchronize()
    out = dp.outputs()
    raw = dp.out.cpu().numpy()
    lay = dp.layout
    dp.close()
    return out, raw, lay


# Local bounds, so that an error confined to a few rows or keys cannot hide in an output's
# pooled NMSE. Each row (a dQ row, a dK / dV key row, or one LSE / delta value) whose reference
# magnitude m (its norm) is at least LOCAL_FLOOR times the root mean square m_rms of all rows'
# magnitudes must have error norm <= tol * m; a smaller row must have error <= tol * LOCAL_FLOOR
# * m_rms. tol is LOCAL_TOL_VEC for vector rows and LOCAL_TOL_SCA for scalars. A row's fp16
# operand rounding gives it an error of a few 1e-4 of its terms; a wrong tile gives errors of
# order 1. A row whose gradient cancels (e.g. one that sees three keys, whose dS sums to 0) keeps
# an absolute error set by its terms, not by its result: hence the floor. A key row that one
# query row alone reaches (G * N = 1) is a single term dS_j q, and dS_j = P_j (dP_j - delta)
# cancels inside: with fp16 operands (emulated on the CPU) one such row of a D = 256 case comes
# to 1.2e-2 of the floored bound. So 2e-2, which still leaves a wrong tile 50 times over.
LOCAL_TOL_VEC, LOCAL_TOL_SCA, LOCAL_FLOOR = 2e-2, 5e-2, 1e-1
VECTOR_KEYS = ("dq", "dk", "dv")


def local_error(g, r, vector, floor=LOCAL_FLOOR):
    """Worst per-row error of g against r, in units of the bound: <= 1 passes. Non-finite
    reference entries are left out (their pattern is checked exactly elsewhere)."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if vector:
        g = g.reshape(-1, g.shape[-1])
        r = r.reshape(-1, r.shape[-1])
        fin = np.isfinite(r).all(axis=1)
        err = np.sqrt(((g[fin] - r[fin]) ** 2).sum(axis=1))
        mag = np.sqrt((r[fin] ** 2).sum(axis=1))
        tol = LOCAL_TOL_VEC
    else:
        g = g.ravel()
        r = r.ravel()
        fin = np.isfinite(r)
        err = np.abs(g[fin] - r[fin])
        mag = np.abs(r[fin])
        tol = LOCAL_TOL_SCA
    rms = math.sqrt(float(np.mean(mag ** 2))) if mag.size else 0.0
    if rms == 0.0:
        return 0.0 if not err.size or err.max() == 0.0 else math.inf
    bound = tol * np.maximum(mag, floor * rms)
    return float((err / bound).max())


def compare(got, ref, keys=KEYS, tol=TOL, local=True):
    """Per-output NMSE (finite entries), exact agreement of the non-finite pattern, and (local)
    the per-row bounds above."""
    errs = {}
    worst = {}
    for k in keys:
        g = np.asarray(got[k], dtype=np.float64)
        r = np.asarray(ref[k], dtype=np.float64)
        assert g.shape == r.shape, (k, g.shape, r.shape)
        fin = np.isfinite(r)
        assert np.array_equal(np.isfinite(g), fin), f"{k}: non-finite pattern differs"
        if (~fin).any():
            assert np.array_equal(g[~fin], r[~fin]), f"{k}: -inf entries differ"
        errs[k] = O.nmse(g[fin], r[fin])
        if local:
            worst[k] = local_error(g, r, k in VECTOR_KEYS)
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, f"NMSE above {tol}: {bad} (all: {errs})"
    if local:
        say("   local " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
        badl = {k: e for k, e in worst.items() if not e <= 1.0}
        assert not badl, f"per-row error above its bound (units of the bound): {badl}"
    return errs


def walk1(p, mode):
    """The same problem with the LSE/delta walk forced by its descriptor flag: 'rows', 'keys',
    'rows_image' (rows, with the cache decoded into the image: the row walk's own kernel, and dQ
    by walk 2), or 'rows_ds' (rows, with dQ from the dS the key side stores)."""
    F = fab.fa_back
    bit = {"keys": F.FLAG_WALK1_KEYS, "rows": F.FLAG_WALK1_ROWS,
           "rows_image": F.FLAG_WALK1_ROWS | F.FLAG_KV_IMAGE | F.FLAG_DS_RECOMPUTE,
           "rows_ds": F.FLAG_WALK1_ROWS | F.FLAG_DS_STORE}[mode]
    clear = F.FLAG_WALK1_KEYS | F.FLAG_WALK1_ROWS
    if mode in ("rows_image", "rows_ds"):
        clear |= F.FLAG_KV_IMAGE | F.FLAG_KV_INLINE | F.FLAG_DS_STORE | F.FLAG_DS_RECOMPUTE
    return dataclasses.replace(p, flags=(p.flags & ~clear) | bit)
