"""CPU oracle for the flash-attention backward operator FLASH_ATTN_BACK.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link this
module: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
It shares no code with the HIP implementation.

What it computes is the plain definition, in float64, materialising the score matrix
one head at a time. Sources (page "CambrianTech/llama.cpp PR #63", first review):
  - "The math in fattn_back_q": online-softmax lse; delta = sum_j p_j (dO . v_j), which is
    rowsum(dO o O) without forming O; dQ = scale * sum_j p_j (dp_j - delta) k_j.
  - "The math in fattn_back_kv": dK_j = scale * sum over (h in group, i) of
    p (dp - delta_i) q_i; dV_j = sum p dO_i.
  - "Layout and shape": d (dO) is indexed [Dv, H, N]; mask index [M, N, h % Hm] with
    Hm in {1, H}; GQA head map hk = h / (H / Hkv); the packed delta follows lse by N*H.
  - "Masking and q8_0": a fully masked row gives lse = -inf, so dQ and delta are 0 and the
    kv side skips it; q8_0 values are read block-wise (one fp16 scale per 32 int8).
  - Second review (the a0ea747 review, "Verified" list): output index (h*N+i)*D for dQ and (hk*M+j)*D for dK/dV;
    dS = p * (dp - delta) by direct subtraction.
Readings where the pages are silent or ambiguous:
  - s_ij = scale * q_i . k_j + mask_ij (additive mask after scaling, slope 1).
  - LSE/delta row index is h*N + i; the oracle returns them as (H, N) arrays.
  - dV carries no `scale`; dQ and dK do.
  - scale enters as float64(float32(scale)), as the operator's parameter is a float.
  - a row is fully masked iff every one of its M mask entries is -inf.
  - q8_0 block = fp16 scale (little-endian) then 32 int8; value = float64(scale) * q.
  - q4_0 (the served cache's type on the "torad-labs/llama.cpp PR #71" page; the pages do not
    spell out its block): the ggml block, fp16 scale then 16 bytes, byte t holding element t
    in its low nibble and element t + 16 in its high one; value = float64(scale) * (nibble - 8).
  - q4_1, q5_0, q5_1 (ggml block types that the pages do not name; their blocks are read as
    ggml lays them out, with every field little-endian):
    q4_1 = fp16 scale d, fp16 minimum m, 16 bytes of nibbles as in q4_0; value = d * n + m.
    q5_0 = fp16 d, a 32-bit word h, 16 bytes of nibbles; element t's code is its nibble plus 16
    times bit t of h, value = d * (code - 16). q5_1 = fp16 d, fp16 m, the word h, 16 bytes;
    value = d * code + m. (float64 throughout: every value is exact.)
Every function here is pinned by tests/test_oracle_*.py (finite differences, a hand-worked
example, closed forms, invariants and an independent pure-Python loop implementation).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ----------------------------------------------------------------------------- decoding

def widen(x: np.ndarray, typ: str, width: int | None = None) -> np.ndarray:
    """Exact float64 values of a stored tensor.

    f32/f16: the stored numbers. bf16: uint16 bit patterns placed in the top half of a
    float32. q8_0: rows of `width` values stored as width/32 blocks of 34 bytes, each the
    fp16 scale (little-endian) followed by 32 int8; value = scale * int8."""
    if typ == "f32" or typ == "f16":
        return np.asarray(x, dtype=np.float64)
    if typ == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if typ == "q8_0":
        raw = np.asarray(x, dtype=np.uint8)
        nblk = raw.shape[-1] // 34
        if width is not None and nblk * 32 != width:
            raise ValueError("q8_0 row width mismatch")
        blocks = np.ascontiguousarray(raw).reshape(*raw.shape[:-1], nblk, 34)
        step = np.ascontiguousarray(blocks[..., 0:2]).view(np.float16)[..., 0].astype(np.float64)
        qv = np.ascontiguousarray(blocks[..., 2:34]).view(np.int8).astype(np.float64)
        return (step[..., None] * qv).reshape(*raw.shape[:-1], nblk * 32)
    if typ == "q4_0":
        # 18-byte blocks: fp16 scale, then 16 bytes; byte t holds element t (low nibble) and
        # element t + 16 (high nibble); value = scale * (nibble - 8)
        raw = np.asarray(x, dtype=np.uint8)
        nblk = raw.shape[-1] // 18
        if width is not None and nblk * 32 != width:
            raise ValueError("q4_0 row width mismatch")
        blocks = np.ascontiguousarray(raw).reshape(*raw.shape[:-1], nblk, 18)
        step = np.ascontiguousarray(blocks[..., 0:2]).view(np.float16)[..., 0].astype(np.float64)
        qs = blocks[..., 2:18].astype(np.int64)
        nib = np.concatenate([qs & 15, qs >> 4], axis=-1).astype(np.float64) - 8.0
        return (step[..., None] * nib).reshape(*raw.shape[:-1], nblk * 32)
    if typ in ("q4_1", "q5_0", "q5_1"):
        # 20 / 22 / 24-byte blocks: fp16 d, [fp16 m], [32-bit word h], 16 bytes of nibbles,
        # byte t holding element t (low nibble) and element t + 16 (high nibble)
        nbytes = BLOCK_BYTES[typ]
        raw = np.asarray(x, dtype=np.uint8)
        nblk = raw.shape[-1] // nbytes
        if width is not None and nblk * 32 != width:
            raise ValueError(f"{typ} row width mismatch")
        blocks = np.ascontiguousarray(raw).reshape(*raw.shape[:-1], nblk, nbytes)
        d = np.ascontiguousarray(blocks[..., 0:2]).view(np.float16)[..., 0].astype(np.float64)
        at = 2
        m = np.zeros_like(d)
        if typ != "q5_0":
            m = np.ascontiguousarray(blocks[..., 2:4]).view(np.float16)[..., 0].astype(np.float64)
            at = 4
        code = np.zeros((*blocks.shape[:-1], 32), dtype=np.int64)
        if typ != "q4_1":
            h = np.ascontiguousarray(blocks[..., at:at + 4]).view("<u4")[..., 0].astype(np.int64)
            code += ((h[..., None] >> np.arange(32)) & 1) << 4
            at += 4
        qs = blocks[..., at:at + 16].astype(np.int64)
        code += np.concatenate([qs & 15, qs >> 4], axis=-1)
        if typ == "q5_0":
            val = d[..., None] * (code.astype(np.float64) - 16.0)
        else:
            val = d[..., None] * code.astype(np.float64) + m[..., None]
        return val.reshape(*raw.shape[:-1], nblk * 32)
    raise ValueError(f"unknown type {typ}")


# bytes of one 32-value block of the ggml block types
BLOCK_BYTES = {"q8_0": 34, "q4_0": 18, "q4_1": 20, "q5_0": 22, "q5_1": 24}


def problem_arrays(p):
    """float64 (q, k, v, dO, mask) of a Problem-like object in the logical shapes
    q (H,N,D), k (Hkv,M,D), v (Hkv,M,Dv), dO (N,H,Dv), mask (Hm,N,M) or None."""
    q = widen(p.q, p.q_type)
    k = widen(p.k, p.k_type, p.D)
    v = widen(p.v, p.v_type, p.Dv)
    do = widen(p.d, p.d_type)
    mask = None if p.mask is None else np.asarray(p.mask, dtype=np.float64)
    return q, k, v, do, mask


def _scale64(scale: float) -> float:
    return float(np.float32(scale))


# ----------------------------------------------------------------------------- full oracle

def flash_attn_back(q, k, v, do, mask, scale):
    """Backward of single-sequence attention, float64, plain definition.

    q (H,N,D), k (Hkv,M,D), v (Hkv,M,Dv), do (N,H,Dv), mask (Hm,N,M) or None; all float64.
    Returns dict(dq (H,N,D), dk (Hkv,M,D), dv (Hkv,M,Dv), lse (H,N), delta (H,N))."""
    H, N, D = q.shape
    Hkv, M, _ = k.shape
    Dv = v.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    Hm = 0 if mask is None else mask.shape[0]
    if mask is not None and Hm not in (1, H):
        raise ValueError("mask heads must be 1 or H")
    sc = _scale64(scale)
    dq = np.zeros((H, N, D))
    dk = np.zeros((Hkv, M, D))
    dv = np.zeros((Hkv, M, Dv))
    lse = np.zeros((H, N))
    delta = np.zeros((H, N))
    for h in range(H):
        hk = h // G
        Kh, Vh = k[hk], v[hk]
        dOh = do[:, h, :]                          # (N, Dv): dO indexed [Dv, H, N]
        S = sc * (q[h] @ Kh.T)                     # (N, M)
        if mask is not None:
            S = S + mask[h % Hm]
        m = S.max(axis=1, initial=NEG_INF)         # a row with no keys counts as masked
        dead = ~np.isfinite(m)                     # every entry of the row is -inf
        m_safe = np.where(dead, 0.0, m)
        ssum = np.exp(S - m_safe[:, None]).sum(axis=1)
        with np.errstate(divide="ignore"):
            L = np.where(dead, NEG_INF, m_safe + np.log(np.where(dead, 1.0, ssum)))
        P = np.where(dead[:, None], 0.0, np.exp(S - np.where(dead, 0.0, L)[:, None]))
        dP = dOh @ Vh.T                            # (N, M)
        dl = (P * dP).sum(axis=1)
        dS = P * (dP - dl[:, None])
        dq[h] = sc * (dS @ Kh)
        dk[hk] += sc * (dS.T @ q[h])
        dv[hk] += P.T @ dOh
        lse[h] = L
        delta[h] = dl
    return {"dq": dq, "dk": dk, "dv": dv, "lse": lse, "delta": delta}


def run_problem(p):
    """Oracle outputs for a Problem-like object (see fa_inputs.Problem)."""
    q, k, v, do, mask = problem_arrays(p)
    return flash_attn_back(q, k, v, do, mask, p.scale)


def forward_outputs(q, k, v, mask, scale):
    """What a forward pass saves: per head, S = scale q k^T + mask, lse = log sum_j exp(s_ij)
    and O = softmax(S) V (the attention output whose rowsum(dO o O) is delta, first review,
    "The math in fattn_back_q"). A fully masked row has lse = -inf and O = 0. float64,
    plain definition. Returns (lse (H,N), o (H,N,Dv))."""
    H, N, _ = q.shape
    Hkv, M, _ = k.shape
    G = H // Hkv
    Hm = 0 if mask is None else mask.shape[0]
    sc = _scale64(scale)
    lse = np.zeros((H, N))
    o = np.zeros((H, N, v.shape[2]))
    for h in range(H):
        S = sc * (q[h] @ k[h // G].T)
        if mask is not None:
            S = S + mask[h % Hm]
        m = S.max(axis=1, initial=NEG_INF)
        dead = ~np.isfinite(m)
        m_safe = np.where(dead, 0.0, m)
        E = np.where(dead[:, None], 0.0, np.exp(S - m_safe[:, None]))
        ssum = E.sum(axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            lse[h] = np.where(dead, NEG_INF, m_safe + np.log(np.where(dead, 1.0, ssum)))
            o[h] = np.where(dead[:, None], 0.0, (E @ v[h // G]) / np.where(dead, 1.0, ssum)[:, None])
    return lse, o


def forward_problem(p):
    """forward_outputs for a Problem-like object."""
    q, k, v, _, mask = problem_arrays(p)
    return forward_outputs(q, k, v, mask, p.scale)


# ----------------------------------------------------------------------------- sampled outputs

def _row_block(q, k, v, do, mask, sc, h, rows, G, Hm):
    """S, P, dP, lse, delta for rows `rows` (array of i) of head h, each row taken whole."""
    hk = h // G
    S = sc * (q[h, rows] @ k[hk].T)
    if mask is not None:
        S = S + mask[h % Hm][rows]
    m = S.max(axis=1, initial=NEG_INF)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    ssum = np.exp(S - m_safe[:, None]).sum(axis=1)
    with np.errstate(divide="ignore"):
        L = np.where(dead, NEG_INF, m_safe + np.log(np.where(dead, 1.0, ssum)))
    P = np.where(dead[:, None], 0.0, np.exp(S - np.where(dead, 0.0, L)[:, None]))
    dP = do[rows, h, :] @ v[hk].T
    dl = (P * dP).sum(axis=1)
    return S, P, dP, L, dl


def query_rows(q, k, v, do, mask, scale, picks):
    """dQ, lse and delta for selected query rows only. picks: list of (h, i).
    Returns arrays dq (n, D), lse (n,), delta (n,)."""
    H = q.shape[0]
    G = H // k.shape[0]
    Hm = 0 if mask is None else mask.shape[0]
    sc = _scale64(scale)
    out_dq, out_l, out_d = [], [], []
    for h, i in picks:
        hk = h // G
        _, P, dP, L, dl = _row_block(q, k, v, do, mask, sc, h, np.array([i]), G, Hm)
        dS = P * (dP - dl[:, None])
        out_dq.append((sc * (dS @ k[hk]))[0])
        out_l.append(L[0]); out_d.append(dl[0])
    return np.array(out_dq), np.array(out_l), np.array(out_d)


def key_rows(q, k, v, do, mask, scale, picks, chunk=256):
    """dK and dV for selected keys only. picks: list of (hk, j). Each needs every query
    row of the group, so every row's lse and delta is computed whole (per row, over all
    M keys) before the key columns are formed. Returns dk (n, D), dv (n, Dv)."""
    H, N, _ = q.shape
    Hkv = k.shape[0]
    G = H // Hkv
    Hm = 0 if mask is None else mask.shape[0]
    sc = _scale64(scale)
    by_hk = {}
    for idx, (hk, j) in enumerate(picks):
        by_hk.setdefault(hk, []).append((idx, j))
    dk_out = np.zeros((len(picks), k.shape[2]))
    dv_out = np.zeros((len(picks), v.shape[2]))
    for hk, lst in by_hk.items():
        js = np.array([j for _, j in lst])
        for h in range(hk * G, (hk + 1) * G):
            for r0 in range(0, N, chunk):
                rows = np.arange(r0, min(N, r0 + chunk))
                S, P, dP, L, dl = _row_block(q, k, v, do, mask, sc, h, rows, G, Hm)
                Pj = P[:, js]
                dSj = Pj * (dP[:, js] - dl[:, None])
                dk_part = sc * (dSj.T @ q[h, rows])
                dv_part = Pj.T @ do[rows, h, :]
                for t, (idx, _) in enumerate(lst):
                    dk_out[idx] += dk_part[t]
                    dv_out[idx] += dv_part[t]
    return dk_out, dv_out


# ----------------------------------------------------------------------------- loop oracle

def flash_attn_back_loops(q, k, v, do, mask, scale):
    """The same definition written as scalar Python loops with math.fsum; for tiny cases.
    Independent of the numpy version above (used to cross-check it)."""
    H, N, D = q.shape
    Hkv, M, _ = k.shape
    Dv = v.shape[2]
    G = H // Hkv
    Hm = 0 if mask is None else mask.shape[0]
    sc = _scale64(scale)
    dq = np.zeros((H, N, D)); dk = np.zeros((Hkv, M, D)); dv = np.zeros((Hkv, M, Dv))
    lse = np.zeros((H, N)); delta = np.zeros((H, N))
    for h in range(H):
        hk = h // G
        for i in range(N):
            s = []
            for j in range(M):
                val = sc * math.fsum(float(q[h, i, c]) * float(k[hk, j, c]) for c in range(D))
                if mask is not None:
                    val += float(mask[h % Hm, i, j])
                s.append(val)
            finite = [x for x in s if x != NEG_INF]
            if not finite:
                lse[h, i] = NEG_INF
                continue                          # p = 0: no dQ, no delta, no dK/dV
            mx = max(finite)
            L = mx + math.log(math.fsum(math.exp(x - mx) for x in finite))
            lse[h, i] = L
            p = [0.0 if x == NEG_INF else math.exp(x - L) for x in s]
            dp = [math.fsum(float(do[i, h, c]) * float(v[hk, j, c]) for c in range(Dv))
                  for j in range(M)]
            dl = math.fsum(p[j] * dp[j] for j in range(M))
            delta[h, i] = dl
            for j in range(M):
                ds = p[j] * (dp[j] - dl)
                for c in range(D):
                    dq[h, i, c] += sc * ds * float(k[hk, j, c])
                    dk[hk, j, c] += sc * ds * float(q[h, i, c])
                for c in range(Dv):
                    dv[hk, j, c] += p[j] * float(do[i, h, c])
    return {"dq": dq, "dk": dk, "dv": dv, "lse": lse, "delta": delta}


# ----------------------------------------------------------------------------- comparison

def nmse(x, ref) -> float:
    """sum (x - ref)^2 / sum ref^2 over entries where ref is finite. If sum ref^2 == 0 the
    result is 0 when x is also zero there, else inf."""
    x = np.asarray(x, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    fin = np.isfinite(ref)
    num = float(np.sum((x[fin] - ref[fin]) ** 2))
    den = float(np.sum(ref[fin] ** 2))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den
