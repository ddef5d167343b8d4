"""Seeded synthetic inputs for the flash-attention backward operator (FLASH_ATTN_BACK).

This module is shared by the tests, the benchmark and the smoke check. It holds input
generation only: random draws, the q8_0 *encoding* of a drawn cache, bf16 rounding of
drawn values, mask construction and the storage layout of each tensor. It holds none of
the operator's arithmetic (no scores, softmax, gradients, q8_0 decoding), so the oracle
and the HIP path cannot share anything through it.

Tensor layouts follow the operator's ggml ne-order (innermost index first), see
"CambrianTech/llama.cpp PR #63", first review (layout and shape paragraph):
  q    [D,  N, H  ]  -> numpy (H,   N, D)
  k    [D,  M, Hkv]  -> numpy (Hkv, M, D)      (q8_0: (Hkv, M, D/32*34) uint8)
  v    [Dv, M, Hkv]  -> numpy (Hkv, M, Dv)
  d=dO [Dv, H, N  ]  -> numpy (N,   H, Dv)     (note the (H, N) order differs from q)
  mask [M,  N, Hm ]  -> numpy (Hm,  N, M)      Hm in {1, H}

Element types: 'f32' (np.float32), 'f16' (np.float16), 'bf16' (np.uint16 bit patterns),
'q8_0' (np.uint8 blocks: fp16 scale little-endian, then 32 int8 values).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

QK8_0 = 32                 # values per q8_0 block
Q8_0_BLOCK_BYTES = 34      # 2-byte fp16 scale + 32 int8


def q8_0_row_bytes(d: int) -> int:
    assert d % QK8_0 == 0
    return d // QK8_0 * Q8_0_BLOCK_BYTES


@dataclasses.dataclass
class Problem:
    """One operator invocation. Arrays are numpy, in the logical shapes listed above.

    `k` and `v` may be non-contiguous views (e.g. heads interleaved per cache cell);
    byte strides are taken from the numpy strides."""
    name: str
    D: int
    Dv: int
    H: int
    Hkv: int
    N: int
    M: int
    scale: float
    q: np.ndarray
    q_type: str
    k: np.ndarray
    k_type: str
    v: np.ndarray
    v_type: str
    d: np.ndarray
    d_type: str
    mask: Optional[np.ndarray] = None
    mask_type: str = "none"
    seed: int = 0
    note: str = ""
    flags: int = 0          # descriptor flags (1: centre V before its fp16 rounding)

    @property
    def Hm(self) -> int:
        return 0 if self.mask is None else self.mask.shape[0]

    @property
    def G(self) -> int:
        return self.H // self.Hkv


# ----------------------------------------------------------------------------- encoders

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def encode_q8_0(x: np.ndarray) -> np.ndarray:
    """Encode float32 rows (last axis = D, D % 32 == 0) as q8_0 blocks.

    Per block of 32: amax = max|x|, step = amax/127 (float32), q = x/step rounded half
    away from zero and clamped to [-127, 127] (0 for an all-zero block), stored step =
    fp16(step) round-to-nearest-even. Returns uint8 (..., D/32*34)."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    blk = x.reshape(*x.shape[:-1], D // QK8_0, QK8_0)
    amax = np.abs(blk).max(axis=-1, keepdims=True)
    step = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(step > 0, step, np.float32(1.0))
    t = np.where(step > 0, blk / safe, np.float32(0.0)).astype(np.float32)
    qv = np.sign(t) * np.floor(np.abs(t) + np.float32(0.5))
    qv = np.clip(qv, -127, 127).astype(np.int8)
    out = np.empty((*x.shape[:-1], D // QK8_0, Q8_0_BLOCK_BYTES), dtype=np.uint8)
    out[..., 0:2] = step.astype(np.float16).view(np.uint8).reshape(*step.shape[:-1], 2)
    out[..., 2:] = qv.view(np.uint8)
    return out.reshape(*x.shape[:-1], D // QK8_0 * Q8_0_BLOCK_BYTES)


Q4_0_BLOCK_BYTES = 18      # 2-byte fp16 scale + 16 bytes of 4-bit values


def encode_q4_0(x: np.ndarray) -> np.ndarray:
    """Encode float32 rows (last axis = D, D % 32 == 0) as q4_0 blocks.

    Per block of 32: m = the value of largest magnitude (with its sign), step = m / -8
    (float32), code = floor(x/step + 8.5) clamped to [0, 15] (8 for an all-zero block), stored
    step = fp16(step). Byte t of the 16 holds code t in its low nibble and code t + 16 in its
    high nibble. Returns uint8 (..., D/32*18)."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    blk = x.reshape(*x.shape[:-1], D // 32, 32)
    idx = np.abs(blk).argmax(axis=-1)[..., None]
    m = np.take_along_axis(blk, idx, axis=-1)
    step = (m / np.float32(-8.0)).astype(np.float32)
    safe = np.where(step != 0, step, np.float32(1.0))
    t = np.where(step != 0, blk / safe, np.float32(0.0)).astype(np.float32)
    code = np.clip(np.floor(t + np.float32(8.5)), 0, 15).astype(np.uint8)
    out = np.empty((*x.shape[:-1], D // 32, Q4_0_BLOCK_BYTES), dtype=np.uint8)
    out[..., 0:2] = step.astype(np.float16).view(np.uint8).reshape(*step.shape[:-1], 2)
    out[..., 2:] = code[..., :16] | (code[..., 16:] << 4)
    return out.reshape(*x.shape[:-1], D // 32 * Q4_0_BLOCK_BYTES)


def _pack_codes(code: np.ndarray) -> np.ndarray:
    """16 bytes per block: byte t holds code t (low nibble) and code t + 16 (high nibble)."""
    c = (code & 15).astype(np.uint8)
    return c[..., :16] | (c[..., 16:] << 4)


def _high_bits(code: np.ndarray) -> np.ndarray:
    """The 32-bit word whose bit t is bit 4 of code t, as 4 little-endian bytes."""
    h = np.zeros(code.shape[:-1], dtype=np.uint32)
    for t in range(32):
        h |= ((code[..., t].astype(np.uint32) >> 4) & 1) << t
    return h[..., None].view(np.uint8).reshape(*h.shape, 4)


def encode_min_step(x: np.ndarray, levels: int) -> tuple:
    """Per block of 32: the minimum m, step d = (max - m) / levels (float32) and codes
    round((x - m) / d) clamped to [0, levels] (0 for a constant block)."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    blk = x.reshape(*x.shape[:-1], D // 32, 32)
    mn = blk.min(axis=-1)
    d = ((blk.max(axis=-1) - mn) / np.float32(levels)).astype(np.float32)
    safe = np.where(d > 0, d, np.float32(1.0))
    code = np.where(d[..., None] > 0, np.floor((blk - mn[..., None]) / safe[..., None] + np.float32(0.5)), 0)
    return mn, d, np.clip(code, 0, levels).astype(np.int64)


def _f16_bytes(v: np.ndarray) -> np.ndarray:
    return v.astype(np.float16).view(np.uint8).reshape(*v.shape, 2)


def encode_q4_1(x: np.ndarray) -> np.ndarray:
    """q4_1 blocks (20 bytes): fp16 step d, fp16 minimum m, then the 16 bytes of 4-bit codes;
    d and codes from encode_min_step(x, 15). Returns uint8 (..., D/32*20)."""
    mn, d, code = encode_min_step(x, 15)
    out = np.concatenate([_f16_bytes(d), _f16_bytes(mn), _pack_codes(code)], axis=-1)
    return out.reshape(*out.shape[:-2], -1)


def encode_q5_1(x: np.ndarray) -> np.ndarray:
    """q5_1 blocks (24 bytes): fp16 d, fp16 m, the word of code bits 4, the 16 bytes of low
    nibbles; d and codes from encode_min_step(x, 31). Returns uint8 (..., D/32*24)."""
    mn, d, code = encode_min_step(x, 31)
    out = np.concatenate([_f16_bytes(d), _f16_bytes(mn), _high_bits(code), _pack_codes(code)], axis=-1)
    return out.reshape(*out.shape[:-2], -1)


def encode_q5_0(x: np.ndarray) -> np.ndarray:
    """q5_0 blocks (22 bytes): fp16 step d, the word of code bits 4, the 16 bytes of low
    nibbles. Per block: m = the value of largest magnitude (with its sign), d = m / -16 (float32),
    code = floor(x/d + 16.5) clamped to [0, 31] (16 for an all-zero block); value d*(code-16).
    Returns uint8 (..., D/32*22)."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    blk = x.reshape(*x.shape[:-1], D // 32, 32)
    idx = np.abs(blk).argmax(axis=-1)[..., None]
    m = np.take_along_axis(blk, idx, axis=-1)[..., 0]
    d = (m / np.float32(-16.0)).astype(np.float32)
    safe = np.where(d != 0, d, np.float32(1.0))
    t = np.where(d[..., None] != 0, blk / safe[..., None], np.float32(0.0)).astype(np.float32)
    code = np.clip(np.floor(t + np.float32(16.5)), 0, 31).astype(np.int64)
    out = np.concatenate([_f16_bytes(d), _high_bits(code), _pack_codes(code)], axis=-1)
    return out.reshape(*out.shape[:-2], -1)


def encode(x: np.ndarray, typ: str) -> np.ndarray:
    if typ == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if typ == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    if typ == "bf16":
        return to_bf16_bits(x)
    if typ == "q8_0":
        return encode_q8_0(x)
    if typ == "q4_0":
        return encode_q4_0(x)
    if typ == "q4_1":
        return encode_q4_1(x)
    if typ == "q5_0":
        return encode_q5_0(x)
    if typ == "q5_1":
        return encode_q5_1(x)
    raise ValueError(typ)


# ----------------------------------------------------------------------------- masks

def causal_tail_mask(N: int, M: int, Hm: int = 1, typ: str = "f16") -> np.ndarray:
    """Additive mask (Hm, N, M): query row i sees keys j <= M - N + i (0), others -inf."""
    j = np.arange(M)[None, :]
    i = np.arange(N)[:, None]
    dt = np.float16 if typ == "f16" else np.float32
    row = np.where(j <= M - N + i, 0.0, -np.inf).astype(dt)
    return np.broadcast_to(row, (Hm, N, M)).copy()


def implicit_causal(p: Problem) -> Problem:
    """The same problem with its one-head causal-tail mask passed as the storage-free mask type
    (the library forms it from i and j). The explicit array stays on the problem for the CPU
    oracle."""
    if p.mask is None or p.mask.shape[0] != 1 or not np.array_equal(
            np.asarray(p.mask, np.float32), causal_tail_mask(p.N, p.M, 1, "f32")):
        raise ValueError(f"{p.name}: the mask is not a one-head causal-tail mask")
    return dataclasses.replace(p, name=p.name + "_implicit", mask_type="causal_tail")


# ----------------------------------------------------------------------------- configs

def _draws(rng, H, Hkv, N, M, D, Dv):
    # draw order: K, V, Q, dO, each in its storage (ABI memory) order
    k = rng.standard_normal((Hkv, M, D), dtype=np.float32)
    v = rng.standard_normal((Hkv, M, Dv), dtype=np.float32)
    q = rng.standard_normal((H, N, D), dtype=np.float32)
    do = rng.standard_normal((N, H, Dv), dtype=np.float32)
    return k, v, q, do


def interleave_heads(x: np.ndarray) -> np.ndarray:
    """Store a (Hkv, M, row) cache with heads interleaved per cell, i.e. memory order
    (M, Hkv, row), and return the logical (Hkv, M, row) view of that storage."""
    store = np.ascontiguousarray(np.transpose(x, (1, 0, 2)))
    return np.transpose(store, (1, 0, 2))


def make(name: str, seed: int = 0, mask_type: str = "f16") -> Problem:
    """Build a named configuration.

    c0        D=Dv=64 H2 Hkv1 N16 M64, F32, causal-tail, head 1 row 0 fully masked (Hm=2)
    c1        D128 H8 Hkv2 N64 M512, Q/dO F32, K/V q8_0, no mask
    c2        c1 with M=8192;  c2b: K F16, V q8_0
    c3        N=M=1024 H32 Hkv8 D128, all bf16, causal;  c3v: V = 1 + 1e-3 z (bf16)
    c4        N2048 M75520 H24 Hkv4 D256, Q/dO F32, K/V q8_0, causal-tail
    c4n8/16   last 8 / 16 query rows of c4 against the same cache
    c4q4      c4 with K/V encoded q4_0 (same draws);  c4q4n16: its last 16 query rows
    Extra cases at the c1 shape: c1_tinydo (dO x 1e-6), c1_strided (K/V heads interleaved
    per cell), c1_causal (causal-tail mask), c1_f32kv, c1_f16kv, c1_bf16kv.
    Scaled-down shapes for quick parity: 'small_*'.
    """
    rng = np.random.default_rng(seed)
    mk = mask_type
    if name == "c0":
        D = Dv = 64; H, Hkv, N, M = 2, 1, 16, 64
        k, v, q, do = _draws(rng, H, Hkv, N, M, D, Dv)
        mask = causal_tail_mask(N, M, Hm=2, typ=mk)
        mask[1, 0, :] = -np.inf
        return Problem(name, D, Dv, H, Hkv, N, M, 1.0 / math.sqrt(D),
                       q, "f32", k, "f32", v, "f32", do, "f32", mask, mk, seed,
                       "tiny F32 case; causal-tail; head 1 row 0 fully masked")
    if name.startswith("c1") or name in ("c2", "c2b"):
        D = Dv = 128; H, Hkv, N = 8, 2, 64
        M = 512 if name.startswith("c1") else 8192
        k, v, q, do = _draws(rng, H, Hkv, N, M, D, Dv)
        kt = vt = "q8_0"
        mask = None; mtype = "none"
        if name == "c2b":
            kt = "f16"
        if name == "c1_tinydo":
            do = (do * np.float32(1e-6)).astype(np.float32)
        if name == "c1_causal":
            mask = causal_tail_mask(N, M, 1, mk); mtype = mk
        if name == "c1_f32kv":
            kt = vt = "f32"
        if name == "c1_f16kv":
            kt = vt = "f16"
        if name == "c1_bf16kv":
            kt = vt = "bf16"
        ke, ve = encode(k, kt), encode(v, vt)
        if name == "c1_strided":
            ke, ve = interleave_heads(ke), interleave_heads(ve)
        return Problem(name, D, Dv, H, Hkv, N, M, 1.0 / math.sqrt(D),
                       q, "f32", ke, kt, ve, vt, do, "f32", mask, mtype, seed)
    if name in ("c3", "c3v"):
        D = Dv = 128; H, Hkv, N, M = 32, 8, 1024, 1024
        k, v, q, do = _draws(rng, H, Hkv, N, M, D, Dv)
        if name == "c3v":
            v = (np.float32(1.0) + np.float32(1e-3) * v).astype(np.float32)
        mask = causal_tail_mask(N, M, 1, mk)
        return Problem(name, D, Dv, H, Hkv, N, M, 1.0 / math.sqrt(D),
                       to_bf16_bits(q), "bf16", to_bf16_bits(k), "bf16",
                       to_bf16_bits(v), "bf16", to_bf16_bits(do), "bf16", mask, mk, seed)
    if name in ("c4", "c4n8", "c4n16", "c4q4", "c4q4n16"):
        D = Dv = 256; H, Hkv, N, M = 24, 4, 2048, 75520
        k, v, q, do = _draws(rng, H, Hkv, N, M, D, Dv)
        Np = {"c4": N, "c4n8": 8, "c4n16": 16, "c4q4": N, "c4q4n16": 16}[name]
        kt = "q4_0" if name.startswith("c4q4") else "q8_0"
        q = np.ascontiguousarray(q[:, N - Np:, :])
        do = np.ascontiguousarray(do[N - Np:, :, :])
        mask = causal_tail_mask(Np, M, 1, mk)
        return Problem(name, D, Dv, H, Hkv, Np, M, 1.0 / math.sqrt(D),
                       q, "f32", encode(k, kt), kt, encode(v, kt), kt,
                       do, "f32", mask, mk, seed)
    if name.startswith("small_"):
        return make_custom(name, seed=seed, mask_type=mask_type)
    raise KeyError(name)


def magnitude_class(N: int, H: int, classes: int) -> np.ndarray:
    """(N, H) class c in 0..classes-1 of dO row (i, h): c = (i * H + h) % classes."""
    return (np.arange(N)[:, None] * H + np.arange(H)[None, :]) % classes


def make_custom(name="custom", *, D=64, H=2, Hkv=1, N=16, M=64, seed=0, q_type="f32",
                k_type="f32", v_type="f32", d_type="f32", mask="tail", mask_type="f16",
                Hm=1, scale=None, v_offset=0.0, v_spread=1.0, k_offset=0.0, k_spread=1.0,
                d_mult=1.0, d_decades=0, d_group_mult=None, masked_rows=(), flags=0,
                **_ignored) -> Problem:
    """A parameterised case with the same draw order and distributions as the named configs.

    mask: 'none' | 'tail' | 'random' (iid -inf with prob 0.3) ; masked_rows: (hm, i) pairs
    whose mask row is set to all -inf. v = v_offset + v_spread * z (likewise k). d_decades = n > 0
    scales dO row (i, h) by 10^-c, c = magnitude_class(N, H, n + 1)[i, h] (rows of n + 1 decades in
    one tensor); d_group_mult = (hk, f) scales the dO rows of every head of KV head hk by f."""
    Dv = D
    rng = np.random.default_rng(seed)
    k, v, q, do = _draws(rng, H, Hkv, N, M, D, Dv)
    v = (np.float32(v_offset) + np.float32(v_spread) * v).astype(np.float32)
    k = (np.float32(k_offset) + np.float32(k_spread) * k).astype(np.float32)
    do = (do * np.float32(d_mult)).astype(np.float32)
    if d_decades:
        cls = magnitude_class(N, H, d_decades + 1)
        do = (do * (np.float32(10.0) ** -cls.astype(np.float32))[:, :, None]).astype(np.float32)
    if d_group_mult is not None:
        hk, f = d_group_mult
        G = H // Hkv
        do[:, hk * G:(hk + 1) * G, :] *= np.float32(f)
    m = None
    if mask == "tail":
        m = causal_tail_mask(N, M, Hm, mask_type)
    elif mask == "random":
        dt = np.float16 if mask_type == "f16" else np.float32
        m = np.where(rng.random((Hm, N, M)) < 0.3, -np.inf, 0.0).astype(dt)
    if m is not None:
        for hm, i in masked_rows:
            m[hm, i, :] = -np.inf
    return Problem(name, D, Dv, H, Hkv, N, M,
                   1.0 / math.sqrt(D) if scale is None else scale,
                   encode(q, q_type) if q_type != "f32" else q, q_type,
                   encode(k, k_type), k_type, encode(v, v_type), v_type,
                   encode(do, d_type) if d_type != "f32" else do, d_type,
                   m, "none" if m is None else mask_type, seed, flags=flags)


# ----------------------------------------------------------------------------- workload size

def visible_pairs(p: Problem) -> int:
    """Number of (query row, key, head) triples whose mask entry is not -inf."""
    if p.mask is None:
        return p.N * p.M * p.H
    per_hm = [int(np.count_nonzero(np.isfinite(p.mask[hm]))) for hm in range(p.Hm)]
    if p.Hm == 1:
        return per_hm[0] * p.H
    return sum(per_hm)


def flop_count(p: Problem) -> dict:
    """Matrix-product work per call.

    full: the five backward products plus the recomputation a two-pass, atomic-free
          backward performs (scores and dO.V^T three times each) = 2*V*(5D + 4Dv).
    five: the five backward products only = 2*V*(3D + 2Dv)."""
    V = visible_pairs(p)
    return {"visible": V, "full": 2 * V * (5 * p.D + 4 * p.Dv), "five": 2 * V * (3 * p.D + 2 * p.Dv)}


def storage_bytes(x: np.ndarray) -> int:
    """Bytes of the elements of a (possibly strided) stored tensor."""
    return int(x.size * x.itemsize)


def min_bytes(p: Problem) -> dict:
    """HBM bytes a backward must move at least: every input read once (q, dO, K, V and the stored
    mask, in their stored types) and every output written once (dQ, dK, dV F32, LSE and delta)."""
    reads = (storage_bytes(p.q) + storage_bytes(p.d) + storage_bytes(p.k) + storage_bytes(p.v) +
             (0 if p.mask is None or p.mask_type == "causal_tail" else storage_bytes(p.mask)))
    writes = 4 * (p.D * p.N * p.H + p.D * p.M * p.Hkv + p.Dv * p.M * p.Hkv + 2 * p.N * p.H)
    return {"read": reads, "write": writes, "total": reads + writes}
