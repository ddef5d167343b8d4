"""Pins of the float64 oracle to things other than itself (CPU only).

- a hand-worked example whose every value was derived on paper (tests/golden);
- central finite differences of the loss sum(dO o O) of an independently written forward;
- delta = rowsum(dO o O) with O from that forward; LSE = logsumexp via math.fsum;
- fully masked rows, GQA as a sum over replicated heads, q8_0 / bf16 decoding of
  hand-built bytes, closed forms (one visible key, Q = 0), invariances (V shift, mask
  shift, linearity in dO), and an independent pure-Python loop implementation.
"""
import json
import math
import os

import numpy as np
import pytest

import fa_inputs
from oracle import fa_back_oracle as O


def _ev(x):
    if isinstance(x, str):
        return float(eval(x, {"log": math.log, "inf": math.inf}))
    return float(x)


def _arr(nested):
    if isinstance(nested, list):
        return np.array([_arr(e) for e in nested], dtype=np.float64)
    return _ev(nested)


# ----------------------------------------------------------------------------- forward

def forward_loss(q, k, v, do, mask, scale):
    """sum over (h, i, c) of dO[i,h,c] * O[h,i,c] with O = softmax(scale q k^T + mask) V.
    A fully masked row has O = 0. Written directly from the attention forward."""
    H, N, _ = q.shape
    Hkv = k.shape[0]
    G = H // Hkv
    total = 0.0
    outs = np.zeros((H, N, v.shape[2]))
    for h in range(H):
        hk = h // G
        for i in range(N):
            s = scale * (k[hk] @ q[h, i])
            if mask is not None:
                s = s + mask[h % mask.shape[0], i]
            if not np.any(np.isfinite(s)):
                continue
            w = np.exp(s - np.max(s))
            o = (w @ v[hk]) / np.sum(w)
            outs[h, i] = o
            total += float(np.dot(do[i, h], o))
    return total, outs


def fd_grad(fun, x, idx, eps=1e-5):
    g = []
    for t in idx:
        old = x.flat[t]
        x.flat[t] = old + eps
        fp = fun()
        x.flat[t] = old - eps
        fm = fun()
        x.flat[t] = old
        g.append((fp - fm) / (2 * eps))
    return np.array(g)


def _micro(seed=3):
    rng = np.random.default_rng(seed)
    H, Hkv, N, M, D = 2, 1, 3, 5, 4
    q = rng.standard_normal((H, N, D))
    k = rng.standard_normal((Hkv, M, D))
    v = rng.standard_normal((Hkv, M, D))
    do = rng.standard_normal((N, H, D))
    mask = np.zeros((H, N, M))
    mask[0, 1, 3] = -np.inf
    mask[1, 0, :] = -np.inf            # fully masked row of head 1
    mask[1, 2, 0] = -np.inf
    mask[0, 2, 4] = -0.7               # a finite additive entry
    return q, k, v, do, mask, 0.37


# ----------------------------------------------------------------------------- tests

def test_hand_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_h2_n2_m3.json")))
    inp, exp = g["inputs"], g["expected"]
    res = O.flash_attn_back(_arr(inp["q_HND"]), _arr(inp["k_HkvMD"]), _arr(inp["v_HkvMDv"]),
                            _arr(inp["dO_NHDv"]), _arr(inp["mask_HmNM"]), inp["scale"])
    for key, name in (("dq", "dq_HND"), ("dk", "dk_HkvMD"), ("dv", "dv_HkvMDv"),
                      ("lse", "lse_HN"), ("delta", "delta_HN")):
        np.testing.assert_allclose(res[key], _arr(exp[name]), rtol=1e-14, atol=1e-14, err_msg=key)
    # the key no row sees gets exactly zero gradients
    assert res["dk"][0, 2, 0] == 0.0 and res["dv"][0, 2, 0] == 0.0


def test_finite_differences_micro_all_params():
    q, k, v, do, mask, scale = _micro()
    scale = float(np.float32(scale))
    res = O.flash_attn_back(q, k, v, do, mask, scale)
    for name, x, key in (("q", q, "dq"), ("k", k, "dk"), ("v", v, "dv")):
        fun = lambda: forward_loss(q, k, v, do, mask, scale)[0]
        g = fd_grad(fun, x, range(x.size))
        np.testing.assert_allclose(res[key].ravel(), g, rtol=1e-7, atol=1e-9, err_msg=name)


def test_finite_differences_config0_sampled():
    p = fa_inputs.make("c0")
    q, k, v, do, mask = O.problem_arrays(p)
    scale = float(np.float32(p.scale))
    res = O.run_problem(p)
    rng = np.random.default_rng(11)
    for name, x, key in (("q", q, "dq"), ("k", k, "dk"), ("v", v, "dv")):
        idx = rng.choice(x.size, size=48, replace=False)
        if name == "q":   # include the fully masked row of head 1 (row 0)
            idx = np.concatenate([idx, np.arange(1 * 16 * 64, 1 * 16 * 64 + 4)])
        fun = lambda: forward_loss(q, k, v, do, mask, scale)[0]
        g = fd_grad(fun, x, idx)
        np.testing.assert_allclose(res[key].ravel()[idx], g, rtol=1e-6, atol=1e-8, err_msg=name)


def test_delta_is_rowsum_dO_times_O():
    for case in (_micro(), ):
        q, k, v, do, mask, scale = case
        res = O.flash_attn_back(q, k, v, do, mask, scale)
        _, outs = forward_loss(q, k, v, do, mask, float(np.float32(scale)))
        expect = np.einsum("nhc,hnc->hn", do, outs)
        np.testing.assert_allclose(res["delta"], expect, rtol=1e-12, atol=1e-14)
    p = fa_inputs.make("c0")
    q, k, v, do, mask = O.problem_arrays(p)
    res = O.run_problem(p)
    _, outs = forward_loss(q, k, v, do, mask, float(np.float32(p.scale)))
    np.testing.assert_allclose(res["delta"], np.einsum("nhc,hnc->hn", do, outs), rtol=1e-11, atol=1e-13)


def test_forward_outputs_match_independent_forward():
    # the saved statistics the oracle hands to the saved-statistics entry: O against the
    # independently written forward above, lse against the backward's own
    for q, k, v, do, mask, scale in (_micro(), ):
        lse, o = O.forward_outputs(q, k, v, mask, scale)
        _, outs = forward_loss(q, k, v, do, mask, float(np.float32(scale)))
        np.testing.assert_allclose(o, outs, rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(lse, O.flash_attn_back(q, k, v, do, mask, scale)["lse"])
    p = fa_inputs.make("c0")                     # head 1 row 0 fully masked: lse -inf, O = 0
    q, k, v, do, mask = O.problem_arrays(p)
    lse, o = O.forward_problem(p)
    _, outs = forward_loss(q, k, v, do, mask, float(np.float32(p.scale)))
    np.testing.assert_allclose(o, outs, rtol=1e-11, atol=1e-13)
    assert lse[1, 0] == -np.inf and not o[1, 0].any()


def test_lse_is_logsumexp_fsum():
    p = fa_inputs.make("c0")
    q, k, v, do, mask = O.problem_arrays(p)
    res = O.run_problem(p)
    sc = float(np.float32(p.scale))
    for h, i in ((0, 0), (0, 7), (1, 1), (1, 15), (0, 15)):
        s = [sc * math.fsum(q[h, i, c] * k[0, j, c] for c in range(p.D)) + mask[h, i, j]
             for j in range(p.M)]
        fin = [x for x in s if x != -math.inf]
        mx = max(fin)
        lse = mx + math.log(math.fsum(math.exp(x - mx) for x in fin))
        assert abs(res["lse"][h, i] - lse) <= 1e-12 * max(1.0, abs(lse))


def test_fully_masked_row():
    p = fa_inputs.make("c0")
    res = O.run_problem(p)
    assert res["lse"][1, 0] == -math.inf
    assert res["delta"][1, 0] == 0.0
    assert np.all(res["dq"][1, 0] == 0.0)
    # the row adds nothing to dK/dV: drop row 0 of head 1 by zeroing its dO and q
    q, k, v, do, mask = O.problem_arrays(p)
    q2, do2 = q.copy(), do.copy()
    q2[1, 0] = 123.0
    do2[0, 1] = -77.0
    res2 = O.flash_attn_back(q2, k, v, do2, mask, p.scale)
    np.testing.assert_array_equal(res2["dk"], res["dk"])
    np.testing.assert_array_equal(res2["dv"], res["dv"])
    # every other row is finite
    fin = np.isfinite(res["lse"])
    assert fin.sum() == fin.size - 1


def test_all_rows_masked():
    q, k, v, do, mask, scale = _micro()
    mask[:] = -np.inf
    res = O.flash_attn_back(q, k, v, do, mask, scale)
    assert np.all(res["lse"] == -np.inf)
    for key in ("dq", "dk", "dv", "delta"):
        assert np.all(res[key] == 0.0), key


def test_gqa_equals_sum_over_replicated_heads():
    rng = np.random.default_rng(5)
    H, Hkv, N, M, D = 6, 2, 5, 9, 8
    q = rng.standard_normal((H, N, D)); do = rng.standard_normal((N, H, D))
    k = rng.standard_normal((Hkv, M, D)); v = rng.standard_normal((Hkv, M, D))
    mask = np.where(rng.random((1, N, M)) < 0.25, -np.inf, 0.0)
    G = H // Hkv
    res = O.flash_attn_back(q, k, v, do, mask, 0.3)
    rep = O.flash_attn_back(q, np.repeat(k, G, axis=0), np.repeat(v, G, axis=0), do, mask, 0.3)
    np.testing.assert_allclose(res["dq"], rep["dq"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(res["lse"], rep["lse"], rtol=1e-14)
    np.testing.assert_allclose(res["delta"], rep["delta"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(res["dk"], rep["dk"].reshape(Hkv, G, M, D).sum(1), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res["dv"], rep["dv"].reshape(Hkv, G, M, D).sum(1), rtol=1e-12, atol=1e-13)


def test_q8_0_decoding_of_hand_built_blocks(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "q8_0_blocks.json")))
    raw = bytearray()
    expect = []
    for b in g["blocks"]:
        h = int(b["scale_fp16_hex"], 16)
        raw += bytes([h & 0xFF, h >> 8])
        raw += bytes([(x + 256) % 256 for x in b["q"]])
        expect += [b["scale"] * x for x in b["q"]]
    arr = np.frombuffer(bytes(raw), dtype=np.uint8).reshape(1, 1, -1)
    got = O.widen(arr, "q8_0", 32 * len(g["blocks"]))
    np.testing.assert_array_equal(got.ravel(), np.array(expect))


def test_q4_0_decoding_of_hand_built_blocks(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "q4_0_blocks.json")))
    raw = bytearray()
    expect = []
    for b in g["blocks"]:
        h = int(b["scale_fp16_hex"], 16)
        raw += bytes([h & 0xFF, h >> 8]) + bytes(b["bytes"])
        expect += b["values"]
    arr = np.frombuffer(bytes(raw), dtype=np.uint8).reshape(1, 1, -1)
    got = O.widen(arr, "q4_0", 32 * len(g["blocks"]))
    np.testing.assert_array_equal(got.ravel(), np.array(expect))


@pytest.mark.parametrize("typ", ["q4_1", "q5_0", "q5_1"])
def test_other_block_types_decoding_of_hand_built_blocks(golden_dir, typ):
    g = json.load(open(os.path.join(golden_dir, f"{typ}_blocks.json")))
    raw = bytearray()
    expect = []
    for b in g["blocks"]:
        raw += bytes(b["bytes"])
        expect += b["values"]
    assert len(raw) == O.BLOCK_BYTES[typ] * len(g["blocks"])
    arr = np.frombuffer(bytes(raw), dtype=np.uint8).reshape(1, 1, -1)
    got = O.widen(arr, typ, 32 * len(g["blocks"]))
    np.testing.assert_array_equal(got.ravel(), np.array(expect))


@pytest.mark.parametrize("typ", ["q4_1", "q5_0", "q5_1"])
def test_other_block_types_run_equals_dequantised_f32_run(typ):
    p = fa_inputs.make_custom(name=typ, D=64, H=4, Hkv=2, N=9, M=40, mask="tail", k_type=typ, v_type=typ)
    nb = O.BLOCK_BYTES[typ]

    # hand decode by integer arithmetic on the bytes (not the oracle's decoder)
    def dec(raw):
        raw = np.asarray(raw).astype(np.int64)
        out = np.empty(raw.shape[:-1] + (raw.shape[-1] // nb * 32,))
        for b in range(raw.shape[-1] // nb):
            blk = raw[..., nb * b:nb * (b + 1)]
            half = lambda i: (blk[..., i] | (blk[..., i + 1] << 8)).astype(np.uint16).view(np.float16).astype(np.float64)
            d = half(0)
            m = half(2) if typ != "q5_0" else 0.0
            at = 2 if typ == "q5_0" else 4
            h = 0
            if typ != "q4_1":
                h = blk[..., at] | (blk[..., at + 1] << 8) | (blk[..., at + 2] << 16) | (blk[..., at + 3] << 24)
                at += 4
            for t in range(32):
                byte = blk[..., at + (t % 16)]
                code = (byte % 16 if t < 16 else byte // 16) + 16 * ((h >> t) & 1)
                val = d * (code - 16) if typ == "q5_0" else d * code + m
                out[..., 32 * b + t] = val
        return out
    kf, vf = dec(p.k), dec(p.v)
    a = O.run_problem(p)
    q, _, _, do, mask = O.problem_arrays(p)
    b = O.flash_attn_back(q, kf, vf, do, mask, p.scale)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_q4_0_run_equals_dequantised_f32_run():
    p = fa_inputs.make_custom(name="q4", D=64, H=4, Hkv=2, N=9, M=40, mask="tail",
                              k_type="q4_0", v_type="q4_0")
    # hand decode by integer nibble arithmetic (not the oracle's decoder)
    def dec(raw):
        raw = np.asarray(raw)
        out = np.empty(raw.shape[:-1] + (raw.shape[-1] // 18 * 32,))
        for b in range(raw.shape[-1] // 18):
            s = raw[..., 18 * b].astype(np.uint16) | (raw[..., 18 * b + 1].astype(np.uint16) << 8)
            sc = s.view(np.float16).astype(np.float64)[..., None]
            body = raw[..., 18 * b + 2:18 * b + 18].astype(np.int64)
            out[..., 32 * b:32 * b + 16] = sc * ((body % 16) - 8)
            out[..., 32 * b + 16:32 * b + 32] = sc * ((body // 16) - 8)
        return out
    kf, vf = dec(p.k), dec(p.v)
    a = O.run_problem(p)
    q, _, _, do, mask = O.problem_arrays(p)
    b = O.flash_attn_back(q, kf, vf, do, mask, p.scale)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_bf16_widening_of_hand_built_bits():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049, 0x0001], dtype=np.uint16)
    expect = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, 3.140625, 2.0 ** -133]
    np.testing.assert_array_equal(O.widen(bits, "bf16"), np.array(expect))


def test_q8_0_run_equals_dequantised_f32_run():
    p = fa_inputs.make("c1")
    # hand decode: scale bytes then int8, through numpy views (not the oracle's decoder)
    def dec(raw):
        raw = np.asarray(raw)
        out = np.empty(raw.shape[:-1] + (raw.shape[-1] // 34 * 32,))
        for b in range(raw.shape[-1] // 34):
            s = raw[..., 34 * b].astype(np.uint16) | (raw[..., 34 * b + 1].astype(np.uint16) << 8)
            out[..., 32 * b:32 * b + 32] = (s.view(np.float16).astype(np.float64)[..., None]
                                             * raw[..., 34 * b + 2:34 * b + 34].view(np.int8))
        return out
    kf, vf = dec(p.k), dec(p.v)
    a = O.run_problem(p)
    q, _, _, do, mask = O.problem_arrays(p)
    b = O.flash_attn_back(q, kf, vf, do, mask, p.scale)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_single_visible_key_closed_form():
    rng = np.random.default_rng(9)
    H, Hkv, N, M, D = 4, 2, 3, 7, 6
    q = rng.standard_normal((H, N, D)); do = rng.standard_normal((N, H, D))
    k = rng.standard_normal((Hkv, M, D)); v = rng.standard_normal((Hkv, M, D))
    mask = np.full((1, N, M), -np.inf)
    mask[0, :, 2] = 0.0                      # every row sees key 2 only
    res = O.flash_attn_back(q, k, v, do, mask, 0.5)
    G = H // Hkv
    for h in range(H):
        hk = h // G
        np.testing.assert_allclose(res["lse"][h], 0.5 * q[h] @ k[hk, 2], rtol=1e-14)
        np.testing.assert_allclose(res["delta"][h], do[:, h] @ v[hk, 2], rtol=1e-13)
    assert np.all(res["dq"] == 0.0) and np.all(res["dk"] == 0.0)
    for hk in range(Hkv):
        np.testing.assert_allclose(res["dv"][hk, 2], do[:, hk * G:(hk + 1) * G].sum(axis=(0, 1)), rtol=1e-13)
        assert np.all(np.delete(res["dv"][hk], 2, axis=0) == 0.0)


def test_zero_query_gives_uniform_weights():
    rng = np.random.default_rng(10)
    H, Hkv, N, M, D = 2, 1, 4, 8, 5
    q = np.zeros((H, N, D)); do = rng.standard_normal((N, H, D))
    k = rng.standard_normal((Hkv, M, D)); v = rng.standard_normal((Hkv, M, D))
    mask = np.where(rng.random((1, N, M)) < 0.4, -np.inf, 0.0)
    mask[0, :, 0] = 0.0
    res = O.flash_attn_back(q, k, v, do, mask, 0.8)
    nvis = np.isfinite(mask[0]).sum(axis=1)
    for h in range(H):
        np.testing.assert_allclose(res["lse"][h], np.log(nvis), rtol=1e-14)
        vbar = np.array([v[0][np.isfinite(mask[0, i])].mean(axis=0) for i in range(N)])
        np.testing.assert_allclose(res["delta"][h], np.sum(do[:, h] * vbar, axis=1), rtol=1e-12)
    assert np.all(res["dk"] == 0.0)


def test_value_shift_invariance():
    q, k, v, do, mask, scale = _micro()
    u = np.array([0.5, -1.25, 2.0, 3.0])
    a = O.flash_attn_back(q, k, v, do, mask, scale)
    b = O.flash_attn_back(q, k, v + u, do, mask, scale)
    for key in ("dq", "dk", "dv"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-10, atol=1e-12, err_msg=key)
    shift = np.einsum("nhc,c->hn", do, u)
    live = np.isfinite(a["lse"])
    np.testing.assert_allclose(b["delta"][live], a["delta"][live] + shift[live], rtol=1e-12)


def test_mask_row_shift_invariance():
    q, k, v, do, mask, scale = _micro()
    m2 = mask.copy()
    m2[0, 1] += 2.5                          # finite shift of a whole row (-inf stays -inf)
    a = O.flash_attn_back(q, k, v, do, mask, scale)
    b = O.flash_attn_back(q, k, v, do, m2, scale)
    assert abs(b["lse"][0, 1] - (a["lse"][0, 1] + 2.5)) < 1e-13
    for key in ("dq", "dk", "dv", "delta"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-12, atol=1e-14, err_msg=key)


def test_linear_in_dO():
    q, k, v, do, mask, scale = _micro()
    a = O.flash_attn_back(q, k, v, do, mask, scale)
    b = O.flash_attn_back(q, k, v, -3.0 * do, mask, scale)
    for key in ("dq", "dk", "dv", "delta"):
        np.testing.assert_allclose(b[key], -3.0 * a[key], rtol=1e-12, atol=1e-14, err_msg=key)
    np.testing.assert_array_equal(b["lse"], a["lse"])


def test_loop_oracle_matches_numpy_oracle_config0():
    p = fa_inputs.make("c0")
    q, k, v, do, mask = O.problem_arrays(p)
    a = O.flash_attn_back(q, k, v, do, mask, p.scale)
    b = O.flash_attn_back_loops(q, k, v, do, mask, p.scale)
    for key in a:
        fin = np.isfinite(a[key])
        np.testing.assert_array_equal(np.isfinite(b[key]), fin)
        np.testing.assert_allclose(b[key][fin], a[key][fin], rtol=1e-12, atol=1e-13, err_msg=key)


def test_sampled_rows_and_keys_match_full_oracle():
    p = fa_inputs.make_custom("s", D=32, H=6, Hkv=2, N=20, M=70, Hm=1, mask="tail",
                              masked_rows=[(0, 3)], seed=4)
    q, k, v, do, mask = O.problem_arrays(p)
    full = O.flash_attn_back(q, k, v, do, mask, p.scale)
    picks = [(0, 0), (5, 19), (2, 3), (3, 7)]
    dq, lse, dl = O.query_rows(q, k, v, do, mask, p.scale, picks)
    for t, (h, i) in enumerate(picks):
        np.testing.assert_allclose(dq[t], full["dq"][h, i], rtol=1e-12, atol=1e-14)
        assert (lse[t] == full["lse"][h, i]) or abs(lse[t] - full["lse"][h, i]) < 1e-12
        assert abs(dl[t] - full["delta"][h, i]) < 1e-12
    kp = [(0, 0), (1, 69), (1, 33), (0, 50)]
    dk, dv = O.key_rows(q, k, v, do, mask, p.scale, kp, chunk=7)
    for t, (hk, j) in enumerate(kp):
        np.testing.assert_allclose(dk[t], full["dk"][hk, j], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(dv[t], full["dv"][hk, j], rtol=1e-11, atol=1e-13)


def test_nmse_definition():
    ref = np.array([1.0, -2.0, -np.inf, 3.0])
    x = np.array([1.0, -2.0, -np.inf, 4.0])
    assert O.nmse(x, ref) == pytest.approx(1.0 / 14.0)
    assert O.nmse(np.zeros(3), np.zeros(3)) == 0.0
    assert O.nmse(np.ones(3), np.zeros(3)) == math.inf
