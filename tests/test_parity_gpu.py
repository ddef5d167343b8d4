"""Parity of the HIP path with the float64 oracle, through the C ABI (GPU only).

Bar: NMSE <= 1e-5 on each of dQ, dK, dV, LSE and delta separately, -inf LSE entries equal,
every defined output byte written (outputs are pre-filled with NaN bytes), bitwise
reproducible runs."""
import dataclasses

import numpy as np
import pytest

import fa_inputs
from flash_attention_backward_amd import fa_back as fab_flags
from oracle import fa_back_oracle as O
from tests.gpu_util import compare, run_gpu, say, walk1

pytestmark = pytest.mark.gpu


def _parity(p):
    got, raw, lay = run_gpu(p)
    ref = O.run_problem(p)
    errs = compare(got, ref)
    say(f"   nmse " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    return got, raw, lay


@pytest.mark.parametrize("name", ["c0", "c1", "c1_causal", "c1_strided", "c1_f32kv", "c1_f16kv",
                                  "c1_bf16kv", "c1_tinydo", "c2", "c2b"])
def test_named_configs(name):
    _parity(fa_inputs.make(name))


@pytest.mark.parametrize("name", ["c3", "c3v"])
def test_square_causal_bf16(name):
    _parity(fa_inputs.make(name))


RAGGED = [
    dict(name="ragged_d128_headmask", D=128, H=6, Hkv=2, N=37, M=203, mask="random", Hm=6,
         masked_rows=[(0, 5), (4, 36)], k_type="q8_0", v_type="f16"),
    dict(name="ragged_d64_q8", D=64, H=4, Hkv=4, N=50, M=130, mask="tail", k_type="q8_0", v_type="q8_0"),
    dict(name="ragged_d256_f32mask", D=256, H=6, Hkv=1, N=11, M=300, mask="tail", mask_type="f32",
         k_type="q8_0", v_type="q8_0"),
    dict(name="d256_bf16_all", D=256, H=4, Hkv=2, N=40, M=129, mask="tail", q_type="bf16",
         d_type="bf16", k_type="bf16", v_type="bf16"),
    dict(name="f16_qd", D=128, H=2, Hkv=1, N=70, M=100, mask="none", q_type="f16", d_type="f16",
         k_type="f32", v_type="q8_0"),
    dict(name="single_key", D=64, H=2, Hkv=1, N=5, M=1, mask="none"),
    dict(name="single_row", D=128, H=8, Hkv=2, N=1, M=777, mask="none", k_type="q8_0", v_type="q8_0"),
    dict(name="all_masked", D=64, H=2, Hkv=1, N=9, M=40, mask="tail",
         masked_rows=[(0, i) for i in range(9)]),
    dict(name="near_const_v_bf16", D=128, H=4, Hkv=1, N=64, M=256, mask="tail", v_offset=1.0,
         v_spread=1e-3, q_type="bf16", d_type="bf16", k_type="bf16", v_type="bf16"),
    # fully masked 32-row blocks (3 and 10) between live ones: the key side skips them
    dict(name="dead_row_blocks", D=128, H=2, Hkv=1, N=200, M=300, mask="random",
         masked_rows=[(0, i) for i in list(range(48, 64)) + list(range(160, 176))],
         k_type="q8_0", v_type="q8_0"),
    # q4_0 caches (the served cache type), alone and beside the other types
    dict(name="q4_0_kv", D=128, H=8, Hkv=2, N=64, M=512, mask="none", k_type="q4_0", v_type="q4_0"),
    dict(name="q4_0_d256_tail", D=256, H=6, Hkv=1, N=40, M=333, mask="tail", k_type="q4_0", v_type="q4_0"),
    dict(name="q4_0_k_q8_0_v", D=64, H=4, Hkv=2, N=33, M=150, mask="tail", k_type="q4_0", v_type="q8_0"),
    dict(name="f16_k_q4_0_v", D=128, H=2, Hkv=1, N=20, M=100, mask="random", k_type="f16", v_type="q4_0"),
    # the other ggml block types: q4_1, q5_0, q5_1, alone, mixed and beside a row type
    dict(name="q4_1_kv", D=128, H=8, Hkv=2, N=64, M=300, mask="none", k_type="q4_1", v_type="q4_1"),
    dict(name="q5_0_d256_tail", D=256, H=6, Hkv=1, N=40, M=333, mask="tail", k_type="q5_0", v_type="q5_0"),
    dict(name="q5_1_d64_random", D=64, H=4, Hkv=2, N=33, M=150, mask="random", Hm=4, k_type="q5_1",
         v_type="q5_1"),
    dict(name="q5_1_k_q4_1_v", D=256, H=4, Hkv=2, N=37, M=210, mask="tail", k_type="q5_1", v_type="q4_1"),
    dict(name="q8_0_k_q5_0_v", D=128, H=4, Hkv=1, N=70, M=129, mask="tail", k_type="q8_0", v_type="q5_0"),
    dict(name="f16_k_q5_1_v", D=128, H=2, Hkv=1, N=20, M=100, mask="random", k_type="f16", v_type="q5_1"),
    # two row blocks per KV head at D=256: the key side's list holds exactly two entries
    dict(name="kv_two_blocks", D=256, H=2, Hkv=1, N=32, M=200, mask="tail", k_type="q8_0", v_type="f16"),
    # four row blocks, the first and the last fully masked: only the middle two are listed
    dict(name="kv_live_middle_blocks", D=128, H=4, Hkv=1, N=32, M=96, mask="random",
         masked_rows=[(0, i) for i in list(range(0, 8)) + list(range(24, 32))],
         k_type="q8_0", v_type="q8_0"),
    # 132000 rows over one KV head (4125 row blocks): every key tile is split into row ranges
    dict(name="long_rows_split", D=64, H=8, Hkv=1, N=16500, M=40, mask="none",
         k_type="q8_0", v_type="q8_0"),
]


@pytest.mark.parametrize("cfg", RAGGED, ids=[c["name"] for c in RAGGED])
def test_ragged_and_degenerate(cfg):
    _parity(fa_inputs.make_custom(**cfg))


@pytest.mark.parametrize("cfg", [dict(name="empty_keys", D=64, H=2, Hkv=1, N=4, M=0, mask="none"),
                                 dict(name="empty_rows", D=128, H=4, Hkv=2, N=0, M=70, mask="tail")],
                         ids=["M0", "N0"])
def test_empty(cfg):
    p = fa_inputs.make_custom(**cfg)
    got, _, _ = run_gpu(p)
    ref = O.run_problem(p)
    for k in ("dq", "dk", "dv", "lse", "delta"):
        assert got[k].shape == ref[k].shape
        np.testing.assert_array_equal(got[k], ref[k].astype(np.float32))


def test_deterministic_bitwise():
    p = fa_inputs.make("c1_causal")
    import flash_attention_backward_amd as fab
    import torch
    dp = fab.DeviceProblem(p, "cuda:0", poison=True)
    outs = []
    for fill in (0xFF, 0x00, 0x7F):
        dp.out.fill_(fill)
        dp.ws.fill_(fill)
        dp.run()
        torch.cuda.synchronize()
        outs.append(fab.fa_back.defined_bytes(dp.out.cpu().numpy(), dp.layout, p))
    dp.close()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_q8_0_equals_dequantised_f32_bitwise():
    p = fa_inputs.make("c1_causal")
    got_q8, _, _ = run_gpu(p)
    q = fa_inputs.Problem(**{**p.__dict__})
    q.name = "c1_causal_dequantised"
    q.k = O.widen(p.k, "q8_0", p.D).astype(np.float32)
    q.v = O.widen(p.v, "q8_0", p.Dv).astype(np.float32)
    q.k_type = q.v_type = "f32"
    got_f32, _, _ = run_gpu(q)
    for k in got_q8:
        assert np.array_equal(got_q8[k].view(np.uint32), got_f32[k].view(np.uint32)), k


@pytest.mark.parametrize("mode", ["rows", "keys"])
def test_q4_0_equals_dequantised_f32_bitwise(mode):
    # every q4_0 value is exact in F32 and rounds once to fp16 on both paths
    p = walk1(fa_inputs.make_custom(name="q4_bits", D=128, H=4, Hkv=2, N=37, M=200, mask="tail",
                                    k_type="q4_0", v_type="q4_0"), mode)
    f = fa_inputs.Problem(**{**p.__dict__})
    f.name = "q4_bits_f32"
    f.k = O.widen(p.k, "q4_0", p.D).astype(np.float32)
    f.v = O.widen(p.v, "q4_0", p.Dv).astype(np.float32)
    f.k_type = f.v_type = "f32"
    a, _, _ = run_gpu(p)
    b, _, _ = run_gpu(f)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


@pytest.mark.parametrize("mode", ["rows", "keys"])
@pytest.mark.parametrize("typ,D", [("q4_1", 128), ("q5_0", 256), ("q5_1", 64)])
def test_block_types_equal_dequantised_f32_bitwise(typ, D, mode):
    # each value of these types is one fp32 rounding of d * code (+ m); an F32 cache holding
    # that value goes through the same fp16 rounding
    p = walk1(fa_inputs.make_custom(name=f"{typ}_bits", D=D, H=4, Hkv=2, N=37, M=200, mask="tail",
                                    k_type=typ, v_type=typ), mode)
    f = fa_inputs.Problem(**{**p.__dict__})
    f.name = f"{typ}_bits_f32"
    f.k = O.widen(p.k, typ, p.D).astype(np.float32)
    f.v = O.widen(p.v, typ, p.Dv).astype(np.float32)
    f.k_type = f.v_type = "f32"
    a, _, _ = run_gpu(p)
    b, _, _ = run_gpu(f)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


def test_strided_cache_equals_contiguous_bitwise():
    a, _, _ = run_gpu(fa_inputs.make("c1"))
    b, _, _ = run_gpu(fa_inputs.make("c1_strided"))
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


@pytest.mark.parametrize("mode", ["rows", "keys"])
def test_gqa_equals_replicated_heads(mode):
    # the same walk-1 variant for both runs: the shape-based choice could differ between them
    p = walk1(fa_inputs.make_custom("gqa", D=128, H=6, Hkv=2, N=33, M=150, mask="tail", k_type="q8_0",
                                    v_type="q8_0"), mode)
    rep = fa_inputs.Problem(**{**p.__dict__})
    rep.name = "gqa_replicated"
    rep.Hkv = p.H
    rep.k = np.repeat(p.k, p.G, axis=0)
    rep.v = np.repeat(p.v, p.G, axis=0)
    a, _, _ = run_gpu(p)
    b, _, _ = run_gpu(rep)
    for k in ("dq", "lse", "delta"):
        assert O.nmse(a[k][np.isfinite(a[k])], b[k][np.isfinite(b[k])]) <= 1e-12, k
    for k in ("dk", "dv"):
        summed = b[k].astype(np.float64).reshape(p.Hkv, p.G, p.M, p.D).sum(axis=1)
        assert O.nmse(a[k], summed) <= 1e-10, k


# Walk 1 runs by row tiles or by key tiles (chosen from the shape unless a descriptor flag picks
# one), and by row tiles in a kernel of its own when the cache is decoded into the image. Each
# must meet the bar on the same inputs.
WALK1_CASES = ["c0", "c1_causal", "ragged_d128_headmask", "ragged_d64_q8", "ragged_d256_f32mask",
               "all_masked", "single_key", "dead_row_blocks", "kv_live_middle_blocks"]


def _walk1_problem(name):
    if name.startswith("c"):
        return fa_inputs.make(name)
    return fa_inputs.make_custom(**next(c for c in RAGGED if c["name"] == name))


@pytest.mark.parametrize("mode", ["rows", "keys", "rows_image", "rows_ds"])
@pytest.mark.parametrize("name", WALK1_CASES)
def test_walk1_variants(name, mode):
    say(f"[walk1 {mode}]")
    _parity(walk1(_walk1_problem(name), mode))


# The causal-tail mask without storage (FA_BACK_CAUSAL_TAIL): the library forms the mask from
# i and j, and must give bitwise the results of the same mask stored as F16, under both walk-1
# variants (N < M, N > M with fully masked rows, N = M, D = 256, the long-cache pilot).
IMPLICIT_CASES = [
    ("c1_causal", None),
    ("c4n16", None),
    ("impl_n_gt_m", dict(D=128, H=4, Hkv=2, N=100, M=60, mask="tail", k_type="q8_0", v_type="q8_0")),
    ("impl_d256", dict(D=256, H=6, Hkv=1, N=45, M=300, mask="tail", k_type="q8_0", v_type="q8_0")),
    ("impl_square", dict(D=64, H=2, Hkv=1, N=150, M=150, mask="tail", q_type="bf16", d_type="bf16",
                         k_type="bf16", v_type="bf16")),
]


def _implicit_problem(name, cfg):
    return fa_inputs.make(name) if cfg is None else fa_inputs.make_custom(name=name, **cfg)


@pytest.mark.parametrize("mode", ["rows", "keys", "rows_image", "rows_ds"])
@pytest.mark.parametrize("name,cfg", IMPLICIT_CASES, ids=[c[0] for c in IMPLICIT_CASES])
def test_implicit_causal_tail_bitwise(name, cfg, mode):
    p = walk1(_implicit_problem(name, cfg), mode)
    a, _, _ = run_gpu(p)
    b, _, _ = run_gpu(fa_inputs.implicit_causal(p))
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


def test_implicit_causal_tail_parity():
    _parity(fa_inputs.implicit_causal(fa_inputs.make_custom(name="impl_parity", **IMPLICIT_CASES[2][1])))


@pytest.mark.parametrize("flags", [0, fab_flags.FLAG_WALK1_KEYS, fab_flags.FLAG_WALK1_ROWS],
                         ids=["default", "walk1_keys", "walk1_rows"])
def test_create_layout_equals_query(flags):
    # the plan reads the device's CU count and LDS size; the layout stays that of the descriptor
    import flash_attention_backward_amd as fab
    for name in ("c0", "c1", "c2", "c3"):
        p = dataclasses.replace(fa_inputs.make(name), flags=flags)
        d = fab_flags.describe(p)
        q = fab.fa_back_layout_query(d)
        plan, lay = fab.fa_back_create(d, 0)
        fab.fa_back_destroy(plan)
        for f, _ in fab_flags.Layout._fields_:
            assert getattr(q, f) == getattr(lay, f), (name, f)
