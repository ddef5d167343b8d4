"""The C ABI on a host without a GPU: the library loads, exports every declared entry point,
validates descriptors with the documented status codes and computes the packed layout."""
import ctypes
import os
import re

import numpy as np
import pytest

import fa_inputs
import flash_attention_backward_amd as fab
from flash_attention_backward_amd import fa_back as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "fa_back.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fa_back_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("fa_back_create", "fa_back_run", "fa_back_destroy", "fa_back_layout_query",
              "fa_back_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = fab.load_library()
    for n in _declared():
        assert hasattr(lib, n), n


def _desc(name="c1"):
    return B.describe(fa_inputs.make(name))


@pytest.mark.parametrize("name", ["c0", "c1", "c1_strided", "c2b", "c3"])
def test_layout(name):
    p = fa_inputs.make(name)
    lay = fab.fa_back_layout_query(B.describe(p))
    assert lay.off_dq == 0
    assert lay.off_dk % 256 == 0 and lay.off_dv % 256 == 0 and lay.off_lse % 256 == 0
    assert lay.off_dk >= 4 * p.D * p.N * p.H
    assert lay.off_dv >= lay.off_dk + 4 * p.D * p.M * p.Hkv
    assert lay.off_lse >= lay.off_dv + 4 * p.Dv * p.M * p.Hkv
    assert lay.off_delta == lay.off_lse + 4 * p.N * p.H
    assert lay.out_bytes >= lay.off_delta + 4 * p.N * p.H and lay.out_bytes % 256 == 0
    assert lay.workspace_bytes > 0


def _expect(rc, mutate, name="c1"):
    d = _desc(name)
    mutate(d)
    lay = B.Layout()
    got = fab.load_library().fa_back_layout_query(ctypes.byref(d), ctypes.byref(lay))
    assert got == rc, (got, rc)


def test_validation_codes():
    _expect(B.OK, lambda d: None)
    _expect(B.EUNSUPPORTED, lambda d: setattr(d.q, "type", B.Q8_0))
    _expect(B.EUNSUPPORTED, lambda d: setattr(d.mask, "type", B.BF16))
    _expect(B.EINVAL, lambda d: setattr(d, "scale", float("nan")))

    def neg(d): d.q.ne[1] = -1
    _expect(B.EINVAL, neg)

    def dmis(d): d.k.ne[0] = 64
    _expect(B.ESHAPE, dmis)

    def hmis(d):
        d.k.ne[2] = 3; d.v.ne[2] = 3
    _expect(B.ESHAPE, hmis)

    def nmis(d): d.d.ne[2] = 63
    _expect(B.ESHAPE, nmis)

    def nb0(d): d.q.nb[0] = 8
    _expect(B.ESTRIDE, nb0)

    def zero_stride(d): d.k.nb[1] = 0
    _expect(B.ESTRIDE, zero_stride)

    def odd_q8(d): d.k.nb[1] = 137
    _expect(B.ESTRIDE, odd_q8)

    def dv_differs(d):
        d.v.ne[0] = 64; d.d.ne[0] = 64; d.v.nb[1] = 68; d.v.nb[2] = 68 * d.v.ne[1]
    _expect(B.EUNSUPPORTED, dv_differs)

    def q8_width(d):
        for t in (d.q, d.k, d.v, d.d):
            t.ne[0] = 48
    _expect(B.ESHAPE, q8_width)


def test_validation_mask_and_kv_alignment():
    def hm3(d): d.mask.ne[2] = 3
    _expect(B.ESHAPE, hm3, "c1_causal")

    def mask_m(d): d.mask.ne[0] = 100
    _expect(B.ESHAPE, mask_m, "c1_causal")

    def f16_rows_unaligned(d): d.k.nb[1] = 264
    _expect(B.ESTRIDE, f16_rows_unaligned, "c1_f16kv")

    def unsupported_d(d):
        for t in (d.q, d.k, d.v, d.d):
            t.ne[0] = 96
        d.q.nb[1] = 4 * 96; d.q.nb[2] = 4 * 96 * 64
    _expect(B.EUNSUPPORTED, unsupported_d, "c1_f32kv")

    # K/V row strides must stay below 2^32 bytes (the DMA forms row addresses in 32 bits)
    def huge_k_row_stride(d): d.k.nb[1] = 1 << 32
    _expect(B.EUNSUPPORTED, huge_k_row_stride)

    def huge_v_row_stride(d): d.v.nb[1] = (1 << 32) + 32
    _expect(B.EUNSUPPORTED, huge_v_row_stride, "c1_f32kv")


def test_null_arguments():
    lib = fab.load_library()
    lay = B.Layout()
    assert lib.fa_back_layout_query(None, ctypes.byref(lay)) == B.EINVAL
    d = _desc()
    assert lib.fa_back_layout_query(ctypes.byref(d), None) == B.EINVAL
    assert lib.fa_back_create(ctypes.byref(d), 0, None, None) == B.EINVAL
    assert lib.fa_back_run(None, *([None] * 8)) == B.EINVAL
    lib.fa_back_destroy(None)


def test_create_without_gpu_reports_unsupported():
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    lib = fab.load_library()
    d = _desc()
    plan = ctypes.c_void_p(1234)
    rc = lib.fa_back_create(ctypes.byref(d), 0, ctypes.byref(plan), None)
    assert rc == B.EUNSUPPORTED
    assert not plan.value


def test_status_strings():
    assert fab.status_string(0) == "ok"
    assert "shape" in fab.status_string(-2)
    assert fab.status_string(12345) == "unknown status"


def test_key_side_row_split_workspace():
    """With more than 2048 row blocks of 32 rows per KV head, the key side splits every key tile
    into row ranges whose partial dK/dV (2 x 128 keys x D floats per range) live in the
    workspace; at 2048 row blocks exactly, nothing is split."""
    def ws(n):
        p = fa_inputs.make_custom(name="split", D=64, H=4, Hkv=1, N=n, M=256, mask="none")
        return fab.fa_back_layout_query(B.describe(p)).workspace_bytes
    at, past = ws(16384), ws(16392)          # G*N/32 = 2048 and 2049 row blocks
    parts = 4 * 2 * 2 * 2 * 128 * 64         # floats: 2 key tiles x 2 ranges x (dK, dV) x 128 keys x D
    assert past - at >= parts
    assert past - at < parts + (1 << 16)     # the other terms grow by 8 query rows only


def test_implicit_causal_tail_descriptor():
    """The storage-free causal-tail mask: extents {M, N, 1}, strides ignored; one mask head
    only; no mask-class table in the workspace."""
    p = fa_inputs.make("c1_causal")
    lib = fab.load_library()
    d = B.describe(fa_inputs.implicit_causal(p))
    lay = B.Layout()
    assert lib.fa_back_layout_query(ctypes.byref(d), ctypes.byref(lay)) == B.OK
    ref = fab.fa_back_layout_query(B.describe(p))
    assert lay.out_bytes == ref.out_bytes and lay.off_delta == ref.off_delta
    assert lay.workspace_bytes < ref.workspace_bytes
    d.mask.ne[2] = 2                                   # more than one mask head
    assert lib.fa_back_layout_query(ctypes.byref(d), ctypes.byref(lay)) == B.ESHAPE
    d.mask.ne[2] = 1
    d.mask.ne[0] = p.M + 1                             # extents must be {M, N, 1}
    assert lib.fa_back_layout_query(ctypes.byref(d), ctypes.byref(lay)) == B.ESHAPE


def test_centre_v_flag_validation():
    # the flag applies to F32 / F16 / BF16 V; block types and unknown bits are refused
    _expect(B.OK, lambda d: setattr(d, "flags", B.FLAG_CENTER_V), "c1_f32kv")
    _expect(B.OK, lambda d: setattr(d, "flags", B.FLAG_CENTER_V), "c3")
    _expect(B.EUNSUPPORTED, lambda d: setattr(d, "flags", B.FLAG_CENTER_V), "c1")
    _expect(B.EINVAL, lambda d: setattr(d, "flags", 1 << 8), "c1_f32kv")
    # the centre takes Hkv * D floats of workspace
    d0 = _desc("c1_f32kv")
    d1 = _desc("c1_f32kv")
    d1.flags = B.FLAG_CENTER_V
    lib = fab.load_library()
    l0, l1 = B.Layout(), B.Layout()
    assert lib.fa_back_layout_query(ctypes.byref(d0), ctypes.byref(l0)) == B.OK
    assert lib.fa_back_layout_query(ctypes.byref(d1), ctypes.byref(l1)) == B.OK
    assert l1.workspace_bytes >= l0.workspace_bytes + 4 * 2 * 128
    assert l1.out_bytes == l0.out_bytes


def test_walk1_and_centre_k_flags():
    # the two walk-1 flags exclude each other; K centring applies to F32 / F16 / BF16 K only
    _expect(B.OK, lambda d: setattr(d, "flags", B.FLAG_WALK1_KEYS))
    _expect(B.OK, lambda d: setattr(d, "flags", B.FLAG_WALK1_ROWS))
    _expect(B.EINVAL, lambda d: setattr(d, "flags", B.FLAG_WALK1_KEYS | B.FLAG_WALK1_ROWS))
    _expect(B.EUNSUPPORTED, lambda d: setattr(d, "flags", B.FLAG_CENTER_K), "c1")
    _expect(B.OK, lambda d: setattr(d, "flags", B.FLAG_CENTER_K), "c1_f32kv")
    _expect(B.OK, lambda d: setattr(d, "flags", B.FLAG_CENTER_K | B.FLAG_CENTER_V), "c3")
    _expect(B.EINVAL, lambda d: setattr(d, "flags", 256), "c1_f32kv")


def _ws(p, flags):
    d = B.describe(p)
    d.flags = flags
    return fab.fa_back_layout_query(d)


def test_walk1_flag_sets_the_workspace():
    """The key-owned walk keeps one record per row and 256-key tile, the row-owned walk one per
    key-range split, of which the workspace holds the most it may take: min(32, 64-key tiles).
    The flags pick the walk (and with it the workspace); without a flag the row-owned walk is
    taken when the cache is decoded into the image, else the key-owned walk for a long cache
    (M >= 2 G N) and the row-owned walk for a short one."""
    long_cache = fa_inputs.make_custom("long", D=64, H=24, Hkv=4, N=256, M=8192, mask="none")
    short = fa_inputs.make_custom("short", D=64, H=4, Hkv=1, N=64, M=300, mask="none")
    for p in (long_cache, short):
        keys, rows = _ws(p, B.FLAG_WALK1_KEYS), _ws(p, B.FLAG_WALK1_ROWS)
        assert keys.out_bytes == rows.out_bytes and keys.off_delta == rows.off_delta
        rows_total = p.Hkv * (-(-(p.H // p.Hkv) * p.N // 32)) * 32
        rec_keys = -(-p.M // 256)
        rec_rows = min(32, -(-p.M // 64))
        want = (rec_keys - rec_rows) * 16 * rows_total
        assert abs((keys.workspace_bytes - rows.workspace_bytes) - want) < 256
    # long_cache has 12 row tiles of 128 rows per KV head, so the image by default
    assert _ws(long_cache, 0).workspace_bytes == _ws(long_cache, B.FLAG_WALK1_ROWS).workspace_bytes
    inline = B.FLAG_KV_INLINE
    assert (_ws(long_cache, inline).workspace_bytes ==
            _ws(long_cache, inline | B.FLAG_WALK1_KEYS).workspace_bytes)
    assert _ws(short, 0).workspace_bytes == _ws(short, B.FLAG_WALK1_ROWS).workspace_bytes


def test_kv_image_flags_and_workspace():
    """The decoded image of the cache takes Hkv * ceil(M / 32) * 128 * D bytes of workspace; the
    two flags exclude each other; without a flag the plan takes the image when at least 4 row
    tiles of 128 rows (per KV head) read each sub-tile: c3 (32 row tiles) yes, c1 (2) no."""
    _expect(B.OK, lambda d: setattr(d, "flags", B.FLAG_KV_IMAGE))
    _expect(B.OK, lambda d: setattr(d, "flags", B.FLAG_KV_INLINE))
    _expect(B.EINVAL, lambda d: setattr(d, "flags", B.FLAG_KV_IMAGE | B.FLAG_KV_INLINE))
    for name, default_image in (("c3", True), ("c1", False)):
        p = fa_inputs.make(name)
        # the walk-1 direction and the dS choice held fixed: the image alone differs
        rows = B.FLAG_WALK1_ROWS | B.FLAG_DS_RECOMPUTE
        img, inl, dflt = _ws(p, B.FLAG_KV_IMAGE | rows), _ws(p, B.FLAG_KV_INLINE | rows), _ws(p, rows)
        image_bytes = p.Hkv * ((p.M + 31) // 32) * 128 * p.D
        assert img.workspace_bytes - inl.workspace_bytes >= image_bytes
        assert img.workspace_bytes - inl.workspace_bytes < image_bytes + 256
        assert img.out_bytes == inl.out_bytes
        assert dflt.workspace_bytes == (img if default_image else inl).workspace_bytes


def test_centre_k_workspace():
    l0 = _ws(fa_inputs.make("c1_f32kv"), 0)
    l1 = _ws(fa_inputs.make("c1_f32kv"), B.FLAG_CENTER_K)
    assert l1.workspace_bytes >= l0.workspace_bytes + 4 * 2 * 128
    assert l1.out_bytes == l0.out_bytes


def test_noalloc_status_and_limit():
    assert "scratch" in fab.status_string(B.ESCRATCH)
    txt = open(os.path.join(ROOT, "include", "fa_back.h")).read()
    assert "#define FA_BACK_NOALLOC_MAX_WORKSPACE (64ull << 20)" in txt
    assert B.NOALLOC_MAX_WORKSPACE == 64 << 20
    lib = fab.load_library()
    assert lib.fa_back_run_noalloc(None, *([None] * 7)) == B.EINVAL


@pytest.mark.parametrize("typ,nbytes", [("q4_1", 20), ("q5_0", 22), ("q5_1", 24)])
def test_other_block_types_accepted_as_cache_only(typ, nbytes):
    # K and V may be any of the ggml block types (2-byte aligned rows of D/32 blocks of nbytes);
    # Q, dO and the mask may not
    p = fa_inputs.make_custom(name=typ, D=128, H=4, Hkv=2, N=20, M=70, mask="tail", k_type=typ,
                              v_type=typ)
    assert p.k.shape[-1] == 128 // 32 * nbytes
    d = B.describe(p)
    assert d.k.type == B.TYPE_IDS[typ] and d.k.nb[0] == nbytes
    lay = fab.fa_back_layout_query(d)
    assert lay.off_dv >= lay.off_dk + 4 * p.D * p.M * p.Hkv
    for field in ("q", "d", "mask"):
        _expect(B.EUNSUPPORTED, lambda dd, f=field: setattr(getattr(dd, f), "type", B.TYPE_IDS[typ]))
    # a row pitch that is odd breaks the 2-byte alignment of the fp16 fields
    d.k.nb[1] += 1
    d.k.nb[2] = d.k.nb[1] * p.M
    lay = B.Layout()
    assert fab.load_library().fa_back_layout_query(ctypes.byref(d), ctypes.byref(lay)) == B.ESTRIDE


def test_stored_ds_flags_and_workspace():
    """DS_STORE stores 2 bytes of dS per (row, key) pair of every 32-row block and 128-key tile
    (Hkv * ceil(G*N/32) * 4 * ceil(M/128) * 2048 bytes) and takes the image of the cache; it
    excludes DS_RECOMPUTE and KV_INLINE. Without a flag the plan stores dS when it takes the
    image."""
    _expect(B.EINVAL, lambda d: setattr(d, "flags", B.FLAG_DS_STORE | B.FLAG_DS_RECOMPUTE))
    _expect(B.EINVAL, lambda d: setattr(d, "flags", B.FLAG_DS_STORE | B.FLAG_KV_INLINE))
    _expect(B.OK, lambda d: setattr(d, "flags", B.FLAG_DS_RECOMPUTE | B.FLAG_KV_INLINE))
    p = fa_inputs.make("c3")   # 32 row tiles of 128 rows: the image by default
    rows = B.FLAG_WALK1_ROWS
    st, rc = _ws(p, B.FLAG_DS_STORE | rows), _ws(p, B.FLAG_DS_RECOMPUTE | rows)
    assert _ws(p, rows).workspace_bytes == st.workspace_bytes   # stored by default with the image
    c1 = fa_inputs.make("c1")   # 2 row tiles: no image, so recompute by default
    assert _ws(c1, 0).workspace_bytes == _ws(c1, B.FLAG_DS_RECOMPUTE).workspace_bytes
    ds_bytes = p.Hkv * (-(-(p.H // p.Hkv) * p.N // 32)) * 4 * (-(-p.M // 128)) * 2048
    assert st.workspace_bytes - rc.workspace_bytes >= ds_bytes
    assert st.out_bytes == rc.out_bytes


def test_layout_reports_the_plan():
    """plan_flags names the plan's choices: c1 (M = 2 G N, 2 row tiles) walks keys, decodes
    inline and recomputes dS; c3 (32 row tiles) walks rows over the image and stores dS; the
    flags override either, and a degenerate shape reports none."""
    F = B
    c1 = fab.fa_back_layout_query(B.describe(fa_inputs.make("c1"))).plan_flags
    assert c1 == F.FLAG_WALK1_KEYS | F.FLAG_KV_INLINE | F.FLAG_DS_RECOMPUTE
    c3 = fab.fa_back_layout_query(B.describe(fa_inputs.make("c3"))).plan_flags
    assert c3 == F.FLAG_WALK1_ROWS | F.FLAG_KV_IMAGE | F.FLAG_DS_STORE
    assert _ws(fa_inputs.make("c3"), F.FLAG_DS_RECOMPUTE).plan_flags & F.FLAG_DS_RECOMPUTE
    assert _ws(fa_inputs.make("c1"), F.FLAG_DS_STORE).plan_flags == (
        F.FLAG_WALK1_ROWS | F.FLAG_KV_IMAGE | F.FLAG_DS_STORE)
    empty = fa_inputs.make_custom(name="e", D=64, H=2, Hkv=1, N=4, M=0, mask="none")
    assert fab.fa_back_layout_query(B.describe(empty)).plan_flags == 0
