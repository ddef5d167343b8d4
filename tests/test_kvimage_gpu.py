"""The decoded image of the cache (FA_BACK_FLAG_KV_IMAGE: K and V decoded once into the
workspace, the query-side walks copy tiles from it) against per-workgroup decoding
(FA_BACK_FLAG_KV_INLINE): bitwise the same outputs. The cases cover every decode the walks
have (q8_0 pairs with 16-byte and other row strides, q4_0 / q8_0 mixes, a block type beside an
F16 row type, the q4_1 / q5_0 / q5_1 blocks, F32 / BF16 rows, centred F16 rows), the three head sizes, ragged caches, stored
and dead mask rows, key-range splits (the walks start mid-cache) and both directions of the
walk that forms LSE and delta (the row-owned one reads the image too)."""
import dataclasses

import numpy as np
import pytest

import fa_inputs
from flash_attention_backward_amd import fa_back as B
from tests.gpu_util import KEYS, run_gpu, say, walk1

CASES = [
    dict(name="img_q8_256", D=256, H=8, Hkv=2, N=70, M=300, mask="tail", k_type="q8_0", v_type="q8_0"),
    dict(name="img_q8_128", D=128, H=6, Hkv=2, N=45, M=203, mask="random", Hm=6,
         masked_rows=[(0, 5), (4, 36)], k_type="q8_0", v_type="q8_0"),
    dict(name="img_q8_64", D=64, H=4, Hkv=4, N=50, M=130, mask="tail", k_type="q8_0", v_type="q8_0"),
    dict(name="img_q4q8_128", D=128, H=4, Hkv=1, N=40, M=257, mask="tail", k_type="q4_0", v_type="q8_0"),
    dict(name="img_q8f16_128", D=128, H=4, Hkv=2, N=33, M=190, mask="none", k_type="q8_0", v_type="f16"),
    dict(name="img_f32bf16_64", D=64, H=4, Hkv=2, N=37, M=99, mask="random", Hm=4, k_type="f32",
         v_type="bf16"),
    dict(name="img_f16_centred_256", D=256, H=4, Hkv=2, N=40, M=129, mask="tail", k_type="f16",
         v_type="f16", k_offset=3.0, k_spread=0.01, v_offset=2.0, v_spread=0.01,
         flags=B.FLAG_CENTER_K | B.FLAG_CENTER_V),
    dict(name="img_split_128", D=128, H=4, Hkv=1, N=64, M=2048, mask="tail", k_type="q8_0", v_type="q8_0"),
    dict(name="img_q5_1q4_1_256", D=256, H=8, Hkv=2, N=70, M=300, mask="tail", k_type="q5_1", v_type="q4_1"),
    dict(name="img_q5_0f16_64", D=64, H=4, Hkv=2, N=50, M=130, mask="random", Hm=4, k_type="q5_0",
         v_type="f16"),
]


def _with(p, bit):
    # dQ by walk 2 in both runs (stored dS, which the plan takes with the image, rounds dS with
    # another exponent and is checked against the oracle elsewhere)
    both = B.FLAG_KV_IMAGE | B.FLAG_KV_INLINE | B.FLAG_DS_STORE
    return dataclasses.replace(p, flags=(p.flags & ~both) | bit | B.FLAG_DS_RECOMPUTE)


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["rows", "keys"])
@pytest.mark.parametrize("cfg", CASES, ids=[c["name"] for c in CASES])
def test_image_matches_inline_decode(cfg, mode):
    p = walk1(fa_inputs.make_custom(**cfg), mode)
    say(f"[gpu] {p.name} ({mode}): image, then inline")
    img, _, lay_i = run_gpu(_with(p, B.FLAG_KV_IMAGE))
    inl, _, lay_n = run_gpu(_with(p, B.FLAG_KV_INLINE))
    assert lay_i.workspace_bytes > lay_n.workspace_bytes   # the image is in the workspace
    for k in KEYS:
        a = np.asarray(img[k])
        b = np.asarray(inl[k])
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), k
