"""q8_0 caches at D = 256 whose rows are padded (a row pitch that is not a multiple of 16 bytes)
or whose head bases start off a 16-byte boundary give exactly the bits of the contiguous cache.
Such layouts move every row's alignment inside the staged tiles: a pitch that is not a multiple
of 16 takes the general staging arithmetic of walk 2, a multiple of 16 with an offset base the
fixed-stride one with a non-zero misalignment, and the walk-1 and key-side setups both. Run
through the C ABI with the cache copied into a padded device buffer and the descriptor's
strides set to match (the Python binding itself only uploads contiguous storage)."""
import numpy as np
import pytest

import fa_inputs
from flash_attention_backward_amd import fa_back as F
from tests.gpu_util import KEYS, run_gpu, say, walk1


def padded_cache(x, pitch, offset):
    """The (Hkv, M, row bytes) q8_0 cache x laid out with row pitch `pitch` bytes and its first
    head starting `offset` bytes into a flat uint8 buffer (head stride M * pitch)."""
    hkv, m, rb = x.shape
    assert pitch >= rb
    buf = np.full(offset + hkv * m * pitch + 64, 0xA5, dtype=np.uint8)
    view = buf[offset: offset + hkv * m * pitch].reshape(hkv, m, pitch)
    view[:, :, :rb] = np.ascontiguousarray(x).view(np.uint8).reshape(hkv, m, rb)
    return buf


def run_layout(p, pitch, offset):
    import torch
    dev = torch.device("cuda:0")
    desc = F.describe(p)
    for t in (desc.k, desc.v):
        t.nb[1] = pitch
        t.nb[2] = p.M * pitch
    plan, lay = F.fa_back_create(desc, 0)
    try:
        dp = F.DeviceProblem(p, dev, poison=False)   # q, dO and the mask, contiguous
        kb = torch.from_numpy(padded_cache(p.k, pitch, offset)).to(dev)
        vb = torch.from_numpy(padded_cache(p.v, pitch, offset)).to(dev)
        out = torch.full((int(lay.out_bytes),), 0xFF, dtype=torch.uint8, device=dev)
        ws = torch.full((int(lay.workspace_bytes),), 0xFF, dtype=torch.uint8, device=dev)
        m = dp.bufs["mask"]
        F.fa_back_run(plan, dp.bufs["q"].data_ptr(), kb.data_ptr() + offset, vb.data_ptr() + offset,
                      dp.bufs["d"].data_ptr(), None if m is None else m.data_ptr(), out.data_ptr(),
                      ws.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
        torch.cuda.synchronize()
        res = F.unpack(out.cpu().numpy(), lay, p)
        dp.close()
        return res
    finally:
        F.fa_back_destroy(plan)


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["rows", "keys"])
@pytest.mark.parametrize("pitch,offset", [(274, 6), (288, 8), (272, 2)])
def test_q8_cache_layouts_bitwise(pitch, offset, mode):
    p = walk1(fa_inputs.make_custom("lay256", D=256, H=4, Hkv=2, N=40, M=300, mask="tail",
                                    k_type="q8_0", v_type="q8_0"), mode)
    assert p.k.shape[-1] == 272 and p.v.shape[-1] == 272
    ref, _, _ = run_gpu(p)
    say(f"[gpu] lay256 pitch {pitch} offset {offset} ({mode})")
    got = run_layout(p, pitch, offset)
    for k in KEYS:
        assert np.array_equal(np.asarray(got[k]).view(np.uint32), np.asarray(ref[k]).view(np.uint32)), k
