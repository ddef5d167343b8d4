"""fa_back_run_noalloc on the GPU, through the C ABI: the entry point that allocates nothing and
uses the library's static scratch as its workspace. Its output must equal fa_back_run's (the same
kernels on the same inputs: bitwise) and meet the oracle bar, on two calls in a row, the second
with a smaller problem (the scratch keeps the first call's contents), and a plan whose workspace
exceeds the scratch is refused before anything runs."""
import dataclasses

import numpy as np
import pytest

import fa_inputs
import flash_attention_backward_amd as fab
from flash_attention_backward_amd import fa_back as B
from oracle import fa_back_oracle as O
from tests.gpu_util import compare, say

pytestmark = pytest.mark.gpu


def _both(p):
    """(fa_back_run's packed output, fa_back_run_noalloc's) as bytes, on the same buffers."""
    import torch
    dp = fab.DeviceProblem(p, "cuda:0", poison=True)
    try:
        assert dp.layout.workspace_bytes <= B.NOALLOC_MAX_WORKSPACE
        dp.run()
        torch.cuda.synchronize()
        ref = dp.out.cpu().numpy().copy()
        dp.out.fill_(0xFF)   # NaN bytes: any defined byte the no-alloc call leaves unwritten shows up
        torch.cuda.synchronize()
        dp.run_noalloc()
        torch.cuda.synchronize()
        got = dp.out.cpu().numpy().copy()
        return ref, got, dp.layout
    finally:
        dp.close()


def test_noalloc_equals_run_twice_second_smaller():
    for name in ("c3", "c1_causal"):            # 49 MiB of workspace, then 0.8 MiB
        # dQ by walk 2: the stored dS tiles (64 MiB for c3) would not fit the scratch
        p = dataclasses.replace(fa_inputs.make(name), flags=B.FLAG_DS_RECOMPUTE)
        say(f"[gpu] noalloc {name}: N={p.N} M={p.M} H={p.H}")
        ref, got, lay = _both(p)
        assert np.array_equal(B.defined_bytes(got, lay, p), B.defined_bytes(ref, lay, p)), name
        errs = compare(B.unpack(got, lay, p), O.run_problem(p))
        say("   nmse " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_noalloc_refuses_a_larger_workspace():
    p = fa_inputs.make("c4n16")
    dp = fab.DeviceProblem(p, "cuda:0", poison=True)
    try:
        assert dp.layout.workspace_bytes > B.NOALLOC_MAX_WORKSPACE
        with pytest.raises(B.FaBackError) as e:
            dp.run_noalloc()
        assert e.value.status == B.ESCRATCH
    finally:
        dp.close()
