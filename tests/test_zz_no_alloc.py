"""The allocation-free block entry point (h3k_block_forward_noalloc) against the block call
with a caller workspace (h3k_block_forward): the same kernels on the same inputs, so the
outputs must be bitwise equal. Two calls in a row, the second with fewer tokens, so the
shared scratch array is reused with a different layout; each call's result is checked."""
import pytest
import torch

import synth_inputs as S
from tests._util import gpu_block

pytestmark = pytest.mark.gpu

h3k = pytest.importorskip("video_diffusion_transformer_03_amd.h3k")


def _case(grid, flags):
    import dataclasses
    wl = dataclasses.replace(S.WORKLOADS["tiny"], grid=grid)
    bw, _ = gpu_block(wl, 0, keep_bf16=bool(flags & h3k.F_BF16_GEMM))
    xdt = torch.float32 if flags & h3k.F_FP32_DEBUG else torch.bfloat16
    x = S.activations(wl).cuda().to(xdt)
    c = S.conditioning(wl).cuda()
    return wl, bw, x, c, h3k.dims_of(wl)


@pytest.mark.parametrize("flags", [0, h3k.F_FP32_DEBUG, h3k.F_ATTN_BF16, h3k.F_BF16_GEMM])
def test_noalloc_matches_workspace_call(flags):
    for grid in [(8, 8, 8), (2, 4, 8)]:  # 512 tokens, then 64
        wl, bw, x, c, dims = _case(grid, flags)
        ref = h3k.block_forward(x, c, bw, dims, flags)
        out = torch.empty_like(x)
        got = h3k.block_forward_noalloc(x, c, bw, dims, flags, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), (grid, flags)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    wl, bw, x, c, dims = _case((8, 8, 8), 0)
    # d = 5120 at L = 4096 needs ~0.5 GB of workspace: refused before any launch
    big = h3k.make_dims(5120, 40, 128, 20480, 5120, (4, 32, 32))
    need = h3k.workspace_bytes(big, 4096, 0)
    assert need > h3k.NOALLOC_MAX_BYTES
    rc = h3k.lib().h3k_block_forward_noalloc(
        x.data_ptr(), x.data_ptr(), c.data_ptr(), None, h3k.C.byref(big), 4096, 0, None)
    assert rc == h3k.EINVAL  # NULL weights are checked first
    wc = bw.c_struct()
    rc = h3k.lib().h3k_block_forward_noalloc(
        x.data_ptr(), x.data_ptr(), c.data_ptr(), h3k.C.byref(wc), h3k.C.byref(big), 4096, 0, None)
    assert rc == h3k.ENOSPC and "scratch" in h3k.last_error()
