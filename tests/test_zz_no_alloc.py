"""The allocation-free routing entry point (moe_build_blocks_noalloc) against
moe_build_blocks with a caller workspace, through the C ABI: bit-exact outputs
on two calls in a row, the second with a smaller problem (its scratch keeps the
first call's contents), at the largest expert count its scratch holds, and on
a side stream; and the expert-count limit refused before any launch."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _topk(rng, T, K, E, drop=0.0):
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    if drop:
        topk[rng.random(topk.shape) < drop] = -1
    return topk


def _both(topk, E, B, N, stream=None):
    import mxfp8_grouped_gemm_amd as mx
    L = mx.lib()
    T, K = topk.shape
    tk = torch.from_numpy(topk).cuda()
    ref = mx.moe_build_blocks(tk, E, B, N)
    tp = torch.full((N * B,), 12345, dtype=torch.int32, device="cuda")
    be = torch.full((N,), 12345, dtype=torch.int32, device="cuda")
    st = None if stream is None else C.c_void_p(stream.cuda_stream)
    rc = L.moe_build_blocks_noalloc(C.c_void_p(tk.data_ptr()), T, K, E, B, N, C.c_void_p(tp.data_ptr()),
                                    C.c_void_p(be.data_ptr()), st)
    assert rc == 0, mx.last_error()
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in ref], [tp.cpu().numpy(), be.cpu().numpy()]


def test_noalloc_build_blocks_matches_the_workspace_entry_point():
    import mxfp8_grouped_gemm_amd as mx
    rng = np.random.default_rng(71)
    cases = [(6000, 8, 128, 128, 0.0),      # many chunks and experts
             (300, 2, 16, 256, 0.2),         # smaller: fewer experts and chunks, dropped selections
             (1024, 4, 4096, 128, 0.0),      # the largest expert count the scratch holds
             (200, 1, 3, 1024, 0.0)]         # smallest again, after the largest
    for T, K, E, B, drop in cases:
        print("noalloc case", (T, K, E, B, drop), flush=True)
        topk = _topk(rng, T, K, E, drop)
        N = oracle.num_blocks(T, K, E, B) + 1
        (rt, rb), (gt, gb) = _both(topk, E, B, N)
        assert np.array_equal(gt, rt) and np.array_equal(gb, rb), (T, K, E, B)
        ot, ob = oracle.build_blocks(topk, E, B, N)
        assert np.array_equal(gt, ot) and np.array_equal(gb, ob), (T, K, E, B)
    # on a side stream, with work already queued there
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        topk = _topk(rng, 2048, 2, 64)
        N = oracle.num_blocks(2048, 2, 64, 128)
        (rt, rb), (gt, gb) = _both(topk, 64, 128, N, stream=s)
    assert np.array_equal(gt, rt) and np.array_equal(gb, rb)
    # the wrapper of the same name
    tk = torch.from_numpy(topk).cuda()
    out = (torch.empty(N * 128, dtype=torch.int32, device="cuda"), torch.empty(N, dtype=torch.int32, device="cuda"))
    mx.moe_build_blocks_noalloc(tk, 64, 128, N, out)
    torch.cuda.synchronize()
    assert np.array_equal(out[0].cpu().numpy(), rt) and np.array_equal(out[1].cpu().numpy(), rb)


def test_noalloc_build_blocks_refuses_more_experts_than_its_scratch():
    import mxfp8_grouped_gemm_amd as mx
    L = mx.lib()
    fake = C.c_void_p(0x10000)
    assert L.moe_build_blocks_noalloc(fake, 8192, 1, 4097, 128, 4200, fake, fake, None) == 2
    assert "4096" in mx.last_error()
