"""The no-allocation GEMM entry point (gemm_bf16_noalloc, workspace in a library-owned device array) against
gemm_bf16 through the C ABI: two calls in a row, the second smaller, both with schedules that use the workspace
(a 2-way K split, then stream-K), each equal to gemm_bf16 bit for bit (same kernels, same fixed summation order)
and within the oracle's bound, and no workspace taken from the library's pool; and a shape whose built-in
schedule outgrows the array, run as 128 x 128 stream-K."""
import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
from implicit_gemm_conv_amd import inputs
from gpu_util import assert_close, host_values, oracle_gemm, say, synchronize, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    igc.lib()


def _call(fn, M, N, K, dA, dB):
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    igc.check(fn(M, N, K, dA, K, igc.ROW_MAJOR, dB, N, igc.ROW_MAJOR, C, N, igc.OUT_F32))
    synchronize()
    return C


def test_noalloc_matches_gemm_bf16():
    for (M, N, K, seed) in ((2048, 1024, 16384, 3), (1000, 512, 8192, 11)):
        t = igc.igc_default_tune(M, N, K)
        assert (t.stream_k > 0 or t.k_splits > 1) and igc.igc_workspace_bytes(igc.OP_GEMM, M, N, K) > 0
        A, lda, B, ldb = inputs.gemm_operands(M, N, K, "row", "row", dtype="bf16", a_dist=("normal", 1.0),
                                              b_dist=("normal", 1.0), seed=seed)
        dA, dB = to_dev(A), to_dev(B)
        say(f"noalloc {M}x{N}x{K}")
        before = igc.igc_pool_allocations()
        mine = _call(igc.gemm_bf16_noalloc, M, N, K, dA, dB)
        assert igc.igc_pool_allocations() == before, "gemm_bf16_noalloc took a pool workspace"
        ref_lib = _call(igc.gemm_bf16, M, N, K, dA, dB)
        assert torch.equal(mine, ref_lib), "gemm_bf16_noalloc differs from gemm_bf16"
        rows = np.random.default_rng(seed).integers(0, M, 3000)
        cols = np.random.default_rng(seed + 1).integers(0, N, 3000)
        import oracle
        ref, S = oracle.gemm_sample(M, N, K, A, lda, 0, B, ldb, 0, oracle.BF16, rows, cols)
        assert_close(host_values(mine)[rows, cols], ref, S, "f32", f"noalloc {M}x{N}x{K}")
    assert igc.igc_take_device_error() == 0


def test_noalloc_falls_back_to_stream_k():
    """A shape whose built-in schedule (8-way split of 256 x 128 tiles, 32 MiB of partials) outgrows the
    array: the no-allocation call runs 128 x 128 stream-K over 256 workgroups instead, equal bit for bit to
    that schedule run with a caller workspace, within the oracle's bound, and allocates nothing."""
    M, N, K = 1024, 1024, 65536
    t = igc.igc_default_tune(M, N, K)
    assert t.k_splits == 8 and igc.igc_workspace_bytes(igc.OP_GEMM, M, N, K) > (16 << 20) + 4096
    fits = igc.tune((128, 128, 64, 4, 8, 16, 0, 4, 0), stream_k=256)
    A, lda, B, ldb = inputs.gemm_operands(M, N, K, "row", "row", dtype="bf16", a_dist=("normal", 1.0),
                                          b_dist=("normal", 1.0), seed=17)
    dA, dB = to_dev(A), to_dev(B)
    say(f"noalloc fallback {M}x{N}x{K}")
    before = igc.igc_pool_allocations()
    mine = _call(igc.gemm_bf16_noalloc, M, N, K, dA, dB)
    assert igc.igc_pool_allocations() == before, "gemm_bf16_noalloc took a pool workspace"
    ws = torch.empty(igc.igc_workspace_bytes(igc.OP_GEMM, M, N, K, fits), dtype=torch.uint8, device="cuda")
    ref_lib = _call(lambda *a: igc.gemm_bf16_ex(*a, fits, ws), M, N, K, dA, dB)
    assert torch.equal(mine, ref_lib), "gemm_bf16_noalloc differs from 128 x 128 stream-K"
    rows = np.random.default_rng(17).integers(0, M, 3000)
    cols = np.random.default_rng(18).integers(0, N, 3000)
    import oracle
    ref, S = oracle.gemm_sample(M, N, K, A, lda, 0, B, ldb, 0, oracle.BF16, rows, cols)
    assert_close(host_values(mine)[rows, cols], ref, S, "f32", f"noalloc fallback {M}x{N}x{K}")
    assert igc.igc_take_device_error() == 0
