"""GPU tests of the schedules around the mainloop: the stream-K bounded wait failing loudly, caller-owned
workspaces (no allocation, same bits as the library's pool), and stream-K calls captured in HIP graphs and
replayed with changed inputs (flags are cleared by a kernel inside the graph, so stale
flags of an earlier replay never count as raised).  Results are compared with the CPU oracle or, where the
schedule is the thing under test, with the eager call bit for bit (the summation order is fixed)."""
import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
from implicit_gemm_conv_amd import inputs
from gpu_util import LAYOUT, assert_close, host_values, oracle_gemm, say, synchronize, to_dev

pytestmark = pytest.mark.gpu

BIG, SMALL = (256, 256, 32, 4, 8, 16, 0, 4, 0), (128, 128, 64, 4, 4, 32, 0, 4, 0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    igc.lib()
    yield
    igc.igc_debug_stream_k(0, -1)


def _gemm(M, N, K, dA, dB, tune=None, ws=None, out=torch.float32):
    C = torch.full((M, N), float("nan"), dtype=out, device="cuda")
    igc.check(igc.gemm_bf16_ex(M, N, K, dA, K, igc.ROW_MAJOR, dB, N, igc.ROW_MAJOR, C, N,
                               igc.OUT_F32 if out == torch.float32 else igc.OUT_BF16, tune, ws))
    return C


def test_stream_k_wait_gives_up_loudly():
    """A partial whose flag never rises (test hook) makes the owner's bounded wait give up: every kernel still
    exits, the owner's tile is written as NaN, the device error word is set, and every other tile is right."""
    M = N = 512
    K = 4096  # 4 tiles of 256 x 256, 32 K units of 128 each; 8 workgroups: each tile shared by two
    A, lda, B, ldb = inputs.gemm_operands(M, N, K, "row", "row", dtype="bf16", seed=90)
    ref, S = oracle_gemm(M, N, K, A, lda, "row", B, ldb, "row")
    dA, dB = to_dev(A), to_dev(B)
    assert igc.igc_take_device_error() == 0
    try:
        igc.igc_debug_stream_k(2000, 0)  # workgroup 0 never raises its flag; its tile's owner is workgroup 1
        say("stream-K with a dropped flag")
        C = _gemm(M, N, K, dA, dB, igc.tune(BIG, stream_k=8))
        synchronize()
    finally:
        igc.igc_debug_stream_k(0, -1)
    y = host_values(C)
    assert igc.igc_take_device_error() == 1
    nan = np.isnan(y)
    assert nan[:256, :256].all(), "the owner's tile is not marked"
    assert not nan[256:, :].any() and not nan[:, 256:].any(), "NaN outside the owner's tile"
    assert_close(y[256:, :], ref[256:, :], S[256:, :], "f32", "tiles below")
    assert_close(y[:256, 256:], ref[:256, 256:], S[:256, 256:], "f32", "tiles beside")
    # the hook is off again: a normal run is right and leaves the error word clear
    say("stream-K after the hook")
    C = _gemm(M, N, K, dA, dB, igc.tune(BIG, stream_k=8))
    synchronize()
    assert_close(host_values(C), ref, S, "f32", "stream-K after the hook")
    assert igc.igc_take_device_error() == 0


@pytest.mark.parametrize("shape,tune", [
    ((2048, 1024, 16384), None),                                  # built-in: 128 x 128, K split in two
    ((1024, 1024, 8192), None),                                   # built-in: 128 x 128 stream-K over 256
    ((1000, 1000, 6144), igc.Tune(*SMALL[:8], 5, 0, 0, 0)),       # K split into 5
    ((1300, 1104, 2304), igc.Tune(*BIG[:8], 1, 8, 0, 1)),         # hybrid: 2 data-parallel rounds + tail
])
def test_caller_workspace(shape, tune):
    """A caller-owned workspace gives the same bits as the library's pool, and the call allocates nothing."""
    M, N, K = shape
    A, lda, B, ldb = inputs.gemm_operands(M, N, K, "row", "row", dtype="bf16", seed=91)
    dA, dB = to_dev(A), to_dev(B)
    need = igc.igc_workspace_bytes(igc.OP_GEMM, M, N, K, tune)
    assert need > 0
    say(f"workspace {shape}: {need} bytes")
    ref_pool = _gemm(M, N, K, dA, dB, tune)
    synchronize()
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)  # stale contents: flags must be cleared by the call itself
    before = igc.igc_pool_allocations()
    for _ in range(2):
        mine = _gemm(M, N, K, dA, dB, tune, ws)
        synchronize()
        assert torch.equal(mine, ref_pool)
    assert igc.igc_pool_allocations() == before, "a call given a workspace allocated one"
    short = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    st = igc.gemm_bf16_ex(M, N, K, dA, K, igc.ROW_MAJOR, dB, N, igc.ROW_MAJOR, mine, N, igc.OUT_F32, tune, short)
    assert st == igc.IGC_ERR_INVALID_VALUE


def test_conv_caller_workspace():
    """The 3x3 workload under the hybrid schedule (256 whole tiles in one data-parallel round, the other 136 split
    by stream-K) with a caller workspace equals the pool path bit for bit and allocates nothing."""
    name = "conv_bf16_n32_56x56_c256_k256_3x3"
    c = inputs.WORKLOADS[name]
    x, w = inputs.workload_operands(name)
    dx, dw = to_dev(x), to_dev(w)
    M, Ng, Kg = igc.conv_gemm_view(igc.OP_CONV_FPROP, c["N"], c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], 1, 1,
                                   1, 1)
    tune = igc.tune(BIG, stream_k=256, sk_hybrid=1)
    need = igc.igc_workspace_bytes(igc.OP_CONV_FPROP, M, Ng, Kg, tune)
    assert need > 0
    outs = []
    for ws in (None, torch.empty(need, dtype=torch.uint8, device="cuda")):
        before = igc.igc_pool_allocations()
        y = torch.full((M * Ng,), float("nan"), dtype=torch.bfloat16, device="cuda")
        igc.check(igc.conv2d_nhwc_implicit_gemm_ex(c["N"], c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], 1, 1, 1, 1,
                                                   1, 1, dx, dw, y, igc.OUT_BF16, tune, ws))
        synchronize()
        assert (igc.igc_pool_allocations() == before) == (ws is not None)
        outs.append(y)
    assert torch.equal(outs[0], outs[1])
    assert not torch.isnan(outs[0].float()).any()


def test_stream_k_graph_replay():
    """A built-in stream-K call (1024 x 1024 x 4096: 64 tiles of 128 x 128 over 256 workgroups; a 4-way split
    would leave 1024 of K per split) captured in a HIP graph with a caller workspace, replayed with new inputs
    each time, eager work and synchronisation between replays: every replay equals the eager call on the same
    inputs bit for bit."""
    M, N, K = 1024, 1024, 4096
    t = igc.igc_default_tune(M, N, K)
    assert t.stream_k > 0
    need = igc.igc_workspace_bytes(igc.OP_GEMM, M, N, K)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dA = torch.empty(M * K, dtype=torch.int16, device="cuda")
    dB = torch.empty(K * N, dtype=torch.int16, device="cuda")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def call():
        igc.check(igc.gemm_bf16_ex(M, N, K, dA, K, igc.ROW_MAJOR, dB, N, igc.ROW_MAJOR, C, N, igc.OUT_F32, None, ws))

    def load(seed):
        A, _, B, _ = inputs.gemm_operands(M, N, K, "row", "row", dtype="bf16", seed=seed)
        dA.copy_(torch.from_numpy(A.view(np.int16).ravel()))
        dB.copy_(torch.from_numpy(B.view(np.int16).ravel()))

    load(200)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    synchronize()
    for r, seed in enumerate((201, 202, 203)):
        load(seed)
        call()
        synchronize()
        eager = C.clone()
        C.fill_(float("nan"))
        synchronize()
        say(f"graph replay {r}")
        graph.replay()
        synchronize()
        assert torch.equal(C, eager), f"replay {r} differs from the eager call"
    assert igc.igc_take_device_error() == 0


@pytest.mark.skip(reason="the per-stream workspace cache was taken out: the GPU run that added it and the capture "
                         "test below faulted (illegal address) in the no-allocation test that runs after them")
def test_cached_workspace_per_stream():
    """Without a caller workspace, the first split call on a stream takes a workspace and later calls on that
    stream reuse it (no allocation); a larger need grows it once; another stream gets its own; after
    igc_release_workspaces the next call takes a new one.  Every result equals the caller-workspace run bit for
    bit."""
    M, N, K = 1024, 512, 4096
    t4, t8 = igc.Tune(*SMALL[:8], 4, 0, 0, 0), igc.Tune(*SMALL[:8], 8, 0, 0, 0)  # K split into 4 and 8
    A, lda, B, ldb = inputs.gemm_operands(M, N, K, "row", "row", dtype="bf16", seed=93)
    dA, dB = to_dev(A), to_dev(B)
    synchronize()
    assert igc.igc_release_workspaces() == igc.IGC_OK

    def call(tune, ws=None):
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        igc.check(igc.gemm_bf16_ex(M, N, K, dA, lda, igc.ROW_MAJOR, dB, ldb, igc.ROW_MAJOR, C, N, igc.OUT_F32,
                                   tune, ws))
        return C

    refs = {}
    for t in (t4, t8):
        need = igc.igc_workspace_bytes(igc.OP_GEMM, M, N, K, t)
        refs[t.k_splits] = call(t, torch.empty(need, dtype=torch.uint8, device="cuda"))
    synchronize()
    base = igc.igc_pool_allocations()
    steps = [(t4, 1), (t4, 1), (t4, 1), (t8, 2), (t4, 2)]  # (tune, allocations so far): t8 needs twice t4's
    for i, (t, want) in enumerate(steps):
        say(f"cached workspace step {i}: k_splits={t.k_splits}")
        y = call(t)
        synchronize()
        assert igc.igc_pool_allocations() - base == want, f"step {i}"
        assert torch.equal(y, refs[t.k_splits]), f"step {i}"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        other = call(t4)
    torch.cuda.current_stream().wait_stream(side)
    synchronize()
    assert igc.igc_pool_allocations() - base == 3, "another stream shares the workspace"
    assert torch.equal(other, refs[4])
    assert igc.igc_release_workspaces() == igc.IGC_OK
    again = call(t4)
    synchronize()
    assert igc.igc_pool_allocations() - base == 4
    assert torch.equal(again, refs[4])


@pytest.mark.skip(reason="faulted the GPU (illegal address, reported in the no-allocation test that runs after it) "
                         "while the library took a pool workspace inside the capture; such calls are now refused "
                         "with IGC_ERR_UNSUPPORTED, and this case stays off the GPU until the cause is shown")
def test_graph_capture_without_workspace():
    """A stream-K call with no caller workspace captured in a HIP graph: under capture the workspace comes from
    the pool as graph nodes (not from the stream's cached one); every replay with new inputs equals the eager
    call bit for bit."""
    M, N, K = 1024, 1024, 8192
    assert igc.igc_default_tune(M, N, K).stream_k > 0
    dA = torch.empty(M * K, dtype=torch.int16, device="cuda")
    dB = torch.empty(K * N, dtype=torch.int16, device="cuda")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def call():
        igc.check(igc.gemm_bf16(M, N, K, dA, K, igc.ROW_MAJOR, dB, N, igc.ROW_MAJOR, C, N, igc.OUT_F32))

    def load(seed):
        A, _, B, _ = inputs.gemm_operands(M, N, K, "row", "row", dtype="bf16", seed=seed)
        dA.copy_(torch.from_numpy(A.view(np.int16).ravel()))
        dB.copy_(torch.from_numpy(B.view(np.int16).ravel()))

    load(210)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside the capture: creates the pool
    torch.cuda.current_stream().wait_stream(side)
    synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    synchronize()
    for r, seed in enumerate((211, 212)):
        load(seed)
        call()
        synchronize()
        eager = C.clone()
        C.fill_(float("nan"))
        synchronize()
        say(f"graph replay without workspace {r}")
        graph.replay()
        synchronize()
        assert torch.equal(C, eager), f"replay {r} differs from the eager call"
    assert igc.igc_take_device_error() == 0
