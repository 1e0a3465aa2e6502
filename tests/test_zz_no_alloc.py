"""lora_apply_noalloc, the entry point for callers that cannot allocate,
against lora_apply with a workspace, through the C ABI: the same bits on
calls in a row that change shape and path (the decode kernel, the tiled
GEMM, base-only, f32), each later call smaller than one before it, so that
what an earlier call left in the shared scratch array cannot leak into a
later result."""
import numpy as np
import pytest

from adapter_lora_bgmv_amd import binding as B
from adapter_lora_bgmv_amd import workloads as WL
from adapter_lora_bgmv_amd.harness import DeviceWorkload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lora_init()


def _bits(y):
    return y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _both(dw, route=True):
    """(lora_apply's y, lora_apply_noalloc's y), each in a NaN-filled buffer."""
    wl = dw.wl
    ref = torch.full_like(dw.y, float("nan"))
    dw.run(route=route, y=ref)
    got = torch.full_like(dw.y, float("nan"))
    B.lora_apply_noalloc(dw.dtype, wl.n_out, wl.k_in, dw.W, wl.k_in, dw.route if route else None, dw.x,
                         dw.x_row_stride, dw.seq_slot if route else None, dw.n, got, dw.y_row_stride)
    torch.cuda.synchronize()
    return _bits(ref), _bits(got)


def _check(dw, what, route=True):
    ref, got = _both(dw, route)
    assert np.array_equal(ref, got), f"{what}: {int((ref != got).sum())} elements differ"


def test_two_calls_in_a_row_the_second_smaller():
    """The decode workload (64 rows, W 4096 x 4096, 16 rank-16 slots), then a
    smaller decode batch (20 rows, 520 x 264, rank 32)."""
    _check(DeviceWorkload(WL.decode_bgmv()), "decode 64 x 4096 x 4096")
    _check(DeviceWorkload(WL.random_small(81, k=520, n_out=264, n=20, n_slots=5, max_rank=32)),
           "decode 20 x 264 x 520")


def test_calls_that_change_path_and_shape():
    """Tiled GEMM (300 rows, split-k free 256-row tiles), a 100-row split-k
    GEMM, a decode batch whose tiles' counters the GEMM calls' data has
    overwritten, base-only, then f32."""
    big = DeviceWorkload(WL.random_small(82, k=2112, n_out=1000, n=300, n_slots=6, max_rank=64))
    _check(big, "gemm 300 x 1000 x 2112")
    _check(DeviceWorkload(WL.random_small(83, k=4096, n_out=1000, n=100, n_slots=6, max_rank=48)),
           "split-k gemm 100 x 1000 x 4096")
    dec = DeviceWorkload(WL.random_small(84, k=2048, n_out=2048, n=48, n_slots=8, max_rank=16))
    _check(dec, "decode 48 x 2048 x 2048")
    _check(dec, "decode again")
    _check(big, "gemm base only", route=False)
    _check(DeviceWorkload(WL.single_projection_f32()), "f32 4 x 256 x 256")


def test_under_graph_capture():
    """Captured with the counter clear, replayed three times with eager calls
    of another shape between the replays: every replay equals lora_apply."""
    dw = DeviceWorkload(WL.decode_bgmv())
    other = DeviceWorkload(WL.random_small(85, k=1024, n_out=512, n=200, n_slots=4, max_rank=16))
    wl = dw.wl
    ref = torch.full_like(dw.y, float("nan"))
    dw.run(y=ref)
    got = torch.full_like(dw.y, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.lora_apply_noalloc(dw.dtype, wl.n_out, wl.k_in, dw.W, wl.k_in, dw.route, dw.x, dw.x_row_stride,
                             dw.seq_slot, dw.n, got, dw.y_row_stride, s)
    torch.cuda.synchronize()
    want = _bits(ref)
    for i in range(3):
        got.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got), want), f"replay {i}"
        _check(other, f"eager GEMM call after replay {i}")
