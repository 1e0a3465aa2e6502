"""The fused apply captured into a HIP graph: every replay equals the eager result.

The library records no memset and allocates nothing, so a serving loop can
capture it (atlas lora_delta.rs apply_lora_bgmv doc: graph-safe launches on
fixed addresses, seq_slot contents re-uploaded each step).  Replays run with
eager work and synchronisations between them, and the routing buffer is
rewritten between replays to check it is read at replay time.
"""
import numpy as np
import pytest

from adapter_lora_bgmv_amd import workloads as WL
from adapter_lora_bgmv_amd.harness import DeviceWorkload, bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("kind", ["decode", "segmented", "moe"])
def test_graph_replays_match_eager(kind):
    if kind == "decode":
        wl = WL.random_small(60, dtype="bf16", k=1024, n_out=256, n=40, n_slots=5, max_rank=16)
    elif kind == "segmented":
        wl = WL.random_small(61, dtype="bf16", k=512, n_out=128, n_slots=3, max_rank=32,
                             kind="segmented", seg_lens=[100, 0, 37, 64])
    else:
        wl = WL.random_small(62, dtype="bf16", k=256, n_out=128, n=33, n_slots=3, max_rank=16,
                             kind="moe", n_experts=6, top_k=2)
    dw = DeviceWorkload(wl)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dw.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = bf16_bits(dw.y).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dw.run()
    for _ in range(3):
        dw.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(dw.y), eager)
        dw.run()                      # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(dw.y), eager)
    if kind == "decode":
        # new routing contents, same buffer: the replay reads them
        dw.seq_slot.copy_(torch.roll(dw.seq_slot, 1))
        dw.run()
        torch.cuda.synchronize()
        eager2 = bf16_bits(dw.y).copy()
        assert not np.array_equal(eager2, eager)
        dw.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(dw.y), eager2)
