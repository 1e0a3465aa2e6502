"""Bit-level invariants of the tiled (more than 64 rows) paths, through the C ABI.

* Skipped rows (slot -1, past the pool, NULL table entry, zero scale) are the
  base-only output bit for bit (ferrox-core "weight_matrix/lora.rs", module
  doc "Cost when absent" and test a_zero_scale_adds_nothing_bit_for_bit;
  atlas "lora_delta.rs", apply_lora_bgmv doc: a NULL or zero entry is a
  base-only slot), whatever tile a row lands in and whatever rank the pool
  has.
* A fused projection applied part by part, each part with its block of B's
  rows and one copy of A, equals the whole call bit for bit and the oracle
  element by element (frink-models "lora_attach.rs", module doc: B (A x)
  over stacked rows is the stacked B_i (A x)).
"""
import numpy as np
import pytest

import oracle
from adapter_lora_bgmv_amd import binding as B
from adapter_lora_bgmv_amd import workloads as WL
from adapter_lora_bgmv_amd.harness import DeviceWorkload, bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lora_init()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def check(y, ref, what):
    err = np.abs(np.asarray(y, np.float64) - ref)
    bad = ~(err <= 1e-2 * np.maximum(1.0, np.abs(ref)))
    assert not bad.any(), f"{what}: {int(bad.sum())} elements over 1e-2*max(1,|ref|)"


def _skipped(slots, st, null_slots=()):
    return np.array([not (0 <= s < len(st) and st[s] != 0 and s not in null_slots) for s in slots])


def test_gate_up_zero_scale_rows_are_base(orc):
    """The fused gate/up workload at full size (W 22016 x 4096, 256 rows, 32
    slots, a quarter of them at scale 0): every row on a zero-scale slot equals
    the base-only call bit for bit."""
    wl = WL.fused_gate_up()
    dw = DeviceWorkload(wl)
    routed = bf16_bits(dw.run().clone())
    base = bf16_bits(dw.run(route=False).clone())
    torch.cuda.synchronize()
    skip = _skipped(dw.seq_slot_host, dw.scale_table_host)
    assert skip.sum() >= 40
    assert np.array_equal(routed[skip], base[skip])
    assert (routed[~skip] != base[~skip]).mean() > 0.5


@pytest.mark.parametrize("seed,k,n_out,n,R", [
    (60, 2112, 1000, 300, 32),   # k stages that do not divide evenly over the workgroups
    (61, 1024, 2048, 520, 16),
    (62, 520, 264, 150, 48),     # a rank that does not divide 64, over 128 rows
    (63, 640, 1000, 300, 128),
    (64, 4096, 512, 129, 64),    # one row past the 128-row tiles
    (68, 4096, 1000, 400, 32),   # 256 x 256 tiles
    (69, 4096, 1000, 400, 48),   # 256 x 128 tiles (a rank that does not divide 64)
    (70, 2048, 1000, 100, 48),   # 128 x 128 tiles, two k ranges
])
def test_skip_rows_are_base_on_tiled_paths(orc, seed, k, n_out, n, R):
    """Rows that skip for every reason, scattered through a batch over 128 rows,
    are the base-only call's rows bit for bit; the routed rows match the oracle."""
    wl = WL.random_small(seed, dtype="bf16", k=k, n_out=n_out, n=n, n_slots=8, max_rank=R)
    st = B.lora_scale_table(wl.adapters)
    st[3] = 0.0  # a switched-off adapter
    dw = DeviceWorkload(wl, scale_table=st, null_slots=[5])
    rng = np.random.default_rng(seed)
    ss = rng.integers(0, 8, size=n).astype(np.int32)
    pick = rng.choice(n, size=n // 3, replace=False)
    ss[pick] = rng.choice([-1, -9, 3, 5, 8, 1000], size=len(pick))
    dw.seq_slot.copy_(torch.from_numpy(ss))
    routed = dw.run().clone()
    base = dw.run(route=False).clone()
    torch.cuda.synchronize()
    rb, bb = bf16_bits(routed), bf16_bits(base)
    skip = _skipped(ss, st, (5,))
    assert skip.sum() >= n // 4
    assert np.array_equal(rb[skip], bb[skip])
    ref = orc.apply(wl.W, oracle.Route(wl.A, wl.B, st, 1, wl.k_in, wl.n_out, wl.max_rank,
                                       null_slots=[5]), wl.x, ss, 1)
    check(dw.y_host(routed), ref, f"seed {seed}")


def test_skip_segments_are_base_on_the_segmented_path(orc):
    """A prefill batch whose segments sit on a switched-off slot, a NULL slot and
    slot -1 between routed ones: those segments' rows are the base-only rows."""
    wl = WL.random_small(65, dtype="bf16", k=1024, n_out=768, n_slots=5, max_rank=64,
                         kind="segmented", seg_lens=[200, 130, 70, 250, 90, 61])
    wl.seg_slot = np.array([0, 2, 1, -1, 3, 4], np.int32)
    st = B.lora_scale_table(wl.adapters)
    st[2] = 0.0
    dw = DeviceWorkload(wl, scale_table=st, null_slots=[3])
    routed = bf16_bits(dw.run().clone())
    base = bf16_bits(dw.run(route=False).clone())
    torch.cuda.synchronize()
    slots = np.repeat(wl.seg_slot, np.diff(wl.seg_indptr))
    skip = _skipped(slots, st, (3,))
    assert skip.sum() == 130 + 250 + 90
    assert np.array_equal(routed[skip], base[skip])


def test_skip_rows_are_base_on_the_moe_gather(orc):
    wl = WL.random_small(66, dtype="bf16", k=264, n_out=256, n=90, n_slots=4, max_rank=16,
                         kind="moe", n_experts=5, top_k=3)
    st = B.lora_scale_table(wl.adapters)
    st[1] = 0.0
    dw = DeviceWorkload(wl, scale_table=st)
    routed = bf16_bits(dw.run().clone())
    base = bf16_bits(dw.run(route=False).clone())
    torch.cuda.synchronize()
    slots = np.repeat(wl.token_slot, wl.top_k)
    skip = _skipped(slots, st)
    assert skip.sum() >= 30
    assert np.array_equal(routed[skip], base[skip])


def _half_call(dw, wl, h, half, y):
    r = B.DeviceRoute(dw.A, dw.Bp, dw.scale_table_host, n_out=half, b_row_offset=h * half)
    ws_bytes = B.lora_workspace_bytes(0, B.LORA_BF16, dw.n, half, wl.k_in, wl.max_rank)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    B.lora_apply(B.LORA_BF16, half, wl.k_in, dw.W[h * half:(h + 1) * half], wl.k_in, r, dw.x,
                 dw.x_row_stride, dw.seq_slot, dw.n, y[:, h * half:], y.shape[1], ws, ws_bytes)
    return ws


def test_gate_up_halves_match_the_oracle_and_the_whole(orc):
    """The fused gate/up workload run as its gate half and its up half (rows
    0..11007 and 11008..22015 of W and of every B, one copy of A each), each
    half writing its columns of the 22016-wide y rows: each half matches the
    oracle's half on sampled rows, and the two halves equal the whole call bit
    for bit."""
    wl = WL.fused_gate_up()
    half = wl.meta["half"]
    dw = DeviceWorkload(wl)
    whole = bf16_bits(dw.run().clone())
    y = torch.full_like(dw.y, float("nan"))
    keep = [_half_call(dw, wl, h, half, y) for h in range(2)]
    torch.cuda.synchronize()
    del keep
    split = bf16_bits(y)
    assert np.array_equal(split, whole)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(dw.n, size=12, replace=False)).astype(np.int32)
    got = dw.y_host(y)
    for h in range(2):
        r = orc.route_for(wl, dw.scale_table_host, b_row_offset=h * half, n_out=half)
        ref = orc.apply(wl.W[h * half:(h + 1) * half], r, wl.x, dw.seq_slot_host, 1, rows=rows)
        check(got[rows, h * half:(h + 1) * half], ref, f"half {h}")


@pytest.mark.parametrize("n,k,n_out,R", [(200, 1024, 1104, 32), (300, 2112, 1000, 64),
                                         (400, 4096, 1000, 16), (180, 4096, 1000, 48),
                                         (100, 4096, 1000, 32)])
def test_split_equals_stacked_on_tiled_paths(n, k, n_out, R):
    """Any cut of the output rows (not only halves), over 128 rows."""
    wl = WL.random_small(67 + n, dtype="bf16", k=k, n_out=n_out, n=n, n_slots=6, max_rank=R)
    dw = DeviceWorkload(wl)
    whole = bf16_bits(dw.run().clone())
    y = torch.full_like(dw.y, float("nan"))
    cuts = [0, 136, 400, n_out]
    keep = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        r = B.DeviceRoute(dw.A, dw.Bp, dw.scale_table_host, n_out=hi - lo, b_row_offset=lo)
        ws_bytes = B.lora_workspace_bytes(0, B.LORA_BF16, dw.n, hi - lo, k, R)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        B.lora_apply(B.LORA_BF16, hi - lo, k, dw.W[lo:hi], k, r, dw.x, dw.x_row_stride,
                     dw.seq_slot, dw.n, y[:, lo:], y.shape[1], ws, ws_bytes)
        keep.append(ws)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y), whole)
