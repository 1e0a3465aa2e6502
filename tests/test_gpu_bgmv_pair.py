"""The standalone two-step delta (lora_shrink, then lora_expand_fold) on the
by-slot kernels and their fallbacks, through the C ABI, against the oracle
(atlas "lora_delta.rs", apply_lora_bgmv doc: kernel 1 the shrink, kernel 2
the expand-and-fold; ferrox-core "weight_matrix/lora.rs", LoraDelta project
and accumulate).

Rows that do not resolve (slot -1, past the pool, a NULL table entry, a zero
scale) are never written: their t keeps its NaN sentinel and their y its
input bits.
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


def check(got, ref, rel, what):
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = ~(err <= rel * np.maximum(1.0, np.abs(ref)))
    assert not bad.any(), f"{what}: {int(bad.sum())} elements over {rel}*max(1,|ref|), max err {err.max():.3e}"


def _workload(seed, k, n_out, n, n_slots, R, slots=None):
    wl = WL.random_small(seed, dtype="bf16", k=k, n_out=n_out, n=n, n_slots=n_slots, max_rank=R)
    st = B.lora_scale_table(wl.adapters)
    if n_slots > 2:
        st[1] = 0.0  # a switched-off adapter
    dw = DeviceWorkload(wl, scale_table=st, null_slots=[2] if n_slots > 3 else None)
    if slots is not None:  # the device buffer and the host copy the checks read
        dw.seq_slot.copy_(torch.from_numpy(np.asarray(slots, np.int32)))
        dw.seq_slot_host = np.asarray(slots, np.int32)
    return wl, dw


def _resolved(dw, null=(2,)):
    st = dw.scale_table_host
    return np.array([0 <= s < len(st) and st[s] != 0 and not (len(st) > 3 and s in null)
                     for s in dw.seq_slot_host])


def _route(orc, wl, dw):
    return orc.route_for(wl, dw.scale_table_host, null_slots=[2] if len(dw.scale_table_host) > 3 else None)


@pytest.mark.parametrize("seed,k,n,n_slots,R,many", [
    (90, 4096, 64, 16, 16, False),   # the decode batch's shape
    (91, 520, 200, 7, 48, False),    # ragged k, rank 48, rows over 64 in the scan
    (92, 2048, 100, 3, 128, True),   # many rows per slot: row chunks of eight, rank 128
    (93, 8200, 5, 4, 16, False),     # k past one 8192-column pass of the four waves
    (94, 64, 1, 4, 32, False),       # one row
    (95, 1024, 1024, 5, 16, True),   # the most rows the by-slot path takes
    (96, 1024, 1030, 5, 16, True),   # past it: the k-split prep shrink units
])
def test_shrink_by_slot(orc, seed, k, n, n_slots, R, many):
    slots = None
    if many:
        rng = np.random.default_rng(seed)
        slots = rng.choice([0, 3, 3, 4, -1, 9], size=n).astype(np.int32)
    wl, dw = _workload(seed, k, 64, n, n_slots, R, slots)
    t = torch.full((dw.n, R), float("nan"), dtype=torch.float32, device="cuda")
    B.lora_shrink(dw.route, dw.x, dw.x_row_stride, dw.seq_slot, dw.n, t)
    torch.cuda.synchronize()
    got = t.cpu().numpy().astype(np.float64)
    live = _resolved(dw)
    assert np.all(np.isnan(got[~live])), "a row that does not resolve was written"
    assert not np.any(np.isnan(got[live])), "a resolved row was not written"
    ref = orc.shrink(_route(orc, wl, dw), wl.x, dw.seq_slot_host)
    check(got[live], ref[live], 1e-4, f"shrink seed {seed}")


@pytest.mark.parametrize("seed,n_out,n,n_slots,R,col", [
    (100, 4096, 64, 16, 16, 0),      # the decode batch's shape
    (101, 520, 37, 5, 16, 0),        # a 512-output chunk and an 8-output tail
    (102, 1000, 200, 6, 64, 0),      # rank 64: B read again per row from the cache
    (103, 264, 9, 4, 128, 0),        # rank 128
    (104, 512, 1024, 5, 16, 0),      # the most rows the by-slot path takes, many per slot
    (105, 256, 40, 5, 32, 4),        # y 8 bytes past a 16-byte boundary: the row-parallel kernel
])
def test_expand_fold_by_slot(orc, seed, n_out, n, n_slots, R, col):
    wl, dw = _workload(seed, 64, n_out, n, n_slots, R)
    rng = np.random.default_rng(seed)
    th = rng.standard_normal((dw.n, R)).astype(np.float32)
    stride = n_out + 8
    yfull = WL.f32_to_bf16_bits(rng.standard_normal((dw.n, stride)).astype(np.float32))
    y = torch.from_numpy(yfull.view(np.int16)).view(torch.bfloat16).cuda()
    t = torch.from_numpy(th).cuda()
    B.lora_expand_fold(dw.route, t, dw.seq_slot, dw.n, y[:, col:], stride)
    torch.cuda.synchronize()
    got = bf16_bits(y)
    live = _resolved(dw)
    # the columns outside [col, col + n_out) and the unresolved rows keep their bits
    outside = np.ones(stride, bool)
    outside[col:col + n_out] = False
    assert np.array_equal(got[:, outside], yfull[:, outside])
    assert np.array_equal(got[~live], yfull[~live])
    yin = yfull[:, col:col + n_out]
    ref = orc.expand_fold(_route(orc, wl, dw), th, dw.seq_slot_host, yin)
    g = (got[:, col:col + n_out].astype(np.uint32) << 16).view(np.float32)
    check(g[live], ref[live], 1e-2, f"expand_fold seed {seed}")


def test_pair_on_the_decode_workload(orc):
    """lora_shrink then lora_expand_fold in place on the decode workload's
    inputs: y_in + s B (A x) for every resolved row, against the oracle's
    shrink and expand-fold on sampled rows."""
    wl = WL.decode_bgmv()
    dw = DeviceWorkload(wl)
    R = wl.max_rank
    yh = WL.f32_to_bf16_bits(np.random.default_rng(7).standard_normal((dw.n, wl.n_out)).astype(np.float32))
    y = torch.from_numpy(yh.view(np.int16)).view(torch.bfloat16).cuda()
    t = torch.full((dw.n, R), float("nan"), dtype=torch.float32, device="cuda")
    B.lora_shrink(dw.route, dw.x, dw.x_row_stride, dw.seq_slot, dw.n, t)
    B.lora_expand_fold(dw.route, t, dw.seq_slot, dw.n, y, wl.n_out)
    torch.cuda.synchronize()
    r = orc.route_for(wl, dw.scale_table_host)
    tref = orc.shrink(r, wl.x, dw.seq_slot_host)
    live = ~np.isnan(tref[:, 0])
    ref = orc.expand_fold(r, np.nan_to_num(tref), dw.seq_slot_host, yh)
    got = (bf16_bits(y).astype(np.uint32) << 16).view(np.float32)
    check(got[live], ref[live], 1e-2, "pair")
    assert np.array_equal(bf16_bits(y)[~live], yh[~live])
