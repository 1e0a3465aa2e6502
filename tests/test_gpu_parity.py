"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerance (fixed by the benchmark spec for this path): every bf16 output
within 1e-2 * max(1, |y_ref|) of the oracle, every f32 output within
1e-4 * max(1, |y_ref|).  Routing is checked bit for bit: rows that skip are
byte-identical to the base-only launch, integer-exact inputs give outputs
identical to the oracle's, and rows a call must not write keep a sentinel.
"""
import numpy as np
import pytest

import golden_cases
import oracle
from adapter_lora_bgmv_amd import binding as B
from adapter_lora_bgmv_amd import workloads as WL
from adapter_lora_bgmv_amd.harness import DeviceWorkload, bf16_bits, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lora_init()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def check(y, ref, dtype, what, mask=None):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    if mask is not None:
        y, ref = y[mask], ref[mask]
    err = np.abs(y - ref)
    bound = TOL[dtype] * np.maximum(1.0, np.abs(ref))
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.nanargmax(np.where(bad, err, -1)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements over the bound; "
                             f"worst at {i}: got {y[i]!r} want {ref[i]!r}")


def run_case(orc, wl, rows=None, **kw):
    dw = DeviceWorkload(wl, **kw)
    y = dw.run()
    torch.cuda.synchronize()
    got = dw.y_host()
    st = dw.scale_table_host
    ref = orc.run(wl, rows=rows, scale_table=st) if not kw.get("null_slots") else None
    return dw, got, ref


# ------------------------------------------------------------------ small random cases
SMALL = [
    # (seed, dtype, k, n_out, n, n_slots, max_rank)
    (0, "bf16", 96, 80, 13, 5, 16),
    (1, "bf16", 200, 136, 70, 6, 32),     # n > 64: 128-row tiles, split 1
    (2, "bf16", 1032, 264, 40, 4, 16),    # ragged k tail and shrink chunk
    (3, "bf16", 4096, 72, 5, 3, 64),      # split-K 4, five rows
    (4, "bf16", 264, 520, 150, 9, 48),    # two row tiles, ragged n_out tile
    (5, "bf16", 64, 64, 1, 2, 16),        # one row
    (8, "bf16", 2048, 192, 20, 4, 128),   # rank 128, split-K 2
    (9, "bf16", 3072, 128, 100, 5, 16),   # 100 rows: 128-row tiles, split-K 3
    (13, "bf16", 160, 88, 7, 3, 16),      # second row block of a tile cut at 8 rows
    (14, "bf16", 1536, 56, 33, 20, 64),   # one ragged tile, 20 slots, rank 64
    (19, "bf16", 3648, 136, 9, 3, 32),    # 57 stages: the last k range is one stage, its second shrink chunk empty
    (20, "bf16", 8192, 72, 5, 2, 16),     # the largest k_in of the decode kernels: 16 k ranges
    (21, "bf16", 8200, 40, 6, 2, 16),     # one column block past it: the tiled path
    (22, "bf16", 520, 296, 200, 6, 32),   # 256 x 128 tiles: ragged rows, outputs and k
    (23, "bf16", 1024, 200, 64, 1, 16),   # most rows on one slot: 3 row groups in its shrink unit
    (50, "bf16", 1024, 200, 64, 1, 16),   # 50 rows on one slot: 4 row groups, the unit after the W loop
    (24, "bf16", 2048, 136, 60, 2, 32),   # two slots, two rank blocks each, full 512-column k ranges
    (6, "f32", 96, 80, 13, 5, 16),
    (7, "f32", 37, 29, 9, 3, 5),          # f32 takes any shape
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}_{c[1]}_k{c[2]}_o{c[3]}_n{c[4]}" for c in SMALL])
def test_decode_small(orc, case):
    seed, dtype, k, n_out, n, n_slots, R = case
    wl = WL.random_small(seed, dtype=dtype, k=k, n_out=n_out, n=n, n_slots=n_slots, max_rank=R)
    dw, got, ref = run_case(orc, wl, x_extra_cols=8 if dtype == "bf16" else 3, y_extra_cols=8)
    check(got, ref, dtype, wl.name)


@pytest.mark.parametrize("seed,dtype,lens", [
    (10, "bf16", [5, 0, 17, 64, 3, 100]),
    (11, "bf16", [512, 300, 1, 0]),
    (13, "bf16", [60, 0, 90, 50]),       # 200 rows: 256 x 128 tiles
    (15, "bf16", [2000, 100, 2100]),     # over 4096 rows: the route kernel ranks the rows
    (12, "f32", [4, 0, 9, 2]),
])
def test_segmented_small(orc, seed, dtype, lens):
    wl = WL.random_small(seed, dtype=dtype, k=136, n_out=96, n_slots=4, max_rank=16,
                         kind="segmented", seg_lens=lens)
    dw = DeviceWorkload(wl)
    dw.y.fill_(float("nan"))
    dw.run()
    torch.cuda.synchronize()
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    check(dw.y_host(), ref, dtype, wl.name)


def test_segmented_rows_outside_and_unsorted_slots(orc):
    """Segments that start after row 0 and end before the last row (the rows
    outside every segment are not written), an empty segment, one slot on two
    segments, slots out of order and a skipping slot: the plan sorts whole
    segments by slot and the result is the oracle's, row by row."""
    wl = WL.random_small(14, dtype="bf16", k=136, n_out=96, n_slots=4, max_rank=16,
                         kind="segmented", seg_lens=[40, 0, 70, 30, 55, 20])
    wl.seg_indptr = np.array([10, 50, 50, 120, 150, 185, 200], np.int32)
    wl.seg_slot = np.array([2, 0, 3, 2, -1, 1], np.int32)
    dw = DeviceWorkload(wl)
    dw.y.fill_(float("nan"))
    dw.run()
    torch.cuda.synchronize()
    got = dw.y_host()
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    out = np.isnan(ref[:, 0])
    assert out.sum() == 10 + 15 and np.all(np.isnan(got[out]))
    check(got[~out], ref[~out], "bf16", wl.name)


@pytest.mark.parametrize("seed,dtype,E,top_k,n_tok,R", [
    (20, "bf16", 5, 2, 37, 16),
    (21, "bf16", 9, 3, 70, 16),
    (22, "f32", 4, 2, 11, 16),
    (23, "bf16", 4, 2, 230, 16),   # ~115 rows per expert: 128-row tiles
    (24, "bf16", 3, 2, 200, 48),   # the same with a rank that does not divide 64
])
def test_moe_small(orc, seed, dtype, E, top_k, n_tok, R):
    wl = WL.random_small(seed, dtype=dtype, k=72, n_out=48, n=n_tok, n_slots=3, max_rank=R,
                         kind="moe", n_experts=E, top_k=top_k)
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    check(dw.y_host(), ref, dtype, wl.name)


def test_moe_wide_tiles(orc):
    """The gather on 512-output tiles (64-row tiles, one row tile per expert
    making one round of workgroups): 600 outputs, so the second column tile
    is ragged, and about 30 rows per expert."""
    wl = WL.random_small(26, dtype="bf16", k=136, n_out=600, n=90, n_slots=3, max_rank=16,
                         kind="moe", n_experts=6, top_k=2)
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    check(dw.y_host(), ref, "bf16", wl.name)


def test_moe_invalid_expert_rows_not_written(orc):
    wl = WL.random_small(23, dtype="bf16", k=64, n_out=32, n=10, n_slots=2, max_rank=16,
                         kind="moe", n_experts=3, top_k=2)
    wl.indices = wl.indices.copy()
    wl.indices[[1, 6]] = [3, -1]
    dw = DeviceWorkload(wl)
    dw.y.fill_(7.0)
    dw.run()
    torch.cuda.synchronize()
    got = dw.y_host()
    assert np.all(got[[1, 6]] == 7.0)
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    keep = np.ones(len(got), bool)
    keep[[1, 6]] = False
    check(got[keep], ref[keep], "bf16", "moe valid rows")


@pytest.mark.parametrize("seed,dtype,E,n,k,n_out,R", [
    (24, "bf16", 5, 90, 72, 48, 16),
    (25, "bf16", 9, 300, 136, 264, 16),   # 300 rows over 9 experts: several row tiles per expert
    (26, "bf16", 64, 200, 64, 32, 16),    # more experts than rows per expert, many empty
    (27, "f32", 4, 23, 37, 29, 16),
    (28, "bf16", 3, 700, 200, 264, 16),   # ~233 rows per expert: one ragged 256-row tile each
    (35, "bf16", 4, 1300, 200, 520, 16),  # ~325 rows per expert: a whole 256-row tile and a ragged one
    (36, "bf16", 3, 700, 200, 264, 48),   # rank 48 (not a divisor of 64): 128-row tiles
])
def test_moe_grouped_small(orc, seed, dtype, E, n, k, n_out, R):
    """atlas moe_lora_grouped_down: rows sorted by expert, ranges from
    expert_offsets; rows outside every range keep their sentinel."""
    wl = WL.random_small(seed, dtype=dtype, k=k, n_out=n_out, n=n, n_slots=3, max_rank=R,
                         kind="moe_grouped", n_experts=E)
    dw = DeviceWorkload(wl)
    dw.y.fill_(float("nan"))
    dw.run()
    torch.cuda.synchronize()
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    got = dw.y_host()
    outside = np.isnan(ref[:, 0])
    assert np.all(np.isnan(got[outside])), "a row outside every expert range was written"
    check(got[~outside], ref[~outside], dtype, wl.name)


def test_moe_grouped_base_only(orc):
    """route == NULL: every row inside an expert range is W_e x, rows outside keep their sentinel."""
    wl = WL.random_small(29, dtype="bf16", k=136, n_out=96, n=150, n_slots=3, max_rank=16,
                         kind="moe_grouped", n_experts=4)
    dw = DeviceWorkload(wl)
    dw.y.fill_(float("nan"))
    dw.run(route=False)
    torch.cuda.synchronize()
    ref = orc.run(wl, route=False)
    got = dw.y_host()
    outside = np.isnan(ref[:, 0])
    assert np.all(np.isnan(got[outside]))
    check(got[~outside], ref[~outside], "bf16", "grouped base only")


def test_moe_grouped_equals_gather_sorted():
    """The grouped call on the gather's routing slots sorted by expert gives the
    gather's rows, bit for bit: each output is reduced row-locally in the same order."""
    wl = WL.random_small(28, dtype="bf16", k=200, n_out=96, n=40, n_slots=3, max_rank=16,
                         kind="moe", n_experts=6, top_k=3)
    dg = DeviceWorkload(wl)
    yg = bf16_bits(dg.run().clone())
    order, off, rs = WL.group_by_expert(wl.indices, wl.token_slot, wl.top_k, wl.n_experts)
    ws = WL.Workload(name="sorted", dtype="bf16", k_in=wl.k_in, n_out=wl.n_out,
                     max_rank=wl.max_rank, W=wl.W, A=wl.A, B=wl.B, x=wl.x[order],
                     adapters=wl.adapters, kind="moe_grouped", n_experts=wl.n_experts,
                     expert_offsets=off, row_slot=rs)
    ds = DeviceWorkload(ws)
    ys = bf16_bits(ds.run().clone())
    torch.cuda.synchronize()
    assert np.array_equal(ys, yg[order])


@pytest.mark.parametrize("dtype,R", [("bf16", 32), ("f32", 8)])
def test_moe_grouped_shrink_and_expand_fold(orc, dtype, R):
    wl = WL.random_small(29, dtype=dtype, k=520, n_out=136 if dtype == "bf16" else 50, n=80,
                         n_slots=3, max_rank=R, kind="moe_grouped", n_experts=5)
    dw = DeviceWorkload(wl, null_slots=[7])  # adapter 1, expert 2
    oroute = orc.route_for(wl, dw.scale_table_host, null_slots=[7])
    t = torch.full((dw.n, R), float("nan"), dtype=torch.float32, device="cuda")
    B.lora_moe_grouped_shrink(dw.route, dw.x, dw.x_row_stride, dw.expert_offsets, dw.seq_slot,
                              dw.n, t)
    rng = np.random.default_rng(4)
    th = rng.standard_normal((dw.n, R)).astype(np.float32)
    yh = rng.standard_normal((dw.n, wl.n_out)).astype(np.float32)
    yh = WL.f32_to_bf16_bits(yh) if dtype == "bf16" else yh
    y = to_device(yh)
    B.lora_moe_grouped_expand_fold(dw.route, to_device(th), dw.expert_offsets, dw.seq_slot, dw.n,
                                   y, wl.n_out)
    torch.cuda.synchronize()
    got_t = t.cpu().numpy().astype(np.float64)
    ref_t = orc.moe_grouped_shrink(oroute, wl.x, wl.expert_offsets, wl.row_slot)
    written = ~np.isnan(ref_t[:, 0])
    assert written.sum() >= 20
    assert np.array_equal(~np.isnan(got_t[:, 0]), written), "rows written differ from rows routed"
    check(got_t[written], ref_t[written], "f32", "grouped shrink")
    ref_y = orc.moe_grouped_expand_fold(oroute, th, wl.expert_offsets, wl.row_slot, yh)
    got = bf16_bits(y)
    if dtype == "bf16":
        assert np.array_equal(got[~written], yh[~written])  # untouched bit for bit
        got = (got.astype(np.uint32) << 16).view(np.float32)
    check(got, ref_y, dtype, "grouped expand_fold")


# ------------------------------------------------------------------ hand cases, bit exact
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hand_cases_bit_exact(dtype):
    for case in golden_cases.load("hand_apply.json")["cases"]:
        if dtype == "bf16" and (case["max_rank"] % 16 or case["k_in"] % 8 or case["n_out"] % 8):
            continue  # the bf16 path takes padded shapes only; see the padded variant below
        wl = golden_cases.hand_workload(case, dtype)
        dw = DeviceWorkload(wl)
        dw.y.fill_(float("nan"))
        dw.run()
        torch.cuda.synchronize()
        assert np.array_equal(dw.y_host(), golden_cases.expected_y(case), equal_nan=True), case["name"]


def _pad_case(case, k_to=8, o_to=8, r_to=16):
    """The hand case zero-padded to bf16-friendly shapes (pads change no value)."""
    c = dict(case)
    k, o, r = case["k_in"], case["n_out"], case["max_rank"]
    K, O, R = -(-k // k_to) * k_to, -(-o // o_to) * o_to, -(-r // r_to) * r_to
    def pad(a, shape):
        a = np.array(a, np.float32)
        out = np.zeros(a.shape[:-len(shape)] + shape if len(shape) <= a.ndim else shape, np.float32)
        sl = tuple(slice(0, s) for s in a.shape)
        out[sl] = a
        return out
    if case["kind"] in ("moe", "moe_grouped"):
        c["W"] = pad(case["W"], (len(case["W"]), O, K)).tolist()
    elif case["kind"] != "embed":
        c["W"] = pad(case["W"], (O, K)).tolist()
    if case["kind"] == "embed":  # the table's rows are n_embd = k_in wide; the vocabulary stays
        c["E"] = pad(case["E"], (o, K)).tolist()
        c["a_file"] = pad(case["a_file"], (len(case["a_file"]), o, R)).tolist()
        c["b_file"] = pad(case["b_file"], (len(case["b_file"]), K, R)).tolist()
        c["k_in"], c["max_rank"] = K, R
        y = np.zeros((len(case["y"]), K))
        y[:, :k] = golden_cases.expected_y(case)
        y[np.isnan(y[:, 0])] = np.nan
        return c, y
    if case["kind"] == "stack":
        c["levels"] = [dict(lv, A=pad(lv["A"], (len(lv["A"]), R, K)).tolist(),
                            B=pad(lv["B"], (len(lv["B"]), O, R)).tolist()) for lv in case["levels"]]
    else:
        c["A"] = pad(case["A"], (len(case["A"]), R, K)).tolist()
        c["B"] = pad(case["B"], (len(case["B"]), O, R)).tolist()
    c["x"] = pad(case["x"], (len(case["x"]), K)).tolist()
    c["k_in"], c["n_out"], c["max_rank"] = K, O, R
    y = np.zeros((len(case["y"]), O))
    y[:, :o] = golden_cases.expected_y(case)
    y[np.isnan(y[:, 0])] = np.nan  # a row that is not written stays NaN in every column
    return c, y


def test_hand_cases_padded_bf16_bit_exact():
    for case in golden_cases.load("hand_apply.json")["cases"]:
        c, want = _pad_case(case)
        wl = golden_cases.hand_workload(c, "bf16")
        dw = DeviceWorkload(wl)
        dw.y.fill_(float("nan"))
        dw.run()
        torch.cuda.synchronize()
        assert np.array_equal(dw.y_host(), want, equal_nan=True), case["name"]


# ------------------------------------------------------------------ exact-integer routing
def _int_pool(rng, S, R, k, n_out, E=1):
    """A and B entries in {-1, 0, 1}, drawn per pair, so every pair is told apart."""
    A = rng.integers(-1, 2, (S * E, R, k)).astype(np.float32)
    Bp = rng.integers(-1, 2, (S * E, n_out, R)).astype(np.float32)
    return A, Bp


@pytest.mark.parametrize("kind", ["decode", "segmented", "moe", "moe_grouped"])
def test_integer_routing_bit_exact(orc, kind):
    """Small integers, power-of-two scales: every partial sum is exact in f32 and
    every output is a multiple of 1/2 below 128, so the GPU must equal the oracle exactly."""
    rng = np.random.default_rng(42)
    k, n_out, R, S = 16, 24, 16, 4
    moe = kind in ("moe", "moe_grouped")
    E = 3 if moe else 1
    W = rng.integers(-1, 2, (E, n_out, k) if moe else (n_out, k)).astype(np.float32)
    A, Bp = _int_pool(rng, S, R, k, n_out, E)
    A[:, 2:, :] = 0    # rank 2 in a rank-16 pool keeps the sums small
    Bp[:, :, 2:] = 0
    ad = [WL.AdapterSpec(2, 0.0, v) for v in (1.0, 0.5, 2.0, 0.0)]
    kw = dict(name="int", dtype="bf16", k_in=k, n_out=n_out, max_rank=R,
              W=WL.f32_to_bf16_bits(W), A=WL.f32_to_bf16_bits(A), B=WL.f32_to_bf16_bits(Bp),
              adapters=ad, kind=kind)
    if kind == "decode":
        x = rng.integers(-1, 2, (20, k)).astype(np.float32)
        ss = np.array([0, 1, 2, 3, -1, 4, 99, -7] + list(rng.integers(-1, 5, 12)), np.int32)
        wl = WL.Workload(x=WL.f32_to_bf16_bits(x), adapter_slots=ss, padded_n=20,
                         meta={"seq_slot": ss}, **kw)
    elif kind == "segmented":
        x = rng.integers(-1, 2, (30, k)).astype(np.float32)
        wl = WL.Workload(x=WL.f32_to_bf16_bits(x), seg_indptr=np.array([0, 7, 7, 19, 30], np.int32),
                         seg_slot=np.array([2, 0, -1, 1], np.int32), **kw)
    elif kind == "moe_grouped":  # rows 0-1 and 27-28 outside every range; expert 1 empty
        x = rng.integers(-1, 2, (29, k)).astype(np.float32)
        rs = np.array([0, 1, 2, 3, -1, 7, 0, 1, 2, 3, 1, 0, 3, 2, 1, 0] + list(rng.integers(-1, 5, 13)),
                      np.int32)
        wl = WL.Workload(x=WL.f32_to_bf16_bits(x), n_experts=E,
                         expert_offsets=np.array([2, 15, 15, 27], np.int32), row_slot=rs, **kw)
    else:
        x = rng.integers(-1, 2, (24, k)).astype(np.float32)
        idx = np.array([rng.choice(E, 2, replace=False) for _ in range(12)], np.int32).reshape(-1)
        wl = WL.Workload(x=WL.f32_to_bf16_bits(x), n_experts=E, top_k=2, indices=idx,
                         token_slot=np.array([0, 1, 2, 3, -1, 7, 0, 1, 2, 3, 1, 0], np.int32), **kw)
    dw = DeviceWorkload(wl)
    dw.y.fill_(float("nan"))
    dw.run()
    torch.cuda.synchronize()
    if kind == "decode":
        ref = orc.apply(wl.W, orc.route_for(wl, dw.scale_table_host), wl.x, ss, 1)
    else:
        ref = orc.run(wl, scale_table=dw.scale_table_host)
    done = ~np.isnan(ref[:, 0])
    assert done.sum() >= 20
    r = ref[done]
    assert np.all(np.abs(r) < 128) and np.array_equal(2 * r, np.round(2 * r))  # halves: exact in bf16
    assert np.array_equal(dw.y_host(), ref, equal_nan=True)


# ------------------------------------------------------------------ byte identity
def test_skip_rows_are_base_bit_for_bit(orc):
    wl = WL.random_small(30, dtype="bf16", k=512, n_out=256, n=48, n_slots=6, max_rank=32)
    st = B.lora_scale_table(wl.adapters)
    st[2] = 0.0                                  # a switched-off adapter
    dw = DeviceWorkload(wl, scale_table=st, null_slots=[4])
    ss = dw.seq_slot_host.copy()
    ss[:8] = [-1, 2, 4, 6, 1000, -5, 0, 1]         # pad, zero scale, NULL, out of range x2
    dw.seq_slot.copy_(torch.from_numpy(ss))
    y_routed = dw.run().clone()
    y_base = dw.run(route=False).clone()
    torch.cuda.synchronize()
    rb, bb = bf16_bits(y_routed), bf16_bits(y_base)
    skip = [i for i, s in enumerate(ss) if not (0 <= s < 6 and s not in (2, 4))]
    live = [i for i in range(len(ss)) if i not in skip]
    assert set(skip) >= {0, 1, 2, 3, 4, 5}
    assert np.array_equal(rb[skip], bb[skip])
    assert (rb[live] != bb[live]).mean() > 0.5
    ref = orc.apply(wl.W, oracle.Route(wl.A, wl.B, st, 1, wl.k_in, wl.n_out, wl.max_rank,
                                       null_slots=[4]), wl.x, ss, 1)
    check(dw.y_host(y_routed), ref, "bf16", "routed with skips")


@pytest.mark.parametrize("kind,seed,k,n_out,n,R", [
    ("decode", 35, 520, 264, 150, 48),     # rank 48: the register-staged LoRA term
    ("decode", 36, 2048, 296, 100, 16),    # classic split-k both ways
    ("segmented", 37, 512, 256, 0, 32),    # 256 x 256 tiles both ways
    ("moe", 38, 200, 96, 60, 16),
])
def test_routed_and_base_only_share_a_workspace(kind, seed, k, n_out, n, R):
    """Routed and base-only calls of one shape alternate on one workspace; each
    gives the bits of the same call on a fresh workspace."""
    if kind == "segmented":
        wl = WL.random_small(seed, dtype="bf16", k=k, n_out=n_out, n_slots=3, max_rank=R,
                             kind="segmented", seg_lens=[100, 70, 0, 130])
    elif kind == "moe":
        wl = WL.random_small(seed, dtype="bf16", k=k, n_out=n_out, n=n, n_slots=3, max_rank=R,
                             kind="moe", n_experts=4, top_k=2)
    else:
        wl = WL.random_small(seed, dtype="bf16", k=k, n_out=n_out, n=n, n_slots=4, max_rank=R)
    fresh = {}
    for route in (True, False):
        d = DeviceWorkload(wl)
        fresh[route] = bf16_bits(d.run(route=route).clone())
    dw = DeviceWorkload(wl)
    for route in (True, False, True, False, True):
        got = bf16_bits(dw.run(route=route).clone())
        torch.cuda.synchronize()
        assert np.array_equal(got, fresh[route]), route


def test_all_rows_skipped_equals_base():
    wl = WL.random_small(31, dtype="bf16", k=256, n_out=128, n=17, n_slots=3, max_rank=16)
    dw = DeviceWorkload(wl)
    dw.seq_slot.fill_(-1)
    a = bf16_bits(dw.run().clone())
    b = bf16_bits(dw.run(route=False).clone())
    assert np.array_equal(a, b)


def test_decode_is_deterministic():
    wl = WL.random_small(32, dtype="bf16", k=2048, n_out=512, n=61, n_slots=7, max_rank=16)
    dw = DeviceWorkload(wl)
    a = bf16_bits(dw.run().clone())
    b = bf16_bits(dw.run().clone())
    assert np.array_equal(a, b)


def test_split_equals_stacked_on_gpu():
    """frink lora_attach.rs: the fused projection applied whole equals its parts
    applied with one copy of A each and their block of B's rows -- bit for bit."""
    wl = WL.random_small(33, dtype="bf16", k=512, n_out=192, n=40, n_slots=5, max_rank=32)
    dw = DeviceWorkload(wl)
    whole = bf16_bits(dw.run().clone())
    h = 96
    y = torch.empty_like(dw.y)
    for part in range(2):
        r = B.DeviceRoute(dw.A, dw.Bp, dw.scale_table_host, n_out=h, b_row_offset=part * h)
        Wp = dw.W[part * h:(part + 1) * h]
        ws_bytes = B.lora_workspace_bytes(0, B.LORA_BF16, dw.n, h, wl.k_in, wl.max_rank)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        B.lora_apply(B.LORA_BF16, h, wl.k_in, Wp, wl.k_in, r, dw.x, dw.x_row_stride, dw.seq_slot,
                     dw.n, y[:, part * h:], dw.y_row_stride, ws, ws_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y)[:, :192], whole[:, :192])


def test_scale_read_at_apply_time(orc):
    wl = WL.random_small(34, dtype="bf16", k=256, n_out=64, n=9, n_slots=2, max_rank=16)
    dw = DeviceWorkload(wl)
    y1 = dw.y_host(dw.run().clone())
    base = dw.y_host(dw.run(route=False).clone())
    dw.route.set_scale_table(dw.scale_table_host * 0.5)
    y2 = dw.y_host(dw.run().clone())
    ref2 = orc.run(wl, scale_table=dw.scale_table_host * np.float32(0.5))
    check(y2, ref2, "bf16", "halved scale")
    assert np.any(y1 != y2) and np.any(y1 != base)


# ------------------------------------------------------------------ shrink / expand_fold
@pytest.mark.parametrize("dtype,k,R", [("bf16", 1000, 32), ("bf16", 4096, 16), ("f32", 300, 8)])
def test_shrink_standalone(orc, dtype, k, R):
    wl = WL.random_small(40, dtype=dtype, k=k, n_out=32, n=45, n_slots=5, max_rank=R)
    dw = DeviceWorkload(wl)
    t = torch.full((dw.n, R), float("nan"), dtype=torch.float32, device="cuda")
    B.lora_shrink(dw.route, dw.x, dw.x_row_stride, dw.seq_slot, dw.n, t)
    torch.cuda.synchronize()
    got = t.cpu().numpy().astype(np.float64)
    ref = orc.shrink(orc.route_for(wl, dw.scale_table_host), wl.x, dw.seq_slot_host)
    written = ~np.isnan(ref[:, 0])
    assert np.array_equal(~np.isnan(got[:, 0]), written), "rows written differ from rows routed"
    check(got[written], ref[written], "f32", "shrink")


@pytest.mark.parametrize("dtype,R", [("bf16", 64), ("f32", 8)])
def test_expand_fold_standalone(orc, dtype, R):
    wl = WL.random_small(41, dtype=dtype, k=64, n_out=200, n=30, n_slots=4, max_rank=R)
    dw = DeviceWorkload(wl)
    rng = np.random.default_rng(3)
    th = rng.standard_normal((dw.n, R)).astype(np.float32)
    yh = rng.standard_normal((dw.n, wl.n_out)).astype(np.float32)
    yh = WL.f32_to_bf16_bits(yh) if dtype == "bf16" else yh
    y = to_device(yh)
    B.lora_expand_fold(dw.route, to_device(th), dw.seq_slot, dw.n, y, wl.n_out)
    torch.cuda.synchronize()
    ref = orc.expand_fold(orc.route_for(wl, dw.scale_table_host), th, dw.seq_slot_host, yh)
    got = bf16_bits(y)
    if dtype == "bf16":
        skip = [i for i, s in enumerate(dw.seq_slot_host)
                if not (0 <= s < len(dw.scale_table_host) and dw.scale_table_host[s] != 0)]
        assert np.array_equal(got[skip], yh[skip])
        got = (got.astype(np.uint32) << 16).view(np.float32)
    check(got, ref, dtype, "expand_fold")


# ------------------------------------------------------------------ edges
def test_empty_batch_is_a_no_op():
    wl = WL.random_small(50, dtype="bf16", k=64, n_out=64, n=3, n_slots=2, max_rank=16)
    dw = DeviceWorkload(wl)
    dw.y.fill_(3.0)
    B.lora_apply(B.LORA_BF16, 64, 64, dw.W, 64, dw.route, dw.x, dw.x_row_stride, dw.seq_slot, 0,
                 dw.y, dw.y_row_stride, dw.workspace, dw.ws_bytes)
    torch.cuda.synchronize()
    assert torch.all(dw.y == 3.0)


def test_max_rank_256_and_many_slots(orc):
    wl = WL.random_small(51, dtype="bf16", k=256, n_out=64, n=33, n_slots=300, max_rank=256,
                         ranks=[256 if s % 2 else 17 for s in range(300)])
    dw, got, ref = run_case(orc, wl)
    check(got, ref, "bf16", "rank 256, 300 slots")


# ------------------------------------------------------------------ the five workloads
def _sample_rows(n, extra=(), k=24, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(int(v) for v in rng.choice(n, size=min(k, n), replace=False)) | set(extra)
    return np.array(sorted(r for r in rows if 0 <= r < n), np.int32)


def test_moe_grouped_full_size(orc):
    """The grouped workload at full size (2048 tokens x top-6 over 64 experts
    [2048 x 1408], rank 16): sampled rows, the first and last row of every
    tenth expert range among them."""
    wl = WL.moe_down_grouped()
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    off = wl.expert_offsets
    edges = [int(v) for e in range(0, wl.n_experts, 10) for v in (off[e], off[e + 1] - 1)]
    rows = _sample_rows(dw.n, extra=edges + [0, dw.n - 1], k=64)
    ref = orc.run(wl, rows=rows, scale_table=dw.scale_table_host)
    check(dw.y_host()[rows], ref, "bf16", wl.name)


@pytest.mark.parametrize("name", list(WL.CONFIGS))
def test_full_config_parity(orc, name):
    wl = WL.CONFIGS[name]()
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    got = dw.y_host()
    if name in ("single_projection_f32", "decode_bgmv"):
        rows = np.arange(dw.n, dtype=np.int32)
    else:
        rows = _sample_rows(dw.n, extra=(0, dw.n - 1), k=24 if name != "moe_down_gather" else 96)
    ref = orc.run(wl, rows=rows, scale_table=dw.scale_table_host)
    check(got[rows], ref, wl.dtype, wl.name)
    if name == "decode_bgmv":  # the seven pad rows equal the base-only output bit for bit
        yb = dw.run(route=False).clone()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(dw.y)[57:], bf16_bits(yb)[57:])


@pytest.mark.parametrize("seed,k,n_out,n,R", [
    (15, 2112, 1000, 300, 32),   # 33 k stages in one range, a ragged last stage
    (16, 128, 8000, 2100, 32),   # 9 x 32 tiles of 256 x 256, 2 stages each, no split
    (17, 1024, 2048, 520, 16),   # rank 16: T's columns past 2R are zero in LDS
    (18, 640, 1000, 300, 128),   # rank 128: 256 x 128 tiles, the register-staged LoRA term
    (19, 4096, 264, 400, 64),    # 256 x 256 tiles over the whole k, a ragged output tile
])
def test_large_batch_tiles(orc, seed, k, n_out, n, R):
    """Batches over 128 rows take 256-output tiles, each over the whole k
    range on one workgroup, the LoRA term after the base contraction; runs
    give the same bits twice."""
    wl = WL.random_small(seed, dtype="bf16", k=k, n_out=n_out, n=n, n_slots=6, max_rank=R)
    dw = DeviceWorkload(wl)
    first = bf16_bits(dw.run().clone())
    again = bf16_bits(dw.run().clone())
    torch.cuda.synchronize()
    assert np.array_equal(first, again)  # the arrival order does not change the sums
    rows = _sample_rows(n, extra=(0, n - 1), k=48, seed=seed)
    ref = orc.run(wl, rows=rows, scale_table=dw.scale_table_host)
    check(dw.y_host()[rows], ref, "bf16", wl.name)


# ------------------------------------------------------------------ token-embedding gather
def _embed_small(seed, dtype, n_vocab, n_embd, n, R, n_slots=4):
    rng = np.random.default_rng(seed)
    ranks = [int(v) for v in rng.integers(1, R + 1, size=n_slots)]
    wl = WL.token_embedding(seed, n_vocab=n_vocab, n_embd=n_embd, n=n, n_slots=n_slots, rank=R,
                            alpha=8.0, dtype=dtype, max_rank=R, ranks=ranks)
    tok = wl.meta["token_ids"].copy()
    tok[[0, n // 2]] = [n_vocab, -5]  # outside the vocabulary: not written
    wl.meta["token_ids"] = tok
    return wl


@pytest.mark.parametrize("seed,dtype,n_vocab,n_embd,n,R,n_slots", [
    (110, "bf16", 1000, 264, 70, 16, 4),
    (111, "bf16", 517, 4104, 9, 32, 4),     # two column blocks, the second ragged
    (112, "f32", 300, 37, 21, 5, 4),
    (113, "bf16", 800, 520, 130, 16, 12),   # more pairs in a workgroup than one pass stages
    (114, "f32", 200, 70, 75, 8, 10),
])
def test_embed_small(orc, seed, dtype, n_vocab, n_embd, n, R, n_slots):
    """ferrox LoraDelta::add_row_to: a gathered row is E[token] plus s times that
    token's row of B A; the pair arrives flipped and is brought into the one
    layout by lora_embedding_pair.  Rows whose token is outside the vocabulary
    keep their sentinel; rows whose slot skips are the table row bit for bit."""
    wl = _embed_small(seed, dtype, n_vocab, n_embd, n, R, n_slots)
    dw = DeviceWorkload(wl)
    dw.y.fill_(float("nan"))
    dw.run()
    torch.cuda.synchronize()
    got = dw.y_host()
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    out = np.isnan(ref[:, 0])
    assert out.sum() == 2 and np.all(np.isnan(got[out]))
    check(got[~out], ref[~out], dtype, wl.name)
    base = dw.y_host(dw.run(route=False).clone())
    torch.cuda.synchronize()
    st = dw.scale_table_host
    skip = [i for i, s in enumerate(wl.meta["seq_slot"])
            if not out[i] and not (0 <= s < len(st) and st[s] != 0)]
    assert skip and np.array_equal(got[skip], base[skip])
    check(base[~out], orc.run(wl, route=False)[~out], dtype, "plain gather")


def test_embed_full_size(orc):
    """E [32000 x 4096] bf16, 8 rank-16 adapters, 4096 tokens: sampled rows."""
    wl = WL.token_embedding()
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    rows = _sample_rows(dw.n, extra=(0, dw.n - 1), k=96)
    ref = orc.run(wl, rows=rows, scale_table=dw.scale_table_host)
    check(dw.y_host()[rows], ref, "bf16", wl.name)


# ------------------------------------------------------------------ adapter stack
@pytest.mark.parametrize("seed,dtype,k,n_out,n,levels,R", [
    (100, "bf16", 136, 96, 37, 2, 16),
    (101, "bf16", 520, 264, 64, 3, 32),
    (102, "bf16", 264, 136, 150, 3, 16),   # over 64 rows: the first level on the tiled path
    (103, "bf16", 1032, 72, 5, 8, 48),     # eight levels
    (104, "f32", 37, 29, 9, 3, 5),
])
def test_stack_small(orc, seed, dtype, k, n_out, n, levels, R):
    """ferrox LoraStack: W x plus every level's delta in order, each level routed
    by its own slot buffer (-1 and past-the-pool slots add nothing)."""
    wl = WL.random_stack(seed, dtype=dtype, k=k, n_out=n_out, n=n, n_levels=levels, n_slots=3,
                         max_rank=R)
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    check(dw.y_host(), ref, dtype, wl.name)


def test_stack_of_one_and_skipping_levels_are_the_apply():
    """A one-level stack is that level's apply, and further levels whose rows all
    skip leave it unchanged -- bit for bit."""
    wl = WL.random_stack(105, dtype="bf16", k=512, n_out=128, n=40, n_levels=3, n_slots=3,
                         max_rank=16)
    dw = DeviceWorkload(wl)
    lv = dw.levels
    ws, wsb = dw.workspace, dw.ws_bytes
    one = torch.empty_like(dw.y)
    B.lora_apply_stack(B.LORA_BF16, wl.n_out, wl.k_in, dw.W, wl.k_in, [lv[0]["route"]], dw.x,
                       dw.x_row_stride, [lv[0]["seq_slot"]], dw.n, one, dw.y_row_stride, ws, wsb)
    ap = torch.empty_like(dw.y)
    aws = torch.zeros(B.lora_workspace_bytes(0, B.LORA_BF16, dw.n, wl.n_out, wl.k_in, 16),
                      dtype=torch.uint8, device="cuda")
    B.lora_apply(B.LORA_BF16, wl.n_out, wl.k_in, dw.W, wl.k_in, lv[0]["route"], dw.x,
                 dw.x_row_stride, lv[0]["seq_slot"], dw.n, ap, dw.y_row_stride, aws, aws.numel())
    off = torch.full((dw.n,), -1, dtype=torch.int32, device="cuda")
    three = torch.empty_like(dw.y)
    B.lora_apply_stack(B.LORA_BF16, wl.n_out, wl.k_in, dw.W, wl.k_in, [v["route"] for v in lv],
                       dw.x, dw.x_row_stride, [lv[0]["seq_slot"], off, off], dw.n, three,
                       dw.y_row_stride, ws, wsb)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(one), bf16_bits(ap))
    assert np.array_equal(bf16_bits(three), bf16_bits(ap))


def test_stack_of_no_levels_is_the_base(orc):
    """n_levels == 0: the base-only output, equal to a base-only apply bit for bit."""
    wl = WL.random_stack(106, dtype="bf16", k=256, n_out=64, n=20, n_levels=2, n_slots=3, max_rank=16)
    dw = DeviceWorkload(wl)
    y0 = bf16_bits(dw.run(route=False).clone())
    ap = torch.empty_like(dw.y)
    aws = torch.zeros(B.lora_workspace_bytes(0, B.LORA_BF16, dw.n, wl.n_out, wl.k_in, 16),
                      dtype=torch.uint8, device="cuda")
    B.lora_apply(B.LORA_BF16, wl.n_out, wl.k_in, dw.W, wl.k_in, None, dw.x, dw.x_row_stride, None,
                 dw.n, ap, dw.y_row_stride, aws, aws.numel())
    torch.cuda.synchronize()
    assert np.array_equal(y0, bf16_bits(ap))
    check(dw.y_host(), orc.run(wl, route=False), "bf16", "stack of no levels")


def test_stack_full_size(orc):
    """Three levels of eight rank-16 adapters on W [4096 x 4096], 64 rows."""
    wl = WL.adapter_stack()
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    check(dw.y_host(), ref, "bf16", wl.name)


# ------------------------------------------------------------------ speculative verify, strided folds
def _qkv_regions(dw):
    """Bits of the Q, K and V column blocks of the interleaved rows."""
    m = dw.wl.meta
    full = bf16_bits(dw.y_full)
    q, kv = m["q_dim"], m["kv_dim"]
    return full[:, :q], full[:, q:q + kv], full[:, q + kv:q + 2 * kv]


@pytest.mark.parametrize("n_seqs,draft", [(4, 9), (1, 9), (3, 5), (2, 1)])
def test_spec_verify_k_fold_into_qkv(orc, n_seqs, draft):
    """atlas lora_gemv_max_m doc: speculative verify presents n_seqs x draft rows
    (up to 4 x 9 = 36), every row of a sequence on the sequence's adapter; the
    apply_lora_bgmv doc: the K projection's output row stride is the interleaved
    [Q|K|V] row, so the result lands in the K columns and Q and V stay as they were."""
    wl = WL.spec_verify_kv(seed=80 + n_seqs * 10 + draft, n_seqs=n_seqs, draft=draft)
    m = wl.meta
    dw = DeviceWorkload(wl, y_col_offset=m["q_dim"], y_extra_cols=m["kv_dim"])
    dw.y_full.fill_(float("nan"))
    dw.run()
    torch.cuda.synchronize()
    q, k, v = _qkv_regions(dw)
    assert np.all(q == 0x7FC0) and np.all(v == 0x7FC0), "a Q or V column was written"
    ref = orc.run(wl, scale_table=dw.scale_table_host)
    check(dw.y_host(), ref, "bf16", wl.name)
    # the batched verify equals each sequence verified on its own, bit for bit
    for s in range(n_seqs):
        rows = slice(s * draft, (s + 1) * draft)
        one = WL.Workload(name="seq", dtype="bf16", k_in=wl.k_in, n_out=wl.n_out,
                          max_rank=wl.max_rank, W=wl.W, A=wl.A, B=wl.B, x=wl.x[rows],
                          adapters=wl.adapters, adapter_slots=wl.adapter_slots[rows],
                          padded_n=draft, meta=dict(m))
        d1 = DeviceWorkload(one, y_col_offset=m["q_dim"], y_extra_cols=m["kv_dim"])
        d1.run()
        torch.cuda.synchronize()
        assert np.array_equal(d1.y_bits(), k[rows]), s


def test_strided_expand_fold_into_v(orc):
    """atlas apply_lora_bgmv doc (STRIDES): the V delta folds into the V columns
    of the interleaved [Q|K|V] rows; rows that skip, and the Q and K columns,
    keep their bits."""
    wl = WL.spec_verify_kv(seed=90, n_seqs=4, draft=9)
    m = wl.meta
    q, kv, row = m["q_dim"], m["kv_dim"], m["qkv_row"]
    dw = DeviceWorkload(wl)
    ss = dw.seq_slot_host.copy()
    ss[[0, 10, 20]] = [-1, 99, -3]
    dw.seq_slot.copy_(torch.from_numpy(ss))
    rng = np.random.default_rng(5)
    full = WL.f32_to_bf16_bits(rng.standard_normal((dw.n, row)).astype(np.float32))
    qkv = to_device(full)
    th = rng.standard_normal((dw.n, wl.max_rank)).astype(np.float32)
    B.lora_expand_fold(dw.route, to_device(th), dw.seq_slot, dw.n, qkv[:, q + kv:], row)
    torch.cuda.synchronize()
    got = bf16_bits(qkv)
    assert np.array_equal(got[:, :q + kv], full[:, :q + kv]), "a Q or K column changed"
    vin = full[:, q + kv:]
    ref = orc.expand_fold(orc.route_for(wl, dw.scale_table_host), th, ss, vin)
    assert np.array_equal(got[[0, 10, 20], q + kv:], vin[[0, 10, 20]])
    check((got[:, q + kv:].astype(np.uint32) << 16).view(np.float32), ref, "bf16", "V fold")


def test_decode_batch_equals_per_row_calls():
    """atlas apply_lora_bgmv doc: the batched call equals n one-row calls.  On the
    decode path every output element is reduced in the same order whatever the
    batch, so the equality holds bit for bit."""
    wl = WL.random_small(70, dtype="bf16", k=1536, n_out=96, n=24, n_slots=4, max_rank=32)
    dw = DeviceWorkload(wl)
    whole = bf16_bits(dw.run().clone())
    for i in range(dw.n):
        one = WL.Workload(name="one", dtype="bf16", k_in=wl.k_in, n_out=wl.n_out,
                          max_rank=wl.max_rank, W=wl.W, A=wl.A, B=wl.B, x=wl.x[i:i + 1],
                          adapters=wl.adapters, adapter_slots=dw.seq_slot_host[i:i + 1],
                          padded_n=1, meta={"seq_slot": dw.seq_slot_host[i:i + 1]})
        d1 = DeviceWorkload(one)
        yi = bf16_bits(d1.run().clone())
        assert np.array_equal(yi[0], whole[i]), i
