"""Pins that tie the fp64 oracle to the pages, independently of the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix.  ``test_oracle_pins``
runs them against the real oracle; ``test_oracle_mutants`` runs them against
builds with planted mistakes and requires every mistake to be caught.

Kinds of pin used here (none re-types the oracle's loops):
  * values the pages print (scale examples, the seq_slot rule) -- tests/golden;
  * cases worked by hand from the definitions -- tests/golden/hand_apply.json;
  * closed forms (rsLoRA scales);
  * brute force on tiny shapes through the materialised dense delta (tests/brute.py);
  * special cases that reduce to a library routine (numpy matmul);
  * invariants the pages state (zero scale / slot -1 byte identity, split ==
    stacked, padded == true rank, batch == per-position, scale read at apply time).
"""
import math

import numpy as np

import brute
import golden_cases
import oracle
from adapter_lora_bgmv_amd import workloads as WL

PINS = []


def pin(fn):
    PINS.append(fn)
    return fn


def _dt(wl):
    return 1 if wl.dtype == "bf16" else 0


def _close(a, b, rel=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b) / np.maximum(1.0, np.abs(b))
    assert np.all(err <= rel), f"{what}: max rel err {err.max():.3e}"


# ------------------------------------------------------------------ scale
@pin
def scale_examples(o):
    g = golden_cases.load("scale_examples.json")
    for ex in g["examples"]:
        got = o.scale(ex["adapter_scale"], ex["alpha"], ex["rank"], ex["rslora"])
        assert abs(got - ex["scale"]) <= 1e-15 * max(1.0, abs(ex["scale"])), (ex, got)


@pin
def scale_table_values(o):
    t = golden_cases.load("scale_examples.json")["table"]
    ad = [WL.AdapterSpec(rank=r, alpha=al, adapter_scale=s, rslora=rs)
          for (s, al, r, rs) in t["adapters"]]
    got = o.scale_table(ad, t["max_loras"])
    want = np.array(t["values_f32"], np.float32)
    assert got.dtype == np.float32 and np.array_equal(got.view(np.uint32), want.view(np.uint32)), got
    # rounded once from the exact value: 16/sqrt(8) as f32
    got = o.scale_table([WL.AdapterSpec(8, 16.0, 1.0, True)], 1)
    assert got[0] == np.float32(4.0 * math.sqrt(2.0)), got


# ------------------------------------------------------------------ seq_slot
@pin
def seq_slot_examples(o):
    g = golden_cases.load("seq_slot_examples.json")
    for ex in g["examples"]:
        got = o.build_seq_slot(ex["adapter_slots"], ex["padded_n"], ex["active"])
        assert list(got) == ex["seq_slot"], (ex, list(got))


# ------------------------------------------------------------------ hand cases
def _hand_run(o, wl, case):
    dt = _dt(wl)
    r = o.route_for(wl)
    if wl.kind == "decode":
        return o.apply(wl.W, r, wl.x, wl.meta["seq_slot"], dt)
    if wl.kind == "segmented":
        return o.apply_segmented(wl.W, r, wl.x, wl.seg_indptr, wl.seg_slot, dt)
    if wl.kind == "moe_grouped":
        return o.apply_moe_grouped(wl.W, r, wl.x, wl.expert_offsets, wl.row_slot, dt)
    if wl.kind in ("stack", "embed"):
        return o.run(wl)
    return o.apply_moe(wl.W, r, wl.x, wl.indices, wl.top_k, wl.token_slot, dt)


@pin
def hand_cases(o):
    for case in golden_cases.load("hand_apply.json")["cases"]:
        for dtype in ("f32", "bf16"):
            wl = golden_cases.hand_workload(case, dtype)
            y = _hand_run(o, wl, case)
            want = golden_cases.expected_y(case)
            assert np.array_equal(y, want, equal_nan=True), (case["name"], dtype, y)


@pin
def hand_split_halves(o):
    case = [c for c in golden_cases.load("hand_apply.json")["cases"] if c["name"] == "split"][0]
    wl = golden_cases.hand_workload(case)
    want = np.array(case["y"], np.float64)
    h = wl.n_out // case["halves"]
    for part in range(case["halves"]):
        r = o.route_for(wl, b_row_offset=part * h, n_out=h)
        y = o.apply(wl.W[part * h:(part + 1) * h], r, wl.x, wl.meta["seq_slot"], 0)
        assert np.array_equal(y, want[:, part * h:(part + 1) * h]), (part, y)


# ------------------------------------------------------------------ brute force
def _padded_x(x, extra, fill):
    """x with `extra` garbage columns after each row (a row stride > k_in)."""
    n, k = x.shape
    out = np.empty((n, k + extra), x.dtype)
    out[:, :k] = x
    out[:, k:] = fill
    return out


@pin
def brute_force_tiny_decode(o):
    for seed in range(6):
        for dtype in ("f32", "bf16"):
            wl = WL.random_small(seed, dtype=dtype, k=11 + seed, n_out=7 + seed, n=6,
                                 n_slots=4, max_rank=4)
            wl.null_slots = [seed % 4] if seed % 3 == 0 else []
            st = o.scale_table(wl.adapters)
            if seed == 2:
                st[1] = 0.0  # a switched-off slot
            ss = o.seq_slot_for(wl)
            fill = WL.f32_to_bf16_bits(np.float32([1e4]))[0] if dtype == "bf16" else 1e4
            xp = _padded_x(wl.x, 3, fill)
            r = o.route_for(wl, scale_table=st)
            y = o.apply(wl.W, r, xp, ss, _dt(wl))
            want = brute.dense_rows(wl.W, wl.A, wl.B, wl.x, dtype, ss, st, wl.null_slots)
            _close(y, want, 1e-12, f"seed {seed} {dtype}")


@pin
def pages_test_shape(o):
    """ferrox lora.rs test matvec_delta_matches_the_materialised_product: rows 7,
    cols 5, rank 3, alpha 6, scale 0.8, a = sin(0.37 i), b = cos(0.53 i), x_i = i - 2."""
    rows, cols, rank = 7, 5, 3
    a = np.array([math.sin(i * 0.37) for i in range(rank * cols)], np.float32).reshape(rank, cols)
    b = np.array([math.cos(i * 0.53) for i in range(rows * rank)], np.float32).reshape(rows, rank)
    x = np.array([[i - 2.0 for i in range(cols)]], np.float32)
    W = np.zeros((rows, cols), np.float32)
    wl = WL.Workload(name="pages", dtype="f32", k_in=cols, n_out=rows, max_rank=rank, W=W,
                     A=a[None], B=b[None], x=x, adapters=[WL.AdapterSpec(rank, 6.0, 0.8)])
    st = o.scale_table(wl.adapters)
    y = o.apply(W, o.route_for(wl, st), x, [0], 0)
    s = float(st[0])
    dense = s * (b.astype(np.float64) @ a.astype(np.float64)) @ x[0].astype(np.float64)
    _close(y[0], dense, 1e-12, "pages test shape")
    # the pages' own tolerance against the f32 scale 1.6
    assert np.all(np.abs(y[0] - 1.6 * (b.astype(np.float64) @ a @ x[0])) < 1e-4)


@pin
def brute_force_tiny_moe(o):
    for seed in range(4):
        wl = WL.random_small(100 + seed, dtype="bf16", k=9, n_out=6, n=5, n_slots=3,
                             max_rank=4, kind="moe", n_experts=4, top_k=2)
        st = o.scale_table(wl.adapters)
        y = o.apply_moe(wl.W, o.route_for(wl, st), wl.x, wl.indices, wl.top_k, wl.token_slot, 1)
        slots = np.repeat(wl.token_slot, wl.top_k)
        want = brute.dense_rows(wl.W, wl.A, wl.B, wl.x, "bf16", slots, st, (),
                                n_experts=wl.n_experts, experts=wl.indices)
        _close(y, want, 1e-12, f"moe seed {seed}")


def _grouped_experts(offsets, n):
    """Each row's expert from the ranges, -1 outside: numpy's searchsorted, not
    the oracle's scan."""
    off = np.asarray(offsets, np.int64)
    e = np.searchsorted(off, np.arange(n), side="right") - 1
    e[(np.arange(n) < off[0]) | (np.arange(n) >= off[-1])] = -1
    return e


@pin
def brute_force_tiny_moe_grouped(o):
    for seed in range(5):
        dtype = "bf16" if seed % 2 == 0 else "f32"
        wl = WL.random_small(300 + seed, dtype=dtype, k=10, n_out=7, n=9, n_slots=3,
                             max_rank=4, kind="moe_grouped", n_experts=4)
        st = o.scale_table(wl.adapters)
        y = o.apply_moe_grouped(wl.W, o.route_for(wl, st), wl.x, wl.expert_offsets,
                                wl.row_slot, _dt(wl))
        ex = _grouped_experts(wl.expert_offsets, wl.n_rows)
        inside = ex >= 0
        assert np.all(np.isnan(y[~inside])), "a row outside every range was written"
        want = brute.dense_rows(wl.W, wl.A, wl.B, wl.x[inside], dtype, wl.row_slot[inside], st,
                                (), n_experts=wl.n_experts, experts=ex[inside])
        _close(y[inside], want, 1e-12, f"moe grouped seed {seed}")


@pin
def grouped_equals_gather_sorted(o):
    """The grouped layout is the gather's routing slots sorted by expert: the same
    rows give the same outputs, bit for bit, in the sorted order."""
    wl = WL.random_small(400, dtype="bf16", k=12, n_out=8, n=6, n_slots=3, max_rank=4,
                         kind="moe", n_experts=5, top_k=3)
    st = o.scale_table(wl.adapters)
    r = o.route_for(wl, st)
    yg = o.apply_moe(wl.W, r, wl.x, wl.indices, wl.top_k, wl.token_slot, 1)
    order, off, rs = WL.group_by_expert(wl.indices, wl.token_slot, wl.top_k, wl.n_experts)
    ys = o.apply_moe_grouped(wl.W, r, wl.x[order], off, rs, 1)
    assert np.array_equal(ys, yg[order])


@pin
def grouped_shrink_and_expand_match_matmul(o):
    wl = WL.random_small(401, dtype="bf16", k=24, n_out=10, n=12, n_slots=3, max_rank=8,
                         kind="moe_grouped", n_experts=3)
    wl.null_slots = [4]  # adapter 1, expert 1
    st = o.scale_table(wl.adapters)
    r = o.route_for(wl, st)
    t = o.moe_grouped_shrink(r, wl.x, wl.expert_offsets, wl.row_slot)
    rng = np.random.default_rng(2)
    tin = rng.standard_normal((wl.n_rows, wl.max_rank)).astype(np.float32)
    yin = WL.f32_to_bf16_bits(rng.standard_normal((wl.n_rows, wl.n_out)).astype(np.float32))
    yo = o.moe_grouped_expand_fold(r, tin, wl.expert_offsets, wl.row_slot, yin)
    Ad, Bd, xd = (brute.widen(v, "bf16") for v in (wl.A, wl.B, wl.x))
    ex = _grouped_experts(wl.expert_offsets, wl.n_rows)
    live = 0
    for j in range(wl.n_rows):
        s, e = int(wl.row_slot[j]), int(ex[j])
        p = s * wl.n_experts + e
        if e >= 0 and brute.resolved(s, len(st), set(), st) and p not in wl.null_slots:
            live += 1
            _close(t[j], Ad[p] @ xd[j], 1e-12, f"grouped shrink row {j}")
            _close(yo[j], brute.widen(yin[j], "bf16") + float(st[s]) * (Bd[p] @ tin[j].astype(np.float64)),
                   1e-12, f"grouped expand row {j}")
        else:
            assert np.all(np.isnan(t[j])), f"skipped row {j} written"
            assert np.array_equal(yo[j], brute.widen(yin[j], "bf16")), f"skipped row {j} changed"
    assert live >= 4


def _stack_routes(o, wl, sts=None):
    levels = wl.meta["levels"]
    sts = sts or [o.scale_table(lv["adapters"]) for lv in levels]
    dt = _dt(wl)
    return [oracle.Route(lv["A"], lv["B"], st, dt, wl.k_in, wl.n_out, wl.max_rank)
            for lv, st in zip(levels, sts)], sts


@pin
def brute_force_tiny_stack(o):
    """ferrox LoraStack: W x + sum over levels of s_l B_l (A_l x), each level routed
    on its own; the brute force materialises W + sum_l s_l B_l A_l per row."""
    for seed in range(4):
        dtype = "bf16" if seed % 2 == 0 else "f32"
        wl = WL.random_stack(500 + seed, dtype=dtype, k=9, n_out=6, n=7, n_levels=2 + seed % 2,
                             n_slots=3, max_rank=4)
        routes, sts = _stack_routes(o, wl)
        levels = wl.meta["levels"]
        y = o.apply_stack(wl.W, routes, wl.x, [lv["seq_slot"] for lv in levels], _dt(wl))
        Wd, xd = brute.widen(wl.W, dtype), brute.widen(wl.x, dtype)
        for i in range(wl.n_rows):
            M = Wd.copy()
            for lv, st in zip(levels, sts):
                s = int(lv["seq_slot"][i])
                if brute.resolved(s, len(st), set(), st):
                    M = M + float(st[s]) * (brute.widen(lv["B"][s], dtype) @ brute.widen(lv["A"][s], dtype))
            _close(y[i], M @ xd[i], 1e-12, f"stack seed {seed} row {i}")


@pin
def stack_of_one_is_the_apply(o):
    """A stack with one adapter is that adapter's apply, bit for bit; a level whose
    rows all skip adds nothing, bit for bit (ferrox: a zero scale is skipped
    before any arithmetic)."""
    wl = WL.random_stack(510, dtype="bf16", k=20, n_out=12, n=9, n_levels=2, n_slots=3, max_rank=8)
    routes, sts = _stack_routes(o, wl)
    lv = wl.meta["levels"]
    one = o.apply_stack(wl.W, routes[:1], wl.x, [lv[0]["seq_slot"]], 1)
    assert np.array_equal(one, o.apply(wl.W, routes[0], wl.x, lv[0]["seq_slot"], 1))
    off = np.full(wl.n_rows, -1, np.int32)
    two = o.apply_stack(wl.W, routes, wl.x, [lv[0]["seq_slot"], off], 1)
    assert np.array_equal(two, one)


def _small_embed(seed, dtype, n_vocab=11, n_embd=9, n=8, max_rank=4, n_slots=3):
    rng = np.random.default_rng(seed)
    ranks = [int(v) for v in rng.integers(1, max_rank + 1, size=n_slots)]
    wl = WL.token_embedding(seed, n_vocab=n_vocab, n_embd=n_embd, n=n, n_slots=n_slots,
                            rank=max_rank, alpha=8.0, dtype=dtype, max_rank=max_rank, ranks=ranks)
    wl.meta["token_ids"] = wl.meta["token_ids"].copy()
    wl.meta["token_ids"][[1, n - 1]] = [n_vocab, -1]  # past the vocabulary: not written
    return wl


@pin
def brute_force_tiny_embed(o):
    """The row gather through the one-layout pair equals the row of the dense
    E + s A_file B_file^T formed straight from the file layout (the graph gathers
    a row of A_file per token and multiplies it by B_file)."""
    for seed in range(4):
        dtype = "bf16" if seed % 2 == 0 else "f32"
        wl = _small_embed(600 + seed, dtype)
        st = o.scale_table(wl.adapters)
        y = o.run(wl, scale_table=st)
        Ed = brute.widen(wl.W, dtype)
        tok, ss = wl.meta["token_ids"], wl.meta["seq_slot"]
        for i in range(wl.n_rows):
            t, s = int(tok[i]), int(ss[i])
            if not 0 <= t < wl.n_out:
                assert np.all(np.isnan(y[i])), f"row {i} with token {t} written"
                continue
            want = Ed[t].copy()
            if brute.resolved(s, len(st), set(), st):
                want = want + float(st[s]) * (brute.widen(wl.meta["a_file"][s], dtype)
                                              @ brute.widen(wl.meta["b_file"][s], dtype).T)[t]
            _close(y[i], want, 1e-12, f"embed seed {seed} row {i}")


@pin
def row_delta_agrees_with_the_matvec(o):
    """ferrox lora.rs test row_delta_agrees_with_the_matvec_on_a_unit_vector: row r
    of the gathered delta at column c is entry r of the matvec delta on e_c."""
    wl = _small_embed(610, "f32", n_vocab=6, n_embd=8, n=6)
    wl.meta["token_ids"] = np.arange(6, dtype=np.int32)
    wl.meta["seq_slot"] = np.full(6, 1, np.int32)
    wl.W = np.zeros_like(wl.W)
    st = o.scale_table(wl.adapters)
    rows = o.run(wl, scale_table=st)
    r = o.embed_route(wl, st)
    eye = np.eye(8, dtype=np.float32)
    cols = o.apply(np.zeros((6, 8), np.float32), r, eye, np.full(8, 1, np.int32), 0)  # [c][r]
    assert np.array_equal(rows, cols.T)
    assert np.any(rows != 0)


@pin
def brute_force_tiny_segmented(o):
    for seed in range(4):
        wl = WL.random_small(200 + seed, dtype="f32", k=10, n_out=5, n_slots=3, max_rank=4,
                             kind="segmented", seg_lens=[2, 0, 3, 1])
        st = o.scale_table(wl.adapters)
        y = o.apply_segmented(wl.W, o.route_for(wl, st), wl.x, wl.seg_indptr, wl.seg_slot, 0)
        slots = np.repeat(wl.seg_slot, np.diff(wl.seg_indptr))
        want = brute.dense_rows(wl.W, wl.A, wl.B, wl.x, "f32", slots, st)
        _close(y, want, 1e-12, f"segmented seed {seed}")


# ------------------------------------------------------------------ library special cases
@pin
def single_slot_is_one_matmul(o):
    """All rows on one slot: y = (W + s B A) X^T, one numpy product (P8)."""
    wl = WL.random_small(7, dtype="bf16", k=64, n_out=48, n=9, n_slots=2, max_rank=16)
    st = o.scale_table(wl.adapters)
    st[0] = np.float32(0.75)
    ss = np.zeros(wl.n_rows, np.int32)
    y = o.apply(wl.W, o.route_for(wl, st), wl.x, ss, 1)
    Wd, Ad, Bd, xd = (brute.widen(v, "bf16") for v in (wl.W, wl.A[0], wl.B[0], wl.x))
    want = xd @ (Wd + 0.75 * (Bd @ Ad)).T
    _close(y, want, 1e-12, "single slot")


@pin
def shrink_and_expand_match_matmul(o):
    wl = WL.random_small(8, dtype="bf16", k=40, n_out=24, n=10, n_slots=3, max_rank=8)
    st = o.scale_table(wl.adapters)
    ss = o.seq_slot_for(wl)
    r = o.route_for(wl, st)
    t = o.shrink(r, wl.x, ss)
    Ad, Bd, xd = (brute.widen(v, "bf16") for v in (wl.A, wl.B, wl.x))
    rng = np.random.default_rng(0)
    tin = rng.standard_normal((wl.n_rows, wl.max_rank)).astype(np.float32)
    yin = WL.f32_to_bf16_bits(rng.standard_normal((wl.n_rows, wl.n_out)).astype(np.float32))
    yo = o.expand_fold(r, tin, ss, yin)
    for i in range(wl.n_rows):
        s = int(ss[i])
        if brute.resolved(s, len(st), set(), st):
            _close(t[i], Ad[s] @ xd[i], 1e-12, f"shrink row {i}")
            _close(yo[i], brute.widen(yin[i], "bf16") + float(st[s]) * (Bd[s] @ tin[i].astype(np.float64)),
                   1e-12, f"expand row {i}")
        else:
            assert np.all(np.isnan(t[i])), f"skipped row {i} written"
            assert np.array_equal(yo[i], brute.widen(yin[i], "bf16")), f"skipped row {i} changed"


# ------------------------------------------------------------------ invariants
@pin
def skip_rows_equal_base_bit_for_bit(o):
    """ferrox lora.rs 'Cost when absent' and test a_zero_scale_adds_nothing_bit_for_bit;
    atlas apply_lora_bgmv doc: slot < 0, NULL and zero-scale slots are base."""
    wl = WL.random_small(9, dtype="bf16", k=33, n_out=20, n=16, n_slots=5, max_rank=8)
    wl.null_slots = [3]
    st = o.scale_table(wl.adapters)
    st[1] = 0.0
    ss = np.array([0, 1, 2, 3, 4, 5, -1, -7, 1, 3, 0, 2, -1, 9, 4, 1], np.int32)
    y = o.apply(wl.W, o.route_for(wl, st), wl.x, ss, 1)
    base = o.apply(wl.W, None, wl.x, None, 1)
    skipped = [i for i, s in enumerate(ss) if not brute.resolved(int(s), 5, {3}, st)]
    assert set(skipped) == {1, 3, 5, 6, 7, 8, 9, 12, 13, 15}
    assert np.array_equal(y[skipped], base[skipped])
    live = [i for i in range(16) if i not in skipped]
    assert not np.any(y[live] == base[live])


@pin
def split_equals_stacked(o):
    """frink lora_attach.rs module doc: B (A x) over stacked rows IS the stacked B_i (A x)."""
    wl = WL.random_small(10, dtype="bf16", k=48, n_out=32, n=7, n_slots=3, max_rank=8)
    st = o.scale_table(wl.adapters)
    ss = o.seq_slot_for(wl)
    full = o.apply(wl.W, o.route_for(wl, st), wl.x, ss, 1)
    for lo, hi in ((0, 12), (12, 32)):
        r = o.route_for(wl, st, b_row_offset=lo, n_out=hi - lo)
        part = o.apply(wl.W[lo:hi], r, wl.x, ss, 1)
        assert np.array_equal(part, full[:, lo:hi]), (lo, hi)


@pin
def batch_equals_per_position(o):
    """ferrox lora.rs test batch_delta_is_the_matvec_delta_per_position; atlas
    apply_lora_bgmv doc: byte-identical to n sequential one-row calls."""
    wl = WL.random_small(11, dtype="f32", k=20, n_out=9, n=8, n_slots=3, max_rank=4)
    st = o.scale_table(wl.adapters)
    ss = o.seq_slot_for(wl)
    r = o.route_for(wl, st)
    y = o.apply(wl.W, r, wl.x, ss, 0)
    for i in range(wl.n_rows):
        yi = o.apply(wl.W, r, wl.x[i:i + 1], ss[i:i + 1], 0)
        assert np.array_equal(yi[0], y[i]), i


@pin
def padded_equals_true_rank(o):
    """atlas lora_delta.rs LoraPair doc: running at max_rank over zero pads is
    bit-identical to the true-rank product."""
    wl = WL.random_small(12, dtype="bf16", k=30, n_out=14, n=6, n_slots=3, max_rank=8,
                         ranks=[2, 5, 8])
    st = o.scale_table(wl.adapters)
    ss = o.seq_slot_for(wl)
    y = o.apply(wl.W, o.route_for(wl, st), wl.x, ss, 1)
    for i in range(wl.n_rows):
        s = int(ss[i])
        if not brute.resolved(s, 3, set(), st):
            continue
        A = wl.A_true[s][None]
        B = wl.B_true[s][None]
        r = len(wl.A_true[s])
        tw = WL.Workload(name="t", dtype="bf16", k_in=wl.k_in, n_out=wl.n_out, max_rank=r,
                         W=wl.W, A=A, B=B, x=wl.x, adapters=[wl.adapters[s]])
        yt = o.apply(wl.W, o.route_for(tw, st[s:s + 1]), wl.x[i:i + 1], [0], 1)
        assert np.array_equal(yt[0], y[i]), i


@pin
def scale_read_at_apply_time(o):
    """ferrox lora.rs test the_scale_is_read_at_apply_time: halving the scale halves the delta."""
    wl = WL.random_small(13, dtype="bf16", k=16, n_out=12, n=5, n_slots=2, max_rank=4)
    st = np.array([1.5, -0.25], np.float32)
    ss = np.array([0, 1, 0, 1, 0], np.int32)
    rng = np.random.default_rng(1)
    t = rng.standard_normal((5, 4)).astype(np.float32)
    y0 = WL.f32_to_bf16_bits(np.zeros((5, 12), np.float32))
    d1 = o.expand_fold(o.route_for(wl, st), t, ss, y0)
    d2 = o.expand_fold(o.route_for(wl, st * np.float32(0.5)), t, ss, y0)
    assert np.array_equal(d2, d1 * 0.5)
    assert not np.all(d1 == 0)


@pin
def integer_routing_exact(o):
    """Exact small integers: every row's result is an integer the brute force
    computes exactly, so a wrong slot, a dropped row or a wrong expert shows."""
    rng = np.random.default_rng(5)
    k, n_out, R, S = 12, 10, 4, 4
    W = rng.integers(-2, 3, (n_out, k)).astype(np.float32)
    A = rng.integers(-2, 3, (S, R, k)).astype(np.float32)
    P = rng.choice([-1.0, 1.0], (n_out, R)).astype(np.float32)
    B = np.stack([(s + 1) * P for s in range(S)]).astype(np.float32)
    x = rng.integers(-2, 3, (9, k)).astype(np.float32)
    st = np.array([1.0, 2.0, 0.5, 0.0], np.float32)
    ss = np.array([0, 1, 2, 3, -1, 4, 1, 0, 2], np.int32)
    wl = WL.Workload(name="int", dtype="f32", k_in=k, n_out=n_out, max_rank=R, W=W, A=A, B=B,
                     x=x, adapters=[WL.AdapterSpec(R, 0.0, 1.0)] * S)
    y = o.apply(W, o.route_for(wl, st), x, ss, 0)
    Wi, Ai, Bi, xi = (v.astype(np.int64) for v in (W, A, B, x))
    for i, s in enumerate(ss):
        want = Wi @ xi[i]
        if 0 <= s < S and st[s] != 0:
            want = want * 2 + int(st[s] * 2) * (Bi[s] @ (Ai[s] @ xi[i]))
            want = want / 2.0
        assert np.array_equal(y[i], want.astype(np.float64)), (i, s)


@pin
def row_subsets_equal_the_full_call(o):
    """Every entry point that takes a list of rows (the sampled checks at full
    size use them) gives, for a list in any order and with a repeat, exactly the
    full call's outputs of the listed rows, position by position: a subset that
    read another row's input or slot, or wrote another position, would show."""
    rows = np.array([5, 0, 3, 5, 7, 2], np.int32)

    def same(full, sub, what):
        assert np.array_equal(sub, full[rows], equal_nan=True), what
        assert not np.all(np.isnan(sub)), what

    wl = WL.random_small(700, dtype="bf16", k=14, n_out=9, n=8, n_slots=4, max_rank=4)
    st = o.scale_table(wl.adapters)
    ss = np.array([1, -1, 0, 2, 3, 0, 9, 1], np.int32)
    r = o.route_for(wl, st)
    same(o.apply(wl.W, r, wl.x, ss, 1), o.apply(wl.W, r, wl.x, ss, 1, rows=rows), "apply")
    wl = WL.random_small(701, dtype="f32", k=10, n_out=6, n_slots=3, max_rank=4,
                         kind="segmented", seg_lens=[2, 3, 0, 3])
    r = o.route_for(wl, o.scale_table(wl.adapters))
    same(o.apply_segmented(wl.W, r, wl.x, wl.seg_indptr, wl.seg_slot, 0),
         o.apply_segmented(wl.W, r, wl.x, wl.seg_indptr, wl.seg_slot, 0, rows=rows), "segmented")
    wl = WL.random_small(702, dtype="bf16", k=9, n_out=6, n=4, n_slots=3, max_rank=4,
                         kind="moe", n_experts=4, top_k=2)
    r = o.route_for(wl, o.scale_table(wl.adapters))
    same(o.apply_moe(wl.W, r, wl.x, wl.indices, wl.top_k, wl.token_slot, 1),
         o.apply_moe(wl.W, r, wl.x, wl.indices, wl.top_k, wl.token_slot, 1, rows=rows), "moe")
    wl = WL.random_small(703, dtype="bf16", k=10, n_out=7, n=9, n_slots=3, max_rank=4,
                         kind="moe_grouped", n_experts=4)
    r = o.route_for(wl, o.scale_table(wl.adapters))
    same(o.apply_moe_grouped(wl.W, r, wl.x, wl.expert_offsets, wl.row_slot, 1),
         o.apply_moe_grouped(wl.W, r, wl.x, wl.expert_offsets, wl.row_slot, 1, rows=rows),
         "moe grouped")
    wl = WL.random_stack(704, dtype="bf16", k=9, n_out=6, n=8, n_levels=2, n_slots=3, max_rank=4)
    routes, _ = _stack_routes(o, wl)
    sl = [lv["seq_slot"] for lv in wl.meta["levels"]]
    same(o.apply_stack(wl.W, routes, wl.x, sl, 1), o.apply_stack(wl.W, routes, wl.x, sl, 1, rows=rows),
         "stack")
    wl = _small_embed(705, "bf16")
    wl.meta["token_ids"][[0, 3]] = [4, 4]  # two rows on one token, different slots
    wl.meta["seq_slot"][[0, 3]] = [0, 1]
    st = o.scale_table(wl.adapters)
    same(o.run(wl, scale_table=st), o.run(wl, rows=rows, scale_table=st), "embed")
