#!/usr/bin/env python3
"""Benchmark of the routed multi-LoRA projection on one MI355X (gfx950).

A step is one pass of the whole hot path over one batch: the fused apply
(route resolve, row plan and grouped shrink in the prep kernel; base
contraction, expand and fold in the fused GEMM) through the C ABI.  The
headline workload is the decode bgmv batch: q_proj W 4096x4096 bf16, a pool
of 16 rank-16 adapters (alpha 32), 57 real rows padded to 64 with slot -1.

Method:
  * inputs are synthetic (seed 0) and resident in HBM before timing starts;
  * every step uses the next of R device copies of the inputs (W, x, the
    adapter pool, the routing, y), so a step never finds its data in the
    256 MiB last-level cache or the L2; the copies share one workspace, as
    the calls of one projection do;
  * W untimed warmup steps run eagerly; the timed region is one replay of a
    HIP graph of exactly K consecutive steps (what a serving loop does; the
    library allocates and synchronises nothing), bracketed by synchronize()
    on both sides; the graph's result is then checked against an eager step;
  * the dominant kernel's time comes from HIP events the library records
    around its kernels (lora_set_profile_events) over K further steps
    launched eagerly -- the same kernels on the same rotation;
  * the oracle (plain fp64 C, OpenMP over rows) is timed on the host cores
    over whole batches of the same workload, as a baseline only: the median
    of three samples on all cores, and one sample on one core.

Prints one JSON line.  `--gpus N` with N > 1 is refused: this build measures
one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "adapted rows/s + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill) vs peak"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published

WORKLOAD_TEXT = {
    "single_projection_f32": "single projection f32: W 256x256, 1 adapter r=8 alpha 16, 4 rows on slot 0",
    "decode_bgmv": "decode bgmv: q_proj W 4096x4096 bf16, 16 slots r=16 alpha 32, 57 real rows + 7 pad rows (slot -1)",
    "fused_gate_up": "fused gate/up: W 22016x4096 bf16, 32 slots r in {8,16,32,64} padded to 64, rsLoRA alpha 16, 8 slots at scale 0, 256 rows",
    "prefill_segmented": "prefill segmented: o_proj W 4096x4096 bf16, 8 segments x 512 tokens, one rank-64 adapter each",
    "moe_down_gather": "MoE down_proj gather: 64 experts W_e 2048x1408 bf16, 512 tokens top-6, rank-16 pair per (adapter, expert), 4 adapters",
    "moe_down_grouped": "MoE down_proj grouped: 64 experts W_e 2048x1408 bf16, 2048 tokens top-6 = 12288 rows sorted by expert (expert_offsets), rank-16 pair per (adapter, expert), 4 adapters",
    "adapter_stack": "adapter stack: q_proj W 4096x4096 bf16, 3 levels x 8 slots r=16 alpha 32, 64 rows, each level's slot per row uniform in [-1, 8)",
    "token_embedding": "token-embedding gather: E 32000x4096 bf16, 8 adapters r=16 alpha 32 stored flipped (A_file [n_vocab][r], B_file [n_embd][r]), 4096 tokens uniform over the vocabulary, slots uniform in [-1, 8)",
    "spec_verify_kv": "speculative verify, K projection: W_k 1024x4096 bf16, 16 slots r=16 alpha 32, 4 sequences x 9 draft tokens = 36 rows, output into the K columns of interleaved [Q|K|V] rows (6144 elements)",
}
ROTATE = {"single_projection_f32": 4, "decode_bgmv": 16, "fused_gate_up": 4,
          "prefill_segmented": 8, "moe_down_gather": 2, "moe_down_grouped": 2,
          "spec_verify_kv": 64, "adapter_stack": 16, "token_embedding": 2}
BOUND = {"single_projection_f32": "latency", "decode_bgmv": "hbm", "fused_gate_up": "hbm",
         "prefill_segmented": "mfma", "moe_down_gather": "hbm", "moe_down_grouped": "hbm",
         "spec_verify_kv": "latency", "adapter_stack": "hbm", "token_embedding": "hbm"}
# the five workloads of the path, then the variants built beyond them
OTHERS = ("single_projection_f32", "fused_gate_up", "prefill_segmented", "moe_down_gather",
          "moe_down_grouped", "spec_verify_kv", "adapter_stack", "token_embedding")


def device_kwargs(wl):
    """Output placement of a workload: the verify K fold writes into [Q|K|V] rows."""
    if wl.name.startswith("spec_verify_kv"):
        return {"y_col_offset": wl.meta["q_dim"], "y_extra_cols": wl.meta["kv_dim"]}
    return {}


def workload(name):
    from adapter_lora_bgmv_amd import workloads as WL
    return {**WL.CONFIGS, **WL.NEXT_WORKLOADS}[name]()


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=320)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--config", default="decode_bgmv")
    p.add_argument("--no-others", action="store_true", help="skip the other workloads")
    p.add_argument("--others", default=None,
                   help="comma-separated subset of the other workloads (decode_bgmv_pair is one)")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    p.add_argument("--no-base", action="store_true", help="skip the base-only (no adapter) timing")
    p.add_argument("--cpu-seconds", type=float, default=5.0)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run one 256 MiB device copy, a known-size reference for "
                        "hardware byte counters")
    return p.parse_args()


# ------------------------------------------------------------------ algorithmic counts
def resolve_rows(wl, scale_table):
    """Per row: the pool index of its pair, or -1 (no delta); dropped rows -2."""
    from adapter_lora_bgmv_amd import binding as B
    P = len(scale_table)
    if wl.kind == "decode":
        ss = wl.meta.get("seq_slot")
        if ss is None:
            ss = B.lora_build_seq_slot(wl.adapter_slots, wl.padded_n, wl.active)
        pairs = [int(s) if 0 <= s < P and scale_table[s] != 0 else -1 for s in ss]
        return np.array(pairs), np.zeros(len(ss), int)
    if wl.kind == "segmented":
        pairs = np.full(wl.n_rows, -2)
        for g in range(len(wl.seg_slot)):
            s = int(wl.seg_slot[g])
            v = s if 0 <= s < P and scale_table[s] != 0 else -1
            pairs[wl.seg_indptr[g]:wl.seg_indptr[g + 1]] = v
        return pairs, np.zeros(wl.n_rows, int)
    E = wl.n_experts
    pairs, groups = [], []
    if wl.kind == "moe_grouped":
        off = wl.expert_offsets
        for j in range(wl.n_rows):
            e = int(np.searchsorted(off, j, side="right")) - 1
            if j < off[0] or j >= off[-1]:
                pairs.append(-2)
                groups.append(0)
                continue
            a = int(wl.row_slot[j])
            groups.append(e)
            pairs.append(a * E + e if 0 <= a < P and scale_table[a] != 0 else -1)
        return np.array(pairs), np.array(groups)
    for j in range(wl.n_rows):
        e = int(wl.indices[j])
        a = int(wl.token_slot[j // wl.top_k])
        groups.append(e)
        pairs.append(a * E + e if 0 <= a < P and scale_table[a] != 0 else -1)
    return np.array(pairs), np.array(groups)


def stack_counts(wl, scale_tables):
    """An adapter stack: W, x and y once; every level's touched slots' A and B once."""
    esz = 2 if wl.dtype == "bf16" else 4
    R, k, o, n = wl.max_rank, wl.k_in, wl.n_out, wl.n_rows
    live = np.zeros(n, bool)
    a_bytes = b_bytes = 0
    lora_flops = expand_flops = 0.0
    first = None
    for lv, st in zip(wl.meta["levels"], scale_tables):
        ss = lv["seq_slot"]
        ok = np.array([0 <= s < len(st) and st[s] != 0 for s in ss])
        touched = len(set(int(s) for s, g in zip(ss, ok) if g))
        a_bytes += touched * R * k * esz
        b_bytes += touched * o * R * esz
        lora_flops += 2.0 * ok.sum() * R * (k + o)
        expand_flops += 2.0 * ok.sum() * R * o
        live |= ok
        if first is None:
            first = (touched * R * k * esz, 2.0 * ok.sum() * R * k)
    w_bytes, x_bytes, y_bytes = o * k * esz, n * k * esz, n * o * esz
    return {"rows": n, "adapted_rows": int(live.sum()), "touched_pairs": None,
            "path_bytes": w_bytes + a_bytes + b_bytes + x_bytes + y_bytes,
            "path_flops": 2.0 * n * o * k + lora_flops,
            # the decode launch: W, x and y once, the first level's touched A
            # (its shrink rides the launch) and every level's touched B; the
            # further levels' A are read by the launch before it
            "main_bytes": w_bytes + x_bytes + y_bytes + first[0] + b_bytes,
            "main_flops": 2.0 * n * o * k + first[1] + expand_flops,
            "main_kernel": "decode_kernel (base + split-K reduction + first level's shrink + every level's expand and fold)"}


def embed_counts(wl, scale_table):
    """A token-embedding gather: the gathered rows of E, each touched slot's A once,
    one row of B per adapted row, y once (plus the token ids and slots)."""
    esz = 2 if wl.dtype == "bf16" else 4
    R, ne, nv = wl.max_rank, wl.k_in, wl.n_out
    tok, ss = wl.meta["token_ids"], wl.meta["seq_slot"]
    live = (tok >= 0) & (tok < nv)
    ok = live & np.array([0 <= s < len(scale_table) and scale_table[s] != 0 for s in ss])
    touched = len(set(int(s) for s, g in zip(ss, ok) if g))
    n = int(live.sum())
    path = n * ne * esz * 2 + touched * R * ne * esz + int(ok.sum()) * R * esz + len(tok) * 8
    flops = 2.0 * int(ok.sum()) * R * ne
    return {"rows": n, "adapted_rows": int(ok.sum()), "touched_pairs": touched,
            "path_bytes": path, "path_flops": flops, "main_bytes": path, "main_flops": flops,
            "main_kernel": "embed_rows_kernel (row gather + delta)"}


def algorithmic_counts(wl, scale_table):
    """Algorithmic bytes and flops: W once (each expert that has rows), each touched
    nonzero-scale pair's A and B once at max_rank, x once, y once."""
    if wl.kind == "stack":
        return stack_counts(wl, scale_table)
    if wl.kind == "embed":
        return embed_counts(wl, scale_table)
    esz = 2 if wl.dtype == "bf16" else 4
    pairs, groups = resolve_rows(wl, scale_table)
    live = pairs[pairs >= -1]
    n = len(live)
    active = int((pairs >= 0).sum())
    touched = len(set(int(p) for p in pairs if p >= 0))
    R, k, o = wl.max_rank, wl.k_in, wl.n_out
    w_bytes = (len(set(groups[pairs >= -1].tolist())) if wl.kind in ("moe", "moe_grouped") else 1) * o * k * esz
    a_bytes = touched * R * k * esz
    b_bytes = touched * o * R * esz
    x_bytes = n * k * esz
    y_bytes = n * o * esz
    t_bytes = active * R * 4
    base_flops = 2.0 * n * o * k
    shrink_flops = 2.0 * active * R * k
    expand_flops = 2.0 * active * R * o
    out = {
        "rows": n, "adapted_rows": active, "touched_pairs": touched,
        "path_bytes": w_bytes + a_bytes + b_bytes + x_bytes + y_bytes,
        "path_flops": base_flops + shrink_flops + expand_flops,
    }
    if decode_path(wl):
        # one launch moves everything: W, x, the touched A and B, y
        out.update(main_bytes=out["path_bytes"], main_flops=out["path_flops"],
                   main_kernel="decode_kernel (base + split-K reduction + shrink + expand + fold, one launch)")
    else:
        # the fused GEMM: W, touched B, x, y, and the f32 t it reads
        out.update(main_bytes=w_bytes + b_bytes + x_bytes + y_bytes + t_bytes, main_flops=base_flops + expand_flops,
                   main_kernel="gemm_bf16_kernel (fused base + expand + fold)")
    return out


def decode_path(wl):
    """The decode kernels take lora_apply batches of at most 64 rows in bf16."""
    return wl.kind in ("decode", "stack") and wl.dtype == "bf16" and len(wl.x) <= 64


# ------------------------------------------------------------------ GPU timing
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def hip_timing_events(n):
    """n HIP events for timing only: no system-scope fence when recorded, so a
    record adds no cache writeback to the span it closes.  The HIP runtime is
    the one torch loaded (same soname)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        rc = hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        evs.append(e)
    return hip, evs


def hip_elapsed_ms(hip, a, b):
    import ctypes
    ms = ctypes.c_float()
    rc = hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
    return ms.value


def time_workload(name, steps, warmup, apply=True):
    import torch
    from adapter_lora_bgmv_amd import binding as B
    from adapter_lora_bgmv_amd import workloads as WL
    from adapter_lora_bgmv_amd.harness import DeviceWorkload

    wl = workload(name)
    R = ROTATE[name]
    dws = [DeviceWorkload(wl, **device_kwargs(wl)) for _ in range(R)]
    # one workspace for every copy, as one projection's calls share theirs
    for d in dws[1:]:
        d.workspace = dws[0].workspace
    counts = algorithmic_counts(wl, dws[0].scale_table_host)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(warmup):
            dws[i % R].run(route=apply)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    # one graph of exactly `steps` consecutive steps, cycling over the copies
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            dws[i % R].run(route=apply)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    # the graph's last write to copy 0 against an eager step on the same inputs
    got = dws[0].y_bits()
    dws[0].run(route=apply)
    torch.cuda.synchronize()
    if not np.array_equal(dws[0].y_bits(), got):
        raise RuntimeError(f"{name}: graph replay differs from the eager result")
    del g

    # per-kernel durations: HIP events the library records around its
    # kernels, created without the system-scope fence (timing-only events)
    hip, evs = hip_timing_events(4 * steps)
    for i in range(steps):
        B.lora_set_profile_events([evs[4 * i + j].value for j in range(4)])
        dws[i % R].run(route=apply)
    B.lora_set_profile_events(None)
    torch.cuda.synchronize()
    spans = np.array([[hip_elapsed_ms(hip, evs[4 * i + a], evs[4 * i + a + 1]) for a in range(3)]
                      for i in range(steps)])
    prep_ms, main_ms, post_ms = spans[:, 0], spans[:, 1], spans[:, 2]
    for e in evs:
        hip.hipEventDestroy(e)
    return wl, counts, {"steps": steps, "rotate": R, "ms_per_step": ms_per_step,
                        "prep_us_mean": float(prep_ms.mean() * 1e3),
                        "main_us_mean": float(main_ms.mean() * 1e3),
                        "main_us_median": float(np.median(main_ms) * 1e3),
                        "post_us_mean": float(post_ms.mean() * 1e3)}


def time_pair(steps, warmup):
    """The standalone two-step delta on the decode workload: lora_shrink then
    lora_expand_fold (y += s B t in place), one graph of `steps` steps over
    rotated input copies.  Its bytes: the touched A and B once, the adapted
    rows' x, y read and written, t written and read."""
    import torch
    from adapter_lora_bgmv_amd import binding as B
    from adapter_lora_bgmv_amd.harness import DeviceWorkload

    wl = workload("decode_bgmv")
    R = ROTATE["decode_bgmv"]
    dws = [DeviceWorkload(wl) for _ in range(R)]
    ts = [torch.empty(d.n, wl.max_rank, dtype=torch.float32, device="cuda") for d in dws]

    def step(i, stream=None):
        d = dws[i % R]
        B.lora_shrink(d.route, d.x, d.x_row_stride, d.seq_slot, d.n, ts[i % R], stream)
        B.lora_expand_fold(d.route, ts[i % R], d.seq_slot, d.n, d.y, d.y_row_stride, stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for i in range(steps):
            step(i, side)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    del g
    pairs, _ = resolve_rows(wl, dws[0].scale_table_host)
    active = int((pairs >= 0).sum())
    touched = len(set(int(q) for q in pairs if q >= 0))
    Rk, k, o = wl.max_rank, wl.k_in, wl.n_out
    path = touched * Rk * (k + o) * 2 + active * k * 2 + 2 * active * o * 2 + 2 * active * Rk * 4
    flops = 2.0 * active * Rk * (k + o)
    step_s = ms_per_step * 1e-3
    return {"workload": "decode bgmv pair: lora_shrink + lora_expand_fold on the decode batch "
                        "(16 slots r=16 over 4096 x 4096, 57 adapted rows), y += s B (A x) in place",
            "ms_per_step": round(ms_per_step, 5), "rows_per_s": active / step_s,
            "path_GBps": path / step_s / 1e9, "path_TFLOPs": flops / step_s / 1e12, "bound": "hbm",
            "algorithmic_bytes": path, "algorithmic_flops": flops,
            "frac_of_peak": path / step_s / 1e9 / HBM_PEAK_GBPS,
            "kernels": "bgmv_shrink_kernel + bgmv_expand_kernel (two launches)"}


def summarize(name, counts, t, base_t=None):
    main_s = t["main_us_mean"] * 1e-6
    step_s = t["ms_per_step"] * 1e-3
    out = {
        "workload": WORKLOAD_TEXT[name],
        "ms_per_step": round(t["ms_per_step"], 5),
        "rows_per_s": counts["adapted_rows"] / step_s if counts["adapted_rows"] else counts["rows"] / step_s,
        "prep_us": round(t["prep_us_mean"], 2),
        "main_us": round(t["main_us_mean"], 2),
        "post_us": round(t["post_us_mean"], 2),
        "path_GBps": counts["path_bytes"] / step_s / 1e9,
        "path_TFLOPs": counts["path_flops"] / step_s / 1e12,
        "main_GBps": counts["main_bytes"] / main_s / 1e9,
        "main_TFLOPs": counts["main_flops"] / main_s / 1e12,
        "bound": BOUND[name],
        "algorithmic_bytes": counts["path_bytes"],
        "algorithmic_flops": counts["path_flops"],
    }
    if BOUND[name] == "mfma":
        out["frac_of_peak"] = out["main_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
    elif BOUND[name] == "hbm":
        out["frac_of_peak"] = out["main_GBps"] / HBM_PEAK_GBPS
    traffic = measured_traffic(counts["main_kernel"].split(" ")[0], name)
    if traffic is not None:
        out["traffic"] = traffic
    if base_t is not None:
        out["base_only_ms_per_step"] = round(base_t["ms_per_step"], 5)
        out["base_only_main_us"] = round(base_t["main_us_mean"], 2)
    return out


# ------------------------------------------------------------------ counters
def measured_traffic(kernel, workload):
    """HBM bytes per dispatch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs, or None when there are none for this kernel and workload or they were
    taken on different kernel or host sources."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", "hbm_traffic.json")) as f:
            rec = json.load(f).get(f"{kernel}:{workload}")
        if not rec:
            return None
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(root, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return rec["fetch_bytes_per_dispatch"] + rec["write_bytes_per_dispatch"]
    except (OSError, ValueError, KeyError):
        return None


# ------------------------------------------------------------------ CPU baseline
# rows of each workload the oracle baseline times per batch (None: all of
# them); a seeded sample keeps every config's CPU time bounded
CPU_SAMPLE_ROWS = {"single_projection_f32": None, "decode_bgmv": None, "fused_gate_up": 32,
                   "prefill_segmented": 32, "moe_down_gather": 96}


def cpu_baseline(name, seconds):
    """The oracle over batches of the workload (or a seeded sample of its rows):
    the median of three samples of about `seconds` each on all host threads,
    and one on one thread, in rows of the workload per second."""
    import oracle
    wl = workload(name)
    orc = oracle.get()
    st = orc.scale_table(wl.adapters)
    counts = algorithmic_counts(wl, st)
    n_rows = counts["rows"]
    k = CPU_SAMPLE_ROWS.get(name)
    rows = None
    if k is not None and k < n_rows:
        rows = np.sort(np.random.default_rng(0).choice(len(wl.x), size=k, replace=False)).astype(np.int32)
    # rows/s: adapted rows per batch for the decode batch (the headline's unit),
    # otherwise every row
    per_batch = (counts["adapted_rows"] if name == "decode_bgmv" else n_rows) if rows is None else len(rows)

    def sample():
        reps = 0
        t0 = time.perf_counter()
        while True:
            orc.run(wl, rows=rows, scale_table=st)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 1000:
                return reps, el

    cores = orc.threads
    samples = [sample() for _ in range(3)]
    rates = sorted(per_batch * r / e for r, e in samples)
    orc.set_threads(1)
    try:
        r1, e1 = sample()
    finally:
        orc.set_threads(cores)
    what = (f"whole {name} batches ({counts['rows']} rows, {counts['adapted_rows']} adapted)" if rows is None
            else f"a seeded sample of {len(rows)} of the {n_rows} rows of {name}")
    return {"value": rates[1], "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"median of 3 samples of {what} through the fp64 oracle, "
                      f"{', '.join(f'{r} in {e:.1f} s' for r, e in samples)}",
            "samples": rates,
            "single_core": {"value": per_batch * r1 / e1, "unit": "rows/s", "cores": 1,
                            "sample": f"{r1} batches in {e1:.1f} s"}}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported by this build "
              "(the projection would shard by output rows, one block of W and B per GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    from adapter_lora_bgmv_amd import binding as B
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    B.lora_init()
    if a.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    name = a.config
    print(f"# bench: {name} steps={a.steps} warmup={a.warmup}", file=sys.stderr, flush=True)
    wl, counts, t = time_workload(name, a.steps, a.warmup)
    tb = None if a.no_base else time_workload(name, a.steps, a.warmup, apply=False)[2]
    head = summarize(name, counts, t, tb)
    print(f"# {name}: {json.dumps(head)}", file=sys.stderr, flush=True)

    others = {}
    pick = set(a.others.split(",")) if a.others else None
    if not a.no_others and name == "decode_bgmv" and (pick is None or "decode_bgmv_pair" in pick):
        others["decode_bgmv_pair"] = time_pair(min(a.steps, 64), 8)
        print(f"# decode_bgmv_pair: {json.dumps(others['decode_bgmv_pair'])}", file=sys.stderr, flush=True)
    if not a.no_others:
        for other in OTHERS:
            if other == name or (pick is not None and other not in pick):
                continue
            _, c2, t2 = time_workload(other, min(a.steps, 64), 8)
            others[other] = summarize(other, c2, t2)
            if not a.no_cpu and other in CPU_SAMPLE_ROWS:
                others[other]["cpu_baseline"] = cpu_baseline(other, a.cpu_seconds / 2)
            print(f"# {other}: {json.dumps(others[other])}", file=sys.stderr, flush=True)

    bound = BOUND[name]
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": head["main_TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": head["main_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the same bytes (or flops) over the whole step, launch gaps included
    roof["step_frac"] = (head["path_TFLOPs"] if bound == "mfma" else head["path_GBps"]) / roof["peak"]
    kname = counts["main_kernel"].split(" ")[0]
    roof["traffic"] = measured_traffic(kname, name)
    roof["kernel"] = counts["main_kernel"]
    roof["algorithmic_bytes_per_launch"] = counts["main_bytes"]
    roof["avg_launch_us"] = head["main_us"]

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(name, a.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": head["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": t["steps"],
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seed 0), inputs resident in HBM, rotated over "
                f"{t['rotate']} copies so each step reads uncached data; one workspace",
        "config": {"workload": WORKLOAD_TEXT[name], "rows": counts["rows"],
                   "adapted_rows": counts["adapted_rows"], "touched_slots": counts["touched_pairs"],
                   "path_GBps": head["path_GBps"], "path_frac_of_hbm_peak": head["path_GBps"] / HBM_PEAK_GBPS,
                   "prep_us": head["prep_us"], "main_us": head["main_us"], "post_us": head["post_us"],
                   "base_only_ms_per_step": head.get("base_only_ms_per_step"),
                   "base_only_main_us": head.get("base_only_main_us")},
        "roofline": roof,
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
