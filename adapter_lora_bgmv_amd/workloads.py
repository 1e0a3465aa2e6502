"""Seeded synthetic inputs for the routed multi-LoRA projection.

This module is shared by the HIP path's callers (tests, bench) and by the CPU
oracle's tests, so it deliberately holds none of the method's arithmetic: no
scale formula, no slot resolution, no products.  It only draws numbers, rounds
them to the storage type, and lays them out the way the adapter pool stores
them (ferrox ``lora.rs`` "Layouts": A is ``[rank][cols]``, B is
``[rows][rank]``; atlas ``lora_delta.rs`` ``LoraPair``: both zero-padded to the
pool's ``max_rank``; metrale ``slot_math.rs`` module header: per slot, A then B).

Every workload is drawn from ``numpy.random.default_rng(seed)`` in a fixed
order -- W, A pool, B pool, x, routing -- as fp64 normals times sigma, rounded
to f32 and then (for bf16 workloads) to bf16 with round-to-nearest-even.
Rank padding is written after the draw, so padded and unpadded pools hold the
same real values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round f32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # in 32 bits: only NaN patterns can wrap, and they are replaced below
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to f32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _store(vals_f64: np.ndarray, dtype: str) -> np.ndarray:
    v32 = vals_f64.astype(np.float32)
    return f32_to_bf16_bits(v32) if dtype == BF16 else v32


# ---------------------------------------------------------------- adapters
@dataclass
class AdapterSpec:
    """Hyper-parameters of one adapter slot, as an adapter file carries them."""

    rank: int                 # true rank r (scale uses this, never max_rank)
    alpha: float              # lora_alpha; 0 means "absent"
    adapter_scale: float = 1.0
    rslora: bool = False


@dataclass
class Workload:
    """One batch of routed-LoRA input, host side.

    Routing comes in the raw form a serving engine holds it; each consumer
    (the HIP path's host helpers, the oracle) turns it into a per-row slot
    buffer and a scale table with its own code.
    """

    name: str
    dtype: str
    k_in: int
    n_out: int
    max_rank: int
    W: np.ndarray                      # [n_out][k_in] (dense) or [E][n_out][k_in] (moe)
    A: np.ndarray                      # [P][max_rank][k_in], pad rows zero
    B: np.ndarray                      # [P][n_out][max_rank], pad cols zero
    x: np.ndarray                      # [n][k_in]
    adapters: List[AdapterSpec]        # one per pool slot (moe: per adapter)
    kind: str = "decode"               # decode | segmented | moe | moe_grouped | stack | embed
    # decode routing (metrale slot_math.rs build_seq_slot_host inputs)
    adapter_slots: Optional[np.ndarray] = None   # [n_real] int32, <0 = active
    padded_n: int = 0
    active: int = 0
    # segmented routing
    seg_indptr: Optional[np.ndarray] = None      # [n_seg+1] int32
    seg_slot: Optional[np.ndarray] = None        # [n_seg] int32
    # moe routing
    n_experts: int = 0
    top_k: int = 0
    indices: Optional[np.ndarray] = None         # [n_tokens*top_k] int32, slot-major
    token_slot: Optional[np.ndarray] = None      # [n_tokens] int32
    # moe grouped routing: rows sorted by expert
    expert_offsets: Optional[np.ndarray] = None  # [n_experts+1] int32, non-decreasing
    row_slot: Optional[np.ndarray] = None        # [n] int32, each sorted row's adapter slot
    # slots whose table entry is NULL (a base-only slot), by pool index
    null_slots: List[int] = field(default_factory=list)
    # the true-rank (unpadded) pool, for padded == true-rank checks
    A_true: Optional[List[np.ndarray]] = None
    B_true: Optional[List[np.ndarray]] = None
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return int(self.x.shape[0])

    @property
    def max_loras(self) -> int:
        return len(self.adapters)


def _pool(rng, ranks, k_in, n_out, max_rank, sigma, dtype):
    """Draw every A (all slots) then every B (all slots) at true rank, pad after."""
    a_true = [rng.standard_normal((r, k_in)) * sigma for r in ranks]
    b_true = [rng.standard_normal((n_out, r)) * sigma for r in ranks]
    P = len(ranks)
    A = np.zeros((P, max_rank, k_in), dtype=np.uint16 if dtype == BF16 else np.float32)
    B = np.zeros((P, n_out, max_rank), dtype=A.dtype)
    At, Bt = [], []
    for p, r in enumerate(ranks):
        a = _store(a_true[p], dtype)
        b = _store(b_true[p], dtype)
        A[p, :r, :] = a
        B[p, :, :r] = b
        At.append(a)
        Bt.append(b)
    return A, B, At, Bt


# ---------------------------------------------------------------- configs
def single_projection_f32(seed: int = 0, k: int = 256, n_out: int = 256, rank: int = 8,
                          n: int = 4, alpha: float = 16.0) -> Workload:
    """fp32 single projection: W [256x256], one rank-8 adapter, 4 rows on slot 0."""
    rng = np.random.default_rng(seed)
    W = _store(rng.standard_normal((n_out, k)) * 0.02, F32)
    A, B, At, Bt = _pool(rng, [rank], k, n_out, rank, 0.02, F32)
    x = _store(rng.standard_normal((n, k)), F32)
    return Workload(name=f"single_projection_f32_{n_out}x{k}_r{rank}_n{n}", dtype=F32,
                    k_in=k, n_out=n_out, max_rank=rank, W=W, A=A, B=B, x=x,
                    adapters=[AdapterSpec(rank, alpha, 1.0)],
                    adapter_slots=np.zeros(n, np.int32), padded_n=n, active=0,
                    A_true=At, B_true=Bt)


def decode_bgmv(seed: int = 0, k: int = 4096, n_out: int = 4096, n_slots: int = 16,
                rank: int = 16, alpha: float = 32.0, n_real: int = 57, padded_n: int = 64,
                dtype: str = BF16) -> Workload:
    """Decode bgmv: q_proj W [4096x4096], 16 slots at rank 16, 57 real rows padded to 64."""
    rng = np.random.default_rng(seed)
    W = _store(rng.standard_normal((n_out, k)) * 0.02, dtype)
    A, B, At, Bt = _pool(rng, [rank] * n_slots, k, n_out, rank, 0.02, dtype)
    # every padded row carries real activations, so the pad rows' byte
    # identity with the base output is a non-trivial check
    x = _store(rng.standard_normal((padded_n, k)), dtype)
    slots = rng.integers(0, n_slots, size=n_real).astype(np.int32)
    return Workload(name=f"decode_bgmv_{n_out}x{k}_s{n_slots}_r{rank}_n{n_real}of{padded_n}",
                    dtype=dtype, k_in=k, n_out=n_out, max_rank=rank, W=W, A=A, B=B, x=x,
                    adapters=[AdapterSpec(rank, alpha, 1.0) for _ in range(n_slots)],
                    adapter_slots=slots, padded_n=padded_n, active=0, A_true=At, B_true=Bt)


GATE_UP_RANKS = (8, 16, 32, 64)


def gate_up_zero_scale_slots(n_slots: int) -> List[int]:
    """The quarter of the pool switched off (adapter_scale 0): k mod 4 == (k div 4) mod 4."""
    return [k for k in range(n_slots) if k % 4 == (k // 4) % 4]


def fused_gate_up(seed: int = 0, k: int = 4096, half: int = 11008, n_slots: int = 32,
                  max_rank: int = 64, n: int = 256, alpha: float = 16.0,
                  ranks=GATE_UP_RANKS) -> Workload:
    """Fused gate/up: W [2*half x k] (gate rows first), mixed ranks padded to 64, rsLoRA."""
    rng = np.random.default_rng(seed)
    n_out = 2 * half
    W = _store(rng.standard_normal((n_out, k)) * 0.02, BF16)
    r_of = [ranks[s % len(ranks)] for s in range(n_slots)]
    A, B, At, Bt = _pool(rng, r_of, k, n_out, max_rank, 0.02, BF16)
    x = _store(rng.standard_normal((n, k)), BF16)
    slots = rng.integers(0, n_slots, size=n).astype(np.int32)
    off = set(gate_up_zero_scale_slots(n_slots))
    adapters = [AdapterSpec(r_of[s], alpha, 0.0 if s in off else 1.0, rslora=True)
                for s in range(n_slots)]
    return Workload(name=f"fused_gate_up_{n_out}x{k}_s{n_slots}_r{max_rank}_n{n}",
                    dtype=BF16, k_in=k, n_out=n_out, max_rank=max_rank, W=W, A=A, B=B,
                    x=x, adapters=adapters, adapter_slots=slots, padded_n=n, active=0,
                    A_true=At, B_true=Bt, meta={"half": half})


def prefill_segmented(seed: int = 0, k: int = 4096, n_out: int = 4096, n_seg: int = 8,
                      seg_len: int = 512, rank: int = 64, seg_lens=None) -> Workload:
    """Prefill: o_proj W [4096x4096]; 8 contiguous 512-token segments, segment g on slot g."""
    rng = np.random.default_rng(seed)
    W = _store(rng.standard_normal((n_out, k)) * 0.02, BF16)
    A, B, At, Bt = _pool(rng, [rank] * n_seg, k, n_out, rank, 0.02, BF16)
    lens = list(seg_lens) if seg_lens is not None else [seg_len] * n_seg
    n = int(sum(lens))
    x = _store(rng.standard_normal((n, k)), BF16)
    indptr = np.zeros(len(lens) + 1, np.int32)
    indptr[1:] = np.cumsum(lens)
    return Workload(name=f"prefill_segmented_{n_out}x{k}_{len(lens)}seg_n{n}_r{rank}",
                    dtype=BF16, k_in=k, n_out=n_out, max_rank=rank, W=W, A=A, B=B, x=x,
                    adapters=[AdapterSpec(rank, 0.0, 1.0) for _ in range(n_seg)],
                    kind="segmented", seg_indptr=indptr,
                    seg_slot=np.arange(len(lens), dtype=np.int32) % n_seg,
                    A_true=At, B_true=Bt)


def moe_down_gather(seed: int = 0, n_experts: int = 64, n_out: int = 2048, k: int = 1408,
                    n_tokens: int = 512, top_k: int = 6, n_adapters: int = 4,
                    rank: int = 16) -> Workload:
    """MoE down_proj gather: 64 experts W_e [2048x1408], top-6, rank-16 pair per (adapter, expert)."""
    rng = np.random.default_rng(seed)
    W = _store(rng.standard_normal((n_experts, n_out, k)) * 0.02, BF16)
    P = n_adapters * n_experts            # pair (a, e) lives at pool index a*E + e
    A, B, At, Bt = _pool(rng, [rank] * P, k, n_out, rank, 0.02, BF16)
    n = n_tokens * top_k
    x = _store(rng.standard_normal((n, k)), BF16)
    idx = np.empty((n_tokens, top_k), np.int32)
    for t in range(n_tokens):
        idx[t] = rng.choice(n_experts, size=top_k, replace=False)
    token_slot = rng.integers(0, n_adapters, size=n_tokens).astype(np.int32)
    return Workload(name=f"moe_down_gather_{n_experts}x{n_out}x{k}_t{n_tokens}_top{top_k}_r{rank}",
                    dtype=BF16, k_in=k, n_out=n_out, max_rank=rank, W=W, A=A, B=B, x=x,
                    adapters=[AdapterSpec(rank, 0.0, 1.0) for _ in range(n_adapters)],
                    kind="moe", n_experts=n_experts, top_k=top_k,
                    indices=idx.reshape(-1), token_slot=token_slot, A_true=At, B_true=Bt)


def group_by_expert(indices: np.ndarray, token_slot: np.ndarray, top_k: int, n_experts: int):
    """Sorts slot-major routing slots by expert (stable).  Returns the order
    (sorted position -> routing slot), expert_offsets [E+1] and each sorted
    row's adapter slot (its token's)."""
    order = np.argsort(indices, kind="stable").astype(np.int32)
    counts = np.bincount(indices, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return order, offsets, token_slot[order // top_k].astype(np.int32)


def moe_down_grouped(seed: int = 0, n_experts: int = 64, n_out: int = 2048, k: int = 1408,
                     n_tokens: int = 2048, top_k: int = 6, n_adapters: int = 4,
                     rank: int = 16) -> Workload:
    """MoE down_proj, grouped: the gather workload's expert and pool shapes with
    a prefill-sized batch (2048 tokens, top-6) whose routing slots come
    sorted by expert, delimited by expert_offsets."""
    rng = np.random.default_rng(seed)
    W = _store(rng.standard_normal((n_experts, n_out, k)) * 0.02, BF16)
    P = n_adapters * n_experts
    A, B, At, Bt = _pool(rng, [rank] * P, k, n_out, rank, 0.02, BF16)
    n = n_tokens * top_k
    x = _store(rng.standard_normal((n, k)), BF16)  # already in sorted order
    idx = np.empty((n_tokens, top_k), np.int32)
    for t in range(n_tokens):
        idx[t] = rng.choice(n_experts, size=top_k, replace=False)
    token_slot = rng.integers(0, n_adapters, size=n_tokens).astype(np.int32)
    order, offsets, row_slot = group_by_expert(idx.reshape(-1), token_slot, top_k, n_experts)
    return Workload(name=f"moe_down_grouped_{n_experts}x{n_out}x{k}_t{n_tokens}_top{top_k}_r{rank}",
                    dtype=BF16, k_in=k, n_out=n_out, max_rank=rank, W=W, A=A, B=B, x=x,
                    adapters=[AdapterSpec(rank, 0.0, 1.0) for _ in range(n_adapters)],
                    kind="moe_grouped", n_experts=n_experts, top_k=top_k,
                    expert_offsets=offsets, row_slot=row_slot, A_true=At, B_true=Bt,
                    meta={"order": order})


# the five workloads, full size, seed 0
CONFIGS = {
    "single_projection_f32": single_projection_f32,
    "decode_bgmv": decode_bgmv,
    "fused_gate_up": fused_gate_up,
    "prefill_segmented": prefill_segmented,
    "moe_down_gather": moe_down_gather,
}


def spec_verify_kv(seed: int = 0, n_seqs: int = 4, draft: int = 9, k: int = 4096,
                   kv_dim: int = 1024, q_dim: int = 4096, n_slots: int = 16, rank: int = 16,
                   alpha: float = 32.0, dtype: str = BF16) -> Workload:
    """Speculative verify on the K projection: n_seqs sequences x `draft` tokens
    = 36 rows, each sequence's rows on its sequence's adapter; W_k [1024 x 4096]
    writing into the K columns of an interleaved [Q|K|V] row (q_dim + 2 kv_dim
    elements)."""
    rng = np.random.default_rng(seed)
    W = _store(rng.standard_normal((kv_dim, k)) * 0.02, dtype)
    A, B, At, Bt = _pool(rng, [rank] * n_slots, k, kv_dim, rank, 0.02, dtype)
    n = n_seqs * draft
    x = _store(rng.standard_normal((n, k)), dtype)
    seq_slots = rng.integers(0, n_slots, size=n_seqs).astype(np.int32)
    slots = np.repeat(seq_slots, draft).astype(np.int32)
    return Workload(name=f"spec_verify_kv_{kv_dim}x{k}_s{n_slots}_r{rank}_{n_seqs}x{draft}",
                    dtype=dtype, k_in=k, n_out=kv_dim, max_rank=rank, W=W, A=A, B=B, x=x,
                    adapters=[AdapterSpec(rank, alpha, 1.0) for _ in range(n_slots)],
                    adapter_slots=slots, padded_n=n, active=0, A_true=At, B_true=Bt,
                    meta={"q_dim": q_dim, "kv_dim": kv_dim, "qkv_row": q_dim + 2 * kv_dim,
                          "n_seqs": n_seqs, "draft": draft, "seq_slots": seq_slots})


def adapter_stack(seed: int = 0, k: int = 4096, n_out: int = 4096, n_levels: int = 3,
                  n_slots: int = 8, rank: int = 16, alpha: float = 32.0, n: int = 64,
                  dtype: str = BF16) -> Workload:
    """Adapter stack on q_proj (W [4096 x 4096]): three levels, each a pool of 8
    rank-16 adapters (alpha 32) with its own per-row slot; 64 rows, every level
    drawing its rows' slots uniformly from [-1, 8) (-1: the level adds nothing)."""
    rng = np.random.default_rng(seed)
    W = _store(rng.standard_normal((n_out, k)) * 0.02, dtype)
    levels = []
    for _ in range(n_levels):
        A, B, At, Bt = _pool(rng, [rank] * n_slots, k, n_out, rank, 0.02, dtype)
        levels.append({"A": A, "B": B, "adapters": [AdapterSpec(rank, alpha, 1.0)] * n_slots})
    x = _store(rng.standard_normal((n, k)), dtype)
    for lv in levels:
        lv["seq_slot"] = rng.integers(-1, n_slots, size=n).astype(np.int32)
    l0 = levels[0]
    return Workload(name=f"adapter_stack_{n_out}x{k}_{n_levels}lv_s{n_slots}_r{rank}_n{n}",
                    dtype=dtype, k_in=k, n_out=n_out, max_rank=rank, W=W, A=l0["A"], B=l0["B"],
                    x=x, adapters=l0["adapters"], kind="stack", adapter_slots=l0["seq_slot"],
                    padded_n=n, active=0, meta={"levels": levels, "seq_slot": l0["seq_slot"]})


def random_stack(seed: int, dtype: str = BF16, k: int = 96, n_out: int = 80, n: int = 13,
                 n_levels: int = 2, n_slots: int = 3, max_rank: int = 16) -> Workload:
    """Small stack with ragged sizes, mixed ranks and -1 / out-of-range slots per level."""
    rng = np.random.default_rng(seed)
    W = _store(rng.standard_normal((n_out, k)) * 0.05, dtype)
    levels = []
    for _ in range(n_levels):
        ranks = [int(rng.integers(1, max_rank + 1)) for _ in range(n_slots)]
        A, B, At, Bt = _pool(rng, ranks, k, n_out, max_rank, 0.1, dtype)
        ad = [AdapterSpec(ranks[s], float(rng.choice([0.0, 8.0])), float(rng.choice([0.5, 1.0])),
                          bool(rng.integers(0, 2))) for s in range(n_slots)]
        levels.append({"A": A, "B": B, "adapters": ad})
    x = _store(rng.standard_normal((n, k)), dtype)
    for lv in levels:
        lv["seq_slot"] = rng.integers(-1, n_slots + 1, size=n).astype(np.int32)
    l0 = levels[0]
    return Workload(name=f"small_stack_s{seed}", dtype=dtype, k_in=k, n_out=n_out,
                    max_rank=max_rank, W=W, A=l0["A"], B=l0["B"], x=x, adapters=l0["adapters"],
                    kind="stack", adapter_slots=l0["seq_slot"], padded_n=n, active=0,
                    meta={"levels": levels, "seq_slot": l0["seq_slot"]})


def token_embedding(seed: int = 0, n_vocab: int = 32000, n_embd: int = 4096, n: int = 4096,
                    n_slots: int = 8, rank: int = 16, alpha: float = 32.0,
                    dtype: str = BF16, max_rank: Optional[int] = None, ranks=None) -> Workload:
    """Token-embedding gather: E [32000 x 4096] bf16, 8 adapters at rank 16
    (alpha 32) stored the way an adapter file stores an embedding pair --
    A_file [n_vocab][rank], B_file [n_embd][rank] (ferrox lora.rs module doc:
    flipped upstream) -- 4096 tokens uniform over the vocabulary, each row's
    slot uniform in [-1, 8).  W holds E; A and B hold the file layout (the
    consumers bring it into the one layout themselves)."""
    rng = np.random.default_rng(seed)
    R = rank if max_rank is None else max_rank
    rk = [rank] * n_slots if ranks is None else list(ranks)
    E = _store(rng.standard_normal((n_vocab, n_embd)) * 0.02, dtype)
    a_file = np.zeros((n_slots, n_vocab, R), np.uint16 if dtype == BF16 else np.float32)
    b_file = np.zeros((n_slots, n_embd, R), a_file.dtype)
    for p in range(n_slots):  # every A_file, then every B_file, at true rank; pads after
        a_file[p, :, :rk[p]] = _store(rng.standard_normal((n_vocab, rk[p])) * 0.02, dtype)
    for p in range(n_slots):
        b_file[p, :, :rk[p]] = _store(rng.standard_normal((n_embd, rk[p])) * 0.02, dtype)
    tokens = rng.integers(0, n_vocab, size=n).astype(np.int32)
    slots = rng.integers(-1, n_slots, size=n).astype(np.int32)
    return Workload(name=f"token_embedding_{n_vocab}x{n_embd}_s{n_slots}_r{rank}_n{n}",
                    dtype=dtype, k_in=n_embd, n_out=n_vocab, max_rank=R, W=E, A=a_file,
                    B=b_file, x=np.zeros((n, 0), E.dtype),
                    adapters=[AdapterSpec(rk[p], alpha, 1.0) for p in range(n_slots)],
                    kind="embed", adapter_slots=slots, padded_n=n, active=0,
                    meta={"token_ids": tokens, "seq_slot": slots, "a_file": a_file,
                          "b_file": b_file})


# workloads of the variants built beyond the five: the grouped MoE layout,
# the speculative-verify K fold, the adapter stack and the token embedding
NEXT_WORKLOADS = {
    "moe_down_grouped": moe_down_grouped,
    "spec_verify_kv": spec_verify_kv,
    "adapter_stack": adapter_stack,
    "token_embedding": token_embedding,
}


def random_small(seed: int, dtype: str = BF16, k: int = 96, n_out: int = 80, n: int = 13,
                 n_slots: int = 5, max_rank: int = 16, ranks=None, kind: str = "decode",
                 n_experts: int = 3, top_k: int = 2, seg_lens=None,
                 sigma_w: float = 0.05, sigma_ab: float = 0.1) -> Workload:
    """Small random case with ragged sizes, mixed ranks, -1 / out-of-range slots.

    Used by parity tests at sizes the oracle finishes instantly.
    """
    rng = np.random.default_rng(seed)
    if ranks is None:
        ranks = [int(rng.integers(1, max_rank + 1)) for _ in range(n_slots)]
    if kind in ("moe", "moe_grouped"):
        W = _store(rng.standard_normal((n_experts, n_out, k)) * sigma_w, dtype)
        P = n_slots * n_experts
        rk = [ranks[p // n_experts] for p in range(P)]
    else:
        W = _store(rng.standard_normal((n_out, k)) * sigma_w, dtype)
        rk = list(ranks)
    A, B, At, Bt = _pool(rng, rk, k, n_out, max_rank, sigma_ab, dtype)
    adapters = [AdapterSpec(int(ranks[s]), float(rng.choice([0.0, 8.0, 16.0])),
                            float(rng.choice([0.5, 1.0, 2.0])), bool(rng.integers(0, 2)))
                for s in range(n_slots)]
    common = dict(dtype=dtype, k_in=k, n_out=n_out, max_rank=max_rank, W=W, A=A, B=B,
                  adapters=adapters, A_true=At, B_true=Bt)
    if kind == "decode":
        x = _store(rng.standard_normal((n, k)), dtype)
        n_real = max(1, n - 2)
        # real rows: valid slots, -1 ("use the active adapter"), and one past the pool
        slots = rng.integers(-1, n_slots + 1, size=n_real).astype(np.int32)
        return Workload(name=f"small_decode_s{seed}", x=x, adapter_slots=slots, padded_n=n,
                        active=int(rng.integers(0, n_slots)), **common)
    if kind == "segmented":
        lens = list(seg_lens) if seg_lens is not None else \
            [int(v) for v in rng.integers(0, 40, size=n_slots + 1)]
        nn = int(sum(lens))
        x = _store(rng.standard_normal((nn, k)), dtype)
        indptr = np.zeros(len(lens) + 1, np.int32)
        indptr[1:] = np.cumsum(lens)
        seg_slot = rng.integers(-1, n_slots + 1, size=len(lens)).astype(np.int32)
        return Workload(name=f"small_segmented_s{seed}", x=x, kind="segmented",
                        seg_indptr=indptr, seg_slot=seg_slot, **common)
    if kind == "moe":
        n_tokens = n
        nn = n_tokens * top_k
        x = _store(rng.standard_normal((nn, k)), dtype)
        idx = np.empty((n_tokens, top_k), np.int32)
        for t in range(n_tokens):
            idx[t] = rng.choice(n_experts, size=top_k, replace=False)
        token_slot = rng.integers(-1, n_slots + 1, size=n_tokens).astype(np.int32)
        common["adapters"] = adapters
        return Workload(name=f"small_moe_s{seed}", x=x, kind="moe", n_experts=n_experts,
                        top_k=top_k, indices=idx.reshape(-1), token_slot=token_slot, **common)
    if kind == "moe_grouped":
        # n rows inside the expert ranges (some experts empty), a few rows
        # before the first range and after the last, which are not written
        counts = rng.multinomial(n, np.full(n_experts, 1.0 / n_experts))
        lead, tail = (int(v) for v in rng.integers(0, 3, size=2))
        offsets = np.zeros(n_experts + 1, np.int32)
        offsets[1:] = np.cumsum(counts)
        offsets += lead
        nn = lead + n + tail
        x = _store(rng.standard_normal((nn, k)), dtype)
        row_slot = rng.integers(-1, n_slots + 1, size=nn).astype(np.int32)
        return Workload(name=f"small_moe_grouped_s{seed}", x=x, kind="moe_grouped",
                        n_experts=n_experts, expert_offsets=offsets, row_slot=row_slot, **common)
    raise ValueError(kind)
