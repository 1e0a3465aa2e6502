"""Brute force for tiny shapes, written from the pages independently of the oracle.

The delta is materialised as the dense matrix s * B A and added to W before a
single matrix-vector product -- the association ferrox-core's tests use as
their reference (weight_matrix/lora.rs, test helper dense_delta) -- instead of
the oracle's shrink-then-expand order.  Route resolution follows atlas
lora_delta.rs apply_lora_bgmv doc (slot < 0 is base; NULL / zero-scale slots
are base-only) plus the reading that a slot past the pool is skipped.
"""
import numpy as np

from adapter_lora_bgmv_amd.workloads import bf16_bits_to_f32


def widen(a, dtype):
    a = np.asarray(a)
    if dtype == "bf16" or a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def resolved(slot, n_slots, null_slots, scale_table):
    return (0 <= slot < n_slots) and (slot not in null_slots) and scale_table[slot] != 0.0


def dense_rows(W, A, B, x, dtype, seq_slot, scale_table, null_slots=(), n_experts=1,
               experts=None):
    """y[i] = (W_i + s B_s A_s) x_i with the materialised delta, row by row."""
    Wd = widen(W, dtype)
    Ad = widen(A, dtype)
    Bd = widen(B, dtype)
    xd = widen(x, dtype)
    out = []
    for i in range(xd.shape[0]):
        s = int(seq_slot[i])
        Wi = Wd if experts is None else Wd[int(experts[i])]
        M = Wi.copy()
        if resolved(s, len(scale_table), set(null_slots), scale_table):
            p = s * n_experts + (0 if experts is None else int(experts[i]))
            if p not in set(null_slots):
                M = M + float(scale_table[s]) * (Bd[p] @ Ad[p])
        out.append(M @ xd[i])
    return np.array(out)
