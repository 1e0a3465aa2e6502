"""Device-side set-up of a ``workloads.Workload`` and one call of the path on it.

Shared by the GPU tests, ``__graft_entry__.smoke()`` and ``bench.py``.  It
uploads the host arrays (bf16 as raw bit patterns), builds the seq_slot
buffer and the scale table with the library's host helpers, builds the
device routing tables, sizes and zero-fills the workspace, and calls the
entry point that fits the workload's kind.  All arithmetic happens in the
HIP library.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import binding as B
from .workloads import Workload


def to_device(a: np.ndarray, device="cuda"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def bf16_bits(t) -> np.ndarray:
    """Raw bit patterns of a device bf16 tensor (uint16) or values of an f32 one."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DeviceWorkload:
    """A workload resident on the GPU, ready to run through the library."""

    def __init__(self, wl: Workload, device="cuda", scale_table=None,
                 null_slots: Optional[Sequence[int]] = None, x_extra_cols: int = 0,
                 y_extra_cols: int = 0, y_col_offset: int = 0):
        import torch
        self.wl = wl
        self.device = device
        self.dtype = B.LORA_BF16 if wl.dtype == "bf16" else B.LORA_F32
        self.W = to_device(wl.W, device)
        if wl.kind == "embed":
            # the file-layout embedding pairs into the one layout, through the
            # library's host helper: A = B_file transposed, B = A_file
            self.A = to_device(np.stack([B.lora_embedding_pair(a, b, wl.n_out, wl.k_in)
                                         for a, b in zip(wl.meta["a_file"], wl.meta["b_file"])]),
                               device)
            self.Bp = to_device(wl.meta["a_file"], device)
        else:
            self.A = to_device(wl.A, device)
            self.Bp = to_device(wl.B, device)
        # a gathered embedding row is n_embd (k_in) wide; a projection's is n_out
        self.out_w = wl.k_in if wl.kind == "embed" else wl.n_out
        n, k = wl.x.shape
        xs = k + x_extra_cols
        xh = np.zeros((n, xs), wl.x.dtype)
        xh[:, :k] = wl.x
        self.x = to_device(xh, device)
        self.x_row_stride = xs
        # y's rows may be wider than n_out, with the projection's columns at
        # y_col_offset inside them (an interleaved [Q|K|V] row, say)
        self.y_row_stride = y_col_offset + self.out_w + y_extra_cols
        self.y_col_offset = y_col_offset
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.y_full = torch.empty((n, self.y_row_stride), dtype=tdt, device=device)
        self.y = self.y_full[:, y_col_offset:]
        self.scale_table_host = (B.lora_scale_table(wl.adapters) if scale_table is None
                                 else np.asarray(scale_table, np.float32))
        ns = wl.null_slots if null_slots is None else null_slots
        self.route = None
        if wl.kind == "embed":
            self.route = B.DeviceRoute(self.A, self.Bp, self.scale_table_host, null_slots=ns)
            self.token_ids = to_device(wl.meta["token_ids"].astype(np.int32), device)
            self.seq_slot_host = np.asarray(wl.meta["seq_slot"], np.int32)
            self.seq_slot = to_device(self.seq_slot_host, device)
            op, groups = None, 1
        elif wl.kind == "moe":
            self.route = B.DeviceRoute(self.A, self.Bp, self.scale_table_host, null_slots=ns,
                                       n_experts=wl.n_experts)
            self.indices = to_device(wl.indices.astype(np.int32), device)
            self.token_slot = to_device(wl.token_slot.astype(np.int32), device)
            op, groups = B.LORA_OP_MOE_GATHER, wl.n_experts
        elif wl.kind == "stack":
            # one route and one per-row slot buffer per level, in order
            self.levels = []
            for lv in wl.meta["levels"]:
                A, Bp = to_device(lv["A"], device), to_device(lv["B"], device)
                st = B.lora_scale_table(lv["adapters"])
                self.levels.append({"A": A, "B": Bp, "scale_table_host": st,
                                    "route": B.DeviceRoute(A, Bp, st),
                                    "seq_slot": to_device(lv["seq_slot"].astype(np.int32), device)})
            self.route = self.levels[0]["route"] if self.levels else None
            self.scale_table_host = [lv["scale_table_host"] for lv in self.levels]
            op, groups = B.LORA_OP_STACK, max(1, len(self.levels))
        elif wl.kind == "moe_grouped":
            self.route = B.DeviceRoute(self.A, self.Bp, self.scale_table_host, null_slots=ns,
                                       n_experts=wl.n_experts)
            self.expert_offsets = to_device(wl.expert_offsets.astype(np.int32), device)
            self.seq_slot_host = np.asarray(wl.row_slot, np.int32)
            self.seq_slot = to_device(self.seq_slot_host, device)
            op, groups = B.LORA_OP_MOE_GROUPED, wl.n_experts
        else:
            self.route = B.DeviceRoute(self.A, self.Bp, self.scale_table_host, null_slots=ns)
            groups = 1
            if wl.kind == "segmented":
                self.seg_indptr = to_device(wl.seg_indptr.astype(np.int32), device)
                self.seg_slot = to_device(wl.seg_slot.astype(np.int32), device)
                op = B.LORA_OP_SEGMENTED
            else:
                ss = wl.meta.get("seq_slot")
                if ss is None:
                    ss = B.lora_build_seq_slot(wl.adapter_slots, wl.padded_n, wl.active)
                self.seq_slot_host = np.asarray(ss, np.int32)
                self.seq_slot = to_device(self.seq_slot_host, device)
                op = B.LORA_OP_APPLY
        self.op = op
        self.ws_bytes = 0 if op is None else B.lora_workspace_bytes(
            op, self.dtype, n, wl.n_out, wl.k_in, wl.max_rank, groups)
        self.workspace = torch.zeros(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)

    @property
    def n(self) -> int:
        return self.wl.n_rows

    def run(self, route: bool = True, y=None, stream=None):
        """One call of the fused entry point; returns y (device tensor)."""
        wl = self.wl
        y = self.y if y is None else y
        r = self.route if route else None
        if wl.kind == "decode":
            B.lora_apply(self.dtype, wl.n_out, wl.k_in, self.W, wl.k_in, r, self.x,
                         self.x_row_stride, self.seq_slot if route else None, self.n, y,
                         self.y_row_stride, self.workspace, self.ws_bytes, stream)
        elif wl.kind == "segmented":
            B.lora_apply_segmented(self.dtype, wl.n_out, wl.k_in, self.W, wl.k_in, r, self.x,
                                   self.x_row_stride, self.seg_indptr, self.seg_slot,
                                   len(wl.seg_slot), self.n, y, self.y_row_stride,
                                   self.workspace, self.ws_bytes, stream)
        elif wl.kind == "embed":
            B.lora_embed_rows(self.dtype, wl.n_out, wl.k_in, self.W, wl.k_in, r, self.token_ids,
                              self.seq_slot if route else None, self.n, y, self.y_row_stride,
                              stream)
        elif wl.kind == "stack":
            lv = self.levels if route else []
            B.lora_apply_stack(self.dtype, wl.n_out, wl.k_in, self.W, wl.k_in,
                               [v["route"] for v in lv], self.x, self.x_row_stride,
                               [v["seq_slot"] for v in lv], self.n, y, self.y_row_stride,
                               self.workspace, self.ws_bytes, stream)
        elif wl.kind == "moe_grouped":
            B.lora_apply_moe_grouped(self.dtype, wl.n_experts, wl.n_out, wl.k_in, self.W,
                                     wl.n_out * wl.k_in, wl.k_in, r, self.x, self.x_row_stride,
                                     self.expert_offsets, self.seq_slot if route else None,
                                     self.n, y, self.y_row_stride, self.workspace, self.ws_bytes,
                                     stream)
        else:
            B.lora_apply_moe_gather(self.dtype, wl.n_experts, wl.n_out, wl.k_in, self.W,
                                    wl.n_out * wl.k_in, wl.k_in, r, self.x, self.x_row_stride,
                                    self.indices, wl.top_k, self.token_slot if route else None,
                                    len(wl.token_slot), y, self.y_row_stride, self.workspace,
                                    self.ws_bytes, stream)
        return y

    def y_host(self, y=None) -> np.ndarray:
        """y as f64 numpy, trimmed to the output's columns."""
        y = self.y if y is None else y
        h = bf16_bits(y)[:, :self.out_w]
        if h.dtype == np.uint16:
            return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return h.astype(np.float64)

    def y_bits(self, y=None) -> np.ndarray:
        y = self.y if y is None else y
        return bf16_bits(y)[:, :self.out_w].copy()
