"""ctypes binding of the HIP library (include/lora_mi355x.h), over torch tensors.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``_lib/liblora_mi355x.so``.  There is no fallback of any kind --
loading fails loudly when the library has not been built, and every call
raises ``LoraError`` (with the library's message) on a non-zero status.
PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path
from typing import Optional, Sequence

import numpy as np

LIB_PATH = Path(__file__).resolve().parent / "_lib" / "liblora_mi355x.so"

LORA_F32, LORA_BF16 = 0, 1
LORA_OP_APPLY, LORA_OP_SEGMENTED, LORA_OP_MOE_GATHER, LORA_OP_MOE_GROUPED, LORA_OP_STACK = 0, 1, 2, 3, 4
LORA_NOALLOC_SCRATCH_BYTES = 32 << 20  # lora_apply_noalloc's device array, per GPU
STATUS = {0: "LORA_OK", -1: "LORA_ERR_SHAPE", -2: "LORA_ERR_NULL_PTR", -3: "LORA_ERR_STRIDE",
          -4: "LORA_ERR_DTYPE", -5: "LORA_ERR_UNSUPPORTED", -6: "LORA_ERR_LAUNCH",
          -7: "LORA_ERR_WORKSPACE"}

# every symbol include/lora_mi355x.h declares
EXPORTS = ("lora_last_error", "lora_version", "lora_init", "lora_scale", "lora_scale_table",
           "lora_build_seq_slot", "lora_workspace_bytes", "lora_shrink", "lora_expand_fold",
           "lora_apply", "lora_apply_noalloc", "lora_apply_segmented", "lora_apply_moe_gather",
           "lora_set_profile_events", "lora_moe_grouped_shrink", "lora_moe_grouped_expand_fold",
           "lora_apply_moe_grouped", "lora_apply_stack", "lora_embedding_pair",
           "lora_embed_rows")


class LoraError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class lora_route(C.Structure):
    _fields_ = [("a_table", C.c_void_p), ("b_table", C.c_void_p), ("scale_table", C.c_void_p),
                ("max_loras", C.c_uint32), ("k_in", C.c_uint32), ("n_out", C.c_uint32),
                ("max_rank", C.c_uint32), ("dtype", C.c_int32)]


class lora_route_moe(C.Structure):
    _fields_ = [("a_table", C.c_void_p), ("b_table", C.c_void_p), ("scale_table", C.c_void_p),
                ("max_loras", C.c_uint32), ("n_experts", C.c_uint32), ("k_in", C.c_uint32),
                ("n_out", C.c_uint32), ("max_rank", C.c_uint32), ("dtype", C.c_int32)]


_lib = None


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"HIP library missing: {LIB_PATH} (run __graft_entry__.build())")
    # torch first: its HIP runtime (same soname) is then the one the library binds
    # to, so torch's streams and device pointers are valid in the library's calls
    import torch  # noqa: F401
    L = C.CDLL(str(LIB_PATH))
    u32, i32, vp, sz = C.c_uint32, C.c_int32, C.c_void_p, C.c_size_t
    L.lora_last_error.restype = C.c_char_p
    L.lora_version.restype = C.c_char_p
    L.lora_scale.restype = C.c_double
    L.lora_scale.argtypes = [C.c_double, C.c_double, u32, i32]
    L.lora_scale_table.argtypes = [u32, vp, vp, vp, vp, u32, vp]
    L.lora_build_seq_slot.argtypes = [vp, u32, u32, i32, vp]
    L.lora_set_profile_events.argtypes = [vp, u32]
    L.lora_workspace_bytes.restype = sz
    L.lora_workspace_bytes.argtypes = [i32, i32, u32, u32, u32, u32, u32]
    RP = C.POINTER(lora_route)
    L.lora_shrink.argtypes = [RP, vp, u32, vp, u32, vp, vp]
    L.lora_expand_fold.argtypes = [RP, vp, vp, u32, vp, u32, vp]
    L.lora_apply.argtypes = [i32, u32, u32, vp, u32, RP, vp, u32, vp, u32, vp, u32, vp, sz, vp]
    L.lora_apply_noalloc.argtypes = [i32, u32, u32, vp, u32, RP, vp, u32, vp, u32, vp, u32, vp]
    L.lora_apply_segmented.argtypes = [i32, u32, u32, vp, u32, RP, vp, u32, vp, vp, u32, u32, vp,
                                       u32, vp, sz, vp]
    L.lora_apply_moe_gather.argtypes = [i32, u32, u32, u32, vp, C.c_uint64, u32,
                                        C.POINTER(lora_route_moe), vp, u32, vp, u32, vp, u32, vp,
                                        u32, vp, sz, vp]
    RM = C.POINTER(lora_route_moe)
    L.lora_moe_grouped_shrink.argtypes = [RM, vp, u32, vp, vp, u32, vp, vp]
    L.lora_moe_grouped_expand_fold.argtypes = [RM, vp, vp, vp, u32, vp, u32, vp]
    L.lora_apply_moe_grouped.argtypes = [i32, u32, u32, u32, vp, C.c_uint64, u32, RM, vp, u32, vp,
                                         vp, u32, vp, u32, vp, sz, vp]
    L.lora_apply_stack.argtypes = [i32, u32, u32, vp, u32, C.POINTER(lora_route), C.POINTER(vp),
                                   u32, vp, u32, u32, vp, u32, vp, sz, vp]
    L.lora_embedding_pair.argtypes = [i32, u32, u32, u32, u32, vp, u32, u32, vp, vp]
    L.lora_embed_rows.argtypes = [i32, u32, u32, vp, u32, C.POINTER(lora_route), vp, vp, u32, vp,
                                  u32, vp]
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise LoraError(rc, lib().lora_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return LORA_F32
    if t.dtype == torch.bfloat16:
        return LORA_BF16
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


# ---------------------------------------------------------------- host helpers
def lora_version() -> str:
    return lib().lora_version().decode()


def lora_init():
    _check(lib().lora_init())


def lora_scale(adapter_scale: float, alpha: float, rank: int, rslora: bool) -> float:
    return float(lib().lora_scale(adapter_scale, alpha, int(rank), int(bool(rslora))))


def lora_scale_table(adapters, max_loras: Optional[int] = None) -> np.ndarray:
    """[max_loras] f32 host table from AdapterSpec-like objects."""
    n = len(adapters)
    m = n if max_loras is None else int(max_loras)
    s = np.array([a.adapter_scale for a in adapters] or [0.0], np.float64)
    al = np.array([a.alpha for a in adapters] or [0.0], np.float64)
    r = np.array([a.rank for a in adapters] or [1], np.uint32)
    rs = np.array([int(a.rslora) for a in adapters] or [0], np.int32)
    out = np.empty(max(m, 1), np.float32)
    _check(lib().lora_scale_table(n, s.ctypes.data, al.ctypes.data, r.ctypes.data, rs.ctypes.data,
                                  m, out.ctypes.data))
    return out[:m]


def lora_build_seq_slot(adapter_slots, padded_n: int, active: int) -> np.ndarray:
    a = np.ascontiguousarray(adapter_slots, np.int32)
    out = np.empty(max(int(padded_n), 1), np.int32)
    _check(lib().lora_build_seq_slot(a.ctypes.data if len(a) else None, len(a), int(padded_n),
                                     int(active), out.ctypes.data))
    return out[:padded_n]


def lora_set_profile_events(events: Optional[Sequence[int]]):
    """Raw hipEvent_t handles (ints) the fused calls record around their kernels, or None."""
    if not events:
        _check(lib().lora_set_profile_events(None, 0))
        return
    arr = (C.c_void_p * len(events))(*events)
    _check(lib().lora_set_profile_events(arr, len(events)))


def lora_workspace_bytes(op: int, dtype: int, n_rows: int, n_out: int, k_in: int, max_rank: int,
                         n_groups: int = 1) -> int:
    return int(lib().lora_workspace_bytes(op, dtype, n_rows, n_out, k_in, max_rank, n_groups))


# ---------------------------------------------------------------- routes
class DeviceRoute:
    """Device-side routing tables over a pool of A/B tensors (atlas LoraRoute).

    ``A`` is ``[P][max_rank][k_in]``, ``B`` is ``[P][n_out_pool][max_rank]`` on
    the device; ``null_slots`` get NULL entries.  ``b_row_offset``/``n_out``
    select a block of B's rows (a fused projection's part).  For the MoE
    gather pass ``n_experts``; pair (a, e) is pool entry a * n_experts + e.
    """

    def __init__(self, A, B, scale_table, *, n_out=None, b_row_offset=0,
                 null_slots: Sequence[int] = (), n_experts: int = 0):
        import torch
        self.A, self.B = A, B
        P, R, k_in = A.shape
        n_out = B.shape[1] if n_out is None else int(n_out)
        esz = A.element_size()
        null = set(int(v) for v in null_slots)
        a_ptrs = [0 if p in null else A.data_ptr() + p * A.stride(0) * esz for p in range(P)]
        b_ptrs = [0 if p in null else B.data_ptr() + (p * B.stride(0) + b_row_offset * R) * esz
                  for p in range(P)]
        dev = A.device
        self.a_table = torch.tensor(a_ptrs, dtype=torch.int64, device=dev)
        self.b_table = torch.tensor(b_ptrs, dtype=torch.int64, device=dev)
        st = torch.as_tensor(np.ascontiguousarray(scale_table, np.float32))
        self.scale_table = st.to(dev)
        self.dtype = _dtype_code(A)
        self.k_in, self.n_out, self.max_rank = int(k_in), int(n_out), int(R)
        self.n_experts = int(n_experts)
        self.max_loras = int(self.scale_table.numel())
        if n_experts:
            self.c = lora_route_moe(self.a_table.data_ptr(), self.b_table.data_ptr(),
                                    self.scale_table.data_ptr(), self.max_loras, self.n_experts,
                                    self.k_in, self.n_out, self.max_rank, self.dtype)
        else:
            self.c = lora_route(self.a_table.data_ptr(), self.b_table.data_ptr(),
                                self.scale_table.data_ptr(), self.max_loras, self.k_in,
                                self.n_out, self.max_rank, self.dtype)

    def set_scale_table(self, values):
        import torch
        self.scale_table.copy_(torch.as_tensor(np.ascontiguousarray(values, np.float32)))


def _route_ref(route):
    return None if route is None else C.byref(route.c)


# ---------------------------------------------------------------- kernels
def lora_shrink(route: DeviceRoute, x, x_row_stride: int, seq_slot, n: int, t, stream=None):
    _check(lib().lora_shrink(C.byref(route.c), _ptr(x), x_row_stride, _ptr(seq_slot), n, _ptr(t),
                             _stream(stream)))


def lora_expand_fold(route: DeviceRoute, t, seq_slot, n: int, y, y_row_stride: int, stream=None):
    _check(lib().lora_expand_fold(C.byref(route.c), _ptr(t), _ptr(seq_slot), n, _ptr(y),
                                  y_row_stride, _stream(stream)))


def lora_apply(dtype: int, n_out: int, k_in: int, W, w_row_stride: int, route, x, x_row_stride: int,
               seq_slot, n: int, y, y_row_stride: int, workspace, workspace_bytes: int,
               stream=None):
    _check(lib().lora_apply(dtype, n_out, k_in, _ptr(W), w_row_stride, _route_ref(route), _ptr(x),
                            x_row_stride, _ptr(seq_slot), n, _ptr(y), y_row_stride,
                            _ptr(workspace), workspace_bytes, _stream(stream)))


def lora_apply_noalloc(dtype: int, n_out: int, k_in: int, W, w_row_stride: int, route, x,
                       x_row_stride: int, seq_slot, n: int, y, y_row_stride: int, stream=None):
    _check(lib().lora_apply_noalloc(dtype, n_out, k_in, _ptr(W), w_row_stride, _route_ref(route),
                                    _ptr(x), x_row_stride, _ptr(seq_slot), n, _ptr(y), y_row_stride,
                                    _stream(stream)))


def lora_apply_segmented(dtype: int, n_out: int, k_in: int, W, w_row_stride: int, route, x,
                         x_row_stride: int, seg_indptr, seg_slot, n_seg: int, n: int, y,
                         y_row_stride: int, workspace, workspace_bytes: int, stream=None):
    _check(lib().lora_apply_segmented(dtype, n_out, k_in, _ptr(W), w_row_stride, _route_ref(route),
                                      _ptr(x), x_row_stride, _ptr(seg_indptr), _ptr(seg_slot),
                                      n_seg, n, _ptr(y), y_row_stride, _ptr(workspace),
                                      workspace_bytes, _stream(stream)))


def lora_apply_moe_gather(dtype: int, n_experts: int, n_out: int, k_in: int, W_experts,
                          expert_stride: int, w_row_stride: int, route, x, x_row_stride: int,
                          indices, top_k: int, token_slot, n_tokens: int, y, y_row_stride: int,
                          workspace, workspace_bytes: int, stream=None):
    _check(lib().lora_apply_moe_gather(dtype, n_experts, n_out, k_in, _ptr(W_experts),
                                       expert_stride, w_row_stride, _route_ref(route), _ptr(x),
                                       x_row_stride, _ptr(indices), top_k, _ptr(token_slot),
                                       n_tokens, _ptr(y), y_row_stride, _ptr(workspace),
                                       workspace_bytes, _stream(stream)))


def lora_moe_grouped_shrink(route: DeviceRoute, x, x_row_stride: int, expert_offsets, seq_slot,
                            n: int, t, stream=None):
    _check(lib().lora_moe_grouped_shrink(C.byref(route.c), _ptr(x), x_row_stride,
                                         _ptr(expert_offsets), _ptr(seq_slot), n, _ptr(t),
                                         _stream(stream)))


def lora_moe_grouped_expand_fold(route: DeviceRoute, t, expert_offsets, seq_slot, n: int, y,
                                 y_row_stride: int, stream=None):
    _check(lib().lora_moe_grouped_expand_fold(C.byref(route.c), _ptr(t), _ptr(expert_offsets),
                                              _ptr(seq_slot), n, _ptr(y), y_row_stride,
                                              _stream(stream)))


def lora_apply_moe_grouped(dtype: int, n_experts: int, n_out: int, k_in: int, W_experts,
                           expert_stride: int, w_row_stride: int, route, x, x_row_stride: int,
                           expert_offsets, seq_slot, n: int, y, y_row_stride: int, workspace,
                           workspace_bytes: int, stream=None):
    _check(lib().lora_apply_moe_grouped(dtype, n_experts, n_out, k_in, _ptr(W_experts),
                                        expert_stride, w_row_stride, _route_ref(route), _ptr(x),
                                        x_row_stride, _ptr(expert_offsets), _ptr(seq_slot), n,
                                        _ptr(y), y_row_stride, _ptr(workspace), workspace_bytes,
                                        _stream(stream)))


def lora_apply_stack(dtype: int, n_out: int, k_in: int, W, w_row_stride: int, routes, x,
                     x_row_stride: int, seq_slots, n: int, y, y_row_stride: int, workspace,
                     workspace_bytes: int, stream=None):
    """routes: DeviceRoutes, one per level; seq_slots: device int32 [n] tensors, one per level."""
    L = len(routes)
    assert L == len(seq_slots)
    rarr = (lora_route * max(L, 1))(*[r.c for r in routes])
    sarr = (C.c_void_p * max(L, 1))(*[_ptr(v) for v in seq_slots])
    _check(lib().lora_apply_stack(dtype, n_out, k_in, _ptr(W), w_row_stride,
                                  rarr if L else None, sarr if L else None, L, _ptr(x),
                                  x_row_stride, n, _ptr(y), y_row_stride, _ptr(workspace),
                                  workspace_bytes, _stream(stream)))


def lora_embedding_pair(a_file: np.ndarray, b_file: np.ndarray, n_vocab: int, n_embd: int) -> np.ndarray:
    """A [rank][n_embd] in the one layout from one file-layout embedding pair
    (A_file [n_vocab][rank], B_file [n_embd][rank]); B is A_file unchanged."""
    a = np.ascontiguousarray(a_file)
    b = np.ascontiguousarray(b_file)
    dt = LORA_BF16 if a.dtype == np.uint16 else LORA_F32
    out = np.empty((b.shape[1] if b.ndim == 2 else 0, n_embd), a.dtype)
    _check(lib().lora_embedding_pair(dt, n_vocab, n_embd, a.shape[0], a.shape[1], a.ctypes.data,
                                     b.shape[0], b.shape[1], b.ctypes.data, out.ctypes.data))
    return out


def lora_embed_rows(dtype: int, n_vocab: int, n_embd: int, E, e_row_stride: int, route,
                    token_ids, seq_slot, n: int, y, y_row_stride: int, stream=None):
    _check(lib().lora_embed_rows(dtype, n_vocab, n_embd, _ptr(E), e_row_stride, _route_ref(route),
                                 _ptr(token_ids), _ptr(seq_slot), n, _ptr(y), y_row_stride,
                                 _stream(stream)))
