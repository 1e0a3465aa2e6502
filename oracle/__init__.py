"""The fp64 CPU oracle for the routed multi-LoRA projection -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The HIP library and its Python
binding never import, load or call anything here, and this package never
imports them: the two sides share only the seeded input generators in
``adapter_lora_bgmv_amd.workloads`` (which hold none of the method's
arithmetic).

The arithmetic lives in ``lora_oracle.c`` (plain C, fp64, sequential sums);
this module only marshals numpy arrays into it.  Pins that tie the oracle to
the pages, independently of itself, are in ``tests/test_oracle_pins.py``.
Parity status of each function is listed in the C file's header; every
function here is pinned (no "parity unpinned" entry).
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_i32p = C.POINTER(C.c_int32)
_f32p = C.POINTER(C.c_float)
_f64p = C.POINTER(C.c_double)

F32, BF16 = 0, 1


class _Route(C.Structure):
    _fields_ = [("a", C.POINTER(C.c_void_p)), ("b", C.POINTER(C.c_void_p)),
                ("scale", _f32p), ("max_loras", C.c_int), ("n_experts", C.c_int),
                ("k_in", C.c_int), ("n_out", C.c_int), ("max_rank", C.c_int),
                ("dtype", C.c_int)]


def _p(a: np.ndarray, t=C.c_void_p):
    return a.ctypes.data_as(t) if t is not C.c_void_p else C.c_void_p(a.ctypes.data)


class Route:
    """Host-pointer route tables over a pool held as numpy arrays.

    ``A``/``B`` are ``[P][max_rank][k_in]`` / ``[P][n_out][max_rank]``;
    ``null_slots`` lists pool indices whose table entries are NULL.
    """

    def __init__(self, A: np.ndarray, B: np.ndarray, scale_table: np.ndarray, dtype: int,
                 k_in: int, n_out: int, max_rank: int, n_experts: int = 1,
                 null_slots: Sequence[int] = (), b_row_offset: int = 0):
        self.A = np.ascontiguousarray(A)
        self.B = np.ascontiguousarray(B)
        self.scale = np.ascontiguousarray(scale_table, dtype=np.float32)
        P = self.A.shape[0]
        esz = self.A.itemsize
        ap = (C.c_void_p * P)()
        bp = (C.c_void_p * P)()
        for p in range(P):
            if p in set(null_slots):
                ap[p] = None
                bp[p] = None
            else:
                ap[p] = self.A.ctypes.data + p * self.A.strides[0]
                # b_row_offset selects a block of B's rows (fused-projection split)
                bp[p] = self.B.ctypes.data + p * self.B.strides[0] + b_row_offset * max_rank * esz
        self._ap, self._bp = ap, bp
        self.c = _Route(C.cast(ap, C.POINTER(C.c_void_p)), C.cast(bp, C.POINTER(C.c_void_p)),
                        _p(self.scale, _f32p), len(self.scale), n_experts, k_in, n_out,
                        max_rank, dtype)


class Oracle:
    def __init__(self, path: Optional[Path] = None):
        path = Path(path) if path is not None else _build.LIB
        if not path.exists():
            _build.build(path)
        self.path = path
        L = C.CDLL(str(path))
        L.orc_scale.restype = C.c_double
        L.orc_scale.argtypes = [C.c_double, C.c_double, C.c_int, C.c_int]
        L.orc_scale_table.argtypes = [C.c_int, _f64p, _f64p, _i32p, _i32p, C.c_int, _f32p]
        L.orc_build_seq_slot.argtypes = [_i32p, C.c_int, C.c_int, C.c_int, _i32p]
        RP = C.POINTER(_Route)
        L.orc_shrink.argtypes = [RP, C.c_void_p, C.c_int, _i32p, C.c_int, _f64p]
        L.orc_expand_fold.argtypes = [RP, _f32p, _i32p, C.c_int, C.c_void_p, C.c_int, _f64p]
        L.orc_apply.argtypes = [C.c_void_p, C.c_int, RP, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                C.c_int, _i32p, C.c_int, _f64p]
        L.orc_apply_rows.argtypes = [C.c_void_p, C.c_int, RP, C.c_int, C.c_int, C.c_int,
                                     C.c_void_p, C.c_int, _i32p, _i32p, C.c_int, _f64p]
        L.orc_apply_segmented.argtypes = [C.c_void_p, C.c_int, RP, C.c_int, C.c_int, C.c_int,
                                          C.c_void_p, C.c_int, _i32p, _i32p, C.c_int, _i32p,
                                          C.c_int, _f64p]
        L.orc_apply_moe_gather.argtypes = [C.c_void_p, C.c_longlong, C.c_int, RP, C.c_int,
                                           C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_int, _i32p,
                                           C.c_int, _i32p, _i32p, C.c_int, _f64p]
        L.orc_apply_moe_grouped.argtypes = [C.c_void_p, C.c_longlong, C.c_int, RP, C.c_int,
                                            C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_int,
                                            _i32p, _i32p, _i32p, C.c_int, _f64p]
        L.orc_moe_grouped_shrink.argtypes = [RP, C.c_void_p, C.c_int, _i32p, _i32p, C.c_int,
                                             _f64p]
        L.orc_moe_grouped_expand_fold.argtypes = [RP, _f32p, _i32p, _i32p, C.c_int, C.c_void_p,
                                                  C.c_int, _f64p]
        L.orc_apply_stack.argtypes = [C.c_void_p, C.c_int, C.POINTER(RP), C.POINTER(_i32p),
                                      C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_int,
                                      _i32p, C.c_int, _f64p]
        L.orc_embed_rows.argtypes = [C.c_void_p, C.c_int, RP, C.c_int, C.c_int, C.c_int, _i32p,
                                     _i32p, _i32p, C.c_int, _f64p]
        L.orc_embedding_pair.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p]
        L.orc_mutant.restype = C.c_int
        L.orc_threads.restype = C.c_int
        L.orc_set_threads.argtypes = [C.c_int]
        self.L = L

    # -------------------------------------------------------------- helpers
    @property
    def threads(self) -> int:
        return int(self.L.orc_threads())

    def set_threads(self, n: int) -> None:
        """Threads the row loops use from now on (timing only)."""
        self.L.orc_set_threads(int(n))

    @property
    def mutant(self) -> int:
        return int(self.L.orc_mutant())

    def scale(self, adapter_scale: float, alpha: float, rank: int, rslora: bool) -> float:
        return float(self.L.orc_scale(adapter_scale, alpha, int(rank), int(bool(rslora))))

    def scale_table(self, adapters, max_loras: Optional[int] = None) -> np.ndarray:
        n = len(adapters)
        m = n if max_loras is None else int(max_loras)
        s = np.array([a.adapter_scale for a in adapters] or [0.0], np.float64)
        al = np.array([a.alpha for a in adapters] or [0.0], np.float64)
        r = np.array([a.rank for a in adapters] or [1], np.int32)
        rs = np.array([int(a.rslora) for a in adapters] or [0], np.int32)
        out = np.empty(max(m, 1), np.float32)
        self.L.orc_scale_table(n, _p(s, _f64p), _p(al, _f64p), _p(r, _i32p), _p(rs, _i32p), m,
                               _p(out, _f32p))
        return out[:m]

    def build_seq_slot(self, adapter_slots, padded_n: int, active: int) -> np.ndarray:
        a = np.ascontiguousarray(adapter_slots, np.int32)
        out = np.empty(max(padded_n, 1), np.int32)
        self.L.orc_build_seq_slot(_p(a, _i32p), len(a), int(padded_n), int(active),
                                  _p(out, _i32p))
        return out[:padded_n]

    def route_for(self, wl, scale_table=None, null_slots=None, b_row_offset=0,
                  n_out=None) -> Route:
        st = self.scale_table(wl.adapters) if scale_table is None else scale_table
        ns = wl.null_slots if null_slots is None else null_slots
        return Route(wl.A, wl.B, st, BF16 if wl.dtype == "bf16" else F32, wl.k_in,
                     wl.n_out if n_out is None else n_out, wl.max_rank,
                     max(1, wl.n_experts), ns, b_row_offset)

    # -------------------------------------------------------------- ops
    def shrink(self, route: Route, x: np.ndarray, seq_slot, x_stride: Optional[int] = None,
               fill: float = np.nan) -> np.ndarray:
        x = np.ascontiguousarray(x)
        n = x.shape[0]
        xs = x.shape[1] if x_stride is None else x_stride
        ss = np.ascontiguousarray(seq_slot, np.int32)
        t = np.full((n, route.c.max_rank), fill, np.float64)
        self.L.orc_shrink(C.byref(route.c), _p(x), xs, _p(ss, _i32p), n, _p(t, _f64p))
        return t

    def expand_fold(self, route: Route, t: np.ndarray, seq_slot, y_in: np.ndarray) -> np.ndarray:
        t = np.ascontiguousarray(t, np.float32)
        y_in = np.ascontiguousarray(y_in)
        n = y_in.shape[0]
        ss = np.ascontiguousarray(seq_slot, np.int32)
        out = np.empty((n, route.c.n_out), np.float64)
        self.L.orc_expand_fold(C.byref(route.c), _p(t, _f32p), _p(ss, _i32p), n, _p(y_in),
                               y_in.shape[1], _p(out, _f64p))
        return out

    def apply(self, W: np.ndarray, route: Optional[Route], x: np.ndarray, seq_slot,
              dtype: int, rows=None) -> np.ndarray:
        """y = W x (+ routed delta) for all rows, or for the listed ``rows``."""
        W = np.ascontiguousarray(W)
        x = np.ascontiguousarray(x)
        n_out, k_in = W.shape
        rp = C.byref(route.c) if route is not None else None
        ss = None if seq_slot is None else np.ascontiguousarray(seq_slot, np.int32)
        ssp = _p(ss, _i32p) if ss is not None else None
        if rows is None:
            y = np.empty((x.shape[0], n_out), np.float64)
            self.L.orc_apply(_p(W), W.shape[1], rp, dtype, k_in, n_out, _p(x), x.shape[1], ssp,
                             x.shape[0], _p(y, _f64p))
            return y
        rr = np.ascontiguousarray(rows, np.int32)
        y = np.empty((len(rr), n_out), np.float64)
        self.L.orc_apply_rows(_p(W), W.shape[1], rp, dtype, k_in, n_out, _p(x), x.shape[1], ssp,
                              _p(rr, _i32p), len(rr), _p(y, _f64p))
        return y

    def apply_segmented(self, W, route, x, seg_indptr, seg_slot, dtype, rows=None,
                        fill=np.nan) -> np.ndarray:
        W = np.ascontiguousarray(W)
        x = np.ascontiguousarray(x)
        n_out, k_in = W.shape
        ip = np.ascontiguousarray(seg_indptr, np.int32)
        sl = np.ascontiguousarray(seg_slot, np.int32)
        rr = np.arange(x.shape[0], dtype=np.int32) if rows is None else \
            np.ascontiguousarray(rows, np.int32)
        y = np.full((len(rr), n_out), fill, np.float64)
        rp = C.byref(route.c) if route is not None else None
        self.L.orc_apply_segmented(_p(W), W.shape[1], rp, dtype, k_in, n_out, _p(x), x.shape[1],
                                   _p(ip, _i32p), _p(sl, _i32p), len(sl), _p(rr, _i32p),
                                   len(rr), _p(y, _f64p))
        return y

    def apply_moe(self, W, route, x, indices, top_k, token_slot, dtype, rows=None,
                  fill=np.nan) -> np.ndarray:
        W = np.ascontiguousarray(W)
        x = np.ascontiguousarray(x)
        E, n_out, k_in = W.shape
        idx = np.ascontiguousarray(indices, np.int32)
        ts = np.ascontiguousarray(token_slot, np.int32)
        rr = np.arange(x.shape[0], dtype=np.int32) if rows is None else \
            np.ascontiguousarray(rows, np.int32)
        y = np.full((len(rr), n_out), fill, np.float64)
        rp = C.byref(route.c) if route is not None else None
        self.L.orc_apply_moe_gather(_p(W), n_out * k_in, k_in, rp, dtype, k_in, n_out, E, _p(x),
                                    x.shape[1], _p(idx, _i32p), int(top_k), _p(ts, _i32p),
                                    _p(rr, _i32p), len(rr), _p(y, _f64p))
        return y

    def apply_moe_grouped(self, W, route, x, expert_offsets, seq_slot, dtype, rows=None,
                          fill=np.nan) -> np.ndarray:
        """Grouped MoE: rows sorted by expert, expert e's rows in
        [expert_offsets[e], expert_offsets[e+1]); rows outside every range
        keep ``fill``."""
        W = np.ascontiguousarray(W)
        x = np.ascontiguousarray(x)
        E, n_out, k_in = W.shape
        off = np.ascontiguousarray(expert_offsets, np.int32)
        assert len(off) == E + 1
        ss = None if seq_slot is None else np.ascontiguousarray(seq_slot, np.int32)
        rr = np.arange(x.shape[0], dtype=np.int32) if rows is None else \
            np.ascontiguousarray(rows, np.int32)
        y = np.full((len(rr), n_out), fill, np.float64)
        rp = C.byref(route.c) if route is not None else None
        self.L.orc_apply_moe_grouped(_p(W), n_out * k_in, k_in, rp, dtype, k_in, n_out, E, _p(x),
                                     x.shape[1], _p(off, _i32p),
                                     _p(ss, _i32p) if ss is not None else None,
                                     _p(rr, _i32p), len(rr), _p(y, _f64p))
        return y

    def moe_grouped_shrink(self, route: Route, x, expert_offsets, seq_slot,
                           fill: float = np.nan) -> np.ndarray:
        x = np.ascontiguousarray(x)
        n = x.shape[0]
        off = np.ascontiguousarray(expert_offsets, np.int32)
        assert len(off) == route.c.n_experts + 1
        ss = np.ascontiguousarray(seq_slot, np.int32)
        t = np.full((n, route.c.max_rank), fill, np.float64)
        self.L.orc_moe_grouped_shrink(C.byref(route.c), _p(x), x.shape[1], _p(off, _i32p),
                                      _p(ss, _i32p), n, _p(t, _f64p))
        return t

    def moe_grouped_expand_fold(self, route: Route, t, expert_offsets, seq_slot,
                                y_in) -> np.ndarray:
        t = np.ascontiguousarray(t, np.float32)
        y_in = np.ascontiguousarray(y_in)
        n = y_in.shape[0]
        off = np.ascontiguousarray(expert_offsets, np.int32)
        assert len(off) == route.c.n_experts + 1
        ss = np.ascontiguousarray(seq_slot, np.int32)
        out = np.empty((n, route.c.n_out), np.float64)
        self.L.orc_moe_grouped_expand_fold(C.byref(route.c), _p(t, _f32p), _p(off, _i32p),
                                           _p(ss, _i32p), n, _p(y_in), y_in.shape[1],
                                           _p(out, _f64p))
        return out

    def apply_stack(self, W, routes, x, seq_slots, dtype, rows=None) -> np.ndarray:
        """y = W x + the deltas of every level in order; routes[l] / seq_slots[l] per level."""
        W = np.ascontiguousarray(W)
        x = np.ascontiguousarray(x)
        n_out, k_in = W.shape
        L = len(routes)
        assert L == len(seq_slots)
        ss = [np.ascontiguousarray(v, np.int32) for v in seq_slots]
        rarr = (C.POINTER(_Route) * max(L, 1))(*[C.pointer(r.c) for r in routes])
        sarr = (_i32p * max(L, 1))(*[_p(v, _i32p) for v in ss])
        rr = np.arange(x.shape[0], dtype=np.int32) if rows is None else \
            np.ascontiguousarray(rows, np.int32)
        y = np.empty((len(rr), n_out), np.float64)
        self.L.orc_apply_stack(_p(W), W.shape[1], rarr, sarr, L, dtype, k_in, n_out, _p(x),
                               x.shape[1], _p(rr, _i32p), len(rr), _p(y, _f64p))
        return y

    def embed_rows(self, E, route: Optional[Route], token_ids, seq_slot, dtype, rows=None,
                   fill=np.nan) -> np.ndarray:
        """y[i] = E[token_ids[i]] (+ s * B[token] A); route k_in = n_embd, n_out = n_vocab."""
        E = np.ascontiguousarray(E)
        n_vocab, n_embd = E.shape
        tok = np.ascontiguousarray(token_ids, np.int32)
        ss = None if seq_slot is None else np.ascontiguousarray(seq_slot, np.int32)
        rr = np.arange(len(tok), dtype=np.int32) if rows is None else \
            np.ascontiguousarray(rows, np.int32)
        y = np.full((len(rr), n_embd), fill, np.float64)
        rp = C.byref(route.c) if route is not None else None
        self.L.orc_embed_rows(_p(E), n_embd, rp, dtype, n_vocab, n_embd, _p(tok, _i32p),
                              _p(ss, _i32p) if ss is not None else None, _p(rr, _i32p), len(rr),
                              _p(y, _f64p))
        return y

    def embedding_pair(self, b_file, dtype: int) -> np.ndarray:
        """A [rank][n_embd] from one pair's B_file [n_embd][rank]."""
        b = np.ascontiguousarray(b_file)
        n_embd, rank = b.shape
        out = np.empty((rank, n_embd), b.dtype)
        self.L.orc_embedding_pair(_p(b), dtype, n_embd, rank, _p(out))
        return out

    def embed_route(self, wl, scale_table=None) -> Route:
        """The route of an embedding workload: its file-layout pool in the one layout."""
        dt = BF16 if wl.dtype == "bf16" else F32
        st = self.scale_table(wl.adapters) if scale_table is None else scale_table
        A = np.stack([self.embedding_pair(b, dt) for b in wl.meta["b_file"]])
        return Route(A, wl.meta["a_file"], st, dt, wl.k_in, wl.n_out, wl.max_rank,
                     null_slots=wl.null_slots)

    # -------------------------------------------------------------- workload glue
    def seq_slot_for(self, wl) -> np.ndarray:
        return self.build_seq_slot(wl.adapter_slots, wl.padded_n, wl.active)

    def run(self, wl, rows=None, route: bool = True, scale_table=None) -> np.ndarray:
        """The whole path for a workload: y (fp64) for all rows or the given ones."""
        dt = BF16 if wl.dtype == "bf16" else F32
        r = self.route_for(wl, scale_table) if route and wl.kind not in ("embed", "stack") else None
        if wl.kind == "decode":
            return self.apply(wl.W, r, wl.x, self.seq_slot_for(wl), dt, rows)
        if wl.kind == "segmented":
            return self.apply_segmented(wl.W, r, wl.x, wl.seg_indptr, wl.seg_slot, dt, rows)
        if wl.kind == "moe":
            return self.apply_moe(wl.W, r, wl.x, wl.indices, wl.top_k, wl.token_slot, dt, rows)
        if wl.kind == "embed":
            r = self.embed_route(wl, scale_table) if route else None
            return self.embed_rows(wl.W, r, wl.meta["token_ids"], wl.meta["seq_slot"] if route
                                   else None, dt, rows)
        if wl.kind == "stack":
            levels = wl.meta["levels"]
            sts = [self.scale_table(lv["adapters"]) for lv in levels] if scale_table is None \
                else scale_table
            routes = [Route(lv["A"], lv["B"], st, dt, wl.k_in, wl.n_out, wl.max_rank)
                      for lv, st in zip(levels, sts)] if route else []
            return self.apply_stack(wl.W, routes, wl.x,
                                    [lv["seq_slot"] for lv in levels] if route else [], dt, rows)
        if wl.kind == "moe_grouped":
            return self.apply_moe_grouped(wl.W, r, wl.x, wl.expert_offsets, wl.row_slot, dt,
                                          rows)
        raise ValueError(wl.kind)


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
