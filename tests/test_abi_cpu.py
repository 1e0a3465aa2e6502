"""The C-ABI library without a GPU: it loads, exports every declared symbol,
its host helpers follow the pages, and its validation refuses bad calls with
messages naming every dimension -- before any HIP call."""
import ctypes as C
import re
from pathlib import Path

import numpy as np
import pytest

import golden_cases
from adapter_lora_bgmv_amd import binding as B
from adapter_lora_bgmv_amd import workloads as WL

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def L():
    return B.lib()


def declared_functions():
    names = set()
    for h in (ROOT / "include").glob("*.h"):
        text = h.read_text()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(lora_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 12, names
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(B.EXPORTS)


def test_version(L):
    assert "gfx950" in B.lora_version()


def test_scale_examples_from_the_pages():
    for ex in golden_cases.load("scale_examples.json")["examples"]:
        got = B.lora_scale(ex["adapter_scale"], ex["alpha"], ex["rank"], ex["rslora"])
        assert abs(got - ex["scale"]) <= 1e-15 * max(1.0, abs(ex["scale"])), ex


def test_scale_table_from_the_pages():
    t = golden_cases.load("scale_examples.json")["table"]
    ad = [WL.AdapterSpec(rank=r, alpha=al, adapter_scale=s, rslora=rs)
          for (s, al, r, rs) in t["adapters"]]
    got = B.lora_scale_table(ad, t["max_loras"])
    assert np.array_equal(got, np.array(t["values_f32"], np.float32))


def test_seq_slot_examples_from_the_pages():
    for ex in golden_cases.load("seq_slot_examples.json")["examples"]:
        got = B.lora_build_seq_slot(ex["adapter_slots"], ex["padded_n"], ex["active"])
        assert list(got) == ex["seq_slot"], ex


def test_seq_slot_refuses_more_rows_than_padding(L):
    a = np.zeros(4, np.int32)
    out = np.zeros(2, np.int32)
    rc = L.lora_build_seq_slot(a.ctypes.data, 4, 2, 0, out.ctypes.data)
    assert rc == -1 and "padded_n 2" in L.lora_last_error().decode()


def test_workspace_bytes():
    assert B.lora_workspace_bytes(0, B.LORA_F32, 64, 4096, 4096, 16) == 0
    assert B.lora_workspace_bytes(0, B.LORA_BF16, 0, 4096, 4096, 16) == 0
    ws = B.lora_workspace_bytes(0, B.LORA_BF16, 64, 4096, 4096, 16)
    assert ws >= 64 * 16 * 4  # at least t
    assert B.lora_workspace_bytes(2, B.LORA_BF16, 3072, 2048, 1408, 16, 64) > 3072 * 16 * 4


# -------------------------------------------------------------- validation
FAKE = 4096  # an aligned non-NULL address; validation fails before it is used


def _route(dtype=B.LORA_BF16, n_out=64, k_in=64, R=16, max_loras=4):
    return B.lora_route(FAKE, FAKE, FAKE, max_loras, k_in, n_out, R, dtype)


def _apply(L, **kw):
    a = dict(dtype=B.LORA_BF16, n_out=64, k_in=64, W=FAKE, w_stride=64, route=_route(), x=FAKE,
             x_stride=64, seq=FAKE, n=8, y=FAKE, y_stride=64, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    r = a["route"]
    rc = L.lora_apply(a["dtype"], a["n_out"], a["k_in"], a["W"], a["w_stride"],
                      C.byref(r) if r is not None else None, a["x"], a["x_stride"], a["seq"], a["n"],
                      a["y"], a["y_stride"], a["ws"], a["ws_bytes"], None)
    return rc, L.lora_last_error().decode()


def test_noalloc_refuses_a_problem_beyond_its_scratch(L):
    """lora_apply_noalloc checks its scratch need before any HIP call: a
    16384-row batch at rank 64 over k_in 4096 needs more than the 32 MiB
    array and is refused, the message naming the need and the limit."""
    need = B.lora_workspace_bytes(0, B.LORA_BF16, 16384, 64, 4096, 64) + (1 << 20)
    assert need > B.LORA_NOALLOC_SCRATCH_BYTES
    r = _route(n_out=64, k_in=4096, R=64)
    rc = L.lora_apply_noalloc(B.LORA_BF16, 64, 4096, FAKE, 4096, C.byref(r), FAKE, 4096, FAKE, 16384,
                              FAKE, 64, None)
    msg = L.lora_last_error().decode()
    assert rc == -7, msg
    assert f"the limit is {B.LORA_NOALLOC_SCRATCH_BYTES}" in msg and "n 16384" in msg


def test_refuses_x_stride_below_k_in(L):
    rc, msg = _apply(L, x_stride=32)
    assert rc == -3
    assert "x_row_stride 32 < k_in 64" in msg and "[n_out 64 x k_in 64]" in msg


def test_refuses_y_stride_below_n_out(L):
    rc, msg = _apply(L, y_stride=8)
    assert rc == -3 and "y_row_stride 8 < n_out 64" in msg


def test_refuses_bad_dtype(L):
    rc, msg = _apply(L, dtype=7)
    assert rc == -4 and "dtype 7" in msg


def test_refuses_route_dtype_mismatch(L):
    rc, msg = _apply(L, route=_route(dtype=B.LORA_F32))
    assert rc == -4 and "route dtype 0" in msg


def test_refuses_route_shape_mismatch(L):
    rc, msg = _apply(L, route=_route(n_out=128))
    assert rc == -1 and "[n_out 128 x k_in 64]" in msg and "[n_out 64 x k_in 64]" in msg


def test_refuses_zero_rank_and_names_it(L):
    rc, msg = _apply(L, route=_route(R=0))
    assert rc == -1 and "max_rank 0" in msg


def test_refuses_bf16_rank_not_multiple_of_16(L):
    rc, msg = _apply(L, route=_route(R=8))
    assert rc == -5 and "max_rank 8" in msg


def test_refuses_misaligned_bf16_shapes(L):
    rc, msg = _apply(L, k_in=60, w_stride=60, x_stride=60, route=_route(k_in=60))
    assert rc == -5 and "k_in 60" in msg


def test_refuses_null_pointers(L):
    rc, msg = _apply(L, W=None)
    assert rc == -2 and "W" in msg
    rc, msg = _apply(L, seq=None)
    assert rc == -2 and "seq_slot" in msg


def test_refuses_small_workspace(L):
    rc, msg = _apply(L, ws_bytes=16)
    # validation precedes the device check, so this is WORKSPACE even with no GPU ...
    # ... unless the device check comes first; both are refusals before any launch
    assert rc in (-7, -6)


def test_refuses_zero_dims(L):
    rc, msg = _apply(L, n_out=0, route=None)
    assert rc == -1 and "n_out 0" in msg


def test_refuses_too_many_rows(L):
    rc, msg = _apply(L, n=1 << 20)
    assert rc == -1 and "rows exceeds" in msg


def test_empty_batch_launches_nothing(L):
    rc, msg = _apply(L, n=0)
    assert rc == 0


def test_no_gpu_is_a_loud_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, msg = _apply(L)
    assert rc in (-6, -7) and msg


def test_moe_refuses_zero_top_k(L):
    rc = L.lora_apply_moe_gather(B.LORA_BF16, 4, 64, 64, FAKE, 64 * 64, 64, None, FAKE, 64, FAKE, 0,
                                 None, 8, FAKE, 64, FAKE, 1 << 20, None)
    assert rc == -1 and "top_k 0" in L.lora_last_error().decode()


def test_shrink_and_expand_refuse_null_route(L):
    assert L.lora_shrink(None, FAKE, 64, FAKE, 4, FAKE, None) == -2
    assert L.lora_expand_fold(None, FAKE, FAKE, 4, FAKE, 64, None) == -2


def _moe_route(E=4, max_loras=2, n_out=64, k_in=64, R=16, dtype=B.LORA_BF16):
    return B.lora_route_moe(FAKE, FAKE, FAKE, max_loras, E, k_in, n_out, R, dtype)


def test_grouped_refuses_null_route_and_null_offsets(L):
    r = _moe_route()
    assert L.lora_moe_grouped_shrink(None, FAKE, 64, FAKE, FAKE, 4, FAKE, None) == -2
    assert L.lora_moe_grouped_expand_fold(None, FAKE, FAKE, FAKE, 4, FAKE, 64, None) == -2
    assert L.lora_moe_grouped_shrink(C.byref(r), FAKE, 64, None, FAKE, 4, FAKE, None) == -2
    assert "expert_offsets" in L.lora_last_error().decode()
    rc = L.lora_apply_moe_grouped(B.LORA_BF16, 4, 64, 64, FAKE, 64 * 64, 64, C.byref(r), FAKE, 64,
                                  None, FAKE, 8, FAKE, 64, FAKE, 1 << 20, None)
    assert rc == -2 and "expert_offsets" in L.lora_last_error().decode()


def test_grouped_refuses_route_over_other_experts(L):
    r = _moe_route(E=8)
    rc = L.lora_apply_moe_grouped(B.LORA_BF16, 4, 64, 64, FAKE, 64 * 64, 64, C.byref(r), FAKE, 64,
                                  FAKE, FAKE, 8, FAKE, 64, FAKE, 1 << 20, None)
    msg = L.lora_last_error().decode()
    assert rc == -1 and "over 8 experts" in msg and "over 4" in msg


def test_grouped_refuses_small_expert_stride_and_bad_strides(L):
    rc = L.lora_apply_moe_grouped(B.LORA_BF16, 4, 64, 64, FAKE, 64 * 63, 64, None, FAKE, 64,
                                  FAKE, None, 8, FAKE, 64, FAKE, 1 << 20, None)
    assert rc == -3 and "expert_stride" in L.lora_last_error().decode()
    r = _moe_route()
    assert L.lora_moe_grouped_shrink(C.byref(r), FAKE, 32, FAKE, FAKE, 4, FAKE, None) == -3
    assert "x_row_stride 32 < k_in 64" in L.lora_last_error().decode()
    assert L.lora_moe_grouped_expand_fold(C.byref(r), FAKE, FAKE, FAKE, 4, FAKE, 16, None) == -3
    assert "y_row_stride 16 < n_out 64" in L.lora_last_error().decode()


def test_grouped_empty_batch_launches_nothing(L):
    r = _moe_route()
    assert L.lora_moe_grouped_shrink(C.byref(r), None, 64, None, None, 0, None, None) == 0
    assert L.lora_moe_grouped_expand_fold(C.byref(r), None, None, None, 0, None, 64, None) == 0
    assert L.lora_apply_moe_grouped(B.LORA_BF16, 4, 64, 64, None, 64 * 64, 64, C.byref(r), None,
                                    64, None, None, 0, None, 64, None, 0, None) == 0


def test_grouped_workspace_counts_expert_tiles(L):
    a = L.lora_workspace_bytes(B.LORA_OP_MOE_GROUPED, B.LORA_BF16, 3072, 2048, 1408, 16, 64)
    g = L.lora_workspace_bytes(B.LORA_OP_MOE_GATHER, B.LORA_BF16, 3072, 2048, 1408, 16, 64)
    assert a == g > 0


def _stack_call(L, routes, n_levels, seq=None, ws_bytes=1 << 30, dtype=B.LORA_BF16, n=8):
    arr = (B.lora_route * max(1, len(routes)))(*routes) if routes else None
    sarr = (C.c_void_p * max(1, n_levels))(*([FAKE] * n_levels)) if seq is None else seq
    return L.lora_apply_stack(dtype, 64, 64, FAKE, 64, arr, sarr if n_levels else None, n_levels,
                              FAKE, 64, n, FAKE, 64, FAKE, ws_bytes, None)


def test_stack_refuses_too_many_levels_and_misfit_levels(L):
    rs = [_route() for _ in range(9)]
    assert _stack_call(L, rs, 9) == -1 and "9 levels" in L.lora_last_error().decode()
    rs = [_route(), _route(n_out=32)]
    rc = _stack_call(L, rs, 2)
    assert rc == -1 and "[n_out 32 x k_in 64]" in L.lora_last_error().decode()
    rs = [_route(), _route(dtype=B.LORA_F32)]
    assert _stack_call(L, rs, 2) == -4


def test_stack_refuses_null_slot_buffers_and_small_workspace(L):
    rs = [_route(), _route()]
    sarr = (C.c_void_p * 2)(FAKE, None)
    assert _stack_call(L, rs, 2, seq=sarr) == -2 and "seq_slots[1]" in L.lora_last_error().decode()
    assert _stack_call(L, rs, 2, ws_bytes=64) == -7
    assert "2 levels" in L.lora_last_error().decode()


def test_stack_workspace_grows_with_levels(L):
    one = L.lora_workspace_bytes(B.LORA_OP_STACK, B.LORA_BF16, 64, 4096, 4096, 16, 1)
    three = L.lora_workspace_bytes(B.LORA_OP_STACK, B.LORA_BF16, 64, 4096, 4096, 16, 3)
    two = L.lora_workspace_bytes(B.LORA_OP_STACK, B.LORA_BF16, 64, 4096, 4096, 16, 2)
    assert three - two == two - one >= 64 * 16 * 4  # a further level: at least its t [n][R]
    assert L.lora_workspace_bytes(B.LORA_OP_STACK, B.LORA_F32, 4, 256, 256, 8, 2) == 256
    assert one >= L.lora_workspace_bytes(B.LORA_OP_APPLY, B.LORA_BF16, 64, 4096, 4096, 16, 1)


def test_stack_empty_batch_launches_nothing(L):
    assert _stack_call(L, [_route(), _route()], 2, n=0) == 0


def test_embedding_pair_is_the_transpose_of_b_file():
    rng = np.random.default_rng(3)
    for dt in (np.float32, np.uint16):
        a_file = rng.integers(0, 60000, (50, 7)).astype(dt)
        b_file = rng.integers(0, 60000, (24, 7)).astype(dt)
        a = B.lora_embedding_pair(a_file, b_file, 50, 24)
        assert a.shape == (7, 24) and np.array_equal(a, b_file.T)


def test_embedding_pair_refuses_misfit_shapes(L):
    a = np.zeros((50, 7), np.float32)
    b = np.zeros((24, 6), np.float32)
    out = np.zeros((7, 24), np.float32)
    rc = L.lora_embedding_pair(B.LORA_F32, 50, 24, 50, 7, a.ctypes.data, 24, 6, b.ctypes.data,
                               out.ctypes.data)
    msg = L.lora_last_error().decode()
    assert rc == -1 and "[50 x 7]" in msg and "[24 x 6]" in msg and "n_vocab 50" in msg


def test_embed_rows_validation(L):
    r = B.lora_route(FAKE, FAKE, FAKE, 4, 64, 1000, 16, B.LORA_BF16)  # k_in n_embd, n_out n_vocab
    call = lambda **k: L.lora_embed_rows(k.get("dt", B.LORA_BF16), k.get("nv", 1000),
                                         k.get("ne", 64), FAKE, k.get("es", 64),
                                         C.byref(k.get("r", r)), FAKE, FAKE, 8, FAKE,
                                         k.get("ys", 64), None)
    assert call(ne=60, es=64, ys=64) == -5 and "multiples of 8" in L.lora_last_error().decode()
    assert call(ys=32) == -3
    assert call(nv=999) == -1  # the route's n_out is the vocabulary
    assert "[n_out 1000 x k_in 64]" in L.lora_last_error().decode()
    assert L.lora_embed_rows(B.LORA_BF16, 1000, 64, None, 64, C.byref(r), None, None, 0, None, 64,
                             None) == 0
