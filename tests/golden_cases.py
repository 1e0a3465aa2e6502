"""Load the hand-worked cases under tests/golden/ as workloads."""
import json
import os

import numpy as np

from adapter_lora_bgmv_amd.workloads import AdapterSpec, Workload, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _arr(v, dtype):
    a = np.array(v, dtype=np.float32)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def expected_y(case):
    """The case's y as fp64, NaN for rows that are not written (null)."""
    n_out = case["k_in"] if case["kind"] == "embed" else case["n_out"]  # a gathered row is n_embd wide
    return np.array([[np.nan] * n_out if r is None else r for r in case["y"]], np.float64)


def _adapters(rows):
    return [AdapterSpec(rank=r, alpha=al, adapter_scale=s, rslora=rs) for (s, al, r, rs) in rows]


def hand_workload(case, dtype="f32"):
    if case["kind"] == "embed":
        a_file, b_file = _arr(case["a_file"], dtype), _arr(case["b_file"], dtype)
        tok = np.array(case["token_ids"], np.int32)
        ss = np.array(case["seq_slot"], np.int32)
        return Workload(name=case["name"], dtype=dtype, k_in=case["k_in"], n_out=case["n_out"],
                        max_rank=case["max_rank"], W=_arr(case["E"], dtype), A=a_file, B=b_file,
                        x=np.zeros((len(tok), 0), np.float32), adapters=_adapters(case["adapters"]),
                        kind="embed", adapter_slots=ss, padded_n=len(tok),
                        meta={"token_ids": tok, "seq_slot": ss, "a_file": a_file, "b_file": b_file})
    if case["kind"] == "stack":
        levels = [{"A": _arr(lv["A"], dtype), "B": _arr(lv["B"], dtype),
                   "adapters": _adapters(lv["adapters"]),
                   "seq_slot": np.array(lv["seq_slot"], np.int32)} for lv in case["levels"]]
        l0 = levels[0]
        return Workload(name=case["name"], dtype=dtype, k_in=case["k_in"], n_out=case["n_out"],
                        max_rank=case["max_rank"], W=_arr(case["W"], dtype), A=l0["A"], B=l0["B"],
                        x=_arr(case["x"], dtype), adapters=l0["adapters"], kind="stack",
                        adapter_slots=l0["seq_slot"], padded_n=len(l0["seq_slot"]),
                        meta={"levels": levels, "seq_slot": l0["seq_slot"]})
    ad = _adapters(case["adapters"])
    kw = dict(name=case["name"], dtype=dtype, k_in=case["k_in"], n_out=case["n_out"],
              max_rank=case["max_rank"], W=_arr(case["W"], dtype), A=_arr(case["A"], dtype),
              B=_arr(case["B"], dtype), x=_arr(case["x"], dtype), adapters=ad, kind=case["kind"])
    if case["kind"] == "decode":
        ss = np.array(case["seq_slot"], np.int32)
        # the hand cases give the device-side seq_slot buffer itself (with -1 rows), so
        # callers pass meta["seq_slot"] straight to the apply rather than building it
        kw.update(adapter_slots=ss, padded_n=len(ss), active=0, meta={"seq_slot": ss})
    elif case["kind"] == "segmented":
        kw.update(seg_indptr=np.array(case["seg_indptr"], np.int32),
                  seg_slot=np.array(case["seg_slot"], np.int32))
    elif case["kind"] == "moe_grouped":
        kw.update(n_experts=case["n_experts"],
                  expert_offsets=np.array(case["expert_offsets"], np.int32),
                  row_slot=np.array(case["seq_slot"], np.int32))
    else:
        kw.update(n_experts=case["n_experts"], top_k=case["top_k"],
                  indices=np.array(case["indices"], np.int32),
                  token_slot=np.array(case["token_slot"], np.int32))
    return Workload(**kw)
