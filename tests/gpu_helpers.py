"""Helpers shared by the GPU tests: move a generated workload to the GPU,
run the library through its C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

from oracle.case_io import decode_tensor

TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3
TOL_FP8_MAX = 6e-2

GUARD = 0x7FC1  # a NaN payload no kernel produces: marks rows that must stay untouched


def to_device(case: dict, device="cuda") -> dict:
    d = dict(case)
    for k in ("query", "block_tables", "seq_lens", "cum_seq_lens_q", "cum_seq_lens_kv",
              "kv_indptr", "kv_indices", "kv_last_page_len"):
        if case.get(k) is not None:
            d[k] = case[k].to(device)
    kv = case["kv_cache"]
    d["kv_cache"] = tuple(t.to(device) for t in kv) if isinstance(kv, tuple) else kv.to(device)
    d["sinks"] = None if case["sinks"] is None else case["sinks"].to(device)
    return d


_WORKSPACES = {}


def workspace(device="cuda") -> torch.Tensor:
    """One zeroed scheduler workspace per device, shared by every call (each
    call leaves it zero again; calls run one after another on one stream)."""
    import paged_kv_prefill_varlen_amd as ppa
    dev = torch.device(device)
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    if key not in _WORKSPACES:
        _WORKSPACES[key] = torch.zeros(ppa.WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    return _WORKSPACES[key]


def split_workspace(dcase: dict, kv_splits: int) -> torch.Tensor:
    """A zeroed workspace large enough for split-KV with this case."""
    import paged_kv_prefill_varlen_amd as ppa
    p = ppa.PpaParams()
    p.num_tokens, p.num_qo_heads, p.head_dim = (int(x) for x in dcase["query"].shape)
    p.kv_splits = kv_splits
    return torch.zeros(ppa.ppa_workspace_bytes(p), dtype=torch.uint8, device=dcase["query"].device)


def run_gpu(dcase: dict, out: torch.Tensor = None, bmm1=None, bmm2=None, stream=None,
            validate=True, schedule="persistent", lse: torch.Tensor = None, kv_splits: int = 0,
            ws: torch.Tensor = None, fp8_compute: bool = False) -> torch.Tensor:
    """schedule: "persistent" (workspace given: balanced persistent workgroups)
    or "grid" (no workspace: one workgroup per work item).  With kv_splits > 1
    a workspace of the needed size is allocated unless ``ws`` is given."""
    import paged_kv_prefill_varlen_amd as ppa
    if out is None:
        out = torch.empty_like(dcase["query"]).view(torch.int16).fill_(GUARD).view(torch.bfloat16)
    assert schedule in ("persistent", "grid")
    if ws is None:
        if kv_splits > 1:
            ws = split_workspace(dcase, kv_splits)
        elif schedule == "persistent":
            ws = workspace(dcase["query"].device)
    flat = dcase.get("kv_indptr") is not None
    ppa.batch_context_with_kv_cache(
        dcase["query"], dcase["kv_cache"], ws, None if flat else dcase["block_tables"], dcase["seq_lens"],
        dcase["max_q_len"], dcase["max_kv_len"],
        dcase["bmm1_scale"] if bmm1 is None else bmm1,
        dcase["bmm2_scale"] if bmm2 is None else bmm2,
        dcase["batch_size"], dcase["cum_seq_lens_q"], dcase["cum_seq_lens_kv"],
        window_left=dcase["window_left"], out=out, kv_layout=dcase["kv_layout"],
        sinks=dcase["sinks"], validate=validate, stream=stream, kv_indptr=dcase.get("kv_indptr"),
        kv_indices=dcase.get("kv_indices"), kv_last_page_len=dcase.get("kv_last_page_len"), lse=lse,
        kv_splits=kv_splits, fp8_compute=fp8_compute)
    return out


def guard_rows_untouched(out: torch.Tensor, written: np.ndarray) -> bool:
    raw = out.detach().cpu().view(torch.int16).numpy()
    return bool((raw[~written] == np.int16(GUARD)).all())


def errors(got: torch.Tensor, want: np.ndarray, rows: np.ndarray):
    g = decode_tensor(got.detach().cpu())[rows]
    w = want[rows]
    if g.size == 0:
        return 0.0, 0.0
    e = np.abs(g - w)
    if np.isnan(e).any():
        return float("nan"), float("nan")
    return float(e.max()), float(e.mean())


def assert_close(got, want, rows, fp8=False, what=""):
    mx, mean = errors(got, want, rows)
    tol_max = TOL_FP8_MAX if fp8 else TOL_BF16_MAX
    assert mx == mx, f"{what}: NaN in output"
    assert mx <= tol_max, f"{what}: max |err| {mx:.3e} > {tol_max}"
    if not fp8:
        assert mean <= TOL_BF16_MEAN, f"{what}: mean |err| {mean:.3e} > {TOL_BF16_MEAN}"
    return mx, mean


# lse = log(sum of bf16-rounded weights) + max: the rounding of each weight
# (relative 2^-9) bounds the sum's relative error, so |d lse| <= ~2e-3.
TOL_LSE = 5e-3


def lse_close(lse, want, written, what=""):
    """Max |lse - oracle| over the written rows, asserted <= TOL_LSE."""
    got = lse.detach().cpu().numpy()[written]
    w = want[written]
    assert np.isfinite(got).all(), f"{what}: non-finite lse"
    err = np.abs(got - w).max() if got.size else 0.0
    assert err <= TOL_LSE, f"{what}: lse max |err| {err:.3e}"
    return err
