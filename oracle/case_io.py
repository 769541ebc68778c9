"""Feeding a generated workload to the CPU oracle.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the
smoke check and the bench's CPU-baseline leg use it.

Values cross from torch to the oracle as raw storage codes (bf16 -> uint16,
float8 e4m3fn -> uint8) and the oracle decodes them with its own tables, so
no torch conversion routine stands between the inputs and the reference.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np
import torch

from .paged_attention import (attention_rows, decode_bf16, decode_e4m3fn,
                              paged_prefill_attention, paged_prefill_lse)


def _codes(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(f"unsupported storage dtype {t.dtype}")


def decode_tensor(t: torch.Tensor) -> np.ndarray:
    """A bf16 / float8_e4m3fn / float32 torch tensor -> float64 numpy."""
    if t.dtype == torch.bfloat16:
        return decode_bf16(_codes(t))
    if t.dtype == torch.float8_e4m3fn:
        return decode_e4m3fn(_codes(t))
    if t.dtype == torch.float32:
        return t.detach().cpu().numpy().astype(np.float64)
    raise TypeError(f"unsupported dtype {t.dtype}")


def oracle_inputs(case: dict) -> dict:
    kv = case["kv_cache"]
    if isinstance(kv, (tuple, list)):
        kv_np = (decode_tensor(kv[0]), decode_tensor(kv[1]))
    else:
        kv_np = decode_tensor(kv)
    sinks = case.get("sinks")
    return dict(
        query=decode_tensor(case["query"]),
        kv_cache=kv_np,
        kv_layout=case["kv_layout"],
        block_tables=None if case.get("kv_indptr") is not None else case["block_tables"].cpu().numpy(),
        kv_indptr=None if case.get("kv_indptr") is None else case["kv_indptr"].cpu().numpy(),
        kv_indices=None if case.get("kv_indices") is None else case["kv_indices"].cpu().numpy(),
        seq_lens=case["seq_lens"].cpu().numpy(),
        cum_seq_lens_q=case["cum_seq_lens_q"].cpu().numpy(),
        page_size=case["page_size"],
        bmm1_scale=float(np.float32(case["bmm1_scale"])),
        bmm2_scale=float(np.float32(case["bmm2_scale"])),
        window_left=case["window_left"],
        sinks=None if sinks is None else sinks.detach().cpu().numpy().astype(np.float64),
    )


def run_oracle(case: dict, requests: Optional[Sequence[int]] = None,
               inputs: Optional[dict] = None) -> Tuple[np.ndarray, np.ndarray]:
    """``(out float64 [num_tokens, H_q, D], written bool [num_tokens])``."""
    a = inputs if inputs is not None else oracle_inputs(case)
    return paged_prefill_attention(requests=requests, **a)


def run_oracle_lse(case: dict, inputs: Optional[dict] = None) -> np.ndarray:
    """``lse float64 [num_tokens, H_q]`` (natural log, sink included)."""
    a = dict(inputs if inputs is not None else oracle_inputs(case))
    return paged_prefill_lse(**a)


def run_oracle_rows(case: dict, rows: Sequence[Tuple[int, int]],
                    inputs: Optional[dict] = None) -> np.ndarray:
    """Selected (token, q head) output rows, ``[len(rows), D]`` float64."""
    a = inputs if inputs is not None else oracle_inputs(case)
    return attention_rows(rows=rows, **a)
