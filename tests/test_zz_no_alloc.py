"""The no-allocation entry point (ppa_paged_prefill_attention_noalloc),
through the C ABI, against the workspace entry point on the same inputs:
both run the same kernels, so outputs must match bit for bit.  Two calls in
a row on the library's shared scratch array, the second with a smaller
batch; split-KV partial states in the scratch; host-side rejections."""
from __future__ import annotations

import sys

import pytest
import torch

from gpu_helpers import GUARD, split_workspace, to_device, workspace
from workloads import make_case, make_custom_case

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _call(d, noalloc, ws=None, kv_splits=0, lse=None):
    import paged_kv_prefill_varlen_amd as ppa
    out = torch.empty_like(d["query"]).view(torch.int16).fill_(GUARD).view(torch.bfloat16)
    ppa.batch_context_with_kv_cache(
        d["query"], d["kv_cache"], None if noalloc else ws, d["block_tables"], d["seq_lens"], d["max_q_len"],
        d["max_kv_len"], d["bmm1_scale"], d["bmm2_scale"], d["batch_size"], d["cum_seq_lens_q"],
        d["cum_seq_lens_kv"], window_left=d["window_left"], out=out, kv_layout=d["kv_layout"], sinks=d["sinks"],
        kv_splits=kv_splits, lse=lse, noalloc=noalloc)
    return out


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_noalloc_matches_workspace_entry_two_calls():
    big = to_device(make_case("chunked"))
    small = to_device(make_custom_case(name="noalloc_small", batch=3, num_qo_heads=8, num_kv_heads=2,
                                       head_dim=64, page_size=16, q_lens=(40, 1, 77), prefix_lens=(9, 300, 0),
                                       window_left=50, sinks=True, seed=73))
    for name, d in (("chunked", big), ("small", small)):
        _say("noalloc", name)
        want = _call(d, noalloc=False, ws=workspace())
        got = _call(d, noalloc=True)
        torch.cuda.synchronize()
        assert _same(got, want), f"{name}: no-allocation entry differs from the workspace entry"
    # the same input again after the smaller one: the shared counters were
    # left in a state the next call accepts
    again = _call(big, noalloc=True)
    ref = _call(big, noalloc=False, ws=workspace())
    torch.cuda.synchronize()
    assert _same(again, ref)


def test_noalloc_split_kv_partials_in_scratch():
    d = to_device(make_custom_case(name="noalloc_split", batch=2, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                                   page_size=32, q_lens=(5, 17), prefix_lens=(2000, 900), sinks=True, seed=91))
    for splits in (3, 2):
        lse_a = torch.full(tuple(d["query"].shape[:2]), float("nan"), device="cuda")
        lse_b = torch.full(tuple(d["query"].shape[:2]), float("nan"), device="cuda")
        want = _call(d, noalloc=False, ws=split_workspace(d, splits), kv_splits=splits, lse=lse_a)
        got = _call(d, noalloc=True, kv_splits=splits, lse=lse_b)
        torch.cuda.synchronize()
        assert _same(got, want), f"split {splits}: outputs differ"
        assert torch.equal(lse_a.nan_to_num(0.0), lse_b.nan_to_num(0.0)), f"split {splits}: lse differs"


def test_noalloc_rejections():
    import paged_kv_prefill_varlen_amd as ppa
    d = to_device(make_custom_case(name="noalloc_rej", batch=1, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                                   page_size=32, q_lens=(1024,), prefix_lens=(0,), seed=5))
    # a workspace given to the entry that brings its own
    p = ppa.make_params(d["query"], d["kv_cache"], workspace(), d["block_tables"], d["seq_lens"], d["max_q_len"],
                        d["max_kv_len"], 0.1, 1.0, 1, d["cum_seq_lens_q"], d["cum_seq_lens_kv"], -1,
                        torch.empty_like(d["query"]), "HND")
    with pytest.raises(ppa.PpaError):
        ppa.ppa_paged_prefill_attention_noalloc(p)
    # split partial states beyond the scratch size
    assert ppa.ppa_noalloc_scratch_bytes() == 16 << 20
    with pytest.raises(ppa.PpaError):
        _call(d, noalloc=True, kv_splits=64)
