"""GPU: the attention call captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed.  Between replays the program does eager work of its own (it
rewrites the captured query buffer and makes eager calls of the same entry
point), and every replay's output must equal, bit for bit, an eager call on
the same inputs.  Covered: the workspace entry point (persistent
scheduler, counters returned to zero by the kernel itself), split-KV with
the merge step, and the no-allocation entry point (its counters cleared by
a kernel, not a memset)."""
from __future__ import annotations

import sys

import pytest
import torch

from gpu_helpers import GUARD, assert_close, run_gpu, split_workspace, to_device, workspace
from oracle.case_io import run_oracle
from workloads import make_custom_case

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _call(d, out, ws, noalloc, kv_splits):
    import paged_kv_prefill_varlen_amd as ppa
    ppa.batch_context_with_kv_cache(
        d["query"], d["kv_cache"], None if noalloc else ws, d["block_tables"], d["seq_lens"], d["max_q_len"],
        d["max_kv_len"], d["bmm1_scale"], d["bmm2_scale"], d["batch_size"], d["cum_seq_lens_q"],
        d["cum_seq_lens_kv"], window_left=d["window_left"], out=out, kv_layout=d["kv_layout"], sinks=d["sinks"],
        kv_splits=kv_splits, noalloc=noalloc)
    return out


def _fresh_out(d):
    return torch.empty_like(d["query"]).view(torch.int16).fill_(GUARD).view(torch.bfloat16)


@pytest.mark.parametrize("mode", ["workspace", "split2", "noalloc"])
def test_graph_replays_match_eager(mode):
    case = make_custom_case(name=f"graph_{mode}", batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                            page_size=16, q_lens=(90, 33, 150), prefix_lens=(60, 400, 0), window_left=300,
                            sinks=True, seed=4242)
    _say("graph", mode, case["q_lens"], case["kv_lens"])
    want, written = run_oracle(case)
    d = to_device(case)
    noalloc = mode == "noalloc"
    splits = 2 if mode == "split2" else 0
    ws = None if noalloc else (split_workspace(d, 2) if splits else workspace())
    q0 = d["query"].clone()
    q_static = d["query"].clone()
    dg = dict(d, query=q_static)
    out_g = _fresh_out(d)
    # eager warm-up on the capture's buffers (first-call set-up happens here)
    _call(dg, out_g, ws, noalloc, splits)
    torch.cuda.synchronize()
    assert_close(out_g, want, written, what=f"{mode} eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(dg, out_g, ws, noalloc, splits)
    torch.cuda.synchronize()
    for r in range(4):
        # eager work between replays: a new query in the captured buffer and
        # an eager call of the same entry point on another output
        q_static.copy_(q0 if r % 2 == 0 else (q0.float() * (0.5 + 0.25 * r)).to(q0.dtype))
        ref = _call(dict(d, query=q_static.clone()), _fresh_out(d), ws, noalloc, splits)
        torch.cuda.synchronize()
        out_g.view(torch.int16).fill_(GUARD)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), ref.view(torch.int16)), f"{mode}: replay {r} != eager"
        if r == 0:
            mx, mean = assert_close(out_g, want, written, what=f"{mode} replay")
            _say(f"  replay 0 against the oracle: max {mx:.2e} mean {mean:.2e}")
    if not noalloc and not splits:
        assert not ws.any(), "scheduler workspace not returned to zero"
    del g
