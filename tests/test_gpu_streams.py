"""GPU: calls on two streams at once, each with its own workspace, must give
the same bits as the same calls made one after the other (the workspace
entry point keeps no state outside the caller's workspace).  Both streams
run at the default priority."""
from __future__ import annotations

import sys

import pytest
import torch

from gpu_helpers import GUARD, to_device
from workloads import make_case, make_custom_case

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _call(d, ws, stream):
    import paged_kv_prefill_varlen_amd as ppa
    out = torch.empty_like(d["query"]).view(torch.int16).fill_(GUARD).view(torch.bfloat16)
    ppa.batch_context_with_kv_cache(
        d["query"], d["kv_cache"], ws, d["block_tables"], d["seq_lens"], d["max_q_len"], d["max_kv_len"],
        d["bmm1_scale"], d["bmm2_scale"], d["batch_size"], d["cum_seq_lens_q"], d["cum_seq_lens_kv"],
        window_left=d["window_left"], out=out, kv_layout=d["kv_layout"], sinks=d["sinks"], stream=stream)
    return out


def test_two_streams_with_own_workspaces():
    a = to_device(make_case("chunked"))
    b = to_device(make_custom_case(name="streams_b", batch=4, num_qo_heads=16, num_kv_heads=2, head_dim=64,
                                   page_size=8, q_lens=(300, 0, 41, 512), prefix_lens=(100, 7, 900, 0),
                                   window_left=127, sinks=True, seed=555))
    import paged_kv_prefill_varlen_amd as ppa
    ws_a, ws_b = (torch.zeros(ppa.WORKSPACE_BYTES, dtype=torch.uint8, device="cuda") for _ in range(2))
    ref_a = _call(a, ws_a, torch.cuda.current_stream())
    ref_b = _call(b, ws_b, torch.cuda.current_stream())
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        _say("two streams, repetition", rep)
        with torch.cuda.stream(s1):
            outs_a = [_call(a, ws_a, s1) for _ in range(3)]
        with torch.cuda.stream(s2):
            outs_b = [_call(b, ws_b, s2) for _ in range(3)]
        torch.cuda.synchronize()
        for o in outs_a:
            assert torch.equal(o.view(torch.int16), ref_a.view(torch.int16)), "stream 1 output differs"
        for o in outs_b:
            assert torch.equal(o.view(torch.int16), ref_b.view(torch.int16)), "stream 2 output differs"
    assert not ws_a.any() and not ws_b.any(), "a workspace was not returned to zero"
