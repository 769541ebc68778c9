"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Every workload, the full-size ones included, is compared element by element
over every written row (max and mean over all of them); the full-size
workloads are also compared first on sampled rows that the oracle computes
one at a time, as a fast pre-check, plus properties that hold at any size
(no NaN, untouched guard rows).  Tolerances: bf16 output max |err| <= 2e-2
and mean |err| <= 2e-3; fp8 KV max |err| <= 6e-2.
"""
from __future__ import annotations

import math
import sys
import zlib

import numpy as np
import pytest
import torch

from gpu_helpers import (GUARD, assert_close, errors, guard_rows_untouched, lse_close, run_gpu, split_workspace,
                         to_device, workspace)
from oracle.case_io import decode_tensor, oracle_inputs, run_oracle, run_oracle_lse, run_oracle_rows
from workloads import make_case, make_custom_case
from workloads.cases import relayout, to_flat_page_table

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# --------------------------------------------------------------------------
# the address unit: paged K/V gathered on the GPU == the generator's tokens
# --------------------------------------------------------------------------

GATHER_CASES = [
    dict(kv_layout="HND", kv_form="split", page_size=16, head_dim=64),
    dict(kv_layout="NHD", kv_form="split", page_size=16, head_dim=64),
    dict(kv_layout="HND", kv_form="combined", page_size=32, head_dim=128),
    dict(kv_layout="NHD", kv_form="combined", page_size=1, head_dim=128),
    dict(kv_layout="NHD", kv_form="combined1", page_size=8, head_dim=64),
    dict(kv_layout="HND", kv_form="split", page_size=64, head_dim=128, kv_dtype="fp8_e4m3fn"),
    dict(kv_layout="NHD", kv_form="split", page_size=128, head_dim=64, kv_dtype="fp8_e4m3fn"),
]


@pytest.mark.parametrize("var", GATHER_CASES, ids=lambda v: "-".join(str(x) for x in v.values()))
def test_gather_bitwise(var):
    import paged_kv_prefill_varlen_amd as ppa
    case = make_custom_case(batch=3, num_qo_heads=4, num_kv_heads=2, q_lens=(40, 0, 130),
                            prefix_lens=(100, 7, 3), seed=11, **var)
    _say("gather", var)
    d = to_device(case)
    out = torch.empty_like(d["query"])
    p = ppa.make_params(d["query"], d["kv_cache"], None, d["block_tables"], d["seq_lens"],
                        d["max_q_len"], d["max_kv_len"], 1.0, 1.0, d["batch_size"],
                        d["cum_seq_lens_q"], d["cum_seq_lens_kv"], -1, out, d["kv_layout"], None)
    rows = sum(case["kv_lens"])
    for kv_idx, logical in ((0, case["logical_k"]), (1, case["logical_v"])):
        dst = torch.zeros((rows, case["num_kv_heads"], case["head_dim"]), dtype=case["cache_dtype"],
                          device="cuda")
        ppa.ppa_gather_paged_kv(p, kv_idx, dst)
        torch.cuda.synchronize()
        want = torch.cat(logical, dim=0)
        g = dst.cpu().view(torch.uint8).numpy()
        w = want.contiguous().view(torch.uint8).numpy()
        assert np.array_equal(g, w), f"gather mismatch plane {kv_idx}"


# --------------------------------------------------------------------------
# small and edge-case workloads, every row
# --------------------------------------------------------------------------

EDGE = {
    "mha_d128_p16": dict(num_qo_heads=2, num_kv_heads=2, head_dim=128, page_size=16,
                         q_lens=(300,), prefix_lens=(100,)),
    "g2_d64_nhd_combined": dict(num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=8,
                                kv_layout="NHD", kv_form="combined",
                                q_lens=(130, 1, 65), prefix_lens=(0, 70, 3)),
    "g3_combined1": dict(num_qo_heads=6, num_kv_heads=2, head_dim=128, page_size=32,
                         kv_form="combined1", q_lens=(200,), prefix_lens=(50,)),
    "g8_window0_sinks": dict(num_qo_heads=16, num_kv_heads=2, head_dim=64, page_size=16,
                             kv_layout="NHD", window_left=0, sinks=True,
                             q_lens=(100, 37), prefix_lens=(0, 20)),
    "g16_window63_sinks": dict(num_qo_heads=16, num_kv_heads=1, head_dim=128, page_size=64,
                               window_left=63, sinks=True, q_lens=(90,), prefix_lens=(200,)),
    "g32_two_head_groups": dict(num_qo_heads=64, num_kv_heads=2, head_dim=64, page_size=4,
                                q_lens=(20, 5), prefix_lens=(10, 0)),
    "empty_requests": dict(num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                           q_lens=(0, 50, 0, 3), prefix_lens=(30, 0, 0, 0), extra_tokens=5),
    "page_size_1": dict(num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=1,
                        q_lens=(70,), prefix_lens=(10,)),
    "g128_mqa_eight_head_groups": dict(num_qo_heads=128, num_kv_heads=1, head_dim=128, page_size=32,
                                       q_lens=(90, 17), prefix_lens=(150, 300)),
    "batch_300_short": dict(num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                            q_lens=tuple((7 * i) % 13 for i in range(300)),
                            prefix_lens=tuple((11 * i) % 41 for i in range(300))),
    "page_size_65536": dict(num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=65536, kv_layout="NHD",
                            q_lens=(300, 50), prefix_lens=(2000, 0), spare_pages=1),
    "page_size_128": dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=128,
                          q_lens=(129,), prefix_lens=(300,)),
    "single_token": dict(num_qo_heads=4, num_kv_heads=4, head_dim=128, page_size=16,
                         q_lens=(1,), prefix_lens=(0,)),
    "bounds_loose": dict(num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                         q_lens=(33, 64), prefix_lens=(5, 64), max_q_len=500, max_kv_len=900),
    "long_prefix": dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=32,
                        q_lens=(1000,), prefix_lens=(3000,)),
    "window_many_tiles": dict(num_qo_heads=8, num_kv_heads=1, head_dim=64, page_size=16,
                              window_left=200, sinks=True, q_lens=(700,), prefix_lens=(500,)),
    "nan_poison": dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                       poison="nan", q_lens=(77, 150), prefix_lens=(19, 0)),
    "neg_bmm1": dict(num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                     bmm1_scale=-0.2, bmm2_scale=0.5, q_lens=(90,), prefix_lens=(40,)),
    "zero_bmm1": dict(num_qo_heads=4, num_kv_heads=2, head_dim=128, page_size=16,
                      bmm1_scale=0.0, q_lens=(90,), prefix_lens=(40,), window_left=20),
    "fp8_d128": dict(num_qo_heads=16, num_kv_heads=2, head_dim=128, page_size=64,
                     kv_dtype="fp8_e4m3fn", q_lens=(150,), prefix_lens=(600,)),
    "fp8_d64_nhd_window_sinks": dict(num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                                     kv_layout="NHD", kv_dtype="fp8_e4m3fn", window_left=31,
                                     sinks=True, q_lens=(77, 33), prefix_lens=(10, 200)),
    "fp8_nan_poison": dict(num_qo_heads=8, num_kv_heads=1, head_dim=128, page_size=16,
                           kv_dtype="fp8_e4m3fn", poison="nan", q_lens=(65,), prefix_lens=(63,)),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_case_parity(name):
    case = make_custom_case(name=name, batch=len(EDGE[name]["q_lens"]), seed=zlib.crc32(name.encode()) % 10000,
                            **EDGE[name])
    _say("edge", name, case["q_lens"], case["kv_lens"])
    want, written = run_oracle(case)
    d = to_device(case)
    out = run_gpu(d)
    grid_out = run_gpu(d, schedule="grid")
    torch.cuda.synchronize()
    assert guard_rows_untouched(out, written), "rows outside the requests were written"
    mx, mean = assert_close(out, want, written, fp8=case["kv_dtype"] != "bf16", what=name)
    _say(f"  max {mx:.2e} mean {mean:.2e}")
    # both schedules run the same per-item arithmetic: identical bits
    assert torch.equal(out.view(torch.int16), grid_out.view(torch.int16)), "persistent != grid schedule"
    assert not workspace().any(), "scheduler workspace not returned to zero"


# Pools larger than 4 GiB: the used pages copied to the top of the pool, so
# that every page the kernels read starts past byte 2^32 of its plane.
POOL_4G_CASES = {
    "hnd_combined_bf16_d128": dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16, kv_layout="HND",
                                   kv_form="combined", q_lens=(150, 70), prefix_lens=(200, 0)),
    "nhd_split_fp8_d128": dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=32, kv_layout="NHD",
                               kv_form="split", kv_dtype="fp8_e4m3fn", q_lens=(300, 40), prefix_lens=(100, 500)),
    "nhd_split_bf16_d64_window": dict(num_qo_heads=16, num_kv_heads=2, head_dim=64, page_size=8, kv_layout="NHD",
                                      kv_form="split", window_left=90, sinks=True, q_lens=(200,),
                                      prefix_lens=(150,)),
}


def _pool_above_4gib(pool: torch.Tensor):
    """A pool of more than 4 GiB whose top pages hold `pool`'s pages; returns
    it and the page-id offset of the copy."""
    page_bytes = pool[0].numel() * pool.element_size()
    off = (1 << 32) // page_bytes + 7
    big = torch.empty((off + pool.shape[0],) + tuple(pool.shape[1:]), dtype=pool.dtype, device=pool.device)
    big[off:] = pool
    return big, off


@pytest.mark.parametrize("name", sorted(POOL_4G_CASES))
def test_pages_beyond_4gib(name):
    """Page ids whose byte offsets lie past 4 GiB of the pool (page addresses
    are formed in 64 bits): the output equals, bit for bit, that of the same
    pages at the bottom of a small pool, and the oracle's within tolerance.
    The fp8 cache at head_dim 128 is also run on the fp8 MFMA."""
    spec = POOL_4G_CASES[name]
    case = make_custom_case(name=name, batch=len(spec["q_lens"]), seed=zlib.crc32(name.encode()) % 10000, **spec)
    _say("pool > 4 GiB", name, case["q_lens"], case["kv_lens"])
    want, written = run_oracle(case)
    d = to_device(case)
    kv = d["kv_cache"]
    if isinstance(kv, tuple):
        (bk, off), (bv, off_v) = _pool_above_4gib(kv[0]), _pool_above_4gib(kv[1])
        assert off == off_v
        big_kv = (bk, bv)
    else:
        big_kv, off = _pool_above_4gib(kv)
    big = dict(d, kv_cache=big_kv, block_tables=d["block_tables"] + off)
    fp8_mma = [False, True] if case["kv_dtype"] != "bf16" and case["head_dim"] == 128 else [False]
    for f8 in fp8_mma:
        small_out = run_gpu(d, fp8_compute=f8)
        out = run_gpu(big, fp8_compute=f8)
        torch.cuda.synchronize()
        assert guard_rows_untouched(out, written), "rows outside the requests were written"
        assert torch.equal(out.view(torch.int16), small_out.view(torch.int16)), "pool offset changed the output"
        if not f8:
            mx, mean = assert_close(out, want, written, fp8=case["kv_dtype"] != "bf16", what=name)
            _say(f"  max {mx:.2e} mean {mean:.2e}")
    assert not workspace().any(), "scheduler workspace not returned to zero"
    del big, big_kv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_strided_query_output_and_table(layout):
    """Q as a view into a fused QKV buffer (token stride (Hq + 2 Hkv) D), the
    output as a view with a padded head stride, the block table as a column
    slice of a wider table: the same bits as the dense tensors, the padding
    untouched, and the oracle's output within tolerance."""
    name = f"strided_{layout}"
    case = make_custom_case(name=name, batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                            kv_layout=layout, q_lens=(70, 0, 131), prefix_lens=(40, 9, 200),
                            seed=zlib.crc32(name.encode()) % 10000)
    _say("strided views", name, case["q_lens"], case["kv_lens"])
    want, written = run_oracle(case)
    d = to_device(case)
    q = d["query"]
    T, Hq, D = q.shape
    Hkv = case["num_kv_heads"]
    qkv = torch.randn((T, Hq + 2 * Hkv, D), device=q.device).to(q.dtype)
    qkv[:, :Hq] = q
    q_view = qkv[:, :Hq]
    out_buf = torch.full((T, Hq, D + 8), GUARD, dtype=torch.int16, device=q.device)
    out_view = out_buf[:, :, :D].view(torch.bfloat16)
    bt = d["block_tables"]
    bt_wide = torch.full((bt.shape[0], bt.shape[1] + 3), 1 << 30, dtype=bt.dtype, device=bt.device)
    bt_wide[:, :bt.shape[1]] = bt
    bt_view = bt_wide[:, :bt.shape[1]]
    assert not q_view.is_contiguous() and not out_view.is_contiguous() and not bt_view.is_contiguous()
    dense = run_gpu(d)
    strided = run_gpu(dict(d, query=q_view, block_tables=bt_view), out=out_view)
    torch.cuda.synchronize()
    dense_raw = dense.view(torch.int16)
    assert torch.equal(out_buf[:, :, :D], dense_raw), "strided views changed the output"
    assert bool((out_buf[:, :, D:] == GUARD).all()), "the output's head padding was written"
    mx, mean = assert_close(dense, want, written, what=name)
    _say(f"  max {mx:.2e} mean {mean:.2e}")


def test_tiny_config_full():
    case = make_case("tiny")
    want, written = run_oracle(case)
    out = run_gpu(to_device(case))
    torch.cuda.synchronize()
    assert guard_rows_untouched(out, written)
    assert_close(out, want, written, what="tiny")


def test_chunked_config_full():
    case = make_case("chunked")
    _say("chunked", case["q_lens"], case["kv_lens"])
    want, written = run_oracle(case)
    d = to_device(case)
    out = run_gpu(d)
    grid_out = run_gpu(d, schedule="grid")
    torch.cuda.synchronize()
    assert guard_rows_untouched(out, written)
    mx, mean = assert_close(out, want, written, what="chunked")
    _say(f"  max {mx:.2e} mean {mean:.2e}")
    assert torch.equal(out.view(torch.int16), grid_out.view(torch.int16))


def _sample_rows(case, n_random=96, seed=0):
    rng = np.random.default_rng(seed)
    cu = case["cum_seq_lens_q"].numpy()
    Hq = case["num_qo_heads"]
    rows = []
    for b in range(case["batch_size"]):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        if q1 == q0:
            continue
        for t in {q0, q1 - 1, q0 + (q1 - q0) // 2, min(q1 - 1, q0 + 63), min(q1 - 1, q0 + 64)}:
            rows.append((t, int(rng.integers(Hq))))
    tot = int(cu[-1])
    for _ in range(n_random):
        rows.append((int(rng.integers(tot)), int(rng.integers(Hq))))
    return rows


@pytest.mark.parametrize("name", ["llama3_8b", "swa_sinks", "fp8_long_prefix"])
def test_full_size_config_sampled(name):
    case = make_case(name)
    _say("full", name, "tokens", sum(case["q_lens"]))
    d = to_device(case)
    out = run_gpu(d)
    grid_out = run_gpu(d, schedule="grid")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), grid_out.view(torch.int16)), "persistent != grid schedule"
    written = np.zeros(case["num_tokens"], dtype=bool)
    written[:int(case["cum_seq_lens_q"][-1])] = True
    assert guard_rows_untouched(out, written)
    o = out.float()
    assert not torch.isnan(o[:int(written.sum())]).any(), "NaN in output"
    rows = _sample_rows(case)
    want = run_oracle_rows(case, rows)
    got = decode_tensor(out.cpu())
    g = np.stack([got[t, h] for t, h in rows])
    err = np.abs(g - want)
    tol = 6e-2 if case["kv_dtype"] != "bf16" else 2e-2
    _say(f"  sampled max {err.max():.2e} mean {err.mean():.2e}")
    assert err.max() <= tol
    if case["kv_dtype"] == "bf16":
        assert err.mean() <= 2e-3


def oracle_by_kv_head(case):
    """The oracle's output for a whole workload, computed one (request, kv
    head) at a time with the oracle's own gather and per-request attention,
    printing a line after each request so a long run shows its progress."""
    import oracle.paged_attention as OA
    a = oracle_inputs(case)
    q, cu, sl = a["query"], a["cum_seq_lens_q"], a["seq_lens"]
    Hq = q.shape[1]
    Hkv = case["num_kv_heads"]
    G = Hq // Hkv
    out = np.full(q.shape, np.nan)
    written = np.zeros(q.shape[0], dtype=bool)
    for b in range(len(sl)):
        q0, q1, kv_len = int(cu[b]), int(cu[b + 1]), int(sl[b])
        if q1 == q0:
            continue
        pages = OA.request_pages(b, a["block_tables"], a["kv_indptr"], a["kv_indices"])
        k = OA.gather_paged_kv(a["kv_cache"], pages, 0, kv_len, a["page_size"], a["kv_layout"])
        v = OA.gather_paged_kv(a["kv_cache"], pages, 1, kv_len, a["page_size"], a["kv_layout"])
        for hk in range(Hkv):
            heads = slice(hk * G, (hk + 1) * G)
            sinks = None if a["sinks"] is None else a["sinks"][heads]
            out[q0:q1, heads] = OA.attention_one_request(q[q0:q1, heads], k[:, hk:hk + 1], v[:, hk:hk + 1],
                                                         a["bmm1_scale"], a["bmm2_scale"], a["window_left"], sinks)
        written[q0:q1] = True
        _say(f"  oracle: request {b + 1}/{len(sl)} ({q1 - q0} rows over {kv_len} keys)")
    return out, written


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["llama3_8b", "swa_sinks", "fp8_long_prefix"])
def test_full_size_config_full(name):
    """Every written element of the full-size workload against the oracle,
    in the launch configuration the bench times (persistent schedule); the
    long-prefix fp8 workload in both arithmetics (widened bf16, the default,
    and fp8 MFMA, the bench setting)."""
    case = make_case(name)
    _say("full, every element:", name, "tokens", sum(case["q_lens"]))
    d = to_device(case)
    fp8 = case["kv_dtype"] != "bf16"
    outs = {"default": run_gpu(d)}
    if fp8:
        outs["fp8_compute"] = run_gpu(d, fp8_compute=True)
    torch.cuda.synchronize()
    want, written = oracle_by_kv_head(case)
    for what, out in outs.items():
        assert guard_rows_untouched(out, written)
        mx, mean = assert_close(out, want, written, fp8=fp8, what=f"{name} {what}")
        _say(f"  {name} {what}: max {mx:.2e} mean {mean:.2e} over {int(written.sum()) * case['num_qo_heads']} rows")


def test_sink_far_above_the_logits():
    """Sinks 100 above every logit: the denominator is dominated by the sink,
    the output tends to 0 and the log-denominator to the sink; both stay
    finite, unsplit and split."""
    case = make_custom_case(name="big_sink", batch=2, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                            q_lens=(70, 33), prefix_lens=(20, 300), sinks=True, seed=612)
    case["sinks"] = case["sinks"] + 100.0
    want, written = run_oracle(case)
    want_lse = run_oracle_lse(case)
    d = to_device(case)
    for splits in (0, 3):
        lse = torch.full(tuple(d["query"].shape[:2]), float("nan"), dtype=torch.float32, device="cuda")
        out = run_gpu(d, lse=lse, kv_splits=splits)
        torch.cuda.synchronize()
        mx, mean = assert_close(out, want, written, what=f"big sink S={splits}")
        err = lse_close(lse, want_lse, written, f"big sink S={splits}")
        _say(f"  big sink S={splits}: max {mx:.2e} lse err {err:.2e}")


# --------------------------------------------------------------------------
# invariances: bit-identical outputs
# --------------------------------------------------------------------------

def _base_case():
    return make_custom_case(name="inv", batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                            page_size=16, q_lens=(100, 7, 260), prefix_lens=(30, 200, 0),
                            sinks=True, window_left=150, seed=77)


def test_relayout_bitwise():
    case = _base_case()
    base = run_gpu(to_device(case)).cpu()
    for lay, form, P, seed in (("NHD", "split", 16, 1), ("HND", "combined", 32, 2),
                               ("NHD", "combined", 4, 3), ("HND", "split", 64, 4)):
        other = relayout(case, kv_layout=lay, kv_form=form, page_size=P, permute_seed=seed)
        got = run_gpu(to_device(other)).cpu()
        assert torch.equal(base.view(torch.int16), got.view(torch.int16)), (lay, form, P)


def test_poison_bitwise_and_determinism():
    a = _base_case()
    b = make_custom_case(**{**a["spec"].__dict__, "poison": "nan"})
    ra = run_gpu(to_device(a)).cpu()
    ra2 = run_gpu(to_device(a)).cpu()
    rb = run_gpu(to_device(b)).cpu()
    assert torch.equal(ra.view(torch.int16), ra2.view(torch.int16)), "two launches differ"
    assert torch.equal(ra.view(torch.int16), rb.view(torch.int16)), "poisoned pages leaked"


def test_full_window_and_neg_inf_sink_bitwise():
    case = _base_case()
    d = to_device(case)
    d_nowin = dict(d, window_left=-1)
    d_bigwin = dict(d, window_left=max(case["kv_lens"]) + 5)
    a = run_gpu(d_nowin).cpu()
    b = run_gpu(d_bigwin).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    d_nosink = dict(d, sinks=None)
    d_infsink = dict(d, sinks=torch.full_like(d["sinks"], -math.inf))
    c = run_gpu(d_nosink).cpu()
    e = run_gpu(d_infsink).cpu()
    assert torch.equal(c.view(torch.int16), e.view(torch.int16))


def test_device_tensor_scales():
    case = _base_case()
    d = to_device(case)
    a = run_gpu(d).cpu()
    b1 = torch.tensor([d["bmm1_scale"]], dtype=torch.float32, device="cuda")
    b2 = torch.tensor([d["bmm2_scale"]], dtype=torch.float32, device="cuda")
    b = run_gpu(d, bmm1=b1, bmm2=b2).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_rejects_bad_metadata_without_launch():
    import paged_kv_prefill_varlen_amd as ppa
    case = _base_case()
    d = to_device(case)
    bad = d["seq_lens"].clone()
    bad[1] = 3  # q_len 7 > kv_len 3
    with pytest.raises(ppa.PpaError):
        run_gpu(dict(d, seq_lens=bad), validate=True)


# --------------------------------------------------------------------------
# the persistent schedule's workspace
# --------------------------------------------------------------------------

def test_schedule_back_to_back_and_workspace_reset():
    """Calls of different sizes, back to back on one stream, sharing one
    workspace: every call sees zeroed counters (the previous call's last
    workgroup reset them), so every call covers all of its work items."""
    cases = [make_custom_case(name="bb%d" % i, batch=b, num_qo_heads=hq, num_kv_heads=hk, head_dim=d,
                              page_size=ps, q_lens=ql, prefix_lens=pl, seed=500 + i)
             for i, (b, hq, hk, d, ps, ql, pl) in enumerate([
                 (3, 32, 8, 128, 32, (700, 64, 300), (100, 0, 900)),    # 8 queues
                 (1, 6, 2, 64, 16, (90,), (10,)),                        # 1 queue, few items
                 (5, 16, 4, 128, 64, (1, 2, 3, 4, 900), (0, 5, 60, 0, 7)),
                 (2, 64, 8, 64, 16, (2000, 17), (0, 3000)),
             ])]
    ws = workspace()
    assert not ws.any()
    wants = [run_oracle(c) for c in cases]
    devs = [to_device(c) for c in cases]
    for rep in range(2):
        outs = [run_gpu(d, validate=False) for d in devs]   # no sync between calls
        torch.cuda.synchronize()
        for c, (want, written), out in zip(cases, wants, outs):
            assert guard_rows_untouched(out, written)
            assert_close(out, want, written, what=c["name"] if "name" in c else "bb")
        assert not ws.any(), "workspace not zero after the calls"


def test_rejects_small_or_misaligned_workspace():
    import paged_kv_prefill_varlen_amd as ppa
    case = make_case("tiny")
    d = to_device(case)
    out = torch.empty_like(d["query"])
    for ws in (torch.zeros(8, dtype=torch.uint8, device="cuda"),
               torch.zeros(ppa.WORKSPACE_BYTES + 16, dtype=torch.uint8, device="cuda")[4:]):
        p = ppa.make_params(d["query"], d["kv_cache"], ws, d["block_tables"], d["seq_lens"], d["max_q_len"],
                            d["max_kv_len"], d["bmm1_scale"], d["bmm2_scale"], d["batch_size"],
                            d["cum_seq_lens_q"], d["cum_seq_lens_kv"], -1, out, d["kv_layout"], None)
        with pytest.raises(ppa.PpaError):
            ppa.ppa_paged_prefill_attention(p)


# --------------------------------------------------------------------------
# the flat (CSR) page table: the same pages as the padded table
# --------------------------------------------------------------------------

FLAT_CASES = {
    "hnd_p16_d128": dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         q_lens=(100, 0, 260), prefix_lens=(30, 9, 0)),
    "nhd_p4_d64_window_sinks": dict(num_qo_heads=16, num_kv_heads=2, head_dim=64, page_size=4,
                                    kv_layout="NHD", window_left=40, sinks=True,
                                    q_lens=(70, 33), prefix_lens=(10, 90)),
    "combined_p64_fp8": dict(num_qo_heads=16, num_kv_heads=2, head_dim=128, page_size=64,
                             kv_form="combined", kv_dtype="fp8_e4m3fn", q_lens=(150,), prefix_lens=(300,)),
    "empty_and_ragged": dict(num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                             q_lens=(0, 50, 0, 3), prefix_lens=(0, 0, 7, 0), extra_tokens=3),
}


@pytest.mark.parametrize("name", list(FLAT_CASES))
@pytest.mark.parametrize("slack,lead", [(0, 0), (3, 5)])
def test_flat_page_table_bitwise(name, slack, lead):
    case = make_custom_case(name=name, batch=len(FLAT_CASES[name]["q_lens"]),
                            seed=zlib.crc32(name.encode()) % 10000, **FLAT_CASES[name])
    flat = to_flat_page_table(case, slack=slack, lead=lead, seed=9)
    _say("flat", name, slack, lead)
    want, written = run_oracle(flat)
    padded = run_gpu(to_device(case))
    d = to_device(flat)
    got = run_gpu(d)
    got_grid = run_gpu(d, schedule="grid")
    torch.cuda.synchronize()
    assert guard_rows_untouched(got, written)
    assert torch.equal(got.view(torch.int16), padded.view(torch.int16)), "flat != padded table"
    assert torch.equal(got_grid.view(torch.int16), padded.view(torch.int16))
    assert_close(got, want, written, fp8=case["kv_dtype"] != "bf16", what=name)


def test_flat_page_table_gather():
    import paged_kv_prefill_varlen_amd as ppa
    case = make_custom_case(batch=3, num_qo_heads=4, num_kv_heads=2, q_lens=(40, 0, 130),
                            prefix_lens=(100, 7, 3), seed=12, page_size=8, head_dim=64, kv_layout="NHD")
    flat = to_flat_page_table(case, slack=2, lead=4, seed=3)
    d = to_device(flat)
    out = torch.empty_like(d["query"])
    p = ppa.make_params(d["query"], d["kv_cache"], None, None, d["seq_lens"], d["max_q_len"], d["max_kv_len"],
                        1.0, 1.0, d["batch_size"], d["cum_seq_lens_q"], d["cum_seq_lens_kv"], -1, out,
                        d["kv_layout"], None, d["kv_indptr"], d["kv_indices"], None)
    rows = sum(case["kv_lens"])
    for kv_idx, logical in ((0, case["logical_k"]), (1, case["logical_v"])):
        dst = torch.zeros((rows, case["num_kv_heads"], case["head_dim"]), dtype=case["cache_dtype"], device="cuda")
        ppa.ppa_gather_paged_kv(p, kv_idx, dst)
        torch.cuda.synchronize()
        want = torch.cat(logical, dim=0)
        assert torch.equal(dst.cpu().view(torch.uint8), want.contiguous().view(torch.uint8))


# --------------------------------------------------------------------------
# log-sum-exp output, split-KV and the merge of partial states
# --------------------------------------------------------------------------

LSE_CASES = ["g2_d64_nhd_combined", "g8_window0_sinks", "g16_window63_sinks", "empty_requests",
             "long_prefix", "window_many_tiles", "neg_bmm1", "zero_bmm1", "fp8_d64_nhd_window_sinks"]


def _edge(name):
    return make_custom_case(name=name, batch=len(EDGE[name]["q_lens"]), seed=zlib.crc32(name.encode()) % 10000,
                            **EDGE[name])


@pytest.mark.parametrize("name", LSE_CASES)
def test_lse_output(name):
    case = _edge(name)
    want, written = run_oracle(case)
    want_lse = run_oracle_lse(case)
    d = to_device(case)
    lse = torch.full(tuple(d["query"].shape[:2]), float("nan"), dtype=torch.float32, device="cuda")
    out = run_gpu(d, lse=lse)
    plain = run_gpu(d)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16)), "lse output changed the output"
    err = lse_close(lse, want_lse, written, name)
    assert torch.isnan(lse.cpu()[~torch.from_numpy(written)]).all(), "lse written outside the requests"
    _say(f"  {name}: lse max err {err:.2e}")


SPLIT_CASES = ["mha_d128_p16", "g8_window0_sinks", "g16_window63_sinks", "empty_requests", "long_prefix",
               "window_many_tiles", "fp8_d128", "page_size_1", "single_token"]


@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("name", SPLIT_CASES)
def test_split_kv(name, splits):
    case = _edge(name)
    want, written = run_oracle(case)
    want_lse = run_oracle_lse(case)
    d = to_device(case)
    lse = torch.full(tuple(d["query"].shape[:2]), float("nan"), dtype=torch.float32, device="cuda")
    ws = None
    out = run_gpu(d, lse=lse, kv_splits=splits)
    torch.cuda.synchronize()
    assert guard_rows_untouched(out, written)
    mx, mean = assert_close(out, want, written, fp8=case["kv_dtype"] != "bf16", what=f"{name} S={splits}")
    err = lse_close(lse, want_lse, written, f"{name} S={splits}")
    _say(f"  {name} S={splits}: max {mx:.2e} mean {mean:.2e} lse {err:.2e}")


def test_split_kv_chunked_config():
    case = make_case("chunked")
    want, written = run_oracle(case)
    d = to_device(case)
    for splits in (2, 4):
        out = run_gpu(d, kv_splits=splits)
        torch.cuda.synchronize()
        assert guard_rows_untouched(out, written)
        mx, mean = assert_close(out, want, written, what=f"chunked S={splits}")
        _say(f"  chunked S={splits}: max {mx:.2e} mean {mean:.2e}")


def test_split_kv_workspace_reused_and_zeroed():
    """Split calls of different sizes share one (large enough) workspace; the
    scheduler counters at its start return to zero after each call."""
    import paged_kv_prefill_varlen_amd as ppa
    a, b = _edge("long_prefix"), _edge("g2_d64_nhd_combined")
    da, db = to_device(a), to_device(b)
    ws = split_workspace(da, 5)
    wa, wra = run_oracle(a)
    wb, wrb = run_oracle(b)
    for _ in range(2):
        oa = run_gpu(da, kv_splits=5, ws=ws, validate=False)
        ob = run_gpu(db, kv_splits=3, ws=ws, validate=False)
        torch.cuda.synchronize()
        assert_close(oa, wa, wra, what="long_prefix S=5")
        assert_close(ob, wb, wrb, what="g2 S=3")
        assert not ws[:ppa.WORKSPACE_BYTES].any()


def test_merge_entry_point():
    import paged_kv_prefill_varlen_amd as ppa
    from oracle.paged_attention import merge_states
    rng = np.random.default_rng(77)
    for S, rows, heads, D in ((1, 5, 3, 64), (4, 33, 8, 128), (9, 7, 2, 64)):
        o = rng.standard_normal((S, rows, heads, D)).astype(np.float32)
        lse = (rng.standard_normal((S, rows, heads)) * 3).astype(np.float32)
        lse[0, 0, :] = -np.inf   # empty parts
        if S > 1:
            lse[:, 1, 0] = -np.inf   # a row with no keys in any part
        sinks = rng.standard_normal(heads).astype(np.float32)
        for with_sink in (False, True):
            out = torch.empty((rows, heads, D), dtype=torch.bfloat16, device="cuda")
            lse_out = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
            ppa.ppa_merge_attention_states(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(), out, lse_out,
                                           torch.from_numpy(sinks).cuda() if with_sink else None)
            torch.cuda.synchronize()
            wo, wl = merge_states(o.astype(np.float64), lse.astype(np.float64),
                                  sinks[None, :].astype(np.float64) if with_sink else None)
            got = decode_tensor(out.cpu())
            assert np.abs(got - wo).max() <= 1e-2 * max(1.0, np.abs(wo).max())
            gl = lse_out.cpu().numpy()
            fin = np.isfinite(wl)
            assert np.array_equal(np.isfinite(gl), fin)
            assert np.abs(gl[fin] - wl[fin]).max() < 1e-4


@pytest.mark.parametrize("splits", [0, 8, 32])
def test_decode_config(splits):
    """The decode-shaped batch (one new token per request over an 8K prefix),
    whole output and lse against the oracle, with and without split-KV."""
    case = make_case("decode")
    want, written = run_oracle(case)
    want_lse = run_oracle_lse(case)
    d = to_device(case)
    lse = torch.full(tuple(d["query"].shape[:2]), float("nan"), dtype=torch.float32, device="cuda")
    out = run_gpu(d, lse=lse, kv_splits=splits)
    torch.cuda.synchronize()
    mx, mean = assert_close(out, want, written, what=f"decode S={splits}")
    err = lse_close(lse, want_lse, written, f"decode S={splits}")
    _say(f"  decode S={splits}: max {mx:.2e} mean {mean:.2e} lse {err:.2e}")


def _planned(d, ws):
    import paged_kv_prefill_varlen_amd as ppa
    out = torch.empty_like(d["query"])
    p = ppa.make_params(d["query"], d["kv_cache"], ws, d["block_tables"], d["seq_lens"], d["max_q_len"],
                        d["max_kv_len"], d["bmm1_scale"], d["bmm2_scale"], d["batch_size"], d["cum_seq_lens_q"],
                        d["cum_seq_lens_kv"], d["window_left"], out, d["kv_layout"], d["sinks"])
    return ppa.ppa_plan_kv_splits(p)


def test_planned_kv_splits():
    """kv_splits="auto": the planner splits the decode-shaped batch (128 work
    items for the device's resident workgroups) and the result is the oracle's
    and bitwise the explicit call with the same count; prefill shapes, which
    already fill the device, stay whole; a workspace with no room for partial
    state gives no split."""
    case = make_case("decode")
    want, written = run_oracle(case)
    d = to_device(case)
    ws = split_workspace(d, 64)
    s = _planned(d, ws)
    _say(f"  planned kv_splits for decode: {s}")
    assert 1 < s <= 64
    auto = run_gpu(d, kv_splits="auto", ws=ws)
    torch.cuda.synchronize()
    assert_close(auto, want, written, what="decode auto")
    explicit = run_gpu(d, kv_splits=s, ws=split_workspace(d, s))
    torch.cuda.synchronize()
    assert torch.equal(auto.view(torch.int16), explicit.view(torch.int16))
    assert _planned(d, split_workspace(d, 1)) == 1
    for name in ("chunked", "swa_sinks"):
        dc = to_device(make_case(name))
        assert _planned(dc, split_workspace(dc, 4)) == 1, name


@pytest.mark.parametrize("name", ["long_prefix", "window_many_tiles", "nan_poison", "fp8_d128",
                                  "fp8_d64_nhd_window_sinks", "single_token", "bounds_loose"])
def test_edge_case_planned_splits(name):
    """kv_splits="auto" on the edge cases: these small batches leave most of
    the device idle, so the planner splits wherever the keys allow it; the
    result must match the oracle whatever count it picks."""
    case = make_custom_case(name=name, batch=len(EDGE[name]["q_lens"]), seed=zlib.crc32(name.encode()) % 10000,
                            **EDGE[name])
    want, written = run_oracle(case)
    d = to_device(case)
    ws = split_workspace(d, 64)
    s = _planned(d, ws)
    _say("edge planned", name, "kv_splits", s)
    out = run_gpu(d, kv_splits="auto", ws=ws)
    torch.cuda.synchronize()
    assert guard_rows_untouched(out, written), "rows outside the requests were written"
    mx, mean = assert_close(out, want, written, fp8=case["kv_dtype"] != "bf16", what=f"{name} auto S={s}")
    _say(f"  max {mx:.2e} mean {mean:.2e}")
