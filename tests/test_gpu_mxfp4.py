"""GPU parity of the MXFP4 output (the API page's FP4 ``out`` with
``o_sf_scale`` / ``o_sf_vec_size``, carried out as OCP MXFP4).

* Rows whose attention output is exact in fp32 (window_left = 0 without a
  sink: each query sees one key, so o = bmm2_scale * v with bmm2_scale and
  o_sf_scale chosen exact) must give bit-identical codes and scale bytes:
  the kernel and the oracle then quantize the same fp32 values.  Also for
  the split-KV merge, and for the standalone merge with one part.
* Elsewhere the kernel's fp32 output differs from the oracle's fp64 one by
  the attention tolerance eps, so the check is the property every correct
  encoding has: each scale byte is the byte of some block maximum within
  eps of the oracle's, and each code is the nearest-even code, at the
  kernel's scale, of some value within eps of the oracle's element (the
  encoding is monotone, so the two ends of the interval bound it).
* Rows outside the requests keep their guard bytes.
"""
from __future__ import annotations

import sys
import zlib

import numpy as np
import pytest
import torch

from gpu_helpers import run_gpu, split_workspace, to_device
from oracle.case_io import run_oracle
from oracle.mxfp4 import E2M1_TABLE, encode_e2m1, mx_scale_byte, mxfp4_output, unpack_e2m1
from workloads import make_case, make_custom_case

pytestmark = pytest.mark.gpu

GUARD_DATA = 0xAB
GUARD_SF = 0xCD


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _mx_out(query, vec, g):
    import paged_kv_prefill_varlen_amd as ppa
    T, H, D = query.shape
    o = ppa.empty_mxfp4(T, H, D, "cuda", vec, g)
    o.data.fill_(GUARD_DATA)
    o.scale.fill_(GUARD_SF)
    return o


def _host(o):
    return o.data.cpu().numpy(), o.scale.cpu().numpy()


def _guards_kept(data, sf, written):
    return bool((data[~written] == GUARD_DATA).all() and (sf[~written] == GUARD_SF).all())


def _check_bracket(data, sf, want, written, vec, g, eps, what):
    """The property check described in the module docstring, over written rows."""
    codes = unpack_e2m1(data[written])                         # [n, H, D]
    sb = sf[written].astype(np.int64)                          # [n, H, D / vec]
    y = (want[written].astype(np.float32) * np.float32(g)).astype(np.float64)
    e = eps * g
    n, H, D = y.shape
    yb = y.reshape(n, H, D // vec, vec)
    amax = np.abs(yb).max(axis=-1)
    lo_b = mx_scale_byte(np.maximum(amax - e, 0).astype(np.float32)).astype(np.int64)
    hi_b = mx_scale_byte(np.nextafter((amax + e).astype(np.float32), np.float32(np.inf))).astype(np.int64)
    bad = (sb < lo_b) | (sb > hi_b)
    assert not bad.any(), f"{what}: {int(bad.sum())} scale bytes outside the bracket"
    scale = np.ldexp(1.0, (sb - 127).astype(np.int32))[..., None]
    lo_v = E2M1_TABLE[encode_e2m1((yb - e) / scale)]
    hi_v = E2M1_TABLE[encode_e2m1((yb + e) / scale)]
    got_v = E2M1_TABLE[codes.reshape(n, H, D // vec, vec)]
    bad = (got_v < lo_v) | (got_v > hi_v)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} codes outside the bracket"
    # and most codes are exactly the oracle's own encoding
    pw, sw = mxfp4_output(want[written], vec, g)
    same = float((unpack_e2m1(pw) == codes).mean())
    assert same > 0.9, f"{what}: only {same:.3f} of codes equal the oracle's"
    return same


def _exact_case(seed, **kw):
    base = dict(batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16, q_lens=(70, 1, 33),
                prefix_lens=(5, 40, 0), window_left=0, sinks=False, bmm1_scale=0.3, bmm2_scale=0.75, seed=seed,
                extra_tokens=3)
    base.update(kw)
    return make_custom_case(**base)


EXACT = {
    "d128_hnd": dict(),
    "d64_nhd_combined": dict(head_dim=64, kv_layout="NHD", kv_form="combined"),
    "d128_fp8": dict(kv_dtype="fp8_e4m3fn", page_size=64),
    "d64_g16": dict(head_dim=64, num_qo_heads=32, num_kv_heads=2, page_size=8),
}


@pytest.mark.parametrize("name", list(EXACT))
@pytest.mark.parametrize("vec", [16, 32])
def test_mxfp4_exact_rows_bitwise(name, vec):
    case = _exact_case(zlib.crc32(name.encode()) % 1000, **EXACT[name])
    want, written = run_oracle(case)
    d = to_device(case)
    for g in (1.0, 0.5, 3.0):
        for schedule in ("persistent", "grid"):
            _say("mxfp4 exact", name, vec, g, schedule)
            o = _mx_out(d["query"], vec, g)
            run_gpu(d, out=o, schedule=schedule)
            torch.cuda.synchronize()
            data, sf = _host(o)
            assert _guards_kept(data, sf, written), "rows outside the requests were written"
            pw, sw = mxfp4_output(want[written], vec, g)
            assert np.array_equal(sf[written], sw), f"scale bytes differ ({name}, vec {vec}, g {g})"
            assert np.array_equal(data[written], pw), f"codes differ ({name}, vec {vec}, g {g})"


@pytest.mark.parametrize("vec", [16, 32])
def test_mxfp4_exact_rows_split_kv_bitwise(vec):
    case = _exact_case(31, q_lens=(90, 20), prefix_lens=(300, 7), batch=2)
    want, written = run_oracle(case)
    d = to_device(case)
    for splits in (2, 5):
        _say("mxfp4 exact split", vec, splits)
        o = _mx_out(d["query"], vec, 2.0)
        run_gpu(d, out=o, kv_splits=splits, ws=split_workspace(d, splits))
        torch.cuda.synchronize()
        data, sf = _host(o)
        assert _guards_kept(data, sf, written)
        pw, sw = mxfp4_output(want[written], vec, 2.0)
        assert np.array_equal(sf[written], sw) and np.array_equal(data[written], pw), f"split {splits}"


GENERAL = {
    "g4_d128_prefix": dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                           q_lens=(300, 45), prefix_lens=(100, 0)),
    "g8_d64_window_sinks": dict(num_qo_heads=16, num_kv_heads=2, head_dim=64, page_size=16, kv_layout="NHD",
                                window_left=63, sinks=True, q_lens=(200, 37), prefix_lens=(80, 20)),
    "fp8_d128": dict(num_qo_heads=16, num_kv_heads=2, head_dim=128, page_size=64, kv_dtype="fp8_e4m3fn",
                     q_lens=(150,), prefix_lens=(600,)),
    "empty_requests": dict(num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                           q_lens=(0, 50, 0, 3), prefix_lens=(30, 0, 0, 0), extra_tokens=5),
}


@pytest.mark.parametrize("name", list(GENERAL))
@pytest.mark.parametrize("vec,g", [(32, 1.0), (16, 0.25)])
def test_mxfp4_general_parity(name, vec, g):
    spec = GENERAL[name]
    case = make_custom_case(name=name, batch=len(spec["q_lens"]), seed=zlib.crc32(name.encode()) % 10000, **spec)
    want, written = run_oracle(case)
    d = to_device(case)
    fp8 = case["kv_dtype"] != "bf16"
    eps = 6e-2 if fp8 else 2e-2
    for splits in (0, 3):
        _say("mxfp4 general", name, vec, g, "splits", splits)
        o = _mx_out(d["query"], vec, g)
        run_gpu(d, out=o, kv_splits=splits)
        torch.cuda.synchronize()
        data, sf = _host(o)
        assert _guards_kept(data, sf, written)
        same = _check_bracket(data, sf, want, written, vec, g, eps, f"{name} splits {splits}")
        _say(f"  codes equal to the oracle's: {same:.4f}")


def test_mxfp4_chunked_config():
    case = make_case("chunked")
    want, written = run_oracle(case)
    d = to_device(case)
    o = _mx_out(d["query"], 32, 1.0)
    run_gpu(d, out=o)
    torch.cuda.synchronize()
    data, sf = _host(o)
    assert _guards_kept(data, sf, written)
    same = _check_bracket(data, sf, want, written, 32, 1.0, 2e-2, "chunked")
    _say(f"chunked: codes equal to the oracle's {same:.4f}")


def test_mxfp4_infinite_block():
    """bmm2_scale = 2^127 overflows the outputs with |v| >= 2 to inf: their
    blocks get the NaN scale byte and zero codes, the others stay exact."""
    case = _exact_case(41, bmm2_scale=2.0 ** 127)
    want, written = run_oracle(case)
    d = to_device(case)
    o = _mx_out(d["query"], 32, 1.0)
    run_gpu(d, out=o)
    torch.cuda.synchronize()
    data, sf = _host(o)
    with np.errstate(over="ignore"):
        pw, sw = mxfp4_output(want[written], 32, 1.0)
    assert (sw == 255).any() and (sw != 255).any()
    assert np.array_equal(sf[written], sw) and np.array_equal(data[written], pw)


def test_mxfp4_subnormal_outputs():
    """Outputs below the smallest normal fp32 (bmm2_scale 2^-130) still
    encode exactly: scale byte 0 and codes of y * 2^127."""
    case = _exact_case(42, bmm2_scale=2.0 ** -130)
    want, written = run_oracle(case)
    d = to_device(case)
    o = _mx_out(d["query"], 32, 1.0)
    run_gpu(d, out=o)
    torch.cuda.synchronize()
    data, sf = _host(o)
    pw, sw = mxfp4_output(want[written], 32, 1.0)
    assert (sw == 0).all() and (pw != 0).any()
    assert np.array_equal(sf[written], sw) and np.array_equal(data[written], pw)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("vec", [16, 32])
def test_mxfp4_merge_entry_point(D, vec):
    import paged_kv_prefill_varlen_amd as ppa
    from oracle.paged_attention import merge_states
    rng = np.random.default_rng(78 + D + vec)
    rows, heads = 37, 4
    # one part with lse 0 and no sink: the merge output is the part itself, exactly
    o1 = (rng.standard_normal((1, rows, heads, D)) * 10.0 ** rng.uniform(-2, 2, (1, rows, heads, 1))).astype(
        np.float32)
    l1 = np.zeros((1, rows, heads), dtype=np.float32)
    out = ppa.empty_mxfp4(rows, heads, D, "cuda", vec, 0.5)
    ppa.ppa_merge_attention_states(torch.from_numpy(o1).cuda(), torch.from_numpy(l1).cuda(), out)
    torch.cuda.synchronize()
    data, sf = _host(out)
    pw, sw = mxfp4_output(o1[0], vec, 0.5)
    assert np.array_equal(sf, sw) and np.array_equal(data, pw)
    # several parts and a sink: property check against the oracle merge
    S = 4
    o = rng.standard_normal((S, rows, heads, D)).astype(np.float32)
    lse = (rng.standard_normal((S, rows, heads)) * 3).astype(np.float32)
    sinks = rng.standard_normal(heads).astype(np.float32)
    out = ppa.empty_mxfp4(rows, heads, D, "cuda", vec, 4.0)
    ppa.ppa_merge_attention_states(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(), out, None,
                                   torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    wo, _ = merge_states(o.astype(np.float64), lse.astype(np.float64), sinks[None, :].astype(np.float64))
    data, sf = _host(out)
    _check_bracket(data, sf, wo, np.ones(rows, dtype=bool), vec, 4.0, 1e-4, "merge")
