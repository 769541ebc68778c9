"""GPU: new tokens written into the paged cache (ppa_append_paged_kv) must
leave exactly the bytes the CPU oracle's append leaves (bit-exact: it is
byte work, and the fp8 codes are integers decided from the same fp32
quotient on both sides), and attention over the appended cache must match
the oracle.  Slots come from the generator's page tables (token i of request
b at position prefix_b + i), with skipped (-1) and out-of-pool entries."""
from __future__ import annotations

import sys
import zlib

import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, guard_rows_untouched, run_gpu, to_device
from oracle.case_io import run_oracle
from oracle.paged_attention import append_paged_kv
from workloads import make_custom_case
from workloads.cases import as_codes

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _slots(case):
    P = case["page_size"]
    bt = case["block_tables"].numpy()
    out = []
    for b, (q, kv) in enumerate(zip(case["q_lens"], case["kv_lens"])):
        for i in range(q):
            pos = kv - q + i
            out.append(int(bt[b, pos // P]) * P + pos % P)
    return np.array(out, dtype=np.int64)


def _planes_codes(kv_cache):
    if isinstance(kv_cache, (tuple, list)):
        return [as_codes(kv_cache[0]), as_codes(kv_cache[1])]
    return [as_codes(kv_cache[:, 0]), as_codes(kv_cache[:, 1])]


VARIANTS = {
    "bf16_hnd_split_d128_p16": dict(kv_layout="HND", kv_form="split", head_dim=128, page_size=16),
    "bf16_nhd_combined_d64_p8": dict(kv_layout="NHD", kv_form="combined", head_dim=64, page_size=8),
    "fp8_hnd_split_d128_p64": dict(kv_layout="HND", kv_form="split", head_dim=128, page_size=64,
                                   kv_dtype="fp8_e4m3fn"),
    "fp8_nhd_combined_d64_p1": dict(kv_layout="NHD", kv_form="combined", head_dim=64, page_size=1,
                                    kv_dtype="fp8_e4m3fn"),
}


def _new_values(n, hkv, d, seed, crafted):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((n, hkv, d), generator=g) * 3.0)
    if crafted:
        # exact midpoints of the e4m3fn grid (ties), saturation and specials
        mids = torch.tensor([1.0625, 1.1875, -1.3125, 17.0, 0.001953125 * 1.5, 240.0, -416.0, 464.0, 500.0,
                             1.0e4, -3.0e5, 0.0, -0.0, float("nan"), 2.0 ** -12])
        flat = x.view(-1)
        flat[:mids.numel()] = mids
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("name", list(VARIANTS))
def test_append_bitwise(name):
    var = VARIANTS[name]
    case = make_custom_case(name=name, batch=3, num_qo_heads=4, num_kv_heads=2, q_lens=(40, 7, 90),
                            prefix_lens=(30, 0, 17), seed=zlib.crc32(name.encode()) % 10000, **var)
    fp8 = var.get("kv_dtype") == "fp8_e4m3fn"
    slots = _slots(case)
    n = len(slots)
    slots[3] = -1                                          # skipped
    slots[5] = case["num_pages"] * case["page_size"] + 2   # page past the pool: skipped by the device
    oracle_slots = slots.copy()
    oracle_slots[5] = -1
    for scale in ((1.0, 1.0), (0.37, 2.5)) if fp8 else ((1.0, 1.0),):
        k_new = _new_values(n, 2, var["head_dim"], 1, crafted=fp8)
        v_new = _new_values(n, 2, var["head_dim"], 2, crafted=fp8)
        _say("append", name, scale)
        want = append_paged_kv(_planes_codes(case["kv_cache"]), var["kv_layout"], var["page_size"],
                               as_codes(k_new), as_codes(v_new), oracle_slots,
                               "fp8" if fp8 else "bf16", scale[0], scale[1])
        import paged_kv_prefill_varlen_amd as ppa
        d = to_device(case)
        ppa.append_paged_kv_cache(k_new.cuda(), v_new.cuda(), torch.from_numpy(slots).cuda(), d["kv_cache"],
                                  var["kv_layout"], scale[0], scale[1])
        torch.cuda.synchronize()
        got = _planes_codes(tuple(t.cpu() for t in d["kv_cache"]) if isinstance(d["kv_cache"], tuple)
                            else d["kv_cache"].cpu())
        for kv_idx in range(2):
            if not np.array_equal(got[kv_idx], want[kv_idx]):
                diff = np.argwhere(got[kv_idx] != want[kv_idx])
                raise AssertionError(f"{name} plane {kv_idx}: {len(diff)} bytes differ, first at {diff[0]}: "
                                     f"got {got[kv_idx][tuple(diff[0])]:#x} want {want[kv_idx][tuple(diff[0])]:#x}")


def test_append_device_scales_and_then_attend():
    """Append the new tokens of a prefill batch into an fp8 cache (scales as
    device scalars), then run attention over it: the same output as the
    oracle on the appended cache."""
    import paged_kv_prefill_varlen_amd as ppa
    case = make_custom_case(name="append_attend", batch=2, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                            page_size=16, kv_dtype="fp8_e4m3fn", q_lens=(70, 33), prefix_lens=(20, 60), seed=321)
    slots = _slots(case)
    n = len(slots)
    k_new = _new_values(n, 2, 128, 7, crafted=False)
    v_new = _new_values(n, 2, 128, 8, crafted=False)
    ks, vs = 0.02, 0.03
    d = to_device(case)
    ppa.append_paged_kv_cache(k_new.cuda(), v_new.cuda(), torch.from_numpy(slots).cuda(), d["kv_cache"],
                              "HND", torch.tensor([ks], device="cuda"), torch.tensor([vs], device="cuda"))
    torch.cuda.synchronize()
    planes = append_paged_kv(_planes_codes(case["kv_cache"]), "HND", 16, as_codes(k_new), as_codes(v_new), slots,
                             "fp8", ks, vs)
    appended = dict(case)
    appended["kv_cache"] = tuple(torch.from_numpy(p).view(torch.float8_e4m3fn) for p in planes)
    got_planes = [as_codes(t.cpu()) for t in d["kv_cache"]]
    assert all(np.array_equal(g, w) for g, w in zip(got_planes, planes))
    want, written = run_oracle(appended)
    out = run_gpu(d)
    torch.cuda.synchronize()
    assert guard_rows_untouched(out, written)
    assert_close(out, want, written, fp8=True, what="append then attend")


def _pool_above_4gib(pool: torch.Tensor):
    """A pool of more than 4 GiB whose top pages hold `pool`'s pages; returns
    it and the page-id offset of the copy."""
    page_bytes = pool[0].numel() * pool.element_size()
    off = (1 << 32) // page_bytes + 7
    big = torch.empty((off + pool.shape[0],) + tuple(pool.shape[1:]), dtype=pool.dtype, device=pool.device)
    big[off:] = pool
    return big, off


@pytest.mark.parametrize("name", ["bf16_hnd_split_d128_p16", "fp8_nhd_combined_d64_p1"])
def test_append_beyond_4gib(name):
    """Slots in pages whose byte offsets lie past 4 GiB of the pool (the page
    address is formed in 64 bits): the appended pages hold exactly the
    oracle's bytes."""
    import paged_kv_prefill_varlen_amd as ppa
    var = VARIANTS[name]
    case = make_custom_case(name=name, batch=2, num_qo_heads=4, num_kv_heads=2, q_lens=(40, 90),
                            prefix_lens=(30, 17), seed=zlib.crc32(name.encode()) % 10000 + 1, **var)
    fp8 = var.get("kv_dtype") == "fp8_e4m3fn"
    slots = _slots(case)
    n = len(slots)
    k_new = _new_values(n, 2, var["head_dim"], 3, crafted=fp8)
    v_new = _new_values(n, 2, var["head_dim"], 4, crafted=fp8)
    want = append_paged_kv(_planes_codes(case["kv_cache"]), var["kv_layout"], var["page_size"], as_codes(k_new),
                           as_codes(v_new), slots, "fp8" if fp8 else "bf16", 1.0, 1.0)
    d = to_device(case)
    kv = d["kv_cache"]
    if isinstance(kv, tuple):
        (bk, off), (bv, off_v) = _pool_above_4gib(kv[0]), _pool_above_4gib(kv[1])
        assert off == off_v
        big = (bk, bv)
    else:
        big, off = _pool_above_4gib(kv)
    _say("append, pool > 4 GiB", name, "page offset", off)
    big_slots = torch.from_numpy(slots + off * var["page_size"]).cuda()
    ppa.append_paged_kv_cache(k_new.cuda(), v_new.cuda(), big_slots, big, var["kv_layout"], 1.0, 1.0)
    torch.cuda.synchronize()
    top = tuple(t[off:].cpu() for t in big) if isinstance(big, tuple) else big[off:].cpu()
    got = _planes_codes(top)
    for kv_idx in range(2):
        assert np.array_equal(got[kv_idx], want[kv_idx]), f"{name} plane {kv_idx}: appended bytes differ"
    del big
    torch.cuda.empty_cache()
