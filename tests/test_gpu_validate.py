"""GPU tests of the device-side metadata check (ppa_validate_metadata_device).

Each case is a valid description with one planted defect (or several, to
check which one is reported first).  The device result's status must equal
what the host validators return on host copies of the same arrays
(ppa_validate_metadata_host, then ppa_validate_page_table_csr_host for the
flat form), and its request index must name the request the planted defect
is in (-1 for defects of the whole batch).  The rules themselves follow from
the definition of the causal paged prefill and the API page's argument list
(the host validators' own tests pin them on the CPU).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from test_abi_host import ERR, OK, _case, _csr

ppa = pytest.importorskip("paged_kv_prefill_varlen_amd")
from paged_kv_prefill_varlen_amd import binding as B  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(x):
    return None if x is None else x.cuda()


def _host_status(p, c):
    csr = p.page_table_form == B.PPA_PAGE_TABLE_CSR
    st, _ = B.ppa_validate_metadata_host(p, c["cuq"], c["cukv"], c["sl"], None if csr else c["bt"])
    if st == OK and csr:
        st, _ = B.ppa_validate_page_table_csr_host(p, c["sl"], c["ptr"], c["idx"], c.get("last"))
    return st


def _run(p, keep):
    # keep: device tensors the params point to (alive until the check has run)
    st, req = B.check_metadata_device(p)
    del keep
    return st, req


def _padded(c, **over):
    d = {k: _dev(c[k]) for k in ("q", "bt", "sl", "cuq", "cukv", "out")}
    kv = tuple(_dev(t) for t in c["kv"]) if isinstance(c["kv"], tuple) else _dev(c["kv"])
    p = B.make_params(d["q"], kv, None, d["bt"], d["sl"], c["max_q"], c["max_kv"], 0.125, 1.0, c["B"],
                      d["cuq"], d["cukv"], c["W"], d["out"], c["layout"], None)
    for k, v in over.items():
        setattr(p, k, v)
    return p, (d, kv)


def _check(c, want_status, want_req, **over):
    p, keep = _padded(c, **over)
    host = _host_status(p, c)
    st, req = _run(p, keep)
    assert host == want_status, (host, want_status)
    assert (st, req) == (want_status, want_req)


def _i(v):
    return torch.tensor(v, dtype=torch.int32)


def test_valid_padded_description_passes():
    c = _case()
    _check(c, OK, -1)


@pytest.mark.parametrize("what,arrays,over,status,req", [
    ("cum_seq_lens_q does not start at 0", dict(cuq=[1, 6, 6, 15]), {}, "PPA_ERR_METADATA", -1),
    ("cum_seq_lens_q decreases at request 1", dict(cuq=[0, 6, 5, 14]), {}, "PPA_ERR_METADATA", 1),
    ("cum_seq_lens_q ends past num_tokens", {}, dict(num_tokens=13), "PPA_ERR_METADATA", -1),
    ("cum_seq_lens_kv step of request 1", dict(cukv=[0, 8, 13, 21]), {}, "PPA_ERR_METADATA", 1),
    ("cum_seq_lens_kv does not start at 0", dict(cukv=[2, 10, 14, 23]), {}, "PPA_ERR_METADATA", -1),
    ("q_len > kv_len in request 0", dict(sl=[4, 4, 9], cukv=[0, 4, 8, 17]), {}, "PPA_ERR_LENGTHS", 0),
    ("negative kv_len in request 1", dict(sl=[8, -1, 9], cukv=[0, 8, 7, 16]), {}, "PPA_ERR_LENGTHS", 1),
    ("q_len > max_q_len in request 2", {}, dict(max_q_len=8), "PPA_ERR_LENGTHS", 2),
])
def test_padded_rules(what, arrays, over, status, req):
    c = _case()
    for k, v in arrays.items():
        c[k] = _i(v)
    _check(c, ERR[status], req, **over)


def test_kv_len_above_max_kv_len():
    # (max_q_len <= max_kv_len is a shape rule, so request 2 gets the longest
    # prefix here)
    c = _case(q_lens=(5, 0, 4), prefix=(3, 4, 8))
    _check(c, ERR["PPA_ERR_LENGTHS"], 2, max_kv_len=8)


@pytest.mark.parametrize("value", [8, -1, 10 ** 6])
def test_page_id_out_of_range(value):
    c = _case()
    c["bt"] = c["bt"].clone()
    c["bt"][2, 0] = value
    _check(c, ERR["PPA_ERR_TABLE"], 2)


def test_columns_past_a_request_are_not_read():
    c = _case(q_lens=(5, 0, 20), prefix=(3, 4, 0))
    c["bt"] = c["bt"].clone()
    c["bt"][0, 1] = -7
    c["bt"][1, 1] = 10 ** 6
    _check(c, OK, -1)


def test_first_violation_wins_across_many_requests():
    # 1000 requests; defects planted in requests 700 (a page id in a long
    # row, checked by the strided loop), 300 (q_len > max_q_len) and 450
    # (cum_seq_lens_kv step): the lowest request is reported, with its rule
    rng = np.random.default_rng(7)
    Bn, P, pages = 1000, 1, 6000
    q_lens = rng.integers(0, 4, Bn)
    prefix = rng.integers(0, 6, Bn)
    prefix[700] = 5000                      # 5000+ pages of one token
    kv_lens = q_lens + prefix
    cols = int(kv_lens.max())
    T = int(q_lens.sum())
    c = dict(q=torch.zeros(T, 2, 64, dtype=torch.bfloat16), out=torch.zeros(T, 2, 64, dtype=torch.bfloat16),
             kv=(torch.zeros(pages, 1, P, 64, dtype=torch.bfloat16), torch.zeros(pages, 1, P, 64, dtype=torch.bfloat16)),
             bt=torch.from_numpy(rng.integers(0, pages, (Bn, cols)).astype(np.int32)),
             sl=torch.from_numpy(kv_lens.astype(np.int32)),
             cuq=torch.from_numpy(np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)),
             cukv=torch.from_numpy(np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)),
             layout="HND", max_q=3, max_kv=int(kv_lens.max()), B=Bn, W=-1)
    _check(c, OK, -1)
    c["bt"][700, 4321] = pages
    _check(c, ERR["PPA_ERR_TABLE"], 700)
    c["cukv"] = c["cukv"].clone()
    c["cukv"][451:] += 1
    _check(c, ERR["PPA_ERR_METADATA"], 450)
    q2 = q_lens.copy()
    q2[300] = 5
    c["cuq"] = torch.from_numpy(np.concatenate([[0], np.cumsum(q2)]).astype(np.int32))
    c["sl"] = torch.from_numpy((q2 + prefix).astype(np.int32))
    c["cukv"] = torch.from_numpy(np.concatenate([[0], np.cumsum(q2 + prefix)]).astype(np.int32))
    c["cukv"][451:] += 1
    c["q"] = c["out"] = torch.zeros(int(q2.sum()), 2, 64, dtype=torch.bfloat16)
    _check(c, ERR["PPA_ERR_LENGTHS"], 300, max_kv_len=int((q2 + prefix).max()))


# ---- the flat (CSR) table ------------------------------------------------

def _csr_check(c, ptr, idx, last, want_status, want_req):
    d = {k: _dev(c[k]) for k in ("q", "sl", "cuq", "cukv", "out")}
    kv = tuple(_dev(t) for t in c["kv"]) if isinstance(c["kv"], tuple) else _dev(c["kv"])
    ip, ix, lp = _dev(ptr), _dev(idx), _dev(last)
    p = B.make_params(d["q"], kv, None, None, d["sl"], c["max_q"], c["max_kv"], 0.125, 1.0, c["B"],
                      d["cuq"], d["cukv"], c["W"], d["out"], c["layout"], None, ip, ix, lp)
    hc = dict(c, ptr=ptr, idx=idx, last=last)
    host = _host_status(p, hc)
    st, req = B.check_metadata_device(p)
    del d, kv, ip, ix, lp
    assert host == want_status, (host, want_status)
    assert (st, req) == (want_status, want_req)


def test_csr_rules():
    c = _case()   # P 16, kv_lens (8, 4, 9): one page each
    ptr, idx, last = _csr(c)
    E = ERR["PPA_ERR_TABLE"]
    _csr_check(c, ptr, idx, last, OK, -1)
    _csr_check(c, ptr, idx, None, OK, -1)
    bad = ptr.clone(); bad[1], bad[2] = bad[2].clone(), bad[1].clone()
    _csr_check(c, bad, idx, last, E, 1)           # kv_indptr decreases at request 1
    bad = ptr.clone(); bad[0] = -1
    _csr_check(c, bad, idx, last, E, -1)          # negative start
    bad = ptr.clone(); bad[-1] = bad[-1] + 1
    _csr_check(c, bad, idx, last, E, -1)          # past the index array
    bad = ptr.clone(); bad[1] = 0
    _csr_check(c, bad, idx, last, E, 0)           # request 0 has no page
    badi = idx.clone(); badi[0] = 8
    _csr_check(c, ptr, badi, last, E, 0)          # page id out of range
    badi[0] = -1
    _csr_check(c, ptr, badi, last, E, 0)
    badl = last.clone(); badl[2] += 1
    _csr_check(c, ptr, idx, badl, E, 2)           # last_page_len inconsistent
    # a length rule comes before every table rule
    sl = c["sl"].clone(); sl[1] = -1
    c2 = dict(c, sl=sl, cukv=None)
    _csr_check(c2, ptr, idx, None, ERR["PPA_ERR_LENGTHS"], 1)


def test_empty_batch_reports_ok():
    c = _case()
    p, keep = _padded(c, batch_size=0)
    assert _run(p, keep) == (OK, -1)
