"""Host-side checks of the C-ABI library (no GPU, no compute calls).

* the shared library loads and exports every function that include/ppa.h
  declares, with the ABI version and struct size the binding expects;
* every rejection of the shape validator and of the host metadata validator
  is forced from the host, each with its own status code (the API page's
  argument list fixes what each array means; lengths, tables and window
  bounds follow from the definition of the causal paged prefill).

The validators read no device memory, so CPU tensors stand in for device
buffers here: only their shapes, strides and base pointers are used.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ppa.h")

ppa = pytest.importorskip("paged_kv_prefill_varlen_amd")
from paged_kv_prefill_varlen_amd import binding as B  # noqa: E402

OK = 0


def _header_text() -> str:
    with open(HEADER) as f:
        return f.read()


def _status_codes() -> dict:
    codes = {}
    for name, val in re.findall(r"\b(PPA_(?:OK|ERR_[A-Z_]+))\s*=\s*(-?\d+)", _header_text()):
        codes[name] = int(val)
    return codes


ERR = _status_codes()  # the ppa_status enum, read back from the header


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(ppa_[a-z0-9_]+)\s*\(", text)))


# --------------------------------------------------------------------------
# the library and its exports
# --------------------------------------------------------------------------

def test_header_declares_the_boundary():
    names = _declared_functions()
    for need in ("ppa_paged_prefill_attention", "ppa_validate_shapes", "ppa_validate_metadata_host",
                 "ppa_validate_metadata_device", "ppa_workspace_bytes", "ppa_strerror", "ppa_gather_paged_kv"):
        assert need in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.library_path())
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_abi_version_and_struct_size():
    assert B.ppa_abi_version() == B.PPA_ABI_VERSION
    assert B.ppa_params_size() == ctypes.sizeof(B.PpaParams)
    m = re.search(r"#define\s+PPA_ABI_VERSION\s+(\d+)", _header_text())
    assert m and int(m.group(1)) == B.PPA_ABI_VERSION


def test_strerror_covers_every_status():
    seen = set()
    for name, code in ERR.items():
        s = B.ppa_strerror(code)
        assert s and s not in seen, (name, s)
        seen.add(s)
    assert "unknown" in B.ppa_strerror(-999).lower()


# --------------------------------------------------------------------------
# a valid host-side description, then one defect at a time
# --------------------------------------------------------------------------

def _case(D=64, Hq=4, Hkv=2, P=16, pages=8, layout="HND", combined=False, kv_dtype=torch.bfloat16,
          q_lens=(5, 0, 9), prefix=(3, 4, 0)):
    kv_lens = [q + p for q, p in zip(q_lens, prefix)]
    T = sum(q_lens)
    cols = max(1, max((k + P - 1) // P for k in kv_lens))
    q = torch.zeros(T, Hq, D, dtype=torch.bfloat16)
    shape = (pages, Hkv, P, D) if layout == "HND" else (pages, P, Hkv, D)
    if combined:
        kv = torch.zeros(pages, 2, *shape[1:], dtype=kv_dtype)
    else:
        kv = (torch.zeros(shape, dtype=kv_dtype), torch.zeros(shape, dtype=kv_dtype))
    bt = torch.zeros(len(q_lens), cols, dtype=torch.int32)
    for b, k in enumerate(kv_lens):
        for j in range((k + P - 1) // P):
            bt[b, j] = (b * 3 + j) % pages
    sl = torch.tensor(kv_lens, dtype=torch.int32)
    cuq = torch.tensor([0] + list(torch.tensor(q_lens).cumsum(0).tolist()), dtype=torch.int32)
    cukv = torch.tensor([0] + list(torch.tensor(kv_lens).cumsum(0).tolist()), dtype=torch.int32)
    out = torch.empty_like(q)
    c = dict(q=q, kv=kv, bt=bt, sl=sl, cuq=cuq, cukv=cukv, out=out, layout=layout,
             max_q=max(q_lens), max_kv=max(kv_lens), B=len(q_lens), sinks=None, W=-1)
    return c


def _params(c, **over):
    p = B.make_params(c["q"], c["kv"], None, c["bt"], c["sl"], c["max_q"], c["max_kv"], 0.125, 1.0, c["B"],
                      c["cuq"], c["cukv"], c["W"], c["out"], c["layout"], c["sinks"])
    for k, v in over.items():
        if isinstance(getattr(p, k), ctypes.Array):
            getattr(p, k)[:] = v
        else:
            setattr(p, k, v)
    return p


def _shapes(p):
    return B.ppa_validate_shapes(p)


def _meta(p, c, **arrays):
    a = dict(cuq=c["cuq"], cukv=c["cukv"], sl=c["sl"], bt=c["bt"])
    a.update(arrays)
    return B.ppa_validate_metadata_host(p, a["cuq"], a["cukv"], a["sl"], a["bt"])


@pytest.mark.parametrize("layout", ["HND", "NHD"])
@pytest.mark.parametrize("combined", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_valid_descriptions_pass(layout, combined, D):
    c = _case(D=D, layout=layout, combined=combined)
    p = _params(c)
    assert _shapes(p) == (OK, "")
    assert _meta(p, c)[0] == OK
    assert B.ppa_workspace_bytes(p) == B.WORKSPACE_BYTES > 0


def test_fp8_kv_and_sinks_pass():
    c = _case(kv_dtype=torch.float8_e4m3fn)
    c["sinks"] = torch.zeros(4, dtype=torch.float32)
    c["W"] = 0
    p = _params(c)
    assert _shapes(p)[0] == OK


def test_fp8_compute_flag():
    """fp8_compute = 1 is accepted with an fp8 cache at head_dim 128 only."""
    assert _shapes(_params(_case(D=128, kv_dtype=torch.float8_e4m3fn), fp8_compute=1))[0] == OK
    assert _shapes(_params(_case(D=128, kv_dtype=torch.float8_e4m3fn), fp8_compute=0))[0] == OK
    for c, v in ((_case(D=128), 1), (_case(D=64, kv_dtype=torch.float8_e4m3fn), 1),
                 (_case(D=128, kv_dtype=torch.float8_e4m3fn), 2), (_case(D=128, kv_dtype=torch.float8_e4m3fn), -1)):
        st, msg = _shapes(_params(c, fp8_compute=v))
        assert st == ERR["PPA_ERR_DTYPE"] and msg, (v, st, msg)


SHAPE_DEFECTS = [
    # (name, overrides of ppa_params, expected status)
    ("abi version", dict(abi_version=99), "PPA_ERR_ABI"),
    ("struct size", dict(struct_size=8), "PPA_ERR_ABI"),
    ("query fp32", dict(query_dtype=B.PPA_DTYPE_FP32), "PPA_ERR_DTYPE"),
    ("out fp8", dict(out_dtype=B.PPA_DTYPE_FP8_E4M3FN), "PPA_ERR_DTYPE"),
    ("kv fp32", dict(kv_dtype=B.PPA_DTYPE_FP32), "PPA_ERR_DTYPE"),
    ("kv dtype 0", dict(kv_dtype=0), "PPA_ERR_DTYPE"),
    ("layout 2", dict(kv_layout=2), "PPA_ERR_LAYOUT"),
    ("form 5", dict(kv_form=5), "PPA_ERR_LAYOUT"),
    ("negative tokens", dict(num_tokens=-1), "PPA_ERR_SHAPE"),
    ("negative batch", dict(batch_size=-2), "PPA_ERR_SHAPE"),
    ("heads not multiple", dict(num_qo_heads=3), "PPA_ERR_HEADS"),
    ("zero kv heads", dict(num_kv_heads=0), "PPA_ERR_HEADS"),
    ("head_dim 96", dict(head_dim=96), "PPA_ERR_HEAD_DIM"),
    ("page 24", dict(page_size=24), "PPA_ERR_PAGE_SIZE"),
    ("page 0", dict(page_size=0), "PPA_ERR_PAGE_SIZE"),
    ("window -2", dict(window_left=-2), "PPA_ERR_WINDOW"),
    ("max_q > max_kv", dict(max_q_len=100), "PPA_ERR_LENGTHS"),
    ("table too narrow", dict(block_tables_cols=0), "PPA_ERR_TABLE"),
    ("table row stride", dict(block_tables_row_stride=0), "PPA_ERR_STRIDE"),
    ("null query", dict(query=None), "PPA_ERR_NULL_POINTER"),
    ("null out", dict(out=None), "PPA_ERR_NULL_POINTER"),
    ("null k", dict(k_cache=None), "PPA_ERR_NULL_POINTER"),
    ("null seq_lens", dict(seq_lens=None), "PPA_ERR_NULL_POINTER"),
    ("null cu_q", dict(cum_seq_lens_q=None), "PPA_ERR_NULL_POINTER"),
    ("null table", dict(block_tables=None), "PPA_ERR_NULL_POINTER"),
    ("query inner stride", dict(query_strides=[256, 64, 2]), "PPA_ERR_STRIDE"),
    ("out inner stride", dict(out_strides=[256, 64, 2]), "PPA_ERR_STRIDE"),
    ("query row not 16B", dict(query_strides=[257, 64, 1]), "PPA_ERR_STRIDE"),
    ("k inner stride", dict(k_cache_strides=[2048, 1024, 64, 2]), "PPA_ERR_STRIDE"),
    ("v token stride not 16B", dict(v_cache_strides=[2048, 1024, 63, 1]), "PPA_ERR_STRIDE"),
]


@pytest.mark.parametrize("name,over,expect", SHAPE_DEFECTS, ids=[d[0] for d in SHAPE_DEFECTS])
def test_shape_validator_rejects(name, over, expect):
    c = _case()
    p = _params(c, **over)
    st, msg = _shapes(p)
    assert st == ERR[expect], (st, msg)
    assert msg, "a rejection carries a message"


def test_shape_validator_rejects_null_params():
    buf = ctypes.create_string_buffer(128)
    lib = ctypes.CDLL(B.library_path())
    lib.ppa_validate_shapes.restype = ctypes.c_int32
    assert lib.ppa_validate_shapes(None, buf, len(buf)) == ERR["PPA_ERR_NULL_POINTER"]


def test_combined_cache_defects():
    c = _case(combined=True)
    assert _shapes(_params(c, kv_planes=3))[0] == ERR["PPA_ERR_LAYOUT"]
    assert _shapes(_params(c, kv_planes=0))[0] == ERR["PPA_ERR_LAYOUT"]
    assert _shapes(_params(c, kv_cache=None))[0] == ERR["PPA_ERR_NULL_POINTER"]
    # a plane stride that is not a 16-byte multiple
    s = list(c["kv"].stride())
    s[1] = 7
    assert _shapes(_params(c, kv_cache_strides=s))[0] == ERR["PPA_ERR_STRIDE"]


def test_misaligned_pointers():
    c = _case()
    p = _params(c)
    assert _shapes(_params(c, query=p.query + 2))[0] in (ERR["PPA_ERR_ALIGNMENT"],)
    assert _shapes(_params(c, k_cache=p.k_cache + 8))[0] == ERR["PPA_ERR_ALIGNMENT"]
    # sinks are fp32: 4-byte alignment is enough, 2 is not
    c["sinks"] = torch.zeros(5, dtype=torch.float32)[1:]
    p = _params(c)
    assert _shapes(p)[0] == OK
    assert _shapes(_params(c, sinks=p.sinks + 2))[0] == ERR["PPA_ERR_ALIGNMENT"]


def test_zero_pages_with_nonzero_kv():
    c = _case()
    assert _shapes(_params(c, num_pages=0))[0] == ERR["PPA_ERR_SHAPE"]


def test_empty_batch_is_valid():
    c = _case()
    p = _params(c, batch_size=0, max_q_len=0, max_kv_len=0)
    assert _shapes(p)[0] == OK
    assert _meta(p, c, cuq=torch.zeros(1, dtype=torch.int32), cukv=torch.zeros(1, dtype=torch.int32))[0] == OK


def _i(xs):
    return torch.tensor(xs, dtype=torch.int32)


def test_metadata_validator_rejects():
    c = _case()  # q_lens (5, 0, 9), kv_lens (8, 4, 9), P 16, 8 pages
    p = _params(c)
    E = ERR
    # cum_seq_lens_q must start at 0, never decrease, and end within num_tokens
    assert _meta(p, c, cuq=_i([1, 6, 6, 15]))[0] == E["PPA_ERR_METADATA"]
    assert _meta(p, c, cuq=_i([0, 6, 5, 14]))[0] == E["PPA_ERR_METADATA"]
    assert _meta(_params(c, num_tokens=13), c)[0] == E["PPA_ERR_METADATA"]
    # cum_seq_lens_kv must be the running sum of seq_lens
    assert _meta(p, c, cukv=_i([0, 8, 13, 21]))[0] == E["PPA_ERR_METADATA"]
    assert _meta(p, c, cukv=_i([2, 10, 14, 23]))[0] == E["PPA_ERR_METADATA"]
    # q_len > kv_len leaves an empty causal span: rejected
    assert _meta(p, c, sl=_i([4, 4, 9]), cukv=_i([0, 4, 8, 17]))[0] == E["PPA_ERR_LENGTHS"]
    # negative kv length
    assert _meta(p, c, sl=_i([8, -1, 9]), cukv=_i([0, 8, 7, 16]))[0] == E["PPA_ERR_LENGTHS"]
    # q_len above max_q_len, kv_len above max_kv_len
    assert _meta(_params(c, max_q_len=8), c)[0] == E["PPA_ERR_LENGTHS"]
    assert _meta(_params(c, max_kv_len=8), c)[0] == E["PPA_ERR_LENGTHS"]
    # a page id out of range, negative, or a table narrower than a request needs
    bt = c["bt"].clone()
    bt[2, 0] = 8
    assert _meta(p, c, bt=bt)[0] == E["PPA_ERR_TABLE"]
    bt[2, 0] = -1
    assert _meta(p, c, bt=bt)[0] == E["PPA_ERR_TABLE"]
    c2 = _case(q_lens=(5, 0, 20), prefix=(3, 4, 0))  # request 2 needs 2 pages of 16
    p2 = _params(c2, block_tables_cols=1, block_tables_row_stride=1)
    assert _meta(p2, c2, bt=c2["bt"][:, :1].contiguous())[0] == E["PPA_ERR_TABLE"]
    # missing host arrays
    assert _meta(p, c, cuq=None)[0] == E["PPA_ERR_NULL_POINTER"]


def test_metadata_ignores_columns_past_a_request():
    # columns past ceil(kv_len / P) are never read: garbage there is accepted
    c = _case(q_lens=(5, 0, 20), prefix=(3, 4, 0))
    bt = c["bt"].clone()
    bt[0, 1] = -7
    bt[1, 1] = 10 ** 6
    assert _meta(_params(c), c, bt=bt)[0] == OK


def test_params_keep_their_tensors_alive():
    # the struct holds raw device pointers: make_params keeps the tensors
    # they point into, so params built from temporaries stay valid
    import gc
    import weakref
    c = _case()
    sl = c["sl"].clone()
    cuq = c["cuq"].clone()
    watch = [weakref.ref(sl), weakref.ref(cuq)]
    p = B.make_params(c["q"], c["kv"], None, c["bt"], sl, c["max_q"], c["max_kv"], 0.125, 1.0, c["B"],
                      cuq, c["cukv"], c["W"], c["out"], c["layout"], None)
    del sl, cuq
    gc.collect()
    assert all(w() is not None for w in watch)
    assert p.seq_lens == watch[0]().data_ptr() and p.cum_seq_lens_q == watch[1]().data_ptr()
    del p
    gc.collect()
    assert all(w() is None for w in watch)


def test_device_metadata_check_rejects_arguments_on_the_host():
    # the entry point validates shapes and its result pointer before any
    # launch: these return without touching a device
    c = _case()
    dev_check = B._lib.ppa_validate_metadata_device
    good = ctypes.c_void_p(1 << 20)   # never dereferenced on these paths
    assert dev_check(ctypes.byref(_params(c, head_dim=96)), good, None) == ERR["PPA_ERR_HEAD_DIM"]
    assert dev_check(ctypes.byref(_params(c, cum_seq_lens_q=None)), good, None) == ERR["PPA_ERR_NULL_POINTER"]
    assert dev_check(ctypes.byref(_params(c)), None, None) == ERR["PPA_ERR_NULL_POINTER"]
    assert dev_check(ctypes.byref(_params(c)), ctypes.c_void_p((1 << 20) + 4), None) == ERR["PPA_ERR_ALIGNMENT"]
    assert dev_check(None, good, None) == ERR["PPA_ERR_NULL_POINTER"]


def test_cum_seq_lens_kv_optional():
    c = _case()
    c["cukv"] = None
    p = _params(c)
    assert _shapes(p)[0] == OK
    assert _meta(p, c, cukv=None)[0] == OK


def test_workspace_is_optional_but_checked_when_given():
    c = _case()
    ws = torch.zeros(B.WORKSPACE_BYTES + 64, dtype=torch.uint8)
    p = _params(c)
    assert _shapes(p)[0] == OK                       # no workspace: plain grid schedule
    p = _params(c, workspace=ws.data_ptr(), workspace_bytes=B.WORKSPACE_BYTES)
    assert _shapes(p)[0] == OK
    p = _params(c, workspace=ws.data_ptr(), workspace_bytes=B.WORKSPACE_BYTES - 4)
    assert _shapes(p)[0] == ERR["PPA_ERR_WORKSPACE"]
    p = _params(c, workspace=ws.data_ptr() + 4, workspace_bytes=B.WORKSPACE_BYTES)
    assert _shapes(p)[0] == ERR["PPA_ERR_ALIGNMENT"]


# --------------------------------------------------------------------------
# the flat (CSR) page table
# --------------------------------------------------------------------------

def _csr(c, slack=0, lead=0):
    ptr = [lead]   # page size 16 (the _case default)
    idx = [0] * lead
    last = []
    for b in range(c["B"]):
        kv = int(c["sl"][b])
        n = (kv + 15) // 16
        idx += [int(x) for x in c["bt"][b, :n]] + [1] * slack
        ptr.append(len(idx))
        last.append(0 if n == 0 else kv - (n - 1) * 16)
    return (torch.tensor(ptr, dtype=torch.int32), torch.tensor(idx or [0], dtype=torch.int32),
            torch.tensor(last, dtype=torch.int32))


def _csr_params(c, ptr, idx, last=None, **over):
    p = B.make_params(c["q"], c["kv"], None, None, c["sl"], c["max_q"], c["max_kv"], 0.125, 1.0, c["B"],
                      c["cuq"], c["cukv"], c["W"], c["out"], c["layout"], c["sinks"], ptr, idx, last)
    for k, v in over.items():
        setattr(p, k, v)
    return p


def test_csr_valid_description_passes():
    c = _case()   # P 16, kv_lens (8, 4, 9)
    ptr, idx, last = _csr(c)
    p = _csr_params(c, ptr, idx, last)
    assert p.page_table_form == B.PPA_PAGE_TABLE_CSR and p.block_tables is None
    assert _shapes(p) == (OK, "")
    assert B.ppa_validate_metadata_host(p, c["cuq"], c["cukv"], c["sl"], None)[0] == OK
    assert B.ppa_validate_page_table_csr_host(p, c["sl"], ptr, idx, last)[0] == OK
    # slack after each request and junk before request 0 are fine without last_page_len
    ptr2, idx2, _ = _csr(c, slack=2, lead=3)
    p2 = _csr_params(c, ptr2, idx2)
    assert B.ppa_validate_page_table_csr_host(p2, c["sl"], ptr2, idx2, None)[0] == OK


def test_csr_rejections():
    c = _case()
    ptr, idx, last = _csr(c)
    E = ERR
    chk = lambda p, ip, ix, lp=None: B.ppa_validate_page_table_csr_host(p, c["sl"], ip, ix, lp)[0]  # noqa: E731
    p = _csr_params(c, ptr, idx, last)
    # null device pointers / bad form
    assert _shapes(_csr_params(c, ptr, idx, kv_indptr=None))[0] == E["PPA_ERR_NULL_POINTER"]
    assert _shapes(_csr_params(c, ptr, idx, kv_indices=None))[0] == E["PPA_ERR_NULL_POINTER"]
    assert _shapes(_csr_params(c, ptr, idx, page_table_form=7))[0] == E["PPA_ERR_LAYOUT"]
    assert _shapes(_csr_params(c, ptr, idx, kv_indices_len=-1))[0] == E["PPA_ERR_SHAPE"]
    # indptr decreasing, negative start, past the index array
    bad = ptr.clone(); bad[1], bad[2] = bad[2], bad[1]
    assert chk(p, bad, idx) == E["PPA_ERR_TABLE"]
    bad = ptr.clone(); bad[0] = -1
    assert chk(p, bad, idx) == E["PPA_ERR_TABLE"]
    bad = ptr.clone(); bad[-1] = bad[-1] + 1
    assert chk(p, bad, idx) == E["PPA_ERR_TABLE"]
    # too few pages for a request, page id out of range
    bad = ptr.clone(); bad[1] = 0
    assert chk(p, bad, idx) == E["PPA_ERR_TABLE"]
    badi = idx.clone(); badi[0] = 8
    assert chk(p, ptr, badi) == E["PPA_ERR_TABLE"]
    badi[0] = -1
    assert chk(p, ptr, badi) == E["PPA_ERR_TABLE"]
    # last_page_len inconsistent with seq_lens, or a slack page with last_page_len
    badl = last.clone(); badl[0] += 1
    assert chk(p, ptr, idx, badl) == E["PPA_ERR_TABLE"]
    badl = last.clone(); badl[2] = 0
    assert chk(p, ptr, idx, badl) == E["PPA_ERR_TABLE"]
    ptr2, idx2, _ = _csr(c, slack=1)
    p2 = _csr_params(c, ptr2, idx2)
    assert chk(p2, ptr2, idx2, last) == E["PPA_ERR_TABLE"]
    # the padded form still requires block_tables
    with pytest.raises(ValueError):
        B.make_params(c["q"], c["kv"], None, None, c["sl"], c["max_q"], c["max_kv"], 0.125, 1.0, c["B"],
                      c["cuq"], c["cukv"], c["W"], c["out"], c["layout"], None)



# --------------------------------------------------------------------------
# log-sum-exp output, split-KV and merge arguments
# --------------------------------------------------------------------------

def test_split_and_lse_rejections():
    c = _case()
    E = ERR
    assert _shapes(_params(c, kv_splits=-1))[0] == E["PPA_ERR_SHAPE"]
    assert _shapes(_params(c, kv_splits=257))[0] == E["PPA_ERR_SHAPE"]
    assert _shapes(_params(c, kv_splits=1))[0] == OK   # 0 and 1 both mean no split
    assert _shapes(_params(c, kv_splits=4))[0] == E["PPA_ERR_WORKSPACE"]   # no workspace
    p = _params(c, kv_splits=4)
    need = B.ppa_workspace_bytes(p)
    T, H, D = c["q"].shape
    assert need == 256 + ((4 * T * H * D * 4 + 255) // 256) * 256 + ((4 * T * H * 4 + 255) // 256) * 256
    ws = torch.zeros(need + 16, dtype=torch.uint8)
    assert _shapes(_params(c, kv_splits=4, workspace=ws.data_ptr(), workspace_bytes=need))[0] == OK
    assert _shapes(_params(c, kv_splits=4, workspace=ws.data_ptr(), workspace_bytes=need - 1))[0] == \
        E["PPA_ERR_WORKSPACE"]
    lse = torch.zeros(T * H + 1, dtype=torch.float32)
    assert _shapes(_params(c, lse=lse.data_ptr(), lse_strides=[H, 1]))[0] == OK
    assert _shapes(_params(c, lse=lse.data_ptr() + 2, lse_strides=[H, 1]))[0] == E["PPA_ERR_ALIGNMENT"]
    assert _shapes(_params(c, lse=lse.data_ptr(), lse_strides=[-1, 1]))[0] == E["PPA_ERR_STRIDE"]


def test_merge_argument_rejections():
    """Bad merge arguments are rejected before anything is launched."""
    E = ERR
    o = torch.zeros(2, 3, 4, 64)
    l = torch.zeros(2, 3, 4)
    out = torch.zeros(3, 4, 64, dtype=torch.bfloat16)

    def m(**over):
        p = B.PpaMergeParams()
        p.abi_version, p.struct_size = B.PPA_ABI_VERSION, ctypes.sizeof(B.PpaMergeParams)
        p.num_parts, p.num_rows, p.num_heads, p.head_dim = 2, 3, 4, 64
        p.o_parts, p.lse_parts, p.out = o.data_ptr(), l.data_ptr(), out.data_ptr()
        p.out_dtype = B.PPA_DTYPE_BF16
        p.out_strides[:] = [256, 64, 1]
        for k, v in over.items():
            if isinstance(getattr(p, k), ctypes.Array):
                getattr(p, k)[:] = v
            else:
                setattr(p, k, v)
        return int(B._lib.ppa_merge_attention_states(ctypes.byref(p), None))

    assert m(abi_version=1) == E["PPA_ERR_ABI"]
    assert m(num_parts=0) == E["PPA_ERR_SHAPE"]
    assert m(num_heads=0) == E["PPA_ERR_SHAPE"]
    assert m(head_dim=96) == E["PPA_ERR_HEAD_DIM"]
    assert m(out_dtype=B.PPA_DTYPE_FP32) == E["PPA_ERR_DTYPE"]
    assert m(o_parts=None) == E["PPA_ERR_NULL_POINTER"]
    assert m(out_strides=[256, 64, 2]) == E["PPA_ERR_STRIDE"]
    assert m(out_strides=[255, 64, 1]) == E["PPA_ERR_STRIDE"]
    assert m(lse_parts=l.data_ptr() + 2) == E["PPA_ERR_ALIGNMENT"]
    assert m(num_rows=0) == OK   # nothing to do, nothing launched


def test_mxfp4_output_validation():
    """MXFP4 output (the API page's FP4 out with o_sf_scale / o_sf_vec_size):
    a valid description passes; each defect has its own status."""
    E = ERR
    for D in (64, 128):
        c = _case(D=D)
        T, H, _ = c["q"].shape
        for vec in (16, 32):
            c["out"] = B.empty_mxfp4(T, H, D, "cpu", vec, 0.5)
            p = _params(c)
            assert p.out_dtype == B.PPA_DTYPE_MXFP4 and p.o_sf_vec_size == vec and p.o_sf_scale == 0.5
            assert list(p.out_strides) == [H * D // 2, D // 2, 1]
            assert list(p.out_sf_strides) == [H * (D // vec), D // vec]
            assert _shapes(p) == (OK, "")
            assert _meta(p, c)[0] == OK
    c = _case(D=64)
    T, H, D = c["q"].shape
    c["out"] = B.empty_mxfp4(T, H, D, "cpu")
    assert _shapes(_params(c, out_sf=None))[0] == E["PPA_ERR_NULL_POINTER"]
    for vec in (0, 8, 64):
        assert _shapes(_params(c, o_sf_vec_size=vec))[0] == E["PPA_ERR_SHAPE"]
    for g in (0.0, -1.0, float("inf"), float("nan")):
        assert _shapes(_params(c, o_sf_scale=g))[0] == E["PPA_ERR_SHAPE"]
    assert _shapes(_params(c, out_strides=[H * D // 2 + 8, D // 2, 1]))[0] == E["PPA_ERR_STRIDE"]
    assert _shapes(_params(c, out_strides=[H * D // 2, D // 2, 2]))[0] == E["PPA_ERR_STRIDE"]
    assert _shapes(_params(c, out_sf_strides=[-1, 2]))[0] == E["PPA_ERR_STRIDE"]
    assert _shapes(_params(c, kv_splits=2, workspace=0))[0] == E["PPA_ERR_WORKSPACE"]
    # the binding refuses shapes that do not match the query
    with pytest.raises(ValueError):
        _params(dict(c, out=B.empty_mxfp4(T, H, 128, "cpu")))
    with pytest.raises(ValueError):
        B.batch_context_with_kv_cache(c["q"], c["kv"], None, c["bt"], c["sl"], c["max_q"], c["max_kv"], 1.0, 1.0,
                                      c["B"], c["cuq"], c["cukv"], out_dtype="nvfp4")


def test_merge_mxfp4_rejections():
    E = ERR
    o = torch.zeros(2, 3, 4, 64)
    l = torch.zeros(2, 3, 4)
    mx = B.empty_mxfp4(3, 4, 64, "cpu")

    def m(**over):
        p = B.PpaMergeParams()
        p.abi_version, p.struct_size = B.PPA_ABI_VERSION, ctypes.sizeof(B.PpaMergeParams)
        p.num_parts, p.num_rows, p.num_heads, p.head_dim = 2, 3, 4, 64
        p.o_parts, p.lse_parts = o.data_ptr(), l.data_ptr()
        B._set_out(p, mx, (3, 4, 64))
        for k, v in over.items():
            if isinstance(getattr(p, k), ctypes.Array):
                getattr(p, k)[:] = v
            else:
                setattr(p, k, v)
        return int(B._lib.ppa_merge_attention_states(ctypes.byref(p), None))

    assert m(o_sf_vec_size=8) == E["PPA_ERR_SHAPE"]
    assert m(o_sf_scale=0.0) == E["PPA_ERR_SHAPE"]
    assert m(out_sf=None) == E["PPA_ERR_NULL_POINTER"]
    assert m(out_sf_strides=[-8, 2]) == E["PPA_ERR_STRIDE"]
    assert m(num_rows=0) == OK


# --------------------------------------------------------------------------
# KV append arguments
# --------------------------------------------------------------------------

def test_append_validation():
    E = ERR
    c = _case(combined=False)
    cache = _params(c)
    k_new = torch.zeros(6, 2, 64, dtype=torch.bfloat16)
    v_new = torch.zeros(6, 2, 64, dtype=torch.bfloat16)
    slots = torch.arange(6, dtype=torch.int64)
    a = B.make_append_params(k_new, v_new, slots)
    assert B.ppa_validate_append(cache, a) == (OK, "")

    def chk(cache_over=None, **over):
        p = _params(c, **(cache_over or {}))
        x = B.make_append_params(k_new, v_new, slots)
        for k, v in over.items():
            if isinstance(getattr(x, k), ctypes.Array):
                getattr(x, k)[:] = v
            else:
                setattr(x, k, v)
        return B.ppa_validate_append(p, x)[0]

    assert chk(abi_version=1) == E["PPA_ERR_ABI"]
    assert chk(new_dtype=B.PPA_DTYPE_FP32) == E["PPA_ERR_DTYPE"]
    assert chk(slot_mapping=None) == E["PPA_ERR_NULL_POINTER"]
    assert chk(k_new_strides=[128, 64, 2]) == E["PPA_ERR_STRIDE"]
    assert chk(v_new_strides=[129, 64, 1]) == E["PPA_ERR_STRIDE"]
    assert chk(slot_mapping=slots.data_ptr() + 4) == E["PPA_ERR_ALIGNMENT"]
    assert chk(k_new=k_new.data_ptr() + 2) == E["PPA_ERR_ALIGNMENT"]
    assert chk(num_new=-1) == E["PPA_ERR_SHAPE"]
    assert chk(num_new=0, slot_mapping=None) == OK          # nothing to write
    assert chk(cache_over=dict(kv_dtype=B.PPA_DTYPE_FP32)) == E["PPA_ERR_DTYPE"]
    assert chk(cache_over=dict(head_dim=96)) == E["PPA_ERR_HEAD_DIM"]
    assert chk(cache_over=dict(page_size=3)) == E["PPA_ERR_PAGE_SIZE"]
    assert chk(cache_over=dict(k_cache=None)) == E["PPA_ERR_NULL_POINTER"]
    # a one-plane combined cache cannot take K and V in separate slots
    c1 = _case(combined=True)
    p1 = _params(c1, kv_planes=1)
    assert B.ppa_validate_append(p1, a)[0] == E["PPA_ERR_LAYOUT"]
    with pytest.raises(TypeError):
        B.make_append_params(k_new, v_new, slots.to(torch.int32))


# --------------------------------------------------------------------------
# the split-KV planner (host only)
# --------------------------------------------------------------------------

def _model_by_hand(items, resident, tiles, max_splits):
    """The cost model as ppa.h states it, evaluated for every S."""
    if min(items, resident, tiles) <= 0 or max_splits <= 1 or items >= resident:
        return 1
    best, best_cost = 1, None
    for s in range(1, max(1, min(tiles // 4, max_splits)) + 1):
        cost = -(-items * s // resident) * (-(-tiles // s) + 3) + 0.5 * s
        if best_cost is None or cost < best_cost:
            best, best_cost = s, cost
    return best


def test_plan_model_cases():
    m = B.ppa_plan_kv_splits_model
    # decode-shaped batch: 16 requests x 8 kv heads = 128 items on 256 CUs,
    # 8192 keys = 128 tiles: two chunks fill the device (the measured best)
    assert m(128, 256, 128, 256) == 2
    # enough work items already: no split
    assert m(256, 256, 4096, 256) == 1 and m(4096, 256, 32, 256) == 1
    # too few tiles to give every chunk four, or no room for partial state
    assert m(8, 256, 7, 256) == 1 and m(8, 256, 512, 1) == 1
    # one request, 8 kv heads, 32K keys: many chunks, bounded by the workspace
    assert m(8, 256, 512, 256) > 8 and m(8, 256, 512, 5) == 5
    for bad in ((0, 256, 10, 8), (8, 0, 10, 8), (8, 256, 0, 8), (-1, 256, 10, 8)):
        assert m(*bad) == 1


def test_plan_model_matches_its_definition():
    m = B.ppa_plan_kv_splits_model
    for items in (1, 3, 8, 50, 100, 127, 128, 200, 255):
        for resident in (64, 256, 512):
            for tiles in (1, 4, 8, 9, 33, 128, 513):
                for mx in (1, 2, 3, 16, 256):
                    assert m(items, resident, tiles, mx) == _model_by_hand(items, resident, tiles, mx), \
                        (items, resident, tiles, mx)


def test_plan_without_workspace_or_with_bad_params():
    c = _case()
    assert B.ppa_plan_kv_splits(_params(c)) == 1     # no workspace: nowhere to put partial state
    with pytest.raises(B.PpaError) as e:
        B.ppa_plan_kv_splits(_params(c, head_dim=96))
    assert e.value.status == ERR["PPA_ERR_HEAD_DIM"]


# --------------------------------------------------------------------------
# metadata lengths and devices (checked by the binding: the C ABI takes bare
# pointers and reads batch_size + 1 offsets, batch_size lengths and
# batch_size table rows)
# --------------------------------------------------------------------------

def _short(t, n):
    return t[:n].clone()


def test_make_params_rejects_short_metadata():
    c = _case()   # batch of 3
    args = lambda **o: dict(dict(query=c["q"], kv_cache=c["kv"], workspace_buffer=None, block_tables=c["bt"],
                                 seq_lens=c["sl"], max_q_len=c["max_q"], max_kv_len=c["max_kv"], bmm1_scale=0.125,
                                 bmm2_scale=1.0, batch_size=c["B"], cum_seq_lens_q=c["cuq"],
                                 cum_seq_lens_kv=c["cukv"], window_left=-1, out=c["out"], kv_layout=c["layout"]),
                            **o)
    B.make_params(**args())   # the full-length arrays pass
    for name, bad in (("seq_lens", _short(c["sl"], 2)), ("cum_seq_lens_q", _short(c["cuq"], 3)),
                      ("cum_seq_lens_kv", _short(c["cukv"], 3)), ("block_tables", _short(c["bt"], 2))):
        with pytest.raises(ValueError, match=name):
            B.make_params(**args(**{name: bad}))
    # a batch_size larger than the arrays: the reading ASan flagged in the
    # host checker before this check existed
    with pytest.raises(ValueError):
        B.make_params(**args(batch_size=4))
    with pytest.raises(ValueError, match="batch_size"):
        B.make_params(**args(batch_size=-1))
    ptr, idx, last = _csr(c)
    B.make_params(**args(block_tables=None, kv_indptr=ptr, kv_indices=idx, kv_last_page_len=last))
    with pytest.raises(ValueError, match="kv_indptr"):
        B.make_params(**args(block_tables=None, kv_indptr=_short(ptr, 3), kv_indices=idx))
    with pytest.raises(ValueError, match="kv_last_page_len"):
        B.make_params(**args(block_tables=None, kv_indptr=ptr, kv_indices=idx, kv_last_page_len=_short(last, 2)))


def test_make_params_rejects_tensors_on_another_device():
    c = _case()
    meta = lambda t: torch.empty(t.shape, dtype=t.dtype, device="meta")
    base = dict(query=c["q"], kv_cache=c["kv"], workspace_buffer=None, block_tables=c["bt"], seq_lens=c["sl"],
                max_q_len=c["max_q"], max_kv_len=c["max_kv"], bmm1_scale=0.125, bmm2_scale=1.0, batch_size=c["B"],
                cum_seq_lens_q=c["cuq"], cum_seq_lens_kv=c["cukv"], window_left=-1, out=c["out"],
                kv_layout=c["layout"])
    for name in ("block_tables", "seq_lens", "cum_seq_lens_q", "cum_seq_lens_kv", "out"):
        with pytest.raises(ValueError, match="device"):
            B.make_params(**dict(base, **{name: meta(base[name])}))
    with pytest.raises(ValueError, match="device"):
        B.make_params(**dict(base, kv_cache=(c["kv"][0], meta(c["kv"][1]))))
    with pytest.raises(ValueError, match="device"):
        B.make_params(**dict(base, workspace_buffer=torch.zeros(256, dtype=torch.uint8, device="meta")))


def test_host_checkers_stay_inside_documented_lengths_under_asan(tmp_path):
    """The host checkers, built with AddressSanitizer, read each metadata
    array only within the length ppa.h documents (exact-size heap copies)."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "validate_bounds"
    src = os.path.join(ROOT, "tests", "host_asan", "validate_bounds.cpp")
    host = os.path.join(ROOT, "paged_kv_prefill_varlen_amd", "csrc", "ppa_host.cpp")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "paged_kv_prefill_varlen_amd", "csrc"),
                    src, host, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in r.stderr, r.stdout + r.stderr
