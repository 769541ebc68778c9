"""ctypes binding of ``include/ppa.h``: argument marshalling only.

``PpaParams`` mirrors ``struct ppa_params`` field for field; its size is
checked against the library's ``ppa_params_size()`` when the library loads.
Torch is used for device pointers, strides and the current stream only.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p
from typing import NamedTuple, Optional, Sequence, Tuple, Union

import numpy as np
import torch

PPA_ABI_VERSION = 6

# enums of ppa.h
PPA_DTYPE_BF16 = 1
PPA_DTYPE_FP8_E4M3FN = 2
PPA_DTYPE_FP32 = 3
PPA_DTYPE_MXFP4 = 4
PPA_KV_LAYOUT_HND = 0
PPA_KV_LAYOUT_NHD = 1
PPA_KV_SPLIT = 0
PPA_KV_COMBINED = 1
PPA_PAGE_TABLE_PADDED = 0
PPA_PAGE_TABLE_CSR = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build by default; PPA_LIBRARY names another build of the same
# C ABI (e.g. to time two builds of the kernels against each other).  Either
# way the call goes to a HIP library: there is no other implementation.
_LIB_PATH = os.environ.get("PPA_LIBRARY", os.path.join(_HERE, "_lib", "libppa.so"))


class PpaParams(ctypes.Structure):
    _fields_ = [
        ("abi_version", c_uint32),
        ("struct_size", c_uint32),
        ("query", c_void_p),
        ("query_dtype", c_int32),
        ("num_tokens", c_int32),
        ("num_qo_heads", c_int32),
        ("head_dim", c_int32),
        ("query_strides", c_int64 * 3),
        ("kv_form", c_int32),
        ("kv_layout", c_int32),
        ("kv_dtype", c_int32),
        ("num_pages", c_int32),
        ("num_kv_heads", c_int32),
        ("page_size", c_int32),
        ("kv_cache", c_void_p),
        ("kv_planes", c_int32),
        ("kv_cache_strides", c_int64 * 5),
        ("k_cache", c_void_p),
        ("v_cache", c_void_p),
        ("k_cache_strides", c_int64 * 4),
        ("v_cache_strides", c_int64 * 4),
        ("workspace", c_void_p),
        ("workspace_bytes", c_size_t),
        ("block_tables", c_void_p),
        ("block_tables_cols", c_int32),
        ("block_tables_row_stride", c_int64),
        ("seq_lens", c_void_p),
        ("cum_seq_lens_q", c_void_p),
        ("cum_seq_lens_kv", c_void_p),
        ("batch_size", c_int32),
        ("max_q_len", c_int32),
        ("max_kv_len", c_int32),
        ("bmm1_scale", c_float),
        ("bmm2_scale", c_float),
        ("bmm1_scale_ptr", c_void_p),
        ("bmm2_scale_ptr", c_void_p),
        ("window_left", c_int32),
        ("sinks", c_void_p),
        ("out", c_void_p),
        ("out_dtype", c_int32),
        ("out_strides", c_int64 * 3),
        ("page_table_form", c_int32),
        ("kv_indptr", c_void_p),
        ("kv_indices", c_void_p),
        ("kv_indices_len", c_int64),
        ("kv_last_page_len", c_void_p),
        ("lse", c_void_p),
        ("lse_strides", c_int64 * 2),
        ("kv_splits", c_int32),
        ("out_sf", c_void_p),
        ("out_sf_strides", c_int64 * 2),
        ("o_sf_scale", c_float),
        ("o_sf_vec_size", c_int32),
        ("fp8_compute", c_int32),
    ]


class PpaAppendParams(ctypes.Structure):
    _fields_ = [
        ("abi_version", c_uint32),
        ("struct_size", c_uint32),
        ("k_new", c_void_p),
        ("v_new", c_void_p),
        ("new_dtype", c_int32),
        ("num_new", c_int32),
        ("k_new_strides", c_int64 * 3),
        ("v_new_strides", c_int64 * 3),
        ("slot_mapping", c_void_p),
        ("k_scale", c_float),
        ("v_scale", c_float),
        ("k_scale_ptr", c_void_p),
        ("v_scale_ptr", c_void_p),
    ]


class PpaMergeParams(ctypes.Structure):
    _fields_ = [
        ("abi_version", c_uint32),
        ("struct_size", c_uint32),
        ("num_parts", c_int32),
        ("num_rows", c_int32),
        ("num_heads", c_int32),
        ("head_dim", c_int32),
        ("o_parts", c_void_p),
        ("lse_parts", c_void_p),
        ("sinks", c_void_p),
        ("out", c_void_p),
        ("out_dtype", c_int32),
        ("out_strides", c_int64 * 3),
        ("lse_out", c_void_p),
        ("lse_out_strides", c_int64 * 2),
        ("out_sf", c_void_p),
        ("out_sf_strides", c_int64 * 2),
        ("o_sf_scale", c_float),
        ("o_sf_vec_size", c_int32),
    ]


class MxFp4Output(NamedTuple):
    """An MXFP4 output: ``data`` uint8 ``[rows, heads, head_dim / 2]`` (two
    E2M1 codes per byte, element 2i in the low nibble), ``scale`` uint8
    ``[rows, heads, head_dim / vec_size]`` (E8M0 block scales), and the
    ``o_sf_scale`` g the output was multiplied by (o ~ code * 2^E / g)."""
    data: torch.Tensor
    scale: torch.Tensor
    vec_size: int = 32
    o_sf_scale: float = 1.0


def empty_mxfp4(rows: int, heads: int, head_dim: int, device, vec_size: int = 32,
                o_sf_scale: float = 1.0) -> MxFp4Output:
    """Allocate an MXFP4 output for ``rows`` x ``heads`` rows of ``head_dim``."""
    if head_dim % vec_size != 0:
        raise ValueError("head_dim must be a multiple of vec_size")
    return MxFp4Output(torch.empty((rows, heads, head_dim // 2), dtype=torch.uint8, device=device),
                       torch.empty((rows, heads, head_dim // vec_size), dtype=torch.uint8, device=device),
                       int(vec_size), float(o_sf_scale))


def _set_out(p, out, shape) -> None:
    """Point a PpaParams / PpaMergeParams at a bf16 tensor or an MxFp4Output
    of logical shape ``shape`` = (rows, heads, head_dim)."""
    rows, heads, d = (int(x) for x in shape)
    if isinstance(out, MxFp4Output):
        if out.data.dtype != torch.uint8 or tuple(out.data.shape) != (rows, heads, d // 2):
            raise ValueError("MXFP4 data must be uint8 [rows, heads, head_dim / 2]")
        if out.scale.dtype != torch.uint8 or tuple(out.scale.shape) != (rows, heads, d // max(1, out.vec_size)):
            raise ValueError("MXFP4 scale must be uint8 [rows, heads, head_dim / vec_size]")
        if out.scale.stride(2) != 1:
            raise ValueError("MXFP4 scale bytes of a row must be contiguous")
        p.out = _ptr(out.data)
        p.out_dtype = PPA_DTYPE_MXFP4
        p.out_strides[:] = list(out.data.stride())
        p.out_sf = _ptr(out.scale)
        p.out_sf_strides[:] = list(out.scale.stride()[:2])
        p.o_sf_scale = float(out.o_sf_scale)
        p.o_sf_vec_size = int(out.vec_size)
    else:
        if out.dim() != 3 or tuple(out.shape) != (rows, heads, d):
            raise ValueError("out must have shape [rows, heads, head_dim]")
        p.out = _ptr(out)
        p.out_dtype = _dt(out)
        p.out_strides[:] = list(out.stride())


class PpaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        self.status = status
        super().__init__(f"ppa status {status} ({ppa_strerror(status)}): {msg}")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"HIP library {_LIB_PATH} is not built; run `python paged_kv_prefill_varlen_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(PpaParams)
    sigs = {
        "ppa_abi_version": (c_int32, []),
        "ppa_params_size": (c_size_t, []),
        "ppa_strerror": (c_char_p, [c_int32]),
        "ppa_validate_shapes": (c_int32, [P, c_char_p, c_size_t]),
        "ppa_validate_metadata_host": (c_int32, [P, c_void_p, c_void_p, c_void_p, c_void_p, c_char_p, c_size_t]),
        "ppa_validate_page_table_csr_host": (c_int32, [P, c_void_p, c_void_p, c_void_p, c_void_p, c_char_p,
                                                       c_size_t]),
        "ppa_validate_metadata_device": (c_int32, [P, c_void_p, c_void_p]),
        "ppa_workspace_bytes": (c_size_t, [P]),
        "ppa_plan_kv_splits_model": (c_int32, [c_int64, c_int64, c_int64, c_int32]),
        "ppa_plan_kv_splits": (c_int32, [P]),
        "ppa_paged_prefill_attention": (c_int32, [P, c_void_p]),
        "ppa_paged_prefill_attention_noalloc": (c_int32, [P, c_void_p]),
        "ppa_noalloc_scratch_bytes": (c_size_t, []),
        "ppa_gather_paged_kv": (c_int32, [P, c_int32, c_void_p, c_int64, c_void_p]),
        "ppa_merge_attention_states": (c_int32, [ctypes.POINTER(PpaMergeParams), c_void_p]),
        "ppa_merge_params_size": (c_size_t, []),
        "ppa_append_params_size": (c_size_t, []),
        "ppa_validate_append": (c_int32, [P, ctypes.POINTER(PpaAppendParams), c_char_p, c_size_t]),
        "ppa_append_paged_kv": (c_int32, [P, ctypes.POINTER(PpaAppendParams), c_void_p]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.ppa_abi_version() != PPA_ABI_VERSION:
        raise ImportError(f"{_LIB_PATH}: ABI version {lib.ppa_abi_version()}, binding expects {PPA_ABI_VERSION}")
    if lib.ppa_append_params_size() != ctypes.sizeof(PpaAppendParams):
        raise ImportError(f"{_LIB_PATH}: sizeof(ppa_append_params) {lib.ppa_append_params_size()} != binding's "
                          f"{ctypes.sizeof(PpaAppendParams)}")
    if lib.ppa_merge_params_size() != ctypes.sizeof(PpaMergeParams):
        raise ImportError(f"{_LIB_PATH}: sizeof(ppa_merge_params) {lib.ppa_merge_params_size()} != binding's "
                          f"{ctypes.sizeof(PpaMergeParams)}")
    if lib.ppa_params_size() != ctypes.sizeof(PpaParams):
        raise ImportError(f"{_LIB_PATH}: sizeof(ppa_params) {lib.ppa_params_size()} != binding's "
                          f"{ctypes.sizeof(PpaParams)}")
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


# --------------------------------------------------------------------------
# one-to-one wrappers of the C entry points
# --------------------------------------------------------------------------

def ppa_abi_version() -> int:
    return int(_lib.ppa_abi_version())


def ppa_params_size() -> int:
    return int(_lib.ppa_params_size())


def ppa_strerror(status: int) -> str:
    return _lib.ppa_strerror(int(status)).decode()


def ppa_validate_shapes(params: PpaParams) -> Tuple[int, str]:
    buf = ctypes.create_string_buffer(512)
    st = _lib.ppa_validate_shapes(ctypes.byref(params), buf, len(buf))
    return int(st), buf.value.decode()


def _host_i32(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def ppa_validate_metadata_host(params: PpaParams, cum_seq_lens_q, cum_seq_lens_kv, seq_lens,
                               block_tables) -> Tuple[int, str]:
    """Deep check on host copies (torch tensors are copied to the host)."""
    cu_q = _host_i32(cum_seq_lens_q)
    cu_kv = _host_i32(cum_seq_lens_kv)
    sl = _host_i32(seq_lens)
    bt = _host_i32(block_tables)
    if bt is not None and bt.ndim != 2:
        raise ValueError("block_tables must be 2-D")
    # the host copy is dense: describe it with its own row stride
    hp = PpaParams.from_buffer_copy(params)
    if bt is not None:
        hp.block_tables_row_stride = bt.shape[1]
    ptr = lambda a: None if a is None else a.ctypes.data_as(c_void_p)  # noqa: E731
    buf = ctypes.create_string_buffer(512)
    st = _lib.ppa_validate_metadata_host(ctypes.byref(hp), ptr(cu_q), ptr(cu_kv), ptr(sl), ptr(bt),
                                         buf, len(buf))
    return int(st), buf.value.decode()


def ppa_validate_page_table_csr_host(params: PpaParams, seq_lens, kv_indptr, kv_indices,
                                     kv_last_page_len=None) -> Tuple[int, str]:
    """Page-table check of the flat (CSR) form on host copies."""
    sl = _host_i32(seq_lens)
    ip = _host_i32(kv_indptr)
    ix = _host_i32(kv_indices)
    lp = _host_i32(kv_last_page_len)
    ptr = lambda a: None if a is None else a.ctypes.data_as(c_void_p)  # noqa: E731
    buf = ctypes.create_string_buffer(512)
    st = _lib.ppa_validate_page_table_csr_host(ctypes.byref(params), ptr(sl), ptr(ip), ptr(ix), ptr(lp), buf,
                                               len(buf))
    return int(st), buf.value.decode()


def ppa_workspace_bytes(params: Optional[PpaParams] = None) -> int:
    return int(_lib.ppa_workspace_bytes(None if params is None else ctypes.byref(params)))


def ppa_plan_kv_splits_model(work_items: int, resident: int, key_tiles: int, max_splits: int) -> int:
    """The split-count cost model (pure; see ppa.h)."""
    return int(_lib.ppa_plan_kv_splits_model(int(work_items), int(resident), int(key_tiles), int(max_splits)))


def ppa_plan_kv_splits(params: PpaParams) -> int:
    """kv_splits the library picks for this call on the current device
    (within params.workspace_bytes); raises PpaError on invalid params."""
    st = int(_lib.ppa_plan_kv_splits(ctypes.byref(params)))
    if st < 1:
        _, msg = ppa_validate_shapes(params)
        raise PpaError(st, msg or ppa_strerror(st))
    return st


# bytes of the optional scheduler workspace (the same for every call)
WORKSPACE_BYTES = ppa_workspace_bytes()


def _stream_handle(device: torch.device, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def ppa_validate_metadata_device(params: PpaParams, result: torch.Tensor,
                                 stream: Union[int, "torch.cuda.Stream", None] = None) -> None:
    """Enqueue the device-side metadata check (ppa.h).  ``result`` is an
    int32 device tensor of two elements, 8-byte aligned; once the stream has
    passed the call it holds (status, request index or -1)."""
    if not (isinstance(result, torch.Tensor) and result.is_cuda and result.dtype == torch.int32
            and result.numel() >= 2 and result.is_contiguous()):
        raise ValueError("result must be a contiguous int32 device tensor of at least two elements")
    h = _stream_handle(result.device, stream)
    st = _lib.ppa_validate_metadata_device(ctypes.byref(params), c_void_p(result.data_ptr()), c_void_p(h))
    if st != 0:
        _, msg = ppa_validate_shapes(params)
        raise PpaError(st, msg or "result pointer")


def check_metadata_device(params: PpaParams, device: Optional[torch.device] = None,
                          stream: Union[int, "torch.cuda.Stream", None] = None) -> Tuple[int, int]:
    """Run ppa_validate_metadata_device and wait for it: (status, request)."""
    result = torch.empty(2, dtype=torch.int32, device=device or torch.device("cuda"))
    ppa_validate_metadata_device(params, result, stream)
    torch.cuda.synchronize(result.device)
    st, req = (int(x) for x in result.cpu())
    return st, req


def ppa_paged_prefill_attention(params: PpaParams, stream: Union[int, "torch.cuda.Stream", None] = None,
                                device: Optional[torch.device] = None) -> None:
    h = _stream_handle(device or torch.device("cuda"), stream)
    st = _lib.ppa_paged_prefill_attention(ctypes.byref(params), c_void_p(h))
    if st != 0:
        _, msg = ppa_validate_shapes(params)
        raise PpaError(st, msg)


def ppa_paged_prefill_attention_noalloc(params: PpaParams, stream: Union[int, "torch.cuda.Stream", None] = None,
                                        device: Optional[torch.device] = None) -> None:
    """The no-allocation entry point: params.workspace must be None; the
    library's per-device scratch array serves as the workspace."""
    h = _stream_handle(device or torch.device("cuda"), stream)
    st = _lib.ppa_paged_prefill_attention_noalloc(ctypes.byref(params), c_void_p(h))
    if st != 0:
        _, msg = ppa_validate_shapes(params)
        raise PpaError(st, msg)


def ppa_noalloc_scratch_bytes() -> int:
    return int(_lib.ppa_noalloc_scratch_bytes())


def ppa_gather_paged_kv(params: PpaParams, kv_idx: int, dst: torch.Tensor, stream=None) -> None:
    if not dst.is_contiguous():
        raise ValueError("dst must be contiguous")
    h = _stream_handle(dst.device, stream)
    st = _lib.ppa_gather_paged_kv(ctypes.byref(params), int(kv_idx), c_void_p(dst.data_ptr()),
                                  int(dst.shape[0]), c_void_p(h))
    if st != 0:
        _, msg = ppa_validate_shapes(params)
        raise PpaError(st, msg)


def ppa_merge_params_size() -> int:
    return int(_lib.ppa_merge_params_size())


def ppa_merge_attention_states(o_parts: torch.Tensor, lse_parts: torch.Tensor, out: torch.Tensor,
                               lse_out: Optional[torch.Tensor] = None, sinks: Optional[torch.Tensor] = None,
                               stream=None) -> None:
    """Log-sum-exp merge of partial states: ``o_parts`` fp32 ``[S, rows,
    heads, D]`` and ``lse_parts`` fp32 ``[S, rows, heads]`` (contiguous),
    into ``out`` (bf16 ``[rows, heads, D]`` or an ``MxFp4Output``) and optionally ``lse_out`` fp32
    ``[rows, heads]``; ``sinks`` fp32 ``[heads]`` adds one denominator term."""
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("o_parts and lse_parts must be float32")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    if o_parts.dim() != 4 or lse_parts.shape != o_parts.shape[:3]:
        raise ValueError("shapes: o_parts [S, rows, heads, D], lse_parts [S, rows, heads], out [rows, heads, D]")
    m = PpaMergeParams()
    m.abi_version = PPA_ABI_VERSION
    m.struct_size = ctypes.sizeof(PpaMergeParams)
    m.num_parts, m.num_rows, m.num_heads, m.head_dim = (int(x) for x in o_parts.shape)
    m.o_parts = _ptr(o_parts)
    m.lse_parts = _ptr(lse_parts)
    if sinks is not None:
        if sinks.dtype != torch.float32 or sinks.numel() != m.num_heads or not sinks.is_contiguous():
            raise ValueError("sinks must be a contiguous float32 tensor of num_heads values")
        m.sinks = _ptr(sinks)
    _set_out(m, out, o_parts.shape[1:])
    if lse_out is not None:
        if lse_out.dtype != torch.float32 or tuple(lse_out.shape) != tuple(o_parts.shape[1:3]):
            raise ValueError("lse_out must be float32 [rows, heads]")
        m.lse_out = _ptr(lse_out)
        m.lse_out_strides[:] = list(lse_out.stride())
    h = _stream_handle(o_parts.device, stream)
    st = _lib.ppa_merge_attention_states(ctypes.byref(m), c_void_p(h))
    if st != 0:
        raise PpaError(st, "merge arguments rejected")


def ppa_append_params_size() -> int:
    return int(_lib.ppa_append_params_size())


def make_append_params(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                       k_scale=1.0, v_scale=1.0) -> PpaAppendParams:
    """New tokens' K / V (bf16 ``[n, H_kv, D]``) and their int64 slots
    (``page * page_size + slot``; negative skips); scales are floats or
    one-element fp32 device tensors."""
    if k_new.dim() != 3 or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [num_new, num_kv_heads, head_dim] of one shape")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1 or not slot_mapping.is_contiguous():
        raise TypeError("slot_mapping must be a contiguous 1-D int64 tensor")
    if slot_mapping.numel() != k_new.shape[0]:
        raise ValueError("slot_mapping needs one entry per new token")
    a = PpaAppendParams()
    a.abi_version = PPA_ABI_VERSION
    a.struct_size = ctypes.sizeof(PpaAppendParams)
    a.k_new, a.v_new = _ptr(k_new), _ptr(v_new)
    a.new_dtype = _dt(k_new) if k_new.dtype == v_new.dtype else 0
    a.num_new = int(k_new.shape[0])
    a.k_new_strides[:] = list(k_new.stride())
    a.v_new_strides[:] = list(v_new.stride())
    a.slot_mapping = _ptr(slot_mapping)
    for name, val in (("k", k_scale), ("v", v_scale)):
        if isinstance(val, torch.Tensor):
            if val.dtype != torch.float32 or val.numel() != 1:
                raise TypeError(f"{name}_scale tensor must be one float32 element")
            setattr(a, f"{name}_scale_ptr", _ptr(val))
            setattr(a, f"{name}_scale", 0.0)
        else:
            setattr(a, f"{name}_scale", float(val))
    a._refs = (k_new, v_new, slot_mapping, k_scale, v_scale)   # the pointers' tensors, kept alive
    return a


def ppa_validate_append(cache: PpaParams, a: PpaAppendParams) -> Tuple[int, str]:
    buf = ctypes.create_string_buffer(512)
    st = _lib.ppa_validate_append(ctypes.byref(cache), ctypes.byref(a), buf, len(buf))
    return int(st), buf.value.decode()


def ppa_append_paged_kv(cache: PpaParams, a: PpaAppendParams, stream=None, device=None) -> None:
    h = _stream_handle(device or torch.device("cuda"), stream)
    st = _lib.ppa_append_paged_kv(ctypes.byref(cache), ctypes.byref(a), c_void_p(h))
    if st != 0:
        _, msg = ppa_validate_append(cache, a)
        raise PpaError(st, msg)


# --------------------------------------------------------------------------
# marshalling torch tensors -> ppa_params
# --------------------------------------------------------------------------

_DTYPES = {torch.bfloat16: PPA_DTYPE_BF16, torch.float8_e4m3fn: PPA_DTYPE_FP8_E4M3FN,
           torch.float32: PPA_DTYPE_FP32}


def _dt(t: torch.Tensor) -> int:
    return _DTYPES.get(t.dtype, 0)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.int32, torch.uint32):
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    if t.dim() == 1 and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _check_metadata(query, kv_cache, workspace_buffer, block_tables, seq_lens, cum_seq_lens_q, cum_seq_lens_kv,
                    kv_indptr, kv_indices, kv_last_page_len, out, sinks, lse, batch_size: int) -> None:
    """Every tensor on query's device, and every metadata array long enough
    for batch_size requests.  The kernel and the host checker read
    cum_seq_lens_q[b + 1], seq_lens[b], a block-table row or kv_indptr[b + 1]
    for every b < batch_size; the C ABI takes bare pointers and cannot see
    their lengths, so they are checked here."""
    B = int(batch_size)
    csr = kv_indptr is not None or kv_indices is not None
    if B < 0:
        raise ValueError(f"batch_size must be >= 0, got {B}")
    dev = query.device
    tensors = [("seq_lens", seq_lens), ("cum_seq_lens_q", cum_seq_lens_q), ("cum_seq_lens_kv", cum_seq_lens_kv),
               ("block_tables", block_tables), ("kv_indptr", kv_indptr), ("kv_indices", kv_indices),
               ("kv_last_page_len", kv_last_page_len), ("workspace_buffer", workspace_buffer), ("lse", lse)]
    if isinstance(kv_cache, (tuple, list)):
        tensors += [(f"kv_cache[{i}]", t) for i, t in enumerate(kv_cache) if isinstance(t, torch.Tensor)]
    else:
        tensors.append(("kv_cache", kv_cache))
    if isinstance(out, torch.Tensor):
        tensors.append(("out", out))
    elif isinstance(out, MxFp4Output):
        tensors += [("out.data", out.data), ("out.scale", out.scale)]
    if isinstance(sinks, torch.Tensor):
        tensors.append(("sinks", sinks))
    for name, t in tensors:
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, query on {dev}: every tensor must be on one device")
    need = [("seq_lens", seq_lens, B), ("cum_seq_lens_q", cum_seq_lens_q, B + 1),
            ("cum_seq_lens_kv", cum_seq_lens_kv, B + 1)]
    if csr:
        need += [("kv_indptr", kv_indptr, B + 1), ("kv_last_page_len", kv_last_page_len, B)]
    for name, t, n in need:
        if t is not None and t.numel() < n:
            raise ValueError(f"{name} has {t.numel()} entries; batch_size {B} needs at least {n}")
    if not csr and block_tables is not None and block_tables.dim() == 2 and block_tables.shape[0] < B:
        raise ValueError(f"block_tables has {block_tables.shape[0]} rows; batch_size {B} needs at least {B}")


def make_params(query: torch.Tensor, kv_cache, workspace_buffer: Optional[torch.Tensor],
                block_tables: Optional[torch.Tensor], seq_lens: torch.Tensor, max_q_len: int, max_kv_len: int,
                bmm1_scale, bmm2_scale, batch_size: int, cum_seq_lens_q: torch.Tensor,
                cum_seq_lens_kv: Optional[torch.Tensor], window_left: int, out: torch.Tensor,
                kv_layout: str = "HND", sinks=None, kv_indptr: Optional[torch.Tensor] = None,
                kv_indices: Optional[torch.Tensor] = None,
                kv_last_page_len: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                kv_splits: int = 0, fp8_compute: bool = False) -> PpaParams:
    """Fill a PpaParams from torch tensors (the FlashInfer API page's argument
    list).  With kv_indptr / kv_indices the flat (CSR) page table is used and
    block_tables may be None.  The returned PpaParams holds device pointers
    and keeps references to the tensors they point into (attribute
    ``_refs``), so that a params object launched later never reads memory
    the allocator has handed to another tensor; a copy of the struct
    (``from_buffer_copy``) does not carry them."""
    if query.dim() != 3:
        raise ValueError("query must be [num_tokens, num_qo_heads, head_dim]")
    _check_metadata(query, kv_cache, workspace_buffer, block_tables, seq_lens, cum_seq_lens_q, cum_seq_lens_kv,
                    kv_indptr, kv_indices, kv_last_page_len, out, sinks, lse, batch_size)
    p = PpaParams()
    p.abi_version = PPA_ABI_VERSION
    p.struct_size = ctypes.sizeof(PpaParams)
    p.query = _ptr(query)
    p.query_dtype = _dt(query)
    p.num_tokens, p.num_qo_heads, p.head_dim = (int(x) for x in query.shape)
    p.query_strides[:] = list(query.stride())

    layout = kv_layout.upper()
    if layout not in ("HND", "NHD"):
        raise ValueError(f"kv_layout must be 'HND' or 'NHD', got {kv_layout!r}")
    p.kv_layout = PPA_KV_LAYOUT_HND if layout == "HND" else PPA_KV_LAYOUT_NHD
    if isinstance(kv_cache, (tuple, list)):
        if len(kv_cache) != 2:
            raise ValueError("a kv_cache tuple must be (k_cache, v_cache)")
        k, v = kv_cache
        if k.dim() != 4 or v.dim() != 4 or k.shape != v.shape or k.dtype != v.dtype:
            raise ValueError("k_cache and v_cache must be 4-D tensors of one shape and dtype")
        p.kv_form = PPA_KV_SPLIT
        p.kv_dtype = _dt(k)
        p.k_cache, p.v_cache = _ptr(k), _ptr(v)
        p.k_cache_strides[:] = list(k.stride())
        p.v_cache_strides[:] = list(v.stride())
        n, a1, a2, d = (int(x) for x in k.shape)
        heads, page = (a1, a2) if layout == "HND" else (a2, a1)
    else:
        if kv_cache.dim() != 5:
            raise ValueError("a single kv_cache must be 5-D [num_pages, 1 or 2, ...]")
        p.kv_form = PPA_KV_COMBINED
        p.kv_dtype = _dt(kv_cache)
        p.kv_cache = _ptr(kv_cache)
        p.kv_cache_strides[:] = list(kv_cache.stride())
        n, planes, a1, a2, d = (int(x) for x in kv_cache.shape)
        p.kv_planes = planes
        heads, page = (a1, a2) if layout == "HND" else (a2, a1)
    if d != p.head_dim:
        raise ValueError(f"cache head_dim {d} != query head_dim {p.head_dim}")
    p.num_pages, p.num_kv_heads, p.page_size = n, heads, page

    if workspace_buffer is not None:
        p.workspace = _ptr(workspace_buffer)
        p.workspace_bytes = workspace_buffer.numel() * workspace_buffer.element_size()

    if kv_indptr is not None or kv_indices is not None:
        if kv_indptr is None or kv_indices is None:
            raise ValueError("the flat page table needs both kv_indptr and kv_indices")
        ip = _i32(kv_indptr, "kv_indptr")
        ix = _i32(kv_indices, "kv_indices")
        if ip.dim() != 1 or ix.dim() != 1:
            raise ValueError("kv_indptr and kv_indices must be 1-D")
        p.page_table_form = PPA_PAGE_TABLE_CSR
        p.kv_indptr = _ptr(ip)
        p.kv_indices = _ptr(ix)
        p.kv_indices_len = int(ix.numel())
        if kv_last_page_len is not None:
            p.kv_last_page_len = _ptr(_i32(kv_last_page_len, "kv_last_page_len"))
    if block_tables is not None:
        bt = _i32(block_tables, "block_tables")
        if bt.dim() != 2 or bt.stride(1) != 1:
            raise ValueError("block_tables must be [batch_size, cols] with unit column stride")
        p.block_tables = _ptr(bt)
        p.block_tables_cols = int(bt.shape[1])
        p.block_tables_row_stride = int(bt.stride(0))
    elif p.page_table_form != PPA_PAGE_TABLE_CSR:
        raise ValueError("block_tables is required unless kv_indptr / kv_indices are given")
    p.seq_lens = _ptr(_i32(seq_lens, "seq_lens"))
    p.cum_seq_lens_q = _ptr(_i32(cum_seq_lens_q, "cum_seq_lens_q"))
    p.cum_seq_lens_kv = None if cum_seq_lens_kv is None else _ptr(_i32(cum_seq_lens_kv, "cum_seq_lens_kv"))
    p.batch_size = int(batch_size)
    p.max_q_len = int(max_q_len)
    p.max_kv_len = int(max_kv_len)

    for name, val in (("bmm1", bmm1_scale), ("bmm2", bmm2_scale)):
        if isinstance(val, torch.Tensor):
            if val.dtype != torch.float32 or val.numel() != 1:
                raise TypeError(f"{name}_scale tensor must be one float32 element")
            setattr(p, f"{name}_scale_ptr", _ptr(val))
            setattr(p, f"{name}_scale", 0.0)
        else:
            setattr(p, f"{name}_scale", float(val))
    p.window_left = int(window_left)

    if sinks is not None:
        if isinstance(sinks, (list, tuple)):
            if len(sinks) != 1:
                raise ValueError("sinks: pass one float32 tensor of num_qo_heads values")
            sinks = sinks[0]
        if sinks.dtype != torch.float32 or sinks.numel() != p.num_qo_heads or not sinks.is_contiguous():
            raise ValueError("sinks must be a contiguous float32 tensor of num_qo_heads values")
        p.sinks = _ptr(sinks)

    _set_out(p, out, query.shape)
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(query.shape[:2]):
            raise ValueError("lse must be float32 [num_tokens, num_qo_heads]")
        p.lse = _ptr(lse)
        p.lse_strides[:] = list(lse.stride())
    p.kv_splits = int(kv_splits)
    p.fp8_compute = 1 if fp8_compute else 0
    p._refs = (query, kv_cache, workspace_buffer, block_tables, seq_lens, cum_seq_lens_q, cum_seq_lens_kv, out,
               sinks, kv_indptr, kv_indices, kv_last_page_len, lse, bmm1_scale, bmm2_scale)
    return p


def append_paged_kv_cache(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor, kv_cache,
                          kv_layout: str = "HND", k_scale=1.0, v_scale=1.0, stream=None) -> None:
    """Write new tokens' K and V into the paged cache at ``slot_mapping``
    (page * page_size + slot per token, negative skips).  fp8 caches store
    e4m3fn(x / scale), nearest-even, saturated at 448."""
    q_stub = torch.empty((1, 1, k_new.shape[2]), dtype=torch.bfloat16, device=k_new.device)
    i32 = torch.zeros(2, dtype=torch.int32, device=k_new.device)
    bt = torch.zeros((1, 1), dtype=torch.int32, device=k_new.device)
    cache = make_params(q_stub, kv_cache, None, bt, i32[:1], 0, 0, 1.0, 1.0, 0, i32, None, -1, q_stub, kv_layout)
    a = make_append_params(k_new, v_new, slot_mapping, k_scale, v_scale)
    ppa_append_paged_kv(cache, a, stream, k_new.device)


def batch_context_with_kv_cache(query: torch.Tensor, kv_cache, workspace_buffer: Optional[torch.Tensor],
                                block_tables: Optional[torch.Tensor], seq_lens: torch.Tensor, max_q_len: int,
                                max_kv_len: int, bmm1_scale, bmm2_scale, batch_size: int,
                                cum_seq_lens_q: torch.Tensor, cum_seq_lens_kv: Optional[torch.Tensor],
                                window_left: int = -1, out: Optional[torch.Tensor] = None,
                                out_dtype=None, kv_layout: str = "HND", sinks=None,
                                validate: bool = False, stream=None, kv_indptr=None, kv_indices=None,
                                kv_last_page_len=None, lse: Optional[torch.Tensor] = None,
                                kv_splits: Union[int, str] = 0, o_sf_scale: Optional[float] = None,
                                o_sf_vec_size: Optional[int] = None, fp8_compute: bool = False,
                                noalloc: bool = False):
    """Batched paged prefill attention; argument list of the API page
    (without the PDL option), plus the optional flat page table (kv_indptr /
    kv_indices / kv_last_page_len) in place of block_tables, an optional fp32
    ``lse`` [num_tokens, num_qo_heads] output (natural-log softmax
    denominators) and ``kv_splits`` (split-KV; needs a workspace of
    ``ppa_workspace_bytes`` bytes; ``"auto"``: the library's planner picks
    it from the shapes, the device and the workspace size).  The FP4 output of the API page is given
    as OCP MXFP4: ``out_dtype="mxfp4"`` (or an ``MxFp4Output`` as ``out``)
    with ``o_sf_scale`` (default 1) and ``o_sf_vec_size`` (16 or 32, default
    32) returns an ``MxFp4Output``.  ``fp8_compute=True`` (fp8 cache,
    head_dim 128) rounds Q and the softmax weights to e4m3fn and runs both
    products on the fp8 MFMA.  ``validate=True`` also runs the deep
    metadata check on host copies (a device-to-host sync).  ``noalloc=True``
    calls the no-allocation entry point (``workspace_buffer`` must be None:
    the library's per-device scratch array takes its place)."""
    if isinstance(out_dtype, str):
        if out_dtype.lower() != "mxfp4":
            raise ValueError(f"out_dtype {out_dtype!r}: the FP4 output here is 'mxfp4' (OCP MX, E8M0 scales)")
        if out is None:
            out = empty_mxfp4(query.shape[0], query.shape[1], query.shape[2], query.device,
                              32 if o_sf_vec_size is None else int(o_sf_vec_size),
                              1.0 if o_sf_scale is None else float(o_sf_scale))
    if out is None:
        dt = query.dtype if out_dtype is None else out_dtype
        out = torch.empty(query.shape, dtype=dt, device=query.device)
    auto = isinstance(kv_splits, str)
    if auto and kv_splits != "auto":
        raise ValueError(f"kv_splits {kv_splits!r}: an int or 'auto'")
    p = make_params(query, kv_cache, workspace_buffer, block_tables, seq_lens, max_q_len, max_kv_len,
                    bmm1_scale, bmm2_scale, batch_size, cum_seq_lens_q, cum_seq_lens_kv, window_left,
                    out, kv_layout, sinks, kv_indptr, kv_indices, kv_last_page_len, lse, 0 if auto else kv_splits,
                    fp8_compute)
    if auto:
        with torch.cuda.device(query.device):
            p.kv_splits = ppa_plan_kv_splits(p)
    if validate:
        st, msg = ppa_validate_metadata_host(p, cum_seq_lens_q, cum_seq_lens_kv, seq_lens, block_tables)
        if st == 0 and p.page_table_form == PPA_PAGE_TABLE_CSR:
            st, msg = ppa_validate_page_table_csr_host(p, seq_lens, kv_indptr, kv_indices, kv_last_page_len)
        if st != 0:
            raise PpaError(st, msg)
    if noalloc:
        ppa_paged_prefill_attention_noalloc(p, stream, query.device)
    else:
        ppa_paged_prefill_attention(p, stream, query.device)
    return out
