"""CPU oracle: batched causal prefill attention over a paged KV cache.

TEST INFRASTRUCTURE.  This module is the slow, plain reference that the GPU
path is checked against.  Only the test suite, the smoke check and the
bench's CPU-baseline leg may import or run it; the library itself never
does, and it shares no code with the HIP path.

Everything is computed in float64 with NumPy, one request and one query head
at a time, in the order the pages define the operation:

1. decode the stored codes (bf16, or OCP float8 e4m3fn) to real values;
2. gather each request's pages into a contiguous token-major K and V of
   shape ``[kv_len, H_kv, D]`` - the VanillaAttention ``_gather_paged_kv``
   step of the TensorRT-LLM attention-backend article (section "path 1:
   VanillaAttention"), with a page id from ``block_tables[b, t // P]`` and the
   slot ``t % P`` (FlashInfer API page, parameters ``kv_cache`` and
   ``block_tables``; article section "physical meaning of handle -> offset"),
   or, for the flat page table, from ``kv_indices[kv_indptr[b] + t // P]``
   (article section on why FlashInfer uses a flat index array with an
   indptr rather than a 2-D table);
3. for each query head, logits ``bmm1_scale * q . k`` (API page, parameter
   ``bmm1_scale``);
4. the causal mask with the new queries at the end of the KV sequence
   (``kv_len = cached prefix + new tokens``, article section on
   TrtllmAttentionMetadata, and the chunked-context figure) and the inclusive
   left window (API page, parameter ``window_left``; -1 means no window);
5. softmax over the valid keys, with the per-head sink as an extra term of
   the denominator only (API page, parameter ``sinks``);
6. the weighted sum of V rows, times ``bmm2_scale`` (API page, parameter
   ``bmm2_scale``).

Readings taken where the pages are silent (each is listed with its reason in
the design notes): GQA query head h reads kv head ``h // (H_q / H_kv)``; a
sink is a logit in the same natural-log units as ``bmm1_scale * q . k``;
a combined cache with one plane in dim 1 holds K and V in the same storage.
Parity unpinned: the GQA head mapping and the units of the sink are
conventions that no page prints a value for; they are pinned only against
torch's SDPA grouping convention and against closed forms.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple, Union

import numpy as np

# ---------------------------------------------------------------------------
# 1. Decoding stored codes
# ---------------------------------------------------------------------------


def decode_bf16(codes: np.ndarray) -> np.ndarray:
    """bf16 codes (uint16) -> float64.  A bf16 number is the upper half of an
    IEEE binary32, so shifting the code into the top 16 bits is exact."""
    c = np.asarray(codes, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # NaN codes stay NaN
        return c.view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """One OCP float8 e4m3fn code -> its real value (OCP 8-bit floating point
    specification): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there
    is no infinity, so the largest magnitude is 1.75 * 2^8 = 448."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """float8 e4m3fn codes (uint8) -> float64 by table lookup."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3fn(y: np.ndarray) -> np.ndarray:
    """Real values -> OCP float8 e4m3fn codes: the nearest representable
    value, ties to the even code (the even mantissa), magnitudes beyond the
    largest finite value 448 saturated to it, NaN to the NaN code with the
    input's sign.  ``y`` is taken exactly (pass the fp32 value to encode)."""
    y = np.asarray(y, dtype=np.float64)
    grid = E4M3FN_TABLE[:127]           # codes 0x00 .. 0x7E, ascending, 0 .. 448
    a = np.minimum(np.abs(y), grid[-1])
    hi = np.searchsorted(grid, a, side="left")          # first grid value >= a
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(np.isnan(y), np.uint8(0x7F), code)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


# ---------------------------------------------------------------------------
# 2. Page gather
# ---------------------------------------------------------------------------


def _plane(kv_cache, kv_idx: int) -> np.ndarray:
    """The K (kv_idx 0) or V (kv_idx 1) page pool of a decoded cache.

    A tuple is (K pool, V pool).  A single array has the K/V planes in dim 1;
    with only one plane there, K and V are read from the same storage."""
    if isinstance(kv_cache, (tuple, list)):
        return kv_cache[kv_idx]
    nplanes = kv_cache.shape[1]
    return kv_cache[:, kv_idx if nplanes == 2 else 0]


def _page_rows(plane: np.ndarray, page_id: int, nslots: int, kv_layout: str) -> np.ndarray:
    """The first ``nslots`` token rows of one page as ``[nslots, H_kv, D]``.
    HND pages are ``[H_kv, P, D]``; NHD pages are ``[P, H_kv, D]``."""
    page = plane[page_id]
    if kv_layout == "HND":
        return np.transpose(page[:, :nslots, :], (1, 0, 2))
    if kv_layout == "NHD":
        return page[:nslots]
    raise ValueError(f"kv_layout must be HND or NHD, got {kv_layout!r}")


def gather_paged_kv(kv_cache, block_ids: Sequence[int], kv_idx: int, num_tokens: int,
                    page_size: int, kv_layout: str) -> np.ndarray:
    """The first ``num_tokens`` logical K or V tokens of one request as a
    contiguous ``[num_tokens, H_kv, D]`` array: logical token t lives in page
    ``block_ids[t // page_size]`` at slot ``t % page_size``."""
    plane = _plane(kv_cache, kv_idx)
    rows = []
    npages = (num_tokens + page_size - 1) // page_size
    for j in range(npages):
        nslots = min(page_size, num_tokens - j * page_size)
        rows.append(_page_rows(plane, int(block_ids[j]), nslots, kv_layout))
    if not rows:
        return np.zeros((0,) + plane.shape[2:] if kv_layout == "NHD" else
                        (0, plane.shape[1], plane.shape[3]), dtype=plane.dtype)
    return np.concatenate(rows, axis=0)


# ---------------------------------------------------------------------------
# 3-6. Attention for one request
# ---------------------------------------------------------------------------


def _kv_head(h: int, num_qo_heads: int, num_kv_heads: int) -> int:
    """GQA: the kv head that query head h reads (contiguous groups)."""
    return h // (num_qo_heads // num_kv_heads)


def _valid_mask(q_len: int, kv_len: int, window_left: int) -> np.ndarray:
    """``[q_len, kv_len]`` bool.  Query row i sits at sequence position
    ``prefix + i`` with ``prefix = kv_len - q_len``; it sees key j when
    ``j <= prefix + i`` and, for ``window_left >= 0``, ``j >= prefix + i -
    window_left`` (the left window is inclusive)."""
    prefix = kv_len - q_len
    i = np.arange(q_len)[:, None]
    j = np.arange(kv_len)[None, :]
    pos = prefix + i
    valid = j <= pos
    if window_left >= 0:
        valid &= j >= pos - window_left
    return valid


def _softmax_weighted_sum(s: np.ndarray, valid: np.ndarray, v: np.ndarray,
                          sink: Optional[float]) -> np.ndarray:
    """Softmax of the valid logits of each row, the sink (if any) adding
    ``exp(sink)`` to the denominator only, then the weighted sum of V rows.
    The row maximum (taken over the valid logits and the sink) is subtracted
    before exponentiating; that leaves every ratio unchanged."""
    s = np.where(valid, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    if sink is not None:
        m = np.maximum(m, sink)
    p = np.where(valid, np.exp(s - m[:, None]), 0.0)
    denom = p.sum(axis=1)
    if sink is not None:
        denom = denom + np.exp(sink - m)
    return (p @ v) / denom[:, None]


def attention_one_request(q: np.ndarray, k: np.ndarray, v: np.ndarray, bmm1_scale: float,
                          bmm2_scale: float, window_left: int,
                          sinks: Optional[np.ndarray], chunk: int = 256) -> np.ndarray:
    """q ``[q_len, H_q, D]``, contiguous k and v ``[kv_len, H_kv, D]`` ->
    ``[q_len, H_q, D]``.  Query rows are taken ``chunk`` at a time to bound
    memory; keys past the chunk's last causal position are masked for every
    row of the chunk and are left out."""
    q_len, num_qo_heads, _ = q.shape
    kv_len, num_kv_heads, head_dim = k.shape
    out = np.empty((q_len, num_qo_heads, v.shape[2]), dtype=np.float64)
    prefix = kv_len - q_len
    full_mask = _valid_mask(q_len, kv_len, window_left)
    for h in range(num_qo_heads):
        hk = _kv_head(h, num_qo_heads, num_kv_heads)
        sink = None if sinks is None else float(sinks[h])
        for r0 in range(0, q_len, chunk):
            r1 = min(q_len, r0 + chunk)
            hi = min(kv_len, prefix + r1)
            s = bmm1_scale * (q[r0:r1, h, :] @ k[:hi, hk, :].T)
            o = _softmax_weighted_sum(s, full_mask[r0:r1, :hi], v[:hi, hk, :], sink)
            out[r0:r1, h, :] = bmm2_scale * o
    return out


def request_pages(b: int, block_tables: Optional[np.ndarray], kv_indptr: Optional[np.ndarray] = None,
                  kv_indices: Optional[np.ndarray] = None) -> np.ndarray:
    """Page ids of request b: row b of the padded table, or the slice
    ``kv_indices[kv_indptr[b]:kv_indptr[b + 1]]`` of the flat one."""
    if kv_indptr is not None:
        return np.asarray(kv_indices)[int(kv_indptr[b]):int(kv_indptr[b + 1])]
    return np.asarray(block_tables[b])


def append_paged_kv(planes, kv_layout: str, page_size: int, k_new_codes: np.ndarray, v_new_codes: np.ndarray,
                    slot_mapping: np.ndarray, kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0):
    """Write new tokens' K and V into a paged cache (the KV save step before
    attention: TokenSpeed backend source, ``_save_kv_and_prepare_q`` with
    ``out_cache_loc``): token i goes to page ``slot_mapping[i] // page_size``,
    slot ``slot_mapping[i] % page_size``; a negative entry skips the token.
    ``planes`` are the cache's K and V code arrays (one array for both when
    they share storage), ``k_new_codes`` / ``v_new_codes`` bf16 codes
    ``[n, H_kv, D]``.  A bf16 cache stores the codes as they are; an fp8
    cache stores ``encode_e4m3fn(fp32(x) / fp32(scale))``.  Returns new code
    arrays; the inputs are not modified."""
    out = [np.array(p, copy=True) for p in planes]
    for kv_idx, (new, scale) in enumerate(((k_new_codes, k_scale), (v_new_codes, v_scale))):
        dst = out[min(kv_idx, len(out) - 1)]
        if kv_dtype == "bf16":
            vals = np.asarray(new, dtype=np.uint16)
        else:
            x = decode_bf16(new).astype(np.float32)
            vals = encode_e4m3fn(x / np.float32(scale))
        for i, loc in enumerate(np.asarray(slot_mapping)):
            loc = int(loc)
            if loc < 0:
                continue
            pid, slot = loc // page_size, loc % page_size
            if kv_layout == "HND":
                dst[pid, :, slot, :] = vals[i]
            else:
                dst[pid, slot, :, :] = vals[i]
    return out


# ---------------------------------------------------------------------------
# 4. Log-sum-exp, partial states and their merge
# ---------------------------------------------------------------------------
#
# The softmax denominator of a row, kept as its natural logarithm, is what
# lets attention over a split key set be recombined: a partial state is the
# normalized output and log-denominator over a subset of the keys; merging
# weights each part by exp(lse_part - lse_total).  Read from the sibling
# decode call of the TokenSpeed backend source (the decode path of the
# TRT-LLM MHA backend), which splits the key set and merges; the sink, a term
# of the denominator only (API page, parameter sinks), is added once, at
# the merge.


def log_sum_exp_rows(s: np.ndarray, valid: np.ndarray, sink: Optional[float]) -> np.ndarray:
    """``log(sum_valid exp(s_ij) [+ exp(sink)])`` per row; -inf for a row
    with no valid key and no sink."""
    s = np.where(valid, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    if sink is not None:
        m = np.maximum(m, sink)
    finite = np.isfinite(m)
    mm = np.where(finite, m, 0.0)
    tot = np.where(valid, np.exp(s - mm[:, None]), 0.0).sum(axis=1)
    if sink is not None:
        tot = tot + np.exp(sink - mm)
    with np.errstate(divide="ignore"):
        return np.where(finite, mm + np.log(tot), -np.inf)


def partial_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, bmm1_scale: float, bmm2_scale: float,
                  window_left: int, key_begin: int, key_end: int) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of one request restricted to the keys in ``[key_begin,
    key_end)`` (and the causal / window mask), without sinks: ``(o, lse)``
    with ``o`` ``[q_len, H_q, D]`` normalized over that key subset (times
    bmm2) and ``lse`` ``[q_len, H_q]``.  A row with no valid key in the
    subset gets ``o = 0`` and ``lse = -inf``."""
    q_len, num_qo_heads, _ = q.shape
    kv_len, num_kv_heads, _ = k.shape
    mask = _valid_mask(q_len, kv_len, window_left)
    sub = np.zeros(kv_len, dtype=bool)
    sub[max(0, key_begin):max(0, min(kv_len, key_end))] = True
    mask = mask & sub[None, :]
    o = np.zeros((q_len, num_qo_heads, v.shape[2]), dtype=np.float64)
    lse = np.full((q_len, num_qo_heads), -np.inf, dtype=np.float64)
    rows = mask.any(axis=1)
    for h in range(num_qo_heads):
        hk = _kv_head(h, num_qo_heads, num_kv_heads)
        s = bmm1_scale * (q[:, h, :] @ k[:, hk, :].T)
        lse[:, h] = log_sum_exp_rows(s, mask, None)
        if rows.any():
            o[rows, h, :] = bmm2_scale * _softmax_weighted_sum(s[rows], mask[rows], v[:, hk, :], None)
    return o, lse


def merge_states(o_parts: np.ndarray, lse_parts: np.ndarray,
                 sink: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Merge S partial states: ``o_parts`` ``[S, ..., D]``, ``lse_parts``
    ``[S, ...]``; ``sink`` (broadcast against ``lse_parts[0]``) is one more
    term of the total denominator.  ``lse = log(sum_s exp(lse_s) [+
    exp(sink)])`` and ``o = sum_s exp(lse_s - lse) o_s``."""
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    terms = lse_parts if sink is None else np.concatenate(
        [lse_parts, np.broadcast_to(np.asarray(sink, dtype=np.float64), lse_parts.shape[1:])[None]], axis=0)
    m = terms.max(axis=0)
    finite = np.isfinite(m)
    mm = np.where(finite, m, 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, mm + np.log(np.exp(terms - mm).sum(axis=0)), -np.inf)
    w = np.where(finite[None], np.exp(lse_parts - np.where(finite, lse, 0.0)[None]), 0.0)
    o = (w[..., None] * np.asarray(o_parts, dtype=np.float64)).sum(axis=0)
    return o, lse


def paged_prefill_lse(query: np.ndarray, kv_cache, kv_layout: str, block_tables: Optional[np.ndarray],
                      seq_lens: np.ndarray, cum_seq_lens_q: np.ndarray, page_size: int, bmm1_scale: float,
                      bmm2_scale: float, window_left: int = -1, sinks: Optional[np.ndarray] = None,
                      kv_indptr: Optional[np.ndarray] = None, kv_indices: Optional[np.ndarray] = None,
                      requests: Optional[Sequence[int]] = None, chunk: int = 256) -> np.ndarray:
    """``[num_tokens, H_q]`` natural-log softmax denominators of the batched
    call (sink included); NaN in rows no request owns."""
    num_tokens, num_qo_heads, _ = query.shape
    lse = np.full((num_tokens, num_qo_heads), np.nan, dtype=np.float64)
    todo = range(len(seq_lens)) if requests is None else requests
    for b in todo:
        q0, q1 = int(cum_seq_lens_q[b]), int(cum_seq_lens_q[b + 1])
        q_len, kv_len = q1 - q0, int(seq_lens[b])
        if q_len == 0:
            continue
        pages = request_pages(b, block_tables, kv_indptr, kv_indices)
        k = gather_paged_kv(kv_cache, pages, 0, kv_len, page_size, kv_layout)
        mask = _valid_mask(q_len, kv_len, window_left)
        num_kv_heads = k.shape[1]
        for h in range(num_qo_heads):
            hk = _kv_head(h, num_qo_heads, num_kv_heads)
            sink = None if sinks is None else float(sinks[h])
            for r0 in range(0, q_len, chunk):
                r1 = min(q_len, r0 + chunk)
                s = bmm1_scale * (query[q0 + r0:q0 + r1, h, :] @ k[:, hk, :].T)
                lse[q0 + r0:q0 + r1, h] = log_sum_exp_rows(s, mask[r0:r1], sink)
    return lse


def paged_prefill_attention(query: np.ndarray, kv_cache, kv_layout: str,
                            block_tables: Optional[np.ndarray], seq_lens: np.ndarray,
                            cum_seq_lens_q: np.ndarray, page_size: int,
                            bmm1_scale: float, bmm2_scale: float,
                            window_left: int = -1,
                            sinks: Optional[np.ndarray] = None,
                            requests: Optional[Sequence[int]] = None,
                            chunk: int = 256, kv_indptr: Optional[np.ndarray] = None,
                            kv_indices: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The whole batched call on decoded float64 inputs.

    ``query`` ``[num_tokens, H_q, D]``; ``kv_cache`` a (K, V) tuple of page
    pools or one array with the K/V planes in dim 1, laid out per
    ``kv_layout``; ``block_tables`` ``[batch, W]`` (or None with the flat
    ``kv_indptr`` / ``kv_indices``); ``seq_lens`` the KV length of each
    request (cached prefix included); ``cum_seq_lens_q`` ``[batch + 1]``.  Returns ``(out, written)``: ``out`` ``[num_tokens, H_q,
    D]`` float64 with NaN in rows no request owns, and ``written`` the bool
    row mask.  ``requests`` restricts the work to some requests (the other
    rows stay NaN / unwritten)."""
    num_tokens, num_qo_heads, head_dim = query.shape
    batch = len(seq_lens)
    out = np.full((num_tokens, num_qo_heads, head_dim), np.nan, dtype=np.float64)
    written = np.zeros(num_tokens, dtype=bool)
    todo = range(batch) if requests is None else requests
    for b in todo:
        q0, q1 = int(cum_seq_lens_q[b]), int(cum_seq_lens_q[b + 1])
        q_len = q1 - q0
        kv_len = int(seq_lens[b])
        if q_len == 0:
            continue
        if q_len > kv_len:
            raise ValueError(f"request {b}: q_len {q_len} > kv_len {kv_len}")
        pages = request_pages(b, block_tables, kv_indptr, kv_indices)
        k = gather_paged_kv(kv_cache, pages, 0, kv_len, page_size, kv_layout)
        v = gather_paged_kv(kv_cache, pages, 1, kv_len, page_size, kv_layout)
        out[q0:q1] = attention_one_request(query[q0:q1], k, v, bmm1_scale, bmm2_scale,
                                           window_left, sinks, chunk)
        written[q0:q1] = True
    return out, written


def attention_rows(query: np.ndarray, kv_cache, kv_layout: str, block_tables: Optional[np.ndarray],
                   seq_lens: np.ndarray, cum_seq_lens_q: np.ndarray, page_size: int,
                   bmm1_scale: float, bmm2_scale: float, window_left: int,
                   sinks: Optional[np.ndarray], rows: Sequence[Tuple[int, int]],
                   kv_indptr: Optional[np.ndarray] = None,
                   kv_indices: Optional[np.ndarray] = None) -> np.ndarray:
    """Selected output rows, one (token, q head) pair at a time: ``[len(rows),
    D]``.  Used to check full-size runs on a sample of outputs."""
    num_tokens, num_qo_heads, head_dim = query.shape
    num_kv_heads = _plane(kv_cache, 0).shape[2 if kv_layout == "NHD" else 1]
    cu = np.asarray(cum_seq_lens_q)
    res = np.empty((len(rows), head_dim), dtype=np.float64)
    cache = {}
    for n, (t, h) in enumerate(rows):
        b = int(np.searchsorted(cu, t, side="right") - 1)
        q0 = int(cu[b])
        kv_len = int(seq_lens[b])
        q_len = int(cu[b + 1]) - q0
        i = t - q0
        if b not in cache:
            pages = request_pages(b, block_tables, kv_indptr, kv_indices)
            cache[b] = (gather_paged_kv(kv_cache, pages, 0, kv_len, page_size, kv_layout),
                        gather_paged_kv(kv_cache, pages, 1, kv_len, page_size, kv_layout))
        k, v = cache[b]
        hk = _kv_head(h, num_qo_heads, num_kv_heads)
        valid = _valid_mask(q_len, kv_len, window_left)[i:i + 1]
        s = bmm1_scale * (query[t:t + 1, h, :] @ k[:, hk, :].T)
        sink = None if sinks is None else float(sinks[h])
        res[n] = bmm2_scale * _softmax_weighted_sum(s, valid, v[:, hk, :], sink)[0]
    return res
