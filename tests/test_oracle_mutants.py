"""Planted mistakes in the CPU oracle must each trip at least one pin.

Every mutant below swaps one step of the oracle (on the CPU, via
monkeypatch) for a plausible wrong version: an off-by-one in the mask, the
wrong causal alignment, a wrong GQA mapping, a mishandled sink, a wrong page
slot or layout, V read from the K plane, a wrong number decoder, a dropped
scale.  The test runs every pin against the mutated oracle and requires at
least one to fail, so the pins are shown to constrain each step.
"""
import numpy as np
import pytest

import oracle.paged_attention as OA
import oracle_pins

_orig_mask = OA._valid_mask
_orig_softmax = OA._softmax_weighted_sum
_orig_attn = OA.attention_one_request
_orig_rows = OA._page_rows
_orig_plane = OA._plane


def _mask_variant(cond):
    def f(q_len, kv_len, window_left):
        prefix = kv_len - q_len
        i = np.arange(q_len)[:, None]
        j = np.arange(kv_len)[None, :]
        return cond(i, j, prefix, window_left)
    return f


MUTANTS = {
    "top_left_causal": ("_valid_mask", _mask_variant(
        lambda i, j, p, w: (j <= i) & ((w < 0) | (j >= i - w)))),
    "strict_causal": ("_valid_mask", _mask_variant(
        lambda i, j, p, w: (j < p + i) & ((w < 0) | (j >= p + i - w)))),
    "window_exclusive": ("_valid_mask", _mask_variant(
        lambda i, j, p, w: (j <= p + i) & ((w < 0) | (j > p + i - w)))),
    "window_one_wider": ("_valid_mask", _mask_variant(
        lambda i, j, p, w: (j <= p + i) & ((w < 0) | (j >= p + i - w - 1)))),
    "gqa_modulo": ("_kv_head", lambda h, hq, hkv: h % hkv),
    "sink_ignored": ("_softmax_weighted_sum",
                     lambda s, valid, v, sink: _orig_softmax(s, valid, v, None)),
    "sink_unshifted": ("_softmax_weighted_sum", None),   # filled below
    "sink_as_value_row": ("_softmax_weighted_sum", None),
    "bmm2_dropped": ("attention_one_request",
                     lambda q, k, v, b1, b2, w, s, chunk=256: _orig_attn(q, k, v, b1, 1.0, w, s, chunk)),
    "bmm1_dropped": ("attention_one_request",
                     lambda q, k, v, b1, b2, w, s, chunk=256: _orig_attn(q, k, v, 1.0, b2, w, s, chunk)),
    "slot_shift": ("_page_rows", None),
    "hnd_reshaped_not_transposed": ("_page_rows", None),
    "v_from_k_plane": ("_plane", lambda kv, idx: _orig_plane(kv, 0)),
    "e4m3_bias_8": ("E4M3FN_TABLE", None),
    "bf16_shift_15": ("decode_bf16", None),
}


def _sink_unshifted(s, valid, v, sink):
    s = np.where(valid, s, -np.inf)
    m = s.max(axis=1)
    p = np.where(valid, np.exp(s - m[:, None]), 0.0)
    den = p.sum(axis=1) + (np.exp(sink) if sink is not None else 0.0)
    return (p @ v) / den[:, None]


def _sink_as_value_row(s, valid, v, sink):
    if sink is None:
        return _orig_softmax(s, valid, v, None)
    s2 = np.concatenate([s, np.full((s.shape[0], 1), sink)], axis=1)
    valid2 = np.concatenate([valid, np.ones((s.shape[0], 1), dtype=bool)], axis=1)
    v2 = np.concatenate([v, np.ones((1, v.shape[1]))], axis=0)
    return _orig_softmax(s2, valid2, v2, None)


def _slot_shift(plane, page_id, nslots, kv_layout):
    page = plane[page_id]
    P = page.shape[1] if kv_layout == "HND" else page.shape[0]
    idx = (np.arange(nslots) + 1) % P
    if kv_layout == "HND":
        return np.transpose(page[:, idx, :], (1, 0, 2))
    return page[idx]


def _hnd_reshaped(plane, page_id, nslots, kv_layout):
    page = plane[page_id]
    if kv_layout == "HND":
        H, P, D = page.shape
        return page.reshape(P, H, D)[:nslots]
    return page[:nslots]


def _bad_table():
    t = []
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 15 and m == 7:
            t.append(np.nan)
        elif e == 0:
            t.append(sign * m / 8 * 2.0 ** -7)
        else:
            t.append(sign * (1 + m / 8) * 2.0 ** (e - 8))
    return np.array(t)


def _bf16_shift_15(codes):
    c = np.asarray(codes, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    with np.errstate(invalid="ignore"):
        return c.view(np.float32).astype(np.float64)


MUTANTS["sink_unshifted"] = ("_softmax_weighted_sum", _sink_unshifted)
MUTANTS["sink_as_value_row"] = ("_softmax_weighted_sum", _sink_as_value_row)
MUTANTS["slot_shift"] = ("_page_rows", _slot_shift)
MUTANTS["hnd_reshaped_not_transposed"] = ("_page_rows", _hnd_reshaped)
MUTANTS["e4m3_bias_8"] = ("E4M3FN_TABLE", _bad_table())
MUTANTS["bf16_shift_15"] = ("decode_bf16", _bf16_shift_15)
_orig_pages = OA.request_pages


def _flat_off_by_one(b, block_tables, kv_indptr=None, kv_indices=None):
    # the flat table read one entry late (indptr taken as exclusive start)
    if kv_indptr is not None:
        return np.asarray(kv_indices)[int(kv_indptr[b]) + 1:int(kv_indptr[b + 1]) + 1]
    return _orig_pages(b, block_tables)


MUTANTS["flat_table_off_by_one"] = ("request_pages", _flat_off_by_one)
_orig_lse = OA.log_sum_exp_rows
_orig_merge = OA.merge_states
_orig_partial = OA.partial_state
MUTANTS["lse_in_log2_units"] = ("log_sum_exp_rows", lambda s, valid, sink: _orig_lse(s, valid, sink) / np.log(2.0))
MUTANTS["lse_sink_ignored"] = ("log_sum_exp_rows", lambda s, valid, sink: _orig_lse(s, valid, None))
MUTANTS["merge_sink_ignored"] = ("merge_states", lambda o, lse, sink=None: _orig_merge(o, lse, None))
MUTANTS["merge_plain_mean"] = ("merge_states",
                               lambda o, lse, sink=None: (np.mean(o, axis=0), _orig_merge(o, lse, sink)[1]))
_orig_encode = OA.encode_e4m3fn


def _encode_truncating(y):
    # rounds toward zero instead of to nearest
    y = np.asarray(y, dtype=np.float64)
    grid = OA.E4M3FN_TABLE[:127]
    code = np.clip(np.searchsorted(grid, np.minimum(np.abs(y), 448.0), side="right") - 1, 0, 126).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code)


MUTANTS["encode_truncates"] = ("encode_e4m3fn", _encode_truncating)
MUTANTS["encode_ties_away"] = ("encode_e4m3fn", lambda y: _orig_encode(np.asarray(y, dtype=np.float64) * (1 + 1e-12)))
MUTANTS["partial_ignores_key_range"] = ("partial_state",
                                        lambda q, k, v, b1, b2, w, k0, k1: _orig_partial(q, k, v, b1, b2, w, 0,
                                                                                         k.shape[0]))

_orig_append = OA.append_paged_kv


def _rows_lookup_left(query, kv_cache, kv_layout, block_tables, seq_lens, cum_seq_lens_q, page_size,
                      bmm1_scale, bmm2_scale, window_left, sinks, rows, kv_indptr=None, kv_indices=None):
    # the row-sampling entry with its request lookup taken on the wrong side
    # of the boundary: a row at the first token of a request (and every row
    # after an empty request) is computed as a row of an earlier request
    num_qo_heads = query.shape[1]
    cu = np.asarray(cum_seq_lens_q)
    res = np.empty((len(rows), query.shape[2]))
    for n, (t, h) in enumerate(rows):
        b = max(int(np.searchsorted(cu, t, side="left") - 1), 0)
        q0, kv_len = int(cu[b]), int(seq_lens[b])
        q_len = int(cu[b + 1]) - q0
        i = min(t - q0, q_len - 1)
        pages = OA.request_pages(b, block_tables, kv_indptr, kv_indices)
        k = OA.gather_paged_kv(kv_cache, pages, 0, kv_len, page_size, kv_layout)
        v = OA.gather_paged_kv(kv_cache, pages, 1, kv_len, page_size, kv_layout)
        hk = OA._kv_head(h, num_qo_heads, k.shape[1])
        valid = OA._valid_mask(q_len, kv_len, window_left)[i:i + 1]
        s = bmm1_scale * (query[t:t + 1, h, :] @ k[:, hk, :].T)
        sink = None if sinks is None else float(sinks[h])
        res[n] = bmm2_scale * OA._softmax_weighted_sum(s, valid, v[:, hk, :], sink)[0]
    return res


def _append_hnd_as_nhd(planes, kv_layout, page_size, k_new_codes, v_new_codes, slot_mapping, kv_dtype,
                       k_scale=1.0, v_scale=1.0):
    # an HND page addressed as if its memory were [slot, head, dim]: the
    # page reshaped instead of indexed [head, slot], so tokens land in the
    # wrong (head, slot) cells without any shape error
    if kv_layout != "HND":
        return _orig_append(planes, kv_layout, page_size, k_new_codes, v_new_codes, slot_mapping, kv_dtype,
                            k_scale, v_scale)
    out = [np.array(p, copy=True) for p in planes]
    for kv_idx, (new, scale) in enumerate(((k_new_codes, k_scale), (v_new_codes, v_scale))):
        dst = out[min(kv_idx, len(out) - 1)]
        if kv_dtype == "bf16":
            vals = np.asarray(new, dtype=np.uint16)
        else:
            vals = OA.encode_e4m3fn(OA.decode_bf16(new).astype(np.float32) / np.float32(scale))
        for i, loc in enumerate(np.asarray(slot_mapping)):
            if loc < 0:
                continue
            pid, slot = int(loc) // page_size, int(loc) % page_size
            H, P, D = dst.shape[1:]
            page = dst[pid].reshape(P, H, D)
            page[slot] = vals[i]
            dst[pid] = page.reshape(H, P, D)
    return out


MUTANTS["rows_request_lookup_off_by_one"] = ("attention_rows", _rows_lookup_left)
MUTANTS["append_hnd_as_nhd"] = ("append_paged_kv", _append_hnd_as_nhd)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, repl = MUTANTS[name]
    monkeypatch.setattr(OA, attr, repl)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception as exc:  # an AssertionError, or the mutant breaking outright
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin detects the planted mistake {name!r}"


# ---- MXFP4 output encoding (oracle.mxfp4) -----------------------------------

import oracle.mxfp4 as MX  # noqa: E402

_mx_encode = MX.encode_e2m1
_mx_scale = MX.mx_scale_byte
_mx_quant = MX.quantize_mxfp4
_mx_out = MX.mxfp4_output


def _mx_round_log2_scale(amax):
    # scale exponent from round(log2(amax)) instead of floor
    a = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.round(np.log2(np.where(a > 0, a, 1.0))) - 2
    return np.where(np.isinf(a), 255, np.clip(e + 127, 0, 254)).astype(np.uint8)


def _mx_swapped_nibbles(y, vec):
    packed, sb = _mx_quant(y, vec)
    return ((packed >> 4) | (packed << 4)).astype(np.uint8), sb


MX_MUTANTS = {
    "e2m1_ties_away": ("encode_e2m1", lambda v: _mx_encode(np.asarray(v, dtype=np.float64) * (1 + 1e-12))),
    "e2m1_truncates": ("encode_e2m1", lambda v: _mx_encode(
        np.sign(np.asarray(v, dtype=np.float64)) * np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])[
            np.clip(np.searchsorted([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.minimum(np.abs(v), 6), side="right") - 1,
                    0, 7)])),
    "e2m1_sign_dropped": ("encode_e2m1", lambda v: _mx_encode(np.abs(np.asarray(v, dtype=np.float64)))),
    "scale_one_low": ("mx_scale_byte", lambda a: np.where(_mx_scale(a) == 255, 255,
                                                          np.maximum(_mx_scale(a).astype(int) - 1, 0)).astype(np.uint8)),
    "scale_rounds_log2": ("mx_scale_byte", _mx_round_log2_scale),
    "nibbles_swapped": ("quantize_mxfp4", _mx_swapped_nibbles),
    "o_sf_scale_ignored": ("mxfp4_output", lambda o, vec, g=1.0: _mx_out(o, vec, 1.0)),
}


@pytest.mark.parametrize("name", sorted(MX_MUTANTS))
def test_mx_mutant_is_caught(name, monkeypatch):
    attr, repl = MX_MUTANTS[name]
    monkeypatch.setattr(MX, attr, repl)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin detects the planted mistake {name!r}"
