"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
an independent fact: a hand-derived closed form, a brute-force evaluation
that reads pages key by key, torch's SDPA, torch's own number decoders, or an
invariance the definition implies.  ``test_oracle.py`` runs them all;
``test_oracle_mutants.py`` plants plausible mistakes in the oracle and checks
that each one trips at least one pin.

The oracle is reached through its module attributes at call time, so a
planted mistake (a monkeypatched step) is what the pins see.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle.mxfp4 as MX
import oracle.paged_attention as OA
from oracle.case_io import decode_tensor, oracle_inputs
from workloads import make_custom_case
from workloads.cases import relayout, to_flat_page_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(case, **over):
    a = oracle_inputs(case)
    a.update(over)
    return OA.paged_prefill_attention(**a)


def _tiny(seed, **kw):
    base = dict(batch=3, num_qo_heads=4, num_kv_heads=2, head_dim=8, page_size=4,
                q_lens=(5, 1, 7), prefix_lens=(3, 0, 6), kv_layout="HND",
                kv_form="split", seed=seed, bmm1_scale=0.7, bmm2_scale=1.3)
    base.update(kw)
    return make_custom_case(**base)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def pin_bf16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = OA.decode_bf16(codes)
    theirs = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(ours, theirs), "bf16 decode differs from torch's cast"


def pin_e4m3fn_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = OA.decode_e4m3fn(codes)
    theirs = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(ours, theirs), "e4m3fn table differs from torch's cast"


def pin_number_format_golden():
    with open(os.path.join(GOLDEN, "number_formats.json")) as f:
        g = json.load(f)
    for code, val in g["e4m3fn"].items():
        got = OA.decode_e4m3fn(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert _same(got, float(val)), f"e4m3fn {code}: {got} != {val}"
    for code, val in g["bf16"].items():
        got = OA.decode_bf16(np.array([int(code, 16)], dtype=np.uint16))[0]
        assert _same(got, float(val)), f"bf16 {code}: {got} != {val}"


# --------------------------------------------------------------------------
# page gather
# --------------------------------------------------------------------------

GATHER_VARIANTS = [
    dict(kv_layout="HND", kv_form="split", page_size=4),
    dict(kv_layout="NHD", kv_form="split", page_size=4),
    dict(kv_layout="HND", kv_form="combined", page_size=3),
    dict(kv_layout="NHD", kv_form="combined", page_size=1),
    dict(kv_layout="NHD", kv_form="combined1", page_size=5),
    dict(kv_layout="HND", kv_form="split", page_size=16, kv_dtype="fp8_e4m3fn"),
]


def pin_gather_reproduces_logical_kv():
    """The generator scatters each request's contiguous K/V into shuffled
    pages; the oracle's gather must give the same tokens back, bit for bit."""
    for n, var in enumerate(GATHER_VARIANTS):
        case = _tiny(100 + n, **var)
        a = oracle_inputs(case)
        for b in range(case["batch_size"]):
            for kv_idx, logical in ((0, case["logical_k"]), (1, case["logical_v"])):
                got = OA.gather_paged_kv(a["kv_cache"], a["block_tables"][b], kv_idx,
                                         case["kv_lens"][b], case["page_size"], case["kv_layout"])
                want = decode_tensor(logical[b])
                assert got.shape == want.shape, (var, got.shape, want.shape)
                assert _same(got, want), f"gather mismatch {var} request {b} plane {kv_idx}"


# --------------------------------------------------------------------------
# brute force, key by key
# --------------------------------------------------------------------------

def _brute_force(case):
    """Every output element as a plain Python sum over keys.  Each key is
    fetched straight from its page through the block table (no gathered
    copy), and the softmax is exp(s) / (sum exp(s) + exp(sink)) with no
    shift."""
    a = oracle_inputs(case)
    q = a["query"]
    P = a["page_size"]
    lay = a["kv_layout"]
    kvc = a["kv_cache"]
    Hq = q.shape[1]
    Hkv = case["num_kv_heads"]
    W = a["window_left"]
    out = np.full(q.shape, np.nan)

    def fetch(plane_idx, pid, slot, hk):
        if isinstance(kvc, tuple):
            pool = kvc[plane_idx]
            return pool[pid, hk, slot] if lay == "HND" else pool[pid, slot, hk]
        pi = plane_idx if kvc.shape[1] == 2 else 0
        return kvc[pid, pi, hk, slot] if lay == "HND" else kvc[pid, pi, slot, hk]

    cu = a["cum_seq_lens_q"]
    for b in range(len(a["seq_lens"])):
        kv_len = int(a["seq_lens"][b])
        q_len = int(cu[b + 1] - cu[b])
        for i in range(q_len):
            t = int(cu[b]) + i
            pos = kv_len - q_len + i
            for h in range(Hq):
                hk = h * Hkv // Hq
                num = np.zeros(q.shape[2])
                den = 0.0
                for j in range(kv_len):
                    if j > pos or (W >= 0 and j < pos - W):
                        continue
                    pid = int(a["block_tables"][b][j // P])
                    kj = fetch(0, pid, j % P, hk)
                    vj = fetch(1, pid, j % P, hk)
                    w = math.exp(a["bmm1_scale"] * float(np.dot(q[t, h], kj)))
                    num = num + w * vj
                    den += w
                if a["sinks"] is not None:
                    den += math.exp(float(a["sinks"][h]))
                out[t, h] = a["bmm2_scale"] * num / den
    return out


BRUTE_CASES = [
    dict(),
    dict(window_left=0),
    dict(window_left=2, sinks=True),
    dict(kv_layout="NHD", kv_form="combined", page_size=3, window_left=4),
    dict(num_qo_heads=6, num_kv_heads=2, sinks=True, page_size=2),
    dict(num_qo_heads=3, num_kv_heads=3, q_lens=(4, 0, 2), prefix_lens=(0, 5, 1)),
    dict(kv_form="combined1", kv_layout="HND", page_size=5),
    dict(kv_dtype="fp8_e4m3fn", page_size=4, sinks=True, window_left=3,
         bmm1_scale=None, bmm2_scale=None),
]


def pin_brute_force():
    for n, var in enumerate(BRUTE_CASES):
        case = _tiny(200 + n, **var)
        got, written = _run(case)
        want = _brute_force(case)
        rows = written
        assert np.array_equal(rows, ~np.isnan(want).all(axis=(1, 2))), var
        err = np.max(np.abs(got[rows] - want[rows])) if rows.any() else 0.0
        assert err <= 1e-12, f"brute force mismatch {var}: {err}"


# --------------------------------------------------------------------------
# torch SDPA (float64, explicit bottom-right mask, grouped kv heads)
# --------------------------------------------------------------------------

SDPA_CASES = [
    dict(prefix_lens=(0, 0, 0)),
    dict(),
    dict(window_left=3),
    dict(num_qo_heads=8, num_kv_heads=2, kv_layout="NHD"),
    dict(num_qo_heads=2, num_kv_heads=2, kv_form="combined", head_dim=16, page_size=8),
]


def pin_torch_sdpa():
    import torch.nn.functional as F
    for n, var in enumerate(SDPA_CASES):
        case = _tiny(300 + n, **var)
        got, written = _run(case)
        a = oracle_inputs(case)
        cu = a["cum_seq_lens_q"]
        G = case["num_qo_heads"] // case["num_kv_heads"]
        for b in range(case["batch_size"]):
            q_len = int(cu[b + 1] - cu[b])
            kv_len = int(a["seq_lens"][b])
            if q_len == 0:
                continue
            # contiguous K/V from the generator's logical tokens
            k = torch.from_numpy(decode_tensor(case["logical_k"][b]))      # [kv, Hkv, D]
            v = torch.from_numpy(decode_tensor(case["logical_v"][b]))
            q = torch.from_numpy(a["query"][int(cu[b]):int(cu[b + 1])])     # [q, Hq, D]
            i = torch.arange(q_len)[:, None] + (kv_len - q_len)
            j = torch.arange(kv_len)[None, :]
            mask = j <= i
            if case["window_left"] >= 0:
                mask &= j >= i - case["window_left"]
            ref = F.scaled_dot_product_attention(
                q.permute(1, 0, 2).unsqueeze(0), k.permute(1, 0, 2).unsqueeze(0),
                v.permute(1, 0, 2).unsqueeze(0), attn_mask=mask,
                scale=a["bmm1_scale"], enable_gqa=G > 1)[0].permute(1, 0, 2)
            ref = (a["bmm2_scale"] * ref).numpy()
            err = np.max(np.abs(got[int(cu[b]):int(cu[b + 1])] - ref))
            assert err <= 1e-12, f"SDPA mismatch {var} request {b}: {err}"


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def pin_window_zero_is_diagonal():
    """window_left 0 leaves only key prefix+i: o_i = bmm2 * v_{prefix+i}."""
    case = _tiny(400, window_left=0)
    got, written = _run(case)
    bmm2 = oracle_inputs(case)["bmm2_scale"]
    cu = case["cum_seq_lens_q"].numpy()
    G = case["num_qo_heads"] // case["num_kv_heads"]
    for b in range(case["batch_size"]):
        v = decode_tensor(case["logical_v"][b])
        pre = case["prefix_lens"][b]
        for i in range(case["q_lens"][b]):
            for h in range(case["num_qo_heads"]):
                want = bmm2 * v[pre + i, h // G]
                assert np.max(np.abs(got[cu[b] + i, h] - want)) <= 1e-12


def pin_window_zero_with_sink():
    """window_left 0 plus a sink: o_i = bmm2 * v / (1 + exp(sink - s_ii))."""
    case = _tiny(401, window_left=0, sinks=True)
    got, _ = _run(case)
    a = oracle_inputs(case)
    cu = a["cum_seq_lens_q"]
    G = case["num_qo_heads"] // case["num_kv_heads"]
    for b in range(case["batch_size"]):
        k = decode_tensor(case["logical_k"][b])
        v = decode_tensor(case["logical_v"][b])
        pre = case["prefix_lens"][b]
        for i in range(case["q_lens"][b]):
            t = int(cu[b]) + i
            for h in range(case["num_qo_heads"]):
                s = a["bmm1_scale"] * float(np.dot(a["query"][t, h], k[pre + i, h // G]))
                want = a["bmm2_scale"] * v[pre + i, h // G] / (1.0 + math.exp(a["sinks"][h] - s))
                assert np.max(np.abs(got[t, h] - want)) <= 1e-12


def pin_zero_scale_is_mean():
    """bmm1_scale 0 makes every valid logit 0: o_i = bmm2 * sum_valid v /
    (n_i + exp(sink)), n_i the number of valid keys."""
    for sinks in (False, True):
        case = _tiny(402 + sinks, bmm1_scale=0.0, window_left=3, sinks=sinks)
        got, _ = _run(case)
        a = oracle_inputs(case)
        cu = a["cum_seq_lens_q"]
        G = case["num_qo_heads"] // case["num_kv_heads"]
        for b in range(case["batch_size"]):
            v = decode_tensor(case["logical_v"][b])
            pre = case["prefix_lens"][b]
            for i in range(case["q_lens"][b]):
                lo = max(0, pre + i - 3)
                hi = pre + i
                n = hi - lo + 1
                for h in range(case["num_qo_heads"]):
                    extra = math.exp(a["sinks"][h]) if sinks else 0.0
                    want = a["bmm2_scale"] * v[lo:hi + 1, h // G].sum(axis=0) / (n + extra)
                    assert np.max(np.abs(got[int(cu[b]) + i, h] - want)) <= 1e-12


def pin_golden_hand_examples():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        g = json.load(f)
    env = {"e": math.e, "exp": math.exp, "__builtins__": {}}
    for ex in g["examples"]:
        if ex["kv_form"] == "split":
            kv = (np.array(ex["k_pool"], dtype=np.float64), np.array(ex["v_pool"], dtype=np.float64))
        else:
            kv = np.array(ex["kv_pool"], dtype=np.float64)
        got, written = OA.paged_prefill_attention(
            query=np.array(ex["query"], dtype=np.float64), kv_cache=kv,
            kv_layout=ex["kv_layout"], block_tables=np.array(ex["block_tables"]),
            seq_lens=np.array(ex["seq_lens"]), cum_seq_lens_q=np.array(ex["cum_seq_lens_q"]),
            page_size=ex["page_size"], bmm1_scale=ex["bmm1_scale"], bmm2_scale=ex["bmm2_scale"],
            window_left=ex["window_left"],
            sinks=None if ex["sinks"] is None else np.array(ex["sinks"], dtype=np.float64))
        for t, row in enumerate(ex["expected"]):
            if row is None:
                assert not written[t], f"{ex['name']}: row {t} should be unwritten"
                continue
            assert written[t], f"{ex['name']}: row {t} not written"
            want = np.array([[eval(x, env) for x in head] for head in row])
            err = np.max(np.abs(got[t] - want))
            assert err <= 1e-12, f"{ex['name']} row {t}: {got[t]} vs {want}"


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------

def pin_sink_neg_inf_is_no_sink():
    case = _tiny(500, window_left=2)
    a = oracle_inputs(case)
    base, _ = OA.paged_prefill_attention(**a)
    a["sinks"] = np.full(case["num_qo_heads"], -np.inf)
    got, _ = OA.paged_prefill_attention(**a)
    assert np.array_equal(base, got, equal_nan=True), "sink -inf differs from no sink"


def pin_full_window_is_no_window():
    case = _tiny(501, sinks=True)
    a = oracle_inputs(case)
    base, _ = OA.paged_prefill_attention(**a)
    a["window_left"] = max(case["kv_lens"])
    got, _ = OA.paged_prefill_attention(**a)
    assert np.array_equal(base, got, equal_nan=True), "window >= kv_len differs from -1"


def pin_chunk_equals_tail_of_full_prefill():
    """A chunk of q new tokens over a p-token prefix equals the last q rows of
    one prefill of p+q tokens over the same K/V."""
    full = _tiny(502, batch=1, q_lens=(11,), prefix_lens=(0,), sinks=True, window_left=5)
    a = oracle_inputs(full)
    out_full, _ = OA.paged_prefill_attention(**a)
    for q in (1, 4, 11):
        c = dict(a)
        c["query"] = a["query"][11 - q:]
        c["cum_seq_lens_q"] = np.array([0, q])
        out_c, _ = OA.paged_prefill_attention(**c)
        assert np.max(np.abs(out_c - out_full[11 - q:])) <= 1e-14


def pin_relayout_invariance():
    """Same logical tokens, other cache: layout, combined/split, page size and
    page permutation leave the output bit-identical."""
    case = _tiny(503, sinks=True, window_left=4)
    base, _ = _run(case)
    for lay, form, P, seed in (("NHD", "split", 4, 1), ("HND", "combined", 2, 2),
                               ("NHD", "combined", 7, 3), ("HND", "split", 1, 4)):
        other = relayout(case, kv_layout=lay, kv_form=form, page_size=P, permute_seed=seed)
        got, _ = _run(other)
        assert np.array_equal(base, got, equal_nan=True), (lay, form, P)


def pin_poison_invariance():
    a_case = _tiny(504, poison="finite")
    b_case = _tiny(504, poison="nan")
    a, _ = _run(a_case)
    b, _ = _run(b_case)
    assert np.array_equal(a, b, equal_nan=True), "unused pages or slots leaked"
    assert not np.isnan(a[:sum(a_case["q_lens"])]).any()


def pin_request_permutation():
    case = _tiny(505, window_left=3)
    base, _ = _run(case)
    a = oracle_inputs(case)
    order = [2, 0, 1]
    cu = a["cum_seq_lens_q"]
    qs = [a["query"][cu[b]:cu[b + 1]] for b in order]
    new_cu = np.concatenate([[0], np.cumsum([len(x) for x in qs])])
    got, _ = OA.paged_prefill_attention(
        query=np.concatenate(qs), kv_cache=a["kv_cache"], kv_layout=a["kv_layout"],
        block_tables=a["block_tables"][order], seq_lens=a["seq_lens"][order],
        cum_seq_lens_q=new_cu, page_size=a["page_size"], bmm1_scale=a["bmm1_scale"],
        bmm2_scale=a["bmm2_scale"], window_left=a["window_left"], sinks=None)
    want = np.concatenate([base[cu[b]:cu[b + 1]] for b in order])
    assert np.array_equal(got, want, equal_nan=True)


def pin_bmm2_linear():
    case = _tiny(506, sinks=True)
    a = oracle_inputs(case)
    a["bmm2_scale"] = 1.0
    one, _ = OA.paged_prefill_attention(**a)
    a["bmm2_scale"] = -2.5
    two, _ = OA.paged_prefill_attention(**a)
    assert np.max(np.abs(two - (-2.5) * one)) <= 1e-12


def pin_gqa_equals_repeated_mha():
    """G query heads sharing one kv head equal an MHA run whose kv heads are
    the shared ones repeated G times in order."""
    case = _tiny(507, num_qo_heads=6, num_kv_heads=2, kv_layout="NHD")
    base, _ = _run(case)
    a = oracle_inputs(case)
    k, v = a["kv_cache"]
    rep = (np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2))
    a["kv_cache"] = rep
    got, _ = OA.paged_prefill_attention(**a)
    assert np.array_equal(base, got, equal_nan=True)


def pin_flat_page_table():
    """The flat page table (kv_indptr / kv_indices) names the same pages as
    the padded one: pages gathered through it reproduce the generator's
    logical K/V, and the output equals the padded-table output bit for bit,
    with junk entries before request 0 and after each request's pages."""
    case = _tiny(611, sinks=True, window_left=3, q_lens=(5, 0, 7), prefix_lens=(3, 2, 6))
    base, _ = _run(case)
    flat = to_flat_page_table(case, slack=2, lead=3, seed=5)
    a = oracle_inputs(flat)
    assert a["block_tables"] is None
    for b, kv in enumerate(case["kv_lens"]):
        pages = OA.request_pages(b, None, a["kv_indptr"], a["kv_indices"])
        for kv_idx, logical in ((0, case["logical_k"]), (1, case["logical_v"])):
            got = OA.gather_paged_kv(a["kv_cache"], pages, kv_idx, kv, case["page_size"], case["kv_layout"])
            want = decode_tensor(logical[b]) if kv else np.zeros((0,) + got.shape[1:])
            assert np.array_equal(got, want), (b, kv_idx)
    got, _ = OA.paged_prefill_attention(**a)
    assert np.array_equal(base, got, equal_nan=True)


def pin_lse_closed_forms():
    """bmm1 = 0 makes every valid logit 0: lse = log(n_valid) (log(n_valid +
    e^sink) with a sink); window 0 leaves the diagonal key alone:
    lse = bmm1 q_i . k_(prefix+i)."""
    case = _tiny(701, bmm1_scale=0.0, window_left=2)
    lse = OA.paged_prefill_lse(**oracle_inputs(case))
    cu = case["cum_seq_lens_q"].numpy()
    for b, (q_len, kv_len) in enumerate(zip(case["q_lens"], case["kv_lens"])):
        pre = kv_len - q_len
        for i in range(q_len):
            n = min(pre + i, 2) + 1
            assert np.allclose(lse[cu[b] + i], math.log(n), rtol=0, atol=1e-13)
    sinks = torch.tensor([0.5, -1.0, 2.0, -3.0])
    case = _tiny(702, bmm1_scale=0.0, sinks=True)
    case["sinks"] = sinks
    lse = OA.paged_prefill_lse(**oracle_inputs(case))
    for b, (q_len, kv_len) in enumerate(zip(case["q_lens"], case["kv_lens"])):
        pre = kv_len - q_len
        for i in range(q_len):
            for h in range(4):
                want = math.log(pre + i + 1 + math.exp(float(sinks[h])))
                assert abs(lse[cu[b] + i, h] - want) < 1e-12
    case = _tiny(703, window_left=0)
    a = oracle_inputs(case)
    lse = OA.paged_prefill_lse(**a)
    q = a["query"]
    for b, (q_len, kv_len) in enumerate(zip(case["q_lens"], case["kv_lens"])):
        pre = kv_len - q_len
        k = decode_tensor(case["logical_k"][b])
        for i in range(q_len):
            for h in range(4):
                s_ii = a["bmm1_scale"] * float(q[cu[b] + i, h] @ k[pre + i, h // 2])
                assert abs(lse[cu[b] + i, h] - s_ii) < 1e-12


def pin_lse_brute_force():
    """Against scipy's logsumexp over logits formed key by key from the
    pages, with the sink as one more term."""
    from scipy.special import logsumexp
    case = _tiny(704, sinks=True, window_left=4)
    a = oracle_inputs(case)
    lse = OA.paged_prefill_lse(**a)
    q, bt, P = a["query"], a["block_tables"], case["page_size"]
    kplane = a["kv_cache"][0]
    cu = case["cum_seq_lens_q"].numpy()
    for b, (q_len, kv_len) in enumerate(zip(case["q_lens"], case["kv_lens"])):
        pre = kv_len - q_len
        for i in range(q_len):
            pos = pre + i
            for h in range(4):
                terms = [float(a["sinks"][h])]
                for j in range(max(0, pos - 4), pos + 1):
                    krow = kplane[bt[b][j // P], h // 2, j % P]   # HND: [page, head, slot, dim]
                    terms.append(a["bmm1_scale"] * float(q[cu[b] + i, h] @ krow))
                assert abs(lse[cu[b] + i, h] - logsumexp(terms)) < 1e-12


def pin_merge_of_key_splits_is_full():
    """Partial states over a partition of the keys (one part empty, one past
    the causal band), merged with the sink, give the full output and lse."""
    case = _tiny(705, sinks=True, window_left=5, q_lens=(6, 9), prefix_lens=(4, 2), batch=2)
    a = oracle_inputs(case)
    full, _ = OA.paged_prefill_attention(**a)
    full_lse = OA.paged_prefill_lse(**a)
    cu = case["cum_seq_lens_q"].numpy()
    for b, kv_len in enumerate(case["kv_lens"]):
        q = a["query"][cu[b]:cu[b + 1]]
        k = OA.gather_paged_kv(a["kv_cache"], a["block_tables"][b], 0, kv_len, case["page_size"], "HND")
        v = OA.gather_paged_kv(a["kv_cache"], a["block_tables"][b], 1, kv_len, case["page_size"], "HND")
        cuts = [0, 3, 3, 7, kv_len, kv_len + 4]
        parts = [OA.partial_state(q, k, v, a["bmm1_scale"], a["bmm2_scale"], 5, c0, c1)
                 for c0, c1 in zip(cuts, cuts[1:])]
        o, lse = OA.merge_states(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                                 a["sinks"][None, :])
        assert np.allclose(o, full[cu[b]:cu[b + 1]], rtol=1e-12, atol=1e-12)
        assert np.allclose(lse, full_lse[cu[b]:cu[b + 1]], rtol=1e-12, atol=1e-12)


def pin_merge_identities():
    """One part merges to itself; an empty part (o 0, lse -inf) changes
    nothing; the order of parts does not matter."""
    rng = np.random.default_rng(706)
    o = rng.standard_normal((3, 5, 2, 8))
    lse = rng.standard_normal((3, 5, 2)) * 4
    o1, l1 = OA.merge_states(o[:1], lse[:1])
    assert np.allclose(o1, o[0], rtol=1e-14, atol=1e-14) and np.allclose(l1, lse[0], rtol=1e-14, atol=1e-14)
    base_o, base_l = OA.merge_states(o, lse)
    eo, el = OA.merge_states(np.concatenate([o, np.zeros((1, 5, 2, 8))]),
                             np.concatenate([lse, np.full((1, 5, 2), -np.inf)]))
    assert np.allclose(eo, base_o, rtol=1e-14, atol=1e-14) and np.allclose(el, base_l, rtol=1e-14, atol=1e-14)
    po, pl = OA.merge_states(o[::-1], lse[::-1])
    assert np.allclose(po, base_o, rtol=1e-13, atol=1e-13) and np.allclose(pl, base_l, rtol=1e-13, atol=1e-13)


def pin_e4m3fn_encode():
    """The encoder inverts the decoder on every finite code, agrees with
    torch's float8_e4m3fn cast wherever that cast is finite (random values,
    exact midpoints between neighbours, subnormals), and saturates beyond
    448 where the cast would give NaN."""
    finite = [c for c in range(256) if not np.isnan(OA.E4M3FN_TABLE[c])]
    codes = np.array(finite, dtype=np.uint8)
    assert np.array_equal(OA.encode_e4m3fn(OA.E4M3FN_TABLE[codes]), codes)
    rng = np.random.default_rng(901)
    y = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(40.0),
        (rng.random(5000).astype(np.float32) * np.float32(2.0 ** -6)),
        # exact midpoints between consecutive positive grid values (ties)
        ((OA.E4M3FN_TABLE[1:126] + OA.E4M3FN_TABLE[2:127]) / 2).astype(np.float32),
        np.array([0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 463.99], dtype=np.float32),
    ])
    y = y[np.abs(y) < 464]
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(OA.encode_e4m3fn(y), want)
    sat = OA.encode_e4m3fn(np.array([448.0, 470.0, 1e9, -1e9, np.inf], dtype=np.float32))
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E]
    assert OA.encode_e4m3fn(np.array([np.nan]))[0] & 0x7F == 0x7F


def pin_append_then_gather():
    """Appended tokens are what a page gather reads back at their sequence
    positions (bf16: the new values; fp8: the encoded x / scale), tokens with
    a negative slot are skipped, and every other slot keeps its contents.
    Checked for both page layouts, split and combined caches: the cache is
    read back by the oracle's gather (the plain token-major copy of the
    VanillaAttention path), which indexes HND pages as [head, slot] and NHD
    pages as [slot, head] on its own."""
    rng = np.random.default_rng(903)
    for n, (layout, form) in enumerate((("NHD", "split"), ("HND", "split"), ("HND", "combined"),
                                        ("NHD", "combined"))):
        case = _tiny(902 + 7 * n, q_lens=(5, 3), prefix_lens=(7, 2), batch=2, page_size=4, kv_layout=layout,
                     num_qo_heads=6, num_kv_heads=3)
        P = case["page_size"]
        Hkv = case["num_kv_heads"]
        pool_shape = tuple(case["kv_cache"][0].shape)
        for kv_dtype, scale in (("bf16", 1.0), ("fp8_e4m3fn", 0.37)):
            code_t = np.uint16 if kv_dtype == "bf16" else np.uint8
            planes = [rng.integers(0, 1 << (16 if kv_dtype == "bf16" else 8), size=pool_shape).astype(code_t)
                      for _ in range(2)]
            n_new = sum(case["q_lens"])
            k_new = torch.randn(n_new, Hkv, 8).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            v_new = torch.randn(n_new, Hkv, 8).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            bt = case["block_tables"].numpy()
            slots, owner = [], []
            for b, (q, kv) in enumerate(zip(case["q_lens"], case["kv_lens"])):
                for i in range(q):
                    pos = kv - q + i
                    slots.append(int(bt[b, pos // P]) * P + pos % P)
                    owner.append((b, pos))
            slots = np.array(slots)
            slots[2] = -1                      # skipped
            out = OA.append_paged_kv(planes, layout, P, k_new, v_new, slots, kv_dtype, scale, scale)
            decode = OA.decode_bf16 if kv_dtype == "bf16" else OA.decode_e4m3fn
            if form == "split":
                before = (decode(planes[0]), decode(planes[1]))
                after = (decode(out[0]), decode(out[1]))
            else:   # one tensor with the K / V planes in dim 1
                before = decode(np.stack(planes, axis=1))
                after = decode(np.stack(out, axis=1))
            for kv_idx, new in ((0, k_new), (1, v_new)):
                if kv_dtype == "bf16":
                    want_new = OA.decode_bf16(new)
                else:
                    want_new = OA.decode_e4m3fn(OA.encode_e4m3fn(
                        OA.decode_bf16(new).astype(np.float32) / np.float32(scale)))
                for b, kv in enumerate(case["kv_lens"]):
                    got = OA.gather_paged_kv(after, bt[b], kv_idx, kv, P, layout)
                    old = OA.gather_paged_kv(before, bt[b], kv_idx, kv, P, layout)
                    written = np.zeros(kv, dtype=bool)
                    for i, (ob, pos) in enumerate(owner):
                        if ob != b or slots[i] < 0:
                            continue
                        assert _same(got[pos], want_new[i]), (layout, form, kv_dtype, kv_idx, b, pos)
                        written[pos] = True
                    assert _same(got[~written], old[~written]), (layout, form, kv_dtype, kv_idx, b)
                # slots no request reaches keep their codes
            for kv_idx in range(2):
                changed = np.zeros(planes[kv_idx].shape, dtype=bool)
                for loc in slots:
                    if loc < 0:
                        continue
                    if layout == "HND":
                        changed[loc // P, :, loc % P] = True
                    else:
                        changed[loc // P, loc % P] = True
                assert np.array_equal(out[kv_idx][~changed], planes[kv_idx][~changed]), (layout, form, kv_dtype)


def pin_attention_rows_match_the_batched_call():
    """The row-sampling entry (used to check full-size runs one (token, q
    head) pair at a time) gives, for every row of tiny batches, what the
    batched call gives and what the key-by-key brute force gives: padded and
    flat page tables, empty requests (repeated cum_seq_lens_q entries),
    window with sinks, GQA groups of 1, 2 and 3, both layouts."""
    variants = [
        dict(),
        dict(num_qo_heads=3, num_kv_heads=3, q_lens=(4, 0, 2), prefix_lens=(0, 5, 1)),
        dict(num_qo_heads=6, num_kv_heads=2, window_left=2, sinks=True, page_size=2),
        dict(q_lens=(0, 3, 0, 4), prefix_lens=(2, 1, 0, 6), batch=4, kv_layout="NHD", kv_form="combined",
             window_left=3, sinks=True),
        dict(q_lens=(6, 0, 2), prefix_lens=(1, 3, 9), flat=True),
    ]
    for n, var in enumerate(variants):
        var = dict(var)
        flat = var.pop("flat", False)
        case = _tiny(950 + n, **var)
        if flat:
            case = to_flat_page_table(case, slack=2, lead=3, seed=951)
        full, written = _run(case)
        brute = None if flat else _brute_force(case)
        a = oracle_inputs(case)
        cu = case["cum_seq_lens_q"].numpy()
        rows = [(t, h) for t in range(int(cu[-1])) for h in range(case["num_qo_heads"])]
        got = OA.attention_rows(rows=rows, **a)
        for r, (t, h) in enumerate(rows):
            assert written[t], (var, t)
            err = np.max(np.abs(got[r] - full[t, h]))
            assert err <= 1e-12, f"attention_rows != batched call {var} row {(t, h)}: {err}"
            if brute is not None:
                err = np.max(np.abs(got[r] - brute[t, h]))
                assert err <= 1e-12, f"attention_rows != brute force {var} row {(t, h)}: {err}"


# --------------------------------------------------------------------------
# MXFP4 output encoding
# --------------------------------------------------------------------------


def _mx_golden():
    with open(os.path.join(GOLDEN, "mxfp4_examples.json")) as f:
        return json.load(f)


def pin_mx_formats_golden():
    """E2M1 codes and E8M0 bytes decode to the format definition's values;
    E8M0 also agrees with torch's float8_e8m0fnu on all 256 bytes."""
    g = _mx_golden()
    for code, val in g["e2m1"].items():
        assert _same(MX.E2M1_TABLE[int(code, 16)], float(val)), f"e2m1 {code}"
    for b, val in g["e8m0"].items():
        assert _same(MX.e8m0_value(int(b, 16)), float(val)), f"e8m0 {b}"
    bytes_ = np.arange(256, dtype=np.uint8)
    theirs = torch.from_numpy(bytes_.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert _same(MX.e8m0_value(bytes_), theirs), "e8m0 decode differs from torch's"


def pin_mx_hand_examples():
    """Hand-worked blocks (scale byte and packed codes) reproduce."""
    for ex in _mx_golden()["blocks"]:
        y = np.array([float(v) for v in ex["y"]], dtype=np.float64)
        packed, sb = MX.mxfp4_output(y[None, :], ex["vec"], float(ex["g"]))
        want = [int(v, 16) for v in ex["packed"]]
        assert sb.tolist() == [[int(ex["scale"], 16)]], (ex["working"], sb)
        assert packed[0].tolist() == want, (ex["working"], [hex(v) for v in packed[0]])


def pin_e2m1_encode_brute_force():
    """The encoder equals an exhaustive nearest search over the 8 magnitudes
    (ties to the even code, clamp at 6, sign of v < 0), on random values,
    every midpoint and values past the largest."""
    rng = np.random.default_rng(911)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    mids = (mags[1:] + mags[:-1]) / 2
    v = np.concatenate([rng.uniform(-8, 8, 4000), mids, -mids, mags, -mags,
                        [6.01, 9.0, 1e30, -1e30, 0.2499, 0.2501, -0.0, -0.1]])
    got = MX.encode_e2m1(v)
    for x, c in zip(v, got):
        a = min(abs(x), 6.0)
        dist = np.abs(mags - a)
        best = np.flatnonzero(dist == dist.min())
        want = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        if math.copysign(1.0, x) < 0:
            want |= 8
        assert int(c) == want, (x, int(c), want)


def pin_mx_scale_exponent():
    """Scale byte b gives amax / 2^(b - 127) in [4, 8) for every normal amax
    (so the block's largest element lands in E2M1's top binade), read here
    through frexp; zero and tiny maxima clamp to byte 0, inf gives 0xFF."""
    rng = np.random.default_rng(912)
    amax = (rng.random(5000) * 2.0 ** rng.integers(-120, 120, 5000)).astype(np.float32)
    amax = amax[amax > 2.0 ** -120]
    b = MX.mx_scale_byte(amax).astype(np.int64)
    for a, bb in zip(amax.astype(np.float64), b):
        m, e = math.frexp(a)                        # a = m 2^e, m in [0.5, 1)
        assert bb - 127 == (e - 1) - 2, (a, bb)
        assert 4.0 <= a / 2.0 ** (bb - 127) < 8.0
    assert MX.mx_scale_byte(np.float32(0.0)) == 0
    assert MX.mx_scale_byte(np.float32(2.0 ** -140)) == 0
    assert MX.mx_scale_byte(np.float32(np.inf)) == 255


def pin_mx_roundtrip():
    """Representable blocks survive quantize -> dequantize exactly; random
    blocks come back within half the local E2M1 spacing times the scale (or
    at the +-6 clamp); scaling a block by 2^k moves the byte by k and keeps
    the codes."""
    rng = np.random.default_rng(913)
    vec = 32
    codes = rng.integers(0, 16, size=(64, vec))
    codes[:, 0] = rng.choice([6, 7, 14, 15], size=64)       # a magnitude in [4, 6] fixes the exponent
    e = rng.integers(-20, 20, size=(64, 1))
    y = (MX.E2M1_TABLE[codes] * 2.0 ** e).astype(np.float32)
    packed, sb = MX.quantize_mxfp4(y, vec)
    assert _same(MX.dequantize_mxfp4(packed, sb, vec), y.astype(np.float64))
    assert MX.encode_e2m1(np.array([-0.0, 0.0, np.nan, -np.nan])).tolist() == [8, 0, 7, 15]
    y = (rng.standard_normal((200, 64)) * 10.0 ** rng.uniform(-3, 3, (200, 1))).astype(np.float32)
    for v in (16, 32):
        packed, sb = MX.quantize_mxfp4(y, v)
        back = MX.dequantize_mxfp4(packed, sb, v)
        scale = np.repeat(MX.e8m0_value(sb), v, axis=-1)
        t = np.abs(y.astype(np.float64)) / scale
        half = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0))
        err = np.abs(back - y)
        ok = (err <= half * scale) | ((t > 6) & (np.abs(back) == 6 * scale))
        assert ok.all()
        p2, s2 = MX.quantize_mxfp4((y * np.float32(2.0 ** 5)).astype(np.float32), v)
        assert np.array_equal(p2, packed) and np.array_equal(s2.astype(int), sb.astype(int) + 5)


def pin_mx_output_of_attention():
    """The MXFP4 output of an attention case dequantizes (code * 2^E / g) to
    the dense output within the format's error, for g = 1 and g != 1."""
    case = _tiny(914, q_lens=(5, 9), prefix_lens=(3, 0), batch=2, head_dim=32)
    o, written = _run(case)
    o = o[written]
    for g in (1.0, 0.125, 48.0):
        for v in (16, 32):
            packed, sb = MX.mxfp4_output(o, v, g)
            back = MX.dequantize_mxfp4(packed, sb, v, g)
            blk = np.abs(o.reshape(o.shape[:-1] + (o.shape[-1] // v, v))).max(axis=-1)
            tol = np.repeat(blk, v, axis=-1) / 4.0 + 1e-30   # half the largest spacing at the block's scale
            assert (np.abs(back - o) <= tol).all(), (g, v)


ALL_PINS = [
    pin_mx_formats_golden,
    pin_mx_hand_examples,
    pin_e2m1_encode_brute_force,
    pin_mx_scale_exponent,
    pin_mx_roundtrip,
    pin_mx_output_of_attention,
    pin_bf16_decode_all_codes,
    pin_e4m3fn_decode_all_codes,
    pin_number_format_golden,
    pin_gather_reproduces_logical_kv,
    pin_brute_force,
    pin_torch_sdpa,
    pin_window_zero_is_diagonal,
    pin_window_zero_with_sink,
    pin_zero_scale_is_mean,
    pin_golden_hand_examples,
    pin_sink_neg_inf_is_no_sink,
    pin_full_window_is_no_window,
    pin_chunk_equals_tail_of_full_prefill,
    pin_relayout_invariance,
    pin_poison_invariance,
    pin_request_permutation,
    pin_bmm2_linear,
    pin_gqa_equals_repeated_mha,
    pin_flat_page_table,
    pin_lse_closed_forms,
    pin_lse_brute_force,
    pin_merge_of_key_splits_is_full,
    pin_merge_identities,
    pin_e4m3fn_encode,
    pin_append_then_gather,
    pin_attention_rows_match_the_batched_call,
]
