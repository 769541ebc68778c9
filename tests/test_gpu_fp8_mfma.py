"""GPU parity of the fp8-MFMA arithmetic for an fp8 cache at head_dim 128
(``fp8_compute=True``): Q and the softmax weights are rounded to e4m3fn and
both products run on gfx950's 32x32x64 fp8 MFMA.  Held to the fp8 KV
tolerance (max |err| <= 6e-2) against the fp64 oracle on long-prefix
batches shaped like the long-prefix fp8 workload.

Accuracy contract (kFp8MinKeys in the kernel, stated in ppa.h): a work item
runs on the fp8 MFMA only when each of its rows sees at least 1024 keys in
the item's key range; other items take the widened-bf16 arithmetic, so on
batches where no item qualifies (short sequences, narrow windows) the output
equals the widened path bit for bit, and on mixed batches the rows of the
short items do.  The fp8 rows are held to 6e-2, and random-data parity on
them pins the operand layouts (the order of keys in P against the
transposed V tile, and of dims in Q against K)."""
from __future__ import annotations

import sys
import zlib

import numpy as np
import pytest
import torch

from gpu_helpers import TOL_FP8_MAX, assert_close, errors, guard_rows_untouched, run_gpu, to_device
from oracle.case_io import decode_tensor, run_oracle, run_oracle_rows
from workloads import make_case, make_custom_case

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # long cached prefixes, as in the long-prefix fp8 workload (its per-tensor
    # scales folded into bmm1 / bmm2 by the generator)
    "prefix_hnd_p64": dict(num_qo_heads=16, num_kv_heads=2, page_size=64, q_lens=(200, 131),
                           prefix_lens=(2000, 1500)),
    "prefix_nhd_p16_combined": dict(num_qo_heads=8, num_kv_heads=1, page_size=16, kv_layout="NHD",
                                    kv_form="combined", q_lens=(96, 257, 33), prefix_lens=(1024, 700, 3000)),
    # a window wide enough that every row of an item sees >= 1024 common keys
    "prefix_window_sinks": dict(num_qo_heads=16, num_kv_heads=2, page_size=32, q_lens=(300,),
                                prefix_lens=(3500,), window_left=2047, sinks=True),
    # long enough that split chunks keep >= 1024 keys each
    "prefix_6000_split": dict(num_qo_heads=16, num_kv_heads=2, page_size=64, q_lens=(100,), prefix_lens=(6000,)),
    # bmm1 negated after the build: the K scale stays folded into it
    "prefix_g8_neg_bmm1": dict(num_qo_heads=16, num_kv_heads=2, page_size=64, q_lens=(150,),
                               prefix_lens=(1800,)),
}


def _case(name):
    spec = CASES[name]
    case = make_custom_case(name=name, batch=len(spec["q_lens"]), head_dim=128, kv_dtype="fp8_e4m3fn",
                            seed=zlib.crc32(name.encode()) % 10000, **spec)
    if name.endswith("neg_bmm1"):
        case["bmm1_scale"] = -case["bmm1_scale"]
    return case


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_mfma_parity(name):
    case = _case(name)
    _say("fp8 mfma", name)
    want, written = run_oracle(case)
    d = to_device(case)
    out = run_gpu(d, fp8_compute=True)
    grid = run_gpu(d, fp8_compute=True, schedule="grid")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), grid.view(torch.int16)), "persistent != grid schedule"
    assert guard_rows_untouched(out, written)
    mx, mean = assert_close(out, want, written, fp8=True, what=name)
    _say(f"  max {mx:.2e} mean {mean:.2e}")


@pytest.mark.parametrize("splits", [2, 5])
def test_fp8_mfma_split_kv(splits):
    case = _case("prefix_6000_split")
    want, written = run_oracle(case)
    d = to_device(case)
    out = run_gpu(d, fp8_compute=True, kv_splits=splits)
    wide = run_gpu(d, kv_splits=splits)
    torch.cuda.synchronize()
    assert not torch.equal(out.view(torch.int16), wide.view(torch.int16)), "the chunks did not run on the fp8 MFMA"
    assert guard_rows_untouched(out, written)
    mx, mean = assert_close(out, want, written, fp8=True, what=f"split {splits}")
    _say(f"  S={splits}: max {mx:.2e} mean {mean:.2e}")


def test_fp8_mfma_window_zero_items_run_widened():
    # window_left = 0: each row sees one key, so no item reaches the key
    # count of the fp8 arithmetic and every row is the widened path's,
    # bmm2 * v exactly
    case = make_custom_case(name="exact8", batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=64,
                            kv_dtype="fp8_e4m3fn", q_lens=(70, 1, 200), prefix_lens=(5, 40, 3000), window_left=0,
                            bmm1_scale=0.3, bmm2_scale=0.75, seed=404)
    want, written = run_oracle(case)
    d = to_device(case)
    f8 = run_gpu(d, fp8_compute=True)
    wide = run_gpu(d)
    torch.cuda.synchronize()
    assert torch.equal(f8.view(torch.int16), wide.view(torch.int16)), "exact rows differ between the two paths"
    mx, _ = errors(f8, want, written)
    assert mx <= 2e-2


# short sequences, where rounding each weight to e4m3fn does not average
# out (a 90-key case reached 6.8e-2 when it ran on the fp8 MFMA): no item
# qualifies, so the output is the widened path's, bit for bit
SHORT = {
    "q90_prefix0": dict(num_qo_heads=8, num_kv_heads=2, page_size=16, q_lens=(90,), prefix_lens=(0,)),
    "q70_33_append_shape": dict(num_qo_heads=8, num_kv_heads=2, page_size=16, q_lens=(70, 33),
                                prefix_lens=(20, 60)),
    "q150_prefix600": dict(num_qo_heads=16, num_kv_heads=2, page_size=64, q_lens=(150,), prefix_lens=(600,)),
    "q65_prefix63_nan_poison": dict(num_qo_heads=8, num_kv_heads=1, page_size=16, poison="nan", q_lens=(65,),
                                    prefix_lens=(63,)),
    "window_511_long_prefix": dict(num_qo_heads=8, num_kv_heads=2, page_size=32, q_lens=(300,),
                                   prefix_lens=(4000,), window_left=511, sinks=True),
}


@pytest.mark.parametrize("name", list(SHORT))
def test_fp8_compute_short_items_are_widened(name):
    spec = SHORT[name]
    case = make_custom_case(name=name, batch=len(spec["q_lens"]), head_dim=128, kv_dtype="fp8_e4m3fn",
                            seed=zlib.crc32(name.encode()) % 10000, **spec)
    want, written = run_oracle(case)
    d = to_device(case)
    f8 = run_gpu(d, fp8_compute=True)
    wide = run_gpu(d)
    torch.cuda.synchronize()
    assert torch.equal(f8.view(torch.int16), wide.view(torch.int16)), f"{name}: short items not widened"
    mx, mean = assert_close(f8, want, written, fp8=True, what=name)
    _say(f"  {name}: max {mx:.2e} mean {mean:.2e}")


def test_fp8_compute_mixed_batch():
    """A chunk of 600 rows over an 800-key prefix, 8 q heads per kv head (32
    tokens per item): items starting before token 224 see fewer than 1024
    keys and run widened (bit-equal to fp8_compute=0), later ones run on the
    fp8 MFMA (and differ from it); all rows within 6e-2 of the oracle."""
    case = make_custom_case(name="mixed8", batch=2, num_qo_heads=16, num_kv_heads=2, head_dim=128, page_size=32,
                            kv_dtype="fp8_e4m3fn", q_lens=(600, 100), prefix_lens=(800, 2000), seed=808)
    want, written = run_oracle(case)
    d = to_device(case)
    f8 = run_gpu(d, fp8_compute=True)
    wide = run_gpu(d)
    torch.cuda.synchronize()
    mx, mean = assert_close(f8, want, written, fp8=True, what="mixed")
    a = f8.view(torch.int16).cpu()
    b = wide.view(torch.int16).cpu()
    assert torch.equal(a[:224], b[:224]), "rows of items under the key count differ from the widened path"
    assert not torch.equal(a[224:600], b[224:600]), "items over the key count did not run on the fp8 MFMA"
    assert not torch.equal(a[600:700], b[600:700]), "the long-prefix request did not run on the fp8 MFMA"
    _say(f"  mixed: max {mx:.2e} mean {mean:.2e}")


def test_fp8_mfma_full_size_sampled():
    """The long-prefix fp8 workload at its full size, in the launch
    configuration the bench times (fp8_compute, persistent schedule)."""
    from test_gpu_parity import _sample_rows
    case = make_case("fp8_long_prefix")
    d = to_device(case)
    out = run_gpu(d, fp8_compute=True)
    torch.cuda.synchronize()
    written = np.zeros(case["num_tokens"], dtype=bool)
    written[:int(case["cum_seq_lens_q"][-1])] = True
    assert guard_rows_untouched(out, written)
    rows = _sample_rows(case)
    want = run_oracle_rows(case, rows)
    got = decode_tensor(out.cpu())
    err = np.abs(np.stack([got[t, h] for t, h in rows]) - want)
    _say(f"  sampled max {err.max():.2e} mean {err.mean():.2e}")
    assert err.max() <= TOL_FP8_MAX
