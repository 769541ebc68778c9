"""Seeded random configurations against the CPU oracle (GPU).

Each seed draws one small batch from the whole argument space of the call:
GQA groups from 1 to 24 (a group above 16 splits into two head groups, the
second partial), head_dim 64 or 128, page sizes 1 to 64, HND or NHD, split,
combined or single-plane combined caches, empty and ragged requests, prefixes
longer than the queries, no window or a window from 0 to 200 keys, sinks,
bf16 or fp8 (e4m3fn) caches and, for a third of the seeds, split-KV with two
or three chunks.  Every written row is compared with the oracle at the
stated tolerances, rows outside the requests must stay untouched, and the
persistent and one-workgroup-per-item schedules must agree bit for bit.
The log-sum-exp output is checked against the oracle's on every seed (and,
with split-KV, the merged one too); asking for it must not change a bit of
the output.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, guard_rows_untouched, lse_close, run_gpu, to_device, workspace
from oracle.case_io import run_oracle, run_oracle_lse
from workloads import make_custom_case

pytestmark = pytest.mark.gpu

GROUPS = (1, 2, 3, 4, 5, 6, 8, 12, 16, 24)
PAGES = (1, 2, 4, 8, 16, 32, 64)


def _draw(seed: int) -> tuple[dict, int]:
    rng = np.random.default_rng(90_000 + seed)
    batch = int(rng.integers(1, 5))
    hkv = int(rng.choice((1, 2)))
    group = int(rng.choice(GROUPS))
    q_lens = tuple(int(x) for x in rng.integers(0, 160, batch))
    if all(q == 0 for q in q_lens):
        q_lens = (int(rng.integers(1, 160)),) + q_lens[1:]
    prefix = tuple(int(x) for x in rng.integers(0, 260, batch))
    spec = dict(name=f"rand{seed}", batch=batch, num_qo_heads=hkv * group, num_kv_heads=hkv,
                head_dim=int(rng.choice((64, 128))), page_size=int(rng.choice(PAGES)),
                kv_layout=str(rng.choice(("HND", "NHD"))),
                kv_form=str(rng.choice(("split", "combined", "combined1"))),
                kv_dtype="fp8_e4m3fn" if rng.random() < 0.25 else "bf16",
                q_lens=q_lens, prefix_lens=prefix,
                window_left=-1 if rng.random() < 0.6 else int(rng.integers(0, 201)),
                sinks=bool(rng.random() < 0.5), seed=seed)
    splits = int(rng.choice((2, 3))) if rng.random() < 0.34 else 0
    return spec, splits


@pytest.mark.parametrize("seed", range(24))
def test_random_config_parity(seed):
    spec, splits = _draw(seed)
    case = make_custom_case(**spec)
    print("random", seed, {k: spec[k] for k in ("num_qo_heads", "num_kv_heads", "head_dim", "page_size",
                                                  "kv_layout", "kv_form", "kv_dtype", "window_left", "sinks")},
          case["q_lens"], case["kv_lens"], "splits", splits, file=sys.stderr, flush=True)
    want, written = run_oracle(case)
    want_lse = run_oracle_lse(case)
    d = to_device(case)
    fp8 = case["kv_dtype"] != "bf16"
    out = run_gpu(d)
    grid = run_gpu(d, schedule="grid")
    lse = torch.full(tuple(d["query"].shape[:2]), float("nan"), dtype=torch.float32, device="cuda")
    with_lse = run_gpu(d, lse=lse)
    torch.cuda.synchronize()
    assert guard_rows_untouched(out, written), "rows outside the requests were written"
    assert_close(out, want, written, fp8=fp8, what=spec["name"])
    assert torch.equal(out.view(torch.int16), grid.view(torch.int16)), "persistent != grid schedule"
    assert torch.equal(out.view(torch.int16), with_lse.view(torch.int16)), "the lse output changed the output"
    lse_close(lse, want_lse, written, spec["name"])
    assert torch.isnan(lse.cpu()[~torch.from_numpy(written)]).all(), "lse written outside the requests"
    assert not workspace().any(), "scheduler workspace not returned to zero"
    if splits:
        sp_lse = torch.full_like(lse, float("nan"))
        sp = run_gpu(d, kv_splits=splits, lse=sp_lse)
        torch.cuda.synchronize()
        assert guard_rows_untouched(sp, written), "split-KV wrote rows outside the requests"
        assert_close(sp, want, written, fp8=fp8, what=f"{spec['name']} kv_splits={splits}")
        lse_close(sp_lse, want_lse, written, f"{spec['name']} kv_splits={splits}")
