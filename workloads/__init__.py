"""Seeded synthetic inputs for batched paged prefill attention.

This package only draws random tensors and lays them out the way the
FlashInfer API page for ``trtllm_batch_context_with_kv_cache`` (section
"Parameters") describes the call's arguments.  It holds none of the
attention arithmetic: it is shared by the CPU oracle's tests, the GPU parity
tests and the bench, and imports neither side.
"""
from .cases import SPECS, Spec, make_case, make_custom_case, spec_by_index  # noqa: F401
