"""MI355X (gfx950) paged prefill attention.

A thin binding over the C ABI declared in ``include/ppa.h`` (library
``_lib/libppa.so``).  The functions named ``ppa_*`` mirror the C entry
points one to one; ``batch_context_with_kv_cache`` mirrors the argument list
of the FlashInfer API page for ``trtllm_batch_context_with_kv_cache`` and
only marshals torch tensors into ``ppa_params``.  Every step of the
attention runs in the HIP kernels; there is no fallback: importing this
package without the built library raises ImportError.
"""
from .binding import (PPA_ABI_VERSION, PPA_DTYPE_MXFP4, WORKSPACE_BYTES, MxFp4Output, empty_mxfp4, PpaAppendParams, PpaError, PpaMergeParams,
                      append_paged_kv_cache, make_append_params, ppa_append_paged_kv, ppa_append_params_size,
                      ppa_merge_attention_states, ppa_validate_append,
                      ppa_merge_params_size, PpaParams, batch_context_with_kv_cache,  # noqa: F401
                      library_path, make_params, ppa_abi_version, ppa_gather_paged_kv,
                      ppa_paged_prefill_attention, ppa_paged_prefill_attention_noalloc, ppa_noalloc_scratch_bytes,
                      ppa_params_size, ppa_strerror,
                      ppa_validate_metadata_host, ppa_validate_page_table_csr_host, ppa_validate_shapes,
                      ppa_validate_metadata_device, check_metadata_device,
                      ppa_workspace_bytes, ppa_plan_kv_splits, ppa_plan_kv_splits_model)
