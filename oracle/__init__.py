"""CPU oracle for batched paged prefill attention - TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The library's own code never does: it must fail loudly when
its HIP extension is missing rather than fall back to anything here.
"""
from .paged_attention import (E4M3FN_TABLE, append_paged_kv, attention_one_request, attention_rows,  # noqa: F401
                              encode_e4m3fn,
                              decode_bf16, decode_e4m3fn, e4m3fn_value, gather_paged_kv,
                              log_sum_exp_rows, merge_states, paged_prefill_attention,
                              paged_prefill_lse, partial_state)
from .mxfp4 import (E2M1_TABLE, dequantize_mxfp4, e8m0_value, encode_e2m1, mx_scale_byte,  # noqa: F401
                     mxfp4_output, quantize_mxfp4, unpack_e2m1)
