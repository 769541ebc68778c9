/*
 * ppa.h - C ABI of the MI355X (gfx950) paged prefill attention library.
 *
 * One call computes batched causal context ("prefill") attention over a
 * paged KV cache, with the semantics of trtllm_batch_context_with_kv_cache as
 * the FlashInfer API page describes it (section "Parameters"):
 *
 *   for request b:  q rows    query[cum_seq_lens_q[b] .. cum_seq_lens_q[b+1])
 *                   kv_len    seq_lens[b]  (cached prefix + new tokens)
 *                   prefix    kv_len - q_len; query row i sits at position
 *                             prefix + i (the chunked-context figure of the
 *                             TensorRT-LLM attention-backend article)
 *                   KV token t  page block_tables[b][t / page_size],
 *                               slot t % page_size; the page's address is the
 *                               pool base + page id x page stride (article
 *                               section "physical meaning of handle -> offset")
 *   logit           s_ij = bmm1_scale * <q_i, k_j>
 *   valid           j <= prefix + i  and  (window_left == -1  or
 *                   j >= prefix + i - window_left)   (inclusive left window)
 *   out_i           bmm2_scale * sum_valid e^{s_ij} v_j /
 *                   (sum_valid e^{s_ij} + [sinks] e^{sinks[h]})
 *   GQA             query head h reads kv head h / (num_qo_heads / num_kv_heads)
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers unless a parameter says "host".
 *     The caller owns every buffer; the library allocates nothing.  The only
 *     state it keeps between calls is a per-device cache of the occupancy
 *     query that sizes the persistent launch (filled on first use, guarded
 *     against concurrent first calls), plus the per-device scratch address of
 *     the no-allocation entry point below.
 *   - Metadata arrays are bare pointers, so their lengths cannot be checked
 *     here: cum_seq_lens_q, cum_seq_lens_kv and kv_indptr must hold at least
 *     batch_size + 1 entries, seq_lens and kv_last_page_len at least
 *     batch_size, block_tables at least batch_size rows.  Shorter arrays are
 *     read past their end (the Python binding checks these lengths).
 *   - Strides are in ELEMENTS of the tensor they describe.  The innermost
 *     (head_dim) stride must be 1.  The stride of a dimension of size 1 is
 *     ignored.
 *   - Functions return PPA_OK (0) or a negative ppa_status; when `msg` is not
 *     NULL a human-readable reason is written there (NUL-terminated, at most
 *     msg_len bytes).  Invalid input is rejected, never clamped or guessed.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Launches are
 *     asynchronous; a device fault surfaces at the caller's next
 *     synchronisation.
 */
#ifndef PPA_H
#define PPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PPA_ABI_VERSION 6

typedef enum ppa_status {
  PPA_OK = 0,
  PPA_ERR_NULL_POINTER = -1,   /* a required pointer is NULL                        */
  PPA_ERR_DTYPE = -2,          /* unsupported dtype combination                     */
  PPA_ERR_LAYOUT = -3,         /* kv_layout / kv_form / kv_planes out of range      */
  PPA_ERR_SHAPE = -4,          /* a size is negative or inconsistent                */
  PPA_ERR_STRIDE = -5,         /* innermost stride != 1, or a row not 16-B aligned  */
  PPA_ERR_HEADS = -6,          /* num_qo_heads not a multiple of num_kv_heads       */
  PPA_ERR_HEAD_DIM = -7,       /* head_dim not 64 or 128                            */
  PPA_ERR_PAGE_SIZE = -8,      /* page_size not a power of two in [1, 65536]        */
  PPA_ERR_WINDOW = -9,         /* window_left < -1                                  */
  PPA_ERR_LENGTHS = -10,       /* a length exceeds max_q_len / max_kv_len, or q > kv */
  PPA_ERR_TABLE = -11,         /* block table too narrow, or a page id out of range */
  PPA_ERR_METADATA = -12,      /* cum_seq_lens not monotone / not matching seq_lens */
  PPA_ERR_ALIGNMENT = -13,     /* a tensor base pointer not 16-byte aligned         */
  PPA_ERR_WORKSPACE = -14,     /* workspace smaller than ppa_workspace_bytes()      */
  PPA_ERR_ABI = -15,           /* abi_version / struct_size mismatch                */
  PPA_ERR_HIP = -16            /* the HIP runtime reported an error at launch       */
} ppa_status;

typedef enum ppa_dtype {
  PPA_DTYPE_BF16 = 1,          /* bfloat16                                          */
  PPA_DTYPE_FP8_E4M3FN = 2,    /* OCP float8 e4m3fn (no infinities, max 448)        */
  PPA_DTYPE_FP32 = 3,
  /* OCP Microscaling FP4 (MXFP4), output only: E2M1 element codes (sign,
     2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5,
     2, 3, 4, 6), two per byte with element 2i in the low nibble, plus one
     E8M0 scale byte (2^(b - 127), 0xFF = NaN) per o_sf_vec_size elements. */
  PPA_DTYPE_MXFP4 = 4
} ppa_dtype;

typedef enum ppa_kv_layout {
  PPA_KV_LAYOUT_HND = 0,       /* page = [num_kv_heads, page_size, head_dim]        */
  PPA_KV_LAYOUT_NHD = 1        /* page = [page_size, num_kv_heads, head_dim]        */
} ppa_kv_layout;

typedef enum ppa_page_table_form {
  PPA_PAGE_TABLE_PADDED = 0,   /* block_tables [batch_size, cols] (API page)      */
  PPA_PAGE_TABLE_CSR = 1       /* kv_indptr / kv_indices (flat, per request)     */
} ppa_page_table_form;

typedef enum ppa_kv_form {
  PPA_KV_SPLIT = 0,            /* two tensors: K pool and V pool                    */
  PPA_KV_COMBINED = 1          /* one tensor with K/V planes in dim 1               */
} ppa_kv_form;

/*
 * Arguments of one batched call.  Field names follow the API page.
 * Fill abi_version = PPA_ABI_VERSION and struct_size = sizeof(ppa_params).
 */
typedef struct ppa_params {
  uint32_t abi_version;
  uint32_t struct_size;

  /* query [num_tokens, num_qo_heads, head_dim], dtype query_dtype (bf16).
     Rows past cum_seq_lens_q[batch_size] are neither read for output nor
     written. */
  const void* query;
  int32_t query_dtype;
  int32_t num_tokens;
  int32_t num_qo_heads;
  int32_t head_dim;
  int64_t query_strides[3];

  /* Paged KV cache, dtype kv_dtype (bf16 or fp8 e4m3fn).
       kv_form = PPA_KV_COMBINED: kv_cache is
         [num_pages, kv_planes, num_kv_heads, page_size, head_dim]   (HND)
         [num_pages, kv_planes, page_size, num_kv_heads, head_dim]   (NHD)
         with kv_cache_strides[5]; plane 0 is K, plane 1 is V; with
         kv_planes == 1, K and V are read from the same plane.
       kv_form = PPA_KV_SPLIT: k_cache and v_cache are each
         [num_pages, num_kv_heads, page_size, head_dim]              (HND)
         [num_pages, page_size, num_kv_heads, head_dim]              (NHD)
         with k_cache_strides[4] / v_cache_strides[4]. */
  int32_t kv_form;
  int32_t kv_layout;
  int32_t kv_dtype;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t page_size;
  const void* kv_cache;
  int32_t kv_planes;
  int64_t kv_cache_strides[5];
  const void* k_cache;
  const void* v_cache;
  int64_t k_cache_strides[4];
  int64_t v_cache_strides[4];

  /* Scratch owned by the caller (API page, parameter workspace_buffer).
     Optional.  When not NULL it must hold at least ppa_workspace_bytes()
     bytes, be 16-byte aligned and be ZERO before its first use; every call
     leaves it zero again.  It holds the work counters of the balanced
     schedule: persistent workgroups pull work items from it, so no compute
     unit idles while work remains.  Calls that share one workspace must not
     run at the same time (enqueue them on one stream).  When NULL, a plain
     one-workgroup-per-item grid is launched instead. */
  void* workspace;
  size_t workspace_bytes;

  /* Metadata, all int32 device arrays.
       block_tables     [batch_size, block_tables_cols], row stride
                        block_tables_row_stride; entries are page ids in
                        [0, num_pages).  Columns past ceil(seq_lens[b] /
                        page_size) are never read.
       seq_lens         [batch_size]  KV length of each request (prefix included)
       cum_seq_lens_q   [batch_size + 1]  ragged query offsets, starting at 0
       cum_seq_lens_kv  [batch_size + 1]  may be NULL; only the host checker
                        reads it (it must equal the running sum of seq_lens).
     max_q_len / max_kv_len are upper bounds of the per-request lengths (they
     size the launch); batch_size may be 0. */
  const int32_t* block_tables;
  int32_t block_tables_cols;
  int64_t block_tables_row_stride;
  const int32_t* seq_lens;
  const int32_t* cum_seq_lens_q;
  const int32_t* cum_seq_lens_kv;
  int32_t batch_size;
  int32_t max_q_len;
  int32_t max_kv_len;

  /* Fused scales (API page, bmm1_scale / bmm2_scale).  When a *_ptr field is
     not NULL it points to one fp32 DEVICE scalar that replaces the value. */
  float bmm1_scale;
  float bmm2_scale;
  const float* bmm1_scale_ptr;
  const float* bmm2_scale_ptr;

  /* Inclusive left window; -1 = the whole sequence. */
  int32_t window_left;

  /* Per-query-head fp32 sink logits [num_qo_heads], or NULL for none. */
  const float* sinks;

  /* out [num_tokens, num_qo_heads, head_dim], dtype out_dtype: bf16, or
     PPA_DTYPE_MXFP4 (see out_sf below), when out holds packed bytes
     [num_tokens, num_qo_heads, head_dim / 2].  Strides count out's own
     units (bf16 elements, or bytes for MXFP4); the last is 1 and the other
     two are non-negative 16-byte multiples.  Only rows [cum_seq_lens_q[0],
     cum_seq_lens_q[batch_size]) are written. */
  void* out;
  int32_t out_dtype;
  int64_t out_strides[3];

  /* Page-table form.  PPA_PAGE_TABLE_PADDED: block_tables above.
     PPA_PAGE_TABLE_CSR: the flat form of the TensorRT-LLM attention-backend
     article (section on why FlashInfer uses a flat index array plus an
     indptr instead of a 2-D table); block_tables is then unused (may be
     NULL):
       kv_indptr        [batch_size + 1] int32 device array, non-decreasing;
                        request b's pages are kv_indices[kv_indptr[b] ..
                        kv_indptr[b + 1])
       kv_indices       [kv_indices_len] int32 device array of page ids in
                        [0, num_pages)
       kv_last_page_len [batch_size] int32 device array or NULL; only the host
                        checker reads it: seq_lens[b] must then equal
                        (pages_b - 1) * page_size + kv_last_page_len[b] with
                        1 <= kv_last_page_len[b] <= page_size (0 pages: 0)
     Only the first ceil(seq_lens[b] / page_size) pages of a request are read;
     indptr values are clamped to [0, kv_indices_len] on the device. */
  int32_t page_table_form;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int64_t kv_indices_len;
  const int32_t* kv_last_page_len;

  /* Log-sum-exp output, optional: fp32 [num_tokens, num_qo_heads] with
     strides lse_strides (elements), the natural log of each row's softmax
     denominator, log(sum_valid e^{s_ij} + [sinks] e^{sinks[h]}) with
     s_ij = bmm1_scale * q_i . k_j.  Written for the same rows as out; NULL:
     not written.  With it, partial results over disjoint key sets can be
     combined by ppa_merge_attention_states. */
  float* lse;
  int64_t lse_strides[2];

  /* Split-KV: the key tiles of every work item are divided into kv_splits
     chunks (0 or 1: no split; at most 256) processed by separate
     workgroups.  Each chunk's partial output and log-sum-exp go to the
     workspace, which is then required and must hold ppa_workspace_bytes(p)
     bytes; a merge pass in the same call combines them and adds the sink
     once.  The result equals the unsplit call up to fp32 summation order. */
  int32_t kv_splits;

  /* FP4 output (FlashInfer API page for trtllm_batch_context_with_kv_cache,
     parameters out (an FP4 tensor), out_dtype, o_sf_scale and
     o_sf_vec_size; the pages' NVIDIA FP4 format is carried out here as OCP
     MXFP4).  Read only when out_dtype == PPA_DTYPE_MXFP4.  Per row, the
     output o (fp32, after bmm2_scale and the softmax normalisation) becomes
     y = fp32(o * o_sf_scale); every o_sf_vec_size consecutive elements of y
     along head_dim form a block with scale 2^E, E = floor(log2(max |y|)) - 2
     (clamped below at -127; an all-zero block stores byte 0, an infinite
     maximum the NaN byte 0xFF with zero codes); each element is stored as
     the E2M1 code nearest to y / 2^E (ties to the even code, saturated at
     6, sign bit set when y < 0).  A reader recovers o ~ code * 2^E /
     o_sf_scale.
       out_sf         E8M0 scale bytes [num_tokens, num_qo_heads,
                      head_dim / o_sf_vec_size], caller-owned device memory
       out_sf_strides token and head strides in bytes (non-negative); the
                      block index is contiguous
       o_sf_scale     finite and > 0 (1 = plain MXFP4)
       o_sf_vec_size  16 or 32 (32 is the OCP block size) */
  uint8_t* out_sf;
  int64_t out_sf_strides[2];
  float o_sf_scale;
  int32_t o_sf_vec_size;

  /* Arithmetic for an fp8 cache.  The TokenSpeed backend source casts Q to
     e4m3fn before the call whenever its KV cache is fp8 (its Q-preparation
     step), with q_scale 1 folded into bmm1_scale (its scale computation);
     here Q stays bf16 at the boundary and the kernel may do that rounding
     itself.
       0  each e4m3fn code is widened to bf16 (exact) and both products run
          on the bf16 MFMA; Q and the softmax weights stay bf16
       1  head_dim 128 only: Q (after the sign of bmm1_scale) and the
          softmax weights are rounded to e4m3fn (nearest even, Q saturated
          at +-448) and both products run on the fp8 MFMA at twice the bf16
          rate; the row sums add the rounded weights.  Each logit then
          carries the rounding of its Q elements (unit roundoff 2^-4).
     Any other value, or 1 with a bf16 cache or head_dim 64, is
     PPA_ERR_DTYPE. */
  int32_t fp8_compute;
} ppa_params;

/*
 * New tokens to write into a paged cache before attention (the KV save step
 * of the TokenSpeed backend source: K and V written at out_cache_loc, with
 * per-tensor scales for an fp8 cache).  The cache itself is described by a
 * ppa_params (its cache, page and head fields; the rest is not read).
 */
typedef struct ppa_append_params {
  uint32_t abi_version;
  uint32_t struct_size;
  const void* k_new;            /* [num_new, num_kv_heads, head_dim], dtype new_dtype (bf16) */
  const void* v_new;
  int32_t new_dtype;
  int32_t num_new;              /* >= 0 */
  int64_t k_new_strides[3];     /* elements; innermost 1, the others 16-byte multiples */
  int64_t v_new_strides[3];
  /* [num_new] int64 DEVICE array: page_id * page_size + slot of each token
     (out_cache_loc); a negative entry skips the token, and an entry whose
     page is >= num_pages is skipped by the device as well. */
  const int64_t* slot_mapping;
  /* fp8 e4m3fn cache: the stored code is e4m3fn(fp32(x) / fp32(scale)),
     nearest value with ties to even, magnitudes beyond 448 saturated to 448,
     NaN kept.  A bf16 cache stores x as it is.  *_ptr, when not NULL, point
     to device fp32 scalars that replace the values. */
  float k_scale;
  float v_scale;
  const float* k_scale_ptr;
  const float* v_scale_ptr;
} ppa_append_params;

/*
 * Partial attention states to combine (log-sum-exp merge): part s holds, per
 * (row, head), an output o_s normalized over its own key set and that set's
 * log-denominator lse_s (natural log; -inf for an empty set).  The merge
 * writes out = sum_s e^{lse_s - L} o_s with L = log(sum_s e^{lse_s} +
 * [sinks] e^{sinks[h]}), and L to lse_out.  Use: combining calls that each
 * saw a slice of the KV (context parallelism), sinks given only here.
 */
typedef struct ppa_merge_params {
  uint32_t abi_version;
  uint32_t struct_size;
  int32_t num_parts;          /* >= 1 */
  int32_t num_rows;           /* >= 0 (tokens) */
  int32_t num_heads;          /* >= 1 */
  int32_t head_dim;           /* 64 or 128 */
  const float* o_parts;       /* [num_parts, num_rows, num_heads, head_dim] fp32, contiguous */
  const float* lse_parts;     /* [num_parts, num_rows, num_heads] fp32, contiguous */
  const float* sinks;         /* [num_heads] fp32 or NULL */
  void* out;                  /* [num_rows, num_heads, head_dim], dtype out_dtype: bf16, or MXFP4
                                 packed bytes [num_rows, num_heads, head_dim / 2] */
  int32_t out_dtype;
  int64_t out_strides[3];     /* out's units (bf16 elements / bytes); out_strides[2] == 1, the others even */
  float* lse_out;             /* [num_rows, num_heads] fp32 or NULL */
  int64_t lse_out_strides[2];
  /* MXFP4 output, as in ppa_params (read only when out_dtype == PPA_DTYPE_MXFP4) */
  uint8_t* out_sf;
  int64_t out_sf_strides[2];
  float o_sf_scale;
  int32_t o_sf_vec_size;
} ppa_merge_params;

/* ABI guards for bindings: the version this library was built with and
   sizeof(ppa_params). */
int32_t ppa_abi_version(void);
size_t ppa_params_size(void);

/* Static description of a status code (never NULL). */
const char* ppa_strerror(int32_t status);

/*
 * Host-only check of everything the call can be checked for without reading
 * device memory: pointers, dtypes, enums, head counts, head_dim, page size,
 * window, strides and alignment, block-table width >= ceil(max_kv_len /
 * page_size) (the table-width rule of the article's TrtllmAttentionMetadata
 * section), workspace size and alignment.  Cheap; ppa_paged_prefill_attention runs it on
 * every call.
 */
int32_t ppa_validate_shapes(const ppa_params* p, char* msg, size_t msg_len);

/*
 * The deep metadata check, on HOST copies of the device metadata (the
 * debug page-table validation of the article's FlashInfer section):
 * cum_seq_lens_q starts at 0, is non-decreasing and ends <= num_tokens;
 * 0 <= q_len <= kv_len for every request (a query row with an empty causal
 * span has no defined output); q_len <= max_q_len, kv_len <= max_kv_len;
 * cum_seq_lens_kv (if not NULL) is the running sum of seq_lens; every table
 * entry a request reaches lies in [0, num_pages).  block_tables uses the
 * row stride of p->block_tables_row_stride; with the CSR page-table form it
 * is not read (may be NULL).  Pure function of its inputs.
 */
int32_t ppa_validate_metadata_host(const ppa_params* p, const int32_t* cum_seq_lens_q,
                                   const int32_t* cum_seq_lens_kv, const int32_t* seq_lens,
                                   const int32_t* block_tables, char* msg, size_t msg_len);

/*
 * The page-table part of the deep check for the CSR form, on HOST copies:
 * kv_indptr[0] >= 0, non-decreasing, kv_indptr[batch_size] <= kv_indices_len;
 * every request has at least ceil(seq_lens[b] / page_size) pages, each a page
 * id in [0, num_pages); with kv_last_page_len, the page count and last-page
 * length reproduce seq_lens exactly.  (ppa_validate_metadata_host checks the
 * lengths and skips the table for this form.)  Pure function of its inputs.
 */
int32_t ppa_validate_page_table_csr_host(const ppa_params* p, const int32_t* seq_lens,
                                         const int32_t* kv_indptr, const int32_t* kv_indices,
                                         const int32_t* kv_last_page_len, char* msg, size_t msg_len);

/*
 * The same checks on the DEVICE arrays of `p` (TensorRT-LLM attention-
 * backend article: the self-check step of its FlashInfer section and the
 * row-count check of its block-offset section ask for bad metadata to fail
 * loudly; the attention call itself only clamps).  Runs ppa_validate_shapes
 * on the host, then enqueues three small kernels on `stream` and returns
 * without waiting; no allocation.  They evaluate every rule of
 * ppa_validate_metadata_host (cum_seq_lens_kv only when not NULL) and, for
 * the CSR form, of ppa_validate_page_table_csr_host (kv_last_page_len only
 * when not NULL), and write the FIRST violated rule in that order
 * (ppa_validate_metadata_host's rules, then the CSR ones) to `result`:
 *   result[0]  PPA_OK, PPA_ERR_LENGTHS, PPA_ERR_TABLE or PPA_ERR_METADATA,
 *              the code the host functions return for that rule
 *   result[1]  the index of the request the rule concerns, or -1 for a rule
 *              on the whole batch (cum_seq_lens_q[0], its last entry,
 *              cum_seq_lens_kv[0], kv_indptr[0], kv_indptr[batch_size])
 * `result` is caller-owned device memory of two int32, 8-byte aligned (it
 * holds a 64-bit key while the kernels run); read it after the stream has
 * passed this call.  The metadata arrays must have the lengths ppa_params
 * states (batch_size + 1 / batch_size entries); table entries are read only
 * inside a request's own row or index slice, and only after the bounds that
 * make the read valid have passed.  Returns a ppa_validate_shapes error,
 * PPA_ERR_NULL_POINTER (result NULL), PPA_ERR_ALIGNMENT (result not 8-byte
 * aligned) or PPA_ERR_HIP (launch failure); otherwise PPA_OK, whatever the
 * metadata holds.
 */
int32_t ppa_validate_metadata_device(const ppa_params* p, int32_t* result, void* stream);

/* Bytes of workspace a call needs: 256 for the balanced schedule's counters,
   plus the partial outputs and log-sum-exps of split-KV (kv_splits > 1:
   kv_splits * num_tokens * num_qo_heads * (head_dim + 1) * 4 bytes, each
   array rounded up to 256).  p may be NULL (then 256). */
size_t ppa_workspace_bytes(const ppa_params* p);

/*
 * Split-KV planning (host only).  The TensorRT-LLM prepare() dissection page,
 * in its FlashInfer backend part, routes the decode segment to a split-K
 * kernel and the prefill segment to the paged-prefill one; here one call
 * serves both, and this chooses kv_splits for it.
 *
 * ppa_plan_kv_splits_model: the cost model, a pure function.  work_items =
 * (query tiles) x batch x kv heads x head groups of the call; resident = the
 * workgroups the device holds at once; key_tiles = 64-key tiles of the
 * longest work item.  With work_items >= resident there is no idle slot and
 * the answer is 1.  Otherwise it returns the S in [1, max_splits] (S <=
 * key_tiles / 4, so a chunk keeps at least four tiles) that minimises
 *   ceil(work_items * S / resident) * (ceil(key_tiles / S) + 3) + S / 2,
 * i.e. rounds of workgroups times the tiles of a chunk plus a per-chunk
 * start-up cost, plus the merge's cost per split; the smallest S on ties.
 * Returns 1 for non-positive inputs.
 *
 * ppa_plan_kv_splits: the model applied to the call `p` on the current
 * device (its compute-unit count times the occupancy of the kernel variant
 * `p` selects).  The kv_splits field of `p` is ignored; only splits whose
 * ppa_workspace_bytes fit p->workspace_bytes are considered (1 when
 * p->workspace is NULL).  Returns the split count (>= 1), or a negative
 * ppa_status if `p` fails ppa_validate_shapes or the device cannot be
 * queried.  The caller then sets p->kv_splits to it.
 */
int32_t ppa_plan_kv_splits_model(int64_t work_items, int64_t resident, int64_t key_tiles, int32_t max_splits);
int32_t ppa_plan_kv_splits(const ppa_params* p);

/*
 * The batched paged prefill attention call.  Runs ppa_validate_shapes, then
 * enqueues the kernel on `stream` and returns without waiting.  No host
 * synchronisation, no allocation.  Metadata values are trusted to pass
 * ppa_validate_metadata_host; if they do not, the output is unspecified but
 * every memory access stays inside the tensors the shapes describe (page ids
 * and table columns are clamped, query rows are bounded by num_tokens).
 */
int32_t ppa_paged_prefill_attention(const ppa_params* p, void* stream);

/*
 * The same call for callers that cannot allocate or own a workspace (code
 * under HIP graph capture, serving loops that forbid hipMalloc): instead of
 * p->workspace, which must be NULL here (else PPA_ERR_WORKSPACE), the
 * library uses a scratch array of ppa_noalloc_scratch_bytes() (16 MiB) in
 * device memory that it owns, one per device, held until the process ends.
 * Calls whose ppa_workspace_bytes(p) exceeds that size (split-KV with many
 * partial rows) return PPA_ERR_WORKSPACE.  The persistent schedule always
 * runs; each call first clears the scheduler counters with a small kernel
 * on `stream`.  The scratch keeps the last call's contents, and every call
 * on one device shares it: calls that overlap in time on one device (on
 * different streams, or from different threads) race.  Otherwise as
 * ppa_paged_prefill_attention: no host synchronisation and no allocation
 * (the first call on a device looks up the array's address).
 */
int32_t ppa_paged_prefill_attention_noalloc(const ppa_params* p, void* stream);

/* Size in bytes of the per-device scratch array of the no-allocation entry
   point. */
size_t ppa_noalloc_scratch_bytes(void);

/*
 * Combine partial attention states (see ppa_merge_params); enqueued on
 * `stream`, no host synchronisation, no allocation.  Returns PPA_ERR_ABI,
 * PPA_ERR_NULL_POINTER, PPA_ERR_SHAPE, PPA_ERR_HEAD_DIM, PPA_ERR_DTYPE,
 * PPA_ERR_STRIDE or PPA_ERR_ALIGNMENT for bad arguments.
 */
int32_t ppa_merge_attention_states(const ppa_merge_params* m, void* stream);

/* sizeof(ppa_merge_params) of this library, for bindings. */
size_t ppa_merge_params_size(void);

/*
 * Host-only check of an append: the cache description in `cache` (dtypes,
 * layout, form (the one-plane combined form is rejected: K and V would share
 * the slots), heads, head_dim, page size, pages, cache pointers, strides,
 * alignment) and the new tokens in `a` (pointers, bf16 dtype, strides,
 * alignment).
 */
int32_t ppa_validate_append(const ppa_params* cache, const ppa_append_params* a, char* msg, size_t msg_len);

/*
 * Write the new tokens of `a` into the cache described by `cache`:
 * ppa_validate_append, then one kernel on `stream`.  No host
 * synchronisation, no allocation.  Tokens sharing a slot race.
 */
int32_t ppa_append_paged_kv(const ppa_params* cache, const ppa_append_params* a, void* stream);

/* sizeof(ppa_append_params) of this library, for bindings. */
size_t ppa_append_params_size(void);

/*
 * Address-unit check: copies the first seq_lens[b] K (kv_idx 0) or V
 * (kv_idx 1) tokens of every request out of the pages into `dst`, a
 * contiguous [dst_rows, num_kv_heads, head_dim] device tensor of the cache
 * dtype, request b at rows [cum_seq_lens_kv[b], cum_seq_lens_kv[b] +
 * seq_lens[b]) - the contiguous token-major gather of the article's
 * VanillaAttention path.  Rows at or past dst_rows are not written.
 * Needs cum_seq_lens_kv.
 */
int32_t ppa_gather_paged_kv(const ppa_params* p, int32_t kv_idx, void* dst, int64_t dst_rows,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PPA_H */
