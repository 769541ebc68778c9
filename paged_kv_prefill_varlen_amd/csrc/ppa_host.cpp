// Host-only part of the C ABI: status strings, the shape validator, the
// host-copy metadata validator and the cache-view resolution.  Plain C++17
// with no HIP headers, so every function here runs on a machine without a
// GPU.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ppa_internal.h"

namespace ppa {

int dtype_bytes(int32_t dtype) {
  switch (dtype) {
    case PPA_DTYPE_BF16: return 2;
    case PPA_DTYPE_FP8_E4M3FN: return 1;
    case PPA_DTYPE_FP32: return 4;
    default: return 0;
  }
}

int32_t fail(int32_t status, char* msg, size_t msg_len, const char* fmt, ...) {
  if (msg != nullptr && msg_len > 0) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, msg_len, fmt, ap);
    va_end(ap);
  }
  return status;
}

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Per-dimension (page, kv head, token slot, head_dim) strides of one plane,
// as given, before zeroing the ones of size-1 dimensions.
struct PlaneStrides {
  int64_t page, head, tok, dim;
};

PlaneStrides plane_strides(const ppa_params* p, int which /*0 K, 1 V*/) {
  PlaneStrides s{};
  const bool hnd = p->kv_layout == PPA_KV_LAYOUT_HND;
  if (p->kv_form == PPA_KV_SPLIT) {
    const int64_t* st = which == 0 ? p->k_cache_strides : p->v_cache_strides;
    s.page = st[0];
    s.head = hnd ? st[1] : st[2];
    s.tok = hnd ? st[2] : st[1];
    s.dim = st[3];
  } else {
    const int64_t* st = p->kv_cache_strides;
    s.page = st[0];
    s.head = hnd ? st[2] : st[3];
    s.tok = hnd ? st[3] : st[2];
    s.dim = st[4];
  }
  return s;
}

// A row stride is usable when it is non-negative and keeps 16-byte row
// alignment; size-1 dimensions are exempt.
bool row_stride_ok(int64_t stride, int64_t extent, int elem_bytes) {
  if (extent <= 1) return true;
  if (stride < 0) return false;
  return (stride * elem_bytes) % 16 == 0;
}

}  // namespace

void resolve_cache(const ppa_params* p, CacheView* v) {
  PlaneStrides ks = plane_strides(p, 0);
  PlaneStrides vs = plane_strides(p, 1);
  const int eb = dtype_bytes(p->kv_dtype);
  if (p->kv_form == PPA_KV_SPLIT) {
    v->k_base = p->k_cache;
    v->v_base = p->v_cache;
  } else {
    v->k_base = p->kv_cache;
    const int64_t plane = p->kv_planes == 2 ? p->kv_cache_strides[1] : 0;
    v->v_base = static_cast<const char*>(p->kv_cache) + plane * eb;
  }
  auto z = [](int64_t stride, int64_t extent) { return extent <= 1 ? 0 : stride; };
  v->k_page = z(ks.page, p->num_pages);
  v->k_head = z(ks.head, p->num_kv_heads);
  v->k_tok = z(ks.tok, p->page_size);
  v->v_page = z(vs.page, p->num_pages);
  v->v_head = z(vs.head, p->num_kv_heads);
  v->v_tok = z(vs.tok, p->page_size);
}

}  // namespace ppa

using namespace ppa;

extern "C" {

int32_t ppa_abi_version(void) { return PPA_ABI_VERSION; }

size_t ppa_params_size(void) { return sizeof(ppa_params); }

const char* ppa_strerror(int32_t status) {
  switch (status) {
    case PPA_OK: return "ok";
    case PPA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case PPA_ERR_DTYPE: return "unsupported dtype";
    case PPA_ERR_LAYOUT: return "invalid kv_layout / kv_form / kv_planes";
    case PPA_ERR_SHAPE: return "invalid or inconsistent shape";
    case PPA_ERR_STRIDE: return "unsupported stride (innermost must be 1, rows 16-byte aligned)";
    case PPA_ERR_HEADS: return "num_qo_heads must be a positive multiple of num_kv_heads";
    case PPA_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case PPA_ERR_PAGE_SIZE: return "page_size must be a power of two in [1, 65536]";
    case PPA_ERR_WINDOW: return "window_left must be >= -1";
    case PPA_ERR_LENGTHS: return "sequence lengths out of range";
    case PPA_ERR_TABLE: return "block table too narrow or page id out of range";
    case PPA_ERR_METADATA: return "inconsistent cum_seq_lens / seq_lens";
    case PPA_ERR_ALIGNMENT: return "tensor base pointer not 16-byte aligned";
    case PPA_ERR_WORKSPACE: return "workspace too small";
    case PPA_ERR_ABI: return "ppa_params ABI mismatch";
    case PPA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t ppa_workspace_bytes(const ppa_params* p) {
  size_t bytes = 256;   // scheduler counters (9 x uint32), rounded up
  if (p != nullptr && p->kv_splits > 1 && p->num_tokens > 0 && p->num_qo_heads > 0 && p->head_dim > 0) {
    const size_t rows = static_cast<size_t>(p->kv_splits) * p->num_tokens * p->num_qo_heads;
    auto round = [](size_t x) { return (x + 255) / 256 * 256; };
    bytes += round(rows * p->head_dim * sizeof(float)) + round(rows * sizeof(float));
  }
  return bytes;
}

int32_t ppa_plan_kv_splits_model(int64_t work_items, int64_t resident, int64_t key_tiles, int32_t max_splits) {
  if (work_items <= 0 || resident <= 0 || key_tiles <= 0 || max_splits <= 1 || work_items >= resident) return 1;
  int64_t top = key_tiles / 4;
  if (top > max_splits) top = max_splits;
  int32_t best = 1;
  double best_cost = 0.0;
  for (int64_t s = 1; s <= (top > 1 ? top : 1); ++s) {
    const int64_t rounds = (work_items * s + resident - 1) / resident;
    const int64_t chunk = (key_tiles + s - 1) / s;
    const double cost = static_cast<double>(rounds) * static_cast<double>(chunk + 3) + 0.5 * static_cast<double>(s);
    if (s == 1 || cost < best_cost) {
      best_cost = cost;
      best = static_cast<int32_t>(s);
    }
  }
  return best;
}

int32_t ppa_validate_shapes(const ppa_params* p, char* msg, size_t msg_len) {
  if (msg != nullptr && msg_len > 0) msg[0] = '\0';
  if (p == nullptr) return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "params is NULL");
  if (p->abi_version != PPA_ABI_VERSION || p->struct_size != sizeof(ppa_params))
    return fail(PPA_ERR_ABI, msg, msg_len, "abi_version %u / struct_size %u, library has %d / %zu",
                p->abi_version, p->struct_size, PPA_ABI_VERSION, sizeof(ppa_params));

  // dtypes
  if (p->query_dtype != PPA_DTYPE_BF16)
    return fail(PPA_ERR_DTYPE, msg, msg_len, "query dtype %d: only bf16 is supported", p->query_dtype);
  if (p->out_dtype != PPA_DTYPE_BF16 && p->out_dtype != PPA_DTYPE_MXFP4)
    return fail(PPA_ERR_DTYPE, msg, msg_len, "out dtype %d: bf16 or mxfp4", p->out_dtype);
  const bool mxfp4 = p->out_dtype == PPA_DTYPE_MXFP4;
  if (mxfp4 && p->o_sf_vec_size != 16 && p->o_sf_vec_size != 32)
    return fail(PPA_ERR_SHAPE, msg, msg_len, "o_sf_vec_size %d: 16 or 32", p->o_sf_vec_size);
  if (mxfp4 && !(p->o_sf_scale > 0.f && p->o_sf_scale <= 3.402823466e38f))
    return fail(PPA_ERR_SHAPE, msg, msg_len, "o_sf_scale must be finite and > 0");
  if (p->kv_dtype != PPA_DTYPE_BF16 && p->kv_dtype != PPA_DTYPE_FP8_E4M3FN)
    return fail(PPA_ERR_DTYPE, msg, msg_len, "kv dtype %d: bf16 or fp8 e4m3fn", p->kv_dtype);
  if (p->fp8_compute != 0 && p->fp8_compute != 1)
    return fail(PPA_ERR_DTYPE, msg, msg_len, "fp8_compute %d: 0 or 1", p->fp8_compute);
  if (p->fp8_compute == 1 && (p->kv_dtype != PPA_DTYPE_FP8_E4M3FN || p->head_dim != 128))
    return fail(PPA_ERR_DTYPE, msg, msg_len, "fp8_compute needs an fp8 e4m3fn cache at head_dim 128");

  // enums
  if (p->kv_layout != PPA_KV_LAYOUT_HND && p->kv_layout != PPA_KV_LAYOUT_NHD)
    return fail(PPA_ERR_LAYOUT, msg, msg_len, "kv_layout %d", p->kv_layout);
  if (p->kv_form != PPA_KV_SPLIT && p->kv_form != PPA_KV_COMBINED)
    return fail(PPA_ERR_LAYOUT, msg, msg_len, "kv_form %d", p->kv_form);
  if (p->kv_form == PPA_KV_COMBINED && p->kv_planes != 1 && p->kv_planes != 2)
    return fail(PPA_ERR_LAYOUT, msg, msg_len, "kv_cache dim 1 is %d, must be 1 or 2", p->kv_planes);
  if (p->page_table_form != PPA_PAGE_TABLE_PADDED && p->page_table_form != PPA_PAGE_TABLE_CSR)
    return fail(PPA_ERR_LAYOUT, msg, msg_len, "page_table_form %d", p->page_table_form);
  const bool csr = p->page_table_form == PPA_PAGE_TABLE_CSR;

  // sizes
  if (p->num_tokens < 0 || p->batch_size < 0 || p->max_q_len < 0 || p->max_kv_len < 0 ||
      p->num_pages < 0 || (!csr && p->block_tables_cols < 0) || (csr && p->kv_indices_len < 0))
    return fail(PPA_ERR_SHAPE, msg, msg_len, "negative size");
  if (p->num_kv_heads <= 0 || p->num_qo_heads <= 0 || p->num_qo_heads % p->num_kv_heads != 0)
    return fail(PPA_ERR_HEADS, msg, msg_len, "num_qo_heads %d, num_kv_heads %d", p->num_qo_heads,
                p->num_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PPA_ERR_HEAD_DIM, msg, msg_len, "head_dim %d", p->head_dim);
  if (p->page_size < 1 || p->page_size > 65536 || (p->page_size & (p->page_size - 1)) != 0)
    return fail(PPA_ERR_PAGE_SIZE, msg, msg_len, "page_size %d", p->page_size);
  if (p->window_left < -1) return fail(PPA_ERR_WINDOW, msg, msg_len, "window_left %d", p->window_left);
  if (p->kv_splits < 0 || p->kv_splits > 256)
    return fail(PPA_ERR_SHAPE, msg, msg_len, "kv_splits %d outside [0, 256]", p->kv_splits);
  if (p->max_q_len > p->max_kv_len)
    return fail(PPA_ERR_LENGTHS, msg, msg_len, "max_q_len %d > max_kv_len %d", p->max_q_len,
                p->max_kv_len);

  const bool work = p->batch_size > 0 && p->max_q_len > 0 && p->num_tokens > 0;
  if (p->batch_size > 0 && csr) {
    if (p->seq_lens == nullptr || p->cum_seq_lens_q == nullptr || p->kv_indptr == nullptr ||
        p->kv_indices == nullptr)
      return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "seq_lens / cum_seq_lens_q / kv_indptr / kv_indices");
    if (p->max_kv_len > 0 && p->num_pages < 1)
      return fail(PPA_ERR_SHAPE, msg, msg_len, "num_pages is 0 but max_kv_len is %d", p->max_kv_len);
  } else if (p->batch_size > 0) {
    if (p->seq_lens == nullptr || p->cum_seq_lens_q == nullptr || p->block_tables == nullptr)
      return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "seq_lens / cum_seq_lens_q / block_tables");
    const int64_t need = (static_cast<int64_t>(p->max_kv_len) + p->page_size - 1) / p->page_size;
    if (p->block_tables_cols < need)
      return fail(PPA_ERR_TABLE, msg, msg_len,
                  "block_tables has %d columns, max_kv_len %d needs %lld pages of %d",
                  p->block_tables_cols, p->max_kv_len, static_cast<long long>(need), p->page_size);
    if (p->batch_size > 1 && p->block_tables_row_stride < p->block_tables_cols)
      return fail(PPA_ERR_STRIDE, msg, msg_len, "block_tables row stride %lld < %d columns",
                  static_cast<long long>(p->block_tables_row_stride), p->block_tables_cols);
    if (p->max_kv_len > 0 && p->num_pages < 1)
      return fail(PPA_ERR_SHAPE, msg, msg_len, "num_pages is 0 but max_kv_len is %d", p->max_kv_len);
  }
  if (!work) return PPA_OK;

  if (p->query == nullptr || p->out == nullptr)
    return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "query / out");
  if (p->kv_form == PPA_KV_SPLIT && (p->k_cache == nullptr || p->v_cache == nullptr))
    return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "k_cache / v_cache");
  if (p->kv_form == PPA_KV_COMBINED && p->kv_cache == nullptr)
    return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "kv_cache");

  // strides and alignment
  const int kb = ppa::dtype_bytes(p->kv_dtype);
  const int D = p->head_dim;
  if (p->query_strides[2] != 1 || p->out_strides[2] != 1)
    return fail(PPA_ERR_STRIDE, msg, msg_len, "query / out head_dim stride must be 1");
  const int ob = mxfp4 ? 1 : 2;   // bytes per unit of out
  if (!row_stride_ok(p->query_strides[0], p->num_tokens, 2) ||
      !row_stride_ok(p->query_strides[1], p->num_qo_heads, 2) ||
      !row_stride_ok(p->out_strides[0], p->num_tokens, ob) ||
      !row_stride_ok(p->out_strides[1], p->num_qo_heads, ob))
    return fail(PPA_ERR_STRIDE, msg, msg_len, "query / out token and head strides must be 16-byte multiples");
  if (mxfp4 && p->out_sf == nullptr) return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "out_sf");
  if (mxfp4 && (p->out_sf_strides[0] < 0 || p->out_sf_strides[1] < 0))
    return fail(PPA_ERR_STRIDE, msg, msg_len, "out_sf strides must be non-negative");
  for (int w = 0; w < 2; ++w) {
    PlaneStrides s = plane_strides(p, w);
    if (s.dim != 1 && D > 1)
      return fail(PPA_ERR_STRIDE, msg, msg_len, "%s cache head_dim stride must be 1", w ? "V" : "K");
    if (!row_stride_ok(s.page, p->num_pages, kb) || !row_stride_ok(s.head, p->num_kv_heads, kb) ||
        !row_stride_ok(s.tok, p->page_size, kb))
      return fail(PPA_ERR_STRIDE, msg, msg_len,
                  "%s cache page/head/token strides must be non-negative 16-byte multiples", w ? "V" : "K");
  }
  if (p->kv_form == PPA_KV_COMBINED && p->kv_planes == 2 &&
      !row_stride_ok(p->kv_cache_strides[1], 2, kb))
    return fail(PPA_ERR_STRIDE, msg, msg_len, "kv_cache plane stride must be a 16-byte multiple");
  if (!aligned16(p->query) || !aligned16(p->out))
    return fail(PPA_ERR_ALIGNMENT, msg, msg_len, "query / out");
  if (p->kv_form == PPA_KV_SPLIT ? (!aligned16(p->k_cache) || !aligned16(p->v_cache))
                                 : !aligned16(p->kv_cache))
    return fail(PPA_ERR_ALIGNMENT, msg, msg_len, "kv cache");
  if ((reinterpret_cast<uintptr_t>(p->sinks) & 3u) != 0)
    return fail(PPA_ERR_ALIGNMENT, msg, msg_len, "sinks");
  if ((reinterpret_cast<uintptr_t>(p->lse) & 3u) != 0)
    return fail(PPA_ERR_ALIGNMENT, msg, msg_len, "lse");
  if (p->lse != nullptr && (p->lse_strides[0] < 0 || p->lse_strides[1] < 0))
    return fail(PPA_ERR_STRIDE, msg, msg_len, "lse strides must be non-negative");

  if (p->kv_splits > 1 && p->workspace == nullptr)
    return fail(PPA_ERR_WORKSPACE, msg, msg_len, "kv_splits %d needs a workspace of %zu bytes", p->kv_splits,
                ppa_workspace_bytes(p));
  if (p->workspace != nullptr && p->workspace_bytes < ppa_workspace_bytes(p))
    return fail(PPA_ERR_WORKSPACE, msg, msg_len, "workspace of %zu bytes, need %zu",
                p->workspace_bytes, ppa_workspace_bytes(p));
  if (!aligned16(p->workspace)) return fail(PPA_ERR_ALIGNMENT, msg, msg_len, "workspace");
  return PPA_OK;
}

int32_t ppa_validate_metadata_host(const ppa_params* p, const int32_t* cu_q, const int32_t* cu_kv,
                                   const int32_t* seq_lens, const int32_t* block_tables, char* msg,
                                   size_t msg_len) {
  if (msg != nullptr && msg_len > 0) msg[0] = '\0';
  if (p == nullptr) return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "params is NULL");
  const int B = p->batch_size;
  if (B < 0) return fail(PPA_ERR_SHAPE, msg, msg_len, "batch_size %d", B);
  if (B == 0) return PPA_OK;
  const bool csr = p->page_table_form == PPA_PAGE_TABLE_CSR;
  if (cu_q == nullptr || seq_lens == nullptr || (!csr && block_tables == nullptr))
    return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "host metadata");
  if (p->page_size < 1) return fail(PPA_ERR_PAGE_SIZE, msg, msg_len, "page_size %d", p->page_size);
  if (cu_q[0] != 0) return fail(PPA_ERR_METADATA, msg, msg_len, "cum_seq_lens_q[0] = %d, must be 0", cu_q[0]);
  const int64_t rs = B > 1 ? p->block_tables_row_stride : p->block_tables_cols;
  int64_t kv_run = 0;
  if (cu_kv != nullptr && cu_kv[0] != 0)
    return fail(PPA_ERR_METADATA, msg, msg_len, "cum_seq_lens_kv[0] = %d, must be 0", cu_kv[0]);
  for (int b = 0; b < B; ++b) {
    const int64_t q_len = static_cast<int64_t>(cu_q[b + 1]) - cu_q[b];
    const int64_t kv_len = seq_lens[b];
    if (q_len < 0)
      return fail(PPA_ERR_METADATA, msg, msg_len, "cum_seq_lens_q decreases at request %d", b);
    if (kv_len < 0) return fail(PPA_ERR_LENGTHS, msg, msg_len, "seq_lens[%d] = %lld", b, (long long)kv_len);
    if (q_len > kv_len)
      return fail(PPA_ERR_LENGTHS, msg, msg_len,
                  "request %d: q_len %lld > kv_len %lld (an empty causal span has no output)", b,
                  (long long)q_len, (long long)kv_len);
    if (q_len > p->max_q_len)
      return fail(PPA_ERR_LENGTHS, msg, msg_len, "request %d: q_len %lld > max_q_len %d", b,
                  (long long)q_len, p->max_q_len);
    if (kv_len > p->max_kv_len)
      return fail(PPA_ERR_LENGTHS, msg, msg_len, "request %d: kv_len %lld > max_kv_len %d", b,
                  (long long)kv_len, p->max_kv_len);
    kv_run += kv_len;
    if (cu_kv != nullptr && cu_kv[b + 1] != kv_run)
      return fail(PPA_ERR_METADATA, msg, msg_len,
                  "cum_seq_lens_kv[%d] = %d, the running sum of seq_lens is %lld", b + 1, cu_kv[b + 1],
                  (long long)kv_run);
    if (csr) continue;   // the table is checked by ppa_validate_page_table_csr_host
    const int64_t pages = (kv_len + p->page_size - 1) / p->page_size;
    if (pages > p->block_tables_cols)
      return fail(PPA_ERR_TABLE, msg, msg_len, "request %d needs %lld pages, table has %d columns", b,
                  (long long)pages, p->block_tables_cols);
    for (int64_t j = 0; j < pages; ++j) {
      const int32_t id = block_tables[b * rs + j];
      if (id < 0 || id >= p->num_pages)
        return fail(PPA_ERR_TABLE, msg, msg_len, "block_tables[%d][%lld] = %d outside [0, %d)", b,
                    (long long)j, id, p->num_pages);
    }
  }
  if (cu_q[B] > p->num_tokens)
    return fail(PPA_ERR_METADATA, msg, msg_len, "cum_seq_lens_q[%d] = %d > num_tokens %d", B, cu_q[B],
                p->num_tokens);
  return PPA_OK;
}

int32_t ppa_validate_page_table_csr_host(const ppa_params* p, const int32_t* seq_lens,
                                         const int32_t* kv_indptr, const int32_t* kv_indices,
                                         const int32_t* kv_last_page_len, char* msg, size_t msg_len) {
  if (msg != nullptr && msg_len > 0) msg[0] = '\0';
  if (p == nullptr) return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "params is NULL");
  const int B = p->batch_size;
  if (B < 0) return fail(PPA_ERR_SHAPE, msg, msg_len, "batch_size %d", B);
  if (B == 0) return PPA_OK;
  if (seq_lens == nullptr || kv_indptr == nullptr || (kv_indices == nullptr && p->kv_indices_len > 0))
    return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "host page table");
  if (p->page_size < 1) return fail(PPA_ERR_PAGE_SIZE, msg, msg_len, "page_size %d", p->page_size);
  if (kv_indptr[0] < 0) return fail(PPA_ERR_TABLE, msg, msg_len, "kv_indptr[0] = %d", kv_indptr[0]);
  for (int b = 0; b < B; ++b)
    if (kv_indptr[b + 1] < kv_indptr[b])
      return fail(PPA_ERR_TABLE, msg, msg_len, "kv_indptr decreases at request %d", b);
  if (kv_indptr[B] > p->kv_indices_len)
    return fail(PPA_ERR_TABLE, msg, msg_len, "kv_indptr[%d] = %d > kv_indices_len %lld", B, kv_indptr[B],
                static_cast<long long>(p->kv_indices_len));
  for (int b = 0; b < B; ++b) {
    const int64_t kv_len = seq_lens[b];
    const int64_t have = static_cast<int64_t>(kv_indptr[b + 1]) - kv_indptr[b];
    const int64_t need = kv_len > 0 ? (kv_len + p->page_size - 1) / p->page_size : 0;
    if (have < need)
      return fail(PPA_ERR_TABLE, msg, msg_len, "request %d needs %lld pages, kv_indptr gives %lld", b,
                  static_cast<long long>(need), static_cast<long long>(have));
    for (int64_t j = 0; j < need; ++j) {
      const int32_t id = kv_indices[kv_indptr[b] + j];
      if (id < 0 || id >= p->num_pages)
        return fail(PPA_ERR_TABLE, msg, msg_len, "kv_indices[%lld] (request %d) = %d outside [0, %d)",
                    static_cast<long long>(kv_indptr[b] + j), b, id, p->num_pages);
    }
    if (kv_last_page_len != nullptr) {
      const int64_t last = kv_last_page_len[b];
      const bool ok = have == 0 ? (kv_len == 0 && last == 0)
                                : (last >= 1 && last <= p->page_size && (have - 1) * p->page_size + last == kv_len);
      if (!ok)
        return fail(PPA_ERR_TABLE, msg, msg_len,
                    "request %d: %lld pages with last_page_len %lld do not give seq_len %lld", b,
                    static_cast<long long>(have), static_cast<long long>(last), static_cast<long long>(kv_len));
    }
  }
  return PPA_OK;
}

size_t ppa_merge_params_size(void) { return sizeof(ppa_merge_params); }

size_t ppa_append_params_size(void) { return sizeof(ppa_append_params); }

int32_t ppa_validate_append(const ppa_params* p, const ppa_append_params* a, char* msg, size_t msg_len) {
  if (msg != nullptr && msg_len > 0) msg[0] = '\0';
  if (p == nullptr || a == nullptr) return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "params is NULL");
  if (p->abi_version != PPA_ABI_VERSION || p->struct_size != sizeof(ppa_params) ||
      a->abi_version != PPA_ABI_VERSION || a->struct_size != sizeof(ppa_append_params))
    return fail(PPA_ERR_ABI, msg, msg_len, "abi_version / struct_size mismatch");
  if (p->kv_dtype != PPA_DTYPE_BF16 && p->kv_dtype != PPA_DTYPE_FP8_E4M3FN)
    return fail(PPA_ERR_DTYPE, msg, msg_len, "kv dtype %d: bf16 or fp8 e4m3fn", p->kv_dtype);
  if (p->fp8_compute != 0 && p->fp8_compute != 1)
    return fail(PPA_ERR_DTYPE, msg, msg_len, "fp8_compute %d: 0 or 1", p->fp8_compute);
  if (p->fp8_compute == 1 && (p->kv_dtype != PPA_DTYPE_FP8_E4M3FN || p->head_dim != 128))
    return fail(PPA_ERR_DTYPE, msg, msg_len, "fp8_compute needs an fp8 e4m3fn cache at head_dim 128");
  if (a->new_dtype != PPA_DTYPE_BF16)
    return fail(PPA_ERR_DTYPE, msg, msg_len, "new K/V dtype %d: only bf16", a->new_dtype);
  if (p->kv_layout != PPA_KV_LAYOUT_HND && p->kv_layout != PPA_KV_LAYOUT_NHD)
    return fail(PPA_ERR_LAYOUT, msg, msg_len, "kv_layout %d", p->kv_layout);
  if (p->kv_form != PPA_KV_SPLIT && p->kv_form != PPA_KV_COMBINED)
    return fail(PPA_ERR_LAYOUT, msg, msg_len, "kv_form %d", p->kv_form);
  if (p->kv_form == PPA_KV_COMBINED && p->kv_planes != 2)
    return fail(PPA_ERR_LAYOUT, msg, msg_len, "append needs separate K and V planes (kv_cache dim 1 is %d)",
                p->kv_planes);
  if (p->num_kv_heads <= 0) return fail(PPA_ERR_HEADS, msg, msg_len, "num_kv_heads %d", p->num_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PPA_ERR_HEAD_DIM, msg, msg_len, "head_dim %d", p->head_dim);
  if (p->page_size < 1 || p->page_size > 65536 || (p->page_size & (p->page_size - 1)) != 0)
    return fail(PPA_ERR_PAGE_SIZE, msg, msg_len, "page_size %d", p->page_size);
  if (a->num_new < 0 || p->num_pages < 0) return fail(PPA_ERR_SHAPE, msg, msg_len, "negative size");
  if (a->num_new == 0) return PPA_OK;
  if (p->num_pages < 1) return fail(PPA_ERR_SHAPE, msg, msg_len, "num_pages is 0");
  if (a->k_new == nullptr || a->v_new == nullptr || a->slot_mapping == nullptr)
    return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "k_new / v_new / slot_mapping");
  if (p->kv_form == PPA_KV_SPLIT ? (p->k_cache == nullptr || p->v_cache == nullptr) : p->kv_cache == nullptr)
    return fail(PPA_ERR_NULL_POINTER, msg, msg_len, "kv cache");
  const int kb = ppa::dtype_bytes(p->kv_dtype);
  for (int w = 0; w < 2; ++w) {
    PlaneStrides st = plane_strides(p, w);
    if (st.dim != 1)
      return fail(PPA_ERR_STRIDE, msg, msg_len, "%s cache head_dim stride must be 1", w ? "V" : "K");
    if (!row_stride_ok(st.page, p->num_pages, kb) || !row_stride_ok(st.head, p->num_kv_heads, kb) ||
        !row_stride_ok(st.tok, p->page_size, kb))
      return fail(PPA_ERR_STRIDE, msg, msg_len,
                  "%s cache page/head/token strides must be non-negative 16-byte multiples", w ? "V" : "K");
    const int64_t* ns = w ? a->v_new_strides : a->k_new_strides;
    if (ns[2] != 1 || !row_stride_ok(ns[0], a->num_new, 2) || !row_stride_ok(ns[1], p->num_kv_heads, 2))
      return fail(PPA_ERR_STRIDE, msg, msg_len, "%s_new strides: head_dim stride 1, others 16-byte multiples",
                  w ? "v" : "k");
  }
  if (p->kv_form == PPA_KV_COMBINED && !row_stride_ok(p->kv_cache_strides[1], 2, kb))
    return fail(PPA_ERR_STRIDE, msg, msg_len, "kv_cache plane stride must be a 16-byte multiple");
  if (!aligned16(a->k_new) || !aligned16(a->v_new) ||
      (p->kv_form == PPA_KV_SPLIT ? (!aligned16(p->k_cache) || !aligned16(p->v_cache)) : !aligned16(p->kv_cache)))
    return fail(PPA_ERR_ALIGNMENT, msg, msg_len, "k_new / v_new / kv cache");
  if ((reinterpret_cast<uintptr_t>(a->slot_mapping) & 7u) != 0)
    return fail(PPA_ERR_ALIGNMENT, msg, msg_len, "slot_mapping");
  return PPA_OK;
}

}  // extern "C"
