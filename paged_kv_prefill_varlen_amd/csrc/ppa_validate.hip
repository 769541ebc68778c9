// Device-side metadata check.
//
// The pages ask for a checked mode that turns bad metadata into an error
// instead of silent wrong output (TensorRT-LLM attention-backend article,
// the self-check step of its FlashInfer section, and the row-count check of
// its block-offset section).  The attention kernels clamp table columns and
// page ids so that bad metadata can never send a read outside the tensors;
// this pass is the loud counterpart for callers whose metadata lives on the
// device: it evaluates the rules of ppa_validate_metadata_host and, for the
// flat table, ppa_validate_page_table_csr_host on the device arrays and
// leaves the first violated rule, in those functions' order, in a device
// word.
//
// Rule keys (uint64, smaller = earlier in the host functions' order):
//   0                       cum_seq_lens_q[0] != 0
//   1                       cum_seq_lens_kv[0] != 0
//   2 + 8 b + r             request b, rule r:
//                             0 q_len < 0            4 kv_len > max_kv_len
//                             1 kv_len < 0           5 cum_seq_lens_kv step != seq_lens[b]
//                             2 q_len > kv_len       6 table narrower than the request's pages
//                             3 q_len > max_q_len    7 a page id outside [0, num_pages)
//   2 + 8 B                 cum_seq_lens_q[B] > num_tokens
//   flat table only, C = 3 + 8 B:
//   C                       kv_indptr[0] < 0
//   C + 1 + b               kv_indptr[b + 1] < kv_indptr[b]
//   C + 1 + B               kv_indptr[B] > kv_indices_len
//   C + 2 + B + 3 b + r     request b, rule r: 0 fewer pages than ceil(seq_lens / page_size),
//                           1 a page id outside [0, num_pages), 2 kv_last_page_len inconsistent
// The running-sum rule of cum_seq_lens_kv is checked as a per-request step
// (cum_seq_lens_kv[b + 1] - cum_seq_lens_kv[b] == seq_lens[b]); with the
// start at 0 (key 1) the first request that breaks either form is the same.
// A thread reads table entries only inside the request's own table row or
// index slice, after checking the bounds it needs; when those bounds fail,
// an earlier key already records the violation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ppa.h"

namespace ppa {
namespace {

struct MetaArgs {
  const int32_t* cu_q;
  const int32_t* cu_kv;        // may be NULL
  const int32_t* seq_lens;
  const int32_t* bt;           // padded table (NULL for the flat form)
  int64_t bt_stride;
  int32_t bt_cols;
  const int32_t* indptr;       // flat table (NULL for the padded form)
  const int32_t* indices;
  int64_t indices_len;
  const int32_t* last_len;     // may be NULL
  int32_t batch;
  int32_t num_tokens;
  int32_t max_q;
  int32_t max_kv;
  int32_t page_size;
  int32_t num_pages;
  unsigned long long* key;     // the caller's result word, as one 64-bit key
};

constexpr unsigned long long kNoViolation = ~0ull;

__device__ __forceinline__ void report(const MetaArgs& m, unsigned long long k) { atomicMin(m.key, k); }

__global__ __launch_bounds__(64) void meta_init(unsigned long long* key) {
  if (threadIdx.x == 0) *key = kNoViolation;
}

// blockIdx.x = request; blockIdx.y, threadIdx.x stride over its table entries
__global__ __launch_bounds__(256) void meta_check(MetaArgs m) {
  const int b = blockIdx.x;
  const int64_t B = m.batch;
  const int64_t C = 3 + 8 * B;
  const bool csr = m.indptr != nullptr;
  const int64_t q_len = static_cast<int64_t>(m.cu_q[b + 1]) - m.cu_q[b];
  const int64_t kv_len = m.seq_lens[b];
  const int64_t need = kv_len > 0 ? (kv_len + m.page_size - 1) / m.page_size : 0;
  const unsigned long long rk = 2 + 8 * static_cast<unsigned long long>(b);
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    if (b == 0) {
      if (m.cu_q[0] != 0) report(m, 0);
      if (m.cu_kv != nullptr && m.cu_kv[0] != 0) report(m, 1);
      if (m.cu_q[B] > m.num_tokens) report(m, 2 + 8 * B);
      if (csr && m.indptr[0] < 0) report(m, C);
      if (csr && m.indptr[B] > m.indices_len) report(m, C + 1 + B);
    }
    // the first failing rule of this request
    int r = -1;
    if (q_len < 0) r = 0;
    else if (kv_len < 0) r = 1;
    else if (q_len > kv_len) r = 2;
    else if (q_len > m.max_q) r = 3;
    else if (kv_len > m.max_kv) r = 4;
    else if (m.cu_kv != nullptr && static_cast<int64_t>(m.cu_kv[b + 1]) - m.cu_kv[b] != kv_len) r = 5;
    else if (!csr && need > m.bt_cols) r = 6;
    if (r >= 0) report(m, rk + r);
    if (csr) {
      const int64_t p0 = m.indptr[b], p1 = m.indptr[b + 1];
      if (p1 < p0) report(m, C + 1 + b);
      const int64_t have = p1 - p0;
      const unsigned long long ck = C + 2 + B + 3 * static_cast<unsigned long long>(b);
      if (have < need) {
        report(m, ck);
      } else if (m.last_len != nullptr) {
        const int64_t last = m.last_len[b];
        const bool ok = have == 0 ? (kv_len == 0 && last == 0)
                                  : (last >= 1 && last <= m.page_size && (have - 1) * m.page_size + last == kv_len);
        if (!ok) report(m, ck + 2);
      }
    }
  }
  // page ids the request reaches
  const int64_t stride = static_cast<int64_t>(gridDim.y) * blockDim.x;
  const int64_t first = static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x;
  if (!csr) {
    if (kv_len <= 0 || need > m.bt_cols) return;
    const int32_t* row = m.bt + b * m.bt_stride;
    for (int64_t j = first; j < need; j += stride) {
      const int32_t id = row[j];
      if (id < 0 || id >= m.num_pages) {
        report(m, rk + 7);
        return;
      }
    }
  } else {
    const int64_t p0 = m.indptr[b], p1 = m.indptr[b + 1];
    if (p0 < 0 || p1 < p0 || p1 > m.indices_len || p1 - p0 < need) return;
    const unsigned long long ck = C + 2 + B + 3 * static_cast<unsigned long long>(b);
    for (int64_t j = first; j < need; j += stride) {
      const int32_t id = m.indices[p0 + j];
      if (id < 0 || id >= m.num_pages) {
        report(m, ck + 1);
        return;
      }
    }
  }
}

// key -> (ppa_status, request index or -1), in place
__global__ __launch_bounds__(64) void meta_finish(unsigned long long* key, int64_t batch) {
  if (threadIdx.x != 0) return;
  const unsigned long long k = *key;
  const int64_t B = batch;
  const uint64_t C = 3 + 8 * B;
  int32_t code = PPA_OK, req = -1;
  if (k == kNoViolation) {
    code = PPA_OK;
  } else if (k < 2) {
    code = PPA_ERR_METADATA;
  } else if (k < 2 + 8 * static_cast<uint64_t>(B)) {
    const int r = static_cast<int>((k - 2) % 8);
    req = static_cast<int32_t>((k - 2) / 8);
    code = (r == 0 || r == 5) ? PPA_ERR_METADATA : (r >= 6 ? PPA_ERR_TABLE : PPA_ERR_LENGTHS);
  } else if (k == 2 + 8 * static_cast<uint64_t>(B)) {
    code = PPA_ERR_METADATA;
  } else {
    code = PPA_ERR_TABLE;
    if (k > C && k <= C + B) req = static_cast<int32_t>(k - C - 1);
    else if (k >= C + 2 + B) req = static_cast<int32_t>((k - C - 2 - B) / 3);
  }
  int32_t* out = reinterpret_cast<int32_t*>(key);
  out[0] = code;
  out[1] = req;
}

}  // namespace
}  // namespace ppa

using namespace ppa;

extern "C" int32_t ppa_validate_metadata_device(const ppa_params* p, int32_t* result, void* stream) {
  char msg[8];
  const int32_t st = ppa_validate_shapes(p, msg, sizeof msg);
  if (st != PPA_OK) return st;
  if (result == nullptr) return PPA_ERR_NULL_POINTER;
  if ((reinterpret_cast<uintptr_t>(result) & 7u) != 0) return PPA_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long* key = reinterpret_cast<unsigned long long*>(result);
  hipLaunchKernelGGL(meta_init, dim3(1), dim3(64), 0, s, key);
  if (p->batch_size > 0) {
    MetaArgs m{};
    m.cu_q = p->cum_seq_lens_q;
    m.cu_kv = p->cum_seq_lens_kv;
    m.seq_lens = p->seq_lens;
    if (p->page_table_form == PPA_PAGE_TABLE_CSR) {
      m.indptr = p->kv_indptr;
      m.indices = p->kv_indices;
      m.indices_len = p->kv_indices_len;
      m.last_len = p->kv_last_page_len;
    } else {
      m.bt = p->block_tables;
      m.bt_stride = p->batch_size > 1 ? p->block_tables_row_stride : 0;
      m.bt_cols = p->block_tables_cols;
    }
    m.batch = p->batch_size;
    m.num_tokens = p->num_tokens;
    m.max_q = p->max_q_len;
    m.max_kv = p->max_kv_len;
    m.page_size = p->page_size;
    m.num_pages = p->num_pages;
    m.key = key;
    hipLaunchKernelGGL(meta_check, dim3(static_cast<unsigned>(p->batch_size), 4), dim3(256), 0, s, m);
  }
  hipLaunchKernelGGL(meta_finish, dim3(1), dim3(64), 0, s, key, static_cast<int64_t>(p->batch_size));
  return hipGetLastError() == hipSuccess ? PPA_OK : PPA_ERR_HIP;
}
