// Host checkers under AddressSanitizer: every metadata array is a heap
// allocation of exactly the length the C ABI documents (batch_size + 1 for
// the cumulative offsets and kv_indptr, batch_size for seq_lens and
// kv_last_page_len, batch_size rows of the block table), so a read past
// what the header promises is reported as a heap-buffer-overflow.  Built and
// run by tests/test_abi_host.py with g++ on the CPU; exit status 0 means
// every case returned the expected status and ASan reported nothing.
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <vector>

#include "ppa.h"

namespace {

int failures = 0;

void expect(int32_t got, int32_t want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

// A description of `batch` requests with q_lens / prefixes, page size 4,
// 2 kv heads, head_dim 64, HND split bf16; pages are numbered in order.
struct Case {
  std::vector<int32_t> cu_q, cu_kv, seq_lens, table, indptr, indices, last;
  int32_t cols = 1, pages = 0, max_q = 0, max_kv = 0;
  ppa_params p{};
  std::vector<uint16_t> q, k, v, out;
};

Case make(const std::vector<int>& q_lens, const std::vector<int>& prefix) {
  Case c;
  const int B = static_cast<int>(q_lens.size()), P = 4;
  c.cu_q.assign(1, 0);
  c.cu_kv.assign(1, 0);
  for (int b = 0; b < B; ++b) {
    const int kv = q_lens[b] + prefix[b];
    c.seq_lens.push_back(kv);
    c.cu_q.push_back(c.cu_q.back() + q_lens[b]);
    c.cu_kv.push_back(c.cu_kv.back() + kv);
    c.cols = std::max(c.cols, (kv + P - 1) / P);
    c.max_q = std::max(c.max_q, q_lens[b]);
    c.max_kv = std::max(c.max_kv, kv);
  }
  c.indptr.assign(1, 0);
  for (int b = 0; b < B; ++b) {
    const int n = (c.seq_lens[b] + P - 1) / P;
    for (int j = 0; j < c.cols; ++j) c.table.push_back(j < n ? c.pages + j : 0);
    for (int j = 0; j < n; ++j) c.indices.push_back(c.pages + j);
    c.indptr.push_back(static_cast<int32_t>(c.indices.size()));
    c.last.push_back(n == 0 ? 0 : c.seq_lens[b] - (n - 1) * P);
    c.pages += n;
  }
  c.pages = std::max(c.pages, 1);
  if (c.indices.empty()) c.indices.push_back(0);
  const int T = std::max(c.cu_q.back(), 1), D = 64, H = 2;
  c.q.assign(static_cast<size_t>(T) * H * D, 0);
  c.out = c.q;
  c.k.assign(static_cast<size_t>(c.pages) * H * P * D, 0);
  c.v = c.k;
  ppa_params& p = c.p;
  p.abi_version = PPA_ABI_VERSION;
  p.struct_size = sizeof(ppa_params);
  p.query = c.q.data();
  p.query_dtype = PPA_DTYPE_BF16;
  p.num_tokens = T;
  p.num_qo_heads = H;
  p.head_dim = D;
  p.query_strides[0] = H * D;
  p.query_strides[1] = D;
  p.query_strides[2] = 1;
  p.kv_form = PPA_KV_SPLIT;
  p.kv_layout = PPA_KV_LAYOUT_HND;
  p.kv_dtype = PPA_DTYPE_BF16;
  p.num_pages = c.pages;
  p.num_kv_heads = H;
  p.page_size = P;
  p.k_cache = c.k.data();
  p.v_cache = c.v.data();
  const int64_t st[4] = {H * P * D, P * D, D, 1};
  for (int i = 0; i < 4; ++i) p.k_cache_strides[i] = p.v_cache_strides[i] = st[i];
  p.block_tables_cols = c.cols;
  p.block_tables_row_stride = c.cols;
  p.batch_size = B;
  p.max_q_len = c.max_q;
  p.max_kv_len = c.max_kv;
  p.bmm1_scale = 0.125f;
  p.bmm2_scale = 1.f;
  p.window_left = -1;
  p.out = c.out.data();
  p.out_dtype = PPA_DTYPE_BF16;
  for (int i = 0; i < 3; ++i) p.out_strides[i] = p.query_strides[i];
  return c;
}

// Exact-length heap copies, so ASan sees each array's documented extent.
template <class T>
T* exact(const std::vector<T>& v, size_t n) {
  T* x = static_cast<T*>(std::malloc(n * sizeof(T) + (n == 0)));
  for (size_t i = 0; i < n; ++i) x[i] = v[i];
  return x;
}

void run(const std::vector<int>& q_lens, const std::vector<int>& prefix, const char* what) {
  Case c = make(q_lens, prefix);
  const size_t B = q_lens.size();
  int32_t* cu_q = exact(c.cu_q, B + 1);
  int32_t* cu_kv = exact(c.cu_kv, B + 1);
  int32_t* sl = exact(c.seq_lens, B);
  int32_t* bt = exact(c.table, B * static_cast<size_t>(c.cols));
  int32_t* ip = exact(c.indptr, B + 1);
  int32_t* ix = exact(c.indices, c.indices.size());
  int32_t* last = exact(c.last, B);
  char msg[256] = {0};
  // the shape check only tests these pointers for NULL; it reads nothing
  c.p.block_tables = bt;
  c.p.seq_lens = sl;
  c.p.cum_seq_lens_q = cu_q;
  c.p.cum_seq_lens_kv = cu_kv;
  expect(ppa_validate_shapes(&c.p, msg, sizeof msg), PPA_OK, what);
  expect(ppa_validate_metadata_host(&c.p, cu_q, cu_kv, sl, bt, msg, sizeof msg), PPA_OK, what);
  expect(ppa_validate_metadata_host(&c.p, cu_q, nullptr, sl, bt, msg, sizeof msg), PPA_OK, what);
  ppa_params csr = c.p;
  csr.page_table_form = PPA_PAGE_TABLE_CSR;
  csr.block_tables = nullptr;
  csr.kv_indptr = ip;
  csr.kv_indices = ix;
  csr.kv_indices_len = static_cast<int64_t>(c.indices.size());
  expect(ppa_validate_metadata_host(&csr, cu_q, cu_kv, sl, nullptr, msg, sizeof msg), PPA_OK, what);
  expect(ppa_validate_page_table_csr_host(&csr, sl, ip, ix, last, msg, sizeof msg), PPA_OK, what);
  expect(ppa_validate_page_table_csr_host(&csr, sl, ip, ix, nullptr, msg, sizeof msg), PPA_OK, what);
  // a bad last entry is still found without reading past the arrays
  if (B > 0) {
    sl[B - 1] += 1;
    const int32_t st = ppa_validate_metadata_host(&c.p, cu_q, cu_kv, sl, bt, msg, sizeof msg);
    if (st == PPA_OK) {
      std::printf("FAIL %s: a seq_lens / cum_seq_lens_kv mismatch passed\n", what);
      ++failures;
    }
    sl[B - 1] -= 1;
  }
  for (int32_t* x : {cu_q, cu_kv, sl, bt, ip, ix, last}) std::free(x);
}

}  // namespace

int main() {
  run({5, 0, 9}, {3, 4, 0}, "three requests, one empty");
  run({1}, {0}, "one token");
  run({}, {}, "empty batch");
  run({7, 2, 3, 1}, {9, 0, 4, 12}, "four requests");
  std::printf("%s\n", failures == 0 ? "ok" : "failed");
  return failures == 0 ? 0 : 1;
}
