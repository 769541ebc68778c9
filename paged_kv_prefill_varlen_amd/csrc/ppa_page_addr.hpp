// Page-table address unit (device side).
//
// A request's logical KV token t lives in page block_tables[b][t >> log2(P)]
// (or kv_indices[kv_indptr[b] + (t >> log2(P))] for the flat form) at slot
// t & (P - 1); the page's first element is the pool base plus
// page id x page stride (FlashInfer API page, parameters kv_cache and
// block_tables; TensorRT-LLM attention-backend article, section "physical
// meaning of handle -> offset": tables hold ids, the kernel multiplies by the
// stride).  Because only strides differ between HND and NHD, and between a
// split and a combined cache, one formula serves all of them:
//
//   row(t, hk) = base + id * page_stride + hk * head_stride + slot * token_stride
//
// Ids are int32; the products are int64 so pools above 4 GiB work.  The
// column index is clamped to the table width and the id to [0, num_pages),
// and a table without columns is not read, so metadata that the host
// checker would reject can never send a read outside the pool.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ppa {

struct PagedPlane {
  const uint8_t* base;   // first byte of the plane (K or V)
  int64_t page_stride;   // elements
  int64_t head_stride;   // elements
  int64_t tok_stride;    // elements
};

struct PageTable {
  const int32_t* row;    // block_tables + b * row_stride, or kv_indices + kv_indptr[b]
  int32_t cols;          // table width (pages of the request for the flat form)
  int32_t num_pages;
  int32_t page_shift;    // log2(page_size)
};

__device__ __forceinline__ int page_id(const PageTable& pt, int token) {
  if (pt.cols <= 0) return 0;   // no pages: never read the table
  int col = token >> pt.page_shift;
  col = col < pt.cols - 1 ? col : pt.cols - 1;
  int id = pt.row[col];
  id = id < 0 ? 0 : id;
  id = id < pt.num_pages ? id : pt.num_pages - 1;
  return id;
}

// The same lookup for a key that is uniform across the wave: the table is
// read through the constant address space, so the load is a scalar one whose
// result does not wait behind the wave's outstanding vector loads.
__device__ __forceinline__ int page_id_uniform(const PageTable& pt, int token) {
  if (pt.cols <= 0) return 0;
  int col = token >> pt.page_shift;
  col = col < pt.cols - 1 ? col : pt.cols - 1;
  const __attribute__((address_space(4))) int32_t* row =
      (const __attribute__((address_space(4))) int32_t*)(pt.row);
  int id = row[col];
  id = id < 0 ? 0 : id;
  id = id < pt.num_pages ? id : pt.num_pages - 1;
  return id;
}

// Row of request b: block_tables (padded form) or kv_indices from kv_indptr[b]
// (flat form, indptr clamped to [0, indices_len]).
__device__ __forceinline__ void request_table(PageTable& pt, int b, const int32_t* block_tables,
                                              int64_t bt_row_stride, int32_t bt_cols, const int32_t* kv_indptr,
                                              const int32_t* kv_indices, int64_t indices_len) {
  if (kv_indptr != nullptr) {
    // scalar loads (constant address space): the kernel never writes the table
    typedef const __attribute__((address_space(4))) int32_t cint32;
    int64_t s0 = ((cint32*)(kv_indptr))[b], s1 = ((cint32*)(kv_indptr))[b + 1];
    s0 = s0 < 0 ? 0 : (s0 > indices_len ? indices_len : s0);
    s1 = s1 < s0 ? s0 : (s1 > indices_len ? indices_len : s1);
    pt.row = kv_indices + s0;
    const int64_t n = s1 - s0;
    pt.cols = static_cast<int32_t>(n < 0x7fffffff ? n : 0x7fffffff);
  } else {
    pt.row = block_tables + static_cast<int64_t>(b) * bt_row_stride;
    pt.cols = bt_cols;
  }
}

// Byte address of element `elem` of token `token` (page `id`) for kv head hk.
template <int ELEM_BYTES>
__device__ __forceinline__ const uint8_t* token_row(const PagedPlane& pl, int id, int page_mask,
                                                    int token, int hk, int elem) {
  const int64_t off = static_cast<int64_t>(id) * pl.page_stride +
                      static_cast<int64_t>(hk) * pl.head_stride +
                      static_cast<int64_t>(token & page_mask) * pl.tok_stride + elem;
  return pl.base + off * ELEM_BYTES;
}

}  // namespace ppa
