// Batched causal prefill attention over a paged KV cache, for gfx950 (CDNA4).
//
// Operation (FlashInfer API page for trtllm_batch_context_with_kv_cache,
// section "Parameters"): for request b, the q_len new query rows sit at the
// end of a kv_len-token sequence (prefix = kv_len - q_len, the chunked-context
// figure of the TensorRT-LLM attention-backend article); row i sees key j
// when j <= prefix + i and, with window_left >= 0, j >= prefix + i -
// window_left.  out = bmm2_scale * softmax(bmm1_scale * q k^T) v, where a
// per-head sink adds e^{sink} to the softmax denominator only.
//
// Work decomposition
//   One workgroup = 4 waves = 256 "rows"; a row is one (token, q head) pair of
//   one request and one kv head.  The GW = min(G, 16) query heads of a GQA
//   group that share the kv head are interleaved (row = token * GW + head), so
//   a K/V tile staged once in LDS serves every head of the group and the
//   causal boundary of a 32-row MFMA tile spans only 32 / GW tokens.
//   Each wave owns 64 rows = two 32-column MFMA tiles.
//   The grid is 1-D and ordered heaviest-first: blockIdx / R picks the query
//   tile from the last (longest causal span) to the first, blockIdx % R picks
//   (request, kv head, head group).  With R a multiple of 8, every tile of one
//   (request, kv head) lands on the same XCD (blocks go round-robin over the
//   8 XCDs), so its K/V stays in one L2.
//
// Per 64-key tile
//   1. page ids -> K rows (natural layout) and V rows (transposed in
//      registers) into double-buffered LDS; fp8 codes are widened to bf16 on
//      the way (exact: every e4m3fn value is a bf16 value);
//   2. S^T = K Q^T on v_mfma_f32_32x32x16_bf16: keys along M, rows along N,
//      so a lane holds 32 keys of one row and its partner lane (lane ^ 32) the
//      other 32: row max / sum need one cross-lane step;
//   3. mask (boundary tiles only), online softmax in the exp2 domain with
//      the running maximum moved only when a row's maximum grows by more than
//      2^8 (exact: softmax does not depend on the subtracted constant);
//   4. O^T += V^T P^T on the same MFMA; P goes from the S accumulator straight
//      into the B operand, because the K rows are fed to the first MFMA in an
//      order (bits 2 and 3 of the row index swapped) that leaves each lane half
//      holding 8 consecutive keys.
//   Tiles wholly outside a wave's causal/window band are skipped; only tiles
//   cut by the band are masked.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "ppa.h"
#include "ppa_internal.h"
#include "ppa_page_addr.hpp"

namespace ppa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kBK = 64;            // keys per tile
constexpr int kLoadWaves = 4;      // waves of threads that stage one operand (K or V) of a tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;   // log2 units
constexpr float kNegInf = -__builtin_inff();
constexpr float kMinScale = 1.17549435e-38f;  // FLT_MIN

struct AttnArgs {
  const uint16_t* q;
  int64_t q_tok, q_head;
  uint16_t* out;
  int64_t o_tok, o_head;
  PagedPlane k, v;
  const int32_t* block_tables;
  int64_t bt_row_stride;
  int32_t bt_cols;
  int32_t num_pages;
  int32_t page_shift;
  const int32_t* seq_lens;
  const int32_t* cu_q;
  int32_t num_tokens;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t group;       // q heads per kv head
  int32_t gw;          // q heads per workgroup
  int32_t n_hg;        // head groups per kv head
  int32_t tq;          // tokens per workgroup
  int32_t n_qt;        // query tiles per request (upper bound)
  int32_t window_left;
  float bmm1, bmm2;
  const float* bmm1_ptr;
  const float* bmm2_ptr;
  const float* sinks;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);   // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, r);
}

// 4 fp8 e4m3fn codes -> 4 bf16 (two packed dwords).  Exact.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return u32x2{pack_bf16(lo[0], lo[1]), pack_bf16(hi[0], hi[1])};
}

// Row index fed to the A operand of the S^T MFMA: bits 2 and 3 swapped.  With
// this order, accumulator element v of lane half h holds key
// 16 * (v / 8) + 8 * h + v % 8 of its 32-key block.
__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Tile geometry.  K and V of a 64-key tile are each staged by 4 loader waves;
// loader wave lw owns the 16 consecutive keys [16 lw, 16 lw + 16) of the tile,
// so with pages of >= 16 tokens its keys lie in one page and the page id and
// base address are wave-uniform.  K goes to LDS in natural [key][dim] layout
// with 16-byte loads; V goes as 4 consecutive keys x V_DPT dims per lane,
// transposed in registers to [dim][key].  Both need RAW dwords per lane.
template <int D, bool FP8>
struct Tile {
  static constexpr int EB = FP8 ? 1 : 2;        // bytes per cache element
  static constexpr int K_CHUNK = 16 / EB;       // elements per 16-byte load
  static constexpr int K_TPR = D / K_CHUNK;     // lanes per key row
  static constexpr int K_RPI = 64 / K_TPR;      // key rows per wave instruction
  static constexpr int K_PASSES = 16 / K_RPI;   // instructions per loader wave
  static constexpr int V_DPT = D / 16;          // head-dim values per lane
  static constexpr int V_DW = V_DPT * EB / 4;   // raw dwords per key
  static constexpr int RAW = D * EB / 16;       // raw dwords per lane and operand
  // LDS row strides in bf16 elements.  K rows are padded by 16 bytes; V rows
  // by 16 bytes plus an XOR swizzle of their 16-byte key chunks by
  // (dim >> 4) & 7, which together keep the MFMA operand reads and the
  // transposed V writes free of bank conflicts.
  static constexpr int KS = D + 8;
  static constexpr int VS = kBK + 8;
  static constexpr int K_ELEMS = kBK * KS;
  static constexpr int V_ELEMS = D * VS;
  static_assert(K_PASSES * K_RPI == 16, "K tile mapping");
  static_assert(K_PASSES * 4 == RAW && 4 * V_DW == RAW, "K and V prefetch sizes");
  static_assert(V_DW >= 1, "V load");
};

__device__ __forceinline__ int vt_offset(int d, int key, int vs) {
  // element offset of V^T[d][key] in the swizzled layout
  const int chunk = (key >> 3) ^ ((d >> 4) & 7);
  return d * vs + chunk * 8 + (key & 7);
}

// ---- staging: global -> registers ---------------------------------------------
// UPAGE: the loader wave's 16 keys share one page (page_size >= 16 and the tile
// is not the last one of the request).  Otherwise every lane resolves its own
// keys, clamped to the sequence, and zero-fills keys past kv_len.
template <int D, bool FP8, bool UPAGE>
__device__ __forceinline__ void fetch_k(uint32_t* raw, const PagedPlane& pl, const PageTable& pt,
                                        int hk, int kb, int kv_len, int page_mask, int lane,
                                        bool tail) {
  using T = Tile<D, FP8>;
  const int kchunk = lane % T::K_TPR;
  const int r0 = lane / T::K_TPR;
  if (UPAGE && !tail) {
    const int id = uniform(page_id(pt, kb));
    const uint8_t* base = pl.base + (static_cast<int64_t>(id) * pl.page_stride +
                                     static_cast<int64_t>(hk) * pl.head_stride) * T::EB;
    const int slot0 = kb & page_mask;
    for (int p = 0; p < T::K_PASSES; ++p) {
      const uint32_t off = static_cast<uint32_t>(
          ((slot0 + p * T::K_RPI + r0) * static_cast<int>(pl.tok_stride) + kchunk * T::K_CHUNK) * T::EB);
      const u32x4 x = *reinterpret_cast<const u32x4*>(base + off);
      for (int i = 0; i < 4; ++i) raw[4 * p + i] = x[i];
    }
  } else {
    for (int p = 0; p < T::K_PASSES; ++p) {
      const int key = kb + p * T::K_RPI + r0;
      const bool ok = key < kv_len;
      const int kc = ok ? key : kv_len - 1;
      const int id = page_id(pt, kc);
      u32x4 x = *reinterpret_cast<const u32x4*>(token_row<T::EB>(pl, id, page_mask, kc, hk, kchunk * T::K_CHUNK));
      for (int i = 0; i < 4; ++i) raw[4 * p + i] = ok ? x[i] : 0u;
    }
  }
}

template <int D, bool FP8, bool UPAGE>
__device__ __forceinline__ void fetch_v(uint32_t* raw, const PagedPlane& pl, const PageTable& pt,
                                        int hk, int kb, int kv_len, int page_mask, int lane,
                                        bool tail) {
  using T = Tile<D, FP8>;
  const int kgl = lane >> 4;   // 4 keys: kb + 4 kgl .. + 3
  const int dg = lane & 15;
  auto load = [&](const uint8_t* src, uint32_t* dst, bool ok) {
    if constexpr (T::V_DW == 4) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(src);
      for (int i = 0; i < 4; ++i) dst[i] = ok ? x[i] : 0u;
    } else if constexpr (T::V_DW == 2) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(src);
      dst[0] = ok ? x[0] : 0u;
      dst[1] = ok ? x[1] : 0u;
    } else {
      const uint32_t x = *reinterpret_cast<const uint32_t*>(src);
      dst[0] = ok ? x : 0u;
    }
  };
  if (UPAGE && !tail) {
    const int id = uniform(page_id(pt, kb));
    const uint8_t* base = pl.base + (static_cast<int64_t>(id) * pl.page_stride +
                                     static_cast<int64_t>(hk) * pl.head_stride) * T::EB;
    const int slot0 = (kb & page_mask) + 4 * kgl;
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = static_cast<uint32_t>(
          ((slot0 + r) * static_cast<int>(pl.tok_stride) + dg * T::V_DPT) * T::EB);
      load(base + off, raw + T::V_DW * r, true);
    }
  } else {
    for (int r = 0; r < 4; ++r) {
      const int key = kb + 4 * kgl + r;
      const bool ok = key < kv_len;
      const int kc = ok ? key : kv_len - 1;
      const int id = page_id(pt, kc);
      load(token_row<T::EB>(pl, id, page_mask, kc, hk, dg * T::V_DPT), raw + T::V_DW * r, ok);
    }
  }
}

// ---- staging: registers -> LDS ---------------------------------------------------
template <int D, bool FP8>
__device__ __forceinline__ void store_k(const uint32_t* raw, __bf16* klds, int lw, int lane) {
  using T = Tile<D, FP8>;
  const int kchunk = lane % T::K_TPR;
  const int r0 = lane / T::K_TPR;
  for (int p = 0; p < T::K_PASSES; ++p) {
    __bf16* dst = klds + (16 * lw + p * T::K_RPI + r0) * T::KS + kchunk * T::K_CHUNK;
    if constexpr (!FP8) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{raw[4 * p], raw[4 * p + 1], raw[4 * p + 2], raw[4 * p + 3]};
    } else {
      const u32x2 a0 = fp8x4_to_bf16x4(raw[4 * p]);
      const u32x2 a1 = fp8x4_to_bf16x4(raw[4 * p + 1]);
      const u32x2 a2 = fp8x4_to_bf16x4(raw[4 * p + 2]);
      const u32x2 a3 = fp8x4_to_bf16x4(raw[4 * p + 3]);
      reinterpret_cast<u32x4*>(dst)[0] = u32x4{a0[0], a0[1], a1[0], a1[1]};
      reinterpret_cast<u32x4*>(dst)[1] = u32x4{a2[0], a2[1], a3[0], a3[1]};
    }
  }
}

template <int D, bool FP8>
__device__ __forceinline__ void store_v(const uint32_t* raw, __bf16* vlds, int lw, int lane) {
  using T = Tile<D, FP8>;
  constexpr int PAIRS = T::V_DPT / 2;   // bf16 pairs per key
  uint32_t w[4][PAIRS];
  for (int r = 0; r < 4; ++r) {
    if constexpr (!FP8) {
      for (int i = 0; i < PAIRS; ++i) w[r][i] = raw[T::V_DW * r + i];
    } else {
      for (int i = 0; i < T::V_DW; ++i) {
        const u32x2 x = fp8x4_to_bf16x4(raw[T::V_DW * r + i]);
        w[r][2 * i] = x[0];
        w[r][2 * i + 1] = x[1];
      }
    }
  }
  const int key0 = 16 * lw + 4 * (lane >> 4);
  const int dg = lane & 15;
  for (int i = 0; i < PAIRS; ++i) {
    // head-dim 2i: low halves of the 4 keys; head-dim 2i+1: high halves
    const uint32_t lo01 = (w[0][i] & 0xffffu) | (w[1][i] << 16);
    const uint32_t lo23 = (w[2][i] & 0xffffu) | (w[3][i] << 16);
    const uint32_t hi01 = (w[0][i] >> 16) | (w[1][i] & 0xffff0000u);
    const uint32_t hi23 = (w[2][i] >> 16) | (w[3][i] & 0xffff0000u);
    const int d = dg * T::V_DPT + 2 * i;
    *reinterpret_cast<u32x2*>(vlds + vt_offset(d, key0, T::VS)) = u32x2{lo01, lo23};
    *reinterpret_cast<u32x2*>(vlds + vt_offset(d + 1, key0, T::VS)) = u32x2{hi01, hi23};
  }
}

// NT: 32-row MFMA column tiles per wave; NW: waves per workgroup.  Every
// configuration has 256 rows per workgroup.  With NW = 8 (two waves per
// SIMD), waves 0-3 stage K and waves 4-7 stage V; with NW = 4 every wave
// stages both.
template <int D, bool FP8, int NT, int NW, bool UPAGE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void paged_prefill_kernel(AttnArgs a) {
  using T = Tile<D, FP8>;
  constexpr int KSTEPS = D / 16;   // MFMA K-steps over head_dim
  constexpr int MD = D / 32;       // 32-wide head_dim tiles of O^T
  constexpr bool SPLIT_STAGING = NW == 8;
  static_assert(NT * NW * 32 == 256, "256 rows per workgroup");
  __shared__ __attribute__((aligned(16))) __bf16 klds[2][T::K_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 vlds[2][T::V_ELEMS];

  // ---- which work item --------------------------------------------------
  const int R = a.batch * a.num_kv_heads * a.n_hg;
  const int L = blockIdx.x;
  const int qt = a.n_qt - 1 - L / R;
  const int rest = L % R;
  const int b = rest / (a.num_kv_heads * a.n_hg);
  const int hk = (rest / a.n_hg) % a.num_kv_heads;
  const int hg = rest % a.n_hg;

  int q1 = a.cu_q[b + 1];
  int q0 = a.cu_q[b];
  q1 = q1 < a.num_tokens ? q1 : a.num_tokens;
  q0 = q0 < 0 ? 0 : (q0 < q1 ? q0 : q1);
  const int q_len = q1 - q0;
  int kv_len = a.seq_lens[b];
  kv_len = kv_len < 0 ? 0 : kv_len;
  const int t0 = qt * a.tq;
  if (t0 >= q_len) return;
  const int ntok = q_len - t0 < a.tq ? q_len - t0 : a.tq;
  const int prefix = kv_len - q_len;
  const int h0 = hk * a.group + hg * a.gw;
  const int nheads = a.group - hg * a.gw < a.gw ? a.group - hg * a.gw : a.gw;
  const int W = a.window_left;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;

  // logits in log2 units: s * c with c = |bmm1| log2(e); the sign of bmm1 is
  // folded into Q (exact for bf16).  c is kept >= FLT_MIN so that a masked
  // logit (-inf) times c stays -inf; with bmm1 = 0 every valid weight is then
  // exp2(0) = 1 exactly, as it should be.
  float c = (a.bmm1_ptr ? *a.bmm1_ptr : a.bmm1) * kLog2e;
  const float bmm2 = a.bmm2_ptr ? *a.bmm2_ptr : a.bmm2;
  const bool negate_q = c < 0.f;
  c = negate_q ? -c : c;
  c = c > kMinScale ? c : kMinScale;

  // ---- the wave's rows ----------------------------------------------------
  constexpr int WROWS = 32 * NT;
  int tok[NT], hd[NT], pos[NT];
  bool rvalid[NT];
  for (int nt = 0; nt < NT; ++nt) {
    const int r = wave * WROWS + nt * 32 + col;
    tok[nt] = r / a.gw;
    hd[nt] = r % a.gw;
    rvalid[nt] = tok[nt] < ntok && hd[nt] < nheads;
    pos[nt] = prefix + t0 + tok[nt];
  }
  const int wtok_first = (wave * WROWS) / a.gw;
  int wtok_last = (wave * WROWS + WROWS - 1) / a.gw;
  wtok_last = wtok_last < ntok - 1 ? wtok_last : ntok - 1;
  const bool wave_active = wtok_first < ntok;
  const int wpos_first = prefix + t0 + wtok_first;
  const int wpos_last = prefix + t0 + wtok_last;
  const int wkey_hi = wpos_last < kv_len - 1 ? wpos_last : kv_len - 1;
  const int wkey_lo = W >= 0 ? (wpos_first - W > 0 ? wpos_first - W : 0) : 0;

  // ---- Q into registers (B operand of S^T = K Q^T) ------------------------
  bf16x8 qf[NT][KSTEPS];
  for (int nt = 0; nt < NT; ++nt) {
    const uint16_t* qrow = a.q + static_cast<int64_t>(q0 + t0 + tok[nt]) * a.q_tok +
                           static_cast<int64_t>(h0 + hd[nt]) * a.q_head;
    for (int s = 0; s < KSTEPS; ++s) {
      u32x4 x = u32x4{0, 0, 0, 0};
      if (rvalid[nt]) x = *reinterpret_cast<const u32x4*>(qrow + s * 16 + half * 8);
      if (negate_q) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qf[nt][s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[NT][MD];
  for (int nt = 0; nt < NT; ++nt)
    for (int md = 0; md < MD; ++md) oacc[nt][md] = f32x16{};
  float m_run[NT], l_part[NT];
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = kNegInf;
    l_part[nt] = 0.f;
  }

  // ---- K/V tile range of the workgroup -------------------------------------
  const int pos_first = prefix + t0;
  const int pos_last = prefix + t0 + ntok - 1;
  const int key_hi = pos_last < kv_len - 1 ? pos_last : kv_len - 1;
  const int key_lo = W >= 0 ? (pos_first - W > 0 ? pos_first - W : 0) : 0;
  const int tile_lo = key_lo / kBK;
  const int tile_hi = key_hi >= 0 ? key_hi / kBK : -1;

  PageTable pt;
  pt.row = a.block_tables + static_cast<int64_t>(b) * a.bt_row_stride;
  pt.cols = a.bt_cols;
  pt.num_pages = a.num_pages;
  pt.page_shift = a.page_shift;
  const int page_mask = (1 << a.page_shift) - 1;

  // staging roles
  const int lw = wave & (kLoadWaves - 1);
  const bool stage_k = !SPLIT_STAGING || wave < kLoadWaves;
  const bool stage_v = !SPLIT_STAGING || wave >= kLoadWaves;
  constexpr int NRAW = SPLIT_STAGING ? 1 : 2;
  uint32_t raw[NRAW][T::RAW];

  auto fetch = [&](int k0) {
    const bool tail = k0 + kBK > kv_len;
    const int kb = k0 + 16 * lw;
    if (stage_k) fetch_k<D, FP8, UPAGE>(raw[0], a.k, pt, hk, kb, kv_len, page_mask, lane, tail);
    if (stage_v) fetch_v<D, FP8, UPAGE>(raw[NRAW - 1], a.v, pt, hk, kb, kv_len, page_mask, lane, tail);
  };
  auto store = [&](int buf) {
    if (stage_k) store_k<D, FP8>(raw[0], klds[buf], lw, lane);
    if (stage_v) store_v<D, FP8>(raw[NRAW - 1], vlds[buf], lw, lane);
  };

  if (tile_lo <= tile_hi) {
    fetch(tile_lo * kBK);
    store(0);
  }
  __syncthreads();

  const int krow_lane = swap_bits23(col);
  const int vrow_base = col * T::VS + ((half ^ (col >> 4)) & 1) * 8;

  for (int tile = tile_lo; tile <= tile_hi; ++tile) {
    const int buf = (tile - tile_lo) & 1;
    const int k0 = tile * kBK;
    const bool more = tile + 1 <= tile_hi;
    if (more) fetch(k0 + kBK);

    const bool wave_tile = wave_active && k0 <= wkey_hi && k0 + kBK - 1 >= wkey_lo;
    if (wave_tile) {
      // S^T = K Q^T over head_dim: all K fragments of the tile first
      const __bf16* kbuf = klds[buf];
      bf16x8 kf[2][KSTEPS];
      for (int s = 0; s < KSTEPS; ++s)
        for (int mt = 0; mt < 2; ++mt)
          kf[mt][s] = *reinterpret_cast<const bf16x8*>(kbuf + (mt * 32 + krow_lane) * T::KS + s * 16 + half * 8);
      f32x16 sacc[2][NT];
      for (int mt = 0; mt < 2; ++mt)
        for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = f32x16{};
      for (int s = 0; s < KSTEPS; ++s)
        for (int mt = 0; mt < 2; ++mt)
          for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = mfma32(kf[mt][s], qf[nt][s], sacc[mt][nt]);

      // mask only tiles cut by the causal / window / length bounds
      const bool need_mask = (k0 + kBK - 1 > wpos_first) || (W >= 0 && k0 < wpos_last - W) ||
                             (k0 + kBK > kv_len);
      float mx[NT];
      for (int nt = 0; nt < NT; ++nt) {
        float m = kNegInf;
        if (need_mask) {
          const int base = k0 + 8 * half;
          const int hi = (pos[nt] < kv_len - 1 ? pos[nt] : kv_len - 1) - base;
          const int lo = (W >= 0 ? pos[nt] - W : -0x40000000) - base;
          for (int mt = 0; mt < 2; ++mt)
            for (int v = 0; v < 16; ++v) {
              const int off = mt * 32 + 16 * (v >> 3) + (v & 7);
              const bool ok = off <= hi && off >= lo;
              sacc[mt][nt][v] = ok ? sacc[mt][nt][v] : kNegInf;
            }
        }
        for (int mt = 0; mt < 2; ++mt)
          for (int v = 0; v < 16; ++v) m = fmaxf(m, sacc[mt][nt][v]);
        mx[nt] = fmaxf(m, __shfl_xor(m, 32));
      }

      // lazy rescale of the running maximum (log2 domain)
      bool need[NT];
      float mtile[NT];
      bool any = false;
      for (int nt = 0; nt < NT; ++nt) {
        mtile[nt] = mx[nt] * c;   // -inf stays -inf (c > 0)
        need[nt] = mtile[nt] > m_run[nt] + kRescaleThreshold;
        any = any || need[nt];
      }
      if (__ballot(any) != 0ull) {
        for (int nt = 0; nt < NT; ++nt) {
          const float m_new = need[nt] ? mtile[nt] : m_run[nt];
          const float alpha = need[nt] ? __builtin_amdgcn_exp2f(m_run[nt] - m_new) : 1.f;
          m_run[nt] = m_new;
          l_part[nt] *= alpha;
          for (int md = 0; md < MD; ++md) oacc[nt][md] *= alpha;
        }
      }

      // P = exp2(c s - m) (masked logits give exp2(-inf) = 0), row partial
      // sums, bf16 B operands of O^T += V^T P^T
      bf16x8 pb[NT][4];
      for (int nt = 0; nt < NT; ++nt) {
        const float mb = m_run[nt] == kNegInf ? 0.f : m_run[nt];
        float sum = 0.f;
        for (int mt = 0; mt < 2; ++mt) {
          float p[16];
          for (int v = 0; v < 16; ++v) {
            p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][nt][v], c, -mb));
            sum += p[v];
          }
          for (int sh = 0; sh < 2; ++sh) {
            u32x4 w;
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16(p[8 * sh + 2 * e], p[8 * sh + 2 * e + 1]);
            pb[nt][2 * mt + sh] = __builtin_bit_cast(bf16x8, w);
          }
        }
        l_part[nt] += sum;
      }

      // O^T += V^T P^T: all V fragments of the tile first
      // lane (col, half) reads dims md*32 + col, keys 16 ks + 8 half .. + 7; in
      // the swizzled layout that key chunk is 2 (ks ^ md) + (half ^ (col >> 4))
      const __bf16* vbuf = vlds[buf] + vrow_base;
      bf16x8 vf[MD][4];
      for (int ks = 0; ks < 4; ++ks)
        for (int md = 0; md < MD; ++md)
          vf[md][ks] = *reinterpret_cast<const bf16x8*>(vbuf + md * 32 * T::VS + ((ks ^ md) & 3) * 16);
      for (int ks = 0; ks < 4; ++ks)
        for (int md = 0; md < MD; ++md)
          for (int nt = 0; nt < NT; ++nt) oacc[nt][md] = mfma32(vf[md][ks], pb[nt][ks], oacc[nt][md]);
    }

    if (more) store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  if (!wave_active) return;
  for (int nt = 0; nt < NT; ++nt) {
    float l = l_part[nt] + __shfl_xor(l_part[nt], 32);
    if (!rvalid[nt]) continue;
    const int h = h0 + hd[nt];
    const float mb = m_run[nt] == kNegInf ? 0.f : m_run[nt];
    if (a.sinks) l += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - mb);
    const float inv = bmm2 / l;
    uint16_t* orow = a.out + static_cast<int64_t>(q0 + t0 + tok[nt]) * a.o_tok +
                     static_cast<int64_t>(h) * a.o_head;
    for (int md = 0; md < MD; ++md) {
      for (int g = 0; g < 4; ++g) {
        const int d = md * 32 + 8 * g + 4 * half;
        const u32x2 w = u32x2{pack_bf16(oacc[nt][md][4 * g] * inv, oacc[nt][md][4 * g + 1] * inv),
                              pack_bf16(oacc[nt][md][4 * g + 2] * inv, oacc[nt][md][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    }
  }
}

// ---- address-unit check: paged K or V -> contiguous [tokens, H_kv, D] ------
struct GatherArgs {
  PagedPlane plane;
  const int32_t* block_tables;
  int64_t bt_row_stride;
  int32_t bt_cols, num_pages, page_shift;
  const int32_t* seq_lens;
  const int32_t* cu_kv;
  int32_t num_kv_heads, head_dim, elem_bytes;
  uint8_t* dst;
  int64_t dst_rows;
};

constexpr int kGatherTokens = 64;

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs g) {
  const int b = blockIdx.y;
  const int kv_len = g.seq_lens[b];
  const int t0 = blockIdx.x * kGatherTokens;
  if (t0 >= kv_len) return;
  PageTable pt;
  pt.row = g.block_tables + static_cast<int64_t>(b) * g.bt_row_stride;
  pt.cols = g.bt_cols;
  pt.num_pages = g.num_pages;
  pt.page_shift = g.page_shift;
  const int page_mask = (1 << g.page_shift) - 1;
  const int row_bytes = g.head_dim * g.elem_bytes;
  const int chunks = row_bytes / 16;                   // 16-byte chunks per (token, head)
  const int per_token = chunks * g.num_kv_heads;
  const int64_t dst0 = g.cu_kv[b];
  for (int i = threadIdx.x; i < kGatherTokens * per_token; i += blockDim.x) {
    const int t = t0 + i / per_token;
    if (t >= kv_len) break;
    const int hk = (i % per_token) / chunks;
    const int ch = i % chunks;
    const int64_t row = dst0 + t;
    if (row < 0 || row >= g.dst_rows) continue;
    const int id = page_id(pt, t);
    const int elem = ch * 16 / g.elem_bytes;
    const uint8_t* src = g.elem_bytes == 2 ? token_row<2>(g.plane, id, page_mask, t, hk, elem)
                                           : token_row<1>(g.plane, id, page_mask, t, hk, elem);
    uint8_t* dst = g.dst + ((row * g.num_kv_heads + hk) * static_cast<int64_t>(row_bytes)) + ch * 16;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
}

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// Kernel shape: 8 waves x 32 rows (two waves per SIMD) unless PPA_WAVES=4
// asks for 4 waves x 64 rows (one wave per SIMD).  UPAGE: page_size >= 16.
template <int D, bool FP8, bool UPAGE>
hipError_t launch_shape(const AttnArgs& a, int grid, hipStream_t stream, int waves) {
  if (waves == 4) {
    hipLaunchKernelGGL((paged_prefill_kernel<D, FP8, 2, 4, UPAGE>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((paged_prefill_kernel<D, FP8, 1, 8, UPAGE>), dim3(grid), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch(const AttnArgs& a, int grid, hipStream_t stream, int waves, bool upage) {
  return upage ? launch_shape<D, FP8, true>(a, grid, stream, waves)
               : launch_shape<D, FP8, false>(a, grid, stream, waves);
}

int waves_setting() {
  static int w = [] {
    const char* s = getenv("PPA_WAVES");
    return (s != nullptr && atoi(s) == 4) ? 4 : 8;
  }();
  return w;
}

}  // namespace
}  // namespace ppa

using namespace ppa;

extern "C" int32_t ppa_paged_prefill_attention(const ppa_params* p, void* stream) {
  char msg[8];
  int32_t st = ppa_validate_shapes(p, msg, sizeof msg);
  if (st != PPA_OK) return st;
  if (p->batch_size == 0 || p->max_q_len == 0 || p->num_tokens == 0) return PPA_OK;

  CacheView cv;
  resolve_cache(p, &cv);
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(p->query);
  a.q_tok = p->num_tokens > 1 ? p->query_strides[0] : 0;
  a.q_head = p->num_qo_heads > 1 ? p->query_strides[1] : 0;
  a.out = static_cast<uint16_t*>(p->out);
  a.o_tok = p->num_tokens > 1 ? p->out_strides[0] : 0;
  a.o_head = p->num_qo_heads > 1 ? p->out_strides[1] : 0;
  a.k = PagedPlane{static_cast<const uint8_t*>(cv.k_base), cv.k_page, cv.k_head, cv.k_tok};
  a.v = PagedPlane{static_cast<const uint8_t*>(cv.v_base), cv.v_page, cv.v_head, cv.v_tok};
  a.block_tables = p->block_tables;
  a.bt_row_stride = p->batch_size > 1 ? p->block_tables_row_stride : 0;
  a.bt_cols = p->block_tables_cols;
  a.num_pages = p->num_pages;
  a.page_shift = log2_exact(p->page_size);
  a.seq_lens = p->seq_lens;
  a.cu_q = p->cum_seq_lens_q;
  a.num_tokens = p->num_tokens;
  a.batch = p->batch_size;
  a.num_kv_heads = p->num_kv_heads;
  a.group = p->num_qo_heads / p->num_kv_heads;
  a.gw = a.group < 16 ? a.group : 16;
  a.n_hg = (a.group + a.gw - 1) / a.gw;
  a.tq = 256 / a.gw;
  a.n_qt = (p->max_q_len + a.tq - 1) / a.tq;
  a.window_left = p->window_left;
  a.bmm1 = p->bmm1_scale;
  a.bmm2 = p->bmm2_scale;
  a.bmm1_ptr = p->bmm1_scale_ptr;
  a.bmm2_ptr = p->bmm2_scale_ptr;
  a.sinks = p->sinks;

  const int64_t grid = static_cast<int64_t>(a.n_qt) * a.batch * a.num_kv_heads * a.n_hg;
  if (grid > 0x7fffffff) return PPA_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  const bool fp8 = p->kv_dtype == PPA_DTYPE_FP8_E4M3FN;
  const int w = waves_setting();
  const int g = static_cast<int>(grid);
  // uniform-page staging needs pages of >= 16 tokens whose byte extent fits
  // the 32-bit in-page offsets
  const int eb = fp8 ? 1 : 2;
  auto extent = [&](const PagedPlane& pl) {
    return (static_cast<int64_t>(p->page_size) * pl.tok_stride +
            static_cast<int64_t>(p->num_kv_heads) * pl.head_stride + p->head_dim) * eb;
  };
  const bool upage = p->page_size >= 16 && extent(a.k) < (int64_t{1} << 31) &&
                     extent(a.v) < (int64_t{1} << 31);
  if (p->head_dim == 128)
    e = fp8 ? launch<128, true>(a, g, s, w, upage) : launch<128, false>(a, g, s, w, upage);
  else
    e = fp8 ? launch<64, true>(a, g, s, w, upage) : launch<64, false>(a, g, s, w, upage);
  return e == hipSuccess ? PPA_OK : PPA_ERR_HIP;
}

extern "C" int32_t ppa_gather_paged_kv(const ppa_params* p, int32_t kv_idx, void* dst, int64_t dst_rows,
                                       void* stream) {
  char msg[8];
  int32_t st = ppa_validate_shapes(p, msg, sizeof msg);
  if (st != PPA_OK) return st;
  if (kv_idx != 0 && kv_idx != 1) return PPA_ERR_SHAPE;
  if (p->batch_size == 0 || p->max_kv_len == 0) return PPA_OK;
  if (p->cum_seq_lens_kv == nullptr || dst == nullptr) return PPA_ERR_NULL_POINTER;
  if (dst_rows < 0) return PPA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(dst) & 15u) != 0) return PPA_ERR_ALIGNMENT;
  if (p->kv_form == PPA_KV_SPLIT ? (p->k_cache == nullptr || p->v_cache == nullptr)
                                 : p->kv_cache == nullptr)
    return PPA_ERR_NULL_POINTER;
  CacheView cv;
  resolve_cache(p, &cv);
  GatherArgs g{};
  g.plane = kv_idx == 0 ? PagedPlane{static_cast<const uint8_t*>(cv.k_base), cv.k_page, cv.k_head, cv.k_tok}
                        : PagedPlane{static_cast<const uint8_t*>(cv.v_base), cv.v_page, cv.v_head, cv.v_tok};
  g.block_tables = p->block_tables;
  g.bt_row_stride = p->batch_size > 1 ? p->block_tables_row_stride : 0;
  g.bt_cols = p->block_tables_cols;
  g.num_pages = p->num_pages;
  g.page_shift = log2_exact(p->page_size);
  g.seq_lens = p->seq_lens;
  g.cu_kv = p->cum_seq_lens_kv;
  g.num_kv_heads = p->num_kv_heads;
  g.head_dim = p->head_dim;
  g.elem_bytes = dtype_bytes(p->kv_dtype);
  g.dst = static_cast<uint8_t*>(dst);
  g.dst_rows = dst_rows;
  dim3 grid((p->max_kv_len + kGatherTokens - 1) / kGatherTokens, p->batch_size);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), g);
  return hipGetLastError() == hipSuccess ? PPA_OK : PPA_ERR_HIP;
}
