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
//   One workgroup = 8 waves = 256 "rows"; a row is one (token, q head) pair of
//   one request and one kv head.  The GW = min(G, 16) query heads of a GQA
//   group that share the kv head are interleaved (row = token * GW + head), so
//   a K/V tile staged once in LDS serves every head of the group and the
//   causal boundary of a 32-row MFMA tile spans only 32 / GW tokens.  Each
//   wave owns 32 rows (one MFMA column tile); two waves share a SIMD.
//   Work items are ordered heaviest-first: item / R counts query tiles back
//   from each request's last one (its longest causal span), item % R picks
//   (request, kv head, head group).  With R a multiple of 8, every tile of one
//   (request, kv head) lands on the same XCD (blocks go round-robin over the
//   8 XCDs), so its K/V stays in one L2.
//
// Per 64-key tile
//   1. staging: each wave copies 8 consecutive keys of K and of V from their
//      pages into an LDS ring, both in natural [key][dim] layout with 16-byte
//      chunks XOR swizzled by key: bf16 pages straight into LDS; fp8 codes
//      straight into LDS for the fp8 MFMA arithmetic, or through registers,
//      widened to bf16 on the way, for the widened one (every e4m3fn value
//      is a bf16 value).  With pages of >= 8 tokens a wave's keys share one
//      page, whose id is read by a scalar load ahead of use;
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

#include <atomic>
#include <mutex>

#include "ppa.h"
#include "ppa_internal.h"
#include "ppa_page_addr.hpp"

namespace ppa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short v4s16;
typedef __attribute__((ext_vector_type(8))) short v8s16;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;   // 32 fp8 codes: one f8f6f4 MFMA operand
typedef __attribute__((ext_vector_type(2))) int v2i32;

constexpr int kBK = 64;            // keys per tile
constexpr int kWaves = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;   // log2 units
constexpr float kNegInf = -__builtin_inff();
constexpr float kMinScale = 1.17549435e-38f;  // FLT_MIN
// fp8 arithmetic (fp8_compute): the fewest keys every row of a work item
// must see for the item to run on the fp8 MFMA
constexpr int kFp8MinKeys = 1024;
// bf16 cache at head_dim 64: the V^T operand is read after the softmax, so
// that S and V^T are never live together; the kernel then fits 128 VGPRs
// and two workgroups share a CU
template <int D>
constexpr bool kLateV = D == 64;
template <int D, bool FP8>
constexpr int kWavesPerEU = (!FP8 && kLateV<D>) ? 4 : 2;

// Scheduler counters in the workspace: kSchedQueues queue heads, then the
// number of workgroups that have finished.
constexpr int kSchedQueues = 8;
constexpr int kSchedDone = kSchedQueues;

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
  const int32_t* kv_indptr;    // flat page table, or NULL
  const int32_t* kv_indices;
  int64_t kv_indices_len;
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
  uint32_t* sched;     // persistent schedule: counters in the workspace
  int32_t n_items;     // n_qt * kv_splits * batch * num_kv_heads * n_hg
  int32_t n_queues;    // 1 or kSchedQueues
  int32_t num_qo_heads;
  float* lse;          // [tokens, H_q] natural-log denominators, or NULL
  int64_t lse_tok, lse_head;
  int32_t kv_splits;   // key-tile chunks per work item (1: none)
  float* o_part;       // split mode: [kv_splits, tokens, H_q, D] partial outputs
  float* lse_part;     // split mode: [kv_splits, tokens, H_q] partial log-denominators
  int32_t out_mx;      // 0: bf16 out; 16 or 32: MXFP4 out (packed bytes) with that block size
  uint8_t* out_sf;     // MXFP4: E8M0 scale bytes [tokens, H_q, D / out_mx]
  int64_t sf_tok, sf_head;
  float o_sf_scale;    // MXFP4: y = fp32(o) * o_sf_scale before blocking
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32x64 MFMA on OCP e4m3fn codes (format 0 for both operands), unit
// block scales (E8M0 127 = 2^0)
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 r = __builtin_convertvector(f32x2{lo, hi}, bf16x2);   // v_cvt_pk_bf16_f32, round to nearest even
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

// Combine the values of the lane pair (l, l ^ 32) without an LDS round trip:
// v_permlane32_swap with both operands holding x leaves x[l % 32] in the
// first and x[32 + l % 32] in the second.  Written as inline asm because
// hipcc (ROCm 7.2) folds the two results of __builtin_amdgcn_permlane32_swap
// into one value (max(r0, r1) becomes r0, r0 + r1 becomes 2 r0).  The nops
// cover the VALU-write -> permlane and permlane -> VALU-read hazards.
__device__ __forceinline__ float pair_max(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return a;
}
__device__ __forceinline__ float pair_sum(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_add_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return a;
}


// ---- MXFP4 output (OCP Microscaling FP4) -------------------------------------
// Elements are encoded by gfx950's scaled FP4 conversion
// (v_cvt_scalef32_pk_fp4_f32: two fp32 values -> two E2M1 codes in one byte
// of the result).  Measured on the device: it divides by 2^(exponent field of
// the scale operand - 127), i.e. it reads the scale as an E8M0 value; rounds
// to the nearest E2M1 value with ties to the even code; saturates at 6; copies
// the sign bit (-0 gives the -0 code); and turns NaN into +-6.  That is the
// encoding the oracle states.

// E8M0 byte of the scale 2^E of a block with maximum magnitude amax:
// E = floor(log2(amax)) - 2 (2 = exponent of E2M1's largest value), read
// from the fp32 exponent field (a normal amax has floor(log2) = field - 127,
// so the byte E + 127 is field - 2), clamped at byte 0 (zero and tiny
// maxima); an infinite maximum gives the NaN byte 255.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const uint32_t ex = (__builtin_bit_cast(uint32_t, amax) >> 23) & 0xffu;
  return ex == 255u ? 255u : (ex > 2u ? ex - 2u : 0u);
}

// The conversion's scale operand for byte b: the float 2^(b - 127) (for
// b = 0 the subnormal 2^-127).  A block with the NaN byte gets zero codes
// from the caller instead.
__device__ __forceinline__ float mx_scale_operand(uint32_t b) {
  return __builtin_bit_cast(float, b != 0u ? b << 23 : 0x00400000u);
}

// Four consecutive elements -> four codes in the low 16 bits.
__device__ __forceinline__ uint32_t mx_pack4(float y0, float y1, float y2, float y3, float scale) {
  const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, scale, 0);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y2, y3, scale, 1);
}

// Tile geometry.  Every wave stages 8 consecutive keys of both K and V of a
// 64-key tile, so the staging work is the same for all waves and, with pages
// of >= 8 tokens, a wave's keys lie in one page whose id is wave-uniform.
// bf16 cache: K and V tiles are copied from the pages into LDS without
// passing through registers (fetch_kv_lds), in natural [key][dim] layout with
// unpadded rows whose 16-byte chunks are XOR swizzled by key (kswz, vswz), in
// a four-stage ring consumed two tiles per barrier.  The PV operand, V^T, is
// read with LDS transpose loads.
// fp8 cache, widened arithmetic: staged through registers (widened to bf16
// once per workgroup) into the same swizzled layout, so both caches share
// the operand reads; two stages.  fp8 cache, fp8 MFMA arithmetic: the codes
// copied like the bf16 tiles (fetch_kv_lds_f8), four stages.
template <int D, bool FP8, bool F8M = false>
struct Tile {
  static constexpr int EB = FP8 ? 1 : 2;        // bytes per cache element
  static constexpr int K_LANE_BYTES = D * EB / 8;              // 8 rows per wave
  static constexpr int K_LOAD = K_LANE_BYTES < 16 ? K_LANE_BYTES : 16;
  static constexpr int K_PASSES = K_LANE_BYTES / K_LOAD;
  static constexpr int K_CHUNK = K_LOAD / EB;   // elements per load
  static constexpr int K_TPR = D / K_CHUNK;     // lanes per key row
  static constexpr int K_RPI = 64 / K_TPR;      // key rows per wave instruction
  static constexpr int V_DPT = D / 32;          // dims per lane (32 dim groups)
  static constexpr int V_KEY_BYTES = V_DPT * EB;   // raw bytes per key per lane
  static constexpr bool DMA = !FP8;             // bf16: pages -> LDS directly
  static constexpr int STAGES = DMA ? 4 : 2;     // LDS ring depth
  static constexpr int K_DW = DMA ? 1 : K_LANE_BYTES / 4;
  static constexpr int V_DW = DMA ? 1 : (4 * V_KEY_BYTES + 3) / 4;
  // fp8 cache at head_dim 128: QK^T and PV on the fp8 MFMA (Q and P
  // quantised to e4m3fn); K and V stay in code bytes [key][dim], 8 KB each,
  // one 16 KB stage of the ring per bf16 stage buffer
  static constexpr bool F8MMA = F8M;
  static_assert(!F8M || (FP8 && D == 128), "fp8 MFMA: fp8 cache at head_dim 128");
  static constexpr int K_ELEMS = kBK * D;   // both: natural [key][dim], swizzled
  static constexpr int V_ELEMS = kBK * D;
  static_assert(K_PASSES * K_RPI == 8, "K staging map");
};


template <int BYTES>
__device__ __forceinline__ void load_bytes(uint32_t* dst, const uint8_t* src, bool ok) {
  if constexpr (BYTES == 16) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(src);
    for (int i = 0; i < 4; ++i) dst[i] = ok ? x[i] : 0u;
  } else if constexpr (BYTES == 8) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(src);
    dst[0] = ok ? x[0] : 0u;
    dst[1] = ok ? x[1] : 0u;
  } else if constexpr (BYTES == 4) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(src);
    dst[0] = ok ? x : 0u;
  }
}

// ---- staging, bf16 cache: pages -> LDS directly --------------------------------
// Swizzle keys: chunk c (16 bytes) of LDS row `key` sits in slot c ^ swz(key).
// K: sixteen lanes read one chunk index of sixteen consecutive rows for the S
// operand; key mod 16 (D = 128, 256-byte rows) or (key / 2) mod 8 (D = 64,
// two rows per 256 bytes) puts them on distinct banks.  V: a transpose load
// makes each 16-lane group read 4 consecutive keys x 32 bytes; 4 (key mod 4)
// (D = 128) or 4 ((key / 2) mod 2) (D = 64) spreads the 32 lanes of a half
// wave over 256 distinct bytes.
template <int D>
__device__ __forceinline__ int kswz(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int key) {
  return D == 128 ? ((key & 3) << 2) : (((key >> 1) & 1) << 2);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// global_load_lds_dwordx4 moves 16 bytes per lane into LDS at the wave-uniform
// base in M0, lane i at base + 16 i: one instruction fills 1 KB, 64 / (D / 8)
// whole rows.  Each lane loads the global chunk that belongs at its slot.
// The copies are issued from inline asm so that the compiler does not see an
// LDS store in flight: it would otherwise wait for it before every LDS read
// of the other stages.  The caller waits with vmcnt for them; vector memory
// operations retire in order, so the compiler's own vmcnt waits stay correct
// (at worst longer) with these in the count.  M0 is written here and nowhere
// else in these kernels, and an LDS copy reading M0 needs one wait state
// after the SALU write (the s_nop).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 in the clobber list: see above
__device__ __forceinline__ void lds_copy16(uint32_t lds_base, const uint8_t* src) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_copy16(uint32_t lds_base, const uint8_t* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase),
               "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// The wave's keys [kb, kb + 8) of K and V into the tile's LDS stage.  Fast
// path (`id` is their page, the tile is not the last of the request): 32-bit
// offsets from the wave-uniform page base.  General path: every lane
// resolves its key through the page table, clamped to the sequence; a
// clamped copy is a valid key whose weight the mask sets to exactly 0.
template <int D, bool FAST>
__device__ __forceinline__ void fetch_kv_lds(__bf16* kt, __bf16* vt, const AttnArgs& a, const PageTable& pt, int id,
                                             int hk, int kb, int kv_len, int page_mask, int wave, int lane) {
  constexpr int TPR = D / 8;      // 16-byte chunks per row
  constexpr int RPI = 64 / TPR;   // rows per copy instruction
  const uint8_t* kbase = a.k.base;
  const uint8_t* vbase = a.v.base;
  // the lane's offsets are recomputed at every call: hoisted out of the
  // loops that call this, they would be held in registers the whole time
  asm volatile("" : "+v"(lane));
  if (FAST) {
    kbase += (static_cast<int64_t>(id) * a.k.page_stride + static_cast<int64_t>(hk) * a.k.head_stride) * 2;
    vbase += (static_cast<int64_t>(id) * a.v.page_stride + static_cast<int64_t>(hk) * a.v.head_stride) * 2;
  }
  for (int p = 0; p < 8 / RPI; ++p) {
    const int rl = p * RPI + lane / TPR;            // key of the wave, 0..7
    const int row = 8 * wave + rl;                   // key of the tile
    const int kc = (lane % TPR) ^ kswz<D>(row);
    const int vc = (lane % TPR) ^ vswz<D>(row);
    const uint32_t kdst = lds_addr(kt + (8 * wave + p * RPI) * D);
    const uint32_t vdst = lds_addr(vt + (8 * wave + p * RPI) * D);
    if (FAST) {
      const int slot = (kb & page_mask) + rl;
      lds_copy16(kdst, kbase, static_cast<uint32_t>((slot * static_cast<int>(a.k.tok_stride) + kc * 8) * 2));
      lds_copy16(vdst, vbase, static_cast<uint32_t>((slot * static_cast<int>(a.v.tok_stride) + vc * 8) * 2));
    } else {
      const int key = kb + rl;
      const int k = key < kv_len ? key : kv_len - 1;
      const int pid = page_id(pt, k);
      lds_copy16(kdst, token_row<2>(a.k, pid, page_mask, k, hk, kc * 8));
      lds_copy16(vdst, token_row<2>(a.v, pid, page_mask, k, hk, vc * 8));
    }
  }
}

// fp8 cache at head_dim 128, fp8 MFMA arithmetic: the wave's keys
// [kb, kb + 8) of K and of V, as stored (e4m3fn codes, 128-byte rows), into
// the tile's K and V stages, 16-byte chunk c of key row r in slot
// c ^ ((r / 2) mod 8).  One copy instruction per plane moves the wave's
// 1 KB: lane i writes row i / 8, slot i mod 8, so it loads the global
// chunk (i mod 8) ^ ((row / 2) mod 8).  Fast and general paths as in
// fetch_kv_lds.
template <bool FAST>
__device__ __forceinline__ void fetch_kv_lds_f8(uint8_t* kt, uint8_t* vt, const AttnArgs& a, const PageTable& pt,
                                                int id, int hk, int kb, int kv_len, int page_mask, int wave,
                                                int lane) {
  asm volatile("" : "+v"(lane));   // recomputed per call, as in fetch_kv_lds
  const int rl = lane >> 3;                       // key of the wave, 0..7
  const int row = 8 * wave + rl;                  // key of the tile
  const int c = (lane & 7) ^ ((row >> 1) & 7);    // global chunk of the lane's slot
  const uint32_t kdst = lds_addr(kt + 8 * wave * 128);
  const uint32_t vdst = lds_addr(vt + 8 * wave * 128);
  if (FAST) {
    const uint8_t* kbase =
        a.k.base + static_cast<int64_t>(id) * a.k.page_stride + static_cast<int64_t>(hk) * a.k.head_stride;
    const uint8_t* vbase =
        a.v.base + static_cast<int64_t>(id) * a.v.page_stride + static_cast<int64_t>(hk) * a.v.head_stride;
    const int slot = (kb & page_mask) + rl;
    lds_copy16(kdst, kbase, static_cast<uint32_t>(slot * static_cast<int>(a.k.tok_stride) + c * 16));
    lds_copy16(vdst, vbase, static_cast<uint32_t>(slot * static_cast<int>(a.v.tok_stride) + c * 16));
  } else {
    const int key = kb + rl;
    const int k = key < kv_len ? key : kv_len - 1;
    const int pid = page_id(pt, k);
    lds_copy16(kdst, token_row<1>(a.k, pid, page_mask, k, hk, c * 16));
    lds_copy16(vdst, token_row<1>(a.v, pid, page_mask, k, hk, c * 16));
  }
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt not waited on), n < 16.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}

// ---- staging, fp8 cache: pages -> registers -------------------------------------
// The wave's keys are [kb, kb + 8).  Fast path (`id` is their page, the tile is
// not the last one of the request): rows are addressed by 32-bit offsets from
// the wave-uniform page base.  General path: every lane resolves its own keys
// through the page table, clamped to the sequence, and zero-fills keys past
// kv_len.
template <int D, bool FP8, bool FAST>
__device__ __forceinline__ void fetch_kv(uint32_t* kraw, uint32_t* vraw, const AttnArgs& a, const PageTable& pt,
                                         int id, int hk, int kb, int kv_len, int page_mask, int lane) {
  using T = Tile<D, FP8>;
  const int r0 = lane / T::K_TPR;
  const int chunk = lane % T::K_TPR;
  const int kgl = lane >> 5;   // V: keys kb + 4 kgl .. + 3
  const int dg = lane & 31;    // V: dims dg * V_DPT .. + V_DPT - 1
  if (FAST) {
    const int64_t page_off = static_cast<int64_t>(id) * a.k.page_stride + static_cast<int64_t>(hk) * a.k.head_stride;
    const int64_t vpage_off = static_cast<int64_t>(id) * a.v.page_stride + static_cast<int64_t>(hk) * a.v.head_stride;
    const uint8_t* kbase = a.k.base + page_off * T::EB;
    const uint8_t* vbase = a.v.base + vpage_off * T::EB;
    const int slot0 = kb & page_mask;
    for (int p = 0; p < T::K_PASSES; ++p) {
      const uint32_t off = static_cast<uint32_t>(
          ((slot0 + p * T::K_RPI + r0) * static_cast<int>(a.k.tok_stride) + chunk * T::K_CHUNK) * T::EB);
      load_bytes<T::K_LOAD>(kraw + p * (T::K_LOAD / 4), kbase + off, true);
    }
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = static_cast<uint32_t>(
          ((slot0 + 4 * kgl + r) * static_cast<int>(a.v.tok_stride) + dg * T::V_DPT) * T::EB);
      if constexpr (T::V_KEY_BYTES >= 4) {
        load_bytes<T::V_KEY_BYTES>(vraw + r * (T::V_KEY_BYTES / 4), vbase + off, true);
      } else {   // 2 bytes per key: pack two keys per dword
        const uint32_t x = *reinterpret_cast<const uint16_t*>(vbase + off);
        vraw[r >> 1] = (r & 1) ? (vraw[r >> 1] | (x << 16)) : x;
      }
    }
  } else {
    for (int p = 0; p < T::K_PASSES; ++p) {
      const int key = kb + p * T::K_RPI + r0;
      const bool ok = key < kv_len;
      const int kc = ok ? key : kv_len - 1;
      const int kid = page_id(pt, kc);
      load_bytes<T::K_LOAD>(kraw + p * (T::K_LOAD / 4),
                            token_row<T::EB>(a.k, kid, page_mask, kc, hk, chunk * T::K_CHUNK), ok);
    }
    for (int r = 0; r < 4; ++r) {
      const int key = kb + 4 * kgl + r;
      const bool ok = key < kv_len;
      const int kc = ok ? key : kv_len - 1;
      const int vid = page_id(pt, kc);
      const uint8_t* src = token_row<T::EB>(a.v, vid, page_mask, kc, hk, dg * T::V_DPT);
      if constexpr (T::V_KEY_BYTES >= 4) {
        load_bytes<T::V_KEY_BYTES>(vraw + r * (T::V_KEY_BYTES / 4), src, ok);
      } else {
        const uint32_t x = ok ? static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(src)) : 0u;
        vraw[r >> 1] = (r & 1) ? (vraw[r >> 1] | (x << 16)) : x;
      }
    }
  }
}

// ---- staging: registers -> LDS ------------------------------------------------
// fp8 cache: the wave's 8 keys, widened to bf16, into the same natural,
// swizzled layout the direct copies produce (16-byte chunk c of key row r
// in slot c ^ kswz(r) for K, c ^ vswz(r) for V), so that both caches share
// the operand reads.
template <int D, bool FP8, bool F8M>
__device__ __forceinline__ void store_kv(const uint32_t* kraw, const uint32_t* vraw, __bf16* klds, __bf16* vlds,
                                         int wave, int lane) {
  using T = Tile<D, FP8, F8M>;
  if constexpr (!FP8) return;   // the bf16 cache is copied straight into LDS
  static_assert(!T::F8MMA, "the fp8 MFMA path copies K and V straight into LDS");
  // K: K_CHUNK fp8 codes of row r0 from element chunk * K_CHUNK, i.e. whole
  // 16-byte bf16 chunks chunk * K_CHUNK / 8 ..
  const int r0 = lane / T::K_TPR;
  const int chunk = lane % T::K_TPR;
  for (int p = 0; p < T::K_PASSES; ++p) {
    const int row = 8 * wave + p * T::K_RPI + r0;
    const uint32_t* x = kraw + p * (T::K_LOAD / 4);
    for (int q = 0; q < T::K_CHUNK / 8; ++q) {
      const u32x2 a0 = fp8x4_to_bf16x4(x[2 * q]);
      const u32x2 a1 = fp8x4_to_bf16x4(x[2 * q + 1]);
      const int c = chunk * (T::K_CHUNK / 8) + q;
      *reinterpret_cast<u32x4*>(klds + row * D + ((c ^ kswz<D>(row)) << 3)) = u32x4{a0[0], a0[1], a1[0], a1[1]};
    }
  }
  // V: keys key0 + r (r = 0..3) x dims dg * V_DPT .. + V_DPT - 1 of the lane
  constexpr int PAIRS = T::V_DPT / 2;   // bf16 pairs per key
  const int key0 = 8 * wave + 4 * (lane >> 5);
  const int dg = lane & 31;
  const int d0 = dg * T::V_DPT;
  for (int r = 0; r < 4; ++r) {
    const int key = key0 + r;
    __bf16* dst = vlds + key * D + (((d0 >> 3) ^ vswz<D>(key)) << 3) + (d0 & 7);
    if constexpr (T::V_KEY_BYTES == 4) {   // 4 fp8 per key
      *reinterpret_cast<u32x2*>(dst) = fp8x4_to_bf16x4(vraw[r]);
    } else {                                // 2 fp8 per key, two keys per dword
      static_assert(!FP8 || PAIRS == 1, "V staging map");
      const uint32_t codes = (vraw[r >> 1] >> (16 * (r & 1))) & 0xffffu;
      *reinterpret_cast<uint32_t*>(dst) = fp8x4_to_bf16x4(codes)[0];
    }
  }
}

// MXFP4 store of one output row from the PV accumulators.  Lane (col, half)
// holds dims md*32 + 8g + 4half + e (e = 0..3) of its row, so a block of VEC
// dims is split between the lane and its partner lane ^ 32, which hold the
// same row: the block maximum is the pair maximum of the two lanes' maxima.
// y = fp32(fp32(acc * inv) * g); codes go out 4 per 16-bit store, the
// scale byte from the half-0 lane.
template <int D, int VEC>
__device__ __forceinline__ void store_mxfp4_row(const f32x16* oacc, float inv, float g, uint8_t* orow,
                                                uint8_t* sfrow, int half) {
  constexpr int GB = VEC / 8;   // 8-dim groups per block
  // codes[G]: this lane's four codes (16 bits) of 8-dim group G of the row,
  // i.e. dims 8 G + 4 half .. + 3
  uint32_t codes[D / 8];
  for (int b = 0; b < D / VEC; ++b) {
    const int md = b * VEC / 32;
    const int g0 = (b * VEC % 32) / 8;
    float y[GB][4];
    float amax = 0.f;
    for (int gg = 0; gg < GB; ++gg)
      for (int e = 0; e < 4; ++e) {
        y[gg][e] = (oacc[md][4 * (g0 + gg) + e] * inv) * g;
        amax = fmaxf(amax, __builtin_fabsf(y[gg][e]));
      }
    amax = pair_max(amax);
    const uint32_t sb = mx_scale_byte(amax);
    const float sc = mx_scale_operand(sb);
    for (int gg = 0; gg < GB; ++gg) {
      const uint32_t w = mx_pack4(y[gg][0], y[gg][1], y[gg][2], y[gg][3], sc);
      codes[b * GB + gg] = sb == 255u ? 0u : (w & 0xffffu);
    }
    if (half == 0) sfrow[b] = static_cast<uint8_t>(sb);
  }
  // Each 64-dim chunk (32 bytes of the row): half 0 stores groups 0-3 and
  // half 1 groups 4-7, each group whole (its two halves' codes side by
  // side), as one 16-byte store per lane instead of eight 2-byte ones.  The
  // lanes exchange (own group k, own group k + 4) words with their partner
  // (v_permlane32_swap: lanes 32-63 of the first register with lanes 0-31
  // of the second, so that each lane ends with its partner's word in one of
  // them).
  for (int c = 0; c < D / 64; ++c) {
    uint32_t res[4];
    for (int k = 0; k < 4; ++k) {
      const uint32_t x = codes[8 * c + k] | (codes[8 * c + k + 4] << 16);
      uint32_t r0 = x, r1 = x;
      asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(r0), "+v"(r1));
      const uint32_t partner = half ? r0 : r1;
      res[k] = half ? ((partner >> 16) | (x & 0xffff0000u)) : ((x & 0xffffu) | (partner << 16));
    }
    *reinterpret_cast<u32x4*>(orow + c * 32 + 16 * half) = u32x4{res[0], res[1], res[2], res[3]};
  }
}

// Final scale of one row's O (lane; no key split): bmm2 over the softmax
// denominator with the sink's term; writes the row's log-sum-exp when asked.
// The sink joins the denominator relative to max(running max, sink), so that
// a sink far above every logit gives l ~ 1 and lse ~ sink instead of an
// infinite l; O is scaled by the same factor (1 when the sink is below the
// running maximum, and for a -inf sink).  Contraction off, as in store_row.
__device__ __forceinline__ float row_scale(const AttnArgs& a, float l, float m_run, float sink, int h, int64_t trow,
                                           int half, float bmm2) {
#pragma clang fp contract(off)
  float mb = m_run == kNegInf ? 0.f : m_run;
  float oscale = 1.f;
  if (a.sinks) {
    const float s2 = sink * kLog2e;
    const float m2 = s2 > mb ? s2 : mb;
    oscale = __builtin_amdgcn_exp2f(mb - m2);
    l = l * oscale + __builtin_amdgcn_exp2f(s2 - m2);
    mb = m2;
  }
  if (a.lse != nullptr && half == 0)
    a.lse[trow * a.lse_tok + static_cast<int64_t>(h) * a.lse_head] = mb * kLn2 + __builtin_logf(l);
  return (bmm2 * oscale) / l;
}

// Epilogue of one row (lane): the row's final output, or in split mode its
// partial state.  l is the row's denominator over the keys it saw (both lane
// halves), m_run its running maximum in log2 units, oacc its unnormalized O
// (this lane's half of the dims).  Contraction is off so that every kernel
// that inlines this rounds the same operations the same way (the persistent
// and the one-item-per-workgroup schedules give identical bits).
template <int D>
__device__ __forceinline__ void store_row(const AttnArgs& a, const f32x16 (&oacc)[D / 32], float l, float m_run,
                                          float sink, int h, int64_t trow, int split, int half, float bmm2) {
#pragma clang fp contract(off)
  constexpr int MD = D / 32;
  float mb = m_run == kNegInf ? 0.f : m_run;
  if (a.kv_splits > 1) {
    // partial state of this key chunk (no sink; a row with no key here
    // gets 0 and -inf): output normalized over the chunk, log-denominator
    const float pinv = l > 0.f ? bmm2 / l : 0.f;
    const int64_t prow = (static_cast<int64_t>(split) * a.num_tokens + trow) * a.num_qo_heads + h;
    float* dst = a.o_part + prow * D;
    for (int md = 0; md < MD; ++md)
      for (int g = 0; g < 4; ++g) {
        const int d = md * 32 + 8 * g + 4 * half;
        typedef __attribute__((ext_vector_type(4))) float f32x4;
        *reinterpret_cast<f32x4*>(dst + d) = f32x4{oacc[md][4 * g] * pinv, oacc[md][4 * g + 1] * pinv,
                                                   oacc[md][4 * g + 2] * pinv, oacc[md][4 * g + 3] * pinv};
      }
    if (half == 0) a.lse_part[prow] = l > 0.f ? mb * kLn2 + __builtin_logf(l) : kNegInf;
    return;
  }
  const float inv = row_scale(a, l, m_run, sink, h, trow, half, bmm2);
  if (a.out_mx != 0) {
    uint8_t* orow8 = reinterpret_cast<uint8_t*>(a.out) + trow * a.o_tok + static_cast<int64_t>(h) * a.o_head;
    uint8_t* sfrow = a.out_sf + trow * a.sf_tok + static_cast<int64_t>(h) * a.sf_head;
    if (a.out_mx == 16) store_mxfp4_row<D, 16>(oacc, inv, a.o_sf_scale, orow8, sfrow, half);
    else store_mxfp4_row<D, 32>(oacc, inv, a.o_sf_scale, orow8, sfrow, half);
    return;
  }
  // Lane half h holds dims 8 g + 4 h .. + 3 of each 32-dim block md.  For
  // each pair of groups (g0, g0 + 1) the halves swap one piece (lanes 32-63
  // of the first register with lanes 0-31 of the second), so that half 0
  // holds dims 8 g0 .. + 7 and half 1 dims 8 (g0 + 1) .. + 7: one 16-byte
  // store per lane writes 32 contiguous bytes of the row per lane pair,
  // half as many store instructions (and memory requests) as 8-byte ones.
  uint16_t* orow = a.out + trow * a.o_tok + static_cast<int64_t>(h) * a.o_head;
  for (int md = 0; md < MD; ++md) {
    for (int g0 = 0; g0 < 4; g0 += 2) {
      uint32_t a0 = pack_bf16(oacc[md][4 * g0] * inv, oacc[md][4 * g0 + 1] * inv);
      uint32_t a1 = pack_bf16(oacc[md][4 * g0 + 2] * inv, oacc[md][4 * g0 + 3] * inv);
      uint32_t b0 = pack_bf16(oacc[md][4 * g0 + 4] * inv, oacc[md][4 * g0 + 5] * inv);
      uint32_t b1 = pack_bf16(oacc[md][4 * g0 + 6] * inv, oacc[md][4 * g0 + 7] * inv);
      asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %2\n\tv_permlane32_swap_b32 %1, %3\n\ts_nop 1"
                   : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1));
      const int d = md * 32 + 8 * (g0 + half);
      *reinterpret_cast<u32x4*>(orow + d) = u32x4{a0, a1, b0, b1};
    }
  }
}

// One work item: `item` = (query tile, request, kv head, head group), counted
// heaviest query tile first.  Per K/V tile: stage tile j+1 into registers, run
// S, softmax and PV for tile j from LDS, store tile j+1 into the other LDS
// buffer, barrier.  Every wave of the workgroup calls this with the same item.
template <int D, bool FP8, bool UPAGE, bool F8M>
__device__ __forceinline__ void attend_item(const AttnArgs& a, const int item) {
  using T = Tile<D, FP8, F8M>;
  constexpr int KSTEPS = D / 16;   // MFMA K-steps over head_dim
  constexpr int MD = D / 32;       // 32-wide head_dim tiles of O^T
  __shared__ __attribute__((aligned(16))) __bf16 klds[T::STAGES][T::K_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 vlds[T::STAGES][T::V_ELEMS];

  // ---- which work item --------------------------------------------------
  // item = (query tile counted from the request's last one, key chunk,
  // request, kv head, head group): the last tiles of all requests (the
  // longest causal spans) come first whatever the requests' lengths
  const int R = a.batch * a.num_kv_heads * a.n_hg;
  const int S = a.kv_splits;
  const int rest = item % R;
  const int split = (item / R) % S;
  const int qk = item / R / S;
  const int b = rest / (a.num_kv_heads * a.n_hg);
  const int hk = (rest / a.n_hg) % a.num_kv_heads;
  const int hg = rest % a.n_hg;

  // request metadata through the constant address space: scalar loads (the
  // kernel never writes these arrays), with the request's page-table row
  typedef const __attribute__((address_space(4))) int32_t cint32;
  int q1 = ((cint32*)(a.cu_q))[b + 1];
  int q0 = ((cint32*)(a.cu_q))[b];
  int kv_len = ((cint32*)(a.seq_lens))[b];
  PageTable pt;
  request_table(pt, b, a.block_tables, a.bt_row_stride, a.bt_cols, a.kv_indptr, a.kv_indices, a.kv_indices_len);
  // Without a window, the first key chunk of an item starts at tile 0, so
  // with the padded table the page ids of the wave's keys in tiles 0..3 are
  // known before the request's lengths: they load in the same scalar batch
  // (raw ids, clamped when used; ids past the request's last page are read
  // from inside the table row and never used).
  const bool spec_ids = UPAGE && T::DMA && a.kv_indptr == nullptr && a.window_left < 0 && split == 0;
  int sid[4] = {0, 0, 0, 0};
  if (spec_ids) {
    const bool empty = a.bt_cols <= 0;
    const int last = empty ? 0 : a.bt_cols - 1;
    cint32* row = (cint32*)(empty ? a.cu_q : pt.row);
    const int w = uniform(static_cast<int>(threadIdx.x >> 6));
    for (int i = 0; i < 4; ++i) {
      int cl = (i * kBK + 8 * w) >> a.page_shift;
      cl = cl < last ? cl : last;
      sid[i] = row[cl];
    }
  }
  // every one of them is taken here, so all loads go out together: otherwise
  // the compiler sinks those used only after the early return below past
  // it, and each costs a serial round trip
  asm volatile("" : : "s"(q0), "s"(q1), "s"(kv_len), "s"(pt.row), "s"(pt.cols), "s"(sid[0]), "s"(sid[1]),
               "s"(sid[2]), "s"(sid[3]));
  q1 = q1 < a.num_tokens ? q1 : a.num_tokens;
  q0 = q0 < 0 ? 0 : (q0 < q1 ? q0 : q1);
  const int q_len = q1 - q0;
  kv_len = kv_len < 0 ? 0 : kv_len;
  const int qt = (q_len + a.tq - 1) / a.tq - 1 - qk;
  if (qt < 0) return;
  const int t0 = qt * a.tq;
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

  // ---- the wave's 32 rows -----------------------------------------------------
  const int r = wave * 32 + col;
  const int tok = r / a.gw;
  const int hd = r % a.gw;
  const bool rvalid = tok < ntok && hd < nheads;
  const int pos = prefix + t0 + tok;
  const int wtok_first = (wave * 32) / a.gw;
  int wtok_last = (wave * 32 + 31) / a.gw;
  wtok_last = wtok_last < ntok - 1 ? wtok_last : ntok - 1;
  const bool wave_active = wtok_first < ntok;
  const int wpos_first = prefix + t0 + wtok_first;
  const int wpos_last = prefix + t0 + wtok_last;
  const int wkey_hi = wpos_last < kv_len - 1 ? wpos_last : kv_len - 1;
  const int wkey_lo = W >= 0 ? (wpos_first - W > 0 ? wpos_first - W : 0) : 0;

  bf16x8 qf[KSTEPS];   // B operand of S^T = K Q^T
  auto load_q = [&]() {
    // invalid rows load a valid row (the item's first) and are zeroed
    const uint16_t* qrow = a.q + static_cast<int64_t>(q0 + t0 + (rvalid ? tok : 0)) * a.q_tok +
                           static_cast<int64_t>(h0 + (rvalid ? hd : 0)) * a.q_head;
    for (int s = 0; s < KSTEPS; ++s) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + s * 16 + half * 8);
      if (!rvalid) x = u32x4{0, 0, 0, 0};
      if (negate_q) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  };
  // fp8 MFMA: the B operand of S^T = K Q^T is 32 e4m3fn codes per lane and
  // 64-dim chunk c, dims 64 c + 32 half + 0..31 in byte order (the K
  // operand takes the same dims in the same bytes, so the MFMA's own order
  // of the contraction index within a lane does not matter).  Values beyond
  // the e4m3fn range saturate at +-448.
  i32x8 qf8[2];
  auto load_q8 = [&]() {
    const uint16_t* qrow = a.q + static_cast<int64_t>(q0 + t0 + (rvalid ? tok : 0)) * a.q_tok +
                           static_cast<int64_t>(h0 + (rvalid ? hd : 0)) * a.q_head;
    for (int cc = 0; cc < 2; ++cc) {
      uint32_t w[16];
      for (int t = 0; t < 4; ++t) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 64 * cc + 32 * half + 8 * t);
        if (!rvalid) x = u32x4{0, 0, 0, 0};
        if (negate_q) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        for (int e = 0; e < 4; ++e) w[4 * t + e] = x[e];
      }
      for (int jd = 0; jd < 8; ++jd) {
        float f[4] = {__builtin_bit_cast(float, w[2 * jd] << 16), __builtin_bit_cast(float, w[2 * jd] & 0xffff0000u),
                      __builtin_bit_cast(float, w[2 * jd + 1] << 16),
                      __builtin_bit_cast(float, w[2 * jd + 1] & 0xffff0000u)};
        for (int e = 0; e < 4; ++e) f[e] = __builtin_fminf(__builtin_fmaxf(f[e], -448.f), 448.f);
        int code = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        code = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], code, true);
        qf8[cc][jd] = code;
      }
    }
  };
  // ---- K/V tile range of the workgroup -------------------------------------
  const int pos_first = prefix + t0;
  const int pos_last = prefix + t0 + ntok - 1;
  const int key_hi = pos_last < kv_len - 1 ? pos_last : kv_len - 1;
  const int key_lo = W >= 0 ? (pos_first - W > 0 ? pos_first - W : 0) : 0;
  int tile_lo = key_lo / kBK;
  int tile_hi = key_hi >= 0 ? key_hi / kBK : -1;
  if (S > 1 && tile_hi >= tile_lo) {   // this chunk's share of the key tiles
    const int n = tile_hi - tile_lo + 1;
    const int first = tile_lo;
    tile_lo = first + (split * n) / S;
    tile_hi = first + ((split + 1) * n) / S - 1;
  }

  // direct-copy path: Q is loaded after the first tile's copies are issued
  // (below), and both are waited for together, so that no later compiler
  // wait for Q covers the prefetched tiles
  if constexpr (!T::DMA && !T::F8MMA) load_q();
  // the row's sink logit, read now so that the epilogue does not wait for it
  const float sink = a.sinks ? a.sinks[h0 + (rvalid ? hd : 0)] : 0.f;

  f32x16 oacc[MD];
  for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};
  float m_run = kNegInf, l_part = 0.f;
  f32x16 sacc[2];
  bf16x8 pb[4];

  pt.num_pages = a.num_pages;
  pt.page_shift = a.page_shift;
  const int page_mask = (1 << a.page_shift) - 1;
  uint32_t kraw[T::K_DW], vraw[T::V_DW];
  int id_next = 0;   // page id of the wave's keys in the next tile to fetch

  const int krow_lane = swap_bits23(col);
  // transpose-load addresses: group G = lane / 16,
  // jj = lane % 16; key 8 (G / 2) + jj / 4 (+ 16 ks, + 4 for the second
  // load), dims md*32 + 16 (G % 2) + 4 (jj % 4), i.e. 16-byte chunk
  // 4 md + 2 (G % 2) + (jj % 4) / 2 at byte 8 (jj % 2) of it, in slot
  // chunk ^ vswz(key) (vswz depends only on jj / 4 here)
  int vt_lane = 0, vt_md[MD];
  {
    const int G = lane >> 4, jj = lane & 15;
    const int key = 8 * (G >> 1) + (jj >> 2);
    vt_lane = key * (2 * D) + (jj & 1) * 8;
    for (int md = 0; md < MD; ++md) vt_md[md] = ((4 * md + 2 * (G & 1) + ((jj & 3) >> 1)) ^ vswz<D>(key)) * 16;
  }

  // fp8 MFMA V^T transpose loads (read_v): group G = lane / 16, jj =
  // lane % 16 points at key 8 (G / 2) + jj / 2 (+ 16 r), 16-byte chunk
  // 2 md + G mod 2 at byte 8 (jj mod 2), in slot chunk ^ ((key / 2) mod 8)
  // ((key / 2) mod 8 does not depend on r)
  int vt8_lane = 0, vt8_md[MD];
  if constexpr (T::F8MMA) {
    const int G = lane >> 4, jj = lane & 15;
    vt8_lane = (8 * (G >> 1) + (jj >> 1)) * 128 + 8 * (jj & 1);
    const int sw = (4 * (G >> 1) + (jj >> 2)) & 7;
    for (int md = 0; md < MD; ++md) vt8_md[md] = ((2 * md + (G & 1)) ^ sw) * 16;
  }

  auto wave_tile = [&](int j) {
    return wave_active && j * kBK <= wkey_hi && j * kBK + kBK - 1 >= wkey_lo;
  };
  auto page_of = [&](int j) { return UPAGE ? page_id_uniform(pt, uniform(j * kBK + 8 * wave)) : 0; };
  // the same without branches, so that several lookups share one scalar
  // round trip: an empty table reads cu_q[0] instead (any readable word
  // will do: the id is clamped to a valid page before use)
  auto page_of_nb = [&](int j) {
    if (!UPAGE) return 0;
    const int token = uniform(j * kBK + 8 * wave);
    const bool empty = pt.cols <= 0;
    int col = token >> pt.page_shift;
    const int last = empty ? 0 : pt.cols - 1;
    col = col < last ? col : last;
    const __attribute__((address_space(4))) int32_t* row =
        (const __attribute__((address_space(4))) int32_t*)(empty ? a.cu_q : pt.row);
    int id = row[col];
    id = id < 0 ? 0 : id;
    return id < pt.num_pages ? id : pt.num_pages - 1;
  };
  // copy the wave's 8 keys of tile j into registers; `id` is their page id
  // LDS stage of tile j
  auto stage = [&](int j) { return T::DMA ? (j - tile_lo) & 3 : (j - tile_lo) & 1; };
  // fp8 MFMA: four 16 KB stages (8 KB of K codes, then 8 KB of V^T codes),
  // one in each of the four 16 KB bf16 stage buffers; stage s of tile j is
  // (j - lo) mod 4
  auto f8k = [&](int j) {
    const int st = (j - tile_lo) & 3;
    return st < 2 ? klds[st] : vlds[st - 2];
  };
  auto f8v = [&](int j) { return f8k(j) + 4096; };
  auto stage_fetch = [&](int j, int id) {
    const int kb = j * kBK + 8 * wave;
    const bool fast = UPAGE && j * kBK + kBK <= kv_len;
    if constexpr (T::F8MMA) {
      uint8_t* kt = reinterpret_cast<uint8_t*>(f8k(j));
      uint8_t* vt = reinterpret_cast<uint8_t*>(f8v(j));
      if (fast) fetch_kv_lds_f8<true>(kt, vt, a, pt, id, hk, kb, kv_len, page_mask, wave, lane);
      else fetch_kv_lds_f8<false>(kt, vt, a, pt, id, hk, kb, kv_len, page_mask, wave, lane);
    } else if constexpr (T::DMA) {
      const int st = stage(j);
      if (fast) fetch_kv_lds<D, true>(klds[st], vlds[st], a, pt, id, hk, kb, kv_len, page_mask, wave, lane);
      else fetch_kv_lds<D, false>(klds[st], vlds[st], a, pt, id, hk, kb, kv_len, page_mask, wave, lane);
    } else {
      if (fast) fetch_kv<D, FP8, true>(kraw, vraw, a, pt, id, hk, kb, kv_len, page_mask, lane);
      else fetch_kv<D, FP8, false>(kraw, vraw, a, pt, id, hk, kb, kv_len, page_mask, lane);
    }
  };
  auto stage_store = [&](int j) {
    if constexpr (!T::F8MMA) {
      const int buf = stage(j);
      store_kv<D, FP8, F8M>(kraw, vraw, klds[buf], vlds[buf], wave, lane);
    }
  };
  // S operand, direct-copy layout: lane (col, half) reads K rows krow_lane
  // (+ 32) at chunk 2 s + half, whose slot is (2 s + half) ^ kswz(row); the
  // swizzle key is the same for both rows
  const int kx = kswz<D>(krow_lane) ^ half;
  auto gemm_s = [&](int j) {
    if constexpr (T::F8MMA) {
      // K operand: row krow_lane (+ 32), bytes 64 c + 32 half .. + 31, i.e.
      // 16-byte chunks 4 c + 2 half (+ 1) in slots chunk ^ ((row / 2) mod 8)
      const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(f8k(j));
      i32x8 kf8[2][2];
      for (int mt = 0; mt < 2; ++mt)
        for (int cc = 0; cc < 2; ++cc) {
          const int row = krow_lane + 32 * mt;
          const int c0 = 4 * cc + 2 * half;
          const u32x4 x0 = *reinterpret_cast<const u32x4*>(kb8 + row * 128 + ((c0 ^ ((row >> 1) & 7)) << 4));
          const u32x4 x1 = *reinterpret_cast<const u32x4*>(kb8 + row * 128 + (((c0 + 1) ^ ((row >> 1) & 7)) << 4));
          kf8[mt][cc] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                              (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
      __builtin_amdgcn_sched_barrier(0);
      sacc[0] = f32x16{};
      sacc[1] = f32x16{};
      for (int cc = 0; cc < 2; ++cc)
        for (int mt = 0; mt < 2; ++mt) sacc[mt] = mfma32_fp8(kf8[mt][cc], qf8[cc], sacc[mt]);
      return;
    }
    bf16x8 kf[2][KSTEPS];
    const __bf16* kbuf = klds[stage(j)] + krow_lane * D;
    for (int s = 0; s < KSTEPS; ++s)
      for (int mt = 0; mt < 2; ++mt)
        kf[mt][s] = *reinterpret_cast<const bf16x8*>(kbuf + mt * 32 * D + ((2 * s) ^ kx) * 8);
    __builtin_amdgcn_sched_barrier(0);
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
    for (int s = 0; s < KSTEPS; ++s)
      for (int mt = 0; mt < 2; ++mt) sacc[mt] = mfma32(kf[mt][s], qf[s], sacc[mt]);
  };
  // V^T operand of tile j, read into registers before the softmax of the
  // tile so that the LDS latency passes under its exponentials
  bf16x8 vf[MD][4];
  i32x8 vf8[MD];
  auto read_v = [&](int j) {
    if constexpr (T::F8MMA) {
      // V^T operand by 8-bit transpose loads from V as stored ([key][128
      // bytes]): in each 16-lane group G, lanes 2e and 2e + 1 point at the
      // two 8-byte halves of 16 bytes of key row k0 + e, and lane jj
      // receives byte jj of those 8 rows.  With k0 = 16 r + 8 (G / 2) and the
      // 16 bytes at dim 32 md + 16 (G mod 2), lane (col, half) receives, for
      // r = 0..3, keys 16 r + 8 half + 0..7 of dim 32 md + col: the byte
      // order of P in the B operand
      typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
      const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(f8v(j)) + vt8_lane;
      for (int md = 0; md < MD; ++md) {
        v2i32 x[4];
        for (int r = 0; r < 4; ++r)
          x[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(
              (__attribute__((address_space(3))) const uint8_t*)(vb8 + vt8_md[md] + 2048 * r)));
        vf8[md] = i32x8{x[0][0], x[0][1], x[1][0], x[1][1], x[2][0], x[2][1], x[3][0], x[3][1]};
      }
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    // V^T operand by transpose loads: in each 16-lane group, lane jj points
    // at key +jj/4, dims +4 (jj%4) and receives keys +0..3 of dim +jj; two
    // loads give the 8 keys 16 ks + 8 half + 0..7 of dim md*32 + col
    const char* vbuf = reinterpret_cast<const char*>(vlds[stage(j)]) + vt_lane;
    for (int ks = 0; ks < 4; ++ks)
      for (int md = 0; md < MD; ++md) {
        typedef __attribute__((address_space(3))) v4s16 lds_v4s16;
        const char* p0 = vbuf + vt_md[md] + (16 * ks) * (2 * D);
        const v4s16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16*)(
            (__attribute__((address_space(3))) char*)p0));
        const v4s16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16*)(
            (__attribute__((address_space(3))) char*)(p0 + 4 * (2 * D))));
        vf[md][ks] = __builtin_bit_cast(bf16x8, v8s16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
    __builtin_amdgcn_sched_barrier(0);
  };
  i32x8 pf8 = {};
  // fp8 path: row sums of the rounded weights, as an MFMA of P against an
  // all-ones operand (e4m3fn 1.0 = 0x38): every element of lane (row, half)
  // is the row's sum over the tile's 64 keys, exact in fp32
  f32x16 lacc = {};
  __shared__ __attribute__((aligned(16))) int ones_lds[8];
  auto gemm_pv = [&](int j) {
    if constexpr (T::F8MMA) {
      for (int md = 0; md < MD; ++md) oacc[md] = mfma32_fp8(vf8[md], pf8, oacc[md]);
      // (the all-ones operand is read from LDS: held in registers it is
      // rebuilt with eight moves per tile, VALU slots this path is short of)
      lacc = mfma32_fp8(*reinterpret_cast<const i32x8*>(ones_lds), pf8, lacc);
      return;
    }
    for (int ks = 0; ks < 4; ++ks)
      for (int md = 0; md < MD; ++md) oacc[md] = mfma32(vf[md][ks], pb[ks], oacc[md]);
  };
  // mask (boundary tiles only), the tile's row maximum and the lazy rescale
  // of the running state; returns the exponent offset of the tile's weights
  auto softmax_max = [&](int j) {
    const int k0 = j * kBK;
    const bool need_mask = (k0 + kBK - 1 > wpos_first) || (W >= 0 && k0 < wpos_last - W) ||
                           (k0 + kBK > kv_len);
    if (need_mask) {
      const int base = k0 + 8 * half;
      const int hi = (pos < kv_len - 1 ? pos : kv_len - 1) - base;
      const int lo = (W >= 0 ? pos - W : -0x40000000) - base;
      for (int mt = 0; mt < 2; ++mt)
        for (int v = 0; v < 16; ++v) {
          const int off = mt * 32 + 16 * (v >> 3) + (v & 7);
          sacc[mt][v] = (off <= hi && off >= lo) ? sacc[mt][v] : kNegInf;
        }
    }
    float m = kNegInf;
    for (int mt = 0; mt < 2; ++mt)
      for (int v = 0; v < 16; ++v) m = fmaxf(m, sacc[mt][v]);
    m = pair_max(m);
    const float mtile = m * c;   // -inf stays -inf (c > 0)
    const bool need = mtile > m_run + kRescaleThreshold;
    if (__ballot(need) != 0ull) {
      const float m_new = need ? mtile : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      m_run = m_new;
      l_part *= alpha;
      for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
      if constexpr (T::F8MMA) lacc *= alpha;
    }
    return m_run == kNegInf ? 0.f : m_run;
  };
  // bf16 weights of the 32 keys of S block mt into the PV operand (K-steps
  // 2 mt, 2 mt + 1), their row sums added to `sum`
  auto exp_half = [&](int mt, float mb, float& sum) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    for (int sh = 0; sh < 2; ++sh) {
      bf16x2 w[4];
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][8 * sh + 2 * e], c, -mb));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][8 * sh + 2 * e + 1], c, -mb));
        w[e] = __builtin_convertvector(f32x2{p0, p1}, bf16x2);   // round to nearest even
        // row sums of the bf16 weights the PV product uses.  (The packed
        // value is fed to v_dot2 directly; reading it back out of a 4-dword
        // vector first was miscompiled - every dot2 got the same operand.)
        sum = __builtin_amdgcn_fdot2_f32_bf16(w[e], ones, sum, false);
      }
      pb[2 * mt + sh] = bf16x8{w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
    }
  };
  auto softmax = [&](int j) {
    const float mb = softmax_max(j);
    if constexpr (T::F8MMA) {
      // P as e4m3fn codes (p <= 2^8 with the lazy maximum: within range),
      // byte 16 mt + v = element v of sacc[mt].  The row sums come from the
      // PV step (an MFMA of these codes against ones), so the numerator and
      // the denominator see the same rounded weights
      for (int mt = 0; mt < 2; ++mt)
        for (int q = 0; q < 4; ++q) {
          float p[4];
          for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][4 * q + e], c, -mb));
          // (the first conversion keeps the upper half of its "old" operand,
          // which the second overwrites: any value will do, and the previous
          // tile's code, already in the register the MFMA operand needs,
          // costs no copy)
          int code = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pf8[4 * mt + q], false);
          code = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], code, true);
          pf8[4 * mt + q] = code;
        }
      return;
    }
    float sum = l_part;
    exp_half(0, mb, sum);
    exp_half(1, mb, sum);
    l_part = sum;
  };

  if (T::DMA && tile_lo <= tile_hi) {
    // four-stage ring, two tiles per barrier: each wave waits for its copies
    // of tiles j and j + 1, the barrier publishes them and frees the stages
    // of tiles j - 2 and j - 1 (read before it), which receive j + 2, j + 3
    const int lo = tile_lo, hi = tile_hi;
    auto clampt = [&](int j) { return j <= hi ? j : hi; };
    auto spec_id = [&](int i) {
      const int id = sid[i] < 0 ? 0 : sid[i];
      return id < pt.num_pages ? id : pt.num_pages - 1;
    };
    const int id0 = spec_ids ? spec_id(0) : page_of_nb(lo);
    const int id1 = spec_ids ? spec_id(1) : page_of_nb(clampt(lo + 1));
    int idn0 = spec_ids ? spec_id(2) : page_of_nb(clampt(lo + 2));
    int idn1 = spec_ids ? spec_id(3) : page_of_nb(clampt(lo + 3));
    load_q();
    stage_fetch(lo, id0);
    if (lo + 1 <= hi) stage_fetch(lo + 1, id1);
    for (int j = lo; j <= hi; j += 2) {
      wait_vmcnt<0>();
      __syncthreads();
      if (j + 2 <= hi) stage_fetch(j + 2, idn0);
      if (j + 3 <= hi) stage_fetch(j + 3, idn1);
      if (j + 4 <= hi) {
        idn0 = page_of_nb(j + 4);
        idn1 = page_of_nb(clampt(j + 5));
      }
      if (wave_tile(j)) {
        gemm_s(j);
        if (!kLateV<D>) read_v(j);
        softmax(j);
        if (kLateV<D>) read_v(j);
        gemm_pv(j);
      }
      if (j + 1 <= hi && wave_tile(j + 1)) {
        gemm_s(j + 1);
        if (!kLateV<D>) read_v(j + 1);
        softmax(j + 1);
        if (kLateV<D>) read_v(j + 1);
        gemm_pv(j + 1);
      }
    }
  } else if (T::F8MMA && tile_lo <= tile_hi) {
    // fp8 MFMA: K and V codes copied straight into a four-stage ring of
    // 16 KB stages (8 KB of K, then 8 KB of V), two tiles per barrier, as
    // for the bf16 cache: the barrier publishes tiles j, j + 1 and frees
    // the stages of j - 2, j - 1 (read before it), which receive j + 2, j + 3
    const int lo = tile_lo, hi = tile_hi;
    auto clampt = [&](int j) { return j <= hi ? j : hi; };
    const int id0 = page_of_nb(lo);
    const int id1 = page_of_nb(clampt(lo + 1));
    int idn0 = page_of_nb(clampt(lo + 2));
    int idn1 = page_of_nb(clampt(lo + 3));
    stage_fetch(lo, id0);
    if (lo + 1 <= hi) stage_fetch(lo + 1, id1);
    load_q8();   // after the first copies: its conversion waits for its loads
    if (threadIdx.x < 8) ones_lds[threadIdx.x] = 0x38383838;   // e4m3fn 1.0 x 4, published by the first barrier
    for (int j = lo; j <= hi; j += 2) {
      wait_vmcnt<0>();
      __syncthreads();
      if (j + 2 <= hi) stage_fetch(j + 2, idn0);
      if (j + 3 <= hi) stage_fetch(j + 3, idn1);
      if (j + 4 <= hi) {
        idn0 = page_of_nb(j + 4);
        idn1 = page_of_nb(clampt(j + 5));
      }
      if (wave_tile(j)) {
        gemm_s(j);
        read_v(j);
        softmax(j);
        gemm_pv(j);
      }
      if (j + 1 <= hi && wave_tile(j + 1)) {
        gemm_s(j + 1);
        read_v(j + 1);
        softmax(j + 1);
        gemm_pv(j + 1);
      }
    }
  } else if (tile_lo <= tile_hi) {
    const int lo = tile_lo, hi = tile_hi;
    stage_fetch(lo, page_of(lo));
    if (lo + 1 <= hi) id_next = page_of(lo + 1);
    stage_store(lo);
    __syncthreads();
    for (int j = lo; j <= hi; ++j) {
      const bool more = j + 1 <= hi;
      if (more) {
        stage_fetch(j + 1, id_next);
        if (j + 2 <= hi) id_next = page_of(j + 2);
      }
      if (wave_tile(j)) {
        gemm_s(j);
        read_v(j);
        softmax(j);
        gemm_pv(j);
      }
      if (more) stage_store(j + 1);
      __syncthreads();
    }
  }

  // ---- epilogue -------------------------------------------------------------
  if (!wave_active) return;
  // (the fp8 path's sums already cover both lane halves' keys)
  float l = T::F8MMA ? lacc[0] : pair_sum(l_part);
  if (!rvalid) return;
  store_row<D>(a, oacc, l, m_run, sink, h0 + hd, q0 + t0 + tok, split, half, bmm2);
}

// fp8 arithmetic (fp8_compute): rounding each softmax weight to e4m3fn
// (relative error up to 2^-4) averages out only over many keys, so an item
// runs on the fp8 MFMA only when every one of its rows sees at least
// kFp8MinKeys keys inside the item's key range (the keys common to all its
// rows, a lower bound for each); otherwise it takes the widened-bf16
// arithmetic.  The item geometry follows attend_item's decode.
__device__ __forceinline__ bool fp8_item(const AttnArgs& a, const int item) {
  const int R = a.batch * a.num_kv_heads * a.n_hg;
  const int S = a.kv_splits;
  const int split = (item / R) % S;
  const int qk = item / R / S;
  const int b = (item % R) / (a.num_kv_heads * a.n_hg);
  typedef const __attribute__((address_space(4))) int32_t cint32;
  int q1 = ((cint32*)(a.cu_q))[b + 1];
  int q0 = ((cint32*)(a.cu_q))[b];
  int kv_len = ((cint32*)(a.seq_lens))[b];
  q1 = q1 < a.num_tokens ? q1 : a.num_tokens;
  q0 = q0 < 0 ? 0 : (q0 < q1 ? q0 : q1);
  kv_len = kv_len < 0 ? 0 : kv_len;
  const int q_len = q1 - q0;
  const int qt = (q_len + a.tq - 1) / a.tq - 1 - qk;
  if (qt < 0) return false;   // nothing to do: either path returns at once
  const int t0 = qt * a.tq;
  const int ntok = q_len - t0 < a.tq ? q_len - t0 : a.tq;
  const int W = a.window_left;
  const int pos_first = kv_len - q_len + t0;
  const int pos_last = pos_first + ntok - 1;
  const int key_hi = pos_last < kv_len - 1 ? pos_last : kv_len - 1;
  const int key_lo = W >= 0 ? (pos_first - W > 0 ? pos_first - W : 0) : 0;
  int tile_lo = key_lo / kBK;
  int tile_hi = key_hi >= 0 ? key_hi / kBK : -1;
  if (S > 1 && tile_hi >= tile_lo) {
    const int n = tile_hi - tile_lo + 1;
    const int first = tile_lo;
    tile_lo = first + (split * n) / S;
    tile_hi = first + ((split + 1) * n) / S - 1;
  }
  const int chunk_lo = tile_lo * kBK;
  const int chunk_hi = tile_hi * kBK + kBK - 1 < kv_len - 1 ? tile_hi * kBK + kBK - 1 : kv_len - 1;
  const int common_lo = W >= 0 ? (pos_last - W > chunk_lo ? pos_last - W : chunk_lo) : chunk_lo;
  const int common_hi = pos_first < chunk_hi ? pos_first : chunk_hi;
  return common_hi - common_lo + 1 >= kFp8MinKeys;
}

template <int D, bool FP8, bool UPAGE, bool F8M>
__device__ __forceinline__ void run_item(const AttnArgs& a, const int item) {
  if constexpr (F8M) {
    if (fp8_item(a, item)) attend_item<D, FP8, UPAGE, true>(a, item);
    else attend_item<D, FP8, UPAGE, false>(a, item);
  } else {
    attend_item<D, FP8, UPAGE, false>(a, item);
  }
}



// One workgroup per work item, in heaviest-first order.
template <int D, bool FP8, bool UPAGE, bool F8M>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<D, FP8>, kWavesPerEU<D, FP8>)))
void paged_prefill_kernel(AttnArgs a) {
  run_item<D, FP8, UPAGE, F8M>(a, blockIdx.x);
}

// Persistent workgroups (as many as fit on the device at once) pull work
// items from counters in the caller's workspace, so a workgroup that finishes
// early takes the next heaviest item instead of idling behind the hardware's
// fixed block-to-engine dealing.  With n_queues = 8, queue x holds the items
// whose index is x mod 8 (all tiles of a fixed set of (request, kv head)
// pairs) and is served by the workgroups with blockIdx % 8 == x, which the
// dispatcher places on one XCD, so that K/V stays in one L2.  The last
// workgroup to finish returns every counter to zero for the next call.
template <int D, bool FP8, bool UPAGE, bool F8M>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<D, FP8>, kWavesPerEU<D, FP8>)))
void paged_prefill_persistent(AttnArgs a) {
  __shared__ uint32_t next_item[2];
  const uint32_t nq = static_cast<uint32_t>(a.n_queues);
  const uint32_t queue = blockIdx.x % nq;
  uint32_t* sched = a.sched;
  for (uint32_t round = 0;; ++round) {
    // two slots: a slow wave may still read the previous round's value
    if (threadIdx.x == 0) next_item[round & 1] = atomicAdd(sched + queue, 1u);
    __syncthreads();
    const uint64_t item = static_cast<uint64_t>(next_item[round & 1]) * nq + queue;
    if (item >= static_cast<uint64_t>(a.n_items)) break;
    run_item<D, FP8, UPAGE, F8M>(a, static_cast<int>(item));
  }
  if (threadIdx.x == 0 && atomicAdd(sched + kSchedDone, 1u) == gridDim.x - 1) {
    // every workgroup has made its last fetch: no counter is read again
    for (int i = 0; i <= kSchedDone; ++i) atomicExch(sched + i, 0u);
  }
}

// ---- address-unit check: paged K or V -> contiguous [tokens, H_kv, D] ------
struct GatherArgs {
  PagedPlane plane;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int64_t kv_indices_len;
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
  request_table(pt, b, g.block_tables, g.bt_row_stride, g.bt_cols, g.kv_indptr, g.kv_indices, g.kv_indices_len);
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

// ---- log-sum-exp merge of partial states ------------------------------------
// One wave per (row, head): the maximum of the parts' log-denominators (and
// the sink), the weights e^{lse_s - max}, their sum, the weighted sum of the
// parts' outputs; each lane owns D / 64 consecutive dims.
struct MergeArgs {
  const float* o_parts;     // [parts, rows, heads, D]
  const float* lse_parts;   // [parts, rows, heads]
  int32_t parts, rows, heads;
  const int32_t* row_limit; // rows at or past *row_limit are skipped, or NULL
  const float* sinks;       // [heads] or NULL
  uint16_t* out;
  int64_t o_row, o_head;
  float* lse_out;
  int64_t l_row, l_head;
  int32_t out_mx;           // 0: bf16 out; 16 or 32: MXFP4 out with that block size
  uint8_t* out_sf;
  int64_t sf_row, sf_head;
  float o_sf_scale;
};

// MXFP4 store of one merged row: lane l holds elements [l E, l E + E), so a
// block of VEC elements spans VEC / E consecutive lanes (an aligned group,
// reduced with xor shuffles).  All 64 lanes of the wave take part.
template <int D>
__device__ __forceinline__ void merge_store_mxfp4(const float* acc, float inv, const MergeArgs& m, int row, int h,
                                                  int lane) {
  constexpr int E = D / 64;
  const int L = m.out_mx / E;   // lanes per block: 8, 16 or 32
  float y[E];
  float amax = 0.f;
  for (int e = 0; e < E; ++e) {
    y[e] = (acc[e] * inv) * m.o_sf_scale;
    amax = fmaxf(amax, __builtin_fabsf(y[e]));
  }
  for (int off = 1; off < L; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const uint32_t sb = mx_scale_byte(amax);
  const float sc = mx_scale_operand(sb);
  uint8_t* orow = reinterpret_cast<uint8_t*>(m.out) + row * m.o_row + h * m.o_head;
  if constexpr (E == 2) {
    const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], sc, 0);
    orow[lane] = static_cast<uint8_t>(sb == 255u ? 0u : w);
  } else {   // the odd lane's element joins the even lane's byte
    const float next = __shfl_down(y[0], 1);
    const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], next, sc, 0);
    if ((lane & 1) == 0) orow[lane >> 1] = static_cast<uint8_t>(sb == 255u ? 0u : w);
  }
  if (lane % L == 0) m.out_sf[row * m.sf_row + h * m.sf_head + lane / L] = static_cast<uint8_t>(sb);
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs m) {
  constexpr int E = D / 64;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= static_cast<int64_t>(m.rows) * m.heads) return;
  const int row = static_cast<int>(w / m.heads);
  const int h = static_cast<int>(w % m.heads);
  if (m.row_limit != nullptr && row >= *m.row_limit) return;
  const int64_t part_stride = static_cast<int64_t>(m.rows) * m.heads;
  float mx = m.sinks ? m.sinks[h] : kNegInf;
  for (int s = 0; s < m.parts; ++s) mx = fmaxf(mx, m.lse_parts[s * part_stride + w]);
  float acc[E];
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float den = 0.f;
  if (mx > kNegInf) {
    for (int s = 0; s < m.parts; ++s) {
      const float ws = __expf(m.lse_parts[s * part_stride + w] - mx);
      den += ws;
      if (ws > 0.f) {
        const float* src = m.o_parts + (s * part_stride + w) * D + lane * E;
        for (int e = 0; e < E; ++e) acc[e] += ws * src[e];
      }
    }
    if (m.sinks) den += __expf(m.sinks[h] - mx);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  if (m.out_mx != 0) {
    merge_store_mxfp4<D>(acc, inv, m, row, h, lane);
  } else {
    uint16_t* orow = m.out + row * m.o_row + h * m.o_head + lane * E;
    if constexpr (E == 2) {
      *reinterpret_cast<uint32_t*>(orow) = pack_bf16(acc[0] * inv, acc[1] * inv);
    } else {
      *orow = static_cast<uint16_t>(pack_bf16(acc[0] * inv, 0.f) & 0xffffu);
    }
  }
  if (m.lse_out != nullptr && lane == 0)
    m.lse_out[row * m.l_row + h * m.l_head] = den > 0.f ? mx + __builtin_logf(den) : kNegInf;
}

hipError_t launch_merge(const MergeArgs& m, int head_dim, hipStream_t stream) {
  const int64_t waves = static_cast<int64_t>(m.rows) * m.heads;
  if (waves == 0) return hipSuccess;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, m);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, m);
  return hipGetLastError();
}

// Workgroups of a persistent kernel that the device holds at once (cached per
// device and kernel).
// The cache is the library's only state besides the no-allocation entry
// point's scratch address: atomic slots, so concurrent first calls on one
// device at worst run the query twice and store the same value.
template <int D, bool FP8, bool UPAGE, bool F8M>
int resident_workgroups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int known = cache[dev].load(std::memory_order_relaxed);
  if (known > 0) return known;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, paged_prefill_persistent<D, FP8, UPAGE, F8M>,
                                                   64 * kWaves, 0) != hipSuccess)
    return 0;
  const int value = cus * (per_cu > 0 ? per_cu : 1);
  cache[dev].store(value, std::memory_order_relaxed);
  return value;
}

template <int D, bool FP8, bool UPAGE, bool F8M>
hipError_t launch_variant(AttnArgs a, int items, hipStream_t stream) {
  const int resident = a.sched ? resident_workgroups<D, FP8, UPAGE, F8M>() : 0;
  if (resident <= 0) {
    hipLaunchKernelGGL((paged_prefill_kernel<D, FP8, UPAGE, F8M>), dim3(items), dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
  }
  const int R = a.batch * a.num_kv_heads * a.n_hg;
  int grid = resident < items ? resident : items;
  a.n_queues = 1;
  if (R % kSchedQueues == 0 && grid >= kSchedQueues) {
    grid -= grid % kSchedQueues;
    a.n_queues = kSchedQueues;
  }
  a.n_items = items;
  hipLaunchKernelGGL((paged_prefill_persistent<D, FP8, UPAGE, F8M>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool FP8, bool F8M = false>
hipError_t launch(const AttnArgs& a, int items, hipStream_t stream, bool upage) {
  return upage ? launch_variant<D, FP8, true, F8M>(a, items, stream)
               : launch_variant<D, FP8, false, F8M>(a, items, stream);
}

// Uniform-page staging (the 8 keys a wave copies lie in one page) needs pages
// of >= 8 tokens whose byte extent fits the 32-bit in-page offsets.
bool uniform_pages(const ppa_params* p, const CacheView& cv) {
  const int eb = p->kv_dtype == PPA_DTYPE_FP8_E4M3FN ? 1 : 2;
  auto extent = [&](int64_t head, int64_t tok) {
    return (static_cast<int64_t>(p->page_size) * tok + static_cast<int64_t>(p->num_kv_heads) * head + p->head_dim) *
           eb;
  };
  return p->page_size >= 8 && extent(cv.k_head, cv.k_tok) < (int64_t{1} << 31) &&
         extent(cv.v_head, cv.v_tok) < (int64_t{1} << 31);
}

template <int D, bool FP8, bool F8M = false>
int resident_for(bool upage) {
  return upage ? resident_workgroups<D, FP8, true, F8M>() : resident_workgroups<D, FP8, false, F8M>();
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
  if (p->page_table_form == PPA_PAGE_TABLE_CSR) {
    a.kv_indptr = p->kv_indptr;
    a.kv_indices = p->kv_indices;
    a.kv_indices_len = p->kv_indices_len;
  }
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
  a.tq = 32 * kWaves / a.gw;
  a.n_qt = (p->max_q_len + a.tq - 1) / a.tq;
  a.window_left = p->window_left;
  a.bmm1 = p->bmm1_scale;
  a.bmm2 = p->bmm2_scale;
  a.bmm1_ptr = p->bmm1_scale_ptr;
  a.bmm2_ptr = p->bmm2_scale_ptr;
  a.sinks = p->sinks;
  a.sched = static_cast<uint32_t*>(p->workspace);
  a.num_qo_heads = p->num_qo_heads;
  a.lse = p->lse;
  a.lse_tok = p->lse_strides[0];
  a.lse_head = p->lse_strides[1];
  if (p->out_dtype == PPA_DTYPE_MXFP4) {
    a.out_mx = p->o_sf_vec_size;
    a.out_sf = p->out_sf;
    a.sf_tok = p->out_sf_strides[0];
    a.sf_head = p->out_sf_strides[1];
    a.o_sf_scale = p->o_sf_scale;
  }
  a.kv_splits = p->kv_splits > 1 ? p->kv_splits : 1;
  if (a.kv_splits > 1) {
    // workspace: counters, then the partial outputs, then their log-denominators
    uint8_t* ws = static_cast<uint8_t*>(p->workspace);
    const size_t rows = static_cast<size_t>(a.kv_splits) * p->num_tokens * p->num_qo_heads;
    a.o_part = reinterpret_cast<float*>(ws + 256);
    a.lse_part = reinterpret_cast<float*>(ws + 256 + (rows * p->head_dim * sizeof(float) + 255) / 256 * 256);
  }

  const int64_t grid = static_cast<int64_t>(a.n_qt) * a.kv_splits * a.batch * a.num_kv_heads * a.n_hg;
  if (grid > 0x7fffffff) return PPA_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  const bool fp8 = p->kv_dtype == PPA_DTYPE_FP8_E4M3FN;
  const int g = static_cast<int>(grid);
  const bool upage = uniform_pages(p, cv);
  if (p->head_dim == 128)
    e = !fp8 ? launch<128, false>(a, g, s, upage)
             : (p->fp8_compute ? launch<128, true, true>(a, g, s, upage) : launch<128, true>(a, g, s, upage));
  else
    e = fp8 ? launch<64, true>(a, g, s, upage) : launch<64, false>(a, g, s, upage);
  if (e == hipSuccess && a.kv_splits > 1) {
    MergeArgs m{};
    m.o_parts = a.o_part;
    m.lse_parts = a.lse_part;
    m.parts = a.kv_splits;
    m.rows = p->num_tokens;
    m.heads = p->num_qo_heads;
    m.row_limit = p->cum_seq_lens_q + p->batch_size;
    m.sinks = p->sinks;
    m.out = static_cast<uint16_t*>(p->out);
    m.o_row = a.o_tok;
    m.o_head = a.o_head;
    m.lse_out = p->lse;
    m.l_row = p->lse_strides[0];
    m.l_head = p->lse_strides[1];
    m.out_mx = a.out_mx;
    m.out_sf = a.out_sf;
    m.sf_row = a.sf_tok;
    m.sf_head = a.sf_head;
    m.o_sf_scale = a.o_sf_scale;
    e = launch_merge(m, p->head_dim, s);
  }
  return e == hipSuccess ? PPA_OK : PPA_ERR_HIP;
}

// ---- no-allocation entry point ------------------------------------------------
// For callers that cannot allocate (graph capture, serving loops that forbid
// hipMalloc): the workspace (the persistent schedule's counters and the
// split-KV partial states) comes from a file-scope device array instead of
// the caller.  Each device holds its own copy for the life of the process;
// every call on a device shares it, so calls that overlap in time on one
// device race.
namespace ppa {
namespace {

constexpr size_t kScratchBytes = size_t{16} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The array's device address, looked up once per device with that device
// current (the host-side name is only a stand-in for the symbol).
void* scratch_address(int dev) {
  static std::mutex lock;
  static void* addr[64];
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> guard(lock);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

// The scheduler counters must start at zero: a fill kernel, not a memset
// node, so that the call stays correct under graph replay.
__global__ __launch_bounds__(64) void clear_counters(uint32_t* c) { c[threadIdx.x] = 0u; }

}  // namespace
}  // namespace ppa

extern "C" int32_t ppa_paged_prefill_attention_noalloc(const ppa_params* p, void* stream) {
  if (p == nullptr) return PPA_ERR_NULL_POINTER;
  if (p->workspace != nullptr) return PPA_ERR_WORKSPACE;   // the library's scratch takes its place
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PPA_ERR_HIP;
  void* ptr = scratch_address(dev);
  if (ptr == nullptr) return PPA_ERR_HIP;
  // the scratch stands in for the workspace: the shape check then also
  // rejects split-KV states larger than it
  ppa_params q = *p;
  q.workspace = ptr;
  q.workspace_bytes = kScratchBytes;
  char msg[8];
  const int32_t st = ppa_validate_shapes(&q, msg, sizeof msg);
  if (st != PPA_OK) return st;
  if (q.batch_size == 0 || q.max_q_len == 0 || q.num_tokens == 0) return PPA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(clear_counters, dim3(1), dim3(64), 0, s, static_cast<uint32_t*>(ptr));
  if (hipGetLastError() != hipSuccess) return PPA_ERR_HIP;
  return ppa_paged_prefill_attention(&q, stream);
}

extern "C" size_t ppa_noalloc_scratch_bytes(void) { return ppa::kScratchBytes; }

extern "C" int32_t ppa_plan_kv_splits(const ppa_params* p) {
  if (p == nullptr) return PPA_ERR_NULL_POINTER;
  ppa_params q = *p;
  q.kv_splits = 0;
  char msg[8];
  const int32_t st = ppa_validate_shapes(&q, msg, sizeof msg);
  if (st != PPA_OK) return st;
  if (q.batch_size == 0 || q.max_q_len == 0 || q.num_tokens == 0 || q.workspace == nullptr) return 1;
  // the largest split count whose partial state fits the caller's workspace
  int32_t max_splits = 1;
  for (int32_t s = 256; s > 1; --s) {
    q.kv_splits = s;
    if (ppa_workspace_bytes(&q) <= q.workspace_bytes) {
      max_splits = s;
      break;
    }
  }
  CacheView cv;
  resolve_cache(&q, &cv);
  const bool upage = uniform_pages(&q, cv);
  const bool fp8 = q.kv_dtype == PPA_DTYPE_FP8_E4M3FN;
  const int resident = q.head_dim == 128 ? (!fp8 ? resident_for<128, false>(upage)
                                                  : (q.fp8_compute ? resident_for<128, true, true>(upage)
                                                                   : resident_for<128, true>(upage)))
                                         : (fp8 ? resident_for<64, true>(upage) : resident_for<64, false>(upage));
  if (resident <= 0) return PPA_ERR_HIP;
  // work items as the launch counts them, and the key tiles of the longest
  const int group = q.num_qo_heads / q.num_kv_heads;
  const int gw = group < 16 ? group : 16;
  const int tq = 32 * kWaves / gw;
  const int64_t items = static_cast<int64_t>((q.max_q_len + tq - 1) / tq) * q.batch_size * q.num_kv_heads *
                        ((group + gw - 1) / gw);
  int64_t keys = q.max_kv_len;
  if (q.window_left >= 0) {
    const int64_t span = static_cast<int64_t>(q.window_left) + (q.max_q_len < tq ? q.max_q_len : tq);
    keys = span < keys ? span : keys;
  }
  return ppa_plan_kv_splits_model(items, resident, (keys + kBK - 1) / kBK, max_splits);
}

// ---- KV append: new tokens' K and V into their page slots -------------------
namespace ppa {
namespace {

struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t kn_tok, kn_head, vn_tok, vn_head;
  const int64_t* slots;
  PagedPlane k, v;
  int32_t num_new, heads, chunks, page_shift, num_pages;
  float k_scale, v_scale;
  const float* k_scale_ptr;
  const float* v_scale_ptr;
};

// x / scale -> e4m3fn code: saturated to +-448 first (NaN kept), then the
// hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  auto sat = [](float x) { return fabsf(x) > 448.f ? copysignf(448.f, x) : x; };
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), r, true);
  return static_cast<uint32_t>(r);
}

// One thread per 8 consecutive elements of one (token, kv head, K or V) row.
template <bool FP8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.num_new) * a.heads * 2 * a.chunks;
  if (u >= total) return;
  const int c = static_cast<int>(u % a.chunks);
  int64_t r = u / a.chunks;
  const int plane = static_cast<int>(r & 1);
  r >>= 1;
  const int h = static_cast<int>(r % a.heads);
  const int64_t i = r / a.heads;
  const int64_t loc = a.slots[i];
  if (loc < 0) return;
  const int64_t page = loc >> a.page_shift;
  if (page >= a.num_pages) return;
  const int64_t slot = loc & ((int64_t{1} << a.page_shift) - 1);
  const uint16_t* src = plane ? a.v_new + i * a.vn_tok + h * a.vn_head : a.k_new + i * a.kn_tok + h * a.kn_head;
  const u32x4 x = *reinterpret_cast<const u32x4*>(src + c * 8);
  const PagedPlane& pl = plane ? a.v : a.k;
  const int64_t off = page * pl.page_stride + h * pl.head_stride + slot * pl.tok_stride + c * 8;
  uint8_t* base = const_cast<uint8_t*>(pl.base);
  if constexpr (!FP8) {
    *reinterpret_cast<u32x4*>(base + off * 2) = x;
  } else {
    const float s = plane ? (a.v_scale_ptr ? *a.v_scale_ptr : a.v_scale) : (a.k_scale_ptr ? *a.k_scale_ptr : a.k_scale);
    float f[8];
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __builtin_bit_cast(float, x[e] << 16) / s;
      f[2 * e + 1] = __builtin_bit_cast(float, x[e] & 0xffff0000u) / s;
    }
    *reinterpret_cast<u32x2*>(base + off) = u32x2{fp8x4(f[0], f[1], f[2], f[3]), fp8x4(f[4], f[5], f[6], f[7])};
  }
}

}  // namespace
}  // namespace ppa

extern "C" int32_t ppa_append_paged_kv(const ppa_params* p, const ppa_append_params* ap, void* stream) {
  char msg[8];
  const int32_t st = ppa_validate_append(p, ap, msg, sizeof msg);
  if (st != PPA_OK) return st;
  if (ap->num_new == 0) return PPA_OK;
  CacheView cv;
  resolve_cache(p, &cv);
  AppendArgs a{};
  a.k_new = static_cast<const uint16_t*>(ap->k_new);
  a.v_new = static_cast<const uint16_t*>(ap->v_new);
  a.kn_tok = ap->k_new_strides[0];
  a.kn_head = ap->k_new_strides[1];
  a.vn_tok = ap->v_new_strides[0];
  a.vn_head = ap->v_new_strides[1];
  a.slots = ap->slot_mapping;
  a.k = PagedPlane{static_cast<const uint8_t*>(cv.k_base), cv.k_page, cv.k_head, cv.k_tok};
  a.v = PagedPlane{static_cast<const uint8_t*>(cv.v_base), cv.v_page, cv.v_head, cv.v_tok};
  a.num_new = ap->num_new;
  a.heads = p->num_kv_heads;
  a.chunks = p->head_dim / 8;
  a.page_shift = log2_exact(p->page_size);
  a.num_pages = p->num_pages;
  a.k_scale = ap->k_scale;
  a.v_scale = ap->v_scale;
  a.k_scale_ptr = ap->k_scale_ptr;
  a.v_scale_ptr = ap->v_scale_ptr;
  const int64_t total = static_cast<int64_t>(a.num_new) * a.heads * 2 * a.chunks;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffff) return PPA_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->kv_dtype == PPA_DTYPE_FP8_E4M3FN)
    hipLaunchKernelGGL(append_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? PPA_OK : PPA_ERR_HIP;
}

extern "C" int32_t ppa_merge_attention_states(const ppa_merge_params* mp, void* stream) {
  if (mp == nullptr) return PPA_ERR_NULL_POINTER;
  if (mp->abi_version != PPA_ABI_VERSION || mp->struct_size != sizeof(ppa_merge_params)) return PPA_ERR_ABI;
  if (mp->num_parts < 1 || mp->num_rows < 0 || mp->num_heads < 1) return PPA_ERR_SHAPE;
  if (mp->head_dim != 64 && mp->head_dim != 128) return PPA_ERR_HEAD_DIM;
  const bool mx = mp->out_dtype == PPA_DTYPE_MXFP4;
  if (mp->out_dtype != PPA_DTYPE_BF16 && !mx) return PPA_ERR_DTYPE;
  if (mx && ((mp->o_sf_vec_size != 16 && mp->o_sf_vec_size != 32) ||
             !(mp->o_sf_scale > 0.f && mp->o_sf_scale <= 3.402823466e38f)))
    return PPA_ERR_SHAPE;
  if (mp->num_rows == 0) return PPA_OK;
  if (mp->o_parts == nullptr || mp->lse_parts == nullptr || mp->out == nullptr) return PPA_ERR_NULL_POINTER;
  if (mx && mp->out_sf == nullptr) return PPA_ERR_NULL_POINTER;
  if (mx && (mp->out_sf_strides[0] < 0 || mp->out_sf_strides[1] < 0)) return PPA_ERR_STRIDE;
  if (mp->out_strides[2] != 1 || mp->out_strides[0] < 0 || mp->out_strides[1] < 0 ||
      (mp->out_strides[0] & 1) != 0 || (mp->out_strides[1] & 1) != 0)
    return PPA_ERR_STRIDE;
  if (mp->lse_out != nullptr && (mp->lse_out_strides[0] < 0 || mp->lse_out_strides[1] < 0)) return PPA_ERR_STRIDE;
  auto mis = [](const void* x, uintptr_t a) { return (reinterpret_cast<uintptr_t>(x) & (a - 1)) != 0; };
  if (mis(mp->o_parts, 4) || mis(mp->lse_parts, 4) || mis(mp->out, 4) || mis(mp->sinks, 4) || mis(mp->lse_out, 4))
    return PPA_ERR_ALIGNMENT;
  MergeArgs m{};
  m.o_parts = mp->o_parts;
  m.lse_parts = mp->lse_parts;
  m.parts = mp->num_parts;
  m.rows = mp->num_rows;
  m.heads = mp->num_heads;
  m.sinks = mp->sinks;
  m.out = static_cast<uint16_t*>(mp->out);
  m.o_row = mp->out_strides[0];
  m.o_head = mp->out_strides[1];
  m.lse_out = mp->lse_out;
  m.l_row = mp->lse_out_strides[0];
  m.l_head = mp->lse_out_strides[1];
  if (mx) {
    m.out_mx = mp->o_sf_vec_size;
    m.out_sf = mp->out_sf;
    m.sf_row = mp->out_sf_strides[0];
    m.sf_head = mp->out_sf_strides[1];
    m.o_sf_scale = mp->o_sf_scale;
  }
  return launch_merge(m, mp->head_dim, static_cast<hipStream_t>(stream)) == hipSuccess ? PPA_OK : PPA_ERR_HIP;
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
  if (p->page_table_form == PPA_PAGE_TABLE_CSR) {
    g.kv_indptr = p->kv_indptr;
    g.kv_indices = p->kv_indices;
    g.kv_indices_len = p->kv_indices_len;
  }
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
