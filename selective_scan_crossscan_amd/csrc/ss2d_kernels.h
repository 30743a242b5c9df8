// SS2D forward kernels for gfx950 (CDNA4, wave64): the kernel templates.
// Included by the compilation units that instantiate them (one per storage
// type and steps per lane, so they build in parallel) and by ss2d_plan.hip.
//
// What is computed (page [SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现"):
//   §3.1/§4  four scan sequences of the H x W map: row-major, column-major and
//            both reversed;
//   §3.2     per channel c = k*D + d and state n:
//              delta_l = softplus(dt_l + dt_bias[c]),  A = -exp(A_log[c, n]),
//              h_l = exp(delta_l * A) * h_{l-1} + delta_l * Bs[n, l] * u_l,  h_{-1} = 0,
//              out_l = sum_n Cs[n, l] * h_l + Ds[c] * u_l,   u_l = x[pixel visited at l];
//   §3.3     y[p] = sum over the four directions of out at the step visiting p.
//
// How it runs.  One workgroup owns one batch b and a block of CH channels and
// does the four directions one after the other, in the order 1, 3, 0, 2.
//   * A sequence (b, k, d) is cut into chunks of G*T steps; a group of G lanes
//     owns one channel's chunk, T consecutive steps per lane.
//   * Per state n a lane turns its T steps into decays a_i = 2^(delta_i*A*log2 e)
//     and inputs b_i = delta_i u_i B_i, folds them into one affine map
//     h -> A_lane h + B_lane, the group combines the maps with an inclusive
//     prefix scan done with fused DPP multiply/FMA (row_shr 1/2/4/8, row_bcast
//     15/31), the state carried from the previous chunk enters through the
//     exclusive prefix, and the lane replays its T steps from its exact incoming
//     state, adding C_i h_i to its outputs.  The combine (A1,B1) then (A2,B2) =
//     (A2 A1, A2 B1 + B2) is associative, so this equals the sequential loop up
//     to rounding order.
//   * Bs/Cs of a chunk are shared by every channel of the workgroup.  They are
//     copied global -> LDS by DMA (the vector load's LDS form: no registers, no
//     wait) in groups of NG states, one group ahead into a two-buffer ring, and
//     dt one chunk ahead; the workgroup synchronises once per group.  The LDS
//     rows are XOR-swizzled so lanes read their steps with conflict-free
//     16-byte loads.
//   * Merge: directions 1 and 3 accumulate into a column-major fp32 plane and
//     direction 0 into a row-major one (y itself for fp32 output), so every
//     access is contiguous along the lane's steps.  Direction 2, last, reads
//     both and writes y = (y0 + y2) + (y1 + y3), rounded once: the order of
//     additions is fixed, so results are deterministic, with no atomics and no
//     separate merge pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "ss2d_internal.h"

namespace ss2d {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxN = 16;
constexpr int kWaves = 4;
// Largest rank of the low-rank step input the scan expands itself (see Params::R).
constexpr int kMaxLowRank = 8;

// LDS floats per lane segment for T steps: multiples of 4 get a stride whose
// 16-byte slot count is odd, so 16-byte reads by consecutive lanes do not
// collide in the LDS banks.
template <int T>
constexpr int seg_stride() {
  return T == 16 ? 20 : T == 12 ? 20 : T == 8 ? 12 : T;
}

// ------------------------------------------------------------------ storage
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// Two floats to two packed bf16, rounded to nearest even by the hardware's packed
// conversion (one instruction on gfx950).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const f32x2_v f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
}

template <typename S>
struct Io;

template <>
struct Io<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ float4 ld4(const float* p, int64_t i) {  // i % 4 == 0
    return *reinterpret_cast<const float4*>(p + i);
  }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
  static __device__ __forceinline__ void st4(float* p, int64_t i, float4 v) {  // i % 4 == 0
    *reinterpret_cast<float4*>(p + i) = v;
  }
};

template <>
struct Io<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ float4 ld4(const uint16_t* p, int64_t i) {
    const uint2 v = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xffffu),
                       bf16_to_f32(v.y >> 16));
  }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_rne(v); }
  static __device__ __forceinline__ void st4(uint16_t* p, int64_t i, float4 v) {  // i % 4 == 0
    *reinterpret_cast<uint2*>(p + i) = make_uint2(bf16x2_rne(v.x, v.y), bf16x2_rne(v.z, v.w));
  }
};

// Four values at positions i..i+3 of a row of length L, zero past the end.
template <typename S>
__device__ __forceinline__ float4 ld4_guarded(const S* row, int i, int L, bool vec) {
  if (vec && i + 3 < L) return Io<S>::ld4(row, i);
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i + 0 < L) r.x = Io<S>::ld(row, i + 0);
  if (i + 1 < L) r.y = Io<S>::ld(row, i + 1);
  if (i + 2 < L) r.z = Io<S>::ld(row, i + 2);
  if (i + 3 < L) r.w = Io<S>::ld(row, i + 3);
  return r;
}

// ------------------------------------------------------------------ math
// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|).  With t = e^-|v| in
// (0, 1], u = 1 + t rounds; c = t - (u - 1) is that rounding error exactly
// (Fast2Sum, 1 >= t), and log1p(t) = log(u) + log(1 + c/u) ~ log(u) + c.
__device__ __forceinline__ float softplus_f32(float v) {
  const float t = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
  const float u = 1.0f + t;
  const float c = t - (u - 1.0f);
  const float l = fmaf(__builtin_amdgcn_logf(u), kLn2, c);
  return fmaxf(v, 0.0f) + l;
}

// The inclusive prefix combine of affine maps h -> A h + B inside groups of G
// lanes (G = 16, 32 or 64): one level per power of two, each a fused
//   B += dpp(B) * A   (v_fmac_f32_dpp),   A = dpp(A) * A   (v_mul_f32_dpp),
// whose DPP source lane is earlier in the sequence.  Lanes whose source is out of
// range (or whose row is masked off) are not written: the identity map.
// All levels are one asm block, so the compiler adds no wait states of its own
// between them.  A DPP read needs two wait states after a VALU write of its
// source: s_nop 1 before the first level (A and B were just computed); after that
// one s_nop 0 per level suffices, since each fmac reads the B written two
// instructions earlier and each mul the A written two instructions earlier.
#define SS2D_SCAN_STEP(DPP) \
  "v_fmac_f32_dpp %1, %1, %0 " DPP " bank_mask:0xf\n\tv_mul_f32_dpp %0, %0, %0 " DPP " bank_mask:0xf\n\t"
#define SS2D_SCAN_NEXT(DPP) "s_nop 0\n\t" SS2D_SCAN_STEP(DPP)

template <int G>
__device__ __forceinline__ void scan_inclusive(float& A, float& B) {
  if constexpr (G == 16) {
    asm volatile("s_nop 1\n\t" SS2D_SCAN_STEP("row_shr:1 row_mask:0xf") SS2D_SCAN_NEXT("row_shr:2 row_mask:0xf")
                     SS2D_SCAN_NEXT("row_shr:4 row_mask:0xf") SS2D_SCAN_NEXT("row_shr:8 row_mask:0xf")
                 : "+v"(A), "+v"(B));
  } else if constexpr (G == 32) {
    asm volatile("s_nop 1\n\t" SS2D_SCAN_STEP("row_shr:1 row_mask:0xf") SS2D_SCAN_NEXT("row_shr:2 row_mask:0xf")
                     SS2D_SCAN_NEXT("row_shr:4 row_mask:0xf") SS2D_SCAN_NEXT("row_shr:8 row_mask:0xf")
                         SS2D_SCAN_NEXT("row_bcast:15 row_mask:0xa")
                 : "+v"(A), "+v"(B));
  } else {
    static_assert(G == 64, "lanes per sequence must be 16, 32 or 64");
    asm volatile("s_nop 1\n\t" SS2D_SCAN_STEP("row_shr:1 row_mask:0xf") SS2D_SCAN_NEXT("row_shr:2 row_mask:0xf")
                     SS2D_SCAN_NEXT("row_shr:4 row_mask:0xf") SS2D_SCAN_NEXT("row_shr:8 row_mask:0xf")
                         SS2D_SCAN_NEXT("row_bcast:15 row_mask:0xa") SS2D_SCAN_NEXT("row_bcast:31 row_mask:0xc")
                 : "+v"(A), "+v"(B));
  }
}

// State entering this lane's steps: the previous lane's inclusive map applied
// to the group's carried state, h = A_prev * carry + B_prev; the group's first
// lane takes the carry itself.  One asm block: the add reads B (last written by
// the scan, well before) through DPP and the product through its plain operand.
// With 16 lanes a group is one DPP row, and row_shr:1 does not write a row's
// first lane (its source lies outside the row), so that lane keeps the carry
// with no select.
template <int G>
__device__ __forceinline__ float incoming_state(float A, float B, float carry, int seg) {
  float h = carry;
  if constexpr (G == 16) {
    asm volatile(
        "s_nop 1\n\t"
        "v_mul_f32_dpp %0, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_add_f32_dpp %0, %2, %0 row_shr:1 row_mask:0xf bank_mask:0xf"
        : "+v"(h)
        : "v"(A), "v"(B));
    return h;
  } else {
    asm volatile(
        "s_nop 1\n\t"
        "v_mul_f32_dpp %0, %1, %0 wave_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_add_f32_dpp %0, %2, %0 wave_shr:1 row_mask:0xf bank_mask:0xf"
        : "+v"(h)
        : "v"(A), "v"(B));
  }
  return seg == 0 ? carry : h;
}

// Wave priority 0..3 (the instruction takes an immediate).
__device__ __forceinline__ void set_priority(int level) {
  switch (level) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

// ------------------------------------------------------------------ kernel state
struct Params {
  const void* x;
  const void* dt;
  const float* A_log;
  const float* dt_bias;
  const void* Bs;
  const void* Cs;
  const float* Ds;
  void* y;
  float* prow;  // directions 0 and 2, row-major fp32: y itself (fp32 output) or a temporary (bf16)
  float* pcol;  // directions 1 and 3, column-major fp32 temporary
  // Long sequences are cut into nseg segments of seg_chunks full chunks each (the
  // last takes the rest).  carries[((b*4 + k)*D + d)*nseg + s][n] = {A, B}: the
  // segment's affine map h -> A h + B, from a carry pass over segments 0..nseg-2.
  float* carries;
  // Transposed copies (null: not used): x as [W][H] per plane, read by the column
  // walks as contiguous rows; the column plane as [H][W], read by direction 2.
  const void* xT;
  const float* pcolT;
  int seg_chunks, nseg;
  int kdir;  // the one direction of a segment output launch
  // Directions: K = 4 (the cross scan: 1, 3, 0, 2) or K = 2 (the row walk and its
  // reverse only: 0, 2, whose per-direction tensors are slots 0 and 1).
  int K;
  // State block: this launch runs states n0 .. n0+N-1 of Nt (the row stride of
  // A_log and the (batch, direction) stride of Bs/Cs are Nt).  skip: add Ds*u
  // (the first block only); acc: the row plane already holds earlier blocks'
  // sums, so direction 0 adds to it; final_out: the last block, which writes y
  // in the storage type (earlier bf16 blocks leave their fp32 sums in the row
  // plane).
  int Nt, n0, skip, acc, final_out;
  // Low-rank step input (R > 0): dt points to the R rows dts (B, K, R, L) in scan
  // order, and the scan forms dt[b,k,d,l] = sum_r wdt[k,d,r] * dts[b,k,r,l] itself
  // ([SS2D] §3.2: dt_projs applied to the low-rank rows) instead of reading a
  // (B, K, D, L) dt.  R <= kMaxLowRank and R <= channels per workgroup.
  int R;
  const float* wdt;  // (K, D, R)
  // Wave priority rotation (0: off): the launch fits one round of prio_levels
  // resident workgroups on each of prio_ncu CUs.
  int prio_ncu, prio_levels;
  int B, D, H, W, N, L;
};

// What one launch does.
enum Mode : int {
  kFused = 0,     // whole sequences, all four directions, merge included
  kCarry = 1,     // segment maps of every direction (no outputs)
  kSegment = 2,   // one direction's outputs per segment, entering with the carried state
};

// Compile-time shape of one kernel variant: G lanes per sequence chunk, T steps
// per lane in full chunks, NG states per Bs/Cs staging group.
template <int G, int T, int NG>
struct Cfg {
  static constexpr int kChans = kWaves * (64 / G);  // channels per workgroup
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kSS = seg_stride<T>();
  static constexpr int kArr = G * kSS;               // LDS floats of one register-staged (state, B or C)
  static constexpr int kBuf = NG * 2 * kArr;         // one register-staged buffer
};

// LDS of a workgroup (bytes), for storage type S.  Separate arrays, so the
// compiler can tell a DMA copy into one from reads of another and does not
// make those reads wait for the copy.
//   ring0, ring1  one Bs/Cs group each, copied in by DMA: [B|C][NG][G*T] of S;
//                 ring0 also holds the register-staged group of a remainder
//                 chunk and the tile of the final transpose
//   dtb           dt of the next full chunk, copied in by DMA: [kChans][G*T] of S
//   par           A*log2(e) and the carried state per (channel, state), then
//                 dt_bias and Ds per channel
template <typename S, int G, int T, int NG, bool VEC>
struct Layout {
  using C = Cfg<G, T, NG>;
  static constexpr int kGT = G * T;
  static constexpr int kGroupBytes = NG * 2 * kGT * (int)sizeof(S);
  // one register-staged group: remainder chunks (at most 8 steps per lane), or
  // every chunk when rows are not aligned for the DMA copy
  static constexpr int kStagedBytes = NG * 2 * G * seg_stride<VEC ? 8 : T>() * 4;
  static constexpr int kTileBytes = 32 * 33 * 4;
  static constexpr int kRing0Bytes = kGroupBytes > kStagedBytes ? (kGroupBytes > kTileBytes ? kGroupBytes : kTileBytes)
                                                                : (kStagedBytes > kTileBytes ? kStagedBytes : kTileBytes);
  static constexpr int kDtBytes = C::kChans * kGT * (int)sizeof(S);
  static constexpr int kParFloats = 3 * C::kChans * kMaxN + 2 * C::kChans + C::kChans * kMaxLowRank;
  // bf16 storage: the group's Bs/Cs rows widened to fp32 (widen_rows)
  static constexpr int kWideBytes = sizeof(S) == 2 ? NG * 2 * kGT * 4 : 0;
  static constexpr int kBytes = kRing0Bytes + kGroupBytes + kDtBytes + 4 * kParFloats + kWideBytes;
};

// ------------------------------------------------------------------ DMA staging
// Rows of G*T elements are copied global -> LDS with the DMA form of the vector
// load (each lane's element goes straight to LDS; no registers, no wait until
// the data is needed).  One wave-wide copy writes 64 consecutive granules, so
// bank-conflict avoidance cannot use padding; instead the 16-byte slots of a
// lane segment (T elements) are XOR-swizzled: slot q of segment s is stored at
// s*SP + (q ^ ((s / (16/SP)) & (SP-1))), SP = slots per segment.  Sixteen
// consecutive segments read at the same q then land on sixteen different
// 16-byte bank groups.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <typename S, int T>
struct Swz {
  static constexpr int kEps = 16 / (int)sizeof(S);  // elements per 16-byte slot
  static constexpr int kSP = T / kEps;              // slots per segment
  static constexpr int kSpan = 16 / kSP;            // segments per sweep of the 16 bank groups
  static_assert(kSP >= 1 && (kSP & (kSP - 1)) == 0, "segment must be a power-of-two number of slots");
  static __device__ __forceinline__ int swz(int seg) { return (seg / kSpan) & (kSP - 1); }
};

// Wait until this wave's outstanding vector-memory operations (DMA copies
// included) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// A row of a staged tensor: its buffer resource and the byte offset of the row
// start in it.  Buffer resources keep the per-copy address arithmetic to a
// 32-bit scalar offset (the lane part is one fixed register).
struct RowRef {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off;
};

// Word 3 of a raw (unformatted, unswizzled) buffer resource on the gfx9 family.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

// A copy of R rows of G*T elements into LDS, swizzled, split over the
// workgroup: each lane moves GB bytes per copy instruction (16: fp32 rows
// 16-byte aligned, else 4), a wave 64*GB bytes, which never straddle two rows.
// The swizzle repeats every kPeriod = 16*SP slots, and a wave's copies all
// start at the same offset inside that period, so a lane's byte offset is a
// per-lane constant plus a wave-uniform part.
template <typename S, int G, int T, int R, int GB>
struct DmaPlan {
  using Z = Swz<S, T>;
  static constexpr int kRowBytes = G * T * (int)sizeof(S);
  static constexpr int kNth = kWaves * 64;
  static constexpr int kGranules = R * kRowBytes / GB;
  static constexpr int kIters = kGranules / kNth;
  static constexpr int kPeriod = 16 * Z::kSP * 16;  // bytes
  static_assert(kGranules % kNth == 0, "DMA copy must split evenly over the workgroup");
  static_assert(kRowBytes % (64 * GB) == 0, "a wave's copy must stay inside one row");
  static_assert((kNth * GB) % kPeriod == 0 && kRowBytes % kPeriod == 0,
                "a wave's copies must sit at one offset inside the swizzle period");
  // Copies are dealt to waves in contiguous runs (a wave's rows then come from one
  // tensor, so its copies share the resource and step the offset) when a wave
  // copy spans whole swizzle periods; otherwise interleaved, every wave at one
  // offset inside the period.
  static constexpr bool kContig = (64 * GB) % kPeriod == 0;
  static __device__ __forceinline__ uint32_t copy_byte(uint32_t w, int it) {
    return kContig ? (w * (uint32_t)kIters + (uint32_t)it) * 64u * GB : ((uint32_t)it * kNth + w * 64u) * GB;
  }
  int wave;
  uint32_t lane_byte;

  __device__ __forceinline__ explicit DmaPlan(int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rb = (wave * 64 * GB) % kPeriod + (tid & 63) * GB;  // lane's byte inside its period
    const int slot = rb >> 4;
    const int seg = slot / Z::kSP;
    const int q = (slot % Z::kSP) ^ Z::swz(seg);
    lane_byte = (seg * T + q * Z::kEps) * (int)sizeof(S) + (rb & 15);
  }

  // Every thread of the workgroup calls it; row(r) gives row r's RowRef, and the
  // copy starts c0 elements into each row.  Only the first lim elements of a row
  // exist (lim < G*T for a partial last chunk): lanes past them copy the last
  // existing granule instead, so nothing outside the tensor is read.
  template <typename RowFn>
  __device__ __forceinline__ void copy(char* dst, RowFn row, int c0, int lim = G * T) const {
    if (lim < G * T) {
      copy_partial(dst, row, c0, lim);
      return;
    }
    // Opaque copies of the plan: the offsets are cheap to form here, and hoisted
    // out of the main loop they would hold registers through it.
    uint32_t w = (uint32_t)wave;
    uint32_t lb = lane_byte;
    asm volatile("" : "+s"(w), "+v"(lb));
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const uint32_t wbyte = copy_byte(w, it);  // first byte of this wave's copy
      const uint32_t rowb = wbyte % (uint32_t)kRowBytes;
      const RowRef rr = row((int)(wbyte / (uint32_t)kRowBytes));
      const uint32_t soff = rr.off + (uint32_t)c0 * (uint32_t)sizeof(S) + (rowb - rowb % (uint32_t)kPeriod);
      if constexpr (GB == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr.r, (lds_void_t*)(dst + wbyte), 16, lb, soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr.r, (lds_void_t*)(dst + wbyte), 4, lb, soff, 0, 0);
    }
  }

  // The partial-chunk form: the whole in-row offset goes into the lane offset,
  // clamped to the last granule that exists (lim is a multiple of 4 elements, a
  // granule is at most 4, so that granule lies wholly inside the row).
  template <typename RowFn>
  __device__ __forceinline__ void copy_partial(char* dst, RowFn row, int c0, int lim) const {
    constexpr uint32_t kEg = GB / (int)sizeof(S);  // elements per granule
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const uint32_t wbyte = copy_byte((uint32_t)wave, it);
      const uint32_t rowb = wbyte % (uint32_t)kRowBytes;
      const RowRef rr = row((int)(wbyte / (uint32_t)kRowBytes));
      const uint32_t e = (rowb - rowb % (uint32_t)kPeriod) / (uint32_t)sizeof(S) + lane_byte / (uint32_t)sizeof(S);
      const uint32_t ec = e < (uint32_t)lim ? e : (uint32_t)lim - kEg;
      const uint32_t voff = ec * (uint32_t)sizeof(S);
      const uint32_t soff = rr.off + (uint32_t)c0 * (uint32_t)sizeof(S);
      if constexpr (GB == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr.r, (lds_void_t*)(dst + wbyte), 16, voff, soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr.r, (lds_void_t*)(dst + wbyte), 4, voff, soff, 0, 0);
    }
  }
};

// A copy of R rows of G*TT elements (a remainder chunk: TT < T) into LDS in
// plain row-major order, row r at r * kRowBytes, segment s of a row at s * TT
// elements.  Each wave-wide copy stays inside the rows of one tensor (row(r)
// gives the same resource for all rows it covers: blocks of 16 rows are one
// tensor), possibly spanning several short rows.  Steps past a row's end read
// the next row or, past the tensor, the zeros a buffer load returns out of
// range; the remainder step gives them delta = 0.
template <typename S, int G, int TT, int R, int GB>
struct PlainCopy {
  static constexpr int kRowBytes = G * TT * (int)sizeof(S);
  static constexpr int kWaveBytes = 64 * GB;
  static constexpr int kCopies = R * kRowBytes / kWaveBytes;
  static_assert((R * kRowBytes) % kWaveBytes == 0, "rows must fill whole wave-wide copies");
  static_assert(kRowBytes % kWaveBytes == 0 || kWaveBytes % kRowBytes == 0, "row and copy sizes must nest");

  template <typename RowFn>
  __device__ __forceinline__ static void copy(char* dst, RowFn row, int c0, int tid) {
    // Opaque, so the address arithmetic stays here instead of being hoisted out of
    // the chunk loop into registers held through it.
    uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t lb = (uint32_t)(tid & 63) * GB;
    asm volatile("" : "+s"(wave), "+v"(lb), "+s"(c0));
#pragma unroll
    for (int j0 = 0; j0 < kCopies; j0 += kWaves) {
      const int j = j0 + (int)wave;
      if (j < kCopies) {
        const uint32_t wbyte = (uint32_t)j * kWaveBytes;
        const uint32_t byte = wbyte + lb;
        const RowRef head = row((int)(wbyte / kRowBytes));  // resource of the copy
        const RowRef mine = row((int)(byte / kRowBytes));   // this lane's row
        const uint32_t voff = mine.off + (uint32_t)c0 * (uint32_t)sizeof(S) + byte % kRowBytes;
        if constexpr (GB == 16)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(head.r, (lds_void_t*)(dst + wbyte), 16, voff, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(head.r, (lds_void_t*)(dst + wbyte), 4, voff, 0, 0, 0);
      }
    }
  }
};

// The TT elements of segment `seg` of a plain row, as floats.
template <typename S, int TT>
__device__ __forceinline__ void read_plain(const char* row, int seg, float (&v)[TT]) {
  const char* p = row + seg * TT * (int)sizeof(S);
  if constexpr (sizeof(S) == 4) {
    if constexpr (TT == 1) {
      v[0] = *reinterpret_cast<const float*>(p);
    } else if constexpr (TT == 2) {
      const float2 q = *reinterpret_cast<const float2*>(p);
      v[0] = q.x; v[1] = q.y;
    } else {
#pragma unroll
      for (int i = 0; i < TT; i += 4) {
        const float4 q = *reinterpret_cast<const float4*>(p + i * 4);
        v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
      }
    }
  } else {
    if constexpr (TT == 1) {
      v[0] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
    } else {
#pragma unroll
      for (int i = 0; i < TT; i += 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p + i * 2);
        v[i] = __uint_as_float(w << 16);
        v[i + 1] = __uint_as_float(w & 0xffff0000u);
      }
    }
  }
}

// The T elements of segment `seg` of a swizzled row, as floats.
template <typename S, int T>
__device__ __forceinline__ void read_seg(const char* row, int seg, float (&v)[T]) {
  using Z = Swz<S, T>;
  const int sw = Z::swz(seg);
#pragma unroll
  for (int q = 0; q < Z::kSP; ++q) {
    const uint4 r = *reinterpret_cast<const uint4*>(row + (seg * Z::kSP + (q ^ sw)) * 16);
    if constexpr (sizeof(S) == 4) {
      v[q * 4 + 0] = __uint_as_float(r.x);
      v[q * 4 + 1] = __uint_as_float(r.y);
      v[q * 4 + 2] = __uint_as_float(r.z);
      v[q * 4 + 3] = __uint_as_float(r.w);
    } else {
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[q * 8 + 2 * j] = __uint_as_float(w[j] << 16);
        v[q * 8 + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    }
  }
}

// The 2*NG Bs/Cs rows of a group, copied into the ring as bf16, rewritten once
// per workgroup as fp32 rows with the fp32 swizzle.  The lanes of every channel
// then read them as fp32 (read_seg<float, T>) instead of each lane unpacking
// every bf16 value it reads, once per channel.  Element 2j of a 32-bit word is
// its low half (little-endian).  NTH threads take 16-byte slots of the bf16
// rows in turn; each slot (8 steps of one lane segment) becomes two fp32 slots.
template <int T, int ROWS, int GT, int NTH>
__device__ __forceinline__ void widen_rows(const char* src, char* dst, int tid) {
  using Zb = Swz<uint16_t, T>;
  using Zf = Swz<float, T>;
  constexpr int kRowSlots = GT * 2 / 16;  // 16-byte slots of a bf16 row
  constexpr int kSlots = ROWS * kRowSlots;
  static_assert(kSlots % NTH == 0, "the slots of a group must divide among the threads");
#pragma unroll 1
  for (int k = 0; k < kSlots / NTH; ++k) {
    const int j = tid + k * NTH;
    const int row = j / kRowSlots, js = j - row * kRowSlots;
    const int sg = js / Zb::kSP;
    const int q = (js - sg * Zb::kSP) ^ Zb::swz(sg);  // holds steps 8q .. 8q+7 of segment sg
    const uint4 w = *reinterpret_cast<const uint4*>(src + row * GT * 2 + js * 16);
    const float4 lo = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    const float4 hi = make_float4(__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xffff0000u),
                                  __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xffff0000u));
    char* drow = dst + row * GT * 4;
    const int sw = Zf::swz(sg);
    *reinterpret_cast<float4*>(drow + (sg * Zf::kSP + ((2 * q) ^ sw)) * 16) = lo;
    *reinterpret_cast<float4*>(drow + (sg * Zf::kSP + ((2 * q + 1) ^ sw)) * 16) = hi;
  }
}

// Walk index (row-major index for row walks, w*H+h for column walks) of step l.
__device__ __forceinline__ int walk_index(bool rev, int l, int L) { return rev ? (L - 1 - l) : l; }

// dt and u for T consecutive steps from l0.  FULL: all steps exist (no bounds
// checks).  VEC: rows are aligned for 16-byte (fp32) / 8-byte (bf16) loads.
template <typename S, int T, bool VEC, bool FULL>
__device__ __forceinline__ void load_x(const S* xrow, bool rev, bool col, int l0, int L, int H, int W,
                                       float (&uv)[T]) {
  // With VEC, L and l0 are multiples of 4 (T % 4 == 0), so each group of 4 steps
  // lies wholly inside or wholly outside the sequence: one guard per group.
  constexpr bool V4 = VEC && (T % 4 == 0);
  if (!col) {
    if constexpr (V4) {
      if (!rev) {
#pragma unroll
        for (int i = 0; i < T; i += 4) {
          float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
          if (FULL || l0 + i < L) q = Io<S>::ld4(xrow, l0 + i);
          uv[i] = q.x; uv[i + 1] = q.y; uv[i + 2] = q.z; uv[i + 3] = q.w;
        }
      } else {
        const int s_lo = L - l0 - T;  // walk indices s_lo .. s_lo+T-1; step i is at s_lo+T-1-i
#pragma unroll
        for (int i = 0; i < T; i += 4) {
          float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
          if (FULL || s_lo + i >= 0) q = Io<S>::ld4(xrow, s_lo + i);
          uv[T - 1 - i] = q.x; uv[T - 2 - i] = q.y; uv[T - 3 - i] = q.z; uv[T - 4 - i] = q.w;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < T; ++i)
        uv[i] = (FULL || l0 + i < L) ? Io<S>::ld(xrow, walk_index(rev, l0 + i, L)) : 0.f;
    }
  } else {
    // column walk: walk index s = w*H + h visits pixel h*W + w
    const int s0 = walk_index(rev, FULL ? l0 : min(l0, L - 1), L);
    int w = s0 / H;
    int h = s0 - w * H;
    const int dh = rev ? -1 : 1;
#pragma unroll
    for (int i = 0; i < T; ++i) {
      uv[i] = (FULL || l0 + i < L) ? Io<S>::ld(xrow, h * W + w) : 0.f;
      h += dh;
      const bool wrap_up = h == H, wrap_dn = h < 0;
      h = wrap_up ? 0 : (wrap_dn ? H - 1 : h);
      w += wrap_up ? 1 : (wrap_dn ? -1 : 0);
    }
  }
}

// x of T consecutive steps of a column walk from l0 (all inside the sequence),
// for H >= T: a lane's steps then change column at most once.  Step i of a
// forward walk is at pixel p0 + i*W until h0 + i reaches H, and one column on
// (1 - H*W further) from there; a reversed walk goes -W per step and one column
// back (H*W - 1 further) once h0 - i drops below 0.  Each load is a buffer load
// whose scalar offset is the step's multiple of W and whose lane offset is one of
// two per lane: a select per step instead of index arithmetic.
// rx: buffer over H*W biasing elements then the block's rows of x (every offset
// stays non-negative and inside it); xlane: this lane's channel row (elements).
template <typename S, int T>
__device__ __forceinline__ void load_x_col(__amdgpu_buffer_rsrc_t rx, uint32_t xlane, bool rev, int l0, int L, int H,
                                           int W, float (&uv)[T]) {
  constexpr uint32_t sz = sizeof(S);
  const int s0 = rev ? L - 1 - l0 : l0;
  const int w0 = s0 / H, h0 = s0 - w0 * H;
  const uint32_t HW = (uint32_t)(H * W), Wb = (uint32_t)W * sz;
  // byte offset of step 0 (forward) or of step T-1's row (reversed), before the change
  uint32_t a = (xlane + HW + (uint32_t)(h0 * W + w0)) * sz;
  if (rev) a -= (uint32_t)(T - 1) * Wb;  // >= 0: H >= T
  const uint32_t b = rev ? a + (HW - 1) * sz : a - (HW - 1) * sz;  // after the change
  const int k = rev ? h0 + 1 : H - h0;                              // first step after the change
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const uint32_t off = i < k ? a : b;
    const int so = (int)((uint32_t)(rev ? T - 1 - i : i) * Wb);
    if constexpr (sizeof(S) == 4)
      uv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, so, 0));
    else
      uv[i] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rx, off, so, 0));
  }
}

// T values of a row from l0 (zero past L).
template <typename S, int T, bool VEC, bool FULL>
__device__ __forceinline__ void load_row(const S* row, int l0, int L, float (&v)[T]) {
  if constexpr (VEC && (T % 4 == 0)) {  // groups of 4 wholly inside or outside (see load_x)
#pragma unroll
    for (int i = 0; i < T; i += 4) {
      float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
      if (FULL || l0 + i < L) q = Io<S>::ld4(row, l0 + i);
      v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i) v[i] = (FULL || l0 + i < L) ? Io<S>::ld(row, l0 + i) : 0.f;
  }
}

// Where a lane's dt comes from: its channel's dt row, or (R > 0) the R low-rank
// rows of its (batch, direction) and its channel's R weights (in LDS).
template <typename S>
struct DtSrc {
  const S* row;    // dt row of the lane's channel (R == 0)
  const S* lr;     // first low-rank row (R > 0); row r at lr + r * L
  const float* w;  // the lane's channel's weights, w[r]
  int R;
};

template <typename S, int T, bool VEC, bool FULL>
__device__ __forceinline__ void load_dt(const DtSrc<S>& src, int l0, int L, float (&dtv)[T]) {
  if (src.R == 0) {
    load_row<S, T, VEC, FULL>(src.row, l0, L, dtv);
    return;
  }
#pragma unroll
  for (int i = 0; i < T; ++i) dtv[i] = 0.f;
#pragma unroll 1
  for (int r = 0; r < src.R; ++r) {
    float v[T];
    load_row<S, T, VEC, FULL>(src.lr + (int64_t)r * L, l0, L, v);
    const float w = src.w[r];
#pragma unroll
    for (int i = 0; i < T; ++i) dtv[i] = fmaf(w, v[i], dtv[i]);
  }
}

template <typename S, int T, bool VEC, bool FULL>
__device__ __forceinline__ void load_inputs(const DtSrc<S>& dsrc, const S* xrow, bool rev, bool col, int l0, int L,
                                            int H, int W, float (&dtv)[T], float (&uv)[T]) {
  load_dt<S, T, VEC, FULL>(dsrc, l0, L, dtv);
  load_x<S, T, VEC, FULL>(xrow, rev, col, l0, L, H, W, uv);
}

// Raw dt/u -> delta, delta*u and the output's skip term D*u; returns sum(delta).
template <int T>
__device__ __forceinline__ float prepare_steps(const float (&dtv)[T], const float (&uv)[T], float bias, float dsk,
                                               bool dvalid, int nvalid, float (&delta)[T], float (&du)[T],
                                               float (&yv)[T]) {
  float sdelta = 0.f;
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const bool valid = dvalid && i < nvalid;
    delta[i] = valid ? softplus_f32(dtv[i] + bias) : 0.f;
    du[i] = delta[i] * uv[i];
    yv[i] = dsk * uv[i];
    sdelta += delta[i];
  }
  return sdelta;
}

template <int G, int T>
__device__ __forceinline__ void state_core(const float (&Bv)[T], const float (&Cv)[T], float A2n, float* carry_slot,
                                           int seg, const float (&delta)[T], const float (&du)[T], float sdelta,
                                           float (&yv)[T]);

// One state n of one chunk; this lane's register-staged B/C are at Bst/Cst.
template <int G, int T>
__device__ __forceinline__ void state_step(const float* Bst, const float* Cst, float A2n, float* carry_slot,
                                           int seg, const float (&delta)[T], const float (&du)[T], float sdelta,
                                           float (&yv)[T]) {
  float Bv[T], Cv[T];
  if constexpr (T % 4 == 0) {
#pragma unroll
    for (int i = 0; i < T; i += 4) {
      const float4 bq = *reinterpret_cast<const float4*>(Bst + i);
      const float4 cq = *reinterpret_cast<const float4*>(Cst + i);
      Bv[i] = bq.x; Bv[i + 1] = bq.y; Bv[i + 2] = bq.z; Bv[i + 3] = bq.w;
      Cv[i] = cq.x; Cv[i + 1] = cq.y; Cv[i + 2] = cq.z; Cv[i + 3] = cq.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i) {
      Bv[i] = Bst[i];
      Cv[i] = Cst[i];
    }
  }
  state_core<G, T>(Bv, Cv, A2n, carry_slot, seg, delta, du, sdelta, yv);
}

// One state n of one chunk from this lane's B/C values.
template <int G, int T>
__device__ __forceinline__ void state_core(const float (&Bv)[T], const float (&Cv)[T], float A2n, float* carry_slot,
                                           int seg, const float (&delta)[T], const float (&du)[T], float sdelta,
                                           float (&yv)[T]) {
  const float cin = *carry_slot;  // read first: its LDS latency hides behind the fold
  float a[T], bb[T];
#pragma unroll
  for (int i = 0; i < T; ++i) {
    a[i] = __builtin_amdgcn_exp2f(delta[i] * A2n);
    bb[i] = du[i] * Bv[i];
  }
  float Bl = bb[0];
#pragma unroll
  for (int i = 1; i < T; ++i) Bl = fmaf(a[i], Bl, bb[i]);
  float Al = __builtin_amdgcn_exp2f(A2n * sdelta);
  scan_inclusive<G>(Al, Bl);
  float h = incoming_state<G>(Al, Bl, cin, seg);
#pragma unroll
  for (int i = 0; i < T; ++i) {
    h = fmaf(a[i], h, bb[i]);
    yv[i] = fmaf(Cv[i], h, yv[i]);
  }
  if (seg == G - 1) *carry_slot = h;
}

// Carry pass: one state n of one chunk, without outputs.  The group's last lane
// holds the chunk's map (A_chunk, B_chunk) after the inclusive scan and folds it
// into the segment's map kept in LDS: carry = A_chunk carry + B_chunk and
// aprod = A_chunk aprod.
template <typename S, int G, int T>
__device__ __forceinline__ void state_carry(const char* Brow, int seg, float A2n, float* carry_slot, float* aprod_slot,
                                            const float (&delta)[T], const float (&du)[T], float sdelta) {
  float Bv[T];
  read_seg<S, T>(Brow, seg, Bv);
  float Bl = du[0] * Bv[0];
#pragma unroll
  for (int i = 1; i < T; ++i) Bl = fmaf(__builtin_amdgcn_exp2f(delta[i] * A2n), Bl, du[i] * Bv[i]);
  float Al = __builtin_amdgcn_exp2f(A2n * sdelta);
  scan_inclusive<G>(Al, Bl);
  if (seg == G - 1) {
    *carry_slot = fmaf(Al, *carry_slot, Bl);
    *aprod_slot *= Al;
  }
}

// Writes (or adds) a lane's outputs of T consecutive steps into its plane.
template <int T, bool VEC, bool FULL>
__device__ __forceinline__ void store_outputs(float* plane, bool rev, bool add, int l0, int L, const float (&yv)[T]) {
  if constexpr (VEC && (T % 4 == 0)) {  // groups of 4 wholly inside or outside (see load_x)
    const int s_lo = rev ? L - l0 - T : l0;
#pragma unroll
    for (int i = 0; i < T; i += 4) {
      if (!FULL && (s_lo + i < 0 || s_lo + i >= L)) continue;
      float4* q = reinterpret_cast<float4*>(plane + s_lo + i);
      float4 v = rev ? make_float4(yv[T - 1 - i], yv[T - 2 - i], yv[T - 3 - i], yv[T - 4 - i])
                     : make_float4(yv[i], yv[i + 1], yv[i + 2], yv[i + 3]);
      if (add) {
        const float4 o = *q;
        v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
      }
      *q = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i) {
      if (FULL || l0 + i < L) {
        float* q = plane + walk_index(rev, l0 + i, L);
        *q = add ? (*q + yv[i]) : yv[i];
      }
    }
  }
}

// The last direction (2, the reversed row walk) finishes the merge in place of a
// separate pass: y[p] = (row plane[p] + out) + column plane[w*H + h] for the
// lane's T pixels p = h*W + w, rounded once to the storage type.  Step l0 + i
// visits pixel L-1-l0-i.  The row plane holds direction 0 (it is y itself for
// fp32 output: each element is read, then written, by the same lane), the
// column plane directions 1 + 3, so y = (y0 + y2) + (y1 + y3).
// pct: the column plane transposed to row-major order, or null (then gathered);
// both null: no column directions (K = 2), y = y0 + y2.
// yf: with bf16 storage, an fp32 destination instead of y (a state block before
// the last leaves its sums in the row plane); null otherwise.
template <typename S, int T, bool VEC, bool FULL>
__device__ __forceinline__ void store_final(const float* prow, const float* pcol, const float* pct, S* y, float* yf,
                                            int l0, int L, int H, int W, const float (&yv)[T]) {
  if constexpr (VEC && (T % 4 == 0)) {
    // pixels s_lo .. s_lo+T-1; pixel s_lo+j holds yv[T-1-j].  A partial chunk's
    // pixels below 0 come in whole groups of 4 (see load_x) and are skipped.
    const int s_lo = L - l0 - T;
    float v[T];
#pragma unroll
    for (int j = 0; j < T; j += 4) {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      if (FULL || s_lo + j >= 0) o = *reinterpret_cast<const float4*>(prow + s_lo + j);
      v[j] = o.x + yv[T - 1 - j];
      v[j + 1] = o.y + yv[T - 2 - j];
      v[j + 2] = o.z + yv[T - 3 - j];
      v[j + 3] = o.w + yv[T - 4 - j];
    }
    if (pct != nullptr) {
#pragma unroll
      for (int j = 0; j < T; j += 4) {
        if (!FULL && s_lo + j < 0) continue;
        const float4 o = *reinterpret_cast<const float4*>(pct + s_lo + j);
        v[j] += o.x;
        v[j + 1] += o.y;
        v[j + 2] += o.z;
        v[j + 3] += o.w;
      }
    } else if (pcol != nullptr) {
      const int s0 = FULL ? s_lo : max(s_lo, 0);
      int h = s0 / W;
      int w = s0 - h * W;
#pragma unroll
      for (int j = 0; j < T; ++j) {
        if (!FULL && s_lo + j < 0) continue;
        v[j] += pcol[w * H + h];
        ++w;
        const bool wrap = w == W;
        w = wrap ? 0 : w;
        h += wrap ? 1 : 0;
      }
    }
    if (sizeof(S) != 4 && yf != nullptr) {
#pragma unroll
      for (int j = 0; j < T; j += 4)
        if (FULL || s_lo + j >= 0) Io<float>::st4(yf, s_lo + j, make_float4(v[j], v[j + 1], v[j + 2], v[j + 3]));
    } else {
#pragma unroll
      for (int j = 0; j < T; j += 4)
        if (FULL || s_lo + j >= 0) Io<S>::st4(y, s_lo + j, make_float4(v[j], v[j + 1], v[j + 2], v[j + 3]));
    }
  } else {
    int pix = L - 1 - (FULL ? l0 : min(l0, L - 1));
    int h = pix / W;
    int w = pix - h * W;
#pragma unroll
    for (int i = 0; i < T; ++i) {
      if (FULL || l0 + i < L) {
        float v = prow[pix] + yv[i];
        if (pct != nullptr)
          v += pct[pix];
        else if (pcol != nullptr)
          v += pcol[w * H + h];
        if (sizeof(S) != 4 && yf != nullptr)
          yf[pix] = v;
        else
          Io<S>::st(y, pix, v);
      }
      --pix;
      --w;
      const bool wrap = w < 0;
      w = wrap ? W - 1 : w;
      h -= wrap ? 1 : 0;
    }
  }
}

// Register staging of Bs/Cs for a remainder chunk: NG states x {B, C} x (G lanes
// x TT steps) from step c0 and state n0 on, each thread holding its share in
// float4 registers until it writes them to LDS.  One (state, array) takes
// kArr = G * seg_stride(TT) floats there, lane segments padded against bank
// conflicts.
template <typename S, int G, int NG, int TT, bool VEC, bool FULL>
struct Stager {
  static constexpr int kNth = kWaves * 64;
  static constexpr int kPer = G * TT / 4;        // float4 per (state, array)
  static constexpr int kF4 = NG * 2 * kPer;      // float4 per group
  static constexpr int kQ = (kF4 + kNth - 1) / kNth;
  static constexpr int kSS = seg_stride<TT>();
  static constexpr int kArr = G * kSS;
  float4 r[kQ];

  __device__ __forceinline__ void fetch(const S* Bbase, const S* Cbase, int tid, int n0, int N, int c0, int L) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int f = tid + q * kNth;
      r[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (f < kF4) {
        const int nn = f / (2 * kPer);
        const int rem = f - nn * (2 * kPer);
        const int arr = rem / kPer;
        const int j = (rem - arr * kPer) * 4;
        if (n0 + nn < N) {
          const S* row = (arr == 0 ? Bbase : Cbase) + (int64_t)(n0 + nn) * L;
          if constexpr (VEC && FULL)
            r[q] = Io<S>::ld4(row, c0 + j);
          else
            r[q] = ld4_guarded<S>(row, c0 + j, L, VEC);
        }
      }
    }
  }
  __device__ __forceinline__ void commit(float* buf, int tid) const {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int f = tid + q * kNth;
      if (f < kF4) {
        const int nn = f / (2 * kPer);
        const int rem = f - nn * (2 * kPer);
        const int arr = rem / kPer;
        const int j = (rem - arr * kPer) * 4;
        *reinterpret_cast<float4*>(buf + (nn * 2 + arr) * kArr + (j / TT) * kSS + (j % TT)) = r[q];
      }
    }
  }
};

struct Lane {
  int tid, seg, dl, b, d0, dsafe;
  bool dvalid;
};

// A remainder chunk of G*TT steps (TT <= T, possibly ragged), staged through
// registers in groups of as many states as fit the LDS area at smem (kAreaBytes);
// with few steps per lane that is all of them, so the chunk synchronises once.
// Inlined: as a call, the calling convention would make the main loop keep its
// values in fewer, callee-saved registers, and the callee spill to scratch.
template <typename S, int G, int T, int NG0, int TT, bool VEC, int kAreaBytes>
__device__ __forceinline__ void tail_chunk(int tid, int seg, int dl, bool dvalid, float* smem, float* a2s, float* carry,
                                        const DtSrc<S>& dsrc, const S* xrow, const S* Bbase, const S* Cbase, float* plane,
                                        const float* pcol, const float* pct, S* yout, float* yf, bool rev, bool col, bool add,
                                        bool last, float bias,
                                        float dsk, int c0, int L, int H, int W, int N) {
  Lane ln;
  ln.tid = tid;
  ln.seg = seg;
  ln.dl = dl;
  ln.dvalid = dvalid;
  constexpr int kStateBytes = 2 * G * seg_stride<TT>() * 4;
  constexpr int kFit = kAreaBytes / kStateBytes;
  constexpr int NG = kFit >= kMaxN ? kMaxN : (kFit >= NG0 ? kFit : NG0);
  static_assert(NG * kStateBytes <= kAreaBytes, "staged group must fit its LDS area");
  using St = Stager<S, G, NG, TT, VEC, false>;
  constexpr int SS = seg_stride<TT>();
  const int l0 = c0 + ln.seg * TT;
  float dtv[TT], uv[TT];
  load_inputs<S, TT, VEC, false>(dsrc, xrow, rev, col, l0, L, H, W, dtv, uv);
  float delta[TT], du[TT], yv[TT];
  const float sdelta = prepare_steps<TT>(dtv, uv, bias, dsk, ln.dvalid, L - l0, delta, du, yv);
  for (int n0 = 0; n0 < N; n0 += NG) {
    St st;
    st.fetch(Bbase, Cbase, ln.tid, n0, N, c0, L);
    st.commit(smem, ln.tid);
    __syncthreads();
#pragma unroll 1
    for (int nn = 0; nn < NG; ++nn) {
      const int n = n0 + nn;
      if (n < N)
        state_step<G, TT>(smem + (nn * 2) * St::kArr + ln.seg * SS, smem + (nn * 2 + 1) * St::kArr + ln.seg * SS,
                          a2s[ln.dl * kMaxN + n], carry + ln.dl * kMaxN + n, ln.seg, delta, du, sdelta, yv);
    }
    __syncthreads();
  }
  if (ln.dvalid) {
    if (last)
      store_final<S, TT, VEC, false>(plane, pcol, pct, yout, yf, l0, L, H, W, yv);
    else
      store_outputs<TT, VEC, false>(plane, rev, add, l0, L, yv);
  }
}

// The first remainder chunk when it was prefetched during the last full chunk:
// dt (one plain row per channel) at dts, Bs then Cs (kMaxN plain rows each) at
// bcs, and x already in uv.  No global load waits here.
template <typename S, int G, int TT, bool VEC>
__device__ __forceinline__ void tail_chunk_lds(const Lane& ln, const char* dts, int R, const float* wl, const char* bcs,
                                               const float (&uv)[TT],
                                               const float* a2s, float* carry, float* plane, const float* pcol,
                                               const float* pct, S* yout, float* yf, bool rev, bool add, bool last, float bias,
                                               float dsk, int c0,
                                               int L, int H, int W, int N) {
  constexpr int RB = G * TT * (int)sizeof(S);
  const int l0 = c0 + ln.seg * TT;
  float dtv[TT];
  if (R == 0) {
    read_plain<S, TT>(dts + ln.dl * RB, ln.seg, dtv);
  } else {  // low-rank rows 0..R-1 of the plain copy, weighted by the channel's weights
#pragma unroll
    for (int i = 0; i < TT; ++i) dtv[i] = 0.f;
#pragma unroll 1
    for (int r = 0; r < R; ++r) {
      float v[TT];
      read_plain<S, TT>(dts + r * RB, ln.seg, v);
      const float w = wl[r];
#pragma unroll
      for (int i = 0; i < TT; ++i) dtv[i] = fmaf(w, v[i], dtv[i]);
    }
  }
  float delta[TT], du[TT], yv[TT];
  const float sdelta = prepare_steps<TT>(dtv, uv, bias, dsk, true, L - l0, delta, du, yv);
#pragma unroll 1
  for (int n = 0; n < N; ++n) {
    float Bv[TT], Cv[TT];
    read_plain<S, TT>(bcs + n * RB, ln.seg, Bv);
    read_plain<S, TT>(bcs + (kMaxN + n) * RB, ln.seg, Cv);
    state_core<G, TT>(Bv, Cv, a2s[ln.dl * kMaxN + n], carry + ln.dl * kMaxN + n, ln.seg, delta, du, sdelta, yv);
  }
  if (ln.dvalid) {
    if (last)
      store_final<S, TT, VEC, false>(plane, pcol, pct, yout, yf, l0, L, H, W, yv);
    else
      store_outputs<TT, VEC, false>(plane, rev, add, l0, L, yv);
  }
}

template <typename S, int G, int T, int NG, bool VEC, int MODE>
__global__ __launch_bounds__(kWaves * 64, T == 8 ? 4 : 3) void ss2d_forward_kernel(Params p) {
  using C = Cfg<G, T, NG>;
  using Y = Layout<S, G, T, NG, VEC>;
  constexpr int CH = C::kChans;
  constexpr int NTH = C::kThreads;
  constexpr int GT = G * T;
  constexpr int GB = (sizeof(S) == 4 && VEC) ? 16 : 4;  // bytes per lane of one DMA copy
  // A remainder chunk of TT steps per lane is prefetched when the Bs/Cs rows of
  // every state fit one ring.  Not for 16 lanes: that variant has no registers to
  // spare, and serves sequences under 512 steps.
  // The plain copies also need whole wave-wide copies for the dt and Bs/Cs rows.
  constexpr auto kTailFits = [](int tt) {
    const int row = G * tt * (int)sizeof(S), wave_bytes = 64 * GB;
    return G >= 32 && kMaxN * tt <= NG * T && (C::kChans * row) % wave_bytes == 0 &&
           (kMaxN * row) % wave_bytes == 0 && (row % wave_bytes == 0 || wave_bytes % row == 0);
  };
  __shared__ __align__(16) char ring0[Y::kRing0Bytes];
  __shared__ __align__(16) char ring1[Y::kGroupBytes];
  __shared__ __align__(16) char dtb[Y::kDtBytes];
  __shared__ float par[Y::kParFloats];
  __shared__ __align__(16) char wide[Y::kWideBytes > 0 ? Y::kWideBytes : 16];
  float* smem = reinterpret_cast<float*>(ring0);
  float* a2s = par;
  float* carry = a2s + CH * kMaxN;
  float* biass = carry + CH * kMaxN;
  float* dss = biass + CH;
  float* aprod = dss + CH;
  float* wts = aprod + CH * kMaxN;  // low-rank weights: [CH][kMaxLowRank]

  // Work id: consecutive ids (same batch and segment, neighbouring channel blocks,
  // which share Bs/Cs) stay on one XCD; workgroups are dealt round-robin over the
  // 8 XCDs.
  const int nb = gridDim.x;
  const int xcd = blockIdx.x & 7, bslot = blockIdx.x >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int work = (xcd < rem) ? xcd * (per + 1) + bslot : rem * (per + 1) + (xcd - rem) * per + bslot;
  // The hardware serves co-resident waves oldest first, so in a launch that fits
  // one round the workgroups of a CU finish one after another, in dispatch order,
  // and the last runs its end alone (on stage-1 shapes 360, 450 and 540 us).  A
  // CU receives one workgroup per round of prio_ncu dispatches; rotating the
  // priority every chunk by (that rank + chunks done) gives each the lead in turn.
  int prio_tick = p.prio_ncu > 0 ? (int)(blockIdx.x / (unsigned)p.prio_ncu) % p.prio_levels : 0;
  auto rotate_priority = [&]() {
    if (p.prio_ncu > 0) {
      set_priority(prio_tick);
      prio_tick = prio_tick + 1 == p.prio_levels ? 0 : prio_tick + 1;
    }
  };

  Lane ln;
  ln.tid = threadIdx.x;
  const int lane = ln.tid & 63, wave = ln.tid >> 6;
  ln.seg = lane % G;
  ln.dl = wave * (64 / G) + lane / G;
  const int nbd = (p.D + CH - 1) / CH;
  const int nsw = MODE == kCarry ? p.nseg - 1 : p.nseg;  // segments handled by this launch
  const int bs = work / nbd;                              // batch * nsw + segment
  ln.b = bs / nsw;
  const int sidx = bs - ln.b * nsw;
  ln.d0 = (work - bs * nbd) * CH;
  ln.dvalid = ln.d0 + ln.dl < p.D;
  ln.dsafe = ln.dvalid ? ln.d0 + ln.dl : 0;
  const int L = p.L, N = p.N, H = p.H, W = p.W, D = p.D;
  const int64_t plane_off = ((int64_t)ln.b * D + ln.dsafe) * L;
  const S* xrow = static_cast<const S*>(p.x) + plane_off;
  const DmaPlan<S, G, T, 2 * NG, GB> bpl(ln.tid);  // one Bs/Cs group
  const DmaPlan<S, G, T, CH, GB> dpl(ln.tid);      // dt of one chunk

  // Full chunks [cbeg, cend) of this workgroup's segment; the remainder steps
  // after the last full chunk belong to the last segment.
  const int nmain = L / GT;
  const int cbeg = sidx * p.seg_chunks;
  const bool last_seg = sidx == p.nseg - 1;
  const int cend = last_seg ? nmain : cbeg + p.seg_chunks;

  // One direction, specialised at compile time (walk order, merge mode).
  auto direction = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    // slot of this direction in the per-direction tensors (K = 2: walks 0 and 2)
    const int slot = p.K == 4 ? k : (k >> 1);
    // per-direction parameters of the block's channels; the state entering the
    // segment is the composition of the maps of the segments before it
    for (int i = ln.tid; i < CH * kMaxN; i += NTH) {
      const int dd = i / kMaxN, n = i - dd * kMaxN;
      const int dg = ln.d0 + dd;
      float v = 0.f, h = 0.f;
      if (dg < D && n < N) {
        v = -expf(p.A_log[(int64_t)(slot * D + dg) * p.Nt + p.n0 + n]) * kLog2e;
        if (MODE == kSegment) {
          const float* cr = p.carries + ((int64_t)(ln.b * p.K + slot) * D + dg) * p.nseg * (2 * kMaxN);
          for (int j = 0; j < sidx; ++j) h = fmaf(cr[j * 2 * kMaxN + 2 * n], h, cr[j * 2 * kMaxN + 2 * n + 1]);
        }
      }
      a2s[i] = v;
      carry[i] = h;
      aprod[i] = 1.f;
    }
    for (int i = ln.tid; i < CH; i += NTH) {
      const int dg = ln.d0 + i;
      biass[i] = dg < D ? p.dt_bias[slot * D + dg] : 0.f;
      dss[i] = (dg < D && p.skip) ? p.Ds[slot * D + dg] : 0.f;
    }
    for (int i = ln.tid; i < CH * kMaxLowRank; i += NTH) {
      const int dd = i / kMaxLowRank, r = i - dd * kMaxLowRank;
      const int dg = ln.d0 + dd;
      wts[i] = (dg < D && r < p.R) ? p.wdt[(int64_t)(slot * D + dg) * p.R + r] : 0.f;
    }
    __syncthreads();

    constexpr bool rev = k >= 2, col = (k & 1) != 0, last = k == 2;
    // direction 3 adds to the column plane direction 1 wrote; direction 0 adds to
    // the row plane when earlier state blocks left their sums there
    const bool add = k == 3 || (k == 0 && p.acc != 0);
    float* plane = (col ? p.pcol : p.prow) + plane_off;
    const float* pcol = p.K == 4 ? p.pcol + plane_off : nullptr;  // null: no column plane to merge
    S* yout = static_cast<S*>(p.y) + plane_off;
    // bf16 state blocks before the last keep fp32 sums in the row plane
    float* yf = (sizeof(S) != 4 && !p.final_out) ? p.prow + plane_off : nullptr;
    // dt rows of this (batch, direction), or its R low-rank rows
    const int drows_all = p.R > 0 ? p.R : D;
    const S* dtdir = static_cast<const S*>(p.dt) + (int64_t)(ln.b * p.K + slot) * drows_all * L;
    DtSrc<S> dsrc;
    dsrc.row = dtdir + (int64_t)(p.R > 0 ? 0 : ln.dsafe) * L;
    dsrc.lr = dtdir;
    dsrc.w = wts + ln.dl * kMaxLowRank;
    dsrc.R = p.R;
    // column walks over the transposed copy of x read contiguous rows; direction 2
    // reads a transposed column plane when there is one
    const bool xt = col && p.xT != nullptr;
    const S* xsrc = xt ? static_cast<const S*>(p.xT) + plane_off : xrow;
    const bool xcol = col && !xt;
    const float* pct = p.pcolT != nullptr ? p.pcolT + plane_off : nullptr;
    const int64_t bc_off = ((int64_t)(ln.b * p.K + slot) * p.Nt + p.n0) * L;
    const S* Bbase = static_cast<const S*>(p.Bs) + bc_off;
    const S* Cbase = static_cast<const S*>(p.Cs) + bc_off;
    const float bias = biass[ln.dl];
    const float dsk = dss[ln.dl];
    const int ngrp = (N + NG - 1) / NG;
    int c0 = cbeg * GT;

    if constexpr (VEC) {
      // ---------------- full chunks: Bs/Cs one group ahead and dt one chunk ahead, by DMA
      // Staged rows: dt of the block's channels (a valid row stands in past D), and
      // per Bs/Cs group the B rows of its NG states, then their C rows (state 0
      // stands in past N).  Resources cover this (batch, direction) only.
      const int nval = D - ln.d0 < CH ? D - ln.d0 : CH;
      const uint32_t rowsz = (uint32_t)L * (uint32_t)sizeof(S);
      // staged dt rows: the block's channels (a valid row stands in past D), or the
      // R low-rank rows (row 0 stands in for the CH - R rows past them)
      const int nrow = p.R > 0 ? p.R : nval;
      const __amdgpu_buffer_rsrc_t rdt =
          make_rsrc(dtdir + (int64_t)(p.R > 0 ? 0 : ln.d0) * L, (uint32_t)nrow * rowsz);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bbase, (uint32_t)N * rowsz);
      const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cbase, (uint32_t)N * rowsz);
      auto dt_rows = [=](int r) { return RowRef{rdt, (uint32_t)(r < nrow ? r : 0) * rowsz}; };
      auto bc_rows = [=](int g) {
        return [=](int r) {
          const int n = g * NG + (r < NG ? r : r - NG);
          return RowRef{r < NG ? rb : rc, (uint32_t)(n < N ? n : 0) * rowsz};
        };
      };
      // A sequence shorter than one chunk but at least half of one runs as a single
      // partial chunk of this pipeline (its steps past L are identity maps)
      // instead of remainder chunks.  Only 16-lane plans see such lengths (32
      // lanes are planned from 512 steps on).
      constexpr bool kPartial = G == 16;
      const bool partial = kPartial && nmain == 0 && 2 * L >= GT;
      // The first remainder chunk (T1 steps per lane) is prefetched during the last
      // full chunk, where nothing else is: its dt into dtb, the Bs/Cs rows of every
      // state into the ring the last group does not read, its x into xn.
      const int Lt = L - cend * GT;
      const int T1 = Lt >= 8 * G ? 8 : Lt >= 4 * G ? 4 : Lt >= 2 * G ? 2 : 1;
      const bool tailpf = MODE != kCarry && last_seg && cend > cbeg && Lt > 0 && kTailFits(T1);
      auto tail_bc_rows = [=](int r) {
        const int n = r & (kMaxN - 1);
        return RowRef{r < kMaxN ? rb : rc, (uint32_t)(n < N ? n : 0) * rowsz};
      };
      auto tail_copy = [&](char* bcdst, bool dt_part, auto tt) {
        constexpr int TT = decltype(tt)::value;
        if constexpr (kTailFits(TT)) {
          if (dt_part)
            PlainCopy<S, G, TT, CH, GB>::copy(dtb, dt_rows, cend * GT, ln.tid);
          else
            PlainCopy<S, G, TT, 2 * kMaxN, GB>::copy(bcdst, tail_bc_rows, cend * GT, ln.tid);
        }
      };
      auto tail_copy_any = [&](char* bcdst, bool dt_part) {
        switch (T1) {
          case 8: tail_copy(bcdst, dt_part, std::integral_constant<int, 8>{}); break;
          case 4: tail_copy(bcdst, dt_part, std::integral_constant<int, 4>{}); break;
          case 2: tail_copy(bcdst, dt_part, std::integral_constant<int, 2>{}); break;
          default: tail_copy(bcdst, dt_part, std::integral_constant<int, 1>{}); break;
        }
      };
      if (cend > cbeg || partial) {
        dpl.copy(dtb, dt_rows, cbeg * GT, partial ? L : GT);
        bpl.copy(ring0, bc_rows(0), cbeg * GT, partial ? L : GT);
        wait_vmem();
        __syncthreads();
      }
      // Group g of every chunk lives in ring(g & 1); the next chunk's group 0 is
      // copied during this chunk's last group when that group is in ring1.
      const bool cross = (ngrp & 1) == 0;
      float xn[T];  // x of the next chunk, loaded a whole chunk ahead
      // x of a full chunk's T steps from l0: column walks with H >= T by the
      // select-per-step gather, everything else by load_x
      const int nxr = D - ln.d0 < CH ? D - ln.d0 : CH;  // valid channel rows of the block
      const __amdgpu_buffer_rsrc_t rx =
          make_rsrc(static_cast<const S*>(p.x) + ((int64_t)ln.b * D + ln.d0) * L - (int64_t)H * W,
                    (uint32_t)((int64_t)H * W + (int64_t)nxr * L) * (uint32_t)sizeof(S));
      const uint32_t xlane = (uint32_t)(ln.dvalid ? ln.dl : 0) * (uint32_t)L;
      auto load_full_x = [&](int l0) {
        if constexpr (col) {
          if (!xt && H >= T) {
            load_x_col<S, T>(rx, xlane, rev, l0, L, H, W, xn);
            return;
          }
        }
        load_x<S, T, VEC, true>(xsrc, rev, xcol, l0, L, H, W, xn);
      };
      if (partial)
        load_x<S, T, VEC, false>(xsrc, rev, xcol, ln.seg * T, L, H, W, xn);
      else if (cbeg < cend)
        load_full_x(cbeg * GT + ln.seg * T);
      auto load_tail_x = [&](float (&xv)[T]) {  // x of the first remainder chunk, into xv[0, T1)
        auto ld = [&](auto tt) {
          constexpr int TT = decltype(tt)::value;
          if constexpr (kTailFits(TT)) {
            float v[TT];
            load_x<S, TT, VEC, false>(xsrc, rev, xcol, cend * GT + ln.seg * TT, L, H, W, v);
#pragma unroll
            for (int i = 0; i < TT; ++i) xv[i] = v[i];
          }
        };
        switch (T1) {
          case 8: ld(std::integral_constant<int, 8>{}); break;
          case 4: ld(std::integral_constant<int, 4>{}); break;
          case 2: ld(std::integral_constant<int, 2>{}); break;
          default: ld(std::integral_constant<int, 1>{}); break;
        }
      };
      // One chunk; PART: the partial last chunk (full chunks keep their checks
      // out of the code).
      auto chunk = [&](int c, auto part_c) {
        constexpr bool PART = decltype(part_c)::value;
        rotate_priority();
        float dtn[T];
        if (p.R == 0) {
          read_seg<S, T>(dtb + ln.dl * GT * (int)sizeof(S), ln.seg, dtn);
        } else {  // dt from the staged low-rank rows and the channel's weights
#pragma unroll
          for (int i = 0; i < T; ++i) dtn[i] = 0.f;
#pragma unroll 1
          for (int r = 0; r < p.R; ++r) {
            float v[T];
            read_seg<S, T>(dtb + r * GT * (int)sizeof(S), ln.seg, v);
            const float w = dsrc.w[r];
#pragma unroll
            for (int i = 0; i < T; ++i) dtn[i] = fmaf(w, v[i], dtn[i]);
          }
        }
        float delta[T], du[T], yv[T];
        // Lanes of a channel past D work on channel d0's data and store nothing; a
        // group of G lanes never mixes channels, so no masking is needed here.
        // Steps past L (partial chunk) get delta = 0: the identity map.
        const int nvalid = PART ? L - (c * GT + ln.seg * T) : T;
        const float sdelta = prepare_steps<T>(dtn, xn, bias, dsk, true, nvalid, delta, du, yv);
        if (!PART && c + 1 < cend) load_full_x((c + 1) * GT + ln.seg * T);
        auto group = [&](const char* cur, char* nxt, int g) {
          const bool more_states = g + 1 < ngrp;
          // nxt was last read before the previous barrier
          if (more_states)
            bpl.copy(nxt, bc_rows(g + 1), c * GT, PART ? L : GT);
          else if (!PART && cross && c + 1 < cend)
            bpl.copy(nxt, bc_rows(0), (c + 1) * GT);
          else if (!PART && tailpf && c + 1 == cend)
            tail_copy_any(nxt, false);
          if (!PART && g == 1 && c + 1 < cend)  // every lane has read this chunk's dt (barrier after group 0)
            dpl.copy(dtb, dt_rows, (c + 1) * GT);
          else if (!PART && g == 1 && tailpf)
            tail_copy_any(dtb, true);
          // bf16 rows: widened to fp32 once for all channels (cur is complete: the
          // previous group waited for its copy; wide was last read before that
          // group's closing barrier)
          constexpr bool kWiden = sizeof(S) == 2 && MODE != kCarry;
          if constexpr (kWiden) {
            widen_rows<T, 2 * NG, GT, NTH>(cur, wide, ln.tid);
            __syncthreads();
          }
          // Unrolled, so the LDS offsets of each state are immediates; the barrier keeps
          // the states apart (interleaved, their registers would not fit).
#pragma unroll
          for (int nn = 0; nn < NG; ++nn) {
            const int n = g * NG + nn;
            __builtin_amdgcn_sched_barrier(0);
            if (n < N) {
              if constexpr (MODE == kCarry) {
                state_carry<S, G, T>(cur + nn * GT * (int)sizeof(S), ln.seg, a2s[ln.dl * kMaxN + n],
                                     carry + ln.dl * kMaxN + n, aprod + ln.dl * kMaxN + n, delta, du, sdelta);
              } else {
                float Bv[T], Cv[T];
                if constexpr (kWiden) {
                  read_seg<float, T>(wide + nn * GT * 4, ln.seg, Bv);
                  read_seg<float, T>(wide + (NG + nn) * GT * 4, ln.seg, Cv);
                } else {
                  read_seg<S, T>(cur + nn * GT * (int)sizeof(S), ln.seg, Bv);
                  read_seg<S, T>(cur + (NG + nn) * GT * (int)sizeof(S), ln.seg, Cv);
                }
                state_core<G, T>(Bv, Cv, a2s[ln.dl * kMaxN + n], carry + ln.dl * kMaxN + n, ln.seg, delta, du,
                                 sdelta, yv);
              }
            }
          }
          wait_vmem();
          __syncthreads();
        };
        for (int g = 0; g < ngrp; g += 2) {
          group(ring0, ring1, g);
          if (g + 1 < ngrp) group(ring1, ring0, g + 1);
        }
        if (!PART && c + 1 < cend && (!cross || ngrp == 1)) {  // nothing was copied ahead: copy now and wait
          if (!cross) bpl.copy(ring0, bc_rows(0), (c + 1) * GT);
          if (ngrp == 1) dpl.copy(dtb, dt_rows, (c + 1) * GT);
          wait_vmem();
          __syncthreads();
        }
        if (!PART && tailpf && c + 1 == cend && ngrp == 1) {  // the remainder's dt was not copied yet
          tail_copy_any(dtb, true);
          wait_vmem();
          __syncthreads();
        }
        // The remainder's x, loaded here rather than a chunk ahead: held through the
        // state loops it would cost registers; here it overlaps this chunk's stores.
        if (!PART && tailpf && c + 1 == cend) load_tail_x(xn);
        if (MODE != kCarry && ln.dvalid) {
          if (last)
            store_final<S, T, VEC, !PART>(plane, pcol, pct, yout, yf, c * GT + ln.seg * T, L, H, W, yv);
          else
            store_outputs<T, VEC, !PART>(plane, rev, add, c * GT + ln.seg * T, L, yv);
        }
      };
      if constexpr (kPartial) {
        if (partial) chunk(0, std::true_type{});
      }
      if (!partial)
        for (int c = cbeg; c < cend; ++c) chunk(c, std::false_type{});
      c0 = partial ? L : cend * GT;
      if (tailpf) {
        char* bcs = (ngrp & 1) ? ring1 : ring0;  // the ring the last group did not read
        auto run = [&](auto tt) {
          constexpr int TT = decltype(tt)::value;
          if constexpr (kTailFits(TT)) {
            float uv[TT];
#pragma unroll
            for (int i = 0; i < TT; ++i) uv[i] = xn[i];
            tail_chunk_lds<S, G, TT, VEC>(ln, dtb, p.R, wts + ln.dl * kMaxLowRank, bcs, uv, a2s, carry, plane, pcol, pct, yout, yf, rev, add, last, bias,
                                          dsk, c0, L, H, W, N);
          }
        };
        switch (T1) {
          case 8: run(std::integral_constant<int, 8>{}); break;
          case 4: run(std::integral_constant<int, 4>{}); break;
          case 2: run(std::integral_constant<int, 2>{}); break;
          default: run(std::integral_constant<int, 1>{}); break;
        }
        c0 = Lt < G * T1 ? L : c0 + G * T1;
        __syncthreads();  // the rings and dtb are free again
      }
    } else {
      // ---------------- rows not 16-byte aligned: every chunk staged through registers
      for (; c0 + GT <= L; c0 += GT)
        tail_chunk<S, G, T, NG, T, VEC, Y::kRing0Bytes>(ln.tid, ln.seg, ln.dl, ln.dvalid, smem, a2s, carry, dsrc, xsrc, Bbase, Cbase,
                                        plane, pcol, pct, yout, yf, rev, xcol, add, last, bias, dsk, c0, L, H, W, N);
    }

    if constexpr (MODE == kCarry) {
      // ---------------- the segment's map per (channel, state)
      __syncthreads();
      for (int i = ln.tid; i < CH * kMaxN; i += NTH) {
        const int dd = i / kMaxN, n = i - dd * kMaxN;
        const int dg = ln.d0 + dd;
        if (dg < D && n < N) {
          float* cr = p.carries + (((int64_t)(ln.b * p.K + slot) * D + dg) * p.nseg + sidx) * (2 * kMaxN);
          cr[2 * n] = aprod[i];
          cr[2 * n + 1] = carry[i];
        }
      }
      __syncthreads();
      return;
    }
    if (!last_seg) {
      __syncthreads();  // this direction's plane writes are complete and visible to the block
      return;
    }

    // ---------------- remainder chunks (fewer steps per lane)
    while (L - c0 >= G * 8) {
      tail_chunk<S, G, T, NG, 8, VEC, Y::kRing0Bytes>(ln.tid, ln.seg, ln.dl, ln.dvalid, smem, a2s, carry, dsrc, xsrc, Bbase, Cbase,
                                      plane, pcol, pct, yout, yf, rev, xcol, add, last, bias, dsk, c0, L, H, W, N);
      c0 += G * 8;
    }
    if (L - c0 >= G * 4) {
      tail_chunk<S, G, T, NG, 4, VEC, Y::kRing0Bytes>(ln.tid, ln.seg, ln.dl, ln.dvalid, smem, a2s, carry, dsrc, xsrc, Bbase, Cbase,
                                      plane, pcol, pct, yout, yf, rev, xcol, add, last, bias, dsk, c0, L, H, W, N);
      c0 += G * 4;
    }
    if (L - c0 >= G * 2) {
      tail_chunk<S, G, T, NG, 2, VEC, Y::kRing0Bytes>(ln.tid, ln.seg, ln.dl, ln.dvalid, smem, a2s, carry, dsrc, xsrc, Bbase, Cbase,
                                      plane, pcol, pct, yout, yf, rev, xcol, add, last, bias, dsk, c0, L, H, W, N);
      c0 += G * 2;
    }
    while (c0 < L) {
      tail_chunk<S, G, T, NG, 1, VEC, Y::kRing0Bytes>(ln.tid, ln.seg, ln.dl, ln.dvalid, smem, a2s, carry, dsrc, xsrc, Bbase, Cbase,
                                      plane, pcol, pct, yout, yf, rev, xcol, add, last, bias, dsk, c0, L, H, W, N);
      c0 += G;
    }
    __syncthreads();  // this direction's plane writes are complete and visible to the block
  };

  if constexpr (MODE == kSegment) {
    switch (p.kdir) {
      case 0: direction(std::integral_constant<int, 0>{}); break;
      case 1: direction(std::integral_constant<int, 1>{}); break;
      case 2: direction(std::integral_constant<int, 2>{}); break;
      default: direction(std::integral_constant<int, 3>{}); break;
    }
  } else {
    // column pair, then row pair: the last direction finishes the merge
    if (p.K == 4) {
      direction(std::integral_constant<int, 1>{});
      direction(std::integral_constant<int, 3>{});
    }
    direction(std::integral_constant<int, 0>{});
    direction(std::integral_constant<int, 2>{});
  }
}

// States per Bs/Cs staging group for G lanes x T steps: one group is 16 KB of
// fp32 (8 KB of bf16) for T = 16, half that for T = 8, so the LDS of a
// workgroup allows three (T = 16) or four (T = 8) workgroups per CU, matching
// the register budget of each.
template <int G, int T>
constexpr int group_states() {
  return T == 16 ? 2048 / (G * T) : 1024 / (G * T);
}

// Plane transpose: out[p][c][r] = in[p][r][c] for `planes` planes of R x C, in
// 64 x 64 tiles through LDS (coalesced reads along c, writes along r).
template <typename S>
__global__ __launch_bounds__(256) void transpose_planes(const S* __restrict__ in, S* __restrict__ out, int R, int C,
                                                        int tiles_r, int tiles_c) {
  __shared__ float tile[64][65];
  const int t = blockIdx.x;
  const int tc = t % tiles_c;
  const int rest = t / tiles_c;
  const int tr = rest % tiles_r;
  const int64_t plane = rest / tiles_r;
  const S* src = in + plane * R * C;
  S* dst = out + plane * R * C;
  const int r0 = tr * 64, c0 = tc * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll 4
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < C) tile[i][tx] = Io<S>::ld(src, (int64_t)r * C + c);
  }
  __syncthreads();
#pragma unroll 4
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < R) Io<S>::st(dst, (int64_t)c * R + r, tile[tx][i]);
  }
}

// The same with R and C multiples of 4 and aligned bases: a thread moves four
// consecutive elements per access (16 bytes fp32, 8 bytes bf16), 16 threads a
// 64-element row of the tile.
template <typename S>
__global__ __launch_bounds__(256) void transpose_planes4(const S* __restrict__ in, S* __restrict__ out, int R, int C,
                                                         int tiles_r, int tiles_c) {
  __shared__ float tile[64][65];
  const int t = blockIdx.x;
  const int tc = t % tiles_c;
  const int rest = t / tiles_c;
  const int tr = rest % tiles_r;
  const int64_t plane = rest / tiles_r;
  const S* src = in + plane * R * C;
  S* dst = out + plane * R * C;
  const int r0 = tr * 64, c0 = tc * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {  // rows ty + 16 u, columns 4 tx .. 4 tx + 3 (all inside or all past C)
    const int r = r0 + ty + 16 * u, c = c0 + 4 * tx;
    const bool ok = r < R && c < C;
    v[u] = Io<S>::ld4(src, ok ? (int64_t)r * C + c : 0);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float* row = &tile[ty + 16 * u][4 * tx];
    row[0] = v[u].x;
    row[1] = v[u].y;
    row[2] = v[u].z;
    row[3] = v[u].w;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {  // output row c = c0 + ty + 16 u, columns r0 + 4 tx .. + 3
    const int c = c0 + ty + 16 * u, r = r0 + 4 * tx;
    if (c < C && r < R)
      Io<S>::st4(dst, (int64_t)c * R + r,
                 make_float4(tile[4 * tx][ty + 16 * u], tile[4 * tx + 1][ty + 16 * u], tile[4 * tx + 2][ty + 16 * u],
                             tile[4 * tx + 3][ty + 16 * u]));
  }
}

// Whole planes of at most kSmallPlane LDS slots (R rows of C + 1) through LDS: workgroup w
// transposes planes w, w + gridDim.x, ...  One element per thread and step, so
// global reads and writes are 256 contiguous bytes per wave (fp32) and the LDS
// rows, padded to C + 1, are read down a column without bank conflicts.
constexpr int kSmallPlane = 12288;  // 48 KB

template <typename S>
__global__ __launch_bounds__(256) void transpose_small(const S* __restrict__ in, S* __restrict__ out, int planes,
                                                       int R, int C) {
  extern __shared__ float tile_s[];  // R rows of C + 1
  const int n = R * C, ld = C + 1;
  const int tid = threadIdx.x;
  // (row, column) of element tid of the plane, and of output element tid, and the
  // steps of both for 256 elements
  const int r0 = tid / C, c0 = tid - r0 * C, dq = 256 / C, dr = 256 - dq * C;
  const int oc0 = tid / R, or0 = tid - oc0 * R, oq = 256 / R, orr = 256 - oq * R;
  for (int64_t pl = blockIdx.x; pl < planes; pl += gridDim.x) {
    const S* src = in + pl * n;
    S* dst = out + pl * n;
    // eight loads in flight per thread before any is written to LDS
    int r = r0, c = c0;
    for (int i0 = tid; i0 < n; i0 += 8 * 256) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 256;
        v[u] = i < n ? Io<S>::ld(src, i) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (i0 + u * 256 < n) tile_s[r * ld + c] = v[u];
        r += dq;
        c += dr;
        if (c >= C) {
          c -= C;
          ++r;
        }
      }
    }
    __syncthreads();
    int oc = oc0, orow = or0;
#pragma unroll 4
    for (int o = tid; o < n; o += 256) {  // output element o = oc * R + orow is input (orow, oc)
      Io<S>::st(dst, o, tile_s[orow * ld + oc]);
      oc += oq;
      orow += orr;
      if (orow >= R) {
        orow -= R;
        ++oc;
      }
    }
    __syncthreads();
  }
}

// V consecutive elements as floats, and back: 16 bytes (fp32 with V = 4, bf16
// with V = 8) or 8 bytes (bf16 with V = 4).
template <typename S, int V>
__device__ __forceinline__ void ld_vec(const S* p, int64_t i, float (&e)[V]) {
  if constexpr (V == 8) {
    static_assert(sizeof(S) == 2, "eight-element accesses are for bf16");
    const uint4 q = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      e[2 * k] = bf16_to_f32(w[k] & 0xffffu);
      e[2 * k + 1] = bf16_to_f32(w[k] >> 16);
    }
  } else {
    const float4 v = Io<S>::ld4(p, i);
    e[0] = v.x;
    e[1] = v.y;
    e[2] = v.z;
    e[3] = v.w;
  }
}
template <typename S, int V>
__device__ __forceinline__ void st_vec(S* p, int64_t i, const float (&e)[V]) {
  if constexpr (V == 8) {
    *reinterpret_cast<uint4*>(p + i) = make_uint4(bf16x2_rne(e[0], e[1]), bf16x2_rne(e[2], e[3]),
                                                  bf16x2_rne(e[4], e[5]), bf16x2_rne(e[6], e[7]));
  } else {
    Io<S>::st4(p, i, make_float4(e[0], e[1], e[2], e[3]));
  }
}

// The same for planes of n = R C elements with n a multiple of V and aligned bases:
// a workgroup takes P consecutive planes (one contiguous block) per step, and each
// access moves V consecutive elements (V = 4 fp32, 8 bf16: 16 bytes).  A thread's
// position in the block, as (plane, row, column) on the way in and (plane, column,
// row) on the way out, advances by a fixed step per 256 V elements without a
// division.
constexpr int kSmallGroup = 4096;  // elements per step: P = kSmallGroup / n planes, at least one

template <typename S, int V>
__global__ __launch_bounds__(256) void transpose_small4(const S* __restrict__ in, S* __restrict__ out, int planes,
                                                        int R, int C, int P) {
  extern __shared__ float tile_s[];  // P planes of R rows of C + 1
  const int n = R * C, ld = C + 1, pst = R * ld;
  const int tid = threadIdx.x;
  constexpr int kStep = V * 256;
  // element V tid and the step of kStep elements, in (plane, row, column) and in
  // (plane, column, row) of the output
  const int e0 = V * tid;
  const int ip = e0 / n, ir = (e0 - ip * n) / C, ic = e0 - ip * n - ir * C;
  const int sp = kStep / n, sr = (kStep - sp * n) / C, sc = kStep - sp * n - sr * C;
  const int op = ip, oc0 = (e0 - op * n) / R, or0 = e0 - op * n - oc0 * R;
  const int soc = (kStep - sp * n) / R, sor = kStep - sp * n - soc * R;
  const int64_t groups = ((int64_t)planes + P - 1) / P;
  for (int64_t g = blockIdx.x; g < groups; g += gridDim.x) {
    const int64_t pl0 = g * P;
    const int np = (int)((int64_t)planes - pl0 < P ? (int64_t)planes - pl0 : P);
    const int mv = np * n / V;  // V-element groups of this step
    const S* src = in + pl0 * n;
    S* dst = out + pl0 * n;
    int pl = ip, r = ir, c = ic;
    for (int q0 = tid; q0 < mv; q0 += 4 * 256) {
      float v[4][V];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u * 256;
        ld_vec<S, V>(src, q < mv ? (int64_t)V * q : 0, v[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (q0 + u * 256 < mv) {
          float* t = tile_s + pl * pst;
          int rr = r, cc = c;
#pragma unroll
          for (int k = 0; k < V; ++k) {  // n % V == 0: the V stay in one plane
            t[rr * ld + cc] = v[u][k];
            if (++cc == C) {
              cc = 0;
              ++rr;
            }
          }
        }
        c += sc;
        if (c >= C) {
          c -= C;
          ++r;
        }
        r += sr;
        if (r >= R) {
          r -= R;
          ++pl;
        }
        pl += sp;
      }
    }
    __syncthreads();
    int opl = op, oc = oc0, orow = or0;
    for (int q = tid; q < mv; q += 256) {  // output element oc R + orow of a plane is input (orow, oc)
      const float* t = tile_s + opl * pst;
      float e[V];
      int rr = orow, cc = oc;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        e[k] = t[rr * ld + cc];
        if (++rr == R) {
          rr = 0;
          ++cc;
        }
      }
      st_vec<S, V>(dst, (int64_t)V * q, e);
      orow += sor;
      if (orow >= R) {
        orow -= R;
        ++oc;
      }
      oc += soc;
      if (oc >= C) {
        oc -= C;
        ++opl;
      }
      opl += sp;
    }
    __syncthreads();
  }
}

template <typename S>
hipError_t launch_transpose(const S* in, S* out, int planes, int R, int C, hipStream_t stream) {
  const int64_t n = (int64_t)R * C;
  const uintptr_t am = sizeof(S) == 4 ? 15 : 7;
  if (n % 4 == 0 && (int64_t)R * (C + 1) <= kSmallPlane && !(((uintptr_t)in | (uintptr_t)out) & am)) {
    const int by_lds = (int)(kSmallPlane / ((int64_t)R * (C + 1)));
    const int by_size = (int)(kSmallGroup / n);
    const int P = by_size < 1 ? 1 : (by_size < by_lds ? by_size : by_lds);
    const int64_t groups = ((int64_t)planes + P - 1) / P;
    const int grid = groups < 4096 ? (int)groups : 4096;
    const size_t lds = (size_t)P * R * (C + 1) * sizeof(float);
    // bf16 planes of a multiple of 8 elements on 16-byte aligned bases: eight per access
    if (sizeof(S) == 2 && n % 8 == 0 && !(((uintptr_t)in | (uintptr_t)out) & 15))
      hipLaunchKernelGGL((transpose_small4<S, sizeof(S) == 2 ? 8 : 4>), dim3((unsigned)grid), dim3(256), lds, stream,
                         in, out, planes, R, C, P);
    else
      hipLaunchKernelGGL((transpose_small4<S, 4>), dim3((unsigned)grid), dim3(256), lds, stream, in, out, planes, R,
                         C, P);
    return hipGetLastError();
  }
  if ((int64_t)R * (C + 1) <= kSmallPlane) {
    const size_t lds = (size_t)R * (C + 1) * sizeof(float);
    const int grid = planes < 2048 ? planes : 2048;
    hipLaunchKernelGGL((transpose_small<S>), dim3((unsigned)grid), dim3(256), lds, stream, in, out, planes, R, C);
    return hipGetLastError();
  }
  const int tiles_r = (R + 63) / 64, tiles_c = (C + 63) / 64;
  const int64_t blocks = (int64_t)planes * tiles_r * tiles_c;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (R % 4 == 0 && C % 4 == 0 && !(((uintptr_t)in | (uintptr_t)out) & am))
    hipLaunchKernelGGL((transpose_planes4<S>), dim3((unsigned)blocks), dim3(256), 0, stream, in, out, R, C, tiles_r,
                       tiles_c);
  else
    hipLaunchKernelGGL((transpose_planes<S>), dim3((unsigned)blocks), dim3(256), 0, stream, in, out, R, C, tiles_r,
                       tiles_c);
  return hipGetLastError();
}

// Compute units of a device (0 if unknown), queried once per device.
inline int cu_count(int device) {
  static std::atomic<int> cache[64];
  if (device < 0 || device >= 64) return 0;
  int v = cache[device].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || v <= 0) return 0;
    cache[device].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Workgroups of `kernel` resident per CU (0 if unknown), queried once per kernel
// and device.
inline int resident_blocks(const void* kernel, int device) {
  struct Entry {
    const void* kernel;
    int device, blocks;
  };
  static std::mutex m;
  static Entry seen[64];
  static int nseen = 0;
  std::lock_guard<std::mutex> lk(m);
  for (int i = 0; i < nseen; ++i)
    if (seen[i].kernel == kernel && seen[i].device == device) return seen[i].blocks;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kWaves * 64, 0) != hipSuccess) {
    n = 0;
    (void)hipGetLastError();  // the query's own error; nothing was launched
  }
  if (nseen < 64) seen[nseen++] = Entry{kernel, device, n};
  return n;
}

template <typename S, int G, int T, bool VEC>
hipError_t launch_variant(const LaunchArgs& a, const Plan& plan, const Scratch& s) {
  Params p;
  p.x = a.x;
  p.dt = a.dt;
  p.A_log = a.A_log;
  p.dt_bias = a.dt_bias;
  p.Bs = a.Bs;
  p.Cs = a.Cs;
  p.Ds = a.Ds;
  p.y = a.y;
  p.prow = s.prow;
  p.pcol = s.pcol;
  p.xT = s.xT;
  p.pcolT = nullptr;
  p.B = (int)a.B;
  p.D = (int)a.D;
  p.H = (int)a.H;
  p.W = (int)a.W;
  p.N = (int)a.N;
  p.L = (int)(a.H * a.W);
  p.carries = s.carries;
  p.seg_chunks = plan.seg_chunks;
  p.nseg = plan.nseg;
  p.kdir = 0;
  p.K = a.K;
  p.R = a.R;
  p.wdt = a.wdt;
  p.Nt = (int)a.Nt;
  p.n0 = (int)a.n0;
  p.skip = a.skip ? 1 : 0;
  p.acc = a.acc ? 1 : 0;
  p.final_out = a.final_out ? 1 : 0;
  constexpr int NG = group_states<G, T>();
  const int64_t units = plan.blocks / plan.nseg;  // (batch, channel block) pairs
  // priority rotation for launches of at most one round (see the kernel)
  auto rotation = [&](const void* kernel, int64_t grid) {
    p.prio_ncu = 0;
    p.prio_levels = 1;
    const int ncu = cu_count(a.device);
    const int per = resident_blocks(kernel, a.device);
    if (ncu > 0 && per >= 2 && per <= 4 && grid <= (int64_t)ncu * per) {
      p.prio_ncu = ncu;
      p.prio_levels = per;
    }
  };
  if (plan.nseg == 1) {
    if (s.xT && !s.xT_given) {
      hipError_t e = launch_transpose<S>(static_cast<const S*>(a.x), static_cast<S*>(s.xT), (int)(a.B * a.D), p.H,
                                         p.W, a.stream);
      if (e != hipSuccess) return e;
    }
    const void* kf = reinterpret_cast<const void*>(&ss2d_forward_kernel<S, G, T, NG, VEC, kFused>);
    rotation(kf, units);
    hipLaunchKernelGGL((ss2d_forward_kernel<S, G, T, NG, VEC, kFused>), dim3((unsigned)units), dim3(kWaves * 64), 0,
                       a.stream, p);
    return hipGetLastError();
  }
  if constexpr (VEC) {
    // carry pass over every segment but the last, then one launch per direction in
    // merge order (column pair, then row pair; each reads what the previous wrote);
    // with transposed copies: x before everything, the column plane before
    // direction 2
    const int planes = (int)(a.B * a.D);
    if (s.xT && !s.xT_given) {
      hipError_t e = launch_transpose<S>(static_cast<const S*>(a.x), static_cast<S*>(s.xT), planes, p.H, p.W, a.stream);
      if (e != hipSuccess) return e;
    }
    rotation(reinterpret_cast<const void*>(&ss2d_forward_kernel<S, G, T, NG, VEC, kCarry>), units * (plan.nseg - 1));
    hipLaunchKernelGGL((ss2d_forward_kernel<S, G, T, NG, VEC, kCarry>), dim3((unsigned)(units * (plan.nseg - 1))),
                       dim3(kWaves * 64), 0, a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int order4[4] = {1, 3, 0, 2}, order2[2] = {0, 2};
    const int* order = a.K == 4 ? order4 : order2;
    rotation(reinterpret_cast<const void*>(&ss2d_forward_kernel<S, G, T, NG, VEC, kSegment>), units * plan.nseg);
    for (int i = 0; i < a.K; ++i) {
      const int k = order[i];
      p.kdir = k;
      if (k == 2 && s.pcolT) {
        // the column plane is complete after direction 3; as pixels [W][H] -> [H][W]
        e = launch_transpose<float>(s.pcol, s.pcolT, planes, p.W, p.H, a.stream);
        if (e != hipSuccess) return e;
        p.pcolT = s.pcolT;
      }
      hipLaunchKernelGGL((ss2d_forward_kernel<S, G, T, NG, VEC, kSegment>), dim3((unsigned)(units * plan.nseg)),
                         dim3(kWaves * 64), 0, a.stream, p);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return hipErrorInvalidValue;  // segments are planned only for rows aligned for the DMA copy
}

template <typename S, int G, int T>
hipError_t launch_gt(const LaunchArgs& a, const Plan& plan, const Scratch& s) {
  if (plan.vec) return launch_variant<S, G, T, true>(a, plan, s);
  return launch_variant<S, G, T, false>(a, plan, s);
}

template <typename S, int G, int T>
size_t lds_bytes_for(bool vec) {
  return vec ? (size_t)Layout<S, G, T, group_states<G, T>(), true>::kBytes
             : (size_t)Layout<S, G, T, group_states<G, T>(), false>::kBytes;
}

template <typename S>
size_t lds_bytes_s(int G, int T, bool vec) {
  if (T == 8) return G == 32 ? lds_bytes_for<S, 32, 8>(vec) : lds_bytes_for<S, 64, 8>(vec);
  return G == 16 ? lds_bytes_for<S, 16, 16>(vec) : G == 32 ? lds_bytes_for<S, 32, 16>(vec) : lds_bytes_for<S, 64, 16>(vec);
}

}  // namespace

// Launchers of the compiled variants, one compilation unit each (steps per lane
// T = 16 for 16/32/64 lanes, T = 8 for 32/64 lanes).
hipError_t launch_f32_t16(const LaunchArgs& a, const Plan& plan, const Scratch& s);
hipError_t launch_f32_t8(const LaunchArgs& a, const Plan& plan, const Scratch& s);
hipError_t launch_bf16_t16(const LaunchArgs& a, const Plan& plan, const Scratch& s);
hipError_t launch_bf16_t8(const LaunchArgs& a, const Plan& plan, const Scratch& s);

}  // namespace ss2d
