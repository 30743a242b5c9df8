// SS2D forward kernels for gfx950 (CDNA4, wave64).
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
// does the four directions one after the other, in the order 0, 2, 1, 3.
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
//     staged through LDS in groups of NG states: while the lanes work through
//     one group, each thread holds its share of the next group in registers
//     (coalesced 16-byte loads issued a whole group ahead), writes it to the
//     other LDS buffer, and the workgroup synchronises once per group.  Lanes
//     read their steps back with conflict-free 16-byte LDS loads.
//   * Merge: directions 0 and 2 accumulate into a row-major fp32 plane (y itself
//     for fp32 output), directions 1 and 3 into a column-major fp32 plane, so
//     every access is contiguous along the lane's steps; a final pass adds the
//     column plane into y through 32x32 LDS-tiled transposes.  The order of
//     additions is fixed, y = (y0 + y2) + (y1 + y3): deterministic, no atomics.
//     (Four separate store-only planes summed at the end measured slower.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ss2d_internal.h"

namespace ss2d {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxN = 16;
constexpr int kWaves = 4;

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

template <typename S>
struct Io;

template <>
struct Io<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ float4 ld4(const float* p, int64_t i) {  // i % 4 == 0
    return *reinterpret_cast<const float4*>(p + i);
  }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
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

// One level of the inclusive prefix combine of affine maps h -> A h + B.  The
// DPP source lane is earlier in the sequence.  Fused forms:
//   B += dpp(B) * A   (v_fmac_f32_dpp),   A = dpp(A) * A   (v_mul_f32_dpp).
// Lanes whose source is out of range (or whose row is masked off) are not
// written, which is the identity map.  s_nop 1 gives the two wait states a DPP
// read needs after a VALU write of its source.
#define SS2D_SCAN_LEVEL(DPP)                                                     \
  asm volatile("s_nop 1\n\t"                                                     \
               "v_fmac_f32_dpp %1, %1, %0 " DPP " bank_mask:0xf\n\t"             \
               "v_mul_f32_dpp %0, %0, %0 " DPP " bank_mask:0xf"                  \
               : "+v"(A), "+v"(B))

// Inclusive scan inside groups of G lanes (G = 16, 32 or 64).
template <int G>
__device__ __forceinline__ void scan_inclusive(float& A, float& B) {
  SS2D_SCAN_LEVEL("row_shr:1 row_mask:0xf");
  SS2D_SCAN_LEVEL("row_shr:2 row_mask:0xf");
  SS2D_SCAN_LEVEL("row_shr:4 row_mask:0xf");
  SS2D_SCAN_LEVEL("row_shr:8 row_mask:0xf");
  if constexpr (G >= 32) SS2D_SCAN_LEVEL("row_bcast:15 row_mask:0xa");
  if constexpr (G >= 64) SS2D_SCAN_LEVEL("row_bcast:31 row_mask:0xc");
}

// State entering this lane's steps: the previous lane's inclusive map applied
// to the group's carried state, h = A_prev * carry + B_prev; the group's first
// lane takes the carry itself.
template <int G>
__device__ __forceinline__ float incoming_state(float A, float B, float carry, int seg) {
  float t = carry;
  float h;
  if constexpr (G == 16) {
    asm volatile("s_nop 1\n\tv_mul_f32_dpp %0, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf" : "+v"(t) : "v"(A));
    h = t;
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf" : "+v"(h) : "v"(B));
  } else {
    asm volatile("s_nop 1\n\tv_mul_f32_dpp %0, %1, %0 wave_shr:1 row_mask:0xf bank_mask:0xf" : "+v"(t) : "v"(A));
    h = t;
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %0 wave_shr:1 row_mask:0xf bank_mask:0xf" : "+v"(h) : "v"(B));
  }
  return seg == 0 ? carry : h;
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
  int B, D, H, W, N, L;
};

// Compile-time shape of one kernel variant: G lanes per sequence chunk, T steps
// per lane in full chunks, NG states per Bs/Cs staging group.
template <int G, int T, int NG>
struct Cfg {
  static constexpr int kChans = kWaves * (64 / G);  // channels per workgroup
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kSS = seg_stride<T>();
  static constexpr int kArr = G * kSS;               // LDS floats of one staged (state, B or C)
  static constexpr int kBuf = NG * 2 * kArr;         // one staging buffer
  static constexpr int kLds = 2 * kBuf + 2 * kChans * kMaxN + 2 * kChans;  // floats
};

// Walk index (row-major index for row walks, w*H+h for column walks) of step l.
__device__ __forceinline__ int walk_index(bool rev, int l, int L) { return rev ? (L - 1 - l) : l; }

// dt and u for T consecutive steps from l0.  FULL: all steps exist (no bounds
// checks).  VEC: rows are aligned for 16-byte (fp32) / 8-byte (bf16) loads.
template <typename S, int T, bool VEC, bool FULL>
__device__ __forceinline__ void load_inputs(const S* dtrow, const S* xrow, bool rev, bool col, int l0, int L, int H,
                                            int W, float (&dtv)[T], float (&uv)[T]) {
  constexpr bool V4 = VEC && FULL && (T % 4 == 0);
  if constexpr (V4) {
#pragma unroll
    for (int i = 0; i < T; i += 4) {
      const float4 q = Io<S>::ld4(dtrow, l0 + i);
      dtv[i] = q.x; dtv[i + 1] = q.y; dtv[i + 2] = q.z; dtv[i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i) dtv[i] = (FULL || l0 + i < L) ? Io<S>::ld(dtrow, l0 + i) : 0.f;
  }
  if (!col) {
    if constexpr (V4) {
      if (!rev) {
#pragma unroll
        for (int i = 0; i < T; i += 4) {
          const float4 q = Io<S>::ld4(xrow, l0 + i);
          uv[i] = q.x; uv[i + 1] = q.y; uv[i + 2] = q.z; uv[i + 3] = q.w;
        }
      } else {
        const int s_lo = L - l0 - T;  // walk indices s_lo .. s_lo+T-1; step i is at s_lo+T-1-i
#pragma unroll
        for (int i = 0; i < T; i += 4) {
          const float4 q = Io<S>::ld4(xrow, s_lo + i);
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

// One state n of one chunk; this lane's staged B/C are at Bst/Cst.
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
  float a[T], bb[T];
  float Bl = 0.f;
#pragma unroll
  for (int i = 0; i < T; ++i) {
    a[i] = __builtin_amdgcn_exp2f(delta[i] * A2n);
    bb[i] = du[i] * Bv[i];
    Bl = fmaf(a[i], Bl, bb[i]);
  }
  float Al = __builtin_amdgcn_exp2f(A2n * sdelta);
  scan_inclusive<G>(Al, Bl);
  float h = incoming_state<G>(Al, Bl, *carry_slot, seg);
#pragma unroll
  for (int i = 0; i < T; ++i) {
    h = fmaf(a[i], h, bb[i]);
    yv[i] = fmaf(Cv[i], h, yv[i]);
  }
  if (seg == G - 1) *carry_slot = h;
}

// Writes (or adds) a lane's outputs of T consecutive steps into its plane.
template <int T, bool VEC, bool FULL>
__device__ __forceinline__ void store_outputs(float* plane, bool rev, bool add, int l0, int L, const float (&yv)[T]) {
  if constexpr (VEC && FULL && (T % 4 == 0)) {
    const int s_lo = rev ? L - l0 - T : l0;
#pragma unroll
    for (int i = 0; i < T; i += 4) {
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

// Bs/Cs staging of one group: NG states x {B, C} x (G lanes x TT steps) for the
// chunk at c0, states n0.. ; thread-private share in float4 registers.
template <typename S, int G, int T, int NG, int TT, bool VEC, bool FULL>
struct Stager {
  static constexpr int kNth = Cfg<G, T, NG>::kThreads;
  static constexpr int kPer = G * TT / 4;        // float4 per (state, array)
  static constexpr int kF4 = NG * 2 * kPer;      // float4 per group
  static constexpr int kQ = (kF4 + kNth - 1) / kNth;
  static constexpr int kSS = seg_stride<TT>();
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
    constexpr int kArr = Cfg<G, T, NG>::kArr;
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

// A remainder chunk of G*TT steps (TT < T, possibly ragged), staged synchronously.
// Out of line, with plain arguments: it runs a few times per direction, and
// inlining it would make the register allocator budget its arrays on top of the
// main loop's.
template <typename S, int G, int T, int NG, int TT, bool VEC>
__device__ __noinline__ void tail_chunk(int tid, int seg, int dl, bool dvalid, float* smem, const S* dtrow,
                                        const S* xrow, const S* Bbase, const S* Cbase, float* plane, bool rev,
                                        bool col, bool add, float bias, float dsk, int c0, int L, int H, int W,
                                        int N) {
  Lane ln;
  ln.tid = tid;
  ln.seg = seg;
  ln.dl = dl;
  ln.dvalid = dvalid;
  using C = Cfg<G, T, NG>;
  float* a2s = smem + 2 * C::kBuf;
  float* carry = a2s + C::kChans * kMaxN;
  constexpr int SS = seg_stride<TT>();
  const int l0 = c0 + ln.seg * TT;
  float dtv[TT], uv[TT];
  load_inputs<S, TT, VEC, false>(dtrow, xrow, rev, col, l0, L, H, W, dtv, uv);
  float delta[TT], du[TT], yv[TT];
  const float sdelta = prepare_steps<TT>(dtv, uv, bias, dsk, ln.dvalid, L - l0, delta, du, yv);
  for (int n0 = 0; n0 < N; n0 += NG) {
    Stager<S, G, T, NG, TT, VEC, false> st;
    st.fetch(Bbase, Cbase, ln.tid, n0, N, c0, L);
    st.commit(smem, ln.tid);
    __syncthreads();
#pragma unroll 1
    for (int nn = 0; nn < NG; ++nn) {
      const int n = n0 + nn;
      if (n < N)
        state_step<G, TT>(smem + (nn * 2) * C::kArr + ln.seg * SS, smem + (nn * 2 + 1) * C::kArr + ln.seg * SS,
                          a2s[ln.dl * kMaxN + n], carry + ln.dl * kMaxN + n, ln.seg, delta, du, sdelta, yv);
    }
    __syncthreads();
  }
  if (ln.dvalid) store_outputs<TT, VEC, false>(plane, rev, add, l0, L, yv);
}

template <typename S, int G, int T, int NG, bool VEC>
__global__ __launch_bounds__(kWaves * 64, 3) void ss2d_forward_kernel(Params p) {
  using C = Cfg<G, T, NG>;
  constexpr int CH = C::kChans;
  constexpr int NTH = C::kThreads;
  constexpr int SS = C::kSS;
  extern __shared__ float smem[];
  float* a2s = smem + 2 * C::kBuf;
  float* carry = a2s + CH * kMaxN;
  float* biass = carry + CH * kMaxN;
  float* dss = biass + CH;

  // Work id: consecutive ids (same batch, neighbouring channel blocks, which share
  // Bs/Cs) stay on one XCD; workgroups are dealt round-robin over the 8 XCDs.
  const int nb = gridDim.x;
  const int xcd = blockIdx.x & 7, bslot = blockIdx.x >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int work = (xcd < rem) ? xcd * (per + 1) + bslot : rem * (per + 1) + (xcd - rem) * per + bslot;

  Lane ln;
  ln.tid = threadIdx.x;
  const int lane = ln.tid & 63, wave = ln.tid >> 6;
  ln.seg = lane % G;
  ln.dl = wave * (64 / G) + lane / G;
  const int nbd = (p.D + CH - 1) / CH;
  ln.b = work / nbd;
  ln.d0 = (work - ln.b * nbd) * CH;
  ln.dvalid = ln.d0 + ln.dl < p.D;
  ln.dsafe = ln.dvalid ? ln.d0 + ln.dl : 0;
  const int L = p.L, N = p.N, H = p.H, W = p.W;
  const int64_t plane_off = ((int64_t)ln.b * p.D + ln.dsafe) * L;
  const S* xrow = static_cast<const S*>(p.x) + plane_off;

#pragma unroll 1
  for (int kk = 0; kk < 4; ++kk) {
    const int k = (kk == 0) ? 0 : (kk == 1) ? 2 : (kk == 2) ? 1 : 3;  // row pair, then column pair
    // per-direction parameters of the block's channels
    for (int i = ln.tid; i < CH * kMaxN; i += NTH) {
      const int dd = i / kMaxN, n = i - dd * kMaxN;
      const int dg = ln.d0 + dd;
      float v = 0.f;
      if (dg < p.D && n < N) v = -expf(p.A_log[(int64_t)(k * p.D + dg) * N + n]) * kLog2e;
      a2s[i] = v;
      carry[i] = 0.f;
    }
    for (int i = ln.tid; i < CH; i += NTH) {
      const int dg = ln.d0 + i;
      biass[i] = dg < p.D ? p.dt_bias[k * p.D + dg] : 0.f;
      dss[i] = dg < p.D ? p.Ds[k * p.D + dg] : 0.f;
    }
    __syncthreads();

    const bool rev = k >= 2, col = (k & 1) != 0, add = k >= 2;
    float* plane = (col ? p.pcol : p.prow) + plane_off;
    const S* dtrow = static_cast<const S*>(p.dt) + ((int64_t)(ln.b * 4 + k) * p.D + ln.dsafe) * L;
    const S* Bbase = static_cast<const S*>(p.Bs) + (int64_t)(ln.b * 4 + k) * N * L;
    const S* Cbase = static_cast<const S*>(p.Cs) + (int64_t)(ln.b * 4 + k) * N * L;
    const float bias = biass[ln.dl];
    const float dsk = dss[ln.dl];

    // ---------------- full chunks, Bs/Cs staged one group ahead
    constexpr int GT = G * T;
    const int nmain = L / GT;
    const int ngrp = (N + NG - 1) / NG;
    if (nmain > 0) {
      float dtn[T], un[T];
      Stager<S, G, T, NG, T, VEC, true> st;
      st.fetch(Bbase, Cbase, ln.tid, 0, N, 0, L);
      st.commit(smem, ln.tid);
      __syncthreads();
      int gflat = 0;
      for (int c = 0; c < nmain; ++c) {
        float delta[T], du[T], yv[T];
        // dt/x of this chunk (a prefetch a chunk ahead would cost 2*T registers and
        // drop the kernel to two waves per SIMD, which measured slower)
        load_inputs<S, T, VEC, true>(dtrow, xrow, rev, col, c * GT + ln.seg * T, L, H, W, dtn, un);
        const float sdelta = prepare_steps<T>(dtn, un, bias, dsk, ln.dvalid, T, delta, du, yv);
        for (int g = 0; g < ngrp; ++g, ++gflat) {
          const bool more_states = g + 1 < ngrp;
          const bool has_next = more_states || c + 1 < nmain;
          if (has_next) st.fetch(Bbase, Cbase, ln.tid, more_states ? (g + 1) * NG : 0, N,
                                 (more_states ? c : c + 1) * GT, L);
          const float* base = smem + (gflat & 1) * C::kBuf;
#pragma unroll 1
          for (int nn = 0; nn < NG; ++nn) {
            const int n = g * NG + nn;
            if (n < N)
              state_step<G, T>(base + (nn * 2) * C::kArr + ln.seg * SS, base + (nn * 2 + 1) * C::kArr + ln.seg * SS,
                               a2s[ln.dl * kMaxN + n], carry + ln.dl * kMaxN + n, ln.seg, delta, du, sdelta, yv);
          }
          if (has_next) st.commit(smem + ((gflat + 1) & 1) * C::kBuf, ln.tid);
          __syncthreads();
        }
        if (ln.dvalid) store_outputs<T, VEC, true>(plane, rev, add, c * GT + ln.seg * T, L, yv);
      }
    }

    // ---------------- remainder chunks (fewer steps per lane)
    int c0 = nmain * GT;
    while (L - c0 >= G * 8) {
      tail_chunk<S, G, T, NG, 8, VEC>(ln.tid, ln.seg, ln.dl, ln.dvalid, smem, dtrow, xrow, Bbase, Cbase, plane, rev, col, add, bias, dsk, c0, L, H, W, N);
      c0 += G * 8;
    }
    if (L - c0 >= G * 4) {
      tail_chunk<S, G, T, NG, 4, VEC>(ln.tid, ln.seg, ln.dl, ln.dvalid, smem, dtrow, xrow, Bbase, Cbase, plane, rev, col, add, bias, dsk, c0, L, H, W, N);
      c0 += G * 4;
    }
    if (L - c0 >= G * 2) {
      tail_chunk<S, G, T, NG, 2, VEC>(ln.tid, ln.seg, ln.dl, ln.dvalid, smem, dtrow, xrow, Bbase, Cbase, plane, rev, col, add, bias, dsk, c0, L, H, W, N);
      c0 += G * 2;
    }
    while (c0 < L) {
      tail_chunk<S, G, T, NG, 1, VEC>(ln.tid, ln.seg, ln.dl, ln.dvalid, smem, dtrow, xrow, Bbase, Cbase, plane, rev, col, add, bias, dsk, c0, L, H, W, N);
      c0 += G;
    }
    __syncthreads();  // this direction's plane writes are complete and visible to the block
  }

  // ---------------- y = row plane + transpose(column plane), 32x32 LDS tiles
  float* tile = smem;  // [32][33]
  S* y = static_cast<S*>(p.y);
  const int tx = ln.tid & 31, ty = ln.tid >> 5;
  for (int dd = 0; dd < CH; ++dd) {
    const int dg = ln.d0 + dd;
    if (dg >= p.D) break;
    const int64_t off = ((int64_t)ln.b * p.D + dg) * L;
    const float* pc = p.pcol + off;
    const float* pr = p.prow + off;
    for (int h0 = 0; h0 < H; h0 += 32) {
      for (int w0 = 0; w0 < W; w0 += 32) {
        for (int r = ty; r < 32; r += NTH / 32) {
          const int w = w0 + r, h = h0 + tx;
          if (w < W && h < H) tile[r * 33 + tx] = pc[(int64_t)w * H + h];
        }
        __syncthreads();
        for (int r = ty; r < 32; r += NTH / 32) {
          const int h = h0 + r, w = w0 + tx;
          if (w < W && h < H) {
            const int64_t pix = (int64_t)h * W + w;
            Io<S>::st(y, off + pix, pr[pix] + tile[tx * 33 + r]);
          }
        }
        __syncthreads();
      }
    }
  }
}

template <int G>
struct Variant;
// Steps per lane and states per staging group, chosen so one staging buffer holds
// NG*2*G*T floats ~ 8 K (LDS ~ 40 KB per workgroup) and each thread prefetches
// at most 4 float4 per group.
template <>
struct Variant<16> { static constexpr int T = 16, NG = 8; };
template <>
struct Variant<32> { static constexpr int T = 16, NG = 4; };
template <>
struct Variant<64> { static constexpr int T = 16, NG = 2; };

template <typename S, int G, bool VEC>
hipError_t launch_variant(const LaunchArgs& a, const Plan& plan, float* const planes[2]) {
  Params p;
  p.x = a.x;
  p.dt = a.dt;
  p.A_log = a.A_log;
  p.dt_bias = a.dt_bias;
  p.Bs = a.Bs;
  p.Cs = a.Cs;
  p.Ds = a.Ds;
  p.y = a.y;
  p.prow = planes[0];
  p.pcol = planes[1];
  p.B = (int)a.B;
  p.D = (int)a.D;
  p.H = (int)a.H;
  p.W = (int)a.W;
  p.N = (int)a.N;
  p.L = (int)(a.H * a.W);
  auto kern = ss2d_forward_kernel<S, G, Variant<G>::T, Variant<G>::NG, VEC>;
  hipLaunchKernelGGL(kern, dim3((unsigned)plan.blocks), dim3(kWaves * 64), plan.lds_bytes, a.stream, p);
  return hipGetLastError();
}

template <typename S, int G>
hipError_t launch_g(const LaunchArgs& a, const Plan& plan, float* const planes[2]) {
  if ((a.H * a.W) % 4 == 0) return launch_variant<S, G, true>(a, plan, planes);
  return launch_variant<S, G, false>(a, plan, planes);
}

template <typename S>
hipError_t launch_s(const LaunchArgs& a, const Plan& plan, float* const planes[2]) {
  switch (plan.lanes_per_seq) {
    case 16: return launch_g<S, 16>(a, plan, planes);
    case 32: return launch_g<S, 32>(a, plan, planes);
    default: return launch_g<S, 64>(a, plan, planes);
  }
}

template <int G>
size_t lds_bytes_for() {
  constexpr int f = Cfg<G, Variant<G>::T, Variant<G>::NG>::kLds;
  return sizeof(float) * (size_t)(f > 32 * 33 ? f : 32 * 33);
}

}  // namespace

Plan make_plan(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int lanes_override) {
  (void)N;
  Plan pl;
  const int64_t L = H * W;
  int G = L < 512 ? 16 : 32;
  if (lanes_override == 16 || lanes_override == 32 || lanes_override == 64) G = lanes_override;
  pl.lanes_per_seq = G;
  pl.waves = kWaves;
  pl.chans_per_block = kWaves * (64 / G);
  pl.blocks = B * ((D + pl.chans_per_block - 1) / pl.chans_per_block);
  pl.lds_bytes = G == 16 ? lds_bytes_for<16>() : G == 32 ? lds_bytes_for<32>() : lds_bytes_for<64>();
  pl.scratch_bytes = (size_t)(dtype == 0 ? 1 : 2) * (size_t)(B * D * L) * sizeof(float);
  return pl;
}

hipError_t launch_forward(const LaunchArgs& a, const Plan& plan, float* scratch) {
  const int64_t plane = a.B * a.D * a.H * a.W;
  // planes: row-major (directions 0, 2), column-major (directions 1, 3)
  if (a.dtype == 0) {
    float* const planes[2] = {static_cast<float*>(a.y), scratch};
    return launch_s<float>(a, plan, planes);
  }
  float* const planes[2] = {scratch + plane, scratch};
  return launch_s<uint16_t>(a, plan, planes);
}

}  // namespace ss2d
