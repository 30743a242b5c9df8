// SS2D forward kernels for gfx950 (CDNA4, wave64).
//
// What is computed (page [SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现"):
//   §3.1/§4  four scan sequences of the H x W map: row-major, column-major and
//            both reversed; step l of direction k visits pixel pix_k(l);
//   §3.2     per channel c = k*D + d and state n:
//              delta_l = softplus(dt_l + dt_bias[c]),  A = -exp(A_log[c, n]),
//              h_l = exp(delta_l * A) * h_{l-1} + delta_l * Bs[n, l] * u_l,  h_{-1} = 0,
//              out_l = sum_n Cs[n, l] * h_l + Ds[c] * u_l,   u_l = x[pix_k(l)];
//   §3.3     y[p] = sum over the four directions of out at the step visiting p.
//
// How it runs (one workgroup = one batch b and a block of channels, all four
// directions, directions processed one after the other):
//   * A sequence (b, k, d) is cut into chunks of G*T steps; G lanes ("a group")
//     each own T consecutive steps of the chunk.  Several groups (channels)
//     share a wave when G < 64.
//   * Per state n: each lane turns its T steps into decay/input pairs
//     (a_i = 2^(delta_i * A * log2 e), b_i = delta_i u_i B_i), folds them into one
//     affine map h -> A_lane h + B_lane, the group combines the maps with an
//     inclusive DPP prefix scan (row_shr 1/2/4/8, row_bcast 15/31), the running
//     state carried from the previous chunk enters through the exclusive prefix,
//     and each lane replays its T steps from its exact incoming state, adding
//     C_i h_i into its outputs.  The pair combine (A1,B1) then (A2,B2) =
//     (A2 A1, A2 B1 + B2) is associative, so this equals the sequential loop up
//     to rounding.
//   * Bs/Cs of the chunk for state n are staged once per workgroup in LDS
//     (shared by every channel of the block, double-buffered over n) and read
//     back with 16-byte LDS loads on a padded, bank-conflict-free layout.
//   * The four directional outputs are merged into an fp32 plane per channel,
//     direction after direction (fixed order, no atomics, deterministic): in
//     LDS when it fits, else in an fp32 global buffer.  The plane is written to
//     y once, rounded to the storage type once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ss2d_internal.h"

namespace ss2d {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxN = 16;
constexpr int kStageStride = 20;  // LDS floats per lane segment, enough for T = 16

// LDS floats per lane segment for T steps: multiples of 4 get a stride whose
// 16-byte slot count is odd (conflict-free b128 reads across lanes).
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
  // four values at i (i % 4 == 0, 16-byte aligned)
  static __device__ __forceinline__ float4 ld4(const float* p, int64_t i) {
    return *reinterpret_cast<const float4*>(p + i);
  }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
  static __device__ __forceinline__ void st4(float* p, int64_t i, float4 v) {
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
  static __device__ __forceinline__ void st4(uint16_t* p, int64_t i, float4 v) {
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
    *reinterpret_cast<uint2*>(p + i) = o;
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

// One level of the inclusive prefix combine of affine maps h -> A h + B across
// lanes.  The lane CTRL points at is earlier in the sequence; lanes without a
// source (or masked rows) read the identity map (1, 0).
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ void scan_level(float& A, float& B) {
  const float Ap = __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(A), CTRL, RM, 0xF, false));
  const float Bp = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(B), CTRL, RM, 0xF, false));
  B = fmaf(A, Bp, B);
  A = A * Ap;
}

// Inclusive scan inside groups of G lanes (G = 16, 32 or 64).
template <int G>
__device__ __forceinline__ void scan_inclusive(float& A, float& B) {
  scan_level<0x111>(A, B);  // row_shr:1
  scan_level<0x112>(A, B);  // row_shr:2
  scan_level<0x114>(A, B);  // row_shr:4
  scan_level<0x118>(A, B);  // row_shr:8
  if constexpr (G >= 32) scan_level<0x142, 0xA>(A, B);  // row_bcast:15 into rows 1 and 3
  if constexpr (G >= 64) scan_level<0x143, 0xC>(A, B);  // row_bcast:31 into rows 2 and 3
}

// Value of the previous lane of the group (identity for the group's first lane).
template <int G>
__device__ __forceinline__ void shift_exclusive(float A, float B, int seg, float& Ae, float& Be) {
  if constexpr (G == 16) {
    Ae = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(A), 0x111, 0xF, 0xF, false));
    Be = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(B), 0x111, 0xF, 0xF, false));
  } else {
    Ae = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(A), 0x138, 0xF, 0xF, false));
    Be = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(B), 0x138, 0xF, 0xF, false));
    if constexpr (G == 32) {
      if (seg == 0) {
        Ae = 1.0f;
        Be = 0.0f;
      }
    }
  }
}

// ------------------------------------------------------------------ kernel
struct Params {
  const void* x;
  const void* dt;
  const float* A_log;
  const float* dt_bias;
  const void* Bs;
  const void* Cs;
  const float* Ds;
  void* y;
  float* gplane;  // fp32 merge plane in global memory (global-plane variant)
  int B, D, H, W, N, L;
  int vec;  // L % 4 == 0: rows are 16-byte (fp32) / 8-byte (bf16) aligned
};

template <int G, int NW>
struct Shape {
  static constexpr int kGroupsPerWave = 64 / G;
  static constexpr int kChans = NW * kGroupsPerWave;  // channels per workgroup
  static constexpr int kThreads = NW * 64;
};

// LDS layout (floats): stage[2 buffers][B, C][G * 20] | a2[chans][16] |
// carry[chans][16] | bias[chans] | dskip[chans] | plane[chans][L] (LDS plane only).
template <int G, int NW>
__host__ __device__ constexpr int lds_fixed_floats() {
  return 4 * G * kStageStride + 2 * Shape<G, NW>::kChans * kMaxN + 2 * Shape<G, NW>::kChans;
}

struct Lane {
  int tid, seg, dl, b, d, d0;
  bool dvalid;
};

// Pixel visited at step l of direction k (row-major walk for even k, column-major
// walk for odd k, reversed for k >= 2), for T consecutive steps starting at l0.
template <int T>
__device__ __forceinline__ void pixels_of(int k, int l0, int L, int H, int W, int (&px)[T]) {
  if ((k & 1) == 0) {
#pragma unroll
    for (int i = 0; i < T; ++i) px[i] = (k == 0) ? (l0 + i) : (L - 1 - l0 - i);
    return;
  }
  // column walk: step s = w*H + h; forward for k = 1, backward for k = 3
  const int s0 = (k == 1) ? l0 : (L - 1 - l0);
  int w = s0 / H;
  int h = s0 - w * H;
#pragma unroll
  for (int i = 0; i < T; ++i) {
    px[i] = h * W + w;
    if (k == 1) {
      ++h;
      if (h == H) { h = 0; ++w; }
    } else {
      --h;
      if (h < 0) { h = H - 1; --w; }
    }
  }
}

template <typename S, int G, int NW, bool LDS_PLANE, int T>
__device__ __forceinline__ void run_chunk(const Params& p, const Lane& ln, float* smem, float* plane_row,
                                          int k, int c0) {
  constexpr int SS = seg_stride<T>();
  constexpr int NTH = Shape<G, NW>::kThreads;
  constexpr int CH = Shape<G, NW>::kChans;
  constexpr int NSLOT = 2 * G * T / 4;          // float4 slots of one state's B and C chunk
  constexpr int Q = (NSLOT + NTH - 1) / NTH;    // slots per thread
  float* stage = smem;
  float* a2s = stage + 4 * G * kStageStride;
  float* carry = a2s + CH * kMaxN;
  float* biass = carry + CH * kMaxN;
  float* dss = biass + CH;

  const int L = p.L, N = p.N;
  const bool vec = p.vec != 0;
  const int l0 = c0 + ln.seg * T;
  const int dsafe = ln.dvalid ? ln.d : 0;

  // ---- per-step inputs of this lane: delta, delta*u, output init D*u
  const S* dtrow = static_cast<const S*>(p.dt) + ((int64_t)(ln.b * 4 + k) * p.D + dsafe) * L;
  const S* xrow = static_cast<const S*>(p.x) + ((int64_t)ln.b * p.D + dsafe) * L;
  int px[T];
  pixels_of<T>(k, l0, L, p.H, p.W, px);
  const float bias = biass[ln.dl];
  const float dsk = dss[ln.dl];
  float delta[T], du[T], yv[T];
  float sdelta = 0.f;
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const bool valid = ln.dvalid && (l0 + i < L);
    float dtv = 0.f, uv = 0.f;
    if (valid) {
      dtv = Io<S>::ld(dtrow, l0 + i);
      uv = Io<S>::ld(xrow, px[i]);
    }
    delta[i] = valid ? softplus_f32(dtv + bias) : 0.f;
    du[i] = delta[i] * uv;
    yv[i] = dsk * uv;
    sdelta += delta[i];
  }

  // ---- B/C staging, double-buffered over n
  const S* Bbase = static_cast<const S*>(p.Bs) + (int64_t)(ln.b * 4 + k) * N * L;
  const S* Cbase = static_cast<const S*>(p.Cs) + (int64_t)(ln.b * 4 + k) * N * L;
  float4 pre[Q];
  auto fetch = [&](int n) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int slot = ln.tid + q * NTH;
      if (slot < NSLOT) {
        const int arr = slot / (G * T / 4);
        const int j = (slot - arr * (G * T / 4)) * 4;
        const S* row = (arr == 0 ? Bbase : Cbase) + (int64_t)n * L;
        pre[q] = ld4_guarded<S>(row, c0 + j, L, vec);
      }
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int slot = ln.tid + q * NTH;
      if (slot < NSLOT) {
        const int arr = slot / (G * T / 4);
        const int j = (slot - arr * (G * T / 4)) * 4;
        float* dst = stage + (buf * 2 + arr) * (G * kStageStride) + (j / T) * SS + (j % T);
        *reinterpret_cast<float4*>(dst) = pre[q];
      }
    }
  };

  fetch(0);
  commit(0);
  __syncthreads();
  for (int n = 0; n < N; ++n) {
    const int buf = n & 1;
    if (n + 1 < N) fetch(n + 1);
    const float* Bst = stage + (buf * 2 + 0) * (G * kStageStride) + ln.seg * SS;
    const float* Cst = stage + (buf * 2 + 1) * (G * kStageStride) + ln.seg * SS;
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
    const float A2n = a2s[ln.dl * kMaxN + n];
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
    float Ae, Be;
    shift_exclusive<G>(Al, Bl, ln.seg, Ae, Be);
    float h = fmaf(Ae, carry[ln.dl * kMaxN + n], Be);
#pragma unroll
    for (int i = 0; i < T; ++i) {
      h = fmaf(a[i], h, bb[i]);
      yv[i] = fmaf(Cv[i], h, yv[i]);
    }
    if (ln.seg == G - 1) carry[ln.dl * kMaxN + n] = h;
    if (n + 1 < N) commit(buf ^ 1);
    __syncthreads();
  }

  // ---- merge this chunk's outputs into the channel's plane (direction order fixed)
  if (ln.dvalid) {
#pragma unroll
    for (int i = 0; i < T; ++i) {
      if (l0 + i < L) {
        float* q = plane_row + px[i];
        *q = (k == 0) ? yv[i] : (*q + yv[i]);
      }
    }
  }
}

template <typename S, int G, int NW, bool LDS_PLANE>
__global__ __launch_bounds__(NW * 64) void ss2d_forward_kernel(Params p) {
  constexpr int CH = Shape<G, NW>::kChans;
  constexpr int NTH = Shape<G, NW>::kThreads;
  extern __shared__ float smem[];
  float* a2s = smem + 4 * G * kStageStride;
  float* carry = a2s + CH * kMaxN;
  float* biass = carry + CH * kMaxN;
  float* dss = biass + CH;
  float* lplane = dss + CH;

  // Work id: consecutive ids (same batch b, neighbouring channel blocks, which
  // share Bs/Cs) are kept on one XCD; the hardware deals workgroups round-robin
  // over the 8 XCDs.
  const int nb = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int work = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;

  Lane ln;
  ln.tid = threadIdx.x;
  const int lane = ln.tid & 63, wave = ln.tid >> 6;
  ln.seg = lane % G;
  ln.dl = wave * (64 / G) + lane / G;
  const int nbd = (p.D + CH - 1) / CH;
  ln.b = work / nbd;
  ln.d0 = (work - ln.b * nbd) * CH;
  ln.d = ln.d0 + ln.dl;
  ln.dvalid = ln.d < p.D;
  const int L = p.L;

  float* plane_row = LDS_PLANE ? lplane + (int64_t)ln.dl * L
                               : p.gplane + ((int64_t)ln.b * p.D + (ln.dvalid ? ln.d : 0)) * L;

  for (int k = 0; k < 4; ++k) {
    for (int i = ln.tid; i < CH * kMaxN; i += NTH) {
      const int dd = i / kMaxN, n = i - dd * kMaxN;
      const int dg = ln.d0 + dd;
      float v = 0.f;
      if (dg < p.D && n < p.N) v = -expf(p.A_log[(int64_t)(k * p.D + dg) * p.N + n]) * kLog2e;
      a2s[i] = v;
      carry[i] = 0.f;
    }
    for (int i = ln.tid; i < CH; i += NTH) {
      const int dg = ln.d0 + i;
      biass[i] = dg < p.D ? p.dt_bias[k * p.D + dg] : 0.f;
      dss[i] = dg < p.D ? p.Ds[k * p.D + dg] : 0.f;
    }
    __syncthreads();

    int c0 = 0;
    while (L - c0 >= G * 16) {
      run_chunk<S, G, NW, LDS_PLANE, 16>(p, ln, smem, plane_row, k, c0);
      c0 += G * 16;
    }
    if (L - c0 >= G * 12) { run_chunk<S, G, NW, LDS_PLANE, 12>(p, ln, smem, plane_row, k, c0); c0 += G * 12; }
    if (L - c0 >= G * 8) { run_chunk<S, G, NW, LDS_PLANE, 8>(p, ln, smem, plane_row, k, c0); c0 += G * 8; }
    if (L - c0 >= G * 4) { run_chunk<S, G, NW, LDS_PLANE, 4>(p, ln, smem, plane_row, k, c0); c0 += G * 4; }
    if (L - c0 >= G * 2) { run_chunk<S, G, NW, LDS_PLANE, 2>(p, ln, smem, plane_row, k, c0); c0 += G * 2; }
    while (c0 < L) {
      run_chunk<S, G, NW, LDS_PLANE, 1>(p, ln, smem, plane_row, k, c0);
      c0 += G;
    }
    __syncthreads();  // direction k's plane updates complete before direction k+1
  }

  // ---- write the merged planes to y (one rounding to the storage type)
  S* y = static_cast<S*>(p.y);
  if (LDS_PLANE || !std::is_same<S, float>::value) {
    for (int dd = 0; dd < CH; ++dd) {
      const int dg = ln.d0 + dd;
      if (dg >= p.D) break;
      const float* src = LDS_PLANE ? lplane + (int64_t)dd * L : p.gplane + ((int64_t)ln.b * p.D + dg) * L;
      const int64_t ybase = ((int64_t)ln.b * p.D + dg) * L;
      if (p.vec) {
        for (int i = ln.tid * 4; i < L; i += NTH * 4)
          Io<S>::st4(y, ybase + i, *reinterpret_cast<const float4*>(src + i));
      } else {
        for (int i = ln.tid; i < L; i += NTH) Io<S>::st(y, ybase + i, src[i]);
      }
    }
  }
}

template <typename S, int G, int NW, bool LDS_PLANE>
hipError_t launch_variant(const LaunchArgs& a, const Plan& plan, float* gplane) {
  Params p;
  p.x = a.x;
  p.dt = a.dt;
  p.A_log = a.A_log;
  p.dt_bias = a.dt_bias;
  p.Bs = a.Bs;
  p.Cs = a.Cs;
  p.Ds = a.Ds;
  p.y = a.y;
  p.gplane = gplane;
  p.B = (int)a.B;
  p.D = (int)a.D;
  p.H = (int)a.H;
  p.W = (int)a.W;
  p.N = (int)a.N;
  p.L = (int)(a.H * a.W);
  p.vec = (p.L % 4 == 0) ? 1 : 0;
  auto kern = ss2d_forward_kernel<S, G, NW, LDS_PLANE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)plan.blocks), dim3(NW * 64), plan.lds_bytes, a.stream, p);
  return hipGetLastError();
}

template <typename S, int G>
hipError_t launch_g(const LaunchArgs& a, const Plan& plan, float* gplane) {
  if (plan.lds_plane) return launch_variant<S, G, 4, true>(a, plan, gplane);
  return launch_variant<S, G, 4, false>(a, plan, gplane);
}

template <typename S>
hipError_t launch_s(const LaunchArgs& a, const Plan& plan, float* gplane) {
  switch (plan.lanes_per_seq) {
    case 16: return launch_g<S, 16>(a, plan, gplane);
    case 32: return launch_g<S, 32>(a, plan, gplane);
    default: return launch_g<S, 64>(a, plan, gplane);
  }
}

}  // namespace

Plan make_plan(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, size_t lds_limit) {
  (void)N;
  Plan pl;
  const int64_t L = H * W;
  pl.lanes_per_seq = L < 256 ? 16 : (L < 768 ? 32 : 64);
  pl.waves = 4;
  pl.chans_per_block = pl.waves * (64 / pl.lanes_per_seq);
  pl.blocks = B * ((D + pl.chans_per_block - 1) / pl.chans_per_block);
  const int G = pl.lanes_per_seq;
  const size_t fixed = sizeof(float) * (size_t)(4 * G * kStageStride + 2 * pl.chans_per_block * kMaxN +
                                                2 * pl.chans_per_block);
  const size_t with_plane = fixed + sizeof(float) * (size_t)pl.chans_per_block * (size_t)L;
  pl.lds_plane = with_plane <= lds_limit;
  pl.lds_bytes = pl.lds_plane ? with_plane : fixed;
  pl.needs_scratch = !pl.lds_plane && dtype != 0;
  return pl;
}

hipError_t launch_forward(const LaunchArgs& a, const Plan& plan, float* scratch_plane) {
  if (a.dtype == 0) {
    float* gplane = plan.lds_plane ? nullptr : static_cast<float*>(a.y);
    return launch_s<float>(a, plan, gplane);
  }
  return launch_s<uint16_t>(a, plan, scratch_plane);
}

}  // namespace ss2d
