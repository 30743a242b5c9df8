// The step after the merge: y (B, D, H, W) to channel-last (B, H, W, D), with an
// optional LayerNorm over the D channels of each pixel (gfx950).
//
// What is computed: page [SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现" §3.3 ends
// the forward by transposing the merged y to (B, H, W, D); [VSSD] §5.3 lists
// fusing the LayerNorm that follows.  With m and v the mean and the (biased)
// variance of y[b, :, p] over its D channels,
//   out[b, p, d] = (y[b, d, p] - m) / sqrt(v + eps) * gamma[d] + beta[d],
// or out[b, p, d] = y[b, d, p] without the normalisation.
//
// How it runs (channel_last_vec_kernel, rows and bases aligned for vector
// access).  A workgroup takes TP = 16 consecutive pixels of one batch with all D
// channels.  Loads read V consecutive pixels of a channel per lane (V = 4 fp32,
// 8 bf16: 16-byte loads) into an LDS tile stored pixel-major, [TP][D + 4], so the
// output side reads V consecutive channels of a pixel with 16-byte LDS reads and
// writes them with one vector store; a tile's output rows are one contiguous
// block.  The statistics are per pixel over K = threads / TP consecutive lanes:
// each lane reads its share of the pixel's channels once, with 16-byte LDS
// reads, into registers, and the mean and then the squared deviations are
// reduced across the K lanes with shuffles (no second LDS pass, no barrier
// between the two).  256 threads up to 512 channels, 512 above.  Consecutive tiles run on one
// XCD (they share 128-byte lines of y).  bf16 output uses the hardware packed
// round-to-nearest-even conversion.  Other shapes (L or D not a multiple of V,
// unaligned bases, D above 900) take channel_last_kernel: channel-major tiles
// of up to 64 pixels, scalar stores.
#include "ss2d_kernels.h"

namespace ss2d {
namespace {

constexpr int kEpiThreads = 256;
constexpr int kEpiLdsFloats = 8192;  // 32 KB for the tile

struct EpiParams {
  const void* y;
  const float* gamma;  // null: 1
  const float* beta;   // null: 0
  void* out;
  float eps;
  int D, L, TP, tiles;
};

// VEC: L and TP are multiples of 4 and y is aligned, so each thread loads four
// consecutive pixels of a channel with one 16-byte (fp32) or 8-byte (bf16) load.
template <typename S, bool NORM, bool VEC>
__global__ __launch_bounds__(kEpiThreads) void channel_last_kernel(EpiParams p) {
  __shared__ float tile[kEpiLdsFloats];
  __shared__ float part[kEpiThreads];
  __shared__ float mean_s[64], rstd_s[64];
  const int D = p.D, L = p.L, TP = p.TP, ld = TP + 1;
  const int tid = threadIdx.x;
  const int t = blockIdx.x % p.tiles;
  const int64_t b = blockIdx.x / p.tiles;
  const int p0 = t * TP;
  const int np = L - p0 < TP ? L - p0 : TP;  // pixels of this tile
  const S* yb = static_cast<const S*>(p.y) + b * D * L;

  // load: element e = d * TP + j (channel d, pixel j), eight in flight per thread
  const int n = D * TP;
  if (VEC) {  // groups of four pixels: group e = d * (TP / 4) + j4
    const int g4 = TP / 4, n4 = D * g4;
    const int dq = kEpiThreads / g4, dr = kEpiThreads - dq * g4;
    int d = tid / g4, j4 = tid - (tid / g4) * g4;
    for (int e0 = tid; e0 < n4; e0 += 8 * kEpiThreads) {
      float4 v[8];
      int dd = d, jj = j4;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = e0 + u * kEpiThreads < n4 && 4 * jj < np;  // np % 4 == 0 as L % 4 == 0
        const float4 x = Io<S>::ld4(yb, ok ? (int64_t)dd * L + p0 + 4 * jj : 0);
        v[u] = ok ? x : make_float4(0.f, 0.f, 0.f, 0.f);
        dd += dq;
        jj += dr;
        if (jj >= g4) {
          jj -= g4;
          ++dd;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (e0 + u * kEpiThreads < n4) {
          float* r = tile + d * ld + 4 * j4;
          r[0] = v[u].x;
          r[1] = v[u].y;
          r[2] = v[u].z;
          r[3] = v[u].w;
        }
        d += dq;
        j4 += dr;
        if (j4 >= g4) {
          j4 -= g4;
          ++d;
        }
      }
    }
  } else {
    const int dq = kEpiThreads / TP, dr = kEpiThreads - dq * TP;
    int d = tid / TP, j = tid - (tid / TP) * TP;
    for (int e0 = tid; e0 < n; e0 += 8 * kEpiThreads) {
      float v[8];
      int dd = d, jj = j;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = e0 + u * kEpiThreads < n && jj < np;
        const float x = Io<S>::ld(yb, ok ? (int64_t)dd * L + p0 + jj : 0);
        v[u] = ok ? x : 0.f;
        dd += dq;
        jj += dr;
        if (jj >= TP) {
          jj -= TP;
          ++dd;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (e0 + u * kEpiThreads < n) tile[d * ld + j] = v[u];
        d += dq;
        j += dr;
        if (j >= TP) {
          j -= TP;
          ++d;
        }
      }
    }
  }
  __syncthreads();

  if (NORM) {
    // k = 256 / TP threads per pixel: thread (j, q) sums channels q, q + k, ...
    const int k = kEpiThreads / TP;
    const int j = tid % TP, q = tid / TP;
    float s = 0.f;
    for (int d = q; d < D; d += k) s += tile[d * ld + j];
    part[tid] = s;
    __syncthreads();
    if (tid < TP) {
      float m = 0.f;
      for (int i = 0; i < k; ++i) m += part[i * TP + tid];
      mean_s[tid] = m / (float)D;
    }
    __syncthreads();
    const float m = mean_s[j];
    float s2 = 0.f;
    for (int d = q; d < D; d += k) {
      const float c = tile[d * ld + j] - m;
      s2 = fmaf(c, c, s2);
    }
    part[tid] = s2;
    __syncthreads();
    if (tid < TP) {
      float v = 0.f;
      for (int i = 0; i < k; ++i) v += part[i * TP + tid];
      rstd_s[tid] = 1.f / sqrtf(v / (float)D + p.eps);
    }
    __syncthreads();
  }

  // store: element o = j * D + d of the tile's channel-last block, consecutive
  // threads on consecutive channels (LDS rows of odd length: no bank conflicts;
  // four channels per thread measured slower for that reason)
  S* ob = static_cast<S*>(p.out) + (b * L + p0) * (int64_t)D;
  auto value = [&](int j, int d) {
    float v = tile[d * ld + j];
    if (NORM) {
      v = (v - mean_s[j]) * rstd_s[j];
      const float g = p.gamma ? p.gamma[d] : 1.f;
      const float be = p.beta ? p.beta[d] : 0.f;
      v = fmaf(v, g, be);
    }
    return v;
  };
  {
    const int m_out = np * D;
    const int oq = kEpiThreads / D, orr = kEpiThreads - oq * D;
    int j = tid / D, d = tid - (tid / D) * D;
#pragma unroll 4
    for (int o = tid; o < m_out; o += kEpiThreads) {
      Io<S>::st(ob, o, value(j, d));
      j += oq;
      d += orr;
      if (d >= D) {
        d -= D;
        ++j;
      }
    }
  }
}

// ------------------------------------------------------------------ vector path
// V consecutive elements of storage type S as floats, and back.
template <typename S, int V>
struct VecIo;
template <>
struct VecIo<float, 4> {
  static __device__ __forceinline__ void ld(const float* p, int64_t i, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p + i);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ void st(float* p, int64_t i, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct VecIo<uint16_t, 4> {
  static __device__ __forceinline__ void ld(const uint16_t* p, int64_t i, float (&v)[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p + i);
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, const float (&v)[4]) {
    *reinterpret_cast<uint2*>(p + i) = make_uint2(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]));
  }
};
template <>
struct VecIo<uint16_t, 8> {
  static __device__ __forceinline__ void ld(const uint16_t* p, int64_t i, float (&v)[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, const float (&v)[8]) {
    *reinterpret_cast<uint4*>(p + i) = make_uint4(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]),
                                                  bf16x2_rne(v[4], v[5]), bf16x2_rne(v[6], v[7]));
  }
};

constexpr int kVecTile = 16;   // pixels per workgroup
constexpr int kVecMaxD = 900;   // [16][D + 4] fp32 tile plus gamma and beta: up to 64 KB of dynamic LDS
constexpr int kVecStatF4 = 8;   // 16-byte values per lane in the statistics: D <= 32 K (K lanes per pixel)
constexpr int kVecNarrowMaxD = 4 * kVecStatF4 * (256 / kVecTile);  // widest D the 256-thread form takes (512)

// Sum over the K consecutive lanes of a group (K a power of two up to 64).
template <int K>
__device__ __forceinline__ float lane_group_sum(float v) {
#pragma unroll
  for (int o = K / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename S, int V, int NT, bool NORM>
__global__ __launch_bounds__(NT) void channel_last_vec_kernel(EpiParams p) {
  constexpr int TP = kVecTile;
  constexpr int K = NT / TP;  // lanes per pixel in the statistics
  extern __shared__ __align__(16) float vtile[];  // [TP][D + 4], then gamma and beta (D each)
  __shared__ float mean_s[TP], rstd_s[TP];
  const int D = p.D, L = p.L, ldd = D + 4;
  const int tid = threadIdx.x;
  float* gam = vtile + TP * ldd;
  float* bet = gam + D;
  if (NORM) {
    for (int i = tid; i < D; i += NT) {
      gam[i] = p.gamma ? p.gamma[i] : 1.f;
      bet[i] = p.beta ? p.beta[i] : 0.f;
    }
  }
  // consecutive tiles (which share lines of y) on one XCD; workgroups are dealt
  // round-robin over the 8 XCDs
  const int nb = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = nb >> 3, rem = nb & 7;
  const int wid = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int t = wid % p.tiles;
  const int64_t b = wid / p.tiles;
  const int p0 = t * TP;
  const int np = L - p0 < TP ? L - p0 : TP;  // a multiple of V: L % V == 0
  const S* yb = static_cast<const S*>(p.y) + b * D * L;

  // load: vector e = d * (TP / V) + jv (channel d, pixels V*jv ..), U in flight per thread
  {
    constexpr int GV = TP / V;
    constexpr int U = 32 / V;
    const int nv = D * GV;
    constexpr int DQ = NT / GV;  // NT is a multiple of GV
    int d = tid / GV;
    const int jv = tid % GV;
    for (int e0 = tid; e0 < nv; e0 += U * NT) {
      float v[U][V];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int dd = d + u * DQ;
        const bool ok = e0 + u * NT < nv && V * jv < np;
        VecIo<S, V>::ld(yb, ok ? (int64_t)dd * L + p0 + V * jv : 0, v[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (e0 + u * NT < nv) {
          float* r = vtile + V * jv * ldd + d + u * DQ;
#pragma unroll
          for (int i = 0; i < V; ++i) r[i * ldd] = v[u][i];
        }
      }
      d += U * DQ;
    }
  }
  __syncthreads();

  if (NORM) {
    // the pixel's channels are read once, 4 at a time (16-byte LDS reads), into
    // registers: lane q of the pixel's K holds channels 4(q + K m) .. + 3
    static_assert(4 * K * kVecStatF4 >= (NT == 256 ? kVecNarrowMaxD : kVecMaxD),
                  "the statistics registers cover every channel the launch allows");
    const int q = tid % K, j = tid / K;
    const float* row = vtile + j * ldd;
    const int D4 = D >> 2;
    float4 xv[kVecStatF4];
    float sum = 0.f;
#pragma unroll
    for (int mm = 0; mm < kVecStatF4; ++mm) {
      const int c4 = q + K * mm;
      xv[mm] = c4 < D4 ? *reinterpret_cast<const float4*>(row + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
      sum += (xv[mm].x + xv[mm].y) + (xv[mm].z + xv[mm].w);
    }
    const float m = lane_group_sum<K>(sum) / (float)D;
    float sq = 0.f;
#pragma unroll
    for (int mm = 0; mm < kVecStatF4; ++mm) {
      if (q + K * mm < D4) {
        const float a0 = xv[mm].x - m, a1 = xv[mm].y - m, a2 = xv[mm].z - m, a3 = xv[mm].w - m;
        sq = fmaf(a0, a0, sq);
        sq = fmaf(a1, a1, sq);
        sq = fmaf(a2, a2, sq);
        sq = fmaf(a3, a3, sq);
      }
    }
    const float var = lane_group_sum<K>(sq) / (float)D;
    if (q == 0) {
      mean_s[j] = m;
      rstd_s[j] = 1.f / sqrtf(var + p.eps);
    }
    __syncthreads();
  }

  // store: vector o = j * (D / V) + c (pixel j, channels V*c ..); the tile's output
  // rows are consecutive, so the workgroup writes one contiguous block
  S* ob = static_cast<S*>(p.out) + (b * L + p0) * (int64_t)D;
  const int DV = D / V, mv = np * DV;
  const int oq = NT / DV, orr = NT - oq * DV;
  int j = tid / DV, c = tid - (tid / DV) * DV;
  for (int o = tid; o < mv; o += NT) {
    const float* src = vtile + j * ldd + V * c;
    float w[V];
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(src + i);
      w[i] = a.x; w[i + 1] = a.y; w[i + 2] = a.z; w[i + 3] = a.w;
    }
    if (NORM) {
      const float m = mean_s[j], r = rstd_s[j];
#pragma unroll
      for (int i = 0; i < V; i += 4) {
        const float4 g = *reinterpret_cast<const float4*>(gam + V * c + i);
        const float4 be = *reinterpret_cast<const float4*>(bet + V * c + i);
        w[i] = fmaf((w[i] - m) * r, g.x, be.x);
        w[i + 1] = fmaf((w[i + 1] - m) * r, g.y, be.y);
        w[i + 2] = fmaf((w[i + 2] - m) * r, g.z, be.z);
        w[i + 3] = fmaf((w[i + 3] - m) * r, g.w, be.w);
      }
    }
    VecIo<S, V>::st(ob, (int64_t)o * V, w);
    j += oq;
    c += orr;
    if (c >= DV) {
      c -= DV;
      ++j;
    }
  }
}

template <typename S, int V, int NT>
hipError_t launch_vec(const EpiParams& p, bool norm, unsigned blocks, hipStream_t stream) {
  const size_t lds = ((size_t)kVecTile * (p.D + 4) + 2 * (size_t)p.D) * sizeof(float);
  if (norm)
    hipLaunchKernelGGL((channel_last_vec_kernel<S, V, NT, true>), dim3(blocks), dim3(NT), lds, stream, p);
  else
    hipLaunchKernelGGL((channel_last_vec_kernel<S, V, NT, false>), dim3(blocks), dim3(NT), lds, stream, p);
  return hipGetLastError();
}

template <typename S, bool VEC>
hipError_t launch_epi(const EpiParams& p, bool norm, unsigned blocks, hipStream_t stream) {
  if (norm)
    hipLaunchKernelGGL((channel_last_kernel<S, true, VEC>), dim3(blocks), dim3(kEpiThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((channel_last_kernel<S, false, VEC>), dim3(blocks), dim3(kEpiThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int epilogue_max_channels() { return kEpiLdsFloats / 2; }

hipError_t launch_channel_last(const EpilogueArgs& a) {
  EpiParams p;
  p.y = a.y;
  p.gamma = a.gamma;
  p.beta = a.beta;
  p.out = a.out;
  p.eps = a.eps;
  p.D = (int)a.D;
  p.L = (int)(a.H * a.W);
  {
    // the vector path: V-element accesses along pixels (loads) and channels (stores)
    const int V = (a.dtype == 1 && p.L % 8 == 0 && p.D % 8 == 0) ? 8 : 4;
    const uintptr_t va = a.dtype == 0 ? 15 : (uintptr_t)(2 * V - 1);
    const bool vec_ok = p.L % V == 0 && p.D % V == 0 && p.D <= kVecMaxD && !((uintptr_t)a.y & va) &&
                        !((uintptr_t)a.out & va);
    if (vec_ok) {
      p.TP = kVecTile;
      p.tiles = (p.L + kVecTile - 1) / kVecTile;
      const int64_t blocks = a.B * p.tiles;
      if (blocks > INT32_MAX) return hipErrorInvalidValue;
      // 256 threads (16 lanes per pixel) for up to 512 channels, else 512 (32 lanes):
      // the statistics registers of a lane cover 32 K channels
      const bool wide = p.D > kVecNarrowMaxD;
      if (a.dtype == 0)
        return wide ? launch_vec<float, 4, 512>(p, a.normalize, (unsigned)blocks, a.stream)
                    : launch_vec<float, 4, 256>(p, a.normalize, (unsigned)blocks, a.stream);
      if (V == 8)
        return wide ? launch_vec<uint16_t, 8, 512>(p, a.normalize, (unsigned)blocks, a.stream)
                    : launch_vec<uint16_t, 8, 256>(p, a.normalize, (unsigned)blocks, a.stream);
      return wide ? launch_vec<uint16_t, 4, 512>(p, a.normalize, (unsigned)blocks, a.stream)
                  : launch_vec<uint16_t, 4, 256>(p, a.normalize, (unsigned)blocks, a.stream);
    }
  }
  // pixels per workgroup: the most (up to 64, a power of two) whose tile fits the LDS
  int tp = 64;
  while (tp > 1 && (int64_t)p.D * (tp + 1) > kEpiLdsFloats) tp >>= 1;
  if ((int64_t)p.D * (tp + 1) > kEpiLdsFloats) return hipErrorInvalidValue;
  p.TP = tp;
  p.tiles = (p.L + tp - 1) / tp;
  const int64_t blocks = a.B * p.tiles;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const uintptr_t am = a.dtype == 0 ? 15 : 7;
  const bool vec = p.L % 4 == 0 && tp % 4 == 0 && !((uintptr_t)a.y & am);
  if (a.dtype == 0)
    return vec ? launch_epi<float, true>(p, a.normalize, (unsigned)blocks, a.stream)
               : launch_epi<float, false>(p, a.normalize, (unsigned)blocks, a.stream);
  return vec ? launch_epi<uint16_t, true>(p, a.normalize, (unsigned)blocks, a.stream)
             : launch_epi<uint16_t, false>(p, a.normalize, (unsigned)blocks, a.stream);
}

}  // namespace ss2d
