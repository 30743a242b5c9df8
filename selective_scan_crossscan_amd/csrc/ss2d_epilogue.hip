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
// How it runs.  A workgroup takes TP consecutive pixels of one batch with all D
// channels into LDS (rows of TP + 1 floats, so reading down a row's pixels is
// free of bank conflicts), eight loads in flight per thread.  The statistics are
// two passes over LDS in fp32 (mean, then the squared deviations), 256 / TP
// threads per pixel.  The output is written pixel by pixel, D contiguous values
// each, consecutive threads on consecutive channels.
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
