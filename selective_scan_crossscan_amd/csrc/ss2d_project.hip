// The per-direction input projections of SS2D on the matrix cores (gfx950).
//
// What is computed (page [SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现", §3.2,
// the parameter projection before the selective scan): for every direction k
// and scan step l, with u the feature vector (D channels) of the pixel that
// direction visits at l,
//   row[c]          = sum_d x_proj_weight[k, c, d] * u[d],   c < C = R + 2N,
//   dt[b, k, d, l]  = sum_r dt_projs_weight[k, d, r] * row[r],   r < R,
//   Bs[b, k, n, l]  = row[R + n],   Cs[b, k, n, l] = row[R + N + n],
// all written in the direction's scan order, which is the layout the selective
// scan reads.  The dt bias is not added here (the scan adds it before softplus).
//
// How it runs.  Directions 0 and 2 visit the pixels in row-major order, 2 in
// reverse; directions 1 and 3 in column-major order, 3 in reverse.  So one
// workgroup (one wave) takes 64 consecutive positions of one orientation (row-
// major from x, column-major from x transposed) and produces the rows of both
// directions of that orientation: direction 0 (or 1) at those positions, and
// direction 2 (or 3) at the mirrored positions L-1-l.
//   * The projection is a (2C x D) by (D x 64) product in fp32 on
//     v_mfma_f32_16x16x4_f32: 2C rows in 16-row tiles, the 64 positions as four
//     16-column tiles whose column j holds position 4j + t of tile t, so each
//     lane loads four consecutive positions with one vector load and holds four
//     consecutive outputs per row for one vector store.  Sixteen channels are
//     consumed per step: lane group g (lanes 16g..16g+15) feeds channels
//     4g..4g+3 over four MFMAs, which is one vector load of the weights too.
//   * The R rows of the rank-R dt input go to LDS; dt = W_dt (D x R) times
//     them is a second MFMA product with R in steps of four.
//   * Every store is a 16-byte (fp32) or 8-byte (bf16) write of four
//     consecutive scan positions; a wave writes 256 contiguous bytes (fp32) of
//     each of four rows.
#include "ss2d_kernels.h"

namespace ss2d {
namespace {

constexpr int kStrip = 64;   // positions per workgroup
constexpr int kMaxTiles = 8;  // 16-row tiles of the stacked projection rows: 2C <= 128

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ProjParams {
  const void* x;   // (B, D, L) row-major pixel order
  const void* xT;  // (B, D, L) column-major pixel order (x with H and W swapped)
  const float* wx;   // (4, C, D)
  const float* wdt;  // (4, D, R)
  void* dt;          // (B, 4, D, L)
  void* Bs;          // (B, 4, N, L)
  void* Cs;          // (B, 4, N, L)
  int D, L, N, R, C, strips;
};

__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float comp(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Four consecutive scan positions pos..pos+3 of a row of length L, written in
// order (forward) or at L-1-pos-i (mirrored direction); positions past L are
// not written.
template <typename S, bool VEC>
__device__ __forceinline__ void put4(S* row, int pos, int L, bool mirror, float4 v) {
  if (VEC) {  // L % 4 == 0, so the four are all inside or all outside
    if (pos >= L) return;
    if (mirror)
      Io<S>::st4(row, L - 4 - pos, make_float4(v.w, v.z, v.y, v.x));
    else
      Io<S>::st4(row, pos, v);
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (pos + i < L) Io<S>::st(row, mirror ? L - 1 - (pos + i) : pos + i, comp(v, i));
}

// MT: 16-row tiles covering the 2C stacked rows.  VEC: L and D are multiples of
// 4 and the bases are aligned for the vector forms.
template <typename S, int MT, bool VEC>
__global__ __launch_bounds__(64) void project_kernel(ProjParams p) {
  extern __shared__ __align__(16) float dts[];  // [2][R][kStrip]
  const int D = p.D, L = p.L, N = p.N, R = p.R, C = p.C;
  const int strip = blockIdx.x % p.strips;
  const int rest = blockIdx.x / p.strips;
  const int o = rest & 1;  // orientation: 0 row-major (directions 0, 2), 1 column-major (1, 3)
  const int b = rest >> 1;
  const int lane = threadIdx.x;
  const int col = lane & 15, g = lane >> 4;
  const int pos = strip * kStrip + 4 * col;  // this lane's four positions
  const S* src = static_cast<const S*>(o ? p.xT : p.x) + (int64_t)b * D * L;

  // A operand rows: stacked row m = mt*16 + col is row c of direction o + 2*kk
  const float* arow[MT];
  bool aval[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + col;
    const int kk = m >= C ? 1 : 0;
    aval[mt] = m < 2 * C;
    arow[mt] = p.wx + (aval[mt] ? ((int64_t)(o + 2 * kk) * C + (m - kk * C)) * D : 0);
  }

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int d0 = 0; d0 < D; d0 += 16) {
    const int dg = d0 + 4 * g;  // channels dg..dg+3 of this lane group
    float4 bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = dg + j;
      bv[j] = d < D ? ld4_guarded<S>(src + (int64_t)d * L, pos, L, VEC) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 av[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      av[mt] = aval[mt] ? ld4_guarded<float>(arow[mt], dg, D, VEC) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_16x16x4(comp(av[mt], j), comp(bv[j], t), acc[mt][t]);
  }

  // lane (g, col) holds stacked rows mt*16 + 4g + i at positions pos..pos+3
  const int64_t bk0 = (int64_t)b * 4 + o;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + 4 * g + i;
      if (m >= 2 * C) continue;
      const int kk = m >= C ? 1 : 0;
      const int c = m - kk * C;
      const float4 v = make_float4(acc[mt][0][i], acc[mt][1][i], acc[mt][2][i], acc[mt][3][i]);
      if (c < R) {
        *reinterpret_cast<float4*>(dts + (kk * R + c) * kStrip + 4 * col) = v;
      } else {
        const int64_t bk = bk0 + 2 * kk;
        S* row = c < R + N ? static_cast<S*>(p.Bs) + (bk * N + (c - R)) * L
                           : static_cast<S*>(p.Cs) + (bk * N + (c - R - N)) * L;
        put4<S, VEC>(row, pos, L, kk == 1, v);
      }
    }
  }
  __syncthreads();

  // dt = W_dt (D x R) times the R rows, per direction, 16 channels at a time
  for (int kk = 0; kk < 2; ++kk) {
    const int k = o + 2 * kk;
    const float* wk = p.wdt + (int64_t)k * D * R;
    S* dtk = static_cast<S*>(p.dt) + (bk0 + 2 * kk) * D * L;
    for (int dm = 0; dm < D; dm += 16) {
      f32x4 c4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) c4[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int da = dm + col;
      for (int r0 = 0; r0 < R; r0 += 4) {
        const int r = r0 + g;
        const float a = (r < R && da < D) ? wk[(int64_t)da * R + r] : 0.f;
        const float4 q = r < R ? *reinterpret_cast<const float4*>(dts + (kk * R + r) * kStrip + 4 * col)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int t = 0; t < 4; ++t) c4[t] = mfma_16x16x4(a, comp(q, t), c4[t]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = dm + 4 * g + i;
        if (d < D) put4<S, VEC>(dtk + (int64_t)d * L, pos, L, kk == 1, make_float4(c4[0][i], c4[1][i], c4[2][i], c4[3][i]));
      }
    }
  }
}

template <typename S, bool VEC>
hipError_t launch_tiles(const ProjParams& p, int tiles, unsigned blocks, size_t lds, hipStream_t stream) {
  switch (tiles) {
#define SS2D_PROJ_CASE(T_)                                                                               \
  case T_:                                                                                               \
    hipLaunchKernelGGL((project_kernel<S, T_, VEC>), dim3(blocks), dim3(64), lds, stream, p);            \
    return hipGetLastError();
    SS2D_PROJ_CASE(1)
    SS2D_PROJ_CASE(2)
    SS2D_PROJ_CASE(3)
    SS2D_PROJ_CASE(4)
    SS2D_PROJ_CASE(5)
    SS2D_PROJ_CASE(6)
    SS2D_PROJ_CASE(7)
    SS2D_PROJ_CASE(8)
#undef SS2D_PROJ_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

int project_max_rows() { return 16 * kMaxTiles; }

hipError_t launch_transpose_x(const void* x, void* xT, int64_t planes, int64_t H, int64_t W, int dtype,
                              hipStream_t stream) {
  if (dtype == 0)
    return launch_transpose<float>(static_cast<const float*>(x), static_cast<float*>(xT), (int)planes, (int)H,
                                   (int)W, stream);
  return launch_transpose<uint16_t>(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(xT), (int)planes,
                                    (int)H, (int)W, stream);
}

hipError_t launch_project(const ProjectArgs& a) {
  ProjParams p;
  p.x = a.x;
  p.xT = a.xT;
  p.wx = a.wx;
  p.wdt = a.wdt;
  p.dt = a.dt;
  p.Bs = a.Bs;
  p.Cs = a.Cs;
  p.D = (int)a.D;
  p.L = (int)(a.H * a.W);
  p.N = (int)a.N;
  p.R = (int)a.R;
  p.C = (int)(a.R + 2 * a.N);
  p.strips = (p.L + kStrip - 1) / kStrip;
  const int tiles = (2 * p.C + 15) / 16;
  if (tiles > kMaxTiles) return hipErrorInvalidValue;
  const int64_t blocks = a.B * 2 * p.strips;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const size_t lds = (size_t)2 * p.R * kStrip * sizeof(float);
  const uintptr_t am = a.dtype == 0 ? 15 : 7;
  const bool vec = p.L % 4 == 0 && p.D % 4 == 0 && !((uintptr_t)a.x & am) && !((uintptr_t)a.xT & am) &&
                   !((uintptr_t)a.dt & am) && !((uintptr_t)a.Bs & am) && !((uintptr_t)a.Cs & am) &&
                   !((uintptr_t)a.wx & 15);
  if (a.dtype == 0)
    return vec ? launch_tiles<float, true>(p, tiles, (unsigned)blocks, lds, a.stream)
               : launch_tiles<float, false>(p, tiles, (unsigned)blocks, lds, a.stream);
  return vec ? launch_tiles<uint16_t, true>(p, tiles, (unsigned)blocks, lds, a.stream)
             : launch_tiles<uint16_t, false>(p, tiles, (unsigned)blocks, lds, a.stream);
}

}  // namespace ss2d
