// The SS2D forward's gradients (gfx950, fp32).
//
// What is computed: the reverse-mode derivative of the forward of page [SS2D]
// "深入解析VMamba中的SS2D模块从理论到代码实现" §3.1-§3.3 (cross scan, selective scan
// with delta = softplus(dt + dt_bias), A = -exp(A_log), h_l = exp(delta A) h_{l-1}
// + delta Bs u, out = Cs h + Ds u, then the merge).  With g the gradient of y
// gathered along each direction's walk (the merge's adjoint) and the state
// adjoint q_l = Cs[n,l] g_l + a_{l+1} q_{l+1} walked from the end:
//   dCs[n,l] = sum_d h_l g_l,            dBs[n,l] = sum_d q_l delta_l u_l,
//   du_l = sum_n q_l delta_l Bs[n,l] + Ds g_l,
//   ddt_l = sigmoid(dt_l + dt_bias) * sum_n q_l (A a_l h_{l-1} + Bs[n,l] u_l),
//   dA_log = A * sum_{b,l} q_l delta_l a_l h_{l-1},  ddt_bias = sum_{b,l} ddt_l,
//   dDs = sum_{b,l} g_l u_l,  dx = the merge of du.
//
// How it runs (a first, plain design: one lane per (batch, direction, channel,
// state) walking the whole sequence).
//   * A workgroup is 16 channels x 16 states of one (batch, direction): a DPP row
//     of 16 lanes holds the states of one channel, so the sums over states are
//     four row rotations.
//   * Pass 1 walks the sequence forwards and stores the state entering every
//     16-step segment.  Pass 2 walks the segments backwards: it recomputes the
//     segment's states from its checkpoint into registers, then walks the steps
//     backwards with the state adjoint.
//   * A segment's operands (x, dy, dt per channel; Bs, Cs per state) are loaded
//     once per workgroup, one value per thread, a segment ahead, and staged in
//     LDS; the sums over states run once per segment for all its steps.
//   * dBs/dCs partials are summed over the workgroup's 16 channels through LDS
//     once per segment and written per channel block; a second kernel sums the
//     blocks in a fixed order, so results are deterministic (no atomics).
//   * Column walks read transposed copies of x and dy (made first), so every
//     operand load is contiguous along the steps.
//   * du goes to a temporary; a gather kernel merges it into dx, and a small
//     kernel sums the per-batch parameter gradients.
#include "ss2d_kernels.h"

namespace ss2d {
namespace {

constexpr int kSeg = 16;      // steps per checkpointed segment
constexpr int kBwdChans = 16;  // channels per workgroup

struct BwdParams {
  const float* x;
  const float* dt;
  const float* A_log;
  const float* dt_bias;
  const float* Bs;
  const float* Cs;
  const float* Ds;
  const float* dy;
  const float* xT;   // x and dy with H and W swapped: column walks read them in order
  const float* dyT;
  float* ddt;  // (B, 4, D, L) out
  float* du;   // (B, 4, D, L) temporary
  float* hck;  // (B*4, nseg, D, N) temporary: state entering each segment
  float* dBp;  // (B*4, nblk, N, L) temporary
  float* dCp;
  float* dAp;  // (B, 4D, N) temporary
  float* dbp;  // (B, 4D) temporary
  float* dDp;
  int D, H, W, L, N, nseg, nblk;
};

// Sum over the 16 lanes of a DPP row (four rotations).
__device__ __forceinline__ float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false));  // row_ror:1
  return v;
}

// Operands of one 16-step segment, staged in LDS once per workgroup: per channel
// (x and dy at the visited pixels, delta = softplus(dt + dt_bias) and its
// derivative sigmoid(dt + dt_bias)) and per state (Bs, Cs).  delta and the
// sigmoid are computed once per (channel, step) by the staging thread.
enum { kOpX, kOpG, kOpDel, kOpSig, kOpB, kOpC, kOps };

__global__ __launch_bounds__(256) void bwd_scan_kernel(BwdParams p) {
  __shared__ float red[2][kSeg][256];
  __shared__ float op[2][kOps][kSeg][16];  // double-buffered, [step][channel or state]
  const int tid = threadIdx.x, n = tid & 15, ch = tid >> 4;
  const int blk = blockIdx.x % p.nblk;
  const int bk = blockIdx.x / p.nblk;  // b * 4 + k
  const int k = bk & 3, b = bk >> 2;
  const int D = p.D, L = p.L, N = p.N;
  const int d = blk * kBwdChans + ch;
  const bool dval = d < D, val = dval && n < N;
  const int ds = dval ? d : 0, ns = n < N ? n : 0;
  const int c = k * D + ds;
  const float A = val ? -expf(p.A_log[(int64_t)c * N + ns]) : 0.f;
  const float Al2 = A * kLog2e;
  const float Dsk = p.Ds[c];
  auto hck = [&](int s) -> float& { return p.hck[(((int64_t)bk * p.nseg + s) * D + ds) * N + ns]; };

  // this thread's share of the staging: step i = tid & 15 of the segment, for
  // channel (tid >> 4) of the per-channel operands and state (tid >> 4) of the
  // per-state ones
  const int si = tid & 15, sr = tid >> 4;
  const int sd = blk * kBwdChans + sr;
  const bool sdv = sd < D, snv = sr < N;
  const int sdc = sdv ? sd : 0, snc = snv ? sr : 0;
  const float sbias = p.dt_bias[k * D + sdc];
  // column walks read the transposed copies, where step l of direction 1 is element l
  const float* sx = ((k & 1) ? p.xT : p.x) + ((int64_t)b * D + sdc) * L;
  const float* sg = ((k & 1) ? p.dyT : p.dy) + ((int64_t)b * D + sdc) * L;
  const float* sdt = p.dt + ((int64_t)bk * D + sdc) * L;
  const float* sB = p.Bs + ((int64_t)bk * N + snc) * L;
  const float* sC = p.Cs + ((int64_t)bk * N + snc) * L;
  auto pixel = [&](int l) {  // element of sx / sg visited at step l of direction k
    return k >= 2 ? L - 1 - l : l;
  };
  float stage[kOps];
  auto load_stage = [&](int s, bool with_g) {
    const int l = s * kSeg + si;
    const bool in = l < L;
    const int px = in ? pixel(l) : 0, lc = in ? l : 0;
    // channels past D stage x = dy = 0 and states past N stage Bs = Cs = 0, so
    // their lanes compute zero states, adjoints and partials with no masks
    stage[kOpX] = sdv ? sx[px] : 0.f;
    stage[kOpG] = with_g && sdv ? sg[px] : 0.f;
    stage[kOpDel] = sdt[lc] + sbias;  // dt + dt_bias until stored
    stage[kOpB] = snv ? sB[lc] : 0.f;
    stage[kOpC] = with_g && snv ? sC[lc] : 0.f;
  };
  auto store_stage = [&](int buf) {
    const float pre = stage[kOpDel];
    stage[kOpDel] = softplus_f32(pre);
    stage[kOpSig] = 1.f / (1.f + __builtin_amdgcn_exp2f(-pre * kLog2e));
#pragma unroll
    for (int j = 0; j < kOps; ++j) op[buf][j][si][sr] = stage[j];
  };

  // pass 1: states entering every segment
  float h = 0.f;
  load_stage(0, false);
  store_stage(0);
  __syncthreads();
  for (int s = 0; s < p.nseg; ++s) {
    const int buf = s & 1;
    if (val) hck(s) = h;
    if (s + 1 < p.nseg) load_stage(s + 1, false);
    const int cnt = L - s * kSeg < kSeg ? L - s * kSeg : kSeg;
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      if (i < cnt) {
        const float del = op[buf][kOpDel][i][ch];
        h = fmaf(__builtin_amdgcn_exp2f(del * Al2), h, del * op[buf][kOpB][i][n] * op[buf][kOpX][i][ch]);
      }
    }
    if (s + 1 < p.nseg) store_stage(buf ^ 1);
    __syncthreads();
  }

  // pass 2: segments from the last, steps from the last
  float q = 0.f, a_next = 0.f, dA = 0.f, dbias = 0.f, dD = 0.f;
  const int64_t row = ((int64_t)bk * D + ds) * L;  // (b, k, d) row of ddt and du
  int buf = 0;
  load_stage(p.nseg - 1, true);
  store_stage(buf);
  __syncthreads();
  for (int s = p.nseg - 1; s >= 0; --s) {
    const int l0 = s * kSeg;
    const int cnt = L - l0 < kSeg ? L - l0 : kSeg;
    const float h_in = val ? hck(s) : 0.f;
    if (s > 0) load_stage(s - 1, true);
    float hs[kSeg], del[kSeg], aa[kSeg];
    float hv = h_in;
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      del[i] = op[buf][kOpDel][i][ch];
      aa[i] = __builtin_amdgcn_exp2f(del[i] * Al2);
      hv = fmaf(aa[i], hv, del[i] * op[buf][kOpB][i][n] * op[buf][kOpX][i][ch]);
      hs[i] = hv;
    }
    float dup[kSeg], ddp[kSeg];
#pragma unroll
    for (int i = kSeg - 1; i >= 0; --i) {
      dup[i] = 0.f;
      ddp[i] = 0.f;
      if (i < cnt) {
        const float g = op[buf][kOpG][i][ch], u = op[buf][kOpX][i][ch];
        const float Bv = op[buf][kOpB][i][n], Cv = op[buf][kOpC][i][n];
        const float hp = i > 0 ? hs[i - 1] : h_in;
        q = fmaf(a_next, q, Cv * g);
        const float qd = q * del[i];
        dA = fmaf(qd * aa[i], hp, dA);
        a_next = aa[i];
        red[0][i][tid] = hs[i] * g;
        red[1][i][tid] = qd * u;
        dup[i] = qd * Bv;
        ddp[i] = q * fmaf(A * aa[i], hp, Bv * u);
      }
    }
    // sums over the 16 states of each channel, all steps of the segment at once
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      dup[i] = row_sum16(dup[i]);
      ddp[i] = row_sum16(ddp[i]);
    }
    if (n == 0 && dval) {
#pragma unroll
      for (int i = 0; i < kSeg; ++i) {
        if (i < cnt) {
          const float g = op[buf][kOpG][i][ch], u = op[buf][kOpX][i][ch];
          const float ddt = ddp[i] * op[buf][kOpSig][i][ch];
          p.ddt[row + l0 + i] = ddt;
          p.du[row + l0 + i] = fmaf(Dsk, g, dup[i]);
          dbias += ddt;
          dD = fmaf(g, u, dD);
        }
      }
    }
    __syncthreads();
    // dCs (0) and dBs (1) partials of the segment, summed over the 16 channels
    for (int o = tid; o < 2 * kSeg * 16; o += 256) {
      const int which = o / (kSeg * 16), rem = o - which * (kSeg * 16);
      const int i = rem >> 4, nn = rem & 15;
      if (i < cnt && nn < N) {
        float sum = 0.f;
#pragma unroll
        for (int c2 = 0; c2 < kBwdChans; ++c2) sum += red[which][i][c2 * 16 + nn];
        float* dst = which == 0 ? p.dCp : p.dBp;
        dst[(((int64_t)bk * p.nblk + blk) * N + nn) * L + l0 + i] = sum;
      }
    }
    if (s > 0) store_stage(buf ^ 1);
    buf ^= 1;
    __syncthreads();
  }
  if (val) p.dAp[((int64_t)b * 4 * D + c) * N + ns] = dA;
  if (n == 0 && dval) {
    p.dbp[(int64_t)b * 4 * D + c] = dbias;
    p.dDp[(int64_t)b * 4 * D + c] = dD;
  }
}

// dBs / dCs: the channel blocks' partials summed in block order.
__global__ __launch_bounds__(256) void bwd_reduce_bc(const float* __restrict__ dBp, const float* __restrict__ dCp,
                                                    float* __restrict__ dBs, float* __restrict__ dCs, int64_t BK,
                                                    int nblk, int N, int L) {
  const int64_t total = BK * N * L;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t bk = e / ((int64_t)N * L), rest = e - bk * N * L;
    float sb = 0.f, sc = 0.f;
    for (int j = 0; j < nblk; ++j) {
      const int64_t src = (bk * nblk + j) * N * L + rest;
      sb += dBp[src];
      sc += dCp[src];
    }
    dBs[e] = sb;
    dCs[e] = sc;
  }
}

// dx[b, d, p] = du of directions 0, 1, 2, 3 at the steps that visit p, added in that order.
__global__ __launch_bounds__(256) void bwd_merge(const float* __restrict__ du, float* __restrict__ dx, int64_t BD,
                                                int D, int H, int W) {
  const int L = H * W;
  const int64_t total = BD * L;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t bd = e / L;
    const int px = (int)(e - bd * L);
    const int64_t b = bd / D, d = bd - b * D;
    const int hh = px / W, ww = px - hh * W;
    const int lc = ww * H + hh;
    const float* r0 = du + ((b * 4 + 0) * D + d) * L;
    const float* r1 = du + ((b * 4 + 1) * D + d) * L;
    const float* r2 = du + ((b * 4 + 2) * D + d) * L;
    const float* r3 = du + ((b * 4 + 3) * D + d) * L;
    dx[e] = ((r0[px] + r1[lc]) + r2[L - 1 - px]) + r3[L - 1 - lc];
  }
}

// Per-channel parameter gradients: sums over the batch in batch order.
__global__ __launch_bounds__(256) void bwd_params(const float* __restrict__ A_log, const float* __restrict__ dAp,
                                                 const float* __restrict__ dbp, const float* __restrict__ dDp,
                                                 float* __restrict__ dA_log, float* __restrict__ ddt_bias,
                                                 float* __restrict__ dDs, int B, int C4, int N) {
  const int e = blockIdx.x * 256 + threadIdx.x;  // (c, n)
  if (e >= C4 * N) return;
  const int c = e / N, n = e - c * N;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += dAp[((int64_t)b * C4 + c) * N + n];
  dA_log[e] = -expf(A_log[e]) * s;
  if (n == 0) {
    float sb = 0.f, sd = 0.f;
    for (int b = 0; b < B; ++b) {
      sb += dbp[(int64_t)b * C4 + c];
      sd += dDp[(int64_t)b * C4 + c];
    }
    ddt_bias[c] = sb;
    dDs[c] = sd;
  }
}

}  // namespace

size_t backward_scratch_bytes(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N) {
  const int64_t L = H * W, nseg = (L + kSeg - 1) / kSeg, nblk = (D + kBwdChans - 1) / kBwdChans;
  auto up = [](int64_t v) { return (size_t)((v * 4 + 255) & ~(int64_t)255); };
  return up(B * 4 * D * L) + up(B * 4 * nseg * D * N) + 2 * up(B * 4 * nblk * N * L) + up(B * 4 * D * N) +
         2 * up(B * 4 * D) + 2 * up(B * D * L);
}

hipError_t launch_backward(const BackwardArgs& a, void* scratch) {
  const int64_t L = a.H * a.W, nseg = (L + kSeg - 1) / kSeg, nblk = (a.D + kBwdChans - 1) / kBwdChans;
  auto up = [](int64_t v) { return (size_t)((v * 4 + 255) & ~(int64_t)255); };
  char* base = static_cast<char*>(scratch);
  BwdParams p;
  p.x = a.x;
  p.dt = a.dt;
  p.A_log = a.A_log;
  p.dt_bias = a.dt_bias;
  p.Bs = a.Bs;
  p.Cs = a.Cs;
  p.Ds = a.Ds;
  p.dy = a.dy;
  p.ddt = a.ddt;
  p.du = reinterpret_cast<float*>(base);
  base += up(a.B * 4 * a.D * L);
  p.hck = reinterpret_cast<float*>(base);
  base += up(a.B * 4 * nseg * a.D * a.N);
  p.dBp = reinterpret_cast<float*>(base);
  base += up(a.B * 4 * nblk * a.N * L);
  p.dCp = reinterpret_cast<float*>(base);
  base += up(a.B * 4 * nblk * a.N * L);
  p.dAp = reinterpret_cast<float*>(base);
  base += up(a.B * 4 * a.D * a.N);
  p.dbp = reinterpret_cast<float*>(base);
  base += up(a.B * 4 * a.D);
  p.dDp = reinterpret_cast<float*>(base);
  base += up(a.B * 4 * a.D);
  float* xT = reinterpret_cast<float*>(base);
  base += up(a.B * a.D * L);
  float* dyT = reinterpret_cast<float*>(base);
  p.xT = xT;
  p.dyT = dyT;
  p.D = (int)a.D;
  p.H = (int)a.H;
  p.W = (int)a.W;
  p.L = (int)L;
  p.N = (int)a.N;
  p.nseg = (int)nseg;
  p.nblk = (int)nblk;
  const int64_t blocks = a.B * 4 * nblk;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipError_t e = launch_transpose<float>(a.x, xT, (int)(a.B * a.D), (int)a.H, (int)a.W, a.stream);
  if (e != hipSuccess) return e;
  if ((e = launch_transpose<float>(a.dy, dyT, (int)(a.B * a.D), (int)a.H, (int)a.W, a.stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scan_kernel, dim3((unsigned)blocks), dim3(256), 0, a.stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_bc, dim3(4096), dim3(256), 0, a.stream, p.dBp, p.dCp, a.dBs, a.dCs, a.B * 4,
                     (int)nblk, (int)a.N, (int)L);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_merge, dim3(4096), dim3(256), 0, a.stream, p.du, a.dx, a.B * a.D, (int)a.D, (int)a.H,
                     (int)a.W);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int C4 = (int)(4 * a.D);
  hipLaunchKernelGGL(bwd_params, dim3((unsigned)((C4 * a.N + 255) / 256)), dim3(256), 0, a.stream, a.A_log, p.dAp,
                     p.dbp, p.dDp, a.dA_log, a.ddt_bias, a.dDs, (int)a.B, C4, (int)a.N);
  return hipGetLastError();
}

}  // namespace ss2d
