// Roofline probes: the rates the SS2D forward is measured against, taken on the
// device it runs on (one kernel per rate, timed with HIP events on the caller's
// stream).  Each kernel keeps its result live through a store that depends on
// every value it computes, so none of the work can be removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss2d_internal.h"
#include "ss2d_kernels.h"

namespace ss2d {
namespace {

constexpr int kChains = 8;      // independent dependency chains per lane
constexpr int kThreads = 256;
constexpr float kNever = -12345.5f;  // a sum the probes never reach

// v_exp_f32: x <- 2^-x stays in (0, 1].
__global__ __launch_bounds__(kThreads) void probe_exp(float* sink, int iters, float seed) {
  float x[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) x[j] = seed + 0.01f * j + 1e-6f * threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += x[j];
  if (s == kNever) sink[blockIdx.x] = s;
}

// Plain (non-packed) fp32 FMA.
__global__ __launch_bounds__(kThreads) void probe_fma(float* sink, int iters, float seed) {
  float x[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) x[j] = seed + 0.01f * j + 1e-6f * threadIdx.x;
  const float a = 0.9999f, b = 1e-4f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) x[j] = fmaf(x[j], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += x[j];
  if (s == kNever) sink[blockIdx.x] = s;
}

// The state update's mix, per chain and iteration: one exp2 and four VALU
// (exponent product, input product, state FMA, output FMA), each feeding the
// next iteration so nothing is loop-invariant.
__global__ __launch_bounds__(kThreads) void probe_update(float* sink, int iters, float seed) {
  float u[kChains], h[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    u[j] = seed + 0.01f * j + 1e-6f * threadIdx.x;
    h[j] = 0.f;
  }
  const float A = -0.7f, Bv = 0.3f, Cv = -1e-3f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      const float e = __builtin_amdgcn_exp2f(u[j] * A);
      h[j] = fmaf(e, h[j], u[j] * Bv);
      u[j] = fmaf(Cv, h[j], u[j]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += u[j] + h[j];
  if (s == kNever) sink[blockIdx.x] = s;
}

// The scan's state loop alone, every operand already on chip: the rate its
// arithmetic form reaches at the forward's occupancy (three workgroups of four
// waves per CU), against which the whole kernel (softplus and the other
// per-step work, memory, waits, merge, remainders) is compared.  Each lane
// holds 16 steps of one channel (delta, delta*u and outputs formed once) and
// runs the states of a chunk through the forward's own state step: fold, DPP
// prefix combine over the 32-lane group, state carried in LDS, replay with the
// output FMA; B and C come from swizzled LDS rows read as the scan reads them, and
// the states run in groups of four with one barrier per group, in a loop that
// is not unrolled, as in the scan.  Every pass reads the carried state the last
// one wrote and adds into the same outputs, so no work is loop-invariant.
constexpr int kFormG = 32, kFormT = 16, kFormStates = 16, kFormRows = 4;
constexpr int kFormRow = kFormG * kFormT;              // floats per LDS row (one chunk of steps)
constexpr int kFormChans = kThreads / kFormG;           // channels per workgroup

__global__ __launch_bounds__(kThreads, 3) void probe_state_loop(float* sink, int passes, int nstates, float seed) {
  __shared__ __align__(16) float bc[2 * kFormRows * kFormRow];  // B rows, then C rows (swizzled)
  __shared__ float a2s[kFormChans * kFormStates];
  __shared__ float carry[kFormChans * kFormStates];
  const int tid = threadIdx.x, seg = tid % kFormG, dl = tid / kFormG;
  for (int i = tid; i < 2 * kFormRows * kFormRow; i += kThreads) bc[i] = 0.05f * ((i * 37) % 41 - 20);
  for (int i = tid; i < kFormChans * kFormStates; i += kThreads) {
    a2s[i] = -(1.f + (i % kFormStates)) * kLog2e;
    carry[i] = 0.f;
  }
  __syncthreads();
  float dtv[kFormT], u[kFormT], delta[kFormT], du[kFormT], yv[kFormT];
#pragma unroll
  for (int i = 0; i < kFormT; ++i) {
    dtv[i] = 0.3f * ((i * 7 + seg) % 11 - 5);
    u[i] = seed + 0.01f * i + 1e-6f * tid;
  }
  const float sdelta = prepare_steps<kFormT>(dtv, u, -4.f, 1.f, true, kFormT, delta, du, yv);
  auto group = [&](int n0) {
#pragma unroll
    for (int r = 0; r < kFormRows; ++r) {
      const int n = n0 + r;
      __builtin_amdgcn_sched_barrier(0);
      if (n < nstates) {  // as in the scan: each state its own block, so its FMAs stay in it
        const char* rows = reinterpret_cast<const char*>(bc);
        float Bv[kFormT], Cv[kFormT];
        read_seg<float, kFormT>(rows + r * kFormRow * 4, seg, Bv);
        read_seg<float, kFormT>(rows + (kFormRows + r) * kFormRow * 4, seg, Cv);
        state_core<kFormG, kFormT>(Bv, Cv, a2s[dl * kFormStates + n], carry + dl * kFormStates + n, seg, delta, du,
                                   sdelta, yv);
      }
    }
    __syncthreads();
  };
#pragma unroll 1
  for (int it = 0; it < passes; ++it) {
#pragma unroll 1
    for (int n0 = 0; n0 < nstates; n0 += 2 * kFormRows) {
      group(n0);
      group(n0 + kFormRows);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kFormT; ++i) s += yv[i];
  if (s == kNever) sink[blockIdx.x] = s;
}

// Streaming read of n4 float4.
__global__ __launch_bounds__(kThreads) void probe_read(const float4* __restrict__ p, int64_t n4, float* sink) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    const float4 v = p[i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  if (acc.x + acc.y + acc.z + acc.w == kNever) sink[blockIdx.x] = acc.x;
}

// Device copy of n4 float4 (read + write).
__global__ __launch_bounds__(kThreads) void probe_copy(const float4* __restrict__ src, float4* __restrict__ dst,
                                                       int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) dst[i] = src[i];
}

// LDS reads of 16 bytes per lane, consecutive lanes on consecutive slots.
__global__ __launch_bounds__(kThreads) void probe_lds(float* sink, int iters) {
  constexpr int kSlots = 4 * kThreads;
  __shared__ float4 buf[kSlots];
  for (int i = threadIdx.x; i < kSlots; i += kThreads) buf[i] = make_float4(1e-3f * i, 1.f, 2.f, 3.f);
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 v = buf[(threadIdx.x + k * kThreads + it) & (kSlots - 1)];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
  }
  if (acc.x + acc.y + acc.z + acc.w == kNever) sink[blockIdx.x] = acc.x;
}

// Runs `launch` once untimed and `reps` times timed; returns the best time in seconds.
template <typename F>
hipError_t best_time(hipStream_t s, hipEvent_t e0, hipEvent_t e1, int reps, F launch, double* secs) {
  launch();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  double best = 1e30;
  for (int r = 0; r < reps; ++r) {
    if ((e = hipEventRecord(e0, s)) != hipSuccess) return e;
    launch();
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipEventRecord(e1, s)) != hipSuccess) return e;
    if ((e = hipEventSynchronize(e1)) != hipSuccess) return e;
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) return e;
    if (ms * 1e-3 < best) best = ms * 1e-3;
  }
  *secs = best;
  return hipSuccess;
}

}  // namespace

hipError_t measure_peaks(PeakRates* out, int64_t hbm_bytes, hipStream_t stream) {
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  const int blocks = ncu * 8;  // 8 workgroups of 4 waves per CU: 8 waves per SIMD
  const int iters = 2048;
  const int reps = 3;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  float* sink = nullptr;
  char* buf = nullptr;
  const int64_t n4 = hbm_bytes / 32;  // float4 in each half of the buffer
  double t = 0.0;
  auto done = [&](hipError_t r) {
    if (sink) (void)hipFreeAsync(sink, stream);
    if (buf) (void)hipFreeAsync(buf, stream);
    (void)hipStreamSynchronize(stream);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    return r;
  };
  if ((e = hipEventCreate(&e0)) != hipSuccess) return done(e);
  if ((e = hipEventCreate(&e1)) != hipSuccess) return done(e);
  if ((e = hipMallocAsync(reinterpret_cast<void**>(&sink), (size_t)blocks * sizeof(float), stream)) != hipSuccess)
    return done(e);
  if ((e = hipMallocAsync(reinterpret_cast<void**>(&buf), (size_t)n4 * 32, stream)) != hipSuccess) return done(e);
  if ((e = hipMemsetAsync(buf, 0, (size_t)n4 * 32, stream)) != hipSuccess) return done(e);

  const double lanes = (double)blocks * kThreads * iters * kChains;
  e = best_time(stream, e0, e1, reps, [&] {
    hipLaunchKernelGGL(probe_exp, dim3(blocks), dim3(kThreads), 0, stream, sink, iters, 0.5f);
  }, &t);
  if (e != hipSuccess) return done(e);
  out->exp_per_s = lanes / t;
  e = best_time(stream, e0, e1, reps, [&] {
    hipLaunchKernelGGL(probe_fma, dim3(blocks), dim3(kThreads), 0, stream, sink, iters, 0.5f);
  }, &t);
  if (e != hipSuccess) return done(e);
  out->fma_per_s = lanes / t;
  e = best_time(stream, e0, e1, reps, [&] {
    hipLaunchKernelGGL(probe_update, dim3(blocks), dim3(kThreads), 0, stream, sink, iters, 0.5f);
  }, &t);
  if (e != hipSuccess) return done(e);
  out->update_mix_per_s = lanes / t;
  const int form_blocks = ncu * 3, form_passes = 256;
  e = best_time(stream, e0, e1, reps, [&] {
    hipLaunchKernelGGL(probe_state_loop, dim3(form_blocks), dim3(kThreads), 0, stream, sink, form_passes, kFormStates,
                       0.5f);
  }, &t);
  if (e != hipSuccess) return done(e);
  out->state_loop_per_s = (double)form_blocks * kThreads * form_passes * kFormT * kFormStates / t;

  const float4* lo = reinterpret_cast<const float4*>(buf);
  float4* hi = reinterpret_cast<float4*>(buf + n4 * 16);
  e = best_time(stream, e0, e1, reps, [&] {
    hipLaunchKernelGGL(probe_read, dim3(blocks), dim3(kThreads), 0, stream, lo, 2 * n4, sink);
  }, &t);
  if (e != hipSuccess) return done(e);
  out->hbm_read_Bps = (double)n4 * 32 / t;
  e = best_time(stream, e0, e1, reps, [&] {
    hipLaunchKernelGGL(probe_copy, dim3(blocks), dim3(kThreads), 0, stream, lo, hi, n4);
  }, &t);
  if (e != hipSuccess) return done(e);
  out->hbm_copy_Bps = (double)n4 * 32 / t;  // bytes read + bytes written
  const int lds_iters = 4096;
  e = best_time(stream, e0, e1, reps, [&] {
    hipLaunchKernelGGL(probe_lds, dim3(blocks), dim3(kThreads), 0, stream, sink, lds_iters);
  }, &t);
  if (e != hipSuccess) return done(e);
  out->lds_read_Bps = (double)blocks * kThreads * lds_iters * 4 * 16 / t;
  out->compute_units = ncu;
  return done(hipSuccess);
}

}  // namespace ss2d
