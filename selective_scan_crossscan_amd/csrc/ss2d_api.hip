// C ABI of libss2d.so: argument validation, planning, launch, error reporting.
// The declarations and their contract are in include/ss2d.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "ss2d.h"
#include "ss2d_internal.h"

namespace {

constexpr int kVersion = 1 * 10000 + 2 * 100 + 0;  // 1.2.0
thread_local char g_last_hip_error[256] = "";

void remember(hipError_t e) {
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s (%d)", hipGetErrorString(e), (int)e);
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Shape checks shared by the entry points; max_n: the largest N the caller takes.
int check_shape(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int64_t max_n = 16) {
  if (B < 1 || D < 1 || H < 1 || W < 1) return SS2D_ERR_SHAPE;
  int64_t L, t;
  // Every element count and byte count must fit comfortably: the kernels use
  // 32-bit in-row offsets and 32-bit channel/batch indices, and address staged
  // rows of up to 16 states or channels with 32-bit byte offsets (16 * L * 4 must
  // stay below 2^31).
  if (!mul_ok(H, W, &L) || L > INT32_MAX / 64) return SS2D_ERR_SHAPE;
  if (!mul_ok(B, 4, &t) || !mul_ok(t, D, &t) || !mul_ok(t, L, &t) || !mul_ok(t, 4, &t)) return SS2D_ERR_SHAPE;
  if (B > INT32_MAX / 4 || D > INT32_MAX / 4) return SS2D_ERR_SHAPE;
  if (N < 1 || N > max_n) return SS2D_ERR_UNSUPPORTED_N;
  if (dtype != SS2D_F32 && dtype != SS2D_BF16) return SS2D_ERR_DTYPE;
  return SS2D_OK;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// The temporary of the no-allocation forward (ss2d_forward_noalloc), for callers
// that cannot allocate: one array on every device the library runs on, held until
// the process ends.  Host code never passes its name to a kernel or a copy (on
// the host it only stands for the device variable); it uses the device address
// hipGetSymbolAddress returns for the device in question, kept per device.
constexpr size_t kNoAllocBytes = (size_t)128 << 20;
static __device__ __align__(256) char scratch[kNoAllocBytes];

struct DeviceInfo {
  int device = -1;
  hipMemPool_t pool = nullptr;  // the library's own memory pool on that device
  void* noalloc = nullptr;      // device address of `scratch` on that device
};

// Per-device one-time setup, done with that device current: the library's own
// stream-ordered memory pool for its temporaries (its release threshold keeps
// freed blocks for the next call; other users of the device's default pool are
// not affected), and the device address of the no-allocation array.
struct DevState {
  bool ready = false;
  hipMemPool_t pool = nullptr;
  void* noalloc = nullptr;
};
std::mutex g_dev_mutex;
DevState g_dev[64];

int device_info(DeviceInfo* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    if (e != hipSuccess) remember(e);
    return SS2D_ERR_NO_DEVICE;
  }
  std::lock_guard<std::mutex> lk(g_dev_mutex);
  DevState& st = g_dev[dev];
  if (!st.ready) {
    hipMemPoolProps props;
    memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) {
      remember(e);
      return SS2D_ERR_NO_DEVICE;
    }
    uint64_t threshold = UINT64_MAX;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold);
    if (e != hipSuccess) {
      remember(e);
      (void)hipMemPoolDestroy(pool);
      return SS2D_ERR_NO_DEVICE;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      remember(e != hipSuccess ? e : hipErrorInvalidSymbol);
      (void)hipMemPoolDestroy(pool);
      return SS2D_ERR_NO_DEVICE;
    }
    st.pool = pool;
    st.noalloc = ptr;
    st.ready = true;
  }
  out->device = dev;
  out->pool = st.pool;
  out->noalloc = st.noalloc;
  return SS2D_OK;
}

// Stream-ordered temporary from the library's pool (nothing for 0 bytes).
hipError_t tmp_alloc(const DeviceInfo& di, void** p, size_t bytes, hipStream_t st) {
  *p = nullptr;
  if (bytes == 0) return hipSuccess;
  return hipMallocFromPoolAsync(p, bytes, di.pool, st);
}

hipError_t tmp_free(void* p, hipStream_t st) { return p ? hipFreeAsync(p, st) : hipSuccess; }

}  // namespace

extern "C" {

int ss2d_version(void) { return kVersion; }

int ss2d_trim_memory(void) {
  std::lock_guard<std::mutex> lk(g_dev_mutex);
  for (int d = 0; d < 64; ++d) {
    if (!g_dev[d].ready) continue;
    const hipError_t e = hipMemPoolTrimTo(g_dev[d].pool, 0);
    if (e != hipSuccess) {
      remember(e);
      return SS2D_ERR_HIP;
    }
  }
  return SS2D_OK;
}

const char* ss2d_last_hip_error(void) { return g_last_hip_error; }

int ss2d_measure_peaks(ss2d_peaks* out, int64_t hbm_bytes, void* stream) {
  if (!out) return SS2D_ERR_NULL;
  if (hbm_bytes < (1 << 20) || hbm_bytes > ((int64_t)64 << 30) || hbm_bytes % 32 != 0) return SS2D_ERR_SHAPE;
  DeviceInfo di;
  const int rc = device_info(&di);
  if (rc != SS2D_OK) return rc;
  ss2d::PeakRates r{};
  const hipError_t e = ss2d::measure_peaks(&r, hbm_bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  out->exp_per_s = r.exp_per_s;
  out->fma_per_s = r.fma_per_s;
  out->update_mix_per_s = r.update_mix_per_s;
  out->hbm_read_Bps = r.hbm_read_Bps;
  out->hbm_copy_Bps = r.hbm_copy_Bps;
  out->lds_read_Bps = r.lds_read_Bps;
  out->compute_units = r.compute_units;
  out->state_loop_per_s = r.state_loop_per_s;
  return SS2D_OK;
}

const char* ss2d_status_string(int status) {
  switch (status) {
    case SS2D_OK: return "ok";
    case SS2D_ERR_NULL: return "a required pointer is NULL";
    case SS2D_ERR_SHAPE: return "invalid shape: B, D, H, W must be >= 1 and sizes must fit";
    case SS2D_ERR_UNSUPPORTED_N: return "unsupported state size N (1..256; projections: 1..16)";
    case SS2D_ERR_DTYPE: return "unknown dtype (0 = fp32, 1 = bf16)";
    case SS2D_ERR_ALIAS: return "output y overlaps an input";
    case SS2D_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case SS2D_ERR_NO_DEVICE: return "no usable HIP device";
    case SS2D_ERR_HIP: return "a HIP call or kernel launch failed";
    case SS2D_ERR_NOALLOC_LIMIT: return "the shape needs more temporary memory than ss2d_forward_noalloc holds";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Validation shared by the forward entry points (K directions).  *aligned: every
// storage-type base allows the vector paths (16-byte fp32 / 8-byte bf16
// alignment); element-aligned bases that are not take the scalar path.
int check_forward(const void* x, const void* dt, const float* A_log, const float* dt_bias, const void* Bs,
                  const void* Cs, const float* Ds, const void* y, int64_t B, int64_t D, int64_t H, int64_t W,
                  int64_t N, int dtype, int K, bool* aligned) {
  if (!x || !dt || !A_log || !dt_bias || !Bs || !Cs || !Ds || !y) return SS2D_ERR_NULL;
  const int rc = check_shape(B, D, H, W, N, dtype, ss2d::kMaxStates);
  if (rc != SS2D_OK) return rc;
  const int64_t L = H * W;
  const int64_t s = dtype == SS2D_BF16 ? 2 : 4;
  const int64_t xbytes = B * D * L * s, dtbytes = B * K * D * L * s, bcbytes = B * K * N * L * s;
  const int64_t pbytes = K * D * N * 4, vbytes = K * D * 4;
  if (overlaps(y, xbytes, x, xbytes) || overlaps(y, xbytes, dt, dtbytes) || overlaps(y, xbytes, Bs, bcbytes) ||
      overlaps(y, xbytes, Cs, bcbytes) || overlaps(y, xbytes, A_log, pbytes) ||
      overlaps(y, xbytes, dt_bias, vbytes) || overlaps(y, xbytes, Ds, vbytes))
    return SS2D_ERR_ALIAS;
  const uintptr_t m = (uintptr_t)(s - 1);
  if (((uintptr_t)x & m) || ((uintptr_t)dt & m) || ((uintptr_t)Bs & m) || ((uintptr_t)Cs & m) ||
      ((uintptr_t)y & m) || ((uintptr_t)A_log & 3) || ((uintptr_t)dt_bias & 3) || ((uintptr_t)Ds & 3))
    return SS2D_ERR_ALIGN;
  const uintptr_t vm = (uintptr_t)(4 * s - 1);
  *aligned = !(((uintptr_t)x & vm) || ((uintptr_t)dt & vm) || ((uintptr_t)Bs & vm) || ((uintptr_t)Cs & vm) ||
               ((uintptr_t)y & vm));
  return SS2D_OK;
}

bool lanes_ok(int lanes) { return lanes == 0 || lanes == 16 || lanes == 32 || lanes == 64; }

// noalloc: run from the per-device static array (no transposed copies, so the
// temporary is the merge planes and segment maps only), or fail with
// SS2D_ERR_NOALLOC_LIMIT before touching the device when it does not fit.
int forward_impl(const void* x, const void* dt, const float* A_log, const float* dt_bias, const void* Bs,
                 const void* Cs, const float* Ds, void* y, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                 int dtype, int K, int lanes, void* stream, bool noalloc = false) {
  bool aligned = false;
  int rc = check_forward(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, H, W, N, dtype, K, &aligned);
  if (rc != SS2D_OK) return rc;
  if (!lanes_ok(lanes)) return SS2D_ERR_SHAPE;
  const ss2d::Plan plan = ss2d::make_plan(B, D, H, W, N, dtype, lanes, K, aligned, noalloc);
  if (noalloc && plan.scratch_bytes > kNoAllocBytes) return SS2D_ERR_NOALLOC_LIMIT;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc != SS2D_OK) return rc;

  ss2d::LaunchArgs a;
  a.x = x;
  a.dt = dt;
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.Bs = Bs;
  a.Cs = Cs;
  a.Ds = Ds;
  a.y = y;
  a.B = B;
  a.D = D;
  a.H = H;
  a.W = W;
  a.N = N;
  a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  a.device = di.device;
  a.K = K;

  if (noalloc) {
    const hipError_t e = ss2d::launch_forward(a, plan, static_cast<float*>(di.noalloc));
    if (e != hipSuccess) {
      remember(e);
      return SS2D_ERR_HIP;
    }
    return SS2D_OK;
  }
  void* tmp = nullptr;
  hipError_t e = tmp_alloc(di, &tmp, plan.scratch_bytes, a.stream);
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  e = ss2d::launch_forward(a, plan, static_cast<float*>(tmp));
  const hipError_t e2 = tmp_free(tmp, a.stream);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  return SS2D_OK;
}

int describe_impl(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int lanes, char* buf,
                  int64_t len) {
  if (!buf || len < 1) return SS2D_ERR_NULL;
  const int rc = check_shape(B, D, H, W, N, dtype, ss2d::kMaxStates);
  if (rc != SS2D_OK) return rc;
  if (!lanes_ok(lanes)) return SS2D_ERR_SHAPE;
  const ss2d::Plan pl = ss2d::make_plan(B, D, H, W, N, dtype, lanes);
  snprintf(buf, (size_t)len,
           "kernel=chunked_dpp_scan lanes_per_seq=%d steps_per_lane=%d waves=%d chans_per_block=%d "
           "segments=%d x_transposed=%d plane_transposed=%d blocks=%lld lds_bytes=%zu scratch_bytes=%zu "
           "state_blocks=%d backward_segments=%lld backward_blocks_per_workgroup=%lld "
           "bidir_backward_segments=%lld bidir_backward_blocks_per_workgroup=%lld",
           pl.lanes_per_seq, pl.steps_per_lane, pl.waves, pl.chans_per_block, pl.nseg, pl.xtrans ? 1 : 0,
           pl.transpose ? 1 : 0, (long long)pl.blocks, pl.lds_bytes, pl.scratch_bytes, pl.state_blocks,
           (long long)ss2d::backward_segments(B, D, H, W, N, dtype),
           (long long)ss2d::backward_blocks_per_workgroup(B, D, H, W, N, dtype),
           (long long)ss2d::backward_segments(B, D, 1, H * W, N, dtype, 2),
           (long long)ss2d::backward_blocks_per_workgroup(B, D, 1, H * W, N, dtype, 2));
  return SS2D_OK;
}

}  // namespace

extern "C" {

int ss2d_describe(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, char* buf, int64_t len) {
  return describe_impl(B, D, H, W, N, dtype, 0, buf, len);
}

int ss2d_describe_lanes(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int lanes_per_seq,
                        char* buf, int64_t len) {
  return describe_impl(B, D, H, W, N, dtype, lanes_per_seq, buf, len);
}

int ss2d_forward(const void* x, const void* dt, const float* A_log, const float* dt_bias, const void* Bs,
                 const void* Cs, const float* Ds, void* y, int64_t B, int64_t D, int64_t H, int64_t W,
                 int64_t N, int dtype, void* stream) {
  return forward_impl(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, H, W, N, dtype, 4, 0, stream);
}

int ss2d_forward_noalloc(const void* x, const void* dt, const float* A_log, const float* dt_bias, const void* Bs,
                         const void* Cs, const float* Ds, void* y, int64_t B, int64_t D, int64_t H, int64_t W,
                         int64_t N, int dtype, void* stream) {
  return forward_impl(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, H, W, N, dtype, 4, 0, stream, true);
}

int ss2d_forward_lanes(const void* x, const void* dt, const float* A_log, const float* dt_bias, const void* Bs,
                       const void* Cs, const float* Ds, void* y, int64_t B, int64_t D, int64_t H, int64_t W,
                       int64_t N, int dtype, int lanes_per_seq, void* stream) {
  return forward_impl(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, H, W, N, dtype, 4, lanes_per_seq, stream);
}

int ss2d_bidir_forward(const void* x, const void* dt, const float* A_log, const float* dt_bias, const void* Bs,
                       const void* Cs, const float* Ds, void* y, int64_t B, int64_t D, int64_t L, int64_t N,
                       int dtype, void* stream) {
  // one row of L pixels: the row walk is the sequence order, its reverse the backward path
  return forward_impl(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, 1, L, N, dtype, 2, 0, stream);
}

}  // extern "C"

namespace {

// Checks shared by the two projection entry points: R, the weights' sizes, and
// element alignment of the weights.
int check_projection(int64_t D, int64_t N, int64_t R, const float* wx, const float* wdt) {
  if (R < 1 || R > INT32_MAX / 4 || 2 * (R + 2 * N) > ss2d::project_max_rows()) return SS2D_ERR_SHAPE;
  if (((uintptr_t)wx & 3) || ((uintptr_t)wdt & 3)) return SS2D_ERR_ALIGN;
  (void)D;
  return SS2D_OK;
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// The backward of ss2d_backward (K = 4) and ss2d_bidir_backward (K = 2).
int backward_impl(const void* x, const void* dt, const float* A_log, const float* dt_bias, const void* Bs,
                  const void* Cs, const float* Ds, const void* dy, void* dx, void* ddt, float* dA_log,
                  float* ddt_bias, void* dBs, void* dCs, float* dDs, int64_t B, int64_t D, int64_t H, int64_t W,
                  int64_t N, int dtype, int K, void* stream) {
  if (!x || !dt || !A_log || !dt_bias || !Bs || !Cs || !Ds || !dy || !dx || !ddt || !dA_log || !ddt_bias || !dBs ||
      !dCs || !dDs)
    return SS2D_ERR_NULL;
  int rc = check_shape(B, D, H, W, N, dtype, ss2d::kMaxStates);
  if (rc != SS2D_OK) return rc;
  const int64_t L = H * W;
  const int64_t sz = dtype == SS2D_BF16 ? 2 : 4;
  const int64_t xb = B * D * L * sz, dtb = B * K * D * L * sz, bcb = B * K * N * L * sz, pb = K * D * N * 4,
                vb = K * D * 4;
  const void* ins[8] = {x, dt, A_log, dt_bias, Bs, Cs, Ds, dy};
  const int64_t isz[8] = {xb, dtb, pb, vb, bcb, bcb, vb, xb};
  const void* outs[7] = {dx, ddt, dA_log, ddt_bias, dBs, dCs, dDs};
  const int64_t osz[7] = {xb, dtb, pb, vb, bcb, bcb, vb};
  for (int i = 0; i < 7; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlaps(outs[i], osz[i], ins[j], isz[j])) return SS2D_ERR_ALIAS;
    for (int j = i + 1; j < 7; ++j)
      if (overlaps(outs[i], osz[i], outs[j], osz[j])) return SS2D_ERR_ALIAS;
  }
  // storage-type tensors need element alignment, the fp32 per-channel ones 4 bytes
  const bool io_in[8] = {true, true, false, false, true, true, false, true};
  const bool io_out[7] = {true, true, false, false, true, true, false};
  for (int j = 0; j < 8; ++j)
    if ((uintptr_t)ins[j] & (uintptr_t)(io_in[j] ? sz - 1 : 3)) return SS2D_ERR_ALIGN;
  for (int i = 0; i < 7; ++i)
    if ((uintptr_t)outs[i] & (uintptr_t)(io_out[i] ? sz - 1 : 3)) return SS2D_ERR_ALIGN;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc != SS2D_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* tmp = nullptr;
  hipError_t e = tmp_alloc(di, &tmp, ss2d::backward_scratch_bytes(B, D, H, W, N, dtype, K), st);
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  ss2d::BackwardArgs a{x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, dx, ddt, dA_log, ddt_bias, dBs, dCs, dDs,
                       B, D, H, W, N, dtype, st, K};
  e = ss2d::launch_backward(a, tmp);
  hipError_t e2 = tmp_free(tmp, st);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  return SS2D_OK;
}

// Largest rank for which ss2d_forward_from_x hands the scan the low-rank rows.
constexpr int64_t kFromXLowRankUpTo = 8;

}  // namespace

extern "C" {

int ss2d_project(const void* x, const float* x_proj_weight, const float* dt_projs_weight, void* dt, void* Bs,
                 void* Cs, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int64_t R, int dtype,
                 void* stream) {
  if (!x || !x_proj_weight || !dt_projs_weight || !dt || !Bs || !Cs) return SS2D_ERR_NULL;
  int rc = check_shape(B, D, H, W, N, dtype);
  if (rc != SS2D_OK) return rc;
  rc = check_projection(D, N, R, x_proj_weight, dt_projs_weight);
  if (rc != SS2D_OK) return rc;
  const int64_t L = H * W;
  const int64_t s = dtype == SS2D_BF16 ? 2 : 4;
  const int64_t xbytes = B * D * L * s, dtbytes = B * 4 * D * L * s, bcbytes = B * 4 * N * L * s;
  const int64_t wxbytes = 4 * (R + 2 * N) * D * 4, wdtbytes = 4 * D * R * 4;
  const void* outs[3] = {dt, Bs, Cs};
  const int64_t osz[3] = {dtbytes, bcbytes, bcbytes};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], osz[i], x, xbytes) || overlaps(outs[i], osz[i], x_proj_weight, wxbytes) ||
        overlaps(outs[i], osz[i], dt_projs_weight, wdtbytes))
      return SS2D_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], osz[i], outs[j], osz[j])) return SS2D_ERR_ALIAS;
  }
  const uintptr_t m = (uintptr_t)(s - 1);
  if (((uintptr_t)x & m) || ((uintptr_t)dt & m) || ((uintptr_t)Bs & m) || ((uintptr_t)Cs & m)) return SS2D_ERR_ALIGN;

  DeviceInfo di;
  rc = device_info(&di);
  if (rc != SS2D_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* xT = nullptr;
  hipError_t e = tmp_alloc(di, &xT, (size_t)xbytes, st);
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  e = ss2d::launch_transpose_x(x, xT, B * D, H, W, dtype, st);
  if (e == hipSuccess) {
    ss2d::ProjectArgs pa{x, xT, x_proj_weight, dt_projs_weight, dt, Bs, Cs, B, D, H, W, N, R, dtype, st};
    e = ss2d::launch_project(pa);
  }
  hipError_t e2 = tmp_free(xT, st);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  return SS2D_OK;
}

int ss2d_forward_from_x(const void* x, const float* x_proj_weight, const float* dt_projs_weight,
                        const float* A_log, const float* dt_bias, const float* Ds, void* y, int64_t B, int64_t D,
                        int64_t H, int64_t W, int64_t N, int64_t R, int dtype, void* stream) {
  if (!x || !x_proj_weight || !dt_projs_weight || !A_log || !dt_bias || !Ds || !y) return SS2D_ERR_NULL;
  int rc = check_shape(B, D, H, W, N, dtype);
  if (rc != SS2D_OK) return rc;
  rc = check_projection(D, N, R, x_proj_weight, dt_projs_weight);
  if (rc != SS2D_OK) return rc;
  const int64_t L = H * W;
  const int64_t s = dtype == SS2D_BF16 ? 2 : 4;
  const int64_t xbytes = B * D * L * s, dtbytes = B * 4 * D * L * s, bcbytes = B * 4 * N * L * s;
  const int64_t wxbytes = 4 * (R + 2 * N) * D * 4, wdtbytes = 4 * D * R * 4;
  const int64_t pbytes = 4 * D * N * 4, vbytes = 4 * D * 4;
  if (overlaps(y, xbytes, x, xbytes) || overlaps(y, xbytes, x_proj_weight, wxbytes) ||
      overlaps(y, xbytes, dt_projs_weight, wdtbytes) || overlaps(y, xbytes, A_log, pbytes) ||
      overlaps(y, xbytes, dt_bias, vbytes) || overlaps(y, xbytes, Ds, vbytes))
    return SS2D_ERR_ALIAS;
  const uintptr_t m = (uintptr_t)(s - 1);
  if (((uintptr_t)x & m) || ((uintptr_t)y & m) || ((uintptr_t)A_log & 3) || ((uintptr_t)dt_bias & 3) ||
      ((uintptr_t)Ds & 3))
    return SS2D_ERR_ALIGN;
  // dt, Bs and Cs live in the library's (aligned) temporary; x and y may be
  // element-aligned only, which takes the scalar paths
  const uintptr_t vm = (uintptr_t)(4 * s - 1);
  const bool aligned = !(((uintptr_t)x & vm) || ((uintptr_t)y & vm));

  DeviceInfo di;
  rc = device_info(&di);
  if (rc != SS2D_OK) return rc;
  const ss2d::Plan plan = ss2d::make_plan(B, D, H, W, N, dtype, 0, 4, aligned);
  // Low-rank step input: for small ranks the projection writes the R rows and the
  // scan forms dt from them, instead of writing and reading back the D rows of dt
  // (measured: faster at rank 6 on 56x56 and 256x256 maps; larger ranks add R
  // FMAs per channel and step to an ALU-bound scan and keep the dt map).
  const bool lowrank = R <= kFromXLowRankUpTo && R <= ss2d::kMaxLowRankInput && R <= plan.chans_per_block;
  const int64_t dtrows_bytes = lowrank ? B * 4 * R * L * s : dtbytes;
  // one temporary: x transposed, dt (or its low-rank rows), Bs, Cs, then what the scan itself needs
  const size_t o_dt = up256((size_t)xbytes), o_b = o_dt + up256((size_t)dtrows_bytes);
  const size_t o_c = o_b + up256((size_t)bcbytes), o_scan = o_c + up256((size_t)bcbytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* tmp = nullptr;
  hipError_t e = tmp_alloc(di, reinterpret_cast<void**>(&tmp), o_scan + plan.scratch_bytes, st);
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  void* xT = tmp;
  void *dt = tmp + o_dt, *Bs = tmp + o_b, *Cs = tmp + o_c;
  e = ss2d::launch_transpose_x(x, xT, B * D, H, W, dtype, st);
  if (e == hipSuccess) {
    ss2d::ProjectArgs pa{x, xT, x_proj_weight, dt_projs_weight, lowrank ? nullptr : dt, Bs, Cs, B, D, H, W, N, R,
                         dtype, st};
    pa.dts = lowrank ? dt : nullptr;
    e = ss2d::launch_project(pa);
  }
  if (e == hipSuccess) {
    ss2d::LaunchArgs a;
    a.R = lowrank ? (int)R : 0;
    a.wdt = dt_projs_weight;
    a.x = x;
    a.dt = dt;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.Bs = Bs;
    a.Cs = Cs;
    a.Ds = Ds;
    a.y = y;
    a.B = B;
    a.D = D;
    a.H = H;
    a.W = W;
    a.N = N;
    a.dtype = dtype;
    a.stream = st;
    a.device = di.device;
    // the scan's column walks read the transposed copy made for the projections
    e = ss2d::launch_forward(a, plan, reinterpret_cast<float*>(tmp + o_scan), xT);
  }
  hipError_t e2 = tmp_free(tmp, st);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  return SS2D_OK;
}

int ss2d_channel_last(const void* y, const float* gamma, const float* beta, float eps, int normalize, void* out,
                      int64_t B, int64_t D, int64_t H, int64_t W, int dtype, void* stream) {
  if (!y || !out) return SS2D_ERR_NULL;
  int rc = check_shape(B, D, H, W, 1, dtype);
  if (rc != SS2D_OK) return rc;
  if (D > ss2d::epilogue_max_channels()) return SS2D_ERR_SHAPE;
  if (normalize != 0 && normalize != 1) return SS2D_ERR_SHAPE;
  if (normalize && !(eps >= 0.f && eps <= 1e30f)) return SS2D_ERR_SHAPE;  // also rejects NaN
  const int64_t s = dtype == SS2D_BF16 ? 2 : 4;
  const int64_t ybytes = B * D * H * W * s, vbytes = D * 4;
  if (overlaps(out, ybytes, y, ybytes) || (gamma && overlaps(out, ybytes, gamma, vbytes)) ||
      (beta && overlaps(out, ybytes, beta, vbytes)))
    return SS2D_ERR_ALIAS;
  const uintptr_t m = (uintptr_t)(s - 1);
  if (((uintptr_t)y & m) || ((uintptr_t)out & m) || ((uintptr_t)gamma & 3) || ((uintptr_t)beta & 3))
    return SS2D_ERR_ALIGN;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc != SS2D_OK) return rc;
  ss2d::EpilogueArgs a{y, gamma, beta, out, eps, normalize != 0, B, D, H, W, dtype, static_cast<hipStream_t>(stream)};
  hipError_t e = ss2d::launch_channel_last(a);
  if (e != hipSuccess) {
    remember(e);
    return SS2D_ERR_HIP;
  }
  return SS2D_OK;
}

int ss2d_backward(const void* x, const void* dt, const float* A_log, const float* dt_bias, const void* Bs,
                  const void* Cs, const float* Ds, const void* dy, void* dx, void* ddt, float* dA_log,
                  float* ddt_bias, void* dBs, void* dCs, float* dDs, int64_t B, int64_t D, int64_t H, int64_t W,
                  int64_t N, int dtype, void* stream) {
  return backward_impl(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, dx, ddt, dA_log, ddt_bias, dBs, dCs, dDs, B, D, H, W, N,
                       dtype, 4, stream);
}

int ss2d_bidir_backward(const void* x, const void* dt, const float* A_log, const float* dt_bias, const void* Bs,
                        const void* Cs, const float* Ds, const void* dy, void* dx, void* ddt, float* dA_log,
                        float* ddt_bias, void* dBs, void* dCs, float* dDs, int64_t B, int64_t D, int64_t L,
                        int64_t N, int dtype, void* stream) {
  // one row of L tokens, as for ss2d_bidir_forward: the two paths are the row walk and its reverse
  return backward_impl(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, dx, ddt, dA_log, ddt_bias, dBs, dCs, dDs, B, D, 1, L, N,
                       dtype, 2, stream);
}

}  // extern "C"
