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
// workgroup takes 64 consecutive positions of one orientation (row-major from x,
// column-major from x transposed) and produces the rows of both directions of
// that orientation: direction 0 (or 1) at those positions, and direction 2 (or
// 3) at the mirrored positions L-1-l.  On short maps, where the strips give few
// workgroups, each of the two directions gets a workgroup of its own.
//   * The projection is a (2C x D) by (D x 64) product in fp32 on
//     v_mfma_f32_16x16x4_f32: 2C rows in 16-row tiles dealt to the four waves,
//     the 64 positions as four 16-column tiles whose column j holds position
//     4j + t of tile t, so each lane loads four consecutive positions with one
//     vector load and holds four consecutive outputs per row for one vector
//     store.  Sixteen channels are consumed per step: lane group g (lanes
//     16g..16g+15) feeds channels 4g..4g+3 over four MFMAs, which is one vector
//     load of the weights too.  A wave multiplies only the tiles it holds, and
//     loads the operands two steps ahead.
//   * The R rows of the rank-R dt input go to LDS; dt = W_dt (D x R) times
//     them is a second MFMA product with R in steps of four, its 16-channel
//     blocks dealt to the four waves.
//   * Every store is a 16-byte (fp32) or 8-byte (bf16) write of four
//     consecutive scan positions; a wave writes 256 contiguous bytes (fp32) of
//     each of four rows.
#include "ss2d_kernels.h"

namespace ss2d {
namespace {

constexpr int kStrip = 64;   // positions per workgroup
constexpr int kMaxTiles = 8;  // 16-row tiles of the stacked projection rows: 2C <= 128
constexpr int kMaxRSteps = 16;  // steps of four over R in the dt map (R <= 64 follows from 2C <= 128)
constexpr int64_t kSplitBelow = 512;  // workgroups (B x 2 orientations x strips) under which directions split
constexpr int kKC = 32;  // STAGED: channels per staged chunk

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ProjParams {
  const void* x;   // (B, D, L) row-major pixel order
  const void* xT;  // (B, D, L) column-major pixel order (x with H and W swapped)
  const float* wx;   // (4, C, D)
  const float* wdt;  // (4, D, R)
  void* dt;          // (B, 4, D, L)
  void* Bs;          // (B, 4, N, L)
  void* Cs;          // (B, 4, N, L)
  void* dts;         // (B, 4, R, L) or null: write the low-rank rows instead of the dt map
  int D, L, N, R, C, strips;
  int split;  // 1: a workgroup takes one direction of its orientation (C rows), 0: both (2C rows)
  int tiles;  // 16-row tiles of the workgroup's stacked rows
  int stage_off;  // STAGED: byte offset of the staging buffers in the dynamic LDS (after the dts rows)
};

__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float comp(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// An MFMA operand: four values at i..i+3 of a row of length n, and whether they
// are real (else they count as zero).  VEC: n and i are multiples of 4 and the
// row is aligned, so the four are all there or all missing; the load then
// always happens, at a clamped address, with no branch, and the mask is applied
// where the operand is used: a branch or a select right after each load would
// make the compiler wait for every load in turn.
struct Operand {
  float4 v;
  bool ok;
  __device__ __forceinline__ float4 get() const { return ok ? v : make_float4(0.f, 0.f, 0.f, 0.f); }
};

template <typename S, bool VEC>
__device__ __forceinline__ Operand ld4_operand(const S* row, int i, int n, bool row_ok) {
  if (VEC) {
    const bool ok = row_ok && i < n;
    return Operand{Io<S>::ld4(row, ok ? i : 0), ok};
  }
  return Operand{row_ok ? ld4_guarded<S>(row, i, n, false) : make_float4(0.f, 0.f, 0.f, 0.f), true};
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

// One workgroup of four waves per 64 positions.  The 16-row tiles of the 2C
// stacked rows are dealt to the waves (wave w takes tiles w and w + 4: MTW is
// how many a wave may hold); the dt blocks (direction, 16 channels) likewise.
// When the strips alone would give few workgroups (short maps), each direction
// of an orientation gets its own workgroup (split): C stacked rows, its own dt
// blocks, the same x strip (read twice, the second time mostly from L2).
// VEC: L and D are multiples of 4 and the bases are aligned for the vector forms.
// STAGED (VEC, D a multiple of 32, bf16 rows a multiple of 8): the operands come
// through LDS instead, 32 channels at a time in two buffers: every wave copies
// its share of the next chunk's x strip (32 rows of 64 positions) and weight
// columns (the workgroup's stacked rows, 32 channels each) with the LDS form of
// the 16-byte buffer load while the current chunk is multiplied, so the loads
// hold no registers and one wait and barrier per chunk cover them.  The weight
// rows are 128 bytes, so their 16-byte granules are XOR-swizzled by row pair
// (granule q of row r sits in slot q ^ ((r / 2) % 8)) and the sixteen rows a
// lane group reads land in sixteen different bank groups.  The products are the
// same MFMAs on the same operands in the same order as the register form.
template <typename S, int MTW, bool VEC, bool STAGED>
__global__ __launch_bounds__(256) void project_kernel(ProjParams p) {
  extern __shared__ __align__(16) float dts[];  // [directions of the workgroup][R][kStrip]
  const int D = p.D, L = p.L, N = p.N, R = p.R, C = p.C, MT = p.tiles;
  const int strip = blockIdx.x % p.strips;
  const int rest = blockIdx.x / p.strips;
  const int o = rest & 1;  // orientation: 0 row-major (directions 0, 2), 1 column-major (1, 3)
  const bool split = p.split != 0;
  const int kfix = split ? (rest >> 1) & 1 : 0;  // split: the workgroup's direction is o + 2 kfix
  const int b = rest >> (split ? 2 : 1);
  const int nrows = split ? C : 2 * C;  // stacked rows of this workgroup
  // stacked row m: direction o + 2 kk, row c of it, and its slot kl in the dts buffer
  auto row_of = [&](int m, int& kk, int& c, int& kl) {
    kl = split ? 0 : (m >= C ? 1 : 0);
    kk = split ? kfix : kl;
    c = m - kl * C;
  };
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int pos = strip * kStrip + 4 * col;  // this lane's four positions
  const S* src = static_cast<const S*>(o ? p.xT : p.x) + (int64_t)b * D * L;

  // A operand rows: stacked row m = mt*16 + col is row c of direction o + 2*kk
  const float* arow[MTW];
  bool aval[MTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    const int m = (wave + 4 * i) * 16 + col;
    int kk, c, kl;
    row_of(m, kk, c, kl);
    aval[i] = m < nrows;
    arow[i] = p.wx + (aval[i] ? ((int64_t)(o + 2 * kk) * C + c) * D : 0);
  }
  const bool any = wave < MT;  // this wave holds at least one tile
  const int held = (MT - wave + 3) / 4;  // tiles this wave holds (wave-uniform): only theirs are loaded and multiplied

  f32x4 acc[MTW][4];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (STAGED) {
    constexpr int kXB = kKC * kStrip * (int)sizeof(S);  // bytes of a staged x chunk
    constexpr int kXCopies = kXB / 1024;                // wave-wide 16-byte copies per x chunk
    constexpr int kXRowB = kStrip * (int)sizeof(S);     // bytes of a staged x row
    const int wbytes = MT * 16 * kKC * 4;               // bytes of a staged weight chunk
    char* stg = reinterpret_cast<char*>(dts) + p.stage_off;
    char* const xbuf0 = stg;
    char* const wbuf0 = stg + 2 * kXB;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(src, (uint32_t)((int64_t)D * L * (int64_t)sizeof(S)));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.wx, (uint32_t)((int64_t)4 * C * D * 4));
    const int nwc = MT * 16 / 8;  // weight copies per chunk: eight 128-byte rows each
    auto issue = [&](int d0, int buf) {
#pragma unroll
      for (int j0 = 0; j0 < kXCopies; j0 += 4) {
        const int j = j0 + wave;
        if (j < kXCopies) {
          // lane's 16 bytes: row and first position inside the chunk
          const int per = 64 * 16 / kXRowB;  // rows per copy
          const int row = j * per + lane / (64 / per), e = (lane % (64 / per)) * (16 / (int)sizeof(S));
          const uint32_t voff = (uint32_t)(((int64_t)(d0 + row) * L + strip * kStrip + e) * (int64_t)sizeof(S));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t*)(xbuf0 + buf * kXB + j * 1024), 16, voff, 0, 0,
                                                   0);
        }
      }
      for (int j = wave; j < nwc; j += 4) {
        const int r = 8 * j + (lane >> 3);          // stacked row
        const int q = (lane & 7) ^ ((r >> 1) & 7);  // the granule this lane's slot holds
        int kk, c, kl;
        row_of(r < nrows ? r : 0, kk, c, kl);
        const uint32_t voff = (uint32_t)((((int64_t)(o + 2 * kk) * C + c) * D + d0 + 4 * q) * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_t*)(wbuf0 + buf * wbytes + j * 1024), 16, voff, 0, 0,
                                                 0);
      }
    };
    const int nck = D / kKC;
    issue(0, 0);
    for (int ck = 0; ck < nck; ++ck) {
      wait_vmem();      // this wave's copies of chunk ck: the only memory operations in flight
      __syncthreads();  // every wave's copies are visible, and chunk ck - 1's buffers are free
      if (ck + 1 < nck) issue((ck + 1) * kKC, (ck + 1) & 1);
      if (!any) continue;
      const char* xc = xbuf0 + (ck & 1) * kXB;
      const char* wc = wbuf0 + (ck & 1) * wbytes;
#pragma unroll
      for (int st = 0; st < 2; ++st) {  // two steps of 16 channels
        float4 bc[4], ac[MTW];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const char* xp = xc + (16 * st + 4 * g + j) * kXRowB + 4 * col * (int)sizeof(S);
          if constexpr (sizeof(S) == 4) {
            bc[j] = *reinterpret_cast<const float4*>(xp);
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(xp);
            bc[j] = make_float4(bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xffffu),
                                bf16_to_f32(v.y >> 16));
          }
        }
#pragma unroll
        for (int i = 0; i < MTW; ++i) {
          if (i >= held) break;
          const int r = (wave + 4 * i) * 16 + col;
          const int qs = (4 * st + g) ^ ((r >> 1) & 7);
          ac[i] = *reinterpret_cast<const float4*>(wc + r * (kKC * 4) + 16 * qs);
        }
#pragma unroll
        for (int i = 0; i < MTW; ++i) {
          if (i >= held) break;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[i][t] = mfma_16x16x4(comp(ac[i], j), comp(bc[j], t), acc[i][t]);
        }
      }
    }
  }
  if (any && !STAGED) {
    // operands of 16 channels: x rows dg..dg+3 at this lane's positions, and the
    // weights of this lane's rows at channels dg..dg+3 (dg = d0 + 4g), in two
    // register sets: the operands two steps ahead are loaded before this step's
    // products
    Operand bv[2][4], av[2][MTW] = {};
    auto load_step = [&](int d0, int set) {
      const int dg = d0 + 4 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = dg + j;
        bv[set][j] = ld4_operand<S, VEC>(src + (int64_t)(d < D ? d : 0) * L, pos, L, d < D);
      }
#pragma unroll
      for (int i = 0; i < MTW; ++i)
        if (i < held) av[set][i] = ld4_operand<float, VEC>(arow[i], dg, D, aval[i]);
    };
    auto mma_step = [&](int d0, int set) {
      float4 bc[4], ac[MTW];
#pragma unroll
      for (int j = 0; j < 4; ++j) bc[j] = bv[set][j].get();
#pragma unroll
      for (int i = 0; i < MTW; ++i) ac[i] = i < held ? av[set][i].get() : make_float4(0.f, 0.f, 0.f, 0.f);
      if (d0 + 32 < D) load_step(d0 + 32, set);
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
        if (i >= held) break;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[i][t] = mfma_16x16x4(comp(ac[i], j), comp(bc[j], t), acc[i][t]);
      }
    };
    load_step(0, 0);
    if (16 < D) load_step(16, 1);
    for (int d0 = 0; d0 < D; d0 += 32) {
      mma_step(d0, 0);
      if (d0 + 16 < D) mma_step(d0 + 16, 1);
    }
  }
  if (any) {
    // lane (g, col) holds stacked rows mt*16 + 4g + r at positions pos..pos+3
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      if (i >= held) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = (wave + 4 * i) * 16 + 4 * g + r;
        if (m >= nrows) continue;
        int kk, c, kl;
        row_of(m, kk, c, kl);
        const float4 v = make_float4(acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]);
        if (c < R && p.dts == nullptr) {
          *reinterpret_cast<float4*>(dts + (kl * R + c) * kStrip + 4 * col) = v;
        } else if (c < R) {  // the low-rank rows themselves, in scan order
          const int64_t bk = (int64_t)b * 4 + o + 2 * kk;
          put4<S, VEC>(static_cast<S*>(p.dts) + (bk * R + c) * L, pos, L, kk == 1, v);
        } else {
          const int64_t bk = (int64_t)b * 4 + o + 2 * kk;
          S* row = c < R + N ? static_cast<S*>(p.Bs) + (bk * N + (c - R)) * L
                             : static_cast<S*>(p.Cs) + (bk * N + (c - R - N)) * L;
          put4<S, VEC>(row, pos, L, kk == 1, v);
        }
      }
    }
  }
  if (p.dts != nullptr) return;  // the scan forms dt from the low-rank rows itself
  __syncthreads();

  // dt = W_dt (D x R) times the R rows, per direction, 16 channels at a time.
  // Block jb of the 2 * nd (direction, 16 channels) blocks goes to wave jb % 4;
  // per lane it needs W_dt[k, 16m + col, 4q + g] for the R steps q, and the
  // wave's next block's are loaded before this block's products.
  const int nd = (D + 15) / 16, nrq = (R + 3) / 4, nblk = (split ? 1 : 2) * nd;
  float an[kMaxRSteps] = {};
  auto load_a = [&](int jb) {
    const int kl = jb >= nd ? 1 : 0, kk = split ? kfix : kl;
    const int da = (jb - kl * nd) * 16 + col;
    const float* wrow = p.wdt + ((int64_t)(o + 2 * kk) * D + (da < D ? da : 0)) * R;
#pragma unroll
    for (int q = 0; q < kMaxRSteps; ++q) {
      const int r = 4 * q + g;
      if (q < nrq) an[q] = (r < R && da < D) ? wrow[r] : 0.f;
    }
  };
  if (wave < nblk) load_a(wave);
  for (int jb = wave; jb < nblk; jb += 4) {
    const int kl = jb >= nd ? 1 : 0, kk = split ? kfix : kl;
    const int dm = (jb - kl * nd) * 16;
    float ac[kMaxRSteps];
#pragma unroll
    for (int q = 0; q < kMaxRSteps; ++q) ac[q] = an[q];
    if (jb + 4 < nblk) load_a(jb + 4);
    f32x4 c4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) c4[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < kMaxRSteps; ++q) {
      if (q >= nrq) continue;
      const int r = 4 * q + g;
      const float4 v = r < R ? *reinterpret_cast<const float4*>(dts + (kl * R + r) * kStrip + 4 * col)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int t = 0; t < 4; ++t) c4[t] = mfma_16x16x4(ac[q], comp(v, t), c4[t]);
    }
    S* dtk = static_cast<S*>(p.dt) + ((int64_t)b * 4 + o + 2 * kk) * D * L;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = dm + 4 * g + i;
      if (d < D)
        put4<S, VEC>(dtk + (int64_t)d * L, pos, L, kk == 1, make_float4(c4[0][i], c4[1][i], c4[2][i], c4[3][i]));
    }
  }
}

template <typename S, bool VEC, bool STAGED>
hipError_t launch_tiles(const ProjParams& p, unsigned blocks, size_t lds, hipStream_t stream) {
  if (p.tiles <= 4)
    hipLaunchKernelGGL((project_kernel<S, 1, VEC, STAGED>), dim3(blocks), dim3(256), lds, stream, p);
  else
    hipLaunchKernelGGL((project_kernel<S, 2, VEC, STAGED>), dim3(blocks), dim3(256), lds, stream, p);
  return hipGetLastError();
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
  p.dts = a.dts;
  p.stage_off = 0;
  p.D = (int)a.D;
  p.L = (int)(a.H * a.W);
  p.N = (int)a.N;
  p.R = (int)a.R;
  p.C = (int)(a.R + 2 * a.N);
  p.strips = (p.L + kStrip - 1) / kStrip;
  // one workgroup per direction when the strips of both orientations give fewer
  // than two per compute unit (14x14 maps: 256 strips)
  p.split = a.B * 2 * p.strips < kSplitBelow ? 1 : 0;
  p.tiles = ((p.split ? 1 : 2) * p.C + 15) / 16;
  if ((2 * p.C + 15) / 16 > kMaxTiles) return hipErrorInvalidValue;
  const int64_t blocks = a.B * 2 * p.strips * (p.split ? 2 : 1);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  size_t lds = a.dts ? 0 : (size_t)(p.split ? 1 : 2) * p.R * kStrip * sizeof(float);
  const uintptr_t am = a.dtype == 0 ? 15 : 7;
  const void* dtout = a.dts ? a.dts : a.dt;
  const bool vec = p.L % 4 == 0 && p.D % 4 == 0 && !((uintptr_t)a.x & am) && !((uintptr_t)a.xT & am) &&
                   !((uintptr_t)dtout & am) && !((uintptr_t)a.Bs & am) && !((uintptr_t)a.Cs & am) &&
                   !((uintptr_t)a.wx & 15);
  // staged operands: whole 32-channel chunks, 16-byte copies of x rows (a bf16 row
  // of a multiple of 8 elements), byte offsets inside 32 bits
  const int esz = a.dtype == 0 ? 4 : 2;
  const size_t stage_off = (lds + 15) & ~(size_t)15;
  const size_t staged_lds = stage_off + 2 * ((size_t)kKC * kStrip * esz + (size_t)p.tiles * 16 * kKC * 4);
  const bool staged = vec && p.D % kKC == 0 && (a.dtype == 0 || p.L % 8 == 0) && staged_lds <= 65536 &&
                      (int64_t)p.D * p.L * esz < ((int64_t)1 << 31) && (int64_t)4 * p.C * p.D * 4 < ((int64_t)1 << 31);
  if (staged) {
    p.stage_off = (int)stage_off;
    lds = staged_lds;
  }
  if (a.dtype == 0)
    return staged ? launch_tiles<float, true, true>(p, (unsigned)blocks, lds, a.stream)
                  : vec ? launch_tiles<float, true, false>(p, (unsigned)blocks, lds, a.stream)
                        : launch_tiles<float, false, false>(p, (unsigned)blocks, lds, a.stream);
  return staged ? launch_tiles<uint16_t, true, true>(p, (unsigned)blocks, lds, a.stream)
                : vec ? launch_tiles<uint16_t, true, false>(p, (unsigned)blocks, lds, a.stream)
                      : launch_tiles<uint16_t, false, false>(p, (unsigned)blocks, lds, a.stream);
}

}  // namespace ss2d
