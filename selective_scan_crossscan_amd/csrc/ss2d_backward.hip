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
// How it runs (the forward's decomposition, run twice).
//   * A workgroup takes one or two blocks of 16 channels of one (batch,
//     direction); a DPP row of 16 lanes owns one channel, lane s the 8
//     consecutive steps 8s.. of each 128-step chunk, and every lane loops over
//     the states.  What belongs to state n of a channel (its A, carries, dA) is
//     held by lane n of the row.
//   * Pass A walks the chunks forwards: per state each lane folds its steps into
//     one affine map h -> P h + Q, an inclusive prefix scan of the row's maps
//     (DPP row_shr) gives every lane its entering state, which is stored; lane
//     15 carries the chunk's last state to the next chunk.
//   * Pass B walks the chunks backwards: per state each lane recomputes its
//     states from the stored one, folds the adjoint q_l = a_{l+1} q_{l+1} +
//     Cs_l g_l over its steps from the right, a suffix scan (DPP row_shl) gives
//     every lane the adjoint entering from its right, and the lane walks its
//     steps backwards accumulating du and ddelta over the states in registers.
//     Lane 0 carries q and a of the chunk's first step to the chunk before.
//   * dBs/dCs terms are summed per state and chunk over a wave's four channels
//     with lane swaps, over the four waves through LDS, and over the workgroup's
//     blocks in a per-thread LDS accumulator, then written as one partial per
//     workgroup; a second kernel sums the partials in a fixed order, so results
//     are deterministic (no atomics).
//   * Column walks read transposed copies of x and dy (made first), so every
//     operand load is contiguous along the steps; with L a multiple of 4 and
//     aligned rows a lane's eight steps are two 16-byte (bf16: 8-byte) loads per
//     operand and two stores per output, also along the reversed walks.
//   * du goes to a temporary; a merge kernel (whole planes in LDS up to 4096
//     pixels, else 32 x 32 tiles) sums it into dx, and a small kernel sums the
//     per-batch (and per-segment) parameter gradients.
//   * Maps too long for one workgroup per channel block to fill the chip are cut
//     into segments of consecutive chunks, one workgroup each, in three launches:
//     pass A from a zero state, which also folds the segment's whole forward map
//     h -> P h + F and adjoint map r -> P r + R (r: the adjoint entering from the
//     right times the decay of the step it enters at); a small kernel chains the
//     segments in order to their true entering state and adjoint; pass B, which
//     corrects each stored state by the entering state times the decay since the
//     segment's start.
#include <algorithm>

#include "ss2d_kernels.h"

namespace ss2d {
namespace {

constexpr int kBwdChans = 16;  // channels per channel block (a workgroup takes one or two)
constexpr int kBwdStates = 16;  // states per pass (a DPP row holds one per lane); larger N runs in passes

struct BwdParams {
  const void* x;  // x, dt, Bs, Cs, dy, xT, dyT and ddt in the storage type
  const void* dt;
  const float* A_log;
  const float* dt_bias;
  const void* Bs;
  const void* Cs;
  const float* Ds;
  const void* dy;
  const void* xT;   // x and dy with H and W swapped: column walks read them in order
  const void* dyT;
  void* ddt;   // (B, 4, D, L) out
  float* du;   // (B, 4, D, L) temporary
  float* hck;  // (B*4, nseg, D, N, 16) temporary: state entering each lane's steps of each chunk
  float* dBp;  // (B*4, ceil(nblk / CPB), N, L) temporary: one partial per workgroup's channel blocks
  float* dCp;
  float* dAp;  // (B, nsp, 4D, N) temporary
  float* dbp;  // (B, nsp, 4D) temporary
  float* dDp;
  float* cdl;   // (B*4, nseg, D, 16): delta summed from the segment's start to each lane's first step (nsp > 1)
  float* segP;  // (B*4, nsp, D, N): the segment's decay, forward offset, adjoint offset; the carry kernel
  float* segF;  //   turns F into the state entering the segment and R into the adjoint entering it
  float* segR;
  int D, H, W, L, N;
  int K;           // directions: 4 (the cross scan) or 2 (the two-path scan over a 1 x L sequence)
  int Nt, n0;      // all states (the row stride of A_log, Bs, Cs, dA) and this pass's first state
  int pass;        // state blocks of 16: 0 the only pass, 1 the first of several, 2 a middle one, 3 the last
  float* ddt_acc;  // (B, 4, D, L) fp32 sum of ddt over the passes so far (passes 1-3)
  int nseg, nblk;  // 128-step chunks per sequence, 16-channel blocks
  int nsp, cps;    // segments, chunks per segment
};

// Sum over the 16 lanes of a DPP row (four rotations).
__device__ __forceinline__ float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false));  // row_ror:1
  return v;
}

// ---------------------------------------------------------------- chunked form
// The same gradients with the forward's decomposition: a DPP row of 16 lanes owns
// one channel, lane s the kCT consecutive steps s*kCT.. of each 128-step chunk,
// and every lane loops over the states.  The recurrence crosses the lanes as an
// inclusive prefix scan of affine maps h -> P h + Q (pass A, chunks left to
// right), its adjoint q_l = a_{l+1} q_{l+1} + Cs_l g_l as a suffix scan of the
// same maps (pass B, chunks right to left), so the sums over states are plain
// register accumulations and each step costs a few operations per state.
constexpr int kCT = 8;                // steps per lane in a chunk
constexpr int kChunk = 16 * kCT;      // steps per chunk
constexpr int kPad = kChunk + 16;     // LDS row: one pad slot per lane's run, so a row's lanes hit distinct banks

// Sums over the four rows of a wave (its four channels), by halves.  The 32-lane
// swap exchanges lanes 32-63 of x with lanes 0-31 of y; adding the two results
// leaves x summed over rows r and r + 2 in lanes 0-31 and y summed likewise in
// lanes 32-63.  The 16-lane swap exchanges the odd rows of x with the even rows of
// y; adding leaves x summed over rows r and r + 1 in rows 0 and 2 and y in rows 1
// and 3.
__device__ __forceinline__ float swap_add32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_add16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dppf(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Value of lane j (0..15) of this lane's row.
__device__ __forceinline__ float row_lane(float v, int j) {
  const int lane = threadIdx.x & 63;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane & ~15) + j) << 2, __float_as_int(v)));
}

constexpr int kRowShr = 0x110;  // row_shr:n = 0x110 + n (from lane i - n)
constexpr int kRowShl = 0x100;  // row_shl:n = 0x100 + n (from lane i + n)

// Scans over a row of maps x -> P x + Q.  Prefix: scan_inclusive<16> (lane i
// composes lanes 0..i, the lower lanes applied first) and incoming_state<16> (the
// previous lane's map applied to a carry).  Suffix, for the adjoint, which runs
// from the end: the same fused levels reading from the right (row_shl), lane i
// composing lanes i..15, the higher lanes applied first; a lane past the row edge
// is not written, which is the identity.  Wait states as in the prefix forms.
__device__ __forceinline__ void scan_suffix16(float& P, float& Q) {
  asm volatile("s_nop 1\n\t" SS2D_SCAN_STEP("row_shl:1 row_mask:0xf") SS2D_SCAN_NEXT("row_shl:2 row_mask:0xf")
                   SS2D_SCAN_NEXT("row_shl:4 row_mask:0xf") SS2D_SCAN_NEXT("row_shl:8 row_mask:0xf")
               : "+v"(P), "+v"(Q));
}

// The next lane's map applied to carry: P[i+1] * carry + Q[i+1]; lane 15 keeps
// carry (its source is past the row edge).
__device__ __forceinline__ float from_right16(float P, float Q, float carry) {
  float h = carry;
  asm volatile(
      "s_nop 1\n\t"
      "v_mul_f32_dpp %0, %1, %0 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %0, %2, %0 row_shl:1 row_mask:0xf bank_mask:0xf"
      : "+v"(h)
      : "v"(P), "v"(Q));
  return h;
}

// MODE kWhole: one workgroup walks every chunk, pass A then pass B.  kSegMaps: pass
// A over one segment from a zero state, with the segment's maps as records.
// kSegGrads: pass B over one segment, from the chained records.  CPB channel
// blocks per workgroup share each chunk's Bs/Cs staging and write one dBs/dCs
// partial between them.
enum BwdMode { kWhole = 0, kSegMaps = 1, kSegGrads = 2 };

// One channel as seen by the lanes of its DPP row: validity, parameters and the
// rows it reads.
template <typename S>
struct BwdChan {
  bool valid;
  int d, c_idx;  // channel (0 when invalid) and its index k * D + d in the per-channel parameters
  float bias, dsk;
  const S* xs;   // u along the direction's walk (x or its transpose)
  const S* gs;   // g likewise
  const S* dtr;  // dt row
  int64_t row;   // start of the (b, k, d) row in (B, K, D, L) tensors
  __device__ BwdChan(const BwdParams& p, int bk, int dd) {
    // slot j of K; the walk k: 0 rows, 1 columns, 2 and 3 the same reversed (K = 2: 0 and 2)
    const int j = p.K == 4 ? (bk & 3) : (bk & 1), b = p.K == 4 ? bk >> 2 : bk >> 1;
    const int k = p.K == 4 ? j : 2 * j, D = p.D, L = p.L;
    valid = dd < D;
    d = valid ? dd : 0;
    c_idx = j * D + d;
    bias = p.dt_bias[c_idx];
    dsk = p.Ds[c_idx];
    xs = static_cast<const S*>((k & 1) ? p.xT : p.x) + ((int64_t)b * D + d) * L;
    gs = static_cast<const S*>((k & 1) ? p.dyT : p.dy) + ((int64_t)b * D + d) * L;
    dtr = static_cast<const S*>(p.dt) + ((int64_t)bk * D + d) * L;
    row = ((int64_t)bk * D + d) * L;
  }
};

// Per channel block, lane s's register copy of what belongs to state s of its
// row's channel (read by the row's lanes with row_lane), and the lane's sums.
struct BwdRegs {
  float a2;      // A * log2(e)
  float h;       // pass A: the state carried to the next chunk; kSegGrads: the state entering the segment
  float q, a;    // pass B: the adjoint and the decay at the first step of the chunk walked last
  float dA;      // sum of q delta a h_{l-1}
  float ap, aq;  // kSegMaps: the adjoint map of the chunks walked so far
  float dbias, dD;
};

// At most 168 VGPRs (three waves per SIMD): two blocks per workgroup would
// otherwise take 188 and run at two; the few values spilled are reloaded per
// chunk, outside the state loop.  VEC: L is a multiple of 4 and the rows are
// aligned, so a lane's steps (a multiple of 8 from the chunk's start) come in
// groups of four wholly inside or past the sequence, read and written with one
// 16-byte (fp32) or 8-byte (bf16) access each, also along the reversed walks.
template <typename S, int MODE, int CPB, bool VEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void bwd_chunk_kernel(BwdParams p) {
  __shared__ float sB[16][kPad];
  __shared__ float sC[16][kPad];
  __shared__ float wred[2][4][2][kPad];    // [state parity][wave][dCs, dBs][step]: the waves' four-channel sums
  __shared__ float acc[16][256];  // [state][thread]: the sums at the thread's step, over the blocks so far
  // The blocks take turns in one register set: after each block the thread swaps
  // it with its stash slot (the other block's, CPB = 2), so the loop over blocks
  // stays rolled and the registers those of one block.
  __shared__ BwdRegs stash[CPB > 1 ? 256 : 1];
  static_assert(CPB == 1 || CPB == 2, "one or two channel blocks per workgroup");
  const int tid = threadIdx.x, s = tid & 15, ch = tid >> 4;
  // Workgroups are dealt round-robin over the 8 XCDs; consecutive work ids (the
  // segments and channel groups of one batch and direction, which read the same
  // Bs/Cs, then the directions of one batch, which read the same x and dy) are
  // put on one XCD, so that they share its L2.
  const int nb = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = nb >> 3, rem = nb & 7;
  const int wid = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int sg = wid % p.nsp;
  const int grp = wid / p.nsp;
  const int ngrp = (p.nblk + CPB - 1) / CPB;
  const int blk0 = (grp % ngrp) * CPB;  // this workgroup's first channel block
  const int bk = grp / ngrp;            // b * K + the direction's slot
  const int k = p.K == 4 ? (bk & 3) : 2 * (bk & 1), b = p.K == 4 ? bk >> 2 : bk >> 1;
  const int D = p.D, L = p.L, N = p.N, nch = p.nseg;
  const int c0 = sg * p.cps, c1 = min(nch, c0 + p.cps);
  const int j0 = s * kCT, jp0 = j0 + s;  // first step of this lane in the chunk, and its padded LDS slot
  const S* Bb = static_cast<const S*>(p.Bs) + ((int64_t)bk * p.Nt + p.n0) * L;
  const S* Cb = static_cast<const S*>(p.Cs) + ((int64_t)bk * p.Nt + p.n0) * L;
  // this thread's dCs (tid < kChunk) or dBs output step in a chunk
  static_assert(2 * kChunk == 256, "one dCs or dBs sum per thread");
  const int which = tid / kChunk, jo = tid - which * kChunk, jpo = jo + jo / kCT;

  BwdRegs rr;  // the current block's
  auto next_block = [&]() {  // rr <-> stash (CPB = 2): blocks 0, 1, 0, 1, ...
    if (CPB > 1) {
      const BwdRegs t = stash[tid];
      stash[tid] = rr;
      rr = t;
    }
  };
#pragma unroll 1
  for (int cb = 0; cb < CPB; ++cb) {
    const BwdChan<S> cn(p, bk, (blk0 + cb) * kBwdChans + ch);
    const bool rval = cn.valid && s < N;
    const int64_t rec = (((int64_t)bk * p.nsp + sg) * D + cn.d) * N + s;  // this lane's segment record (state s)
    rr.a2 = rval ? -expf(p.A_log[(int64_t)cn.c_idx * p.Nt + p.n0 + s]) * kLog2e : 0.f;
    rr.h = MODE == kSegGrads && rval ? p.segF[rec] : 0.f;
    rr.q = MODE == kSegGrads && rval ? p.segR[rec] : 0.f;
    rr.a = 1.f;
    rr.dA = 0.f;
    rr.ap = 1.f;
    rr.aq = 0.f;
    rr.dbias = rr.dD = 0.f;
    next_block();
  }

  // Per lane and chunk: delta, u, xu = delta * u (the input's factor of every
  // state), g and sigmoid(dt + bias).  (Reading u and dt again at the chunk's end
  // instead of keeping them measured slower.)
  float del[kCT], uu[kCT], xu[kCT], gg[kCT], sig[kCT];
  auto lane_step = [&](const BwdChan<S>& cn, int c, int i, int& li, int& xi) {
    const int l = c * kChunk + j0 + i;
    const bool in = cn.valid && l < L;
    li = in ? l : 0;
    xi = in ? (k >= 2 ? L - 1 - l : l) : 0;
    return in;
  };
  // Every load is issued first, at in-bounds (clamped) indices, so that all of
  // them are in flight together; steps past the end are zeroed afterwards.
  // (Loads under a per-step condition were issued and waited for one by one.)
  auto load_lane = [&](const BwdChan<S>& cn, int c, bool with_g) {
    float dtv[kCT];
    bool inr[kCT];
    if constexpr (VEC) {
      static_assert(kCT % 4 == 0, "groups of four steps");
      const bool rev = k >= 2;
      float4 dq[kCT / 4], uq[kCT / 4], gq[kCT / 4];
#pragma unroll
      for (int g = 0; g < kCT / 4; ++g) {
        const int l = c * kChunk + j0 + 4 * g;
        const bool in = cn.valid && l < L;
        const int li = in ? l : 0, xi = in ? (rev ? L - 4 - l : l) : 0;
        dq[g] = Io<S>::ld4(cn.dtr, li);
        uq[g] = Io<S>::ld4(cn.xs, xi);
        gq[g] = with_g ? Io<S>::ld4(cn.gs, xi) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) inr[4 * g + i] = in;
      }
#pragma unroll
      for (int g = 0; g < kCT / 4; ++g) {
        const float4 u4 = uq[g], g4 = gq[g];
        dtv[4 * g] = dq[g].x; dtv[4 * g + 1] = dq[g].y; dtv[4 * g + 2] = dq[g].z; dtv[4 * g + 3] = dq[g].w;
        uu[4 * g] = rev ? u4.w : u4.x; uu[4 * g + 1] = rev ? u4.z : u4.y;
        uu[4 * g + 2] = rev ? u4.y : u4.z; uu[4 * g + 3] = rev ? u4.x : u4.w;
        gg[4 * g] = rev ? g4.w : g4.x; gg[4 * g + 1] = rev ? g4.z : g4.y;
        gg[4 * g + 2] = rev ? g4.y : g4.z; gg[4 * g + 3] = rev ? g4.x : g4.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kCT; ++i) {
        int li, xi;
        inr[i] = lane_step(cn, c, i, li, xi);
        dtv[i] = Io<S>::ld(cn.dtr, li);
        uu[i] = Io<S>::ld(cn.xs, xi);
        gg[i] = with_g ? Io<S>::ld(cn.gs, xi) : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < kCT; ++i) {
      const float pre = dtv[i] + cn.bias;
      const bool in = inr[i];
      del[i] = in ? softplus_f32(pre) : 0.f;
      uu[i] = in ? uu[i] : 0.f;
      sig[i] = in ? __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-pre * kLog2e)) : 0.f;  // 1-ulp reciprocal
      xu[i] = del[i] * uu[i];
      gg[i] = in ? gg[i] : 0.f;
    }
  };
  // Bs (and Cs) of chunk c into LDS: element e = tid + 256 r is state 2 r + tid / 128
  // at step tid % 128, so a wave reads 64 consecutive steps of one state row.  All
  // of a thread's loads are in flight together, as in load_lane; the row offsets
  // are wave-uniform (scalar), and past the end the address is clamped in bounds.
  auto stage = [&](int c, bool with_c) {
    constexpr int kPer = 16 * kChunk / 256;  // elements per thread and tensor
    if constexpr (VEC) {
      // four steps of kPer / 4 state rows per thread: thread tid reads steps
      // 4 (tid % 32) .. + 3 of rows tid / 32 + 8 r, so a wave reads two whole rows
      static_assert(kChunk == 128 && kPer == 8, "a row is 32 groups of four steps");
      const int j = 4 * (tid & 31), l = c * kChunk + j, n0 = tid >> 5;
      const bool lin = l < L;  // the four steps are all inside or all past the end
      const int lc = lin ? l : 0;
      float4 vb[2], vc[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int n = n0 + 8 * r, nc = n < N ? n : N - 1;
        vb[r] = Io<S>::ld4(Bb + (int64_t)nc * L, lc);
        vc[r] = with_c ? Io<S>::ld4(Cb + (int64_t)nc * L, lc) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      const int jp = j + j / kCT;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int n = n0 + 8 * r;
        const bool in = n < N && lin;
        const float4 zb = in ? vb[r] : make_float4(0.f, 0.f, 0.f, 0.f);
        sB[n][jp] = zb.x; sB[n][jp + 1] = zb.y; sB[n][jp + 2] = zb.z; sB[n][jp + 3] = zb.w;
        if (with_c) {
          const float4 zc = in ? vc[r] : make_float4(0.f, 0.f, 0.f, 0.f);
          sC[n][jp] = zc.x; sC[n][jp + 1] = zc.y; sC[n][jp + 2] = zc.z; sC[n][jp + 3] = zc.w;
        }
      }
      return;
    }
    const int hi = __builtin_amdgcn_readfirstlane(tid >> 7);
    const int j = tid & (kChunk - 1), l = c * kChunk + j;
    const int lc = l < L ? l : L - 1;
    float vb[kPer], vc[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int n = 2 * r + hi, nc = n < N ? n : N - 1;
      vb[r] = Io<S>::ld(Bb + lc, (int64_t)nc * L);
      vc[r] = with_c ? Io<S>::ld(Cb + lc, (int64_t)nc * L) : 0.f;
    }
    const int jp = j + j / kCT;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int n = 2 * r + hi;
      const bool in = n < N && l < L;
      sB[n][jp] = in ? vb[r] : 0.f;
      if (with_c) sC[n][jp] = in ? vc[r] : 0.f;
    }
  };
  auto hck = [&](const BwdChan<S>& cn, int c, int n) -> float& {
    return p.hck[((((int64_t)bk * nch + c) * D + cn.d) * N + n) * 16 + s];
  };
  auto cdl = [&](const BwdChan<S>& cn, int c) -> float& {
    return p.cdl[(((int64_t)bk * nch + c) * D + cn.d) * 16 + s];
  };

  if (MODE != kSegGrads) {
    // pass A: the state entering each lane's steps of every chunk
    constexpr bool seg = MODE == kSegMaps;
    static_assert(MODE != kSegMaps || CPB == 1, "segment maps take one block per workgroup");
    float cum = 0.f;  // kSegMaps: delta summed over the segment's chunks before this one
    for (int c = c0; c < c1; ++c) {
      stage(c, seg);
#pragma unroll 1
      for (int cb = 0; cb < CPB; ++cb) {
        const BwdChan<S> cn(p, bk, (blk0 + cb) * kBwdChans + ch);
        load_lane(cn, c, seg);
        if (cb == 0) __syncthreads();  // the chunk's Bs (and Cs) staged
        float sdel = 0.f;
#pragma unroll
        for (int i = 0; i < kCT; ++i) sdel += del[i];
        if (seg) {
          float incl = sdel;  // inclusive prefix over the row
          incl += dppf<kRowShr + 1>(0.f, incl);
          incl += dppf<kRowShr + 2>(0.f, incl);
          incl += dppf<kRowShr + 4>(0.f, incl);
          incl += dppf<kRowShr + 8>(0.f, incl);
          if (cn.valid) cdl(cn, c) = cum + (incl - sdel);
          cum += row_lane(incl, 15);
        }
        // Two states per iteration (n and n1 = n + 1, or n again for an odd last
        // one): their chains are independent, so the scheduler can interleave them.
        // Every LDS and cross-lane read of both comes first (the scans' asm blocks
        // order memory accesses around them); stores and lane updates come after
        // both.  Lane n1's carried state is read before lane n's is updated, which
        // it does not depend on.
        for (int n = 0; n < N; n += 2) {
          const int n1 = n + 1 < N ? n + 1 : n;
          const int nn[2] = {n, n1};
          float hin[2], hout[2], Pb0[2], R0[2], A2v[2], hcv[2], bv[2][kCT], cv[2][kCT];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            A2v[t] = row_lane(rr.a2, nn[t]);
            hcv[t] = row_lane(rr.h, nn[t]);
#pragma unroll
            for (int i = 0; i < kCT; ++i) {
              bv[t][i] = sB[nn[t]][jp0 + i];
              cv[t][i] = seg ? sC[nn[t]][jp0 + i] : 0.f;
            }
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float A2 = A2v[t], hc = hcv[t];
            const float Pl = __builtin_amdgcn_exp2f(A2 * sdel);
            float P = Pl, Q = 0.f, a[kCT];
#pragma unroll
            for (int i = 0; i < kCT; ++i) {
              a[i] = __builtin_amdgcn_exp2f(del[i] * A2);
              Q = fmaf(a[i], Q, xu[i] * bv[t][i]);
            }
            if (seg) {
              // the lane's adjoint map r -> Pl r + R (r enters after its last step),
              // composed over the row: lane 0 holds the chunk's
              float Pb = Pl, R = 0.f;
#pragma unroll
              for (int i = kCT - 1; i >= 0; --i) R = a[i] * fmaf(cv[t][i], gg[i], R);
              scan_suffix16(Pb, R);
              Pb0[t] = row_lane(Pb, 0);
              R0[t] = row_lane(R, 0);
            }
            scan_inclusive<16>(P, Q);
            hin[t] = incoming_state<16>(P, Q, hc, s);
            hout[t] = row_lane(fmaf(P, hc, Q), 15);  // the state leaving the chunk (lane 15's)
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (t == 1 && n1 == n) break;
            const int m = nn[t];
            if (seg && s == m) {  // the chunks so far, then this one: (ap, aq) o (Pb0, R0)
              rr.aq = fmaf(rr.ap, R0[t], rr.aq);
              rr.ap *= Pb0[t];
            }
            if (s == m) rr.h = hout[t];
            if (cn.valid) hck(cn, c, m) = hin[t];
          }
        }
        next_block();
      }
      __syncthreads();  // the next chunk's staging overwrites Bs/Cs
    }
    if (seg) {
      const BwdChan<S> cn(p, bk, blk0 * kBwdChans + ch);
      if (cn.valid && s < N) {
        const int64_t rec = (((int64_t)bk * p.nsp + sg) * D + cn.d) * N + s;
        p.segP[rec] = rr.ap;
        p.segF[rec] = rr.h;
        p.segR[rec] = rr.aq;
      }
      return;
    }
  }

  // pass B: chunks from the last; the adjoint enters each lane from the right.
  // Per step, over the states: tq = sum_n q Bs and sa = sum_n q A a h_{l-1}, so
  // that du = delta tq + Ds g and ddelta = sa + u tq take no per-state product.
  int par = 0;  // consecutive states use alternate wred buffers
  // The four waves' sums of state n (buffer b) at this thread's step, added to
  // the earlier blocks' in the thread's own accumulator entry.
  auto wave_sums = [&](int b, int n, int cb) {
    const float sum = ((wred[b][0][which][jpo] + wred[b][1][which][jpo]) + wred[b][2][which][jpo]) +
                      wred[b][3][which][jpo];
    acc[n][tid] = cb > 0 ? acc[n][tid] + sum : sum;  // the earlier blocks first
  };
  for (int c = c1 - 1; c >= c0; --c) {
    stage(c, true);
    const int lo = c * kChunk + jo;  // this thread's dCs/dBs step
#pragma unroll 1
    for (int cb = 0; cb < CPB; ++cb) {
      const BwdChan<S> cn(p, bk, (blk0 + cb) * kBwdChans + ch);
      load_lane(cn, c, true);
      if (cb == 0) __syncthreads();  // the chunk's Bs/Cs staged
      float tq[kCT], sa[kCT];
#pragma unroll
      for (int i = 0; i < kCT; ++i) tq[i] = sa[i] = 0.f;
      float sd1 = 0.f;  // delta summed over the lane's steps after its first
#pragma unroll
      for (int i = 1; i < kCT; ++i) sd1 += del[i];
      const float cum = MODE == kSegGrads && cn.valid ? cdl(cn, c) : 0.f;
      // the stored state of the next state index is loaded one iteration ahead
      // (the channel index is clamped, so the address is in bounds)
      // and what it reads from the row's other lanes likewise (lane n + 1's carries
      // are not changed by iteration n, which only updates lane n's)
      float h_next = hck(cn, c, 0);
      float A2n = row_lane(rr.a2, 0), acn = row_lane(rr.a, 0), qcn = row_lane(rr.q, 0);
      float hsn = MODE == kSegGrads ? row_lane(rr.h, 0) : 0.f;
      for (int n = 0; n < N; ++n) {
        const float A2 = A2n, A = A2 * kLn2, acar = acn, qcar = qcn, hseg = hsn;
        float a[kCT], h[kCT], cg[kCT];
        float h_in = cn.valid ? h_next : 0.f;
        if (n + 1 < N) {
          h_next = hck(cn, c, n + 1);
          A2n = row_lane(rr.a2, n + 1);
          acn = row_lane(rr.a, n + 1);
          qcn = row_lane(rr.q, n + 1);
          if (MODE == kSegGrads) hsn = row_lane(rr.h, n + 1);
        }
        // a segment's stored states start from zero: add the entering state's decayed part
        if (MODE == kSegGrads) h_in = fmaf(__builtin_amdgcn_exp2f(A2 * cum), hseg, h_in);
        float hv = h_in;
#pragma unroll
        for (int i = 0; i < kCT; ++i) {
          a[i] = __builtin_amdgcn_exp2f(del[i] * A2);
          hv = fmaf(a[i], hv, xu[i] * sB[n][jp0 + i]);
          h[i] = hv;
        }
        const float a_right = dppf<kRowShl + 1>(acar, a[0]);  // decay of the step after this lane's last
        // the lane's map q_after -> P q_after + Q: P is the decay over its steps after the first, then a_right
        float P = a_right * __builtin_amdgcn_exp2f(A2 * sd1), Q = 0.f;
#pragma unroll
        for (int i = kCT - 1; i >= 0; --i) {
          const float an = i == kCT - 1 ? a_right : a[i + 1];
          cg[i] = sC[n][jp0 + i] * gg[i];
          Q = fmaf(an, Q, cg[i]);
        }
        scan_suffix16(P, Q);
        float q = from_right16(P, Q, qcar);  // adjoint at the step after this lane's last
        float dA = 0.f, hg[kCT], qx[kCT];  // the dCs and dBs terms of each step
#pragma unroll
        for (int i = kCT - 1; i >= 0; --i) {
          const float an = i == kCT - 1 ? a_right : a[i + 1];
          q = fmaf(an, q, cg[i]);
          const float hp = i > 0 ? h[i - 1] : h_in;
          const float w = q * a[i] * hp;
          tq[i] = fmaf(q, sB[n][jp0 + i], tq[i]);
          sa[i] = fmaf(A, w, sa[i]);
          dA = fmaf(del[i], w, dA);
          hg[i] = h[i] * gg[i];
          qx[i] = q * xu[i];
        }
        const float q0 = row_lane(q, 0), a0 = row_lane(a[0], 0);
        dA = row_sum16(dA);
        if (s == n) {  // carried to the chunk before
          rr.q = q0;
          rr.a = a0;
          rr.dA += dA;
        }
        // the terms summed over the wave's four channels: after the two swap rounds,
        // lane (row r, s) holds, for t = 0..3, the sum for step 2t + (r & 1) of lane
        // s's run, of dCs for r < 2 and of dBs for r >= 2
        float h2[kCT];
#pragma unroll
        for (int m = 0; m < kCT; ++m) h2[m] = swap_add32(hg[m], qx[m]);
        {
          const int rw = ch & 3;
          float* wr = &wred[par][tid >> 6][rw >> 1][jp0 + (rw & 1)];
#pragma unroll
          for (int t = 0; t < kCT / 2; ++t) wr[2 * t] = swap_add16(h2[2 * t], h2[2 * t + 1]);
        }
        // The previous state's four wave sums (written before the last barrier) are
        // summed while this state's are being written; one barrier per state: the
        // next state writes the other buffer, and the one after it writes this one
        // only past the next barrier, which every thread reaches after reading it.
        if (n > 0) wave_sums(par ^ 1, n - 1, cb);
        __syncthreads();
        par ^= 1;
      }
      wave_sums(par ^ 1, N - 1, cb);
      if (cb + 1 == CPB && lo < L) {
        // the workgroup's partial, one row per state, written after the state loop
        // (no global store inside it, so its only memory wait is the prefetched state)
        float* dst = (which == 0 ? p.dCp : p.dBp) + ((int64_t)bk * ngrp + blk0 / CPB) * N * L + lo;
        for (int n = 0; n < N; ++n) dst[(int64_t)n * L] = acc[n][tid];
      }
      // ddt_bias sums the ddt products as rounded (no fused multiply-add), so that
      // both access paths add the same values
      if constexpr (VEC) {
#pragma unroll
        for (int g = 0; g < kCT / 4; ++g) {
          const int l = c * kChunk + j0 + 4 * g;
          if (cn.valid && l < L) {
#pragma clang fp contract(off)
            float dv[4], uv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int i = 4 * g + t;
              dv[t] = fmaf(uu[i], tq[i], sa[i]) * sig[i];
              rr.dbias += dv[t];
              rr.dD = fmaf(gg[i], uu[i], rr.dD);
            }
            if (p.pass == 0) {  // all states in one pass
#pragma unroll
              for (int t = 0; t < 4; ++t) uv[t] = fmaf(del[4 * g + t], tq[4 * g + t], cn.dsk * gg[4 * g + t]);
              Io<S>::st4(static_cast<S*>(p.ddt), cn.row + l, make_float4(dv[0], dv[1], dv[2], dv[3]));
            } else {
              // later state passes add their du and ddt terms to the earlier ones'
              const float4 du0 = p.pass >= 2 ? *reinterpret_cast<const float4*>(p.du + cn.row + l)
                                             : make_float4(0.f, 0.f, 0.f, 0.f);
              const float4 dt0 = p.pass >= 2 ? *reinterpret_cast<const float4*>(p.ddt_acc + cn.row + l)
                                             : make_float4(0.f, 0.f, 0.f, 0.f);
              const float du0v[4] = {du0.x, du0.y, du0.z, du0.w}, dt0v[4] = {dt0.x, dt0.y, dt0.z, dt0.w};
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const int i = 4 * g + t;
                uv[t] = p.pass >= 2 ? du0v[t] + del[i] * tq[i] : fmaf(del[i], tq[i], cn.dsk * gg[i]);
                if (p.pass >= 2) dv[t] = dt0v[t] + dv[t];
              }
              if (p.pass == 1 || p.pass == 2)
                *reinterpret_cast<float4*>(p.ddt_acc + cn.row + l) = make_float4(dv[0], dv[1], dv[2], dv[3]);
              else
                Io<S>::st4(static_cast<S*>(p.ddt), cn.row + l, make_float4(dv[0], dv[1], dv[2], dv[3]));
            }
            *reinterpret_cast<float4*>(p.du + cn.row + l) = make_float4(uv[0], uv[1], uv[2], uv[3]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kCT; ++i) {
          int li, xi;
          if (lane_step(cn, c, i, li, xi)) {
#pragma clang fp contract(off)
            const float ddt = fmaf(uu[i], tq[i], sa[i]) * sig[i];
            const float dsum = p.pass >= 2 ? p.ddt_acc[cn.row + li] + ddt : ddt;
            if (p.pass == 1 || p.pass == 2)
              p.ddt_acc[cn.row + li] = dsum;
            else
              Io<S>::st(static_cast<S*>(p.ddt), cn.row + li, dsum);
            p.du[cn.row + li] = p.pass >= 2 ? p.du[cn.row + li] + del[i] * tq[i] : fmaf(del[i], tq[i], cn.dsk * gg[i]);
            rr.dbias += ddt;
            rr.dD = fmaf(gg[i], uu[i], rr.dD);
          }
        }
      }
      next_block();
    }
  }
#pragma unroll 1
  for (int cb = 0; cb < CPB; ++cb) {
    const BwdChan<S> cn(p, bk, (blk0 + cb) * kBwdChans + ch);
    const float dbias = row_sum16(rr.dbias), dD = row_sum16(rr.dD);
    const int64_t pc = ((int64_t)b * p.nsp + sg) * p.K * D + cn.c_idx;  // this channel's per-(batch, segment) slot
    if (cn.valid && s < N) p.dAp[pc * p.Nt + p.n0 + s] = rr.dA;
    if (cn.valid && s == 0) {
      // ddt_bias adds every pass's ddt terms (in pass order); the g u sum of dDs
      // does not depend on the states and is written by the first pass
      p.dbp[pc] = p.pass >= 2 ? p.dbp[pc] + dbias : dbias;
      if (p.pass <= 1) p.dDp[pc] = dD;
    }
    next_block();
  }
}

// The segments of each (batch, direction, channel, state) chained in order:
// F becomes the state entering the segment, R the adjoint entering it from the right.
__global__ __launch_bounds__(256) void bwd_seg_carry(const float* __restrict__ segP, float* __restrict__ segF,
                                                    float* __restrict__ segR, int64_t cols, int64_t DN, int nsp) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (bk, d, n)
  if (e >= cols) return;
  const int64_t bk = e / DN;
  const int64_t base = bk * nsp * DN + (e - bk * DN);
  float h = 0.f;
  for (int sg = 0; sg < nsp; ++sg) {
    const int64_t i = base + sg * DN;
    const float f = segF[i];
    segF[i] = h;
    h = fmaf(segP[i], h, f);
  }
  float r = 0.f;
  for (int sg = nsp - 1; sg >= 0; --sg) {
    const int64_t i = base + sg * DN;
    const float q = segR[i];
    segR[i] = r;
    r = fmaf(segP[i], r, q);
  }
}

// dBs / dCs: the workgroups' partials (one per channel-block group) summed in order,
// into rows n0 .. n0 + N - 1 of each (batch, direction)'s Nt rows (orow = Nt L, o0 = n0 L).
template <typename S>
__global__ __launch_bounds__(256) void bwd_reduce_bc(const float* __restrict__ dBp, const float* __restrict__ dCp,
                                                    S* __restrict__ dBs, S* __restrict__ dCs, int64_t BK,
                                                    int nblk, int N, int L, int64_t orow, int64_t o0) {
  const int64_t total = BK * N * L;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t bk = e / ((int64_t)N * L), rest = e - bk * N * L;
    float sb = 0.f, sc = 0.f;
    for (int j = 0; j < nblk; ++j) {
      const int64_t src = (bk * nblk + j) * N * L + rest;
      sb += dBp[src];
      sc += dCp[src];
    }
    Io<S>::st(dBs, bk * orow + o0 + rest, sb);
    Io<S>::st(dCs, bk * orow + o0 + rest, sc);
  }
}

// The same sums, four consecutive (n, l) elements per thread with 16-byte loads and
// one store each (N * L a multiple of 4, aligned outputs).
template <typename S>
__global__ __launch_bounds__(256) void bwd_reduce_bc4(const float* __restrict__ dBp, const float* __restrict__ dCp,
                                                     S* __restrict__ dBs, S* __restrict__ dCs, int64_t BK,
                                                     int nblk, int64_t NL, int64_t orow, int64_t o0) {
  const int64_t total4 = BK * NL / 4;
  for (int64_t e4 = (int64_t)blockIdx.x * 256 + threadIdx.x; e4 < total4; e4 += (int64_t)gridDim.x * 256) {
    const int64_t e = 4 * e4;
    const int64_t bk = e / NL, rest = e - bk * NL;
    float4 sb = make_float4(0.f, 0.f, 0.f, 0.f), sc = sb;
    for (int j = 0; j < nblk; ++j) {
      const int64_t src = (bk * nblk + j) * NL + rest;
      const float4 vb = *reinterpret_cast<const float4*>(dBp + src);
      const float4 vc = *reinterpret_cast<const float4*>(dCp + src);
      sb = make_float4(sb.x + vb.x, sb.y + vb.y, sb.z + vb.z, sb.w + vb.w);
      sc = make_float4(sc.x + vc.x, sc.y + vc.y, sc.z + vc.z, sc.w + vc.w);
    }
    Io<S>::st4(dBs, bk * orow + o0 + rest, sb);
    Io<S>::st4(dCs, bk * orow + o0 + rest, sc);
  }
}

// dx[b, d, p] = du of directions 0, 1, 2, 3 at the steps that visit p, added in that
// order.  A workgroup takes a kMergeTile x kMergeTile pixel tile of one (b, d)
// plane: the column directions' values are read along their walk (down the tile's
// columns) into LDS and read back across its rows, so every global access is
// contiguous (rows of odd LDS length: both sides free of bank conflicts).
constexpr int kMergeTile = 32;

template <typename S>
__global__ __launch_bounds__(256) void bwd_merge(const float* __restrict__ du, S* __restrict__ dx, int D, int H,
                                                int W, int tiles_w, int tiles) {
  __shared__ float t1[kMergeTile][kMergeTile + 1], t3[kMergeTile][kMergeTile + 1];  // [w][h]
  const int64_t bd = blockIdx.x / tiles;
  const int t = (int)(blockIdx.x - bd * tiles);
  const int h0 = (t / tiles_w) * kMergeTile, w0 = (t % tiles_w) * kMergeTile;
  const int64_t b = bd / D, d = bd - b * D;
  const int L = H * W;
  const float* r0 = du + ((b * 4 + 0) * D + d) * L;
  const float* r1 = du + ((b * 4 + 1) * D + d) * L;
  const float* r2 = du + ((b * 4 + 2) * D + d) * L;
  const float* r3 = du + ((b * 4 + 3) * D + d) * L;
  const int a = threadIdx.x & 31, c = threadIdx.x >> 5;
#pragma unroll
  for (int m = 0; m < kMergeTile / 8; ++m) {  // pixel (h0 + a, w0 + ww) is step (w0 + ww) * H + h0 + a of the column walk
    const int ww = c + 8 * m;
    if (h0 + a < H && w0 + ww < W) {
      const int lc = (w0 + ww) * H + h0 + a;
      t1[ww][a] = r1[lc];
      t3[ww][a] = r3[L - 1 - lc];
    }
  }
  __syncthreads();
  S* out = dx + bd * L;
#pragma unroll
  for (int m = 0; m < kMergeTile / 8; ++m) {
    const int hh = c + 8 * m;
    if (h0 + hh < H && w0 + a < W) {
      const int px = (h0 + hh) * W + w0 + a;
      Io<S>::st(out, px, ((r0[px] + t1[a][hh]) + r2[L - 1 - px]) + t3[a][hh]);
    }
  }
}

// The same merge with whole (b, d) planes in LDS, for planes of L <= 4096 pixels
// with L a multiple of 4 and a 16-byte (fp32) or 8-byte (bf16) aligned dx.  TPP
// threads take one plane (a workgroup 256 / TPP planes): the column directions'
// values are read along their walk four steps at a time into row-major LDS copies,
// then each thread sums four consecutive pixels in the same order as above and
// writes them with one store.  Every global access is a 16-byte (8-byte) one.
constexpr int kMergePlaneMax = 4096;  // pixels: two fp32 planes of LDS (32 KB)

template <typename S>
__global__ __launch_bounds__(256) void bwd_merge_plane(const float* __restrict__ du, S* __restrict__ dx, int64_t BD,
                                                       int D, int H, int W, int TPP) {
  extern __shared__ __align__(16) float mtile[];  // per plane of the workgroup: t1[L], then t3[L]
  const int L = H * W, L4 = L >> 2;
  const int lt = threadIdx.x % TPP;
  const int64_t bd = (int64_t)blockIdx.x * (256 / TPP) + threadIdx.x / TPP;
  float* t1 = mtile + (threadIdx.x / TPP) * 2 * L;
  float* t3 = t1 + L;
  const bool live = bd < BD;  // the last workgroup's planes past the end only reach the barrier
  const int64_t bdc = live ? bd : BD - 1, b = bdc / D, d = bdc - b * D;
  const float* r0 = du + ((b * 4 + 0) * D + d) * L;
  const float* r1 = du + ((b * 4 + 1) * D + d) * L;
  const float* r2 = du + ((b * 4 + 2) * D + d) * L;
  const float* r3 = du + ((b * 4 + 3) * D + d) * L;
  if (live) {
    for (int q = lt; q < L4; q += TPP) {
      // column-walk steps 4q .. 4q+3: step l visits pixel (l mod H, l / H)
      int w = (4 * q) / H, h = 4 * q - w * H;
      const float4 a = *reinterpret_cast<const float4*>(r1 + 4 * q);
      const float4 c = *reinterpret_cast<const float4*>(r3 + (L - 4 - 4 * q));  // steps 4q+3 .. 4q, reversed
      const float av[4] = {a.x, a.y, a.z, a.w}, cv[4] = {c.w, c.z, c.y, c.x};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int p = h * W + w;
        t1[p] = av[k];
        t3[p] = cv[k];
        if (++h == H) {
          h = 0;
          ++w;
        }
      }
    }
  }
  __syncthreads();
  if (!live) return;
  S* out = dx + bd * L;
  for (int q = lt; q < L4; q += TPP) {
    const int p = 4 * q;  // pixels p .. p+3 in row-major order
    const float4 v0 = *reinterpret_cast<const float4*>(r0 + p);
    const float4 v2 = *reinterpret_cast<const float4*>(r2 + (L - 4 - p));  // pixels p+3 .. p, reversed
    const float4 v1 = *reinterpret_cast<const float4*>(t1 + p);
    const float4 v3 = *reinterpret_cast<const float4*>(t3 + p);
    Io<S>::st4(out, p, make_float4(((v0.x + v1.x) + v2.w) + v3.x, ((v0.y + v1.y) + v2.z) + v3.y,
                                   ((v0.z + v1.z) + v2.y) + v3.z, ((v0.w + v1.w) + v2.x) + v3.w));
  }
}

// dx of the two-path scan: dx[b, d, t] = du of path 0 at step t plus du of path 1
// at step L-1-t (du rows (b, 0, d) and (b, 1, d)), in that order.  V4: L a
// multiple of 4 and dx aligned, four tokens per thread with 16-byte accesses.
template <typename S>
__global__ __launch_bounds__(256) void bwd_merge_bidir(const float* __restrict__ du, S* __restrict__ dx, int64_t BD,
                                                      int D, int L, bool v4) {
  const int64_t total = v4 ? BD * L / 4 : BD * L;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t i = v4 ? 4 * e : e;
    const int64_t bd = i / L, t = i - bd * L, b = bd / D, d = bd - b * D;
    const float* r0 = du + ((b * 2 + 0) * D + d) * L;
    const float* r1 = du + ((b * 2 + 1) * D + d) * L;
    if (v4) {
      const float4 a = *reinterpret_cast<const float4*>(r0 + t);
      const float4 c = *reinterpret_cast<const float4*>(r1 + (L - 4 - t));  // steps L-1-t .. L-4-t, reversed
      Io<S>::st4(dx, i, make_float4(a.x + c.w, a.y + c.z, a.z + c.y, a.w + c.x));
    } else {
      Io<S>::st(dx, i, r0[t] + r1[L - 1 - t]);
    }
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
  // sums in batch order; unrolled so that eight loads are in flight at a time
  float s = 0.f;
#pragma unroll 8
  for (int b = 0; b < B; ++b) s += dAp[((int64_t)b * C4 + c) * N + n];
  dA_log[e] = -expf(A_log[e]) * s;
  if (n == 0) {
    float sb = 0.f, sd = 0.f;
#pragma unroll 8
    for (int b = 0; b < B; ++b) {
      sb += dbp[(int64_t)b * C4 + c];
      sd += dDp[(int64_t)b * C4 + c];
    }
    ddt_bias[c] = sb;
    dDs[c] = sd;
  }
}

// The chunked scan: one launch, or three for a segmented map.
template <typename S, bool VEC>
hipError_t launch_chunks(const BackwardArgs& a, const BwdParams& p, int cpb, unsigned blocks) {
  hipError_t e = hipSuccess;
  if (p.nsp == 1) {
    if (cpb == 2)
      hipLaunchKernelGGL((bwd_chunk_kernel<S, kWhole, 2, VEC>), dim3(blocks), dim3(256), 0, a.stream, p);
    else
      hipLaunchKernelGGL((bwd_chunk_kernel<S, kWhole, 1, VEC>), dim3(blocks), dim3(256), 0, a.stream, p);
  } else {
    hipLaunchKernelGGL((bwd_chunk_kernel<S, kSegMaps, 1, VEC>), dim3(blocks), dim3(256), 0, a.stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t cols = a.B * a.K * a.D * p.N;
    hipLaunchKernelGGL(bwd_seg_carry, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, a.stream, p.segP, p.segF,
                       p.segR, cols, a.D * p.N, p.nsp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_chunk_kernel<S, kSegGrads, 1, VEC>), dim3(blocks), dim3(256), 0, a.stream, p);
  }
  return hipGetLastError();
}

// The kernels that read or write the storage type: transposes of x and dy, then
// per block of up to 16 states the chunked scan (one launch, or three for a
// segmented map) and the dBs/dCs sums, then the dx merge.
template <typename S>
hipError_t launch_io(const BackwardArgs& a, BwdParams p, int64_t L, int cpb) {
  hipError_t e = hipSuccess;
  if (a.K == 4) {  // the column walks read transposed copies
    e = launch_transpose<S>(static_cast<const S*>(a.x), static_cast<S*>(const_cast<void*>(p.xT)), (int)(a.B * a.D),
                            (int)a.H, (int)a.W, a.stream);
    if (e != hipSuccess) return e;
    e = launch_transpose<S>(static_cast<const S*>(a.dy), static_cast<S*>(const_cast<void*>(p.dyT)), (int)(a.B * a.D),
                            (int)a.H, (int)a.W, a.stream);
    if (e != hipSuccess) return e;
  }
  const int ngrp = (p.nblk + cpb - 1) / cpb;
  const unsigned blocks = (unsigned)(a.B * a.K * ngrp * p.nsp);
  // 16-byte (fp32) or 8-byte (bf16) accesses when every row the chunks read or
  // write starts aligned: L a multiple of 4 and aligned bases
  const uintptr_t vm = sizeof(S) == 4 ? 15 : 7;
  const bool vec = L % 4 == 0 && !(((uintptr_t)a.x | (uintptr_t)a.dt | (uintptr_t)a.Bs | (uintptr_t)a.Cs |
                                    (uintptr_t)a.dy | (uintptr_t)a.ddt | (uintptr_t)p.xT | (uintptr_t)p.dyT) & vm);
  const int Nt = (int)a.N, passes = (Nt + kBwdStates - 1) / kBwdStates;
  const uintptr_t om = sizeof(S) == 4 ? 15 : 7;
  for (int ps = 0; ps < passes; ++ps) {
    // passes in state order: du, ddt and ddt_bias add up over them in that order
    p.n0 = ps * kBwdStates;
    p.N = Nt - p.n0 < kBwdStates ? Nt - p.n0 : kBwdStates;
    p.pass = passes == 1 ? 0 : ps == 0 ? 1 : ps + 1 < passes ? 2 : 3;
    e = vec ? launch_chunks<S, true>(a, p, cpb, blocks) : launch_chunks<S, false>(a, p, cpb, blocks);
    if (e != hipSuccess) return e;
    const int64_t orow = (int64_t)Nt * L, o0 = (int64_t)p.n0 * L;
    if (((int64_t)p.N * L) % 4 == 0 && orow % 4 == 0 && o0 % 4 == 0 && !((uintptr_t)a.dBs & om) &&
        !((uintptr_t)a.dCs & om))
      hipLaunchKernelGGL((bwd_reduce_bc4<S>), dim3(4096), dim3(256), 0, a.stream, p.dBp, p.dCp,
                         static_cast<S*>(a.dBs), static_cast<S*>(a.dCs), a.B * a.K, ngrp, (int64_t)p.N * L, orow,
                         o0);
    else
      hipLaunchKernelGGL((bwd_reduce_bc<S>), dim3(4096), dim3(256), 0, a.stream, p.dBp, p.dCp,
                         static_cast<S*>(a.dBs), static_cast<S*>(a.dCs), a.B * a.K, ngrp, p.N, (int)L, orow, o0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const uintptr_t am = sizeof(S) == 4 ? 15 : 7;
  if (a.K == 2) {  // dx of the two-path scan: the forward path's du plus the reversed path's, token by token
    const bool v4 = L % 4 == 0 && !((uintptr_t)a.dx & am);
    hipLaunchKernelGGL((bwd_merge_bidir<S>), dim3(4096), dim3(256), 0, a.stream, p.du, static_cast<S*>(a.dx),
                       a.B * a.D, (int)a.D, (int)L, v4);
    return hipGetLastError();
  }
  if (L <= kMergePlaneMax && L % 4 == 0 && !((uintptr_t)a.dx & am)) {
    // threads per plane: the fewest of 64, 128, 256 that give each a group of four pixels
    const int TPP = L / 4 <= 64 ? 64 : (L / 4 <= 128 ? 128 : 256), ppw = 256 / TPP;
    const int64_t BD = a.B * a.D;
    const size_t lds = (size_t)ppw * 2 * L * sizeof(float);
    hipLaunchKernelGGL((bwd_merge_plane<S>), dim3((unsigned)((BD + ppw - 1) / ppw)), dim3(256), lds, a.stream, p.du,
                       static_cast<S*>(a.dx), BD, (int)a.D, (int)a.H, (int)a.W, TPP);
    return hipGetLastError();
  }
  const int tiles_w = (int)((a.W + kMergeTile - 1) / kMergeTile);
  const int tiles = (int)((a.H + kMergeTile - 1) / kMergeTile) * tiles_w;
  hipLaunchKernelGGL((bwd_merge<S>), dim3((unsigned)(a.B * a.D * tiles)), dim3(256), 0, a.stream, p.du,
                     static_cast<S*>(a.dx), (int)a.D, (int)a.H, (int)a.W, tiles_w, tiles);
  return hipGetLastError();
}

// Workgroups that fill the chip once at three per compute unit.
constexpr int64_t kBwdPairBlocks = 768;
// Segments: a map whose channel blocks alone give fewer workgroups than fill the
// chip once is cut into segments of at least kMinSegChunks chunks, toward about
// six workgroups per compute unit.  From one full round up, whole sequences are
// faster than segments (their map and carry passes cost more than a second round
// of workgroups saves).
constexpr int64_t kBwdTargetBlocks = 1536;
constexpr int64_t kMinSegChunks = 4;

struct BwdLayout {
  int64_t L, nch, nblk, nsp, cps, cpb;
  size_t du, hck, dBp, dCp, dAp, dbp, dDp, cdl, segP, segF, segR, ddt_acc, xT, dyT, total;  // byte offsets
};

BwdLayout bwd_layout(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int K) {
  BwdLayout o;
  o.L = H * W;
  o.nch = (o.L + kChunk - 1) / kChunk;
  o.nblk = (D + kBwdChans - 1) / kBwdChans;
  const int64_t base = B * K * o.nblk;
  int64_t nsp = 1;
  if (base < kBwdPairBlocks) nsp = std::min((kBwdTargetBlocks + base - 1) / base, o.nch / kMinSegChunks);
  if (nsp < 2) nsp = 1;
  o.cps = (o.nch + nsp - 1) / nsp;
  o.nsp = (o.nch + o.cps - 1) / o.cps;  // no empty segment
  // two channel blocks per workgroup (sharing Bs/Cs staging and the dBs/dCs
  // partial) where that still leaves a full round of workgroups
  o.cpb = o.nsp == 1 && B * K * ((o.nblk + 1) / 2) >= kBwdPairBlocks ? 2 : 1;
  const int64_t ngrp = (o.nblk + o.cpb - 1) / o.cpb;
  auto up = [](int64_t v) { return (size_t)((v * 4 + 255) & ~(int64_t)255); };
  size_t off = 0;
  auto take = [&](size_t& at, int64_t floats) {
    at = off;
    off += up(floats);
  };
  const int64_t Nb = N < kBwdStates ? N : kBwdStates;  // states of one pass
  take(o.du, B * K * D * o.L);
  take(o.hck, B * K * o.nch * D * Nb * 16);
  take(o.dBp, B * K * ngrp * Nb * o.L);
  take(o.dCp, B * K * ngrp * Nb * o.L);
  take(o.dAp, B * o.nsp * K * D * N);
  take(o.dbp, B * o.nsp * K * D);
  take(o.dDp, B * o.nsp * K * D);
  const bool seg = o.nsp > 1;
  take(o.cdl, seg ? B * K * o.nch * D * 16 : 0);
  take(o.segP, seg ? B * K * o.nsp * D * Nb : 0);
  take(o.segF, seg ? B * K * o.nsp * D * Nb : 0);
  take(o.segR, seg ? B * K * o.nsp * D * Nb : 0);
  take(o.ddt_acc, N > kBwdStates ? B * K * D * o.L : 0);  // ddt summed over the passes
  // the transposed copies (the cross scan's column walks), sized for fp32 (bf16 uses half)
  take(o.xT, K == 4 ? B * D * o.L : 0);
  take(o.dyT, K == 4 ? B * D * o.L : 0);
  o.total = off;
  return o;
}

}  // namespace

size_t backward_scratch_bytes(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int K) {
  return bwd_layout(B, D, H, W, N, dtype, K).total;
}

int64_t backward_segments(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int K) {
  return bwd_layout(B, D, H, W, N, dtype, K).nsp;
}

int64_t backward_blocks_per_workgroup(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int K) {
  return bwd_layout(B, D, H, W, N, dtype, K).cpb;
}

hipError_t launch_backward(const BackwardArgs& a, void* scratch) {
  if (a.K != 4 && a.K != 2) return hipErrorInvalidValue;
  const BwdLayout o = bwd_layout(a.B, a.D, a.H, a.W, a.N, a.dtype, a.K);
  char* base = static_cast<char*>(scratch);
  auto f = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
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
  p.du = f(o.du);
  p.hck = f(o.hck);
  p.dBp = f(o.dBp);
  p.dCp = f(o.dCp);
  p.dAp = f(o.dAp);
  p.dbp = f(o.dbp);
  p.dDp = f(o.dDp);
  p.cdl = f(o.cdl);
  p.segP = f(o.segP);
  p.segF = f(o.segF);
  p.segR = f(o.segR);
  p.xT = a.K == 4 ? base + o.xT : nullptr;  // the two-path scan has no column walks
  p.dyT = a.K == 4 ? base + o.dyT : nullptr;
  p.D = (int)a.D;
  p.H = (int)a.H;
  p.W = (int)a.W;
  p.L = (int)o.L;
  p.N = (int)a.N;
  p.K = a.K;
  p.Nt = (int)a.N;
  p.n0 = 0;
  p.pass = 0;
  p.ddt_acc = a.N > kBwdStates ? f(o.ddt_acc) : nullptr;
  p.nseg = (int)o.nch;
  p.nblk = (int)o.nblk;
  p.nsp = (int)o.nsp;
  p.cps = (int)o.cps;
  const int64_t merge_tiles = ((a.H + kMergeTile - 1) / kMergeTile) * ((a.W + kMergeTile - 1) / kMergeTile);
  if (a.B * a.K * o.nblk * o.nsp > INT32_MAX || a.B * a.D * merge_tiles > INT32_MAX) return hipErrorInvalidValue;
  hipError_t e = a.dtype == 0 ? launch_io<float>(a, p, o.L, (int)o.cpb) : launch_io<uint16_t>(a, p, o.L, (int)o.cpb);
  if (e != hipSuccess) return e;
  const int C4 = (int)(a.K * a.D);
  hipLaunchKernelGGL(bwd_params, dim3((unsigned)((C4 * a.N + 255) / 256)), dim3(256), 0, a.stream, a.A_log, p.dAp,
                     p.dbp, p.dDp, a.dA_log, a.ddt_bias, a.dDs, (int)(a.B * o.nsp), C4, (int)a.N);
  return hipGetLastError();
}

}  // namespace ss2d
