// Launch planning and dispatch of the SS2D forward (the kernels are compiled in
// the ss2d_{f32,bf16}_t{16,8}.hip units).
#include "ss2d_kernels.h"

namespace ss2d {

// Maps from this many pixels on transpose x first (below it the transpose costs
// more than the gathers it saves: measured on 14x14 and 28x28 maps).
constexpr int64_t kTransposeXFrom = 2048;

Plan make_plan(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int lanes_override, int K,
               bool aligned, bool no_copies) {
  Plan pl;
  const int64_t L = H * W;
  // 16 lanes per sequence: short sequences, or longer ones when little is left
  // after whole 256-step chunks (the 16-lane remainder is not prefetched) and
  // either the 16-channel blocks still give at least three workgroups per CU or a
  // 32-lane plan would be cut into segments anyway.  Each workgroup then shares
  // its Bs/Cs staging among twice the channels, the scan across lanes is one
  // level shorter, and segmented maps can take twice the segments.  Measured
  // 2-15% faster on 24x24 to 48x48 maps and up to 16% on segmented ones (never
  // more than 0.3% slower there); slower on unsegmented maps with fewer blocks or
  // longer remainders.
  const int64_t units16 = B * ((D + kWaves * 4 - 1) / (kWaves * 4));
  const int64_t units32 = B * ((D + kWaves * 2 - 1) / (kWaves * 2));
  const bool seg32 = L % 4 == 0 && units32 < 512 && L / 512 >= 8;  // a 32-lane plan would be segmented
  int G = (L < 512 || ((units16 >= 768 || seg32) && L % 256 <= 64)) ? 16 : 32;
  if (lanes_override == 16 || lanes_override == 32 || lanes_override == 64) G = lanes_override;
  // Steps per lane: 16, unless the remainder after whole 16-step chunks would fill
  // at least one 8-step chunk, which then runs at full speed instead of in the
  // remainder path (8-step chunks exist for 32 and 64 lanes).
  int T = 16;
  if (G != 16 && L % (16 * G) >= 8 * G) T = 8;
  pl.lanes_per_seq = G;
  pl.steps_per_lane = T;
  pl.waves = kWaves;
  pl.chans_per_block = kWaves * (64 / G);
  const bool vec = L % 4 == 0 && aligned;
  pl.vec = vec;
  pl.state_blocks = (int)((N + kStatesPerLaunch - 1) / kStatesPerLaunch);
  // Too few (batch, channel block) pairs to fill the machine and long sequences:
  // cut each sequence into segments of at least four full chunks, aiming at about
  // three workgroups per CU; a carry pass then supplies each segment's entering
  // state.
  const int64_t units = B * ((D + pl.chans_per_block - 1) / pl.chans_per_block);
  const int64_t nmain = L / (G * T);
  pl.nseg = 1;
  pl.seg_chunks = (int)(nmain > 0 ? nmain : 1);
  if (vec && units < 512 && nmain >= 8) {
    int64_t nseg = (768 + units - 1) / units;
    if (nseg > nmain / 4) nseg = nmain / 4;
    if (nseg > 1) {
      const int64_t per = (nmain + nseg - 1) / nseg;
      pl.seg_chunks = (int)per;
      pl.nseg = (int)((nmain + per - 1) / per);
    }
  }
  pl.blocks = units * pl.nseg;
  pl.lds_bytes = dtype == 0 ? lds_bytes_s<float>(G, T, vec) : lds_bytes_s<uint16_t>(G, T, vec);
  // fp32 planes: the column plane (K = 4), and for bf16 output the row plane
  const size_t nplanes = (size_t)(K == 4 ? 1 : 0) + (size_t)(dtype == 0 ? 0 : 1);
  const size_t planes = nplanes * (size_t)(B * D * L) * sizeof(float);
  pl.carry_offset = planes;
  pl.scratch_bytes = planes + (pl.nseg > 1 ? (size_t)(B * K * D) * pl.nseg * 2 * kMaxN * sizeof(float) : 0);
  // A column walk reading x in place touches one cache line per step and lane;
  // those gathers load the same L1 path the Bs/Cs copies use.  So on large maps
  // x is transposed once first and the column walks read the copy.  Segmented
  // plans (large maps, whose working set outgrows L2) also transpose the column
  // merge plane before direction 2.
  pl.xtrans = K == 4 && !no_copies && vec && (pl.nseg > 1 || L >= kTransposeXFrom);
  pl.transpose = K == 4 && !no_copies && pl.nseg > 1;
  pl.xt_offset = pl.pct_offset = 0;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  if (pl.xtrans) {
    pl.xt_offset = up(pl.scratch_bytes);
    pl.scratch_bytes = pl.xt_offset + (size_t)(B * D * L) * (dtype == 0 ? 4 : 2);
  }
  if (pl.transpose) {
    pl.pct_offset = up(pl.scratch_bytes);
    pl.scratch_bytes = pl.pct_offset + (size_t)(B * D * L) * sizeof(float);
  }
  return pl;
}

hipError_t launch_forward(const LaunchArgs& a, const Plan& plan, float* scratch, const void* xT) {
  const int64_t plane = a.B * a.D * a.H * a.W;
  char* base = reinterpret_cast<char*>(scratch);
  Scratch s;
  // planes: column-major (directions 1, 3; K = 4 only), then row-major
  // (directions 0, 2): y itself for fp32 output
  const int64_t ncol = a.K == 4 ? 1 : 0;
  s.pcol = a.K == 4 ? scratch : nullptr;
  s.prow = a.dtype == 0 ? static_cast<float*>(a.y) : scratch + ncol * plane;
  s.carries = reinterpret_cast<float*>(base + plan.carry_offset);
  s.xT = xT ? const_cast<void*>(xT) : plan.xtrans ? static_cast<void*>(base + plan.xt_offset) : nullptr;
  s.xT_given = xT != nullptr;
  s.pcolT = plan.transpose ? reinterpret_cast<float*>(base + plan.pct_offset) : nullptr;
  const bool t8 = plan.steps_per_lane == 8;
  // N > 16: one launch sequence per block of at most 16 states.  y is linear in
  // each state's contribution, so the blocks' outputs add up: the first block
  // adds the skip term Ds*u, later blocks add onto the row plane, and only the
  // last rounds to the storage type.
  for (int blk = 0; blk < plan.state_blocks; ++blk) {
    LaunchArgs b = a;
    b.Nt = a.N;
    b.n0 = (int64_t)blk * kStatesPerLaunch;
    b.N = a.N - b.n0 < kStatesPerLaunch ? a.N - b.n0 : kStatesPerLaunch;
    b.skip = blk == 0;
    b.acc = blk > 0;
    b.final_out = blk + 1 == plan.state_blocks;
    hipError_t e;
    if (a.dtype == 0)
      e = t8 ? launch_f32_t8(b, plan, s) : launch_f32_t16(b, plan, s);
    else
      e = t8 ? launch_bf16_t8(b, plan, s) : launch_bf16_t16(b, plan, s);
    if (e != hipSuccess) return e;
    s.xT_given = s.xT != nullptr;  // transposed once, by the first block's launches
  }
  return hipSuccess;
}

}  // namespace ss2d
