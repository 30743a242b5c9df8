// Internal interface between the C ABI layer (ss2d_api.hip) and the kernels
// (ss2d_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss2d {

// Everything a forward launch needs, already validated by the ABI layer.
struct LaunchArgs {
  const void* x;
  const void* dt;
  const float* A_log;
  const float* dt_bias;
  const void* Bs;
  const void* Cs;
  const float* Ds;
  void* y;
  int64_t B, D, H, W, N;
  int dtype;  // 0 = fp32, 1 = bf16
  hipStream_t stream;
  int device;  // current device of the calling thread
  // Directions: 4 (the cross scan) or 2 (the row walk and its reverse; the
  // per-direction tensors then hold two slots).
  int K = 4;
  // State block of one launch: N states from n0 of Nt (A_log rows and the Bs/Cs
  // (batch, direction) slices have Nt states).  launch_forward sets these.
  int64_t Nt = 0, n0 = 0;
  bool skip = true, acc = false, final_out = true;
  // Low-rank step input: R > 0 means dt holds the R rows dts (B, K, R, L) and the
  // scan forms dt = wdt (K, D, R) times them itself (R <= kMaxLowRankInput and at
  // most the plan's channels per workgroup).
  int R = 0;
  const float* wdt = nullptr;
};

// Largest rank of the low-rank step input the scan expands itself.
constexpr int kMaxLowRankInput = 8;

// How a shape is mapped onto the machine.
struct Plan {
  int lanes_per_seq;     // G: lanes that share one (b, k, d) sequence per chunk
  int steps_per_lane;    // T: consecutive steps of one lane in a full chunk (16 or 8)
  int waves;             // waves per workgroup
  int chans_per_block;   // D channels one workgroup owns
  int nseg;              // segments per sequence (1: whole sequences in one launch)
  int seg_chunks;        // full chunks per segment
  int64_t blocks;        // workgroups of one output launch
  size_t lds_bytes;      // LDS per workgroup
  size_t scratch_bytes;  // device temporary: fp32 merge planes, segment maps, transposed copies
  size_t carry_offset;   // byte offset of the segment maps in the temporary
  bool xtrans;           // x is transposed first; column walks read the copy
  bool transpose;        // the column merge plane is transposed before the last direction (segmented plans)
  size_t xt_offset;      // byte offsets of those copies in the temporary
  size_t pct_offset;
  bool vec;              // rows and bases aligned for 16-byte (fp32) / 8-byte (bf16) access: the DMA path
  int state_blocks;      // launches over blocks of at most 16 states (N > 16)
};

// Largest N one kernel launch takes; larger N runs in blocks of this many states.
constexpr int kStatesPerLaunch = 16;
// Largest N the forward accepts.
constexpr int kMaxStates = 256;

// Device buffers of one forward, carved from the temporary.
struct Scratch {
  float* prow;     // row-major merge plane (directions 0, 2): y itself for fp32 output
  float* pcol;     // column-major merge plane (directions 1, 3)
  float* carries;  // segment maps
  void* xT;        // x with H and W swapped, or null
  float* pcolT;    // the column plane in row-major order, or null
  bool xT_given;   // xT already holds the transpose (made by the caller)
};

// Rates measured on the device (see ss2d_measure_peaks in ss2d.h).
struct PeakRates {
  double exp_per_s, fma_per_s, update_mix_per_s, hbm_read_Bps, hbm_copy_Bps, lds_read_Bps;
  int compute_units;
  double state_loop_per_s;
};

// Runs the roofline probes on the current device, on `stream` (synchronises it).
hipError_t measure_peaks(PeakRates* out, int64_t hbm_bytes, hipStream_t stream);

// lanes_override: 0 = automatic, else 16, 32 or 64 lanes per sequence.
// K: directions (4 or 2).  aligned: the caller's bases allow the vector paths
// (with L % 4 == 0 they then take the DMA path).  no_copies: no transposed
// copies in the temporary (the column walks and the final merge gather instead).
Plan make_plan(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int lanes_override, int K = 4,
               bool aligned = true, bool no_copies = false);

// Enqueue the forward.  `scratch` holds plan.scratch_bytes.  `xT`, when not null,
// already holds x with H and W swapped (B*D planes of W x H): column walks then
// read it instead of gathering.  Returns hipSuccess or the first HIP error.
hipError_t launch_forward(const LaunchArgs& a, const Plan& plan, float* scratch, const void* xT = nullptr);

// The per-direction input projections (x_proj, split, rank-R dt map), written in
// scan order.  xT must already hold x with H and W swapped.
struct ProjectArgs {
  const void* x;
  const void* xT;
  const float* wx;   // (4, R + 2N, D)
  const float* wdt;  // (4, D, R)
  void* dt;          // (B, 4, D, L), or null when dts is given
  void* Bs;          // (B, 4, N, L)
  void* Cs;          // (B, 4, N, L)
  int64_t B, D, H, W, N, R;
  int dtype;
  hipStream_t stream;
  void* dts = nullptr;  // (B, 4, R, L): the low-rank rows instead of the dt map
};
hipError_t launch_project(const ProjectArgs& a);
// Largest 2 * (R + 2N) the projection kernel takes.
int project_max_rows();
// y (B, D, H, W) -> out (B, H, W, D), optionally normalised over D per pixel.
struct EpilogueArgs {
  const void* y;
  const float* gamma;  // (D) or null (scale 1)
  const float* beta;   // (D) or null (shift 0)
  void* out;
  float eps;
  bool normalize;
  int64_t B, D, H, W;
  int dtype;
  hipStream_t stream;
};
hipError_t launch_channel_last(const EpilogueArgs& a);
// Largest D the epilogue takes.
int epilogue_max_channels();

// Gradients of the forward: every output fully written.  x, dt, Bs, Cs, dy, dx,
// ddt, dBs, dCs in the storage type; the per-channel tensors fp32.
struct BackwardArgs {
  const void* x;
  const void* dt;
  const float* A_log;
  const float* dt_bias;
  const void* Bs;
  const void* Cs;
  const float* Ds;
  const void* dy;
  void* dx;
  void* ddt;
  float* dA_log;
  float* ddt_bias;
  void* dBs;
  void* dCs;
  float* dDs;
  int64_t B, D, H, W, N;
  int dtype;
  hipStream_t stream;
  int K = 4;  // 4: the cross scan of an H x W map; 2: the two-path scan of a 1 x L sequence
};
size_t backward_scratch_bytes(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int K = 4);
// Segments each backward sequence is cut into (1: one workgroup walks the whole map).
int64_t backward_segments(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int K = 4);
// Channel blocks of 16 channels each backward workgroup takes (1 or 2).
int64_t backward_blocks_per_workgroup(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int K = 4);
hipError_t launch_backward(const BackwardArgs& a, void* scratch);

// x (B*D planes of H x W) -> xT (planes of W x H).
hipError_t launch_transpose_x(const void* x, void* xT, int64_t planes, int64_t H, int64_t W, int dtype,
                              hipStream_t stream);

}  // namespace ss2d
