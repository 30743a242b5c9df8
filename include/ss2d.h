/*
 * ss2d.h -- C ABI of the MI355X (gfx950) SS2D forward library, libss2d.so.
 *
 * One call computes the whole SS2D forward hot path of a VMamba block:
 *   CrossScan  -- the H x W map is read as four sequences of length L = H*W:
 *                 row by row (direction 0), column by column (direction 1),
 *                 and both of those reversed (directions 2 and 3);
 *   selective scan over each sequence, per channel c = k*D + d and state n:
 *                 delta = softplus(dt + dt_bias[c]), A = -exp(A_log[c, n]),
 *                 h = exp(delta*A) * h + delta * Bs[n] * u  (h starts at 0),
 *                 out = sum_n Cs[n] * h + Ds[c] * u;
 *   CrossMerge -- the four directional outputs are mapped back to the map and
 *                 summed (accumulated in fp32, rounded once to `dtype`).
 * Passages that define it, on the page [SS2D] "深入解析VMamba中的SS2D模块从理论到
 * 代码实现": §3.1 (the four sequences), §3.2 (the selective_scan call: -exp of
 * A_logs, delta_bias, delta_softplus, shared per-direction B/C), §3.3 (the
 * merge), §4 (direction table).  Zero initial state: [DAMamba] page §3.1.
 *
 * All functions are plain C; no HIP or torch types appear in the signatures.
 */
#ifndef SS2D_H_
#define SS2D_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of x, dt, Bs, Cs and y.  A_log, dt_bias and Ds are always fp32,
 * and the scan state and every accumulation are fp32 for both types. */
typedef enum { SS2D_F32 = 0, SS2D_BF16 = 1 } ss2d_dtype;

typedef enum {
  SS2D_OK = 0,
  SS2D_ERR_NULL = -1,           /* a required pointer is NULL                     */
  SS2D_ERR_SHAPE = -2,          /* B, D, H or W < 1, H*W > 2^25 - 1, or a size    */
                                /* overflows int64                                */
  SS2D_ERR_UNSUPPORTED_N = -3,  /* N outside 1..256 (1..16 for the projections)   */
  SS2D_ERR_DTYPE = -4,          /* dtype is not an ss2d_dtype value               */
  SS2D_ERR_ALIAS = -5,          /* y overlaps one of the inputs                   */
  SS2D_ERR_ALIGN = -6,          /* a pointer is not aligned to its element size   */
  SS2D_ERR_NO_DEVICE = -7,      /* no HIP device, or the device query failed      */
  SS2D_ERR_HIP = -8,            /* a HIP call or kernel launch failed             */
  SS2D_ERR_NOALLOC_LIMIT = -9   /* ss2d_forward_noalloc: the shape's temporary    */
                                /* exceeds the library's static array (128 MiB)   */
} ss2d_status;

/*
 * ss2d_forward -- enqueue one SS2D forward on `stream`.
 *
 * Every pointer is DEVICE memory owned by the caller; all tensors are dense and
 * row-major (C order).  L = H*W.  "dtype" below means the storage type chosen by
 * `dtype` (fp32 or bf16).
 *   x       [B, D, H, W]   dtype  channel-first feature map.
 *   dt      [B, 4, D, L]   dtype  step input of direction k, channel d, in the
 *                                 order direction k visits the map (its scan order).
 *   A_log   [4*D, N]       fp32   row c = k*D + d.
 *   dt_bias [4*D]          fp32
 *   Bs, Cs  [B, 4, N, L]   dtype  per-direction projections in scan order, shared
 *                                 by all D channels of that direction.
 *   Ds      [4*D]          fp32
 *   y       [B, D, H, W]   dtype  output; fully overwritten, never read.  Must not
 *                                 overlap any input.
 *   N       number of states, 1..256.  Up to 16 states run in one pass; larger N
 *           runs in passes over blocks of 16 states whose outputs are summed in
 *           fp32 in a fixed order (y is linear in each state's contribution).
 *           d_state = 256 is the large-state setting of the [VSSD] page
 *           ("项目概述：当视觉Transformer遇到状态空间模型", §4.1).
 *   stream  a hipStream_t (NULL = the default stream).
 *
 * Alignment: every pointer must be aligned to its element size (SS2D_ERR_ALIGN
 * otherwise).  Bases aligned to 16 bytes (fp32) or 8 bytes (bf16) -- as torch
 * allocations are -- with L % 4 == 0 take the vector/DMA path; other
 * element-aligned bases take a slower scalar path with the same results.
 *
 * Behaviour: arguments are validated before any device work (codes above).  On
 * SS2D_OK the work has been enqueued asynchronously; execution faults surface at
 * the caller's next synchronisation.  Nothing is printed, thrown or aborted.
 * Each call takes a stream-ordered temporary of B*D*H*W fp32 values (2*B*D*H*W
 * for bf16) for the merge.  Maps of 2048 pixels or more add a copy of x with H
 * and W swapped; when a long map is cut into segments it also holds 32 fp32
 * values per (batch, direction, channel, segment) and an fp32 B*D*H*W
 * transposed merge plane (ss2d_describe shows the plan and the exact size).
 * The temporary is allocated and freed on `stream` from a memory pool the
 * library creates per device (freed blocks stay reserved there for the next
 * call until ss2d_trim_memory; the device's default pool is left untouched).
 * A call then runs one kernel (two with the transpose of x), or seven for
 * segmented maps (a transpose of x, a carry pass, one launch per direction and
 * a transpose of the merge plane before the last), per block of 16 states, all
 * on `stream`.  NaN and Inf propagate.  Thread-safe.
 */
int ss2d_forward(const void* x, const void* dt, const float* A_log, const float* dt_bias,
                 const void* Bs, const void* Cs, const float* Ds, void* y,
                 int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                 int dtype, void* stream);

/*
 * ss2d_forward_lanes -- ss2d_forward with the number of lanes that share one
 * sequence chunk chosen by the caller: 16, 32 or 64 (0 = the automatic choice
 * ss2d_forward makes).  The result is the same function up to rounding order;
 * for tests and tuning.  Any other value is SS2D_ERR_SHAPE.  No state is kept
 * between calls.
 */
int ss2d_forward_lanes(const void* x, const void* dt, const float* A_log, const float* dt_bias,
                       const void* Bs, const void* Cs, const float* Ds, void* y,
                       int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                       int dtype, int lanes_per_seq, void* stream);

/*
 * ss2d_forward_noalloc -- ss2d_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): it calls no hipMalloc, hipFree or allocating library
 * routine.  Its temporary is a static device array of 128 MiB that the library
 * holds on every device it runs on until the process ends, so only shapes whose
 * temporary fits run: it holds the fp32 merge plane(s) (B*D*H*W fp32 values, twice
 * that for bf16 output) and, for long maps cut into segments, 32 fp32 values per
 * (batch, direction, channel, segment).  Larger shapes return
 * SS2D_ERR_NOALLOC_LIMIT before any device work (VMamba-T stage-1 fp32, 77 MB,
 * and 2 x 192 x 256 x 256 fp32, 107 MB, fit; bf16 B=64, D=384, 28 x 28 does not).
 * Unlike ss2d_forward it makes no transposed copies: column walks and the final
 * merge gather from x and the column plane in place.  Same arguments, results
 * (the same function up to rounding order), validation and error codes as
 * ss2d_forward.  Every call on a device uses that device's one array, and nothing
 * in it needs to start at any value; calls whose work overlaps on one device
 * (other streams, other threads) race on it and must be serialised by the
 * caller.
 */
int ss2d_forward_noalloc(const void* x, const void* dt, const float* A_log, const float* dt_bias,
                         const void* Bs, const void* Cs, const float* Ds, void* y,
                         int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                         int dtype, void* stream);

/*
 * ss2d_bidir_forward -- enqueue the two-direction (bidirectional) selective scan
 * of a sequence of L tokens on `stream`: a forward path that visits the tokens
 * t = 0 .. L-1 and a backward path that visits t = L-1 .. 0, each with its own
 * parameters, and their outputs summed per token.  [VSSD] page "项目概述：当视觉
 * Transformer遇到状态空间模型", §2.2 (non-causal dual paths; the backward path
 * changes the recursion direction instead of reversing the input: x is read
 * backwards in place, never flipped).  The page fuses the two paths with a
 * learned gate; that gate belongs to the model around this path, and here the
 * paths are summed as the cross merge sums directions.
 *   Path j = 0 (forward) or 1 (backward), channel c = j*D + d, step l of path j
 *   visits token t_j(l) = l (j = 0) or L-1-l (j = 1):
 *     delta_l = softplus(dt[b,j,d,l] + dt_bias[c]),  A = -exp(A_log[c, n]),
 *     h_l = exp(delta_l*A) * h_{l-1} + delta_l * Bs[b,j,n,l] * x[b,d,t_j(l)],  h_{-1} = 0,
 *     out_j[l] = sum_n Cs[b,j,n,l] * h_l + Ds[c] * x[b,d,t_j(l)];
 *   y[b,d,t] = out_0[t] + out_1[L-1-t]  (fp32, rounded once to `dtype`).
 * As for ss2d_forward, each path's dt, Bs and Cs are in the order that path
 * visits the tokens (its scan order).  This is ss2d_forward restricted to its
 * directions 0 and 2 on a 1 x L map.
 *   x       [B, D, L]      dtype    (for instance a feature map flattened row by row)
 *   dt      [B, 2, D, L]   dtype
 *   A_log   [2*D, N]       fp32
 *   dt_bias [2*D]          fp32
 *   Bs, Cs  [B, 2, N, L]   dtype
 *   Ds      [2*D]          fp32
 *   y       [B, D, L]      dtype    fully overwritten; must not overlap an input
 *   N       1..256
 * Temporaries (none for fp32 output unless L is long enough to be cut into
 * segments; one fp32 B*D*L plane for bf16), validation, alignment, error
 * reporting and thread safety as for ss2d_forward with H = 1, W = L.
 */
int ss2d_bidir_forward(const void* x, const void* dt, const float* A_log, const float* dt_bias,
                       const void* Bs, const void* Cs, const float* Ds, void* y,
                       int64_t B, int64_t D, int64_t L, int64_t N, int dtype, void* stream);

/*
 * ss2d_project -- enqueue the per-direction input projections of SS2D on `stream`:
 * from the feature map and the projection weights, the dt, Bs and Cs that
 * ss2d_forward consumes.  Page [SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现"
 * §3.2 (the parameter projection before the selective scan: x_proj over the four
 * scan sequences, the split into dts / Bs / Cs, and the dt_projs map); the rank
 * R is sized ceil(d_model / 16) there (§1), any R >= 1 is accepted here.
 *
 * Every pointer is DEVICE memory owned by the caller, dense, row-major.  With
 * C = R + 2N and u the D channels of the pixel direction k visits at step l:
 *   x                [B, D, H, W]   dtype  channel-first feature map.
 *   x_proj_weight    [4, C, D]      fp32   row c of direction k: the c-th
 *                                          projection (rows 0..R-1 feed dt,
 *                                          R..R+N-1 are Bs, R+N..C-1 are Cs).
 *   dt_projs_weight  [4, D, R]      fp32
 *   dt               [B, 4, D, L]   dtype  out: sum_r dt_projs_weight[k,d,r] *
 *                                          (x_proj_weight[k,r,:] . u); no bias.
 *   Bs, Cs           [B, 4, N, L]   dtype  out: x_proj_weight[k,R+n,:] . u and
 *                                          x_proj_weight[k,R+N+n,:] . u.
 * All three outputs are in scan order, the layout ss2d_forward reads, and are
 * fully overwritten; they must not overlap each other or any input
 * (SS2D_ERR_ALIAS).  Products and sums are fp32 on the matrix cores; bf16
 * outputs are rounded once, to nearest even.  2*(R + 2N) may be at most 128
 * (SS2D_ERR_SHAPE otherwise, as for R < 1); N is 1..16 as for ss2d_forward.
 * Takes a stream-ordered temporary of one copy of x (with H and W swapped) and
 * runs two kernels on `stream`.  Validation, error reporting and thread safety
 * as for ss2d_forward; the weights need 4-byte alignment (SS2D_ERR_ALIGN).
 */
int ss2d_project(const void* x, const float* x_proj_weight, const float* dt_projs_weight,
                 void* dt, void* Bs, void* Cs,
                 int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int64_t R,
                 int dtype, void* stream);

/*
 * ss2d_forward_from_x -- enqueue the SS2D forward from the feature map and the
 * projection weights: ss2d_project, then ss2d_forward on its outputs, with the
 * intermediate dt, Bs and Cs (in `dtype`) kept in a stream-ordered temporary.
 * Page [SS2D] §3.2 steps in order: projections, selective scan (A = -exp(A_log),
 * delta bias dt_bias, softplus), then §3.3 the merge.  Arguments as for the two
 * calls; y must not overlap any input.  The temporary holds x transposed, dt,
 * Bs, Cs and what ss2d_forward needs; the scan's column walks read the
 * transposed copy of x.  Three kernels (more for segmented maps) on `stream`.
 */
int ss2d_forward_from_x(const void* x, const float* x_proj_weight, const float* dt_projs_weight,
                        const float* A_log, const float* dt_bias, const float* Ds, void* y,
                        int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int64_t R,
                        int dtype, void* stream);

/*
 * ss2d_channel_last -- enqueue the step after the merge on `stream`: y in
 * channel-first layout to channel-last, optionally normalised over its channels.
 * Page [SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现" §3.3 (the merged y is
 * transposed to (B, H, W, D)); [VSSD] §5.3 (fusing the LayerNorm that follows).
 *   y      [B, D, H, W]   dtype  device memory, read only.
 *   gamma  [D]            fp32   per-channel scale, or NULL for 1.
 *   beta   [D]            fp32   per-channel shift, or NULL for 0.
 *   out    [B, H, W, D]   dtype  fully overwritten; must not overlap y, gamma or
 *                                beta (SS2D_ERR_ALIAS).
 * normalize = 0: out[b,h,w,d] = y[b,d,h,w] (gamma, beta and eps unused).
 * normalize = 1: with m and v the mean and the biased variance of the D values
 *   y[b,:,h,w], out[b,h,w,d] = (y[b,d,h,w] - m) / sqrt(v + eps) * gamma[d] + beta[d],
 *   statistics in fp32; bf16 output is rounded once.  eps must be >= 0 and finite.
 * D may be at most 4096 and normalize must be 0 or 1 (SS2D_ERR_SHAPE otherwise;
 * a bad eps is SS2D_ERR_SHAPE too).  One kernel on `stream`, no temporary.
 * Validation, error reporting and thread safety as for ss2d_forward.
 */
int ss2d_channel_last(const void* y, const float* gamma, const float* beta, float eps, int normalize,
                      void* out, int64_t B, int64_t D, int64_t H, int64_t W, int dtype, void* stream);

/*
 * ss2d_backward -- enqueue the gradients of the forward on `stream`: given dy,
 * the gradient of a loss with respect to y, write the gradients with respect to
 * every input of ss2d_forward.  Page [SS2D] "深入解析VMamba中的SS2D模块从理论到
 * 代码实现" §3.1-§3.3 define the forward; the gradients follow by the chain rule,
 * with the state adjoint q_l = Cs[n,l] dy_l + exp(delta_{l+1} A) q_{l+1} walked
 * from the end of each sequence (dy_l: dy at the pixel the direction visits).
 *   inputs  x, dt, A_log, dt_bias, Bs, Cs, Ds  as for ss2d_forward;
 *           dy      [B, D, H, W]   dtype
 *   outputs dx      [B, D, H, W]   dtype
 *           ddt     [B, 4, D, L]   dtype
 *           dA_log  [4*D, N]       fp32   summed over the batch
 *           ddt_bias[4*D]          fp32   summed over the batch and steps
 *           dBs, dCs[B, 4, N, L]   dtype  summed over the D channels
 *           dDs     [4*D]          fp32   summed over the batch and steps
 * Every output is fully overwritten (no accumulation into existing values) and
 * must not overlap an input or another output (SS2D_ERR_ALIAS).  All arithmetic
 * is fp32; bf16 outputs are rounded once.  N is 1..256: more than 16 states run
 * in passes of 16 states, each writing its states' dA_log, dBs and dCs, with du,
 * ddt and ddt_bias summed over the passes in pass order (ddt in fp32 until the
 * last pass rounds it).  All sums run in a fixed order, so results are
 * deterministic.  Takes a stream-ordered temporary of at most about
 * B*4*D*L + 2*B*D*L + 2*B*4*ceil(D/16)*n*L + 16*B*4*D*n*ceil(L/128) + B*4*D*N
 * fp32 values with n = min(N, 16) (du, transposed copies of x and dy, dBs and
 * dCs partials, one per workgroup of one or two 16-channel blocks, the state
 * entering every 8 steps, the dA_log partials), plus B*4*D*L for the ddt sum
 * when N > 16, and runs four kernels per pass and three more on `stream`.
 * When B*4*ceil(D/16) is below 768, each sequence is cut into S segments of at least
 * 512 steps (S from ss2d_describe): two more kernels, and about
 * 16*B*4*D*ceil(L/128) + 3*B*4*S*D*n more temporary values.
 * Validation, error reporting and thread safety as for ss2d_forward; pointers
 * need element alignment: the storage type for the dtype tensors, 4 bytes for
 * the fp32 ones (SS2D_ERR_ALIGN).  With L a multiple of 4 and bases aligned to
 * 16 bytes (fp32) or 8 bytes (bf16), as torch allocates them, the kernels move
 * four elements per access; element-aligned bases take one-element accesses and
 * give identical results.
 */
int ss2d_backward(const void* x, const void* dt, const float* A_log, const float* dt_bias,
                  const void* Bs, const void* Cs, const float* Ds, const void* dy,
                  void* dx, void* ddt, float* dA_log, float* ddt_bias, void* dBs, void* dCs,
                  float* dDs, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                  int dtype, void* stream);

/*
 * ss2d_bidir_backward -- the gradients of ss2d_bidir_forward given dy, the
 * gradient of a loss with respect to y: the chain rule along each of the two
 * paths of [VSSD] page "项目概述：当视觉Transformer遇到状态空间模型" §2.2, exactly as
 * ss2d_backward does along the cross scan's directions, with the state adjoint
 * q_l = Cs[b,j,n,l] dy[b,d,t_j(l)] + exp(delta_{l+1} A) q_{l+1} walked from the
 * end of each path.
 *   inputs  x, dt, A_log, dt_bias, Bs, Cs, Ds  as for ss2d_bidir_forward;
 *           dy      [B, D, L]      dtype
 *   outputs dx      [B, D, L]      dtype  (both paths' terms at each token)
 *           ddt     [B, 2, D, L]   dtype  (each path's step order)
 *           dA_log  [2*D, N]       fp32   summed over the batch
 *           ddt_bias[2*D]          fp32   summed over the batch and steps
 *           dBs, dCs[B, 2, N, L]   dtype  summed over the D channels
 *           dDs     [2*D]          fp32   summed over the batch and steps
 *   N       1..256 (passes of 16 states, as in ss2d_backward)
 * Overwrite, aliasing, arithmetic, determinism, temporaries (without the
 * transposed copies: a sequence has no column walk), validation, alignment,
 * error reporting and thread safety as for ss2d_backward with H = 1, W = L.
 */
int ss2d_bidir_backward(const void* x, const void* dt, const float* A_log, const float* dt_bias,
                        const void* Bs, const void* Cs, const float* Ds, const void* dy,
                        void* dx, void* ddt, float* dA_log, float* ddt_bias, void* dBs, void* dCs,
                        float* dDs, int64_t B, int64_t D, int64_t L, int64_t N,
                        int dtype, void* stream);

/* Static English text for a status code (never NULL). */
const char* ss2d_status_string(int status);

/* Text of the last HIP error seen by this thread (for SS2D_ERR_HIP); "" if none. */
const char* ss2d_last_hip_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int ss2d_version(void);

/*
 * ss2d_describe -- write a one-line, NUL-terminated description of how
 * ss2d_forward would run this shape with 16/8-byte aligned bases (kernel
 * variant, lanes per sequence, channels per workgroup, grid size, LDS and
 * temporary sizes, passes over state blocks), followed by the number of
 * segments ss2d_backward cuts each sequence into and the number of 16-channel
 * blocks each of its workgroups takes, then the same two numbers for
 * ss2d_bidir_backward over a sequence of L = H*W tokens, into buf[0..len).
 * Host only; no device work.  Returns SS2D_OK or a validation code.
 * ss2d_describe_lanes: the same for ss2d_forward_lanes.
 */
int ss2d_describe(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype,
                  char* buf, int64_t len);
int ss2d_describe_lanes(int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype,
                        int lanes_per_seq, char* buf, int64_t len);

/*
 * ss2d_trim_memory -- return the freed blocks the library's memory pools hold
 * (one pool per device the library has run on) to the system.  Call only when no
 * library work is in flight.  SS2D_OK or SS2D_ERR_HIP.
 */
int ss2d_trim_memory(void);

/*
 * ss2d_measure_peaks -- measure, on the current device, the rates the forward is
 * measured against (its roofline), one probe kernel per rate, each timed with HIP
 * events as the best of three runs on `stream`:
 *   exp_per_s         v_exp_f32 results per second (8 independent chains per lane)
 *   fma_per_s         plain fp32 FMA results per second
 *   update_mix_per_s  state-update-shaped work per second: one exp2 and four fp32
 *                     VALU operations per update, as the scan's inner loop needs
 *   hbm_read_Bps      streaming read bandwidth over hbm_bytes
 *   hbm_copy_Bps      device copy of hbm_bytes/2, bytes read plus bytes written
 *   lds_read_Bps      16-byte LDS reads, all CUs
 *   compute_units     CUs of the device
 *   state_loop_per_s  state updates per second of the forward's state loop
 *                     alone (per state the fold, the DPP prefix combine over 32
 *                     lanes, the carried state and the replay with the output FMA,
 *                     16 steps per lane, one barrier per four states), operands in
 *                     LDS and registers, at the forward's occupancy: what the
 *                     chunked form reaches without its per-step work, memory
 *                     traffic, waits or merge
 * The probes allocate hbm_bytes (1 MiB .. 64 GiB, multiple of 32) plus a small
 * sink from the device's default memory pool on `stream` and free them; the call
 * returns after synchronising `stream`.  Codes: SS2D_ERR_NULL (out), SS2D_ERR_SHAPE
 * (hbm_bytes), SS2D_ERR_NO_DEVICE, SS2D_ERR_HIP.  For benchmarking only; not
 * needed by ss2d_forward.
 */
typedef struct {
  double exp_per_s;
  double fma_per_s;
  double update_mix_per_s;
  double hbm_read_Bps;
  double hbm_copy_Bps;
  double lds_read_Bps;
  int compute_units;
  double state_loop_per_s;
} ss2d_peaks;
int ss2d_measure_peaks(ss2d_peaks* out, int64_t hbm_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SS2D_H_ */
