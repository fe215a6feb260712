/*
 * ssdq.h -- C ABI of the INT8-input Mamba-2 SSD scan for AMD MI355X (gfx950).
 *
 * The library evaluates the selective state-space recurrence of Mamba-2
 * (stated in Ternary Mamba, Section 1, as h_t = Abar_t h_{t-1} + Bbar_t x_t)
 * with the zero-order-hold decay Abar_t = exp(dt_t A_h), Bbar_t = dt_t B_t and
 * the readout y_t = C_t . h_t + D_h x_t, where x, B and C arrive as INT8 codes
 * with static scales: one fp32 scale per head for x and one per state group
 * for B and C (Quamba2 rebuttal: 8-bit SSD inputs B, C, x and per-state-group
 * quantization; SSDi8 Table 10: per-H(G) scales; Quamba project page: static
 * scales).  Prefill uses the chunked state-space-duality evaluation (SSDi8
 * abstract and Figure 1b: chunk state, chunk-level C.B^T on INT8, state
 * passing); decode is one recurrence step per call (Quamba2 rebuttal: the SSD
 * update is the decode-time latency and memory bottleneck).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless stated otherwise, must be 16-byte
 *    aligned, and address contiguous row-major tensors in the layouts given.
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates or frees device memory, never synchronizes the device, keeps no
 *    global state and is safe to call from several host threads.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream) of the
 *    current HIP device.
 *  - Arguments are validated on the host before anything is enqueued; any
 *    status other than SSDQ_SUCCESS means nothing was enqueued.  Validation
 *    cannot read device memory, so NaN/Inf or out-of-range VALUES in device
 *    buffers are not detected (see each call for what they produce).
 *  - y (fp16) never aliases an input.  The only aliases allowed are the ones
 *    each call names.
 */
#ifndef SSDQ_H_
#define SSDQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSDQ_SUCCESS = 0,
  SSDQ_ERROR_INVALID_VALUE = 1,       /* null / misaligned pointer, non-positive size, H % G != 0 */
  SSDQ_ERROR_UNSUPPORTED = 2,         /* a shape the kernels do not handle (see each call) */
  SSDQ_ERROR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below ssdq_chunk_scan_workspace_size() */
  SSDQ_ERROR_LAUNCH = 4,              /* the HIP runtime rejected a kernel launch */
  SSDQ_ERROR_SCRATCH_LIMIT = 5        /* ssdq_chunk_scan_noalloc: the shape needs more than the static scratch */
} ssdq_status;

/* Human-readable name of a status (host; static storage; never NULL). */
const char* ssdq_status_string(ssdq_status status);

/*
 * Static INT8 quantizer (the 8-bit SSD inputs of the Quamba2 rebuttal; static
 * per-head / per-group scales of SSDi8 Table 10).
 *
 *   q[r, k, i] = clamp(round_half_even(float(x[r, k, i]) / scale[k]), -127, 127)
 *
 * with the fp32 quotient correctly rounded (not a reciprocal multiply).
 * A NaN quotient gives 0 and +-Inf gives +-127; -128 is never produced.
 *   x_f16 : (rows, nscale, inner) IEEE binary16, device
 *   q     : (rows, nscale, inner) int8, device, written
 *   scale : [nscale] fp32, device (positive finite for meaningful codes)
 * Use for x (b, L, H, P): rows = b*L, nscale = H, inner = P; for B or C
 * (b, L, G, N): rows = b*L, nscale = G, inner = N.  Any rows >= 0 (0 = no-op),
 * nscale >= 1, inner >= 1.  q must not overlap x_f16.
 */
ssdq_status ssdq_quantize(const void* x_f16, int8_t* q, const float* scale, int64_t rows, int32_t nscale,
                          int32_t inner, hipStream_t stream);

/* One tensor of a batched quantize: the arguments of ssdq_quantize. */
typedef struct {
  const void* x_f16;   /* (rows, nscale, inner) IEEE binary16, device */
  int8_t* q;           /* (rows, nscale, inner) int8, device, written */
  const float* scale;  /* [nscale] fp32, device */
  int64_t rows;
  int32_t nscale;
  int32_t inner;
} ssdq_quantize_job;

#define SSDQ_QUANTIZE_MAX_JOBS 8

/*
 * The same static INT8 quantizer applied to several tensors (x, B and C of one step) in
 * one kernel launch where their shapes allow it: each job's codes equal those of
 * ssdq_quantize with the same arguments.  Jobs whose inner is a multiple of 16 share one
 * launch; any other job is launched on its own (same stream, same result).
 *   jobs  : host array of `count` jobs, read during the call only
 *   count : 1 .. SSDQ_QUANTIZE_MAX_JOBS
 * Every job is validated as ssdq_quantize validates its arguments before anything is
 * launched (one invalid job: nothing runs).  Jobs with rows == 0 are skipped.  No output
 * may overlap another job's output or any job's input.
 */
ssdq_status ssdq_quantize_batch(const ssdq_quantize_job* jobs, int32_t count, hipStream_t stream);

/*
 * The static INT8 quantizer with one scale per (k, i) instead of one per k: B or C with a scale per
 * (group, state), the finer granularity of SSDi8 Table 10 (per-P(N) together with per-H(G)), or x
 * with a scale per (head, channel) (rows = b*L, nscale = H, inner = P, scale (H, P)).
 *
 *   q[r, k, i] = clamp(round_half_even(float(x[r, k, i]) / scale[k, i]), -127, 127)
 *
 *   scale : (nscale, inner) fp32, device (each positive finite)
 * Arguments, layout, rounding, special values and validation otherwise as ssdq_quantize (B or C
 * (b, L, G, N): rows = b*L, nscale = G, inner = N, scale (G, N)); codes bit-exact to the
 * correctly rounded quotient.
 */
ssdq_status ssdq_quantize_per_channel(const void* x_f16, int8_t* q, const float* scale, int64_t rows,
                                      int32_t nscale, int32_t inner, hipStream_t stream);

/* Bytes of workspace ssdq_chunk_scan needs for this shape (host; 0 on invalid shapes).
 * Layout (stable, used by the stage-level tests), with nchunks = ceil(seqlen / chunk) and
 * each region starting at a 256-byte boundary:
 *   Acs     fp32 (batch, nheads, nchunks, chunk): within-chunk inclusive cumsum of dt * A
 *           (padded past the sequence end with the last value)           -- written by stage 0
 *   Dtc     fp32 (batch, nheads, nchunks, chunk): dt in the same chunk order, 0 past the
 *           sequence end (one contiguous row per chunk for stage 2)      -- written by stage 0
 *   S       fp32 (batch, nchunks, nheads, headdim, dstate): chunk states  -- written by stage 0
 *   Hprev   int8 (batch, nchunks, nheads, 2, headdim, dstate) and
 *   Hscale  fp32 (batch, nchunks, nheads, headdim): the state entering each chunk is
 *           (Hprev[..., 0, p, n] + Hprev[..., 1, p, n] / 256) * Hscale[..., p], two INT8
 *           limbs with a power-of-two scale per state row           -- written by stage 1
 *           Within each full 64-state block of a row, the 4 bytes of states
 *           64 blk + 16 t + 4 k + (0..3) are stored at 64 blk + 16 k + 4 t + (0..3) (a 4x4
 *           transpose of 4-byte groups: the writing lanes store 16 contiguous bytes); a
 *           partial last block (dstate % 64 != 0) is stored in natural order.
 * When ssdq_chunk_scan_state_fused(batch, nheads) is 1, stage 0 writes Acs, Dtc, Hprev, Hscale
 * (and h_final) itself, stage 1 does nothing, and S is not written. */
size_t ssdq_chunk_scan_workspace_size(int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim,
                                      int32_t dstate, int32_t chunk);

/*
 * Prefill: the chunked SSD scan over INT8 inputs (SSDi8 Figure 1b pipeline).
 *
 *   for every (b, h):  h_{-1} = h0[b, h] (or 0),
 *     h_t = exp(dt[b,t,h] A[h]) h_{t-1} + dt[b,t,h] * xhat[b,t,h,:] (x) Bhat[b,t,g,:]
 *     y[b,t,h,:] = h_t . Chat[b,t,g,:] + D[h] * xhat[b,t,h,:]
 *   with xhat = x_scale[h] * x, Bhat = B_scale[g] * B, Chat = C_scale[g] * C and
 *   g = h / (nheads / ngroups).
 *
 *   x  : (batch, seqlen, nheads, headdim) int8      x_scale : [nheads] fp32
 *   B  : (batch, seqlen, ngroups, dstate) int8      B_scale : [ngroups] fp32
 *   C  : (batch, seqlen, ngroups, dstate) int8      C_scale : [ngroups] fp32
 *   (every scale finite and > 0: the output kernel divides by them, and a zero or non-finite
 *   scale gives non-finite y; calibration gives a zero-absmax group the scale 1)
 *   dt : (batch, seqlen, nheads) fp32, > 0, already passed through softplus
 *   A  : [nheads] fp32, finite, <= 0          D : [nheads] fp32 or NULL (= 0)
 *   h0 : (batch, nheads, headdim, dstate) fp32 or NULL (= 0)
 *   y  : (batch, seqlen, nheads, headdim) fp16, written
 *   h_final : (batch, nheads, headdim, dstate) fp32 or NULL; may alias h0
 *   workspace : device scratch of at least ssdq_chunk_scan_workspace_size() bytes,
 *               owned by the caller, not shared with a concurrent call
 * Supported shapes: headdim % 16 == 0 and headdim <= 64; dstate % 16 == 0 and
 * dstate <= 128; chunk in {64, 128, 256}; any seqlen >= 1 (a ragged last chunk
 * is masked); nheads % ngroups == 0; nheads * headdim * chunk < 2^30,
 * ngroups * dstate * chunk < 2^31 and batch * seqlen * nheads < 2^31.  Others
 * return SSDQ_ERROR_UNSUPPORTED.
 * Accuracy: y within 2e-3 * max|y| and h_final within 1e-4 * max|h| of the exact
 * recurrence over the same codes (fp32 accumulation, fp16 y).
 */
ssdq_status ssdq_chunk_scan(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                            const int8_t* C, const float* C_scale, const float* dt, const float* A,
                            const float* D, const float* h0, void* y, float* h_final, int32_t batch,
                            int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                            int32_t chunk, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Number of stages ssdq_chunk_scan runs, in order: 0 chunk cumsum + chunk state,
 * 1 state passing, 2 chunk output. */
#define SSDQ_CHUNK_SCAN_STAGES 3

/*
 * 1 if, on the current device, ssdq_chunk_scan folds state passing into stage 0 for this
 * batch and head count, else 0 (also for non-positive arguments or without a device).
 * Folding applies when batch * nheads is at least the device's CU count: one block per
 * (batch, head) sequence then walks its chunks in order (Mamba-2 SSD state passing,
 * Ternary Mamba sec. 1 recurrence per chunk) and the fp32 chunk states never reach memory.
 */
int32_t ssdq_chunk_scan_state_fused(int32_t batch, int32_t nheads);

/*
 * The form of stage 0 that ssdq_chunk_scan (scale_layout 0) or ssdq_chunk_scan_scaled takes on
 * the current device for this batch and head count (host; informational, the results do not
 * depend on it beyond fp32 rounding):
 *   0 : three kernels (chunk states in parallel, then state passing; ssdq_chunk_scan_state_fused 0)
 *   8 : the folded state kernel in blocks of eight waves, one block per CU at a time
 *   4 : the folded state kernel in blocks of four waves, two blocks per CU (many more sequences
 *       than CUs)
 *  -1 : non-positive sizes or unknown scale_layout bits.
 */
int32_t ssdq_chunk_scan_plan(int32_t batch, int32_t nheads, uint32_t scale_layout);

/*
 * One stage of ssdq_chunk_scan, with the same arguments and validation.
 * Running stages 0..2 in order on one stream is exactly ssdq_chunk_scan; the
 * intermediate results are in the workspace layout documented above.  This
 * lets a caller time each kernel with its own events and lets tests inspect
 * the intermediates.  stage outside [0, SSDQ_CHUNK_SCAN_STAGES) is INVALID_VALUE.
 */
ssdq_status ssdq_chunk_scan_stage(int32_t stage, const int8_t* x, const float* x_scale, const int8_t* B,
                                  const float* B_scale, const int8_t* C, const float* C_scale,
                                  const float* dt, const float* A, const float* D, const float* h0, void* y,
                                  float* h_final, int32_t batch, int64_t seqlen, int32_t nheads,
                                  int32_t headdim, int32_t dstate, int32_t ngroups, int32_t chunk,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ssdq_chunk_scan with SSDi8's output correction: every output also receives a per-(head,
 * channel) term (the SSDi8 abstract describes a correction derived from error statistics gathered
 * per channel, Figure 1b labels it a mean correction; Tables 6 and 16).  The pages give no algebra for it; the reading
 * taken is the plainest they support: an additive term, calibrated offline (like the static
 * scales) as the mean over a calibration set of the unquantized scan's y minus the quantized
 * scan's y, channel by channel.  Calibration is the caller's; the library only applies it:
 *
 *   y[b,t,h,p] = (the output of ssdq_chunk_scan) + y_corr[h, p]     (added in fp32 before the fp16 rounding)
 *
 *   y_corr : (nheads, headdim) fp32, device, 16-byte aligned (NULL: SSDQ_ERROR_INVALID_VALUE)
 * Every other argument, the shapes, the accuracy and the validation are those of ssdq_chunk_scan,
 * and h_final does not depend on y_corr.
 */
ssdq_status ssdq_chunk_scan_corrected(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                                      const int8_t* C, const float* C_scale, const float* dt, const float* A,
                                      const float* D, const float* y_corr, const float* h0, void* y, float* h_final,
                                      int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                                      int32_t ngroups, int32_t chunk, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * ssdq_chunk_scan with B and C scales per (group, state) (SSDi8 Table 10: per-P(N) together with
 * per-H(G)) and an optional output correction:
 *
 *   Bhat[b,t,g,n] = B_scale[g, n] B[b,t,g,n],   Chat[b,t,g,n] = C_scale[g, n] C[b,t,g,n]
 *   (the recurrence and readout of ssdq_chunk_scan over these), plus y_corr[h, p] on every y
 *
 *   B_scale, C_scale : (ngroups, dstate) fp32, device, each finite and > 0
 *   y_corr           : (nheads, headdim) fp32 or NULL (no correction)
 * Everything else as ssdq_chunk_scan, except:
 *  - C.B^T over the per-state scales runs on the INT8 matrix cores with the product
 *    B_scale C_scale of each state folded into the B codes as a 16-bit fixed-point number (two
 *    INT8 limbs) relative to the group's largest product: each term of the sum carries at most
 *    2^-9 of that largest product times |C code|, well inside the stated y accuracy;
 *  - the workspace regions of the chunk states and the carried state hold those states times
 *    C_scale[g, n] of each state column (h_final is unscaled).
 */
ssdq_status ssdq_chunk_scan_per_state(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                                      const int8_t* C, const float* C_scale, const float* dt, const float* A,
                                      const float* D, const float* y_corr, const float* h0, void* y, float* h_final,
                                      int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                                      int32_t ngroups, int32_t chunk, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Scale layouts for ssdq_chunk_scan_scaled and ssdq_state_update_scaled (bit flags; 0 is the
 * layout of ssdq_chunk_scan: one x scale per head, one B and one C scale per group). */
#define SSDQ_SCALES_BC_PER_STATE 1u  /* B_scale, C_scale: (ngroups, dstate) */
#define SSDQ_SCALES_X_PER_CHANNEL 2u /* x_scale: (nheads, headdim) */

/*
 * ssdq_chunk_scan under any of the static scale layouts, with an optional output correction.
 * With SSDQ_SCALES_X_PER_CHANNEL, x has one static scale per (head, channel):
 *
 *   xhat[b,t,h,p] = x_scale[h, p] x[b,t,h,p]
 *
 * the granularity that Quamba2's sort-and-cluster of the x channels produces (its rebuttal names
 * the sort-and-cluster and the per-state-group quantization as the two steps; each channel cluster
 * of a head shares one scale, given here expanded to every channel of the cluster, so any
 * clustering, sorted or not, is one (nheads, headdim) table).  Such a scale factors out of every
 * contraction of the scan (they sum over tokens and states, never over channels), and is applied
 * in fp32 per output channel and per state row.  With SSDQ_SCALES_BC_PER_STATE, B and C have
 * one scale per (group, state) as in ssdq_chunk_scan_per_state.  Both bits may be set.
 *
 *   x_scale      : (nheads) fp32, or (nheads, headdim) with SSDQ_SCALES_X_PER_CHANNEL; each
 *                  finite and > 0
 *   B_scale, C_scale : (ngroups) fp32, or (ngroups, dstate) with SSDQ_SCALES_BC_PER_STATE
 *   y_corr       : (nheads, headdim) fp32 or NULL (no correction)
 *   scale_layout : SSDQ_SCALES_* bits (other bits: SSDQ_ERROR_INVALID_VALUE)
 * Everything else (shapes, workspace, accuracy, validation) as ssdq_chunk_scan; the codes of x are
 * those of ssdq_quantize_per_channel under the (nheads, headdim) table.
 */
ssdq_status ssdq_chunk_scan_scaled(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                                   const int8_t* C, const float* C_scale, const float* dt, const float* A,
                                   const float* D, const float* y_corr, const float* h0, void* y, float* h_final,
                                   int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                                   int32_t ngroups, int32_t chunk, uint32_t scale_layout, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Bytes of the library's static device scratch that ssdq_chunk_scan_noalloc uses (per device). */
#define SSDQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * ssdq_chunk_scan without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The
 * intermediates (Acs, the chunk-ordered dt, the chunk states of the three-kernel plan, the
 * carried-state limbs and their row scales) live in one static device array of SSDQ_NOALLOC_SCRATCH_BYTES that the
 * library holds on every device it runs on until the process ends; the call allocates and
 * frees nothing.  Arguments, shapes, accuracy and validation are those of ssdq_chunk_scan, and
 * the results are those of ssdq_chunk_scan with the same arguments (the same kernels run).
 *   - A shape whose intermediates exceed the scratch (ssdq_chunk_scan_noalloc_scratch_size()
 *     above SSDQ_NOALLOC_SCRATCH_BYTES) returns SSDQ_ERROR_SCRATCH_LIMIT and launches nothing.
 *   - Every call on a device shares that device's scratch, and it keeps the last call's contents:
 *     calls that overlap on one device (concurrent streams, or several host threads without
 *     ordering) race on it and must be serialized by the caller.  Calls on one stream are
 *     ordered and safe.  Nothing in the scratch needs to start at zero.
 *   - The first call on a device looks up the scratch's device address (hipGetSymbolAddress);
 *     if that fails the call returns SSDQ_ERROR_LAUNCH.
 */
ssdq_status ssdq_chunk_scan_noalloc(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                                    const int8_t* C, const float* C_scale, const float* dt, const float* A,
                                    const float* D, const float* h0, void* y, float* h_final, int32_t batch,
                                    int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                                    int32_t ngroups, int32_t chunk, hipStream_t stream);

/* Scratch bytes ssdq_chunk_scan_noalloc needs for this shape on the current device (host; 0 on
 * invalid shapes): the Acs, Dtc, carried-state and row-scale regions, plus the fp32 chunk states when
 * the three-kernel plan runs, each rounded up to 256 bytes. */
size_t ssdq_chunk_scan_noalloc_scratch_size(int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim,
                                            int32_t dstate, int32_t chunk);

/*
 * Decode: one recurrence step per sequence, state updated IN PLACE (the
 * decode-time SSD update of the Quamba2 rebuttal, Tables R7/R8).
 *
 *   state[b,h,p,n] <- exp(dt[b,h] A[h]) state[b,h,p,n] + dt[b,h] xhat[b,h,p] Bhat[b,g,n]
 *   y[b,h,p] = sum_n Chat[b,g,n] state[b,h,p,n] (updated) + D[h] xhat[b,h,p]
 *
 *   state : (batch, nheads, headdim, dstate) fp32, read and written
 *   x : (batch, nheads, headdim) int8     B, C : (batch, ngroups, dstate) int8
 *   dt : (batch, nheads) fp32   A : [nheads]   D : [nheads] or NULL   y : (batch, nheads, headdim) fp16
 * Supported: dstate == 128 or dstate == 64, headdim <= 64, nheads % ngroups == 0.
 */
ssdq_status ssdq_state_update(float* state, const int8_t* x, const float* x_scale, const int8_t* B,
                              const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                              const float* A, const float* D, void* y, int32_t batch, int32_t nheads,
                              int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream);

/*
 * The decode step with the state cached in IEEE binary16: half the bytes per step of the fp32
 * state on the HBM-bound update (a lower-precision cached SSM state, as the Quamba2
 * rebuttal's Tables R7/R8 discuss for decode-time memory and latency).
 *
 *   u[b,h,p,n] = exp(dt[b,h] A[h]) state[b,h,p,n] + dt[b,h] xhat[b,h,p] Bhat[b,g,n]   (fp32)
 *   y[b,h,p]   = sum_n Chat[b,g,n] u[b,h,p,n] + D[h] xhat[b,h,p]                   (from u)
 *   state[b,h,p,n] <- u rounded to the nearest binary16 (ties to even; |u| beyond the
 *                     format's range gives +-inf)
 *
 *   state : (batch, nheads, headdim, dstate) IEEE binary16, read and written
 * Every other argument, the shapes supported and the validation are those of
 * ssdq_state_update.  Each step rounds the state once (2^-11 relative at most), so after T
 * steps the cached state is within T * 2^-11 of the largest state magnitude of the fp32
 * recurrence; the caller chooses it where that is acceptable.
 */
ssdq_status ssdq_state_update_f16(void* state, const int8_t* x, const float* x_scale, const int8_t* B,
                                  const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                                  const float* A, const float* D, void* y, int32_t batch, int32_t nheads,
                                  int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream);

/*
 * The decode step with the state cached as 8-bit codes and one binary32 scale per state row
 * (b, h, p): a quarter of the fp32 state's bytes per step (the 8-bit cached SSM states of the
 * Quamba2 rebuttal, Tables R7/R8; the pages do not fix the scale granularity, one scale per
 * row and the symmetric max/127 rule are the choice made here).
 *
 *   u[b,h,p,n] = exp(dt[b,h] A[h]) scale[b,h,p] state[b,h,p,n] + dt[b,h] xhat[b,h,p] Bhat[b,g,n]  (fp32)
 *   y[b,h,p]   = sum_n Chat[b,g,n] u[b,h,p,n] + D[h] xhat[b,h,p]                               (from u)
 *   scale[b,h,p] <- max_n |u[b,h,p,n]| / 127     (binary32; 0, with zero codes, when that is below 2^-126)
 *   state[b,h,p,n] <- u / scale rounded to nearest, ties to even, within [-127, 127] (0 if scale is 0)
 *
 *   state       : (batch, nheads, headdim, dstate) int8 codes, read and written
 *   state_scale : (batch, nheads, headdim) float32, read and written; 16-byte aligned
 * Every other argument, the shapes supported and the validation are those of
 * ssdq_state_update; a NULL or misaligned state_scale gives SSDQ_ERROR_INVALID_VALUE.  Each step
 * moves every element by at most half a code step (max|row| / 254), so after T steps the cached
 * state is within T/254 of the largest row magnitude of the fp32 recurrence; the values must
 * stay finite (a non-finite update makes its row's scale non-finite).  Codes where the update
 * falls within fp32 rounding of a midpoint between two codes may take either neighbour.
 */
ssdq_status ssdq_state_update_i8(int8_t* state, float* state_scale, const int8_t* x, const float* x_scale,
                                 const int8_t* B, const float* B_scale, const int8_t* C, const float* C_scale,
                                 const float* dt, const float* A, const float* D, void* y, int32_t batch,
                                 int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                                 hipStream_t stream);

/* Formats of the decode state for ssdq_state_update_corrected. */
typedef enum {
  SSDQ_STATE_F32 = 0,   /* fp32 state, as ssdq_state_update */
  SSDQ_STATE_F16 = 1,   /* IEEE binary16 cache, as ssdq_state_update_f16 */
  SSDQ_STATE_I8 = 2     /* 8-bit codes + row scales, as ssdq_state_update_i8 */
} ssdq_state_format;

/*
 * The decode step with the output correction of ssdq_chunk_scan_corrected: the step of the given
 * state format (its arguments, layout, validation and in-place update unchanged) whose y also
 * receives y_corr[h, p]:
 *
 *   y[b,h,p] = (the y of the plain step) + y_corr[h, p]
 *
 *   state_format : SSDQ_STATE_F32, SSDQ_STATE_F16 or SSDQ_STATE_I8 (else SSDQ_ERROR_INVALID_VALUE)
 *   state        : (batch, nheads, headdim, dstate) fp32, binary16 or int8 codes, read and written
 *   state_scale  : (batch, nheads, headdim) fp32 row scales for SSDQ_STATE_I8, read and written;
 *                  ignored (may be NULL) for the other formats
 *   y_corr       : (nheads, headdim) fp32, device, 16-byte aligned (NULL: SSDQ_ERROR_INVALID_VALUE)
 * The state does not depend on y_corr.
 */
ssdq_status ssdq_state_update_corrected(int32_t state_format, void* state, float* state_scale, const int8_t* x,
                                        const float* x_scale, const int8_t* B, const float* B_scale, const int8_t* C,
                                        const float* C_scale, const float* dt, const float* A, const float* D,
                                        const float* y_corr, void* y, int32_t batch, int32_t nheads, int32_t headdim,
                                        int32_t dstate, int32_t ngroups, hipStream_t stream);

/*
 * The decode step of ssdq_state_update_corrected with B and C scales per (group, state):
 * B_scale, C_scale (ngroups, dstate) fp32; y_corr (nheads, headdim) fp32 or NULL (no correction).
 * Formats, arguments, layouts and validation otherwise as ssdq_state_update_corrected.  (On the
 * 8-bit cached state, y is then summed in fp32 over the per-state C values instead of by integer
 * dot products.)
 */
ssdq_status ssdq_state_update_per_state(int32_t state_format, void* state, float* state_scale, const int8_t* x,
                                        const float* x_scale, const int8_t* B, const float* B_scale, const int8_t* C,
                                        const float* C_scale, const float* dt, const float* A, const float* D,
                                        const float* y_corr, void* y, int32_t batch, int32_t nheads, int32_t headdim,
                                        int32_t dstate, int32_t ngroups, hipStream_t stream);

/*
 * The decode step of ssdq_state_update_corrected under any of the static scale layouts of
 * ssdq_chunk_scan_scaled (scale_layout: SSDQ_SCALES_* bits; x_scale (nheads, headdim) with
 * SSDQ_SCALES_X_PER_CHANNEL, B_scale and C_scale (ngroups, dstate) with
 * SSDQ_SCALES_BC_PER_STATE); y_corr (nheads, headdim) fp32 or NULL.  Formats, arguments, layouts
 * and validation otherwise as ssdq_state_update_corrected; other bits: SSDQ_ERROR_INVALID_VALUE.
 */
ssdq_status ssdq_state_update_scaled(int32_t state_format, void* state, float* state_scale, const int8_t* x,
                                     const float* x_scale, const int8_t* B, const float* B_scale, const int8_t* C,
                                     const float* C_scale, const float* dt, const float* A, const float* D,
                                     const float* y_corr, void* y, int32_t batch, int32_t nheads, int32_t headdim,
                                     int32_t dstate, int32_t ngroups, uint32_t scale_layout, hipStream_t stream);

/*
 * Front end of the SSD block, fused with the static quantizer: the causal convolution that the
 * pages keep in FP16 ahead of the SSD box (Quamba2 rebuttal Tables R6/R7; SSDi8 Table 16, Conv
 * column), read as Mamba-2's depthwise convolution of width 4 over the tokens of every channel
 * of the in-projection output, with a per-channel bias and SiLU; its binary16 output is
 * quantized as ssdq_quantize does, straight into the scan's layouts; and dt = softplus(dt_raw
 * + dt_bias), the positive step size the scan takes.
 *
 *   xbc    : (batch, seqlen, nheads*headdim + 2*ngroups*dstate) binary16, channels [x | B | C]
 *            (x channel h*headdim + p, then B channel g*dstate + n, then C likewise)
 *   conv_w : (channels, d_conv) float32; tap k multiplies token t - d_conv + 1 + k (zero before 0)
 *   conv_b : (channels) float32, or NULL for no bias
 *   a[b,t,c] = binary16( SiLU( conv_b[c] + sum_k conv_w[c,k] xbc[b, t-3+k, c] ) ),  SiLU(v) = v / (1 + e^-v)
 *   x      : (batch, seqlen, nheads, headdim) int8 = quantize(a[.., x channels], x_scale (nheads))
 *   B, C   : (batch, seqlen, ngroups, dstate) int8 = quantize(a[.., B / C channels], B_scale / C_scale (ngroups))
 *   dt_raw : (batch, seqlen, nheads) float32; dt_bias: (nheads) float32 or NULL
 *   dt     : (batch, seqlen, nheads) float32 = softplus(dt_raw + dt_bias) = max(v,0) + log1p(e^-|v|)
 * The codes are those of ssdq_quantize applied to a (bit-exact); a is formed in fp32, so an
 * element whose exact SiLU value lies within fp32 rounding of a binary16 midpoint may take the
 * other neighbour (and its code).  seqlen 0 is a no-op (after the size checks; pointers are not
 * looked at then).  Errors: NULL or misaligned (16-byte) pointers, non-positive sizes or nheads % ngroups != 0 -> SSDQ_ERROR_INVALID_VALUE; d_conv other
 * than 4, headdim or dstate not a multiple of 8, or batch * ceil(channels / 256) * ceil(seqlen / 16)
 * >= 2^31 ->
 * SSDQ_ERROR_UNSUPPORTED.  All pointers are device memory owned by the caller.
 */
ssdq_status ssdq_frontend(const void* xbc, const float* conv_w, const float* conv_b, int32_t d_conv,
                          const float* x_scale, const float* B_scale, const float* C_scale, const float* dt_raw,
                          const float* dt_bias, int8_t* x, int8_t* B, int8_t* C, float* dt, int32_t batch,
                          int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                          hipStream_t stream);

/*
 * ssdq_frontend for one decode token per sequence, with the convolution's history carried in a
 * conv state: the same output, codes and dt as ssdq_frontend gives for the last token of a
 * sequence whose three previous tokens are the state's rows (the cached convolution states of
 * the Quamba2 rebuttal, Table R7).
 *
 *   conv_state : (batch, 3, channels) binary16, read and written: rows are the inputs of tokens
 *                t-3, t-2, t-1 before the call and t-2, t-1, t after it (zeros at the start)
 *   xbc        : (batch, channels) binary16, token t
 *   x (batch, nheads, headdim), B and C (batch, ngroups, dstate) int8; dt_raw, dt (batch, nheads)
 * Every other argument, its layout and the validation are those of ssdq_frontend (d_conv 4;
 * headdim and dstate multiples of 8); all pointers are device memory owned by the caller.
 */
ssdq_status ssdq_frontend_step(void* conv_state, const void* xbc, const float* conv_w, const float* conv_b,
                               int32_t d_conv, const float* x_scale, const float* B_scale, const float* C_scale,
                               const float* dt_raw, const float* dt_bias, int8_t* x, int8_t* B, int8_t* C, float* dt,
                               int32_t batch, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSDQ_H_ */
