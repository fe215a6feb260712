// C ABI of libssdq: host-side validation, workspace carving and the launch sequence.
// No HIP runtime call is made before every argument has been validated, so the error
// paths can be exercised on a machine without a GPU.
#include <stdint.h>

#include <mutex>

#include "ssdq_internal.h"

using namespace ssdq;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// Shape validation for the prefill scan; fills `s` on success.
ssdq_status check_scan_shape(int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                             int32_t ngroups, int32_t chunk, ScanShape* s) {
  if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 || chunk <= 0)
    return SSDQ_ERROR_INVALID_VALUE;
  if (nheads % ngroups != 0) return SSDQ_ERROR_INVALID_VALUE;
  if (headdim % 16 != 0 || headdim > 64) return SSDQ_ERROR_UNSUPPORTED;
  if (dstate % 16 != 0 || dstate > 128) return SSDQ_ERROR_UNSUPPORTED;
  if (chunk != 64 && chunk != 128 && chunk != 256) return SSDQ_ERROR_UNSUPPORTED;
  const int64_t nchunks = (seqlen + chunk - 1) / chunk;
  // grid sizes and 32-bit block indices
  if (int64_t(batch) * nchunks * nheads > (int64_t(1) << 30)) return SSDQ_ERROR_UNSUPPORTED;
  if (nchunks > 65535) return SSDQ_ERROR_UNSUPPORTED;
  // (token, head) rows of x, y and dt are indexed in 32 bits
  if (int64_t(batch) * seqlen * nheads >= (int64_t(1) << 31)) return SSDQ_ERROR_UNSUPPORTED;
  // the kernels address one chunk of x, y, B, C (chunk rows of nheads*headdim or
  // ngroups*dstate elements) with 32-bit offsets from a per-chunk base, and 2^31 is the offset
  // that is never in range: a chunk of fp16 y must stay below it
  if (int64_t(nheads) * headdim * chunk >= (int64_t(1) << 30)) return SSDQ_ERROR_UNSUPPORTED;
  if (int64_t(ngroups) * dstate * chunk >= (int64_t(1) << 31)) return SSDQ_ERROR_UNSUPPORTED;
  s->batch = batch;
  s->seqlen = seqlen;
  s->nheads = nheads;
  s->headdim = headdim;
  s->dstate = dstate;
  s->ngroups = ngroups;
  s->chunk = chunk;
  s->nchunks = int32_t(nchunks);
  s->acs_bytes = round256(sizeof(float) * size_t(batch) * nheads * nchunks * chunk);
  s->state_bytes = sizeof(float) * size_t(batch) * nchunks * nheads * headdim * dstate;
  s->hprev_bytes = round256(2 * size_t(batch) * nchunks * nheads * headdim * dstate);
  s->hscale_bytes = round256(sizeof(float) * size_t(batch) * nchunks * nheads * headdim);
  return SSDQ_SUCCESS;
}

// Workspace regions in order, each at a 256-byte boundary: Acs, the chunk-ordered dt, the fp32
// chunk states (left out of the compact layout when the folded state kernel runs), the
// carried-state limbs and their row scales.
void carve(const ScanShape& s, char* base, bool with_states, ScanArgs* a) {
  size_t off = 0;
  a->acs = reinterpret_cast<float*>(base + off);
  off += s.acs_bytes;
  a->dtc = reinterpret_cast<float*>(base + off);
  off += s.acs_bytes;
  a->states = reinterpret_cast<float*>(base + off);   // not read or written by the folded plan
  if (with_states) off += round256(s.state_bytes);
  a->hprev = reinterpret_cast<int8_t*>(base + off);
  off += s.hprev_bytes;
  a->hscale = reinterpret_cast<float*>(base + off);
}

ssdq_status check_scan_args(int32_t stage, const int8_t* x, const float* x_scale, const int8_t* B,
                            const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                            const float* A, const float* D, const float* h0, void* y, float* h_final,
                            int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                            int32_t ngroups, int32_t chunk, void* workspace, size_t workspace_bytes,
                            ScanShape* s, ScanArgs* a) {
  (void)stage;
  if (!ok_ptr(x) || !ok_ptr(x_scale) || !ok_ptr(B) || !ok_ptr(B_scale) || !ok_ptr(C) || !ok_ptr(C_scale) ||
      !ok_ptr(dt) || !ok_ptr(A) || !ok_ptr(y) || !ok_ptr(workspace) || !ok_opt(D) || !ok_opt(h0) ||
      !ok_opt(h_final))
    return SSDQ_ERROR_INVALID_VALUE;
  const ssdq_status st = check_scan_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, s);
  if (st != SSDQ_SUCCESS) return st;
  if (workspace_bytes < s->total_bytes()) return SSDQ_ERROR_WORKSPACE_TOO_SMALL;
  a->x = x;
  a->x_scale = x_scale;
  a->B = B;
  a->B_scale = B_scale;
  a->C = C;
  a->C_scale = C_scale;
  a->dt = dt;
  a->A = A;
  a->D = D;
  a->ycorr = nullptr;
  a->bc_per_state = false;
  a->x_per_channel = false;
  a->h0 = h0;
  a->y = static_cast<_Float16*>(y);
  a->h_final = h_final;
  carve(*s, static_cast<char*>(workspace), true, a);
  return SSDQ_SUCCESS;
}

// With at least one (batch, head) sequence per CU, stage 0 carries the state across chunks
// itself (chunk states never reach memory) and stage 1 has nothing left to do.
ssdq_status run_stage(int32_t stage, const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  const bool fused = state_scan_fused(s.batch, s.nheads);
  hipError_t e = hipSuccess;
  switch (stage) {
    case 0: e = fused ? launch_state_scan(s, a, stream) : launch_chunk_state(s, a, stream); break;
    case 1: e = fused ? hipSuccess : launch_state_passing(s, a, stream); break;
    case 2: e = launch_chunk_output(s, a, stream); break;
    default: return SSDQ_ERROR_INVALID_VALUE;
  }
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}

// Scratch of the allocation-free prefill entry point: one file-scope device array, which every
// GPU the library runs on holds for the life of the process.  Host code never uses the array's
// name as an address (on the host it only names the symbol): the device address is looked up once
// per device with hipGetSymbolAddress, with that device current, and kept here.
__device__ __attribute__((aligned(256))) uint8_t scratch[SSDQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call on that device), or nullptr
// if the runtime cannot provide it.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// The compact scratch layout of one prefill call: Acs, the chunk-ordered dt, the fp32 chunk
// states only when the three-kernel plan runs (fused = false), the carried-state limbs and their
// row scales, each region starting at a 256-byte boundary.
size_t noalloc_bytes(const ScanShape& s, bool fused) {
  return 2 * s.acs_bytes + (fused ? 0 : round256(s.state_bytes)) + s.hprev_bytes + s.hscale_bytes;
}

}  // namespace

extern "C" {

const char* ssdq_status_string(ssdq_status status) {
  switch (status) {
    case SSDQ_SUCCESS: return "SSDQ_SUCCESS";
    case SSDQ_ERROR_INVALID_VALUE: return "SSDQ_ERROR_INVALID_VALUE";
    case SSDQ_ERROR_UNSUPPORTED: return "SSDQ_ERROR_UNSUPPORTED";
    case SSDQ_ERROR_WORKSPACE_TOO_SMALL: return "SSDQ_ERROR_WORKSPACE_TOO_SMALL";
    case SSDQ_ERROR_LAUNCH: return "SSDQ_ERROR_LAUNCH";
    case SSDQ_ERROR_SCRATCH_LIMIT: return "SSDQ_ERROR_SCRATCH_LIMIT";
  }
  return "SSDQ_UNKNOWN_STATUS";
}

ssdq_status ssdq_quantize(const void* x_f16, int8_t* q, const float* scale, int64_t rows, int32_t nscale,
                          int32_t inner, hipStream_t stream) {
  if (rows < 0 || nscale <= 0 || inner <= 0) return SSDQ_ERROR_INVALID_VALUE;
  if (rows == 0) return SSDQ_SUCCESS;
  if (!ok_ptr(x_f16) || !ok_ptr(q) || !ok_ptr(scale)) return SSDQ_ERROR_INVALID_VALUE;
  const hipError_t e =
      launch_quantize(static_cast<const uint16_t*>(x_f16), q, scale, rows, nscale, inner, stream);
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}

ssdq_status ssdq_quantize_per_channel(const void* x_f16, int8_t* q, const float* scale, int64_t rows, int32_t nscale,
                                      int32_t inner, hipStream_t stream) {
  if (rows < 0 || nscale <= 0 || inner <= 0) return SSDQ_ERROR_INVALID_VALUE;
  if (rows == 0) return SSDQ_SUCCESS;
  if (!ok_ptr(x_f16) || !ok_ptr(q) || !ok_ptr(scale)) return SSDQ_ERROR_INVALID_VALUE;
  const hipError_t e =
      launch_quantize_per_channel(static_cast<const uint16_t*>(x_f16), q, scale, rows, nscale, inner, stream);
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}

ssdq_status ssdq_quantize_batch(const ssdq_quantize_job* jobs, int32_t count, hipStream_t stream) {
  if (jobs == nullptr || count < 1 || count > SSDQ_QUANTIZE_MAX_JOBS) return SSDQ_ERROR_INVALID_VALUE;
  bool work = false;
  for (int32_t k = 0; k < count; ++k) {
    const ssdq_quantize_job& j = jobs[k];
    if (j.rows < 0 || j.nscale <= 0 || j.inner <= 0) return SSDQ_ERROR_INVALID_VALUE;
    if (j.rows > 0 && (!ok_ptr(j.x_f16) || !ok_ptr(j.q) || !ok_ptr(j.scale))) return SSDQ_ERROR_INVALID_VALUE;
    work = work || j.rows > 0;
  }
  if (!work) return SSDQ_SUCCESS;
  const hipError_t e = launch_quantize_batch(jobs, count, stream);
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}

size_t ssdq_chunk_scan_workspace_size(int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim,
                                      int32_t dstate, int32_t chunk) {
  ScanShape s;
  // ngroups does not change the workspace; 1 always divides nheads
  if (check_scan_shape(batch, seqlen, nheads, headdim, dstate, 1, chunk, &s) != SSDQ_SUCCESS) return 0;
  return s.total_bytes();
}

int32_t ssdq_chunk_scan_state_fused(int32_t batch, int32_t nheads) {
  if (batch <= 0 || nheads <= 0) return 0;
  return state_scan_fused(batch, nheads) ? 1 : 0;
}

int32_t ssdq_chunk_scan_plan(int32_t batch, int32_t nheads, uint32_t scale_layout) {
  if (batch <= 0 || nheads <= 0) return -1;
  if (scale_layout & ~uint32_t(SSDQ_SCALES_BC_PER_STATE | SSDQ_SCALES_X_PER_CHANNEL)) return -1;
  return state_scan_waves(batch, nheads, (scale_layout & SSDQ_SCALES_BC_PER_STATE) != 0);
}

ssdq_status ssdq_chunk_scan_stage(int32_t stage, const int8_t* x, const float* x_scale, const int8_t* B,
                                  const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                                  const float* A, const float* D, const float* h0, void* y, float* h_final,
                                  int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                                  int32_t ngroups, int32_t chunk, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (stage < 0 || stage >= SSDQ_CHUNK_SCAN_STAGES) return SSDQ_ERROR_INVALID_VALUE;
  ScanShape s;
  ScanArgs a;
  const ssdq_status st = check_scan_args(stage, x, x_scale, B, B_scale, C, C_scale, dt, A, D, h0, y, h_final,
                                         batch, seqlen, nheads, headdim, dstate, ngroups, chunk, workspace,
                                         workspace_bytes, &s, &a);
  if (st != SSDQ_SUCCESS) return st;
  return run_stage(stage, s, a, stream);
}

ssdq_status ssdq_chunk_scan(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                            const int8_t* C, const float* C_scale, const float* dt, const float* A, const float* D,
                            const float* h0, void* y, float* h_final, int32_t batch, int64_t seqlen,
                            int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups, int32_t chunk,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ScanShape s;
  ScanArgs a;
  const ssdq_status st = check_scan_args(0, x, x_scale, B, B_scale, C, C_scale, dt, A, D, h0, y, h_final, batch,
                                         seqlen, nheads, headdim, dstate, ngroups, chunk, workspace,
                                         workspace_bytes, &s, &a);
  if (st != SSDQ_SUCCESS) return st;
  for (int32_t stage = 0; stage < SSDQ_CHUNK_SCAN_STAGES; ++stage) {
    const ssdq_status r = run_stage(stage, s, a, stream);
    if (r != SSDQ_SUCCESS) return r;
  }
  return SSDQ_SUCCESS;
}

ssdq_status ssdq_chunk_scan_corrected(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                                      const int8_t* C, const float* C_scale, const float* dt, const float* A,
                                      const float* D, const float* y_corr, const float* h0, void* y, float* h_final,
                                      int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                                      int32_t ngroups, int32_t chunk, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  if (!ok_ptr(y_corr)) return SSDQ_ERROR_INVALID_VALUE;
  ScanShape s;
  ScanArgs a;
  const ssdq_status st = check_scan_args(0, x, x_scale, B, B_scale, C, C_scale, dt, A, D, h0, y, h_final, batch,
                                         seqlen, nheads, headdim, dstate, ngroups, chunk, workspace,
                                         workspace_bytes, &s, &a);
  if (st != SSDQ_SUCCESS) return st;
  a.ycorr = y_corr;
  for (int32_t stage = 0; stage < SSDQ_CHUNK_SCAN_STAGES; ++stage) {
    const ssdq_status r = run_stage(stage, s, a, stream);
    if (r != SSDQ_SUCCESS) return r;
  }
  return SSDQ_SUCCESS;
}

ssdq_status ssdq_chunk_scan_per_state(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                                      const int8_t* C, const float* C_scale, const float* dt, const float* A,
                                      const float* D, const float* y_corr, const float* h0, void* y, float* h_final,
                                      int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                                      int32_t ngroups, int32_t chunk, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  if (!ok_opt(y_corr)) return SSDQ_ERROR_INVALID_VALUE;
  ScanShape s;
  ScanArgs a;
  const ssdq_status st = check_scan_args(0, x, x_scale, B, B_scale, C, C_scale, dt, A, D, h0, y, h_final, batch,
                                         seqlen, nheads, headdim, dstate, ngroups, chunk, workspace,
                                         workspace_bytes, &s, &a);
  if (st != SSDQ_SUCCESS) return st;
  a.ycorr = y_corr;
  a.bc_per_state = true;
  for (int32_t stage = 0; stage < SSDQ_CHUNK_SCAN_STAGES; ++stage) {
    const ssdq_status r = run_stage(stage, s, a, stream);
    if (r != SSDQ_SUCCESS) return r;
  }
  return SSDQ_SUCCESS;
}

ssdq_status ssdq_chunk_scan_scaled(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                                   const int8_t* C, const float* C_scale, const float* dt, const float* A,
                                   const float* D, const float* y_corr, const float* h0, void* y, float* h_final,
                                   int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                                   int32_t ngroups, int32_t chunk, uint32_t scale_layout, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  if (!ok_opt(y_corr)) return SSDQ_ERROR_INVALID_VALUE;
  if (scale_layout & ~uint32_t(SSDQ_SCALES_BC_PER_STATE | SSDQ_SCALES_X_PER_CHANNEL)) return SSDQ_ERROR_INVALID_VALUE;
  ScanShape s;
  ScanArgs a;
  const ssdq_status st = check_scan_args(0, x, x_scale, B, B_scale, C, C_scale, dt, A, D, h0, y, h_final, batch,
                                         seqlen, nheads, headdim, dstate, ngroups, chunk, workspace,
                                         workspace_bytes, &s, &a);
  if (st != SSDQ_SUCCESS) return st;
  a.ycorr = y_corr;
  a.bc_per_state = (scale_layout & SSDQ_SCALES_BC_PER_STATE) != 0;
  a.x_per_channel = (scale_layout & SSDQ_SCALES_X_PER_CHANNEL) != 0;
  for (int32_t stage = 0; stage < SSDQ_CHUNK_SCAN_STAGES; ++stage) {
    const ssdq_status r = run_stage(stage, s, a, stream);
    if (r != SSDQ_SUCCESS) return r;
  }
  return SSDQ_SUCCESS;
}

size_t ssdq_chunk_scan_noalloc_scratch_size(int32_t batch, int64_t seqlen, int32_t nheads, int32_t headdim,
                                            int32_t dstate, int32_t chunk) {
  ScanShape s;
  if (check_scan_shape(batch, seqlen, nheads, headdim, dstate, 1, chunk, &s) != SSDQ_SUCCESS) return 0;
  return noalloc_bytes(s, state_scan_fused(batch, nheads));
}

ssdq_status ssdq_chunk_scan_noalloc(const int8_t* x, const float* x_scale, const int8_t* B, const float* B_scale,
                                    const int8_t* C, const float* C_scale, const float* dt, const float* A,
                                    const float* D, const float* h0, void* y, float* h_final, int32_t batch,
                                    int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
                                    int32_t ngroups, int32_t chunk, hipStream_t stream) {
  // every check the workspace entry point makes, with a stand-in workspace pointer that is only
  // tested for alignment (the scratch regions are carved below)
  ScanShape s;
  ScanArgs a;
  static const uint8_t kAlignedStandIn alignas(256) = 0;
  ssdq_status st = check_scan_args(0, x, x_scale, B, B_scale, C, C_scale, dt, A, D, h0, y, h_final, batch, seqlen,
                                   nheads, headdim, dstate, ngroups, chunk,
                                   const_cast<uint8_t*>(&kAlignedStandIn), SIZE_MAX, &s, &a);
  if (st != SSDQ_SUCCESS) return st;
  const bool fused = state_scan_fused(batch, nheads);
  if (noalloc_bytes(s, fused) > size_t(SSDQ_NOALLOC_SCRATCH_BYTES)) return SSDQ_ERROR_SCRATCH_LIMIT;
  char* base = static_cast<char*>(device_scratch());
  if (base == nullptr) return SSDQ_ERROR_LAUNCH;
  carve(s, base, !fused, &a);
  for (int32_t stage = 0; stage < SSDQ_CHUNK_SCAN_STAGES; ++stage) {
    const ssdq_status r = run_stage(stage, s, a, stream);
    if (r != SSDQ_SUCCESS) return r;
  }
  return SSDQ_SUCCESS;
}

namespace {
// Arguments of a decode step (fp32 or binary16 state alike).
ssdq_status check_decode(const void* state, const int8_t* x, const float* x_scale, const int8_t* B,
                         const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                         const float* A, const float* D, void* y, int32_t batch, int32_t nheads, int32_t headdim,
                         int32_t dstate, int32_t ngroups) {
  if (!ok_ptr(state) || !ok_ptr(x) || !ok_ptr(x_scale) || !ok_ptr(B) || !ok_ptr(B_scale) || !ok_ptr(C) ||
      !ok_ptr(C_scale) || !ok_ptr(dt) || !ok_ptr(A) || !ok_ptr(y) || !ok_opt(D))
    return SSDQ_ERROR_INVALID_VALUE;
  if (batch <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0) return SSDQ_ERROR_INVALID_VALUE;
  if (nheads % ngroups != 0) return SSDQ_ERROR_INVALID_VALUE;
  if ((dstate != 64 && dstate != 128) || headdim > 64) return SSDQ_ERROR_UNSUPPORTED;
  if (int64_t(batch) * nheads > (int64_t(1) << 30)) return SSDQ_ERROR_UNSUPPORTED;
  return SSDQ_SUCCESS;
}
}  // namespace

ssdq_status ssdq_state_update(float* state, const int8_t* x, const float* x_scale, const int8_t* B,
                              const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                              const float* A, const float* D, void* y, int32_t batch, int32_t nheads,
                              int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream) {
  const ssdq_status st =
      check_decode(state, x, x_scale, B, B_scale, C, C_scale, dt, A, D, y, batch, nheads, headdim, dstate, ngroups);
  if (st != SSDQ_SUCCESS) return st;
  const hipError_t e = launch_state_update(state, x, x_scale, B, B_scale, C, C_scale, dt, A, D, nullptr,
                                           static_cast<_Float16*>(y), batch, nheads, headdim, dstate, ngroups,
                                           stream);
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}

ssdq_status ssdq_state_update_f16(void* state, const int8_t* x, const float* x_scale, const int8_t* B,
                                  const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                                  const float* A, const float* D, void* y, int32_t batch, int32_t nheads,
                                  int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream) {
  const ssdq_status st =
      check_decode(state, x, x_scale, B, B_scale, C, C_scale, dt, A, D, y, batch, nheads, headdim, dstate, ngroups);
  if (st != SSDQ_SUCCESS) return st;
  const hipError_t e = launch_state_update_f16(static_cast<uint16_t*>(state), x, x_scale, B, B_scale, C, C_scale,
                                               dt, A, D, nullptr, static_cast<_Float16*>(y), batch, nheads, headdim,
                                               dstate, ngroups, stream);
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}

ssdq_status ssdq_state_update_i8(int8_t* state, float* state_scale, const int8_t* x, const float* x_scale,
                                 const int8_t* B, const float* B_scale, const int8_t* C, const float* C_scale,
                                 const float* dt, const float* A, const float* D, void* y, int32_t batch,
                                 int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                                 hipStream_t stream) {
  if (!ok_ptr(state_scale)) return SSDQ_ERROR_INVALID_VALUE;
  const ssdq_status st =
      check_decode(state, x, x_scale, B, B_scale, C, C_scale, dt, A, D, y, batch, nheads, headdim, dstate, ngroups);
  if (st != SSDQ_SUCCESS) return st;
  const hipError_t e = launch_state_update_i8(state, state_scale, x, x_scale, B, B_scale, C, C_scale, dt, A, D,
                                              nullptr, static_cast<_Float16*>(y), batch, nheads, headdim, dstate,
                                              ngroups, stream);
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}

namespace {
ssdq_status decode_any(int32_t state_format, void* state, float* state_scale, const int8_t* x, const float* x_scale,
                       const int8_t* B, const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                       const float* A, const float* D, const float* y_corr, void* y, int32_t batch, int32_t nheads,
                       int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream, int32_t scales);
}  // namespace

ssdq_status ssdq_state_update_per_state(int32_t state_format, void* state, float* state_scale, const int8_t* x,
                                        const float* x_scale, const int8_t* B, const float* B_scale, const int8_t* C,
                                        const float* C_scale, const float* dt, const float* A, const float* D,
                                        const float* y_corr, void* y, int32_t batch, int32_t nheads, int32_t headdim,
                                        int32_t dstate, int32_t ngroups, hipStream_t stream) {
  if (!ok_opt(y_corr)) return SSDQ_ERROR_INVALID_VALUE;
  return decode_any(state_format, state, state_scale, x, x_scale, B, B_scale, C, C_scale, dt, A, D, y_corr, y, batch,
                    nheads, headdim, dstate, ngroups, stream, SSDQ_SCALES_BC_PER_STATE);
}

ssdq_status ssdq_state_update_scaled(int32_t state_format, void* state, float* state_scale, const int8_t* x,
                                     const float* x_scale, const int8_t* B, const float* B_scale, const int8_t* C,
                                     const float* C_scale, const float* dt, const float* A, const float* D,
                                     const float* y_corr, void* y, int32_t batch, int32_t nheads, int32_t headdim,
                                     int32_t dstate, int32_t ngroups, uint32_t scale_layout, hipStream_t stream) {
  if (!ok_opt(y_corr)) return SSDQ_ERROR_INVALID_VALUE;
  if (scale_layout & ~uint32_t(SSDQ_SCALES_BC_PER_STATE | SSDQ_SCALES_X_PER_CHANNEL)) return SSDQ_ERROR_INVALID_VALUE;
  return decode_any(state_format, state, state_scale, x, x_scale, B, B_scale, C, C_scale, dt, A, D, y_corr, y, batch,
                    nheads, headdim, dstate, ngroups, stream, int32_t(scale_layout));
}

ssdq_status ssdq_state_update_corrected(int32_t state_format, void* state, float* state_scale, const int8_t* x,
                                        const float* x_scale, const int8_t* B, const float* B_scale, const int8_t* C,
                                        const float* C_scale, const float* dt, const float* A, const float* D,
                                        const float* y_corr, void* y, int32_t batch, int32_t nheads, int32_t headdim,
                                        int32_t dstate, int32_t ngroups, hipStream_t stream) {
  if (!ok_ptr(y_corr)) return SSDQ_ERROR_INVALID_VALUE;
  return decode_any(state_format, state, state_scale, x, x_scale, B, B_scale, C, C_scale, dt, A, D, y_corr, y, batch,
                    nheads, headdim, dstate, ngroups, stream, 0);
}

}  // extern "C"

namespace {
ssdq_status decode_any(int32_t state_format, void* state, float* state_scale, const int8_t* x, const float* x_scale,
                       const int8_t* B, const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                       const float* A, const float* D, const float* y_corr, void* y, int32_t batch, int32_t nheads,
                       int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream, int32_t scales) {
  if (state_format != SSDQ_STATE_F32 && state_format != SSDQ_STATE_F16 && state_format != SSDQ_STATE_I8)
    return SSDQ_ERROR_INVALID_VALUE;
  if (state_format == SSDQ_STATE_I8 && !ok_ptr(state_scale)) return SSDQ_ERROR_INVALID_VALUE;
  const ssdq_status st =
      check_decode(state, x, x_scale, B, B_scale, C, C_scale, dt, A, D, y, batch, nheads, headdim, dstate, ngroups);
  if (st != SSDQ_SUCCESS) return st;
  _Float16* yo = static_cast<_Float16*>(y);
  hipError_t e;
  if (state_format == SSDQ_STATE_F32)
    e = launch_state_update(static_cast<float*>(state), x, x_scale, B, B_scale, C, C_scale, dt, A, D, y_corr, yo,
                            batch, nheads, headdim, dstate, ngroups, stream, scales);
  else if (state_format == SSDQ_STATE_F16)
    e = launch_state_update_f16(static_cast<uint16_t*>(state), x, x_scale, B, B_scale, C, C_scale, dt, A, D, y_corr,
                                yo, batch, nheads, headdim, dstate, ngroups, stream, scales);
  else
    e = launch_state_update_i8(static_cast<int8_t*>(state), state_scale, x, x_scale, B, B_scale, C, C_scale, dt, A, D,
                               y_corr, yo, batch, nheads, headdim, dstate, ngroups, stream, scales);
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}
}  // namespace

extern "C" {

ssdq_status ssdq_frontend(const void* xbc, const float* conv_w, const float* conv_b, int32_t d_conv,
                          const float* x_scale, const float* B_scale, const float* C_scale, const float* dt_raw,
                          const float* dt_bias, int8_t* x, int8_t* B, int8_t* C, float* dt, int32_t batch,
                          int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                          hipStream_t stream) {
  if (batch <= 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
      nheads % ngroups != 0)
    return SSDQ_ERROR_INVALID_VALUE;
  if (d_conv != 4 || headdim % 8 != 0 || dstate % 8 != 0) return SSDQ_ERROR_UNSUPPORTED;
  const int64_t channels = int64_t(nheads) * headdim + 2 * int64_t(ngroups) * dstate;
  const int64_t blocks =   // front-end launch
      int64_t(batch) * ((channels / kFeChannels + 63) / 64) * ((seqlen + kFeTokens - 1) / kFeTokens);
  if (channels >= (int64_t(1) << 31) || blocks >= (int64_t(1) << 31)) return SSDQ_ERROR_UNSUPPORTED;
  if (seqlen == 0) return SSDQ_SUCCESS;   // nothing to read or write (empty tensors may have no address)
  if (!ok_ptr(xbc) || !ok_ptr(conv_w) || !ok_opt(conv_b) || !ok_ptr(x_scale) || !ok_ptr(B_scale) ||
      !ok_ptr(C_scale) || !ok_ptr(dt_raw) || !ok_opt(dt_bias) || !ok_ptr(x) || !ok_ptr(B) || !ok_ptr(C) ||
      !ok_ptr(dt))
    return SSDQ_ERROR_INVALID_VALUE;
  const hipError_t e = launch_frontend(static_cast<const uint16_t*>(xbc), conv_w, conv_b, x_scale, B_scale, C_scale,
                                       dt_raw, dt_bias, x, B, C, dt, batch, seqlen, nheads, headdim, dstate, ngroups,
                                       stream);
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}

ssdq_status ssdq_frontend_step(void* conv_state, const void* xbc, const float* conv_w, const float* conv_b,
                               int32_t d_conv, const float* x_scale, const float* B_scale, const float* C_scale,
                               const float* dt_raw, const float* dt_bias, int8_t* x, int8_t* B, int8_t* C, float* dt,
                               int32_t batch, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                               hipStream_t stream) {
  if (!ok_ptr(conv_state) || !ok_ptr(xbc) || !ok_ptr(conv_w) || !ok_opt(conv_b) || !ok_ptr(x_scale) ||
      !ok_ptr(B_scale) || !ok_ptr(C_scale) || !ok_ptr(dt_raw) || !ok_opt(dt_bias) || !ok_ptr(x) || !ok_ptr(B) ||
      !ok_ptr(C) || !ok_ptr(dt))
    return SSDQ_ERROR_INVALID_VALUE;
  if (batch <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 || nheads % ngroups != 0)
    return SSDQ_ERROR_INVALID_VALUE;
  if (d_conv != 4 || headdim % 8 != 0 || dstate % 8 != 0) return SSDQ_ERROR_UNSUPPORTED;
  const int64_t channels = int64_t(nheads) * headdim + 2 * int64_t(ngroups) * dstate;
  if (channels >= (int64_t(1) << 31) || int64_t(batch) * channels * 3 >= (int64_t(1) << 40))
    return SSDQ_ERROR_UNSUPPORTED;
  const hipError_t e = launch_frontend_step(static_cast<uint16_t*>(conv_state), static_cast<const uint16_t*>(xbc),
                                            conv_w, conv_b, x_scale, B_scale, C_scale, dt_raw, dt_bias, x, B, C, dt,
                                            batch, nheads, headdim, dstate, ngroups, stream);
  return e == hipSuccess ? SSDQ_SUCCESS : SSDQ_ERROR_LAUNCH;
}

}  // extern "C"
