// Internal declarations shared by the HIP translation units of libssdq.
// Everything here is CDNA4 (gfx950, wave64) specific.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssdq.h"

namespace ssdq {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Division by an invariant divisor d for n < 2^31 (round-up multiplier):
// l = ceil(log2 d), m = ceil(2^(32+l) / d) - 2^32, n / d = (mulhi(n, m) + n) >> l.
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << (32 + l)) + d - 1) / d - (uint64_t(1) << 32);
  return FastDiv{d, uint32_t(m), l};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.l; }

// Shape of one prefill call after validation.
struct ScanShape {
  int32_t batch;
  int64_t seqlen;
  int32_t nheads, headdim, dstate, ngroups, chunk;
  int32_t nchunks;
  size_t acs_bytes;     // Acs region, rounded up to 256 bytes (the chunk-ordered dt region has the same size)
  size_t state_bytes;   // chunk-state region (fp32)
  size_t hprev_bytes;   // state entering each chunk as two int8 limbs, rounded up to 256 bytes
  size_t hscale_bytes;  // its per-row scales, rounded up to 256 bytes
  size_t total_bytes() const { return 2 * acs_bytes + state_bytes + hprev_bytes + hscale_bytes; }
};

struct ScanArgs {
  const int8_t* x;
  const float* x_scale;
  const int8_t* B;
  const float* B_scale;
  const int8_t* C;
  const float* C_scale;
  const float* dt;
  const float* A;
  const float* D;
  const float* ycorr;   // (nheads, headdim) fp32 output correction or nullptr
  const float* h0;
  _Float16* y;
  float* h_final;
  float* acs;         // workspace: (batch, nheads, nchunks, chunk)
  float* dtc;         // workspace: dt in the same (batch, nheads, nchunks, chunk) order, 0 past the end
  float* states;      // workspace: (batch, nchunks, nheads, headdim, dstate) fp32
  int8_t* hprev;      // workspace: (batch, nchunks, nheads, 2, headdim, dstate) int8 limbs
  float* hscale;      // workspace: (batch, nchunks, nheads, headdim)
  bool bc_per_state;  // B_scale and C_scale hold one scale per (group, state), not one per group
  bool x_per_channel; // x_scale holds one scale per (head, channel), not one per head
};

// Kernel launchers (one per translation unit).  They return hipGetLastError().
hipError_t launch_quantize_batch(const ssdq_quantize_job* jobs, int32_t count, hipStream_t stream);
hipError_t launch_quantize(const uint16_t* x, int8_t* q, const float* scale, int64_t rows, int32_t nscale,
                           int32_t inner, hipStream_t stream);
hipError_t launch_quantize_per_channel(const uint16_t* x, int8_t* q, const float* scale, int64_t rows,
                                      int32_t nscale, int32_t inner, hipStream_t stream);
hipError_t launch_chunk_state(const ScanShape& s, const ScanArgs& a, hipStream_t stream);
hipError_t launch_state_passing(const ScanShape& s, const ScanArgs& a, hipStream_t stream);
// Stages 0 and 1 in one kernel (one block per (batch, head), chunks in order); used when
// state_scan_fused(batch, nheads), i.e. when there are at least as many sequences as CUs.
bool state_scan_fused(int32_t batch, int32_t nheads);
// Waves per block of the folded state kernel for this shape (4 or 8), or 0 when it does not run.
int state_scan_waves(int32_t batch, int32_t nheads, bool bc_per_state);
hipError_t launch_state_scan(const ScanShape& s, const ScanArgs& a, hipStream_t stream);
hipError_t launch_chunk_output(const ScanShape& s, const ScanArgs& a, hipStream_t stream);
// front-end launch geometry: a lane owns kFeChannels channels and a strip of kFeTokens tokens;
// blocks of 64 lanes (the host checks the block count against the grid limit with these)
constexpr int kFeChannels = 4;
constexpr int kFeTokens = 16;
hipError_t launch_frontend(const uint16_t* xbc, const float* conv_w, const float* conv_b, const float* x_scale,
                           const float* B_scale, const float* C_scale, const float* dt_raw, const float* dt_bias,
                           int8_t* x, int8_t* B, int8_t* C, float* dt, int32_t batch, int64_t seqlen,
                           int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream);
hipError_t launch_frontend_step(uint16_t* conv_state, const uint16_t* xbc, const float* conv_w, const float* conv_b,
                                const float* x_scale, const float* B_scale, const float* C_scale,
                                const float* dt_raw, const float* dt_bias, int8_t* x, int8_t* B, int8_t* C,
                                float* dt, int32_t batch, int32_t nheads, int32_t headdim, int32_t dstate,
                                int32_t ngroups, hipStream_t stream);
// Decode launchers: `scales` is the scale layout (bit 0: B, C per (group, state); bit 1: x per
// (head, channel)).
hipError_t launch_state_update_i8(int8_t* state, float* state_scale, const int8_t* x, const float* x_scale,
                                  const int8_t* B, const float* B_scale, const int8_t* C, const float* C_scale,
                                  const float* dt, const float* A, const float* D, const float* ycorr, _Float16* y,
                                  int32_t batch, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                                  hipStream_t stream, int32_t scales = 0);
hipError_t launch_state_update_f16(uint16_t* state, const int8_t* x, const float* x_scale, const int8_t* B,
                                   const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                                   const float* A, const float* D, const float* ycorr, _Float16* y, int32_t batch,
                                   int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                                   hipStream_t stream, int32_t scales = 0);
hipError_t launch_state_update(float* state, const int8_t* x, const float* x_scale, const int8_t* B,
                               const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                               const float* A, const float* D, const float* ycorr, _Float16* y, int32_t batch,
                               int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream,
                               int32_t scales = 0);

// ---------------------------------------------------------------------------------------------
// device helpers

// Raw buffer loads (gfx9 buffer resource: base address, size in bytes, dword 3 = 0x00020000).
// A load whose byte offset is at or past the size returns zeros without touching memory: the
// kernels use this to zero-pad ragged chunk tails and padded tiles with no clamps or selects.
// Sizes and offsets stay below 2^31 (the host bounds one chunk of any operand below that).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOutOfRange = 0x80000000u;   // a byte offset that is never in range
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ v4u buf_load16(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ float buf_loadf(Rsrc r, uint32_t off) { return __uint_as_float(buf_load4(r, off)); }
// 16 bytes per lane from a buffer straight into LDS: a wave's lanes fill 16 * 64 consecutive
// bytes starting at the wave-uniform `lds`, in lane order (no registers involved).  Completion
// is tracked by vmcnt.  (Called through this plain function: used directly inside a kernel
// template, the builtin keeps the host pass from emitting the kernel's launch stub.)
__device__ __forceinline__ void buf_load16_lds(Rsrc r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

// Blocks are dispatched round-robin over the 8 XCDs (block i -> XCD i % 8).  Remap the
// linear block index so that consecutive *logical* tiles land on the same XCD and share
// its L2 (neighbouring heads read the same 128-byte lines of x and the same B/C rows).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int per = nblocks / kXcd;            // full rounds
  const int full = per * kXcd;
  if (bid >= full) return bid;               // tail blocks keep their index
  return (bid % kXcd) * per + bid / kXcd;
}

// Maximum over each group of LPR consecutive lanes (LPR a power of two up to the wave),
// left in every lane of the group, entirely in registers: DPP lane moves within a 16-lane row
// and gfx950's 16- and 32-lane half swaps across rows (no LDS round trip, so no wait that
// would also drain outstanding loads).  For values >= 0: a lane masked off reads as 0.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(moved));
}
template <int LPR>
__device__ __forceinline__ float group_max(float m) {
  if constexpr (LPR >= 2) m = dpp_max<0xB1>(m);    // quad_perm [1, 0, 3, 2]: lane ^ 1
  if constexpr (LPR >= 4) m = dpp_max<0x4E>(m);    // quad_perm [2, 3, 0, 1]: lane ^ 2
  if constexpr (LPR >= 8) m = dpp_max<0x141>(m);   // row_half_mirror: the other quad of the 8
  if constexpr (LPR >= 16) m = dpp_max<0x140>(m);  // row_mirror: the other half of the row
  if constexpr (LPR >= 32) {                       // rows 0 and 1, rows 2 and 3
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (LPR >= 64) {                       // the two halves of the wave
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return m;
}
__device__ __forceinline__ float wave_max(float v) { return group_max<kWave>(v); }

// Sum over each group of LPR consecutive lanes (LPR a power of two up to 16), left in every
// lane of the group: the same DPP pairings as group_max, each joining two disjoint sub-groups.
template <int CTRL>
__device__ __forceinline__ float dpp_sum(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return v + __int_as_float(moved);
}
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LPR >= 1 && LPR <= 16, "groups within one 16-lane row");
  if constexpr (LPR >= 2) v = dpp_sum<0xB1>(v);
  if constexpr (LPR >= 4) v = dpp_sum<0x4E>(v);
  if constexpr (LPR >= 8) v = dpp_sum<0x141>(v);
  if constexpr (LPR >= 16) v = dpp_sum<0x140>(v);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers: a Hillis-Steele scan inside
// each 16-lane row with DPP right shifts (lanes shifted in from outside the row read 0), then
// the row totals carried across rows with DPP row broadcasts.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
  return v + __int_as_float(moved);
}
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  v = dpp_add<0x111, 0xF>(v);   // row_shr:1
  v = dpp_add<0x112, 0xF>(v);   // row_shr:2
  v = dpp_add<0x114, 0xF>(v);   // row_shr:4
  v = dpp_add<0x118, 0xF>(v);   // row_shr:8   -> inclusive sums within each row
  v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 -> rows 1 and 3 add lane 15 of the row before
  v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 -> rows 2 and 3 add lane 31
  return v;
}
__device__ __forceinline__ float lane_broadcast(float v, int src_lane) {   // src_lane uniform
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_lane));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ceil(log2(v)) for finite v > 0 as an exponent e with v <= 2^e, from the fp32 bits
// (exact; no libm).  v == 0 gives -126.
__device__ __forceinline__ int ceil_log2_pos(float v) {
  if (!(v > 0.f)) return -126;
  const uint32_t bits = __float_as_uint(v);
  int e = int((bits >> 23) & 0xff) - 127;
  const uint32_t mant = bits & 0x7fffff;
  if (e == -127) {  // subnormal
    return -126;
  }
  return mant ? e + 1 : e;
}

// 2^e as a float for e in [-126, 127] (exact).
__device__ __forceinline__ float exp2i(int e) {
  e = e < -126 ? -126 : (e > 127 ? 127 : e);
  return __uint_as_float(uint32_t(e + 127) << 23);
}

}  // namespace ssdq
