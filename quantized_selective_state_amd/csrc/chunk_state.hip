// Stage 0 of the chunked SSD scan, one block (4 waves) per (batch, chunk, head), compiled per
// chunk size:
//
//  (a) chunk cumsum: Acs[j] = sum_{i <= j} dt_i A_h inside the chunk (tokens past the end
//      of the sequence add 0), written to the workspace for the later stages, and dt itself in
//      the same chunk order (one contiguous row per chunk and head for the output stage, where
//      the token-major dt would cost a separate cache line per token);
//  (b) chunk state: the state the chunk contributes on its own,
//
//        S_c[p, n] = sum_j w_j xhat[j, p] Bhat[j, n],   w_j = exp(Acs_last - Acs_j) dt_j
//
//      (w_j is SSDi8's LUT_state, Figure 3a), computed the way SSDi8 reformulates it
//      (abstract; Figure 3a): the element-wise X_scaled[j, p] = w_j q_x[j, p] first, then a
//      plain product with the INT8 codes of B on the INT8 matrix cores.
//
// One INT8 copy of X_scaled is too coarse for a 1e-4 state bound, so X_scaled is carried
// as three INT8 limbs (the multi-component idea of the Multi-Scale Dequant abstract):
// with 2^e >= max_j w_j and t = X_scaled 2^-e (|t| <= 127), the integer
// V = floor(65536 t + 32896) has the base-256 digits  V = l1 65536 + (l2+128) 256 + (l3+128),
// so t = l1 + l2/256 + l3/65536 to within 2^-16, with l1, l2, l3 signed bytes.  V is built
// in integer arithmetic, one 24-bit multiply-add per element: W = 256 V (to within 256) =
// (q + 128) OM_j + CB_j with OM_j = round(w_j 2^(24-e)) and CB_j = 256 * 32896 - 128 OM_j,
// so the limbs are bytes 3, 2, 1 of W, and a 4x4 byte transpose of four tokens' W yields the
// MFMA operand words directly.  Each limb goes through v_mfma_i32_16x16x64_i8 with exact
// int32 sums (|sum| <= Q 128 127 < 2^23) and an fp32 epilogue recombines them.
//
// Both operands contract over tokens, the slow axis in memory.  x and B are copied into LDS
// in their natural token-major layout (16-byte pieces, XOR-swizzled per row), and the MFMA
// operands are read with gfx950's transposing LDS read ds_read_b64_tr_b8: within a group of
// 16 lanes, lane i receives byte (i % 8) of the 8-byte chunks addressed by lanes 2k + i / 8,
// k = 0..7.  With lane 2k + h of a group addressing token row j0 + k at columns c0 + 8 h,
// lane i gets the 8 tokens j0..j0+7 of column c0 + i, so two reads give a lane its 16
// K-consecutive bytes with no byte transposes in registers.  Each wave owns one 16-channel
// tile of S across all states and tokens, so every limb is built exactly once, in registers,
// right before its MFMAs.
#include <type_traits>

#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxP = 64;
constexpr int kMaxN = 128;
constexpr float kLog2e = 1.4426950408889634f;

// LDS layouts (byte offsets), token-major with the 16-byte chunks of each row XOR-swizzled so
// that both the 16-byte copies and the transposing reads are free of bank conflicts:
//   x codes [Q][64]:  chunk c of row j at c ^ ((j >> 2) & 3)
//   B codes [Q][128]: chunk c of row j at c ^ ((j >> 1) & 7)
__device__ __forceinline__ int xpos(int j, int byte) {
  return j * kMaxP + ((((byte >> 4) ^ ((j >> 2) & 3)) << 4) | (byte & 15));
}
__device__ __forceinline__ int bpos(int j, int byte) {
  return j * kMaxN + ((((byte >> 4) ^ ((j >> 1) & 7)) << 4) | (byte & 15));
}

// a * b + c for a, b < 2^24 (one v_mad_u32_u24), modulo 2^32
__device__ __forceinline__ uint32_t mad24(uint32_t a, uint32_t b, uint32_t c) { return __umul24(a, b) + c; }
// a * b + c for signed 24-bit a, b (one v_mad_i32_i24), |a b + c| < 2^31
__device__ __forceinline__ int32_t mad24s(int32_t a, int32_t b, int32_t c) { return __mul24(a, b) + c; }
// byte k of x, sign-extended (one v_bfe_i32)
__device__ __forceinline__ int32_t sbyte(uint32_t x, int k) { return __builtin_amdgcn_sbfe(int32_t(x), 8 * k, 8); }

// 4x4 byte transpose: out[i] byte r = in[r] byte i.
__device__ __forceinline__ void transpose4x4(const uint32_t in[4], uint32_t out[4]) {
  const uint32_t t01lo = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
  const uint32_t t01hi = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
  const uint32_t t23lo = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t t23hi = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t23lo, t01lo, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t23lo, t01lo, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t23hi, t01hi, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t23hi, t01hi, 0x07060302u);
}

__device__ __forceinline__ v2u tr8(const uint8_t* lds_byte) {
  return __builtin_bit_cast(v2u, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                     (__attribute__((address_space(3))) v2i*)(lds_byte)));
}

// The x and B codes of the chunk as 16-byte pieces (x: 4 per token row, B: 8), loaded at kernel
// entry and copied to LDS after the cumsum.  Loads go through a buffer whose size ends at the
// chunk's last valid row, so rows past the sequence end read as zeros; pieces past P or N use
// an out-of-range offset and read as zeros too.
template <int Q>
struct Staged {
  static constexpr int kX = Q * (kMaxP / 16) / kThreads;
  static constexpr int kB = Q * (kMaxN / 16) / kThreads;
  v4u x[kX];
  v4u b[kB];
};

// 3 waves per SIMD (<= 168 VGPRs): three blocks per CU, bounded by LDS as well.
template <int Q>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) chunk_state_kernel(
    const int8_t* __restrict__ x, const float* __restrict__ x_scale, const int8_t* __restrict__ Bm,
    const float* __restrict__ B_scale, const float* __restrict__ C_scale_ps, const float* __restrict__ dt,
    const float* __restrict__ A, float* __restrict__ acs, float* __restrict__ dtc, float* __restrict__ states,
    int64_t seqlen, int32_t nheads,
    int32_t headdim, int32_t dstate, int32_t ngroups, int32_t nchunks, int32_t x_pc) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[Q * kMaxP];
  __shared__ __attribute__((aligned(16))) uint8_t bs[Q * kMaxN];
  __shared__ __attribute__((aligned(16))) uint32_t om[Q];   // OM_j
  __shared__ __attribute__((aligned(16))) uint32_t cb[Q];   // CB_j
  __shared__ float red[kWaves];
  __shared__ float acs_last_s;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: scalar descriptors, no waterfall
  const int lane = tid % kWave;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bid % nheads;
  const int c = (bid / nheads) % nchunks;
  const int b = bid / (nheads * nchunks);
  const int g = h / (nheads / ngroups);
  const int64_t t0 = int64_t(c) * Q;
  const int len = int(seqlen - t0 < Q ? seqlen - t0 : Q);
  const int P = headdim, N = dstate;

  // ---- global loads: dt of this thread's token, then the x and B codes of the chunk
  const uint32_t xrow = uint32_t(nheads * P), brow = uint32_t(ngroups * N);
  const Rsrc rdt = make_rsrc(dt + (int64_t(b) * seqlen + t0) * nheads + h, (uint32_t(len - 1) * nheads + 1u) * 4u);
  const float d = tid < Q ? buf_loadf(rdt, uint32_t(tid) * uint32_t(nheads) * 4u) : 0.f;   // 0 past the end
  Staged<Q> st;
  {
    const Rsrc rx = make_rsrc(x + ((int64_t(b) * seqlen + t0) * nheads + h) * P, uint32_t(len - 1) * xrow + P);
    const Rsrc rb = make_rsrc(Bm + ((int64_t(b) * seqlen + t0) * ngroups + g) * N, uint32_t(len - 1) * brow + N);
#pragma unroll
    for (int k = 0; k < Staged<Q>::kX; ++k) {
      const int piece = tid + k * kThreads, j = piece >> 2, cc = piece & 3;
      st.x[k] = buf_load16(rx, 16 * cc < P ? uint32_t(j) * xrow + 16 * cc : kOutOfRange);
    }
#pragma unroll
    for (int k = 0; k < Staged<Q>::kB; ++k) {
      const int piece = tid + k * kThreads, j = piece >> 3, cc = piece & 7;
      st.b[k] = buf_load16(rb, 16 * cc < N ? uint32_t(j) * brow + 16 * cc : kOutOfRange);
    }
  }

  // ---- (a) chunk cumsum of dt A, one token per thread of waves 0..Q/64-1
  const float v = wave_inclusive_sum(d * A[h]);
  if (lane == kWave - 1) red[wave] = v;
  __syncthreads();
  float pre = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < kWaves - 1; ++w2) pre += w2 < wave ? red[w2] : 0.f;
  const float acs_t = v + pre;
  if (tid < Q) {
    const int64_t o = ((int64_t(b) * nheads + h) * nchunks + c) * Q + tid;
    acs[o] = acs_t;
    dtc[o] = d;   // dt in chunk order for the output stage (0 past the end)
  }
  if (tid == len - 1) acs_last_s = acs_t;
  __syncthreads();

  // ---- LUT_state weights and their power-of-two range
  const float w = d > 0.f ? __builtin_amdgcn_exp2f((acs_last_s - acs_t) * kLog2e) * d : 0.f;
  const float wm = wave_max(w);
  __syncthreads();   // red[] reuse
  if (lane == 0) red[wave] = wm;
  __syncthreads();
  float wmax = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) wmax = fmaxf(wmax, red[i]);
  const int e = min(max(ceil_log2_pos(wmax), -100), 100);
  if (tid < Q) {
    const uint32_t o = uint32_t(fminf(w * exp2i(24 - e), 16777215.f) + 0.5f);
    om[tid] = o;
    cb[tid] = 8421376u - (o << 7);   // 256 * 32896 - 128 OM (mod 2^32)
  }

  // ---- the x and B codes of the chunk into LDS (16-byte copies)
#pragma unroll
  for (int k = 0; k < Staged<Q>::kX; ++k) {
    const int piece = tid + k * kThreads;
    *reinterpret_cast<v4u*>(xs + xpos(piece >> 2, 16 * (piece & 3))) = st.x[k];
  }
#pragma unroll
  for (int k = 0; k < Staged<Q>::kB; ++k) {
    const int piece = tid + k * kThreads;
    *reinterpret_cast<v4u*>(bs + bpos(piece >> 3, 16 * (piece & 7))) = st.b[k];
  }
  __syncthreads();

  // ---- S tiles on the zero-padded 64 x 128 space: wave w owns channel tile w and all eight
  // 16-state tiles; the K loop is unrolled, its first step starts the accumulators.
  const int lcol = lane % 16, kg = lane / 16;
  const int pt = wave;
  constexpr int kNt = kMaxN / 16;
  // transposing-read addresses: lane 2k + h of its group addresses token row 16 kg + k (+ 8 for
  // the second read) at column 16 tile + 8 h; the K step adds 64 rows (a constant offset)
  const int rowb = 16 * kg + (lcol >> 1), half8 = 8 * (lcol & 1);
  const int xa0 = xpos(rowb, 16 * pt + half8), xa1 = xpos(rowb + 8, 16 * pt + half8);
  // B: bpos(rowb + 8 hh, 16 t + half8) = ba[t ^ 4 hh] + 8 hh * 128, since the row swizzle of
  // rowb + 8 is that of rowb with bit 2 flipped
  int ba[kNt];
#pragma unroll
  for (int t = 0; t < kNt; ++t) ba[t] = bpos(rowb, 16 * t + half8);
  v4i acc[kNt][3];
#pragma unroll
  for (int kb = 0; kb < Q; kb += 64) {
    const int j0 = kb + 16 * kg;
    const v2u xlo = tr8(xs + xa0 + kb * kMaxP), xhi = tr8(xs + xa1 + kb * kMaxP);
    const uint32_t xw[4] = {xlo[0], xlo[1], xhi[0], xhi[1]};   // tokens j0..j0+15 of channel p
    v4i l1, l2, l3;
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const v4u o4 = *reinterpret_cast<const v4u*>(&om[j0 + 4 * dw]);
      const v4u c4 = *reinterpret_cast<const v4u*>(&cb[j0 + 4 * dw]);
      const uint32_t u = xw[dw] ^ 0x80808080u;   // biased codes q + 128
      uint32_t W[4], pl[4];
      W[0] = mad24(u & 0xffu, o4[0], c4[0]);
      W[1] = mad24((u >> 8) & 0xffu, o4[1], c4[1]);
      W[2] = mad24((u >> 16) & 0xffu, o4[2], c4[2]);
      W[3] = mad24(u >> 24, o4[3], c4[3]);
      transpose4x4(W, pl);
      l1[dw] = int(pl[3]);
      l2[dw] = int(pl[2] ^ 0x80808080u);
      l3[dw] = int(pl[1] ^ 0x80808080u);
    }
#pragma unroll
    for (int t = 0; t < kNt; ++t) {
      const v2u blo = tr8(bs + ba[t] + kb * kMaxN), bhi = tr8(bs + ba[t ^ 4] + (kb + 8) * kMaxN);
      const v4i bop = {int(blo[0]), int(blo[1]), int(bhi[0]), int(bhi[1])};
      const v4i z = {0, 0, 0, 0};
      acc[t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(l1, bop, kb == 0 ? z : acc[t][0], 0, 0, 0);
      acc[t][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(l2, bop, kb == 0 ? z : acc[t][1], 0, 0, 0);
      acc[t][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(l3, bop, kb == 0 ? z : acc[t][2], 0, 0, 0);
    }
  }
  // ---- epilogue.  D layout of a 16x16 MFMA: lane holds rows 4 (lane/16) + i, column lane % 16.
  // Rows past P and states past N are skipped with wave-uniform tests (P, N multiples of 16).
  if (16 * pt >= P) return;
  // per group: the B scale of the group; with scales per (group, state) (C_scale_ps non-null) the
  // state column's B scale times its C scale: the chunk states are then written scaled by the C
  // scale of each state (the form the carried state takes for the output stage)
  // (x_pc: x scales per (head, channel), one per row of S)
  const float post = x_scale[h] * (C_scale_ps ? 1.f : B_scale[g]) * exp2i(e);
  const float post_lo = post * (1.f / 65536.f);
  // buffer stores: lane offset + row offset (scalar) + state-tile offset (immediate)
  const Rsrc rs = make_rsrc(states + ((int64_t(b) * nchunks + c) * nheads + h) * int64_t(P) * N, uint32_t(P * N) * 4u);
  const uint32_t lane_off = (uint32_t(16 * pt + 4 * kg) * uint32_t(N) + lcol) * 4u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row_off = i * N * 4;   // uniform
    float pst = post, pst_lo = post_lo;
    if (x_pc) {   // uniform
      pst = x_scale[h * P + 16 * pt + 4 * kg + i] * (C_scale_ps ? 1.f : B_scale[g]) * exp2i(e);
      pst_lo = pst * (1.f / 65536.f);
    }
#pragma unroll
    for (int t = 0; t < kNt; ++t) {
      if (16 * t >= N) break;
      const int32_t lo = (acc[t][1][i] << 8) + acc[t][2][i];   // exact: |lo| < 2^31
      float sv = fmaf(float(lo), pst_lo, float(acc[t][0][i]) * pst);
      if (C_scale_ps) {   // uniform
        const int n = 16 * t + lcol;
        sv *= B_scale[g * N + n] * C_scale_ps[g * N + n];
      }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv), rs, lane_off + 64u * t, row_off, 0);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Stages 0 and 1 fused, for shapes with at least one (batch, head) sequence per CU: one block
// per (batch, head) walks the chunks in order and carries the running state H in registers,
//
//   Hprev_c = H (written as two INT8 limbs + a power-of-two row scale, as stage 1 writes it),
//   H <- exp(Acs_c[last]) H + S_c,
//
// with S_c from the same INT8-limb MFMAs as above, so the fp32 chunk states never leave the
// CU.  S_c is computed transposed (the B codes as the A operand), so that a lane holds four
// consecutive states n = 16 t + 4 kg + i of one channel row p = 16 pt + lcol: the limb bytes of
// four states are one 4-byte store and the row max is a short shuffle.  Eight waves: waves w and
// w + 4 own channel tile w % 4 and split the chunk's 64-token steps between them (no limb is
// built twice); each converts its partial S to fp32, hands the other the half of the state
// tiles it does not own through LDS, and updates its own half of H.  The next chunk's dt, x and
// B loads are issued before the current chunk's MFMAs.
constexpr int kSThreads = 512;
template <int v>
struct Parity {
  static constexpr int value = v;
};
constexpr int kSWaves = kSThreads / kWave;
constexpr int kGroup = kSWaves;   // chunks whose weights one prologue prepares (one per wave)
static_assert(kGroup % 2 == 0, "groups start at even chunks (tile buffer parity)");

// kPS: B and C scales per (group, state).  The running state is then kept scaled by the C scale
// of each state, H_C[p, n] = C_scale[g, n] H[p, n] (h0 scaled on the way in, h_final unscaled on
// the way out), so that each chunk adds sigma[n] S'[p, n] with sigma = B_scale C_scale and S' the
// products without the B scale, and the carried state the output stage reads out with the C codes
// already holds the C scale of its state.
// kPC: x scales per (head, channel); each lane's channel row takes its own (fixed per block).
template <int Q, bool kPS, bool kPC>
__global__ void __launch_bounds__(kSThreads) __attribute__((amdgpu_waves_per_eu(2))) state_scan_kernel(
    const int8_t* __restrict__ x, const float* __restrict__ x_scale, const int8_t* __restrict__ Bm,
    const float* __restrict__ B_scale, const float* __restrict__ C_scale, const float* __restrict__ dt,
    const float* __restrict__ A,
    const float* h0, float* h_final, float* __restrict__ acs, float* __restrict__ dtc, int8_t* __restrict__ hprev,
    float* __restrict__ hscale, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
    int32_t ngroups, int32_t nchunks) {
  // double-buffered chunk tiles, as separate objects so that the compiler can tell the buffer
  // being filled from the one being read (no wait on the fill before each read)
  __shared__ __attribute__((aligned(16))) uint8_t xs0[Q * kMaxP];
  __shared__ __attribute__((aligned(16))) uint8_t xs1[Q * kMaxP];
  __shared__ __attribute__((aligned(16))) uint8_t bs0[Q * kMaxN];
  __shared__ __attribute__((aligned(16))) uint8_t bs1[Q * kMaxN];
  __shared__ __attribute__((aligned(16))) uint32_t om[kGroup][Q];       // OM_j of the group's chunks
  __shared__ __attribute__((aligned(16))) v4f xch[kSWaves][4][kWave];   // partial S handed over
  __shared__ float rmax[2][kMaxP];                                      // half-row maxima
  __shared__ float gdec[kGroup];                                        // exp(Acs_last) per chunk
  __shared__ int gexp[kGroup];                                          // 2^e >= max_j w_j per chunk

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: scalar descriptors, no waterfall
  const int lane = tid % kWave;
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bh % nheads;
  const int b = bh / nheads;
  const int g = h / (nheads / ngroups);
  const int P = headdim, N = dstate;
  const int lcol = lane % 16, kg = lane / 16;
  const int pt = wave & 3, kh = wave >> 2;   // channel tile; half of the K steps and of the state tiles
  constexpr int kNt = kMaxN / 16;
  constexpr int kOwn = kNt / 2;               // state tiles 4 kh .. 4 kh + 3 belong to this wave
  constexpr int kTok = Q / kWave;              // tokens per lane in a group prologue
  const bool prow = 16 * pt < P;               // this wave's channel tile exists (uniform)
  const uint32_t xrow = uint32_t(nheads * P), brow = uint32_t(ngroups * N);
  const float sxB = x_scale[kPC ? h * P + min(16 * pt + lcol, P - 1) : h] * (kPS ? 1.f : B_scale[g]);
  const float Ah = A[h];

  // ---- running state H[p = 16 pt + lcol][n = 16 (4 kh + t) + 4 kg + i], own tiles t = 0..3
  const int64_t pn = int64_t(P) * N;
  const uint32_t hoff = (uint32_t(16 * pt + lcol) * uint32_t(N) + 64 * kh + 4 * kg) * 4u;   // bytes
  v4f H[kOwn];
  v4f sig[kPS ? kOwn : 1];   // per state: B_scale C_scale of this lane's own states
  {
    const Rsrc r0 = make_rsrc(h0 ? h0 + int64_t(bh) * pn : h0, h0 && prow ? uint32_t(pn) * 4u : 0u);
#pragma unroll
    for (int t = 0; t < kOwn; ++t)
      H[t] = __builtin_bit_cast(v4f, buf_load16(r0, 16 * (kOwn * kh + t) < N ? hoff + 64u * t : kOutOfRange));
    if constexpr (kPS) {
      const Rsrc rsb = make_rsrc(B_scale + g * N, uint32_t(N) * 4u), rsc = make_rsrc(C_scale + g * N, uint32_t(N) * 4u);
#pragma unroll
      for (int t = 0; t < kOwn; ++t) {
        const uint32_t o = 16 * (kOwn * kh + t) < N ? uint32_t(64 * kh + 16 * t + 4 * kg) * 4u : kOutOfRange;
        const v4f sb = __builtin_bit_cast(v4f, buf_load16(rsb, o)), sc = __builtin_bit_cast(v4f, buf_load16(rsc, o));
        sig[t] = sb * sc;
        H[t] = H[t] * sc;   // H_C
      }
    }
  }

  // ---- the x and B codes of chunk c, straight into LDS tile buffer c % 2 (buffer loads to LDS:
  // a wave's 64 lanes fill 1 KB of LDS in lane order, so each lane loads the global piece that
  // belongs at its slot of the swizzled layout).  A chunk past the end gets empty buffers: its
  // loads write zeros and touch no memory.
  constexpr int kXd = Q * (kMaxP / 16) / kSThreads;   // 16-byte x slots per thread (0 for Q = 64: below)
  constexpr int kBd = Q * (kMaxN / 16) / kSThreads;
  constexpr int kXs = kXd > 0 ? kXd : 1;
  uint32_t xoff[kXs], boff[kBd];
#pragma unroll
  for (int k = 0; k < kXs; ++k) {
    const int slot = k * kSThreads + tid, j = slot >> 2, pc = slot & 3, cc = pc ^ ((j >> 2) & 3);
    xoff[k] = (16 * cc < P && j < Q) ? uint32_t(j) * xrow + 16 * cc : kOutOfRange;
  }
#pragma unroll
  for (int k = 0; k < kBd; ++k) {
    const int slot = k * kSThreads + tid, j = slot >> 3, pc = slot & 7, cc = pc ^ ((j >> 1) & 7);
    boff[k] = (16 * cc < N && j < Q) ? uint32_t(j) * brow + 16 * cc : kOutOfRange;
  }
  auto dma_chunk = [&](int c, auto par) {
    const bool ok = c < nchunks;
    const int64_t t0 = ok ? int64_t(c) * Q : 0;
    const int len = ok ? int(seqlen - t0 < Q ? seqlen - t0 : Q) : 1;
    const Rsrc rx = make_rsrc(x + ((int64_t(b) * seqlen + t0) * nheads + h) * P, ok ? uint32_t(len - 1) * xrow + P : 0u);
    const Rsrc rb = make_rsrc(Bm + ((int64_t(b) * seqlen + t0) * ngroups + g) * N, ok ? uint32_t(len - 1) * brow + N : 0u);
    uint8_t* xd = par.value ? xs1 : xs0;
    uint8_t* bd = par.value ? bs1 : bs0;
#pragma unroll
    for (int k = 0; k < kXs; ++k) {
      if (kXd == 0 && wave >= Q * 4 / kWave) break;   // Q = 64: 256 slots, waves 0..3
      buf_load16_lds(rx, xd + 16 * (k * kSThreads + kWave * wave), xoff[k]);
    }
#pragma unroll
    for (int k = 0; k < kBd; ++k)
      buf_load16_lds(rb, bd + 16 * (k * kSThreads + kWave * wave), boff[k]);
  };
  // ---- dt of a group of kGroup chunks: wave w takes chunk g0 + w, lane l its tokens
  // l * kTok .. l * kTok + kTok - 1 (zeros past the sequence end)
  float dtg[kTok];
  auto load_dt_group = [&](int g0) {
    const int c = g0 + wave;
    const bool ok = c < nchunks;
    const int64_t t0 = ok ? int64_t(c) * Q : 0;
    const int len = ok ? int(seqlen - t0 < Q ? seqlen - t0 : Q) : 1;
    const Rsrc rdt = make_rsrc(dt + (int64_t(b) * seqlen + t0) * nheads + h, ok ? (uint32_t(len - 1) * nheads + 1u) * 4u : 0u);
#pragma unroll
    for (int u = 0; u < kTok; ++u) dtg[u] = buf_loadf(rdt, uint32_t(lane * kTok + u) * uint32_t(nheads) * 4u);
  };
  // ---- per-chunk quantities of a group, one chunk per wave and no block barriers: the chunk
  // cumsum of dt A (written to the workspace with dt in chunk order), its decay exp(Acs_last), the LUT_state weights
  // w_j = exp(Acs_last - Acs_j) dt_j, their power-of-two range 2^e and the integer limb
  // coefficients OM_j, CB_j
  auto group_prologue = [&](int g0) {
    const int c = g0 + wave;
    if (c >= nchunks) return;   // wave-uniform
    const int64_t t0 = int64_t(c) * Q;
    const int len = int(seqlen - t0 < Q ? seqlen - t0 : Q);
    float a[kTok];
    float run = 0.f;
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      run += dtg[u] * Ah;   // tokens past the end have dt = 0
      a[u] = run;
    }
    const float incl = wave_inclusive_sum(run);   // inclusive scan of the lane totals
    const float excl = incl - run;
#pragma unroll
    for (int u = 0; u < kTok; ++u) a[u] += excl;
    const int64_t ro = ((int64_t(b) * nheads + h) * nchunks + c) * Q + lane * kTok;
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      acs[ro + u] = a[u];
      dtc[ro + u] = dtg[u];   // dt in chunk order for the output stage (0 past the end)
    }
    // Acs at the chunk's last token
    const int lastl = (len - 1) / kTok, lastu = (len - 1) % kTok;
    float asel = a[0];
#pragma unroll
    for (int u = 1; u < kTok; ++u) asel = lastu == u ? a[u] : asel;
    const float a_last = lane_broadcast(asel, lastl);
    float w[kTok], wm = 0.f;
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      w[u] = dtg[u] > 0.f ? __builtin_amdgcn_exp2f((a_last - a[u]) * kLog2e) * dtg[u] : 0.f;
      wm = fmaxf(wm, w[u]);
    }
    const int e = min(max(ceil_log2_pos(wave_max(wm)), -100), 100);
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      // a signed 24-bit weight (23 bits of magnitude): OM_j = round(w_j 2^(23 - e))
      om[wave][lane * kTok + u] = uint32_t(fminf(w[u] * exp2i(23 - e), 8388607.f) + 0.5f);
    }
    if (lane == 0) {
      gdec[wave] = __builtin_amdgcn_exp2f(a_last * kLog2e);
      gexp[wave] = e;
    }
  };
  load_dt_group(0);
  dma_chunk(0, Parity<0>{});

  // transposing-read addresses (as in the kernel above)
  const int rowb = 16 * kg + (lcol >> 1), half8 = 8 * (lcol & 1);
  const int xa0 = xpos(rowb, 16 * pt + half8), xa1 = xpos(rowb + 8, 16 * pt + half8);
  // accumulator t holds state tile (t + 4 kh) % 8: the wave's own tiles are always acc[0..3]
  // and the ones it hands over acc[4..7], with no selects on kh (tile u ^ 4 stays at t ^ 4)
  int ba[kNt];
#pragma unroll
  for (int t = 0; t < kNt; ++t) ba[t] = bpos(rowb, 16 * ((t + kOwn * kh) % kNt) + half8);

  // one 64-token step of S^T into acc (first step starts the accumulators)
  auto kstep = [&](v4i (&acc)[kNt][3], const uint8_t* xt, const uint8_t* bt, int cl, int kb, bool first)
      {
    const int j0 = kb + 16 * kg;
    const v2u xlo = tr8(xt + xa0 + kb * kMaxP), xhi = tr8(xt + xa1 + kb * kMaxP);
    const uint32_t xw[4] = {xlo[0], xlo[1], xhi[0], xhi[1]};
    v4i l1, l2, l3;
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const v4u o4 = *reinterpret_cast<const v4u*>(&om[cl][j0 + 4 * dw]);
      // W = q OM + 256 * 32896: floor(W / 256) = floor(65536 t + 32896), t = q OM / 2^24
      uint32_t W[4], pl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) W[k] = uint32_t(mad24s(sbyte(xw[dw], k), int32_t(o4[k]), 8421376));
      transpose4x4(W, pl);
      l1[dw] = int(pl[3]);
      l2[dw] = int(pl[2] ^ 0x80808080u);
      l3[dw] = int(pl[1] ^ 0x80808080u);
    }
#pragma unroll
    for (int t = 0; t < kNt; ++t) {
      const v2u blo = tr8(bt + ba[t] + kb * kMaxN), bhi = tr8(bt + ba[t ^ 4] + (kb + 8) * kMaxN);
      const v4i bop = {int(blo[0]), int(blo[1]), int(bhi[0]), int(bhi[1])};
      const v4i z = {0, 0, 0, 0};
      acc[t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bop, l1, first ? z : acc[t][0], 0, 0, 0);
      acc[t][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bop, l2, first ? z : acc[t][1], 0, 0, 0);
      acc[t][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bop, l3, first ? z : acc[t][2], 0, 0, 0);
    }
  };

  for (int g0 = 0; g0 < nchunks; g0 += kGroup) {
    group_prologue(g0);
    load_dt_group(g0 + kGroup);   // in flight during the group's chunks
    const int gend = min(g0 + kGroup, nchunks);
    auto chunk_body = [&](int c, auto par) {   // par: c % 2, a compile-time constant
      const int cl = c - g0;
      const uint8_t* xt = par.value ? xs1 : xs0;
      const uint8_t* bt = par.value ? bs1 : bs0;
      v4i acc[kNt][3];
      // half-row maxima of the state entering the chunk (own 16 states x the 4 lanes of the row)
      {
        float m = 0.f;
#pragma unroll
        for (int t = 0; t < kOwn; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(H[t][i]));
        // lanes l ^ 16 and l ^ 32 (the row's other kg) by swapping 16- and 32-lane halves in
        // registers: no LDS round trip on the way to the barrier
        {
          const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
          m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
        }
        {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
          m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
        }
        if (kg == 0) rmax[kh][16 * pt + lcol] = m;
      }
      // this chunk's tiles (loaded into LDS one chunk ago) have landed: wait for every
      // outstanding vector-memory operation of this wave, then for all waves
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      __syncthreads();   // tiles, rmax (and, at a group start, the prologue's weights) visible
      // ---- the next chunk's tiles, into the other buffer (its last readers passed the barrier)
      dma_chunk(c + 1, Parity<1 - par.value>{});

      // ---- S_c^T partial over this wave's 64-token steps (interleaved between the two waves)
      if constexpr (Q == 64) {
        if (kh == 0) {
          kstep(acc, xt, bt, cl, 0, true);
        } else {
#pragma unroll
          for (int t = 0; t < kNt; ++t)
#pragma unroll
            for (int k = 0; k < 3; ++k) acc[t][k] = v4i{0, 0, 0, 0};
        }
      } else {
        kstep(acc, xt, bt, cl, 64 * kh, true);
        if constexpr (Q == 256) kstep(acc, xt, bt, cl, 64 * kh + 128, false);
        // let the scheduler interleave the operand reads, the limb arithmetic and the products
        __builtin_amdgcn_iglp_opt(0);
      }

      // ---- the state entering the chunk, Hprev_c = H, as two INT8 limbs and a power-of-two row
      // scale (after the products are issued: this VALU work runs while the matrix cores do)
      if (prow) {
        const float m = fmaxf(rmax[0][16 * pt + lcol], rmax[1][16 * pt + lcol]);
        const int ex = min(max(ceil_log2_pos(m * (1.f / 127.f)), -120), 120);
        const float inv = exp2i(8 - ex);
        const int64_t blk = (int64_t(b) * nchunks + c) * nheads + h;
        const Rsrc rh = make_rsrc(hprev + blk * 2 * pn, uint32_t(2 * pn));
        // this lane's 16 states of the row (4 tiles x 4): one 16-byte piece per limb when the
        // 64-state block is full (the workspace stores full blocks dword-transposed), else
        // 4-byte pieces in natural order
        // V = trunc(256 t + 128), |t| <= 127: limb 1 is byte 1 of V, limb 2 byte 0 with the bias
        // bit flipped; byte permutes gather them four at a time
        v4u Q1, Q2;
#pragma unroll
        for (int t = 0; t < kOwn; ++t) {
          uint32_t V[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) V[i] = uint32_t(int32_t(fmaf(H[t][i], inv, 128.f)));
          const uint32_t b1lo = __builtin_amdgcn_perm(V[1], V[0], 0x0c0c0501u), b1hi = __builtin_amdgcn_perm(V[3], V[2], 0x0c0c0501u);
          const uint32_t b0lo = __builtin_amdgcn_perm(V[1], V[0], 0x0c0c0400u), b0hi = __builtin_amdgcn_perm(V[3], V[2], 0x0c0c0400u);
          Q1[t] = __builtin_amdgcn_perm(b1hi, b1lo, 0x05040100u);
          Q2[t] = __builtin_amdgcn_perm(b0hi, b0lo, 0x05040100u) ^ 0x80808080u;
        }
        const uint32_t row = uint32_t(16 * pt + lcol) * uint32_t(N) + 64 * kh;
        if (64 * kh + 64 <= N) {
          __builtin_amdgcn_raw_buffer_store_b128(Q1, rh, row + 16 * kg, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(Q2, rh, row + 16 * kg, int(pn), 0);
        } else {
#pragma unroll
          for (int t = 0; t < kOwn; ++t) {
            if (64 * kh + 16 * t >= N) break;
            __builtin_amdgcn_raw_buffer_store_b32(Q1[t], rh, row + 16 * t + 4 * kg, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(Q2[t], rh, row + 16 * t + 4 * kg, int(pn), 0);
          }
        }
        if (kh == 0 && kg == 0) hscale[blk * P + 16 * pt + lcol] = exp2i(ex);
      }


      // ---- fp32 partials; hand over the other wave's tiles, then H <- exp(Acs_last) H + S_c
      const float post = sxB * exp2i(gexp[cl] + 1);   // t = x_scaled / 2^(e + 1) (23-bit weights)
      // partial S / post = acc0 + (256 acc1 + acc2) / 65536; post is applied once, in the update
      auto partial = [&](int t) {
        v4f r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t lo = (acc[t][1][i] << 8) + acc[t][2][i];
          r[i] = fmaf(float(lo), 1.f / 65536.f, float(acc[t][0][i]));
        }
        return r;
      };
#pragma unroll
      for (int t = 0; t < kOwn; ++t) xch[wave][t][lane] = partial(kOwn + t);
      v4f mine[kOwn];
#pragma unroll
      for (int t = 0; t < kOwn; ++t) mine[t] = partial(t);
      const float decay = gdec[cl];   // read before the barrier: the next group's prologue rewrites it
      __syncthreads();
#pragma unroll
      for (int t = 0; t < kOwn; ++t) {
        const v4f other = xch[wave ^ 4][t][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kPS)
            H[t][i] = fmaf(decay, H[t][i], (mine[t][i] + other[i]) * (post * sig[t][i]));
          else
            H[t][i] = fmaf(decay, H[t][i], (mine[t][i] + other[i]) * post);
        }
      }
    };
    for (int c = g0; c < gend; c += 2) {   // g0 is even
      chunk_body(c, Parity<0>{});
      if (c + 1 < gend) chunk_body(c + 1, Parity<1>{});
    }
  }

  // ---- final state (per state: H_C / C_scale)
  if (h_final && prow) {
    const Rsrc rf = make_rsrc(h_final + int64_t(bh) * pn, uint32_t(pn) * 4u);
#pragma unroll
    for (int t = 0; t < kOwn; ++t) {
      if (16 * (kOwn * kh + t) >= N) break;
      v4f hf = H[t];
      if constexpr (kPS) {
        const v4f sc = *reinterpret_cast<const v4f*>(C_scale + g * N + 64 * kh + 16 * t + 4 * kg);
#pragma unroll
        for (int i = 0; i < 4; ++i) hf[i] = hf[i] / sc[i];
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, hf), rf, hoff + 64u * t, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Four-wave form of the folded state kernel, for shapes with many (batch, head) sequences per
// CU: one block of four waves per sequence, wave w owning channel tile w over all of a chunk's
// tokens and all states.  A chunk's products then need no partial exchange between waves (the
// three limbs of all K steps accumulate in one wave's int32 registers), a state row's maximum
// is a reduction inside the wave, and the carried-state encoding covers a whole row per lane
// group.
//
// The chunk is staged in units of up to 128 tokens through two LDS buffers (~57 KB in all at
// chunk 256 with the weights' two slots, so two blocks share a CU), one barrier per unit, and
// the loads of unit u + 1 are issued right after unit u's barrier.  The products of a chunk do
// not depend on the running state, so they are software-pipelined against it: the first unit of
// chunk c folds chunk c - 1's products into H tile by tile (H_c = exp(Acs_last) H_{c-1} +
// S_{c-1}) and, as each tile's accumulators are consumed, issues chunk c's first MFMAs into
// them; the last unit of chunk c issues its MFMAs and then encodes H_c (the state entering the
// chunk) while they complete.  The matrix cores thus work under the VALU's update and encoding
// instead of after them.  The chunk weights are
// prepared one group of four chunks ahead (one chunk per wave) into a second LDS slot.
constexpr int kS4Threads = 256;
constexpr int kS4Waves = kS4Threads / kWave;
constexpr int kGroup4 = kS4Waves;   // chunks whose weights one prologue prepares (one per wave)

template <int Q, bool kPS, bool kPC>
__global__ void __launch_bounds__(kS4Threads) __attribute__((amdgpu_waves_per_eu(2))) state_scan4_kernel(
    const int8_t* __restrict__ x, const float* __restrict__ x_scale, const int8_t* __restrict__ Bm,
    const float* __restrict__ B_scale, const float* __restrict__ C_scale, const float* __restrict__ dt,
    const float* __restrict__ A,
    const float* h0, float* h_final, float* __restrict__ acs, float* __restrict__ dtc, int8_t* __restrict__ hprev,
    float* __restrict__ hscale, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
    int32_t ngroups, int32_t nchunks) {
  constexpr int kU = Q > 128 ? 128 : Q;   // tokens per staged unit
  constexpr int kUnits = Q / kU;          // units per chunk
  constexpr int kKs = kU / 64;            // K steps per unit
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][kU * kMaxP];
  __shared__ __attribute__((aligned(16))) uint8_t bs[2][kU * kMaxN];
  __shared__ __attribute__((aligned(16))) uint32_t om[2][kGroup4][Q];
  __shared__ float gdec[2][kGroup4];
  __shared__ int gexp[2][kGroup4];
  __shared__ __attribute__((aligned(16))) float sig_s[kPS ? kMaxN : 4];   // kPS: B_scale C_scale per state

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bh % nheads;
  const int b = bh / nheads;
  const int g = h / (nheads / ngroups);
  const int P = headdim, N = dstate;
  const int lcol = lane % 16, kg = lane / 16;
  const int pt = wave;
  constexpr int kNt = kMaxN / 16;
  constexpr int kTok = Q / kWave;
  const bool prow = 16 * pt < P;
  const uint32_t xrow = uint32_t(nheads * P), brow = uint32_t(ngroups * N);
  const float sxB = x_scale[kPC ? h * P + min(16 * pt + lcol, P - 1) : h] * (kPS ? 1.f : B_scale[g]);
  const float Ah = A[h];

  // running state H[p = 16 pt + lcol][n = 16 t + 4 kg + i], all eight state tiles
  const int64_t pn = int64_t(P) * N;
  const uint32_t hoff = (uint32_t(16 * pt + lcol) * uint32_t(N) + 4 * kg) * 4u;
  v4f H[kNt];
  {
    const Rsrc r0 = make_rsrc(h0 ? h0 + int64_t(bh) * pn : h0, h0 && prow ? uint32_t(pn) * 4u : 0u);
#pragma unroll
    for (int t = 0; t < kNt; ++t)
      H[t] = __builtin_bit_cast(v4f, buf_load16(r0, 16 * t < N ? hoff + 64u * t : kOutOfRange));
    if constexpr (kPS) {
      // the running state is kept as H_C (scaled by each state's C scale); the products' factor
      // per state, B_scale C_scale, waits in LDS (read back per chunk: registers are short here)
      const Rsrc rsc = make_rsrc(C_scale + g * N, uint32_t(N) * 4u);
#pragma unroll
      for (int t = 0; t < kNt; ++t) {
        const uint32_t o = 16 * t < N ? uint32_t(16 * t + 4 * kg) * 4u : kOutOfRange;
        H[t] = H[t] * __builtin_bit_cast(v4f, buf_load16(rsc, o));
      }
      if (tid < kMaxN) sig_s[tid] = tid < N ? B_scale[g * N + tid] * C_scale[g * N + tid] : 0.f;
      // (made visible by the first unit's barrier)
    }
  }

  // unit tiles by buffer loads straight into LDS (16 bytes per lane, swizzled slots)
  constexpr int kXd = kU * (kMaxP / 16) / kS4Threads;   // kU / 64
  constexpr int kBd = kU * (kMaxN / 16) / kS4Threads;   // kU / 32
  // slot k * 256 + tid of a unit tile: row j, 16-byte chunk pc in LDS, global chunk cc
  auto xoff = [&](int k) {
    const int slot = k * kS4Threads + tid, j = slot >> 2, pc = slot & 3, cc = pc ^ ((j >> 2) & 3);
    return 16 * cc < P ? uint32_t(j) * xrow + 16 * cc : kOutOfRange;
  };
  auto boff = [&](int k) {
    const int slot = k * kS4Threads + tid, j = slot >> 3, pc = slot & 7, cc = pc ^ ((j >> 1) & 7);
    return 16 * cc < N ? uint32_t(j) * brow + 16 * cc : kOutOfRange;
  };
  // unit u: tokens [c Q + (u % kUnits) kU, + kU) of chunk c = u / kUnits; rows past the sequence
  // end (a whole unit, in a short last chunk) read as zeros
  auto dma_unit = [&](int u) {
    const int64_t t0 = int64_t(u / kUnits) * Q + (u % kUnits) * kU;
    const bool ok = t0 < seqlen;
    const int len = ok ? int(seqlen - t0 < kU ? seqlen - t0 : kU) : 1;
    const int64_t tb = ok ? t0 : 0;
    const Rsrc rx = make_rsrc(x + ((int64_t(b) * seqlen + tb) * nheads + h) * P, ok ? uint32_t(len - 1) * xrow + P : 0u);
    const Rsrc rb = make_rsrc(Bm + ((int64_t(b) * seqlen + tb) * ngroups + g) * N, ok ? uint32_t(len - 1) * brow + N : 0u);
    uint8_t* xd = xs[u & 1];
    uint8_t* bd = bs[u & 1];
#pragma unroll
    for (int k = 0; k < kXd; ++k) buf_load16_lds(rx, xd + 16 * (k * kS4Threads + kWave * wave), xoff(k));
#pragma unroll
    for (int k = 0; k < kBd; ++k) buf_load16_lds(rb, bd + 16 * (k * kS4Threads + kWave * wave), boff(k));
  };
  float dtg[kTok];
  auto load_dt_group = [&](int g0) {
    const int c = g0 + wave;
    const bool ok = c < nchunks;
    const int64_t t0 = ok ? int64_t(c) * Q : 0;
    const int len = ok ? int(seqlen - t0 < Q ? seqlen - t0 : Q) : 1;
    const Rsrc rdt = make_rsrc(dt + (int64_t(b) * seqlen + t0) * nheads + h, ok ? (uint32_t(len - 1) * nheads + 1u) * 4u : 0u);
#pragma unroll
    for (int u = 0; u < kTok; ++u) dtg[u] = buf_loadf(rdt, uint32_t(lane * kTok + u) * uint32_t(nheads) * 4u);
  };
  // chunk g0 + wave's cumsum (to the workspace, with dt in chunk order) and its weights as
  // 23-bit integers under a power-of-two exponent, into LDS slot s
  auto group_prologue = [&](int g0, int s) {
    const int c = g0 + wave;
    if (c >= nchunks) return;
    const int64_t t0 = int64_t(c) * Q;
    const int len = int(seqlen - t0 < Q ? seqlen - t0 : Q);
    float a[kTok];
    float run = 0.f;
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      run += dtg[u] * Ah;
      a[u] = run;
    }
    const float incl = wave_inclusive_sum(run);
    const float excl = incl - run;
#pragma unroll
    for (int u = 0; u < kTok; ++u) a[u] += excl;
    const int64_t ro = ((int64_t(b) * nheads + h) * nchunks + c) * Q + lane * kTok;
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      acs[ro + u] = a[u];
      dtc[ro + u] = dtg[u];
    }
    const int lastl = (len - 1) / kTok, lastu = (len - 1) % kTok;
    float asel = a[0];
#pragma unroll
    for (int u = 1; u < kTok; ++u) asel = lastu == u ? a[u] : asel;
    const float a_last = lane_broadcast(asel, lastl);
    float w[kTok], wm = 0.f;
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      w[u] = dtg[u] > 0.f ? __builtin_amdgcn_exp2f((a_last - a[u]) * kLog2e) * dtg[u] : 0.f;
      wm = fmaxf(wm, w[u]);
    }
    const int e = min(max(ceil_log2_pos(wave_max(wm)), -100), 100);
#pragma unroll
    for (int u = 0; u < kTok; ++u) om[s][wave][lane * kTok + u] = uint32_t(fminf(w[u] * exp2i(23 - e), 8388607.f) + 0.5f);
    if (lane == 0) {
      gdec[s][wave] = __builtin_amdgcn_exp2f(a_last * kLog2e);
      gexp[s][wave] = e;
    }
  };

  const int rowb = 16 * kg + (lcol >> 1), half8 = 8 * (lcol & 1);
  const int xa0 = xpos(rowb, 16 * pt + half8), xa1 = xpos(rowb + 8, 16 * pt + half8);
  int ba[kNt];
#pragma unroll
  for (int t = 0; t < kNt; ++t) ba[t] = bpos(rowb, 16 * t + half8);

  // the three limbs of X_scaled for the K step at unit row kb (weights omu: the unit's first token)
  auto limbs = [&](v4i (&l)[3], const uint8_t* xb, const uint32_t* omu, int kb) {
    const int j0 = kb + 16 * kg;
    const v2u xlo = tr8(xb + xa0 + kb * kMaxP), xhi = tr8(xb + xa1 + kb * kMaxP);
    const uint32_t xw[4] = {xlo[0], xlo[1], xhi[0], xhi[1]};
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const v4u o4 = *reinterpret_cast<const v4u*>(&omu[j0 + 4 * dw]);
      uint32_t W[4], pl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) W[k] = uint32_t(mad24s(sbyte(xw[dw], k), int32_t(o4[k]), 8421376));
      transpose4x4(W, pl);
      l[0][dw] = int(pl[3]);
      l[1][dw] = int(pl[2] ^ 0x80808080u);
      l[2][dw] = int(pl[1] ^ 0x80808080u);
    }
  };
  // state tile t's three products for the K step at unit row kb
  auto mfma_tile = [&](v4i (&a)[3], const v4i (&l)[3], const uint8_t* bb, int t, int kb, bool first) {
    const v2u blo = tr8(bb + ba[t] + kb * kMaxN), bhi = tr8(bb + ba[t ^ 4] + (kb + 8) * kMaxN);
    const v4i bop = {int(blo[0]), int(blo[1]), int(bhi[0]), int(bhi[1])};
    const v4i z = {0, 0, 0, 0};
    a[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bop, l[0], first ? z : a[0], 0, 0, 0);
    a[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bop, l[1], first ? z : a[1], 0, 0, 0);
    a[2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bop, l[2], first ? z : a[2], 0, 0, 0);
  };
  // H[t] <- decay H[t] + S[t], S recombined from its three limbs' sums
  auto update_tile = [&](const v4i (&a)[3], int t, float decay, float post) {
    v4f sg = {1.f, 1.f, 1.f, 1.f};
    if constexpr (kPS) sg = *reinterpret_cast<const v4f*>(&sig_s[16 * t + 4 * kg]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t lo = (a[1][i] << 8) + a[2][i];
      const float sv = fmaf(float(lo), 1.f / 65536.f, float(a[0][i]));
      if constexpr (kPS)
        H[t][i] = fmaf(decay, H[t][i], sv * (post * sg[i]));
      else
        H[t][i] = fmaf(decay, H[t][i], sv * post);
    }
  };
  // the state entering chunk c as two INT8 limbs + a power-of-two row scale
  auto encode = [&](int c) {
    float m = 0.f;
#pragma unroll
    for (int t = 0; t < kNt; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(H[t][i]));
    {   // the row's four lanes (kg = 0..3) by half-wave swaps
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if (!prow) return;
    const int ex = min(max(ceil_log2_pos(m * (1.f / 127.f)), -120), 120);
    const float inv = exp2i(8 - ex);
    const int64_t blk = (int64_t(b) * nchunks + c) * nheads + h;
    const Rsrc rh = make_rsrc(hprev + blk * 2 * pn, uint32_t(2 * pn));
    const uint32_t row = uint32_t(16 * pt + lcol) * uint32_t(N);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {   // 64-state blocks
      if (64 * hb >= N) break;
      v4u Q1, Q2;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = 4 * hb + tt;
        uint32_t V[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) V[i] = uint32_t(int32_t(fmaf(H[t][i], inv, 128.f)));
        const uint32_t b1lo = __builtin_amdgcn_perm(V[1], V[0], 0x0c0c0501u), b1hi = __builtin_amdgcn_perm(V[3], V[2], 0x0c0c0501u);
        const uint32_t b0lo = __builtin_amdgcn_perm(V[1], V[0], 0x0c0c0400u), b0hi = __builtin_amdgcn_perm(V[3], V[2], 0x0c0c0400u);
        Q1[tt] = __builtin_amdgcn_perm(b1hi, b1lo, 0x05040100u);
        Q2[tt] = __builtin_amdgcn_perm(b0hi, b0lo, 0x05040100u) ^ 0x80808080u;
      }
      if (64 * hb + 64 <= N) {
        __builtin_amdgcn_raw_buffer_store_b128(Q1, rh, row + 64 * hb + 16 * kg, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(Q2, rh, row + 64 * hb + 16 * kg, int(pn), 0);
      } else {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (64 * hb + 16 * tt >= N) break;
          __builtin_amdgcn_raw_buffer_store_b32(Q1[tt], rh, row + 64 * hb + 16 * tt + 4 * kg, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(Q2[tt], rh, row + 64 * hb + 16 * tt + 4 * kg, int(pn), 0);
        }
      }
    }
    if (kg == 0) hscale[blk * P + 16 * pt + lcol] = exp2i(ex);
  };

  load_dt_group(0);
  dma_unit(0);
  group_prologue(0, 0);
  load_dt_group(kGroup4);

  v4i acc[kNt][3];
  float dec_prev = 1.f, post_prev = 0.f;   // chunk c - 1's decay and products' scale
  for (int c = 0; c < nchunks; ++c) {
    const int s = (c / kGroup4) & 1, cl = c % kGroup4;
#pragma unroll
    for (int hu = 0; hu < kUnits; ++hu) {
      const int u = c * kUnits + hu;
      const int ub = kUnits == 2 ? hu : (c & 1);   // u & 1
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this unit's tiles have landed
      __syncthreads();                      // tiles visible; every wave is done with unit u - 1
      float dec_c = 0.f, post_c = 0.f;
      if (hu == 0) {
        dec_c = gdec[s][cl];
        post_c = sxB * exp2i(gexp[s][cl] + 1);
      }
      if (hu + 1 < kUnits || c + 1 < nchunks) dma_unit(u + 1);   // into the buffer unit u - 1 used
      if (hu == 0 && cl == 0) {             // a group start: the next group's weights, other slot
        group_prologue(c + kGroup4, s ^ 1);
        load_dt_group(c + 2 * kGroup4);
      }
      const uint8_t* xb = xs[ub];
      const uint8_t* bb = bs[ub];
      const uint32_t* omu = &om[s][cl][hu * kU];
      v4i l[kKs][3];
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) limbs(l[ks], xb, omu, 64 * ks);
      if (hu == 0) {
        if (c > 0) {
#pragma unroll
          for (int t = 0; t < kNt; ++t) {
            update_tile(acc[t], t, dec_prev, post_prev);
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) mfma_tile(acc[t], l[ks], bb, t, 64 * ks, ks == 0);
          }
        } else {
#pragma unroll
          for (int t = 0; t < kNt; ++t)
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) mfma_tile(acc[t], l[ks], bb, t, 64 * ks, ks == 0);
        }
        dec_prev = dec_c;
        post_prev = post_c;
      } else {
#pragma unroll
        for (int t = 0; t < kNt; ++t)
#pragma unroll
          for (int ks = 0; ks < kKs; ++ks) mfma_tile(acc[t], l[ks], bb, t, 64 * ks, false);
      }
      if (hu == kUnits - 1) encode(c);
    }
  }
#pragma unroll
  for (int t = 0; t < kNt; ++t) update_tile(acc[t], t, dec_prev, post_prev);   // the last chunk's S

  if (h_final && prow) {
    const Rsrc rf = make_rsrc(h_final + int64_t(bh) * pn, uint32_t(pn) * 4u);
#pragma unroll
    for (int t = 0; t < kNt; ++t) {
      if (16 * t >= N) break;
      v4f hf = H[t];
      if constexpr (kPS) {
        const v4f sc = *reinterpret_cast<const v4f*>(C_scale + g * N + 16 * t + 4 * kg);
#pragma unroll
        for (int i = 0; i < 4; ++i) hf[i] = hf[i] / sc[i];
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, hf), rf, hoff + 64u * t, 0, 0);
    }
  }
}

}  // namespace

hipError_t launch_chunk_state(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  const int nblocks = s.batch * s.nchunks * s.nheads;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(nblocks), dim3(kThreads), 0, stream, a.x, a.x_scale, a.B, a.B_scale,
                       a.bc_per_state ? a.C_scale : nullptr, a.dt, a.A, a.acs, a.dtc, a.states, s.seqlen, s.nheads,
                       s.headdim, s.dstate, s.ngroups, s.nchunks, a.x_per_channel ? 1 : 0);
  };
  switch (s.chunk) {
    case 64: go(chunk_state_kernel<64>); break;
    case 128: go(chunk_state_kernel<128>); break;
    default: go(chunk_state_kernel<256>); break;
  }
  return hipGetLastError();
}

}  // namespace ssdq

namespace ssdq {

namespace {
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    return 0;
  return cus;
}
}  // namespace

bool state_scan_fused(int32_t batch, int32_t nheads) {
  const int cus = device_cus();
  return cus > 0 && int64_t(batch) * nheads >= cus;
}

// With C CUs, b H sequences take ceil(bH / 2C) rounds of two co-resident 4-wave blocks per CU
// against ceil(bH / C) rounds of one 8-wave block, and a 4-wave block sharing its CU takes ~1.77
// times as long as an 8-wave block alone (113 against 64 us per block at mamba2-8b-prefill); the
// four-wave form runs when that model gives it fewer such units (the scale layout does not
// change the choice).
int state_scan_waves(int32_t batch, int32_t nheads, bool bc_per_state) {
  (void)bc_per_state;
  const int cus = device_cus();
  const int64_t bh = int64_t(batch) * nheads;
  if (cus <= 0 || bh < cus) return 0;
  const int64_t r4 = (bh + 2 * cus - 1) / (2 * cus), r8 = (bh + cus - 1) / cus;
  return 177 * r4 < 100 * r8 ? 4 : 8;
}

hipError_t launch_state_scan(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  const int nblocks = s.batch * s.nheads;
  if (state_scan_waves(s.batch, s.nheads, a.bc_per_state) == 4) {
    auto go4 = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(nblocks), dim3(kS4Threads), 0, stream, a.x, a.x_scale, a.B, a.B_scale,
                         a.C_scale, a.dt, a.A, a.h0, a.h_final, a.acs, a.dtc, a.hprev, a.hscale, s.seqlen, s.nheads,
                         s.headdim, s.dstate, s.ngroups, s.nchunks);
    };
    auto by_chunk4 = [&](auto ps, auto pc) {
      constexpr bool kPS = decltype(ps)::value, kPC = decltype(pc)::value;
      switch (s.chunk) {
        case 64: go4(state_scan4_kernel<64, kPS, kPC>); break;
        case 128: go4(state_scan4_kernel<128, kPS, kPC>); break;
        default: go4(state_scan4_kernel<256, kPS, kPC>); break;
      }
    };
    using T = std::true_type;
    using F = std::false_type;
    if (a.bc_per_state)
      a.x_per_channel ? by_chunk4(T{}, T{}) : by_chunk4(T{}, F{});
    else
      a.x_per_channel ? by_chunk4(F{}, T{}) : by_chunk4(F{}, F{});
    return hipGetLastError();
  }
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(nblocks), dim3(kSThreads), 0, stream, a.x, a.x_scale, a.B, a.B_scale, a.C_scale,
                       a.dt, a.A, a.h0, a.h_final, a.acs, a.dtc, a.hprev, a.hscale, s.seqlen, s.nheads, s.headdim,
                       s.dstate, s.ngroups, s.nchunks);
  };
  auto by_chunk = [&](auto ps, auto pc) {
    constexpr bool kPS = decltype(ps)::value, kPC = decltype(pc)::value;
    switch (s.chunk) {
      case 64: go(state_scan_kernel<64, kPS, kPC>); break;
      case 128: go(state_scan_kernel<128, kPS, kPC>); break;
      default: go(state_scan_kernel<256, kPS, kPC>); break;
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  if (a.bc_per_state)
    a.x_per_channel ? by_chunk(T{}, T{}) : by_chunk(T{}, F{});
  else
    a.x_per_channel ? by_chunk(F{}, T{}) : by_chunk(F{}, F{});
  return hipGetLastError();
}

}  // namespace ssdq
