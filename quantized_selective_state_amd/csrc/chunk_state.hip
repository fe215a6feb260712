// Stage 0 of the chunked SSD scan, one block (4 waves) per (batch, chunk, head), compiled per
// chunk size:
//
//  (a) chunk cumsum: Acs[j] = sum_{i <= j} dt_i A_h inside the chunk (tokens past the end
//      of the sequence add 0), written to the workspace for the later stages;
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
// Both operands contract over tokens, the slow axis in memory, so x and B are transposed
// into LDS (token-contiguous 256-byte rows).  Rows use a 16-byte-chunk XOR swizzle that
// keeps both the transposing writes (rows 4q+i of 16 consecutive q) and the MFMA operand
// reads (16 consecutive rows) free of bank conflicts.  Each wave owns one 16-channel tile of
// S across all states and tokens, so every limb is built exactly once, in registers, from the
// x^T rows right before its MFMAs.
#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxP = 64;
constexpr int kMaxN = 128;
constexpr float kLog2e = 1.4426950408889634f;

// byte offset of (row, token byte) in a swizzled [rows][Q] int8 matrix: 16-byte chunk c of
// row r is stored at chunk c ^ swz(r), swz(r) < Q / 16.  For rows 4q + i (i < 4),
// swz(4q + i) = swz(4q) ^ i (Q / 16 >= 4), so tpos(4q + i, b) = (tpos(4q, b) ^ 16 i) + Q i.
template <int Q>
__device__ __forceinline__ int swz(int row) { return ((row & 15) ^ ((row >> 4) & 3)) & (Q / 16 - 1); }
template <int Q>
__device__ __forceinline__ int tpos(int row, int byte) {
  return row * Q + ((((byte >> 4) ^ swz<Q>(row)) << 4) | (byte & 15));
}

// a * b + c for a, b < 2^24 (one v_mad_u32_u24), modulo 2^32
__device__ __forceinline__ uint32_t mad24(uint32_t a, uint32_t b, uint32_t c) { return __umul24(a, b) + c; }

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

// Transposing the int8 codes of the chunk (kChan channel rows) into the swizzled
// token-contiguous LDS matrix.  A task is 4 channels x 4 tokens; a wave's 64 lanes take 16
// consecutive channel quads x 4 consecutive token quads, which makes the swizzled LDS writes
// conflict-free.  The global loads are issued first (stage_load, at kernel entry) and
// committed to LDS later (stage_commit), so their latency overlaps the chunk cumsum.  Loads
// go through a buffer whose size ends at the chunk's last valid row, so rows past the
// sequence end read as zeros; channel quads past `channels` use an out-of-range offset.
template <int Q, int kChan>
struct Staged {
  static constexpr int kXq = kChan / 4;             // channel quads (multiple of 16)
  static constexpr int kHi = kXq / 16;
  static constexpr int kIters = kXq * (Q / 4) / kThreads;
  static_assert(kXq * (Q / 4) % kThreads == 0, "tasks must tile the block");
  uint32_t v[kIters][4];
};

template <int kChan>
__device__ __forceinline__ void task_of(int task, int& xq, int& jq) {
  constexpr int kHi = kChan / 64;
  const int rest = task >> 6;
  xq = (task & 15) + 16 * (rest % kHi);
  jq = ((task >> 4) & 3) + 4 * (rest / kHi);
}

template <int Q, int kChan>
__device__ __forceinline__ void stage_load(Staged<Q, kChan>& st, Rsrc r, uint32_t stride, int channels, int tid) {
#pragma unroll
  for (int it = 0; it < Staged<Q, kChan>::kIters; ++it) {
    int xq, jq;
    task_of<kChan>(tid + it * kThreads, xq, jq);
    const uint32_t o = 4 * xq < channels ? uint32_t(4 * jq) * stride + 4 * xq : kOutOfRange;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) st.v[it][rr] = buf_load4(r, o + uint32_t(rr) * stride);
  }
}

template <int Q, int kChan>
__device__ __forceinline__ void stage_commit(uint8_t* lds, const Staged<Q, kChan>& st, int tid) {
#pragma unroll
  for (int it = 0; it < Staged<Q, kChan>::kIters; ++it) {
    int xq, jq;
    task_of<kChan>(tid + it * kThreads, xq, jq);
    uint32_t out[4];
    transpose4x4(st.v[it], out);
    const int t0 = tpos<Q>(4 * xq, 4 * jq);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(lds + (t0 ^ (16 * i)) + Q * i) = out[i];
  }
}

// 3 waves per SIMD (<= 168 VGPRs): three blocks per CU, bounded by LDS as well.
template <int Q>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) chunk_state_kernel(
    const int8_t* __restrict__ x, const float* __restrict__ x_scale, const int8_t* __restrict__ Bm,
    const float* __restrict__ B_scale, const float* __restrict__ dt, const float* __restrict__ A,
    float* __restrict__ acs, float* __restrict__ states, int64_t seqlen, int32_t nheads, int32_t headdim,
    int32_t dstate, int32_t ngroups, int32_t nchunks) {
  __shared__ __attribute__((aligned(16))) uint8_t xT[kMaxP * Q];
  __shared__ __attribute__((aligned(16))) uint8_t BT[kMaxN * Q];
  __shared__ __attribute__((aligned(16))) uint32_t om[Q];   // OM_j
  __shared__ __attribute__((aligned(16))) uint32_t cb[Q];   // CB_j
  __shared__ float red[kWaves];
  __shared__ float acs_last_s;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
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
  Staged<Q, kMaxP> xs;
  Staged<Q, kMaxN> bs;
  stage_load(xs, make_rsrc(x + ((int64_t(b) * seqlen + t0) * nheads + h) * P, uint32_t(len - 1) * xrow + P),
             xrow, P, tid);
  stage_load(bs, make_rsrc(Bm + ((int64_t(b) * seqlen + t0) * ngroups + g) * N, uint32_t(len - 1) * brow + N),
             brow, N, tid);

  // ---- (a) chunk cumsum of dt A, one token per thread of waves 0..Q/64-1
  float v = d * A[h];
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const float up = __shfl_up(v, o, kWave);
    if (lane >= o) v += up;
  }
  if (lane == kWave - 1) red[wave] = v;
  __syncthreads();
  float pre = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < kWaves - 1; ++w2) pre += w2 < wave ? red[w2] : 0.f;
  const float acs_t = v + pre;
  if (tid < Q) acs[((int64_t(b) * nheads + h) * nchunks + c) * Q + tid] = acs_t;
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

  // ---- x and B codes of the chunk, token-contiguous in LDS
  stage_commit(xT, xs, tid);
  stage_commit(BT, bs, tid);
  __syncthreads();

  // ---- S tiles on the zero-padded 64 x 128 space: wave w owns channel tile w and all eight
  // 16-state tiles; the K loop is unrolled, its first step starts the accumulators
  const int lcol = lane % 16, kg = lane / 16;
  const int pt = wave;
  constexpr int kNt = kMaxN / 16;
  v4i acc[kNt][3];
  const int p = 16 * pt + lcol;
#pragma unroll
  for (int kb = 0; kb < Q; kb += 64) {
    const int j0 = kb + 16 * kg;
    const v4u xw = *reinterpret_cast<const v4u*>(xT + tpos<Q>(p, j0));
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
      const v4i bop = *reinterpret_cast<const v4i*>(BT + tpos<Q>(16 * t + lcol, j0));
      const v4i z = {0, 0, 0, 0};
      acc[t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(l1, bop, kb == 0 ? z : acc[t][0], 0, 0, 0);
      acc[t][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(l2, bop, kb == 0 ? z : acc[t][1], 0, 0, 0);
      acc[t][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(l3, bop, kb == 0 ? z : acc[t][2], 0, 0, 0);
    }
  }
  // ---- epilogue.  D layout of a 16x16 MFMA: lane holds rows 4 (lane/16) + i, column lane % 16.
  // Rows past P and states past N are skipped with wave-uniform tests (P, N multiples of 16).
  if (16 * pt >= P) return;
  const float post = x_scale[h] * B_scale[g] * exp2i(e);
  const float post_lo = post * (1.f / 65536.f);
  float* Sc = states + ((int64_t(b) * nchunks + c) * nheads + h) * int64_t(P) * N + int64_t(16 * pt) * N;
  const uint32_t lane_off = uint32_t(4 * kg) * uint32_t(N) + lcol;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* Srow = Sc + int64_t(i) * N;   // uniform
#pragma unroll
    for (int t = 0; t < kNt; ++t) {
      if (16 * t >= N) break;
      const int32_t lo = (acc[t][1][i] << 8) + acc[t][2][i];   // exact: |lo| < 2^31
      Srow[lane_off + 16 * t] = fmaf(float(lo), post_lo, float(acc[t][0][i]) * post);
    }
  }
}

}  // namespace

hipError_t launch_chunk_state(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  const int nblocks = s.batch * s.nchunks * s.nheads;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(nblocks), dim3(kThreads), 0, stream, a.x, a.x_scale, a.B, a.B_scale, a.dt, a.A,
                       a.acs, a.states, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.nchunks);
  };
  switch (s.chunk) {
    case 64: go(chunk_state_kernel<64>); break;
    case 128: go(chunk_state_kernel<128>); break;
    default: go(chunk_state_kernel<256>); break;
  }
  return hipGetLastError();
}

}  // namespace ssdq
