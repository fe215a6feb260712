// Stage 0 of the chunked SSD scan, one block (4 waves) per (batch, chunk, head):
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
// V = trunc(65536 t + 32896) has the base-256 digits  V = l1 65536 + (l2+128) 256 + (l3+128),
// so t = l1 + l2/256 + l3/65536 to within 2^-16, with l1, l2, l3 signed bytes.  The bytes
// of V are the limbs, so a 4x4 byte transpose of four tokens' V yields the MFMA operand
// words directly.  Each limb goes through v_mfma_i32_16x16x64_i8 with exact int32 sums
// (|sum| <= Q 128 127 < 2^23) and an fp32 epilogue recombines them.
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
constexpr int kMaxQ = 256;
constexpr int kMaxP = 64;
constexpr int kMaxN = 128;
constexpr int kRow = kMaxQ;          // bytes per token-contiguous LDS row
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swz(int row) { return (row & 15) ^ ((row >> 4) & 3); }
// byte offset of (row, token byte) in a swizzled [rows][256] int8 matrix
__device__ __forceinline__ int tpos(int row, int byte) {
  return row * kRow + ((((byte >> 4) ^ swz(row)) << 4) | (byte & 15));
}

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

// Transposing the int8 codes of the chunk for `channels` (<= kChan) channels into the swizzled
// token-contiguous LDS matrix of kChan rows.  A task is 4 channels x 4 tokens; a wave's 64
// lanes take 16 consecutive channel quads x 4 consecutive token quads, which makes the
// swizzled LDS writes conflict-free.  Tasks cover all kMaxQ token positions of a row.
//
// The global loads are issued first (stage_load, at kernel entry) and committed to LDS later
// (stage_commit), so their latency overlaps the chunk cumsum.  Every load is unconditional:
// rows past the sequence end and channel quads past `channels` read a clamped in-chunk
// address, and stage_commit replaces them with zeros.  Addresses are 32-bit offsets from the
// chunk's base (the host bounds a chunk of x and of B below 2^31 bytes).
template <int kChan>
struct Staged {
  static constexpr int kXq = kChan / 4;             // channel quads (multiple of 16)
  static constexpr int kHi = kXq / 16;
  static constexpr int kIters = kXq * (kMaxQ / 4) / kThreads;
  uint32_t v[kIters][4];
};

template <int kChan>
__device__ __forceinline__ void task_of(int task, int& xq, int& jq) {
  constexpr int kHi = Staged<kChan>::kHi;
  const int rest = task >> 6;
  xq = (task & 15) + 16 * (rest % kHi);
  jq = ((task >> 4) & 3) + 4 * (rest / kHi);
}

template <int kChan>
__device__ __forceinline__ void stage_load(Staged<kChan>& st, const int8_t* base, uint32_t stride, int channels,
                                           int len, int tid) {
#pragma unroll
  for (int it = 0; it < Staged<kChan>::kIters; ++it) {
    int xq, jq;
    task_of<kChan>(tid + it * kThreads, xq, jq);
    const uint32_t xx = uint32_t(min(4 * xq, channels - 4));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t j = uint32_t(min(4 * jq + r, len - 1));
      st.v[it][r] = *reinterpret_cast<const uint32_t*>(base + (j * stride + xx));
    }
  }
}

template <int kChan>
__device__ __forceinline__ void stage_commit(uint8_t* lds, const Staged<kChan>& st, int channels, int len,
                                             int tid) {
#pragma unroll
  for (int it = 0; it < Staged<kChan>::kIters; ++it) {
    int xq, jq;
    task_of<kChan>(tid + it * kThreads, xq, jq);
    const bool chan_ok = 4 * xq < channels;
    uint32_t in[4], out[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) in[r] = (chan_ok && 4 * jq + r < len) ? st.v[it][r] : 0u;
    transpose4x4(in, out);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(lds + tpos(4 * xq + i, 4 * jq)) = out[i];
  }
}

// 3 waves per SIMD (<= 168 VGPRs): three blocks per CU, bounded by LDS as well.
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) chunk_state_kernel(
    const int8_t* __restrict__ x, const float* __restrict__ x_scale, const int8_t* __restrict__ Bm,
    const float* __restrict__ B_scale, const float* __restrict__ dt, const float* __restrict__ A,
    float* __restrict__ acs, float* __restrict__ states, int64_t seqlen, int32_t nheads, int32_t headdim,
    int32_t dstate, int32_t ngroups, int32_t chunk, int32_t nchunks) {
  __shared__ __attribute__((aligned(16))) uint8_t xT[kMaxP * kRow];
  __shared__ __attribute__((aligned(16))) uint8_t BT[kMaxN * kRow];
  __shared__ __attribute__((aligned(16))) float om[kMaxQ];   // w_j 2^-e 65536
  __shared__ __attribute__((aligned(16))) float cb[kMaxQ];   // 32896 - 128 om_j
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
  const int64_t t0 = int64_t(c) * chunk;
  const int len = int(seqlen - t0 < chunk ? seqlen - t0 : chunk);
  const int Q = chunk, P = headdim, N = dstate;

  // ---- global loads: dt of this thread's token, then the x and B codes of the chunk
  const float dt_raw = dt[(int64_t(b) * seqlen + t0 + min(tid, len - 1)) * nheads + h];
  Staged<kMaxP> xs;
  Staged<kMaxN> bs;
  stage_load(xs, x + ((int64_t(b) * seqlen + t0) * nheads + h) * P, uint32_t(nheads * P), P, len, tid);
  stage_load(bs, Bm + ((int64_t(b) * seqlen + t0) * ngroups + g) * N, uint32_t(ngroups * N), N, len, tid);

  // ---- (a) chunk cumsum of dt A, one token per thread of waves 0..Q/64-1
  const float d = tid < len ? dt_raw : 0.f;
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
  if (tid < Q) acs[((int64_t(b) * nheads + h) * nchunks + c) * chunk + tid] = acs_t;
  if (tid == len - 1) acs_last_s = acs_t;
  __syncthreads();

  // ---- LUT_state weights and their power-of-two range
  float w = 0.f;
  if (tid < len) w = exp2f((acs_last_s - acs_t) * kLog2e) * d;
  const float wm = wave_max(w);
  __syncthreads();   // red[] reuse
  if (lane == 0) red[wave] = wm;
  __syncthreads();
  float wmax = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) wmax = fmaxf(wmax, red[i]);
  const int e = min(max(ceil_log2_pos(wmax), -110), 110);
  if (tid < Q) {
    const float o = w * exp2i(16 - e);
    om[tid] = o;
    cb[tid] = 32896.f - 128.f * o;
  }

  // ---- x and B codes of the chunk, token-contiguous in LDS
  stage_commit(xT, xs, P, len, tid);
  stage_commit(BT, bs, N, len, tid);
  __syncthreads();

  // ---- S tiles on the zero-padded 64 x 128 space: wave w owns channel tile w and all eight
  // 16-state tiles
  const float post = x_scale[h] * B_scale[g] * exp2i(e);
  float* Sc = states + ((int64_t(b) * nchunks + c) * nheads + h) * int64_t(P) * N;
  const int lcol = lane % 16, kg = lane / 16;
  const int pt = wave;
  constexpr int kNt = kMaxN / 16;
  v4i acc[kNt][3];
#pragma unroll
  for (int t = 0; t < kNt; ++t)
#pragma unroll
    for (int k = 0; k < 3; ++k) acc[t][k] = v4i{0, 0, 0, 0};
  const int p = 16 * pt + lcol;
  for (int kb = 0; kb < Q; kb += 64) {
    const int j0 = kb + 16 * kg;
    const v4u xw = *reinterpret_cast<const v4u*>(xT + tpos(p, j0));
    v4i l1, l2, l3;
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const float4 o4 = *reinterpret_cast<const float4*>(&om[j0 + 4 * dw]);
      const float4 c4 = *reinterpret_cast<const float4*>(&cb[j0 + 4 * dw]);
      const uint32_t u = xw[dw] ^ 0x80808080u;   // biased codes q + 128
      uint32_t V[4], pl[4];
      V[0] = uint32_t(int32_t(fmaf(float(u & 0xffu), o4.x, c4.x)));
      V[1] = uint32_t(int32_t(fmaf(float((u >> 8) & 0xffu), o4.y, c4.y)));
      V[2] = uint32_t(int32_t(fmaf(float((u >> 16) & 0xffu), o4.z, c4.z)));
      V[3] = uint32_t(int32_t(fmaf(float(u >> 24), o4.w, c4.w)));
      transpose4x4(V, pl);
      l1[dw] = int(pl[2]);
      l2[dw] = int(pl[1] ^ 0x80808080u);
      l3[dw] = int(pl[0] ^ 0x80808080u);
    }
#pragma unroll
    for (int t = 0; t < kNt; ++t) {
      const v4i bop = *reinterpret_cast<const v4i*>(BT + tpos(16 * t + lcol, j0));
      acc[t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(l1, bop, acc[t][0], 0, 0, 0);
      acc[t][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(l2, bop, acc[t][1], 0, 0, 0);
      acc[t][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(l3, bop, acc[t][2], 0, 0, 0);
    }
  }
  // D layout of a 16x16 MFMA: lane holds rows 4 (lane/16) + i, column lane % 16
#pragma unroll
  for (int t = 0; t < kNt; ++t) {
    const int n = 16 * t + lcol;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pr = 16 * pt + 4 * kg + i;
      const float sv = float(acc[t][0][i]) + float(acc[t][1][i]) * (1.f / 256.f) +
                       float(acc[t][2][i]) * (1.f / 65536.f);
      if (pr < P && n < N) Sc[int64_t(pr) * N + n] = sv * post;
    }
  }
}

}  // namespace

hipError_t launch_chunk_state(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  const int nblocks = s.batch * s.nchunks * s.nheads;
  hipLaunchKernelGGL(chunk_state_kernel, dim3(nblocks), dim3(kThreads), 0, stream, a.x, a.x_scale, a.B, a.B_scale,
                     a.dt, a.A, a.acs, a.states, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk,
                     s.nchunks);
  return hipGetLastError();
}

}  // namespace ssdq
