// Stage 1 of the chunked SSD scan: the state each chunk contributes on its own,
//
//   S_c[p, n] = sum_{j in chunk c} w_j * xhat[j, p] * Bhat[j, n],
//   w_j = exp(Acs[c, last] - Acs[c, j]) * dt_j          (SSDi8's LUT_state, Figure 3a)
//
// computed as SSDi8 reformulates it (abstract; Figure 3a): first the element-wise
// X_scaled[j, p] = w_j * q_x[j, p], then a plain matrix product with the INT8 codes of B
// on the INT8 matrix cores.  A single INT8 copy of X_scaled loses too much precision for a
// 1e-4 state bound, so X_scaled is split into three exact INT8 limbs (the multi-component
// idea of the Multi-Scale Dequant abstract):
//
//   t = X_scaled / 2^e  with 2^e >= max_j w_j, so |t| <= 127;
//   t = l1 + l2 / 128 + l3 / 128^2 + r,   l1 in [-127, 127], l2, l3 in [-64, 64], |r| <= 2^-15
//
// Each limb is contracted with q_B on v_mfma_i32_16x16x64_i8 with exact int32 accumulation
// (|sum| <= Q * 127 * 127 < 2^24), and the fp32 epilogue recombines the limbs.
//
// One block (8 waves) per (batch, chunk, head).  Both MFMA operands contract over the token
// axis, which is the slow axis in memory, so the block writes the limbs and B to LDS
// token-contiguous ("transposed"): limbT[limb][p][j], BT[n][j].
#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 512;
constexpr int kMaxQ = 256;
constexpr int kMaxP = 64;
constexpr int kMaxN = 128;
constexpr int kRowPad = 16;                 // bytes; keeps 16-row b128 reads conflict-free
constexpr int kStride = kMaxQ + kRowPad;    // LDS row stride (bytes) for token-contiguous rows
constexpr float kMagic = 12582912.0f;       // 1.5 * 2^23: x + kMagic rounds x to an integer (ties to even)

__device__ __forceinline__ uint32_t pack_low_bytes(float a0, float a1, float a2, float a3) {
  const uint32_t p01 = __builtin_amdgcn_perm(__float_as_uint(a1), __float_as_uint(a0), 0x0c0c0400u);
  const uint32_t p23 = __builtin_amdgcn_perm(__float_as_uint(a3), __float_as_uint(a2), 0x0c0c0400u);
  return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
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

__device__ __forceinline__ float sbyte(uint32_t w, int i) {
  return float(int32_t(w << (24 - 8 * i)) >> 24);
}

__global__ void __launch_bounds__(kThreads) chunk_state_kernel(
    const int8_t* __restrict__ x, const float* __restrict__ x_scale, const int8_t* __restrict__ Bm,
    const float* __restrict__ B_scale, const float* __restrict__ dt, const float* __restrict__ acs,
    float* __restrict__ states, int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate,
    int32_t ngroups, int32_t chunk, int32_t nchunks) {
  __shared__ __attribute__((aligned(16))) uint8_t limbT[3][kMaxP][kStride];
  __shared__ __attribute__((aligned(16))) uint8_t BT[kMaxN][kStride];
  __shared__ float omega[kMaxQ];
  __shared__ float red[kThreads / kWave];

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

  // ---- per-token weights w_j = exp(Acs_last - Acs_j) dt_j and their power-of-two scale
  const float* acs_c = acs + ((int64_t(b) * nheads + h) * nchunks + c) * chunk;
  const float acs_last = acs_c[len - 1];
  float w = 0.f;
  if (tid < Q && tid < len) {
    const float d = dt[(int64_t(b) * seqlen + t0 + tid) * nheads + h];
    w = __expf(acs_last - acs_c[tid]) * d;
  }
  const float wm = wave_max(w);
  if (lane == 0) red[wave] = wm;
  __syncthreads();
  float wmax = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) wmax = fmaxf(wmax, red[i]);
  const int e = ceil_log2_pos(wmax);
  if (tid < Q) omega[tid] = w * exp2i(-e);
  __syncthreads();

  // ---- limbs of X_scaled / 2^e, written token-contiguous: limbT[k][p][j]
  // task = (4 tokens) x (4 channels); channels fastest so a wave's loads cover whole x rows
  const int pq_n = P / 4, jq_n = Q / 4;
  const int8_t* xb = x + ((int64_t(b) * seqlen + t0) * nheads + h) * P;
  const int64_t xrow = int64_t(nheads) * P;
  for (int task = tid; task < pq_n * jq_n; task += kThreads) {
    const int pq = task % pq_n, jq = task / pq_n;
    float t[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * jq + r;
      uint32_t wx = 0;
      if (j < len) wx = *reinterpret_cast<const uint32_t*>(xb + int64_t(j) * xrow + 4 * pq);
      const float om = omega[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) t[r][i] = om * sbyte(wx, i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a1[4], a2[4], a3[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float tt = t[r][i];
        a1[r] = tt + kMagic;                       // l1 in the low mantissa bits
        const float l1 = a1[r] - kMagic;
        const float d1 = (tt - l1) * 128.f;        // exact
        a2[r] = d1 + kMagic;
        const float l2 = a2[r] - kMagic;
        const float d2 = (d1 - l2) * 128.f;        // exact
        a3[r] = d2 + kMagic;
      }
      const int p = 4 * pq + i;
      *reinterpret_cast<uint32_t*>(&limbT[0][p][4 * jq]) = pack_low_bytes(a1[0], a1[1], a1[2], a1[3]);
      *reinterpret_cast<uint32_t*>(&limbT[1][p][4 * jq]) = pack_low_bytes(a2[0], a2[1], a2[2], a2[3]);
      *reinterpret_cast<uint32_t*>(&limbT[2][p][4 * jq]) = pack_low_bytes(a3[0], a3[1], a3[2], a3[3]);
    }
  }

  // ---- B codes of the chunk, token-contiguous: BT[n][j]
  const int nq_n = N / 4;
  const int8_t* Bb = Bm + ((int64_t(b) * seqlen + t0) * ngroups + g) * N;
  const int64_t brow = int64_t(ngroups) * N;
  for (int task = tid; task < nq_n * jq_n; task += kThreads) {
    const int nq = task % nq_n, jq = task / nq_n;
    uint32_t in[4], out[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * jq + r;
      in[r] = (j < len) ? *reinterpret_cast<const uint32_t*>(Bb + int64_t(j) * brow + 4 * nq) : 0u;
    }
    transpose4x4(in, out);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(&BT[4 * nq + i][4 * jq]) = out[i];
  }
  __syncthreads();

  // ---- S[p, n] tiles of 16 x 16: 3 limb accumulators each, K = tokens in steps of 64
  const float post = x_scale[h] * B_scale[g] * exp2i(e);
  float* Sc = states + ((int64_t(b) * nchunks + c) * nheads + h) * int64_t(P) * N;
  const int ptn = P / 16, ntn = N / 16;
  const int row = lane % 16, kg = lane / 16;
  for (int tile = wave; tile < ptn * ntn; tile += kThreads / kWave) {
    const int pt = tile % ptn, nt = tile / ptn;
    v4i acc1 = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0}, acc3 = {0, 0, 0, 0};
    for (int kb = 0; kb < Q; kb += 64) {
      const int col = kb + 16 * kg;
      const v4i bop = *reinterpret_cast<const v4i*>(&BT[nt * 16 + row][col]);
      const v4i a1 = *reinterpret_cast<const v4i*>(&limbT[0][pt * 16 + row][col]);
      const v4i a2 = *reinterpret_cast<const v4i*>(&limbT[1][pt * 16 + row][col]);
      const v4i a3 = *reinterpret_cast<const v4i*>(&limbT[2][pt * 16 + row][col]);
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bop, acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, bop, acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, bop, acc3, 0, 0, 0);
    }
    // D layout of a 16x16 MFMA: lane holds rows 4*(lane/16) + i, column lane % 16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = pt * 16 + 4 * kg + i;
      const int n = nt * 16 + row;
      const float v = (float(acc1[i]) + float(acc2[i]) * (1.f / 128.f) + float(acc3[i]) * (1.f / 16384.f)) * post;
      Sc[int64_t(p) * N + n] = v;
    }
  }
}

}  // namespace

hipError_t launch_chunk_state(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  const int nblocks = s.batch * s.nchunks * s.nheads;
  hipLaunchKernelGGL(chunk_state_kernel, dim3(nblocks), dim3(kThreads), 0, stream, a.x, a.x_scale, a.B, a.B_scale,
                     a.dt, a.acs, a.states, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk,
                     s.nchunks);
  return hipGetLastError();
}

}  // namespace ssdq
