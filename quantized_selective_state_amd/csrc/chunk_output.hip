// Stage 2 of the chunked SSD scan: the output of chunk c,
//
//   y[l, p] = sum_{j <= l} M[l, j] xhat[j, p]  +  exp(Acs_l) Chat_l . Hprev_c[p, :]  +  D xhat[l, p]
//   M[l, j] = (Chat_l . Bhat_j) exp(Acs_l - Acs_j) dt_j
//
// (the state-space-duality form: the masked "attention" C B^T inside a chunk plus the
// carried state read out by C; SSDi8 Figure 1b / Table 5: ChunkBMM C.B^T on INT8).
//
// One block (16 waves) per (batch, chunk, head); each wave owns one 16-row output block.
//  - G^T[j, l] = sum_n q_B[j, n] q_C[l, n] on v_mfma_i32_16x16x64_i8 (exact int32).
//  - Decay mask, SSDi8-style decoupled from the matrix products: for a 32-token block that
//    lies entirely before the 16 output rows l0..l0+15, exp(Acs_l - Acs_j) =
//    exp(Acs_l - Acs_l0) exp(Acs_l0 - Acs_j), both factors <= 1, so the per-element work is
//    G * w_j (w_j = exp(Acs_l0 - Acs_j) dt_j, once per token) and the row factor
//    u_l = exp(Acs_l - Acs_l0) is applied in the epilogue.  The block holding the diagonal
//    uses the exact per-element exp with the causal mask.
//  - The masked fragment, rounded to fp16 under a power-of-two guard, feeds the next product
//    as its B operand straight from registers: the fp16 MFMA's K slots are matched to the
//    rows the int32 fragment holds, and x^T is read from LDS in the same slot order.
//  - y^T += x^T M^T and y_off^T = Hprev C^T on v_mfma_f32_16x16x32_f16 (fp32 accumulation):
//    x codes are exact in fp16; Hprev arrives as fp16 with one power-of-two scale per row.
//  - LDS matrices use 16-byte-chunk XOR swizzles so that the transposing writes and the
//    MFMA operand reads are free of bank conflicts.
#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 1024;   // 16 waves: one 16-row output block each at chunk 256
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxQ = 256;
constexpr int kMaxP = 64;
constexpr int kMaxN = 128;
constexpr float kLog2e = 1.4426950408889634f;

// x^T: [p][j] fp16, 512-byte rows, 16-byte chunk c stored at c ^ xswz(p)
__device__ __forceinline__ int xswz(int p) { return (p & 15) ^ ((p >> 4) & 3); }
__device__ __forceinline__ int xpos(int p, int j) { return p * kMaxQ + ((((j >> 3) ^ xswz(p)) << 3) | (j & 7)); }
// B codes: [j][n] int8, 128-byte rows, chunk c stored at c ^ ((j >> 1) & 7)
__device__ __forceinline__ int bpos(int j, int byte) {
  return j * kMaxN + ((((byte >> 4) ^ ((j >> 1) & 7)) << 4) | (byte & 15));
}
// Hprev: [p][n] fp16, 256-byte rows, chunk c stored at c ^ (p & 15)
__device__ __forceinline__ int hpos(int p, int n) { return p * kMaxN + ((((n >> 3) ^ (p & 15)) << 3) | (n & 7)); }

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

// Four int8 codes (biased by 128, i.e. XORed with 0x80 per byte) -> four exact fp16 values:
// the fp16 with bits 0x64XX is 1024 + XX, so subtracting 1152 leaves the signed code.
__device__ __forceinline__ v4h codes_to_f16(uint32_t biased) {
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, biased, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, biased, 0x04030402u);
  const v2h off = {_Float16(-1152.f), _Float16(-1152.f)};
  const v2h a = __builtin_bit_cast(v2h, lo) + off;
  const v2h b = __builtin_bit_cast(v2h, hi) + off;
  return v4h{a[0], a[1], b[0], b[1]};
}

__global__ void __launch_bounds__(kThreads) chunk_output_kernel(
    const int8_t* __restrict__ x, const float* __restrict__ x_scale, const int8_t* __restrict__ Bm,
    const float* __restrict__ B_scale, const int8_t* __restrict__ Cm, const float* __restrict__ C_scale,
    const float* __restrict__ dt, const float* __restrict__ D, const float* __restrict__ acs,
    const _Float16* __restrict__ hprev, const float* __restrict__ hscale, _Float16* __restrict__ y,
    int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups, int32_t chunk,
    int32_t nchunks) {
  __shared__ __attribute__((aligned(16))) _Float16 xT[kMaxP * kMaxQ];
  __shared__ __attribute__((aligned(16))) int8_t Bs[kMaxQ * kMaxN];
  __shared__ __attribute__((aligned(16))) _Float16 Hh[kMaxP * kMaxN];
  __shared__ __attribute__((aligned(16))) float hsc[kMaxP];
  __shared__ __attribute__((aligned(16))) float acs2[kMaxQ];   // Acs * log2(e)
  __shared__ __attribute__((aligned(16))) float dts[kMaxQ];    // dt * 2^-kM
  __shared__ __attribute__((aligned(16))) float wl[kWaves][kMaxQ];
  __shared__ float red[kWaves];

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

  // All products run on the zero-padded 64-channel x 128-state tile space; the loads below
  // use clamped addresses and selects (no load sits behind a branch), the stores of padded
  // rows and columns are skipped.

  // ---- per-token decay log and dt
  const float* acs_c = acs + ((int64_t(b) * nheads + h) * nchunks + c) * chunk;
  float dtv = 0.f;
  if (tid < kMaxQ) {
    const int t = min(tid, Q - 1);
    const float av = acs_c[t];
    const float dv = dt[(int64_t(b) * seqlen + t0 + min(t, len - 1)) * nheads + h];
    if (tid < Q) acs2[tid] = av * kLog2e;
    dtv = (tid < len) ? dv : 0.f;
  }
  {
    const float dm = wave_max(dtv);
    if (lane == 0) red[wave] = dm;
  }
  // ---- B codes: row-major [token][state], 8 chunks of 16 bytes per row
  {
    const int8_t* Bb = Bm + ((int64_t(b) * seqlen + t0) * ngroups + g) * N;
#pragma unroll
    for (int it = 0; it < kMaxQ * 8 / kThreads; ++it) {
      const int task = tid + it * kThreads;
      const int j = task >> 3, sg = task & 7;
      const bool ok = j < len && 16 * sg < N;
      const v4u v = *reinterpret_cast<const v4u*>(Bb + int64_t(min(j, len - 1)) * ngroups * N +
                                                  (16 * sg < N ? 16 * sg : 0));
      const v4u z = {0u, 0u, 0u, 0u};
      if (j < Q) *reinterpret_cast<v4u*>(Bs + bpos(j, 16 * sg)) = ok ? v : z;
    }
  }
  // ---- Hprev (fp16) and its per-row scales
  {
    const _Float16* Hb = hprev + ((int64_t(b) * nchunks + c) * nheads + h) * int64_t(P) * N;
#pragma unroll
    for (int it = 0; it < kMaxP * 16 / kThreads; ++it) {
      const int task = tid + it * kThreads;
      const int p = task >> 4, sg = task & 15;
      const bool ok = p < P && 8 * sg < N;
      const v4u v = *reinterpret_cast<const v4u*>(Hb + int64_t(min(p, P - 1)) * N + (8 * sg < N ? 8 * sg : 0));
      const v4u z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<v4u*>(Hh + hpos(p, 8 * sg)) = ok ? v : z;
    }
    if (tid < kMaxP) {
      const float sv = hscale[((int64_t(b) * nchunks + c) * nheads + h) * P + min(tid, P - 1)];
      hsc[tid] = tid < P ? sv : 0.f;
    }
  }
  // ---- x codes as exact fp16, token-contiguous: xT[p][j]
  {
    const int8_t* xb = x + ((int64_t(b) * seqlen + t0) * nheads + h) * P;
    const int ntasks = 16 * (Q / 4);
#pragma unroll
    for (int it = 0; it < 16 * (kMaxQ / 4) / kThreads; ++it) {
      const int task = tid + it * kThreads;
      const int pq = task & 15, jq = task >> 4;
      const bool chan_ok = 4 * pq < P;
      uint32_t in[4], out[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * jq + r;
        const uint32_t v = *reinterpret_cast<const uint32_t*>(xb + int64_t(min(j, len - 1)) * nheads * P +
                                                              (chan_ok ? 4 * pq : 0));
        in[r] = ((chan_ok && j < len) ? v : 0u) ^ 0x80808080u;
      }
      transpose4x4(in, out);
      if (task < ntasks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<v4h*>(xT + xpos(4 * pq + i, 4 * jq)) = codes_to_f16(out[i]);
      }
    }
  }
  __syncthreads();

  float dtmax = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) dtmax = fmaxf(dtmax, red[i]);
  // |M'| <= N 127^2 dtmax 2^-kM <= 2^15; clamped so that 2^kM and 2^-kM are exact
  const int kM = min(max(ceil_log2_pos(float(N) * 16129.f * dtmax) - 15, -120), 120);
  if (tid < kMaxQ) dts[tid] = dtv * exp2i(-kM);
  __syncthreads();

  // ---- one 16-row output block per wave
  const int l0 = 16 * wave;
  if (l0 >= Q) return;
  const int lcol = lane % 16, kg = lane / 16;
  const float sx = x_scale[h], sB = B_scale[g], sC = C_scale[g];
  const float Dh = D ? D[h] : 0.f;
  const float s_in = sx * sC * sB * exp2i(kM);
  const int l = l0 + lcol;
  const bool lvalid = l < len;
  const int8_t* Crow = Cm + ((int64_t(b) * seqlen + t0 + min(l, len - 1)) * ngroups + g) * N;
  const int jdiag = l0 & ~31;          // the 32-token block that holds the diagonal
  const float a_l = acs2[l];
  const float a_0 = acs2[l0];
  float* wlw = wl[wave];

  // weights of the blocks before the diagonal, relative to row l0
  for (int j = lane; j < jdiag; j += kWave) wlw[j] = exp2f(a_0 - acs2[j]) * dts[j];
  __builtin_amdgcn_wave_barrier();
  const float u_l = exp2f(a_l - a_0);

  // C row of this lane's output token: int8 K-slices for C.B^T, fp16 K-slices for Hprev.C^T
  v4i cq[2];
  v8h cop[4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int off = 64 * s + 16 * kg;
    const v4i v = *reinterpret_cast<const v4i*>(Crow + (off < N ? off : 0));
    cq[s] = (lvalid && off < N) ? v : v4i{0, 0, 0, 0};
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int off = 32 * k + 8 * kg;
    const v2u v = *reinterpret_cast<const v2u*>(Crow + (off < N ? off : 0));
    const v2u raw = (lvalid && off < N) ? v : v2u{0u, 0u};
    const v4h c0 = codes_to_f16(raw[0] ^ 0x80808080u);
    const v4h c1 = codes_to_f16(raw[1] ^ 0x80808080u);
    cop[k] = v8h{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  }

  v4f yf[4], yd[4], yo[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    yf[pt] = v4f{0.f, 0.f, 0.f, 0.f};
    yd[pt] = v4f{0.f, 0.f, 0.f, 0.f};
    yo[pt] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  // carried state read out by C: y_off^T[p][l] = sum_n Hprev[p][n] q_C[l][n]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const v8h hop = *reinterpret_cast<const v8h*>(Hh + hpos(16 * pt + lcol, 32 * k + 8 * kg));
      yo[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hop, cop[k], yo[pt], 0, 0, 0);
    }
  }

  // intra-chunk part, 32 tokens per step: blocks before the diagonal use the factorized decay
  for (int jb = 0; jb < jdiag; jb += 32) {
    v4i gm[2];
    float4 w4[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int js = jb + 16 * sb;
      const v4i b0 = *reinterpret_cast<const v4i*>(Bs + bpos(js + lcol, 16 * kg));
      const v4i b1 = *reinterpret_cast<const v4i*>(Bs + bpos(js + lcol, 64 + 16 * kg));
      w4[sb] = *reinterpret_cast<const float4*>(&wlw[js + 4 * kg]);
      gm[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b0, cq[0], v4i{0, 0, 0, 0}, 0, 0, 0);
      gm[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b1, cq[1], gm[sb], 0, 0, 0);
    }
    v8h xop[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int p = 16 * pt + lcol;
      const v4h lo = *reinterpret_cast<const v4h*>(xT + xpos(p, jb + 4 * kg));
      const v4h hi = *reinterpret_cast<const v4h*>(xT + xpos(p, jb + 16 + 4 * kg));
      xop[pt] = v8h{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    v8h mop;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      mop[4 * sb + 0] = _Float16(float(gm[sb][0]) * w4[sb].x);
      mop[4 * sb + 1] = _Float16(float(gm[sb][1]) * w4[sb].y);
      mop[4 * sb + 2] = _Float16(float(gm[sb][2]) * w4[sb].z);
      mop[4 * sb + 3] = _Float16(float(gm[sb][3]) * w4[sb].w);
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) yf[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop[pt], mop, yf[pt], 0, 0, 0);
  }
  // the block holding the diagonal: exact per-element decay and the causal mask
  {
    const int jb = jdiag;
    v4i gm[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int js = min(jb + 16 * sb, Q - 16);
      const v4i b0 = *reinterpret_cast<const v4i*>(Bs + bpos(js + lcol, 16 * kg));
      const v4i b1 = *reinterpret_cast<const v4i*>(Bs + bpos(js + lcol, 64 + 16 * kg));
      gm[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b0, cq[0], v4i{0, 0, 0, 0}, 0, 0, 0);
      gm[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b1, cq[1], gm[sb], 0, 0, 0);
    }
    v8h mop;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int jq = min(jb + 16 * sb, Q - 16) + 4 * kg;
      const float4 a4 = *reinterpret_cast<const float4*>(&acs2[jq]);
      const float4 d4 = *reinterpret_cast<const float4*>(&dts[jq]);
      const float av[4] = {a4.x, a4.y, a4.z, a4.w};
      const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = jb + 16 * sb + 4 * kg + i;     // > l (masked) whenever the clamp applied
        const float m = float(gm[sb][i]) * exp2f(fminf(a_l - av[i], 0.f)) * dv[i];
        mop[4 * sb + i] = _Float16(j <= l ? m : 0.f);
      }
    }
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int p = 16 * pt + lcol;
      const int j1 = min(jb + 16, Q - 16);
      const v4h lo = *reinterpret_cast<const v4h*>(xT + xpos(p, jb + 4 * kg));
      const v4h hi = *reinterpret_cast<const v4h*>(xT + xpos(p, j1 + 4 * kg));
      const v8h xop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      yd[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, mop, yd[pt], 0, 0, 0);
    }
  }

  // ---- epilogue: lane holds y[l, 16 pt + 4 kg + i], i = 0..3
  const float s_off = exp2f(a_l) * sC;
  _Float16* yrow = y + ((int64_t(b) * seqlen + t0 + l) * nheads + h) * P;
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const float4 hs = *reinterpret_cast<const float4*>(&hsc[16 * pt + 4 * kg]);
    const float hv[4] = {hs.x, hs.y, hs.z, hs.w};
    v4h out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 16 * pt + 4 * kg + i;
      const float xd = float(xT[xpos(p, l)]) * sx * Dh;
      out[i] = _Float16((u_l * yf[pt][i] + yd[pt][i]) * s_in + yo[pt][i] * (s_off * hv[i]) + xd);
    }
    if (lvalid && 16 * pt + 4 * kg < P) *reinterpret_cast<v4h*>(yrow + 16 * pt + 4 * kg) = out;
  }
}

}  // namespace

hipError_t launch_chunk_output(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  const int nblocks = s.batch * s.nchunks * s.nheads;
  hipLaunchKernelGGL(chunk_output_kernel, dim3(nblocks), dim3(kThreads), 0, stream, a.x, a.x_scale, a.B, a.B_scale,
                     a.C, a.C_scale, a.dt, a.D, a.acs, a.hprev, a.hscale, a.y, s.seqlen, s.nheads, s.headdim,
                     s.dstate, s.ngroups, s.chunk, s.nchunks);
  return hipGetLastError();
}

}  // namespace ssdq
