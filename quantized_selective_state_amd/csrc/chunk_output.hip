// Stage 3 of the chunked SSD scan: the output of chunk c,
//
//   y[l, p] = sum_{j <= l} M[l, j] xhat[j, p]  +  exp(Acs_l) Chat_l . Hprev_c[p, :]  +  D xhat[l, p]
//   M[l, j] = (Chat_l . Bhat_j) exp(Acs_l - Acs_j) dt_j
//
// (the state-space-duality form: the masked "attention" C B^T inside a chunk plus the
// carried state read out by C; SSDi8 Figure 1b / Table 5: ChunkBMM C.B^T on INT8).
//
// Per block (8 waves) = one (batch, chunk, head); each wave owns 16-row output blocks.
//  - G^T[j, l] = sum_n q_B[j, n] q_C[l, n]: v_mfma_i32_16x16x64_i8, exact int32.
//  - The decay mask and dt are applied to the accumulator fragment in registers and the
//    result, converted to fp16 with a power-of-two guard against overflow, is fed straight
//    into the next product as its B operand (no LDS round trip): the K slots of the fp16
//    MFMA are matched to the rows the int32 fragment holds, and the x operand is read from
//    LDS in the same slot order.
//  - y^T += x^T M^T and y_off^T = Hprev C^T: v_mfma_f32_16x16x32_f16 (fp32 accumulation),
//    x codes exact in fp16, Hprev scaled by a power of two and rounded to fp16.
//  - fp32 epilogue applies the scales, adds D x, rounds to fp16, stores 8-byte rows.
#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxQ = 256;
constexpr int kMaxP = 64;
constexpr int kMaxN = 128;
constexpr int kBStride = kMaxN + 16;      // bytes per token row of B codes in LDS
constexpr int kXStride = kMaxQ + 8;       // halves per channel row of x^T in LDS
constexpr int kHStride = kMaxN + 8;       // halves per channel row of Hprev in LDS

__device__ __forceinline__ float sbyte(uint32_t w, int i) {
  return float(int32_t(w << (24 - 8 * i)) >> 24);
}

__global__ void __launch_bounds__(kThreads) chunk_output_kernel(
    const int8_t* __restrict__ x, const float* __restrict__ x_scale, const int8_t* __restrict__ Bm,
    const float* __restrict__ B_scale, const int8_t* __restrict__ Cm, const float* __restrict__ C_scale,
    const float* __restrict__ dt, const float* __restrict__ D, const float* __restrict__ acs,
    const float* __restrict__ hprev, _Float16* __restrict__ y, int64_t seqlen, int32_t nheads, int32_t headdim,
    int32_t dstate, int32_t ngroups, int32_t chunk, int32_t nchunks) {
  __shared__ __attribute__((aligned(16))) int8_t Bs[kMaxQ][kBStride];
  __shared__ __attribute__((aligned(16))) _Float16 xT[kMaxP][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 Hh[kMaxP][kHStride];
  __shared__ __attribute__((aligned(16))) float acs_s[kMaxQ];
  __shared__ __attribute__((aligned(16))) float dts_s[kMaxQ];
  __shared__ float red[2][kWaves];

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
  const int NP = (N + 63) & ~63;   // K extent of the int8 product (zero padded)
  const int NH = (N + 31) & ~31;   // K extent of the fp16 product (zero padded)

  // ---- per-token decay log and dt; dt max -> power-of-two guard for M in fp16
  const float* acs_c = acs + ((int64_t(b) * nheads + h) * nchunks + c) * chunk;
  float dtv = 0.f;
  if (tid < Q) {
    acs_s[tid] = acs_c[tid];
    if (tid < len) dtv = dt[(int64_t(b) * seqlen + t0 + tid) * nheads + h];
  }
  // Hprev tile (P x N fp32) into registers: 16 floats per thread at most
  const float* Hsrc = hprev + ((int64_t(b) * nchunks + c) * nheads + h) * int64_t(P) * N;
  const int pn4 = P * N / 4;
  float4 hv[4];
  float hmax = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + k * kThreads;
    hv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (idx < pn4) hv[k] = *reinterpret_cast<const float4*>(Hsrc + 4 * idx);
    hmax = fmaxf(hmax, fmaxf(fmaxf(fabsf(hv[k].x), fabsf(hv[k].y)), fmaxf(fabsf(hv[k].z), fabsf(hv[k].w))));
  }
  {
    const float dm = wave_max(dtv);
    const float hm = wave_max(hmax);
    if (lane == 0) {
      red[0][wave] = dm;
      red[1][wave] = hm;
    }
  }

  // ---- B codes of the chunk, row-major, zero padded to NP columns and Q rows
  {
    const int segs = NP / 16;
    const int8_t* Bb = Bm + ((int64_t(b) * seqlen + t0) * ngroups + g) * N;
    for (int task = tid; task < Q * segs; task += kThreads) {
      const int j = task / segs, sg = task % segs;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (j < len && 16 * sg < N) v = *reinterpret_cast<const uint4*>(Bb + int64_t(j) * ngroups * N + 16 * sg);
      *reinterpret_cast<uint4*>(&Bs[j][16 * sg]) = v;
    }
  }
  // ---- x codes of the chunk as fp16, transposed: xT[p][j]
  {
    const int pq_n = P / 4, jq_n = Q / 4;
    const int8_t* xb = x + ((int64_t(b) * seqlen + t0) * nheads + h) * P;
    for (int task = tid; task < pq_n * jq_n; task += kThreads) {
      const int pq = task % pq_n, jq = task / pq_n;
      uint32_t wv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * jq + r;
        wv[r] = (j < len) ? *reinterpret_cast<const uint32_t*>(xb + int64_t(j) * nheads * P + 4 * pq) : 0u;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4h col;
#pragma unroll
        for (int r = 0; r < 4; ++r) col[r] = _Float16(sbyte(wv[r], i));
        *reinterpret_cast<v4h*>(&xT[4 * pq + i][4 * jq]) = col;
      }
    }
  }
  __syncthreads();

  float dtmax = red[0][0], hmx = red[1][0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) {
    dtmax = fmaxf(dtmax, red[0][i]);
    hmx = fmaxf(hmx, red[1][i]);
  }
  // |M'| <= N * 127^2 * dtmax * 2^-kM <= 2^15 ;  |Hprev| * 2^-eh <= 2^14
  // exponents clamped so that both 2^e and 2^-e are exact normal floats
  const int kM = min(max(ceil_log2_pos(float(N) * 16129.f * dtmax) - 15, -120), 120);
  const int eh = min(max(ceil_log2_pos(hmx) - 14, -120), 120);
  const float mscale = exp2i(-kM);
  const float hscale = exp2i(-eh);
  if (tid < Q) dts_s[tid] = dtv * mscale;
  // Hprev -> fp16 in LDS, zero padded to NH columns
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + k * kThreads;
    if (idx < pn4) {
      const int p = (4 * idx) / N, n = (4 * idx) % N;
      v4h hh;
      hh[0] = _Float16(hv[k].x * hscale);
      hh[1] = _Float16(hv[k].y * hscale);
      hh[2] = _Float16(hv[k].z * hscale);
      hh[3] = _Float16(hv[k].w * hscale);
      *reinterpret_cast<v4h*>(&Hh[p][n]) = hh;
    }
  }
  if (NH > N) {
    for (int idx = tid; idx < P * (NH - N); idx += kThreads) {
      const int p = idx / (NH - N), n = N + idx % (NH - N);
      Hh[p][n] = _Float16(0.f);
    }
  }
  __syncthreads();

  // ---- per-wave 16-row output blocks
  const int nlb = Q / 16;
  const int lcol = lane % 16, kg = lane / 16;
  const int ptn = P / 16;
  const float sx = x_scale[h], sB = B_scale[g], sC = C_scale[g];
  const float Dh = D ? D[h] : 0.f;
  const int8_t* Cb = Cm + ((int64_t(b) * seqlen + t0) * ngroups + g) * N;

  for (int pass = 0; pass < 2; ++pass) {
    const int lb = (pass == 0) ? wave : (2 * kWaves - 1 - wave);
    if (lb >= nlb || (pass == 1 && nlb <= kWaves)) continue;
    const int l0 = 16 * lb;
    const int l = l0 + lcol;
    const bool lvalid = l < len;
    const int8_t* Crow = Cb + int64_t(l) * ngroups * N;

    // C row of this lane's output token as int8 K-slices (for C.B^T) ...
    v4i cq[kMaxN / 64];
#pragma unroll
    for (int s = 0; s < kMaxN / 64; ++s) {
      cq[s] = v4i{0, 0, 0, 0};
      const int off = 64 * s + 16 * kg;
      if (64 * s < NP && lvalid && off < N) cq[s] = *reinterpret_cast<const v4i*>(Crow + off);
    }

    v4f yin[kMaxP / 16], yoff[kMaxP / 16];
#pragma unroll
    for (int pt = 0; pt < kMaxP / 16; ++pt) {
      yin[pt] = v4f{0.f, 0.f, 0.f, 0.f};
      yoff[pt] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    // ... and as fp16 K-slices (for Hprev.C^T)
    for (int kb = 0; kb < NH; kb += 32) {
      const int off = kb + 8 * kg;
      uint2 raw = make_uint2(0u, 0u);
      if (lvalid && off < N) raw = *reinterpret_cast<const uint2*>(Crow + off);
      v8h cop;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cop[i] = _Float16(sbyte(raw.x, i));
        cop[4 + i] = _Float16(sbyte(raw.y, i));
      }
#pragma unroll
      for (int pt = 0; pt < kMaxP / 16; ++pt) {
        if (pt < ptn) {
          const v8h hop = *reinterpret_cast<const v8h*>(&Hh[16 * pt + lcol][off]);
          yoff[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hop, cop, yoff[pt], 0, 0, 0);
        }
      }
    }

    const float acs_l = acs_s[l < Q ? l : Q - 1];
    for (int jb = 0; jb <= l0 + 15; jb += 32) {
      // G^T for the two 16-token sub-blocks of this 32-token K block
      v4i gm[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        gm[sb] = v4i{0, 0, 0, 0};
        const int js = jb + 16 * sb;
        if (js <= l0 + 15) {
#pragma unroll
          for (int s = 0; s < kMaxN / 64; ++s) {
            if (64 * s < NP) {
              const v4i bop = *reinterpret_cast<const v4i*>(&Bs[js + lcol][64 * s + 16 * kg]);
              gm[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bop, cq[s], gm[sb], 0, 0, 0);
            }
          }
        }
      }
      // decay mask + dt -> fp16 B operand; slot s holds token j(kg, s)
      v8h mop;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int jq = jb + 16 * sb + 4 * kg;
        const float4 aj = *reinterpret_cast<const float4*>(&acs_s[jq < Q ? jq : 0]);
        const float4 dj = *reinterpret_cast<const float4*>(&dts_s[jq < Q ? jq : 0]);
        const float av[4] = {aj.x, aj.y, aj.z, aj.w};
        const float dv[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = jq + i;
          float m = 0.f;
          if (j <= l && jq < Q) m = float(gm[sb][i]) * __expf(acs_l - av[i]) * dv[i];
          mop[4 * sb + i] = _Float16(m);
        }
      }
#pragma unroll
      for (int pt = 0; pt < kMaxP / 16; ++pt) {
        if (pt < ptn) {
          const v4h lo = *reinterpret_cast<const v4h*>(&xT[16 * pt + lcol][jb + 4 * kg]);
          const v4h hi = *reinterpret_cast<const v4h*>(&xT[16 * pt + lcol][jb + 16 + 4 * kg]);
          const v8h xop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          yin[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, mop, yin[pt], 0, 0, 0);
        }
      }
    }

    // ---- epilogue: lane holds y[l, 16 pt + 4 kg + i], i = 0..3
    if (lvalid) {
      const float s_in = sx * sC * sB * exp2i(kM);
      const float s_off = __expf(acs_l) * sC * exp2i(eh);
      _Float16* yrow = y + ((int64_t(b) * seqlen + t0 + l) * nheads + h) * P;
#pragma unroll
      for (int pt = 0; pt < kMaxP / 16; ++pt) {
        if (pt < ptn) {
          v4h out;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = 16 * pt + 4 * kg + i;
            const float xd = float(xT[p][l]) * sx * Dh;
            out[i] = _Float16(yin[pt][i] * s_in + yoff[pt][i] * s_off + xd);
          }
          *reinterpret_cast<v4h*>(yrow + 16 * pt + 4 * kg) = out;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_output(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  const int nblocks = s.batch * s.nchunks * s.nheads;
  hipLaunchKernelGGL(chunk_output_kernel, dim3(nblocks), dim3(kThreads), 0, stream, a.x, a.x_scale, a.B, a.B_scale,
                     a.C, a.C_scale, a.dt, a.D, a.acs, a.states, a.y, s.seqlen, s.nheads, s.headdim, s.dstate,
                     s.ngroups, s.chunk, s.nchunks);
  return hipGetLastError();
}

}  // namespace ssdq
