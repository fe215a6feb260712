// Decode: one step of the recurrence per sequence, state updated in place
// (the SSD update that the Quamba2 rebuttal names as the decode-time latency and
// memory bottleneck as batch grows, Tables R7/R8):
//
//   h[p, n] <- exp(dt A) h[p, n] + (dt xhat[p]) Bhat[n];    y[p] = sum_n Chat[n] h[p, n] + D xhat[p]
//
// HBM-bound: every state element is read once and written once (8 bytes) for ~6 flops.
// One block per (batch, head).  Thread t owns the 4 consecutive state columns 4 (t % (N/4))
// of rows t / (N/4) + R k (R = 1024 / N rows per pass), so each pass of the block covers a
// contiguous 4 KiB stretch with 16-byte loads.  Every load of the step is issued before any
// arithmetic (addresses of rows past headdim are clamped, so no load sits behind a branch),
// and y[p] is reduced across the N/4 lanes of row p with DPP row shifts (an in-row prefix
// sum; lane 15 of each 16-lane DPP row holds its row total, row_bcast15 joins two rows).
#include <type_traits>

#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float sbyte(uint32_t w, int i) {
  return float(int32_t(w << (24 - 8 * i)) >> 24);
}

template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false);
  return v + __int_as_float(moved);
}

// Sum over groups of LPR consecutive lanes (16 or 32); the total lands in the group's last lane.
template <int LPR>
__device__ __forceinline__ float group_sum_to_last_lane(float v) {
  v = dpp_add<0x111, 0xF>(v);   // row_shr:1
  v = dpp_add<0x112, 0xF>(v);   // row_shr:2
  v = dpp_add<0x114, 0xF>(v);   // row_shr:4
  v = dpp_add<0x118, 0xF>(v);   // row_shr:8   -> lane 15 of each row: row total
  if constexpr (LPR == 32) v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  return v;
}

// kSc, the scale layout: bit 0 (kPS) B_scale and C_scale hold one scale per (group, state)
// (ngroups x N) instead of one per group; bit 1 (kPC) x_scale holds one scale per (head, channel)
// (nheads x headdim) instead of one per head.
template <int N, int kSc>
__global__ void __launch_bounds__(kThreads) state_update_kernel(
    float* __restrict__ state, const int8_t* __restrict__ x, const float* __restrict__ x_scale,
    const int8_t* __restrict__ Bm, const float* __restrict__ B_scale, const int8_t* __restrict__ Cm,
    const float* __restrict__ C_scale, const float* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ D, const float* __restrict__ ycorr, _Float16* __restrict__ y, int32_t nheads,
    int32_t headdim, int32_t ngroups) {
  constexpr int kLanesPerRow = N / 4;
  constexpr int kRows = kThreads / kLanesPerRow;   // rows per pass
  constexpr int kPasses = 64 / kRows;              // headdim <= 64
  constexpr bool kPS = kSc & 1, kPC = (kSc & 2) != 0;
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bh % nheads;
  const int b = bh / nheads;
  const int g = h / (nheads / ngroups);
  const int tid = threadIdx.x;
  const int nq = tid % kLanesPerRow;
  const int r0 = tid / kLanesPerRow;
  const int P = headdim;

  float* st = state + int64_t(bh) * P * N;
  const int8_t* xr = x + int64_t(bh) * P;
  v4f hv[kPasses];
  int xq[kPasses];
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int p = min(r0 + kRows * k, P - 1);
    hv[k] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(st + int64_t(p) * N + 4 * nq));
  }
#pragma unroll
  for (int k = 0; k < kPasses; ++k) xq[k] = xr[min(r0 + kRows * k, P - 1)];
  float sxq[kPC ? kPasses : 1];   // kPC: the x scale of each of the lane's rows
  if constexpr (kPC) {
#pragma unroll
    for (int k = 0; k < kPasses; ++k) sxq[k] = x_scale[h * P + min(r0 + kRows * k, P - 1)];
  }
  const uint32_t bw = *reinterpret_cast<const uint32_t*>(Bm + (int64_t(b) * ngroups + g) * N + 4 * nq);
  const uint32_t cw = *reinterpret_cast<const uint32_t*>(Cm + (int64_t(b) * ngroups + g) * N + 4 * nq);
  const float d = dt[bh];
  const float a = __expf(d * A[h]);
  const float sx = kPC ? 1.f : x_scale[h];
  const float dx = d * sx;
  const float Dh = D ? D[h] : 0.f;
  const float Dsx = Dh * sx;
  float bh4[4], ch4[4];
  if constexpr (kPS) {
    const v4f sb4 = *reinterpret_cast<const v4f*>(B_scale + g * N + 4 * nq);
    const v4f sc4 = *reinterpret_cast<const v4f*>(C_scale + g * N + 4 * nq);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bh4[i] = sb4[i] * sbyte(bw, i);
      ch4[i] = sc4[i] * sbyte(cw, i);
    }
  } else {
    const float sB = B_scale[g], sC = C_scale[g];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bh4[i] = sB * sbyte(bw, i);
      ch4[i] = sC * sbyte(cw, i);
    }
  }

#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int p = r0 + kRows * k;
    const float xp = float(xq[k]);
    const float u = (kPC ? d * sxq[k] : dx) * xp;
    const float Dx = kPC ? Dh * sxq[k] : Dsx;
    v4f v = hv[k];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = a * v[i] + u * bh4[i];
    if (p < P) __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(st + int64_t(p) * N + 4 * nq));
    float part = ch4[0] * v[0] + ch4[1] * v[1] + ch4[2] * v[2] + ch4[3] * v[3];
    part = group_sum_to_last_lane<kLanesPerRow>(part);
    if (p < P && nq == kLanesPerRow - 1)
      y[int64_t(bh) * P + p] = _Float16(part + Dx * xp + (ycorr ? ycorr[h * P + p] : 0.f));
  }
}

// The same step with the state cached in IEEE binary16 (half the bytes of the fp32 state):
// thread t owns the 8 consecutive state columns 8 (t % (N/8)) of its rows (one 16-byte load
// and store per row), forms the update in fp32 from the cached value, reads y out of that
// update and stores it rounded to nearest binary16 (ties to even; past the format's range:
// inf).  y[p] is summed across the N/8 lanes of row p with DPP lane pairings.
template <int N, int kSc>
__global__ void __launch_bounds__(kThreads) state_update_f16_kernel(
    uint16_t* __restrict__ state, const int8_t* __restrict__ x, const float* __restrict__ x_scale,
    const int8_t* __restrict__ Bm, const float* __restrict__ B_scale, const int8_t* __restrict__ Cm,
    const float* __restrict__ C_scale, const float* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ D, const float* __restrict__ ycorr, _Float16* __restrict__ y, int32_t nheads,
    int32_t headdim, int32_t ngroups) {
  constexpr int kLanesPerRow = N / 8;               // 16 (N = 128) or 8 (N = 64)
  constexpr int kRows = kThreads / kLanesPerRow;    // rows per pass
  constexpr int kPasses = 64 / kRows;               // headdim <= 64
  constexpr bool kPS = kSc & 1, kPC = (kSc & 2) != 0;
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bh % nheads;
  const int b = bh / nheads;
  const int g = h / (nheads / ngroups);
  const int tid = threadIdx.x;
  const int nq = tid % kLanesPerRow;
  const int r0 = tid / kLanesPerRow;
  const int P = headdim;

  uint16_t* st = state + int64_t(bh) * P * N;
  const int8_t* xr = x + int64_t(bh) * P;
  v4u hv[kPasses];
  int xq[kPasses];
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int p = min(r0 + kRows * k, P - 1);   // rows past headdim: a clamped, unused load
    hv[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(st + int64_t(p) * N + 8 * nq));
  }
#pragma unroll
  for (int k = 0; k < kPasses; ++k) xq[k] = xr[min(r0 + kRows * k, P - 1)];
  float sxq[kPC ? kPasses : 1];   // kPC: the x scale of each of the lane's rows
  if constexpr (kPC) {
#pragma unroll
    for (int k = 0; k < kPasses; ++k) sxq[k] = x_scale[h * P + min(r0 + kRows * k, P - 1)];
  }
  const v2u bw = *reinterpret_cast<const v2u*>(Bm + (int64_t(b) * ngroups + g) * N + 8 * nq);
  const v2u cw = *reinterpret_cast<const v2u*>(Cm + (int64_t(b) * ngroups + g) * N + 8 * nq);
  const float d = dt[bh];
  const float a = __expf(d * A[h]);
  const float sx = kPC ? 1.f : x_scale[h];
  const float dx = d * sx;
  const float Dh = D ? D[h] : 0.f;
  const float Dsx = Dh * sx;
  float bh8[8], ch8[8];
  if constexpr (kPS) {
    const v4f* sbp = reinterpret_cast<const v4f*>(B_scale + g * N + 8 * nq);
    const v4f* scp = reinterpret_cast<const v4f*>(C_scale + g * N + 8 * nq);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bh8[i] = sbp[i >> 2][i & 3] * sbyte(bw[i >> 2], i & 3);
      ch8[i] = scp[i >> 2][i & 3] * sbyte(cw[i >> 2], i & 3);
    }
  } else {
    const float sB = B_scale[g], sC = C_scale[g];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bh8[i] = sB * sbyte(bw[i >> 2], i & 3);
      ch8[i] = sC * sbyte(cw[i >> 2], i & 3);
    }
  }

#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int p = r0 + kRows * k;
    const float xp = float(xq[k]);
    const float u = (kPC ? d * sxq[k] : dx) * xp;
    const float Dx = kPC ? Dh * sxq[k] : Dsx;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = hv[k][i >> 1];
      const float cached = float(__builtin_bit_cast(_Float16, uint16_t((i & 1) ? w >> 16 : w & 0xffffu)));
      v[i] = a * cached + u * bh8[i];
    }
    v4u out;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[j] = uint32_t(__builtin_bit_cast(uint16_t, _Float16(v[2 * j]))) |
               (uint32_t(__builtin_bit_cast(uint16_t, _Float16(v[2 * j + 1]))) << 16);
    if (p < P) __builtin_nontemporal_store(out, reinterpret_cast<v4u*>(st + int64_t(p) * N + 8 * nq));
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) part = fmaf(ch8[i], v[i], part);
    part = group_sum<kLanesPerRow>(part);
    if (p < P && nq == 0) y[int64_t(bh) * P + p] = _Float16(part + Dx * xp + (ycorr ? ycorr[h * P + p] : 0.f));
  }
}

// The same step on a state cached as 8-bit codes with one binary32 scale per state row (the
// 8-bit cached SSM states of the Quamba2 rebuttal, Tables R7/R8; one scale per row is the
// granularity chosen here): the row is decoded (scale times code), updated in fp32, y is read
// from the update, and the row is re-quantized with s = max|row| / 127 and codes rounded to
// nearest even.  A row of N codes is N/16 lanes with one 16-byte load each, so the row maximum
// and y's dot product are reductions over at most 8 neighbouring lanes (DPP, in registers).
//
// At 1 byte per element the step would be VALU-bound with a plain float loop, so:
//  - y needs no per-element float work: with u = (e s) q + (dt xhat sB) b (q the cached codes,
//    b the B codes, e = exp(dt A)), sum_n c_n u_n = (e s) <c, q> + (dt xhat sB) <c, b>, and
//    both dot products are over int8 codes: four-way int8 dot instructions, exact in int32;
//  - the new code is one fma into the binade of 1.5 * 2^23, whose unit spacing makes the fma's
//    own rounding the round-to-nearest-even of u / s and leaves the code in the low byte, and
//    byte permutes pack four codes per dword.
constexpr int kI8Threads = 128;   // two waves per (batch, head): four row passes per lane amortize the set-up

// kSc bit 0 (kPS): per-(group, state) B and C scales.  The B scale then goes into each state's B
// value and y is summed in fp32 over the C values scaled per state (the int8 dot products factor
// only with one C scale per row).  Bit 1 (kPC): x scales per (head, channel), one per state row.
template <int N, int kSc>
__global__ void __launch_bounds__(kI8Threads) state_update_i8_kernel(
    int8_t* __restrict__ state, float* __restrict__ state_scale, const int8_t* __restrict__ x,
    const float* __restrict__ x_scale, const int8_t* __restrict__ Bm, const float* __restrict__ B_scale,
    const int8_t* __restrict__ Cm, const float* __restrict__ C_scale, const float* __restrict__ dt,
    const float* __restrict__ A, const float* __restrict__ D, const float* __restrict__ ycorr,
    _Float16* __restrict__ y, int32_t nheads, int32_t headdim, int32_t ngroups) {
  constexpr int kLanesPerRow = N / 16;                 // 8 (N = 128) or 4 (N = 64)
  constexpr int kRows = kI8Threads / kLanesPerRow;     // rows per pass: 16 or 32
  constexpr int kPasses = (64 + kRows - 1) / kRows;    // headdim <= 64
  constexpr float kMagic = 12582912.f;                 // 1.5 * 2^23: unit spacing, code in the low byte
  constexpr bool kPS = kSc & 1, kPC = (kSc & 2) != 0;
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bh % nheads;
  const int b = bh / nheads;
  const int g = h / (nheads / ngroups);
  const int tid = threadIdx.x;
  const int nq = tid % kLanesPerRow;
  const int r0 = tid / kLanesPerRow;
  const int P = headdim;

  int8_t* st = state + int64_t(bh) * P * N;
  float* ss = state_scale + int64_t(bh) * P;
  const int8_t* xr = x + int64_t(bh) * P;
  v4u hv[kPasses];
  float so[kPasses];
  int xq[kPasses];
  float sxq[kPC ? kPasses : 1];   // kPC: the x scale of each of the lane's rows
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int p = min(r0 + kRows * k, P - 1);   // rows past headdim: a clamped, unused load
    hv[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(st + int64_t(p) * N + 16 * nq));
  }
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int p = min(r0 + kRows * k, P - 1);
    so[k] = ss[p];
    xq[k] = xr[p];
    if constexpr (kPC) sxq[k] = x_scale[h * P + p];
  }
  const v4u bw = *reinterpret_cast<const v4u*>(Bm + (int64_t(b) * ngroups + g) * N + 16 * nq);
  const v4u cw = *reinterpret_cast<const v4u*>(Cm + (int64_t(b) * ngroups + g) * N + 16 * nq);
  const float d = dt[bh];
  const float a = __expf(d * A[h]);
  const float sx = kPC ? 1.f : x_scale[h];
  const float dB = d * (kPS ? 1.f : B_scale[g]);
  const float dxB = d * sx * (kPS ? 1.f : B_scale[g]);
  const float Dh = D ? D[h] : 0.f;
  const float Dsx = Dh * sx;
  const float sC = kPS ? 1.f : C_scale[g];
  float bq[16];   // the B codes as floats (per group: the scale is applied per row; per state: included)
  float cf[kPS ? 16 : 1];   // per state: the C values sC[n] c_n
  if constexpr (kPS) {
    const v4f* sbp = reinterpret_cast<const v4f*>(B_scale + g * N + 16 * nq);
    const v4f* scp = reinterpret_cast<const v4f*>(C_scale + g * N + 16 * nq);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      bq[i] = sbp[i >> 2][i & 3] * sbyte(bw[i >> 2], i & 3);
      cf[i] = scp[i >> 2][i & 3] * sbyte(cw[i >> 2], i & 3);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) bq[i] = sbyte(bw[i >> 2], i & 3);
  }
  int cb = 0;     // <c, b> over this lane's 16 states (per group only)
  if constexpr (!kPS) {
#pragma unroll
    for (int j = 0; j < 4; ++j) cb = __builtin_amdgcn_sdot4(int(cw[j]), int(bw[j]), cb, false);
  }
  const float cbf = float(cb);

#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int p = r0 + kRows * k;
    const float xp = float(xq[k]);
    const float uB = (kPC ? dB * sxq[k] : dxB) * xp;   // dt xhat[p] sB
    const float Dx = kPC ? Dh * sxq[k] : Dsx;
    const float as = a * so[k];         // exp(dt A) times the cached row's scale
    float v[16];
    float m = 0.f;
    int cq = 0;                         // <c, q> over this lane's 16 cached codes (per group only)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (!kPS) cq = __builtin_amdgcn_sdot4(int(cw[j]), int(hv[k][j]), cq, false);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[4 * j + i] = fmaf(as, sbyte(hv[k][j], i), uB * bq[4 * j + i]);
        m = fmaxf(m, fabsf(v[4 * j + i]));
      }
    }
    m = group_max<kLanesPerRow>(m);
    // m / 127 by one fma refinement of m * (1/127) instead of a full IEEE division per lane and
    // row (equal to the correctly rounded quotient on every one of 2 M sampled m; at worst an
    // ulp from it, which moves a code only where u / s is that close to a midpoint)
    const float q0 = m * (1.f / 127.f);
    const float sq = fmaf(fmaf(-q0, 127.f, m), 1.f / 127.f, q0);
    // a scale below the normal range flushes the row (zero codes, s = 0); with s normal,
    // m / s <= 127 (1 + 2^-23) and the reciprocal's ulp keep every |u| inv below 127.5, so the
    // rounded codes need no clamp
    const float s = sq >= 0x1p-126f ? sq : 0.f;
    // 1 / s to within an ulp: a code can move only where u / s is that close to a midpoint
    const float inv = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
    v4u out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t t[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = fmaf(v[4 * j + i], inv, kMagic);
        t[i] = __float_as_uint(c);
      }
      const uint32_t lo = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u);   // bytes: t0.b0, t1.b0, 0, 0
      const uint32_t hi = __builtin_amdgcn_perm(t[3], t[2], 0x0c0c0400u);
      out[j] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);                   // lo.b0, lo.b1, hi.b0, hi.b1
    }
    if (p < P) __builtin_nontemporal_store(out, reinterpret_cast<v4u*>(st + int64_t(p) * N + 16 * nq));
    float part;
    if constexpr (kPS) {
      part = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) part = fmaf(cf[i], v[i], part);
    } else {
      part = fmaf(as, float(cq), uB * cbf);
    }
    part = group_sum<kLanesPerRow>(part);
    if (p < P && nq == 0) {
      ss[p] = s;
      y[int64_t(bh) * P + p] = _Float16(fmaf(sC, part, Dx * xp) + (ycorr ? ycorr[h * P + p] : 0.f));
    }
  }
}

// Calls go(kernel template instance) for the (dstate, scale layout) at hand; kernels are
// instantiated for dstate 64 and 128 and the four scale layouts.
template <template <int, int> class K, typename Go>
void dispatch(int32_t dstate, int32_t scales, Go&& go) {
  auto by_scales = [&](auto n) {
    constexpr int N = decltype(n)::value;
    switch (scales & 3) {
      case 0: go(K<N, 0>::fn); break;
      case 1: go(K<N, 1>::fn); break;
      case 2: go(K<N, 2>::fn); break;
      default: go(K<N, 3>::fn); break;
    }
  };
  if (dstate == 128)
    by_scales(std::integral_constant<int, 128>{});
  else
    by_scales(std::integral_constant<int, 64>{});
}
template <int N, int S>
struct F32 {
  static constexpr auto fn = state_update_kernel<N, S>;
};
template <int N, int S>
struct F16 {
  static constexpr auto fn = state_update_f16_kernel<N, S>;
};
template <int N, int S>
struct I8 {
  static constexpr auto fn = state_update_i8_kernel<N, S>;
};

}  // namespace

hipError_t launch_state_update_f16(uint16_t* state, const int8_t* x, const float* x_scale, const int8_t* B,
                                   const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                                   const float* A, const float* D, const float* ycorr, _Float16* y, int32_t batch,
                                   int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                                   hipStream_t stream, int32_t scales) {
  const int nblocks = batch * nheads;
  dispatch<F16>(dstate, scales, [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(nblocks), dim3(kThreads), 0, stream, state, x, x_scale, B, B_scale, C, C_scale,
                       dt, A, D, ycorr, y, nheads, headdim, ngroups);
  });
  return hipGetLastError();
}

hipError_t launch_state_update_i8(int8_t* state, float* state_scale, const int8_t* x, const float* x_scale,
                                  const int8_t* B, const float* B_scale, const int8_t* C, const float* C_scale,
                                  const float* dt, const float* A, const float* D, const float* ycorr, _Float16* y,
                                  int32_t batch, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                                  hipStream_t stream, int32_t scales) {
  const int nblocks = batch * nheads;
  dispatch<I8>(dstate, scales, [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(nblocks), dim3(kI8Threads), 0, stream, state, state_scale, x, x_scale, B, B_scale,
                       C, C_scale, dt, A, D, ycorr, y, nheads, headdim, ngroups);
  });
  return hipGetLastError();
}

hipError_t launch_state_update(float* state, const int8_t* x, const float* x_scale, const int8_t* B,
                               const float* B_scale, const int8_t* C, const float* C_scale, const float* dt,
                               const float* A, const float* D, const float* ycorr, _Float16* y, int32_t batch,
                               int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream,
                               int32_t scales) {
  const int nblocks = batch * nheads;
  dispatch<F32>(dstate, scales, [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(nblocks), dim3(kThreads), 0, stream, state, x, x_scale, B, B_scale, C, C_scale,
                       dt, A, D, ycorr, y, nheads, headdim, ngroups);
  });
  return hipGetLastError();
}

}  // namespace ssdq
