// Static INT8 quantizer for the SSD inputs x, B, C (Quamba2 rebuttal: 8-bit SSD
// inputs; SSDi8 Table 10: one static scale per head for x and per state group
// for B and C).  code = clamp(rint(float(v) / s), -127, 127), the quotient
// correctly rounded, NaN -> 0.
//
// HBM-bound elementwise pass: 2 bytes in, 1 byte out per element.  Each thread
// handles 8 consecutive elements: one 16-byte load and one 8-byte store.
#include "ssdq_internal.h"

namespace ssdq {
namespace {

__device__ __forceinline__ uint32_t code_of(float v, float s) {
  const float t = __fdiv_rn(v, s);   // IEEE-correct fp32 division, no reciprocal shortcut
  if (t != t) return 0u;             // NaN
  float r = rintf(t);                // round to nearest, ties to even
  r = fminf(fmaxf(r, -127.f), 127.f);
  return uint32_t(int32_t(r)) & 0xffu;
}

// inner % 8 == 0: the 8 elements of a thread share one scale.
__global__ void __launch_bounds__(256) quantize_vec8(const v4u* __restrict__ x, v2u* __restrict__ q,
                                                     const float* __restrict__ scale, int64_t nvec,
                                                     int32_t nscale, int32_t inner_vec) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const int k = int((i / inner_vec) % nscale);
    const float s = scale[k];
    const v4u raw = __builtin_nontemporal_load(x + i);
    const uint32_t w[4] = {raw[0], raw[1], raw[2], raw[3]};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 h0 = __builtin_bit_cast(_Float16, uint16_t(w[e] & 0xffffu));
      const _Float16 h1 = __builtin_bit_cast(_Float16, uint16_t(w[e] >> 16));
      const uint32_t c = code_of(float(h0), s) | (code_of(float(h1), s) << 8);
      if (e < 2) lo |= c << (16 * e);
      else hi |= c << (16 * (e - 2));
    }
    __builtin_nontemporal_store(v2u{lo, hi}, q + i);
  }
}

// Any inner: one element per iteration (used for shapes whose rows are not 8-element aligned,
// and for the < 8 trailing elements of the vector kernel).
__global__ void __launch_bounds__(256) quantize_scalar(const uint16_t* __restrict__ x, int8_t* __restrict__ q,
                                                       const float* __restrict__ scale, int64_t begin,
                                                       int64_t n, int32_t nscale, int32_t inner) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t e = begin + int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) {
    const int k = int((e / inner) % nscale);
    const _Float16 h = __builtin_bit_cast(_Float16, x[e]);
    q[e] = int8_t(code_of(float(h), scale[k]));
  }
}

int grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  const int64_t cap = 256 * 64;  // enough blocks to fill 256 CUs; grid-stride beyond that
  if (g > cap) g = cap;
  return int(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_quantize(const uint16_t* x, int8_t* q, const float* scale, int64_t rows, int32_t nscale,
                           int32_t inner, hipStream_t stream) {
  const int64_t n = rows * int64_t(nscale) * inner;
  if (n == 0) return hipSuccess;
  int64_t done = 0;
  if (inner % 8 == 0) {
    const int64_t nvec = n / 8;
    hipLaunchKernelGGL(quantize_vec8, dim3(grid_for(nvec, 256)), dim3(256), 0, stream,
                       reinterpret_cast<const v4u*>(x), reinterpret_cast<v2u*>(q), scale, nvec, nscale,
                       inner / 8);
    done = nvec * 8;
  }
  if (done < n) {
    hipLaunchKernelGGL(quantize_scalar, dim3(grid_for(n - done, 256)), dim3(256), 0, stream, x, q, scale, done,
                       n, nscale, inner);
  }
  return hipGetLastError();
}

}  // namespace ssdq
