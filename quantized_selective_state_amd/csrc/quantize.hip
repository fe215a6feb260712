// Static INT8 quantizer for the SSD inputs x, B, C (Quamba2 rebuttal: 8-bit SSD
// inputs; SSDi8 Table 10: one static scale per head for x and per state group
// for B and C).  code = clamp(rint(float(v) / s), -127, 127), the quotient
// correctly rounded, NaN -> 0.
//
// HBM-bound elementwise pass: 2 bytes in, 1 byte out per element.  The main kernel gives each
// thread 16 consecutive elements of one row (two 16-byte loads issued together, one 16-byte
// store), so that enough bytes are in flight to cover the memory latency.  Plain (cached)
// loads and stores: on MI355X they stream faster here than nontemporal ones.
//
// Exactness without a division per element: with r = rcp(s) (the hardware reciprocal, within
// 1 ulp) and the exact product y = v r (inside an fma), |y - v/s| <= 2^-23 |v/s|, and
// |fl(v/s) - v/s| <= 2^-24 |v/s|, so for |v/s| < 256 the two are within 2^-14.  rint(y) and
// rint(fl(v/s)) can only differ when a half-integer lies in between, i.e. when y is within
// 2^-13 of one; those (rare) elements, NaN and infinities take the exact division.  The fast
// code rounds through the binade of 1.5 * 2^23, where the float spacing is 1: fl(y + 1.5 * 2^23)
// = 1.5 * 2^23 + rint(y) (ties to even) for |y| < 2^22, and the integer image of that float is
// 0x4B400000 + rint(y), so the clamp to +-127 is one integer median and the code is the low
// byte.  Past 2^22 the sum is still monotonic in y and lands beyond either clamp bound, and from
// |v/s| >= 127 on both sides give +-127, so large values need no exact division either.
#include "ssdq_internal.h"

namespace ssdq {
namespace {

__device__ __forceinline__ uint32_t code_exact(float v, float s) {
  const float t = __fdiv_rn(v, s);   // IEEE-correct fp32 division
  if (t != t) return 0u;             // NaN
  float r = rintf(t);                // round to nearest, ties to even
  r = fminf(fmaxf(r, -127.f), 127.f);
  return uint32_t(int32_t(r)) & 0xffu;
}

constexpr float kRound = 12582912.f;        // 1.5 * 2^23
constexpr int32_t kRoundBits = 0x4B400000;  // its binary32 image

// fast code in the low byte of the result (the upper bytes are not cleared), and whether the
// exact division must decide this element: y within 2^-13 of a half-integer, NaN or infinity
// (their residual d is NaN or large)
__device__ __forceinline__ uint32_t code_fast(float v, float rcp, bool& slow) {
  const float t = fmaf(v, rcp, kRound);   // 1.5 * 2^23 + rint(v rcp)
  const float k = t - kRound;             // rint(v rcp), exact
  const float d = fmaf(v, rcp, -k);       // v rcp - k
  slow = !(fabsf(d) <= 0.5f - 1.0f / 8192.f);
  const int32_t b = __builtin_bit_cast(int32_t, t);
  return uint32_t(min(max(b, kRoundBits - 127), kRoundBits + 127));
}

// n codes of one scale: the fast path for all, the exact division only for the elements that
// need it, behind one branch for the n elements (a wave enters it only when one of its lanes
// has such an element)
template <int n>
__device__ __forceinline__ void codes(const float (&v)[n], float s, uint32_t (&c)[n]) {
  const float rcp = __builtin_amdgcn_rcpf(s);
  bool slow[n];
#pragma unroll
  for (int e = 0; e < n; ++e) c[e] = code_fast(v[e], rcp, slow[e]);
#pragma unroll
  for (int e = 0; e < n; ++e)
    if (slow[e]) c[e] = code_exact(v[e], s);
}

__device__ __forceinline__ void unpack8(v4u raw, float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = float(__builtin_bit_cast(_Float16, uint16_t(raw[e] & 0xffffu)));
    v[2 * e + 1] = float(__builtin_bit_cast(_Float16, uint16_t(raw[e] >> 16)));
  }
}

// the low bytes of c[0..3] in one word (v_perm_b32: selector bytes 0-3 take bytes of the second
// operand, 4-7 of the first, 0x0c gives zero)
__device__ __forceinline__ uint32_t pack4(const uint32_t* c) {
  const uint32_t lo = __builtin_amdgcn_perm(c[1], c[0], 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(c[3], c[2], 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// inner % 16 == 0: a thread quantizes 16 consecutive elements of one row (one scale index).
// Pair indices i < 2^31 (host-checked), so the scale index uses 32-bit invariant division.
__device__ __forceinline__ void quantize16(const v4u* __restrict__ x, v4u* __restrict__ q,
                                           const float* __restrict__ scale, uint32_t i, FastDiv by_inner,
                                           FastDiv by_nscale) {
  const v4u raw0 = x[2 * i];
  const v4u raw1 = x[2 * i + 1];
  const uint32_t row = fdiv(i, by_inner);
  const int k = int(row - fdiv(row, by_nscale) * by_nscale.d);
  float v[16];
  unpack8(raw0, *reinterpret_cast<float(*)[8]>(&v[0]));
  unpack8(raw1, *reinterpret_cast<float(*)[8]>(&v[8]));
  uint32_t c[16];
  codes(v, scale[k], c);
  q[i] = v4u{pack4(c), pack4(c + 4), pack4(c + 8), pack4(c + 12)};
}

__global__ void __launch_bounds__(256) quantize_vec16(const v4u* __restrict__ x, v4u* __restrict__ q,
                                                      const float* __restrict__ scale, uint32_t npair,
                                                      FastDiv by_inner, FastDiv by_nscale) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < npair; i += stride)
    quantize16(x, q, scale, i, by_inner, by_nscale);
}

// One scale per (k, i) (B or C with a scale per (group, state)): inner % 16 == 0, a thread's 16
// consecutive elements of one row take the 16 consecutive scales scale[k, i0 .. i0 + 15] (four
// 16-byte loads, cached: the scale table is small), each element its own reciprocal.
__global__ void __launch_bounds__(256) quantize_vec16_pc(const v4u* __restrict__ x, v4u* __restrict__ q,
                                                         const float* __restrict__ scale, uint32_t npair,
                                                         FastDiv by_inner, FastDiv by_nscale, int32_t inner) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < npair; i += stride) {
    const v4u raw0 = x[2 * i];
    const v4u raw1 = x[2 * i + 1];
    const uint32_t row = fdiv(i, by_inner);                        // (r, k) row of `inner` elements
    const uint32_t i0 = 16u * (i - row * by_inner.d);              // first inner index
    const uint32_t k = row - fdiv(row, by_nscale) * by_nscale.d;
    const v4f* sp = reinterpret_cast<const v4f*>(scale + int64_t(k) * inner + i0);
    float v[16], sv[16];
    unpack8(raw0, *reinterpret_cast<float(*)[8]>(&v[0]));
    unpack8(raw1, *reinterpret_cast<float(*)[8]>(&v[8]));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v4f s4 = sp[t];
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[4 * t + e] = s4[e];
    }
    uint32_t c[16];
    bool slow[16];
    bool any = false;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      c[e] = code_fast(v[e], __builtin_amdgcn_rcpf(sv[e]), slow[e]);
      any = any || slow[e];
    }
    if (any) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (slow[e]) c[e] = code_exact(v[e], sv[e]);
    }
    q[i] = v4u{pack4(c), pack4(c + 4), pack4(c + 8), pack4(c + 12)};
  }
}

// Any inner: one element per iteration, one scale per (k, i).
__global__ void __launch_bounds__(256) quantize_scalar_pc(const uint16_t* __restrict__ x, int8_t* __restrict__ q,
                                                          const float* __restrict__ scale, int64_t n, int32_t nscale,
                                                          int32_t inner) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) {
    const int64_t ki = e % (int64_t(nscale) * inner);   // k * inner + i
    const _Float16 h = __builtin_bit_cast(_Float16, x[e]);
    q[e] = int8_t(code_exact(float(h), scale[ki]));
  }
}

// Several tensors in one launch: job k owns the blocks block0 .. block0 + nblocks - 1 and walks
// its pairs grid-stride over them.
struct Job16 {
  const v4u* x;
  v4u* q;
  const float* scale;
  uint32_t npair, block0, nblocks;
  FastDiv by_inner, by_nscale;
};
struct Jobs16 {
  Job16 job[SSDQ_QUANTIZE_MAX_JOBS];
  int32_t count;
};

__global__ void __launch_bounds__(256) quantize_vec16_batch(const Jobs16 jobs) {
  int k = 0;   // the job of this block (uniform)
  for (int t = 1; t < jobs.count; ++t) k = blockIdx.x >= jobs.job[t].block0 ? t : k;
  const Job16& J = jobs.job[k];
  const uint32_t stride = J.nblocks * blockDim.x;
  for (uint32_t i = (blockIdx.x - J.block0) * blockDim.x + threadIdx.x; i < J.npair; i += stride)
    quantize16(J.x, J.q, J.scale, i, J.by_inner, J.by_nscale);
}

// inner % 8 == 0: the 8 elements of a thread share one scale index.
// Vector indices i < 2^31 (host-checked), so the scale index uses 32-bit invariant division.
__global__ void __launch_bounds__(256) quantize_vec8(const v4u* __restrict__ x, v2u* __restrict__ q,
                                                     const float* __restrict__ scale, uint32_t nvec,
                                                     FastDiv by_inner, FastDiv by_nscale) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const v4u raw = x[i];
    const uint32_t row = fdiv(i, by_inner);
    const int k = int(row - fdiv(row, by_nscale) * by_nscale.d);
    float v[8];
    unpack8(raw, v);
    uint32_t c[8];
    codes(v, scale[k], c);
    q[i] = v2u{pack4(c), pack4(c + 4)};
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
    q[e] = int8_t(code_exact(float(h), scale[k]));
  }
}

int grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  // one work unit per thread (a 16-element piece, say): at the benchmark's sizes a grid of
  // 2^14 grid-striding blocks was 5% slower than a block per 256 pieces; grid-stride only past
  // 2^22 blocks (so that a 32-bit grid stride stays below 2^30)
  const int64_t cap = int64_t(1) << 22;
  if (g > cap) g = cap;
  return int(g < 1 ? 1 : g);
}

// Front end of the SSD block fused with the quantizer: the depthwise causal convolution of
// width 4 over the tokens of every in-projection channel (channels x | B | C, zero before the
// first token) plus a bias, SiLU, the binary16 module output, and its static INT8 code written
// straight into the scan's x, B or C layout (the causal convolution the pages keep in FP16
// ahead of the SSD box: Quamba2 rebuttal Tables R6/R7, SSDi8 Table 16's Conv column).  One
// read of the fp16 activations and one write of the codes, instead of a convolution pass that
// writes fp16 and a quantize pass that reads it again.
//
// A lane owns kFeChannels = 4 consecutive channels (one 8-byte load per token) and walks a strip
// of kFeTokens = 16 tokens, keeping the three previous tokens in registers; only the three
// tokens before the strip are read twice (from L2: the neighbouring strip just read them).  All
// of the strip's loads are issued before any arithmetic.  The kernel is bound by its VALU work
// (two transcendentals per element for SiLU, then the code), so the lane is kept narrow: at 4
// channels it needs 80 VGPRs, six waves per SIMD to overlap that arithmetic with the loads (at
// 8 channels per lane, 125 VGPRs and four waves, it took 16% longer at the 8B-shaped layer).
// kCh fp16 values of one token: 8 -> one 16-byte word, 4 -> one 8-byte word
template <int kCh> struct ChVec;
template <> struct ChVec<8> { using T = v4u; };
template <> struct ChVec<4> { using T = v2u; };

template <int kCh>
__device__ __forceinline__ void unpack_ch(typename ChVec<kCh>::T raw, float (&v)[kCh]) {
#pragma unroll
  for (int e = 0; e < kCh / 2; ++e) {
    v[2 * e] = float(__builtin_bit_cast(_Float16, uint16_t(raw[e] & 0xffffu)));
    v[2 * e + 1] = float(__builtin_bit_cast(_Float16, uint16_t(raw[e] >> 16)));
  }
}

template <int kCh>
__global__ void __launch_bounds__(64) frontend_kernel(
    const uint16_t* __restrict__ xbc, const float* __restrict__ w, const float* __restrict__ bias,
    const float* __restrict__ x_scale, const float* __restrict__ B_scale, const float* __restrict__ C_scale,
    int8_t* __restrict__ qx, int8_t* __restrict__ qB, int8_t* __restrict__ qC, int64_t seqlen, int32_t HP,
    int32_t GN, int32_t P, int32_t N, int32_t nvec, int32_t vec_blocks, int32_t strips) {
  using VT = typename ChVec<kCh>::T;
  const int lb = xcd_remap(blockIdx.x, gridDim.x);
  const int strip = lb % strips;
  const int vb = (lb / strips) % vec_blocks;
  const int64_t b = lb / strips / vec_blocks;
  const int vec = vb * 64 + int(threadIdx.x);
  if (vec >= nvec) return;   // no barriers below
  const int C = HP + 2 * GN;
  const int ch0 = kCh * vec;
  const int64_t t0 = int64_t(strip) * kFeTokens;
  const int64_t t1 = min(t0 + kFeTokens, seqlen);
  int8_t* dst;
  int64_t stride;
  float s;
  if (ch0 < HP) {
    dst = qx + ch0;
    stride = HP;
    s = x_scale[ch0 / P];
  } else if (ch0 < HP + GN) {
    dst = qB + (ch0 - HP);
    stride = GN;
    s = B_scale[(ch0 - HP) / N];
  } else {
    dst = qC + (ch0 - HP - GN);
    stride = GN;
    s = C_scale[(ch0 - HP - GN) / N];
  }
  float tap[4][kCh], bi[kCh];
#pragma unroll
  for (int q = 0; q < kCh; ++q) {
    const v4f t = *reinterpret_cast<const v4f*>(w + int64_t(ch0) * 4 + 4 * q);
#pragma unroll
    for (int k = 0; k < 4; ++k) tap[k][q] = t[k];
  }
#pragma unroll
  for (int e = 0; e < kCh; ++e) bi[e] = bias ? bias[ch0 + e] : 0.f;
  const uint16_t* src = xbc + b * seqlen * C + ch0;
  float h1[kCh], h2[kCh], h3[kCh];   // tokens t - 1, t - 2, t - 3
  {
    VT raw[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int64_t t = t0 - 1 - j;
      raw[j] = t >= 0 ? *reinterpret_cast<const VT*>(src + t * C) : VT{};
    }
    unpack_ch<kCh>(raw[0], h1);
    unpack_ch<kCh>(raw[1], h2);
    unpack_ch<kCh>(raw[2], h3);
  }
  int8_t* out = dst + b * seqlen * stride;
  VT raw[kFeTokens];
#pragma unroll
  for (int u = 0; u < kFeTokens; ++u)
    raw[u] = t0 + u < t1 ? *reinterpret_cast<const VT*>(src + (t0 + u) * C) : VT{};
#pragma unroll
  for (int u = 0; u < kFeTokens; ++u) {   // fully unrolled; tokens past the strip are not stored
    float cur[kCh], a[kCh];
    unpack_ch<kCh>(raw[u], cur);
#pragma unroll
    for (int e = 0; e < kCh; ++e) {
      float v = fmaf(tap[0][e], h3[e], bi[e]);
      v = fmaf(tap[1][e], h2[e], v);
      v = fmaf(tap[2][e], h1[e], v);
      v = fmaf(tap[3][e], cur[e], v);
      const float silu = v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
      a[e] = float(_Float16(silu));   // the module's binary16 output (round to nearest even)
      h3[e] = h2[e];
      h2[e] = h1[e];
      h1[e] = cur[e];
    }
    uint32_t c[kCh];
    codes<kCh>(a, s, c);
    if (t0 + u < t1) {
      if constexpr (kCh == 8)
        *reinterpret_cast<v2u*>(out + (t0 + u) * stride) = v2u{pack4(c), pack4(c + 4)};
      else
        *reinterpret_cast<uint32_t*>(out + (t0 + u) * stride) = pack4(c);
    }
  }
}

// The front end for one decode token: the convolution's history is the caller's conv state,
// (batch, 3, channels) binary16 holding the inputs of tokens t-3, t-2, t-1; the step forms
// token t's output exactly as frontend_kernel does (same arithmetic, same order) and shifts
// the state in place to t-2, t-1, t.  A lane owns 8 channels of one sequence.
__global__ void __launch_bounds__(256) frontend_step_kernel(
    uint16_t* __restrict__ conv_state, const uint16_t* __restrict__ xbc, const float* __restrict__ w,
    const float* __restrict__ bias, const float* __restrict__ x_scale, const float* __restrict__ B_scale,
    const float* __restrict__ C_scale, int8_t* __restrict__ qx, int8_t* __restrict__ qB, int8_t* __restrict__ qC,
    int32_t HP, int32_t GN, int32_t P, int32_t N, int32_t nvec, int32_t batch) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(nvec) * batch) return;
  const int vec = int(i % nvec);
  const int64_t b = i / nvec;
  const int C = HP + 2 * GN;
  const int ch0 = 8 * vec;
  int8_t* dst;
  float s;
  if (ch0 < HP) {
    dst = qx + b * HP + ch0;
    s = x_scale[ch0 / P];
  } else if (ch0 < HP + GN) {
    dst = qB + b * GN + (ch0 - HP);
    s = B_scale[(ch0 - HP) / N];
  } else {
    dst = qC + b * GN + (ch0 - HP - GN);
    s = C_scale[(ch0 - HP - GN) / N];
  }
  uint16_t* st = conv_state + b * 3 * C + ch0;
  const v4u r3 = *reinterpret_cast<const v4u*>(st);           // t - 3
  const v4u r2 = *reinterpret_cast<const v4u*>(st + C);       // t - 2
  const v4u r1 = *reinterpret_cast<const v4u*>(st + 2 * C);   // t - 1
  const v4u r0 = *reinterpret_cast<const v4u*>(xbc + b * C + ch0);
  float h3[8], h2[8], h1[8], cur[8], a[8];
  unpack8(r3, h3);
  unpack8(r2, h2);
  unpack8(r1, h1);
  unpack8(r0, cur);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const v4f t = *reinterpret_cast<const v4f*>(w + int64_t(ch0) * 4 + 4 * q);
    const float bq = bias ? bias[ch0 + q] : 0.f;
    float v = fmaf(t[0], h3[q], bq);
    v = fmaf(t[1], h2[q], v);
    v = fmaf(t[2], h1[q], v);
    v = fmaf(t[3], cur[q], v);
    const float silu = v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
    a[q] = float(_Float16(silu));
  }
  uint32_t c[8];
  codes<8>(a, s, c);
  *reinterpret_cast<v2u*>(dst) = v2u{pack4(c), pack4(c + 4)};
  *reinterpret_cast<v4u*>(st) = r2;
  *reinterpret_cast<v4u*>(st + C) = r1;
  *reinterpret_cast<v4u*>(st + 2 * C) = r0;
}

// dt = softplus(dt_raw + dt_bias[h]) = max(v, 0) + log1p(exp(-|v|)), one element per thread
__global__ void __launch_bounds__(256) softplus_dt_kernel(const float* __restrict__ raw,
                                                          const float* __restrict__ dt_bias,
                                                          float* __restrict__ dt, int64_t n, int32_t H) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = raw[i] + (dt_bias ? dt_bias[i % H] : 0.f);
  dt[i] = fmaxf(v, 0.f) + log1pf(__expf(-fabsf(v)));
}

}  // namespace

hipError_t launch_quantize_batch(const ssdq_quantize_job* jobs, int32_t count, hipStream_t stream) {
  // jobs with 16-element rows share one launch, smallest first (their blocks are dispatched
  // first and finish under the large job); the others take their own launches
  int order[SSDQ_QUANTIZE_MAX_JOBS];
  int64_t size[SSDQ_QUANTIZE_MAX_JOBS];
  for (int k = 0; k < count; ++k) {
    order[k] = k;
    size[k] = jobs[k].rows * int64_t(jobs[k].nscale) * jobs[k].inner;
  }
  for (int a = 1; a < count; ++a)
    for (int k = a; k > 0 && size[order[k]] < size[order[k - 1]]; --k) {
      const int t = order[k];
      order[k] = order[k - 1];
      order[k - 1] = t;
    }
  Jobs16 p{};
  uint32_t blocks = 0;
  for (int a = 0; a < count; ++a) {
    const ssdq_quantize_job& j = jobs[order[a]];
    const int64_t n = size[order[a]];
    if (n == 0) continue;
    if (j.inner % 16 == 0 && n / 16 < (int64_t(1) << 31)) {
      const uint32_t npair = uint32_t(n / 16), nb = uint32_t(grid_for(npair, 256));
      p.job[p.count++] = Job16{static_cast<const v4u*>(j.x_f16), reinterpret_cast<v4u*>(j.q), j.scale, npair, blocks,
                               nb, make_fastdiv(uint32_t(j.inner / 16)), make_fastdiv(uint32_t(j.nscale))};
      blocks += nb;
    } else {
      const hipError_t e = launch_quantize(static_cast<const uint16_t*>(j.x_f16), j.q, j.scale, j.rows, j.nscale,
                                           j.inner, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (p.count > 0) hipLaunchKernelGGL(quantize_vec16_batch, dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, int8_t* q, const float* scale, int64_t rows, int32_t nscale,
                           int32_t inner, hipStream_t stream) {
  const int64_t n = rows * int64_t(nscale) * inner;
  if (n == 0) return hipSuccess;
  int64_t done = 0;
  if (inner % 16 == 0 && n / 16 < (int64_t(1) << 31)) {
    const int64_t npair = n / 16;
    hipLaunchKernelGGL(quantize_vec16, dim3(grid_for(npair, 256)), dim3(256), 0, stream,
                       reinterpret_cast<const v4u*>(x), reinterpret_cast<v4u*>(q), scale, uint32_t(npair),
                       make_fastdiv(uint32_t(inner / 16)), make_fastdiv(uint32_t(nscale)));
    done = npair * 16;
  } else if (inner % 8 == 0 && n / 8 < (int64_t(1) << 31)) {
    const int64_t nvec = n / 8;
    hipLaunchKernelGGL(quantize_vec8, dim3(grid_for(nvec, 256)), dim3(256), 0, stream,
                       reinterpret_cast<const v4u*>(x), reinterpret_cast<v2u*>(q), scale, uint32_t(nvec),
                       make_fastdiv(uint32_t(inner / 8)), make_fastdiv(uint32_t(nscale)));
    done = nvec * 8;
  }
  if (done < n) {
    hipLaunchKernelGGL(quantize_scalar, dim3(grid_for(n - done, 256)), dim3(256), 0, stream, x, q, scale, done,
                       n, nscale, inner);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_per_channel(const uint16_t* x, int8_t* q, const float* scale, int64_t rows,
                                      int32_t nscale, int32_t inner, hipStream_t stream) {
  const int64_t n = rows * int64_t(nscale) * inner;
  if (n == 0) return hipSuccess;
  if (inner % 16 == 0 && n / 16 < (int64_t(1) << 31)) {
    const int64_t npair = n / 16;
    hipLaunchKernelGGL(quantize_vec16_pc, dim3(grid_for(npair, 256)), dim3(256), 0, stream,
                       reinterpret_cast<const v4u*>(x), reinterpret_cast<v4u*>(q), scale, uint32_t(npair),
                       make_fastdiv(uint32_t(inner / 16)), make_fastdiv(uint32_t(nscale)), inner);
  } else {
    hipLaunchKernelGGL(quantize_scalar_pc, dim3(grid_for(n, 256)), dim3(256), 0, stream, x, q, scale, n, nscale,
                       inner);
  }
  return hipGetLastError();
}

hipError_t launch_frontend(const uint16_t* xbc, const float* conv_w, const float* conv_b, const float* x_scale,
                           const float* B_scale, const float* C_scale, const float* dt_raw, const float* dt_bias,
                           int8_t* x, int8_t* B, int8_t* C, float* dt, int32_t batch, int64_t seqlen,
                           int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups, hipStream_t stream) {
  const int32_t HP = nheads * headdim, GN = ngroups * dstate;
  const int32_t nvec = (HP + 2 * GN) / kFeChannels;
  const int32_t vec_blocks = (nvec + 63) / 64;
  const int32_t strips = int32_t((seqlen + kFeTokens - 1) / kFeTokens);
  const int32_t nblocks = batch * vec_blocks * strips;   // < 2^31 (host-checked)
  hipLaunchKernelGGL(frontend_kernel<kFeChannels>, dim3(nblocks), dim3(64), 0, stream, xbc, conv_w, conv_b, x_scale, B_scale,
                     C_scale, x, B, C, seqlen, HP, GN, headdim, dstate, nvec, vec_blocks, strips);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = int64_t(batch) * seqlen * nheads;
  hipLaunchKernelGGL(softplus_dt_kernel, dim3(uint32_t((n + 255) / 256)), dim3(256), 0, stream, dt_raw, dt_bias, dt,
                     n, nheads);
  return hipGetLastError();
}

hipError_t launch_frontend_step(uint16_t* conv_state, const uint16_t* xbc, const float* conv_w, const float* conv_b,
                                const float* x_scale, const float* B_scale, const float* C_scale,
                                const float* dt_raw, const float* dt_bias, int8_t* x, int8_t* B, int8_t* C,
                                float* dt, int32_t batch, int32_t nheads, int32_t headdim, int32_t dstate,
                                int32_t ngroups, hipStream_t stream) {
  const int32_t HP = nheads * headdim, GN = ngroups * dstate;
  const int32_t nvec = (HP + 2 * GN) / 8;
  const int64_t lanes = int64_t(nvec) * batch;
  hipLaunchKernelGGL(frontend_step_kernel, dim3(uint32_t((lanes + 255) / 256)), dim3(256), 0, stream, conv_state, xbc,
                     conv_w, conv_b, x_scale, B_scale, C_scale, x, B, C, HP, GN, headdim, dstate, nvec, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = int64_t(batch) * nheads;
  hipLaunchKernelGGL(softplus_dt_kernel, dim3(uint32_t((n + 255) / 256)), dim3(256), 0, stream, dt_raw, dt_bias, dt,
                     n, nheads);
  return hipGetLastError();
}

}  // namespace ssdq
