// Stage 2 of the chunked SSD scan: carry the state across chunks,
//
//   H_0 = h0 (or 0);   Hprev_c = H_c;   H_{c+1} = exp(Acs[c, last]) H_c + S_c;   h_final = H_nc
//
// i.e. the recurrence h_t = exp(dt_t A) h_{t-1} + ... of the pages applied once per chunk
// with the chunk's total decay.  Sequential over chunks, parallel over (batch, head, state
// element); each chunk state S_c is overwritten in place by Hprev_c, the state entering
// chunk c, which the output stage reads.  HBM-bound: 4 bytes read + 4 written per element
// per chunk, with the next chunk's load issued before the current one is stored.
#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 256;
constexpr int kPerBlock = kThreads * 4;

__global__ void __launch_bounds__(kThreads) state_passing_kernel(float* __restrict__ states,
                                                                 const float* __restrict__ acs,
                                                                 const float* h0,  // may alias h_final
                                                                 float* h_final, int64_t seqlen,
                                                                 int32_t nheads, int32_t pn, int32_t chunk,
                                                                 int32_t nchunks, int32_t blocks_per_bh) {
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = bid / blocks_per_bh;
  const int part = bid % blocks_per_bh;
  const int h = bh % nheads;
  const int b = bh / nheads;
  const int e = part * kPerBlock + threadIdx.x * 4;
  if (e >= pn) return;

  float4 H = make_float4(0.f, 0.f, 0.f, 0.f);
  if (h0) H = *reinterpret_cast<const float4*>(h0 + int64_t(bh) * pn + e);
  const float* acs_bh = acs + int64_t(bh) * nchunks * chunk;
  const int64_t cstride = int64_t(nheads) * pn;  // between consecutive chunks of one (b, h)
  float* S = states + (int64_t(b) * nchunks * nheads + h) * pn + e;

  float4 s_next = *reinterpret_cast<const float4*>(S);
  for (int c = 0; c < nchunks; ++c) {
    const float4 s = s_next;
    if (c + 1 < nchunks) s_next = *reinterpret_cast<const float4*>(S + (c + 1) * cstride);
    const int64_t rem = seqlen - int64_t(c) * chunk;
    const int last = int(rem < chunk ? rem : chunk) - 1;
    const float decay = __expf(acs_bh[int64_t(c) * chunk + last]);
    *reinterpret_cast<float4*>(S + c * cstride) = H;
    H.x = decay * H.x + s.x;
    H.y = decay * H.y + s.y;
    H.z = decay * H.z + s.z;
    H.w = decay * H.w + s.w;
  }
  if (h_final) *reinterpret_cast<float4*>(h_final + int64_t(bh) * pn + e) = H;
}

}  // namespace

hipError_t launch_state_passing(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  const int pn = s.headdim * s.dstate;
  const int per_bh = (pn + kPerBlock - 1) / kPerBlock;
  const int nblocks = s.batch * s.nheads * per_bh;
  hipLaunchKernelGGL(state_passing_kernel, dim3(nblocks), dim3(kThreads), 0, stream, a.states, a.acs, a.h0,
                     a.h_final, s.seqlen, s.nheads, pn, s.chunk, s.nchunks, per_bh);
  return hipGetLastError();
}

}  // namespace ssdq
