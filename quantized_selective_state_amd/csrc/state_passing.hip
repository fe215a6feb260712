// Stage 1 of the chunked SSD scan: carry the state across chunks,
//
//   H_0 = h0 (or 0);   H_{c+1} = exp(Acs[c, last]) H_c + S_c;   h_final = H_nc
//
// i.e. the recurrence h_t = exp(dt_t A) h_{t-1} + ... of the pages applied once per chunk
// with the chunk's total decay.  Sequential over chunks, parallel over (batch, head, state
// row).  The state entering chunk c, Hprev_c = H_c, is what the output stage reads; it is
// written as two INT8 limbs per element with one power-of-two scale 2^e per state row p
// (2 bytes per element, half of fp32; full 64-state blocks of a row dword-transposed), so that
// the output stage can read it out with C on
// the INT8 matrix cores: with t = H 2^-e (|t| <= 127) and V = trunc(256 t + 128),
// V = 256 l1 + (l2 + 128), so H = 2^e (l1 + l2 / 256) to within 2^e / 256.  The running
// state and h_final stay fp32.
//
// Thread layout: a state row of N floats is handled by LPR = next_pow2(N/4) lanes with
// 4 consecutive columns each, so the row max is a reduction inside the wave (DPP lane moves
// and a cross-row swap: no LDS traffic, hence no wait that would also drain the loads).
#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 256;
constexpr int kDepth = 4;   // chunks of states in flight per thread

template <int LPR>
__global__ void __launch_bounds__(kThreads) state_passing_kernel(
    const float* __restrict__ states, const float* __restrict__ acs, const float* h0,  // h0 may alias h_final
    float* h_final, int8_t* __restrict__ hprev, float* __restrict__ hscale, const float* __restrict__ C_scale_ps,
    int64_t seqlen, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups, int32_t chunk, int32_t nchunks,
    int32_t blocks_per_bh) {
  constexpr int lanes_per_row = LPR;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = bid / blocks_per_bh;
  const int part = bid % blocks_per_bh;
  const int h = bh % nheads;
  const int b = bh / nheads;
  const int P = headdim, N = dstate;
  const int rows_per_block = kThreads / lanes_per_row;
  const int p = part * rows_per_block + threadIdx.x / lanes_per_row;
  const int nq = threadIdx.x % lanes_per_row;
  const bool active = p < P && 4 * nq < N;
  const int64_t pn = int64_t(P) * N;
  const int64_t e = int64_t(p) * N + 4 * nq;
  // position of this lane's 4 states in a carried-state row: full 64-state blocks are stored
  // dword-transposed (states 64 blk + 16 t + 4 k + i at 64 blk + 16 k + 4 t + i)
  const int n0 = 4 * nq, blk = n0 >> 6, m = n0 & 63;
  const int64_t eh = int64_t(p) * N + (64 * blk + 64 <= N ? 64 * blk + 16 * ((m >> 2) & 3) + 4 * (m >> 4) : n0);
  const uint32_t eh_off = active ? uint32_t(eh) : kOutOfRange;

  // with B and C scales per (group, state) (C_scale_ps non-null) the chunk states arrive scaled by
  // the C scale of each state, and the running state is kept so (h0 scaled in, h_final scaled out)
  v4f sc = {1.f, 1.f, 1.f, 1.f};
  if (C_scale_ps && active) sc = *reinterpret_cast<const v4f*>(C_scale_ps + (h / (nheads / ngroups)) * N + 4 * nq);
  v4f H = {0.f, 0.f, 0.f, 0.f};
  if (active && h0) H = *reinterpret_cast<const v4f*>(h0 + int64_t(bh) * pn + e) * sc;
  const float* acs_bh = acs + int64_t(bh) * nchunks * chunk;
  const int64_t cstride = int64_t(nheads) * pn;  // between consecutive chunks of one (b, h)
  const int64_t base = (int64_t(b) * nchunks * nheads + h) * pn;

  // The chunk states are read kDepth chunks ahead (a ring of registers, the loop unrolled by
  // its depth so that every index is static): enough bytes in flight to cover the HBM latency
  // with the few blocks a small batch launches.  (Deeper rings measured slower: 8 chunks +8%,
  // 16 chunks +87% at a 2.7B-shaped layer.)  The chunks' Acs[c, last] come 64 at a time as
  // one vector load (lane k: chunk 64 i + k; the next 64 in flight) and are picked out with
  // readlane, so the loop holds no scalar load that a wait would have to drain.
  const int lane = int(threadIdx.x) % kWave;
  auto acs_last_of = [&](int c) -> float {   // per lane; 0 past the last chunk
    if (c >= nchunks) return 0.f;
    const int64_t rem = seqlen - int64_t(c) * chunk;
    const int last = int(rem < chunk ? rem : chunk) - 1;
    return acs_bh[int64_t(c) * chunk + last];
  };
  float acs_cur = acs_last_of(lane), acs_nxt = acs_last_of(kWave + lane);
  v4f ring[kDepth];
  // buffer loads: a scalar descriptor per chunk and one lane offset for all chunks, so that a
  // chunk in flight costs its four data registers only (chunks past the end and lanes past the
  // row load zeros)
  const uint32_t e_off = active ? uint32_t(e) * 4u : kOutOfRange;
  auto load_chunk = [&](int c, v4f& sv) {
    const Rsrc rs = make_rsrc(states + base + int64_t(c < nchunks ? c : 0) * cstride, c < nchunks ? uint32_t(pn) * 4u : 0u);
    sv = __builtin_bit_cast(v4f, buf_load16(rs, e_off));
  };
#pragma unroll
  for (int k = 0; k < kDepth; ++k) load_chunk(k, ring[k]);
  static_assert(kWave % kDepth == 0, "a group of 64 chunks starts at a ring boundary");
  for (int c0 = 0; c0 < nchunks; c0 += kDepth) {
    if (c0 > 0 && c0 % kWave == 0) {   // uniform: the next 64 chunks' Acs[c, last]
      acs_cur = acs_nxt;
      acs_nxt = acs_last_of(c0 + kWave + lane);
    }
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int c = c0 + k;
      if (c >= nchunks) break;   // uniform
      const v4f sv = ring[k];
      const float al = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acs_cur), c % kWave));
      const float decay = exp2f(al * 1.4426950408889634f);
      load_chunk(c + kDepth, ring[k]);
      // two INT8 limbs of H_c with a per-row power-of-two scale 2^ex >= row max / 127
      float m = fmaxf(fmaxf(fabsf(H[0]), fabsf(H[1])), fmaxf(fabsf(H[2]), fabsf(H[3])));
      m = group_max<LPR>(m);
      const int ex = min(max(ceil_log2_pos(m * (1.f / 127.f)), -120), 120);
      const float inv = exp2i(8 - ex);   // 256 / 2^ex
      {
        uint32_t q1 = 0, q2 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t V = int32_t(fmaf(H[i], inv, 128.f));   // 256 t + 128, |t| <= 127
          q1 |= (uint32_t(V >> 8) & 0xffu) << (8 * i);
          q2 |= ((uint32_t(V) & 0xffu) ^ 0x80u) << (8 * i);
        }
        // per (b, c, h): limb-1 plane [P][N] then limb-2 plane [P][N] (inactive lanes store to
        // an offset outside the buffer: dropped)
        const Rsrc rh = make_rsrc(hprev + 2 * (base + c * cstride), 2u * uint32_t(pn));
        __builtin_amdgcn_raw_buffer_store_b32(q1, rh, eh_off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(q2, rh, eh_off, int(pn), 0);
        if (active && nq == 0) hscale[(base + c * cstride) / N + p] = exp2i(ex);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) H[i] = decay * H[i] + sv[i];
    }
  }
  if (active && h_final) {
    if (C_scale_ps) {
#pragma unroll
      for (int i = 0; i < 4; ++i) H[i] = H[i] / sc[i];
    }
    *reinterpret_cast<v4f*>(h_final + int64_t(bh) * pn + e) = H;
  }
}

}  // namespace

hipError_t launch_state_passing(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  int lanes = 1;
  while (lanes < s.dstate / 4) lanes <<= 1;   // next power of two of N/4 (<= 32 for N <= 128)
  const int rows_per_block = kThreads / lanes;
  const int per_bh = (s.headdim + rows_per_block - 1) / rows_per_block;
  const int nblocks = s.batch * s.nheads * per_bh;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(nblocks), dim3(kThreads), 0, stream, a.states, a.acs, a.h0, a.h_final, a.hprev,
                       a.hscale, a.bc_per_state ? a.C_scale : nullptr, s.seqlen, s.nheads, s.headdim, s.dstate,
                       s.ngroups, s.chunk, s.nchunks, per_bh);
  };
  switch (lanes) {   // N / 4 = 4 .. 32 for the supported dstate
    case 4: go(state_passing_kernel<4>); break;
    case 8: go(state_passing_kernel<8>); break;
    case 16: go(state_passing_kernel<16>); break;
    default: go(state_passing_kernel<32>); break;
  }
  return hipGetLastError();
}

}  // namespace ssdq
