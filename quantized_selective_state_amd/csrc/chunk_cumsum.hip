// Stage 0 of the chunked SSD scan: Acs[b, h, c, j] = sum_{i <= j} dt[b, cQ + i, h] * A[h]
// (the log of the cumulative decay exp(dt A) inside chunk c; tokens past the end of the
// sequence contribute 0, so a ragged last chunk is padded with its last value).
//
// One block per (batch, chunk, 32-head tile).  The dt tile (Q tokens x 32 heads) is read
// with coalesced 128-byte rows, transposed through LDS, and each head is scanned by one
// wave (4 tokens per lane, then a wave-wide prefix over lane totals).
#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kHeadTile = 32;
constexpr int kMaxChunk = 256;

__global__ void __launch_bounds__(256) chunk_cumsum_kernel(const float* __restrict__ dt, const float* __restrict__ A,
                                                           float* __restrict__ acs, int64_t seqlen, int32_t nheads,
                                                           int32_t chunk, int32_t nchunks) {
  __shared__ float tile[kMaxChunk][kHeadTile + 1];
  const int htile = blockIdx.x;
  const int c = blockIdx.y;
  const int b = blockIdx.z;
  const int h0 = htile * kHeadTile;
  const int tid = threadIdx.x;
  const int64_t t0 = int64_t(c) * chunk;
  const int len = int(seqlen - t0 < chunk ? seqlen - t0 : chunk);

  for (int r = tid / kHeadTile; r < chunk; r += 256 / kHeadTile) {
    const int hh = tid % kHeadTile;
    float v = 0.f;
    if (r < len && h0 + hh < nheads) v = dt[(int64_t(b) * seqlen + t0 + r) * nheads + h0 + hh];
    tile[r][hh] = v;
  }
  __syncthreads();

  const int wave = tid / kWave;
  const int lane = tid % kWave;
  for (int hh = wave; hh < kHeadTile && h0 + hh < nheads; hh += 256 / kWave) {
    const int h = h0 + hh;
    const float a = A[h];
    float v[4];
    float run = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = 4 * lane + k;
      run += (j < chunk) ? tile[j][hh] * a : 0.f;
      v[k] = run;
    }
    // exclusive prefix of lane totals
    float incl = run;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const float up = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += up;
    }
    const float excl = incl - run;
    if (4 * lane < chunk) {
      float4 out = make_float4(v[0] + excl, v[1] + excl, v[2] + excl, v[3] + excl);
      *reinterpret_cast<float4*>(acs + ((int64_t(b) * nheads + h) * nchunks + c) * chunk + 4 * lane) = out;
    }
  }
}

}  // namespace

hipError_t launch_chunk_cumsum(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  dim3 grid((s.nheads + kHeadTile - 1) / kHeadTile, s.nchunks, s.batch);
  hipLaunchKernelGGL(chunk_cumsum_kernel, grid, dim3(256), 0, stream, a.dt, a.A, a.acs, s.seqlen, s.nheads, s.chunk,
                     s.nchunks);
  return hipGetLastError();
}

}  // namespace ssdq
