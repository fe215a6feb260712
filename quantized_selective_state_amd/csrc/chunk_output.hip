// Stage 2 of the chunked SSD scan: the output of chunk c,
//
//   y[l, p] = sum_{j <= l} M[l, j] xhat[j, p]  +  exp(Acs_l) Chat_l . Hprev_c[p, :]  +  D xhat[l, p]
//   M[l, j] = (Chat_l . Bhat_j) exp(Acs_l - Acs_j) dt_j
//
// (the state-space-duality form: the masked "attention" C B^T inside a chunk plus the
// carried state read out by C; SSDi8 Figure 1b / Table 5: ChunkBMM C.B^T on INT8).
//
// A persistent block (8 waves) walks (batch, chunk, head) items; each wave owns two 16-row
// output blocks of an item (l and 15 - l, for balance), and the next item's global loads are in flight while an item is
// computed (register prefetch, committed to LDS after the item).
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
//  - y^T += x^T M^T on v_mfma_f32_16x16x32_f16 (fp32 accumulation, x codes exact in fp16).
//  - y_off^T = Hprev C^T on v_mfma_i32_16x16x64_i8: Hprev arrives as two INT8 limbs with one
//    power-of-two scale per row and meets the C codes directly (persistent INT8 operands).
//  - LDS matrices are padded or 16-byte-chunk XOR swizzled so that the MFMA operand reads
//    are free of bank conflicts with addresses that advance linearly in the hot loop.
#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 512;    // 8 waves: two 16-row output blocks (l and 15 - l) each at chunk 256
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxQ = 256;
constexpr int kMaxP = 64;
constexpr int kMaxN = 128;
constexpr float kLog2e = 1.4426950408889634f;

// x^T: [p][j] fp16, rows padded to 264 halves (528 bytes = 132 banks, i.e. 4 banks apart),
// so the hot-loop reads of 16 consecutive rows are conflict-free with linear addresses
constexpr int kXS = kMaxQ + 8;
__device__ __forceinline__ int xpos(int p, int j) { return p * kXS + j; }
// B codes: [j][n] int8, 128-byte rows, chunk c stored at c ^ ((j >> 1) & 7)
__device__ __forceinline__ int bpos(int j, int byte) {
  return j * kMaxN + ((((byte >> 4) ^ ((j >> 1) & 7)) << 4) | (byte & 15));
}
// Hprev limbs: two [p][n] int8 planes, 128-byte rows, same swizzle as the B codes
constexpr int kHPlane = kMaxP * kMaxN;
__device__ __forceinline__ int hpos(int p, int byte) { return bpos(p, byte); }

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

struct Item {
  int b, c, h, g, len;
  int64_t t0;
};

__device__ __forceinline__ Item item_of(int it, int nheads, int nchunks, int ngroups, int64_t seqlen, int chunk) {
  Item r;
  r.h = it % nheads;
  r.c = (it / nheads) % nchunks;
  r.b = it / (nheads * nchunks);
  r.g = r.h / (nheads / ngroups);
  r.t0 = int64_t(r.c) * chunk;
  r.len = int(seqlen - r.t0 < chunk ? seqlen - r.t0 : chunk);
  return r;
}

// Global data of one work item held in registers between its load and its LDS commit.
constexpr int kBTasks = kMaxQ * 8 / kThreads;          // 16-byte B pieces per thread
constexpr int kHTasks = 2 * kMaxP * 8 / kThreads;      // 16-byte Hprev-limb pieces per thread
constexpr int kXTasks = 16 * (kMaxQ / 4) / kThreads;   // 4x4 x transposition tasks per thread
struct Prefetch {
  float acs, dt, hs;
  v4u bq[kBTasks];
  v4u hq[kHTasks];
  uint32_t xw[kXTasks][4];
};

struct Params {
  const int8_t* x;
  const float* x_scale;
  const int8_t* B;
  const float* B_scale;
  const int8_t* C;
  const float* C_scale;
  const float* dt;
  const float* D;
  const float* acs;
  const int8_t* hprev;
  const float* hscale;
  _Float16* y;
  int64_t seqlen;
  int nheads, P, N, ngroups, Q, nchunks, nitems;
};

// Per-lane byte offsets that do not depend on the work item (computed once per block).  Pieces
// that fall outside the operand (channels past P, states past N) get kOutOfRange and load as
// zeros; rows past the sequence end load as zeros through the item's buffer sizes.
struct LaneConst {
  uint32_t b_off[kBTasks];      // B piece: token row j * G*N + 16-byte column group
  int b_lds[kBTasks];
  uint32_t h_off[kHTasks];      // Hprev-limb piece in its (b, c, h) block
  int h_lds[kHTasks];
  uint32_t x_off[kXTasks];      // first row (4 jq) of an x transposition task, channel quad
  int x_lds[kXTasks];
  uint32_t c_off[2][2];         // C codes of this lane's output row, per pass and K half
  uint32_t acs_off, dt_off, hs_off;
};

// Buffer resources of one item: base at the item's first element, size up to the end of its
// last valid row.
struct ItemRsrc {
  Rsrc acs, dt, hs, B, H, x;
};

__device__ __forceinline__ ItemRsrc item_rsrc(const Item& it, const Params& a) {
  const int P = a.P, N = a.N, G = a.ngroups, H = a.nheads;
  const uint32_t last = uint32_t(it.len - 1);
  ItemRsrc r;
  r.acs = make_rsrc(a.acs + ((int64_t(it.b) * H + it.h) * a.nchunks + it.c) * a.Q, uint32_t(a.Q) * 4u);
  r.dt = make_rsrc(a.dt + (int64_t(it.b) * a.seqlen + it.t0) * H + it.h, (last * uint32_t(H) + 1u) * 4u);
  r.hs = make_rsrc(a.hscale + ((int64_t(it.b) * a.nchunks + it.c) * H + it.h) * P, uint32_t(P) * 4u);
  r.B = make_rsrc(a.B + ((int64_t(it.b) * a.seqlen + it.t0) * G + it.g) * N, last * uint32_t(G * N) + N);
  r.H = make_rsrc(a.hprev + ((int64_t(it.b) * a.nchunks + it.c) * H + it.h) * int64_t(2 * P) * N,
                  uint32_t(2 * P * N));
  r.x = make_rsrc(a.x + ((int64_t(it.b) * a.seqlen + it.t0) * H + it.h) * P, last * uint32_t(H * P) + P);
  return r;
}

// Issue every global load of one item (nothing waits here).
__device__ __forceinline__ void prefetch(Prefetch& f, const ItemRsrc& r, const LaneConst& lc, uint32_t xrow) {
  f.acs = buf_loadf(r.acs, lc.acs_off);
  f.dt = buf_loadf(r.dt, lc.dt_off);
  f.hs = buf_loadf(r.hs, lc.hs_off);
#pragma unroll
  for (int k = 0; k < kBTasks; ++k) f.bq[k] = buf_load16(r.B, lc.b_off[k]);
#pragma unroll
  for (int k = 0; k < kHTasks; ++k) f.hq[k] = buf_load16(r.H, lc.h_off[k]);
#pragma unroll
  for (int k = 0; k < kXTasks; ++k)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) f.xw[k][rr] = buf_load4(r.x, lc.x_off[k] + uint32_t(rr) * xrow);
}

__global__ void __launch_bounds__(kThreads) chunk_output_kernel(Params a) {
  __shared__ __attribute__((aligned(16))) _Float16 xT[kMaxP * kXS];
  __shared__ __attribute__((aligned(16))) int8_t Bs[kMaxQ * kMaxN];
  __shared__ __attribute__((aligned(16))) int8_t Hq[2 * kHPlane];
  __shared__ __attribute__((aligned(16))) float hsc[kMaxP];
  __shared__ __attribute__((aligned(16))) float acs2[kMaxQ];   // Acs * log2(e)
  __shared__ __attribute__((aligned(16))) float dts[kMaxQ];    // dt (0 past the sequence end)
  __shared__ __attribute__((aligned(16))) float wl[kWaves][kMaxQ];
  __shared__ float red[kWaves];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int Q = a.Q, P = a.P, N = a.N;
  const int lcol = lane % 16, kg = lane / 16;
  const int nlb = Q / 16;

  // ---- lane constants (item independent)
  const uint32_t gn = uint32_t(a.ngroups * N), xrow = uint32_t(a.nheads * P);
  LaneConst lc;
#pragma unroll
  for (int k = 0; k < kBTasks; ++k) {
    const int task = tid + k * kThreads;
    const int j = task >> 3, sg = task & 7;
    lc.b_off[k] = 16 * sg < N ? uint32_t(j) * gn + 16 * sg : kOutOfRange;
    lc.b_lds[k] = bpos(j, 16 * sg);
  }
#pragma unroll
  for (int k = 0; k < kHTasks; ++k) {
    const int task = tid + k * kThreads;
    const int limb = task / (kMaxP * 8), p = (task / 8) % kMaxP, sg = task & 7;
    lc.h_off[k] = (p < P && 16 * sg < N) ? uint32_t(limb * P * N + p * N + 16 * sg) : kOutOfRange;
    lc.h_lds[k] = limb * kHPlane + hpos(p, 16 * sg);
  }
  {
    const int pq = tid & 15;
#pragma unroll
    for (int k = 0; k < kXTasks; ++k) {
      const int jq = (tid + k * kThreads) >> 4;
      lc.x_off[k] = 4 * pq < P ? uint32_t(4 * jq) * xrow + 4 * pq : kOutOfRange;
      lc.x_lds[k] = xpos(4 * pq, 4 * jq);
    }
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int lbp = pass == 0 ? wave : 2 * kWaves - 1 - wave;
    const uint32_t l = uint32_t(16 * lbp + lcol);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      lc.c_off[pass][s2] = (lbp < nlb && 64 * s2 + 16 * kg < N) ? l * gn + 64 * s2 + 16 * kg : kOutOfRange;
  }
  lc.acs_off = uint32_t(tid & (kMaxQ - 1)) * 4u;
  lc.dt_off = uint32_t(tid & (kMaxQ - 1)) * uint32_t(a.nheads) * 4u;
  lc.hs_off = uint32_t(tid & (kMaxP - 1)) * 4u;
  // hot-loop LDS bases: for rows js + lcol with js a multiple of 16 the B swizzle term depends
  // on lcol only, so every hot-loop address is a per-lane base plus a multiple of the step
  const int8_t* bs_lane = Bs + bpos(lcol, 16 * kg);                    // + js * 128
  const int bs_half = bpos(lcol, 64 + 16 * kg) - bpos(lcol, 16 * kg);   // second K half
  const _Float16* xt_lane = xT + xpos(lcol, 4 * kg);                    // + 16 pt rows, + jb
  float* wlw = wl[wave];
  const float* wl_lane = wlw + 4 * kg;
  int hq_lane[2][4];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) hq_lane[s2][pt] = hpos(16 * pt + lcol, 64 * s2 + 16 * kg);

  // Persistent block: items slot, slot + gridDim.x, ...  The global loads of the next item are
  // issued right after the current item is committed to LDS and complete while the current
  // item is computed.  slot is XCD-aware: the blocks of one XCD take consecutive items, i.e.
  // neighbouring heads of one (batch, chunk), so that chunk's B and C and the dt lines it
  // shares across heads are fetched into one L2 rather than into all of them.
  int it = xcd_remap(blockIdx.x, gridDim.x);
  if (it >= a.nitems) return;
  Prefetch f;
  prefetch(f, item_rsrc(item_of(it, a.nheads, a.nchunks, a.ngroups, a.seqlen, Q), a), lc, xrow);

  for (; it < a.nitems; it += gridDim.x) {
    const Item cur = item_of(it, a.nheads, a.nchunks, a.ngroups, a.seqlen, Q);
    const int len = cur.len;

    // ---- commit the prefetched item to LDS.  Rows past the sequence end arrived as zeros;
    // channels past P and states past N hold zeros or values that only meet zeros (the C codes
    // past N are zero, and rows past P are never stored).
    if (tid < kMaxQ) {
      acs2[tid] = f.acs * kLog2e;
      dts[tid] = f.dt;
    }
    {
      const float dm = wave_max(f.dt);   // waves 4..7 hold the same tokens as waves 0..3
      if (lane == 0) red[wave] = dm;
    }
    if (tid < kMaxP) hsc[tid] = f.hs;
#pragma unroll
    for (int k = 0; k < kBTasks; ++k) *reinterpret_cast<v4u*>(Bs + lc.b_lds[k]) = f.bq[k];
#pragma unroll
    for (int k = 0; k < kHTasks; ++k) *reinterpret_cast<v4u*>(Hq + lc.h_lds[k]) = f.hq[k];
#pragma unroll
    for (int k = 0; k < kXTasks; ++k) {
      uint32_t in[4], out[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) in[r] = f.xw[k][r] ^ 0x80808080u;
      transpose4x4(in, out);
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<v4h*>(xT + lc.x_lds[k] + i * kXS) = codes_to_f16(out[i]);
    }
    __syncthreads();

    // ---- loads the current item still needs, for both of this wave's row blocks.  They are
    // issued and consumed before the next item's prefetch: vmcnt retires in order, so any
    // wait on a load issued after the prefetch would also wait for the prefetch.
    const Rsrc crs = make_rsrc(a.C + ((int64_t(cur.b) * a.seqlen + cur.t0) * a.ngroups + cur.g) * N,
                               uint32_t(len - 1) * gn + N);
    v4i cqs[2][2];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) cqs[pass][s2] = __builtin_bit_cast(v4i, buf_load16(crs, lc.c_off[pass][s2]));
    const int hu = __builtin_amdgcn_readfirstlane(cur.h);
    const int gu = __builtin_amdgcn_readfirstlane(cur.g);
    const float sx = a.x_scale[hu], sB = a.B_scale[gu], sC = a.C_scale[gu];
    const float Dh = a.D ? a.D[hu] : 0.f;
    _Float16* ybase = a.y + ((int64_t(cur.b) * a.seqlen + cur.t0) * a.nheads + cur.h) * P;
    __builtin_amdgcn_sched_barrier(0);

    // unconditional (the last item re-reads a valid item): a prefetch behind a branch would
    // make the wait counts after it conservative
    const int nx = min(it + int(gridDim.x), a.nitems - 1);
    prefetch(f, item_rsrc(item_of(nx, a.nheads, a.nchunks, a.ngroups, a.seqlen, Q), a), lc, xrow);
    __builtin_amdgcn_sched_barrier(0);

    float dtmax = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) dtmax = fmaxf(dtmax, red[i]);
    // |M'| <= N 127^2 dtmax 2^-kM <= 2^15; clamped so that 2^kM and 2^-kM are exact
    const int kM = min(max(ceil_log2_pos(float(N) * 16129.f * dtmax) - 15, -120), 120);
    const float s_in = sx * sC * sB * exp2i(kM);
    const float fkM = float(kM);
    const float sxD = sx * Dh;

#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int lb = pass == 0 ? wave : 2 * kWaves - 1 - wave;
      if (lb >= nlb || (pass == 1 && nlb <= kWaves)) continue;
      const int l0 = 16 * lb;
      const int l = l0 + lcol;
      const bool lvalid = l < len;
      const v4i cq[2] = {pass == 0 ? cqs[0][0] : cqs[1][0], pass == 0 ? cqs[0][1] : cqs[1][1]};
      const int jdiag = l0 & ~31;          // the 32-token block that holds the diagonal
      const float a_l = acs2[l];
      const float a_0 = acs2[l0];

      // weights of the blocks before the diagonal, relative to row l0, times 2^-kM (<= 1 each)
      for (int j = lane; j < jdiag; j += kWave) wlw[j] = __builtin_amdgcn_exp2f(a_0 - acs2[j] - fkM) * dts[j];
      __builtin_amdgcn_wave_barrier();
      const float u_l = __builtin_amdgcn_exp2f(a_l - a_0);

      v4f yf[4], yd[4];
      v4i yo1[4], yo2[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        yf[pt] = v4f{0.f, 0.f, 0.f, 0.f};
        yd[pt] = v4f{0.f, 0.f, 0.f, 0.f};
        yo1[pt] = v4i{0, 0, 0, 0};
        yo2[pt] = v4i{0, 0, 0, 0};
      }

      // carried state read out by C: y_off^T[p][l] = sum_n Hprev[p][n] q_C[l][n], both limbs
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const v4i h1 = *reinterpret_cast<const v4i*>(Hq + hq_lane[s2][pt]);
          const v4i h2 = *reinterpret_cast<const v4i*>(Hq + kHPlane + hq_lane[s2][pt]);
          yo1[pt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(h1, cq[s2], yo1[pt], 0, 0, 0);
          yo2[pt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(h2, cq[s2], yo2[pt], 0, 0, 0);
        }
      }

      // intra-chunk part, 32 tokens per step: blocks before the diagonal use the factorized decay
#pragma unroll 2
      for (int jb = 0; jb < jdiag; jb += 32) {
        v4i gm[2];
        float4 w4[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int js = jb + 16 * sb;
          const int8_t* bp = bs_lane + js * kMaxN;
          const v4i b0 = *reinterpret_cast<const v4i*>(bp);
          const v4i b1 = *reinterpret_cast<const v4i*>(bp + bs_half);
          w4[sb] = *reinterpret_cast<const float4*>(wl_lane + js);
          gm[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b0, cq[0], v4i{0, 0, 0, 0}, 0, 0, 0);
          gm[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b1, cq[1], gm[sb], 0, 0, 0);
        }
        v8h xop[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const _Float16* xp = xt_lane + 16 * pt * kXS + jb;
          const v4h lo = *reinterpret_cast<const v4h*>(xp);
          const v4h hi = *reinterpret_cast<const v4h*>(xp + 16);
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
        for (int pt = 0; pt < 4; ++pt)
          yf[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop[pt], mop, yf[pt], 0, 0, 0);
      }
      // the block holding the diagonal: exact per-element decay and the causal mask
      {
        const int jb = jdiag;
        const int j1 = min(jb + 16, Q - 16);   // second sub-block (fully masked when clamped)
        v4i gm[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int8_t* bp = bs_lane + (sb == 0 ? jb : j1) * kMaxN;
          const v4i b0 = *reinterpret_cast<const v4i*>(bp);
          const v4i b1 = *reinterpret_cast<const v4i*>(bp + bs_half);
          gm[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b0, cq[0], v4i{0, 0, 0, 0}, 0, 0, 0);
          gm[sb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b1, cq[1], gm[sb], 0, 0, 0);
        }
        const float a_lk = a_l - fkM;
        v8h mop;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int jq = (sb == 0 ? jb : j1) + 4 * kg;
          const float4 a4 = *reinterpret_cast<const float4*>(&acs2[jq]);
          const float4 d4 = *reinterpret_cast<const float4*>(&dts[jq]);
          const float av[4] = {a4.x, a4.y, a4.z, a4.w};
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = jb + 16 * sb + 4 * kg + i;     // > l (masked) whenever the clamp applied
            const float m = float(gm[sb][i]) * __builtin_amdgcn_exp2f(fminf(a_lk - av[i], -fkM)) * dv[i];
            mop[4 * sb + i] = _Float16(j <= l ? m : 0.f);
          }
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const _Float16* xp = xt_lane + 16 * pt * kXS;
          const v4h lo = *reinterpret_cast<const v4h*>(xp + jb);
          const v4h hi = *reinterpret_cast<const v4h*>(xp + j1);
          const v8h xop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          yd[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, mop, yd[pt], 0, 0, 0);
        }
      }

      // ---- epilogue: lane holds y[l, 16 pt + 4 kg + i], i = 0..3
      const float s_off = __builtin_amdgcn_exp2f(fminf(a_l, 0.f)) * sC;
      const float c_f = u_l * s_in;
      _Float16* yrow = ybase + uint32_t(min(l, len - 1)) * uint32_t(a.nheads * P);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const float4 hs = *reinterpret_cast<const float4*>(&hsc[16 * pt + 4 * kg]);
        const float hv[4] = {hs.x, hs.y, hs.z, hs.w};
        v4h out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = 16 * pt + 4 * kg + i;
          const float c1 = s_off * hv[i];
          float v = float(xT[xpos(p, l)]) * sxD;
          v = fmaf(float(yo2[pt][i]), c1 * (1.f / 256.f), v);
          v = fmaf(float(yo1[pt][i]), c1, v);
          v = fmaf(yd[pt][i], s_in, v);
          v = fmaf(yf[pt][i], c_f, v);
          out[i] = _Float16(v);
        }
        if (lvalid && 16 * pt + 4 * kg < P) *reinterpret_cast<v4h*>(yrow + 16 * pt + 4 * kg) = out;
      }
    }
    __syncthreads();   // LDS is rewritten by the next item's commit
  }
}

}  // namespace

hipError_t launch_chunk_output(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  Params p{a.x, a.x_scale, a.B, a.B_scale, a.C, a.C_scale, a.dt, a.D, a.acs, a.hprev, a.hscale, a.y,
           s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk, s.nchunks,
           s.batch * s.nchunks * s.nheads};
  // one persistent block per CU (the LDS footprint allows one resident block)
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    cus = 256;
  const int nblocks = p.nitems < cus ? p.nitems : cus;
  hipLaunchKernelGGL(chunk_output_kernel, dim3(nblocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ssdq
