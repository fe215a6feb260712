// Stage 2 of the chunked SSD scan: the output of chunk c,
//
//   y[l, p] = sum_{j <= l} M[l, j] xhat[j, p]  +  exp(Acs_l) Chat_l . Hprev_c[p, :]  +  D xhat[l, p]
//   M[l, j] = (Chat_l . Bhat_j) exp(Acs_l - Acs_j) dt_j
//
// (the state-space-duality form: the masked "attention" C B^T inside a chunk plus the
// carried state read out by C; SSDi8 Figure 1b / Table 5: ChunkBMM C.B^T on INT8).
//
// A persistent block (8 waves) walks (batch, chunk, head) items; each wave owns two 16-row
// output blocks of an item (see row_block), and the next item's global loads are in flight
// while an item is computed (register prefetch, committed into the other of two LDS tile
// buffers as soon as the wave's own passes are done: one barrier per item).
//  - G^T[j, l] = sum_n q_B[j, n] q_C[l, n] on v_mfma_i32_16x16x64_i8 (exact int32).
//  - Decay mask, SSDi8-style decoupled from the matrix products: for a 32-token block that
//    lies entirely before the 16 output rows l0..l0+15, exp(Acs_l - Acs_j) =
//    exp(Acs_l - Acs_l0) exp(Acs_l0 - Acs_j), both factors <= 1, so the per-element work is
//    G * w_j (w_j = exp(Acs_l0 - Acs_j) dt_j, once per token) and the row factor
//    u_l = exp(Acs_l - Acs_l0) is applied in the epilogue.  The 32-token block holding the
//    diagonal is split around its first token m instead (a row factor exp(Acs_l - Acs_m) <= 1
//    times a token weight exp(Acs_m - Acs_j) dt_j), with the causal mask; when its weights
//    would leave the safe fp32 range it takes the exact per-element exp.
//  - The masked fragment, rounded to fp16 under a power-of-two guard, feeds the next product
//    as its B operand straight from registers: the fp16 MFMA's K slots are matched to the
//    rows the int32 fragment holds, and x^T is read from LDS in the same slot order.
//  - y^T += x^T M^T on v_mfma_f32_16x16x32_f16 (fp32 accumulation, x codes exact in fp16).
//  - y_off^T = Hprev C^T on v_mfma_i32_16x16x64_i8: Hprev arrives as two INT8 limbs with one
//    power-of-two scale per row and meets the C codes directly (persistent INT8 operands).
//  - LDS matrices are padded or 16-byte-chunk XOR swizzled so that the MFMA operand reads
//    are free of bank conflicts with addresses that advance linearly in the hot loop.
#include <type_traits>

#include "ssdq_internal.h"

namespace ssdq {
namespace {

constexpr int kThreads = 512;    // 8 waves: two 16-row output blocks each at chunk 256
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxQ = 256;
constexpr int kMaxP = 64;
constexpr int kMaxN = 128;
constexpr float kLog2e = 1.4426950408889634f;

// x: [j][p] fp16 (token-major, 128-byte rows), 16-byte chunk c of row j stored at c ^ xswz(j),
// xswz(j) = 4 bit2(j) + 3 bit1(j): with this swizzle the 16-byte commit stores and the
// transposing operand reads (ds_read_b64_tr_b16) are both free of bank conflicts.
__device__ __forceinline__ int xswz(int j) { return (((j >> 2) & 1) << 2) | (((j >> 1) & 1) * 3); }
__device__ __forceinline__ int xpos(int j, int p) { return j * kMaxP + ((((p >> 3) ^ xswz(j)) << 3) | (p & 7)); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element i % 4 of the
// 8-byte chunks addressed by lanes 4 k + i / 4, k = 0..3.  With lane 4 k + q of a group
// addressing x[j0 + k][16 pt + 4 q], lane i gets x[j0 + k][16 pt + i] for k = 0..3.
__device__ __forceinline__ v4h tr16(const _Float16* lds) {
  return __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                     (__attribute__((address_space(3))) v4s*)(lds)));
}
// B codes: [j][n] int8, 128-byte rows, chunk c stored at c ^ ((j >> 1) & 7); within a full
// 64-state block the states are in the carried state's order (dword-transposed), so that
// C.B^T and C.Hprev share the C operand
__device__ __forceinline__ int bpos(int j, int byte) {
  return j * kMaxN + ((((byte >> 4) ^ ((j >> 1) & 7)) << 4) | (byte & 15));
}
// Hprev limbs: two [p][n] int8 planes, 128-byte rows in the workspace's byte order (a full
// 64-state block dword-transposed), same 16-byte-chunk swizzle as the B codes.  C.Hprev sums
// over the states in that order: the C operand of a full block is loaded in the same order.
constexpr int kHPlane = kMaxP * kMaxN;
__device__ __forceinline__ int hpos(int p, int byte) { return bpos(p, byte); }

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

// LDS pointers whose per-lane base is opaque to the compiler: the hot loops then address every
// read as that base plus an immediate offset (the arrays lie past the 16-bit offset range of
// the LDS instructions, so a known array base would cost an add per read).
#define LDSP __attribute__((address_space(3)))
template <typename T>
__device__ __forceinline__ const LDSP T* lds_base(const T* p) {
  uint32_t a = uint32_t(uintptr_t((const LDSP T*)p));
  asm volatile("" : "+v"(a));
  return (const LDSP T*)uintptr_t(a);
}
// lds_base where the instance uses the array, nothing (and no instruction) where it does not
template <bool kOn, typename T>
__device__ __forceinline__ const LDSP T* lds_base_if(const T* p) {
  if constexpr (kOn)
    return lds_base(p);
  else
    return nullptr;
}
template <typename V, typename T>
__device__ __forceinline__ V lds_ld(const LDSP T* p, int off) {
  return *reinterpret_cast<const LDSP V*>(p + off);
}
__device__ __forceinline__ float4 lds_f4(const LDSP float* p, int off) {
  const v4f v = lds_ld<v4f>(p, off);
  return float4{v[0], v[1], v[2], v[3]};
}

// The 16-row output block of a wave's pass.  Waves s and s + 4 share a SIMD and together own
// blocks s, 15 - s, 4 + s, 11 - s, whose causal work (blocks before the diagonal: floor(b / 2))
// is the same on every SIMD.  The SIMD issues the older wave s first, so it takes the larger
// share (15 - s and 4 + s: 9 steps against 5), and the pair finishes together instead of
// leaving wave s + 4 to run alone at the end.  Blocks at or past Q / 16 do not exist.
static_assert(kWaves == 8 && kMaxQ == 256, "row_block covers 16 blocks with 8 waves");
__device__ __forceinline__ int row_block(int wave, int pass) {
  const int s = wave & 3;
  return (wave >> 2) == 0 ? (pass == 0 ? 15 - s : 4 + s) : (pass == 0 ? s : 11 - s);
}

struct Item {
  int b, c, h, g, len;
  int64_t t0;
};

// item index -> (batch, chunk, head), head fastest; invariant divisions by multipliers
__device__ __forceinline__ Item item_of(int it, FastDiv by_heads, FastDiv by_chunks, FastDiv by_hpg, int64_t seqlen,
                                        int chunk) {
  Item r;
  const uint32_t q1 = fdiv(uint32_t(it), by_heads);
  const uint32_t q2 = fdiv(q1, by_chunks);
  r.h = int(uint32_t(it) - q1 * by_heads.d);
  r.c = int(q1 - q2 * by_chunks.d);
  r.b = int(q2);
  r.g = int(fdiv(uint32_t(r.h), by_hpg));
  r.t0 = int64_t(r.c) * chunk;
  r.len = int(seqlen - r.t0 < chunk ? seqlen - r.t0 : chunk);
  return r;
}

// Global data of one work item held in registers between its load and its LDS commit.
constexpr int kBTasks = kMaxQ * 8 / kThreads;          // 16-byte B pieces per thread
static_assert(2 * kMaxP * (kMaxN / 32) == kThreads, "two 16-byte carried-state pieces per thread");
constexpr int kXTasks = kMaxQ * (kMaxP / 16) / kThreads;   // 16-byte x pieces per thread
struct Prefetch {
  float acs, dt, hs, mu, sxp;   // sxp: the x scale of channel tid (x scales per (head, channel))
  v4i cq[2][2];                 // C codes of this lane's two output rows (per pass, K half)
  v4u bq[kBTasks];
  v4u hq[2];                    // two 16-byte pieces of one limb row
  v4u xq[kXTasks];
};

struct Params {
  const int8_t* x;
  const float* x_scale;
  const int8_t* B;
  const float* B_scale;
  const int8_t* C;
  const float* C_scale;
  const float* dtc;   // dt in chunk order: (batch, nheads, nchunks, chunk), 0 past the end
  const float* D;
  const float* acs;
  const int8_t* hprev;
  const float* hscale;
  const float* ycorr;   // (nheads, headdim) output correction, read only by the corrected instance
  _Float16* y;
  int64_t seqlen;
  int nheads, P, N, ngroups, Q, nchunks, nitems;
  FastDiv by_heads, by_chunks, by_hpg;   // nheads, nchunks, nheads / ngroups
};

// Per-lane byte offsets that do not depend on the work item (computed once per block).  Pieces
// that fall outside the operand (channels past P, states past N) get kOutOfRange and load as
// zeros; rows past the sequence end load as zeros through the item's buffer sizes.
struct LaneConst {
  uint32_t b_off[kBTasks];      // B piece: token row j * G*N + 16-byte column group
  int b_lds[kBTasks];
  uint32_t h_off[2];            // this thread's two carried-state pieces (limb, row, 32 bytes)
  int h_lds[2];                 // their LDS positions (the workspace order is kept)
  uint32_t x_off[kXTasks];      // x piece: token row j * H*P + 16-byte column group
  int x_lds[kXTasks];           // LDS position (halves) of its first 8 channels
  uint32_t c_off[2][2];         // C codes of this lane's output row, per pass and K half
  uint32_t acs_off, hs_off;   // acs_off also addresses the chunk-ordered dt row
};

// Buffer resources of one item: base at the item's first element, size up to the end of its
// last valid row.
struct ItemRsrc {
  Rsrc acs, dt, hs, mu, B, H, x, C, sx;
};

// One work item's position, as 32-bit row indices into its operands (every index is below
// batch * seqlen * nheads < 2^31).  Consecutive items of a block's range are mostly consecutive
// heads of one (batch, chunk): the next one is then reached by adding fixed steps, and only a
// change of (batch, chunk) decodes the item index again.
struct ItemPos {
  int h, g, hg, len;   // hg: the head's index within its group
  uint32_t row;        // (b seqlen + t0) nheads + h: first (token, head) row of x and y
  uint32_t grow;       // (b seqlen + t0) ngroups + g: first (token, group) row of B and C
  uint32_t seg;        // (b nchunks + c) nheads + h: carried-state slot (limbs, row scales)
  uint32_t aseg;       // (b nheads + h) nchunks + c: the Acs row
};

__device__ __forceinline__ ItemPos item_at(int it, const Params& a) {
  const Item r = item_of(it, a.by_heads, a.by_chunks, a.by_hpg, a.seqlen, a.Q);
  const uint32_t tok = uint32_t(int64_t(r.b) * a.seqlen + r.t0);
  ItemPos p;
  p.h = r.h;
  p.g = r.g;
  p.hg = r.h - r.g * int(a.by_hpg.d);
  p.len = r.len;
  p.row = tok * uint32_t(a.nheads) + uint32_t(r.h);
  p.grow = tok * uint32_t(a.ngroups) + uint32_t(r.g);
  p.seg = (uint32_t(r.b) * uint32_t(a.nchunks) + uint32_t(r.c)) * uint32_t(a.nheads) + uint32_t(r.h);
  p.aseg = (uint32_t(r.b) * uint32_t(a.nheads) + uint32_t(r.h)) * uint32_t(a.nchunks) + uint32_t(r.c);
  return p;
}

// p (item it) becomes item it + 1; returns whether the (batch, chunk, group) changed
__device__ __forceinline__ bool item_next(ItemPos& p, int it, const Params& a) {
  if (p.h + 1 < a.nheads) {
    p.h += 1;
    p.row += 1;
    p.seg += 1;
    p.aseg += uint32_t(a.nchunks);
    if (++p.hg < int(a.by_hpg.d)) return false;
    p.hg = 0;
    p.g += 1;
    p.grow += 1;
    return true;
  }
  p = item_at(it + 1, a);
  return true;
}

__device__ __forceinline__ uint64_t wide(uint32_t i, uint32_t stride) { return uint64_t(i) * stride; }

template <bool kPC = false>
__device__ __forceinline__ ItemRsrc item_rsrc(const ItemPos& p, const Params& a) {
  const uint32_t last = uint32_t(p.len - 1), gn = uint32_t(a.ngroups * a.N), P = uint32_t(a.P), N = uint32_t(a.N);
  ItemRsrc r;
  r.acs = make_rsrc(a.acs + wide(p.aseg, uint32_t(a.Q)), uint32_t(a.Q) * 4u);
  r.dt = make_rsrc(a.dtc + wide(p.aseg, uint32_t(a.Q)), uint32_t(a.Q) * 4u);
  r.hs = make_rsrc(a.hscale + wide(p.seg, P), P * 4u);
  r.mu = make_rsrc(a.ycorr + uint32_t(p.h) * P, a.ycorr ? P * 4u : 0u);
  r.B = make_rsrc(a.B + wide(p.grow, N), last * gn + N);
  r.H = make_rsrc(a.hprev + wide(p.seg, 2u * P * N), 2u * P * N);
  r.x = make_rsrc(a.x + wide(p.row, P), last * uint32_t(a.nheads) * P + P);
  r.C = make_rsrc(a.C + wide(p.grow, N), last * gn + N);
  if constexpr (kPC) r.sx = make_rsrc(a.x_scale + uint32_t(p.h) * P, P * 4u);
  return r;
}

// Issue the global loads of one item except its x codes (nothing waits here); B and C only when
// the item starts a new (batch, chunk, group) (bc, block-uniform); the head's output correction
// only in the corrected instance.
template <bool kCorr, bool kPC>
__device__ __forceinline__ void prefetch(Prefetch& f, const ItemRsrc& r, const LaneConst& lc, uint32_t xrow, bool bc,
                                         int N, int kg) {
  if (bc) {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint32_t o = lc.c_off[pass][s2];
        if (64 * s2 + 64 <= N) {
          // a full 64-state block: the carried state sits in LDS in its workspace order
          // (dword-transposed), so this operand takes the same K order: dword t holds states
          // 64 s2 + 16 t + 4 kg + (0..3)
          const uint32_t ob = o == kOutOfRange ? kOutOfRange : o - 12u * uint32_t(kg);
          v4u c;
#pragma unroll
          for (int t = 0; t < 4; ++t) c[t] = buf_load4(r.C, ob == kOutOfRange ? kOutOfRange : ob + 16u * t);
          f.cq[pass][s2] = __builtin_bit_cast(v4i, c);
        } else {
          f.cq[pass][s2] = __builtin_bit_cast(v4i, buf_load16(r.C, o));
        }
      }
#pragma unroll
    for (int k = 0; k < kBTasks; ++k) f.bq[k] = buf_load16(r.B, lc.b_off[k]);
  }
  if (threadIdx.x < kMaxQ) {   // wave-uniform: one value per token
    f.acs = buf_loadf(r.acs, lc.acs_off);
    f.dt = buf_loadf(r.dt, lc.acs_off);
  }
  if (threadIdx.x < kMaxP) {
    f.hs = buf_loadf(r.hs, lc.hs_off);
    if constexpr (kCorr) f.mu = buf_loadf(r.mu, lc.hs_off);
    if constexpr (kPC) f.sxp = buf_loadf(r.sx, lc.hs_off);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) f.hq[k] = buf_load16(r.H, lc.h_off[k]);
}
// The x codes of one item: issued apart from the rest, so that fewer loads queue at once for the
// CU's address units and the wave stalls less at their issue.
__device__ __forceinline__ void prefetch_x(Prefetch& f, const ItemRsrc& r, const LaneConst& lc) {
#pragma unroll
  for (int k = 0; k < kXTasks; ++k) f.xq[k] = buf_load16(r.x, lc.x_off[k]);
}

// kCorr: y also receives the per-(head, channel) output correction ycorr[h, p] (SSDi8's mean
// correction), added in the epilogue.
// kPS: B and C scales per (group, state) (SSDi8 Table 10: per-P(N) together with per-H(G)).  The
// carried state then arrives scaled by each state's C scale (the state stages do that), so C.Hprev
// needs no C scale; C.B^T needs sigma[n] = B_scale[n] C_scale[n] inside the sum over states.  It is
// carried by the B operand: with 2^s >= max sigma, V[j, n] = rint(256 q_B[j, n] sigma[n] / 2^s)
// (|V| <= 32512) is split into two INT8 limbs V = 256 hi + lo (hi = floor((V + 128) / 256), so
// lo is in [-128, 127]), both planes go through the INT8 matrix cores against the C codes, and
// 256 G_hi + G_lo (exact int32) stands for sum_n sigma[n] q_C q_B to within 2^(s - 9) per term.
// The second B plane takes the LDS of the second x tile buffer, so this instance commits the next
// item's x after a barrier instead of into a free buffer.
// kPC: x scales per (head, channel).  Every term of y is linear in x of its own channel p except
// the carried-state readout (its state already holds the x scales), so the item runs with unit
// x scale and the epilogue multiplies channel p by x_scale[h, p]; the carried-state row scale of
// row p is stored divided by that scale so that the readout comes out unscaled.
template <bool kCorr, bool kPS, bool kPC>
__global__ void __launch_bounds__(kThreads) chunk_output_kernel(Params a) {
  // Per-item tiles in two buffers (item k of the block in buffer k % 2): a wave commits the next
  // item into the other buffer as soon as its own passes are done, and one barrier per item
  // separates it from the waves still reading the current one.  B changes only with the group
  // and has one buffer.
  __shared__ __attribute__((aligned(16))) _Float16 xs_buf[kPS ? 1 : 2][kMaxQ * kMaxP];
  __shared__ __attribute__((aligned(16))) int8_t Hq_buf[2][2 * kHPlane];
  __shared__ __attribute__((aligned(16))) float hsc_buf[2][kMaxP];
  __shared__ __attribute__((aligned(16))) float mu_buf[2][kCorr ? kMaxP : 4];
  __shared__ __attribute__((aligned(16))) float sxc_buf[2][kPC ? kMaxP : 4];   // kPC: x scale per channel
  __shared__ __attribute__((aligned(16))) float acs2_buf[2][kMaxQ];   // Acs * log2(e)
  __shared__ __attribute__((aligned(16))) float dts_buf[2][kMaxQ];    // dt (0 past the sequence end)
  __shared__ float red_buf[2][kWaves];
  __shared__ __attribute__((aligned(16))) int8_t Bs[(kPS ? 2 : 1) * kMaxQ * kMaxN];   // kPS: hi plane, lo plane
  __shared__ float sig2_s;   // kPS: 2^s >= max_n sigma[n] of the current group
  __shared__ __attribute__((aligned(16))) float wl[kWaves][kMaxQ];

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
  {
    // limb tid / 256, row (tid / 4) % 64, bytes 32 (tid % 4) .. + 31 of the row
    const int limb = tid >> 8, p = (tid >> 2) & (kMaxP - 1), b0 = 32 * (tid & 3);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      lc.h_off[q] = (p < P && b0 + 16 * q < N) ? uint32_t(limb * P * N + p * N + b0 + 16 * q) : kOutOfRange;
      lc.h_lds[q] = limb * kHPlane + hpos(p, b0 + 16 * q);
    }
  }
#pragma unroll
  for (int k = 0; k < kXTasks; ++k) {
    const int piece = tid + k * kThreads;
    const int j = piece >> 2, cc = piece & 3;
    lc.x_off[k] = 16 * cc < P ? uint32_t(j) * xrow + 16 * cc : kOutOfRange;
    lc.x_lds[k] = xpos(j, 16 * cc);
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int lbp = row_block(wave, pass);
    const uint32_t l = uint32_t(16 * lbp + lcol);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      lc.c_off[pass][s2] = (lbp < nlb && 64 * s2 + 16 * kg < N) ? l * gn + 64 * s2 + 16 * kg : kOutOfRange;
  }
  lc.acs_off = uint32_t(tid & (kMaxQ - 1)) * 4u;
  lc.hs_off = uint32_t(tid & (kMaxP - 1)) * 4u;
  // hot-loop LDS bases: for rows js + lcol with js a multiple of 16 the B swizzle term depends
  // on lcol only, so every hot-loop address is a per-lane base plus a multiple of the step
  const LDSP int8_t* const bs_lane = lds_base(Bs + bpos(lcol, 16 * kg));   // + js * 128
  const LDSP int8_t* const bs_lane2 = lds_base(Bs + bpos(lcol, 64 + 16 * kg));   // second K half
  // transposing x reads: lane 4 k + q of its group addresses token row 4 kg + k at channels
  // 16 pt + 4 q; a step adds whole 32-token blocks (the swizzle repeats every 8 rows)
  int xa[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) xa[pt] = xpos(4 * kg + (lcol >> 2), 16 * pt + 4 * (lcol & 3));
  float* wlw = wl[wave];
  const LDSP float* const wl_lane = lds_base(wlw + 4 * kg);
  // carried-state rows 16 pt + lcol: the swizzle repeats every 16 rows, so row block pt lies
  // 16 pt rows (2048 bytes) past row lcol for both K halves
  const int hq_lane[2] = {hpos(lcol, 16 * kg), hpos(lcol, 64 + 16 * kg)};

  // Persistent block: a contiguous range of items, i.e. consecutive heads of one (batch, chunk)
  // (heads are the fastest item index).  Heads of one group share that chunk's B and C codes:
  // they are loaded and committed only when the group changes, and C's registers and the B
  // tile in LDS serve all the group's items of the range.  The global loads of the next item
  // are issued while the current item is computed (at the start of its trip, the x codes
  // between its two passes).  The range is XCD-aware: the blocks of one XCD take consecutive
  // ranges, so a chunk's B, C and the x lines its heads share are fetched into one L2.
  const int per = (a.nitems + int(gridDim.x) - 1) / int(gridDim.x);
  int it = xcd_remap(blockIdx.x, gridDim.x) * per;
  const int it_end = min(it + per, a.nitems);
  if (it >= it_end) return;
  Prefetch f{};
  v4i cqs[2][2];   // C codes of this lane's output rows (per pass, K half) for the current group

  // x codes of the prefetched item into x tile buffer xb, as fp16
  auto commit_x = [&](int xb) {
#pragma unroll
    for (int k = 0; k < kXTasks; ++k) {
      const v4u u = f.xq[k] ^ 0x80808080u;
      const v4h h0 = codes_to_f16(u[0]), h1 = codes_to_f16(u[1]), h2 = codes_to_f16(u[2]), h3 = codes_to_f16(u[3]);
      *reinterpret_cast<v8h*>(xs_buf[xb] + lc.x_lds[k]) = v8h{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      // the second 8 channels: chunk + 1 before the swizzle
      *reinterpret_cast<v8h*>(xs_buf[xb] + (lc.x_lds[k] ^ 8)) = v8h{h2[0], h2[1], h2[2], h2[3], h3[0], h3[1], h3[2], h3[3]};
    }
  };
  // ---- commit a prefetched item to LDS.  Rows past the sequence end arrived as zeros;
  // channels past P and states past N hold zeros or values that only meet zeros (the C codes
  // past N are zero, and rows past P are never stored).
  auto commit = [&](int bf) {
    if (tid < kMaxQ) {
      acs2_buf[bf][tid] = f.acs * kLog2e;
      dts_buf[bf][tid] = f.dt;
    }
    {
      const float dm = tid < kMaxQ ? wave_max(f.dt) : 0.f;   // dt >= 0; waves 4..7 load none
      if (lane == 0) red_buf[bf][wave] = dm;
    }
    if (tid < kMaxP) {
      hsc_buf[bf][tid] = kPC ? f.hs / f.sxp : f.hs;
      if constexpr (kCorr) mu_buf[bf][tid] = f.mu;
      if constexpr (kPC) sxc_buf[bf][tid] = f.sxp;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) *reinterpret_cast<v4u*>(Hq_buf[bf] + lc.h_lds[q]) = f.hq[q];
    if constexpr (!kPS) commit_x(bf);
  };
  // B of a new group (its prefetch arrived with the item's); written while no wave reads B.
  // kPS: the two limb planes of V = rint(256 q_B sigma[n] / 2^s); this thread's pieces all hold
  // states 16 (tid % 8) .. + 15, and the 8 threads tid % 8 = 0..7 together cover the 128 states,
  // so 2^s is an 8-lane maximum
  auto commit_b = [&](int grp) {
    // B goes to LDS in the same state order as the carried state and the C operand: in a full
    // 64-state block, dword q of natural piece t (states 16 t + 4 q ..) lands at dword t of
    // piece q (the 16-byte-chunk swizzle keeps the dword position)
    const int t = tid & 3;                             // piece within its 64-state block
    const bool full = 64 * ((tid >> 2) & 1) + 64 <= N;   // that block is full
    auto store_piece = [&](int plane, int k, const v4u& w) {
      int8_t* const bp = Bs + plane * kMaxQ * kMaxN;
      if (full) {
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<uint32_t*>(bp + ((lc.b_lds[k] ^ ((t ^ q) << 4)) + 4 * t)) = w[q];
      } else {
        *reinterpret_cast<v4u*>(bp + lc.b_lds[k]) = w;
      }
    };
    if constexpr (kPS) {
      const int sg = tid & 7;
      const Rsrc rsb = make_rsrc(a.B_scale + grp * N, uint32_t(N) * 4u), rsc = make_rsrc(a.C_scale + grp * N, uint32_t(N) * 4u);
      float sig[16];
      float m = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t o = 16 * sg < N ? uint32_t(16 * sg + 4 * u) * 4u : kOutOfRange;
        const v4f sb = __builtin_bit_cast(v4f, buf_load16(rsb, o)), sc = __builtin_bit_cast(v4f, buf_load16(rsc, o));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sig[4 * u + i] = sb[i] * sc[i];
          m = fmaxf(m, sig[4 * u + i]);
        }
      }
      m = group_max<8>(m);
      const int s2 = ceil_log2_pos(m);
      const float r256 = exp2i(8 - s2);   // 256 / 2^s
      if (tid == 0) sig2_s = exp2i(s2);
#pragma unroll
      for (int i = 0; i < 16; ++i) sig[i] *= r256;   // exact: a power of two
#pragma unroll
      for (int k = 0; k < kBTasks; ++k) {
        v4u hi, lo;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t wh = 0, wl = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int code = int(int8_t((f.bq[k][q] >> (8 * i)) & 0xffu));
            const int V = __float2int_rn(float(code) * sig[4 * q + i]);
            const int vh = (V + 128) >> 8;   // floor((V + 128) / 256): V - 256 vh in [-128, 127]
            wh |= (uint32_t(vh) & 0xffu) << (8 * i);
            wl |= (uint32_t(V - 256 * vh) & 0xffu) << (8 * i);
          }
          hi[q] = wh;
          lo[q] = wl;
        }
        store_piece(0, k, hi);
        store_piece(1, k, lo);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kBTasks; ++k) store_piece(0, k, f.bq[k]);
    }
  };
  // the C codes of this lane's output rows arrive with a new group's prefetch; they are kept
  // before the next prefetch reuses the registers
  auto keep_c = [&] {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) cqs[pass][s2] = f.cq[pass][s2];
  };

  // The loop is rotated: an item's prefetch, its predecessor's stores and its commit all lie in
  // one trip, so the commit's wait for the prefetched data counts back over a fixed number of
  // stores (unconditional buffer stores) and never waits for the stores themselves.
  ItemPos cur = item_at(it, a);
  prefetch<kCorr, kPC>(f, item_rsrc<kPC>(cur, a), lc, xrow, true, N, kg);
  prefetch_x(f, item_rsrc(cur, a), lc);
  commit(0);
  if constexpr (kPS) commit_x(0);
  commit_b(cur.g);
  __syncthreads();
  keep_c();
  int buf = 0;   // the current item's buffer

  for (; it < it_end; ++it) {
    const int len = cur.len;
    const int hu = __builtin_amdgcn_readfirstlane(cur.h);
    const int gu = __builtin_amdgcn_readfirstlane(cur.g);
    // per-item scalars through the scalar cache (read-only data)
    typedef const __attribute__((address_space(4))) float* cfp;
    const float sx = kPC ? 1.f : *cfp(a.x_scale + hu);
    const float sB = kPS ? 1.f : *cfp(a.B_scale + gu), sC = kPS ? 1.f : *cfp(a.C_scale + gu);
    const float Dh = a.D ? *cfp(a.D + hu) : 0.f;
    const uint32_t yrow = uint32_t(a.nheads * P);
    const Rsrc ry = make_rsrc(a.y + wide(cur.row, uint32_t(P)), (uint32_t(len - 1) * yrow + uint32_t(P)) * 2u);
    __builtin_amdgcn_sched_barrier(0);

    // the next item's loads (the last trip re-reads its own item); only the B and C loads
    // depend on whether the next item starts a new group
    ItemPos nxt = cur;
    bool nxt_bc = false;
    if (it + 1 < it_end) nxt_bc = item_next(nxt, it, a);
    const ItemRsrc nrs = item_rsrc<kPC>(nxt, a);
    prefetch<kCorr, kPC>(f, nrs, lc, xrow, nxt_bc, N, kg);
    __builtin_amdgcn_sched_barrier(0);

    // this trip's view of the per-item tiles
    const _Float16* const xs = xs_buf[kPS ? 0 : buf];
    const int8_t* const Hq = Hq_buf[buf];
    const LDSP int8_t* const hqb[2] = {lds_base(Hq + hq_lane[0]), lds_base(Hq + hq_lane[1])};
    const LDSP float* const hsb = lds_base(hsc_buf[buf] + 4 * kg);   // + 16 pt: this lane's row scales
    const LDSP float* const mub = lds_base(mu_buf[buf] + (kCorr ? 4 * kg : 0));   // + 16 pt: its corrections
    const LDSP float* const sxb = lds_base_if<kPC>(sxc_buf[buf] + 4 * kg);   // + 16 pt: its x scales
    const float* const acs2 = acs2_buf[buf];
    const float* const dts = dts_buf[buf];
    const float* const red = red_buf[buf];
    float dtmax = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) dtmax = fmaxf(dtmax, red[i]);
    // Power-of-two guard 2^-kM on the fp16 operand M': the masked C.B^T entries stay within
    // |M'| <= N 127^2 dtmax 2^-kM <= 2^15 and the D term folded into its diagonal within
    // |D'| = |D| / (sC sB) 2^-kM <= 2^14, so their sum is a finite fp16.  Clamped so that 2^kM
    // and 2^-kM are exact.
    // (kPS: the C.B^T entries are 256 G_hi + G_lo in units of 2^s / 256, |.| <= N 127 32512)
    const float sCB = kPS ? sig2_s * (1.f / 256.f) : sC * sB;
    const float DsCB = Dh * __builtin_amdgcn_rcpf(sCB);   // scales are positive: |D| / (sC sB) = |D / (sC sB)|
    const int kM = min(max(max(ceil_log2_pos(float(N) * (kPS ? 127.f * 32512.f : 16129.f) * dtmax) - 15,
                               ceil_log2_pos(fabsf(DsCB)) - 14),
                           -120), 120);
    const float s_in = sx * sCB * exp2i(kM);
    const float fkM = float(kM);
    const float Dp = DsCB * exp2i(-kM);   // D' (0 without D)
    // carried-state readout factor sC / (256 s_in) = 2^-(kM + 8) / (sx sB), times exp(Acs_l0) per
    // pass (kPS: the carried state already holds the C scales, so 1 / (256 s_in))
    const float Ek = __builtin_amdgcn_rcpf(kPS ? sx * sCB : sx * sB) * exp2i(-kM - 8);

    // The lane index is re-materialized per item (an empty asm makes it opaque), so that the
    // per-lane masks below (causal mask, store guards) are recomputed with a few compares
    // instead of being hoisted out of the item loop into scalar registers that would spill.
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
    const int lcol_v = lane_v & 15, kg_v = lane_v >> 4;

    auto do_pass = [&](const int lb, const v4i (&cq)[2]) {
      const int l0 = 16 * lb;
      const int l = l0 + lcol_v;
      const bool lvalid = l < len;
      // the 32-token block that holds the diagonal (uniform: scalar loop bounds below)
      const int jdiag = __builtin_amdgcn_readfirstlane(l0 & ~31);
      const bool half = l0 != jdiag;       // its first 16 tokens lie before row l0
      const float a_l = acs2[l];
      const float a_0 = acs2[l0];

      // Token weights times 2^-kM.  Blocks before the diagonal: relative to row l0,
      // exp(Acs_l0 - Acs_j) dt_j <= dt_j.  The 32 tokens of the diagonal block: relative to its
      // first token m = jdiag, exp(Acs_m - Acs_j) dt_j >= dt_j, which with the row factor
      // exp(Acs_l - Acs_m) <= 1 gives the decay of each entry.  That factorized form is used
      // while the block's weights stay below 2^100 (their products with the int32 C.B^T
      // entries are then finite fp32); otherwise every entry's decay is taken on its own.
      const float a_m = acs2[jdiag];
      bool big = false;
      {
        const int j = 4 * lane;   // four tokens per lane, all on one side of jdiag (a multiple of 32)
        if (j < jdiag + 32) {
          const float4 a4 = *reinterpret_cast<const float4*>(&acs2[j]);
          const float4 d4 = *reinterpret_cast<const float4*>(&dts[j]);
          const float r = (j < jdiag ? a_0 : a_m) - fkM;
          float4 w;
          w.x = __builtin_amdgcn_exp2f(r - a4.x) * d4.x;
          w.y = __builtin_amdgcn_exp2f(r - a4.y) * d4.y;
          w.z = __builtin_amdgcn_exp2f(r - a4.z) * d4.z;
          w.w = __builtin_amdgcn_exp2f(r - a4.w) * d4.w;
          *reinterpret_cast<float4*>(&wlw[j]) = w;
          // the weights are >= 0, so their sum bounds each; an inf weight times dt = 0 (rows past
          // the sequence end) is NaN, which fails the comparison as well
          const bool fin = (w.x + w.y) + (w.z + w.w) < 0x1p100f;
          big = (j >= jdiag) & !fin;
        }
      }
      const bool factored = __builtin_amdgcn_ballot_w64(big) == 0;
      __builtin_amdgcn_wave_barrier();
      const float u_l = __builtin_amdgcn_exp2f(a_l - a_0);

      // carried state read out by C on the INT8 matrix cores: y_off^T[p][l] =
      // exp(Acs_l) sC hs_p / 256 * (256 yo1 + yo2).  It starts the accumulator of the blocks
      // before the diagonal, which the epilogue scales by u_l s_in = exp(Acs_l - Acs_l0) s_in,
      // hence the factor kap_p = exp(Acs_l0) sC hs_p / (256 s_in).
      v4i yo1[4], yo2[4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const v4i h1 = lds_ld<v4i>(hqb[s2], 16 * kMaxN * pt);
          const v4i h2 = lds_ld<v4i>(hqb[s2], kHPlane + 16 * kMaxN * pt);
          const v4i z = {0, 0, 0, 0};
          yo1[pt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(h1, cq[s2], s2 == 0 ? z : yo1[pt], 0, 0, 0);
          yo2[pt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(h2, cq[s2], s2 == 0 ? z : yo2[pt], 0, 0, 0);
        }
      }
      const float E = __builtin_amdgcn_exp2f(fminf(a_0, 0.f)) * Ek;
      v4f yf[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const float4 hs = lds_f4(hsb, 16 * pt);
        const float hv[4] = {hs.x, hs.y, hs.z, hs.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) yf[pt][i] = float((yo1[pt][i] << 8) + yo2[pt][i]) * (E * hv[i]);
      }

      // G^T of the 16 tokens from jj against this pass's rows (kPS: 256 G_hi + G_lo of the two
      // B limb planes; the lo plane lies one plane past the hi plane)
      auto cbt = [&](int jj) {
        const v4i b0 = lds_ld<v4i>(bs_lane, jj * kMaxN);
        const v4i b1 = lds_ld<v4i>(bs_lane2, jj * kMaxN);
        v4i g = __builtin_amdgcn_mfma_i32_16x16x64_i8(b0, cq[0], v4i{0, 0, 0, 0}, 0, 0, 0);
        g = __builtin_amdgcn_mfma_i32_16x16x64_i8(b1, cq[1], g, 0, 0, 0);
        if constexpr (kPS) {
          const v4i l0 = lds_ld<v4i>(bs_lane, jj * kMaxN + kMaxQ * kMaxN);
          const v4i l1 = lds_ld<v4i>(bs_lane2, jj * kMaxN + kMaxQ * kMaxN);
          v4i gl = __builtin_amdgcn_mfma_i32_16x16x64_i8(l0, cq[0], v4i{0, 0, 0, 0}, 0, 0, 0);
          gl = __builtin_amdgcn_mfma_i32_16x16x64_i8(l1, cq[1], gl, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) g[i] = (g[i] << 8) + gl[i];   // exact: |.| <= 128 127 32512 < 2^31
        }
        return g;
      };

      // intra-chunk part, 32 tokens per step: blocks before the diagonal use the factorized decay.
      // G^T for a step on the INT8 matrix cores, then M' = fp16(G w) and y^T += x^T M'^T; two
      // steps at a time with their own G and M' registers, so that the second step's integer
      // products overlap the first step's conversions.
      auto gstep = [&](int jb, v4i (&gm)[2], float4 (&w4)[2]) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int js = jb + 16 * sb;
          w4[sb] = lds_f4(wl_lane, js);
          gm[sb] = cbt(js);
        }
      };
      auto mstep = [&](int jb, const v4i (&gm)[2], const float4 (&w4)[2]) {
        v8h xop[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const v4h lo = tr16(xs + xa[pt] + jb * kMaxP);
          const v4h hi = tr16(xs + xa[pt] + (jb + 16) * kMaxP);
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
      };
      int jb = 0;
      for (; jb + 32 < jdiag; jb += 64) {
        v4i ga[2], gb[2];
        float4 wa[2], wb[2];
        gstep(jb, ga, wa);
        gstep(jb + 32, gb, wb);
        mstep(jb, ga, wa);
        mstep(jb + 32, gb, wb);
      }
      if (jb < jdiag) {
        v4i ga[2];
        float4 wa[2];
        gstep(jb, ga, wa);
        mstep(jb, ga, wa);
      }

      // the block holding the diagonal, each entry with its own decay (factorized around the
      // block's first token, or the exact exp): sub-block 0 (tokens jdiag..+15) lies before row
      // l0 when `half`, else it holds the diagonal and sub-block 1 is masked entirely; the
      // diagonal sub-block gets the causal mask and D' on j == l.
      v4f yd[4];
      {
        const int jb = jdiag;
        const int j1 = jb + 16;   // sub-block 1 (jdiag <= 224: inside the 256-row tiles)
        v4i gm[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) gm[sb] = cbt(sb == 0 ? jb : j1);
        v8h mop;
        if (factored) {
          const float e_l = __builtin_amdgcn_exp2f(a_l - a_m);   // rows l >= m: <= 1
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            const bool diag_sb = half ? sb == 1 : sb == 0;
            if (!half && sb == 1) {   // entirely after the block's rows
#pragma unroll
              for (int i = 0; i < 4; ++i) mop[4 + i] = _Float16(0.f);
              continue;
            }
            const float4 f4 = lds_f4(wl_lane, sb == 0 ? jb : j1);
            const float fv[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float m = float(gm[sb][i]) * fv[i] * e_l;
              if (diag_sb) {
                const int j = jb + 16 * sb + 4 * kg_v + i;
                m = j < l ? m : (j == l ? m + Dp : 0.f);
              }
              mop[4 * sb + i] = _Float16(m);
            }
          }
        } else {
          const float a_lk = a_l - fkM;
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            const bool diag_sb = half ? sb == 1 : sb == 0;
            if (!half && sb == 1) {
#pragma unroll
              for (int i = 0; i < 4; ++i) mop[4 + i] = _Float16(0.f);
              continue;
            }
            const int jq = (sb == 0 ? jb : j1) + 4 * kg;
            const float4 a4 = *reinterpret_cast<const float4*>(&acs2[jq]);
            const float4 d4 = *reinterpret_cast<const float4*>(&dts[jq]);
            const float av[4] = {a4.x, a4.y, a4.z, a4.w};
            const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float m = float(gm[sb][i]) * __builtin_amdgcn_exp2f(fminf(a_lk - av[i], -fkM)) * dv[i];
              if (diag_sb) {
                const int j = jb + 16 * sb + 4 * kg_v + i;
                m = j < l ? m : (j == l ? m + Dp : 0.f);
              }
              mop[4 * sb + i] = _Float16(m);
            }
          }
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const v4h lo = tr16(xs + xa[pt] + jb * kMaxP);
          const v4h hi = tr16(xs + xa[pt] + j1 * kMaxP);
          const v8h xop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          yd[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, mop, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
      }

      // ---- epilogue: lane holds y[l, 16 pt + 4 kg + i], i = 0..3
      const float c_f = u_l * s_in;
      v2u o4[4];   // channels 16 pt + 4 kg .. + 3 of row l, as fp16
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        v4h out;
        if constexpr (kPC) {
          const float4 x4 = lds_f4(sxb, 16 * pt);
          const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
          float mv[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (kCorr) {
            const float4 m4 = lds_f4(mub, 16 * pt);
            mv[0] = m4.x, mv[1] = m4.y, mv[2] = m4.z, mv[3] = m4.w;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = _Float16(fmaf(xv[i], fmaf(yf[pt][i], c_f, yd[pt][i] * s_in), mv[i]));
        } else if constexpr (kCorr) {
          const float4 m4 = lds_f4(mub, 16 * pt);
          const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = _Float16(fmaf(yf[pt][i], c_f, fmaf(yd[pt][i], s_in, mv[i])));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = _Float16(fmaf(yf[pt][i], c_f, yd[pt][i] * s_in));
        }
        o4[pt] = __builtin_bit_cast(v2u, out);
      }
      // Channel tiles pt and pt + 1 trade halves between 16-lane rows (the odd rows of the first
      // operand with the even rows of the second): a lane then holds 8 consecutive channels,
      // 16 (pt + kg % 2) + 8 (kg / 2) .. + 7, and stores them with one 16-byte store.
#pragma unroll
      for (int pp = 0; pp < 4; pp += 2) {
        v4u v;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto r = __builtin_amdgcn_permlane16_swap(o4[pp][d], o4[pp + 1][d], false, false);
          v[d] = r[0];
          v[2 + d] = r[1];
        }
        const int ch0 = 16 * (pp + (kg_v & 1)) + 8 * (kg_v >> 1);
        // unconditional store: rows past len and channels past P go out of range (dropped)
        const uint32_t voff = (uint32_t(l) * yrow + uint32_t(ch0)) * 2u;
        const bool ok = lvalid & (ch0 < P);   // a select, not a branch
        __builtin_amdgcn_raw_buffer_store_b128(v, ry, ok ? voff : kOutOfRange, 0, 0);
      }
    };

    // two 16-row blocks per wave, l and 15 - l (balanced work), the next item's x codes loaded
    // between them.  Both passes run on every trip (a block past Q / 16 computes on zero rows and
    // stores nothing), so that the number of stores after each load is the same on every path.
    do_pass(row_block(wave, 0), cqs[0]);
    __builtin_amdgcn_sched_barrier(0);
    prefetch_x(f, nrs, lc);
    __builtin_amdgcn_sched_barrier(0);
    do_pass(row_block(wave, 1), cqs[1]);
    commit(buf ^ 1);   // the other buffer: its last readers passed the previous barrier
    __syncthreads();   // the next item is in LDS, and every wave is done with this one
    if constexpr (kPS) commit_x(0);   // the single x tile: every wave is done with it now
    if (nxt_bc) {
      commit_b(nxt.g);
      __syncthreads();
      keep_c();
    } else {
      if constexpr (kPS) __syncthreads();
    }
    cur = nxt;
    buf ^= 1;
  }
}

}  // namespace

hipError_t launch_chunk_output(const ScanShape& s, const ScanArgs& a, hipStream_t stream) {
  Params p{a.x, a.x_scale, a.B, a.B_scale, a.C, a.C_scale, a.dtc, a.D, a.acs, a.hprev, a.hscale, a.ycorr, a.y,
           s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk, s.nchunks,
           s.batch * s.nchunks * s.nheads,
           make_fastdiv(uint32_t(s.nheads)), make_fastdiv(uint32_t(s.nchunks)),
           make_fastdiv(uint32_t(s.nheads / s.ngroups))};
  // one persistent block per CU (the LDS footprint allows one resident block)
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    cus = 256;
  const int nblocks = p.nitems < cus ? p.nitems : cus;
  auto go = [&](auto corr, auto ps, auto pc) {
    hipLaunchKernelGGL((chunk_output_kernel<decltype(corr)::value, decltype(ps)::value, decltype(pc)::value>),
                       dim3(nblocks), dim3(kThreads), 0, stream, p);
  };
  using T = std::true_type;
  using F = std::false_type;
  const int sel = (p.ycorr ? 4 : 0) | (a.bc_per_state ? 2 : 0) | (a.x_per_channel ? 1 : 0);
  switch (sel) {
    case 0: go(F{}, F{}, F{}); break;
    case 1: go(F{}, F{}, T{}); break;
    case 2: go(F{}, T{}, F{}); break;
    case 3: go(F{}, T{}, T{}); break;
    case 4: go(T{}, F{}, F{}); break;
    case 5: go(T{}, F{}, T{}); break;
    case 6: go(T{}, T{}, F{}); break;
    default: go(T{}, T{}, T{}); break;
  }
  return hipGetLastError();
}

}  // namespace ssdq
