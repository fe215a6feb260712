/*
 * ssd_oracle.c -- CPU oracle for the INT8-input Mamba-2 SSD scan.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * HIP path is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product library never does, and it
 * shares no code, header or constant with the HIP sources.
 *
 * What it computes (all state arithmetic in IEEE double):
 *
 *  - oracle_quantize_f16: the static INT8 quantizer.  The 8-bit SSD inputs
 *    x, B, C (Quamba2 rebuttal, "impact of SSD quantization") use one static
 *    scale per head for x and one per state group for B and C (SSDi8,
 *    Table 10, per-H(G); Quamba project page, static quantization).  A code is
 *    rint(v / s) with the fp32 quotient correctly rounded, rounding to nearest
 *    with ties to even, then saturated to [-127, 127]; NaN quotients give 0.
 *
 *  - oracle_ssd_sequential: the selective-SSM recurrence written out token by
 *    token (Ternary Mamba, Section 1: h_t = Abar_t h_{t-1} + Bbar_t x_t), with
 *    the zero-order-hold decay Abar_t = exp(dt_t * A_h) and Bbar_t = dt_t * B_t,
 *    and the readout y_t = C_t . h_t + D_h x_t, over the DEQUANTIZED codes
 *    x = s_x[h] q_x, B = s_B[g] q_B, C = s_C[g] q_C (exact in double), or, with scales
 *    per (group, state) (SSDi8 Table 10: per-P(N) and per-H(G) together), B = s_B[g, n] q_B
 *    and C = s_C[g, n] q_C; with x scales per (head, channel), x = s_x[h, p] q_x (the static
 *    scales that Quamba2's sort-and-cluster of channels leaves behind, one per channel
 *    cluster, expanded to every channel).  The last argument holds the scale layout: bit 0 set
 *    for B, C per (group, state), bit 1 for x per (head, channel).  Head h reads group
 *    g = h / (H / G).  Optionally records the state at every chunk boundary (the state
 *    entering chunk c, i.e. after token cQ - 1).
 *
 *  - oracle_ssd_sequential_state_f16: the same recurrence with the state cached
 *    in IEEE binary16 between tokens (a lower-precision cached decode state, as
 *    the Quamba2 rebuttal's Tables R7/R8 discuss for 8-bit states): each token's
 *    update is formed in double from the cached value, y_t reads that update,
 *    and the cache keeps it rounded to the nearest binary16 (ties to even).
 *
 *  - oracle_ssd_sequential_state_i8: the same recurrence with the state cached
 *    as 8-bit codes (the 8-bit cached states of those tables) with one binary32
 *    scale per state row: each token's update in double from the decoded cache,
 *    y_t from that update, then every row re-quantized symmetrically to
 *    [-127, 127] with s = max|row| / 127 (the reading stated at
 *    requantize_row_i8).
 *
 *  - the output correction (SSDi8's mean correction: its abstract describes a correction derived
 *    from error statistics gathered per channel, Figure 1b labels it a mean correction, Table 6
 *    ablates it and Table 16 times it; no algebra is given): every y the recurrences above produce may carry a
 *    per-(head, channel) additive term y_corr[h, p].  oracle_ssd_sequential_values runs the same
 *    recurrence over real-valued (unquantized) inputs; the calibration of y_corr as the mean,
 *    over a calibration draw's (batch, token) positions, of that reference's y minus the
 *    quantized recurrence's y is written out in oracle/__init__.py (mean_correction).
 *
 *  - oracle_frontend / oracle_softplus_dt: the block's front end ahead of the
 *    quantizer (depthwise causal conv1d + bias + SiLU, rounded to binary16) and
 *    dt = softplus(dt_raw + dt_bias), each as the reading stated at the function.
 *
 *  - oracle_chunk_cumsum / oracle_chunk_state: the two per-chunk quantities of
 *    the chunked (state-space-duality) evaluation, each from its definition:
 *    Acs[c, j] = sum_{i <= j} dt_{cQ+i} A_h  and
 *    S_c[p, n] = sum_j exp(Acs[c, last] - Acs[c, j]) dt_j x[j, p] B[j, n]
 *    (the decay-times-dt factor is SSDi8's LUT_state, Figure 3a).
 *
 * Parity pins that make this trustworthy live in tests/ (closed forms,
 * brute force, an independent numpy chunked evaluation, invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE binary16 -> double, by the format's definition:
 * normal: (-1)^s 2^(e-15) (1 + m/1024); subnormal: (-1)^s 2^-14 (m/1024). */
static double half_bits_to_double(uint16_t bits) {
  int s = bits >> 15;
  int e = (bits >> 10) & 0x1f;
  int m = bits & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24);
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25);
  }
  return s ? -v : v;
}

static int8_t quantize_one(uint16_t bits, float scale) {
  float v = (float)half_bits_to_double(bits); /* exact: binary16 is a subset of binary32 */
  volatile float t = v / scale;               /* one IEEE binary32 division */
  if (isnan(t)) return 0;
  float r = rintf(t); /* default rounding mode: nearest, ties to even */
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

/* q[r, k, i] = quantize(x[r, k, i], scale[k]) for a tensor viewed as (rows, nscale, inner). */
void oracle_quantize_f16(const uint16_t* x, int8_t* q, const float* scale, int64_t rows, int32_t nscale,
                         int32_t inner) {
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t k = 0; k < nscale; ++k)
      for (int32_t i = 0; i < inner; ++i) {
        int64_t e = (r * nscale + k) * (int64_t)inner + i;
        q[e] = quantize_one(x[e], scale[k]);
      }
}

/* The same quantizer with one scale per (k, i): q[r, k, i] = quantize(x[r, k, i], scale[k * inner + i])
 * (B and C with a scale per (group, state), SSDi8 Table 10's per-P(N) axis together with per-H(G)). */
void oracle_quantize_f16_per_channel(const uint16_t* x, int8_t* q, const float* scale, int64_t rows, int32_t nscale,
                                     int32_t inner) {
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t k = 0; k < nscale; ++k)
      for (int32_t i = 0; i < inner; ++i) {
        int64_t e = (r * nscale + k) * (int64_t)inner + i;
        q[e] = quantize_one(x[e], scale[(int64_t)k * inner + i]);
      }
}

/* One (b, h) sequence of the recurrence.
 *  qx (batch, L, H, P) int8, qB/qC (batch, L, G, N) int8, dt (batch, L, H),
 *  A[H], D[H] (NULL = 0), h0 (batch, H, P, N) float (NULL = 0).
 *  y_out: L x P doubles; h_out: P x N doubles (final state).
 *  bound_out (optional, chunk > 0): ceil(L/chunk) x P x N doubles, the state
 *  entering each chunk. */
/* The binary16 value nearest to v (ties to even), by the format's definition: binary16 has
 * 11 significant bits, exponents -14 .. 15 and subnormals spaced 2^-24, so in the binade
 * [2^E, 2^(E+1)) the representable values are the multiples of 2^(E-10) (2^-24 below 2^-14);
 * magnitudes that round to 2^16 or beyond overflow to infinity.  NaN stays NaN. */
static double round_to_binary16(double v) {
  if (v != v || v == 0.0) return v;
  const double a = fabs(v);
  double quantum = 0x1p-24;
  if (a >= 0x1p-14) {
    int e2;
    frexp(a, &e2);                    /* a = f 2^e2, f in [0.5, 1): binade exponent E = e2 - 1 */
    quantum = ldexp(1.0, e2 - 1 - 10);
  }
  const double r = nearbyint(a / quantum) * quantum;   /* a / quantum is exact; ties to even */
  if (r >= 65536.0) return copysign(INFINITY, v);
  return copysign(r, v);
}

/* out[i] = the binary16 value nearest to in[i] (for pinning the rounding on its own). */
void oracle_round_binary16(const double* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_to_binary16(in[i]);
}

/* One state row cached as 8-bit codes with one binary32 scale (an 8-bit cached SSM state,
 * Quamba2 rebuttal Tables R7/R8; the scale granularity, one per state row (b, h, p), and
 * its choice from the row's largest magnitude are this oracle's reading, the same symmetric
 * max/127 rule the pages use for activations).  s = binary32(max_n |row[n]| / 127); each
 * code is row[n] / s rounded to nearest with ties to even and saturated to [-127, 127]; the
 * row becomes s * code.  A row whose scale would not be a normal binary32 (zero, or below
 * 2^-126, i.e. max|row| below about 1.5e-36) is flushed: zero codes and s = 0. */
static void requantize_row_i8(double* row, int32_t N, int8_t* q, float* s_out) {
  double m = 0.0;
  for (int32_t n = 0; n < N; ++n) m = fmax(m, fabs(row[n]));
  float s = (float)(m / 127.0);
  if (s < 0x1p-126f) s = 0.0f;
  for (int32_t n = 0; n < N; ++n) {
    double c = 0.0;
    if (s > 0.0f) {
      c = nearbyint(row[n] / (double)s);
      c = c > 127.0 ? 127.0 : (c < -127.0 ? -127.0 : c);
    }
    q[n] = (int8_t)c;
    row[n] = (double)s * c;
  }
  *s_out = s;
}

/* Re-quantize rows on their own (for pinning): rows x N doubles in; codes, scales and the
 * decoded rows out. */
void oracle_requantize_rows_i8(const double* in, int64_t rows, int32_t N, int8_t* q, float* s, double* out) {
  for (int64_t r = 0; r < rows; ++r) {
    memcpy(out + r * N, in + r * N, sizeof(double) * N);
    requantize_row_i8(out + r * N, N, q + r * N, s + r);
  }
}

/* round_state: 0 none, 1 binary16 per element, 2 8-bit codes per row (requantize_row_i8).
 * q0/s0 (mode 2, optional): the starting state as codes (batch, H, P, N) and row scales
 * (batch, H, P); q_out/s_out: the final codes and scales; u_last: the last token's update
 * before it is re-quantized (P x N); s_steps (optional): every token's row scales (L x P). */
static void ssd_sequential(const int8_t* qx, const float* sx, const int8_t* qB, const float* sB,
                           const int8_t* qC, const float* sC, const float* dt, const float* A,
                           const float* D, const float* h0, int32_t batch, int64_t L, int32_t H,
                           int32_t P, int32_t N, int32_t G, int32_t b, int32_t h, double* y_out,
                           double* h_out, int32_t chunk, double* bound_out, int round_state,
                           const int8_t* q0, const float* s0, int8_t* q_out, float* s_out, double* u_last,
                           float* s_steps, const float* ycorr, int32_t scale_flags) {
  (void)batch;
  const int32_t g = h / (H / G);
  const int bc_per_state = scale_flags & 1, x_per_channel = (scale_flags >> 1) & 1;
  double* S = (double*)calloc((size_t)P * N, sizeof(double));
  double* xv = (double*)malloc(sizeof(double) * P);
  double* Bv = (double*)malloc(sizeof(double) * N);
  double* Cv = (double*)malloc(sizeof(double) * N);
  int8_t* codes = (int8_t*)calloc((size_t)P * N, 1);
  float* scales = (float*)calloc((size_t)P, sizeof(float));
  if (h0) {
    const float* src = h0 + ((int64_t)b * H + h) * P * N;
    for (int64_t i = 0; i < (int64_t)P * N; ++i) S[i] = (double)src[i];
  }
  if (q0 && s0) {
    const int64_t bh = (int64_t)b * H + h;
    for (int32_t p = 0; p < P; ++p)
      for (int32_t n = 0; n < N; ++n)
        S[(int64_t)p * N + n] = (double)s0[bh * P + p] * (double)q0[(bh * P + p) * N + n];
  }
  const double Ah = (double)A[h];
  const double Dh = D ? (double)D[h] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    if (chunk > 0 && bound_out && t % chunk == 0)
      memcpy(bound_out + (t / chunk) * (int64_t)P * N, S, sizeof(double) * P * N);
    const int64_t row = (int64_t)b * L + t;
    const double d = (double)dt[row * H + h];
    const double a = exp(d * Ah);
    for (int32_t p = 0; p < P; ++p)   /* x's scale of head h, or of (head h, channel p) */
      xv[p] = (double)sx[x_per_channel ? (int64_t)h * P + p : h] * (double)qx[(row * H + h) * P + p];
    for (int32_t n = 0; n < N; ++n) {
      const int32_t k = bc_per_state ? g * N + n : g;   /* scale of state n of group g */
      Bv[n] = (double)sB[k] * (double)qB[(row * G + g) * N + n];
      Cv[n] = (double)sC[k] * (double)qC[(row * G + g) * N + n];
    }
    for (int32_t p = 0; p < P; ++p) {
      double* Sp = S + (int64_t)p * N;
      const double u = d * xv[p];
      double acc = 0.0;
      for (int32_t n = 0; n < N; ++n) {
        Sp[n] = a * Sp[n] + u * Bv[n];
        acc += Cv[n] * Sp[n];
        if (round_state == 1) Sp[n] = round_to_binary16(Sp[n]);
      }
      const double mu = ycorr ? (double)ycorr[(int64_t)h * P + p] : 0.0;
      y_out[t * P + p] = acc + Dh * xv[p] + mu;
      if (round_state == 2) {
        if (u_last && t == L - 1) memcpy(u_last + (int64_t)p * N, Sp, sizeof(double) * N);
        requantize_row_i8(Sp, N, codes + (int64_t)p * N, scales + p);
        if (s_steps) s_steps[t * P + p] = scales[p];
      }
    }
  }
  memcpy(h_out, S, sizeof(double) * P * N);
  if (q_out) memcpy(q_out, codes, (size_t)P * N);
  if (s_out) memcpy(s_out, scales, sizeof(float) * P);
  free(codes);
  free(scales);
  free(S);
  free(xv);
  free(Bv);
  free(Cv);
}

/* The recurrence with an fp32-exact (double) state. */
void oracle_ssd_sequential(const int8_t* qx, const float* sx, const int8_t* qB, const float* sB,
                           const int8_t* qC, const float* sC, const float* dt, const float* A,
                           const float* D, const float* h0, int32_t batch, int64_t L, int32_t H,
                           int32_t P, int32_t N, int32_t G, int32_t b, int32_t h, double* y_out,
                           double* h_out, int32_t chunk, double* bound_out, const float* ycorr,
                           int32_t scale_flags) {
  ssd_sequential(qx, sx, qB, sB, qC, sC, dt, A, D, h0, batch, L, H, P, N, G, b, h, y_out, h_out, chunk, bound_out, 0,
                 NULL, NULL, NULL, NULL, NULL, NULL, ycorr, scale_flags);
}

/* The recurrence with the state cached in binary16 between tokens (h0 is taken as given). */
void oracle_ssd_sequential_state_f16(const int8_t* qx, const float* sx, const int8_t* qB, const float* sB,
                                     const int8_t* qC, const float* sC, const float* dt, const float* A,
                                     const float* D, const float* h0, int32_t batch, int64_t L, int32_t H,
                                     int32_t P, int32_t N, int32_t G, int32_t b, int32_t h, double* y_out,
                                     double* h_out, const float* ycorr, int32_t scale_flags) {
  ssd_sequential(qx, sx, qB, sB, qC, sC, dt, A, D, h0, batch, L, H, P, N, G, b, h, y_out, h_out, 0, NULL, 1,
                 NULL, NULL, NULL, NULL, NULL, NULL, ycorr, scale_flags);
}

/* The recurrence with the state cached as 8-bit codes and one scale per state row between
 * tokens, starting from codes q0 (batch, H, P, N) with row scales s0 (batch, H, P) (both NULL:
 * a zero state).  h_out: the final state decoded (P x N); q_out/s_out: its codes and scales;
 * u_last (optional): the last token's update before re-quantization; s_steps (optional): the
 * row scales after every token (L x P). */
void oracle_ssd_sequential_state_i8(const int8_t* qx, const float* sx, const int8_t* qB, const float* sB,
                                    const int8_t* qC, const float* sC, const float* dt, const float* A,
                                    const float* D, const int8_t* q0, const float* s0, int32_t batch, int64_t L,
                                    int32_t H, int32_t P, int32_t N, int32_t G, int32_t b, int32_t h,
                                    double* y_out, double* h_out, int8_t* q_out, float* s_out, double* u_last,
                                    float* s_steps, const float* ycorr, int32_t scale_flags) {
  ssd_sequential(qx, sx, qB, sB, qC, sC, dt, A, D, NULL, batch, L, H, P, N, G, b, h, y_out, h_out, 0, NULL, 2,
                 q0, s0, q_out, s_out, u_last, s_steps, ycorr, scale_flags);
}

/* The same recurrence over real-valued inputs, for one (b, h): x (batch, L, H, P), B and C
 * (batch, L, G, N) given as doubles (e.g. the binary16 activations before quantization), dt, A,
 * D, h0 as in oracle_ssd_sequential.  This is the unquantized reference the output correction is
 * calibrated against.  y_out: L x P; h_out: P x N. */
void oracle_ssd_sequential_values(const double* x, const double* Bm, const double* Cm, const float* dt,
                                  const float* A, const float* D, const float* h0, int32_t batch, int64_t L,
                                  int32_t H, int32_t P, int32_t N, int32_t G, int32_t b, int32_t h, double* y_out,
                                  double* h_out) {
  (void)batch;
  const int32_t g = h / (H / G);
  double* S = (double*)calloc((size_t)P * N, sizeof(double));
  if (h0) {
    const float* src = h0 + ((int64_t)b * H + h) * P * N;
    for (int64_t i = 0; i < (int64_t)P * N; ++i) S[i] = (double)src[i];
  }
  const double Ah = (double)A[h];
  const double Dh = D ? (double)D[h] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const int64_t row = (int64_t)b * L + t;
    const double d = (double)dt[row * H + h];
    const double a = exp(d * Ah);
    const double* xr = x + (row * H + h) * P;
    const double* Br = Bm + (row * G + g) * N;
    const double* Cr = Cm + (row * G + g) * N;
    for (int32_t p = 0; p < P; ++p) {
      double* Sp = S + (int64_t)p * N;
      const double u = d * xr[p];
      double acc = 0.0;
      for (int32_t n = 0; n < N; ++n) {
        Sp[n] = a * Sp[n] + u * Br[n];
        acc += Cr[n] * Sp[n];
      }
      y_out[t * P + p] = acc + Dh * xr[p];
    }
  }
  memcpy(h_out, S, sizeof(double) * P * N);
  free(S);
}

/* Front end of the SSD block (the causal convolution ahead of the SSD box, Quamba2 rebuttal
 * Tables R6/R7, kept in FP16 as Ternary Mamba's quantization section lists; SSDi8 Table 16's
 * Conv column).  The pages give no algebra for it; the reading taken is the one the rest
 * supports: a depthwise causal convolution of width dconv along the tokens of every channel of
 * the in-projection output xBC (channels x, then B, then C), zero before the first token, plus a
 * per-channel bias, then SiLU(v) = v / (1 + exp(-v)); the module's FP16 output is that value
 * rounded to binary16 (then quantized by the static quantizer above).
 *   xbc: (batch, L, C) binary16 bits; w: (C, dconv) (tap k multiplies token t - dconv + 1 + k);
 *   bias: (C) or NULL.  pre_out (optional): the convolution + bias; act_out: SiLU of it (both
 *   double, unrounded); act16_out: act rounded to the nearest binary16 (as a double). */
void oracle_frontend(const uint16_t* xbc, const float* w, const float* bias, int32_t dconv, int32_t batch,
                     int64_t L, int32_t C, double* pre_out, double* act_out, double* act16_out) {
  for (int32_t b = 0; b < batch; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int32_t ch = 0; ch < C; ++ch) {
        double v = bias ? (double)bias[ch] : 0.0;
        for (int32_t k = 0; k < dconv; ++k) {
          const int64_t src = t - dconv + 1 + k;
          if (src < 0) continue;
          v += (double)w[(int64_t)ch * dconv + k] * half_bits_to_double(xbc[((int64_t)b * L + src) * C + ch]);
        }
        const int64_t o = ((int64_t)b * L + t) * C + ch;
        const double a = v / (1.0 + exp(-v));
        if (pre_out) pre_out[o] = v;
        if (act_out) act_out[o] = a;
        act16_out[o] = round_to_binary16(a);
      }
}

/* dt = softplus(dt_raw + dt_bias[h]) (Ternary Mamba names dt_bias among the SSM parameters; the
 * softplus is Mamba's positive map for dt), softplus(v) = log(1 + exp(v)) evaluated as
 * max(v, 0) + log1p(exp(-|v|)), which is the same function without overflow.
 * dt_raw: (rows, H); out: (rows, H) double. */
void oracle_softplus_dt(const float* dt_raw, const float* dt_bias, int64_t rows, int32_t H, double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t h = 0; h < H; ++h) {
      const double v = (double)dt_raw[r * H + h] + (dt_bias ? (double)dt_bias[h] : 0.0);
      out[r * H + h] = fmax(v, 0.0) + log1p(exp(-fabs(v)));
    }
}

/* Acs for one (b, h): out[c * chunk + j] = sum_{i <= j} dt[cQ + i] * A[h] within chunk c,
 * for every token of the (possibly ragged) last chunk; entries past L are left untouched. */
void oracle_chunk_cumsum(const float* dt, const float* A, int64_t L, int32_t H, int32_t b, int32_t h,
                         int32_t chunk, double* out) {
  const int64_t nc = (L + chunk - 1) / chunk;
  for (int64_t c = 0; c < nc; ++c) {
    double acc = 0.0;
    for (int32_t j = 0; j < chunk && c * chunk + j < L; ++j) {
      acc += (double)dt[((int64_t)b * L + c * chunk + j) * H + h] * (double)A[h];
      out[c * chunk + j] = acc;
    }
  }
}

/* S_c for one (b, h): out[c][p][n] = sum_{j in chunk c} exp(Acs[c,last] - Acs[c,j]) dt_j x[j,p] B[j,n],
 * where `last` is the chunk's last valid token. */
void oracle_chunk_state(const int8_t* qx, const float* sx, const int8_t* qB, const float* sB,
                        const float* dt, const float* A, int64_t L, int32_t H, int32_t P, int32_t N,
                        int32_t G, int32_t b, int32_t h, int32_t chunk, double* out, int32_t scale_flags) {
  const int32_t g = h / (H / G);
  const int bc_per_state = scale_flags & 1, x_per_channel = (scale_flags >> 1) & 1;
  const int64_t nc = (L + chunk - 1) / chunk;
  double* acs = (double*)malloc(sizeof(double) * nc * chunk);
  oracle_chunk_cumsum(dt, A, L, H, b, h, chunk, acs);
  for (int64_t c = 0; c < nc; ++c) {
    double* Sc = out + c * (int64_t)P * N;
    for (int64_t i = 0; i < (int64_t)P * N; ++i) Sc[i] = 0.0;
    int64_t len = L - c * chunk;
    if (len > chunk) len = chunk;
    const double last = acs[c * chunk + len - 1];
    for (int64_t j = 0; j < len; ++j) {
      const int64_t row = (int64_t)b * L + c * chunk + j;
      const double w = exp(last - acs[c * chunk + j]) * (double)dt[row * H + h];
      for (int32_t p = 0; p < P; ++p) {
        const double xw = w * (double)sx[x_per_channel ? (int64_t)h * P + p : h] * (double)qx[(row * H + h) * P + p];
        for (int32_t n = 0; n < N; ++n)
          Sc[(int64_t)p * N + n] += xw * (double)sB[bc_per_state ? g * N + n : g] * (double)qB[(row * G + g) * N + n];
      }
    }
  }
  free(acs);
}
