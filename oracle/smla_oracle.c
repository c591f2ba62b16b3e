/*
 * smla_oracle.c -- plain, slow CPU oracle for sparse MLA attention over a
 * paged, quantized latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * Sources (the three pages this work is built from):
 *  - FlashInfer PR #4802 "Refactor Sparse MLA SM120", review of
 *    decode_dsv3_2_kernel.cuh: a DSv3.2 cache row is 656 bytes -- bytes
 *    [0,512) hold 512 e4m3 values, [512,528) four FP32 scales (one per
 *    128-element tile), [528,656) a 64-element BF16 rope part; DSv3.2
 *    stores power-of-two scales.
 *  - Same PR, PR description ("Runtime envelopes", "Dispatch"): page block
 *    64, indices are int32 rows that may be row-strided views, per-token
 *    topk_length truncation, per-head attention sinks, FP32 LSE output.
 *  - Same PR, commit notes: decode splits the candidate list into 64-wide
 *    chunks and merges per-split partial results ("per-split merge term").
 *  - AppMana flash-mla-ampere-dsv4 releases, "decode H6": the split merge is
 *    a log-sum-exp combine over splits; "native int8_ds_mla entry": an INT8
 *    variant of the cache exists.
 *  - vLLM PR #57673 "Native-head Triton sparse MLA", Test Result: d=512
 *    value width, combined top-k lists, attn_sink + topk_length.
 *
 * Where the pages are silent the plainest reading is taken (listed in the
 * repository's design notes): standard softmax attention with K = the
 * 576-element dequantized latent and V = its first 512 elements; natural-log
 * LSE that excludes the sink; the sink is one extra logit per head (in
 * scaled-score units) that carries no value; an empty candidate set gives
 * out = 0 and lse = -inf; scales are 2^ceil(log2(amax/448)) (FP8),
 * amax/448 (FP8 with arbitrary scales, the GLM_NSA rows of FlashInfer #4802's
 * KV layout comment) or amax/127 (INT8), amax = 0 giving scale 1.  GLM53_NOPE
 * rows (the same layout comment) are FP8 rows whose bytes [528, 656) are
 * reserved padding: they are never written or read, and scores use the 512
 * nope dimensions only (q rows hold 512 values); every index outside
 * [0, num_blocks*64) -- -1 padding included -- contributes nothing.
 *
 * DOTS3_SWA rows (FlashInfer PR #4802 description: d_qk = 1088, d_v = 1024,
 * 1160 bytes per token with the scales in a footer): K is 1024 nope values
 * plus 64 rope values and V the 1024 nope values.  The row is read as
 * [0,1024) e4m3 codes, [1024,1152) the 64 BF16 rope values, [1152,1160) one
 * scale byte per 128-element tile.  The byte count leaves one byte per
 * scale, read as an unsigned power-of-two exponent with bias 127 (the
 * E8M0 scale of the OCP microscaling formats: 2^(b-127), 255 = NaN).  The
 * writer takes the same power-of-two scale as the FP8 rows, raised to at
 * least 2^-126 so that the byte is never 0.
 *
 * DSv4 rows (FlashInfer PR #4802 gives only their size, 584 bytes, and that
 * the V3.2-family models share d_v = 512): read as 448 nope values and 64
 * rope values (d_qk = 512, K's first 512 values -- all of them -- are V, the
 * rule every row follows), [0,448) e4m3 codes, [448,576) the rope values in
 * BF16, [576,583) one exponent byte per 64-element tile of the nope part
 * (448 = 7 x 64; 128-element tiles would not divide it), [583] padding that
 * the writer sets to 0 and no reader uses.  Scale bytes as for DOTS3_SWA.
 *
 * Precision: all attention arithmetic is float64.  The quantizer runs in
 * float32, because float32 arithmetic decides its integer codes and the
 * stored scales are float32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define D_NOPE 512 /* nope values of every row but DOTS3_SWA's */
#define D_ROPE 64
#define D_QK 576
#define D_NOPE_MAX 1024
#define D_QK_MAX (D_NOPE_MAX + D_ROPE)
#define D_V_MAX D_NOPE_MAX
#define PAGE_BLOCK 64
#define TILE 128 /* quantization tile width along the nope part */

enum { FMT_BF16 = 0, FMT_FP8 = 1, FMT_INT8 = 2, FMT_FP8_ANY = 3, FMT_FP8_NOPE = 4, FMT_FP8_DOTS3 = 5,
       FMT_FP8_DSV4 = 6 };

#define DSV4_NOPE 448
#define DSV4_TILE 64 /* its quantization tile */

/* nope values of a row; K holds these plus D_ROPE rope values (zero for
 * rows without rope dimensions); V is K's first d_v values */
static int d_nope(int32_t fmt) { return fmt == FMT_FP8_DOTS3 ? D_NOPE_MAX : fmt == FMT_FP8_DSV4 ? DSV4_NOPE : D_NOPE; }
static int d_k(int32_t fmt) { return d_nope(fmt) + D_ROPE; }
static int d_v(int32_t fmt) { return fmt == FMT_FP8_DSV4 ? d_k(fmt) : d_nope(fmt); }
/* elements of a query row that enter a score */
static int q_dims(int32_t fmt) { return fmt == FMT_FP8_NOPE ? D_NOPE : d_k(fmt); }

int32_t oracle_d_k(int32_t fmt) { return d_k(fmt); }
int32_t oracle_d_v(int32_t fmt) { return d_v(fmt); }

/* ---------------------------------------------------------------------- */
/* Scalar helpers                                                          */
/* ---------------------------------------------------------------------- */

static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round a double to the nearest BF16 (ties to even), returned as raw bits. */
uint16_t oracle_double_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int e;
  frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
  int q = e - 8;                /* BF16 keeps 8 significant bits */
  if (q < -133) q = -133;       /* subnormal quantum 2^-133 */
  double r = nearbyint(ldexp(a, -q)); /* ties to even (default rounding) */
  double v = ldexp(r, q);
  if (v >= 3.402823669209385e38) /* 2^128: overflow */
    return sign | 0x7F80;
  float f = (float)v; /* exact: at most 9 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

/* OCP OFP8 E4M3: S EEEE MMM, bias 7, E = 0 subnormal M * 2^-9,
 * S.1111.111 is NaN, no infinities, largest finite 448. */
double oracle_e4m3_decode(uint8_t code) {
  int s = code >> 7, E = (code >> 3) & 15, M = code & 7;
  if (E == 15 && M == 7) return NAN;
  double v = (E == 0) ? ldexp((double)M, -9) : ldexp(1.0 + M / 8.0, E - 7);
  return s ? -v : v;
}

/* Nearest E4M3 value to y, ties to the even mantissa, sign kept (so a
 * negative value that rounds to zero gives 0x80).  Magnitudes of 448 and
 * above saturate to 448. */
uint8_t oracle_e4m3_encode(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0;
  double a = fabs((double)y);
  if (isnan(y)) return sign | 0x7F;
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: quantum 2^-9; code value m in 0..8 (8 is 2^-6) */
    int m = (int)nearbyint(a * 512.0);
    return sign | (uint8_t)m;
  }
  int k;
  frexp(a, &k);
  int E = k - 1;                      /* a in [2^E, 2^(E+1)) */
  int mant = (int)nearbyint((ldexp(a, -E) - 1.0) * 8.0);
  if (mant == 8) { mant = 0; E += 1; }
  int code = ((E + 7) << 3) | mant;
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

/* FP8 tile scale: amax = 0 -> 1; otherwise the smallest power of two s with
 * amax / s <= 448, found from r = amax / 448 (float32) as 2^ceil(log2 r),
 * and at least 2^-126: the stored scale is a normal float32 power of two
 * (tiles with amax below 448 * 2^-126 then use codes below 448). */
float oracle_fp8_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  float r = amax / 448.0f;
  int k;
  float f = frexpf(r, &k); /* r = f * 2^k, f in [0.5, 1) */
  int e = (f == 0.5f) ? k - 1 : k;
  if (e < -126) e = -126;
  return ldexpf(1.0f, e);
}

/* Tile scale of FP8 rows with arbitrary scales: amax = 0 -> 1; otherwise
 * amax / 448 (float32), so the tile's largest magnitude maps to the largest
 * e4m3 value. */
float oracle_fp8_any_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  return amax / 448.0f;
}

/* INT8 tile scale: amax = 0 -> 1; otherwise amax / 127 (float32). */
float oracle_int8_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  return amax / 127.0f;
}

int8_t oracle_int8_encode(float x, float scale) {
  float q = rintf(x / scale); /* IEEE float32 division, ties to even */
  if (q > 127.0f) q = 127.0f;
  if (q < -127.0f) q = -127.0f;
  return (int8_t)q;
}

/* DOTS3_SWA tile scale byte: the FP8 power-of-two scale 2^e, e raised to
 * at least -126, stored as e + 127 (so 1..254). */
uint8_t oracle_e8m0_scale(float amax) {
  int e;
  frexpf(oracle_fp8_scale(amax), &e); /* the scale is 2^(e-1) */
  e -= 1;
  if (e < -126) e = -126;
  return (uint8_t)(e + 127);
}

/* 2^(b-127); 255 is NaN */
double oracle_e8m0_decode(uint8_t b) { return b == 255 ? NAN : ldexp(1.0, (int)b - 127); }

int32_t oracle_row_bytes(int32_t fmt) {
  if (fmt == FMT_BF16) return 2 * D_QK;
  if (fmt == FMT_FP8_DOTS3) return D_NOPE_MAX + 2 * D_ROPE + D_NOPE_MAX / TILE;
  if (fmt == FMT_FP8_DSV4) return DSV4_NOPE + 2 * D_ROPE + DSV4_NOPE / DSV4_TILE + 1;
  return D_NOPE + 4 * (D_NOPE / TILE) + 2 * D_ROPE;
}

/* ---------------------------------------------------------------------- */
/* Cache writer                                                            */
/* ---------------------------------------------------------------------- */

/* Quantize one BF16 latent row (d_k(fmt) raw bf16 values) into a pool row. */
static void quantize_row(const uint16_t* x, int32_t fmt, uint8_t* row) {
  if (fmt == FMT_BF16) {
    memcpy(row, x, 2 * D_QK);
    return;
  }
  if (fmt == FMT_FP8_DOTS3) {
    for (int g = 0; g < D_NOPE_MAX / TILE; ++g) {
      float amax = 0.0f;
      for (int i = g * TILE; i < (g + 1) * TILE; ++i) {
        float v = fabsf(bf16_bits_to_float(x[i]));
        if (v > amax) amax = v;
      }
      uint8_t b = oracle_e8m0_scale(amax);
      float scale = ldexpf(1.0f, (int)b - 127);
      for (int i = g * TILE; i < (g + 1) * TILE; ++i) row[i] = oracle_e4m3_encode(bf16_bits_to_float(x[i]) / scale);
      row[D_NOPE_MAX + 2 * D_ROPE + g] = b;
    }
    memcpy(row + D_NOPE_MAX, x + D_NOPE_MAX, 2 * D_ROPE);
    return;
  }
  if (fmt == FMT_FP8_DSV4) {
    for (int g = 0; g < DSV4_NOPE / DSV4_TILE; ++g) {
      float amax = 0.0f;
      for (int i = g * DSV4_TILE; i < (g + 1) * DSV4_TILE; ++i) {
        float v = fabsf(bf16_bits_to_float(x[i]));
        if (v > amax) amax = v;
      }
      uint8_t b = oracle_e8m0_scale(amax);
      float scale = ldexpf(1.0f, (int)b - 127);
      for (int i = g * DSV4_TILE; i < (g + 1) * DSV4_TILE; ++i)
        row[i] = oracle_e4m3_encode(bf16_bits_to_float(x[i]) / scale);
      row[DSV4_NOPE + 2 * D_ROPE + g] = b;
    }
    row[DSV4_NOPE + 2 * D_ROPE + DSV4_NOPE / DSV4_TILE] = 0; /* padding */
    memcpy(row + DSV4_NOPE, x + DSV4_NOPE, 2 * D_ROPE);
    return;
  }
  for (int g = 0; g < D_NOPE / TILE; ++g) {
    float amax = 0.0f;
    for (int i = g * TILE; i < (g + 1) * TILE; ++i) {
      float v = fabsf(bf16_bits_to_float(x[i]));
      if (v > amax) amax = v;
    }
    float scale = (fmt == FMT_FP8 || fmt == FMT_FP8_NOPE) ? oracle_fp8_scale(amax)
                  : (fmt == FMT_FP8_ANY) ? oracle_fp8_any_scale(amax)
                                         : oracle_int8_scale(amax);
    for (int i = g * TILE; i < (g + 1) * TILE; ++i) {
      float xv = bf16_bits_to_float(x[i]);
      if (fmt != FMT_INT8)
        row[i] = oracle_e4m3_encode(xv / scale);
      else
        row[i] = (uint8_t)oracle_int8_encode(xv, scale);
    }
    memcpy(row + D_NOPE + 4 * g, &scale, 4);
  }
  if (fmt != FMT_FP8_NOPE) memcpy(row + D_NOPE + 4 * (D_NOPE / TILE), x + D_NOPE, 2 * D_ROPE);
}

/* Write n latent rows (row i at kv + i*kv_stride elements) into the pool at
 * the given flat slot ids (block = slot / 64, offset = slot % 64).  Slots
 * outside [0, num_blocks*64) -- -1 included -- are skipped. */
int oracle_quantize_kv(const uint16_t* kv, int64_t n, int64_t kv_stride, const int32_t* slots,
                       uint8_t* pool, int64_t num_blocks, int64_t block_stride_bytes,
                       int32_t fmt) {
  int64_t rb = oracle_row_bytes(fmt);
  for (int64_t i = 0; i < n; ++i) {
    int64_t s = slots[i];
    if (s < 0 || s >= num_blocks * PAGE_BLOCK) continue;
    uint8_t* row = pool + (s / PAGE_BLOCK) * block_stride_bytes + (s % PAGE_BLOCK) * rb;
    quantize_row(kv + i * kv_stride, fmt, row);
  }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Cache reader                                                            */
/* ---------------------------------------------------------------------- */

/* Dequantize pool row `slot` into K[d_k(fmt)] (V is K[0:d_v(fmt)]). */
static void dequant_row(const uint8_t* pool, int64_t block_stride_bytes, int32_t fmt,
                        int64_t slot, double* K) {
  int64_t rb = oracle_row_bytes(fmt);
  const uint8_t* row = pool + (slot / PAGE_BLOCK) * block_stride_bytes + (slot % PAGE_BLOCK) * rb;
  if (fmt == FMT_FP8_DOTS3) {
    for (int i = 0; i < D_NOPE_MAX; ++i)
      K[i] = oracle_e4m3_decode(row[i]) * oracle_e8m0_decode(row[D_NOPE_MAX + 2 * D_ROPE + i / TILE]);
    for (int r = 0; r < D_ROPE; ++r) {
      uint16_t b;
      memcpy(&b, row + D_NOPE_MAX + 2 * r, 2);
      K[D_NOPE_MAX + r] = bf16_bits_to_float(b);
    }
    return;
  }
  if (fmt == FMT_FP8_DSV4) {
    for (int i = 0; i < DSV4_NOPE; ++i)
      K[i] = oracle_e4m3_decode(row[i]) * oracle_e8m0_decode(row[DSV4_NOPE + 2 * D_ROPE + i / DSV4_TILE]);
    for (int r = 0; r < D_ROPE; ++r) {
      uint16_t b;
      memcpy(&b, row + DSV4_NOPE + 2 * r, 2);
      K[DSV4_NOPE + r] = bf16_bits_to_float(b);
    }
    return;
  }
  if (fmt == FMT_BF16) {
    for (int i = 0; i < D_QK; ++i) {
      uint16_t b;
      memcpy(&b, row + 2 * i, 2);
      K[i] = bf16_bits_to_float(b);
    }
    return;
  }
  float scale[D_NOPE / TILE];
  memcpy(scale, row + D_NOPE, sizeof scale);
  for (int i = 0; i < D_NOPE; ++i) {
    double c = (fmt != FMT_INT8) ? oracle_e4m3_decode(row[i]) : (double)(int8_t)row[i];
    K[i] = c * (double)scale[i / TILE];
  }
  for (int r = 0; r < D_ROPE; ++r) {
    if (fmt == FMT_FP8_NOPE) { /* padding: not part of the row's data */
      K[D_NOPE + r] = 0.0;
      continue;
    }
    uint16_t b;
    memcpy(&b, row + D_NOPE + sizeof scale + 2 * r, 2);
    K[D_NOPE + r] = bf16_bits_to_float(b);
  }
}

void oracle_dequant_rows(const uint8_t* pool, int64_t block_stride_bytes, int32_t fmt,
                         const int32_t* slots, int64_t n, double* out /* [n][d_k(fmt)] */) {
  for (int64_t i = 0; i < n; ++i) dequant_row(pool, block_stride_bytes, fmt, slots[i], out + i * d_k(fmt));
}

/* ---------------------------------------------------------------------- */
/* Attention                                                               */
/* ---------------------------------------------------------------------- */

typedef struct {
  const uint16_t* q;
  int64_t T;
  int32_t H;
  int64_t q_stride_t, q_stride_h; /* elements */
  const uint8_t* pool;
  int64_t num_blocks, block_stride_bytes;
  int32_t fmt;
  const int32_t* indices;
  int32_t topk;
  int64_t idx_stride_t; /* elements */
  const int32_t* topk_length; /* [T] or NULL */
  double sm_scale;
} problem;

/* The candidate list of token t restricted to positions [j0, j1): entries
 * j < L_t whose index is a slot of the pool, kept in j order. */
static int64_t candidates(const problem* P, int64_t t, int64_t j0, int64_t j1, int32_t* out) {
  int64_t L = P->topk;
  if (P->topk_length) {
    L = P->topk_length[t];
    if (L < 0) L = 0;
    if (L > P->topk) L = P->topk;
  }
  if (j1 > L) j1 = L;
  int64_t n = 0, nslots = P->num_blocks * PAGE_BLOCK;
  for (int64_t j = j0; j < j1; ++j) {
    int64_t s = P->indices[t * P->idx_stride_t + j];
    if (s >= 0 && s < nslots) out[n++] = (int32_t)s;
  }
  return n;
}

/* Softmax attention of one query row over n dequantized rows.
 * Writes the unnormalized-sink result:  m (max score), l = sum exp(s - m),
 * acc[d] = sum exp(s - m) * V[d].  Returns nothing for n == 0 (m = -inf). */
static void attend(const problem* P, int64_t t, int32_t h, const double* rows, int64_t n,
                   double* scores, double* m_out, double* l_out, double* acc) {
  const uint16_t* qr = P->q + t * P->q_stride_t + (int64_t)h * P->q_stride_h;
  const int dk = d_k(P->fmt), dv = d_v(P->fmt);
  double q[D_QK_MAX];
  for (int i = 0; i < dk; ++i) q[i] = i < q_dims(P->fmt) ? bf16_bits_to_float(qr[i]) : 0.0;
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    double dot = 0.0;
    for (int i = 0; i < dk; ++i) dot += q[i] * rows[j * dk + i];
    scores[j] = P->sm_scale * dot;
    if (scores[j] > m) m = scores[j];
  }
  double l = 0.0;
  for (int d = 0; d < dv; ++d) acc[d] = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    double p = exp(scores[j] - m);
    l += p;
    for (int d = 0; d < dv; ++d) acc[d] += p * rows[j * dk + d];
  }
  *m_out = m;
  *l_out = l;
}

static int nthreads_or_default(int nthreads) {
#ifdef _OPENMP
  return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

/* Prefill form.  For each selected token t (all when token_list is NULL)
 * and head h:
 *   lse = m + ln l over the candidate set (natural log, sink excluded),
 *   out = sum_j exp(s_j - m*) V_j / Z with m* = max(m, sink_h) and
 *   Z = sum_j exp(s_j - m*) + exp(sink_h - m*) (sink term only when a sink
 *   is given); an empty set gives out = 0, lse = -inf.
 * out is rounded to BF16 (ties to even); out_f64 / lse_f64 (optional,
 * dense [T][H][d_v] / [T][H]) receive the unrounded values. */
int oracle_prefill(const uint16_t* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                   const uint8_t* pool, int64_t num_blocks, int64_t block_stride_bytes, int32_t fmt,
                   const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                   const int32_t* topk_length, const float* sink, float sm_scale,
                   uint16_t* out, int64_t out_stride_t, int64_t out_stride_h,
                   float* lse, int64_t lse_stride_t,
                   double* out_f64, double* lse_f64,
                   const int64_t* token_list, int64_t n_tokens, int nthreads) {
  problem P = {q, T, H, q_stride_t, q_stride_h, pool, num_blocks, block_stride_bytes, fmt,
               indices, topk, idx_stride_t, topk_length, (double)sm_scale};
  const int dk = d_k(fmt), dv = d_v(fmt);
  int64_t count = token_list ? n_tokens : T;
  int nt = nthreads_or_default(nthreads);
  int failed = 0;
#pragma omp parallel num_threads(nt)
  {
    int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (topk > 0 ? topk : 1));
    double* rows = (double*)malloc(sizeof(double) * dk * (topk > 0 ? topk : 1));
    double* scores = (double*)malloc(sizeof(double) * (topk > 0 ? topk : 1));
    if (!cand || !rows || !scores) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t it = 0; it < count; ++it) {
        int64_t t = token_list ? token_list[it] : it;
        int64_t n = candidates(&P, t, 0, topk, cand);
        for (int64_t j = 0; j < n; ++j) dequant_row(pool, block_stride_bytes, fmt, cand[j], rows + j * dk);
        for (int32_t h = 0; h < H; ++h) {
          double acc[D_V_MAX], m = -INFINITY, l = 0.0, res_lse;
          double o[D_V_MAX];
          if (n == 0) {
            for (int d = 0; d < dv; ++d) o[d] = 0.0;
            res_lse = -INFINITY;
          } else {
            attend(&P, t, h, rows, n, scores, &m, &l, acc);
            res_lse = m + log(l);
            double ms = m, z;
            if (sink && (double)sink[h] > ms) ms = (double)sink[h];
            double a = exp(m - ms); /* rescales exp(s - m) to exp(s - m*) */
            z = l * a + (sink ? exp((double)sink[h] - ms) : 0.0);
            for (int d = 0; d < dv; ++d) o[d] = acc[d] * a / z;
          }
          uint16_t* orow = out + t * out_stride_t + (int64_t)h * out_stride_h;
          for (int d = 0; d < dv; ++d) orow[d] = oracle_double_to_bf16(o[d]);
          lse[t * lse_stride_t + h] = (float)res_lse;
          if (out_f64) memcpy(out_f64 + (t * H + h) * dv, o, sizeof(double) * dv);
          if (lse_f64) lse_f64[t * H + h] = res_lse;
        }
      }
    }
    free(cand);
    free(rows);
    free(scores);
  }
  return failed ? -1 : 0;
}

/* Width of one decode split: whole 64-wide chunks, ceil(ceil(topk/S)/64). */
int32_t oracle_split_width(int32_t topk, int32_t num_splits) {
  int32_t per = (topk + num_splits - 1) / num_splits;
  return ((per + 63) / 64) * 64;
}

/* Decode split form.  Split s covers list positions [s*w, min((s+1)*w, topk))
 * (w from oracle_split_width); for each token t, split s, head h it yields
 * part_lse = m + ln l over the split's candidates (-inf if none) and
 * part_out = sum exp(s_j - m) V_j / l (0 if none).  No sink here. */
int oracle_decode_split(const uint16_t* q, int64_t T, int32_t H, int64_t q_stride_t,
                        int64_t q_stride_h, const uint8_t* pool, int64_t num_blocks,
                        int64_t block_stride_bytes, int32_t fmt, const int32_t* indices,
                        int32_t topk, int64_t idx_stride_t, const int32_t* topk_length,
                        float sm_scale, int32_t num_splits,
                        double* part_out /* [T][S][H][d_v] */, double* part_lse /* [T][S][H] */,
                        const int64_t* token_list, int64_t n_tokens, int nthreads) {
  problem P = {q, T, H, q_stride_t, q_stride_h, pool, num_blocks, block_stride_bytes, fmt,
               indices, topk, idx_stride_t, topk_length, (double)sm_scale};
  int32_t w = oracle_split_width(topk, num_splits);
  const int dk = d_k(fmt), dv = d_v(fmt);
  int64_t count = token_list ? n_tokens : T;
  int nt = nthreads_or_default(nthreads);
  int failed = 0;
#pragma omp parallel num_threads(nt)
  {
    int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (w > 0 ? w : 1));
    double* rows = (double*)malloc(sizeof(double) * dk * (w > 0 ? w : 1));
    double* scores = (double*)malloc(sizeof(double) * (w > 0 ? w : 1));
    if (!cand || !rows || !scores) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1) collapse(2)
      for (int64_t it = 0; it < count; ++it) {
        for (int32_t s = 0; s < num_splits; ++s) {
          int64_t t = token_list ? token_list[it] : it;
          int64_t j0 = (int64_t)s * w, j1 = j0 + w;
          if (j1 > topk) j1 = topk;
          int64_t n = j0 < j1 ? candidates(&P, t, j0, j1, cand) : 0;
          for (int64_t j = 0; j < n; ++j) dequant_row(pool, block_stride_bytes, fmt, cand[j], rows + j * dk);
          for (int32_t h = 0; h < H; ++h) {
            double* po = part_out + (((t * num_splits) + s) * H + h) * dv;
            double* pl = part_lse + ((t * num_splits) + s) * H + h;
            if (n == 0) {
              for (int d = 0; d < dv; ++d) po[d] = 0.0;
              *pl = -INFINITY;
              continue;
            }
            double acc[D_V_MAX], m, l;
            attend(&P, t, h, rows, n, scores, &m, &l, acc);
            for (int d = 0; d < dv; ++d) po[d] = acc[d] / l;
            *pl = m + log(l);
          }
        }
      }
    }
    free(cand);
    free(rows);
    free(scores);
  }
  return failed ? -1 : 0;
}

/* Log-sum-exp merge of decode splits.  M = max_s LSE_s; if M = -inf the
 * result is out = 0, lse = -inf.  Otherwise w_s = exp(LSE_s - M),
 * W = sum w_s, lse = M + ln W, o = sum (w_s / W) O_s; with a sink the output
 * is scaled by 1 / (1 + exp(sink_h - lse)); out = bf16(o).  part_out rows
 * hold dv values (512, or 1024 for DOTS3_SWA). */
int oracle_combine(const double* part_out, const double* part_lse, int64_t T, int32_t num_splits,
                   int32_t H, int32_t dv, const float* sink, uint16_t* out, int64_t out_stride_t,
                   int64_t out_stride_h, float* lse, int64_t lse_stride_t, double* out_f64,
                   double* lse_f64, const int64_t* token_list, int64_t n_tokens) {
  int64_t count = token_list ? n_tokens : T;
  if (dv < 1 || dv > D_V_MAX) return -1;
  for (int64_t it = 0; it < count; ++it) {
    int64_t t = token_list ? token_list[it] : it;
    for (int32_t h = 0; h < H; ++h) {
      double M = -INFINITY;
      for (int32_t s = 0; s < num_splits; ++s) {
        double v = part_lse[((t * num_splits) + s) * H + h];
        if (v > M) M = v;
      }
      double o[D_V_MAX], res;
      for (int d = 0; d < dv; ++d) o[d] = 0.0;
      if (M == -INFINITY) {
        res = -INFINITY;
      } else {
        double W = 0.0;
        for (int32_t s = 0; s < num_splits; ++s) W += exp(part_lse[((t * num_splits) + s) * H + h] - M);
        res = M + log(W);
        for (int32_t s = 0; s < num_splits; ++s) {
          double ws = exp(part_lse[((t * num_splits) + s) * H + h] - M) / W;
          if (ws == 0.0) continue;
          const double* po = part_out + (((t * num_splits) + s) * H + h) * dv;
          for (int d = 0; d < dv; ++d) o[d] += ws * po[d];
        }
        if (sink) {
          double f = 1.0 / (1.0 + exp((double)sink[h] - res));
          for (int d = 0; d < dv; ++d) o[d] *= f;
        }
      }
      uint16_t* orow = out + t * out_stride_t + (int64_t)h * out_stride_h;
      for (int d = 0; d < dv; ++d) orow[d] = oracle_double_to_bf16(o[d]);
      lse[t * lse_stride_t + h] = (float)res;
      if (out_f64) memcpy(out_f64 + (t * H + h) * dv, o, sizeof(double) * dv);
      if (lse_f64) lse_f64[t * H + h] = res;
    }
  }
  return 0;
}

/* Softmax probabilities of one (token, head): p[j] for every list position
 * j < topk (0 for entries that are masked), and the sink's share. */
int oracle_probs(const uint16_t* q, int64_t T, int32_t H, int64_t q_stride_t, int64_t q_stride_h,
                 const uint8_t* pool, int64_t num_blocks, int64_t block_stride_bytes, int32_t fmt,
                 const int32_t* indices, int32_t topk, int64_t idx_stride_t,
                 const int32_t* topk_length, const float* sink, float sm_scale, int64_t t,
                 int32_t h, double* p /* [topk] */, double* p_sink) {
  problem P = {q, T, H, q_stride_t, q_stride_h, pool, num_blocks, block_stride_bytes, fmt,
               indices, topk, idx_stride_t, topk_length, (double)sm_scale};
  const uint16_t* qr = q + t * q_stride_t + (int64_t)h * q_stride_h;
  int64_t L = topk;
  if (topk_length) {
    L = topk_length[t];
    if (L < 0) L = 0;
    if (L > topk) L = topk;
  }
  int64_t nslots = num_blocks * PAGE_BLOCK;
  double m = sink ? (double)sink[h] : -INFINITY;
  double K[D_QK_MAX];
  double* s = (double*)malloc(sizeof(double) * (topk > 0 ? topk : 1));
  if (!s) return -1;
  for (int64_t j = 0; j < topk; ++j) {
    int64_t idx = indices[t * idx_stride_t + j];
    if (j >= L || idx < 0 || idx >= nslots) {
      s[j] = -INFINITY;
      continue;
    }
    dequant_row(pool, block_stride_bytes, fmt, idx, K);
    double dot = 0.0;
    for (int i = 0; i < q_dims(fmt); ++i) dot += (double)bf16_bits_to_float(qr[i]) * K[i];
    s[j] = P.sm_scale * dot;
    if (s[j] > m) m = s[j];
  }
  double z = 0.0;
  for (int64_t j = 0; j < topk; ++j) z += (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
  if (sink) z += exp((double)sink[h] - m);
  for (int64_t j = 0; j < topk; ++j) p[j] = (s[j] == -INFINITY || z == 0.0) ? 0.0 : exp(s[j] - m) / z;
  *p_sink = (sink && z > 0.0) ? exp((double)sink[h] - m) / z : 0.0;
  free(s);
  return 0;
}
