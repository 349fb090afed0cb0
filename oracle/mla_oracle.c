/*
 * mla_oracle.c -- FP64 CPU oracle for MLA attention over a latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the bench's CPU-baseline
 * leg use it.  It shares no source with the HIP library.
 *
 * What it computes (plain definitions, no blocking, no fusion, no reordering):
 *
 *  - Latent KV row.  Every cached position holds one 576-wide row that serves
 *    as the key; its first 512 entries serve as the value.  Keys and values are
 *    projections into one shared latent space (InferenceX blog on Kimi K2.5,
 *    section "PR #35850 修复了什么"), a row costs 576 FP8 bytes per position and
 *    layer (Kimi K3 engineering report, section "缓存可复用，还要能一致地恢复"),
 *    and query heads attend independently over the same history without
 *    expanding it (same report, section "并行度必须适配真正的形状").
 *    Absorbed-form MLA is therefore multi-query attention with key width 576
 *    and value width 512; the 64 rotary dims are stored already rotated and
 *    are treated like every other key dim.
 *
 *  - Softmax attention per query row (b, j, h):
 *        s_t   = sigma * sum_d q_d k_{t,d}                t in visible set
 *        m     = max_t s_t
 *        l     = sum_t exp(s_t - m)
 *        out_e = sum_t exp(s_t - m) v_{t,e} / l
 *        lse   = m + ln l
 *    An empty visible set gives out = 0 and lse = -inf.
 *
 *  - Merge of partial results by their normalisers (Kimi K3 report, section
 *    "缓存可复用，还要能一致地恢复": position shards swap queries, attend over
 *    their own positions and combine the pieces using each piece's normaliser):
 *        M = max_p lse_p,  lse = M + ln sum_p exp(lse_p - M),
 *        out = sum_p exp(lse_p - lse) out_p;  all lse_p = -inf gives 0 / -inf.
 *
 *  - Latent-row cache write and top-k renormalisation of probability rows: see
 *    the comments above mla_oracle_cache_write and mla_oracle_top_k_renorm.
 *
 * Inputs are the raw bytes both paths consume: BF16 bit patterns for queries
 * and BF16 caches, OCP FP8 E4M3FN codes plus one fp32 per-tensor scale for FP8
 * caches.  Every input value is decoded exactly into a double; the product of
 * an FP8 value (4 significant bits) and the fp32 scale (24 bits) is exact in a
 * double, so the oracle sees the exact real dequantised key.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DK 576 /* key width: 512 latent + 64 rotary */
#define ORACLE_DV 512 /* value width: the latent part of the same row */

/* ---- exact decoders ------------------------------------------------------ */

/* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent 0 is subnormal (m * 2^-9); exponent 15 with mantissa 7 is NaN;
 * there are no infinities, so the largest finite magnitude is 1.75 * 2^8. */
double mla_oracle_fp8_e4m3fn_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* BF16 is the upper half of an IEEE binary32. */
double mla_oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ---- key source: paged or contiguous latent rows ------------------------- */

typedef struct {
  const void* base;      /* [num_slots, 576] codes */
  int fp8;               /* 1: FP8 E4M3FN codes, 0: BF16 bits */
  double scale;          /* per-tensor dequant scale (1 for BF16) */
  const int32_t* table;  /* block table row of this sequence, or NULL */
  int block_size;        /* tokens per block when table != NULL */
  const double* fp8_lut; /* 256 exact FP8 values */
} kv_view;

static const void* kv_row(const kv_view* v, long t) {
  long slot = t;
  if (v->table) slot = (long)v->table[t / v->block_size] * v->block_size + t % v->block_size;
  return (const char*)v->base + (size_t)slot * ORACLE_DK * (v->fp8 ? 1 : 2);
}

static double kv_elem(const kv_view* v, const void* row, int d) {
  if (v->fp8) return v->fp8_lut[((const uint8_t*)row)[d]] * v->scale;
  return mla_oracle_bf16_value(((const uint16_t*)row)[d]);
}

/* Softmax attention of one query row over keys [begin, end) of one sequence.
 * scores: scratch of at least (end - begin) doubles. */
static void attend_row(const uint16_t* q_bits, const kv_view* kv, long begin, long end,
                       double sigma, double* scores, double* out, double* lse) {
  double q[ORACLE_DK];
  for (int d = 0; d < ORACLE_DK; ++d) q[d] = mla_oracle_bf16_value(q_bits[d]);
  for (int e = 0; e < ORACLE_DV; ++e) out[e] = 0.0;
  if (end <= begin) {
    *lse = -INFINITY;
    return;
  }
  /* pass 1: scores and their maximum */
  double m = -INFINITY;
  for (long t = begin; t < end; ++t) {
    const void* row = kv_row(kv, t);
    double dot = 0.0;
    for (int d = 0; d < ORACLE_DK; ++d) dot += q[d] * kv_elem(kv, row, d);
    double s = sigma * dot;
    scores[t - begin] = s;
    if (s > m) m = s;
  }
  /* pass 2: normaliser and weighted sum of the value part of each row */
  double l = 0.0;
  for (long t = begin; t < end; ++t) {
    double w = exp(scores[t - begin] - m);
    l += w;
    const void* row = kv_row(kv, t);
    for (int e = 0; e < ORACLE_DV; ++e) out[e] += w * kv_elem(kv, row, e);
  }
  for (int e = 0; e < ORACLE_DV; ++e) out[e] /= l;
  *lse = m + log(l);
}

static void fill_fp8_lut(double* lut) {
  for (int c = 0; c < 256; ++c) lut[c] = mla_oracle_fp8_e4m3fn_value((uint8_t)c);
}

/*
 * Decode / speculative verify over a paged latent cache.
 *
 * q            [B, P, H, 576] BF16 bits; query j of sequence b is context
 *              position seq_lens[b] - P + j (the last P positions).
 * kv           [num_blocks, block_size, 576] BF16 bits (kv_fp8 = 0) or
 *              FP8 E4M3FN codes (kv_fp8 = 1) with value code * kv_scale.
 * block_table  [B, max_blocks]: logical block i of sequence b lives in
 *              physical block block_table[b * max_blocks + i].
 * seq_lens     [B] context length including the P query positions.
 * kv_begin     [B] or NULL (0): first key of the range this call covers.
 * kv_end       [B] or NULL (seq_lens): end of the covered key range.
 * Query j of sequence b sees keys t with
 *              max(kv_begin, 0) <= t < min(kv_end, seq_lens - P + j + 1).
 * rows         NULL: compute all B*P*H rows; else n_rows flat row indices
 *              ((b * P + j) * H + h) to compute, in that order.
 * out          [n, 512] doubles, lse [n] doubles, n = B*P*H or n_rows.
 * Returns 0, or -1 on a bad argument.
 */
int mla_oracle_decode(const uint16_t* q, const void* kv, int kv_fp8, float kv_scale,
                      const int32_t* block_table, int max_blocks, int block_size,
                      const int32_t* seq_lens, const int32_t* kv_begin, const int32_t* kv_end,
                      int B, int P, int H, float softmax_scale, const int64_t* rows,
                      long n_rows, double* out, double* lse, int threads) {
  if (!q || !kv || !block_table || !seq_lens || !out || !lse) return -1;
  if (B < 0 || P < 1 || H < 1 || block_size < 1 || max_blocks < 1) return -1;
  double lut[256];
  fill_fp8_lut(lut);
  long total = (long)B * P * H;
  long n = rows ? n_rows : total;
  long max_len = 0;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] > max_len) max_len = seq_lens[b];
  const double sigma = (double)softmax_scale;
  int bad = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#endif
#pragma omp parallel reduction(| : bad)
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    if (!scores) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (long i = 0; i < n; ++i) {
      long flat = rows ? rows[i] : i;
      if (!scores || flat < 0 || flat >= total) {
        bad = 1;
        continue;
      }
      int j = (int)((flat / H) % P);
      int b = (int)(flat / ((long)H * P));
      kv_view v = {kv, kv_fp8, kv_fp8 ? (double)kv_scale : 1.0,
                   block_table + (size_t)b * max_blocks, block_size, lut};
      long begin = kv_begin ? kv_begin[b] : 0;
      if (begin < 0) begin = 0;
      long end = (long)seq_lens[b] - P + j + 1;
      if (kv_end && kv_end[b] < end) end = kv_end[b];
      attend_row(q + (size_t)flat * ORACLE_DK, &v, begin, end, sigma, scores,
                 out + (size_t)i * ORACLE_DV, lse + i);
    }
    free(scores);
  }
  return bad ? -1 : 0;
}

/*
 * Causal prefill over packed variable-length sequences.
 *
 * q          [T, H, 576] BF16 bits, kv [T, 576] BF16 bits or FP8 codes.
 * cu_seqlens [B + 1]: sequence b owns tokens [cu_seqlens[b], cu_seqlens[b+1]).
 * Token g of sequence b (cu_seqlens[b] <= g) sees keys cu_seqlens[b] .. g.
 * tokens     NULL: all T tokens; else n_tokens global token indices, each
 *            computed for all H heads, in that order.
 * out        [n, H, 512] doubles, lse [n, H] doubles.
 */
int mla_oracle_prefill(const uint16_t* q, const void* kv, int kv_fp8, float kv_scale,
                       const int32_t* cu_seqlens, int B, int H, float softmax_scale,
                       const int64_t* tokens, long n_tokens, double* out, double* lse,
                       int threads) {
  if (!q || !kv || !cu_seqlens || !out || !lse || B < 0 || H < 1) return -1;
  double lut[256];
  fill_fp8_lut(lut);
  long T = cu_seqlens[B];
  long n = tokens ? n_tokens : T;
  long max_len = 1;
  for (int b = 0; b < B; ++b)
    if (cu_seqlens[b + 1] - cu_seqlens[b] > max_len) max_len = cu_seqlens[b + 1] - cu_seqlens[b];
  const double sigma = (double)softmax_scale;
  int bad = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#endif
#pragma omp parallel reduction(| : bad)
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)max_len);
    if (!scores) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (long r = 0; r < n * H; ++r) {
      long i = r / H;
      int h = (int)(r % H);
      long g = tokens ? tokens[i] : i;
      if (!scores || g < 0 || g >= T) {
        bad = 1;
        continue;
      }
      int b = 0;
      while (b < B && cu_seqlens[b + 1] <= g) ++b;
      kv_view v = {kv, kv_fp8, kv_fp8 ? (double)kv_scale : 1.0, NULL, 1, lut};
      attend_row(q + ((size_t)g * H + h) * ORACLE_DK, &v, cu_seqlens[b], g + 1, sigma, scores,
                 out + ((size_t)i * H + h) * ORACLE_DV, lse + (size_t)i * H + h);
    }
    free(scores);
  }
  return bad ? -1 : 0;
}

/*
 * Merge of S partial results over disjoint key ranges by their normalisers.
 * part_out [S, N, 512], part_lse [S, N]  ->  out [N, 512], lse [N].
 */
int mla_oracle_merge(const double* part_out, const double* part_lse, int S, long N,
                     double* out, double* lse) {
  if (!part_out || !part_lse || !out || !lse || S < 1 || N < 0) return -1;
  for (long n = 0; n < N; ++n) {
    double M = -INFINITY;
    for (int s = 0; s < S; ++s) {
      double x = part_lse[(size_t)s * N + n];
      if (x > M) M = x;
    }
    for (int e = 0; e < ORACLE_DV; ++e) out[n * ORACLE_DV + e] = 0.0;
    if (M == -INFINITY) {
      lse[n] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int s = 0; s < S; ++s) {
      double x = part_lse[(size_t)s * N + n];
      if (x != -INFINITY) sum += exp(x - M);
    }
    double L = M + log(sum);
    lse[n] = L;
    for (int s = 0; s < S; ++s) {
      double x = part_lse[(size_t)s * N + n];
      if (x == -INFINITY) continue;
      double w = exp(x - L);
      const double* o = part_out + ((size_t)s * N + n) * ORACLE_DV;
      for (int e = 0; e < ORACLE_DV; ++e) out[n * ORACLE_DV + e] += w * o[e];
    }
  }
  return 0;
}

/* Number of OpenMP threads a parallel region would use (0 without OpenMP). */
/* ---- latent-row cache write: quantise and scatter --------------------------
 *
 * New positions' 576-wide latent rows (BF16) go into their cache slots: copied
 * for a BF16 cache; for an FP8 cache each value x is divided by the per-tensor
 * scale in fp32 (y = fp32(x / kv_scale), the same real number every reader
 * multiplies back) and encoded as the E4M3FN code nearest to y after clamping to
 * the largest finite magnitude 448, ties going to the code with an even
 * mantissa; a NaN gives code 0x7F.  A row costs 576 FP8 bytes per position (Kimi
 * K3 engineering report, section "缓存可复用，还要能一致地恢复"); FP8 latent caches
 * are what the FP8 KV paths store (InferenceX blog on Kimi K2.5, section
 * "PR #35850 修复了什么"). */

/* Nearest finite E4M3FN code to y, by comparing against every finite code. */
uint8_t mla_oracle_fp8_e4m3fn_encode(float y) {
  if (isnan(y)) return 0x7F;
  const int neg = signbit(y) ? 1 : 0;
  double a = fabs((double)y);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c < 0x7F; ++c) { /* 0x00 .. 0x7E: the non-negative finite codes */
    const double err = fabs(mla_oracle_fp8_e4m3fn_value((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(best | (neg << 7));
}

/* latent [N, 576] BF16 bits; slot [N] (rows with a slot outside [0, num_slots)
 * are skipped); kv [num_slots, 576] BF16 bits or FP8 codes, updated in place. */
int mla_oracle_cache_write(const uint16_t* latent, long N, const int32_t* slot, void* kv,
                           int kv_fp8, float kv_scale, long num_slots) {
  for (long n = 0; n < N; ++n) {
    const long s = slot[n];
    if (s < 0 || s >= num_slots) continue;
    const uint16_t* x = latent + (size_t)n * ORACLE_DK;
    if (kv_fp8) {
      uint8_t* row = (uint8_t*)kv + (size_t)s * ORACLE_DK;
      for (int d = 0; d < ORACLE_DK; ++d) {
        const float xf = (float)mla_oracle_bf16_value(x[d]); /* exact */
        row[d] = mla_oracle_fp8_e4m3fn_encode(xf / kv_scale);
      }
    } else {
      memcpy((uint16_t*)kv + (size_t)s * ORACLE_DK, x, ORACLE_DK * sizeof(uint16_t));
    }
  }
  return 0;
}

int mla_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 0;
#endif
}

/*
 * Top-k renormalisation of probability rows, the acceptance-sampling step that
 * follows speculative verify (tahou.com article, section "ROCm适配迎来突破，软件
 * 壁垒不再高不可攀"; 66bd.net article, section "我们是如何做到的"): of each row,
 * keep the k largest entries, set every other entry to zero and divide the kept
 * ones by their sum, so the row sums to one again.
 *
 * Readings where the pages say no more:
 *  - exactly k entries are kept; entries rank by value, a -0 below a +0, and
 *    among equal values the lower index ranks first;
 *  - k <= 0 or k >= vocab keeps the whole row (renormalisation only);
 *  - a kept sum of zero gives a row of zeros;
 *  - NaN entries have no rank: the call returns -1.
 * The ranking is a plain sort with that order; the sum is taken in double.
 */
typedef struct {
  float v;
  long i;
} oracle_entry;

/* -1 when a ranks before b (a is "larger" in the order above). */
static int oracle_rank_cmp(const void* pa, const void* pb) {
  const oracle_entry* a = (const oracle_entry*)pa;
  const oracle_entry* b = (const oracle_entry*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  const int sa = signbit(a->v) ? 1 : 0, sb = signbit(b->v) ? 1 : 0;
  if (sa != sb) return sa ? 1 : -1; /* equal values differing in sign: both zero */
  return (a->i < b->i) ? -1 : (a->i > b->i);
}

int mla_oracle_top_k_renorm(const float* probs, const int32_t* top_k, long rows, long vocab,
                            double* out) {
  for (long n = 0; n < rows * vocab; ++n)
    if (isnan(probs[n])) return -1;
  int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long r = 0; r < rows; ++r) {
    const float* p = probs + r * vocab;
    double* o = out + r * vocab;
    oracle_entry* e = (oracle_entry*)malloc((size_t)(vocab > 0 ? vocab : 1) * sizeof(oracle_entry));
    if (!e) {
#pragma omp atomic write
      status = -2;
      continue;
    }
    for (long i = 0; i < vocab; ++i) {
      e[i].v = p[i];
      e[i].i = i;
    }
    qsort(e, (size_t)vocab, sizeof(oracle_entry), oracle_rank_cmp);
    const long k = (top_k[r] <= 0 || top_k[r] >= vocab) ? vocab : top_k[r];
    double sum = 0.0;
    for (long j = 0; j < k; ++j) sum += (double)e[j].v;
    for (long i = 0; i < vocab; ++i) o[i] = 0.0;
    if (sum != 0.0)
      for (long j = 0; j < k; ++j) o[e[j].i] = (double)e[j].v / sum;
    free(e);
  }
  return status;
}
