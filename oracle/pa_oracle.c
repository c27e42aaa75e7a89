/*
 * CPU oracle for one paged-attention step.  TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct C (C11 + OpenMP) that computes what the
 * paged-attention step computes, straight from its definition, in double
 * precision.  Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no source, header,
 * table or build rule with the HIP library, and the HIP library never calls it.
 *
 * Pages followed (cited by title and section):
 *   [P1] "vLLM 推理流程分析" (blog.chen3feng.top, vLLM V1 inference-flow analysis)
 *   [P5] "vLLM 源码完全拆解（十六）：把十五篇机制拼成一张可执行的源码阅读地图"
 *        (pinghaoyang.com.cn, vLLM V1 source-reading map)
 *
 * The pool is stored in the pages' layout: key_cache and value_cache are each
 * [num_blocks][block_size][num_kv_heads][head_dim]  ([P1] §6.2, the comments
 * on key_cache / value_cache).  Element types: float (fp32), uint16_t holding
 * bfloat16 bits, uint8_t holding OCP FP8 E4M3FN codes.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *  - slot = block_table[req][p / S] * S + p % S with integer division  ([P1]
 *    §5.1.2 compute_slot_mapping; [P5] third walk-through path, whose display
 *    formula is lost in extraction).
 *  - query_start_loc[0] = 0, query_start_loc[i+1] = query_start_loc[i] + c_i
 *    ([P5] fourth walk-through path, display formula lost; [P1] §5.1.2).
 *  - causal alignment: new token t of a request with seq_len L and c new
 *    tokens sits at position L - c + t ([P1] §5.1.2 positions =
 *    num_computed + offset) and sees keys 0 .. L - c + t  ([P1] §10.1).
 *  - GQA: query head h reads kv head h / (Hq / Hkv).
 *  - fp8: y = x / scale in float32 (IEEE division), encoded to the nearest
 *    finite E4M3FN value, ties to the even code, |y| > 448 saturating to
 *    +-448, NaN -> 0x7F.  Decoding is exact; the dequantised value is
 *    code_value * scale evaluated exactly in double.
 *  - slot < 0 means "do not write this token".
 *
 * Parity status: every function here is pinned by tests under tests/
 * (worked values printed on the pages, closed forms, invariants, a library
 * special case and brute force on tiny inputs); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8 2

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_EVALID 4

typedef struct {
  void *k, *v;
  int32_t num_blocks, block_size, num_kv_heads, head_dim, dtype;
  float k_scale, v_scale;
} oracle_pool;

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------------- */
/* Element codecs                                                          */
/* ---------------------------------------------------------------------- */

static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16; /* bfloat16 is the high half of a binary32 */
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Value of an OCP E4M3FN code: sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN; there
 * is no infinity. */
double oracle_e4m3_decode(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Encode: the finite E4M3FN value nearest to y, ties to the code whose
 * lowest bit is 0, magnitudes above the largest finite value (448)
 * saturate, NaN gives 0x7F.  The non-negative finite magnitudes are the codes
 * 0x00..0x7E in increasing order, so "nearest" is a binary search in that
 * sorted list followed by a comparison of the two neighbours. */
uint8_t oracle_e4m3_encode(float y) {
  if (isnan(y)) return 0x7F;
  int neg = signbit(y) ? 1 : 0;
  double a = fabs((double)y);
  int best;
  if (a >= 448.0) {
    best = 0x7E;
  } else {
    int lo = 0, hi = 0x7E; /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
      int mid = (lo + hi) / 2;
      if (oracle_e4m3_decode((uint8_t)mid) <= a)
        lo = mid;
      else
        hi = mid;
    }
    double dlo = a - oracle_e4m3_decode((uint8_t)lo);
    double dhi = oracle_e4m3_decode((uint8_t)hi) - a;
    if (dlo < dhi)
      best = lo;
    else if (dhi < dlo)
      best = hi;
    else
      best = (lo % 2 == 0) ? lo : hi;
  }
  return (uint8_t)((neg << 7) | best);
}

/* Decoded pool element as a double ([P1] §6.3: the cache stores either the
 * input's own type or fp8 with a per-tensor scale). */
static double pool_elem(const oracle_pool *p, const void *base, size_t idx, float scale) {
  switch (p->dtype) {
    case ORC_F32: return (double)((const float *)base)[idx];
    case ORC_BF16: return bf16_value(((const uint16_t *)base)[idx]);
    default: return oracle_e4m3_decode(((const uint8_t *)base)[idx]) * (double)scale;
  }
}

static double io_elem(const void *base, int dtype, size_t idx) {
  if (dtype == ORC_F32) return (double)((const float *)base)[idx];
  return bf16_value(((const uint16_t *)base)[idx]);
}

static size_t pool_index(const oracle_pool *p, int64_t block, int64_t off, int64_t head, int64_t dim) {
  return (((size_t)block * p->block_size + off) * p->num_kv_heads + head) * p->head_dim + dim;
}

/* ---------------------------------------------------------------------- */
/* a0: step metadata  ([P1] §5.1.2; [P5] fourth walk-through path)         */
/* ---------------------------------------------------------------------- */

int oracle_query_start_loc(int32_t n, const int32_t *num_scheduled, int32_t *qsl) {
  if (n < 0) return ORC_EINVAL;
  qsl[0] = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (num_scheduled[i] < 0) return ORC_EINVAL;
    qsl[i + 1] = qsl[i] + num_scheduled[i];
  }
  return ORC_OK;
}

/* seq_len = num_computed_tokens + num_scheduled_tokens  ([P1] §5.1.2) */
int oracle_seq_lens(int32_t n, const int32_t *num_computed, const int32_t *num_scheduled,
                    int32_t *seq_lens) {
  for (int32_t i = 0; i < n; ++i) {
    if (num_computed[i] < 0 || num_scheduled[i] < 0) return ORC_EINVAL;
    seq_lens[i] = num_computed[i] + num_scheduled[i];
  }
  return ORC_OK;
}

/* The shape checks the source-reading map lists for this layer ([P5] fourth
 * walk-through path, debugging order): query_start_loc starts at 0, is
 * non-decreasing and ends at the token count; every request's tokens fit in
 * its length; the block table covers every length; block ids are in range. */
int oracle_validate(int32_t n, int32_t num_tokens, const int32_t *qsl, const int32_t *seq_lens,
                    const int32_t *bt, int32_t bt_stride, int32_t block_size, int32_t num_blocks) {
  if (qsl[0] != 0) return ORC_EVALID;
  for (int32_t i = 0; i < n; ++i) {
    int32_t c = qsl[i + 1] - qsl[i];
    if (c < 0) return ORC_EVALID;
    if (seq_lens[i] < c) return ORC_EVALID;
    int32_t nb = (seq_lens[i] + block_size - 1) / block_size;
    if (nb > bt_stride) return ORC_EVALID;
    for (int32_t b = 0; b < nb; ++b) {
      int32_t blk = bt[(size_t)i * bt_stride + b];
      if (blk < 0 || blk >= num_blocks) return ORC_EVALID;
    }
  }
  if (qsl[n] != num_tokens) return ORC_EVALID;
  return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* a1: slot derivation  ([P1] §5.1.2 compute_slot_mapping, §10.1;          */
/*     [P5] third walk-through path)                                       */
/* ---------------------------------------------------------------------- */

int oracle_slot_mapping(int32_t n, const int32_t *qsl, const int32_t *seq_lens, const int32_t *bt,
                        int32_t bt_stride, int32_t block_size, int64_t *slots) {
  if (block_size <= 0) return ORC_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    int32_t c = qsl[i + 1] - qsl[i];
    for (int32_t t = 0; t < c; ++t) {
      int64_t pos = (int64_t)seq_lens[i] - c + t; /* num_computed + offset */
      int64_t b = pos / block_size;               /* logical block */
      int64_t o = pos % block_size;               /* offset in block */
      int64_t phys = bt[(size_t)i * bt_stride + b];
      slots[qsl[i] + t] = phys * block_size + o;
    }
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* a2: KV write  ([P1] §6.3 reshape_and_cache_flash)                       */
/* ---------------------------------------------------------------------- */

static int store_elem(const oracle_pool *p, void *dst, size_t di, const void *src, int in_dtype,
                      size_t si, float scale) {
  if (p->dtype == ORC_F32) {
    if (in_dtype != ORC_F32) return ORC_EINVAL;
    ((float *)dst)[di] = ((const float *)src)[si];
  } else if (p->dtype == ORC_BF16) {
    if (in_dtype != ORC_BF16) return ORC_EINVAL;
    ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
  } else {
    float x = (float)io_elem(src, in_dtype, si); /* exact: bf16/fp32 -> fp32 */
    float y = x / scale;                         /* IEEE fp32 division */
    ((uint8_t *)dst)[di] = oracle_e4m3_encode(y);
  }
  return ORC_OK;
}

int oracle_write_kv(const oracle_pool *p, const void *key, const void *value, int32_t in_dtype,
                    const int64_t *slots, int32_t num_tokens) {
  const int64_t S = p->block_size, H = p->num_kv_heads, D = p->head_dim;
  const int64_t cap = (int64_t)p->num_blocks * S;
  for (int32_t n = 0; n < num_tokens; ++n) {
    int64_t slot = slots[n];
    if (slot < 0) continue;  /* padding token: nothing written */
    if (slot >= cap) return ORC_EVALID;
    int64_t blk = slot / S, off = slot % S;
    for (int64_t h = 0; h < H; ++h)
      for (int64_t e = 0; e < D; ++e) {
        size_t si = ((size_t)n * H + h) * D + e;
        size_t di = pool_index(p, blk, off, h, e);
        if (store_elem(p, p->k, di, key, in_dtype, si, p->k_scale)) return ORC_EINVAL;
        if (store_elem(p, p->v, di, value, in_dtype, si, p->v_scale)) return ORC_EINVAL;
      }
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* a4-a7: attention  ([P5] third walk-through path: paging changes only   */
/* where K/V are fetched, not the attention definition; [P1] §6.2         */
/* flash_attn_varlen_func(..., causal=True), §10.1 causal mask)            */
/* ---------------------------------------------------------------------- */

typedef struct {
  int32_t req, t, c, L;
} tok_info;

static int locate_token(int32_t n, const int32_t *qsl, const int32_t *seq_lens, int32_t tok,
                        tok_info *ti) {
  for (int32_t i = 0; i < n; ++i)
    if (tok >= qsl[i] && tok < qsl[i + 1]) {
      ti->req = i;
      ti->t = tok - qsl[i];
      ti->c = qsl[i + 1] - qsl[i];
      ti->L = seq_lens[i];
      return 1;
    }
  return 0;
}

/* Keys visible to new token t: 0 .. L - c + t when causal, 0 .. L - 1 when not. */
static int32_t visible_keys(const tok_info *ti, int causal) {
  return causal ? (ti->L - ti->c + ti->t + 1) : ti->L;
}

/* Gather key/value j of a request through its block table. */
static size_t kv_index(const oracle_pool *p, const int32_t *bt_row, int64_t j, int64_t kvh,
                       int64_t e) {
  int64_t b = j / p->block_size, o = j % p->block_size;
  return pool_index(p, bt_row[b], o, kvh, e);
}

/* Attention for one (token, q head) over keys [k0, k1): unnormalised output
 * acc[e] = sum_j exp(s_j - m) v_j[e] with m = max_j s_j over the range, and
 * l = sum_j exp(s_j - m).  With k0 = 0, k1 = all visible keys, O = acc / l is
 * the softmax-weighted average ([P5] third walk-through path, m = max_j s_j
 * stabilises the softmax). */
static void attend_range(const oracle_pool *p, const int32_t *bt_row, const void *q, int32_t q_dtype,
                         size_t q_off, int64_t kvh, double scale, int64_t k0, int64_t k1,
                         double *scores, double *m_out, double *l_out, double *acc) {
  const int64_t D = p->head_dim;
  double m = -INFINITY;
  for (int64_t j = k0; j < k1; ++j) {
    double s = 0.0;
    for (int64_t e = 0; e < D; ++e)
      s += io_elem(q, q_dtype, q_off + e) * pool_elem(p, p->k, kv_index(p, bt_row, j, kvh, e), p->k_scale);
    s *= scale;
    scores[j - k0] = s;
    if (s > m) m = s;
  }
  double l = 0.0;
  for (int64_t e = 0; e < D; ++e) acc[e] = 0.0;
  for (int64_t j = k0; j < k1; ++j) {
    double w = exp(scores[j - k0] - m);
    l += w;
    for (int64_t e = 0; e < D; ++e)
      acc[e] += w * pool_elem(p, p->v, kv_index(p, bt_row, j, kvh, e), p->v_scale);
  }
  *m_out = m;
  *l_out = l;
}

/*
 * out: [n_out][Hq][D] doubles, where the rows are the tokens listed in
 * token_subset (or all num_tokens tokens when token_subset is NULL).
 * Requests with zero visible keys produce zeros (cannot happen for a valid
 * step with causal masking: a new token always sees itself).
 */
int oracle_attention(const oracle_pool *p, int32_t n, const int32_t *qsl, const int32_t *seq_lens,
                     const int32_t *bt, int32_t bt_stride, const void *q, int32_t q_dtype,
                     int32_t num_q_heads, float softmax_scale, int32_t causal, double *out,
                     const int32_t *token_subset, int32_t n_subset) {
  const int64_t H = p->num_kv_heads, D = p->head_dim, Hq = num_q_heads;
  if (H <= 0 || Hq % H) return ORC_EINVAL;
  const int64_t g = Hq / H;
  const int32_t n_out = token_subset ? n_subset : qsl[n];
  int32_t max_L = 1;
  for (int32_t i = 0; i < n; ++i)
    if (seq_lens[i] > max_L) max_L = seq_lens[i];
  int err = ORC_OK;
#pragma omp parallel
  {
    double *scores = (double *)malloc(sizeof(double) * (size_t)max_L);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int32_t r = 0; r < n_out; ++r)
      for (int64_t h = 0; h < Hq; ++h) {
        int32_t tok = token_subset ? token_subset[r] : r;
        tok_info ti;
        double *o = out + ((size_t)r * Hq + h) * D;
        if (!locate_token(n, qsl, seq_lens, tok, &ti)) {
#pragma omp atomic write
          err = ORC_EINVAL;
          continue;
        }
        int64_t kvh = h / g;
        int64_t nvis = visible_keys(&ti, causal);
        if (nvis <= 0) {
          for (int64_t e = 0; e < D; ++e) o[e] = 0.0;
          continue;
        }
        double m, l;
        attend_range(p, bt + (size_t)ti.req * bt_stride, q, q_dtype, ((size_t)tok * Hq + h) * D, kvh,
                     (double)softmax_scale, 0, nvis, scores, &m, &l, acc);
        for (int64_t e = 0; e < D; ++e) o[e] = acc[e] / l;
      }
    free(scores);
    free(acc);
  }
  return err;
}

/* Probabilities exp(s_j - m) / l of one (token, q head) row, j = 0 .. nvis-1.
 * Returns nvis (or -1 on error).  probs must hold max seq_len entries. */
int32_t oracle_attention_probs(const oracle_pool *p, int32_t n, const int32_t *qsl,
                               const int32_t *seq_lens, const int32_t *bt, int32_t bt_stride,
                               const void *q, int32_t q_dtype, int32_t num_q_heads,
                               float softmax_scale, int32_t causal, int32_t tok, int32_t head,
                               double *probs) {
  const int64_t H = p->num_kv_heads, D = p->head_dim, Hq = num_q_heads;
  if (H <= 0 || Hq % H) return -1;
  tok_info ti;
  if (!locate_token(n, qsl, seq_lens, tok, &ti)) return -1;
  int64_t nvis = visible_keys(&ti, causal);
  if (nvis <= 0) return 0;
  double *acc = (double *)malloc(sizeof(double) * (size_t)D);
  double m, l;
  attend_range(p, bt + (size_t)ti.req * bt_stride, q, q_dtype, ((size_t)tok * Hq + head) * D,
               head / (Hq / H), (double)softmax_scale, 0, nvis, probs, &m, &l, acc);
  for (int64_t j = 0; j < nvis; ++j) probs[j] = exp(probs[j] - m) / l;
  free(acc);
  return (int32_t)nvis;
}

/*
 * Partitioned evaluation ([P5] third walk-through path, the V2 partitioned
 * PagedAttention): the visible keys are cut into consecutive ranges of
 * `part` keys; each range r yields a local (m_r, l_r, o_r) with o_r the
 * range's own normalised output; the ranges are then merged by
 *   m = max_r m_r,  l = sum_r exp(m_r - m) l_r,
 *   O = sum_r exp(m_r - m) l_r o_r / l,
 * i.e. every local result is rescaled by the same exponential factor.  (The
 * display formula is lost from the page; this is the reading that keeps the
 * result independent of the partition, which the page requires.)
 */
int oracle_attention_partitioned(const oracle_pool *p, int32_t n, const int32_t *qsl,
                                 const int32_t *seq_lens, const int32_t *bt, int32_t bt_stride,
                                 const void *q, int32_t q_dtype, int32_t num_q_heads,
                                 float softmax_scale, int32_t causal, int32_t part, double *out) {
  const int64_t H = p->num_kv_heads, D = p->head_dim, Hq = num_q_heads;
  if (H <= 0 || Hq % H || part <= 0) return ORC_EINVAL;
  const int64_t g = Hq / H;
  const int32_t T = qsl[n];
  int32_t max_L = 1;
  for (int32_t i = 0; i < n; ++i)
    if (seq_lens[i] > max_L) max_L = seq_lens[i];
  int32_t nparts_max = (max_L + part - 1) / part;
  int err = ORC_OK;
#pragma omp parallel
  {
    double *scores = (double *)malloc(sizeof(double) * (size_t)part);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    double *ms = (double *)malloc(sizeof(double) * (size_t)nparts_max);
    double *ls = (double *)malloc(sizeof(double) * (size_t)nparts_max);
    double *os = (double *)malloc(sizeof(double) * (size_t)nparts_max * D);
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int32_t tok = 0; tok < T; ++tok)
      for (int64_t h = 0; h < Hq; ++h) {
        tok_info ti;
        double *o = out + ((size_t)tok * Hq + h) * D;
        if (!locate_token(n, qsl, seq_lens, tok, &ti)) {
#pragma omp atomic write
          err = ORC_EINVAL;
          continue;
        }
        int64_t nvis = visible_keys(&ti, causal);
        int64_t R = (nvis + part - 1) / part;
        for (int64_t r = 0; r < R; ++r) {
          int64_t k0 = r * part, k1 = k0 + part < nvis ? k0 + part : nvis;
          attend_range(p, bt + (size_t)ti.req * bt_stride, q, q_dtype, ((size_t)tok * Hq + h) * D,
                       h / g, (double)softmax_scale, k0, k1, scores, &ms[r], &ls[r], acc);
          for (int64_t e = 0; e < D; ++e) os[r * D + e] = acc[e] / ls[r];
        }
        double m = -INFINITY;
        for (int64_t r = 0; r < R; ++r)
          if (ms[r] > m) m = ms[r];
        double l = 0.0;
        for (int64_t r = 0; r < R; ++r) l += exp(ms[r] - m) * ls[r];
        for (int64_t e = 0; e < D; ++e) {
          double s = 0.0;
          for (int64_t r = 0; r < R; ++r) s += exp(ms[r] - m) * ls[r] * os[r * D + e];
          o[e] = R ? s / l : 0.0;
        }
      }
    free(scores);
    free(acc);
    free(ms);
    free(ls);
    free(os);
  }
  return err;
}

/* Array forms of the codec (used by the tests to sweep many inputs). */
void oracle_e4m3_encode_array(const float *y, uint8_t *codes, int64_t count) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) codes[i] = oracle_e4m3_encode(y[i]);
}

void oracle_e4m3_decode_array(const uint8_t *codes, double *vals, int64_t count) {
  for (int64_t i = 0; i < count; ++i) vals[i] = oracle_e4m3_decode(codes[i]);
}
