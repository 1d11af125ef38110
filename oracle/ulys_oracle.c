/*
 * ulys_oracle.c -- plain, slow, obviously correct CPU oracle for the per-rank
 * hot path of DeepSpeed-Ulysses (pack -> head-sharded attention -> unpack).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * cpu_baseline leg may load this library.  It shares no code, header, table
 * or helper with the HIP path, and the HIP path never loads it.
 *
 * Sources (the pages this follows; every function below names its passage):
 *   [ATLAS]  "02 · DeepSpeed-Ulysses" (llm-infra-atlas, parallel/04_cp),
 *            §1 "attention 沿 head 维并行", §2 "all-to-all 的转置与重分布",
 *            §3 "复杂度对比与 head 数约束".
 *   [DSU]    "DeepSpeed-Ulysses 深度解析：用 All-to-All 序列并行撑起百万 Token
 *            超长序列训练", section "核心设计：沿序列切分 + 两次 All-to-All",
 *            steps 1-5.
 *   [SPCP]   "长上下文训练中的 SP 与 CP：从 Megatron 到分布式 Attention",
 *            section "Ulysses：用 All-to-All 把序列分片换成 head 分片".
 *   [COLL]   "【深度长文】大模型分布式训练通信原语及其应用", primitive
 *            "5. AllToAll（全交换）".
 *   [CMP]    "Ulysses vs Ring Attention：序列并行深度对比", §三 (Q, K and V
 *            take the same all-to-all; SP is capped by num_kv_heads).
 *
 * Conventions (row-major, last axis fastest):
 *   rank-local shard   x  [s/P, b, h, d]
 *   send buffer        y  [P, s/P, b, h/P, d]      block r goes to rank r
 *   head-sharded share    [s, b, h/P, d]           (q, k, v, o of one rank)
 * Layout routines move elt-byte words with memcpy and never convert them,
 * so every bit pattern (NaN payloads, -0, subnormals) is preserved.
 * Attention is fp64 throughout; bf16 inputs are widened exactly.
 *
 * Parity pins: every routine here is pinned by the CPU tests against the
 * pages' worked examples, closed forms, invariants and an independent
 * library evaluation; none is "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EARG (-1)
#define ORC_ENOMEM (-2)

/* ------------------------------------------------------------------------ */
/* Layout: the local halves of the two all-to-alls                          */
/* ------------------------------------------------------------------------ */

static int layout_args_ok(int64_t s, int64_t b, int64_t h, int64_t d, int64_t P,
                          int64_t elt) {
  if (s <= 0 || b <= 0 || h <= 0 || d <= 0 || P <= 0 || elt <= 0) return 0;
  if (s % P != 0 || h % P != 0) return 0; /* [ATLAS] §3: heads % cp == 0 */
  return 1;
}

/*
 * Send side of the seq->head all-to-all, one rank.  [ATLAS] §2: the local
 * [s/cp, heads, d] is split along the head axis into cp parts and part j is
 * sent to rank j; [DSU] step 3.  The send buffer holds the parts in rank
 * order: y[r] = x[:, :, r*hp:(r+1)*hp, :].
 */
int orc_pack(const void *x, void *y, int64_t s, int64_t b, int64_t h, int64_t d,
             int64_t P, int64_t elt) {
  if (!layout_args_ok(s, b, h, d, P, elt)) return ORC_EARG;
  const int64_t sl = s / P, hp = h / P;
  const char *src = (const char *)x;
  char *dst = (char *)y;
  for (int64_t r = 0; r < P; ++r)
    for (int64_t t = 0; t < sl; ++t)
      for (int64_t be = 0; be < b; ++be)
        for (int64_t k = 0; k < hp; ++k)
          for (int64_t e = 0; e < d; ++e) {
            int64_t yi = (((r * sl + t) * b + be) * hp + k) * d + e;
            int64_t xi = ((t * b + be) * h + (r * hp + k)) * d + e;
            memcpy(dst + yi * elt, src + xi * elt, (size_t)elt);
          }
  return ORC_OK;
}

/*
 * Receive side of the head->seq all-to-all, one rank.  [ATLAS] §2: the
 * second all-to-all is the inverse of the first -- blocks received from the
 * P ranks (block r holds head group r) are concatenated along the head axis;
 * [DSU] step 5.  x[:, :, r*hp:(r+1)*hp, :] = y[r].
 */
int orc_unpack(const void *y, void *x, int64_t s, int64_t b, int64_t h, int64_t d,
               int64_t P, int64_t elt) {
  if (!layout_args_ok(s, b, h, d, P, elt)) return ORC_EARG;
  const int64_t sl = s / P, hp = h / P;
  const char *src = (const char *)y;
  char *dst = (char *)x;
  for (int64_t t = 0; t < sl; ++t)
    for (int64_t be = 0; be < b; ++be)
      for (int64_t r = 0; r < P; ++r)
        for (int64_t k = 0; k < hp; ++k)
          for (int64_t e = 0; e < d; ++e) {
            int64_t xi = ((t * b + be) * h + (r * hp + k)) * d + e;
            int64_t yi = (((r * sl + t) * b + be) * hp + k) * d + e;
            memcpy(dst + xi * elt, src + yi * elt, (size_t)elt);
          }
  return ORC_OK;
}

/*
 * The whole seq->head all-to-all across P emulated ranks, written as the
 * pages describe it rather than as pack + routing.  [ATLAS] §2: rank r
 * receives, from every rank j, the j-th token segment of head group r and
 * concatenates them along the sequence axis; [COLL] AllToAll: each rank
 * sends its i-th slice to rank i and concatenates what it receives in
 * source-rank order; [SPCP] X_{i,j} blocks.
 *   X_all [P][s/P][b][h][d]  (shard of rank j at X_all[j])
 *   Y_all [P][s][b][h/P][d]  (share of rank r at Y_all[r])
 */
int orc_seq2head(const void *X_all, void *Y_all, int64_t s, int64_t b, int64_t h,
                 int64_t d, int64_t P, int64_t elt) {
  if (!layout_args_ok(s, b, h, d, P, elt)) return ORC_EARG;
  const int64_t sl = s / P, hp = h / P;
  const char *src = (const char *)X_all;
  char *dst = (char *)Y_all;
  for (int64_t r = 0; r < P; ++r)         /* receiving rank            */
    for (int64_t j = 0; j < P; ++j)       /* source rank, in order     */
      for (int64_t t = 0; t < sl; ++t)    /* token within j's segment  */
        for (int64_t be = 0; be < b; ++be)
          for (int64_t k = 0; k < hp; ++k)
            for (int64_t e = 0; e < d; ++e) {
              int64_t tg = j * sl + t; /* position along the concatenated sequence */
              int64_t yi = (((r * s + tg) * b + be) * hp + k) * d + e;
              int64_t xi = (((j * sl + t) * b + be) * h + (r * hp + k)) * d + e;
              memcpy(dst + yi * elt, src + xi * elt, (size_t)elt);
            }
  return ORC_OK;
}

/*
 * The whole head->seq all-to-all across P emulated ranks.  [ATLAS] §2: split
 * along the sequence, send segment j to rank j, concatenate along the head
 * axis.  Rank j receives from rank r the j-th sequence segment of head
 * group r.
 *   Y_all [P][s][b][h/P][d]  ->  X_all [P][s/P][b][h][d]
 */
int orc_head2seq(const void *Y_all, void *X_all, int64_t s, int64_t b, int64_t h,
                 int64_t d, int64_t P, int64_t elt) {
  if (!layout_args_ok(s, b, h, d, P, elt)) return ORC_EARG;
  const int64_t sl = s / P, hp = h / P;
  const char *src = (const char *)Y_all;
  char *dst = (char *)X_all;
  for (int64_t j = 0; j < P; ++j)         /* receiving rank (sequence owner) */
    for (int64_t r = 0; r < P; ++r)       /* source rank = head group        */
      for (int64_t t = 0; t < sl; ++t)
        for (int64_t be = 0; be < b; ++be)
          for (int64_t k = 0; k < hp; ++k)
            for (int64_t e = 0; e < d; ++e) {
              int64_t tg = j * sl + t;
              int64_t yi = (((r * s + tg) * b + be) * hp + k) * d + e;
              int64_t xi = (((j * sl + t) * b + be) * h + (r * hp + k)) * d + e;
              memcpy(dst + xi * elt, src + yi * elt, (size_t)elt);
            }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Fewer KV heads than ranks: replication and its backward                  */
/* ------------------------------------------------------------------------ */

/*
 * Send side of the seq->head all-to-all for K or V when the model has fewer
 * KV heads than ranks.  [CMP] §三: Q, K and V take the same all-to-all, so
 * with one KV head on four ranks three ranks would receive no KV head at all;
 * [SPCP] (Ulysses section): replicating KV heads lifts the requirement that
 * P divide the KV head count, at a cost in memory and traffic; [DSU]:
 * num_kv_heads is passed when the heads do not divide evenly.  Reading
 * taken: with h_kv < P and h_kv | P, rank r receives KV head
 * floor(r * h_kv / P) -- the head its query heads [r*h/P, (r+1)*h/P) use
 * under the contiguous grouping -- so the send buffer holds P blocks of one
 * head each: y[r] = x[:, :, floor(r*h_kv/P), :].  With P | h_kv it is
 * orc_pack.
 *   x [s/P, b, h_kv, d]  ->  y [P, s/P, b, max(1, h_kv/P), d]
 */
int orc_pack_kv(const void *x, void *y, int64_t s, int64_t b, int64_t h_kv, int64_t d,
                int64_t P, int64_t elt) {
  if (s <= 0 || b <= 0 || h_kv <= 0 || d <= 0 || P <= 0 || elt <= 0) return ORC_EARG;
  if (h_kv % P == 0) return orc_pack(x, y, s, b, h_kv, d, P, elt);
  if (P % h_kv != 0 || s % P != 0) return ORC_EARG;
  const int64_t sl = s / P;
  const char *src = (const char *)x;
  char *dst = (char *)y;
  for (int64_t r = 0; r < P; ++r) {
    const int64_t g = r * h_kv / P; /* the KV head rank r's queries read */
    for (int64_t t = 0; t < sl; ++t)
      for (int64_t be = 0; be < b; ++be)
        for (int64_t e = 0; e < d; ++e) {
          int64_t yi = ((r * sl + t) * b + be) * d + e;
          int64_t xi = ((t * b + be) * h_kv + g) * d + e;
          memcpy(dst + yi * elt, src + xi * elt, (size_t)elt);
        }
  }
  return ORC_OK;
}

static double widen(const void *base, int dtype, int64_t i);

/* Nearest-even rounding of a double to bf16 bits, from the format's
 * definition: 8 significant bits for normal numbers, multiples of 2^-133
 * below 2^-126, infinity past the largest finite value. */
static uint16_t round_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  const double a = fabs(v);
  double q;
  if (a < ldexp(1.0, -126)) {
    q = nearbyint(a * ldexp(1.0, 133)) * ldexp(1.0, -133);
  } else {
    int e;
    const double m = frexp(a, &e); /* a = m 2^e, m in [0.5, 1) */
    q = ldexp(nearbyint(ldexp(m, 8)), e - 8);
  }
  float f = (float)q; /* exact: q has at most 8 significant bits, or is out of range */
  if (q >= ldexp(1.0, 128)) f = INFINITY;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)((u >> 16) | (v < 0 ? 0x8000u : 0u));
}

/*
 * Backward of orc_pack_kv, receive side: the gradient blocks sent back by the
 * P ranks (block r is the gradient of KV head floor(r*h_kv/P) seen by rank
 * r's queries) are summed per KV head -- the gradient of a replicated value
 * is the sum of its copies' gradients ([SPCP]: a K/V row used by many queries
 * receives the sum of their gradients).  The sum is exact in fp64 and rounded
 * once to the dtype (0 fp32, 1 bf16 bits).  With P | h_kv it is orc_unpack.
 *   y [P, s/P, b, max(1, h_kv/P), d]  ->  x [s/P, b, h_kv, d]
 */
int orc_unpack_kv_sum(const void *y, void *x, int64_t s, int64_t b, int64_t h_kv, int64_t d,
                      int64_t P, int dtype) {
  if (dtype != 0 && dtype != 1) return ORC_EARG;
  const int64_t elt = dtype == 0 ? 4 : 2;
  if (s <= 0 || b <= 0 || h_kv <= 0 || d <= 0 || P <= 0) return ORC_EARG;
  if (h_kv % P == 0) return orc_unpack(y, x, s, b, h_kv, d, P, elt);
  if (P % h_kv != 0 || s % P != 0) return ORC_EARG;
  const int64_t sl = s / P, R = P / h_kv;
  for (int64_t t = 0; t < sl; ++t)
    for (int64_t be = 0; be < b; ++be)
      for (int64_t g = 0; g < h_kv; ++g)
        for (int64_t e = 0; e < d; ++e) {
          double acc = 0.0;
          for (int64_t r = g * R; r < (g + 1) * R; ++r) /* the ranks holding head g */
            acc += widen(y, dtype, ((r * sl + t) * b + be) * d + e);
          const int64_t xi = ((t * b + be) * h_kv + g) * d + e;
          if (dtype == 0) {
            ((float *)x)[xi] = (float)acc;
          } else {
            ((uint16_t *)x)[xi] = round_bf16(acc);
          }
        }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention on one rank's share                                            */
/* ------------------------------------------------------------------------ */

/* dtype codes of the inputs: 0 = fp32, 1 = bf16 (raw 16-bit patterns) */
static double widen(const void *base, int dtype, int64_t i) {
  if (dtype == 0) return (double)((const float *)base)[i];
  uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double *widen_all(const void *base, int dtype, int64_t n) {
  double *out = (double *)malloc((size_t)n * sizeof(double));
  if (!out) return NULL;
  for (int64_t i = 0; i < n; ++i) out[i] = widen(base, dtype, i);
  return out;
}

typedef struct {
  const double *q, *k, *v; /* q [s,b,nq,d], k/v [s,b,nkv,d] */
  int64_t s, b, nq, nkv, d;
  int causal;
  const int64_t *rows; /* NULL: every (beta, i, t); else triples */
  int64_t nrows;
  double *o;   /* rows==NULL: [s,b,nq,d]; else [nrows,d] */
  double *lse; /* rows==NULL: [b,nq,s];   else [nrows]   */
  int64_t first, last; /* work range handled by one thread */
  int status;
} attn_job;

/*
 * One query row, by the definition.  [DSU] step 4: each device runs standard
 * attention on its heads, softmax(Q K^T / sqrt(d)) V; [SPCP] (Ring section)
 * writes the scale as 1/sqrt(d_h).  Causal: key j is visible to query t iff
 * j <= t, positions being global ([DSU], the mask is rebuilt from global
 * position ids).  GQA: query head i reads KV head i / (nq/nkv), the grouping
 * under which an even split of Q heads and of KV heads over P ranks keeps
 * each group on one rank ([SPCP] needs P | h_kv; [DSU] num_kv_heads).
 * Two passes over the stored scores: max, then weights, then the weighted
 * sum, all in index order.
 */
static void attn_row(const attn_job *J, int64_t be, int64_t i, int64_t t, double *scores,
                     double *o_row, double *lse_out) {
  const int64_t d = J->d, nq = J->nq, nkv = J->nkv, b = J->b;
  const int64_t g = i / (nq / nkv);
  const int64_t nkeys = J->causal ? t + 1 : J->s;
  const double scale = 1.0 / sqrt((double)d);
  const double *qrow = J->q + ((t * b + be) * nq + i) * d;
  double m = -INFINITY;
  for (int64_t j = 0; j < nkeys; ++j) {
    const double *krow = J->k + ((j * b + be) * nkv + g) * d;
    double acc = 0.0;
    for (int64_t e = 0; e < d; ++e) acc += qrow[e] * krow[e];
    scores[j] = acc * scale;
    if (scores[j] > m) m = scores[j];
  }
  for (int64_t e = 0; e < d; ++e) o_row[e] = 0.0;
  if (nkeys == 0 || m == -INFINITY) { /* no visible key: O = 0, LSE = -inf */
    *lse_out = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j < nkeys; ++j) {
    double w = exp(scores[j] - m);
    l += w;
    const double *vrow = J->v + ((j * b + be) * nkv + g) * d;
    for (int64_t e = 0; e < d; ++e) o_row[e] += w * vrow[e];
  }
  for (int64_t e = 0; e < d; ++e) o_row[e] /= l;
  *lse_out = m + log(l);
}

static void *attn_worker(void *arg) {
  attn_job *J = (attn_job *)arg;
  double *scores = (double *)malloc((size_t)J->s * sizeof(double));
  if (!scores) {
    J->status = ORC_ENOMEM;
    return NULL;
  }
  for (int64_t w = J->first; w < J->last; ++w) {
    int64_t be, i, t;
    double *o_row, *lse_p;
    if (J->rows) {
      be = J->rows[3 * w + 0];
      i = J->rows[3 * w + 1];
      t = J->rows[3 * w + 2];
      o_row = J->o + w * J->d;
      lse_p = J->lse + w;
    } else { /* w enumerates (be, i, t) with t fastest */
      t = w % J->s;
      i = (w / J->s) % J->nq;
      be = w / (J->s * J->nq);
      o_row = J->o + ((t * J->b + be) * J->nq + i) * J->d;
      lse_p = J->lse + (be * J->nq + i) * J->s + t;
    }
    attn_row(J, be, i, t, scores, o_row, lse_p);
  }
  free(scores);
  J->status = ORC_OK;
  return NULL;
}

static int run_attention(const void *q, const void *k, const void *v, double *o, double *lse,
                         int64_t s, int64_t b, int64_t nq, int64_t nkv, int64_t d, int causal,
                         int dtype, const int64_t *rows, int64_t nrows, int nthreads) {
  if (s <= 0 || b <= 0 || nq <= 0 || nkv <= 0 || d <= 0) return ORC_EARG;
  if (nq % nkv != 0 || (dtype != 0 && dtype != 1)) return ORC_EARG;
  if (!q || !k || !v || !o || !lse) return ORC_EARG;
  if (rows) {
    for (int64_t w = 0; w < nrows; ++w) {
      if (rows[3 * w] < 0 || rows[3 * w] >= b || rows[3 * w + 1] < 0 ||
          rows[3 * w + 1] >= nq || rows[3 * w + 2] < 0 || rows[3 * w + 2] >= s)
        return ORC_EARG;
    }
  }
  if (nthreads < 1) nthreads = 1;
  double *qd = widen_all(q, dtype, s * b * nq * d);
  double *kd = widen_all(k, dtype, s * b * nkv * d);
  double *vd = widen_all(v, dtype, s * b * nkv * d);
  attn_job *jobs = (attn_job *)calloc((size_t)nthreads, sizeof(attn_job));
  pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  int rc = ORC_OK;
  if (!qd || !kd || !vd || !jobs || !tid) {
    rc = ORC_ENOMEM;
    goto done;
  }
  const int64_t total = rows ? nrows : b * nq * s;
  for (int n = 0; n < nthreads; ++n) {
    attn_job *J = &jobs[n];
    J->q = qd; J->k = kd; J->v = vd;
    J->s = s; J->b = b; J->nq = nq; J->nkv = nkv; J->d = d;
    J->causal = causal;
    J->rows = rows; J->nrows = nrows;
    J->o = o; J->lse = lse;
    /* interleaved chunks so causal rows of every length spread over threads */
    J->first = total * n / nthreads;
    J->last = total * (n + 1) / nthreads;
    J->status = ORC_ENOMEM;
  }
  if (nthreads == 1) {
    attn_worker(&jobs[0]);
  } else {
    for (int n = 0; n < nthreads; ++n) pthread_create(&tid[n], NULL, attn_worker, &jobs[n]);
    for (int n = 0; n < nthreads; ++n) pthread_join(tid[n], NULL);
  }
  for (int n = 0; n < nthreads; ++n)
    if (jobs[n].status != ORC_OK) rc = jobs[n].status;
done:
  free(qd); free(kd); free(vd); free(jobs); free(tid);
  return rc;
}

/*
 * Head-sharded attention on one rank's share.  [ATLAS] §1: after the first
 * all-to-all each card holds the whole sequence for heads/cp heads and runs
 * attention for those heads locally; [DSU] step 4.
 *   q [s, b, h/P, d], k/v [s, b, h_kv/P, d] (dtype 0 fp32, 1 bf16 bits)
 *   o [s, b, h/P, d] fp64, lse [b, h/P, s] fp64 (natural log)
 */
int orc_attn(const void *q, const void *k, const void *v, double *o, double *lse, int64_t s,
             int64_t b, int64_t h, int64_t h_kv, int64_t d, int64_t P, int causal, int dtype,
             int nthreads) {
  if (P <= 0 || h % P != 0 || h_kv <= 0 || h_kv % P != 0) return ORC_EARG;
  return run_attention(q, k, v, o, lse, s, b, h / P, h_kv / P, d, causal, dtype, NULL, 0,
                       nthreads);
}

/*
 * The same attention evaluated only on listed rows: rows holds nrows
 * triples (beta, local head i, query t); o is [nrows, d], lse [nrows].
 * Used where the full share is too large for the CPU.
 */
int orc_attn_rows(const void *q, const void *k, const void *v, const int64_t *rows,
                  int64_t nrows, double *o, double *lse, int64_t s, int64_t b, int64_t h,
                  int64_t h_kv, int64_t d, int64_t P, int causal, int dtype, int nthreads) {
  if (P <= 0 || h % P != 0 || h_kv <= 0 || h_kv % P != 0 || nrows < 0) return ORC_EARG;
  if (nrows == 0) return ORC_OK;
  return run_attention(q, k, v, o, lse, s, b, h / P, h_kv / P, d, causal, dtype, rows, nrows,
                       nthreads);
}

/* ------------------------------------------------------------------------ */
/* Attention backward on one rank's share                                   */
/* ------------------------------------------------------------------------ */

/*
 * [ATLAS] §5: both all-to-alls are linear, so their backward is the same
 * exchange with the split and concatenation axes swapped, and the local
 * attention's backward is the ordinary attention backward.  The pages print
 * no formula for the latter; it is the gradient of the forward definition
 * (attn_row above).  For one query row with visible keys J, scores
 * S_j = q.k_j / sqrt(d), P = softmax(S) and o = sum_j P_j v_j, a cotangent
 * dout on o gives, by the chain rule through the softmax Jacobian
 * diag(P) - P P^T:
 *   dv_j += P_j dout
 *   dP_j  = dout . v_j
 *   D     = sum_j P_j dP_j            (= dout . o)
 *   dS_j  = P_j (dP_j - D)
 *   dq    = sum_j dS_j k_j / sqrt(d)
 *   dk_j += dS_j q / sqrt(d)
 * dk and dv of a KV head sum the contributions of every query head of its
 * GQA group and every query row that sees the key ([SPCP] notes that one
 * K_j, V_j serving many queries receives the sum of their gradients).
 */
typedef struct {
  const double *q, *k, *v, *dout; /* q, dout [s,b,nq,d]; k, v [s,b,nkv,d] */
  int64_t s, b, nq, nkv, d;
  int causal;
  double *dq, *dk, *dv; /* dq [s,b,nq,d]; dk, dv [s,b,nkv,d] */
  int64_t first, last;  /* range of (beta, kv head) pairs of this thread */
  int status;
} bwd_job;

/* Softmax row of query (be, i, t): fills p[0..nkeys) and returns nkeys. */
static int64_t softmax_row(const double *q, const double *k, int64_t s, int64_t b, int64_t nq,
                           int64_t nkv, int64_t d, int causal, int64_t be, int64_t i, int64_t t,
                           double *p) {
  const int64_t g = i / (nq / nkv);
  const int64_t nkeys = causal ? t + 1 : s;
  const double scale = 1.0 / sqrt((double)d);
  const double *qrow = q + ((t * b + be) * nq + i) * d;
  double m = -INFINITY;
  for (int64_t j = 0; j < nkeys; ++j) {
    const double *krow = k + ((j * b + be) * nkv + g) * d;
    double acc = 0.0;
    for (int64_t e = 0; e < d; ++e) acc += qrow[e] * krow[e];
    p[j] = acc * scale;
    if (p[j] > m) m = p[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < nkeys; ++j) {
    p[j] = exp(p[j] - m);
    l += p[j];
  }
  for (int64_t j = 0; j < nkeys; ++j) p[j] /= l;
  return nkeys;
}

/* dP_j = dout_t . v_j for every visible key, and D = sum_j P_j dP_j. */
static double dp_row(const double *v, const double *dout, int64_t b, int64_t nq, int64_t nkv,
                     int64_t d, int64_t be, int64_t i, int64_t t, const double *p, int64_t nkeys,
                     double *dp) {
  const int64_t g = i / (nq / nkv);
  const double *drow = dout + ((t * b + be) * nq + i) * d;
  double D = 0.0;
  for (int64_t j = 0; j < nkeys; ++j) {
    const double *vrow = v + ((j * b + be) * nkv + g) * d;
    double acc = 0.0;
    for (int64_t e = 0; e < d; ++e) acc += drow[e] * vrow[e];
    dp[j] = acc;
    D += p[j] * acc;
  }
  return D;
}

static void *bwd_worker(void *arg) {
  bwd_job *J = (bwd_job *)arg;
  const int64_t s = J->s, b = J->b, nq = J->nq, nkv = J->nkv, d = J->d, G = nq / nkv;
  const double scale = 1.0 / sqrt((double)d);
  double *p = (double *)malloc((size_t)s * sizeof(double));
  double *dp = (double *)malloc((size_t)s * sizeof(double));
  if (!p || !dp) {
    free(p); free(dp);
    J->status = ORC_ENOMEM;
    return NULL;
  }
  for (int64_t w = J->first; w < J->last; ++w) {
    const int64_t be = w / nkv, g = w % nkv;
    for (int64_t i = g * G; i < (g + 1) * G; ++i) {
      for (int64_t t = 0; t < s; ++t) {
        const int64_t nkeys = softmax_row(J->q, J->k, s, b, nq, nkv, d, J->causal, be, i, t, p);
        const double D = dp_row(J->v, J->dout, b, nq, nkv, d, be, i, t, p, nkeys, dp);
        const double *qrow = J->q + ((t * b + be) * nq + i) * d;
        const double *drow = J->dout + ((t * b + be) * nq + i) * d;
        double *dqrow = J->dq + ((t * b + be) * nq + i) * d;
        for (int64_t e = 0; e < d; ++e) dqrow[e] = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
          const double ds = p[j] * (dp[j] - D);
          const double *krow = J->k + ((j * b + be) * nkv + g) * d;
          double *dkrow = J->dk + ((j * b + be) * nkv + g) * d;
          double *dvrow = J->dv + ((j * b + be) * nkv + g) * d;
          for (int64_t e = 0; e < d; ++e) {
            dqrow[e] += ds * krow[e] * scale;
            dkrow[e] += ds * qrow[e] * scale;
            dvrow[e] += p[j] * drow[e];
          }
        }
      }
    }
  }
  free(p); free(dp);
  J->status = ORC_OK;
  return NULL;
}

/*
 * Merge of two partial attention results over disjoint key sets, one query
 * row at a time.  [SPCP] (Ring section): each query row keeps the running
 * max m of its scores, the sum l of exp(score - m) and the weighted sum A of
 * the values at that scale; a block arriving from another key range is
 * brought to the common max and added, and O = A / l once every block is in.
 * A finished partial result over a key range J carries the same state as
 * lse_J = m + ln l (natural log) and O_J = A / l, so two of them combine as
 *   lse = ln(exp(lse_a) + exp(lse_b)),
 *   O   = exp(lse_a - lse) O_a + exp(lse_b - lse) O_b,
 * written here with the larger lse factored out.  A partial over no key
 * (lse = -inf) contributes nothing; if both are empty, O = 0 and lse = -inf
 * (as for a fully masked row).  The hierarchical scheme ([ATLAS] §4: all-to-all
 * inside a node, a ring across nodes) and USP ([SPCP]: Ulysses groups whose
 * same-head ranks exchange KV around a ring) merge partial results this way.
 * Layouts are those the attention produces for one share:
 *   o_a, o_b, o [s, b, hp, d]; lse_a, lse_b, lse [b, hp, s]; fp64 throughout
 */
int orc_attn_merge(const double *o_a, const double *lse_a, const double *o_b,
                   const double *lse_b, double *o, double *lse, int64_t s, int64_t b,
                   int64_t hp, int64_t d) {
  if (s <= 0 || b <= 0 || hp <= 0 || d <= 0) return ORC_EARG;
  if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return ORC_EARG;
  for (int64_t t = 0; t < s; ++t)
    for (int64_t be = 0; be < b; ++be)
      for (int64_t i = 0; i < hp; ++i) {
        const int64_t li = (be * hp + i) * s + t;  /* this row's lse */
        const int64_t oi = ((t * b + be) * hp + i) * d; /* and its output row */
        const double la = lse_a[li], lb = lse_b[li];
        const double m = la > lb ? la : lb;
        if (m == -INFINITY) {
          for (int64_t e = 0; e < d; ++e) o[oi + e] = 0.0;
          lse[li] = -INFINITY;
          continue;
        }
        const double ea = exp(la - m), eb = exp(lb - m); /* exp(-inf) = 0 */
        const double l = ea + eb;
        for (int64_t e = 0; e < d; ++e) o[oi + e] = (ea * o_a[oi + e] + eb * o_b[oi + e]) / l;
        lse[li] = m + log(l);
      }
  return ORC_OK;
}

/*
 * Backward of the head-sharded attention on one rank's share.
 *   q, dout [s, b, h/P, d]; k, v [s, b, h_kv/P, d] (dtype 0 fp32, 1 bf16 bits)
 *   dq [s, b, h/P, d], dk, dv [s, b, h_kv/P, d] fp64
 */
int orc_attn_bwd(const void *q, const void *k, const void *v, const void *dout, double *dq,
                 double *dk, double *dv, int64_t s, int64_t b, int64_t h, int64_t h_kv, int64_t d,
                 int64_t P, int causal, int dtype, int nthreads) {
  if (P <= 0 || h % P != 0 || h_kv <= 0 || h_kv % P != 0) return ORC_EARG;
  const int64_t nq = h / P, nkv = h_kv / P;
  if (s <= 0 || b <= 0 || nq <= 0 || nkv <= 0 || d <= 0) return ORC_EARG;
  if (nq % nkv != 0 || (dtype != 0 && dtype != 1)) return ORC_EARG;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return ORC_EARG;
  if (nthreads < 1) nthreads = 1;
  double *qd = widen_all(q, dtype, s * b * nq * d);
  double *kd = widen_all(k, dtype, s * b * nkv * d);
  double *vd = widen_all(v, dtype, s * b * nkv * d);
  double *dd = widen_all(dout, dtype, s * b * nq * d);
  bwd_job *jobs = (bwd_job *)calloc((size_t)nthreads, sizeof(bwd_job));
  pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  int rc = ORC_OK;
  if (!qd || !kd || !vd || !dd || !jobs || !tid) {
    rc = ORC_ENOMEM;
    goto done;
  }
  for (int64_t n = 0; n < s * b * nkv * d; ++n) dk[n] = dv[n] = 0.0;
  const int64_t pairs = b * nkv;
  for (int n = 0; n < nthreads; ++n) {
    bwd_job *J = &jobs[n];
    J->q = qd; J->k = kd; J->v = vd; J->dout = dd;
    J->s = s; J->b = b; J->nq = nq; J->nkv = nkv; J->d = d;
    J->causal = causal;
    J->dq = dq; J->dk = dk; J->dv = dv;
    J->first = pairs * n / nthreads;
    J->last = pairs * (n + 1) / nthreads;
    J->status = ORC_ENOMEM;
  }
  if (nthreads == 1) {
    bwd_worker(&jobs[0]);
  } else {
    for (int n = 0; n < nthreads; ++n) pthread_create(&tid[n], NULL, bwd_worker, &jobs[n]);
    for (int n = 0; n < nthreads; ++n) pthread_join(tid[n], NULL);
  }
  for (int n = 0; n < nthreads; ++n)
    if (jobs[n].status != ORC_OK) rc = jobs[n].status;
done:
  free(qd); free(kd); free(vd); free(dd); free(jobs); free(tid);
  return rc;
}

/*
 * The same gradients evaluated only where listed: qrows holds nqr triples
 * (beta, local query head i, query t) whose dq rows go to dq [nqr, d]; krows
 * holds nkr triples (beta, local KV head g, key j) whose dk and dv rows go
 * to dk, dv [nkr, d].  A key's gradients visit every query row that sees it
 * (t >= j when causal), each with its whole softmax row, so late keys of a
 * causal share are cheap and early ones cost a full pass.  Single-threaded
 * per listed item, threads over items.
 */
typedef struct {
  const double *q, *k, *v, *dout;
  int64_t s, b, nq, nkv, d;
  int causal;
  const int64_t *qrows, *krows;
  int64_t nqr, nkr;
  double *dq, *dk, *dv;
  int64_t first, last; /* items [0, nqr) are query rows, [nqr, nqr + nkr) keys */
  int status;
} bwd_rows_job;

static void *bwd_rows_worker(void *arg) {
  bwd_rows_job *J = (bwd_rows_job *)arg;
  const int64_t s = J->s, b = J->b, nq = J->nq, nkv = J->nkv, d = J->d, G = nq / nkv;
  const double scale = 1.0 / sqrt((double)d);
  double *p = (double *)malloc((size_t)s * sizeof(double));
  double *dp = (double *)malloc((size_t)s * sizeof(double));
  if (!p || !dp) {
    free(p); free(dp);
    J->status = ORC_ENOMEM;
    return NULL;
  }
  for (int64_t w = J->first; w < J->last; ++w) {
    if (w < J->nqr) {
      const int64_t be = J->qrows[3 * w], i = J->qrows[3 * w + 1], t = J->qrows[3 * w + 2];
      const int64_t g = i / G;
      const int64_t nkeys = softmax_row(J->q, J->k, s, b, nq, nkv, d, J->causal, be, i, t, p);
      const double D = dp_row(J->v, J->dout, b, nq, nkv, d, be, i, t, p, nkeys, dp);
      double *dqrow = J->dq + w * d;
      for (int64_t e = 0; e < d; ++e) dqrow[e] = 0.0;
      for (int64_t j = 0; j < nkeys; ++j) {
        const double ds = p[j] * (dp[j] - D);
        const double *krow = J->k + ((j * b + be) * nkv + g) * d;
        for (int64_t e = 0; e < d; ++e) dqrow[e] += ds * krow[e] * scale;
      }
    } else {
      const int64_t u = w - J->nqr;
      const int64_t be = J->krows[3 * u], g = J->krows[3 * u + 1], j = J->krows[3 * u + 2];
      double *dkrow = J->dk + u * d;
      double *dvrow = J->dv + u * d;
      for (int64_t e = 0; e < d; ++e) dkrow[e] = dvrow[e] = 0.0;
      for (int64_t i = g * G; i < (g + 1) * G; ++i) {
        for (int64_t t = J->causal ? j : 0; t < s; ++t) {
          const int64_t nkeys = softmax_row(J->q, J->k, s, b, nq, nkv, d, J->causal, be, i, t, p);
          const double D = dp_row(J->v, J->dout, b, nq, nkv, d, be, i, t, p, nkeys, dp);
          const double ds = p[j] * (dp[j] - D);
          const double *qrow = J->q + ((t * b + be) * nq + i) * d;
          const double *drow = J->dout + ((t * b + be) * nq + i) * d;
          for (int64_t e = 0; e < d; ++e) {
            dkrow[e] += ds * qrow[e] * scale;
            dvrow[e] += p[j] * drow[e];
          }
        }
      }
    }
  }
  free(p); free(dp);
  J->status = ORC_OK;
  return NULL;
}

int orc_attn_bwd_rows(const void *q, const void *k, const void *v, const void *dout,
                      const int64_t *qrows, int64_t nqr, const int64_t *krows, int64_t nkr,
                      double *dq, double *dk, double *dv, int64_t s, int64_t b, int64_t h,
                      int64_t h_kv, int64_t d, int64_t P, int causal, int dtype, int nthreads) {
  if (P <= 0 || h % P != 0 || h_kv <= 0 || h_kv % P != 0 || nqr < 0 || nkr < 0) return ORC_EARG;
  const int64_t nq = h / P, nkv = h_kv / P;
  if (s <= 0 || b <= 0 || nq <= 0 || nkv <= 0 || d <= 0) return ORC_EARG;
  if (nq % nkv != 0 || (dtype != 0 && dtype != 1)) return ORC_EARG;
  if (!q || !k || !v || !dout) return ORC_EARG;
  if ((nqr > 0 && (!qrows || !dq)) || (nkr > 0 && (!krows || !dk || !dv))) return ORC_EARG;
  for (int64_t w = 0; w < nqr; ++w)
    if (qrows[3 * w] < 0 || qrows[3 * w] >= b || qrows[3 * w + 1] < 0 ||
        qrows[3 * w + 1] >= nq || qrows[3 * w + 2] < 0 || qrows[3 * w + 2] >= s)
      return ORC_EARG;
  for (int64_t u = 0; u < nkr; ++u)
    if (krows[3 * u] < 0 || krows[3 * u] >= b || krows[3 * u + 1] < 0 ||
        krows[3 * u + 1] >= nkv || krows[3 * u + 2] < 0 || krows[3 * u + 2] >= s)
      return ORC_EARG;
  if (nqr + nkr == 0) return ORC_OK;
  if (nthreads < 1) nthreads = 1;
  double *qd = widen_all(q, dtype, s * b * nq * d);
  double *kd = widen_all(k, dtype, s * b * nkv * d);
  double *vd = widen_all(v, dtype, s * b * nkv * d);
  double *dd = widen_all(dout, dtype, s * b * nq * d);
  bwd_rows_job *jobs = (bwd_rows_job *)calloc((size_t)nthreads, sizeof(bwd_rows_job));
  pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  int rc = ORC_OK;
  if (!qd || !kd || !vd || !dd || !jobs || !tid) {
    rc = ORC_ENOMEM;
    goto done;
  }
  const int64_t total = nqr + nkr;
  for (int n = 0; n < nthreads; ++n) {
    bwd_rows_job *J = &jobs[n];
    J->q = qd; J->k = kd; J->v = vd; J->dout = dd;
    J->s = s; J->b = b; J->nq = nq; J->nkv = nkv; J->d = d;
    J->causal = causal;
    J->qrows = qrows; J->krows = krows; J->nqr = nqr; J->nkr = nkr;
    J->dq = dq; J->dk = dk; J->dv = dv;
    J->first = total * n / nthreads;
    J->last = total * (n + 1) / nthreads;
    J->status = ORC_ENOMEM;
  }
  if (nthreads == 1) {
    bwd_rows_worker(&jobs[0]);
  } else {
    for (int n = 0; n < nthreads; ++n) pthread_create(&tid[n], NULL, bwd_rows_worker, &jobs[n]);
    for (int n = 0; n < nthreads; ++n) pthread_join(tid[n], NULL);
  }
  for (int n = 0; n < nthreads; ++n)
    if (jobs[n].status != ORC_OK) rc = jobs[n].status;
done:
  free(qd); free(kd); free(vd); free(dd); free(jobs); free(tid);
  return rc;
}
