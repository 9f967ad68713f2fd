/*
 * CPU oracle for one grouped-query decode-attention step followed by the
 * output projection, plus the dense fp16 GEMM check.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct
 * definition that the GPU kernels are compared against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it. It shares
 * no code, header, table or helper with the HIP library.
 *
 * Every floating-point step is done in IEEE double. Inputs arrive as raw
 * 16-bit words (bf16 or fp16) and are widened exactly; outputs are rounded
 * once, directly from the double result, to the nearest bf16/fp16 value with
 * ties to even.
 *
 * Sources (the pages this follows):
 *  [F16]  "PyPTO 开箱性能调优实战：Decode Attention 多 Matmul 独立 TileShape
 *         配置 F-16" -- section "代码对比" (the three matmul calls of one
 *         decode-attention forward: q_grouped x k_cache^T to fp32 scores, the
 *         elided vector ops, attn_weights x v_cache to bf16, then
 *         attn_output_flat x o_weight to bf16) and the table in section
 *         "三个 Matmul 的 Shape 特征分析" (M/K/N of each matmul).
 *  [KPP]  CANN msKPP "自动调优流程 / Kernel级自动调优" -- the BasicMatmul
 *         example: C = A x B, fp16, row-major, checked with np.matmul.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - the elided "vector ops" are: multiply each score by softmax_scale
 *    (1/sqrt(head_dim) by default), then the max-subtracted softmax over the
 *    keys j < seq_len[b] of that sequence;
 *  - query head qh reads KV head qh / G with G = Hq / Hkv (consecutive groups,
 *    which is what "q_grouped" names);
 *  - attn_output_flat is head-major: column qh*D + d;
 *  - o_weight has no b_trans, so it is [K = Hq*D, N] row-major;
 *  - the k_cache/v_cache of one (batch, kv head) are [max_seq_len, D]
 *    row-major; rows >= seq_len[b] are never read.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-2)
#define ORACLE_ENOMEM (-6)

/* ---------------------------------------------------------------------- */
/* 16-bit float words <-> double                                          */
/* ---------------------------------------------------------------------- */

/* A bf16 word is the top half of an IEEE binary32 word. */
double oracle_bf16_to_double(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0x1f) {
    v = f ? NAN : INFINITY;
  } else if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  } else {
    v = ldexp((double)(f | 0x400), e - 25); /* (1024 + f) * 2^(e-15-10) */
  }
  return sign ? -v : v;
}

/*
 * Round |a| (finite, > 0) to a multiple of 2^qexp with ties to even.
 * a / 2^qexp is computed exactly (power-of-two scaling), so the only rounding
 * is the explicit one below.
 */
static double round_to_quantum(double a, int qexp) {
  double t = ldexp(a, -qexp);
  double fl = floor(t);
  double frac = t - fl; /* exact: t and fl share an exponent range */
  double r;
  if (frac > 0.5) {
    r = fl + 1.0;
  } else if (frac < 0.5) {
    r = fl;
  } else {
    r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
  }
  return ldexp(r, qexp);
}

/*
 * Nearest value with `sig` significant bits, exponent of the leading bit at
 * least `emin` (below it the quantum stays 2^(emin - sig + 1): subnormals).
 */
static double round_sig(double a, int sig, int emin) {
  int e2;
  frexp(a, &e2); /* a = m * 2^e2, m in [0.5, 1): leading bit has exponent e2-1 */
  int lead = e2 - 1;
  if (lead < emin) lead = emin;
  return round_to_quantum(a, lead - (sig - 1));
}

/* double -> bf16 word, round to nearest even, NaN stays NaN, overflow -> inf. */
uint16_t oracle_bf16_from_double(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return (uint16_t)(sign | 0x7fc0);
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7f80);
  double r = round_sig(a, 8, -126);
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7f80);
  /* r is exactly representable as binary32 with the low 16 bits zero. */
  float f = (float)r;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | ((u >> 16) & 0x7fff));
}

/* double -> IEEE binary16 word, round to nearest even, overflow -> inf. */
uint16_t oracle_f16_from_double(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return (uint16_t)(sign | 0x7e00);
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7c00);
  double r = round_sig(a, 11, -14);
  if (r >= 65536.0) return (uint16_t)(sign | 0x7c00); /* 65520 and up round to inf */
  if (r == 0.0) return sign;
  int e2;
  double m = frexp(r, &e2); /* r = m * 2^e2 */
  int lead = e2 - 1;
  if (lead < -14) {
    /* subnormal: r = f * 2^-24 */
    uint16_t f = (uint16_t)ldexp(r, 24);
    return (uint16_t)(sign | f);
  }
  uint16_t ebits = (uint16_t)(lead + 15);
  uint16_t frac = (uint16_t)(ldexp(m, 11) - 1024.0); /* 11-bit significand minus hidden bit */
  return (uint16_t)(sign | (ebits << 10) | frac);
}

/* ---------------------------------------------------------------------- */
/* thread pool over independent units (each unit is computed sequentially) */
/* ---------------------------------------------------------------------- */

typedef void (*unit_fn)(void* ctx, long unit);
typedef struct {
  unit_fn fn;
  void* ctx;
  long nunits;
  int tid, nthreads;
} worker_arg;

static void* worker_main(void* p) {
  worker_arg* w = (worker_arg*)p;
  for (long u = w->tid; u < w->nunits; u += w->nthreads) w->fn(w->ctx, u);
  return NULL;
}

static int run_units(unit_fn fn, void* ctx, long nunits, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nunits) nthreads = (int)(nunits > 0 ? nunits : 1);
  if (nthreads == 1) {
    for (long u = 0; u < nunits; u++) fn(ctx, u);
    return ORACLE_OK;
  }
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  worker_arg* wa = (worker_arg*)calloc((size_t)nthreads, sizeof(worker_arg));
  if (!th || !wa) {
    free(th);
    free(wa);
    return ORACLE_ENOMEM;
  }
  for (int t = 0; t < nthreads; t++) {
    wa[t].fn = fn;
    wa[t].ctx = ctx;
    wa[t].nunits = nunits;
    wa[t].tid = t;
    wa[t].nthreads = nthreads;
  }
  int started = 0;
  for (int t = 0; t < nthreads; t++) {
    if (pthread_create(&th[t], NULL, worker_main, &wa[t]) != 0) break;
    started++;
  }
  /* any unit whose thread failed to start is run here */
  for (int t = started; t < nthreads; t++) worker_main(&wa[t]);
  for (int t = 0; t < started; t++) pthread_join(th[t], NULL);
  free(th);
  free(wa);
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* attention: [F16] first two matmuls and the vector ops between them     */
/* ---------------------------------------------------------------------- */

typedef struct {
  const uint16_t *q, *k, *v;
  const int32_t* seq_lens;
  int B, Hq, Hkv, D, Lmax;
  double scale;
  double* attn_ref;    /* [B, Hq*D] unrounded, or NULL */
  uint16_t* flat;      /* [B, Hq*D] bf16 words */
  double* scores;      /* [B, Hq, Lmax] scaled scores, or NULL */
  double* lse;         /* [B, Hq] natural-log sum-exp of the scaled scores, or NULL */
  double* probs;       /* [B, Hq, Lmax] softmax weights, or NULL */
  int err;
} attn_ctx;

/* One unit = one (batch b, kv head h) pair: all G query heads that share it. */
static void attn_unit(void* p, long unit) {
  attn_ctx* c = (attn_ctx*)p;
  const int G = c->Hq / c->Hkv;
  const int D = c->D;
  const int b = (int)(unit / c->Hkv);
  const int h = (int)(unit % c->Hkv);
  const int L = c->seq_lens[b];
  const size_t kv_base = ((size_t)b * c->Hkv + h) * (size_t)c->Lmax * D;
  double* s = (double*)malloc(sizeof(double) * (size_t)L);
  double* e = (double*)malloc(sizeof(double) * (size_t)L);
  if (!s || !e) {
    free(s);
    free(e);
    c->err = ORACLE_ENOMEM;
    return;
  }
  for (int g = 0; g < G; g++) {
    const int qh = h * G + g;
    const uint16_t* qrow = c->q + ((size_t)b * c->Hq + qh) * D;
    /* scores: s_j = (sum_d q_d * K_jd) * scale  (q x k_cache^T, fp32-or-wider) */
    for (int j = 0; j < L; j++) {
      const uint16_t* krow = c->k + kv_base + (size_t)j * D;
      double dot = 0.0;
      for (int d = 0; d < D; d++) dot += oracle_bf16_to_double(qrow[d]) * oracle_bf16_to_double(krow[d]);
      s[j] = dot * c->scale;
    }
    /* softmax over every key of the sequence, max-subtracted */
    double mx = s[0];
    for (int j = 1; j < L; j++)
      if (s[j] > mx) mx = s[j];
    double Z = 0.0;
    for (int j = 0; j < L; j++) {
      e[j] = exp(s[j] - mx);
      Z += e[j];
    }
    /* attn_weights x v_cache: o_d = sum_j p_j * V_jd */
    const size_t out_row = (size_t)b * c->Hq * D + (size_t)qh * D;
    for (int d = 0; d < D; d++) {
      double o = 0.0;
      for (int j = 0; j < L; j++) o += (e[j] / Z) * oracle_bf16_to_double(c->v[kv_base + (size_t)j * D + d]);
      if (c->attn_ref) c->attn_ref[out_row + d] = o;
      c->flat[out_row + d] = oracle_bf16_from_double(o);
    }
    const size_t srow = ((size_t)b * c->Hq + qh) * (size_t)c->Lmax;
    if (c->scores)
      for (int j = 0; j < L; j++) c->scores[srow + j] = s[j];
    if (c->probs)
      for (int j = 0; j < L; j++) c->probs[srow + j] = e[j] / Z;
    if (c->lse) c->lse[(size_t)b * c->Hq + qh] = mx + log(Z);
  }
  free(s);
  free(e);
}

static int check_attn_args(int B, int Hq, int Hkv, int D, int Lmax, const int32_t* seq_lens) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || Lmax < 1) return ORACLE_EINVAL;
  if (Hq % Hkv != 0) return ORACLE_EINVAL;
  for (int b = 0; b < B; b++)
    if (seq_lens[b] < 1 || seq_lens[b] > Lmax) return ORACLE_EINVAL;
  return ORACLE_OK;
}

/*
 * Attention only. q [B,Hq,D], k/v [B,Hkv,Lmax,D] (bf16 words), seq_lens [B].
 * Writes flat [B, Hq*D] (bf16 words) and, when non-NULL, the unrounded
 * output, the scaled scores, the softmax weights and the log-sum-exp.
 */
int oracle_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seq_lens, int B,
                     int Hq, int Hkv, int D, int Lmax, double scale, double* attn_ref, uint16_t* flat,
                     double* scores, double* probs, double* lse, int nthreads) {
  int rc = check_attn_args(B, Hq, Hkv, D, Lmax, seq_lens);
  if (rc) return rc;
  attn_ctx c = {.q = q, .k = k, .v = v, .seq_lens = seq_lens, .B = B, .Hq = Hq, .Hkv = Hkv, .D = D, .Lmax = Lmax,
                .scale = scale, .attn_ref = attn_ref, .flat = flat, .scores = scores, .lse = lse, .probs = probs,
                .err = 0};
  rc = run_units(attn_unit, &c, (long)B * Hkv, nthreads);
  return rc ? rc : c.err;
}

/* ---------------------------------------------------------------------- */
/* context (prefill) attention: a chunk of T new tokens per sequence       */
/* ---------------------------------------------------------------------- */
/*
 * The page "CCCL → Triton 方法论迁移" (section 二, 2.1 prefix_prefill.py,
 * Context Attention) names this kernel next to the decode attention but does
 * not spell out what it computes;
 * the plainest reading is taken: sequence b holds ctx_lens[b] cached keys,
 * the last T of which belong to the chunk's tokens, and token t (absolute
 * position ctx_lens[b] - T + t) attends causally to keys 0 .. its own
 * position, with the same scaled, max-subtracted softmax as the decode step.
 * T = 1 is exactly the decode step.
 */
typedef struct {
  const uint16_t *q, *k, *v;
  const int32_t* ctx_lens;
  int B, T, Hq, Hkv, D, Lmax;
  double scale;
  double* ref;    /* [B, T, Hq*D] unrounded, or NULL */
  uint16_t* out;  /* [B, T, Hq*D] bf16 words */
  int err;
} prefill_ctx;

/* One unit = one (batch b, kv head h) pair: every token of the chunk and every
 * query head of the group. */
static void prefill_unit(void* p, long unit) {
  prefill_ctx* c = (prefill_ctx*)p;
  const int G = c->Hq / c->Hkv;
  const int D = c->D;
  const int b = (int)(unit / c->Hkv);
  const int h = (int)(unit % c->Hkv);
  const int ctx = c->ctx_lens[b];
  const size_t kv_base = ((size_t)b * c->Hkv + h) * (size_t)c->Lmax * D;
  double* s = (double*)malloc(sizeof(double) * (size_t)ctx);
  if (!s) {
    c->err = ORACLE_ENOMEM;
    return;
  }
  for (int t = 0; t < c->T; t++) {
    const int L = ctx - c->T + t + 1; /* keys up to and including the token's own position */
    for (int g = 0; g < G; g++) {
      const int qh = h * G + g;
      const uint16_t* qrow = c->q + (((size_t)b * c->T + t) * c->Hq + qh) * D;
      for (int j = 0; j < L; j++) {
        const uint16_t* krow = c->k + kv_base + (size_t)j * D;
        double dot = 0.0;
        for (int d = 0; d < D; d++) dot += oracle_bf16_to_double(qrow[d]) * oracle_bf16_to_double(krow[d]);
        s[j] = dot * c->scale;
      }
      double mx = s[0];
      for (int j = 1; j < L; j++)
        if (s[j] > mx) mx = s[j];
      double Z = 0.0;
      for (int j = 0; j < L; j++) {
        s[j] = exp(s[j] - mx);
        Z += s[j];
      }
      const size_t out_row = (((size_t)b * c->T + t) * c->Hq + qh) * D;
      for (int d = 0; d < D; d++) {
        double o = 0.0;
        for (int j = 0; j < L; j++) o += (s[j] / Z) * oracle_bf16_to_double(c->v[kv_base + (size_t)j * D + d]);
        if (c->ref) c->ref[out_row + d] = o;
        c->out[out_row + d] = oracle_bf16_from_double(o);
      }
    }
  }
  free(s);
}

/*
 * q [B, T, Hq, D], k/v [B, Hkv, Lmax, D] (bf16 words), ctx_lens [B] with
 * T <= ctx_lens[b] <= Lmax. Writes out [B, T, Hq*D] (bf16 words) and, when
 * non-NULL, the unrounded output.
 */
int oracle_prefill_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* ctx_lens,
                             int B, int T, int Hq, int Hkv, int D, int Lmax, double scale, double* ref,
                             uint16_t* out, int nthreads) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1 || Lmax < 1 || Hq % Hkv != 0) return ORACLE_EINVAL;
  for (int b = 0; b < B; b++)
    if (ctx_lens[b] < T || ctx_lens[b] > Lmax) return ORACLE_EINVAL;
  prefill_ctx c = {.q = q, .k = k, .v = v, .ctx_lens = ctx_lens, .B = B, .T = T, .Hq = Hq, .Hkv = Hkv, .D = D,
                   .Lmax = Lmax, .scale = scale, .ref = ref, .out = out, .err = 0};
  int rc = run_units(prefill_unit, &c, (long)B * Hkv, nthreads);
  return rc ? rc : c.err;
}

/* ---------------------------------------------------------------------- */
/* output projection: [F16] third matmul, attn_output_flat x o_weight      */
/* ---------------------------------------------------------------------- */

typedef struct {
  const uint16_t *x, *w;
  int M, K, N;
  int is_f16; /* 0: bf16 words, 1: fp16 words (inputs and output) */
  double* out_ref;
  uint16_t* out;
} mm_ctx;

#define MM_COLS_PER_UNIT 64

/* One unit = a block of output columns for all rows. */
static void mm_unit(void* p, long unit) {
  mm_ctx* c = (mm_ctx*)p;
  const int n0 = (int)unit * MM_COLS_PER_UNIT;
  const int n1 = n0 + MM_COLS_PER_UNIT < c->N ? n0 + MM_COLS_PER_UNIT : c->N;
  for (int m = 0; m < c->M; m++) {
    for (int n = n0; n < n1; n++) {
      double acc = 0.0;
      for (int kk = 0; kk < c->K; kk++) {
        uint16_t xa = c->x[(size_t)m * c->K + kk];
        uint16_t wb = c->w[(size_t)kk * c->N + n];
        double xv = c->is_f16 ? oracle_f16_to_double(xa) : oracle_bf16_to_double(xa);
        double wv = c->is_f16 ? oracle_f16_to_double(wb) : oracle_bf16_to_double(wb);
        acc += xv * wv;
      }
      if (c->out_ref) c->out_ref[(size_t)m * c->N + n] = acc;
      c->out[(size_t)m * c->N + n] = c->is_f16 ? oracle_f16_from_double(acc) : oracle_bf16_from_double(acc);
    }
  }
}

static int run_mm(const uint16_t* x, const uint16_t* w, int M, int K, int N, int is_f16, double* out_ref,
                  uint16_t* out, int nthreads) {
  if (M < 1 || K < 1 || N < 1) return ORACLE_EINVAL;
  mm_ctx c = {.x = x, .w = w, .M = M, .K = K, .N = N, .is_f16 = is_f16, .out_ref = out_ref, .out = out};
  return run_units(mm_unit, &c, (N + MM_COLS_PER_UNIT - 1) / MM_COLS_PER_UNIT, nthreads);
}

/* out[m,n] = sum_k x[m,k] * w[k,n]; x [M,K], w [K,N] bf16 words, row-major. */
int oracle_oproj(const uint16_t* x, const uint16_t* w, int M, int K, int N, double* out_ref, uint16_t* out,
                 int nthreads) {
  return run_mm(x, w, M, K, N, 0, out_ref, out, nthreads);
}

/* [KPP] C = A x B, A [M,K], B [K,N], C [M,N], fp16 words, row-major. */
int oracle_gemm_f16(const uint16_t* A, const uint16_t* B, int M, int N, int K, double* c_ref, uint16_t* C,
                    int nthreads) {
  return run_mm(A, B, M, K, N, 1, c_ref, C, nthreads);
}

/*
 * The whole decode step: attention, head-major flatten (rounded to bf16, as
 * the attn_output matmul of [F16] writes bf16), then the output projection
 * of that bf16 vector. out [B, N] bf16 words.
 */
int oracle_decode_step(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seq_lens,
                       const uint16_t* o_weight, int B, int Hq, int Hkv, int D, int Lmax, int N, double scale,
                       double* attn_ref, uint16_t* flat, double* out_ref, uint16_t* out, int nthreads) {
  int rc = oracle_attention(q, k, v, seq_lens, B, Hq, Hkv, D, Lmax, scale, attn_ref, flat, NULL, NULL, NULL,
                            nthreads);
  if (rc) return rc;
  return oracle_oproj(flat, o_weight, B, Hq * D, N, out_ref, out, nthreads);
}
