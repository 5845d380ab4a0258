/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  Never linked into, loaded by or
 * called from the product path; only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py use it.
 *
 * A plain, slow, obviously correct fp64 reference for
 *   (1) scaled dot-product attention, Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V
 *       ("Attention Is All You Need" section 3.2.1, Eq. 1, as restated on the
 *       vlmlib.cn paper summary of 1706.03762 and on the rockcohen.cc deep read,
 *       section 5.1), and
 *   (2) multi-head attention, MultiHead = Concat(head_1..head_h) W^O with
 *       head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V) (paper section 3.2.2; the
 *       vlmlib.cn summary and rockcohen.cc section 5.2), and
 *   (3) one projection of that block, y = x . W (no bias), and
 *   (4) one decoding step over a key/value cache (the newest n_q positions of
 *       each sequence under the causal mask),
 *   (5) restricted self-attention over a neighbourhood of radius r,
 *   (6) the gradients of SDPA with respect to Q, K and V, and
 *   (7) the attention sublayer around the MHA: sinusoidal positional encoding
 *       added to the input, then LayerNorm(x + MultiHead(x, ...)).
 *
 * Definitions followed literally, one query row at a time:
 *   legal(j)  <=>  j < n_kv  and  (no key lengths or j < L_kv[b])
 *                            and  (no causal mask  or j <= i)
 *     (causal: the "illegal connections" of the decoder are the keys after the
 *      query; they are set to -inf at the softmax input, which gives them an
 *      exact zero weight -- rockcohen.cc sections 5.3 and 6.3.)
 *   s_j  = scale * sum_c Q[i,c] K[j,c]             for legal j
 *   m    = max_j s_j,  e_j = exp(s_j - m),  Z = sum_j e_j
 *          (the max shift leaves the softmax unchanged -- rockcohen.cc 3.2)
 *   O[i] = sum_j (e_j / Z) V[j],   lse = m + ln Z
 *   Query rows with i >= L_q[b] (when query lengths are given) and rows with
 *   no legal key are defined as O = 0, lse = -inf.
 * The MHA projections have no bias (the formula in the paper has none);
 * weights are row-major W[in][out] and the product is X.W.  Head h owns the
 * contiguous columns [h*d_k, (h+1)*d_k) of each projection and the output
 * columns [h*d_v, (h+1)*d_v) of the concatenation.
 *
 * Every sum runs in index order in a single fp64 accumulator, so results do
 * not depend on the number of threads.  No fusion, tiling or reordering.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* ---- bf16 storage rounding (diagnostic mode of the MHA only) ------------ */
/* Round an fp64 value to the nearest bf16 value, ties to even, computed from
 * the definition: the spacing of bf16 numbers near x is 2^(e-7) where 2^e <=
 * |x| < 2^(e+1) (e clamped at -126 for subnormals).  x/spacing is exact in
 * fp64, and nearbyint rounds half to even in the default rounding mode. */
static double round_bf16(double x) {
  if (!isfinite(x) || x == 0.0) return x;
  int e;
  frexp(x, &e);             /* x = f * 2^e with 0.5 <= |f| < 1 -> 2^(e-1) <= |x| */
  int ex = e - 1;
  if (ex < -126) ex = -126;
  double spacing = ldexp(1.0, ex - 7);
  double r = nearbyint(x / spacing) * spacing;
  if (fabs(r) >= ldexp(1.0, 128)) r = copysign(INFINITY, x);
  return r;
}

/* ---- one query row of SDPA ---------------------------------------------- */
/* q: d_k values; key j's row at K + j*k_stride, value j's row at V + j*v_stride.
 * Keys legal_begin..legal_end-1 pass the length and window tests; causal_i >= 0
 * adds the causal test j <= causal_i.  s: scratch of n_kv doubles. */
static void sdpa_row(const double* q, const double* K, int64_t k_stride, const double* V,
                     int64_t v_stride, int n_kv, int d_k, int d_v, double scale, int legal_begin,
                     int legal_end, int causal_i, double* s, double* out, double* lse) {
#define LEGAL(j) ((j) >= legal_begin && (j) < legal_end && (causal_i < 0 || (j) <= causal_i))
  int any = 0;
  double m = -INFINITY;
  for (int j = 0; j < n_kv; ++j) {              /* scores of the legal keys, and their max */
    if (!LEGAL(j)) continue;
    double dot = 0.0;
    const double* kj = K + (int64_t)j * k_stride;
    for (int c = 0; c < d_k; ++c) dot += q[c] * kj[c];
    s[j] = scale * dot;
    if (!any || s[j] > m) m = s[j];
    any = 1;
  }
  for (int c = 0; c < d_v; ++c) out[c] = 0.0;
  if (!any) { if (lse) *lse = -INFINITY; return; }
  double Z = 0.0;
  for (int j = 0; j < n_kv; ++j) {              /* e_j = exp(s_j - m); illegal keys weigh 0 */
    if (!LEGAL(j)) continue;
    s[j] = exp(s[j] - m);
    Z += s[j];
  }
  for (int j = 0; j < n_kv; ++j) {              /* O = sum_j (e_j / Z) V_j */
    if (!LEGAL(j)) continue;
    double w = s[j] / Z;
    const double* vj = V + (int64_t)j * v_stride;
    for (int c = 0; c < d_v; ++c) out[c] += w * vj[c];
  }
  if (lse) *lse = m + log(Z);
#undef LEGAL
}

/* ---- simple thread pool over an index range ----------------------------- */
typedef void (*range_fn)(void* ctx, int64_t begin, int64_t end, double* scratch);
typedef struct {
  range_fn fn; void* ctx; int64_t begin, end; int64_t scratch_len; int failed;
} range_job;

static void* range_thread(void* p) {
  range_job* job = (range_job*)p;
  double* scratch = NULL;
  if (job->scratch_len > 0) {
    scratch = (double*)malloc((size_t)job->scratch_len * sizeof(double));
    if (!scratch) { job->failed = 1; return NULL; }
  }
  job->fn(job->ctx, job->begin, job->end, scratch);
  free(scratch);
  return NULL;
}

static int parallel_for(int64_t n, int nthreads, int64_t scratch_len, range_fn fn, void* ctx) {
  if (n <= 0) return ORACLE_OK;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = (int)n;
  range_job* jobs = (range_job*)calloc((size_t)nthreads, sizeof(range_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !tids) { free(jobs); free(tids); return ORACLE_ENOMEM; }
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn; jobs[t].ctx = ctx; jobs[t].scratch_len = scratch_len;
    jobs[t].begin = n * t / nthreads; jobs[t].end = n * (t + 1) / nthreads;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&tids[t], NULL, range_thread, &jobs[t]) != 0) break;
    started = t;
  }
  range_thread(&jobs[0]);
  for (int t = started + 1; t < nthreads; ++t) range_thread(&jobs[t]);  /* not started: run here */
  for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
  int failed = 0;
  for (int t = 0; t < nthreads; ++t) failed |= jobs[t].failed;
  free(jobs); free(tids);
  return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ---- SDPA over contiguous [B,H,n,d] tensors ------------------------------ */
typedef struct {
  int B, H, n_q, n_kv, d_k, d_v; double scale; int causal;
  const double *q, *k, *v; double *o, *lse;
  const int *seqlens_q, *seqlens_kv;
  const int64_t* rows;   /* NULL: row r is flat index r; else rows[r] is the flat index */
  int decode;            /* 1: query i is sequence position L_kv[b] - n_q + i (see below) */
  int window;            /* >= 0: only keys with |i - j| <= window are legal */
} sdpa_ctx;

static void sdpa_range(void* p, int64_t begin, int64_t end, double* s) {
  const sdpa_ctx* c = (const sdpa_ctx*)p;
  for (int64_t r = begin; r < end; ++r) {
    int64_t flat = c->rows ? c->rows[r] : r;          /* flat = (b*H + h)*n_q + i */
    int i = (int)(flat % c->n_q);
    int64_t bh = flat / c->n_q;
    int b = (int)(bh / c->H);
    double* out = c->o + r * c->d_v;
    double* lse = c->lse ? c->lse + r : NULL;
    if (c->seqlens_q && i >= c->seqlens_q[b]) {       /* padded query row */
      for (int x = 0; x < c->d_v; ++x) out[x] = 0.0;
      if (lse) *lse = -INFINITY;
      continue;
    }
    int legal_end = c->n_kv;
    if (c->seqlens_kv && c->seqlens_kv[b] < legal_end) legal_end = c->seqlens_kv[b];
    const double* q = c->q + flat * c->d_k;
    const double* K = c->k + bh * c->n_kv * c->d_k;
    const double* V = c->v + bh * c->n_kv * c->d_v;
    int causal_i = c->causal ? i : -1;
    if (c->decode) {                                  /* the last n_q positions of the sequence */
      int pos = legal_end - c->n_q + i;
      if (pos < 0) legal_end = 0;                     /* before the sequence: no legal key */
      else causal_i = pos;
    }
    int legal_begin = 0;
    if (c->window >= 0) {                             /* restricted: the neighbourhood |i - j| <= r */
      /* in 64 bits: i + r + 1 exceeds int range for a radius near INT_MAX */
      const long long lo = (long long)i - c->window, hi = (long long)i + c->window + 1;
      legal_begin = lo < 0 ? 0 : (int)lo;
      if (hi < legal_end) legal_end = (int)hi;
    }
    sdpa_row(q, K, c->d_k, V, c->d_v, c->n_kv, c->d_k, c->d_v, c->scale, legal_begin, legal_end,
             causal_i, s, out, lse);
  }
}

static int check_lengths(const int* lens, int B, int cap) {
  if (!lens) return 1;
  for (int b = 0; b < B; ++b) if (lens[b] < 0 || lens[b] > cap) return 0;
  return 1;
}

/* Full SDPA: q [B,H,n_q,d_k], k [B,H,n_kv,d_k], v [B,H,n_kv,d_v] -> o [B,H,n_q,d_v],
 * lse [B,H,n_q] (may be NULL).  seqlens_q / seqlens_kv: NULL or [B]. */
int oracle_sdpa_f64(int B, int H, int n_q, int n_kv, int d_k, int d_v, const double* q,
                    const double* k, const double* v, double* o, double* lse, double scale,
                    int causal, const int* seqlens_q, const int* seqlens_kv, int nthreads) {
  if (B < 0 || H < 0 || n_q < 0 || n_kv < 0 || d_k < 1 || d_v < 1 || !(scale > 0.0)) return ORACLE_EINVAL;
  if (!check_lengths(seqlens_q, B, n_q) || !check_lengths(seqlens_kv, B, n_kv)) return ORACLE_EINVAL;
  sdpa_ctx c = {B, H, n_q, n_kv, d_k, d_v, scale, causal, q, k, v, o, lse, seqlens_q, seqlens_kv, NULL, 0, -1};
  return parallel_for((int64_t)B * H * n_q, nthreads, n_kv > 0 ? n_kv : 1, sdpa_range, &c);
}

/* Restricted self-attention: query i only attends to the keys of its
 * neighbourhood of radius r, |i - j| <= r (a window of 2r + 1 positions
 * centred on i, cut at the sequence ends), on top of the length and causal
 * tests -- the paper's proposal for very long inputs, cost O(r n d) instead of
 * O(n^2 d) (section 4 and Table 1; the csdn blog, section 4.3; the vlmlib.cn
 * summary's limitations paragraph). */
int oracle_sdpa_window_f64(int B, int H, int n_q, int n_kv, int d_k, int d_v, const double* q,
                           const double* k, const double* v, double* o, double* lse, double scale,
                           int causal, const int* seqlens_q, const int* seqlens_kv, int window,
                           int nthreads) {
  if (B < 0 || H < 0 || n_q < 0 || n_kv < 0 || d_k < 1 || d_v < 1 || !(scale > 0.0) || window < 0)
    return ORACLE_EINVAL;
  if (!check_lengths(seqlens_q, B, n_q) || !check_lengths(seqlens_kv, B, n_kv)) return ORACLE_EINVAL;
  sdpa_ctx c = {B, H, n_q, n_kv, d_k, d_v, scale, causal, q, k, v, o, lse, seqlens_q, seqlens_kv, NULL, 0,
                window};
  return parallel_for((int64_t)B * H * n_q, nthreads, n_kv > 0 ? n_kv : 1, sdpa_range, &c);
}

/* One decoding step over a key/value cache: the n_q queries are the newest
 * n_q positions of each sequence, L_kv[b] - n_q + i for query i (L_kv = n_kv
 * when no lengths are given), and each attends to the cache up to and
 * including its own position -- the decoder's causal mask of section 3.2.3
 * (rockcohen.cc 5.3) applied to the last rows only, as autoregressive
 * generation evaluates it one step at a time (attention-paper-guide sections
 * 05 and 07+, misconception 03; the vlmlib.cn summary's training-objective
 * paragraph; the csdn blog, section 3.6).  A query whose position is negative
 * (L_kv[b] < n_q) has no legal key: O = 0, lse = -inf. */
int oracle_decode_f64(int B, int H, int n_q, int n_kv, int d_k, int d_v, const double* q,
                      const double* k, const double* v, double* o, double* lse, double scale,
                      const int* seqlens_kv, int nthreads) {
  if (B < 0 || H < 0 || n_q < 0 || n_kv < 0 || d_k < 1 || d_v < 1 || !(scale > 0.0)) return ORACLE_EINVAL;
  if (!check_lengths(seqlens_kv, B, n_kv)) return ORACLE_EINVAL;
  sdpa_ctx c = {B, H, n_q, n_kv, d_k, d_v, scale, 0, q, k, v, o, lse, NULL, seqlens_kv, NULL, 1, -1};
  return parallel_for((int64_t)B * H * n_q, nthreads, n_kv > 0 ? n_kv : 1, sdpa_range, &c);
}

/* Same, for selected rows only: rows[r] = (b*H + h)*n_q + i; o is [nrows, d_v],
 * lse is [nrows] (may be NULL). */
int oracle_sdpa_rows_f64(int B, int H, int n_q, int n_kv, int d_k, int d_v, const double* q,
                         const double* k, const double* v, const int64_t* rows, int64_t nrows,
                         double* o, double* lse, double scale, int causal, const int* seqlens_q,
                         const int* seqlens_kv, int nthreads) {
  if (B < 0 || H < 0 || n_q < 0 || n_kv < 0 || d_k < 1 || d_v < 1 || !(scale > 0.0)) return ORACLE_EINVAL;
  if (!check_lengths(seqlens_q, B, n_q) || !check_lengths(seqlens_kv, B, n_kv)) return ORACLE_EINVAL;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * H * n_q) return ORACLE_EINVAL;
  sdpa_ctx c = {B, H, n_q, n_kv, d_k, d_v, scale, causal, q, k, v, o, lse, seqlens_q, seqlens_kv, rows, 0, -1};
  return parallel_for(nrows, nthreads, n_kv > 0 ? n_kv : 1, sdpa_range, &c);
}

/* ---- SDPA backward -------------------------------------------------------- */
/* Gradients of the loss sum_{i,c} dO[i,c] O[i,c] with respect to Q, K and V,
 * written out from the chain rule through the definition above (the paper
 * trains the model end to end: the vlmlib.cn summary's training-objective
 * paragraph; attention-paper-guide section 05).  Per (b, h), for every valid
 * query row i and its legal keys j, in index order:
 *   P_ij = exp(s_ij - m_i) / Z_i                    (the forward weights)
 *   O_i  = sum_j P_ij V_j,   D_i = sum_c dO_ic O_ic
 *   dP_ij = sum_c dO_ic V_jc
 *   dS_ij = P_ij (dP_ij - D_i)                      (softmax Jacobian)
 *   dQ_i  = scale sum_j dS_ij K_j
 *   dK_j += scale dS_ij Q_i,   dV_j += P_ij dO_i
 * Padded query rows (i >= L_q) and illegal keys take no part: their O is a
 * constant, so their gradients are zero. */
typedef struct {
  int B, H, n_q, n_kv, d_k, d_v; double scale; int causal;
  const double *q, *k, *v, *dout; double *dq, *dk, *dv;
  const int *seqlens_q, *seqlens_kv;
} bwd_ctx;

static void sdpa_bwd_range(void* p, int64_t begin, int64_t end, double* scratch) {
  const bwd_ctx* c = (const bwd_ctx*)p;
  double* P = scratch;                    /* n_kv */
  double* O = scratch + c->n_kv;          /* d_v  */
  for (int64_t bh = begin; bh < end; ++bh) {
    int b = (int)(bh / c->H);
    const double* Q = c->q + bh * c->n_q * c->d_k;
    const double* K = c->k + bh * c->n_kv * c->d_k;
    const double* V = c->v + bh * c->n_kv * c->d_v;
    const double* dO = c->dout + bh * c->n_q * c->d_v;
    double* dQ = c->dq + bh * c->n_q * c->d_k;
    double* dK = c->dk + bh * c->n_kv * c->d_k;
    double* dV = c->dv + bh * c->n_kv * c->d_v;
    for (int64_t x = 0; x < (int64_t)c->n_q * c->d_k; ++x) dQ[x] = 0.0;
    for (int64_t x = 0; x < (int64_t)c->n_kv * c->d_k; ++x) dK[x] = 0.0;
    for (int64_t x = 0; x < (int64_t)c->n_kv * c->d_v; ++x) dV[x] = 0.0;
    int Lq = c->seqlens_q ? c->seqlens_q[b] : c->n_q;
    int Lkv = c->seqlens_kv ? c->seqlens_kv[b] : c->n_kv;
    for (int i = 0; i < Lq; ++i) {
      int jend = Lkv;
      if (c->causal && i + 1 < jend) jend = i + 1;
      if (jend <= 0) continue;                          /* no legal key: O = 0, no gradient */
      const double* qi = Q + (int64_t)i * c->d_k;
      const double* doi = dO + (int64_t)i * c->d_v;
      double m = -INFINITY;
      for (int j = 0; j < jend; ++j) {                  /* scores and their max */
        double dot = 0.0;
        for (int x = 0; x < c->d_k; ++x) dot += qi[x] * K[(int64_t)j * c->d_k + x];
        P[j] = c->scale * dot;
        if (P[j] > m) m = P[j];
      }
      double Z = 0.0;
      for (int j = 0; j < jend; ++j) { P[j] = exp(P[j] - m); Z += P[j]; }
      for (int j = 0; j < jend; ++j) P[j] /= Z;
      for (int x = 0; x < c->d_v; ++x) O[x] = 0.0;
      for (int j = 0; j < jend; ++j)
        for (int x = 0; x < c->d_v; ++x) O[x] += P[j] * V[(int64_t)j * c->d_v + x];
      double D = 0.0;
      for (int x = 0; x < c->d_v; ++x) D += doi[x] * O[x];
      double* dqi = dQ + (int64_t)i * c->d_k;
      for (int j = 0; j < jend; ++j) {
        const double* vj = V + (int64_t)j * c->d_v;
        double dp = 0.0;
        for (int x = 0; x < c->d_v; ++x) dp += doi[x] * vj[x];
        double ds = P[j] * (dp - D);
        const double* kj = K + (int64_t)j * c->d_k;
        double* dkj = dK + (int64_t)j * c->d_k;
        double* dvj = dV + (int64_t)j * c->d_v;
        for (int x = 0; x < c->d_k; ++x) dqi[x] += c->scale * ds * kj[x];
        for (int x = 0; x < c->d_k; ++x) dkj[x] += c->scale * ds * qi[x];
        for (int x = 0; x < c->d_v; ++x) dvj[x] += P[j] * doi[x];
      }
    }
  }
}

/* q, k, v, dout as in oracle_sdpa_f64 (dout [B,H,n_q,d_v]); writes dq, dk, dv
 * of the same shapes as q, k, v. */
int oracle_sdpa_bwd_f64(int B, int H, int n_q, int n_kv, int d_k, int d_v, const double* q,
                        const double* k, const double* v, const double* dout, double* dq, double* dk,
                        double* dv, double scale, int causal, const int* seqlens_q,
                        const int* seqlens_kv, int nthreads) {
  if (B < 0 || H < 0 || n_q < 0 || n_kv < 0 || d_k < 1 || d_v < 1 || !(scale > 0.0)) return ORACLE_EINVAL;
  if (!check_lengths(seqlens_q, B, n_q) || !check_lengths(seqlens_kv, B, n_kv)) return ORACLE_EINVAL;
  bwd_ctx c = {B, H, n_q, n_kv, d_k, d_v, scale, causal, q, k, v, dout, dq, dk, dv, seqlens_q, seqlens_kv};
  return parallel_for((int64_t)B * H, nthreads, (int64_t)n_kv + d_v + 1, sdpa_bwd_range, &c);
}

/* ---- dense product C[r,:] = A[r,:] . W  (W row-major [K][N]) ------------- */
typedef struct {
  const double* a; int64_t a_stride; const int64_t* a_rows;   /* a_rows NULL: row r */
  const double* w; int K, N; double* c; int round_out;
} gemm_ctx;

static void gemm_range(void* p, int64_t begin, int64_t end, double* unused) {
  (void)unused;
  const gemm_ctx* g = (const gemm_ctx*)p;
  for (int64_t r = begin; r < end; ++r) {
    const double* a = g->a + (g->a_rows ? g->a_rows[r] : r) * g->a_stride;
    double* c = g->c + r * g->N;
    for (int n = 0; n < g->N; ++n) c[n] = 0.0;
    for (int kk = 0; kk < g->K; ++kk) {            /* c[n] = sum_k a[k] w[k][n], k in order */
      double ak = a[kk];
      const double* wk = g->w + (int64_t)kk * g->N;
      for (int n = 0; n < g->N; ++n) c[n] += ak * wk[n];
    }
    if (g->round_out) for (int n = 0; n < g->N; ++n) c[n] = round_bf16(c[n]);
  }
}

/* One projection of the multi-head block, y = x . w (no bias): the products
 * X W_i^Q, X W_i^K, X W_i^V and Concat(head_1..h) W^O of the paper's section
 * 3.2.2 all have this form.  x rows have stride x_stride; rows (NULL or
 * [M]) selects which rows of x produce the M rows of y; w is row-major
 * [K][N]; y is [M][N]. */
int oracle_linear_f64(int M, int K, int N, const double* x, int64_t x_stride, const int64_t* rows,
                      int64_t x_rows, const double* w, double* y, int nthreads) {
  if (M < 0 || K < 0 || N < 0 || x_stride < K || x_rows < 0) return ORACLE_EINVAL;
  if (rows)
    for (int64_t r = 0; r < M; ++r)
      if (rows[r] < 0 || rows[r] >= x_rows) return ORACLE_EINVAL;
  if (!rows && M > x_rows) return ORACLE_EINVAL;
  gemm_ctx g = {x, x_stride, rows, w, K, N, y, 0};
  return parallel_for(M, nthreads, 0, gemm_range, &g);
}

/* ---- multi-head attention ------------------------------------------------ */
typedef struct {
  int B, n_q, n_kv, H, d_k, d_v, causal; double scale;
  const double *qp, *kp, *vp;        /* qp rows indexed by r (sampled) or b*n_q+i */
  const int64_t* rows;               /* NULL: all rows; else rows[r] = b*n_q + i */
  int kv_batch_fixed;                /* >= 0: kp/vp hold batch kv_batch_fixed only */
  const int *seqlens_q, *seqlens_kv;
  double* ocat; int round_out;
} mha_attn_ctx;

static void mha_attn_range(void* p, int64_t begin, int64_t end, double* s) {
  const mha_attn_ctx* c = (const mha_attn_ctx*)p;
  int64_t wq = (int64_t)c->H * c->d_k, wv = (int64_t)c->H * c->d_v;
  for (int64_t r = begin; r < end; ++r) {
    int64_t row = c->rows ? c->rows[r] : r;
    int b = (int)(row / c->n_q), i = (int)(row % c->n_q);
    double* ocat = c->ocat + r * wv;
    if (c->seqlens_q && i >= c->seqlens_q[b]) {
      for (int64_t x = 0; x < wv; ++x) ocat[x] = 0.0;
      continue;
    }
    int legal_end = c->n_kv;
    if (c->seqlens_kv && c->seqlens_kv[b] < legal_end) legal_end = c->seqlens_kv[b];
    int64_t kvb = c->kv_batch_fixed >= 0 ? 0 : b;
    for (int h = 0; h < c->H; ++h) {
      const double* q = c->qp + r * wq + (int64_t)h * c->d_k;
      const double* K = c->kp + kvb * c->n_kv * wq + (int64_t)h * c->d_k;
      const double* V = c->vp + kvb * c->n_kv * wv + (int64_t)h * c->d_v;
      sdpa_row(q, K, wq, V, wv, c->n_kv, c->d_k, c->d_v, c->scale, 0, legal_end,
               c->causal ? i : -1, s, ocat + (int64_t)h * c->d_v, NULL);
    }
    if (c->round_out) for (int64_t x = 0; x < wv; ++x) ocat[x] = round_bf16(ocat[x]);
  }
}

static int mha_args_ok(int B, int n_q, int n_kv, int d_model, int H, int d_k, int d_v, double scale,
                       const int* lq, const int* lkv) {
  if (B < 0 || n_q < 0 || n_kv < 0 || d_model < 1 || H < 1 || d_k < 1 || d_v < 1 || !(scale > 0.0)) return 0;
  return check_lengths(lq, B, n_q) && check_lengths(lkv, B, n_kv);
}

/* Full MHA.  x_q [B,n_q,d_model], x_kv [B,n_kv,d_model]; w_q, w_k [d_model, H*d_k];
 * w_v [d_model, H*d_v]; w_o [H*d_v, d_model]; y [B,n_q,d_model].
 * flags bit 0: round the projections and the concatenation to bf16 where a
 * bf16 implementation stores them (diagnostic only; the definition is flags=0). */
int oracle_mha_f64(int B, int n_q, int n_kv, int d_model, int H, int d_k, int d_v,
                   const double* x_q, const double* x_kv, const double* w_q, const double* w_k,
                   const double* w_v, const double* w_o, double* y, double scale, int causal,
                   const int* seqlens_q, const int* seqlens_kv, int flags, int nthreads) {
  if (!mha_args_ok(B, n_q, n_kv, d_model, H, d_k, d_v, scale, seqlens_q, seqlens_kv)) return ORACLE_EINVAL;
  int rnd = flags & 1;
  int64_t wq = (int64_t)H * d_k, wv = (int64_t)H * d_v;
  double* qp = (double*)malloc(sizeof(double) * (size_t)((int64_t)B * n_q * wq + 1));
  double* kp = (double*)malloc(sizeof(double) * (size_t)((int64_t)B * n_kv * wq + 1));
  double* vp = (double*)malloc(sizeof(double) * (size_t)((int64_t)B * n_kv * wv + 1));
  double* oc = (double*)malloc(sizeof(double) * (size_t)((int64_t)B * n_q * wv + 1));
  int rc = ORACLE_ENOMEM;
  if (qp && kp && vp && oc) {
    gemm_ctx gq = {x_q, d_model, NULL, w_q, d_model, (int)wq, qp, rnd};
    gemm_ctx gk = {x_kv, d_model, NULL, w_k, d_model, (int)wq, kp, rnd};
    gemm_ctx gv = {x_kv, d_model, NULL, w_v, d_model, (int)wv, vp, rnd};
    mha_attn_ctx ac = {B, n_q, n_kv, H, d_k, d_v, causal, scale, qp, kp, vp, NULL, -1,
                       seqlens_q, seqlens_kv, oc, rnd};
    gemm_ctx go = {oc, wv, NULL, w_o, (int)wv, d_model, y, 0};
    rc = parallel_for((int64_t)B * n_q, nthreads, 0, gemm_range, &gq);
    if (!rc) rc = parallel_for((int64_t)B * n_kv, nthreads, 0, gemm_range, &gk);
    if (!rc) rc = parallel_for((int64_t)B * n_kv, nthreads, 0, gemm_range, &gv);
    if (!rc) rc = parallel_for((int64_t)B * n_q, nthreads, n_kv > 0 ? n_kv : 1, mha_attn_range, &ac);
    if (!rc) rc = parallel_for((int64_t)B * n_q, nthreads, 0, gemm_range, &go);
  }
  free(qp); free(kp); free(vp); free(oc);
  return rc;
}

/* MHA for selected output rows only: rows[r] = b*n_q + i, y is [nrows, d_model].
 * The key/value projections are computed in full for each batch element that
 * the selection touches. */
int oracle_mha_rows_f64(int B, int n_q, int n_kv, int d_model, int H, int d_k, int d_v,
                        const double* x_q, const double* x_kv, const double* w_q,
                        const double* w_k, const double* w_v, const double* w_o,
                        const int64_t* rows, int64_t nrows, double* y, double scale, int causal,
                        const int* seqlens_q, const int* seqlens_kv, int flags, int nthreads) {
  if (!mha_args_ok(B, n_q, n_kv, d_model, H, d_k, d_v, scale, seqlens_q, seqlens_kv)) return ORACLE_EINVAL;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * n_q) return ORACLE_EINVAL;
  int rnd = flags & 1;
  int64_t wq = (int64_t)H * d_k, wv = (int64_t)H * d_v;
  double* kp = (double*)malloc(sizeof(double) * (size_t)((int64_t)n_kv * wq + 1));
  double* vp = (double*)malloc(sizeof(double) * (size_t)((int64_t)n_kv * wv + 1));
  double* qp = (double*)malloc(sizeof(double) * (size_t)(nrows * wq + 1));
  double* oc = (double*)malloc(sizeof(double) * (size_t)(nrows * wv + 1));
  int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows + 1));
  int64_t* xrow = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows + 1));
  int rc = (kp && vp && qp && oc && sel && xrow) ? ORACLE_OK : ORACLE_ENOMEM;
  for (int b = 0; b < B && !rc; ++b) {
    int64_t ns = 0;
    for (int64_t r = 0; r < nrows; ++r)
      if (rows[r] / n_q == b) { sel[ns] = rows[r]; xrow[ns] = r; ++ns; }
    if (!ns) continue;
    gemm_ctx gk = {x_kv + (int64_t)b * n_kv * d_model, d_model, NULL, w_k, d_model, (int)wq, kp, rnd};
    gemm_ctx gv = {x_kv + (int64_t)b * n_kv * d_model, d_model, NULL, w_v, d_model, (int)wv, vp, rnd};
    gemm_ctx gq = {x_q, d_model, sel, w_q, d_model, (int)wq, qp, rnd};
    mha_attn_ctx ac = {B, n_q, n_kv, H, d_k, d_v, causal, scale, qp, kp, vp, sel, b,
                       seqlens_q, seqlens_kv, oc, rnd};
    rc = parallel_for(n_kv, nthreads, 0, gemm_range, &gk);
    if (!rc) rc = parallel_for(n_kv, nthreads, 0, gemm_range, &gv);
    if (!rc) rc = parallel_for(ns, nthreads, 0, gemm_range, &gq);
    if (!rc) rc = parallel_for(ns, nthreads, n_kv > 0 ? n_kv : 1, mha_attn_range, &ac);
    if (!rc) {
      double* ytmp = (double*)malloc(sizeof(double) * (size_t)(ns * d_model + 1));
      if (!ytmp) { rc = ORACLE_ENOMEM; break; }
      gemm_ctx go = {oc, wv, NULL, w_o, (int)wv, d_model, ytmp, 0};
      rc = parallel_for(ns, nthreads, 0, gemm_range, &go);
      for (int64_t t = 0; t < ns && !rc; ++t)
        memcpy(y + xrow[t] * d_model, ytmp + t * d_model, sizeof(double) * (size_t)d_model);
      free(ytmp);
    }
  }
  free(kp); free(vp); free(qp); free(oc); free(sel); free(xrow);
  return rc;
}

/* ---- Positional encoding, LayerNorm, the attention sublayer -------------- */
/* Sinusoidal positional encoding (paper section 3.5, restated on the
 * vlmlib.cn summary and rockcohen.cc section 5.4):
 *   PE[pos][2i]   = sin(pos / 10000^(2i/d_model))
 *   PE[pos][2i+1] = cos(pos / 10000^(2i/d_model))
 * pos counts from 0; for odd d_model the last column is a sine. */
int oracle_pe_f64(int n, int d_model, double* pe) {
  if (n < 0 || d_model < 1) return ORACLE_EINVAL;
  for (int pos = 0; pos < n; ++pos)
    for (int c = 0; c < d_model; ++c) {
      int i2 = c - (c & 1);                                   /* 2i */
      double angle = (double)pos / pow(10000.0, (double)i2 / (double)d_model);
      pe[(int64_t)pos * d_model + c] = (c & 1) ? cos(angle) : sin(angle);
    }
  return ORACLE_OK;
}

/* LayerNorm over the last dimension (the ai-master transformer_lab page, its
 * section on the other core components: LN(x) = gamma (x - mu) / sqrt(var +
 * eps) + beta, with mu and var the mean and the (population) variance of the
 * d features of one position; rockcohen.cc section 5.5).  Two passes per row:
 * the mean, then the mean of squared deviations. */
int oracle_layernorm_f64(int64_t rows, int d, const double* z, const double* gamma,
                         const double* beta, double eps, double* y) {
  if (rows < 0 || d < 1 || !(eps >= 0.0)) return ORACLE_EINVAL;
  for (int64_t r = 0; r < rows; ++r) {
    const double* zr = z + r * d;
    double mu = 0.0, var = 0.0;
    for (int c = 0; c < d; ++c) mu += zr[c];
    mu /= d;
    for (int c = 0; c < d; ++c) var += (zr[c] - mu) * (zr[c] - mu);
    var /= d;
    double rstd = 1.0 / sqrt(var + eps);
    for (int c = 0; c < d; ++c) y[r * d + c] = gamma[c] * (zr[c] - mu) * rstd + beta[c];
  }
  return ORACLE_OK;
}

/* The attention sublayer of the encoder and decoder (paper section 3.1, post-LN:
 * the vlmlib.cn summary's formula Sublayer_out(x) = LayerNorm(x + Sublayer(x));
 * rockcohen.cc section 5.5):
 *   h = x_q + PE          (add_pe; the embedding layer's input to the first
 *                          layer, paper section 3.5; self-attention only)
 *   z = h + MultiHead(h, kv, kv),  kv = h for self-attention (x_kv == NULL),
 *                                  else x_kv (cross-attention, no PE)
 *   y = LayerNorm(z)
 * All in fp64, no rounding.  z_out (optional) receives z. */
static int block_prologue(int B, int n_q, int d_model, const double* x_q, int add_pe, double** h_out) {
  int64_t nh = (int64_t)B * n_q * d_model;
  double* h = (double*)malloc(sizeof(double) * (size_t)(nh + 1));
  double* pe = (double*)malloc(sizeof(double) * (size_t)((int64_t)n_q * d_model + 1));
  if (!h || !pe) { free(h); free(pe); return ORACLE_ENOMEM; }
  oracle_pe_f64(n_q, d_model, pe);
  for (int b = 0; b < B; ++b)
    for (int64_t t = 0; t < (int64_t)n_q * d_model; ++t)
      h[(int64_t)b * n_q * d_model + t] = x_q[(int64_t)b * n_q * d_model + t] + (add_pe ? pe[t] : 0.0);
  free(pe);
  *h_out = h;
  return ORACLE_OK;
}

int oracle_mha_block_f64(int B, int n_q, int n_kv, int d_model, int H, int d_k, int d_v,
                         const double* x_q, const double* x_kv, int add_pe, const double* w_q,
                         const double* w_k, const double* w_v, const double* w_o,
                         const double* gamma, const double* beta, double eps, double* y,
                         double* z_out, double scale, int causal, const int* seqlens_q,
                         const int* seqlens_kv, int nthreads) {
  if (add_pe && x_kv) return ORACLE_EINVAL;
  if (!x_kv && n_kv != n_q) return ORACLE_EINVAL;
  double* h = NULL;
  int rc = block_prologue(B, n_q, d_model, x_q, add_pe, &h);
  if (rc) return rc;
  int64_t nz = (int64_t)B * n_q * d_model;
  double* z = (double*)malloc(sizeof(double) * (size_t)(nz + 1));
  if (!z) { free(h); return ORACLE_ENOMEM; }
  rc = oracle_mha_f64(B, n_q, n_kv, d_model, H, d_k, d_v, h, x_kv ? x_kv : h, w_q, w_k, w_v, w_o, z,
                      scale, causal, seqlens_q, seqlens_kv, 0, nthreads);
  if (!rc) {
    for (int64_t t = 0; t < nz; ++t) z[t] += h[t];               /* residual */
    rc = oracle_layernorm_f64((int64_t)B * n_q, d_model, z, gamma, beta, eps, y);
    if (!rc && z_out) memcpy(z_out, z, sizeof(double) * (size_t)nz);
  }
  free(h); free(z);
  return rc;
}

/* The same sublayer for selected output rows only (rows[r] = b*n_q + i; y and
 * z_out are [nrows, d_model]). */
int oracle_mha_block_rows_f64(int B, int n_q, int n_kv, int d_model, int H, int d_k, int d_v,
                              const double* x_q, const double* x_kv, int add_pe, const double* w_q,
                              const double* w_k, const double* w_v, const double* w_o,
                              const double* gamma, const double* beta, double eps,
                              const int64_t* rows, int64_t nrows, double* y, double* z_out,
                              double scale, int causal, const int* seqlens_q, const int* seqlens_kv,
                              int nthreads) {
  if (add_pe && x_kv) return ORACLE_EINVAL;
  if (!x_kv && n_kv != n_q) return ORACLE_EINVAL;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * n_q) return ORACLE_EINVAL;
  double* h = NULL;
  int rc = block_prologue(B, n_q, d_model, x_q, add_pe, &h);
  if (rc) return rc;
  double* z = (double*)malloc(sizeof(double) * (size_t)(nrows * d_model + 1));
  if (!z) { free(h); return ORACLE_ENOMEM; }
  rc = oracle_mha_rows_f64(B, n_q, n_kv, d_model, H, d_k, d_v, h, x_kv ? x_kv : h, w_q, w_k, w_v, w_o,
                           rows, nrows, z, scale, causal, seqlens_q, seqlens_kv, 0, nthreads);
  if (!rc) {
    for (int64_t r = 0; r < nrows; ++r)
      for (int c = 0; c < d_model; ++c) z[r * d_model + c] += h[rows[r] * d_model + c];
    rc = oracle_layernorm_f64(nrows, d_model, z, gamma, beta, eps, y);
    if (!rc && z_out) memcpy(z_out, z, sizeof(double) * (size_t)(nrows * d_model));
  }
  free(h); free(z);
  return rc;
}

/* Exposed so the storage-rounding helper itself can be pinned by tests. */
double oracle_round_bf16(double x) { return round_bf16(x); }
