/*
 * The oracle's layer step in plain C, fp64, on all host cores: the CPU baseline's form of the
 * oracle in oracle/__init__.py (the same definition, written out as loops instead of numpy).
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the benchmark's
 * CPU-baseline leg load this library; it shares no code with the HIP library.
 *
 * What it computes, for one layer step of T new tokens per sequence:
 *  1. K = X·Wk, V = X·Wv and Q = X·Wq without bias — "Paper Notes: DirectKV", section
 *     "Fundamental Underlying Technologies / Kernel Fusion (Projection + Attention)", step 1 of
 *     the standard path. Every product is a sum over the model width in index order, in fp64.
 *  2. The new K/V rows are rounded to the cache dtype (round to nearest, ties to even) and written
 *     at token rows [past_len[b], past_len[b] + T) of the host cache — same page, section "System
 *     Architecture", KV Cache Manager. Q stays in fp64.
 *  3. softmax(Q·Kᵀ/√d)·V over the keys a query may see — same page, "Kernel Fusion", step 2 of
 *     the standard path. Readings (the same as the numpy oracle's): scale 1/√d; query head h reads
 *     kv head h / (Hq / Hkv); new token t of sequence b sees cache rows 0 .. past_len[b] + t, its
 *     own row included. The softmax subtracts the row maximum before exp (the result is the same
 *     as without, up to rounding).
 *
 * Work is shared by threads over (sequence, kv head, block of 16 query tokens): each item reads
 * the group's key and value rows once for all its query rows. That changes which thread computes
 * a value, never the order of any sum, so results do not depend on the thread count.
 *
 * Arrays (row-major): x [B][T][D] and weights wq [D][Hq*d], wk, wv [D][Hkv*d] as float32 holding
 * values exact in the dtype; caches kc, vc [B][Hkv][cap][d] float32 (appended to in place);
 * t_index [n_t] the new tokens whose attention output is wanted; out [B][n_t][Hq][d] fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* significand precision p (hidden bit included), minimum normal exponent, maximum exponent */
static const int kFormat[3][3] = {{24, -126, 127}, {11, -14, 15}, {8, -126, 127}};   /* f32, f16, bf16 */

/* x rounded to the nearest value of dtype (0 f32, 1 f16, 2 bf16), ties to even, with gradual
   underflow and overflow to infinity (IEEE 754 roundTiesToEven). */
double oref_round(double x, int dtype) {
  if (dtype < 0 || dtype > 2 || x == 0.0 || !isfinite(x)) return x;
  const int p = kFormat[dtype][0], emin = kFormat[dtype][1], emax = kFormat[dtype][2];
  int e2;
  frexp(x, &e2);                       /* x = m 2^e2, 1/2 <= |m| < 1 */
  int lead = e2 - 1;                   /* exponent of the leading bit */
  if (lead < emin) lead = emin;        /* subnormal range: fixed spacing */
  const double quantum = ldexp(1.0, lead - (p - 1));
  const double r = nearbyint(x / quantum) * quantum;   /* default rounding mode: ties to even */
  const double max_finite = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
  if (fabs(r) > max_finite) return copysign(INFINITY, x);
  return r;
}

typedef struct {
  const float *x, *wq, *wk, *wv;
  float *kc, *vc;
  const int32_t* past_len;
  int B, T, D, Hq, Hkv, d, cap, dtype;
  const int32_t* t_index;
  int n_t;
  double* q;      /* [B][n_t][Hq][d] */
  double* out;    /* [B][n_t][Hq][d] */
  int n_items;
  int next;       /* shared work counter */
  int phase;      /* 0: K/V projection + append, 1: Q projection, 2: attention */
  int err;
} Step;

enum { kTokBlock = 16 };

/* y[j] = sum_k x[k] w[k][c0 + j] for j < n, each sum taken over k in index order (the loop over j
   is inside the loop over k only so that the weight rows are read in memory order) */
static void project_row(const float* x, const float* w, int D, int ldw, int c0, int n, double* y) {
  for (int j = 0; j < n; ++j) y[j] = 0.0;
  for (int k = 0; k < D; ++k) {
    const double xk = (double)x[k];
    const float* wk = w + (size_t)k * ldw + c0;
    for (int j = 0; j < n; ++j) y[j] += xk * (double)wk[j];
  }
}

/* phase 0, item (b, t): the new token's K and V rows, rounded and appended */
static void kv_item(Step* st, int it, double* tmp) {
  const int b = it / st->T, t = it % st->T;
  const int Hkv = st->Hkv, d = st->d, D = st->D;
  const float* xr = st->x + ((size_t)b * st->T + t) * D;
  const size_t row = (size_t)st->past_len[b] + t;
  for (int which = 0; which < 2; ++which) {
    const float* w = which ? st->wv : st->wk;
    float* cache = which ? st->vc : st->kc;
    project_row(xr, w, D, Hkv * d, 0, Hkv * d, tmp);
    for (int g = 0; g < Hkv; ++g)
      for (int i = 0; i < d; ++i)
        cache[(((size_t)b * Hkv + g) * st->cap + row) * d + i] = (float)oref_round(tmp[g * d + i], st->dtype);
  }
}

/* phase 1, item (b, r): the query of token t_index[r], every head, unrounded */
static void q_item(Step* st, int it) {
  const int b = it / st->n_t, r = it % st->n_t;
  const int t = st->t_index[r];
  const float* xr = st->x + ((size_t)b * st->T + t) * st->D;
  project_row(xr, st->wq, st->D, st->Hq * st->d, 0, st->Hq * st->d, st->q + ((size_t)b * st->n_t + r) * st->Hq * st->d);
}

/* phase 2, item (b, g, block of query tokens): attention of every head of group g for those tokens */
static int attn_item(Step* st, int it) {
  const int nblk = (st->n_t + kTokBlock - 1) / kTokBlock;
  const int b = it / (st->Hkv * nblk), g = (it / nblk) % st->Hkv, blk = it % nblk;
  const int G = st->Hq / st->Hkv, d = st->d;
  const int r0 = blk * kTokBlock, r1 = r0 + kTokBlock < st->n_t ? r0 + kTokBlock : st->n_t;
  const int L = st->past_len[b];
  int nkeys = 0;                                   /* keys seen by the block's last query */
  for (int r = r0; r < r1; ++r)
    if (L + st->t_index[r] + 1 > nkeys) nkeys = L + st->t_index[r] + 1;
  const int nrows = (r1 - r0) * G;
  double* s = (double*)malloc((size_t)nrows * nkeys * sizeof(double));
  double* m = (double*)malloc((size_t)nrows * 2 * sizeof(double));
  if (!s || !m) {
    free(s);
    free(m);
    return 1;
  }
  double* l = m + nrows;
  const float* K = st->kc + ((size_t)b * st->Hkv + g) * st->cap * d;
  const float* V = st->vc + ((size_t)b * st->Hkv + g) * st->cap * d;
  const double sqrt_d = sqrt((double)d);
  /* scores s = q·k / √d of every visible key, row max */
  for (int row = 0; row < nrows; ++row) m[row] = -INFINITY;
  for (int j = 0; j < nkeys; ++j) {
    const float* kj = K + (size_t)j * d;
    for (int row = 0; row < nrows; ++row) {
      const int r = r0 + row / G, h = g * G + row % G;
      if (j > L + st->t_index[r]) continue;        /* causal: a later key */
      const double* q = st->q + (((size_t)b * st->n_t + r) * st->Hq + h) * d;
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += q[i] * (double)kj[i];
      const double v = dot / sqrt_d;
      s[(size_t)row * nkeys + j] = v;
      if (v > m[row]) m[row] = v;
    }
  }
  /* weights exp(s - max), their sum, and the weighted sum of value rows, keys in order */
  for (int row = 0; row < nrows; ++row) {
    const int r = r0 + row / G, h = g * G + row % G;
    double* o = st->out + (((size_t)b * st->n_t + r) * st->Hq + h) * d;
    memset(o, 0, (size_t)d * sizeof(double));
    l[row] = 0.0;
  }
  for (int j = 0; j < nkeys; ++j) {
    const float* vj = V + (size_t)j * d;
    for (int row = 0; row < nrows; ++row) {
      const int r = r0 + row / G, h = g * G + row % G;
      if (j > L + st->t_index[r]) continue;
      const double w = exp(s[(size_t)row * nkeys + j] - m[row]);
      l[row] += w;
      double* o = st->out + (((size_t)b * st->n_t + r) * st->Hq + h) * d;
      for (int i = 0; i < d; ++i) o[i] += w * (double)vj[i];
    }
  }
  for (int row = 0; row < nrows; ++row) {
    const int r = r0 + row / G, h = g * G + row % G;
    double* o = st->out + (((size_t)b * st->n_t + r) * st->Hq + h) * d;
    for (int i = 0; i < d; ++i) o[i] /= l[row];
  }
  free(s);
  free(m);
  return 0;
}

static void* worker(void* arg) {
  Step* st = (Step*)arg;
  double* tmp = (double*)malloc((size_t)st->Hkv * st->d * sizeof(double));
  if (!tmp) {
    __atomic_store_n(&st->err, 1, __ATOMIC_SEQ_CST);
    return NULL;
  }
  for (;;) {
    const int it = __atomic_fetch_add(&st->next, 1, __ATOMIC_SEQ_CST);
    if (it >= st->n_items) break;
    if (st->phase == 0) kv_item(st, it, tmp);
    else if (st->phase == 1) q_item(st, it);
    else if (attn_item(st, it)) __atomic_store_n(&st->err, 1, __ATOMIC_SEQ_CST);
  }
  free(tmp);
  return NULL;
}

static int run_phase(Step* st, int phase, int n_items, int n_threads) {
  st->phase = phase;
  st->n_items = n_items;
  st->next = 0;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  pthread_t th[256];
  int started = 0;
  for (; started < n_threads - 1; ++started)
    if (pthread_create(&th[started], NULL, worker, st) != 0) break;
  worker(st);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  return st->err;
}

/* One layer step (see the header). Returns 0, or 1 on a bad argument or a failed allocation. */
int oref_layer_step(const float* x, const float* wq, const float* wk, const float* wv, float* kc, float* vc,
                    const int32_t* past_len, int B, int T, int D, int Hq, int Hkv, int d, int cap, int dtype,
                    const int32_t* t_index, int n_t, double* out, int n_threads) {
  if (B <= 0 || T < 0 || D <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || dtype < 0 || dtype > 2 || n_t < 0) return 1;
  for (int b = 0; b < B; ++b)
    if (past_len[b] < 0 || past_len[b] + T > cap) return 1;
  for (int r = 0; r < n_t; ++r)
    if (t_index[r] < 0 || t_index[r] >= T) return 1;
  Step st;
  memset(&st, 0, sizeof(st));
  st.x = x;
  st.wq = wq;
  st.wk = wk;
  st.wv = wv;
  st.kc = kc;
  st.vc = vc;
  st.past_len = past_len;
  st.B = B;
  st.T = T;
  st.D = D;
  st.Hq = Hq;
  st.Hkv = Hkv;
  st.d = d;
  st.cap = cap;
  st.dtype = dtype;
  st.t_index = t_index;
  st.n_t = n_t;
  st.out = out;
  st.q = (double*)malloc(((size_t)B * n_t * Hq * d + 1) * sizeof(double));
  if (!st.q) return 1;
  int err = run_phase(&st, 0, B * T, n_threads);
  if (!err) err = run_phase(&st, 1, B * n_t, n_threads);
  if (!err) err = run_phase(&st, 2, B * Hkv * ((n_t + kTokBlock - 1) / kTokBlock), n_threads);
  free(st.q);
  return err;
}
