/*
 * lfattn oracle: TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, double-precision CPU implementation of the forward pass of
 * band + global sparse self-attention.  It exists only to check the GPU
 * library.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may load or call it; the GPU library never links or loads it,
 * and it shares no code, header, table or constant with that library.
 *
 * What is computed, for one (batch b, head h, query row i), all in double:
 *
 *   S_i = { 0, 1, ..., N-1 }                                   if i is global
 *   S_i = { i + d*k : -hw <= k <= hw, 0 <= i + d*k < N }  u  G  otherwise
 *   z_j = scale * sum_c Q[i,c] * K[j,c]                          for j in S_i
 *   O_i = sum_{j in S_i} exp(z_j - max z) V_j / sum_{j in S_i} exp(z_j - max z)
 *
 * with hw = floor(window / 2), d = the head's dilation and G the set of global
 * token positions.  The general form (lfo_attention_ex) also takes
 *   - a set G_b per batch element b (G above is then G_b of the row's batch);
 *   - separate projections Qg, Kg, Vg: a global row i takes
 *       z_j = scale * sum_c Qg[i,c] * Kg[j,c],  O_i = sum_j softmax(z)_j Vg_j
 *     over all N keys, while every other row keeps Q, K, V, for its band and
 *     for the global keys alike.
 * A causal variant keeps only the band's left half and the row itself,
 *   S_i = { i + d*k : -hw <= k <= 0, i + d*k >= 0 }
 * (no global tokens).  The chunked variant (GMAT's C x k chunked
 * self-attention with M memory tokens) replaces the band by the row's chunk:
 *   S_i = { 0, ..., N-1 }                                      if i < M
 *   S_i = { 0, ..., M-1 }  u  { c0, ..., min(c0 + C, N) - 1 }    otherwise,
 *   c0 = M + C * floor((i - M) / C).
 * Sources:
 *   - attention itself, softmax(Q K^T / sqrt(d_k)) V: "Unlimiformer:
 *     Long-Range Transformers with Unlimited Length Input", section 2.3, Eq. (1);
 *     the default scale is 1/sqrt(D) from that equation.
 *   - subtracting max z before exp: same section, footnote 3 (softmax does not
 *     change when one constant is added to all of its inputs).
 *   - the band: Ultralytics glossary "Longformer", section on how the attention
 *     works, sliding-window bullet (256 neighbours on each side), and the
 *     mask-counting sample in that section, whose predicate is
 *     |pos_i - pos_j| <= window // 2 (inclusive, floor).
 *   - dilation: same section, dilated sliding-window bullet (attended positions
 *     are spaced out so a head sees further at the same cost).  The page gives
 *     no formula; the reading used here keeps the 2*hw+1 offsets and spaces
 *     them d apart: keys i + d*k.
 *   - global tokens: same section, global-attention bullet (chosen tokens attend
 *     to every position and every position attends to them); the sample sets
 *     row 0 and column 0 of the boolean mask, so a global key that is already
 *     inside a row's band is counted once (set union).
 *   - separate projections: same bullet (global attention has its own query,
 *     key and value projections).  The page does not say which scores they
 *     enter; the reading taken is that they are the global rows' own attention
 *     (a global query over every key), and that the other rows score the global
 *     keys with the ordinary projections, as part of their own attention.
 *   - one global set per batch element: the page's closing paragraph (the
 *     Hugging Face implementation takes the global tokens as a
 *     global_attention_mask input, one mask row per sequence of the batch).
 *   - causal band: the dilated-window bullet's use case, a character-level
 *     language model, predicts each character from the ones before it; the
 *     page gives no causal rule, and the reading taken keeps the same offsets
 *     restricted to k <= 0.
 *   - chunked self-attention: "GMAT: Global Memory Augmentation for
 *     Transformers", section "Chunked self-attention": the main sequence is cut
 *     into contiguous chunks of length C, each token attends to the tokens of
 *     its chunk and to the memory, not to other chunks (the last chunk may be
 *     shorter when the length is not a multiple of C: a reading, the page
 *     takes length C*k).
 *   - memory tokens: "GMAT: Global Memory Augmentation for Transformers",
 *     section "Global Memory": M memory tokens are prefixed; they attend to all
 *     M+L positions, and main tokens attend to all memory tokens plus a sparse
 *     pattern over the main sequence.  With a band as the sparse pattern this is
 *     exactly the set above with G = {0, ..., M-1}.
 *
 * Inputs are float (fp32 data, or bf16 data already widened to fp32 exactly);
 * every product and sum is formed in double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LFO_OK 0
#define LFO_EINVAL (-1)
#define LFO_ENOMEM (-2)

/* Band half-width: the page's sample compares |i - j| with window // 2. */
static int64_t half_width(int window) { return (int64_t)window / 2; }

static int is_global(const int* glob, int n_glob, int i) {
  for (int t = 0; t < n_glob; ++t)
    if (glob[t] == i) return 1;
  return 0;
}

static int cmp_int(const void* a, const void* b) {
  int x = *(const int*)a, y = *(const int*)b;
  return (x > y) - (x < y);
}

static int check_globals(int N, const int* glob, int n_glob) {
  if (n_glob < 0 || (n_glob > 0 && glob == NULL)) return 0;
  for (int t = 0; t < n_glob; ++t)
    if (glob[t] < 0 || glob[t] >= N) return 0;
  return 1;
}

/*
 * The allowed key set S_i of query row i, written to keys[] in increasing
 * order without repeats (capacity: N + n_glob ints).  Returns |S_i|, or
 * LFO_EINVAL on bad arguments.  Sources: the Longformer glossary page's
 * sliding-window, dilated-window and global-attention bullets and its mask
 * sample; the GMAT page's "Global Memory" section (see the file header).
 */
int64_t lfo_allowed_set_ex(int N, int window, int dilation, int causal, const int* glob,
                           int n_glob, int i, int* keys) {
  if (N <= 0 || window < 0 || dilation < 1 || i < 0 || i >= N || keys == NULL)
    return LFO_EINVAL;
  if (!check_globals(N, glob, n_glob)) return LFO_EINVAL;
  if (causal && n_glob > 0) return LFO_EINVAL; /* the causal band has no global tokens */

  if (is_global(glob, n_glob, i)) {
    /* A global row attends to every position. */
    for (int j = 0; j < N; ++j) keys[j] = j;
    return N;
  }

  const int64_t hw = half_width(window);
  const int64_t d = dilation;
  int64_t n = 0;
  /* Only offsets k with 0 <= i + d*k < N can contribute; the loop visits
   * exactly those inside [-hw, hw] and checks the range again. */
  int64_t k_lo = -((int64_t)i / d);
  int64_t k_hi = ((int64_t)(N - 1) - i) / d;
  if (k_lo < -hw) k_lo = -hw;
  if (k_hi > hw) k_hi = hw;
  if (causal && k_hi > 0) k_hi = 0; /* causal: the row and the keys before it */
  for (int64_t k = k_lo; k <= k_hi; ++k) {
    int64_t j = (int64_t)i + d * k;
    if (j >= 0 && j < N) keys[n++] = (int)j;
  }
  /* Every row also attends to every global token. */
  for (int t = 0; t < n_glob; ++t) keys[n++] = glob[t];

  /* Set union: sort, then drop repeats. */
  qsort(keys, (size_t)n, sizeof(int), cmp_int);
  int64_t u = 0;
  for (int64_t t = 0; t < n; ++t)
    if (u == 0 || keys[u - 1] != keys[t]) keys[u++] = keys[t];
  return u;
}

/*
 * The allowed key set of row i under C x k chunked attention with M memory
 * tokens (positions 0..M-1; the chunks start at M), in increasing order.
 * Returns |S_i| or LFO_EINVAL.  Source: the GMAT page, sections "Global
 * Memory" and "Chunked self-attention" (see the file header).
 */
int64_t lfo_allowed_set_chunked(int N, int chunk, int n_memory, int i, int* keys) {
  if (N <= 0 || chunk < 1 || n_memory < 0 || n_memory > N || i < 0 || i >= N || !keys)
    return LFO_EINVAL;
  int64_t n = 0;
  if (i < n_memory) {
    /* A memory token attends to all M + L positions. */
    for (int j = 0; j < N; ++j) keys[n++] = j;
    return n;
  }
  /* The memory first (all of it), then the row's chunk. */
  for (int j = 0; j < n_memory; ++j) keys[n++] = j;
  const int64_t c0 = n_memory + (int64_t)chunk * ((i - n_memory) / chunk);
  const int64_t c1 = c0 + chunk < N ? c0 + chunk : N;
  for (int64_t j = c0; j < c1; ++j) keys[n++] = (int)j;
  return n;
}

/* The symmetric band (see lfo_allowed_set_ex). */
int64_t lfo_allowed_set(int N, int window, int dilation, const int* glob, int n_glob, int i,
                        int* keys) {
  return lfo_allowed_set_ex(N, window, dilation, 0, glob, n_glob, i, keys);
}

/*
 * Total number of scored (query, key) pairs, summed over B batches, H heads
 * and N rows, by building every S_i explicitly.  dilation: H entries, or NULL
 * for all 1.  This is the quantity the Longformer glossary page counts with
 * mask.sum() in its sample.  Returns the count, or LFO_EINVAL / LFO_ENOMEM.
 */
int64_t lfo_count_pairs_ex(int B, int H, int N, int window, const int* dilation, int causal,
                           const int* glob, int n_glob) {
  if (B <= 0 || H <= 0 || N <= 0 || window < 0) return LFO_EINVAL;
  if (!check_globals(N, glob, n_glob)) return LFO_EINVAL;
  int* keys = (int*)malloc(sizeof(int) * ((size_t)N + (size_t)n_glob + 1));
  if (!keys) return LFO_ENOMEM;
  int64_t total = 0;
  for (int h = 0; h < H; ++h) {
    int d = dilation ? dilation[h] : 1;
    if (d < 1) { free(keys); return LFO_EINVAL; }
    int64_t per_head = 0;
    for (int i = 0; i < N; ++i) {
      int64_t n = lfo_allowed_set_ex(N, window, d, causal, glob, n_glob, i, keys);
      if (n < 0) { free(keys); return n; }
      per_head += n;
    }
    total += per_head * B; /* the pattern does not depend on the batch */
  }
  free(keys);
  return total;
}

int64_t lfo_count_pairs(int B, int H, int N, int window, const int* dilation, const int* glob,
                        int n_glob) {
  return lfo_count_pairs_ex(B, H, N, window, dilation, 0, glob, n_glob);
}

/* ---- attention values ---------------------------------------------------- */

typedef struct {
  const float *Q, *K, *V;
  const float *Qg, *Kg, *Vg; /* the global rows' projections (= Q, K, V if none) */
  double* O;
  int B, H, N, D, window, n_glob, causal;
  int chunk, n_memory; /* chunk > 0: chunked attention (window, glob unused) */
  const int* dilation;
  const int* glob;
  const int* goff; /* per-batch lists: G_b = glob[goff[b] .. goff[b+1]), or NULL */
  double scale;
  const int64_t* rows; /* flattened (b*H + h)*N + i, or NULL for all rows */
  int64_t n_rows;
  int64_t first, last; /* this worker's share of the row list */
  int status;
} lfo_job;

/*
 * One query row: Eq. (1) of the Unlimiformer page restricted to S_i, with the
 * max subtracted first (footnote 3 of that section).  Two passes over S_i:
 * scores and their maximum, then weights, their sum and the weighted sum of V.
 */
static int one_row(const lfo_job* jb, int64_t flat, int* keys, double* z,
                   double* acc, double* out) {
  const int N = jb->N, D = jb->D;
  const int64_t bh = flat / N;
  const int i = (int)(flat % N);
  const int h = (int)(bh % jb->H);
  const int b = (int)(bh / jb->H);
  const int d = jb->dilation ? jb->dilation[h] : 1;
  /* The global set of this row's batch element. */
  const int* gl = jb->goff ? jb->glob + jb->goff[b] : jb->glob;
  const int ng = jb->goff ? jb->goff[b + 1] - jb->goff[b] : jb->n_glob;
  /* A global row takes its own projections. */
  const int grow = jb->chunk > 0 ? i < jb->n_memory : is_global(gl, ng, i);
  const float* q = (grow ? jb->Qg : jb->Q) + (size_t)flat * D;
  const float* Kbh = (grow ? jb->Kg : jb->K) + (size_t)bh * N * D;
  const float* Vbh = (grow ? jb->Vg : jb->V) + (size_t)bh * N * D;

  int64_t n = jb->chunk > 0 ? lfo_allowed_set_chunked(N, jb->chunk, jb->n_memory, i, keys)
                            : lfo_allowed_set_ex(N, jb->window, d, jb->causal, gl, ng, i, keys);
  if (n <= 0) return LFO_EINVAL; /* never empty: k = 0 gives j = i */

  double zmax = -INFINITY;
  for (int64_t t = 0; t < n; ++t) {
    const float* kr = Kbh + (size_t)keys[t] * D;
    double s = 0.0;
    for (int c = 0; c < D; ++c) s += (double)q[c] * (double)kr[c];
    z[t] = jb->scale * s;
    if (z[t] > zmax) zmax = z[t];
  }
  double den = 0.0;
  for (int c = 0; c < D; ++c) acc[c] = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    double e = exp(z[t] - zmax);
    den += e;
    const float* vr = Vbh + (size_t)keys[t] * D;
    for (int c = 0; c < D; ++c) acc[c] += e * (double)vr[c];
  }
  for (int c = 0; c < D; ++c) out[c] = acc[c] / den;
  return LFO_OK;
}

static void* worker(void* arg) {
  lfo_job* jb = (lfo_job*)arg;
  const int N = jb->N, D = jb->D;
  int* keys = (int*)malloc(sizeof(int) * ((size_t)N + (size_t)jb->n_glob + 1));
  double* z = (double*)malloc(sizeof(double) * ((size_t)N + (size_t)jb->n_glob + 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)D);
  if (!keys || !z || !acc) {
    jb->status = LFO_ENOMEM;
  } else {
    for (int64_t r = jb->first; r < jb->last; ++r) {
      int64_t flat = jb->rows ? jb->rows[r] : r;
      int st = one_row(jb, flat, keys, z, acc, jb->O + (size_t)r * D);
      if (st != LFO_OK) { jb->status = st; break; }
    }
  }
  free(keys); free(z); free(acc);
  return NULL;
}

static int run_jobs(const lfo_job* base, int nthreads);

/*
 * Attention output for a list of rows, general form.  Q, K, V: [B, H, N, D]
 * row-major floats; Qg, Kg, Vg: the same shape, the global rows' projections,
 * each NULL to use Q, K or V.  goff: NULL for one global set glob[0..n_glob)
 * shared by every batch element, or B+1 offsets with G_b = glob[goff[b] ..
 * goff[b+1]) (then n_glob = goff[B]).  rows: flattened indices
 * (b*H + h)*N + i, n_rows of them, or NULL with n_rows = B*H*N for every row.
 * O: n_rows x D doubles, in the order of rows.  scale <= 0 selects 1/sqrt(D).
 * nthreads >= 1 workers split the row list into contiguous ranges.  Returns
 * LFO_OK or a negative error.
 */
int lfo_attention_ex(const float* Q, const float* K, const float* V,
                     const float* Qg, const float* Kg, const float* Vg, double* O,
                     int B, int H, int N, int D, int window, const int* dilation, int causal,
                     const int* glob, const int* goff, int n_glob, double scale,
                     const int64_t* rows, int64_t n_rows, int nthreads) {
  if (!Q || !K || !V || !O || B <= 0 || H <= 0 || N <= 0 || D <= 0 ||
      window < 0 || n_rows < 0)
    return LFO_EINVAL;
  if (goff) {
    if (goff[0] != 0 || goff[B] != n_glob) return LFO_EINVAL;
    for (int b = 0; b < B; ++b)
      if (goff[b + 1] < goff[b]) return LFO_EINVAL;
  }
  if (!check_globals(N, glob, n_glob)) return LFO_EINVAL;
  if (causal && n_glob > 0) return LFO_EINVAL;
  if (dilation)
    for (int h = 0; h < H; ++h)
      if (dilation[h] < 1) return LFO_EINVAL;
  const int64_t total = (int64_t)B * H * N;
  if (!rows && n_rows != total) return LFO_EINVAL;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= total) return LFO_EINVAL;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  lfo_job base;
  memset(&base, 0, sizeof(base));
  base.Q = Q; base.K = K; base.V = V; base.O = O;
  base.Qg = Qg ? Qg : Q; base.Kg = Kg ? Kg : K; base.Vg = Vg ? Vg : V;
  base.B = B; base.H = H; base.N = N; base.D = D; base.window = window;
  base.dilation = dilation; base.glob = glob; base.n_glob = n_glob; base.goff = goff;
  base.causal = causal;
  base.scale = scale; base.rows = rows; base.n_rows = n_rows;
  return run_jobs(&base, nthreads);
}

/* Split the row list of `base` over nthreads workers and run them. */
static int run_jobs(const lfo_job* base, int nthreads) {
  const int64_t n_rows = base->n_rows;
  if (nthreads < 1) nthreads = 1;
  if (n_rows == 0) return LFO_OK;
  if ((int64_t)nthreads > n_rows) nthreads = (int)n_rows;
  lfo_job* jobs = (lfo_job*)calloc((size_t)nthreads, sizeof(lfo_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !tids) { free(jobs); free(tids); return LFO_ENOMEM; }
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = *base;
    jobs[t].first = n_rows * t / nthreads;
    jobs[t].last = n_rows * (t + 1) / nthreads;
    jobs[t].status = LFO_OK;
  }
  char* created = (char*)calloc((size_t)nthreads, 1);
  if (!created) { free(jobs); free(tids); return LFO_ENOMEM; }
  for (int t = 1; t < nthreads; ++t)
    created[t] = (char)(pthread_create(&tids[t], NULL, worker, &jobs[t]) == 0);
  worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) {
    if (created[t]) pthread_join(tids[t], NULL);
    else worker(&jobs[t]); /* no thread could be started: do its share here */
  }
  int st = LFO_OK;
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status != LFO_OK) st = jobs[t].status;
  free(jobs); free(tids); free(created);
  return st;
}

/* One global set for every batch element, the ordinary projections. */
int lfo_attention(const float* Q, const float* K, const float* V, double* O,
                  int B, int H, int N, int D, int window, const int* dilation,
                  const int* glob, int n_glob, double scale,
                  const int64_t* rows, int64_t n_rows, int nthreads) {
  return lfo_attention_ex(Q, K, V, NULL, NULL, NULL, O, B, H, N, D, window, dilation, 0, glob,
                          NULL, n_glob, scale, rows, n_rows, nthreads);
}

/*
 * Attention output under C x k chunked attention with M memory tokens (the
 * memory rows use Qg, Kg, Vg when given, as global rows).  Arguments as
 * lfo_attention_ex; chunk >= 1, 0 <= n_memory <= N.
 */
int lfo_attention_chunked(const float* Q, const float* K, const float* V,
                          const float* Qg, const float* Kg, const float* Vg, double* O,
                          int B, int H, int N, int D, int chunk, int n_memory, double scale,
                          const int64_t* rows, int64_t n_rows, int nthreads) {
  if (!Q || !K || !V || !O || B <= 0 || H <= 0 || N <= 0 || D <= 0 || chunk < 1 ||
      n_memory < 0 || n_memory > N || n_rows < 0)
    return LFO_EINVAL;
  const int64_t total = (int64_t)B * H * N;
  if (!rows && n_rows != total) return LFO_EINVAL;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= total) return LFO_EINVAL;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  lfo_job base;
  memset(&base, 0, sizeof(base));
  base.Q = Q; base.K = K; base.V = V; base.O = O;
  base.Qg = Qg ? Qg : Q; base.Kg = Kg ? Kg : K; base.Vg = Vg ? Vg : V;
  base.B = B; base.H = H; base.N = N; base.D = D;
  base.chunk = chunk; base.n_memory = n_memory;
  base.scale = scale; base.rows = rows; base.n_rows = n_rows;
  return run_jobs(&base, nthreads);
}

/* ---- gradients ----------------------------------------------------------- */

/*
 * Gradients of the attention above with respect to Q, K and V, for an upstream
 * gradient dO (all [B, H, N, D]; outputs in double).  Pattern arguments as
 * lfo_attention_ex (ordinary projections only) and chunk/n_memory as
 * lfo_attention_chunked (chunk > 0 selects the chunked pattern).  For each row
 * i with key set S_i, P = softmax over S_i of z_j = scale * Q_i . K_j, and by
 * the chain rule through that softmax (Eq. (1) of the Unlimiformer page):
 *   dP_j   = dO_i . V_j
 *   Delta  = sum_{j in S_i} P_j dP_j            (= dO_i . O_i)
 *   dS_j   = P_j (dP_j - Delta)
 *   dQ_i  += scale * sum_j dS_j K_j
 *   dK_j  += scale * dS_j Q_i
 *   dV_j  += P_j dO_i
 * One worker per (batch, head) pair, so the K and V gradients need no locks.
 * With separate projections for the global rows (the reading of
 * lfo_attention_ex), a global row i takes Qg_i, Kg_j, Vg_j in place of Q_i,
 * K_j, V_j in all of the above, and its terms go to dQg_i, dKg_j, dVg_j.
 */
typedef struct {
  const float *Q, *K, *V, *dO;
  const float *Qg, *Kg, *Vg;  /* NULL: the global rows share Q, K, V */
  double *dQ, *dK, *dV;
  double *dQg, *dKg, *dVg;    /* used when Qg is not NULL */
  int B, H, N, D, window, causal, chunk, n_memory, n_glob;
  const int* dilation;
  const int* glob;
  const int* goff;
  double scale;
  int64_t first_bh, last_bh;
  int status;
} lfo_grad_job;

static void* grad_worker(void* arg) {
  lfo_grad_job* jb = (lfo_grad_job*)arg;
  const int N = jb->N, D = jb->D;
  int* keys = (int*)malloc(sizeof(int) * ((size_t)N + (size_t)jb->n_glob + 1));
  double* p = (double*)malloc(sizeof(double) * ((size_t)N + (size_t)jb->n_glob + 1));
  double* dp = (double*)malloc(sizeof(double) * ((size_t)N + (size_t)jb->n_glob + 1));
  if (!keys || !p || !dp) {
    jb->status = LFO_ENOMEM;
    free(keys); free(p); free(dp);
    return NULL;
  }
  for (int64_t bh = jb->first_bh; bh < jb->last_bh && jb->status == LFO_OK; ++bh) {
    const int h = (int)(bh % jb->H), b = (int)(bh / jb->H);
    const int d = jb->dilation ? jb->dilation[h] : 1;
    const int* gl = jb->goff ? jb->glob + jb->goff[b] : jb->glob;
    const int ng = jb->goff ? jb->goff[b + 1] - jb->goff[b] : jb->n_glob;
    const size_t off = (size_t)bh * N * D;
    const float* dOh = jb->dO + off;
    for (int i = 0; i < N; ++i) {
      int64_t n = jb->chunk > 0 ? lfo_allowed_set_chunked(N, jb->chunk, jb->n_memory, i, keys)
                                : lfo_allowed_set_ex(N, jb->window, d, jb->causal, gl, ng, i, keys);
      if (n <= 0) { jb->status = LFO_EINVAL; break; }
      /* The row's projections and gradient outputs. */
      const int own = jb->Qg != NULL &&
                      (jb->chunk > 0 ? i < jb->n_memory : is_global(gl, ng, i));
      const float *Qh = (own ? jb->Qg : jb->Q) + off, *Kh = (own ? jb->Kg : jb->K) + off;
      const float* Vh = (own ? jb->Vg : jb->V) + off;
      double *dQh = (own ? jb->dQg : jb->dQ) + off, *dKh = (own ? jb->dKg : jb->dK) + off;
      double* dVh = (own ? jb->dVg : jb->dV) + off;
      const float* q = Qh + (size_t)i * D;
      const float* g = dOh + (size_t)i * D;
      /* Softmax over S_i (max subtracted first). */
      double zmax = -INFINITY;
      for (int64_t t = 0; t < n; ++t) {
        const float* kr = Kh + (size_t)keys[t] * D;
        double s = 0.0;
        for (int c = 0; c < D; ++c) s += (double)q[c] * (double)kr[c];
        p[t] = jb->scale * s;
        if (p[t] > zmax) zmax = p[t];
      }
      double den = 0.0;
      for (int64_t t = 0; t < n; ++t) { p[t] = exp(p[t] - zmax); den += p[t]; }
      double delta = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        p[t] /= den;
        const float* vr = Vh + (size_t)keys[t] * D;
        double s = 0.0;
        for (int c = 0; c < D; ++c) s += (double)g[c] * (double)vr[c];
        dp[t] = s;
        delta += p[t] * s;
      }
      for (int64_t t = 0; t < n; ++t) {
        const int j = keys[t];
        const double ds = p[t] * (dp[t] - delta);
        const float* kr = Kh + (size_t)j * D;
        for (int c = 0; c < D; ++c) {
          dQh[(size_t)i * D + c] += jb->scale * ds * (double)kr[c];
          dKh[(size_t)j * D + c] += jb->scale * ds * (double)q[c];
          dVh[(size_t)j * D + c] += p[t] * (double)g[c];
        }
      }
    }
  }
  free(keys); free(p); free(dp);
  return NULL;
}

/*
 * Gradients dQ, dK, dV (doubles, [B, H, N, D], overwritten) for the upstream
 * gradient dO.  window, dilation, causal, glob/goff/n_glob as
 * lfo_attention_ex; chunk > 0 selects chunked attention with n_memory memory
 * tokens instead.  Returns LFO_OK or a negative error.
 */
/*
 * As lfo_attention_grad, with separate projections Qg, Kg, Vg for the global
 * rows (the memory rows when chunk > 0) and their gradients dQg, dKg, dVg
 * (doubles, [B, H, N, D], overwritten).  Qg, Kg, Vg all NULL (and dQg, dKg,
 * dVg ignored): the shared-projection gradients of lfo_attention_grad.
 */
int lfo_attention_grad_ex(const float* Q, const float* K, const float* V, const float* Qg,
                          const float* Kg, const float* Vg, const float* dO, double* dQ,
                          double* dK, double* dV, double* dQg, double* dKg, double* dVg, int B,
                          int H, int N, int D, int window, const int* dilation, int causal,
                          const int* glob, const int* goff, int n_glob, int chunk, int n_memory,
                          double scale, int nthreads) {
  const int proj = Qg != NULL;
  if (proj && (!Kg || !Vg || !dQg || !dKg || !dVg)) return LFO_EINVAL;
  if (!proj && (Kg || Vg)) return LFO_EINVAL;
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV || B <= 0 || H <= 0 || N <= 0 || D <= 0 ||
      window < 0 || chunk < 0 || n_memory < 0 || n_memory > N)
    return LFO_EINVAL;
  if (goff) {
    if (goff[0] != 0 || goff[B] != n_glob) return LFO_EINVAL;
    for (int b = 0; b < B; ++b)
      if (goff[b + 1] < goff[b]) return LFO_EINVAL;
  }
  if (!check_globals(N, glob, n_glob)) return LFO_EINVAL;
  if (causal && n_glob > 0) return LFO_EINVAL;
  if (dilation)
    for (int h = 0; h < H; ++h)
      if (dilation[h] < 1) return LFO_EINVAL;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  const size_t total = (size_t)B * H * N * D;
  memset(dQ, 0, total * sizeof(double));
  memset(dK, 0, total * sizeof(double));
  memset(dV, 0, total * sizeof(double));
  if (proj) {
    memset(dQg, 0, total * sizeof(double));
    memset(dKg, 0, total * sizeof(double));
    memset(dVg, 0, total * sizeof(double));
  }
  const int64_t n_bh = (int64_t)B * H;
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > n_bh) nthreads = (int)n_bh;
  lfo_grad_job* jobs = (lfo_grad_job*)calloc((size_t)nthreads, sizeof(lfo_grad_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  char* created = (char*)calloc((size_t)nthreads, 1);
  if (!jobs || !tids || !created) { free(jobs); free(tids); free(created); return LFO_ENOMEM; }
  for (int t = 0; t < nthreads; ++t) {
    lfo_grad_job* jb = &jobs[t];
    jb->Q = Q; jb->K = K; jb->V = V; jb->dO = dO; jb->dQ = dQ; jb->dK = dK; jb->dV = dV;
    jb->Qg = proj ? Qg : NULL; jb->Kg = Kg; jb->Vg = Vg;
    jb->dQg = dQg; jb->dKg = dKg; jb->dVg = dVg;
    jb->B = B; jb->H = H; jb->N = N; jb->D = D; jb->window = window; jb->causal = causal;
    jb->chunk = chunk; jb->n_memory = n_memory; jb->n_glob = n_glob;
    jb->dilation = dilation; jb->glob = glob; jb->goff = goff; jb->scale = scale;
    jb->first_bh = n_bh * t / nthreads;
    jb->last_bh = n_bh * (t + 1) / nthreads;
    jb->status = LFO_OK;
  }
  for (int t = 1; t < nthreads; ++t)
    created[t] = (char)(pthread_create(&tids[t], NULL, grad_worker, &jobs[t]) == 0);
  grad_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) {
    if (created[t]) pthread_join(tids[t], NULL);
    else grad_worker(&jobs[t]);
  }
  int st = LFO_OK;
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status != LFO_OK) st = jobs[t].status;
  free(jobs); free(tids); free(created);
  return st;
}

int lfo_attention_grad(const float* Q, const float* K, const float* V, const float* dO,
                       double* dQ, double* dK, double* dV, int B, int H, int N, int D,
                       int window, const int* dilation, int causal, const int* glob,
                       const int* goff, int n_glob, int chunk, int n_memory, double scale,
                       int nthreads) {
  return lfo_attention_grad_ex(Q, K, V, NULL, NULL, NULL, dO, dQ, dK, dV, NULL, NULL, NULL, B, H,
                               N, D, window, dilation, causal, glob, goff, n_glob, chunk,
                               n_memory, scale, nthreads);
}

/*
 * Per-row log-sum-exp of the scaled scores, lse_i = log sum_{j in S_i}
 * exp(scale * Q_i . K_j) (natural log, the max taken out first), for every
 * row, [B, H, N] doubles.  Pattern arguments as lfo_attention_grad.
 */
int lfo_row_lse(const float* Q, const float* K, double* lse, int B, int H, int N, int D,
                int window, const int* dilation, int causal, const int* glob, const int* goff,
                int n_glob, int chunk, int n_memory, double scale) {
  if (!Q || !K || !lse || B <= 0 || H <= 0 || N <= 0 || D <= 0 || window < 0 || chunk < 0 ||
      n_memory < 0 || n_memory > N)
    return LFO_EINVAL;
  if (!check_globals(N, glob, n_glob)) return LFO_EINVAL;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  int* keys = (int*)malloc(sizeof(int) * ((size_t)N + (size_t)n_glob + 1));
  double* z = (double*)malloc(sizeof(double) * ((size_t)N + (size_t)n_glob + 1));
  if (!keys || !z) { free(keys); free(z); return LFO_ENOMEM; }
  int st = LFO_OK;
  for (int64_t bh = 0; bh < (int64_t)B * H && st == LFO_OK; ++bh) {
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int d = dilation ? dilation[h] : 1;
    const int* gl = goff ? glob + goff[b] : glob;
    const int ng = goff ? goff[b + 1] - goff[b] : n_glob;
    for (int i = 0; i < N; ++i) {
      int64_t n = chunk > 0 ? lfo_allowed_set_chunked(N, chunk, n_memory, i, keys)
                            : lfo_allowed_set_ex(N, window, d, causal, gl, ng, i, keys);
      if (n <= 0) { st = LFO_EINVAL; break; }
      const float* q = Q + ((size_t)bh * N + i) * D;
      double zmax = -INFINITY;
      for (int64_t t = 0; t < n; ++t) {
        const float* kr = K + ((size_t)bh * N + keys[t]) * D;
        double s = 0.0;
        for (int c = 0; c < D; ++c) s += (double)q[c] * (double)kr[c];
        z[t] = scale * s;
        if (z[t] > zmax) zmax = z[t];
      }
      double sum = 0.0;
      for (int64_t t = 0; t < n; ++t) sum += exp(z[t] - zmax);
      lse[(size_t)bh * N + i] = zmax + log(sum);
    }
  }
  free(keys); free(z);
  return st;
}
