/*
 * ssd_oracle.c -- plain fp64 CPU oracle for the Mamba-2 SSD (state space
 * duality) layer: the sequential recurrence and its hand-derived reverse
 * adjoint.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; it exists so that the tests, the package's smoke check and
 * the CPU-baseline leg of the benchmark can compare the GPU library against
 * an independent, obviously-correct computation.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * What is computed (page "Deterministic bwd kernel for mamba2", state-spaces/
 * mamba PR 827, whose per-kernel table lists the backward of this layer; the
 * pages print no equations, so the recurrence below is the plain SSD
 * recurrence that the kernels named there -- chunk_cumsum, chunk_state,
 * state passing, chunk_scan -- evaluate in chunked form):
 *
 *   per batch row b and head h, for every sequence s starting at t0
 *   (a start is t == 0 or seq_idx[b,t] != seq_idx[b,t-1]):
 *       h_{t0-1} = h0[s]   (zero when no initial states are given)
 *       a_t  = dt_t * A_h
 *       h_t  = exp(a_t) * h_{t-1} + dt_t * x_t (outer) B_t     (P x N)
 *       y_t  = h_t C_t + D_h * x_t                              (P)
 *   The loss whose gradients are returned is  l = sum_t dy_t . y_t, plus
 *   <d_last[b], h_{L-1}>_F for every batch row b when d_last is given (the
 *   gradient that arrives for the state after a row's last position, which is
 *   what a later stretch of the same sequence hands back).
 *
 * Reverse adjoint, lambda_t = dl/dh_t, running t downwards:
 *       lambda_t = dy_t (outer) C_t + [t+1 in same sequence] exp(a_{t+1}) lambda_{t+1}
 *                  (+ d_last[b] at t = L-1)
 *       dC_t  += h_t^T dy_t                    (summed over the heads of a group)
 *       dx_t   = dt_t lambda_t B_t + D_h dy_t
 *       dB_t  += dt_t lambda_t^T x_t           (summed over the heads of a group)
 *       da_t   = exp(a_t) <lambda_t, h_{t-1}>_F
 *       ddt_t  = x_t^T lambda_t B_t + A_h da_t
 *       dA_h  += dt_t da_t ,  dD_h += dy_t . x_t
 *       d_h0[s] = exp(a_{t0}) lambda_{t0}
 *
 * Head h belongs to group h / (H/G).  Sequences are numbered in row-major
 * (b, t) order of their starts; with no seq_idx every batch row is one
 * sequence.
 *
 * Memory plan: the forward state is checkpointed every CKPT steps and each
 * block is recomputed during the reverse sweep.  Work items are (b, h) pairs
 * run on host threads; the per-head dB/dC contributions are kept per item and
 * summed over the heads of a group in ascending head order, and dA/dD are
 * summed over batch rows in ascending order, so the oracle itself is
 * deterministic.
 *
 * Parity pins for this file live in the CPU tests (quadratic masked form,
 * torch autograd of that form, finite differences, closed forms, a
 * hand-derived example).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CKPT 64

typedef struct {
  int64_t batch, seqlen, nheads, headdim, ngroups, dstate, nseqs;
} ssdo_shape;

enum { SSDO_OK = 0, SSDO_EINVAL = -1, SSDO_ENOMEM = -2 };

/* ---- sequence bookkeeping ------------------------------------------------ */

/* start[b*L+t] = 1 iff a sequence starts at (b, t); seq[b*L+t] = index of the
 * sequence that (b, t) belongs to.  Returns the number of sequences. */
static int64_t find_sequences(const ssdo_shape* s, const int32_t* seq_idx,
                              uint8_t* start, int64_t* seq) {
  int64_t n = 0;
  for (int64_t b = 0; b < s->batch; ++b) {
    for (int64_t t = 0; t < s->seqlen; ++t) {
      int64_t i = b * s->seqlen + t;
      int st = (t == 0);
      if (!st && seq_idx) st = (seq_idx[i] != seq_idx[i - 1]);
      start[i] = (uint8_t)st;
      if (st) ++n;
      seq[i] = n - 1;
    }
  }
  return n;
}

/* ---- problem context shared by the worker threads ------------------------ */

typedef struct {
  const ssdo_shape* s;
  const double *x, *dt, *A, *B, *C, *D, *h0, *dy, *d_last;
  const uint8_t* start;
  const int64_t* seq;
  int64_t head_lo, head_hi;
  /* forward outputs */
  double *y, *final_states;
  /* backward outputs */
  double *dx, *ddt, *dA_part, *dD_part, *d_h0;
  double *dB_item, *dC_item; /* per work item: (L, N) each */
  /* chunk exports */
  int64_t chunk;
  double *chunk_states, *chunk_dout;
  /* work distribution */
  int64_t n_items;
  int64_t next_item;
  pthread_mutex_t lock;
  int mode; /* 0 = forward, 1 = backward */
  int failed;
} ctx_t;

#define IDX_BLH(s, b, t, h) ((((b) * (s)->seqlen + (t)) * (s)->nheads) + (h))
#define IDX_X(s, b, t, h, p) (IDX_BLH(s, b, t, h) * (s)->headdim + (p))
#define IDX_BC(s, b, t, g, n) (((((b) * (s)->seqlen + (t)) * (s)->ngroups) + (g)) * (s)->dstate + (n))

/* One forward step for one (b, h): hcur = exp(a) * hprev + dt * x (outer) B. */
static void step_state(const ctx_t* c, int64_t b, int64_t t, int64_t h,
                       const double* hprev, double* hcur) {
  const ssdo_shape* s = c->s;
  const int64_t P = s->headdim, N = s->dstate;
  const int64_t g = h / (s->nheads / s->ngroups);
  const double dtv = c->dt[IDX_BLH(s, b, t, h)];
  const double decay = exp(dtv * c->A[h]);
  const double* xt = c->x + IDX_X(s, b, t, h, 0);
  const double* Bt = c->B + IDX_BC(s, b, t, g, 0);
  for (int64_t p = 0; p < P; ++p) {
    const double xs = dtv * xt[p];
    for (int64_t n = 0; n < N; ++n)
      hcur[p * N + n] = decay * hprev[p * N + n] + xs * Bt[n];
  }
}

/* The state that precedes position t: the running state, or the sequence's
 * initial state when t starts a sequence. */
static const double* prev_state(const ctx_t* c, int64_t b, int64_t t, int64_t h,
                                const double* running, const double* zeros) {
  const ssdo_shape* s = c->s;
  const int64_t i = b * s->seqlen + t;
  if (!c->start[i]) return running;
  if (!c->h0) return zeros;
  return c->h0 + ((c->seq[i] * s->nheads + h) * s->headdim) * s->dstate;
}

static void forward_item(ctx_t* c, int64_t b, int64_t h, double* hA, double* hB,
                         const double* zeros) {
  const ssdo_shape* s = c->s;
  const int64_t P = s->headdim, N = s->dstate, L = s->seqlen;
  const int64_t g = h / (s->nheads / s->ngroups);
  double* run = hA;
  double* nxt = hB;
  memset(run, 0, sizeof(double) * P * N);
  for (int64_t t = 0; t < L; ++t) {
    const double* hp = prev_state(c, b, t, h, run, zeros);
    step_state(c, b, t, h, hp, nxt);
    double* tmp = run; run = nxt; nxt = tmp;
    const double* Ct = c->C + IDX_BC(s, b, t, g, 0);
    const double* xt = c->x + IDX_X(s, b, t, h, 0);
    const double Dh = c->D ? c->D[h] : 0.0;
    for (int64_t p = 0; p < P; ++p) {
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) acc += run[p * N + n] * Ct[n];
      c->y[IDX_X(s, b, t, h, p)] = acc + Dh * xt[p];
    }
    const int last_of_seq = (t == L - 1) || c->start[b * L + t + 1];
    if (last_of_seq && c->final_states) {
      const int64_t sq = c->seq[b * L + t];
      memcpy(c->final_states + ((sq * s->nheads + h) * P) * N, run, sizeof(double) * P * N);
    }
  }
}

static void backward_item(ctx_t* c, int64_t item, int64_t b, int64_t h,
                          double* ckpt, double* hs, double* lam, double* lamB,
                          const double* zeros) {
  const ssdo_shape* s = c->s;
  const int64_t P = s->headdim, N = s->dstate, L = s->seqlen, PN = P * N;
  const int64_t g = h / (s->nheads / s->ngroups);
  const int64_t nblk = (L + CKPT - 1) / CKPT;
  const double Ah = c->A[h];
  const double Dh = c->D ? c->D[h] : 0.0;
  double* dBi = c->dB_item + item * L * N;
  double* dCi = c->dC_item + item * L * N;
  memset(dBi, 0, sizeof(double) * L * N);
  memset(dCi, 0, sizeof(double) * L * N);

  /* Forward sweep: ckpt[k] = state after position k*CKPT - 1 (zeros for k=0). */
  memset(ckpt, 0, sizeof(double) * PN);
  for (int64_t k = 0; k < nblk; ++k) {
    const int64_t t0 = k * CKPT, t1 = (t0 + CKPT < L) ? t0 + CKPT : L;
    const double* run = ckpt + k * PN;
    for (int64_t t = t0; t < t1; ++t) {
      double* out = hs + (t - t0) * PN;
      step_state(c, b, t, h, prev_state(c, b, t, h, run, zeros), out);
      run = out;
    }
    if (k + 1 < nblk) memcpy(ckpt + (k + 1) * PN, run, sizeof(double) * PN);
  }

  /* Reverse sweep.  lam holds the carry [t+1 same seq] exp(a_{t+1}) lambda_{t+1}
   * on entry to position t; on entry to L-1 it is d_last[b] (zero without it). */
  if (c->d_last)
    memcpy(lam, c->d_last + ((b * s->nheads + h) * PN), sizeof(double) * PN);
  else
    memset(lam, 0, sizeof(double) * PN);
  double dA_acc = 0.0, dD_acc = 0.0;
  for (int64_t k = nblk - 1; k >= 0; --k) {
    const int64_t t0 = k * CKPT, t1 = (t0 + CKPT < L) ? t0 + CKPT : L;
    /* recompute the block's states */
    {
      const double* run = ckpt + k * PN;
      for (int64_t t = t0; t < t1; ++t) {
        double* out = hs + (t - t0) * PN;
        step_state(c, b, t, h, prev_state(c, b, t, h, run, zeros), out);
        run = out;
      }
    }
    for (int64_t t = t1 - 1; t >= t0; --t) {
      const int64_t i = b * L + t;
      const double* ht = hs + (t - t0) * PN;
      const double* run_prev = (t > t0) ? hs + (t - t0 - 1) * PN : ckpt + k * PN;
      const double* hp = prev_state(c, b, t, h, run_prev, zeros);
      const double* xt = c->x + IDX_X(s, b, t, h, 0);
      const double* dyt = c->dy + IDX_X(s, b, t, h, 0);
      const double* Bt = c->B + IDX_BC(s, b, t, g, 0);
      const double* Ct = c->C + IDX_BC(s, b, t, g, 0);
      const double dtv = c->dt[IDX_BLH(s, b, t, h)];
      const double decay = exp(dtv * Ah);

      /* chunk export of the incoming carry = gradient w.r.t. the state at
       * the end of this chunk, as seen from later positions */
      if (c->chunk > 0 && ((t + 1) % c->chunk == 0 || t == L - 1) && c->chunk_dout) {
        const int64_t nc = (L + c->chunk - 1) / c->chunk, cc = t / c->chunk;
        memcpy(c->chunk_dout + (((b * nc + cc) * s->nheads + h) * PN), lam, sizeof(double) * PN);
      }

      /* lambda_t = dy_t (outer) C_t + carry */
      for (int64_t p = 0; p < P; ++p)
        for (int64_t n = 0; n < N; ++n) lam[p * N + n] += dyt[p] * Ct[n];

      /* dC_t += h_t^T dy_t */
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t p = 0; p < P; ++p) acc += ht[p * N + n] * dyt[p];
        dCi[t * N + n] = acc;
      }
      /* lamB = lambda_t B_t ; dx_t ; dB_t */
      double xlb = 0.0, dyx = 0.0;
      for (int64_t p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += lam[p * N + n] * Bt[n];
        lamB[p] = acc;
        c->dx[IDX_X(s, b, t, h, p)] = dtv * acc + Dh * dyt[p];
        xlb += xt[p] * acc;
        dyx += dyt[p] * xt[p];
      }
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t p = 0; p < P; ++p) acc += lam[p * N + n] * xt[p];
        dBi[t * N + n] = dtv * acc;
      }
      /* da_t = exp(a_t) <lambda_t, h_{t-1}> */
      double inner = 0.0;
      for (int64_t q = 0; q < PN; ++q) inner += lam[q] * hp[q];
      const double da = decay * inner;
      c->ddt[IDX_BLH(s, b, t, h)] = xlb + Ah * da;
      dA_acc += dtv * da;
      dD_acc += dyx;

      /* carry to t-1, or the initial-state gradient at a sequence start */
      if (c->start[i]) {
        if (c->d_h0) {
          double* dst = c->d_h0 + ((c->seq[i] * s->nheads + h) * PN);
          for (int64_t q = 0; q < PN; ++q) dst[q] = decay * lam[q];
        }
        memset(lam, 0, sizeof(double) * PN);
      } else {
        for (int64_t q = 0; q < PN; ++q) lam[q] *= decay;
      }
    }
  }
  c->dA_part[b * s->nheads + h] = dA_acc;
  c->dD_part[b * s->nheads + h] = dD_acc;
}

static void* worker(void* arg) {
  ctx_t* c = (ctx_t*)arg;
  const ssdo_shape* s = c->s;
  const int64_t P = s->headdim, N = s->dstate, PN = P * N;
  const int64_t nblk = (s->seqlen + CKPT - 1) / CKPT;
  double* zeros = (double*)calloc((size_t)PN, sizeof(double));
  double* bufA = (double*)malloc(sizeof(double) * PN);
  double* bufB = (double*)malloc(sizeof(double) * PN);
  double* ckpt = c->mode ? (double*)malloc(sizeof(double) * PN * nblk) : NULL;
  double* hs = c->mode ? (double*)malloc(sizeof(double) * PN * CKPT) : NULL;
  double* lamB = (double*)malloc(sizeof(double) * P);
  if (!zeros || !bufA || !bufB || !lamB || (c->mode && (!ckpt || !hs))) {
    pthread_mutex_lock(&c->lock);
    c->failed = 1;
    pthread_mutex_unlock(&c->lock);
  } else {
    const int64_t nh = c->head_hi - c->head_lo;
    for (;;) {
      pthread_mutex_lock(&c->lock);
      const int64_t it = c->next_item++;
      pthread_mutex_unlock(&c->lock);
      if (it >= c->n_items) break;
      const int64_t b = it / nh, h = c->head_lo + it % nh;
      if (c->mode == 0) forward_item(c, b, h, bufA, bufB, zeros);
      else backward_item(c, it, b, h, ckpt, hs, bufA, lamB, zeros);
    }
  }
  free(zeros); free(bufA); free(bufB); free(ckpt); free(hs); free(lamB);
  return NULL;
}

static int run_threads(ctx_t* c, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > c->n_items) nthreads = (int)c->n_items;
  if (nthreads < 1) return SSDO_OK;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  if (!th) return SSDO_ENOMEM;
  pthread_mutex_init(&c->lock, NULL);
  int started = 0;
  for (int i = 0; i < nthreads; ++i)
    if (pthread_create(&th[i], NULL, worker, c) == 0) ++started;
  if (started == 0) worker(c);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&c->lock);
  free(th);
  return c->failed ? SSDO_ENOMEM : SSDO_OK;
}

static int check_shape(const ssdo_shape* s) {
  if (!s || s->batch < 1 || s->seqlen < 1 || s->nheads < 1 || s->headdim < 1 ||
      s->ngroups < 1 || s->dstate < 1 || s->nheads % s->ngroups)
    return SSDO_EINVAL;
  return SSDO_OK;
}

/* Number of sequences that seq_idx (nullable) describes. */
int64_t ssdo_count_sequences(const ssdo_shape* s, const int32_t* seq_idx) {
  if (check_shape(s)) return SSDO_EINVAL;
  const int64_t BL = s->batch * s->seqlen;
  uint8_t* st = (uint8_t*)malloc((size_t)BL);
  int64_t* sq = (int64_t*)malloc(sizeof(int64_t) * BL);
  int64_t n = SSDO_ENOMEM;
  if (st && sq) n = find_sequences(s, seq_idx, st, sq);
  free(st); free(sq);
  return n;
}

/* Forward: y (B,L,H,P); final_states (S,H,P,N) nullable. */
int ssdo_forward(const ssdo_shape* s, const double* x, const double* dt, const double* A,
                 const double* B, const double* C, const double* D, const double* h0,
                 const int32_t* seq_idx, double* y, double* final_states, int nthreads) {
  if (check_shape(s) || !x || !dt || !A || !B || !C || !y) return SSDO_EINVAL;
  const int64_t BL = s->batch * s->seqlen;
  ctx_t c;
  memset(&c, 0, sizeof(c));
  uint8_t* st = (uint8_t*)malloc((size_t)BL);
  int64_t* sq = (int64_t*)malloc(sizeof(int64_t) * BL);
  if (!st || !sq) { free(st); free(sq); return SSDO_ENOMEM; }
  const int64_t ns = find_sequences(s, seq_idx, st, sq);
  if (ns != s->nseqs) { free(st); free(sq); return SSDO_EINVAL; }
  c.s = s; c.x = x; c.dt = dt; c.A = A; c.B = B; c.C = C; c.D = D; c.h0 = h0;
  c.start = st; c.seq = sq; c.y = y; c.final_states = final_states;
  c.head_lo = 0; c.head_hi = s->nheads;
  c.n_items = s->batch * s->nheads;
  c.mode = 0;
  const int rc = run_threads(&c, nthreads);
  free(st); free(sq);
  return rc;
}

/*
 * Backward over heads [head_lo, head_hi).  dB/dC are written only for the
 * groups all of whose heads lie in the range.
 * Outputs (all fp64, caller-owned, written only for the covered heads/groups):
 *   dx (B,L,H,P), ddt (B,L,H), dA (H), dB (B,L,G,N), dC (B,L,G,N), dD (H),
 *   d_h0 (S,H,P,N, nullable).
 *   d_last (B,H,P,N, nullable): gradient input for the state after position
 *   L-1 of each batch row (the final state of the row's last sequence).
 * Optional exports for chunk-level checks (chunk > 0):
 *   chunk_states (B,nc,H,P,N): state after position c*chunk - 1 (zeros for c=0),
 *   chunk_dout  (B,nc,H,P,N): gradient w.r.t. the state at the end of chunk c
 *                              flowing from later positions.
 */
int ssdo_backward(const ssdo_shape* s, const double* x, const double* dt, const double* A,
                  const double* B, const double* C, const double* D, const double* h0,
                  const int32_t* seq_idx, const double* dy, int64_t head_lo, int64_t head_hi,
                  double* dx, double* ddt, double* dA, double* dB, double* dC, double* dD,
                  double* d_h0, int64_t chunk, double* chunk_states, double* chunk_dout,
                  const double* d_last, int nthreads) {
  if (check_shape(s) || !x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB ||
      !dC || !dD)
    return SSDO_EINVAL;
  const int64_t hpg = s->nheads / s->ngroups;
  if (head_lo < 0 || head_hi > s->nheads || head_lo >= head_hi) return SSDO_EINVAL;
  const int64_t L = s->seqlen, N = s->dstate, P = s->headdim, BL = s->batch * L;
  const int64_t nh = head_hi - head_lo;
  ctx_t c;
  memset(&c, 0, sizeof(c));
  uint8_t* st = (uint8_t*)malloc((size_t)BL);
  int64_t* sq = (int64_t*)malloc(sizeof(int64_t) * BL);
  double* dAp = (double*)calloc((size_t)(s->batch * s->nheads), sizeof(double));
  double* dDp = (double*)calloc((size_t)(s->batch * s->nheads), sizeof(double));
  double* dBi = (double*)malloc(sizeof(double) * (size_t)(s->batch * nh * L * N));
  double* dCi = (double*)malloc(sizeof(double) * (size_t)(s->batch * nh * L * N));
  int rc = SSDO_ENOMEM;
  if (!st || !sq || !dAp || !dDp || !dBi || !dCi) goto done;
  rc = SSDO_EINVAL;
  if (find_sequences(s, seq_idx, st, sq) != s->nseqs) goto done;
  c.s = s; c.x = x; c.dt = dt; c.A = A; c.B = B; c.C = C; c.D = D; c.h0 = h0; c.dy = dy;
  c.start = st; c.seq = sq; c.head_lo = head_lo; c.head_hi = head_hi;
  c.d_last = d_last;
  c.dx = dx; c.ddt = ddt; c.dA_part = dAp; c.dD_part = dDp; c.d_h0 = d_h0;
  c.dB_item = dBi; c.dC_item = dCi;
  c.chunk = chunk; c.chunk_states = chunk_states; c.chunk_dout = chunk_dout;
  c.n_items = s->batch * nh;
  c.mode = 1;
  rc = run_threads(&c, nthreads);
  if (rc) goto done;

  /* fixed-order merges */
  for (int64_t h = head_lo; h < head_hi; ++h) {
    double a = 0.0, d = 0.0;
    for (int64_t b = 0; b < s->batch; ++b) { a += dAp[b * s->nheads + h]; d += dDp[b * s->nheads + h]; }
    dA[h] = a;
    dD[h] = d;
  }
  /* dB/dC only for the groups whose heads are all covered */
  for (int64_t b = 0; b < s->batch; ++b)
    for (int64_t g = (head_lo + hpg - 1) / hpg; g < head_hi / hpg; ++g)
      for (int64_t t = 0; t < L; ++t)
        for (int64_t n = 0; n < N; ++n) {
          double sb = 0.0, sc = 0.0;
          for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
            const int64_t item = b * nh + (h - head_lo);
            sb += dBi[(item * L + t) * N + n];
            sc += dCi[(item * L + t) * N + n];
          }
          dB[IDX_BC(s, b, t, g, n)] = sb;
          dC[IDX_BC(s, b, t, g, n)] = sc;
        }

  /* chunk-state export: a plain forward sweep over the covered heads */
  if (chunk > 0 && chunk_states) {
    const int64_t nc = (L + chunk - 1) / chunk, PN = P * N;
    double* zeros = (double*)calloc((size_t)PN, sizeof(double));
    double* run = (double*)malloc(sizeof(double) * PN);
    double* nxt = (double*)malloc(sizeof(double) * PN);
    if (!zeros || !run || !nxt) { free(zeros); free(run); free(nxt); rc = SSDO_ENOMEM; goto done; }
    for (int64_t b = 0; b < s->batch; ++b)
      for (int64_t h = head_lo; h < head_hi; ++h) {
        memset(run, 0, sizeof(double) * PN);
        for (int64_t t = 0; t < L; ++t) {
          if (t % chunk == 0)
            memcpy(chunk_states + (((b * nc + t / chunk) * s->nheads + h) * PN), run, sizeof(double) * PN);
          step_state(&c, b, t, h, prev_state(&c, b, t, h, run, zeros), nxt);
          double* tmp = run; run = nxt; nxt = tmp;
        }
      }
    free(zeros); free(run); free(nxt);
  }
  rc = SSDO_OK;
done:
  free(st); free(sq); free(dAp); free(dDp); free(dBi); free(dCi);
  return rc;
}
