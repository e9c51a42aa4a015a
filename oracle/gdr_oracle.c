/*
 * Float64 CPU oracle for the gated delta rule (GDN scalar gate and KDA
 * per-channel gate): token-by-token forward recurrence and its hand-derived
 * reverse-time adjoint.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links or calls this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
 * shares no code with the HIP path.
 *
 * What it computes (per sequence n and head h, all in double):
 *   qn = q * rho_q,  rho_q = (|q|^2 + 1e-6)^(-1/2)      (likewise kn)
 *       -- the L2 normalisation recomputed by the FlashKDA backward prepare
 *          kernel (yuyanqi.com, "FlashKDA backward (K1)", §3.1; eps inside the
 *          square root as in its listing's Phase 1+2)
 *   beta = sigmoid(b)                                    (same page, §6)
 *   lambda = g                         (scalar gate, the given log decay)
 *   lambda = -exp(A_log) * softplus(g_raw + dt_bias)     (per-channel gate)
 *   lambda = gate_scale * sigmoid(exp(A_log) * (g_raw + dt_bias))
 *                                     (per-channel gate, bounded sigmoid form,
 *                                      FlashKDA K1 page, section 5.2; natural log)
 *   For t = 1..T, with S a Dv x Dk matrix (S = h0 or 0 at t = 0):
 *     St  = S * Diag(exp(lambda_t))
 *     e   = St kn_t,   u = beta_t (v_t - e),   S = St + u kn_t^T
 *     o_t = scale * S qn_t
 *   This is S_t = S_{t-1} Diag(e^{g_t}) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   with the rank-one update expanded.
 *
 * The backward is the exact gradient of L = sum_t <dO_t, o_t> + <dht, S_T>
 * obtained by running the adjoint of each forward statement in reverse order.
 * States inside a chunk are recomputed from a checkpoint saved every `chunk`
 * tokens.  The epilogue maps the gradients of qn, kn, beta and lambda back to
 * q, k, the beta logit and the gate inputs: L2-norm backward (K1 page §3.3),
 * sigmoid backward (§6) and the gate-function backward with the per-head sums
 * for dA_log and ddt_bias (§5.2).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  /* shape */
  int32_t N, H, K, V;
  int32_t gate;       /* 0: scalar log decay [T][H]; 1, 2: per-channel gate from g_raw [T][H][K]
                         (1 softplus form, 2 bounded sigmoid form) */
  int32_t chunk;      /* checkpoint spacing, also the chunking of the exports */
  int32_t nthreads;   /* worker threads (<= 0: 1) */
  int32_t do_backward;
  double scale;
  const int64_t* cu;  /* [N+1] sequence offsets into the packed token axis */
  /* inputs, token-major: x[t][h][d] with t in [0, cu[N]) */
  const double *q, *k;     /* [T][H][K] */
  const double *v, *dO;    /* [T][H][V] */
  const double *b;         /* [T][H] beta logit */
  const double *g;         /* [T][H] (gate 0) or [T][H][K] (gate 1) */
  const double *A_log;     /* [H]     (gate 1) */
  const double *dt_bias;   /* [H][K]  (gate 1) */
  const double *h0, *dht;  /* [N][H][V][K] or NULL (zero) */
  /* outputs, NULL to skip */
  double *o;               /* [T][H][V] */
  double *ht;              /* [N][H][V][K] */
  double *dq, *dk;         /* [T][H][K] */
  double *dv;              /* [T][H][V] */
  double *dg;              /* [T][H] (gate 0) or [T][H][K] (gate 1) */
  double *db;              /* [T][H] */
  double *dh0;             /* [N][H][V][K] */
  double *dA_log;          /* [H] */
  double *ddt_bias;        /* [H][K] */
  /* intermediate exports, NULL to skip; chunk c of sequence n has global
   * index c + sum_{m<n} ceil(len_m / chunk) */
  double *S_chunk;         /* [H][NC][V][K] state at the start of each chunk */
  double *dS_chunk;        /* [H][NC][V][K] gradient w.r.t. the state at the end of each chunk */
  double *u_out;           /* [T][H][V] the written value u_t */
  double *dqn, *dkn;       /* [T][H][K] gradients w.r.t. the normalised q, k */
  double *dbeta;           /* [T][H] gradient w.r.t. beta (after the sigmoid) */
  double *dlam;            /* [T][H] (gate 0) or [T][H][K] (gate 1) gradient w.r.t. lambda_t */
  double gate_scale;       /* gate 2: the bound of the per-token log decay */
  int32_t Hk;              /* key heads of q, k, dq, dk ([T][Hk][K]); 0 = H.  Value head h reads
                              key head h / (H / Hk) (grouped query attention) */
} oracle_args;

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

typedef struct {
  const oracle_args* a;
  int64_t* chunk_base;   /* [N] global index of each sequence's first chunk */
  int64_t NC;
  double* part_dA;       /* [N][H] */
  double* part_ddt;      /* [N][H][K] */
  double *dq_v, *dk_v;   /* grouped heads: dq, dk per value head [T][H][K], summed per group at the end */
  int next;              /* work counter */
  pthread_mutex_t mu;
  int failed;
} pool_t;

/* One (sequence, head) pair: forward, backward and epilogue. */
static int run_item(pool_t* P, int n, int h) {
  const oracle_args* a = P->a;
  const int H = a->H, K = a->K, V = a->V, C = a->chunk;
  const int Hk = a->Hk > 0 ? a->Hk : H, hk = h / (H / Hk);
  double* const dq_out = P->dq_v ? P->dq_v : a->dq;   /* indexed per value head below */
  double* const dk_out = P->dk_v ? P->dk_v : a->dk;
  const int64_t t0 = a->cu[n];
  const int len = (int)(a->cu[n + 1] - a->cu[n]);
  const int nck = (len + C - 1) / C;
  const size_t VK = (size_t)V * K;

  double* qn = calloc((size_t)(len > 0 ? len : 1) * K, sizeof(double));
  double* kn = calloc((size_t)(len > 0 ? len : 1) * K, sizeof(double));
  double* rq = calloc(len > 0 ? len : 1, sizeof(double));
  double* rk = calloc(len > 0 ? len : 1, sizeof(double));
  double* beta = calloc(len > 0 ? len : 1, sizeof(double));
  double* lam = calloc((size_t)(len > 0 ? len : 1) * K, sizeof(double));
  double* S = calloc(VK, sizeof(double));
  double* ckpt = calloc((size_t)(nck > 0 ? nck : 1) * VK, sizeof(double));
  double* pre = calloc((size_t)C * VK, sizeof(double));
  double* ub = calloc((size_t)C * V, sizeof(double));
  double* eb = calloc((size_t)C * V, sizeof(double));
  double* dS = calloc(VK, sizeof(double));
  double* St = calloc(VK, sizeof(double));
  double* dqn = calloc((size_t)(len > 0 ? len : 1) * K, sizeof(double));
  double* dkn = calloc((size_t)(len > 0 ? len : 1) * K, sizeof(double));
  double* dbeta = calloc(len > 0 ? len : 1, sizeof(double));
  double* dlam = calloc((size_t)(len > 0 ? len : 1) * K, sizeof(double));
  double* du = calloc(V, sizeof(double));
  double* dec = calloc(K, sizeof(double));
  if (!qn || !kn || !rq || !rk || !beta || !lam || !S || !ckpt || !pre || !ub || !eb || !dS ||
      !St || !dqn || !dkn || !dbeta || !dlam || !du || !dec) {
    free(qn); free(kn); free(rq); free(rk); free(beta); free(lam); free(S); free(ckpt);
    free(pre); free(ub); free(eb); free(dS); free(St); free(dqn); free(dkn); free(dbeta);
    free(dlam); free(du); free(dec);
    return -1;
  }

  /* ---- per-token prologue: normalisation, beta, log decay ---- */
  for (int t = 0; t < len; ++t) {
    const int64_t row = (t0 + t) * H + h;
    const double* qt = a->q + ((t0 + t) * Hk + hk) * K;
    const double* kt = a->k + ((t0 + t) * Hk + hk) * K;
    double sq = 0.0, sk = 0.0;
    for (int j = 0; j < K; ++j) { sq += qt[j] * qt[j]; sk += kt[j] * kt[j]; }
    rq[t] = 1.0 / sqrt(sq + 1e-6);
    rk[t] = 1.0 / sqrt(sk + 1e-6);
    for (int j = 0; j < K; ++j) {
      qn[(size_t)t * K + j] = qt[j] * rq[t];
      kn[(size_t)t * K + j] = kt[j] * rk[t];
    }
    beta[t] = sigmoid(a->b[row]);
    if (a->gate == 0) {
      for (int j = 0; j < K; ++j) lam[(size_t)t * K + j] = a->g[row];
    } else if (a->gate == 1) {
      const double ea = exp(a->A_log[h]);
      for (int j = 0; j < K; ++j)
        lam[(size_t)t * K + j] = -ea * softplus(a->g[row * K + j] + a->dt_bias[(size_t)h * K + j]);
    } else {
      const double ea = exp(a->A_log[h]);
      for (int j = 0; j < K; ++j)
        lam[(size_t)t * K + j] = a->gate_scale * sigmoid(ea * (a->g[row * K + j] + a->dt_bias[(size_t)h * K + j]));
    }
  }

  /* ---- forward ---- */
  if (a->h0) memcpy(S, a->h0 + ((size_t)n * H + h) * VK, VK * sizeof(double));
  for (int t = 0; t < len; ++t) {
    const int64_t row = (t0 + t) * H + h;
    const double* knt = kn + (size_t)t * K;
    const double* qnt = qn + (size_t)t * K;
    if (t % C == 0) memcpy(ckpt + (size_t)(t / C) * VK, S, VK * sizeof(double));
    for (int j = 0; j < K; ++j) dec[j] = exp(lam[(size_t)t * K + j]);
    for (int i = 0; i < V; ++i) {
      double* Si = S + (size_t)i * K;
      double e = 0.0;
      for (int j = 0; j < K; ++j) { Si[j] *= dec[j]; e += Si[j] * knt[j]; }
      const double u = beta[t] * (a->v[row * V + i] - e);
      if (a->u_out) a->u_out[row * V + i] = u;
      double o = 0.0;
      for (int j = 0; j < K; ++j) { Si[j] += u * knt[j]; o += Si[j] * qnt[j]; }
      if (a->o) a->o[row * V + i] = a->scale * o;
    }
  }
  if (a->ht) memcpy(a->ht + ((size_t)n * H + h) * VK, S, VK * sizeof(double));
  if (a->S_chunk)
    for (int c = 0; c < nck; ++c)
      memcpy(a->S_chunk + ((size_t)h * P->NC + P->chunk_base[n] + c) * VK, ckpt + (size_t)c * VK,
             VK * sizeof(double));

  if (!a->do_backward) goto done;

  /* ---- backward: chunks last to first, states recomputed from checkpoints ---- */
  if (a->dht) memcpy(dS, a->dht + ((size_t)n * H + h) * VK, VK * sizeof(double));
  for (int c = nck - 1; c >= 0; --c) {
    const int ts = c * C, te = (ts + C < len) ? ts + C : len;
    /* recompute: pre[t] = S_{t-1}, ub[t] = u_t, eb[t] = e_t */
    memcpy(S, ckpt + (size_t)c * VK, VK * sizeof(double));
    for (int t = ts; t < te; ++t) {
      const int64_t row = (t0 + t) * H + h;
      const double* knt = kn + (size_t)t * K;
      memcpy(pre + (size_t)(t - ts) * VK, S, VK * sizeof(double));
      for (int j = 0; j < K; ++j) dec[j] = exp(lam[(size_t)t * K + j]);
      for (int i = 0; i < V; ++i) {
        double* Si = S + (size_t)i * K;
        double e = 0.0;
        for (int j = 0; j < K; ++j) { Si[j] *= dec[j]; e += Si[j] * knt[j]; }
        const double u = beta[t] * (a->v[row * V + i] - e);
        eb[(size_t)(t - ts) * V + i] = e;
        ub[(size_t)(t - ts) * V + i] = u;
        for (int j = 0; j < K; ++j) Si[j] += u * knt[j];
      }
    }
    if (a->dS_chunk)
      memcpy(a->dS_chunk + ((size_t)h * P->NC + P->chunk_base[n] + c) * VK, dS, VK * sizeof(double));
    for (int t = te - 1; t >= ts; --t) {
      const int64_t row = (t0 + t) * H + h;
      const double* knt = kn + (size_t)t * K;
      const double* qnt = qn + (size_t)t * K;
      const double* dOt = a->dO + row * V;
      const double* ut = ub + (size_t)(t - ts) * V;
      const double* et = eb + (size_t)(t - ts) * V;
      double* dqt = dqn + (size_t)t * K;
      double* dkt = dkn + (size_t)t * K;
      for (int j = 0; j < K; ++j) dec[j] = exp(lam[(size_t)t * K + j]);
      /* St = S_{t-1} Diag(dec) (the decayed state before the write) */
      for (size_t x = 0; x < VK; ++x) St[x] = pre[(size_t)(t - ts) * VK + x] * dec[x % K];
      /* o_t = scale * (St + u kn^T) qn */
      for (int i = 0; i < V; ++i) {
        const double* Sti = St + (size_t)i * K;
        double* dSi = dS + (size_t)i * K;
        const double w = a->scale * dOt[i];
        for (int j = 0; j < K; ++j) {
          dSi[j] += w * qnt[j];
          dqt[j] += w * (Sti[j] + ut[i] * knt[j]);
        }
      }
      /* S_t = St + u kn^T */
      double dbt = 0.0;
      for (int i = 0; i < V; ++i) {
        const double* dSi = dS + (size_t)i * K;
        double s = 0.0;
        for (int j = 0; j < K; ++j) { s += dSi[j] * knt[j]; dkt[j] += dSi[j] * ut[i]; }
        du[i] = s;
        /* u = beta (v - e) */
        if (a->dv) a->dv[row * V + i] = beta[t] * s;
        dbt += s * (a->v[row * V + i] - et[i]);
      }
      dbeta[t] = dbt;
      /* e = St kn: de = -beta du; dSt += de kn^T; dkn += St^T de */
      for (int i = 0; i < V; ++i) {
        const double* Sti = St + (size_t)i * K;
        double* dSi = dS + (size_t)i * K;
        const double de = -beta[t] * du[i];
        for (int j = 0; j < K; ++j) { dSi[j] += de * knt[j]; dkt[j] += Sti[j] * de; }
      }
      /* St = S_{t-1} Diag(dec): dlam_j = sum_i dSt_ij St_ij ; dS_{t-1} = dSt Diag(dec) */
      double* dlt = dlam + (size_t)t * K;
      for (int j = 0; j < K; ++j) dlt[j] = 0.0;
      for (int i = 0; i < V; ++i) {
        const double* Sti = St + (size_t)i * K;
        double* dSi = dS + (size_t)i * K;
        for (int j = 0; j < K; ++j) { dlt[j] += dSi[j] * Sti[j]; dSi[j] *= dec[j]; }
      }
    }
  }
  if (a->dh0) memcpy(a->dh0 + ((size_t)n * H + h) * VK, dS, VK * sizeof(double));

  /* ---- epilogue ---- */
  {
    const double ea = (a->gate >= 1) ? exp(a->A_log[h]) : 0.0;
    double* pdA = P->part_dA + (size_t)n * H + h;
    double* pdt = P->part_ddt + ((size_t)n * H + h) * K;
    for (int t = 0; t < len; ++t) {
      const int64_t row = (t0 + t) * H + h;
      const double* qnt = qn + (size_t)t * K;
      const double* knt = kn + (size_t)t * K;
      const double* dqt = dqn + (size_t)t * K;
      const double* dkt = dkn + (size_t)t * K;
      const double* dlt = dlam + (size_t)t * K;
      double pq = 0.0, pk = 0.0;
      for (int j = 0; j < K; ++j) { pq += qnt[j] * dqt[j]; pk += knt[j] * dkt[j]; }
      for (int j = 0; j < K; ++j) {
        if (dq_out) dq_out[row * K + j] = rq[t] * (dqt[j] - qnt[j] * pq);
        if (dk_out) dk_out[row * K + j] = rk[t] * (dkt[j] - knt[j] * pk);
        if (a->dqn) a->dqn[row * K + j] = dqt[j];
        if (a->dkn) a->dkn[row * K + j] = dkt[j];
      }
      if (a->db) a->db[row] = dbeta[t] * beta[t] * (1.0 - beta[t]);
      if (a->dbeta) a->dbeta[row] = dbeta[t];
      if (a->gate == 0) {
        double s = 0.0;
        for (int j = 0; j < K; ++j) s += dlt[j];
        if (a->dg) a->dg[row] = s;
        if (a->dlam) a->dlam[row] = s;
      } else if (a->gate == 1) {
        /* d lambda / d x = -e^A_log sigmoid(x), d lambda / d A_log = lambda */
        for (int j = 0; j < K; ++j) {
          const double x = a->g[row * K + j] + a->dt_bias[(size_t)h * K + j];
          const double dgr = dlt[j] * (-ea * sigmoid(x));
          if (a->dg) a->dg[row * K + j] = dgr;
          if (a->dlam) a->dlam[row * K + j] = dlt[j];
          pdt[j] += dgr;
          *pdA += dlt[j] * lam[(size_t)t * K + j];
        }
      } else {
        /* z = e^A_log x: d lambda / dz = gate_scale sigmoid(z) (1 - sigmoid(z)),
         * dz / dx = e^A_log, dz / d A_log = e^A_log x */
        for (int j = 0; j < K; ++j) {
          const double x = a->g[row * K + j] + a->dt_bias[(size_t)h * K + j];
          const double sz = sigmoid(ea * x);
          const double dz = dlt[j] * a->gate_scale * sz * (1.0 - sz);
          if (a->dg) a->dg[row * K + j] = dz * ea;
          if (a->dlam) a->dlam[row * K + j] = dlt[j];
          pdt[j] += dz * ea;
          *pdA += dz * ea * x;
        }
      }
    }
  }

done:
  free(qn); free(kn); free(rq); free(rk); free(beta); free(lam); free(S); free(ckpt);
  free(pre); free(ub); free(eb); free(dS); free(St); free(dqn); free(dkn); free(dbeta);
  free(dlam); free(du); free(dec);
  return 0;
}

static void* worker(void* arg) {
  pool_t* P = (pool_t*)arg;
  const int total = P->a->N * P->a->H;
  for (;;) {
    pthread_mutex_lock(&P->mu);
    const int it = P->next++;
    pthread_mutex_unlock(&P->mu);
    if (it >= total) break;
    if (run_item(P, it / P->a->H, it % P->a->H) != 0) {
      pthread_mutex_lock(&P->mu);
      P->failed = 1;
      pthread_mutex_unlock(&P->mu);
    }
  }
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int oracle_run(const oracle_args* a) {
  if (!a || a->N < 0 || a->H <= 0 || a->K <= 0 || a->V <= 0 || a->chunk <= 0 || !a->cu) return -1;
  if (!a->q || !a->k || !a->v || !a->b || !a->g) return -1;
  if (a->do_backward && !a->dO) return -1;
  if (a->gate < 0 || a->gate > 2) return -1;
  if (a->gate >= 1 && (!a->A_log || !a->dt_bias)) return -1;
  if (a->Hk < 0 || (a->Hk > 0 && a->H % a->Hk != 0)) return -1;
  for (int n = 0; n < a->N; ++n)
    if (a->cu[n + 1] < a->cu[n]) return -1;

  pool_t P;
  memset(&P, 0, sizeof(P));
  P.a = a;
  P.chunk_base = calloc(a->N > 0 ? a->N : 1, sizeof(int64_t));
  P.part_dA = calloc((size_t)(a->N > 0 ? a->N : 1) * a->H, sizeof(double));
  P.part_ddt = calloc((size_t)(a->N > 0 ? a->N : 1) * a->H * a->K, sizeof(double));
  const int Hk = a->Hk > 0 ? a->Hk : a->H, G = a->H / Hk;
  const int64_t TT = a->N > 0 ? a->cu[a->N] : 0;
  if (G > 1 && a->do_backward) {
    P.dq_v = calloc((size_t)(TT > 0 ? TT : 1) * a->H * a->K, sizeof(double));
    P.dk_v = calloc((size_t)(TT > 0 ? TT : 1) * a->H * a->K, sizeof(double));
  }
  if (!P.chunk_base || !P.part_dA || !P.part_ddt || (G > 1 && a->do_backward && (!P.dq_v || !P.dk_v))) {
    free(P.chunk_base); free(P.part_dA); free(P.part_ddt); free(P.dq_v); free(P.dk_v);
    return -2;
  }
  for (int n = 0; n < a->N; ++n) {
    P.chunk_base[n] = P.NC;
    P.NC += (a->cu[n + 1] - a->cu[n] + a->chunk - 1) / a->chunk;
  }
  pthread_mutex_init(&P.mu, NULL);
  int nt = a->nthreads > 0 ? a->nthreads : 1;
  if (nt > a->N * a->H) nt = a->N * a->H > 0 ? a->N * a->H : 1;
  pthread_t* th = calloc(nt, sizeof(pthread_t));
  int started = 0;
  for (int i = 0; i < nt && th; ++i)
    if (pthread_create(&th[i], NULL, worker, &P) == 0) ++started;
  if (started == 0) worker(&P);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&P.mu);

  if (a->do_backward && a->gate >= 1) {
    /* per-head parameter gradients: sum over sequences in a fixed order */
    for (int h = 0; h < a->H; ++h) {
      double s = 0.0;
      for (int n = 0; n < a->N; ++n) s += P.part_dA[(size_t)n * a->H + h];
      if (a->dA_log) a->dA_log[h] = s;
      for (int j = 0; j < a->K; ++j) {
        double sj = 0.0;
        for (int n = 0; n < a->N; ++n) sj += P.part_ddt[((size_t)n * a->H + h) * a->K + j];
        if (a->ddt_bias) a->ddt_bias[(size_t)h * a->K + j] = sj;
      }
    }
  }
  if (P.dq_v) {
    /* grouped heads: the key head's gradient is the sum over its G value heads, in order */
    for (int64_t t = 0; t < TT; ++t)
      for (int hk = 0; hk < Hk; ++hk)
        for (int j = 0; j < a->K; ++j) {
          double sq = 0.0, sk = 0.0;
          for (int g = 0; g < G; ++g) {
            const size_t i = ((size_t)t * a->H + (size_t)hk * G + g) * a->K + j;
            sq += P.dq_v[i];
            sk += P.dk_v[i];
          }
          if (a->dq) a->dq[((size_t)t * Hk + hk) * a->K + j] = sq;
          if (a->dk) a->dk[((size_t)t * Hk + hk) * a->K + j] = sk;
        }
  }
  const int failed = P.failed;
  free(P.chunk_base); free(P.part_dA); free(P.part_ddt); free(P.dq_v); free(P.dk_v);
  return failed ? -2 : 0;
}
