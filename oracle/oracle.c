/*
 * oracle.c -- plain fp64 CPU oracle for the linear-recurrent token mixers.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or constant with the GPU path.
 *
 * What it computes (per batch b and head h, one token at a time, in fp64):
 *
 *   The mixers are described in the AMD ROCm blog "Pretraining hybrid LLMs
 *   with Primus" (section "How hybrid models are defined in Primus", the
 *   mixer list under Table 2):
 *     - Mamba2: a selective SSM whose state is decayed by one scalar gate per
 *       head;
 *     - Gated DeltaNet: Mamba2 plus the delta rule -- the association stored
 *       for the current key is overwritten instead of only accumulated -- with
 *       one scalar forget gate per head;
 *     - Kimi Delta Attention: GDN with the gate refined to one value per key
 *       dimension (the low-rank projection that produces it is an input here).
 *
 *   The state is kept as H = S^T with shape [d_k, d_v] (S is the d_v x d_k
 *   matrix of the Gated DeltaNet recurrence S_t = a_t S_{t-1}(I - b_t k k^T)
 *   + b_t v k^T, o_t = S_t q_t).  In that orientation:
 *
 *     GDN: u_t = beta_t (v_t - a_t H_{t-1}^T k_t);  H_t = a_t H_{t-1} + k_t u_t^T
 *     SSD: H_t = a_t H_{t-1} + k_t v_t^T            (no beta, no delta term)
 *     KDA: X = Diag(a_t) H_{t-1};  u_t = beta_t (v_t - X^T k_t);  H_t = X + k_t u_t^T
 *     all: o_t = H_t^T q_t  (the output reads the state after token t's write),
 *          a_t = exp(log_a_t), H_0 = h0 (or zero), ht = H_T.
 *
 *   Columns of H (the d_v index) never mix in any of the three recurrences,
 *   so the forward can be evaluated on a range of value columns only; the
 *   full-size parity checks use that to sample outputs of very long inputs.
 *
 *   The backward is plain back-propagation through time of the same
 *   recurrence (derivatives written out by hand, pinned by finite
 *   differences in the tests).  States are checkpointed every SEG tokens and
 *   each segment is recomputed forward before it is walked backwards.
 *
 * Dtypes of the typed inputs: 0 = fp32, 1 = bf16 (raw 16-bit patterns),
 * 2 = fp64.  Every element is widened to fp64 on read, so the oracle sees
 * exactly the values the GPU path sees.  All outputs are fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_GDN 0
#define OR_SSD 1
#define OR_KDA 2
#define SEG 64

static double rd(const void* p, int dt, size_t i) {
  if (dt == 0) return (double)((const float*)p)[i];
  if (dt == 2) return ((const double*)p)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

static int bad_dt(int dt) { return dt != 0 && dt != 1 && dt != 2; }

/* Forward over value columns [c0, c0+nc).  o: [B,T,H,nc], ht: [B,H,dk,nc]. */
int oracle_fwd(int variant, const void* q, const void* k, const void* v, int dtype,
               const void* log_a, const void* beta, const void* h0, int gdtype,
               double* o, double* ht, int B, int T, int H, int dk, int dv, int c0, int nc,
               int nthreads) {
  if (variant < 0 || variant > 2 || bad_dt(dtype) || bad_dt(gdtype) || gdtype == 1) return -1;
  if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1 || c0 < 0 || nc < 1 || c0 + nc > dv) return -2;
  if (!q || !k || !v || !log_a || (variant != OR_SSD && !beta)) return -3;
  long ntask = (long)B * H;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long task = 0; task < ntask; ++task) {
    int b = (int)(task / H), h = (int)(task % H);
    double* S = (double*)calloc((size_t)dk * nc, sizeof(double));
    double* kk = (double*)malloc(sizeof(double) * dk);
    double* qq = (double*)malloc(sizeof(double) * dk);
    double* aa = (double*)malloc(sizeof(double) * dk);
    double* vv = (double*)malloc(sizeof(double) * nc);
    if (!S || !kk || !qq || !aa || !vv) {
#pragma omp atomic write
      fail = 1;
      free(S); free(kk); free(qq); free(aa); free(vv);
      continue;
    }
    if (h0)
      for (int i = 0; i < dk; ++i)
        for (int c = 0; c < nc; ++c)
          S[(size_t)i * nc + c] = rd(h0, gdtype, (((size_t)b * H + h) * dk + i) * dv + c0 + c);
    for (int t = 0; t < T; ++t) {
      size_t row = ((size_t)b * T + t) * H + h; /* (b,t,h) */
      for (int i = 0; i < dk; ++i) {
        kk[i] = rd(k, dtype, row * dk + i);
        qq[i] = rd(q, dtype, row * dk + i);
      }
      for (int c = 0; c < nc; ++c) vv[c] = rd(v, dtype, row * dv + c0 + c);
      if (variant == OR_KDA) {
        for (int i = 0; i < dk; ++i) aa[i] = exp(rd(log_a, gdtype, row * dk + i));
      } else {
        double a = exp(rd(log_a, gdtype, row));
        for (int i = 0; i < dk; ++i) aa[i] = a;
      }
      double bt = variant == OR_SSD ? 1.0 : rd(beta, gdtype, row);
      for (int c = 0; c < nc; ++c) {
        /* decay, then (for the delta variants) read the decayed state at k */
        double xk = 0.0;
        for (int i = 0; i < dk; ++i) {
          S[(size_t)i * nc + c] *= aa[i];
          xk += S[(size_t)i * nc + c] * kk[i];
        }
        double u = variant == OR_SSD ? vv[c] : bt * (vv[c] - xk);
        double oc = 0.0;
        for (int i = 0; i < dk; ++i) {
          S[(size_t)i * nc + c] += kk[i] * u;
          oc += S[(size_t)i * nc + c] * qq[i];
        }
        if (o) o[row * nc + c] = oc;
      }
    }
    if (ht)
      for (int i = 0; i < dk; ++i)
        for (int c = 0; c < nc; ++c)
          ht[(((size_t)b * H + h) * dk + i) * nc + c] = S[(size_t)i * nc + c];
    free(S); free(kk); free(qq); free(aa); free(vv);
  }
  return fail ? -4 : 0;
}

/*
 * One token's step of the recurrence on a full [dk,dv] state, in place.
 * Used to rebuild the states of a segment during the backward.
 */
static void step_fwd(int variant, double* S, const double* kk, const double* aa, const double* vv,
                     double bt, int dk, int dv) {
  for (int c = 0; c < dv; ++c) {
    double xk = 0.0;
    for (int i = 0; i < dk; ++i) {
      S[(size_t)i * dv + c] *= aa[i];
      xk += S[(size_t)i * dv + c] * kk[i];
    }
    double u = variant == OR_SSD ? vv[c] : bt * (vv[c] - xk);
    for (int i = 0; i < dk; ++i) S[(size_t)i * dv + c] += kk[i] * u;
  }
}

/*
 * Backward by back-propagation through time.  G is the gradient of the loss
 * with respect to H_t; walking t = T..1:
 *   G += q_t do_t^T ;  dq_t = H_t do_t
 *   X = Diag(a_t) H_{t-1}  (a_t uniform over d_k for GDN/SSD)
 *   r = G^T k_t ;  xk = X^T k_t
 *   GDN/KDA:  dv_t = beta r ;  dbeta_t = r.(v_t - xk)
 *             dk_t = beta (G v_t - G xk - X r)
 *             dX = G - beta k_t r^T
 *   SSD:      dv_t = r ;  dk_t = G v_t ;  dX = G
 *   dlog_a_t[i] = a_t[i] * sum_c dX[i][c] H_{t-1}[i][c]   (summed over i for the
 *                 scalar-gate variants)
 *   G <- Diag(a_t) dX
 * and finally dh0 = G.
 * Gradient arrays have the layouts of the matching inputs; dlog_a is
 * [B,T,H] for GDN/SSD and [B,T,H,dk] for KDA; dbeta is ignored for SSD.
 */
int oracle_bwd(int variant, const void* q, const void* k, const void* v, int dtype,
               const void* log_a, const void* beta, const void* h0, int gdtype,
               const void* d_o, const void* dht,
               double* dq, double* dk_out, double* dv_out, double* dlog_a, double* dbeta,
               double* dh0, int B, int T, int H, int dk, int dv, int nthreads) {
  if (variant < 0 || variant > 2 || bad_dt(dtype) || bad_dt(gdtype) || gdtype == 1) return -1;
  if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return -2;
  if (!q || !k || !v || !log_a || !d_o || (variant != OR_SSD && !beta)) return -3;
  long ntask = (long)B * H;
  int nseg = (T + SEG - 1) / SEG;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long task = 0; task < ntask; ++task) {
    int b = (int)(task / H), h = (int)(task % H);
    size_t st = (size_t)dk * dv;
    /* checkpoints: state before each segment; seg states: H_{s-1} .. H_{e} */
    double* ck = (double*)malloc(sizeof(double) * st * (size_t)(nseg + 1));
    double* hs = (double*)malloc(sizeof(double) * st * (SEG + 1));
    double* G = (double*)calloc(st, sizeof(double));
    double* dX = (double*)malloc(sizeof(double) * st);
    double* kk = (double*)malloc(sizeof(double) * dk);
    double* qq = (double*)malloc(sizeof(double) * dk);
    double* aa = (double*)malloc(sizeof(double) * dk);
    double* vv = (double*)malloc(sizeof(double) * dv);
    double* dd = (double*)malloc(sizeof(double) * dv);
    double* r = (double*)malloc(sizeof(double) * dv);
    double* xk = (double*)malloc(sizeof(double) * dv);
    if (!ck || !hs || !G || !dX || !kk || !qq || !aa || !vv || !dd || !r || !xk) {
#pragma omp atomic write
      fail = 1;
      free(ck); free(hs); free(G); free(dX); free(kk); free(qq); free(aa); free(vv);
      free(dd); free(r); free(xk);
      continue;
    }
#define LOAD_TOKEN(t)                                                                 \
  do {                                                                                \
    size_t row_ = ((size_t)b * T + (t)) * H + h;                                      \
    for (int i = 0; i < dk; ++i) {                                                    \
      kk[i] = rd(k, dtype, row_ * dk + i);                                            \
      qq[i] = rd(q, dtype, row_ * dk + i);                                            \
    }                                                                                 \
    for (int c = 0; c < dv; ++c) {                                                    \
      vv[c] = rd(v, dtype, row_ * dv + c);                                            \
      dd[c] = rd(d_o, dtype, row_ * dv + c);                                          \
    }                                                                                 \
    if (variant == OR_KDA) {                                                          \
      for (int i = 0; i < dk; ++i) aa[i] = exp(rd(log_a, gdtype, row_ * dk + i));     \
    } else {                                                                          \
      double a_ = exp(rd(log_a, gdtype, row_));                                       \
      for (int i = 0; i < dk; ++i) aa[i] = a_;                                        \
    }                                                                                 \
    bt = variant == OR_SSD ? 1.0 : rd(beta, gdtype, row_);                            \
  } while (0)

    double bt = 1.0;
    /* forward: record the state at the start of every segment */
    memset(ck, 0, sizeof(double) * st);
    if (h0)
      for (size_t e = 0; e < st; ++e) ck[e] = rd(h0, gdtype, ((size_t)b * H + h) * st + e);
    for (int s = 0; s < nseg; ++s) {
      memcpy(ck + (size_t)(s + 1) * st, ck + (size_t)s * st, sizeof(double) * st);
      int t1 = (s + 1) * SEG < T ? (s + 1) * SEG : T;
      for (int t = s * SEG; t < t1; ++t) {
        LOAD_TOKEN(t);
        step_fwd(variant, ck + (size_t)(s + 1) * st, kk, aa, vv, bt, dk, dv);
      }
    }
    if (dht)
      for (size_t e = 0; e < st; ++e) G[e] = rd(dht, gdtype, ((size_t)b * H + h) * st + e);
    /* backward, one segment at a time, latest first */
    for (int s = nseg - 1; s >= 0; --s) {
      int t0 = s * SEG, t1 = (s + 1) * SEG < T ? (s + 1) * SEG : T;
      memcpy(hs, ck + (size_t)s * st, sizeof(double) * st);
      for (int t = t0; t < t1; ++t) {
        LOAD_TOKEN(t);
        memcpy(hs + (size_t)(t - t0 + 1) * st, hs + (size_t)(t - t0) * st, sizeof(double) * st);
        step_fwd(variant, hs + (size_t)(t - t0 + 1) * st, kk, aa, vv, bt, dk, dv);
      }
      for (int t = t1 - 1; t >= t0; --t) {
        LOAD_TOKEN(t);
        size_t row = ((size_t)b * T + t) * H + h;
        const double* Hc = hs + (size_t)(t - t0 + 1) * st; /* H_t */
        const double* Hp = hs + (size_t)(t - t0) * st;     /* H_{t-1} */
        /* o_t = H_t^T q_t */
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int c = 0; c < dv; ++c) {
            G[(size_t)i * dv + c] += qq[i] * dd[c];
            acc += Hc[(size_t)i * dv + c] * dd[c];
          }
          if (dq) dq[row * dk + i] = acc;
        }
        for (int c = 0; c < dv; ++c) {
          double rc = 0.0, xc = 0.0;
          for (int i = 0; i < dk; ++i) {
            rc += G[(size_t)i * dv + c] * kk[i];
            xc += aa[i] * Hp[(size_t)i * dv + c] * kk[i];
          }
          r[c] = rc;
          xk[c] = xc;
        }
        if (variant == OR_SSD) {
          for (int c = 0; c < dv; ++c)
            if (dv_out) dv_out[row * dv + c] = r[c];
          for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int c = 0; c < dv; ++c) acc += G[(size_t)i * dv + c] * vv[c];
            if (dk_out) dk_out[row * dk + i] = acc;
          }
          memcpy(dX, G, sizeof(double) * st);
        } else {
          double db = 0.0;
          for (int c = 0; c < dv; ++c) {
            if (dv_out) dv_out[row * dv + c] = bt * r[c];
            db += r[c] * (vv[c] - xk[c]);
          }
          if (dbeta) dbeta[row] = db;
          for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int c = 0; c < dv; ++c)
              acc += G[(size_t)i * dv + c] * (vv[c] - xk[c]) - aa[i] * Hp[(size_t)i * dv + c] * r[c];
            if (dk_out) dk_out[row * dk + i] = bt * acc;
          }
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c)
              dX[(size_t)i * dv + c] = G[(size_t)i * dv + c] - bt * kk[i] * r[c];
        }
        double ga = 0.0;
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int c = 0; c < dv; ++c) acc += dX[(size_t)i * dv + c] * Hp[(size_t)i * dv + c];
          acc *= aa[i];
          if (variant == OR_KDA) {
            if (dlog_a) dlog_a[row * dk + i] = acc;
          } else {
            ga += acc;
          }
          for (int c = 0; c < dv; ++c) G[(size_t)i * dv + c] = aa[i] * dX[(size_t)i * dv + c];
        }
        if (variant != OR_KDA && dlog_a) dlog_a[row] = ga;
      }
    }
    if (dh0) memcpy(dh0 + ((size_t)b * H + h) * st, G, sizeof(double) * st);
#undef LOAD_TOKEN
    free(ck); free(hs); free(G); free(dX); free(kk); free(qq); free(aa); free(vv);
    free(dd); free(r); free(xk);
  }
  return fail ? -4 : 0;
}

/* Threads the OpenMP runtime will use (for the CPU-baseline report). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
