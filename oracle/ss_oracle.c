/* CPU oracle for the Mamba-1 selective scan (forward and backward).
 *
 * TEST INFRASTRUCTURE ONLY.  It exists to check the HIP library; only the
 * tests, the smoke check and the bench's CPU-baseline leg may load it.  It
 * shares no code with the HIP path.
 *
 * A plain sequential loop over time per channel (b, d), in double precision
 * with libm exp / log1p, threaded over blocks of channels d.  The forward
 * follows the "Algorithm summary" of the baracuda-kernels page
 * "src/attention/selective_scan.rs":
 *
 *     delta_eff = softplus(delta[t,d] + delta_bias[d])   (softplus optional)
 *     a         = exp(delta_eff * A[d,n])
 *     h[n]      = a * h[n] + delta_eff * B[t,n] * u[t,d]   (h = h0 or 0 before t = 0)
 *     y[t,d]    = sum_n C[t,n] h[n]  (+ D[d] u[t,d])  (* silu(z[t,d]))
 *     last_state[b,d,:] = h after the last step
 *
 * Reductions across threads (dB and dC are sums over d) add the per-thread
 * parts in thread order, so results are deterministic for a fixed thread
 * count.  Every function returns 0 on success, nonzero on bad arguments or
 * allocation failure.
 *
 * A second build of the same loop in float ("_f32" entry points) gives the
 * rounding floor a straightforward single-precision implementation reaches.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t batch, seqlen, dim, dstate;
  int32_t delta_softplus;
} ss_oracle_problem;

#define REAL double
#define FN(name) name##_f64
#include "ss_oracle_impl.h"
#undef REAL
#undef FN
#define REAL float
#define FN(name) name##_f32
#include "ss_oracle_impl.h"
#undef REAL
#undef FN

static int clamp_threads(int nthreads, int64_t work) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (work < nthreads) nthreads = work > 0 ? (int)work : 1;
  return nthreads;
}

static int valid(const ss_oracle_problem* p) {
  return p && p->batch >= 0 && p->seqlen >= 0 && p->dim >= 0 && p->dstate >= 0;
}

/* ---------------------------------------------------------------- forward */

#define DEFINE_FWD(REALT, SUF)                                                             \
  typedef struct {                                                                         \
    const ss_oracle_problem* p;                                                            \
    const REALT *u, *delta, *A, *Bm, *Cm, *Dskip, *z, *bias, *h0;                          \
    REALT *y, *last_state;                                                                 \
    const int64_t *chan_b, *chan_d; /* subset mode when non-NULL */                        \
    int64_t c0, c1;                 /* channel range: (b*D + d) or subset index */         \
    int status;                                                                            \
  } fwd_job_##SUF;                                                                         \
  static void* fwd_worker_##SUF(void* arg) {                                               \
    fwd_job_##SUF* j = (fwd_job_##SUF*)arg;                                                \
    const ss_oracle_problem* p = j->p;                                                     \
    REALT* h = (REALT*)malloc(sizeof(REALT) * (size_t)(p->dstate > 0 ? p->dstate : 1));    \
    if (!h) { j->status = 1; return NULL; }                                                \
    for (int64_t c = j->c0; c < j->c1; ++c) {                                              \
      if (j->chan_b) {                                                                     \
        const REALT* h0r = j->h0 ? j->h0 + (j->chan_b[c] * p->dim + j->chan_d[c]) * p->dstate \
                                 : NULL;                                                   \
        fwd_channel_##SUF(p, j->u, j->delta, j->A, j->Bm, j->Cm, j->Dskip, j->z, j->bias,   \
                          h0r, j->chan_b[c], j->chan_d[c], j->y + c * p->seqlen, 1,        \
                          j->last_state ? j->last_state + c * p->dstate : NULL, h);        \
      } else {                                                                             \
        int64_t b = c / p->dim, d = c % p->dim;                                            \
        fwd_channel_##SUF(p, j->u, j->delta, j->A, j->Bm, j->Cm, j->Dskip, j->z, j->bias,   \
                          j->h0 ? j->h0 + c * p->dstate : NULL,                            \
                          b, d, j->y + b * p->seqlen * p->dim + d, p->dim,                 \
                          j->last_state ? j->last_state + (b * p->dim + d) * p->dstate     \
                                        : NULL,                                            \
                          h);                                                              \
      }                                                                                    \
    }                                                                                      \
    free(h);                                                                               \
    return NULL;                                                                           \
  }                                                                                        \
  static int run_fwd_##SUF(const ss_oracle_problem* p, const REALT* u, const REALT* delta, \
                           const REALT* A, const REALT* Bm, const REALT* Cm,               \
                           const REALT* Dskip, const REALT* z, const REALT* bias,          \
                           const REALT* h0, REALT* y, REALT* last_state,                   \
                           const int64_t* chan_b, const int64_t* chan_d, int64_t nchan,    \
                           int nthreads) {                                                 \
    if (!valid(p)) return 1;                                                               \
    if (nchan == 0) return 0;                                                              \
    if (!u || !delta || !A || !Bm || !Cm || !y) return 1;                                  \
    nthreads = clamp_threads(nthreads, nchan);                                             \
    fwd_job_##SUF jobs[256];                                                               \
    pthread_t tid[256];                                                                    \
    int started[256];                                                                      \
    for (int i = 0; i < nthreads; ++i) {                                                   \
      fwd_job_##SUF jb = {p,     u,     delta,      A,      Bm,     Cm,                    \
                          Dskip, z,     bias,       h0,     y,      last_state,            \
                          chan_b, chan_d, nchan * i / nthreads, nchan * (i + 1) / nthreads, \
                          0};                                                              \
      jobs[i] = jb;                                                                        \
    }                                                                                      \
    for (int i = 1; i < nthreads; ++i)                                                     \
      started[i] = pthread_create(&tid[i], NULL, fwd_worker_##SUF, &jobs[i]) == 0;         \
    fwd_worker_##SUF(&jobs[0]);                                                            \
    int st = jobs[0].status;                                                               \
    for (int i = 1; i < nthreads; ++i) {                                                   \
      if (started[i]) pthread_join(tid[i], NULL);                                          \
      else fwd_worker_##SUF(&jobs[i]);                                                     \
      st |= jobs[i].status;                                                                \
    }                                                                                      \
    return st;                                                                             \
  }

DEFINE_FWD(double, f64)
DEFINE_FWD(float, f32)

/* Full forward: y [B, L, D]; h0 [B, D, N] or NULL (zero initial state);
 * last_state [B, D, N] or NULL. */
int ss_oracle_fwd_f64(const ss_oracle_problem* p, const double* u, const double* delta,
                      const double* A, const double* Bm, const double* Cm, const double* Dskip,
                      const double* z, const double* bias, const double* h0, double* y,
                      double* last_state, int nthreads) {
  if (!valid(p)) return 1;
  return run_fwd_f64(p, u, delta, A, Bm, Cm, Dskip, z, bias, h0, y, last_state, NULL, NULL,
                     p->batch * p->dim, nthreads);
}

int ss_oracle_fwd_f32(const ss_oracle_problem* p, const float* u, const float* delta,
                      const float* A, const float* Bm, const float* Cm, const float* Dskip,
                      const float* z, const float* bias, const float* h0, float* y,
                      float* last_state, int nthreads) {
  if (!valid(p)) return 1;
  return run_fwd_f32(p, u, delta, A, Bm, Cm, Dskip, z, bias, h0, y, last_state, NULL, NULL,
                     p->batch * p->dim, nthreads);
}

/* Forward of a list of channels (chan_b[c], chan_d[c]), c < nchan.
 * h0: [B, D, N] or NULL; y_out: [nchan, L]; ls_out: [nchan, N] or NULL. */
int ss_oracle_fwd_channels_f64(const ss_oracle_problem* p, const double* u, const double* delta,
                               const double* A, const double* Bm, const double* Cm,
                               const double* Dskip, const double* z, const double* bias,
                               const double* h0, const int64_t* chan_b, const int64_t* chan_d,
                               int64_t nchan, double* y_out, double* ls_out, int nthreads) {
  if (!valid(p) || nchan < 0 || (nchan > 0 && (!chan_b || !chan_d))) return 1;
  for (int64_t c = 0; c < nchan; ++c)
    if (chan_b[c] < 0 || chan_b[c] >= p->batch || chan_d[c] < 0 || chan_d[c] >= p->dim)
      return 1;
  return run_fwd_f64(p, u, delta, A, Bm, Cm, Dskip, z, bias, h0, y_out, ls_out, chan_b,
                     chan_d, nchan, nthreads);
}

/* --------------------------------------------------------------- backward */

#define DEFINE_BWD(REALT, SUF)                                                             \
  typedef struct {                                                                         \
    const ss_oracle_problem* p;                                                            \
    const REALT *u, *delta, *A, *Bm, *Cm, *Dskip, *z, *bias, *h0, *dy;                     \
    REALT *du, *ddelta, *dA, *dB_part, *dC_part, *dD, *dz, *dbias, *dh0;                   \
    int64_t d0, d1;                                                                        \
    int status;                                                                            \
  } bwd_job_##SUF;                                                                         \
  static void* bwd_worker_##SUF(void* arg) {                                               \
    bwd_job_##SUF* j = (bwd_job_##SUF*)arg;                                                \
    const ss_oracle_problem* p = j->p;                                                     \
    size_t L = (size_t)p->seqlen, N = (size_t)(p->dstate > 0 ? p->dstate : 1);             \
    REALT* hist = (REALT*)malloc(sizeof(REALT) * (L + 1) * N);                             \
    REALT* ahist = (REALT*)malloc(sizeof(REALT) * (L + 1) * N);                            \
    REALT* dls = (REALT*)malloc(sizeof(REALT) * (L + 1));                                  \
    REALT* xs = (REALT*)malloc(sizeof(REALT) * (L + 1));                                   \
    REALT* os = (REALT*)malloc(sizeof(REALT) * (L + 1));                                   \
    REALT* dh = (REALT*)malloc(sizeof(REALT) * N);                                         \
    if (!hist || !ahist || !dls || !xs || !os || !dh) {                                    \
      j->status = 1;                                                                       \
    } else {                                                                               \
      bwd_range_##SUF(p, j->u, j->delta, j->A, j->Bm, j->Cm, j->Dskip, j->z, j->bias,       \
                      j->h0, j->dy, j->du, j->ddelta, j->dA, j->dB_part, j->dC_part,       \
                      j->dD, j->dz, j->dbias, j->dh0, j->d0, j->d1, hist, ahist, dls, xs,  \
                      os, dh);                                                             \
    }                                                                                      \
    free(hist); free(ahist); free(dls); free(xs); free(os); free(dh);                      \
    return NULL;                                                                           \
  }                                                                                        \
  int ss_oracle_bwd_##SUF(const ss_oracle_problem* p, const REALT* u, const REALT* delta,  \
                          const REALT* A, const REALT* Bm, const REALT* Cm,                \
                          const REALT* Dskip, const REALT* z, const REALT* bias,           \
                          const REALT* h0, const REALT* dy, REALT* du, REALT* ddelta,      \
                          REALT* dA, REALT* dB, REALT* dC, REALT* dD, REALT* dz,           \
                          REALT* dbias, REALT* dh0, int nthreads) {                        \
    if (!valid(p)) return 1;                                                               \
    const int64_t B = p->batch, L = p->seqlen, D = p->dim, N = p->dstate;                  \
    if (!u || !delta || !A || !Bm || !Cm || !dy || !du || !ddelta || !dA || !dB || !dC)    \
      return 1;                                                                            \
    if ((!Dskip) != (!dD) || (!z) != (!dz) || (!bias) != (!dbias) || (!h0) != (!dh0))     \
      return 1;                                                                            \
    if (dh0) /* with L = 0 the loss does not depend on h0 */                              \
      memset(dh0, 0, sizeof(REALT) * (size_t)(B * D * N));                                 \
    const size_t bln = (size_t)(B * L * N);                                                \
    memset(dB, 0, sizeof(REALT) * bln);                                                    \
    memset(dC, 0, sizeof(REALT) * bln);                                                    \
    memset(dA, 0, sizeof(REALT) * (size_t)(D * N));                                        \
    if (dD) memset(dD, 0, sizeof(REALT) * (size_t)D);                                      \
    if (dbias) memset(dbias, 0, sizeof(REALT) * (size_t)D);                                \
    if (D == 0 || B == 0 || L == 0) return 0;                                              \
    nthreads = clamp_threads(nthreads, D);                                                 \
    REALT* parts = (REALT*)calloc((size_t)nthreads * 2 * (bln ? bln : 1), sizeof(REALT));  \
    if (!parts) return 1;                                                                  \
    bwd_job_##SUF jobs[256];                                                               \
    pthread_t tid[256];                                                                    \
    int started[256];                                                                      \
    for (int i = 0; i < nthreads; ++i) {                                                   \
      bwd_job_##SUF jb = {p,  u,      delta, A,  Bm,                                       \
                          Cm, Dskip,  z,     bias, h0, dy,                                 \
                          du, ddelta, dA,    parts + (size_t)(2 * i) * bln,                \
                          parts + (size_t)(2 * i + 1) * bln, dD, dz, dbias, dh0,           \
                          D * i / nthreads, D * (i + 1) / nthreads, 0};                    \
      jobs[i] = jb;                                                                        \
    }                                                                                      \
    for (int i = 1; i < nthreads; ++i)                                                     \
      started[i] = pthread_create(&tid[i], NULL, bwd_worker_##SUF, &jobs[i]) == 0;         \
    bwd_worker_##SUF(&jobs[0]);                                                            \
    int st = jobs[0].status;                                                               \
    for (int i = 1; i < nthreads; ++i) {                                                   \
      if (started[i]) pthread_join(tid[i], NULL);                                          \
      else bwd_worker_##SUF(&jobs[i]);                                                     \
      st |= jobs[i].status;                                                                \
    }                                                                                      \
    for (int i = 0; i < nthreads; ++i) /* fixed order: thread 0, 1, ... */                 \
      for (size_t k = 0; k < bln; ++k) {                                                   \
        dB[k] += parts[(size_t)(2 * i) * bln + k];                                         \
        dC[k] += parts[(size_t)(2 * i + 1) * bln + k];                                     \
      }                                                                                    \
    free(parts);                                                                           \
    return st;                                                                             \
  }

/* Full backward.  Saved forward inputs (h0 [B, D, N] or NULL) plus dy
 * [B, L, D]; outputs du, ddelta, dz [B, L, D]; dB, dC [B, L, N]; dA [D, N];
 * dD, dbias [D]; dh0 [B, D, N].  dD / dz / dbias / dh0 must be given exactly
 * when Dskip / z / bias / h0 are.  Outputs are overwritten. */
DEFINE_BWD(double, f64)
DEFINE_BWD(float, f32)
