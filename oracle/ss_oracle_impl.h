/* Body of the CPU oracle, included twice by ss_oracle.c: once with REAL =
 * double (the oracle proper) and once with REAL = float (the "sequential f32
 * floor" diagnostic: the same loop, same order, in single precision).
 *
 * TEST INFRASTRUCTURE ONLY: nothing on the product path may call this.
 *
 * What it computes is the Mamba-1 selective scan as defined on the
 * baracuda-kernels page "src/attention/selective_scan.rs", module docs,
 * section "Algorithm summary" (forward), with the tensor shapes of its
 * "Shape contract" table, and the backward gradient set listed by that page's
 * SelectiveScanBackwardArgs (du, dB, dC, ddelta, dA, dD, dz, ddelta_bias).
 * The backward equations are not printed on any page; they are the exact
 * adjoint of the forward, obtained by the chain rule (the per-(b,d) reverse
 * sweep over time mirrors the mamba-rs page "mamba_ssm/gpu/backward.rs",
 * stage B3 "SSM BPTT + reductions").
 *
 * Requires macros: REAL, FN(name).
 */

/* softplus(x) = log(1 + e^x), evaluated without overflow. */
static REAL FN(softplus)(REAL x) {
  if (x > 0) return x + (REAL)log1p(exp(-(double)x));
  return (REAL)log1p(exp((double)x));
}

static REAL FN(sigmoid)(REAL x) { return (REAL)1 / ((REAL)1 + (REAL)exp(-(double)x)); }

/* Forward of one channel (b, d).  Writes y[b, t, d] for every t to
 * y_out[t * y_stride]; if ls_out is not NULL, writes the state after the last
 * step to ls_out[0 .. N-1].  h0_row: this channel's state before t = 0
 * ([N]), or NULL for zero (the carried per-layer state of the mamba-rs page
 * "mamba_ssm/gpu/backward.rs", whose forward pipeline runs the SSM from
 * carried states).  h: [N] scratch. */
static void FN(fwd_channel)(const ss_oracle_problem* p, const REAL* u, const REAL* delta,
                            const REAL* A, const REAL* Bm, const REAL* Cm, const REAL* Dskip,
                            const REAL* z, const REAL* bias, const REAL* h0_row, int64_t b,
                            int64_t d, REAL* y_out, int64_t y_stride, REAL* ls_out, REAL* h) {
  const int64_t L = p->seqlen, D = p->dim, N = p->dstate;
  for (int64_t n = 0; n < N; ++n) h[n] = h0_row ? h0_row[n] : 0;  /* state before t = 0 */
  for (int64_t t = 0; t < L; ++t) {
    const int64_t i = (b * L + t) * D + d;             /* [B, L, D] */
    const REAL* Bt = Bm + (b * L + t) * N;             /* [B, L, N] */
    const REAL* Ct = Cm + (b * L + t) * N;
    REAL x = delta[i] + (bias ? bias[d] : (REAL)0);
    REAL dl = p->delta_softplus ? FN(softplus)(x) : x;
    REAL o = 0;
    for (int64_t n = 0; n < N; ++n) {
      REAL a = (REAL)exp((double)(dl * A[d * N + n]));  /* A is [D, N] */
      h[n] = a * h[n] + dl * Bt[n] * u[i];
      o += Ct[n] * h[n];
    }
    if (Dskip) o += Dskip[d] * u[i];
    if (z) o = o * z[i] * FN(sigmoid)(z[i]);
    y_out[t * y_stride] = o;
  }
  if (ls_out)
    for (int64_t n = 0; n < N; ++n) ls_out[n] = h[n];
}

/* Backward for the channels d in [d0, d1), every b.
 * Per-channel outputs (du, ddelta, dz, dA, dD, dbias, dh0) are written
 * directly: each (d, *) belongs to exactly one range.  dB and dC are sums over
 * d, so this range accumulates into its own dB_part / dC_part ([B, L, N],
 * zeroed by the caller); the caller adds the ranges' parts in range order.
 * h0 / dh0: [B, D, N] state before t = 0 and its gradient, both NULL or both
 * given (dh0 = dL/dh_{-1}, what the reverse sweep carries past t = 0).
 * hist: [L + 1, N] scratch (h_{-1} .. h_{L-1}); ahist: [L, N]; dl/xs/os: [L]. */
static void FN(bwd_range)(const ss_oracle_problem* p, const REAL* u, const REAL* delta,
                          const REAL* A, const REAL* Bm, const REAL* Cm, const REAL* Dskip,
                          const REAL* z, const REAL* bias, const REAL* h0, const REAL* dy,
                          REAL* du, REAL* ddelta, REAL* dA, REAL* dB_part, REAL* dC_part,
                          REAL* dD, REAL* dz, REAL* dbias, REAL* dh0, int64_t d0, int64_t d1,
                          REAL* hist, REAL* ahist, REAL* dls, REAL* xs, REAL* os, REAL* dh) {
  const int64_t B = p->batch, L = p->seqlen, D = p->dim, N = p->dstate;
  for (int64_t d = d0; d < d1; ++d) {
    for (int64_t n = 0; n < N; ++n) dA[d * N + n] = 0;
    if (dD) dD[d] = 0;
    if (dbias) dbias[d] = 0;
  }
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t d = d0; d < d1; ++d) {
      /* forward, keeping every state, decay, delta and pre-gate output */
      for (int64_t n = 0; n < N; ++n)                  /* row 0 = h_{-1} */
        hist[n] = h0 ? h0[(b * D + d) * N + n] : 0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t i = (b * L + t) * D + d;
        const REAL* Bt = Bm + (b * L + t) * N;
        const REAL* Ct = Cm + (b * L + t) * N;
        REAL x = delta[i] + (bias ? bias[d] : (REAL)0);
        REAL dl = p->delta_softplus ? FN(softplus)(x) : x;
        xs[t] = x;
        dls[t] = dl;
        REAL o = 0;
        for (int64_t n = 0; n < N; ++n) {
          REAL a = (REAL)exp((double)(dl * A[d * N + n]));
          ahist[t * N + n] = a;
          hist[(t + 1) * N + n] = a * hist[t * N + n] + dl * Bt[n] * u[i];
          o += Ct[n] * hist[(t + 1) * N + n];
        }
        if (Dskip) o += Dskip[d] * u[i];
        os[t] = o;                                     /* output before the gate */
      }
      /* reverse sweep; dh[n] holds a_{t+1} * dL/dh_{t+1} on entry to step t */
      for (int64_t n = 0; n < N; ++n) dh[n] = 0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t i = (b * L + t) * D + d;
        const REAL* Bt = Bm + (b * L + t) * N;
        const REAL* Ct = Cm + (b * L + t) * N;
        REAL g = dy[i];                                /* dL/d(pre-gate output) */
        if (z) {
          REAL s = FN(sigmoid)(z[i]);
          dz[i] = dy[i] * os[t] * s * ((REAL)1 + z[i] * ((REAL)1 - s));
          g = dy[i] * z[i] * s;
        }
        REAL dui = Dskip ? g * Dskip[d] : (REAL)0;
        if (Dskip) dD[d] += g * u[i];
        REAL ddl = 0;                                  /* dL/d(delta_eff) */
        for (int64_t n = 0; n < N; ++n) {
          const REAL a = ahist[t * N + n];
          const REAL hprev = hist[t * N + n];
          const REAL hcur = hist[(t + 1) * N + n];
          dh[n] += g * Ct[n];                          /* now dL/dh_t */
          dC_part[(b * L + t) * N + n] += g * hcur;
          const REAL ga = dh[n] * hprev;               /* dL/da_t */
          ddl += ga * a * A[d * N + n] + dh[n] * Bt[n] * u[i];
          dA[d * N + n] += ga * a * dls[t];
          dB_part[(b * L + t) * N + n] += dh[n] * dls[t] * u[i];
          dui += dh[n] * dls[t] * Bt[n];
          dh[n] *= a;
        }
        REAL dx = p->delta_softplus ? ddl * FN(sigmoid)(xs[t]) : ddl;
        ddelta[i] = dx;
        if (dbias) dbias[d] += dx;
        du[i] = dui;
      }
      if (dh0)                                         /* dh = a_0 dL/dh_0 = dL/dh_{-1} */
        for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = dh[n];
    }
  }
}
