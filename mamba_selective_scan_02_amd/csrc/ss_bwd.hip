// Backward (BPTT) selective scan kernels for gfx950.
//
// The gradient set is the one of SelectiveScanBackwardArgs on the
// baracuda-kernels page "src/attention/selective_scan.rs" (du, dB, dC,
// ddelta, dA, dD, dz, ddelta_bias).  The equations are the chain rule through
// the forward recurrence of that page's "Algorithm summary"; per channel, with
// g_t = dL/d(pre-gate output) = dy * silu(z) (or dy):
//   dh_t    = g_t C_t + a_{t+1} dh_{t+1}                (dh after L-1 is 0)
//   dC_t   += g_t h_t,   dB_t += dh_t dt_t u_t          (summed over d)
//   q_t     = dh_t a_t h_{t-1}                         (= dL/da_t * a_t)
//   ddt_t   = sum_n (q_t A_n + dh_t B_t u_t),  dA_n += q_t dt_t
//   du_t    = dt_t sum_n dh_t B_t + g_t D
//   ddelta_t = ddt_t * sigmoid(x_t) (softplus) or ddt_t,  ddelta_bias += ddelta_t
//   dz_t    = dy_t o_t s (1 + z_t (1 - s)),  s = sigmoid(z_t),  dD += g_t u_t
// The per-channel reverse sweep follows stage B3 "SSM BPTT + reductions" of the
// mamba-rs page "mamba_ssm/gpu/backward.rs"; the reductions there are
// per-channel partials followed by fixed-order reduction kernels, which is also
// the scheme here (no atomics anywhere, so every output is bitwise
// reproducible).
//
// Schedule.  Time is cut into chunks of at most kBwdTile = 8 steps (one
// register tile).
//  1. bwd_summary: per chunk, from zero: S (forward end state), Sb (the
//     adjoint the chunk hands to the step before it, sum_s (prod_{r<=s} a_r)
//     g_s C_s, accumulated forward with a running decay product) and sum dt.
//  2. bwd_carry: per (b, n, d) the forward chain h_in(k+1) = P_k h_in(k) + S_k
//     and the reverse chain c_{k-1} = P_k c_k + Sb_k, P_k = exp(A sum_k dt).
//  3. bwd_main: per chunk, one state n at a time: recompute the chunk's states
//     from h_in into registers, sweep back from c, accumulate the per-t sums
//     (ddt, du, o) in registers; dB and dC partials are summed over the 256
//     channels of the workgroup through LDS in a fixed order.
//  4. bwd_finalize: fixed-order sums of the partials (dB / dC and dA / dD /
//     ddelta_bias in one launch).
#include "ss_device.h"
#include "ss_plan.h"

namespace ss {

constexpr int T = kBwdTile;            // steps per chunk (max)
static_assert(4 * T <= 32, "two states' dB / dC rows fill the 32-row reduction buffer");
constexpr int kRedStride = 257;        // LDS row stride of the dB/dC reduction buffer

// Per-chunk inputs shared by all channels of a workgroup: B and C for the
// chunk's steps, as f32 in LDS, [n][t] with t fastest; steps beyond the chunk
// are zero (their dt is zero too, so they are identity steps).
template <typename Tio>
__device__ __forceinline__ void load_bc_tile(float* sB, float* sC, const Tio* B, const Tio* C,
                                             int64_t row0, int nt, int64_t N, int64_t ldb,
                                             int64_t ldc) {
  const int64_t total = N * T;
  for (int64_t idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int64_t tt = idx / N, n = idx % N;   // n fastest: coalesced global reads
    float bv = 0.0f, cv = 0.0f;
    if (tt < nt) {
      bv = ld(B, (row0 + tt) * ldb + n);
      cv = ld(C, (row0 + tt) * ldc + n);
    }
    sB[n * T + tt] = bv;
    sC[n * T + tt] = cv;
  }
}

// ---------------------------------------------------------------- summary

template <typename Tio>
__global__ __launch_bounds__(kChannelsPerBlock) void bwd_summary(const BwdArgs a) {
  extern __shared__ float smem[];
  float* sB = smem;
  float* sC = smem + a.N * T;
  const int64_t nbd = a.nwgd;
  int64_t blk = blockIdx.x;
  const int64_t db = blk % nbd;
  blk /= nbd;
  const int64_t k = blk % a.K;
  const int64_t b = blk / a.K;
  const int64_t D = a.D, N = a.N;
  const int64_t d_raw = db * kChannelsPerBlock + threadIdx.x;
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;
  const SeqRows sr = seq_rows(a.cu, b, a.L, a.Lt);
  const int64_t t0 = k * a.chunk_len;
  int nt = (int)((t0 + a.chunk_len < sr.len ? t0 + a.chunk_len : sr.len) - t0);
  if (nt < 0) nt = 0;                        // a chunk past a short sequence's end

  load_bc_tile(sB, sC, static_cast<const Tio*>(a.B), static_cast<const Tio*>(a.C),
               sr.start + t0, nt, N, a.ldb, a.ldc);

  const float bv = a.bias ? ld_param(a.bias, d, a.param_dtype) : 0.0f;
  const bool has_z = a.z != nullptr, sp = a.softplus != 0;
  const Tio* up = static_cast<const Tio*>(a.u) + d;           // + row * D
  const Tio* dp = static_cast<const Tio*>(a.delta) + d;
  const Tio* zp = has_z ? static_cast<const Tio*>(a.z) + d : up;
  const Tio* yp = static_cast<const Tio*>(a.dy) + d;
  float dl[T], xu[T], gg[T];
  float dsum = 0.0f;
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    const bool ok = tt < nt;
    // past the chunk: a step of it, or row 0 for an empty chunk (never used)
    const int64_t t = nt > 0 ? sr.start + t0 + (ok ? tt : nt - 1) : 0;
    const float uu = ld(up, t * D), x = ld(dp, t * D) + bv;
    const float dlv = sp ? softplus_acc(x) : x;
    float g = ld(yp, t * D);
    if (has_z) { const float zz = ld(zp, t * D); g *= zz * sigmoid(zz); }
    dl[tt] = ok ? dlv : 0.0f;
    xu[tt] = ok ? dlv * uu : 0.0f;
    gg[tt] = ok ? g : 0.0f;
    dsum += dl[tt];
  }
  __syncthreads();

  // each state's A loaded one state ahead (a load at the top of the
  // iteration would hold the state's whole update chain)
  float nA = N > 0 ? ld_param(a.A, d * N, a.param_dtype) : 0.0f;
  for (int64_t n = 0; n < N; ++n) {
    const float A2 = nA * kLog2e;
    nA = ld_param(a.A, d * N + (n + 1 < N ? n + 1 : n), a.param_dtype);
    const float* bn = sB + n * T;
    const float* cn = sC + n * T;
    float h = 0.0f, E = 1.0f, Sb = 0.0f;
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const float av = fast_exp2(dl[tt] * A2);
      h = __builtin_fmaf(av, h, xu[tt] * bn[tt]);
      E *= av;
      Sb = __builtin_fmaf(E, gg[tt] * cn[tt], Sb);
    }
    if (active) {
      const int64_t o = ((b * a.K + k) * N + n) * D + d;
      a.fstate[o] = h;
      a.bstate[o] = Sb;
    }
  }
  if (active) a.dsum[(b * a.K + k) * D + d] = dsum;
}

// ------------------------------------------------------------------ carry

// One chain per (direction, b, n, d), G lanes each (carry_chain's in-wave
// scan), 256 / G chains (consecutive d) per workgroup: the forward chain over
// k = 0 .. K-2 (fstate slot k becomes the state entering chunk k+1) and the
// reverse chain over k = K-1 .. 1 (bstate slot k becomes the adjoint at the
// end of chunk k-1, c_{k-1} = P_k c_k + Sb_k).
template <int G>
__global__ __launch_bounds__(kChannelsPerBlock) void bwd_carry(const BwdArgs a) {
  constexpr int CPB = kChannelsPerBlock / G;
  const int64_t nbd = (a.D + CPB - 1) / CPB;
  int64_t blk = blockIdx.x;
  const int64_t db = blk % nbd;
  blk /= nbd;
  const int64_t n = blk % a.N;
  blk /= a.N;
  const int64_t b = blk % a.Bn;
  const bool reverse = blk / a.Bn != 0;
  const int64_t d = db * CPB + threadIdx.x / G;
  if (d >= a.D) return;                      // the chain's lanes leave together
  const int64_t D = a.D, N = a.N, K = a.K;
  const float Av = ld_param(a.A, d * N + n, a.param_dtype);
  float* st = (reverse ? a.bstate : a.fstate) + (b * K * N + n) * D + d;   // + k * N * D
  const double c0 = (!reverse && a.h0) ? ld_param(a.h0, (b * D + d) * N + n, a.param_dtype) : 0.0;
  carry_chain<G>(st, N * D, a.dsum + b * K * D + d, D, Av, c0, K - 1, K, reverse);
}

// ------------------------------------------------------------------- main

template <typename Tio>
__global__ __launch_bounds__(kChannelsPerBlock) void bwd_main(const BwdArgs a) {
  extern __shared__ float smem[];
  float* sB = smem;
  float* sC = smem + a.N * T;
  float* red = smem + 2 * a.N * T;  // [32][kRedStride]: 4T rows (two states) used
  const int tid = threadIdx.x;
  const int64_t nbd = a.nwgd;
  int64_t blk = blockIdx.x;
  const int64_t db = blk % nbd;
  blk /= nbd;
  const int64_t kg = blk % a.KG;
  const int64_t b = blk / a.KG;
  const int64_t D = a.D, N = a.N, K = a.K;
  const SeqRows sr = seq_rows(a.cu, b, a.L, a.Lt);
  const int64_t d_raw = db * kChannelsPerBlock + tid;
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;
  const float bv = a.bias ? ld_param(a.bias, d, a.param_dtype) : 0.0f;
  const float Dv = a.Dskip ? ld_param(a.Dskip, d, a.param_dtype) : 0.0f;
  const bool has_z = a.z != nullptr, has_D = a.Dskip != nullptr, sp = a.softplus != 0;
  const Tio* up = static_cast<const Tio*>(a.u) + d;           // + row * D
  const Tio* dp = static_cast<const Tio*>(a.delta) + d;
  const Tio* zp = has_z ? static_cast<const Tio*>(a.z) + d : up;
  const Tio* yp = static_cast<const Tio*>(a.dy) + d;
  Tio* dup = static_cast<Tio*>(a.du) + d;
  Tio* ddp = static_cast<Tio*>(a.ddelta) + d;
  Tio* dzp = has_z ? static_cast<Tio*>(a.dz) + d : dup;

  // reduction lane roles: value v (per state of a round: T of dB, T of dC),
  // channel slice p
  const int rv = tid >> 3, rp = tid & 7;
  float dD_acc = 0.0f, db_acc = 0.0f;
  const int64_t k_lo = kg * kBwdChunksPerGroup;
  const int64_t k_hi = (k_lo + kBwdChunksPerGroup < K) ? k_lo + kBwdChunksPerGroup : K;

  for (int64_t k = k_hi - 1; k >= k_lo; --k) {
    const int64_t t0 = k * a.chunk_len;
    int nt = (int)((t0 + a.chunk_len < sr.len ? t0 + a.chunk_len : sr.len) - t0);
    if (nt < 0) nt = 0;                      // a chunk past a short sequence's end
    __syncthreads();  // previous chunk's tile readers are done
    load_bc_tile(sB, sC, static_cast<const Tio*>(a.B), static_cast<const Tio*>(a.C),
                 sr.start + t0, nt, N, a.ldb, a.ldc);

    float uu[T], dl[T], xu[T], gg[T], gz[T], sx[T], oo[T], ddl[T], dua[T];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const bool ok = tt < nt;
      const int64_t t = nt > 0 ? sr.start + t0 + (ok ? tt : nt - 1) : 0;   // row
      const float u_ = ld(up, t * D), x = ld(dp, t * D) + bv, dy = ld(yp, t * D);
      float dlv, sxv;
      if (sp) { dlv = softplus_acc(x); sxv = sigmoid_acc(x); } else { dlv = x; sxv = 1.0f; }
      float g = dy, gzv = 0.0f;
      if (has_z) {
        const float zz = ld(zp, t * D), s = sigmoid(zz);
        g = dy * zz * s;
        gzv = dy * s * __builtin_fmaf(zz, 1.0f - s, 1.0f);
      }
      uu[tt] = ok ? u_ : 0.0f;
      dl[tt] = ok ? dlv : 0.0f;
      xu[tt] = ok ? dlv * u_ : 0.0f;
      gg[tt] = ok ? g : 0.0f;
      gz[tt] = gzv;
      sx[tt] = sxv;
      oo[tt] = 0.0f;
      ddl[tt] = 0.0f;
      dua[tt] = 0.0f;
    }
    __syncthreads();  // tile visible

    // each state's A, carried-in state and carried adjoint, loaded one state
    // ahead (the loop's barriers would otherwise leave each state waiting for
    // its own loads)
    auto state_in = [&](int64_t n, float& An_, float& hin_, float& dh_) {
      const int64_t nn = n < N ? n : N - 1;
      An_ = ld_param(a.A, d * N + nn, a.param_dtype);
      hin_ = (k > 0)  ? a.fstate[((b * K + (k - 1)) * N + nn) * D + d]
             : a.h0   ? ld_param(a.h0, (b * D + d) * N + nn, a.param_dtype)
                      : 0.0f;
      dh_ = (k < K - 1) ? a.bstate[((b * K + (k + 1)) * N + nn) * D + d] : 0.0f;
    };
    float nA = 0.0f, nh = 0.0f, nd = 0.0f;
    if (N > 0) state_in(0, nA, nh, nd);
    for (int64_t n = 0; n < N; ++n) {
      const float An = nA;
      const float A2 = An * kLog2e;
      const float hin = nh;
      float dh = nd;
      state_in(n + 1, nA, nh, nd);
      const float* bn = sB + n * T;
      const float* cn = sC + n * T;
      float hs[T], ah[T];
      float hp = hin;
#pragma unroll
      for (int tt = 0; tt < T; ++tt) {
        const float av = fast_exp2(dl[tt] * A2);
        hp = __builtin_fmaf(av, hp, xu[tt] * bn[tt]);
        hs[tt] = hp;
        ah[tt] = av;
        oo[tt] = __builtin_fmaf(cn[tt], hp, oo[tt]);
      }
      float vB[T], vC[T];
      float dA_acc = 0.0f;
#pragma unroll
      for (int tt = T - 1; tt >= 0; --tt) {
        dh = __builtin_fmaf(gg[tt], cn[tt], dh);         // dL/dh_t
        vC[tt] = gg[tt] * hs[tt];
        vB[tt] = dh * xu[tt];
        dua[tt] = __builtin_fmaf(dh, bn[tt], dua[tt]);
        const float m = dh * ah[tt];
        const float q = m * (tt > 0 ? hs[tt - 1] : hin);
        ddl[tt] = __builtin_fmaf(q, An, ddl[tt]);
        dA_acc = __builtin_fmaf(q, dl[tt], dA_acc);
        dh = m;
      }
      if (active) {
        float* pa = a.part_dA + ((b * a.KG + kg) * N + n) * D + d;
        *pa = (k == k_hi - 1) ? dA_acc : *pa + dA_acc;
        // after step 0 of chunk 0, dh is dL/dh_{-1}
        if (k == 0 && a.dh0) st_param(a.dh0, (b * D + d) * N + n, a.param_dtype, dh);
      }
      // dB / dC for this n: sum over the workgroup's channels in LDS, two
      // states per round (rows [2T * (n % 2), 2T * (n % 2) + 2T) of red:
      // T of dB, then T of dC).  Inactive (tail) lanes contribute zero.
      const int half = (int)(n & 1) * 2 * T;
#pragma unroll
      for (int tt = 0; tt < T; ++tt) {
        red[(half + tt) * kRedStride + tid] = active ? vB[tt] : 0.0f;
        red[(half + T + tt) * kRedStride + tid] = active ? vC[tt] : 0.0f;
      }
      if ((n & 1) == 0 && n + 1 < N) continue;   // the round's second state first
      __syncthreads();
      // 4T values (two states), 8 threads each; rows rv >= 4T are unused
      const int64_t nb = n & ~int64_t(1);        // the round's first state
      const int rows = (n & 1) ? 4 * T : 2 * T;  // an odd last state rounds alone
      float s = 0.0f;
      if (rv < rows) {
#pragma unroll
        for (int i = 0; i < 32; ++i) s += red[rv * kRedStride + rp * 32 + ((i + 8 * rp) & 31)];
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if (rp == 0 && rv < rows) {
        const int ns = rv / (2 * T), w = rv % (2 * T);
        const int tt = w % T, which = w / T;
        if (tt < nt)
          a.part_bc[((sr.start + t0 + tt) * a.nwgd + db) * 2 * N + which * N + nb + ns] = s;
      }
      __syncthreads();  // red free for the next round
    }

#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      if (tt < nt && active) {
        const int64_t t = sr.start + t0 + tt;   // row
        const float du = __builtin_fmaf(dl[tt], dua[tt], has_D ? gg[tt] * Dv : 0.0f);
        const float dde = __builtin_fmaf(uu[tt], dua[tt], ddl[tt]);
        const float dx = dde * sx[tt];
        dup[t * D] = from_f32<Tio>(du);
        ddp[t * D] = from_f32<Tio>(dx);
        if (has_z) dzp[t * D] = from_f32<Tio>(gz[tt] * __builtin_fmaf(Dv, uu[tt], oo[tt]));
        db_acc += dx;
        dD_acc = __builtin_fmaf(gg[tt], uu[tt], dD_acc);
      }
    }
  }
  if (active) {
    a.part_dD[(b * a.KG + kg) * D + d] = dD_acc;
    a.part_db[(b * a.KG + kg) * D + d] = db_acc;
  }
}

// --------------------------------------------------------------- finalize

// dB[b,t,n], dC[b,t,n] = sums over the channel blocks, in block order (loads
// are issued in batches of 16, the adds stay in index order).
template <typename Tio>
__device__ __forceinline__ void finalize_bc(const BwdArgs& a, int64_t i) {  // i = row * N + n
  const int64_t N = a.N;
  if (i >= a.Lt * N) return;
  const int64_t bt = i / N, n = i % N;
  const float* p = a.part_bc + bt * a.nwgd * 2 * N + n;
  float sb = 0.0f, sc = 0.0f;
  constexpr int U = 16;
  int64_t w = 0;
  for (; w + U <= a.nwgd; w += U) {
    float vb[U], vc[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      vb[j] = p[(w + j) * 2 * N];
      vc[j] = p[(w + j) * 2 * N + N];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) { sb += vb[j]; sc += vc[j]; }
  }
  for (; w < a.nwgd; ++w) {
    sb += p[w * 2 * N];
    sc += p[w * 2 * N + N];
  }
  static_cast<Tio*>(a.dB)[bt * a.ldb + n] = from_f32<Tio>(sb);
  static_cast<Tio*>(a.dC)[bt * a.ldc + n] = from_f32<Tio>(sc);
}

// Fixed-order sum of `count` partials p[0], p[stride], ... (loads batched).
__device__ __forceinline__ float ordered_sum(const float* p, int64_t count, int64_t stride) {
  float s = 0.0f;
  constexpr int U = 16;
  int64_t j = 0;
  for (; j + U <= count; j += U) {
    float v[U];
#pragma unroll
    for (int q = 0; q < U; ++q) v[q] = p[(j + q) * stride];
#pragma unroll
    for (int q = 0; q < U; ++q) s += v[q];
  }
  for (; j < count; ++j) s += p[j * stride];
  return s;
}

// dA[d,n] = sum over (b, chunk group) in that order; dD, ddelta_bias likewise.
// Thread per (n', d), d fastest, n' < max(N, 1); n' = 0 also does dD / dbias.
__device__ __forceinline__ void finalize_d(const BwdArgs& a, int64_t i) {
  const int64_t N = a.N, D = a.D;
  const int64_t nn = N > 0 ? N : 1;
  if (i >= nn * D) return;
  const int64_t n = i / D, d = i % D;
  const int64_t cnt = a.Bn * a.KG;
  if (N > 0) st_param(a.dA, d * N + n, a.param_dtype, ordered_sum(a.part_dA + n * D + d, cnt, N * D));
  if (n == 0) {
    if (a.dD) st_param(a.dD, d, a.param_dtype, ordered_sum(a.part_dD + d, cnt, D));
    if (a.dbias) st_param(a.dbias, d, a.param_dtype, ordered_sum(a.part_db + d, cnt, D));
  }
}

// Both finalizes in one launch: the first nbd blocks sum the per-channel
// partials (few threads, each a chain of dependent-address loads, so they
// start first), the rest the dB / dC partials.
template <typename Tio>
__global__ void bwd_finalize(const BwdArgs a, int64_t nbd) {
  const int64_t blk = blockIdx.x;
  if (blk < nbd) finalize_d(a, blk * blockDim.x + threadIdx.x);
  else finalize_bc<Tio>(a, (blk - nbd) * blockDim.x + threadIdx.x);
}

__global__ void fill_zero_words(uint16_t* p, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Zero the first N elements of each of `rows` rows lying ld elements apart.
template <typename W>
__global__ void fill_zero_rows(W* p, int64_t rows, int64_t N, int64_t ld) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < rows * N) p[(i / N) * ld + i % N] = W(0);
}

static hipError_t zero_rows(void* p, int64_t rows, int64_t N, int64_t ld, int64_t es,
                            hipStream_t s) {
  const int64_t n = rows * N;
  if (!p || n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (es == 4) fill_zero_rows<<<grid, dim3(256), 0, s>>>(static_cast<uint32_t*>(p), rows, N, ld);
  else fill_zero_rows<<<grid, dim3(256), 0, s>>>(static_cast<uint16_t*>(p), rows, N, ld);
  return hipGetLastError();
}

static hipError_t zero_bytes(void* p, int64_t bytes, hipStream_t s) {
  if (!p || bytes <= 0) return hipSuccess;
  const int64_t n = bytes / 2;  // every element type here is 2 or 4 bytes
  fill_zero_words<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
      static_cast<uint16_t*>(p), n);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launch

hipError_t launch_bwd_carry(const BwdArgs& a, hipStream_t s) {
  if (a.K <= 1 || a.N <= 0) return hipSuccess;
  const int G = carry_lanes(a.K - 1, 2 * a.Bn * a.N * a.D);
  const int64_t nbd = (a.D + kChannelsPerBlock / G - 1) / (kChannelsPerBlock / G);
  const dim3 grid((unsigned)(2 * a.Bn * a.N * nbd)), block(kChannelsPerBlock);
  switch (G) {
    case 1: bwd_carry<1><<<grid, block, 0, s>>>(a); break;
    case 4: bwd_carry<4><<<grid, block, 0, s>>>(a); break;
    default: bwd_carry<8><<<grid, block, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_finalize(const BwdArgs& a, hipStream_t s) {
  const int64_t nd = (a.N > 0 ? a.N : 1) * a.D;
  const int64_t nbd = (nd + 255) / 256;
  const int64_t nbc = (a.Lt * a.N + 255) / 256;
  const dim3 grid((unsigned)(nbd + nbc));
  switch (a.io_dtype) {
    case 0: bwd_finalize<float><<<grid, dim3(256), 0, s>>>(a, nbd); break;
    case 1: bwd_finalize<f16_t><<<grid, dim3(256), 0, s>>>(a, nbd); break;
    default: bwd_finalize<bf16_t><<<grid, dim3(256), 0, s>>>(a, nbd); break;
  }
  return hipGetLastError();
}

template <typename Tio>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int64_t Bn = a.Bn, N = a.N;
  hipError_t e;
  const size_t tile_bytes = sizeof(float) * 2 * (size_t)N * T;
  if (a.K > 1) {
    bwd_summary<Tio><<<dim3((unsigned)(Bn * a.K * a.nwgd)), dim3(kChannelsPerBlock), tile_bytes,
                       s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_bwd_carry(a, s)) != hipSuccess) return e;
  }
  const size_t main_bytes = tile_bytes + sizeof(float) * 32 * kRedStride;
  if (main_bytes > 64 * 1024) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_main<Tio>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)main_bytes);
    if (e != hipSuccess) return e;
  }
  bwd_main<Tio><<<dim3((unsigned)(Bn * a.KG * a.nwgd)), dim3(kChannelsPerBlock), main_bytes, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_bwd_finalize(a, s);
}

hipError_t launch_bwd_tile(const BwdArgs& a, int ns, hipStream_t s);  // ss_bwd_tile.hip

hipError_t launch_bwd(const BwdArgs& a_in, const Plan& p, int io_dtype, hipStream_t s) {
  BwdArgs a = a_in;
  const int64_t Bn = a.Bn, D = a.D, N = a.N, rows = a.Lt;
  const int64_t io = a.io_dtype == 0 ? 4 : 2, pa = a.param_dtype == 0 ? 4 : 2;
  if (Bn * rows * D == 0) {
    // No (b, t, d) terms: every reduced gradient is an empty sum.
    hipError_t e = zero_bytes(a.dA, D * N * pa, s);
    if (e == hipSuccess) e = zero_bytes(a.dD, D * pa, s);
    if (e == hipSuccess) e = zero_bytes(a.dbias, D * pa, s);
    if (e == hipSuccess) e = zero_rows(a.dB, rows, N, a.ldb, io, s);
    if (e == hipSuccess) e = zero_rows(a.dC, rows, N, a.ldc, io, s);
    if (e == hipSuccess) e = zero_bytes(a.dh0, Bn * D * N * pa, s);  // L = 0: y ignores h0
    return e;
  }
  a.dsum = reinterpret_cast<float*>(a.ws + p.off_dsum);
  a.fstate = reinterpret_cast<float*>(a.ws + p.off_state);
  a.bstate = reinterpret_cast<float*>(a.ws + p.off_bstate);
  a.part_bc = reinterpret_cast<float*>(a.ws + p.off_part_bc);
  a.part_dA = reinterpret_cast<float*>(a.ws + p.off_part_dA);
  a.part_dD = reinterpret_cast<float*>(a.ws + p.off_part_dD);
  a.part_db = reinterpret_cast<float*>(a.ws + p.off_part_db);
  a.KG = p.KG;
  a.nwgd = p.nwgd;
  if (p.bwd_tile) return launch_bwd_tile(a, p.NS, s);
  switch (io_dtype) {
    case 0: return launch_bwd_t<float>(a, s);
    case 1: return launch_bwd_t<f16_t>(a, s);
    case 2: return launch_bwd_t<bf16_t>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ss
