// The general forward scan kernel (N > 64; N <= 64 runs the 8-lane tile
// kernels of ss_fwd_tile.hip).  ss_fwd_scan.hip instantiates it, one I/O type
// per object.
//
// Recurrence: baracuda-kernels page "src/attention/selective_scan.rs", module
// docs, "Algorithm summary".  Per channel (b, d) and state n:
//   dt = softplus(delta + bias) (or delta + bias), a = exp(dt * A[d,n]),
//   h = a * h + dt * B[b,t,n] * u[b,t,d], y = (sum_n C[b,t,n] h + D u) * silu(z).
//
// Mapping.  G = 8 (N <= 128) or 16 consecutive lanes share a channel d of one
// batch row b, lane g holding NS = 16 states, 16 g .. 16 g + 15.  A workgroup
// is 256 lanes = 256 / G consecutive channels, so loads and stores of u /
// delta / z / y are coalesced along D.  The lane keeps its states h[n] and its
// row of A (pre-scaled by log2 e) in VGPRs.  B[b,t,:] and C[b,t,:] are the
// same for every channel of the workgroup: a wave reads G distinct NS-state
// pieces of each row per step.  Every lane of a channel prepares the step
// itself (dt, gate): at 16 states per lane that is about 2 operations per
// update.  Measured on 2x2048x2048 (f32): N = 128 989 -> 836 us, N = 256
// 3279 -> 1114 us against 64 states per lane (G = 2 / 4: 512 registers and a
// spill); 32 states per lane spilled too (1453 / 2874 us); 8 states per lane
// (G = 16 / 32) ran 895 / 1148 us.
//
// Time is walked sequentially inside a chunk.  When B * D alone cannot fill the
// GPU, L is cut into K chunks and the scan runs in two levels:
//   1. fwd_scan<SUMMARY>: every chunk but the last runs from h = 0 and writes
//      its end state S_k[n] and sum_k = sum of dt over the chunk;
//   2. fwd_carry: per (b, d, n), h_in(k+1) = exp(A * sum_k) * h_in(k) + S_k,
//      the composition (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) of the chunk
//      summaries, folded over k (the product of a chunk's decays is
//      exp(A * sum of its dt) in closed form);
//   3. fwd_scan<FULL>: every chunk runs again from its carried-in state and
//      writes y (and last_state for the final chunk).
// With K = 1 only step 3 runs, from h = 0.
#pragma once

#include <type_traits>

#include "ss_device.h"

namespace ss {

enum { MODE_FULL = 0, MODE_SUMMARY = 1 };
constexpr int kBlock = 256;

// The streamed tensors are separate __restrict__ arguments: that tells the
// compiler the y stores never alias B / C, which lets it keep the uniform
// B / C loads on the scalar path inside the loop.
//
// The time loop has no data-dependent or flag-dependent branches: z presence
// is a template parameter, the other options are selects, and the y store is
// unconditional (tail lanes compute the clamped channel D-1 and store the same
// value to the same address).  Branches inside the loop would force the
// compiler to drain outstanding loads at every join and undo the prefetch.
template <typename T, int NS, int G, bool EXACT, int MODE, bool HAS_Z>
__global__ __launch_bounds__(kBlock) void fwd_scan(const T* __restrict__ u_in,
                                                   const T* __restrict__ delta_in,
                                                   const T* __restrict__ B_in,
                                                   const T* __restrict__ C_in,
                                                   const T* __restrict__ z_in,
                                                   T* __restrict__ y_out, const FwdArgs a) {
  constexpr int CPB = kBlock / G;  // channels per workgroup
  const int tid = threadIdx.x;
  const int g = (G == 1) ? 0 : (tid % G);
  const int cl = (G == 1) ? tid : (tid / G);
  const int64_t nbd = (a.D + CPB - 1) / CPB;
  int64_t blk = blockIdx.x;
  const int64_t db = blk % nbd;
  blk /= nbd;
  // the summary pass covers chunks 0 .. K-2 only (the last chunk's end state
  // is never needed), the full pass all K chunks
  const int64_t Kg = (MODE == MODE_SUMMARY) ? a.K - 1 : a.K;
  const int64_t k = blk % Kg;
  const int64_t b = blk / Kg;
  const int64_t d_raw = db * CPB + cl;
  const bool active = d_raw < a.D;
  const int64_t d = active ? d_raw : a.D - 1;  // tail lanes compute on a valid channel
  const int64_t D = a.D, N = a.N;
  const SeqRows sr = seq_rows(a.cu, b, a.L, a.Lt);
  const int64_t t0 = k * a.chunk_len;
  int64_t t1 = (t0 + a.chunk_len < sr.len) ? t0 + a.chunk_len : sr.len;
  if (t1 < t0) t1 = t0;                         // a chunk past a short sequence's end
  const int n0 = g * NS;

  float A2[NS], h[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int n = n0 + i;
    const bool ok = n < N;               // (EXACT rows may be padded past N)
    A2[i] = ok ? ld_param(a.A, d * N + n, a.param_dtype) * kLog2e : 0.0f;
    h[i] = 0.0f;
    if (MODE == MODE_FULL && k > 0 && ok)
      h[i] = a.chunk_state[((b * a.K + (k - 1)) * N + n) * D + d];
    else if (MODE == MODE_FULL && k == 0 && ok && a.h0)
      h[i] = ld_param(a.h0, (b * D + d) * N + n, a.param_dtype);
  }
  const float Dv = a.Dskip ? ld_param(a.Dskip, d, a.param_dtype) : 0.0f;
  const float bv = a.bias ? ld_param(a.bias, d, a.param_dtype) : 0.0f;
  const bool sp = a.softplus != 0;

  const T* up = u_in + sr.start * D + d;
  const T* dp = delta_in + sr.start * D + d;
  const T* zp = HAS_Z ? z_in + sr.start * D + d : up;
  T* yp = y_out + sr.start * D + d;
  const int64_t ldb = a.ldb, ldc = a.ldc;
  const T* Bp = B_in + sr.start * ldb + n0;
  const T* Cp = C_in + sr.start * ldc + n0;

  // B / C rows, software-pipelined one step ahead.
  // EXACT rows are prefetched as raw 32-bit words and converted at their use
  // one step later: a conversion right after the load would make the wave wait
  // for the load immediately (scalar-load waits cannot be partial).
  constexpr bool PAIRS = EXACT && sizeof(T) == 2;
  constexpr int RW = PAIRS ? NS / 2 : NS;  // row words
  using RowT = typename std::conditional<PAIRS, uint32_t, float>::type;
  auto fetch_rows = [&](int64_t t, RowT* Br, RowT* Cr) {
    if constexpr (PAIRS) {
      const uint32_t* bw = reinterpret_cast<const uint32_t*>(Bp + t * ldb);
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(Cp + t * ldc);
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        Br[i] = bw[i];
        if (MODE == MODE_FULL) Cr[i] = cw[i];
      }
    } else {
      // states past N read state N-1 (the load stays unconditional, so that
      // the row's loads stay in flight together) and are zeroed after
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const bool ok = EXACT || n0 + i < N;
        const int64_t ii = EXACT ? i : (ok ? i : N - 1 - n0);
        const float bv = ld(Bp, t * ldb + ii);
        Br[i] = ok ? bv : 0.0f;
        if (MODE == MODE_FULL) {
          const float cv = ld(Cp, t * ldc + ii);
          Cr[i] = ok ? cv : 0.0f;
        } else {
          Cr[i] = 0.0f;
        }
      }
    }
  };
  auto unpack_row = [&](const RowT* r, float* out) {
    if constexpr (PAIRS) {
#pragma unroll
      for (int i = 0; i < RW; ++i) split_pair(r[i], Bp, &out[2 * i], &out[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < NS; ++i) out[i] = r[i];
    }
  };
  RowT Bc[RW], Cc[RW];
  if (t1 > t0) fetch_rows(t0, Bc, Cc);

  float dsum = 0.0f;
  auto step = [&](int64_t t, float uu, float dr, float zz) {
    RowT Bn[RW], Cn[RW];
    fetch_rows((t + 1 < t1) ? t + 1 : t, Bn, Cn);
    float Bt[NS], Ct[NS];
    unpack_row(Bc, Bt);
    if (MODE == MODE_FULL) unpack_row(Cc, Ct);
    const float x = dr + bv;
    float spx = softplus_acc(x);
    // keep the select branch-free: the empty asm makes spx a computed value
    // the compiler cannot sink into a branch on the (uniform) flag
    __asm__ volatile("" : "+v"(spx));
    const float dl = sp ? spx : x;
    const float xu = dl * uu;
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const float dA = fast_exp2(dl * A2[i]);
      h[i] = __builtin_fmaf(dA, h[i], xu * Bt[i]);
      if (MODE == MODE_FULL) o = __builtin_fmaf(Ct[i], h[i], o);
    }
    if (MODE == MODE_SUMMARY) dsum += dl;
    if (MODE == MODE_FULL) {
#pragma unroll
      for (int m = 1; m < G; m <<= 1) o += __shfl_xor(o, m, 64);
      o = __builtin_fmaf(Dv, uu, o);
      if (HAS_Z) o *= zz * sigmoid(zz);
      yp[t * D] = from_f32<T>(o);   // every lane of a channel holds the same o
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) { Bc[i] = Bn[i]; Cc[i] = Cn[i]; }
  };

  // Software pipeline for the per-lane inputs: the next U steps are loaded
  // while the current U steps compute.  Indices are clamped into the chunk,
  // so every load is in bounds; clamped values are never used.
  constexpr int U = 4;
  float cu[U], cd[U], cz[U];
  auto load_group = [&](int64_t tb, float* lu, float* ldl, float* lz) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t tt = (tb + j < t1) ? tb + j : t1 - 1;
      lu[j] = ld(up, tt * D);
      ldl[j] = ld(dp, tt * D);
      lz[j] = (MODE == MODE_FULL && HAS_Z) ? ld(zp, tt * D) : 0.0f;
    }
  };
  if (t1 > t0) {                                // (clamped indices need a step)
    load_group(t0, cu, cd, cz);
    int64_t t = t0;
    for (; t + U <= t1; t += U) {
      float nu[U], nd[U], nz[U];
      load_group(t + U, nu, nd, nz);
#pragma unroll
      for (int j = 0; j < U; ++j) step(t + j, cu[j], cd[j], cz[j]);
#pragma unroll
      for (int j = 0; j < U; ++j) { cu[j] = nu[j]; cd[j] = nd[j]; cz[j] = nz[j]; }
    }
    for (int j = 0; j < U - 1; ++j)
      if (t + j < t1) step(t + j, cu[j], cd[j], cz[j]);
  }

  if (!active) return;
  if (MODE == MODE_SUMMARY) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (n0 + i < N) a.chunk_state[((b * a.K + k) * N + n0 + i) * D + d] = h[i];
    if (g == 0) a.chunk_dsum[(b * a.K + k) * D + d] = dsum;
  } else if (a.last_state != nullptr && k == last_chunk(sr.len, a.chunk_len)) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (n0 + i < N) st_param(a.last_state, (b * D + d) * N + n0 + i, a.param_dtype, h[i]);
  }
}

hipError_t launch_fwd_carry(const FwdArgs& a, hipStream_t s);   // ss_fwd.hip


template <typename T, int NS, int G, bool EXACT, bool HAS_Z>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  const T* U = static_cast<const T*>(a.u);
  const T* DL = static_cast<const T*>(a.delta);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  const T* Z = static_cast<const T*>(a.z);
  T* Y = static_cast<T*>(a.y);
  const int64_t cpb = kBlock / G;
  const int64_t nbd = (a.D + cpb - 1) / cpb;
  if (a.K > 1) {
    const int64_t grid_sum = a.Bn * (a.K - 1) * nbd;  // chunks 0 .. K-2
    fwd_scan<T, NS, G, EXACT, MODE_SUMMARY, false><<<dim3((unsigned)grid_sum), dim3(kBlock), 0, s>>>(
        U, DL, Bm, Cm, Z, Y, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((e = launch_fwd_carry(a, s)) != hipSuccess) return e;
  }
  const int64_t grid = a.Bn * a.K * nbd;
  fwd_scan<T, NS, G, EXACT, MODE_FULL, HAS_Z><<<dim3((unsigned)grid), dim3(kBlock), 0, s>>>(
      U, DL, Bm, Cm, Z, Y, a);
  return hipGetLastError();
}

}  // namespace ss
