// Device-side helpers for the selective-scan kernels (gfx950 only).
//
// Element access (f32 / f16 / bf16 storage, f32 arithmetic), the softplus and
// gate maps of the recurrence, and the launch-parameter blocks shared by the
// forward and backward kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage types.  bf16 and f16 are kept as raw 16-bit words and converted
// explicitly so that every load is a plain integer load.
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(v.bits) << 16);
}
__device__ __forceinline__ float to_f32(f16_t v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, v.bits));
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  // Round to nearest even (hardware conversion on gfx950).
  return bf16_t{__builtin_bit_cast(uint16_t, static_cast<__bf16>(v))};
}
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float v) {
  return f16_t{__builtin_bit_cast(uint16_t, static_cast<_Float16>(v))};
}

template <typename T>
__device__ __forceinline__ float ld(const T* __restrict__ p, int64_t i) { return to_f32(p[i]); }

// Two consecutive 16-bit elements from one 32-bit word (element 2i in the low
// half).  For wave-uniform addresses this keeps the load on the scalar path
// (there are no 16-bit scalar loads); for bf16 the split is two bit ops.
__device__ __forceinline__ void split_pair(uint32_t w, const bf16_t*, float* lo, float* hi) {
  *lo = __builtin_bit_cast(float, w << 16);
  *hi = __builtin_bit_cast(float, w & 0xffff0000u);
}
__device__ __forceinline__ void split_pair(uint32_t w, const f16_t*, float* lo, float* hi) {
  *lo = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
  *hi = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// Load NS consecutive elements row[0 .. NS-1] as f32.  PAIRS: 16-bit type,
// row 4-byte aligned, NS even.
template <typename T, int NS, bool PAIRS>
__device__ __forceinline__ void ld_row(const T* row, float* out) {
  if constexpr (PAIRS && sizeof(T) == 2) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
    for (int i = 0; i < NS / 2; ++i) split_pair(w[i], row, &out[2 * i], &out[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < NS; ++i) out[i] = to_f32(row[i]);
  }
}

// Parameters (A, D, delta_bias, last_state, dA, dD, ddelta_bias) are either f32
// or the io type; the choice is a kernel argument, read once per lane.
__device__ __forceinline__ float ld_param(const void* p, int64_t i, int dtype) {
  if (dtype == 0) return static_cast<const float*>(p)[i];
  if (dtype == 2) return to_f32(static_cast<const bf16_t*>(p)[i]);
  return to_f32(static_cast<const f16_t*>(p)[i]);
}
__device__ __forceinline__ void st_param(void* p, int64_t i, int dtype, float v) {
  if (dtype == 0) static_cast<float*>(p)[i] = v;
  else if (dtype == 2) static_cast<bf16_t*>(p)[i] = from_f32<bf16_t>(v);
  else static_cast<f16_t*>(p)[i] = from_f32<f16_t>(v);
}

// exp2 / log2 / reciprocal on the transcendental unit (v_exp_f32, v_log_f32,
// v_rcp_f32: about 1 ulp on gfx950).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// 2^x in place for 4, 8 or 16 values as one run of v_exp_f32 (a run costs the
// SIMD about 4.3 ns per exp, one exp between dependent FP32 operations about
// 5.3 ns: measured).  The compiler schedules independent work between exps,
// so the run is one asm statement; it ends with s_nop 1 because a VALU
// operation that reads a transcendental result needs a wait state on gfx950,
// which the compiler's hazard check cannot see inside the statement.
__device__ __forceinline__ void exp2_run(float (&e)[4]) {
  __asm__ volatile(
      "v_exp_f32 %0, %0\n\tv_exp_f32 %1, %1\n\tv_exp_f32 %2, %2\n\tv_exp_f32 %3, %3\n\t"
      "s_nop 1"
      : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]));
}
__device__ __forceinline__ void exp2_run(float (&e)[8]) {
  __asm__ volatile(
      "v_exp_f32 %0, %0\n\tv_exp_f32 %1, %1\n\tv_exp_f32 %2, %2\n\tv_exp_f32 %3, %3\n\t"
      "v_exp_f32 %4, %4\n\tv_exp_f32 %5, %5\n\tv_exp_f32 %6, %6\n\tv_exp_f32 %7, %7\n\t"
      "s_nop 1"
      : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]), "+v"(e[6]),
        "+v"(e[7]));
}
__device__ __forceinline__ void exp2_run(float (&e)[16]) {
  float (&lo)[8] = *reinterpret_cast<float(*)[8]>(&e[0]);
  float (&hi)[8] = *reinterpret_cast<float(*)[8]>(&e[8]);
  exp2_run(lo);
  exp2_run(hi);
}
__device__ __forceinline__ void exp2_run(float (&e)[32]) {
  float (&lo)[16] = *reinterpret_cast<float(*)[16]>(&e[0]);
  float (&hi)[16] = *reinterpret_cast<float(*)[16]>(&e[16]);
  exp2_run(lo);
  exp2_run(hi);
}

// log(1 + w) for 0 <= w <= 1, accurate in relative terms also for tiny w.
// With s = 1 + w rounded, c = w - (s - 1) is the rounding error of s, computed
// exactly (s - 1 and the difference are exact by Sterbenz's lemma), and
// log(1 + w) = log(s) + log(1 + c / s) ~= log(s) + c.  Replacing c / s by c
// errs by |c| * w <= 2^-24 * w, i.e. below 1.5 ulp of the result; no division.
__device__ __forceinline__ float log1p_pos(float w) {
  const float s = 1.0f + w;
  const float c = w - (s - 1.0f);
  return __builtin_fmaf(fast_log2(s), kLn2, c);
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log(1 + e^{-|x|}), the short
// form used by the VALU-bound forward tile kernels: measured on gfx950 it is
// within 0.6 ulp rms for |x| < 2 but errs by up to ~10 ulp (biased upwards by
// about one ulp) for -10 < x < -2, where the transcendental unit's log of
// s = 1 + w near 1 is inexact; softplus_acc below costs ~5% there.
__device__ __forceinline__ float softplus(float x) {
  const float e = fast_exp2(-__builtin_fabsf(x) * kLog2e);
  return __builtin_fmaxf(x, 0.0f) + log1p_pos(e);
}

// Decay of a whole chunk for the carries across chunks: exp(A * sum of the
// chunk's dt), the closed form of the product of its per-step decays.  It is
// taken in double precision (A and the sum exact in double, one rounding to
// float at the end) because every chunk boundary of a long sequence passes
// through it: a float exp2 of a rounded A * log2(e) adds one to two ulps per
// boundary, which accumulate along slowly decaying states.  The carries run
// once per (b, chunk, n, d), a small share of a call.
//
// The double exp is written out (no library call, no branches): x = k ln 2 +
// r with |r| <= ln2 / 2 (Cody and Waite's reduction, ln 2 in two parts whose
// first part times k is exact), e^r by its Taylor series through r^10
// (truncation below 3e-13 relative), then 2^k by ldexp; far below the one
// float rounding of the carried state that follows.  The carries run it once per chunk and state
// on a sequential chain, where a library exp's latency showed (long sequence:
// 27.8 us for the forward carry).
__device__ __forceinline__ double exp_dbl(double x) {
  // arguments past the double range saturate (the float result is 0 or inf
  // long before); A * dt is positive only with softplus off or A > 0
  x = x < -745.0 ? -745.0 : (x > 709.0 ? 709.0 : x);
  constexpr double kInvLn2 = 1.4426950408889634;
  constexpr double kLn2A = 6.93147180369123816490e-01;   // 32 leading bits of ln 2
  constexpr double kLn2B = 1.90821492927058770002e-10;   // the rest
  const double kd = __builtin_rint(x * kInvLn2);
  double r = __builtin_fma(-kd, kLn2A, x);
  r = __builtin_fma(-kd, kLn2B, r);
  double p = 1.0 / 3628800.0;                          // 1/10!
  p = __builtin_fma(p, r, 1.0 / 362880.0);
  p = __builtin_fma(p, r, 1.0 / 40320.0);
  p = __builtin_fma(p, r, 1.0 / 5040.0);
  p = __builtin_fma(p, r, 1.0 / 720.0);
  p = __builtin_fma(p, r, 1.0 / 120.0);
  p = __builtin_fma(p, r, 1.0 / 24.0);
  p = __builtin_fma(p, r, 1.0 / 6.0);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(p, static_cast<int>(kd));
}
// A chunk's decay exp(A * sum of its dt), in double: the carries fold their
// chains in double and round each carried state to float once, so that a
// state passed through many chunks does not collect a float rounding per chunk.
__device__ __forceinline__ double chunk_decay(float A, float dsum) {
  return exp_dbl(static_cast<double>(A) * static_cast<double>(dsum));
}

// ------------------------------------------------------------ chunk carries
//
// The carries across chunks fold, per chain, c_j = P_j c_{j-1} + S_j over the
// chunk records j = 0 .. M-1 from c_{-1} = c0 (the recurrence of the
// baracuda-kernels page "src/attention/selective_scan.rs", "Algorithm
// summary", applied to whole chunks: a chunk maps the state entering it to
// P h + S, P the product of its decays, S its end state from zero).  Maps of
// this form compose associatively: (P1, S1) then (P2, S2) is
// (P1 P2, P2 S1 + S2).  A chain takes G = 1, 2, 4 or 8 neighbouring lanes of
// a wave; lane g owns a run of consecutive records and
//   1. folds its run from zero into one pair (P_g, S_g),
//   2. scans the G pairs in the wave (DPP row shifts by 1, 2 and 4 lanes; a
//      lane combines only with lanes of its own chain), which gives every
//      lane the composition of the runs before its own,
//   3. applies that to c0 and walks its run again, writing every c_j.
// Everything runs in double and each written value is rounded to float once.
// The scan pays where it shortens the chain of dependent steps, from M to
// about 2 M / G, on a launch too small to hide that chain behind other
// chains: chains of at most 2 RUN records, and launches whose chains fill
// 2048 waves on one lane each, keep one lane (G = 1: step 3 alone, in rounds
// of RUN records whose loads are issued together); otherwise G = 4 up to 4 RUN
// records and 8 above, as far as the launch stays within 2048 waves; chains
// longer than G RUN records take several rounds, each starting from the
// previous round's last value.  A run's loads are unconditional (past the
// chain's end they re-read its last record), so that they all stay in flight
// together.  Measured: the long sequence (8192 chains of 127 records) 24 us
// with one lane per chain, 9 us with 8; the backward workload's 32 chunks
// with two lanes 18 against 14 us; 2x2048x2048 with N = 64 (2 x 262144 chains
// of 255 records, a bandwidth-bound launch with one lane each) took 300 us
// longer per backward call with 8 lanes.
constexpr int kCarryRun = 16;    // records per lane and round, at most

// Lanes per chain for `chains` chains of M records each.
inline int carry_lanes(int64_t M, int64_t chains) {
  constexpr int64_t kMaxLanes = int64_t(2048) * 64;
  if (M <= 2 * kCarryRun) return 1;
  const int g = M <= 4 * kCarryRun ? 4 : 8;
  if (chains * g <= kMaxLanes) return g;
  return chains * 4 <= kMaxLanes ? 4 : 1;
}

// v of the lane CTRL's row shift names (row_shr:k reads lane i - k of the same
// row of 16); lanes whose source lies outside the row read 0.
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf,
                                                            true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                            0xf, 0xf, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114;

// Records per lane and round for a chain of M records over G lanes.
template <int G, int RUN>
__device__ __forceinline__ int carry_run(int64_t M) {
  const int64_t q = (M + G - 1) / G;
  return (int)(q < RUN ? q : RUN);
}

// One real chain over G lanes (all lanes of the chain call it together; lane
// g = threadIdx.x % G).  Record j lives in slot kj = (rev ? K-1-j : j): its
// end state from zero at st[kj * ss] (overwritten with c_j) and its dt sum at
// ds[kj * dss]; P_j = exp(A * dt sum).
template <int G>
__device__ __forceinline__ void carry_chain(float* st, int64_t ss, const float* ds, int64_t dss,
                                            float A, double c0, int64_t M, int64_t K, bool rev) {
  constexpr int RUN = kCarryRun;
  const int g = (int)(threadIdx.x & (G - 1));
  const int run = carry_run<G, RUN>(M);       // uniform
  for (int64_t r0 = 0; r0 < M; r0 += (int64_t)G * run) {
    const int64_t j0 = r0 + (int64_t)g * run;
    const int cnt = (int)(M - j0 <= 0 ? 0 : (M - j0 < run ? M - j0 : run));
    float sv[RUN], dv[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
      const int64_t j = j0 + i < M ? j0 + i : M - 1;
      const int64_t kj = rev ? K - 1 - j : j;
      sv[i] = st[kj * ss];
      dv[i] = ds[kj * dss];
    }
    double pv[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i)
      if (i < run) pv[i] = chunk_decay(A, dv[i]);
    double c = c0;
    if constexpr (G > 1) {
      double P = 1.0, S = 0.0;   // this lane's run from zero
#pragma unroll
      for (int i = 0; i < RUN; ++i) {
        if (i < run) {
          const bool in = i < cnt;
          S = in ? __builtin_fma(pv[i], S, static_cast<double>(sv[i])) : S;
          P = in ? P * pv[i] : P;
        }
      }
      // inclusive scan over the chain's lanes: (P, S) of runs 0 .. g
      {
        const double Pp = dpp_d<kRowShr1>(P), Sp = dpp_d<kRowShr1>(S);
        if (g >= 1) { S = __builtin_fma(P, Sp, S); P *= Pp; }
      }
      if constexpr (G > 2) {
        const double Pp = dpp_d<kRowShr2>(P), Sp = dpp_d<kRowShr2>(S);
        if (g >= 2) { S = __builtin_fma(P, Sp, S); P *= Pp; }
      }
      if constexpr (G > 4) {
        const double Pp = dpp_d<kRowShr4>(P), Sp = dpp_d<kRowShr4>(S);
        if (g >= 4) { S = __builtin_fma(P, Sp, S); P *= Pp; }
      }
      // runs 0 .. g-1 applied to c0, then this lane's run
      const double Pe = dpp_d<kRowShr1>(P), Se = dpp_d<kRowShr1>(S);
      if (g >= 1) c = __builtin_fma(Pe, c0, Se);
    }
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
      if (i < cnt) {
        c = __builtin_fma(pv[i], c, static_cast<double>(sv[i]));
        st[(rev ? K - 1 - (j0 + i) : j0 + i) * ss] = static_cast<float>(c);
      }
    }
    // the round's last value (the last lane ends there also when its run is empty)
    if constexpr (G > 1) c0 = __shfl(c, G - 1, G);
    else c0 = c;
  }
}

// sigmoid(x) = 1 / (1 + e^{-x}); exp overflow gives rcp(inf) = 0.
__device__ __forceinline__ float sigmoid(float x) {
  return fast_rcp(1.0f + fast_exp2(-x * kLog2e));
}

// log2(e) as a float plus the float nearest to the remainder.
constexpr float kLog2eHi = 1.44269502162933349609375f;
constexpr float kLog2eLo = 1.925963033500011e-08f;

// e^v for v <= 0 with the conversion to base 2 carried as yh + yl (the
// product's rounding error from an FMA): rounding v * log2(e) to a float
// alone errs by up to |v| / 2 ulp of the result (4 ulp at v = -8).
__device__ __forceinline__ float exp_neg_acc(float v) {
  const float yh = v * kLog2eHi;
  const float yl = __builtin_fmaf(v, kLog2eHi, -yh) + v * kLog2eLo;
  return fast_exp2(yh) * __builtin_fmaf(yl, kLn2, 1.0f);
}

// softplus to about an ulp and without bias, for the kernels where dt's
// accuracy shows (the backward, the general and short-sequence forwards).
// softplus(x) = max(x, 0) + log(1 + w), w = e^{-|x|}.  For w <= e^-2 the
// logarithm is the Taylor series through w^9 (truncation below 2e-9
// relative): the transcendental unit's log of s = 1 + w near 1 errs by up to
// ~10 ulp of the small result and is biased upwards by about one ulp over
// -10 < x < -2, the range of Mamba's dt initialisation (measured on gfx950).
__device__ __forceinline__ float softplus_acc(float x) {
  const float w = exp_neg_acc(-__builtin_fabsf(x));
  float q = 1.0f / 9.0f;
  q = __builtin_fmaf(q, w, -1.0f / 8.0f);
  q = __builtin_fmaf(q, w, 1.0f / 7.0f);
  q = __builtin_fmaf(q, w, -1.0f / 6.0f);
  q = __builtin_fmaf(q, w, 1.0f / 5.0f);
  q = __builtin_fmaf(q, w, -1.0f / 4.0f);
  q = __builtin_fmaf(q, w, 1.0f / 3.0f);
  q = __builtin_fmaf(q, w, -0.5f);
  q = __builtin_fmaf(q, w, 1.0f);
  const float lp = w <= 0.1353352832366127f ? w * q : log1p_pos(w);
  return __builtin_fmaxf(x, 0.0f) + lp;
}

// sigmoid with the exponent's argument carried as in exp_neg_acc:
// 1 / (1 + e^{-x}) for x >= 0, e^x / (1 + e^x) for x < 0.
__device__ __forceinline__ float sigmoid_acc(float x) {
  const float e = exp_neg_acc(-__builtin_fabsf(x));
  const float r = fast_rcp(1.0f + e);
  return x >= 0.0f ? r : e * r;
}

// Buffer resources (raw, stride 0) over a byte range: loads beyond the range
// return 0 and stores beyond it are dropped, which replaces clamping and
// predication for tails.  Offsets are 32-bit (the range is < 2^31 bytes).
constexpr int kBufferFlags = 0x00020000;  // gfx9 family raw buffer, 32-bit dwords
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}
template <typename T> __device__ __forceinline__ float buf_ld(__amdgpu_buffer_rsrc_t r, int voff, int soff);
template <> __device__ __forceinline__ float buf_ld<float>(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
template <> __device__ __forceinline__ float buf_ld<bf16_t>(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return to_f32(bf16_t{__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)});
}
template <> __device__ __forceinline__ float buf_ld<f16_t>(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return to_f32(f16_t{__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)});
}
template <typename T> __device__ __forceinline__ void buf_st(float v, __amdgpu_buffer_rsrc_t r, int voff, int soff);
template <> __device__ __forceinline__ void buf_st<float>(float v, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
}
template <> __device__ __forceinline__ void buf_st<bf16_t>(float v, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b16(from_f32<bf16_t>(v).bits, r, voff, soff, 0);
}
template <> __device__ __forceinline__ void buf_st<f16_t>(float v, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b16(from_f32<f16_t>(v).bits, r, voff, soff, 0);
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.
// Within every aligned group of 16 workgroup ids this remap puts logical
// neighbours 2j and 2j+1 on the same XCD (ids r and r + 8), so two channel
// blocks that share 128-byte lines fetch them through one L2.
__device__ __forceinline__ int64_t xcd_pair_remap(int64_t x, int64_t total) {
  const int64_t q = x >> 4, r = x & 15;
  return (q * 16 + 16 <= total) ? q * 16 + 2 * (r & 7) + (r >> 3) : x;
}

// Rows of sequence b in the [rows, D] / [rows, N] tensors: dense problems
// hold B sequences of L steps (rows b*L ..); packed variable-length problems
// (cu = cu_seqlens, device, [B+1]) hold sequence b at rows cu[b] .. cu[b+1].
// The bounds are clamped to [0, Lt] (Lt = total rows) and the length to L,
// so that no entry of cu can send an access outside the tensors.
struct SeqRows { int64_t start, len; };
__device__ __forceinline__ SeqRows seq_rows(const int32_t* cu, int64_t b, int64_t L, int64_t Lt) {
  if (!cu) return {b * L, L};
  int64_t s = cu[b], e = cu[b + 1];
  s = s < 0 ? 0 : (s > Lt ? Lt : s);
  e = e < s ? s : (e > Lt ? Lt : e);
  return {s, (e - s < L) ? e - s : L};
}

// Bytes from the first row of nrows rows of a [*, N] matrix whose rows lie
// ld elements apart, to the end of the last row's N elements.
__device__ __forceinline__ int64_t rows_bytes(int64_t nrows, int64_t ld, int64_t N, int es) {
  return nrows > 0 ? ((nrows - 1) * ld + N) * es : 0;
}

// Chunk of sequence length len that holds its last step (0 when len = 0).
__device__ __forceinline__ int64_t last_chunk(int64_t len, int64_t chunk_len) {
  return len > 0 ? (len - 1) / chunk_len : 0;
}

// Forward launch parameters.
struct FwdArgs {
  const void* u;
  const void* delta;
  const void* A;
  const void* B;
  const void* C;
  const void* Dskip;       // nullable
  const void* z;           // nullable
  const void* bias;        // nullable
  void* y;
  void* last_state;        // nullable
  const void* h0;          // nullable: [Bn, D, N] state before t = 0 (param dtype)
  float* chunk_dsum;       // [Bn, K, D]   sum of delta_eff over each chunk
  float* chunk_state;      // [Bn, K, N, D] chunk-end state from zero / carried-in state
  int64_t Bn, L, D, N;
  int64_t chunk_len, K;    // chunk length and number of chunks
  const int32_t* cu;       // nullable: cu_seqlens [Bn+1] of a packed problem
  int64_t Lt;              // rows of the [rows, D] tensors (Bn*L when dense)
  int64_t ldb, ldc;        // elements between consecutive rows of B / C (N when packed)
  int softplus;
  int param_dtype;
  // General scan (N > 64) with N short of its lanes' NS * G states: B / C are
  // first copied into rows of NS * G elements, zero past N (workspace).
  void* b_pad;             // nullable
  void* c_pad;             // nullable
};

// Backward launch parameters.  Workspace sub-buffers (f32):
//   dsum    [Bn, K, D]       sum of dt over each chunk
//   fstate  [Bn, K, N, D]    chunk-end state from zero, then (after the carry)
//                            slot k = state entering chunk k+1
//   bstate  [Bn, K, N, D]    chunk reverse summary, then slot k = adjoint
//                            handed to the end of chunk k-1
//   part_bc [Bn, L, nwgd, 2, N]  per channel-block partial sums of dB, dC
//   part_dA [Bn, KG, N, D], part_dD / part_db [Bn, KG, D]  per chunk-group
//                            partial sums of dA, dD, ddelta_bias
struct BwdArgs {
  const void* u;
  const void* delta;
  const void* A;
  const void* B;
  const void* C;
  const void* Dskip;       // nullable
  const void* z;           // nullable
  const void* bias;        // nullable
  const void* h0;          // nullable: [Bn, D, N] state before t = 0 (param dtype)
  const void* dy;
  void* du;
  void* ddelta;
  void* dA;
  void* dB;
  void* dC;
  void* dD;                // nullable (iff Dskip)
  void* dz;                // nullable (iff z)
  void* dbias;             // nullable (iff bias)
  void* dh0;               // nullable (iff h0): [Bn, D, N] gradient of h0
  char* ws;
  float* dsum;
  float* fstate;
  float* bstate;
  float* part_bc;
  float* part_dA;
  float* part_dD;
  float* part_db;
  int64_t Bn, L, D, N;
  int64_t chunk_len, K, KG, nwgd;
  const int32_t* cu;       // nullable: cu_seqlens [Bn+1] of a packed problem
  int64_t Lt;              // rows of the [rows, D] tensors (Bn*L when dense)
  int64_t ldb, ldc;        // elements between consecutive rows of B / C (N when packed)
  int softplus;
  int param_dtype;
  int io_dtype;
};


// ---------------------------------------------------------------------------
// Lane map and cross-lane sums of the 8-lanes-per-channel backward tile
// kernels.  In a 256-lane workgroup, wave w's lane c + 8g is lane g of channel
// 8w + c, so a channel's 8 lanes sit 8 apart.  (The forward tile kernels put a
// channel's lanes in one row of 16 instead: wide_g / wide_channel in
// ss_fwd_tile.hip.)

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xf, 0xf, true));
}

// A channel's 8 lanes are 8 apart in the wave (lane c + 8g), so that its
// butterfly partners are 32, 16 and 8 lanes away: the first two stages are
// the gfx950 lane swaps, the last a DPP rotate within a row of 16.
//   permlane32_swap(p, q) returns (p, p of lane + 32) in lanes 0-31 and
//   (q of lane - 32, q) in lanes 32-63; permlane16_swap does the same between
//   rows 0/1 and 2/3 of 16 lanes.  Summing the two results gives the pair's
//   sum of p in the lower lane and of q in the upper one, with no selects.
// (The halves are copied to scalars before the float casts: this compiler
// turns __builtin_bit_cast of the second vector element into a read of the
// first.)
__device__ __forceinline__ void swap32(float p, float q, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(q), false,
                                                  false);
  const unsigned r0 = r[0], r1 = r[1];
  lo = __uint_as_float(r0);
  hi = __uint_as_float(r1);
}
__device__ __forceinline__ void swap16(float p, float q, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(q), false,
                                                  false);
  const unsigned r0 = r[0], r1 = r[1];
  lo = __uint_as_float(r0);
  hi = __uint_as_float(r1);
}

// Reduce-scatter over a channel's 8 lanes: lane g holds o[0..7]; on return it
// holds the channel's sum of o[g].  Stage 1 (partner g ^ 4, 32 lanes away):
// lanes with g < 4 keep indices 0-3, the others 4-7; stage 2 (g ^ 2, 16
// away) halves that again; stage 3 (g ^ 1, 8 away, DPP row_ror:8) keeps one
// value with a select pair.  15 VALU ops for 8 sums (4 + 2 swaps, 7 adds,
// 2 selects).
__device__ __forceinline__ float reduce_scatter8(const float (&o)[8], int g) {
  float ra[4], rb[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float x, y;
    swap32(o[k], o[4 + k], x, y);
    ra[k] = x + y;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float x, y;
    swap16(ra[k], ra[2 + k], x, y);
    rb[k] = x + y;
  }
  const bool lo1 = (g & 1) == 0;
  const float send = lo1 ? rb[1] : rb[0];
  const float keep = lo1 ? rb[0] : rb[1];
  return keep + dpp<0x128>(send);       // row_ror:8: lane i <-> i ^ 8 within a row
}

// Sum over a channel's 8 lanes; every lane gets the channel's sum (the two
// addends of each stage are the same pair in both lanes, so both round alike).
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0x128>(v);   // row_ror:8
  float x, y;
  swap16(v, v, x, y);
  v = x + y;
  swap32(v, v, x, y);
  return x + y;
}

__device__ __forceinline__ int lane_g(int tid) { return (tid >> 3) & 7; }
__device__ __forceinline__ int lane_channel(int tid) { return ((tid >> 6) << 3) | (tid & 7); }

}  // namespace ss
