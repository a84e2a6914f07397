// Forward selective scan kernels for gfx950.
//
// Recurrence: baracuda-kernels page "src/attention/selective_scan.rs", module
// docs, "Algorithm summary".  Per channel (b, d) and state n:
//   dt = softplus(delta + bias) (or delta + bias), a = exp(dt * A[d,n]),
//   h = a * h + dt * B[b,t,n] * u[b,t,d], y = (sum_n C[b,t,n] h + D u) * silu(z).
//
// This file holds the carry across chunks (fwd_carry), the short-sequence
// (decode-step) kernel fwd_short, and the dispatch over the forward kernels:
// fwd_short for L <= 16, the tile kernels of ss_fwd_tile.hip for N <= 64, the
// general scan of ss_fwd_scan.h for N > 64.
//
// When B * D alone cannot fill the GPU, L is cut into K chunks and the scan
// runs in two levels: a first pass writes every chunk's end state from zero
// S_k and its sum of dt; fwd_carry turns them into the state entering each
// chunk, h_in(k+1) = exp(A * sum_k) h_in(k) + S_k (the product of a chunk's
// decays is exp(A * sum of its dt) in closed form); a second pass runs each
// chunk from its carried-in state.  With K = 1 only the second pass runs.
#include "ss_fwd_scan.h"

namespace ss {

// Carry across chunks, one chain per (b, n, d): slot k of chunk_state holds
// S_k on entry and h_in(k+1) = state entering chunk k+1 on exit (k = 0 ..
// K-2; the last chunk's summary is never produced or used).  G lanes per
// chain (carry_chain's in-wave scan), 256 / G chains (consecutive d) per
// workgroup.
template <int G>
__global__ __launch_bounds__(kBlock) void fwd_carry(const FwdArgs a) {
  constexpr int CPB = kBlock / G;
  const int64_t nbd = (a.D + CPB - 1) / CPB;
  int64_t blk = blockIdx.x;
  const int64_t db = blk % nbd;
  blk /= nbd;
  const int64_t n = blk % a.N;
  const int64_t b = blk / a.N;
  const int64_t d = db * CPB + threadIdx.x / G;
  if (d >= a.D) return;                      // the chain's lanes leave together
  const int64_t D = a.D, N = a.N, K = a.K;
  const float Av = ld_param(a.A, d * N + n, a.param_dtype);
  const double h0 = a.h0 ? ld_param(a.h0, (b * D + d) * N + n, a.param_dtype) : 0.0;
  carry_chain<G>(a.chunk_state + (b * K * N + n) * D + d, N * D, a.chunk_dsum + b * K * D + d, D,
                 Av, h0, K - 1, K, false);
}

// ------------------------------------------------------------------ launch

template <int G>
static hipError_t launch_fwd_carry_g(const FwdArgs& a, hipStream_t s) {
  const int64_t nbd = (a.D + kBlock / G - 1) / (kBlock / G);
  fwd_carry<G><<<dim3((unsigned)(a.Bn * a.N * nbd)), dim3(kBlock), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd_carry(const FwdArgs& a, hipStream_t s) {
  if (a.N <= 0 || a.K <= 1) return hipSuccess;
  switch (carry_lanes(a.K - 1, a.Bn * a.N * a.D)) {
    case 1: return launch_fwd_carry_g<1>(a, s);
    case 4: return launch_fwd_carry_g<4>(a, s);
    default: return launch_fwd_carry_g<8>(a, s);
  }
}

hipError_t launch_fwd_tile(const FwdArgs& a, int io_dtype, int ns, hipStream_t s);
hipError_t launch_fwd_scan_f32(const FwdArgs& a, int ns, int gl, hipStream_t s);
hipError_t launch_fwd_scan_f16(const FwdArgs& a, int ns, int gl, hipStream_t s);
hipError_t launch_fwd_scan_bf16(const FwdArgs& a, int ns, int gl, hipStream_t s);

// ------------------------------------------------------- short sequences
//
// L <= 16 (decode steps), N <= 32: 4 lanes per channel, lane g holds states
// g*NS .. g*NS+NS-1; every lane prepares its channel's step itself (cheap at
// this length), the readout is a 2-step DPP sum over the channel's lanes.  A
// 256-lane workgroup covers 64 channels of one batch row; no LDS, no chunks.
// A step's inputs are loaded one step ahead, the first step's before the
// parameters and the state; with VEC the lane's B / C pieces are read as
// 32-bit words (one 8-byte piece of a bf16 row in two loads instead of four).
// On one in-place step of the 2.8B-shaped layer both took a graph-replayed
// step from 3.98 to 3.30 us (element loads of B / C in the step loop before).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xf, 0xf, true));
}

// NS consecutive f32 values at p + off as 16-byte loads / stores (VEC: the
// caller checked 16-byte alignment and N == 4 * NS), else element by element
// in the parameter dtype with states n >= N read as 0 / not written.
template <int NS, bool VEC>
__device__ __forceinline__ void row_ld(const void* p, int64_t off, int n0, int64_t N, int dtype,
                                       float* out) {
  if constexpr (VEC && NS % 4 == 0) {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + off);
#pragma unroll
    for (int j = 0; j < NS / 4; ++j) {
      const float4 v = q[j];
      out[4 * j] = v.x; out[4 * j + 1] = v.y; out[4 * j + 2] = v.z; out[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < NS; ++k) out[k] = n0 + k < N ? ld_param(p, off + k, dtype) : 0.0f;
  }
}
template <int NS, bool VEC>
__device__ __forceinline__ void row_st(void* p, int64_t off, int n0, int64_t N, int dtype,
                                       const float* v) {
  if constexpr (VEC && NS % 4 == 0) {
    float4* q = reinterpret_cast<float4*>(static_cast<float*>(p) + off);
#pragma unroll
    for (int j = 0; j < NS / 4; ++j) q[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
  } else {
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (n0 + k < N) st_param(p, off + k, dtype, v[k]);
  }
}

template <typename T, int NS, bool HAS_Z, bool VEC>
__global__ __launch_bounds__(kBlock) void fwd_short(const T* __restrict__ u_in,
                                                    const T* __restrict__ delta_in,
                                                    const T* __restrict__ B_in,
                                                    const T* __restrict__ C_in,
                                                    const T* __restrict__ z_in,
                                                    T* __restrict__ y_out, const FwdArgs a) {
  constexpr int G = 4, CPB = kBlock / G;
  const int g = threadIdx.x % G;
  const int64_t nbd = (a.D + CPB - 1) / CPB;
  const int64_t db = blockIdx.x % nbd, b = blockIdx.x / nbd;
  const int64_t d_raw = db * CPB + threadIdx.x / G;
  const bool active = d_raw < a.D;
  const int64_t d = active ? d_raw : a.D - 1;
  const int64_t D = a.D, N = a.N;
  const SeqRows sr = seq_rows(a.cu, b, a.L, a.Lt);
  const int64_t L = sr.len;
  const int n0 = g * NS;
  // the first step's inputs first (the softplus chain waits on delta), then
  // the parameters and the state; each later step's inputs one step ahead
  // (row index clamped to the sequence, or to row 0 when it is empty)
  struct Step { float uu, dr, zz, bb[NS], cc[NS]; };
  auto fetch = [&](int64_t t) {
    Step r;
    const int64_t row = L > 0 ? sr.start + (t < L ? t : L - 1) : 0;
    const int64_t i = row * D + d;
    r.uu = ld(u_in, i);
    r.dr = ld(delta_in, i);
    r.zz = HAS_Z ? ld(z_in, i) : 0.0f;
    const T* Bt = B_in + row * a.ldb;
    const T* Ct = C_in + row * a.ldc;
    if constexpr (VEC) {
      ld_row<T, NS, true>(Bt + n0, r.bb);
      ld_row<T, NS, true>(Ct + n0, r.cc);
    } else {
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const bool ok = n0 + k < N;
        r.bb[k] = ok ? ld(Bt, n0 + k) : 0.0f;
        r.cc[k] = ok ? ld(Ct, n0 + k) : 0.0f;
      }
    }
    return r;
  };
  Step nx = fetch(0);
  float A2[NS], h[NS];
  row_ld<NS, VEC>(a.A, d * N + n0, n0, N, a.param_dtype, A2);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    A2[i] *= kLog2e;
    h[i] = 0.0f;
  }
  if (a.h0) row_ld<NS, VEC>(a.h0, (b * D + d) * N + n0, n0, N, a.param_dtype, h);
  const float Dv = a.Dskip ? ld_param(a.Dskip, d, a.param_dtype) : 0.0f;
  const float bv = a.bias ? ld_param(a.bias, d, a.param_dtype) : 0.0f;
  for (int64_t t = 0; t < L; ++t) {
    const Step cur = nx;
    nx = fetch(t + 1);
    const int64_t i = (sr.start + t) * D + d;
    const float uu = cur.uu;
    const float x = cur.dr + bv;
    const float dl = a.softplus ? softplus_acc(x) : x;
    const float xu = dl * uu;
    float o = 0.0f;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      h[k] = __builtin_fmaf(fast_exp2(dl * A2[k]), h[k], xu * cur.bb[k]);
      o = __builtin_fmaf(cur.cc[k], h[k], o);
    }
    o += dpp_f<0xB1>(o);   // quad_perm [1,0,3,2]
    o += dpp_f<0x4E>(o);   // quad_perm [2,3,0,1]: every lane of the quad has the sum
    float yv = __builtin_fmaf(Dv, uu, o);
    if (HAS_Z) {
      const float zz = cur.zz;
      yv *= zz * sigmoid(zz);
    }
    if (active && g == 0) y_out[i] = from_f32<T>(yv);
  }
  if (active && a.last_state) row_st<NS, VEC>(a.last_state, (b * D + d) * N + n0, n0, N,
                                               a.param_dtype, h);
}

template <typename T, bool HAS_Z, bool VEC>
static hipError_t launch_short_z(const FwdArgs& a, int ns, hipStream_t s) {
  const T* U = static_cast<const T*>(a.u);
  const T* DL = static_cast<const T*>(a.delta);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  const T* Z = static_cast<const T*>(a.z);
  T* Y = static_cast<T*>(a.y);
  const dim3 grid((unsigned)(a.Bn * ((a.D + kBlock / 4 - 1) / (kBlock / 4))));
  switch (ns) {
    case 1: fwd_short<T, 1, HAS_Z, VEC><<<grid, dim3(kBlock), 0, s>>>(U, DL, Bm, Cm, Z, Y, a); break;
    case 2: fwd_short<T, 2, HAS_Z, VEC><<<grid, dim3(kBlock), 0, s>>>(U, DL, Bm, Cm, Z, Y, a); break;
    case 4: fwd_short<T, 4, HAS_Z, VEC><<<grid, dim3(kBlock), 0, s>>>(U, DL, Bm, Cm, Z, Y, a); break;
    case 8: fwd_short<T, 8, HAS_Z, VEC><<<grid, dim3(kBlock), 0, s>>>(U, DL, Bm, Cm, Z, Y, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_short(const FwdArgs& a, int ns, hipStream_t s) {
  auto al = [](const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  // VEC: f32 parameters, N = 4 NS, 16-byte aligned A / h0 / last_state rows,
  // and B / C rows readable as 32-bit words
  auto al4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; };
  const bool vec = a.param_dtype == 0 && (ns == 4 || ns == 8) && a.N == 4 * ns && al(a.A) &&
                   al(a.h0) && al(a.last_state) && al4(a.B) && al4(a.C) &&
                   (a.ldb * (int64_t)sizeof(T)) % 4 == 0 && (a.ldc * (int64_t)sizeof(T)) % 4 == 0;
  if (vec) return a.z ? launch_short_z<T, true, true>(a, ns, s) : launch_short_z<T, false, true>(a, ns, s);
  return a.z ? launch_short_z<T, true, false>(a, ns, s) : launch_short_z<T, false, false>(a, ns, s);
}

// B and C rows (row stride ld, n elements) copied into rows of npad elements,
// zero past n: the general scan then reads whole rows as vectors.
template <typename W>
__global__ void pad_bc_rows(const W* __restrict__ B, const W* __restrict__ C, W* __restrict__ Bp,
                            W* __restrict__ Cp, int64_t rows, int64_t n, int64_t ldb, int64_t ldc,
                            int64_t npad) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * npad) return;
  const int64_t r = i / npad, c = i % npad;
  Bp[i] = c < n ? B[r * ldb + c] : W(0);
  Cp[i] = c < n ? C[r * ldc + c] : W(0);
}

hipError_t launch_fwd(const FwdArgs& a, int io_dtype, int ns, int gl, hipStream_t s) {
  if (gl == 4 && ns <= 8) {                     // short sequences (single chunk)
    switch (io_dtype) {
      case 0: return launch_short<float>(a, ns, s);
      case 1: return launch_short<f16_t>(a, ns, s);
      case 2: return launch_short<bf16_t>(a, ns, s);
    }
    return hipErrorInvalidValue;
  }
  if (gl == 8 && ns <= 8) return launch_fwd_tile(a, io_dtype, ns, s);
  FwdArgs g = a;
  if (a.b_pad != nullptr && a.N > 0 && a.Lt > 0) {   // N short of ns * gl: padded rows
    const int64_t npad = (int64_t)ns * gl, total = a.Lt * npad;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (io_dtype == 0)
      pad_bc_rows<uint32_t><<<grid, dim3(256), 0, s>>>(
          static_cast<const uint32_t*>(a.B), static_cast<const uint32_t*>(a.C),
          static_cast<uint32_t*>(a.b_pad), static_cast<uint32_t*>(a.c_pad), a.Lt, a.N, a.ldb,
          a.ldc, npad);
    else
      pad_bc_rows<uint16_t><<<grid, dim3(256), 0, s>>>(
          static_cast<const uint16_t*>(a.B), static_cast<const uint16_t*>(a.C),
          static_cast<uint16_t*>(a.b_pad), static_cast<uint16_t*>(a.c_pad), a.Lt, a.N, a.ldb,
          a.ldc, npad);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    g.B = a.b_pad;
    g.C = a.c_pad;
    g.ldb = g.ldc = npad;
  }
  switch (io_dtype) {
    case 0: return launch_fwd_scan_f32(g, ns, gl, s);
    case 1: return launch_fwd_scan_f16(g, ns, gl, s);
    case 2: return launch_fwd_scan_bf16(g, ns, gl, s);
  }
  return hipErrorInvalidValue;
}

// Fill a float / param-typed buffer with zeros (used for last_state when
// L = 0).  A kernel rather than a memset so the call can be graph-captured.
__global__ void fill_zero_param(void* p, int64_t n, int dtype) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) st_param(p, i, dtype, 0.0f);
}

hipError_t launch_zero_param(void* p, int64_t n, int dtype, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_zero_param<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(p, n, dtype);
  return hipGetLastError();
}

// Copy a param-typed buffer (last_state = h0 when L = 0).
__global__ void copy_param(void* dst, const void* src, int64_t n, int dtype) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) st_param(dst, i, dtype, ld_param(src, i, dtype));
}

hipError_t launch_copy_param(void* dst, const void* src, int64_t n, int dtype, hipStream_t s) {
  if (n <= 0 || dst == src) return hipSuccess;
  copy_param<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(dst, src, n, dtype);
  return hipGetLastError();
}

}  // namespace ss
