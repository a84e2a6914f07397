// Forward selective scan with a channel's states split over 8 lanes (gfx950).
//
// Same recurrence as ss_fwd.hip (baracuda-kernels page
// "src/attention/selective_scan.rs", module docs, "Algorithm summary"), for
// N <= 32.  Mapping:
//
//   * 8 consecutive lanes own one channel d: lane g holds states
//     n = g*NS .. g*NS+NS-1 (NS = 1, 2 or 4).  A wave covers 8 channels, a
//     256-lane workgroup 32.  This gives 8x the waves of one-lane-per-channel,
//     which the wave-per-SIMD issue rate needs (a lone wave issues far below
//     the VALU rate; several resident waves per SIMD are needed to fill it).
//   * Per-(t, d) work is time-shared: in every tile of 8 steps, lane g loads
//     u / delta / z of step t0+g, computes dt = softplus(delta + bias),
//     dt*u and the gate silu(z) for that step only, and hands (dt, dt*u) to
//     the other 7 lanes of its channel through a per-wave LDS exchange.
//   * The readout sum over a channel's states is a sum over its 8 lanes, done
//     once per 8-step tile as a DPP reduce-scatter: lane g ends with the sum of
//     step t0+g and applies the skip term and the gate to it.
//   * B and C are staged per workgroup in LDS as f32, [n][t] per 64-step tile,
//     double buffered, rows padded to 68 floats (16-byte aligned, conflict-free
//     128-bit reads); states n >= N are zero rows, so padded states stay 0.
//
// Chunk summaries, the carry and the chunked final pass follow the same
// two-level scheme as ss_fwd.hip and share its workspace layout.
#include <type_traits>

#include "ss_device.h"

namespace ss {

namespace {

constexpr int kBlockT = 256;
constexpr int GL = 8;                 // lanes per channel
constexpr int CPW = kBlockT / GL;     // channels per workgroup (32)
constexpr int TB = 64;                // steps per B/C staging tile
constexpr int TS = 68;                // LDS row stride of a staged row (floats)
constexpr int XS = 10;                // exchange row stride (float2) per channel

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xf, 0xf, true));
}

// Reduce-scatter over each group of 8 consecutive lanes: lane g of the group
// holds o[0..7]; on return it holds the group's sum of o[g].  Three butterfly
// stages (partners g^7 via row_half_mirror, g^2, g^1): at each stage a lane
// keeps the half of its values whose index bit matches its own lane bit and
// sends the other half, so each stage is one DPP add per kept value plus two
// selects.  21 VALU ops for 8 sums instead of 8 x (3 DPP adds + 1 select).
__device__ __forceinline__ float reduce_scatter8(const float (&o)[8], int g) {
  const bool lo4 = (g & 4) == 0, lo2 = (g & 2) == 0, lo1 = (g & 1) == 0;
  float ra[4], rb[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float send = lo4 ? o[4 + k] : o[k];
    const float keep = lo4 ? o[k] : o[4 + k];
    ra[k] = keep + dpp<0x141>(send);    // row_half_mirror: lane g <-> 7 - g
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float send = lo2 ? ra[2 + k] : ra[k];
    const float keep = lo2 ? ra[k] : ra[2 + k];
    rb[k] = keep + dpp<0x4E>(send);     // quad_perm [2,3,0,1]: g <-> g ^ 2
  }
  const float send = lo1 ? rb[1] : rb[0];
  const float keep = lo1 ? rb[0] : rb[1];
  return keep + dpp<0xB1>(send);        // quad_perm [1,0,3,2]: g <-> g ^ 1
}

// Sum over each group of 8 consecutive lanes; every lane gets its group's sum.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror: lane i <-> 7 - i within 8
  return v;
}

}  // namespace

enum { TMODE_FULL = 0, TMODE_SUMMARY = 1 };

template <typename T, int NS, int MODE, bool HAS_Z>
__global__ __launch_bounds__(kBlockT) void fwd_tile(const T* __restrict__ u_in,
                                                    const T* __restrict__ delta_in,
                                                    const T* __restrict__ B_in,
                                                    const T* __restrict__ C_in,
                                                    const T* __restrict__ z_in,
                                                    T* __restrict__ y_out, const FwdArgs a) {
  constexpr int NP = NS * GL;                       // padded state count
  constexpr int RB = (TB * NP + kBlockT - 1) / kBlockT;  // staged elements per thread
  __shared__ __attribute__((aligned(16))) float sBC[2][2][NP][TS];
  __shared__ __attribute__((aligned(16))) float2 xch[2][CPW][XS];

  const int tid = threadIdx.x;
  const int g = tid % GL;
  const int cl = tid / GL;
  const int64_t nbd = (a.D + CPW - 1) / CPW;
  int64_t blk = xcd_pair_remap(blockIdx.x, gridDim.x);
  const int64_t db = blk % nbd;
  blk /= nbd;
  const int64_t Kg = (MODE == TMODE_SUMMARY) ? a.K - 1 : a.K;
  const int64_t k = blk % Kg;
  const int64_t b = blk / Kg;
  const int64_t d_raw = db * CPW + cl;
  const bool active = d_raw < a.D;
  const int64_t d = active ? d_raw : a.D - 1;   // tail lanes duplicate channel D-1
  const int64_t L = a.L, D = a.D, N = a.N;
  const int64_t t0 = k * a.chunk_len;
  const int64_t t1 = (t0 + a.chunk_len < L) ? t0 + a.chunk_len : L;
  const int n0 = g * NS;

  float A2[NS], h[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int n = n0 + i;
    A2[i] = n < N ? ld_param(a.A, d * N + n, a.param_dtype) * kLog2e : 0.0f;
    h[i] = 0.0f;
    if (MODE == TMODE_FULL && k > 0 && n < N)
      h[i] = a.chunk_state[((b * a.K + (k - 1)) * N + n) * D + d];
  }
  const float Dv = a.Dskip ? ld_param(a.Dskip, d, a.param_dtype) : 0.0f;
  const float bv = a.bias ? ld_param(a.bias, d, a.param_dtype) : 0.0f;
  const bool sp = a.softplus != 0;

  // Streamed tensors through buffer resources covering this chunk's rows:
  // the lane's own-step element (t0 + p*8 + g, d) sits at byte offset
  // voff_own + soff(p), steps past the chunk read 0 / are not stored.
  constexpr int ES = sizeof(T);
  const int64_t nsteps = t1 - t0;
  const int64_t row0 = (b * L + t0) * D;
  const auto rs_u = make_rsrc(u_in + row0, nsteps * D * ES);
  const auto rs_d = make_rsrc(delta_in + row0, nsteps * D * ES);
  const auto rs_z = make_rsrc(HAS_Z ? z_in + row0 : u_in + row0, nsteps * D * ES);
  const auto rs_y = make_rsrc(y_out + row0, nsteps * D * ES);
  const int voff_own = (int)((g * D + d) * ES);
  const int soff_step = (int)(GL * D * ES);            // one 8-step tile
  const auto rs_B = make_rsrc(B_in + (b * L + t0) * N, nsteps * N * ES);
  const auto rs_C = make_rsrc(C_in + (b * L + t0) * N, nsteps * N * ES);

  // ---- B / C staging (whole workgroup) ----
  float rb[RB], rc[RB];
  auto stage_load = [&](int64_t tb) {
    const int trow = (int)(tb - t0);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int e = tid + r * kBlockT;
      const int tt = e / NP, n = e % NP;
      const bool ok = n < N;                       // rows past the chunk read 0
      const int off = ((trow + tt) * (int)N + (ok ? n : 0)) * ES;
      const float vb = buf_ld<T>(rs_B, off, 0);
      rb[r] = ok ? vb : 0.0f;
      if (MODE == TMODE_FULL) {
        const float vc = buf_ld<T>(rs_C, off, 0);
        rc[r] = ok ? vc : 0.0f;
      }
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int e = tid + r * kBlockT;
      const int tt = e / NP, n = e % NP;
      sBC[buf][0][n][tt] = rb[r];
      if (MODE == TMODE_FULL) sBC[buf][1][n][tt] = rc[r];
    }
  };

  // ---- per-lane inputs of its own step, prefetched two 8-step tiles ahead ----
  auto load_own = [&](int p, float& lu, float& ldl, float& lz) {
    const int soff = p * soff_step;
    lu = buf_ld<T>(rs_u, voff_own, soff);
    ldl = buf_ld<T>(rs_d, voff_own, soff);
    lz = (MODE == TMODE_FULL && HAS_Z) ? buf_ld<T>(rs_z, voff_own, soff) : 0.0f;
  };
  float pu0, pd0, pz0, pu1, pd1, pz1;
  load_own(0, pu0, pd0, pz0);
  load_own(1, pu1, pd1, pz1);
  // (prefetch distance: tile p+1's inputs are in registers while tile p runs,
  //  tile p+2's loads are in flight)

  stage_load(t0);
  stage_store(0);
  __syncthreads();

  float dsum = 0.0f;
  // Per-step inputs of one 8-step tile, prepared by lane g for step
  // t0 + p*8 + g: dt, dt*u (handed to the channel's 8 lanes through xch), u
  // and the gate (kept by lane g for the output).  Steps past the chunk get
  // dt = dt*u = 0, i.e. they leave the states unchanged.
  struct Prep { float dl, xu, uu, gate; };
  auto prep = [&](int p, float uu, float dr, float zz) {
    Prep r;
    const bool valid = (int64_t)p * GL + g < nsteps;
    const float x = dr + bv;
    float spx = softplus(x);
    __asm__ volatile("" : "+v"(spx));
    const float dl = sp ? spx : x;
    r.dl = valid ? dl : 0.0f;
    r.xu = valid ? dl * uu : 0.0f;
    r.uu = uu;
    r.gate = (MODE == TMODE_FULL && HAS_Z) ? zz * sigmoid(zz) : 1.0f;
    return r;
  };
  // xch is double buffered: tile p+1's values are written while tile p's are
  // still in use (one wave: its LDS operations complete in program order).
  Prep cur = prep(0, pu0, pd0, pz0);
  pu0 = pu1; pd0 = pd1; pz0 = pz1;
  load_own(2, pu1, pd1, pz1);
  xch[0][cl][g] = make_float2(cur.dl, cur.xu);

  const int nprep = (int)((nsteps + GL - 1) / GL);
  for (int p = 0; p < nprep; ++p) {
    const int tile = p / (TB / GL);
    const int pt = p % (TB / GL);
    const int buf = tile & 1;
    const int64_t tb = t0 + (int64_t)tile * TB;
    const bool has_next_tile = tb + TB < t1;
    if (pt == 0 && has_next_tile) stage_load(tb + TB);

    float2 ex[GL];
#pragma unroll
    for (int j = 0; j < GL; j += 2) {
      const float4 v = *reinterpret_cast<const float4*>(&xch[p & 1][cl][j]);
      ex[j] = make_float2(v.x, v.y);
      ex[j + 1] = make_float2(v.z, v.w);
    }
    // next tile's per-step inputs (independent of this tile's recurrence)
    const Prep nxt = prep(p + 1, pu0, pd0, pz0);
    pu0 = pu1; pd0 = pd1; pz0 = pz1;
    load_own(p + 3, pu1, pd1, pz1);
    xch[(p + 1) & 1][cl][g] = make_float2(nxt.dl, nxt.xu);
    if (MODE == TMODE_SUMMARY) dsum += cur.dl;

    float ot[GL];                                  // this lane's partial readout per step
    const int ls0 = pt * GL;
#pragma unroll
    for (int jh = 0; jh < GL; jh += 4) {
      float4 bq[NS], cq[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        bq[i] = *reinterpret_cast<const float4*>(&sBC[buf][0][n0 + i][ls0 + jh]);
        if (MODE == TMODE_FULL)
          cq[i] = *reinterpret_cast<const float4*>(&sBC[buf][1][n0 + i][ls0 + jh]);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = jh + jj;
        const float dlj = ex[j].x, xuj = ex[j].y;
        float o = 0.0f;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const float bvj = jj == 0 ? bq[i].x : jj == 1 ? bq[i].y : jj == 2 ? bq[i].z : bq[i].w;
          const float dA = fast_exp2(dlj * A2[i]);
          h[i] = __builtin_fmaf(dA, h[i], xuj * bvj);
          if (MODE == TMODE_FULL) {
            const float cvj = jj == 0 ? cq[i].x : jj == 1 ? cq[i].y : jj == 2 ? cq[i].z : cq[i].w;
            o = __builtin_fmaf(cvj, h[i], o);
          }
        }
        ot[j] = o;
      }
    }
    if (MODE == TMODE_FULL) {
      const float o_own = reduce_scatter8(ot, g);   // full readout of step t0 + p*8 + g
      const float yv = __builtin_fmaf(Dv, cur.uu, o_own) * cur.gate;
      // tail lanes (d >= D) store channel D-1's value to channel D-1's
      // address; steps past the chunk fall outside the buffer and are dropped
      buf_st<T>(yv, rs_y, voff_own, p * soff_step);
    }
    cur = nxt;

    if (pt == TB / GL - 1 || p == nprep - 1) {
      if (has_next_tile) stage_store(buf ^ 1);
      __syncthreads();
    }
  }

  if (MODE == TMODE_SUMMARY) dsum = sum8(dsum);
  if (!active) return;
  if (MODE == TMODE_SUMMARY) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (n0 + i < N) a.chunk_state[((b * a.K + k) * N + n0 + i) * D + d] = h[i];
    if (g == 0) a.chunk_dsum[(b * a.K + k) * D + d] = dsum;
  } else if (a.last_state != nullptr && k == a.K - 1) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (n0 + i < N) st_param(a.last_state, (b * D + d) * N + n0 + i, a.param_dtype, h[i]);
  }
}

hipError_t launch_fwd_carry(const FwdArgs& a, hipStream_t s);  // ss_fwd.hip

template <typename T, int NS, bool HAS_Z>
static hipError_t launch_tile_t(const FwdArgs& a, hipStream_t s) {
  const T* U = static_cast<const T*>(a.u);
  const T* DL = static_cast<const T*>(a.delta);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  const T* Z = static_cast<const T*>(a.z);
  T* Y = static_cast<T*>(a.y);
  const int64_t nbd = (a.D + CPW - 1) / CPW;
  hipError_t e;
  if (a.K > 1) {
    const int64_t gs = a.Bn * (a.K - 1) * nbd;
    fwd_tile<T, NS, TMODE_SUMMARY, false><<<dim3((unsigned)gs), dim3(kBlockT), 0, s>>>(
        U, DL, Bm, Cm, Z, Y, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_fwd_carry(a, s)) != hipSuccess) return e;
  }
  const int64_t gf = a.Bn * a.K * nbd;
  fwd_tile<T, NS, TMODE_FULL, HAS_Z><<<dim3((unsigned)gf), dim3(kBlockT), 0, s>>>(
      U, DL, Bm, Cm, Z, Y, a);
  return hipGetLastError();
}

template <typename T, int NS>
static hipError_t launch_tile_ns(const FwdArgs& a, hipStream_t s) {
  return a.z ? launch_tile_t<T, NS, true>(a, s) : launch_tile_t<T, NS, false>(a, s);
}

template <typename T>
static hipError_t launch_tile_ty(const FwdArgs& a, int ns, hipStream_t s) {
  switch (ns) {
    case 1: return launch_tile_ns<T, 1>(a, s);
    case 2: return launch_tile_ns<T, 2>(a, s);
    case 4: return launch_tile_ns<T, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_tile(const FwdArgs& a, int io_dtype, int ns, hipStream_t s) {
  switch (io_dtype) {
    case 0: return launch_tile_ty<float>(a, ns, s);
    case 1: return launch_tile_ty<f16_t>(a, ns, s);
    case 2: return launch_tile_ty<bf16_t>(a, ns, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ss
