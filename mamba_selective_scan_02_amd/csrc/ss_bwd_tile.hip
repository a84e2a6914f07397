// Backward selective scan for N <= 16 with a channel's states split over 8
// lanes (gfx950).
//
// Same gradients and equations as ss_bwd.hip (chain rule through the
// recurrence of the baracuda-kernels page "src/attention/selective_scan.rs",
// "Algorithm summary"; gradient set of its SelectiveScanBackwardArgs;
// per-channel reverse sweep and fixed-order partial reductions as in stage B3
// of the mamba-rs page "mamba_ssm/gpu/backward.rs").  Mapping: 8 lanes own a
// channel (8 apart in the wave: lane_g / lane_channel in ss_device.h), lane g
// holds states n = g*NS .. g*NS+NS-1 (NS = 1, 2 or 4); a wave is 8 channels, a
// 256-lane workgroup 32; per 8-step tile, lane g prepares the per-step
// scalars of step t0 + 8j + g and hands them to the channel's lanes through
// LDS; sums over a channel's states are reduce-scatters over its 8 lanes
// (lane swaps and DPP).
//
// Time is cut into chunks of at most 64 steps (8 tiles; 32 steps with NS = 4):
//   bwd_tile_sum   per chunk, from zero: forward end state S, reverse summary
//                  Sb = sum_s (prod_{r<=s} a_r) g_s C_s (built per 8-step tile
//                  and combined with the tiles' decays), and sum of dt;
//   bwd_carry      (ss_bwd.hip) the forward and reverse chains over chunks;
//   bwd_tile_main  per chunk: pass 1 runs forward from the carried-in state
//                  and keeps the state at every tile start (LDS); pass 2 walks
//                  the tiles backwards, recomputes each tile's states and
//                  decays in registers and runs the adjoint from the carried
//                  end-of-chunk adjoint, reset at each tile start from a
//                  tile-level chain (accuracy: see pass 2).  dB / dC are summed over the
//                  workgroup's 32 channels through LDS in a fixed order and
//                  written as per-channel-block partials; dA / dD / dbias are
//                  written as per-chunk partials.
//   bwd_finalize_* (ss_bwd.hip) fixed-order sums of the partials.
#include "ss_device.h"
#include "ss_plan.h"

namespace ss {

namespace {

constexpr int kBT = 256;              // threads per workgroup
constexpr int BGL = 8;                // lanes per channel
constexpr int BCPW = kBT / BGL;       // channels per workgroup (32)
// Steps per chunk (at most): 64 (8 tiles) with NS <= 2 states per lane; 32
// with NS = 4, whose tile-start states and dB/dC rows take twice the LDS per
// step (two workgroups per CU either way).
template <int NS> constexpr int btc() { return NS <= 2 ? 64 : 32; }
// Resident waves per SIMD the main kernel's registers are held to.
template <int NS> constexpr int bmain_waves() { return NS <= 2 ? 3 : 2; }
constexpr int BXS = 9;                // exchange row stride (float4) per channel

}  // namespace

// Decoded position of a workgroup / lane (shared by the two kernels).
struct BTilePos {
  int g, cl;
  int64_t db, k, b, d, t0, t1, start;   // start: the sequence's first row
  bool active;
};

__device__ __forceinline__ BTilePos btile_pos(const BwdArgs& a) {
  BTilePos p;
  const int tid = threadIdx.x;
  p.g = lane_g(tid);
  p.cl = lane_channel(tid);
  int64_t blk = xcd_pair_remap(blockIdx.x, gridDim.x);
  p.db = blk % a.nwgd;
  blk /= a.nwgd;
  p.k = blk % a.K;
  p.b = blk / a.K;
  const int64_t d_raw = p.db * BCPW + p.cl;
  p.active = d_raw < a.D;
  p.d = p.active ? d_raw : a.D - 1;
  p.t0 = p.k * a.chunk_len;
  const SeqRows sr = seq_rows(a.cu, p.b, a.L, a.Lt);
  p.start = sr.start;
  p.t1 = (p.t0 + a.chunk_len < sr.len) ? p.t0 + a.chunk_len : sr.len;
  if (p.t1 < p.t0) p.t1 = p.t0;                 // a chunk past a short sequence's end
  return p;
}

// Stage the chunk's B and C rows as f32, [n][t], rows padded; states n >= N
// and steps past the chunk are zero.
template <typename T, int NP, int BTC, int BTS>
__device__ __forceinline__ void bstage(float (*sB)[BTS], float (*sC)[BTS], const T* B, const T* C,
                                       int64_t row0, int64_t nsteps,
                                       int64_t N, int64_t ldb, int64_t ldc) {
  constexpr int ES = sizeof(T);
  const auto rB = make_rsrc(B + row0 * ldb, rows_bytes(nsteps, ldb, N, ES));
  const auto rC = make_rsrc(C + row0 * ldc, rows_bytes(nsteps, ldc, N, ES));
  for (int e = threadIdx.x; e < BTC * NP; e += kBT) {
    const int tt = e / NP, n = e % NP;
    const bool ok = n < N;
    const int nn = ok ? n : 0;
    const float vb = buf_ld<T>(rB, (tt * (int)ldb + nn) * ES, 0);
    const float vc = buf_ld<T>(rC, (tt * (int)ldc + nn) * ES, 0);
    sB[n][tt] = ok ? vb : 0.0f;
    sC[n][tt] = ok ? vc : 0.0f;
  }
}

// ----------------------------------------------------------------- summary

template <typename T, int NS, bool HAS_Z>
__global__ __launch_bounds__(kBT) void bwd_tile_sum(const T* __restrict__ u_in,
                                                    const T* __restrict__ delta_in,
                                                    const T* __restrict__ B_in,
                                                    const T* __restrict__ C_in,
                                                    const T* __restrict__ z_in,
                                                    const T* __restrict__ dy_in, const BwdArgs a) {
  constexpr int NP = NS * BGL;
  constexpr int ES = sizeof(T);
  constexpr int BTC = btc<NS>(), BTS = BTC + 4;
  __shared__ __attribute__((aligned(16))) float sB[NP][BTS];
  __shared__ __attribute__((aligned(16))) float sC[NP][BTS];
  __shared__ __attribute__((aligned(16))) float4 xch[BCPW][BXS];
  const BTilePos P = btile_pos(a);
  const int g = P.g, cl = P.cl, n0 = g * NS;
  const int64_t D = a.D, N = a.N, b = P.b, d = P.d;
  const int64_t nsteps = P.t1 - P.t0;

  bstage<T, NP, BTC, BTS>(sB, sC, B_in, C_in, P.start + P.t0, nsteps, N, a.ldb, a.ldc);

  // Sb is built two-level: per tile from its own start (E, sbl) and then
  // Sb += (decay of the chunk's earlier tiles) * sbl, the decay of a tile
  // being exp2(A2 * sum of its dt); a product of per-step decays over 64 steps
  // would drift by one rounding per step.  (Running sbl backwards from the
  // tile's end, sbl <- a_s (g_s C_s + sbl), takes two operations per update
  // instead of three, but holds the tile's decays and C in registers: 95
  // instead of 73 VGPRs, 5 instead of 6 waves per SIMD, and no faster in a
  // kernel-level A/B: 53.5 / 52.9 against 54.4 / 53.2 us.)
  float A2[NS], h[NS], Sb[NS], PP[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int n = n0 + i;
    A2[i] = n < N ? ld_param(a.A, d * N + n, a.param_dtype) * kLog2e : 0.0f;
    h[i] = 0.0f;
    Sb[i] = 0.0f;
    PP[i] = 1.0f;
  }
  const float bv = a.bias ? ld_param(a.bias, d, a.param_dtype) : 0.0f;
  const bool sp = a.softplus != 0;
  const int64_t row0 = (P.start + P.t0) * D;
  const auto rs_u = make_rsrc(u_in + row0, nsteps * D * ES);
  const auto rs_d = make_rsrc(delta_in + row0, nsteps * D * ES);
  const auto rs_z = make_rsrc(HAS_Z ? z_in + row0 : u_in + row0, nsteps * D * ES);
  const auto rs_y = make_rsrc(dy_in + row0, nsteps * D * ES);
  const int voff = (int)((g * D + d) * ES);
  const int sstep = (int)(BGL * D * ES);
  __syncthreads();

  float dsum = 0.0f;
  const int ntile = (int)((nsteps + BGL - 1) / BGL);
  // the lane's own-step inputs, loaded one tile ahead
  auto raw = [&](int j, float& uu, float& dr, float& dyv, float& zz) {
    const int so = __builtin_amdgcn_readfirstlane(j * sstep);
    uu = buf_ld<T>(rs_u, voff, so);
    dr = buf_ld<T>(rs_d, voff, so);
    dyv = buf_ld<T>(rs_y, voff, so);
    zz = HAS_Z ? buf_ld<T>(rs_z, voff, so) : 0.0f;
  };
  float nu, nd, ny, nz;
  raw(0, nu, nd, ny, nz);
  for (int j = 0; j < ntile; ++j) {
    const float uu = nu, dr = nd, dyv = ny, zz = nz;
    raw(j + 1, nu, nd, ny, nz);                       // past the chunk: reads 0
    const bool valid = (int64_t)j * BGL + g < nsteps;
    const float x = dr + bv;
    float spx = softplus_acc(x);
    __asm__ volatile("" : "+v"(spx));
    float dl = sp ? spx : x;
    float gg = HAS_Z ? dyv * zz * sigmoid(zz) : dyv;
    dl = valid ? dl : 0.0f;
    const float xu = valid ? dl * uu : 0.0f;
    gg = valid ? gg : 0.0f;
    dsum += dl;
    xch[cl][g] = make_float4(dl, xu, gg, 0.0f);
    const float dst = sum8(dl);       // the tile's sum of dt (same on the 8 lanes)
    float4 ex[BGL];
#pragma unroll
    for (int s = 0; s < BGL; ++s) ex[s] = xch[cl][s];
    float E[NS], sbl[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      E[i] = 1.0f;
      sbl[i] = 0.0f;
    }
#pragma unroll
    for (int sh = 0; sh < BGL; sh += 4) {
      float4 bq[NS], cq[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        bq[i] = *reinterpret_cast<const float4*>(&sB[n0 + i][j * BGL + sh]);
        cq[i] = *reinterpret_cast<const float4*>(&sC[n0 + i][j * BGL + sh]);
      }
      float ea[4 * NS];                    // the half tile's decays as one run
#pragma unroll
      for (int ss = 0; ss < 4; ++ss)
#pragma unroll
        for (int i = 0; i < NS; ++i) ea[ss * NS + i] = ex[sh + ss].x * A2[i];
      exp2_run(ea);
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        const float4 e = ex[sh + ss];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const float bvs = ss == 0 ? bq[i].x : ss == 1 ? bq[i].y : ss == 2 ? bq[i].z : bq[i].w;
          const float cvs = ss == 0 ? cq[i].x : ss == 1 ? cq[i].y : ss == 2 ? cq[i].z : cq[i].w;
          const float av = ea[ss * NS + i];
          h[i] = __builtin_fmaf(av, h[i], e.y * bvs);
          E[i] *= av;
          sbl[i] = __builtin_fmaf(E[i], e.z * cvs, sbl[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      Sb[i] = __builtin_fmaf(PP[i], sbl[i], Sb[i]);
      PP[i] *= fast_exp2(A2[i] * dst);
    }
  }
  dsum = sum8(dsum);
  if (!P.active) return;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int n = n0 + i;
    if (n < N) {
      const int64_t o = ((b * a.K + P.k) * N + n) * D + d;
      a.fstate[o] = h[i];
      a.bstate[o] = Sb[i];
    }
  }
  if (g == 0) a.dsum[(b * a.K + P.k) * D + d] = dsum;
}

// -------------------------------------------------------------------- main

template <typename T, int NS, bool HAS_Z>
__global__ __launch_bounds__(kBT, bmain_waves<NS>()) void bwd_tile_main(const T* __restrict__ u_in,
                                                     const T* __restrict__ delta_in,
                                                     const T* __restrict__ B_in,
                                                     const T* __restrict__ C_in,
                                                     const T* __restrict__ z_in,
                                                     const T* __restrict__ dy_in,
                                                     T* __restrict__ du_out,
                                                     T* __restrict__ ddelta_out,
                                                     T* __restrict__ dz_out, const BwdArgs a) {
  constexpr int NP = NS * BGL;
  constexpr int ES = sizeof(T);
  constexpr int RP = BGL * NP + 4;      // reduction row (one channel: 8 steps x NP) + pad
  constexpr int BTC = btc<NS>(), BNT = BTC / BGL, BTS = BTC + 4;
  __shared__ __attribute__((aligned(16))) float sB[NP][BTS];
  __shared__ __attribute__((aligned(16))) float sC[NP][BTS];
  __shared__ __attribute__((aligned(16))) float4 xch[BCPW][BXS];
  __shared__ __attribute__((aligned(16))) float hts[BNT][NS][kBT];  // tile-start states
  // dB / dC of one tile, per pair of channels (pre-summed across the pair)
  __shared__ __attribute__((aligned(16))) float red[2][BCPW / 2][RP];
  const BTilePos P = btile_pos(a);
  const int tid = threadIdx.x;
  const int g = P.g, cl = P.cl, n0 = g * NS;
  const int64_t D = a.D, N = a.N, K = a.K, b = P.b, d = P.d, k = P.k;
  const int64_t nsteps = P.t1 - P.t0;

  bstage<T, NP, BTC, BTS>(sB, sC, B_in, C_in, P.start + P.t0, nsteps, N, a.ldb, a.ldc);

  float A2[NS], An[NS], h[NS], dh[NS], dA_acc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int n = n0 + i;
    An[i] = n < N ? ld_param(a.A, d * N + n, a.param_dtype) : 0.0f;
    A2[i] = An[i] * kLog2e;
    h[i] = (k > 0 && n < N) ? a.fstate[((b * K + (k - 1)) * N + n) * D + d]
           : (a.h0 && n < N) ? ld_param(a.h0, (b * D + d) * N + n, a.param_dtype)
                             : 0.0f;
    dh[i] = (k < K - 1 && n < N) ? a.bstate[((b * K + (k + 1)) * N + n) * D + d] : 0.0f;
    dA_acc[i] = 0.0f;
  }
  const float bv = a.bias ? ld_param(a.bias, d, a.param_dtype) : 0.0f;
  const float Dv = a.Dskip ? ld_param(a.Dskip, d, a.param_dtype) : 0.0f;
  const bool sp = a.softplus != 0;
  const int64_t row0 = (P.start + P.t0) * D;
  const int64_t rbytes = nsteps * D * ES;
  const auto rs_u = make_rsrc(u_in + row0, rbytes);
  const auto rs_d = make_rsrc(delta_in + row0, rbytes);
  const auto rs_z = make_rsrc(HAS_Z ? z_in + row0 : u_in + row0, rbytes);
  const auto rs_y = make_rsrc(dy_in + row0, rbytes);
  const auto ws_du = make_rsrc(du_out + row0, rbytes);
  const auto ws_dd = make_rsrc(ddelta_out + row0, rbytes);
  const auto ws_dz = make_rsrc(HAS_Z ? dz_out + row0 : du_out + row0, HAS_Z ? rbytes : 0);
  const int voff = (int)((g * D + d) * ES);
  // Tail channels (d >= D) compute a copy of channel D-1 with zero input
  // drive and gradient (so they add nothing to the dB / dC sums); their
  // stores go past the buffer range and are dropped.
  const int voff_st = P.active ? voff : (int)rbytes;
  const int sstep = (int)(BGL * D * ES);
  // (uniform, and kept in a scalar register: the tile index feeds the buffer
  // instructions' scalar offsets, which the compiler otherwise fills through
  // per-lane loops when it keeps the index in a vector register)
  const int ntile = __builtin_amdgcn_readfirstlane((int)((nsteps + BGL - 1) / BGL));
  __syncthreads();

  // raw inputs of the lane's own step in tile j (loaded one tile ahead)
  struct Raw { float uu, dr, dyv, zz; };
  auto raw = [&](int j, bool full) {
    Raw r;
    const int so = __builtin_amdgcn_readfirstlane(j * sstep);
    r.uu = buf_ld<T>(rs_u, voff, so);
    r.dr = buf_ld<T>(rs_d, voff, so);
    r.dyv = full ? buf_ld<T>(rs_y, voff, so) : 0.0f;
    r.zz = (full && HAS_Z) ? buf_ld<T>(rs_z, voff, so) : 0.0f;
    return r;
  };
  // per-step scalars of the lane's own step in tile j
  struct Own { float uu, dl, xu, gg, sx, gz; bool valid; };
  auto own = [&](int j, bool full, const Raw& rw) {
    Own o;
    o.uu = rw.uu;
    const float dr = rw.dr;
    o.valid = (int64_t)j * BGL + g < nsteps;
    const bool drive = o.valid && P.active;
    const float x = dr + bv;
    float spx = softplus_acc(x);
    __asm__ volatile("" : "+v"(spx));
    const float dl = sp ? spx : x;
    o.dl = o.valid ? dl : 0.0f;
    o.xu = drive ? dl * o.uu : 0.0f;
    o.gg = 0.0f;
    o.sx = 1.0f;
    o.gz = 0.0f;
    if (full) {
      const float dyv = rw.dyv;
      float gv = dyv;
      if (HAS_Z) {
        const float zz = rw.zz;
        const float s = sigmoid(zz);
        gv = dyv * zz * s;
        o.gz = dyv * s * __builtin_fmaf(zz, 1.0f - s, 1.0f);
      }
      o.gg = drive ? gv : 0.0f;
      float sxv = sigmoid_acc(x);
      __asm__ volatile("" : "+v"(sxv));
      o.sx = sp ? sxv : 1.0f;
    }
    return o;
  };

  // ---- pass 1: forward from the carried-in state, keep tile-start states
  Raw nxt = raw(0, false);
  for (int j = 0; j < ntile; ++j) {
#pragma unroll
    for (int i = 0; i < NS; ++i) hts[j][i][tid] = h[i];
    const Raw cur = nxt;
    nxt = raw(j + 1, false);                          // past the chunk: reads 0
    const Own o = own(j, false, cur);
    xch[cl][g] = make_float4(o.dl, o.xu, 0.0f, 0.0f);
    float4 ex[BGL];
#pragma unroll
    for (int s = 0; s < BGL; ++s) ex[s] = xch[cl][s];
#pragma unroll
    for (int sh = 0; sh < BGL; sh += 4) {
      float4 bq[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i)
        bq[i] = *reinterpret_cast<const float4*>(&sB[n0 + i][j * BGL + sh]);
      float ea[4 * NS];                    // the half tile's decays as one run
#pragma unroll
      for (int ss = 0; ss < 4; ++ss)
#pragma unroll
        for (int i = 0; i < NS; ++i) ea[ss * NS + i] = ex[sh + ss].x * A2[i];
      exp2_run(ea);
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        const float4 e = ex[sh + ss];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const float bvs = ss == 0 ? bq[i].x : ss == 1 ? bq[i].y : ss == 2 ? bq[i].z : bq[i].w;
          h[i] = __builtin_fmaf(ea[ss * NS + i], h[i], e.y * bvs);
        }
      }
    }
  }

  // ---- pass 2: tiles backwards.  Within a tile the adjoint dh runs step by
  // step; at each tile start it is replaced by the tile-level chain
  // cj <- exp2(A2 * tile sum of dt) * cj + (tile's reverse summary from zero),
  // so that rounding accumulates over at most 8 steps plus one step per tile.
  float cj[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) cj[i] = dh[i];
  float dD_acc = 0.0f, db_acc = 0.0f;
  Raw prv = raw(ntile - 1, true);
  for (int j = ntile - 1; j >= 0; --j) {
    const Raw cur = prv;
    prv = raw(__builtin_amdgcn_readfirstlane(j > 0 ? j - 1 : 0), true);
    const Own o = own(j, true, cur);
    const float dst = sum8(o.dl);
    xch[cl][g] = make_float4(o.dl, o.xu, o.gg, 0.0f);
    float4 ex[BGL];
#pragma unroll
    for (int s = 0; s < BGL; ++s) ex[s] = xch[cl][s];

    // recompute the tile's states and decays from the tile-start state
    float hh[BGL][NS], aa[BGL][NS], h0[NS], po[BGL];
#pragma unroll
    for (int i = 0; i < NS; ++i) h0[i] = hts[j][i][tid];
    float bt[BGL][NS], ct[BGL][NS];
#pragma unroll
    for (int sh = 0; sh < BGL; sh += 4) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const float4 bq = *reinterpret_cast<const float4*>(&sB[n0 + i][j * BGL + sh]);
        const float4 cq = *reinterpret_cast<const float4*>(&sC[n0 + i][j * BGL + sh]);
        bt[sh][i] = bq.x; bt[sh + 1][i] = bq.y; bt[sh + 2][i] = bq.z; bt[sh + 3][i] = bq.w;
        ct[sh][i] = cq.x; ct[sh + 1][i] = cq.y; ct[sh + 2][i] = cq.z; ct[sh + 3][i] = cq.w;
      }
    }
#pragma unroll
    for (int sh = 0; sh < BGL; sh += 4) {   // the tile's decays in runs of exps
      float ea[4 * NS];
#pragma unroll
      for (int ss = 0; ss < 4; ++ss)
#pragma unroll
        for (int i = 0; i < NS; ++i) ea[ss * NS + i] = ex[sh + ss].x * A2[i];
      exp2_run(ea);
#pragma unroll
      for (int ss = 0; ss < 4; ++ss)
#pragma unroll
        for (int i = 0; i < NS; ++i) aa[sh + ss][i] = ea[ss * NS + i];
    }
#pragma unroll
    for (int s = 0; s < BGL; ++s) {
      float ov = 0.0f;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const float prev = s > 0 ? hh[s - 1][i] : h0[i];
        hh[s][i] = __builtin_fmaf(aa[s][i], prev, ex[s].y * bt[s][i]);
        ov = __builtin_fmaf(ct[s][i], hh[s][i], ov);
      }
      po[s] = ov;
    }
    // adjoint sweep (dl0: the tile's adjoint from zero at its end)
    float pdua[BGL], pddl[BGL], dl0[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) dl0[i] = 0.0f;
#pragma unroll
    for (int s = BGL - 1; s >= 0; --s) {
      float vdua = 0.0f, vddl = 0.0f;
      float vb[NS], vc[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        dh[i] = __builtin_fmaf(ex[s].z, ct[s][i], dh[i]);          // dL/dh_t
        dl0[i] = __builtin_fmaf(ex[s].z, ct[s][i], dl0[i]);
        vc[i] = ex[s].z * hh[s][i];
        vb[i] = dh[i] * ex[s].y;
        vdua = __builtin_fmaf(dh[i], bt[s][i], vdua);
        const float m = dh[i] * aa[s][i];
        const float q = m * (s > 0 ? hh[s - 1][i] : h0[i]);
        vddl = __builtin_fmaf(q, An[i], vddl);
        dA_acc[i] = __builtin_fmaf(q, ex[s].x, dA_acc[i]);
        dh[i] = m;
        dl0[i] *= aa[s][i];
      }
      pdua[s] = vdua;
      pddl[s] = vddl;
      // dB / dC of (step s, these states) for the workgroup reduction: the
      // channel pair (2m, 2m + 1), neighbouring lanes with the same g, is
      // summed first (tail lanes contribute exact zeros).  Both lanes of the
      // pair hold the same sum (the two addends swapped), so both store it to
      // the pair's slot: no branch, and the DPP move fuses into the add.
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        // (rounded products first: an fma would round the two lanes' sums differently)
        __asm__ volatile("" : "+v"(vb[i]), "+v"(vc[i]));
        vb[i] += dpp<0xB1>(vb[i]);       // quad_perm [1,0,3,2]: the pair's other channel
        vc[i] += dpp<0xB1>(vc[i]);
      }
      if constexpr (NS == 4) {
        *reinterpret_cast<float4*>(&red[0][cl >> 1][s * NP + n0]) =
            make_float4(vb[0], vb[1], vb[2], vb[3]);
        *reinterpret_cast<float4*>(&red[1][cl >> 1][s * NP + n0]) =
            make_float4(vc[0], vc[1], vc[2], vc[3]);
      } else if constexpr (NS == 2) {
        *reinterpret_cast<float2*>(&red[0][cl >> 1][s * NP + n0]) = make_float2(vb[0], vb[1]);
        *reinterpret_cast<float2*>(&red[1][cl >> 1][s * NP + n0]) = make_float2(vc[0], vc[1]);
      } else {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          red[0][cl >> 1][s * NP + n0 + i] = vb[i];
          red[1][cl >> 1][s * NP + n0 + i] = vc[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      cj[i] = __builtin_fmaf(fast_exp2(A2[i] * dst), cj[i], dl0[i]);
      dh[i] = cj[i];
    }
    // per-step sums over the channel's states: lane g gets its own step's
    const float o_own = reduce_scatter8(po, g);
    const float dua_own = reduce_scatter8(pdua, g);
    const float ddl_own = reduce_scatter8(pddl, g);
    const float du = __builtin_fmaf(o.dl, dua_own, o.gg * Dv);
    const float dx = o.valid ? __builtin_fmaf(o.uu, dua_own, ddl_own) * o.sx : 0.0f;
    const int so = __builtin_amdgcn_readfirstlane(j * sstep);
    buf_st<T>(du, ws_du, voff_st, so);       // steps past the chunk are dropped
    buf_st<T>(dx, ws_dd, voff_st, so);
    if (HAS_Z) buf_st<T>(o.gz * __builtin_fmaf(Dv, o.uu, o_own), ws_dz, voff_st, so);
    dD_acc = __builtin_fmaf(o.gg, o.uu, dD_acc);
    db_acc += dx;

    // dB / dC of this tile: sum over the workgroup's 16 channel pairs (fixed order)
    __syncthreads();
    for (int v = tid; v < 2 * BGL * NP; v += kBT) {
      const int w = v / (BGL * NP), sn = v % (BGL * NP);
      const int s = sn / NP, n = sn % NP;
      float acc = 0.0f;
#pragma unroll 8
      for (int c = 0; c < BCPW / 2; ++c) acc += red[w][c][sn];
      const int64_t t = (int64_t)j * BGL + s;
      if (n < N && t < nsteps)
        a.part_bc[((P.start + P.t0 + t) * a.nwgd + P.db) * 2 * N + w * N + n] = acc;
    }
    __syncthreads();
  }
  // tail channels (d >= D) duplicate channel D-1: they must not add to the sums
  if (!P.active) { dD_acc = 0.0f; db_acc = 0.0f; }
  dD_acc = sum8(dD_acc);
  db_acc = sum8(db_acc);
  if (!P.active) return;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (n0 + i < N) a.part_dA[((b * a.KG + k) * N + n0 + i) * D + d] = dA_acc[i];
    // after tile 0 of chunk 0, dh is the adjoint carried past t = 0: dL/dh_{-1}
    if (k == 0 && a.dh0 && n0 + i < N)
      st_param(a.dh0, (b * D + d) * N + n0 + i, a.param_dtype, dh[i]);
  }
  if (g == 0) {
    a.part_dD[(b * a.KG + k) * D + d] = dD_acc;
    a.part_db[(b * a.KG + k) * D + d] = db_acc;
  }
}

hipError_t launch_bwd_carry(const BwdArgs& a, hipStream_t s);   // ss_bwd.hip
hipError_t launch_bwd_finalize(const BwdArgs& a, hipStream_t s);  // ss_bwd.hip

template <typename T, int NS, bool HAS_Z>
static hipError_t launch_btile_t(const BwdArgs& a, hipStream_t s) {
  const T* U = static_cast<const T*>(a.u);
  const T* DL = static_cast<const T*>(a.delta);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  const T* Z = static_cast<const T*>(a.z);
  const T* DY = static_cast<const T*>(a.dy);
  const unsigned grid = (unsigned)(a.Bn * a.K * a.nwgd);
  hipError_t e;
  if (a.K > 1) {
    bwd_tile_sum<T, NS, HAS_Z><<<dim3(grid), dim3(kBT), 0, s>>>(U, DL, Bm, Cm, Z, DY, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_bwd_carry(a, s)) != hipSuccess) return e;
  }
  bwd_tile_main<T, NS, HAS_Z><<<dim3(grid), dim3(kBT), 0, s>>>(
      U, DL, Bm, Cm, Z, DY, static_cast<T*>(a.du), static_cast<T*>(a.ddelta),
      static_cast<T*>(a.dz), a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_bwd_finalize(a, s);
}

template <typename T>
static hipError_t launch_btile_ty(const BwdArgs& a, int ns, hipStream_t s) {
  const bool z = a.z != nullptr;
  if (ns == 1) return z ? launch_btile_t<T, 1, true>(a, s) : launch_btile_t<T, 1, false>(a, s);
  if (ns == 2) return z ? launch_btile_t<T, 2, true>(a, s) : launch_btile_t<T, 2, false>(a, s);
  if (ns == 4) return z ? launch_btile_t<T, 4, true>(a, s) : launch_btile_t<T, 4, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_tile(const BwdArgs& a, int ns, hipStream_t s) {
  switch (a.io_dtype) {
    case 0: return launch_btile_ty<float>(a, ns, s);
    case 1: return launch_btile_ty<f16_t>(a, ns, s);
    case 2: return launch_btile_ty<bf16_t>(a, ns, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ss
