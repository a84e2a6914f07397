// Forward selective scan with a channel's states split over 8 lanes (gfx950).
//
// Same recurrence as ss_fwd_scan.h (baracuda-kernels page
// "src/attention/selective_scan.rs", module docs, "Algorithm summary"), for
// N <= 64.  Mapping:
//
//   * 8 lanes own one channel d, all in one row of 16 lanes of the wave
//     (wide_g / wide_channel: placed so that the readout's first two reduce
//     stages are bank-masked DPP adds), and lane g of the channel holds states
//     n = g*NS .. g*NS+NS-1 (NS = 1, 2, 4 or 8).  A wave covers 8 channels, a
//     256-lane workgroup 32.  This gives 8x the waves of one lane per
//     channel, which the wave-per-SIMD issue rate needs (a lone wave issues
//     far below the VALU rate; several resident waves per SIMD are needed).
//   * Per-(t, d) work is time-shared: in every tile of 8 steps, lane g loads
//     u / delta / z of step t0+g, computes dt = softplus(delta + bias),
//     dt*u and the gate silu(z) for that step only, and hands (dt, dt*u) to
//     the other 7 lanes of its channel through a per-wave LDS exchange.
//   * The readout sum over a channel's states is a sum over its 8 lanes, done
//     once per 8-step tile as a reduce-scatter through DPP moves within the
//     row (the same code in both kernels, so their results agree bit for
//     bit): lane g ends with the sum of step t0+g and applies the skip term
//     and the gate to it.
//   * The decays of each half tile issue as one run of exps (exp2_run).
//   * B and C are staged per workgroup in LDS as f32, [n][t] per 64-step tile,
//     double buffered, rows padded to 68 floats (16-byte aligned, conflict-free
//     128-bit reads); states n >= N are zero rows, so padded states stay 0.
//
// Chunked sequences share the workspace layout and the carry of ss_fwd_scan.h.
// fwd_tile follows its two-level scheme (summaries from zero, carry, a final
// pass from the carried states).  fwd_wide writes y in its first pass:
//   LOCAL  runs every chunk from h = 0 and writes y, the chunk end states and
//          the chunks' dt sums;
//   carry  turns them into the true state entering each chunk;
//   FIXUP  reruns each chunk from that state beside a copy of the LOCAL
//          recurrence, writing y, and stops at the first stage end (every 32
//          or 64 steps) at which all states of the workgroup equal the copy's
//          bit for bit.
// From that step on the two passes perform the same operations on the same
// values, so the LOCAL pass's y of the rest of the chunk is exactly what the
// rerun would write: the result is that of a full final pass.  Decaying states
// forget their start within tens to hundreds of steps, so FIXUP usually
// covers a few stages per chunk; states that never forget it (A = 0) make it a
// full second pass.
#include <type_traits>

#include "ss_device.h"

namespace ss {

namespace {

constexpr int kBlockT = 256;
constexpr int GL = 8;                 // lanes per channel (the lane maps below assume 8)
constexpr int CPW = kBlockT / GL;     // channels per workgroup (32)
constexpr int TB = 64;                // steps per B/C staging tile
constexpr int TS = 68;                // LDS row stride of a staged row (floats)
constexpr int XS = 10;                // exchange row stride (float2) per channel

}  // namespace

// FULL: one pass from h0 (or, after a carry, from the carried state).
// SUMMARY: chunk end state and dt sum from h = 0 (fwd_tile's chunked scheme).
// LOCAL / FIXUP: fwd_wide's chunked scheme (see launch_tile_t).
enum { TMODE_FULL = 0, TMODE_SUMMARY = 1, TMODE_LOCAL = 2, TMODE_FIXUP = 3 };

// Resident waves per SIMD the register budget is held to: a 2.8B-shaped grid
// (5120 waves of 8 channels) is exactly 5 waves on each of the 1024 SIMDs, and
// 5 waves fit 96 VGPRs.  NS = 4 needs more registers and gets 3.
// The fix-up pass carries a second set of states and is short: 4 waves.
template <int NS, int MODE = TMODE_FULL>
constexpr int tile_waves_per_simd() {
  return NS <= 2 ? (MODE == TMODE_FIXUP ? 4 : 5) : NS <= 4 ? 3 : 2;
}

// Lane map of the forward tile kernels: a channel's 8 lanes lie in one row of
// 16 lanes, wave lane l = 16 r + 8 q + 4 s + 2 c + p holding lane
// g = 4 q + 2 s + p of channel c + 2 r (of the wave's 8).  The partners of the readout's first two
// butterfly stages (g ^ 4 = l ^ 8, g ^ 2 = l ^ 4) then sit in other 4-lane
// banks of the row, so each of those stages is two DPP adds per value that
// write disjoint banks (bank_mask), with no selects; the last stage (g ^ 1 =
// l ^ 1) is a quad permutation.
__device__ __forceinline__ int wide_g(int tid) { return (tid & 1) | ((tid >> 1) & 6); }
__device__ __forceinline__ int wide_channel(int tid) {
  return ((tid >> 6) << 3) | ((tid >> 3) & 6) | ((tid >> 1) & 1);
}

// Reduce-scatter over a channel's 8 lanes (wide_g map): lane g holds o[0..7]
// and ends with the channel's sum of o[g]; stage s adds partners g ^ 4, g ^ 2,
// g ^ 1 (a lane keeps the half of its values picked by that bit of g).  Stage 1: lanes of banks 0-1 (g < 4) add the row_ror:8
// partner's o[k] to theirs, banks 2-3 its o[4 + k]; stage 2: banks 0 and 2
// take their partner 4 lanes up (row_ror:12: lane i reads lane i - 12 mod 16),
// banks 1 and 3 the one 4 lanes down (row_ror:4).  The DPP adds are written
// out (the compiler does not form bank-masked adds); s_nop 1 gives the two
// wait states a DPP read of a VGPR written by the previous VALU op needs.
// 12 DPP adds, 2 selects, 1 DPP add (a select-based version: 14 selects and
// 7 DPP adds).
__device__ __forceinline__ float reduce_scatter8_banked(const float (&o)[8], int g) {
  float a0, a1, a2, a3, b0, b1;
  __asm__ volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %6, %6 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %10, %10 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %7, %7 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %11, %11 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %8, %8 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %12, %12 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %9, %9 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %13, %13 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %4, %0, %0 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %4, %2, %2 row_ror:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %5, %1, %1 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %5, %3, %3 row_ror:4 row_mask:0xf bank_mask:0xa"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1)
      : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "v"(o[5]), "v"(o[6]),
        "v"(o[7]));
  const bool b0sel = (g & 1) != 0;
  const float keep = b0sel ? b1 : b0;
  const float send = b0sel ? b0 : b1;
  return keep + dpp<0xB1>(send);          // quad_perm [1,0,3,2]: lane l ^ 1
}

template <typename T, int NS, int MODE, bool HAS_Z>
__global__ __launch_bounds__(kBlockT, tile_waves_per_simd<NS>()) void fwd_tile(const T* __restrict__ u_in,
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
  const int g = wide_g(tid);
  const int cl = wide_channel(tid);
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
    A2[i] = n < N ? ld_param(a.A, d * N + n, a.param_dtype) * kLog2e : 0.0f;
    h[i] = 0.0f;
    if (MODE == TMODE_FULL && k > 0 && n < N)
      h[i] = a.chunk_state[((b * a.K + (k - 1)) * N + n) * D + d];
    else if (MODE == TMODE_FULL && k == 0 && n < N && a.h0)
      h[i] = ld_param(a.h0, (b * D + d) * N + n, a.param_dtype);
  }
  const float Dv = a.Dskip ? ld_param(a.Dskip, d, a.param_dtype) : 0.0f;
  const float bv = a.bias ? ld_param(a.bias, d, a.param_dtype) : 0.0f;
  const bool sp = a.softplus != 0;

  // Streamed tensors through buffer resources covering this chunk's rows:
  // the lane's own-step element (t0 + p*8 + g, d) sits at byte offset
  // voff_own + soff(p), steps past the chunk read 0 / are not stored.
  constexpr int ES = sizeof(T);
  const int64_t nsteps = t1 - t0;
  const int64_t row0 = (sr.start + t0) * D;
  const auto rs_u = make_rsrc(u_in + row0, nsteps * D * ES);
  const auto rs_d = make_rsrc(delta_in + row0, nsteps * D * ES);
  const auto rs_z = make_rsrc(HAS_Z ? z_in + row0 : u_in + row0, nsteps * D * ES);
  const auto rs_y = make_rsrc(y_out + row0, nsteps * D * ES);
  const int voff_own = (int)((g * D + d) * ES);
  const int soff_step = (int)(GL * D * ES);            // one 8-step tile
  const auto rs_B = make_rsrc(B_in + (sr.start + t0) * a.ldb, rows_bytes(nsteps, a.ldb, N, ES));
  const auto rs_C = make_rsrc(C_in + (sr.start + t0) * a.ldc, rows_bytes(nsteps, a.ldc, N, ES));
  const int ldb = (int)a.ldb, ldc = (int)a.ldc;

  // ---- B / C staging (whole workgroup) ----
  float rb[RB], rc[RB];
  auto stage_load = [&](int64_t tb) {
    const int trow = (int)(tb - t0);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int e = tid + r * kBlockT;
      const int tt = e / NP, n = e % NP;
      const bool ok = n < N;                       // rows past the chunk read 0
      const int nn = ok ? n : 0;
      const float vb = buf_ld<T>(rs_B, ((trow + tt) * ldb + nn) * ES, 0);
      rb[r] = ok ? vb : 0.0f;
      if (MODE == TMODE_FULL) {
        const float vc = buf_ld<T>(rs_C, ((trow + tt) * ldc + nn) * ES, 0);
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
    const bool valid = p * GL + g < (int)nsteps;
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

  // The time loop runs 64-step stages (8 tiles, unrolled, so that every LDS
  // offset is an immediate and the prefetch registers rotate by renaming).
  // The last stage stops after the chunk's last tile; inside that tile, steps
  // past the chunk are identity steps (dt = 0) whose stores fall outside the
  // buffer range and are dropped.
  const int nstage = (int)((nsteps + TB - 1) / TB);
  for (int st = 0; st < nstage; ++st) {
    const int buf = st & 1;
    const bool has_next = st + 1 < nstage;
    if (has_next) stage_load(t0 + (int64_t)(st + 1) * TB);
    // (the summary pass, with no readout to order the exps, would hoist them
    //  across the unrolled tiles and spill; it keeps a rolled loop)
    constexpr int kUnroll = MODE == TMODE_FULL ? TB / GL : 1;
#pragma unroll kUnroll
    for (int pt = 0; pt < TB / GL; ++pt) {
      if (pt * GL >= (int)nsteps - st * TB) break;   // tiles past the chunk (uniform)
      const int p = st * (TB / GL) + pt;
      float2 ex[GL];
#pragma unroll
      for (int j = 0; j < GL; j += 2) {
        const float4 v = *reinterpret_cast<const float4*>(&xch[pt & 1][cl][j]);
        ex[j] = make_float2(v.x, v.y);
        ex[j + 1] = make_float2(v.z, v.w);
      }
      // next tile's per-step inputs (independent of this tile's recurrence)
      const Prep nxt = prep(p + 1, pu0, pd0, pz0);
      pu0 = pu1; pd0 = pd1; pz0 = pz1;
      load_own(p + 3, pu1, pd1, pz1);
      xch[(pt + 1) & 1][cl][g] = make_float2(nxt.dl, nxt.xu);
      if (MODE == TMODE_SUMMARY) dsum += cur.dl;

      float ot[GL];                                // this lane's partial readout per step
#pragma unroll
      for (int jh = 0; jh < GL; jh += 4) {
        float4 bq[NS], cq[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          bq[i] = *reinterpret_cast<const float4*>(&sBC[buf][0][n0 + i][pt * GL + jh]);
          if (MODE == TMODE_FULL)
            cq[i] = *reinterpret_cast<const float4*>(&sBC[buf][1][n0 + i][pt * GL + jh]);
        }
        // the half tile's decays as one run of exps (exp2_run)
        float ea[4 * NS];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int i = 0; i < NS; ++i) ea[jj * NS + i] = ex[jh + jj].x * A2[i];
        exp2_run(ea);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = jh + jj;
          const float xuj = ex[j].y;
          float o = 0.0f;
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            const float bvj = jj == 0 ? bq[i].x : jj == 1 ? bq[i].y : jj == 2 ? bq[i].z : bq[i].w;
            const float dA = ea[jj * NS + i];
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
        const float o_own = reduce_scatter8_banked(ot, g);   // full readout of step t0 + p*8 + g
        const float yv = __builtin_fmaf(Dv, cur.uu, o_own) * cur.gate;
        // tail lanes (d >= D) store channel D-1's value to channel D-1's
        // address; steps past the chunk fall outside the buffer and are dropped
        buf_st<T>(yv, rs_y, voff_own, p * soff_step);
      }
      cur = nxt;
    }
    if (has_next) stage_store(buf ^ 1);
    __syncthreads();
  }

  if (MODE == TMODE_SUMMARY) {                     // the channel's sum over its 8 lanes
    dsum += dpp<0x128>(dsum);   // row_ror:8: the pair g, g ^ 4
    dsum += dpp<0x124>(dsum);   // row_ror:4: adds the other pair of the row half
    dsum += dpp<0xB1>(dsum);    // quad_perm [1,0,3,2]: g ^ 1
  }
  if (!active) return;
  if (MODE == TMODE_SUMMARY) {
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

// ------------------------------------------------------------------ wide
//
// The same computation for rows whose byte length is a multiple of 16 (and
// 16-byte aligned tensors): u / delta / z and y go through LDS, so that every
// global access of these streams is 16 bytes per lane.  A workgroup's rows are
// only 32 channels (64 or 128 bytes) wide, and one 16-bit element per lane per
// 8 steps, as fwd_tile loads them, reaches about half the bandwidth of 16-byte
// pieces on such strips.
//
// Per stage of TB steps (one 16-byte piece per thread and tensor):
//   start: issue the next stage's loads (u, delta, z, B, C) into registers;
//   tiles: lane g of a channel reads its own step's u / delta / z from LDS,
//          prepares it, and the 8 lanes run the tile as in fwd_tile; y goes
//          to an LDS row buffer;
//   end:   barrier; the registers go to LDS and y leaves in 16-byte pieces;
//          barrier.
template <typename T>
struct WideCfg {
  static constexpr int ES = sizeof(T);
  static constexpr int TB = 128 / ES;                  // steps per stage: 64 (16-bit), 32 (f32)
  static constexpr int ROWB = CPW * ES;                // bytes of one row of the block: 64 / 128
  static constexpr int LPR = ROWB / 16;                // 16-byte pieces per row: 4 / 8
  static constexpr int RS = ROWB + (ES == 2 ? 16 : 32);  // padded LDS row stride (bytes)
  static constexpr int TSW = TB + 4;                   // staged B/C row stride (floats)
  static_assert(TB * LPR == kBlockT, "one piece per thread and tensor");
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ float lds_elem(const uint8_t* p) {
  if constexpr (sizeof(T) == 4) return *reinterpret_cast<const float*>(p);
  else return to_f32(T{*reinterpret_cast<const uint16_t*>(p)});
}
template <typename T>
__device__ __forceinline__ void lds_put(uint8_t* p, float v) {
  if constexpr (sizeof(T) == 4) *reinterpret_cast<float*>(p) = v;
  else *reinterpret_cast<uint16_t*>(p) = from_f32<T>(v).bits;
}

template <typename T, int NS, int MODE, bool HAS_Z>
__global__ __launch_bounds__(kBlockT, (tile_waves_per_simd<NS, MODE>())) void fwd_wide(
    const T* __restrict__ u_in, const T* __restrict__ delta_in, const T* __restrict__ B_in,
    const T* __restrict__ C_in, const T* __restrict__ z_in, T* __restrict__ y_out,
    const FwdArgs a) {
  using W = WideCfg<T>;
  constexpr int ES = W::ES, TB = W::TB, RS = W::RS, TSW = W::TSW;
  constexpr int NP = NS * GL;                          // == N on this path
  constexpr bool OUT = MODE != TMODE_SUMMARY;          // readout and y
  constexpr bool SUMM = MODE == TMODE_SUMMARY || MODE == TMODE_LOCAL;  // chunk summaries
  constexpr bool CARRIED = MODE == TMODE_FULL || MODE == TMODE_FIXUP;  // starts from h_in
  constexpr bool FIX = MODE == TMODE_FIXUP;
  constexpr int NT = (OUT && HAS_Z) ? 3 : 2;           // streamed inputs: u, delta[, z]
  constexpr int NTILE = TB / GL;
  // B / C of a stage in 16-byte pieces: PPR per row, PB per tensor, NPC per thread
  constexpr int EPP = 16 / ES;
  constexpr int PPR = NP * ES / 16;
  constexpr int PB = TB * PPR;
  constexpr int NBC = OUT ? 2 : 1;
  constexpr int NPC = (NBC * PB + kBlockT - 1) / kBlockT;
  static_assert(PB % 64 == 0, "a wave's pieces come from one tensor");
  // u, delta[, z] rows of the stage; y of row t replaces delta of row t once
  // the lane that owns (t, channel) has prepared that step (it is delta's
  // only reader), so the stage's y leaves from sIn[1].
  __shared__ __attribute__((aligned(16))) uint8_t sIn[NT][TB * RS];
  __shared__ __attribute__((aligned(16))) float sBC[OUT ? 2 : 1][NP][TSW];
  __shared__ __attribute__((aligned(16))) float2 xch[2][CPW][XS];
  __shared__ int vote[2][kBlockT / 64];                // FIXUP: per-wave "all states agree"

  const int tid = threadIdx.x;
  const int g = wide_g(tid);
  const int cl = wide_channel(tid);
  const int64_t nbd = (a.D + CPW - 1) / CPW;
  int64_t blk = xcd_pair_remap(blockIdx.x, gridDim.x);
  const int64_t db = blk % nbd;
  blk /= nbd;
  // FIXUP skips chunk 0 when there is no h0 (its LOCAL pass was exact)
  const int64_t kf = (FIX && a.h0 == nullptr) ? 1 : 0;
  const int64_t Kg = MODE == TMODE_SUMMARY ? a.K - 1 : a.K - kf;
  const int64_t k = kf + blk % Kg;
  const int64_t b = blk / Kg;
  const int64_t d0 = db * CPW;
  const int64_t d_raw = d0 + cl;
  const bool active = d_raw < a.D;
  const int64_t d = active ? d_raw : a.D - 1;
  const int64_t D = a.D, N = a.N;
  const SeqRows sr = seq_rows(a.cu, b, a.L, a.Lt);
  const int64_t t0 = k * a.chunk_len;
  int64_t t1 = (t0 + a.chunk_len < sr.len) ? t0 + a.chunk_len : sr.len;
  if (t1 < t0) t1 = t0;                         // a chunk past a short sequence's end
  const int n0 = g * NS;

  float A2[NS], h[NS], hl[NS];   // hl: FIXUP's copy of the LOCAL pass's states
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int n = n0 + i;
    A2[i] = n < N ? ld_param(a.A, d * N + n, a.param_dtype) * kLog2e : 0.0f;
    h[i] = 0.0f;
    hl[i] = 0.0f;
    if (CARRIED && k > 0 && n < N) h[i] = a.chunk_state[((b * a.K + (k - 1)) * N + n) * D + d];
    else if (CARRIED && k == 0 && n < N && a.h0)
      h[i] = ld_param(a.h0, (b * D + d) * N + n, a.param_dtype);
  }
  const float Dv = a.Dskip ? ld_param(a.Dskip, d, a.param_dtype) : 0.0f;
  const float bv = a.bias ? ld_param(a.bias, d, a.param_dtype) : 0.0f;
  const bool sp = a.softplus != 0;

  const int64_t nsteps = t1 - t0;
  const int64_t row0 = (sr.start + t0) * D;
  const int64_t rbytes = nsteps * D * ES;
  __amdgpu_buffer_rsrc_t rs_in[NT];
  rs_in[0] = make_rsrc(u_in + row0, rbytes);
  rs_in[1] = make_rsrc(delta_in + row0, rbytes);
  if constexpr (NT == 3) rs_in[2] = make_rsrc(z_in + row0, rbytes);
  const auto rs_y = make_rsrc(y_out + row0, OUT ? rbytes : 0);
  const auto rs_B = make_rsrc(B_in + (sr.start + t0) * a.ldb, rows_bytes(nsteps, a.ldb, N, ES));
  const auto rs_C = make_rsrc(C_in + (sr.start + t0) * a.ldc, rows_bytes(nsteps, a.ldc, N, ES));

  // this thread's 16-byte piece of every stage: row pr, piece pq of the block's row
  const int pr = tid / W::LPR, pq = tid % W::LPR;
  const int voff_piece = (int)(((int64_t)pr * D + d0) * ES) + pq * 16;
  const int soff_stage = (int)((int64_t)TB * D * ES);
  const int lds_piece = pr * RS + pq * 16;
  const int lds_own_col = cl * ES;                    // column of this lane's channel

  u32x4 rin[NT], rbc[NPC];
  auto issue_loads = [&](int st) {
#pragma unroll
    for (int q = 0; q < NT; ++q)
      rin[q] = __builtin_amdgcn_raw_buffer_load_b128(rs_in[q], voff_piece, st * soff_stage, 0);
#pragma unroll
    for (int r = 0; r < NPC; ++r) {
      const int pi = tid + r * kBlockT;
      const int q = pi % PB;                          // rows past the chunk read 0
      // PB is a multiple of 64, so B or C is a per-wave choice
      const bool isB = __builtin_amdgcn_readfirstlane(pi / PB) == 0;
      const int ld = isB ? (int)a.ldb : (int)a.ldc;
      const int off = ((st * TB + q / PPR) * ld + (q % PPR) * EPP) * ES;
      rbc[r] = __builtin_amdgcn_raw_buffer_load_b128(isB ? rs_B : rs_C, off, 0, 0);
    }
  };
  auto commit_loads = [&]() {
#pragma unroll
    for (int q = 0; q < NT; ++q) *reinterpret_cast<u32x4*>(&sIn[q][lds_piece]) = rin[q];
#pragma unroll
    for (int r = 0; r < NPC; ++r) {
      const int pi = tid + r * kBlockT;
      if (pi < NBC * PB) {
        const int w = pi / PB, q = pi % PB;
        const int tt = q / PPR, n = (q % PPR) * EPP;
        const uint32_t v[4] = {rbc[r].x, rbc[r].y, rbc[r].z, rbc[r].w};
#pragma unroll
        for (int e = 0; e < EPP; ++e) {
          float f;
          if constexpr (ES == 4) f = __builtin_bit_cast(float, v[e]);
          else f = to_f32(T{(uint16_t)(e & 1 ? v[e / 2] >> 16 : v[e / 2] & 0xffffu)});
          sBC[w][n + e][tt] = f;
        }
      }
    }
  };
  // y of the stage just finished leaves in 16-byte pieces; the last channel
  // block of a row, where the block runs past D, stores element by element.
  const bool full_row = d0 + CPW <= D;
  // Full rows: each thread drains exactly the 16-byte piece it commits next,
  // so drain and commit need no barrier between them.
  auto drain_y = [&](int st) {
    if (full_row) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&sIn[1][lds_piece]);
      __builtin_amdgcn_raw_buffer_store_b128(v, rs_y, voff_piece, st * soff_stage, 0);
    } else {
      const int rowb = (int)(D * ES), colb = (int)(d0 * ES);
      for (int e = tid; e < TB * CPW; e += kBlockT) {
        const int r = e / CPW, c = e % CPW;
        if (d0 + c < D) {
          const float v = lds_elem<T>(&sIn[1][r * RS + c * ES]);
          buf_st<T>(v, rs_y, r * rowb + colb + c * ES, st * soff_stage);
        }
      }
    }
  };

  issue_loads(0);
  commit_loads();
  __syncthreads();

  // Per-step inputs of this lane's own step (stage row `row`): dt, dt*u
  // (handed to the channel's 8 lanes through xch), u and the gate (kept for
  // the output).  Rows past the chunk (masked stages only) get dt = dt*u = 0.
  struct Prep { float dl, xu, uu, gate; };
  auto prep = [&](int row, bool valid) {
    const uint8_t* own = &sIn[0][row * RS + lds_own_col];
    const float uu = lds_elem<T>(own);
    const float x = lds_elem<T>(own + TB * RS) + bv;
    float spx = softplus(x);
    __asm__ volatile("" : "+v"(spx));
    const float dl0 = sp ? spx : x;
    Prep r;
    r.dl = valid ? dl0 : 0.0f;
    r.xu = valid ? dl0 * uu : 0.0f;
    r.uu = uu;
    r.gate = 1.0f;
    if constexpr (OUT && HAS_Z) {
      const float zz = lds_elem<T>(own + 2 * TB * RS);
      r.gate = zz * sigmoid(zz);
    }
    return r;
  };

  float dsum = 0.0f;
  const int nstage = (int)((nsteps + TB - 1) / TB);
  // One stage of tiles.  The lane's step of tile pt+1 is prepared while tile
  // pt runs (xch double buffered: one wave's LDS operations complete in
  // program order), so the exchange's LDS round trip overlaps the updates.
  // MASKED: the chunk ends inside this stage; otherwise no step is checked.
  // In a single pass over a grid of 5 waves per SIMD (busy: FULL, NS <= 2, a
  // full grid), a wave raises its issue priority for the stage's last two
  // tiles and the two barriers after them, and drops it after the stage, so
  // that waves nearing a barrier, which hold up their workgroup, go first:
  // 2.8B forward 325.9 -> 320.5 and 329.0 -> 323.0 us in A/B runs.  Left off
  // elsewhere, where it measured neutral or worse: the chunked passes (long
  // sequence -0.2 to -2.2%, 2x2048x2048 f32 +1.3%), the 130M forward (under
  // one wave per SIMD, +1 us), N = 64 (NS = 8, 2 waves per SIMD: 379 -> 614 us).
  const bool busy = MODE == TMODE_FULL && NS <= 2 && gridDim.x >= 1024;
  auto run_stage = [&](int st, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int left = (int)nsteps - st * TB;          // steps of the chunk from this stage on
    Prep cur = prep(g, !MASKED || g < left);
    xch[0][cl][g] = make_float2(cur.dl, cur.xu);
    constexpr int kUnroll = OUT ? NTILE : 1;
#pragma unroll kUnroll
    for (int pt = 0; pt < NTILE; ++pt) {
      if (MASKED && pt * GL >= left) break;          // tiles past the chunk (uniform)
      if (busy && pt == NTILE - 2) __builtin_amdgcn_s_setprio(2);   // see run_stage's comment
      float2 ex[GL];
#pragma unroll
      for (int j = 0; j < GL; j += 2) {
        const float4 v = *reinterpret_cast<const float4*>(&xch[pt & 1][cl][j]);
        ex[j] = make_float2(v.x, v.y);
        ex[j + 1] = make_float2(v.z, v.w);
      }
      Prep nxt = cur;
      if (pt + 1 < NTILE) {
        const int row = (pt + 1) * GL + g;
        nxt = prep(row, !MASKED || row < left);
        xch[(pt + 1) & 1][cl][g] = make_float2(nxt.dl, nxt.xu);
      }
      if (SUMM) dsum += cur.dl;
      float ot[GL];
#pragma unroll
      for (int jh = 0; jh < GL; jh += 4) {
        float4 bq[NS], cq[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          bq[i] = *reinterpret_cast<const float4*>(&sBC[0][n0 + i][pt * GL + jh]);
          if (OUT) cq[i] = *reinterpret_cast<const float4*>(&sBC[OUT ? 1 : 0][n0 + i][pt * GL + jh]);
        }
        // the half tile's decays as one run of exps (exp2_run)
        float ea[4 * NS];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int i = 0; i < NS; ++i) ea[jj * NS + i] = ex[jh + jj].x * A2[i];
        exp2_run(ea);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = jh + jj;
          const float xuj = ex[j].y;
          float o = 0.0f;
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            const float bvj = jj == 0 ? bq[i].x : jj == 1 ? bq[i].y : jj == 2 ? bq[i].z : bq[i].w;
            const float dA = ea[jj * NS + i];
            const float xb = xuj * bvj;
            h[i] = __builtin_fmaf(dA, h[i], xb);
            if (FIX) hl[i] = __builtin_fmaf(dA, hl[i], xb);   // the LOCAL pass's operations
            if (OUT) {
              const float cvj = jj == 0 ? cq[i].x : jj == 1 ? cq[i].y : jj == 2 ? cq[i].z : cq[i].w;
              o = __builtin_fmaf(cvj, h[i], o);
            }
          }
          ot[j] = o;
        }
      }
      if constexpr (OUT) {
        const float o_own = reduce_scatter8_banked(ot, g);   // full readout of this lane's step
        lds_put<T>(&sIn[1][(pt * GL + g) * RS + lds_own_col],
                   __builtin_fmaf(Dv, cur.uu, o_own) * cur.gate);
      }
      cur = nxt;
    }
  };
  bool stopped = false;   // FIXUP: left before the chunk's end (states had converged)
  for (int st = 0; st < nstage; ++st) {
    const bool has_next = st + 1 < nstage;
    if (has_next) issue_loads(st + 1);
    if ((st + 1) * TB <= (int)nsteps) run_stage(st, std::false_type{});
    else run_stage(st, std::true_type{});
    if constexpr (FIX) {
      // bitwise equality of every state of the workgroup with the LOCAL
      // pass's: from here on both passes compute the same values, and the
      // LOCAL pass's y of the rest of the chunk is already in place
      bool same = true;
#pragma unroll
      for (int i = 0; i < NS; ++i)
        same = same && __builtin_bit_cast(uint32_t, h[i]) == __builtin_bit_cast(uint32_t, hl[i]);
      const bool wave_same = __builtin_amdgcn_ballot_w64(!same) == 0;
      if ((tid & 63) == 0) vote[st & 1][tid >> 6] = wave_same ? 1 : 0;
    }
    __syncthreads();
    if constexpr (FIX) {
      int all = 1;
#pragma unroll
      for (int w = 0; w < kBlockT / 64; ++w) all &= vote[st & 1][w];
      stopped = all != 0 && has_next;                 // (vote[st & 1] is rewritten two stages on)
    }
    if (OUT) {
      drain_y(st);                                  // steps past the chunk are dropped
      if (!full_row && has_next) __syncthreads();   // element-wise drain reads others' pieces
    }
    if (stopped) break;                             // uniform over the workgroup
    if (has_next) commit_loads();
    __syncthreads();
    if (busy) __builtin_amdgcn_s_setprio(0);
  }

  if (SUMM) {                                       // the channel's sum over its 8 lanes
    dsum += dpp<0x128>(dsum);   // row_ror:8: the pair g, g ^ 4
    dsum += dpp<0x124>(dsum);   // row_ror:4: adds the other pair of the row half
    dsum += dpp<0xB1>(dsum);    // quad_perm [1,0,3,2]: g ^ 1
  }
  if (!active) return;
  if (SUMM) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (n0 + i < N) a.chunk_state[((b * a.K + k) * N + n0 + i) * D + d] = h[i];
    if (g == 0) a.chunk_dsum[(b * a.K + k) * D + d] = dsum;
  }
  // last_state: FULL, and LOCAL from its zero start (exact for chunk 0 without
  // h0, and what FIXUP converges to when it stops early); FIXUP rewrites it
  // when it ran to the chunk's end
  if (MODE != TMODE_SUMMARY && !stopped && a.last_state != nullptr &&
      k == last_chunk(sr.len, a.chunk_len)) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (n0 + i < N) st_param(a.last_state, (b * D + d) * N + n0 + i, a.param_dtype, h[i]);
  }
}

hipError_t launch_fwd_carry(const FwdArgs& a, hipStream_t s);  // ss_fwd.hip

// fwd_wide takes rows of a multiple of 16 bytes, N = 8 * NS (B / C rows of 16,
// 32 or 64 bytes) and 16-byte aligned streams.
static bool wide_ok(const FwdArgs& a, int es, int ns) {
  auto al = [](const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  return (a.D * es) % 16 == 0 && a.N == 8 * ns && al(a.u) && al(a.delta) && al(a.z) &&
         al(a.y) && al(a.B) && al(a.C) && (a.ldb * es) % 16 == 0 && (a.ldc * es) % 16 == 0;
}

template <typename T, int NS, bool HAS_Z>
static hipError_t launch_tile_t(const FwdArgs& a, hipStream_t s) {
  const T* U = static_cast<const T*>(a.u);
  const T* DL = static_cast<const T*>(a.delta);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  const T* Z = static_cast<const T*>(a.z);
  T* Y = static_cast<T*>(a.y);
  const int64_t nbd = (a.D + CPW - 1) / CPW;
  const bool wide = wide_ok(a, (int)sizeof(T), NS);
  hipError_t e;
  if (wide && a.K > 1) {
    // Chunked, fwd_wide: LOCAL runs every chunk from h = 0 (chunk 0 from 0
    // too), writing y, the chunk end states and dt sums; the carry turns the
    // summaries into each chunk's true starting state; FIXUP reruns each
    // chunk from that state next to a copy of the LOCAL recurrence and stops
    // at the first stage end where the two agree bit for bit in every state
    // of the workgroup: the rest of the chunk's y is then exactly what FIXUP
    // would write.  Where the states forget their start quickly, FIXUP
    // covers a few stages per chunk instead of the whole sequence again.
    fwd_wide<T, NS, TMODE_LOCAL, HAS_Z><<<dim3((unsigned)(a.Bn * a.K * nbd)), dim3(kBlockT), 0,
                                         s>>>(U, DL, Bm, Cm, Z, Y, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_fwd_carry(a, s)) != hipSuccess) return e;
    const int64_t kf = a.h0 ? 0 : 1;
    fwd_wide<T, NS, TMODE_FIXUP, HAS_Z><<<dim3((unsigned)(a.Bn * (a.K - kf) * nbd)),
                                         dim3(kBlockT), 0, s>>>(U, DL, Bm, Cm, Z, Y, a);
    return hipGetLastError();
  }
  if (a.K > 1) {
    // Chunked, fwd_tile: summaries from h = 0, the carry, then every chunk
    // again from its carried-in state.
    fwd_tile<T, NS, TMODE_SUMMARY, false><<<dim3((unsigned)(a.Bn * (a.K - 1) * nbd)),
                                           dim3(kBlockT), 0, s>>>(U, DL, Bm, Cm, Z, Y, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_fwd_carry(a, s)) != hipSuccess) return e;
  }
  const dim3 gf((unsigned)(a.Bn * a.K * nbd));
  if (wide)
    fwd_wide<T, NS, TMODE_FULL, HAS_Z><<<gf, dim3(kBlockT), 0, s>>>(U, DL, Bm, Cm, Z, Y, a);
  else
    fwd_tile<T, NS, TMODE_FULL, HAS_Z><<<gf, dim3(kBlockT), 0, s>>>(U, DL, Bm, Cm, Z, Y, a);
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
    case 8: return launch_tile_ns<T, 8>(a, s);
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
