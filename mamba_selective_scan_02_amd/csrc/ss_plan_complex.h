// Schedule and workspace layout of the complex calls (host side, pure
// arithmetic), beside the real calls' in ss_plan.h.
#pragma once

#include "ss_plan.h"

namespace ss {

// Complex variant (A, B, C and the state complex, stored as (re, im) float
// pairs).  Forward: G lanes per channel with NS complex states each
// (NS * G >= N, NS <= 4 up to N = 64), 256 / G channels per workgroup; for
// 8 < N <= 16 one lane per (channel, state) (G = 16, NS = 1); chunks chosen as
// for the real scan.  Backward, N <= 16: one lane per (channel, state), 16
// channels per workgroup, chunks of at most kCplxBwdLanesTile steps.  N > 16:
// one lane per channel looping over the states, chunks of at most
// kCplxBwdTile steps, 256 channels per workgroup.  Both write partials per
// group of kBwdChunksPerGroup chunks.  A chunk's decay is carried as the
// product of its steps' decays, stored beside its end state (4 floats per
// (b, k, n, d)): the closed form exp(A * sum dt) would turn the rounding of
// the sum into a phase error of |Im A| times it.
constexpr int kCplxBwdTile = 8;
constexpr int kCplxBwdLanesTile = 16;
constexpr int kCplxLanesCPW = 16;      // channels per workgroup of the lane-per-state kernels

inline Plan make_plan_complex(const ss_desc& d, bool backward) {
  Plan p;
  const int64_t Bn = d.batch, L = d.seqlen, D = d.dim, N = d.dstate;
  // At most 4 states per lane up to N = 64: the complex step is long (exp
  // and sin / cos from their series per state), so more lanes per channel buy
  // the waves that hide its latency at little cost in the readout sum.
  if (N <= 4) {
    p.G = 1;
    p.NS = N <= 1 ? 1 : N <= 2 ? 2 : 4;
  } else if (N <= 8) {
    p.NS = 4;
    p.G = 2;
  } else if (N <= 16) {
    p.NS = 1;           // one lane per (channel, state), 16 channels per workgroup
    p.G = 16;
  } else if (N <= 64) {
    p.NS = 4;
    p.G = N <= 32 ? 8 : 16;
  } else {
    p.G = 16;
    p.NS = N <= 128 ? 8 : 16;
  }
  if (Bn * L * D == 0) {
    p.chunk_len = L;
    p.K = 1;
    p.n_launches = 0;
    return p;
  }
  if (!backward) {
    int64_t lc;
    if (d.chunk_len > 0) {
      lc = d.chunk_len < L ? d.chunk_len : L;
    } else {
      const int64_t waves = Bn * ((D * p.G + 63) / 64);
      int64_t K = 1;
      if (waves < 3072) {
        K = (4096 + waves - 1) / waves;
        const int64_t kmax = (L + 63) / 64;
        if (K > kmax) K = kmax;
        if (K < 1) K = 1;
      }
      lc = (L + K - 1) / K;
      lc = (lc + 3) & ~int64_t(3);
    }
    p.chunk_len = lc;
    p.K = (L + lc - 1) / lc;
    size_t off = 0;
    if (p.K > 1) {
      p.off_state = off;   // (S re, S im, P re, P im) per (b, k, n, d)
      off = align256(off + 4 * sizeof(float) * (size_t)(Bn * p.K * N * D));
    }
    p.ws_bytes = off;
    p.n_launches = p.K > 1 ? (N > 0 ? 3 : 2) : 1;
    return p;
  }
  const bool lanes = N <= 16;
  int64_t lc = lanes ? kCplxBwdLanesTile : kCplxBwdTile;
  if (d.chunk_len > 0 && d.chunk_len < lc) lc = d.chunk_len;
  if (lc > L) lc = L;
  p.chunk_len = lc;
  p.K = (L + lc - 1) / lc;
  p.NS = 1;
  p.G = lanes ? 16 : 1;
  p.KG = (p.K + kBwdChunksPerGroup - 1) / kBwdChunksPerGroup;
  const int64_t cpw = lanes ? kCplxLanesCPW : kChannelsPerBlock;
  p.nwgd = (D + cpw - 1) / cpw;
  size_t off = 0;
  p.off_state = off;   // (S re, S im, E re, E im), E = product of conj(a)
  off = align256(off + 4 * sizeof(float) * (size_t)(Bn * p.K * N * D));
  p.off_bstate = off;
  off = align256(off + 2 * sizeof(float) * (size_t)(Bn * p.K * N * D));
  p.off_part_bc = off;
  off = align256(off + 4 * sizeof(float) * (size_t)(Bn * L * p.nwgd * N));
  p.off_part_dA = off;
  off = align256(off + 2 * sizeof(float) * (size_t)(Bn * p.KG * N * D));
  p.off_part_dD = off;
  off = align256(off + sizeof(float) * (size_t)(Bn * p.KG * D));
  p.off_part_db = off;
  off = align256(off + sizeof(float) * (size_t)(Bn * p.KG * D));
  p.ws_bytes = off;
  p.n_launches = p.K > 1 ? (N > 0 ? 5 : 4) : 3;
  return p;
}

}  // namespace ss
