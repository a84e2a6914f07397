// Schedule and workspace layout of one call (host side, pure arithmetic).
//
// The schedule is a function of the descriptor only (never of the device),
// so results do not depend on how many compute units a device exposes.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/ss.h"

namespace ss {

// Backward register tile: time steps one lane holds per chunk (general path,
// N > 16).  8 steps keep the main kernel at 208 VGPRs (2 waves per SIMD);
// 16 steps took 336 (1 wave): 2x2048x2048 backward, N = 32 982 -> 894 us,
// N = 64 1794 -> 1584 us (twice the chunk records, but twice the waves).
constexpr int kBwdTile = 8;
// Backward chunk length of the tile path: 8 tiles of 8 steps (N <= 16), 4
// tiles with 4 states per lane (N <= 32: the tile-start states and dB/dC rows
// take twice the LDS per step).
constexpr int kBwdTileChunk = 64;
constexpr int kBwdTileChunk4 = 32;
// Chunks of one channel block handled by one backward workgroup (their dA /
// dD / ddelta_bias partials are summed in registers / in place).
constexpr int kBwdChunksPerGroup = 4;
// Channels per workgroup.
constexpr int kChannelsPerBlock = 256;
// Tile kernels: steps that the own-step loads may run past a chunk (the last
// 64-step stage is run whole and loads are prefetched three 8-step tiles
// ahead); those byte offsets must also stay below 2^31.
constexpr int64_t GL_MAX_TILE = 128;

struct Plan {
  int NS = 4, G = 1;          // forward: states per lane, lanes per channel
  int64_t chunk_len = 0, K = 1;
  int n_launches = 0;
  // workspace (bytes, 256-aligned offsets)
  size_t off_dsum = 0, off_state = 0, off_bstate = 0, off_part_bc = 0, off_part_dA = 0,
         off_part_dD = 0, off_part_db = 0;
  size_t off_bpad = 0, off_cpad = 0;   // forward, N > 64 short of NS * G: padded B / C rows
  bool pad_rows = false;
  size_t ws_bytes = 0;
  int64_t KG = 0, nwgd = 0;   // backward: chunk groups, channel blocks
  bool bwd_tile = false;      // backward: 8-lanes-per-channel tile kernels (N <= 32)
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Forward mapping by state count: N <= 64 uses 8 lanes per channel with NS
// states each (the tile kernels; NS = 8 runs 2 waves per SIMD); larger N the
// general scan with 16 states per lane, G = 8 (N <= 128) or 16 lanes per
// channel.
inline void pick_bucket(int64_t N, int* NS, int* G) {
  if (N <= 8) { *NS = 1; *G = 8; }
  else if (N <= 16) { *NS = 2; *G = 8; }
  else if (N <= 32) { *NS = 4; *G = 8; }
  else if (N <= 64) { *NS = 8; *G = 8; }
  else if (N <= 128) { *NS = 16; *G = 8; }
  else { *NS = 16; *G = 16; }
}

// Forward sequences of at most this many steps (decode steps) with N <= 32
// run the short-sequence kernel: 4 lanes per channel, NS = N/4 (rounded up
// to 1, 2, 4 or 8) states each, no staging (the tile kernel's 64-step stages
// would be mostly empty).
constexpr int64_t kShortSeq = 16;

inline Plan make_plan(const ss_desc& d, bool backward) {
  Plan p;
  const int64_t Bn = d.batch, L = d.seqlen, D = d.dim, N = d.dstate;
  pick_bucket(N, &p.NS, &p.G);
  const bool short_seq = !backward && L <= kShortSeq && N <= 32;
  if (short_seq) {
    p.NS = N <= 4 ? 1 : N <= 8 ? 2 : N <= 16 ? 4 : 8;
    p.G = 4;
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
      // Waves that one chunk index provides.  Chunking adds two launches and,
      // where states forget their start slowly, a second sweep over the data
      // (the fix-up pass of the 16-byte-row kernel runs until the carried-in
      // states have decayed into the zero-start ones, and the general kernels
      // always sweep twice), so it pays only when the grid leaves most SIMDs
      // (1024) idle: below 640 waves the time axis is cut into chunks until
      // the grid reaches about 8 waves per SIMD, with chunks of at least 128
      // steps (a sequence of fewer than 256 steps does not earn the extra
      // launches back: 1x128x32x16 takes 17.8 us in 3 launches).
      // Measured (cold medians): 4x1024x1536x16 (768 waves, dt down to 1e-3:
      // slow decay) 67.8 us in one pass, 75.9 / 79.4 / 92.5 us with chunks of
      // 128 / 256 / 512 steps; 1x262144x512x16 (64 waves) 559 / 530 / 539 /
      // 636 us with chunks of 1024 / 2048 / 4096 / 8192 steps.
      const int64_t cpw = 64 / p.G;
      const int64_t waves = Bn * ((D + cpw - 1) / cpw);
      const int64_t target = 8192;
      int64_t K = 1;
      if (waves < 640) {
        K = (target + waves - 1) / waves;
        const int64_t kmax = L / 128;
        if (K > kmax) K = kmax;
        if (K < 1) K = 1;
      }
      lc = (L + K - 1) / K;
      lc = (lc + 3) & ~int64_t(3);
    }
    // a chunk's rows of one [B, L, D] tensor must fit a 32-bit buffer range
    const int64_t lc_cap = (int64_t)0x7fffffff / ((D > 0 ? D : 1) * 4) - GL_MAX_TILE;
    if (lc > lc_cap) lc = lc_cap > 8 ? lc_cap & ~int64_t(7) : 8;
    if (short_seq) lc = L;   // one kernel over the whole sequence (64-bit addressing)
    p.chunk_len = lc;
    p.K = (L + lc - 1) / lc;
    size_t off = 0;
    if (p.K > 1) {
      p.off_dsum = off;
      off = align256(off + sizeof(float) * (size_t)(Bn * p.K * D));
      p.off_state = off;
      off = align256(off + sizeof(float) * (size_t)(Bn * p.K * N * D));
    }
    // The general scan reads whole B / C rows of NS * G elements as vectors;
    // a shorter N gets them copied into such rows first (zero past N): with
    // element loads instead, N = 100 ran 2.6x slower per update than N = 128.
    const int64_t npad = (int64_t)p.NS * p.G;
    if (!short_seq && N > 64 && N != npad) {
      const size_t es = d.io_dtype == 0 ? 4 : 2;
      p.pad_rows = true;
      p.off_bpad = off;
      off = align256(off + es * (size_t)(Bn * L * npad));
      p.off_cpad = off;
      off = align256(off + es * (size_t)(Bn * L * npad));
    }
    p.ws_bytes = off;
    p.n_launches = (p.K > 1 ? (N > 0 ? 3 : 2) : 1) + (p.pad_rows ? 1 : 0);
    return p;
  }
  // backward.  N <= 32: tile kernels, chunks of up to 64 steps (32 above
  // N = 16), 32 channels per workgroup, per-chunk partials.  Otherwise the
  // general kernels: chunks of up to kBwdTile steps (one register tile), 256
  // channels per workgroup, partials per group of 4 chunks.
  p.bwd_tile = N <= 32;
  int64_t lc = !p.bwd_tile ? kBwdTile : N <= 16 ? kBwdTileChunk : kBwdTileChunk4;
  if (d.chunk_len > 0 && d.chunk_len < lc) lc = d.chunk_len;
  if (lc > L) lc = L;
  const int64_t lc_cap = (int64_t)0x7fffffff / ((D > 0 ? D : 1) * 4) - GL_MAX_TILE;
  if (lc > lc_cap) lc = lc_cap > 1 ? lc_cap : 1;
  p.chunk_len = lc;
  p.K = (L + lc - 1) / lc;
  if (p.bwd_tile) {
    p.NS = N <= 8 ? 1 : N <= 16 ? 2 : 4;
    p.G = 8;
    p.KG = p.K;
    p.nwgd = (D + 31) / 32;
  } else {
    p.NS = 1;
    p.G = 1;
    p.KG = (p.K + kBwdChunksPerGroup - 1) / kBwdChunksPerGroup;
    p.nwgd = (D + kChannelsPerBlock - 1) / kChannelsPerBlock;
  }
  size_t off = 0;
  p.off_dsum = off;
  off = align256(off + sizeof(float) * (size_t)(Bn * p.K * D));
  p.off_state = off;
  off = align256(off + sizeof(float) * (size_t)(Bn * p.K * N * D));
  p.off_bstate = off;
  off = align256(off + sizeof(float) * (size_t)(Bn * p.K * N * D));
  p.off_part_bc = off;
  off = align256(off + sizeof(float) * (size_t)(Bn * L * p.nwgd * 2 * N));
  p.off_part_dA = off;
  off = align256(off + sizeof(float) * (size_t)(Bn * p.KG * N * D));
  p.off_part_dD = off;
  off = align256(off + sizeof(float) * (size_t)(Bn * p.KG * D));
  p.off_part_db = off;
  off = align256(off + sizeof(float) * (size_t)(Bn * p.KG * D));
  p.ws_bytes = off;
  p.n_launches = p.K > 1 ? 4 : 2;
  return p;
}

}  // namespace ss
