// Host-side planning of the kernels' grids and scratch: split counts and
// persistent grid sizes.  Plain host C++, shared by the launchers, the
// workspace-size queries and the argument checks of the C ABI.
#include "launch.hpp"

namespace flare {

EncodePlan plan_encode(int B, int H, int M, int64_t N, int D, int is_f32, int max_splits) {
  (void)D;
  (void)is_f32;
  EncodePlan pl;
  const int64_t bh = (int64_t)B * H;
  // 32 latents per wave, up to 256 latents (8 waves) per workgroup; more
  // latents take further workgroups along grid.z.
  pl.waves = M <= 64 ? 2 : M <= 128 ? 4 : 8;
  pl.lat_blocks = (M + 255) / 256;
  // About 1024 workgroups in all (a few per compute unit, a few rounds), at
  // least two 128-token tiles per split when there are enough tokens.  The
  // matrix-core path gives split s the tiles s, s + S, ...; the fp32 path
  // takes S contiguous ranges of tokens_per_split tokens (the last ones may
  // be empty and merge with weight 0).
  const int64_t tiles = (N + kEncT - 1) / kEncT;
  int64_t S = (1024 + bh - 1) / bh;
  int64_t max_s = tiles / 2;
  if (max_s < 1) max_s = 1;
  if (S > max_s) S = max_s;
  if (max_splits > 0 && S > max_splits) S = max_splits;
  if (S < 1) S = 1;
  pl.S = (int)S;
  pl.tokens_per_split = (tiles + S - 1) / S * kEncT;
  return pl;
}

size_t decode_bf16_lds(int M, int D) {
  const int MC = (M + 31) / 32;
  return (size_t)MC * (D / 16) * 64 * 16 + (size_t)MC * 2 * 64 * 16 + (size_t)kDecWaves * kDecGroup * D * 2;
}

// A persistent grid: as many workgroups as fit on the 256 compute units at
// once (LDS and the 3-waves-per-SIMD register budget decide), spread evenly
// over the heads; each takes every G-th pass of its head.
int64_t plan_decode_bf16(int B, int H, int M, int64_t N, int D) {
  const int64_t lds = (int64_t)decode_bf16_lds(M, D);
  int64_t per_cu = (160 * 1024) / lds;
  if (per_cu > 12 / kDecWaves) per_cu = 12 / kDecWaves;
  if (per_cu < 1) per_cu = 1;
  const int64_t bh = (int64_t)B * H;
  const int64_t pass = (int64_t)kDecWaves * kDecGroup;
  const int64_t passes = (N + pass - 1) / pass;
  int64_t per_bh = (256 * per_cu + bh - 1) / bh;
  if (per_bh > passes) per_bh = passes;
  if (per_bh < 1) per_bh = 1;
  return per_bh;
}

// Token splits of the backward latent passes: about 768 workgroups of 256
// latents in all, at most one split per 64-token tile.  At M = 256 the
// decoder role runs one 8-wave workgroup per compute unit (three even
// rounds) and the encoder role two 4-wave workgroups per (split, head), three
// per compute unit (two even rounds); 1024 workgroups timed 2-3 % slower.
int plan_bwd_splits(int B, int H, int M, int64_t N) {
  const int64_t bh = (int64_t)B * H * ((M + 255) / 256);
  const int64_t tiles = (N + kLatBwdTile - 1) / kLatBwdTile;
  int64_t S = (768 + bh - 1) / bh;
  if (S > tiles) S = tiles;
  if (S < 1) S = 1;
  return (int)S;
}

}  // namespace flare
