// Pointwise projections Y_p = X W_p on gfx950 bf16 matrix cores
// ("FLARE++: Low-Rank Attention with Dynamic Attention Routing", section 3:
// K = X W_K and V = X W_V in "Full self-attention" / "FLARE: fixed-query
// latent routing", the extra eK, eV of equation 7, and the output
// projection).  At C <= 256 the reduction is short and the outputs outweigh
// the input, so the kernel is built around HBM traffic:
//   - a wave loads its 32 rows of X once into registers, already as the B
//     operand of Y^T = W^T X^T (lane (g, r): row r, inputs 8g..8g+7 of each
//     32-wide step), and keeps them for every output column of every
//     projection, so X is read from HBM once (32 rows keep it at 64
//     registers: two 8-wave workgroups per CU, one loading while the other
//     computes and stores);
//   - the weights are rearranged once per call into operand order, in
//     32-column blocks of 2 KB per k-step; the workgroup streams the blocks
//     into LDS with buffer loads straight to LDS (four stages, three blocks in
//     flight, one barrier per block) and all eight waves read them;
//   - inside a block the two 16-column tiles are interleaved (tile t covers
//     columns 8(m/4) + 4t + m%4 of its rows m), so each lane ends with eight
//     consecutive output columns of one row and writes them as one 16-byte
//     store.
#include "common.hpp"
#include "launch.hpp"

namespace flare {

typedef __attribute__((address_space(3))) void lds_void_t;

// For 32-column block pb, k-step ks and tile t: the A operand of 16 output
// columns as 64 lanes x 8 bf16,
//   wsw[((pb KS + ks) 2 + t) 512 + 8 lane + j]
//     = W[32 ks + 8 (lane / 16) + j][32 pb + 8 (m / 4) + 4 t + m % 4],  m = lane % 16.
// One thread writes the 8 values of one (pb, ks, t, lane) as a 16-byte store;
// blockIdx.y picks the weight, so one launch serves every projection.
__global__ __launch_bounds__(256) void swizzle_weights_kernel(SwizzleParams p) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)p.Cin * p.Cout / 8) return;
  const bf16* __restrict__ w = reinterpret_cast<const bf16*>(p.w[blockIdx.y]);
  bf16x8* __restrict__ wsw = reinterpret_cast<bf16x8*>(p.wsw[blockIdx.y]);
  const int lane = (int)(g & 63);
  const int t = (int)((g >> 6) & 1);
  const int64_t rest = g >> 7;
  const int KS = p.Cin / 32;
  const int ks = (int)(rest % KS);
  const int pb = (int)(rest / KS);
  const int m = lane & 15;
  const int c0 = 32 * ks + 8 * (lane >> 4);
  const int col = 32 * pb + 8 * (m >> 2) + 4 * t + (m & 3);
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = w[(int64_t)(c0 + j) * p.Cout + col];
  wsw[g] = v;
}

constexpr int kGemmWaves = 8;

// RB 16-row tiles per wave (two, or one for small R so that the grid still
// covers the chip), eight waves per workgroup.  PAIR (row-major outputs with
// an even number of 32-column blocks): the results of an even block are held
// in registers until the next block is computed, and both are stored
// together, so each 128-byte line of an output row (64 columns) is written
// whole by one wave within a few instructions instead of in two halves a
// block apart.
template <int CIN, int RB, bool PAIR>
__global__ __launch_bounds__(64 * kGemmWaves, 4) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NW = kGemmWaves;
  constexpr int kGemmRowsPerWave = 16 * RB;
  constexpr int kGemmRowsPerBlock = kGemmRowsPerWave * NW;
  constexpr int KS = CIN / 32;
  constexpr int BLK = KS * 2 * 512;  // bf16 elements of one 32-column block
  constexpr int OPS = BLK / 512;     // 1 KB loads per block
  constexpr int OPW = (OPS + NW - 1) / NW;
  __shared__ __attribute__((aligned(16))) bf16 s0[BLK];
  __shared__ __attribute__((aligned(16))) bf16 s1[BLK];
  __shared__ __attribute__((aligned(16))) bf16 s2[BLK];
  __shared__ __attribute__((aligned(16))) bf16 s3[BLK];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wave
  const int64_t row0 = (int64_t)blockIdx.x * kGemmRowsPerBlock + wave * kGemmRowsPerWave;
  const bf16* xin = reinterpret_cast<const bf16*>(p.x);
  const int pairs = p.Cout / 32;
  const int nblk = p.n_proj * pairs;
  // Waves issue either OPW loads per block or none.
  const int my_ops = wave * OPW < OPS ? OPW : 0;

  // X rows as B operands, held for all output columns.
  bf16x8 xb[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t row = row0 + 16 * rb + r;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row < p.R) {
        xb[rb][ks] = *reinterpret_cast<const bf16x8*>(xin + row * CIN + 32 * ks + 8 * g);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xb[rb][ks][j] = (bf16)0.0f;
      }
    }
  }

  // Block b (projection b / pairs, column block b % pairs) into stage S.
  auto issue = [&](auto stage_tag, int b) {
    constexpr int S = decltype(stage_tag)::value;
    bf16* st = S == 0 ? s0 : S == 1 ? s1 : S == 2 ? s2 : s3;
    const int pr = b / pairs, pb = b - pr * pairs;
    const bf16* src = reinterpret_cast<const bf16*>(p.wt[pr]) + (int64_t)pb * BLK;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(src), (short)0, BLK * (int)sizeof(bf16), kBufferFlags);
#pragma unroll
    for (int q = 0; q < OPW; ++q) {
      const int op = wave * OPW + q;
      if (op < OPS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(st + op * 512), 16, lane * 16, op * 1024, 0, 0);
    }
  };

  // Element offset of (row row0 + 16 rb + r, column 0) in the output: row-major
  // [R, Cout], or head-major [B, H, N, D] with R = B N (head 0 of the row's
  // token; a column c adds (c / D) N D + c % D).
  int64_t row_off[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t row = min(row0 + 16 * rb + r, p.R - 1);
    if (p.head_major) {
      const int64_t bi = row / p.N, n = row - bi * p.N;
      row_off[rb] = (bi * (p.Cout / p.D) * p.N + n) * p.D;
    } else {
      row_off[rb] = row * p.Cout;
    }
  }

  // Store of one output row tile: lane (g, r) holds columns 8g .. 8g+7 of
  // block pb (tile 0 gives 8g..8g+3, tile 1 gives 8g+4..8g+7) for row
  // row0 + 16 rb + r.
  auto pack_row_tile = [&](const f32x4 (&acc)[2]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (bf16)acc[0][i];
      v[4 + i] = (bf16)acc[1][i];
    }
    return v;
  };
  auto store_packed = [&](bf16x8 v, int rb, int pr, int64_t col_off) {
    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(p.y[pr]) + row_off[rb] + col_off) = v;
  };
  bf16x8 carry[RB];  // PAIR: the packed results of the last even block

  const bool full_rows = row0 + kGemmRowsPerWave <= p.R;  // uniform in the wave
  auto compute_block = [&](auto stage_tag, int b) {
    constexpr int S = decltype(stage_tag)::value;
    const bf16* st = S == 0 ? s0 : S == 1 ? s1 : S == 2 ? s2 : s3;
    f32x4 acc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + ((ks * 2 + t) * 64 + lane) * 8);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb][t] = mfma_16x16x32(a, xb[rb][ks], acc[rb][t]);
      }
    const int pr = b / pairs, pb = b - pr * pairs;
    const int col = 32 * pb + 8 * g;
    int64_t col_off = col;
    if (p.head_major) {
      const int hd = col / p.D;
      col_off = (int64_t)hd * p.N * p.D + (col - hd * p.D);
    }
    if constexpr (PAIR) {
      if ((pb & 1) == 0) {  // uniform: kept for the next block
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) carry[rb] = pack_row_tile(acc[rb]);
        return;
      }
    }
    // full rows: exactly RB stores per block (2 RB for a pair), which the
    // step's wait counts
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (full_rows || row0 + 16 * rb + r < p.R) {
        if constexpr (PAIR) store_packed(carry[rb], rb, pr, col_off - 32);
        store_packed(pack_row_tile(acc[rb]), rb, pr, col_off);
      }
    }
  };

  // Block b lives in stage b % 4.  Step b: start the load of block b + 3,
  // compute and store block b, then wait until this wave's load of block
  // b + 1 has landed and meet at the barrier.  vmcnt counts loads and
  // stores in issue order, so the wait allows exactly the operations issued
  // after that load: the loads of blocks b + 2 and b + 3 and the stores
  // between them (RB per block; with PAIR, 2 RB at odd blocks and none at
  // even ones, so the stores of block b - 1 when b is even).
  auto step = [&](auto stage_tag, int b) {
    constexpr int S = decltype(stage_tag)::value;
    if (b + 3 < nblk) issue(std::integral_constant<int, (S + 3) % 4>(), b + 3);
    compute_block(stage_tag, b);
    const int later = ((b + 3 < nblk) + (b + 2 < nblk)) * (my_ops != 0);  // loads issued after block b + 1
    const int stores = PAIR ? (b > 0 ? 2 * RB : 0) : RB;  // stores issued after block b + 1's load
    if (!full_rows)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    else if (stores == 0) {
      if (later == 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * OPW));
      else if (later == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(OPW));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    } else if (stores == RB) {
      if (later == 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * OPW + RB));
      else if (later == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(OPW + RB));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(RB));
    } else {
      if (later == 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * OPW + 2 * RB));
      else if (later == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(OPW + 2 * RB));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * RB));
    }
    barrier_keep_loads();
  };

  issue(std::integral_constant<int, 0>(), 0);
  if (nblk > 1) issue(std::integral_constant<int, 1>(), 1);
  if (nblk > 2) issue(std::integral_constant<int, 2>(), 2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // X rows and the first blocks
  barrier_keep_loads();
  for (int b = 0; b < nblk; b += 4) {
    step(std::integral_constant<int, 0>(), b);
    if (b + 1 >= nblk) break;
    step(std::integral_constant<int, 1>(), b + 1);
    if (b + 2 >= nblk) break;
    step(std::integral_constant<int, 2>(), b + 2);
    if (b + 3 >= nblk) break;
    step(std::integral_constant<int, 3>(), b + 3);
  }
}

// Weight sets of at most kGemmPreloadBytes (all blocks of every projection,
// e.g. four 128 x 128 weights): every block is laid out in LDS once at the
// start, from the row-major weights, and the blocks are then computed with no
// further waits.  In the streamed kernel above, each block's wait for its
// weights also waits for the output stores issued before that load (one
// counter covers both), so with short blocks the store latency sets the pace.
// A thread takes 8 x 8 tiles of a weight (eight inputs of one k-step and
// lane group, eight consecutive output columns), transposes each in
// registers and writes it as eight 16-byte operand slots, in the order
// swizzle_weights_kernel gives the streamed kernel.
template <int CIN, bool PAIR>
__global__ __launch_bounds__(64 * kGemmWaves, 2) void gemm_bf16_preload_kernel(GemmParams p) {
  constexpr int NW = kGemmWaves;
  constexpr int KS = CIN / 32;
  constexpr int BLK = KS * 2 * 512;  // bf16 elements of one 32-column block
  extern __shared__ __attribute__((aligned(16))) bf16 wl[];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t row = (int64_t)blockIdx.x * 16 * NW + wave * 16 + r;
  const bf16* xin = reinterpret_cast<const bf16*>(p.x);
  const int pairs = p.Cout / 32;
  const int nblk = p.n_proj * pairs;

  // every block of every projection
  const int cchunks = p.Cout / 8;              // 8-column chunks of a weight row
  const int tiles = (CIN / 8) * cchunks;        // 8 x 8 tiles per weight
  for (int u = tid; u < p.n_proj * tiles; u += 64 * NW) {
    const int pr = u / tiles, t8 = u - pr * tiles;
    const int rg = t8 / cchunks, cc = t8 - rg * cchunks;  // rows 8 rg .. +7, columns 8 cc .. +7
    const bf16* src = reinterpret_cast<const bf16*>(p.w[pr]) + (int64_t)(8 * rg) * p.Cout + 8 * cc;
    bf16x8 rows[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rows[j] = *reinterpret_cast<const bf16x8*>(src + (int64_t)j * p.Cout);
    // column 8 cc + e sits in block (pr, cc / 4), k-step rg / 4, tile e / 4,
    // lane 16 (rg % 4) + 4 (cc % 4) + e % 4; row 8 rg + j is element j
    bf16* blk = wl + (int64_t)(pr * pairs + cc / 4) * BLK;
    const int ks = rg >> 2, lg = 16 * (rg & 3) + 4 * (cc & 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x8 col;
#pragma unroll
      for (int j = 0; j < 8; ++j) col[j] = rows[j][e];
      *reinterpret_cast<bf16x8*>(blk + ((ks * 2 + (e >> 2)) * 64 + lg + (e & 3)) * 8) = col;
    }
  }
  bf16x8 xb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (row < p.R) {
      xb[ks] = *reinterpret_cast<const bf16x8*>(xin + row * CIN + 32 * ks + 8 * g);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[ks][j] = (bf16)0.0f;
    }
  }
  int64_t row_off;
  {
    const int64_t rr = min(row, p.R - 1);
    if (p.head_major) {
      const int64_t bi = rr / p.N, n = rr - bi * p.N;
      row_off = (bi * (p.Cout / p.D) * p.N + n) * p.D;
    } else {
      row_off = rr * p.Cout;
    }
  }
  __syncthreads();  // the weight blocks are in LDS

  bf16x8 carry = {};
  for (int b = 0; b < nblk; ++b) {
    const bf16* st = wl + (int64_t)b * BLK;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + ((ks * 2 + t) * 64 + lane) * 8);
        acc[t] = mfma_16x16x32(a, xb[ks], acc[t]);
      }
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (bf16)acc[0][i];
      v[4 + i] = (bf16)acc[1][i];
    }
    const int pr = b / pairs, pb = b - pr * pairs;
    const int col = 32 * pb + 8 * g;
    int64_t col_off = col;
    if (p.head_major) {
      const int hd = col / p.D;
      col_off = (int64_t)hd * p.N * p.D + (col - hd * p.D);
    }
    bf16* yp = reinterpret_cast<bf16*>(p.y[pr]) + row_off + col_off;
    if constexpr (PAIR) {
      if ((pb & 1) == 0) {
        carry = v;
        continue;
      }
      if (row < p.R) *reinterpret_cast<bf16x8*>(yp - 32) = carry;
    }
    if (row < p.R) *reinterpret_cast<bf16x8*>(yp) = v;
  }
}

hipError_t launch_swizzle_weights(const SwizzleParams& p, int n, hipStream_t st) {
  const int64_t groups = (int64_t)p.Cin * p.Cout / 8;
  hipLaunchKernelGGL(swizzle_weights_kernel, dim3((unsigned)((groups + 255) / 256), (unsigned)n), dim3(256), 0,
                     st, p);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t st) {
  // two row tiles per wave once that still gives 512 workgroups (two per CU)
  const int rb = (p.R + 16 * 2 * kGemmWaves - 1) / (16 * 2 * kGemmWaves) >= 512 ? 2 : 1;
  const int64_t rows_per_block = 16 * rb * kGemmWaves;
  dim3 grid((unsigned)((p.R + rows_per_block - 1) / rows_per_block));
  dim3 block(64 * kGemmWaves);
  // whole 128-byte output lines per wave for row-major outputs of an even
  // number of 32-column blocks
  const bool pair = !p.head_major && (p.Cout / 32) % 2 == 0;
  const size_t wbytes = (size_t)p.n_proj * p.Cin * p.Cout * sizeof(bf16);
  if (gemm_preloads(p.R, p.n_proj, p.Cin, p.Cout)) {
    dim3 pgrid((unsigned)((p.R + 16 * kGemmWaves - 1) / (16 * kGemmWaves)));
#define FLARE_GEMM_PRE(C)                                                                                  \
  {                                                                                                        \
    hipError_t e;                                                                                          \
    if (pair) {                                                                                            \
      if ((e = hipFuncSetAttribute((const void*)gemm_bf16_preload_kernel<C, true>,                         \
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)wbytes)) != hipSuccess) \
        return e;                                                                                          \
      hipLaunchKernelGGL((gemm_bf16_preload_kernel<C, true>), pgrid, block, wbytes, st, p);                \
    } else {                                                                                               \
      if ((e = hipFuncSetAttribute((const void*)gemm_bf16_preload_kernel<C, false>,                        \
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)wbytes)) != hipSuccess) \
        return e;                                                                                          \
      hipLaunchKernelGGL((gemm_bf16_preload_kernel<C, false>), pgrid, block, wbytes, st, p);               \
    }                                                                                                      \
  }
    switch (p.Cin) {
      case 32: FLARE_GEMM_PRE(32); break;
      case 64: FLARE_GEMM_PRE(64); break;
      case 128: FLARE_GEMM_PRE(128); break;
      case 256: FLARE_GEMM_PRE(256); break;
      default: return hipErrorInvalidValue;
    }
#undef FLARE_GEMM_PRE
    return hipGetLastError();
  }
#define FLARE_GEMM(C)                                                                  \
  if (rb == 2 && pair)                                                               \
    hipLaunchKernelGGL((gemm_bf16_kernel<C, 2, true>), grid, block, 0, st, p);       \
  else if (rb == 2)                                                                  \
    hipLaunchKernelGGL((gemm_bf16_kernel<C, 2, false>), grid, block, 0, st, p);      \
  else if (pair)                                                                     \
    hipLaunchKernelGGL((gemm_bf16_kernel<C, 1, true>), grid, block, 0, st, p);       \
  else                                                                               \
    hipLaunchKernelGGL((gemm_bf16_kernel<C, 1, false>), grid, block, 0, st, p)
  switch (p.Cin) {
    case 32: FLARE_GEMM(32); break;
    case 64: FLARE_GEMM(64); break;
    case 128: FLARE_GEMM(128); break;
    case 256: FLARE_GEMM(256); break;
    default: return hipErrorInvalidValue;
  }
#undef FLARE_GEMM
  return hipGetLastError();
}

}  // namespace flare
