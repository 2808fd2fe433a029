// Pointwise projections Y_p = X W_p on gfx950 bf16 matrix cores
// ("FLARE++: Low-Rank Attention with Dynamic Attention Routing", section 3:
// K = X W_K and V = X W_V in "Full self-attention" / "FLARE: fixed-query
// latent routing", the extra eK, eV of equation 7, and the output
// projection).  At C <= 1024 the reduction is short, so the kernel is built
// around reading X from HBM once:
//   - a wave loads its 64 rows of X once into registers, already as the B
//     operand of Y^T = W^T X^T (lane (g, r): row r, inputs 8g..8g+7 of each
//     32-wide step), and keeps them for every output column;
//   - the weights are pre-swizzled (once per call, a few hundred KB) into
//     operand order, so a 16-column block is a contiguous 1 KB per k-step that
//     the workgroup copies into LDS (double buffered) and all four waves read;
//   - the output tile comes out transposed, so each lane holds 4 consecutive
//     output columns of one row and stores them as one 8-byte write.
#include "common.hpp"
#include "launch.hpp"

namespace flare {

// wsw[cb][ks][lane][j] = W[32 ks + 8 (lane/16) + j][16 cb + lane%16]
__global__ __launch_bounds__(256) void swizzle_weights_kernel(const bf16* __restrict__ w,
                                                              bf16* __restrict__ wsw, int Cin,
                                                              int Cout) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)Cin * Cout;
  if (idx >= total) return;
  const int j = (int)(idx & 7);
  const int lane = (int)((idx >> 3) & 63);
  const int64_t rest = idx >> 9;
  const int KS = Cin / 32;
  const int ks = (int)(rest % KS);
  const int cb = (int)(rest / KS);
  const int c = 32 * ks + 8 * (lane >> 4) + j;
  const int col = 16 * cb + (lane & 15);
  wsw[idx] = w[(int64_t)c * Cout + col];
}

constexpr int kGemmRowsPerWave = 64;
constexpr int kGemmWaves = 4;

template <int CIN>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmParams p, int cb_per_group) {
  constexpr int KS = CIN / 32;
  constexpr int BLK = KS * 64 * 8;  // bf16 elements of one swizzled 16-column block
  __shared__ __attribute__((aligned(16))) bf16 w_lds[2][BLK];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int64_t row0 = (int64_t)blockIdx.x * (kGemmRowsPerWave * kGemmWaves) + wave * kGemmRowsPerWave;
  const int cb_per_proj = p.Cout / 16;
  const int cb_total = p.n_proj * cb_per_proj;
  const int cb_begin = blockIdx.y * cb_per_group;
  const int cb_end = min(cb_total, cb_begin + cb_per_group);
  const bf16* xin = reinterpret_cast<const bf16*>(p.x);

  // X rows as B operands, held for all output columns.
  bf16x8 xb[4][KS];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
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

  constexpr int CHUNKS = BLK / 8;  // 16-byte chunks per block
  constexpr int PER = (CHUNKS + 255) / 256;
  u32x4 stage[PER];
  auto src_block = [&](int cb) -> const bf16* {
    const int pr = cb / cb_per_proj, cbl = cb - pr * cb_per_proj;
    return reinterpret_cast<const bf16*>(p.wt[pr]) + (int64_t)cbl * BLK;
  };
  auto load_block = [&](int cb) {
    const u32x4* src = reinterpret_cast<const u32x4*>(src_block(cb));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + 256 * i;
      if (u < CHUNKS) stage[i] = src[u];
    }
  };
  auto store_block = [&](int buf) {
    u32x4* dst = reinterpret_cast<u32x4*>(w_lds[buf]);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + 256 * i;
      if (u < CHUNKS) dst[u] = stage[i];
    }
  };

  if (cb_begin < cb_end) {
    load_block(cb_begin);
    store_block(0);
  }
  __syncthreads();
  for (int cb = cb_begin; cb < cb_end; ++cb) {
    const int buf = (cb - cb_begin) & 1;
    if (cb + 1 < cb_end) load_block(cb + 1);
    f32x4 acc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&w_lds[buf][(ks * 64 + lane) * 8]);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb] = mfma_16x16x32(a, xb[rb][ks], acc[rb]);
    }
    // lane (g, r) of tile rb holds output columns 16cbl + 4g .. +3 of row
    // row0 + 16rb + r
    const int pr = cb / cb_per_proj, cbl = cb - pr * cb_per_proj;
    const int col = 16 * cbl + 4 * g;
    bf16* yout = reinterpret_cast<bf16*>(p.y[pr]);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int64_t row = row0 + 16 * rb + r;
      if (row >= p.R) continue;
      int64_t off;
      if (p.head_major) {
        const int64_t bi = row / p.N, n = row - bi * p.N;
        const int hd = col / p.D, d = col - hd * p.D;
        const int H = p.Cout / p.D;
        off = ((bi * H + hd) * p.N + n) * p.D + d;
      } else {
        off = row * p.Cout + col;
      }
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (bf16)acc[rb][i];
      *reinterpret_cast<bf16x4*>(yout + off) = v;
    }
    if (cb + 1 < cb_end) store_block(buf ^ 1);
    __syncthreads();
  }
}

hipError_t launch_transpose_weights(const void* w, void* wt, int Cin, int Cout, hipStream_t st) {
  const int64_t total = (int64_t)Cin * Cout;
  hipLaunchKernelGGL(swizzle_weights_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const bf16*>(w), reinterpret_cast<bf16*>(wt), Cin, Cout);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t st) {
  const int64_t rows_per_block = kGemmRowsPerWave * kGemmWaves;
  const int64_t row_blocks = (p.R + rows_per_block - 1) / rows_per_block;
  const int cb_total = p.n_proj * (p.Cout / 16);
  // Enough workgroups to cover 256 compute units several times: split the
  // output columns across workgroups when there are few row blocks.
  int groups = 1;
  while (row_blocks * groups < 1024 && groups * 2 <= cb_total) groups *= 2;
  const int per = (cb_total + groups - 1) / groups;
  groups = (cb_total + per - 1) / per;
  dim3 grid((unsigned)row_blocks, groups);
  switch (p.Cin) {
    case 32: hipLaunchKernelGGL((gemm_bf16_kernel<32>), grid, dim3(256), 0, st, p, per); break;
    case 64: hipLaunchKernelGGL((gemm_bf16_kernel<64>), grid, dim3(256), 0, st, p, per); break;
    case 128: hipLaunchKernelGGL((gemm_bf16_kernel<128>), grid, dim3(256), 0, st, p, per); break;
    case 256: hipLaunchKernelGGL((gemm_bf16_kernel<256>), grid, dim3(256), 0, st, p, per); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace flare
