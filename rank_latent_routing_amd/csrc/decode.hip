// FLARE decoder for gfx950: Y_h = SDPA(K_h, Q_h, Z_h), every token takes a
// softmax over the M latents and gathers their values ("FLARE++: Low-Rank
// Attention with Dynamic Attention Routing", section 3, "FLARE: fixed-query
// latent routing", the second SDPA call; "FLARE++: dynamic token routing" uses
// the synthesized Q_h(X) here).
//
// A workgroup stages its head's latent side once in LDS, already in matrix-core
// operand order: Q in bf16 (A operand of S^T = Q K^T) and Z transposed (A
// operand of Y^T = Z^T P^T).  Each wave then streams 64-token groups of K
// straight from HBM into registers (one 16-byte load per lane and 16-token
// block), walks the latents 32 at a time and keeps every token's softmax
// inside the wave: a token's 32 scores of a chunk sit in 4 lanes x 8
// registers, the weights are packed to bf16 in place as the B operand of the
// Z^T P^T product, and the normaliser is the dot2 sum of those packed
// weights, reduced over the 4 lanes at the end.  No score leaves registers.
//
// As in the encoder, the first pass uses weights 2^x without a maximum; a
// 64-token group whose normaliser leaves [2^-100, 2^100] (or whose output is
// not finite) is recomputed with the exact two-pass softmax (row maximum
// across the lanes of the token first).  FLARE_FLAG_EXACT_SOFTMAX forces it.
#include "common.hpp"
#include "launch.hpp"

namespace flare {

// Latent row m of chunk c that lane group g, element j of a B/A operand with
// K = 32 latents refers to (the layout the S^T output tiles produce).
__device__ __forceinline__ int chunk_latent(int c, int g, int j) {
  return 32 * c + (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
}

constexpr int kDecWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kDecWaves, 4) void decode_bf16_kernel(DecodeParams p) {
  using Op = QkOp<D>;
  using op_t = typename Op::type;
  constexpr int PL = Op::per_lane;
  constexpr int NW = kDecWaves;
  constexpr int NT = 64 * NW;
  constexpr int DB = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int bh = blockIdx.y;
  const int b = bh / p.H, h = bh - b * p.H;
  const int MC = (p.M + 31) / 32;  // 32-latent chunks
  const int MB = 2 * MC;           // 16-latent blocks
  const bool m_ragged = p.M != 32 * MC;
  op_t* q_lds = reinterpret_cast<op_t*>(smem);                                           // [MB][64]
  bf16x8* z_lds = reinterpret_cast<bf16x8*>(smem + (size_t)MB * 64 * sizeof(op_t));  // [MC][DB][64]

  // Stage Q: lane (g, r) of block nb holds latent 16nb + r, columns g*PL...
  for (int u = tid; u < MB * 64; u += NT) {
    const int nb = u >> 6, ln = u & 63, gg = ln >> 4, rr = ln & 15;
    const int m = 16 * nb + rr;
    float qv[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) qv[j] = 0.f;
    if (m < p.M) load_as_f32<PL>(p.q.data, p.q.is_f32, b * p.q.sb + h * p.q.sh + (int64_t)m * p.q.sl + gg * PL, qv);
    op_t qb;
#pragma unroll
    for (int j = 0; j < PL; ++j) qb[j] = (bf16)qv[j];
    q_lds[nb * 64 + ln] = qb;
  }
  // Stage Z^T: row r of column block e is feature d = sigma(e, r), chosen so
  // that the output tile rows 4g..4g+3 of both blocks are 8 contiguous
  // features 8g..8g+7 (D = 32) or 4g..4g+3 (D = 16) of one token.
  for (int u = tid; u < MC * DB * 64; u += NT) {
    const int c = u / (DB * 64), e = (u >> 6) % DB, ln = u & 63, gg = ln >> 4, rr = ln & 15;
    const int d = D == 32 ? 8 * (rr >> 2) + 4 * e + (rr & 3) : rr;
    bf16x8 val;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = chunk_latent(c, gg, j);
      float zv = 0.f;
      if (m < p.M) load_as_f32<1>(p.z.data, p.z.is_f32, b * p.z.sb + h * p.z.sh + (int64_t)m * p.z.sl + d, &zv);
      val[j] = (bf16)zv;
    }
    z_lds[(c * DB + e) * 64 + ln] = val;
  }
  __syncthreads();

  const bf16 zero = (bf16)0.0f;
  const float cs = p.c;
  const bf16* kbase = reinterpret_cast<const bf16*>(p.k.data) + b * p.k.sb + h * p.k.sh;
  const int64_t n_begin = (int64_t)blockIdx.x * p.tokens_per_block;
  const int64_t n_end = min(p.N, n_begin + p.tokens_per_block);

  const int MCF = p.M / 32;  // chunks with all 32 latents valid

  // B operands of S^T = Q K^T: lane (g, r) holds token base + 16t + r,
  // features g*PL ...; the next 64-token group is loaded while the current
  // one is computed.
  auto load_k = [&](op_t (&kk)[4], int64_t base) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t n = base + 16 * t + r;
      if (n < n_end) {
        kk[t] = *reinterpret_cast<const op_t*>(kbase + n * p.k.sl + g * PL);
      } else {
#pragma unroll
        for (int j = 0; j < PL; ++j) kk[t][j] = zero;
      }
    }
  };
  op_t kb[4], kn[4];
  load_k(kb, n_begin + 64 * wave);
  // Wait for the first group here, outside the loop: vmcnt counts loads and
  // stores in order, and without this the compiler waits for everything
  // (the next group's prefetch included) at the head of the latent loop.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0) expcnt(7) lgkmcnt(15)

  for (int64_t base = n_begin + 64 * wave; base < n_end; base += 64 * NW) {
    load_k(kn, base + 64 * NW);

    f32x4 yacc[4][DB];
    float lsum[4], mx[4];
    // One 32-latent chunk against the 64 tokens.  MASK (only the last chunk
    // when M is not a multiple of 32) gives padded latents weight 0.
    auto chunk = [&](auto exact_tag, auto mask_tag, int c) {
      constexpr bool EXACT = decltype(exact_tag)::value;
      constexpr bool MASK = decltype(mask_tag)::value;
      const op_t q0 = q_lds[(2 * c) * 64 + lane];
      const op_t q1 = q_lds[(2 * c + 1) * 64 + lane];
      bf16x8 za[DB];
#pragma unroll
      for (int e = 0; e < DB; ++e) za[e] = z_lds[(c * DB + e) * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 s0 = Op::mma(q0, kb[t], f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 s1 = Op::mma(q1, kb[t], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (EXACT) {
            s0[i] = exp2_fast(s0[i] * cs - mx[t]);
            s1[i] = exp2_fast(s1[i] * cs - mx[t]);
          } else {
            s0[i] = exp2_fast(s0[i] * cs);
            s1[i] = exp2_fast(s1[i] * cs);
          }
          if constexpr (MASK) {
            if (32 * c + 4 * g + i >= p.M) s0[i] = 0.f;
            if (32 * c + 16 + 4 * g + i >= p.M) s1[i] = 0.f;
          }
        }
        const bf16x8 pb = pack8(s0, s1);
        lsum[t] = rowsum_bf16x8(pb, lsum[t]);
#pragma unroll
        for (int e = 0; e < DB; ++e) yacc[t][e] = mfma_16x16x32(za[e], pb, yacc[t][e]);
      }
    };
    auto pass = [&](auto exact_tag) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int e = 0; e < DB; ++e) yacc[t][e] = f32x4{0.f, 0.f, 0.f, 0.f};
        lsum[t] = 0.f;
      }
      for (int c = 0; c < MCF; ++c) chunk(exact_tag, std::integral_constant<bool, false>(), c);
      if (m_ragged) chunk(exact_tag, std::integral_constant<bool, true>(), MC - 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lsum[t] += shfl_xor_f(lsum[t], 16);
        lsum[t] += shfl_xor_f(lsum[t], 32);
      }
    };

    bool exact = p.exact != 0;
    if (!exact) {
      pass(std::integral_constant<bool, false>());
      bool bad = false;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float l = lsum[t];
        bool ok = l >= kSafeLo && l <= kSafeHi;
#pragma unroll
        for (int e = 0; e < DB; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) ok = ok && __builtin_isfinite(yacc[t][e][i]);
        bad = bad || (base + 16 * t + r < n_end && !ok);
      }
      exact = __any(bad);
    }
    if (exact) {
      // Row maximum of every token over all valid latents.
#pragma unroll
      for (int t = 0; t < 4; ++t) mx[t] = -INFINITY;
      for (int nb = 0; nb < MB; ++nb) {
        const op_t qb = q_lds[nb * 64 + lane];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 sc = Op::mma(qb, kb[t], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * nb + 4 * g + i < p.M) mx[t] = fmaxf(mx[t], sc[i] * cs);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        mx[t] = fmaxf(mx[t], shfl_xor_f(mx[t], 16));
        mx[t] = fmaxf(mx[t], shfl_xor_f(mx[t], 32));
      }
      pass(std::integral_constant<bool, true>());
    }

    // Output: lane (g, r) holds token base + 16t + r, features 8g..8g+7
    // (D = 32: rows 4g..4g+3 of block 0 then of block 1) or 4g..4g+3 (D = 16).
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t n = base + 16 * t + r;
      if (n >= n_end) continue;
      const float inv = 1.0f / lsum[t];
      float out[4 * DB];
#pragma unroll
      for (int e = 0; e < DB; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[4 * e + i] = yacc[t][e][i] * inv;
      const int64_t off = b * p.y_sb + h * p.y_sh + n * p.y_sl + g * 4 * DB;
      if (p.y_f32) {
        float* yp = reinterpret_cast<float*>(p.y) + off;
#pragma unroll
        for (int j = 0; j < 4 * DB; j += 4)
          *reinterpret_cast<f32x4*>(yp + j) = f32x4{out[j], out[j + 1], out[j + 2], out[j + 3]};
      } else {
        bf16* yp = reinterpret_cast<bf16*>(p.y) + off;
        if constexpr (DB == 2) {
          bf16x8 v;
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = (bf16)out[j];
          *reinterpret_cast<bf16x8*>(yp) = v;
        } else {
          bf16x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (bf16)out[j];
          *reinterpret_cast<bf16x4*>(yp) = v;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) kb[t] = kn[t];
  }
}

// ---------------------------------------------------------------- fp32 path
// One thread per token; Q (times scale*log2 e) and Z staged in LDS; exact
// two-pass softmax over the M latents in fp32.
template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* q_s = reinterpret_cast<float*>(smem);
  float* z_s = q_s + (size_t)p.M * D;
  const int tid = threadIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, h = bh - b * p.H;
  for (int u = tid; u < p.M * D; u += 256) {
    const int m = u / D, d = u % D;
    float qv, zv;
    load_as_f32<1>(p.q.data, p.q.is_f32, b * p.q.sb + h * p.q.sh + (int64_t)m * p.q.sl + d, &qv);
    load_as_f32<1>(p.z.data, p.z.is_f32, b * p.z.sb + h * p.z.sh + (int64_t)m * p.z.sl + d, &zv);
    q_s[u] = qv * p.c;
    z_s[u] = zv;
  }
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * 256 + tid;
  if (n >= p.N) return;
  const float* kp = reinterpret_cast<const float*>(p.k.data) + b * p.k.sb + h * p.k.sh + n * p.k.sl;
  float k[D];
#pragma unroll
  for (int d = 0; d < D; ++d) k[d] = kp[d];
  float mx = -INFINITY;
  for (int m = 0; m < p.M; ++m) {
    float x = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) x = fmaf(k[d], q_s[m * D + d], x);
    mx = fmaxf(mx, x);
  }
  float l = 0.f, acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  for (int m = 0; m < p.M; ++m) {
    float x = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) x = fmaf(k[d], q_s[m * D + d], x);
    const float pw = exp2f(x - mx);
    l += pw;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(pw, z_s[m * D + d], acc[d]);
  }
  const float inv = 1.0f / l;
  const int64_t off = b * p.y_sb + h * p.y_sh + n * p.y_sl;
  if (p.y_f32) {
    float* yp = reinterpret_cast<float*>(p.y) + off;
#pragma unroll
    for (int d = 0; d < D; ++d) yp[d] = acc[d] * inv;
  } else {
    bf16* yp = reinterpret_cast<bf16*>(p.y) + off;
#pragma unroll
    for (int d = 0; d < D; ++d) yp[d] = (bf16)(acc[d] * inv);
  }
}

// ---------------------------------------------------------------- launchers

size_t decode_bf16_lds(int M, int D) {
  const int MC = (M + 31) / 32;
  const size_t op_bytes = D == 32 ? 16 : 8;
  return (size_t)2 * MC * 64 * op_bytes + (size_t)MC * (D / 16) * 64 * 16;
}

// Kernels that stage more than 64 KB of LDS must opt in to the larger limit.
template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_decode_bf16(const DecodeParams& p, int D, int B, hipStream_t st) {
  const int64_t blocks = (p.N + p.tokens_per_block - 1) / p.tokens_per_block;
  dim3 grid((unsigned)blocks, B * p.H);
  const size_t lds = decode_bf16_lds(p.M, D);
  hipError_t e;
  if (D == 32) {
    if ((e = allow_lds(decode_bf16_kernel<32>, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((decode_bf16_kernel<32>), grid, dim3(64 * kDecWaves), lds, st, p);
  } else {
    if ((e = allow_lds(decode_bf16_kernel<16>, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((decode_bf16_kernel<16>), grid, dim3(64 * kDecWaves), lds, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeParams& p, int D, int B, hipStream_t st) {
  dim3 grid((unsigned)((p.N + 255) / 256), B * p.H);
  const size_t lds = (size_t)p.M * D * 2 * sizeof(float);
  hipError_t e;
  if (D == 32) {
    if ((e = allow_lds(decode_f32_kernel<32>, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((decode_f32_kernel<32>), grid, dim3(256), lds, st, p);
  } else {
    if ((e = allow_lds(decode_f32_kernel<16>, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((decode_f32_kernel<16>), grid, dim3(256), lds, st, p);
  }
  return hipGetLastError();
}

}  // namespace flare
