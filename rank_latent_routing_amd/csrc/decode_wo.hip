// FLARE decoder with the output projection in its epilogue, for the FLARE++
// block: out = [Y_1 ... Y_H] W_O with Y_h = SDPA(K_h, Q_h, Z_h)
// ("FLARE++: Low-Rank Attention with Dynamic Attention Routing", section 3,
// "Full self-attention" for W_O and "FLARE: fixed-query latent routing" for
// the decoder call).
//
// The plain path runs the decoder per head, writes Y (bf16, [B, N, C]) and
// projects it with the GEMM.  Here one workgroup takes a window of 32 NW
// tokens of one batch element through every head: per head it brings the
// head's latent operands (Q in matrix-core order and Z^T, prepared once per
// call by stage_latents_kernel) into one of two LDS buffers by LDS-DMA while
// the other head computes, each wave computes its 32 tokens' outputs of that
// head exactly as the decoder does (one 32-token block per wave), and keeps
// them as packed bf16 in registers (16 per lane per head).  After the last
// head the workgroup brings W_O^T (prepared once per call by
// swizzle_wo_kernel) into LDS and each wave forms out^T = W_O^T Y^T for its
// tokens, 32 output columns at a time, and writes whole 128-byte lines of
// the row-major output.  Y never leaves registers.
//
// Layouts: the Z^T rows are permuted so that lane half h of a head's output
// holds features 8h .. 8h + 7 and 16 + 8h .. 16 + 8h + 7 of its token, which
// are the B operands of the head's two 16-feature k-steps of W_O^T Y^T; the
// W_O^T rows are permuted so that lane half h of a product holds the 16
// contiguous output columns 16h .. 16h + 15 of its token.  Both are the
// decoder's own trick (any fixed row order of the A operand is a free
// permutation of the product's rows).
#include "common.hpp"
#include "launch.hpp"

namespace flare {

typedef __attribute__((address_space(3))) void lds_void_t;

// Feature held in row r of the Z^T operand (see above).
__device__ __forceinline__ int wo_sigma_y(int r) {
  return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}
// Output column (within a 32-column block) held in row r of the W_O^T operand.
__device__ __forceinline__ int wo_sigma_o(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// Latent of element j of the Z^T operand of chunk ch, group ug, lane half h
// (the K order the packed weights of a 32 x 32 score tile give).
__device__ __forceinline__ int wo_chunk_latent(int ch, int ug, int h, int j) {
  return 32 * ch + 16 * ug + (j < 4 ? 4 * h + j : 8 + 4 * h + (j - 4));
}

// One 16-byte unit per thread: for (b, h) = blockIdx.y, unit u of
//   q_ops [MC][2][64]  Q operand: lane (hh, cc) of chunk ch, slice sd: latent
//                      32 ch + cc, features 16 sd + 8 hh .. +7
//   z_ops [MC][2][64]  Z^T operand: lane (hh, r) of chunk ch, group ug:
//                      element j is latent wo_chunk_latent(ch, ug, hh, j),
//                      feature wo_sigma_y(r)
// written back to back (MC * 4 KB per (b, h)); latents past M are zero.
__global__ __launch_bounds__(256) void stage_latents_kernel(DecodeWoParams p) {
  const int MC = (p.M + 31) / 32;
  const int units = MC * 4 * 64;
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int bh = blockIdx.y, b = bh / p.H, hd = bh - b * p.H;
  const int half = u / (MC * 2 * 64), v = u - half * (MC * 2 * 64);
  const int ch = v >> 7, k2 = (v >> 6) & 1, ln = v & 63, hh = ln >> 5, cc = ln & 31;
  bf16x8 out;
  if (half == 0) {
    const int m = 32 * ch + cc;
    float qv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[j] = 0.f;
    if (m < p.M) load_as_f32<8>(p.q.data, p.q.is_f32, b * p.q.sb + hd * p.q.sh + (int64_t)m * p.q.sl + 16 * k2 + 8 * hh, qv);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = (bf16)qv[j];
  } else {
    const int d = wo_sigma_y(cc);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = wo_chunk_latent(ch, k2, hh, j);
      float zv = 0.f;
      if (m < p.M) load_as_f32<1>(p.z.data, p.z.is_f32, b * p.z.sb + hd * p.z.sh + (int64_t)m * p.z.sl + d, &zv);
      out[j] = (bf16)zv;
    }
  }
  reinterpret_cast<bf16x8*>(p.lat_ops)[(int64_t)bh * units + u] = out;
}

// W_O [C, C] (row-major, input feature x output column) into the LDS order
// of its transpose: row rr is output column 32 (rr / 32) + wo_sigma_o(rr %
// 32); its C / 8 chunks of 8 input features are stored at chunk position
// kc ^ (rr % (C / 8)), so that the 32 rows an operand read touches fall in
// distinct bank groups.
__global__ __launch_bounds__(256) void swizzle_wo_kernel(const bf16* __restrict__ w, bf16* __restrict__ wt, int C) {
  const int KC = C / 8;
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= C * KC) return;
  const int rr = g / KC, kc = g - rr * KC;
  const int col = 32 * (rr >> 5) + wo_sigma_o(rr & 31);
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = w[(int64_t)(8 * kc + j) * C + col];
  reinterpret_cast<bf16x8*>(wt)[(int64_t)rr * KC + (kc ^ (rr % KC))] = v;
}

template <int HH>
__global__ __launch_bounds__(64 * kDecWoWaves, 3) void decode_wo_kernel(DecodeWoParams p) {
  constexpr int NW = kDecWoWaves;
  constexpr int SD = 2;  // head width 32: two 16-wide feature slices
  constexpr int C = 32 * HH, KC = C / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y;
  const int MC = (p.M + 31) / 32;
  const bool m_ragged = p.M != 32 * MC;
  const int lat_bytes = MC * 4096;
  const int64_t n = (int64_t)blockIdx.x * 32 * NW + 32 * wave + c;  // this lane's token
  const bool valid = n < p.N;
  const float cs = p.c;

  // Contiguous bytes [src, src + bytes) into LDS at dst: wave-wide 1 KB
  // buffer loads straight into LDS, spread over the waves (bytes is a
  // multiple of 1 KB; every lane offset lies inside the range).
  auto dma = [&](const unsigned char* src, int bytes, unsigned char* dst) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(src), (short)0, bytes, kBufferFlags);
    for (int op = wave; op < bytes / 1024; op += NW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + op * 1024), 16, lane * 16, op * 1024, 0, 0);
  };
  unsigned char* buf0 = smem;
  unsigned char* buf1 = smem + p.buf_bytes;
  const unsigned char* lat_b = p.lat_ops + (int64_t)b * HH * lat_bytes;

  // B operands of S^T = Q K^T for head hd: lane (h, c) holds token n,
  // features 16 sd + 8h .. +7 (zeros past the end).
  auto load_k = [&](int hd, bf16x8 (&kb)[SD]) {
    const bf16* kp = reinterpret_cast<const bf16*>(p.k.data) + b * p.k.sb + hd * p.k.sh + (valid ? n : 0) * p.k.sl;
#pragma unroll
    for (int sd = 0; sd < SD; ++sd) {
      if (valid) {
        kb[sd] = *reinterpret_cast<const bf16x8*>(kp + 16 * sd + 8 * h);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) kb[sd][j] = (bf16)0.0f;
      }
    }
  };

  bf16x8 ybuf[HH][2];  // each head's output, packed: the epilogue's B operands
  bf16x8 kb[SD], kn[SD];
  dma(lat_b, lat_bytes, buf0);
  load_k(0, kb);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  barrier_keep_loads();

#pragma unroll
  for (int hd = 0; hd < HH; ++hd) {
    const unsigned char* cur = (hd & 1) ? buf1 : buf0;
    // the next head's latent operands and K, while this head computes (its
    // buffer held head hd - 1, which every wave finished before the barrier)
    if (hd + 1 < HH) {
      dma(lat_b + (hd + 1) * lat_bytes, lat_bytes, (hd & 1) ? buf0 : buf1);
      load_k(hd + 1, kn);
    }
    const bf16x8* q_lds = reinterpret_cast<const bf16x8*>(cur);  // [MC][SD][64]
    const bf16x8* z_lds = q_lds + MC * SD * 64;                   // [MC][2][64]

    f32x16 yacc;
    float lsum, mx = 0.f;
    auto load_q = [&](bf16x8 (&qa)[SD], int ch) {
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) qa[sd] = q_lds[(ch * SD + sd) * 64 + lane];
    };
    auto qk = [&](const bf16x8 (&qa)[SD]) {
      f32x16 sc = zero16();
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) sc = mfma_32x32x16(qa[sd], kb[sd], sc);
      return sc;
    };
    // Weights of one score tile (element i: latent 32 ch + 8(i/4) + 4h + i%4
    // of token n), their row sums, and Y^T += Z^T P^T.
    auto softmax_pv = [&](auto exact_tag, auto mask_tag, f32x16 sc, int ch, float (&ls)[2]) {
      constexpr bool EXACT = decltype(exact_tag)::value;
      constexpr bool MASK = decltype(mask_tag)::value;
      const bf16x8 za0 = z_lds[(ch * 2 + 0) * 64 + lane];
      const bf16x8 za1 = z_lds[(ch * 2 + 1) * 64 + lane];
      const int rel = p.M - 32 * ch - 4 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (EXACT)
          sc[i] = exp2_fast(sc[i] * cs - mx);
        else
          sc[i] = exp2_fast(sc[i] * cs);
        if constexpr (MASK) {
          if (8 * (i >> 2) + (i & 3) >= rel) sc[i] = 0.f;
        }
      }
#pragma unroll
      for (int ug = 0; ug < 2; ++ug) {
        const bf16x8 pb = pack8_16(sc, ug);
        const u32x4 w = __builtin_bit_cast(u32x4, pb);
#pragma unroll
        for (int j = 0; j < 4; ++j) ls[j & 1] = dot2_ones(w[j], ls[j & 1]);
        yacc = mfma_32x32x16(ug == 0 ? za0 : za1, pb, yacc);
      }
    };
    // All chunks; the next chunk's scores are formed before this chunk's
    // weights, so the matrix cores run under the exponentials.
    auto pass = [&](auto exact_tag) {
      float ls[2] = {0.f, 0.f};
      yacc = zero16();
      bf16x8 qa[SD];
      load_q(qa, 0);
      f32x16 s0 = qk(qa);
      for (int ch = 0; ch + 1 < MC; ++ch) {
        load_q(qa, ch + 1);
        const f32x16 s1 = qk(qa);
        softmax_pv(exact_tag, std::integral_constant<bool, false>(), s0, ch, ls);
        s0 = s1;
      }
      if (m_ragged)
        softmax_pv(exact_tag, std::integral_constant<bool, true>(), s0, MC - 1, ls);
      else
        softmax_pv(exact_tag, std::integral_constant<bool, false>(), s0, MC - 1, ls);
      lsum = ls[0] + ls[1];
      lsum += shfl_xor_f(lsum, 32);
    };

    // Fast pass (weights 2^x without a maximum), kept when every token's
    // normaliser over its M weights lies in [M 2^-102, 2^100] and its outputs
    // are finite; otherwise the wave reruns the head with the row maximum.
    bool exact = p.exact != 0;
    if (!exact) {
      pass(std::integral_constant<bool, false>());
      bool ok = lsum >= (float)(32 * MC) * kSafeLoPerTerm && lsum <= kSafeHi;
#pragma unroll
      for (int i = 0; i < 16; ++i) ok = ok && __builtin_isfinite(yacc[i]);
      exact = __any(valid && !ok);
    }
    if (exact) {
      mx = -INFINITY;
      for (int ch = 0; ch < MC; ++ch) {
        bf16x8 qa[SD];
        load_q(qa, ch);
        const f32x16 sc = qk(qa);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * ch + 8 * (i >> 2) + 4 * h + (i & 3) < p.M) mx = fmaxf(mx, sc[i] * cs);
      }
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      pass(std::integral_constant<bool, true>());
    }
    // normalised outputs: element i is feature wo_sigma_y(8(i/4) + 4h + i%4),
    // i.e. 8h + i for i < 8 and 16 + 8h + (i - 8) above
    const float inv = __builtin_amdgcn_rcpf(lsum);
#pragma unroll
    for (int i = 0; i < 16; ++i) yacc[i] *= inv;
    ybuf[hd][0] = pack8_16(yacc, 0);
    ybuf[hd][1] = pack8_16(yacc, 1);

    // the next head's operands have landed and every wave is done with this
    // head's buffer
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    barrier_keep_loads();
    if (hd + 1 < HH) {
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) kb[sd] = kn[sd];
    }
  }

  // Epilogue: W_O^T into the two buffers (output columns 0 .. C/2 - 1, then
  // C/2 .. C - 1), then out^T = W_O^T Y^T, 32 columns at a time.
  const int half_bytes = C * C;  // C/2 rows x C bf16
  dma(p.wt, half_bytes, buf0);
  dma(p.wt + half_bytes, half_bytes, buf1);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  barrier_keep_loads();
  bf16* orow = reinterpret_cast<bf16*>(p.out) + ((int64_t)b * p.N + (valid ? n : 0)) * C;
  bf16x8 carry0, carry1;
#pragma unroll
  for (int cb = 0; cb < C / 32; ++cb) {
    const bf16x8* wl = reinterpret_cast<const bf16x8*>(cb < C / 64 ? buf0 : buf1);
    const int rr = (cb % (C / 64)) * 32 + c;  // row within the half
    f32x16 acc = zero16();
#pragma unroll
    for (int hd = 0; hd < HH; ++hd)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int kc = 4 * hd + 2 * s + h;
        acc = mfma_32x32x16(wl[rr * KC + (kc ^ (rr % KC))], ybuf[hd][s], acc);
      }
    // lane half h holds output columns 32 cb + 16h .. +15 of token n; two
    // blocks' results go out together, so each 128-byte line of the row is
    // written by the two lane halves within a few instructions
    const bf16x8 v0 = pack8_16(acc, 0), v1 = pack8_16(acc, 1);
    if ((cb & 1) == 0) {
      carry0 = v0;
      carry1 = v1;
    } else if (valid) {
      bf16* o0 = orow + 32 * (cb - 1) + 16 * h;
      bf16* o1 = orow + 32 * cb + 16 * h;
      *reinterpret_cast<bf16x8*>(o0) = carry0;
      *reinterpret_cast<bf16x8*>(o0 + 8) = carry1;
      *reinterpret_cast<bf16x8*>(o1) = v0;
      *reinterpret_cast<bf16x8*>(o1 + 8) = v1;
    }
  }
}

size_t decode_wo_lds(int M, int C) {
  const size_t lat = (size_t)((M + 31) / 32) * 4096;
  const size_t wo = (size_t)C * C;  // half of W_O^T
  return 2 * (lat > wo ? lat : wo);
}

hipError_t launch_decode_wo(const DecodeWoParams& p, int B, const void* w_o, hipStream_t st) {
  const int C = 32 * p.H;
  const int MC = (p.M + 31) / 32;
  hipLaunchKernelGGL(swizzle_wo_kernel, dim3((unsigned)((C * (C / 8) + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const bf16*>(w_o), reinterpret_cast<bf16*>(p.wt), C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stage_latents_kernel, dim3((unsigned)((MC * 4 * 64 + 255) / 256), (unsigned)(B * p.H)),
                     dim3(256), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  DecodeWoParams q = p;
  q.buf_bytes = (int)(decode_wo_lds(p.M, C) / 2);
  const size_t lds = decode_wo_lds(p.M, C);
  dim3 grid((unsigned)((p.N + 32 * kDecWoWaves - 1) / (32 * kDecWoWaves)), (unsigned)B);
  if (p.H == 8) {
    if ((e = hipFuncSetAttribute((const void*)decode_wo_kernel<8>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL((decode_wo_kernel<8>), grid, dim3(64 * kDecWoWaves), lds, st, q);
  } else if (p.H == 4) {
    if ((e = hipFuncSetAttribute((const void*)decode_wo_kernel<4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL((decode_wo_kernel<4>), grid, dim3(64 * kDecWoWaves), lds, st, q);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace flare
