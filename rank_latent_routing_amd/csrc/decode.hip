// FLARE decoder for gfx950: Y_h = SDPA(K_h, Q_h, Z_h), every token takes a
// softmax over the M latents and gathers their values ("FLARE++: Low-Rank
// Attention with Dynamic Attention Routing", section 3, "FLARE: fixed-query
// latent routing", the second SDPA call; "FLARE++: dynamic token routing" uses
// the synthesized Q_h(X) here).
//
// A workgroup stages its head's latent side once in LDS, already in matrix-core
// operand order: Q in bf16 (A operand of S^T = Q K^T) and Z transposed (A
// operand of Y^T = Z^T P^T).  Each wave then streams 64-token groups of K
// from HBM into a private LDS slot by buffer loads that write LDS directly
// (the next group's load is in flight while the current group is computed),
// reads the B operands from that slot, and walks the latents 32 at a time with
// v_mfma_f32_32x32x16_bf16.  A lane's 16 scores of a chunk all belong to its
// token, so every token's softmax stays in two lanes: the weights are packed
// to bf16 in place as the B operand of Z^T P^T, the normaliser is the dot2 sum
// of those packed weights, and the two lane halves are added at the end.  No
// score leaves registers, and each lane writes 16 contiguous features of its
// token.
//
// As in the encoder, the first pass uses weights 2^x without a maximum; a
// 64-token group in which some token's normaliser over its M latents leaves
// [M 2^-102, 2^100] (or whose output is not finite) is recomputed with the
// exact two-pass softmax (row maximum first).  The bounds keep the weights
// finite and the mass of flushed weights below fp32 rounding.
// FLARE_FLAG_EXACT_SOFTMAX forces the exact form.
#include "common.hpp"
#include "launch.hpp"

namespace flare {

// Latent of element j (K slot (h, j)) of 16-latent group u in 32-latent chunk
// ch: the rows the 32x32 score tile gives lane half h.
__device__ __forceinline__ int chunk_latent(int ch, int u, int h, int j) {
  return 32 * ch + 16 * u + (j < 4 ? 4 * h + j : 8 + 4 * h + (j - 4));
}


typedef __attribute__((address_space(3))) void lds_void_t;

// Position of 16-byte chunk dc of token t in a wave's K slot: the chunk index
// is XOR-swizzled with bits 2..3 of the token so that the operand reads (32
// lanes = 32 consecutive tokens, one chunk each) hit distinct bank groups.
template <int D>
__device__ __forceinline__ int dec_k_pos(int token, int dc) {
  if constexpr (D == 32) return token * 4 + (dc ^ ((token >> 2) & 3));
  else return token * 2 + (dc ^ ((token >> 2) & 1));
}

template <int D>
__global__ __launch_bounds__(64 * kDecWaves, 3) void decode_bf16_kernel(DecodeParams p) {
  constexpr int NW = kDecWaves;
  constexpr int NT = 64 * NW;
  constexpr int SD = D / 16;
  constexpr int ROWC = D / 8;                       // 16-byte chunks per token row
  constexpr int KOPS = kDecGroup * ROWC / 64;       // wave-wide DMA loads per group
  constexpr int KSLOT = kDecGroup * D;              // bf16 elements of a wave's K slot
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wave
  const int bh = blockIdx.y;
  const int b = bh / p.H, hd = bh - b * p.H;
  const int MC = (p.M + 31) / 32;  // 32-latent chunks
  const bool m_ragged = p.M != 32 * MC;
  bf16x8* q_lds = reinterpret_cast<bf16x8*>(smem);                                          // [MC][SD][64]
  bf16x8* z_lds = reinterpret_cast<bf16x8*>(smem + (size_t)MC * SD * 64 * sizeof(bf16x8));  // [MC][2][64]
  bf16* kslot = reinterpret_cast<bf16*>(smem + (size_t)MC * (SD + 2) * 64 * sizeof(bf16x8)) + wave * KSLOT;
  // merged Z [32 MC][D] in fp32, only when Z is merged here from the split results
  float* zm = reinterpret_cast<float*>(smem + (size_t)MC * (SD + 2) * 64 * sizeof(bf16x8) +
                                       (size_t)NW * KSLOT * sizeof(bf16));

  // Zero this wave's K slot: lanes past the last token may leave their chunk
  // unwritten, and the stale data must be finite (its scores are discarded).
  {
    const bf16x8 z8 = {};
    for (int u = lane; u < KSLOT / 8; u += 64) reinterpret_cast<bf16x8*>(kslot)[u] = z8;
  }
  // the zeros are in LDS before the first group's loads can land in the slot
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  const bf16* kbase = reinterpret_cast<const bf16*>(p.k.data) + b * p.k.sb + hd * p.k.sh;
  // Workgroup b owns the (NW x 64)-token passes b, b + G, b + 2G, ... of its
  // head (G = gridDim.x), so the resident workgroups sweep one window of K.
  // Its 64-token groups (group j: slot j % NW of its pass j / NW) go to the
  // waves in order: wave w starts with group w and then claims the next
  // unclaimed one from an LDS counter.  A SIMD favours its oldest wave, so
  // with fixed shares the oldest waves finished far ahead of the youngest
  // (at 50 %, 75 % and 100 % of the kernel's time at the bench size) and each
  // SIMD ran the rest with fewer waves; claimed groups keep all three waves
  // busy to the end.  The outputs do not depend on which wave takes a group.
  const int64_t n_end = p.N;
  auto group_base = [&](unsigned j) -> int64_t {
    return ((int64_t)blockIdx.x + (int64_t)(j / NW) * gridDim.x) * (kDecGroup * NW) + (int64_t)(j % NW) * kDecGroup;
  };

  // K of a 64-token group comes by buffer loads into the wave's LDS slot
  // (a uniform descriptor covering exactly the group's valid rows, and
  // loop-invariant 32-bit lane offsets).  The next group's load is in flight
  // while the current group is computed.
  // Load t covers tokens (64 / ROWC) t .. +63 / ROWC; lane l reads token
  // (64 / ROWC) t + l / ROWC.  The swizzle depends on token bits 2..3 only,
  // so it is the same for every t.  The whole byte offset sits in the lane
  // (VGPR) operand, the part the hardware compares with the descriptor's
  // range: a lane whose token is past the end reads zeros instead of memory
  // beyond the tensor.  (The scalar offset operand is not range-checked, so
  // it stays 0.)
  const int k_tok = lane / ROWC, k_sw = lane % ROWC;
  const int k_dc = D == 32 ? (k_sw ^ ((k_tok >> 2) & 3)) : (k_sw ^ ((k_tok >> 2) & 1));
  const uint32_t k_off0 = (uint32_t)((k_tok * p.k.sl + k_dc * 8) * (int64_t)sizeof(bf16));
  const uint32_t k_step = (uint32_t)((64 / ROWC) * p.k.sl * (int64_t)sizeof(bf16));  // bytes per load
  auto issue_k = [&](int64_t g0) {
    const int64_t rows = g0 < n_end ? min((int64_t)kDecGroup, n_end - g0) : 0;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>(kbase + (g0 < n_end ? g0 : 0) * p.k.sl), (short)0,
        (int)(rows * p.k.sl * (int64_t)sizeof(bf16)), kBufferFlags);
#pragma unroll
    for (int t = 0; t < KOPS; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(kslot + t * 512), 16, k_off0 + t * k_step, 0, 0, 0);
  };

  int64_t base = group_base(wave), nbase = 0;
  if (base < n_end) issue_k(base);
  // The first group's K loads are in flight while Q and Z are staged below.

  // Stage Q: lane (h, c) of chunk ch, slice sd holds latent 32ch + c,
  // features 16sd + 8h .. +7 in bf16; the scale multiplies the fp32 scores.
  for (int u = tid; u < MC * SD * 64; u += NT) {
    const int ch = u / (SD * 64), sd = (u >> 6) % SD, ln = u & 63, hh = ln >> 5, cc = ln & 31;
    const int m = 32 * ch + cc;
    float qv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[j] = 0.f;
    if (m < p.M) load_as_f32<8>(p.q.data, p.q.is_f32, b * p.q.sb + hd * p.q.sh + (int64_t)m * p.q.sl + 16 * sd + 8 * hh, qv);
    bf16x8 qb;
#pragma unroll
    for (int j = 0; j < 8; ++j) qb[j] = (bf16)qv[j];
    q_lds[(ch * SD + sd) * 64 + ln] = qb;
  }
  // With zm_part_o, Z is first merged from the encoder's split results (the
  // same fold as the merge kernel, splits in order) into LDS, four features
  // per thread, and staged from there.
  const bool z_merge = p.zm_part_o != nullptr;
  if (z_merge) {
    const int64_t MD = (int64_t)p.M * D;
    for (int u = tid; u < p.M * (D / 4); u += NT) {
      const int m = u / (D / 4), d4 = 4 * (u % (D / 4));
      const f32x4 v = merge_splits4(p.zm_part_l + (int64_t)bh * p.zm_S * p.M + m, p.M,
                                    reinterpret_cast<const f32x4*>(p.zm_part_o + (int64_t)bh * p.zm_S * MD +
                                                                   (int64_t)m * D + d4),
                                    MD / 4, p.zm_S);
      *reinterpret_cast<f32x4*>(zm + m * D + d4) = v;
    }
    __syncthreads();
  }
  // Stage Z^T: row r (lane c = r) of the A operand is feature
  // sigma(r) = 16((r >> 2) & 1) + 4(r >> 3) + (r & 3), chosen so that the
  // output rows lane half h receives (8q + 4h + i%4) are the 16 contiguous
  // features 16h .. 16h + 15 of its token; rows with sigma(r) >= D are zero.
  // z_bounded: every staged value below 2^26 in magnitude (false for NaN).
  bool z_bounded = true;
  for (int u = tid; u < MC * 2 * 64; u += NT) {
    const int ch = u >> 7, ug = (u >> 6) & 1, ln = u & 63, hh = ln >> 5, r = ln & 31;
    const int d = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
    bf16x8 val;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = chunk_latent(ch, ug, hh, j);
      float zv = 0.f;
      if (m < p.M && d < D) {
        if (z_merge)
          zv = zm[m * D + d];
        else
          load_as_f32<1>(p.z.data, p.z.is_f32, b * p.z.sb + hd * p.z.sh + (int64_t)m * p.z.sl + d, &zv);
      }
      val[j] = (bf16)zv;
      z_bounded = z_bounded && fabsf((float)val[j]) < 67108864.0f;
    }
    z_lds[(ch * 2 + ug) * 64 + ln] = val;
  }
  // Each weight is at most the normaliser l it sums into, so with every
  // |Z| < 2^26 and l <= 2^100 the unnormalised outputs stay below 2^126:
  // only l needs checking before the fast result is kept.
  __shared__ unsigned next_group;  // the workgroup's next unclaimed 64-token group
  if (tid == 0) next_group = NW;
  const bool z_small = __syncthreads_and(z_bounded) != 0;

  const float cs = p.c;
  for (; base < n_end; base = nbase) {
    // B operands of S^T = Q K^T: lane (h, c) holds token base + 32tb + c,
    // features 16sd + 8h .. +7.
    bf16x8 kb[2][SD];
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int sd = 0; sd < SD; ++sd)
        kb[tb][sd] = *reinterpret_cast<const bf16x8*>(kslot + 8 * dec_k_pos<D>(32 * tb + c, 2 * sd + h));
    // the slot is read before the next group's load may overwrite it
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    unsigned jn = 0;
    if (lane == 0) jn = atomicAdd(&next_group, 1u);
    nbase = group_base(__builtin_amdgcn_readfirstlane(jn));
    if (nbase < n_end) issue_k(nbase);

    f32x16 yacc[2];
    float lsum[2], mx[2];
    // S^T of 32-latent chunk ch against token block tb (32 tokens) with the
    // chunk's Q operands qa.  Element i of a score tile is latent
    // 32ch + 8(i/4) + 4h + i%4 of token c.
    auto load_q = [&](bf16x8 (&qa)[SD], int ch) {
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) qa[sd] = q_lds[(ch * SD + sd) * 64 + lane];
    };
    auto qk = [&](const bf16x8 (&qa)[SD], int tb) {
      f32x16 sc = zero16();
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) sc = mfma_32x32x16(qa[sd], kb[tb][sd], sc);
      return sc;
    };
    // Weights of one score tile, their row sums (two independent
    // accumulators) and Y^T += Z^T P^T.  MASK (only the last chunk when M is
    // not a multiple of 32) gives padded latents weight 0.
    auto softmax_pv = [&](auto exact_tag, auto mask_tag, f32x16 sc, int ch, int tb, float (&ls)[2][2]) {
      constexpr bool EXACT = decltype(exact_tag)::value;
      constexpr bool MASK = decltype(mask_tag)::value;
      const bf16x8 za0 = z_lds[(ch * 2 + 0) * 64 + lane];
      const bf16x8 za1 = z_lds[(ch * 2 + 1) * 64 + lane];
      // latent 32ch + 8(i/4) + 4h + i%4 is valid iff 8(i/4) + i%4 < rel
      const int rel = p.M - 32 * ch - 4 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (EXACT)
          sc[i] = exp2_fast(sc[i] * cs - mx[tb]);
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
        for (int j = 0; j < 4; ++j) ls[tb][j & 1] = dot2_ones(w[j], ls[tb][j & 1]);
        yacc[tb] = mfma_32x32x16(ug == 0 ? za0 : za1, pb, yacc[tb]);
      }
    };
    // All chunks, software-pipelined over the units (chunk, token block):
    // the S^T product of the next unit is issued before the softmax of the
    // current one, so the matrix cores run under the exponentials.  The last
    // chunk is peeled off (it carries the padding mask when M is not a
    // multiple of 32).
    auto pass = [&](auto exact_tag) {
      float ls[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        yacc[tb] = zero16();
        ls[tb][0] = ls[tb][1] = 0.f;
      }
      bf16x8 qa[SD];
      load_q(qa, 0);
      f32x16 s0 = qk(qa, 0);
      for (int ch = 0; ch + 1 < MC; ++ch) {
        load_q(qa, ch);
        const f32x16 s1 = qk(qa, 1);
        softmax_pv(exact_tag, std::integral_constant<bool, false>(), s0, ch, 0, ls);
        load_q(qa, ch + 1);
        s0 = qk(qa, 0);
        softmax_pv(exact_tag, std::integral_constant<bool, false>(), s1, ch, 1, ls);
      }
      load_q(qa, MC - 1);
      const f32x16 s1 = qk(qa, 1);
      if (m_ragged) {
        softmax_pv(exact_tag, std::integral_constant<bool, true>(), s0, MC - 1, 0, ls);
        softmax_pv(exact_tag, std::integral_constant<bool, true>(), s1, MC - 1, 1, ls);
      } else {
        softmax_pv(exact_tag, std::integral_constant<bool, false>(), s0, MC - 1, 0, ls);
        softmax_pv(exact_tag, std::integral_constant<bool, false>(), s1, MC - 1, 1, ls);
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        lsum[tb] = ls[tb][0] + ls[tb][1];
        lsum[tb] += shfl_xor_f(lsum[tb], 32);
      }
    };

    bool exact = p.exact != 0;
    if (!exact) {
      // each token's normaliser sums 32 MC weights
      const float lsum_lo = (float)(32 * MC) * kSafeLoPerTerm;
      pass(std::integral_constant<bool, false>());
      bool bad = false;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        bool ok = lsum[tb] >= lsum_lo && lsum[tb] <= kSafeHi;
        if (!z_small) {
#pragma unroll
          for (int i = 0; i < 16; ++i) ok = ok && __builtin_isfinite(yacc[tb][i]);
        }
        bad = bad || (base + 32 * tb + c < n_end && !ok);
      }
      exact = __any(bad);
    }
    if (exact) {
      // Row maximum of every token over all valid latents.
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) mx[tb] = -INFINITY;
      for (int ch = 0; ch < MC; ++ch) {
        bf16x8 qa[SD];
        load_q(qa, ch);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const f32x16 sc = qk(qa, tb);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * ch + 8 * (i >> 2) + 4 * h + (i & 3) < p.M) mx[tb] = fmaxf(mx[tb], sc[i] * cs);
        }
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) mx[tb] = fmaxf(mx[tb], shfl_xor_f(mx[tb], 32));
      pass(std::integral_constant<bool, true>());
    }

    // Row normalisers (natural log) for the backward pass.
    if (p.lse && h == 0) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int64_t n = base + 32 * tb + c;
        if (n < n_end) p.lse[(int64_t)bh * p.N + n] = ((exact ? mx[tb] : 0.f) + __log2f(lsum[tb])) * kLn2;
      }
    }
    // Output: lane (h, c) holds token base + 32tb + c, features 16h .. 16h+15.
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t n = base + 32 * tb + c;
      if (n >= n_end || 16 * h >= D) continue;
      const float inv = __builtin_amdgcn_rcpf(lsum[tb]);  // 1 ulp
      const int64_t off = b * p.y_sb + hd * p.y_sh + n * p.y_sl + 16 * h;
      if (p.y_f32) {
        float* yp = reinterpret_cast<float*>(p.y) + off;
#pragma unroll
        for (int j = 0; j < 16; j += 4)
          *reinterpret_cast<f32x4*>(yp + j) =
              f32x4{yacc[tb][j] * inv, yacc[tb][j + 1] * inv, yacc[tb][j + 2] * inv, yacc[tb][j + 3] * inv};
      } else {
        bf16* yp = reinterpret_cast<bf16*>(p.y) + off;
#pragma unroll
        for (int j = 0; j < 16; j += 8) {
          bf16x8 v;
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = (bf16)(yacc[tb][j + k] * inv);
          *reinterpret_cast<bf16x8*>(yp + j) = v;
        }
      }
    }
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
  if (p.lse) p.lse[(int64_t)blockIdx.y * p.N + n] = (mx + log2f(l)) * kLn2;
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

// Kernels that stage more than 64 KB of LDS must opt in to the larger limit.
template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_decode_bf16(const DecodeParams& p, int D, int B, hipStream_t st) {
  const int64_t blocks = p.tokens_per_block;  // workgroups per head
  dim3 grid((unsigned)blocks, B * p.H);
  const size_t lds = decode_bf16_lds(p.M, D) + (p.zm_part_o ? decode_merge_lds(p.M, D) : 0);
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
