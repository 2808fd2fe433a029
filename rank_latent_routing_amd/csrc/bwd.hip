// Backward of the FLARE encoder and decoder on gfx950 bf16 matrix cores.
//
// Both calls are standard scaled dot-product attention ("FLARE++: Low-Rank
// Attention with Dynamic Attention Routing", section 3, "FLARE: fixed-query
// latent routing"), so their gradients are the standard SDPA gradients: with
// s = scale q . k, P the softmax weights, o the output and do its gradient,
//   delta = do . o (per query row),  dS = P (do . v - delta),
//   dq = scale sum dS k,  dk = scale sum dS q,  dv = sum P do.
// P is recomputed from the log-normaliser each forward call returns
// (P = 2^(c s - L) with c = scale log2 e and L the base-2 normaliser), so no
// score leaves the chip and no running maximum is needed.
//
// Every gradient is a sum over one axis of the token x latent score matrix.
// Sums over latents (dK, dV) run token-parallel in the decoder's layout
// (tok_bwd_kernel, one call's role; tok_pair_kernel, both roles of a FLARE
// encode/decode pair at once); sums over tokens (dQ, dZ) run latent-parallel
// over token splits in the encoder's layout (lat_bwd_kernel), with fp32
// partials per split added by sum_splits_kernel.  The operand layouts are
// those of the forward kernels: see encode_kernel.hpp and decode.hip.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace flare {

// Latent of element j (K slot (h, j)) of 16-latent group u in 32-latent chunk
// ch, as in the decoder: the rows a 32x32 score tile gives lane half h.
__device__ __forceinline__ int bwd_chunk_latent(int ch, int u, int h, int j) {
  return 32 * ch + 16 * u + (j < 4 ? 4 * h + j : 8 + 4 * h + (j - 4));
}

// Stage a latent-side [M, D] block of one head into LDS in the two operand
// layouts the token-parallel pass uses:
//   a_lds  [MC][SD][64]: A operand of a product against tokens (lane (h, c):
//                        latent 32ch + c, features 16sd + 8h .. +7);
//   at_lds [MC][2][64]:  transposed A operand (rows are features sigma(r),
//                        K slots latents), so each lane ends with 16
//                        contiguous features of its token; skipped when null;
//   alo_lds (optional):  the bf16 rounding residual of a_lds, for products
//                        whose fp32 input must keep about 16 mantissa bits.
template <int D>
__device__ void stage_latent_block(const View& v, int b, int hd, int M, int MC, bf16x8* a_lds, bf16x8* at_lds,
                                   int tid, int nt, bf16x8* alo_lds = nullptr) {
  constexpr int SD = D / 16;
  for (int u = tid; u < MC * SD * 64; u += nt) {
    const int ch = u / (SD * 64), sd = (u >> 6) % SD, ln = u & 63, hh = ln >> 5, cc = ln & 31;
    const int m = 32 * ch + cc;
    float vv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = 0.f;
    if (m < M) load_as_f32<8>(v.data, v.is_f32, b * v.sb + hd * v.sh + (int64_t)m * v.sl + 16 * sd + 8 * hh, vv);
    bf16x8 o, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      o[j] = (bf16)vv[j];
      lo[j] = (bf16)(vv[j] - (float)o[j]);
    }
    a_lds[(ch * SD + sd) * 64 + ln] = o;
    if (alo_lds) alo_lds[(ch * SD + sd) * 64 + ln] = lo;
  }
  if (!at_lds) return;
  for (int u = tid; u < MC * 2 * 64; u += nt) {
    const int ch = u >> 7, ug = (u >> 6) & 1, ln = u & 63, hh = ln >> 5, r = ln & 31;
    const int d = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = bwd_chunk_latent(ch, ug, hh, j);
      float x = 0.f;
      if (m < M && d < D) load_as_f32<1>(v.data, v.is_f32, b * v.sb + hd * v.sh + (int64_t)m * v.sl + d, &x);
      o[j] = (bf16)x;
    }
    at_lds[(ch * 2 + ug) * 64 + ln] = o;
  }
}

// The view's rows from m0 on (latent-side tensors).
__device__ __forceinline__ View rows_from(View v, int m0) {
  v.data = reinterpret_cast<const char*>(v.data) + (int64_t)m0 * v.sl * (v.is_f32 ? 4 : 2);
  return v;
}

// Store 16 gradient values of one lane (features f .. f + 15 of a token) at
// p: fp32 as four 16-byte stores, or bf16 as two; with accumulate the old
// values are added first (in fp32; the bf16 sum rounds once).
__device__ __forceinline__ void store_grad16(void* p, bool bf16_out, bool accumulate, const float (&v)[16]) {
  if (bf16_out) {
    bf16x8* q = reinterpret_cast<bf16x8*>(p);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 o;
      const bf16x8 old = accumulate ? q[half] : bf16x8{};
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = (bf16)(accumulate ? v[8 * half + j] + (float)old[j] : v[8 * half + j]);
      q[half] = o;
    }
  } else {
    f32x4* q = reinterpret_cast<f32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 o = {v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
      if (accumulate) o += q[j];
      q[j] = o;
    }
  }
}

// ------------------------------------------------------- token-parallel pass
// waves per workgroup: 4 in the decode role, 8 in the encode role (whose
// larger latent staging leaves one workgroup per CU)
template <bool ENC>
constexpr int tok_bwd_waves() { return ENC ? 8 : 4; }

// The offset L / c of a padded row: c (S - offset) is then about -2.5e29 |c|
// for either sign of the exponent scale c, so the row's weight is exactly 0.
__device__ __forceinline__ float pad_offset(float c) { return c > 0.f ? 1e30f : -1e30f; }

// In the encode role dP = dZ . V is reduced against delta_m = dZ . Z, and
// when the encoder's weights are concentrated the two nearly cancel.  Below
// kDzSplitBelowM latents dZ enters the product as bf16 high and low parts
// (about 16 mantissa bits) and delta_m is formed from the fp32 dZ.  From
// kDzSplitBelowM latents on dZ enters in bf16 alone and delta_m is formed
// from the same bf16 values, so that dP - delta_m = bf16(dZ) . (V_n - Z_m)
// carries only the rounding of dZ itself.  (A seeded sweep of sharp cases
// put the single-part form within 10 % of the two-part error from 8 latents
// on, and up to 55 % above it at 1 to 3 latents.)
constexpr int kDzSplitBelowM = 32;
__device__ __forceinline__ float dz_for_delta(float dz, bool split) { return split ? dz : (float)(bf16)dz; }

// v as three bf16 terms, written to e[at], e[at + 1], e[at + 2], whose sum
// carries v to about fp32 precision.
__device__ __forceinline__ void split3_bf16(float v, bf16x8& e, int at) {
  const bf16 a = (bf16)v;
  float r = v - (float)a;
  const bf16 b = (bf16)r;
  r -= (float)b;
  e[at] = a;
  e[at + 1] = b;
  e[at + 2] = (bf16)r;
}

// Per-latent terms of the encode role enter the score products as one more
// 16-wide matrix-core K step: with A holding (t1, t2, t3) of latent m in
// columns 0..2 and B holding -1 there, S' = S - (t1 + t2 + t3) for every
// token.  With t1 + t2 + t3 = L_m / c (the normaliser over the exponent
// scale) the exponent c S' equals c S - L_m, and with the delta terms
// dP' = dP - delta_m; the products are exact and the fp32 accumulation
// rounds like the subtraction itself.  Each lane of an A operand holds one
// latent, so this replaces a per-element LDS read of the row's normaliser
// and delta by one 16-byte read per lane and chunk.

template <int D, bool ENC, bool DZS>
__global__ __launch_bounds__(64 * tok_bwd_waves<ENC>(), 2) void tok_bwd_kernel(TokBwdParams p) {
  constexpr int NW = tok_bwd_waves<ENC>();
  constexpr int SD = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.y, b = bh / p.H, hd = bh - b * p.H;
  // this launch's latents [m0, m0 + mb)
  const int MC = (p.mb + 31) / 32;
  const View qv = rows_from(p.q, p.m0), wv = rows_from(p.w, p.m0), zv = rows_from(p.z, p.m0);
  bf16x8* q_lds = reinterpret_cast<bf16x8*>(smem);
  bf16x8* w_lds = q_lds + MC * SD * 64;
  bf16x8* qt_lds = w_lds + MC * SD * 64;
  bf16x8* wt_lds = qt_lds + MC * 2 * 64;           // encode role
  bf16x8* aug_lds = wt_lds + MC * 2 * 64;          // encode role: MC * 32 latents + a zero slot
  bf16x8* wlo_lds = aug_lds + (MC * 32 + 1);        // encode role, few latents: dZ - bf16(dZ)
  constexpr bool dz_split = ENC && DZS;  // dZ as high and low parts (fewer than kDzSplitBelowM latents)

  stage_latent_block<D>(qv, b, hd, p.mb, MC, q_lds, qt_lds, tid, 64 * NW);
  // In the encode role W = dZ is an fp32 gradient (its high and low bf16
  // parts with few latents)
  stage_latent_block<D>(wv, b, hd, p.mb, MC, w_lds, ENC ? wt_lds : nullptr, tid, 64 * NW,
                        dz_split ? wlo_lds : nullptr);
  if constexpr (ENC) {
    // per latent m: L_m / c (base-2 normaliser over the exponent scale) and
    // delta_m = dZ_m . Z_m (dZ as it enters dP), three bf16 terms each: (t1, t2, t3, 0, d1, d2, d3,
    // 0).  Padded latents get a huge finite offset (weight exactly 0); the
    // slot after the last latent stays zero for the lanes of the second K half.
    for (int m = tid; m <= MC * 32; m += 64 * NW) {
      bf16x8 e = {};
      if (m < MC * 32) {
        float v = pad_offset(p.c), dl = 0.f;
        if (m < p.mb) {
          v = p.lse[(int64_t)bh * p.M + p.m0 + m] * kLog2e / p.c;
          for (int d = 0; d < D; ++d) {
            float a, z;
            load_as_f32<1>(wv.data, wv.is_f32, b * wv.sb + hd * wv.sh + (int64_t)m * wv.sl + d, &a);
            load_as_f32<1>(zv.data, zv.is_f32, b * zv.sb + hd * zv.sh + (int64_t)m * zv.sl + d, &z);
            dl = fmaf(dz_for_delta(a, dz_split), z, dl);
          }
        }
        split3_bf16(v, e, 0);
        split3_bf16(dl, e, 4);
      }
      aug_lds[m] = e;
    }
  }
  __shared__ unsigned next_grp;  // the workgroup's next unclaimed token group
  if (tid == 0) next_grp = NW;
  __syncthreads();

  // B operand of the extra K step: -1 in K rows 0..2 (lane half 0), else 0
  bf16x8 bneg = {};
  if (h == 0) bneg[0] = bneg[1] = bneg[2] = (bf16)-1.0f;

  const bf16* kbase = reinterpret_cast<const bf16*>(p.k.data) + b * p.k.sb + hd * p.k.sh;
  const bf16* xbase = reinterpret_cast<const bf16*>(p.x.data) + b * p.x.sb + hd * p.x.sh;
  const float cs = p.c;
  // A wave takes 64 tokens at a time, two blocks of 32 (lane (h, c): token
  // base + 32 tb + c): every LDS read of a latent chunk serves two score
  // tiles, and the products of the second block run under the first block's
  // exponentials.
  // Workgroup b owns the 64-token groups of the (NW x 64)-token passes b,
  // b + G, ... (G = gridDim.x); wave w starts with group w and then claims
  // the next unclaimed group from an LDS counter (a SIMD favours its oldest
  // wave: with fixed shares the youngest waves finished last, alone).
  auto grp = [&](unsigned j) -> int64_t {
    return ((int64_t)blockIdx.x + (int64_t)(j / NW) * gridDim.x) * (NW * 64) + (int64_t)(j % NW) * 64;
  };
  auto claim = [&]() -> unsigned {
    unsigned jn = 0;
    if (lane == 0) jn = atomicAdd(&next_grp, 1u);
    return __builtin_amdgcn_readfirstlane(jn);
  };
  for (int64_t base = grp(wave); base < p.N; base = grp(claim())) {
    // B operands: token n, features 16sd + 8h .. +7 of K and of X
    bf16x8 kb[2][SD], xb[2][SD];
    float l2n[2] = {0.f, 0.f}, dln[2] = {0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t n = base + 32 * tb + c;
      const bool valid = n < p.N;
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) {
        if (valid) {
          kb[tb][sd] = *reinterpret_cast<const bf16x8*>(kbase + n * p.k.sl + 16 * sd + 8 * h);
          xb[tb][sd] = *reinterpret_cast<const bf16x8*>(xbase + n * p.x.sl + 16 * sd + 8 * h);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) kb[tb][sd][j] = xb[tb][sd][j] = (bf16)0.0f;
        }
      }
      if constexpr (!ENC) {
        // delta_n = dY_n . Y_n over the token's D features (half per lane half)
        const bf16* ybase = reinterpret_cast<const bf16*>(p.y.data) + b * p.y.sb + hd * p.y.sh;
        float part = 0.f;
        if (valid) {
#pragma unroll
          for (int sd = 0; sd < SD; ++sd) {
            const bf16x8 yv = *reinterpret_cast<const bf16x8*>(ybase + n * p.y.sl + 16 * sd + 8 * h);
#pragma unroll
            for (int j = 0; j < 8; ++j) part = fmaf((float)xb[tb][sd][j], (float)yv[j], part);
          }
          l2n[tb] = p.lse[(int64_t)bh * p.N + n] * kLog2e;
        }
        dln[tb] = part + shfl_xor_f(part, 32);
        if (h == 0 && valid) p.delta[(int64_t)bh * p.N + n] = dln[tb];
      }
    }

    f32x16 dk[2], dv[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) dk[tb] = dv[tb] = zero16();
    for (int ch = 0; ch < MC; ++ch) {
      // S^T and dP^T of both token blocks; element i of a tile is latent
      // 32ch + 8(i/4) + 4h + i%4
      f32x16 sc[2], dp[2];
      {
        bf16x8 qa[SD], wa[SD], wl[SD];
#pragma unroll
        for (int sd = 0; sd < SD; ++sd) {
          qa[sd] = q_lds[(ch * SD + sd) * 64 + lane];
          wa[sd] = w_lds[(ch * SD + sd) * 64 + lane];
          if constexpr (dz_split) wl[sd] = wlo_lds[(ch * SD + sd) * 64 + lane];
        }
        bf16x8 as = {}, ad = {};
        if constexpr (ENC) {
          const u32x4 e = __builtin_bit_cast(u32x4, aug_lds[h == 0 ? 32 * ch + c : MC * 32]);
          as = __builtin_bit_cast(bf16x8, u32x4{e[0], e[1], 0u, 0u});
          ad = __builtin_bit_cast(bf16x8, u32x4{e[2], e[3], 0u, 0u});
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          sc[tb] = zero16();
          dp[tb] = zero16();
#pragma unroll
          for (int sd = 0; sd < SD; ++sd) {
            sc[tb] = mfma_32x32x16(qa[sd], kb[tb][sd], sc[tb]);
            dp[tb] = mfma_32x32x16(wa[sd], xb[tb][sd], dp[tb]);
            if constexpr (dz_split) dp[tb] = mfma_32x32x16(wl[sd], xb[tb][sd], dp[tb]);
          }
          if constexpr (ENC) {
            sc[tb] = mfma_32x32x16(as, bneg, sc[tb]);
            dp[tb] = mfma_32x32x16(ad, bneg, dp[tb]);
          }
        }
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        f32x16 pw, ds;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (ENC) {
            pw[i] = exp2_fast(sc[tb][i] * cs);
            ds[i] = pw[i] * dp[tb][i];
          } else {
            pw[i] = exp2_fast(sc[tb][i] * cs - l2n[tb]);
            ds[i] = pw[i] * (dp[tb][i] - dln[tb]);
          }
        }
#pragma unroll
        for (int ug = 0; ug < 2; ++ug) {
          dk[tb] = mfma_32x32x16(qt_lds[(ch * 2 + ug) * 64 + lane], pack8_16(ds, ug), dk[tb]);
          if constexpr (ENC) dv[tb] = mfma_32x32x16(wt_lds[(ch * 2 + ug) * 64 + lane], pack8_16(pw, ug), dv[tb]);
        }
      }
    }
    // lane (h, c): token base + 32 tb + c, features 16h .. 16h + 15
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t n = base + 32 * tb + c;
      if (n >= p.N || 16 * h >= D) continue;
      const int es = p.grad_bf16 ? 2 : 4;  // bytes per gradient element
      float g[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) g[j] = dk[tb][j] * p.scale;
      store_grad16(reinterpret_cast<char*>(p.dk) + (b * p.dk_sb + hd * p.dk_sh + n * p.dk_sl + 16 * h) * es,
                   p.grad_bf16, p.accumulate, g);
      if constexpr (ENC) {
#pragma unroll
        for (int j = 0; j < 16; ++j) g[j] = dv[tb][j];
        store_grad16(reinterpret_cast<char*>(p.dv) + (b * p.dv_sb + hd * p.dv_sh + n * p.dv_sl + 16 * h) * es,
                     p.grad_bf16, p.accumulate_v, g);
      }
    }
  }
}

// ------------------------------------------- token-parallel pass, both roles
// For the pair Z = SDPA(Q, K, V), Y = SDPA(K, Q, Z) the two calls score the
// same products s = scale q . k: the encoder normalises them per latent, the
// decoder per token.  One pass over the token x latent tiles therefore serves
// both token-side gradients,
//   dk_n = scale sum_m (P_d (dP_d - delta_n) + P_e (dP_e - delta_m)) q_m,
//   dv_n = sum_m P_e dZ_m,
// with P_d, dP_d = dY_n . Z_m from the decoder and P_e, dP_e = dZ_m . V_n from
// the encoder.  dK is written once, with no second pass reading it back.
constexpr int kTokPairWaves = 8;

template <int D, bool DZS>
__global__ __launch_bounds__(64 * kTokPairWaves, 2) void tok_pair_kernel(TokPairParams p) {
  constexpr int NW = kTokPairWaves;
  constexpr int SD = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.y, b = bh / p.H, hd = bh - b * p.H;
  const int MC = (p.M + 31) / 32;
  bf16x8* q_lds = reinterpret_cast<bf16x8*>(smem);  // A of S^T = Q K^T
  bf16x8* z_lds = q_lds + MC * SD * 64;             // A of dP_d^T = Z dY^T
  bf16x8* dz_lds = z_lds + MC * SD * 64;            // A of dP_e^T = dZ V^T
  bf16x8* qt_lds = dz_lds + MC * SD * 64;           // A of dK^T += Q^T dS^T
  bf16x8* dzt_lds = qt_lds + MC * 2 * 64;           // A of dV^T += dZ^T P_e^T
  bf16x8* aug_lds = dzt_lds + MC * 2 * 64;          // per latent L_m / c and delta_m; zero slot
  bf16x8* dzlo_lds = aug_lds + (MC * 32 + 1);       // few latents: dZ - bf16(dZ), the low part of dP_e's A
  constexpr bool dz_split = DZS;  // dZ as high and low parts (fewer than kDzSplitBelowM latents)

  stage_latent_block<D>(p.q, b, hd, p.M, MC, q_lds, qt_lds, tid, 64 * NW);
  stage_latent_block<D>(p.z, b, hd, p.M, MC, z_lds, nullptr, tid, 64 * NW);
  // dZ enters dP_e = dZ . V in bf16 (as high and low parts with few latents)
  stage_latent_block<D>(p.dz, b, hd, p.M, MC, dz_lds, dzt_lds, tid, 64 * NW, dz_split ? dzlo_lds : nullptr);
  for (int m = tid; m <= MC * 32; m += 64 * NW) {
    bf16x8 e = {};
    if (m < MC * 32) {
      float v = pad_offset(p.c), dl = 0.f;
      if (m < p.M) {
        v = p.lse_e[(int64_t)bh * p.M + m] * kLog2e / p.c;
        for (int d = 0; d < D; ++d) {
          float a, z;
          load_as_f32<1>(p.dz.data, p.dz.is_f32, b * p.dz.sb + hd * p.dz.sh + (int64_t)m * p.dz.sl + d, &a);
          load_as_f32<1>(p.z.data, p.z.is_f32, b * p.z.sb + hd * p.z.sh + (int64_t)m * p.z.sl + d, &z);
          dl = fmaf(dz_for_delta(a, dz_split), z, dl);
        }
      }
      split3_bf16(v, e, 0);
      split3_bf16(dl, e, 4);
    }
    aug_lds[m] = e;
  }
  __shared__ unsigned next_grp;  // the workgroup's next unclaimed token group
  if (tid == 0) next_grp = NW;
  __syncthreads();

  bf16x8 bneg = {};
  if (h == 0) bneg[0] = bneg[1] = bneg[2] = (bf16)-1.0f;
  const bf16* kbase = reinterpret_cast<const bf16*>(p.k.data) + b * p.k.sb + hd * p.k.sh;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v.data) + b * p.v.sb + hd * p.v.sh;
  const bf16* gbase = reinterpret_cast<const bf16*>(p.dy.data) + b * p.dy.sb + hd * p.dy.sh;
  const float cs = p.c;
  // The wave's next 32 tokens are loaded while the current ones are
  // computed: lane (h, c) holds token n, B operands with features
  // 16sd + 8h .. +7 of K, V and dY, and the token's normaliser and delta.
  bf16x8 nk[SD], nv[SD], ng[SD];
  float nl2 = 0.f, ndd = 0.f;
  auto fetch = [&](int64_t base) {
    const int64_t n = base + c;
    const bool valid = n < p.N;
#pragma unroll
    for (int sd = 0; sd < SD; ++sd) {
      if (valid) {
        nk[sd] = *reinterpret_cast<const bf16x8*>(kbase + n * p.k.sl + 16 * sd + 8 * h);
        nv[sd] = *reinterpret_cast<const bf16x8*>(vbase + n * p.v.sl + 16 * sd + 8 * h);
        ng[sd] = *reinterpret_cast<const bf16x8*>(gbase + n * p.dy.sl + 16 * sd + 8 * h);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) nk[sd][j] = nv[sd][j] = ng[sd][j] = (bf16)0.0f;
      }
    }
    nl2 = valid ? p.lse_d[(int64_t)bh * p.N + n] : 0.f;
    ndd = valid ? p.delta_d[(int64_t)bh * p.N + n] : 0.f;
  };
  // Workgroup b owns the 32-token groups of the (NW x 32)-token passes b,
  // b + G, ... (G = gridDim.x); wave w starts with group w and then claims
  // the next unclaimed group from an LDS counter, so that the waves a SIMD
  // favours (its oldest) take more groups and all finish together.
  auto grp = [&](unsigned j) -> int64_t {
    return ((int64_t)blockIdx.x + (int64_t)(j / NW) * gridDim.x) * (NW * 32) + (int64_t)(j % NW) * 32;
  };
  int64_t base = grp(wave), nbase = 0;
  if (base < p.N) fetch(base);
  for (; base < p.N; base = nbase) {
    const int64_t n = base + c;
    const bool valid = n < p.N;
    bf16x8 kb[SD], vb[SD], gb[SD];
#pragma unroll
    for (int sd = 0; sd < SD; ++sd) {
      kb[sd] = nk[sd];
      vb[sd] = nv[sd];
      gb[sd] = ng[sd];
    }
    const float l2d = nl2 * kLog2e;
    // dP_d - delta_n: the token's -delta_n starts every chunk's dP_d product
    f32x16 ddneg;
#pragma unroll
    for (int i = 0; i < 16; ++i) ddneg[i] = -ndd;
    unsigned jn = 0;
    if (lane == 0) jn = atomicAdd(&next_grp, 1u);
    nbase = grp(__builtin_amdgcn_readfirstlane(jn));
    if (nbase < p.N) fetch(nbase);

    f32x16 dk = zero16(), dv = zero16();
    for (int ch = 0; ch < MC; ++ch) {
      // element i of a tile: latent 32ch + 8(i/4) + 4h + i%4 of token n
      f32x16 sc = zero16(), dpd = ddneg, dpe = zero16();
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) {
        sc = mfma_32x32x16(q_lds[(ch * SD + sd) * 64 + lane], kb[sd], sc);
        dpd = mfma_32x32x16(z_lds[(ch * SD + sd) * 64 + lane], gb[sd], dpd);
        dpe = mfma_32x32x16(dz_lds[(ch * SD + sd) * 64 + lane], vb[sd], dpe);
        if constexpr (dz_split) dpe = mfma_32x32x16(dzlo_lds[(ch * SD + sd) * 64 + lane], vb[sd], dpe);
      }
      // the encoder's per-latent normaliser and delta as one more K step
      const u32x4 e = __builtin_bit_cast(u32x4, aug_lds[h == 0 ? 32 * ch + c : MC * 32]);
      const f32x16 se = mfma_32x32x16(__builtin_bit_cast(bf16x8, u32x4{e[0], e[1], 0u, 0u}), bneg, sc);
      dpe = mfma_32x32x16(__builtin_bit_cast(bf16x8, u32x4{e[2], e[3], 0u, 0u}), bneg, dpe);
      f32x16 pe, ds;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pd = exp2_fast(sc[i] * cs - l2d);
        pe[i] = exp2_fast(se[i] * cs);
        ds[i] = fmaf(pe[i], dpe[i], pd * dpd[i]);
      }
#pragma unroll
      for (int ug = 0; ug < 2; ++ug) {
        dk = mfma_32x32x16(qt_lds[(ch * 2 + ug) * 64 + lane], pack8_16(ds, ug), dk);
        dv = mfma_32x32x16(dzt_lds[(ch * 2 + ug) * 64 + lane], pack8_16(pe, ug), dv);
      }
    }
    // lane (h, c): token n, features 16h .. 16h + 15
    if (valid && 16 * h < D) {
      const int es = p.grad_bf16 ? 2 : 4;  // bytes per gradient element
      float g[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) g[j] = dk[j] * p.scale;
      store_grad16(reinterpret_cast<char*>(p.dk) + (b * p.dk_sb + hd * p.dk_sh + n * p.dk_sl + 16 * h) * es,
                   p.grad_bf16, p.accumulate, g);
#pragma unroll
      for (int j = 0; j < 16; ++j) g[j] = dv[j];
      store_grad16(reinterpret_cast<char*>(p.dv) + (b * p.dv_sb + hd * p.dv_sh + n * p.dv_sl + 16 * h) * es,
                   p.grad_bf16, false, g);
    }
  }
}

// ------------------------------------------------------ latent-parallel pass

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// 16-byte chunk slot of (token, chunk dc) in a staged token tile: the chunk
// index is XOR-swizzled with bits 2..3 (D = 32) or bit 2 (D = 16) of the
// token, so that the A-operand reads (a 16-lane group reads one chunk of 16
// consecutive tokens) spread over all bank groups.  The transposing reads
// take whole rows per 32-lane pass and stay conflict-free under any
// permutation of a row's chunks.
template <int D>
__device__ __forceinline__ int lat_chunk_pos(int token, int dc) {
  if constexpr (D == 32) return token * 4 + (dc ^ ((token >> 2) & 3));
  else return token * 2 + (dc ^ ((token >> 2) & 1));
}

// One workgroup is (batch*head, token split s, block of 32 NW latents); each
// wave owns 32 latents, one per lane column of its score tiles.  The split's
// 64-token tiles s, s + S, ... pass through registers (loaded one tile ahead)
// into LDS, shared by all waves; per tile a wave forms S^T and dP^T for its
// latents, the weights and score gradients, and adds dQ (and in the decode
// role dZ) by products with the staged tokens.  It ends by writing its
// split's fp32 partials.  The encoder role takes 4-wave workgroups from
// M = 128 on, three per compute unit (168 VGPRs): with one 8-wave workgroup
// per unit, each tile's barrier left its SIMDs idle.  The decoder role needs
// 199 VGPRs and keeps 8 waves at M = 256 (4-wave workgroups, two per unit,
// timed slower).
template <int D, bool ENC, int NW, bool DZS = false>
__global__ __launch_bounds__(64 * NW, (ENC && NW == 4) ? 3 : 2) void lat_bwd_kernel(LatBwdParams p) {
  constexpr int SD = D / 16;
  constexpr int T = kLatBwdTile;
  constexpr int NB = ENC ? 1 : 2;  // token tile buffers (the decode role double-buffers)
  __shared__ __attribute__((aligned(16))) bf16 kt_s[NB * T * D];
  __shared__ __attribute__((aligned(16))) bf16 xt_s[NB * T * D];
  __shared__ __attribute__((aligned(16))) bf16x8 aug_s[NB * (T + 1)];  // decode role: per token, and a zero slot
  const bf16* kt = kt_s;  // the buffer being computed
  const bf16* xt = xt_s;
  const bf16x8* augt = aug_s;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31, i16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x, bh = blockIdx.y, b = bh / p.H, hd = bh - b * p.H;
  const int lat0 = blockIdx.z * 32 * NW;
  const int m_lane = lat0 + wave * 32 + c;
  constexpr bool dz_split = ENC && DZS;  // dZ as high and low parts (fewer than kDzSplitBelowM latents)

  // B operands of the two products against this lane's latent: Q and W
  bf16x8 qop[SD], wop[SD], wlo[SD];
  float dpart = 0.f;
#pragma unroll
  for (int sd = 0; sd < SD; ++sd) {
    float qv[8], wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[j] = wv[j] = 0.f;
    if (m_lane < p.M) {
      load_as_f32<8>(p.q.data, p.q.is_f32, b * p.q.sb + hd * p.q.sh + (int64_t)m_lane * p.q.sl + 16 * sd + 8 * h, qv);
      load_as_f32<8>(p.w.data, p.w.is_f32, b * p.w.sb + hd * p.w.sh + (int64_t)m_lane * p.w.sl + 16 * sd + 8 * h, wv);
      if constexpr (ENC) {
        float zv[8];
        load_as_f32<8>(p.z.data, p.z.is_f32, b * p.z.sb + hd * p.z.sh + (int64_t)m_lane * p.z.sl + 16 * sd + 8 * h, zv);
#pragma unroll
        for (int j = 0; j < 8; ++j) dpart = fmaf(dz_for_delta(wv[j], dz_split), zv[j], dpart);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qop[sd][j] = (bf16)qv[j];
      wop[sd][j] = (bf16)wv[j];
      // encode role with few latents: W = dZ also as its bf16 rounding residual
      wlo[sd][j] = (bf16)(wv[j] - (float)wop[sd][j]);
    }
  }
  // encode role: this lane's latent's base-2 normaliser and delta_m = dZ . Z
  // (dZ as it enters dP)
  float l2m = INFINITY, dlm = 0.f;
  if constexpr (ENC) {
    dlm = dpart + shfl_xor_f(dpart, 32);
    if (m_lane < p.M) l2m = p.lse[(int64_t)bh * p.M + m_lane] * kLog2e;
  }

  const bf16* kbase = reinterpret_cast<const bf16*>(p.k.data) + b * p.k.sb + hd * p.k.sh;
  const bf16* xbase = reinterpret_cast<const bf16*>(p.x.data) + b * p.x.sb + hd * p.x.sh;
  const float cs = p.c;
  const bf16 zero = (bf16)0.0f;
  f32x16 dq = zero16(), dz = zero16();
  // B operand of the extra K step: -1 in K rows 0..2 (lane half 0), else 0
  bf16x8 bneg = {};
  if (h == 0) bneg[0] = bneg[1] = bneg[2] = (bf16)-1.0f;
  // encode role: delta_m as one more K step on dP (B: its three bf16 terms in
  // K rows 0..2 of the latent's column; A: -1 there for every token row)
  bf16x8 dlmop = {};
  if constexpr (ENC) {
    if (h == 0) split3_bf16(dlm, dlmop, 0);
  }

  // The staged tile's products for this wave's 32 latents.  RAGGED (encode
  // role, last tile only) gives tokens past the end weight 0 through an
  // infinite normaliser; in the decode role their staged offset already
  // does.
  auto tile = [&](auto ragged_tag, int rem) {
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    // S^T and dP^T of 32-token half qt: element i is token
    // 32qt + 8(i/4) + 4h + i%4 of latent c.  In the decode role the token's
    // normaliser and delta enter as an extra K step, as in the token pass.
    auto products = [&](int qt, f32x16& sc, f32x16& dp) {
      sc = zero16();
      dp = zero16();
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) {
        const int slot = 8 * lat_chunk_pos<D>(32 * qt + c, 2 * sd + h);
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + slot);
        const bf16x8 xa = *reinterpret_cast<const bf16x8*>(xt + slot);
        sc = mfma_32x32x16(ka, qop[sd], sc);
        dp = mfma_32x32x16(xa, wop[sd], dp);
        if constexpr (dz_split) dp = mfma_32x32x16(xa, wlo[sd], dp);
      }
      if constexpr (ENC) dp = mfma_32x32x16(bneg, dlmop, dp);
      if constexpr (!ENC) {
        const u32x4 e = __builtin_bit_cast(u32x4, augt[h == 0 ? 32 * qt + c : T]);
        sc = mfma_32x32x16(__builtin_bit_cast(bf16x8, u32x4{e[0], e[1], 0u, 0u}), bneg, sc);
        dp = mfma_32x32x16(__builtin_bit_cast(bf16x8, u32x4{e[2], e[3], 0u, 0u}), bneg, dp);
      }
    };
    // Weights and score gradients of half qt, then dQ (and dZ) += their
    // products with the staged tokens.
    auto finish = [&](int qt, const f32x16& sc, const f32x16& dp) {
      f32x16 pw, ds;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (ENC) {
          const int row = 32 * qt + 8 * (i >> 2) + 4 * h + (i & 3);
          const float l2 = (!RAGGED || row < rem) ? l2m : INFINITY;
          pw[i] = exp2_fast(sc[i] * cs - l2);
          ds[i] = pw[i] * dp[i];
        } else {
          pw[i] = exp2_fast(sc[i] * cs);
          ds[i] = pw[i] * dp[i];
        }
      }
#pragma unroll
      for (int ug = 0; ug < 2; ++ug) {
        // B operands K[token slot][d = c] (and X) by transposing reads, as the
        // encoder reads V; with D = 16 the padding columns c >= 16 read valid
        // addresses and are zeroed
        bf16x8 kb, xb;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int row = 32 * qt + 16 * ug + 8 * half + 4 * h + (i16 >> 2);
          const int col = (D == 32 ? 16 * (c >> 4) : 0) + 4 * (i16 & 3);
          const int off = 8 * lat_chunk_pos<D>(row, col >> 3) + (col & 7);
          const bf16x4 k4 = __builtin_bit_cast(
              bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)((lds_void_t*)(kt + off))));
#pragma unroll
          for (int j = 0; j < 4; ++j) kb[4 * half + j] = k4[j];
          if constexpr (!ENC) {
            const bf16x4 x4 = __builtin_bit_cast(
                bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)((lds_void_t*)(xt + off))));
#pragma unroll
            for (int j = 0; j < 4; ++j) xb[4 * half + j] = x4[j];
          }
        }
        if constexpr (D == 16) {
          const uint32_t keep = c < 16 ? 0xffffffffu : 0u;
          const u32x4 kbits = __builtin_bit_cast(u32x4, kb);
          kb = __builtin_bit_cast(bf16x8, u32x4{kbits[0] & keep, kbits[1] & keep, kbits[2] & keep, kbits[3] & keep});
          if constexpr (!ENC) {
            const u32x4 xbits = __builtin_bit_cast(u32x4, xb);
            xb = __builtin_bit_cast(bf16x8, u32x4{xbits[0] & keep, xbits[1] & keep, xbits[2] & keep, xbits[3] & keep});
          }
        }
        dq = mfma_32x32x16(pack8_16(ds, ug), kb, dq);
        if constexpr (!ENC) dz = mfma_32x32x16(pack8_16(pw, ug), xb, dz);
      }
    };
    f32x16 sc0, dp0, sc1, dp1;
    products(0, sc0, dp0);
    if constexpr (ENC) {
      finish(0, sc0, dp0);
      products(1, sc1, dp1);
    } else {
      // the second half's products run under the first half's exponentials
      products(1, sc1, dp1);
      finish(0, sc0, dp0);
    }
    finish(1, sc1, dp1);
  };

  constexpr int UNITS = T * D / 8;  // 16-byte chunks per tensor and tile
  const int64_t tiles = (p.N + T - 1) / T;
  if constexpr (ENC) {
    // Token tiles t = s, s + S, ... of this split, staged through registers:
    // the next tile's loads are in flight while the current one is computed.
    constexpr int UPT = (UNITS + 64 * NW - 1) / (64 * NW);  // per thread
    bf16x8 kv[UPT], xv[UPT];
    auto fetch = [&](int64_t t) {
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        const int u = tid + q * 64 * NW;
        const int tok = u / (D / 8), dc = u % (D / 8);
        const int64_t n = t * T + tok;
        if (u < UNITS && n < p.N) {
          kv[q] = *reinterpret_cast<const bf16x8*>(kbase + n * p.k.sl + 8 * dc);
          xv[q] = *reinterpret_cast<const bf16x8*>(xbase + n * p.x.sl + 8 * dc);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) kv[q][j] = xv[q][j] = zero;
        }
      }
    };
    if (s < tiles) fetch(s);
    for (int64_t t = s; t < tiles; t += p.S) {
      __syncthreads();  // every wave is done with the previous tile
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        const int u = tid + q * 64 * NW;
        if (u < UNITS) {
          const int pos = lat_chunk_pos<D>(u / (D / 8), u % (D / 8));
          reinterpret_cast<bf16x8*>(kt_s)[pos] = kv[q];
          reinterpret_cast<bf16x8*>(xt_s)[pos] = xv[q];
        }
      }
      __syncthreads();
      if (t + p.S < tiles) fetch(t + p.S);
      const int rem = (int)min((int64_t)T, p.N - t * T);
      if (rem < T)
        tile(std::integral_constant<bool, true>(), rem);
      else
        tile(std::integral_constant<bool, false>(), rem);
    }
  } else {
    // Decode role: two tile buffers and one barrier per tile.  The next
    // tile's loads are in flight while the current one is computed; each
    // wave then prepares its share and writes it into the other buffer as it
    // finishes, while the other waves still compute.  The 2 UNITS units of a
    // tile are spread over all threads: units below UNITS take a dY chunk
    // (with its Y chunk when delta is computed here) and, for the token's
    // first chunk, its delta; the rest take a K chunk and the token's
    // normaliser.  Per token the two terms sit in the two halves of its
    // 16-byte slot: L / c in bf16 0..2, delta in bf16 4..6.
    constexpr int UPT = (2 * UNITS + 64 * NW - 1) / (64 * NW);
    bf16x8 cv[UPT], yv[UPT];
    float sv[UPT];
    const bool self_delta = p.y.data != nullptr;
    const bf16* ybase = self_delta ? reinterpret_cast<const bf16*>(p.y.data) + b * p.y.sb + hd * p.y.sh : nullptr;
    auto fetch = [&](int64_t t) {
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        // the side is uniform in the wave (UNITS is a multiple of 64)
        const int w2 = wave * 64 + q * 64 * NW;
        const bool xs = w2 < UNITS;
        const int u = tid + q * 64 * NW - (xs ? 0 : UNITS);
        const int tok = u / (D / 8), dc = u % (D / 8);
        const int64_t n = t * T + tok;
        const bool valid = w2 < 2 * UNITS && n < p.N;
        const bf16* sbase = xs ? xbase : kbase;
        const int64_t sl = xs ? p.x.sl : p.k.sl;
        if (valid) {
          cv[q] = *reinterpret_cast<const bf16x8*>(sbase + n * sl + 8 * dc);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) cv[q][j] = zero;
        }
        if (xs && self_delta) {
          if (valid) {
            yv[q] = *reinterpret_cast<const bf16x8*>(ybase + n * p.y.sl + 8 * dc);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) yv[q][j] = zero;
          }
        }
        sv[q] = 0.f;
        if (!xs || !self_delta) {
          const float* sp = xs ? p.delta : p.lse;
          if (valid && dc == 0) sv[q] = sp[(int64_t)bh * p.N + n];
        }
      }
    };
    auto stage = [&](int64_t t, int buf) {
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        const int w2 = wave * 64 + q * 64 * NW;
        if (w2 >= 2 * UNITS) continue;
        const bool xs = w2 < UNITS;
        const int u = tid + q * 64 * NW - (xs ? 0 : UNITS);
        const int tok = u / (D / 8), dc = u % (D / 8);
        const int64_t n = t * T + tok;
        const bool valid = n < p.N;
        float v = sv[q];
        if (xs && self_delta) {
          // delta_n = dY_n . Y_n: the D / 8 chunks of a token sit in
          // adjacent lanes of one wave
          float a0 = 0.f, a1 = 0.f;
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            a0 = fmaf((float)cv[q][j], (float)yv[q][j], a0);
            a1 = fmaf((float)cv[q][j + 1], (float)yv[q][j + 1], a1);
          }
          v = a0 + a1;
          v += shfl_xor_f(v, 1);
          if constexpr (D == 32) v += shfl_xor_f(v, 2);
          if (dc == 0 && valid && p.delta_out && blockIdx.z == 0) p.delta_out[(int64_t)bh * p.N + n] = v;
        }
        if (!xs) v = valid ? v * kLog2e / p.c : pad_offset(p.c);  // tokens past the end: weight 0
        const int pos = lat_chunk_pos<D>(tok, dc);
        reinterpret_cast<bf16x8*>((xs ? xt_s : kt_s) + buf * T * D)[pos] = cv[q];
        if (dc == 0) {
          bf16x8 e = {};
          split3_bf16(v, e, 0);
          const u32x4 eb = __builtin_bit_cast(u32x4, e);
          reinterpret_cast<u32x2*>(aug_s + buf * (T + 1) + tok)[xs ? 1 : 0] = u32x2{eb[0], eb[1]};
        }
      }
    };
    if (tid == 0) aug_s[T] = aug_s[2 * T + 1] = bf16x8{};  // zero slots for the lanes of the second K half
    if (s < tiles) {
      fetch(s);
      stage(s, 0);
    }
    __syncthreads();
    int cur = 0;
    for (int64_t t = s; t < tiles; t += p.S) {
      const bool more = t + p.S < tiles;
      if (more) fetch(t + p.S);
      kt = kt_s + cur * T * D;
      xt = xt_s + cur * T * D;
      augt = aug_s + cur * (T + 1);
      tile(std::integral_constant<bool, false>(), T);
      if (more) stage(t + p.S, cur ^ 1);
      // this wave's LDS writes have landed; the loads stay in flight
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
      barrier_keep_loads();
      cur ^= 1;
    }
  }

  // Partials of this split: accumulator row i of lane (h, c) is latent
  // lat0 + wave*32 + 8(i/4) + 4h + i%4, feature c.
  float* dqp = p.dq_part + ((int64_t)bh * p.S + s) * p.M * D;
  float* dzp = ENC ? nullptr : p.dz_part + ((int64_t)bh * p.S + s) * p.M * D;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = lat0 + wave * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (m < p.M && c < D) {
      dqp[(int64_t)m * D + c] = dq[i];
      if constexpr (!ENC) dzp[(int64_t)m * D + c] = dz[i];
    }
  }
}

// out[r, e] = (accumulate ? out[r, e] : 0) + factor * sum_{b < nb} sum_s part[r, b, s, e],
// with part[r, b, s, e] at (r S + s) MD + b bstride + e: one (batch, head)
// row per r when nb = 1, or for a query block shared by the batch one head
// per r with the batch summed (nb = B, bstride = H S MD).  A workgroup covers
// 256 consecutive e of one r, four per thread with 16-byte loads (MD is a
// multiple of 16), in four split groups: each thread takes every fourth
// split, loading eight of them before adding any.  The groups are combined
// through LDS.
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                         int S, int64_t MD, int nb, int64_t bstride, float factor,
                                                         int accumulate) {
  __shared__ f32x4 red[4][64];
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int64_t r = blockIdx.y;
  const int64_t e = ((int64_t)blockIdx.x * 64 + lane) * 4;
  const int64_t step = MD / 4;  // f32x4 per split
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (e < MD) {
    for (int bi = 0; bi < nb; ++bi) {
      const f32x4* ps = reinterpret_cast<const f32x4*>(part + r * S * MD + bi * bstride + e);
      for (int s0 = grp; s0 < S; s0 += 32) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int s = s0 + 4 * j;
          v[j] = s < S ? ps[(int64_t)s * step] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += v[j];
      }
    }
  }
  red[grp][lane] = acc;
  __syncthreads();
  if (grp == 0 && e < MD) {
    const f32x4 sum = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    float* o = out + r * MD + e;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (accumulate ? o[i] : 0.f) + factor * sum[i];
  }
}

// ---------------------------------------------------------------- launchers

static size_t tok_bwd_lds(int M, int D, bool enc, bool dz_split) {
  const int MC = (M + 31) / 32;
  size_t bytes = (size_t)MC * (D / 16) * 64 * 16 * 2 + (size_t)MC * 2 * 64 * 16;
  if (enc) bytes += (size_t)MC * 2 * 64 * 16 + (size_t)(MC * 32 + 1) * 16;
  if (enc && dz_split) bytes += (size_t)MC * (D / 16) * 64 * 16;
  return bytes;
}

template <typename K>
static hipError_t allow_lds_bwd(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_tok_bwd(const TokBwdParams& p, int D, int B, bool encode_role, hipStream_t st) {
  dim3 grid((unsigned)p.blocks_per_head, B * p.H);
  // The encode role stages four latent blocks (five with few latents): it
  // runs per block of 256 latents, later blocks adding into dK and dV.
  const int step = encode_role ? 256 : p.M;
  hipError_t e = hipSuccess;
  for (int m0 = 0; m0 < p.M; m0 += step) {
    TokBwdParams q = p;
    q.m0 = m0;
    q.mb = std::min(step, p.M - m0);
    q.accumulate = m0 > 0 ? 1 : p.accumulate;
    q.accumulate_v = m0 > 0 ? 1 : 0;
    const size_t lds = tok_bwd_lds(q.mb, D, encode_role, p.M < kDzSplitBelowM);
#define FLARE_TOK(DD, EE, SS)                                                              \
  if ((e = allow_lds_bwd(tok_bwd_kernel<DD, EE, SS>, lds)) != hipSuccess) return e;          \
  hipLaunchKernelGGL((tok_bwd_kernel<DD, EE, SS>), grid, dim3(64 * tok_bwd_waves<EE>()), lds, st, q)
    const bool split = p.M < kDzSplitBelowM;
    if (D == 32) {
      if (!encode_role) { FLARE_TOK(32, false, false); } else if (split) { FLARE_TOK(32, true, true); } else { FLARE_TOK(32, true, false); }
    } else {
      if (!encode_role) { FLARE_TOK(16, false, false); } else if (split) { FLARE_TOK(16, true, true); } else { FLARE_TOK(16, true, false); }
    }
#undef FLARE_TOK
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return e;
}

static size_t tok_pair_lds(int M, int D) {
  const int MC = (M + 31) / 32;
  return (size_t)MC * (D / 16) * 64 * 16 * (M < kDzSplitBelowM ? 4 : 3) + (size_t)MC * 2 * 64 * 16 * 2 +
         (size_t)(MC * 32 + 1) * 16;
}

hipError_t launch_tok_pair(const TokPairParams& p, int D, int B, hipStream_t st) {
  if (p.M > kTokPairMaxM) return hipErrorInvalidValue;
  dim3 grid((unsigned)p.blocks_per_head, B * p.H);
  const size_t lds = tok_pair_lds(p.M, D);
  hipError_t e;
#define FLARE_PAIR(DD, SS)                                                                  \
  if ((e = allow_lds_bwd(tok_pair_kernel<DD, SS>, lds)) != hipSuccess) return e;              \
  hipLaunchKernelGGL((tok_pair_kernel<DD, SS>), grid, dim3(64 * kTokPairWaves), lds, st, p)
  const bool split = p.M < kDzSplitBelowM;
  if (D == 32) {
    if (split) { FLARE_PAIR(32, true); } else { FLARE_PAIR(32, false); }
  } else {
    if (split) { FLARE_PAIR(16, true); } else { FLARE_PAIR(16, false); }
  }
#undef FLARE_PAIR
  return hipGetLastError();
}

hipError_t launch_lat_bwd(const LatBwdParams& p, int D, int B, bool encode_role, hipStream_t st) {
  const int NW = p.M <= 64 ? 2 : (encode_role || p.M <= 128) ? 4 : 8;
  const int lat_blocks = (p.M + 32 * NW - 1) / (32 * NW);
  dim3 grid(p.S, B * p.H, lat_blocks);
#define FLARE_LAT(DD, EE, WW) hipLaunchKernelGGL((lat_bwd_kernel<DD, EE, WW>), grid, dim3(64 * WW), 0, st, p)
#define FLARE_LAT_W(DD, EE) \
  if (NW == 2) FLARE_LAT(DD, EE, 2); else if (NW == 4) FLARE_LAT(DD, EE, 4); else FLARE_LAT(DD, EE, 8)
  // with fewer than kDzSplitBelowM latents the encode role takes dZ in two
  // parts (and 2-wave workgroups)
  const bool split = encode_role && p.M < kDzSplitBelowM;
  if (D == 32) {
    if (split) { hipLaunchKernelGGL((lat_bwd_kernel<32, true, 2, true>), grid, dim3(128), 0, st, p); }
    else if (encode_role) { FLARE_LAT_W(32, true); } else { FLARE_LAT_W(32, false); }
  } else {
    if (split) { hipLaunchKernelGGL((lat_bwd_kernel<16, true, 2, true>), grid, dim3(128), 0, st, p); }
    else if (encode_role) { FLARE_LAT_W(16, true); } else { FLARE_LAT_W(16, false); }
  }
#undef FLARE_LAT_W
#undef FLARE_LAT
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, float* out, int B, int H, int S, int64_t MD, bool batch_sum,
                             float factor, int accumulate, hipStream_t st) {
  const int64_t rows = batch_sum ? H : (int64_t)B * H;
  const int nb = batch_sum ? B : 1;
  const int64_t bstride = (int64_t)H * S * MD;
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((MD + 255) / 256), (unsigned)rows), dim3(256), 0, st, part,
                     out, S, MD, nb, bstride, factor, accumulate);
  return hipGetLastError();
}

}  // namespace flare
