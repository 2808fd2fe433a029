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
// (tok_bwd_kernel); sums over tokens (dQ, dZ) run latent-parallel over token
// splits in the encoder's layout (lat_bwd_kernel), with fp32 partials per
// split added by sum_splits_kernel.  The operand layouts are those of the
// forward kernels: see encode.hip and decode.hip.
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
//                        contiguous features of its token; skipped when null.
template <int D>
__device__ void stage_latent_block(const View& v, int b, int hd, int M, int MC, bf16x8* a_lds, bf16x8* at_lds,
                                   int tid, int nt) {
  constexpr int SD = D / 16;
  for (int u = tid; u < MC * SD * 64; u += nt) {
    const int ch = u / (SD * 64), sd = (u >> 6) % SD, ln = u & 63, hh = ln >> 5, cc = ln & 31;
    const int m = 32 * ch + cc;
    float vv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = 0.f;
    if (m < M) load_as_f32<8>(v.data, v.is_f32, b * v.sb + hd * v.sh + (int64_t)m * v.sl + 16 * sd + 8 * hh, vv);
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (bf16)vv[j];
    a_lds[(ch * SD + sd) * 64 + ln] = o;
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

// ------------------------------------------------------- token-parallel pass
constexpr int kTokBwdWaves = 4;

template <int D, bool ENC>
__global__ __launch_bounds__(64 * kTokBwdWaves) void tok_bwd_kernel(TokBwdParams p) {
  constexpr int NW = kTokBwdWaves;
  constexpr int SD = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.y, b = bh / p.H, hd = bh - b * p.H;
  const int MC = (p.M + 31) / 32;
  bf16x8* q_lds = reinterpret_cast<bf16x8*>(smem);
  bf16x8* w_lds = q_lds + MC * SD * 64;
  bf16x8* qt_lds = w_lds + MC * SD * 64;
  bf16x8* wt_lds = qt_lds + MC * 2 * 64;                                    // encode role
  float* l2_lds = reinterpret_cast<float*>(wt_lds + (ENC ? MC * 2 * 64 : 0));  // encode role
  float* dl_lds = l2_lds + MC * 32;                                          // encode role

  stage_latent_block<D>(p.q, b, hd, p.M, MC, q_lds, qt_lds, tid, 64 * NW);
  stage_latent_block<D>(p.w, b, hd, p.M, MC, w_lds, ENC ? wt_lds : nullptr, tid, 64 * NW);
  if constexpr (ENC) {
    // per latent: base-2 normaliser (+inf pads the last chunk: weight 0) and
    // delta_m = dZ_m . Z_m
    for (int m = tid; m < MC * 32; m += 64 * NW) {
      float l2 = INFINITY, dl = 0.f;
      if (m < p.M) {
        l2 = p.lse[(int64_t)bh * p.M + m] * kLog2e;
        for (int d = 0; d < D; ++d) {
          float a, z;
          load_as_f32<1>(p.w.data, p.w.is_f32, b * p.w.sb + hd * p.w.sh + (int64_t)m * p.w.sl + d, &a);
          load_as_f32<1>(p.z.data, p.z.is_f32, b * p.z.sb + hd * p.z.sh + (int64_t)m * p.z.sl + d, &z);
          dl = fmaf(a, z, dl);
        }
      }
      l2_lds[m] = l2;
      dl_lds[m] = dl;
    }
  }
  __syncthreads();

  const bf16* kbase = reinterpret_cast<const bf16*>(p.k.data) + b * p.k.sb + hd * p.k.sh;
  const bf16* xbase = reinterpret_cast<const bf16*>(p.x.data) + b * p.x.sb + hd * p.x.sh;
  const float cs = p.c;
  const int64_t stride = (int64_t)gridDim.x * NW * 32;
  for (int64_t base = ((int64_t)blockIdx.x * NW + wave) * 32; base < p.N; base += stride) {
    const int64_t n = base + c;
    const bool valid = n < p.N;
    // B operands: token n, features 16sd + 8h .. +7 of K and of X
    bf16x8 kb[SD], xb[SD];
#pragma unroll
    for (int sd = 0; sd < SD; ++sd) {
      if (valid) {
        kb[sd] = *reinterpret_cast<const bf16x8*>(kbase + n * p.k.sl + 16 * sd + 8 * h);
        xb[sd] = *reinterpret_cast<const bf16x8*>(xbase + n * p.x.sl + 16 * sd + 8 * h);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) kb[sd][j] = xb[sd][j] = (bf16)0.0f;
      }
    }
    float l2n = 0.f, dln = 0.f;
    if constexpr (!ENC) {
      // delta_n = dY_n . Y_n over the token's D features (half per lane half)
      const bf16* ybase = reinterpret_cast<const bf16*>(p.y.data) + b * p.y.sb + hd * p.y.sh;
      float part = 0.f;
      if (valid) {
#pragma unroll
        for (int sd = 0; sd < SD; ++sd) {
          const bf16x8 yv = *reinterpret_cast<const bf16x8*>(ybase + n * p.y.sl + 16 * sd + 8 * h);
#pragma unroll
          for (int j = 0; j < 8; ++j) part = fmaf((float)xb[sd][j], (float)yv[j], part);
        }
        l2n = p.lse[(int64_t)bh * p.N + n] * kLog2e;
      }
      dln = part + shfl_xor_f(part, 32);
      if (h == 0 && valid) p.delta[(int64_t)bh * p.N + n] = dln;
    }

    f32x16 dk = zero16(), dv = zero16();
    for (int ch = 0; ch < MC; ++ch) {
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) {
        sc = mfma_32x32x16(q_lds[(ch * SD + sd) * 64 + lane], kb[sd], sc);
        dp = mfma_32x32x16(w_lds[(ch * SD + sd) * 64 + lane], xb[sd], dp);
      }
      // element i: latent 32ch + 8(i/4) + 4h + i%4 of token n
      f32x16 pw, ds;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float l2v[4], dlv[4];
        if constexpr (ENC) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(l2_lds + 32 * ch + 8 * q4 + 4 * h);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dl_lds + 32 * ch + 8 * q4 + 4 * h);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            l2v[j] = a[j];
            dlv[j] = d4[j];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            l2v[j] = l2n;
            dlv[j] = dln;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * q4 + j;
          pw[i] = exp2_fast(sc[i] * cs - l2v[j]);
          ds[i] = pw[i] * (dp[i] - dlv[j]);
        }
      }
#pragma unroll
      for (int ug = 0; ug < 2; ++ug) {
        dk = mfma_32x32x16(qt_lds[(ch * 2 + ug) * 64 + lane], pack8_16(ds, ug), dk);
        if constexpr (ENC) dv = mfma_32x32x16(wt_lds[(ch * 2 + ug) * 64 + lane], pack8_16(pw, ug), dv);
      }
    }
    // lane (h, c): token n, features 16h .. 16h + 15
    if (valid && 16 * h < D) {
      float* kp = p.dk + b * p.dk_sb + hd * p.dk_sh + n * p.dk_sl + 16 * h;
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        f32x4 v = {dk[j] * p.scale, dk[j + 1] * p.scale, dk[j + 2] * p.scale, dk[j + 3] * p.scale};
        if (p.accumulate) v += *reinterpret_cast<const f32x4*>(kp + j);
        *reinterpret_cast<f32x4*>(kp + j) = v;
      }
      if constexpr (ENC) {
        float* vp = p.dv + b * p.dv_sb + hd * p.dv_sh + n * p.dv_sl + 16 * h;
#pragma unroll
        for (int j = 0; j < 16; j += 4)
          *reinterpret_cast<f32x4*>(vp + j) = f32x4{dv[j], dv[j + 1], dv[j + 2], dv[j + 3]};
      }
    }
  }
}

// ------------------------------------------------------ latent-parallel pass
constexpr int kLatBwdTile = 64;  // tokens per LDS tile

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

template <int D, bool ENC, int NW>
__global__ __launch_bounds__(64 * NW) void lat_bwd_kernel(LatBwdParams p) {
  constexpr int SD = D / 16;
  constexpr int T = kLatBwdTile;
  __shared__ __attribute__((aligned(16))) bf16 kt[T * D];
  __shared__ __attribute__((aligned(16))) bf16 xt[T * D];
  __shared__ __attribute__((aligned(16))) float l2t[T];
  __shared__ __attribute__((aligned(16))) float dlt[T];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31, i16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x, bh = blockIdx.y, b = bh / p.H, hd = bh - b * p.H;
  const int lat0 = blockIdx.z * 32 * NW;
  const int m_lane = lat0 + wave * 32 + c;

  // B operands of the two products against this lane's latent: Q and W
  bf16x8 qop[SD], wop[SD];
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
        for (int j = 0; j < 8; ++j) dpart = fmaf(wv[j], zv[j], dpart);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qop[sd][j] = (bf16)qv[j];
      wop[sd][j] = (bf16)wv[j];
    }
  }
  // encode role: this lane's latent's base-2 normaliser and delta_m = dZ . Z
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
  const int64_t tiles = (p.N + T - 1) / T;
  for (int64_t t = s; t < tiles; t += p.S) {
    const int64_t t0 = t * T;
    __syncthreads();
    for (int u = tid; u < T * D / 8; u += 64 * NW) {
      const int tok = u / (D / 8), dc = u % (D / 8);
      const int64_t n = t0 + tok;
      bf16x8 kv, xv;
      if (n < p.N) {
        kv = *reinterpret_cast<const bf16x8*>(kbase + n * p.k.sl + 8 * dc);
        xv = *reinterpret_cast<const bf16x8*>(xbase + n * p.x.sl + 8 * dc);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) kv[j] = xv[j] = zero;
      }
      reinterpret_cast<bf16x8*>(kt)[u] = kv;
      reinterpret_cast<bf16x8*>(xt)[u] = xv;
    }
    if constexpr (!ENC) {
      for (int u = tid; u < T; u += 64 * NW) {
        const int64_t n = t0 + u;
        l2t[u] = n < p.N ? p.lse[(int64_t)bh * p.N + n] * kLog2e : INFINITY;
        dlt[u] = n < p.N ? p.delta[(int64_t)bh * p.N + n] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int qt = 0; qt < T / 32; ++qt) {
      // S^T and dP^T: element i is token 32qt + 8(i/4) + 4h + i%4 of latent c
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + (32 * qt + c) * D + 16 * sd + 8 * h);
        const bf16x8 xa = *reinterpret_cast<const bf16x8*>(xt + (32 * qt + c) * D + 16 * sd + 8 * h);
        sc = mfma_32x32x16(ka, qop[sd], sc);
        dp = mfma_32x32x16(xa, wop[sd], dp);
      }
      f32x16 pw, ds;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int row = 32 * qt + 8 * q4 + 4 * h;
        float l2v[4], dlv[4];
        if constexpr (ENC) {
          const int rem = (int)min((int64_t)T, p.N - t0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            l2v[j] = row + j < rem ? l2m : INFINITY;
            dlv[j] = dlm;
          }
        } else {
          const f32x4 a = *reinterpret_cast<const f32x4*>(l2t + row);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlt + row);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            l2v[j] = a[j];
            dlv[j] = d4[j];
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * q4 + j;
          pw[i] = exp2_fast(sc[i] * cs - l2v[j]);
          ds[i] = pw[i] * (dp[i] - dlv[j]);
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
          const bf16x4 k4 = __builtin_bit_cast(
              bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)((lds_void_t*)(kt + row * D + col))));
#pragma unroll
          for (int j = 0; j < 4; ++j) kb[4 * half + j] = k4[j];
          if constexpr (!ENC) {
            const bf16x4 x4 = __builtin_bit_cast(
                bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)((lds_void_t*)(xt + row * D + col))));
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
// 64 consecutive e of one r with four split groups (each thread takes every
// fourth split, coalesced across the 64 lanes), combined through LDS.
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                         int S, int64_t MD, int nb, int64_t bstride, float factor,
                                                         int accumulate) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int64_t r = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * 64 + lane;
  float acc = 0.f;
  if (e < MD) {
    for (int bi = 0; bi < nb; ++bi) {
      const float* ps = part + r * S * MD + bi * bstride + e;
      for (int s = grp; s < S; s += 4) acc += ps[(int64_t)s * MD];
    }
  }
  red[grp][lane] = acc;
  __syncthreads();
  if (grp == 0 && e < MD) {
    const float sum = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    const int64_t idx = r * MD + e;
    out[idx] = (accumulate ? out[idx] : 0.f) + factor * sum;
  }
}

// ---------------------------------------------------------------- launchers

int plan_bwd_splits(int B, int H, int M, int64_t N) {
  const int64_t bh = (int64_t)B * H * ((M + 255) / 256);
  const int64_t tiles = (N + kLatBwdTile - 1) / kLatBwdTile;
  int64_t S = (1024 + bh - 1) / bh;
  if (S > tiles) S = tiles;
  if (S < 1) S = 1;
  return (int)S;
}

static size_t tok_bwd_lds(int M, int D, bool enc) {
  const int MC = (M + 31) / 32;
  size_t bytes = (size_t)MC * (D / 16) * 64 * 16 * 2 + (size_t)MC * 2 * 64 * 16;
  if (enc) bytes += (size_t)MC * 2 * 64 * 16 + (size_t)MC * 32 * 4 * 2;
  return bytes;
}

template <typename K>
static hipError_t allow_lds_bwd(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_tok_bwd(const TokBwdParams& p, int D, int B, bool encode_role, hipStream_t st) {
  dim3 grid((unsigned)p.blocks_per_head, B * p.H);
  const size_t lds = tok_bwd_lds(p.M, D, encode_role);
  hipError_t e;
#define FLARE_TOK(DD, EE)                                                                  \
  if ((e = allow_lds_bwd(tok_bwd_kernel<DD, EE>, lds)) != hipSuccess) return e;              \
  hipLaunchKernelGGL((tok_bwd_kernel<DD, EE>), grid, dim3(64 * kTokBwdWaves), lds, st, p)
  if (D == 32) {
    if (encode_role) { FLARE_TOK(32, true); } else { FLARE_TOK(32, false); }
  } else {
    if (encode_role) { FLARE_TOK(16, true); } else { FLARE_TOK(16, false); }
  }
#undef FLARE_TOK
  return hipGetLastError();
}

hipError_t launch_lat_bwd(const LatBwdParams& p, int D, int B, bool encode_role, hipStream_t st) {
  const int lat_blocks = (p.M + 255) / 256;
  const int NW = p.M <= 64 ? 2 : p.M <= 128 ? 4 : 8;
  dim3 grid(p.S, B * p.H, lat_blocks);
#define FLARE_LAT(DD, EE, WW) hipLaunchKernelGGL((lat_bwd_kernel<DD, EE, WW>), grid, dim3(64 * WW), 0, st, p)
#define FLARE_LAT_W(DD, EE) \
  if (NW == 2) FLARE_LAT(DD, EE, 2); else if (NW == 4) FLARE_LAT(DD, EE, 4); else FLARE_LAT(DD, EE, 8)
  if (D == 32) {
    if (encode_role) { FLARE_LAT_W(32, true); } else { FLARE_LAT_W(32, false); }
  } else {
    if (encode_role) { FLARE_LAT_W(16, true); } else { FLARE_LAT_W(16, false); }
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
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((MD + 63) / 64), (unsigned)rows), dim3(256), 0, st, part,
                     out, S, MD, nb, bstride, factor, accumulate);
  return hipGetLastError();
}

}  // namespace flare
