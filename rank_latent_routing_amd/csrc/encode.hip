// Split-token FLARE encoder for gfx950, and the exact merge of its splits.
//
// Z_h = SDPA(Q_h, K_h, V_h) = softmax over tokens of (scale Q_h K_h^T) V_h
// ("FLARE++: Low-Rank Attention with Dynamic Attention Routing", section 3,
// "FLARE: fixed-query latent routing", equation 5).  The FLARE++ query
// synthesis (equation 8) is the same call with learned seeds as Q.
//
// The N tokens of each (batch, head) are cut into S contiguous splits.  One
// workgroup owns one split and every latent of its head: it streams 64-token
// K/V tiles from HBM into LDS (double buffered, one barrier per tile) and each
// wave multiplies them against its 64 latents on bf16 matrix cores.  Per split
// it emits the normalised partial output and the split's log-normaliser; the
// merge kernel combines splits exactly by logsumexp, the reduction the pages
// give for token-sharded encoders ("Multi-GPU context parallelism").
//
// Softmax: scores are formed directly in log2 units by splitting
// scale*log2(e)*Q into a bf16 hi + lo pair (two MFMAs, ~2^-17 relative), so
// p = exp2(x) needs no multiply.  The first pass runs without a running
// maximum (weights relative to 2^0); a split is accepted when every latent's
// normaliser lies in [2^-100, 2^100] and its output is finite, which rules
// out overflow and underflow, and the weights then equal the max-shifted ones
// up to rounding.  Otherwise the workgroup reruns the split with the exact
// running-maximum online softmax (always used with FLARE_FLAG_EXACT_SOFTMAX).
#include "common.hpp"
#include "launch.hpp"

namespace flare {

constexpr int kEncT = 64;  // tokens per tile

template <int D, int NW>
struct EncodeKernel {
  using Op = QkOp<D>;
  using op_t = typename Op::type;
  static constexpr int PL = Op::per_lane;
  static constexpr int NT = 64 * NW;
  static constexpr int KROW = D + 8;  // padded LDS row: conflict-free operand reads
  static constexpr int DB = D / 16;   // 16-wide column blocks of D
  static constexpr int NB = 4;        // 16-latent blocks per wave (64 latents)
  static constexpr int K_UNITS = kEncT * D / 8;          // 16-byte chunks of a K tile
  static constexpr int V_UNITS = (kEncT / 4) * (D / 2);  // (token quad, d pair) of a V tile
  static constexpr int K_PER = (K_UNITS + NT - 1) / NT;
  static constexpr int V_PER = (V_UNITS + NT - 1) / NT;
  static constexpr int K_ELEMS = kEncT * KROW;
  static constexpr int V_ELEMS = 2 * DB * 64 * 8;
};

template <int D, int NW, bool EXACT>
__device__ __forceinline__ void encode_pass(
    const EncodeParams& p, const bf16* __restrict__ kbase, const bf16* __restrict__ vbase,
    int64_t n_begin, int64_t n_end, int ntiles, bf16* k_lds, bf16* v_lds,
    const typename QkOp<D>::type (&qhi)[4], const typename QkOp<D>::type (&qlo)[4],
    f32x4 (&o)[4][D / 16], f32x4 (&o1)[4], float (&mrun)[4]) {
  using KC = EncodeKernel<D, NW>;
  using op_t = typename KC::op_t;
  constexpr int PL = KC::PL, NT = KC::NT, KROW = KC::KROW, DB = KC::DB, NB = KC::NB;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int e = 0; e < DB; ++e) o[nb][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    o1[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    mrun[nb] = -INFINITY;
  }

  u32x4 kreg[KC::K_PER];
  uint32_t vreg[KC::V_PER][4];

  auto load_tile = [&](int it) {
    const int64_t t0 = n_begin + (int64_t)it * kEncT;
#pragma unroll
    for (int ui = 0; ui < KC::K_PER; ++ui) {
      const int u = tid + ui * NT;
      kreg[ui] = u32x4{0u, 0u, 0u, 0u};
      if (u < KC::K_UNITS) {
        const int n = u / (D / 8), dc = u % (D / 8);
        const int64_t tok = t0 + n;
        if (tok < n_end)
          kreg[ui] = *reinterpret_cast<const u32x4*>(kbase + tok * p.k.sl + dc * 8);
      }
    }
#pragma unroll
    for (int ui = 0; ui < KC::V_PER; ++ui) {
      const int u = tid + ui * NT;
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[ui][i] = 0u;
      if (u < KC::V_UNITS) {
        const int q4 = u / (D / 2), dp = u % (D / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t tok = t0 + 4 * q4 + i;
          if (tok < n_end)
            vreg[ui][i] = *reinterpret_cast<const uint32_t*>(vbase + tok * p.v.sl + 2 * dp);
        }
      }
    }
  };

  // K tile: plain rows [token][d] (padded).  V tile: the B operand of the
  // P V product, transposed so that lane (g, r) of chunk c and column block e
  // finds its 8 tokens contiguous: j < 4 -> token 32c + 4g + j,
  // j >= 4 -> token 32c + 16 + 4g + (j - 4), column d = 16e + r.
  auto store_tile = [&](int buf) {
    bf16* kt = k_lds + buf * KC::K_ELEMS;
    bf16* vt = v_lds + buf * KC::V_ELEMS;
#pragma unroll
    for (int ui = 0; ui < KC::K_PER; ++ui) {
      const int u = tid + ui * NT;
      if (u < KC::K_UNITS) {
        const int n = u / (D / 8), dc = u % (D / 8);
        *reinterpret_cast<u32x4*>(kt + n * KROW + dc * 8) = kreg[ui];
      }
    }
#pragma unroll
    for (int ui = 0; ui < KC::V_PER; ++ui) {
      const int u = tid + ui * NT;
      if (u < KC::V_UNITS) {
        const int q4 = u / (D / 2), dp = u % (D / 2);
        const uint32_t* w = vreg[ui];
        // (token i, d even) halves and (token i, d odd) halves, paired by token
        const uint32_t lo01 = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
        const int c = q4 >> 3, qq = q4 & 7, gg = qq & 3, half = qq >> 2;
        const int d0 = 2 * dp, e0 = d0 >> 4, rr0 = d0 & 15;
        const int off0 = ((c * DB + e0) * 64 + 16 * gg + rr0) * 8 + half * 4;
        *reinterpret_cast<u32x2*>(vt + off0) = u32x2{lo01, lo23};
        *reinterpret_cast<u32x2*>(vt + off0 + 8) = u32x2{hi01, hi23};
      }
    }
  };

  const bf16 one = (bf16)1.0f, zero = (bf16)0.0f;

  auto compute_tile = [&](int buf, int it) {
    const bf16* kt = k_lds + buf * KC::K_ELEMS;
    const bf16* vt = v_lds + buf * KC::V_ELEMS;
    const int64_t t0 = n_begin + (int64_t)it * kEncT;
    const bool ragged = t0 + kEncT > n_end;

    // scores S^T[token][latent] in log2 units: lane (g, r) of tile (t, nb)
    // holds token 16t + 4g + i against latent 16nb + r
    f32x4 sc[4][NB];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const op_t ka = *reinterpret_cast<const op_t*>(kt + (16 * t + r) * KROW + g * PL);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
        a = KC::Op::mma(ka, qhi[nb], a);
        a = KC::Op::mma(ka, qlo[nb], a);
        sc[t][nb] = a;
      }
    }

    if constexpr (EXACT) {
      if (ragged) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + 16 * t + 4 * g + i >= n_end)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) sc[t][nb][i] = -INFINITY;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[t][nb][i]);
        mx = fmaxf(mx, shfl_xor_f(mx, 16));
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        const float mnew = fmaxf(mrun[nb], mx);
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = exp2_fast(mrun[nb] - mref);
        mrun[nb] = mnew;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[t][nb][i] = exp2_fast(sc[t][nb][i] - mref);
        // accumulator row 4g + i belongs to latent 16nb + 4g + i, whose
        // factor sits in lane r = 4g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
          for (int e = 0; e < DB; ++e) o[nb][e][i] *= ai;
          o1[nb][i] *= ai;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[t][nb][i] = exp2_fast(sc[t][nb][i]);
    }

    // O[latent][d] += P V and the normaliser via a ones column block;
    // padded tokens carry V = 0 and a 0 in the ones operand.
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 vb[DB];
#pragma unroll
      for (int e = 0; e < DB; ++e)
        vb[e] = *reinterpret_cast<const bf16x8*>(vt + ((c * DB + e) * 64 + lane) * 8);
      bf16x8 ones;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = 32 * c + (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
        ones[j] = (!ragged || t0 + n < n_end) ? one : zero;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 pa = pack8(sc[2 * c][nb], sc[2 * c + 1][nb]);
#pragma unroll
        for (int e = 0; e < DB; ++e) o[nb][e] = mfma_16x16x32(pa, vb[e], o[nb][e]);
        o1[nb] = mfma_16x16x32(pa, ones, o1[nb]);
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) load_tile(it + 1);
    compute_tile(it & 1, it);
    if (it + 1 < ntiles) store_tile((it + 1) & 1);
    __syncthreads();
  }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void encode_bf16_kernel(EncodeParams p) {
  using KC = EncodeKernel<D, NW>;
  using op_t = typename KC::op_t;
  constexpr int PL = KC::PL, DB = KC::DB, NB = KC::NB;
  __shared__ __attribute__((aligned(16))) bf16 k_lds[2 * KC::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 v_lds[2 * KC::V_ELEMS];
  __shared__ int need_exact;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int s = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t n_begin = (int64_t)s * p.tokens_per_split;
  const int64_t n_end = min(p.N, n_begin + p.tokens_per_split);
  const int ntiles = n_end > n_begin ? (int)((n_end - n_begin + kEncT - 1) / kEncT) : 0;
  const bf16* kbase = reinterpret_cast<const bf16*>(p.k.data) + b * p.k.sb + h * p.k.sh;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v.data) + b * p.v.sb + h * p.v.sh;

  // B operands of S^T = K Q^T: lane (g, r) holds latent 16nb + r, columns
  // g*PL .. g*PL+PL-1 of scale*log2(e)*Q as a bf16 hi/lo pair.
  op_t qhi[NB], qlo[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int m = wave * 64 + nb * 16 + r;
    float qv[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) qv[j] = 0.f;
    if (m < p.M) load_as_f32<PL>(p.q.data, p.q.is_f32, b * p.q.sb + h * p.q.sh + m * p.q.sl + g * PL, qv);
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      bf16 hi, lo;
      split_bf16(qv[j] * p.c, hi, lo);
      qhi[nb][j] = hi;
      qlo[nb][j] = lo;
    }
  }

  f32x4 o[NB][DB], o1[NB];
  float mrun[NB];
  if (tid == 0) need_exact = p.exact;
  __syncthreads();
  bool exact = need_exact != 0;
  if (!exact) {
    encode_pass<D, NW, false>(p, kbase, vbase, n_begin, n_end, ntiles, k_lds, v_lds, qhi, qlo, o, o1, mrun);
    bool bad = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wave * 64 + nb * 16 + 4 * g + i;
        const float l = o1[nb][i];
        bool ok = l >= kSafeLo && l <= kSafeHi;
#pragma unroll
        for (int e = 0; e < DB; ++e) ok = ok && __builtin_isfinite(o[nb][e][i]);
        bad = bad || (m < p.M && n_end > n_begin && !ok);
      }
    if (__any(bad) && lane == 0) need_exact = 1;
    __syncthreads();
    exact = need_exact != 0;
  }
  if (exact)
    encode_pass<D, NW, true>(p, kbase, vbase, n_begin, n_end, ntiles, k_lds, v_lds, qhi, qlo, o, o1, mrun);

  // Epilogue: normalised split output and log2-normaliser of every latent.
  float* po = p.part_o + ((int64_t)bh * p.S + s) * p.M * D;
  float* pl = p.part_l + ((int64_t)bh * p.S + s) * p.M;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mr_lane = exact ? mrun[nb] : 0.f;
      const float mref = __shfl(mr_lane, 4 * g + i, 64);
      const int m = wave * 64 + nb * 16 + 4 * g + i;
      const float l = o1[nb][i];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const float lse2 = l > 0.f ? __log2f(l) + (mref == -INFINITY ? 0.f : mref) : -INFINITY;
      if (m < p.M) {
#pragma unroll
        for (int e = 0; e < DB; ++e) po[(int64_t)m * D + 16 * e + r] = o[nb][e][i] * inv;
        if (r == 0) pl[m] = lse2;
      }
    }
}

// ---------------------------------------------------------------- fp32 path
// One thread per latent, exact running-maximum online softmax in fp32 over
// the split's tokens staged through LDS.
template <int D>
__global__ __launch_bounds__(256) void encode_f32_kernel(EncodeParams p) {
  __shared__ float k_t[kEncT * D];
  __shared__ float v_t[kEncT * D];
  const int tid = threadIdx.x;
  const int s = blockIdx.x, bh = blockIdx.y;
  const int m = blockIdx.z * 256 + tid;
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t n_begin = (int64_t)s * p.tokens_per_split;
  const int64_t n_end = min(p.N, n_begin + p.tokens_per_split);
  const float* kbase = reinterpret_cast<const float*>(p.k.data) + b * p.k.sb + h * p.k.sh;
  const float* vbase = reinterpret_cast<const float*>(p.v.data) + b * p.v.sb + h * p.v.sh;

  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = 0.f;
  if (m < p.M) load_as_f32<D>(p.q.data, p.q.is_f32, b * p.q.sb + h * p.q.sh + m * p.q.sl, q);
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] *= p.c;

  float mrun = -INFINITY, l = 0.f, acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;

  for (int64_t t0 = n_begin; t0 < n_end; t0 += kEncT) {
    const int cnt = (int)min((int64_t)kEncT, n_end - t0);
    __syncthreads();
    for (int u = tid; u < kEncT * D; u += 256) {
      const int n = u / D, d = u % D;
      k_t[u] = n < cnt ? kbase[(t0 + n) * p.k.sl + d] : 0.f;
      v_t[u] = n < cnt ? vbase[(t0 + n) * p.v.sl + d] : 0.f;
    }
    __syncthreads();
    for (int n = 0; n < cnt; ++n) {
      float x = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) x = fmaf(q[d], k_t[n * D + d], x);
      if (x > mrun) {
        const float alpha = exp2f(mrun - x);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
        mrun = x;
      }
      const float pw = exp2f(x - mrun);
      l += pw;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(pw, v_t[n * D + d], acc[d]);
    }
  }
  if (m < p.M) {
    float* po = p.part_o + (((int64_t)bh * p.S + s) * p.M + m) * D;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) po[d] = acc[d] * inv;
    p.part_l[((int64_t)bh * p.S + s) * p.M + m] = l > 0.f ? log2f(l) + mrun : -INFINITY;
  }
}

// ------------------------------------------------------------------- merge
// L = log2 sum_s 2^{L_s};  Z = sum_s 2^{L_s - L} O_s  (the exact combination
// of split encoders; an empty split has L_s = -inf and weight 0).
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int bh = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.M * p.D) return;
  const int m = idx / p.D, d = idx - m * p.D;
  const float* pl = p.part_l + (int64_t)bh * p.S * p.M + m;
  const float* po = p.part_o + (int64_t)bh * p.S * p.M * p.D + idx;
  float mx = -INFINITY;
  for (int s = 0; s < p.S; ++s) mx = fmaxf(mx, pl[(int64_t)s * p.M]);
  float sum = 0.f;
  if (mx != -INFINITY)
    for (int s = 0; s < p.S; ++s) sum += exp2f(pl[(int64_t)s * p.M] - mx);
  const float L = mx != -INFINITY ? mx + log2f(sum) : -INFINITY;
  float z = 0.f;
  if (mx != -INFINITY)
    for (int s = 0; s < p.S; ++s) {
      const float w = exp2f(pl[(int64_t)s * p.M] - L);
      z = fmaf(w, po[(int64_t)s * p.M * p.D], z);
    }
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t off = b * p.z_sb + h * p.z_sh + (int64_t)m * p.z_sl + d;
  if (p.z_f32)
    reinterpret_cast<float*>(p.z)[off] = z;
  else
    reinterpret_cast<bf16*>(p.z)[off] = (bf16)z;
  if (p.lse && d == 0) p.lse[(int64_t)bh * p.M + m] = L * kLn2;
}

// ---------------------------------------------------------------- launchers

EncodePlan plan_encode(int B, int H, int M, int64_t N, int D, int is_f32) {
  (void)D;
  EncodePlan pl;
  const int64_t bh = (int64_t)B * H;
  pl.waves = M <= 64 ? 1 : M <= 128 ? 2 : M <= 256 ? 4 : 8;
  // Fill the 256 compute units several times over; a split holds at least
  // 256 tokens (4 tiles) so per-split overheads stay small.
  const int64_t target = is_f32 ? 512 : (pl.waves == 8 ? 512 : 1024);
  int64_t S = (target + bh - 1) / bh;
  const int64_t max_s = (N + 255) / 256;
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  int64_t tps = (N + S - 1) / S;
  tps = (tps + kEncT - 1) / kEncT * kEncT;
  pl.tokens_per_split = tps;
  pl.S = (int)((N + tps - 1) / tps);
  return pl;
}

hipError_t launch_encode_bf16(const EncodeParams& p, int D, int B, int waves, hipStream_t st) {
  dim3 grid(p.S, B * p.H);
#define FLARE_ENC(DD, NW) \
  hipLaunchKernelGGL((encode_bf16_kernel<DD, NW>), grid, dim3(64 * NW), 0, st, p)
  if (D == 32) {
    switch (waves) {
      case 1: FLARE_ENC(32, 1); break;
      case 2: FLARE_ENC(32, 2); break;
      case 4: FLARE_ENC(32, 4); break;
      default: FLARE_ENC(32, 8); break;
    }
  } else {
    switch (waves) {
      case 1: FLARE_ENC(16, 1); break;
      case 2: FLARE_ENC(16, 2); break;
      case 4: FLARE_ENC(16, 4); break;
      default: FLARE_ENC(16, 8); break;
    }
  }
#undef FLARE_ENC
  return hipGetLastError();
}

hipError_t launch_encode_f32(const EncodeParams& p, int D, int B, hipStream_t st) {
  dim3 grid(p.S, B * p.H, (p.M + 255) / 256);
  if (D == 32)
    hipLaunchKernelGGL((encode_f32_kernel<32>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((encode_f32_kernel<16>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, int B, hipStream_t st) {
  dim3 grid((p.M * p.D + 255) / 256, B * p.H);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace flare
