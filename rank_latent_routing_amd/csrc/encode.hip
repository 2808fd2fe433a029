// Split-token FLARE encoder for gfx950, and the exact merge of its splits.
//
// Z_h = SDPA(Q_h, K_h, V_h) = softmax over tokens of (scale Q_h K_h^T) V_h
// ("FLARE++: Low-Rank Attention with Dynamic Attention Routing", section 3,
// "FLARE: fixed-query latent routing", equation 5).  The FLARE++ query
// synthesis (equation 8) is the same call with learned seeds as Q.
//
// The N tokens of each (batch, head) are cut into S contiguous splits.  One
// workgroup owns one split and all latents of its head (64 per wave): it
// streams 64-token K/V tiles from HBM into LDS (double buffered, one barrier
// per tile) and every wave multiplies them against its latents on bf16
// matrix cores, 32 tokens at a time.  Per split it writes the normalised
// partial output and the split's log-normaliser; the merge kernel combines
// the splits exactly by logsumexp, the reduction the pages give for
// token-sharded encoders ("Multi-GPU context parallelism").
//
// On gfx950 matrix-core and vector work largely add up rather than overlap,
// so the per-score instruction count is what the design minimises:
//   scores   s = K Q^T on v_mfma_f32_16x16x32_bf16 (bf16 Q, fp32 accumulate),
//   weights  p = exp2(s * scale*log2 e): one v_mul, one v_exp_f32,
//   packing  two weights per v_cvt_pk_bf16_f32 (the A operand of P V),
//   row sums v_dot2c_f32_bf16 of the packed weights against (1, 1), i.e. the
//            normaliser sums exactly the rounded weights the numerator uses.
// The first pass runs without a running maximum (weights relative to 2^0);
// a split is accepted when every latent's normaliser lies in [2^-100, 2^100]
// and its output is finite, which rules out overflow and underflow, and the
// weights are then the max-shifted ones up to rounding.  Otherwise the
// workgroup reruns the split with the exact running-maximum online softmax
// (always used with FLARE_FLAG_EXACT_SOFTMAX).
#include "common.hpp"
#include "launch.hpp"

namespace flare {

constexpr int kEncT = 128;  // tokens per LDS tile (four 32-token quarters)

template <int D, int NW, int NB_>
struct EncodeKernel {
  using Op = QkOp<D>;
  using op_t = typename Op::type;
  static constexpr int PL = Op::per_lane;
  static constexpr int NT = 64 * NW;
  static constexpr int KROW = D + 8;  // padded LDS row: conflict-free operand reads
  static constexpr int DB = D / 16;   // 16-wide column blocks of D
  static constexpr int NB = NB_;      // 16-latent blocks per wave
  static constexpr int NQ = kEncT / 32;                  // 32-token quarters per tile
  static constexpr int K_UNITS = kEncT * D / 8;          // 16-byte chunks of a K tile
  static constexpr int V_UNITS = (kEncT / 4) * (D / 2);  // (token quad, d pair) of a V tile
  static constexpr int K_PER = (K_UNITS + NT - 1) / NT;
  static constexpr int V_PER = (V_UNITS + NT - 1) / NT;
  static constexpr int K_ELEMS = kEncT * KROW;
  static constexpr int V_ELEMS = NQ * DB * 64 * 8;
};

// V staging unit u -> (token quad q4 of the tile, column pair dp, which of the
// pair's two rows is written first).  The destination bank of a V write
// depends only on (column r = d % 16, half = which 4 of the lane's 8 tokens),
// so the mapping spreads every wave's 64 lanes over all 32 (r, half) slots,
// twice: a 2-way access, the minimum for 512 bytes.
template <int D>
__device__ __forceinline__ void v_unit(int u, int& q4, int& dp, int& par) {
  if constexpr (D == 32) {
    dp = u & 15;
    const int j = (u >> 4) & 3, w = u >> 6;
    const int half = j & 1, c = ((w >> 2) << 1) | (j >> 1), gg = w & 3;
    q4 = c * 8 + half * 4 + gg;
    par = dp >> 3;
  } else {
    dp = u & 7;
    const int b3 = (u >> 3) & 1, half = (u >> 4) & 1, b5 = (u >> 5) & 1, c = u >> 6;
    const int gg = b3 | (b5 << 1);
    q4 = c * 8 + half * 4 + gg;
    par = b3;
  }
}

template <int D, int NW, int NB_, bool EXACT>
__device__ __forceinline__ void encode_pass(
    const EncodeParams& p, const bf16* __restrict__ kbase, const bf16* __restrict__ vbase,
    int64_t n_begin, int64_t n_end, int ntiles, bf16* k_lds, bf16* v_lds,
    const typename QkOp<D>::type (&qop)[NB_], f32x4 (&o)[NB_][D / 16], float (&lsum)[NB_],
    float (&mrun)[NB_]) {
  using KC = EncodeKernel<D, NW, NB_>;
  using op_t = typename KC::op_t;
  constexpr int PL = KC::PL, NT = KC::NT, KROW = KC::KROW, DB = KC::DB, NB = KC::NB, NQ = KC::NQ;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const float cs = p.c;

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int e = 0; e < DB; ++e) o[nb][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    lsum[nb] = 0.f;
    mrun[nb] = -INFINITY;
  }

  struct Stage {
    u32x4 k[KC::K_PER];
    uint32_t v[KC::V_PER][4];
  };
  Stage sa, sb;

  auto load_tile = [&](Stage& st, int it) {
    u32x4 (&kreg)[KC::K_PER] = st.k;
    uint32_t (&vreg)[KC::V_PER][4] = st.v;
    const int64_t t0 = n_begin + (int64_t)it * kEncT;
#pragma unroll
    for (int ui = 0; ui < KC::K_PER; ++ui) {
      const int u = tid + ui * NT;
      kreg[ui] = u32x4{0u, 0u, 0u, 0u};
      if (u < KC::K_UNITS) {
        const int n = u / (D / 8), dc = u % (D / 8);
        const int64_t tok = t0 + n;
        if (tok < n_end) kreg[ui] = *reinterpret_cast<const u32x4*>(kbase + tok * p.k.sl + dc * 8);
      }
    }
#pragma unroll
    for (int ui = 0; ui < KC::V_PER; ++ui) {
      const int u = tid + ui * NT;
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[ui][i] = 0u;
      if (u < KC::V_UNITS) {
        int q4, dp, par;
        v_unit<D>(u, q4, dp, par);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t tok = t0 + 4 * q4 + i;
          if (tok < n_end) vreg[ui][i] = *reinterpret_cast<const uint32_t*>(vbase + tok * p.v.sl + 2 * dp);
        }
      }
    }
  };

  // K tile: plain rows [token][d] (padded).  V tile: the B operand of the
  // P V product, transposed so that lane (g, r) of quarter c and column block
  // e finds its 8 tokens contiguous: j < 4 -> token 32c + 4g + j,
  // j >= 4 -> token 32c + 16 + 4g + (j - 4), column d = 16e + r.
  auto store_tile = [&](const Stage& st, int buf) {
    const u32x4 (&kreg)[KC::K_PER] = st.k;
    const uint32_t (&vreg)[KC::V_PER][4] = st.v;
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
        int q4, dp, par;
        v_unit<D>(u, q4, dp, par);
        const uint32_t* w = vreg[ui];
        // the four tokens' even-d halves, and their odd-d halves, paired
        const u32x2 even = {__builtin_amdgcn_perm(w[1], w[0], 0x05040100u),
                            __builtin_amdgcn_perm(w[3], w[2], 0x05040100u)};
        const u32x2 odd = {__builtin_amdgcn_perm(w[1], w[0], 0x07060302u),
                           __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)};
        const int c = q4 >> 3, qq = q4 & 7, gg = qq & 3, half = qq >> 2;
        const int d0 = 2 * dp, e0 = d0 >> 4, rr0 = d0 & 15;
        const int off0 = ((c * DB + e0) * 64 + 16 * gg + rr0) * 8 + half * 4;
        if (par) {
          *reinterpret_cast<u32x2*>(vt + off0 + 8) = odd;
          *reinterpret_cast<u32x2*>(vt + off0) = even;
        } else {
          *reinterpret_cast<u32x2*>(vt + off0) = even;
          *reinterpret_cast<u32x2*>(vt + off0 + 8) = odd;
        }
      }
    }
  };

  // 32 tokens (quarter c of the tile) against the wave's 64 latents.  The
  // RAGGED variant (only the last tile of a split) gives the tokens past the
  // end weight 0.
  auto compute_quarter = [&](auto ragged_tag, const bf16* kt, const bf16* vt, int64_t t0, int c) {
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    // S^T tiles: lane (g, r) of (tt, nb) holds token 32c + 16tt + 4g + i
    // against latent 16nb + r (raw dot products).
    f32x4 s[2][NB];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const op_t ka = *reinterpret_cast<const op_t*>(kt + (32 * c + 16 * tt + r) * KROW + g * PL);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[tt][nb] = KC::Op::mma(ka, qop[nb], f32x4{0.f, 0.f, 0.f, 0.f});
    }
    if constexpr (EXACT) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool valid = !RAGGED || t0 + 32 * c + 16 * tt + 4 * g + i < n_end;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s[tt][nb][i] = valid ? s[tt][nb][i] * cs : -INFINITY;
        }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = fmaxf(fmaxf(fmaxf(s[0][nb][0], s[0][nb][1]), fmaxf(s[0][nb][2], s[0][nb][3])),
                         fmaxf(fmaxf(s[1][nb][0], s[1][nb][1]), fmaxf(s[1][nb][2], s[1][nb][3])));
        mx = fmaxf(mx, shfl_xor_f(mx, 16));
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        const float mnew = fmaxf(mrun[nb], mx);
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = exp2_fast(mrun[nb] - mref);
        mrun[nb] = mnew;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[tt][nb][i] = exp2_fast(s[tt][nb][i] - mref);
        lsum[nb] *= alpha;
        // accumulator row 4g + i is latent 16nb + 4g + i, whose factor sits in
        // lane r = 4g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
          for (int e = 0; e < DB; ++e) o[nb][e][i] *= ai;
        }
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[tt][nb][i] = exp2_fast(s[tt][nb][i] * cs);
      if constexpr (RAGGED) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool valid = t0 + 32 * c + 16 * tt + 4 * g + i < n_end;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s[tt][nb][i] = valid ? s[tt][nb][i] : 0.f;
          }
      }
    }
    bf16x8 vb[DB];
#pragma unroll
    for (int e = 0; e < DB; ++e) vb[e] = *reinterpret_cast<const bf16x8*>(vt + ((c * DB + e) * 64 + lane) * 8);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 pa = pack8(s[0][nb], s[1][nb]);
      lsum[nb] = rowsum_bf16x8(pa, lsum[nb]);
#pragma unroll
      for (int e = 0; e < DB; ++e) o[nb][e] = mfma_16x16x32(pa, vb[e], o[nb][e]);
    }
  };

  auto compute_tile = [&](int it) {
    const int buf = it & 1;
    const bf16* kt = k_lds + buf * KC::K_ELEMS;
    const bf16* vt = v_lds + buf * KC::V_ELEMS;
    const int64_t t0 = n_begin + (int64_t)it * kEncT;
    if (t0 + kEncT <= n_end) {
#pragma unroll 1
      for (int c = 0; c < NQ; ++c) compute_quarter(std::integral_constant<bool, false>(), kt, vt, t0, c);
    } else {
#pragma unroll 1
      for (int c = 0; c < NQ; ++c) compute_quarter(std::integral_constant<bool, true>(), kt, vt, t0, c);
    }
  };

  // Two-deep prefetch: while tile it is computed from LDS buffer it % 2, the
  // loads of tile it + 2 are in flight into one register set and tile it + 1
  // (loaded one tile earlier) is written from the other set into the free
  // buffer.  The loop is unrolled by two so both register sets are static.
  load_tile(sa, 0);
  if (ntiles > 1) load_tile(sb, 1);
  store_tile(sa, 0);
  __syncthreads();
  for (int it = 0; it < ntiles; it += 2) {
    // even tile: compute it, stream it + 2 into sa, write it + 1 from sb
    if (it + 2 < ntiles) load_tile(sa, it + 2);
    compute_tile(it);
    if (it + 1 < ntiles) store_tile(sb, 1);
    __syncthreads();
    if (it + 1 >= ntiles) break;
    // odd tile: compute it + 1, stream it + 3 into sb, write it + 2 from sa
    if (it + 3 < ntiles) load_tile(sb, it + 3);
    compute_tile(it + 1);
    if (it + 2 < ntiles) store_tile(sa, 0);
    __syncthreads();
  }
}

template <int D, int NW, int NB_>
__global__ __launch_bounds__(64 * NW, (NW >= 8 ? 4 : 3)) void encode_bf16_kernel(EncodeParams p) {
  using KC = EncodeKernel<D, NW, NB_>;
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
  // g*PL .. g*PL + PL - 1 of Q in bf16 (fp32 queries are rounded once).
  op_t qop[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int m = wave * 16 * NB + nb * 16 + r;
    float qv[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) qv[j] = 0.f;
    if (m < p.M) load_as_f32<PL>(p.q.data, p.q.is_f32, b * p.q.sb + h * p.q.sh + m * p.q.sl + g * PL, qv);
#pragma unroll
    for (int j = 0; j < PL; ++j) qop[nb][j] = (bf16)qv[j];
  }

  f32x4 o[NB][DB];
  float lsum[NB], mrun[NB];
  if (tid == 0) need_exact = p.exact;
  __syncthreads();
  bool exact = need_exact != 0;
  if (!exact) {
    encode_pass<D, NW, NB_, false>(p, kbase, vbase, n_begin, n_end, ntiles, k_lds, v_lds, qop, o, lsum, mrun);
    bool bad = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float l = lsum[nb];
      l += shfl_xor_f(l, 16);
      l += shfl_xor_f(l, 32);
      const bool ok_l = l >= kSafeLo && l <= kSafeHi;
      bool ok_o = true;
#pragma unroll
      for (int e = 0; e < DB; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) ok_o = ok_o && __builtin_isfinite(o[nb][e][i]);
      bad = bad || (wave * 16 * NB + nb * 16 + r < p.M && !ok_l) || (wave * 16 * NB + nb * 16 + 4 * g < p.M && !ok_o);
    }
    if (__any(bad) && lane == 0) need_exact = 1;
    __syncthreads();
    exact = need_exact != 0 && n_end > n_begin;
  }
  if (exact)
    encode_pass<D, NW, NB_, true>(p, kbase, vbase, n_begin, n_end, ntiles, k_lds, v_lds, qop, o, lsum, mrun);

  // Epilogue: normalised split output and log2-normaliser of every latent.
  float* po = p.part_o + ((int64_t)bh * p.S + s) * p.M * D;
  float* pl = p.part_l + ((int64_t)bh * p.S + s) * p.M;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l = lsum[nb];  // score layout: lane (g, r) holds latent 16nb + r
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    const float mr = exact ? mrun[nb] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(l, 4 * g + i, 64);  // output layout: row 4g + i
      const float mi = __shfl(mr, 4 * g + i, 64);
      const int m = wave * 16 * NB + nb * 16 + 4 * g + i;
      const float inv = li > 0.f ? 1.0f / li : 0.f;
      const float lse2 = li > 0.f ? __log2f(li) + (mi == -INFINITY ? 0.f : mi) : -INFINITY;
      if (m < p.M) {
#pragma unroll
        for (int e = 0; e < DB; ++e) po[(int64_t)m * D + 16 * e + r] = o[nb][e][i] * inv;
        if (r == 0) pl[m] = lse2;
      }
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
// of split encoders; an empty split has L_s = -inf and weight 0).  One
// workgroup per (batch*head, latent): 256 threads = G split groups x D
// features; every thread folds its splits with an online logsumexp, and the
// G partial results are combined through LDS.
constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p) {
  __shared__ float sm_m[kMergeThreads], sm_l[kMergeThreads], sm_a[kMergeThreads];
  const int bh = blockIdx.y, m = blockIdx.x, tid = threadIdx.x;
  const int G = kMergeThreads / p.D;  // split groups
  const int grp = tid / p.D, d = tid - grp * p.D;
  const float* pl = p.part_l + (int64_t)bh * p.S * p.M + m;
  const float* po = p.part_o + ((int64_t)bh * p.S * p.M + m) * p.D + d;
  float mx = -INFINITY, sum = 0.f, acc = 0.f;
  for (int s = grp; s < p.S; s += G) {
    const float ls = pl[(int64_t)s * p.M];
    const float os = po[(int64_t)s * p.M * p.D];
    if (ls == -INFINITY) continue;
    if (ls > mx) {
      const float a = exp2f(mx - ls);
      sum *= a;
      acc *= a;
      mx = ls;
    }
    const float w = exp2f(ls - mx);
    sum += w;
    acc = fmaf(w, os, acc);
  }
  sm_m[tid] = mx;
  sm_l[tid] = sum;
  sm_a[tid] = acc;
  __syncthreads();
  if (grp != 0) return;
  float M_ = -INFINITY;
  for (int q = 0; q < G; ++q) M_ = fmaxf(M_, sm_m[q * p.D + d]);
  float L = 0.f, A = 0.f;
  if (M_ != -INFINITY)
    for (int q = 0; q < G; ++q) {
      const float w = exp2f(sm_m[q * p.D + d] - M_);
      L += w * sm_l[q * p.D + d];
      A += w * sm_a[q * p.D + d];
    }
  const float z = L > 0.f ? A / L : 0.f;
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t off = b * p.z_sb + h * p.z_sh + (int64_t)m * p.z_sl + d;
  if (p.z_f32)
    reinterpret_cast<float*>(p.z)[off] = z;
  else
    reinterpret_cast<bf16*>(p.z)[off] = (bf16)z;
  if (p.lse && d == 0) p.lse[(int64_t)bh * p.M + m] = L > 0.f ? (M_ + log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- launchers

EncodePlan plan_encode(int B, int H, int M, int64_t N, int D, int is_f32) {
  (void)D;
  EncodePlan pl;
  const int64_t bh = (int64_t)B * H;
  // 32 latents per wave; all latents of a head in one workgroup.
  pl.waves = M <= 64 ? 2 : M <= 128 ? 4 : M <= 256 ? 8 : 16;
  pl.lat_blocks = 2;
  // About two workgroups per compute unit at a time, a few rounds in all; a
  // split holds at least 256 tokens (2 tiles) so per-split overheads stay small.
  const int64_t target = is_f32 ? 512 : 1024;
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

hipError_t launch_encode_bf16(const EncodeParams& p, int D, int B, int waves, int lat_blocks, hipStream_t st) {
  dim3 grid(p.S, B * p.H);
#define FLARE_ENC(DD, NW, NB) \
  hipLaunchKernelGGL((encode_bf16_kernel<DD, NW, NB>), grid, dim3(64 * NW), 0, st, p)
  (void)lat_blocks;
  if (D == 32) {
    if (waves == 2) FLARE_ENC(32, 2, 2);
    else if (waves == 4) FLARE_ENC(32, 4, 2);
    else if (waves == 8) FLARE_ENC(32, 8, 2);
    else FLARE_ENC(32, 16, 2);
  } else {
    if (waves == 2) FLARE_ENC(16, 2, 2);
    else if (waves == 4) FLARE_ENC(16, 4, 2);
    else if (waves == 8) FLARE_ENC(16, 8, 2);
    else FLARE_ENC(16, 16, 2);
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
  dim3 grid(p.M, B * p.H);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace flare
