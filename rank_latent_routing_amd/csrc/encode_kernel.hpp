// The split-token FLARE encoder kernel for gfx950 (its splits are merged by
// merge_kernel in encode.hip).  Included by encode.hip (every instantiation
// but one) and encode_wide.hip (the 8-wave, 32-feature kernel of the
// large-latent workloads, built with its own instruction-scheduling
// strategy).
//
// Z_h = SDPA(Q_h, K_h, V_h) = softmax over tokens of (scale Q_h K_h^T) V_h
// ("FLARE++: Low-Rank Attention with Dynamic Attention Routing", section 3,
// "FLARE: fixed-query latent routing", equation 5).  The FLARE++ query
// synthesis (equation 8) is the same call with learned seeds as Q.
//
// The N tokens of each (batch, head) are cut into S contiguous splits.  One
// workgroup owns one split and all latents of its head, 32 per wave: it
// streams 128-token K/V tiles from HBM straight into LDS with
// global_load_lds_dwordx4 (four LDS stages, three tiles in flight, one barrier
// per tile, no registers or vector instructions spent on staging) and every
// wave multiplies them against its latents on bf16 matrix cores, 32 tokens at
// a time.  V stays token-major in LDS; the transposed B operand of P V comes
// from ds_read_b64_tr_b16.  Per split it writes the
// normalised partial output and the split's log-normaliser; the merge kernel
// combines the splits exactly by logsumexp, the reduction the pages give for
// token-sharded encoders ("Multi-GPU context parallelism").
//
// Per 32 tokens x 32 latents a wave runs four v_mfma_f32_32x32x16_bf16 (two
// for S^T = K Q^T, two for O += P V).  A lane's 16 scores all belong to its
// latent, so the softmax stays in the lane: one v_mul by scale*log2(e), one
// v_exp_f32, a v_cvt_pk_bf16_f32 per pair (which is directly the A operand of
// P V), and v_dot2c_f32_bf16 row sums of those packed weights (the
// normaliser sums exactly the rounded weights the numerator uses).  On gfx950
// that vector work (a v_exp_f32 alone takes 8 cycles of a SIMD) outlasts the
// four products, which run under it, so this per-score instruction count is
// what the design minimises.
//
// The first pass runs without a running maximum (weights relative to 2^0).
// A split of n tokens is accepted when every latent's normaliser l lies in
// [n 2^-102, 2^100] and its output is finite.  The upper end rules out
// overflow.  At the lower end, the weights the exponential flushes to zero
// (each below 2^-126) carry less than 2^-24 of l, so the result equals the
// max-shifted softmax up to fp32 rounding.  Otherwise the workgroup reruns
// the split with the exact running-maximum online softmax (always used with
// FLARE_FLAG_EXACT_SOFTMAX).
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace flare {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// LDS stages of K/V tiles: four (three tiles in flight) for 8-wave
// workgroups; two (one in flight) for the narrower workgroups of small M,
// whose splits are short and which need several workgroups per CU to hide
// the loads (four stages would hold them at one or two waves per SIMD).
constexpr int enc_stages(int nw) { return nw >= 8 ? 4 : 2; }
// Waves per SIMD the LDS of a workgroup allows (at most 4, the 128-register
// budget): the launch bound asks the compiler for exactly that.
constexpr int enc_waves_per_simd(int d, int nw) {
  const int lds = 2 * enc_stages(nw) * kEncT * d * 2 + 4;
  const int per_simd = (160 * 1024 / lds) * nw / 4;
  return per_simd < 1 ? 1 : per_simd > 4 ? 4 : per_simd;
}

template <int D, int NW>
struct EncodeKernel {
  static constexpr int NT = 64 * NW;
  static constexpr int SD = D / 16;                 // 16-wide d slices (K dim of S^T)
  static constexpr int NQ = kEncT / 32;             // 32-token quarters per tile
  static constexpr int ROWC = D / 8;                // 16-byte chunks per token row
  static constexpr int TILE_ELEMS = kEncT * D;      // bf16 elements of one K (or V) tile
  static constexpr int TILE_CHUNKS = kEncT * ROWC;  // 16-byte chunks of one tile
  // Each tile is brought in by TILE_CHUNKS / 64 wave-wide 16-byte DMA loads
  // for K and as many for V, spread evenly over the waves.
  static constexpr int OPS = 2 * TILE_CHUNKS / 64;
  static constexpr int OPS_PER_WAVE = (OPS + NW - 1) / NW;
  static_assert(OPS % NW == 0 || NW > OPS, "uneven DMA split");
};

// K tile chunk position of (token, 16-byte chunk dc): the chunk index is
// XOR-swizzled with bits 2..3 of the token so that the A-operand reads
// (lanes of a 16-lane group = 16 consecutive tokens, one chunk each) touch
// 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_chunk_pos(int token, int dc) {
  if constexpr (D == 32) return token * 4 + (dc ^ ((token >> 2) & 3));
  else return token * 2 + (dc ^ ((token >> 2) & 1));
}

template <int D, int NW, bool EXACT>
__device__ __forceinline__ void encode_pass(
    const EncodeParams& p, const bf16* __restrict__ kbase, const bf16* __restrict__ vbase,
    int64_t tile0, int64_t tstride, int64_t n_end, int ntiles, bf16* k0, bf16* k1, bf16* k2, bf16* k3,
    bf16* v0, bf16* v1, bf16* v2, bf16* v3, const bf16x8 (&qop)[D / 16], f32x16& o,
    float (&ls)[4], float& mrun) {
  using KC = EncodeKernel<D, NW>;
  constexpr int SD = KC::SD, NQ = KC::NQ, ROWC = KC::ROWC;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wave
  const int i16 = lane & 15;
  const float cs = p.c;

  o = zero16();
#pragma unroll
  for (int a = 0; a < 4; ++a) ls[a] = 0.f;
  mrun = -INFINITY;

  // DMA of tile it into stage S: wave-wide 16-byte buffer loads straight
  // into LDS, lane l of load t filling chunk (t * 64 + l) of the stage.  K
  // chunks are swizzled; V chunks stay in token-major order.  Which load a
  // wave issues, and so its source tensor, is uniform across the wave: the
  // buffer descriptor (tile base, valid byte range) lives in scalar registers
  // and each lane adds a loop-invariant 32-bit offset.  In the ragged last
  // tile, lanes past the end fall outside the descriptor's range and read
  // zeros (finite data whose weight is then set to 0).
  uint32_t op_off[KC::OPS_PER_WAVE];
#pragma unroll
  for (int q = 0; q < KC::OPS_PER_WAVE; ++q) {
    const int op = wave * KC::OPS_PER_WAVE + q;
    const bool is_v = op >= KC::OPS / 2;
    const int t = is_v ? op - KC::OPS / 2 : op;
    const int pos = t * 64 + lane;
    const int token = pos / ROWC, sw = pos % ROWC;
    const int dc = is_v ? sw : D == 32 ? (sw ^ ((token >> 2) & 3)) : (sw ^ ((token >> 2) & 1));
    op_off[q] = (uint32_t)((token * (is_v ? p.v.sl : p.k.sl) + dc * 8) * (int64_t)sizeof(bf16));
  }
  auto issue = [&](auto stage_tag, int it) {
    constexpr int S = decltype(stage_tag)::value;
    bf16* kd = S == 0 ? k0 : S == 1 ? k1 : S == 2 ? k2 : k3;
    bf16* vd = S == 0 ? v0 : S == 1 ? v1 : S == 2 ? v2 : v3;
    const int64_t t0 = (tile0 + (int64_t)it * tstride) * kEncT;
    const int64_t rows = min((int64_t)kEncT, n_end - t0);
#pragma unroll
    for (int q = 0; q < KC::OPS_PER_WAVE; ++q) {
      const int op = wave * KC::OPS_PER_WAVE + q;
      if (op < KC::OPS) {
        const bool is_v = op >= KC::OPS / 2;
        const int t = is_v ? op - KC::OPS / 2 : op;
        const int64_t sl = is_v ? p.v.sl : p.k.sl;
        const bf16* base = (is_v ? vbase : kbase) + t0 * sl;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16*>(base), (short)0, (int)(rows * sl * (int64_t)sizeof(bf16)), kBufferFlags);
        bf16* dst = (is_v ? vd : kd) + t * 512;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 16, op_off[q], 0, 0, 0);
      }
    }
  };

  // S^T for quarter qt (32 tokens) of a tile against the wave's 32 latents:
  // the K operands (LDS reads) and the two products.  Element i of the score
  // tile is token 32qt + 8(i/4) + 4h + i%4 of latent c.
  auto k_operands = [&](const bf16* kt, int qt, bf16x8 (&ka)[SD]) {
#pragma unroll
    for (int sd = 0; sd < SD; ++sd)
      ka[sd] = *reinterpret_cast<const bf16x8*>(kt + 8 * k_chunk_pos<D>(32 * qt + c, 2 * sd + h));
  };
  auto qk = [&](const bf16x8 (&ka)[SD]) {
    f32x16 sc = zero16();
#pragma unroll
    for (int sd = 0; sd < SD; ++sd) sc = mfma_32x32x16(ka[sd], qop[sd], sc);
    return sc;
  };

  // B operand V[token slot (h, j)][d = c] of the 16-token group ug of quarter
  // qt by two transposing reads: lane i of a 16-lane group points at row
  // 16ug + 8(j0/4) + 4h + i/4, features 16(c/16) + 4(i%4) .. +3, and receives
  // rows +0..+3 of feature c.
  auto v_operand = [&](const bf16* vt, int qt, int ug) {
    // With D = 16 the columns c >= 16 of the product are padding: those lanes
    // read the same (valid) addresses as lane c - 16 and zero the operand,
    // without a divergent branch.
    bf16x8 vb;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 32 * qt + 16 * ug + 8 * half + 4 * h + (i16 >> 2);
      const int col = (D == 32 ? 16 * (c >> 4) : 0) + 4 * (i16 & 3);
      const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)((lds_void_t*)(vt + row * D + col)));
      const bf16x4 b4 = __builtin_bit_cast(bf16x4, v4);
#pragma unroll
      for (int j = 0; j < 4; ++j) vb[4 * half + j] = b4[j];
    }
    if constexpr (D == 16) {
      const u32x4 bits = __builtin_bit_cast(u32x4, vb);
      const uint32_t keep = c < 16 ? 0xffffffffu : 0u;
      vb = __builtin_bit_cast(bf16x8, u32x4{bits[0] & keep, bits[1] & keep, bits[2] & keep, bits[3] & keep});
    }
    return vb;
  };

  // Weights of the scores sc of quarter qt, their row sums, and O += P V
  // with the V operands vb0, vb1.  The row sums go to four independent
  // accumulators (no serial chain of dependent dot products).  rem: tokens
  // of the tile before the end (only read for the ragged tile).
  auto softmax_pv = [&](auto ragged_tag, f32x16 sc, bf16x8 vb0, bf16x8 vb1, int rem, int qt) {
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    // token 32qt + 8(i/4) + 4h + i%4 is valid iff 8(i/4) + i%4 < rel
    const int rel = rem - 32 * qt - 4 * h;
    if constexpr (EXACT) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool valid = !RAGGED || 8 * (i >> 2) + (i & 3) < rel;
        sc[i] = valid ? sc[i] * cs : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float mnew = fmaxf(mrun, mx);
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2_fast(mrun - mref);
      mrun = mnew;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = exp2_fast(sc[i] - mref);
#pragma unroll
      for (int a = 0; a < 4; ++a) ls[a] *= alpha;
      // accumulator row i is latent 8(i/4) + 4h + i%4, whose factor sits in
      // the lanes of that latent
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] *= __shfl(alpha, 8 * (i >> 2) + 4 * h + (i & 3), 64);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = exp2_fast(sc[i] * cs);
      if constexpr (RAGGED) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + (i & 3) >= rel) sc[i] = 0.f;
      }
    }
#pragma unroll
    for (int ug = 0; ug < 2; ++ug) {
      const bf16x8 pa = pack8_16(sc, ug);
      const u32x4 w = __builtin_bit_cast(u32x4, pa);
#pragma unroll
      for (int a = 0; a < 4; ++a) ls[a] = dot2_ones(w[a], ls[a]);
      o = mfma_32x32x16(pa, ug == 0 ? vb0 : vb1, o);
    }
  };

  // One tile.  On the fast path its quarters are software-pipelined: the
  // S^T product of quarter qt + 1 is issued before the softmax of quarter
  // qt, so the matrix cores work while the same wave computes exponentials.
  // The exact fallback keeps one quarter in flight (fewer live registers).
  auto compute_tile = [&](auto stage_tag, int it) {
    constexpr int S = decltype(stage_tag)::value;
    const bf16* kt = S == 0 ? k0 : S == 1 ? k1 : S == 2 ? k2 : k3;
    const bf16* vt = S == 0 ? v0 : S == 1 ? v1 : S == 2 ? v2 : v3;
    const int64_t t0 = (tile0 + (int64_t)it * tstride) * kEncT;
    const int rem = (int)min((int64_t)kEncT, n_end - t0);
    auto run = [&](auto ragged_tag) {
      if constexpr (EXACT) {
#pragma unroll 1
        for (int qt = 0; qt < NQ; ++qt) {
          bf16x8 ka[SD];
          k_operands(kt, qt, ka);
          softmax_pv(ragged_tag, qk(ka), v_operand(vt, qt, 0), v_operand(vt, qt, 1), rem, qt);
        }
      } else {
        bf16x8 ka[SD];
        k_operands(kt, 0, ka);
        f32x16 sc = qk(ka);
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt) {
          f32x16 nx;
          if (qt + 1 < NQ) {
            k_operands(kt, qt + 1, ka);
            nx = qk(ka);
          }
          softmax_pv(ragged_tag, sc, v_operand(vt, qt, 0), v_operand(vt, qt, 1), rem, qt);
          if (qt + 1 < NQ) sc = nx;
        }
      }
    };
    if (rem == kEncT)
      run(std::integral_constant<bool, false>());
    else
      run(std::integral_constant<bool, true>());
  };

  constexpr int ST = enc_stages(NW);
  if constexpr (ST == 4) {
    // Tile it lives in stage it % 4.  Step it: start the DMA of tile it + 3,
    // compute tile it, then wait for this wave's DMA of tile it + 1 (the
    // loads of tiles it + 2 and it + 3 may still be outstanding) and meet at
    // the barrier, after which every wave's part of tile it + 1 is in LDS and
    // every wave is done reading tile it (whose stage the next step refills).
    auto step = [&](auto stage_tag, int it) {
      constexpr int S = decltype(stage_tag)::value;
      if (it + 3 < ntiles) issue(std::integral_constant<int, (S + 3) % 4>(), it + 3);
      compute_tile(stage_tag, it);
      const int later = (it + 3 < ntiles) + (it + 2 < ntiles);  // tiles issued after it + 1
      if (later == 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * KC::OPS_PER_WAVE));
      else if (later == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(KC::OPS_PER_WAVE));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      barrier_keep_loads();
    };

    issue(std::integral_constant<int, 0>(), 0);
    if (ntiles > 1) issue(std::integral_constant<int, 1>(), 1);
    if (ntiles > 2) issue(std::integral_constant<int, 2>(), 2);
    if (ntiles > 2)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * KC::OPS_PER_WAVE));
    else if (ntiles > 1)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(KC::OPS_PER_WAVE));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    barrier_keep_loads();
    for (int it = 0; it < ntiles; it += 4) {
      step(std::integral_constant<int, 0>(), it);
      if (it + 1 >= ntiles) break;
      step(std::integral_constant<int, 1>(), it + 1);
      if (it + 2 >= ntiles) break;
      step(std::integral_constant<int, 2>(), it + 2);
      if (it + 3 >= ntiles) break;
      step(std::integral_constant<int, 3>(), it + 3);
    }
  } else {
    // Two stages: tile it lives in stage it % 2.  Step it: start the DMA of
    // tile it + 1 into the other stage (every wave finished reading it, tile
    // it - 1, before the last barrier), compute tile it, wait for this
    // wave's DMA and meet at the barrier.
    auto step = [&](auto stage_tag, int it) {
      constexpr int S = decltype(stage_tag)::value;
      if (it + 1 < ntiles) issue(std::integral_constant<int, (S + 1) % 2>(), it + 1);
      compute_tile(stage_tag, it);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      barrier_keep_loads();
    };

    issue(std::integral_constant<int, 0>(), 0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    barrier_keep_loads();
    for (int it = 0; it < ntiles; it += 2) {
      step(std::integral_constant<int, 0>(), it);
      if (it + 1 >= ntiles) break;
      step(std::integral_constant<int, 1>(), it + 1);
    }
  }
}

template <int D, int NW>
// Eight waves (256 latents) run at four waves per SIMD, two workgroups per
// compute unit (128 VGPRs); narrower workgroups, with two LDS stages, fit
// several per compute unit at four waves per SIMD.
__global__ __launch_bounds__(64 * NW, enc_waves_per_simd(D, NW)) void encode_bf16_kernel(EncodeParams p) {
  using KC = EncodeKernel<D, NW>;
  constexpr int SD = KC::SD;
  constexpr int ST = enc_stages(NW);
  constexpr int HI = ST > 2 ? KC::TILE_ELEMS : 8;  // stages 2 and 3 (unused with two stages)
  // Separate arrays per stage, so that the compiler can tell a DMA into one
  // stage from reads of another and adds no waits between them.
  __shared__ __attribute__((aligned(16))) bf16 k0[KC::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 k1[KC::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 k2[HI];
  __shared__ __attribute__((aligned(16))) bf16 k3[HI];
  __shared__ __attribute__((aligned(16))) bf16 v0[KC::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 v1[KC::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 v2[HI];
  __shared__ __attribute__((aligned(16))) bf16 v3[HI];
  __shared__ int need_exact;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wave
  const int s = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, hd = bh - b * p.H;
  // Split s takes the tiles s, s + S, s + 2S, ... of its head: at any time
  // the workgroups of a head stream one contiguous window of K and V instead
  // of S scattered regions (the merge is exact for any assignment of tokens
  // to splits).
  const int64_t n_end = p.N;
  const int64_t tiles_all = (p.N + kEncT - 1) / kEncT;
  const int ntiles = tiles_all > s ? (int)((tiles_all - 1 - s) / p.S + 1) : 0;
  const bf16* kbase = reinterpret_cast<const bf16*>(p.k.data) + b * p.k.sb + hd * p.k.sh;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v.data) + b * p.v.sb + hd * p.v.sh;
  const int lat0 = blockIdx.z * 32 * NW;  // first latent of this workgroup
  const int m_lane = lat0 + wave * 32 + c;  // this lane's latent in the score tiles

  // B operands of S^T = K Q^T: lane (h, c) holds latent m_lane, features
  // 16 sd + 8h .. +7 of Q in bf16 (fp32 queries are rounded once).  The
  // scale multiplies the fp32 scores: folding it into bf16 Q would add a
  // rounding whose score error grows with the score.
  bf16x8 qop[SD];
#pragma unroll
  for (int sd = 0; sd < SD; ++sd) {
    float qv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[j] = 0.f;
    if (m_lane < p.M)
      load_as_f32<8>(p.q.data, p.q.is_f32, b * p.q.sb + hd * p.q.sh + m_lane * p.q.sl + 16 * sd + 8 * h, qv);
#pragma unroll
    for (int j = 0; j < 8; ++j) qop[sd][j] = (bf16)qv[j];
  }

  // Zero the stages once: a lane past the end of the tokens may leave its
  // chunk unwritten, and stale data must be finite (its weight is 0).
  {
    bf16* stages[8] = {k0, k1, v0, v1, k2, k3, v2, v3};
    const bf16x8 z8 = {};
#pragma unroll
    for (int st = 0; st < 2 * ST; ++st)
      for (int u = tid; u < KC::TILE_CHUNKS; u += KC::NT) reinterpret_cast<bf16x8*>(stages[st])[u] = z8;
  }
  f32x16 o;
  float ls[4], mrun;
  if (tid == 0) need_exact = p.exact;
  __syncthreads();
  bool exact = need_exact != 0;
  if (!exact) {
    encode_pass<D, NW, false>(p, kbase, vbase, s, p.S, n_end, ntiles, k0, k1, k2, k3, v0, v1, v2, v3, qop, o, ls, mrun);
    const float lp = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    float l = lp + shfl_xor_f(lp, 32);
    // the split sums at most ntiles * kEncT weights
    const float lo = (float)ntiles * (float)kEncT * kSafeLoPerTerm;
    bool ok = l >= lo && l <= kSafeHi;
#pragma unroll
    for (int i = 0; i < 16; ++i) ok = ok && __builtin_isfinite(o[i]);
    const bool bad = m_lane < p.M && !ok;
    if (__any(bad) && lane == 0) need_exact = 1;
    __syncthreads();
    exact = need_exact != 0 && ntiles > 0;
  }
  if (exact)
    encode_pass<D, NW, true>(p, kbase, vbase, s, p.S, n_end, ntiles, k0, k1, k2, k3, v0, v1, v2, v3, qop, o, ls, mrun);

  // Epilogue: normalised split output and log2-normaliser of every latent.
  // Accumulator row i of lane (h, c) is latent wave*32 + 8(i/4) + 4h + i%4,
  // feature c; the normaliser of latent r sits in lanes r and r + 32.
  float* po = p.part_o + ((int64_t)bh * p.S + s) * p.M * D;
  float* pl = p.part_l + ((int64_t)bh * p.S + s) * p.M;
  const float lp = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  const float l = lp + shfl_xor_f(lp, 32);
  const float mr = exact ? mrun : 0.f;
  if (h == 0 && m_lane < p.M)  // lanes 0..31 own the latent scalars
    pl[m_lane] = l > 0.f ? __log2f(l) + (mr == -INFINITY ? 0.f : mr) : -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + 4 * h + (i & 3);
    const float li = __shfl(l, r, 64);
    const int m = lat0 + wave * 32 + r;
    if (m < p.M && c < D) po[(int64_t)m * D + c] = li > 0.f ? o[i] / li : 0.f;
  }
}

}  // namespace flare
