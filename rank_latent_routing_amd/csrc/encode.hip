// Split-token FLARE encoder for gfx950: the instantiations of the kernel in
// encode_kernel.hpp for narrow workgroups (M up to 128) and 16-feature heads,
// the fp32 path, the merge of the split results and the launchers.  The
// 8-wave, 32-feature instantiation lives in encode_wide.hip.
#include "encode_kernel.hpp"

namespace flare {

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
// of split encoders; an empty split has L_s = -inf and weight 0).  A
// workgroup of 256 threads covers 4R consecutive latent features of one
// batch*head, R = 256 / G: thread (g, r) takes the four features 4r .. 4r + 3
// of the block (one latent, since D is a multiple of 4), folds the splits
// g, g + G, ... with an online logsumexp, and for G > 1 the G partial results
// are combined through LDS.  Each split's part of a block is 16R contiguous
// bytes read with 16-byte loads; G grows with the number of splits (up to 8)
// so that each thread folds about eight of them, loaded together.
constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p) {
  __shared__ float sm_m[kMergeThreads], sm_l[kMergeThreads];
  __shared__ f32x4 sm_a[kMergeThreads];
  const int G = p.G, R = kMergeThreads / G;
  const int tid = threadIdx.x, g = tid / R, r = tid - g * R;
  const int bh = blockIdx.y;
  const int64_t MD = (int64_t)p.M * p.D;
  const int64_t e = ((int64_t)blockIdx.x * R + r) * 4;  // first of the thread's four features
  const bool valid = e < MD;
  const int m = valid ? (int)(e / p.D) : 0;
  const int d = valid ? (int)(e - (int64_t)m * p.D) : 0;
  float mx = -INFINITY, sum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const float* pl = p.part_l + (int64_t)bh * p.S * p.M + m;
    const f32x4* po = reinterpret_cast<const f32x4*>(p.part_o + (int64_t)bh * p.S * MD + e);
    const int64_t ostep = MD / 4;  // f32x4 per split
    // eight splits' values are loaded before any is folded, so their loads
    // are in flight together
    for (int s0 = g; s0 < p.S; s0 += 8 * G) {
      float lsv[8];
      f32x4 osv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = s0 + j * G;
        lsv[j] = s < p.S ? pl[(int64_t)s * p.M] : -INFINITY;
        osv[j] = s < p.S ? po[(int64_t)s * ostep] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ls = lsv[j];
        if (ls == -INFINITY) continue;
        if (ls > mx) {
          const float a = exp2f(mx - ls);
          sum *= a;
          acc *= a;
          mx = ls;
        }
        const float w = exp2f(ls - mx);
        sum += w;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, osv[j][i], acc[i]);
      }
    }
  }
  float M_ = mx, L = sum;
  f32x4 A = acc;
  if (G > 1) {
    sm_m[tid] = mx;
    sm_l[tid] = sum;
    sm_a[tid] = acc;
    __syncthreads();
    if (g != 0) return;
    M_ = -INFINITY;
    for (int q = 0; q < G; ++q) M_ = fmaxf(M_, sm_m[q * R + r]);
    L = 0.f;
    A = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M_ != -INFINITY)
      for (int q = 0; q < G; ++q) {
        const float w = exp2f(sm_m[q * R + r] - M_);
        L += w * sm_l[q * R + r];
        const f32x4 a = sm_a[q * R + r];
#pragma unroll
        for (int i = 0; i < 4; ++i) A[i] += w * a[i];
      }
  }
  if (!valid) return;
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t off = b * p.z_sb + h * p.z_sh + (int64_t)m * p.z_sl + d;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (p.z_f32)
      reinterpret_cast<float*>(p.z)[off + i] = A[i] * inv;
    else
      reinterpret_cast<bf16*>(p.z)[off + i] = (bf16)(A[i] * inv);
  }
  if (p.lse && d == 0) p.lse[(int64_t)bh * p.M + m] = L > 0.f ? (M_ + log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_encode_bf16(const EncodeParams& p, int D, int B, int waves, int lat_blocks, hipStream_t st) {
  dim3 grid(p.S, B * p.H, lat_blocks);
#define FLARE_ENC(DD, NW) \
  hipLaunchKernelGGL((encode_bf16_kernel<DD, NW>), grid, dim3(64 * NW), 0, st, p)
  if (D == 32) {
    if (waves == 2) FLARE_ENC(32, 2);
    else if (waves == 4) FLARE_ENC(32, 4);
    else return launch_encode_bf16_wide(p, grid, st);
  } else {
    if (waves == 2) FLARE_ENC(16, 2);
    else if (waves == 4) FLARE_ENC(16, 4);
    else FLARE_ENC(16, 8);
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
  MergeParams q = p;
  q.G = 1;
  while (q.G < 8 && q.G * 8 < q.S) q.G *= 2;
  const int64_t features = 4 * (kMergeThreads / q.G);  // per workgroup
  dim3 grid((unsigned)(((int64_t)q.M * q.D + features - 1) / features), B * q.H);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeThreads), 0, st, q);
  return hipGetLastError();
}

}  // namespace flare
