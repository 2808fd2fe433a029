// Device-side types and helpers shared by the gfx950 kernels.
//
// Matrix-core layouts used throughout (CDNA3/CDNA4 MFMA, wave64):
//   v_mfma_f32_32x32x16_bf16  A: lane l holds A[l%32][8*(l/32) + j], j < 8
//                             B: lane l holds B[8*(l/32) + j][l%32]
//                             C/D: lane l holds C[8*(i/4) + 4*(l/32) + i%4][l%32], i < 16
//   v_mfma_f32_16x16x32_bf16  A: lane l holds A[l%16][8*(l/16) + j], j < 8
//                             B: lane l holds B[8*(l/16) + j][l%16]
//                             C/D: lane l holds C[4*(l/16) + i][l%16], i < 4
//   v_mfma_f32_16x16x16_bf16  same with 4 K-elements per lane: k = 4*(l/16) + j
// With 32x32 tiles we write h = l/32 and c = l%32; with 16x16 tiles g = l/16
// and r = l%16.  Only the (row, column) placement matters for correctness:
// both operands of a product always put the same reduction index in the same
// (lane group, element) slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flare {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Acceptance of a softmax normaliser l computed without the running maximum
// (weights 2^x relative to 2^0; see the encode and decode kernels).
//  - Upper end: l <= 2^100 keeps every weight and every sum of weights finite.
//  - Lower end: v_exp_f32 returns 0 for results below 2^-126, so each of the
//    n weights a normaliser sums may lose up to 2^-126 of mass, n 2^-126 in
//    all.  Requiring l >= n 2^-102 bounds that loss by 2^-24 l, below the
//    rounding of the fp32 sum itself, for any n.
constexpr float kSafeLoPerTerm = 1.9721522630525295e-31f;  // 2^-102
constexpr float kSafeHi = 1.2676506002282294e30f;          // 2^100

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                    __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Operand vector of a QK^T product: 8 bf16 for D = 32 (16x16x32), 4 for D = 16 (16x16x16).
template <int D> struct QkOp;
template <> struct QkOp<32> {
  typedef bf16x8 type;
  static constexpr int per_lane = 8;
  __device__ static __forceinline__ f32x4 mma(type a, type b, f32x4 c) { return mfma_16x16x32(a, b, c); }
};
template <> struct QkOp<16> {
  typedef bf16x4 type;
  static constexpr int per_lane = 4;
  __device__ static __forceinline__ f32x4 mma(type a, type b, f32x4 c) { return mfma_16x16x16(a, b, c); }
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + p.lo + p.hi for a dword holding two bf16 weights: v_dot2c_f32_bf16
// against the constant pair (1.0, 1.0), exact in fp32.  Written as inline asm
// (an ALU instruction, no memory access) because the ROCm 7.2 compiler picks
// the wrong source sub-register when __builtin_amdgcn_fdot2_f32_bf16 is fed
// pairs extracted from an 8-wide bf16 vector (every pair sums the first one).
__device__ __forceinline__ float dot2_ones(uint32_t pair, float acc) {
  asm("v_dot2c_f32_bf16 %0, 0x3f803f80, %1" : "+v"(acc) : "v"(pair));
  return acc;
}

// Sum of the 8 bf16 weights of a matrix-core operand, added to acc.
__device__ __forceinline__ float rowsum_bf16x8(bf16x8 p, float acc) {
  const u32x4 w = __builtin_bit_cast(u32x4, p);
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = dot2_ones(w[j], acc);
  return acc;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
  r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
  return r;
}

__device__ __forceinline__ bf16x8 pack8_16(const f32x16& v, int half) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)v[8 * half + j];
  return r;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Load n consecutive elements (bf16 or fp32) starting at element offset
// `off` of `base` and return them as floats.
template <int n>
__device__ __forceinline__ void load_as_f32(const void* base, int is_f32, int64_t off, float* out) {
  if (is_f32) {
    const float* p = reinterpret_cast<const float*>(base) + off;
#pragma unroll
    for (int j = 0; j < n; ++j) out[j] = p[j];
  } else {
    const bf16* p = reinterpret_cast<const bf16*>(base) + off;
#pragma unroll
    for (int j = 0; j < n; ++j) out[j] = (float)p[j];
  }
}

// Workgroup barrier that keeps global loads and LDS-DMA transfers in flight.
// __syncthreads() is a workgroup release/acquire fence around s_barrier, and
// on gfx9 that fence waits for every outstanding vector-memory operation
// (vmcnt(0)), which would drain a prefetch pipeline at every tile.  Here the
// caller first waits explicitly for exactly the transfers the other waves
// need (s_waitcnt vmcnt(n) lgkmcnt(0)); the empty asm statements only stop
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediates for gfx9: vmcnt(n) lgkmcnt(0) (expcnt left at 7).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

// Word 3 of a raw (stride 0) buffer descriptor on CDNA: 32-bit data format,
// no swizzle; reads past num_records return zero.
constexpr int kBufferFlags = 0x00020000;

// The exact combination of split encoders for four features of one latent
// ("FLARE++", section 3, "Multi-GPU context parallelism": partial results
// merge by their log-normalisers): with L_s the log2-normaliser of split s
// (at pl[s * lstride]; -inf for an empty split) and O_s its normalised output
// (at po[s * ostride]), returns sum_s 2^{L_s - L} O_s, L = log2 sum_s 2^{L_s},
// folded in split order with a running maximum.  Sixteen splits' values are
// loaded before any is folded (one memory round trip for up to 16 splits).
__device__ __forceinline__ f32x4 merge_splits4(const float* pl, int64_t lstride, const f32x4* po, int64_t ostride,
                                               int S) {
  constexpr int kBatch = 16;
  float mx = -INFINITY, sum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float lsv[kBatch];
    f32x4 osv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = s0 + j;
      lsv[j] = s < S ? pl[(int64_t)s * lstride] : -INFINITY;
      osv[j] = s < S ? po[(int64_t)s * ostride] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
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
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  return acc * inv;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace flare
