// Issue-rate probes for gfx950: how many SIMD cycles the instructions of the
// encode/decode inner loops cost, alone and mixed with matrix-core products.
//
// Each probe runs a loop whose body is a fixed sequence of instructions on
// registers that depend only on themselves (every MFMA chain and every VALU
// register is independent of the others), so the loop measures issue and
// execution throughput, not latency.  The sequence is written as separate
// asm statements, which the compiler keeps in order.  No instruction reads the
// result of a matrix-core product except the same chain's next product, four
// products later.  Each wave reads the shader clock (s_memtime) before and
// after the loop; the loop's results are stored once at the end, one float per
// lane, so nothing is optimised away.
//
// Mixes (one loop iteration):
//   kMfma        8 x v_mfma_f32_32x32x16_bf16 (4 chains)
//   kMul         32 x v_mul_f32
//   kExp         32 x v_exp_f32
//   kCvt         16 x v_cvt_pk_bf16_f32
//   kDot2        16 x v_dot2c_f32_bf16
//   kMulExp      16 x (v_mul_f32, v_exp_f32) alternating
//   kMfmaMul<k>  8 x (1 MFMA, k x v_mul_f32)
//   kMfmaExp<k>  8 x (1 MFMA, k x v_exp_f32)
//   kBlock       one encoder block's work per wave: 4 MFMA, 16 mul, 16 exp,
//                8 cvt, 8 dot2, interleaved as a scheduler could
//   kBlockNoMul  the same without the 16 multiplies
//   kBlockNoDot  the same without the 8 row-sum dot2
//   kBlockDep    one block's work with the encoder's dependencies: each score
//                is multiplied, exponentiated, packed in pairs and summed
//   kAgpr        8 MFMAs with their accumulators in AGPRs
//   kAgprMul8    8 x (1 MFMA accumulating in AGPRs, 8 x v_mul_f32)
//   kAgprExp16   8 x (1 MFMA accumulating in AGPRs, 16 x v_exp_f32)
//   kMfma16      16 x v_mfma_f32_16x16x32_bf16 (same flops as kMfma)
//   kMfma16Mul8  8 x (2 x 16x16x32 MFMA, 8 x v_mul_f32)
//   kMfma16Exp16 8 x (2 x 16x16x32 MFMA, 16 x v_exp_f32)
//   kBlockAgpr   kBlock with the two weighted-sum products accumulating in AGPRs
//   kBlockHiLo   a block whose scale is folded into bf16 high and low query
//                parts: 6 MFMA (4 score products, 2 weighted sums), no multiply
//   kBlockHiLoAgpr  the same with the weighted sums in AGPRs
//   kBlockNoMulAgpr kBlockNoMul with the weighted sums in AGPRs
//   split roles: waves of one half run the first mix, the other half the second
#include <hip/hip_runtime.h>

#include <stdint.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum Mix {
  kMfma = 0,
  kMul = 1,
  kExp = 2,
  kCvt = 3,
  kDot2 = 4,
  kMulExp = 5,
  kMfmaMul4 = 6,
  kMfmaMul8 = 7,
  kMfmaMul16 = 8,
  kMfmaExp4 = 9,
  kMfmaExp8 = 10,
  kMfmaExp16 = 11,
  kBlock = 12,
  kBlockNoMul = 13,
  kBlockNoDot = 14,
  kBlockDep = 15,
  kIdle = 16,
  kAgprMul8 = 17,
  kAgprExp16 = 18,
  kMfma16 = 19,
  kMfma16Mul8 = 20,
  kMfma16Exp16 = 21,
  kBlockAgpr = 22,
  kBlockHiLo = 23,
  kBlockHiLoAgpr = 24,
  kBlockNoMulAgpr = 25,
  kAgpr = 26,
  kNumMix = 27
};

#define MFMA(acc) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
#define MFMA_A(acc) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b))
#define MFMA16(acc) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
#define VMUL(x) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(cm))
#define VEXP(x) asm volatile("v_exp_f32 %0, -%0" : "+v"(x))
#define VCVT(d, x, y) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "+v"(d) : "v"(x), "v"(y))
#define VDOT(s, d) asm volatile("v_dot2c_f32_bf16 %0, 0x3f803f80, %1" : "+v"(s) : "v"(d))

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Regs {
  f32x16 acc[4];
  f32x16 acca[4];  // only ever in AGPRs
  f32x4 acc4[8];
  float x[32];
  uint32_t pk[8];
  float s[8];
};

template <int MIX>
__device__ __forceinline__ void body(Regs& r, bf16x8 a, bf16x8 b, float cm) {
  if constexpr (MIX == kMfma) {
#pragma unroll
    for (int j = 0; j < 8; ++j) MFMA(r.acc[j & 3]);
  } else if constexpr (MIX == kMul) {
#pragma unroll
    for (int j = 0; j < 32; ++j) VMUL(r.x[j]);
  } else if constexpr (MIX == kExp) {
#pragma unroll
    for (int j = 0; j < 32; ++j) VEXP(r.x[j]);
  } else if constexpr (MIX == kCvt) {
#pragma unroll
    for (int j = 0; j < 16; ++j) VCVT(r.pk[j & 7], r.x[2 * j], r.x[2 * j + 1]);
  } else if constexpr (MIX == kDot2) {
#pragma unroll
    for (int j = 0; j < 16; ++j) VDOT(r.s[j & 7], r.pk[j & 7]);
  } else if constexpr (MIX == kMulExp) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      VMUL(r.x[j]);
      VEXP(r.x[16 + j]);
    }
  } else if constexpr (MIX >= kMfmaMul4 && MIX <= kMfmaMul16) {
    constexpr int K = MIX == kMfmaMul4 ? 4 : MIX == kMfmaMul8 ? 8 : 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      MFMA(r.acc[j & 3]);
#pragma unroll
      for (int i = 0; i < K; ++i) VMUL(r.x[(j * K + i) & 31]);
    }
  } else if constexpr (MIX >= kMfmaExp4 && MIX <= kMfmaExp16) {
    constexpr int K = MIX == kMfmaExp4 ? 4 : MIX == kMfmaExp8 ? 8 : 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      MFMA(r.acc[j & 3]);
#pragma unroll
      for (int i = 0; i < K; ++i) VEXP(r.x[(j * K + i) & 31]);
    }
  } else if constexpr (MIX == kAgpr) {
#pragma unroll
    for (int j = 0; j < 8; ++j) MFMA_A(r.acca[j & 3]);
  } else if constexpr (MIX == kAgprMul8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      MFMA_A(r.acca[j & 3]);
#pragma unroll
      for (int i = 0; i < 8; ++i) VMUL(r.x[(j * 8 + i) & 31]);
    }
  } else if constexpr (MIX == kAgprExp16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      MFMA_A(r.acca[j & 3]);
#pragma unroll
      for (int i = 0; i < 16; ++i) VEXP(r.x[(j * 16 + i) & 31]);
    }
  } else if constexpr (MIX == kMfma16) {
#pragma unroll
    for (int j = 0; j < 16; ++j) MFMA16(r.acc4[j & 7]);
  } else if constexpr (MIX == kMfma16Mul8 || MIX == kMfma16Exp16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      MFMA16(r.acc4[(2 * j) & 7]);
      MFMA16(r.acc4[(2 * j + 1) & 7]);
      if constexpr (MIX == kMfma16Mul8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) VMUL(r.x[(j * 8 + i) & 31]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) VEXP(r.x[(j * 16 + i) & 31]);
      }
    }
  } else if constexpr (MIX == kBlockAgpr || MIX == kBlockNoMulAgpr || MIX == kBlockHiLo ||
                       MIX == kBlockHiLoAgpr) {
    // two score products (four with high and low query parts) into VGPRs,
    // two weighted sums into VGPRs or AGPRs
    constexpr bool HILO = MIX == kBlockHiLo || MIX == kBlockHiLoAgpr;
    constexpr bool AG = MIX != kBlockHiLo;
    constexpr bool MUL = MIX == kBlockAgpr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 2) {
        MFMA(r.acc[j]);
        if constexpr (HILO) MFMA(r.acc[j]);
      } else {
        if constexpr (AG) MFMA_A(r.acca[j - 2]); else MFMA(r.acc[j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (MUL) VMUL(r.x[4 * j + i]);
        VEXP(r.x[16 + 4 * j + i]);
      }
      VCVT(r.pk[2 * j], r.x[4 * j], r.x[4 * j + 1]);
      VCVT(r.pk[2 * j + 1], r.x[4 * j + 2], r.x[4 * j + 3]);
      VDOT(r.s[2 * j], r.pk[(2 * j + 3) & 7]);
      VDOT(r.s[2 * j + 1], r.pk[(2 * j + 4) & 7]);
    }
  } else if constexpr (MIX == kBlockDep) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      MFMA(r.acc[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) VMUL(r.x[4 * j + i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) VEXP(r.x[4 * j + i]);
      VCVT(r.pk[2 * j], r.x[4 * j], r.x[4 * j + 1]);
      VCVT(r.pk[2 * j + 1], r.x[4 * j + 2], r.x[4 * j + 3]);
      VDOT(r.s[2 * j], r.pk[2 * j]);
      VDOT(r.s[2 * j + 1], r.pk[2 * j + 1]);
    }
  } else if constexpr (MIX == kBlock || MIX == kBlockNoMul || MIX == kBlockNoDot) {
    // per MFMA: 4 mul, 4 exp, 2 cvt, 2 dot2 (the encoder's per-block mix)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      MFMA(r.acc[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (MIX != kBlockNoMul) VMUL(r.x[4 * j + i]);
        VEXP(r.x[16 + 4 * j + i]);
      }
      VCVT(r.pk[2 * j], r.x[4 * j], r.x[4 * j + 1]);
      VCVT(r.pk[2 * j + 1], r.x[4 * j + 2], r.x[4 * j + 3]);
      if constexpr (MIX != kBlockNoDot) {
        VDOT(r.s[2 * j], r.pk[(2 * j + 3) & 7]);
        VDOT(r.s[2 * j + 1], r.pk[(2 * j + 4) & 7]);
      }
    }
  }
}

// Which accumulator arrays a mix touches (the others stay dead, so the
// register budget of 4 waves per SIMD holds).
constexpr bool uses_acca(int m) {
  return m == kAgpr || m == kAgprMul8 || m == kAgprExp16 || m == kBlockAgpr || m == kBlockHiLoAgpr ||
         m == kBlockNoMulAgpr;
}
constexpr bool uses_acc4(int m) { return m == kMfma16 || m == kMfma16Mul8 || m == kMfma16Exp16; }
constexpr bool block_agpr(int m) { return m == kBlockAgpr || m == kBlockHiLoAgpr || m == kBlockNoMulAgpr; }
constexpr bool uses_acc(int m) { return !uses_acca(m) || block_agpr(m); }

// Mixes that hold accumulators in AGPRs as well as VGPRs run at most two
// waves per SIMD (a 256-register budget), where the compiler's split of the
// register file between the two kinds leaves room for both.
constexpr int max_threads(int m) { return block_agpr(m) ? 512 : 1024; }

template <int MIX0, int MIX1>
__global__ __launch_bounds__(max_threads(MIX0)) void probe_kernel(float* out, long long* cycles, int iters,
                                                                  int role_shift) {
  // per wave w: cycles[4 w], cycles[4 w + 1] = shader clock at the start and
  // the end of its loop; cycles[4 w + 2], cycles[4 w + 3] = the same instants
  // on the constant 100 MHz real-time counter
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Regs r;
  const float f = 1.0f + 1e-3f * (float)lane;
  constexpr bool A = uses_acc(MIX0) || uses_acc(MIX1);
  constexpr bool AA = uses_acca(MIX0) || uses_acca(MIX1);
  constexpr bool A4 = uses_acc4(MIX0) || uses_acc4(MIX1);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) r.acc[c][i] = r.acca[c][i] = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) r.acc4[c][i] = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) r.x[i] = 0.5f * f + 1e-4f * (float)i;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r.pk[i] = 0x3f803f80u + (uint32_t)i;
    r.s[i] = 0.f;
  }
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(f * 0.01f);
    b[i] = (__bf16)(0.02f * (float)(i + 1));
  }
  const float cm = 0.9999f;
  // role: the first mix on waves whose bit `role_shift` is 0, the second on
  // the others (role_shift < 0: the first mix everywhere)
  const bool second = role_shift >= 0 && ((wave >> role_shift) & 1);
  const long long r0 = wall_clock64();
  const long long t0 = clock64();
  if (!second) {
    for (int it = 0; it < iters; ++it) body<MIX0>(r, a, b, cm);
  } else {
    for (int it = 0; it < iters; ++it) body<MIX1>(r, a, b, cm);
  }
  const long long t1 = clock64();
  const long long r1 = wall_clock64();
  float acc = 0.f;
  // the mixes with AGPR weighted sums use acc[0..1] and acca[0..1] only
  constexpr int NC = block_agpr(MIX0) && block_agpr(MIX1) ? 2 : 4;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (A) acc += r.acc[c][i];
      if constexpr (AA) acc += r.acca[c][i];
    }
  if constexpr (A4) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += r.acc4[c][i];
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) acc += r.x[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += r.s[i] + (float)(r.pk[i] & 1u);
  out[(size_t)blockIdx.x * blockDim.x + tid] = acc;
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * (blockDim.x >> 6) + wave;
    cycles[4 * w] = t0;
    cycles[4 * w + 1] = t1;
    cycles[4 * w + 2] = r0;
    cycles[4 * w + 3] = r1;
  }
}

template <int M0, int M1>
static hipError_t launch(int blocks, int threads, float* out, long long* cyc, int iters, int role_shift,
                         hipStream_t st) {
  if (threads > max_threads(M0)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((probe_kernel<M0, M1>), dim3(blocks), dim3(threads), 0, st, out, cyc, iters, role_shift);
  return hipGetLastError();
}

extern "C" {

// Runs mix `mix0` (and `mix1` on the waves selected by role_shift >= 0) on
// `blocks` workgroups of `threads` threads (a multiple of 64, at most 1024),
// `iters` loop iterations.  out: blocks * threads floats; cycles: four per
// wave (4 * blocks * threads / 64).  Returns a hipError_t.
int probe_run(int mix0, int mix1, int blocks, int threads, int iters, int role_shift, float* out,
              long long* cycles, void* stream) {
  if (blocks < 1 || threads < 64 || threads > 1024 || threads % 64 || iters < 1) return (int)hipErrorInvalidValue;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
#define P1(M) \
  if (mix0 == M && role_shift < 0) return (int)launch<M, M>(blocks, threads, out, cycles, iters, role_shift, st);
  P1(kMfma) P1(kMul) P1(kExp) P1(kCvt) P1(kDot2) P1(kMulExp) P1(kMfmaMul4) P1(kMfmaMul8) P1(kMfmaMul16)
  P1(kMfmaExp4) P1(kMfmaExp8) P1(kMfmaExp16) P1(kBlock) P1(kBlockNoMul) P1(kBlockNoDot) P1(kBlockDep)
  P1(kAgpr) P1(kAgprMul8) P1(kAgprExp16) P1(kMfma16) P1(kMfma16Mul8) P1(kMfma16Exp16) P1(kBlockAgpr)
  P1(kBlockHiLo) P1(kBlockHiLoAgpr) P1(kBlockNoMulAgpr)
#undef P1
#define P2(A, B) \
  if (mix0 == A && mix1 == B && role_shift >= 0) return (int)launch<A, B>(blocks, threads, out, cycles, iters, role_shift, st);
  P2(kMfma, kExp) P2(kMfma, kMul) P2(kMfma, kIdle) P2(kExp, kMul) P2(kExp, kIdle) P2(kMul, kIdle)
#undef P2
  return (int)hipErrorInvalidValue;
}

}  // extern "C"
