// X reuse across heads.  A kernel that fused the projections into the
// per-head attention kernels would have every head's workgroup read all C
// input features of its tokens, so each token's X row would be read once per
// head.  Does a second head's workgroup over the same token window find X in
// L2, or fetch it again from memory?
//
// Each workgroup (256 threads) reads the X rows of one row block, all C bf16
// features, with 16-byte loads, reduces them and stores one float per wave,
// so nothing is optimised away.  The grid has (row blocks) x H workgroups; the
// template ORDER maps the dispatch index to (row block, head):
//   0  head-major: every row block of head 0, then of head 1, ... (a head's
//      sweep is far larger than L2, so nothing is reused in L2);
//   1  head-interleaved: the H workgroups of a row block are consecutive in
//      dispatch order, which spreads them over the eight XCDs (workgroup i
//      goes to XCD i mod 8, each XCD with its own L2);
//   2  head-interleaved per XCD: the H workgroups of a row block are
//      consecutive among the workgroups that one XCD receives, so they meet
//      in that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int ORDER, int CH>
__global__ __launch_bounds__(256) void xreuse_kernel(const bf16x8* __restrict__ x, int64_t R, int H,
                                                     int rows_per_block, float* __restrict__ out) {
  const int64_t wg = blockIdx.x;
  const int64_t nrb = (R + rows_per_block - 1) / rows_per_block;
  int64_t rb, h;
  if constexpr (ORDER == 0) {
    h = wg / nrb;
    rb = wg - h * nrb;
  } else if constexpr (ORDER == 1) {
    rb = wg / H;
    h = wg - rb * H;
  } else {
    const int64_t xcd = wg & 7, j = wg >> 3;
    rb = (j / H) * 8 + xcd;
    h = j - (j / H) * H;
  }
  const int64_t r0 = rb * rows_per_block;
  float acc = 0.f;
  for (int u = threadIdx.x; u < rows_per_block * CH; u += 256) {
    const int64_t row = r0 + u / CH;
    if (row < R) {
      const bf16x8 v = x[row * CH + u % CH];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += (float)v[j];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) out[wg * 4 + (threadIdx.x >> 6)] = acc * (float)(h + 1);
}

template <int CH>
hipError_t launch(int order, const void* x, int64_t R, int H, int rpb, float* out, hipStream_t st) {
  const int64_t nrb = (R + rpb - 1) / rpb;
  const dim3 grid((unsigned)(nrb * H));
  const bf16x8* xv = reinterpret_cast<const bf16x8*>(x);
  if (order == 0)
    hipLaunchKernelGGL((xreuse_kernel<0, CH>), grid, dim3(256), 0, st, xv, R, H, rpb, out);
  else if (order == 1)
    hipLaunchKernelGGL((xreuse_kernel<1, CH>), grid, dim3(256), 0, st, xv, R, H, rpb, out);
  else
    hipLaunchKernelGGL((xreuse_kernel<2, CH>), grid, dim3(256), 0, st, xv, R, H, rpb, out);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Reads X [R, C] bf16 (16-byte aligned rows, C = 128 or 256) once per head in
// dispatch order `order` (0, 1 or 2, above), in row blocks of rows_per_block
// rows (64, 128 or 256).  out: 4 floats per workgroup, (R / rows_per_block) x
// H x 4 in all.  Order 2 needs the row-block count to be a multiple of 8.
// Returns a hipError_t.
int xreuse_run(const void* x, long long R, int C, int H, int order, int rows_per_block, float* out,
               void* stream) {
  if (!x || !out || R < 1 || H < 1 || H > 64 || order < 0 || order > 2) return (int)hipErrorInvalidValue;
  if (rows_per_block != 64 && rows_per_block != 128 && rows_per_block != 256) return (int)hipErrorInvalidValue;
  const long long nrb = (R + rows_per_block - 1) / rows_per_block;
  if (order == 2 && nrb % 8) return (int)hipErrorInvalidValue;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (C == 256) return (int)launch<32>(order, x, R, H, rows_per_block, out, st);
  if (C == 128) return (int)launch<16>(order, x, R, H, rows_per_block, out, st);
  return (int)hipErrorInvalidValue;
}

}  // extern "C"
