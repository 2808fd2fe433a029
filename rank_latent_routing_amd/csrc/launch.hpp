// Parameter blocks and launchers of the gfx950 kernels (internal to the
// library; the public surface is include/flare.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace flare {

// Tile sizes shared by the kernels and the host-side planners (plan.cpp).
constexpr int kEncT = 128;        // encoder: tokens per LDS tile (four 32-token quarters)
constexpr int kDecWaves = 12;     // decoder: one workgroup per compute unit, 3 waves per SIMD
constexpr int kDecGroup = 64;     // decoder: tokens per wave per step
constexpr int kLatBwdTile = 64;   // backward latent pass: tokens per LDS tile

// Strided [B, H, L, D] view in elements, D contiguous.
struct View {
  const void* data;
  int is_f32;
  int64_t sb, sh, sl;
};

struct EncodeParams {
  View q;             // [B, H, M, D] (sb may be 0)
  View k, v;          // [B, H, N, D]
  float* part_o;      // [B*H, S, M, D] normalised split outputs
  float* part_l;      // [B*H, S, M] split log2-normalisers (of scale*log2e*q.k)
  int H, M, S;
  int64_t N, tokens_per_split;
  float c;            // scale * log2(e)
  int exact;          // 1: running-maximum softmax only
};

struct MergeParams {
  const float* part_o;
  const float* part_l;
  void* z;            // [B, H, M, D]
  int z_f32;
  int64_t z_sb, z_sh, z_sl;
  float* lse;         // [B, H, M] natural log, may be null
  int H, M, S, D;
  int G;              // split groups per feature (set by launch_merge)
};

struct DecodeParams {
  View k;             // [B, H, N, D]
  View q, z;          // [B, H, M, D]
  void* y;            // [B, H, N, D]
  int y_f32;
  int64_t y_sb, y_sh, y_sl;
  int H, M;
  int64_t N;
  int64_t tokens_per_block;  // bf16 path: workgroups per head; fp32 path: tokens per workgroup
  float c;
  int exact;
  float* lse;         // [B, H, N] natural-log row normalisers, may be null
  // When zm_part_o is set, Z is not read from z but merged from the
  // encoder's split results ([B*H, zm_S, M, D] and [B*H, zm_S, M]) while it
  // is staged: the mixer's encoder without a merge launch.
  const float* zm_part_o;
  const float* zm_part_l;
  int zm_S;
};

// Backward, token-parallel pass (decoder layout): per token, dK (and dV).
//   decode role: P = softmax over latents of the decoder, W = Z, X = dY;
//                writes dK and delta_n = dY_n . Y_n.
//   encode role: P = softmax over tokens of the encoder (per-latent
//                normaliser), W = dZ, X = V; writes dK and dV.
struct TokBwdParams {
  View k, x, y;          // token-side bf16 [B, H, N, D]; y: decode role only
  View q, w, z;          // latent-side [B, H, M, D]; z: encode role only
  const float* lse;      // natural-log normalisers: [B, H, N] (decode) or [B, H, M] (encode)
  void* dk;              // [B, H, N, D] view, fp32 or (grad_bf16) bf16
  int64_t dk_sb, dk_sh, dk_sl;
  void* dv;              // encode role only; same dtype as dk
  int64_t dv_sb, dv_sh, dv_sl;
  int grad_bf16;         // dk and dv are bf16 (accumulation adds in fp32, then rounds)
  float* delta;          // decode role: [B, H, N] written
  int H, M;
  int64_t N;
  float c, scale;        // c = scale * log2(e)
  int accumulate;        // add into dk instead of overwriting
  int blocks_per_head;
  // set by the launcher: this launch covers latents [m0, m0 + mb) and adds
  // into dv when accumulate_v (the encode role runs in latent blocks)
  int m0, mb, accumulate_v;
};

// Backward of a FLARE encode/decode pair, token-parallel pass of both roles
// at once: the scores Q K^T serve the encoder's and the decoder's weights,
// and dK takes both roles' gradients in one accumulator.
struct TokPairParams {
  View k, v, dy;         // token-side bf16 [B, H, N, D]
  View q, z, dz;         // latent-side [B, H, M, D]
  const float* lse_e;    // encoder normalisers [B, H, M], natural log
  const float* lse_d;    // decoder normalisers [B, H, N], natural log
  const float* delta_d;  // dY . Y [B, H, N]
  void* dk;              // [B, H, N, D] views, fp32 or (grad_bf16) bf16
  int64_t dk_sb, dk_sh, dk_sl;
  void* dv;
  int64_t dv_sb, dv_sh, dv_sl;
  int grad_bf16;
  int H, M;
  int64_t N;
  float c, scale;
  int accumulate;        // add into dk instead of overwriting
  int blocks_per_head;
};

// Backward, latent-parallel pass over token splits (encoder layout): per
// latent, fp32 partial sums of dQ (and dZ) for each split.
//   decode role: W = Z, X = dY, per-token normaliser and delta; dQ and dZ.
//   encode role: W = dZ, X = V, per-latent normaliser; dQ.
struct LatBwdParams {
  View k, x;             // token-side bf16 [B, H, N, D]
  View q, w, z;          // latent-side [B, H, M, D]; z: encode role only
  const float* lse;      // [B, H, N] (decode) or [B, H, M] (encode), natural log
  const float* delta;    // decode role: [B, H, N], read unless y is given
  View y;                // decode role, optional: Y, to compute delta = dY . Y in place
  float* delta_out;      // with y: delta written here ([B, H, N]) when non-null
  float* dq_part;        // [B*H, S, M, D]
  float* dz_part;        // decode role only
  int H, M, S;
  int64_t N;
  float c;
};

// Decoder with the output projection in its epilogue (D = 32, C = 32 H with
// H = 4 or 8, bf16 out [B, N, C] row-major).
constexpr int kDecWoWaves = 12;  // one workgroup of 12 waves per compute unit, 3 per SIMD
struct DecodeWoParams {
  View k;                 // [B, H, N, D] bf16
  View q, z;              // [B|1, H, M, D] latent side (fp32 or bf16)
  unsigned char* lat_ops; // scratch: B H (M/32 rounded up) 4 KB, latent operands in LDS order
  unsigned char* wt;      // scratch: C C 2 bytes, W_O^T in LDS order
  void* out;              // [B, N, C] bf16
  int H, M;
  int64_t N;
  float c;                // scale * log2(e)
  int exact;
  int buf_bytes;          // set by the launcher
};
// LDS bytes of one workgroup (two buffers).
size_t decode_wo_lds(int M, int C);
// Bytes of scratch the two prepared operands need.
inline size_t decode_wo_scratch(int B, int H, int M) {
  return (size_t)B * H * ((M + 31) / 32) * 4096 + (size_t)(32 * H) * (32 * H) * 2;
}
hipError_t launch_decode_wo(const DecodeWoParams& p, int B, const void* w_o, hipStream_t s);

struct GemmParams {
  const void* x;      // [R, Cin] bf16 row-major
  const void* w[5];   // weights [Cin, Cout] bf16 row-major (read by the preloading kernel)
  const void* wt[5];  // the weights in operand order (launch_swizzle_weights; the streaming kernel)
  void* y[5];         // outputs
  int n_proj;
  int64_t R;
  int Cin, Cout;
  int head_major;     // 1: y is [B, H, N, D] with R = B*N, Cout = H*D
  int64_t N;          // tokens per batch element (head_major)
  int D;              // head width (head_major)
};

// Split planning shared by the workspace-size query and the launcher.
struct EncodePlan {
  int S;                    // number of token splits
  int64_t tokens_per_split; // fp32 path: contiguous tokens per split (multiple of 128)
  int waves;                // waves per workgroup (bf16 path)
  int lat_blocks;           // 16-latent blocks per wave (bf16 path)
};
// max_splits > 0 caps the number of splits (fewer, longer splits need less
// scratch for their partial results; the merged result differs by rounding).
EncodePlan plan_encode(int B, int H, int M, int64_t N, int D, int is_f32, int max_splits = 0);

hipError_t launch_encode_bf16(const EncodeParams& p, int D, int B, int waves, int lat_blocks, hipStream_t s);
// The 8-wave, 32-feature encoder (encode_wide.hip) on the given grid.
hipError_t launch_encode_bf16_wide(const EncodeParams& p, dim3 grid, hipStream_t s);
hipError_t launch_encode_f32(const EncodeParams& p, int D, int B, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, int B, hipStream_t s);
// Workgroups per (batch, head) of the bf16 decoder.
int64_t plan_decode_bf16(int B, int H, int M, int64_t N, int D);
// LDS bytes of one decoder workgroup.
size_t decode_bf16_lds(int M, int D);
// Extra LDS of a decoder that merges Z from split results while staging it.
inline size_t decode_merge_lds(int M, int D) { return (size_t)((M + 31) / 32) * 32 * D * sizeof(float); }
// Split results (per batch*head) that a consumer kernel may merge itself
// while staging them, in place of a merge launch.
constexpr int64_t kConsumerMergeBytes = 128 * 1024;
hipError_t launch_decode_bf16(const DecodeParams& p, int D, int B, hipStream_t s);
hipError_t launch_decode_f32(const DecodeParams& p, int D, int B, hipStream_t s);
int plan_bwd_splits(int B, int H, int M, int64_t N);
hipError_t launch_tok_bwd(const TokBwdParams& p, int D, int B, bool encode_role, hipStream_t s);
hipError_t launch_lat_bwd(const LatBwdParams& p, int D, int B, bool encode_role, hipStream_t s);
// Largest M the pair pass stages (its latent operands must fit one CU's LDS).
constexpr int kTokPairMaxM = 256;
hipError_t launch_tok_pair(const TokPairParams& p, int D, int B, hipStream_t s);
hipError_t launch_sum_splits(const float* part, float* out, int B, int H, int S, int64_t MD, bool batch_sum,
                             float factor, int accumulate, hipStream_t st);
// Weights [Cin, Cout] row-major -> the GEMM's A-operand order, up to five at once.
struct SwizzleParams {
  const void* w[5];
  void* wsw[5];
  int Cin, Cout;
};
hipError_t launch_swizzle_weights(const SwizzleParams& p, int n, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t s);

// The projection kernel's two forms.  With one 16-row tile per wave (fewer
// than 512 workgroups of two) and at most kGemmPreloadBytes of weights, each
// workgroup lays out every weight block in LDS itself, from the row-major
// weights, before computing.  Otherwise the weights are first rearranged into
// operand order in the workspace (launch_swizzle_weights) and streamed.
constexpr int64_t kGemmPreloadBytes = 128 * 1024;
inline bool gemm_preloads(int64_t R, int n_proj, int Cin, int Cout) {
  const bool one_tile = (R + 16 * 2 * 8 - 1) / (16 * 2 * 8) < 512;
  return one_tile && (int64_t)n_proj * Cin * Cout * 2 <= kGemmPreloadBytes;
}

}  // namespace flare
