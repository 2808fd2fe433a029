// C ABI of the FLARE / FLARE++ mixer library (declared in include/flare.h).
//
// Host side only: argument validation (done completely before any HIP call,
// so a rejected call never touches the device), split planning, carving of
// the caller's workspace, and kernel launches on the caller's stream.  The
// library allocates nothing and keeps no mutable state.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstring>

#include "../../include/flare.h"
#include "api_internal.hpp"
#include "launch.hpp"

using namespace flare;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxM = 512;
constexpr int64_t kMaxBH = 65535;  // grid.y

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_dtype(int32_t d) { return d == FLARE_F32 || d == FLARE_BF16; }

bool sizes_ok(int B, int H, int M, int64_t N, int D) {
  return B >= 1 && H >= 1 && M >= 1 && N >= 1 && (int64_t)B * H <= kMaxBH && M <= kMaxM &&
         (D == 16 || D == 32) && N <= (int64_t(1) << 40);
}

// Token-side tensors are read/written with vector accesses: rows must be
// 16-byte aligned.
bool token_tensor_ok(const flare_tensor* t) {
  if (!t || !t->data || !is_dtype(t->dtype)) return false;
  if (reinterpret_cast<uintptr_t>(t->data) % 16) return false;
  const int64_t q = t->dtype == FLARE_BF16 ? 8 : 4;
  if (t->stride_b < 0 || t->stride_h < 0 || t->stride_l < 0) return false;
  // the kernels address a 128-token tile with 32-bit byte offsets
  if (t->stride_l >= (int64_t(1) << 22)) return false;
  return t->stride_b % q == 0 && t->stride_h % q == 0 && t->stride_l % q == 0;
}

// Latent-side tensors (queries, seeds, latent values) are read element-wise.
bool latent_tensor_ok(const flare_tensor* t) {
  if (!t || !t->data || !is_dtype(t->dtype)) return false;
  const size_t el = t->dtype == FLARE_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(t->data) % el) return false;
  return t->stride_b >= 0 && t->stride_h >= 0 && t->stride_l >= 0;
}

bool scale_ok(float scale) { return std::isfinite(scale); }

float log2_scale(float scale, int D) {
  const float s = scale == 0.0f ? 1.0f / std::sqrt((float)D) : scale;
  return s * 1.4426950408889634f;  // log2(e)
}

View view_of(const flare_tensor* t) {
  View v;
  v.data = t->data;
  v.is_f32 = t->dtype == FLARE_F32;
  v.sb = t->stride_b;
  v.sh = t->stride_h;
  v.sl = t->stride_l;
  return v;
}

flare_status hip_status(hipError_t e) { return e == hipSuccess ? FLARE_OK : FLARE_E_HIP; }

size_t encode_ws(int B, int H, int M, int64_t N, int D, int is_f32, int max_splits = 0) {
  const EncodePlan pl = plan_encode(B, H, M, N, D, is_f32, max_splits);
  const size_t parts = (size_t)B * H * pl.S * M;
  return align_up(parts * D * sizeof(float)) + align_up(parts * sizeof(float));
}

// Encoder on validated arguments: split kernel + merge into Z (and lse).
// max_splits > 0 caps the split count (the workspace then needs
// encode_ws(..., max_splits) bytes).
flare_status encode_impl(const View& q, const View& k, const View& v, void* z, int z_f32,
                         int64_t z_sb, int64_t z_sh, int64_t z_sl, float* lse, int B, int H, int M,
                         int64_t N, int D, float c, unsigned flags, void* ws, hipStream_t st,
                         int max_splits = 0) {
  const EncodePlan pl = plan_encode(B, H, M, N, D, k.is_f32, max_splits);
  const size_t parts = (size_t)B * H * pl.S * M;
  EncodeParams ep;
  std::memset(&ep, 0, sizeof(ep));
  ep.q = q;
  ep.k = k;
  ep.v = v;
  ep.part_o = reinterpret_cast<float*>(ws);
  ep.part_l = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align_up(parts * D * sizeof(float)));
  ep.H = H;
  ep.M = M;
  ep.S = pl.S;
  ep.N = N;
  ep.tokens_per_split = pl.tokens_per_split;
  ep.c = c;
  ep.exact = (flags & FLARE_FLAG_EXACT_SOFTMAX) ? 1 : 0;
  hipError_t e = k.is_f32 ? launch_encode_f32(ep, D, B, st) : launch_encode_bf16(ep, D, B, pl.waves, pl.lat_blocks, st);
  if (e != hipSuccess) return FLARE_E_HIP;
  MergeParams mp;
  mp.part_o = ep.part_o;
  mp.part_l = ep.part_l;
  mp.z = z;
  mp.z_f32 = z_f32;
  mp.z_sb = z_sb;
  mp.z_sh = z_sh;
  mp.z_sl = z_sl;
  mp.lse = lse;
  mp.H = H;
  mp.M = M;
  mp.S = pl.S;
  mp.D = D;
  return hip_status(launch_merge(mp, B, st));
}

// The mixer's split encoder without its merge launch: the decoder merges the
// split results (written at ws) while it stages them.
flare_status encode_splits(const View& q, const View& k, const View& v, int B, int H, int M, int64_t N, int D,
                           float c, unsigned flags, void* ws, hipStream_t st) {
  const EncodePlan pl = plan_encode(B, H, M, N, D, 0);
  const size_t parts = (size_t)B * H * pl.S * M;
  EncodeParams ep;
  std::memset(&ep, 0, sizeof(ep));
  ep.q = q;
  ep.k = k;
  ep.v = v;
  ep.part_o = reinterpret_cast<float*>(ws);
  ep.part_l = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align_up(parts * D * sizeof(float)));
  ep.H = H;
  ep.M = M;
  ep.S = pl.S;
  ep.N = N;
  ep.tokens_per_split = pl.tokens_per_split;
  ep.c = c;
  ep.exact = (flags & FLARE_FLAG_EXACT_SOFTMAX) ? 1 : 0;
  return hip_status(launch_encode_bf16(ep, D, B, pl.waves, pl.lat_blocks, st));
}

// zm_o / zm_l / zm_S (bf16 path only): merge Z from the encoder's split results
// while staging it instead of reading z.
flare_status decode_impl(const View& k, const View& q, const View& z, void* y, int y_f32,
                         int64_t y_sb, int64_t y_sh, int64_t y_sl, float* lse, int B, int H, int M,
                         int64_t N, int D, float c, unsigned flags, hipStream_t st,
                         const float* zm_o = nullptr, const float* zm_l = nullptr, int zm_S = 0) {
  DecodeParams dp;
  std::memset(&dp, 0, sizeof(dp));
  dp.lse = lse;
  dp.zm_part_o = zm_o;
  dp.zm_part_l = zm_l;
  dp.zm_S = zm_S;
  dp.k = k;
  dp.q = q;
  dp.z = z;
  dp.y = y;
  dp.y_f32 = y_f32;
  dp.y_sb = y_sb;
  dp.y_sh = y_sh;
  dp.y_sl = y_sl;
  dp.H = H;
  dp.M = M;
  dp.N = N;
  dp.c = c;
  dp.exact = (flags & FLARE_FLAG_EXACT_SOFTMAX) ? 1 : 0;
  if (k.is_f32) {
    dp.tokens_per_block = 256;
    return hip_status(launch_decode_f32(dp, D, B, st));
  }
  dp.tokens_per_block = plan_decode_bf16(B, H, M, N, D);  // workgroups per head
  return hip_status(launch_decode_bf16(dp, D, B, st));
}

float natural_scale(float scale, int D) { return scale == 0.0f ? 1.0f / std::sqrt((float)D) : scale; }

bool f32_ptr_ok(const void* p) { return p && reinterpret_cast<uintptr_t>(p) % 4 == 0; }

constexpr unsigned kBwdFlags = FLARE_ACCUMULATE_DQ | FLARE_ACCUMULATE_DK | FLARE_SUM_DQ_OVER_BATCH;

// Token-side gradients (dK, dV) are written in fp32 or bf16.
bool grad_dtype_ok(int32_t d) { return d == FLARE_F32 || d == FLARE_BF16; }

flare_status bwd_common_checks(int B, int H, int M, int64_t N, int D, float scale) {
  if (!sizes_ok(B, H, M, N, D)) {
    if (B >= 1 && H >= 1 && M >= 1 && N >= 1 && (M > kMaxM || !(D == 16 || D == 32)))
      return FLARE_E_UNSUPPORTED;
    return FLARE_E_INVALID;
  }
  if (!scale_ok(scale)) return FLARE_E_INVALID;
  return FLARE_OK;
}

// Workgroups per head of the token-parallel backward pass: about `total` in
// all, each step of a workgroup covering `step` tokens (4 waves x 64 tokens in
// the decode role; 8 x 64 in the encode role, one workgroup per CU).
int64_t tok_bwd_blocks(int B, int H, int64_t N, int64_t step, int64_t total) {
  const int64_t bh = (int64_t)B * H;
  const int64_t steps = (N + step - 1) / step;
  int64_t per = (total + bh - 1) / bh;
  if (per > steps) per = steps;
  return per < 1 ? 1 : per;
}

// Workgroups per head of the pair pass (8 waves x 32 tokens per step): one
// per CU in all, so each stages its head's latent operands once.
int64_t tok_pair_blocks(int B, int H, int64_t N) {
  const int64_t bh = (int64_t)B * H;
  const int64_t steps = (N + 255) / 256;
  int64_t per = (256 + bh - 1) / bh;
  if (per > steps) per = steps;
  return per < 1 ? 1 : per;
}

bool proj_shape_ok(int64_t R, int Cin, int Cout, int n_proj) {
  return R >= 1 && (Cin == 32 || Cin == 64 || Cin == 128 || Cin == 256) && Cout >= 32 &&
         Cout % 32 == 0 && Cout <= 4096 && n_proj >= 1 && n_proj <= 5 &&
         (R + 511) / 512 <= 0x7fffffff;
}

size_t proj_ws(int Cin, int Cout, int n_proj) {
  return (size_t)n_proj * align_up((size_t)Cin * Cout * 2);
}

flare_status project_impl(const void* X, const void* const* W, void* const* Y, int n_proj, int64_t R,
                          int Cin, int Cout, int head_major, int B, int head_dim, void* ws,
                          hipStream_t st) {
  GemmParams gp;
  std::memset(&gp, 0, sizeof(gp));
  gp.x = X;
  gp.n_proj = n_proj;
  gp.R = R;
  gp.Cin = Cin;
  gp.Cout = Cout;
  gp.head_major = head_major;
  gp.N = head_major ? R / B : R;
  gp.D = head_major ? head_dim : Cout;
  SwizzleParams sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.Cin = Cin;
  sp.Cout = Cout;
  for (int i = 0; i < n_proj; ++i) {
    void* wt = reinterpret_cast<char*>(ws) + i * align_up((size_t)Cin * Cout * 2);
    sp.w[i] = W[i];
    sp.wsw[i] = wt;
    gp.w[i] = W[i];
    gp.wt[i] = wt;
    gp.y[i] = Y[i];
  }
  if (!gemm_preloads(R, n_proj, Cin, Cout) && launch_swizzle_weights(sp, n_proj, st) != hipSuccess)
    return FLARE_E_HIP;
  return hip_status(launch_gemm_bf16(gp, st));
}

}  // namespace

namespace flare {

flare_status encode_validate(const flare_tensor* Q, const flare_tensor* K, const flare_tensor* V,
                             const flare_tensor* Z, const float* lse, int B, int H, int M, int64_t N,
                             int D, float scale, unsigned flags) {
  if (!sizes_ok(B, H, M, N, D)) {
    if (B >= 1 && H >= 1 && M >= 1 && N >= 1 && (M > kMaxM || !(D == 16 || D == 32)))
      return FLARE_E_UNSUPPORTED;
    return FLARE_E_INVALID;
  }
  if (!latent_tensor_ok(Q) || !token_tensor_ok(K) || !token_tensor_ok(V) || !latent_tensor_ok(Z))
    return FLARE_E_INVALID;
  if (K->dtype != V->dtype) return FLARE_E_INVALID;
  if (!scale_ok(scale) || (flags & ~FLARE_FLAG_EXACT_SOFTMAX)) return FLARE_E_INVALID;
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4) return FLARE_E_INVALID;
  return FLARE_OK;
}

int encode_splits_within(int B, int H, int M, int64_t N, int D, int is_f32, size_t max_bytes) {
  int S = plan_encode(B, H, M, N, D, is_f32).S;
  while (S > 1 && encode_ws(B, H, M, N, D, is_f32, S) > max_bytes) {
    // the bytes are linear in S: jump close to the largest S that fits
    const size_t one = encode_ws(B, H, M, N, D, is_f32, 1);
    const int fit = (int)std::max<size_t>(1, max_bytes / std::max<size_t>(one, 1));
    S = std::min(S - 1, fit);
  }
  return encode_ws(B, H, M, N, D, is_f32, S) <= max_bytes ? S : 0;
}

flare_status encode_run(const flare_tensor* Q, const flare_tensor* K, const flare_tensor* V,
                        const flare_tensor* Z, float* lse, int B, int H, int M, int64_t N, int D,
                        float scale, unsigned flags, void* ws, int max_splits, void* stream) {
  return encode_impl(view_of(Q), view_of(K), view_of(V), Z->data, Z->dtype == FLARE_F32, Z->stride_b,
                     Z->stride_h, Z->stride_l, lse, B, H, M, N, D, log2_scale(scale, D), flags, ws,
                     reinterpret_cast<hipStream_t>(stream), max_splits);
}

}  // namespace flare

extern "C" {

const char* flare_version(void) { return "0.1.0"; }

const char* flare_status_string(int s) {
  switch (s) {
    case FLARE_OK: return "ok";
    case FLARE_E_INVALID: return "invalid argument";
    case FLARE_E_UNSUPPORTED: return "unsupported configuration";
    case FLARE_E_WORKSPACE: return "workspace missing or too small";
    case FLARE_E_HIP: return "HIP runtime error";
    case FLARE_E_SCRATCH: return "sizes exceed the static scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

size_t flare_encode_workspace_size(int B, int H, int M, int64_t N, int D) {
  if (!sizes_ok(B, H, M, N, D)) return 0;
  const size_t a = encode_ws(B, H, M, N, D, 0), b = encode_ws(B, H, M, N, D, 1);
  return a > b ? a : b;
}

static flare_status encode_checked(const flare_tensor* Q, const flare_tensor* K, const flare_tensor* V,
                                   const flare_tensor* Z, float* lse, int B, int H, int M, int64_t N,
                                   int D, float scale, unsigned flags, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const flare_status v = flare::encode_validate(Q, K, V, Z, lse, B, H, M, N, D, scale, flags);
  if (v != FLARE_OK) return v;
  const size_t need = encode_ws(B, H, M, N, D, K->dtype == FLARE_F32);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 16)
    return FLARE_E_WORKSPACE;
  return flare::encode_run(Q, K, V, Z, lse, B, H, M, N, D, scale, flags, workspace, 0, stream);
}

flare_status flare_encode(const flare_tensor* Q, const flare_tensor* K, const flare_tensor* V,
                          const flare_tensor* Z, float* lse, int B, int H, int M, int64_t N, int D,
                          float scale, unsigned flags, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return encode_checked(Q, K, V, Z, lse, B, H, M, N, D, scale, flags, workspace, workspace_bytes,
                        stream);
}

flare_status flare_route_queries(const flare_tensor* seeds, const flare_tensor* eK,
                                 const flare_tensor* eV, const flare_tensor* Qx, float* lse, int B,
                                 int H, int M, int64_t N, int D, float scale, unsigned flags,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return encode_checked(seeds, eK, eV, Qx, lse, B, H, M, N, D, scale, flags, workspace,
                        workspace_bytes, stream);
}

flare_status flare_decode(const flare_tensor* K, const flare_tensor* Q, const flare_tensor* Z,
                          const flare_tensor* Y, float* lse, int B, int H, int M, int64_t N, int D,
                          float scale, unsigned flags, void* stream) {
  if (!sizes_ok(B, H, M, N, D)) {
    if (B >= 1 && H >= 1 && M >= 1 && N >= 1 && (M > kMaxM || !(D == 16 || D == 32)))
      return FLARE_E_UNSUPPORTED;
    return FLARE_E_INVALID;
  }
  if (!token_tensor_ok(K) || !latent_tensor_ok(Q) || !latent_tensor_ok(Z) || !token_tensor_ok(Y))
    return FLARE_E_INVALID;
  if (!scale_ok(scale) || (flags & ~FLARE_FLAG_EXACT_SOFTMAX)) return FLARE_E_INVALID;
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4) return FLARE_E_INVALID;
  return decode_impl(view_of(K), view_of(Q), view_of(Z), Y->data, Y->dtype == FLARE_F32, Y->stride_b,
                     Y->stride_h, Y->stride_l, lse, B, H, M, N, D, log2_scale(scale, D), flags,
                     reinterpret_cast<hipStream_t>(stream));
}

size_t flare_project_workspace_size(int C_in, int C_out, int n_proj) {
  if (!proj_shape_ok(1, C_in, C_out, n_proj)) return 0;
  return proj_ws(C_in, C_out, n_proj);
}

flare_status flare_project(const void* X, const void* const* W, void* const* Y, int n_proj, int64_t R,
                           int C_in, int C_out, int out_head_major, int B, int head_dim,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!proj_shape_ok(R, C_in, C_out, n_proj)) {
    if (R >= 1 && n_proj >= 1 && n_proj <= 5 && C_in > 0 && C_out > 0) return FLARE_E_UNSUPPORTED;
    return FLARE_E_INVALID;
  }
  if (!X || !W || !Y || reinterpret_cast<uintptr_t>(X) % 16) return FLARE_E_INVALID;
  for (int i = 0; i < n_proj; ++i)
    if (!W[i] || !Y[i] || reinterpret_cast<uintptr_t>(W[i]) % 2 || reinterpret_cast<uintptr_t>(Y[i]) % 16)
      return FLARE_E_INVALID;
  if (out_head_major) {
    if (B < 1 || R % B || (head_dim != 16 && head_dim != 32) || C_out % head_dim) return FLARE_E_INVALID;
  }
  if (!workspace || workspace_bytes < proj_ws(C_in, C_out, n_proj) ||
      reinterpret_cast<uintptr_t>(workspace) % 16)
    return FLARE_E_WORKSPACE;
  return project_impl(X, W, Y, n_proj, R, C_in, C_out, out_head_major, B, head_dim, workspace,
                      reinterpret_cast<hipStream_t>(stream));
}

// Workspace of flare_mix, in order: K, V (, eK, eV) head-major bf16;
// Q(X) fp32 (dynamic); Z fp32; Y bf16 (with W_O); swizzled input weights;
// swizzled W_O; encoder split partials; with W_O, the fused output
// projection's latent operands and W_O^T.
namespace {
struct MixLayout {
  size_t kv, qx, z, y, wsw, wosw, enc, wof, total;
  bool fold;  // the encoder's split results are small enough for the decoder to merge
};
static MixLayout mix_layout(int B, int64_t N, int C, int H, int M, int dynamic, int has_wo) {
  MixLayout L;
  const int D = C / H;
  const size_t act = align_up((size_t)B * N * C * 2);
  const int n_in = dynamic ? 4 : 2;
  const size_t lat = align_up((size_t)B * H * M * D * 4);
  size_t off = 0;
  L.kv = off;
  off += n_in * act;
  L.qx = off;
  off += dynamic ? lat : 0;
  L.z = off;
  off += lat;
  L.y = off;
  off += has_wo ? act : 0;
  L.wsw = off;
  off += proj_ws(C, C, n_in);
  L.wosw = off;
  off += has_wo ? proj_ws(C, C, 1) : 0;
  L.enc = off;
  off += encode_ws(B, H, M, N, D, 0);
  // Small split sets (at most kConsumerMergeBytes of split results per batch
  // x head, and room for the merged Z in the decoder's LDS): the decoder
  // merges the encoder's split results while staging Z, in place of a merge
  // launch.  (The synthesis keeps its merge launch: every split workgroup of
  // the encoder would merge the same queries again.)
  const EncodePlan pl = plan_encode(B, H, M, N, D, 0);
  L.fold = (int64_t)pl.S * M * (D + 1) * 4 <= kConsumerMergeBytes &&
           decode_bf16_lds(M, D) + decode_merge_lds(M, D) <= 160 * 1024;
  // the fused output projection's prepared operands (reserved whenever W_O
  // is given, so the size does not depend on the flags)
  L.wof = off;
  off += has_wo ? align_up(decode_wo_scratch(B, H, M)) : 0;
  L.total = off;
  return L;
}
static bool mix_shape_ok(int B, int64_t N, int C, int H, int M) {
  if (B < 1 || N < 1 || C < 1 || H < 1 || M < 1 || C % H) return false;
  return sizes_ok(B, H, M, N, C / H) && (C == 32 || C == 64 || C == 128 || C == 256) &&
         ((int64_t)B * N + 255) / 256 <= 0x7fffffff;
}
}  // namespace

size_t flare_mix_workspace_size(int B, int64_t N, int C, int H, int M, int dynamic, int has_wo) {
  if (!mix_shape_ok(B, N, C, H, M)) return 0;
  return mix_layout(B, N, C, H, M, dynamic != 0, has_wo != 0).total;
}

flare_status flare_mix(const void* X, const void* W_K, const void* W_V, const void* W_eK,
                       const void* W_eV, const void* Q_or_seeds, const void* W_O, void* out,
                       int dtype, int B, int64_t N, int C, int H, int M, float scale,
                       unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || N < 1 || C < 1 || H < 1 || M < 1 || C % H) return FLARE_E_INVALID;
  if (!is_dtype(dtype)) return FLARE_E_INVALID;
  if (dtype != FLARE_BF16 || !mix_shape_ok(B, N, C, H, M)) return FLARE_E_UNSUPPORTED;
  if (!X || !W_K || !W_V || !Q_or_seeds || !out) return FLARE_E_INVALID;
  if ((W_eK == nullptr) != (W_eV == nullptr)) return FLARE_E_INVALID;
  if (reinterpret_cast<uintptr_t>(X) % 16 || reinterpret_cast<uintptr_t>(out) % 16) return FLARE_E_INVALID;
  if (!scale_ok(scale) || (flags & ~(FLARE_FLAG_EXACT_SOFTMAX | FLARE_MIX_FUSED_WO))) return FLARE_E_INVALID;
  const int dynamic = W_eK != nullptr, has_wo = W_O != nullptr;
  const MixLayout L = mix_layout(B, N, C, H, M, dynamic, has_wo);
  if (!workspace || workspace_bytes < L.total || reinterpret_cast<uintptr_t>(workspace) % 256)
    return FLARE_E_WORKSPACE;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int D = C / H;
  const float c = log2_scale(scale, D);
  char* ws = reinterpret_cast<char*>(workspace);
  const size_t act = align_up((size_t)B * N * C * 2);
  void* kp = ws + L.kv;
  void* vp = ws + L.kv + act;
  // FLARE++ with shared projections (the synthesis reuses K and V) when the
  // caller passes the same weights for both pairs: two projections, not four.
  const bool shared = dynamic && W_eK == W_K && W_eV == W_V;
  void* ekp = shared ? kp : ws + L.kv + 2 * act;
  void* evp = shared ? vp : ws + L.kv + 3 * act;

  // (a) projections, written head-major [B, H, N, D]
  const void* w_in[4] = {W_K, W_V, W_eK, W_eV};
  void* y_in[4] = {kp, vp, ekp, evp};
  flare_status s = project_impl(X, w_in, y_in, dynamic && !shared ? 4 : 2, (int64_t)B * N, C, C, 1, B, D,
                                ws + L.wsw, st);
  if (s != FLARE_OK) return s;

  auto head_major = [&](void* p) {
    View v;
    v.data = p;
    v.is_f32 = 0;
    v.sb = (int64_t)H * N * D;
    v.sh = N * D;
    v.sl = D;
    return v;
  };
  View qs;
  qs.data = Q_or_seeds;
  qs.is_f32 = 0;
  qs.sb = 0;
  qs.sh = (int64_t)M * D;
  qs.sl = D;
  View q = qs;
  const int64_t lat_sb = (int64_t)H * M * D, lat_sh = (int64_t)M * D, lat_sl = D;
  const bool fused_wo = has_wo && (flags & FLARE_MIX_FUSED_WO) && D == 32 && (H == 4 || H == 8);
  View z;
  z.data = ws + L.z;
  z.is_f32 = 1;
  z.sb = lat_sb;
  z.sh = lat_sh;
  z.sl = lat_sl;
  // (b) FLARE++: Q(X) = SDPA(seeds, eK, eV), kept in fp32
  if (dynamic) {
    s = encode_impl(qs, head_major(ekp), head_major(evp), ws + L.qx, 1, lat_sb, lat_sh, lat_sl, nullptr,
                    B, H, M, N, D, c, flags, ws + L.enc, st);
    if (s != FLARE_OK) return s;
    q.data = ws + L.qx;
    q.is_f32 = 1;
    q.sb = lat_sb;
    q.sh = lat_sh;
    q.sl = lat_sl;
  }
  // (c) Z = SDPA(Q, K, V); for small split sets the decoder merges the split
  // results while staging Z (no merge launch)
  if (L.fold && !fused_wo) {
    s = encode_splits(q, head_major(kp), head_major(vp), B, H, M, N, D, c, flags, ws + L.enc, st);
    if (s != FLARE_OK) return s;
    const EncodePlan pl = plan_encode(B, H, M, N, D, 0);
    const float* part_o = reinterpret_cast<const float*>(ws + L.enc);
    const float* part_l = reinterpret_cast<const float*>(ws + L.enc + align_up((size_t)B * H * pl.S * M * D * 4));
    void* ydst = has_wo ? (void*)(ws + L.y) : out;
    s = decode_impl(head_major(kp), q, z, ydst, 0, N * C, D, C, nullptr, B, H, M, N, D, c, flags, st, part_o, part_l,
                    pl.S);
    if (s != FLARE_OK) return s;
    if (has_wo) {
      const void* wo[1] = {W_O};
      void* yo[1] = {out};
      s = project_impl(ws + L.y, wo, yo, 1, (int64_t)B * N, C, C, 0, B, D, ws + L.wosw, st);
    }
    return s;
  }
  s = encode_impl(q, head_major(kp), head_major(vp), ws + L.z, 1, lat_sb, lat_sh, lat_sl, nullptr, B,
                  H, M, N, D, c, flags, ws + L.enc, st);
  if (s != FLARE_OK) return s;
  // (d, e) fused: out = [SDPA(K_h, Q_h, Z_h)]_h W_O in one pass
  if (fused_wo) {
    DecodeWoParams dw;
    std::memset(&dw, 0, sizeof(dw));
    dw.k = head_major(kp);
    dw.q = q;
    dw.z = z;
    dw.lat_ops = reinterpret_cast<unsigned char*>(ws + L.wof);
    dw.wt = dw.lat_ops + (size_t)B * H * ((M + 31) / 32) * 4096;
    dw.out = out;
    dw.H = H;
    dw.M = M;
    dw.N = N;
    dw.c = c;
    dw.exact = (flags & FLARE_FLAG_EXACT_SOFTMAX) ? 1 : 0;
    return hip_status(launch_decode_wo(dw, B, W_O, st));
  }
  // (d) Y = SDPA(K, Q, Z), heads concatenated into [B, N, C]
  void* ydst = has_wo ? (void*)(ws + L.y) : out;
  s = decode_impl(head_major(kp), q, z, ydst, 0, N * C, D, C, nullptr, B, H, M, N, D, c, flags, st);
  if (s != FLARE_OK) return s;
  // (e) out = Y W_O
  if (has_wo) {
    const void* wo[1] = {W_O};
    void* yo[1] = {out};
    s = project_impl(ws + L.y, wo, yo, 1, (int64_t)B * N, C, C, 0, B, D, ws + L.wosw, st);
  }
  return s;
}

// ---------------------------------------------------------------- backward

size_t flare_decode_backward_workspace_size(int B, int H, int M, int64_t N, int D) {
  if (!sizes_ok(B, H, M, N, D)) return 0;
  const int S = plan_bwd_splits(B, H, M, N);
  const size_t part = align_up((size_t)B * H * S * M * D * 4);
  return align_up((size_t)B * H * N * 4) + 2 * part;
}

size_t flare_encode_backward_workspace_size(int B, int H, int M, int64_t N, int D) {
  if (!sizes_ok(B, H, M, N, D)) return 0;
  const int S = plan_bwd_splits(B, H, M, N);
  return align_up((size_t)B * H * S * M * D * 4);
}

flare_status flare_decode_backward(const flare_tensor* K, const flare_tensor* Q, const flare_tensor* Z,
                                   const flare_tensor* Y, const float* lse, const flare_tensor* dY,
                                   const flare_tensor* dK, float* dQ, float* dZ, unsigned flags, int B,
                                   int H, int M, int64_t N, int D, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  flare_status v = bwd_common_checks(B, H, M, N, D, scale);
  if (v != FLARE_OK) return v;
  if (!token_tensor_ok(K) || !token_tensor_ok(Y) || !token_tensor_ok(dY) || !token_tensor_ok(dK) ||
      !latent_tensor_ok(Q) || !latent_tensor_ok(Z))
    return FLARE_E_INVALID;
  if (K->dtype != FLARE_BF16 || Y->dtype != FLARE_BF16 || dY->dtype != FLARE_BF16 || !grad_dtype_ok(dK->dtype))
    return FLARE_E_UNSUPPORTED;
  if (!f32_ptr_ok(lse) || !f32_ptr_ok(dQ) || !f32_ptr_ok(dZ)) return FLARE_E_INVALID;
  if (flags & ~kBwdFlags) return FLARE_E_INVALID;
  const size_t need = flare_decode_backward_workspace_size(B, H, M, N, D);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256)
    return FLARE_E_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int S = plan_bwd_splits(B, H, M, N);
  char* ws = reinterpret_cast<char*>(workspace);
  float* delta = reinterpret_cast<float*>(ws);
  float* dq_part = reinterpret_cast<float*>(ws + align_up((size_t)B * H * N * 4));
  float* dz_part = dq_part + align_up((size_t)B * H * S * M * D * 4) / 4;

  TokBwdParams tp;
  std::memset(&tp, 0, sizeof(tp));
  tp.k = view_of(K);
  tp.x = view_of(dY);
  tp.y = view_of(Y);
  tp.q = view_of(Q);
  tp.w = view_of(Z);
  tp.z = tp.w;
  tp.lse = lse;
  tp.dk = dK->data;
  tp.grad_bf16 = dK->dtype == FLARE_BF16;
  tp.dk_sb = dK->stride_b;
  tp.dk_sh = dK->stride_h;
  tp.dk_sl = dK->stride_l;
  tp.delta = delta;
  tp.H = H;
  tp.M = M;
  tp.N = N;
  tp.c = log2_scale(scale, D);
  tp.scale = natural_scale(scale, D);
  tp.accumulate = (flags & FLARE_ACCUMULATE_DK) ? 1 : 0;
  tp.blocks_per_head = tok_bwd_blocks(B, H, N, 256, 2048);
  hipError_t e = launch_tok_bwd(tp, D, B, false, st);
  if (e != hipSuccess) return FLARE_E_HIP;

  LatBwdParams lp;
  std::memset(&lp, 0, sizeof(lp));
  lp.k = tp.k;
  lp.x = tp.x;
  lp.q = tp.q;
  lp.w = tp.w;
  lp.z = tp.w;
  lp.lse = lse;
  lp.delta = delta;
  lp.dq_part = dq_part;
  lp.dz_part = dz_part;
  lp.H = H;
  lp.M = M;
  lp.S = S;
  lp.N = N;
  lp.c = tp.c;
  if ((e = launch_lat_bwd(lp, D, B, false, st)) != hipSuccess) return FLARE_E_HIP;
  if ((e = launch_sum_splits(dq_part, dQ, B, H, S, (int64_t)M * D, (flags & FLARE_SUM_DQ_OVER_BATCH) != 0,
                             tp.scale, (flags & FLARE_ACCUMULATE_DQ) ? 1 : 0, st)) != hipSuccess)
    return FLARE_E_HIP;
  if ((e = launch_sum_splits(dz_part, dZ, B, H, S, (int64_t)M * D, false, 1.0f, 0, st)) != hipSuccess)
    return FLARE_E_HIP;
  return FLARE_OK;
}

flare_status flare_encode_backward(const flare_tensor* Q, const flare_tensor* K, const flare_tensor* V,
                                   const flare_tensor* Z, const float* lse, const float* dZ, float* dQ,
                                   const flare_tensor* dK, const flare_tensor* dV, unsigned flags,
                                   int B, int H, int M, int64_t N, int D, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  flare_status v = bwd_common_checks(B, H, M, N, D, scale);
  if (v != FLARE_OK) return v;
  if (!token_tensor_ok(K) || !token_tensor_ok(V) || !token_tensor_ok(dK) || !token_tensor_ok(dV) ||
      !latent_tensor_ok(Q) || !latent_tensor_ok(Z))
    return FLARE_E_INVALID;
  if (K->dtype != FLARE_BF16 || V->dtype != FLARE_BF16 || !grad_dtype_ok(dK->dtype) || dV->dtype != dK->dtype)
    return FLARE_E_UNSUPPORTED;
  if (!f32_ptr_ok(lse) || !f32_ptr_ok(dZ) || !f32_ptr_ok(dQ)) return FLARE_E_INVALID;
  if (flags & ~kBwdFlags) return FLARE_E_INVALID;
  const size_t need = flare_encode_backward_workspace_size(B, H, M, N, D);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256)
    return FLARE_E_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int S = plan_bwd_splits(B, H, M, N);
  float* dq_part = reinterpret_cast<float*>(workspace);

  View dzv;
  dzv.data = dZ;
  dzv.is_f32 = 1;
  dzv.sb = (int64_t)H * M * D;
  dzv.sh = (int64_t)M * D;
  dzv.sl = D;

  LatBwdParams lp;
  std::memset(&lp, 0, sizeof(lp));
  lp.k = view_of(K);
  lp.x = view_of(V);
  lp.q = view_of(Q);
  lp.w = dzv;
  lp.z = view_of(Z);
  lp.lse = lse;
  lp.dq_part = dq_part;
  lp.H = H;
  lp.M = M;
  lp.S = S;
  lp.N = N;
  lp.c = log2_scale(scale, D);
  hipError_t e = launch_lat_bwd(lp, D, B, true, st);
  if (e != hipSuccess) return FLARE_E_HIP;
  if ((e = launch_sum_splits(dq_part, dQ, B, H, S, (int64_t)M * D, (flags & FLARE_SUM_DQ_OVER_BATCH) != 0,
                             natural_scale(scale, D), (flags & FLARE_ACCUMULATE_DQ) ? 1 : 0, st)) !=
      hipSuccess)
    return FLARE_E_HIP;

  TokBwdParams tp;
  std::memset(&tp, 0, sizeof(tp));
  tp.k = lp.k;
  tp.x = lp.x;
  tp.q = lp.q;
  tp.w = dzv;
  tp.z = lp.z;
  tp.lse = lse;
  tp.dk = dK->data;
  tp.grad_bf16 = dK->dtype == FLARE_BF16;
  tp.dk_sb = dK->stride_b;
  tp.dk_sh = dK->stride_h;
  tp.dk_sl = dK->stride_l;
  tp.dv = dV->data;
  tp.dv_sb = dV->stride_b;
  tp.dv_sh = dV->stride_h;
  tp.dv_sl = dV->stride_l;
  tp.H = H;
  tp.M = M;
  tp.N = N;
  tp.c = lp.c;
  tp.scale = natural_scale(scale, D);
  tp.accumulate = (flags & FLARE_ACCUMULATE_DK) ? 1 : 0;
  tp.blocks_per_head = tok_bwd_blocks(B, H, N, 512, 512);
  if ((e = launch_tok_bwd(tp, D, B, true, st)) != hipSuccess) return FLARE_E_HIP;
  return FLARE_OK;
}

size_t flare_encdec_backward_workspace_size(int B, int H, int M, int64_t N, int D) {
  if (!sizes_ok(B, H, M, N, D)) return 0;
  const size_t dz = align_up((size_t)B * H * M * D * 4);
  const size_t rest = std::max(flare_decode_backward_workspace_size(B, H, M, N, D),
                               flare_encode_backward_workspace_size(B, H, M, N, D));
  return dz + rest;
}

flare_status flare_encdec_backward(const flare_tensor* Q, const flare_tensor* K, const flare_tensor* V,
                                   const flare_tensor* Z, const float* lse_enc, const flare_tensor* Y,
                                   const float* lse_dec, const flare_tensor* dY, float* dQ,
                                   const flare_tensor* dK, const flare_tensor* dV, unsigned flags, int B,
                                   int H, int M, int64_t N, int D, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  flare_status v = bwd_common_checks(B, H, M, N, D, scale);
  if (v != FLARE_OK) return v;
  if (!token_tensor_ok(K) || !token_tensor_ok(V) || !token_tensor_ok(Y) || !token_tensor_ok(dY) ||
      !token_tensor_ok(dK) || !token_tensor_ok(dV) || !latent_tensor_ok(Q) || !latent_tensor_ok(Z))
    return FLARE_E_INVALID;
  if (K->dtype != FLARE_BF16 || V->dtype != FLARE_BF16 || Y->dtype != FLARE_BF16 || dY->dtype != FLARE_BF16 ||
      !grad_dtype_ok(dK->dtype) || dV->dtype != dK->dtype)
    return FLARE_E_UNSUPPORTED;
  if (!f32_ptr_ok(lse_enc) || !f32_ptr_ok(lse_dec) || !f32_ptr_ok(dQ)) return FLARE_E_INVALID;
  if (flags & ~kBwdFlags) return FLARE_E_INVALID;
  const size_t need = flare_encdec_backward_workspace_size(B, H, M, N, D);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256)
    return FLARE_E_WORKSPACE;
  char* ws = reinterpret_cast<char*>(workspace);
  float* dZ = reinterpret_cast<float*>(ws);
  char* rest = ws + align_up((size_t)B * H * M * D * 4);
  const size_t rest_bytes = workspace_bytes - align_up((size_t)B * H * M * D * 4);
  const unsigned q_sum = flags & FLARE_SUM_DQ_OVER_BATCH;
  if (M > kTokPairMaxM) {
    // the pair pass's latent operands would not fit one CU's LDS: the two
    // calls one after the other, the encoder's dQ and dK added on
    flare_status st = flare_decode_backward(K, Q, Z, Y, lse_dec, dY, dK, dQ, dZ, flags, B, H, M, N, D, scale,
                                            rest, rest_bytes, stream);
    if (st != FLARE_OK) return st;
    return flare_encode_backward(Q, K, V, Z, lse_enc, dZ, dQ, dK, dV,
                                 FLARE_ACCUMULATE_DQ | FLARE_ACCUMULATE_DK | q_sum, B, H, M, N, D, scale, rest,
                                 rest_bytes, stream);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int S = plan_bwd_splits(B, H, M, N);
  float* delta = reinterpret_cast<float*>(rest);
  float* dq_part = reinterpret_cast<float*>(rest + align_up((size_t)B * H * N * 4));
  float* dz_part = dq_part + align_up((size_t)B * H * S * M * D * 4) / 4;
  const float c = log2_scale(scale, D), sc = natural_scale(scale, D);
  const int64_t MD = (int64_t)M * D;

  // (1) latent pass of the decoder: dQ, dZ partials; delta = dY . Y
  LatBwdParams lp;
  std::memset(&lp, 0, sizeof(lp));
  lp.k = view_of(K);
  lp.x = view_of(dY);
  lp.y = view_of(Y);
  lp.q = view_of(Q);
  lp.w = view_of(Z);
  lp.z = lp.w;
  lp.lse = lse_dec;
  lp.delta_out = delta;
  lp.dq_part = dq_part;
  lp.dz_part = dz_part;
  lp.H = H;
  lp.M = M;
  lp.S = S;
  lp.N = N;
  lp.c = c;
  hipError_t e = launch_lat_bwd(lp, D, B, false, st);
  if (e != hipSuccess) return FLARE_E_HIP;
  if ((e = launch_sum_splits(dz_part, dZ, B, H, S, MD, false, 1.0f, 0, st)) != hipSuccess) return FLARE_E_HIP;
  if ((e = launch_sum_splits(dq_part, dQ, B, H, S, MD, q_sum != 0, sc, (flags & FLARE_ACCUMULATE_DQ) ? 1 : 0,
                             st)) != hipSuccess)
    return FLARE_E_HIP;

  // (2) latent pass of the encoder with dZ: its dQ added on
  View dzv;
  dzv.data = dZ;
  dzv.is_f32 = 1;
  dzv.sb = (int64_t)H * MD;
  dzv.sh = MD;
  dzv.sl = D;
  LatBwdParams le;
  std::memset(&le, 0, sizeof(le));
  le.k = view_of(K);
  le.x = view_of(V);
  le.q = view_of(Q);
  le.w = dzv;
  le.z = view_of(Z);
  le.lse = lse_enc;
  le.dq_part = dq_part;
  le.H = H;
  le.M = M;
  le.S = S;
  le.N = N;
  le.c = c;
  if ((e = launch_lat_bwd(le, D, B, true, st)) != hipSuccess) return FLARE_E_HIP;
  if ((e = launch_sum_splits(dq_part, dQ, B, H, S, MD, q_sum != 0, sc, 1, st)) != hipSuccess) return FLARE_E_HIP;

  // (3) token pass of both roles: dK, dV
  TokPairParams tp;
  std::memset(&tp, 0, sizeof(tp));
  tp.k = view_of(K);
  tp.v = view_of(V);
  tp.dy = view_of(dY);
  tp.q = view_of(Q);
  tp.z = view_of(Z);
  tp.dz = dzv;
  tp.lse_e = lse_enc;
  tp.lse_d = lse_dec;
  tp.delta_d = delta;
  tp.dk = dK->data;
  tp.grad_bf16 = dK->dtype == FLARE_BF16;
  tp.dk_sb = dK->stride_b;
  tp.dk_sh = dK->stride_h;
  tp.dk_sl = dK->stride_l;
  tp.dv = dV->data;
  tp.dv_sb = dV->stride_b;
  tp.dv_sh = dV->stride_h;
  tp.dv_sl = dV->stride_l;
  tp.H = H;
  tp.M = M;
  tp.N = N;
  tp.c = c;
  tp.scale = sc;
  tp.accumulate = (flags & FLARE_ACCUMULATE_DK) ? 1 : 0;
  tp.blocks_per_head = tok_pair_blocks(B, H, N);
  if ((e = launch_tok_pair(tp, D, B, st)) != hipSuccess) return FLARE_E_HIP;
  return FLARE_OK;
}

}  // extern "C"
