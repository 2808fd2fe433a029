/*
 * flare.h - C ABI of the MI355X (gfx950) FLARE / FLARE++ token-mixer library.
 *
 * The operator (page "FLARE++: Low-Rank Attention with Dynamic Attention
 * Routing", section 3, Method):
 *   - every step is one scaled dot-product attention (SDPA) call,
 *     SDPA(Q, K, V) = softmax(scale * Q K^T) V with the softmax along each
 *     query's row ("Full self-attention");
 *   - FLARE encode:  Z_h = SDPA(Q_h, K_h, V_h), M latents gather N tokens;
 *     FLARE decode:  Y_h = SDPA(K_h, Q_h, Z_h), the latents are sent back
 *     ("FLARE: fixed-query latent routing", equation 5 is the encoder);
 *   - FLARE++ query synthesis: Q_h(X) = SDPA(seeds_h, eK_h, eV_h) with learned
 *     per-head seeds and the extra projections eK = X W_eK, eV = X W_eV
 *     ("FLARE++: dynamic token routing", equations 7 and 8);
 *   - the encoder exposes its row log-normaliser, which makes a token-split
 *     encode mergeable exactly by logsumexp ("Multi-GPU context parallelism").
 *
 * Conventions shared by every call:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; scratch comes from a caller
 *     workspace sized by the matching *_workspace_size function.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream).  Outputs are ready when the stream reaches
 *     that point.  Calls are thread-safe; the library holds no mutable state.
 *   - Argument errors are reported synchronously, before anything is
 *     launched, and leave every output untouched.  FLARE_E_HIP means a launch
 *     failed; outputs are then undefined.
 *   - Sizes: B >= 1, H >= 1, 1 <= M <= 512, N >= 1, D in {16, 32}.
 *   - scale: multiplier of the dot products inside the softmax; 0 selects the
 *     pages' 1/sqrt(D).  Any other finite value is used as given.
 *   - Precision: bf16 inputs are multiplied on bf16 matrix cores with fp32
 *     accumulation and an fp32 softmax; fp32 inputs run an all-fp32 path.
 */
#ifndef FLARE_H
#define FLARE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum flare_status {
  FLARE_OK = 0,
  FLARE_E_INVALID = -1,     /* null pointer, size out of range, bad stride/alignment */
  FLARE_E_UNSUPPORTED = -2, /* valid request outside what the library implements */
  FLARE_E_WORKSPACE = -3,   /* workspace NULL or smaller than required */
  FLARE_E_HIP = -4,         /* a HIP launch/runtime error */
  FLARE_E_SCRATCH = -5      /* sizes beyond flare_encode_static's static scratch */
} flare_status;

typedef enum flare_dtype { FLARE_F32 = 0, FLARE_BF16 = 1 } flare_dtype;

/* Force the exact running-maximum softmax in every kernel.  Without it the
 * kernels first try a range-checked form without the maximum and fall back
 * to the exact form for any token split (encoder) or token group (decoder)
 * in which a normaliser l summing n weights leaves [n 2^-102, 2^100]; inside
 * that range no weight overflows and the weights the exponential flushes to
 * zero carry less than 2^-24 of l, so both forms give the same softmax up to
 * fp32 rounding. */
#define FLARE_FLAG_EXACT_SOFTMAX 1u

/* flare_mix only: with W_O, apply the output projection in the decoder's
 * epilogue ("FLARE++: Low-Rank Attention with Dynamic Attention Routing",
 * section 3, "Full self-attention": out = [Y_1 ... Y_H] W_O) instead of
 * writing Y and projecting it in a second pass.  Taken when D = 32 and
 * C in {128, 256}; other shapes run the two-pass form.  Both give out within
 * the bf16 tolerance of the same result (they sum the projection in a
 * different order). */
#define FLARE_MIX_FUSED_WO 2u

/*
 * A [B, H, L, D] view of device memory: element (b, h, l, d) lives at
 *   data + b*stride_b + h*stride_h + l*stride_l + d     (in elements).
 * The last axis (D) is contiguous.  stride_b may be 0 (one block shared by
 * the batch, e.g. learned queries or seeds).  Token-major activations
 * [B, N, H*D] are stride_b = N*H*D, stride_h = D, stride_l = H*D; head-major
 * [B, H, N, D] are stride_b = H*N*D, stride_h = N*D, stride_l = D.
 * Requirements for token-side tensors (K, V, eK, eV, Y): data 16-byte
 * aligned; stride_h and stride_l multiples of 8 elements (bf16) or 4
 * elements (fp32); stride_b a multiple of the same or 0; stride_l below 2^22
 * elements (a 128-token tile is addressed with 32-bit byte offsets).
 * Latent-side tensors (Q, seeds, Z) need only element alignment.
 */
typedef struct flare_tensor {
  void* data;
  int32_t dtype; /* flare_dtype */
  int32_t reserved;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_l;
} flare_tensor;

/* Bytes of workspace flare_encode / flare_route_queries need (split-token
 * partial outputs and log-normalisers).  Depends only on the sizes. */
size_t flare_encode_workspace_size(int B, int H, int M, int64_t N, int D);

/*
 * FLARE encoder, Z[b,h] = SDPA(Q[b,h], K[b,h], V[b,h]): M latent queries
 * gather N tokens ("FLARE: fixed-query latent routing", equation 5).
 *   Q   [B, H, M, D]  bf16 or fp32 (stride_b 0 = shared by the batch)
 *   K,V [B, H, N, D]  bf16 (matrix-core path) or fp32 (fp32 path); same dtype
 *   Z   [B, H, M, D]  output, bf16 or fp32
 *   lse [B, H, M]     optional fp32 output (contiguous), the natural-log row
 *                     normaliser log sum_n exp(scale q_m . k_n); NULL = skip
 * The tokens are cut into splits that run in parallel; each split's partial
 * result is merged exactly by logsumexp ("Multi-GPU context parallelism",
 * applied inside one GPU).  Requires workspace_bytes >=
 * flare_encode_workspace_size(B, H, M, N, D).
 */
flare_status flare_encode(const flare_tensor* Q, const flare_tensor* K,
                          const flare_tensor* V, const flare_tensor* Z,
                          float* lse, int B, int H, int M, int64_t N, int D,
                          float scale, unsigned flags, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * FLARE++ query synthesis, Qx[b,h] = SDPA(seeds[h], eK[b,h], eV[b,h])
 * ("FLARE++: dynamic token routing", equation 8): the same encoder with the
 * learned seeds as queries.  seeds [H, M, D] (stride_b normally 0);
 * eK, eV [B, H, N, D]; Qx [B, H, M, D] output (fp32 keeps the synthesized
 * queries unrounded for the encode/decode that follow); lse [B, H, M]
 * optional fp32 output as in flare_encode (flare_encode_backward needs it),
 * NULL = skip.
 */
flare_status flare_route_queries(const flare_tensor* seeds,
                                 const flare_tensor* eK,
                                 const flare_tensor* eV,
                                 const flare_tensor* Qx, float* lse, int B,
                                 int H, int M, int64_t N, int D, float scale,
                                 unsigned flags,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * FLARE decoder, Y[b,h] = SDPA(K[b,h], Q[b,h], Z[b,h]): every token takes a
 * softmax over the M latents and gathers their values ("FLARE: fixed-query
 * latent routing", the second call).
 *   K [B, H, N, D]  bf16 or fp32;  Q, Z [B, H, M, D] bf16 or fp32
 *   Y [B, H, N, D]  output, same dtype as K (token-major strides give the
 *                   concatenated-heads [B, N, H*D] layout directly)
 *   lse [B, H, N]   optional fp32 output (contiguous), each token's natural-log
 *                   normaliser log sum_m exp(scale k_n . q_m); NULL = skip.
 *                   flare_decode_backward needs it.
 * Needs no workspace.
 */
flare_status flare_decode(const flare_tensor* K, const flare_tensor* Q,
                          const flare_tensor* Z, const flare_tensor* Y,
                          float* lse, int B, int H, int M, int64_t N, int D,
                          float scale, unsigned flags, void* stream);

/*
 * Pointwise projections of one token matrix, Y_p = X W_p for p < n_proj
 * ("Full self-attention": K = X W_K etc., weights [C_in, C_out] with y = x W,
 * no bias).  X [R, C_in] row-major bf16; each W_p [C_in, C_out] row-major
 * bf16; each Y_p bf16 written either row-major [R, C_out]
 * (out_head_major = 0) or head-major [B, H, N, D] with R = B*N and
 * C_out = H*D (out_head_major = 1, D = head_dim).  C_in in {32, 64, 128,
 * 256}; C_out a multiple of 32, at most 4096; 1 <= n_proj <= 5; X and every
 * Y_p 16-byte aligned (FLARE_E_UNSUPPORTED / FLARE_E_INVALID otherwise).
 * Workspace holds the weights rearranged into matrix-core operand order:
 * flare_project_workspace_size(C_in, C_out, n_proj) bytes.
 */
size_t flare_project_workspace_size(int C_in, int C_out, int n_proj);
flare_status flare_project(const void* X, const void* const* W, void* const* Y,
                           int n_proj, int64_t R, int C_in, int C_out,
                           int out_head_major, int B, int head_dim,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * The whole mixer on a token matrix X [B, N, C], C = H*D, bf16:
 *   FLARE   (W_eK == NULL): K = X W_K, V = X W_V; Q_or_seeds [H, M, D] are
 *           the learned queries; Z = SDPA(Q, K, V); Y = SDPA(K, Q, Z).
 *   FLARE++ (W_eK != NULL): also eK = X W_eK, eV = X W_eV; Q_or_seeds are the
 *           seeds and Q(X) = SDPA(seeds, eK, eV) replaces the learned queries
 *           in both the encode and the decode.  Passing W_eK == W_K and
 *           W_eV == W_V (the same pointers) selects the variant with shared
 *           projections: the synthesis attends over K and V themselves and
 *           only two input projections run.
 * Heads are concatenated into out [B, N, C]; if W_O != NULL, out = Y W_O.
 * All weights [C, C] with y = x W.  dtype must be FLARE_BF16; C = H*D with
 * D in {16, 32} and C in {32, 64, 128, 256} (FLARE_E_UNSUPPORTED otherwise);
 * X and out 16-byte aligned; Q_or_seeds [H, M, D] bf16, contiguous.
 * flags: FLARE_FLAG_EXACT_SOFTMAX, FLARE_MIX_FUSED_WO.
 * Requires a 256-byte aligned workspace of workspace_bytes >=
 * flare_mix_workspace_size(B, N, C, H, M, W_eK != NULL, W_O != NULL).
 */
size_t flare_mix_workspace_size(int B, int64_t N, int C, int H, int M,
                                int dynamic, int has_wo);
flare_status flare_mix(const void* X, const void* W_K, const void* W_V,
                       const void* W_eK, const void* W_eV,
                       const void* Q_or_seeds, const void* W_O, void* out,
                       int dtype, int B, int64_t N, int C, int H, int M,
                       float scale, unsigned flags, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Backward of the two calls.  Each call is standard SDPA ("FLARE:
 * fixed-query latent routing"; the query synthesis of "FLARE++: dynamic
 * token routing", equation 8, is the encoder again), so with
 * s = scale q . k, P the softmax weights, o the output and do its gradient:
 *   delta = do . o per query row,  dS = P (do . v - delta),
 *   dq = scale sum dS k,  dk = scale sum dS q,  dv = sum P do.
 * P is recomputed from the normaliser the forward call returned (lse).
 * Token-side inputs (K, V, Y, dY) must be bf16; token-side gradients (dK,
 * dV) are [B, H, N, D] views in fp32 or bf16, both of one dtype (bf16
 * gradients are formed in fp32 and rounded once when written; accumulation
 * adds the stored value in fp32 before that rounding); dZ and dQ are
 * contiguous fp32 arrays,
 * dZ [B, H, M, D], dQ [B, H, M, D] or, with FLARE_SUM_DQ_OVER_BATCH, [H, M, D]
 * holding the sum over the batch (the gradient of a query block shared by
 * the batch: FLARE's learned queries, FLARE++'s seeds).
 * FLARE_E_UNSUPPORTED for other dtypes; FLARE_E_INVALID for unknown flags.
 * Flags:
 *   FLARE_ACCUMULATE_DQ      add into dQ instead of overwriting it
 *   FLARE_ACCUMULATE_DK      add into dK instead of overwriting it
 *   FLARE_SUM_DQ_OVER_BATCH  dQ is [H, M, D] and receives the sum over b
 * The first two carry the chain rule through a decoder and an encoder that
 * share Q and K.  Calls on one stream are ordered; accumulation assumes no
 * other call writes the same dQ / dK concurrently.
 */
#define FLARE_ACCUMULATE_DQ 1u
#define FLARE_ACCUMULATE_DK 2u
#define FLARE_SUM_DQ_OVER_BATCH 4u

/* Decoder: gradients of Y = SDPA(K, Q, Z) given dY.  lse is flare_decode's
 * [B, H, N] output for the same inputs.  Writes dK, dQ (per the flags) and
 * dZ (always overwritten). */
size_t flare_decode_backward_workspace_size(int B, int H, int M, int64_t N,
                                            int D);
flare_status flare_decode_backward(const flare_tensor* K, const flare_tensor* Q,
                                   const flare_tensor* Z, const flare_tensor* Y,
                                   const float* lse, const flare_tensor* dY,
                                   const flare_tensor* dK, float* dQ, float* dZ,
                                   unsigned flags, int B, int H, int M,
                                   int64_t N, int D, float scale,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Encoder and FLARE++ query synthesis: gradients of Z = SDPA(Q, K, V) given
 * dZ.  lse is the [B, H, M] output of the forward call (flare_encode or
 * flare_route_queries).  Writes dQ and dK per the flags and dV (always
 * overwritten). */
size_t flare_encode_backward_workspace_size(int B, int H, int M, int64_t N,
                                            int D);
flare_status flare_encode_backward(const flare_tensor* Q, const flare_tensor* K,
                                   const flare_tensor* V, const flare_tensor* Z,
                                   const float* lse, const float* dZ, float* dQ,
                                   const flare_tensor* dK, const flare_tensor* dV,
                                   unsigned flags, int B, int H, int M,
                                   int64_t N, int D, float scale,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* The FLARE pair, Z = SDPA(Q, K, V) then Y = SDPA(K, Q, Z) ("FLARE:
 * fixed-query latent routing"): dQ, dK, dV of sum(dY * Y) through both calls
 * in one call.  It equals flare_decode_backward followed by
 * flare_encode_backward with FLARE_ACCUMULATE_DQ | FLARE_ACCUMULATE_DK, but
 * the two token-side passes share their score products and dK is written
 * once.
 *   Q, Z, lse_enc   flare_encode's inputs and outputs (Z as flare_decode used
 *                   it); lse_enc [B, H, M]
 *   Y, lse_dec      flare_decode's output and its [B, H, N] normalisers
 *   dY              upstream gradient of Y (bf16, like K, V, Y)
 *   dQ              fp32 [B, H, M, D] (or [H, M, D] with
 *                   FLARE_SUM_DQ_OVER_BATCH); dK, dV [B, H, N, D] views, both fp32
 *                   or both bf16
 * Flags as for the two calls (accumulation into dQ / dK, batch sum of dQ).
 * M above 256 runs the two calls internally.  Workspace:
 * flare_encdec_backward_workspace_size bytes, 256-byte aligned. */
size_t flare_encdec_backward_workspace_size(int B, int H, int M, int64_t N,
                                            int D);
flare_status flare_encdec_backward(const flare_tensor* Q, const flare_tensor* K,
                                   const flare_tensor* V, const flare_tensor* Z,
                                   const float* lse_enc, const flare_tensor* Y,
                                   const float* lse_dec, const flare_tensor* dY,
                                   float* dQ, const flare_tensor* dK,
                                   const flare_tensor* dV, unsigned flags,
                                   int B, int H, int M, int64_t N, int D,
                                   float scale, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * flare_encode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Arguments, layouts, results and errors are those of
 * flare_encode.  The split partials live in a static device array of
 * flare_encode_static_scratch_bytes() bytes (64 MiB), one per GPU, held from
 * the library's first use on that GPU until the process ends; the call itself
 * allocates nothing.  When the encoder's own split plan needs more, the call
 * uses fewer, longer splits (the merged result then differs from flare_encode's
 * by rounding only); when even one split per (batch, head) needs more
 * (B*H*M*(D+1)*4 bytes, rounded up to 256-byte blocks), it returns
 * FLARE_E_SCRATCH before launching anything.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, two host threads) race on it and must be ordered by the
 * caller.  The stream must belong to the current device.
 */
size_t flare_encode_static_scratch_bytes(void);
flare_status flare_encode_static(const flare_tensor* Q, const flare_tensor* K,
                                 const flare_tensor* V, const flare_tensor* Z,
                                 float* lse, int B, int H, int M, int64_t N,
                                 int D, float scale, unsigned flags,
                                 void* stream);

/* Static text for a status code. */
const char* flare_status_string(int status);

/* Library version as "major.minor.patch". */
const char* flare_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLARE_H */
