/*
 * flare_oracle.c - plain, slow, fp64 CPU oracle for the FLARE / FLARE++
 * low-rank token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can compare the HIP library against the
 * plain definition of what the method computes.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * Sources (page titles as published; sections named on the page):
 *   [P1] "FLARE++: Low-Rank Attention with Dynamic Attention Routing",
 *        section 3 (Method): "Full self-attention", "FLARE: fixed-query latent
 *        routing" (the encoder is its equation 5), "FLARE++: dynamic token
 *        routing" (equations 7 and 8), "Computational complexity",
 *        "Multi-GPU context parallelism".
 *   [P2] "FLARE: Fast Low-rank Attention Routing Engine" (abstract).
 *
 * Everything is double precision and uses libm exp/log.  Inputs arrive as
 * double arrays (bf16 and fp32 values widen to double exactly).  Every
 * matrix is (base pointer, row stride in elements) with contiguous rows, so
 * a head slice of a [N, C] token matrix is (base + h*D, C).
 *
 * OpenMP is used only across independent output rows; inside a row every sum
 * runs in index order.  No blocking, fusion or online rescaling: the softmax
 * is the two-pass stable form (maximum, then normalised exponentials), which
 * equals the textbook definition exactly in real arithmetic.
 *
 * Pins (tests/test_oracle_pins.py): library SDPA, closed forms, invariants
 * and brute force for every function.  The full FLARE++ mixer is pinned by
 * the composition of pinned parts, token-permutation equivariance and its
 * zero-synthesis special cases; beyond those it is parity unpinned (the pages
 * print no worked example of the mixer).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -2

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Scaled dot-product attention, the one primitive every step of the mixer
 * is built from ([P1] "Full self-attention": S = Q K^T / sqrt(D),
 * Y = softmax(S) V, the softmax taken along each query's row).
 *
 *   o[i, :] = sum_j softmax_j(scale * q_i . k_j) v_j      for i < Lq
 *   lse[i]  = log sum_j exp(scale * q_i . k_j)            (natural log)
 *
 * q is [Lq, D], k is [Lk, D], v is [Lk, Dv], o is [Lq, Dv]; lse may be NULL.
 * Lk == 0 (an empty key set, e.g. an empty shard in the context-parallel
 * merge) returns o = 0 and lse = -inf, the value whose merge weight is 0.
 */
int oracle_sdpa(const double* q, int64_t q_rs, const double* k, int64_t k_rs,
                const double* v, int64_t v_rs, double* o, int64_t o_rs,
                double* lse, int64_t Lq, int64_t Lk, int D, int Dv,
                double scale) {
  if (Lq < 0 || Lk < 0 || D <= 0 || Dv <= 0) return ORACLE_EINVAL;
  if (Lq == 0) return ORACLE_OK;
  if (Lk == 0) {
    for (int64_t i = 0; i < Lq; ++i) {
      for (int e = 0; e < Dv; ++e) o[i * o_rs + e] = 0.0;
      if (lse) lse[i] = -INFINITY;
    }
    return ORACLE_OK;
  }
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Lk);
    double* acc = (double*)malloc(sizeof(double) * (size_t)Dv);
    if (!s || !acc) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int64_t i = 0; i < Lq; ++i) {
      if (!s || !acc) continue;
      const double* qi = q + i * q_rs;
      /* scores of query i against every key */
      for (int64_t j = 0; j < Lk; ++j) {
        const double* kj = k + j * k_rs;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
        s[j] = scale * dot;
      }
      /* pass 1: the row maximum */
      double mx = s[0];
      for (int64_t j = 1; j < Lk; ++j) mx = s[j] > mx ? s[j] : mx;
      /* pass 2: exponentials, their sum, and the weighted sum of values */
      double l = 0.0;
      for (int e = 0; e < Dv; ++e) acc[e] = 0.0;
      for (int64_t j = 0; j < Lk; ++j) {
        double p = exp(s[j] - mx);
        l += p;
        const double* vj = v + j * v_rs;
        for (int e = 0; e < Dv; ++e) acc[e] += p * vj[e];
      }
      double* oi = o + i * o_rs;
      for (int e = 0; e < Dv; ++e) oi[e] = acc[e] / l;
      if (lse) lse[i] = mx + log(l);
    }
    free(s);
    free(acc);
  }
  return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Gradient of one SDPA call.  Training with the mixer runs it backwards
 * ([P1] "FLARE: fixed-query latent routing": encoder and decoder are
 * standard SDPA calls, so their gradients are the standard SDPA gradients).
 * With s_ij = scale q_i . k_j, P = softmax_j(s), o_i = sum_j P_ij v_j and an
 * upstream gradient do (of o), differentiating the definition gives
 *   delta_i = do_i . o_i
 *   dS_ij   = P_ij (do_i . v_j - delta_i)          (gradient of s_ij)
 *   dq_i    = scale sum_j dS_ij k_j
 *   dk_j    = scale sum_i dS_ij q_i
 *   dv_j    = sum_i P_ij do_i
 * Three passes: row statistics (P recomputed with the two-pass softmax,
 * o, delta), then dq by rows, then dk and dv by keys.  Nothing is
 * materialised beyond two doubles per row.
 */
int oracle_sdpa_backward(const double* q, int64_t q_rs, const double* k, int64_t k_rs,
                         const double* v, int64_t v_rs, const double* dout, int64_t do_rs,
                         double* dq, int64_t dq_rs, double* dk, int64_t dk_rs, double* dv,
                         int64_t dv_rs, int64_t Lq, int64_t Lk, int D, int Dv, double scale) {
  if (Lq <= 0 || Lk <= 0 || D <= 0 || Dv <= 0) return ORACLE_EINVAL;
  double* lse = (double*)malloc(sizeof(double) * (size_t)Lq);
  double* delta = (double*)malloc(sizeof(double) * (size_t)Lq);
  if (!lse || !delta) {
    free(lse);
    free(delta);
    return ORACLE_ENOMEM;
  }
  int failed = 0;
  /* pass 1: per row, the log-normaliser and delta = do . o */
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Lk);
    double* o = (double*)malloc(sizeof(double) * (size_t)Dv);
    if (!s || !o) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int64_t i = 0; i < Lq; ++i) {
      if (!s || !o) continue;
      const double* qi = q + i * q_rs;
      for (int64_t j = 0; j < Lk; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qi[d] * k[j * k_rs + d];
        s[j] = scale * dot;
      }
      double mx = s[0];
      for (int64_t j = 1; j < Lk; ++j) mx = s[j] > mx ? s[j] : mx;
      double l = 0.0;
      for (int e = 0; e < Dv; ++e) o[e] = 0.0;
      for (int64_t j = 0; j < Lk; ++j) {
        const double p = exp(s[j] - mx);
        l += p;
        for (int e = 0; e < Dv; ++e) o[e] += p * v[j * v_rs + e];
      }
      double dl = 0.0;
      for (int e = 0; e < Dv; ++e) dl += dout[i * do_rs + e] * (o[e] / l);
      lse[i] = mx + log(l);
      delta[i] = dl;
    }
    free(s);
    free(o);
  }
  if (failed) {
    free(lse);
    free(delta);
    return ORACLE_ENOMEM;
  }
  /* pass 2: dq by rows */
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < Lq; ++i) {
    const double* qi = q + i * q_rs;
    double* dqi = dq + i * dq_rs;
    for (int d = 0; d < D; ++d) dqi[d] = 0.0;
    for (int64_t j = 0; j < Lk; ++j) {
      double dot = 0.0, dp = 0.0;
      for (int d = 0; d < D; ++d) dot += qi[d] * k[j * k_rs + d];
      for (int e = 0; e < Dv; ++e) dp += dout[i * do_rs + e] * v[j * v_rs + e];
      const double ds = exp(scale * dot - lse[i]) * (dp - delta[i]);
      for (int d = 0; d < D; ++d) dqi[d] += scale * ds * k[j * k_rs + d];
    }
  }
  /* pass 3: dk and dv by keys */
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < Lk; ++j) {
    const double* kj = k + j * k_rs;
    double* dkj = dk + j * dk_rs;
    double* dvj = dv + j * dv_rs;
    for (int d = 0; d < D; ++d) dkj[d] = 0.0;
    for (int e = 0; e < Dv; ++e) dvj[e] = 0.0;
    for (int64_t i = 0; i < Lq; ++i) {
      double dot = 0.0, dp = 0.0;
      for (int d = 0; d < D; ++d) dot += q[i * q_rs + d] * kj[d];
      for (int e = 0; e < Dv; ++e) dp += dout[i * do_rs + e] * v[j * v_rs + e];
      const double p = exp(scale * dot - lse[i]);
      const double ds = p * (dp - delta[i]);
      for (int d = 0; d < D; ++d) dkj[d] += scale * ds * q[i * q_rs + d];
      for (int e = 0; e < Dv; ++e) dvj[e] += p * dout[i * do_rs + e];
    }
  }
  free(lse);
  free(delta);
  return ORACLE_OK;
}

/*
 * Pointwise projection y = x W ([P1] "Full self-attention" and "FLARE:
 * fixed-query latent routing": K = X W_K, V = X W_V with W in R^{C x C};
 * "FLARE++: dynamic token routing": the two extra projections of
 * equation 7).  x is [R, Cin], W is [Cin, Cout] (y = x W, no bias), y is
 * [R, Cout].  Each output element sums over c in index order.
 */
int oracle_matmul(const double* x, int64_t x_rs, const double* w, int64_t w_rs,
                  double* y, int64_t y_rs, int64_t R, int Cin, int Cout) {
  if (R < 0 || Cin <= 0 || Cout <= 0) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    const double* xr = x + r * x_rs;
    double* yr = y + r * y_rs;
    for (int j = 0; j < Cout; ++j) yr[j] = 0.0;
    /* y[r][j] accumulates x[r][c] w[c][j] for c = 0, 1, ... in order; the
       loop over j is innermost only so that W is read along its rows. */
    for (int c = 0; c < Cin; ++c) {
      const double xc = xr[c];
      const double* wc = w + (int64_t)c * w_rs;
      for (int j = 0; j < Cout; ++j) yr[j] += xc * wc[j];
    }
  }
  return ORACLE_OK;
}

/*
 * Exact merge of shard-local encoder results ([P1] "Multi-GPU context
 * parallelism"): every shard r contributes its normalised output O_r and its
 * row log-normaliser L_r; the global result is
 *   L = logsumexp_r L_r,   Z = sum_r exp(L_r - L) O_r.
 * o_parts is [R][Lq, Dv] (part r at o_parts + r * part_stride), l_parts is
 * [R][Lq] (part r at l_parts + r * Lq).  A shard with L_r = -inf (no tokens)
 * gets weight 0.
 */
int oracle_merge(const double* o_parts, int64_t part_stride,
                 const double* l_parts, int R, int64_t Lq, int Dv, double* z,
                 double* lse) {
  if (R <= 0 || Lq < 0 || Dv <= 0) return ORACLE_EINVAL;
  for (int64_t i = 0; i < Lq; ++i) {
    double mx = -INFINITY;
    for (int r = 0; r < R; ++r) {
      double lr = l_parts[(int64_t)r * Lq + i];
      mx = lr > mx ? lr : mx;
    }
    for (int e = 0; e < Dv; ++e) z[i * Dv + e] = 0.0;
    if (mx == -INFINITY) { /* every shard empty: no tokens at all */
      if (lse) lse[i] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int r = 0; r < R; ++r) sum += exp(l_parts[(int64_t)r * Lq + i] - mx);
    double L = mx + log(sum);
    for (int r = 0; r < R; ++r) {
      double w = exp(l_parts[(int64_t)r * Lq + i] - L);
      const double* orow = o_parts + (int64_t)r * part_stride + i * Dv;
      for (int e = 0; e < Dv; ++e) z[i * Dv + e] += w * orow[e];
    }
    if (lse) lse[i] = L;
  }
  return ORACLE_OK;
}

/*
 * The encoder applied shard by shard and merged ([P1] "Multi-GPU context
 * parallelism"): the token range [0, Lk) is cut at bounds[0] = 0 <= bounds[1]
 * <= ... <= bounds[R] = Lk (empty shards allowed); each shard runs the plain
 * SDPA on its own keys and values, then oracle_merge combines them.  Used to
 * check that the sharded form equals the unsharded encoder.
 */
int oracle_sharded_encode(const double* q, int64_t q_rs, const double* k,
                          int64_t k_rs, const double* v, int64_t v_rs,
                          const int64_t* bounds, int R, double* z, double* lse,
                          int64_t Lq, int D, int Dv, double scale) {
  if (R <= 0) return ORACLE_EINVAL;
  for (int r = 0; r < R; ++r)
    if (bounds[r] < 0 || bounds[r + 1] < bounds[r]) return ORACLE_EINVAL;
  int64_t part = Lq * Dv;
  double* o_parts = (double*)malloc(sizeof(double) * (size_t)(part * R + 1));
  double* l_parts = (double*)malloc(sizeof(double) * (size_t)(Lq * R + 1));
  if (!o_parts || !l_parts) {
    free(o_parts);
    free(l_parts);
    return ORACLE_ENOMEM;
  }
  int rc = ORACLE_OK;
  for (int r = 0; r < R && rc == ORACLE_OK; ++r) {
    int64_t b0 = bounds[r], n = bounds[r + 1] - bounds[r];
    rc = oracle_sdpa(q, q_rs, k + b0 * k_rs, k_rs, v + b0 * v_rs, v_rs,
                     o_parts + r * part, Dv, l_parts + (int64_t)r * Lq, Lq, n,
                     D, Dv, scale);
  }
  if (rc == ORACLE_OK) rc = oracle_merge(o_parts, part, l_parts, R, Lq, Dv, z, lse);
  free(o_parts);
  free(l_parts);
  return rc;
}

/* Row softmax of a dense [rows, cols] matrix in place (two-pass form). */
static void softmax_rows(double* a, int64_t rows, int64_t cols) {
  for (int64_t i = 0; i < rows; ++i) {
    double* r = a + i * cols;
    double mx = r[0];
    for (int64_t j = 1; j < cols; ++j) mx = r[j] > mx ? r[j] : mx;
    double l = 0.0;
    for (int64_t j = 0; j < cols; ++j) {
      r[j] = exp(r[j] - mx);
      l += r[j];
    }
    for (int64_t j = 0; j < cols; ++j) r[j] /= l;
  }
}

/*
 * The effective token-to-token mixing matrix of one head, materialised
 * ([P1] "FLARE: fixed-query latent routing": W_eff = W_dec W_enc with the
 * encoder weights W_enc = softmax over tokens of S = Q K^T * scale (one row
 * per latent) and the decoder weights W_dec = softmax over latents of S^T
 * (one row per token)).  Only for tiny N: w is [N, N].
 * Optionally returns w_dec [N, M] and w_enc [M, N].
 */
int oracle_mixing_matrix(const double* q, int64_t q_rs, const double* k,
                         int64_t k_rs, int64_t N, int M, int D, double scale,
                         double* w, double* w_dec_out, double* w_enc_out) {
  if (N <= 0 || M <= 0 || D <= 0) return ORACLE_EINVAL;
  double* enc = (double*)malloc(sizeof(double) * (size_t)(M * N));
  double* dec = (double*)malloc(sizeof(double) * (size_t)(N * M));
  if (!enc || !dec) {
    free(enc);
    free(dec);
    return ORACLE_ENOMEM;
  }
  for (int m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += q[m * q_rs + d] * k[n * k_rs + d];
      enc[m * N + n] = scale * dot;
      dec[n * M + m] = scale * dot;
    }
  softmax_rows(enc, M, N); /* W_enc: each latent's weights over tokens */
  softmax_rows(dec, N, M); /* W_dec: each token's weights over latents */
  for (int64_t i = 0; i < N; ++i)
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0.0;
      for (int m = 0; m < M; ++m) acc += dec[i * M + m] * enc[m * N + j];
      w[i * N + j] = acc;
    }
  if (w_dec_out) memcpy(w_dec_out, dec, sizeof(double) * (size_t)(N * M));
  if (w_enc_out) memcpy(w_enc_out, enc, sizeof(double) * (size_t)(M * N));
  free(enc);
  free(dec);
  return ORACLE_OK;
}

/*
 * FLARE encode-decode for every (batch, head) with keys and values given
 * ([P1] "FLARE: fixed-query latent routing"):
 *   Z_h = SDPA(Q_h, K_h, V_h)          (encode: M latents gather N tokens)
 *   Y_h = SDPA(K_h, Q_h, Z_h)          (decode: the latents are sent back)
 * k, v, y are [B, N, H*D] token-major (head h = columns [hD, (h+1)D));
 * q is [H, M, D] when q_bs == 0 (one learned set shared by the batch) or
 * [B, H, M, D] with batch stride q_bs.  z_out [B, H, M, D] and
 * lse_out [B, H, M] may be NULL.  heads_lo/heads_hi restrict the heads
 * computed (a bounded sample for timing); the rest of y is left untouched.
 */
int oracle_flare_encdec(const double* q, int64_t q_bs, const double* k,
                        const double* v, double* y, double* z_out,
                        double* lse_out, int B, int64_t N, int H, int M, int D,
                        double scale, int heads_lo, int heads_hi) {
  if (B <= 0 || N <= 0 || H <= 0 || M <= 0 || D <= 0) return ORACLE_EINVAL;
  if (heads_lo < 0 || heads_hi > H || heads_lo > heads_hi) return ORACLE_EINVAL;
  int64_t C = (int64_t)H * D;
  double* z = (double*)malloc(sizeof(double) * (size_t)M * D);
  if (!z) return ORACLE_ENOMEM;
  int rc = ORACLE_OK;
  for (int b = 0; b < B && rc == ORACLE_OK; ++b)
    for (int h = heads_lo; h < heads_hi && rc == ORACLE_OK; ++h) {
      const double* qh = q + b * q_bs + (int64_t)h * M * D;
      const double* kh = k + (int64_t)b * N * C + (int64_t)h * D;
      const double* vh = v + (int64_t)b * N * C + (int64_t)h * D;
      double* lse = lse_out ? lse_out + ((int64_t)b * H + h) * M : NULL;
      rc = oracle_sdpa(qh, D, kh, C, vh, C, z, D, lse, M, N, D, D, scale);
      if (rc != ORACLE_OK) break;
      if (z_out) memcpy(z_out + ((int64_t)b * H + h) * M * D, z, sizeof(double) * (size_t)M * D);
      rc = oracle_sdpa(kh, C, qh, D, z, D, y + (int64_t)b * N * C + (int64_t)h * D, C,
                       NULL, N, M, D, D, scale);
    }
  free(z);
  return rc;
}

/*
 * The whole mixer on a token matrix X [B, N, C], C = H*D.
 *   FLARE   (w_ek == NULL): K = X W_K, V = X W_V; Q_h = qs[h] (learned);
 *   FLARE++ (w_ek != NULL): additionally eK = X W_eK, eV = X W_eV
 *            (equation 7) and the routing queries are synthesised per input,
 *            Q_h(X) = SDPA(seeds_h, eK_h, eV_h) (equation 8);
 *   then Z_h = SDPA(Q_h, K_h, V_h), Y_h = SDPA(K_h, Q_h, Z_h), heads are
 *   concatenated, and out = Y W_O when w_o != NULL (else out = Y).
 * ([P1] "FLARE: fixed-query latent routing", "FLARE++: dynamic token
 * routing", "Full self-attention" for the output projection.)
 * All weights are [C, C] with y = x W.  qs is [H, M, D].  qx_out and z_out
 * ([B, H, M, D]) may be NULL.
 */
int oracle_flare_mix(const double* x, const double* w_k, const double* w_v,
                     const double* w_ek, const double* w_ev, const double* qs,
                     const double* w_o, double* out, double* qx_out,
                     double* z_out, int B, int64_t N, int C, int H, int M,
                     double scale) {
  if (B <= 0 || N <= 0 || C <= 0 || H <= 0 || M <= 0 || C % H) return ORACLE_EINVAL;
  int D = C / H;
  int dynamic = w_ek != NULL;
  if (dynamic && !w_ev) return ORACLE_EINVAL;
  size_t nc = (size_t)N * C;
  double* K = (double*)malloc(sizeof(double) * nc);
  double* V = (double*)malloc(sizeof(double) * nc);
  double* eK = dynamic ? (double*)malloc(sizeof(double) * nc) : NULL;
  double* eV = dynamic ? (double*)malloc(sizeof(double) * nc) : NULL;
  double* Y = (double*)malloc(sizeof(double) * nc);
  double* Q = (double*)malloc(sizeof(double) * (size_t)M * D);
  double* Z = (double*)malloc(sizeof(double) * (size_t)M * D);
  int rc = ORACLE_OK;
  if (!K || !V || !Y || !Q || !Z || (dynamic && (!eK || !eV))) rc = ORACLE_ENOMEM;
  for (int b = 0; b < B && rc == ORACLE_OK; ++b) {
    const double* xb = x + (size_t)b * nc;
    oracle_matmul(xb, C, w_k, C, K, C, N, C, C);
    oracle_matmul(xb, C, w_v, C, V, C, N, C, C);
    if (dynamic) {
      oracle_matmul(xb, C, w_ek, C, eK, C, N, C, C);
      oracle_matmul(xb, C, w_ev, C, eV, C, N, C, C);
    }
    for (int h = 0; h < H && rc == ORACLE_OK; ++h) {
      const double* seeds = qs + (size_t)h * M * D;
      if (dynamic)
        rc = oracle_sdpa(seeds, D, eK + h * D, C, eV + h * D, C, Q, D, NULL, M, N, D, D, scale);
      else
        memcpy(Q, seeds, sizeof(double) * (size_t)M * D);
      if (rc == ORACLE_OK)
        rc = oracle_sdpa(Q, D, K + h * D, C, V + h * D, C, Z, D, NULL, M, N, D, D, scale);
      if (rc == ORACLE_OK)
        rc = oracle_sdpa(K + h * D, C, Q, D, Z, D, Y + h * D, C, NULL, N, M, D, D, scale);
      size_t lat = ((size_t)b * H + h) * M * D;
      if (qx_out) memcpy(qx_out + lat, Q, sizeof(double) * (size_t)M * D);
      if (z_out) memcpy(z_out + lat, Z, sizeof(double) * (size_t)M * D);
    }
    if (rc != ORACLE_OK) break;
    if (w_o)
      oracle_matmul(Y, C, w_o, C, out + (size_t)b * nc, C, N, C, C);
    else
      memcpy(out + (size_t)b * nc, Y, sizeof(double) * nc);
  }
  free(K);
  free(V);
  free(eK);
  free(eV);
  free(Y);
  free(Q);
  free(Z);
  return rc;
}
