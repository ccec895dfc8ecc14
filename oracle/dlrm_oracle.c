/*
 * CPU oracle for the DLRM hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct reference implementations of what the GPU
 * library computes.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this file's library; the product path never does.  It
 * shares no code, header or constant with the GPU library.
 *
 * Sources (web pages on DLRM, cited by page and section):
 *   [EXPL] "Deep Learning Recommendation Model (DLRM)" explainer
 *          (nadeemcite.github.io), sections "Core Idea" and "Key Method Details".
 *   [SU]   "DLRM - Deep Learning Recommendation Model" (briansu.co/recsys/dlrm),
 *          "How it works", "Key equations" (Interaction, Output),
 *          "Limitations & trade-offs".
 *
 * Precision: floating point is fp64 except where the contract fixes fp32:
 * pooled embeddings and SGD-updated rows are defined bit-exactly as fp32
 * sums in a fixed order (bag order; for the SGD rows, blocks of 128
 * occurrences in position order), so those two functions compute in fp32 in
 * that order.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math).  OpenMP splits
 * only independent outputs, so results do not depend on the thread count.
 *
 * Parity pins: every function here is pinned by the CPU tests against closed
 * forms, invariants, brute force or independent library routines.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* fp32 -> nearest bf16 (ties to even), returned as the fp32 value of that
 * bf16.  NaN stays NaN (quietened).  bf16 is fp32 with the low 16 mantissa
 * bits removed. */
static float bf16_round(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u) {
    u = (u | 0x00400000u) & 0xffff0000u;
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);
    u &= 0xffff0000u;
  }
  float y;
  memcpy(&y, &u, sizeof y);
  return y;
}

void oracle_bf16_round(const float* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(in[i]);
}

/*
 * Embedding lookup with sum pooling.
 * [EXPL] Key Method Details, "Embedding tables": feature k owns a table of
 * m_k rows of width d (d shared by all features).  [SU] How it works: each
 * sparse feature looks up a row in its own table.  A bag of several indices
 * is pooled by summation (one-index bags are exactly the lookup).
 *
 * Bag (k, b) owns idx[off[k*B+b] .. off[k*B+b+1]); its pooled vector is
 *   out[b*out_ld + out_col0 + k*d + c] = sum over p ascending of T_k[idx[p]][c],
 * accumulated in fp32 starting from +0.0f (an empty bag gives +0.0).
 */
void oracle_embbag_fwd(const float* const* tables, int32_t K, int32_t d, const int64_t* idx,
                       const int64_t* off, int64_t B, float* out, int64_t out_ld, int64_t out_col0) {
  const int64_t bags = (int64_t)K * B;
#pragma omp parallel for schedule(static)
  for (int64_t kb = 0; kb < bags; ++kb) {
    const int64_t k = kb / B, b = kb % B;
    float* o = out + b * out_ld + out_col0 + k * (int64_t)d;
    for (int32_t c = 0; c < d; ++c) o[c] = 0.0f;
    for (int64_t p = off[kb]; p < off[kb + 1]; ++p) {
      const float* row = tables[k] + idx[p] * (int64_t)d;
      for (int32_t c = 0; c < d; ++c) o[c] = o[c] + row[c];
    }
  }
}

/*
 * Embedding lookup with sum pooling from low-precision table rows.
 * The page "Deep Learning Recommendation Model for Personalization and
 * Recommendation Systems" (mlsanity summary), Citations in the corpus,
 * carries a quantisation survey's note that quantisation pays where a
 * problem is bandwidth-bound, as recommendation is; the pages fix no
 * format, so two plain ones are read here.  Every stored value is first turned into an fp32 number v, then the
 * bag is pooled exactly as oracle_embbag_fwd (fp32, ascending position,
 * from +0.0f):
 *   dtype 1 (bf16):  v = the bf16 value widened to fp32 (exact: the 16 bits
 *                    become the high half of the fp32 word).
 *   dtype 2 (int8):  v = fl(fl(s * q) + z) with the row's fp32 scale s and
 *                    bias z (sb[k][2r], sb[k][2r+1]): the product is rounded
 *                    to fp32, then the sum.
 */
static float lp_value(const void* table, const float* sb, int32_t dtype, int64_t r, int32_t d, int32_t c) {
  if (dtype == 1) {
    const uint16_t h = ((const uint16_t*)table)[r * d + c];
    const uint32_t u = (uint32_t)h << 16;
    float v;
    memcpy(&v, &u, sizeof v);
    return v;
  }
  const int8_t q = ((const int8_t*)table)[r * d + c];
  const float prod = sb[2 * r] * (float)q;
  return prod + sb[2 * r + 1];
}

void oracle_embbag_fwd_lp(const void* const* tables, int32_t dtype, const float* const* sb, int32_t K, int32_t d,
                          const int64_t* idx, const int64_t* off, int64_t B, float* out, int64_t out_ld,
                          int64_t out_col0) {
  const int64_t bags = (int64_t)K * B;
#pragma omp parallel for schedule(static)
  for (int64_t kb = 0; kb < bags; ++kb) {
    const int64_t k = kb / B, b = kb % B;
    float* o = out + b * out_ld + out_col0 + k * (int64_t)d;
    for (int32_t c = 0; c < d; ++c) o[c] = +0.0f;
    for (int64_t pos = off[kb]; pos < off[kb + 1]; ++pos)
      for (int32_t c = 0; c < d; ++c) o[c] = o[c] + lp_value(tables[k], sb ? sb[k] : 0, dtype, idx[pos], d, c);
  }
}

/*
 * Pairwise dot-product interaction and concatenation.
 * [SU] Key equations, Interaction: Z = tril(X X^T), X = [x_dense; e_1; ...; e_K]
 * of shape (K+1) x d.  [EXPL] Key Method Details, "Interaction layer": only
 * pairs of distinct vectors are kept, n(n-1)/2 values.  [SU] Key equations,
 * Output: the top MLP input is [x_dense, vec(Z)], dense vector first.
 *
 * X row 0 is x_dense (the bottom MLP's output), rows 1..K the pooled
 * embeddings.  Sample b's output row is
 *   out[b][c]                      = X_b[0][c]                       c < d
 *   out[b][d + i(i-1)/2 + j]       = sum_c X_b[i][c] * X_b[j][c]     0 <= j < i < n
 * i.e. the strict lower triangle, row by row.  The sum is exact products
 * accumulated in fp64, rounded once to fp32.
 */
void oracle_interact_fwd(const float* X, int64_t B, int32_t n, int32_t d, int64_t x_ld, float* out,
                         int64_t out_ld) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    const float* x = X + b * x_ld;
    float* o = out + b * out_ld;
    for (int32_t c = 0; c < d; ++c) o[c] = x[c];
    for (int32_t i = 1; i < n; ++i) {
      for (int32_t j = 0; j < i; ++j) {
        double s = 0.0;
        for (int32_t c = 0; c < d; ++c) s += (double)x[(int64_t)i * d + c] * (double)x[(int64_t)j * d + c];
        o[d + (int64_t)i * (i - 1) / 2 + j] = (float)s;
      }
    }
  }
}

/*
 * Interaction, backward (the training pass through the interaction above).
 * [SU] Key equations, Interaction and Output define the forward map
 * X -> y = [X_0, Z]; [EXPL] Key Method Details, Loss: the model is trained
 * on binary cross-entropy, so the top MLP hands back g = dL/dy.  By the
 * chain rule, each kept pair value Z_ij = <X_i, X_j> (j < i) sends
 * g_ij * X_j to row i and g_ij * X_i to row j, and the dense copy sends g_c
 * to row 0:
 *   dX[i][c] = [i == 0] g[c] + sum over j != i of g_pair(i, j) * X[j][c]
 * with g_pair(i, j) = g[d + a(a-1)/2 + b], a = max(i, j), b = min(i, j).
 * Every term is an exact product accumulated in fp64, rounded once to fp32.
 */
void oracle_interact_bwd(const float* X, int64_t B, int32_t n, int32_t d, int64_t x_ld, const float* g, int64_t g_ld,
                         float* dX, int64_t dx_ld) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    const float* xr = X + b * x_ld;
    const float* gb = g + b * g_ld;
    float* o = dX + b * dx_ld;
    for (int32_t i = 0; i < n; ++i) {
      for (int32_t c = 0; c < d; ++c) {
        double s = (i == 0) ? (double)gb[c] : 0.0;
        for (int32_t j = 0; j < n; ++j) {
          if (j == i) continue;
          const int32_t a = i > j ? i : j, e = i > j ? j : i;
          s += (double)gb[d + (int64_t)a * (a - 1) / 2 + e] * (double)xr[(int64_t)j * d + c];
        }
        o[(int64_t)i * d + c] = (float)s;
      }
    }
  }
}

/*
 * Multilayer perceptron, forward.
 * [EXPL] Key Method Details, "Bottom MLP": fully connected layers with ReLU
 * whose output has dimension d.  "Top MLP": fully connected layers with ReLU
 * ending in a sigmoid.  [SU] Key equations, Output: y = sigma(MLP_top(...)).
 *
 * Layer l maps width dims[l] to dims[l+1]:  y[o] = act( b[o] + sum_i W[o][i] x[i] )
 * with W row-major [dims[l+1]][dims[l]].  The sum is exact products in fp64
 * plus the bias, rounded once to fp32.  act is ReLU on every layer except the
 * last, which has ReLU only when last_relu != 0 (bottom MLP) and is linear
 * otherwise (top MLP: its output is the logit).
 *
 * quant_bf16 != 0 models a network with bf16 inputs: each layer's input
 * vector x is rounded to the nearest bf16 before use (W must then already
 * hold bf16 values).  Outputs stay fp32.
 *
 * out: [B][out_ld], the last layer's fp32 output.  prob (nullable, only when
 * dims[L] == 1): 1 / (1 + exp(-logit)).  acts (nullable): array of L+1
 * pointers; acts[l] ([B][dims[l]]) receives layer l's input as used (after
 * rounding), acts[L] the final output -- what the backward pass needs.
 */
void oracle_mlp_fwd(const float* in, int64_t in_ld, int64_t B, int32_t L, const int32_t* dims,
                    const float* const* W, const float* const* bias, int32_t quant_bf16, int32_t last_relu,
                    float* out, int64_t out_ld, float* prob, float* const* acts) {
  int32_t wmax = 0;
  for (int32_t l = 0; l <= L; ++l)
    if (dims[l] > wmax) wmax = dims[l];
#pragma omp parallel
  {
    float* h = (float*)malloc(sizeof(float) * (size_t)wmax);
    float* x = (float*)malloc(sizeof(float) * (size_t)wmax);
#pragma omp for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
      for (int32_t i = 0; i < dims[0]; ++i) h[i] = in[b * in_ld + i];
      for (int32_t l = 0; l < L; ++l) {
        const int32_t fi = dims[l], fo = dims[l + 1];
        for (int32_t i = 0; i < fi; ++i) x[i] = quant_bf16 ? bf16_round(h[i]) : h[i];
        if (acts) memcpy(acts[l] + b * fi, x, sizeof(float) * (size_t)fi);
        const int relu = (l < L - 1) || last_relu;
        for (int32_t o = 0; o < fo; ++o) {
          const float* w = W[l] + (int64_t)o * fi;
          double s = 0.0;
          for (int32_t i = 0; i < fi; ++i) s += (double)w[i] * (double)x[i];
          float y = (float)(s + (double)bias[l][o]);
          if (relu && !(y > 0.0f)) y = 0.0f;
          h[o] = y;
        }
      }
      const int32_t fo = dims[L];
      for (int32_t o = 0; o < fo; ++o) out[b * out_ld + o] = h[o];
      if (acts) memcpy(acts[L] + b * fo, h, sizeof(float) * (size_t)fo);
      if (prob && fo == 1) prob[b] = (float)(1.0 / (1.0 + exp(-(double)h[0])));
    }
    free(h);
    free(x);
  }
}

/*
 * Multilayer perceptron, backward (textbook backpropagation, fp64 inside).
 * Training minimises binary cross-entropy ([EXPL] Key Method Details, "Loss");
 * the caller supplies dY = dLoss/d(output), e.g. (sigma(logit) - y)/B.
 *
 * Inputs are the saved activations of oracle_mlp_fwd (acts[l] = layer l's
 * input as used, acts[L] = final output) and the same weights.  For layer l
 * (in reverse), with output y_l (acts[l+1], or acts[L] for the last layer):
 *   delta = g * 1[y_l > 0]     (ReLU layers; identity for a linear last layer)
 *   dW_l[o][i] = sum_b delta[b][o] * x_l[b][i]
 *   db_l[o]    = sum_b delta[b][o]
 *   g_prev[b][i] = sum_o delta[b][o] * W_l[o][i]
 * The rounding of layer inputs to bf16 is treated as the identity (its
 * derivative is taken as 1).  dX (nullable) receives g_prev of layer 0.
 */
void oracle_mlp_bwd(int64_t B, int32_t L, const int32_t* dims, const float* const* W, const float* const* acts,
                    int32_t last_relu, const float* dY, float* const* dW, float* const* db, float* dX) {
  int32_t wmax = 0;
  for (int32_t l = 0; l <= L; ++l)
    if (dims[l] > wmax) wmax = dims[l];
  double* g = (double*)malloc(sizeof(double) * (size_t)B * (size_t)wmax);
  double* delta = (double*)malloc(sizeof(double) * (size_t)B * (size_t)wmax);
  const int32_t fl = dims[L];
  for (int64_t i = 0; i < B * fl; ++i) g[i] = (double)dY[i];
  for (int32_t l = L - 1; l >= 0; --l) {
    const int32_t fi = dims[l], fo = dims[l + 1];
    const float* y = acts[l + 1];
    const float* x = acts[l];
    const int relu = (l < L - 1) || last_relu;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b)
      for (int32_t o = 0; o < fo; ++o) {
        const double gv = g[b * fo + o];
        delta[b * fo + o] = (relu && !(y[b * fo + o] > 0.0f)) ? 0.0 : gv;
      }
    /* Every sum below runs over b (or o) in ascending order from 0.0; the
     * loops over i are innermost only so that rows are read contiguously. */
#pragma omp parallel
    {
      double* s = (double*)malloc(sizeof(double) * (size_t)fi);
#pragma omp for schedule(static)
      for (int32_t o = 0; o < fo; ++o) {
        double sb = 0.0;
        for (int32_t i = 0; i < fi; ++i) s[i] = 0.0;
        for (int64_t b = 0; b < B; ++b) {
          const double dv = delta[b * fo + o];
          sb += dv;
          for (int32_t i = 0; i < fi; ++i) s[i] += dv * (double)x[b * fi + i];
        }
        db[l][o] = (float)sb;
        for (int32_t i = 0; i < fi; ++i) dW[l][(int64_t)o * fi + i] = (float)s[i];
      }
      free(s);
    }
    if (l > 0 || dX) {
#pragma omp parallel for schedule(static)
      for (int64_t b = 0; b < B; ++b) {
        double* gb = g + b * fi;
        for (int32_t i = 0; i < fi; ++i) gb[i] = 0.0;
        for (int32_t o = 0; o < fo; ++o) {
          const double dv = delta[b * fo + o];
          for (int32_t i = 0; i < fi; ++i) gb[i] += dv * (double)W[l][(int64_t)o * fi + i];
        }
      }
    }
  }
  if (dX)
    for (int64_t i = 0; i < B * dims[0]; ++i) dX[i] = (float)g[i];
  free(g);
  free(delta);
}

/*
 * Sparse embedding backward with row-wise SGD, in place.
 * Sum pooling sends the gradient of bag (k, b) unchanged to every row it
 * looked up, once per occurrence.  For each row r of table k that the batch
 * touches, with its occurrences p_0 < p_1 < ... in table k's bags (position
 * order) and x_i = G[b(p_i)*g_ld + g_col0 + k*d + c]:
 *   S_j  = the sum of the block x_{128j} .. x_{128j+127} (or to the last
 *          occurrence), in order, fp32 from +0.0f
 *   g[c] = the sum of S_0, S_1, ... in order, fp32 from +0.0f
 *   T_k[r][c] = T_k[r][c] - (lr * g[c])        (two fp32 roundings, no FMA)
 * The pages define the row's gradient as the plain sum of its occurrences'
 * gradients and fix no order for it; this order (blocks of SGD_BLOCK in
 * position order) is one a parallel machine reaches, and for at most
 * SGD_BLOCK + 1 occurrences it is the plain left-to-right sum.
 * Rows the batch does not touch are left as they are.  rows[k] is the row
 * count of table k.
 */
#define SGD_BLOCK 128
void oracle_embbag_bwd_sgd(float* const* tables, const int64_t* rows, int32_t K, int32_t d, const int64_t* idx,
                           const int64_t* off, int64_t B, const float* G, int64_t g_ld, int64_t g_col0,
                           float lr) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t k = 0; k < K; ++k) {
    float* acc = (float*)calloc((size_t)rows[k] * (size_t)d, sizeof(float)); /* sum of finished blocks */
    float* blk = (float*)calloc((size_t)rows[k] * (size_t)d, sizeof(float)); /* the open block's sum */
    int64_t* count = (int64_t*)calloc((size_t)rows[k], sizeof(int64_t));     /* occurrences so far */
    unsigned char* touched = (unsigned char*)calloc((size_t)rows[k], 1);
    for (int64_t b = 0; b < B; ++b) {
      const float* gb = G + b * g_ld + g_col0 + (int64_t)k * d;
      for (int64_t p = off[(int64_t)k * B + b]; p < off[(int64_t)k * B + b + 1]; ++p) {
        const int64_t r = idx[p];
        touched[r] = 1;
        float* a = acc + r * (int64_t)d;
        float* bs = blk + r * (int64_t)d;
        if (count[r] > 0 && count[r] % SGD_BLOCK == 0) /* a block is full: it joins the total */
          for (int32_t c = 0; c < d; ++c) {
            a[c] = a[c] + bs[c];
            bs[c] = 0.0f;
          }
        for (int32_t c = 0; c < d; ++c) bs[c] = bs[c] + gb[c];
        count[r] += 1;
      }
    }
    float* T = tables[k];
    for (int64_t r = 0; r < rows[k]; ++r) {
      if (!touched[r]) continue;
      for (int32_t c = 0; c < d; ++c) {
        const float g = acc[r * (int64_t)d + c] + blk[r * (int64_t)d + c]; /* the last block */
        const float step = lr * g;
        T[r * (int64_t)d + c] = T[r * (int64_t)d + c] - step;
      }
    }
    free(acc);
    free(blk);
    free(count);
    free(touched);
  }
}
