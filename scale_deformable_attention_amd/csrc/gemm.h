// gemm.h -- internal interface of the matrix-core GEMM in linear.hip, used by
// the layer entry points. Not part of the C ABI.
#pragma once
#include <stdint.h>

#include "msda.h"

// Blocks of the matrix-core GEMM resident at once on the whole GPU (3 per CU
// on 256 CUs): reduction splits are chosen so that one launch offers about
// this many work items.
constexpr int64_t kGemmResidentBlocks = 768;

// C[m, n] = sum_k A(m, k) B(k, n) (+ bias[n]) (+ C[m, n] if accumulate), fp32.
//   a_kmajor: A(m, k) = A[m * lda + k], else A[k * lda + m]
//   b_kmajor: B(k, n) = B[n * ldb + k], else B[k * ldb + n]
// splits > 1 splits the reduction over blocks into `partials` (splits * M * N
// floats, device) and sums them with a second kernel. With a_colsum set, the
// same pass also writes a_colsum[m] = sum over k of A(m, k) (through
// a_colsum_partials, splits * M floats, when splits > 1).
msda_status_t msda_gemm(bool a_kmajor, bool b_kmajor, int M, int N, int K, const float* A,
                        int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                        const float* bias, bool accumulate, int splits, float* partials,
                        hipStream_t stream, float* a_colsum = nullptr,
                        float* a_colsum_partials = nullptr);

// One product of a batch: C = A B (+ bias) (+ C), as msda_gemm, optionally
// with a second reduction segment appended (C += A2 B2 over K2 more k; K a
// multiple of 16, no split).
struct GemmSpec {
    bool a_kmajor = true, b_kmajor = true;
    int M = 0, N = 0, K = 0;
    const float* A = nullptr;
    int64_t lda = 0;
    const float* B = nullptr;
    int64_t ldb = 0;
    float* C = nullptr;
    int64_t ldc = 0;
    const float* bias = nullptr;
    bool accumulate = false;
    int splits = 1;
    float* partials = nullptr;          // splits * M * N floats when splits > 1
    float* a_colsum = nullptr;          // optional column sums of A
    float* a_colsum_partials = nullptr; // splits * M floats when splits > 1
    const float* A2 = nullptr;
    int64_t lda2 = 0;
    const float* B2 = nullptr;
    int64_t ldb2 = 0;
    int K2 = 0;
};

// Up to 4 independent products with the same operand layouts in one launch
// (their split reductions follow). Distinct partial buffers per product.
msda_status_t msda_gemm_batch(const GemmSpec* specs, int count, hipStream_t stream);

// out[n] (+)= sum over the R rows of g[r * ldg + n], through `partials`
// (splits * N floats, device).
msda_status_t msda_colsum(int R, int N, const float* g, int64_t ldg, float* out, int splits,
                          float* partials, bool accumulate, hipStream_t stream);

// Reduction splits used for a weight gradient over `rows` rows, and the
// workspace floats a linear backward needs.
int msda_linear_splits(int64_t rows, int64_t in_features, int64_t out_features);
size_t msda_linear_workspace_floats(int64_t rows, int64_t in_features, int64_t out_features);
