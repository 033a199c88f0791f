// Dense / sparse selection for one weight matrix (lscd_attach_dense, lscd_linear and the
// cost model behind them).  Declared and documented in include/lscd.h.
//
// The Flash-LLM review (xllm-io, section 5 "FasterTransformer integration" and section 6
// "N dimension") describes a GEMM wrapper that picks the dense or the sparse MatMul per
// call, because the sparse kernel only wins while the product is memory-bound (small N);
// once N is large the work is compute-bound and the dense library GEMM is faster.  Here
// the dense copy is decoded from the encoding itself, and the dense product is a rocBLAS
// fp16 GEMM with fp32 accumulation.

#include <math.h>

#include <algorithm>

#include <rocblas/rocblas.h>

#include "lscd_internal.h"

namespace {

// Cost model, fitted to MI355X measurements of both paths: N = 8 .. 1024 sweeps on the OPT-30B
// MLP1 and OPT-175B OutProj shapes plus N = 8 .. 64 on every benchmark shape (it picks the
// faster path in all 40 of those cases).  Skinny kernels (N <= 64): the packed words stream
// at a sustained rate and the N-dependent on-chip work adds on top.  Wide kernel: per launch,
// the larger of the stream time and the MFMA time (it overlaps the two).  Dense GEMM:
// matrix stream plus MFMA time.
constexpr double kSparseBytesPerUs = 6.8e6;   // packed words, B/us
constexpr double kNarrowFlopsPerUs = 2.0e9;   // dense-equivalent flop/us, N <= 64
constexpr double kWideFlopsPerUs = 4.5e8;     // dense-equivalent flop/us, N > 64
constexpr double kSparseCallUs = 8.0;         // fixed cost per sparse launch
constexpr double kDenseBytesPerUs = 5.8e6;
constexpr double kDenseFlopsPerUs = 1.8e9;
constexpr double kDenseCallUs = 6.0;

void model(int64_t M, int64_t K, int64_t nnz_padded, int64_t T, int32_t N, double* ts, double* td) {
    const double m = (double)M, k = (double)K, n = (double)N;
    const double words = 4.0 * (double)nnz_padded + 4.0 * (double)(T + 1);
    if (N <= LSCD_NARROW_MAX_N) {
        const double npad = N <= 16 ? 16 : (N <= 32 ? 32 : 64);
        *ts = kSparseCallUs + (words + 2 * k * n + 2 * m * n) / kSparseBytesPerUs +
              2 * m * k * npad / kNarrowFlopsPerUs;
    } else {
        *ts = 0;
        for (int32_t c0 = 0; c0 < N; c0 += lscd::kWideMaxN) {
            const double nb = (double)std::min(N - c0, lscd::kWideMaxN);
            const double npad = ceil(nb / 64.0) * 64.0;
            const double stream = (words + 2 * k * nb + 2 * m * nb) / kSparseBytesPerUs;
            const double mfma = 2 * m * k * npad / (nb <= LSCD_NARROW_MAX_N ? kNarrowFlopsPerUs : kWideFlopsPerUs);
            *ts += kSparseCallUs + (nb <= LSCD_NARROW_MAX_N ? stream + mfma : std::max(stream, mfma));
        }
    }
    *td = kDenseCallUs + (2 * m * k + 2 * k * n + 2 * m * n) / kDenseBytesPerUs + 2 * m * k * n / kDenseFlopsPerUs;
}

lscd_status_t hip_st(hipError_t e) {
    if (e == hipSuccess) return LSCD_SUCCESS;
    return e == hipErrorOutOfMemory ? LSCD_ERROR_OUT_OF_MEMORY : LSCD_ERROR_HIP;
}

lscd_status_t on_device(const lscd_handle_s* h) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LSCD_ERROR_HIP;
    return dev == h->device ? LSCD_SUCCESS : LSCD_ERROR_INVALID_VALUE;
}

bool use_dense(const lscd_handle_s* h, int32_t N) {
    if (!h->d_dense) return false;
    if (h->crossover >= 0) return N > h->crossover;
    double ts, td;
    model(h->g.M, h->g.K, h->nnz_padded, h->g.T, N, &ts, &td);
    return td < ts;
}

}  // namespace

namespace lscd {

void release_dense(lscd_handle_s* h) {
    if (h->blas) (void)rocblas_destroy_handle((rocblas_handle)h->blas);
    if (h->d_dense) (void)hipFree(h->d_dense);
    h->blas = nullptr;
    h->d_dense = nullptr;
}

}  // namespace lscd

extern "C" {

lscd_status_t lscd_linear_model(int64_t M, int64_t K, int64_t nnz_padded, int64_t num_tiles, int32_t N,
                                double* t_sparse_us, double* t_dense_us) {
    if (M < 1 || K < 1 || nnz_padded < 0 || num_tiles < 1 || N < 1 || !t_sparse_us || !t_dense_us)
        return LSCD_ERROR_INVALID_VALUE;
    model(M, K, nnz_padded, num_tiles, N, t_sparse_us, t_dense_us);
    return LSCD_SUCCESS;
}

lscd_status_t lscd_attach_dense(lscd_handle_t h) {
    if (!h) return LSCD_ERROR_INVALID_VALUE;
    if (h->g.tk != lscd::kTileK) return LSCD_ERROR_NOT_SUPPORTED;  // lscd_debug_decode checks the rest
    if (h->g.M > INT32_MAX || h->g.K > INT32_MAX) return LSCD_ERROR_NOT_SUPPORTED;
    lscd_status_t st = on_device(h);
    if (st != LSCD_SUCCESS) return st;
    if (h->d_dense) return LSCD_SUCCESS;
    hipError_t e = hipMalloc((void**)&h->d_dense, (size_t)h->g.M * h->g.K * 2);
    if (e != hipSuccess) {
        h->d_dense = nullptr;
        return hip_st(e);
    }
    rocblas_handle rh = nullptr;
    if (rocblas_create_handle(&rh) != rocblas_status_success) {
        lscd::release_dense(h);
        return LSCD_ERROR_HIP;
    }
    h->blas = rh;
    lscd_status_t ds = lscd_debug_decode(h, h->d_dense, nullptr);
    if (ds == LSCD_SUCCESS) ds = hip_st(hipDeviceSynchronize());
    if (ds != LSCD_SUCCESS) lscd::release_dense(h);
    return ds;
}

lscd_status_t lscd_set_linear_crossover(lscd_handle_t h, int32_t n_max_sparse) {
    if (!h || n_max_sparse < -1) return LSCD_ERROR_INVALID_VALUE;
    h->crossover = n_max_sparse;
    return LSCD_SUCCESS;
}

lscd_status_t lscd_linear_path(lscd_handle_t h, int32_t N, int32_t* path) {
    if (!h || !path || N < 0) return LSCD_ERROR_INVALID_VALUE;
    *path = use_dense(h, N) ? 1 : 0;
    return LSCD_SUCCESS;
}

lscd_status_t lscd_linear(lscd_handle_t h, const void* B, void* C, int32_t N, void* stream) {
    if (!h || N < 0) return LSCD_ERROR_INVALID_VALUE;
    if (N == 0) return LSCD_SUCCESS;
    if (!use_dense(h, N)) return lscd_spmm(h, B, C, N, stream);
    if (!B || !C || ((uintptr_t)B & 15u) || ((uintptr_t)C & 15u)) return LSCD_ERROR_INVALID_VALUE;
    if (N > LSCD_MAX_N) return LSCD_ERROR_NOT_SUPPORTED;
    lscd_status_t st = on_device(h);
    if (st != LSCD_SUCCESS) return st;
    rocblas_handle rh = (rocblas_handle)h->blas;
    if (rocblas_set_stream(rh, (hipStream_t)stream) != rocblas_status_success) return LSCD_ERROR_HIP;
    // Column-major view: C (N x M row-major) is the M x N matrix A * B^T with ldc = M; A (M x
    // K row-major) is A^T in column-major with lda = K; B (N x K row-major) is K x N, ldb = K.
    const float alpha = 1.0f, beta = 0.0f;
    const int m = (int)h->g.M, n = N, k = (int)h->g.K;
    rocblas_status rs = rocblas_gemm_ex(rh, rocblas_operation_transpose, rocblas_operation_none, m, n, k, &alpha,
                                        h->d_dense, rocblas_datatype_f16_r, k, B, rocblas_datatype_f16_r, k, &beta, C,
                                        rocblas_datatype_f16_r, m, C, rocblas_datatype_f16_r, m,
                                        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    return rs == rocblas_status_success ? LSCD_SUCCESS : LSCD_ERROR_HIP;
}

}  // extern "C"
