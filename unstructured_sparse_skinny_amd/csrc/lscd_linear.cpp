// Dense / sparse selection for one weight matrix (lscd_attach_dense, lscd_linear and the
// cost model behind them).  Declared and documented in include/lscd.h.
//
// The Flash-LLM review (xllm-io, section 5 "FasterTransformer integration" and section 6
// "N dimension") describes a GEMM wrapper that picks the dense or the sparse MatMul per
// call, because the sparse kernel only wins while the product is memory-bound (small N);
// once N is large the work is compute-bound and the dense library GEMM is faster.  Here
// the dense copy is decoded from the encoding itself, and the dense product is an fp16 GEMM
// with fp32 accumulation: hipBLASLt with the fastest of its heuristic's candidates once
// lscd_tune_dense has timed them for that N, rocBLAS otherwise.

#include <math.h>

#include <algorithm>

#include <hipblaslt/hipblaslt.h>
#include <rocblas/rocblas.h>

#include <utility>
#include <vector>

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

// hipBLASLt state of a handle with a dense copy.
struct LtState {
    hipblasLtHandle_t handle = nullptr;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    struct Tuned {
        int32_t N;
        hipblasLtMatmulAlgo_t algo;
        double us;         // measured mean time per GEMM
        double sparse_us;  // the sparse product's, measured the same way (< 0: not measured)
    };
    std::vector<Tuned> tuned;
};
constexpr size_t kLtWorkspace = (size_t)64 << 20;
constexpr int kLtCandidates = 16;

// Descriptors of C (N x M row-major = M x N column-major) = A (M x K row-major, i.e. K x M
// column-major, transposed) times B (N x K row-major = K x N column-major).
struct LtProblem {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
    bool make(int64_t M, int64_t K, int32_t N) {
        const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
        return hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
               hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta) ==
                   HIPBLAS_STATUS_SUCCESS &&
               hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb) ==
                   HIPBLAS_STATUS_SUCCESS &&
               hipblasLtMatrixLayoutCreate(&a, HIP_R_16F, (uint64_t)K, (uint64_t)M, K) == HIPBLAS_STATUS_SUCCESS &&
               hipblasLtMatrixLayoutCreate(&b, HIP_R_16F, (uint64_t)K, (uint64_t)N, K) == HIPBLAS_STATUS_SUCCESS &&
               hipblasLtMatrixLayoutCreate(&c, HIP_R_16F, (uint64_t)M, (uint64_t)N, M) == HIPBLAS_STATUS_SUCCESS;
    }
    ~LtProblem() {
        if (c) (void)hipblasLtMatrixLayoutDestroy(c);
        if (b) (void)hipblasLtMatrixLayoutDestroy(b);
        if (a) (void)hipblasLtMatrixLayoutDestroy(a);
        if (desc) (void)hipblasLtMatmulDescDestroy(desc);
    }
};

hipblasStatus_t lt_run(const void* A, LtState* lt, LtProblem& pb, const hipblasLtMatmulAlgo_t* algo, const void* B,
                       void* C, hipStream_t s) {
    const float alpha = 1.0f, beta = 0.0f;
    return hipblasLtMatmul(lt->handle, pb.desc, &alpha, A, pb.a, B, pb.b, &beta, C, pb.c, C, pb.c, algo, lt->ws,
                           lt->ws_bytes, s);
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

// Bitmap and three-level kernels cost about the same per tile at any density (their decode
// works per position, not per kept entry): a fixed part plus a time per tile, for N padded to
// 16, 32 and 64, fitted to the OPT-shape measurements of both formats (within about 20 %).
struct TileCost {
    double us0, ns_per_tile;
};
constexpr TileCost kBitmapCost[3] = {{5.0, 0.90}, {5.0, 0.98}, {8.0, 1.20}};
constexpr TileCost kThreeLevelCost[3] = {{5.0, 1.00}, {10.0, 1.20}, {13.0, 1.54}};

// Sparse time of the handle's product: the model's for Tiled-CSL; bitmap and three-level
// handles run one launch per 64 columns, each costed per tile.
double sparse_time(const lscd_handle_s* h, int32_t N) {
    if (h->format == 0) {
        double ts = 0, td = 0;
        model(h->g.M, h->g.K, h->nnz_padded, h->g.T, N, &ts, &td);
        return ts;
    }
    const TileCost* cost = h->format == 1 ? kBitmapCost : kThreeLevelCost;
    const int32_t per = h->format == 1 ? lscd::kBitmapMaxN : lscd::kThreeLevelMaxN;
    double sum = 0;
    for (int32_t c0 = 0; c0 < N; c0 += per) {
        const int32_t n = std::min(N - c0, per);
        const TileCost& c = cost[n <= 16 ? 0 : (n <= 32 ? 1 : 2)];
        sum += c.us0 + 1e-3 * c.ns_per_tile * (double)h->g.T;
    }
    return sum;
}

// The times behind lscd_linear's choice for N: both measured by lscd_tune_dense when it has
// run for this N, the cost model's otherwise (a tuned dense time without a sparse one -- the
// sparse timing failed -- is set against the model's sparse estimate).
void linear_times(const lscd_handle_s* h, int32_t N, double* ts, double* td, bool* measured) {
    double ms, md;
    model(h->g.M, h->g.K, h->nnz_padded, h->g.T, N, &ms, &md);
    *ts = sparse_time(h, N);
    *td = md;
    *measured = false;
    if (const LtState* lt = (const LtState*)h->lt)
        for (const auto& t : lt->tuned)
            if (t.N == N) {
                *td = t.us;
                if (t.sparse_us > 0) {
                    *ts = t.sparse_us;
                    *measured = true;
                }
            }
}

// Dense iff its time is lower (linear_times).
bool use_dense(const lscd_handle_s* h, int32_t N) {
    if (!h->d_dense) return false;
    if (h->crossover >= 0) return N > h->crossover;
    double ts, td;
    bool measured;
    linear_times(h, N, &ts, &td, &measured);
    return td < ts;
}

// Mean time per call (us) of `runs` calls call(r, stream), r = 0 .. runs - 1, run the way a
// model's layer loop runs them: captured once into a HIP graph on a private stream, replayed
// twice untimed, then once between two events.  < 0 when the calls cannot be captured or a
// call fails (the error is cleared; the caller then times them eagerly).
template <typename F>
double graph_time(F call, int runs, hipEvent_t e0, hipEvent_t e1) {
    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    hipGraph_t g = nullptr;
    hipGraphExec_t ge = nullptr;
    double us = -1;
    bool ok = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) == hipSuccess;
    if (ok) {
        for (int r = 0; r < runs && ok; ++r) ok = call(r, s);
        ok = (hipStreamEndCapture(s, &g) == hipSuccess) && ok && g != nullptr;
    }
    if (ok) ok = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) == hipSuccess;
    for (int w = 0; w < 2 && ok; ++w) ok = hipGraphLaunch(ge, s) == hipSuccess;
    float ms = 0;
    if (ok) ok = hipEventRecord(e0, s) == hipSuccess && hipGraphLaunch(ge, s) == hipSuccess &&
                 hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
                 hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
    if (ok) us = 1e3 * (double)ms / runs;
    (void)hipStreamSynchronize(s);
    if (ge) (void)hipGraphExecDestroy(ge);
    if (g) (void)hipGraphDestroy(g);
    (void)hipStreamDestroy(s);
    if (!ok) (void)hipGetLastError();
    return us;
}

// The same, eagerly on the default stream: 2 untimed calls, then `runs` between two events.
template <typename F>
double eager_time(F call, int runs, hipEvent_t e0, hipEvent_t e1) {
    bool ok = true;
    for (int r = 0; r < 2 && ok; ++r) ok = call(r, nullptr);
    if (!ok) return -1;
    (void)hipEventRecord(e0, nullptr);
    for (int r = 0; r < runs && ok; ++r) ok = call(r, nullptr);
    (void)hipEventRecord(e1, nullptr);
    float ms = 0;
    if (hipEventSynchronize(e1) != hipSuccess || !ok || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return -1;
    return 1e3 * (double)ms / runs;
}

}  // namespace

namespace lscd {

void release_dense(lscd_handle_s* h) {
    if (h->lt) {
        LtState* lt = (LtState*)h->lt;
        if (lt->handle) (void)hipblasLtDestroy(lt->handle);
        if (lt->ws) (void)hipFree(lt->ws);
        delete lt;
        h->lt = nullptr;
    }
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

lscd_status_t lscd_linear_times(lscd_handle_t h, int32_t N, double* sparse_us, double* dense_us, int32_t* measured) {
    if (!h || N < 1 || N > LSCD_MAX_N || !sparse_us || !dense_us || !measured) return LSCD_ERROR_INVALID_VALUE;
    bool m = false;
    linear_times(h, N, sparse_us, dense_us, &m);
    *measured = m ? 1 : 0;
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
    if (LtState* lt = (LtState*)h->lt) {
        for (auto& t : lt->tuned) {
            if (t.N != N) continue;
            LtProblem pb;
            if (!pb.make(h->g.M, h->g.K, N)) return LSCD_ERROR_HIP;
            return lt_run(h->d_dense, lt, pb, &t.algo, B, C, (hipStream_t)stream) == HIPBLAS_STATUS_SUCCESS ? LSCD_SUCCESS
                                                                                                 : LSCD_ERROR_HIP;
        }
    }
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

lscd_status_t lscd_tune_dense(lscd_handle_t h, const void* B, void* C, int32_t N, double* best_us,
                              int32_t* candidates) {
    if (!h || !B || !C || !best_us || !candidates || N < 1 || N > LSCD_MAX_N) return LSCD_ERROR_INVALID_VALUE;
    if (((uintptr_t)B & 15u) || ((uintptr_t)C & 15u)) return LSCD_ERROR_INVALID_VALUE;
    if (!h->d_dense) return LSCD_ERROR_NOT_SUPPORTED;
    lscd_status_t st = on_device(h);
    if (st != LSCD_SUCCESS) return st;
    LtState* lt = (LtState*)h->lt;
    if (!lt) {
        lt = new (std::nothrow) LtState();
        if (!lt) return LSCD_ERROR_OUT_OF_MEMORY;
        h->lt = lt;
        if (hipblasLtCreate(&lt->handle) != HIPBLAS_STATUS_SUCCESS) return LSCD_ERROR_HIP;
        hipError_t e = hipMalloc(&lt->ws, kLtWorkspace);
        if (e != hipSuccess) {
            lt->ws = nullptr;
            return hip_st(e);
        }
        lt->ws_bytes = kLtWorkspace;
    }
    LtProblem pb;
    hipblasLtMatmulPreference_t pref = nullptr;
    if (!pb.make(h->g.M, h->g.K, N) || hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS)
        return LSCD_ERROR_HIP;
    const uint64_t wsb = lt->ws_bytes;
    (void)hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof wsb);
    hipblasLtMatmulHeuristicResult_t res[kLtCandidates];
    int got = 0;
    hipblasStatus_t hs = hipblasLtMatmulAlgoGetHeuristic(lt->handle, pb.desc, pb.a, pb.b, pb.c, pb.c, pref,
                                                         kLtCandidates, res, &got);
    (void)hipblasLtMatmulPreferenceDestroy(pref);
    if (hs != HIPBLAS_STATUS_SUCCESS || got < 1) return LSCD_ERROR_NOT_SUPPORTED;
    // Timed as the GEMM runs in a model's layer loop, with its weights coming from HBM rather than
    // from the 256 MiB Infinity Cache: kLtTimedRuns calls over rotating copies of the dense matrix
    // (made here and freed before returning) whose total exceeds three times that cache, as one
    // HIP graph (graph_time; eagerly if it cannot be captured).  One copy run back to back would
    // be served partly from the cache and flatter the GEMM.
    constexpr int kLtTimedRuns = 20;
    const size_t dense_bytes = (size_t)h->g.M * (size_t)h->g.K * 2;
    const size_t mall = (size_t)256 << 20;
    const int ncopies = (int)std::max<size_t>(2, std::min<size_t>(8, (3 * mall + dense_bytes - 1) / dense_bytes + 1));
    std::vector<void*> copies(1, (void*)h->d_dense);
    hipError_t ce = hipSuccess;
    for (int c = 1; c < ncopies && ce == hipSuccess; ++c) {
        void* p = nullptr;
        ce = hipMalloc(&p, dense_bytes);
        if (ce == hipSuccess) {
            copies.push_back(p);
            ce = hipMemcpy(p, h->d_dense, dense_bytes, hipMemcpyDeviceToDevice);
        }
    }
    auto free_copies = [&]() {
        for (size_t c = 1; c < copies.size(); ++c) (void)hipFree(copies[c]);
    };
    if (ce != hipSuccess) {
        free_copies();
        return hip_st(ce);
    }
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) {
        free_copies();
        return LSCD_ERROR_HIP;
    }
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        free_copies();
        return LSCD_ERROR_HIP;
    }
    // The sparse product of the same N, timed the same way: rotating over copies of the packed
    // words (views of this handle that differ only in their words) whose total exceeds three
    // times the cache.  Timed before and after the GEMMs, the lower time kept (timed only after
    // them it came out 4-5 % above bench.py's graph-replay time on the OPT-175B shapes at
    // N <= 64).
    const size_t wbytes = std::max<size_t>(16, (size_t)h->nnz_padded * 4);
    const int nsc = (int)std::max<size_t>(2, std::min<size_t>(8, (3 * mall + wbytes - 1) / wbytes + 1));
    std::vector<lscd_handle_s> views(1, *h);
    std::vector<void*> wcopies;
    hipError_t we = hipSuccess;
    for (int c = 1; c < nsc && we == hipSuccess && h->nnz_padded > 0; ++c) {
        void* p = nullptr;
        we = hipMalloc(&p, wbytes);
        if (we != hipSuccess) break;
        wcopies.push_back(p);
        we = hipMemcpy(p, h->d_words, (size_t)h->nnz_padded * 4, hipMemcpyDeviceToDevice);
        views.push_back(*h);
        views.back().d_words = (uint32_t*)p;
    }
    const bool words_ok = we == hipSuccess;
    if (!words_ok) (void)hipGetLastError();  // sparse timing skipped: clear the failed call's error
    auto time_sparse = [&]() {
        const int nv = (int)views.size();
        auto product = [&](int r, hipStream_t st) { return lscd_spmm(&views[r % nv], B, C, N, st) == LSCD_SUCCESS; };
        double us = graph_time(product, kLtTimedRuns, e0, e1);
        return us < 0 ? eager_time(product, kLtTimedRuns, e0, e1) : us;
    };
    double sparse_us = words_ok ? time_sparse() : -1;

    double best = -1;
    int best_i = -1, tried = 0;
    const int nc = (int)copies.size();
    for (int i = 0; i < got; ++i) {
        if (res[i].state != HIPBLAS_STATUS_SUCCESS || res[i].workspaceSize > lt->ws_bytes) continue;
        auto gemm = [&](int r, hipStream_t st) {
            return lt_run(copies[r % nc], lt, pb, &res[i].algo, B, C, st) == HIPBLAS_STATUS_SUCCESS;
        };
        double us = graph_time(gemm, kLtTimedRuns, e0, e1);
        if (us < 0) us = eager_time(gemm, kLtTimedRuns, e0, e1);
        if (us < 0) continue;
        ++tried;
        if (best < 0 || us < best) {
            best = us;
            best_i = i;
        }
    }
    free_copies();
    if (words_ok) {
        const double again = time_sparse();
        if (again > 0 && (sparse_us < 0 || again < sparse_us)) sparse_us = again;
    }
    for (void* p : wcopies) (void)hipFree(p);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (best_i < 0) return LSCD_ERROR_NOT_SUPPORTED;
    bool found = false;
    for (auto& t : lt->tuned)
        if (t.N == N) {
            t.algo = res[best_i].algo;
            t.us = best;
            t.sparse_us = sparse_us;
            found = true;
        }
    if (!found) lt->tuned.push_back({N, res[best_i].algo, best, sparse_us});
    *best_us = best;
    *candidates = tried;
    return LSCD_SUCCESS;
}

}  // extern "C"
