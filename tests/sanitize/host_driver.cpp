// Drives the library's host code through its C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with hip_host_stub.cpp in place of the GPU): the three
// encoders on ragged and degenerate shapes, import validation of valid and invalid encodings,
// the handle life cycle (import, info, export, destroy), argument errors, and the
// allocation-failure path.  Every result is checked here as well; the sanitizers check the
// memory and arithmetic, and the leak checker that every handle and failed import frees what
// it took.  Prints "ok" and exits 0 when every check passes.  Test infrastructure only.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "lscd.h"

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

struct Mat {
    int64_t M, K;
    std::vector<uint16_t> A;
    std::vector<uint8_t> mask;
};

static Mat random_mat(int64_t M, int64_t K, double keep, uint32_t seed) {
    Mat m{M, K, std::vector<uint16_t>((size_t)(M * K)), std::vector<uint8_t>((size_t)(M * K))};
    std::mt19937 rng(seed);
    std::uniform_real_distribution<double> u(0.0, 1.0);
    for (size_t i = 0; i < m.A.size(); ++i) {
        m.A[i] = (uint16_t)(rng() & 0xFFFFu);
        if ((m.A[i] & 0x7C00u) == 0x7C00u) m.A[i] &= 0xBFFFu;  // no inf / NaN patterns
        m.mask[i] = u(rng) < keep ? 1 : 0;
    }
    return m;
}

// Plain decode of a Tiled-CSL encoding (value bits [15:0], in-tile index bits [31:16]).
static bool decode_matches(const Mat& m, const std::vector<uint32_t>& w, const std::vector<uint32_t>& o, int tm,
                           int tk) {
    const int64_t KT = (m.K + tk - 1) / tk;
    std::vector<uint16_t> d((size_t)(m.M * m.K), 0);
    for (size_t t = 0; t + 1 < o.size(); ++t) {
        const int64_t bm = (int64_t)t / KT, bk = (int64_t)t % KT;
        for (uint32_t i = o[t]; i < o[t + 1]; ++i) {
            const uint32_t idx = w[i] >> 16;
            const int64_t r = bm * tm + idx / tk, c = bk * tk + idx % tk;
            if (r >= m.M || c >= m.K) return false;
            d[(size_t)(r * m.K + c)] = (uint16_t)(w[i] & 0xFFFFu);
        }
    }
    for (size_t i = 0; i < d.size(); ++i)
        if (d[i] != (m.mask[i] ? m.A[i] : 0)) return false;
    return true;
}

static void tiled_csl_round_trip(int64_t M, int64_t K, double keep, int tm, int tk, uint32_t seed) {
    Mat m = random_mat(M, K, keep, seed);
    int64_t nw = -1, T = -1;
    CHECK(lscd_pack_size(m.A.data(), m.mask.data(), M, K, tm, tk, &nw, &T) == LSCD_SUCCESS);
    std::vector<uint32_t> w((size_t)(nw > 0 ? nw : 1)), o((size_t)T + 1);
    CHECK(lscd_pack(m.A.data(), m.mask.data(), M, K, tm, tk, w.data(), nw, o.data(), T + 1) == LSCD_SUCCESS);
    w.resize((size_t)nw);
    CHECK(decode_matches(m, w, o, tm, tk));
    // a buffer one word short is refused
    if (nw > 0)
        CHECK(lscd_pack(m.A.data(), m.mask.data(), M, K, tm, tk, w.data(), nw - 1, o.data(), T + 1) ==
              LSCD_ERROR_INVALID_VALUE);
    lscd_handle_t h = nullptr;
    CHECK(lscd_import(w.data(), nw, o.data(), M, K, tm, tk, &h) == LSCD_SUCCESS);
    if (!h) return;
    lscd_info_t info;
    CHECK(lscd_get_info(h, &info) == LSCD_SUCCESS);
    CHECK(info.nnz_padded == nw && info.num_tiles == T && info.M == M && info.K == K);
    std::vector<uint32_t> w2((size_t)(nw > 0 ? nw : 1)), o2((size_t)T + 1);
    CHECK(lscd_export(h, w2.data(), o2.data()) == LSCD_SUCCESS);
    CHECK(memcmp(w2.data(), w.data(), (size_t)nw * 4) == 0);
    CHECK(o2 == o);
    // no GPU behind the stub: a well-formed product call reaches the launch and reports it
    std::vector<uint16_t> B(16 * (size_t)K + 8), C(16 * (size_t)M + 8);
    void* Bp = (void*)(((uintptr_t)B.data() + 15) & ~(uintptr_t)15);
    void* Cp = (void*)(((uintptr_t)C.data() + 15) & ~(uintptr_t)15);
    if (tk == 64 && (tm == 64 || tm == 80 || tm == 96 || tm == 112 || tm == 128)) {
        CHECK(lscd_spmm(h, Bp, Cp, 8, nullptr) == LSCD_ERROR_HIP);
    } else {
        CHECK(lscd_spmm(h, Bp, Cp, 8, nullptr) == LSCD_ERROR_NOT_SUPPORTED);
    }
    CHECK(lscd_spmm(h, (char*)Bp + 2, Cp, 8, nullptr) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_spmm(h, Bp, Cp, 0, nullptr) == LSCD_SUCCESS);
    CHECK(lscd_spmm(h, Bp, Cp, -1, nullptr) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_destroy(h) == LSCD_SUCCESS);
}

static void invalid_imports() {
    Mat m = random_mat(40, 70, 0.5, 7);
    const int tm = 16, tk = 32;
    int64_t nw = 0, T = 0;
    CHECK(lscd_pack_size(m.A.data(), m.mask.data(), m.M, m.K, tm, tk, &nw, &T) == LSCD_SUCCESS);
    std::vector<uint32_t> w((size_t)nw), o((size_t)T + 1);
    CHECK(lscd_pack(m.A.data(), m.mask.data(), m.M, m.K, tm, tk, w.data(), nw, o.data(), T + 1) == LSCD_SUCCESS);
    auto expect_bad = [&](const std::vector<uint32_t>& ww, const std::vector<uint32_t>& oo, int64_t n) {
        lscd_handle_t h = nullptr;
        CHECK(lscd_import(ww.data(), n, oo.data(), m.M, m.K, tm, tk, &h) == LSCD_ERROR_INVALID_FORMAT);
        CHECK(h == nullptr);
    };
    {
        auto o2 = o;
        o2[0] = 4;
        expect_bad(w, o2, nw);
    }
    {
        auto o2 = o;
        std::swap(o2[1], o2[2]);
        if (o2[1] != o2[2]) expect_bad(w, o2, nw);
    }
    {
        auto o2 = o;
        o2[1] += 1;
        expect_bad(w, o2, nw);
    }
    expect_bad(w, o, nw - 4);
    {
        auto w2 = w;
        w2[0] = (w2[0] & 0xFFFFu) | ((uint32_t)(tm * tk) << 16);  // outside the tile
        expect_bad(w2, o, nw);
    }
    {
        auto w2 = w;  // the last tile is an edge tile (70 = 2 * 32 + 6 columns): column 31 is outside A
        const size_t t = o.size() - 2;
        if (o[t + 1] > o[t]) {
            w2[o[t]] = (w2[o[t]] & 0xFFFFu) | ((uint32_t)31 << 16);
            expect_bad(w2, o, nw);
        }
    }
    {
        auto w2 = w;  // a second word at the first word's position with other bits
        if (o[1] - o[0] >= 2) {
            w2[o[0] + 1] = (w2[o[0]] & 0xFFFF0000u) | ((w2[o[0]] + 1u) & 0xFFFFu);
            expect_bad(w2, o, nw);
        }
    }
    lscd_handle_t h = nullptr;
    CHECK(lscd_import(nullptr, nw, o.data(), m.M, m.K, tm, tk, &h) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_import(w.data(), nw, nullptr, m.M, m.K, tm, tk, &h) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_import(w.data(), nw, o.data(), 0, m.K, tm, tk, &h) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_import(w.data(), nw, o.data(), m.M, m.K, 300, 300, &h) == LSCD_ERROR_INVALID_VALUE);
}

static void variant_formats(int64_t M, int64_t K, double keep, uint32_t seed) {
    Mat m = random_mat(M, K, keep, seed);
    int64_t nw = -1, T = -1;
    CHECK(lscd_pack_bitmap_size(m.A.data(), m.mask.data(), M, K, &nw, &T) == LSCD_SUCCESS);
    std::vector<uint32_t> w((size_t)(nw > 0 ? nw : 1)), o((size_t)T + 1);
    CHECK(lscd_pack_bitmap(m.A.data(), m.mask.data(), M, K, w.data(), nw, o.data(), T + 1) == LSCD_SUCCESS);
    CHECK((int64_t)o[(size_t)T] * 4 == nw);
    lscd_handle_t h = nullptr;
    CHECK(lscd_encode_bitmap(m.A.data(), m.mask.data(), M, K, &h) == LSCD_SUCCESS);
    if (h) {
        std::vector<uint32_t> w2((size_t)(nw > 0 ? nw : 1)), o2((size_t)T + 1);
        CHECK(lscd_export(h, w2.data(), o2.data()) == LSCD_SUCCESS);
        CHECK(memcmp(w2.data(), w.data(), (size_t)nw * 4) == 0 && o2 == o);
        CHECK(lscd_destroy(h) == LSCD_SUCCESS);
    }
    CHECK(lscd_pack_three_level_size(m.A.data(), m.mask.data(), M, K, &nw, &T) == LSCD_SUCCESS);
    w.assign((size_t)(nw > 0 ? nw : 1), 0);
    o.assign((size_t)T + 1, 0);
    CHECK(lscd_pack_three_level(m.A.data(), m.mask.data(), M, K, w.data(), nw, o.data(), T + 1) == LSCD_SUCCESS);
    h = nullptr;
    CHECK(lscd_encode_three_level(m.A.data(), m.mask.data(), M, K, &h) == LSCD_SUCCESS);
    if (h) {
        std::vector<uint32_t> w2((size_t)(nw > 0 ? nw : 1)), o2((size_t)T + 1);
        CHECK(lscd_export(h, w2.data(), o2.data()) == LSCD_SUCCESS);
        CHECK(memcmp(w2.data(), w.data(), (size_t)nw * 4) == 0 && o2 == o);
        CHECK(lscd_destroy(h) == LSCD_SUCCESS);
    }
}

static void allocation_failure() {
    Mat m = random_mat(130, 200, 0.3, 11);
    int64_t nw = 0, T = 0;
    CHECK(lscd_pack_size(m.A.data(), m.mask.data(), m.M, m.K, 64, 64, &nw, &T) == LSCD_SUCCESS);
    std::vector<uint32_t> w((size_t)nw), o((size_t)T + 1);
    CHECK(lscd_pack(m.A.data(), m.mask.data(), m.M, m.K, 64, 64, w.data(), nw, o.data(), T + 1) == LSCD_SUCCESS);
    setenv("LSCD_TEST_FAIL_ALLOC", "1", 1);
    lscd_handle_t h = nullptr;
    CHECK(lscd_import(w.data(), nw, o.data(), m.M, m.K, 64, 64, &h) == LSCD_ERROR_OUT_OF_MEMORY);
    CHECK(h == nullptr);
    CHECK(lscd_encode(m.A.data(), m.mask.data(), m.M, m.K, &h) == LSCD_ERROR_OUT_OF_MEMORY);
    CHECK(h == nullptr);
    CHECK(lscd_encode_bitmap(m.A.data(), m.mask.data(), m.M, m.K, &h) == LSCD_ERROR_OUT_OF_MEMORY);
    CHECK(h == nullptr);
    unsetenv("LSCD_TEST_FAIL_ALLOC");
    CHECK(lscd_import(w.data(), nw, o.data(), m.M, m.K, 64, 64, &h) == LSCD_SUCCESS);
    CHECK(lscd_destroy(h) == LSCD_SUCCESS);
    CHECK(lscd_destroy(nullptr) == LSCD_SUCCESS);
}

static void argument_errors() {
    Mat m = random_mat(10, 10, 0.5, 3);
    int64_t nw = 0, T = 0;
    CHECK(lscd_pack_size(nullptr, nullptr, 10, 10, 64, 64, &nw, &T) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_pack_size(m.A.data(), nullptr, 10, 10, 0, 64, &nw, &T) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_pack_size(m.A.data(), nullptr, 10, 10, 256, 257, &nw, &T) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_pack_size(m.A.data(), nullptr, 0, 10, 64, 64, &nw, &T) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_pack_size(m.A.data(), nullptr, 10, 10, 64, 64, nullptr, &T) == LSCD_ERROR_INVALID_VALUE);
    lscd_info_t info;
    CHECK(lscd_get_info(nullptr, &info) == LSCD_ERROR_INVALID_VALUE);
    CHECK(lscd_spmm(nullptr, nullptr, nullptr, 8, nullptr) == LSCD_ERROR_INVALID_VALUE);
    CHECK(strlen(lscd_status_string(LSCD_ERROR_HIP)) > 0 && strlen(lscd_status_string((lscd_status_t)99)) > 0);
    int32_t tm = 0;
    CHECK(lscd_default_tile_m(28672, 7168, &tm) == LSCD_SUCCESS && tm == 112);
    CHECK(lscd_default_tile_m(12288, 49152, &tm) == LSCD_SUCCESS && tm == 64);
}

int main() {
    const int shapes[][2] = {{1, 1}, {1, 70}, {63, 1}, {64, 64}, {65, 130}, {200, 333}, {257, 129}};
    const double keeps[] = {0.0, 0.05, 0.4, 1.0};
    uint32_t seed = 1;
    for (auto& s : shapes)
        for (double k : keeps) {
            tiled_csl_round_trip(s[0], s[1], k, 64, 64, seed++);
            tiled_csl_round_trip(s[0], s[1], k, 112, 64, seed++);
            tiled_csl_round_trip(s[0], s[1], k, 7, 9, seed++);
            variant_formats(s[0], s[1], k, seed++);
        }
    tiled_csl_round_trip(300, 400, 0.3, 128, 64, seed++);
    tiled_csl_round_trip(300, 400, 0.3, 256, 256, seed++);
    {  // the host encoder's bank-ordering off: still a valid encoding
        setenv("LSCD_NO_REORDER", "1", 1);
        tiled_csl_round_trip(200, 300, 0.3, 64, 64, seed++);
        unsetenv("LSCD_NO_REORDER");
    }
    invalid_imports();
    allocation_failure();
    argument_errors();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
