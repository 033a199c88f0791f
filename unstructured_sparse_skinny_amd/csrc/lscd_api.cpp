// C-ABI layer: handles, argument checks, split-K planning and launches.
// Entry points are declared and documented in include/lscd.h.

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "lscd_internal.h"


namespace {

using lscd::Grid;

lscd_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return LSCD_SUCCESS;
    if (e == hipErrorOutOfMemory) return LSCD_ERROR_OUT_OF_MEMORY;
    return LSCD_ERROR_HIP;
}

void free_handle(lscd_handle_s* h) {
    if (!h) return;
    if (h->d_words) (void)hipFree(h->d_words);
    if (h->d_offs) (void)hipFree(h->d_offs);
    if (h->d_part) (void)hipFree(h->d_part);
    lscd::release_dense(h);
    delete h;
}

// Encodings below this size run without K splits (one launch; see plan_splits).
constexpr int64_t kSmallFormatBytes = (int64_t)16 << 20;

// Number of K splits for one N padding.  LSCD_SPLITK overrides (tests and tuning).
//
// Independent-wavefront variants (one workgroup per row block and split): each work item is
// 1/S of a row block's k range, and a CU ends up with ceil(groups * S / CUs) of them, so the
// busiest CU carries ceil(groups * S / CUs) / S row blocks of work.  S minimises that, with
// a 1 % charge per split for the fp32 partial sums and the second pass.  E.g. 192 row blocks
// on 256 CUs: S = 1, 2, 3 leave the busiest CU one full block, S = 4 three quarters
// (measured 6-14 % faster than 2 splits on 12288-row matrices).  Every split keeps at least
// tiles_per_split_min k tiles.
//
// Shared-B variant: as many workgroups as the GPU holds at once (CUs x resident workgroups
// per CU, from the kernel's real occupancy), so the whole grid runs in a single wave.
int plan_splits(const Grid& g, int cus, int blocks_per_cu, int64_t groups, int tiles_per_split_min, bool indep,
                bool widen_low_fill = false, int64_t format_bytes = -1) {
    int64_t S = 1;
    const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(g.KT / tiles_per_split_min, 64));
    const char* e = getenv("LSCD_SPLITK");
    if (e && atoll(e) > 0) {
        S = atoll(e);
    } else if (format_bytes >= 0 && format_bytes < kSmallFormatBytes) {
        // A product this small is bound by launch latency, not by how its tiles spread over the
        // CUs: a second (reduction) launch costs more than a split can save.  Measured on
        // 1024 x 1024 at 80 % sparsity, N = 8: 6.7 us with 2 splits, 6.2 us with one launch.
        S = 1;
    } else if (indep) {
        // at most 4: measured on OPT-175B QKV (80-row tiles), 6 splits cost 22 % over 1
        // although the count above favours them -- each split adds a pipeline start-up and
        // an fp32 partial per workgroup
        double best = 0;
        for (int64_t s = 1; s <= std::min<int64_t>(smax, 4); ++s) {
            const double load = (double)((groups * s + cus - 1) / cus) / (double)s * (1.0 + 0.01 * (double)s);
            if (s == 1 || load < best) {
                best = load;
                S = s;
            }
        }
    } else {
        const int64_t slots = (int64_t)cus * std::max(1, blocks_per_cu);
        S = std::min<int64_t>(slots / groups, smax);
        // Slots less than 80 % full: twice the splits, i.e. a second, partial round of
        // workgroups.  Measured on the Tiled-CSL shared-B and N > 64 kernels: 192 row blocks
        // (OPT-175B OutProj, MLP2, config 4) at N = 128 go 105 -> 99, 381 -> 341 and 339 ->
        // 301 us, and OPT-175B MLP1 at N = 64 (192 groups of 4) 248 -> 232 us.  Fills of 90 %
        // and more (config 2, OPT-175B QKV and MLP1 at N = 128, config 4 at N = 64) were
        // already the fastest count.  Three-level tiles at N = 64 likewise: OPT-175B MLP1
        // 240 -> 224 us.
        if (widen_low_fill && S * groups * 5 < slots * 4) S = std::min<int64_t>(2 * S, smax);
    }
    S = std::max<int64_t>(1, std::min<int64_t>(S, g.KT));
    return (int)S;
}

// K splits of the bitmap kernel: the load of the busiest CU, ceil(G*S / cus) / S row-block
// ranges, times the start-up of each wavefront's pipeline (about 4 tiles against its KT / (S
// * waves) tiles).  This picks the measured best of 1, 2 and 4 splits on the OPT shapes: 1 for
// OPT-30B MLP1, OPT-66B QKV and OPT-175B MLP1; 2 for OPT-175B QKV; 4 for OutProj and MLP2.
int plan_splits_bitmap(const Grid& g, int cus, int waves) {
    if (const char* e = getenv("LSCD_SPLITK"); e && atoll(e) > 0)
        return (int)std::max<int64_t>(1, std::min<int64_t>(atoll(e), g.KT));
    const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(g.KT / waves, 8));
    int64_t S = 1;
    double best = 0;
    for (int64_t s = 1; s <= smax; ++s) {
        const double load = (double)((g.MB * s + cus - 1) / cus) / (double)s;
        const double cost = load * (1.0 + 4.0 * (double)(s * waves) / (double)g.KT);
        if (s == 1 || cost < best) {
            best = cost;
            S = s;
        }
    }
    return (int)S;
}

// Tile shapes with product kernels: 64 columns, 64 / 80 / 96 / 112 / 128 rows.
bool kernel_shape(const Grid& g) {
    return g.tk == lscd::kTileK && (g.tm == 64 || g.tm == 80 || g.tm == 96 || g.tm == 112 || g.tm == 128);
}

// Tile height for a matrix of M rows on a GPU of `cus` CUs.  Without a K split every row
// block is one workgroup, so the busiest CU handles ceil(blocks / cus) blocks; a taller tile
// is taken when it cuts that CU's rows by at least 10 % (e.g. 28672 rows: 448 blocks of 64,
// two on most CUs = 128 rows, against 256 blocks of 112 = 112 rows).  Taller tiles also
// serve each staged B tile to more rows.  When 64-row blocks do not fill the GPU, K splits
// balance the work and the tile stays at 64.  LSCD_TILE_M overrides (tuning only).
int32_t choose_tile_m(int64_t M, int cus) {
    if (const char* e = getenv("LSCD_TILE_M")) {
        const int v = atoi(e);
        if (v == 64 || v == 80 || v == 96 || v == 112 || v == 128) return v;
    }
    const int64_t mb64 = (M + 63) / 64;
    if (mb64 <= cus) return 64;
    int32_t best = 64;
    int64_t best_rows = (mb64 + cus - 1) / cus * 64;
    for (int tm : {80, 96, 112, 128}) {
        const int64_t mb = (M + tm - 1) / tm;
        const int64_t rows = (mb + cus - 1) / cus * tm;
        if (rows * 10 < best_rows * 9) {
            best = tm;
            best_rows = rows;
        }
    }
    return best;
}

int current_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -1;
    return cus;
}

int64_t row_groups(const Grid& g, int kind) {
    if (kind == lscd::kKernelShared3) return (g.MB + 2) / 3;
    return kind == lscd::kKernelShared ? (g.MB + lscd::kWaves - 1) / lscd::kWaves : g.MB;
}

// Variant per N padding (measured on MI355X): independent wavefronts for N <= 32 (at N = 32
// they tie with the shared B tile on 12288-row matrices and are 10 % faster on 49152 rows);
// the shared B tile for N = 64, where a per-wavefront B tile would not fit next to the A tile.
// LSCD_KERNEL=shared|indep|indep8 overrides where the variant exists (tuning only).
int pick_kind(int npad) {
    const char* e = getenv("LSCD_KERNEL");
    if (npad > 32) return lscd::kKernelShared;
    if (e && strcmp(e, "shared") == 0) return lscd::kKernelShared;
    if (e && strcmp(e, "indep") == 0) return lscd::kKernelIndep;
    if (e && strcmp(e, "indep8") == 0) return lscd::kKernelIndep8;
    return npad <= 32 ? lscd::kKernelIndep : lscd::kKernelShared;
}

int npad_index(int N) { return N <= 16 ? 0 : (N <= 32 ? 1 : 2); }

// Shared-B kernel at N padded to 64: four or three row blocks per workgroup.  The planner
// fills the resident slots in one wave of workgroups, and slots left over land on some CUs
// only: 192 row blocks in groups of four give 48 x 10 = 480 workgroups for 512 slots, and the
// 32 CUs that get one workgroup idle for the last quarter of the kernel while the other 224
// run two.  Groups of three give 64 x 8 = 512, two on every CU.  The cost compared is the
// busiest CU's work (its workgroups times row blocks times k tiles each).  Measured on the
// OPT-175B shapes at N = 64 (us, four -> three row blocks):
//   - a tie with fewer splits: MLP1 230.5 -> 199.8 (50 % sparsity) and 189.2 -> 174.1 (60 %)
//     (four: 4 splits, 1.5 waves of workgroups; three: 2 splits, one wave), QKV 169.6 -> 162.3;
//   - 6 % less work on the busiest CU with short K ranges: OutProj 57.7 -> 55.3 (60 %);
//   - the same with long ones (96 k tiles per workgroup): the OPT-175B MLP2 shape gains at
//     50 % sparsity, 219.2 -> 199.9, where its tiles take two pipeline stages, and loses at
//     60 %, 172.3 -> 173.3 (config 4 likewise), where they take three: with six wavefronts per
//     CU instead of eight the deeper pipelines lose what the balance gains, so four stay.
// LSCD_KERNEL=shared keeps four, =shared3 forces three.
void plan_shared_rows(const Grid& g, lscd_handle_s* h, int64_t format_bytes) {
    const char* e = getenv("LSCD_KERNEL");
    const bool force3 = e && strcmp(e, "shared3") == 0;
    if (e && !force3) return;
    const int occ3 = lscd::spmm_blocks_per_cu(lscd::kKernelShared3, 64, h->R, (int)std::min<int64_t>(g.K, 1 << 30), g.tm);
    const int64_t g3 = row_groups(g, lscd::kKernelShared3), g4 = row_groups(g, lscd::kKernelShared);
    const int s3 = plan_splits(g, h->cus, occ3, g3, 2, false, true, format_bytes);
    const int s4 = h->S[2];
    auto busiest = [&](int64_t groups, int w, int s) {
        return (double)((groups * s + h->cus - 1) / h->cus) * (double)w * (double)g.KT / (double)s;
    };
    if (occ3 < 2) return;  // no instantiation for this stage and tile height, or one per CU
    const double l3 = busiest(g3, 3, s3), l4 = busiest(g4, 4, s4);
    const bool tie_fewer_splits = l3 >= 0.99 * l4 && l3 <= 1.01 * l4 && s3 < s4;
    const bool lighter = l3 < 0.99 * l4 && (g.KT <= 64 * (int64_t)s3 || lscd::shared_stages(h->R, g.tm) < 3);
    if (force3 || tie_fewer_splits || lighter) {
        h->kind[2] = lscd::kKernelShared3;
        h->S[2] = s3;
    }
}

}  // namespace

namespace lscd {

// Staging registers per lane (vectors of 4 words) of the register stage, from the instantiated
// choices; LSCD_MAX_R caps it (tests use it to force the path past the stage).
static const int kRegChoices[] = {2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 16};

int pick_reg_vectors(int32_t max_tile_words) {
    const int need = ((max_tile_words / 4) + 63) / 64;
    int cap = 16;
    if (const char* e = getenv("LSCD_MAX_R")) cap = atoi(e) > 0 ? atoi(e) : 16;
    int best = 2;
    for (int r : kRegChoices) {
        if (r > cap) break;
        best = r;
        if (r >= need) break;
    }
    return best;
}

int pick_reg_vectors_tall(int32_t max_tile_words) {
    const int r = pick_reg_vectors(max_tile_words);
    return r <= 4 ? 4 : (r <= 6 ? 6 : (r >= 12 ? 12 : r));
}

int pick_reg_vectors_wide(int32_t max_tile_words) {
    const int need = ((max_tile_words / 4) + kThreads - 1) / kThreads;
    return need <= 1 ? 1 : (need <= 2 ? 2 : (need <= 4 ? 4 : 8));
}

// A handle for grid g with its kernel plan (variants, K splits) and split-K workspace; the
// caller supplies the encoding buffers.
lscd_status_t new_handle(const Grid& g, int64_t nnz, int64_t nwords, int32_t maxw, lscd_handle_s** out, int format) {
    lscd_handle_s* h = new (std::nothrow) lscd_handle_s();
    if (!h) return LSCD_ERROR_OUT_OF_MEMORY;
    h->g = g;
    h->nnz = nnz;
    h->nnz_padded = nwords;
    h->max_tile_words = maxw;
    h->format = format;
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) {
        free_handle(h);
        return LSCD_ERROR_HIP;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) == hipSuccess && cus > 0)
        h->cus = cus;
    const bool kernel_tile = kernel_shape(g);
    const bool tall = g.tm != kTileM;
    int64_t part = 0;
    if (format == 1) {
        // bitmap tiles: one kernel, launches of <= 64 columns
        for (int i = 0; i < 3 && kernel_tile; ++i) {
            const int npad = 16 << i;
            h->kind[i] = kKernelBitmap;
            h->S[i] = plan_splits_bitmap(g, h->cus, kBitmapWaves);
            if (h->S[i] > 1) part = std::max<int64_t>(part, (int64_t)h->S[i] * g.M * npad * 4);
        }
    }
    if (format == 2) {
        // three-level tiles: one kernel, launches of <= 64 columns
        for (int i = 0; i < 3 && kernel_tile; ++i) {
            const int npad = 16 << i;
            h->kind[i] = kKernelThreeLevel;
            const int occ = spmm_blocks_per_cu(kKernelThreeLevel, npad, 0, (int)std::min<int64_t>(g.K, 1 << 30));
            // N padded to 64: workgroups of four row blocks sharing the B tile, splits that fill
            // the resident slots; N <= 32: one row block per workgroup, splits that balance the
            // busiest CU (OPT-175B QKV at N = 16: 145 -> 131 us with 4 splits)
            const int64_t groups = npad == 64 ? (g.MB + kWaves - 1) / kWaves : g.MB;
            h->S[i] = plan_splits(g, h->cus, occ, groups, 8, npad != 64, true);
            if (h->S[i] > 1) part = std::max<int64_t>(part, (int64_t)h->S[i] * g.M * npad * 4);
        }
    }
    h->R = format != 0 ? 0 : (tall ? pick_reg_vectors_tall(maxw) : pick_reg_vectors(maxw));
    for (int i = 0; i < 3 && kernel_tile && format == 0; ++i) {
        // Tiles taller than 64 rows: eight wavefronts per row block for N <= 32, the shared B
        // tile above.
        h->kind[i] = tall ? (i < 2 ? kKernelIndep8 : kKernelShared) : pick_kind(16 << i);
        const int occ = spmm_blocks_per_cu(h->kind[i], 16 << i, h->R, (int)std::min<int64_t>(g.K, 1 << 30), g.tm);
        const int min_tiles = h->kind[i] == kKernelIndep ? 8 : (h->kind[i] == kKernelIndep8 ? 16 : 2);
        const bool indep = h->kind[i] == kKernelIndep || h->kind[i] == kKernelIndep8;
        h->S[i] = plan_splits(g, h->cus, occ, row_groups(g, h->kind[i]), min_tiles, indep, true, 4 * nwords);
        if (h->kind[i] == kKernelShared && i == 2) plan_shared_rows(g, h, 4 * nwords);
        // the shared-B kernels store partial sums in blocks of whole tiles (MB * tm rows)
        const bool blocked = h->kind[i] == kKernelShared || h->kind[i] == kKernelShared3;
        if (h->S[i] > 1) part = std::max<int64_t>(part, (int64_t)h->S[i] * (blocked ? g.MB * g.tm : g.M) * (16 << i) * 4);
    }
    h->Rw = pick_reg_vectors_wide(maxw);
    for (int i = 0; i < 3 && kernel_tile && format == 0; ++i) {
        const int npad = 128 + 64 * i;
        const int occ = spmm_blocks_per_cu(kKernelWide, npad, h->Rw, (int)std::min<int64_t>(g.K, 1 << 30), g.tm);
        h->Sw[i] = plan_splits(g, h->cus, occ, g.MB, 4, false, true);
        // Fewer splits than would fill every resident slot: each split adds fp32 partial sums,
        // and past about three workgroups per CU they cost more than the extra workgroups hide.
        // At most 3 * CUs / row blocks splits (measured: OPT-175B MLP2 shape at 60 % and N = 96
        // and 128, 192 row blocks, 4 splits instead of 5: 297.1 -> 277.9 and 340.2 -> 317.9 us;
        // OPT-175B QKV at 50 % and N = 128, 576 row blocks, 1 instead of 2: 266.8 -> 248.7 us),
        // and at most two where the row blocks alone about fill the CUs (0.9 - 2 per CU; OPT-30B
        // MLP1 and OPT-66B QKV shapes, 256 and 247 row blocks of 112, at N = 96 and 128: 72.5 ->
        // 65.7, 83.4 -> 76.4 and 112.6 -> 105.7 us against three).
        if (!getenv("LSCD_SPLITK")) {
            h->Sw[i] = (int)std::min<int64_t>(h->Sw[i], std::max<int64_t>(1, 3 * (int64_t)h->cus / g.MB));
            if (g.MB * 10 >= (int64_t)h->cus * 9 && g.MB < 2 * (int64_t)h->cus) h->Sw[i] = std::min(h->Sw[i], 2);
        }
        if (h->Sw[i] > 1) part = std::max<int64_t>(part, (int64_t)h->Sw[i] * g.M * npad * 4);
    }
    // Tall tiles denser than the shared-B kernel's register stage (R vectors of 4 words per
    // lane of each wavefront): N = 33..64 runs the N > 64 kernel instead, whose workgroup
    // decodes each tile together, with N padded to 128.  OPT-30B MLP1 at 50 % sparsity and
    // N = 64: 122 -> 93 us.  Where the tiles fit (60 %) the two tie; at 80 % shared-B is faster.
    if (tall && kernel_tile && format == 0 && (int64_t)maxw > (int64_t)h->R * 64 * 4) {
        h->kind[2] = kKernelWide;
        h->S[2] = h->Sw[0];
    }
    if (const char* fa = getenv("LSCD_TEST_FAIL_ALLOC"); fa && fa[0] == '1') {
        free_handle(h);
        return LSCD_ERROR_OUT_OF_MEMORY;
    }
    if (part > 0) {
        h->part_bytes = part;
        if ((e = hipMalloc((void**)&h->d_part, (size_t)h->part_bytes)) != hipSuccess) {
            h->d_part = nullptr;
            free_handle(h);
            return hip_status(e);
        }
    }
    *out = h;
    return LSCD_SUCCESS;
}

void delete_handle(lscd_handle_s* h) { free_handle(h); }

}  // namespace lscd

namespace {

// Upload a host encoding into a new handle.
lscd_status_t make_handle(const uint32_t* words, int64_t nwords, const uint32_t* offs, const Grid& g,
                          int64_t nnz, int32_t maxw, lscd_handle_t* out, int format = 0) {
    lscd_handle_s* h = nullptr;
    lscd_status_t st = lscd::new_handle(g, nnz, nwords, maxw, &h, format);
    if (st != LSCD_SUCCESS) return st;
    hipError_t e;
    const size_t wbytes = (size_t)std::max<int64_t>(nwords, 4) * 4 + (format == 1 ? lscd::kBitmapSlackBytes : 0);
    if ((e = hipMalloc((void**)&h->d_words, wbytes)) != hipSuccess ||
        (e = hipMalloc((void**)&h->d_offs, (size_t)(g.T + 1) * 4)) != hipSuccess) {
        free_handle(h);
        return hip_status(e);
    }
    if (format == 0 && kernel_shape(g)) {
        // device form of the words (lds byte offset | value << 16), uploaded in slices
        const int64_t slice = (int64_t)1 << 22;
        std::vector<uint32_t> buf((size_t)std::min<int64_t>(std::max<int64_t>(nwords, 1), slice));
        for (int64_t o = 0; o < nwords; o += slice) {
            const int64_t n = std::min<int64_t>(slice, nwords - o);
            lscd::to_device_words(words + o, buf.data(), n);
            if ((e = hipMemcpy(h->d_words + o, buf.data(), (size_t)n * 4, hipMemcpyHostToDevice)) != hipSuccess) {
                free_handle(h);
                return hip_status(e);
            }
        }
    } else if (nwords > 0 &&
               (e = hipMemcpy(h->d_words, words, (size_t)nwords * 4, hipMemcpyHostToDevice)) != hipSuccess) {
        free_handle(h);
        return hip_status(e);
    }
    if ((e = hipMemcpy(h->d_offs, offs, (size_t)(g.T + 1) * 4, hipMemcpyHostToDevice)) != hipSuccess) {
        free_handle(h);
        return hip_status(e);
    }
    *out = h;
    return LSCD_SUCCESS;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

lscd_status_t check_device(const lscd_handle_s* h) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LSCD_ERROR_HIP;
    return dev == h->device ? LSCD_SUCCESS : LSCD_ERROR_INVALID_VALUE;
}

}  // namespace

extern "C" {

const char* lscd_status_string(lscd_status_t s) {
    switch (s) {
        case LSCD_SUCCESS: return "success";
        case LSCD_ERROR_INVALID_VALUE: return "invalid value";
        case LSCD_ERROR_NOT_SUPPORTED: return "not supported";
        case LSCD_ERROR_OUT_OF_MEMORY: return "out of memory";
        case LSCD_ERROR_INVALID_FORMAT: return "invalid format";
        case LSCD_ERROR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

lscd_status_t lscd_pack_size(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, int32_t tile_m,
                             int32_t tile_k, int64_t* nnz_padded, int64_t* num_tiles) {
    try {
        Grid g;
        if (!A || !nnz_padded || !num_tiles || !lscd::make_grid(M, K, tile_m, tile_k, &g))
            return LSCD_ERROR_INVALID_VALUE;
        std::vector<uint32_t> offs;
        int64_t nnz = 0;
        lscd_status_t st = lscd::pack_offsets(A, mask, g, &offs, &nnz);
        if (st != LSCD_SUCCESS) return st;
        *nnz_padded = offs[(size_t)g.T];
        *num_tiles = g.T;
        return LSCD_SUCCESS;
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_pack(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, int32_t tile_m,
                        int32_t tile_k, uint32_t* nonzeros, int64_t nonzeros_len, uint32_t* tile_offsets,
                        int64_t tile_offsets_len) {
    try {
        Grid g;
        if (!A || !tile_offsets || !lscd::make_grid(M, K, tile_m, tile_k, &g)) return LSCD_ERROR_INVALID_VALUE;
        std::vector<uint32_t> offs;
        int64_t nnz = 0;
        lscd_status_t st = lscd::pack_offsets(A, mask, g, &offs, &nnz);
        if (st != LSCD_SUCCESS) return st;
        const int64_t nw = offs[(size_t)g.T];
        if (tile_offsets_len < g.T + 1 || nonzeros_len < nw || (nw > 0 && !nonzeros)) return LSCD_ERROR_INVALID_VALUE;
        lscd::pack_fill(A, mask, g, offs.data(), nonzeros);
        memcpy(tile_offsets, offs.data(), (size_t)(g.T + 1) * 4);
        return LSCD_SUCCESS;
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_encode_tiled(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, int32_t tile_m,
                                int32_t tile_k, lscd_handle_t* out) {
    try {
        Grid g;
        if (!A || !out || !lscd::make_grid(M, K, tile_m, tile_k, &g)) return LSCD_ERROR_INVALID_VALUE;
        *out = nullptr;
        std::vector<uint32_t> offs;
        int64_t nnz = 0;
        lscd_status_t st = lscd::pack_offsets(A, mask, g, &offs, &nnz);
        if (st != LSCD_SUCCESS) return st;
        const int64_t nw = offs[(size_t)g.T];
        std::vector<uint32_t> words((size_t)std::max<int64_t>(nw, 1));
        lscd::pack_fill(A, mask, g, offs.data(), words.data());
        int32_t maxw = 0;
        for (int64_t t = 0; t < g.T; ++t) maxw = std::max<int32_t>(maxw, (int32_t)(offs[t + 1] - offs[t]));
        return make_handle(words.data(), nw, offs.data(), g, nnz, maxw, out);
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_default_tile_m(int64_t M, int64_t K, int32_t* tile_m) {
    if (!tile_m || M < 1 || K < 1) return LSCD_ERROR_INVALID_VALUE;
    const int cus = current_cus();
    if (cus < 0) return LSCD_ERROR_HIP;
    *tile_m = choose_tile_m(M, cus);
    return LSCD_SUCCESS;
}

lscd_status_t lscd_encode(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, lscd_handle_t* out) {
    int32_t tm = LSCD_DEFAULT_TILE_M;
    if (M >= 1 && K >= 1) {
        lscd_status_t st = lscd_default_tile_m(M, K, &tm);
        if (st != LSCD_SUCCESS) return st;
    }
    return lscd_encode_tiled(A, mask, M, K, tm, LSCD_DEFAULT_TILE_K, out);
}

lscd_status_t lscd_pack_bitmap_size(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                                    int64_t* nwords, int64_t* num_tiles) {
    try {
        Grid g;
        if (!A || !nwords || !num_tiles || !lscd::make_grid(M, K, lscd::kTileM, lscd::kTileK, &g))
            return LSCD_ERROR_INVALID_VALUE;
        std::vector<uint32_t> offs;
        int64_t nnz = 0;
        lscd_status_t st = lscd::bitmap_offsets(A, mask, g, &offs, &nnz);
        if (st != LSCD_SUCCESS) return st;
        *nwords = 4 * (int64_t)offs[(size_t)g.T];
        *num_tiles = g.T;
        return LSCD_SUCCESS;
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_pack_bitmap(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, uint32_t* words,
                               int64_t words_len, uint32_t* tile_offsets, int64_t tile_offsets_len) {
    try {
        Grid g;
        if (!A || !tile_offsets || !lscd::make_grid(M, K, lscd::kTileM, lscd::kTileK, &g))
            return LSCD_ERROR_INVALID_VALUE;
        std::vector<uint32_t> offs;
        int64_t nnz = 0;
        lscd_status_t st = lscd::bitmap_offsets(A, mask, g, &offs, &nnz);
        if (st != LSCD_SUCCESS) return st;
        const int64_t nw = 4 * (int64_t)offs[(size_t)g.T];
        if (tile_offsets_len < g.T + 1 || words_len < nw || (nw > 0 && !words)) return LSCD_ERROR_INVALID_VALUE;
        lscd::bitmap_fill(A, mask, g, offs.data(), words);
        memcpy(tile_offsets, offs.data(), (size_t)(g.T + 1) * 4);
        return LSCD_SUCCESS;
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_encode_bitmap(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, lscd_handle_t* out) {
    try {
        Grid g;
        if (!A || !out || !lscd::make_grid(M, K, lscd::kTileM, lscd::kTileK, &g)) return LSCD_ERROR_INVALID_VALUE;
        *out = nullptr;
        std::vector<uint32_t> offs;
        int64_t nnz = 0;
        lscd_status_t st = lscd::bitmap_offsets(A, mask, g, &offs, &nnz);
        if (st != LSCD_SUCCESS) return st;
        const int64_t nw = 4 * (int64_t)offs[(size_t)g.T];
        std::vector<uint32_t> words((size_t)std::max<int64_t>(nw, 1));
        lscd::bitmap_fill(A, mask, g, offs.data(), words.data());
        int32_t maxw = 0;
        for (int64_t t = 0; t < g.T; ++t) maxw = std::max<int32_t>(maxw, (int32_t)(4 * (offs[t + 1] - offs[t])));
        return make_handle(words.data(), nw, offs.data(), g, nnz, maxw, out, 1);
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_pack_three_level_size(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                                         int64_t* nwords, int64_t* num_tiles) {
    try {
        Grid g;
        if (!A || !nwords || !num_tiles || !lscd::make_grid(M, K, lscd::kTileM, lscd::kTileK, &g))
            return LSCD_ERROR_INVALID_VALUE;
        std::vector<uint32_t> offs;
        int64_t nnz = 0;
        lscd_status_t st = lscd::three_level_offsets(A, mask, g, &offs, &nnz);
        if (st != LSCD_SUCCESS) return st;
        *nwords = 4 * (int64_t)offs[(size_t)g.T];
        *num_tiles = g.T;
        return LSCD_SUCCESS;
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_pack_three_level(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, uint32_t* words,
                                    int64_t words_len, uint32_t* tile_offsets, int64_t tile_offsets_len) {
    try {
        Grid g;
        if (!A || !tile_offsets || !lscd::make_grid(M, K, lscd::kTileM, lscd::kTileK, &g))
            return LSCD_ERROR_INVALID_VALUE;
        std::vector<uint32_t> offs;
        int64_t nnz = 0;
        lscd_status_t st = lscd::three_level_offsets(A, mask, g, &offs, &nnz);
        if (st != LSCD_SUCCESS) return st;
        const int64_t nw = 4 * (int64_t)offs[(size_t)g.T];
        if (tile_offsets_len < g.T + 1 || words_len < nw || (nw > 0 && !words)) return LSCD_ERROR_INVALID_VALUE;
        lscd::three_level_fill(A, mask, g, offs.data(), words);
        memcpy(tile_offsets, offs.data(), (size_t)(g.T + 1) * 4);
        return LSCD_SUCCESS;
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_encode_three_level(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                                      lscd_handle_t* out) {
    try {
        Grid g;
        if (!A || !out || !lscd::make_grid(M, K, lscd::kTileM, lscd::kTileK, &g)) return LSCD_ERROR_INVALID_VALUE;
        *out = nullptr;
        std::vector<uint32_t> offs;
        int64_t nnz = 0;
        lscd_status_t st = lscd::three_level_offsets(A, mask, g, &offs, &nnz);
        if (st != LSCD_SUCCESS) return st;
        const int64_t nw = 4 * (int64_t)offs[(size_t)g.T];
        std::vector<uint32_t> words((size_t)std::max<int64_t>(nw, 1));
        lscd::three_level_fill(A, mask, g, offs.data(), words.data());
        int32_t maxw = 0;
        for (int64_t t = 0; t < g.T; ++t) maxw = std::max<int32_t>(maxw, (int32_t)(4 * (offs[t + 1] - offs[t])));
        return make_handle(words.data(), nw, offs.data(), g, nnz, maxw, out, 2);
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_encode_device(const void* A, const void* mask, int64_t M, int64_t K, void* stream,
                                 lscd_handle_t* out) {
    Grid g;
    if (!A || !out || ((uintptr_t)A & 1u) || M < 1 || K < 1) return LSCD_ERROR_INVALID_VALUE;
    *out = nullptr;
    const int cus = current_cus();
    if (cus < 0) return LSCD_ERROR_HIP;
    if (!lscd::make_grid(M, K, choose_tile_m(M, cus), lscd::kTileK, &g)) return LSCD_ERROR_INVALID_VALUE;
    hipStream_t s = (hipStream_t)stream;
    uint32_t* counts = nullptr;
    uint32_t* offs = nullptr;
    uint32_t* words = nullptr;
    unsigned long long* stats = nullptr;
    unsigned long long hs[4] = {0, 0, 0, 0};
    lscd_handle_s* h = nullptr;
    lscd_status_t st = LSCD_SUCCESS;
    hipError_t e;
    if ((e = hipMalloc((void**)&counts, (size_t)g.T * 4)) != hipSuccess ||
        (e = hipMalloc((void**)&offs, (size_t)(g.T + 1) * 4)) != hipSuccess ||
        (e = hipMalloc((void**)&stats, sizeof(hs))) != hipSuccess) {
        st = hip_status(e);
        goto done;
    }
    if ((e = lscd::encode_device((const uint16_t*)A, (const uint8_t*)mask, g, counts, offs, stats, s)) != hipSuccess ||
        (e = hipMemcpyAsync(hs, stats, sizeof(hs), hipMemcpyDeviceToHost, s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess) {
        st = hip_status(e);
        goto done;
    }
    if (hs[3]) {
        st = LSCD_ERROR_NOT_SUPPORTED;  // 2^32 words or more
        goto done;
    }
    if ((st = lscd::new_handle(g, (int64_t)hs[0], (int64_t)hs[1], (int32_t)hs[2], &h)) != LSCD_SUCCESS) goto done;
    if ((e = hipMalloc((void**)&words, (size_t)std::max<unsigned long long>(hs[1], 4) * 4)) != hipSuccess ||
        (e = lscd::encode_device_fill((const uint16_t*)A, (const uint8_t*)mask, g, offs, words,
                                      lscd::reorder_enabled(), s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess) {
        st = hip_status(e);
        goto done;
    }
    h->d_words = words;
    h->d_offs = offs;
    words = nullptr;
    offs = nullptr;
    *out = h;
    h = nullptr;
done:
    if (h) free_handle(h);
    if (words) (void)hipFree(words);
    if (offs) (void)hipFree(offs);
    if (counts) (void)hipFree(counts);
    if (stats) (void)hipFree(stats);
    return st;
}

lscd_status_t lscd_import(const uint32_t* nonzeros, int64_t nnz_padded, const uint32_t* tile_offsets, int64_t M,
                          int64_t K, int32_t tile_m, int32_t tile_k, lscd_handle_t* out) {
    try {
        Grid g;
        if (!tile_offsets || !out || nnz_padded < 0 || (nnz_padded > 0 && !nonzeros) ||
            !lscd::make_grid(M, K, tile_m, tile_k, &g))
            return LSCD_ERROR_INVALID_VALUE;
        *out = nullptr;
        if (nnz_padded >= ((int64_t)1 << 32)) return LSCD_ERROR_NOT_SUPPORTED;
        int64_t nnz = 0;
        int32_t maxw = 0;
        lscd_status_t st = lscd::validate_format(nonzeros, nnz_padded, tile_offsets, g, &nnz, &maxw);
        if (st != LSCD_SUCCESS) return st;
        return make_handle(nonzeros, nnz_padded, tile_offsets, g, nnz, maxw, out);
    } catch (const std::bad_alloc&) {
        return LSCD_ERROR_OUT_OF_MEMORY;
    } catch (...) {
        return LSCD_ERROR_INVALID_VALUE;
    }
}

lscd_status_t lscd_export(lscd_handle_t h, uint32_t* nonzeros, uint32_t* tile_offsets) {
    if (!h || !tile_offsets || (h->nnz_padded > 0 && !nonzeros)) return LSCD_ERROR_INVALID_VALUE;
    lscd_status_t st = check_device(h);
    if (st != LSCD_SUCCESS) return st;
    hipError_t e;
    if (h->nnz_padded > 0 &&
        (e = hipMemcpy(nonzeros, h->d_words, (size_t)h->nnz_padded * 4, hipMemcpyDeviceToHost)) != hipSuccess)
        return hip_status(e);
    if (h->format == 0 && kernel_shape(h->g)) lscd::to_format_words(nonzeros, h->nnz_padded);
    if ((e = hipMemcpy(tile_offsets, h->d_offs, (size_t)(h->g.T + 1) * 4, hipMemcpyDeviceToHost)) != hipSuccess)
        return hip_status(e);
    return LSCD_SUCCESS;
}

lscd_status_t lscd_get_info(lscd_handle_t h, lscd_info_t* info) {
    if (!h || !info) return LSCD_ERROR_INVALID_VALUE;
    memset(info, 0, sizeof(*info));
    info->M = h->g.M;
    info->K = h->g.K;
    info->tile_m = h->g.tm;
    info->tile_k = h->g.tk;
    info->num_tiles = h->g.T;
    info->nnz = h->nnz;
    info->nnz_padded = h->nnz_padded;
    info->format_bytes = 4 * h->nnz_padded + 4 * (h->g.T + 1);
    info->max_tile_words = h->max_tile_words;
    info->device = h->device;
    info->workspace_bytes = h->part_bytes;
    info->reg_vectors = h->R;
    for (int i = 0; i < 3; ++i) {
        info->splits[i] = h->S[i];
        info->variant[i] = h->kind[i];
        info->splits_wide[i] = h->Sw[i];
    }
    info->reg_vectors_wide = h->Rw;
    info->format = h->format;
    return LSCD_SUCCESS;
}

}  // extern "C"

namespace {

// The product behind lscd_spmm and lscd_spmm_noalloc: `part` receives the fp32 partial sums of
// K-split launches and holds `part_bytes`; a launch whose partials would not fit is refused
// with NOT_SUPPORTED before anything is launched.
lscd_status_t spmm_impl(lscd_handle_t h, const void* B, void* C, int32_t N, void* stream, float* part,
                        int64_t part_bytes) {
    if (!h || N < 0) return LSCD_ERROR_INVALID_VALUE;
    if (N == 0) return LSCD_SUCCESS;
    if (!B || !C || !aligned16(B) || !aligned16(C)) return LSCD_ERROR_INVALID_VALUE;
    if (N > LSCD_MAX_N) return LSCD_ERROR_NOT_SUPPORTED;
    if (!kernel_shape(h->g) || (h->format != 0 && h->g.tm != lscd::kTileM)) return LSCD_ERROR_NOT_SUPPORTED;
    const int nb = std::min(N, lscd::kWideMaxN);  // columns of B read by one launch
    if ((int64_t)nb * h->g.K * 2 >= ((int64_t)1 << 31)) return LSCD_ERROR_NOT_SUPPORTED;  // B as one buffer
    lscd_status_t st = check_device(h);
    if (st != LSCD_SUCCESS) return st;
    hipStream_t s = (hipStream_t)stream;
    lscd::SpmmArgs a;
    a.words = h->d_words;
    a.offs = h->d_offs;
    a.part = part;
    a.M = (int32_t)h->g.M;
    a.K = (int32_t)h->g.K;
    a.MB = (int32_t)h->g.MB;
    a.KT = (int32_t)h->g.KT;
    a.TM = h->g.tm;
    a.PB = 0;
    if (h->format == 1) {
        // bitmap tiles: launches of up to 64 columns (the packed tile is read once per launch)
        for (int32_t c0 = 0; c0 < N; c0 += lscd::kBitmapMaxN) {
            const int32_t n = std::min(N - c0, lscd::kBitmapMaxN);
            const int npad = n <= 16 ? 16 : (n <= 32 ? 32 : 64);
            a.B = (const uint16_t*)B + (int64_t)c0 * h->g.K;
            a.C = (uint16_t*)C + (int64_t)c0 * h->g.M;
            a.N = n;
            a.G = (int32_t)h->g.MB;
            a.S = h->S[npad_index(n)];
            a.items = a.G * a.S;
            a.per_xcd = (a.items + 7) / 8;
            if (a.S > 1 && (int64_t)a.S * a.N * h->g.M * 4 > part_bytes) return LSCD_ERROR_NOT_SUPPORTED;
            hipError_t e = lscd::launch_spmm(lscd::kKernelBitmap, npad, 0, a, 8 * a.per_xcd, s);
            if (e != hipSuccess) return hip_status(e);
            if (a.S > 1) {
                e = lscd::launch_reduce(part, a.C, a.S, n, a.M, 0, 0, s);
                if (e != hipSuccess) return hip_status(e);
            }
        }
        return LSCD_SUCCESS;
    }
    if (h->format == 2) {
        // three-level tiles: launches of up to 64 columns
        for (int32_t c0 = 0; c0 < N; c0 += lscd::kThreeLevelMaxN) {
            const int32_t n = std::min(N - c0, lscd::kThreeLevelMaxN);
            const int npad = n <= 16 ? 16 : (n <= 32 ? 32 : 64);
            a.B = (const uint16_t*)B + (int64_t)c0 * h->g.K;
            a.C = (uint16_t*)C + (int64_t)c0 * h->g.M;
            a.N = n;
            a.G = (int32_t)(npad == 64 ? (h->g.MB + lscd::kWaves - 1) / lscd::kWaves : h->g.MB);
            a.S = h->S[npad_index(n)];
            a.items = a.G * a.S;
            a.per_xcd = (a.items + 7) / 8;
            if (a.S > 1 && (int64_t)a.S * a.N * h->g.M * 4 > part_bytes) return LSCD_ERROR_NOT_SUPPORTED;
            hipError_t e = lscd::launch_spmm(lscd::kKernelThreeLevel, npad, 0, a, 8 * a.per_xcd, s);
            if (e != hipSuccess) return hip_status(e);
            if (a.S > 1) {
                e = lscd::launch_reduce(part, a.C, a.S, n, a.M, 0, 0, s);
                if (e != hipSuccess) return hip_status(e);
            }
        }
        return LSCD_SUCCESS;
    }
    // N <= 64: one launch of a skinny kernel.  N > 64: launches of up to 256 columns of the
    // wide kernel (the packed words are read once per launch); a last slice of <= 64 columns
    // goes to the skinny kernels.
    for (int32_t c0 = 0; c0 < N; c0 += lscd::kWideMaxN) {
        const int32_t n = std::min(N - c0, lscd::kWideMaxN);
        int kind, npad, R, S;
        if (n <= LSCD_NARROW_MAX_N && h->kind[npad_index(n)] != lscd::kKernelWide) {
            kind = h->kind[npad_index(n)];
            npad = n <= 16 ? 16 : (n <= 32 ? 32 : 64);
            R = h->R;
            S = h->S[npad_index(n)];
        } else {
            kind = lscd::kKernelWide;
            npad = n <= 128 ? 128 : (n <= 192 ? 192 : 256);
            R = h->Rw;
            S = h->Sw[(npad - 128) / 64];
        }
        a.B = (const uint16_t*)B + (int64_t)c0 * h->g.K;
        a.C = (uint16_t*)C + (int64_t)c0 * h->g.M;
        a.N = n;
        a.G = (int32_t)(kind == lscd::kKernelWide ? h->g.MB : row_groups(h->g, kind));
        a.S = S;
        a.items = a.G * a.S;
        a.per_xcd = (a.items + 7) / 8;
        // the shared-B kernels store partial sums in blocks of whole tiles
        a.PB = (kind == lscd::kKernelShared || kind == lscd::kKernelShared3) ? h->g.tm : 0;
        const int64_t part_rows = a.PB ? (int64_t)a.MB * a.PB : h->g.M;
        if (a.S > 1 && (int64_t)a.S * a.N * part_rows * 4 > part_bytes) return LSCD_ERROR_NOT_SUPPORTED;
        hipError_t e = lscd::launch_spmm(kind, npad, R, a, 8 * a.per_xcd, s);
        if (e != hipSuccess) return hip_status(e);
        if (S > 1) {
            e = lscd::launch_reduce(part, a.C, S, n, a.M, a.PB, a.MB, s);
            if (e != hipSuccess) return hip_status(e);
        }
    }
    return LSCD_SUCCESS;
}

}  // namespace

extern "C" {

lscd_status_t lscd_spmm(lscd_handle_t h, const void* B, void* C, int32_t N, void* stream) {
    return spmm_impl(h, B, C, N, stream, h ? h->d_part : nullptr, h ? h->part_bytes : 0);
}

lscd_status_t lscd_spmm_noalloc(lscd_handle_t h, const void* B, void* C, int32_t N, void* stream) {
    if (!h || N < 0) return LSCD_ERROR_INVALID_VALUE;
    if (N == 0) return LSCD_SUCCESS;
    lscd_status_t st = check_device(h);
    if (st != LSCD_SUCCESS) return st;
    float* part = nullptr;
    hipError_t e = lscd::scratch_partials(h->device, &part);
    if (e != hipSuccess) return hip_status(e);
    return spmm_impl(h, B, C, N, stream, part, lscd::kScratchBytes);
}

lscd_status_t lscd_debug_decode(lscd_handle_t h, void* A_dense, void* stream) {
    if (!h || !A_dense || !aligned16(A_dense)) return LSCD_ERROR_INVALID_VALUE;
    if (!kernel_shape(h->g) || (h->format != 0 && h->g.tm != lscd::kTileM)) return LSCD_ERROR_NOT_SUPPORTED;
    lscd_status_t st = check_device(h);
    if (st != LSCD_SUCCESS) return st;
    lscd::DecodeArgs a;
    a.words = h->d_words;
    a.offs = h->d_offs;
    a.A = (uint16_t*)A_dense;
    a.M = (int32_t)h->g.M;
    a.K = (int32_t)h->g.K;
    a.MB = (int32_t)h->g.MB;
    a.KT = (int32_t)h->g.KT;
    a.T = h->g.T;
    a.TM = h->g.tm;
    const int64_t grid = (h->g.T + lscd::kWaves - 1) / lscd::kWaves;
    if (h->format == 1) return hip_status(lscd::launch_decode_bitmap(a, (int)grid, (hipStream_t)stream));
    if (h->format == 2) return hip_status(lscd::launch_decode_three_level(a, (int)grid, (hipStream_t)stream));
    return hip_status(lscd::launch_decode(h->R, a, (int)grid, (hipStream_t)stream));
}

lscd_status_t lscd_stream_read(const void* src, int64_t bytes, int32_t blocks_per_cu, void* sink, void* stream) {
    if (!src || !sink || !aligned16(src) || ((uintptr_t)sink & 3u) || bytes < 0 || blocks_per_cu < 1 ||
        blocks_per_cu > 64)
        return LSCD_ERROR_INVALID_VALUE;
    const int cus = current_cus();
    if (cus < 0) return LSCD_ERROR_HIP;
    return hip_status(lscd::launch_stream_read(src, bytes & ~(int64_t)15, cus * blocks_per_cu, (uint32_t*)sink,
                                               (hipStream_t)stream));
}

lscd_status_t lscd_destroy(lscd_handle_t h) {
    free_handle(h);
    return LSCD_SUCCESS;
}

}  // extern "C"
