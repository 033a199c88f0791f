// Internal declarations shared by the host encoder, the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "lscd.h"

namespace lscd {

// Tile shape the gfx950 product kernel is built for: one 64 x 64 tile per wavefront,
// i.e. 4 row blocks of 16 for the 16x16x32 MFMA and two 32-deep k steps.
constexpr int kTileM = 64;
constexpr int kTileK = 64;
// Wavefronts per workgroup; each owns one row block, all share the staged B tile.
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// ---------------------------------------------------------------- host encoder
struct Grid {
    int64_t M, K;
    int32_t tm, tk;
    int64_t MB, KT, T;
};
bool make_grid(int64_t M, int64_t K, int32_t tm, int32_t tk, Grid* g);

struct Packed {
    std::vector<uint32_t> words;
    std::vector<uint32_t> offsets;
    int64_t nnz = 0;
    int32_t max_tile_words = 0;
};

// Count pass only: padded words per tile -> offsets (no words).  Returns NOT_SUPPORTED
// when the total reaches 2^32 words.
lscd_status_t pack_offsets(const uint16_t* A, const uint8_t* mask, const Grid& g,
                           std::vector<uint32_t>* offsets, int64_t* nnz);
// Fill pass into caller storage, offsets from pack_offsets.
void pack_fill(const uint16_t* A, const uint8_t* mask, const Grid& g, const uint32_t* offsets,
               uint32_t* words);
// Bitmap-tile variant: count pass -> offsets in 16-byte units; fill pass into caller storage.
lscd_status_t bitmap_offsets(const uint16_t* A, const uint8_t* mask, const Grid& g,
                             std::vector<uint32_t>* offsets, int64_t* nnz);
void bitmap_fill(const uint16_t* A, const uint8_t* mask, const Grid& g, const uint32_t* offsets, uint32_t* words);
// Three-level variant (4:2 layer, slot filling, residual), 64 x 64 tiles: count pass -> offsets
// in 16-byte units; fill pass into caller storage.
constexpr int kThreeLevelValueWords = 1024;  // 4 operands x 64 lanes x 8 fp16 slots
constexpr int kThreeLevelMetaWords = 256;    // per lane: positions 0|1, positions 2|3, fill mask, codes
constexpr int kThreeLevelFixedWords = kThreeLevelValueWords + kThreeLevelMetaWords;
constexpr int kThreeLevelMaxCodes = 8;
lscd_status_t three_level_offsets(const uint16_t* A, const uint8_t* mask, const Grid& g,
                                  std::vector<uint32_t>* offsets, int64_t* nnz);
void three_level_fill(const uint16_t* A, const uint8_t* mask, const Grid& g, const uint32_t* offsets,
                      uint32_t* words);
// Device form of a Tiled-CSL word on a kernel tile shape (64 columns, 64..128 rows): the
// entry's byte offset in the kernels' swizzled LDS tile (row r at r*128 bytes, 16-byte chunk
// (c/8) ^ (r%8), 2 bytes per column) in bits [15:0], the fp16 value in bits [31:16].  The
// format's word is value | (r*64 + c) << 16; handles keep the device form so that the
// product places a word with one mask, and lscd_export converts back.
__host__ __device__ inline uint32_t device_word(uint32_t idx, uint32_t value) {
    const uint32_t r = idx >> 6, c = idx & 63u;
    return (r * 128u + ((c * 2u) ^ ((r & 7u) << 4))) | (value << 16);
}
__host__ __device__ inline uint32_t format_word(uint32_t dw) {
    const uint32_t b = dw & 0xFFFFu, r = b >> 7;
    const uint32_t c = ((((b >> 4) & 7u) ^ (r & 7u)) << 3) | ((b >> 1) & 7u);
    return (dw >> 16) | ((r * 64u + c) << 16);
}
// Format words <-> device words, n words, on the host threads.
void to_device_words(const uint32_t* in, uint32_t* out, int64_t n);
void to_format_words(uint32_t* words, int64_t n);
// Validate an imported encoding; fills nnz and the largest tile.
lscd_status_t validate_format(const uint32_t* words, int64_t nwords, const uint32_t* offsets,
                              const Grid& g, int64_t* nnz, int32_t* max_tile_words);
// Whether the encoder orders the words of a tile for LDS banks (env LSCD_NO_REORDER=1 turns
// it off, for measurements).
bool reorder_enabled();

// ---------------------------------------------------------------- device side
struct SpmmArgs {
    const uint32_t* words;     // nonzeros, tile after tile
    const uint32_t* offs;      // tile offsets, T + 1
    const uint16_t* B;         // [N][K] fp16
    uint16_t* C;               // [N][M] fp16 (used when S == 1)
    float* part;               // [S][N][M] fp32 partial sums (used when S > 1)
    int32_t M, K, N;
    int32_t MB, KT;            // row blocks, k tiles
    int32_t G, S;              // row groups (kWaves row blocks each), K splits
    int32_t items, per_xcd;    // G * S work items, items per XCD slot range
    int32_t TM;                // rows of the format's tiles: 64, 80, 96, 112 or 128
    int32_t PB;                // partial sums in blocks of PB rows, [S][MB][N][PB]; 0: [S][N][M]
};

struct DecodeArgs {
    const uint32_t* words;
    const uint32_t* offs;
    uint16_t* A;               // [M][K] fp16 out
    int32_t M, K, MB, KT;
    int64_t T;
    int32_t TM;                // rows of the format's tiles
};

// Staging registers per lane and tile that have kernel instantiations.
int pick_reg_vectors(int32_t max_tile_words);
// The same for tiles taller than 64 rows (their kernels exist for R in {4, 6 .. 12}).
int pick_reg_vectors_tall(int32_t max_tile_words);
// Product kernel variants: kKernelShared -- four row blocks per workgroup sharing a B tile
// in LDS (any N); kKernelIndep -- one row block per workgroup, its k range split over the
// wavefronts, B in registers (N <= 32).
constexpr int kKernelShared = 0;
constexpr int kKernelIndep = 1;   // 4 wavefronts per row block
constexpr int kKernelIndep8 = 2;  // 8 wavefronts per row block
// N > 64: one row block per workgroup, its tile decoded by all four wavefronts, 64 columns
// of B per wavefront (N padded to 128, 192 or 256 per launch).
constexpr int kKernelWide = 3;
constexpr int kWideMaxN = 256;
// Bitmap-tile format: one row block per workgroup, kBitmapWaves wavefronts over its k range,
// N padded to 16, 32 or 64 per launch (wider N runs launches of 64 columns).  The allocation of a
// bitmap blob carries kBitmapSlackBytes past its end: a tile's value loads may read up to that
// far past its last value.
constexpr int kKernelBitmap = 4;
constexpr int kBitmapMaxN = 64;
constexpr int kBitmapWaves = 4;
constexpr int kBitmapSlackBytes = 16;
// Three-level tiles (4:2 layer on the structured-sparse MFMA, slot filling, residual): one
// kernel, launches of <= 64 columns.
constexpr int kKernelThreeLevel = 5;
constexpr int kThreeLevelMaxN = 64;
// Tiled-CSL shared-B kernel with three row blocks per workgroup (N padded to 64 only).
constexpr int kKernelShared3 = 6;
// Register stages of the shared-B kernels' prefetch pipeline for R staging vectors per lane
// and TM-row tiles: deeper when a tile needs few registers; taller tiles take two (their
// accumulators leave no room for a third).
constexpr int shared_stages(int R, int TM) { return TM != kTileM ? 2 : (R <= 4 ? 4 : (R <= 8 ? 3 : 2)); }
hipError_t launch_decode_three_level(const DecodeArgs& a, int grid, hipStream_t s);
hipError_t launch_decode_bitmap(const DecodeArgs& a, int grid, hipStream_t s);
// Staging registers per thread and tile of the wide variant (1, 2 or 4).
int pick_reg_vectors_wide(int32_t max_tile_words);
hipError_t launch_spmm(int kind, int npad, int R, const SpmmArgs& a, int grid, hipStream_t s);
// Per-family launch tables (one source file each, compiled in parallel).  occ != nullptr:
// report resident workgroups per CU in *occ instead of launching.
hipError_t launch_kind_skinny16(int kind, int R, const SpmmArgs& a, int grid, hipStream_t s, int* occ);
hipError_t launch_kind_skinny32(int kind, int R, const SpmmArgs& a, int grid, hipStream_t s, int* occ);
hipError_t launch_kind_skinny64(int kind, int R, const SpmmArgs& a, int grid, hipStream_t s, int* occ);
hipError_t launch_kind_wide(int npad, int R, const SpmmArgs& a, int grid, hipStream_t s, int* occ);
hipError_t launch_kind_bitmap(int npad, const SpmmArgs& a, int grid, hipStream_t s, int* occ);
hipError_t launch_kind_three_level(int npad, const SpmmArgs& a, int grid, hipStream_t s, int* occ);
// Workgroups of a product kernel (variant, N padding, stage size) resident per CU.
int spmm_blocks_per_cu(int kind, int npad, int R, int K, int TM = kTileM);
// Split-K pass: C[n][m] = fp16(sum over s of the partial sums), layout [S][N][M] (PB = 0) or
// [S][MB][N][PB] (MB blocks of PB rows).
hipError_t launch_reduce(const float* part, uint16_t* C, int S, int N, int M, int PB, int MB, hipStream_t s);
hipError_t launch_decode(int R, const DecodeArgs& a, int grid, hipStream_t s);
// Partial-sum scratch of lscd_spmm_noalloc: a file-scope device array of kScratchBytes, one
// per GPU, held until the process ends.  scratch_partials returns its address on `device`
// (looked up once per device, then cached).
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
hipError_t scratch_partials(int device, float** ptr);
// Streaming-read reference over `bytes` (a multiple of 16) with `blocks` workgroups.
hipError_t launch_stream_read(const void* src, int64_t bytes, int blocks, uint32_t* sink, hipStream_t s);

// A new handle for grid g: kernel plan, split-K workspace; d_words / d_offs left null for
// the caller to fill.  delete_handle frees a handle and every buffer it holds.
lscd_status_t new_handle(const Grid& g, int64_t nnz, int64_t nwords, int32_t maxw, struct ::lscd_handle_s** out,
                         int format = 0);
void delete_handle(struct ::lscd_handle_s* h);
// Device encoder (64 x 64 tiles): count + scan into counts[T], offs[T+1] and stats
// {nnz, words, largest tile, overflow flag}; then the bank-ordered fill into words.
hipError_t encode_device(const uint16_t* A, const uint8_t* mask, const Grid& g, uint32_t* counts, uint32_t* offs,
                         unsigned long long* stats, hipStream_t s);
hipError_t encode_device_fill(const uint16_t* A, const uint8_t* mask, const Grid& g, const uint32_t* offs,
                              uint32_t* words, bool reorder, hipStream_t s);
// Frees the dense copy and the GEMM library handle of lscd_linear, if any.
void release_dense(struct ::lscd_handle_s* h);

}  // namespace lscd

// The object behind lscd_handle_t.
struct lscd_handle_s {
    lscd::Grid g;
    int device = 0;
    int cus = 256;
    int64_t nnz = 0;
    int64_t nnz_padded = 0;
    int32_t max_tile_words = 0;
    int R = 2;
    int S[3] = {1, 1, 1};     // K splits used by lscd_spmm for N padded to 16, 32, 64
    int kind[3] = {0, 0, 0};  // product kernel variant for N padded to 16, 32, 64
    int format = 0;           // 0 Tiled-CSL, 1 bitmap tiles, 2 three-level tiles
    int Rw = 1;               // staging vectors per thread of the wide (N > 64) variant
    int Sw[3] = {1, 1, 1};    // K splits of the wide variant for N padded to 128, 192, 256
    uint32_t* d_words = nullptr;
    uint32_t* d_offs = nullptr;
    float* d_part = nullptr;
    int64_t part_bytes = 0;
    // dense path of lscd_linear (lscd_attach_dense)
    uint16_t* d_dense = nullptr;  // M x K fp16, row-major
    void* blas = nullptr;         // rocblas_handle
    void* lt = nullptr;           // hipBLASLt state: handle, workspace, tuned algorithms per N
    int32_t crossover = -1;       // sparse iff N <= crossover; -1: cost model
};
