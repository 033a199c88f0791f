// Device-side building blocks shared by the gfx950 product kernels of the Load-as-Sparse,
// Compute-as-Dense skinny product (every kernel source includes this header).
//
// Method (Flash-LLM paper review, xllm-io, sections 2-4): the sparse weights are
// streamed from HBM in their packed form, unpacked on chip into a zero-filled dense
// tile ("sparse-to-dense transform"), and multiplied densely on the matrix cores with
// fp32 accumulation; loads of later tiles overlap the unpacking and the multiply of the
// current one.  The pages' design targets A100 Tensor Cores (mma.sync m16n8k16,
// ldmatrix, cp.async); what is kept here is the method, re-laid for CDNA4:
//
//  * one wavefront owns one 64 x 64 format tile per k step: it streams the tile's words
//    with 128-bit buffer loads straight into VGPRs (no LDS staging for the sparse
//    stream), zero-fills its own 8 KB LDS tile, scatters each word with a 16-bit LDS
//    store, and feeds v_mfma_f32_16x16x32_f16 from LDS;
//  * the loads of the next tiles are in flight while the current one is unpacked and
//    multiplied (register stages), and the workgroup's four wavefronts share one B tile
//    staged in LDS, double-buffered, with a single barrier per k step;
//  * tall-skinny shapes are split along K across workgroups; fp32 partial sums go to a
//    workspace and a second kernel adds them in ascending split order (deterministic);
//  * workgroup ids are remapped so that consecutive work items (the same K split,
//    hence the same slice of B) land on the same XCD and share its L2;
//  * for N <= 32 a second variant drops the shared B tile and the barrier: each wavefront
//    of a workgroup takes a quarter of one row block's k range with its own B tile, and
//    the quarters are added through LDS at the end;
//  * for N > 64 a third variant decodes each A tile once per workgroup and gives every
//    wavefront 64 columns of B (up to 256 per launch).
//
// LDS tile layout (A and B alike): 128-byte rows of 64 fp16, 16-byte chunks XOR-swizzled
// by (row & 7), so the 16 rows read by one MFMA operand load spread over the banks.

#pragma once

#include <hip/hip_runtime.h>

#include "lscd_internal.h"

namespace lscd {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(4))) const uint32_t kconst_u32;

constexpr int kRowBytes = kTileK * 2;           // 128
constexpr int kTileBytes = kTileM * kRowBytes;  // 8192
constexpr int kBufWord3 = 0x00020000;           // raw buffer descriptor, word 3 (gfx9)
constexpr int kStreamPolicy = 2;                // "nt": the packed words are read exactly once

__device__ __forceinline__ uint32_t lds_chunk(uint32_t r, uint32_t chunk) {
    return r * kRowBytes + (((chunk ^ r) & 7u) << 4);
}

__device__ __forceinline__ uint16_t f16_bits(float x) {
    _Float16 h = (_Float16)x;  // v_cvt_f16_f32, round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// Place one word of the Tiled-CSL layout as written by the encoder (fp16 value in bits
// [15:0], row-major in-tile index r*64 + c in bits [31:16]) into the wavefront's LDS tile.
// The index is masked to the 4096-entry tile, so no word can reach outside the wavefront's
// own 8 KB.  Used for the residual words of the three-level format.
__device__ __forceinline__ void put_word(unsigned char* As, uint32_t w) {
    uint32_t b = (w >> 15) & 0x1FFEu;  // byte offset r*128 + c*2
    b ^= (b >> 3) & 0x70u;             // chunk ^= row & 7
    *reinterpret_cast<uint16_t*>(As + b) = (uint16_t)w;
}

// Issue the loads of one tile's words: lane l of slot j gets vector 64*j + l.  The buffer
// descriptor covers exactly the tile, so lanes past its end read zero without touching
// memory (and a tile of 0 vectors costs no traffic).
template <int R>
__device__ __forceinline__ void load_tile(u32x4 (&wb)[R], const uint32_t* words, uint32_t first,
                                          int nvec, int lane) {
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(words + first), (short)0, nvec * 16, kBufWord3);
#pragma unroll
    for (int j = 0; j < R; ++j)
        wb[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (j * 64 + lane) * 16, 0, kStreamPolicy);
}

__device__ __forceinline__ void zero_tile(unsigned char* As, int lane) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kTileBytes / 1024; ++j) *reinterpret_cast<u32x4*>(As + (j * 64 + lane) * 16) = z;
}

// Tile of TM rows (a multiple of 16, at most 128): TM * 128 bytes, cleared 1 KB per store.
template <int TM>
__device__ __forceinline__ void zero_rows(unsigned char* As, int lane) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < TM * kRowBytes / 1024; ++j) *reinterpret_cast<u32x4*>(As + (j * 64 + lane) * 16) = z;
}

// Scatter the register stage and keep, in place of each stored word, its LDS address: once
// the tile has been multiplied, unscatter() writes zeros at exactly those addresses, which
// returns the tile to all zeros for a fraction of the cost of clearing all 8 KB.  Words past
// the register stage (tiles of more than R * 64 vectors) are placed by scatter_rest(); such
// a tile is cleared whole afterwards.
//
// Device words.  A Tiled-CSL handle on a kernel tile shape keeps its words on the device as
// (LDS byte offset | fp16 value << 16): the offset is where the entry lands in the swizzled
// LDS tile (row r*128 bytes, 16-byte chunk (c/8) ^ (r%8), 2 bytes per column), worked out once
// when the words are uploaded or encoded on the device instead of for every word of every
// product; lscd_export turns them back into the format.
__device__ __forceinline__ uint32_t lds_offset(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint16_t word_value(uint32_t w) { return (uint16_t)(w >> 16); }

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// 32-bit LDS address of a pointer into shared memory, and a 2-byte store at such an address.
__device__ __forceinline__ uint32_t lds_address(unsigned char* p) {
    return (uint32_t)(uintptr_t)(lds_u8*)p;  // address-space cast: shared -> LDS
}
__device__ __forceinline__ void lds_store16(uint32_t addr, uint16_t v) {
    *(lds_u16*)(uintptr_t)addr = v;
}

// The register stage keeps each word's absolute LDS address, so the reset costs no address
// arithmetic at all.
template <int R>
__device__ __forceinline__ void scatter_keep(u32x4 (&wb)[R], int nvec, unsigned char* As, int lane) {
    const uint32_t base = lds_address(As);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j * 64 + lane < nvec) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = wb[j][e];
                const uint32_t a = base + lds_offset(w);
                lds_store16(a, word_value(w));
                wb[j][e] = a;
            }
        }
    }
}

// Scatter without keeping the addresses (the tile is cleared whole afterwards).
template <int R>
__device__ __forceinline__ void scatter_place(const u32x4 (&wb)[R], int nvec, unsigned char* As, int lane) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j * 64 + lane < nvec) {
#pragma unroll
            for (int e = 0; e < 4; ++e) *reinterpret_cast<uint16_t*>(As + lds_offset(wb[j][e])) = word_value(wb[j][e]);
        }
    }
}

template <int R>
__device__ __forceinline__ void scatter_rest(int nvec, unsigned char* As, const uint32_t* tile_words, int lane) {
    for (int v = R * 64 + lane; v < nvec; v += 64) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(tile_words + 4 * (size_t)v);
#pragma unroll
        for (int e = 0; e < 4; ++e) *reinterpret_cast<uint16_t*>(As + lds_offset(x[e])) = word_value(x[e]);
    }
}

template <int R>
__device__ __forceinline__ void unscatter(const u32x4 (&wb)[R], int nvec, int lane) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j * 64 + lane < nvec) {
#pragma unroll
            for (int e = 0; e < 4; ++e) lds_store16(wb[j][e], 0);
        }
    }
}

// Workgroup-cooperative forms: thread t of the workgroup takes vectors t, t + 256, ...
// R * 256 vectors cover the largest 64 x 64 tile (1024 vectors) for R = 4.
template <int R>
__device__ __forceinline__ void load_tile_wg(u32x4 (&wb)[R], const uint32_t* words, uint32_t first, int nvec,
                                             int tid) {
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(words + first), (short)0, nvec * 16, kBufWord3);
#pragma unroll
    for (int j = 0; j < R; ++j)
        wb[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (j * kThreads + tid) * 16, 0, kStreamPolicy);
}

// Clear BYTES (a multiple of 16) of LDS with the workgroup's threads, 16 bytes per store.
template <int BYTES>
__device__ __forceinline__ void zero_buf_wg(unsigned char* buf, int tid) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    constexpr int kChunks = BYTES / 16;
#pragma unroll
    for (int j = 0; j < (kChunks + kThreads - 1) / kThreads; ++j) {
        const int c = j * kThreads + tid;
        if (kChunks % kThreads == 0 || c < kChunks) *reinterpret_cast<u32x4*>(buf + c * 16) = z;
    }
}

// Words past the workgroup's register stage (R * 256 vectors): an encoding may repeat a
// tile's words any number of times, so the stage does not bound a tile; the rest is loaded
// and placed here, thread t taking vectors R * 256 + t, + 256, ...
template <int R>
__device__ __forceinline__ void scatter_rest_wg(int nvec, unsigned char* As, const uint32_t* tile_words, int tid) {
    for (int v = R * kThreads + tid; v < nvec; v += kThreads) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(tile_words + 4 * (size_t)v);
#pragma unroll
        for (int e = 0; e < 4; ++e) *reinterpret_cast<uint16_t*>(As + lds_offset(x[e])) = word_value(x[e]);
    }
}

template <int R>
__device__ __forceinline__ void scatter_tile_wg(const u32x4 (&wb)[R], int nvec, unsigned char* As, int tid) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j * kThreads + tid < nvec) {
#pragma unroll
            for (int e = 0; e < 4; ++e) *reinterpret_cast<uint16_t*>(As + lds_offset(wb[j][e])) = word_value(wb[j][e]);
        }
    }
}

// B tile (64 k x NPAD n) staging: 16-byte chunks, 8 per row of 64 k.  Each pipeline stage
// holds the B chunks of the same k tile as its packed words, so that waiting for a stage
// (the oldest loads in flight; the vector-memory counter retires in order) never waits on
// loads issued for later tiles.
template <int NPAD, bool VEC, int THREADS = kThreads>
struct BStage {
    static constexpr int kChunks = NPAD * 8;
    static constexpr int kPer = (kChunks + THREADS - 1) / THREADS;
    u32x4 r[kPer];

    // VEC (K % 8 == 0): one 16-byte buffer load per chunk; chunks outside B (n >= N, k >= K,
    // or a tile past the split) get an out-of-range offset and read zero without a fetch,
    // so the load sequence has no branches.  Otherwise element-wise guarded loads.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rb, const uint16_t* B, int N, int K, int kt,
                                         int tid, bool valid) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int ch = tid + u * THREADS;
            const int n = ch >> 3, c = ch & 7;
            const int k0 = kt * kTileK + c * 8;
            const bool in = valid && ch < kChunks && n < N && k0 < K;
            if constexpr (VEC) {
                const uint32_t off = in ? (uint32_t)((n * K + k0) * 2) : 0x80000000u;
                r[u] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
            } else {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (in) {
                    const uint16_t* p = B + (size_t)n * K + k0;
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[e] = (k0 + e < K) ? p[e] : 0u;
                    v[0] = h[0] | (h[1] << 16);
                    v[1] = h[2] | (h[3] << 16);
                    v[2] = h[4] | (h[5] << 16);
                    v[3] = h[6] | (h[7] << 16);
                }
                r[u] = v;
            }
        }
    }
    __device__ __forceinline__ void store(unsigned char* Bs, int N, int tid) const {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int ch = tid + u * THREADS;
            const int n = ch >> 3, c = ch & 7;
            if (ch < kChunks && n < N) *reinterpret_cast<u32x4*>(Bs + lds_chunk(n, c)) = r[u];
        }
    }
};

// acc[i][j] += A rows 16i..16i+15 (x 64 k) times B columns 16j..16j+15, i < RG.
template <int NPAD, int RG>
__device__ __forceinline__ void mma_rows(f32x4 (&acc)[RG][NPAD / 16], const unsigned char* As,
                                         const unsigned char* Bs, int lane) {
    const uint32_t rl = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        half8 bf[NPAD / 16];
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j)
            bf[j] = *reinterpret_cast<const half8*>(Bs + lds_chunk(j * 16 + rl, ks * 4 + kq));
#pragma unroll
        for (int i = 0; i < RG; ++i) {
            const half8 af = *reinterpret_cast<const half8*>(As + lds_chunk(i * 16 + rl, ks * 4 + kq));
#pragma unroll
            for (int j = 0; j < NPAD / 16; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
        }
    }
}

// The same product with every operand read issued before the first MFMA: all 2 * (RG + NPAD/16)
// 16-byte LDS reads of the tile are in flight together and the MFMAs then run back to back,
// instead of each MFMA waiting out the latency of its own A read (the compiler, left to
// itself, keeps one or two reads ahead).  Costs 8 * (RG + NPAD/16) VGPRs; for kernels whose
// occupancy the LDS already bounds.
template <int NPAD, int RG>
__device__ __forceinline__ void mma_rows_prefetched(f32x4 (&acc)[RG][NPAD / 16], const unsigned char* As,
                                                    const unsigned char* Bs, int lane) {
    const uint32_t rl = lane & 15, kq = lane >> 4;
    half8 bf[2][NPAD / 16];
    half8 af[2][RG];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j)
            bf[ks][j] = *reinterpret_cast<const half8*>(Bs + lds_chunk(j * 16 + rl, ks * 4 + kq));
#pragma unroll
        for (int i = 0; i < RG; ++i)
            af[ks][i] = *reinterpret_cast<const half8*>(As + lds_chunk(i * 16 + rl, ks * 4 + kq));
    }
    // nothing moves across this point: the scheduler would otherwise sink each read to its MFMA
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < RG; ++i)
#pragma unroll
            for (int j = 0; j < NPAD / 16; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[ks][i], bf[ks][j], acc[i][j], 0, 0, 0);
}

// acc[i][j] += A rows 16i..16i+15 (x 64 k) times B columns 16j..16j+15.
template <int NPAD>
__device__ __forceinline__ void mma_tile(f32x4 (&acc)[4][NPAD / 16], const unsigned char* As,
                                         const unsigned char* Bs, int lane) {
    const uint32_t rl = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        half8 bf[NPAD / 16];
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j)
            bf[j] = *reinterpret_cast<const half8*>(Bs + lds_chunk(j * 16 + rl, ks * 4 + kq));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half8 af = *reinterpret_cast<const half8*>(As + lds_chunk(i * 16 + rl, ks * 4 + kq));
#pragma unroll
            for (int j = 0; j < NPAD / 16; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
        }
    }
}

// Per-wavefront B tile (64 k x NPAD n) staged through registers with coalesced loads: lane l
// of load u takes row n = 8u + (l >> 3), 16-byte chunk (l & 7), so eight consecutive lanes
// read one contiguous 128-byte row segment.  (Loading straight into the MFMA operand layout
// would give every lane of a load a different row of B, one cache access per lane.)  The
// stage is written to the wavefront's own LDS B area right before its MFMAs read it.
template <int NPAD, bool VEC>
struct BWave {
    static constexpr int kPer = NPAD * 8 / 64;
    u32x4 r[kPer];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rb, const uint16_t* B, int N, int K, int kt, int lane,
                                         bool valid) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int n = 8 * u + (lane >> 3), c = lane & 7;
            const int k0 = kt * kTileK + c * 8;
            const bool in = valid && n < N && k0 < K;
            if constexpr (VEC) {
                const uint32_t off = in ? (uint32_t)((n * K + k0) * 2) : 0x80000000u;
                r[u] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
            } else {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (in) {
                    const uint16_t* p = B + (size_t)n * K + k0;
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[e] = (k0 + e < K) ? p[e] : 0u;
                    v[0] = h[0] | (h[1] << 16);
                    v[1] = h[2] | (h[3] << 16);
                    v[2] = h[4] | (h[5] << 16);
                    v[3] = h[6] | (h[7] << 16);
                }
                r[u] = v;
            }
        }
    }
    // rows n >= N are written too (as zeros): the area is private to the wavefront
    __device__ __forceinline__ void store(unsigned char* Bw, int lane) const {
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            *reinterpret_cast<u32x4*>(Bw + lds_chunk(8 * u + (lane >> 3), lane & 7)) = r[u];
    }
};

// Write one wavefront's results: RG x NCB blocks of 16 x 16 fp32 sums in the MFMA layout
// (lane l holds column l & 15, rows 4 * (l >> 4) + 0..3 of each block) for rows m0 .. m0 + 16 RG - 1
// and columns n0 .. n0 + 16 NCB - 1; fp16 to C (N x M) when a.S == 1, else the fp32 partial sums
// of split s.  They leave through `red`, LDS private to the wavefront (16 * LD floats), 16
// columns at a time, transposed so that each store writes whole 128-byte lines: a column's rows
// are contiguous in C and in the partial sums.  (Stored straight from the MFMA layout, a store
// instruction would write 16 columns x 4 rows, a 64-byte piece of 16 different lines.)  The
// wavefront's LDS operations run in order, so no barrier is needed.
template <int RG, int NCB, int LD>
__device__ __forceinline__ void store_results(const f32x4 (&acc)[RG][NCB], float* red, const SpmmArgs& a, int s,
                                              int m0, int n0, int lane) {
    constexpr int TM = 16 * RG;
    static_assert(LD >= TM, "a column of the block fits its stride");
    const int ncol = lane & 15;
    const int mq = (lane >> 4) * 4;
    const bool vec_m = (a.M & 3) == 0;
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
#pragma unroll
        for (int i = 0; i < RG; ++i) *reinterpret_cast<f32x4*>(red + ncol * LD + i * 16 + mq) = acc[i][j];
#pragma unroll
        for (int it = lane; it < 16 * (TM / 4); it += 64) {
            const int c = it / (TM / 4);
            const int ml = (it - c * (TM / 4)) * 4;
            const int n = n0 + j * 16 + c;
            const int m = m0 + ml;
            if (n >= a.N || m >= a.M) continue;
            const f32x4 v = *reinterpret_cast<const f32x4*>(red + c * LD + ml);
            if (a.S == 1) {
                uint16_t* dst = a.C + (int64_t)n * a.M + m;
                if (vec_m && m + 3 < a.M) {
                    uint2 pk;
                    pk.x = (uint32_t)f16_bits(v[0]) | ((uint32_t)f16_bits(v[1]) << 16);
                    pk.y = (uint32_t)f16_bits(v[2]) | ((uint32_t)f16_bits(v[3]) << 16);
                    *reinterpret_cast<uint2*>(dst) = pk;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (m + e < a.M) dst[e] = f16_bits(v[e]);
                }
            } else if (a.PB) {
                // partial sums in blocks of TM rows: the workgroup's rows of every column lie
                // together; rows past M in the last block are padding the split-K pass never reads
                *reinterpret_cast<f32x4*>(a.part + (((int64_t)s * a.MB + m0 / TM) * a.N + n) * TM + ml) = v;
            } else {
                float* dst = a.part + ((int64_t)s * a.N + n) * a.M + m;
                if (vec_m && m + 3 < a.M) {
                    *reinterpret_cast<f32x4*>(dst) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (m + e < a.M) dst[e] = v[e];
                }
            }
        }
    }
}

template <typename Kern>
hipError_t run(Kern k, const SpmmArgs& a, int grid, hipStream_t st, int* occ, int threads = kThreads) {
    if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, k, threads, 0);
    hipLaunchKernelGGL(k, dim3(grid), dim3(threads), 0, st, a);
    return hipGetLastError();
}


}  // namespace
}  // namespace lscd
