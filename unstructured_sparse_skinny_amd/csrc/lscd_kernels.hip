// gfx950 kernels of the Load-as-Sparse, Compute-as-Dense skinny product.
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
template <int NPAD, bool VEC>
struct BStage {
    static constexpr int kChunks = NPAD * 8;
    static constexpr int kPer = (kChunks + kThreads - 1) / kThreads;
    u32x4 r[kPer];

    // VEC (K % 8 == 0): one 16-byte buffer load per chunk; chunks outside B (n >= N, k >= K,
    // or a tile past the split) get an out-of-range offset and read zero without a fetch,
    // so the load sequence has no branches.  Otherwise element-wise guarded loads.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rb, const uint16_t* B, int N, int K, int kt,
                                         int tid, bool valid) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int ch = tid + u * kThreads;
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
            const int ch = tid + u * kThreads;
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

template <int NPAD, int R, int P, bool VEC, int RG>
__global__ __launch_bounds__(kThreads) void spmm_kernel(SpmmArgs a) {
    constexpr int TM = 16 * RG;          // rows of the format's tiles
    constexpr int kTB = TM * kRowBytes;  // one wavefront's LDS tile
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * kTB + 2 * NPAD * kRowBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* As = smem + wave * kTB;
    unsigned char* Bs0 = smem + kWaves * kTB;

    // XCD-aware work mapping: hardware places workgroup b on XCD b % 8; give each XCD a
    // contiguous run of work items (items are split-major, so a run shares a B slice).
    const int bid = blockIdx.x;
    const int item = (bid & 7) * a.per_xcd + (bid >> 3);
    if (item >= a.items) return;  // whole workgroup
    const int s = item / a.G;
    const int g = item - s * a.G;
    const int kt0 = (int)(((int64_t)s * a.KT) / a.S);
    const int kt1 = (int)(((int64_t)(s + 1) * a.KT) / a.S);
    const int rb = g * kWaves + wave;
    const bool active = rb < a.MB;
    // Tile offsets are read through the constant address space: the offsets are never
    // written by the kernel, and this lets the compiler use scalar loads (counted apart
    // from the vector loads of the packed words) for these wave-uniform addresses.
    const kconst_u32* toff = (const kconst_u32*)(a.offs) + (int64_t)(active ? rb : 0) * a.KT;
    // B as a buffer of N*K fp16 (requires N*K*2 < 2^31, checked by the host)
    const __amdgpu_buffer_rsrc_t bsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.B, (short)0, a.N * a.K * 2, kBufWord3);

    // B rows n >= N stay zero for the whole kernel (both buffers).
    for (int ch = tid; ch < 2 * NPAD * 8; ch += kThreads) {
        const int row = ch >> 3;
        if (row % NPAD >= a.N) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(Bs0 + row * kRowBytes + (ch & 7) * 16) = z;
        }
    }

    // Tile offsets are scalar loads; the one a refill needs is fetched a step earlier, so the
    // loads of a tile are never held up by a round trip for its own offset.
    auto off_at = [&](int i) -> uint32_t { return (active && i <= kt1) ? toff[i] : 0u; };

    u32x4 wb[P][R];
    BStage<NPAD, VEC> bst[P];
    int nv[P];
    uint32_t first[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int k = kt0 + q;
        uint32_t o0 = 0, o1 = 0;
        if (active && k < kt1) {
            o0 = toff[k];
            o1 = toff[k + 1];
        }
        first[q] = o0;
        nv[q] = (int)((o1 - o0) >> 2);
        bst[q].load(bsrc, a.B, a.N, a.K, k, tid, k < kt1);
        load_tile<R>(wb[q], a.words, o0, nv[q], lane);
    }
    uint32_t o_next = off_at(kt0 + P);      // start of the next tile to fetch
    uint32_t o_pf = off_at(kt0 + P + 1);    // its end, prefetched

    f32x4 acc[RG][NPAD / 16];
#pragma unroll
    for (int i = 0; i < RG; ++i)
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Every stage issues its loads on every step, also past the end of the split (those
    // tiles are empty: zero-length descriptors and out-of-range B offsets fetch nothing).
    // With no conditional loads the compiler can count exactly how many younger loads are in
    // flight and waits only for the stage it consumes.
    for (int kt = kt0; kt < kt1; kt += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int k = kt + q;
            {
                unsigned char* Bs = Bs0 + (k & 1) * NPAD * kRowBytes;
                const int kn = k + P;
                const uint32_t o_pf2 = off_at(kn + 2);  // issued early: the barrier waits for it
                bst[q].store(Bs, a.N, tid);
                const int n = nv[q];
                if (n > 0) {
                    zero_rows<TM>(As, lane);
                    scatter_place<R>(wb[q], n, As, lane);
                    if (n > R * 64) scatter_rest<R>(n, As, a.words + first[q], lane);
                }
                // refill this register stage with tile k + P
                uint32_t o0 = 0, o1 = 0;
                if (active && kn < kt1) {
                    o0 = o_next;
                    o1 = o_pf;
                }
                o_next = o_pf;
                o_pf = o_pf2;
                first[q] = o0;
                nv[q] = (int)((o1 - o0) >> 2);
                bst[q].load(bsrc, a.B, a.N, a.K, kn, tid, kn < kt1);
                load_tile<R>(wb[q], a.words, o0, nv[q], lane);
                __syncthreads();
                if (n > 0) mma_rows<NPAD, RG>(acc, As, Bs, lane);
            }
        }
    }
    // MFMA 16x16 result layout: lane holds column (lane & 15), rows 4*(lane >> 4) + 0..3.
    const int ncol = lane & 15;
    const int mrow = rb * TM + (lane >> 4) * 4;
    const bool vec_m = (a.M & 3) == 0;
    if (active) {
#pragma unroll
        for (int i = 0; i < RG; ++i) {
#pragma unroll
            for (int j = 0; j < NPAD / 16; ++j) {
                const int n = j * 16 + ncol;
                const int m = mrow + i * 16;
                if (n >= a.N || m >= a.M) continue;
                const f32x4 v = acc[i][j];
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

// Independent-wavefront variant for N <= 32.  A workgroup owns one 64-row block; its
// wavefronts split the block's k range among themselves and run with no barrier at all:
// each stages its own B tile (coalesced loads at the same pipeline depth as its packed
// words, then a private LDS area) next to its own LDS A tile, and the LDS executes one
// wavefront's writes and reads in program order.  At the end the wavefronts' fp32
// sums are added through LDS in a fixed wavefront order, so no cross-workgroup partial
// sums are needed unless the K range is also split across workgroups.
template <int NPAD, int R, int P, bool VEC, int WK, int RG>
__global__ __launch_bounds__(WK * 64) void spmm_indep_kernel(SpmmArgs a) {
    constexpr int TM = 16 * RG;             // rows of the format's tiles
    constexpr int kTB = TM * kRowBytes;     // the wavefront's LDS tile
    constexpr int kUnscatterMaxWords = TM * kTileK / 4;
    static_assert(NPAD * TM * 4 <= kTB, "the reduction reuses each wavefront's tile");
    constexpr int kBBytes = NPAD * kRowBytes;  // the wavefront's B tile
    __shared__ __attribute__((aligned(16))) unsigned char smem[WK * (kTB + kBBytes)];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* As = smem + wave * kTB;
    unsigned char* Bw = smem + WK * kTB + wave * kBBytes;

    const int bid = blockIdx.x;
    const int item = (bid & 7) * a.per_xcd + (bid >> 3);
    if (item >= a.items) return;
    const int s = item / a.G;       // G = row blocks here
    const int rb = item - s * a.G;
    const int ks0 = (int)(((int64_t)s * a.KT) / a.S);
    const int ks1 = (int)(((int64_t)(s + 1) * a.KT) / a.S);
    const int kt0 = ks0 + (wave * (ks1 - ks0)) / WK;
    const int kt1 = ks0 + ((wave + 1) * (ks1 - ks0)) / WK;
    const kconst_u32* toff = (const kconst_u32*)(a.offs) + (int64_t)rb * a.KT;
    const __amdgpu_buffer_rsrc_t bsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.B, (short)0, a.N * a.K * 2, kBufWord3);
    auto off_at = [&](int i) -> uint32_t { return i <= kt1 ? toff[i] : 0u; };

    zero_rows<TM>(As, lane);  // kept all-zero between tiles by unscatter()
    u32x4 wb[P][R];
    BWave<NPAD, VEC> bf[P];
    int nv[P];
    uint32_t first[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int k = kt0 + q;
        uint32_t o0 = 0, o1 = 0;
        if (k < kt1) {
            o0 = toff[k];
            o1 = toff[k + 1];
        }
        first[q] = o0;
        nv[q] = (int)((o1 - o0) >> 2);
        bf[q].load(bsrc, a.B, a.N, a.K, k, lane, k < kt1);
        load_tile<R>(wb[q], a.words, o0, nv[q], lane);
    }
    uint32_t o_next = off_at(kt0 + P);
    uint32_t o_pf = off_at(kt0 + P + 1);

    f32x4 acc[RG][NPAD / 16];
#pragma unroll
    for (int i = 0; i < RG; ++i)
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kt = kt0; kt < kt1; kt += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int k = kt + q;
            const int kn = k + P;
            const uint32_t o_pf2 = off_at(kn + 2);
            const int n = nv[q];
            if (n > 0) {
                scatter_keep<R>(wb[q], n, As, lane);
                if (n > R * 64) scatter_rest<R>(n, As, a.words + first[q], lane);
                bf[q].store(Bw, lane);
                mma_rows<NPAD, RG>(acc, As, Bw, lane);
                // Reset: rewriting the scattered positions costs one 2-byte store per word,
                // clearing the tile TM / 8 16-byte stores per lane; the former wins only for
                // sparse tiles (at most a quarter of the tile's positions).
                if (n > R * 64 || 4 * n > kUnscatterMaxWords)
                    zero_rows<TM>(As, lane);
                else
                    unscatter<R>(wb[q], n, lane);
            }
            uint32_t o0 = 0, o1 = 0;
            if (kn < kt1) {
                o0 = o_next;
                o1 = o_pf;
            }
            o_next = o_pf;
            o_pf = o_pf2;
            first[q] = o0;
            nv[q] = (int)((o1 - o0) >> 2);
            bf[q].load(bsrc, a.B, a.N, a.K, kn, lane, kn < kt1);
            load_tile<R>(wb[q], a.words, o0, nv[q], lane);
        }
    }

    // Sum the wavefronts' results: each dumps its fp32 block as [NPAD][64] into its own tile,
    // then every (n, 4 rows) item is added over wavefronts 0, 1, ..., WK-1 in that order.
    float* red = reinterpret_cast<float*>(As);
    const int ncol = lane & 15;
    const int mq = (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < RG; ++i)
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j)
            *reinterpret_cast<f32x4*>(red + (j * 16 + ncol) * TM + i * 16 + mq) = acc[i][j];
    __syncthreads();
    const bool vec_m = (a.M & 3) == 0;
    for (int it = tid; it < a.N * (TM / 4); it += WK * 64) {
        const int n = it / (TM / 4);
        const int ml = (it - n * (TM / 4)) * 4;
        f32x4 sum = *reinterpret_cast<const f32x4*>(smem + (n * TM + ml) * 4);
#pragma unroll
        for (int w = 1; w < WK; ++w)
            sum += *reinterpret_cast<const f32x4*>(smem + w * kTB + (n * TM + ml) * 4);
        const int m = rb * TM + ml;
        if (m >= a.M) continue;
        if (a.S == 1) {
            uint16_t* dst = a.C + (int64_t)n * a.M + m;
            if (vec_m) {
                uint2 pk;
                pk.x = (uint32_t)f16_bits(sum[0]) | ((uint32_t)f16_bits(sum[1]) << 16);
                pk.y = (uint32_t)f16_bits(sum[2]) | ((uint32_t)f16_bits(sum[3]) << 16);
                *reinterpret_cast<uint2*>(dst) = pk;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (m + e < a.M) dst[e] = f16_bits(sum[e]);
            }
        } else {
            float* dst = a.part + ((int64_t)s * a.N + n) * a.M + m;
            if (vec_m) {
                *reinterpret_cast<f32x4*>(dst) = sum;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (m + e < a.M) dst[e] = sum[e];
            }
        }
    }
}

// Wide-N variant (64 < N <= 256 per launch).  Above N = 64 one A tile feeds enough MFMA
// work to keep a whole workgroup busy, so the four wavefronts decode each tile together
// (each loads, and scatters, a quarter of its words) and wavefront w multiplies it with
// columns 64w .. 64w + 63 of B.  Three LDS A buffers rotate so that one barrier per k step
// orders everything: at step k the workgroup zero-fills buffer (k+1) % 3, whose last
// readers were the MFMAs of step k-2 (all past the barrier of step k-1), and scatters
// into buffer k % 3, whose zero-fill was done before the barrier of step k-1.
template <int NW, int R, bool VEC, int RG>
__global__ __launch_bounds__(kThreads) void spmm_wide_kernel(SpmmArgs a) {
    constexpr int TM = 16 * RG;          // rows of the format's tiles
    constexpr int kTB = TM * kRowBytes;  // one A buffer
    static_assert(kThreads == 256, "four wavefronts of 64 columns each");
    constexpr int NPAD = NW * 64;
    constexpr int P = 2;
    constexpr int kBBytes = NPAD * kRowBytes;
    __shared__ __attribute__((aligned(16))) unsigned char smem[3 * kTB + 2 * kBBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* Bs0 = smem + 3 * kTB;

    const int bid = blockIdx.x;
    const int item = (bid & 7) * a.per_xcd + (bid >> 3);
    if (item >= a.items) return;
    const int s = item / a.G;  // G = row blocks
    const int rb = item - s * a.G;
    const int kt0 = (int)(((int64_t)s * a.KT) / a.S);
    const int kt1 = (int)(((int64_t)(s + 1) * a.KT) / a.S);
    const kconst_u32* toff = (const kconst_u32*)(a.offs) + (int64_t)rb * a.KT;
    const __amdgpu_buffer_rsrc_t bsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.B, (short)0, a.N * a.K * 2, kBufWord3);
    auto off_at = [&](int i) -> uint32_t { return i <= kt1 ? toff[i] : 0u; };

    // B rows n >= N stay zero in both buffers; A buffer 0 starts zeroed.
    for (int ch = tid; ch < 2 * NPAD * 8; ch += kThreads) {
        const int row = ch >> 3;
        if (row % NPAD >= a.N) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(Bs0 + row * kRowBytes + (ch & 7) * 16) = z;
        }
    }
    zero_buf_wg<kTB>(smem, tid);

    u32x4 wb[P][R];
    BStage<NPAD, VEC> bst[P];
    int nv[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int k = kt0 + q;
        uint32_t o0 = 0, o1 = 0;
        if (k < kt1) {
            o0 = toff[k];
            o1 = toff[k + 1];
        }
        nv[q] = (int)((o1 - o0) >> 2);
        bst[q].load(bsrc, a.B, a.N, a.K, k, tid, k < kt1);
        load_tile_wg<R>(wb[q], a.words, o0, nv[q], tid);
    }
    uint32_t o_next = off_at(kt0 + P);
    uint32_t o_pf = off_at(kt0 + P + 1);
    __syncthreads();

    f32x4 acc[RG][4];
#pragma unroll
    for (int i = 0; i < RG; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    int ab = 0;  // A buffer of the current k step
    for (int kt = kt0; kt < kt1; kt += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int k = kt + q;
            const int kn = k + P;
            const int an = ab == 2 ? 0 : ab + 1;
            unsigned char* As = smem + ab * kTB;
            unsigned char* Bs = Bs0 + (k & 1) * kBBytes;
            const uint32_t o_pf2 = off_at(kn + 2);
            zero_buf_wg<kTB>(smem + an * kTB, tid);
            bst[q].store(Bs, a.N, tid);
            const int n = nv[q];
            scatter_tile_wg<R>(wb[q], n, As, tid);
            uint32_t o0 = 0, o1 = 0;
            if (kn < kt1) {
                o0 = o_next;
                o1 = o_pf;
            }
            o_next = o_pf;
            o_pf = o_pf2;
            nv[q] = (int)((o1 - o0) >> 2);
            bst[q].load(bsrc, a.B, a.N, a.K, kn, tid, kn < kt1);
            load_tile_wg<R>(wb[q], a.words, o0, nv[q], tid);
            __syncthreads();
            if (n > 0 && wave < NW) mma_rows<64, RG>(acc, As, Bs + wave * 64 * kRowBytes, lane);
            ab = an;
        }
    }
    if (wave >= NW) return;
    const int ncol = lane & 15;
    const int mrow = rb * TM + (lane >> 4) * 4;
    const bool vec_m = (a.M & 3) == 0;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = wave * 64 + j * 16 + ncol;
            const int m = mrow + i * 16;
            if (n >= a.N || m >= a.M) continue;
            const f32x4 v = acc[i][j];
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

// ---------------------------------------------------------------- bitmap tiles
// Variant format with one bit per position (the pages' follow-up summary, section
// "Problematica").  Positions are numbered in the operand order of the 16x16x32 MFMA: lane
// l's mask bit b (chunk g = b/8, element b%8) is tile row 16*(g/2) + l%16, column
// 32*(g%2) + 8*(l/16) + b%8, so lane l's 64 bits are exactly the 8 A-operand vectors it feeds
// to the matrix unit (chunk g = row group g/2, k step g%2).  A non-empty tile holds the 64
// lane masks (512 bytes), then its values chunk by chunk (chunk g of lanes 0..63 in lane
// order), padded to 16-byte vectors; offsets count 16-byte units.
//
// Decoding needs no LDS tile: a lane finds where each of its 8 chunk runs starts in the value
// stream (a prefix over the wavefront of its chunk counts, plus the chunk totals before it),
// fetches each run with one dword-aligned 16-byte load, shifts each 4-bit group's values into
// place (v_alignbit_b32) and spreads them to the group's positions with two byte permutes
// (v_perm_b32) whose selectors come from a 256-entry table indexed by the chunk's mask byte.
// In chunk-major order the lanes of one load read neighbouring runs, a few cache lines per
// instruction.  Measured: the product is bound by the number of vector memory instructions
// per tile more than by their bytes (one 8-byte load per group at 2-byte alignment cost about
// 1000 CU cycles per tile at any density, one dword-aligned 12-byte load per group about 650;
// one 16-byte load per chunk instead took 17-25 % off that), then by VALU issue.
constexpr int kMaskUnits = kTileM * 8 / 16;     // 16-byte units of a tile's masks (32)
constexpr int kMaskBytes = kMaskUnits * 16;     // 512
constexpr int kBitmapTableBytes = 256 * 16;    // selector table: 256 chunk masks x 4 dwords
constexpr int kBitmapSlack = kBitmapSlackBytes;  // readable bytes past a tile's values

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Entry b (a chunk's 8 mask bits): v_perm_b32 selectors of the chunk's output dwords 0..3
// (elements 0-1, 2-3 of the low 4-bit group, then of the high group).  A group's values sit
// packed at the front of its 8 aligned bytes (value r in bytes 2r, 2r+1); element e of group q
// takes value popc(q & ((1 << e) - 1)) when bit e is set, the constant zero byte (selector 12)
// otherwise.  Built by the workgroup's first 256 threads, one entry each.
__device__ __forceinline__ void bitmap_table(unsigned char* tbl, int tid) {
    if (tid < 256) {
        uint32_t sel[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t q = ((uint32_t)tid >> (4 * h)) & 0xFu;
            uint32_t r = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t v = 0x0C0Cu;
                if ((q >> e) & 1u) {
                    v = (2u * r) | ((2u * r + 1u) << 8);
                    ++r;
                }
                sel[2 * h + (e >> 1)] |= v << (16 * (e & 1));
            }
        }
        *reinterpret_cast<u32x4*>(tbl + tid * 16) = u32x4{sel[0], sel[1], sel[2], sel[3]};
    }
}

// Inclusive prefix sum over the wavefront (row shifts within rows of 16 lanes, then the row
// broadcasts of lanes 15 and 31).
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Value index (from the tile's first value) where each of the lane's 8 chunk runs starts,
// times 16 (the form v_alignbit_b32 takes as a shift: bits 4:0 are 16 for an odd start).
// Chunk counts are packed 10 bits a field, three fields a word, so three wavefront scans give
// every chunk's lane prefix; the chunk totals (lane 63's inclusive sums) are wave-uniform.
__device__ __forceinline__ void bitmap_chunk_starts(uint32_t lo, uint32_t hi, uint32_t (&first)[8]) {
    uint32_t c[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        c[g] = (uint32_t)__popc((lo >> (8 * g)) & 0xFFu);
        c[g + 4] = (uint32_t)__popc((hi >> (8 * g)) & 0xFFu);
    }
    const uint32_t p0 = c[0] | (c[1] << 10) | (c[2] << 20);
    const uint32_t p1 = c[3] | (c[4] << 10) | (c[5] << 20);
    const uint32_t p2 = c[6] | (c[7] << 10);
    const uint32_t i0 = wave_scan(p0), i1 = wave_scan(p1), i2 = wave_scan(p2);
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)i0, 63);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)i1, 63);
    const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)i2, 63);
    const uint32_t e[3] = {i0 - p0, i1 - p1, i2 - p2};
    const uint32_t t[3] = {t0, t1, t2};
    uint32_t base = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const int w = g / 3, f = 10 * (g % 3);
        first[g] = (base + ((e[w] >> f) & 0x3FFu)) << 4;
        base += (t[w] >> f) & 0x3FFu;
    }
}

// The 8 value loads of a tile: for each chunk, the dword-aligned 16 bytes from the start of
// the lane's run.  The descriptor covers the values plus the slack, and every load lies
// wholly inside it (it ends at most 16 bytes past the run's start, which is at most the
// value count).
__device__ __forceinline__ void bitmap_load_values(u32x4 (&x)[8], const uint32_t* words, uint32_t first_unit,
                                                   uint32_t units, const uint32_t (&first)[8]) {
    const __amdgpu_buffer_rsrc_t vs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(words + 4 * (size_t)first_unit + 4 * kMaskUnits), (short)0,
        units > (uint32_t)kMaskUnits ? (int)((units - kMaskUnits) * 16 + kBitmapSlack) : 0, kBufWord3);
#pragma unroll
    for (int g = 0; g < 8; ++g) x[g] = __builtin_amdgcn_raw_buffer_load_b128(vs, (first[g] >> 3) & ~3u, 0, 0);
}

// Lane masks of a tile (zero for an empty tile: the descriptor then covers nothing).
__device__ __forceinline__ u32x2 bitmap_load_masks(const uint32_t* words, uint32_t first_unit, uint32_t units,
                                                   int lane) {
    const __amdgpu_buffer_rsrc_t ms = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(words + 4 * (size_t)first_unit), (short)0, units > 0 ? kMaskBytes : 0, kBufWord3);
    return __builtin_amdgcn_raw_buffer_load_b64(ms, lane * 8, 0, kStreamPolicy);
}

// A operand of lane `lane` for chunk g: 4 dwords, elements 8g .. 8g+7 of its mask, from the
// chunk's 16-byte window w (8 halves from the run's start rounded down to even).  The low
// group's values start at half F & 1, the high group's at o = (F & 1) + popc(low group), so
// the high group reads dwords o/2 .. o/2 + 2 of the window.  Only a full chunk (8 values) at an
// odd start needs a ninth half; it is the first half of the next lane's window (that lane's run
// starts right after), moved over with a wavefront shift -- lane 63, which has no next lane,
// reads it with a scalar load (m63: lane 63's mask word of this chunk).  Every lane of the
// wavefront must call it (a shift from an inactive lane reads nothing useful).  first[] holds
// F << 4: v_alignbit_b32 reads bits 4:0 of its shift, 16 for an odd start.
__device__ __forceinline__ u32x4 bitmap_chunk(const u32x4 (&x)[8], const uint32_t (&first)[8], uint32_t lo,
                                              uint32_t hi, uint32_t m63, const unsigned char* tbl,
                                              const kconst_u32* vw, int lane, int g) {
    const uint32_t m = g < 4 ? lo : hi;
    const int bit = 8 * (g & 3);
    const u32x4 w = x[g];
    const uint32_t F16 = first[g];
    uint32_t w4 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w[0], 0x130, 0xf, 0xf, false);  // wave_shl:1
    if (((m63 >> bit) & 0xFFu) == 0xFFu) {  // lane 63's chunk is full
        const uint32_t f63 = (uint32_t)__builtin_amdgcn_readlane((int)F16, 63) >> 4;
        if (f63 & 1u) {
            const uint32_t sv = vw[(f63 + 7u) >> 1];
            if (lane == 63) w4 = sv;
        }
    }
    const u32x4 sel = *reinterpret_cast<const u32x4*>(tbl + (((m >> bit) & 0xFFu) << 4));
    u32x4 r;
    const uint32_t a0 = __builtin_amdgcn_alignbit(w[1], w[0], F16);
    const uint32_t a1 = __builtin_amdgcn_alignbit(w[2], w[1], F16);
    r[0] = __builtin_amdgcn_perm(a1, a0, sel[0]);
    r[1] = __builtin_amdgcn_perm(a1, a0, sel[1]);
    const uint32_t o = ((F16 >> 4) & 1u) + (uint32_t)__popc((m >> bit) & 0xFu);
    const bool j1 = o >= 2u, j2 = o >= 4u;
    const uint32_t y0 = j2 ? w[2] : (j1 ? w[1] : w[0]);
    const uint32_t y1 = j2 ? w[3] : (j1 ? w[2] : w[1]);
    const uint32_t y2 = j2 ? w4 : (j1 ? w[3] : w[2]);
    const uint32_t sh1 = o << 4;
    const uint32_t b0 = __builtin_amdgcn_alignbit(y1, y0, sh1);
    const uint32_t b1 = __builtin_amdgcn_alignbit(y2, y1, sh1);
    r[2] = __builtin_amdgcn_perm(b1, b0, sel[2]);
    r[3] = __builtin_amdgcn_perm(b1, b0, sel[3]);
    return r;
}

// Bitmap-tile product for N <= 64 per launch: a workgroup owns one row block and its WK
// wavefronts split the k range; each wavefront keeps its own B tile in LDS and needs no
// barrier until the final sum over wavefronts.  Pipeline of P stages: masks P tiles ahead,
// values P - 1 tiles ahead (their offsets need the masks).  B is one tile ahead in one set of
// registers, loaded first in each step: waiting for it never waits for the value loads.
template <int NPAD, int WK, int P, bool VEC>
__global__ __launch_bounds__(WK * 64) void spmm_bitmap_kernel(SpmmArgs a) {
    constexpr int kBBytes = NPAD * kRowBytes;
    constexpr int kRedBytes = NPAD * kTileM * 4;
    constexpr int kWaveBytes = kBBytes > kRedBytes ? kBBytes : kRedBytes;
    static_assert(WK * 64 >= 256, "the workgroup builds the 256-entry selector table");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kBitmapTableBytes + WK * kWaveBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int bid = blockIdx.x;
    const int item = (bid & 7) * a.per_xcd + (bid >> 3);
    if (item >= a.items) return;
    unsigned char* tbl = smem;
    unsigned char* area = smem + kBitmapTableBytes;
    unsigned char* Bw = area + wave * kWaveBytes;
    bitmap_table(tbl, tid);
    __syncthreads();

    const int s = item / a.G;
    const int rb = item - s * a.G;
    const int ks0 = (int)(((int64_t)s * a.KT) / a.S);
    const int ks1 = (int)(((int64_t)(s + 1) * a.KT) / a.S);
    const int kt0 = ks0 + (wave * (ks1 - ks0)) / WK;
    const int kt1 = ks0 + ((wave + 1) * (ks1 - ks0)) / WK;
    const kconst_u32* toff = (const kconst_u32*)(a.offs) + (int64_t)rb * a.KT;
    const __amdgpu_buffer_rsrc_t bsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.B, (short)0, a.N * a.K * 2, kBufWord3);

    u32x2 mk[P];          // lane masks of the tile in each stage
    uint32_t fu[P];       // its first 16-byte unit
    uint32_t nu[P];       // its 16-byte units (0: empty)
    u32x4 xv[P][8];       // its value windows, one per chunk
    uint32_t vf[P][8];    // and the chunk runs' first values
    BWave<NPAD, VEC> bw;  // B tile of the current step's tile
    auto fetch_masks = [&](int q, int k) {
        uint32_t o0 = 0, o1 = 0;
        if (k < kt1) {
            o0 = toff[k];
            o1 = toff[k + 1];
        }
        fu[q] = o0;
        nu[q] = o1 - o0;
        mk[q] = bitmap_load_masks(a.words, o0, o1 - o0, lane);
    };
    auto fetch_values = [&](int q) {
        bitmap_chunk_starts(mk[q][0], mk[q][1], vf[q]);
        bitmap_load_values(xv[q], a.words, fu[q], nu[q], vf[q]);
    };
    bw.load(bsrc, a.B, a.N, a.K, kt0, lane, kt0 < kt1);
#pragma unroll
    for (int q = 0; q < P; ++q) fetch_masks(q, kt0 + q);
    // issue order as in the loop (the masks of later tiles before the values of earlier
    // ones), so that waiting for masks leaves the values in flight
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q + 1 < P; ++q) fetch_values(q);

    f32x4 acc[4][NPAD / 16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint32_t rl = lane & 15, kq = lane >> 4;
    for (int kt = kt0; kt < kt1; kt += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int k = kt + q;
            const u32x2 m = mk[q];
            const uint32_t units = nu[q];
            const kconst_u32* vw = (const kconst_u32*)(a.words) + 4 * (size_t)fu[q] + 4 * kMaskUnits;
            if (units > 0) bw.store(Bw, lane);
            bw.load(bsrc, a.B, a.N, a.K, k + 1, lane, k + 1 < kt1);
            fetch_masks(q, k + P);
            fetch_values((q + P - 1) % P);  // tile k + P - 1
            if (units > 0) {
                const uint32_t m63lo = (uint32_t)__builtin_amdgcn_readlane((int)m[0], 63);
                const uint32_t m63hi = (uint32_t)__builtin_amdgcn_readlane((int)m[1], 63);
                // chunk g = 2i + ks, expanded right before its MFMAs (k step outer, so that
                // consecutive MFMAs write different accumulators)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    half8 bfr[NPAD / 16];
#pragma unroll
                    for (int j = 0; j < NPAD / 16; ++j)
                        bfr[j] = *reinterpret_cast<const half8*>(Bw + lds_chunk(j * 16 + rl, ks * 4 + kq));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const half8 af =
                            __builtin_bit_cast(half8, bitmap_chunk(xv[q], vf[q], m[0], m[1], (2 * i + ks) < 4 ? m63lo : m63hi, tbl, vw, lane, 2 * i + ks));
#pragma unroll
                        for (int j = 0; j < NPAD / 16; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bfr[j], acc[i][j], 0, 0, 0);
                    }
                }
            }
        }
    }

    // the wavefronts' sums, added in wavefront order
    float* red = reinterpret_cast<float*>(Bw);
    const int ncol = lane & 15;
    const int mq = (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j)
            *reinterpret_cast<f32x4*>(red + (j * 16 + ncol) * kTileM + i * 16 + mq) = acc[i][j];
    __syncthreads();
    const bool vec_m = (a.M & 3) == 0;
    for (int it = tid; it < a.N * (kTileM / 4); it += WK * 64) {
        const int nn = it / (kTileM / 4);
        const int ml = (it - nn * (kTileM / 4)) * 4;
        f32x4 sum = *reinterpret_cast<const f32x4*>(area + (nn * kTileM + ml) * 4);
#pragma unroll
        for (int w = 1; w < WK; ++w)
            sum += *reinterpret_cast<const f32x4*>(area + w * kWaveBytes + (nn * kTileM + ml) * 4);
        const int mm = rb * kTileM + ml;
        if (mm >= a.M) continue;
        if (a.S == 1) {
            uint16_t* dst = a.C + (int64_t)nn * a.M + mm;
            if (vec_m) {
                uint2 pk;
                pk.x = (uint32_t)f16_bits(sum[0]) | ((uint32_t)f16_bits(sum[1]) << 16);
                pk.y = (uint32_t)f16_bits(sum[2]) | ((uint32_t)f16_bits(sum[3]) << 16);
                *reinterpret_cast<uint2*>(dst) = pk;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (mm + e < a.M) dst[e] = f16_bits(sum[e]);
            }
        } else {
            float* dst = a.part + ((int64_t)s * a.N + nn) * a.M + mm;
            if (vec_m) {
                *reinterpret_cast<f32x4*>(dst) = sum;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (mm + e < a.M) dst[e] = sum[e];
            }
        }
    }
}

// ---------------------------------------------------------------- three-level tiles
// Format (follow-up summary of the pages, section "Metodologia", three-level storage):
// a 64 x 64 tile holds 1024 words of 4:2 slots, stored in the operand registers' order of
// v_smfmac_f32_16x16x64_f16 (operand i, lane l: row 16i + l%16, columns 16*(l/16) .. +15,
// two slots per group of four columns), 256 words of per-lane metadata (2-bit positions of
// operands 0|1 and 2|3, fill mask, 4-bit distance codes) and the residual words.  Load as
// sparse, compute as sparse: the slots go from HBM into the structured-sparse MFMA without
// passing through LDS.  The entries that do not fit the 4:2 pattern -- slot-filled ones
// (their value sits in a slot the 4:2 layer leaves unused, their position is the running sum
// of the codes) and residual ones -- are placed into a dense LDS tile, as in Tiled-CSL, and
// enter through a dense MFMA on the same B operand registers.
constexpr int kTLFixedUnits = kThreeLevelFixedWords / 4;  // 16-byte units before the residual words
constexpr int kTLValueBytes = kThreeLevelValueWords * 4;
constexpr int kTLSlotStride = 80;  // bytes per lane of the slot copy: 16-byte stores of 8 lanes hit distinct banks

// Slot-filling layer of one tile: copy the lane's 32 slots to Ps, move each filled slot's
// value to its decoded position in the dense tile As and clear the slot, then reload the
// slots.  p runs over the lane's region (4 rows x 16 columns): p = 16*i + column % 16.
// Slots and positions are worked out first, so that the LDS reads of all eight points are in
// flight together.
__device__ __forceinline__ uint32_t three_level_fill(u32x4 (&va)[4], uint32_t fill, uint32_t codes, unsigned char* As,
                                                     unsigned char* Ps, uint32_t (&dst)[kThreeLevelMaxCodes], int lane) {
    u32x4* pv = reinterpret_cast<u32x4*>(Ps + lane * kTLSlotStride);
    uint16_t* ph = reinterpret_cast<uint16_t*>(Ps + lane * kTLSlotStride);
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = va[i];
    uint32_t slot[kThreeLevelMaxCodes];
    uint32_t p = 0xFFFFFFFFu;
    const uint32_t n = (uint32_t)__popc(fill);
#pragma unroll
    for (int k = 0; k < kThreeLevelMaxCodes; ++k) {
        slot[k] = (uint32_t)__builtin_ctz(fill | 0x80000000u);  // filled slot 8*i + s = halfword of the copy
        fill &= fill - 1u;
        p += ((codes >> (4 * k)) & 15u) + 1u;
        const uint32_t r = 16u * ((p >> 4) & 3u) + ((uint32_t)lane & 15u);
        const uint32_t c = 16u * ((uint32_t)lane >> 4) + (p & 15u);
        dst[k] = r * kRowBytes + ((c * 2u) ^ ((r & 7u) << 4));
    }
    uint16_t x[kThreeLevelMaxCodes];
#pragma unroll
    for (int k = 0; k < kThreeLevelMaxCodes; ++k) x[k] = (uint32_t)k < n ? ph[slot[k]] : (uint16_t)0;
#pragma unroll
    for (int k = 0; k < kThreeLevelMaxCodes; ++k) {
        if ((uint32_t)k < n) {
            ph[slot[k]] = 0;
            *reinterpret_cast<uint16_t*>(As + dst[k]) = x[k];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) va[i] = pv[i];
    return n;
}

// Reset of the dense tile after a step: zeros at the slot-filled points (n of them, offsets
// dst) and at the residual words held in registers (the lane's unit of the first 64); a tile
// with more residual units was cleared whole instead.
__device__ __forceinline__ void three_level_reset(unsigned char* As, const uint32_t (&dst)[kThreeLevelMaxCodes],
                                                  uint32_t n, const u32x4& vr, bool has_res) {
#pragma unroll
    for (int k = 0; k < kThreeLevelMaxCodes; ++k)
        if ((uint32_t)k < n) *reinterpret_cast<uint16_t*>(As + dst[k]) = 0;
    if (has_res) {
#pragma unroll
        for (int e = 0; e < 4; ++e) put_word(As, vr[e] & 0xFFFF0000u);
    }
}

// acc[i][j] += 4:2 slots of operand i (x B columns 16j..16j+15) and, when `dense`, the dense
// tile As; both read the same B registers (k = 8q..8q+7 and 32+8q..32+8q+7 for q = lane/16).
template <int NPAD>
__device__ __forceinline__ void three_level_mma(f32x4 (&acc)[4][NPAD / 16], const u32x4 (&va)[4], uint32_t idx01,
                                                uint32_t idx23, const unsigned char* As, const unsigned char* Bw,
                                                bool dense, int lane) {
    const uint32_t rl = lane & 15, kq = lane >> 4;
    const half8 a0 = __builtin_bit_cast(half8, va[0]), a1 = __builtin_bit_cast(half8, va[1]);
    const half8 a2 = __builtin_bit_cast(half8, va[2]), a3 = __builtin_bit_cast(half8, va[3]);
    half8 f[4][2];
    if (dense) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i][0] = *reinterpret_cast<const half8*>(As + lds_chunk(i * 16 + rl, kq));
            f[i][1] = *reinterpret_cast<const half8*>(As + lds_chunk(i * 16 + rl, 4 + kq));
        }
    }
#pragma unroll
    for (int j = 0; j < NPAD / 16; ++j) {
        const half8 b0 = *reinterpret_cast<const half8*>(Bw + lds_chunk(j * 16 + rl, kq));
        const half8 b1 = *reinterpret_cast<const half8*>(Bw + lds_chunk(j * 16 + rl, 4 + kq));
        const half16 bb = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        acc[0][j] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a0, bb, acc[0][j], (int)idx01, 0, 0);
        acc[1][j] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a1, bb, acc[1][j], (int)idx01, 0, 1);
        acc[2][j] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a2, bb, acc[2][j], (int)idx23, 0, 0);
        acc[3][j] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a3, bb, acc[3][j], (int)idx23, 0, 1);
        if (dense) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[i][0], b0, acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[i][1], b1, acc[i][j], 0, 0, 0);
            }
        }
    }
}

// Three-level product, organised like the bitmap kernel: a workgroup owns one row block and
// its WK wavefronts split the k range; each wavefront has its own dense tile, slot copy and B
// tile, and needs no barrier until the final sum over wavefronts.
template <int NPAD, int WK, bool VEC>
__global__ __launch_bounds__(WK * 64) void spmm_three_level_kernel(SpmmArgs a) {
    constexpr int P = 2;
    constexpr int kBBytes = NPAD * kRowBytes;
    constexpr int kWaveBytes = kTileBytes + 64 * kTLSlotStride + kBBytes;
    static_assert(NPAD * kTileM * 4 <= kWaveBytes, "the reduction reuses each wavefront's area");
    __shared__ __attribute__((aligned(16))) unsigned char smem[WK * kWaveBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* As = smem + wave * kWaveBytes;
    unsigned char* Ps = As + kTileBytes;
    unsigned char* Bw = Ps + 64 * kTLSlotStride;

    const int bid = blockIdx.x;
    const int item = (bid & 7) * a.per_xcd + (bid >> 3);
    if (item >= a.items) return;
    const int s = item / a.G;
    const int rb = item - s * a.G;
    const int ks0 = (int)(((int64_t)s * a.KT) / a.S);
    const int ks1 = (int)(((int64_t)(s + 1) * a.KT) / a.S);
    const int kt0 = ks0 + (wave * (ks1 - ks0)) / WK;
    const int kt1 = ks0 + ((wave + 1) * (ks1 - ks0)) / WK;
    const kconst_u32* toff = (const kconst_u32*)(a.offs) + (int64_t)rb * a.KT;
    const __amdgpu_buffer_rsrc_t bsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.B, (short)0, a.N * a.K * 2, kBufWord3);

    u32x4 va[P][4];  // 4:2 slots of operands 0..3
    u32x4 vm[P];     // metadata: positions 0|1, positions 2|3, fill mask, codes
    u32x4 vr[P];     // residual words of unit `lane`
    int nres[P];     // residual units of the tile, -1 for an empty tile
    uint32_t first[P];
    BWave<NPAD, VEC> bf[P];
    auto fetch = [&](int q, int k) {
        uint32_t o0 = 0, o1 = 0;
        if (k < kt1) {
            o0 = toff[k];
            o1 = toff[k + 1];
        }
        const int units = (int)(o1 - o0);
        first[q] = o0;
        nres[q] = units > 0 ? units - kTLFixedUnits : -1;
        // the descriptor covers exactly the tile: an empty tile or a lane past the residual
        // words reads zeros without a fetch
        __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.words + 4 * (size_t)o0), (short)0, units * 16, kBufWord3);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            va[q][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (i * 64 + lane) * 16, 0, kStreamPolicy);
        vm[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, kTLValueBytes + lane * 16, 0, kStreamPolicy);
        vr[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, (kTLFixedUnits + lane) * 16, 0, kStreamPolicy);
        bf[q].load(bsrc, a.B, a.N, a.K, k, lane, k < kt1);
    };
#pragma unroll
    for (int q = 0; q < P; ++q) fetch(q, kt0 + q);

    zero_tile(As, lane);
    f32x4 acc[4][NPAD / 16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kt = kt0; kt < kt1; kt += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int k = kt + q;
            const int nr = nres[q];
            if (nr >= 0) {
                bf[q].store(Bw, lane);
                const uint32_t fill = vm[q][2];
                const bool any_fill = __any(fill != 0u);
                const bool dense = any_fill || nr > 0;
                uint32_t dst[kThreeLevelMaxCodes];
                if (any_fill) (void)three_level_fill(va[q], fill, vm[q][3], As, Ps, dst, lane);
                if (nr > 0) {
                    if (lane < nr) {
                        put_word(As, vr[q][0]);
                        put_word(As, vr[q][1]);
                        put_word(As, vr[q][2]);
                        put_word(As, vr[q][3]);
                    }
                    const uint32_t* rw = a.words + 4 * ((size_t)first[q] + kTLFixedUnits);
                    for (int u = 64 + lane; u < nr; u += 64) {
                        const u32x4 x = *reinterpret_cast<const u32x4*>(rw + 4 * (size_t)u);
                        put_word(As, x[0]);
                        put_word(As, x[1]);
                        put_word(As, x[2]);
                        put_word(As, x[3]);
                    }
                }
                three_level_mma<NPAD>(acc, va[q], vm[q][0], vm[q][1], As, Bw, dense, lane);
                // cleared whole: measured faster here than rewriting the placed positions
                // (which the shared-B kernel for N = 64 does)
                if (dense) zero_tile(As, lane);
            }
            fetch(q, k + P);
        }
    }

    // the wavefronts' sums, added in wavefront order
    float* red = reinterpret_cast<float*>(smem + wave * kWaveBytes);
    const int ncol = lane & 15;
    const int mq = (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j)
            *reinterpret_cast<f32x4*>(red + (j * 16 + ncol) * kTileM + i * 16 + mq) = acc[i][j];
    __syncthreads();
    const bool vec_m = (a.M & 3) == 0;
    for (int it = tid; it < a.N * (kTileM / 4); it += WK * 64) {
        const int nn = it / (kTileM / 4);
        const int ml = (it - nn * (kTileM / 4)) * 4;
        f32x4 sum = *reinterpret_cast<const f32x4*>(smem + (nn * kTileM + ml) * 4);
#pragma unroll
        for (int w = 1; w < WK; ++w)
            sum += *reinterpret_cast<const f32x4*>(smem + w * kWaveBytes + (nn * kTileM + ml) * 4);
        const int m = rb * kTileM + ml;
        if (m >= a.M) continue;
        if (a.S == 1) {
            uint16_t* dst = a.C + (int64_t)nn * a.M + m;
            if (vec_m) {
                uint2 pk;
                pk.x = (uint32_t)f16_bits(sum[0]) | ((uint32_t)f16_bits(sum[1]) << 16);
                pk.y = (uint32_t)f16_bits(sum[2]) | ((uint32_t)f16_bits(sum[3]) << 16);
                *reinterpret_cast<uint2*>(dst) = pk;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (m + e < a.M) dst[e] = f16_bits(sum[e]);
            }
        } else {
            float* dst = a.part + ((int64_t)s * a.N + nn) * a.M + m;
            if (vec_m) {
                *reinterpret_cast<f32x4*>(dst) = sum;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (m + e < a.M) dst[e] = sum[e];
            }
        }
    }
}

// N padded to 64: four wavefronts own four consecutive row blocks and share one B tile per k
// step, staged by the whole workgroup into a double buffer (one barrier per step).  With a
// private B tile per wavefront, the 8 KB of B per step would outweigh the ~5.5 KB of the A
// tile it multiplies (B is re-read from L2 by every row block).
template <int NPAD, bool VEC>
__global__ __launch_bounds__(kThreads) void spmm_three_level_shared_kernel(SpmmArgs a) {
    constexpr int P = 2;
    constexpr int kWaveBytes = kTileBytes + 64 * kTLSlotStride;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * kWaveBytes + 2 * NPAD * kRowBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* As = smem + wave * kWaveBytes;
    unsigned char* Ps = As + kTileBytes;
    unsigned char* Bs0 = smem + kWaves * kWaveBytes;

    const int bid = blockIdx.x;
    const int item = (bid & 7) * a.per_xcd + (bid >> 3);
    if (item >= a.items) return;  // whole workgroup
    const int s = item / a.G;
    const int g = item - s * a.G;
    const int kt0 = (int)(((int64_t)s * a.KT) / a.S);
    const int kt1 = (int)(((int64_t)(s + 1) * a.KT) / a.S);
    const int rb = g * kWaves + wave;
    const bool active = rb < a.MB;
    const kconst_u32* toff = (const kconst_u32*)(a.offs) + (int64_t)(active ? rb : 0) * a.KT;
    const __amdgpu_buffer_rsrc_t bsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.B, (short)0, a.N * a.K * 2, kBufWord3);

    // B rows n >= N stay zero for the whole kernel (both buffers).
    for (int ch = tid; ch < 2 * NPAD * 8; ch += kThreads) {
        const int row = ch >> 3;
        if (row % NPAD >= a.N) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(Bs0 + row * kRowBytes + (ch & 7) * 16) = z;
        }
    }

    u32x4 va[P][4];
    u32x4 vm[P];
    u32x4 vr[P];
    int nres[P];
    uint32_t first[P];
    BStage<NPAD, VEC> bst[P];
    auto fetch = [&](int q, int k) {
        uint32_t o0 = 0, o1 = 0;
        if (active && k < kt1) {
            o0 = toff[k];
            o1 = toff[k + 1];
        }
        const int units = (int)(o1 - o0);
        first[q] = o0;
        nres[q] = units > 0 ? units - kTLFixedUnits : -1;
        __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.words + 4 * (size_t)o0), (short)0, units * 16, kBufWord3);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            va[q][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (i * 64 + lane) * 16, 0, kStreamPolicy);
        vm[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, kTLValueBytes + lane * 16, 0, kStreamPolicy);
        vr[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, (kTLFixedUnits + lane) * 16, 0, kStreamPolicy);
        bst[q].load(bsrc, a.B, a.N, a.K, k, tid, k < kt1);
    };
#pragma unroll
    for (int q = 0; q < P; ++q) fetch(q, kt0 + q);

    zero_tile(As, lane);
    f32x4 acc[4][NPAD / 16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NPAD / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kt = kt0; kt < kt1; kt += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int k = kt + q;
            unsigned char* Bs = Bs0 + (k & 1) * NPAD * kRowBytes;
            bst[q].store(Bs, a.N, tid);
            const int nr = nres[q];
            bool dense = false;
            u32x4 cur[4] = {va[q][0], va[q][1], va[q][2], va[q][3]};
            const uint32_t idx01 = vm[q][0], idx23 = vm[q][1];
            const u32x4 res = vr[q];
            uint32_t dst[kThreeLevelMaxCodes];
            uint32_t npts = 0;
            if (nr >= 0) {
                const uint32_t fill = vm[q][2];
                const bool any_fill = __any(fill != 0u);
                dense = any_fill || nr > 0;
                if (any_fill) npts = three_level_fill(cur, fill, vm[q][3], As, Ps, dst, lane);
                if (nr > 0) {
                    if (lane < nr) {
                        put_word(As, vr[q][0]);
                        put_word(As, vr[q][1]);
                        put_word(As, vr[q][2]);
                        put_word(As, vr[q][3]);
                    }
                    const uint32_t* rw = a.words + 4 * ((size_t)first[q] + kTLFixedUnits);
                    for (int u = 64 + lane; u < nr; u += 64) {
                        const u32x4 x = *reinterpret_cast<const u32x4*>(rw + 4 * (size_t)u);
                        put_word(As, x[0]);
                        put_word(As, x[1]);
                        put_word(As, x[2]);
                        put_word(As, x[3]);
                    }
                }
            }
            fetch(q, k + P);
            __syncthreads();
            if (nr >= 0) three_level_mma<NPAD>(acc, cur, idx01, idx23, As, Bs, dense, lane);
            if (nr > 64)
                zero_tile(As, lane);
            else if (dense)
                three_level_reset(As, dst, npts, res, lane < nr);
        }
    }
    // MFMA 16x16 result layout: lane holds column (lane & 15), rows 4*(lane >> 4) + 0..3.
    const int ncol = lane & 15;
    const int mrow = rb * kTileM + (lane >> 4) * 4;
    const bool vec_m = (a.M & 3) == 0;
    if (active) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < NPAD / 16; ++j) {
                const int n = j * 16 + ncol;
                const int m = mrow + i * 16;
                if (n >= a.N || m >= a.M) continue;
                const f32x4 v = acc[i][j];
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
}

// Dense view of a three-level encoding: slot filling and residual through the product
// kernel's placement code, then the 4:2 slots that are not filled, at their positions.
__global__ __launch_bounds__(kThreads) void decode_three_level_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * (kTileBytes + 64 * kTLSlotStride)];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* As = smem + wave * (kTileBytes + 64 * kTLSlotStride);
    unsigned char* Ps = As + kTileBytes;
    const int64_t t = (int64_t)blockIdx.x * kWaves + wave;
    const bool act = t < a.T;
    uint32_t o0 = 0, o1 = 0;
    if (act) {
        o0 = a.offs[t];
        o1 = a.offs[t + 1];
    }
    zero_tile(As, lane);
    if (o1 > o0) {
        const uint32_t* tw = a.words + 4 * (size_t)o0;
        const int nr = (int)(o1 - o0) - kTLFixedUnits;
        u32x4 va[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) va[i] = *reinterpret_cast<const u32x4*>(tw + 4 * (i * 64 + lane));
        const u32x4 vm = *reinterpret_cast<const u32x4*>(tw + kThreeLevelValueWords + 4 * lane);
        uint32_t dst[kThreeLevelMaxCodes];
        (void)three_level_fill(va, vm[2], vm[3], As, Ps, dst, lane);
        for (int u = lane; u < nr; u += 64) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(tw + 4 * ((size_t)kTLFixedUnits + u));
            put_word(As, x[0]);
            put_word(As, x[1]);
            put_word(As, x[2]);
            put_word(As, x[3]);
        }
        const uint32_t r0 = (uint32_t)lane & 15u, cq = 16u * ((uint32_t)lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t idx = (i < 2 ? vm[0] : vm[1]) >> (16 * (i & 1));
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                if ((vm[2] >> (8 * i + sl)) & 1u) continue;
                const uint32_t r = 16u * i + r0;
                const uint32_t c = cq + 4u * (sl >> 1) + ((idx >> (2 * sl)) & 3u);
                const uint16_t v = (uint16_t)(va[i][sl >> 1] >> (16 * (sl & 1)));
                *reinterpret_cast<uint16_t*>(As + r * kRowBytes + ((c * 2u) ^ ((r & 7u) << 4))) = v;
            }
        }
    }
    if (!act) return;
    const int64_t bm = t / a.KT, bk = t - bm * a.KT;
    // the tile in row order: lane -> (row, 16-byte chunk); 8 chunks per row
    for (int v = lane; v < kTileM * 8; v += 64) {
        const int r = v >> 3, ch = v & 7;
        const int64_t gr = bm * kTileM + r;
        if (gr >= a.M) continue;
        const u32x4 x = *reinterpret_cast<const u32x4*>(As + lds_chunk(r, ch));
        const int64_t gc = bk * kTileK + ch * 8;
        uint16_t* dst = a.A + gr * a.K + gc;
        const uint16_t h[8] = {(uint16_t)x[0], (uint16_t)(x[0] >> 16), (uint16_t)x[1], (uint16_t)(x[1] >> 16),
                               (uint16_t)x[2], (uint16_t)(x[2] >> 16), (uint16_t)x[3], (uint16_t)(x[3] >> 16)};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (gc + e < a.K) dst[e] = h[e];
    }
}

// Dense view of a bitmap encoding through the same offset, load and expansion code: one
// wavefront per tile, lane l writes its 8 operand chunks (8 columns each) to their rows.
__global__ __launch_bounds__(kThreads) void decode_bitmap_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char tbl[kBitmapTableBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    bitmap_table(tbl, tid);
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * kWaves + wave;
    if (t >= a.T) return;
    const uint32_t o0 = a.offs[t], units = a.offs[t + 1] - o0;
    const u32x2 m = bitmap_load_masks(a.words, o0, units, lane);
    uint32_t first[8];
    bitmap_chunk_starts(m[0], m[1], first);
    u32x4 x[8];
    bitmap_load_values(x, a.words, o0, units, first);
    const kconst_u32* vw = (const kconst_u32*)(a.words) + 4 * (size_t)o0 + 4 * kMaskUnits;
    const uint32_t m63lo = (uint32_t)__builtin_amdgcn_readlane((int)m[0], 63);
    const uint32_t m63hi = (uint32_t)__builtin_amdgcn_readlane((int)m[1], 63);
    const int bm = (int)(t / a.KT), bk = (int)(t % a.KT);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        // every lane expands (the wavefront shift inside reads the next lane), then stores
        const u32x4 v = bitmap_chunk(x, first, m[0], m[1], g < 4 ? m63lo : m63hi, tbl, vw, lane, g);
        const int gi = bm * kTileM + 16 * (g >> 1) + (lane & 15);
        const int gj = bk * kTileK + 32 * (g & 1) + 8 * (lane >> 4);
        if (gi >= a.M || gj >= a.K) continue;
        uint16_t* dst = a.A + (int64_t)gi * a.K + gj;
        if ((a.K & 7) == 0 && gj + 8 <= a.K) {
            *reinterpret_cast<u32x4*>(dst) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (gj + e < a.K) dst[e] = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
        }
    }
}

// Second pass of split-K: C = fp16( ((P0 + P1) + P2) + ... ), fixed ascending order.  A
// separate launch: the kernel boundary makes every workgroup's partial sums visible to
// every XCD without cache write-backs inside the product kernel.
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, uint16_t* __restrict__ C,
                                                     int S, int64_t NM) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    if ((NM & 3) == 0) {
        const int64_t n4 = NM >> 2;
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
            f32x4 acc = reinterpret_cast<const f32x4*>(part)[i];
            for (int s = 1; s < S; ++s) acc += reinterpret_cast<const f32x4*>(part + (int64_t)s * NM)[i];
            uint2 pk;
            pk.x = (uint32_t)f16_bits(acc[0]) | ((uint32_t)f16_bits(acc[1]) << 16);
            pk.y = (uint32_t)f16_bits(acc[2]) | ((uint32_t)f16_bits(acc[3]) << 16);
            reinterpret_cast<uint2*>(C)[i] = pk;
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < NM; i += stride) {
            float acc = part[i];
            for (int s = 1; s < S; ++s) acc += part[(int64_t)s * NM + i];
            C[i] = f16_bits(acc);
        }
    }
}

// Dense view of the encoding through the product's own load and extract path: one
// wavefront per tile, then the LDS tile is copied out un-swizzled.
template <int R, int RG>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    constexpr int TM = 16 * RG;
    constexpr int kTB = TM * kRowBytes;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * kTB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* As = smem + wave * kTB;
    const int64_t t = (int64_t)blockIdx.x * kWaves + wave;
    const bool act = t < a.T;
    uint32_t o0 = 0, o1 = 0;
    if (act) {
        o0 = a.offs[t];
        o1 = a.offs[t + 1];
    }
    const int nvec = (int)((o1 - o0) >> 2);
    u32x4 wb[R];
    load_tile<R>(wb, a.words, o0, nvec, lane);
    zero_rows<TM>(As, lane);
    scatter_place<R>(wb, nvec, As, lane);
    if (nvec > R * 64) scatter_rest<R>(nvec, As, a.words + o0, lane);
    __syncthreads();
    if (!act) return;
    const int bm = (int)(t / a.KT), bk = (int)(t % a.KT);
    const bool vec_ok = (a.K & 7) == 0;
#pragma unroll
    for (int p = 0; p < 2 * RG; ++p) {
        const int ch = p * 64 + lane;
        const int r = ch >> 3, c = ch & 7;
        const int gi = bm * TM + r, gj = bk * kTileK + c * 8;
        if (gi >= a.M || gj >= a.K) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(As + lds_chunk(r, c));
        uint16_t* dst = a.A + (int64_t)gi * a.K + gj;
        if (vec_ok && gj + 8 <= a.K) {
            *reinterpret_cast<u32x4*>(dst) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (gj + e < a.K) dst[e] = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
        }
    }
}

// Register stages of the prefetch pipeline: deeper when a tile needs few registers.
template <int R>
constexpr int stages() {
#ifdef LSCD_STAGES
    return LSCD_STAGES;
#else
    return R <= 4 ? 4 : (R <= 8 ? 3 : 2);
#endif
}
template <int NPAD, int R>
constexpr int stages_indep() {
#ifdef LSCD_STAGES_INDEP
    return LSCD_STAGES_INDEP;
#else
    return (NPAD == 16 && R <= 4) ? 3 : 2;
#endif
}

template <typename Kern>
hipError_t run(Kern k, const SpmmArgs& a, int grid, hipStream_t st, int* occ, int threads = kThreads) {
    if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, k, threads, 0);
    hipLaunchKernelGGL(k, dim3(grid), dim3(threads), 0, st, a);
    return hipGetLastError();
}

// Tile heights with kernel instantiations: 64 rows for every variant; 80, 96, 112 and 128
// rows (RG = 5..8 row groups of 16) for the 8-wavefront independent variant (N <= 32), the
// shared-B variant (N <= 64), the wide variant and the decode kernel.  Taller tiles come
// with staging stages R in {4, 6, 8, 10, 12}; denser tiles take the path past the stage
// (R = 16 with eight wavefronts spills registers).
//
// K % 8 != 0 (rows of B not 16-byte aligned) runs the element-wise B path, instantiated
// only with the largest register stage.  occ != nullptr: report resident workgroups per CU
// instead of launching.
template <int NPAD, int R, int RG>
hipError_t launch_spmm_rg(int kind, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    const bool vec = (a.K & 7) == 0;
    if constexpr (NPAD <= 32) {
        if (kind == kKernelIndep) {
            if constexpr (RG != 4) return hipErrorInvalidValue;
            if (!vec) return run(spmm_indep_kernel<NPAD, 16, 2, false, 4, RG>, a, grid, st, occ, 256);
            return run(spmm_indep_kernel<NPAD, R, stages_indep<NPAD, R>(), true, 4, RG>, a, grid, st, occ, 256);
        }
        if (kind == kKernelIndep8) {
            if (!vec) return run(spmm_indep_kernel<NPAD, (RG == 4 ? 16 : 12), 2, false, 8, RG>, a, grid, st, occ, 512);
            return run(spmm_indep_kernel<NPAD, R, (RG == 4 ? stages_indep<NPAD, R>() : 2), true, 8, RG>, a, grid, st,
                       occ, 512);
        }
    }
    if (kind != kKernelShared) return hipErrorInvalidValue;
    if (!vec) return run(spmm_kernel<NPAD, (RG == 4 ? 16 : 12), 2, false, RG>, a, grid, st, occ);
    // tall tiles: two stages (the accumulators of RG row groups leave no room for a third)
    return run(spmm_kernel<NPAD, R, (RG == 4 ? stages<R>() : 2), true, RG>, a, grid, st, occ);
}

template <int NPAD, int RG>
hipError_t launch_spmm_r(int kind, int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    if constexpr (RG == 4) {
        switch (R) {
            case 2: return launch_spmm_rg<NPAD, 2, RG>(kind, a, grid, st, occ);
            case 3: return launch_spmm_rg<NPAD, 3, RG>(kind, a, grid, st, occ);
            case 5: return launch_spmm_rg<NPAD, 5, RG>(kind, a, grid, st, occ);
            case 16: return launch_spmm_rg<NPAD, 16, RG>(kind, a, grid, st, occ);
            default: break;
        }
    }
    switch (R) {
        case 4: return launch_spmm_rg<NPAD, 4, RG>(kind, a, grid, st, occ);
        case 6: return launch_spmm_rg<NPAD, 6, RG>(kind, a, grid, st, occ);
        case 8: return launch_spmm_rg<NPAD, 8, RG>(kind, a, grid, st, occ);
        case 10: return launch_spmm_rg<NPAD, 10, RG>(kind, a, grid, st, occ);
        case 12: return launch_spmm_rg<NPAD, 12, RG>(kind, a, grid, st, occ);
        default: return hipErrorInvalidValue;
    }
}

template <int NPAD>
hipError_t launch_spmm_n(int kind, int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    switch (a.TM) {
        case 64: return launch_spmm_r<NPAD, 4>(kind, R, a, grid, st, occ);
        case 80: return launch_spmm_r<NPAD, 5>(kind, R, a, grid, st, occ);
        case 96: return launch_spmm_r<NPAD, 6>(kind, R, a, grid, st, occ);
        case 112: return launch_spmm_r<NPAD, 7>(kind, R, a, grid, st, occ);
        case 128: return launch_spmm_r<NPAD, 8>(kind, R, a, grid, st, occ);
        default: return hipErrorInvalidValue;
    }
}

template <int NPAD, int WK>
hipError_t launch_bitmap_n(const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    constexpr int P = 2;  // three stages measured no faster
    if ((a.K & 7) != 0) return run(spmm_bitmap_kernel<NPAD, WK, P, false>, a, grid, st, occ, WK * 64);
    return run(spmm_bitmap_kernel<NPAD, WK, P, true>, a, grid, st, occ, WK * 64);
}

hipError_t launch_bitmap_any(int npad, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    switch (npad) {
        case 16: return launch_bitmap_n<16, kBitmapWaves>(a, grid, st, occ);
        case 32: return launch_bitmap_n<32, kBitmapWaves>(a, grid, st, occ);
        case 64: return launch_bitmap_n<64, kBitmapWaves>(a, grid, st, occ);
        default: return hipErrorInvalidValue;
    }
}

template <int NPAD, int WK>
hipError_t launch_three_level_n(const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    if ((a.K & 7) != 0) return run(spmm_three_level_kernel<NPAD, WK, false>, a, grid, st, occ, WK * 64);
    return run(spmm_three_level_kernel<NPAD, WK, true>, a, grid, st, occ, WK * 64);
}

// N <= 32: the wavefronts of a workgroup split the k range of one row block; N padded to 64:
// four row blocks share the staged B tile.
hipError_t launch_three_level_any(int npad, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    switch (npad) {
        case 16: return launch_three_level_n<16, 4>(a, grid, st, occ);
        case 32: return launch_three_level_n<32, 4>(a, grid, st, occ);
        case 64:
            if ((a.K & 7) != 0) return run(spmm_three_level_shared_kernel<64, false>, a, grid, st, occ);
            return run(spmm_three_level_shared_kernel<64, true>, a, grid, st, occ);
        default: return hipErrorInvalidValue;
    }
}

template <int NW, int RG>
hipError_t launch_wide_rg(int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    if ((a.K & 7) != 0) return run(spmm_wide_kernel<NW, (RG == 4 ? 4 : 8), false, RG>, a, grid, st, occ);
    switch (R) {
        case 1: return run(spmm_wide_kernel<NW, 1, true, RG>, a, grid, st, occ);
        case 2: return run(spmm_wide_kernel<NW, 2, true, RG>, a, grid, st, occ);
        case 4: return run(spmm_wide_kernel<NW, 4, true, RG>, a, grid, st, occ);
        case 8:
            if constexpr (RG != 4) return run(spmm_wide_kernel<NW, 8, true, RG>, a, grid, st, occ);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <int NW>
hipError_t launch_wide_nw(int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    switch (a.TM) {
        case 64: return launch_wide_rg<NW, 4>(R, a, grid, st, occ);
        case 80: return launch_wide_rg<NW, 5>(R, a, grid, st, occ);
        case 96: return launch_wide_rg<NW, 6>(R, a, grid, st, occ);
        case 112: return launch_wide_rg<NW, 7>(R, a, grid, st, occ);
        case 128: return launch_wide_rg<NW, 8>(R, a, grid, st, occ);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_wide_any(int npad, int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    switch (npad) {
        case 128: return launch_wide_nw<2>(R, a, grid, st, occ);
        case 192: return launch_wide_nw<3>(R, a, grid, st, occ);
        case 256: return launch_wide_nw<4>(R, a, grid, st, occ);
        default: return hipErrorInvalidValue;
    }
}

template <int RG>
hipError_t launch_decode_rg(int R, const DecodeArgs& a, int grid, hipStream_t st) {
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, st, a);
        return hipGetLastError();
    };
    if constexpr (RG == 4) {
        switch (R) {
            case 2: return go(decode_kernel<2, RG>);
            case 3: return go(decode_kernel<3, RG>);
            case 5: return go(decode_kernel<5, RG>);
            case 16: return go(decode_kernel<16, RG>);
            default: break;
        }
    }
    switch (R) {
        case 4: return go(decode_kernel<4, RG>);
        case 6: return go(decode_kernel<6, RG>);
        case 8: return go(decode_kernel<8, RG>);
        case 10: return go(decode_kernel<10, RG>);
        case 12: return go(decode_kernel<12, RG>);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

static const int kRegChoices[] = {2, 3, 4, 5, 6, 8, 10, 12, 16};

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

hipError_t launch_spmm(int kind, int npad, int R, const SpmmArgs& a, int grid, hipStream_t st) {
    if (kind == kKernelWide) return launch_wide_any(npad, R, a, grid, st, nullptr);
    if (kind == kKernelBitmap) return launch_bitmap_any(npad, a, grid, st, nullptr);
    if (kind == kKernelThreeLevel) return launch_three_level_any(npad, a, grid, st, nullptr);
    switch (npad) {
        case 16: return launch_spmm_n<16>(kind, R, a, grid, st, nullptr);
        case 32: return launch_spmm_n<32>(kind, R, a, grid, st, nullptr);
        case 64: return launch_spmm_n<64>(kind, R, a, grid, st, nullptr);
        default: return hipErrorInvalidValue;
    }
}

int spmm_blocks_per_cu(int kind, int npad, int R, int K, int TM) {
    int occ = 0;
    SpmmArgs dummy{};
    dummy.K = K;
    dummy.TM = TM;
    hipError_t e = hipErrorInvalidValue;
    if (kind == kKernelWide) return (launch_wide_any(npad, R, dummy, 0, nullptr, &occ) == hipSuccess && occ > 0) ? occ : 1;
    if (kind == kKernelBitmap)
        return (launch_bitmap_any(npad, dummy, 0, nullptr, &occ) == hipSuccess && occ > 0) ? occ : 1;
    if (kind == kKernelThreeLevel)
        return (launch_three_level_any(npad, dummy, 0, nullptr, &occ) == hipSuccess && occ > 0) ? occ : 1;
    switch (npad) {
        case 16: e = launch_spmm_n<16>(kind, R, dummy, 0, nullptr, &occ); break;
        case 32: e = launch_spmm_n<32>(kind, R, dummy, 0, nullptr, &occ); break;
        case 64: e = launch_spmm_n<64>(kind, R, dummy, 0, nullptr, &occ); break;
    }
    return (e == hipSuccess && occ > 0) ? occ : 1;
}

hipError_t launch_reduce(const float* part, uint16_t* C, int S, int64_t NM, hipStream_t st) {
    const int64_t work = (NM & 3) == 0 ? NM / 4 : NM;
    int64_t blocks = (work + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, part, C, S, NM);
    return hipGetLastError();
}

hipError_t launch_decode_bitmap(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL(decode_bitmap_kernel, dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_decode_three_level(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL(decode_three_level_kernel, dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_decode(int R, const DecodeArgs& a, int grid, hipStream_t st) {
    switch (a.TM) {
        case 64: return launch_decode_rg<4>(R, a, grid, st);
        case 80: return launch_decode_rg<5>(R, a, grid, st);
        case 96: return launch_decode_rg<6>(R, a, grid, st);
        case 112: return launch_decode_rg<7>(R, a, grid, st);
        case 128: return launch_decode_rg<8>(R, a, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lscd
