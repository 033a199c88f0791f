// Bitmap-tile format: product kernel and dense decode.

#include "lscd_device.h"

namespace lscd {
namespace {

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

}  // namespace

hipError_t launch_kind_bitmap(int npad, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    return launch_bitmap_any(npad, a, grid, st, occ);
}

hipError_t launch_decode_bitmap(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL(decode_bitmap_kernel, dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace lscd
