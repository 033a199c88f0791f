// Three-level format (4:2 layer, slot filling, residual): product kernels and dense decode.

#include "lscd_device.h"

namespace lscd {
namespace {

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
    if (active) store_results<4, NPAD / 16, kTileM + 4>(acc, reinterpret_cast<float*>(As), a, s, rb * kTileM, 0, lane);
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

}  // namespace

hipError_t launch_kind_three_level(int npad, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    return launch_three_level_any(npad, a, grid, st, occ);
}

hipError_t launch_decode_three_level(const DecodeArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL(decode_three_level_kernel, dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace lscd
