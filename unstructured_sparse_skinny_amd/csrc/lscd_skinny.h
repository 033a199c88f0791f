// Tiled-CSL product kernels for N <= 64 (shared-B and independent-wavefront variants) and
// their launch tables; instantiated once per N padding, one source file each.

#pragma once

#include "lscd_device.h"

namespace lscd {
namespace {

// Shared-B variant: a workgroup of W wavefronts takes W consecutive row blocks over one K
// split; they share each staged B tile (double-buffered in LDS, one barrier per k step).  W = 4
// in general; W = 3 where it spreads the work more evenly over the CUs (see the planner).
// (Three wavefronts alone would let the compiler take every register of a SIMD; two
// workgroups of three per CU need two wavefronts per SIMD, as four-wavefront workgroups get.)
template <int NPAD, int R, int P, bool VEC, int RG, int W = kWaves>
__global__ __launch_bounds__(64 * W, W == 3 ? 2 : 1) void spmm_kernel(SpmmArgs a) {
    constexpr int TM = 16 * RG;          // rows of the format's tiles
    constexpr int kTB = TM * kRowBytes;  // one wavefront's LDS tile
    constexpr int THREADS = 64 * W;
    __shared__ __attribute__((aligned(16))) unsigned char smem[W * kTB + 2 * NPAD * kRowBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* As = smem + wave * kTB;
    unsigned char* Bs0 = smem + W * kTB;

    // XCD-aware work mapping: hardware places workgroup b on XCD b % 8; give each XCD a
    // contiguous run of work items (items are split-major, so a run shares a B slice).
    const int bid = blockIdx.x;
    const int item = (bid & 7) * a.per_xcd + (bid >> 3);
    if (item >= a.items) return;  // whole workgroup
    const int s = item / a.G;
    const int g = item - s * a.G;
    const int kt0 = (int)(((int64_t)s * a.KT) / a.S);
    const int kt1 = (int)(((int64_t)(s + 1) * a.KT) / a.S);
    const int rb = g * W + wave;
    const bool active = rb < a.MB;
    // Tile offsets are read through the constant address space: the offsets are never
    // written by the kernel, and this lets the compiler use scalar loads (counted apart
    // from the vector loads of the packed words) for these wave-uniform addresses.
    const kconst_u32* toff = (const kconst_u32*)(a.offs) + (int64_t)(active ? rb : 0) * a.KT;
    // B as a buffer of N*K fp16 (requires N*K*2 < 2^31, checked by the host)
    const __amdgpu_buffer_rsrc_t bsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.B, (short)0, a.N * a.K * 2, kBufWord3);

    // B rows n >= N stay zero for the whole kernel (both buffers).
    for (int ch = tid; ch < 2 * NPAD * 8; ch += THREADS) {
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
    BStage<NPAD, VEC, THREADS> bst[P];
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
    // padded column stride: the 16 columns of a block start on different LDS banks
    if (active) store_results<RG, NPAD / 16, TM + 4>(acc, reinterpret_cast<float*>(As), a, s, rb * TM, 0, lane);
}


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
                // Operand prefetch where the LDS already holds one workgroup per CU and its
                // registers fit beside the accumulators and stages (OPT-66B QKV shape, 112-row
                // tiles at N = 32: 55.2 us with it and 2 spilled registers, 54.8 without).
                if constexpr (WK == 8 && (NPAD == 16 || R + RG <= 16))
                    mma_rows_prefetched<NPAD, RG>(acc, As, Bw, lane);
                else
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

template <int R>
constexpr int stages() {
    return shared_stages(R, kTileM);
}
template <int R, int RG>
constexpr bool shared3_fits() {
    return RG == 4 ? (R != 8 && R != 16) : (RG == 5 ? R <= 10 : (RG <= 7 ? R <= 8 : R <= 6));
}
template <int NPAD, int R>
constexpr int stages_indep() {
    return (NPAD == 16 && R <= 4) ? 3 : 2;
}

// Tile heights with kernel instantiations: 64 rows for every variant; 80, 96, 112 and 128
// rows (RG = 5..8 row groups of 16) for the 8-wavefront independent variant (N <= 32), the
// shared-B variant (N <= 64), the wide variant and the decode kernel.  Taller tiles come
// with staging stages R in {4, 6 .. 12}; denser tiles take the path past the stage (R = 16
// with eight wavefronts spills registers).  Each load of a stage past the tile's end still
// issues (reading nothing), so a stage close to the tiles' size pays: OPT-30B MLP1 at 80 %
// sparsity (112-row tiles of at most 1584 words) 29.9 -> 29.6 us with 7 vectors instead of
// 8 at N = 16, 57.7 -> 56.8 at N = 64; the OPT-175B shapes at 50 % (64-row tiles of at most
// about 2200 words, 80-row ones of 2712) 0.5-1.4 % faster with 9 and 11 vectors instead of 10
// and 12, except QKV at N = 64 (0.9 % slower).
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
    if constexpr (NPAD == 64) {
        if (kind == kKernelShared3) {
            // only where two workgroups of three fit a CU without spilling registers (the
            // three-wavefront B stage takes 3 registers of 4 per stage and thread, not 2)
            if constexpr (shared3_fits<R, RG>())
                if (vec) return run(spmm_kernel<NPAD, R, (RG == 4 ? stages<R>() : 2), true, RG, 3>, a, grid, st, occ, 192);
            return hipErrorInvalidValue;
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
        case 7: return launch_spmm_rg<NPAD, 7, RG>(kind, a, grid, st, occ);
        case 8: return launch_spmm_rg<NPAD, 8, RG>(kind, a, grid, st, occ);
        case 9: return launch_spmm_rg<NPAD, 9, RG>(kind, a, grid, st, occ);
        case 10: return launch_spmm_rg<NPAD, 10, RG>(kind, a, grid, st, occ);
        case 11: return launch_spmm_rg<NPAD, 11, RG>(kind, a, grid, st, occ);
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


}  // namespace
}  // namespace lscd
