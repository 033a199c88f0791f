// Tiled-CSL product kernel for N > 64 (up to 256 columns per launch).

#include "lscd_device.h"

namespace lscd {
namespace {

// B operands of one k tile for one wavefront's NB blocks of 16 columns, loaded from global
// memory straight into the layout of v_mfma_f32_16x16x32_f16: for column block j and k step ks,
// lane l holds column n0 + 16j + l % 16 and k = 64 kt + 32 ks + 8 (l / 16) .. +7, i.e. 16
// contiguous bytes of that row of B ([N][K]).  Lanes outside B (n >= N, k >= K, a tile past the split) read
// zero: VEC (K % 8 == 0) through an out-of-range offset of the buffer load, otherwise with
// element-wise guarded loads.
template <int NB, bool VEC>
struct BRegs {
    half8 v[NB][2];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rb, const uint16_t* B, int N, int K, int kt, int n0,
                                         int lane, bool valid) {
        const int rl = lane & 15, kq = lane >> 4;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int n = n0 + j * 16 + rl;
                const int k0 = kt * kTileK + (ks * 4 + kq) * 8;
                const bool in = valid && n < N && k0 < K;
                if constexpr (VEC) {
                    const uint32_t off = in ? (uint32_t)((n * K + k0) * 2) : 0x80000000u;
                    v[j][ks] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
                } else {
                    u32x4 w = {0u, 0u, 0u, 0u};
                    if (in) {
                        const uint16_t* p = B + (size_t)n * K + k0;
                        uint32_t h[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) h[e] = (k0 + e < K) ? p[e] : 0u;
                        w[0] = h[0] | (h[1] << 16);
                        w[1] = h[2] | (h[3] << 16);
                        w[2] = h[4] | (h[5] << 16);
                        w[3] = h[6] | (h[7] << 16);
                    }
                    v[j][ks] = __builtin_bit_cast(half8, w);
                }
            }
        }
    }
};

// acc[i][j] += A rows 16i..16i+15 of the LDS tile (x 64 k) times the B operands in registers.
template <int RG, int NB>
__device__ __forceinline__ void mma_rows_breg(f32x4 (&acc)[RG][NB], const unsigned char* As, const half8 (&bv)[NB][2],
                                              int lane) {
    const uint32_t rl = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < RG; ++i) {
            const half8 af = *reinterpret_cast<const half8*>(As + lds_chunk(i * 16 + rl, ks * 4 + kq));
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bv[j][ks], acc[i][j], 0, 0, 0);
        }
    }
}

// Wide-N variant (64 < N <= 256 per launch; N padded to NW * 64 columns).  Above N = 64 one A
// tile feeds enough MFMA work to keep a whole workgroup busy, so the four wavefronts decode
// each tile together (each loads, and scatters, a quarter of its words) and wavefront w
// multiplies it with its quarter of the columns, NW blocks of 16 from column 16 NW w on, whose
// B operands it loads from global memory into registers (the B tile never passes through LDS:
// the LDS holds only A, so two workgroups fit a CU).  Three LDS A buffers rotate so that one
// barrier per k step orders everything: at step k the workgroup zero-fills buffer (k+1) % 3,
// whose last readers were the MFMAs of step k-2 (all past the barrier of step k-1), and
// scatters into buffer k % 3, whose zero-fill was done before the barrier of step k-1.  The B
// operands of tile k + P are loaded into the registers the MFMAs of tile k have just read.
template <int NW, int R, bool VEC, int RG>
__global__ __launch_bounds__(kThreads) void spmm_wide_kernel(SpmmArgs a) {
    constexpr int TM = 16 * RG;          // rows of the format's tiles
    constexpr int kTB = TM * kRowBytes;  // one A buffer
    static_assert(kThreads == 256, "four wavefronts of 64 columns each");
    constexpr int P = 2;
    __shared__ __attribute__((aligned(16))) unsigned char smem[3 * kTB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
    const int n0 = wave * NW * 16;  // the wavefront's first column

    zero_buf_wg<kTB>(smem, tid);  // A buffer 0 starts zeroed

    u32x4 wb[P][R];
    BRegs<NW, VEC> br[P];
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
        load_tile_wg<R>(wb[q], a.words, o0, nv[q], tid);
        br[q].load(bsrc, a.B, a.N, a.K, k, n0, lane, k < kt1);
    }
    uint32_t o_next = off_at(kt0 + P);
    uint32_t o_pf = off_at(kt0 + P + 1);
    __syncthreads();

    f32x4 acc[RG][NW];
#pragma unroll
    for (int i = 0; i < RG; ++i)
#pragma unroll
        for (int j = 0; j < NW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    int ab = 0;  // A buffer of the current k step
    for (int kt = kt0; kt < kt1; kt += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int k = kt + q;
            const int kn = k + P;
            const int an = ab == 2 ? 0 : ab + 1;
            unsigned char* As = smem + ab * kTB;
            const uint32_t o_pf2 = off_at(kn + 2);
            zero_buf_wg<kTB>(smem + an * kTB, tid);
            const int n = nv[q];
            scatter_tile_wg<R>(wb[q], n, As, tid);
            if (n > R * kThreads) scatter_rest_wg<R>(n, As, a.words + first[q], tid);
            uint32_t o0 = 0, o1 = 0;
            if (kn < kt1) {
                o0 = o_next;
                o1 = o_pf;
            }
            o_next = o_pf;
            o_pf = o_pf2;
            first[q] = o0;
            nv[q] = (int)((o1 - o0) >> 2);
            load_tile_wg<R>(wb[q], a.words, o0, nv[q], tid);
            __syncthreads();
            if (n > 0) mma_rows_breg<RG, NW>(acc, As, br[q].v, lane);
            br[q].load(bsrc, a.B, a.N, a.K, kn, n0, lane, kn < kt1);
            ab = an;
        }
    }
    // Stored straight from the MFMA layout: the whole-line stores through LDS of the other
    // kernels (store_results) measured 1-2 % slower here (OPT-30B MLP1 and OPT-175B OutProj
    // shapes at N = 128).
    const int ncol = lane & 15;
    const int mrow = rb * TM + (lane >> 4) * 4;
    const bool vec_m = (a.M & 3) == 0;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            const int n = n0 + j * 16 + ncol;
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

template <int NW, int RG>
hipError_t launch_wide_rg(int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    if ((a.K & 7) != 0) return run(spmm_wide_kernel<NW, (RG == 4 ? 4 : 8), false, RG>, a, grid, st, occ);
    switch (R) {
        case 1: return run(spmm_wide_kernel<NW, 1, true, RG>, a, grid, st, occ);
        case 2: return run(spmm_wide_kernel<NW, 2, true, RG>, a, grid, st, occ);
        case 4: return run(spmm_wide_kernel<NW, 4, true, RG>, a, grid, st, occ);
        case 8:
            // a 64-row tile holds at most 4096 distinct entries (R = 4 covers them); words past
            // the register stage (duplicates of an imported encoding) take the tail loop
            if constexpr (RG != 4) return run(spmm_wide_kernel<NW, 8, true, RG>, a, grid, st, occ);
            return run(spmm_wide_kernel<NW, 4, true, RG>, a, grid, st, occ);
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

}  // namespace

hipError_t launch_kind_wide(int npad, int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    return launch_wide_any(npad, R, a, grid, st, occ);
}

}  // namespace lscd
