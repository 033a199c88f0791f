// Dispatch of the gfx950 product kernels, the split-K reduction and the Tiled-CSL decode.
// The kernels themselves live in lscd_skinny{16,32,64}.hip (N <= 64), lscd_wide.hip (N > 64),
// lscd_bitmap.hip and lscd_three_level.hip; lscd_device.h holds what they share.

#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "lscd_device.h"

namespace lscd {
namespace {

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

// The same over partial sums in blocks of PB rows ([S][MB][N][PB]): workgroup row y of the grid
// takes column n = y, its threads four consecutive rows m at a time (one block holds them all:
// PB and m are multiples of 4), or one row where M is not a multiple of 4.
__global__ __launch_bounds__(256) void reduce_blocked_kernel(const float* __restrict__ part, uint16_t* __restrict__ C,
                                                             int S, int N, int M, int PB, int MB) {
    const int n = blockIdx.y;
    const int64_t split = (int64_t)MB * N * PB;
    const int step = gridDim.x * 256;
    uint16_t* c = C + (int64_t)n * M;
    if ((M & 3) == 0) {
        for (int m = 4 * (blockIdx.x * 256 + threadIdx.x); m < M; m += 4 * step) {
            const int b = m / PB;
            const int64_t idx = ((int64_t)b * N + n) * PB + (m - b * PB);
            f32x4 acc = *reinterpret_cast<const f32x4*>(part + idx);
            for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const f32x4*>(part + s * split + idx);
            uint2 pk;
            pk.x = (uint32_t)f16_bits(acc[0]) | ((uint32_t)f16_bits(acc[1]) << 16);
            pk.y = (uint32_t)f16_bits(acc[2]) | ((uint32_t)f16_bits(acc[3]) << 16);
            *reinterpret_cast<uint2*>(c + m) = pk;
        }
    } else {
        for (int m = blockIdx.x * 256 + threadIdx.x; m < M; m += step) {
            const int b = m / PB;
            const int64_t idx = ((int64_t)b * N + n) * PB + (m - b * PB);
            float acc = part[idx];
            for (int s = 1; s < S; ++s) acc += part[s * split + idx];
            c[m] = f16_bits(acc);
        }
    }
}

// Streaming-read reference: how fast this GPU streams a buffer of a given size from HBM with
// the product kernels' own load (128-bit buffer loads, non-temporal policy), with no on-chip
// work beyond an XOR per load.  Workgroup w reads one contiguous range of 16-byte vectors, its
// 256 threads 8 vectors apiece per step (32 KB in flight per workgroup), the way a row block's
// wavefronts stream their tiles.  The sink is written only if the XOR of everything read
// equals a key, which keeps the loads alive and almost never writes.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint32_t* __restrict__ src, int64_t nvec,
                                                          int64_t per_wg, uint32_t key, uint32_t* __restrict__ sink) {
    const int64_t v0 = (int64_t)blockIdx.x * per_wg;
    const int64_t v1 = v0 + per_wg < nvec ? v0 + per_wg : nvec;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t base = v0; base < v1; base += 8 * 256) {
        // a descriptor bounded to this step's window: vectors past the range read zero
        const int64_t n = v1 - base < 8 * 256 ? v1 - base : 8 * 256;
        __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(src + 4 * base), (short)0, (int)(n * 16), kBufWord3);
        u32x4 x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (j * 256 + (int)threadIdx.x) * 16, 0, kStreamPolicy);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= x[j];
    }
    const uint32_t h = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (h == key) sink[0] = h;
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
        case 7: return go(decode_kernel<7, RG>);
        case 8: return go(decode_kernel<8, RG>);
        case 9: return go(decode_kernel<9, RG>);
        case 10: return go(decode_kernel<10, RG>);
        case 11: return go(decode_kernel<11, RG>);
        case 12: return go(decode_kernel<12, RG>);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_spmm(int kind, int npad, int R, const SpmmArgs& a, int grid, hipStream_t st) {
    if (kind == kKernelWide) return launch_kind_wide(npad, R, a, grid, st, nullptr);
    if (kind == kKernelBitmap) return launch_kind_bitmap(npad, a, grid, st, nullptr);
    if (kind == kKernelThreeLevel) return launch_kind_three_level(npad, a, grid, st, nullptr);
    switch (npad) {
        case 16: return launch_kind_skinny16(kind, R, a, grid, st, nullptr);
        case 32: return launch_kind_skinny32(kind, R, a, grid, st, nullptr);
        case 64: return launch_kind_skinny64(kind, R, a, grid, st, nullptr);
        default: return hipErrorInvalidValue;
    }
}

int spmm_blocks_per_cu(int kind, int npad, int R, int K, int TM) {
    int occ = 0;
    SpmmArgs dummy{};
    dummy.K = K;
    dummy.TM = TM;
    hipError_t e = hipErrorInvalidValue;
    if (kind == kKernelWide) return (launch_kind_wide(npad, R, dummy, 0, nullptr, &occ) == hipSuccess && occ > 0) ? occ : 1;
    if (kind == kKernelBitmap)
        return (launch_kind_bitmap(npad, dummy, 0, nullptr, &occ) == hipSuccess && occ > 0) ? occ : 1;
    if (kind == kKernelThreeLevel)
        return (launch_kind_three_level(npad, dummy, 0, nullptr, &occ) == hipSuccess && occ > 0) ? occ : 1;
    switch (npad) {
        case 16: e = launch_kind_skinny16(kind, R, dummy, 0, nullptr, &occ); break;
        case 32: e = launch_kind_skinny32(kind, R, dummy, 0, nullptr, &occ); break;
        case 64: e = launch_kind_skinny64(kind, R, dummy, 0, nullptr, &occ); break;
    }
    return (e == hipSuccess && occ > 0) ? occ : 1;
}

hipError_t launch_reduce(const float* part, uint16_t* C, int S, int N, int M, int PB, int MB, hipStream_t st) {
    if (PB > 0) {
        const int64_t work = (M & 3) == 0 ? M / 4 : M;
        int64_t bx = (work + 255) / 256;
        const int64_t cap = std::max<int64_t>(1, 4096 / std::max(N, 1));
        if (bx > cap) bx = cap;
        if (bx < 1) bx = 1;
        hipLaunchKernelGGL(reduce_blocked_kernel, dim3((unsigned)bx, (unsigned)N), dim3(256), 0, st, part, C, S, N, M,
                           PB, MB);
        return hipGetLastError();
    }
    const int64_t NM = (int64_t)N * M;
    const int64_t work = (NM & 3) == 0 ? NM / 4 : NM;
    int64_t blocks = (work + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, part, C, S, NM);
    return hipGetLastError();
}
// The partial sums of lscd_spmm_noalloc live here instead of in a handle's workspace.  In host
// code `scratch` names a host-side stand-in, not device memory: only the address that
// hipGetSymbolAddress returns for the current device may be handed to kernels or copies.
static __device__ __align__(256) float scratch[kScratchBytes / 4];

hipError_t scratch_partials(int device, float** ptr) {
    static std::mutex mu;
    static std::vector<float*> addr;  // per device, filled on first use
    std::lock_guard<std::mutex> lock(mu);
    if (device < 0) return hipErrorInvalidDevice;
    if ((size_t)device >= addr.size()) addr.resize((size_t)device + 1, nullptr);
    if (!addr[(size_t)device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device) return hipErrorInvalidDevice;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[(size_t)device] = (float*)p;
    }
    *ptr = addr[(size_t)device];
    return hipSuccess;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, int blocks, uint32_t* sink, hipStream_t st) {
    const int64_t nvec = bytes / 16;
    if (nvec <= 0 || blocks <= 0) return hipSuccess;
    const int64_t per_wg = (nvec + blocks - 1) / blocks;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint32_t*)src, nvec,
                       per_wg, 0x9E3779B9u, sink);
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
