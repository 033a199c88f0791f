// Device-side encoder: a dense fp16 matrix (and mask) already in HBM -> the Tiled-CSL
// encoding (64-column tiles of 64 to 128 rows), built by GPU kernels.  The pages build the format
// ahead of time on the host (Flash-LLM paper review, xllm-io, section 3 "Tiled-CSL" and
// "ahead-of-time data reordering"); this is the same encoding, word for word, for callers
// whose weights are already on the GPU (loading or re-pruning a model).
//
//   1. count:  one wavefront per tile counts its kept entries (lane = column, one row at a time);
//   2. scan:   one workgroup turns the per-tile counts into padded word offsets (64-bit
//              running sum, so an encoding of 2^32 words or more is reported, not wrapped),
//              plus the totals the host needs to size the word array;
//   3. fill:   one wavefront per tile writes each kept entry straight to its final slot.
//
// Word order inside a tile is the host encoder's: the kept entries in row-major order are
// bucketed by the LDS bank their scatter store hits (64 banks of the product kernel's
// swizzled tile), and the buckets are dealt round-robin in bank order, each bucket keeping
// ascending index order.  An entry of bank b that is the i-th of its bucket therefore sits
// at sequence position  sum_{r<i} #{banks with more than r entries}  +  #{banks b' < b with
// more than i entries}.  The sequence is padded to whole 128-bit vectors with copies of
// its last word and laid out instruction-major for the wave64 scatter: position q goes to
// slot j = q / 256, and inside the slot (of L = min(64, nvec - 64 j) lanes) to word
// e = u / L of lane l = u % L, u = q - 256 j, i.e. word 4 (64 j + l) + e.

#include <hip/hip_runtime.h>

#include "lscd_internal.h"

namespace lscd {
namespace {

constexpr int kEncWaves = 4;
constexpr int kEncMaxRows = 128;  // tallest tile

struct EncArgs {
    const uint16_t* A;      // [M][K] fp16 bits
    const uint8_t* mask;    // [M][K] or null: keep (bits & 0x7FFF) != 0
    int64_t M, K;
    int64_t MB, KT, T;
    int32_t tm;             // tile rows
    uint32_t* counts;       // [T] kept entries per tile
    uint32_t* offs;         // [T + 1] padded word offsets
    uint32_t* words;        // [offs[T]]
    unsigned long long* stats;  // [0] nnz, [1] words, [2] largest tile (words), [3] overflow
    int reorder;
};

__device__ __forceinline__ bool kept_at(const EncArgs& a, int64_t i) {
    return a.mask ? a.mask[i] != 0 : (a.A[i] & 0x7FFFu) != 0;
}

// LDS bank (of 64 four-byte banks) the product kernel's 16-bit store of in-tile index idx
// hits: 128-byte rows, 16-byte chunks XOR-swizzled by (row & 7).
__device__ __forceinline__ uint32_t scatter_bank(uint32_t idx) {
    uint32_t b = idx * 2u;
    b ^= (b >> 3) & 0x70u;
    return (b >> 2) & 63u;
}

__global__ __launch_bounds__(kEncWaves * 64) void enc_count_kernel(EncArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kEncWaves + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int64_t bm = t / a.KT, bk = t - bm * a.KT;
    const int64_t r0 = bm * a.tm, c = bk * kTileK + lane;
    const int rows = (int)min<int64_t>(a.tm, a.M - r0);
    uint32_t n = 0;
    if (c < a.K)
        for (int r = 0; r < rows; ++r) n += kept_at(a, (r0 + r) * a.K + c) ? 1u : 0u;
    // wave sum
    for (int d = 32; d >= 1; d >>= 1) n += __shfl_xor(n, d, 64);
    if (lane == 0) a.counts[t] = n;
}

// One workgroup: chunk per thread, block scan of the chunk sums, write-back.
__global__ __launch_bounds__(1024) void enc_scan_kernel(EncArgs a) {
    __shared__ unsigned long long part[1024];
    __shared__ unsigned long long nnzs[1024];
    __shared__ unsigned int maxs[1024];
    const int tid = threadIdx.x;
    const int64_t per = (a.T + 1023) / 1024;
    const int64_t lo = min<int64_t>(a.T, tid * per), hi = min<int64_t>(a.T, lo + per);
    unsigned long long sum = 0, nnz = 0;
    unsigned int mx = 0;
    for (int64_t t = lo; t < hi; ++t) {
        const unsigned int c = a.counts[t];
        const unsigned int w = (c + 3u) & ~3u;
        sum += w;
        nnz += c;
        mx = max(mx, w);
    }
    part[tid] = sum;
    nnzs[tid] = nnz;
    maxs[tid] = mx;
    __syncthreads();
    // inclusive Hillis-Steele scan over the 1024 chunk sums (plus reductions)
    for (int d = 1; d < 1024; d <<= 1) {
        const unsigned long long v = tid >= d ? part[tid - d] : 0ull;
        const unsigned long long z = tid >= d ? nnzs[tid - d] : 0ull;
        const unsigned int m = tid >= d ? maxs[tid - d] : 0u;
        __syncthreads();
        part[tid] += v;
        nnzs[tid] += z;
        maxs[tid] = max(maxs[tid], m);
        __syncthreads();
    }
    unsigned long long run = part[tid] - sum;  // exclusive prefix of this chunk
    if (tid == 0) a.offs[0] = 0u;
    for (int64_t t = lo; t < hi; ++t) {
        run += (a.counts[t] + 3u) & ~3u;
        a.offs[t + 1] = (uint32_t)run;  // wraps only when stats[3] says so
    }
    if (tid == 1023) {
        a.stats[0] = nnzs[1023];
        a.stats[1] = part[1023];
        a.stats[2] = maxs[1023];
        a.stats[3] = part[1023] >= (1ull << 32) ? 1ull : 0ull;
    }
}

// Word slot of sequence position q in a tile of nvec vectors (instruction-major layout).
__device__ __forceinline__ uint32_t slot_of(uint32_t q, uint32_t nvec) {
    const uint32_t j = q >> 8, u = q & 255u;
    const uint32_t L = min(64u, nvec - 64u * j);
    const uint32_t e = u / L, l = u - e * L;
    return 4u * (64u * j + l) + e;
}

__global__ __launch_bounds__(kEncWaves * 64) void enc_fill_kernel(EncArgs a) {
    // per wavefront: bucket counters, each entry's rank in its bucket, round masks / offsets
    __shared__ uint32_t cntb[kEncWaves][64];
    __shared__ uint8_t rank[kEncWaves][kEncMaxRows * kTileK];           // a bucket holds <= 2 * rows entries
    __shared__ unsigned long long rmask[kEncWaves][2 * kEncMaxRows];
    __shared__ uint32_t roff[kEncWaves][2 * kEncMaxRows];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kEncWaves + wave;
    if (t >= a.T) return;  // whole wavefront; no barriers below
    const uint32_t o0 = a.offs[t], o1 = a.offs[t + 1];
    if (o1 == o0) return;
    const uint32_t nvec = (o1 - o0) >> 2;
    uint32_t* out = a.words + o0;
    const int64_t bm = t / a.KT, bk = t - bm * a.KT;
    const int64_t r0 = bm * a.tm, c = bk * kTileK + lane;
    const int rows = (int)min<int64_t>(a.tm, a.M - r0);
    const bool col_ok = c < a.K;
    const unsigned long long below = (1ull << lane) - 1ull;

    if (!a.reorder) {
        // row-major order
        uint32_t base = 0;
        uint32_t last_q = 0xFFFFFFFFu, last_w = 0;
        for (int r = 0; r < rows; ++r) {
            const int64_t i = (r0 + r) * a.K + c;
            const bool k = col_ok && kept_at(a, i);
            const unsigned long long bal = __ballot(k);
            if (k) {
                const uint32_t q = base + (uint32_t)__popcll(bal & below);
                const uint32_t w = device_word((uint32_t)(r * kTileK + lane), a.A[i]);
                out[slot_of(q, nvec)] = w;
                last_q = q;
                last_w = w;
            }
            base += (uint32_t)__popcll(bal);
        }
        // padding: copies of the last word of the sequence
        if (last_q == base - 1u)
            for (uint32_t q = base; q < 4u * nvec; ++q) out[slot_of(q, nvec)] = last_w;
        return;
    }

    // pass 1: bucket sizes, and each kept entry's rank inside its bucket (row-major order)
    cntb[wave][lane] = 0u;
    for (int r = 0; r < rows; ++r) {
        const int64_t i = (r0 + r) * a.K + c;
        const bool k = col_ok && kept_at(a, i);
        const unsigned long long bal = __ballot(k);
        const uint32_t bank = scatter_bank((uint32_t)(r * kTileK + lane));
        // columns 2m and 2m + 1 share one bank; the odd one comes second
        const uint32_t before = (lane & 1) ? (uint32_t)((bal >> (lane - 1)) & 1ull) : 0u;
        const uint32_t cur = cntb[wave][bank];
        if (k) rank[wave][r * kTileK + lane] = (uint8_t)(cur + before);
        if ((lane & 1) == 0) cntb[wave][bank] = cur + (uint32_t)__popcll((bal >> lane) & 3ull);
    }
    const uint32_t mycnt = cntb[wave][lane];  // bucket size of bank `lane`
    uint32_t mx = mycnt;
    for (int d = 32; d >= 1; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d, 64));
    uint32_t acc = 0;
    for (uint32_t i = 0; i < mx; ++i) {
        const unsigned long long m = __ballot(mycnt > i);
        if (lane == 0) {
            rmask[wave][i] = m;
            roff[wave][i] = acc;
        }
        acc += (uint32_t)__popcll(m);
    }
    const uint32_t n = acc;
    // pass 2: every kept entry to its slot; the entry at position n - 1 also writes the padding
    for (int r = 0; r < rows; ++r) {
        const int64_t i = (r0 + r) * a.K + c;
        if (!(col_ok && kept_at(a, i))) continue;
        const uint32_t idx = (uint32_t)(r * kTileK + lane);
        const uint32_t bank = scatter_bank(idx);
        const uint32_t ri = rank[wave][idx];
        const uint32_t q = roff[wave][ri] + (uint32_t)__popcll(rmask[wave][ri] & ((1ull << bank) - 1ull));
        const uint32_t w = device_word(idx, a.A[i]);
        out[slot_of(q, nvec)] = w;
        if (q == n - 1u)
            for (uint32_t p = n; p < 4u * nvec; ++p) out[slot_of(p, nvec)] = w;
    }
}

}  // namespace

hipError_t encode_device(const uint16_t* A, const uint8_t* mask, const Grid& g, uint32_t* counts, uint32_t* offs,
                         unsigned long long* stats, hipStream_t s) {
    EncArgs a{};
    a.A = A;
    a.mask = mask;
    a.M = g.M;
    a.K = g.K;
    a.MB = g.MB;
    a.KT = g.KT;
    a.T = g.T;
    a.tm = g.tm;
    a.counts = counts;
    a.offs = offs;
    a.stats = stats;
    const unsigned grid = (unsigned)((g.T + kEncWaves - 1) / kEncWaves);
    hipLaunchKernelGGL(enc_count_kernel, dim3(grid), dim3(kEncWaves * 64), 0, s, a);
    hipLaunchKernelGGL(enc_scan_kernel, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
}

hipError_t encode_device_fill(const uint16_t* A, const uint8_t* mask, const Grid& g, const uint32_t* offs,
                              uint32_t* words, bool reorder, hipStream_t s) {
    EncArgs a{};
    a.A = A;
    a.mask = mask;
    a.M = g.M;
    a.K = g.K;
    a.MB = g.MB;
    a.KT = g.KT;
    a.T = g.T;
    a.tm = g.tm;
    a.offs = const_cast<uint32_t*>(offs);
    a.words = words;
    a.reorder = reorder ? 1 : 0;
    const unsigned grid = (unsigned)((g.T + kEncWaves - 1) / kEncWaves);
    hipLaunchKernelGGL(enc_fill_kernel, dim3(grid), dim3(kEncWaves * 64), 0, s, a);
    return hipGetLastError();
}

}  // namespace lscd
