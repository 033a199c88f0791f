// Host-side Tiled-CSL encoder and import validator.
//
// Format (Flash-LLM paper review, xllm-io, section 3 "Tiled-CSL sparse encoding format"):
// the weight matrix is cut into tiles; each kept entry becomes a 32-bit word of
// fp16 value (bits 15:0) and in-tile row-major index (bits 31:16); words are stored tile
// after tile and a per-tile offset array locates each tile.  Tiles are padded to whole
// 128-bit vectors with copies of one of their own words.
//
// Ahead-of-time reorder (same section, "ahead-of-time data reordering"): the order of
// words inside a tile is free, and the pages reorder them offline so that the lanes of
// one store instruction hit different shared-memory banks.  Here the order is built for
// the gfx950 kernel's wave64 scatter: lane l of load slot j holds vector 64*j + l, and
// store instruction (j, e) writes word e of every lane's vector.  Words are dealt
// round-robin over the 64 LDS banks of the kernel's swizzled tile layout, so the lanes of
// one instruction see as many distinct banks as the tile's contents allow.

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "lscd_internal.h"

namespace lscd {

// Largest M and K an encoding accepts.
constexpr int64_t kMaxDim = (int64_t)1 << 30;

bool make_grid(int64_t M, int64_t K, int32_t tm, int32_t tk, Grid* g) {
    if (M < 1 || K < 1 || tm < 1 || tk < 1 || (int64_t)tm * tk > 65536) return false;
    // The kernels index rows and columns, the last row block's padding included, in 32 bits.
    if (M > kMaxDim || K > kMaxDim) return false;
    g->M = M;
    g->K = K;
    g->tm = tm;
    g->tk = tk;
    g->MB = (M + tm - 1) / tm;
    g->KT = (K + tk - 1) / tk;
    g->T = g->MB * g->KT;
    return true;
}

bool reorder_enabled() {
    const char* e = getenv("LSCD_NO_REORDER");
    return !(e && e[0] == '1');
}

namespace {

inline bool kept(const uint16_t* A, const uint8_t* mask, size_t i) {
    return mask ? mask[i] != 0 : (A[i] & 0x7FFF) != 0;
}

// Run body(lo, hi) over [0, n) on a few host threads.
template <class F>
void parallel_for(int64_t n, F body) {
    unsigned hw = std::thread::hardware_concurrency();
    int64_t nt = std::max<int64_t>(1, std::min<int64_t>(hw ? hw : 4, 32));
    nt = std::min(nt, n);
    if (nt <= 1) {
        body(0, n);
        return;
    }
    std::vector<std::thread> pool;
    std::atomic<int64_t> next(0);
    const int64_t chunk = std::max<int64_t>(1, n / (nt * 8));
    for (int64_t t = 0; t < nt; ++t) {
        pool.emplace_back([&]() {
            for (;;) {
                int64_t lo = next.fetch_add(chunk);
                if (lo >= n) break;
                body(lo, std::min(n, lo + chunk));
            }
        });
    }
    for (auto& th : pool) th.join();
}

// LDS bank (of 64 four-byte banks) that the kernel's store of in-tile index `idx` hits
// in its 64 x 64 tile: 128-byte rows, 16-byte chunks XOR-swizzled by (row & 7).
inline int lds_bank(uint32_t idx) {
    uint32_t b = idx * 2u;
    b ^= (b >> 3) & 0x70u;
    return (int)((b >> 2) & 63u);
}

// Place n real words (+ padding) of one tile into out[0 .. 4*nvec), bank-aware.
void place_tile(const uint32_t* w, int n, uint32_t* out, bool reorder, std::vector<uint32_t>& seq,
                std::vector<int>& head, std::vector<int>& nxt) {
    const int nvec = (n + 3) / 4;
    const int np = nvec * 4;
    seq.resize(np);
    if (reorder) {
        // bucket by bank (linked lists keep the ascending index order inside a bucket)
        head.assign(64, -1);
        nxt.assign(n, -1);
        std::vector<int> tail(64, -1);
        for (int i = 0; i < n; ++i) {
            int bk = lds_bank(w[i] >> 16);
            if (tail[bk] < 0) head[bk] = i; else nxt[tail[bk]] = i;
            tail[bk] = i;
        }
        int q = 0;
        while (q < n) {
            for (int bk = 0; bk < 64; ++bk) {
                if (head[bk] >= 0) {
                    seq[q++] = w[head[bk]];
                    head[bk] = nxt[head[bk]];
                }
            }
        }
    } else {
        std::copy(w, w + n, seq.begin());
    }
    for (int q = n; q < np; ++q) seq[q] = seq[n - 1];  // padding: copies of a real word
    // sequence -> (slot j, word e, lane l) instruction-major
    int q = 0;
    for (int j = 0; 64 * j < nvec; ++j) {
        const int L = std::min(64, nvec - 64 * j);
        for (int e = 0; e < 4; ++e)
            for (int l = 0; l < L; ++l) out[4 * (64 * j + l) + e] = seq[q++];
    }
}

}  // namespace

lscd_status_t pack_offsets(const uint16_t* A, const uint8_t* mask, const Grid& g,
                           std::vector<uint32_t>* offsets, int64_t* nnz_out) {
    std::vector<int64_t> cnt((size_t)g.T, 0);
    parallel_for(g.MB, [&](int64_t lo, int64_t hi) {
        for (int64_t bm = lo; bm < hi; ++bm) {
            int64_t* c = cnt.data() + bm * g.KT;
            const int64_t r1 = std::min<int64_t>(g.M, (bm + 1) * g.tm);
            for (int64_t r = bm * g.tm; r < r1; ++r) {
                const size_t base = (size_t)r * (size_t)g.K;
                for (int64_t bk = 0; bk < g.KT; ++bk) {
                    const int64_t c1 = std::min<int64_t>(g.K, (bk + 1) * g.tk);
                    int64_t n = 0;
                    for (int64_t k = bk * g.tk; k < c1; ++k) n += kept(A, mask, base + (size_t)k);
                    c[bk] += n;
                }
            }
        }
    });
    offsets->assign((size_t)g.T + 1, 0);
    uint64_t run = 0;
    int64_t nnz = 0;
    for (int64_t t = 0; t < g.T; ++t) {
        nnz += cnt[(size_t)t];
        run += (uint64_t)((cnt[(size_t)t] + 3) / 4 * 4);
        if (run >= ((uint64_t)1 << 32)) return LSCD_ERROR_NOT_SUPPORTED;
        (*offsets)[(size_t)t + 1] = (uint32_t)run;
    }
    *nnz_out = nnz;
    return LSCD_SUCCESS;
}

void pack_fill(const uint16_t* A, const uint8_t* mask, const Grid& g, const uint32_t* offsets,
               uint32_t* words) {
    // the bank of an index depends only on its row's low bits and its column: any row count
    const bool reorder = reorder_enabled() && g.tk == kTileK && g.tm <= 128;
    parallel_for(g.MB, [&](int64_t lo, int64_t hi) {
        std::vector<uint32_t> buf, seq;
        std::vector<int> head, nxt;
        buf.reserve((size_t)g.tm * g.tk);
        for (int64_t bm = lo; bm < hi; ++bm) {
            const int64_t r0 = bm * g.tm, r1 = std::min<int64_t>(g.M, r0 + g.tm);
            for (int64_t bk = 0; bk < g.KT; ++bk) {
                const int64_t c0 = bk * g.tk, c1 = std::min<int64_t>(g.K, c0 + g.tk);
                buf.clear();
                for (int64_t r = r0; r < r1; ++r) {
                    const size_t base = (size_t)r * (size_t)g.K;
                    for (int64_t c = c0; c < c1; ++c) {
                        if (kept(A, mask, base + (size_t)c)) {
                            uint32_t idx = (uint32_t)((r - r0) * g.tk + (c - c0));
                            buf.push_back((idx << 16) | A[base + (size_t)c]);
                        }
                    }
                }
                const int64_t t = bm * g.KT + bk;
                if (!buf.empty()) place_tile(buf.data(), (int)buf.size(), words + offsets[t], reorder, seq, head, nxt);
            }
        }
    });
}

// ---------------------------------------------------------------- bitmap tiles
// Layout (follow-up summary of the pages, section "Problematica": one bit per position in
// place of per-entry positions), 64 x 64 tiles: the positions of a tile are numbered in the
// operand order of the 16x16x32 MFMA -- lane l, bit b (chunk g = b/8, element b%8) is tile row
// 16*(g/2) + l%16, column 32*(g%2) + 8*(l/16) + b%8 -- and a tile with k kept entries stores the
// 64 lane masks (64-bit, little-endian), then its values chunk by chunk: for g = 0..7 the
// values of bits 8g..8g+7 of lanes 0..63, lane after lane, each lane's in ascending bit order;
// padded with zeros to a multiple of 8 values.  An empty tile stores nothing.  Offsets count
// 16-byte units.

lscd_status_t bitmap_offsets(const uint16_t* A, const uint8_t* mask, const Grid& g, std::vector<uint32_t>* offsets,
                             int64_t* nnz_out) {
    if (g.tm != 64 || g.tk != 64) return LSCD_ERROR_INVALID_VALUE;
    std::vector<int64_t> cnt((size_t)g.T, 0);
    parallel_for(g.MB, [&](int64_t lo, int64_t hi) {
        for (int64_t bm = lo; bm < hi; ++bm) {
            int64_t* c = cnt.data() + bm * g.KT;
            const int64_t r1 = std::min<int64_t>(g.M, (bm + 1) * g.tm);
            for (int64_t r = bm * g.tm; r < r1; ++r) {
                const size_t base = (size_t)r * (size_t)g.K;
                for (int64_t bk = 0; bk < g.KT; ++bk) {
                    const int64_t c1 = std::min<int64_t>(g.K, (bk + 1) * g.tk);
                    int64_t n = 0;
                    for (int64_t k = bk * g.tk; k < c1; ++k) n += kept(A, mask, base + (size_t)k);
                    c[bk] += n;
                }
            }
        }
    });
    offsets->assign((size_t)g.T + 1, 0);
    uint64_t run = 0;
    int64_t nnz = 0;
    for (int64_t t = 0; t < g.T; ++t) {
        const int64_t n = cnt[(size_t)t];
        nnz += n;
        if (n > 0) run += (uint64_t)(g.tm / 2) + (uint64_t)((n + 7) / 8);  // masks: tm * 8 bytes
        if (run * 4 >= ((uint64_t)1 << 32)) return LSCD_ERROR_NOT_SUPPORTED;
        (*offsets)[(size_t)t + 1] = (uint32_t)run;
    }
    *nnz_out = nnz;
    return LSCD_SUCCESS;
}

void bitmap_fill(const uint16_t* A, const uint8_t* mask, const Grid& g, const uint32_t* offsets, uint32_t* words) {
    parallel_for(g.MB, [&](int64_t lo, int64_t hi) {
        for (int64_t bm = lo; bm < hi; ++bm) {
            const int64_t r0 = bm * 64, r1 = std::min<int64_t>(g.M, r0 + 64);
            for (int64_t bk = 0; bk < g.KT; ++bk) {
                const int64_t t = bm * g.KT + bk;
                if (offsets[t + 1] == offsets[t]) continue;
                uint32_t* out = words + 4 * (size_t)offsets[t];
                const size_t nwords = 4 * (size_t)(offsets[t + 1] - offsets[t]);
                memset(out, 0, nwords * 4);
                const int64_t c0 = bk * 64, c1 = std::min<int64_t>(g.K, c0 + 64);
                uint64_t m[64] = {};
                for (int64_t r = r0; r < r1; ++r) {
                    const size_t base = (size_t)r * (size_t)g.K;
                    const int rr = (int)(r - r0);
                    for (int64_t c = c0; c < c1; ++c) {
                        if (!kept(A, mask, base + (size_t)c)) continue;
                        const int cc = (int)(c - c0);
                        const int lane = rr % 16 + 16 * ((cc % 32) / 8);
                        const int bit = 8 * (2 * (rr / 16) + cc / 32) + cc % 8;
                        m[lane] |= (uint64_t)1 << bit;
                    }
                }
                for (int l = 0; l < 64; ++l) {
                    out[2 * l] = (uint32_t)m[l];
                    out[2 * l + 1] = (uint32_t)(m[l] >> 32);
                }
                uint16_t* vals = reinterpret_cast<uint16_t*>(out + 128);
                size_t v = 0;
                for (int gg = 0; gg < 8; ++gg) {
                    for (int l = 0; l < 64; ++l) {
                        for (int bit = 8 * gg; bit < 8 * gg + 8; ++bit) {
                            if (!((m[l] >> bit) & 1)) continue;
                            const int rr = 16 * (gg / 2) + l % 16, cc = 32 * (gg % 2) + 8 * (l / 16) + bit % 8;
                            vals[v++] = A[(size_t)(r0 + rr) * (size_t)g.K + (size_t)(c0 + cc)];
                        }
                    }
                }
            }
        }
    });
}

// ---------------------------------------------------------------- three-level tiles
// Layout (follow-up summary of the pages, section "Metodologia", three-level storage format):
// 64 x 64 tiles; operand i (0..3) and lane l (0..63) of a tile own row 16i + l%16 and
// columns 16*(l/16) .. +15, the lane mapping of the 16x16x64 structured-sparse MFMA.
//   4:2 layer: per group of four columns, slots 2g and 2g+1 hold the first two kept entries
//     with their 2-bit in-group positions; an unused slot holds +0 and the lowest in-group
//     position without a kept entry.
//   slot filling: the third and fourth kept entries of the groups of a lane's region (its 4
//     rows x 16 columns) go, in ascending region position p = 16i + column%16, into the
//     region's unused slots in slot order j = 8i + s; each costs a 4-bit code d - 1 (d = its
//     distance to the previous one, from -1); a gap above 16 gets a +0 dummy 16 positions on;
//     at most 8 codes; the first entry or dummy without a slot or a code stops the placement.
//   residual: the rest, as (fp16 | (r*64 + c) << 16) words in ascending position, padded to
//     a multiple of four with copies of the last word.
// Blob per non-empty tile: 1024 value words (operand-major, 4 words per lane), 256 metadata
// words (per lane: positions of operands 0|1, positions of operands 2|3, fill mask, codes),
// residual words.  Offsets count 16-byte units.

namespace {

struct ThreeLevelTile {
    uint32_t fixed[kThreeLevelFixedWords];
    std::vector<uint32_t> residual;
};

// Build tile (bm, bk) of the three-level format; false when it has no kept entry.
bool three_level_tile(const uint16_t* A, const uint8_t* mask, const Grid& g, int64_t bm, int64_t bk,
                      ThreeLevelTile* out, int64_t* nnz) {
    uint8_t km[64][64];
    uint16_t kv[64][64];
    memset(km, 0, sizeof km);
    memset(kv, 0, sizeof kv);
    int64_t n = 0;
    const int64_t r0 = bm * 64, c0 = bk * 64;
    const int64_t r1 = std::min<int64_t>(g.M, r0 + 64), c1 = std::min<int64_t>(g.K, c0 + 64);
    for (int64_t r = r0; r < r1; ++r) {
        const size_t base = (size_t)r * (size_t)g.K;
        for (int64_t c = c0; c < c1; ++c) {
            if (kept(A, mask, base + (size_t)c)) {
                km[r - r0][c - c0] = 1;
                kv[r - r0][c - c0] = A[base + (size_t)c];
                ++n;
            }
        }
    }
    *nnz = n;
    if (n == 0) return false;
    memset(out->fixed, 0, sizeof out->fixed);
    out->residual.clear();
    uint16_t* vals = reinterpret_cast<uint16_t*>(out->fixed);  // [operand][lane][slot]
    uint32_t* meta = out->fixed + kThreeLevelValueWords;       // [lane][4]
    for (int l = 0; l < 64; ++l) {
        const int q = l >> 4, lr = l & 15;
        int ex_p[32], ex_rc[32], nex = 0;
        uint16_t ex_v[32];
        int unused[32], nun = 0;
        uint32_t idx16[4] = {0, 0, 0, 0};
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * i + lr;
            for (int gi = 0; gi < 4; ++gi) {
                const int cb = 16 * q + 4 * gi;
                int kc[4], fc[4], nk = 0, nf = 0;
                for (int c = 0; c < 4; ++c) {
                    if (km[r][cb + c]) kc[nk++] = c;
                    else fc[nf++] = c;
                }
                for (int s = 0; s < 2; ++s) {
                    const int slot = 2 * gi + s;
                    if (s < nk) {
                        vals[(i * 64 + l) * 8 + slot] = kv[r][cb + kc[s]];
                        idx16[i] |= (uint32_t)kc[s] << (2 * slot);
                    } else {
                        idx16[i] |= (uint32_t)fc[s - nk] << (2 * slot);
                        unused[nun++] = 8 * i + slot;
                    }
                }
                for (int e = 2; e < nk; ++e) {  // ascending region position by construction
                    ex_p[nex] = 16 * i + 4 * gi + kc[e];
                    ex_rc[nex] = r * 64 + cb + kc[e];
                    ex_v[nex] = kv[r][cb + kc[e]];
                    ++nex;
                }
            }
        }
        uint32_t fill = 0, codes = 0;
        int prev = -1, k = 0, u = 0;
        bool stopped = false;
        for (int e = 0; e < nex; ++e) {
            if (!stopped) {
                while (ex_p[e] - prev > 16) {
                    if (u >= nun || k >= kThreeLevelMaxCodes) {
                        stopped = true;
                        break;
                    }
                    fill |= 1u << unused[u++];  // dummy point: the slot keeps +0
                    codes |= 15u << (4 * k++);
                    prev += 16;
                }
                if (!stopped && (u >= nun || k >= kThreeLevelMaxCodes)) stopped = true;
            }
            if (stopped) {
                out->residual.push_back((uint32_t)ex_v[e] | ((uint32_t)ex_rc[e] << 16));
                continue;
            }
            const int j = unused[u++];
            fill |= 1u << j;
            codes |= (uint32_t)(ex_p[e] - prev - 1) << (4 * k++);
            prev = ex_p[e];
            vals[((j >> 3) * 64 + l) * 8 + (j & 7)] = ex_v[e];
        }
        meta[4 * l + 0] = idx16[0] | (idx16[1] << 16);
        meta[4 * l + 1] = idx16[2] | (idx16[3] << 16);
        meta[4 * l + 2] = fill;
        meta[4 * l + 3] = codes;
    }
    std::vector<uint32_t>& rw = out->residual;
    std::sort(rw.begin(), rw.end(), [](uint32_t x, uint32_t y) { return (x >> 16) < (y >> 16); });
    while (!rw.empty() && (rw.size() & 3)) rw.push_back(rw.back());
    return true;
}

}  // namespace

lscd_status_t three_level_offsets(const uint16_t* A, const uint8_t* mask, const Grid& g,
                                  std::vector<uint32_t>* offsets, int64_t* nnz_out) {
    if (g.tm != 64 || g.tk != 64) return LSCD_ERROR_INVALID_VALUE;
    std::vector<uint32_t> units((size_t)g.T, 0);
    std::vector<int64_t> cnt((size_t)g.MB, 0);
    parallel_for(g.MB, [&](int64_t lo, int64_t hi) {
        ThreeLevelTile tile;
        for (int64_t bm = lo; bm < hi; ++bm) {
            for (int64_t bk = 0; bk < g.KT; ++bk) {
                int64_t n = 0;
                if (three_level_tile(A, mask, g, bm, bk, &tile, &n))
                    units[(size_t)(bm * g.KT + bk)] = (uint32_t)((kThreeLevelFixedWords + tile.residual.size()) / 4);
                cnt[(size_t)bm] += n;
            }
        }
    });
    offsets->assign((size_t)g.T + 1, 0);
    uint64_t run = 0;
    int64_t nnz = 0;
    for (int64_t bm = 0; bm < g.MB; ++bm) nnz += cnt[(size_t)bm];
    for (int64_t t = 0; t < g.T; ++t) {
        run += units[(size_t)t];
        if (run * 4 >= ((uint64_t)1 << 32)) return LSCD_ERROR_NOT_SUPPORTED;
        (*offsets)[(size_t)t + 1] = (uint32_t)run;
    }
    *nnz_out = nnz;
    return LSCD_SUCCESS;
}

void three_level_fill(const uint16_t* A, const uint8_t* mask, const Grid& g, const uint32_t* offsets,
                      uint32_t* words) {
    parallel_for(g.MB, [&](int64_t lo, int64_t hi) {
        ThreeLevelTile tile;
        for (int64_t bm = lo; bm < hi; ++bm) {
            for (int64_t bk = 0; bk < g.KT; ++bk) {
                const int64_t t = bm * g.KT + bk;
                int64_t n = 0;
                if (!three_level_tile(A, mask, g, bm, bk, &tile, &n)) continue;
                uint32_t* dst = words + 4 * (size_t)offsets[t];
                memcpy(dst, tile.fixed, sizeof tile.fixed);
                if (!tile.residual.empty())
                    memcpy(dst + kThreeLevelFixedWords, tile.residual.data(), tile.residual.size() * 4);
            }
        }
    });
}

void to_device_words(const uint32_t* in, uint32_t* out, int64_t n) {
    parallel_for((n + 65535) / 65536, [&](int64_t lo, int64_t hi) {
        const int64_t e = std::min<int64_t>(n, hi * 65536);
        for (int64_t i = lo * 65536; i < e; ++i) out[i] = device_word(in[i] >> 16, in[i] & 0xFFFFu);
    });
}

void to_format_words(uint32_t* words, int64_t n) {
    parallel_for((n + 65535) / 65536, [&](int64_t lo, int64_t hi) {
        const int64_t e = std::min<int64_t>(n, hi * 65536);
        for (int64_t i = lo * 65536; i < e; ++i) words[i] = format_word(words[i]);
    });
}

lscd_status_t validate_format(const uint32_t* words, int64_t nwords, const uint32_t* offsets,
                              const Grid& g, int64_t* nnz_out, int32_t* maxw_out) {
    if (offsets[0] != 0 || (int64_t)offsets[g.T] != nwords) return LSCD_ERROR_INVALID_FORMAT;
    for (int64_t t = 0; t < g.T; ++t) {
        if (offsets[t + 1] < offsets[t]) return LSCD_ERROR_INVALID_FORMAT;
        if ((offsets[t + 1] - offsets[t]) & 3u) return LSCD_ERROR_INVALID_FORMAT;
    }
    std::atomic<bool> bad(false);
    std::atomic<int64_t> nnz(0);
    std::atomic<int32_t> maxw(0);
    const uint32_t area = (uint32_t)g.tm * (uint32_t)g.tk;
    parallel_for(g.T, [&](int64_t lo, int64_t hi) {
        std::vector<uint32_t> stamp(area, 0), val(area, 0);
        uint32_t gen = 0;
        int64_t local = 0;
        int32_t lmax = 0;
        for (int64_t t = lo; t < hi && !bad.load(std::memory_order_relaxed); ++t) {
            if (++gen == 0) {  // stamp wrap-around: clear
                std::fill(stamp.begin(), stamp.end(), 0);
                gen = 1;
            }
            const int64_t bm = t / g.KT, bk = t % g.KT;
            const int64_t rows = std::min<int64_t>(g.tm, g.M - bm * g.tm);
            const int64_t cols = std::min<int64_t>(g.tk, g.K - bk * g.tk);
            const uint32_t a = offsets[t], b = offsets[t + 1];
            lmax = std::max<int32_t>(lmax, (int32_t)(b - a));
            for (uint32_t i = a; i < b; ++i) {
                const uint32_t w = words[i];
                const uint32_t idx = w >> 16;
                if (idx >= area || (int64_t)(idx / g.tk) >= rows || (int64_t)(idx % g.tk) >= cols) {
                    bad = true;
                    break;
                }
                if (stamp[idx] == gen) {
                    if (val[idx] != (w & 0xFFFFu)) {
                        bad = true;
                        break;
                    }
                } else {
                    stamp[idx] = gen;
                    val[idx] = w & 0xFFFFu;
                    ++local;
                }
            }
        }
        nnz += local;
        int32_t cur = maxw.load();
        while (lmax > cur && !maxw.compare_exchange_weak(cur, lmax)) {
        }
    });
    if (bad) return LSCD_ERROR_INVALID_FORMAT;
    *nnz_out = nnz.load();
    *maxw_out = maxw.load();
    return LSCD_SUCCESS;
}

}  // namespace lscd
