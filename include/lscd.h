/*
 * lscd.h -- Load-as-Sparse, Compute-as-Dense (LSCD) sparse x skinny matrix product
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (Flash-LLM paper review, xllm-io, section 3 "core formulas"):
 *     C = A x B,  A: M x K pruned fp16 weights (unstructured sparsity),
 *                 B: K x N dense fp16 activations, N small (1..64 here).
 * The product is memory-bound for small N, so A is moved in a compressed form and
 * decompressed on chip into a dense tile that the matrix cores multiply (section 2
 * "solution": load as sparse, compute as dense; redundant multiplications by the
 * pruned zeros are accepted).
 *
 * Memory layouts (the pages leave them open; this library's convention):
 *   B: device fp16, N rows of K elements, row-major      (B[n*K + k], i.e. K x N column-major)
 *   C: device fp16, N rows of M elements, row-major      (C[n*M + m], i.e. M x N column-major)
 *   This is the layout of Y = X . W^T for a batch of N token vectors X[N][K].
 *   fp16 values travel as their 16-bit patterns (uint16_t) on the host side.
 *
 * The compressed format (Tiled-CSL; same review, section 3 "Tiled-CSL sparse encoding
 * format"): A is cut into tile_m x tile_k tiles, ordered row-block-major
 * (t = bm * ceil(K/tile_k) + bk).  Each kept entry is one 32-bit word:
 *     bits [15:0]  fp16 value bits,
 *     bits [31:16] in-tile index r * tile_k + c (row-major inside the tile),
 * so tile_m * tile_k <= 65536.  Words are stored tile after tile; a tile holding n
 * entries occupies round_up(n, 4) words (whole 128-bit vectors), the extra words being
 * exact copies of one of the tile's real words; an empty tile occupies none.  The word
 * order inside a tile is free (this library's encoder orders it for LDS banks).
 * tile_offsets has num_tiles + 1 entries: tile t holds words
 * [tile_offsets[t], tile_offsets[t+1]); tile_offsets[0] = 0.
 *
 * Errors: every call returns a status and never aborts or throws across this ABI.
 * Thread safety: distinct handles may be used from distinct threads; one handle must
 * not run lscd_spmm concurrently on two streams (it owns one split-K workspace).
 */
#ifndef LSCD_H_
#define LSCD_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lscd_handle_s* lscd_handle_t;

typedef enum {
    LSCD_SUCCESS = 0,
    LSCD_ERROR_INVALID_VALUE = 1,   /* bad pointer, size, alignment, device or tile shape   */
    LSCD_ERROR_NOT_SUPPORTED = 2,   /* valid request outside what the kernels implement     */
    LSCD_ERROR_OUT_OF_MEMORY = 3,   /* host or device allocation failed                      */
    LSCD_ERROR_INVALID_FORMAT = 4,  /* imported arrays are not a valid encoding              */
    LSCD_ERROR_HIP = 5              /* a HIP runtime call failed (launch or copy)            */
} lscd_status_t;

typedef struct {
    int64_t M, K;               /* matrix shape                                            */
    int32_t tile_m, tile_k;     /* tile shape of the format                                */
    int64_t num_tiles;          /* ceil(M/tile_m) * ceil(K/tile_k)                         */
    int64_t nnz;                /* stored positions (distinct entries), padding excluded   */
    int64_t nnz_padded;         /* words in the nonzeros array                             */
    int64_t format_bytes;       /* 4 * nnz_padded + 4 * (num_tiles + 1)                    */
    int32_t max_tile_words;     /* largest tile, in words                                  */
    int32_t device;             /* HIP device the handle's buffers live on                 */
    int64_t workspace_bytes;    /* device split-K workspace owned by the handle            */
    int32_t reg_vectors;        /* 128-bit staging registers per lane and tile of the
                                   Tiled-CSL kernels; 0 for formats 1 and 2 (fixed loads)   */
    int32_t splits[3];          /* K-splits across workgroups lscd_spmm uses for N padded to
                                   16, 32 and 64 (1: no second pass)                        */
    int32_t variant[3];         /* product kernel variant for N padded to 16, 32, 64:
                                   0 shared B tile, 1 / 2 independent wavefronts (4 / 8),
                                   3 the N > 64 kernel with N padded to 128 (tiles taller
                                   than 64 rows that overflow the shared-B register stage;
                                   splits[2] then equals splits_wide[0]), 4 bitmap tiles,
                                   5 three-level tiles, 6 shared B tile with three row
                                   blocks per workgroup instead of four (N padded to 64)    */
    int32_t splits_wide[3];     /* K-splits for N > 64, per launch of N padded to 128, 192,
                                   256 (N > 256 runs one launch per 256 columns)            */
    int32_t reg_vectors_wide;   /* 128-bit staging registers per thread, N > 64 kernel      */
    int32_t format;             /* 0 Tiled-CSL, 1 bitmap tiles (lscd_encode_bitmap), 2 three-
                                   level tiles (lscd_encode_three_level); for formats 1 and 2
                                   nnz_padded counts the blob's 32-bit words                */
} lscd_info_t;

#define LSCD_DEFAULT_TILE_M 64
#define LSCD_DEFAULT_TILE_K 64
#define LSCD_NARROW_MAX_N 64   /* largest N of the skinny kernels (one launch)               */
#define LSCD_MAX_N 65535       /* largest N lscd_spmm accepts                                 */

/*
 * lscd_pack_size -- host only, no GPU needed.  Sizes of the encoding of (A, mask).
 *   A      host, M*K fp16 bit patterns, row-major; read only.
 *   mask   host, M*K bytes, nonzero = keep; NULL keeps every entry whose value is not
 *          +0/-0 ((bits & 0x7FFF) != 0).  With a mask, kept zeros are stored as well.
 *   tile_m, tile_k  tile shape, 1 <= tile_m*tile_k <= 65536.
 *   nnz_padded, num_tiles  out: words and tiles of the encoding.
 * Returns INVALID_VALUE for null outputs/A, M or K < 1 or above 2^30 (every encoder and
 * lscd_import), or a bad tile; NOT_SUPPORTED when the encoding would need 2^32 words or more.
 */
lscd_status_t lscd_pack_size(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                             int32_t tile_m, int32_t tile_k, int64_t* nnz_padded, int64_t* num_tiles);

/*
 * lscd_pack -- host only, no GPU needed.  Ahead-of-time encoding of (A, mask) into
 * caller-owned host arrays (Flash-LLM review, section 3: the format is built offline).
 *   nonzeros      out, nonzeros_len >= nnz_padded words.
 *   tile_offsets  out, tile_offsets_len >= num_tiles + 1 entries.
 * Same argument rules as lscd_pack_size; INVALID_VALUE if an output is too short.
 */
lscd_status_t lscd_pack(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                        int32_t tile_m, int32_t tile_k,
                        uint32_t* nonzeros, int64_t nonzeros_len,
                        uint32_t* tile_offsets, int64_t tile_offsets_len);

/*
 * lscd_default_tile_m -- the tile height lscd_encode and lscd_encode_device use for an M x K
 * matrix on the current device (tiles are 64 columns wide; 64, 80, 96, 112 or 128 rows).
 * Without a K split each row block of tiles is one workgroup, so the busiest CU handles
 * ceil(blocks / CUs) blocks; a taller tile is chosen when it cuts that CU's rows by at least
 * 10 %, e.g. 112 rows for M = 28672 on 256 CUs (256 blocks instead of 448).  Matrices whose
 * 64-row blocks do not fill the GPU keep 64 (K splits balance them).  The choice favours
 * N <= 32 (measured on MI355X, 28672 x 7168 at 80 %: N = 16 / 32 / 128 run 10-22 % faster
 * on 112-row tiles, N = 64 ties; 27648 x 9216 at 70 %: N = 64 is 18 % slower);
 * lscd_encode_tiled fixes the height instead.
 * LSCD_ERROR_HIP if there is no device.
 */
lscd_status_t lscd_default_tile_m(int64_t M, int64_t K, int32_t* tile_m);

/*
 * lscd_encode -- pack (A, mask) with 64-column tiles of lscd_default_tile_m rows and upload
 * it to the current HIP device.  Synchronous: the upload is complete on return.  *out
 * receives a handle that owns all device buffers (format and split-K workspace) until
 * lscd_destroy.  A and mask are read only during the call.
 */
lscd_status_t lscd_encode(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                          lscd_handle_t* out);

/* lscd_encode_tiled -- lscd_encode with an explicit tile shape.  Any shape with
 * tile_m * tile_k <= 65536 encodes; lscd_spmm and lscd_debug_decode run tile_k = 64 with
 * tile_m in {64, 80, 96, 112, 128} and return NOT_SUPPORTED for other shapes. */
lscd_status_t lscd_encode_tiled(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                                int32_t tile_m, int32_t tile_k, lscd_handle_t* out);

/*
 * Bitmap-tile variant of the format (the pages' follow-up summary, section "Problematica":
 * per-entry position metadata is as large as the values near 50% sparsity, one bit per
 * position is not).  Same 64 x 64 tiles and tile order as above.  Positions follow the
 * operand layout of the 16x16x32 fp16 MFMA: lane l (0..63), mask bit b (chunk g = b/8) is
 * tile row 16*(g/2) + l%16, column 32*(g%2) + 8*(l/16) + b%8.  A tile with k kept entries
 * stores the 64 lane masks (uint64, little-endian), then its k fp16 values chunk by chunk --
 * for g = 0..7 the values of bits 8g..8g+7 of lanes 0..63, lane after lane, each lane's in
 * ascending bit order -- padded with 0x0000 to a multiple of 8 values; an empty tile stores
 * nothing.  tile_offsets (num_tiles + 1 entries) count 16-byte units.  Bytes:
 * 512 + 16*ceil(k/8) per non-empty tile, against 16*ceil(k/4) for Tiled-CSL.
 *
 * lscd_pack_bitmap_size / lscd_pack_bitmap -- host only.  The encoding of (A, mask) (same
 *   argument rules as lscd_pack; tiles are always 64 x 64) into caller arrays of nwords
 *   32-bit words and num_tiles + 1 offsets.
 * lscd_encode_bitmap -- pack and upload, like lscd_encode.  The handle works with every
 *   entry point taking a handle: lscd_spmm runs the bitmap kernel in launches of up to 64
 *   columns; lscd_export returns the blob and its offsets; lscd_debug_decode and
 *   lscd_attach_dense decode it.
 */
lscd_status_t lscd_pack_bitmap_size(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                                    int64_t* nwords, int64_t* num_tiles);
lscd_status_t lscd_pack_bitmap(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, uint32_t* words,
                               int64_t words_len, uint32_t* tile_offsets, int64_t tile_offsets_len);
lscd_status_t lscd_encode_bitmap(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, lscd_handle_t* out);

/*
 * Three-level tiles (the follow-up summary of the pages, gist.science, section "Metodologia",
 * part 1: a 4:2 structured layer for the sparse matrix instructions, a slot-filling layer
 * whose entries occupy the slots the 4:2 layer leaves unused and whose positions are 4-bit
 * distances, and a residual layer).  Tiles are 64 x 64, in row-block-major order; an empty
 * tile stores nothing; tile_offsets (num_tiles + 1 entries) count 16-byte units.  A non-empty
 * tile is 1280 words plus its residual words:
 *   words 0..1023: 4:2 slots, fp16, in the operand order of v_smfmac_f32_16x16x64_f16:
 *     operand i (0..3), lane l (0..63) at words 4*(64*i + l) .. +3 hold row 16*i + l%16,
 *     columns 16*(l/16) .. +15; slot s (0..7) covers the group of columns 4*(s/2) .. +3 and
 *     sits in the low (even s) or high half of word s/2.  The first two kept entries of a
 *     group (ascending column) take its two slots; an unused slot holds +0.
 *   words 1024 + 4*l .. +3 (lane l): 2-bit in-group positions of operands 0 and 1 (low and
 *     high 16 bits, slot s at bits 2s..2s+1), the same for operands 2 and 3, the fill mask
 *     (bit 8*i + s: the slot holds a slot-filling entry), the codes (code k in bits
 *     4k..4k+3).  An unused slot's position is the lowest in-group position with no kept
 *     entry.
 *   slot filling: the third and fourth kept entries of the groups in lane l's region (its
 *     four rows x 16 columns; region position p = 16*i + column % 16) are placed, in
 *     ascending p, into the region's unused slots in order 8*i + s.  Code k is d - 1 for the
 *     distance d to the previous placed point (the first from p = -1); a gap above 16 is
 *     bridged by a dummy point (+0) 16 positions on; at most 8 codes.  The first entry or
 *     dummy that finds no free slot or code ends the placement for the region.
 *   residual: the remaining entries as (fp16 bits | (r*64 + c) << 16) words in ascending
 *     in-tile position, padded to a multiple of four with copies of the last word.
 *
 * lscd_pack_three_level_size / lscd_pack_three_level -- host only, same argument rules as
 *   lscd_pack_bitmap: the encoding into caller arrays of nwords words and num_tiles + 1
 *   offsets.
 * lscd_encode_three_level -- pack and upload.  lscd_spmm runs the three-level kernel in
 *   launches of up to 64 columns (4:2 slots on the structured-sparse MFMA straight from
 *   registers; slot-filling and residual entries through a dense LDS tile and the dense
 *   MFMA); lscd_export, lscd_debug_decode and lscd_attach_dense work as for the bitmap format.
 */
lscd_status_t lscd_pack_three_level_size(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                                         int64_t* nwords, int64_t* num_tiles);
lscd_status_t lscd_pack_three_level(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K, uint32_t* words,
                                    int64_t words_len, uint32_t* tile_offsets, int64_t tile_offsets_len);
lscd_status_t lscd_encode_three_level(const uint16_t* A, const uint8_t* mask, int64_t M, int64_t K,
                                      lscd_handle_t* out);

/*
 * lscd_encode_device -- lscd_encode for a matrix already in device memory: the encoding
 * (64-column tiles of lscd_default_tile_m rows) is built by GPU kernels (per-tile counts, a prefix sum of the
 * padded counts, then a fill that writes every kept entry straight to its slot) and is
 * word for word the one lscd_encode produces for the same inputs (same bank-aware order
 * inside each tile).  The pages build the format ahead of time on the host (Flash-LLM
 * review, section 3); this serves weights that are loaded or re-pruned on the GPU.
 *   A      device, M*K fp16 row-major, 2-byte aligned; read only.
 *   mask   device, M*K bytes (nonzero = keep), or NULL (keep (bits & 0x7FFF) != 0).
 *   stream the kernels run on it; the call returns when the handle is complete.
 * Allocates the handle's buffers plus O(num_tiles) temporary device memory.  Errors as
 * lscd_encode (INVALID_VALUE for a misaligned A, NOT_SUPPORTED for 2^32 words or more).
 */
lscd_status_t lscd_encode_device(const void* A, const void* mask, int64_t M, int64_t K, void* stream,
                                 lscd_handle_t* out);

/*
 * lscd_import -- validate a caller-built encoding (host arrays, as described above) and
 * upload it to the current device.  Returns INVALID_FORMAT when tile_offsets is not
 * non-decreasing from 0, a tile's word count is not a multiple of 4, the last offset is
 * not the word count given, an index leaves its tile or the matrix, or two words of a
 * tile address one position with different values.
 *   nnz_padded  number of words in nonzeros (must equal tile_offsets[num_tiles]).
 */
lscd_status_t lscd_import(const uint32_t* nonzeros, int64_t nnz_padded, const uint32_t* tile_offsets,
                          int64_t M, int64_t K, int32_t tile_m, int32_t tile_k, lscd_handle_t* out);

/* lscd_export -- copy the handle's encoding back into host arrays of nnz_padded words
 * and num_tiles + 1 offsets (sizes from lscd_get_info).  Synchronous.  The words are in the
 * format's layout (value | in-tile index << 16) whatever form the device copy keeps: on
 * kernel tile shapes the handle stores each word with its LDS byte offset in place of the
 * index, and the export converts back. */
lscd_status_t lscd_export(lscd_handle_t h, uint32_t* nonzeros, uint32_t* tile_offsets);

/* lscd_get_info -- describe a handle (no device work). */
lscd_status_t lscd_get_info(lscd_handle_t h, lscd_info_t* info);

/*
 * lscd_spmm -- C = A x B on `stream` (a hipStream_t; NULL = the null stream).
 *   B  device, N x K fp16 row-major, 16-byte aligned, read only.
 *   C  device, N x M fp16 row-major, 16-byte aligned, fully overwritten.
 *   N  0 is a no-op; 1..LSCD_MAX_N.  Up to 64 columns run in one launch of the skinny
 *      kernels; above that, launches of up to 256 columns each, whose wavefronts share each
 *      decoded A tile (the packed words are read once per launch).  N > LSCD_MAX_N returns
 *      NOT_SUPPORTED, as does a launch whose 256 x K slice of B reaches 2^31 bytes.
 * Asynchronous: returns after enqueueing; launch failures return LSCD_ERROR_HIP.  No
 * allocation or synchronisation inside.  The current device must be the handle's
 * device (INVALID_VALUE otherwise).  Accumulation is fp32, C is rounded once to fp16
 * (nearest-even).  When K is split across workgroups, fp32 partial sums are added in
 * ascending split order by a second pass, so results are bit-reproducible run to run.
 */
lscd_status_t lscd_spmm(lscd_handle_t h, const void* B, void* C, int32_t N, void* stream);

/*
 * lscd_spmm_noalloc -- lscd_spmm for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * layouts, kernels, plan and result (bit-identical to lscd_spmm on the same handle), but the
 * fp32 partial sums of K-split launches go to a static device array of the library, 64 MiB
 * per GPU (allocated with the library's code on each device it runs on and held until the
 * process ends), not to the handle's workspace.  Allocates nothing and calls no allocating
 * routine; the first call on a device looks up that device's copy of the array.
 * Errors: those of lscd_spmm, plus NOT_SUPPORTED when one launch's partials (splits x N x M x
 * 4 bytes, at most 256 columns per launch; M rounded up to whole tiles where N is padded to 64)
 * exceed 64 MiB.  The array is shared by every call
 * on that GPU and keeps the last call's contents (each launch writes every partial it reads,
 * so nothing needs clearing): calls that overlap on one GPU -- on different streams, or from
 * different threads -- race and must be serialized by the caller.
 */
lscd_status_t lscd_spmm_noalloc(lscd_handle_t h, const void* B, void* C, int32_t N, void* stream);

/*
 * lscd_debug_decode -- write the dense M x K fp16 matrix the handle encodes into the
 * device buffer A_dense (row-major, 16-byte aligned), on `stream`.  Uses the same
 * load-and-extract device code as lscd_spmm, so it shows exactly what the product
 * multiplies.  Asynchronous like lscd_spmm.
 */
lscd_status_t lscd_debug_decode(lscd_handle_t h, void* A_dense, void* stream);

/*
 * Dense / sparse selection (Flash-LLM review, section 5 "FasterTransformer integration": the
 * GEMM wrapper picks the dense or the sparse MatMul per call; section 6: the sparse kernel
 * wins while N is small and the product memory-bound, the dense GEMM once N is large).
 *
 * lscd_attach_dense -- decode the handle's encoding into a dense M x K fp16 copy owned by
 * the handle (current device = the handle's) and create the dense GEMM library handle.
 * Synchronous; allocates M*K*2 device bytes; a second call is a no-op.  Freed by
 * lscd_destroy.  NOT_SUPPORTED for tile shapes the kernels are not built for.
 */
lscd_status_t lscd_attach_dense(lscd_handle_t h);

/*
 * lscd_linear -- C = A x B like lscd_spmm (same B, C layouts, alignment and errors), run as
 * the sparse product or, when a dense copy is attached and lscd_linear_path says so, as an
 * fp16 GEMM with fp32 accumulation and one fp16 rounding: the hipBLASLt algorithm that
 * lscd_tune_dense chose for this N, else rocBLAS.  Asynchronous on `stream`.  The dense path
 * may allocate inside the GEMM library on its first call.
 */
lscd_status_t lscd_linear(lscd_handle_t h, const void* B, void* C, int32_t N, void* stream);

/*
 * lscd_tune_dense -- time up to 16 candidates of hipBLASLt's heuristic for the dense GEMM of
 * this handle at width N (the comparison the pages make against the vendor dense library,
 * Flash-LLM review section 6) and keep the fastest for lscd_linear's dense path.  B (N x K)
 * and C (N x M) are caller device buffers as for lscd_spmm; C is overwritten.  Each candidate
 * is timed as 20 calls captured into one HIP graph on a private stream (replayed twice
 * untimed, then once between two events; 2 + 20 eager calls on the default stream if the
 * calls cannot be captured), rotating over copies of the dense matrix whose total exceeds
 * three times the 256 MiB Infinity Cache (2 to 8 copies), so the weights come from HBM as in
 * a model's layer loop rather than from the cache.  *best_us receives the fastest candidate's
 * mean time per GEMM, *candidates how many were timed.  It then times the handle's sparse
 * product at this N the same way (rotating over 2 to 8 copies of the packed words), so that
 * lscd_linear compares two measurements taken alike (lscd_linear_times).  Synchronous.  Needs
 * lscd_attach_dense first (NOT_SUPPORTED otherwise); allocates a 64 MiB workspace on its first
 * call, freed by lscd_destroy, and the extra copies (1 to 7 times M*K*2 bytes, then 1 to 7
 * times the packed words) for the duration of the call; when the copies of the words cannot
 * be allocated the sparse time stays the model's.
 */
lscd_status_t lscd_tune_dense(lscd_handle_t h, const void* B, void* C, int32_t N, double* best_us,
                              int32_t* candidates);

/*
 * lscd_linear_times -- the two times lscd_linear_path compares for N (microseconds): the
 * sparse product's and the dense GEMM's.  *measured = 1 when both come from lscd_tune_dense
 * for this N, 0 when one or both are lscd_linear_model's predictions (or, for bitmap and
 * three-level handles, the per-tile cost).  No device work.
 */
lscd_status_t lscd_linear_times(lscd_handle_t h, int32_t N, double* sparse_us, double* dense_us, int32_t* measured);

/* lscd_linear_path -- the path lscd_linear takes for N: *path = 0 sparse, 1 dense (dense
 * only with a dense copy attached): dense iff its time is below the sparse product's, taking
 * both times from lscd_tune_dense when it has run for this N (lscd_linear_times), and
 * predictions otherwise: lscd_linear_model's for a Tiled-CSL handle, while for a bitmap or
 * three-level handle, which runs one launch per 64 columns whose kernels cost about the
 * same per tile at any density, the sparse time is a fixed part plus a time per tile for each
 * launch (bitmap about 0.9, 1.0 and 1.2 ns per tile for N padded to 16, 32 and 64;
 * three-level 1.0, 1.2 and 1.5).  No device work. */
lscd_status_t lscd_linear_path(lscd_handle_t h, int32_t N, int32_t* path);

/* lscd_set_linear_crossover -- fix the choice: sparse iff N <= n_max_sparse; -1 returns
 * to the cost model (the default). */
lscd_status_t lscd_set_linear_crossover(lscd_handle_t h, int32_t n_max_sparse);

/*
 * lscd_linear_model -- host only.  The cost model behind lscd_linear_path: predicted times
 * (microseconds, MI355X) of the sparse product and of the dense GEMM for an encoding of
 * nnz_padded words in num_tiles tiles of an M x K matrix, times B of N columns.  The sparse
 * estimate counts one read of the packed words per launch of <= 256 columns, B and C once,
 * and the MFMA work of N padded to the kernel width; the dense one counts the fp16 matrix,
 * B and C, and 2*M*N*K flops.
 */
lscd_status_t lscd_linear_model(int64_t M, int64_t K, int64_t nnz_padded, int64_t num_tiles, int32_t N,
                                double* t_sparse_us, double* t_dense_us);

/*
 * lscd_stream_read -- measurement reference, not part of the product: read `bytes` bytes of
 * device memory at `src` (16-byte aligned; bytes rounded down to a multiple of 16) with the
 * product kernels' own 128-bit non-temporal buffer loads and no other work, in
 * `blocks_per_cu` x CUs workgroups of 256 threads, each streaming one contiguous range.  It
 * tells how fast this GPU streams a buffer of that size from HBM -- the ceiling a memory-bound
 * kernel of the same byte count can approach (Flash-LLM review, section 4: the skinny product
 * is bound by global-memory bandwidth).  `sink` is a 4-byte device buffer that is written only
 * in the rare case the XOR of everything read equals a fixed key.  Asynchronous on `stream`;
 * no allocation.  INVALID_VALUE for a null or misaligned pointer or blocks_per_cu outside
 * 1..64.
 */
lscd_status_t lscd_stream_read(const void* src, int64_t bytes, int32_t blocks_per_cu, void* sink, void* stream);

/* lscd_destroy -- free the handle and its device buffers; NULL is a no-op.  The caller
 * must make sure no work using the handle is still running. */
lscd_status_t lscd_destroy(lscd_handle_t h);

/* lscd_status_string -- static text for a status code. */
const char* lscd_status_string(lscd_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* LSCD_H_ */
