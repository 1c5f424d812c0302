/*
 * cda.h -- C ABI of the compact decode-attention library (libcda_hip.so).
 *
 * What it implements (FastDMS page, "FastDMS: 6.4X KV-cache compression
 * running faster than vLLM BF16/FP8"):
 *   - DMS paragraph: each (layer, KV head) keeps only the tokens its learned
 *     eviction decision retains.  The decision is an input here: one keep
 *     byte per (sequence, KV head, position), nonzero = keep.
 *   - Release paragraph: a compact KV store that physically reclaims evicted
 *     slots.  kv_compact turns a keep mask into prefix-sum offsets and
 *     stream-compacts K and V into one packed segment per (sequence, KV head).
 *   - Memory-table paragraph, "cache or cache + staging": the W most recent
 *     tokens (the current one included) are always kept, in a ring of W rows
 *     at the front of each segment; a token leaving the ring moves to the
 *     compact tail if its keep bit is set (decode-time append).
 *   - Summary bullets, FP8 and BF16: rows are stored as BF16 or as OCP
 *     E4M3FN FP8 with one absmax scale per (sequence, KV head) for K and one
 *     for V.
 *   - Memory table, the 4-bit vLLM row (a format the page leaves undefined):
 *     a 4-bit store, read here as the OCP MX FP4 element type E2M1 with the
 *     same per-(sequence, KV head) absmax scales, two elements per byte.
 *   - decode_attn_compact: single-token GQA decode attention over the
 *     variable-length compact segments, split into work units whose partial
 *     softmax states are combined by a log-sum-exp merge.  With FP8 the
 *     codes are converted in registers and the scales are folded into the
 *     logit scale and the output (the decompress-in-matvec idea of the
 *     PackKV abstract).
 *
 * One library call = one layer.  All buffers are device memory owned by the
 * caller; the library never allocates, frees or synchronises, and enqueues
 * everything on the caller's stream (a hipStream_t passed as void*, NULL =
 * the null stream).  It keeps no global state and is re-entrant; two calls
 * that touch the same cache must be ordered by the caller (same stream).
 *
 * Storage layout of one layer (all sizes in rows of D elements):
 *   segment i = b*Hkv + h starts at pool row seg_base[i]; its rows are
 *     [0, W)               ring: position p lives in row p mod W
 *     [W, W + seg_cap[i])  compact rows, in ascending position order
 *   and its size W + seg_cap[i] is rounded up to CDA_SEG_ALIGN rows, so
 *   seg_base[i+1] = seg_base[i] + roundup(W + seg_cap[i], CDA_SEG_ALIGN).
 *   The rows holding data are always the contiguous run [0, n_i) with
 *   n_i = min(W, pos[b]) + comp_len[i].
 *   Both pools are split into tiles of CDA_SEG_ALIGN = 64 rows (tile t =
 *   pool rows [64t, 64t+64), 64 * D * e bytes, e = 2 for BF16, 1 for FP8,
 *   1/2 for FP4).
 *   k_pool: rows are cut into 16-byte chunks; chunk c of row r (r taken
 *     inside its tile) is at tile byte
 *       ((m * (D*e/64) + c / 4) * 1024) + (c % 4) * 256 + g * 16,
 *       m = (r / 4) % 4,  g = (r / 16) * 4 + r % 4,
 *     so that every 1 KB of a tile is what one 64-lane load of the attention
 *     kernel needs (the rows of a tile are a permutation of its bytes).
 *   v_pool: a tile is four blocks of 16 rows, each block stored
 *     column-major: element (r, d) at byte
 *       (r / 64) * 64 * D * e + (((r % 64) / 16) * D + d) * 16 * e + (r % 16) * e,
 *     so that 16 consecutive rows of one column are contiguous and the D
 *     values of one row lie in D * 16 * e bytes (FP4, e = 1/2: the low
 *     nibble of that byte for even r, the high nibble for odd r).
 *   FP4 elements of a K row: element d is the low nibble of row byte d / 2
 *     when d is even, the high nibble when odd.
 *   FP8: code = E4M3FN_RNE_SATURATE(f32(x) * inv), inv = 448 / amax and
 *   value = code * s, s = amax / 448 (both single f32 divisions; s = inv = 1
 *   when amax is 0 or not finite).  amax is the largest |x| over the
 *   stored prefill tokens, per (sequence, KV head), for K and V separately;
 *   decode-time tokens use these frozen scales and saturate at +-448.
 *   FP4: code = E2M1_RNE_SATURATE(f32(x) * inv), inv = 6 / amax, value =
 *   code * s, s = amax / 6; NaN encodes as +-6 with its sign (E2M1 has no
 *   NaN).  FP4 needs D = 128 (a K row must fill 64 bytes).
 *
 * Paged store (optional; cache->page_table != NULL).  The release
 * paragraph's point, that the compact store hands evicted memory back to
 * the allocator, carried across requests: the pools are pool_rows / 64
 * pages, a page being one 64-row tile in the formats above, and segment
 * row r (ring and compact rows numbered as above) is row r mod 64 of page
 * page_table[i * max_pages + r / 64].  A segment's pages are the leading
 * entries of its page-table row that are not -1 (the rest are -1), and
 * seg_cap = max(64 * pages - W, 0); seg_base is not used.  Free pages are a
 * stack: free_pages[0 .. *free_top), taken from the top.  Sequences are
 * admitted and released one range at a time (seq_begin, seq_count of
 * cda_compact_args), so requests of different lengths come and go without
 * moving any other sequence's rows:
 *   PAGE_INIT  every page free (free_pages[j] = n - 1 - j, so pages are
 *              first taken in ascending order), page tables -1, pos = -1
 *              (idle), comp_len = seg_cap = 0, err = 0.
 *   COUNT      as for contiguous segments, for the range's sequences, then
 *              takes ceil((W + comp_len + reserve) / 64) pages per segment
 *              (segments in index order, pages in row order, each the top
 *              of the stack), all or nothing: CDA_DEVERR_PAGES if the stack
 *              is short or a segment needs more than max_pages.
 *   PACK       as for contiguous segments, for the range (pos[b] = T);
 *              sequences that COUNT left idle are skipped.
 *   APPEND, decode_step_compact: as for contiguous segments, over all B
 *              sequences; idle ones (pos[b] < 0) are left untouched.
 *   REFILL     for every live segment (pos >= 0), in index order, takes
 *              pages until 64 * pages >= W + comp_len + reserve (at most
 *              max_pages); a short stack serves earlier segments first and
 *              sets CDA_DEVERR_PAGES.  An append uses at most one compact
 *              row per segment, so REFILL with reserve R once every R
 *              steps means no append finds its segment full.
 *   RELEASE    returns the pages of the range's segments to the stack
 *              (segments in index order, pages in row order, so the last
 *              page released is the next taken) and makes them idle.
 * With one range covering the batch right after PAGE_INIT, the pages are
 * laid out exactly as the contiguous segments of the same capacities.
 */
#ifndef CDA_H
#define CDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CDA_VERSION 7
#define CDA_SEG_ALIGN 64        /* rows; segment sizes are rounded up to this */
#define CDA_MAX_GQA 16          /* largest Hq / Hkv supported */
#define CDA_SCRATCH_BYTES (4u << 20) /* device scratch of decode_step_compact_noalloc, per GPU */
#define CDA_MAX_CHUNK 64        /* largest chunk of chunk_attn_compact */
#define CDA_MAX_CHUNK_WINDOW 4096   /* largest W chunk_attn_compact takes */

/* Return codes of every call. */
enum cda_status {
    CDA_OK = 0,
    CDA_ERR_INVALID_ARG = 1,    /* NULL or misaligned pointer, bad size/stride */
    CDA_ERR_UNSUPPORTED = 2,    /* head_dim not 64/128, Hq % Hkv != 0, Hq/Hkv > 16, dtype */
    CDA_ERR_WORKSPACE = 3,      /* workspace smaller than cda_attn_workspace_bytes (noalloc:
                                   the call needs more than CDA_SCRATCH_BYTES) */
    CDA_ERR_HIP = 4             /* a kernel launch failed (hipGetLastError) */
};

/* Bits of the device error word cache->err (set with atomic OR on the GPU;
 * the host sees them only after it synchronises and copies the word). */
#define CDA_DEVERR_CAPACITY 1   /* APPEND: a segment's compact region was full; that token was dropped */
#define CDA_DEVERR_POOL 2       /* PACK/APPEND: a row fell outside [0, pool_rows); not written.
                                   Attention, chunk: a tile of stored rows lies outside the pool
                                   (pool_rows below seg_base[B*Hkv]); not read */
#define CDA_DEVERR_PAGES 8      /* paged COUNT / REFILL: not enough free pages, or a segment
                                   would need more than max_pages (see the paged store) */
#define CDA_DEVERR_MERGE 16     /* attention: a split segment's partial results did not all
                                   arrive within the merge's bounded wait (a bug or a wedged
                                   device, never expected); that call's outputs are not reliable */
#define CDA_DEVERR_PLAN 32      /* attention: seg_base_host differs from the device's seg_base
                                   (a COUNT changed the layout after the host copy was taken);
                                   the segments concerned read nothing and are not appended to,
                                   so that call's outputs and the store are not reliable */

enum cda_kv_dtype { CDA_KV_BF16 = 0, CDA_KV_FP8_E4M3 = 1, CDA_KV_FP4_E2M1 = 2 };
enum cda_out_dtype { CDA_OUT_BF16 = 0, CDA_OUT_F32 = 1 };
enum cda_compact_op { CDA_OP_COUNT = 0, CDA_OP_PACK = 1, CDA_OP_APPEND = 2,
                      CDA_OP_PAGE_INIT = 3, CDA_OP_REFILL = 4, CDA_OP_RELEASE = 5 };

/*
 * One layer's compact store.  The struct itself is host memory read by
 * each call; every pointer in it is device memory owned by the caller.
 * Pointers must be 16-byte aligned (k_pool, v_pool) or naturally aligned.
 */
typedef struct cda_kv_cache {
    int32_t B;          /* sequences */
    int32_t Hkv;        /* KV heads */
    int32_t D;          /* head_dim: 64 or 128 */
    int32_t W;          /* always-kept recent window (ring rows), >= 0 */
    int32_t kv_dtype;   /* enum cda_kv_dtype */
    int32_t spare_rows; /* hint, >= 0 (0 = none): rows at the end of every segment's capacity
                           the caller expects to hold no data in this call, typically the
                           COUNT reserve not yet filled.  With seg_base_host, the tiles of a
                           segment's span lying wholly past (span - spare_rows + 64) rows are
                           read only once the segment's metadata shows data in them, instead
                           of ahead of it.  Changes no result, only which reads go out early
                           (a wrong hint costs time, never correctness) */
    int64_t pool_rows;  /* rows allocated in k_pool and v_pool (multiple of 64) */
    void *k_pool;       /* [pool_rows / 64] tiles of 64 x D, chunk-permuted (see above) */
    void *v_pool;       /* [pool_rows / 64][4][D][16 rows] */
    int64_t *seg_base;  /* [B*Hkv + 1]; written by COUNT; [B*Hkv] = rows needed */
    int32_t *seg_cap;   /* [B*Hkv]; written by COUNT */
    int32_t *comp_len;  /* [B*Hkv]; written by COUNT, grown by APPEND */
    int32_t *pos;       /* [B]; tokens seen so far (next position); PACK sets T */
    uint8_t *ring_keep; /* [B*Hkv*W]; keep bit of the token each ring row holds */
    float *k_amax;      /* [B*Hkv]; FP8/FP4 absmax of K (PACK computes or takes it) */
    float *v_amax;      /* [B*Hkv]; FP8/FP4 absmax of V */
    int32_t *err;       /* [1]; device error word, CDA_DEVERR_* bits; COUNT clears it */
    const int64_t *seg_base_host; /* optional HOST memory (may be NULL): a copy of seg_base
                           [0 .. B*Hkv] as COUNT wrote it, contiguous segments only.  With it,
                           decode_attn_compact and decode_step_compact plan their work units on
                           the host and pass the plan with the kernel arguments, so the kernel
                           reads K and V before the segment metadata has arrived.  Checked on
                           every call (non-decreasing multiples of 64, last entry <= pool_rows,
                           CDA_ERR_INVALID_ARG otherwise); a copy that no longer matches the
                           device's seg_base sets CDA_DEVERR_PLAN.  Ignored by the paged store
                           and by kv_compact */
    int32_t *page_table;   /* NULL: contiguous segments.  Else the paged store:
                              [B*Hkv*max_pages] page ids, -1 = none */
    int32_t max_pages;     /* paged: page-table entries per segment, >= 1 */
    int32_t reserved1;     /* must be 0 */
    int32_t *free_pages;   /* paged: [pool_rows/64] stack of free page ids (pool_rows >= 64) */
    int32_t *free_top;     /* paged: [1] number of free pages */
} cda_kv_cache;

/*
 * Arguments of kv_compact.  Element strides are in elements of the BF16
 * input; rows of D elements must be contiguous and 16-byte aligned.
 */
typedef struct cda_compact_args {
    int32_t op;         /* enum cda_compact_op */
    int32_t T;          /* COUNT, PACK: prefill length, 0 <= T <= 2^24 */
    int32_t reserve;    /* COUNT: spare compact rows per segment for decode growth (>= 0) */
    int32_t scale_mode; /* PACK with FP8/FP4: 0 = compute k_amax/v_amax, 1 = use them as given */
    const uint8_t *keep;/* COUNT, PACK: row i = b*Hkv+h at keep + i*keep_ld, first T bytes used;
                           APPEND: [B*Hkv] bytes, one per head for the new token */
    int64_t keep_ld;    /* COUNT, PACK: bytes between keep rows (>= T) */
    const void *k;      /* PACK: BF16, (b,t,h,d) at b*stride_b + t*stride_t + h*stride_h + d;
                           APPEND: BF16, (b,h,d) at b*stride_b + h*stride_h + d */
    const void *v;      /* same layout as k */
    int64_t stride_b, stride_t, stride_h;
    int32_t *dst_out;   /* COUNT, optional (may be NULL): [B*Hkv*T] int32, the segment row
                           each position is stored in (ring p mod W or W + rank), -1 if evicted */
    int32_t seq_begin;  /* paged COUNT, PACK, RELEASE: sequences [seq_begin, seq_begin +
                           seq_count); keep, k, v and dst_out then start at sequence seq_begin
                           (their sequence index is b - seq_begin).  seq_count = 0: all B
                           (seq_begin 0).  Contiguous segments: both 0 */
    int32_t seq_count;
} cda_compact_args;

/*
 * kv_compact -- prefill compaction and decode-time append of one layer.
 *
 * CDA_OP_COUNT: per segment, counts kept positions p <= T-1-W (comp_len),
 *   sets seg_cap = comp_len + reserve, and writes seg_base by an exclusive
 *   prefix sum of the aligned segment sizes; seg_base[B*Hkv] is the number
 *   of pool rows to allocate.  Optionally writes dst_out.
 *   Clears *err.
 *   Reads keep; needs seg_base, seg_cap, comp_len, err (pools may be NULL).
 * CDA_OP_PACK: after COUNT (same keep, T), writes every stored prefill row
 *   (the W most recent positions and every kept older one) to its pool row,
 *   fills ring_keep, sets pos[b] = T and, for FP8/FP4 with scale_mode 0,
 *   computes k_amax/v_amax first.  Pools are written in whole 64-row
 *   tiles: unused rows inside a tile that holds ring or stored rows are set
 *   to zero; tiles past them are not written.
 * CDA_OP_PAGE_INIT, CDA_OP_REFILL, CDA_OP_RELEASE: paged store only (see
 *   the paged store above; REFILL reads reserve, RELEASE the range).
 * CDA_OP_APPEND: one decode step: for each sequence b (P = pos[b]) and head,
 *   the token at P-W leaves the ring and, if its keep bit is set, is copied
 *   to compact row W + comp_len (comp_len += 1; CDA_DEVERR_CAPACITY if
 *   comp_len == seg_cap); then the new token is written to ring row P mod W
 *   (W = 0: straight to the compact tail if kept) and pos[b] = P + 1.
 *
 * Returns CDA_OK or an error code; errors are detected before anything is
 * enqueued, except CDA_ERR_HIP.  Never prints, never aborts.
 */
int32_t kv_compact(const cda_kv_cache *cache, const cda_compact_args *args, void *stream);

/*
 * decode_attn_compact -- single-token GQA decode attention of one layer.
 *
 * For sequence b and query head j (KV head h = j / (Hq / Hkv)):
 *   z_p = sm_scale * q[b,j,:] . k^_p    over the n_i stored rows of segment i
 *   out[b,j,:] = sum_p softmax(z)_p v^_p,   lse[b,j] = log sum_p exp(z_p)
 * where k^, v^ are the stored values (BF16, or FP8/FP4 code * scale).  A segment
 * with no stored rows gives out = 0 and lse = -inf.
 *
 *   q            BF16 [B, Hq, D] contiguous, 16-byte aligned
 *   sm_scale     softmax scale; <= 0 means 1/sqrt(D)
 *   out          [B, Hq, D] contiguous, BF16 or F32 per out_dtype
 *   lse          optional F32 [B, Hq] (natural log), may be NULL
 *   split_tokens rows per work unit (one workgroup), rounded up to a
 *                multiple of 64; 0 = default, chosen from pool_rows and
 *                B*Hkv: the smallest of 256 (pools under 65536 rows only),
 *                512, 768, 1024, 1536, ... 4096 for which the estimated
 *                number of units, pool_rows/split + B*Hkv/2, stays at or
 *                below 248 (about one resident 8-wave workgroup per compute
 *                unit); 512 when none does.  Segments longer than one unit
 *                are split and their partials merged.  With seg_base_host
 *                the units cover each segment's capacity (W + seg_cap
 *                rows), otherwise the rows holding data (decode_step: the
 *                capacity as well).
 *   workspace    device scratch of at least cda_attn_workspace_bytes()
 *                bytes, 16-byte aligned: one completion counter per segment
 *                and per sequence, then one partial-result slot per work
 *                unit.  It must be zero-filled before its first use; every
 *                completed call leaves it zero-filled again, so one
 *                workspace can serve any later call (any cache, any split)
 *                ordered after it on a stream.  Calls that may run
 *                concurrently need separate workspaces.
 */
int32_t decode_attn_compact(const cda_kv_cache *cache, const void *q, int32_t Hq,
                            float sm_scale, void *out, int32_t out_dtype, float *lse,
                            int32_t split_tokens, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * decode_step_compact -- one decode step of one layer in a single launch:
 * the APPEND operation of kv_compact followed by decode_attn_compact over
 * the appended store (FastDMS memory-table paragraph, "cache + staging",
 * for the append; decode over the compact store as above).
 *
 *   args         the APPEND arguments of kv_compact (op must be
 *                CDA_OP_APPEND): the new token's BF16 K and V rows and its
 *                keep byte per (sequence, KV head)
 *   other arguments as for decode_attn_compact, with the same workspace.
 *
 * Afterwards the cache (pools, comp_len, ring_keep, pos, err) is bit for bit
 * what kv_compact(APPEND) leaves, and out / lse are the attention of q over
 * the stored rows after the append.  The attention is computed from the
 * rows as they were before the append plus the new token in registers, so
 * the kernel never reads a row that the append writes in the same launch.
 * Errors as for the two calls it replaces.
 */
int32_t decode_step_compact(const cda_kv_cache *cache, const cda_compact_args *args,
                            const void *q, int32_t Hq, float sm_scale, void *out,
                            int32_t out_dtype, float *lse, int32_t split_tokens,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * decode_step_compact_noalloc -- decode_step_compact for callers that cannot
 * allocate device memory or own a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments
 * and results as decode_step_compact, without the workspace: the library
 * keeps one static device array of CDA_SCRATCH_BYTES per GPU (allocated
 * with the code object, held until the process ends) and uses it in its
 * place.  Nothing is allocated or freed by the call.
 *
 *   Returns CDA_ERR_WORKSPACE, before anything is enqueued, when the call
 *   needs more scratch than CDA_SCRATCH_BYTES (cda_attn_workspace_bytes of
 *   the same cache, Hq and split_tokens); CDA_ERR_INVALID_ARG when the
 *   stream does not belong to the current device.  The first call on a GPU
 *   enqueues the array's zero fill ahead of its kernel; every completed call
 *   leaves it zero-filled again.  All calls on one GPU share its array:
 *   calls that may run concurrently on one GPU (different streams without
 *   ordering between them) race and must not be issued.
 */
int32_t decode_step_compact_noalloc(const cda_kv_cache *cache, const cda_compact_args *args,
                                    const void *q, int32_t Hq, float sm_scale, void *out,
                                    int32_t out_dtype, float *lse, int32_t split_tokens,
                                    void *stream);

/* Workspace bytes decode_attn_compact and decode_step_compact need for this
 * cache, Hq and split. */
size_t cda_attn_workspace_bytes(const cda_kv_cache *cache, int32_t Hq, int32_t split_tokens);

/*
 * chunk_attn_compact -- a chunk of M new tokens per sequence: multi-query
 * attention over the compact store, then their append.
 *
 * The step around the decode path, given by PyramidInfer's point that the
 * cache is compressed already while the prompt is processed, on the FastDMS
 * store (memory-table paragraph: compact cache plus W-token staging): the
 * prompt continues chunk by chunk on top of a compacted context (or several
 * draft tokens are scored at once).  Sequence b receives tokens at positions
 * P .. P+M-1 (P = pos[b]); query t is answered exactly as decode_step_compact
 * would answer it at position P + t after appending tokens P .. P+t one at a
 * time:
 *   out[b,t,j,:] = sum_p softmax(z)_p v^_p over the rows stored after token
 *   P + t, z_p = sm_scale * q[b,t,j,:] . k^_p, lse[b,t,j] = log sum_p exp(z_p)
 * (the compact rows; ring rows and chunk tokens t' <= t that are still in
 * query t's window or kept).  Afterwards the cache is bit for bit what M
 * successive kv_compact(APPEND) calls leave (pos[b] += M).
 *
 *   args       APPEND arguments: k, v BF16, token t of head h of sequence b
 *              at b*stride_b + t*stride_t + h*stride_h + d (16-byte aligned
 *              rows); keep [B, M, Hkv] bytes at keep + (b*M + t)*Hkv + h
 *   M          1 .. CDA_MAX_CHUNK
 *   q          BF16 [B, M, Hq, D] contiguous, 16-byte aligned
 *   out        [B, M, Hq, D] contiguous, BF16 or F32 per out_dtype, 16-byte aligned
 *   lse        optional F32 [B, M, Hq]
 *   workspace  at least cda_chunk_workspace_bytes() bytes, 256-byte aligned,
 *              any contents (the chunk's encoded rows and the partial states)
 * Every sequence of a contiguous store takes part; with a paged store, idle
 * sequences (pos < 0) give out = 0, lse = -inf and are not appended to.
 * Errors as for kv_compact and decode_attn_compact; W above
 * CDA_MAX_CHUNK_WINDOW is CDA_ERR_UNSUPPORTED; the compact region must have
 * room for the chunk (CDA_DEVERR_CAPACITY otherwise, as for APPEND).
 */
int32_t chunk_attn_compact(const cda_kv_cache *cache, const cda_compact_args *args, int32_t M,
                           const void *q, int32_t Hq, float sm_scale, void *out,
                           int32_t out_dtype, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Workspace bytes chunk_attn_compact needs for this cache, Hq and M (0 if
 * they are invalid). */
size_t cda_chunk_workspace_bytes(const cda_kv_cache *cache, int32_t Hq, int32_t M);

/* Static text for a cda_status value. */
const char *cda_status_string(int32_t status);

/* CDA_VERSION of the built library. */
int32_t cda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CDA_H */
