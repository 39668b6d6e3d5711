/*
 * pda.h - paged split-K decode attention on AMD Instinct MI355X (gfx950).
 *
 * The operation (vllm-rdna pull request #33, "perf(rocm): FA-RDNA2 decode,
 * scores on every wave and 4 barriers per tile", section "Purpose"): for
 * every new query token t of sequence b and every query head h,
 *
 *     out[t, h, :] = softmax_j(scale * q[t, h, :] . k_j) . v_j
 *
 * over the keys j the token can see. K and V live in fixed-size pages of a
 * shared pool, reached through the sequence's block-table row; query head h
 * reads KV head h / G with G = num_q_heads / num_kv_heads (consecutive query
 * heads share a KV head). A sequence holds seq_lens[b] keys, its q_lens[b]
 * new tokens included: token i sits at position p = seq_lens[b] - q_lens[b]
 * + i and sees keys lo..p, with lo = 0, or lo = max(0, p - window + 1) under a
 * sliding window of `window` keys. A token that sees no key (p < 0) gets an
 * all-zero row. The behaviours named in the pull request's "Test Plan" (zero
 * rows, a caller scale written into a caller `out`, sliding window,
 * multi-token queries, split decode) are part of this contract.
 *
 * Work is split along the key axis into `num_splits` contiguous chunks per
 * (sequence, KV head), aligned to 16 keys; each chunk yields a partial
 * (m, l, o) and a second kernel merges the partials (the split-K combine of
 * the same section).
 *
 * Conventions for every entry point
 *  - All tensors are contiguous, row-major, and live in device memory of the
 *    current HIP device; the caller owns them. The library never allocates,
 *    frees or synchronizes and issues no memsets, so a call can be captured
 *    in a HIP graph; with automatic splits a captured call balances whatever
 *    seq_lens / q_lens hold when it is replayed. Its only device state is the
 *    scratch array of pda_paged_decode_attention_noalloc (a module global,
 *    one per device, never allocated at run time).
 *  - Every launch goes on the caller's `stream` (the pull request passes the
 *    current stream to every launch); calls return after enqueueing.
 *  - Arguments are validated on the host before any HIP call; a failure
 *    returns a negative pda_status and sets pda_last_error(). Values that
 *    live in device memory are a contract, not checked (checking would need
 *    a synchronization): 0 <= seq_lens[b] <= max_pages_per_seq * page_size;
 *    1 <= q_lens[b] <= max_q_len; sum(q_lens) == num_tokens; the block-table
 *    entries of the first ceil(seq_lens[b] / page_size) columns of row b are
 *    in [0, num_pages). Other table entries, and page slots past a
 *    sequence's length, are never read and may hold anything (NaN included).
 *  - The environment variable PDA_PREFILL_CUS, read at each call, set to a
 *    positive count below the device's CU count sizes the long-query
 *    kernel's persistent grid for that many CUs instead (a small problem then
 *    runs many work items per workgroup in turn); results do not depend on it.
 */
#ifndef PDA_H_
#define PDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pda_status {
  PDA_OK = 0,
  PDA_ERR_NULL = -1,        /* a required pointer is NULL */
  PDA_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
  PDA_ERR_ALIGN = -3,       /* a data pointer is not 16-byte aligned */
  PDA_ERR_UNSUPPORTED = -4, /* valid, but no compiled kernel covers it */
  PDA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than needed */
  PDA_ERR_DEVICE = -6       /* the HIP runtime reported an error */
} pda_status;

/* Element type of the KV cache. fp16 is IEEE binary16. fp8 is OCP E4M3
 * ("fn": bias 7, no infinities, max 448). int8 is symmetric signed with no
 * zero point. For fp8 and int8 the value of a code is code_value * scale with
 * one fp32 scale per KV head for K and one for V (the pull request's fp8 and
 * int8 decode wrappers, section "Purpose"). */
typedef enum pda_kv_dtype {
  PDA_KV_F16 = 0,
  PDA_KV_FP8_E4M3 = 1,
  PDA_KV_INT8 = 2
} pda_kv_dtype;

/* Cache layout: where key j's row of KV head g sits inside its page.
 *  PDA_LAYOUT_NHD: [num_pages, P, Hkv, D] (page, slot, KV head, dim), the
 *    cache writer's layout (PR #33 "Test Plan").
 *  PDA_LAYOUT_HND: [num_pages, Hkv, P, D] (page, KV head, slot, dim): each
 *    head's rows of a page are contiguous. */
typedef enum pda_kv_layout {
  PDA_LAYOUT_NHD = 0,
  PDA_LAYOUT_HND = 1
} pda_kv_layout;

/* Decode kernel family. Both compute the same function and are checked
 * against the same reference; they differ in where the arithmetic runs.
 *  PDA_KERNEL_VECTOR: scores with packed fp16 v_dot2 (fp32 accumulation) and
 *    DPP cross-lane sums, P.V with fp32 FMAs; the pull request's "packed
 *    fdot2" design (section "Purpose") carried to wave64.
 *  PDA_KERNEL_MATRIX: Q.K^T and P.V on the MFMA units (fp16 operands, fp32
 *    accumulation; P rounded to fp16 for the P.V product).
 *  PDA_KERNEL_PREFILL: the long-query kernel: one workgroup per block of
 *    new tokens of a sequence and KV head (128 or 256 query rows at D=128,
 *    128 at D=256), K/V staged once per workgroup through LDS for all its
 *    rows, MFMA for both products.
 *    For prefill, chunked prefill and long verification runs; always one
 *    split (num_splits 0 or 1).
 *  PDA_KERNEL_AUTO: the matrix kernel while (Hq / Hkv) * max_q_len <=
 *    PDA_MAX_ROWS, the prefill kernel above that. */
typedef enum pda_kernel {
  PDA_KERNEL_AUTO = 0,
  PDA_KERNEL_VECTOR = 1,
  PDA_KERNEL_MATRIX = 2,
  PDA_KERNEL_PREFILL = 3
} pda_kernel;

/* Sizes of one call. */
typedef struct pda_decode_dims {
  int32_t batch;             /* B: sequences (0: nothing to do) */
  int32_t num_tokens;        /* T = sum(q_lens); B when q_lens is NULL */
  int32_t num_q_heads;       /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;      /* Hkv */
  int32_t head_dim;          /* D: 128 or 256 */
  int32_t page_size;         /* P: keys per page: 16, 32, 64, 128 or 256
                                (16 only for PDA_KERNEL_VECTOR) */
  int32_t num_pages;         /* pages in each of the K and V pools */
  int32_t max_pages_per_seq; /* columns of block_table */
  int32_t max_q_len;         /* bound on q_lens[b]; 1 when q_lens is NULL */
  int32_t kv_dtype;          /* a pda_kv_dtype */
  int32_t kernel;            /* a pda_kernel: which decode kernel family runs */
  int32_t kv_layout;         /* a pda_kv_layout (NHD only for PDA_KERNEL_VECTOR) */
} pda_decode_dims;

/* Largest (num_q_heads / num_kv_heads) * max_q_len of the decode kernels
 * (vector, matrix); larger calls run the prefill kernel, which takes any
 * max_q_len with num_q_heads / num_kv_heads <= PDA_MAX_GROUP. */
#define PDA_MAX_ROWS 32
#define PDA_MAX_GROUP 128
/* Largest number of key splits. */
#define PDA_MAX_SPLITS 256

/*
 * Decode attention, written into `out`.
 *
 *  q            fp16 [T, Hq, D]; the tokens of sequence b are rows
 *               off_b .. off_b + q_lens[b] - 1, off_b = sum of q_lens[<b].
 *  k_cache      [num_pages, P, Hkv, D] (NHD) or [num_pages, Hkv, P, D]
 *  v_cache      (HND) of kv_dtype elements, per dims->kv_layout; one page
 *               (P * Hkv * D elements) must be under 2 GiB.
 *  block_table  int32 [B, max_pages_per_seq]: key j of sequence b is slot
 *               j % P of page block_table[b][j / P].
 *  seq_lens     int32 [B]: keys held by each sequence, new tokens included.
 *  q_lens       int32 [B], or NULL: every sequence has one new token.
 *  scale        multiplier of q.k (fp32), e.g. 1/sqrt(D).
 *  window       sliding window in keys; <= 0: none.
 *  num_splits   key splits per (sequence, KV head), 1..PDA_MAX_SPLITS; or 0
 *               for an automatic choice (below).
 *  out          fp16 [T, Hq, D], fully overwritten.
 *  k_scale      fp32 [Hkv] for fp8/int8 KV (NULL for fp16).
 *  v_scale      fp32 [Hkv] for fp8/int8 KV (NULL for fp16).
 *  workspace    device scratch for the split partials, at least
 *               pda_decode_workspace_bytes(dims, window, num_splits) bytes,
 *               16-byte aligned; may be NULL when that size is 0 (one split).
 *               Calls that overlap on one workspace race.
 *
 * With one split the decode kernel writes `out` directly; with more, it
 * writes partials and a second launch (the combine kernel) merges them. Both
 * launches go on `stream`.
 *
 * Automatic splits (num_splits 0) with the matrix kernel balance the work
 * over the batch when it has fewer sequences than the workgroups that fit on
 * the device at once: the decode kernel reads seq_lens and q_lens and cuts
 * every sequence into chunks of one common size (in 16-key tiles), the
 * smallest size whose chunks all fit in one round of workgroups, so a ragged
 * batch's long sequences get proportionally more splits (at most
 * PDA_MAX_SPLITS per row). A sequence that gets one chunk is written to `out`
 * by the decode kernel; the combine merges the others. A uniform batch gets
 * the same chunks as a fixed count would give it. Otherwise (vector kernel,
 * or a batch as large as one round) the automatic count is
 * pda_decode_resolve_splits's, the same for every sequence. The result does
 * not depend on the split choice beyond fp32 rounding.
 *
 * Cache reads: when the K and V bytes a call can touch (every page its block
 * table can name, or its window) exceed 256 MB, more than MI355X's last-level
 * cache holds, the matrix kernel reads them with non-temporal loads; below
 * that, with ordinary loads, so that repeated calls find them in that cache.
 * The values read, and the result, are the same either way.
 */
pda_status pda_paged_decode_attention(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_lens,
    float scale, int32_t window, int32_t num_splits, void* out,
    const float* k_scale, const float* v_scale, const pda_decode_dims* dims,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The two launches of pda_paged_decode_attention, one call each, for callers
 * that time them apart or put other work between them. Called in this
 * order, on one stream, with the same arguments and the same workspace, they
 * do exactly what pda_paged_decode_attention does. The decode stage writes
 * `out` for rows it finishes alone and the workspace for the rest; the
 * combine stage merges the workspace into `out` (it launches nothing when
 * the call has one split). Between them the workspace layout is private to
 * the library.
 */
pda_status pda_attention_decode_stage(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_lens,
    float scale, int32_t window, int32_t num_splits, void* out,
    const float* k_scale, const float* v_scale, const pda_decode_dims* dims,
    void* workspace, size_t workspace_bytes, hipStream_t stream);
pda_status pda_attention_combine_stage(
    void* out, const pda_decode_dims* dims, int32_t window, int32_t num_splits,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The decode stage alone: writes the per-split partials of every row into
 * `workspace` (always, also for one split) and launches nothing else.
 * Arguments as for pda_paged_decode_attention, without `out`; `num_splits`
 * 0 resolves to pda_decode_resolve_splits's count (one count for every
 * sequence: no balancing). Partials layout, with S the resolved split count:
 *
 *   partial_o  = (float*)workspace                       [T, Hq, S, D]
 *   partial_ml = (float*)workspace + T * Hq * S * D      [T, Hq, S, 2]
 *
 * For split s of row (t, h): m = partial_ml[..., 0] is the largest score of
 * the split in base-2 units (scale * log2(e) * q.k), l = partial_ml[..., 1]
 * = sum of 2^(score - m) over the split's visible keys, and partial_o =
 * sum of 2^(score - m) * v (unnormalized, v dequantized). A split that sees
 * no key has m = -inf, l = 0, o = 0.
 */
pda_status pda_paged_decode_partials(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_lens,
    float scale, int32_t window, int32_t num_splits,
    const float* k_scale, const float* v_scale, const pda_decode_dims* dims,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Split-K combine: out[t, h, :] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
 * with M the largest m_s over splits with l_s > 0; a row whose splits are all
 * empty is written as zeros. partial_o / partial_ml as laid out above
 * (num_splits >= 1); out fp16 [T, Hq, D]. One launch on `stream`.
 */
pda_status pda_split_combine(const float* partial_o, const float* partial_ml,
                             void* out, int32_t num_tokens, int32_t num_q_heads,
                             int32_t head_dim, int32_t num_splits,
                             hipStream_t stream);

/*
 * The one-call path without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Arguments and results as for
 * pda_paged_decode_attention, which it runs; the split partials and chunk
 * lists go to a scratch array of PDA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on, from load until the process ends. It
 * calls no allocator. A call needing more workspace than that
 * (pda_decode_workspace_bytes) returns PDA_ERR_WORKSPACE before any launch.
 * Every call on a device shares that device's array: calls that overlap on
 * one device (two streams, or two host threads) race, and must be ordered by
 * the caller. Nothing in the array needs clearing between calls (each call
 * writes what it reads).
 */
#define PDA_NOALLOC_SCRATCH_BYTES (64u << 20)
pda_status pda_paged_decode_attention_noalloc(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_lens,
    float scale, int32_t window, int32_t num_splits, void* out,
    const float* k_scale, const float* v_scale, const pda_decode_dims* dims,
    hipStream_t stream);
/* Bytes of the scratch array of pda_paged_decode_attention_noalloc. */
size_t pda_noalloc_scratch_bytes(void);

/* Sizes of a cache write. */
typedef struct pda_cache_dims {
  int32_t num_tokens;   /* T: rows of key / value (0: nothing to do) */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* D: a multiple of 8 */
  int32_t page_size;    /* P >= 1 */
  int32_t num_pages;    /* pages in each cache; num_pages * P must fit in int32 */
  int32_t kv_dtype;     /* a pda_kv_dtype: the element type of both caches */
  int32_t kv_layout;    /* a pda_kv_layout */
} pda_cache_dims;

/*
 * KV-cache writer: stores the K and V rows of T new tokens in the paged
 * caches, in the layout the decode entry points read (the cache writer's
 * layout that PR #33's "Test Plan" checks the decode against; fp8 and int8
 * caches as in its "Purpose" section).
 *
 *  key, value    fp16 [T, Hkv, D], 16-byte aligned.
 *  slot_mapping  int32 [T]: token t goes to slot s = page * P + position,
 *                i.e. rows [s / P, s % P, :, :] (NHD) or [s / P, :, s % P, :]
 *                (HND) of each cache. Tokens with s < 0 (padding) or
 *                s >= num_pages * P are not written.
 *  k_cache       [num_pages, P, Hkv, D] (NHD) or [num_pages, Hkv, P, D] (HND)
 *                of kv_dtype, written in place; only
 *  v_cache       the rows of written slots change. 16-byte aligned (fp16) or
 *                8-byte aligned (fp8 / int8).
 *  k_scale       fp32 [Hkv] for fp8 / int8 caches (NULL for fp16).
 *  v_scale
 *
 * fp16 caches store the values unchanged. A quantized code is q = x / scale
 * (fp32, IEEE division), clamped to the largest finite magnitude (448 for
 * e4m3fn, 127 for int8; -128 is never written) and rounded to the nearest
 * code, ties to even. Inputs must be finite. Two tokens mapped to the same
 * slot race (either may win). One launch on `stream`.
 */
pda_status pda_write_kv_cache(const void* key, const void* value,
                              const int32_t* slot_mapping, void* k_cache,
                              void* v_cache, const float* k_scale,
                              const float* v_scale, const pda_cache_dims* dims,
                              hipStream_t stream);

/* Split count of a call with one count for every sequence: `num_splits`
 * itself when it is >= 1, otherwise the automatic choice for a device with
 * `num_cus` compute units (num_cus <= 0: the current device's count), which
 * pda_paged_decode_partials uses (pda_paged_decode_attention may balance
 * counts per sequence instead). Host-only; no launch. Returns a value in
 * 1..PDA_MAX_SPLITS, or a negative pda_status. */
int32_t pda_decode_resolve_splits(const pda_decode_dims* dims, int32_t window,
                                  int32_t num_splits, int32_t num_cus);

/* Workspace bytes pda_paged_decode_attention (and its two stages) needs
 * for these arguments on the current device (0 for one split);
 * pda_paged_decode_partials needs pda_decode_partials_bytes, with the split
 * count resolved as above. Host-only. Negative on invalid sizes. */
int64_t pda_decode_workspace_bytes(const pda_decode_dims* dims, int32_t window,
                                   int32_t num_splits);
int64_t pda_decode_partials_bytes(const pda_decode_dims* dims, int32_t window,
                                  int32_t num_splits);

/*
 * Measurement aid (not part of the attention path): reads `bytes` of device
 * memory at `src` (both multiples of 16) once, as fast as one launch of
 * `workgroups` workgroups of 256 threads can (16-byte non-temporal loads in
 * a grid-stride loop), and writes one XOR word per workgroup to `sink`
 * (uint32 [workgroups], device memory). Timed over a buffer larger than the
 * on-package caches, it gives the streaming-read rate of this device's HBM,
 * the practical roof of the decode kernels. One launch on `stream`.
 */
pda_status pda_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink,
                              int32_t workgroups, hipStream_t stream);

/* Message of the calling thread's last non-OK status ("" if none). */
const char* pda_last_error(void);

/* Library version string. */
const char* pda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PDA_H_ */
