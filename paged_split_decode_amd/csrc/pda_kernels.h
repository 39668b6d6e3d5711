// Internal interface between the host layer (pda_api.hip) and the gfx950
// kernels (pda_decode_*.hip, pda_combine.hip). Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pda {

enum KvKind : int { kKvF16 = 0, kKvFp8 = 1, kKvI8 = 2 };

constexpr int kPageSize = 16;     // keys per tile: the page size of the vector
                                  // kernel; the matrix kernel takes pages of
                                  // 16 * 2^k keys as runs of such tiles
constexpr int kLanesPerKey = 16;  // lanes sharing one key row in a wave

// Query rows per wave (RW) of the vector kernel that are compiled: those whose
// working set stays in registers (no scratch in the compiler's resource
// report). fp16 at D=128 skips RW = 2, for which the compiler keeps part of
// the load ring in scratch memory; a call with 2 rows per wave runs RW = 3
// with one padding row. More rows than the largest RW take several row
// groups (waves that share keys).
constexpr bool vector_rw_compiled(int head_dim, int kv_kind, int rw) {
  if (rw < 1) return false;
  if (head_dim == 128) return kv_kind == kKvF16 ? (rw <= 5 && rw != 2) : rw <= 6;
  return kv_kind == kKvI8 ? rw <= 3 : rw <= 4;
}
constexpr int vector_max_rw(int head_dim, int kv_kind) {
  int r = 1;
  for (int k = 1; k <= 8; ++k)
    if (vector_rw_compiled(head_dim, kv_kind, k)) r = k;
  return r;
}
// Smallest compiled RW >= rw (rw <= vector_max_rw).
constexpr int vector_rw_for(int head_dim, int kv_kind, int rw) {
  for (int k = rw; k <= 8; ++k)
    if (vector_rw_compiled(head_dim, kv_kind, k)) return k;
  return -1;
}

// Keys one pipeline unit of a wave covers: 4 keys per wave instruction
// (64 lanes / 16 lanes per key) times the key iterations per unit. A unit
// keeps at most 32 dwords of K+V per lane in flight.
constexpr int key_iters(int head_dim, int kv_kind) {
  return (kv_kind == kKvF16 && head_dim == 256) ? 2 : 4;
}
constexpr int unit_keys(int head_dim, int kv_kind) {
  return 4 * key_iters(head_dim, kv_kind);
}

struct DecodeArgs {
  const uint8_t* q;       // fp16 [T, Hq, D]
  const uint8_t* k;       // [num_pages, P, Hkv, D] elements
  const uint8_t* v;
  const int32_t* block_table;  // [B, max_pages]
  const int32_t* seq_lens;     // [B]
  const int32_t* q_lens;       // [B] or nullptr
  const float* k_scale;        // [Hkv] or nullptr
  const float* v_scale;        // [Hkv] or nullptr
  uint16_t* out;               // fp16 [T, Hq, D] (direct mode)
  float* part_o;               // [T, Hq, S, D]   (partials mode)
  float* part_ml;              // [T, Hq, S, 2]
  float qk_mult;               // scale * log2(e)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;               // G = Hq / Hkv
  int32_t max_pages;
  int32_t max_q_len;
  int32_t window;
  int32_t num_splits;
  int32_t row_groups;          // waves of a workgroup sharing keys, split by rows
  int32_t key_waves;           // waves sharing one KV head's key range
  int32_t heads_per_group;     // KV heads per workgroup (matrix kernel)
  int32_t direct;              // 1: write out (one split); 0: write partials
  int32_t batch;               // B
  int32_t longest_first;       // matrix kernel: grid row z takes the z-th longest
                               // sequence (needs B <= 64)
  uint32_t key_stride;         // matrix kernel: bytes between slots of one head
  uint32_t head_stride;        // matrix kernel: bytes between heads within a page
  uint64_t page_bytes;         // matrix kernel: bytes of one page (all heads)
  int32_t tile_shift;          // matrix kernel: log2(page_size / 16)
  int32_t rows;                // G * max_q_len (matrix kernel)
  int32_t wave_lds_bytes;      // LDS bytes per wave (matrix kernel)
  // Length-balanced splits (matrix kernel, automatic split count): grid x
  // has `chunks` slots per KV-head group, filled by the chunks of every
  // sequence (see balanced_chunk); partials go to per-chunk records and
  // `meta` gets, per token, {first chunk slot, chunk count, token index in
  // its sequence, 0}.
  int32_t balanced;
  int32_t chunks;
  int32_t min_chunk;           // fewest 16-key tiles in a chunk
  int32_t* meta;               // [T][4]
  // Prefill kernel: token blocks per (sequence, KV head), and items (token
  // blocks x KV heads x sequences) shared by its workgroups.
  int32_t prefill_blocks;
  int32_t prefill_items;
};

// Launch the decode kernel for (head_dim, kv_kind, rows_per_wave) with
// grid (num_splits, Hkv, B) and row_groups * key_waves waves per workgroup.
// Returns hipErrorInvalidValue when no instantiation covers the request.
hipError_t launch_decode_f16(int head_dim, int rows_per_wave, dim3 grid,
                             int threads, size_t lds, hipStream_t stream,
                             const DecodeArgs& args);
hipError_t launch_decode_fp8(int head_dim, int rows_per_wave, dim3 grid,
                             int threads, size_t lds, hipStream_t stream,
                             const DecodeArgs& args);
hipError_t launch_decode_i8(int head_dim, int rows_per_wave, dim3 grid,
                            int threads, size_t lds, hipStream_t stream,
                            const DecodeArgs& args);

// Matrix-core (MFMA) decode kernel for (head_dim, kv_kind, row_tiles of 16
// query rows), grid (num_splits, Hkv, B), `threads` / 64 waves per workgroup;
// stream_kv: K and V by non-temporal loads.
hipError_t launch_decode_mfma_f16(int head_dim, int row_tiles, bool stream_kv, dim3 grid, int threads,
                                  size_t lds, hipStream_t stream, const DecodeArgs& args);
hipError_t launch_decode_mfma_fp8(int head_dim, int row_tiles, bool stream_kv, dim3 grid, int threads,
                                  size_t lds, hipStream_t stream, const DecodeArgs& args);
hipError_t launch_decode_mfma_i8(int head_dim, int row_tiles, bool stream_kv, dim3 grid, int threads,
                                 size_t lds, hipStream_t stream, const DecodeArgs& args);
// Waves per SIMD the matrix kernel's register allocation leaves room for:
// two wherever the working set fits in 256 registers (a second wave hides the
// first one's memory and MFMA latency); one for fp16 at D=256 (its K+V ring
// alone is 128 registers) and for two row tiles except with 1-byte KV at
// D=128 (fp16 two row tiles at D=128 at two waves, with a 2-page ring, ran
// the ragged multi-token verify batch in 249 us per call against 234 with
// automatic splits, and equal with 8). A workgroup holds at most 4 x this
// many waves.
constexpr int mfma_waves_per_simd(int head_dim, int kv_kind, int row_tiles) {
  if (row_tiles == 1) return (head_dim == 256 && kv_kind == kKvF16) ? 1 : 2;
  return (head_dim == 128 && kv_kind != kKvF16) ? 2 : 1;
}

// LDS bytes one wave of the matrix kernel needs: its fp16 V tile (16 rows of
// D + 16 halves) during the loop, then its merge records (per row: m, l, two
// pad floats, o[D]); the two uses alias. Rounded up to 256 bytes.
inline size_t mfma_wave_lds_bytes(int head_dim, int rows) {
  const size_t tile = (size_t)16 * (head_dim + 16) * 2;
  const size_t merge = (size_t)rows * (head_dim + 4) * 4;
  const size_t bytes = tile > merge ? tile : merge;
  return (bytes + 255) & ~(size_t)255;
}

// Bytes of dynamic LDS the decode kernel needs for the final merge.
inline size_t decode_lds_bytes(int waves, int rows_per_wave, int head_dim) {
  return (size_t)waves * rows_per_wave * (head_dim + 2) * sizeof(float);
}

// Long-query (prefill) kernel: 32 (token, head) rows per wave; K and V go
// through LDS 64 keys (four 16-key tiles) per step, as fp16 in the order the
// matrix instructions read them. A workgroup has 8 waves at D=128 when the
// keys before the new tokens are long (at least 3 times as many as the new
// tokens, from the table's capacity) or a KV head has at least 512 query
// rows: a staged key then serves twice the rows (with the token blocks of a
// sequence on one XCD, 8-wave workgroups measured 3.7% faster than two 4-wave
// ones per CU on a fresh prefill of 4 x 2048 tokens). Fewer rows take 4 waves
// (128 rows per workgroup). At D=256 a workgroup has 8 waves in pairs that
// share 32 rows, split the scores by key half (exchanged through LDS) and
// the output by dims (128 rows per workgroup).
inline int prefill_waves(int head_dim, int max_q_len, int64_t key_capacity, int group) {
  if (head_dim == 256) return 8;
  return (4 * (int64_t)max_q_len <= key_capacity || (int64_t)group * max_q_len >= 512) ? 8 : 4;
}
constexpr int prefill_tiles(int) { return 4; }  // 64 keys per LDS step (two halves of 32)
// Bytes of one step of K and V in LDS (fp16, unpadded).
constexpr int prefill_step_bytes(int head_dim) {
  return 2 * prefill_tiles(head_dim) * 16 * head_dim * 2;
}
// Step buffers in LDS: fp16 caches load straight into LDS, three steps deep
// for 8-wave workgroups at D=128 (96 KB, one workgroup per CU) and two
// otherwise (64 KB at D=128: two 4-wave workgroups per CU; 128 KB at D=256,
// plus 32 KB for the pairs' score exchange);
// 1-byte codes are converted in registers and stored into two buffers.
#ifndef PDA_PREFILL_NBUF8
#define PDA_PREFILL_NBUF8 3
#endif
constexpr int prefill_buffers(int head_dim, int kv_kind, int waves) {
  return kv_kind == kKvF16 && head_dim == 128 && waves == 8 ? PDA_PREFILL_NBUF8 : 2;
}
// LDS the output tiles take after the loop: 32 rows per wave of the dims it
// writes (half of D in the 8-wave D=256 pairs), unpadded (the 16-byte pieces
// of a row are stored in an order that depends on the row).
constexpr size_t prefill_out_lds_bytes(int head_dim, int waves) {
  return (size_t)waves * 32 * 2 * ((head_dim == 256 && waves == 8) ? head_dim / 2 : head_dim);
}
// The score exchange of the D=256 pairs: 16 floats per lane and wave.
constexpr size_t prefill_xchg_bytes(int head_dim, int waves) {
  return head_dim == 256 && waves == 8 ? (size_t)waves * 64 * 16 * 4 : 0;
}
// fp16 KV stages Q through LDS: at D=128 with 8 waves in 64 KB of its own
// after the three step buffers (160 KB in all; the output tiles go there
// too), else in step buffer 1.
constexpr bool prefill_q_own(int head_dim, int kv_kind, int waves) {
  return kv_kind == kKvF16 && head_dim == 128 && waves == 8 && prefill_buffers(head_dim, kv_kind, waves) == 3;
}
constexpr size_t prefill_lds_bytes(int head_dim, int kv_kind, int waves) {
  const size_t steps = (size_t)prefill_buffers(head_dim, kv_kind, waves) * prefill_step_bytes(head_dim) +
                       prefill_xchg_bytes(head_dim, waves);
  const size_t out = prefill_out_lds_bytes(head_dim, waves);
  return prefill_q_own(head_dim, kv_kind, waves) ? steps + out : (steps > out ? steps : out);
}
hipError_t launch_prefill_f16(int head_dim, int waves, dim3 items, int cus, size_t lds, hipStream_t stream,
                              const DecodeArgs& args);
hipError_t launch_prefill_fp8(int head_dim, int waves, dim3 items, int cus, size_t lds, hipStream_t stream,
                              const DecodeArgs& args);
hipError_t launch_prefill_i8(int head_dim, int waves, dim3 items, int cus, size_t lds, hipStream_t stream,
                             const DecodeArgs& args);

// Host-side error state shared by every entry point: records a message for
// pda_last_error() and returns `status`.
int host_fail(int status, const char* fmt, ...);
const char* host_last_error();

// Slices of the head dim the combine cuts each row into (1, 2 or 4, at
// least 64 dims each) so that rows x slices workgroups cover the compute
// units when there are few rows.
int combine_dim_parts(int rows, int head_dim, int num_cus);

// Where the combine finds a row's partials. Fixed split count (meta ==
// nullptr): row r's split s is record r * num_splits + s. Balanced splits:
// row (t, h) of KV head k = h / group has meta[t] = {first chunk slot P,
// chunk count n, token index i, 0}; its split s is record
// (k * rows + i * group + h % group) * chunks + P + s, and a row with n <= 1
// was written by the decode kernel itself. Record e holds o at part_o + e * D
// and (m, l) at part_ml + 2 e.
struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  uint16_t* out;
  const int32_t* meta;
  int32_t num_splits;
  int32_t num_q_heads;
  int32_t group;
  int32_t rows;
  int32_t chunks;
  int32_t per_seq;    // balanced: chunk slots per sequence (chunks / B)
  int32_t max_q_len;  // balanced: tokens per sequence of a uniform batch
};

// Waves per combine workgroup for a fixed split count: one per 16 splits.
inline int combine_waves(int num_splits) { return (num_splits + 15) / 16; }

hipError_t launch_combine(const CombineArgs& args, int rows, int head_dim, int waves,
                          int dim_parts, hipStream_t stream);

}  // namespace pda
