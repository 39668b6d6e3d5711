// Host layer of the C ABI declared in include/pda.h: argument validation,
// split-count policy, launch shape, and the launches themselves on the
// caller's stream. No allocation, no synchronization, no device state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "pda.h"
#include "pda_kernels.h"

namespace pda {

namespace {
thread_local std::string g_last_error;
}  // namespace

int host_fail(int st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

const char* host_last_error() { return g_last_error.c_str(); }

}  // namespace pda

namespace {

template <typename... Args>
pda_status fail(pda_status st, const char* fmt, Args... args) {
  return static_cast<pda_status>(pda::host_fail(st, fmt, args...));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device, queried once per device.
int device_cu_count() {
  static std::mutex mu;
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if (counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return -1;
    counts[dev] = n;
  }
  return counts[dev];
}

int kv_kind(int32_t kv_dtype) {
  switch (kv_dtype) {
    case PDA_KV_F16: return pda::kKvF16;
    case PDA_KV_FP8_E4M3: return pda::kKvFp8;
    case PDA_KV_INT8: return pda::kKvI8;
    default: return -1;
  }
}

// Launch shape for one call.
struct Plan {
  int prefill;     // 1: long-query kernel (one split, direct output)
  int matrix;      // 1: MFMA kernel, 0: v_dot2 kernel
  int row_tiles;   // MFMA kernel: 16-row tiles
  size_t wave_lds; // MFMA kernel: LDS bytes per wave
  int rows;        // G * max_q_len query rows per (sequence, KV head)
  int rows_per_wave;
  int row_groups;
  int key_waves;       // waves per KV head (matrix) / per key range (v_dot2)
  int heads_per_group; // matrix kernel: KV heads per workgroup
  int head_groups;     // grid y: workgroups across the KV heads
  int longest_first;   // matrix kernel: order grid rows by sequence length
  int balanced;        // matrix kernel: per-sequence split counts on the device
  int chunks;          // balanced: chunk slots per KV-head group (grid x)
  int min_chunk;       // balanced: fewest 16-key tiles per chunk
  int combine_waves;   // balanced: waves per combine workgroup
  int splits;
  int threads;
  size_t lds;
  int stream_kv;       // matrix kernel: K and V by non-temporal loads
};

pda_status check_dims(const pda_decode_dims* d) {
  if (!d) return fail(PDA_ERR_NULL, "dims is NULL");
  if (d->batch < 0 || d->num_tokens < 0)
    return fail(PDA_ERR_SHAPE, "batch (%d) and num_tokens (%d) must be >= 0", d->batch,
                d->num_tokens);
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads)
    return fail(PDA_ERR_SHAPE, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  if (d->head_dim != 128 && d->head_dim != 256)
    return fail(PDA_ERR_UNSUPPORTED, "head_dim %d: compiled for 128 and 256", d->head_dim);
  if (d->page_size < pda::kPageSize || d->page_size > 256 ||
      (d->page_size & (d->page_size - 1)))
    return fail(PDA_ERR_UNSUPPORTED, "page_size %d: 16, 32, 64, 128 or 256", d->page_size);
  if (d->kv_layout != PDA_LAYOUT_NHD && d->kv_layout != PDA_LAYOUT_HND)
    return fail(PDA_ERR_UNSUPPORTED, "kv_layout %d is not a pda_kv_layout", d->kv_layout);
  if (d->kernel == PDA_KERNEL_VECTOR &&
      (d->page_size != pda::kPageSize || d->kv_layout != PDA_LAYOUT_NHD))
    return fail(PDA_ERR_UNSUPPORTED, "the vector kernel reads 16-key pages in the NHD layout");
  if (d->num_pages <= 0 || d->max_pages_per_seq <= 0)
    return fail(PDA_ERR_SHAPE, "num_pages (%d) and max_pages_per_seq (%d) must be > 0",
                d->num_pages, d->max_pages_per_seq);
  if (d->max_q_len < 1) return fail(PDA_ERR_SHAPE, "max_q_len %d must be >= 1", d->max_q_len);
  if (kv_kind(d->kv_dtype) < 0)
    return fail(PDA_ERR_UNSUPPORTED, "kv_dtype %d is not a pda_kv_dtype", d->kv_dtype);
  if (d->kernel < PDA_KERNEL_AUTO || d->kernel > PDA_KERNEL_PREFILL)
    return fail(PDA_ERR_UNSUPPORTED, "kernel %d is not a pda_kernel", d->kernel);
  const int64_t rows = (int64_t)(d->num_q_heads / d->num_kv_heads) * d->max_q_len;
  if (rows > PDA_MAX_ROWS && (d->kernel == PDA_KERNEL_VECTOR || d->kernel == PDA_KERNEL_MATRIX))
    return fail(PDA_ERR_UNSUPPORTED,
                "(num_q_heads/num_kv_heads)*max_q_len = %lld exceeds %d for the decode kernels",
                (long long)rows, PDA_MAX_ROWS);
  if (d->num_q_heads / d->num_kv_heads > PDA_MAX_GROUP)
    return fail(PDA_ERR_UNSUPPORTED, "num_q_heads/num_kv_heads exceeds %d", PDA_MAX_GROUP);
  if ((int64_t)d->max_pages_per_seq * d->page_size > INT32_MAX / 2)
    return fail(PDA_ERR_SHAPE, "max_pages_per_seq * page_size too large");
  if ((int64_t)d->page_size * d->num_kv_heads * d->head_dim * 2 >= ((int64_t)1 << 31))
    return fail(PDA_ERR_SHAPE, "one page (page_size * num_kv_heads * head_dim) must be < 2 GiB");
  return PDA_OK;
}

// Waves of a vector-kernel workgroup (its launch bound: 512 threads).
constexpr int kVectorMaxWaves = 8;

// Splits for the v_dot2 kernel: about one workgroup per compute unit.
int auto_splits(const pda_decode_dims* d, int window, int uk, int key_waves, int num_cus) {
  int64_t keys = (int64_t)d->max_pages_per_seq * d->page_size;
  if (window > 0) keys = std::min<int64_t>(keys, (int64_t)window + d->max_q_len - 1 + uk);
  const int64_t units = (keys + uk - 1) / uk;
  const int64_t work = std::max<int64_t>(1, (int64_t)d->batch * d->num_kv_heads);
  const int64_t target = (int64_t)num_cus;
  int64_t s = (target + work - 1) / work;
  s = std::min<int64_t>(s, std::max<int64_t>(1, units / (2 * key_waves)));
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, PDA_MAX_SPLITS));
}

// 16-key tiles a call's longest sequence can have visible.
int64_t visible_tiles(const pda_decode_dims* d, int window) {
  int64_t keys = (int64_t)d->max_pages_per_seq * d->page_size;
  if (window > 0)
    keys = std::min<int64_t>(keys, (int64_t)window + d->max_q_len - 1 + pda::kPageSize);
  return (keys + pda::kPageSize - 1) / pda::kPageSize;
}

// Workgroup shape and split count of the matrix kernel.
//  * Automatic splits with length balancing (allowed for the one-call path):
//    the grid has as many chunk slots as workgroups fit at once, and the
//    kernel cuts every sequence into chunks of one common size, so each
//    workgroup gets about the same number of pages however ragged the batch
//    is (a fixed split count per sequence leaves the compute units that hold
//    the longest sequences working alone at the end). Used while the batch
//    is smaller than the slot count; a uniform batch gets the same chunks as
//    a fixed count would give it.
//  * Up to 4 KV heads share a workgroup, one wave each: the heads of a page
//    block (contiguous in the pool) are then fetched together, which measures
//    faster than one head per workgroup. Fewer heads leave room for several
//    waves per head (key_waves), to keep 4-wave workgroups.
//  * Automatic splits: enough workgroups to fill every SIMD's wave slots once
//    (all workgroups resident together), each wave keeping at least 2 pages.
//  * A caller's split count: the head group shrinks until the workgroups
//    cover every compute unit, and key_waves grows to fill the wave slots.
void matrix_plan(const pda_decode_dims* d, int window, int num_splits, int num_cus,
                 int waves_per_simd, int max_waves, bool allow_balanced, Plan* p) {
  const int64_t pages = visible_tiles(d, window);  // in 16-key tiles
  const int64_t B = std::max(1, d->batch);
  const int Hkv = d->num_kv_heads;
  auto groups = [&](int h) { return (int64_t)((Hkv + h - 1) / h); };
  int hpw = std::min({Hkv, 4, max_waves});
  int kw = std::max(1, std::min(4, max_waves) / hpw);
  int64_t S;
  if (num_splits < 1) {
    // Fill every SIMD's wave slots once, never a second round. (At two
    // waves per SIMD the second workgroup per CU hides the first one's
    // latency: the headline shape decodes in 27.3 us at 32 splits against
    // 30.0 us at 16, more than the combine saves.)
    S = (int64_t)num_cus * waves_per_simd / (B * groups(hpw));
    S = std::min<int64_t>(S, std::max<int64_t>(1, pages / (2 * kw)));
    S = std::max<int64_t>(1, std::min<int64_t>(S, PDA_MAX_SPLITS));
  } else {
    S = num_splits;
  }
  // Workgroup shape for S splits per sequence: the head group shrinks until
  // the workgroups cover every compute unit, and key_waves grows to fill the
  // wave slots.
  hpw = std::min({Hkv, 4, max_waves});
  while (hpw > 1 && S * B * groups(hpw) < num_cus) hpw = (hpw + 1) / 2;
  const int64_t slots = (int64_t)num_cus * 4 * waves_per_simd;
  const int64_t want = slots / (S * B * groups(hpw) * hpw);
  const int64_t by_pages = std::max<int64_t>(1, pages / (2 * S));
  kw = (int)std::max<int64_t>(1, std::min<int64_t>({want, max_waves / hpw, by_pages}));
  p->heads_per_group = hpw;
  p->key_waves = kw;
  p->head_groups = (int)groups(hpw);
  p->splits = (int)S;
  p->balanced = 0;
  p->chunks = 0;
  p->min_chunk = 0;
  p->combine_waves = 0;
  // With more workgroups than fit at once, dispatch the longest sequences
  // first (ragged batches then finish together); with one round the order
  // cannot matter.
  const int64_t wgs = S * B * groups(hpw);
  const int64_t wg_fit = (int64_t)num_cus * std::max(1, 4 * waves_per_simd / (hpw * kw));
  p->longest_first = d->batch <= 64 && wgs > wg_fit;
  // Automatic splits, balanced: the same workgroups (S per sequence on
  // average), cut by length on the device.
  if (num_splits < 1 && allow_balanced && S >= 2 && d->batch < 256) {
    p->balanced = 1;
    p->chunks = (int)(S * B);
    p->min_chunk = 2 * kw;
    // Waves of a combine workgroup: one per 16 splits of a uniform batch's
    // row; the longer rows of a ragged batch take more passes.
    p->combine_waves = (int)((S + 15) / 16);
    p->longest_first = 0;
  }
}

// The most K and V bytes a call can read: every sequence at the table's
// capacity, or its window. Above the last-level cache (256 MB of Infinity
// Cache on MI355X) the matrix kernel streams K and V with non-temporal loads
// (measured 8-10% faster on 0.5-4.3 GB calls); below it, repeated calls over
// the same cache find K and V there, which ordinary loads keep (the
// non-temporal ones measured up to 19% slower on calls of 17-134 MB).
constexpr int64_t kStreamKvBytes = (int64_t)256 << 20;
int64_t kv_bytes_bound(const pda_decode_dims* d, int window) {
  const int64_t elem = d->kv_dtype == PDA_KV_F16 ? 2 : 1;
  return visible_tiles(d, window) * pda::kPageSize * d->batch * d->num_kv_heads * d->head_dim * elem * 2;
}

pda_status make_plan(const pda_decode_dims* d, int32_t window, int32_t num_splits, int num_cus,
                     Plan* p, bool allow_balanced = false) {
  pda_status st = check_dims(d);
  if (st != PDA_OK) return st;
  *p = Plan{};
  if (num_splits < 0 || num_splits > PDA_MAX_SPLITS)
    return fail(PDA_ERR_SHAPE, "num_splits %d outside 0..%d", num_splits, PDA_MAX_SPLITS);
  p->rows = (d->num_q_heads / d->num_kv_heads) * d->max_q_len;
  p->prefill = d->kernel == PDA_KERNEL_PREFILL ||
               (d->kernel == PDA_KERNEL_AUTO && p->rows > PDA_MAX_ROWS);
  if (p->prefill) {
    if (num_splits > 1)
      return fail(PDA_ERR_UNSUPPORTED, "the prefill kernel runs one split (num_splits 0 or 1)");
    const int G = d->num_q_heads / d->num_kv_heads;
    const int waves = pda::prefill_waves(d->head_dim, d->max_q_len,
                                         (int64_t)d->max_pages_per_seq * d->page_size, G);
    const int bq = 32 * (d->head_dim == 256 ? waves / 2 : waves) / G;  // tokens per workgroup
    p->rows = bq * G;                      // rows per workgroup
    p->row_tiles = (d->max_q_len + bq - 1) / bq;  // grid x: token blocks
    p->matrix = 1;
    p->splits = 1;
    p->threads = 64 * waves;
    p->lds = pda::prefill_lds_bytes(d->head_dim, kv_kind(d->kv_dtype), waves);
    p->wave_lds = 0;
    p->rows_per_wave = 32;
    p->row_groups = 4;
    p->key_waves = 1;
    p->heads_per_group = 1;
    p->head_groups = d->num_kv_heads;
    p->longest_first = 0;
    p->balanced = 0;
    return PDA_OK;
  }
  // The matrix-core kernel is faster on every measured shape; the v_dot2
  // kernel stays selectable.
  p->matrix = d->kernel != PDA_KERNEL_VECTOR;
  if (num_cus <= 0 && (p->matrix || num_splits < 1)) num_cus = device_cu_count();
  if (num_cus <= 0 && (p->matrix || num_splits < 1))
    return fail(PDA_ERR_DEVICE, "cannot query the device's compute units");
  if (p->matrix) {
    p->row_tiles = (p->rows + 15) / 16;
    p->wave_lds = pda::mfma_wave_lds_bytes(d->head_dim, p->rows);
    const int waves_per_simd =
        pda::mfma_waves_per_simd(d->head_dim, kv_kind(d->kv_dtype), p->row_tiles);
    const int lds_waves = (int)std::max<size_t>(1, 65536 / p->wave_lds);
    matrix_plan(d, window, num_splits, num_cus, waves_per_simd,
                std::min(4 * waves_per_simd, lds_waves), allow_balanced, p);
    const int waves = p->heads_per_group * p->key_waves;
    p->row_groups = 1;
    p->rows_per_wave = p->rows;
    p->threads = 64 * waves;
    p->lds = (size_t)waves * p->wave_lds;  // V tiles, then merge records
    p->stream_kv = kv_bytes_bound(d, window) > kStreamKvBytes;
    return PDA_OK;
  }
  // Rows per wave: at most the largest compiled count, rounded up to a
  // compiled one (the extra rows are padding: their tokens do not exist).
  const int kk = kv_kind(d->kv_dtype);
  const int cap = pda::vector_max_rw(d->head_dim, kk);
  p->row_groups = (p->rows + cap - 1) / cap;
  p->rows_per_wave =
      pda::vector_rw_for(d->head_dim, kk, (p->rows + p->row_groups - 1) / p->row_groups);
  if (p->row_groups > kVectorMaxWaves)
    return fail(PDA_ERR_UNSUPPORTED,
                "the vector kernel takes at most %d query rows per KV head with this head_dim "
                "and kv_dtype ((num_q_heads/num_kv_heads)*max_q_len = %d); use the matrix kernel",
                kVectorMaxWaves * cap, p->rows);
  p->key_waves = std::max(1, (4 + p->row_groups - 1) / p->row_groups);
  if (p->row_groups >= 4) p->key_waves = 1;
  const int waves = p->row_groups * p->key_waves;
  p->threads = 64 * waves;
  p->lds = pda::decode_lds_bytes(waves, p->rows_per_wave, d->head_dim);
  p->row_tiles = 0;
  p->wave_lds = 0;
  p->heads_per_group = 1;
  p->head_groups = d->num_kv_heads;
  p->longest_first = 0;
  p->balanced = 0;
  p->splits = num_splits >= 1
                  ? num_splits
                  : auto_splits(d, window, pda::unit_keys(d->head_dim, kv_kind(d->kv_dtype)),
                                p->key_waves, num_cus);
  return PDA_OK;
}

// Whether a (valid) call runs the long-query kernel.
bool routes_to_prefill(const pda_decode_dims* d) {
  const int64_t rows = (int64_t)(d->num_q_heads / d->num_kv_heads) * d->max_q_len;
  return d->kernel == PDA_KERNEL_PREFILL || (d->kernel == PDA_KERNEL_AUTO && rows > PDA_MAX_ROWS);
}

// The split count alone (for size queries): a caller's count needs no device.
pda_status resolve_split_count(const pda_decode_dims* d, int32_t window, int32_t num_splits,
                               int num_cus, int* splits) {
  pda_status st = check_dims(d);
  if (st != PDA_OK) return st;
  if (routes_to_prefill(d)) {
    if (num_splits > 1)
      return fail(PDA_ERR_UNSUPPORTED, "the prefill kernel runs one split (num_splits 0 or 1)");
    *splits = 1;
    return PDA_OK;
  }
  if (num_splits >= 1 && num_splits <= PDA_MAX_SPLITS) {
    *splits = num_splits;
    return PDA_OK;
  }
  Plan p;
  if ((st = make_plan(d, window, num_splits, num_cus, &p))) return st;
  *splits = p.splits;
  return PDA_OK;
}

int64_t partials_bytes(const pda_decode_dims* d, int splits) {
  return (int64_t)d->num_tokens * d->num_q_heads * splits * (d->head_dim + 2) *
         (int64_t)sizeof(float);
}

// Workspace of the one-call path. Fixed split count: the partials as laid
// out for pda_paged_decode_partials (none for one split). Balanced splits:
// records [KV head][G * max_q_len rows][chunk slot] (o, then (m, l) padded
// to 16 bytes), then the per-token chunk lists.
struct WsLayout {
  int64_t ml;    // byte offset of the (m, l) records
  int64_t meta;  // byte offset of the chunk lists (balanced)
  int64_t total;
};

WsLayout fixed_ws_layout(const pda_decode_dims* d, int splits) {
  WsLayout w{0, 0, 0};
  if (splits > 1) {
    w.ml = (int64_t)d->num_tokens * d->num_q_heads * splits * d->head_dim * 4;
    w.total = partials_bytes(d, splits);
  }
  return w;
}

WsLayout attention_ws_layout(const pda_decode_dims* d, const Plan& p) {
  WsLayout w{0, 0, 0};
  if (p.balanced) {
    const int64_t records =
        (int64_t)p.head_groups * p.chunks * p.heads_per_group * p.rows;
    w.ml = records * d->head_dim * 4;
    w.meta = w.ml + ((records * 8 + 15) & ~(int64_t)15);
    w.total = w.meta + (int64_t)d->num_tokens * 16;
  } else if (!p.prefill) {
    w = fixed_ws_layout(d, p.splits);
  }
  return w;
}

pda_status check_pointers(const void* q, const void* k, const void* v, const int32_t* bt,
                          const int32_t* sl, const float* ks, const float* vs,
                          const pda_decode_dims* d) {
  if (!q || !k || !v || !bt || !sl)
    return fail(PDA_ERR_NULL, "q, k_cache, v_cache, block_table and seq_lens must be non-NULL");
  const bool quant = d->kv_dtype != PDA_KV_F16;
  if (quant && (!ks || !vs))
    return fail(PDA_ERR_NULL, "fp8/int8 KV needs k_scale and v_scale");
  if (!quant && (ks || vs))
    return fail(PDA_ERR_SHAPE, "k_scale/v_scale must be NULL for fp16 KV");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(PDA_ERR_ALIGN, "q, k_cache and v_cache must be 16-byte aligned");
  return PDA_OK;
}

// CUs the persistent prefill grid is sized for: the device's, or fewer when
// the environment variable PDA_PREFILL_CUS holds a smaller positive count (a
// small problem then runs many items per workgroup in turn, as a large one
// does on the whole device).
int prefill_grid_cus() {
  const int cus = device_cu_count();
  const char* e = std::getenv("PDA_PREFILL_CUS");
  if (cus > 0 && e != nullptr) {
    const long n = std::strtol(e, nullptr, 10);
    if (n > 0 && n < cus) return (int)n;
  }
  return cus;
}

pda_status launch_decode(const Plan& p, const pda_decode_dims* d, pda::DecodeArgs& args,
                         hipStream_t stream) {
  hipError_t e;
  if (p.prefill) {
    // (items: token blocks x KV heads x sequences; the launcher sizes the grid)
    const dim3 items(p.row_tiles, d->num_kv_heads, d->batch);
    const int cus = prefill_grid_cus();
    if (cus <= 0) return fail(PDA_ERR_DEVICE, "cannot read the device's CU count");
    const int waves = p.threads / 64;
    switch (kv_kind(d->kv_dtype)) {
      case pda::kKvF16:
        e = pda::launch_prefill_f16(d->head_dim, waves, items, cus, p.lds, stream, args);
        break;
      case pda::kKvFp8:
        e = pda::launch_prefill_fp8(d->head_dim, waves, items, cus, p.lds, stream, args);
        break;
      default:
        e = pda::launch_prefill_i8(d->head_dim, waves, items, cus, p.lds, stream, args);
        break;
    }
    if (e != hipSuccess) return fail(PDA_ERR_DEVICE, "prefill launch: %s", hipGetErrorString(e));
    return PDA_OK;
  }
  const dim3 grid(p.balanced ? p.chunks : p.splits, p.head_groups, p.balanced ? 1 : d->batch);
  if (p.matrix) {
    switch (kv_kind(d->kv_dtype)) {
      case pda::kKvF16:
        e = pda::launch_decode_mfma_f16(d->head_dim, p.row_tiles, p.stream_kv, grid, p.threads, p.lds, stream,
                                        args);
        break;
      case pda::kKvFp8:
        e = pda::launch_decode_mfma_fp8(d->head_dim, p.row_tiles, p.stream_kv, grid, p.threads, p.lds, stream,
                                        args);
        break;
      default:
        e = pda::launch_decode_mfma_i8(d->head_dim, p.row_tiles, p.stream_kv, grid, p.threads, p.lds, stream,
                                       args);
        break;
    }
    if (e != hipSuccess) return fail(PDA_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
    return PDA_OK;
  }
  switch (kv_kind(d->kv_dtype)) {
    case pda::kKvF16:
      e = pda::launch_decode_f16(d->head_dim, p.rows_per_wave, grid, p.threads, p.lds, stream, args);
      break;
    case pda::kKvFp8:
      e = pda::launch_decode_fp8(d->head_dim, p.rows_per_wave, grid, p.threads, p.lds, stream, args);
      break;
    default:
      e = pda::launch_decode_i8(d->head_dim, p.rows_per_wave, grid, p.threads, p.lds, stream, args);
      break;
  }
  if (e != hipSuccess) return fail(PDA_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
  return PDA_OK;
}

pda::DecodeArgs make_args(const void* q, const void* k, const void* v, const int32_t* bt,
                          const int32_t* sl, const int32_t* ql, float scale, int32_t window,
                          const float* ks, const float* vs, const pda_decode_dims* d,
                          const Plan& p) {
  pda::DecodeArgs a{};
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.block_table = bt;
  a.seq_lens = sl;
  a.q_lens = d->max_q_len == 1 ? nullptr : ql;  // every q_len is 1: offsets are b
  a.k_scale = ks;
  a.v_scale = vs;
  a.qk_mult = scale * 1.4426950408889634f;  // scores in base-2 units
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.group = d->num_q_heads / d->num_kv_heads;
  a.max_pages = d->max_pages_per_seq;
  a.max_q_len = d->max_q_len;
  a.window = window;
  a.num_splits = p.splits;
  a.row_groups = p.row_groups;
  a.key_waves = p.key_waves;
  a.heads_per_group = p.heads_per_group;
  a.batch = d->batch;
  a.longest_first = p.longest_first;
  const uint32_t row = (uint32_t)d->head_dim * (d->kv_dtype == PDA_KV_F16 ? 2u : 1u);
  const bool hnd = d->kv_layout == PDA_LAYOUT_HND;
  a.key_stride = hnd ? row : row * (uint32_t)d->num_kv_heads;
  a.head_stride = hnd ? row * (uint32_t)d->page_size : row;
  a.page_bytes = (uint64_t)row * d->num_kv_heads * d->page_size;
  a.tile_shift = __builtin_ctz((unsigned)(d->page_size / pda::kPageSize));
  a.rows = p.rows;
  a.wave_lds_bytes = (int32_t)p.wave_lds;
  a.balanced = p.balanced;
  a.chunks = p.chunks;
  a.min_chunk = p.min_chunk;
  a.prefill_blocks = p.prefill ? p.row_tiles : 0;
  a.prefill_items = p.prefill ? p.row_tiles * d->num_kv_heads * d->batch : 0;
  return a;
}

pda_status check_q_lens(const int32_t* q_lens, const pda_decode_dims* d) {
  if (!q_lens && (d->num_tokens != d->batch || d->max_q_len != 1))
    return fail(PDA_ERR_SHAPE,
                "without q_lens every sequence has one token: num_tokens (%d) must equal "
                "batch (%d) and max_q_len (%d) must be 1",
                d->num_tokens, d->batch, d->max_q_len);
  if (q_lens && (int64_t)d->num_tokens > (int64_t)d->batch * d->max_q_len)
    return fail(PDA_ERR_SHAPE, "num_tokens %d exceeds batch * max_q_len", d->num_tokens);
  return PDA_OK;
}

pda_status check_out(const void* out) {
  if (!out) return fail(PDA_ERR_NULL, "out must be non-NULL");
  if (!aligned16(out)) return fail(PDA_ERR_ALIGN, "out must be 16-byte aligned");
  return PDA_OK;
}

pda_status check_workspace(const void* workspace, size_t workspace_bytes, const WsLayout& w) {
  if (w.total > 0) {
    if (!workspace || (int64_t)workspace_bytes < w.total)
      return fail(PDA_ERR_WORKSPACE, "workspace of %zu bytes at %p; %lld needed",
                  workspace_bytes, workspace, (long long)w.total);
    if (!aligned16(workspace)) return fail(PDA_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  return PDA_OK;
}

// Launch plan of the one-call path: automatic splits may be balanced per
// sequence (matrix kernel); otherwise the automatic count is resolved first
// and planned as a caller's count.
pda_status attention_plan(const pda_decode_dims* d, int32_t window, int32_t num_splits,
                          Plan* p, WsLayout* w, bool check_ws = false,
                          const void* workspace = nullptr, size_t workspace_bytes = 0) {
  if (num_splits < 0 || num_splits > PDA_MAX_SPLITS)
    return fail(PDA_ERR_SHAPE, "num_splits %d outside 0..%d", num_splits, PDA_MAX_SPLITS);
  *w = WsLayout{0, 0, 0};
  if (d->batch == 0 || d->num_tokens == 0) return PDA_OK;
  // A caller's count fixes the workspace without the device: check it first.
  if (num_splits >= 1 && !routes_to_prefill(d) && check_ws &&
      check_workspace(workspace, workspace_bytes, fixed_ws_layout(d, num_splits)) != PDA_OK)
    return PDA_ERR_WORKSPACE;
  const pda_status st = make_plan(d, window, num_splits, 0, p, /*allow_balanced=*/true);
  if (st != PDA_OK) return st;
  *w = attention_ws_layout(d, *p);
  return check_ws ? check_workspace(workspace, workspace_bytes, *w) : PDA_OK;
}

}  // namespace

extern "C" {

pda_status pda_attention_decode_stage(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      const int32_t* q_lens, float scale, int32_t window,
                                      int32_t num_splits, void* out, const float* k_scale,
                                      const float* v_scale, const pda_decode_dims* dims,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  pda_status st = check_dims(dims);
  if (st != PDA_OK) return st;
  if ((st = check_pointers(q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, dims)))
    return st;
  if ((st = check_q_lens(q_lens, dims))) return st;
  Plan p;
  WsLayout w;
  if ((st = check_out(out))) return st;
  if ((st = attention_plan(dims, window, num_splits, &p, &w, true, workspace, workspace_bytes)))
    return st;
  if (dims->batch == 0 || dims->num_tokens == 0) return PDA_OK;
  pda::DecodeArgs a = make_args(q, k_cache, v_cache, block_table, seq_lens, q_lens, scale,
                                window, k_scale, v_scale, dims, p);
  a.out = static_cast<uint16_t*>(out);
  a.direct = !p.balanced && p.splits == 1;
  if (w.total > 0) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(ws + w.ml);
    a.meta = p.balanced ? reinterpret_cast<int32_t*>(ws + w.meta) : nullptr;
  }
  return launch_decode(p, dims, a, stream);
}

pda_status pda_attention_combine_stage(void* out, const pda_decode_dims* dims, int32_t window,
                                       int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  pda_status st = check_dims(dims);
  if (st != PDA_OK) return st;
  Plan p;
  WsLayout w;
  if ((st = check_out(out))) return st;
  if ((st = attention_plan(dims, window, num_splits, &p, &w, true, workspace, workspace_bytes)))
    return st;
  if (dims->batch == 0 || dims->num_tokens == 0 || w.total == 0) return PDA_OK;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  pda::CombineArgs c{};
  c.part_o = reinterpret_cast<const float*>(ws);
  c.part_ml = reinterpret_cast<const float*>(ws + w.ml);
  c.out = static_cast<uint16_t*>(out);
  c.meta = p.balanced ? reinterpret_cast<const int32_t*>(ws + w.meta) : nullptr;
  c.num_splits = p.splits;
  c.num_q_heads = dims->num_q_heads;
  c.group = dims->num_q_heads / dims->num_kv_heads;
  c.rows = p.rows;
  c.chunks = p.chunks;
  c.per_seq = p.splits;
  c.max_q_len = dims->max_q_len;
  const int rows = dims->num_tokens * dims->num_q_heads;
  const int waves = p.balanced ? p.combine_waves : pda::combine_waves(p.splits);
  const hipError_t e = pda::launch_combine(
      c, rows, dims->head_dim, waves, pda::combine_dim_parts(rows, dims->head_dim, device_cu_count()),
      stream);
  if (e != hipSuccess) return fail(PDA_ERR_DEVICE, "combine launch: %s", hipGetErrorString(e));
  return PDA_OK;
}

pda_status pda_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      const int32_t* q_lens, float scale, int32_t window,
                                      int32_t num_splits, void* out, const float* k_scale,
                                      const float* v_scale, const pda_decode_dims* dims,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  const pda_status st = pda_attention_decode_stage(
      q, k_cache, v_cache, block_table, seq_lens, q_lens, scale, window, num_splits, out,
      k_scale, v_scale, dims, workspace, workspace_bytes, stream);
  if (st != PDA_OK) return st;
  return pda_attention_combine_stage(out, dims, window, num_splits, workspace, workspace_bytes,
                                     stream);
}

pda_status pda_paged_decode_partials(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const int32_t* q_lens, float scale, int32_t window,
                                     int32_t num_splits, const float* k_scale,
                                     const float* v_scale, const pda_decode_dims* dims,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  pda_status st = check_dims(dims);
  if (st != PDA_OK) return st;
  if ((st = check_pointers(q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, dims)))
    return st;
  if ((st = check_q_lens(q_lens, dims))) return st;
  if (num_splits < 0 || num_splits > PDA_MAX_SPLITS)
    return fail(PDA_ERR_SHAPE, "num_splits %d outside 0..%d", num_splits, PDA_MAX_SPLITS);
  if (routes_to_prefill(dims))
    return fail(PDA_ERR_UNSUPPORTED, "partials come from the decode kernels only "
                "((num_q_heads/num_kv_heads)*max_q_len <= %d, kernel not PREFILL)", PDA_MAX_ROWS);
  if (dims->batch == 0 || dims->num_tokens == 0) return PDA_OK;
  int splits = 0;
  if ((st = resolve_split_count(dims, window, num_splits, 0, &splits))) return st;
  const int64_t need = partials_bytes(dims, splits);
  if (!workspace || (int64_t)workspace_bytes < need)
    return fail(PDA_ERR_WORKSPACE, "workspace of %zu bytes at %p; %lld needed for %d splits",
                workspace_bytes, workspace, (long long)need, splits);
  if (!aligned16(workspace)) return fail(PDA_ERR_ALIGN, "workspace must be 16-byte aligned");
  Plan p;
  if ((st = make_plan(dims, window, splits, 0, &p))) return st;
  pda::DecodeArgs a = make_args(q, k_cache, v_cache, block_table, seq_lens, q_lens, scale,
                                window, k_scale, v_scale, dims, p);
  a.direct = 0;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = a.part_o + (size_t)dims->num_tokens * dims->num_q_heads * p.splits * dims->head_dim;
  return launch_decode(p, dims, a, stream);
}

pda_status pda_split_combine(const float* partial_o, const float* partial_ml, void* out,
                             int32_t num_tokens, int32_t num_q_heads, int32_t head_dim,
                             int32_t num_splits, hipStream_t stream) {
  if (!partial_o || !partial_ml || !out)
    return fail(PDA_ERR_NULL, "partial_o, partial_ml and out must be non-NULL");
  if (num_tokens < 0 || num_q_heads <= 0)
    return fail(PDA_ERR_SHAPE, "num_tokens %d / num_q_heads %d", num_tokens, num_q_heads);
  if (head_dim != 128 && head_dim != 256)
    return fail(PDA_ERR_UNSUPPORTED, "head_dim %d: compiled for 128 and 256", head_dim);
  if (num_splits < 1 || num_splits > PDA_MAX_SPLITS)
    return fail(PDA_ERR_SHAPE, "num_splits %d outside 1..%d", num_splits, PDA_MAX_SPLITS);
  if (!aligned16(partial_o) || !aligned16(out))
    return fail(PDA_ERR_ALIGN, "partial_o and out must be 16-byte aligned");
  if (num_tokens == 0) return PDA_OK;
  const int64_t rows = (int64_t)num_tokens * num_q_heads;
  if (rows > INT32_MAX) return fail(PDA_ERR_SHAPE, "num_tokens * num_q_heads too large");
  pda::CombineArgs c{};
  c.part_o = partial_o;
  c.part_ml = partial_ml;
  c.out = static_cast<uint16_t*>(out);
  c.num_splits = num_splits;
  const hipError_t e = pda::launch_combine(
      c, (int)rows, head_dim, pda::combine_waves(num_splits),
      pda::combine_dim_parts((int)rows, head_dim, device_cu_count()), stream);
  if (e != hipSuccess) return fail(PDA_ERR_DEVICE, "combine launch: %s", hipGetErrorString(e));
  return PDA_OK;
}

int32_t pda_decode_resolve_splits(const pda_decode_dims* dims, int32_t window,
                                  int32_t num_splits, int32_t num_cus) {
  int splits = 0;
  const pda_status st = resolve_split_count(dims, window, num_splits, num_cus, &splits);
  return st == PDA_OK ? splits : st;
}

int64_t pda_decode_partials_bytes(const pda_decode_dims* dims, int32_t window,
                                  int32_t num_splits) {
  int splits = 0;
  const pda_status st = resolve_split_count(dims, window, num_splits, 0, &splits);
  return st == PDA_OK ? partials_bytes(dims, splits) : st;
}

int64_t pda_decode_workspace_bytes(const pda_decode_dims* dims, int32_t window,
                                   int32_t num_splits) {
  pda_status st = check_dims(dims);
  if (st != PDA_OK) return st;
  if (num_splits >= 1 && num_splits <= PDA_MAX_SPLITS) {  // no device needed
    if (!routes_to_prefill(dims)) return fixed_ws_layout(dims, num_splits).total;
    if (num_splits > 1)
      return fail(PDA_ERR_UNSUPPORTED, "the prefill kernel runs one split (num_splits 0 or 1)");
    return 0;
  }
  Plan p;
  WsLayout w;
  st = attention_plan(dims, window, num_splits, &p, &w);
  return st == PDA_OK ? w.total : st;
}

const char* pda_last_error(void) { return pda::host_last_error(); }

const char* pda_version(void) { return "pda 0.1.0 gfx950"; }

}  // extern "C"
