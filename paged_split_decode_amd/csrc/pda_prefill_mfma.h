// Paged attention for long query runs (prefill, chunked prefill, long
// verify) on the gfx950 matrix cores: the same operation as the decode
// kernels, for many new tokens per sequence.
//
// A workgroup takes a block of new tokens of one sequence and all G query
// heads of one KV head: 32 (token, head) rows per wave, 4 or 8 waves (8 at
// D=128 when the keys before the new tokens are long, or a KV head has many
// rows); at D=256, 8 waves in pairs that share 32 rows, each computing the
// scores of half of a step's keys (the halves are swapped through LDS) and
// accumulating half of the output dims. K and V go through LDS once per
// workgroup and serve all its waves, 64 keys (four 16-key tiles) per step,
// stored as fp16 in the order the matrix instructions read them. fp16 pages
// go straight from the paged cache into LDS (16-byte direct loads, half the
// waves loading K and half V, two or three steps deep, explicit waits and one
// barrier per step); 1-byte codes are loaded into registers, converted to
// fp16 exactly and stored, two buffers deep.
//
// Per wave and 64 keys: S^T = K . Q^T with v_mfma_f32_32x32x16_f16 (K
// fragments read from LDS, the wave's 32 Q rows as the B operand; lane l then
// holds 16 scores of query row l % 32 per 32 keys), an online softmax with a
// lazily moved reference, and O^T += V^T . P^T with the same instruction: P
// from the score registers, V^T from ds_read_b64_tr_b16. Each row has its own
// causal limit (its position) and window; a step no row of the wave sees is
// skipped, and keys a row does not see get score -inf. Workgroups run in an
// XCD-aware order, the token blocks with the most keys first.
#pragma once

#include "pda_decode_mfma.h"

// Diagnostic builds only (-DPDA_PREFILL_TIMELINE=1; the library is otherwise
// unchanged): per item, wave 0 reads the 100 MHz clock at the end of each
// phase of its start and end, and the shader clock at the item's start and
// end, waiting for each reading at once (so that its latency is not charged
// to a later phase), and writes them over the first values of the item's
// first output row. paged_split_decode_amd/timeline.py builds, runs and reads
// them.
#ifndef PDA_PREFILL_TIMELINE
#define PDA_PREFILL_TIMELINE 0
#endif

namespace pda {

typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// A compile-time bool carried by value (selects a lambda body variant).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

template <int I>
struct IntC {
  static constexpr int value = I;
};

// LDS allows one workgroup per CU (two at D=128 with 4 waves), so at most two
// waves share a SIMD; the compiler is told so, and keeps loads ahead in
// registers instead of trimming them for a third wave that never comes.
template <int D, int KV, int WAVES>
__global__ void __launch_bounds__(64 * WAVES, (D == 128 || WAVES == 8) ? 2 : 1)
__attribute__((amdgpu_waves_per_eu(1, (D == 128 || WAVES == 8) ? 2 : 1)))
pda_prefill_mfma_kernel(const DecodeArgs a) {
  // LDS holds K and V of 64-key steps as fp16, each in the order the matrix
  // instructions read it, so that every read is a contiguous run with no
  // bank conflict and no padding:
  //  - K of a 32-key half h and k-step t (16 dims): one 1 KB block whose
  //    16-byte slot l holds key 32 h + l % 32, dims 16 t + 8 (l / 32) .. + 7,
  //    which is lane l's A fragment of v_mfma_f32_32x32x16_f16;
  //  - V of a 16-key tile and 32 dims (group dg): one 1 KB block whose slot s
  //    holds key 8 (s / 32) + 4 (s / 16 % 2) + s / 4 % 4 of the tile, dims
  //    32 dg + 8 (s % 4) .. + 7; each 32-lane pass of the transposing reads
  //    then covers 256 contiguous bytes.
  // fp16 caches go to LDS by direct 16-byte loads (global_load_lds_dwordx4:
  // lane l of a wave's load lands at 16 l bytes from the block start), NBUF
  // step buffers deep with no staging registers; 1-byte codes go through
  // registers (NREG sets) to be converted to fp16 on the way.
  constexpr int KT = prefill_tiles(D);  // 16-key tiles per step
  constexpr int NK = D / 16;            // QK k-steps = K blocks of a half
  constexpr int NDV = D / 32;           // V blocks of a tile
  constexpr int KH_BYTES = NK * 1024;   // K of one 32-key half
  constexpr int VT_BYTES = NDV * 1024;  // V of one 16-key tile
  constexpr int BUF_BYTES = 2 * KH_BYTES + KT * VT_BYTES;
  static_assert(BUF_BYTES == prefill_step_bytes(D), "host and kernel agree on the step size");
  constexpr int NBUF = prefill_buffers(D, KV, WAVES);
  constexpr bool DMA = KV == kKvF16;
  constexpr int NTHREADS = 64 * WAVES;
  constexpr int CHUNKS = 2 * KT * 16 * (D / 16);     // 16-byte code chunks of a step (1-byte KV)
  constexpr int LOADS = DMA ? 1 : CHUNKS / NTHREADS;  // per thread and step
  // Steps whose loads are in flight in registers (1-byte KV, each in its own
  // set): the loads of step s + NREG + 1 are issued when step s ends and go
  // to LDS when step s + NREG ends.
  constexpr int NREG = DMA ? 1 : (WAVES == 8 && D == 128) ? 2 : 1;
  static_assert(DMA || (NBUF == 2 && CHUNKS % NTHREADS == 0), "register staging: two buffers");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];

  const int tid = threadIdx.x;
  const int lane0 = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // At D=256 (8 waves) waves 2 r and 2 r + 1 share the rows 32 r .. + 31:
  // each computes the scores of one 32-key half of a step (all D dims) and
  // hands them to the other through LDS; both then run the softmax over all
  // 64 keys, and each accumulates half of the output dims. o takes 64
  // registers instead of 128, so two waves fit per SIMD, and no score is
  // computed twice. The partners sit on different SIMDs (waves w and w + 4
  // share one), so that while one pair waits for its scores, the other
  // pair's wave on the same SIMD keeps the matrix unit busy.
  constexpr bool PAIR = D == 256 && WAVES == 8;
  // Persistent workgroups at D=128 (below); at D=256 one item per workgroup
  // measured faster.
  constexpr bool PERSIST = !PAIR;
  // Q through LDS (fp16 KV): in 64 KB of its own after the three step
  // buffers at D=128 with 8 waves (where the output tiles then go too),
  // else in step buffer 1, which no load reaches before the first step.
  constexpr bool QLDS = DMA;
  constexpr bool Q_OWN = QLDS && prefill_q_own(D, KV, WAVES);
  constexpr int QS_AT = Q_OWN ? NBUF * BUF_BYTES : BUF_BYTES;
  static_assert(!QLDS || Q_OWN || NBUF == 2, "Q in step buffer 1: only step 0 loads before the first step");
  static_assert(!QLDS || (PAIR ? WAVES / 2 : WAVES) * 32 * 2 * D <=
                             (Q_OWN ? (int)prefill_out_lds_bytes(D, WAVES) : BUF_BYTES),
                "Q fits its region");
  const int rg = PAIR ? (wave >> 1) : wave;  // row block
  const int dh = PAIR ? (wave & 1) : 0;      // key half of the scores, output dim half
  // One item (token block, KV head, sequence) per call of `item`, by its
  // logical index lg. Dispatch slot v goes to XCD v % 8 (the dispatcher
  // hands workgroups to the 8 XCDs in turn), and each XCD has its own L2;
  // the token blocks of one (sequence, KV head) read the same keys, so they
  // should run on one XCD at about the same time: slot v takes logical index
  // lg such that XCD x owns a contiguous run of them.
  auto item = [&](const uint32_t lg) __attribute__((always_inline)) {
    // (the lane index made opaque per item: what derives from it is computed
    // inside the item, where it is used, not once before the item loop and
    // kept in registers through every item)
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    // (diagnostic builds: stamp k ends phase k - 1; 0 at the item's start)
    uint32_t tl[7] = {0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint64_t tl_cycles = 0;
    auto stamp = [&](int k) __attribute__((always_inline)) {
      if constexpr (PDA_PREFILL_TIMELINE) {
        __builtin_amdgcn_sched_barrier(0);
        tl[k] = (uint32_t)__builtin_amdgcn_s_memrealtime();
        if (k == 0) tl_cycles = __builtin_amdgcn_s_memtime();
        if (k == 6) tl_cycles = __builtin_amdgcn_s_memtime() - tl_cycles;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    stamp(0);
    // Item lg -> (token block, KV head, sequence): token block fastest, the
    // blocks with the most keys first.
    int g, b, blk;
    {
      const uint32_t nx = (uint32_t)a.prefill_blocks, ny = (uint32_t)a.num_kv_heads;
      const uint32_t rest = lg / nx;
      blk = (int)(nx - 1 - (lg - rest * nx));
      g = (int)(rest % ny);
      b = (int)(rest / ny);
    }
    const int dcol = dh * (D / 2);  // first output dim of this wave
    const int G = a.group;
    const int Hq = a.num_q_heads;
    const int BQ = a.rows / G;                   // tokens per workgroup
    const int L = a.seq_lens[b];
    const int Qb = a.q_lens ? a.q_lens[b] : 1;
    const int i0 = blk * BQ;
    if (i0 >= Qb) return;  // the whole workgroup: no barrier is skipped by a part of it
    const int pos0 = L - Qb;  // position of token 0
    const int W = a.window;
    auto lo_of = [&](int pos) { return W > 0 ? max(0, pos - W + 1) : 0; };

    // Key range of the workgroup, in tiles: [lo of its first token, its last
    // token's position].
    const int ilast = min(Qb, i0 + BQ) - 1;
    const int khi = pos0 + ilast;
    const int klo = lo_of(pos0 + i0);
    const int t_lo = klo / kPageSize;
    const int n_tiles = khi >= 0 ? khi / kPageSize - t_lo + 1 : 0;
    const int n_steps = (n_tiles + KT - 1) / KT;

    // Wave-uniform summaries of this wave's rows 32 rg .. + 31 for the skip /
    // unmasked tests: their tokens run from i_a to i_b (rows past the
    // workgroup's, tokens past the sequence's and negative positions left
    // out), and the bounds of a token's keys grow with its position.
    int lo_min = 0x7fffffff, lo_max = 0, hi_min = 0x7fffffff, hi_max = -1;
    {
      const int r_b = min(32 * rg + 31, a.rows - 1);
      const int i_a = max(i0 + (32 * rg) / G, -pos0);
      const int i_b = min(i0 + r_b / G, Qb - 1);
      if (32 * rg <= r_b && i_a <= i_b) {
        hi_min = pos0 + i_a;
        hi_max = pos0 + i_b;
        lo_min = lo_of(hi_min);
        lo_max = lo_of(hi_max);
      }
    }

    // Cache addressing (as in the decode kernel): tile u of sequence b starts
    // at bt[u >> tile_shift] * page_bytes + (u & mask) * 16 * key_stride; slot
    // j of head g at j * key_stride + g * head_stride inside it.
    typedef const __attribute__((address_space(4))) int32_t* bt_ptr_t;
    const bt_ptr_t bt = (bt_ptr_t)(a.block_table + (size_t)b * a.max_pages);
    const int tshift = a.tile_shift;
    const int tmask = (1 << tshift) - 1;
    const uint32_t key_stride = a.key_stride;
    const uint32_t head_off = (uint32_t)g * a.head_stride;
    auto tile_base = [&](int u) -> size_t {
      return (size_t)bt[u >> tshift] * a.page_bytes + (size_t)((u & tmask) * kPageSize) * key_stride;
    };

    // First tile of step `step` (past the last step: tiles past the range,
    // which tile_at clamps).
    auto step_tile = [&](int step) __attribute__((always_inline)) { return t_lo + step * KT; };
    // Tile tt of step `step`; tiles past the workgroup's range are read from
    // its last tile (in bounds; all their keys are masked).
    const int last_tile = t_lo + n_tiles - 1;
    auto tile_at = [&](int step, int tt) __attribute__((always_inline)) {
      return tile_base(min(step_tile(step) + tt, last_tile));
    };
    const uint32_t lds_u32 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)lds_raw;
    // One direct 16-byte load per lane into LDS at byte dst + 16 lane (dst
    // wave-uniform, in M0; one wait state after M0 is written). Written as asm
    // so that the compiler's wait insertion does not track an LDS write in
    // flight: it would make LDS reads wait for every outstanding load,
    // including those of the steps ahead. The waits this pipeline needs are
    // explicit (wait_vm before each barrier).
    auto lds_load16 = [](const uint8_t* src, uint32_t dst) __attribute__((always_inline)) {
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(dst))
                   : "memory");
    };

    // fp16 caches, direct loads: waves [0, WAVES / 2) load K, the others V, in
    // whole 1 KB blocks, PERK per K wave and PERV per V wave and step; a K
    // wave's blocks lie in one half, a V wave's cover whole tiles. Each lane's
    // byte offset within a tile is fixed: K, key lane % 16 of the lane's tile
    // (lane / 16 % 2 of the half) at dims 8 (lane / 32) ..; V, the key row of
    // slot `lane` at dims 8 (lane % 4) ...
    constexpr int PERK = 2 * NK / (WAVES / 2);
    constexpr int PERV = KT * NDV / (WAVES / 2);
    static_assert(NK % PERK == 0 && PERV % NDV == 0, "a wave's blocks: one half, or whole tiles");
    const bool kwave = wave < WAVES / 2;
    const int wk = kwave ? wave : wave - WAVES / 2;
    const int vrow = 8 * (lane >> 5) + 4 * ((lane >> 4) & 1) + ((lane >> 2) & 3);
    const uint32_t lane_off = kwave ? (uint32_t)(lane & 15) * key_stride + head_off + 16u * (lane >> 5)
                                    : (uint32_t)vrow * key_stride + head_off + 16u * (lane & 3);
    // The tiles a wave loads each step: a K wave tiles ta and ta + 1 (its
    // half), a V wave tiles ta .. ta + PERV / NDV - 1 (at most two). Inside the
    // step loop their bases come from the block table before the barrier of
    // the step before, so the scalar loads' latency hides under the barrier.
    const int ta = kwave ? 2 * ((wk * PERK) / NK) : (wk * PERV) / NDV;
    static_assert(PERV / NDV <= 2, "a V wave loads at most two tiles a step");
    auto dma_bases = [&](size_t b0, size_t b1, int buf) __attribute__((always_inline)) {
      const uint32_t dst0 = lds_u32 + (uint32_t)(buf * BUF_BYTES);
      if (kwave) {
        const int t0 = (wk * PERK) % NK;
        const uint8_t* src = a.k + ((lane & 16) ? b1 : b0) + lane_off + 32 * t0;
        const uint32_t dst = dst0 + (uint32_t)((ta / 2) * KH_BYTES + t0 * 1024);
  #pragma unroll
        for (int i = 0; i < PERK; ++i) lds_load16(src + 32 * i, dst + 1024u * i);
      } else {
  #pragma unroll
        for (int q = 0; q < PERV / NDV; ++q) {
          const uint8_t* src = a.v + (q == 0 ? b0 : b1) + lane_off;
          const uint32_t dst = dst0 + (uint32_t)(2 * KH_BYTES + (ta + q) * VT_BYTES);
  #pragma unroll
          for (int dg = 0; dg < NDV; ++dg) lds_load16(src + 64 * dg, dst + 1024u * dg);
        }
      }
    };
    // After a V wave's loads of a step have landed: V slots of keys at or past
    // the sequence's end hold whatever the page has there (a weight 0 times a
    // NaN would spoil P.V), so they become zeros. (For a tile read in place of
    // one past the range, keys counted at the tile's own place are past every
    // slot it copies that lies past the end.) K there only meets masked scores.
    auto dma_zero_tail = [&](int step, int buf) __attribute__((always_inline)) {
      const int key_base = step_tile(step) * kPageSize;
      if (kwave || key_base + KT * kPageSize <= L) return;
      uint8_t* const dst0 = lds_raw + buf * BUF_BYTES + 2 * KH_BYTES;
  #pragma unroll
      for (int q = 0; q < PERV / NDV; ++q) {
        const int tt = (wk * PERV) / NDV + q;
        if (key_base + tt * kPageSize + vrow >= L) {
  #pragma unroll
          for (int dg = 0; dg < NDV; ++dg)
            *reinterpret_cast<u32x4*>(dst0 + tt * VT_BYTES + dg * 1024 + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    // s_waitcnt with vmcnt(VM) and lgkmcnt(0) (expcnt untouched).
    // The empty asm after it keeps the compiler from moving LDS accesses (the
    // zeroing of a step's tail, say) above the wait for the direct loads they
    // depend on; the loads' asm carries a memory clobber for the same reason.
    auto wait_vm = [](auto vm_c) __attribute__((always_inline)) {
      constexpr int VM = decltype(vm_c)::value;
      __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
      asm volatile("" ::: "memory");
    };
    // Workgroup barrier without a memory fence (the waits before it are
    // explicit); the empty asm statements keep the compiler from moving memory
    // accesses across it.
    auto barrier = []() __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    // 1-byte codes, register staging: chunk c = tid + NTHREADS l of a step is
    // K or V (kv), key row r64 of the step's 64, dims 16 j .. + 15; its 16
    // codes become two fp16 slots (K: k-step j of the row's half, slot
    // r64 % 32 and that + 32; V: block j / 2 of the row's tile, slots s and
    // s + 1). All of that is fixed per thread; each step only moves the
    // (scalar) tile bases.
    uint32_t src_off[LOADS];
    uint32_t lds_off[LOADS], lds_off2[LOADS];
    int row_of[LOADS], tt_of[LOADS];
    bool is_v[LOADS];
    if constexpr (!DMA) {
  #pragma unroll
      for (int l = 0; l < LOADS; ++l) {
        const int c = tid + NTHREADS * l;
        const int kv = c / (CHUNKS / 2);
        const int rem = c - kv * (CHUNKS / 2);
        const int r64 = rem / (D / 16), j = rem % (D / 16);
        tt_of[l] = r64 >> 4;
        row_of[l] = r64 & 15;
        is_v[l] = kv != 0;
        src_off[l] = (uint32_t)row_of[l] * key_stride + head_off + 16u * j;
        if (!kv) {
          lds_off[l] = (uint32_t)((r64 >> 5) * KH_BYTES + j * 1024 + 16 * (r64 & 31));
          lds_off2[l] = lds_off[l] + 512;
        } else {
          const int r = r64 & 15;
          const int slot = 32 * (r >> 3) + 16 * ((r >> 2) & 1) + 4 * (r & 3) + 2 * (j & 1);
          lds_off[l] = (uint32_t)(2 * KH_BYTES + tt_of[l] * VT_BYTES + (j >> 1) * 1024 + 16 * slot);
          lds_off2[l] = lds_off[l] + 16;
        }
      }
    }
    uint32_t stage_regs[NREG][LOADS][4];
    auto stage_load = [&](int step, auto set_c) __attribute__((always_inline)) {
      auto& stage = stage_regs[decltype(set_c)::value];
      size_t base[KT];
  #pragma unroll
      for (int tt = 0; tt < KT; ++tt) base[tt] = tile_at(step, tt);
  #pragma unroll
      for (int l = 0; l < LOADS; ++l) {
        const uint8_t* src = (is_v[l] ? a.v : a.k) + base[tt_of[l]] + src_off[l];
        const u32x4 x = *reinterpret_cast<const u32x4*>(src);
  #pragma unroll
        for (int e = 0; e < 4; ++e) stage[l][e] = x[e];
      }
    };
    auto stage_store = [&](int step, int buf, auto set_c) __attribute__((always_inline)) {
      auto& stage = stage_regs[decltype(set_c)::value];
      const int t0 = step_tile(step);
      const int j0 = t0 * kPageSize;
      uint8_t* const dst0 = lds_raw + buf * BUF_BYTES;
      // Slots past the sequence (arbitrary contents), and tiles past this
      // workgroup's range, become zeros. Only a step that reaches past either
      // needs the per-slot test (wave-uniform).
      auto put = [&](auto checked) __attribute__((always_inline)) {
  #pragma unroll
        for (int l = 0; l < LOADS; ++l) {
          bool live = true;
          if constexpr (decltype(checked)::value) {
            const int u = t0 + tt_of[l];
            live = u < t_lo + n_tiles && j0 + tt_of[l] * kPageSize + row_of[l] < L;
          }
          h2_t hv[8];
          to_pairs<KV>(stage[l], hv);
          u32x4 w0, w1;
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            w0[e] = live ? __builtin_bit_cast(uint32_t, hv[e]) : 0u;
            w1[e] = live ? __builtin_bit_cast(uint32_t, hv[4 + e]) : 0u;
          }
          *reinterpret_cast<u32x4*>(dst0 + lds_off[l]) = w0;
          *reinterpret_cast<u32x4*>(dst0 + lds_off2[l]) = w1;
        }
      };
      if (t0 - t_lo + KT <= n_tiles && j0 + KT * kPageSize <= L)
        put(BoolC<false>{});
      else
        put(BoolC<true>{});
    };

    // The tile bases of the first steps (their scalar loads, with no branch
    // between them, are in flight together with the offset's loads below; an
    // index clamped to 0 is in bounds when there are no steps).
    size_t tb[NBUF - 1][2];
    if constexpr (DMA) {
  #pragma unroll
      for (int j = 0; j < NBUF - 1; ++j) {
        tb[j][0] = tile_base(max(min(step_tile(j) + ta, last_tile), 0));
        tb[j][1] = tile_base(max(min(step_tile(j) + ta + 1, last_tile), 0));
      }
    }
    // First token of sequence b in q and out (read before any cache load
    // goes out, so that the wait for it waits for nothing else).
    int off = b;
    if (a.q_lens) {
      int sum = 0;
      for (int i = lane; i < b; i += 64) sum += a.q_lens[i];
      off = wave_sum_i(sum);
    }
    stamp(1);

    // 32 x 32 x 16 MFMA lane layouts (A: lane l holds row l % 32, k = 8 h + 0..7
    // with h = l / 32; B: column l % 32, same k; C: column l % 32, rows
    // 8 j + 4 h + i in element 4 j + i). So lane l works on query row rr = l % 32
    // of this wave's 32 rows; lanes l and l + 32 share the row.
    const int rr = lane & 31;
    const int hh = lane >> 5;
    const int myr = 32 * rg + rr;  // the workgroup row of this lane
    const int my_i = i0 + myr / G;
    const bool my_row = myr < a.rows && my_i < Qb;
    const int my_pos = pos0 + my_i;
    const int my_lo = (my_row && my_pos >= 0) ? lo_of(my_pos) : 0;
    const int my_hi = (my_row && my_pos >= 0) ? my_pos : -1;

    // Q^T as the B operand: lane l holds row rr, dims 16 t + 8 hh .. + 7 of
    // k-step t. A negative scale flips q's sign.
    typedef const __attribute__((address_space(4))) float* scale_ptr_t;
    float qk = a.qk_mult * (a.k_scale ? ((scale_ptr_t)a.k_scale)[g] : 1.0f);
    const uint32_t qflip = qk < 0.0f ? 0x80008000u : 0u;
    // Scores of keys a row does not see are set to -inf before the softmax;
    // with a zero scale -inf * 0 would be NaN, so a zero multiplier becomes
    // the smallest normal float: every product with a finite score is then
    // too small to change exp2 in fp32, and the weights stay exactly 1.
    qk = fabsf(qk) > 0.0f ? fabsf(qk) : __FLT_MIN__;
    constexpr int NDT = (PAIR ? D / 2 : D) / 32;  // 32-dim output tiles of this wave
    // The Q loads go out before the first steps' cache loads, and Q is first
    // read after the wait for those: the two latencies overlap, and the cache
    // loads stay the youngest, as the explicit waits below count on. (A row
    // without a token reads its token clamped into the sequence, in bounds,
    // and keeps zeros.)
    //   fp16 KV: Q goes through LDS by direct loads of whole rows (a 1 KB load
    //   covers 1024 / (2 D) rows, instead of 16-byte pieces of 32 rows, four
    //   times the cache lines per load); the wave's 32 rows (at D=256, half
    //   of its pair's 32 rows each) are stored row after row, 16-byte piece c
    //   of row r at piece c ^ (r % 16), so that the reads of 16 rows' piece c
    //   (one pass) fall on 16 distinct piece slots. 1-byte KV: Q goes to
    //   registers directly.
    u32x4 qx[NK];
    uint8_t* const qs = lds_raw + QS_AT + rg * 32 * (2 * D);  // this row block's Q rows
    // (only with a step to wait for: the wait for step 0 covers these loads,
    // and an item without steps writes its zero rows through the same LDS)
    if (QLDS && n_steps > 0) {
      constexpr int RB = 2 * D;          // bytes per row
      constexpr int RPL = 1024 / RB;     // rows per 1 KB load
      constexpr int SPR = RB / 16;       // 16-byte pieces per row
      constexpr int NQL = 8;             // loads per wave
      static_assert(NQL * RPL == (PAIR ? 16 : 32), "a wave loads its share of its 32 rows");
      const int r0 = PAIR ? 16 * dh : 0;
  #pragma unroll
      for (int k = 0; k < NQL; ++k) {
        const int r = r0 + k * RPL + lane / SPR;  // row in the row block
        const int sl = lane % SPR;                 // its piece slot
        const int wr = 32 * rg + r;                // the workgroup row
        const int qi = min(i0 + wr / G, Qb - 1);
        const uint8_t* src = a.q + ((size_t)(off + qi) * Hq + g * G + (wr - (wr / G) * G)) * RB +
                             16 * (sl ^ (r & 15));
        lds_load16(src, lds_u32 + (uint32_t)(QS_AT + rg * 32 * RB + (r0 + k * RPL) * RB));
      }
    } else if (!QLDS) {
      const uint8_t* qrow =
          a.q + ((size_t)(off + min(my_i, Qb - 1)) * Hq + g * G + (myr - (myr / G) * G)) * (D * 2);
  #pragma unroll
      for (int t = 0; t < NK; ++t) qx[t] = *reinterpret_cast<const u32x4*>(qrow + 32 * t + 16 * hh);
    }
    if constexpr (DMA) {
  #pragma unroll
      for (int j = 0; j < NBUF - 1; ++j)
        if (j < n_steps) dma_bases(tb[j][0], tb[j][1], j);
    } else {
      if (n_steps > 0) stage_load(0, IntC<0>{});
    }
    stamp(2);
    h8_t qb[NK];
    // After the barrier that follows the wait for the first step (and Q).
    auto q_ready = [&]() __attribute__((always_inline)) {
      if constexpr (QLDS) {
  #pragma unroll
        for (int t = 0; t < NK; ++t)
          qx[t] = *reinterpret_cast<const u32x4*>(qs + rr * (2 * D) + 16 * ((2 * t + hh) ^ (rr & 15)));
      }
      const uint32_t keep = my_row ? 0xFFFFFFFFu : 0u;
  #pragma unroll
      for (int t = 0; t < NK; ++t) {
  #pragma unroll
        for (int e = 0; e < 4; ++e) qx[t][e] = (qx[t][e] & keep) ^ qflip;
        qb[t] = __builtin_bit_cast(h8_t, qx[t]);
      }
      // Q staged in step buffer 1: every wave has read it before the first
      // step's loads go there.
      if constexpr (QLDS && !Q_OWN) {
        wait_vm(IntC<63>{});
        barrier();
      }
    };

    constexpr float kNoMax = -1e30f;
    constexpr float kLazy = 8.0f;
    float m = kNoMax, mx = kNoMax, lsum = 0.0f;
    f16v_t o[NDT];
  #pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f16v_t{};

    typedef short s4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4_t lds_s4_t;
    auto tr_read = [&](const uint8_t* src) __attribute__((always_inline)) {
      return __builtin_bit_cast(h4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s4_t*)(__attribute__((address_space(3))) uint8_t*)src));
    };
    const int q16 = lane >> 4, i16 = lane & 15;  // 16-lane group and lane in it
    // The transposing V reads: lane l takes 4 dims (8 bytes) of key row
    // 4 hh + i16 / 4 (+ 8 for the upper 8 keys of a k-step) at dims
    // 16 (q16 % 2) + 4 (i16 % 4) of a 32-dim group: slot
    // 16 hh + 4 (i16 / 4) + 2 (q16 % 2) + (i16 % 4) / 2 of the group's block,
    // second 8 bytes when i16 is odd.
    const uint32_t v_lane = 16u * (16 * hh + 4 * (i16 >> 2) + 2 * (q16 & 1) + ((i16 & 3) >> 1)) +
                            8u * (i16 & 1);

    // Whether this wave has work on the 32 keys from key0 (wave-uniform).
    auto active = [&](int key0) { return hi_max >= 0 && key0 <= hi_max && key0 + 31 >= lo_min; };
    // S^T[key][row] of 32 keys: lane l gets row rr, keys 8 j + 4 hh + i in
    // st[4 j + i]. The two halves' chains of dependent MFMAs are interleaved
    // (scores2), with each k-step's K fragments read one step ahead. (At D=256,
    // one wave per SIMD, this order measured 0.8% faster than computing each
    // half's scores just before its softmax; its extra registers go to AGPRs.)
    auto frag = [&](const uint8_t* kh, int t) __attribute__((always_inline)) {
      return *reinterpret_cast<const h8_t*>(kh + 1024 * t + 16 * lane);
    };
    auto scores2 = [&](const uint8_t* kb0, const uint8_t* kb1, f16v_t& s0, f16v_t& s1) __attribute__((always_inline)) {
      h8_t k0 = frag(kb0, 0), k1 = frag(kb1, 0);
      s0 = f16v_t{};
      s1 = f16v_t{};
  #pragma unroll
      for (int t = 0; t < NK; ++t) {
        h8_t n0 = k0, n1 = k1;
        if (t + 1 < NK) {
          n0 = frag(kb0, t + 1);
          n1 = frag(kb1, t + 1);
        }
        // (the next k-step's reads stay ahead of this one's MFMAs)
        __builtin_amdgcn_sched_barrier(0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, qb[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, qb[t], s1, 0, 0, 0);
        k0 = n0;
        k1 = n1;
      }
    };
    // Scores of one 32-key half (PAIR): one chain of MFMAs, K read a k-step
    // ahead (the partner wave on the SIMD fills the matrix unit between them).
    auto scores1 = [&](const uint8_t* kh, f16v_t& s) __attribute__((always_inline)) {
      h8_t k = frag(kh, 0);
      s = f16v_t{};
  #pragma unroll
      for (int t = 0; t < NK; ++t) {
        h8_t n = k;
        if (t + 1 < NK) n = frag(kh, t + 1);
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(k, qb[t], s, 0, 0, 0);
        k = n;
      }
    };
    // Softmax and P.V of the 64 keys from key0 whose scores are st[0] (keys
    // key0 ..) and st[1] (key0 + 32 ..). Where some row of the wave sees only
    // part of the keys (a uniform test), the scores of keys a row does not see
    // become -inf first: they leave the maximum alone and get weight
    // exp2(-inf) = 0. Every other step runs no per-key test. One maximum and
    // one rescale test cover both halves, so the weights and P.V of both run in
    // one block (the exponentials of one half can issue under the other's
    // matrix instructions).
    auto softmax_pv = [&](f16v_t (&st)[2], const uint8_t* vb, int key0) __attribute__((always_inline)) {
      if (!(key0 >= lo_max && key0 + 63 <= hi_min)) {
  #pragma unroll
        for (int h = 0; h < 2; ++h) {
          // lane's key of slot v: key0 + 32 h + 8 (v / 4) + 4 hh + v % 4
          const int d_lo = my_lo - key0 - 32 * h - 4 * hh, d_hi = my_hi - key0 - 32 * h - 4 * hh;
  #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int c = 8 * (v >> 2) + (v & 3);
            st[h][v] = (c >= d_lo && c <= d_hi) ? st[h][v] : -INFINITY;
          }
        }
      }
      float mt;
      {
        float a[8];
  #pragma unroll
        for (int h = 0; h < 2; ++h)
  #pragma unroll
          for (int q = 0; q < 4; ++q)
            a[4 * h + q] = fmaxf(fmaxf(st[h][4 * q], st[h][4 * q + 1]),
                                 fmaxf(st[h][4 * q + 2], st[h][4 * q + 3]));
        mt = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])),
                   fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7])));
      }
      {  // the other half of the row's keys sits in lane l ^ 32
        auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, mt),
                                                   __builtin_bit_cast(int, mt), false, false);
        mt = fmaxf(__builtin_bit_cast(float, (int)sw[0]), __builtin_bit_cast(float, (int)sw[1]));
      }
      mt = mt == -INFINITY ? kNoMax : qk * mt;
      mx = fmaxf(mx, mt);
      if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {
        const float alpha = __builtin_amdgcn_exp2f(m - mx);
        lsum *= alpha;
  #pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        m = mx;
      }
      // O^T[dim][row] += V^T . P^T over four 16-key k-steps. k-step 2 h + ks
      // takes the lane's keys of half h, j = 2 ks, 2 ks + 1 (slots 8 hh + e:
      // key 32 h + 16 ks + 4 hh + e, then 32 h + 16 ks + 8 + 4 hh + e); V^T's A
      // operand uses the same key order: two transposing reads of 4
      // consecutive key rows at this lane's dim. The denominator adds the same
      // fp16 weights that P.V multiplies V by (v_dot2 with ones: each fp16
      // value enters the fp32 sum exactly).
      const h2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
      h8_t pb[2][2];
  #pragma unroll
      for (int h = 0; h < 2; ++h) {
  #pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            pb[h][ks][e] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(st[h][8 * ks + e], qk, -m));
            pb[h][ks][4 + e] =
                (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(st[h][8 * ks + 4 + e], qk, -m));
          }
  #pragma unroll
          for (int e = 0; e < 8; e += 2)
            lsum = __builtin_amdgcn_fdot2(h2_t{pb[h][ks][e], pb[h][ks][e + 1]}, one2, lsum, false);
        }
      }
      // V^T fragment of tile g = 2 h + ks, dims dcol + 32 dt
      auto vfrag = [&](int g, int dt) __attribute__((always_inline)) {
        const uint8_t* vt = vb + g * VT_BYTES + (dcol / 32) * 1024 + v_lane + 1024 * dt;
        const h4_t lo = tr_read(vt);
        const h4_t hi = tr_read(vt + 512);
        return h8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      if constexpr (!PAIR) {
        // (each tile's fragments read one tile ahead of their MFMAs; the
        // scheduling barriers keep them there)
        h8_t vf[2][NDT];
  #pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vf[0][dt] = vfrag(0, dt);
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g + 1 < 4) {
  #pragma unroll
            for (int dt = 0; dt < NDT; ++dt) vf[(g + 1) & 1][dt] = vfrag(g + 1, dt);
          }
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[g & 1][dt], pb[g >> 1][g & 1], o[dt], 0, 0, 0);
        }
      } else {
  #pragma unroll
        for (int g = 0; g < 4; ++g)
  #pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vfrag(g, dt), pb[g >> 1][g & 1], o[dt], 0, 0, 0);
      }
    };

    // One step's compute on LDS buffer buf. A step no row of the wave sees is
    // skipped. (A half that no row sees still gets scores, from finite LDS
    // data, when the other half is needed; they are masked to weight 0. The
    // score registers live only inside the branch that uses them: a value
    // merged from a path that skips them would be zero-filled every step.)
    // PAIR: the score exchange, after the step buffers: wave w's 16 scores
    // per lane in four 1 KB blocks (floats 4 c .. 4 c + 3 of lane l at
    // 1024 c + 16 l, conflict-free). The two waves meet there without a
    // workgroup barrier: each score's lowest mantissa bit carries the parity
    // of the pair's count of computed steps (a change of at most 2^-23
    // relative, and both waves use the same tagged values), so the reader
    // waits until every word it reads carries this step's tag. The blocks
    // start out tagged 1 (before the first barrier), the first step writes
    // tag 0. A word is read after it is written (the reader polls) and
    // written again only after the next barrier, which the reader reaches
    // after reading it.
    uint8_t* const xs = lds_raw + NBUF * BUF_BYTES;
    int x_count = 0;  // steps this pair has computed
    if constexpr (PAIR) {
  #pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<u32x4*>(xs + wave * 4096 + 1024 * c + 16 * lane) = u32x4{1u, 1u, 1u, 1u};
    }
    static_assert(!PAIR || WAVES * 4096 == (int)prefill_xchg_bytes(D, WAVES), "exchange size");
    // mid() runs once per step, after the scores (or at once on a skipped
    // step): the V waves issue their loads there.
    auto compute = [&](int step, int buf, auto&& mid) __attribute__((always_inline)) {
      const uint8_t* kb = lds_raw + buf * BUF_BYTES;
      const int key0 = step_tile(step) * kPageSize;
      if constexpr (PAIR) {
        // Both waves of a pair have the same rows, hence the same test.
        if (!(active(key0) || active(key0 + 32))) {
          mid();
        } else {
          const uint32_t tag = (uint32_t)(x_count & 1);
          ++x_count;
          f16v_t mine;
          scores1(kb + dh * KH_BYTES, mine);
          // (through a scalar: __builtin_bit_cast of a vector element lvalue
          // reads element 0)
  #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float x = mine[v];
            mine[v] = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & ~1u) | tag);
          }
  #pragma unroll
          for (int c = 0; c < 4; ++c)
            *reinterpret_cast<f32x4_t*>(xs + wave * 4096 + 1024 * c + 16 * lane) =
                f32x4_t{mine[4 * c], mine[4 * c + 1], mine[4 * c + 2], mine[4 * c + 3]};
          asm volatile("" ::: "memory");  // the writes stay ahead of the polls
          mid();
          // The partner's scores: poll until all of them carry the tag. (A
          // bound on the polls keeps every wave finite whatever happens; the
          // partner writes within the same step, so it is never reached.)
          typedef const volatile __attribute__((address_space(3))) u32x4 lds_vu4_t;
          lds_vu4_t* src = (lds_vu4_t*)(__attribute__((address_space(3))) uint8_t*)(xs + (wave ^ 1) * 4096 + 16 * lane);
          u32x4 w[4];
          uint32_t stale = ~0u;  // no poll yet; left nonzero if the bound ends the polls
          for (int polls = 0; polls < (1 << 20) && stale != 0u; ++polls) {
            uint32_t bad = 0u;
  #pragma unroll
            for (int c = 0; c < 4; ++c) {
              w[c] = src[64 * c];
  #pragma unroll
              for (int e = 0; e < 4; ++e) bad |= (w[c][e] & 1u) ^ tag;
            }
            stale = __builtin_amdgcn_ballot_w64(bad != 0u) != 0 ? 1u : 0u;
            if (stale != 0u) __builtin_amdgcn_s_sleep(1);
          }
          // (should the bound ever end the polls, the scores become NaN, so the
          // rows' output shows it instead of silently using old scores)
          f16v_t other;
  #pragma unroll
          for (int c = 0; c < 4; ++c)
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t x = stale != 0u ? 0x7fc00000u : w[c][e];
              other[4 * c + e] = __builtin_bit_cast(float, x);
            }
          f16v_t st[2];
          st[0] = dh ? other : mine;
          st[1] = dh ? mine : other;
          softmax_pv(st, kb + 2 * KH_BYTES, key0);
        }
      } else if (active(key0) || active(key0 + 32)) {
        f16v_t st[2];
        scores2(kb, kb + KH_BYTES, st[0], st[1]);
        mid();
        softmax_pv(st, kb + 2 * KH_BYTES, key0);
      } else {
        mid();
      }
    };

    if constexpr (DMA) {
      // Step s computes on buffer s % NBUF; its start issues the loads of step
      // s + NBUF - 1 (that buffer was last read in step s - 1, which every
      // wave has left at the barrier); its end waits for this wave's loads of
      // step s + 1 (the loads of step s + 2 may stay in flight), zeroes
      // that step's tail, and meets the other waves at the barrier.
      static_assert(NBUF >= 2 && NBUF <= 4, "two to four step buffers");
      // Wait for this wave's loads of step `need`, with the loads of the steps
      // after it that were issued (up to `issued_to`, at most two) in flight.
      auto wait_step = [&](int need, int issued_to) __attribute__((always_inline)) {
        const int after = min(issued_to, n_steps - 1) - need;
        if (after >= 2) {
          if (kwave)
            wait_vm(IntC<2 * PERK>{});
          else
            wait_vm(IntC<2 * PERV>{});
        } else if (after == 1) {
          if (kwave)
            wait_vm(IntC<PERK>{});
          else
            wait_vm(IntC<PERV>{});
        } else {
          wait_vm(IntC<0>{});
        }
      };
      if (n_steps > 0) {
        // (steps 0 .. NBUF - 2 were issued above; Q loads may follow them)
        wait_step(0, NBUF - 2);
        stamp(3);
        dma_zero_tail(0, 0);
        wait_vm(IntC<63>{});
        barrier();
        stamp(4);
        q_ready();
        int buf = 0;
        size_t nb0 = tile_at(NBUF - 1, ta), nb1 = tile_at(NBUF - 1, ta + 1);
        for (int step = 0; step < n_steps; ++step) {
          const int nb = buf + 1 == NBUF ? 0 : buf + 1;  // buffer of step + 1
          const int lb = buf == 0 ? NBUF - 1 : buf - 1;  // of step + NBUF - 1
          // (At D=256 the V waves issue their loads after the scores: a
          // step's 64 KB of loads from all waves at once back up the memory
          // pipeline and stall the waves that issue last, and V of a step is
          // read last. Measured 2% faster there, 3-5% slower at D=128.)
          const bool issue = step + NBUF - 1 < n_steps;
          constexpr bool LATE_V = PAIR;
          if ((kwave || !LATE_V) && issue) dma_bases(nb0, nb1, lb);
          compute(step, buf, [&]() __attribute__((always_inline)) {
            if (LATE_V && !kwave && issue) dma_bases(nb0, nb1, lb);
          });
          if (step + 1 < n_steps) {
            wait_step(step + 1, step + NBUF - 1);
            dma_zero_tail(step + 1, nb);
            wait_vm(IntC<63>{});
            // (tile_at clamps, so a step past the last reads a valid entry)
            nb0 = tile_at(step + NBUF, ta);
            nb1 = tile_at(step + NBUF, ta + 1);
            barrier();
          }
          buf = nb;
        }
      }
    } else if (n_steps > 0) {
      stage_store(0, 0, IntC<0>{});
      if (n_steps > 1) stage_load(1, IntC<0>{});
      if constexpr (NREG >= 2) {
        if (n_steps > 2) stage_load(2, IntC<1>{});
      }
      __syncthreads();
      q_ready();
      // Step `step` reads LDS buffer step & 1; register set SET holds step + 1.
      auto step_body = [&](int step, auto set_c) __attribute__((always_inline)) {
        const int buf = step & 1;
        compute(step, buf, []() {});
        if (step + 1 < n_steps) stage_store(step + 1, buf ^ 1, set_c);
        if (step + 1 + NREG < n_steps) stage_load(step + 1 + NREG, set_c);
        __syncthreads();
      };
      for (int step = 0; step < n_steps; step += NREG) {
        step_body(step, IntC<0>{});
        if constexpr (NREG >= 2) {
          if (step + 1 < n_steps) step_body(step + 1, IntC<1>{});
        }
      }
    }

    stamp(5);
    // Bring o, l to the row maximum, add the two lane halves' l, and write
    // fp16 out (a row that sees no key is 0), one division per row: o times
    // alpha * v_scale / l. Lane l holds dims 32 dt + 8 j + 4 hh .. + 3 of row
    // rr; the rows go through a wave-private LDS tile so that the global
    // stores are whole rows, 16 lanes x 16 bytes each, instead of 8-byte
    // pieces of 32 rows. In the tile (rows of 256 bytes, no padding), 16-byte
    // piece c of row r sits at piece c ^ (r % 16) of the row, with its two
    // 8-byte halves swapped in rows 16 .. 31: the 32 lanes of a write pass
    // (32 rows, one half each) then fill all 64 banks once, and so do the 16
    // lanes of a read pass (the 16 pieces of a row).
    const float alpha = __builtin_amdgcn_exp2f(m - mx);
    lsum *= alpha;
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, lsum),
                                                 __builtin_bit_cast(int, lsum), false, false);
      lsum = __builtin_bit_cast(float, (int)sw[0]) + __builtin_bit_cast(float, (int)sw[1]);
    }
    const float vs = a.v_scale ? ((scale_ptr_t)a.v_scale)[g] : 1.0f;
    const float f = lsum > 0.0f ? (alpha * vs) / lsum : 0.0f;
    constexpr int DW = PAIR ? D / 2 : D;  // dims this wave writes
    constexpr int RS = 2 * DW;           // LDS bytes per row
    constexpr int PPR = DW / 8;          // 16-byte pieces of a row
    static_assert(PPR == 16, "the piece order assumes 16 pieces per row");
    static_assert(WAVES * 32 * RS == (int)prefill_out_lds_bytes(D, WAVES), "out tile size");
    // The tiles: in the Q region where it is the wave's own (its Q rows were
    // read at the start). With two step buffers and tiles that fit in one,
    // in the buffer the last step did not use: no load goes there after the
    // last step, and every wave read it last before the barrier this wave
    // passed ahead of the last step (with one step, it held Q, which every
    // wave read before the barrier after Q), so no barrier is needed. Else
    // over the step buffers, once every wave has left the last step's reads.
    constexpr bool FREE_BUF = !Q_OWN && NBUF == 2 && WAVES * 32 * RS <= BUF_BYTES;
    if constexpr (!Q_OWN && !FREE_BUF) __syncthreads();
    uint8_t* const tile =
        lds_raw + (Q_OWN ? QS_AT : FREE_BUF ? (n_steps & 1) * BUF_BYTES : 0) + wave * 32 * RS;
  #pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        h4_t y;
  #pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (_Float16)(o[dt][4 * j + e] * f);
        *reinterpret_cast<h4_t*>(tile + rr * RS + 16 * ((4 * dt + j) ^ (rr & 15)) + 8 * (hh ^ (rr >> 4))) = y;
      }
    }
    // (all of a lane's pieces read first, then stored; row (64 p + lane) / 16
    // is at least 16 exactly when p >= 4)
    constexpr int NP = 32 * PPR / 64;
    u32x4 pv[NP];
  #pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = (64 * p + lane) / PPR, pc = lane % PPR;
      const u32x4 w = *reinterpret_cast<const u32x4*>(tile + r * RS + 16 * (pc ^ (r & 15)));
      pv[p] = p >= NP / 2 ? u32x4{w[2], w[3], w[0], w[1]} : w;
    }
  #pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = (64 * p + lane) / PPR, pc = lane % PPR;
      const int wr = 32 * rg + r;  // the workgroup row
      const int i = i0 + wr / G;
      if (wr < a.rows && i < Qb) {
        const size_t hrow = (size_t)(off + i) * Hq + g * G + (wr - (wr / G) * G);
        *reinterpret_cast<u32x4*>(a.out + hrow * D + dcol + 8 * pc) = pv[p];
      }
    }
    stamp(6);
    if constexpr (PDA_PREFILL_TIMELINE) {
      // (the item's first row: workgroup row 0, written by wave 0 above)
      if (wave == 0 && lane == 0) {
        uint32_t* const tp = reinterpret_cast<uint32_t*>(a.out + ((size_t)(off + i0) * Hq + g * G) * D);
        for (int k = 0; k < 7; ++k) tp[k] = tl[k];
        tp[7] = (uint32_t)tl_cycles;
        tp[8] = (uint32_t)n_steps;
        tp[9] = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));   // HW_ID: CU, SH, SE
        tp[10] = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (31 << 11));  // XCC_ID
      }
    }
  };
  auto slot_item = [](uint32_t v, uint32_t n) {
    const uint32_t xcd = v & 7u, k = v >> 3;
    return xcd * (n >> 3) + min(xcd, n & 7u) + k;
  };
  const uint32_t n_items = (uint32_t)a.prefill_items;
  if constexpr (PERSIST) {
    // Persistent workgroups (as many as fit on the device): round r gives
    // them the slots r P .. r P + P - 1 (P = gridDim.x); on each XCD its
    // j-th workgroup takes the XCD's j-th slot of the round in even rounds
    // and the j-th from the end in odd ones. Items come longest first within
    // a (sequence, KV head), so the workgroup with the longest items of one
    // round gets the shortest of the next. No workgroup waits to be
    // dispatched behind another's exit. (A grid that is not a multiple of
    // 8 has one round: one item per workgroup.)
    const uint32_t P = gridDim.x, per = P >> 3, x8 = blockIdx.x & 7u, j8 = blockIdx.x >> 3;
    for (uint32_t r = 0;; ++r) {
      const uint32_t v = (P & 7u) ? blockIdx.x + r * P : 8u * (r * per + ((r & 1u) ? per - 1u - j8 : j8)) + x8;
      if (v >= n_items) break;
      item(slot_item(v, n_items));
      // (the next item's first loads go to step buffers 0 and 1, which a
      // slower wave may still read for this item's last step or, where the
      // output tiles lie over the step buffers, for its output)
      __syncthreads();
    }
  } else {
    item(slot_item(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), n_items));
  }
}

// At D=128 a persistent grid: as many workgroups as fit on the device at
// once (the occupancy the runtime reports for the kernel, block and LDS
// size, times the CU count), at most one per item; at D=256 one workgroup
// per item (grid = token blocks x KV heads x sequences).
template <int KV>
hipError_t launch_prefill_kv(int head_dim, int waves, dim3 items, int cus, size_t lds, hipStream_t stream,
                             const DecodeArgs& args) {
#define PDA_PCASE(DD, WW)                                                                            \
  if (head_dim == DD && waves == WW) {                                                               \
    auto* kern = pda_prefill_mfma_kernel<DD, KV, WW>;                                                \
    dim3 grid = items;                                                                               \
    if (DD == 128) {                                                                                 \
      static int per_cu = 0; /* the same on every MI355X; a race writes the same value */          \
      if (per_cu <= 0) {                                                                             \
        int n = 0;                                                                                   \
        const hipError_t oe = hipOccupancyMaxActiveBlocksPerMultiprocessor(                          \
            &n, reinterpret_cast<const void*>(kern), 64 * WW, lds);                                  \
        if (oe != hipSuccess) return oe;                                                             \
        per_cu = n > 0 ? n : 1;                                                                      \
      }                                                                                              \
      const int64_t n_items = (int64_t)items.x * items.y * items.z;                                  \
      grid = dim3((unsigned)std::min<int64_t>(n_items, (int64_t)cus * per_cu));                      \
    }                                                                                                \
    if (grid.x * grid.y * grid.z == 0) return hipSuccess;                                            \
    hipLaunchKernelGGL(kern, grid, dim3(64 * WW), lds, stream, args);                                \
    return hipGetLastError();                                                                        \
  }
  PDA_PCASE(128, 4)
  PDA_PCASE(128, 8)
  PDA_PCASE(256, 8)  // (D=256 always takes 8 waves)
#undef PDA_PCASE
  return hipErrorInvalidValue;
}

}  // namespace pda
