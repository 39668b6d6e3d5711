// Paged attention for long query runs (prefill, chunked prefill, long
// verify) on the gfx950 matrix cores: the same operation as the decode
// kernels, for many new tokens per sequence.
//
// A workgroup takes a block of new tokens of one sequence and all G query
// heads of one KV head: 32 (token, head) rows per wave, 4 or 8 waves (8 at
// D=128 when the keys before the new tokens are long: chunked prefill); at
// D=256, 8 waves in pairs that share 32 rows and split the output dims. K and
// V go through LDS once per workgroup and serve all its waves: each step the
// threads gather 64 keys (four 16-key tiles) of K and V from the paged cache
// with 16-byte loads, convert 1-byte codes to fp16 (exactly), and write them
// to one of two fp16 LDS buffers while the waves compute on the other; one
// barrier per step. A step's loads are issued when the step before the one
// that stores them ends (NREG = 1), or one step earlier still with 8 waves
// (NREG = 2: each thread stages half as much, so two register sets fit).
//
// Per wave and 32 keys: S^T = K . Q^T with v_mfma_f32_32x32x16_f16 (K
// fragments read from the LDS tile, the wave's 32 Q rows as the B operand;
// lane l then holds 16 scores of query row l % 32), an online softmax with a
// lazily moved reference, and O^T += V^T . P^T with the same instruction: P
// from the score registers, V^T from ds_read_b64_tr_b16. Each row has its own
// causal limit (its position) and window; 32 keys after all of a wave's rows,
// or before all their windows, are skipped by that wave. Workgroups with the
// most keys (the last token blocks) are dispatched first.
#pragma once

#include "pda_decode_mfma.h"

namespace pda {

typedef float f16v_t __attribute__((ext_vector_type(16)));

// A compile-time bool carried by value (selects a lambda body variant).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

template <int I>
struct IntC {
  static constexpr int value = I;
};

template <int D, int KV, int WAVES>
__global__ void __launch_bounds__(64 * WAVES, (D == 128 || WAVES == 8) ? 2 : 1)
pda_prefill_mfma_kernel(const DecodeArgs a) {
  // LDS row strides (halves): K rows D + 8 (4 dwords mod 64: the 16 rows of a
  // 128-bit fragment read pass hit disjoint banks), V rows D + 32 (16 dwords
  // mod 64: a 32-lane pass of the transposing reads covers 4 rows of 64
  // bytes, on disjoint banks; with D + 16 they overlapped 2-way).
  constexpr int LRK = D + 8;
  constexpr int LRV = D + 32;
  constexpr int TILEK = 16 * LRK;  // halves of one 16-key K tile
  constexpr int TILEV = 16 * LRV;
  constexpr int KT = prefill_tiles(D);
  constexpr int EB = KV == kKvF16 ? 2 : 1;
  constexpr int PIECES = D * EB / 16;                // 16-byte pieces of a cache row
  constexpr int NPIECE = 2 * KT * 16 * PIECES;      // K and V pieces of one step
  constexpr int NTHREADS = 64 * WAVES;
  constexpr int LOADS = NPIECE / NTHREADS;           // per thread and step
  // Steps whose loads are in flight in registers (each in its own set): the
  // loads of step s + NREG + 1 are issued when step s ends and go to LDS when
  // step s + NREG ends.
#ifdef PDA_PREFILL_NREG8
  constexpr int NREG = WAVES == 8 ? PDA_PREFILL_NREG8 : 1;  // tuning override
#else
  constexpr int NREG = (WAVES == 8 && D == 128) ? 2 : 1;
#endif
  static_assert(NREG >= 1 && NREG <= 3, "one to three register sets");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  _Float16* lds = reinterpret_cast<_Float16*>(lds_raw);
  // buffer x: K tiles at lds + x * KT * (TILEK + TILEV), V tiles KT * TILEK later
  constexpr int BUF = KT * (TILEK + TILEV);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // At D=256 waves w and w + 4 share the rows 32 (w % 4) .. + 31 and each
  // accumulates half of the output dims: both compute the rows' scores and
  // softmax, but o takes 64 registers instead of 128, so two waves fit per
  // SIMD and hide each other's LDS latency (a single wave waited for every K
  // fragment read right before its MFMA). Measured 6% faster than one wave
  // per row block.
  constexpr bool PAIR = D == 256 && WAVES == 8;
  const int rg = PAIR ? (wave & 3) : wave;  // row block
  const int dh = PAIR ? (wave >> 2) : 0;    // output dim half
  // Workgroup -> (token block, KV head, sequence), XCD-aware: the dispatcher
  // hands workgroups to the 8 XCDs in turn (id % 8), and each XCD has its own
  // L2. The token blocks of one (sequence, KV head) read the same keys, so
  // they should run on one XCD at about the same time: XCD x takes a
  // contiguous run of logical indices (token block fastest), in dispatch
  // order. Within a (sequence, KV head) the blocks with the most keys go
  // first.
  int g, b, blk;
  {
    const uint32_t nx = gridDim.x, ny = gridDim.y;
    const uint32_t n = nx * ny * gridDim.z;
    const uint32_t p = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const uint32_t xcd = p & 7u, k = p >> 3;
    const uint32_t lg = xcd * (n >> 3) + min(xcd, n & 7u) + k;
    const uint32_t rest = lg / nx;
    blk = (int)(nx - 1 - (lg - rest * nx));
    g = (int)(rest % ny);
    b = (int)(rest / ny);
  }
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int BQ = a.rows / G;                   // tokens per workgroup
  const int L = a.seq_lens[b];
  const int Qb = a.q_lens ? a.q_lens[b] : 1;
  const int i0 = blk * BQ;
  if (i0 >= Qb) return;  // the whole workgroup: no barrier is skipped by a part of it
  int off = b;
  if (a.q_lens) {
    int sum = 0;
    for (int i = lane; i < b; i += 64) sum += a.q_lens[i];
    off = wave_sum_int(sum);
  }
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

  // This wave's rows (16 rt + c of its 32): bounds per lane, and wave-uniform
  // summaries for the skip / unmasked tests.
  int lo_min = 0x7fffffff, lo_max = 0, hi_min = 0x7fffffff, hi_max = -1;
  for (int r = 32 * rg; r < 32 * rg + 32 && r < a.rows; ++r) {
    const int i = i0 + r / G;
    const int pos = pos0 + i;
    if (i < Qb && pos >= 0) {
      lo_min = min(lo_min, lo_of(pos));
      lo_max = max(lo_max, lo_of(pos));
      hi_min = min(hi_min, pos);
      hi_max = max(hi_max, pos);
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

  // Staging: thread piece p = tid + NTHREADS l (< NPIECE) is K or V (kv),
  // tile tt of the step, key row, 16-byte piece; all of that is fixed per
  // thread, so its byte offset within a tile and its LDS position are computed
  // once. Each step only moves the (scalar) tile bases.
  static_assert(NPIECE % NTHREADS == 0, "every thread stages whole pieces");
  uint32_t src_off[LOADS];
  uint32_t lds_off[LOADS];  // in halves
  int row_of[LOADS], tt_of[LOADS];
  bool is_v[LOADS];
#pragma unroll
  for (int l = 0; l < LOADS; ++l) {
    const int p = tid + NTHREADS * l;
    const int kv = p / (KT * 16 * PIECES);
    const int rem = p - kv * (KT * 16 * PIECES);
    tt_of[l] = rem / (16 * PIECES);
    row_of[l] = (rem / PIECES) % 16;
    const int piece = rem % PIECES;
    is_v[l] = kv != 0;
    src_off[l] = (uint32_t)row_of[l] * key_stride + head_off + 16u * piece;
    lds_off[l] = (uint32_t)(kv ? KT * TILEK + tt_of[l] * TILEV + row_of[l] * LRV
                               : tt_of[l] * TILEK + row_of[l] * LRK) + piece * (16 / EB);
  }
  uint32_t stage_regs[NREG][LOADS][4];
  auto stage_load = [&](int step, auto set_c) __attribute__((always_inline)) {
    auto& stage = stage_regs[decltype(set_c)::value];
    const int u0 = t_lo + step * KT;
    size_t base[KT];
#pragma unroll
    for (int tt = 0; tt < KT; ++tt) base[tt] = tile_base(min(u0 + tt, t_lo + n_tiles - 1));
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
    const int j0 = (t_lo + step * KT) * kPageSize;
    _Float16* dst0 = lds + (size_t)buf * BUF;
    // Slots past the sequence (arbitrary contents), and tiles past this
    // workgroup's range (staged from a clamped tile), become zeros. Only a
    // step that reaches past either needs the per-slot test (wave-uniform).
    auto put = [&](auto checked) __attribute__((always_inline)) {
#pragma unroll
      for (int l = 0; l < LOADS; ++l) {
        bool live = true;
        if constexpr (decltype(checked)::value) {
          const int u = t_lo + step * KT + tt_of[l];
          live = u < t_lo + n_tiles && j0 + tt_of[l] * kPageSize + row_of[l] < L;
        }
        _Float16* dst = dst0 + lds_off[l];
        if constexpr (KV == kKvF16) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = live ? stage[l][e] : 0u;
          *reinterpret_cast<u32x4*>(dst) = w;
        } else {
          h2_t hv[8];
          to_pairs<KV>(stage[l], hv);
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              w[e] = live ? __builtin_bit_cast(uint32_t, hv[4 * hh + e]) : 0u;
            *reinterpret_cast<u32x4*>(dst + 8 * hh) = w;
          }
        }
      }
    };
    if ((step + 1) * KT <= n_tiles && j0 + KT * kPageSize <= L)
      put(BoolC<false>{});
    else
      put(BoolC<true>{});
  };

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
  float qk = a.qk_mult * (a.k_scale ? a.k_scale[g] : 1.0f);
  const uint32_t qflip = qk < 0.0f ? 0x80008000u : 0u;
  qk = fabsf(qk);
  constexpr int NK = D / 16;   // QK k-steps
  constexpr int NDT = (PAIR ? D / 2 : D) / 32;  // 32-dim output tiles of this wave
  const int dcol = dh * (D / 2);
  h8_t qb[NK];
  {
    const uint8_t* qrow =
        a.q + ((size_t)(off + my_i) * Hq + g * G + (myr - (myr / G) * G)) * (D * 2);
#pragma unroll
    for (int t = 0; t < NK; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (my_row) x = *reinterpret_cast<const u32x4*>(qrow + 32 * t + 16 * hh);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] ^= qflip;
      qb[t] = __builtin_bit_cast(h8_t, x);
    }
  }

  constexpr float kNoMax = -1e30f;
  constexpr float kLazy = 8.0f;
  float m = kNoMax, mx = kNoMax, lsum = 0.0f;
  f16v_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f16v_t{};

  typedef short s4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4_t lds_s4_t;
  auto tr_read = [&](const _Float16* src) __attribute__((always_inline)) {
    return __builtin_bit_cast(h4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4_t*)(__attribute__((address_space(3))) _Float16*)src));
  };
  const int q16 = lane >> 4, i16 = lane & 15;  // 16-lane group and lane in it

  // One step of 32 keys (K rows kb[0..31], V rows vb[0..31] in LDS).
  // Whether this wave has work on the 32 keys from key0 (wave-uniform).
  auto active = [&](int key0) { return hi_max >= 0 && key0 <= hi_max && key0 + 31 >= lo_min; };
  // S^T[key][row] of 32 keys: lane l gets row rr, keys 8 j + 4 hh + i in
  // st[4 j + i]. The two halves' chains of dependent MFMAs are interleaved
  // (scores2), with each k-step's K fragments read one step ahead. (At D=256,
  // one wave per SIMD, this order measured 0.8% faster than computing each
  // half's scores just before its softmax; its extra registers go to AGPRs.)
  auto frag = [&](const _Float16* kb, int t) __attribute__((always_inline)) {
    return *reinterpret_cast<const h8_t*>(kb + rr * LRK + 16 * t + 8 * hh);
  };
  auto scores2 = [&](const _Float16* kb0, const _Float16* kb1, f16v_t& s0, f16v_t& s1) __attribute__((always_inline)) {
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
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, qb[t], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, qb[t], s1, 0, 0, 0);
      k0 = n0;
      k1 = n1;
    }
  };
  // Softmax and P.V of 32 keys from key0 whose scores are st.
  auto softmax_pv = [&](f16v_t st, const _Float16* vb, int key0) __attribute__((always_inline)) {
    const bool full = key0 >= lo_max && key0 + 31 <= hi_min;
    uint32_t vis = 0xFFFFu;  // bit 4 j + i: key key0 + 8 j + 4 hh + i visible to row rr
    float mt;
    if (full) {
      float a0 = fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3]));
      float a1 = fmaxf(fmaxf(st[4], st[5]), fmaxf(st[6], st[7]));
      float a2 = fmaxf(fmaxf(st[8], st[9]), fmaxf(st[10], st[11]));
      float a3 = fmaxf(fmaxf(st[12], st[13]), fmaxf(st[14], st[15]));
      mt = fmaxf(fmaxf(a0, a1), fmaxf(a2, a3));
    } else {
      vis = 0u;
      mt = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = key0 + 8 * (v >> 2) + 4 * hh + (v & 3);
        const bool ok = j >= my_lo && j <= my_hi;
        vis |= ok ? 1u << v : 0u;
        mt = fmaxf(mt, ok ? st[v] : -INFINITY);
      }
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
    float p[16];
    if (full) {
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[v], qk, -m));
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(st[v], qk, -m));
        p[v] = (vis >> v) & 1u ? e : 0.0f;
      }
    }
    // O^T[dim][row] += V^T . P^T over two 16-key k-steps. k-step ks takes the
    // lane's keys of j = 2 ks, 2 ks + 1 (slots 8 hh + e: key 16 ks + 4 hh + e,
    // then 16 ks + 8 + 4 hh + e); V^T's A operand uses the same key order:
    // two transposing reads of 4 consecutive key rows at this lane's dim.
    // The denominator adds the same fp16 weights that P.V multiplies V by
    // (v_dot2 with ones: each fp16 value enters the fp32 sum exactly).
    const h2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      h8_t pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[e] = (_Float16)p[8 * ks + e];
        pb[4 + e] = (_Float16)p[8 * ks + 4 + e];
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        lsum = __builtin_amdgcn_fdot2(h2_t{pb[e], pb[e + 1]}, one2, lsum, false);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int col = dcol + 32 * dt + 16 * (q16 & 1) + 4 * (i16 & 3);
        const h4_t lo = tr_read(vb + (16 * ks + 4 * hh + (i16 >> 2)) * LRV + col);
        const h4_t hi = tr_read(vb + (16 * ks + 8 + 4 * hh + (i16 >> 2)) * LRV + col);
        const h8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb, o[dt], 0, 0, 0);
      }
    }
  };

  if (n_steps > 0) {
    stage_load(0, IntC<0>{});
    stage_store(0, 0, IntC<0>{});
    if (n_steps > 1) stage_load(1, IntC<0>{});
    if constexpr (NREG >= 2) {
      if (n_steps > 2) stage_load(2, IntC<1>{});
    }
    if constexpr (NREG >= 3) {
      if (n_steps > 3) stage_load(3, IntC<2>{});
    }
    __syncthreads();
    // Step `step` reads LDS buffer step & 1; register set SET holds step + 1.
    auto step_body = [&](int step, auto set_c) __attribute__((always_inline)) {
      const int buf = step & 1;
      const _Float16* kb = lds + (size_t)buf * BUF;
      const _Float16* vb = kb + KT * TILEK;
      const int key0 = (t_lo + step * KT) * kPageSize;
      // Both halves' scores first: the second half's softmax can run under
      // the first half's P.V. (A half that no row of the wave sees still gets
      // scores, from finite LDS data, when the other half is needed; its
      // softmax and P.V are skipped.)
      const bool a0 = active(key0), a1 = active(key0 + 32);
      // (The score registers live only inside the branch that uses them: a
      // value merged from a path that skips them would be zero-filled every
      // step.)
      if (a0 || a1) {
        f16v_t st0, st1;
        scores2(kb, kb + 2 * TILEK, st0, st1);
        if (a0) softmax_pv(st0, vb, key0);
        if (a1) softmax_pv(st1, vb + 2 * TILEV, key0 + 32);
      }
      if (step + 1 < n_steps) stage_store(step + 1, buf ^ 1, set_c);
      if (step + 1 + NREG < n_steps) stage_load(step + 1 + NREG, set_c);
      __syncthreads();
    };
    for (int step = 0; step < n_steps; step += NREG) {
      step_body(step, IntC<0>{});
      if constexpr (NREG >= 2) {
        if (step + 1 < n_steps) step_body(step + 1, IntC<1>{});
      }
      if constexpr (NREG >= 3) {
        if (step + 2 < n_steps) step_body(step + 2, IntC<2>{});
      }
    }
  }

  // Bring o, l to the row maximum, add the two lane halves' l, write fp16 out
  // (a row that sees no key is 0). Lane l writes dims 32 dt + 8 j + 4 hh .. + 3.
  const float alpha = __builtin_amdgcn_exp2f(m - mx);
  lsum *= alpha;
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, lsum),
                                               __builtin_bit_cast(int, lsum), false, false);
    lsum = __builtin_bit_cast(float, (int)sw[0]) + __builtin_bit_cast(float, (int)sw[1]);
  }
  if (my_row) {
    const float vs = a.v_scale ? a.v_scale[g] : 1.0f;
    const size_t hrow = (size_t)(off + my_i) * Hq + g * G + (myr - (myr / G) * G);
    uint16_t* dst = a.out + hrow * D + dcol + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h4_t y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = lsum > 0.0f ? (_Float16)((o[dt][4 * j + e] * alpha * vs) / lsum) : (_Float16)0.0f;
        *reinterpret_cast<h4_t*>(dst + 32 * dt + 8 * j) = y;
      }
    }
  }
}

template <int KV>
hipError_t launch_prefill_kv(int head_dim, int waves, dim3 grid, size_t lds, hipStream_t stream,
                             const DecodeArgs& args) {
#define PDA_PCASE(DD, WW)                                                                      \
  if (head_dim == DD && waves == WW) {                                                         \
    hipLaunchKernelGGL((pda_prefill_mfma_kernel<DD, KV, WW>), grid, dim3(64 * WW), lds, stream, \
                       args);                                                                  \
    return hipGetLastError();                                                                  \
  }
  PDA_PCASE(128, 4)
  PDA_PCASE(128, 8)
  PDA_PCASE(256, 4)
  PDA_PCASE(256, 8)
#undef PDA_PCASE
  return hipErrorInvalidValue;
}

}  // namespace pda
