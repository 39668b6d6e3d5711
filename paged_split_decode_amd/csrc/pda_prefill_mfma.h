// Paged attention for long query runs (prefill, chunked prefill, long
// verify) on the gfx950 matrix cores: the same operation as the decode
// kernels, for many new tokens per sequence.
//
// A workgroup takes a block of new tokens of one sequence and all G query
// heads of one KV head: 128 (token, head) rows, 32 per wave as two 16-row
// tiles. K and V go through LDS once per workgroup and serve all 4 waves:
// each step the 256 threads gather 32 keys (16 at D=256) of K and V
// from the paged cache with 16-byte loads, convert 1-byte codes to fp16
// (exactly), and write them to one of two fp16 LDS buffers while the waves
// compute on the other; one barrier per step.
//
// Per wave and tile the arithmetic is the decode kernel's: S^T = K . Q^T with
// v_mfma_f32_16x16x32_f16 (K fragments read from the LDS tile, the wave's Q
// rows as the B operand), an online softmax with a lazily moved reference,
// and O^T += V^T . P^T with v_mfma_f32_16x16x16_f16, V fragments read with
// ds_read_b64_tr_b16. Each row has its own causal limit (its position) and
// window; a tile after all of a wave's rows, or before all their windows, is
// skipped by that wave. Workgroups with the most keys (the last token
// blocks) are dispatched first.
#pragma once

#include "pda_decode_mfma.h"

namespace pda {

template <int D, int KV>
__global__ void __launch_bounds__(256, D == 128 ? 2 : 1)
pda_prefill_mfma_kernel(const DecodeArgs a) {
  constexpr int NS = D / 32;       // QK k-steps of 32 dims
  constexpr int NDT = D / 16;      // PV output tiles of 16 dims
  constexpr int NRT = 2;           // row tiles per wave
  constexpr int LR = D + 8;        // LDS row stride, halves
  constexpr int TILE = 16 * LR;    // halves of one 16-key tile
  constexpr int KT = prefill_tiles(D);
  constexpr int EB = KV == kKvF16 ? 2 : 1;
  constexpr int PIECES = D * EB / 16;                // 16-byte pieces of a cache row
  constexpr int NPIECE = 2 * KT * 16 * PIECES;      // K and V pieces of one step
  constexpr int LOADS = (NPIECE + 255) / 256;        // per thread

  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  _Float16* lds = reinterpret_cast<_Float16*>(lds_raw);
  // buffer x: K tiles at lds + x * 2 * KT * TILE, V tiles KT * TILE later

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane >> 4;
  const int c = lane & 15;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int blk = gridDim.x - 1 - blockIdx.x;  // the most keys first
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
  int lo_c[NRT], hi_c[NRT];
  int lo_min = 0x7fffffff, lo_max = 0, hi_min = 0x7fffffff, hi_max = -1;
  for (int r = 32 * wave; r < 32 * wave + 32 && r < a.rows; ++r) {
    const int i = i0 + r / G;
    const int pos = pos0 + i;
    if (i < Qb && pos >= 0) {
      lo_min = min(lo_min, lo_of(pos));
      lo_max = max(lo_max, lo_of(pos));
      hi_min = min(hi_min, pos);
      hi_max = max(hi_max, pos);
    }
  }
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = 32 * wave + 16 * rt + c;
    const int i = i0 + r / G;
    const int pos = pos0 + i;
    const bool active = r < a.rows && i < Qb && pos >= 0;
    lo_c[rt] = active ? lo_of(pos) : 0;
    hi_c[rt] = active ? pos : -1;
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

  // Staging: thread piece p = tid + 256 l (< NPIECE) is K or V (kv), tile tt
  // of the step, key row, 16-byte piece; all of that is fixed per thread, so
  // its byte offset within a tile and its LDS position are computed once.
  // Each step only moves the (scalar) tile bases.
  static_assert(NPIECE % 256 == 0, "every thread stages whole pieces");
  uint32_t src_off[LOADS];
  uint32_t lds_off[LOADS];  // in halves
  int row_of[LOADS], tt_of[LOADS];
  bool is_v[LOADS];
#pragma unroll
  for (int l = 0; l < LOADS; ++l) {
    const int p = tid + 256 * l;
    const int kv = p / (KT * 16 * PIECES);
    const int rem = p - kv * (KT * 16 * PIECES);
    tt_of[l] = rem / (16 * PIECES);
    row_of[l] = (rem / PIECES) % 16;
    const int piece = rem % PIECES;
    is_v[l] = kv != 0;
    src_off[l] = (uint32_t)row_of[l] * key_stride + head_off + 16u * piece;
    lds_off[l] = (uint32_t)((kv * KT + tt_of[l]) * TILE + row_of[l] * LR + piece * (16 / EB));
  }
  uint32_t stage[LOADS][4];
  auto stage_load = [&](int step) {
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
  auto stage_store = [&](int step, int buf) {
    const int j0 = (t_lo + step * KT) * kPageSize;
    _Float16* dst0 = lds + (size_t)buf * 2 * KT * TILE;
#pragma unroll
    for (int l = 0; l < LOADS; ++l) {
      // slots past the sequence (arbitrary contents) become zeros
      const bool live = j0 + tt_of[l] * kPageSize + row_of[l] < L;
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
          for (int e = 0; e < 4; ++e) w[e] = live ? __builtin_bit_cast(uint32_t, hv[4 * hh + e]) : 0u;
          *reinterpret_cast<u32x4*>(dst + 8 * hh) = w;
        }
      }
    }
  };

  // Q rows as the B operand: lane (s, c) holds row 16 rt + c, dims
  // 32 t + 8 s .. + 7 of step t. A negative scale flips q's sign.
  float qk = a.qk_mult * (a.k_scale ? a.k_scale[g] : 1.0f);
  const uint32_t qflip = qk < 0.0f ? 0x80008000u : 0u;
  qk = fabsf(qk);
  h8_t qb[NRT][NS];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = 32 * wave + 16 * rt + c;
    const int i = i0 + r / G;
    const bool exists = r < a.rows && i < Qb;
    const uint8_t* qrow = a.q + ((size_t)(off + i) * Hq + g * G + (r - (r / G) * G)) * (D * 2);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (exists) x = *reinterpret_cast<const u32x4*>(qrow + 64 * t + 16 * s);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] ^= qflip;
      qb[rt][t] = __builtin_bit_cast(h8_t, x);
    }
  }

  constexpr float kNoMax = -1e30f;
  constexpr float kLazy = 8.0f;
  float m[NRT], mx[NRT], l[NRT];
  f4_t o[NRT][NDT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m[rt] = kNoMax;
    mx[rt] = kNoMax;
    l[rt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rt][dt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  typedef short s4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4_t lds_s4_t;

  auto compute_tile = [&](const _Float16* kt, const _Float16* vt, int u) {
    const int j0 = u * kPageSize;
    if (hi_max < 0 || j0 > hi_max || j0 + kPageSize - 1 < lo_min) return;  // wave-uniform
    const bool full = j0 >= lo_max && j0 + kPageSize - 1 <= hi_min;
    h4_t va[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const _Float16* src = vt + (4 * s + (c >> 2)) * LR + 16 * dt + 4 * (c & 3);
      va[dt] = __builtin_bit_cast(h4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s4_t*)(__attribute__((address_space(3))) _Float16*)src));
    }
    h8_t ka[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) ka[t] = *reinterpret_cast<const h8_t*>(kt + c * LR + 32 * t + 8 * s);
    f4_t sc[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      sc[rt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < NS; ++t)
        sc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[t], qb[rt][t], sc[rt], 0, 0, 0);
    }
    // Online softmax. Unmasked tiles (every key visible to every row of the
    // wave) and masked ones take separate, wave-uniform branches.
    float pv[NRT][4];
    uint32_t vis[NRT];  // bit i: key j0 + 4 s + i visible to this lane's row
    bool behind = false;
    if (full) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const float mt =
            qk * max4(fmaxf(fmaxf(sc[rt][0], sc[rt][1]), fmaxf(sc[rt][2], sc[rt][3])));
        mx[rt] = fmaxf(mx[rt], mt);
        behind |= mx[rt] > m[rt] + kLazy;
        vis[rt] = 0xFu;
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int j = j0 + 4 * s;
        float mt = -INFINITY;
        vis[rt] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool v = j + i >= lo_c[rt] && j + i <= hi_c[rt];
          vis[rt] |= v ? 1u << i : 0u;
          mt = fmaxf(mt, v ? sc[rt][i] : -INFINITY);
        }
        mt = max4(mt);
        mt = mt == -INFINITY ? kNoMax : qk * mt;
        mx[rt] = fmaxf(mx[rt], mt);
        behind |= mx[rt] > m[rt] + kLazy;
      }
    }
    if (__builtin_amdgcn_ballot_w64(behind) != 0) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const float alpha = __builtin_amdgcn_exp2f(m[rt] - mx[rt]);
        l[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[rt][dt] *= alpha;
        m[rt] = mx[rt];
      }
    }
    h4_t pb[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[rt][i], qk, -m[rt]));
        pv[rt][i] = (vis[rt] >> i) & 1u ? e : 0.0f;
      }
      l[rt] += (pv[rt][0] + pv[rt][1]) + (pv[rt][2] + pv[rt][3]);
      pb[rt] = h4_t{(_Float16)pv[rt][0], (_Float16)pv[rt][1], (_Float16)pv[rt][2], (_Float16)pv[rt][3]};
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[dt], pb[rt], o[rt][dt], 0, 0, 0);
  };

  if (n_steps > 0) {
    stage_load(0);
    stage_store(0, 0);
    __syncthreads();
    for (int step = 0; step < n_steps; ++step) {
      const int buf = step & 1;
      if (step + 1 < n_steps) stage_load(step + 1);
      const _Float16* kb = lds + (size_t)buf * 2 * KT * TILE;
#pragma unroll
      for (int tt = 0; tt < KT; ++tt) {
        const int u = t_lo + step * KT + tt;
        if (u < t_lo + n_tiles) compute_tile(kb + tt * TILE, kb + (KT + tt) * TILE, u);
      }
      if (step + 1 < n_steps) stage_store(step + 1, buf ^ 1);
      __syncthreads();
    }
  }

  // Rows of this wave: bring o, l to the row maximum, sum l over the 4 lane
  // groups, write fp16 out (a row that sees no key is 0).
  const float vs = a.v_scale ? a.v_scale[g] : 1.0f;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float alpha = __builtin_amdgcn_exp2f(m[rt] - mx[rt]);
    l[rt] = add4(l[rt] * alpha);
    const int r = 32 * wave + 16 * rt + c;
    const int i = i0 + r / G;
    if (r >= a.rows || i >= Qb) continue;
    const size_t hrow = (size_t)(off + i) * Hq + g * G + (r - (r / G) * G);
    uint16_t* dst = a.out + hrow * D + 4 * s;
    const float lsum = l[rt];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      h4_t y;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = lsum > 0.0f ? (_Float16)((o[rt][dt][e] * alpha * vs) / lsum) : (_Float16)0.0f;
      *reinterpret_cast<h4_t*>(dst + 16 * dt) = y;
    }
  }
}

template <int KV>
hipError_t launch_prefill_kv(int head_dim, dim3 grid, size_t lds, hipStream_t stream,
                             const DecodeArgs& args) {
  if (head_dim == 128) {
    hipLaunchKernelGGL((pda_prefill_mfma_kernel<128, KV>), grid, dim3(256), lds, stream, args);
    return hipGetLastError();
  }
  if (head_dim == 256) {
    hipLaunchKernelGGL((pda_prefill_mfma_kernel<256, KV>), grid, dim3(256), lds, stream, args);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace pda
