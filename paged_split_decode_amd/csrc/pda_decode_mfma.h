// Paged split-K decode attention on the gfx950 matrix cores.
//
// Work split: one workgroup per (split, group of KV heads, sequence). Its
// waves are heads_per_group x key_waves: each KV head of the group gets
// key_waves waves, each streaming a contiguous run of the split's pages with
// its own online softmax. The waves of one workgroup read the same pages of
// the pool at about the same time, one head's rows each, so the page blocks
// (all heads of 16 slots, contiguous in memory) are fetched together. With
// one wave per head a wave writes its result from registers; otherwise the
// waves of a head merge through LDS.
//
// Counters on the v_dot2 kernel (pda_decode_impl.h) show it issue-bound
// (about 480 VALU instructions per 8 KB of K+V, VALU active half the time at
// one wave per SIMD), so both products go to MFMA here and the VALU keeps
// only the softmax:
//
//  * Scores as S^T = K . Q^T with v_mfma_f32_16x16x32_f16: the page's 16 keys
//    are the A rows, the head's query rows (up to 16 per row tile, zero
//    padded) the B columns. Lane (s = lane/16, c = lane%16) loads 16 bytes of
//    key c per 32-dim step, so a wave instruction reads 16 keys x 64 bytes.
//    The result leaves lane (s, c) holding row c's scores for keys 4s..4s+3.
//  * That is exactly the B layout of P^T for O^T = V^T . P^T with
//    v_mfma_f32_16x16x16_f16 (k = the page's 16 keys), so P needs no
//    transpose. V is loaded coalesced (16 lanes per key row), written once to
//    a wave-private LDS tile and read back as the A operand with gfx950's
//    transposing LDS read (one ds_read_b64_tr_b16 per 16 dims). O^T
//    leaves lane (s, c) holding row c, so the online-softmax rescale is
//    lane-local.
//  * The row max crosses the wave's 4 lane groups with permlane16/32 swaps;
//    the denominator l stays per lane and is summed once at the end.
//  * fp8-e4m3 / int8 K and V are converted to fp16 exactly in registers; the
//    per-KV-head scales fold into the score multiplier and the output.
//  * Query rows beyond the real ones are zero; more than 16 rows take a
//    second row tile (up to 32).
#pragma once

#include "pda_decode_impl.h"

namespace pda {

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <int D, int KV>
struct MGeom {
  static constexpr int kElemBytes = KV == kKvF16 ? 2 : 1;
  static constexpr int kSteps = D / 32;                 // QK k-steps of 32 dims
  static constexpr int kKLoads = kSteps * kElemBytes / 2;  // 16-byte K loads per lane
  static constexpr int kVDims = D / 16;                 // V dims per lane per key row
  static constexpr int kVRaw = kVDims * kElemBytes / 4; // raw V dwords per lane per key
  static constexpr int kDTiles = D / 16;                // PV output tiles of 16 dims
  // LDS V row stride in halves: 16 halves of pad shift each row by 8 banks,
  // so the 8 rows x 32 bytes of one pass of a transposing read fall on
  // disjoint banks (an 8-half pad gave 2-way conflicts: a quarter of the
  // kernel's LDS cycles at fp16).
  static constexpr int kLdsRow = D + 16;
  static constexpr int kRowBytes = D * kElemBytes;
};

// Pages in a wave's load ring (NB - 1 pages in flight while one is used).
// Deeper rings measured no faster (the full grid keeps enough bytes in flight
// for the gather rate; deeper ones only add registers). PDA_RING overrides it
// when tuning.
template <int D, int KV, int NRT>
constexpr int mfma_ring_depth() {
#ifdef PDA_RING
  return PDA_RING;
#else
  if (mfma_waves_per_simd(D, KV, NRT) == 2) return (D == 256 || NRT == 2) ? 2 : 3;
  return D == 128 ? 3 : 2;
#endif
}

// 16-key tiles sequence b must read: those holding a key that one of its
// new tokens sees (from the first token's window start to the last key).
__device__ __forceinline__ int visible_tile_count(int L, int Qb, int window) {
  const int klo = window > 0 ? max(0, L - Qb + 1 - window) : 0;
  return max(0, (L + kPageSize - 1) / kPageSize - klo / kPageSize);
}

// Wave-wide integer sum / max through DPP within rows of 16 lanes and
// permlane swaps across rows (no LDS round trips); every lane gets the result.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_i<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_i<0x141>(v);  // row_half_mirror
  v += dpp_i<0x140>(v);  // row_mirror
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = (int)a[0] + (int)a[1];
  auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (int)c[0] + (int)c[1];
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x141>(v));
  v = max(v, dpp_i<0x140>(v));
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((int)a[0], (int)a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((int)c[0], (int)c[1]);
}
// Inclusive prefix sum over the wave's lanes: row_shr steps of 1, 2, 4, 8
// within each row of 16 (lanes shifted in from before the row read 0), then
// the totals of the rows before.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += dpp_i<0x111>(v);
  v += dpp_i<0x112>(v);
  v += dpp_i<0x114>(v);
  v += dpp_i<0x118>(v);
  const int t0 = __builtin_amdgcn_readlane(v, 15);
  const int t1 = __builtin_amdgcn_readlane(v, 31);
  const int t2 = __builtin_amdgcn_readlane(v, 47);
  const int r = lane >> 4;
  return v + (r >= 1 ? t0 : 0) + (r >= 2 ? t1 : 0) + (r >= 3 ? t2 : 0);
}

// Length-balanced chunks (automatic split count). A uniform batch (every
// sequence with the same tile count and q_len) takes the fixed split: S =
// slots / B chunks per sequence. Otherwise sequence b, with w_b tiles
// to read, is cut into n_b = max(1, ceil(w_b / C)) chunks, where C is the
// smallest chunk size (at least a.min_chunk tiles, and at least
// ceil(max_b w_b / 256) so that no row gets more than 256 partials) for which
// the chunks of all sequences fit in the grid's a.chunks slots. Slot x then
// holds chunk x - P_b of the sequence b with P_b <= x < P_b + n_b, P_b =
// n_0 + ... + n_{b-1}; slots past the last chunk hold nothing. Every
// workgroup derives the same C from seq_lens and q_lens (the host uses this
// mode only with at least two slots per sequence, so some C fits:
// with C = ceil(W / (slots - B)), W = sum of w_b, the counts add up to at most
// W / C + B <= slots, and with C >= max w_b they add up to B). A lane holds
// sequences lane + 64 k, k < NK: NK = 1 for B <= 64 (the total of at most 64
// counts of < 2^26 tiles fits in 32 bits), NK = 4 up to B = 255 (64-bit
// total).
struct BalancedChunk {
  int b, split, count, first, len, qlen, off;  // off: the sequence's first token
  bool live;
};

template <int NK>
struct BalancedLens {
  int L[NK], Q[NK];  // seq_lens / q_lens of sequences lane + 64 k (0 past the batch)
};

template <int NK>
__device__ __forceinline__ BalancedLens<NK> balanced_lens(const DecodeArgs& a, int lane) {
  // Branch-free (every lane reads an in-bounds entry, unused values are
  // discarded), so that later loads can be waited for apart from these.
  BalancedLens<NK> r;
  const int32_t* ql = a.q_lens ? a.q_lens : a.seq_lens;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int bb = lane + 64 * k;
    const bool in = bb < a.batch;
    const int bc = in ? bb : 0;
    const int Lv = a.seq_lens[bc];
    const int Qv = ql[bc];
    r.L[k] = in ? Lv : 0;
    r.Q[k] = in ? (a.q_lens ? Qv : 1) : 0;
  }
  return r;
}

template <int NK>
__device__ __forceinline__ BalancedChunk balanced_chunk(const DecodeArgs& a, int lane, int x,
                                                        const BalancedLens<NK>& ln) {
  const int B = a.batch;
  int w[NK], Ls[NK], Qs[NK];
  int wsum = 0, wmax = 0, wmin = 0x7fffffff, qmax = 0, qmin = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const bool in = lane + 64 * k < B;
    Ls[k] = ln.L[k];
    Qs[k] = ln.Q[k];
    w[k] = in ? visible_tile_count(Ls[k], Qs[k], a.window) : -1;  // -1: not a sequence
    wsum += in ? w[k] : 0;
    wmax = max(wmax, w[k]);
    wmin = in ? min(wmin, w[k]) : wmin;
    qmax = in ? max(qmax, Qs[k]) : qmax;
    qmin = in ? min(qmin, Qs[k]) : qmin;
  }
  // The reductions are wave-uniform: keep them (and the search below) in
  // scalar registers.
  wmax = __builtin_amdgcn_readfirstlane(wave_max_i(wmax));
  BalancedChunk r{0, 0, 0, 0, 0, 1, 0, false};
  // A batch whose sequences all read as many tiles, with as many new tokens:
  // the fixed split (S = slots / B chunks each, sequence x / S), which
  // balances it as well and needs no search.
  if (__builtin_amdgcn_readfirstlane(-wave_max_i(-wmin)) == wmax &&
      __builtin_amdgcn_readfirstlane(wave_max_i(qmax)) ==
          __builtin_amdgcn_readfirstlane(-wave_max_i(-qmin))) {
    const int S = a.num_splits;
    r.b = x / S;
    r.split = x - r.b * S;
    r.count = S;
    r.first = r.b * S;
    // Equal tile counts do not mean equal lengths: sequence r.b's own length
    // sits in lane r.b % 64 of Ls[r.b / 64] (r.b < B, since x < S * B).
    int Lb = Ls[0];
#pragma unroll
    for (int k = 1; k < NK; ++k) Lb = (r.b >> 6) == k ? Ls[k] : Lb;
    r.len = __builtin_amdgcn_readlane(Lb, r.b & 63);
    r.qlen = __builtin_amdgcn_readfirstlane(Qs[0]);  // one q_len for every sequence
    r.off = r.b * r.qlen;
    r.live = true;
    return r;
  }
  long long wtot;
  if constexpr (NK == 1) {
    wtot = (uint32_t)__builtin_amdgcn_readfirstlane(wave_sum_i(wsum));  // < 64 x 2^26 = 2^32
  } else {
    // Sum the high and low 16 bits apart (both sums fit) and join them.
    wtot = ((long long)__builtin_amdgcn_readfirstlane(wave_sum_i(wsum >> 16)) << 16) +
           __builtin_amdgcn_readfirstlane(wave_sum_i(wsum & 0xFFFF));
  }
  const int N = a.chunks;
  auto count_for = [&](int C, int k) {
    return w[k] < 0 ? 0 : (w[k] <= C ? 1 : (int)(((uint32_t)w[k] + C - 1) / (uint32_t)C));
  };
  auto total_for = [&](int C) {
    int n = 0;
#pragma unroll
    for (int k = 0; k < NK; ++k) n += count_for(C, k);
    return __builtin_amdgcn_readfirstlane(wave_sum_i(n));
  };
  // Any C >= max w_b gives every sequence one chunk (B <= N slots), so the
  // search stays at or below cap; below lo the chunks cannot fit.
  const int cap = max(max(wmax, a.min_chunk), 1);
  int lo, hi;
  if (wtot < 0x7FFFFFFFll) {
    const uint32_t wt = (uint32_t)wtot;
    lo = (int)min((uint32_t)cap, (wt + N - 1) / (uint32_t)N);
    hi = (int)min((uint32_t)cap, (wt + (N - B) - 1) / (uint32_t)(N - B));
  } else {
    lo = (int)min((long long)cap, (wtot + N - 1) / N);
    hi = (int)min((long long)cap, (wtot + (N - B) - 1) / (N - B));
  }
  lo = min(cap, max(max(a.min_chunk, 1), max((wmax + 255) / 256, lo)));
  hi = max(lo, hi);
  if (lo < hi && total_for(lo) <= N) hi = lo;  // the usual case: uniform and near-uniform batches
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (total_for(mid) <= N) hi = mid; else lo = mid + 1;
  }
  const int C = lo;
  int base = 0;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int n = count_for(C, k);
    const int incl = wave_incl_scan(n, lane) + base;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(w[k] >= 0 && incl > x);
    if (hit != 0) {
      const int j = (int)__builtin_ctzll(hit);
      r.b = 64 * k + j;
      r.count = __builtin_amdgcn_readlane(n, j);
      r.first = __builtin_amdgcn_readlane(incl, j) - r.count;
      r.split = x - r.first;
      r.len = __builtin_amdgcn_readlane(Ls[k], j);
      r.qlen = __builtin_amdgcn_readlane(Qs[k], j);
      r.live = true;
      break;
    }
    base = __builtin_amdgcn_readlane(incl, 63);
  }
  // Token offset of sequence b: the q_lens of the sequences before it.
  r.off = r.b;
  if (r.live && a.q_lens) {
    int q = 0;
#pragma unroll
    for (int k = 0; k < NK; ++k) q += lane + 64 * k < r.b ? Qs[k] : 0;
    r.off = __builtin_amdgcn_readfirstlane(wave_sum_i(q));
  }
  return r;
}

// STREAM: K and V by non-temporal loads (calls whose K and V exceed the
// last-level cache; see the launcher's caller).
template <int D, int KV, int NRT, bool STREAM>
__global__ void __launch_bounds__(256 * mfma_waves_per_simd(D, KV, NRT),
                                  mfma_waves_per_simd(D, KV, NRT))
pda_decode_mfma_kernel(const DecodeArgs a) {
  using Mg = MGeom<D, KV>;
  constexpr int NS = Mg::kSteps;
  constexpr int NKL = Mg::kKLoads;
  constexpr int VR = Mg::kVRaw;
  constexpr int NDT = Mg::kDTiles;
  constexpr int LR = Mg::kLdsRow;
  constexpr int NB = mfma_ring_depth<D, KV, NRT>();
  // Hold all of a page's V fragments from the tile write to P.V, except where
  // they do not fit beside the rest (two row tiles; D=256 at two waves per
  // SIMD).
  constexpr bool kHoistV = !(NRT == 2 || (D == 256 && mfma_waves_per_simd(D, KV, NRT) == 2));

  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = lane >> 4;  // lane group: keys 4s..4s+3 of a page in the scores
  const int c = lane & 15;  // key of the page (loads) / query row (scores, output)
  int split = blockIdx.x;
  const int KW = a.key_waves;   // waves sharing this KV head's key range
  const int hw = wave / KW;     // head slot of this wave in the workgroup
  const int kw = wave - hw * KW;
  const int g_raw = blockIdx.y * a.heads_per_group + hw;
  const bool head_ok = g_raw < a.num_kv_heads;  // the last group may be short
  const int g = head_ok ? g_raw : 0;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  // Token of query row r (rows are token-major, G per token): r / G, as a
  // float product: for r < 32 and G <= 32 the quotient sits at least 1/64
  // from the next integer, far beyond the reciprocal's rounding error.
  const float inv_g = 1.0f / (float)G;
  auto token_of = [&](int r) { return (int)(((float)r + 0.5f) * inv_g); };
  int S = a.num_splits;
  const int R = a.rows;  // G * max_q_len
  const size_t wave_lds = a.wave_lds_bytes;
  uint8_t* my_lds = lds_raw + (size_t)wave * wave_lds;
  _Float16* vt = reinterpret_cast<_Float16*>(my_lds);

  // Sequence of this workgroup row. In a grid of several rounds, row z takes
  // the sequence of z-th largest length (ties in index order), so the longest
  // ones are dispatched first and the short ones fill in behind them.
  int b = blockIdx.z;
  int L;
  int Qb;
  int off = b;
  bool direct = a.direct;
  int first_chunk = 0;

  // This wave's run of 16-key tiles for split `sp` of `ns_total` of a
  // sequence of L_ keys and Q_ new tokens: every tile a new token can see,
  // cut into ns_total chunks, then into one run per wave of the head.
  auto run_of = [&](int L_, int Q_, int sp, int ns_total, int& wl, int& nn) {
    const int klo = a.window > 0 ? max(0, L_ - Q_ + 1 - a.window) : 0;
    const int u_lo = klo / kPageSize;
    const int nu = max(0, (L_ + kPageSize - 1) / kPageSize - u_lo);
    const int per_split = (nu + ns_total - 1) / ns_total;
    const int s_lo = u_lo + min(nu, sp * per_split);
    const int ns = min(nu, (sp + 1) * per_split) - min(nu, sp * per_split);
    const int per_wave = KW == 1 ? ns : (ns + KW - 1) / KW;
    wl = s_lo + min(ns, kw * per_wave);
    const int wh = s_lo + min(ns, (kw + 1) * per_wave);
    nn = (L_ >= 1 && head_ok) ? wh - wl : 0;  // no key visible, or no such head
  };
  // Byte offsets of the first 2 NB - 1 tiles of a run (the ring's preload
  // and its first lookahead), clamped to the run's last tile. A "page" of
  // this loop is a tile of 16 keys; a pool page of 16 * 2^tile_shift keys
  // holds 2^tile_shift consecutive tiles. The table entries come from one
  // vector load (lane k: tile k, clamped into the run, so every lane reads an
  // entry the sequence uses) instead of 2 NB - 1 dependent scalar loads.
  typedef const __attribute__((address_space(4))) int32_t* bt_ptr_t;
  const size_t page_bytes = a.page_bytes;
  const int tshift = a.tile_shift;
  const int tmask = (1 << tshift) - 1;
  const uint32_t key_stride = a.key_stride;
  size_t pre[2 * NB - 1];
  int pre_entry = 0;  // lane k: table entry of tile k of the run
  int pre_lo = 0, pre_n = 0;
  bool pre_ok = false;
  auto fetch_pre = [&](int bb, int wl, int nn) {  // nn = 0: entry 0 of the row, unused
    pre_lo = wl;
    pre_n = nn;
    const int col = nn > 0 ? (wl + min(lane, nn - 1)) >> tshift : 0;
    pre_entry = a.block_table[(size_t)bb * a.max_pages + col];
  };
  auto fill_pre = [&]() {
#pragma unroll
    for (int k = 0; k < 2 * NB - 1; ++k) {
      const int u = pre_lo + min(k, pre_n - 1);
      pre[k] = (size_t)__builtin_amdgcn_readlane(pre_entry, k) * page_bytes +
               (size_t)((u & tmask) * kPageSize) * key_stride;
    }
  };

  if (a.balanced) {
    BalancedChunk ch;
    if (a.batch <= 64) {
      const BalancedLens<1> ln = balanced_lens<1>(a, lane);
      // While the lengths for the search are in flight, take the chunk a
      // uniform batch would give this slot (sequence x / S, split x % S) and
      // fetch its first table entries; they are used if the search agrees.
      const int Sg = a.num_splits;
      const int bg = (int)blockIdx.x / Sg;
      const int sg = (int)blockIdx.x - bg * Sg;
      int wlg, ng;
      const int32_t* ql = a.q_lens ? a.q_lens : a.seq_lens;
      const int Lg = a.seq_lens[bg], Qg = ql[bg];
      run_of(Lg, a.q_lens ? Qg : 1, sg, Sg, wlg, ng);
      fetch_pre(bg, wlg, ng);
      ch = balanced_chunk<1>(a, lane, blockIdx.x, ln);
      pre_ok = ng > 0 && ch.b == bg && ch.split == sg && ch.count == Sg;
    } else {
      ch = balanced_chunk<4>(a, lane, blockIdx.x, balanced_lens<4>(a, lane));
    }
    if (!ch.live) return;  // a slot past the last chunk (uniform over the workgroup)
    // All wave-uniform: keep them in scalar registers.
    b = __builtin_amdgcn_readfirstlane(ch.b);
    L = __builtin_amdgcn_readfirstlane(ch.len);
    Qb = __builtin_amdgcn_readfirstlane(ch.qlen);
    split = __builtin_amdgcn_readfirstlane(ch.split);
    S = __builtin_amdgcn_readfirstlane(ch.count);
    first_chunk = __builtin_amdgcn_readfirstlane(ch.first);
    direct = S == 1;
    off = __builtin_amdgcn_readfirstlane(ch.off);
  } else if (a.longest_first) {
    const int B = a.batch;
    const int my_len = lane < B ? a.seq_lens[lane] : -1;
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int lj = __builtin_amdgcn_readlane(my_len, j);
      rank += (lj > my_len || (lj == my_len && j < lane)) ? 1 : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && rank == (int)blockIdx.z);
    b = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
    L = __builtin_amdgcn_readlane(my_len, b);
  } else {
    // The token offset (q_lens of the sequences before b) is loaded
    // together with the length.
    int sum = 0;
    if (a.q_lens)
      for (int i = lane; i < b; i += 64) sum += a.q_lens[i];
    L = a.seq_lens[b];
    off = a.q_lens ? __builtin_amdgcn_readfirstlane(wave_sum_i(sum)) : b;
  }
  if (!a.balanced) Qb = a.q_lens ? a.q_lens[b] : 1;
  if (a.longest_first) {
    off = b;  // the token offset with one token per sequence
    if (a.q_lens) {
      int sum = 0;
      for (int i = lane; i < b; i += 64) sum += a.q_lens[i];
      off = __builtin_amdgcn_readfirstlane(wave_sum_i(sum));
    }
  }
  const int pos0 = L - Qb;
  // Balanced splits: the sequence's first workgroup records where the combine
  // finds each of its tokens' partials.
  if (a.balanced && split == 0 && blockIdx.y == 0 && wave == 0 && lane < Qb)
    *reinterpret_cast<int4*>(a.meta + 4 * (size_t)(off + lane)) = int4{first_chunk, S, lane, 0};

  // This wave's run of tiles.
  int w_lo, n;
  run_of(L, Qb, split, S, w_lo, n);

  // Visibility bounds: uniform summary over the real rows (fast-path test),
  // and this lane's own rows (16 * rt + c) for masked pages. Token i sits at
  // pos0 + i; the first token that sees a key is i_lo = max(0, -pos0), the
  // last one (position L - 1) has the latest window start.
  const int hi_min = max(pos0, 0);
  const int lo_max = a.window > 0 ? max(0, L - a.window) : 0;
  int lo_c[NRT], hi_c[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int row = 16 * rt + c;
    const int i = token_of(row);
    const int pos = pos0 + i;
    const bool active = row < R && i < Qb && pos >= 0;
    lo_c[rt] = active ? (a.window > 0 ? max(0, pos - a.window + 1) : 0) : 0;
    hi_c[rt] = active ? pos : -1;
  }

  // Addresses. Within a page, slot j of head g starts at j * key_stride + g
  // * head_stride (NHD: key_stride = Hkv * row, head_stride = row; HND:
  // key_stride = row, head_stride = P * row).
  const uint32_t head_off = (uint32_t)g * a.head_stride;
  const uint32_t koff = (uint32_t)c * key_stride + head_off + 16u * s;
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    voff[i] = (uint32_t)(s + 4 * i) * key_stride + head_off + lane_piece_offset<D, KV>(c);
  const bt_ptr_t bt = (bt_ptr_t)(a.block_table + (size_t)b * a.max_pages);
  if (!pre_ok && n > 0) fetch_pre(b, w_lo, n);
  if (n > 0) fill_pre();
  // Byte offset of the k-th tile of this wave's run (clamped to the last).
  auto pid_of = [&](int k) -> size_t {
    const int u = w_lo + min(k, n - 1);
    return (size_t)bt[u >> tshift] * page_bytes +
           (size_t)((u & tmask) * kPageSize) * key_stride;
  };

  auto load_page = [&](uint32_t (&kr)[NKL][4], uint32_t (&vr)[4][VR], size_t base) {
    const uint8_t* kp = a.k + base;
    const uint8_t* vp = a.v + base;
#pragma unroll
    for (int t = 0; t < NKL; ++t) {
      const u32x4 x = ld_global<STREAM, u32x4>(kp + koff + 64 * t);
#pragma unroll
      for (int e = 0; e < 4; ++e) kr[t][e] = x[e];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) load_slice<D, KV, VR, STREAM>(vr[i], vp + voff[i]);
  };

  uint32_t kb[NB][NKL][4], vb[NB][4][VR];
  if (n > 0) {
#pragma unroll
    for (int st = 0; st < NB - 1; ++st) load_page(kb[st], vb[st], pre[st]);
  }

  // Q^T as the B operand: lane (s, c) holds row 16 rt + c, dims of step t in
  // the same order as its K slice. A negative scale flips q's sign.
  float qk = a.qk_mult * (a.k_scale ? a.k_scale[g] : 1.0f);
  const uint32_t qflip = qk < 0.0f ? 0x80008000u : 0u;
  qk = fabsf(qk);
  h8_t qb[NRT][NS];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int row = 16 * rt + c;
    const int i = token_of(row);
    const bool exists = head_ok && row < R && i < Qb;
    const uint8_t* qrow = a.q + ((size_t)(off + i) * Hq + g * G + (row - i * G)) * (D * 2);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      // fp16 KV: step t covers K bytes 64t + 16s (dims 32t + 8s ..);
      // 1-byte KV: K bytes 64(t/2) + 16s hold dims 64(t/2) + 16s + 8(t%2) ...
      const int qbyte = KV == kKvF16 ? 64 * t + 16 * s : 128 * (t / 2) + 32 * s + 16 * (t % 2);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (exists) x = *reinterpret_cast<const u32x4*>(qrow + qbyte);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] ^= qflip;
      qb[rt][t] = __builtin_bit_cast(h8_t, x);
    }
  }

  // Online softmax with a lazily moved reference: p = 2^(score - m) with m a
  // reference that trails the row's running maximum mx by at most kLazy (so
  // p <= 2^kLazy, well inside fp16), and o, l are rescaled only when mx gets
  // further ahead than that. The result is the same function; after the last
  // page o and l are brought to m = mx once, so a split's m is its maximum.
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

  auto process_page = [&](uint32_t (&kr)[NKL][4], uint32_t (&vr)[4][VR], int u) {
    const int j0 = u * kPageSize;
    const bool full = j0 >= lo_max && j0 + kPageSize - 1 <= hi_min;

    // V rows past the sequence end are zeroed (their contents are arbitrary),
    // then the page's V goes to this wave's LDS tile as fp16 rows.
    if (!full) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j0 + 4 * i + s >= L) {
#pragma unroll
          for (int e = 0; e < VR; ++e) vr[i][e] = 0u;
        }
    }
    // With 1-byte codes at D=256 a lane's 16 B of codes are the 16 dims of
    // output tile c, widened to 32 B and written in two 16-byte halves. A
    // 16-byte write is served 8 lanes (128 bytes) at a time, and in row order
    // lanes c and c + 4 of those 8 would share banks; tiles with c & 4 keep
    // their two 8-dim halves swapped, so each write's 8 lanes fall on distinct
    // banks. The transposing reads of those tiles undo the swap.
    constexpr bool kSwap = KV != kKvF16 && D == 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h2_t vh[D / 32];
      to_pairs<KV>(vr[i], vh);
      _Float16* row = vt + (4 * i + s) * LR;
#pragma unroll
      for (int e8 = 0; e8 < D / 128; ++e8) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(uint32_t, vh[4 * e8 + e]);
        const int d0 = kSwap ? 16 * c + 8 * (e8 ^ ((c >> 2) & 1)) : dim_of<D, KV>(c, 8 * e8);
        *reinterpret_cast<u32x4*>(row + d0) = w;
      }
    }

    // The A operand of P.V (lane (s, c): V[4s + k][16 dt + c], k = 0..3) comes
    // from the row-major tile with one transposing read per 16 dims: within
    // each 16-lane group, ds_read_b64_tr_b16 hands lane i element i % 4 of the
    // 8-byte rows addressed by lanes i/4 + 4k, so lane (s, c) points at row
    // 4s + c/4, dims 16 dt + 4 (c % 4) .. + 3 (in a swapped tile, 8 halves
    // further or back). Where registers allow, all
    // reads are issued here, so their latency hides behind the scores and the
    // softmax; the scheduling barrier keeps the compiler from sinking them
    // next to their uses (which serializes one LDS round trip per read).
    typedef short s4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4_t lds_s4_t;
    auto read_va = [&](int dt) -> h4_t {
      const int col = (4 * (c & 3)) ^ (kSwap && (dt & 4) ? 8 : 0);
      _Float16* src = vt + (4 * s + (c >> 2)) * LR + 16 * dt + col;
      return __builtin_bit_cast(h4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                          (lds_s4_t*)(__attribute__((address_space(3))) _Float16*)src));
    };
    h4_t va[kHoistV ? NDT : 1];
    if constexpr (kHoistV) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) va[dt] = read_va(dt);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Scores S^T[key 4s+i][row c] for every row tile.
    h8_t ka[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if constexpr (KV == kKvF16) {
        ka[t] = __builtin_bit_cast(h8_t, u32x4{kr[t][0], kr[t][1], kr[t][2], kr[t][3]});
      } else {
        uint32_t raw[2] = {kr[t / 2][2 * (t % 2)], kr[t / 2][2 * (t % 2) + 1]};
        h2_t kh[4];
        to_pairs<KV>(raw, kh);
        ka[t] = __builtin_bit_cast(h8_t, u32x4{__builtin_bit_cast(uint32_t, kh[0]),
                                                __builtin_bit_cast(uint32_t, kh[1]),
                                                __builtin_bit_cast(uint32_t, kh[2]),
                                                __builtin_bit_cast(uint32_t, kh[3])});
      }
    }
    f4_t sc[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      sc[rt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < NS; ++t)
        sc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[t], qb[rt][t], sc[rt], 0, 0, 0);
    }

    // Online softmax per row (lane-local row c; the max crosses lane groups).
    auto visible = [&](int rt, int i) {
      const int j = j0 + 4 * s + i;
      return j >= lo_c[rt] && j <= hi_c[rt];
    };
    bool behind = false;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      float mt;
      if (full) {
        mt = qk * max4(fmaxf(fmaxf(sc[rt][0], sc[rt][1]), fmaxf(sc[rt][2], sc[rt][3])));
      } else {
        mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, visible(rt, i) ? sc[rt][i] : -INFINITY);
        mt = max4(mt);
        mt = mt == -INFINITY ? kNoMax : qk * mt;
      }
      mx[rt] = fmaxf(mx[rt], mt);
      behind |= mx[rt] > m[rt] + kLazy;
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
      // Every p is computed; only partial pages then zero the hidden ones
      // (a wave-uniform branch around selects, none on full pages).
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[rt][i], qk, -m[rt]));
      if (!full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = visible(rt, i) ? p[i] : 0.0f;
      }
      pb[rt] = h4_t{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
      // The denominator adds the same fp16 weights that P.V multiplies V by
      // (v_dot2 with ones: each fp16 value enters the fp32 sum exactly), so
      // numerator and denominator weigh every key alike.
      const h2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
      l[rt] = __builtin_amdgcn_fdot2(h2_t{pb[rt][0], pb[rt][1]}, one2,
                                     __builtin_amdgcn_fdot2(h2_t{pb[rt][2], pb[rt][3]}, one2,
                                                            l[rt], false),
                                     false);
    }

    // O^T[dims][rows] += V^T . P^T. Without room to hold every V fragment,
    // they are read in batches of 8 (4 with two row tiles), one LDS wait per
    // batch.
    if constexpr (kHoistV) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
          o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[dt], pb[rt], o[rt][dt], 0, 0, 0);
    } else {
      constexpr int VB = NRT == 2 ? 4 : (NDT < 8 ? NDT : 8);
#pragma unroll
      for (int d0 = 0; d0 < NDT; d0 += VB) {
        h4_t vb8[VB];
#pragma unroll
        for (int j = 0; j < VB; ++j) vb8[j] = read_va(d0 + j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < VB; ++j)
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
            o[rt][d0 + j] =
                __builtin_amdgcn_mfma_f32_16x16x16f16(vb8[j], pb[rt], o[rt][d0 + j], 0, 0, 0);
      }
    }
  };

  if (n > 0) {
    size_t pid_s[NB];
#pragma unroll
    for (int st = 0; st < NB; ++st) pid_s[st] = pre[NB - 1 + st];
    const int n_main = n - n % NB;
    for (int it = 0; it < n_main; it += NB) {
#pragma unroll
      for (int st = 0; st < NB; ++st) {
        const int k_issue = it + st + NB - 1;
        load_page(kb[(st + NB - 1) % NB], vb[(st + NB - 1) % NB], pid_s[st]);
        pid_s[st] = pid_of(k_issue + NB);
        process_page(kb[st], vb[st], w_lo + it + st);
      }
    }
#pragma unroll
    for (int st = 0; st < NB - 1; ++st)
      if (n_main + st < n) process_page(kb[st], vb[st], w_lo + n_main + st);
  }

  // Bring o and l to the row maximum (m = mx unless the reference trails),
  // then sum the denominators over the 4 lane groups; m and mx are already
  // the same in them.
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float alpha = __builtin_amdgcn_exp2f(m[rt] - mx[rt]);
    l[rt] *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rt][dt] *= alpha;
    m[rt] = mx[rt];
    l[rt] = add4(l[rt]);
  }

  // Partial record of (head slot hs, row = i * G + j) for token i of this
  // sequence: rec_a(hs) + row * rec_b + i * rec_c. Fixed split count: record
  // ((off + i) * Hq + head * G + j) * S + split. Balanced splits: record
  // (head * R + row) * chunks + slot, so a row's chunks are adjacent.
  const size_t rec_b = a.balanced ? (size_t)a.chunks : (size_t)S;
  const size_t rec_c = a.balanced ? 0 : (size_t)(Hq - G) * S;
  auto rec_a = [&](int hs) -> size_t {
    const size_t gg = (size_t)blockIdx.y * a.heads_per_group + hs;
    return a.balanced ? gg * R * a.chunks + blockIdx.x : ((size_t)off * Hq + gg * G) * S + split;
  };

  // One wave per head: write the result from registers (lane (s, c) holds
  // row 16 rt + c, dims 16 dt + 4 s .. + 3).
  if (KW == 1) {
    if (!head_ok) return;
    const float vs = a.v_scale ? a.v_scale[g] : 1.0f;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int row = 16 * rt + c;
      const int i = token_of(row);
      if (row >= R || i >= Qb) continue;
      const size_t hrow = (size_t)(off + i) * Hq + g * G + (row - i * G);
      const float lsum = l[rt];
      if (direct) {
        uint16_t* dst = a.out + hrow * D + 4 * s;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          h4_t y;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            y[e] = lsum > 0.0f ? (_Float16)((o[rt][dt][e] * vs) / lsum) : (_Float16)0.0f;
          *reinterpret_cast<h4_t*>(dst + 16 * dt) = y;
        }
      } else {
        const size_t prow = rec_a(hw) + (size_t)row * rec_b + (size_t)i * rec_c;
        float* dst = a.part_o + prow * D + 4 * s;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f4_t*>(dst + 16 * dt) = o[rt][dt] * vs;
        if (s == 0) {
          a.part_ml[prow * 2] = lsum > 0.0f ? m[rt] : -INFINITY;
          a.part_ml[prow * 2 + 1] = lsum;
        }
      }
    }
    return;
  }

  // Several waves per head: merge them through LDS; per wave, rows [R] of
  // (m, l, -, -, o[D]).
  __syncthreads();  // every wave is done with its V tile (the region aliases)
  float* wm = reinterpret_cast<float*>(my_lds);
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int row = 16 * rt + c;
    if (row < R) {
      float* rec = wm + (size_t)row * (D + 4);
      if (s == 0) { rec[0] = m[rt]; rec[1] = l[rt]; }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f4_t*>(rec + 4 + 16 * dt + 4 * s) = o[rt][dt];
    }
  }
  __syncthreads();

  const int HPW = a.heads_per_group;
  for (int idx = threadIdx.x; idx < HPW * R * D; idx += blockDim.x) {
    const int hs = idx / (R * D);
    const int rem = idx - hs * (R * D);
    const int row = rem / D;
    const int d = rem - row * D;
    const int gg = blockIdx.y * HPW + hs;
    const int i = token_of(row);
    if (gg >= a.num_kv_heads || i >= Qb) continue;
    const int h = gg * G + (row - i * G);
    const int t = off + i;
    const int w0 = hs * KW;
    float M = -INFINITY;
    for (int w = w0; w < w0 + KW; ++w)
      M = fmaxf(M, reinterpret_cast<const float*>(lds_raw + (size_t)w * wave_lds)[(size_t)row * (D + 4)]);
    float lsum = 0.0f, osum = 0.0f;
    for (int w = w0; w < w0 + KW; ++w) {
      const float* rec = reinterpret_cast<const float*>(lds_raw + (size_t)w * wave_lds) +
                         (size_t)row * (D + 4);
      const float wt = __builtin_amdgcn_exp2f(rec[0] - M);
      lsum += wt * rec[1];
      osum += wt * rec[4 + d];
    }
    osum *= a.v_scale ? a.v_scale[gg] : 1.0f;
    if (direct) {
      const _Float16 y = lsum > 0.0f ? (_Float16)(osum / lsum) : (_Float16)0.0f;
      a.out[((size_t)t * Hq + h) * D + d] = __builtin_bit_cast(uint16_t, y);
    } else {
      const size_t prow = rec_a(hs) + (size_t)row * rec_b + (size_t)i * rec_c;
      a.part_o[prow * D + d] = osum;
      if (d == 0) {
        a.part_ml[prow * 2] = lsum > 0.0f ? M : -INFINITY;
        a.part_ml[prow * 2 + 1] = lsum;
      }
    }
  }
}

template <int KV>
hipError_t launch_mfma_kv(int head_dim, int row_tiles, bool stream_kv, dim3 grid, int threads, size_t lds,
                          hipStream_t stream, const DecodeArgs& args) {
#define PDA_MCASE(DD, NT, ST)                                                              \
  if (head_dim == DD && row_tiles == NT && stream_kv == ST) {                              \
    hipLaunchKernelGGL((pda_decode_mfma_kernel<DD, KV, NT, ST>), grid, dim3(threads), lds, \
                       stream, args);                                                      \
    return hipGetLastError();                                                              \
  }
  PDA_MCASE(128, 1, false)
  PDA_MCASE(128, 2, false)
  PDA_MCASE(256, 1, false)
  PDA_MCASE(256, 2, false)
  PDA_MCASE(128, 1, true)
  PDA_MCASE(128, 2, true)
  PDA_MCASE(256, 1, true)
  PDA_MCASE(256, 2, true)
#undef PDA_MCASE
  return hipErrorInvalidValue;
}

}  // namespace pda
