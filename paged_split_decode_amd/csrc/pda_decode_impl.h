// Paged split-K decode attention kernel for gfx950 (CDNA4, wave64).
//
// The computation is the per-head paged split-K decode kernel of vllm-rdna
// pull request #33 ("perf(rocm): FA-RDNA2 decode, scores on every wave and 4
// barriers per tile", section "Purpose"): softmax(scale * q.K^T) . V per query
// head over a paged KV cache, the key axis split across workgroups, partials
// merged by a combine kernel. The gfx1030 wave32 schedule described there is
// prior art; this is the wave64 design:
//
//  * One workgroup per (split, KV head, sequence). It carries every query row
//    of that KV head's GQA group (G heads x the sequence's new tokens); the
//    rows stay in registers (the pull request also keeps Q out of LDS).
//    Waves are arranged as row_groups x key_waves: waves of one row group
//    share rows and split the workgroup's key range; row groups split rows
//    when a group has more than 8 of them and share keys.
//  * Each wave owns a contiguous run of key "units" (one page, or half a page
//    at D=256 fp16) with its own online softmax: no barrier and no LDS
//    traffic per tile. 16 lanes share one key row (16-byte loads, so a
//    16-lane group reads 256 contiguous bytes), 4 keys per instruction, and
//    the next unit's K and V are loaded while the current one is computed;
//    block-table entries are read two units ahead.
//  * Scores: packed fp16 v_dot2 with fp32 accumulation (the pull request's
//    "packed fdot2"), then a 4-step DPP butterfly over the 16 lanes of a key.
//    The tile max crosses the 4 key groups of a wave with permlane16/32 swaps.
//  * P.V: each lane accumulates its own dims over its group's keys in fp32
//    (fp16 V operands feed v_fma_mix directly); key groups and waves merge
//    once per workgroup, through LDS, at the end ("l accumulates per wave and
//    is summed once per CTA" in the pull request; here o is merged the same
//    way).
//  * fp8-e4m3 and int8 KV are converted to fp16 pairs in registers (exact)
//    and run the same bodies; their per-KV-head scales fold into the score
//    multiplier (K) and the output (V).
//  * Masking (sequence length, causal position of each new token, sliding
//    window) happens by select on units that are not entirely visible; V rows
//    past the sequence end are zeroed so that poison there cannot leak
//    through p = 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda_kernels.h"

namespace pda {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D, int KV>
struct Geom {
  static constexpr int kElemBytes = KV == kKvF16 ? 2 : 1;
  static constexpr int kDimsPerLane = D / kLanesPerKey;         // 8 or 16
  static constexpr int kLaneBytes = kDimsPerLane * kElemBytes;  // 8..32
  static constexpr int kRawDwords = kLaneBytes / 4;             // 2..8
  static constexpr int kPairs = kDimsPerLane / 2;               // fp16 pairs
  static constexpr int kKeyIters = key_iters(D, KV);
  static constexpr int kUnitKeys = 4 * kKeyIters;
  static constexpr int kUnitsPerPage = kPageSize / kUnitKeys;
  static constexpr int kRowBytes = D * kElemBytes;
  static_assert(kPageSize % kUnitKeys == 0, "unit must divide a page");
};

// Global dim of lane-local element e for the lane at key-chunk c.
// Units of K+V kept in flight per wave (registers: 32 dwords per unit, 16
// for 1-byte KV at D=128).
constexpr int pipeline_stages(int D, int KV, int RW) {
  return (D == 128 && RW <= 4) ? 3 : 2;
}

template <int D, int KV>
__device__ __forceinline__ int dim_of(int c, int e) {
  if constexpr (KV == kKvF16 && D == 256) {
    return e < 8 ? 8 * c + e : 128 + 8 * c + (e - 8);
  } else {
    return Geom<D, KV>::kDimsPerLane * c + e;
  }
}

// ---------------------------------------------------------------------------
// Cross-lane helpers
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane gets the same bits.
__device__ __forceinline__ float sum16(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

// Max / sum over the 4 rows of 16 lanes (the 4 key groups of a wave).
__device__ __forceinline__ float max4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x),
                                            __builtin_bit_cast(int, x), false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                            __builtin_bit_cast(int, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)b[0]), __builtin_bit_cast(float, (int)b[1]));
}

__device__ __forceinline__ float add4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x),
                                            __builtin_bit_cast(int, x), false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                            __builtin_bit_cast(int, x), false, false);
  return __builtin_bit_cast(float, (int)b[0]) + __builtin_bit_cast(float, (int)b[1]);
}

__device__ __forceinline__ int wave_sum_int(int x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// ---------------------------------------------------------------------------
// Element conversion: NR raw dwords of one key row slice -> fp16 pairs
// ---------------------------------------------------------------------------

template <int KV, int NR, int NO>
__device__ __forceinline__ void to_pairs(const uint32_t (&raw)[NR], h2_t (&out)[NO]) {
  static_assert(NO == (KV == kKvF16 ? NR : 2 * NR), "pair count");
  if constexpr (KV == kKvF16) {
#pragma unroll
    for (int j = 0; j < NR; ++j) out[j] = __builtin_bit_cast(h2_t, raw[j]);
  } else if constexpr (KV == kKvFp8) {
    // OCP E4M3 -> fp16 is exact (every E4M3 value is an fp16 value).
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      out[2 * j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[j], 1.0f, false);
      out[2 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[j], 1.0f, true);
    }
  } else {
    // int8 b -> fp16 with bit pattern 0x6400 | (b ^ 0x80), i.e. 1152 + b,
    // then subtract 1152: exact for every code.
    const h2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const uint32_t x = raw[j] ^ 0x80808080u;
      const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
      const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
      out[2 * j] = __builtin_bit_cast(h2_t, lo) - bias;
      out[2 * j + 1] = __builtin_bit_cast(h2_t, hi) - bias;
    }
  }
}

// Byte offset of this lane's first 16-byte (8-byte for 1-byte KV at D=128)
// piece within a key row; fp16 at D=256 has a second piece 256 bytes later.
template <int D, int KV>
__device__ __forceinline__ uint32_t lane_piece_offset(int c) {
  return (uint32_t)(Geom<D, KV>::kLaneBytes == 8 ? 8 * c : 16 * c);
}

// A global load, non-temporal when NTL (the data is read once: streaming
// loads then keep it from displacing other lines in the caches).
template <bool NTL, typename T>
__device__ __forceinline__ T ld_global(const uint8_t* p) {
  if constexpr (NTL)
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else
    return *reinterpret_cast<const T*>(p);
}

// Load this lane's slice of one key row (K or V); `p` points at its first piece.
template <int D, int KV, int N, bool NTL = false>
__device__ __forceinline__ void load_slice(uint32_t (&dst)[N], const uint8_t* p) {
  using Gm = Geom<D, KV>;
  static_assert(N == Gm::kRawDwords, "slice size");
  if constexpr (Gm::kLaneBytes == 32) {  // fp16, D=256: two 256-byte halves
    const u32x4 a = ld_global<NTL, u32x4>(p);
    const u32x4 b = ld_global<NTL, u32x4>(p + 256);
#pragma unroll
    for (int j = 0; j < 4; ++j) { dst[j] = a[j]; dst[4 + j] = b[j]; }
  } else if constexpr (Gm::kLaneBytes == 16) {
    const u32x4 a = ld_global<NTL, u32x4>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = a[j];
  } else {  // 1-byte, D=128
    const u32x2 a = ld_global<NTL, u32x2>(p);
    dst[0] = a[0];
    dst[1] = a[1];
  }
}

// Load this lane's query slice (fp16, same dims as its K slice) of one row.
template <int D, int KV, int N>
__device__ __forceinline__ void load_q(uint32_t (&dst)[N], const uint8_t* qrow, int c) {
  static_assert(N == Geom<D, KV>::kPairs, "query slice size");
  if constexpr (KV == kKvF16 && D == 256) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(qrow + 16 * c);
    const u32x4 b = *reinterpret_cast<const u32x4*>(qrow + 256 + 16 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) { dst[j] = a[j]; dst[4 + j] = b[j]; }
  } else if constexpr (D == 256) {  // 1-byte KV: dims 16c..16c+15
    const u32x4 a = *reinterpret_cast<const u32x4*>(qrow + 32 * c);
    const u32x4 b = *reinterpret_cast<const u32x4*>(qrow + 32 * c + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) { dst[j] = a[j]; dst[4 + j] = b[j]; }
  } else {  // D=128: dims 8c..8c+7
    const u32x4 a = *reinterpret_cast<const u32x4*>(qrow + 16 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = a[j];
  }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <int D, int KV, int RW>
__global__ void __launch_bounds__(512) pda_decode_kernel(const DecodeArgs a) {
  constexpr int NB = pipeline_stages(D, KV, RW);
  using Gm = Geom<D, KV>;
  constexpr int DPL = Gm::kDimsPerLane;
  constexpr int NR = Gm::kRawDwords;
  constexpr int NP = Gm::kPairs;
  constexpr int KI = Gm::kKeyIters;
  constexpr int UK = Gm::kUnitKeys;
  constexpr int UPP = Gm::kUnitsPerPage;

  extern __shared__ float lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane >> 4;  // key group within the wave
  const int c = lane & 15;     // 16-byte chunk of the key row
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int nrg = a.row_groups;
  const int rg = wave % nrg;
  const int kw = wave / nrg;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int S = a.num_splits;

  const int L = a.seq_lens[b];
  const int Qb = a.q_lens ? a.q_lens[b] : 1;
  int off = b;
  if (a.q_lens) {
    int sum = 0;
    for (int i = lane; i < b; i += 64) sum += a.q_lens[i];
    off = wave_sum_int(sum);
  }
  const int pos0 = L - Qb;  // position of the sequence's first new token

  // Keys any new token can see: [klo, L). Cut into units, then into
  // `num_splits` contiguous chunks, then into `key_waves` runs per chunk.
  const int klo = a.window > 0 ? max(0, pos0 + 1 - a.window) : 0;
  const int u_lo = klo / UK;
  const int nu = max(0, (L + UK - 1) / UK - u_lo);
  const int per_split = (nu + S - 1) / S;
  const int s_lo = u_lo + min(nu, split * per_split);
  const int ns = min(nu, (split + 1) * per_split) - min(nu, split * per_split);
  const int per_wave = (ns + a.key_waves - 1) / a.key_waves;
  const int w_lo = s_lo + min(ns, kw * per_wave);
  int w_hi = s_lo + min(ns, (kw + 1) * per_wave);

  // Rows of this wave: row r is new token i = gr / G, head g*G + gr % G.
  // A row is "active" when its token exists and sees at least one key.
  int lo_r[RW], hi_r[RW];
  int lo_max = 0, hi_min = 0x7fffffff;
  bool any_active = false;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int i = (rg * RW + r) / G;
    const int pos = pos0 + i;
    const bool active = i < Qb && pos >= 0;
    lo_r[r] = active ? (a.window > 0 ? max(0, pos - a.window + 1) : 0) : 0;
    hi_r[r] = active ? pos : -1;
    if (active) {
      lo_max = max(lo_max, lo_r[r]);
      hi_min = min(hi_min, hi_r[r]);
      any_active = true;
    }
  }
  if (!any_active) w_hi = w_lo;
  const int n = w_hi - w_lo;

  // Addresses: a uniform (SGPR) page pointer per unit plus per-lane 32-bit
  // offsets computed once.
  const uint32_t key_stride = (uint32_t)a.num_kv_heads * Gm::kRowBytes;
  const size_t page_bytes = (size_t)kPageSize * key_stride;
  uint32_t loff[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i)
    loff[i] = (uint32_t)(slot + 4 * i) * key_stride + (uint32_t)g * Gm::kRowBytes +
              lane_piece_offset<D, KV>(c);
  // Block-table row read through the constant address space: scalar loads,
  // waited on with lgkmcnt, independent of the vector-load pipeline.
  typedef const __attribute__((address_space(4))) int32_t* bt_ptr_t;
  const bt_ptr_t bt = (bt_ptr_t)(a.block_table + (size_t)b * a.max_pages);
  // Page id of the wave's k-th unit (clamped to its last unit, whose
  // repeated reads hit in cache).
  auto pid_of = [&](int k) -> int { return bt[(w_lo + min(k, n - 1)) / UPP]; };

  auto load_unit = [&](uint32_t (&kr)[KI][NR], uint32_t (&vr)[KI][NR], int pid, int u) {
    const size_t base = (size_t)pid * page_bytes + (size_t)(u % UPP) * UK * key_stride;
    const uint8_t* kp = a.k + base;
    const uint8_t* vp = a.v + base;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      load_slice<D, KV>(kr[i], kp + loff[i]);
      load_slice<D, KV>(vr[i], vp + loff[i]);
    }
  };

  // First NB-1 units of K and V go out before anything else waits on memory.
  uint32_t kb[NB][KI][NR], vb[NB][KI][NR];
  if (n > 0) {
#pragma unroll
    for (int st = 0; st < NB - 1; ++st) load_unit(kb[st], vb[st], pid_of(st), w_lo + min(st, n - 1));
  }

  // Query rows (fp16, this lane's dims). Scores stay unscaled; the scale
  // (times log2 e, times the K scale for quantized KV) enters through the
  // exponent. A negative scale is folded into q's sign so that the running
  // max of unscaled scores is the max of scaled ones.
  float qk = a.qk_mult * (a.k_scale ? a.k_scale[g] : 1.0f);
  const uint32_t qflip = qk < 0.0f ? 0x80008000u : 0u;
  qk = fabsf(qk);
  uint32_t qr[RW][NP];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int gr = rg * RW + r;
    const int i = gr / G;
    if (i < Qb) {
      const uint8_t* qrow = a.q + ((size_t)(off + i) * Hq + g * G + (gr - i * G)) * (D * 2);
      load_q<D, KV>(qr[r], qrow, c);
#pragma unroll
      for (int j = 0; j < NP; ++j) qr[r][j] ^= qflip;
    } else {
#pragma unroll
      for (int j = 0; j < NP; ++j) qr[r][j] = 0u;
    }
  }

  // Running state. kNoMax is a finite stand-in for "no key yet": it keeps
  // exp2(m - m_new) finite and equal to 1 while a row has seen nothing.
  constexpr float kNoMax = -1e30f;
  float m[RW], l[RW], o[RW][DPL];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    m[r] = kNoMax;
    l[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[r][e] = 0.0f;
  }

  auto process_unit = [&](uint32_t (&kr)[KI][NR], uint32_t (&vr)[KI][NR], int u) {
    float s[KI][RW];  // raw q.k, then p
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      h2_t kh[NP];
      to_pairs<KV>(kr[i], kh);
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NP; ++j)
          acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, qr[r][j]), kh[j], acc, false);
        s[i][r] = sum16(acc);
      }
    }

    bool rescale = false;
    float alpha[RW];
    const int j0 = u * UK;
    if (j0 >= lo_max && j0 + UK - 1 <= hi_min) {
      // Every key of the unit is visible to every active row.
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        float mt = s[0][r];
#pragma unroll
        for (int i = 1; i < KI; ++i) mt = fmaxf(mt, s[i][r]);
        const float mn = fmaxf(m[r], qk * max4(mt));
        alpha[r] = __builtin_amdgcn_exp2f(m[r] - mn);
        rescale |= mn != m[r];
        m[r] = mn;
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          s[i][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i][r], qk, -mn));
          ps += s[i][r];
        }
        l[r] = __builtin_fmaf(l[r], alpha[r], ps);
      }
    } else {
      // Boundary unit: per-key visibility by select (never by arithmetic, so
      // poison past the sequence end cannot leak), V rows past the end zeroed.
      bool valid[KI][RW];
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int j = j0 + 4 * i + slot;
#pragma unroll
        for (int r = 0; r < RW; ++r) valid[i][r] = j >= lo_r[r] && j <= hi_r[r];
        if (j >= L) {
#pragma unroll
          for (int e = 0; e < NR; ++e) vr[i][e] = 0u;
        }
      }
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < KI; ++i) mt = fmaxf(mt, valid[i][r] ? s[i][r] : -INFINITY);
        mt = max4(mt);
        const float mn = fmaxf(m[r], mt == -INFINITY ? kNoMax : qk * mt);
        alpha[r] = __builtin_amdgcn_exp2f(m[r] - mn);
        rescale |= mn != m[r];
        m[r] = mn;
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i][r], qk, -mn));
          s[i][r] = valid[i][r] ? p : 0.0f;
          ps += s[i][r];
        }
        l[r] = __builtin_fmaf(l[r], alpha[r], ps);
      }
    }
    // m is the same in every lane, so the ballot is all or nothing: a scalar branch.
    if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[r][e] *= alpha[r];
    }
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      h2_t vh[NP];
      to_pairs<KV>(vr[i], vh);
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const float p = s[i][r];
#pragma unroll
        for (int e = 0; e < DPL; ++e)
          o[r][e] = __builtin_fmaf(p, (float)vh[e >> 1][e & 1], o[r][e]);
      }
    }
  };

  if (n > 0) {
    // NB-stage ring of units in registers: the loads of unit k + NB - 1 are
    // issued before unit k is computed; page ids are fetched NB units before
    // the loads that use them.
    int pid_s[NB];
#pragma unroll
    for (int st = 0; st < NB; ++st) pid_s[st] = pid_of(NB - 1 + st);
    // Whole groups of NB units: straight-line bodies, so the ring stays in
    // fixed registers and the loads stay in flight across units.
    const int n_main = n - n % NB;
    for (int it = 0; it < n_main; it += NB) {
#pragma unroll
      for (int st = 0; st < NB; ++st) {
        const int k_issue = it + st + NB - 1;
        load_unit(kb[(st + NB - 1) % NB], vb[(st + NB - 1) % NB], pid_s[st],
                  w_lo + min(k_issue, n - 1));
        pid_s[st] = pid_of(k_issue + NB);
        process_unit(kb[st], vb[st], w_lo + it + st);
      }
    }
    // The last n % NB units already sit in kb[0 ..] (their loads were issued
    // by the prologue or the last group).
#pragma unroll
    for (int st = 0; st < NB - 1; ++st)
      if (n_main + st < n) process_unit(kb[st], vb[st], w_lo + n_main + st);
  }

  // Merge the 4 key groups of the wave (same m everywhere in the wave).
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    l[r] = add4(l[r]);
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[r][e] = add4(o[r][e]);
  }

  // Merge the waves of each row group through LDS.
  float* wbase = lds + (size_t)wave * RW * (D + 2);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RW; ++r) { wbase[r] = m[r]; wbase[RW + r] = l[r]; }
  }
  if (slot == 0) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int e = 0; e < DPL; ++e) wbase[2 * RW + r * D + dim_of<D, KV>(c, e)] = o[r][e];
  }
  __syncthreads();

  const float vs = a.v_scale ? a.v_scale[g] : 1.0f;
  const int total = nrg * RW * D;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int rgi = idx / (RW * D);
    const int r = (idx / D) % RW;
    const int d = idx % D;
    const int gr = rgi * RW + r;
    const int i = gr / G;
    if (i >= Qb) continue;
    const int h = g * G + (gr - i * G);
    const int t = off + i;
    const bool active = pos0 + i >= 0;
    float M = -INFINITY;
    for (int k = 0; k < a.key_waves; ++k)
      M = fmaxf(M, lds[(size_t)(k * nrg + rgi) * RW * (D + 2) + r]);
    float lsum = 0.0f, osum = 0.0f;
    if (active) {
      for (int k = 0; k < a.key_waves; ++k) {
        const float* wb = lds + (size_t)(k * nrg + rgi) * RW * (D + 2);
        const float wt = __builtin_amdgcn_exp2f(wb[r] - M);
        lsum += wt * wb[RW + r];
        osum += wt * wb[2 * RW + r * D + d];
      }
    }
    osum *= vs;
    if (a.direct) {
      const _Float16 y = lsum > 0.0f ? (_Float16)(osum / lsum) : (_Float16)0.0f;
      a.out[((size_t)t * Hq + h) * D + d] = __builtin_bit_cast(uint16_t, y);
    } else {
      const size_t prow = ((size_t)t * Hq + h) * S + split;
      a.part_o[prow * D + d] = osum;
      if (d == 0) {
        a.part_ml[prow * 2] = lsum > 0.0f ? M : -INFINITY;
        a.part_ml[prow * 2 + 1] = lsum;
      }
    }
  }
}

template <int D, int KV>
hipError_t launch_rw(int rw, dim3 grid, int threads, size_t lds, hipStream_t stream,
                     const DecodeArgs& args) {
  // Only the row counts of vector_rw_compiled are instantiated.
  switch (rw) {
#define PDA_CASE(R)                                                           \
  case R:                                                                     \
    if constexpr (vector_rw_compiled(D, KV, R)) {                             \
      hipLaunchKernelGGL((pda_decode_kernel<D, KV, R>), grid, dim3(threads), \
                         lds, stream, args);                                  \
      return hipGetLastError();                                               \
    }                                                                         \
    return hipErrorInvalidValue;
    PDA_CASE(1)
    PDA_CASE(2)
    PDA_CASE(3)
    PDA_CASE(4)
    PDA_CASE(5)
    PDA_CASE(6)
    PDA_CASE(7)
    PDA_CASE(8)
#undef PDA_CASE
    default:
      return hipErrorInvalidValue;
  }
}

template <int KV>
hipError_t launch_kv(int head_dim, int rw, dim3 grid, int threads, size_t lds,
                     hipStream_t stream, const DecodeArgs& args) {
  if (head_dim == 128) return launch_rw<128, KV>(rw, grid, threads, lds, stream, args);
  if (head_dim == 256) return launch_rw<256, KV>(rw, grid, threads, lds, stream, args);
  return hipErrorInvalidValue;
}

}  // namespace pda
