// Split-K combine for gfx950: merges the per-split partials (m, l, o) of each
// (token, query head) row into the fp16 output. This is the merge step of the
// split-K decode in vllm-rdna pull request #33 ("perf(rocm): FA-RDNA2 decode,
// scores on every wave and 4 barriers per tile"), sections "Purpose" and
// "Test Result" (split-K combine).
//
// One workgroup per row and slice of D / DP dims. With a fixed split count S
// it has ceil(S / 16) waves; wave w owns splits 16w .. 16w + 15 and issues
// all of their o loads at once
// (lane = D / (64 DP) contiguous dims of a split row), so the partials cost
// about one memory round trip whatever S is. With few rows (small batches)
// the dims are cut into DP slices so that more compute units share the
// loads. Every wave reads all (m, l) pairs into lanes
// (split s in lane s % 64, slot s / 64) to get the global max M and the
// denominator; a split's weight is 2^(m_s - M). Several waves add up through
// LDS. A split with l = 0 (no visible key) has weight 0 and its o is never
// used; a row with no live split is written as zeros. With balanced splits
// (a per-sequence split count read from the decode kernel's chunk lists) the
// waves are those a uniform batch needs, the longer rows of a ragged batch
// take batches of 16 splits nwaves * 16 apart, and the partials' loads for a
// uniform batch's layout go out together with the chunk list's load (issued
// again only when the list differs).
#include "pda_kernels.h"

namespace pda {

constexpr int kSplitsPerWave = 16;
constexpr int kMaxSplitSlots = 4;  // (m, l) slots per lane: 4 x 64 >= PDA_MAX_SPLITS
constexpr int kMaxCombineWaves = 64 * kMaxSplitSlots / kSplitsPerWave;

// Wave-wide max and sum without LDS: DPP within each 16-lane row (swap
// neighbours, then pairs, then mirror 8- and 16-lane halves), then the row
// pairs and halves of the wave through permlane16/32 swaps. Every lane ends
// with the result.
template <int kCtrl>
__device__ __forceinline__ float dpp_get(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float swap16(float v, bool sum) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                            false, false);
  const float x = __builtin_bit_cast(float, (int)a[0]), y = __builtin_bit_cast(float, (int)a[1]);
  return sum ? x + y : fmaxf(x, y);
}
__device__ __forceinline__ float swap32(float v, bool sum) {
  auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                            false, false);
  const float x = __builtin_bit_cast(float, (int)a[0]), y = __builtin_bit_cast(float, (int)a[1]);
  return sum ? x + y : fmaxf(x, y);
}
constexpr int kQuadSwap1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kQuadSwap2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kRowMirror = 0x140;   // lane i <-> 15 - i within each 16 lanes
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_get<kQuadSwap1>(v));
  v = fmaxf(v, dpp_get<kQuadSwap2>(v));
  v = fmaxf(v, dpp_get<kHalfMirror>(v));
  v = fmaxf(v, dpp_get<kRowMirror>(v));
  return swap32(swap16(v, false), false);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_get<kQuadSwap1>(v);
  v += dpp_get<kQuadSwap2>(v);
  v += dpp_get<kHalfMirror>(v);
  v += dpp_get<kRowMirror>(v);
  return swap32(swap16(v, true), true);
}

template <int D, int DP>
__global__ void __launch_bounds__(64 * kMaxCombineWaves)
pda_combine_kernel(const CombineArgs a) {
  constexpr int DW = D / DP;  // dims of this workgroup's slice
  constexpr int DT = DW / 64;
  static_assert(DT >= 1, "a lane holds at least one dim");
  typedef float fv_t __attribute__((ext_vector_type(DT)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  extern __shared__ float red[];  // [waves][DW] when there are several waves
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const size_t row = blockIdx.x;
  const int d0 = DW * blockIdx.y;

  // Every load of the first batch is issued before any is used, with no
  // branches between them: indexes past the last split are clamped to it (in
  // bounds) and their weight is 0. First this wave's o rows (splits s0 ..
  // s0 + 15; later batches, s0 + 16 nwaves .., only with more splits than
  // 16 per wave), then every split's (m, l): split lane + 64 k in slot k of
  // the lane. A row's splits are adjacent records from rec0 on.
  size_t rec0;
  int S = a.num_splits;
  const float* src;
  fv_t x[kSplitsPerWave];
  f2_t p[kMaxSplitSlots];
  const int s_first = kSplitsPerWave * wave;
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int j = 0; j < kSplitsPerWave; ++j)
      x[j] = *reinterpret_cast<const fv_t*>(src + (size_t)min(s0 + j, S - 1) * D);
  };
  auto issue = [&]() {
    src = a.part_o + rec0 * D + d0 + lane * DT;
    if (s_first < S) load_batch(s_first);
    const float* ml = a.part_ml + 2 * rec0;
#pragma unroll
    for (int k = 0; k < kMaxSplitSlots; ++k)
      p[k] = *reinterpret_cast<const f2_t*>(ml + 2 * min(lane + 64 * k, S - 1));
  };
  if (a.meta) {
    // Balanced splits: the row's chunk list gives its first chunk slot and
    // count. The loads for a uniform batch's layout (every sequence
    // max_q_len tokens and per_seq chunks) go out with the list's load, and
    // are issued again only if the list says otherwise.
    const int Hq = a.num_q_heads;
    const size_t t = row / Hq;
    const int h = (int)(row - t * Hq);
    const int k = h / a.group;
    const int4 mt = *reinterpret_cast<const int4*>(a.meta + 4 * t);
    const size_t rec_k = (size_t)k * a.rows + (h - k * a.group);
    const int bg = (int)(t / a.max_q_len);
    const int ig = (int)t - bg * a.max_q_len;
    S = a.per_seq;
    rec0 = (rec_k + (size_t)ig * a.group) * a.chunks + (size_t)bg * a.per_seq;
    issue();
    if (mt.x != bg * a.per_seq || mt.y != a.per_seq || mt.z != ig) {
      S = mt.y;
      if (S <= 1) return;  // one chunk: the decode kernel wrote this row
      rec0 = (rec_k + (size_t)mt.z * a.group) * a.chunks + mt.x;
      issue();
    }
  } else {
    rec0 = row * S;
    issue();
  }

  float mv[kMaxSplitSlots], lv[kMaxSplitSlots];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMaxSplitSlots; ++k) {
    const bool live = lane + 64 * k < S && p[k][1] > 0.0f;
    mv[k] = live ? p[k][0] : -INFINITY;
    lv[k] = live ? p[k][1] : 0.0f;
    M = fmaxf(M, mv[k]);
  }
  M = wave_max(M);
  float wv[kMaxSplitSlots];
  float den = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxSplitSlots; ++k) {
    wv[k] = lv[k] > 0.0f ? __builtin_amdgcn_exp2f(mv[k] - M) : 0.0f;
    den += wv[k] * lv[k];
  }
  den = wave_sum(den);

  // Weights of splits s0 .. s0 + 15: slot s0 / 64, lanes s0 % 64 + j. A
  // split with weight 0 (no visible key, or past S) is never added: its o may
  // hold anything.
  fv_t acc = {};
  for (int s0 = s_first; s0 < S; s0 += kSplitsPerWave * nwaves) {
    if (s0 != s_first) load_batch(s0);
    const int slot = s0 >> 6;
    const float wsel = slot == 0 ? wv[0] : slot == 1 ? wv[1] : slot == 2 ? wv[2] : wv[3];
    const int lane0 = s0 & 63;
#pragma unroll
    for (int j = 0; j < kSplitsPerWave; ++j) {
      const float w = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wsel), lane0 + j));
      const fv_t t = acc + w * x[j];
#pragma unroll
      for (int e = 0; e < DT; ++e) acc[e] = w > 0.0f ? t[e] : acc[e];
    }
  }

  if (nwaves == 1) {
    typedef _Float16 hv_t __attribute__((ext_vector_type(DT)));
    hv_t y;
#pragma unroll
    for (int e = 0; e < DT; ++e) y[e] = den > 0.0f ? (_Float16)(acc[e] / den) : (_Float16)0.0f;
    *reinterpret_cast<hv_t*>(a.out + row * D + d0 + lane * DT) = y;
    return;
  }
  *reinterpret_cast<fv_t*>(red + wave * DW + lane * DT) = acc;
  __syncthreads();
  for (int d = threadIdx.x; d < DW; d += blockDim.x) {
    float o = 0.0f;
    for (int w = 0; w < nwaves; ++w) o += red[w * DW + d];
    const _Float16 y = den > 0.0f ? (_Float16)(o / den) : (_Float16)0.0f;
    a.out[row * D + d0 + d] = __builtin_bit_cast(uint16_t, y);
  }
}

int combine_dim_parts(int rows, int head_dim, int num_cus) {
  int dp = 1;
  while (2 * dp * 64 <= head_dim && (int64_t)rows * dp < num_cus) dp *= 2;
  return dp;
}

hipError_t launch_combine(const CombineArgs& args, int rows, int head_dim, int waves,
                          int dim_parts, hipStream_t stream) {
  if (waves < 1 || waves > kMaxCombineWaves) return hipErrorInvalidValue;
  if (!args.meta && (args.num_splits < 1 || args.num_splits > 64 * kMaxSplitSlots))
    return hipErrorInvalidValue;
  const dim3 grid(rows, dim_parts), block(64 * waves);
  const size_t lds = waves > 1 ? (size_t)waves * (head_dim / dim_parts) * sizeof(float) : 0;
#define PDA_CCASE(DD, PP)                                                                  \
  if (head_dim == DD && dim_parts == PP) {                                                 \
    hipLaunchKernelGGL((pda_combine_kernel<DD, PP>), grid, block, lds, stream, args);      \
    return hipGetLastError();                                                              \
  }
  PDA_CCASE(128, 1)
  PDA_CCASE(128, 2)
  PDA_CCASE(256, 1)
  PDA_CCASE(256, 2)
  PDA_CCASE(256, 4)
#undef PDA_CCASE
  return hipErrorInvalidValue;
}

}  // namespace pda
