// Split-K combine for gfx950: merges the per-split partials (m, l, o) of each
// (token, query head) row into the fp16 output. This is the merge step of the
// split-K decode in vllm-rdna pull request #33 ("perf(rocm): FA-RDNA2 decode,
// scores on every wave and 4 barriers per tile"), sections "Purpose" and
// "Test Result" (split-K combine).
//
// One workgroup (4 waves) per row. Every wave reads the row's (m, l) pairs
// into lanes (split s in lane s % 64), so the global max M and each split's
// weight 2^(m_s - M) sit in registers; wave w then streams the o rows of
// splits w, w+4, ... (lane = D/64 contiguous dims, one coalesced row per
// split, 8 independent loads in flight) and the 4 waves add up through LDS.
// A split with l = 0 (no visible key) has weight 0 and its o is never used;
// a row with no live split is written as zeros.
#include "pda_kernels.h"

namespace pda {

constexpr int kCombineWaves = 4;
constexpr int kMaxSplitSlots = 4;  // splits per lane: 4 x 64 >= PDA_MAX_SPLITS

template <int D>
__global__ void __launch_bounds__(64 * kCombineWaves)
pda_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                   uint16_t* __restrict__ out, int S) {
  constexpr int DT = D / 64;
  __shared__ float red[kCombineWaves][D + 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t row = blockIdx.x;
  const float* ml = part_ml + row * S * 2;

  float mv[kMaxSplitSlots], lv[kMaxSplitSlots];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMaxSplitSlots; ++k) {
    const int s = lane + 64 * k;
    mv[k] = -INFINITY;
    lv[k] = 0.0f;
    if (s < S) {
      mv[k] = ml[2 * s];
      lv[k] = ml[2 * s + 1];
    }
    if (lv[k] > 0.0f) M = fmaxf(M, mv[k]);
  }
  for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k, 64));

  float wv[kMaxSplitSlots];
  float den = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxSplitSlots; ++k) {
    wv[k] = (lv[k] > 0.0f) ? __builtin_amdgcn_exp2f(mv[k] - M) : 0.0f;
    den += wv[k] * lv[k];
  }
  for (int k = 32; k >= 1; k >>= 1) den += __shfl_xor(den, k, 64);

  float acc[DT];
#pragma unroll
  for (int e = 0; e < DT; ++e) acc[e] = 0.0f;
  const float* src = part_o + row * S * D + lane * DT;
#pragma unroll
  for (int k = 0; k < kMaxSplitSlots; ++k) {
    const int n = min(64, S - 64 * k);
#pragma unroll 8
    for (int j = wave; j < n; j += kCombineWaves) {
      const float w = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wv[k]), j));
      const float* p = src + (size_t)(64 * k + j) * D;
#pragma unroll
      for (int e = 0; e < DT; ++e) {
        const float x = p[e];
        acc[e] += w > 0.0f ? w * x : 0.0f;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < DT; ++e) red[wave][lane * DT + e] = acc[e];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < kCombineWaves; ++w) o += red[w][d];
    const _Float16 y = den > 0.0f ? (_Float16)(o / den) : (_Float16)0.0f;
    out[row * D + d] = __builtin_bit_cast(uint16_t, y);
  }
}

hipError_t launch_combine(const float* part_o, const float* part_ml, uint16_t* out,
                          int rows, int head_dim, int num_splits, hipStream_t stream) {
  if (num_splits > 64 * kMaxSplitSlots) return hipErrorInvalidValue;
  const dim3 grid(rows), block(64 * kCombineWaves);
  if (head_dim == 128) {
    hipLaunchKernelGGL(pda_combine_kernel<128>, grid, block, 0, stream, part_o, part_ml, out,
                       num_splits);
  } else if (head_dim == 256) {
    hipLaunchKernelGGL(pda_combine_kernel<256>, grid, block, 0, stream, part_o, part_ml, out,
                       num_splits);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pda
