// Split-K combine for gfx950: merges the per-split partials (m, l, o) of each
// (token, query head) row into the fp16 output. This is the merge step of the
// split-K decode in vllm-rdna pull request #33 ("perf(rocm): FA-RDNA2 decode,
// scores on every wave and 4 barriers per tile"), sections "Purpose" and
// "Test Result" (split-K combine).
//
// One wave per row; each lane owns D/64 contiguous dims, so a split's o row
// is one coalesced 512/1024-byte read. Splits are visited in order; a split
// with l = 0 (no visible key) drops out; a row with no live split is 0.
#include "pda_kernels.h"

namespace pda {

template <int D>
__global__ void __launch_bounds__(256)
pda_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                   uint16_t* __restrict__ out, int rows, int S) {
  constexpr int DT = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* ml = part_ml + (size_t)row * S * 2;

  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) {
    const float l = ml[2 * s + 1];
    if (l > 0.0f) M = fmaxf(M, ml[2 * s]);
  }
  for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k, 64));

  float acc[DT];
#pragma unroll
  for (int e = 0; e < DT; ++e) acc[e] = 0.0f;
  float den = 0.0f;
  if (M != -INFINITY) {
    const float* src = part_o + (size_t)row * S * D + lane * DT;
    for (int s = 0; s < S; ++s) {
      const float l = ml[2 * s + 1];
      if (l > 0.0f) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
        den += w * l;
#pragma unroll
        for (int e = 0; e < DT; ++e) acc[e] += w * src[(size_t)s * D + e];
      }
    }
  }
  uint16_t* dst = out + (size_t)row * D + lane * DT;
#pragma unroll
  for (int e = 0; e < DT; ++e) {
    const _Float16 y = den > 0.0f ? (_Float16)(acc[e] / den) : (_Float16)0.0f;
    dst[e] = __builtin_bit_cast(uint16_t, y);
  }
}

hipError_t launch_combine(const float* part_o, const float* part_ml, uint16_t* out,
                          int rows, int head_dim, int num_splits, hipStream_t stream) {
  constexpr int kWaves = 4;
  const dim3 grid((rows + kWaves - 1) / kWaves);
  if (head_dim == 128) {
    hipLaunchKernelGGL(pda_combine_kernel<128>, grid, dim3(64 * kWaves), 0, stream,
                       part_o, part_ml, out, rows, num_splits);
  } else if (head_dim == 256) {
    hipLaunchKernelGGL(pda_combine_kernel<256>, grid, dim3(64 * kWaves), 0, stream,
                       part_o, part_ml, out, rows, num_splits);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pda
