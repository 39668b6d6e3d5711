// Streaming-read probe: how fast one launch can read a large buffer from
// HBM on this device. It gives the decode kernels' measured roof (their
// traffic is a gather of whole 16-key pages: contiguous runs of 2-8 KB), next
// to the 8 TB/s published peak.
//
// Every thread reads 16-byte vectors in a grid-stride loop, kUnroll of them
// in flight per iteration (the buffer is cut into kUnroll interleaved
// streams so that a wave's loads in one iteration are each 1 KB contiguous),
// and folds them into one XOR word; one word per workgroup goes to `sink`,
// so that no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda.h"
#include "pda_kernels.h"

namespace pda {
namespace {

typedef uint32_t u32x4_p __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(kProbeThreads)
pda_hbm_read_kernel(const u32x4_p* __restrict__ src, uint64_t n_vec, uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
  const uint64_t span = stride * kUnroll;
  uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4_p acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n_vec; i += span) {
    u32x4_p v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k];
  }
  for (; i < n_vec; i += stride) acc ^= src[i];  // the tail
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __shared__ uint32_t red[kProbeThreads / 64];
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) y ^= red[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace
}  // namespace pda

extern "C" {

pda_status pda_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                              hipStream_t stream) {
  if (!src || !sink)
    return static_cast<pda_status>(pda::host_fail(PDA_ERR_NULL, "src and sink must be non-NULL"));
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (bytes & 15u))
    return static_cast<pda_status>(
        pda::host_fail(PDA_ERR_ALIGN, "src and bytes must be multiples of 16"));
  if (workgroups < 1 || workgroups > (1 << 20))
    return static_cast<pda_status>(
        pda::host_fail(PDA_ERR_SHAPE, "workgroups %d outside 1..2^20", workgroups));
  if (bytes == 0) return PDA_OK;
  hipLaunchKernelGGL(pda::pda_hbm_read_kernel, dim3(workgroups), dim3(pda::kProbeThreads), 0,
                     stream, static_cast<const pda::u32x4_p*>(src), (uint64_t)(bytes / 16), sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return static_cast<pda_status>(
        pda::host_fail(PDA_ERR_DEVICE, "probe launch: %s", hipGetErrorString(e)));
  return PDA_OK;
}

}  // extern "C"
