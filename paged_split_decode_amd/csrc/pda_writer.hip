// Paged KV-cache writer for gfx950: new tokens' K and V rows go to their page
// slots, as fp16 or quantized to fp8-e4m3 / int8 codes with one fp32 scale per
// KV head. This produces the layout the decode kernels read (the cache
// writer's layout that vllm-rdna pull request #33, "perf(rocm): FA-RDNA2
// decode, scores on every wave and 4 barriers per tile", tests the decode
// against in its "Test Plan"; fp8 and int8 caches per its "Purpose").
//
// One thread per 16-byte chunk (8 elements) of a (token, KV head) row of K
// and the same chunk of V: the loads and stores of a wave are contiguous runs
// of whole rows. A quantized code is q = x / scale in fp32 (IEEE division),
// clamped to the format's largest finite magnitude, then rounded to nearest
// with ties to even: fp8 by v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950), int8 by
// v_rndne_f32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda.h"
#include "pda_kernels.h"

namespace pda {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_w __attribute__((ext_vector_type(4)));

constexpr float kE4m3Max = 448.0f;
constexpr float kInt8Max = 127.0f;

__device__ inline float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ inline float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// 8 fp16 values (4 dwords) -> 8 codes (2 dwords).
template <int KV>
__device__ inline u32x2 quantize8(u32x4_w x, float scale) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = half_lo(x[i]) / scale;
    f[2 * i + 1] = half_hi(x[i]) / scale;
  }
  u32x2 out;
  if constexpr (KV == kKvFp8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = fminf(fmaxf(f[i], -kE4m3Max), kE4m3Max);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      int packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w], f[4 * w + 1], 0, false);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w + 2], f[4 * w + 3], packed, true);
      out[w] = (uint32_t)packed;
    }
  } else {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = fminf(fmaxf(__builtin_rintf(f[4 * w + i]), -kInt8Max), kInt8Max);
        word |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * i);
      }
      out[w] = word;
    }
  }
  return out;
}

template <int KV>
__global__ void __launch_bounds__(256)
pda_write_kv_kernel(const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
                    const int32_t* __restrict__ slot_mapping, uint8_t* __restrict__ k_cache,
                    uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
                    const float* __restrict__ v_scale, int64_t chunks, int row_chunks,
                    int num_kv_heads, int head_dim, int page_size, int hnd,
                    int64_t num_slots) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= chunks) return;
  const int64_t per_token = (int64_t)num_kv_heads * row_chunks;
  const int64_t t = idx / per_token;
  const int64_t rem = idx - t * per_token;
  const int h = (int)(rem / row_chunks);
  const int c = (int)(rem - (int64_t)h * row_chunks);
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool: not written

  const size_t src = ((size_t)t * num_kv_heads + h) * head_dim + 8 * c;          // elements
  // destination row: NHD [page][pos][h][:] is slot-major; HND [page][h][pos][:]
  const size_t dst_row =
      hnd ? ((size_t)(slot / page_size) * num_kv_heads + h) * page_size + (size_t)(slot % page_size)
          : (size_t)slot * num_kv_heads + h;
  const size_t dst = dst_row * head_dim + 8 * c;  // elements
  const u32x4_w kx = *reinterpret_cast<const u32x4_w*>(key + src);
  const u32x4_w vx = *reinterpret_cast<const u32x4_w*>(value + src);
  if constexpr (KV == kKvF16) {
    *reinterpret_cast<u32x4_w*>(k_cache + 2 * dst) = kx;
    *reinterpret_cast<u32x4_w*>(v_cache + 2 * dst) = vx;
  } else {
    *reinterpret_cast<u32x2*>(k_cache + dst) = quantize8<KV>(kx, k_scale[h]);
    *reinterpret_cast<u32x2*>(v_cache + dst) = quantize8<KV>(vx, v_scale[h]);
  }
}

}  // namespace
}  // namespace pda

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

pda_status wfail(pda_status st, const char* msg) {
  return static_cast<pda_status>(pda::host_fail(st, "%s", msg));
}

}  // namespace

extern "C" pda_status pda_write_kv_cache(const void* key, const void* value,
                                         const int32_t* slot_mapping, void* k_cache,
                                         void* v_cache, const float* k_scale,
                                         const float* v_scale, const pda_cache_dims* dims,
                                         hipStream_t stream) {
  if (!dims) return wfail(PDA_ERR_NULL, "dims is NULL");
  const pda_cache_dims& d = *dims;
  if (d.num_tokens < 0) return wfail(PDA_ERR_SHAPE, "num_tokens must be >= 0");
  if (d.num_kv_heads <= 0 || d.head_dim <= 0 || d.page_size <= 0 || d.num_pages <= 0)
    return wfail(PDA_ERR_SHAPE, "num_kv_heads, head_dim, page_size and num_pages must be > 0");
  if (d.head_dim % 8)
    return wfail(PDA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 (16-byte rows)");
  if (d.kv_dtype != PDA_KV_F16 && d.kv_dtype != PDA_KV_FP8_E4M3 && d.kv_dtype != PDA_KV_INT8)
    return wfail(PDA_ERR_UNSUPPORTED, "kv_dtype is not a pda_kv_dtype");
  if (d.kv_layout != PDA_LAYOUT_NHD && d.kv_layout != PDA_LAYOUT_HND)
    return wfail(PDA_ERR_UNSUPPORTED, "kv_layout is not a pda_kv_layout");
  if ((int64_t)d.num_pages * d.page_size > INT32_MAX)
    return wfail(PDA_ERR_SHAPE, "num_pages * page_size must fit in int32 (slot indices)");
  if (d.num_tokens == 0) return PDA_OK;
  if (!key || !value || !slot_mapping || !k_cache || !v_cache)
    return wfail(PDA_ERR_NULL, "key, value, slot_mapping, k_cache and v_cache must be non-NULL");
  const bool quant = d.kv_dtype != PDA_KV_F16;
  if (quant && (!k_scale || !v_scale))
    return wfail(PDA_ERR_NULL, "fp8/int8 caches need k_scale and v_scale");
  if (!quant && (k_scale || v_scale))
    return wfail(PDA_ERR_SHAPE, "k_scale/v_scale must be NULL for fp16 caches");
  if (!aligned(key, 16) || !aligned(value, 16))
    return wfail(PDA_ERR_ALIGN, "key and value must be 16-byte aligned");
  if (!aligned(k_cache, quant ? 8 : 16) || !aligned(v_cache, quant ? 8 : 16))
    return wfail(PDA_ERR_ALIGN, "k_cache and v_cache must be 16-byte (fp16) or 8-byte aligned");

  const int row_chunks = d.head_dim / 8;
  const int64_t chunks = (int64_t)d.num_tokens * d.num_kv_heads * row_chunks;
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > INT32_MAX) return wfail(PDA_ERR_SHAPE, "too many tokens for one launch");
  const int64_t num_slots = (int64_t)d.num_pages * d.page_size;
  const int hnd = d.kv_layout == PDA_LAYOUT_HND;
  const dim3 grid((unsigned)blocks), block(256);
  auto k = static_cast<const uint16_t*>(key);
  auto v = static_cast<const uint16_t*>(value);
  auto kc = static_cast<uint8_t*>(k_cache);
  auto vc = static_cast<uint8_t*>(v_cache);
  switch (d.kv_dtype) {
    case PDA_KV_F16:
      hipLaunchKernelGGL(pda::pda_write_kv_kernel<pda::kKvF16>, grid, block, 0, stream, k, v,
                         slot_mapping, kc, vc, k_scale, v_scale, chunks, row_chunks,
                         d.num_kv_heads, d.head_dim, d.page_size, hnd, num_slots);
      break;
    case PDA_KV_FP8_E4M3:
      hipLaunchKernelGGL(pda::pda_write_kv_kernel<pda::kKvFp8>, grid, block, 0, stream, k, v,
                         slot_mapping, kc, vc, k_scale, v_scale, chunks, row_chunks,
                         d.num_kv_heads, d.head_dim, d.page_size, hnd, num_slots);
      break;
    default:
      hipLaunchKernelGGL(pda::pda_write_kv_kernel<pda::kKvI8>, grid, block, 0, stream, k, v,
                         slot_mapping, kc, vc, k_scale, v_scale, chunks, row_chunks,
                         d.num_kv_heads, d.head_dim, d.page_size, hnd, num_slots);
      break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return static_cast<pda_status>(
        pda::host_fail(PDA_ERR_DEVICE, "cache write launch: %s", hipGetErrorString(e)));
  return PDA_OK;
}
