// Paged KV-cache writer for gfx950: new tokens' K and V rows go to their page
// slots, as fp16 or quantized to fp8-e4m3 / int8 codes with one fp32 scale per
// KV head. This produces the layout the decode kernels read (the cache
// writer's layout that vllm-rdna pull request #33, "perf(rocm): FA-RDNA2
// decode, scores on every wave and 4 barriers per tile", tests the decode
// against in its "Test Plan"; fp8 and int8 caches per its "Purpose").
//
// One thread per 16-byte chunk (8 elements) of a (token, KV head) row of K
// and the same chunk of V: the loads and stores of a wave are contiguous runs
// of whole rows. A quantized code is that of q = x / scale in fp32 (IEEE
// division), clamped to the format's largest finite magnitude, then rounded
// to nearest with ties to even: fp8 by v_cvt_pk_fp8_f32 (OCP E4M3 on
// gfx950), int8 by v_rndne_f32.
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

// Code of the exact quotient x / scale (fp32, IEEE division), clamped to the
// format's largest finite magnitude, rounded to nearest even.
template <int KV>
__device__ inline uint32_t exact_code(float x, float scale) {
  const float q = x / scale;
  if constexpr (KV == kKvFp8) {
    const float c = __builtin_amdgcn_fmed3f(q, -kE4m3Max, kE4m3Max);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
  } else {
    const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(q), -kInt8Max, kInt8Max);
    return (uint32_t)(int32_t)r & 0xFFu;
  }
}

// 8 fp16 values (4 dwords) -> 8 codes (2 dwords), each the code of the exact
// quotient x / scale. The quotient is first taken as x * (1 / scale) (the
// reciprocal to about one ulp, so that product is within a few ulp of the
// exact quotient), and the code is computed at both ends of a bracket 2^-20
// (8 ulp) around it: the code is a non-decreasing function of the quotient,
// so equal codes at both ends are the exact quotient's code. Only a word of 4
// values with a bracket that straddles a rounding boundary takes the IEEE
// divisions (rare: a boundary within 8 ulp).
template <int KV>
__device__ inline u32x2 quantize8(u32x4_w x, float scale, float rcp) {
  constexpr float kLo = 1.0f - 0x1p-20f, kHi = 1.0f + 0x1p-20f;
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = half_lo(x[i]);
    f[2 * i + 1] = half_hi(x[i]);
  }
  u32x2 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t lo = 0, hi = 0;
    if constexpr (KV == kKvFp8) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float q = f[4 * w + i] * rcp;
        a[i] = __builtin_amdgcn_fmed3f(q * kLo, -kE4m3Max, kE4m3Max);
        b[i] = __builtin_amdgcn_fmed3f(q * kHi, -kE4m3Max, kE4m3Max);
      }
      lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
          a[2], a[3], __builtin_amdgcn_cvt_pk_fp8_f32(a[0], a[1], 0, false), true);
      hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
          b[2], b[3], __builtin_amdgcn_cvt_pk_fp8_f32(b[0], b[1], 0, false), true);
    } else {
      // Clamped to [-127, 127], then rounded to an integer by adding
      // 1.5 * 2^23 (the fp32 add rounds to nearest even, and the integer
      // lands in the low mantissa bits: its two's-complement low byte is
      // the code); clamping before rounding gives the same code as after.
      constexpr float kMagic = 12582912.0f;
      uint32_t ra[4], rb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float q = f[4 * w + i] * rcp;
        ra[i] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_fmed3f(q * kLo, -kInt8Max, kInt8Max) + kMagic);
        rb[i] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_fmed3f(q * kHi, -kInt8Max, kInt8Max) + kMagic);
      }
      // low bytes of the four words into one word (byte selects of v_perm:
      // 0-3 the second operand's bytes, 4-7 the first's, 0x0C a zero byte)
      auto pack = [](const uint32_t (&r)[4]) {
        const uint32_t p01 = __builtin_amdgcn_perm(r[1], r[0], 0x0C0C0400u);
        const uint32_t p23 = __builtin_amdgcn_perm(r[3], r[2], 0x0C0C0400u);
        return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
      };
      lo = pack(ra);
      hi = pack(rb);
    }
    if (lo != hi) {
      lo = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) lo |= exact_code<KV>(f[4 * w + i], scale) << (8 * i);
    }
    out[w] = lo;
  }
  return out;
}

// One thread per 16-byte chunk (8 elements) of a (token, KV head) row of K
// and the same chunk of V; a workgroup covers `tokens_per_wg` whole tokens
// (per_token = num_kv_heads * row_chunks threads each), or, for tokens of
// more than 256 chunks, 256 chunks of one token (grid y: the slice), so a
// thread's token, head and chunk come from its workgroup index and
// small-integer divisions.
template <int KV>
__global__ void __launch_bounds__(256)
pda_write_kv_kernel(const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
                    const int32_t* __restrict__ slot_mapping, uint8_t* __restrict__ k_cache,
                    uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
                    const float* __restrict__ v_scale, int num_tokens, int tokens_per_wg,
                    int row_chunks, int num_kv_heads, int head_dim, int page_size, int hnd,
                    int64_t num_slots) {
  const int per_token = num_kv_heads * row_chunks;
  // tid / per_token and the chunk / row_chunks: float quotients of integers
  // below 2^16 offset by one half, exact here (the quotient sits at least
  // 1 / 2 per divisor from the next integer, far beyond the rounding error).
  const int tid = threadIdx.x;
  const int tt = (int)(((float)tid + 0.5f) / (float)per_token);
  const int rem = (int)blockIdx.y * 256 + tid - tt * per_token;
  const int h = (int)(((float)rem + 0.5f) / (float)row_chunks);
  const int c = rem - h * row_chunks;
  const int64_t t = (int64_t)blockIdx.x * tokens_per_wg + tt;
  if (tt >= tokens_per_wg || rem >= per_token || t >= num_tokens) return;
  // The row loads do not depend on the slot: they go out with its load.
  // Rows are read once and cache slots written once, by non-temporal loads
  // and stores (they then displace no other lines in the caches; 2-6%
  // faster at 32768 tokens, equal at 64).
  const size_t src = ((size_t)t * num_kv_heads + h) * head_dim + 8 * c;  // elements
  const u32x4_w kx = __builtin_nontemporal_load(reinterpret_cast<const u32x4_w*>(key + src));
  const u32x4_w vx = __builtin_nontemporal_load(reinterpret_cast<const u32x4_w*>(value + src));
  const int64_t slot = slot_mapping[t];
  float ks = 1.0f, vs = 1.0f;
  if constexpr (KV != kKvF16) {
    ks = k_scale[h];
    vs = v_scale[h];
  }
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool: not written

  // destination row: NHD [page][pos][h][:] is slot-major; HND [page][h][pos][:]
  const size_t dst_row =
      hnd ? ((size_t)(slot / page_size) * num_kv_heads + h) * page_size + (size_t)(slot % page_size)
          : (size_t)slot * num_kv_heads + h;
  const size_t dst = dst_row * head_dim + 8 * c;  // elements
  if constexpr (KV == kKvF16) {
    __builtin_nontemporal_store(kx, reinterpret_cast<u32x4_w*>(k_cache + 2 * dst));
    __builtin_nontemporal_store(vx, reinterpret_cast<u32x4_w*>(v_cache + 2 * dst));
  } else {
    __builtin_nontemporal_store(quantize8<KV>(kx, ks, __builtin_amdgcn_rcpf(ks)),
                                reinterpret_cast<u32x2*>(k_cache + dst));
    __builtin_nontemporal_store(quantize8<KV>(vx, vs, __builtin_amdgcn_rcpf(vs)),
                                reinterpret_cast<u32x2*>(v_cache + dst));
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
  const int64_t per_token = (int64_t)d.num_kv_heads * row_chunks;
  if (per_token >= (1 << 16))
    return wfail(PDA_ERR_SHAPE, "num_kv_heads * head_dim must be below 2^19");
  const int tokens_per_wg = per_token <= 256 ? (int)(256 / per_token) : 1;
  const int64_t slices = per_token <= 256 ? 1 : (per_token + 255) / 256;
  const int64_t blocks = ((int64_t)d.num_tokens + tokens_per_wg - 1) / tokens_per_wg;
  const int64_t num_slots = (int64_t)d.num_pages * d.page_size;
  const int hnd = d.kv_layout == PDA_LAYOUT_HND;
  const dim3 grid((unsigned)blocks, (unsigned)slices),
      block((unsigned)(per_token <= 256 ? tokens_per_wg * per_token : 256));
  auto k = static_cast<const uint16_t*>(key);
  auto v = static_cast<const uint16_t*>(value);
  auto kc = static_cast<uint8_t*>(k_cache);
  auto vc = static_cast<uint8_t*>(v_cache);
  switch (d.kv_dtype) {
    case PDA_KV_F16:
      hipLaunchKernelGGL(pda::pda_write_kv_kernel<pda::kKvF16>, grid, block, 0, stream, k, v,
                         slot_mapping, kc, vc, k_scale, v_scale, d.num_tokens, tokens_per_wg,
                         row_chunks, d.num_kv_heads, d.head_dim, d.page_size, hnd, num_slots);
      break;
    case PDA_KV_FP8_E4M3:
      hipLaunchKernelGGL(pda::pda_write_kv_kernel<pda::kKvFp8>, grid, block, 0, stream, k, v,
                         slot_mapping, kc, vc, k_scale, v_scale, d.num_tokens, tokens_per_wg,
                         row_chunks, d.num_kv_heads, d.head_dim, d.page_size, hnd, num_slots);
      break;
    default:
      hipLaunchKernelGGL(pda::pda_write_kv_kernel<pda::kKvI8>, grid, block, 0, stream, k, v,
                         slot_mapping, kc, vc, k_scale, v_scale, d.num_tokens, tokens_per_wg,
                         row_chunks, d.num_kv_heads, d.head_dim, d.page_size, hnd, num_slots);
      break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return static_cast<pda_status>(
        pda::host_fail(PDA_ERR_DEVICE, "cache write launch: %s", hipGetErrorString(e)));
  return PDA_OK;
}
