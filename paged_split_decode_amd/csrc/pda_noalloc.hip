// The one-call decode path for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): the split partials and chunk lists go to a scratch array that
// the library holds on each device, instead of a caller's workspace.
//
// The array is a file-scope device variable, so every device the library
// runs on holds its own copy from module load until the process ends. Host
// code never uses the array's name as an address (on the host that name is
// only a stand-in): the device address is fetched once per device with
// hipGetSymbolAddress, with that device current, and passed to the kernels
// like a caller's workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pda.h"
#include "pda_kernels.h"

namespace {

constexpr size_t kScratchBytes = (size_t)PDA_NOALLOC_SCRATCH_BYTES;

// Zero-initialized at load; the kernels write every byte they later read
// (partials before the combine, chunk lists before the combine), so nothing
// needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (fetched on the first
// call there), or nullptr with the HIP error in *err.
void* scratch_address(hipError_t* err) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {nullptr};
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

pda_status fail(pda_status st, const char* fmt, long long a = 0, long long b = 0) {
  return static_cast<pda_status>(pda::host_fail(st, fmt, a, b));
}

}  // namespace

extern "C" {

size_t pda_noalloc_scratch_bytes(void) { return kScratchBytes; }

pda_status pda_paged_decode_attention_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    const int32_t* seq_lens, const int32_t* q_lens, float scale, int32_t window,
    int32_t num_splits, void* out, const float* k_scale, const float* v_scale,
    const pda_decode_dims* dims, hipStream_t stream) {
  // The workspace this call needs (host-only planning: no allocation, no
  // launch); negative is a validation error with its message already set.
  const int64_t need = pda_decode_workspace_bytes(dims, window, num_splits);
  if (need < 0) return static_cast<pda_status>(need);
  if ((uint64_t)need > kScratchBytes)
    return fail(PDA_ERR_WORKSPACE,
                "this call needs %lld bytes of split workspace; the library's scratch holds "
                "%lld (use pda_paged_decode_attention with a workspace)",
                (long long)need, (long long)kScratchBytes);
  hipError_t e = hipSuccess;
  void* ws = need > 0 ? scratch_address(&e) : nullptr;
  if (need > 0 && !ws)
    return static_cast<pda_status>(
        pda::host_fail(PDA_ERR_DEVICE, "scratch address: %s", hipGetErrorString(e)));
  return pda_paged_decode_attention(q, k_cache, v_cache, block_table, seq_lens, q_lens, scale,
                                    window, num_splits, out, k_scale, v_scale, dims, ws,
                                    ws ? kScratchBytes : 0, stream);
}

}  // extern "C"
