// Instantiations of the long-query (prefill) kernel for every KV element type.
#include "pda_prefill_mfma.h"

namespace pda {

hipError_t launch_prefill_f16(int head_dim, int waves, dim3 items, int cus, size_t lds, hipStream_t stream,
                              const DecodeArgs& args) {
  return launch_prefill_kv<kKvF16>(head_dim, waves, items, cus, lds, stream, args);
}
hipError_t launch_prefill_fp8(int head_dim, int waves, dim3 items, int cus, size_t lds, hipStream_t stream,
                              const DecodeArgs& args) {
  return launch_prefill_kv<kKvFp8>(head_dim, waves, items, cus, lds, stream, args);
}
hipError_t launch_prefill_i8(int head_dim, int waves, dim3 items, int cus, size_t lds, hipStream_t stream,
                             const DecodeArgs& args) {
  return launch_prefill_kv<kKvI8>(head_dim, waves, items, cus, lds, stream, args);
}

}  // namespace pda
