// Decode-kernel instantiations for fp8 KV (head_dim 128 and 256, 1..8 rows
// per wave). The kernel template and its design notes are in
// pda_decode_impl.h.
#include "pda_decode_impl.h"

namespace pda {

hipError_t launch_decode_fp8(int head_dim, int rows_per_wave, dim3 grid,
                             int threads, size_t lds, hipStream_t stream,
                             const DecodeArgs& args) {
  return launch_kv<kKvFp8>(head_dim, rows_per_wave, grid, threads, lds, stream, args);
}

}  // namespace pda
