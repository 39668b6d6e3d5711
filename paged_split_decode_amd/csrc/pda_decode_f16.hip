// Decode-kernel instantiations for f16 KV (head_dim 128 and 256, 1..8 rows
// per wave; matrix-core kernel with 1 or 2 row tiles). The kernel templates
// and their design notes are in pda_decode_impl.h and pda_decode_mfma.h.
#include "pda_decode_impl.h"
#include "pda_decode_mfma.h"

namespace pda {

hipError_t launch_decode_f16(int head_dim, int rows_per_wave, dim3 grid,
                             int threads, size_t lds, hipStream_t stream,
                             const DecodeArgs& args) {
  return launch_kv<kKvF16>(head_dim, rows_per_wave, grid, threads, lds, stream, args);
}

hipError_t launch_decode_mfma_f16(int head_dim, int row_tiles, bool stream_kv, dim3 grid,
                               int threads, size_t lds, hipStream_t stream, const DecodeArgs& args) {
  return launch_mfma_kv<kKvF16>(head_dim, row_tiles, stream_kv, grid, threads, lds, stream, args);
}

}  // namespace pda
