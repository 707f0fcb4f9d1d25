// Row stride of the activation code buffers the prefill GEMMs copy from (the
// x and h codes in expert-sorted row order, and the dense path's x codes):
// a row's bytes (K E4M3 codes, or K/2 bytes of E2M1 blocks) rounded up to
// whole 128-byte lines, so that each K step's 128-byte piece of a row is one
// aligned line (with the unpadded 2880-byte rows every other row's piece
// straddles two lines).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

__host__ __device__ inline int64_t code_row_bytes(int64_t K, bool e2m1) {
  const int64_t b = e2m1 ? K / 2 : K;
  return (b + 127) / 128 * 128;
}

// E4M3 codes of `rows` rows of `row_len` values (row_len a multiple of 16)
// written at a row stride of `ld` bytes, with the per-tensor scale of
// *amax_bits (launch_encode_fp8 of a row-major matrix).
hipError_t launch_encode_fp8_rows(const void* in, bool in_bf16, int64_t rows, int64_t row_len, int64_t ld,
                                  uint8_t* codes, const uint32_t* amax_bits, float* scale_out, hipStream_t s);
// amax over the matrix, then launch_encode_fp8_rows.
hipError_t launch_quant_fp8_rows(const void* in, bool in_bf16, int64_t rows, int64_t row_len, int64_t ld,
                                 uint8_t* codes, uint32_t* amax_bits, float* scale_out, hipStream_t s);

}  // namespace mx
