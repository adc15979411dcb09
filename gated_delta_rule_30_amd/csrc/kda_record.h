// The per-(chunk, head) record of the chunk path: what the record kernels (prep_kernel, and
// rec256_kernel at 256 key channels) write and the state kernel reads. Device-side layout only.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ====================================================================== record layout
// Matrices are stored as MFMA A-operand fragments: for a matrix with R rows and reduction
// length L, the 16-byte slot of (row tile, reduction step, lane) is at element
//     ((tile * (L / KS) + step) * 64 + lane) * EPL
// and element e of the slot of lane (m, g) is (row 16*tile + m, index KS*step + kk(g, e)).
template <int K, typename MT>
struct Rec {
  static constexpr size_t oW = 0;                                // [CHUNK rows][K]
  static constexpr size_t oQ = oW + (size_t)CHUNK * K;           // [CHUNK rows][K]
  static constexpr size_t oKt = oQ + (size_t)CHUNK * K;          // [K rows][CHUNK]
  static constexpr size_t oTb = oKt + (size_t)K * CHUNK;         // [CHUNK rows][CHUNK]
  static constexpr size_t oPb = oTb + (size_t)CHUNK * CHUNK;     // [CHUNK rows][CHUNK]
  static constexpr size_t nMat = oPb + (size_t)CHUNK * CHUNK;
  static constexpr size_t oGamBytes = nMat * sizeof(MT);         // K fp32
  static constexpr size_t bytes = (oGamBytes + K * 4 + 1023) / 1024 * 1024;  // whole 1 KB slots
  // then V of the chunk, slice-major: slice c (value columns 16c .. 16c+15) is CHUNK rows of 16
  // values, 16 * CHUNK * sizeof(MT) bytes, at oVBytes + c * 16 * CHUNK * sizeof(MT)
  static constexpr size_t oVBytes = bytes;
  static constexpr size_t vslice_bytes = (size_t)16 * CHUNK * sizeof(MT);
};

template <typename MT>
__device__ __forceinline__ size_t slot_elem(int tile, int step, int lane, int L) {
  return ((size_t)(tile * (L / Mma<MT>::KS) + step) * 64 + lane) * Mma<MT>::EPL;
}

}  // namespace kda
