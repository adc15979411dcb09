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
  // values, 16 * CHUNK * sizeof(MT) bytes, at oVBytes + c * 16 * CHUNK * sizeof(MT).
  // In the U form of the record (bf16, 128 value columns, up to 128 key channels) the same
  // bytes hold U = T'V instead, and the T' slots are not written: slice c holds the four
  // 16 x 16 result tiles of U (token tile t, value columns 16c ..), lane l's four values of
  // tile t at byte ((t / 2) * 64 + l) * 16 + (t % 2) * 8 of the slice (two tiles per 16 bytes).
  static constexpr size_t oVBytes = bytes;
  static constexpr size_t vslice_bytes = (size_t)16 * CHUNK * sizeof(MT);
  __device__ __forceinline__ static size_t u_tile_byte(int slice, int t, int lane) {
    return oVBytes + (size_t)slice * vslice_bytes + ((size_t)(t >> 1) * 64 + lane) * 16 + (t & 1) * 8;
  }
};

template <typename MT>
__device__ __forceinline__ size_t slot_elem(int tile, int step, int lane, int L) {
  return ((size_t)(tile * (L / Mma<MT>::KS) + step) * 64 + lane) * Mma<MT>::EPL;
}

}  // namespace kda
