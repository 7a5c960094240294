// Packed MXFP4 weight tiles streamed into registers in the block-scaled MFMA's B layout.
#pragma once
#include "device_common.h"

namespace moe {

// Packed-weight tiles. A 16-row tile of a weight matrix (rows of K/2 bytes, one 16-byte
// block per 32 contraction entries) is read in chunks of 256 contraction entries (8
// blocks). Each of the two 16-byte loads per lane covers 8 rows x 128 contiguous bytes, so
// every load instruction touches whole cache lines: lane l loads block 8c + l/8 of row l%8
// (first) and of row 8 + l%8 (second).
__device__ __forceinline__ void load_tile_chunk(const uint8_t *rows, int64_t row_bytes, int c, int nblocks,
                                                int lane, uint4 &first, uint4 &second) {
    const int kb = min(8 * c + (lane >> 3), nblocks - 1);   // clamped: the tail re-reads a real block
    const uint8_t *p = rows + (lane & 7) * row_bytes + kb * 16;
    first = *reinterpret_cast<const uint4 *>(p);
    second = *reinterpret_cast<const uint4 *>(p + 8 * row_bytes);
}

__device__ __forceinline__ uint32_t ror8_in_row(uint32_t v) {   // DPP row_ror:8 (lane n <-> n ^ 8)
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xf, 0xf, false));
}

// Afterwards lane (n = l%16, g = l/16) holds blocks 8c + 2g (lo) and 8c + 2g + 1 (hi) of
// row n. Lanes n < 8 loaded (row n, block 8c + 2g) and lanes n >= 8 (row n, block 8c + 2g +
// 1) themselves; the other halves are exchanged between lanes n and n ^ 8 by one rotation
// within each 16-lane row.
__device__ __forceinline__ void tile_chunk_to_mfma(const uint4 &first, const uint4 &second, int lane, uint4 &lo,
                                                   uint4 &hi) {
    const bool low = (lane & 15) < 8;
    const uint4 send = low ? second : first;
    const uint4 recv = make_uint4(ror8_in_row(send.x), ror8_in_row(send.y), ror8_in_row(send.z),
                                  ror8_in_row(send.w));
    lo = low ? first : recv;
    hi = low ? recv : second;
}

}  // namespace moe
