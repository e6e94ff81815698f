// DEV_V1 layout of a group-64 affine-quantized matrix (host and device).
//
// Row-tile of 64 rows x one group of 64 columns per block; inside a block
// the codes are ordered so that one 16-byte load per lane gives each lane
// whole 8-column (4-bit) or 4-column (8-bit) runs of four rows, and the
// (scale, bias) pairs of the block follow its codes.  The full description
// is in include/moegemv.h.
#pragma once
#include <stdint.h>

namespace mq {

constexpr int kGroup = 64;
constexpr int kTileRows = 64;
constexpr int kBlk4 = 2304;       // 4-bit: 2048 B codes + 256 B pairs
constexpr int kBlk8 = 4352;       // 8-bit: 4096 B codes + 256 B pairs
constexpr int kCodes4 = 2048;
constexpr int kCodes8 = 4096;

inline constexpr int blk_bytes(int bits) { return bits == 4 ? kBlk4 : kBlk8; }
inline constexpr int code_bytes(int bits) { return bits == 4 ? kCodes4 : kCodes8; }
inline constexpr int64_t pad_rows(int64_t rows) { return (rows + kTileRows - 1) / kTileRows * kTileRows; }

// Canonical 4-bit word (column e of eight at bit 4e) -> device order
// (column e at bit 4*(e/2) + 16*(e%2)), and back.
inline uint32_t compact_nibbles(uint32_t v) {   // low nibbles of the 4 bytes -> bits 0..15
    v &= 0x0F0F0F0Fu;
    v = (v | (v >> 4)) & 0x00FF00FFu;
    return (v | (v >> 8)) & 0x0000FFFFu;
}
inline uint32_t spread_nibbles(uint32_t v) {    // inverse of compact_nibbles
    v &= 0x0000FFFFu;
    v = (v | (v << 8)) & 0x00FF00FFu;
    return (v | (v << 4)) & 0x0F0F0F0Fu;
}
inline uint32_t nib_to_dev(uint32_t w) { return compact_nibbles(w) | (compact_nibbles(w >> 4) << 16); }
inline uint32_t nib_from_dev(uint32_t w) { return spread_nibbles(w) | (spread_nibbles(w >> 16) << 4); }

}  // namespace mq
