// Load-time transcode of the Huffman form into the direct-palette form, on
// the device (Unweight page, section 六: the direct-palette pipeline reads
// weights that were transcoded into the compact 4-bit form when the model was
// loaded; section 十: the distribution bundle compresses every MLP matrix).
//
// Input: the exponent bytes of a whole matrix as the Huffman decoder writes
// them for pipeline 2 (runs of 16 in the 512-chunk interleaved order: run r
// of chunk c at byte 16 * (((c / 512) * 16 + r) * 512 + c % 512)).  Output:
// exactly the tables the host encoder builds (per-brick raw map and raw
// groups before, 4-bit codes in serial order, raw groups' exponents).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace uw {

// code_of[e] = palette index of exponent value e, or -1 outside the palette.
struct CodeOfTable {
  int8_t c[256];
};

// Bricks per workgroup of the transcode kernels, and their workgroup count.
constexpr int kTranscodeBricks = 16;
inline uint64_t transcode_groups(uint64_t bricks) { return (bricks + kTranscodeBricks - 1) / kTranscodeBricks; }

// rawmap[b] = bit r set when row r of brick b holds an exponent outside the
// palette (its 64-weight group is stored raw); wg_count[g] = raw groups of
// bricks 16g..16g+15.
hipError_t launch_raw_rows(const uint8_t* exps, uint64_t bricks, const CodeOfTable& code_of, uint32_t* rawmap,
                           uint32_t* wg_count, hipStream_t s);

// wg_before[g] = sum of wg_count[0..g-1]; *total = the sum of all `groups`.
hipError_t launch_raw_scan(const uint32_t* wg_count, uint64_t groups, uint32_t* wg_before, uint32_t* total,
                           hipStream_t s);

// meta[b] = {rawmap[b], raw groups in bricks 0..b-1}, the 4-bit codes (nib,
// may be null; zeros on raw rows) and the raw groups' exponents (side, may
// be null; 64 bytes per raw group at meta[b].y + rank of the row).
hipError_t launch_palette_pack(const uint8_t* exps, uint64_t bricks, const CodeOfTable& code_of,
                               const uint32_t* rawmap, const uint32_t* wg_before, uint2* meta, uint8_t* nib,
                               uint8_t* side, hipStream_t s);

}  // namespace uw
