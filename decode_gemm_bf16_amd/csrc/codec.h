// Host-side encoder of the exponent codec (Unweight page, sections 三, 四, 六).
//
// Builds, from a row-major bf16 matrix, the serial sign+mantissa stream, the
// 4-bit palette form with its raw-group tables, and the 12-bit length-limited
// canonical Huffman form with its chunk bit offsets and decode table.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace uw {

constexpr int kBrickRows = 16;
constexpr int kBrickCols = 64;
constexpr int kBrickWeights = kBrickRows * kBrickCols;  // 1024
constexpr int kRun = 16;                                // weights of one row per run
constexpr int kChunk = 256;                             // Huffman symbols per chunk
constexpr int kLmax = 12;                               // longest code, bits
constexpr int kLutSize = 1 << kLmax;                    // decode table entries
constexpr int kStreamPadWords = 8;                      // zero words after the stream

struct HostFormat {
  int64_t rows = 0, cols = 0;
  uint32_t formats = 0;
  uint64_t hist[256] = {};
  uint32_t distinct = 0;
  std::vector<uint8_t> sm;  // serial sign+mantissa bytes

  // palette form
  uint8_t palette[16] = {};
  std::vector<uint8_t> nib;         // serial 4-bit codes, 8 codes per 4 bytes
  std::vector<uint32_t> rawmap;     // per brick: bit r = row r's group is raw
  std::vector<uint32_t> rawbefore;  // per brick: raw groups in earlier bricks
  std::vector<uint8_t> side;        // 64 original exponents per raw group
  uint64_t n_raw = 0;
  uint32_t max_row_raw = 0xFFFFFFFFu;  // most raw groups in one brick-row (16 rows); unknown: all ones

  // Huffman form
  uint8_t lengths[256] = {};
  uint32_t codes[256] = {};
  std::vector<uint32_t> words;      // payload + kStreamPadWords zero words
  uint64_t stream_bits = 0;
  std::vector<uint32_t> offsets;    // first bit of each chunk
  std::vector<uint16_t> lut;        // 4096 entries: symbol | length << 8

  uint64_t n() const { return uint64_t(rows) * uint64_t(cols); }
  uint64_t bricks() const { return n() / kBrickWeights; }
  double bpw_palette() const;
  double bpw_huffman() const;
};

// Most raw groups in one brick-row (kbn consecutive bricks) from the per-brick
// raw maps and raw-groups-before counts.
uint32_t max_row_raw(const uint32_t* rawmap, const uint32_t* rawbefore, uint64_t bricks, uint64_t kbn);

// Returns an empty string on success, else the reason.  `formats` uses the
// UW_FMT_* flags of uw.h (palette tables are built for PALETTE or RAWAUX).
std::string encode_host(const uint16_t* w, int64_t rows, int64_t cols, uint32_t formats,
                        HostFormat& out);

// Multi-symbol decode table: for each 12-bit window, the whole codes it
// starts with, greedily and at most three: bits 0-23 the symbols (first in the
// low byte), bits 24-25 their count (>= 1 for a complete code), bits 26-29
// the bits they take.  Built from the one-symbol table `lut`.
std::vector<uint32_t> multi_symbol_table(const std::vector<uint16_t>& lut);

// Decode table for pipeline 3: for each 12-bit window, the 4-bit palette
// codes (code_of[symbol]; symbols outside the palette, which only occur in
// raw groups, get 0) of the whole codes it starts with, greedily and at most
// five: bits 0-19 the codes (first in the low nibble), bits 20-23 the bits
// they take, bits 24-31 four times their count (the bits they fill).
std::vector<uint32_t> multi_code_table(const std::vector<uint16_t>& lut, const uint8_t code_of[256]);

// Section 四: the palette of a histogram (the 16 most frequent exponents, ties
// to the smaller value, padded with entry 0) and code_of[e] = e's palette
// index or -1.  Returns the number of distinct palette entries (<= 16).
int select_palette(const uint64_t hist[256], uint8_t palette[16], int16_t code_of[256]);

// The canonical code of f.hist: lengths, codes, stream_bits and the one-symbol
// decode table (f.words and f.offsets are left alone).  Empty string on
// success, else the reason.
std::string huffman_tables(HostFormat& f);

// Length-limited optimal code lengths over a 256-symbol histogram.
void limited_code_lengths(const uint64_t hist[256], int lmax, uint8_t lengths[256]);

}  // namespace uw
