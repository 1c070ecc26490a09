// Host-side encoder: split, histogram, palette, raw groups, length-limited
// canonical Huffman, chunk offsets.  Unweight page, sections 三, 四 and 六.
#include "codec.h"

#include <algorithm>
#include <array>
#include <cstring>
#include <numeric>

#include "../../include/uw.h"

namespace uw {
namespace {

// Visit the weights of W in serial order: bricks of 16x64 (brick-rows, then
// bricks left to right), inside a brick 64 runs of 16 (run l = row l%16,
// columns 16*(l/16)..), calling f(serial_index, row_major_index) per run start.
template <class F>
void for_each_run(int64_t rows, int64_t cols, F&& f) {
  const int64_t bcols = cols / kBrickCols;
  uint64_t s = 0;
  for (int64_t tb = 0; tb < rows / kBrickRows; ++tb)
    for (int64_t kb = 0; kb < bcols; ++kb)
      for (int l = 0; l < 64; ++l, s += kRun) {
        const int64_t r = tb * kBrickRows + (l % 16);
        const int64_t c = kb * kBrickCols + kRun * (l / 16);
        f(s, uint64_t(r * cols + c));
      }
}

struct PmEntry {
  uint64_t weight;
  int32_t leaf;   // >= 0: leaf index into the sorted leaves; -1: package
  int32_t child;  // package: index of its first child in the previous list
};

}  // namespace

// Package-merge (optimal prefix code lengths with a length limit).  Leaves are
// ordered by (count, symbol) ascending; a leaf is taken before a package of the
// same weight; the 2n-2 lightest entries of the final list are kept and a
// leaf's code length is the number of kept entries it belongs to.
void limited_code_lengths(const uint64_t hist[256], int lmax, uint8_t lengths[256]) {
  std::memset(lengths, 0, 256);
  std::vector<int> leaves;
  for (int s = 0; s < 256; ++s)
    if (hist[s]) leaves.push_back(s);
  if (leaves.empty()) return;
  if (leaves.size() == 1) {  // one symbol: pair it with the smallest unused byte value
    const int only = leaves[0];
    lengths[only] = 1;
    lengths[only == 0 ? 1 : 0] = 1;
    return;
  }
  std::stable_sort(leaves.begin(), leaves.end(), [&](int a, int b) { return hist[a] < hist[b]; });
  const int n = int(leaves.size());

  std::vector<std::vector<PmEntry>> level(lmax);
  level[0].reserve(n);
  for (int i = 0; i < n; ++i) level[0].push_back({hist[leaves[i]], i, -1});
  for (int d = 1; d < lmax; ++d) {
    const auto& prev = level[d - 1];
    auto& cur = level[d];
    cur.reserve(2 * n);
    size_t li = 0, pi = 0;
    const size_t npack = prev.size() / 2;
    while (li < size_t(n) || pi < npack) {
      const bool leaf_first =
          pi >= npack ||
          (li < size_t(n) && hist[leaves[li]] <= prev[2 * pi].weight + prev[2 * pi + 1].weight);
      if (leaf_first) {
        cur.push_back({hist[leaves[li]], int32_t(li), -1});
        ++li;
      } else {
        cur.push_back({prev[2 * pi].weight + prev[2 * pi + 1].weight, -1, int32_t(2 * pi)});
        ++pi;
      }
    }
  }
  // Count leaf occurrences among the kept entries, level by level downwards.
  std::vector<int> depth(n, 0);
  std::vector<char> keep(level[lmax - 1].size(), 0);
  std::fill(keep.begin(), keep.begin() + std::min<size_t>(2 * n - 2, keep.size()), 1);
  for (int d = lmax - 1; d >= 0; --d) {
    const auto& cur = level[d];
    std::vector<char> below(d > 0 ? level[d - 1].size() : 0, 0);
    for (size_t i = 0; i < cur.size(); ++i) {
      if (!keep[i]) continue;
      if (cur[i].leaf >= 0) {
        ++depth[cur[i].leaf];
      } else {
        below[cur[i].child] = 1;
        below[cur[i].child + 1] = 1;
      }
    }
    keep.swap(below);
  }
  for (int i = 0; i < n; ++i) lengths[leaves[i]] = uint8_t(depth[i]);
}

double HostFormat::bpw_palette() const {
  const double bits = 12.0 * double(n()) + 512.0 * double(n_raw) + 64.0 * double(bricks()) + 128.0;
  return bits / double(n());
}

double HostFormat::bpw_huffman() const {
  const uint64_t payload_words = (stream_bits + 31) / 32;
  const double bits = 8.0 * double(n()) + 32.0 * double(payload_words) + 32.0 * double(offsets.size()) + 2048.0;
  return bits / double(n());
}

uint32_t max_row_raw(const uint32_t* rawmap, const uint32_t* rawbefore, uint64_t bricks, uint64_t kbn) {
  uint32_t best = 0;
  for (uint64_t b0 = 0; b0 + kbn <= bricks; b0 += kbn) {
    const uint64_t last = b0 + kbn - 1;
    const uint32_t n = rawbefore[last] + uint32_t(__builtin_popcount(rawmap[last])) - rawbefore[b0];
    if (n > best) best = n;
  }
  return best;
}

std::string encode_host(const uint16_t* w, int64_t rows, int64_t cols, uint32_t formats, HostFormat& f) {
  if (!w) return "null weight pointer";
  if (rows <= 0 || cols <= 0 || rows % kBrickRows || cols % kBrickCols)
    return "rows must be a positive multiple of 16 and cols a positive multiple of 64";
  if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31) || rows * cols > (int64_t(1) << 40))
    return "matrix too large";
  f = HostFormat();
  f.rows = rows;
  f.cols = cols;
  f.formats = formats;
  const uint64_t n = f.n();

  // Section 三: exponent byte and sign+mantissa byte, in serial order.
  std::vector<uint8_t> ex(n);
  f.sm.resize(n);
  for_each_run(rows, cols, [&](uint64_t s, uint64_t src) {
    for (int j = 0; j < kRun; ++j) {
      const uint16_t v = w[src + j];
      ex[s + j] = uint8_t(v >> 7);
      f.sm[s + j] = uint8_t(((v >> 8) & 0x80u) | (v & 0x7Fu));
    }
  });
  for (uint64_t i = 0; i < n; ++i) ++f.hist[ex[i]];
  for (int s = 0; s < 256; ++s) f.distinct += f.hist[s] != 0;

  const bool want_pal = formats & (UW_FMT_PALETTE | UW_FMT_RAWAUX);
  if (want_pal) {
    int16_t code_of[256];
    select_palette(f.hist, f.palette, code_of);

    const uint64_t nb = f.bricks();
    f.rawmap.assign(nb, 0);
    f.rawbefore.assign(nb, 0);
    if (formats & UW_FMT_PALETTE) f.nib.assign(n / 2, 0);
    uint64_t seen = 0;
    for (uint64_t b = 0; b < nb; ++b) {
      f.rawbefore[b] = uint32_t(seen);
      const uint8_t* eb = ex.data() + b * kBrickWeights;
      uint32_t map = 0;
      for (int r = 0; r < 16; ++r) {
        bool raw = false;
        for (int q = 0; q < 4 && !raw; ++q)
          for (int j = 0; j < kRun; ++j)
            if (code_of[eb[(q * 16 + r) * kRun + j]] < 0) { raw = true; break; }
        if (raw) map |= 1u << r;
      }
      f.rawmap[b] = map;
      // the raw groups' exponents, row by row, columns in order
      for (int r = 0; r < 16; ++r) {
        if (!(map >> r & 1)) continue;
        for (int q = 0; q < 4; ++q)
          f.side.insert(f.side.end(), eb + (q * 16 + r) * kRun, eb + (q * 16 + r + 1) * kRun);
        ++seen;
      }
      if (formats & UW_FMT_PALETTE) {
        uint8_t* nb4 = f.nib.data() + b * (kBrickWeights / 2);
        for (int l = 0; l < 64; ++l) {
          const bool raw = map >> (l % 16) & 1;
          for (int u = 0; u < 2; ++u) {  // two units of 8 codes per run
            for (int bb = 0; bb < 4; ++bb) {
              const int lo = raw ? 0 : code_of[eb[l * kRun + u * 8 + bb]];
              const int hi = raw ? 0 : code_of[eb[l * kRun + u * 8 + bb + 4]];
              nb4[l * 8 + u * 4 + bb] = uint8_t(lo | (hi << 4));
            }
          }
        }
      }
    }
    if (seen > 0xFFFFFFFFull) return "too many raw groups";
    f.max_row_raw = max_row_raw(f.rawmap.data(), f.rawbefore.data(), nb, uint64_t(cols) / 64);
    f.n_raw = seen;
  }

  if (formats & UW_FMT_HUFFMAN) {
    std::string err = huffman_tables(f);
    if (!err.empty()) return err;
    const uint64_t total = f.stream_bits;
    const uint64_t payload = (total + 31) / 32;
    f.words.assign(payload + kStreamPadWords, 0);
    f.offsets.resize((n + kChunk - 1) / kChunk);
    uint64_t acc = 0;  // pending bits, right-aligned
    int pending = 0;
    uint64_t wi = 0, bitpos = 0;
    for (uint64_t i = 0; i < n; ++i) {
      if (i % kChunk == 0) f.offsets[i / kChunk] = uint32_t(bitpos);
      const int len = f.lengths[ex[i]];
      acc = (acc << len) | f.codes[ex[i]];
      pending += len;
      bitpos += len;
      if (pending >= 32) {
        pending -= 32;
        f.words[wi++] = uint32_t(acc >> pending);
        acc &= (uint64_t(1) << pending) - 1;
      }
    }
    if (pending) f.words[wi++] = uint32_t(acc << (32 - pending));
  }
  return std::string();
}

int select_palette(const uint64_t hist[256], uint8_t palette[16], int16_t code_of[256]) {
  // Section 四: the 16 most frequent exponents, ties to the smaller value;
  // with fewer than 16 distinct exponents the rest repeat entry 0
  std::array<int, 256> order;
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return hist[a] > hist[b]; });
  int distinct = 0;
  for (int s = 0; s < 256; ++s) distinct += hist[s] != 0;
  const int used = std::min(16, distinct);
  for (int i = 0; i < 16; ++i) palette[i] = uint8_t(order[i < used ? i : 0]);
  for (int s = 0; s < 256; ++s) code_of[s] = -1;
  for (int i = used - 1; i >= 0; --i) code_of[palette[i]] = int16_t(i);
  return used;
}

std::string huffman_tables(HostFormat& f) {
  limited_code_lengths(f.hist, kLmax, f.lengths);
  // Canonical codes: (length, symbol) order, consecutive values per length.
  std::array<int, 256> order;
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    const int la = f.lengths[a] ? f.lengths[a] : 99, lb = f.lengths[b] ? f.lengths[b] : 99;
    return la < lb;
  });
  std::memset(f.codes, 0, sizeof f.codes);
  uint32_t code = 0;
  int prev_len = f.lengths[order[0]];
  for (int i = 0; i < 256 && f.lengths[order[i]]; ++i) {
    const int s = order[i];
    code <<= (f.lengths[s] - prev_len);
    prev_len = f.lengths[s];
    f.codes[s] = code++;
  }
  uint64_t total = 0;
  for (int s = 0; s < 256; ++s) total += f.hist[s] * f.lengths[s];
  // bit positions are 32-bit on the device, look-ahead past the last code included
  if (total >= (uint64_t(1) << 32) - 1024) return "Huffman stream longer than 2^32 - 1024 bits";
  f.stream_bits = total;
  // Decode table: every 12-bit window starting with a code maps to it.
  f.lut.assign(kLutSize, 0);
  for (int s = 0; s < 256; ++s) {
    const int len = f.lengths[s];
    if (!len) continue;
    const uint32_t first = f.codes[s] << (kLmax - len), count = 1u << (kLmax - len);
    for (uint32_t k = 0; k < count; ++k) f.lut[first + k] = uint16_t(s | (len << 8));
  }
  return std::string();
}

std::vector<uint32_t> multi_symbol_table(const std::vector<uint16_t>& lut) {
  std::vector<uint32_t> out(kLutSize, 0);
  for (uint32_t p = 0; p < uint32_t(kLutSize); ++p) {
    uint32_t syms = 0, cnt = 0, pos = 0;
    while (cnt < 3) {
      // the code starting `pos` bits into the window (bits past the window read
      // as zeros: only a code that ends inside the window is taken)
      const uint16_t e = lut[(p << pos) & uint32_t(kLutSize - 1)];
      const uint32_t len = e >> 8;
      if (len == 0 || pos + len > uint32_t(kLmax)) break;
      syms |= uint32_t(e & 0xFF) << (8 * cnt);
      ++cnt;
      pos += len;
    }
    out[p] = syms | (cnt << 24) | (pos << 26);
  }
  return out;
}

std::vector<uint32_t> multi_code_table(const std::vector<uint16_t>& lut, const uint8_t code_of[256]) {
  std::vector<uint32_t> out(kLutSize, 0);
  for (uint32_t p = 0; p < uint32_t(kLutSize); ++p) {
    uint32_t codes = 0, cnt = 0, pos = 0;
    while (cnt < 5) {
      const uint16_t e = lut[(p << pos) & uint32_t(kLutSize - 1)];
      const uint32_t len = e >> 8;
      if (len == 0 || pos + len > uint32_t(kLmax)) break;
      codes |= uint32_t(code_of[e & 0xFF] & 0xFu) << (4 * cnt);
      ++cnt;
      pos += len;
    }
    out[p] = codes | (pos << 20) | ((4 * cnt) << 24);
  }
  return out;
}

}  // namespace uw
