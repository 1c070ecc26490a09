"""Oracle: length-limited canonical Huffman code of the exponent stream.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg.  Shares no code with the HIP library.

The Unweight page (section 四) Huffman-codes the exponent bytes only, giving
short codes to common exponents and long ones to rare exponents; the
sign+mantissa bytes stay verbatim.  It names no code-length limit, no code
assignment and no bit order.  Readings taken here:

* Optimal code lengths under a 12-bit limit (package-merge over the symbols
  that occur).  Leaves are ordered by (count, symbol) ascending and, when a
  leaf and a package weigh the same, the leaf is taken first.  A stream with a
  single distinct exponent adds the smallest unused byte value as a phantom
  symbol so that both get 1-bit codes.
* Canonical codes in (length, symbol) order: the first code is all zeros and
  each next code is the previous plus one, shifted left by the length step.
* Bits are written most-significant first into little-endian 32-bit words:
  bit 31 of word 0 is the first bit of the stream; the tail is zero-padded.
* The symbol sequence is the serial (brick) order of ``codec.serial_index``; the
  stream is cut into chunks of 256 symbols and ``offsets[c]`` is the bit at
  which chunk c starts, so any chunk decodes on its own.
"""
from __future__ import annotations

import numpy as np

from .codec import CHUNK, LMAX, check_shape, histogram, split, join, to_serial, from_serial


def kraft_sum(lengths: np.ndarray) -> float:
    from fractions import Fraction
    return float(sum(Fraction(1, 2 ** int(l)) for l in lengths if l > 0))


def huffman_lengths(cnt: np.ndarray, lmax: int = LMAX) -> np.ndarray:
    """Optimal code lengths with no code longer than ``lmax`` bits (package-merge)."""
    cnt = np.asarray(cnt, dtype=np.int64)
    lengths = np.zeros(len(cnt), dtype=np.int64)
    present = [s for s in range(len(cnt)) if cnt[s] > 0]
    if not present:
        raise ValueError("empty histogram")
    if len(present) == 1:
        phantom = min(s for s in range(len(cnt)) if s != present[0])
        lengths[present[0]] = 1
        lengths[phantom] = 1
        return lengths
    if len(present) > 2 ** lmax:
        raise ValueError("alphabet too large for the length limit")
    leaves = sorted(present, key=lambda s: (int(cnt[s]), s))
    n = len(leaves)
    # an entry is (weight, how many times each leaf occurs inside it)
    leaf_entries = []
    for i, s in enumerate(leaves):
        v = np.zeros(n, dtype=np.int64)
        v[i] = 1
        leaf_entries.append((int(cnt[s]), v))

    current = list(leaf_entries)
    for _ in range(lmax - 1):
        packages = [(current[2 * i][0] + current[2 * i + 1][0], current[2 * i][1] + current[2 * i + 1][1])
                    for i in range(len(current) // 2)]
        merged = []
        a = b = 0
        while a < len(leaf_entries) or b < len(packages):
            take_leaf = b >= len(packages) or (a < len(leaf_entries) and leaf_entries[a][0] <= packages[b][0])
            if take_leaf:
                merged.append(leaf_entries[a])
                a += 1
            else:
                merged.append(packages[b])
                b += 1
        current = merged
    chosen = current[:2 * n - 2]
    depth = np.sum([v for _, v in chosen], axis=0)
    for i, s in enumerate(leaves):
        lengths[s] = depth[i]
    return lengths


def canonical_codes(lengths: np.ndarray) -> np.ndarray:
    """Canonical code value of each symbol (0 where the length is 0)."""
    order = sorted([s for s in range(len(lengths)) if lengths[s] > 0], key=lambda s: (int(lengths[s]), s))
    codes = np.zeros(len(lengths), dtype=np.int64)
    code = 0
    prev = int(lengths[order[0]])
    for s in order:
        code <<= int(lengths[s]) - prev
        prev = int(lengths[s])
        codes[s] = code
        code += 1
    return codes


def _pack_bits(symbols: np.ndarray, lengths: np.ndarray, codes: np.ndarray) -> tuple[np.ndarray, np.ndarray, int]:
    L = lengths[symbols]
    C = codes[symbols]
    starts = np.zeros(len(symbols), dtype=np.int64)
    if len(symbols) > 1:
        starts[1:] = np.cumsum(L)[:-1]
    total = int(L.sum())
    nwords = (total + 31) // 32
    bits = np.zeros(nwords * 32, dtype=np.uint8)
    for j in range(int(L.max())):
        m = L > j
        bits[starts[m] + j] = (C[m] >> (L[m] - 1 - j)) & 1
    words = np.frombuffer(np.packbits(bits).tobytes(), dtype=">u4").astype(np.uint32)
    return words, starts, total


def huffman_encode(w: np.ndarray, chunk: int = CHUNK, lmax: int = LMAX) -> dict:
    """Huffman format of a [rows, cols] bf16 matrix: code lengths, bitstream,
    chunk offsets and the verbatim sign+mantissa bytes (all in serial order)."""
    w = np.asarray(w, dtype=np.uint16)
    rows, cols = w.shape
    check_shape(rows, cols)
    e, sm = split(w)
    cnt = histogram(e)
    lengths = huffman_lengths(cnt, lmax)
    codes = canonical_codes(lengths)
    es = to_serial(e)
    words, starts, total = _pack_bits(es.astype(np.int64), lengths, codes)
    if total >= 2 ** 32:
        raise ValueError("stream longer than 2^32 bits")
    offsets = starts[::chunk].astype(np.uint32)
    return dict(rows=rows, cols=cols, counts=cnt, lengths=lengths.astype(np.uint8), codes=codes,
                words=words, offsets=offsets, total_bits=total, chunk=chunk, sm=to_serial(sm))


def _decode_tables(lengths: np.ndarray):
    lmax = int(lengths.max())
    count = [0] * (lmax + 2)
    for l in lengths:
        if l > 0:
            count[int(l)] += 1
    first = [0] * (lmax + 2)
    index = [0] * (lmax + 2)
    code = 0
    idx = 0
    for l in range(1, lmax + 1):
        code = (code + count[l - 1]) << 1 if l > 1 else 0
        first[l] = code
        index[l] = idx
        idx += count[l]
    ordered = sorted([s for s in range(len(lengths)) if lengths[s] > 0], key=lambda s: (int(lengths[s]), s))
    return lmax, count, first, index, ordered


def decode_chunk(words: np.ndarray, start_bit: int, nsym: int, lengths: np.ndarray, _tables=None) -> np.ndarray:
    """Decode ``nsym`` symbols from bit ``start_bit``, one bit at a time."""
    lmax, count, first, index, ordered = _tables or _decode_tables(lengths)
    out = np.empty(nsym, dtype=np.uint8)
    pos = int(start_bit)
    for i in range(nsym):
        code = 0
        l = 0
        while True:
            bit = (int(words[pos >> 5]) >> (31 - (pos & 31))) & 1
            pos += 1
            code = (code << 1) | bit
            l += 1
            if l > lmax:
                raise ValueError("invalid code in stream")
            if count[l] and 0 <= code - first[l] < count[l]:
                out[i] = ordered[index[l] + code - first[l]]
                break
    return out


def huffman_decode_chunks(enc: dict, chunk_ids) -> dict:
    """Decode selected chunks; returns {chunk id: exponent bytes in serial order}."""
    tables = _decode_tables(enc["lengths"])
    n = enc["rows"] * enc["cols"]
    ch = enc["chunk"]
    out = {}
    for c in chunk_ids:
        c = int(c)
        nsym = min(ch, n - c * ch)
        out[c] = decode_chunk(enc["words"], int(enc["offsets"][c]), nsym, enc["lengths"], tables)
    return out


def huffman_decode(enc: dict) -> np.ndarray:
    """Full decode back to the [rows, cols] bf16 bit patterns."""
    rows, cols = enc["rows"], enc["cols"]
    nchunks = len(enc["offsets"])
    parts = huffman_decode_chunks(enc, range(nchunks))
    es = np.concatenate([parts[c] for c in range(nchunks)])
    e = from_serial(es, rows, cols)
    sm = from_serial(np.asarray(enc["sm"], dtype=np.uint8), rows, cols)
    return join(e, sm)


def huffman_bits_per_weight(enc: dict) -> float:
    """Stored bits per weight: sign+mantissa 8 + stream (whole words) + 32-bit chunk
    offsets + the 256 code lengths."""
    n = enc["rows"] * enc["cols"]
    bits = 8 * n + 32 * len(enc["words"]) + 32 * len(enc["offsets"]) + 8 * 256
    return bits / n
