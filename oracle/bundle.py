"""Distribution bundle and load-time transcode, plainly (TEST INFRASTRUCTURE).

Unweight page, section 十: the distribution bundle ships every MLP matrix in
compressed form; section 六: the direct-palette pipeline reads weights that
were transcoded to the 4-bit palette form when the model was loaded.

The bundle is the Huffman form of one matrix written to a file.  Its byte
layout (little-endian) is a choice of this project, fixed here and in the
library's header independently:

    header, 64 bytes:  b"UWBUNDLE", u32 version (1), u32 header bytes (64),
                       i64 rows, i64 cols, u64 stream bits, u32 chunk (256),
                       u32 code-length limit (12), u64 payload words,
                       u64 chunk offsets
    u64 counts[256]    exponent histogram (the canonical code is rebuilt from it)
    u32 offsets[...]   first bit of each chunk
    u32 words[...]     the bitstream, MSB first, no padding words
    u8  sm[rows*cols]  sign+mantissa bytes in serial order

The load-time transcode is defined as: decode the Huffman form back to the
weights, then build the palette form from them.
"""
import struct

import numpy as np

from .codec import CHUNK, LMAX, palette_encode
from .huffman import canonical_codes, huffman_decode, huffman_lengths

MAGIC = b"UWBUNDLE"
_HEADER = struct.Struct("<8sIIqqQIIQQ")


def write_bundle(path: str, enc: dict) -> None:
    """Write a ``huffman_encode`` result."""
    n = enc["rows"] * enc["cols"]
    words = np.asarray(enc["words"], dtype="<u4")
    offsets = np.asarray(enc["offsets"], dtype="<u4")
    head = _HEADER.pack(MAGIC, 1, _HEADER.size, enc["rows"], enc["cols"], int(enc["total_bits"]), CHUNK, LMAX,
                        len(words), len(offsets))
    with open(path, "wb") as f:
        f.write(head)
        f.write(np.asarray(enc["counts"], dtype="<u8").tobytes())
        f.write(offsets.tobytes())
        f.write(words.tobytes())
        f.write(np.asarray(enc["sm"], dtype=np.uint8).reshape(n).tobytes())


def read_bundle(path: str) -> dict:
    """Read a bundle into the fields of a ``huffman_encode`` result."""
    data = open(path, "rb").read()
    magic, version, hbytes, rows, cols, bits, chunk, lmax, nwords, noff = _HEADER.unpack_from(data, 0)
    if magic != MAGIC or version != 1 or hbytes != _HEADER.size:
        raise ValueError("not a version-1 bundle")
    n = rows * cols
    pos = hbytes
    counts = np.frombuffer(data, dtype="<u8", count=256, offset=pos).astype(np.int64)
    pos += 256 * 8
    offsets = np.frombuffer(data, dtype="<u4", count=noff, offset=pos).astype(np.uint32)
    pos += 4 * noff
    words = np.frombuffer(data, dtype="<u4", count=nwords, offset=pos).astype(np.uint32)
    pos += 4 * nwords
    sm = np.frombuffer(data, dtype=np.uint8, count=n, offset=pos).copy()
    pos += n
    if pos != len(data):
        raise ValueError("bundle size does not match its header")
    lengths = huffman_lengths(counts, lmax).astype(np.uint8)
    return dict(rows=rows, cols=cols, counts=counts, lengths=lengths, codes=canonical_codes(lengths),
                words=words, offsets=offsets, total_bits=bits, chunk=chunk, sm=sm)


def transcode_bundle(enc: dict) -> dict:
    """Palette form of the matrix a Huffman form holds: decode, then encode."""
    return palette_encode(huffman_decode(enc))
