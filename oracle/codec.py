"""Oracle: BF16 field split, palette format and the serial (brick) order.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg.  Shares no code with the HIP library.

Readings of the Unweight page taken here (the page leaves them open):

* The split (section 三): exponent byte ``e = (w >> 7) & 0xFF``; the
  sign+mantissa byte keeps the sign in bit 7 and the 7 mantissa bits in bits
  6..0.
* A "row of 64 weights" (section 四) is 64 consecutive weights along the input
  dimension of one output row of W[rows, cols]; cols must be a multiple of 64.
* One palette per matrix: the 16 most frequent exponents, ranked by
  (count descending, exponent ascending); index = rank; fewer than 16 distinct
  exponents pads with the first entry.
* Serial order.  Every per-weight stream (sign+mantissa bytes, exponent
  bytes, palette codes, the Huffman symbol sequence) lists the weights in
  "brick" order: bricks of 16 rows x 64 columns, brick-rows top to bottom and
  bricks left to right inside a brick-row; inside a brick, 64 runs of 16
  weights, run ``l`` (0..63) covering row ``l % 16`` and columns
  ``16*(l//16) .. 16*(l//16)+15``.  This needs rows % 16 == 0.
* Palette codes are packed 8 to 4 bytes: of 8 consecutive serial codes, byte b
  (0..3) holds code b in its low nibble and code b+4 in its high nibble.
  Every code of a raw group is 0.
* Raw groups: per brick a 16-bit map (bit r set when row r's 64-weight group in
  that brick is raw) and the number of raw groups in all earlier bricks; the
  side table lists the raw groups' 64 original exponent bytes, brick by brick
  and, inside a brick, by row.
"""
from __future__ import annotations

import numpy as np

BRICK_ROWS = 16
BRICK_COLS = 64
GROUP = 64            # weights per palette group ("row of 64 weights", section 四)
RUN = 16              # weights of one row inside a brick that form one serial run
CHUNK = 256           # Huffman symbols per independently decodable chunk
LMAX = 12             # longest Huffman code
PALETTE_SIZE = 16     # 4-bit palette


def check_shape(rows: int, cols: int) -> None:
    if rows <= 0 or cols <= 0 or rows % BRICK_ROWS or cols % BRICK_COLS:
        raise ValueError(f"shape {rows}x{cols}: rows must be a multiple of 16 and cols of 64")


def split(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """BF16 bit patterns -> (exponent bytes, sign+mantissa bytes).  Section 三."""
    w = np.asarray(w, dtype=np.uint16)
    e = ((w >> 7) & 0xFF).astype(np.uint8)
    sign = (w >> 15) & 1
    mant = w & 0x7F
    sm = ((sign << 7) | mant).astype(np.uint8)
    return e, sm


def join(e: np.ndarray, sm: np.ndarray) -> np.ndarray:
    """Inverse of split: sign<<15 | exponent<<7 | mantissa."""
    e = np.asarray(e, dtype=np.uint16)
    sm = np.asarray(sm, dtype=np.uint16)
    sign = (sm >> 7) & 1
    mant = sm & 0x7F
    return ((sign << 15) | (e << 7) | mant).astype(np.uint16)


def serial_index(rows: int, cols: int) -> np.ndarray:
    """Row-major flat index of the weight at each serial position (brick order)."""
    check_shape(rows, cols)
    flat = np.arange(rows * cols, dtype=np.int64)
    # axes of the reshaped index: brick-row, row in brick, brick-column, quarter, j
    flat = flat.reshape(rows // BRICK_ROWS, BRICK_ROWS, cols // BRICK_COLS, BRICK_COLS // RUN, RUN)
    # serial order: brick-row, brick-column, run l = quarter*16 + row, j
    return flat.transpose(0, 2, 3, 1, 4).reshape(-1)


def to_serial(a: np.ndarray) -> np.ndarray:
    rows, cols = a.shape
    return np.ascontiguousarray(a).reshape(-1)[serial_index(rows, cols)]


def from_serial(s: np.ndarray, rows: int, cols: int) -> np.ndarray:
    out = np.empty(rows * cols, dtype=s.dtype)
    out[serial_index(rows, cols)] = s
    return out.reshape(rows, cols)


def histogram(e: np.ndarray) -> np.ndarray:
    """Count of each of the 256 exponent values."""
    return np.bincount(np.asarray(e, dtype=np.uint8).reshape(-1), minlength=256).astype(np.int64)


def entropy_bits(cnt: np.ndarray) -> float:
    """Shannon entropy (bits per exponent) of a histogram."""
    p = cnt[cnt > 0] / cnt.sum()
    return float(-(p * np.log2(p)).sum())


def top_k_coverage(cnt: np.ndarray, k: int = PALETTE_SIZE) -> float:
    return float(np.sort(cnt)[::-1][:k].sum() / cnt.sum())


def choose_palette(cnt: np.ndarray) -> np.ndarray:
    """The 16 most frequent exponents, (count desc, exponent asc); padded with entry 0."""
    present = [s for s in range(256) if cnt[s] > 0]
    ranked = sorted(present, key=lambda s: (-int(cnt[s]), s))[:PALETTE_SIZE]
    while len(ranked) < PALETTE_SIZE:
        ranked.append(ranked[0])
    return np.array(ranked, dtype=np.uint8)


def raw_group_flags(e: np.ndarray, palette: np.ndarray) -> np.ndarray:
    """flags[r, g] = True when any exponent in W[r, 64g:64g+64] is outside the palette."""
    rows, cols = e.shape
    inside = np.isin(e, palette)
    return ~inside.reshape(rows, cols // GROUP, GROUP).all(axis=2)


def palette_encode(w: np.ndarray) -> dict:
    """The direct-palette format of a [rows, cols] bf16 matrix (section 四, section 六)."""
    w = np.asarray(w, dtype=np.uint16)
    rows, cols = w.shape
    check_shape(rows, cols)
    e, sm = split(w)
    cnt = histogram(e)
    pal = choose_palette(cnt)
    flags = raw_group_flags(e, pal)

    # code of each exponent value: its first position in the palette
    code_of = np.zeros(256, dtype=np.uint8)
    for i in range(PALETTE_SIZE - 1, -1, -1):
        code_of[pal[i]] = i
    codes = code_of[e]
    codes[np.repeat(flags, GROUP, axis=1)] = 0

    codes_s = to_serial(codes)
    sm_s = to_serial(sm)
    units = codes_s.reshape(-1, 8).astype(np.uint8)
    nib = (units[:, 0:4] | (units[:, 4:8] << 4)).astype(np.uint8).reshape(-1)

    n_brow, n_bcol = rows // BRICK_ROWS, cols // BRICK_COLS
    bitmap = np.zeros(n_brow * n_bcol, dtype=np.uint32)
    before = np.zeros(n_brow * n_bcol, dtype=np.uint32)
    side = []
    seen = 0
    for tb in range(n_brow):
        for kb in range(n_bcol):
            b = tb * n_bcol + kb
            before[b] = seen
            for r in range(BRICK_ROWS):
                row = tb * BRICK_ROWS + r
                if flags[row, kb]:
                    bitmap[b] |= np.uint32(1 << r)
                    side.append(e[row, kb * GROUP:(kb + 1) * GROUP])
                    seen += 1
    side_tab = np.concatenate(side).astype(np.uint8) if side else np.zeros(0, dtype=np.uint8)
    return dict(rows=rows, cols=cols, palette=pal, counts=cnt, flags=flags,
                nibbles=nib, sm=sm_s, brick_rawmap=bitmap, brick_rawbefore=before,
                side=side_tab, n_raw=seen)


def palette_decode(enc: dict) -> np.ndarray:
    """Rebuild the bf16 bit patterns from the palette format."""
    rows, cols = enc["rows"], enc["cols"]
    nib = np.asarray(enc["nibbles"], dtype=np.uint8).reshape(-1, 4)
    codes_s = np.empty((nib.shape[0], 8), dtype=np.uint8)
    codes_s[:, 0:4] = nib & 0x0F
    codes_s[:, 4:8] = nib >> 4
    e_s = enc["palette"][codes_s.reshape(-1)]
    e = from_serial(e_s, rows, cols)
    n_bcol = cols // BRICK_COLS
    side = enc["side"]
    for b, bm in enumerate(enc["brick_rawmap"]):
        k = int(enc["brick_rawbefore"][b])
        tb, kb = divmod(b, n_bcol)
        for r in range(BRICK_ROWS):
            if int(bm) >> r & 1:
                e[tb * BRICK_ROWS + r, kb * GROUP:(kb + 1) * GROUP] = side[k * GROUP:(k + 1) * GROUP]
                k += 1
    sm = from_serial(np.asarray(enc["sm"], dtype=np.uint8), rows, cols)
    return join(e, sm)


def palette_bits_per_weight(enc: dict) -> float:
    """Stored bits per weight: sign+mantissa 8, code 4, raw side table, per-brick
    map + count (2 x 32 bits), palette 16 bytes."""
    n = enc["rows"] * enc["cols"]
    nbricks = len(enc["brick_rawmap"])
    bits = 8 * n + 4 * n + 8 * GROUP * enc["n_raw"] + 64 * nbricks + 8 * PALETTE_SIZE
    return bits / n
