"""CPU oracle for the lossless BF16 exponent codec and its matmul.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  It shares no code, table or helper with the HIP library in
``decode_gemm_bf16_amd``, and never imports it.

Everything here is plain, slow and meant to be checked by eye against the
Unweight page ("Unweight: how Cloudflare compresses large models by 22% without
losing precision"):

* section 三 (the pattern inside BF16 weights): a BF16 word is 1 sign bit,
  8 exponent bits and 7 mantissa bits; sign and mantissa look random, the
  exponent byte is highly redundant;
* section 四 (compression strategy): only the exponent byte is Huffman coded,
  sign and mantissa are kept verbatim; a 16-entry palette of the most common
  exponents; a 64-weight row holding any exponent outside the palette is stored
  raw;
* section 六 (four pipelines): the palette form is 4 bits per exponent;
* section 十 (results): the round trip is bit-exact.

The matmul reference is fp64 over the original BF16 values, independent of any
codec.  Parity status of each function is listed in ``PARITY``.
"""
from .codec import (  # noqa: F401
    BRICK_ROWS, BRICK_COLS, GROUP, CHUNK, LMAX, PALETTE_SIZE,
    split, join, serial_index, to_serial, from_serial, histogram,
    choose_palette, raw_group_flags, palette_encode, palette_decode,
    palette_bits_per_weight, entropy_bits, top_k_coverage,
)
from .huffman import (  # noqa: F401
    huffman_lengths, canonical_codes, huffman_encode, huffman_decode,
    huffman_decode_chunks, huffman_bits_per_weight, kraft_sum,
)
from .bundle import read_bundle, write_bundle, transcode_bundle  # noqa: F401
from .gemm import (  # noqa: F401
    bf16_to_f64, f64_to_bf16_rne, matmul_fp64, matmul_fp64_rows, silu_mul_bf16,
    mlp_layer_fp64, rel_err,
)

# Every oracle function and what pins it (tests/test_oracle_*.py).  None is
# "parity unpinned".
PARITY = {
    "split/join": "exhaustive 65,536-pattern round trip; bit-field identities",
    "serial_index": "bijection; brick/lane coordinates recomputed by loops on a small case",
    "histogram/choose_palette": "brute-force count; hand cases with ties and <16 symbols",
    "raw_group_flags": "brute-force scan; <=16 distinct exponents gives no raw group",
    "palette_encode/decode": "bit-exact round trip incl. all 65,536 patterns; nibble packing by hand",
    "huffman_lengths": "Kraft equality; dyadic closed form; brute-force optimum on tiny alphabets; "
                       "independent DP optimum for length-limited codes; Shannon bound",
    "canonical_codes": "prefix-free by brute force; hand-worked example",
    "huffman_encode/decode": "bit-exact round trip; hand-worked bitstream fixture",
    "matmul_fp64": "exact rational (Fraction) sums on the tiny case; one-hot identity",
    "silu_mul_bf16": "closed-form values; RNE ties by hand",
    "write_bundle/read_bundle": "round trip to the original weights; byte-equal to the library's own writer "
                                "(an independent implementation of the same layout); header fields by struct",
    "transcode_bundle": "equals palette_encode of the original weights (the Huffman round trip is exact)",
}
