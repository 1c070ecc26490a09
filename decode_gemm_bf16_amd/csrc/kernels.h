// Launchers of the gfx950 kernels (definitions in *.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace uw {

// What a fused kernel reads for W (all per-weight streams in serial brick order).
struct FusedW {
  const uint8_t* sm;       // sign+mantissa bytes, 1 per weight
  const uint8_t* codes;    // palette mode: 4-bit codes (0.5 B/weight); exponent mode: exponent bytes
  const uint2* meta;       // palette mode: per brick {raw map, raw groups before}
  const uint8_t* side;     // palette mode: raw groups' exponent bytes
  uint64_t side_bytes;     // size of side (at least 64)
  uint32_t lut[4];         // palette mode: entry i = rotr8(palette[i], 1) at byte i%4 of lut[i/4]
  int64_t rows, cols;
  bool exp_mode;           // codes are exponent bytes (pipeline 2)
  bool codes_ilv;          // codes are in the interleaved scratch order (pipelines 2, 3; see recon.h)
  uint64_t codes_bytes;    // size of the codes buffer
  uint32_t max_row_raw;    // palette mode: most raw groups in one brick-row (all ones: unknown)
};

// Fused-kernel variants.  Small-batch kernels (tokens <= 64): one workgroup per
// 16 rows, `waves` waves splitting the K loop, optional split of K across
// `ksplit` workgroups (atomic accumulation into a zeroed Y).  Large-batch
// kernels (tokens > 64): see fused_large.hip.
struct Variant {
  int kind;    // 0 = small batch, 1 = large batch, 2 = gemv (x in LDS), 3 = mid (K slices of x in LDS),
               // 4 = rowk (whole K per workgroup, x slices streamed through LDS)
  int waves;   // small/gemv/mid: waves per workgroup; rowk: waves per brick-row
  int ksplit;  // small: workgroups along K; rowk: bricks per wave per slice
  int unroll;  // small: bricks in flight per wave; gemv/mid/rowk: ring depth
  int tile;    // large: tile shape id; rowk: brick-rows per workgroup
};
int variant_count(int64_t tokens);
bool variant_get(int64_t tokens, int id, Variant* v);  // id 0 = default for (tokens, shape)
Variant variant_default(int64_t tokens, int64_t rows, int64_t cols);
// The default gemv variant (the one the default picks where gemv applies).
Variant variant_gemv();
// The variant that actually launches for v (a choice that does not apply to
// the shape or form falls back to the default of its family).
Variant variant_effective(int64_t tokens, int64_t rows, int64_t cols, bool exp_mode, const Variant& v);
// Activations kept in LDS by the gemv variants: tokens x cols <= kGemvXElems
// bf16 and at most kGemvKbnMax 64-column bricks per row.
constexpr int64_t kGemvXElems = 16384;
// Whether a rowk variant's LDS fits for this shape (else it cannot launch).
bool rowk_fits(int64_t tokens, int64_t rows, int64_t cols, const Variant& v);
constexpr int64_t kGemvKbnMax = 1024;
// Longest K (in 64-column bricks) of the wide large-batch tile (tile 22),
// whose LDS holds its 8 brick-rows' tables.
constexpr int64_t kWideKbnMax = 256;
// LDS budget of the mid kernels (a K slice of the activations plus the
// per-brick tables, or the epilogue's partial sums): two workgroups per CU.
constexpr size_t kMidLdsBytes = 81920;
// Bricks per K slice of the mid kernels for `tokens` tokens and `waves`
// brick-rows per workgroup, and its LDS bytes.
int mid_slice_kb(int64_t tokens, int64_t rows, int64_t cols, int waves);
size_t mid_lds_bytes(int64_t tokens, int waves, int slice_kb);
const char* variant_name(int64_t tokens, int id);
// Name of a variant (its list entry, else a description of its fields).
void variant_describe(int64_t tokens, const Variant& v, char* buf, size_t len);

hipError_t launch_fused(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                        hipStream_t s);

// One gemv launch over n <= kFusedGroupMax matrices of one shape in the
// palette form or as 4-bit codes in scratch (pipelines 4 and 3), each with its
// own activations, outputs and 1..16 tokens that fit the gemv variants; v is
// a gemv variant (kind 2).
constexpr int kFusedGroupMax = 16;
struct FusedJob {
  const uint8_t* sm;
  const uint8_t* codes;
  const uint2* meta;
  const uint8_t* side;
  uint64_t side_bytes;
  uint64_t codes_bytes;
  uint32_t lut[4];
  const uint16_t* x;
  float* y;
  int32_t tokens;
  int32_t codes_ilv;  // codes in the interleaved scratch order
};
struct FusedGroup {
  FusedJob job[kFusedGroupMax];
};
hipError_t launch_fused_gemv_group(const FusedW* ws, const uint16_t* const* xs, float* const* ys,
                                   const int64_t* tokens, int n, const Variant& v, hipStream_t s);
// The same for the whole-K variants (kind 4, the R4 P4 U2 D2 and R4 P2 U2 D2
// shapes, 1..64 tokens), all n matrices with `tokens` tokens; the palette form
// or 4-bit codes in scratch.
hipError_t launch_fused_rowk_group(const FusedW* ws, const uint16_t* const* xs, float* const* ys, int n,
                                   int64_t tokens, const Variant& v, hipStream_t s);

// Huffman decode of every chunk (one lane per 256-symbol chunk).
enum DecodeEmit { EMIT_BF16 = 0, EMIT_EXP = 1, EMIT_NIBBLE = 2 };
struct HuffDev {
  const uint32_t* words;
  const uint32_t* offsets;
  const uint32_t* lut;      // 4096 entries: up to 3 symbols | count << 24 | bits << 26
  const uint32_t* lut_codes;  // EMIT_NIBBLE: up to five 4-bit palette codes (bits 0-19) instead of symbols
  const uint8_t* sm;        // EMIT_BF16
  const uint2* meta;        // EMIT_NIBBLE: per-brick raw map
  uint64_t total_bits;      // payload bits of the stream (words holds 8 zero words more)
  int64_t rows, cols;
};
hipError_t launch_huff_decode(const HuffDev& h, DecodeEmit emit, void* out, hipStream_t s);

// Palette form -> bf16 W row-major (decode without a Huffman stream).  beside:
// the decode runs on a side stream next to other kernels (a kernel that holds
// no LDS, so that theirs find room).
hipError_t launch_palette_decode(const FusedW& w, uint16_t* out, hipStream_t s, bool beside = false);

hipError_t launch_silu_mul(const float* g, const float* u, uint16_t* h, int64_t n, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s);
hipError_t launch_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_read(const void* src, void* sink, size_t bytes, hipStream_t s);

}  // namespace uw
