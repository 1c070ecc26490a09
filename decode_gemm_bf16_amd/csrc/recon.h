// Device helpers: rebuild packed bf16 pairs from the stored bytes.
//
// A BF16 word (Unweight page, section 三) is sign<<15 | exponent<<7 | mantissa.
// Its low byte is (exponent & 1)<<7 | mantissa and its high byte is
// sign<<7 | exponent>>1.  With V = the exponent rotated right by one bit
// (bit 7 = exponent & 1, bits 6..0 = exponent >> 1) and S = the stored
// sign+mantissa byte (bit 7 = sign, bits 6..0 = mantissa):
//     low  byte = (S & 0x7F) | (V & 0x80)
//     high byte = (S & 0x80) | (V & 0x7F)
// so four weights take two bit-selects on whole dwords and two byte permutes
// to become two dwords of bf16 pairs -- no per-weight shifts.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace uw {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  // byte i of the result = byte sel.byte[i] of the 8-byte value hi:lo
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// S: 4 sign+mantissa bytes, V: the 4 matching rotated exponents.
// Returns the bf16 pairs (w0,w1) and (w2,w3).
__device__ __forceinline__ void assemble_v(uint32_t S, uint32_t V, uint32_t& p01, uint32_t& p23) {
  const uint32_t L = (S & 0x7F7F7F7Fu) | (V & 0x80808080u);
  const uint32_t H = (S & 0x80808080u) | (V & 0x7F7F7F7Fu);
  p01 = perm(H, L, 0x05010400u);
  p23 = perm(H, L, 0x07030602u);
}

// Same, from 4 plain exponent bytes E.
__device__ __forceinline__ void assemble_e(uint32_t S, uint32_t E, uint32_t& p01, uint32_t& p23) {
  const uint32_t L = (S & 0x7F7F7F7Fu) | ((E << 7) & 0x80808080u);
  const uint32_t H = (S & 0x80808080u) | ((E >> 1) & 0x7F7F7F7Fu);
  p01 = perm(H, L, 0x05010400u);
  p23 = perm(H, L, 0x07030602u);
}

// Four exponent bytes rotated right by one bit each.
__device__ __forceinline__ uint32_t rot_exp(uint32_t E) {
  return ((E >> 1) & 0x7F7F7F7Fu) | ((E << 7) & 0x80808080u);
}

// 16-entry palette lookup of 8 codes packed in N (byte b: code b low nibble,
// code b+4 high nibble).  lut[q] holds entries 4q..4q+3.  Low three code bits
// index two 8-entry halves with one byte permute each; the fourth bit then
// picks, per byte, the half through a third permute.
__device__ __forceinline__ void palette_lookup(uint32_t N, const uint32_t lut[4], uint32_t& Va, uint32_t& Vb) {
  const uint32_t ia = N & 0x07070707u;
  const uint32_t ib = (N >> 4) & 0x07070707u;
  const uint32_t sa = ((N >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t sb = ((N >> 5) & 0x04040404u) | 0x03020100u;
  Va = perm(perm(lut[3], lut[2], ia), perm(lut[1], lut[0], ia), sa);
  Vb = perm(perm(lut[3], lut[2], ib), perm(lut[1], lut[0], ib), sb);
}

// Rotated exponents of one lane's 16 weights from its 8 code bytes.
__device__ __forceinline__ void palette_v(const u32x2& n, const uint32_t lut[4], uint32_t v[4]) {
  palette_lookup(n.x, lut, v[0], v[1]);
  palette_lookup(n.y, lut, v[2], v[3]);
}

__device__ __forceinline__ void rebuild_v(const u32x4& s, const uint32_t v[4], uint32_t p[8]) {
  assemble_v(s.x, v[0], p[0], p[1]);
  assemble_v(s.y, v[1], p[2], p[3]);
  assemble_v(s.z, v[2], p[4], p[5]);
  assemble_v(s.w, v[3], p[6], p[7]);
}

// One lane's 16 weights of a brick -> 8 dwords of bf16 pairs, weights in order.
__device__ __forceinline__ void rebuild_palette(const u32x4& s, const u32x2& n, const uint32_t lut[4],
                                                uint32_t p[8]) {
  uint32_t v[4];
  palette_v(n, lut, v);
  rebuild_v(s, v, p);
}

// Same, straight into the two MFMA operand vectors (weights 0-7 and 8-15).
__device__ __forceinline__ void rebuild_v2(const u32x4& s, const uint32_t v[4], u32x4& a0, u32x4& a1) {
  uint32_t p[8];
  assemble_v(s.x, v[0], p[0], p[1]);
  assemble_v(s.y, v[1], p[2], p[3]);
  assemble_v(s.z, v[2], p[4], p[5]);
  assemble_v(s.w, v[3], p[6], p[7]);
  a0 = u32x4{p[0], p[1], p[2], p[3]};
  a1 = u32x4{p[4], p[5], p[6], p[7]};
}

__device__ __forceinline__ void rebuild_exp2(const u32x4& s, const u32x4& e, u32x4& a0, u32x4& a1) {
  uint32_t p[8];
  assemble_e(s.x, e.x, p[0], p[1]);
  assemble_e(s.y, e.y, p[2], p[3]);
  assemble_e(s.z, e.z, p[4], p[5]);
  assemble_e(s.w, e.w, p[6], p[7]);
  a0 = u32x4{p[0], p[1], p[2], p[3]};
  a1 = u32x4{p[4], p[5], p[6], p[7]};
}

// A wave-uniform value copied into a vector register once, so that loops do not
// re-materialise it from a scalar register at every use (v_perm_b32 takes at
// most one scalar operand).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t s) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(s));
  return v;
}

__device__ __forceinline__ void rebuild_exp(const u32x4& s, const u32x4& e, uint32_t p[8]) {
  assemble_e(s.x, e.x, p[0], p[1]);
  assemble_e(s.y, e.y, p[2], p[3]);
  assemble_e(s.z, e.z, p[4], p[5]);
  assemble_e(s.w, e.w, p[6], p[7]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Raw buffer access: a scalar resource (base, size) plus a per-lane 32-bit byte
// offset and a wave-uniform byte offset.  Loads cost no per-lane address
// arithmetic, and the per-lane part of an offset is computed once per kernel.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Where run r (row r of the brick) of quarter q of brick b sits in a stream of
// S bytes per run (exponent bytes: 16, 4-bit codes: 8).  Serial order: run
// 64b + 16q + r.  Interleaved order, the pipeline 2/3 scratch that the Huffman
// decoder writes: chunk c = 4b + q (a quarter brick), chunks grouped by 512
// (one decoder workgroup), run r of chunk c is run (c/512 * 16 + r) * 512 +
// c%512 -- so that the decoder's workgroup stores one run of all its chunks
// as one contiguous block.  The offset splits into a per-lane part and a
// wave-uniform per-brick part.
__device__ __forceinline__ uint32_t code_lane_off(int q, int r, uint32_t S, bool ilv) {
  return ilv ? (uint32_t)(r * 512 + q) * S : (uint32_t)(q * 16 + r) * S;
}
__device__ __forceinline__ uint32_t code_brick_off(uint32_t b, uint32_t S, bool ilv) {
  return ilv ? ((b >> 7) * 8192u + (b & 127u) * 4u) * S : b * 64u * S;
}

// A per-lane offset past every range make_rsrc sets: the buffer unit's range
// check turns such a load into zeros without a memory access.
constexpr uint32_t kOffRange = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ u32x2 ld8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

// Streaming loads of data read once per launch: the non-temporal cache
// policy (aux bit 1) marks the lines for early eviction, which measurably
// raises the read rate of a streaming kernel (stores take the same policy).
constexpr int kAuxStream = 2;
__device__ __forceinline__ u32x4 ld16s(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kAuxStream));
}
__device__ __forceinline__ u32x2 ld8s(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kAuxStream));
}

}  // namespace uw
