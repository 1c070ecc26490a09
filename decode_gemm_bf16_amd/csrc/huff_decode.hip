// Chunk-parallel canonical-Huffman decoder of the exponent stream (gfx950).
//
// Unweight page, section 六: the first three pipelines run a Huffman
// preprocessing step before the matmul -- a full rebuild of the BF16 weights
// (pipeline 1), the exponent bytes only (pipeline 2, half the write traffic)
// or a transcode to 4-bit palette codes (pipeline 3, a quarter).
//
// A lane decodes two chunks of 256 symbols, from their bit offsets, in
// lockstep (two independent dependency chains per lane); a workgroup of four
// waves takes 512 consecutive chunks.  The code-length limit of 12 bits lets
// one 4096-entry table in LDS decode, from the 12 bits at a chain's position,
// every whole code those bits start with: up to three exponent symbols
// (pipelines 1, 2; about 2.9 a lookup on exponent statistics) or up to five
// 4-bit palette codes (pipeline 3; about 4.2).  Each chain keeps the two
// stream words around its position in registers and requests the next word
// one step ahead, so a lookup waits for one LDS round trip; a word moves in
// after every second lookup (two lookups take at most 24 bits).  All steps
// are branch-free, so a wave whose lanes are at different points of their
// runs runs one instruction stream.
//
// Decoded symbols go to a small per-chunk slot in LDS: exponent symbols as
// bytes (three byte stores a lookup: an unaligned dword store stalls the
// LDS), palette codes through a 64-bit register queue whose low dword is
// stored, aligned, after every lookup.  A run (16 symbols) is emitted once
// both chains of every lane of the wave hold one; a chain may run up to half
// a run ahead (palette codes: a whole run, which spares the wave 7% of its
// lookup steps -- it waits less often for its slowest chain).  The table and
// the workgroup's bits are first moved into LDS by buffer loads straight to
// LDS (a workgroup whose span does not fit, which needs more than 2.8 bits
// per exponent on average -- 3.1 for pipeline 3 -- reads its words from
// global memory).  The grid gives every workgroup the
// same number of chunks (at most 512), chosen so that the workgroups fill
// whole rounds of two per CU: on the 14336 x 4096 gate 512 workgroups of 448
// chunks instead of 448 of 512, which left a quarter of the CUs with one
// workgroup and the rest with two.
//
// A chunk is a quarter brick: 16 runs of 16 symbols, run i = row i of the
// brick, 16 consecutive columns.  Pipelines 2 and 3 write run r of chunk c at
// slot ((c / 512) * 16 + r) * 512 + c % 512: the workgroup's 512 chunks store
// one run as one contiguous block, and the blocks of successive runs follow
// each other.  Pipeline 1 writes bf16 W row-major.
#include <algorithm>

#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

constexpr int kThreads = 256;                   // four waves, two chunks per lane
constexpr int kChunksPerBlock = 2 * kThreads;   // the interleave group of the scratch order
constexpr int kStreamPad = 8;                   // zero words after the stream (the encoder's padding)
constexpr int kSymSlot = 36;                    // bytes per chunk (9 dwords: the lanes' slots start in distinct banks)
constexpr uint32_t kSymLead = 24;               // a pair of lookups is taken while a slot holds fewer symbols
constexpr int kCodeSlot = 6;                    // dwords per chunk for palette codes
constexpr uint32_t kCodeLead = 4;               // a pair is taken while fewer dwords are full

// Staged bitstream, in words: LDS per workgroup = 16 KB table + stage + slots,
// two workgroups per CU.
template <int EMIT>
constexpr int stage_words() {
  return EMIT == EMIT_NIBBLE ? 13056 : 11520;
}

// Exponent bytes and palette codes are written once and read by a later
// GEMM: non-temporal stores keep them from evicting lines that are still
// read here (11-13% faster on the gate, and the fused GEMM after it does not
// slow down).  The bf16 output of pipeline 1 keeps plain stores: the library
// GEMM reading it slows down by more than the decode gains.
__device__ __forceinline__ void st8(rsrc_t r, u32x2 v, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, (int)soff, kAuxStream);
}
__device__ __forceinline__ void st16(rsrc_t r, u32x4 v, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, kAuxStream);
}

// A chain's place in the stream: the words holding bits [32*wb, 32*wb + 64),
// the position kept as r = 50 - (offset in them) so that one 64-bit right
// shift puts the 12-bit window, times 4 (a table byte offset), at bits 2-13,
// and the next word, requested ahead.  r >= 7 at a lookup (offset <= 43),
// r >= -5 after the second of a pair.
struct BitBuf {
  uint32_t b0, b1, nw, wb;
  int32_t r;
};

template <class Src>
__device__ __forceinline__ void bits_init(Src src, uint32_t pos, BitBuf& bb) {
  bb.wb = pos >> 5;
  bb.r = 50 - (int32_t)(pos & 31);
  bb.b0 = src(bb.wb);
  bb.b1 = src(bb.wb + 1);
  bb.nw = src(bb.wb + 2);
}

__device__ __forceinline__ uint32_t table_entry(const BitBuf& bb, const uint8_t* lut) {
  const uint64_t two = ((uint64_t)bb.b0 << 32) | bb.b1;
  return *(const uint32_t*)(lut + ((uint32_t)(two >> bb.r) & 0x3FFCu));
}

// After a pair of lookups: move on by a word if the position left b0, and
// request the word after the new b1.
template <class Src>
__device__ __forceinline__ void refill(Src src, BitBuf& bb) {
  const bool adv = bb.r <= 18;
  bb.b0 = adv ? bb.b1 : bb.b0;
  bb.b1 = adv ? bb.nw : bb.b1;
  bb.r += adv ? 32 : 0;
  bb.wb += adv ? 1u : 0u;
  bb.nw = src(bb.wb + 2);
}

// Exponent symbols: an entry holds up to three symbols (bits 0-23), their
// count (24-25) and the bits they take (26-29); they are appended to the slot
// at p (an entry not taken appends nothing and leaves the position).
__device__ __forceinline__ void lookup_sym(BitBuf& bb, uint32_t& p, bool take, uint8_t* slot, const uint8_t* lut) {
  uint32_t ent = table_entry(bb, lut);
  ent = take ? ent : 0u;
  bb.r -= (int32_t)(ent >> 26);
  slot[p] = (uint8_t)ent;
  slot[p + 1] = (uint8_t)(ent >> 8);
  slot[p + 2] = (uint8_t)(ent >> 16);
  p += (ent >> 24) & 3u;
}

// The run's 16 symbols; the ones decoded past it move to the slot's start.
__device__ __forceinline__ u32x4 take_sym_run(uint8_t* slot, uint32_t& p) {
  uint32_t* w = (uint32_t*)slot;
  const u32x4 e = {w[0], w[1], w[2], w[3]};
  const uint32_t r0 = w[4], r1 = w[5], r2 = w[6], r3 = w[7];
  w[0] = r0;
  w[1] = r1;
  w[2] = r2;
  w[3] = r3;
  p -= 16;
  return e;
}

// Palette codes: an entry holds up to five codes (bits 0-19), the bits they
// take (20-23) and four times their count (the top byte, which an add reads
// through a byte select: no separate extract).  The codes not yet
// completing a dword wait in q (qs bits of it); a lookup shifts its codes by
// qs as one 64-bit value, stores q with their low part at byte kb of the slot,
// and when the dword is full moves on to the next one, keeping the high part.
struct CodeQ {
  uint32_t q, qs, kb;
};

__device__ __forceinline__ void lookup_code(BitBuf& bb, CodeQ& cq, bool take, uint8_t* slot, const uint8_t* lut) {
  uint32_t ent = table_entry(bb, lut);
  ent = take ? ent : 0u;
  bb.r -= (int32_t)((ent >> 20) & 15u);
  const uint64_t c = (uint64_t)(ent & 0xFFFFFu) << cq.qs;
  const uint32_t lo = cq.q | (uint32_t)c;
  *(uint32_t*)(slot + cq.kb) = lo;
  const uint32_t sum = cq.qs + (ent >> 24);
  const bool mv = sum >= 32u;
  cq.q = mv ? (uint32_t)(c >> 32) : lo;
  cq.qs = sum & 31u;
  cq.kb += mv ? 4u : 0u;
}

// Pipeline 2 and 3 store offset of chunk c's run 0 (bytes; run r adds
// r * 512 * S), S bytes per run.
__device__ __forceinline__ uint32_t ilv_lane(int64_t c, uint32_t S) {
  return (uint32_t)(((c >> 9) * (16 * kChunksPerBlock) + (c & (kChunksPerBlock - 1))) * S);
}

template <int EMIT, class Src>
__device__ __forceinline__ void decode_sym(Src src, uint32_t base, int64_t ca, int64_t cb, bool has_b,
                                           const uint32_t* __restrict__ offsets, const uint8_t* lut,
                                           uint8_t* slot_a, uint8_t* slot_b, const uint8_t* __restrict__ sm,
                                           void* __restrict__ out, uint64_t out_bytes, int cols) {
  BitBuf ba, bb;
  bits_init(src, offsets[ca] - base * 32, ba);
  bits_init(src, has_b ? offsets[cb] - base * 32 : offsets[ca] - base * 32, bb);
  uint32_t na = 0, nb = 0;
  const rsrc_t rs_out = make_rsrc(out, out_bytes);
  const uint32_t va = ilv_lane(ca, 16), vb = ilv_lane(cb, 16);
  // bf16 output: a chunk's 256 sign+mantissa bytes (two whole cache lines)
  // are requested before its first lookup and held in registers (P1 on the
  // 14336 x 4096 gate 58 -> 46 us against 16 bytes a run requested one to
  // four runs ahead, where 64 lanes touch 64 lines per instruction, each line
  // sixteen times over the decode).
  u32x4 la[16], lb[16];
  if (EMIT == EMIT_BF16) {
    const uint8_t* pb = sm + (has_b ? cb : ca) * 256;
#pragma unroll
    for (int d = 0; d < 16; ++d) la[d] = *(const u32x4*)(sm + ca * 256 + d * 16);
#pragma unroll
    for (int d = 0; d < 16; ++d) lb[d] = *(const u32x4*)(pb + d * 16);
  }
#pragma unroll
  for (int run = 0; run < 16; ++run) {
    // every taken lookup yields a symbol, so 8 pairs complete any run
    for (int it = 0; it < 8; ++it) {
      const bool take_a = na < kSymLead, take_b = nb < kSymLead;
      lookup_sym(ba, na, take_a, slot_a, lut);
      lookup_sym(bb, nb, take_b, slot_b, lut);
      lookup_sym(ba, na, take_a, slot_a, lut);
      lookup_sym(bb, nb, take_b, slot_b, lut);
      refill(src, ba);
      refill(src, bb);
      if (!__any(na < 16u || nb < 16u)) break;
    }
    const u32x4 ea = take_sym_run(slot_a, na);
    const u32x4 eb = take_sym_run(slot_b, nb);
    if (EMIT == EMIT_EXP) {
      st16(rs_out, ea, va, (uint32_t)run * (16u * kChunksPerBlock));
      if (has_b) st16(rs_out, eb, vb, (uint32_t)run * (16u * kChunksPerBlock));
    } else {
      // bf16: lanes with consecutive chunks write consecutive 32-byte pieces
      // of one output row
      const int kbn = cols >> 6;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && !has_b) break;
        const int64_t c = h ? cb : ca;
        uint32_t p[8];
        rebuild_exp(h ? lb[run] : la[run], h ? eb : ea, p);
        const int64_t brick = c >> 2, tr = brick / kbn, kb = brick % kbn;
        uint16_t* o = (uint16_t*)out + (tr * 16 + run) * (int64_t)cols + kb * 64 + (c & 3) * 16;
        *(u32x4*)o = u32x4{p[0], p[1], p[2], p[3]};
        *(u32x4*)(o + 8) = u32x4{p[4], p[5], p[6], p[7]};
      }
    }
  }
}

// a run's 16 codes (code i at bits 4i of d0:d1) in the stored form -- of 8
// codes, byte b = code b | code b+4 << 4 -- or zeros for a raw row
__device__ __forceinline__ u32x2 stored_codes(uint32_t d0, uint32_t d1, bool raw) {
  const uint32_t d[2] = {d0, d1};
  uint32_t nw[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t even = d[h] & 0x0F0F0F0Fu;        // codes 0,2,4,6
    const uint32_t odd = (d[h] >> 4) & 0x0F0F0F0Fu;  // codes 1,3,5,7
    const uint32_t first = __builtin_amdgcn_perm(odd, even, 0x05010400u);   // codes 0..3
    const uint32_t second = __builtin_amdgcn_perm(odd, even, 0x07030602u);  // codes 4..7
    nw[h] = raw ? 0u : (first | (second << 4));
  }
  return u32x2{nw[0], nw[1]};
}

template <class Src>
__device__ __forceinline__ void decode_codes(Src src, uint32_t base, int64_t ca, int64_t cb, bool has_b,
                                             const uint32_t* __restrict__ offsets, const uint8_t* lut,
                                             uint32_t* slot_a, uint32_t* slot_b, const uint2* __restrict__ meta,
                                             void* __restrict__ out, uint64_t out_bytes) {
  BitBuf ba, bb;
  bits_init(src, offsets[ca] - base * 32, ba);
  bits_init(src, has_b ? offsets[cb] - base * 32 : offsets[ca] - base * 32, bb);
  // raw rows of the brick: their codes are stored as zeros
  const uint32_t rawa = meta[ca >> 2].x;
  const uint32_t rawb = has_b ? meta[cb >> 2].x : 0u;
  CodeQ qa = {0u, 0u, 0u}, qb = {0u, 0u, 0u};
  const rsrc_t rs_out = make_rsrc(out, out_bytes);
  const uint32_t va = ilv_lane(ca, 8), vb = ilv_lane(cb, 8);
  uint8_t* sa = (uint8_t*)slot_a;
  uint8_t* sb = (uint8_t*)slot_b;
  for (int run = 0; run < 16; ++run) {
    for (int it = 0; it < 8; ++it) {
      const bool take_a = qa.kb < 4 * kCodeLead, take_b = qb.kb < 4 * kCodeLead;
      lookup_code(ba, qa, take_a, sa, lut);
      lookup_code(bb, qb, take_b, sb, lut);
      lookup_code(ba, qa, take_a, sa, lut);
      lookup_code(bb, qb, take_b, sb, lut);
      refill(src, ba);
      refill(src, bb);
      if (!__any(qa.kb < 8u || qb.kb < 8u)) break;
    }
    // (up to 5 full dwords: the run's 2 leave, the other 3 move down)
    const uint32_t a0 = slot_a[0], a1 = slot_a[1], a2 = slot_a[2], a3 = slot_a[3], a4 = slot_a[4];
    const uint32_t b0 = slot_b[0], b1 = slot_b[1], b2 = slot_b[2], b3 = slot_b[3], b4 = slot_b[4];
    slot_a[0] = a2;
    slot_a[1] = a3;
    slot_a[2] = a4;
    slot_b[0] = b2;
    slot_b[1] = b3;
    slot_b[2] = b4;
    qa.kb -= 8u;
    qb.kb -= 8u;
    st8(rs_out, stored_codes(a0, a1, (rawa >> run) & 1u), va, (uint32_t)run * (8u * kChunksPerBlock));
    if (has_b) st8(rs_out, stored_codes(b0, b1, (rawb >> run) & 1u), vb, (uint32_t)run * (8u * kChunksPerBlock));
  }
}

// 16 bytes per lane from a buffer straight into LDS: a wave's 64 lanes fill
// the 1 KB at `lds` (wave-uniform) in lane order.
__device__ __forceinline__ void dma16(rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, 0, 0, 0);
}

template <int EMIT>
__global__ __launch_bounds__(kThreads) void huff_decode_kernel(
    const uint32_t* __restrict__ words, uint64_t total_bits, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ lut_g, const uint8_t* __restrict__ sm, const uint2* __restrict__ meta,
    void* __restrict__ out, uint64_t out_bytes, int64_t nchunks, int cols, int cpw) {
  constexpr int kStage = stage_words<EMIT>();
  constexpr int kSlotBytes = EMIT == EMIT_NIBBLE ? kCodeSlot * 4 : kSymSlot;
  static_assert(kStage % 256 == 0, "the stage takes whole 1 KB copy blocks");
  __shared__ __attribute__((aligned(1024))) uint32_t lut[4096];
  __shared__ __attribute__((aligned(1024))) uint32_t stage_buf[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t slots[kChunksPerBlock * kSlotBytes];
  // this workgroup's chunks: c0 .. c_end - 1, at most 2 * kThreads
  const int64_t c0 = (int64_t)blockIdx.x * cpw;
  const int64_t c_end = c0 + cpw < nchunks ? c0 + cpw : nchunks;
  // words read: from the first chunk's start to 5 words past the last
  // chunk's end (a chain keeps taking lookups while its slot has room: at
  // most 8 of at most 12 bits past its end; the bit buffer reads 2 words
  // past its position)
  const uint32_t w0 = offsets[c0] >> 5;
  const uint64_t end_bit = c_end < nchunks ? (uint64_t)offsets[c_end] : total_bits;
  const uint32_t w1 = (uint32_t)(end_bit >> 5) + 6;
  // The copy starts at the 16-byte aligned word a0 <= w0 and writes whole
  // 1 KB blocks (lanes past the span write zeros): those must fit the stage.
  const uint32_t a0 = w0 & ~3u;
  const bool staged = ((w1 - a0 + 255) & ~255u) <= (uint32_t)kStage;
  const uint32_t* stage = stage_buf + (w0 - a0);  // stage[i] = word w0 + i
  {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const rsrc_t rs_lut = make_rsrc(lut_g, 4096 * 4);
    const rsrc_t rs_words = make_rsrc(words, (((total_bits + 31) >> 5) + kStreamPad) * 4);
    for (int c = wave; c < 16; c += kThreads / 64) dma16(rs_lut, (uint8_t*)lut + c * 1024, (c * 64 + lane) * 16);
    const uint32_t nvec = staged ? (w1 - a0 + 3) / 4 : 0u;
    for (uint32_t c = wave; c * 64 < nvec; c += kThreads / 64) {
      const uint32_t i = c * 64 + lane;
      dma16(rs_words, (uint8_t*)stage_buf + c * 1024, i < nvec ? (a0 + 4 * i) * 4 : kOffRange);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  // chain a of lane t decodes chunk c0 + t, chain b chunk c0 + half + t
  const int half = (int)((c_end - c0 + 1) / 2);
  if ((int)threadIdx.x >= half) return;
  const int64_t ca = c0 + threadIdx.x, cb = ca + half;
  const bool has_b = cb < c_end;
  const uint8_t* lutb = (const uint8_t*)lut;
  if constexpr (EMIT == EMIT_NIBBLE) {
    uint32_t* slot_a = (uint32_t*)slots + threadIdx.x * kCodeSlot;
    uint32_t* slot_b = (uint32_t*)slots + (threadIdx.x + kThreads) * kCodeSlot;
    if (staged) {
      auto src = [&](uint32_t i) { return stage[i]; };
      decode_codes(src, w0, ca, cb, has_b, offsets, lutb, slot_a, slot_b, meta, out, out_bytes);
    } else {
      auto src = [&](uint32_t i) { return words[i]; };
      decode_codes(src, 0u, ca, cb, has_b, offsets, lutb, slot_a, slot_b, meta, out, out_bytes);
    }
  } else {
    uint8_t* slot_a = slots + threadIdx.x * kSymSlot;
    uint8_t* slot_b = slots + (threadIdx.x + kThreads) * kSymSlot;
    if (staged) {
      auto src = [&](uint32_t i) { return stage[i]; };
      decode_sym<EMIT>(src, w0, ca, cb, has_b, offsets, lutb, slot_a, slot_b, sm, out, out_bytes, cols);
    } else {
      auto src = [&](uint32_t i) { return words[i]; };
      decode_sym<EMIT>(src, 0u, ca, cb, has_b, offsets, lutb, slot_a, slot_b, sm, out, out_bytes, cols);
    }
  }
}

// Compute units of the current device (256 on MI355X), read once per device.
int device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

hipError_t launch_huff_decode(const HuffDev& h, DecodeEmit emit, void* out, hipStream_t s) {
  const int64_t nchunks = h.rows * h.cols / 256;
  if (nchunks <= 0) return hipSuccess;
  // pipelines 2 and 3: the interleaved order pads to whole groups of 512 chunks
  const uint64_t groups = (uint64_t)(nchunks + kChunksPerBlock - 1) / kChunksPerBlock;
  const uint64_t out_bytes = emit == EMIT_EXP      ? groups * kChunksPerBlock * 256
                             : emit == EMIT_NIBBLE ? groups * kChunksPerBlock * 128
                                                   : (uint64_t)nchunks * 512;
  // buffer stores take 32-bit offsets within a 2 GB range
  if (emit != EMIT_BF16 && out_bytes > 0x7FFFFFF0ull) return hipErrorInvalidValue;
  // Chunks per workgroup: the fewest (a multiple of 64, at most 512) that
  // fill whole rounds of two workgroups per CU (their LDS allows two).
  const int64_t slots = 2 * (int64_t)device_cus();
  const int64_t rounds = (nchunks + slots * kChunksPerBlock - 1) / (slots * kChunksPerBlock);
  int64_t cpw = (nchunks + slots * rounds - 1) / (slots * rounds);
  cpw = std::min<int64_t>(kChunksPerBlock, ((cpw + 63) / 64) * 64);
  const dim3 grid((unsigned)((nchunks + cpw - 1) / cpw));
#define UW_LAUNCH(E)                                                                                           \
  hipLaunchKernelGGL(huff_decode_kernel<E>, grid, dim3(kThreads), 0, s, h.words, h.total_bits, h.offsets,          \
                     E == EMIT_NIBBLE ? h.lut_codes : h.lut, h.sm, h.meta, out, out_bytes, nchunks, (int)h.cols,   \
                     (int)cpw)
  switch (emit) {
    case EMIT_BF16: UW_LAUNCH(EMIT_BF16); break;
    case EMIT_EXP: UW_LAUNCH(EMIT_EXP); break;
    default: UW_LAUNCH(EMIT_NIBBLE);
  }
#undef UW_LAUNCH
  return hipGetLastError();
}

}  // namespace uw
