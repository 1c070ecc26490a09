// Chunk-parallel canonical-Huffman decoder of the exponent stream (gfx950).
//
// Unweight page, section 六: the first three pipelines run a Huffman
// preprocessing step before the matmul -- a full rebuild of the BF16 weights
// (pipeline 1), the exponent bytes only (pipeline 2, half the write traffic)
// or a transcode to 4-bit palette codes (pipeline 3, a quarter).
//
// A lane decodes two chunks of 256 symbols each, from their bit offsets, in
// lockstep (two independent dependency chains per lane).  Decoding is a chain
// of dependent table lookups -- the position of a code is known only once the
// previous one is decoded -- so its time is the chain's length times the LDS
// round trip.  The 12-bit code limit lets one 4096-entry table in LDS decode,
// from the 12 bits at the chain's bit position, every whole code those bits
// hold, up to three: with exponent codes of 2-3 bits on average a lookup
// yields about three symbols, a third of the chain.  A step reads the two
// stream words around the position (one LDS instruction) and shifts out a
// 32-bit window -- no bit buffer to refill -- and every step is branch-free,
// so a wave whose lanes are at different points of their runs runs one
// instruction stream.  Symbols gather in a 64-bit queue per chunk; a run (16
// symbols) is emitted once both chains of every lane of the wave hold one.
// Pipeline 3 uses a second table whose entries hold the symbols' 4-bit palette
// codes, so the transcode is a nibble shuffle per 8 codes.
// The 256 chunks of a workgroup are consecutive in the stream, so their bits
// are first copied into LDS with coalesced 16-byte loads.  (A workgroup whose
// span does not fit, which needs about 3 bits per exponent on average, reads
// its words from global memory.)
//
// A chunk is a quarter brick: 16 runs of 16 symbols, run i = row i of the
// brick, 16 consecutive columns.  All lanes of a wave emit a run in the same
// step; for the bf16 output consecutive lanes write consecutive 32-byte
// pieces of one output row.
#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

constexpr int kChunksPerBlock = 256;
constexpr int kThreads = 128;      // two chunks per lane
constexpr int kStreamPad = 8;      // zero words after the stream (the encoder's padding)
constexpr int kStageWords = 6016;  // 23.5 KB of staged bitstream: with the 16 KB table, 4 workgroups per CU

// The next 32 bits of the stream from bit `pos` (MSB first): two consecutive
// words and a 64-bit shift.
template <class Src>
__device__ __forceinline__ uint32_t window(Src src, uint32_t pos) {
  const uint32_t wi = pos >> 5;
  const uint64_t two = ((uint64_t)src(wi) << 32) | src(wi + 1);
  return (uint32_t)((two << (pos & 31)) >> 32);
}

// Symbols (or 4-bit codes) decoded but not yet placed in a run, first in the
// low bits.
struct Queue {
  uint64_t q;
  int n;
};

// One chain step, branch-free.  BITS = 8: the table yields exponent symbols;
// BITS = 4: it yields their palette codes (pipeline 3).  A lookup on the 12
// bits at `pos` appends its 1 to 3 entries to the queue when the queue holds
// less than a dword (else the entry is dropped and nothing moves); then a
// dword of queued entries moves into the run being built when the run is not
// complete -- the run's dwords shift down one place and the new one enters
// last, so they end in order.
template <int BITS, class Src>
__device__ __forceinline__ void step(Src src, uint32_t& pos, Queue& qu, uint32_t* e, int& k, const uint32_t* lut) {
  constexpr int PER = 32 / BITS;       // entries per dword
  constexpr int RD = 16 * BITS / 32;   // dwords per run
  constexpr uint32_t MASK = BITS == 8 ? 0xFFFFFFu : 0xFFFu;
  uint32_t ent = lut[window(src, pos) >> 20];
  ent = qu.n < PER ? ent : 0u;
  pos += ent >> 26;
  qu.q |= (uint64_t)(ent & MASK) << (BITS * qu.n);
  qu.n += (int)((ent >> 24) & 3u);
  const bool mv = qu.n >= PER && k < RD;
  if constexpr (RD == 4) {
    e[0] = mv ? e[1] : e[0];
    e[1] = mv ? e[2] : e[1];
    e[2] = mv ? e[3] : e[2];
    e[3] = mv ? (uint32_t)qu.q : e[3];
  } else {
    e[0] = mv ? e[1] : e[0];
    e[1] = mv ? (uint32_t)qu.q : e[1];
  }
  qu.q = mv ? qu.q >> 32 : qu.q;
  qu.n -= mv ? PER : 0;
  k += mv ? 1 : 0;
}

template <int EMIT>
__device__ __forceinline__ void emit_run(const uint32_t* ew, int64_t c, int run, const u32x4& s, uint32_t rawmap,
                                         void* __restrict__ out, int cols) {
  // exponent bytes and 4-bit codes go to the interleaved scratch order (runs
  // of 64 consecutive chunks side by side, see code_lane_off in recon.h): the
  // 64 lanes of a wave, 64 consecutive chunks, store one run as one
  // contiguous block instead of 64 pieces 256 bytes apart
  const int64_t ilv_run = ((c >> 6) * 16 + run) * 64 + (c & 63);
  if (EMIT == EMIT_EXP) {
    *(u32x4*)((uint8_t*)out + ilv_run * 16) = u32x4{ew[0], ew[1], ew[2], ew[3]};
  } else if (EMIT == EMIT_NIBBLE) {
    // ew[0..1]: the run's 16 codes in order, 8 per dword (code i at bits 4i);
    // stored form: of 8 codes, byte b = code b | code b+4 << 4
    uint32_t nw[2] = {0u, 0u};
    if (!((rawmap >> run) & 1u)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t even = ew[h] & 0x0F0F0F0Fu;         // codes 0,2,4,6
        const uint32_t odd = (ew[h] >> 4) & 0x0F0F0F0Fu;   // codes 1,3,5,7
        const uint32_t first = __builtin_amdgcn_perm(odd, even, 0x05010400u);   // codes 0..3
        const uint32_t second = __builtin_amdgcn_perm(odd, even, 0x07030602u);  // codes 4..7
        nw[h] = first | (second << 4);
      }
    }
    *(u32x2*)((uint8_t*)out + ilv_run * 8) = u32x2{nw[0], nw[1]};
  } else {
    uint32_t p[8];
    rebuild_exp(s, u32x4{ew[0], ew[1], ew[2], ew[3]}, p);
    const int kbn = cols >> 6;
    const int64_t brick = c >> 2, tb = brick / kbn, kb = brick % kbn;
    uint16_t* o = (uint16_t*)out + (tb * 16 + run) * (int64_t)cols + kb * 64 + (c & 3) * 16;
    *(u32x4*)o = u32x4{p[0], p[1], p[2], p[3]};
    *(u32x4*)(o + 8) = u32x4{p[4], p[5], p[6], p[7]};
  }
}

// Two chunks per lane, decoded in lockstep: their lookups are independent, so
// one chain's LDS latency hides behind the other's.  A run needs at most 16
// steps (each step's lookup yields at least one symbol), which bounds the
// loop; the wave leaves it as soon as every run of the wave is complete.
template <int EMIT, class Src>
__device__ __forceinline__ void decode_two(Src src, uint32_t base, int64_t ca, int64_t cb, bool has_b,
                                           const uint32_t* __restrict__ offsets, const uint32_t* lut,
                                           const uint8_t* __restrict__ sm,
                                           const uint2* __restrict__ meta, void* __restrict__ out, int cols) {
  uint32_t pa = offsets[ca] - base * 32;
  uint32_t pb = has_b ? offsets[cb] - base * 32 : pa;
  const uint32_t rawa = EMIT == EMIT_NIBBLE ? meta[ca >> 2].x : 0u;
  const uint32_t rawb = (EMIT == EMIT_NIBBLE && has_b) ? meta[cb >> 2].x : 0u;
  Queue qa = {0ull, 0}, qb = {0ull, 0};
  // bf16 output: the run's sign+mantissa bytes, requested one run ahead
  u32x4 sa = {0u, 0u, 0u, 0u}, sb = {0u, 0u, 0u, 0u}, na = sa, nb = sb;
  if (EMIT == EMIT_BF16) {
    na = *(const u32x4*)(sm + ca * 256);
    if (has_b) nb = *(const u32x4*)(sm + cb * 256);
  }
  for (int run = 0; run < 16; ++run) {
    if (EMIT == EMIT_BF16) {
      sa = na;
      sb = nb;
      if (run + 1 < 16) {
        na = *(const u32x4*)(sm + ca * 256 + (run + 1) * 16);
        if (has_b) nb = *(const u32x4*)(sm + cb * 256 + (run + 1) * 16);
      }
    }
    constexpr int BITS = EMIT == EMIT_NIBBLE ? 4 : 8, RD = 16 * BITS / 32;
    uint32_t ea[RD] = {}, eb[RD] = {};
    int ka = 0, kb = 0;
    for (int it = 0; it < 16; ++it) {
      step<BITS>(src, pa, qa, ea, ka, lut);
      step<BITS>(src, pb, qb, eb, kb, lut);
      if (!__any(ka < RD || kb < RD)) break;  // every run of the wave is complete
    }
    emit_run<EMIT>(ea, ca, run, sa, rawa, out, cols);
    if (has_b) emit_run<EMIT>(eb, cb, run, sb, rawb, out, cols);
  }
}

template <int EMIT>
__global__ __launch_bounds__(kThreads) void huff_decode_kernel(
    const uint32_t* __restrict__ words, uint64_t total_bits, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ lut_g, const uint8_t* __restrict__ sm, const uint2* __restrict__ meta,
    void* __restrict__ out, int64_t nchunks, int cols) {
  __shared__ uint32_t lut[4096];
  __shared__ uint32_t stage[kStageWords];
  const int64_t c0 = (int64_t)blockIdx.x * kChunksPerBlock;
  const int64_t c_end = c0 + kChunksPerBlock < nchunks ? c0 + kChunksPerBlock : nchunks;
  // words that the chunks c0 .. c_end-1 read: from the first chunk's start to
  // 3 words past the last chunk's end (the bit buffer's look-ahead)
  const uint32_t w0 = offsets[c0] >> 5;
  const uint64_t end_bit = c_end < nchunks ? (uint64_t)offsets[c_end] : total_bits;
  const uint32_t w1 = (uint32_t)(end_bit >> 5) + 4;
  const bool staged = w1 - w0 <= (uint32_t)kStageWords;
  {
    // The decode table and the 16-byte aligned span of words [w0 & ~3, w1)
    // go to LDS: every load is issued before the first store, so the copy
    // costs one memory latency, not one per iteration.
    constexpr int LV = 4096 * 4 / 16 / kThreads;             // table pieces per thread
    constexpr int SV = (kStageWords / 4 + 2 + kThreads - 1) / kThreads;  // stream pieces per thread
    const rsrc_t rs_lut = make_rsrc(lut_g, 4096 * 4);
    const rsrc_t rs_words = make_rsrc(words, (((total_bits + 31) >> 5) + kStreamPad) * 4);
    const uint32_t a0 = w0 & ~3u;
    const uint32_t nvec = staged ? (w1 - a0 + 3) / 4 : 0u;
    u32x4 lv[LV], sv[SV];
#pragma unroll
    for (int k = 0; k < LV; ++k) lv[k] = ld16(rs_lut, (threadIdx.x + k * kThreads) * 16, 0);
#pragma unroll
    for (int k = 0; k < SV; ++k) {
      const uint32_t i = threadIdx.x + k * kThreads;
      sv[k] = ld16(rs_words, i < nvec ? (a0 + 4 * i) * 4 : kOffRange, 0);
    }
#pragma unroll
    for (int k = 0; k < LV; ++k) ((u32x4*)lut)[threadIdx.x + k * kThreads] = lv[k];
#pragma unroll
    for (int k = 0; k < SV; ++k) {
      const uint32_t i = threadIdx.x + k * kThreads;
      if (i < nvec) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int32_t d = (int32_t)(a0 + 4 * i + kk) - (int32_t)w0;
          if (d >= 0 && d < kStageWords) stage[d] = sv[k][kk];
        }
      }
    }
  }
  __syncthreads();
  const int64_t ca = c0 + threadIdx.x, cb = ca + kThreads;
  if (ca >= nchunks) return;
  const bool has_b = cb < nchunks;
  if (staged) {
    auto src = [&](uint32_t i) { return stage[i]; };
    decode_two<EMIT>(src, w0, ca, cb, has_b, offsets, lut, sm, meta, out, cols);
  } else {
    auto src = [&](uint32_t i) { return words[i]; };
    decode_two<EMIT>(src, 0u, ca, cb, has_b, offsets, lut, sm, meta, out, cols);
  }
}

}  // namespace

hipError_t launch_huff_decode(const HuffDev& h, DecodeEmit emit, void* out, hipStream_t s) {
  const int64_t nchunks = h.rows * h.cols / 256;
  const dim3 grid((unsigned)((nchunks + kChunksPerBlock - 1) / kChunksPerBlock));
#define UW_LAUNCH(E)                                                                                          \
  hipLaunchKernelGGL(huff_decode_kernel<E>, grid, dim3(kThreads), 0, s, h.words, h.total_bits, h.offsets,          \
                     E == EMIT_NIBBLE ? h.lut_codes : h.lut, h.sm, h.meta, out, nchunks, (int)h.cols)
  switch (emit) {
    case EMIT_BF16: UW_LAUNCH(EMIT_BF16); break;
    case EMIT_EXP: UW_LAUNCH(EMIT_EXP); break;
    default: UW_LAUNCH(EMIT_NIBBLE);
  }
#undef UW_LAUNCH
  return hipGetLastError();
}

}  // namespace uw
