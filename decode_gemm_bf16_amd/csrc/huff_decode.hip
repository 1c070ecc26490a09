// Chunk-parallel canonical-Huffman decoder of the exponent stream (gfx950).
//
// Unweight page, section 六: the first three pipelines run a Huffman
// preprocessing step before the matmul -- a full rebuild of the BF16 weights
// (pipeline 1), the exponent bytes only (pipeline 2, half the write traffic)
// or a transcode to 4-bit palette codes (pipeline 3, a quarter).
//
// A lane decodes two chunks of 256 symbols each, from their bit offsets, in
// lockstep (two independent dependency chains per lane).  The 12-bit code limit makes one 4096-entry table (symbol | length
// << 8) in LDS decode any code with a single lookup on the top 12 bits of a
// 64-bit bit buffer.  The 256 chunks of a workgroup are consecutive in the
// stream, so their bits are first copied into LDS with coalesced 16-byte
// loads; the bit buffer then refills from LDS, never waiting on HBM inside the
// symbol loop.  (A workgroup whose span does not fit, which needs more than
// 4 bits per exponent on average, reads its words from global memory.)
//
// A chunk is a quarter brick: 16 runs of 16 symbols, run i = row i of the
// brick, 16 consecutive columns.  All lanes of a wave finish a run in the same
// step, so a run is emitted by the whole wave at once; for the bf16 output
// consecutive lanes write consecutive 32-byte pieces of one output row.
#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

constexpr int kChunksPerBlock = 256;
constexpr int kThreads = 128;      // two chunks per lane
constexpr int kStageWords = 7680;  // 30 KB of staged bitstream: 4 workgroups fit one CU's LDS

// Bit reader over one chunk: a 64-bit buffer with `nbits` valid bits at the
// top, the next stream word already fetched, and the index of the one after.
struct Reader {
  uint64_t buf;
  int nbits;
  uint32_t next;
  uint32_t wi;
};

template <class Src>
__device__ __forceinline__ Reader reader_at(Src src, uint32_t base, uint32_t start) {
  Reader rd;
  uint32_t wi = (start >> 5) - base;
  rd.buf = (((uint64_t)src(wi) << 32) | src(wi + 1)) << (start & 31);
  rd.nbits = 64 - (int)(start & 31);  // >= 33
  rd.next = src(wi + 2);
  rd.wi = wi + 3;
  return rd;
}

// Decode one symbol: a single lookup on the top 12 bits.
__device__ __forceinline__ uint32_t take(Reader& rd, const uint16_t* lut) {
  const uint32_t ent = lut[(uint32_t)(rd.buf >> 52)];
  const int len = (int)(ent >> 8);
  rd.buf <<= len;
  rd.nbits -= len;
  return ent & 0xFFu;
}

// After two symbols (at most 24 bits) keep at least 32 valid bits.
template <class Src>
__device__ __forceinline__ void refill(Reader& rd, Src src) {
  if (rd.nbits < 32) {
    rd.buf |= (uint64_t)rd.next << (32 - rd.nbits);
    rd.nbits += 32;
    rd.next = src(rd.wi++);
  }
}

template <int EMIT>
__device__ __forceinline__ void emit_run(const uint32_t ew[4], int64_t c, int run, const uint8_t* code_of,
                                         const uint8_t* __restrict__ sm, uint32_t rawmap, void* __restrict__ out,
                                         int cols) {
  const int64_t serial = c * 256 + run * 16;
  if (EMIT == EMIT_EXP) {
    *(u32x4*)((uint8_t*)out + serial) = u32x4{ew[0], ew[1], ew[2], ew[3]};
  } else if (EMIT == EMIT_NIBBLE) {
    uint32_t nw0 = 0u, nw1 = 0u;
    if (!((rawmap >> run) & 1u)) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t code = code_of[(ew[j >> 2] >> (8 * (j & 3))) & 0xFFu];
        const int jj = j & 7;
        const int shift = 8 * (jj & 3) + 4 * (jj >> 2);
        if (j < 8) nw0 |= code << shift; else nw1 |= code << shift;
      }
    }
    *(u32x2*)((uint8_t*)out + serial / 2) = u32x2{nw0, nw1};
  } else {
    const u32x4 s = *(const u32x4*)(sm + serial);
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
// one chain's LDS latency hides behind the other's.
template <int EMIT, class Src>
__device__ __forceinline__ void decode_two(Src src, uint32_t base, int64_t ca, int64_t cb, bool has_b,
                                           const uint32_t* __restrict__ offsets, const uint16_t* lut,
                                           const uint8_t* code_of, const uint8_t* __restrict__ sm,
                                           const uint2* __restrict__ meta, void* __restrict__ out, int cols) {
  Reader ra = reader_at(src, base, offsets[ca]);
  Reader rb = has_b ? reader_at(src, base, offsets[cb]) : ra;
  const uint32_t rawa = EMIT == EMIT_NIBBLE ? meta[ca >> 2].x : 0u;
  const uint32_t rawb = (EMIT == EMIT_NIBBLE && has_b) ? meta[cb >> 2].x : 0u;
  for (int run = 0; run < 16; ++run) {
    uint32_t ea[4] = {0u, 0u, 0u, 0u}, eb[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      ea[j >> 2] |= take(ra, lut) << (8 * (j & 3));
      eb[j >> 2] |= take(rb, lut) << (8 * (j & 3));
      if (j & 1) {
        refill(ra, src);
        refill(rb, src);
      }
    }
    emit_run<EMIT>(ea, ca, run, code_of, sm, rawa, out, cols);
    if (has_b) emit_run<EMIT>(eb, cb, run, code_of, sm, rawb, out, cols);
  }
}

template <int EMIT>
__global__ __launch_bounds__(kThreads) void huff_decode_kernel(
    const uint32_t* __restrict__ words, uint64_t total_bits, const uint32_t* __restrict__ offsets,
    const uint16_t* __restrict__ lut_g, const uint8_t* __restrict__ sm, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ code_of_g, void* __restrict__ out, int64_t nchunks, int cols) {
  __shared__ uint16_t lut[4096];
  __shared__ uint8_t code_of[256];
  __shared__ uint32_t stage[kStageWords];
  {
    const u32x4* src = (const u32x4*)lut_g;
    u32x4* dst = (u32x4*)lut;
    for (int i = threadIdx.x; i < 4096 * 2 / 16; i += kThreads) dst[i] = src[i];
    if (EMIT == EMIT_NIBBLE)
      for (int i = threadIdx.x; i < 256; i += kThreads) code_of[i] = code_of_g[i];
  }
  const int64_t c0 = (int64_t)blockIdx.x * kChunksPerBlock;
  const int64_t c_end = c0 + kChunksPerBlock < nchunks ? c0 + kChunksPerBlock : nchunks;
  // words that the chunks c0 .. c_end-1 read: from the first chunk's start to
  // 3 words past the last chunk's end (the bit buffer's look-ahead)
  const uint32_t w0 = offsets[c0] >> 5;
  const uint64_t end_bit = c_end < nchunks ? (uint64_t)offsets[c_end] : total_bits;
  const uint32_t w1 = (uint32_t)(end_bit >> 5) + 4;
  const bool staged = w1 - w0 <= (uint32_t)kStageWords;
  if (staged) {
    // 16-byte aligned copy of words [w0 & ~3, w1), clipped to the stage
    const uint32_t a0 = w0 & ~3u;
    const uint32_t nvec = (w1 - a0 + 3) / 4;
    for (uint32_t i = threadIdx.x; i < nvec; i += kThreads) {
      const uint32_t wv = a0 + 4 * i;
      const u32x4 v = *(const u32x4*)(words + wv);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int32_t d = (int32_t)(wv + k) - (int32_t)w0;
        if (d >= 0 && d < kStageWords) stage[d] = v[k];
      }
    }
  }
  __syncthreads();
  const int64_t ca = c0 + threadIdx.x, cb = ca + kThreads;
  if (ca >= nchunks) return;
  const bool has_b = cb < nchunks;
  if (staged) {
    auto src = [&](uint32_t i) { return stage[i]; };
    decode_two<EMIT>(src, w0, ca, cb, has_b, offsets, lut, code_of, sm, meta, out, cols);
  } else {
    auto src = [&](uint32_t i) { return words[i]; };
    decode_two<EMIT>(src, 0u, ca, cb, has_b, offsets, lut, code_of, sm, meta, out, cols);
  }
}

}  // namespace

hipError_t launch_huff_decode(const HuffDev& h, DecodeEmit emit, void* out, hipStream_t s) {
  const int64_t nchunks = h.rows * h.cols / 256;
  const dim3 grid((unsigned)((nchunks + kChunksPerBlock - 1) / kChunksPerBlock));
#define UW_LAUNCH(E)                                                                                          \
  hipLaunchKernelGGL(huff_decode_kernel<E>, grid, dim3(kThreads), 0, s, h.words, h.total_bits, h.offsets, h.lut, \
                     h.sm, h.meta, h.code_of, out, nchunks, (int)h.cols)
  switch (emit) {
    case EMIT_BF16: UW_LAUNCH(EMIT_BF16); break;
    case EMIT_EXP: UW_LAUNCH(EMIT_EXP); break;
    default: UW_LAUNCH(EMIT_NIBBLE);
  }
#undef UW_LAUNCH
  return hipGetLastError();
}

}  // namespace uw
