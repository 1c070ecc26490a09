// Chunk-parallel canonical-Huffman decoder of the exponent stream (gfx950).
//
// Unweight page, section 六: the first three pipelines run a Huffman
// preprocessing step before the matmul -- a full rebuild of the BF16 weights
// (pipeline 1), the exponent bytes only (pipeline 2, half the write traffic)
// or a transcode to 4-bit palette codes (pipeline 3, a quarter).
//
// One lane decodes one chunk of 256 symbols, starting at the chunk's bit
// offset.  The 12-bit code limit makes one 4096-entry table (symbol | length
// << 8) in LDS decode any code with a single lookup on the top 12 bits of a
// 64-bit bit buffer.  A chunk is a quarter brick: 16 runs of 16 symbols, run i
// = row i of the brick, 16 consecutive columns.  All lanes of a wave finish a
// run in the same step (16 symbols each), so a run is emitted by the whole
// wave at once; for the bf16 output consecutive lanes write consecutive 32-byte
// pieces of the same output row.
#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

constexpr int kThreads = 256;

template <int EMIT>
__global__ __launch_bounds__(kThreads) void huff_decode_kernel(
    const uint32_t* __restrict__ words, const uint32_t* __restrict__ offsets, const uint16_t* __restrict__ lut_g,
    const uint8_t* __restrict__ sm, const uint2* __restrict__ meta, const uint8_t* __restrict__ code_of_g,
    void* __restrict__ out, int64_t nchunks, int cols) {
  __shared__ uint16_t lut[4096];
  __shared__ uint8_t code_of[256];
  {
    const u32x4* src = (const u32x4*)lut_g;
    u32x4* dst = (u32x4*)lut;
    for (int i = threadIdx.x; i < 4096 * 2 / 16; i += kThreads) dst[i] = src[i];
    if (EMIT == EMIT_NIBBLE) code_of[threadIdx.x] = code_of_g[threadIdx.x];
  }
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= nchunks) return;

  const uint32_t start = offsets[c];
  uint32_t wi = start >> 5;
  uint64_t buf = ((uint64_t)words[wi] << 32) | words[wi + 1];
  buf <<= (start & 31);
  int nbits = 64 - (int)(start & 31);  // valid bits at the top of buf (>= 33)
  uint32_t next = words[wi + 2];
  wi += 3;

  const int64_t brick = c >> 2;
  const int quarter = (int)(c & 3);
  const int kbn = cols >> 6;
  uint32_t rawmap = 0;
  if (EMIT == EMIT_NIBBLE) rawmap = meta[brick].x;

  for (int run = 0; run < 16; ++run) {
    uint32_t ew[4] = {0u, 0u, 0u, 0u};  // 16 symbols, byte j%4 of word j/4
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t ent = lut[(uint32_t)(buf >> 52)];
      const int len = (int)(ent >> 8);
      buf <<= len;
      nbits -= len;
      ew[j >> 2] |= (ent & 0xFFu) << (8 * (j & 3));
      if (j & 1) {  // two codes take at most 24 bits; keep at least 32 valid
        if (nbits < 32) {
          buf |= (uint64_t)next << (32 - nbits);
          nbits += 32;
          next = words[wi++];
        }
      }
    }
    const int64_t serial = c * 256 + run * 16;
    if (EMIT == EMIT_EXP) {
      u32x4 v = {ew[0], ew[1], ew[2], ew[3]};
      *(u32x4*)((uint8_t*)out + serial) = v;
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
      u32x2 v = {nw0, nw1};
      *(u32x2*)((uint8_t*)out + serial / 2) = v;
    } else {
      const u32x4 s = *(const u32x4*)(sm + serial);
      uint32_t p[8];
      u32x4 ev = {ew[0], ew[1], ew[2], ew[3]};
      rebuild_exp(s, ev, p);
      const int64_t tb = brick / kbn, kb = brick % kbn;
      const int64_t row = tb * 16 + run;
      uint16_t* o = (uint16_t*)out + row * cols + kb * 64 + quarter * 16;
      u32x4 v0 = {p[0], p[1], p[2], p[3]}, v1 = {p[4], p[5], p[6], p[7]};
      *(u32x4*)o = v0;
      *(u32x4*)(o + 8) = v1;
    }
  }
}

}  // namespace

hipError_t launch_huff_decode(const HuffDev& h, DecodeEmit emit, void* out, hipStream_t s) {
  const int64_t nchunks = h.rows * h.cols / 256;
  const dim3 grid((unsigned)((nchunks + kThreads - 1) / kThreads));
  switch (emit) {
    case EMIT_BF16:
      hipLaunchKernelGGL(huff_decode_kernel<EMIT_BF16>, grid, dim3(kThreads), 0, s, h.words, h.offsets, h.lut, h.sm,
                         h.meta, h.code_of, out, nchunks, (int)h.cols);
      break;
    case EMIT_EXP:
      hipLaunchKernelGGL(huff_decode_kernel<EMIT_EXP>, grid, dim3(kThreads), 0, s, h.words, h.offsets, h.lut, h.sm,
                         h.meta, h.code_of, out, nchunks, (int)h.cols);
      break;
    default:
      hipLaunchKernelGGL(huff_decode_kernel<EMIT_NIBBLE>, grid, dim3(kThreads), 0, s, h.words, h.offsets, h.lut,
                         h.sm, h.meta, h.code_of, out, nchunks, (int)h.cols);
  }
  return hipGetLastError();
}

}  // namespace uw
