// Load-time transcode, Huffman form -> direct-palette form (Unweight page,
// section 六: direct palette reads weights transcoded to 4-bit codes at model
// load; section 四: a 64-weight row holding an exponent outside the top 16 is
// stored raw).  Three small kernels over the decoded exponents: raw rows per
// brick, a prefix count of raw groups, then the codes and the raw groups'
// exponents.  HBM-bound and run once per matrix.
#include "transcode.h"

namespace uw {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Byte offset of run r (row r of the brick's 16) of chunk c in the
// interleaved exponent order; chunk 4b+q is column block q of brick b.
__device__ __forceinline__ uint64_t run_off(uint64_t c, int r) {
  return (((c >> 9) * 16 + (uint64_t)r) * 512 + (c & 511)) * 16;
}

__device__ __forceinline__ bool any_outside(const u32x4& v, const int8_t* code_of) {
  bool out = false;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = v[k];
#pragma unroll
    for (int j = 0; j < 4; ++j) out |= code_of[(w >> (8 * j)) & 0xFF] < 0;
  }
  return out;
}

// A workgroup covers 16 bricks; thread = (brick, row).  Also counts the
// workgroup's raw groups for the scan.
__global__ __launch_bounds__(256) void raw_rows_kernel(const uint8_t* __restrict__ exps, uint64_t bricks,
                                                       CodeOfTable cof, uint32_t* __restrict__ rawmap,
                                                       uint32_t* __restrict__ wg_count) {
  __shared__ int8_t code_of[256];
  __shared__ uint32_t wave_count[4];
  code_of[threadIdx.x] = cof.c[threadIdx.x];
  __syncthreads();
  const uint64_t b = (uint64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int r = threadIdx.x & 15;
  bool raw = false;
  if (b < bricks) {
#pragma unroll
    for (int q = 0; q < 4; ++q) raw |= any_outside(*(const u32x4*)(exps + run_off(4 * b + q, r)), code_of);
  }
  // the wave's 64 lanes are 4 bricks x 16 rows
  const uint64_t m = __ballot(raw);
  if (r == 0 && b < bricks) rawmap[b] = (uint32_t)(m >> (threadIdx.x & 48)) & 0xFFFFu;
  if ((threadIdx.x & 63) == 0) wave_count[threadIdx.x >> 6] = (uint32_t)__popcll(m);
  __syncthreads();
  if (threadIdx.x == 0) wg_count[blockIdx.x] = wave_count[0] + wave_count[1] + wave_count[2] + wave_count[3];
}

// Exclusive prefix sum of the per-workgroup counts, 1024 at a time (one
// workgroup of 1024 threads, Hillis-Steele within a tile, a running carry
// across tiles).
__global__ __launch_bounds__(1024) void raw_scan_kernel(const uint32_t* __restrict__ count, uint64_t n,
                                                        uint32_t* __restrict__ before, uint32_t* __restrict__ total) {
  __shared__ uint32_t part[1024];
  uint32_t carry = 0;
  for (uint64_t base = 0; base < n; base += 1024) {
    const uint64_t i = base + threadIdx.x;
    const uint32_t v = i < n ? count[i] : 0u;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const uint32_t add = threadIdx.x >= (unsigned)d ? part[threadIdx.x - d] : 0u;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < n) before[i] = carry + part[threadIdx.x] - v;
    carry += part[1023];
    __syncthreads();  // the next tile overwrites part
  }
  if (threadIdx.x == 0) *total = carry;
}

// Same mapping as raw_rows_kernel.  Writes meta = {raw map, raw groups in
// earlier bricks}, the codes of run l = q*16 + r (byte u*4 + j holds weight
// 8u + j in its low nibble and weight 8u + j + 4 in its high one) and each
// raw row's 64 exponents.
__global__ __launch_bounds__(256) void palette_pack_kernel(const uint8_t* __restrict__ exps, uint64_t bricks,
                                                           CodeOfTable cof, const uint32_t* __restrict__ rawmap,
                                                           const uint32_t* __restrict__ wg_before,
                                                           uint2* __restrict__ meta, uint8_t* __restrict__ nib,
                                                           uint8_t* __restrict__ side) {
  __shared__ int8_t code_of[256];
  __shared__ uint32_t maps[16];
  code_of[threadIdx.x] = cof.c[threadIdx.x];
  const uint64_t b0 = (uint64_t)blockIdx.x * 16;
  if (threadIdx.x < 16) maps[threadIdx.x] = b0 + threadIdx.x < bricks ? rawmap[b0 + threadIdx.x] : 0u;
  __syncthreads();
  const int j = threadIdx.x >> 4, r = threadIdx.x & 15;
  const uint64_t b = b0 + j;
  if (b >= bricks) return;
  uint32_t before = wg_before[blockIdx.x];
  for (int k = 0; k < j; ++k) before += __builtin_popcount(maps[k]);
  const uint32_t map = maps[j];
  if (r == 0) meta[b] = uint2{map, before};
  const bool raw = (map >> r) & 1u;
  const uint32_t rank = __builtin_popcount(map & ((1u << r) - 1u));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = *(const u32x4*)(exps + run_off(4 * b + q, r));
    if (nib) {
      uint32_t out[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t lo = v[2 * u], hi = v[2 * u + 1];  // weights 8u..8u+3 and 8u+4..8u+7
        uint32_t o = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t cl = raw ? 0u : (uint32_t)code_of[(lo >> (8 * k)) & 0xFF] & 0xFu;
          const uint32_t ch = raw ? 0u : (uint32_t)code_of[(hi >> (8 * k)) & 0xFF] & 0xFu;
          o |= (cl | (ch << 4)) << (8 * k);
        }
        out[u] = o;
      }
      *(u32x2*)(nib + b * 512 + (uint64_t)(q * 16 + r) * 8) = u32x2{out[0], out[1]};
    }
    if (side && raw) *(u32x4*)(side + ((uint64_t)before + rank) * 64 + q * 16) = v;
  }
}

}  // namespace

hipError_t launch_raw_rows(const uint8_t* exps, uint64_t bricks, const CodeOfTable& code_of, uint32_t* rawmap,
                           uint32_t* wg_count, hipStream_t s) {
  if (bricks == 0) return hipSuccess;
  hipLaunchKernelGGL(raw_rows_kernel, dim3((unsigned)transcode_groups(bricks)), dim3(256), 0, s, exps, bricks, code_of,
                     rawmap, wg_count);
  return hipGetLastError();
}

hipError_t launch_raw_scan(const uint32_t* wg_count, uint64_t groups, uint32_t* wg_before, uint32_t* total,
                           hipStream_t s) {
  hipLaunchKernelGGL(raw_scan_kernel, dim3(1), dim3(1024), 0, s, wg_count, groups, wg_before, total);
  return hipGetLastError();
}

hipError_t launch_palette_pack(const uint8_t* exps, uint64_t bricks, const CodeOfTable& code_of,
                               const uint32_t* rawmap, const uint32_t* wg_before, uint2* meta, uint8_t* nib,
                               uint8_t* side, hipStream_t s) {
  if (bricks == 0) return hipSuccess;
  hipLaunchKernelGGL(palette_pack_kernel, dim3((unsigned)transcode_groups(bricks)), dim3(256), 0, s, exps, bricks,
                     code_of, rawmap, wg_before, meta, nib, side);
  return hipGetLastError();
}

}  // namespace uw
