// Small element-wise kernels: SwiGLU glue, float->bf16, zero fill, a plain
// copy (the measured HBM ceiling) and the palette-form decode to bf16.
#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + (((u >> 16) & 1u) + 0x7FFFu)) >> 16);
}

// h = bf16(silu(g) * u): the SwiGLU product (Unweight page, section 十一 names
// SwiGLU models; gate, up and down are the three compressed projections).
__global__ void silu_mul_kernel(const float* __restrict__ g, const float* __restrict__ u, uint16_t* __restrict__ h,
                                int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    const f32x4 gv = *(const f32x4*)(g + i), uv = *(const f32x4*)(u + i);
    uint32_t o0 = f32_to_bf16_rne(gv.x / (1.f + __expf(-gv.x)) * uv.x) |
                  ((uint32_t)f32_to_bf16_rne(gv.y / (1.f + __expf(-gv.y)) * uv.y) << 16);
    uint32_t o1 = f32_to_bf16_rne(gv.z / (1.f + __expf(-gv.z)) * uv.z) |
                  ((uint32_t)f32_to_bf16_rne(gv.w / (1.f + __expf(-gv.w)) * uv.w) << 16);
    *(u32x2*)(h + i) = u32x2{o0, o1};
  } else {
    for (int64_t k = i; k < n; ++k) h[k] = f32_to_bf16_rne(g[k] / (1.f + __expf(-g[k])) * u[k]);
  }
}

__global__ void f32_to_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = f32_to_bf16_rne(in[i]);
}

__global__ void zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    *(f32x4*)(p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    for (int64_t k = i; k < n; ++k) p[k] = 0.f;
  }
}

// Each thread keeps four independent 16-byte loads in flight.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  if (base + 768 < n16) {
    const u32x4 a = src[base], b = src[base + 256], c = src[base + 512], d = src[base + 768];
    dst[base] = a;
    dst[base + 256] = b;
    dst[base + 512] = c;
    dst[base + 768] = d;
  } else {
    for (int64_t i = base; i < n16 && i < base + 1024; i += 256) dst[i] = src[i];
  }
}

// Read-only stream: four 16-byte loads in flight per thread, XOR-folded so
// the loads cannot be dropped; lanes whose fold is nonzero write it to sink
// (any of them: the value only keeps the loads alive).
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ sink,
                                                   int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (base + 768 < n16) {
    acc = src[base] ^ src[base + 256] ^ src[base + 512] ^ src[base + 768];
  } else {
    for (int64_t i = base; i < n16 && i < base + 1024; i += 256) acc ^= src[i];
  }
  if ((acc.x | acc.y | acc.z | acc.w) == 0x9E3779B9u) *sink = acc;
}

// Palette form -> row-major bf16, one wave per brick (lane = run).
__global__ __launch_bounds__(256) void palette_decode_kernel(const uint8_t* __restrict__ sm,
                                                             const uint8_t* __restrict__ nib,
                                                             const uint2* __restrict__ meta,
                                                             const uint8_t* __restrict__ side, uint32_t lut0,
                                                             uint32_t lut1, uint32_t lut2, uint32_t lut3,
                                                             uint16_t* __restrict__ out, int64_t bricks, int cols) {
  const int64_t b = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  if (b >= bricks) return;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const uint32_t lut[4] = {lut0, lut1, lut2, lut3};
  // the compressed streams are read once: non-temporal loads; the bf16 output
  // is read next by the GEMM, so its stores keep the default policy
  const uint64_t nw = (uint64_t)bricks * 1024;
  const u32x4 s = ld16s(make_rsrc(sm, nw), lane * 16, (uint32_t)b * 1024);
  const u32x2 n = ld8s(make_rsrc(nib, nw / 2), lane * 8, (uint32_t)b * 512);
  const uint2 m = meta[b];
  uint32_t p[8];
  rebuild_palette(s, n, lut, p);
  if ((m.x >> r) & 1u) {
    const uint32_t rank = __builtin_popcount(m.x & ((1u << r) - 1u));
    const u32x4 ev = *(const u32x4*)(side + ((size_t)m.y + rank) * 64 + q * 16);
    rebuild_exp(s, ev, p);
  }
  // The brick's 16 rows x 128 bytes go through this wave's LDS (rows padded
  // to 144 bytes) so that each store instruction writes 8 whole 128-byte row
  // segments: lane l stores row 8 i + l / 8, bytes 16 (l % 8) .. + 15.
  __shared__ __attribute__((aligned(16))) uint8_t tp[4][16 * 144];
  uint8_t* t = tp[threadIdx.x >> 6];
  *(u32x4*)(t + r * 144 + q * 32) = u32x4{p[0], p[1], p[2], p[3]};
  *(u32x4*)(t + r * 144 + q * 32 + 16) = u32x4{p[4], p[5], p[6], p[7]};
  __builtin_amdgcn_wave_barrier();
  // (brick indices fit 32 bits: a matrix holds fewer than 2^31 weights)
  const uint32_t kbn = (uint32_t)cols >> 6, bu = (uint32_t)b;
  const uint32_t brow = bu / kbn, kb = bu - brow * kbn;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = 8 * i + (lane >> 3);
    const u32x4 v = *(const u32x4*)(t + rr * 144 + (lane & 7) * 16);
    *(u32x4*)(out + ((int64_t)brow * 16 + rr) * cols + kb * 64 + (lane & 7) * 8) = v;
  }
}

// The same without LDS, each lane storing its own 32 bytes: for decodes on a
// side stream beside the library GEMM, whose large tiles need a CU's LDS (a
// decode workgroup holding 9 KB of LDS keeps a GEMM workgroup off its CU:
// the 70B-shaped stack at 1024 tokens with the decodes overlapped ran 119.5
// ms with the transposing kernel, 114.2 with this one).
__global__ __launch_bounds__(256) void palette_decode_direct_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ nib, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint32_t lut0, uint32_t lut1, uint32_t lut2, uint32_t lut3,
    uint16_t* __restrict__ out, int64_t bricks, int cols) {
  const int64_t b = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  if (b >= bricks) return;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const uint32_t lut[4] = {lut0, lut1, lut2, lut3};
  // the compressed streams are read once: non-temporal loads; the bf16 output
  // is read next by the GEMM, so its stores keep the default policy
  const uint64_t nw = (uint64_t)bricks * 1024;
  const u32x4 s = ld16s(make_rsrc(sm, nw), lane * 16, (uint32_t)b * 1024);
  const u32x2 n = ld8s(make_rsrc(nib, nw / 2), lane * 8, (uint32_t)b * 512);
  const uint2 m = meta[b];
  uint32_t p[8];
  rebuild_palette(s, n, lut, p);
  if ((m.x >> r) & 1u) {
    const uint32_t rank = __builtin_popcount(m.x & ((1u << r) - 1u));
    const u32x4 ev = *(const u32x4*)(side + ((size_t)m.y + rank) * 64 + q * 16);
    rebuild_exp(s, ev, p);
  }
  const int kbn = cols >> 6;
  const int64_t row = (b / kbn) * 16 + r;
  uint16_t* o = out + row * cols + (b % kbn) * 64 + q * 16;
  *(u32x4*)o = u32x4{p[0], p[1], p[2], p[3]};
  *(u32x4*)(o + 8) = u32x4{p[4], p[5], p[6], p[7]};
}

}  // namespace

hipError_t launch_silu_mul(const float* g, const float* u, uint16_t* h, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, g, u, h, n);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = (n16 + 1023) / 1024;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

hipError_t launch_read(const void* src, void* sink, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = (n16 + 1023) / 1024;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)src, (u32x4*)sink, n16);
  return hipGetLastError();
}

hipError_t launch_palette_decode(const FusedW& w, uint16_t* out, hipStream_t s, bool beside) {
  const int64_t bricks = w.rows * w.cols / 1024;
  const dim3 grid((unsigned)((bricks + 3) / 4)), block(256);
  if (beside)
    hipLaunchKernelGGL(palette_decode_direct_kernel, grid, block, 0, s, w.sm, w.codes, w.meta, w.side, w.lut[0],
                       w.lut[1], w.lut[2], w.lut[3], out, bricks, (int)w.cols);
  else
    hipLaunchKernelGGL(palette_decode_kernel, grid, block, 0, s, w.sm, w.codes, w.meta, w.side, w.lut[0], w.lut[1],
                       w.lut[2], w.lut[3], out, bricks, (int)w.cols);
  return hipGetLastError();
}

}  // namespace uw
