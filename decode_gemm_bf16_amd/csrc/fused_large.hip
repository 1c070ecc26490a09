// Fused reconstruct-matmul for large batches (> 64 tokens) on gfx950.
//
// Unweight page, section 七 (reconstructing matmul) and section 十 (at large
// batch the cost is re-rebuilding the same weight tile for every token tile).
// Each weight brick is rebuilt once per workgroup, in registers, directly in
// the layout of the A operand of v_mfma_f32_16x16x32_bf16, and then used for
// every token block of the workgroup; activations go through LDS once per
// workgroup and are read by all its waves.
//
// Tile: a wave owns RB bricks along the rows (16*RB rows) and 16*TBK tokens;
// WAVES waves stack along the rows.  Rows of the activation tile in LDS are
// padded by 16 bytes so that the 16 tokens of one B fragment spread over the
// banks.  Global loads of the next K step (weights and activations) are issued
// before the matrix work of the current step.
#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

constexpr int kXStride = 72;  // bf16 elements per activation row in LDS (64 + 8 pad)

template <int WAVES, int RB, int TBK, bool EXPM>
__global__ __launch_bounds__(WAVES * 64) void fused_large_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint32_t lut0, uint32_t lut1, uint32_t lut2, uint32_t lut3,
    const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols, int ksplit,
    int n_tblk) {
  constexpr int TOK = 16 * TBK;                    // tokens per workgroup
  constexpr int XCHUNKS = TOK * 8;                 // 16-byte pieces of one activation tile
  constexpr int XPER = XCHUNKS / (WAVES * 64);     // pieces per thread
  static_assert(XCHUNKS % (WAVES * 64) == 0, "activation tile split");
  __shared__ uint16_t xs[2][TOK * kXStride];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int kbn = cols >> 6;
  const int brows = rows >> 4;

  // workgroup -> (token block, row block, K slice); neighbouring workgroups land
  // on different XCDs and take different token blocks of the same rows.
  const int g = blockIdx.x;
  const int tblk = g % n_tblk;
  const int rest = g / n_tblk;
  const int ks = rest % ksplit;
  const int rblk = rest / ksplit;
  const int lo = (int)(((int64_t)ks * kbn) / ksplit);
  const int hi = (int)(((int64_t)(ks + 1) * kbn) / ksplit);
  const int tok0 = tblk * TOK;
  const int brow0 = (rblk * WAVES + wave) * RB;    // first brick-row of this wave
  const uint32_t lut[4] = {lut0, lut1, lut2, lut3};

  f32x4 acc[RB][TBK];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int t = 0; t < TBK; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_x = [&](int kb, u32x4 (&xr)[XPER]) {
#pragma unroll
    for (int j = 0; j < XPER; ++j) {
      const int c = threadIdx.x + j * WAVES * 64;
      const int t = c >> 3, piece = c & 7;
      const int tok = tok0 + t;
      xr[j] = u32x4{0u, 0u, 0u, 0u};
      if (tok < tokens) xr[j] = *(const u32x4*)(x + (size_t)tok * cols + kb * 64 + piece * 8);
    }
  };
  auto store_x = [&](int buf, const u32x4 (&xr)[XPER]) {
#pragma unroll
    for (int j = 0; j < XPER; ++j) {
      const int c = threadIdx.x + j * WAVES * 64;
      const int t = c >> 3, piece = c & 7;
      *(u32x4*)(&xs[buf][t * kXStride + piece * 8]) = xr[j];
    }
  };

  u32x4 ws[RB], we[RB];
  u32x2 wn[RB];
  uint2 wm[RB];
  auto load_w = [&](int kb) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (brow0 + i < brows) {
        const size_t b = (size_t)(brow0 + i) * kbn + kb;
        ws[i] = *(const u32x4*)(sm + b * 1024 + lane * 16);
        if (EXPM) {
          we[i] = *(const u32x4*)(codes + b * 1024 + lane * 16);
        } else {
          wn[i] = *(const u32x2*)(codes + b * 512 + lane * 8);
          wm[i] = meta[b];
        }
      }
    }
  };

  {
    u32x4 xr[XPER];
    load_x(lo, xr);
    store_x(0, xr);
  }
  if (lo < hi) load_w(lo);
  __syncthreads();

  for (int kb = lo; kb < hi; ++kb) {
    const int cur = (kb - lo) & 1;
    // rebuild this step's A fragments from the registers loaded last step
    bf16x8 a[RB][2];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      uint32_t p[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      if (brow0 + i < brows) {
        if (EXPM) {
          rebuild_exp(ws[i], we[i], p);
        } else {
          rebuild_palette(ws[i], wn[i], lut, p);
          const uint32_t map = wm[i].x;
          if (map) {
            if ((map >> r) & 1u) {
              const uint32_t rank = __builtin_popcount(map & ((1u << r) - 1u));
              const u32x4 ev = *(const u32x4*)(side + ((size_t)wm[i].y + rank) * 64 + q * 16);
              rebuild_exp(ws[i], ev, p);
            }
          }
        }
      }
      a[i][0] = as_bf16x8(p[0], p[1], p[2], p[3]);
      a[i][1] = as_bf16x8(p[4], p[5], p[6], p[7]);
    }
    // issue next step's global loads
    u32x4 xr[XPER];
    const bool more = kb + 1 < hi;
    if (more) {
      load_x(kb + 1, xr);
      load_w(kb + 1);
    }
    // matrix work on the current activation tile
    const uint16_t* xb = &xs[cur][0];
#pragma unroll
    for (int t = 0; t < TBK; ++t) {
      const uint16_t* xp = xb + (t * 16 + r) * kXStride + q * 16;
      const bf16x8 b0 = as_bf16x8(*(const u32x4*)xp);
      const bf16x8 b1 = as_bf16x8(*(const u32x4*)(xp + 8));
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][0], b0, acc[i][t], 0, 0, 0);
        acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][1], b1, acc[i][t], 0, 0, 0);
      }
    }
    if (more) store_x(cur ^ 1, xr);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(l/16)+0..3 of each brick-row, token l%16
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    if (brow0 + i >= brows) continue;
#pragma unroll
    for (int t = 0; t < TBK; ++t) {
      const int tok = tok0 + t * 16 + r;
      if (tok >= tokens) continue;
      float* yp = y + (size_t)tok * rows + (size_t)(brow0 + i) * 16 + 4 * q;
      if (ksplit == 1) {
        *(f32x4*)yp = acc[i][t];
      } else {
        atomicAdd(yp + 0, acc[i][t].x);
        atomicAdd(yp + 1, acc[i][t].y);
        atomicAdd(yp + 2, acc[i][t].z);
        atomicAdd(yp + 3, acc[i][t].w);
      }
    }
  }
}

template <int WAVES, int RB, int TBK>
hipError_t launch_large_t(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int ksplit, hipStream_t s) {
  const int n_tblk = (int)((tokens + 16 * TBK - 1) / (16 * TBK));
  const int brows = (int)(w.rows / 16);
  const int n_rblk = (brows + WAVES * RB - 1) / (WAVES * RB);
  const dim3 grid((unsigned)(n_tblk * ksplit * n_rblk));
  if (w.exp_mode)
    hipLaunchKernelGGL((fused_large_kernel<WAVES, RB, TBK, true>), grid, dim3(WAVES * 64), 0, s, w.sm, w.codes,
                       w.meta, w.side, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens, (int)w.rows,
                       (int)w.cols, ksplit, n_tblk);
  else
    hipLaunchKernelGGL((fused_large_kernel<WAVES, RB, TBK, false>), grid, dim3(WAVES * 64), 0, s, w.sm, w.codes,
                       w.meta, w.side, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens, (int)w.rows,
                       (int)w.cols, ksplit, n_tblk);
  return hipGetLastError();
}

}  // namespace

// tile ids: 0 = 4 waves x (64 rows x 128 tokens); 1 = 4 waves x (32 rows x 128 tokens);
//           2 = 2 waves x (64 rows x 128 tokens); 3 = 4 waves x (64 rows x 64 tokens)
hipError_t launch_fused_large(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                              hipStream_t s) {
  const int ks = v.ksplit < 1 ? 1 : v.ksplit;
  if (ks > 1) {
    hipError_t e = launch_zero(y, tokens * w.rows, s);
    if (e != hipSuccess) return e;
  }
  switch (v.tile) {
    case 0: return launch_large_t<4, 4, 8>(w, x, y, tokens, ks, s);
    case 1: return launch_large_t<4, 2, 8>(w, x, y, tokens, ks, s);
    case 2: return launch_large_t<2, 4, 8>(w, x, y, tokens, ks, s);
    case 3: return launch_large_t<4, 4, 4>(w, x, y, tokens, ks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uw
