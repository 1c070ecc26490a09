// Fused reconstruct-matmul for large batches (> 64 tokens) on gfx950.
//
// Unweight page, section 七 (reconstructing matmul) and section 十 (at large
// batch the cost is re-rebuilding the same weight tile for every token tile).
// Each weight brick is rebuilt once per workgroup, in registers, directly in
// the layout of the A operand of v_mfma_f32_16x16x32_bf16, and used for every
// token block of the workgroup; activations go through LDS once per workgroup
// and are read by all its waves.
//
// Tile: a wave owns RB bricks along the rows (16*RB rows) and 16*TBK tokens;
// WAVES waves stack along the rows.  Rows of the activation tile in LDS are
// padded by 16 bytes so that the 16 tokens of one B fragment spread over the
// banks.  Every global load is issued one K step ahead of its use -- weight
// bytes, raw side-table bytes (addresses from the per-brick table, read one
// step earlier still) and the next activation tile -- so the matrix work of
// step k overlaps the memory traffic of step k+1.
#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

constexpr int kXStride = 72;  // bf16 elements per activation row in LDS (64 + 8 pad)

template <int RB, bool EXPM>
struct WRegs {
  u32x4 s[RB];
  u32x4 e[RB];   // exponent bytes (exponent mode) or raw side-table bytes
  u32x2 n[RB];
  uint32_t anyraw[RB];
  bool raw[RB];
};

template <int WAVES, int RB, int TBK, bool EXPM>
__global__ __launch_bounds__(WAVES * 64) void fused_large_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    int ksplit, int n_tblk, int n_rblk) {
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

  // workgroup -> (token block, K slice, row block).  Workgroup g runs on XCD
  // g % 8, and each XCD has its own L2: give every XCD whole row blocks and let
  // the consecutive workgroups of an XCD take the token blocks of one row block,
  // so the compressed weight tile fetched from HBM by the first of them is read
  // from that XCD's L2 by the others (instead of once per token block from HBM).
  const int g = blockIdx.x;
  const int per_rb = n_tblk * ksplit;
  int tblk, ks, rblk;
  if ((n_rblk & 7) == 0) {
    const int slot = g >> 3, within = slot % per_rb;
    rblk = (slot / per_rb) * 8 + (g & 7);
    tblk = within % n_tblk;
    ks = within / n_tblk;
  } else {
    tblk = g % n_tblk;
    ks = (g / n_tblk) % ksplit;
    rblk = g / per_rb;
  }
  const int lo = (int)(((int64_t)ks * kbn) / ksplit);
  const int hi = (int)(((int64_t)(ks + 1) * kbn) / ksplit);
  const int tok0 = tblk * TOK;
  const int brow0 = (rblk * WAVES + wave) * RB;    // first brick-row of this wave
  const uint32_t lut[4] = {in_vgpr(lut0), in_vgpr(lut1), in_vgpr(lut2), in_vgpr(lut3)};
  const uint32_t nweights = (uint32_t)rows * (uint32_t)cols;
  const rsrc_t rs_sm = make_rsrc(sm, nweights);
  const rsrc_t rs_codes = make_rsrc(codes, EXPM ? nweights : nweights / 2);
  const rsrc_t rs_side = make_rsrc(side, side_bytes);
  const rsrc_t rs_x = make_rsrc(x, (uint64_t)tokens * cols * 2);
  const uint32_t lane16 = lane * 16, lane8 = lane * 8;
  // activation pieces this thread stages: token row and byte offset inside a K step
  uint32_t xoff[XPER];
  bool xlive[XPER];
#pragma unroll
  for (int j = 0; j < XPER; ++j) {
    const int c = threadIdx.x + j * WAVES * 64;
    const int t = c >> 3, piece = c & 7;
    xlive[j] = tok0 + t < tokens;
    xoff[j] = ((uint32_t)(tok0 + t) * cols) * 2 + piece * 16;
  }

  f32x4 acc[RB][TBK];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int t = 0; t < TBK; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_x = [&](int kb, u32x4 (&xr)[XPER]) {
#pragma unroll
    for (int j = 0; j < XPER; ++j) {
      xr[j] = u32x4{0u, 0u, 0u, 0u};
      if (xlive[j]) xr[j] = ld16(rs_x, xoff[j], kb * 128);
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
  uint2 mnext[RB];  // per-brick table of the step fetched next
  auto load_meta = [&](int kb) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
      mnext[i] = (!EXPM && kb < hi && brow0 + i < brows) ? meta[(size_t)(brow0 + i) * kbn + kb] : uint2{0u, 0u};
  };
  auto load_w = [&](WRegs<RB, EXPM>& wr, int kb) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      wr.anyraw[i] = 0u;
      if (brow0 + i < brows) {
        const uint32_t b = (uint32_t)(brow0 + i) * kbn + kb;
        wr.s[i] = ld16(rs_sm, lane16, b * 1024);
        if (EXPM) {
          wr.e[i] = ld16(rs_codes, lane16, b * 1024);
        } else {
          wr.n[i] = ld8(rs_codes, lane8, b * 512);
          const uint32_t map = mnext[i].x;
          wr.anyraw[i] = map;
          wr.raw[i] = (map >> r) & 1u;
          if (map && wr.raw[i]) {
            const uint32_t rank = __builtin_popcount(map & ((1u << r) - 1u));
            wr.e[i] = ld16(rs_side, (mnext[i].y + rank) * 64 + q * 16, 0);
          }
        }
      }
    }
  };
  // One K step: rebuild the A fragments from the weight bytes loaded during the
  // previous step, refill the same registers with the next step's bytes (one
  // register stage keeps the wave under 256 registers, so two waves share a
  // SIMD and cover each other's load latency), then multiply.
  WRegs<RB, EXPM> w;
  auto step = [&](int kb) {
    const int cur = (kb - lo) & 1;
    const bool more = kb + 1 < hi;
    // (rows past the end rebuild whatever the registers hold: their results are
    // never stored)
    bf16x8 a[RB][2];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      u32x4 a0, a1;
      if (EXPM) {
        rebuild_exp2(w.s[i], w.e[i], a0, a1);
      } else {
        uint32_t v[4];
        palette_v(w.n[i], lut, v);
        if (w.anyraw[i]) {
          if (w.raw[i]) {
            v[0] = rot_exp(w.e[i].x);
            v[1] = rot_exp(w.e[i].y);
            v[2] = rot_exp(w.e[i].z);
            v[3] = rot_exp(w.e[i].w);
          }
        }
        rebuild_v2(w.s[i], v, a0, a1);
      }
      a[i][0] = as_bf16x8(a0);
      a[i][1] = as_bf16x8(a1);
    }
    u32x4 xr[XPER];
    if (more) {
      load_x(kb + 1, xr);
      load_w(w, kb + 1);
      load_meta(kb + 2);
    }
    // B fragments come from LDS one token block ahead of the MFMAs using them.
    // The k-half is the outer loop: the two MFMAs that update one accumulator
    // are RB*TBK instructions apart, enough independent work to keep the
    // 16x16x32 pipeline full (dependent pairs closer than ~16 apart stall it).
    const uint16_t* xb = &xs[cur][r * kXStride + q * 16];
    u32x4 bf[2];
    bf[0] = *(const u32x4*)xb;
#pragma unroll
    for (int j = 0; j < 2 * TBK; ++j) {
      const int h = j / TBK, t = j % TBK;
      if (j + 1 < 2 * TBK) {
        const int h1 = (j + 1) / TBK, t1 = (j + 1) % TBK;
        bf[(j + 1) & 1] = *(const u32x4*)(xb + t1 * 16 * kXStride + h1 * 8);
      }
      const bf16x8 bv = as_bf16x8(bf[j & 1]);
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][h], bv, acc[i][t], 0, 0, 0);
      // fence: fragment reads stay one block ahead instead of being hoisted
      // (hoisting them all would cost 64 registers and halve the occupancy)
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) store_x(cur ^ 1, xr);
    __syncthreads();
  };

  {
    u32x4 xr[XPER];
    load_x(lo, xr);
    load_meta(lo);
    load_w(w, lo);
    load_meta(lo + 1);
    store_x(0, xr);
  }
  __syncthreads();
  for (int kb = lo; kb < hi; ++kb) step(kb);

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
                       w.meta, w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens,
                       (int)w.rows, (int)w.cols, ksplit, n_tblk, n_rblk);
  else
    hipLaunchKernelGGL((fused_large_kernel<WAVES, RB, TBK, false>), grid, dim3(WAVES * 64), 0, s, w.sm, w.codes,
                       w.meta, w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens,
                       (int)w.rows, (int)w.cols, ksplit, n_tblk, n_rblk);
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
