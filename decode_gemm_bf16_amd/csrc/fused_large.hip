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
    int ksplit, int n_tblk, int n_rblk, uint64_t codes_bytes, int codes_ilv) {
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
  const rsrc_t rs_codes = make_rsrc(codes, codes_bytes);
  const rsrc_t rs_side = make_rsrc(side, side_bytes);
  const rsrc_t rs_x = make_rsrc(x, (uint64_t)tokens * cols * 2);
  const uint32_t lane16 = lane * 16;
  constexpr uint32_t CS = EXPM ? 16 : 8;  // code-stream bytes per run
  const uint32_t clane = code_lane_off(q, r, CS, codes_ilv);
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
          wr.e[i] = ld16(rs_codes, clane, code_brick_off(b, CS, codes_ilv));
        } else {
          wr.n[i] = ld8(rs_codes, clane, code_brick_off(b, CS, codes_ilv));
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
                       (int)w.rows, (int)w.cols, ksplit, n_tblk, n_rblk, w.codes_bytes, (int)w.codes_ilv);
  else
    hipLaunchKernelGGL((fused_large_kernel<WAVES, RB, TBK, false>), grid, dim3(WAVES * 64), 0, s, w.sm, w.codes,
                       w.meta, w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens,
                       (int)w.rows, (int)w.cols, ksplit, n_tblk, n_rblk, w.codes_bytes, (int)w.codes_ilv);
  return hipGetLastError();
}

// The same tile built on v_mfma_f32_32x32x16_bf16, twice the work of the 16x16x32
// form per instruction.  Its A operand is 32 rows x 16 k: lane l supplies row
// l%32 and k-slot l/32 (8 values).  A wave takes pairs of brick-rows (32 rows);
// lane l loads the whole 16-weight run of row l%16 of brick (l/16)%2 of the
// pair in quarter 2p + l/32 of the brick, so one load feeds two instructions:
// the run's first 8 weights go to the instruction of K pair p, half 0, the
// last 8 to half 1.  Each instruction's 16 k are then, for k-slot 0, columns
// 32p + 8h .. +7 and, for k-slot 1, columns 32p + 16 + 8h .. +7; the B operand
// (lane l: token l%32, k-slot l/32) reads exactly those columns from LDS.
// D layout: lane l, value v holds row 8*(v/4) + 4*(l/32) + v%4, token l%32.
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int RB2, bool EXPM>
struct WRegs32 {
  u32x4 s[RB2][2];
  u32x4 e[RB2][2];  // exponent bytes (exponent mode) or raw side-table bytes
  u32x2 n[RB2][2];
  uint32_t anyraw[RB2];
  bool raw[RB2];
};

template <int WAVES, int RB2, int TB2, bool EXPM>
__global__ __launch_bounds__(WAVES * 64) void fused_large32_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    int ksplit, int n_tblk, int n_rblk, uint64_t codes_bytes, int codes_ilv) {
  constexpr int TOK = 32 * TB2;                    // tokens per workgroup
  constexpr int XCHUNKS = TOK * 8;                 // 16-byte pieces of one activation tile
  constexpr int XPER = XCHUNKS / (WAVES * 64);     // pieces per thread
  static_assert(XCHUNKS % (WAVES * 64) == 0, "activation tile split");
  __shared__ uint16_t xs[2][TOK * kXStride];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;         // row inside the brick
  const int pb = (lane >> 4) & 1;  // which brick of the pair
  const int ks2 = lane >> 5;       // k-slot
  const int kbn = cols >> 6;
  const int brows = rows >> 4;

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
  const int brow0 = (rblk * WAVES + wave) * 2 * RB2;  // first brick-row of this wave
  const uint32_t lut[4] = {in_vgpr(lut0), in_vgpr(lut1), in_vgpr(lut2), in_vgpr(lut3)};
  const uint32_t nweights = (uint32_t)rows * (uint32_t)cols;
  const rsrc_t rs_sm = make_rsrc(sm, nweights);
  const rsrc_t rs_codes = make_rsrc(codes, codes_bytes);
  const rsrc_t rs_side = make_rsrc(side, side_bytes);
  const rsrc_t rs_x = make_rsrc(x, (uint64_t)tokens * cols * 2);
  // per-lane offsets of the lane's run inside brick-row brow0 + 2rb (rows past
  // the matrix read past the buffers' ends and get zeros)
  const uint32_t run = (uint32_t)(ks2 * 16 + r);  // run index inside the brick for K pair 0
  uint32_t voff_s[RB2], voff_n[RB2];
#pragma unroll
  for (int rb = 0; rb < RB2; ++rb) {
    const bool ok = brow0 + 2 * rb + pb < brows;
    voff_s[rb] = ok ? run * 16 + (uint32_t)pb * kbn * 1024 : kOffRange;
    voff_n[rb] = ok ? 0u : kOffRange;  // 0: the row exists; its code offset is computed per step
  }
  uint32_t xoff[XPER];
  bool xlive[XPER];
#pragma unroll
  for (int j = 0; j < XPER; ++j) {
    const int c = threadIdx.x + j * WAVES * 64;
    const int t = c >> 3, piece = c & 7;
    xlive[j] = tok0 + t < tokens;
    xoff[j] = ((uint32_t)(tok0 + t) * cols) * 2 + piece * 16;
  }

  f32x16 acc[RB2][TB2];
#pragma unroll
  for (int i = 0; i < RB2; ++i)
#pragma unroll
    for (int t = 0; t < TB2; ++t) acc[i][t] = f32x16{};

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
  // per-brick tables of the step fetched next: both bricks of each pair
  uint2 mnext[RB2][2];
  auto load_meta = [&](int kb) {
#pragma unroll
    for (int i = 0; i < RB2; ++i)
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
        const int br = brow0 + 2 * i + b2;
        mnext[i][b2] = (!EXPM && kb < hi && br < brows) ? meta[(size_t)br * kbn + kb] : uint2{0u, 0u};
      }
  };
  auto load_w = [&](WRegs32<RB2, EXPM>& wr, int kb) {
#pragma unroll
    for (int i = 0; i < RB2; ++i) {
      const uint32_t b = (uint32_t)(brow0 + 2 * i) * kbn + kb;  // first brick of the pair
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        wr.s[i][p] = ld16(rs_sm, voff_s[i], b * 1024 + p * 512);
        if (EXPM)
          wr.e[i][p] = ld16(rs_codes, voff_n[i] | (code_brick_off(b + (uint32_t)pb * kbn, 16, codes_ilv) +
                                                 code_lane_off(2 * p + ks2, r, 16, codes_ilv)), 0);
        else
          wr.n[i][p] = ld8(rs_codes, voff_n[i] | (code_brick_off(b + (uint32_t)pb * kbn, 8, codes_ilv) +
                                                code_lane_off(2 * p + ks2, r, 8, codes_ilv)), 0);
      }
      if (!EXPM) {
        const uint32_t mapa = mnext[i][0].x, mapb = mnext[i][1].x;
        const uint32_t map = pb ? mapb : mapa;
        const uint32_t before = pb ? mnext[i][1].y : mnext[i][0].y;
        wr.anyraw[i] = mapa | mapb;
        wr.raw[i] = (map >> r) & 1u;
        if ((mapa | mapb) && wr.raw[i]) {
          const uint32_t rank = __builtin_popcount(map & ((1u << r) - 1u));
          const uint32_t base = (before + rank) * 64 + ks2 * 16;
          wr.e[i][0] = ld16(rs_side, base, 0);
          wr.e[i][1] = ld16(rs_side, base + 32, 0);
        }
      }
    }
  };
  WRegs32<RB2, EXPM> w;
  auto step = [&](int kb) {
    const int cur = (kb - lo) & 1;
    const bool more = kb + 1 < hi;
    bf16x8 a[RB2][2][2];  // [row pair][K pair][half]
#pragma unroll
    for (int i = 0; i < RB2; ++i)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        u32x4 a0, a1;
        if (EXPM) {
          rebuild_exp2(w.s[i][p], w.e[i][p], a0, a1);
        } else {
          uint32_t v[4];
          palette_v(w.n[i][p], lut, v);
          if (w.anyraw[i]) {
            if (w.raw[i]) {
              v[0] = rot_exp(w.e[i][p].x);
              v[1] = rot_exp(w.e[i][p].y);
              v[2] = rot_exp(w.e[i][p].z);
              v[3] = rot_exp(w.e[i][p].w);
            }
          }
          rebuild_v2(w.s[i][p], v, a0, a1);
        }
        a[i][p][0] = as_bf16x8(a0);
        a[i][p][1] = as_bf16x8(a1);
      }
    u32x4 xr[XPER];
    if (more) {
      load_x(kb + 1, xr);
      load_w(w, kb + 1);
      load_meta(kb + 2);
    }
    // B fragments one block ahead of the instructions using them
    const uint16_t* xb = &xs[cur][(lane & 31) * kXStride + ks2 * 16];
    u32x4 bf[2];
    bf[0] = *(const u32x4*)xb;
#pragma unroll
    for (int j = 0; j < 4 * TB2; ++j) {
      const int ph = j / TB2, t = j % TB2;  // ph = 2p + h
      if (j + 1 < 4 * TB2) {
        const int ph1 = (j + 1) / TB2, t1 = (j + 1) % TB2;
        bf[(j + 1) & 1] = *(const u32x4*)(xb + t1 * 32 * kXStride + (ph1 >> 1) * 32 + (ph1 & 1) * 8);
      }
      const bf16x8 bv = as_bf16x8(bf[j & 1]);
#pragma unroll
      for (int i = 0; i < RB2; ++i)
        acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][ph >> 1][ph & 1], bv, acc[i][t], 0, 0, 0);
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

#pragma unroll
  for (int i = 0; i < RB2; ++i) {
#pragma unroll
    for (int t = 0; t < TB2; ++t) {
      const int tok = tok0 + t * 32 + (lane & 31);
      if (tok >= tokens) continue;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int row = (brow0 + 2 * i) * 16 + 8 * v4 + 4 * ks2;
        if (row >= rows) continue;
        float* yp = y + (size_t)tok * rows + row;
        const f32x4 val = {acc[i][t][4 * v4 + 0], acc[i][t][4 * v4 + 1], acc[i][t][4 * v4 + 2], acc[i][t][4 * v4 + 3]};
        if (ksplit == 1) {
          *(f32x4*)yp = val;
        } else {
          atomicAdd(yp + 0, val.x);
          atomicAdd(yp + 1, val.y);
          atomicAdd(yp + 2, val.z);
          atomicAdd(yp + 3, val.w);
        }
      }
    }
  }
}

template <int WAVES, int RB2, int TB2>
hipError_t launch_large32_t(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int ksplit,
                            hipStream_t s) {
  const int n_tblk = (int)((tokens + 32 * TB2 - 1) / (32 * TB2));
  const int brows = (int)(w.rows / 16);
  const int n_rblk = (brows + WAVES * 2 * RB2 - 1) / (WAVES * 2 * RB2);
  const dim3 grid((unsigned)(n_tblk * ksplit * n_rblk));
  if (w.exp_mode)
    hipLaunchKernelGGL((fused_large32_kernel<WAVES, RB2, TB2, true>), grid, dim3(WAVES * 64), 0, s, w.sm, w.codes,
                       w.meta, w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens,
                       (int)w.rows, (int)w.cols, ksplit, n_tblk, n_rblk, w.codes_bytes, (int)w.codes_ilv);
  else
    hipLaunchKernelGGL((fused_large32_kernel<WAVES, RB2, TB2, false>), grid, dim3(WAVES * 64), 0, s, w.sm, w.codes,
                       w.meta, w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens,
                       (int)w.rows, (int)w.cols, ksplit, n_tblk, n_rblk, w.codes_bytes, (int)w.codes_ilv);
  return hipGetLastError();
}

// 64 rows x 256 tokens per wave (one wave per SIMD), with the weight rebuild
// of the next K step interleaved into the current step's 32x32x16
// instructions.  At 1024 tokens the rebuild (VALU) work of the smaller tiles
// exceeds the matrix work and, done in a block of its own, adds to it; here
// each instruction group is one MFMA followed by a few VALU and LDS
// operations, so the VALU issues while the matrix core is busy.  The rebuild
// block has no branches: palette lookups run for every row, and rows of raw
// groups are patched afterwards (wave-uniform branch, rare).  Lane mapping
// and D layout as in fused_large32_kernel.
template <bool EXPM>
struct WIl {
  u32x4 s[2][2];
  u32x4 e[2][2];
  u32x2 n[2][2];
  uint32_t anyraw[2];
  bool raw[2];
};

template <bool EXPM, bool GROUPED>
__global__ __launch_bounds__(256) void fused_large_il_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    int ksplit, int n_tblk, int n_rblk, uint64_t codes_bytes, int codes_ilv) {
  constexpr int WAVES = 4, RB2 = 2, TB2 = 8;
  constexpr int TOK = 32 * TB2;
  constexpr int XPER = TOK * 8 / (WAVES * 64);
  constexpr int NXB = GROUPED ? 3 : 2;  // activation tiles in LDS
  __shared__ uint16_t xs[NXB][TOK * kXStride];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, pb = (lane >> 4) & 1, ks2 = lane >> 5;
  const int kbn = cols >> 6;
  const int brows = rows >> 4;
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
  const int brow0 = (rblk * WAVES + wave) * 2 * RB2;
  const uint32_t lut[4] = {in_vgpr(lut0), in_vgpr(lut1), in_vgpr(lut2), in_vgpr(lut3)};
  const uint32_t nweights = (uint32_t)rows * (uint32_t)cols;
  const rsrc_t rs_sm = make_rsrc(sm, nweights);
  const rsrc_t rs_codes = make_rsrc(codes, codes_bytes);
  const rsrc_t rs_side = make_rsrc(side, side_bytes);
  const rsrc_t rs_x = make_rsrc(x, (uint64_t)tokens * cols * 2);
  const uint32_t run = (uint32_t)(ks2 * 16 + r);
  uint32_t voff_s[RB2], voff_n[RB2];
#pragma unroll
  for (int rb = 0; rb < RB2; ++rb) {
    const bool ok = brow0 + 2 * rb + pb < brows;
    voff_s[rb] = ok ? run * 16 + (uint32_t)pb * kbn * 1024 : kOffRange;
    voff_n[rb] = ok ? 0u : kOffRange;  // 0: the row exists; its code offset is computed per step
  }
  uint32_t xoff[XPER];
#pragma unroll
  for (int j = 0; j < XPER; ++j) {
    const int c = threadIdx.x + j * WAVES * 64;
    const int t = c >> 3, piece = c & 7;
    xoff[j] = tok0 + t < tokens ? ((uint32_t)(tok0 + t) * cols) * 2 + piece * 16 : kOffRange;
  }

  f32x16 acc[RB2][TB2];
#pragma unroll
  for (int i = 0; i < RB2; ++i)
#pragma unroll
    for (int t = 0; t < TB2; ++t) acc[i][t] = f32x16{};

  auto load_x = [&](int kb, u32x4 (&xr)[XPER]) {
#pragma unroll
    for (int j = 0; j < XPER; ++j) xr[j] = ld16(rs_x, xoff[j], kb * 128);
  };
  auto store_x = [&](int buf, const u32x4 (&xr)[XPER]) {
#pragma unroll
    for (int j = 0; j < XPER; ++j) {
      const int c = threadIdx.x + j * WAVES * 64;
      const int t = c >> 3, piece = c & 7;
      *(u32x4*)(&xs[buf][t * kXStride + piece * 8]) = xr[j];
    }
  };
  // weight bytes of step kb (per-brick tables read with scalar loads first)
  auto load_w = [&](WIl<EXPM>& wr, int kb) {
    kb = min(kb, hi - 1);  // past the end: re-read the last step (never used)
#pragma unroll
    for (int i = 0; i < RB2; ++i) {
      const uint32_t b = (uint32_t)(brow0 + 2 * i) * kbn + kb;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        wr.s[i][p] = ld16(rs_sm, voff_s[i], b * 1024 + p * 512);
        if (EXPM)
          wr.e[i][p] = ld16(rs_codes, voff_n[i] | (code_brick_off(b + (uint32_t)pb * kbn, 16, codes_ilv) +
                                                 code_lane_off(2 * p + ks2, r, 16, codes_ilv)), 0);
        else
          wr.n[i][p] = ld8(rs_codes, voff_n[i] | (code_brick_off(b + (uint32_t)pb * kbn, 8, codes_ilv) +
                                                code_lane_off(2 * p + ks2, r, 8, codes_ilv)), 0);
      }
      if (!EXPM) {
        uint2 ma = uint2{0u, 0u}, mb = uint2{0u, 0u};
        if (brow0 + 2 * i < brows) ma = meta[(size_t)(brow0 + 2 * i) * kbn + kb];
        if (brow0 + 2 * i + 1 < brows) mb = meta[(size_t)(brow0 + 2 * i + 1) * kbn + kb];
        const uint32_t map = pb ? mb.x : ma.x;
        const uint32_t before = pb ? mb.y : ma.y;
        wr.anyraw[i] = ma.x | mb.x;
        wr.raw[i] = (map >> r) & 1u;
        const uint32_t rank = __builtin_popcount(map & ((1u << r) - 1u));
        const uint32_t base = wr.raw[i] ? (before + rank) * 64 + ks2 * 16 : kOffRange;
        wr.e[i][0] = ld16(rs_side, base, 0);
        wr.e[i][1] = ld16(rs_side, base + 32, 0);
      }
    }
  };
  // branch-free part of the rebuild of row pair i (palette rows; exponent form is all of it)
  auto rebuild_rb = [&](const WIl<EXPM>& wr, bf16x8 (&a)[RB2][2][2], int i) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x4 a0, a1;
      if (EXPM) {
        rebuild_exp2(wr.s[i][p], wr.e[i][p], a0, a1);
      } else {
        uint32_t v[4];
        palette_v(wr.n[i][p], lut, v);
        rebuild_v2(wr.s[i][p], v, a0, a1);
      }
      a[i][p][0] = as_bf16x8(a0);
      a[i][p][1] = as_bf16x8(a1);
    }
  };
  // rows of raw groups: rebuild from the side-table bytes (wave-uniform test)
  auto patch_raw = [&](const WIl<EXPM>& wr, bf16x8 (&a)[RB2][2][2]) {
    if (EXPM) return;
#pragma unroll
    for (int i = 0; i < RB2; ++i) {
      if (wr.anyraw[i]) {
        if (wr.raw[i]) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            u32x4 a0, a1;
            rebuild_exp2(wr.s[i][p], wr.e[i][p], a0, a1);
            a[i][p][0] = as_bf16x8(a0);
            a[i][p][1] = as_bf16x8(a1);
          }
        }
      }
    }
  };

  WIl<EXPM> w;
  bf16x8 acur[RB2][2][2], anext[RB2][2][2];
  // MFMAs of K pair p of the current step (2 halves x TB2 token blocks x RB2 row pairs)
  auto mfma_pair = [&](const uint16_t* xb, int p, bf16x8 (&ac)[RB2][2][2]) {
    u32x4 bf[2];
    bf[0] = *(const u32x4*)(xb + p * 32);
#pragma unroll
    for (int j = 0; j < 2 * TB2; ++j) {
      const int h = j / TB2, t = j % TB2;
      if (j + 1 < 2 * TB2) {
        const int h1 = (j + 1) / TB2, t1 = (j + 1) % TB2;
        bf[(j + 1) & 1] = *(const u32x4*)(xb + t1 * 32 * kXStride + p * 32 + h1 * 8);
      }
      const bf16x8 bv = as_bf16x8(bf[j & 1]);
#pragma unroll
      for (int i = 0; i < RB2; ++i)
        acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[i][p][h], bv, acc[i][t], 0, 0, 0);
    }
  };
  // each MFMA followed by a few VALU ops (32 MFMAs and ~90 VALU per half step)
  auto interleave = [&]() {
#pragma unroll
    for (int j = 0; j < 2 * TB2 * RB2; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // One K step: MFMAs of step kb on ac, interleaved with the rebuild of step
  // kb+1 into an from the bytes in w; the activation tile of step kb+1 goes
  // to LDS between the two halves (its registers are free for the second);
  // then the bytes of step kb+2 are requested.
  // B fragments of one (K pair, half) group: the TB2 token blocks
  auto read_group = [&](const uint16_t* xb, int grp, u32x4 (&bg)[TB2]) {
#pragma unroll
    for (int t = 0; t < TB2; ++t) bg[t] = *(const u32x4*)(xb + t * 32 * kXStride + (grp >> 1) * 32 + (grp & 1) * 8);
  };
  // rebuild quarter q of the next step: row pair q/2, K pair q%2
  auto rebuild_q = [&](const WIl<EXPM>& wr, bf16x8 (&a)[RB2][2][2], int q) {
    const int i = q >> 1, p = q & 1;
    u32x4 a0, a1;
    if (EXPM) {
      rebuild_exp2(wr.s[i][p], wr.e[i][p], a0, a1);
    } else {
      uint32_t v[4];
      palette_v(wr.n[i][p], lut, v);
      rebuild_v2(wr.s[i][p], v, a0, a1);
    }
    a[i][p][0] = as_bf16x8(a0);
    a[i][p][1] = as_bf16x8(a1);
  };
  // B fragments of group 0 of the next step, read during the last group of the
  // current one (grouped form)
  u32x4 bg[2][TB2];
  auto step = [&](int kb, bf16x8 (&ac)[RB2][2][2], bf16x8 (&an)[RB2][2][2]) {
    const int cur = GROUPED ? (kb - lo) % 3 : (kb - lo) & 1;
    const int nxt = GROUPED ? (cur == 2 ? 0 : cur + 1) : cur ^ 1;
    const bool more = kb + 1 < hi;
    u32x4 xr[XPER];
    if (more) load_x(kb + 1, xr);
    const uint16_t* xb = &xs[cur][(lane & 31) * kXStride + ks2 * 16];
    if (GROUPED) {
      // four groups (K pair p, half h) of TB2 x RB2 MFMAs; the next group's B
      // fragments are read during the current one, a quarter of the next
      // step's rebuild is spread over each group, and the next activation
      // tile is stored after group 1 and published by the step's only
      // barrier, so that group 3 can already read the next step's group 0.
      // Three tiles in LDS: when a wave writes tile kb+2 (step kb+1, group 1)
      // every wave has passed step kb's barrier, so none still reads tile kb-1.
      const uint16_t* xn = &xs[nxt][(lane & 31) * kXStride + ks2 * 16];
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        if (grp + 1 < 4)
          read_group(xb, grp + 1, bg[(grp + 1) & 1]);
        else if (more)
          read_group(xn, 0, bg[0]);
#pragma unroll
        for (int t = 0; t < TB2; ++t)
#pragma unroll
          for (int i = 0; i < RB2; ++i)
            acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[i][grp >> 1][grp & 1], as_bf16x8(bg[grp & 1][t]),
                                                               acc[i][t], 0, 0, 0);
        rebuild_q(w, an, (grp & 1) * 2 + (grp >> 1));
#pragma unroll
        for (int j = 0; j < TB2 * RB2; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          if (j & 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (grp == 1) {
          if (more) store_x(nxt, xr);
          __syncthreads();
        }
      }
      patch_raw(w, an);
      load_w(w, kb + 2);
    } else {
      mfma_pair(xb, 0, ac);
      rebuild_rb(w, an, 0);
      interleave();
      if (more) store_x(nxt, xr);
      mfma_pair(xb, 1, ac);
      rebuild_rb(w, an, 1);
      interleave();
      patch_raw(w, an);
      load_w(w, kb + 2);
      __syncthreads();
    }
  };

  {
    u32x4 xr[XPER];
    load_x(lo, xr);
    load_w(w, lo);
    store_x(0, xr);
  }
  __syncthreads();
  rebuild_rb(w, acur, 0);
  rebuild_rb(w, acur, 1);
  patch_raw(w, acur);
  load_w(w, lo + 1);
  if (GROUPED) read_group(&xs[0][(lane & 31) * kXStride + ks2 * 16], 0, bg[0]);
  int kb = lo;
  for (; kb + 1 < hi; kb += 2) {
    step(kb, acur, anext);
    step(kb + 1, anext, acur);
  }
  if (kb < hi) step(kb, acur, anext);

#pragma unroll
  for (int i = 0; i < RB2; ++i) {
#pragma unroll
    for (int t = 0; t < TB2; ++t) {
      const int tok = tok0 + t * 32 + (lane & 31);
      if (tok >= tokens) continue;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int row = (brow0 + 2 * i) * 16 + 8 * v4 + 4 * ks2;
        if (row >= rows) continue;
        float* yp = y + (size_t)tok * rows + row;
        const f32x4 val = {acc[i][t][4 * v4 + 0], acc[i][t][4 * v4 + 1], acc[i][t][4 * v4 + 2], acc[i][t][4 * v4 + 3]};
        if (ksplit == 1) {
          *(f32x4*)yp = val;
        } else {
          atomicAdd(yp + 0, val.x);
          atomicAdd(yp + 1, val.y);
          atomicAdd(yp + 2, val.z);
          atomicAdd(yp + 3, val.w);
        }
      }
    }
  }
}

template <bool GROUPED>
hipError_t launch_large_il(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int ksplit, hipStream_t s) {
  const int n_tblk = (int)((tokens + 255) / 256);
  const int brows = (int)(w.rows / 16);
  const int n_rblk = (brows + 15) / 16;
  const dim3 grid((unsigned)(n_tblk * ksplit * n_rblk));
  if (w.exp_mode)
    hipLaunchKernelGGL((fused_large_il_kernel<true, GROUPED>), grid, dim3(256), 0, s, w.sm, w.codes, w.meta, w.side,
                       w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens, (int)w.rows,
                       (int)w.cols, ksplit, n_tblk, n_rblk, w.codes_bytes, (int)w.codes_ilv);
  else
    hipLaunchKernelGGL((fused_large_il_kernel<false, GROUPED>), grid, dim3(256), 0, s, w.sm, w.codes, w.meta, w.side,
                       w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens, (int)w.rows,
                       (int)w.cols, ksplit, n_tblk, n_rblk, w.codes_bytes, (int)w.codes_ilv);
  return hipGetLastError();
}

}  // namespace

// tile ids, 16x16x32 instructions: 0 = 4 waves x (64 rows x 128 tokens); 1 = 4 waves x (32 rows x 128 tokens);
//           2 = 2 waves x (64 rows x 128 tokens); 3 = 4 waves x (64 rows x 64 tokens)
// 32x32x16 instructions: 4 = 4 waves x (64 rows x 128 tokens); 5 = 4 waves x (32 rows x 128 tokens);
//           6 = 2 waves x (64 rows x 128 tokens); 7 = 4 waves x (64 rows x 64 tokens);
//           8 = 4 waves x (64 rows x 256 tokens); 9 = 4 waves x (32 rows x 256 tokens)
// 10 = tile 8 with the next step's rebuild interleaved into the MFMAs; 11 = 10 with B fragments
// read in groups of 8, one group ahead; 12-14: deep-prefetch tiles of fused_ring.hip
hipError_t launch_fused_ring(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int tile, hipStream_t s);
hipError_t launch_fused_wide(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, hipStream_t s);

hipError_t launch_fused_large(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                              hipStream_t s) {
  if (v.tile == 22) return launch_fused_wide(w, x, y, tokens, s);  // no K split
  if (v.tile >= 12) return launch_fused_ring(w, x, y, tokens, v.tile, s);  // no K split
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
    case 4: return launch_large32_t<4, 2, 4>(w, x, y, tokens, ks, s);
    case 5: return launch_large32_t<4, 1, 4>(w, x, y, tokens, ks, s);
    case 6: return launch_large32_t<2, 2, 4>(w, x, y, tokens, ks, s);
    case 7: return launch_large32_t<4, 2, 2>(w, x, y, tokens, ks, s);
    case 8: return launch_large32_t<4, 2, 8>(w, x, y, tokens, ks, s);
    case 9: return launch_large32_t<4, 1, 8>(w, x, y, tokens, ks, s);
    case 10: return launch_large_il<false>(w, x, y, tokens, ks, s);
    case 11: return launch_large_il<true>(w, x, y, tokens, ks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uw
