// Fused reconstruct-GEMM for a few hundred tokens (gfx950): deep prefetch of
// both operands.
//
// Unweight page, sections 七 and 十: each weight brick is rebuilt once per
// workgroup, in registers, straight into the A operand of
// v_mfma_f32_32x32x16_bf16, and used for every token block of the workgroup.
// Tile and lane mapping are those of the 32x32x16 tiles of fused_large.hip
// (a wave owns RB2 pairs of brick-rows, the workgroup 32*TB2 tokens).  What
// differs is how far ahead the operands are requested.  Those tiles issue
// every load one K step ahead; with one wave per SIMD a step of MFMAs lasts
// ~0.25 us, well under the memory latency of a loaded chip, so the waves wait
// on memory most of the time (81 us for 256 tokens on the 14336 x 4096 gate,
// against ~16 us of matrix work).  Here
//  * the weight bytes of step k+D are requested at step k into a ring of D
//    register stages (the raw side-table loads are unconditional, with
//    out-of-range offsets off raw rows, so every step issues the same number
//    of loads and the waits stay static);
//  * the activation tile of step k+X-1 goes straight from memory to LDS
//    (buffer_load ... lds) into a ring of X tiles, so it needs no registers;
//    at the end of a step each wave waits for its part of the next tile and
//    the step's barrier publishes it;
//  * the per-brick tables of the workgroup's brick-rows are copied to LDS
//    once, so no scalar load sits on a step's critical path.
// Tiles in LDS have no padding (the DMA writes 1 KB runs); the 16-byte piece
// p of token t sits at piece p ^ ((t/2) & 7) of its 128-byte row instead,
// which spreads a B fragment's 32 tokens over the banks.
#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int RB2, bool EXPM>
struct RStage {
  u32x4 s[RB2][2];  // sign+mantissa runs, K pairs 0 and 1
  u32x4 e[RB2][2];  // exponent bytes (exponent form) or raw side-table bytes (zeros off raw rows)
  u32x2 n[RB2][2];  // 4-bit codes
  bool raw[RB2];
};

// 16 bytes per lane from a buffer straight into LDS: the wave's 64 lanes fill
// the 1 KB at `lds` (wave-uniform) in lane order.
__device__ __forceinline__ void lds_dma16(rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff,
                                           (int)soff, 0, 0);
}

// s_waitcnt with only the vector-memory count limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int RB2, int TB2, int D, int X, int BPF, bool EXPM>
__global__ __launch_bounds__(256) void fused_ring_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    int n_tblk, int n_rblk, uint64_t codes_bytes, int codes_ilv) {
  constexpr int WAVES = 4;
  constexpr int TOK = 32 * TB2;                // tokens per workgroup
  constexpr int TILE = TOK * 128;              // bytes of one activation tile (64 K x TOK tokens)
  constexpr int XL = TILE / 1024 / WAVES;      // 1 KB DMA loads per wave per step (= TB2)
  constexpr int BR = WAVES * 2 * RB2;          // brick-rows of the workgroup
  constexpr int WL = RB2 * (EXPM ? 4 : 6);     // weight loads per wave per step
  static_assert(XL * WAVES * 1024 == TILE, "activation tile split");
  extern __shared__ __attribute__((aligned(16))) uint8_t ring_lds[];
  uint2* mtab = (uint2*)(ring_lds + X * TILE);  // [BR][kbn]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;         // row inside the brick
  const int pb = (lane >> 4) & 1;  // which brick of the pair
  const int ks2 = lane >> 5;       // k-slot
  const int kbn = cols >> 6;
  const int brows = rows >> 4;

  // workgroup -> (token block, row block), the token blocks of one row block
  // on one XCD (workgroup g runs on XCD g % 8) so that they share its L2
  const int g = blockIdx.x;
  int tblk, rblk;
  if ((n_rblk & 7) == 0) {
    const int slot = g >> 3;
    rblk = (slot / n_tblk) * 8 + (g & 7);
    tblk = slot % n_tblk;
  } else {
    tblk = g % n_tblk;
    rblk = g / n_tblk;
  }
  const int tok0 = tblk * TOK;
  const int wbr0 = rblk * BR;                  // first brick-row of the workgroup
  const int brow0 = wbr0 + wave * 2 * RB2;     // first brick-row of this wave
  const uint32_t lut[4] = {in_vgpr(lut0), in_vgpr(lut1), in_vgpr(lut2), in_vgpr(lut3)};
  const uint32_t nweights = (uint32_t)rows * (uint32_t)cols;
  const rsrc_t rs_sm = make_rsrc(sm, nweights);
  const rsrc_t rs_codes = make_rsrc(codes, codes_bytes);
  const rsrc_t rs_side = make_rsrc(side, side_bytes);
  const rsrc_t rs_x = make_rsrc(x, (uint64_t)tokens * cols * 2);
  const uint32_t run = (uint32_t)(ks2 * 16 + r);
  uint32_t voff_s[RB2];
  bool row_ok[RB2];
#pragma unroll
  for (int rb = 0; rb < RB2; ++rb) {
    row_ok[rb] = brow0 + 2 * rb + pb < brows;
    voff_s[rb] = row_ok[rb] ? run * 16 + (uint32_t)pb * kbn * 1024 : kOffRange;
  }
  // activation DMA: load j of this wave moves chunk c = j*WAVES + wave (8
  // tokens x 128 bytes); lane i carries token t = 8c + i/8, stored piece i%8,
  // which holds global piece (i%8) ^ ((t/2) & 7)
  uint32_t xoff[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int c = j * WAVES + wave, t = c * 8 + (lane >> 3);
    const int p = (lane & 7) ^ ((t >> 1) & 7);
    xoff[j] = tok0 + t < tokens ? ((uint32_t)(tok0 + t) * cols + p * 8) * 2 : kOffRange;
  }
  auto issue_x = [&](int kb) {
    const int buf = kb % X;
    const bool live = kb < kbn;  // past the end: zeros into a free tile, same load count
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int c = j * WAVES + wave;
      lds_dma16(rs_x, ring_lds + buf * TILE + c * 1024, live ? xoff[j] : kOffRange, live ? kb * 128 : 0);
    }
  };
  // B fragment offsets: token lane%32 of a 32-token block, piece p(ph) =
  // 2*ks2 + 4*(ph/2) + ph%2 for the (K pair, half) group ph.  With the swizzle
  // by (token/2) % 8 the 64 lanes of a read (32 tokens, two pieces) fall four
  // to each 16-byte bank group of a 256-byte bank row: no conflicts beyond
  // the four passes 1 KB needs.
  uint32_t bsw[4];
#pragma unroll
  for (int ph = 0; ph < 4; ++ph) {
    const int p = 2 * ks2 + 4 * (ph >> 1) + (ph & 1);
    bsw[ph] = (uint32_t)(lane & 31) * 128 + (uint32_t)((p ^ (((lane & 31) >> 1) & 7)) * 16);
  }

  auto table = [&](int i, int b2, int kb, bool in_lds) -> uint2 {
    const int br = brow0 + 2 * i + b2;
    if (EXPM || br >= brows) return uint2{0u, 0u};
    return in_lds ? mtab[(br - wbr0) * kbn + kb] : meta[(size_t)br * kbn + kb];
  };
  // code loads: a per-lane part (run, and out of range for absent rows), the
  // brick's wave-uniform part as the scalar offset, and for the second brick
  // of the pair the (uniform) difference of the two
  constexpr uint32_t CS = EXPM ? 16 : 8;
  uint32_t clo[RB2][2];
#pragma unroll
  for (int i = 0; i < RB2; ++i)
#pragma unroll
    for (int p = 0; p < 2; ++p) clo[i][p] = row_ok[i] ? code_lane_off(2 * p + ks2, r, CS, codes_ilv) : kOffRange;
  auto load_w = [&](RStage<RB2, EXPM>& w, int kb, bool in_lds) {
    kb = min(kb, kbn - 1);  // past the end: re-read the last step (never used)
#pragma unroll
    for (int i = 0; i < RB2; ++i) {
      const uint32_t b = (uint32_t)(brow0 + 2 * i) * kbn + kb;  // first brick of the pair
      const uint32_t cb0 = code_brick_off(b, CS, codes_ilv), cb1 = code_brick_off(b + kbn, CS, codes_ilv);
      const uint32_t dpb = pb ? cb1 - cb0 : 0u;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        w.s[i][p] = ld16(rs_sm, voff_s[i], b * 1024 + p * 512);
        if (EXPM)
          w.e[i][p] = ld16(rs_codes, clo[i][p] + dpb, cb0);
        else
          w.n[i][p] = ld8(rs_codes, clo[i][p] + dpb, cb0);
      }
      if (!EXPM) {
        const uint2 ma = table(i, 0, kb, in_lds), mb = table(i, 1, kb, in_lds);
        const uint32_t mapa = __builtin_amdgcn_readfirstlane(ma.x), mapb = __builtin_amdgcn_readfirstlane(mb.x);
        const uint32_t bfa = __builtin_amdgcn_readfirstlane(ma.y), bfb = __builtin_amdgcn_readfirstlane(mb.y);
        const uint32_t map = pb ? mapb : mapa;
        const uint32_t before = pb ? bfb : bfa;
        w.raw[i] = (map >> r) & 1u;
        const uint32_t rank = __builtin_popcount(map & ((1u << r) - 1u));
        const uint32_t base = w.raw[i] ? (before + rank) * 64 + ks2 * 16 : kOffRange;
        w.e[i][0] = ld16(rs_side, base, 0);
        w.e[i][1] = ld16(rs_side, w.raw[i] ? base + 32 : kOffRange, 0);
      }
    }
  };

  f32x16 acc[RB2][TB2];
#pragma unroll
  for (int i = 0; i < RB2; ++i)
#pragma unroll
    for (int t = 0; t < TB2; ++t) acc[i][t] = f32x16{};

  RStage<RB2, EXPM> w[D];
  // prologue: weights of steps 0..D-1 (tables from global memory), the
  // activation tiles of steps 0..X-2, then the workgroup's tables to LDS
#pragma unroll
  for (int j = 0; j < D; ++j) load_w(w[j], j, false);
#pragma unroll
  for (int j = 0; j < X - 1; ++j) issue_x(j);
  if (!EXPM) {
    for (int i = threadIdx.x; i < BR * kbn; i += 256) {
      const int br = wbr0 + i / kbn;
      mtab[i] = br < brows ? meta[(size_t)br * kbn + (i % kbn)] : uint2{0u, 0u};
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // every load of the prologue (the first tile included)
  __syncthreads();

  // A fragments of a step
  auto rebuild = [&](const RStage<RB2, EXPM>& ws, bf16x8 (&an)[RB2][2][2]) {
#pragma unroll
    for (int i = 0; i < RB2; ++i)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        u32x4 a0, a1;
        if (EXPM) {
          rebuild_exp2(ws.s[i][p], ws.e[i][p], a0, a1);
        } else {
          // rows of raw groups take their exponents from the side table: a
          // per-lane select, so the whole rebuild stays branch-free and can
          // be interleaved with the MFMAs
          uint32_t v[4];
          palette_v(ws.n[i][p], lut, v);
          const bool raw = ws.raw[i];
          v[0] = raw ? rot_exp(ws.e[i][p].x) : v[0];
          v[1] = raw ? rot_exp(ws.e[i][p].y) : v[1];
          v[2] = raw ? rot_exp(ws.e[i][p].z) : v[2];
          v[3] = raw ? rot_exp(ws.e[i][p].w) : v[3];
          rebuild_v2(ws.s[i][p], v, a0, a1);
        }
        an[i][p][0] = as_bf16x8(a0);
        an[i][p][1] = as_bf16x8(a1);
      }
  };

  bf16x8 a[2][RB2][2][2];
  rebuild(w[0], a[0]);
  // One step: request the weights of step kb+D (into the stage step kb was
  // rebuilt from) and the tile of step kb+X-1; the MFMAs of step kb on a[C],
  // each followed by a few VALU ops of the rebuild of step kb+1 into a[C^1]
  // (one wave per SIMD: the VALU issues while the matrix core works); then
  // the wait for this wave's part of tile kb+1 and the barrier that
  // publishes it.
  auto step = [&](RStage<RB2, EXPM>& wcur, const RStage<RB2, EXPM>& wnext, bf16x8 (&ac)[RB2][2][2],
                  bf16x8 (&an)[RB2][2][2], int kb) {
    load_w(wcur, kb + D, true);
    issue_x(kb + X - 1);
    const uint8_t* xb = ring_lds + (kb % X) * TILE;
    // B fragments are read BPF groups ahead (one wave per SIMD: nothing else
    // hides the LDS latency), from a ring of BPF + 1 registers
    constexpr int NG = 4 * TB2, NB = BPF + 1;
    auto read_b = [&](int g) {
      const int ph = g / TB2, t = g % TB2;
      return *(const u32x4*)(xb + t * 4096 + bsw[ph]);
    };
    u32x4 bf[NB];
#pragma unroll
    for (int g = 0; g < BPF && g < NG; ++g) bf[g] = read_b(g);
#pragma unroll
    for (int jj = 0; jj < NG; ++jj) {
      const int ph = jj / TB2, t = jj % TB2;
      if (jj + BPF < NG) bf[(jj + BPF) % NB] = read_b(jj + BPF);
      const bf16x8 bv = as_bf16x8(bf[jj % NB]);
#pragma unroll
      for (int i = 0; i < RB2; ++i)
        acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[i][ph >> 1][ph & 1], bv, acc[i][t], 0, 0, 0);
    }
    rebuild(wnext, an);
    if constexpr (BPF > 1) __builtin_amdgcn_sched_group_barrier(0x100, BPF, 0);  // the first B reads
#pragma unroll
    for (int jj = 0; jj < 4 * TB2 * RB2; ++jj) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // then up to six VALU ops
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // and an LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    // this wave's part of tile kb+1 (requested X-2 steps ago) has landed once
    // at most the loads of the X-2 later steps are outstanding
    wait_vmcnt<(X - 2) * (WL + XL)>();
    __syncthreads();
  };

  static_assert(D % 2 == 0, "the A fragments alternate with the ring stage");
  int kb = 0;
  for (; kb + D <= kbn; kb += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) step(w[j], w[(j + 1) % D], a[j & 1], a[(j + 1) & 1], kb + j);
  }
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (kb + j < kbn) step(w[j], w[(j + 1) % D], a[j & 1], a[(j + 1) & 1], kb + j);

  // Epilogue through LDS (the activation tiles, idle once every copy into
  // them has landed and every wave has passed its last step): a lane holds 4
  // consecutive rows of one token per accumulator group, so stored directly
  // one instruction would write 16-byte pieces of 32 token rows.  Per 32
  // rows x 32 tokens (4 KB of this wave's own LDS) the accumulators go in
  // token-major (16-byte chunk c of token t at c ^ ((t / 2) % 8)), and each
  // store instruction then writes 8 tokens' 128 contiguous bytes.
  wait_vmcnt<0>();
  __syncthreads();
  uint8_t* ep = ring_lds + wave * 4096;
#pragma unroll
  for (int i = 0; i < RB2; ++i) {
#pragma unroll
    for (int t = 0; t < TB2; ++t) {
      const int tw = lane & 31;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int chunk = 2 * v4 + ks2;  // rows 4 chunk .. 4 chunk + 3 of the block
        const f32x4 val = {acc[i][t][4 * v4 + 0], acc[i][t][4 * v4 + 1], acc[i][t][4 * v4 + 2],
                           acc[i][t][4 * v4 + 3]};
        *(f32x4*)(ep + tw * 128 + ((chunk ^ ((tw >> 1) & 7)) << 4)) = val;
      }
      __builtin_amdgcn_wave_barrier();
      const int chunk = lane & 7;
      const int row = (brow0 + 2 * i) * 16 + chunk * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tt = 8 * j + (lane >> 3);
        const f32x4 val = *(const f32x4*)(ep + tt * 128 + ((chunk ^ ((tt >> 1) & 7)) << 4));
        const int tok = tok0 + t * 32 + tt;
        if (tok < tokens && row < rows) *(f32x4*)(y + (size_t)tok * rows + row) = val;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <int RB2, int TB2, int D, int X, int BPF = 1>
hipError_t launch_ring_t(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, hipStream_t s) {
  const int n_tblk = (int)((tokens + 32 * TB2 - 1) / (32 * TB2));
  const int brows = (int)(w.rows / 16);
  const int n_rblk = (brows + 8 * RB2 - 1) / (8 * RB2);
  const int kbn = (int)(w.cols / 64);
  const size_t lds = (size_t)X * 32 * TB2 * 128 + (size_t)8 * RB2 * kbn * 8;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(n_tblk * n_rblk));
#define UW_LAUNCH(E)                                                                                              \
  hipLaunchKernelGGL((fused_ring_kernel<RB2, TB2, D, X, BPF, E>), grid, dim3(256), lds, s, w.sm, w.codes, w.meta,     \
                     w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens,             \
                     (int)w.rows, (int)w.cols, n_tblk, n_rblk, w.codes_bytes, (int)w.codes_ilv)
  if (w.exp_mode)
    UW_LAUNCH(true);
  else
    UW_LAUNCH(false);
#undef UW_LAUNCH
  return hipGetLastError();
}

}  // namespace

// tile ids 12..: 12 = 4 waves x (32 rows x 128 tokens), D 4, X 3; 13 = 4 waves x
// (32 rows x 64 tokens), D 4, X 3; 14 = 4 waves x (64 rows x 128 tokens), D 2, X 3;
// 15 = 12 with X 8; 16 = 13 with X 8; 17 = 12 with D 6, X 6; 18-21: 12, 16, 15 and 14
// with the B fragments read 3, 3, 4 and 2 groups ahead (the others read one ahead)
hipError_t launch_fused_ring(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int tile, hipStream_t s) {
  switch (tile) {
    case 12: return launch_ring_t<1, 4, 4, 3>(w, x, y, tokens, s);
    case 13: return launch_ring_t<1, 2, 4, 3>(w, x, y, tokens, s);
    case 14: return launch_ring_t<2, 4, 2, 3>(w, x, y, tokens, s);
    case 15: return launch_ring_t<1, 4, 4, 8>(w, x, y, tokens, s);
    case 16: return launch_ring_t<1, 2, 4, 8>(w, x, y, tokens, s);
    case 17: return launch_ring_t<1, 4, 6, 6>(w, x, y, tokens, s);
    case 18: return launch_ring_t<1, 4, 4, 3, 3>(w, x, y, tokens, s);
    case 19: return launch_ring_t<1, 2, 4, 8, 3>(w, x, y, tokens, s);
    case 20: return launch_ring_t<1, 4, 4, 8, 4>(w, x, y, tokens, s);
    case 21: return launch_ring_t<2, 4, 2, 3, 2>(w, x, y, tokens, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uw
