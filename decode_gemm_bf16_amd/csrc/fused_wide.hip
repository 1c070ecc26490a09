// Fused reconstruct-GEMM for about a thousand tokens (gfx950): every weight
// rebuilt once per 512 tokens and shared through LDS.
//
// Unweight page, sections 七 and 十: the reconstructing matmul, and at large
// batch the cost of rebuilding the same weight tile again for every token
// tile.  The tiles of fused_large.hip and fused_ring.hip rebuild each brick in
// the registers of the wave that multiplies it, so a weight is rebuilt once
// per 128 or 256 tokens.  Here a workgroup owns 128 rows (8 brick-rows) and
// 512 tokens; its four waves split the tokens (128 each) and all multiply the
// same 128 rows, whose bf16 values the workgroup rebuilds once per 32-column
// sub-step into LDS -- one 16-weight run per lane -- so a weight is rebuilt
// twice for 1024 tokens.
//
// One wave per SIMD (256 accumulators), so nothing but the depth of the
// prefetch hides memory latency:
//  * activations: each wave moves its own 128 tokens x 32 columns (8 KB) of
//    sub-step u + 3 straight from memory into a private ring of four LDS
//    tiles (buffer_load ... lds: no registers; 16 tokens x 64 bytes per
//    instruction); no other wave reads them, so no barrier is involved;
//  * compressed weights (sign+mantissa, 4-bit codes, raw side-table bytes)
//    of sub-step u + 4 into a ring of four register stages;
//  * sub-step u + 1 is rebuilt into the other of two bf16 tiles while the
//    32 MFMAs (32x32x16) of sub-step u run; one barrier per sub-step
//    publishes it.
// The vector-memory counter completes in issue order.  Each sub-step issues
// its weight loads before its activation DMAs, so waiting for a stage's
// weights never waits for activations requested with it, and the explicit
// wait for the activations of sub-step u counts exactly the loads of the two
// sub-steps after theirs.  K is padded to whole groups of four sub-steps:
// a sub-step past the end multiplies zero activations (out-of-range loads,
// dropped by the buffer unit) by finite weights rebuilt from zero bytes.
//
// LDS tiles are 64 bytes a row (token); the 16-byte piece pc of row t sits
// at pc ^ ((t / 4) & 3), so the 16 rows a read touches at once fall into
// distinct banks.
#include <type_traits>

#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 128;                  // rows of a workgroup (8 brick-rows)
constexpr int kBR = kRows / 16;
constexpr int kRB = kRows / 32;             // 32-row blocks (MFMA M) of a wave
constexpr int kTBW = 4;                     // 32-token blocks of a wave
constexpr int kTokW = 32 * kTBW;            // tokens of a wave (128)
constexpr int kTok = kTokW * kWaves;        // tokens of a workgroup (512)
constexpr int kNX = 4;                      // activation tiles per wave (sub-steps)
constexpr int kLX = kNX - 1;                // sub-steps an activation tile is requested ahead
constexpr int kDW = 4;                      // weight register stages (sub-steps ahead)
constexpr int kATile = kRows * 64;          // bytes of one rebuilt bf16 tile (32 columns)
constexpr int kXTile = kTokW * 64;          // bytes of one wave's activation tile
constexpr int kMaxKbn = (int)kWideKbnMax;  // longest K (in 64-column bricks) whose tables fit LDS
constexpr int kUnroll = 4;                  // sub-steps per loop trip (stage, tile and parity indices static)
static_assert(kUnroll % kNX == 0 && kUnroll % kDW == 0 && kUnroll % 2 == 0, "static ring indices");

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the rebuilt tiles: this wave's LDS stores complete,
// then s_barrier.  __syncthreads() would also wait for every load in flight
// (the activation DMAs write LDS, so its fence drains them), emptying the
// prefetch ring at every sub-step; the DMAs' own LDS tiles are private to
// the wave and covered by the explicit vector-memory waits.  The "memory"
// clobber keeps the compiler from moving LDS or memory accesses across it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t tile_off(int row, int piece) {
  return (uint32_t)row * 64u + (uint32_t)((piece ^ ((row >> 2) & 3)) << 4);
}

template <bool EXPM>
struct WStage {
  u32x4 s;   // sign+mantissa of the lane's run
  u32x4 e;   // exponent bytes (exponent form) or raw side-table bytes (zeros off raw rows)
  u32x2 n;   // 4-bit codes
  bool raw;
};

template <bool EXPM>
__global__ __launch_bounds__(kThreads) void fused_wide_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    int n_tblk, int n_rblk, uint64_t codes_bytes, int codes_ilv) {
  constexpr int WL = EXPM ? 2 : 3;  // weight loads per lane per sub-step
  constexpr int XL = kXTile / 1024;  // activation DMAs per lane per sub-step (8)
  // Separate LDS objects for the rebuilt tiles, each activation ring stage
  // and the tables: the compiler then sees that a read of one does not
  // depend on the DMAs into the others, and waits only for those it must.
  __shared__ __attribute__((aligned(1024))) uint8_t at0[kATile], at1[kATile];
  __shared__ __attribute__((aligned(1024))) uint8_t xr0[kWaves * kXTile], xr1[kWaves * kXTile],
      xr2[kWaves * kXTile], xr3[kWaves * kXTile];
  __shared__ __attribute__((aligned(16))) uint2 mtab[kBR * kMaxKbn];
  static_assert(kNX == 4, "one LDS object per activation stage");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto atile = [&](int i) -> uint8_t* { return (i & 1) ? at1 : at0; };
  auto xstage = [&](int i) -> uint8_t* {  // this wave's tile of stage i
    uint8_t* b = i == 0 ? xr0 : i == 1 ? xr1 : i == 2 ? xr2 : xr3;
    return b + wave * kXTile;
  };
  const int kbn = cols >> 6;
  const int brows = rows >> 4;
  const int nsub = 2 * kbn;

  // workgroup -> (token block, row block); the token blocks of one row block
  // on one XCD (workgroup g runs on XCD g % 8), so they share its L2
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
  const int wbr0 = rblk * kBR;                  // first brick-row of the workgroup
  const int tok0 = tblk * kTok + wave * kTokW;  // first token of this wave

  // ---- rebuild role: brick-row br of the workgroup, row r, quarter 2p + qh
  // of sub-step p of a brick column
  const int br = (int)threadIdx.x >> 5;  // = 2 * wave + (lane >> 5)
  const int r = lane & 15, qh = (lane >> 4) & 1, pb = lane >> 5;
  const bool row_ok = wbr0 + br < brows;
  const uint32_t lut[4] = {in_vgpr(lut0), in_vgpr(lut1), in_vgpr(lut2), in_vgpr(lut3)};
  const uint32_t nweights = (uint32_t)rows * (uint32_t)cols;
  const rsrc_t rs_sm = make_rsrc(sm, nweights);
  const rsrc_t rs_codes = make_rsrc(codes, codes_bytes);
  const rsrc_t rs_side = make_rsrc(side, side_bytes);
  const rsrc_t rs_x = make_rsrc(x, (uint64_t)tokens * cols * 2);
  constexpr uint32_t CS = EXPM ? 16 : 8;  // code bytes per run
  uint32_t vsm[2], vcode[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = 2 * p + qh;
    vsm[p] = row_ok ? (uint32_t)pb * (uint32_t)kbn * 1024u + (uint32_t)(q * 16 + r) * 16u : kOffRange;
    vcode[p] = row_ok ? code_lane_off(q, r, CS, codes_ilv) : kOffRange;
  }

  // ---- activation DMA: instruction j moves tokens 16j .. 16j+15 of the
  // wave, 4 lanes a token (lane i: token 16j + i/4, stored piece i%4, which
  // holds global piece (i%4) ^ ((token/4) & 3))
  uint32_t xoff[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int tl = 16 * j + (lane >> 2), t = tok0 + tl;
    const int pc = (lane & 3) ^ ((tl >> 2) & 3);
    xoff[j] = t < tokens ? (uint32_t)t * (uint32_t)cols * 2u + (uint32_t)pc * 16u : kOffRange;
  }

  // the workgroup's per-brick tables to LDS (palette form)
  if (!EXPM) {
    for (int i = threadIdx.x; i < kBR * kbn; i += kThreads) {
      const int b = wbr0 + i / kbn;
      mtab[i] = b < brows ? meta[(size_t)b * kbn + (i % kbn)] : uint2{0u, 0u};
    }
  }
  __syncthreads();

  // weights of sub-step u (brick column u/2, quarters 2(u%2), +1): the lane's run
  // (m: the brick's table entry, read a sub-step earlier so that no LDS
  // round trip sits between these loads)
  auto table_of = [&](int u) -> uint2 {
    return EXPM ? uint2{0u, 0u} : mtab[br * kbn + min(u >> 1, kbn - 1)];
  };
  // Past the end of K the last brick column is read again (its product
  // with the zero activations of those sub-steps adds nothing); every
  // offset is computed without a branch, out-of-range lanes by OR-ing in
  // kOffRange.
  auto load_w = [&](WStage<EXPM>& w, int u, uint2 m) {
    const int p = u & 1;
    const int kc = min(u >> 1, kbn - 1);
    const uint32_t bw = (uint32_t)(wbr0 + 2 * wave) * (uint32_t)kbn + (uint32_t)kc;  // the wave's first brick
    const uint32_t cb0 = code_brick_off(bw, CS, codes_ilv), cb1 = code_brick_off(bw + kbn, CS, codes_ilv);
    const uint32_t dpb = pb ? cb1 - cb0 : 0u;
    w.s = ld16(rs_sm, vsm[p], bw * 1024u);
    if (EXPM) {
      w.e = ld16(rs_codes, vcode[p] + dpb, cb0);
      w.raw = false;
    } else {
      w.n = ld8(rs_codes, vcode[p] + dpb, cb0);
      const bool raw = row_ok && ((m.x >> r) & 1u);
      const uint32_t rank = __builtin_popcount(m.x & ((1u << r) - 1u));
      w.e = ld16(rs_side, ((m.y + rank) * 64u + (uint32_t)(2 * p + qh) * 16u) | (raw ? 0u : kOffRange), 0);
      w.raw = raw;
    }
  };

  // activations of sub-step u into this wave's tile u % kNX
  auto issue_x = [&](int u, int j) {
    const int kb = u >> 1, p = u & 1;
    const bool live = kb < kbn;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs_x, (__attribute__((address_space(3))) void*)(xstage(u % kNX) + j * 1024), 16,
        (int)(xoff[j] | (live ? 0u : kOffRange)), live ? kb * 128 + 64 * p : 0, 0, 0);
  };

  // Rebuild of the lane's run of sub-step u (stage w) into tile u % 2, in
  // three parts that the sub-step spreads over its MFMAs: the rotated
  // exponents of the 16 weights (palette lookups, raw rows from the side
  // table), then weights 0-7 and 8-15 assembled and stored.
  auto rebuild_v = [&](const WStage<EXPM>& w, uint32_t (&v)[4]) {
    if (EXPM) {
      v[0] = rot_exp(w.e.x);
      v[1] = rot_exp(w.e.y);
      v[2] = rot_exp(w.e.z);
      v[3] = rot_exp(w.e.w);
    } else {
      palette_v(w.n, lut, v);
      v[0] = w.raw ? rot_exp(w.e.x) : v[0];
      v[1] = w.raw ? rot_exp(w.e.y) : v[1];
      v[2] = w.raw ? rot_exp(w.e.z) : v[2];
      v[3] = w.raw ? rot_exp(w.e.w) : v[3];
    }
  };
  auto rebuild_half = [&](const WStage<EXPM>& w, const uint32_t (&v)[4], int u, int half) {
    uint32_t p[4];
    assemble_v(half ? w.s.z : w.s.x, v[2 * half], p[0], p[1]);
    assemble_v(half ? w.s.w : w.s.y, v[2 * half + 1], p[2], p[3]);
    *(u32x4*)(atile(u) + tile_off(br * 16 + r, 2 * qh + half)) = u32x4{p[0], p[1], p[2], p[3]};
  };
  auto rebuild = [&](const WStage<EXPM>& w, int u) {
    uint32_t v[4];
    rebuild_v(w, v);
    rebuild_half(w, v, u, 0);
    rebuild_half(w, v, u, 1);
  };

  f32x16 acc[kRB][kTBW];
#pragma unroll
  for (int i = 0; i < kRB; ++i)
#pragma unroll
    for (int t = 0; t < kTBW; ++t) acc[i][t] = f32x16{};

  // prologue: weights of sub-steps 0..kDW-1, activations of 0..kLX-1, then
  // sub-step 0's tile
  WStage<EXPM> ws[kDW];
#pragma unroll
  for (int u = 0; u < kDW; ++u) load_w(ws[u], u, table_of(u));
  uint2 mnext = table_of(kDW);
#pragma unroll
  for (int u = 0; u < kLX; ++u)
#pragma unroll
    for (int j = 0; j < XL; ++j) issue_x(u, j);
  wait_vm<0>();
  rebuild(ws[0], 0);
  __syncthreads();

  // One sub-step u (U = u % kUnroll, static): wait for this wave's
  // activation tile of u (requested three sub-steps ago: the loads of the
  // two sub-steps after it may still be in flight), request the weights of
  // u + kDW (into the stage u's weights left) and the activations of u + kLX
  // (into the tile u - 1 left), 32 MFMAs on tile u % 2 and the wave's tile,
  // with the rebuild of u + 1 into the other tile interleaved; the barrier
  // publishes it.
  auto substep = [&](int u, auto Uc) {
    constexpr int U = decltype(Uc)::value;
    wait_vm<2 * (WL + XL)>();
    const uint8_t* at = atile(U);
    const uint8_t* xt = xstage(U % kNX);
    // A fragment (rb, h): row 32 rb + lane%32, piece 2 (lane/32) + h (lanes
    // 0-31 carry quarter 2p, lanes 32-63 quarter 2p + 1, each half h); B
    // the same for token 32 tb + lane%32 of the wave's tile
    u32x4 af[kRB][2];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        af[rb][h] = *(const u32x4*)(at + tile_off(rb * 32 + (lane & 31), 2 * (lane >> 5) + h));
    auto read_b = [&](int tb, int h) {
      return *(const u32x4*)(xt + tile_off(tb * 32 + (lane & 31), 2 * (lane >> 5) + h));
    };
    u32x4 bq[2][2];
    bq[0][0] = read_b(0, 0);
    bq[0][1] = read_b(0, 1);
    load_w(ws[U % kDW], u + kDW, mnext);
    // the next sub-step's rebuild: its palette lookups fill the wait for
    // these reads, the rest goes between the MFMA groups below
    const WStage<EXPM>& wn = ws[(U + 1) % kDW];
    uint32_t v[4];
    if (!EXPM) palette_lookup(wn.n.x, lut, v[0], v[1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < kTBW; ++tb) {
      if (tb + 1 < kTBW) {
        bq[(tb + 1) & 1][0] = read_b(tb + 1, 0);
        bq[(tb + 1) & 1][1] = read_b(tb + 1, 1);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[rb][h]), as_bf16x8(bq[tb & 1][h]),
                                                                acc[rb][tb], 0, 0, 0);
          if (h == 1 && rb < XL / kTBW) issue_x(u + kLX, tb * (XL / kTBW) + rb);
        }
      if (tb == 0) {
        if (EXPM) {
          v[0] = rot_exp(wn.e.x);
          v[1] = rot_exp(wn.e.y);
          v[2] = rot_exp(wn.e.z);
          v[3] = rot_exp(wn.e.w);
        } else {
          palette_lookup(wn.n.y, lut, v[2], v[3]);
          v[0] = wn.raw ? rot_exp(wn.e.x) : v[0];
          v[1] = wn.raw ? rot_exp(wn.e.y) : v[1];
          v[2] = wn.raw ? rot_exp(wn.e.z) : v[2];
          v[3] = wn.raw ? rot_exp(wn.e.w) : v[3];
        }
      }
      if (tb == 1 || tb == 2) rebuild_half(wn, v, u + 1, tb - 1);
      if (tb == 3) mnext = table_of(u + kDW + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    tile_barrier();
  };

  constexpr std::integral_constant<int, 0> U0{};
  constexpr std::integral_constant<int, 1> U1{};
  constexpr std::integral_constant<int, 2> U2{};
  constexpr std::integral_constant<int, 3> U3{};
  for (int u = 0; u < nsub; u += kUnroll) {
    substep(u, U0);
    substep(u + 1, U1);
    substep(u + 2, U2);
    substep(u + 3, U3);
  }
  wait_vm<0>();

  // Epilogue through the wave's own (now idle) activation tile: a lane holds
  // 4 consecutive rows of one token per accumulator group, so stored
  // directly one instruction would write 32-byte pieces of 32 token rows.
  // Per 32 tokens x 64 rows (8 KB) the wave writes its accumulators into
  // LDS token-major (16-byte chunk c of token t at c ^ (t % 16)), then each
  // store instruction writes 4 tokens' 256 contiguous bytes.
  uint8_t* ep = xstage(0);
  const int row0 = wbr0 * 16;
#pragma unroll
  for (int tb = 0; tb < kTBW; ++tb) {
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
      const int t = lane & 31;
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int rb = 2 * rh + r2;
          const int chunk = r2 * 8 + 2 * v4 + (lane >> 5);  // rows 4 chunk .. 4 chunk + 3 of the half
          const f32x4 val = {acc[rb][tb][4 * v4 + 0], acc[rb][tb][4 * v4 + 1], acc[rb][tb][4 * v4 + 2],
                             acc[rb][tb][4 * v4 + 3]};
          *(f32x4*)(ep + t * 256 + ((chunk ^ (t & 15)) << 4)) = val;
        }
      __builtin_amdgcn_wave_barrier();
      const int chunk = lane & 15;
      const int row = row0 + rh * 64 + chunk * 4;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tt = 4 * j + (lane >> 4);
        const f32x4 val = *(const f32x4*)(ep + tt * 256 + ((chunk ^ (tt & 15)) << 4));
        const int tok = tok0 + tb * 32 + tt;
        if (tok < tokens && row < rows) *(f32x4*)(y + (size_t)tok * rows + row) = val;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

}  // namespace


// tile 22: 4 waves x (128 rows x 128 tokens), weights rebuilt into LDS once
// per 512 tokens
hipError_t launch_fused_wide(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, hipStream_t s) {
  const int n_tblk = (int)((tokens + kTok - 1) / kTok);
  const int brows = (int)(w.rows / 16);
  const int n_rblk = (brows + kBR - 1) / kBR;
  if (w.cols / 64 > kMaxKbn) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(n_tblk * n_rblk));
#define UW_LAUNCH(E)                                                                                          \
  hipLaunchKernelGGL((fused_wide_kernel<E>), grid, dim3(kThreads), 0, s, w.sm, w.codes, w.meta, w.side,       \
                     w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens, (int)w.rows,   \
                     (int)w.cols, n_tblk, n_rblk, w.codes_bytes, (int)w.codes_ilv)
  if (w.exp_mode)
    UW_LAUNCH(true);
  else
    UW_LAUNCH(false);
#undef UW_LAUNCH
  return hipGetLastError();
}

}  // namespace uw
