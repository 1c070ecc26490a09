// Fused reconstruct-GEMM for a few dozen tokens (gfx950): the activations of
// one K slice in LDS, shared by many brick-rows.
//
// Unweight page, sections 六 and 七: the weights are rebuilt from their
// stored bytes in registers, used as the matrix operand and never written
// back.  For 17..64 tokens the activations (tokens x K bf16) no longer fit
// LDS whole, and reading them from L2 per 16-row brick-row (what the small
// kernel does) reads them once per brick-row: at 64 tokens 470 MB of L2
// reads for the 14336 x 4096 gate against 88 MB of weights.  Here a
// workgroup of WAVES waves takes WAVES brick-rows (one per wave) and one K
// slice of slice_kb bricks: the slice's activations go to LDS once, every
// wave streams its brick-row's bytes through a ring of D stages as the GEMV
// kernel does, and the K slices of a brick-row add into a zeroed Y with
// atomics.  Per brick a wave rebuilds 16 weights per lane once and issues two
// 16x16x32 MFMAs per 16-token block.
#include <algorithm>

#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

struct MStage {
  u32x4 s;       // sign+mantissa bytes
  u32x4 e;       // exponent form: exponent bytes; palette form: raw side-table bytes (zeros off raw rows)
  u32x2 n;       // palette form: 4-bit codes
  uint32_t map;  // palette form: wave-uniform raw-row map of the brick
};

// two workgroups per CU: at most 64 VGPRs for 16 waves, 128 for 8
template <int WAVES, int TB, int D, bool EXPM>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WAVES / 2, 8))) void fused_mid_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    int slice_kb, int ksplit, uint64_t codes_bytes, int codes_ilv) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int kbn = cols >> 6, brows = rows >> 4;
  const int brow = blockIdx.x * WAVES + wave;
  const int kb0 = blockIdx.y * slice_kb;
  const int nk = min(slice_kb, kbn - kb0);  // bricks of the slice (> 0: the host sizes the grid)
  const bool has_row = brow < brows;
  const uint32_t lut[4] = {lut0, lut1, lut2, lut3};
  const uint32_t nweights = (uint32_t)rows * (uint32_t)cols;
  const rsrc_t rs_sm = make_rsrc(sm, nweights);
  const rsrc_t rs_codes = make_rsrc(codes, codes_bytes);
  const rsrc_t rs_side = make_rsrc(side, side_bytes);
  const rsrc_t rs_x = make_rsrc(x, (uint64_t)tokens * cols * 2);
  constexpr uint32_t CS = EXPM ? 16 : 8;
  const uint32_t lane16 = lane * 16;
  const uint32_t clane = code_lane_off(q, r, CS, codes_ilv);
  // LDS: the slice's activations, token t at row t (xrow bytes, 16 more than
  // the slice so that consecutive tokens start 4 banks apart), a 32-byte zero
  // tail read by lanes of absent tokens, then the per-brick tables of the
  // waves' brick-rows
  extern __shared__ __attribute__((aligned(16))) uint8_t mid_lds[];
  const uint32_t xrow = (uint32_t)slice_kb * 128 + 16;
  const uint32_t xbytes = (uint32_t)tokens * xrow;
  uint2* ms = (uint2*)(mid_lds + xbytes + 32);
  uint32_t xl[TB], xs[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = tb * 16 + r;
    xl[tb] = t < tokens ? (uint32_t)t * xrow + q * 32 : xbytes;
    xs[tb] = t < tokens ? 128u : 0u;  // bytes per brick along a token row
  }

  const uint32_t brick0 = (uint32_t)brow * kbn + kb0;
  auto fetch = [&](MStage& st, int i, bool table_in_lds) {
    i = min(i, nk - 1);  // a stage past the end re-reads the last brick; compute skips it
    const uint32_t b = brick0 + i;
    st.s = ld16s(rs_sm, has_row ? lane16 : kOffRange, b * 1024);
    if (EXPM) {
      st.e = ld16s(rs_codes, has_row ? clane : kOffRange, code_brick_off(b, 16, codes_ilv));
    } else {
      const uint2 m = has_row ? (table_in_lds ? ms[wave * slice_kb + i] : meta[b]) : uint2{0u, 0u};
      const uint32_t map = __builtin_amdgcn_readfirstlane(m.x);
      const uint32_t before = __builtin_amdgcn_readfirstlane(m.y);
      st.n = ld8s(rs_codes, has_row ? clane : kOffRange, code_brick_off(b, 8, codes_ilv));
      st.map = map;
      const bool raw = (map >> r) & 1u;
      const uint32_t rank = __builtin_popcount(map & ((1u << r) - 1u));
      st.e = ld16s(rs_side, raw ? (before + rank) * 64 + q * 16 : kOffRange, 0);
    }
  };
  f32x4 acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const MStage& st, int i) {
    u32x4 w0, w1;
    if (EXPM) {
      rebuild_exp2(st.s, st.e, w0, w1);
    } else {
      uint32_t v[4];
      palette_v(st.n, lut, v);
      if (st.map) {  // wave-uniform: the brick holds a raw group
        if ((st.map >> r) & 1u) {
          v[0] = rot_exp(st.e.x);
          v[1] = rot_exp(st.e.y);
          v[2] = rot_exp(st.e.z);
          v[3] = rot_exp(st.e.w);
        }
      }
      rebuild_v2(st.s, v, w0, w1);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const u32x4* p = (const u32x4*)(mid_lds + xl[tb] + (uint32_t)i * xs[tb]);
      acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w0), as_bf16x8(p[0]), acc[tb], 0, 0, 0);
      acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w1), as_bf16x8(p[1]), acc[tb], 0, 0, 0);
    }
  };

  MStage st[D];
#pragma unroll
  for (int j = 0; j < D; ++j) fetch(st[j], j, false);  // the first stages read the table from global memory
  {
    // the slice's activations (16-byte pieces, 8 per brick and token) and the
    // tables, every load issued before the first store
    constexpr int NT = WAVES * 64;
    constexpr int NXV = (int)((kMidLdsBytes / 16 + NT - 1) / NT);
    const int per_tok = nk * 8, pieces = tokens * per_tok;
    u32x4 xv[NXV];
#pragma unroll
    for (int k = 0; k < NXV; ++k) {
      const int idx = threadIdx.x + k * NT;
      const int t = idx / per_tok, rem = idx - t * per_tok;
      xv[k] = ld16(rs_x, idx < pieces ? ((uint32_t)t * cols + (uint32_t)kb0 * 64 + rem * 8) * 2 : kOffRange, 0);
    }
#pragma unroll
    for (int k = 0; k < NXV; ++k) {
      const int idx = threadIdx.x + k * NT;
      if (idx < pieces) {
        const int t = idx / per_tok, rem = idx - t * per_tok;
        *(u32x4*)(mid_lds + (uint32_t)t * xrow + rem * 16) = xv[k];
      }
    }
    if (!EXPM) {
      for (int i = threadIdx.x; i < WAVES * nk; i += NT) {
        const int wv = i / nk, kk = i - wv * nk;
        const int br = blockIdx.x * WAVES + wv;
        ms[wv * slice_kb + kk] = br < brows ? meta[(size_t)br * kbn + kb0 + kk] : uint2{0u, 0u};
      }
    }
    if (threadIdx.x < 2) ((u32x4*)(mid_lds + xbytes))[threadIdx.x] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  for (int i = 0; i < nk; i += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (i + j < nk) compute(st[j], i + j);
      fetch(st[j], i + j + D, true);
    }
  }
  // Epilogue: the partial sums go through LDS (the activation region, free
  // once every wave has passed the barrier) so that Y is written -- or, with
  // K split across workgroups, added atomically -- in runs of consecutive
  // rows: a float atomic per element costs several times more when the
  // lanes of an instruction address 16 different tokens.
  __syncthreads();
  float* out = (float*)mid_lds;  // [token][WAVES * 16 rows]
  constexpr int WR = WAVES * 16;
  // D layout: lane l holds rows 4*(l/16)+0..3 of column (token) l%16
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int tok = tb * 16 + r;
    if (tok < tokens) *(f32x4*)&out[tok * WR + wave * 16 + 4 * q] = acc[tb];
  }
  __syncthreads();
  const int row0 = blockIdx.x * WR;
  const int nrow = min(WR, rows - row0);
  for (int e = threadIdx.x; e < tokens * WR; e += WAVES * 64) {
    const int tok = e / WR, rr = e - tok * WR;
    if (rr >= nrow) continue;
    float* yp = y + (size_t)tok * rows + row0 + rr;
    if (ksplit == 1)
      *yp = out[e];
    else
      unsafeAtomicAdd(yp, out[e]);
  }
}

template <int WAVES, int TB, int D>
hipError_t launch_mid_t(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int slice_kb, int ksplit,
                        size_t lds, hipStream_t s) {
  const dim3 grid((unsigned)((w.rows / 16 + WAVES - 1) / WAVES), (unsigned)ksplit);
#define UW_LAUNCH(E)                                                                                                \
  hipLaunchKernelGGL((fused_mid_kernel<WAVES, TB, D, E>), grid, dim3(WAVES * 64), lds, s, w.sm, w.codes, w.meta,   \
                     w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens,               \
                     (int)w.rows, (int)w.cols, slice_kb, ksplit, w.codes_bytes, (int)w.codes_ilv)
  if (w.exp_mode)
    UW_LAUNCH(true);
  else
    UW_LAUNCH(false);
#undef UW_LAUNCH
  return hipGetLastError();
}

template <int WAVES, int D>
hipError_t launch_mid_w(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int slice_kb, int ksplit,
                        size_t lds, hipStream_t s) {
  switch ((tokens + 15) / 16) {
    case 1: return launch_mid_t<WAVES, 1, D>(w, x, y, tokens, slice_kb, ksplit, lds, s);
    case 2: return launch_mid_t<WAVES, 2, D>(w, x, y, tokens, slice_kb, ksplit, lds, s);
    case 3: return launch_mid_t<WAVES, 3, D>(w, x, y, tokens, slice_kb, ksplit, lds, s);
    default: return launch_mid_t<WAVES, 4, D>(w, x, y, tokens, slice_kb, ksplit, lds, s);
  }
}

}  // namespace

size_t mid_lds_bytes(int64_t tokens, int waves, int slice_kb) {
  const size_t in = (size_t)tokens * ((size_t)slice_kb * 128 + 16) + 32 + (size_t)waves * slice_kb * 8;
  const size_t out = (size_t)tokens * waves * 16 * 4;  // the epilogue's partial-sum tile
  return in > out ? in : out;
}

int mid_slice_kb(int64_t tokens, int64_t rows, int64_t cols, int waves) {
  // the largest slice whose activations fit the LDS budget ...
  const int kbn = (int)(cols / 64);
  int s = kbn;
  while (s > 1 && mid_lds_bytes(tokens, waves, s) > kMidLdsBytes) --s;
  // ... split further only until there is a workgroup per CU: every split
  // adds a float atomic per output element, and those cost more than the
  // activations' reuse saves
  const int64_t groups = (rows / 16 + waves - 1) / waves;
  const int64_t want = (256 + groups - 1) / groups;
  const int64_t ks = std::max<int64_t>((kbn + s - 1) / s, std::min<int64_t>(want, kbn));
  return (int)((kbn + ks - 1) / ks);
}

hipError_t launch_fused_mid(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                            hipStream_t s) {
  if (tokens < 1 || tokens > 64) return hipErrorInvalidValue;
  const int kbn = (int)(w.cols / 64);
  const int slice_kb = mid_slice_kb(tokens, w.rows, w.cols, v.waves);
  const int ksplit = (kbn + slice_kb - 1) / slice_kb;
  const size_t lds = mid_lds_bytes(tokens, v.waves, slice_kb);
  if (lds > kMidLdsBytes) return hipErrorInvalidValue;
  if (ksplit > 1) {
    hipError_t e = launch_zero(y, tokens * w.rows, s);
    if (e != hipSuccess) return e;
  }
#define UW_CASE(W, D) \
  if (v.waves == W && v.unroll == D) return launch_mid_w<W, D>(w, x, y, tokens, slice_kb, ksplit, lds, s);
  UW_CASE(16, 2) UW_CASE(8, 2) UW_CASE(16, 3) UW_CASE(4, 2)
#undef UW_CASE
  return hipErrorInvalidValue;
}

}  // namespace uw
