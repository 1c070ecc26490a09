// Fused reconstruct-matmul for small batches (1..64 tokens) on gfx950.
//
// Unweight page, section 七 (the reconstructing matmul) and section 五 (weights
// are rebuilt on chip and never written back to HBM).  The pages' Hopper design
// (TMA producer filling a shared-memory ring, consumers issuing WGMMA) is not
// used: here every lane streams its own 16 B of sign+mantissa bytes and 8 B of
// 4-bit codes (or 16 B of exponent bytes) straight from HBM into registers, the
// bf16 words are rebuilt in registers (recon.h) and fed as the A operand of
// v_mfma_f32_16x16x32_bf16; activations are the B operand.  With weights as A,
// a 16-row brick feeds 16 tokens per instruction, so batch 1 and batch 16 cost
// the same matrix-core time, which is negligible next to the HBM stream.
//
// Work split: one workgroup per 16-row brick-row (x `ksplit` slices of K);
// its waves take every WAVES-th group of U bricks along K.  Loads are software
// pipelined: while stage i (U bricks) is rebuilt and multiplied, every load of
// stage i+1 is in flight -- weights, activations and, for bricks holding raw
// groups, the raw side-table bytes, whose addresses come from the per-brick
// table read one stage earlier still.  Partial sums meet in LDS; with
// ksplit > 1 the slices add into a zeroed Y with float atomics.
#include <algorithm>

#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

template <int U, int TB, bool EXPM>
struct Stage {
  u32x4 s[U];          // sign+mantissa bytes
  u32x4 e[U];          // exponent bytes (exponent mode) or raw side-table bytes
  u32x2 n[U];          // 4-bit codes (palette mode)
  u32x4 x[U][TB][2];   // activations: B operand of the two k-halves
  uint32_t anyraw[U];  // wave-uniform: some row of the brick is raw
  bool raw[U];         // this lane's row is raw
};

template <int WAVES, int TB, bool EXPM, int U>
__global__ __launch_bounds__(WAVES * 64) void fused_small_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    int ksplit, uint64_t codes_bytes, int codes_ilv) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;  // row inside the brick (A operand row) / token inside a block (B column)
  const int q = lane >> 4;  // which 16-column quarter of the brick
  const int kbn = cols >> 6;
  const int lo = (int)(((int64_t)blockIdx.y * kbn) / ksplit);
  const int hi = (int)(((int64_t)(blockIdx.y + 1) * kbn) / ksplit);
  const size_t brick_row0 = (size_t)blockIdx.x * kbn;
  const uint32_t lut[4] = {lut0, lut1, lut2, lut3};  // scalar: registers are scarce here
  constexpr int STEP = WAVES * U;
  const uint32_t nweights = (uint32_t)rows * (uint32_t)cols;
  const rsrc_t rs_sm = make_rsrc(sm, nweights);
  const rsrc_t rs_codes = make_rsrc(codes, codes_bytes);
  const rsrc_t rs_side = make_rsrc(side, side_bytes);
  const rsrc_t rs_x = make_rsrc(x, (uint64_t)tokens * cols * 2);
  // per-lane byte offsets, fixed for the whole kernel
  const uint32_t lane16 = lane * 16;
  constexpr uint32_t CS = EXPM ? 16 : 8;  // code-stream bytes per run
  const uint32_t clane = code_lane_off(q, r, CS, codes_ilv);
  uint32_t xlane[TB];
  bool xlive[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int tok = t * 16 + r;
    xlive[t] = tok < tokens;
    xlane[t] = ((uint32_t)tok * cols + q * 16) * 2;
  }

  f32x4 acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-brick table of the stage that will be fetched next
  uint2 mnext[U];
  auto load_meta = [&](int kb0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + u * WAVES;
      mnext[u] = (!EXPM && kb < hi) ? meta[brick_row0 + kb] : uint2{0u, 0u};
    }
  };
  auto fetch = [&](Stage<U, TB, EXPM>& st, int kb0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + u * WAVES;
      if (kb >= hi) break;
      const uint32_t b = (uint32_t)brick_row0 + kb;
      st.s[u] = ld16s(rs_sm, lane16, b * 1024);
      if (EXPM) {
        st.e[u] = ld16s(rs_codes, clane, code_brick_off(b, CS, codes_ilv));
      } else {
        st.n[u] = ld8s(rs_codes, clane, code_brick_off(b, CS, codes_ilv));
        const uint32_t map = mnext[u].x;
        st.anyraw[u] = map;
        st.raw[u] = (map >> r) & 1u;
        if (map && st.raw[u]) {
          const uint32_t rank = __builtin_popcount(map & ((1u << r) - 1u));
          st.e[u] = ld16s(rs_side, (mnext[u].y + rank) * 64 + q * 16, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        st.x[u][t][0] = u32x4{0u, 0u, 0u, 0u};
        st.x[u][t][1] = u32x4{0u, 0u, 0u, 0u};
        if (xlive[t]) {
          st.x[u][t][0] = ld16(rs_x, xlane[t], kb * 128);
          st.x[u][t][1] = ld16(rs_x, xlane[t] + 16, kb * 128);
        }
      }
    }
  };
  auto compute = [&](const Stage<U, TB, EXPM>& st, int kb0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb0 + u * WAVES >= hi) break;
      u32x4 w0, w1;
      if (EXPM) {
        rebuild_exp2(st.s[u], st.e[u], w0, w1);
      } else {
        uint32_t v[4];
        palette_v(st.n[u], lut, v);
        if (st.anyraw[u]) {  // wave-uniform: the brick holds a raw group
          if (st.raw[u]) {
            v[0] = rot_exp(st.e[u].x);
            v[1] = rot_exp(st.e[u].y);
            v[2] = rot_exp(st.e[u].z);
            v[3] = rot_exp(st.e[u].w);
          }
        }
        rebuild_v2(st.s[u], v, w0, w1);
      }
      const bf16x8 a0 = as_bf16x8(w0);
      const bf16x8 a1 = as_bf16x8(w1);
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(st.x[u][t][0]), acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_bf16x8(st.x[u][t][1]), acc[t], 0, 0, 0);
      }
    }
  };

  Stage<U, TB, EXPM> sa, sb;
  int kb = lo + wave;
  load_meta(kb);
  fetch(sa, kb);
  load_meta(kb + STEP);
  while (kb < hi) {
    if (kb + STEP < hi) fetch(sb, kb + STEP);
    load_meta(kb + 2 * STEP);
    compute(sa, kb);
    kb += STEP;
    if (kb >= hi) break;
    if (kb + STEP < hi) fetch(sa, kb + STEP);
    load_meta(kb + 2 * STEP);
    compute(sb, kb);
    kb += STEP;
  }

  // D layout of the 16x16 result: lane l holds rows 4*(l/16)+0..3, column l%16.
  __shared__ f32x4 red[WAVES][TB][64];
#pragma unroll
  for (int t = 0; t < TB; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  for (int i = threadIdx.x; i < TB * 64; i += WAVES * 64) {
    const int t = i >> 6, l = i & 63;
    f32x4 sum = red[0][t][l];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[w][t][l];
    const int tok = t * 16 + (l & 15);
    if (tok >= tokens) continue;
    float* yp = y + (size_t)tok * rows + (size_t)blockIdx.x * 16 + 4 * (l >> 4);
    if (ksplit == 1) {
      *(f32x4*)yp = sum;
    } else {
      atomicAdd(yp + 0, sum.x);
      atomicAdd(yp + 1, sum.y);
      atomicAdd(yp + 2, sum.z);
      atomicAdd(yp + 3, sum.w);
    }
  }
}

// Few tokens whose activations fit in LDS (tokens x cols <= kGemvX): the same
// brick-row-per-workgroup split, arranged so that each wave keeps only weight
// bytes in its load pipeline.  At the start the workgroup moves x, its
// brick-row's per-brick table and the raw groups' side-table bytes of the
// brick-row (one contiguous range: raw groups are numbered in brick order,
// placed by the first and last table entries, read with scalar loads issued
// first) straight from memory into LDS (buffer loads to LDS: no registers, no
// LDS stores), behind the first weight loads, and waits once.  A brick then
// costs two buffer loads: sign+mantissa and codes.  A matrix with a brick-row
// of more raw groups than the LDS copy holds (kGemvSideCap; a quarter of the
// groups at 4096 columns) runs the SIDE_LDS = false form, which reads raw
// groups' bytes from global memory when it meets them instead.
//
// Each wave runs a ring of D + 1 register stages: the loads of brick i + D
// are issued before brick i is rebuilt and multiplied, so D bricks are in
// flight while one is computed.  The main loop holds no branch around the
// loads (a load past the wave's last brick takes an out-of-range offset that
// the buffer unit drops without a memory access), so the compiler's waits
// count exactly the D stages behind the one computed; the last D bricks are
// computed after the loop.  Partial sums are reduced one output per thread.
constexpr int kGemvX = (int)kGemvXElems;   // bf16 elements of x held in LDS
constexpr int kGemvKbn = (int)kGemvKbnMax;  // brick columns whose table fits the LDS copy
constexpr int kGemvSideCap = 256;           // raw groups per brick-row whose bytes fit the LDS copy

// 16 bytes per lane from a buffer straight into LDS: the wave's 64 lanes fill
// the 1 KB at `lds` (wave-uniform) in lane order (4 bytes: 256 B).
__device__ __forceinline__ void lds_dma16_g(rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, 0, 0, 0);
}
__device__ __forceinline__ void lds_dma4_g(rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, (int)voff, 0, 0, 0);
}

// LDS layout of the gemv kernel (bytes): [0, 32) zeros, read as x by the lanes
// of absent tokens; x at kGemvX0, padded to 1 KB; the per-brick table, padded
// to 256 B; the raw-group bytes, padded to 1 KB (whole DMA blocks everywhere:
// lanes past the end of a copy may write zeros into the padding).
constexpr uint32_t kGemvX0 = 1024;
__host__ __device__ inline uint32_t gemv_xpad(uint32_t xbytes) { return (xbytes + 1023) & ~1023u; }
__host__ __device__ inline uint32_t gemv_mpad(uint32_t kbn) { return (kbn * 8 + 255) & ~255u; }
__host__ __device__ inline uint32_t gemv_spad(uint32_t cap) { return (cap * 64 + 1023) & ~1023u; }

struct GStage {
  u32x4 s;          // sign+mantissa bytes
  u32x2 n;          // 4-bit codes
  uint32_t map;     // wave-uniform raw-row map of the brick
  uint32_t before;  // wave-uniform raw groups before the brick
};

// One brick-row (brow) of one matrix: the body of the gemv kernels.
template <int WAVES, int D, bool SIDE_LDS>
__device__ __forceinline__ void gemv_brick_row(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    uint64_t codes_bytes, int codes_ilv, int side_cap, uint32_t brow) {
  constexpr int R = D + 1;  // register stages
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int kbn = cols >> 6;
  const uint32_t brick_row0 = brow * (uint32_t)kbn;
  const uint32_t lut[4] = {lut0, lut1, lut2, lut3};
  const uint32_t nweights = (uint32_t)rows * (uint32_t)cols;
  const rsrc_t rs_sm = make_rsrc(sm, nweights);
  const rsrc_t rs_codes = make_rsrc(codes, codes_bytes);
  const rsrc_t rs_side = make_rsrc(side, side_bytes);
  const rsrc_t rs_x = make_rsrc(x, (uint64_t)tokens * cols * 2);
  const rsrc_t rs_meta = make_rsrc(meta + brick_row0, (uint64_t)kbn * 8);
  const uint32_t lane16 = lane * 16;
  const uint32_t clane = code_lane_off(q, r, 8, codes_ilv);
  const bool live = r < tokens;
  extern __shared__ __attribute__((aligned(1024))) uint8_t gemv_lds[];
  const uint32_t xbytes = (uint32_t)tokens * cols * 2;
  uint8_t* lx = gemv_lds + kGemvX0;
  uint8_t* lm = lx + gemv_xpad(xbytes);
  const uint2* ms = (const uint2*)lm;
  uint8_t* sl = lm + gemv_mpad(kbn);
  const uint32_t xl_lane = live ? kGemvX0 + ((uint32_t)r * cols + q * 16) * 2 : 0u;
  const uint32_t xl_step = live ? 128u : 0u;
  const int nmine = (kbn - wave + WAVES - 1) / WAVES;  // bricks kb = wave + WAVES*i of this wave

  // the first and last table entries place the brick-row's raw-group bytes
  uint2 m_first = {0u, 0u}, m_last = {0u, 0u};
  if (SIDE_LDS) {
    m_first = meta[brick_row0];
    m_last = meta[brick_row0 + kbn - 1];
  }
  // a stage's weight loads (past the wave's last brick: dropped by the range check)
  auto fetch_loads = [&](GStage& st, int i) {
    const bool past = i >= nmine;
    const uint32_t b = brick_row0 + wave + WAVES * i;
    st.s = ld16s(rs_sm, past ? kOffRange : lane16, past ? 0u : b * 1024);
    st.n = ld8s(rs_codes, past ? kOffRange : clane, past ? 0u : code_brick_off(b, 8, codes_ilv));
  };
  auto fetch_table = [&](GStage& st, int i) {
    const uint2 m = ms[wave + WAVES * min(i, nmine - 1)];
    st.map = __builtin_amdgcn_readfirstlane(m.x);
    st.before = __builtin_amdgcn_readfirstlane(m.y);
  };
  GStage st[R];
#pragma unroll
  for (int j = 0; j < D; ++j) fetch_loads(st[j], j);
  if (threadIdx.x < 2) ((u32x4*)gemv_lds)[threadIdx.x] = u32x4{0u, 0u, 0u, 0u};
  {
    const int n16 = (int)(xbytes / 16);
    for (int c = wave; c * 64 < n16; c += WAVES) {
      const int i = c * 64 + lane;
      lds_dma16_g(rs_x, lx + c * 1024, i < n16 ? i * 16 : kOffRange);
    }
    const int nm4 = kbn * 2;
    for (int c = wave; c * 64 < nm4; c += WAVES) {
      const int i = c * 64 + lane;
      lds_dma4_g(rs_meta, lm + c * 256, i < nm4 ? i * 4 : kOffRange);
    }
  }
  uint32_t raw0 = 0;  // the brick-row's raw groups: raw0 .. raw0 + nraw - 1
  if (SIDE_LDS) {
    raw0 = __builtin_amdgcn_readfirstlane(m_first.y);
    const uint32_t nraw = __builtin_amdgcn_readfirstlane(m_last.y) +
                          __builtin_popcount(__builtin_amdgcn_readfirstlane(m_last.x)) - raw0;
    const int ns16 = (int)min(nraw, (uint32_t)side_cap) * 4;
    for (int c = wave; c * 64 < ns16; c += WAVES) {
      const int i = c * 64 + lane;
      lds_dma16_g(rs_side, sl + c * 1024, i < ns16 ? raw0 * 64 + i * 16 : kOffRange);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < D; ++j) fetch_table(st[j], j);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const GStage& st, int i) {
    const int kb = wave + WAVES * i;
    const u32x4* p = (const u32x4*)(gemv_lds + xl_lane + kb * xl_step);
    const u32x4 xb0 = p[0], xb1 = p[1];
    uint32_t v[4];
    palette_v(st.n, lut, v);
    if (st.map) {  // wave-uniform: the brick holds a raw group
      if ((st.map >> r) & 1u) {
        const uint32_t g = st.before + __builtin_popcount(st.map & ((1u << r) - 1u));  // this row's raw group
        u32x4 e;
        if constexpr (SIDE_LDS) {
          e = *(const u32x4*)(sl + (g - raw0) * 64 + q * 16);
        } else {
          e = ld16(rs_side, g * 64 + q * 16, 0);
        }
        v[0] = rot_exp(e.x);
        v[1] = rot_exp(e.y);
        v[2] = rot_exp(e.z);
        v[3] = rot_exp(e.w);
      }
    }
    u32x4 w0, w1;
    rebuild_v2(st.s, v, w0, w1);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w0), as_bf16x8(xb0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w1), as_bf16x8(xb1), acc, 0, 0, 0);
  };
  // brick i sits in stage i % R; brick i + D is requested before brick i is computed
  int i = 0;
  for (; i + R <= nmine; i += R) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      fetch_loads(st[(j + D) % R], i + j + D);
      fetch_table(st[(j + D) % R], i + j + D);
      compute(st[j], i + j);
    }
  }
#pragma unroll
  for (int j = 0; j < R - 1; ++j)
    if (i + j < nmine) compute(st[j], i + j);

  // partial sums of all waves; each output summed by one thread, waves in order
  __shared__ float red[WAVES][256];
  *(f32x4*)&red[wave][lane * 4] = acc;
  __syncthreads();
  for (int k = threadIdx.x; k < 256; k += WAVES * 64) {
    const int l = k >> 2, j = k & 3;
    const int tok = l & 15;  // D layout: lane l holds rows 4*(l/16)+0..3 of column (token) l%16
    if (tok >= tokens) continue;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[w][k];
    y[(size_t)tok * rows + (size_t)brow * 16 + 4 * (l >> 4) + j] = sum;
  }
}

template <int WAVES, int D, bool SIDE_LDS>
__global__ __launch_bounds__(WAVES * 64) void fused_gemv_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    uint64_t codes_bytes, int codes_ilv, int side_cap) {
  gemv_brick_row<WAVES, D, SIDE_LDS>(sm, codes, meta, side, side_bytes, lut0, lut1, lut2, lut3, x, y, tokens, rows,
                                     cols, codes_bytes, codes_ilv, side_cap, blockIdx.x);
}

// Several matrices of one shape in one launch (the active experts of a
// mixture-of-experts projection, each with its own rows of X and Y):
// workgroup g takes brick-row g % (rows / 16) of job g / (rows / 16).  The
// job table travels in the kernel arguments.
template <int WAVES, int D, bool SIDE_LDS>
__global__ __launch_bounds__(WAVES * 64) void fused_gemv_group_kernel(FusedGroup g, int rows, int cols, int side_cap) {
  const uint32_t brows = (uint32_t)rows >> 4;
  const uint32_t e = blockIdx.x / brows, brow = blockIdx.x - e * brows;
  const FusedJob& j = g.job[e];
  gemv_brick_row<WAVES, D, SIDE_LDS>(j.sm, j.codes, j.meta, j.side, j.side_bytes, j.lut[0], j.lut[1], j.lut[2],
                                     j.lut[3], j.x, j.y, j.tokens, rows, cols, j.codes_bytes, j.codes_ilv, side_cap, brow);
}

template <int WAVES, int D>
hipError_t launch_gemv(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, hipStream_t s) {
  const bool side_lds = w.max_row_raw <= (uint32_t)kGemvSideCap;
  const uint32_t cap = side_lds ? w.max_row_raw : 0u;
  const size_t lds = kGemvX0 + gemv_xpad((uint32_t)(tokens * w.cols * 2)) + gemv_mpad((uint32_t)(w.cols / 64)) +
                     (side_lds ? gemv_spad(cap) : 0u);
  if (side_lds)
    hipLaunchKernelGGL((fused_gemv_kernel<WAVES, D, true>), dim3((unsigned)(w.rows / 16)), dim3(WAVES * 64), lds, s,
                       w.sm, w.codes, w.meta, w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y,
                       (int)tokens, (int)w.rows, (int)w.cols, w.codes_bytes, (int)w.codes_ilv, (int)cap);
  else
    hipLaunchKernelGGL((fused_gemv_kernel<WAVES, D, false>), dim3((unsigned)(w.rows / 16)), dim3(WAVES * 64), lds, s,
                       w.sm, w.codes, w.meta, w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y,
                       (int)tokens, (int)w.rows, (int)w.cols, w.codes_bytes, (int)w.codes_ilv, 0);
  return hipGetLastError();
}

template <int WAVES, int D>
hipError_t launch_gemv_group(const FusedGroup& g, int n, int64_t rows, int64_t cols, int64_t max_tokens,
                             uint32_t max_row_raw, hipStream_t s) {
  const bool side_lds = max_row_raw <= (uint32_t)kGemvSideCap;
  const uint32_t cap = side_lds ? max_row_raw : 0u;
  const size_t lds = kGemvX0 + gemv_xpad((uint32_t)(max_tokens * cols * 2)) + gemv_mpad((uint32_t)(cols / 64)) +
                     (side_lds ? gemv_spad(cap) : 0u);
  const dim3 grid((unsigned)(n * (rows / 16)));
  if (side_lds)
    hipLaunchKernelGGL((fused_gemv_group_kernel<WAVES, D, true>), grid, dim3(WAVES * 64), lds, s, g, (int)rows,
                       (int)cols, (int)cap);
  else
    hipLaunchKernelGGL((fused_gemv_group_kernel<WAVES, D, false>), grid, dim3(WAVES * 64), lds, s, g, (int)rows,
                       (int)cols, 0);
  return hipGetLastError();
}

template <int WAVES, int TB, bool EXPM, int U>
hipError_t launch_one(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int ksplit, hipStream_t s) {
  dim3 grid((unsigned)(w.rows / 16), (unsigned)ksplit);
  hipLaunchKernelGGL((fused_small_kernel<WAVES, TB, EXPM, U>), grid, dim3(WAVES * 64), 0, s, w.sm, w.codes,
                     w.meta, w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens,
                     (int)w.rows, (int)w.cols, ksplit, w.codes_bytes, (int)w.codes_ilv);
  return hipGetLastError();
}

template <int WAVES, int TB, int U>
hipError_t launch_mode(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int ksplit, hipStream_t s) {
  return w.exp_mode ? launch_one<WAVES, TB, true, U>(w, x, y, tokens, ksplit, s)
                    : launch_one<WAVES, TB, false, U>(w, x, y, tokens, ksplit, s);
}

template <int WAVES, int U>
hipError_t launch_tb(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int ksplit, hipStream_t s) {
  switch ((tokens + 15) / 16) {
    case 1: return launch_mode<WAVES, 1, U>(w, x, y, tokens, ksplit, s);
    case 2: return launch_mode<WAVES, 2, U>(w, x, y, tokens, ksplit, s);
    case 3: return launch_mode<WAVES, 3, U>(w, x, y, tokens, ksplit, s);
    default: return launch_mode<WAVES, 4, U>(w, x, y, tokens, ksplit, s);
  }
}

}  // namespace

hipError_t launch_fused_gemv(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                             hipStream_t s) {
  if (w.exp_mode || tokens < 1 || tokens > 16 || tokens * w.cols > kGemvX || w.cols / 64 > kGemvKbn)
    return hipErrorInvalidValue;
#define UW_CASE(W, D) \
  if (v.waves == W && v.unroll == D) return launch_gemv<W, D>(w, x, y, tokens, s);
  UW_CASE(8, 2) UW_CASE(8, 1) UW_CASE(4, 2) UW_CASE(16, 2) UW_CASE(8, 3) UW_CASE(4, 3)
#undef UW_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fused_gemv_group(const FusedW* ws, const uint16_t* const* xs, float* const* ys,
                                   const int64_t* tokens, int n, const Variant& v, hipStream_t s) {
  if (n < 1 || n > kFusedGroupMax) return hipErrorInvalidValue;
  const int64_t rows = ws[0].rows, cols = ws[0].cols;
  if (rows < 16 || rows % 16 || (rows / 16) * n > 0x7FFFFFFF) return hipErrorInvalidValue;
  FusedGroup g = {};
  int64_t max_tokens = 0;
  uint32_t max_raw = 0;
  for (int e = 0; e < n; ++e) {
    const FusedW& w = ws[e];
    if (w.rows != rows || w.cols != cols || w.exp_mode || tokens[e] < 1 || tokens[e] > 16 ||
        tokens[e] * cols > kGemvX || cols / 64 > kGemvKbn)
      return hipErrorInvalidValue;
    FusedJob& j = g.job[e];
    j.sm = w.sm;
    j.codes = w.codes;
    j.meta = w.meta;
    j.side = w.side;
    j.side_bytes = w.side_bytes;
    j.codes_bytes = w.codes_bytes;
    for (int k = 0; k < 4; ++k) j.lut[k] = w.lut[k];
    j.x = xs[e];
    j.y = ys[e];
    j.tokens = (int32_t)tokens[e];
    j.codes_ilv = w.codes_ilv ? 1 : 0;
    max_tokens = std::max(max_tokens, tokens[e]);
    max_raw = std::max(max_raw, w.max_row_raw);
  }
#define UW_CASE(W, D) \
  if (v.waves == W && v.unroll == D) return launch_gemv_group<W, D>(g, n, rows, cols, max_tokens, max_raw, s);
  UW_CASE(8, 2) UW_CASE(8, 1) UW_CASE(4, 2) UW_CASE(16, 2) UW_CASE(8, 3) UW_CASE(4, 3)
#undef UW_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fused_small(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                              hipStream_t s) {
  if (tokens < 1 || tokens > 64) return hipErrorInvalidValue;
  const int ks = v.ksplit < 1 ? 1 : v.ksplit;
  if (ks > 1) {
    hipError_t e = launch_zero(y, tokens * w.rows, s);
    if (e != hipSuccess) return e;
  }
#define UW_CASE(W, U) \
  if (v.waves == W && v.unroll == U) return launch_tb<W, U>(w, x, y, tokens, ks, s);
  UW_CASE(4, 1) UW_CASE(4, 2) UW_CASE(4, 4)
  UW_CASE(8, 1) UW_CASE(8, 2) UW_CASE(8, 4)
  UW_CASE(16, 1) UW_CASE(16, 2)
#undef UW_CASE
  return hipErrorInvalidValue;
}

}  // namespace uw
