// Fused reconstruct-GEMM for a few dozen tokens without a K split (gfx950).
//
// Unweight page, sections 六 and 七: the weights are rebuilt from their
// stored bytes in registers, used as the matrix operand and never written
// back.  The K-slice kernel (fused_mid.hip) splits K across workgroups and
// adds the slices into Y with float atomics; at 48-64 tokens those atomics
// (one per output element and slice, coalesced) cost about as much as the
// whole weight stream.  Here a workgroup owns R brick-rows over the whole of
// K, so each output is written once:
//  * P waves share a brick-row, wave p taking bricks p, p+P, p+2P, ... (the
//    GEMV kernel's interleave) through a ring of D register stages (D a
//    multiple of U, so a stage's index is fixed within an unrolled step);
//  * the activations stream through LDS in slices of S = P*U bricks, double
//    buffered: the loads of slice j+1 are issued before the MFMAs of slice j
//    and stored after them, and one barrier per slice publishes them;
//  * at the end the P partial sums of a brick-row are added in LDS and Y is
//    written in runs of R*16 consecutive rows.
// Each workgroup reads the activations once from L2 (tokens x cols x 2
// bytes), so R trades that traffic against the number of workgroups.  Short
// matrices (few brick-rows, long K) would leave CUs idle: there the grid also
// splits K into a few ranges of whole slices that add into Y atomically --
// a handful of additions per output instead of one per LDS-sized slice.
#include <algorithm>

#include "kernels.h"
#include "recon.h"

namespace uw {
namespace {

struct KStage {
  u32x4 s;       // sign+mantissa bytes
  u32x4 e;       // exponent form: exponent bytes; palette form: raw side-table bytes (zeros off raw rows)
  u32x2 n;       // palette form: 4-bit codes
  uint32_t map;  // palette form: wave-uniform raw-row map of the brick
};

constexpr size_t kRowkLdsBytes = 160 * 1024;  // one workgroup may take a whole CU's LDS

// Row group rg (brick-rows rg*R ..) of one matrix: the body of the kernels.
template <int R, int P, int U, int D, int TB, bool EXPM>
__device__ __forceinline__ void rowk_row_group(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    int kper, int ksplit, uint64_t codes_bytes, int codes_ilv, int rg) {
  constexpr int WAVES = R * P, NT = WAVES * 64, S = P * U;
  static_assert(D % U == 0, "ring stages must repeat every D / U slices");
  constexpr int SL = D / U;  // slices per unrolled loop step
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rw = wave / P, p = wave - rw * P;
  const int r = lane & 15, q = lane >> 4;
  const int kbn = cols >> 6, brows = rows >> 4;
  // K range of the workgroup (the whole of K unless the grid splits it):
  // bricks [kb0, kb0 + nkb), a multiple of S long except the last
  const int kb0 = blockIdx.y * kper, nkb = min(kper, kbn - kb0);
  const int brow = rg * R + rw;
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

  // LDS: two activation buffers, token t at row t of xrow bytes (16 more
  // than the slice, so consecutive tokens start 4 banks apart), 32 zero bytes
  // read by lanes of absent tokens, then the per-brick tables of the R
  // brick-rows.  The epilogue reuses the buffers.
  extern __shared__ __attribute__((aligned(16))) uint8_t rowk_lds[];
  constexpr uint32_t xrow = S * 128 + 16;
  const uint32_t xbuf = (uint32_t)tokens * xrow;
  const uint32_t zoff = 2 * xbuf;
  uint2* ms = (uint2*)(rowk_lds + zoff + 32);
  uint32_t xl[TB], xm[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = tb * 16 + r;
    xl[tb] = t < tokens ? (uint32_t)t * xrow + q * 32 : zoff;
    xm[tb] = t < tokens ? 1u : 0u;
  }

  const int nmine = max(0, (nkb - p + P - 1) / P);  // bricks kb0 + p + P*i of this wave (may be 0)
  const uint32_t brick0 = (uint32_t)brow * kbn + kb0;
  auto fetch = [&](KStage& st, int i, bool table_in_lds) {
    // past the end (or for a wave without bricks): re-read a valid brick, never used
    const int kb = min(p + P * max(0, min(i, nmine - 1)), nkb - 1);
    const uint32_t b = brick0 + kb;
    st.s = ld16s(rs_sm, has_row ? lane16 : kOffRange, b * 1024);
    if (EXPM) {
      st.e = ld16s(rs_codes, has_row ? clane : kOffRange, code_brick_off(b, 16, codes_ilv));
    } else {
      const uint2 m = has_row ? (table_in_lds ? ms[rw * kper + kb] : meta[b]) : uint2{0u, 0u};
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
  // brick at position lb of the slice held in buffer buf
  auto compute = [&](const KStage& st, uint32_t buf, int lb) {
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
    const uint32_t off = buf * xbuf + (uint32_t)lb * 128;
    // B fragments read LA token blocks ahead of their MFMAs (left to itself
    // the compiler reuses one register pair and waits on every read)
    constexpr int LA = TB < 3 ? TB : 2;
    u32x4 bq[LA + 1][2];
    auto read_b = [&](u32x4 (&d)[2], int tb) {
      const u32x4* px = (const u32x4*)(rowk_lds + xl[tb] + xm[tb] * off);
      d[0] = px[0];
      d[1] = px[1];
    };
#pragma unroll
    for (int tb = 0; tb < LA; ++tb) read_b(bq[tb], tb);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      if (tb + LA < TB) read_b(bq[(tb + LA) % (LA + 1)], tb + LA);
      const u32x4(&bc)[2] = bq[tb % (LA + 1)];
      acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w0), as_bf16x8(bc[0]), acc[tb], 0, 0, 0);
      acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w1), as_bf16x8(bc[1]), acc[tb], 0, 0, 0);
    }
    // keep that order: the first LA blocks' reads, then per block two MFMAs
    // and the reads of the block LA ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (tb + LA < TB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };
  // activations of slice j: 16-byte pieces, S*8 per token
  constexpr int PER_TOK = S * 8;
  constexpr int NXV = (TB * 16 * PER_TOK + NT - 1) / NT;
  const int pieces = tokens * PER_TOK;
  u32x4 xv[NXV];
  auto issue_x = [&](int j) {
#pragma unroll
    for (int k = 0; k < NXV; ++k) {
      const int idx = threadIdx.x + k * NT;
      const int t = idx / PER_TOK, rem = idx - t * PER_TOK;
      const int col = (kb0 + j * S) * 64 + rem * 8;
      xv[k] = ld16(rs_x, idx < pieces && col < cols ? ((uint32_t)t * cols + col) * 2 : kOffRange, 0);
    }
  };
  auto store_x = [&](uint32_t buf) {
#pragma unroll
    for (int k = 0; k < NXV; ++k) {
      const int idx = threadIdx.x + k * NT;
      if (idx < pieces) {
        const int t = idx / PER_TOK, rem = idx - t * PER_TOK;
        *(u32x4*)(rowk_lds + buf * xbuf + (uint32_t)t * xrow + rem * 16) = xv[k];
      }
    }
  };

  const int nslices = (nkb + S - 1) / S;
  KStage st[D];
#pragma unroll
  for (int j = 0; j < D; ++j) fetch(st[j], j, false);  // the first stages read the table from global memory
  issue_x(0);
  if (!EXPM) {
    for (int i = threadIdx.x; i < R * kper; i += NT) {
      const int br = rg * R + i / kper, kk = i % kper;
      ms[i] = br < brows && kk < nkb ? meta[(size_t)br * kbn + kb0 + kk] : uint2{0u, 0u};
    }
  }
  if (threadIdx.x < 2) ((u32x4*)(rowk_lds + zoff))[threadIdx.x] = u32x4{0u, 0u, 0u, 0u};
  store_x(0);
  __syncthreads();

  for (int j0 = 0; j0 < nslices; j0 += SL) {
#pragma unroll
    for (int jj = 0; jj < SL; ++jj) {
      const int j = j0 + jj;
      if (j < nslices) {  // workgroup-uniform
        if (j + 1 < nslices) issue_x(j + 1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = j * U + u;
          const int s = (jj * U + u) % D;
          if (i < nmine) compute(st[s], (uint32_t)(j & 1), p + P * u);
          fetch(st[s], i + D, true);
        }
        if (j + 1 < nslices) store_x((uint32_t)((j + 1) & 1));
        __syncthreads();
      }
    }
  }

  // Epilogue: waves 1..P-1 of a brick-row hand their partial sums to wave 0
  // through LDS (lane-major, no bank conflicts), wave 0 adds them and puts
  // the brick-row's tile into an output tile [token][R*16 rows] (rows padded
  // by 4), and Y is written from that in runs of R*16 consecutive rows.
  constexpr int WR = R * 16, OROW = WR + 4;
  f32x4* red = (f32x4*)rowk_lds;  // [rw][p-1][tb][lane]
  float* out = (float*)(rowk_lds + (size_t)R * (P - 1) * TB * 64 * 16);
  if (p > 0) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) red[((rw * (P - 1) + p - 1) * TB + tb) * 64 + lane] = acc[tb];
  }
  __syncthreads();
  if (p == 0) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      f32x4 sum = acc[tb];
#pragma unroll
      for (int pp = 1; pp < P; ++pp) sum += red[((rw * (P - 1) + pp - 1) * TB + tb) * 64 + lane];
      // D layout: lane l holds rows 4*(l/16)+0..3 of column (token) l%16
      *(f32x4*)&out[(tb * 16 + r) * OROW + rw * 16 + 4 * q] = sum;
    }
  }
  __syncthreads();
  const int row0 = rg * WR;
  const int nrow = min(WR, rows - row0);
  for (int e = threadIdx.x; e < tokens * WR; e += NT) {
    const int tok = e / WR, rr = e - tok * WR;
    if (rr >= nrow) continue;
    const float v = out[tok * OROW + rr];
    if (ksplit == 1)
      y[(size_t)tok * rows + row0 + rr] = v;
    else
      unsafeAtomicAdd(y + (size_t)tok * rows + row0 + rr, v);
  }
}

template <int R, int P, int U, int D, int TB, bool EXPM>
__global__ __launch_bounds__(R * P * 64) void fused_rowk_kernel(
    const uint8_t* __restrict__ sm, const uint8_t* __restrict__ codes, const uint2* __restrict__ meta,
    const uint8_t* __restrict__ side, uint64_t side_bytes, uint32_t lut0, uint32_t lut1, uint32_t lut2,
    uint32_t lut3, const uint16_t* __restrict__ x, float* __restrict__ y, int tokens, int rows, int cols,
    int kper, int ksplit, uint64_t codes_bytes, int codes_ilv) {
  rowk_row_group<R, P, U, D, TB, EXPM>(sm, codes, meta, side, side_bytes, lut0, lut1, lut2, lut3, x, y, tokens, rows,
                                       cols, kper, ksplit, codes_bytes, codes_ilv, blockIdx.x);
}

// Several matrices of one shape and token count in one launch (gate and up
// of a layer): workgroup (g, k) takes row group g % ngroups of job
// g / ngroups, K range k.  The job table travels in the kernel arguments.
template <int R, int P, int U, int D, int TB>
__global__ __launch_bounds__(R * P * 64) void fused_rowk_group_kernel(FusedGroup g, int tokens, int rows, int cols,
                                                                      int kper, int ksplit, int ngroups) {
  const int e = blockIdx.x / ngroups, rg = blockIdx.x - e * ngroups;
  const FusedJob& j = g.job[e];
  rowk_row_group<R, P, U, D, TB, false>(j.sm, j.codes, j.meta, j.side, j.side_bytes, j.lut[0], j.lut[1], j.lut[2],
                                        j.lut[3], j.x, j.y, tokens, rows, cols, kper, ksplit, j.codes_bytes,
                                        j.codes_ilv, rg);
}

template <int R, int P, int U, int D, int TB>
hipError_t launch_rowk_group_t(const FusedGroup& g, int n, int64_t tokens, int64_t rows, int64_t cols, int kper,
                               int ksplit, size_t lds, hipStream_t s) {
  const int ngroups = (int)((rows / 16 + R - 1) / R);
  const dim3 grid((unsigned)(n * ngroups), (unsigned)ksplit);
  hipLaunchKernelGGL((fused_rowk_group_kernel<R, P, U, D, TB>), grid, dim3(R * P * 64), lds, s, g, (int)tokens,
                     (int)rows, (int)cols, kper, ksplit, ngroups);
  return hipGetLastError();
}

template <int R, int P, int U, int D, int TB>
hipError_t launch_rowk_t(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int kper, int ksplit,
                         size_t lds, hipStream_t s) {
  const dim3 grid((unsigned)((w.rows / 16 + R - 1) / R), (unsigned)ksplit);
#define UW_LAUNCH(E)                                                                                             \
  hipLaunchKernelGGL((fused_rowk_kernel<R, P, U, D, TB, E>), grid, dim3(R * P * 64), lds, s, w.sm, w.codes, w.meta, \
                     w.side, w.side_bytes, w.lut[0], w.lut[1], w.lut[2], w.lut[3], x, y, (int)tokens,            \
                     (int)w.rows, (int)w.cols, kper, ksplit, w.codes_bytes, (int)w.codes_ilv)
  if (w.exp_mode)
    UW_LAUNCH(true);
  else
    UW_LAUNCH(false);
#undef UW_LAUNCH
  return hipGetLastError();
}

template <int R, int P, int U, int D>
hipError_t launch_rowk_c(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, int kper, int ksplit,
                         size_t lds, hipStream_t s) {
  if (tokens > 64) return hipErrorInvalidValue;
  switch ((tokens + 15) / 16) {
    case 1: return launch_rowk_t<R, P, U, D, 1>(w, x, y, tokens, kper, ksplit, lds, s);
    case 2: return launch_rowk_t<R, P, U, D, 2>(w, x, y, tokens, kper, ksplit, lds, s);
    case 3: return launch_rowk_t<R, P, U, D, 3>(w, x, y, tokens, kper, ksplit, lds, s);
    default: return launch_rowk_t<R, P, U, D, 4>(w, x, y, tokens, kper, ksplit, lds, s);
  }
}

}  // namespace

// token blocks of 16 the kernel is instantiated with for `tokens`
int rowk_tb(int64_t tokens) {
  return tokens <= 64 ? (int)((tokens + 15) / 16) : tokens <= 96 ? 6 : tokens <= 128 ? 8 : tokens <= 192 ? 12 : 16;
}

size_t rowk_lds_bytes(int64_t tokens, int kper, int r, int p, int u) {
  const size_t xrow = (size_t)p * u * 128 + 16;
  const size_t in = 2 * (size_t)tokens * xrow + 32 + (size_t)r * kper * 8;
  // epilogue: the partial sums of waves 1..P-1 and the output tile
  const size_t red = (size_t)r * (p - 1) * rowk_tb(tokens) * 64 * 16 + (size_t)rowk_tb(tokens) * 16 * (r * 16 + 4) * 4;
  return std::max(in, red);
}

size_t rowk_plan(int64_t tokens, int64_t rows, int64_t cols, const Variant& v, int* kper_out, int* ks_out) {
  const int R = v.tile, P = v.waves, U = v.ksplit, S = P * U;
  // Split K only when the workgroups (one per R brick-rows) would leave most
  // CUs idle: into ranges of whole slices, at least two slices long, and no
  // more workgroups than CUs (one per CU when the slices are large); the
  // ranges then add into a zeroed Y.
  const int kbn = (int)(cols / 64);
  const int64_t groups = (rows / 16 + R - 1) / R;
  int ks = 1;
  if (groups <= 128) ks = (int)std::max<int64_t>(1, std::min<int64_t>(256 / groups, kbn / (2 * S)));
  const int kper = ((kbn + ks - 1) / ks + S - 1) / S * S;
  ks = (kbn + kper - 1) / kper;
  if (kper_out) *kper_out = kper;
  if (ks_out) *ks_out = ks;
  return rowk_lds_bytes(tokens, kper, R, P, U);
}

// shapes built for 65..128 tokens: {R, P, U, D}
bool big_shape(const Variant& v) {
  const int R = v.tile, P = v.waves, U = v.ksplit, D = v.unroll;
  return (R == 4 && P == 4 && U == 1 && D == 2) || (R == 4 && P == 2 && U == 2 && D == 2);
}

// shape built for 129..256 tokens: 2-brick slices, whose activations still
// fit LDS twice
bool huge_shape(const Variant& v) { return v.tile == 4 && v.waves == 2 && v.ksplit == 1 && v.unroll == 2; }

bool rowk_fits(int64_t tokens, int64_t rows, int64_t cols, const Variant& v) {
  if (tokens < 1 || tokens > 256) return false;
  if (tokens > 128 && !huge_shape(v)) return false;
  // above 64 tokens only the R4 P4 U1 and R4 P2 U2 shapes are built
  if (tokens > 64 && tokens <= 128 && !big_shape(v)) return false;
  return rowk_plan(tokens, rows, cols, v, nullptr, nullptr) <= kRowkLdsBytes;
}

hipError_t launch_fused_rowk_group(const FusedW* ws, const uint16_t* const* xs, float* const* ys, int n,
                                   int64_t tokens, const Variant& v, hipStream_t s) {
  if (n < 1 || n > kFusedGroupMax || tokens < 1 || tokens > 64) return hipErrorInvalidValue;
  const int64_t rows = ws[0].rows, cols = ws[0].cols;
  if (!rowk_fits(tokens, rows, cols, v)) return hipErrorInvalidValue;
  const int R = v.tile, P = v.waves, U = v.ksplit, D = v.unroll;
  int kper = 0, ks = 0;
  const size_t lds = rowk_plan(tokens, rows, cols, v, &kper, &ks);
  if (lds > kRowkLdsBytes || (int64_t)n * ((rows / 16 + R - 1) / R) > 0x7FFFFFFF) return hipErrorInvalidValue;
  FusedGroup g = {};
  for (int e = 0; e < n; ++e) {
    const FusedW& w = ws[e];
    if (w.rows != rows || w.cols != cols || w.exp_mode) return hipErrorInvalidValue;
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
    j.tokens = (int32_t)tokens;
    j.codes_ilv = w.codes_ilv ? 1 : 0;
  }
  if (ks > 1) {
    for (int e = 0; e < n; ++e) {
      hipError_t err = launch_zero(ys[e], tokens * rows, s);
      if (err != hipSuccess) return err;
    }
  }
#define UW_CASE(RR, PP, UU, DD)                                                                          \
  if (R == RR && P == PP && U == UU && D == DD) {                                                        \
    switch ((tokens + 15) / 16) {                                                                        \
      case 1: return launch_rowk_group_t<RR, PP, UU, DD, 1>(g, n, tokens, rows, cols, kper, ks, lds, s); \
      case 2: return launch_rowk_group_t<RR, PP, UU, DD, 2>(g, n, tokens, rows, cols, kper, ks, lds, s); \
      case 3: return launch_rowk_group_t<RR, PP, UU, DD, 3>(g, n, tokens, rows, cols, kper, ks, lds, s); \
      default: return launch_rowk_group_t<RR, PP, UU, DD, 4>(g, n, tokens, rows, cols, kper, ks, lds, s); \
    }                                                                                                    \
  }
  UW_CASE(4, 4, 2, 2) UW_CASE(4, 2, 2, 2)
#undef UW_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fused_rowk(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                             hipStream_t s) {
  if (!rowk_fits(tokens, w.rows, w.cols, v)) return hipErrorInvalidValue;
  const int R = v.tile, P = v.waves, U = v.ksplit, D = v.unroll;
  int kper = 0, ks = 0;
  const size_t lds = rowk_plan(tokens, w.rows, w.cols, v, &kper, &ks);
  if (lds > kRowkLdsBytes) return hipErrorInvalidValue;
  if (ks > 1) {
    hipError_t e = launch_zero(y, tokens * w.rows, s);
    if (e != hipSuccess) return e;
  }
  if (tokens > 128) {  // 129..256 tokens: 12 or 16 token blocks
    if (tokens <= 192) return launch_rowk_t<4, 2, 1, 2, 12>(w, x, y, tokens, kper, ks, lds, s);
    return launch_rowk_t<4, 2, 1, 2, 16>(w, x, y, tokens, kper, ks, lds, s);
  }
  if (tokens > 64) {  // 65..128 tokens: 6 or 8 token blocks
#define UW_BIG(RR, PP, UU, DD)                                                             \
  if (R == RR && P == PP && U == UU && D == DD) {                                          \
    if (tokens <= 96) return launch_rowk_t<RR, PP, UU, DD, 6>(w, x, y, tokens, kper, ks, lds, s); \
    return launch_rowk_t<RR, PP, UU, DD, 8>(w, x, y, tokens, kper, ks, lds, s);            \
  }
    UW_BIG(4, 4, 1, 2) UW_BIG(4, 2, 2, 2)
#undef UW_BIG
    return hipErrorInvalidValue;
  }
#define UW_CASE(RR, PP, UU, DD) \
  if (R == RR && P == PP && U == UU && D == DD)  \
    return launch_rowk_c<RR, PP, UU, DD>(w, x, y, tokens, kper, ks, lds, s);
  UW_CASE(2, 4, 1, 2) UW_CASE(4, 4, 1, 2) UW_CASE(4, 4, 2, 2) UW_CASE(4, 4, 2, 4) UW_CASE(4, 2, 2, 2)
  UW_CASE(4, 2, 4, 4) UW_CASE(2, 4, 2, 2) UW_CASE(1, 8, 1, 2) UW_CASE(2, 8, 1, 2)
#undef UW_CASE
  return hipErrorInvalidValue;
}

}  // namespace uw
