// Fused-kernel variants: the kernel shapes the autotuner chooses from
// (Unweight page, section 九: pipeline x kernel variant x decode/compute split).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>

#include "kernels.h"

namespace uw {

hipError_t launch_fused_small(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                              hipStream_t s);
hipError_t launch_fused_large(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                              hipStream_t s);
hipError_t launch_fused_gemv(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                             hipStream_t s);
hipError_t launch_fused_mid(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                            hipStream_t s);
hipError_t launch_fused_rowk(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                             hipStream_t s);

namespace {

struct Named {
  Variant v;
  const char* name;
};

// small batch: kind 0, {waves, ksplit, unroll}; kind 2, {waves, -, ring depth}
const Named kSmall[] = {
    {{0, 8, 1, 2, 0}, "small:w8:k1:u2"},  {{0, 4, 1, 2, 0}, "small:w4:k1:u2"},
    {{0, 16, 1, 1, 0}, "small:w16:k1:u1"}, {{0, 8, 1, 4, 0}, "small:w8:k1:u4"},
    {{0, 4, 1, 4, 0}, "small:w4:k1:u4"},  {{0, 8, 2, 2, 0}, "small:w8:k2:u2"},
    {{0, 8, 4, 2, 0}, "small:w8:k4:u2"},  {{0, 4, 2, 2, 0}, "small:w4:k2:u2"},
    {{0, 16, 1, 2, 0}, "small:w16:k1:u2"}, {{0, 4, 4, 2, 0}, "small:w4:k4:u2"},
    {{0, 8, 1, 1, 0}, "small:w8:k1:u1"},  {{0, 4, 4, 4, 0}, "small:w4:k4:u4"},
    // x held in LDS (palette forms, tokens x cols <= 16384); {waves, ring depth}
    {{2, 8, 1, 2, 0}, "gemv:w8:d2"},      {{2, 16, 1, 2, 0}, "gemv:w16:d2"},
    {{2, 8, 1, 3, 0}, "gemv:w8:d3"},      {{2, 4, 1, 3, 0}, "gemv:w4:d3"},
    {{2, 8, 1, 1, 0}, "gemv:w8:d1"},      {{2, 4, 1, 2, 0}, "gemv:w4:d2"},
    // a K slice of x in LDS shared by `waves` brick-rows; {waves, ring depth}
    {{3, 16, 1, 2, 0}, "mid:w16:d2"},     {{3, 8, 1, 2, 0}, "mid:w8:d2"},
    {{3, 16, 1, 3, 0}, "mid:w16:d3"},     {{3, 4, 1, 2, 0}, "mid:w4:d2"},
    // whole K per workgroup (no split): R brick-rows x P waves each, slices of
    // P*U bricks of x double-buffered in LDS; {P, U, ring depth D, R}
    {{4, 4, 2, 2, 4}, "rowk:r4p4u2d2"},   {{4, 4, 2, 4, 4}, "rowk:r4p4u2d4"},
    {{4, 4, 1, 2, 4}, "rowk:r4p4u1d2"},   {{4, 2, 2, 2, 4}, "rowk:r4p2u2d2"},
    {{4, 2, 4, 4, 4}, "rowk:r4p2u4d4"},   {{4, 4, 2, 2, 2}, "rowk:r2p4u2d2"},
    {{4, 4, 1, 2, 2}, "rowk:r2p4u1d2"},   {{4, 8, 1, 2, 1}, "rowk:r1p8u1d2"},
    {{4, 8, 1, 2, 2}, "rowk:r2p8u1d2"},
};
// large batch: kind 1, {tile, ksplit}
const Named kLarge[] = {
    {{1, 0, 1, 0, 0}, "large:t0(4x64r x128t):k1"}, {{1, 0, 2, 0, 0}, "large:t0(4x64r x128t):k2"},
    {{1, 0, 4, 0, 0}, "large:t0(4x64r x128t):k4"}, {{1, 0, 8, 0, 0}, "large:t0(4x64r x128t):k8"},
    {{1, 0, 16, 0, 0}, "large:t0(4x64r x128t):k16"}, {{1, 0, 1, 0, 1}, "large:t1(4x32r x128t):k1"},
    {{1, 0, 2, 0, 1}, "large:t1(4x32r x128t):k2"}, {{1, 0, 1, 0, 2}, "large:t2(2x64r x128t):k1"},
    {{1, 0, 2, 0, 2}, "large:t2(2x64r x128t):k2"}, {{1, 0, 1, 0, 3}, "large:t3(4x64r x64t):k1"},
    {{1, 0, 2, 0, 3}, "large:t3(4x64r x64t):k2"},
    // 32x32x16 instructions
    {{1, 0, 1, 0, 4}, "large:t4(4x64r x128t,32x32):k1"}, {{1, 0, 2, 0, 4}, "large:t4(4x64r x128t,32x32):k2"},
    {{1, 0, 4, 0, 4}, "large:t4(4x64r x128t,32x32):k4"}, {{1, 0, 1, 0, 5}, "large:t5(4x32r x128t,32x32):k1"},
    {{1, 0, 2, 0, 5}, "large:t5(4x32r x128t,32x32):k2"}, {{1, 0, 1, 0, 6}, "large:t6(2x64r x128t,32x32):k1"},
    {{1, 0, 1, 0, 7}, "large:t7(4x64r x64t,32x32):k1"},  {{1, 0, 2, 0, 7}, "large:t7(4x64r x64t,32x32):k2"},
    {{1, 0, 1, 0, 8}, "large:t8(4x64r x256t,32x32):k1"}, {{1, 0, 2, 0, 8}, "large:t8(4x64r x256t,32x32):k2"},
    {{1, 0, 1, 0, 9}, "large:t9(4x32r x256t,32x32):k1"}, {{1, 0, 2, 0, 9}, "large:t9(4x32r x256t,32x32):k2"},
    {{1, 0, 1, 0, 10}, "large:t10(4x64r x256t,32x32,interleaved):k1"},
    {{1, 0, 2, 0, 10}, "large:t10(4x64r x256t,32x32,interleaved):k2"},
    {{1, 0, 1, 0, 11}, "large:t11(4x64r x256t,32x32,interleaved,B groups):k1"},
    {{1, 0, 2, 0, 11}, "large:t11(4x64r x256t,32x32,interleaved,B groups):k2"},
    // weights requested D steps ahead into registers, activations X-1 steps ahead straight to LDS
    {{1, 0, 1, 0, 12}, "large:t12(4x32r x128t,32x32,ring d4 x3)"},
    {{1, 0, 1, 0, 13}, "large:t13(4x32r x64t,32x32,ring d4 x3)"},
    {{1, 0, 1, 0, 14}, "large:t14(4x64r x128t,32x32,ring d2 x3)"},
    {{1, 0, 1, 0, 15}, "large:t15(4x32r x128t,32x32,ring d4 x8)"},
    {{1, 0, 1, 0, 16}, "large:t16(4x32r x64t,32x32,ring d4 x8)"},
    {{1, 0, 1, 0, 17}, "large:t17(4x32r x128t,32x32,ring d6 x6)"},
    {{1, 0, 1, 0, 18}, "large:t18(4x32r x128t,32x32,ring d4 x3 b3)"},
    {{1, 0, 1, 0, 19}, "large:t19(4x32r x64t,32x32,ring d4 x8 b3)"},
    {{1, 0, 1, 0, 20}, "large:t20(4x32r x128t,32x32,ring d4 x8 b4)"},
    {{1, 0, 1, 0, 21}, "large:t21(4x64r x128t,32x32,ring d2 x3 b2)"},
    // 128 rows rebuilt once per 512 tokens into LDS, shared by 4 waves of 128 tokens
    {{1, 0, 1, 0, 22}, "large:t22(128r x 4x128t,32x32,wide)"},
    // whole K per workgroup, 16x16x32 instructions, up to 128 tokens
    {{4, 4, 1, 2, 4}, "rowk:r4p4u1d2"},   {{4, 2, 2, 2, 4}, "rowk:r4p2u2d2"},
    {{4, 2, 1, 2, 4}, "rowk:r4p2u1d2"},   // up to 256 tokens
};
constexpr int kNSmall = sizeof(kSmall) / sizeof(kSmall[0]);
constexpr int kNLarge = sizeof(kLarge) / sizeof(kLarge[0]);

}  // namespace

int variant_count(int64_t tokens) { return 1 + (tokens <= 64 ? kNSmall : kNLarge); }

bool variant_get(int64_t tokens, int id, Variant* v) {
  if (id < 1 || id >= variant_count(tokens)) return false;
  *v = tokens <= 64 ? kSmall[id - 1].v : kLarge[id - 1].v;
  return true;
}

const char* variant_name(int64_t tokens, int id) {
  if (id == 0) return tokens <= 64 ? "small:default" : "large:default";
  if (id < 0 || id >= variant_count(tokens)) return nullptr;
  return tokens <= 64 ? kSmall[id - 1].name : kLarge[id - 1].name;
}

void variant_describe(int64_t tokens, const Variant& v, char* buf, size_t len) {
  if (!buf || len == 0) return;
  const Named* list = tokens <= 64 ? kSmall : kLarge;
  const int n = tokens <= 64 ? kNSmall : kNLarge;
  for (int i = 0; i < n; ++i) {
    const Variant& u = list[i].v;
    if (u.kind == v.kind && u.waves == v.waves && u.ksplit == v.ksplit && u.unroll == v.unroll && u.tile == v.tile) {
      snprintf(buf, len, "%s", list[i].name);
      return;
    }
  }
  if (v.kind == 1)
    snprintf(buf, len, "large:t%d:k%d", v.tile, v.ksplit);
  else if (v.kind == 2)
    snprintf(buf, len, "gemv:w%d:d%d", v.waves, v.unroll);
  else if (v.kind == 3)
    snprintf(buf, len, "mid:w%d:d%d", v.waves, v.unroll);
  else if (v.kind == 4)
    snprintf(buf, len, "rowk:r%dp%du%dd%d", v.tile, v.waves, v.ksplit, v.unroll);
  else
    snprintf(buf, len, "small:w%d:k%d:u%d", v.waves, v.ksplit, v.unroll);
}

// Built-in choice when no plan is set (measured on MI355X with the 8B-shaped
// projections; the autotuner refines it per matrix and batch).
namespace {

Variant small_default(int64_t tokens, int64_t rows, int64_t cols) {
  const int64_t brows = rows / 16, kbn = cols / 64;
  // one 16-row brick-row per workgroup already gives >= 4096 waves for the
  // 4096-row down projection; K is split only for very short matrices
  Variant v{0, tokens <= 16 ? 16 : 8, 1, 1, 0};
  if (brows < 128) v.ksplit = (int)std::min<int64_t>({8, (256 + brows - 1) / brows, kbn});
  return v;
}

}  // namespace

Variant variant_gemv() { return Variant{2, 8, 1, 2, 0}; }

Variant variant_default(int64_t tokens, int64_t rows, int64_t cols) {
  const int64_t brows = rows / 16, kbn = cols / 64;
  if (tokens <= 64) {
    // activations in LDS when they fit and there are enough brick-rows to
    // fill the chip without splitting K (the launch falls back to the small
    // kernel for the exponent form)
    // (8 waves per brick-row, two bricks in flight while one is computed:
    // measured best or within 1% on 14336x4096, 4096x14336, 28672x8192 and
    // 128256x4096 at one token)
    if (tokens <= 16 && tokens * cols <= kGemvXElems && kbn <= kGemvKbnMax && brows >= 128) return variant_gemv();
    // from 12 tokens (20 for matrices too short to fill the chip without a
    // K split): four brick-rows per workgroup over the whole of K, the
    // activations streamed through LDS in 8-brick slices
    // (two waves per brick-row and 4-brick slices when 4-brick-row
    // workgroups would need a second round on the CUs: half the LDS, two
    // workgroups per CU)
    const int64_t groups = (brows + 3) / 4;
    const Variant rowk = groups > 256 && groups <= 512 ? Variant{4, 2, 2, 2, 4} : Variant{4, 4, 2, 2, 4};
    if (tokens >= 12 && (tokens >= 20 || groups >= 128) && rowk_fits(tokens, rows, cols, rowk)) return rowk;
    // fewer tokens whose activations do not fit the gemv kernel's LDS copy
    // (long K, e.g. 8192x28672): the whole-K kernel where it fills the chip
    // (58.6 against 61.6 us for the small kernel at one token)
    if (tokens < 12 && groups >= 128 && rowk_fits(tokens, rows, cols, Variant{4, 4, 2, 2, 4}))
      return Variant{4, 4, 2, 2, 4};
    // from 16 tokens: K slices of the activations in LDS shared by 8
    // brick-rows (the small kernel reads them from L2 once per brick-row)
    if (tokens >= 16) return Variant{3, 8, 1, 2, 0};
    return small_default(tokens, rows, cols);
  }
  // up to 128 tokens: the whole-K kernel (16x16x32 instructions, two waves
  // per brick-row, activations streamed through LDS in 4-brick slices)
  const Variant rowk{4, 2, 2, 2, 4};
  if (tokens <= 128 && rowk_fits(tokens, rows, cols, rowk)) return rowk;
  // from 768 tokens: 128-row x 512-token workgroups that rebuild each weight
  // once for their 512 tokens into LDS, where they fill most of the chip and
  // the brick tables fit their LDS
  const int64_t wg22 = ((brows + 7) / 8) * ((tokens + 511) / 512);
  if (tokens >= 768 && kbn <= kWideKbnMax && wg22 >= 192) return Variant{1, 0, 1, 0, 22};
  // 256 x 256 tiles with the rebuild interleaved into the MFMAs once there are
  // enough tokens to fill the chip with them (one workgroup per CU)
  const int64_t wg11 = ((brows + 15) / 16) * ((tokens + 255) / 256);
  if (tokens >= 512 && wg11 >= 192) return Variant{1, 0, 1, 0, 11};
  // below that, the deep-prefetch tiles (128 rows; 128 tokens, B fragments
  // read three groups ahead, where that fills the chip, else 64 tokens).
  // They do not split K: for K of 256 bricks and more the K-split tiles
  // below do better.
  const int64_t rb8 = (brows + 7) / 8;
  if (kbn < 256) {
    const int64_t wg128 = rb8 * ((tokens + 127) / 128);
    // (eight activation tiles in flight when one workgroup per CU suffices,
    // three -- two or three workgroups per CU -- otherwise)
    if (wg128 >= 192) return Variant{1, 0, 1, 0, wg128 <= 256 ? 20 : 18};
    if (rb8 * ((tokens + 63) / 64) >= 192) return Variant{1, 0, 1, 0, tokens <= 192 ? 13 : 16};
  }
  // up to 256 tokens on matrices the deep-prefetch tiles do not fill: the
  // whole-K kernel with 2-brick slices (K split for short matrices)
  const Variant rowk256{4, 2, 1, 2, 4};
  if (tokens <= 256 && rowk_fits(tokens, rows, cols, rowk256)) return rowk256;
  const int64_t tblk = (tokens + 127) / 128;
  const int64_t wg0 = ((brows + 15) / 16) * tblk;  // tile 0: 256 rows per workgroup
  const int64_t wg1 = ((brows + 7) / 8) * tblk;    // tiles 1/5: 128 rows per workgroup
  Variant v{1, 0, 1, 0, wg0 >= 384 ? 0 : 1};
  const int64_t wgs = v.tile == 0 ? wg0 : wg1;
  if (wgs < 128)
    v.ksplit = (int)std::min<int64_t>({8, (256 + wgs - 1) / wgs, kbn});
  else if (wgs < 384 && kbn >= 128)
    v.ksplit = 2;
  if (v.tile == 1 && v.ksplit == 1) v.tile = 5;  // same tile on 32x32x16 instructions
  return v;
}

Variant variant_effective(int64_t tokens, int64_t rows, int64_t cols, bool exp_mode, const Variant& v0) {
  Variant v = v0;
  // (kinds 0 and 1 split K across workgroups; rowk's field is its slice shape)
  if (v.kind == 0 || v.kind == 1) v.ksplit = (int)std::max<int64_t>(1, std::min<int64_t>(v.ksplit, cols / 64));
  // x in LDS where it fits; elsewhere (exponent form, more activations) the
  // same choice falls back to the small kernel's default shape
  if (tokens <= 64 && v.kind == 2 &&
      !(!exp_mode && tokens <= 16 && tokens * cols <= kGemvXElems && cols / 64 <= kGemvKbnMax))
    v = small_default(tokens, rows, cols);
  // the wide tile keeps the brick tables of its 8 brick-rows in LDS
  if (v.kind == 1 && v.tile == 22 && cols / 64 > kWideKbnMax) v = variant_default(tokens, rows, cols);
  // a whole-K shape whose slices and tables do not fit LDS (or more tokens
  // than it is built for): the K-slice kernel, or the large-batch default
  if (v.kind == 4 && !rowk_fits(tokens, rows, cols, v))
    v = tokens <= 64 ? Variant{3, 8, 1, 2, 0} : variant_default(tokens, rows, cols);
  return v;
}

hipError_t launch_fused(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v0,
                        hipStream_t s) {
  const Variant v = variant_effective(tokens, w.rows, w.cols, w.exp_mode, v0);
  if (tokens <= 64) {
    if (v.kind == 2) return launch_fused_gemv(w, x, y, tokens, v, s);
    if (v.kind == 3) return launch_fused_mid(w, x, y, tokens, v, s);
    if (v.kind == 4) return launch_fused_rowk(w, x, y, tokens, v, s);
    if (v.kind != 0) return hipErrorInvalidValue;
    return launch_fused_small(w, x, y, tokens, v, s);
  }
  if (v.kind == 4) return launch_fused_rowk(w, x, y, tokens, v, s);
  if (v.kind != 1) return hipErrorInvalidValue;
  return launch_fused_large(w, x, y, tokens, v, s);
}

}  // namespace uw
