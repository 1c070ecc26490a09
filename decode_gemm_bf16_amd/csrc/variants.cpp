// Fused-kernel variants: the kernel shapes the autotuner chooses from
// (Unweight page, section 九: pipeline x kernel variant x decode/compute split).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.h"

namespace uw {

hipError_t launch_fused_small(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                              hipStream_t s);
hipError_t launch_fused_large(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                              hipStream_t s);
hipError_t launch_fused_gemv(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v,
                             hipStream_t s);
bool gemv_applies(const FusedW& w, int64_t tokens);

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
};
// large batch: kind 1, {tile, ksplit}
const Named kLarge[] = {
    {{1, 0, 1, 0, 0}, "large:t0(4x64r x128t):k1"}, {{1, 0, 2, 0, 0}, "large:t0(4x64r x128t):k2"},
    {{1, 0, 4, 0, 0}, "large:t0(4x64r x128t):k4"}, {{1, 0, 8, 0, 0}, "large:t0(4x64r x128t):k8"},
    {{1, 0, 16, 0, 0}, "large:t0(4x64r x128t):k16"}, {{1, 0, 1, 0, 1}, "large:t1(4x32r x128t):k1"},
    {{1, 0, 2, 0, 1}, "large:t1(4x32r x128t):k2"}, {{1, 0, 1, 0, 2}, "large:t2(2x64r x128t):k1"},
    {{1, 0, 2, 0, 2}, "large:t2(2x64r x128t):k2"}, {{1, 0, 1, 0, 3}, "large:t3(4x64r x64t):k1"},
    {{1, 0, 2, 0, 3}, "large:t3(4x64r x64t):k2"},
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

Variant variant_default(int64_t tokens, int64_t rows, int64_t cols) {
  const int64_t brows = rows / 16, kbn = cols / 64;
  if (tokens <= 64) {
    // activations in LDS when they fit and there are enough brick-rows to
    // fill the chip without splitting K (the launch falls back to the small
    // kernel for the exponent form)
    if (tokens <= 16 && tokens * cols <= 16384 && kbn <= 1024 && brows >= 128) return Variant{2, 8, 1, 2, 0};
    return small_default(tokens, rows, cols);
  }
  const int64_t tblk = (tokens + 127) / 128;
  const int64_t wg0 = ((brows + 15) / 16) * tblk;  // tile 0: 256 rows per workgroup
  const int64_t wg1 = ((brows + 7) / 8) * tblk;    // tile 1: 128 rows per workgroup
  Variant v{1, 0, 1, 0, wg0 >= 384 ? 0 : 1};
  const int64_t wgs = v.tile == 0 ? wg0 : wg1;
  if (wgs < 128)
    v.ksplit = (int)std::min<int64_t>({8, (256 + wgs - 1) / wgs, kbn});
  else if (wgs < 384 && kbn >= 128)
    v.ksplit = 2;
  return v;
}

hipError_t launch_fused(const FusedW& w, const uint16_t* x, float* y, int64_t tokens, const Variant& v0,
                        hipStream_t s) {
  Variant v = v0;
  v.ksplit = (int)std::max<int64_t>(1, std::min<int64_t>(v.ksplit, w.cols / 64));
  if (tokens <= 64) {
    if (v.kind == 2) {
      // x in LDS where it fits; elsewhere (exponent form, more activations)
      // the same choice falls back to the small kernel's default shape
      if (gemv_applies(w, tokens)) return launch_fused_gemv(w, x, y, tokens, v, s);
      v = small_default(tokens, w.rows, w.cols);
    }
    if (v.kind != 0) return hipErrorInvalidValue;
    return launch_fused_small(w, x, y, tokens, v, s);
  }
  if (v.kind != 1) return hipErrorInvalidValue;
  return launch_fused_large(w, x, y, tokens, v, s);
}

}  // namespace uw
