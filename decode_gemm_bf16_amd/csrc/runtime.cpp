// C ABI (include/uw.h): handles, device upload, the four pipelines (Unweight
// page, section 六) and the palette-form full decode, side-stream preprocessing (section 八), plans from the
// autotuner (section 九), the SwiGLU layer and layer-stack runners, and the
// hipBLASLt call used by pipelines 1 and 5 and by the uncompressed baseline.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/uw.h"
#include "codec.h"
#include "kernels.h"
#include "runtime_internal.h"
#include "transcode.h"

namespace {

thread_local std::string g_err;

uw_status fail(uw_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define UW_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) return fail(UW_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Last-consumer event of each scratch buffer: a preprocessing step on a side
// stream must not overwrite scratch that the main stream still reads.
std::mutex g_scratch_mu;
std::map<void*, hipEvent_t> g_scratch_consumed;

hipEvent_t scratch_event(void* p) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_consumed.find(p);
  if (it != g_scratch_consumed.end()) return it->second;
  hipEvent_t ev = nullptr;
  if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return nullptr;
  g_scratch_consumed[p] = ev;
  return ev;
}

void scratch_forget(void* p) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_consumed.find(p);
  if (it != g_scratch_consumed.end()) {
    (void)hipEventDestroy(it->second);
    g_scratch_consumed.erase(it);
  }
}

// ---- hipBLASLt (pipeline 1's library GEMM and the uncompressed baseline) ----
struct GemmPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulAlgo_t algo;
};
std::mutex g_blas_mu;
hipblasLtHandle_t g_blas = nullptr;
constexpr size_t kBlasWs = size_t(64) << 20;
std::map<std::tuple<int64_t, int64_t, int64_t>, GemmPlan> g_plans;
// One hipBLASLt workspace per stream: library GEMMs in flight on different
// streams (split-K algorithms write the workspace) must not share one.
std::map<hipStream_t, void*> g_blas_ws;

uw_status gemm_bf16(const uint16_t* x, const uint16_t* w, float* y, int64_t m, int64_t n, int64_t k,
                    hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  if (!g_blas && hipblasLtCreate(&g_blas) != HIPBLAS_STATUS_SUCCESS) {
    g_blas = nullptr;
    return fail(UW_ERR_HIP, "hipblasLtCreate failed");
  }
  void*& ws_of_stream = g_blas_ws[s];
  if (!ws_of_stream && hipMalloc(&ws_of_stream, kBlasWs) != hipSuccess) {
    ws_of_stream = nullptr;
    g_blas_ws.erase(s);
    return fail(UW_ERR_OOM, "hipBLASLt workspace");
  }
  void* const ws = ws_of_stream;
  auto key = std::make_tuple(m, n, k);
  auto it = g_plans.find(key);
  if (it == g_plans.end()) {
    // Column-major view: Y^T[n, m] = W[n, k] * X^T[k, m]; W row-major [n, k] is
    // a column-major k x n matrix used transposed, X row-major is k x m.
    GemmPlan p;
    hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, k, n, k) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, k, m, k) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.c, HIP_R_32F, n, m, n) == HIPBLAS_STATUS_SUCCESS;
    if (!ok) return fail(UW_ERR_HIP, "hipBLASLt descriptor setup failed");
    hipblasLtMatmulPreference_t pref = nullptr;
    uint64_t ws = kBlasWs;
    hipblasLtMatmulPreferenceCreate(&pref);
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof ws);
    constexpr int kCand = 16;
    hipblasLtMatmulHeuristicResult_t res[kCand];
    int got = 0;
    hipblasStatus_t hs =
        hipblasLtMatmulAlgoGetHeuristic(g_blas, p.desc, p.a, p.b, p.c, p.c, pref, kCand, res, &got);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (hs != HIPBLAS_STATUS_SUCCESS || got < 1)
      return fail(UW_ERR_HIP, "hipBLASLt has no bf16->f32 algorithm for m=%lld n=%lld k=%lld", (long long)m,
                  (long long)n, (long long)k);
    p.algo = res[0].algo;
    // The library's first-ranked algorithm is not always its fastest (8B
    // down projection at 1024 tokens, weights read from HBM: 118 against 98
    // us for the third): on the first call of a shape, time the candidates on
    // the caller's buffers and keep the fastest.  Each timed call follows a
    // 512 MiB read that evicts the operands from L2 and the Infinity Cache,
    // as in use, where the weights stream from HBM (timed on cache-resident
    // operands the choice is a different, slower one at small batch).  Every
    // call writes the same y; the real call follows.  Skipped while the
    // stream is being captured into a graph, or when the eviction buffer
    // cannot be allocated.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    void* flush = nullptr;
    constexpr size_t kFlush = size_t(512) << 20;
    if (got > 1 && hipStreamIsCapturing(s, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone &&
        hipMalloc(&flush, kFlush + 16) == hipSuccess) {
      hipEvent_t e0 = nullptr, e1 = nullptr;
      if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
        const float alpha = 1.f, beta = 0.f;
        float best = 0.f;
        bool have_best = false;  // a candidate ran and was timed (the first may fail to run)
        for (int i = 0; i < got; ++i) {
          // warm-up (and a check that the candidate runs)
          if (hipblasLtMatmul(g_blas, p.desc, &alpha, w, p.a, x, p.b, &beta, y, p.c, y, p.c, &res[i].algo,
                              ws_of_stream, kBlasWs, s) != HIPBLAS_STATUS_SUCCESS)
            continue;
          constexpr int kReps = 3;
          float total = 0.f;
          bool ok = true;
          for (int r = 0; r < kReps && ok; ++r) {
            float ms = 0.f;
            ok = uw::launch_read(flush, static_cast<uint8_t*>(flush) + kFlush, kFlush, s) == hipSuccess &&
                 hipEventRecord(e0, s) == hipSuccess &&
                 hipblasLtMatmul(g_blas, p.desc, &alpha, w, p.a, x, p.b, &beta, y, p.c, y, p.c, &res[i].algo,
                                 ws_of_stream, kBlasWs, s) == HIPBLAS_STATUS_SUCCESS &&
                 hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
                 hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
            total += ms;
          }
          if (!ok) break;
          if (!have_best || total < best) {
            best = total;
            have_best = true;
            p.algo = res[i].algo;
          }
        }
      }
      if (e0) (void)hipEventDestroy(e0);
      if (e1) (void)hipEventDestroy(e1);
      (void)hipStreamSynchronize(s);
      (void)hipFree(flush);
    }
    it = g_plans.emplace(key, p).first;
  }
  const float alpha = 1.f, beta = 0.f;
  GemmPlan& p = it->second;
  hipblasStatus_t hs = hipblasLtMatmul(g_blas, p.desc, &alpha, w, p.a, x, p.b, &beta, y, p.c, y, p.c, &p.algo,
                                       ws, kBlasWs, s);
  if (hs != HIPBLAS_STATUS_SUCCESS) return fail(UW_ERR_HIP, "hipblasLtMatmul failed (%d)", (int)hs);
  return UW_OK;
}

}  // namespace

struct uw_matrix {
  uw::HostFormat hf;
  bool host_only = false;
  bool keep_host = false;  // the host streams stay after uw_upload (for uw_evict / re-upload)
  void* pinned = nullptr;  // uw_upload: page-locked image of the device allocation
  size_t pinned_bytes = 0;
  int64_t rows = 0, cols = 0;
  uint32_t formats = 0;
  // one device allocation holding every resident stream
  void* dmem = nullptr;
  size_t dmem_bytes = 0;
  uint8_t* d_sm = nullptr;
  uint8_t* d_nib = nullptr;
  uint2* d_meta = nullptr;
  uint8_t* d_side = nullptr;
  uint32_t* d_words = nullptr;
  uint32_t* d_offsets = nullptr;
  uint32_t* d_lut = nullptr;  // multi-symbol decode table (4096 entries)
  uint32_t* d_lut_codes = nullptr;  // the same with 4-bit palette codes (palette tables present)
  uint32_t lut_v[4] = {};
  uint64_t words_total = 0;  // payload + padding words on the device
  hipStream_t main = nullptr, side = nullptr;
  void* scratch = nullptr;
  size_t scratch_cap = 0;
  bool own_scratch = false;
  hipEvent_t prep_done = nullptr;
  int prep_pipeline = 0;  // pipeline whose preprocessed scratch is pending
  int plan_n = 0;
  int32_t plan_tok[16] = {}, plan_pipe[16] = {}, plan_var[16] = {};
  int variant = 0;

  bool has(uint32_t f) const { return (formats & f) != 0; }
  bool has_pal_tables() const { return has(UW_FMT_PALETTE) || has(UW_FMT_RAWAUX); }
  size_t scratch_need(int p) const {
    // pipelines 2 and 3: the interleaved order pads to whole groups of 512
    // chunks (512 x 256 weights)
    const size_t n = size_t(rows) * size_t(cols), groups = (n / 256 + 511) / 512;
    switch (p) {
      case 1:
      case 5: return align256(2 * n);
      case 2: return groups * 512 * 256;
      case 3: return groups * 512 * 128;
      default: return 0;
    }
  }
};

namespace {

// codes: the resident 4-bit codes (serial order) or the pipeline 2/3 scratch
// (interleaved order, written by the Huffman decoder)
uw::FusedW fused_view(const uw_matrix* h, bool exp_mode, const uint8_t* codes) {
  uw::FusedW f;
  f.sm = h->d_sm;
  f.codes = codes;
  f.codes_ilv = codes != h->d_nib;
  f.codes_bytes = f.codes_ilv ? h->scratch_need(exp_mode ? 2 : 3) : size_t(h->rows) * size_t(h->cols) / 2;
  f.meta = h->d_meta;
  f.side = h->d_side;
  f.side_bytes = std::max<uint64_t>(h->hf.n_raw * 64, 64);
  f.max_row_raw = h->hf.max_row_raw;
  for (int i = 0; i < 4; ++i) f.lut[i] = h->lut_v[i];
  f.rows = h->rows;
  f.cols = h->cols;
  f.exp_mode = exp_mode;
  return f;
}

uw::HuffDev huff_view(const uw_matrix* h) {
  uw::HuffDev d;
  d.words = h->d_words;
  d.offsets = h->d_offsets;
  d.lut = h->d_lut;
  d.lut_codes = h->d_lut_codes;
  d.sm = h->d_sm;
  d.meta = h->d_meta;
  d.total_bits = h->hf.stream_bits;
  d.rows = h->rows;
  d.cols = h->cols;
  return d;
}

uw_status check_pipeline(const uw_matrix* h, int p) {
  switch (p) {
    case 1:
    case 2:
      if (!h->has(UW_FMT_HUFFMAN)) return fail(UW_ERR_UNSUPPORTED, "pipeline %d needs the Huffman format", p);
      return UW_OK;
    case 3:
      if (!h->has(UW_FMT_HUFFMAN) || !h->has_pal_tables())
        return fail(UW_ERR_UNSUPPORTED, "pipeline 3 needs the Huffman format and the palette tables");
      return UW_OK;
    case 4:
    case 5:
      if (!h->has(UW_FMT_PALETTE)) return fail(UW_ERR_UNSUPPORTED, "pipeline %d needs the palette format", p);
      return UW_OK;
    default:
      return fail(UW_ERR_INVALID_ARG, "unknown pipeline %d", p);
  }
}

int resolve_pipeline(const uw_matrix* h, int64_t tokens, int pipeline, int* variant) {
  *variant = h->variant;
  if (pipeline != UW_P_AUTO) return pipeline;
  for (int i = 0; i < h->plan_n; ++i)
    if (tokens <= h->plan_tok[i]) {
      // a variant id names a kernel of its batch family (<= 64 tokens or
      // more): an entry tuned in the other family keeps only its pipeline
      *variant = (tokens <= 64) == (h->plan_tok[i] <= 64) ? h->plan_var[i] : 0;
      return h->plan_pipe[i];
    }
  *variant = 0;
  if (h->has(UW_FMT_PALETTE)) return 4;
  if (h->has(UW_FMT_HUFFMAN) && h->has_pal_tables()) return 3;
  return 1;
}

uw_status ensure_scratch(uw_matrix* h, int p) {
  const size_t need = h->scratch_need(p);
  if (h->scratch && h->scratch_cap >= need) return UW_OK;
  if (h->scratch && !h->own_scratch)
    return fail(UW_ERR_INVALID_ARG, "bound scratch holds %zu bytes, pipeline %d needs %zu", h->scratch_cap, p, need);
  if (h->scratch) {
    UW_HIP(hipStreamSynchronize(h->main));
    if (h->side != h->main) UW_HIP(hipStreamSynchronize(h->side));
    scratch_forget(h->scratch);
    (void)hipFree(h->scratch);
    h->scratch = nullptr;
  }
  if (hipMalloc(&h->scratch, need) != hipSuccess) {
    h->scratch = nullptr;
    return fail(UW_ERR_OOM, "scratch allocation of %zu bytes failed", need);
  }
  h->scratch_cap = need;
  h->own_scratch = true;
  return UW_OK;
}

uw_status launch_preprocess(uw_matrix* h, int p, hipStream_t s) {
  if (p == 5) {
    UW_HIP(uw::launch_palette_decode(fused_view(h, false, h->d_nib), (uint16_t*)h->scratch, s, s != h->main));
    return UW_OK;
  }
  const uw::HuffDev d = huff_view(h);
  const uw::DecodeEmit emit = p == 1 ? uw::EMIT_BF16 : p == 2 ? uw::EMIT_EXP : uw::EMIT_NIBBLE;
  UW_HIP(uw::launch_huff_decode(d, emit, h->scratch, s));
  return UW_OK;
}

// Make the main stream's copy of the preprocessed scratch ready.
uw_status prepare(uw_matrix* h, int p) {
  uw_status st = ensure_scratch(h, p);
  if (st != UW_OK) return st;
  if (h->prep_pipeline == p) {
    UW_HIP(hipStreamWaitEvent(h->main, h->prep_done, 0));
    h->prep_pipeline = 0;
    return UW_OK;
  }
  if (h->prep_pipeline != 0) {
    // the side stream is still writing this scratch for another pipeline:
    // the main stream's own preprocessing must not start before it ends
    UW_HIP(hipStreamWaitEvent(h->main, h->prep_done, 0));
    h->prep_pipeline = 0;
  }
  return launch_preprocess(h, p, h->main);
}

uw_status mark_consumed(uw_matrix* h) {
  hipEvent_t ev = scratch_event(h->scratch);
  if (!ev) return fail(UW_ERR_HIP, "event creation failed");
  UW_HIP(hipEventRecord(ev, h->main));
  return UW_OK;
}

// The fused kernels address the activations through a buffer resource whose
// range is a 32-bit byte count (recon.h, make_rsrc): X may hold at most this
// many bytes on pipelines 2-4.  The library GEMM of pipelines 1 and 5 has no
// such limit.
constexpr int64_t kMaxFusedXBytes = 0x7FFFFFF0;

// Everything uw_matmul checks before it launches: arguments, shape limits,
// the pipeline and variant.  Host only, so that it also runs on host-only
// handles (which then fail with UW_ERR_UNSUPPORTED after these checks).
uw_status matmul_check(const uw_matrix* h, const void* x, const void* y, int64_t tokens, int pipeline, int* p_out,
                       uw::Variant* v_out) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  if (!x || !y) return fail(UW_ERR_INVALID_ARG, "null activation or output pointer");
  if (tokens < 1) return fail(UW_ERR_INVALID_ARG, "tokens must be >= 1");
  if (tokens > (int64_t(1) << 24)) return fail(UW_ERR_INVALID_ARG, "tokens too large");
  int var = 0;
  const int p = resolve_pipeline(h, tokens, pipeline, &var);
  uw_status st = check_pipeline(h, p);
  if (st != UW_OK) return st;
  if ((p == 2 || p == 3 || p == 4) && tokens * h->cols * 2 > kMaxFusedXBytes)
    return fail(UW_ERR_SHAPE, "pipeline %d: activations of %lld x %lld bf16 exceed the fused kernels' %lld-byte limit",
                p, (long long)tokens, (long long)h->cols, (long long)kMaxFusedXBytes);
  uw::Variant v = uw::variant_default(tokens, h->rows, h->cols);
  if (var != 0 && !uw::variant_get(tokens, var, &v))
    return fail(UW_ERR_INVALID_ARG, "variant %d does not exist for %lld tokens", var, (long long)tokens);
  if (h->host_only) return fail(UW_ERR_UNSUPPORTED, "host-only handle");
  *p_out = p;
  *v_out = v;
  return UW_OK;
}

uw_status matmul_impl(uw_matrix* h, const uint16_t* x, float* y, int64_t tokens, int pipeline) {
  int p = 0;
  uw::Variant v;
  uw_status st = matmul_check(h, x, y, tokens, pipeline, &p, &v);
  if (st != UW_OK) return st;
  switch (p) {
    case 4:
      UW_HIP(uw::launch_fused(fused_view(h, false, h->d_nib), x, y, tokens, v, h->main));
      return UW_OK;
    case 3:
    case 2: {
      if ((st = prepare(h, p)) != UW_OK) return st;
      UW_HIP(uw::launch_fused(fused_view(h, p == 2, (const uint8_t*)h->scratch), x, y, tokens, v, h->main));
      return mark_consumed(h);
    }
    case 1:
    case 5: {
      if ((st = prepare(h, p)) != UW_OK) return st;
      if ((st = gemm_bf16(x, (const uint16_t*)h->scratch, y, tokens, h->rows, h->cols, h->main)) != UW_OK) return st;
      return mark_consumed(h);
    }
  }
  return fail(UW_ERR_INVALID_ARG, "unknown pipeline %d", p);
}

template <class T>
T* carve(uint8_t*& cur, size_t bytes) {
  T* p = reinterpret_cast<T*>(cur);
  cur += align256(bytes);
  return p;
}

// Byte offsets of the resident streams in the handle's one device
// allocation (absent streams: kNone).
constexpr size_t kNone = ~size_t(0);
struct Layout {
  size_t sm = kNone, nib = kNone, meta = kNone, side = kNone, words = kNone, offsets = kNone, lut = kNone,
         lutc = kNone, total = 0;
};

Layout layout_of(const uw_matrix* h) {
  const uw::HostFormat& f = h->hf;
  const uint64_t n = f.n(), nb = f.bricks();
  const bool pal = h->has(UW_FMT_PALETTE), tabs = h->has_pal_tables(), huf = h->has(UW_FMT_HUFFMAN);
  Layout L;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur += align256(bytes);
    return at;
  };
  L.sm = take(n);
  if (pal) L.nib = take(n / 2);
  if (tabs || huf) {
    L.meta = take(nb * 8);
    L.side = take(std::max<size_t>(f.n_raw * 64, 64));
  }
  if (huf) {
    L.words = take(f.words.size() * 4);
    L.offsets = take(f.offsets.size() * 4);
    L.lut = take(uw::kLutSize * 4);
    L.lutc = take(uw::kLutSize * 4);
  }
  L.total = cur;
  return L;
}

void assign_pointers(uw_matrix* h, const Layout& L) {
  uint8_t* base = static_cast<uint8_t*>(h->dmem);
  auto at = [&](size_t off) { return off == kNone ? nullptr : base + off; };
  h->d_sm = at(L.sm);
  h->d_nib = at(L.nib);
  h->d_meta = reinterpret_cast<uint2*>(at(L.meta));
  h->d_side = at(L.side);
  h->d_words = reinterpret_cast<uint32_t*>(at(L.words));
  h->d_offsets = reinterpret_cast<uint32_t*>(at(L.offsets));
  h->d_lut = reinterpret_cast<uint32_t*>(at(L.lut));
  h->d_lut_codes = reinterpret_cast<uint32_t*>(at(L.lutc));
  h->words_total = h->has(UW_FMT_HUFFMAN) ? h->hf.words.size() : 0;
  if (h->has_pal_tables()) {
    // palette entry i, exponent rotated right by one bit, at byte i%4 of lut_v[i/4]
    for (int i = 0; i < 4; ++i) h->lut_v[i] = 0;
    for (int i = 0; i < 16; ++i) {
      const uint32_t e = h->hf.palette[i];
      const uint32_t v = ((e >> 1) | (e << 7)) & 0xFFu;
      h->lut_v[i / 4] |= v << (8 * (i % 4));
    }
  }
}

// Hand every host stream to put(offset, bytes, source) at its layout offset,
// the derived tables (per-brick meta, decode tables) built on the way.  With
// device_tables the palette codes, meta and side table are skipped (kernels
// write them).
template <class Put>
uw_status put_streams(const uw_matrix* h, const Layout& L, bool device_tables, Put&& put) {
  const uw::HostFormat& f = h->hf;
  const uint64_t n = f.n(), nb = f.bricks();
  uw_status st;
  if ((st = put(L.sm, n, f.sm.data())) != UW_OK) return st;
  if (L.nib != kNone && !device_tables && (st = put(L.nib, n / 2, f.nib.data())) != UW_OK) return st;
  if (L.meta != kNone && !device_tables) {
    // per-brick {raw map, raw groups before}; all zero for a Huffman-only matrix
    std::vector<uint2> meta(nb, uint2{0, 0});
    if (h->has_pal_tables())
      for (uint64_t b = 0; b < nb; ++b) meta[b] = uint2{f.rawmap[b], f.rawbefore[b]};
    if ((st = put(L.meta, nb * 8, meta.data())) != UW_OK) return st;
    if (!f.side.empty() && (st = put(L.side, f.side.size(), f.side.data())) != UW_OK) return st;
  }
  if (L.words != kNone) {
    if ((st = put(L.words, f.words.size() * 4, f.words.data())) != UW_OK) return st;
    if ((st = put(L.offsets, f.offsets.size() * 4, f.offsets.data())) != UW_OK) return st;
    const std::vector<uint32_t> lut3 = uw::multi_symbol_table(f.lut);
    if ((st = put(L.lut, uw::kLutSize * 4, lut3.data())) != UW_OK) return st;
    // pipeline 3 decodes straight to palette codes
    uint8_t code_of[256];
    std::memset(code_of, 0, sizeof code_of);
    if (h->has_pal_tables()) {
      const int used = std::min<int>(16, int(f.distinct));
      for (int i = used - 1; i >= 0; --i) code_of[f.palette[i]] = uint8_t(i);
    }
    const std::vector<uint32_t> lutc = uw::multi_code_table(f.lut, code_of);
    if ((st = put(L.lutc, uw::kLutSize * 4, lutc.data())) != UW_OK) return st;
  }
  return UW_OK;
}

// Allocate the handle's device memory and copy the host streams into it.
// With device_tables (load-time transcode) the palette tables, codes
// included, are left for the caller's kernels to write.
uw_status upload(uw_matrix* h, bool device_tables = false) {
  const Layout L = layout_of(h);
  if (hipMalloc(&h->dmem, L.total) != hipSuccess) {
    h->dmem = nullptr;
    return fail(UW_ERR_OOM, "device allocation of %zu bytes failed", L.total);
  }
  h->dmem_bytes = L.total;
  assign_pointers(h, L);
  uint8_t* base = static_cast<uint8_t*>(h->dmem);
  uw_status st = put_streams(h, L, device_tables, [&](size_t off, size_t bytes, const void* src) -> uw_status {
    UW_HIP(hipMemcpy(base + off, src, bytes, hipMemcpyHostToDevice));
    return UW_OK;
  });
  if (st != UW_OK) return st;
  UW_HIP(hipEventCreateWithFlags(&h->prep_done, hipEventDisableTiming));
  return UW_OK;
}

void release_host_streams(uw::HostFormat& f) {
  std::vector<uint8_t>().swap(f.sm);
  std::vector<uint8_t>().swap(f.nib);
  std::vector<uint8_t>().swap(f.side);
  std::vector<uint32_t>().swap(f.words);
  // offsets, rawmap/rawbefore and lut are kept small enough? they are dropped too
  std::vector<uint32_t>().swap(f.offsets);
  std::vector<uint32_t>().swap(f.rawmap);
  std::vector<uint32_t>().swap(f.rawbefore);
  std::vector<uint16_t>().swap(f.lut);
}

}  // namespace

// ---- distribution bundle (section 十) and load-time transcode (section 六) ----

namespace {

// File layout, little-endian: a 64-byte header, the exponent histogram
// (256 x u64), the chunk bit offsets (u32), the Huffman payload words (u32,
// without the padding words) and the serial sign+mantissa bytes.
struct BundleHeader {
  char magic[8];          // "UWBUNDLE"
  uint32_t version;       // 1
  uint32_t header_bytes;  // 64
  int64_t rows, cols;
  uint64_t stream_bits;
  uint32_t chunk, lmax;   // 256, 12
  uint64_t words;         // payload words
  uint64_t offsets;       // chunk offsets
};
static_assert(sizeof(BundleHeader) == 64, "bundle header layout");
constexpr char kBundleMagic[8] = {'U', 'W', 'B', 'U', 'N', 'D', 'L', 'E'};

struct FileCloser {
  FILE* f;
  ~FileCloser() {
    if (f) fclose(f);
  }
};

// Device buffers of the load-time transcode, freed on every exit path.
struct DevTemp {
  void* p = nullptr;
  ~DevTemp() {
    if (p) {
      (void)hipDeviceSynchronize();
      (void)hipFree(p);
    }
  }
};

// Build the palette tables (and codes, for UW_FMT_PALETTE) of a loaded
// Huffman form on the device: decode the exponents, find the raw rows, count
// them, then allocate the handle's memory and fill codes and side table.
uw_status transcode_upload(uw_matrix* h) {
  uw::HostFormat& f = h->hf;
  const uint64_t nb = f.bricks();
  int16_t code_of[256];
  uw::select_palette(f.hist, f.palette, code_of);
  uw::CodeOfTable cof;
  for (int i = 0; i < 256; ++i) cof.c[i] = int8_t(code_of[i]);
  const std::vector<uint32_t> lut3 = uw::multi_symbol_table(f.lut);

  uint8_t* cur = nullptr;
  const size_t exps_bytes = h->scratch_need(2);
  const size_t tbytes = align256(f.words.size() * 4) + align256(f.offsets.size() * 4) + align256(lut3.size() * 4) +
                        align256(exps_bytes) + align256(nb * 4) + 2 * align256(uw::transcode_groups(nb) * 4) + 256;
  DevTemp tmp;
  if (hipMalloc(&tmp.p, tbytes) != hipSuccess) {
    tmp.p = nullptr;
    return fail(UW_ERR_OOM, "device allocation of %zu bytes for the transcode failed", tbytes);
  }
  cur = static_cast<uint8_t*>(tmp.p);
  uw::HuffDev d{};
  uint32_t* words = carve<uint32_t>(cur, f.words.size() * 4);
  uint32_t* offsets = carve<uint32_t>(cur, f.offsets.size() * 4);
  uint32_t* lut = carve<uint32_t>(cur, lut3.size() * 4);
  uint8_t* exps = carve<uint8_t>(cur, exps_bytes);
  uint32_t* rawmap = carve<uint32_t>(cur, nb * 4);
  const uint64_t ng = uw::transcode_groups(nb);
  uint32_t* wg_count = carve<uint32_t>(cur, ng * 4);
  uint32_t* wg_before = carve<uint32_t>(cur, ng * 4);
  uint32_t* total = carve<uint32_t>(cur, 4);
  UW_HIP(hipMemcpy(words, f.words.data(), f.words.size() * 4, hipMemcpyHostToDevice));
  UW_HIP(hipMemcpy(offsets, f.offsets.data(), f.offsets.size() * 4, hipMemcpyHostToDevice));
  UW_HIP(hipMemcpy(lut, lut3.data(), lut3.size() * 4, hipMemcpyHostToDevice));
  d.words = words;
  d.offsets = offsets;
  d.lut = lut;
  d.total_bits = f.stream_bits;
  d.rows = h->rows;
  d.cols = h->cols;
  UW_HIP(uw::launch_huff_decode(d, uw::EMIT_EXP, exps, nullptr));
  UW_HIP(uw::launch_raw_rows(exps, nb, cof, rawmap, wg_count, nullptr));
  UW_HIP(uw::launch_raw_scan(wg_count, ng, wg_before, total, nullptr));
  uint32_t n_raw = 0;
  UW_HIP(hipMemcpy(&n_raw, total, 4, hipMemcpyDeviceToHost));
  f.n_raw = n_raw;
  uw_status st = upload(h, true);
  if (st != UW_OK) return st;
  UW_HIP(uw::launch_palette_pack(exps, nb, cof, rawmap, wg_before, h->d_meta,
                                 h->has(UW_FMT_PALETTE) ? h->d_nib : nullptr, h->d_side, nullptr));
  UW_HIP(hipDeviceSynchronize());
  {  // the largest brick-row raw count, from the table just built
    std::vector<uint2> meta(nb);
    UW_HIP(hipMemcpy(meta.data(), h->d_meta, nb * 8, hipMemcpyDeviceToHost));
    std::vector<uint32_t> map(nb), before(nb);
    for (uint64_t b = 0; b < nb; ++b) {
      map[b] = meta[b].x;
      before[b] = meta[b].y;
    }
    f.max_row_raw = uw::max_row_raw(map.data(), before.data(), nb, uint64_t(h->cols) / 64);
  }
  return UW_OK;
}

uw_status load_impl(const char* path, uint32_t formats, uw_matrix* h) {
  FileCloser fc{fopen(path, "rb")};
  if (!fc.f) return fail(UW_ERR_IO, "cannot open %s", path);
  auto read = [&](void* dst, size_t bytes) { return bytes == 0 || fread(dst, 1, bytes, fc.f) == bytes; };
  BundleHeader hd;
  if (!read(&hd, sizeof hd) || std::memcmp(hd.magic, kBundleMagic, 8) != 0)
    return fail(UW_ERR_IO, "%s is not a weight bundle", path);
  if (hd.version != 1 || hd.header_bytes != sizeof hd) return fail(UW_ERR_FORMAT, "bundle version %u unknown", hd.version);
  if (hd.chunk != uint32_t(uw::kChunk) || hd.lmax != uint32_t(uw::kLmax))
    return fail(UW_ERR_FORMAT, "bundle chunk %u / code limit %u differ from this library's", hd.chunk, hd.lmax);
  if (hd.rows <= 0 || hd.cols <= 0 || hd.rows % 16 || hd.cols % 64 || hd.rows > (int64_t(1) << 31) ||
      hd.cols > (int64_t(1) << 31) || hd.rows * hd.cols >= (int64_t(1) << 31))
    return fail(UW_ERR_SHAPE, "bundle shape %lldx%lld not supported", (long long)hd.rows, (long long)hd.cols);
  uw::HostFormat& f = h->hf;
  f.rows = h->rows = hd.rows;
  f.cols = h->cols = hd.cols;
  const uint64_t n = f.n();
  if (hd.offsets != (n + uw::kChunk - 1) / uw::kChunk || hd.words != (hd.stream_bits + 31) / 32)
    return fail(UW_ERR_FORMAT, "bundle table sizes do not match its shape and stream length");
  if (!read(f.hist, sizeof f.hist)) return fail(UW_ERR_IO, "%s: truncated histogram", path);
  uint64_t sum = 0;
  for (int s = 0; s < 256; ++s) {
    sum += f.hist[s];
    f.distinct += f.hist[s] != 0;
  }
  if (sum != n) return fail(UW_ERR_FORMAT, "bundle histogram counts %llu weights, shape holds %llu",
                            (unsigned long long)sum, (unsigned long long)n);
  // the code is rebuilt from the histogram exactly as the encoder built it
  const std::string err = uw::huffman_tables(f);
  if (!err.empty()) return fail(UW_ERR_FORMAT, "%s", err.c_str());
  if (f.stream_bits != hd.stream_bits)
    return fail(UW_ERR_FORMAT, "bundle stream holds %llu bits, its histogram's code gives %llu",
                (unsigned long long)hd.stream_bits, (unsigned long long)f.stream_bits);
  try {
    f.offsets.resize(hd.offsets);
    f.words.assign(hd.words + uw::kStreamPadWords, 0);
    f.sm.resize(n);
  } catch (const std::bad_alloc&) {
    return fail(UW_ERR_OOM, "host allocation failed while reading %s", path);
  }
  if (!read(f.offsets.data(), hd.offsets * 4) || !read(f.words.data(), hd.words * 4) || !read(f.sm.data(), n))
    return fail(UW_ERR_IO, "%s: truncated bundle", path);
  char extra;
  if (fread(&extra, 1, 1, fc.f) != 0) return fail(UW_ERR_FORMAT, "%s: bytes after the bundle", path);
  if (f.offsets[0] != 0) return fail(UW_ERR_FORMAT, "first chunk offset is not 0");
  for (uint64_t c = 1; c < hd.offsets; ++c)
    if (f.offsets[c] < f.offsets[c - 1] || f.offsets[c] > f.stream_bits)
      return fail(UW_ERR_FORMAT, "chunk offset %llu out of order", (unsigned long long)c);

  h->formats = f.formats = formats & 0x7u;
  if (h->host_only) return UW_OK;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(UW_ERR_NO_DEVICE, "no HIP device");
  uw_status st = h->has_pal_tables() ? transcode_upload(h) : upload(h);
  if (st != UW_OK) return st;
  release_host_streams(h->hf);
  return UW_OK;
}

}  // namespace

namespace uw {

uw_status set_error(uw_status st, const char* msg) { return fail(st, "%s", msg); }

// One SwiGLU layer: gate and up into the workspace, h = silu(g) * u, down.
// Every projection is checked before anything is launched.  fused_only
// restricts the projections to pipeline 4, whose kernels need no
// preprocessing scratch and no library GEMM workspace, so the call allocates
// nothing.
uw_status mlp_forward_impl(uw_matrix* gate, uw_matrix* up, uw_matrix* down, const int32_t* pipelines,
                           const uint16_t* x_dev, float* y_dev, int64_t tokens, void* work_dev, size_t work_bytes,
                           bool fused_only) {
  if (!gate || !up || !down || !pipelines || !x_dev || !y_dev || !work_dev)
    return fail(UW_ERR_INVALID_ARG, "null argument");
  const int64_t inter = gate->rows, hidden = gate->cols;
  if (up->rows != inter || up->cols != hidden || down->rows != hidden || down->cols != inter)
    return fail(UW_ERR_SHAPE, "gate/up [inter, hidden] and down [hidden, inter] shapes disagree");
  if (tokens < 1) return fail(UW_ERR_INVALID_ARG, "tokens must be >= 1");
  if (up->main != gate->main || down->main != gate->main)
    return fail(UW_ERR_INVALID_ARG, "gate, up and down must share one main stream");
  if (work_bytes < uw_mlp_workspace_bytes(tokens, inter))
    return fail(UW_ERR_INVALID_ARG, "workspace of %zu bytes, %lld tokens need %zu", work_bytes, (long long)tokens,
                uw_mlp_workspace_bytes(tokens, inter));
  uw_matrix* const hs[3] = {gate, up, down};
  int ps[3] = {0, 0, 0};
  Variant vs[3];
  for (int j = 0; j < 3; ++j) {
    // x_dev stands in for each projection's input: only non-null is checked
    uw_status st = matmul_check(hs[j], x_dev, y_dev, tokens, pipelines[j], &ps[j], &vs[j]);
    if (st != UW_OK) return st;
    if (fused_only && ps[j] != 4)
      return fail(UW_ERR_UNSUPPORTED, "projection %d resolves to pipeline %d; only pipeline 4 runs without allocating",
                  j, ps[j]);
  }
  uint8_t* cur = static_cast<uint8_t*>(work_dev);
  float* g = carve<float>(cur, size_t(tokens) * inter * 4);
  float* u = carve<float>(cur, size_t(tokens) * inter * 4);
  uint16_t* hh = carve<uint16_t>(cur, size_t(tokens) * inter * 2);
  uw_status st;
  // up's and down's preprocessing (Huffman or palette decode into their
  // scratch) goes to their side streams first, where they have one, so that
  // it runs while gate's product does (the page's side-stream decode, within
  // the layer); their products wait for it
  for (int j = 1; j < 3; ++j) {
    const int p = ps[j];
    if ((p == 1 || p == 2 || p == 3 || p == 5) && hs[j]->side != hs[j]->main && hs[j]->prep_pipeline != p &&
        (st = uw_preprocess(hs[j], p)) != UW_OK)
      return st;
  }
  // gate and up read the same activations: when both run the same gemv or
  // whole-K variant on 4-bit codes -- the palette form (pipeline 4) or codes
  // decoded into scratch (pipeline 3, separate scratch buffers) -- they go out
  // as one launch (one ramp and drain of the HBM stream instead of two)
  const bool codes = ps[0] == ps[1] && (ps[0] == 4 || ps[0] == 3);
  const Variant eg = codes ? variant_effective(tokens, inter, hidden, false, vs[0]) : vs[0];
  const Variant eu = codes ? variant_effective(tokens, inter, hidden, false, vs[1]) : vs[1];
  const bool same = eg.kind == eu.kind && eg.waves == eu.waves && eg.ksplit == eu.ksplit &&
                    eg.unroll == eu.unroll && eg.tile == eu.tile;
  const bool rowk_shape = eg.kind == 4 && tokens <= 64 && eg.tile == 4 && eg.ksplit == 2 && eg.unroll == 2 &&
                          (eg.waves == 4 || eg.waves == 2);
  bool group = codes && same && (eg.kind == 2 || rowk_shape);
  if (group && ps[0] == 3) {
    if ((st = ensure_scratch(gate, 3)) != UW_OK || (st = ensure_scratch(up, 3)) != UW_OK) return st;
    group = gate->scratch != up->scratch;
  }
  if (group) {
    const bool p3 = ps[0] == 3;
    if (p3 && ((st = prepare(gate, 3)) != UW_OK || (st = prepare(up, 3)) != UW_OK)) return st;
    const FusedW ws[2] = {fused_view(gate, false, p3 ? (const uint8_t*)gate->scratch : gate->d_nib),
                          fused_view(up, false, p3 ? (const uint8_t*)up->scratch : up->d_nib)};
    const uint16_t* xs[2] = {x_dev, x_dev};
    float* ys[2] = {g, u};
    const int64_t ts[2] = {tokens, tokens};
    if (eg.kind == 2)
      UW_HIP(launch_fused_gemv_group(ws, xs, ys, ts, 2, eg, gate->main));
    else
      UW_HIP(launch_fused_rowk_group(ws, xs, ys, 2, tokens, eg, gate->main));
    if (p3 && ((st = mark_consumed(gate)) != UW_OK || (st = mark_consumed(up)) != UW_OK)) return st;
  } else {
    if ((st = matmul_impl(gate, x_dev, g, tokens, pipelines[0])) != UW_OK) return st;
    if ((st = matmul_impl(up, x_dev, u, tokens, pipelines[1])) != UW_OK) return st;
  }
  UW_HIP(launch_silu_mul(g, u, hh, tokens * inter, gate->main));
  return matmul_impl(down, hh, y_dev, tokens, pipelines[2]);
}

}  // namespace uw

extern "C" {

const char* uw_last_error(void) { return g_err.c_str(); }

uw_status uw_encode(const uint16_t* w_host, int64_t rows, int64_t cols, uint32_t formats, uw_handle* out) {
  if (!out) return fail(UW_ERR_INVALID_ARG, "null output handle pointer");
  *out = nullptr;
  if (!w_host) return fail(UW_ERR_INVALID_ARG, "null weight pointer");
  const uint32_t fmt = formats & 0x7u;
  if (!fmt) return fail(UW_ERR_INVALID_ARG, "no format requested");
  if (formats & ~(0x7u | UW_ENC_HOST_ONLY)) return fail(UW_ERR_INVALID_ARG, "unknown format flags 0x%x", formats);
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 64)
    return fail(UW_ERR_SHAPE, "shape %lldx%lld: rows must be a multiple of 16 and cols of 64", (long long)rows,
                (long long)cols);
  if (rows * cols >= (int64_t(1) << 31))
    return fail(UW_ERR_SHAPE, "matrix of %lld weights: at most 2^31 - 1 weights per matrix", (long long)(rows * cols));
  uw_matrix* h = new (std::nothrow) uw_matrix;
  if (!h) return fail(UW_ERR_OOM, "host allocation failed");
  h->rows = rows;
  h->cols = cols;
  h->formats = fmt;
  h->host_only = (formats & UW_ENC_HOST_ONLY) != 0;
  std::string err;
  try {
    err = uw::encode_host(w_host, rows, cols, fmt, h->hf);
  } catch (const std::bad_alloc&) {
    delete h;
    return fail(UW_ERR_OOM, "host allocation failed during encode");
  }
  if (!err.empty()) {
    delete h;
    return fail(err.find("2^32") != std::string::npos ? UW_ERR_FORMAT : UW_ERR_SHAPE, "%s", err.c_str());
  }
  if (!h->host_only) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
      delete h;
      return fail(UW_ERR_NO_DEVICE, "no HIP device");
    }
    uw_status st = upload(h);
    if (st != UW_OK) {
      if (h->dmem) (void)hipFree(h->dmem);
      if (h->prep_done) (void)hipEventDestroy(h->prep_done);
      delete h;
      return st;
    }
    release_host_streams(h->hf);
  }
  *out = h;
  return UW_OK;
}

uw_status uw_decode(uw_handle h, uint16_t* w_dev_out) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  if (h->host_only) return fail(UW_ERR_UNSUPPORTED, "host-only handle");
  if (!w_dev_out) return fail(UW_ERR_INVALID_ARG, "null output pointer");
  if (h->has(UW_FMT_HUFFMAN)) {
    UW_HIP(uw::launch_huff_decode(huff_view(h), uw::EMIT_BF16, w_dev_out, h->main));
  } else {
    UW_HIP(uw::launch_palette_decode(fused_view(h, false, h->d_nib), w_dev_out, h->main));
  }
  return UW_OK;
}

uw_status uw_matmul(uw_handle h, const uint16_t* x_dev, float* y_dev, int64_t tokens, int pipeline) {
  return matmul_impl(h, x_dev, y_dev, tokens, pipeline);
}

uw_status uw_preprocess(uw_handle h, int pipeline) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  if (h->host_only) return fail(UW_ERR_UNSUPPORTED, "host-only handle");
  if (pipeline < 1 || pipeline == 4 || pipeline > 5)
    return fail(UW_ERR_UNSUPPORTED, "pipeline %d has no preprocessing", pipeline);
  uw_status st = check_pipeline(h, pipeline);
  if (st != UW_OK) return st;
  if ((st = ensure_scratch(h, pipeline)) != UW_OK) return st;
  hipEvent_t consumed = scratch_event(h->scratch);
  if (!consumed) return fail(UW_ERR_HIP, "event creation failed");
  UW_HIP(hipStreamWaitEvent(h->side, consumed, 0));
  if ((st = launch_preprocess(h, pipeline, h->side)) != UW_OK) return st;
  UW_HIP(hipEventRecord(h->prep_done, h->side));
  h->prep_pipeline = pipeline;
  return UW_OK;
}

uw_status uw_set_streams(uw_handle h, void* main_stream, void* side_stream) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  h->main = static_cast<hipStream_t>(main_stream);
  h->side = side_stream ? static_cast<hipStream_t>(side_stream) : h->main;
  return UW_OK;
}

uw_status uw_set_scratch(uw_handle h, void* scratch_dev, size_t bytes) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  if (!scratch_dev || (reinterpret_cast<uintptr_t>(scratch_dev) & 255))
    return fail(UW_ERR_INVALID_ARG, "scratch must be a non-null 256-byte aligned device pointer");
  if (h->scratch && h->own_scratch) {
    if (hipDeviceSynchronize() != hipSuccess) return fail(UW_ERR_HIP, "synchronize failed");
    scratch_forget(h->scratch);
    (void)hipFree(h->scratch);
  }
  h->scratch = scratch_dev;
  h->scratch_cap = bytes;
  h->own_scratch = false;
  h->prep_pipeline = 0;
  return UW_OK;
}

uw_status uw_set_plan(uw_handle h, const int32_t* max_tokens, const int32_t* pipeline, const int32_t* variant,
                      int32_t n) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  if (n < 0 || n > 16) return fail(UW_ERR_INVALID_ARG, "plan size %d out of range", n);
  if (n && (!max_tokens || !pipeline || !variant)) return fail(UW_ERR_INVALID_ARG, "null plan arrays");
  for (int i = 0; i < n; ++i) {
    if (pipeline[i] < 1 || pipeline[i] > 5) return fail(UW_ERR_INVALID_ARG, "plan pipeline %d", pipeline[i]);
    uw_status st = check_pipeline(h, pipeline[i]);
    if (st != UW_OK) return st;
    if (variant[i] < 0 || variant[i] >= uw::variant_count(max_tokens[i]))
      return fail(UW_ERR_INVALID_ARG, "plan variant %d", variant[i]);
  }
  for (int i = 0; i < n; ++i) {
    h->plan_tok[i] = max_tokens[i];
    h->plan_pipe[i] = pipeline[i];
    h->plan_var[i] = variant[i];
  }
  h->plan_n = n;
  return UW_OK;
}

uw_status uw_set_variant(uw_handle h, int32_t variant) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  if (variant < 0) return fail(UW_ERR_INVALID_ARG, "variant %d", variant);
  h->variant = variant;
  return UW_OK;
}

const char* uw_variant_name(int64_t tokens, int32_t variant) { return uw::variant_name(tokens, variant); }

uw_status uw_variant_in_use(uw_handle h, int64_t tokens, int32_t pipeline, int32_t* pipeline_out, char* name,
                            size_t name_len) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  if (tokens < 1) return fail(UW_ERR_INVALID_ARG, "tokens must be >= 1");
  int var = 0;
  const int p = resolve_pipeline(h, tokens, pipeline, &var);
  uw_status st = check_pipeline(h, p);
  if (st != UW_OK) return st;
  uw::Variant v = uw::variant_default(tokens, h->rows, h->cols);
  if (var != 0 && !uw::variant_get(tokens, var, &v))
    return fail(UW_ERR_INVALID_ARG, "variant %d does not exist for %lld tokens", var, (long long)tokens);
  if (pipeline_out) *pipeline_out = p;
  if (name && name_len) {
    if (p == 1 || p == 5)
      snprintf(name, name_len, "hipblaslt");
    else
      uw::variant_describe(tokens, uw::variant_effective(tokens, h->rows, h->cols, p == 2, v), name, name_len);
  }
  return UW_OK;
}

uw_status uw_query(uw_handle h, uw_info* o) {
  if (!h || !o) return fail(UW_ERR_INVALID_ARG, "null argument");
  std::memset(o, 0, sizeof *o);
  const uw::HostFormat& f = h->hf;
  o->rows = h->rows;
  o->cols = h->cols;
  o->formats = h->formats;
  o->chunk = uw::kChunk;
  o->lmax = uw::kLmax;
  o->distinct_exponents = f.distinct;
  std::memcpy(o->palette, f.palette, 16);
  std::memcpy(o->code_lengths, f.lengths, 256);
  o->raw_groups = f.n_raw;
  o->max_row_raw = h->has_pal_tables() ? f.max_row_raw : 0xFFFFFFFFu;
  o->groups = f.n() / 64;
  o->stream_bits = f.stream_bits;
  o->stream_words = (f.stream_bits + 31) / 32;
  o->bpw_palette = h->has_pal_tables() ? f.bpw_palette() : 0.0;
  o->bpw_huffman = h->has(UW_FMT_HUFFMAN) ? f.bpw_huffman() : 0.0;
  // what this handle stores
  const double n = double(f.n());
  double bits = 8.0 * n;
  if (h->has(UW_FMT_PALETTE)) bits += 4.0 * n + 128.0;
  if (h->has_pal_tables()) bits += 512.0 * double(f.n_raw) + 64.0 * double(f.bricks());
  if (h->has(UW_FMT_HUFFMAN))
    bits += 32.0 * double(o->stream_words) + 32.0 * double((f.n() + uw::kChunk - 1) / uw::kChunk) + 2048.0;
  o->bpw_resident = bits / n;
  o->resident_bytes = h->dmem_bytes;
  for (int p = 1; p <= 5; ++p) o->scratch_bytes[p] = h->scratch_need(p);
  return UW_OK;
}

uw_status uw_export(uw_handle h, int which, void* dst, size_t cap, size_t* len) {
  if (!h || !len) return fail(UW_ERR_INVALID_ARG, "null argument");
  const uw::HostFormat& f = h->hf;
  const uint64_t n = f.n(), nb = f.bricks();
  const void* host = nullptr;
  const void* dev = nullptr;
  size_t bytes = 0;
  std::vector<uint32_t> tmp;
  switch (which) {
    case UW_STREAM_SM: bytes = n; host = f.sm.data(); dev = h->d_sm; break;
    case UW_STREAM_NIBBLES:
      if (!h->has(UW_FMT_PALETTE)) return fail(UW_ERR_UNSUPPORTED, "no palette codes");
      bytes = n / 2; host = f.nib.data(); dev = h->d_nib; break;
    case UW_STREAM_RAWMAP:
    case UW_STREAM_RAWBEFORE:
      if (!h->has_pal_tables()) return fail(UW_ERR_UNSUPPORTED, "no palette tables");
      bytes = nb * 4;
      if (h->host_only) {
        host = which == UW_STREAM_RAWMAP ? f.rawmap.data() : f.rawbefore.data();
      } else {
        std::vector<uint2> meta(nb);
        UW_HIP(hipMemcpy(meta.data(), h->d_meta, nb * 8, hipMemcpyDeviceToHost));
        tmp.resize(nb);
        for (uint64_t b = 0; b < nb; ++b) tmp[b] = which == UW_STREAM_RAWMAP ? meta[b].x : meta[b].y;
        host = tmp.data();
      }
      break;
    case UW_STREAM_SIDE:
      if (!h->has_pal_tables()) return fail(UW_ERR_UNSUPPORTED, "no palette tables");
      bytes = f.n_raw * 64; host = f.side.data(); dev = h->d_side; break;
    case UW_STREAM_WORDS:
      if (!h->has(UW_FMT_HUFFMAN)) return fail(UW_ERR_UNSUPPORTED, "no Huffman stream");
      bytes = ((f.stream_bits + 31) / 32) * 4; host = f.words.data(); dev = h->d_words; break;
    case UW_STREAM_OFFSETS:
      if (!h->has(UW_FMT_HUFFMAN)) return fail(UW_ERR_UNSUPPORTED, "no Huffman stream");
      bytes = ((n + uw::kChunk - 1) / uw::kChunk) * 4; host = f.offsets.data(); dev = h->d_offsets; break;
    case UW_STREAM_PALETTE:
      if (!h->has_pal_tables()) return fail(UW_ERR_UNSUPPORTED, "no palette");
      bytes = 16; host = f.palette; break;
    case UW_STREAM_LENGTHS:
      if (!h->has(UW_FMT_HUFFMAN)) return fail(UW_ERR_UNSUPPORTED, "no Huffman stream");
      bytes = 256; host = f.lengths; break;
    default:
      return fail(UW_ERR_INVALID_ARG, "unknown stream %d", which);
  }
  *len = bytes;
  if (!dst || cap < bytes) return fail(UW_ERR_INVALID_ARG, "destination holds %zu bytes, stream needs %zu", cap, bytes);
  if (bytes == 0) return UW_OK;
  const bool from_host = h->host_only || which == UW_STREAM_PALETTE || which == UW_STREAM_LENGTHS || tmp.size();
  if (from_host) {
    std::memcpy(dst, host, bytes);
  } else {
    UW_HIP(hipMemcpy(dst, dev, bytes, hipMemcpyDeviceToHost));
  }
  return UW_OK;
}

uw_status uw_clone(uw_handle h, uw_handle* out) {
  if (!h || !out) return fail(UW_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  if (h->host_only) return fail(UW_ERR_UNSUPPORTED, "host-only handle");
  uw_matrix* c = new (std::nothrow) uw_matrix;
  if (!c) return fail(UW_ERR_OOM, "host allocation failed");
  // scalar fields and the small host tables; the big host streams were released at upload
  c->hf.rows = h->hf.rows;
  c->hf.cols = h->hf.cols;
  c->hf.formats = h->hf.formats;
  std::memcpy(c->hf.hist, h->hf.hist, sizeof c->hf.hist);
  c->hf.distinct = h->hf.distinct;
  std::memcpy(c->hf.palette, h->hf.palette, 16);
  c->hf.n_raw = h->hf.n_raw;
  c->hf.max_row_raw = h->hf.max_row_raw;
  std::memcpy(c->hf.lengths, h->hf.lengths, 256);
  std::memcpy(c->hf.codes, h->hf.codes, sizeof c->hf.codes);
  c->hf.stream_bits = h->hf.stream_bits;
  c->rows = h->rows;
  c->cols = h->cols;
  c->formats = h->formats;
  std::memcpy(c->lut_v, h->lut_v, sizeof c->lut_v);
  c->words_total = h->words_total;
  c->plan_n = h->plan_n;
  std::memcpy(c->plan_tok, h->plan_tok, sizeof c->plan_tok);
  std::memcpy(c->plan_pipe, h->plan_pipe, sizeof c->plan_pipe);
  std::memcpy(c->plan_var, h->plan_var, sizeof c->plan_var);
  c->variant = h->variant;
  if (hipMalloc(&c->dmem, h->dmem_bytes) != hipSuccess) {
    delete c;
    return fail(UW_ERR_OOM, "device allocation of %zu bytes failed", h->dmem_bytes);
  }
  c->dmem_bytes = h->dmem_bytes;
  auto rebase = [&](auto* p) -> decltype(p) {
    if (!p) return nullptr;
    const size_t off = reinterpret_cast<const uint8_t*>(p) - static_cast<const uint8_t*>(h->dmem);
    return reinterpret_cast<decltype(p)>(static_cast<uint8_t*>(c->dmem) + off);
  };
  c->d_sm = rebase(h->d_sm);
  c->d_nib = rebase(h->d_nib);
  c->d_meta = rebase(h->d_meta);
  c->d_side = rebase(h->d_side);
  c->d_words = rebase(h->d_words);
  c->d_offsets = rebase(h->d_offsets);
  c->d_lut = rebase(h->d_lut);
  c->d_lut_codes = rebase(h->d_lut_codes);
  if (hipMemcpy(c->dmem, h->dmem, h->dmem_bytes, hipMemcpyDeviceToDevice) != hipSuccess ||
      hipEventCreateWithFlags(&c->prep_done, hipEventDisableTiming) != hipSuccess) {
    (void)hipFree(c->dmem);
    delete c;
    return fail(UW_ERR_HIP, "device copy failed");
  }
  *out = c;
  return UW_OK;
}

uw_status uw_save(uw_handle h, const char* path) {
  if (!h || !path) return fail(UW_ERR_INVALID_ARG, "null argument");
  if (!h->has(UW_FMT_HUFFMAN)) return fail(UW_ERR_UNSUPPORTED, "a bundle holds the Huffman form; the handle has none");
  const uw::HostFormat& f = h->hf;
  const uint64_t n = f.n();
  BundleHeader hd{};
  std::memcpy(hd.magic, kBundleMagic, 8);
  hd.version = 1;
  hd.header_bytes = sizeof hd;
  hd.rows = h->rows;
  hd.cols = h->cols;
  hd.stream_bits = f.stream_bits;
  hd.chunk = uw::kChunk;
  hd.lmax = uw::kLmax;
  hd.words = (f.stream_bits + 31) / 32;
  hd.offsets = (n + uw::kChunk - 1) / uw::kChunk;
  std::vector<uint32_t> words, offsets;
  std::vector<uint8_t> sm;
  const uint32_t* pw = f.words.data();
  const uint32_t* po = f.offsets.data();
  const uint8_t* ps = f.sm.data();
  if (!h->host_only) {
    try {
      words.resize(hd.words);
      offsets.resize(hd.offsets);
      sm.resize(n);
    } catch (const std::bad_alloc&) {
      return fail(UW_ERR_OOM, "host allocation failed");
    }
    UW_HIP(hipMemcpy(words.data(), h->d_words, hd.words * 4, hipMemcpyDeviceToHost));
    UW_HIP(hipMemcpy(offsets.data(), h->d_offsets, hd.offsets * 4, hipMemcpyDeviceToHost));
    UW_HIP(hipMemcpy(sm.data(), h->d_sm, n, hipMemcpyDeviceToHost));
    pw = words.data();
    po = offsets.data();
    ps = sm.data();
  }
  FileCloser fc{fopen(path, "wb")};
  if (!fc.f) return fail(UW_ERR_IO, "cannot create %s", path);
  auto write = [&](const void* src, size_t bytes) { return bytes == 0 || fwrite(src, 1, bytes, fc.f) == bytes; };
  if (!write(&hd, sizeof hd) || !write(f.hist, sizeof f.hist) || !write(po, hd.offsets * 4) ||
      !write(pw, hd.words * 4) || !write(ps, n))
    return fail(UW_ERR_IO, "write to %s failed", path);
  const int rc = fclose(fc.f);
  fc.f = nullptr;
  if (rc != 0) return fail(UW_ERR_IO, "closing %s failed", path);
  return UW_OK;
}

uw_status uw_load(const char* path, uint32_t formats, uw_handle* out) {
  if (!out) return fail(UW_ERR_INVALID_ARG, "null output handle pointer");
  *out = nullptr;
  if (!path) return fail(UW_ERR_INVALID_ARG, "null path");
  const uint32_t fmt = formats & 0x7u;
  if (!fmt) return fail(UW_ERR_INVALID_ARG, "no format requested");
  if (formats & ~(0x7u | UW_ENC_HOST_ONLY)) return fail(UW_ERR_INVALID_ARG, "unknown format flags 0x%x", formats);
  const bool host_only = (formats & UW_ENC_HOST_ONLY) != 0;
  if (host_only && fmt != UW_FMT_HUFFMAN)
    return fail(UW_ERR_UNSUPPORTED, "palette tables of a bundle are built on the device (no UW_ENC_HOST_ONLY)");
  uw_matrix* h = new (std::nothrow) uw_matrix;
  if (!h) return fail(UW_ERR_OOM, "host allocation failed");
  h->host_only = host_only;
  uw_status st = load_impl(path, fmt, h);
  if (st != UW_OK) {
    if (h->dmem) (void)hipFree(h->dmem);
    if (h->prep_done) (void)hipEventDestroy(h->prep_done);
    delete h;
    return st;
  }
  *out = h;
  return UW_OK;
}

uw_status uw_upload(uw_handle h) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  if (!h->host_only) return UW_OK;
  if (h->hf.sm.empty()) return fail(UW_ERR_UNSUPPORTED, "the handle holds no host streams");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(UW_ERR_NO_DEVICE, "no HIP device");
  const Layout L = layout_of(h);
  if (!h->pinned) {
    // the first upload lays the streams out as on the device, in page-locked
    // memory: every upload is then one DMA of the compressed bytes
    if (hipHostMalloc(&h->pinned, L.total, hipHostMallocDefault) != hipSuccess) {
      h->pinned = nullptr;
      return fail(UW_ERR_OOM, "page-locked host allocation of %zu bytes failed", L.total);
    }
    h->pinned_bytes = L.total;
    uint8_t* img = static_cast<uint8_t*>(h->pinned);
    (void)put_streams(h, L, false, [&](size_t off, size_t bytes, const void* src) -> uw_status {
      std::memcpy(img + off, src, bytes);
      return UW_OK;
    });
  }
  auto undo = [&](uw_status st) {
    if (h->dmem) (void)hipFree(h->dmem);
    if (h->prep_done) (void)hipEventDestroy(h->prep_done);
    h->dmem = nullptr;
    h->prep_done = nullptr;
    return st;
  };
  if (hipMalloc(&h->dmem, L.total) != hipSuccess) {
    h->dmem = nullptr;
    return fail(UW_ERR_OOM, "device allocation of %zu bytes failed", L.total);
  }
  h->dmem_bytes = L.total;
  assign_pointers(h, L);
  if (hipMemcpyAsync(h->dmem, h->pinned, L.total, hipMemcpyHostToDevice, h->main) != hipSuccess)
    return undo(fail(UW_ERR_HIP, "host-to-device copy failed"));
  if (hipEventCreateWithFlags(&h->prep_done, hipEventDisableTiming) != hipSuccess)
    return undo(fail(UW_ERR_HIP, "event creation failed"));
  h->host_only = false;
  h->keep_host = true;
  return UW_OK;
}

uw_status uw_evict(uw_handle h) {
  if (!h) return fail(UW_ERR_INVALID_ARG, "null handle");
  if (h->host_only) return UW_OK;
  if (!h->keep_host) return fail(UW_ERR_UNSUPPORTED, "the handle has no host copy (encode with UW_ENC_HOST_ONLY, then uw_upload)");
  UW_HIP(hipStreamSynchronize(h->main));
  if (h->side != h->main) UW_HIP(hipStreamSynchronize(h->side));
  if (h->scratch && h->own_scratch) {
    scratch_forget(h->scratch);
    (void)hipFree(h->scratch);
  }
  h->scratch = nullptr;
  h->scratch_cap = 0;
  h->own_scratch = false;
  h->prep_pipeline = 0;
  if (h->prep_done) (void)hipEventDestroy(h->prep_done);
  h->prep_done = nullptr;
  (void)hipFree(h->dmem);
  h->dmem = nullptr;
  h->dmem_bytes = 0;
  h->d_sm = h->d_nib = h->d_side = nullptr;
  h->d_meta = nullptr;
  h->d_words = h->d_offsets = h->d_lut = h->d_lut_codes = nullptr;
  h->host_only = true;
  return UW_OK;
}

uw_status uw_grouped_matmul(const uw_handle* experts, int32_t n, const uint16_t* x_dev, const int64_t* row_offsets,
                            float* y_dev, int pipeline) {
  if (!experts || n < 1 || !row_offsets || !x_dev || !y_dev) return fail(UW_ERR_INVALID_ARG, "null or empty argument");
  if (row_offsets[0] != 0) return fail(UW_ERR_INVALID_ARG, "row_offsets[0] must be 0");
  for (int32_t e = 0; e < n; ++e) {
    if (!experts[e]) return fail(UW_ERR_INVALID_ARG, "null expert %d", e);
    if (experts[e]->rows != experts[0]->rows || experts[e]->cols != experts[0]->cols)
      return fail(UW_ERR_SHAPE, "expert %d has another shape than expert 0", e);
    if (row_offsets[e + 1] < row_offsets[e]) return fail(UW_ERR_INVALID_ARG, "row_offsets decrease at %d", e);
  }
  for (int32_t e = 0; e < n; ++e)
    if (experts[e]->host_only) return fail(UW_ERR_UNSUPPORTED, "expert %d is not on the device", e);
  for (int32_t e = 0; e < n; ++e) {
    const int64_t t = row_offsets[e + 1] - row_offsets[e];
    if (t == 0) continue;
    int p = 0;
    uw::Variant v;
    uw_status st = matmul_check(experts[e], x_dev, y_dev, t, pipeline, &p, &v);
    if (st != UW_OK) return st;
  }
  const int64_t rows = experts[0]->rows, cols = experts[0]->cols;
  // Experts whose call resolves to pipeline 4 with few enough tokens for the
  // gemv kernels go out together, up to kFusedGroupMax per launch, on the
  // stream of the first of them: those whose variant is a gemv one, and those
  // left to the default when the group's brick-rows fill the chip (a single
  // short matrix takes the K-split small kernel by default; a group of them
  // does not need it).  Every other expert runs one launch of its own.
  const int64_t kbn = cols / 64, brows = rows / 16;
  struct Call {
    int p = 0, var = 0;
    uw::Variant v{}, ev{};
    bool cand = false;
  };
  std::vector<Call> calls(n);
  int64_t cand_brows = 0;
  for (int32_t e = 0; e < n; ++e) {
    const int64_t t = row_offsets[e + 1] - row_offsets[e];
    if (t == 0) continue;
    Call& c = calls[e];
    uw_status st = matmul_check(experts[e], x_dev, y_dev, t, pipeline, &c.p, &c.v);
    if (st != UW_OK) return st;
    (void)resolve_pipeline(experts[e], t, pipeline, &c.var);
    if (c.p != 4) continue;
    c.ev = uw::variant_effective(t, rows, cols, false, c.v);
    const bool fits = t <= 16 && t * cols <= uw::kGemvXElems && kbn <= uw::kGemvKbnMax;
    c.cand = c.ev.kind == 2 || (c.var == 0 && fits);
    if (c.cand) cand_brows += brows;
  }
  uw::FusedW gw[uw::kFusedGroupMax];
  const uint16_t* gx[uw::kFusedGroupMax];
  float* gy[uw::kFusedGroupMax];
  int64_t gt[uw::kFusedGroupMax];
  int ng = 0;
  bool have_group = false;
  uw::Variant gv{};
  hipStream_t gs = nullptr;
  auto flush = [&]() -> uw_status {
    if (ng == 0) return UW_OK;
    UW_HIP(uw::launch_fused_gemv_group(gw, gx, gy, gt, ng, gv, gs));
    ng = 0;
    return UW_OK;
  };
  for (int32_t e = 0; e < n; ++e) {
    const int64_t t = row_offsets[e + 1] - row_offsets[e];
    if (t == 0) continue;
    const uint16_t* xe = x_dev + row_offsets[e] * cols;
    float* ye = y_dev + row_offsets[e] * rows;
    const Call& c = calls[e];
    // the variant this expert would run in a group
    uw::Variant mine = c.ev;
    if (c.cand && c.ev.kind != 2) mine = cand_brows >= 128 ? uw::variant_gemv() : c.ev;
    const bool joins = c.cand && mine.kind == 2 &&
                       (!have_group || (experts[e]->main == gs && mine.waves == gv.waves && mine.unroll == gv.unroll));
    if (!joins) {
      uw_status st = matmul_impl(experts[e], xe, ye, t, pipeline);
      if (st != UW_OK) return st;
      continue;
    }
    if (!have_group) {
      have_group = true;
      gv = mine;
      gs = experts[e]->main;
    }
    gw[ng] = fused_view(experts[e], false, experts[e]->d_nib);
    gx[ng] = xe;
    gy[ng] = ye;
    gt[ng] = t;
    if (++ng == uw::kFusedGroupMax) {
      uw_status st = flush();
      if (st != UW_OK) return st;
    }
  }
  return flush();
}

void uw_free(uw_handle h) {
  if (!h) return;
  if (h->pinned) {
    if (!h->host_only) (void)hipDeviceSynchronize();
    (void)hipHostFree(h->pinned);
  }
  if (!h->host_only) {
    (void)hipDeviceSynchronize();
    if (h->scratch && h->own_scratch) {
      scratch_forget(h->scratch);
      (void)hipFree(h->scratch);
    }
    if (h->dmem) (void)hipFree(h->dmem);
    if (h->prep_done) (void)hipEventDestroy(h->prep_done);
  }
  delete h;
}

uw_status uw_silu_mul(const float* g, const float* u, uint16_t* hh, int64_t n, void* stream) {
  if (!g || !u || !hh) return fail(UW_ERR_INVALID_ARG, "null pointer");
  if (n < 0) return fail(UW_ERR_INVALID_ARG, "negative size");
  UW_HIP(uw::launch_silu_mul(g, u, hh, n, static_cast<hipStream_t>(stream)));
  return UW_OK;
}

size_t uw_mlp_workspace_bytes(int64_t tokens, int64_t inter) {
  const size_t t = size_t(std::max<int64_t>(tokens, 0)), i = size_t(std::max<int64_t>(inter, 0));
  return 2 * align256(t * i * 4) + align256(t * i * 2);
}

uw_status uw_mlp_forward(uw_handle gate, uw_handle up, uw_handle down, const int32_t* pipelines,
                         const uint16_t* x_dev, float* y_dev, int64_t tokens, void* work_dev, size_t work_bytes) {
  return uw::mlp_forward_impl(gate, up, down, pipelines, x_dev, y_dev, tokens, work_dev, work_bytes, false);
}

size_t uw_stack_workspace_bytes(int64_t tokens, int64_t hidden, int64_t inter) {
  const size_t t = size_t(std::max<int64_t>(tokens, 0)), hd = size_t(std::max<int64_t>(hidden, 0));
  return uw_mlp_workspace_bytes(tokens, inter) + align256(t * hd * 4) + align256(t * hd * 2);
}

uw_status uw_stack_forward(const uw_handle* handles, const int32_t* pipelines, int32_t layers,
                           const uint16_t* x_dev, float* y_dev, int64_t tokens, int32_t overlap, void* work_dev,
                           size_t work_bytes) {
  if (!handles || !pipelines || !x_dev || !y_dev || !work_dev || layers < 1)
    return fail(UW_ERR_INVALID_ARG, "bad argument");
  if (tokens < 1) return fail(UW_ERR_INVALID_ARG, "tokens must be >= 1");
  for (int i = 0; i < 3 * layers; ++i)
    if (!handles[i]) return fail(UW_ERR_INVALID_ARG, "null handle %d", i);
  const int64_t inter = handles[0]->rows, hidden = handles[0]->cols;
  for (int l = 0; l < layers; ++l) {
    const uw_matrix* g = handles[3 * l];
    const uw_matrix* u = handles[3 * l + 1];
    const uw_matrix* d = handles[3 * l + 2];
    // the workspace and the bf16 hand-over between layers are sized from layer 0
    if (g->rows != inter || g->cols != hidden || u->rows != inter || u->cols != hidden || d->rows != hidden ||
        d->cols != inter)
      return fail(UW_ERR_SHAPE, "layer %d differs from layer 0's shape", l);
    if (g->main != handles[0]->main || u->main != handles[0]->main || d->main != handles[0]->main)
      return fail(UW_ERR_INVALID_ARG, "all handles must share one main stream (layer %d differs)", l);
  }
  if (work_bytes < uw_stack_workspace_bytes(tokens, hidden, inter))
    return fail(UW_ERR_INVALID_ARG, "workspace too small");
  const size_t mlp_ws = uw_mlp_workspace_bytes(tokens, inter);
  uint8_t* cur = static_cast<uint8_t*>(work_dev) + mlp_ws;
  float* ytmp = carve<float>(cur, size_t(tokens) * hidden * 4);
  uint16_t* xnext = carve<uint16_t>(cur, size_t(tokens) * hidden * 2);
  hipStream_t main = handles[0]->main;
  auto hard = [&](int l, int j, int* p) {
    int var = 0;
    *p = resolve_pipeline(handles[3 * l + j], tokens, pipelines[3 * l + j], &var);
    return *p != 4;  // pipelines 1-3 and 5 preprocess
  };
  auto issue_prep = [&](int l) -> uw_status {
    for (int j = 0; j < 3; ++j) {
      int p = 0;
      if (hard(l, j, &p)) {
        uw_status st = uw_preprocess(handles[3 * l + j], p);
        if (st != UW_OK) return st;
      }
    }
    return UW_OK;
  };
  uw_status st;
  if (overlap && (st = issue_prep(0)) != UW_OK) return st;
  const uint16_t* xin = x_dev;
  for (int l = 0; l < layers; ++l) {
    if (overlap && l + 1 < layers && (st = issue_prep(l + 1)) != UW_OK) return st;
    int32_t p3[3];
    for (int j = 0; j < 3; ++j) {
      int var = 0;
      p3[j] = resolve_pipeline(handles[3 * l + j], tokens, pipelines[3 * l + j], &var);
    }
    float* yout = l + 1 == layers ? y_dev : ytmp;
    if ((st = uw_mlp_forward(handles[3 * l], handles[3 * l + 1], handles[3 * l + 2], p3, xin, yout, tokens,
                             work_dev, mlp_ws)) != UW_OK)
      return st;
    if (l + 1 < layers) {
      UW_HIP(uw::launch_f32_to_bf16(yout, xnext, tokens * hidden, main));
      xin = xnext;
    }
  }
  return UW_OK;
}

uw_status uw_stream_create(int32_t cu_first, int32_t cu_count, void** out) {
  if (!out) return fail(UW_ERR_INVALID_ARG, "null output");
  int dev = 0;
  UW_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  UW_HIP(hipGetDeviceProperties(&prop, dev));
  const int ncu = prop.multiProcessorCount;
  if (cu_first < 0 || cu_count < 1 || cu_first + cu_count > ncu)
    return fail(UW_ERR_INVALID_ARG, "CU range [%d, %d) outside 0..%d", cu_first, cu_first + cu_count, ncu);
  std::vector<uint32_t> mask((ncu + 31) / 32, 0u);
  for (int c = cu_first; c < cu_first + cu_count; ++c) mask[c / 32] |= 1u << (c % 32);
  hipStream_t s = nullptr;
  UW_HIP(hipExtStreamCreateWithCUMask(&s, (uint32_t)mask.size(), mask.data()));
  *out = s;
  return UW_OK;
}

uw_status uw_stream_destroy(void* stream) {
  if (!stream) return fail(UW_ERR_INVALID_ARG, "null stream");
  UW_HIP(hipStreamDestroy(static_cast<hipStream_t>(stream)));
  return UW_OK;
}

int32_t uw_device_cu_count(void) {
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  return prop.multiProcessorCount;
}

uw_status uw_gemm_bf16(const uint16_t* x_dev, const uint16_t* w_dev, float* y_dev, int64_t tokens, int64_t rows,
                       int64_t cols, void* stream) {
  if (!x_dev || !w_dev || !y_dev) return fail(UW_ERR_INVALID_ARG, "null pointer");
  if (tokens < 1 || rows < 1 || cols < 1) return fail(UW_ERR_SHAPE, "bad shape");
  return gemm_bf16(x_dev, w_dev, y_dev, tokens, rows, cols, static_cast<hipStream_t>(stream));
}

uw_status uw_device_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return fail(UW_ERR_INVALID_ARG, "null pointer");
  if (bytes % 16) return fail(UW_ERR_INVALID_ARG, "size must be a multiple of 16");
  UW_HIP(uw::launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
  return UW_OK;
}

uw_status uw_device_read(const void* src, void* sink, size_t bytes, void* stream) {
  if (!src || !sink) return fail(UW_ERR_INVALID_ARG, "null pointer");
  if (bytes % 16) return fail(UW_ERR_INVALID_ARG, "size must be a multiple of 16");
  UW_HIP(uw::launch_read(src, sink, bytes, static_cast<hipStream_t>(stream)));
  return UW_OK;
}

}  // extern "C"
