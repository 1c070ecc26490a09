/*
 * uw.h -- C ABI of a lossless BF16 weight codec with fused decode-into-matmul
 * kernels for AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the page "Unweight: how Cloudflare
 * compresses large models by 22% without losing precision":
 *   section 三  BF16 = 1 sign + 8 exponent + 7 mantissa bits; the exponent byte
 *               is the redundant part;
 *   section 四  Huffman code on the exponent bytes only, sign+mantissa kept
 *               verbatim; a palette of the 16 most frequent exponents; a row of
 *               64 weights holding any other exponent is stored raw;
 *   section 五  decompress on chip, never write the rebuilt weights to HBM;
 *   section 六  four execution pipelines (full decode + library GEMM,
 *               exponent-only decode, runtime palette transcode, direct palette);
 *   section 七  the reconstructing matmul;
 *   section 八  hard (Huffman) and easy (palette) layers, the next hard layer
 *               decoded on a side stream while an easy layer computes;
 *   section 九  an autotuner choosing the pipeline and decode/compute CU split.
 *
 * Conventions (all entry points):
 *   - Matrices are row-major.  A weight matrix W is [rows, cols] = [out, in]
 *     (a linear layer's weight), bf16 passed as uint16_t bit patterns.
 *     rows must be a multiple of 16 and cols a multiple of 64.
 *   - Activations X are [tokens, cols] bf16 (uint16_t), contiguous, on the
 *     device.  Outputs Y are [tokens, rows] float32, contiguous, on the device,
 *     overwritten (Y = X * W^T).
 *   - Pointers named *_host are host memory, *_dev device memory (hipMalloc or
 *     a torch CUDA tensor).  The caller owns every pointer it passes; the
 *     library only reads host inputs during the call.
 *   - Device work is enqueued on the handle's main stream (default: the null
 *     stream) and the call returns without synchronising.  Results are valid
 *     once that stream is synchronised.  Launch errors come back as
 *     UW_ERR_HIP; a device fault surfaces on a later call.
 *   - Every call returns a uw_status; on failure uw_last_error() gives a
 *     message (thread-local).  No C++ exception crosses this boundary.
 *   - A handle is not safe for concurrent use from several host threads.
 */
#ifndef UW_H
#define UW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct uw_matrix* uw_handle;

typedef enum {
  UW_OK = 0,
  UW_ERR_INVALID_ARG = 1,   /* null pointer, bad enum, tokens <= 0 ...        */
  UW_ERR_SHAPE = 2,         /* rows % 16 != 0, cols % 64 != 0, size overflow  */
  UW_ERR_OOM = 3,           /* host or device allocation failed               */
  UW_ERR_HIP = 4,           /* a HIP / hipBLASLt call failed                  */
  UW_ERR_FORMAT = 5,        /* stream too long for 32-bit offsets, bad table  */
  UW_ERR_UNSUPPORTED = 6,   /* pipeline needs a format the handle lacks, or a
                               device call on a host-only handle              */
  UW_ERR_NO_DEVICE = 7,     /* no gfx950 device visible                       */
  UW_ERR_IO = 8             /* a bundle file cannot be opened, read or written,
                               or is not a bundle                             */
} uw_status;

/* Section 六: the four pipelines, and a fifth that is pipeline 1 fed from the
 * direct-palette form (its full decode reads 1.5 bytes per weight instead of
 * running the Huffman decoder).  UW_P_AUTO picks from the plan set with
 * uw_set_plan (else a built-in rule: direct palette when the handle has it,
 * else runtime palette transcode, else full decode). */
typedef enum {
  UW_P_AUTO = 0,
  UW_P1_FULL_DECODE = 1,       /* Huffman -> bf16 W in scratch, then hipBLASLt     */
  UW_P2_EXP_DECODE = 2,        /* Huffman -> exponent bytes in scratch, fused GEMM */
  UW_P3_PALETTE_TRANSCODE = 3, /* Huffman -> 4-bit codes in scratch, fused GEMM    */
  UW_P4_DIRECT_PALETTE = 4,    /* resident 4-bit codes, fused GEMM, no preprocess  */
  UW_P5_PALETTE_DECODE = 5     /* palette form -> bf16 W in scratch, then hipBLASLt */
} uw_pipeline;

/* Format flags for uw_encode (section 四, section 六). */
#define UW_FMT_HUFFMAN   0x1u   /* Huffman exponent stream + chunk bit offsets     */
#define UW_FMT_PALETTE   0x2u   /* 4-bit codes + raw-group tables (direct palette) */
#define UW_FMT_RAWAUX    0x4u   /* only the palette and raw-group tables: lets a
                                   Huffman matrix run pipeline 3                   */
#define UW_ENC_HOST_ONLY 0x100u /* encode on the host and keep the streams there;
                                   no device is touched (inspection, export)       */

/* Streams of the stored format, for uw_export.  All per-weight streams are in
 * the serial order: 16x64 bricks, brick-rows top to bottom, bricks left to
 * right; inside a brick 64 runs of 16 weights, run l = row l%16, columns
 * 16*(l/16) .. +15. */
typedef enum {
  UW_STREAM_SM = 0,          /* uint8 [rows*cols] sign+mantissa bytes            */
  UW_STREAM_NIBBLES = 1,     /* uint8 [rows*cols/2] 4-bit codes: of 8 serial
                                codes, byte b = code b | code b+4 << 4           */
  UW_STREAM_RAWMAP = 2,      /* uint32 [bricks] bit r = row r's group raw        */
  UW_STREAM_RAWBEFORE = 3,   /* uint32 [bricks] raw groups in earlier bricks     */
  UW_STREAM_SIDE = 4,        /* uint8 [raw groups * 64] original exponent bytes  */
  UW_STREAM_WORDS = 5,       /* uint32 Huffman bitstream, MSB-first per word     */
  UW_STREAM_OFFSETS = 6,     /* uint32 [chunks] first bit of each 256-symbol chunk */
  UW_STREAM_PALETTE = 7,     /* uint8 [16] palette, index = 4-bit code           */
  UW_STREAM_LENGTHS = 8      /* uint8 [256] Huffman code length per exponent     */
} uw_stream;

typedef struct {
  int64_t rows, cols;
  uint32_t formats;            /* UW_FMT_* resident in this handle              */
  uint32_t chunk;              /* Huffman symbols per chunk (256)               */
  uint32_t lmax;               /* longest Huffman code (12)                     */
  uint32_t distinct_exponents;
  uint8_t palette[16];
  uint8_t code_lengths[256];
  uint64_t raw_groups, groups;
  uint64_t stream_bits;        /* Huffman payload bits (without padding)        */
  uint64_t stream_words;       /* payload words (without the 8 padding words)   */
  double bpw_palette;          /* bits/weight of the direct-palette form        */
  double bpw_huffman;          /* bits/weight of the Huffman form               */
  double bpw_resident;         /* bits/weight of what this handle stores        */
  uint64_t resident_bytes;     /* compressed bytes held on the device           */
  uint64_t scratch_bytes[6];   /* scratch that pipeline p (1..5) needs          */
  uint32_t max_row_raw;        /* most raw groups in one brick-row of 16 rows   */
                               /* (0xFFFFFFFF: no palette tables)               */
} uw_info;

/* Encode a bf16 matrix (section 四): split each weight into its exponent and
 * sign+mantissa bytes, build the formats requested in `formats` and upload them
 * to the current HIP device (unless UW_ENC_HOST_ONLY).  w_host: [rows, cols]
 * host array, read only during the call.  *out receives a new handle to free
 * with uw_free.  UW_ERR_SHAPE on bad shape, UW_ERR_FORMAT if the Huffman
 * stream exceeds 2^32 bits. */
uw_status uw_encode(const uint16_t* w_host, int64_t rows, int64_t cols, uint32_t formats,
                    uw_handle* out);

/* Rebuild the original bf16 matrix on the device (section 十: bit-exact).
 * Uses the GPU Huffman decoder when the handle holds UW_FMT_HUFFMAN, else the
 * palette form.  w_dev_out: [rows, cols] uint16 device buffer. */
uw_status uw_decode(uw_handle h, uint16_t* w_dev_out);

/* Y[tokens, rows] = X[tokens, cols] * W^T through `pipeline` (section 六, 七).
 * x_dev, y_dev: device buffers as in the conventions.  1 <= tokens <= 2^24;
 * on pipelines 2-4 (the fused kernels) X may hold at most 0x7FFFFFF0 bytes
 * (tokens * cols * 2), else UW_ERR_SHAPE -- checked before anything else
 * about the device, so host-only handles report it too.
 * Pipelines 1-3 need UW_FMT_HUFFMAN (3 also PALETTE or RAWAUX), 4 and 5 need
 * UW_FMT_PALETTE, else UW_ERR_UNSUPPORTED.  Pipelines 1-3 and 5 first run
 * their preprocessing into the handle's scratch unless uw_preprocess already
 * queued it, in which case the main stream waits for that work. */
uw_status uw_matmul(uw_handle h, const uint16_t* x_dev, float* y_dev, int64_t tokens, int pipeline);

/* Section 八: enqueue the preprocessing of `pipeline` (1-3, 5) on the handle's
 * side stream, writing the handle's scratch, and record an event that the next
 * uw_matmul with the same pipeline waits on.  Returns UW_ERR_UNSUPPORTED for
 * pipeline 4 or a missing format.
 * Scratch contents: pipelines 1 and 5, W as row-major bf16; pipelines 2 and 3, the
 * exponent bytes (16 per run) or 4-bit codes (8 bytes per run) of the serial
 * order regrouped: with chunk c = 256 serial weights (16 runs of 16) and run r
 * of it, the run sits at run slot (c/512 * 16 + r) * 512 + c%512 (whole groups
 * of 512 chunks, uw_info.scratch_bytes). */
uw_status uw_preprocess(uw_handle h, int pipeline);

/* Streams (hipStream_t passed as void*; NULL = the null stream).  The side
 * stream defaults to the main stream. */
uw_status uw_set_streams(uw_handle h, void* main_stream, void* side_stream);

/* Caller-owned device scratch for pipelines 1-3 and 5 (at least
 * uw_info.scratch_bytes[p] bytes, 256-byte aligned).  Without it the handle
 * allocates its own on first use.  Several handles may share one buffer when
 * their use does not overlap in time. */
uw_status uw_set_scratch(uw_handle h, void* scratch_dev, size_t bytes);

/* Autotuner output (section 九): for UW_P_AUTO, the first entry with
 * tokens <= max_tokens[i] selects pipeline[i] and kernel variant[i]
 * (variant 0 = built-in choice).  Variant ids name kernels of one batch
 * family (tokens <= 64, or more; see uw_variant_name): an entry whose
 * max_tokens lies in the other family than the call's token count applies
 * its pipeline with the built-in variant.  n <= 16; n = 0 clears the plan. */
uw_status uw_set_plan(uw_handle h, const int32_t* max_tokens, const int32_t* pipeline,
                      const int32_t* variant, int32_t n);

/* Force the fused-kernel variant for explicit pipelines (0 = built-in choice).
 * Variants are listed by uw_variant_name. */
uw_status uw_set_variant(uw_handle h, int32_t variant);

/* Name of fused-kernel variant `variant` for `tokens`, or NULL past the end. */
const char* uw_variant_name(int64_t tokens, int32_t variant);

/* What uw_matmul(h, ..., tokens, pipeline) would run, without running it:
 * *pipeline_out (if not NULL) receives the pipeline after plan / built-in
 * resolution, and `name` (capacity name_len bytes, NUL-terminated; may be
 * NULL) the fused-kernel variant's name as listed by uw_variant_name (or
 * "hipblaslt" for pipeline 1, whose matmul is the library GEMM).  Errors as
 * uw_matmul for an unusable pipeline or variant.  Host only: no GPU work. */
uw_status uw_variant_in_use(uw_handle h, int64_t tokens, int32_t pipeline, int32_t* pipeline_out, char* name,
                            size_t name_len);

uw_status uw_query(uw_handle h, uw_info* out);

/* Copy one stored stream to host memory `dst` (capacity `cap` bytes);
 * *len receives its size in bytes (set even when dst is NULL or too small,
 * in which case UW_ERR_INVALID_ARG is returned). */
uw_status uw_export(uw_handle h, int which, void* dst, size_t cap, size_t* len);

/* A new handle holding a device copy of h's resident streams (same formats,
 * plan and variant; own scratch, default streams).  Used to place copies of
 * one matrix at distinct addresses, e.g. to rotate weight copies past the
 * 256 MB Infinity Cache when measuring HBM throughput. */
uw_status uw_clone(uw_handle h, uw_handle* out);

/* Distribution bundle (section 十: the bundle that ships every MLP matrix
 * compressed): write h's Huffman form to the file `path` (created or
 * truncated).  Layout, little-endian: a 64-byte header {char[8] "UWBUNDLE";
 * u32 version = 1; u32 header bytes = 64; i64 rows; i64 cols; u64 stream
 * bits; u32 chunk = 256; u32 code-length limit = 12; u64 payload words; u64
 * chunk offsets}, the exponent histogram (256 x u64; the canonical code is
 * rebuilt from it), the chunk bit offsets (u32 each), the payload words (u32,
 * bits MSB first) and the serial sign+mantissa bytes.  h must hold
 * UW_FMT_HUFFMAN (else UW_ERR_UNSUPPORTED); a device handle's streams are
 * copied back to the host first.  UW_ERR_IO if the file cannot be written. */
uw_status uw_save(uw_handle h, const char* path);

/* Read a bundle written by uw_save into a new handle holding `formats`
 * (section 六: the direct-palette pipeline reads weights transcoded to the
 * 4-bit form at model load).  UW_FMT_HUFFMAN uploads the stream as read;
 * UW_FMT_PALETTE and UW_FMT_RAWAUX are built on the current device from the
 * Huffman form: the exponents are decoded, the palette is chosen from the
 * histogram (the encoder's rule), and kernels write the raw-group tables and
 * the 4-bit codes -- the same bytes uw_encode builds on the host.  With
 * UW_ENC_HOST_ONLY only UW_FMT_HUFFMAN is allowed (UW_ERR_UNSUPPORTED
 * otherwise).  Synchronous: the device work has finished on return.  Errors:
 * UW_ERR_IO (cannot open, not a bundle, truncated), UW_ERR_FORMAT (version,
 * table sizes, histogram, stream length or chunk offsets inconsistent, or
 * bytes after the end), UW_ERR_SHAPE, UW_ERR_OOM, UW_ERR_HIP. */
uw_status uw_load(const char* path, uint32_t formats, uw_handle* out);

/* Section 十一 (cold mixture-of-experts weights loaded on demand): make a
 * host-only handle (uw_encode with UW_ENC_HOST_ONLY, or a host-only uw_load)
 * usable on the current device: allocate its device memory and copy its
 * compressed streams there -- the compressed bytes, not bf16, cross the host
 * link (uw_info.resident_bytes of them).  The first call lays the streams out
 * in page-locked host memory exactly as on the device (kept until uw_free, in
 * addition to the host streams); each upload is then one asynchronous copy on
 * the handle's main stream, which later work on that stream waits for, so an
 * upload can overlap other streams' kernels.  uw_evict and a later uw_upload
 * can repeat.  No-op for a handle already on the device.  Errors:
 * UW_ERR_NO_DEVICE, UW_ERR_OOM, UW_ERR_HIP, UW_ERR_UNSUPPORTED (no host
 * streams). */
uw_status uw_upload(uw_handle h);

/* Release the device copy of a handle made resident by uw_upload, after its
 * streams have finished; it is host-only again (its scratch, if the library
 * allocated it, is freed too).  No-op for a host-only handle;
 * UW_ERR_UNSUPPORTED for a handle encoded on the device (no host copy). */
uw_status uw_evict(uw_handle h);

/* Mixture-of-experts form of uw_matmul: for each expert e < n, rows
 * row_offsets[e] .. row_offsets[e+1]-1 of X (the tokens routed to e, grouped
 * by expert by the caller) times expert e's W^T into the same rows of Y.
 * x_dev: [row_offsets[n], cols] bf16, y_dev: [row_offsets[n], rows] fp32,
 * row_offsets: host, n+1 non-decreasing entries from 0.  All experts share one
 * shape and must be on the device; experts without rows are skipped.  Experts
 * whose call resolves to the direct-palette gemv kernels (pipeline 4, few
 * tokens) with the same variant and main stream as the first such expert run
 * together, up to 16 per kernel launch, on that stream (the Unweight page,
 * section 十一: cold experts); every other expert's kernels go to its own main
 * stream, in expert order.  Errors:
 * UW_ERR_INVALID_ARG, UW_ERR_SHAPE (experts differ), UW_ERR_UNSUPPORTED (an
 * expert is host-only or lacks the pipeline's format), as for uw_matmul. */
uw_status uw_grouped_matmul(const uw_handle* experts, int32_t n, const uint16_t* x_dev, const int64_t* row_offsets,
                            float* y_dev, int pipeline);

void uw_free(uw_handle h);

const char* uw_last_error(void);

/* ---- SwiGLU glue and the layer pipeline (section 八, section 十一) ---- */

/* h_dev[i] = bf16(silu(g_dev[i]) * u_dev[i]), silu(g) = g / (1 + exp(-g)),
 * float32 arithmetic, round to nearest even.  n elements, on `stream`. */
uw_status uw_silu_mul(const float* g_dev, const float* u_dev, uint16_t* h_dev, int64_t n, void* stream);

/* One SwiGLU MLP layer y = down(silu(gate x) * up x) with the projections
 * given as handles (gate/up [inter, hidden], down [hidden, inter]).
 * pipelines[3] selects each projection's pipeline (UW_P_AUTO allowed).
 * work_dev: at least uw_mlp_workspace_bytes(tokens, inter) bytes of device
 * memory for the gate/up outputs and h.  Runs on gate's main stream.  When
 * gate and up resolve to the same gemv variant on 4-bit codes (pipeline 4, or
 * pipeline 3 with separate scratch buffers), their products go out as one
 * kernel launch; the results are those of two uw_matmul calls.  up's and
 * down's preprocessing (pipelines 1-3 and 5) is issued first on their side
 * streams where uw_set_streams gave them one, so that it overlaps gate's
 * product (as uw_preprocess would; their products wait for it). */
uw_status uw_mlp_forward(uw_handle gate, uw_handle up, uw_handle down, const int32_t* pipelines,
                         const uint16_t* x_dev, float* y_dev, int64_t tokens, void* work_dev,
                         size_t work_bytes);
size_t uw_mlp_workspace_bytes(int64_t tokens, int64_t inter);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer of
 * uw_mlp_forward with its workspace (gate/up outputs and h) in a fixed device
 * array of UW_STATIC_WORKSPACE_BYTES that the library holds on every device it
 * runs on until the process ends.  Makes no allocation: every projection must
 * resolve to pipeline 4 (direct palette, no preprocessing scratch, no library
 * GEMM workspace), else UW_ERR_UNSUPPORTED.  UW_ERR_SHAPE when
 * uw_mlp_workspace_bytes(tokens, inter) exceeds the array; other errors as
 * uw_mlp_forward.  All calls on one device share its array: calls that
 * overlap in time on one device (other streams, other threads) race and must
 * be ordered by the caller.  Runs on gate's main stream. */
#define UW_STATIC_WORKSPACE_BYTES (32u << 20)
uw_status uw_mlp_forward_noalloc(uw_handle gate, uw_handle up, uw_handle down, const int32_t* pipelines,
                                 const uint16_t* x_dev, float* y_dev, int64_t tokens);

/* A stack of MLP layers (section 八): layer l uses handles[3l .. 3l+2]
 * (gate, up, down) and pipelines[3l .. 3l+2].  Each layer's input is the
 * previous layer's output rounded to bf16; y_dev gets the last layer's output.
 * With overlap != 0, the preprocessing of every hard projection (pipelines
 * 1-3 and 5) is issued on its handle's side stream one layer ahead, while the
 * previous layer computes; handles of consecutive layers must then not share
 * scratch.  work_dev: uw_stack_workspace_bytes(tokens, hidden, inter) bytes. */
uw_status uw_stack_forward(const uw_handle* handles, const int32_t* pipelines, int32_t layers,
                           const uint16_t* x_dev, float* y_dev, int64_t tokens, int32_t overlap,
                           void* work_dev, size_t work_bytes);
size_t uw_stack_workspace_bytes(int64_t tokens, int64_t hidden, int64_t inter);

/* ---- Streams with a CU mask (section 九's decode/compute split) ---- */

/* Create a stream limited to compute units [cu_first, cu_first + cu_count)
 * of the current device (default priority).  *out receives a hipStream_t. */
uw_status uw_stream_create(int32_t cu_first, int32_t cu_count, void** out);
uw_status uw_stream_destroy(void* stream);
int32_t uw_device_cu_count(void);

/* ---- Reference points for measurement ---- */

/* Uncompressed baseline: y[tokens, rows] = x * w^T with w_dev a plain bf16
 * [rows, cols] matrix, through hipBLASLt (the library GEMM of pipelines 1 and
 * 5).  The first call of a (tokens, rows, cols) shape, unless the stream is
 * being captured into a graph, times up to 16 of the library's candidate
 * algorithms on the given buffers and keeps the fastest for that shape (the
 * host waits for it, once); later calls only enqueue. */
uw_status uw_gemm_bf16(const uint16_t* x_dev, const uint16_t* w_dev, float* y_dev, int64_t tokens,
                       int64_t rows, int64_t cols, void* stream);

/* Plain device copy of `bytes` bytes (multiple of 16) with 16-byte loads and
 * stores: the measured HBM ceiling. */
uw_status uw_device_copy(const void* src_dev, void* dst_dev, size_t bytes, void* stream);

/* Read `bytes` bytes (multiple of 16) with 16-byte loads and XOR them into
 * 16 bytes at sink_dev: the measured HBM read ceiling (a fused matmul only
 * reads weights). */
uw_status uw_device_read(const void* src_dev, void* sink_dev, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UW_H */
