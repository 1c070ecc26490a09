"""Python binding of libuw.so, the lossless BF16 weight codec with fused
decode-into-matmul kernels for MI355X (gfx950).

Argument marshalling only: every step runs in the C++/HIP library declared in
``include/uw.h``.  PyTorch supplies device memory and streams.  Importing this
package loads the library and fails loudly if it has not been built
(``python decode_gemm_bf16_amd/build.py``); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuw.so")

# enums and flags of uw.h
OK = 0
ERR_INVALID_ARG, ERR_SHAPE, ERR_OOM, ERR_HIP, ERR_FORMAT, ERR_UNSUPPORTED, ERR_NO_DEVICE, ERR_IO = 1, 2, 3, 4, 5, 6, 7, 8
P_AUTO, P1_FULL_DECODE, P2_EXP_DECODE, P3_PALETTE_TRANSCODE, P4_DIRECT_PALETTE, P5_PALETTE_DECODE = 0, 1, 2, 3, 4, 5
FMT_HUFFMAN, FMT_PALETTE, FMT_RAWAUX, ENC_HOST_ONLY = 0x1, 0x2, 0x4, 0x100
(STREAM_SM, STREAM_NIBBLES, STREAM_RAWMAP, STREAM_RAWBEFORE, STREAM_SIDE, STREAM_WORDS, STREAM_OFFSETS,
 STREAM_PALETTE, STREAM_LENGTHS) = range(9)

EXPORTED = [
    "uw_encode", "uw_decode", "uw_matmul", "uw_preprocess", "uw_set_streams", "uw_set_scratch", "uw_set_plan",
    "uw_set_variant", "uw_variant_name", "uw_variant_in_use", "uw_query", "uw_export", "uw_clone", "uw_save", "uw_load", "uw_upload", "uw_evict", "uw_grouped_matmul", "uw_free", "uw_last_error", "uw_silu_mul",
    "uw_mlp_forward", "uw_mlp_workspace_bytes", "uw_mlp_forward_noalloc", "uw_stack_forward", "uw_stack_workspace_bytes",
    "uw_stream_create", "uw_stream_destroy", "uw_device_cu_count", "uw_gemm_bf16", "uw_device_copy", "uw_device_read",
]


class UwError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"uw status {status}: {msg}")
        self.status = status


class Info(C.Structure):
    _fields_ = [
        ("rows", C.c_int64), ("cols", C.c_int64), ("formats", C.c_uint32), ("chunk", C.c_uint32),
        ("lmax", C.c_uint32), ("distinct_exponents", C.c_uint32), ("palette", C.c_uint8 * 16),
        ("code_lengths", C.c_uint8 * 256), ("raw_groups", C.c_uint64), ("groups", C.c_uint64),
        ("stream_bits", C.c_uint64), ("stream_words", C.c_uint64), ("bpw_palette", C.c_double),
        ("bpw_huffman", C.c_double), ("bpw_resident", C.c_double), ("resident_bytes", C.c_uint64),
        ("scratch_bytes", C.c_uint64 * 6), ("max_row_raw", C.c_uint32),
    ]


def _preload_runtime() -> None:
    """Load the HIP runtime that PyTorch ships before libuw.so, so that both
    resolve to one runtime (one process must not hold two HIP runtimes: they
    would not share devices, memory or streams)."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        return
    tl = os.path.join(list(spec.submodule_search_locations)[0], "lib")
    for name in ("libamdhip64.so", "libhipblaslt.so"):
        path = os.path.join(tl, name)
        if os.path.exists(path):
            C.CDLL(path, mode=C.RTLD_GLOBAL)


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python decode_gemm_bf16_amd/build.py`")
    _preload_runtime()
    lib = C.CDLL(LIB_PATH)
    vp, i64, i32, u32, st = C.c_void_p, C.c_int64, C.c_int32, C.c_uint32, C.c_int
    sig = {
        "uw_encode": ([vp, i64, i64, u32, C.POINTER(vp)], st),
        "uw_decode": ([vp, vp], st),
        "uw_matmul": ([vp, vp, vp, i64, C.c_int], st),
        "uw_preprocess": ([vp, C.c_int], st),
        "uw_set_streams": ([vp, vp, vp], st),
        "uw_set_scratch": ([vp, vp, C.c_size_t], st),
        "uw_set_plan": ([vp, C.POINTER(i32), C.POINTER(i32), C.POINTER(i32), i32], st),
        "uw_set_variant": ([vp, i32], st),
        "uw_variant_name": ([i64, i32], C.c_char_p),
        "uw_variant_in_use": ([vp, i64, i32, C.POINTER(i32), C.c_char_p, C.c_size_t], st),
        "uw_query": ([vp, C.POINTER(Info)], st),
        "uw_export": ([vp, C.c_int, vp, C.c_size_t, C.POINTER(C.c_size_t)], st),
        "uw_clone": ([vp, C.POINTER(vp)], st),
        "uw_save": ([vp, C.c_char_p], st),
        "uw_load": ([C.c_char_p, u32, C.POINTER(vp)], st),
        "uw_upload": ([vp], st),
        "uw_evict": ([vp], st),
        "uw_grouped_matmul": ([C.POINTER(vp), i32, vp, C.POINTER(i64), vp, C.c_int], st),
        "uw_free": ([vp], None),
        "uw_last_error": ([], C.c_char_p),
        "uw_silu_mul": ([vp, vp, vp, i64, vp], st),
        "uw_mlp_forward": ([vp, vp, vp, C.POINTER(i32), vp, vp, i64, vp, C.c_size_t], st),
        "uw_mlp_workspace_bytes": ([i64, i64], C.c_size_t),
        "uw_mlp_forward_noalloc": ([vp, vp, vp, C.POINTER(i32), vp, vp, i64], st),
        "uw_stack_forward": ([C.POINTER(vp), C.POINTER(i32), i32, vp, vp, i64, i32, vp, C.c_size_t], st),
        "uw_stack_workspace_bytes": ([i64, i64, i64], C.c_size_t),
        "uw_stream_create": ([i32, i32, C.POINTER(vp)], st),
        "uw_stream_destroy": ([vp], st),
        "uw_device_cu_count": ([], i32),
        "uw_gemm_bf16": ([vp, vp, vp, i64, i64, i64, vp], st),
        "uw_device_copy": ([vp, vp, C.c_size_t, vp], st),
        "uw_device_read": ([vp, vp, C.c_size_t, vp], st),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != OK:
        raise UwError(status, _lib.uw_last_error().decode(errors="replace"))


def _ptr(t) -> int:
    """Device/host address of a torch tensor or numpy array (None -> 0)."""
    if t is None:
        return 0
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream_ptr(stream) -> int | None:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream


def last_error() -> str:
    return _lib.uw_last_error().decode(errors="replace")


def variant_name(tokens: int, variant: int) -> str | None:
    r = _lib.uw_variant_name(tokens, variant)
    return r.decode() if r is not None else None


def variants(tokens: int) -> list[str]:
    out, i = [], 0
    while (n := variant_name(tokens, i)) is not None:
        out.append(n)
        i += 1
    return out


class Matrix:
    """An encoded weight matrix (an ``uw_handle``)."""

    def __init__(self, w_bits: np.ndarray, formats: int = FMT_HUFFMAN | FMT_PALETTE):
        w = np.ascontiguousarray(w_bits, dtype=np.uint16)
        if w.ndim != 2:
            raise ValueError("weight must be a 2-D array of bf16 bit patterns")
        h = C.c_void_p()
        _check(_lib.uw_encode(w.ctypes.data, w.shape[0], w.shape[1], formats, C.byref(h)))
        self._h = h
        self.rows, self.cols = w.shape
        self.formats = formats
        self._keep = []  # buffers whose lifetime the handle relies on (bound scratch)

    @property
    def handle(self) -> int:
        return self._h.value

    def free(self) -> None:
        if self._h:
            _lib.uw_free(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def clone(self) -> "Matrix":
        """A device copy of this matrix at a new address."""
        h = C.c_void_p()
        _check(_lib.uw_clone(self._h, C.byref(h)))
        m = Matrix.__new__(Matrix)
        m._h, m.rows, m.cols, m.formats, m._keep = h, self.rows, self.cols, self.formats, []
        return m

    def save(self, path: str) -> None:
        """Write the Huffman form to a bundle file (``uw_save``)."""
        _check(_lib.uw_save(self._h, os.fsencode(path)))

    @classmethod
    def load(cls, path: str, formats: int = FMT_HUFFMAN | FMT_PALETTE) -> "Matrix":
        """A matrix read from a bundle file; palette formats are transcoded on
        the device (``uw_load``)."""
        h = C.c_void_p()
        _check(_lib.uw_load(os.fsencode(path), formats, C.byref(h)))
        m = cls.__new__(cls)
        m._h, m.formats, m._keep = h, formats, []
        info = m.info()
        m.rows, m.cols = info["rows"], info["cols"]
        return m

    def upload(self) -> None:
        """Copy a host-only matrix's compressed streams to the device (``uw_upload``)."""
        _check(_lib.uw_upload(self._h))

    def evict(self) -> None:
        """Release the device copy of an uploaded matrix (``uw_evict``)."""
        _check(_lib.uw_evict(self._h))

    def decode(self, out) -> None:
        """bf16 W -> ``out`` (device tensor of rows*cols 16-bit elements)."""
        _check(_lib.uw_decode(self._h, _ptr(out)))

    def matmul(self, x, y, tokens: int | None = None, pipeline: int = P_AUTO) -> None:
        """y[tokens, rows] (float32, device) = x[tokens, cols] (bf16, device) @ W^T."""
        t = x.shape[0] if tokens is None else tokens
        _check(_lib.uw_matmul(self._h, _ptr(x), _ptr(y), t, pipeline))

    def preprocess(self, pipeline: int) -> None:
        _check(_lib.uw_preprocess(self._h, pipeline))

    def set_streams(self, main=None, side=None) -> None:
        _check(_lib.uw_set_streams(self._h, _stream_ptr(main), _stream_ptr(side)))

    def set_scratch(self, buf) -> None:
        nbytes = buf.numel() * buf.element_size()
        _check(_lib.uw_set_scratch(self._h, _ptr(buf), nbytes))
        self._keep = [buf]

    def set_plan(self, entries) -> None:
        """entries: iterable of (max_tokens, pipeline, variant)."""
        entries = list(entries)
        n = len(entries)
        arr = lambda i: (C.c_int32 * max(n, 1))(*[int(e[i]) for e in entries])
        _check(_lib.uw_set_plan(self._h, arr(0), arr(1), arr(2), n))

    def set_variant(self, variant: int) -> None:
        _check(_lib.uw_set_variant(self._h, variant))

    def variant_in_use(self, tokens: int, pipeline: int = 0) -> tuple[int, str]:
        """(pipeline, variant name) that matmul(..., tokens, pipeline) would run."""
        p = C.c_int32(0)
        buf = C.create_string_buffer(96)
        _check(_lib.uw_variant_in_use(self._h, tokens, pipeline, C.byref(p), buf, 96))
        return p.value, buf.value.decode()

    def info(self) -> dict:
        inf = Info()
        _check(_lib.uw_query(self._h, C.byref(inf)))
        d = {k: getattr(inf, k) for k, _ in Info._fields_}
        d["palette"] = list(inf.palette)
        d["code_lengths"] = list(inf.code_lengths)
        d["scratch_bytes"] = list(inf.scratch_bytes)
        return d

    def export(self, which: int) -> np.ndarray:
        n = C.c_size_t()
        _lib.uw_export(self._h, which, None, 0, C.byref(n))
        dtype = np.uint32 if which in (STREAM_RAWMAP, STREAM_RAWBEFORE, STREAM_WORDS, STREAM_OFFSETS) else np.uint8
        buf = np.empty(n.value // np.dtype(dtype).itemsize, dtype=dtype)
        _check(_lib.uw_export(self._h, which, buf.ctypes.data, buf.nbytes, C.byref(n)))
        return buf


def silu_mul(g, u, h, stream=None) -> None:
    _check(_lib.uw_silu_mul(_ptr(g), _ptr(u), _ptr(h), g.numel(), _stream_ptr(stream)))


def gemm_bf16(x, w, y, tokens: int, rows: int, cols: int, stream=None) -> None:
    """Uncompressed baseline through hipBLASLt: y = x @ w^T."""
    _check(_lib.uw_gemm_bf16(_ptr(x), _ptr(w), _ptr(y), tokens, rows, cols, _stream_ptr(stream)))


def device_copy(src, dst, nbytes: int, stream=None) -> None:
    _check(_lib.uw_device_copy(_ptr(src), _ptr(dst), nbytes, _stream_ptr(stream)))


def device_read(src, sink, nbytes: int, stream=None) -> None:
    """Read nbytes of src (HBM read ceiling); sink: >= 16 bytes of device memory."""
    _check(_lib.uw_device_read(_ptr(src), _ptr(sink), nbytes, _stream_ptr(stream)))


def mlp_workspace_bytes(tokens: int, inter: int) -> int:
    return _lib.uw_mlp_workspace_bytes(tokens, inter)


def mlp_forward(gate: Matrix, up: Matrix, down: Matrix, pipelines, x, y, tokens: int, work) -> None:
    p = (C.c_int32 * 3)(*pipelines)
    _check(_lib.uw_mlp_forward(gate._h, up._h, down._h, p, _ptr(x), _ptr(y), tokens, _ptr(work),
                               work.numel() * work.element_size()))


STATIC_WORKSPACE_BYTES = 32 << 20  # UW_STATIC_WORKSPACE_BYTES


def mlp_forward_noalloc(gate: Matrix, up: Matrix, down: Matrix, pipelines, x, y, tokens: int) -> None:
    """The SwiGLU layer with the library's fixed device workspace (no allocation;
    every projection must run the direct palette)."""
    p = (C.c_int32 * 3)(*pipelines)
    _check(_lib.uw_mlp_forward_noalloc(gate._h, up._h, down._h, p, _ptr(x), _ptr(y), tokens))


def stack_workspace_bytes(tokens: int, hidden: int, inter: int) -> int:
    return _lib.uw_stack_workspace_bytes(tokens, hidden, inter)


def stack_forward(mats, pipelines, x, y, tokens: int, work, overlap: bool = True) -> None:
    """mats: flat list [gate0, up0, down0, gate1, ...]."""
    n = len(mats)
    hs = (C.c_void_p * n)(*[m.handle for m in mats])
    p = (C.c_int32 * n)(*pipelines)
    _check(_lib.uw_stack_forward(hs, p, n // 3, _ptr(x), _ptr(y), tokens, int(bool(overlap)), _ptr(work),
                                 work.numel() * work.element_size()))


def stream_create(cu_first: int, cu_count: int) -> int:
    s = C.c_void_p()
    _check(_lib.uw_stream_create(cu_first, cu_count, C.byref(s)))
    return s.value


def stream_destroy(stream: int) -> None:
    _check(_lib.uw_stream_destroy(stream))


def device_cu_count() -> int:
    return int(_lib.uw_device_cu_count())


def bf16_tensor(bits: np.ndarray, device="cuda"):
    """A torch bfloat16 tensor holding exactly the given bf16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def bits_of(t) -> np.ndarray:
    """bf16/int16 torch tensor -> numpy uint16 bit patterns (host copy)."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def grouped_matmul(experts, x, y, row_offsets, pipeline: int = P_AUTO) -> None:
    """y[o[e]:o[e+1]] = x[o[e]:o[e+1]] @ W_e^T for each expert e (``uw_grouped_matmul``)."""
    n = len(experts)
    hs = (C.c_void_p * n)(*[m.handle for m in experts])
    offs = (C.c_int64 * (n + 1))(*[int(v) for v in row_offsets])
    _check(_lib.uw_grouped_matmul(hs, n, _ptr(x), offs, _ptr(y), pipeline))
