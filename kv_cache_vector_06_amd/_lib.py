"""ctypes binding of libtq.so — one Python function per C entry point of
include/tq.h, with the same names. Argument marshalling only: every step of
the computation runs in the library."""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

TQ_OK = 0
TQ_ERR_INVALID_ARG = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_HIP = -3
TQ_ERR_WORKSPACE = -4
TQ_ERR_NO_CONVERGE = -5
TQ_MSE = 0
TQ_PROD = 1
TQ_F32 = 0
TQ_BF16 = 1
TQ_ROT_DENSE = 0
TQ_ROT_HADAMARD = 1
TQ_SPLIT_NONE = 0
TQ_SPLIT_OUTLIER32 = 1
TQ_HEAD_DIM = 128

# Every function include/tq.h declares.
EXPORTED = ("tq_codebook", "tq_prep_bytes", "tq_prepare", "tq_encode",
            "tq_attn_decode_workspace", "tq_attn_decode", "tq_attn_decode_phase",
            "tq_decode_step", "tq_decode_step_phase", "tq_search_workspace", "tq_search",
            "tq_encode_chunked", "tq_search_chunked_workspace", "tq_search_chunked",
            "tq_read_probe", "tq_status_string", "tq_attn_decode_noalloc")
TQ_STATIC_SCRATCH_BYTES = 16 << 20


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {tq_status_string(status)} ({status})")
        self.status = status


class tq_quantizer(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("bits", ctypes.c_int), ("variant", ctypes.c_int),
                ("rot", ctypes.c_void_p), ("proj", ctypes.c_void_p),
                ("centroids", ctypes.c_void_p), ("boundaries", ctypes.c_void_p),
                ("prep", ctypes.c_void_p), ("rotation", ctypes.c_int), ("split", ctypes.c_int),
                ("centroids_o", ctypes.c_void_p), ("boundaries_o", ctypes.c_void_p),
                ("rot_o", ctypes.c_void_p), ("rot_r", ctypes.c_void_p), ("channels_o", ctypes.c_void_p),
                ("proj_o", ctypes.c_void_p), ("proj_r", ctypes.c_void_p)]


class tq_packed(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p),
                ("qjl", ctypes.c_void_p), ("gammas", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libtq.so; raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with kv_cache_vector_06_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.tq_codebook.argtypes = [I, I, P, P, P]
    lib.tq_codebook.restype = I
    lib.tq_prep_bytes.argtypes = []
    lib.tq_prep_bytes.restype = SZ
    lib.tq_prepare.argtypes = [ctypes.POINTER(tq_quantizer), P]
    lib.tq_prepare.restype = I
    lib.tq_encode.argtypes = [ctypes.POINTER(tq_quantizer), P, I, I64, I64, ctypes.POINTER(tq_packed), P, P]
    lib.tq_encode.restype = I
    lib.tq_attn_decode_workspace.argtypes = [I, I, I, I64]
    lib.tq_attn_decode_workspace.restype = SZ
    lib.tq_attn_decode.argtypes = [ctypes.POINTER(tq_quantizer), ctypes.POINTER(tq_quantizer), P,
                                   I, I, I, P, I64, ctypes.POINTER(tq_packed),
                                   ctypes.POINTER(tq_packed), ctypes.c_float, P, P, SZ, P]
    lib.tq_attn_decode.restype = I
    lib.tq_attn_decode_phase.argtypes = [I] + lib.tq_attn_decode.argtypes
    lib.tq_attn_decode_phase.restype = I
    lib.tq_decode_step.argtypes = [ctypes.POINTER(tq_quantizer), ctypes.POINTER(tq_quantizer), P, P, I, I64,
                                   P, I, I, I, P, I64, ctypes.POINTER(tq_packed),
                                   ctypes.POINTER(tq_packed), ctypes.c_float, P, P, SZ, P]
    lib.tq_decode_step.restype = I
    lib.tq_decode_step_phase.argtypes = [I] + lib.tq_decode_step.argtypes
    lib.tq_decode_step_phase.restype = I
    lib.tq_attn_decode_noalloc.argtypes = lib.tq_attn_decode.argtypes[:12] + [P]
    lib.tq_attn_decode_noalloc.restype = I
    lib.tq_search_workspace.argtypes = [I, I64, I]
    lib.tq_search_workspace.restype = SZ
    lib.tq_search.argtypes = [ctypes.POINTER(tq_quantizer), P, I, ctypes.POINTER(tq_packed), I64, I, P, P, P, SZ, P]
    lib.tq_search.restype = I
    lib.tq_encode_chunked.argtypes = [ctypes.POINTER(tq_quantizer), P, I, I64, I, I64, ctypes.POINTER(tq_packed), P]
    lib.tq_encode_chunked.restype = I
    lib.tq_search_chunked_workspace.argtypes = [I, I64, I, I]
    lib.tq_search_chunked_workspace.restype = SZ
    lib.tq_search_chunked.argtypes = [ctypes.POINTER(tq_quantizer), P, I, I, ctypes.POINTER(tq_packed), I64, I, P, P,
                                      P, SZ, P]
    lib.tq_search_chunked.restype = I
    lib.tq_read_probe.argtypes = [P, SZ, P, P]
    lib.tq_read_probe.restype = I
    lib.tq_status_string.argtypes = [I]
    lib.tq_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(st: int, where: str) -> int:
    if st != TQ_OK:
        raise TQError(st, where)
    return st


def tq_status_string(status: int) -> str:
    return load().tq_status_string(int(status)).decode()


def tq_codebook(d: int, bits: int):
    """→ (centroids float64[2^bits], boundaries float64[2^bits-1], mse_unit)."""
    K = 1 << bits
    c = np.zeros(K, np.float64)
    t = np.zeros(max(K - 1, 1), np.float64)
    mse = ctypes.c_double(0.0)
    _check(load().tq_codebook(int(d), int(bits), c.ctypes.data, t.ctypes.data, ctypes.byref(mse)),
           "tq_codebook")
    return c, t[: K - 1], mse.value


def tq_prep_bytes() -> int:
    return int(load().tq_prep_bytes())


def tq_prepare(q: tq_quantizer, stream: int | None) -> None:
    _check(load().tq_prepare(ctypes.byref(q), stream), "tq_prepare")


def tq_encode(q: tq_quantizer, x: int, x_dtype: int, n: int, x_row_stride: int,
              out: tq_packed, out_slot: int | None, stream: int | None) -> None:
    _check(load().tq_encode(ctypes.byref(q), x, int(x_dtype), int(n), int(x_row_stride),
                            ctypes.byref(out), out_slot, stream), "tq_encode")


def tq_attn_decode_workspace(B: int, Hq: int, Hkv: int, max_ctx: int) -> int:
    return int(load().tq_attn_decode_workspace(int(B), int(Hq), int(Hkv), int(max_ctx)))


def tq_attn_decode(kq: tq_quantizer, vq: tq_quantizer, query: int, B: int, Hq: int, Hkv: int,
                   ctx_lens: int | None, max_ctx: int, k_cache: tq_packed, v_cache: tq_packed,
                   scale: float, out: int, workspace: int, ws_bytes: int, stream: int | None) -> None:
    _check(load().tq_attn_decode(ctypes.byref(kq), ctypes.byref(vq), query, int(B), int(Hq), int(Hkv),
                                 ctx_lens, int(max_ctx), ctypes.byref(k_cache), ctypes.byref(v_cache),
                                 float(scale), out, workspace, int(ws_bytes), stream),
           "tq_attn_decode")


def tq_attn_decode_phase(phase: int, kq: tq_quantizer, vq: tq_quantizer, query: int, B: int, Hq: int,
                         Hkv: int, ctx_lens: int | None, max_ctx: int, k_cache: tq_packed,
                         v_cache: tq_packed, scale: float, out: int, workspace: int, ws_bytes: int,
                         stream: int | None) -> None:
    _check(load().tq_attn_decode_phase(int(phase), ctypes.byref(kq), ctypes.byref(vq), query, int(B),
                                       int(Hq), int(Hkv), ctx_lens, int(max_ctx), ctypes.byref(k_cache),
                                       ctypes.byref(v_cache), float(scale), out, workspace,
                                       int(ws_bytes), stream), "tq_attn_decode_phase")


def tq_attn_decode_noalloc(kq: tq_quantizer, vq: tq_quantizer, query: int, B: int, Hq: int, Hkv: int,
                           ctx_lens: int | None, max_ctx: int, k_cache: tq_packed, v_cache: tq_packed,
                           scale: float, out: int, stream: int | None) -> None:
    _check(load().tq_attn_decode_noalloc(ctypes.byref(kq), ctypes.byref(vq), query, int(B), int(Hq), int(Hkv),
                                         ctx_lens, int(max_ctx), ctypes.byref(k_cache), ctypes.byref(v_cache),
                                         float(scale), out, stream), "tq_attn_decode_noalloc")


def tq_decode_step(kq: tq_quantizer, vq: tq_quantizer, k_new: int, v_new: int, x_dtype: int,
                   x_row_stride: int, query: int, B: int, Hq: int, Hkv: int, ctx_lens: int | None,
                   max_ctx: int, k_cache: tq_packed, v_cache: tq_packed, scale: float, out: int,
                   workspace: int, ws_bytes: int, stream: int | None) -> None:
    _check(load().tq_decode_step(ctypes.byref(kq), ctypes.byref(vq), k_new, v_new, int(x_dtype),
                                 int(x_row_stride), query, int(B), int(Hq), int(Hkv), ctx_lens,
                                 int(max_ctx), ctypes.byref(k_cache), ctypes.byref(v_cache), float(scale),
                                 out, workspace, int(ws_bytes), stream), "tq_decode_step")


def tq_decode_step_phase(phase: int, kq: tq_quantizer, vq: tq_quantizer, k_new: int, v_new: int,
                         x_dtype: int, x_row_stride: int, query: int, B: int, Hq: int, Hkv: int,
                         ctx_lens: int | None, max_ctx: int, k_cache: tq_packed, v_cache: tq_packed,
                         scale: float, out: int, workspace: int, ws_bytes: int,
                         stream: int | None) -> None:
    _check(load().tq_decode_step_phase(int(phase), ctypes.byref(kq), ctypes.byref(vq), k_new, v_new,
                                       int(x_dtype), int(x_row_stride), query, int(B), int(Hq), int(Hkv),
                                       ctx_lens, int(max_ctx), ctypes.byref(k_cache), ctypes.byref(v_cache),
                                       float(scale), out, workspace, int(ws_bytes), stream),
           "tq_decode_step_phase")


def tq_encode_chunked(q: tq_quantizer, x: int, x_dtype: int, n: int, chunks: int, x_row_stride: int,
                      out: tq_packed, stream: int | None) -> None:
    _check(load().tq_encode_chunked(ctypes.byref(q), x, int(x_dtype), int(n), int(chunks), int(x_row_stride),
                                    ctypes.byref(out), stream), "tq_encode_chunked")


def tq_search_chunked_workspace(nq: int, n: int, k: int, chunks: int) -> int:
    return int(load().tq_search_chunked_workspace(int(nq), int(n), int(k), int(chunks)))


def tq_search_chunked(q: tq_quantizer, query: int, nq: int, chunks: int, db: tq_packed, n: int, k: int,
                      scores: int, index: int, workspace: int, ws_bytes: int, stream: int | None) -> None:
    _check(load().tq_search_chunked(ctypes.byref(q), query, int(nq), int(chunks), ctypes.byref(db), int(n), int(k),
                                    scores, index, workspace, int(ws_bytes), stream), "tq_search_chunked")


def tq_search_workspace(nq: int, n: int, k: int) -> int:
    return int(load().tq_search_workspace(int(nq), int(n), int(k)))


def tq_search(q: tq_quantizer, query: int, nq: int, db: tq_packed, n: int, k: int, scores: int, index: int,
              workspace: int, ws_bytes: int, stream: int | None) -> None:
    _check(load().tq_search(ctypes.byref(q), query, int(nq), ctypes.byref(db), int(n), int(k), scores, index,
                            workspace, int(ws_bytes), stream), "tq_search")


def tq_read_probe(buf: int, nbytes: int, xor_out: int, stream: int | None) -> None:
    _check(load().tq_read_probe(buf, int(nbytes), xor_out, stream), "tq_read_probe")
