"""Torch-facing helpers over the C ABI: device buffers from PyTorch, the
current HIP stream, and argument marshalling. No arithmetic of the method
happens here; it all runs in libtq.so."""
from __future__ import annotations

import math

import numpy as np
import torch

from . import _lib as L


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


class Quantizer:
    """One TurboQuant quantizer (rotation, optional QJL projection, codebook,
    prepared operands), all resident on `device`."""

    def __init__(self, rot: np.ndarray | None, bits: int, variant: str = "mse",
                 proj: np.ndarray | None = None, device: str = "cuda", rotation: str = "dense",
                 split: tuple | None = None):
        """`rotation` is "dense" (any orthogonal rot) or "hadamard" (rot is the
        randomized Walsh-Hadamard rotation H·diag(s)/√d). `split` =
        (rot_o, rot_r, channels) makes an outlier-channel split quantizer: the
        32 `channels` at bits + 1 bits with rotation rot_o (32×32), the other
        96 at `bits` bits with rot_r (96×96); `rot` is then ignored. A prod
        split adds the groups' sketch matrices: (rot_o, rot_r, channels,
        proj_o (32×32), proj_r (96×96)); `proj` is then ignored."""
        self.split = split is not None
        d = 128 if self.split else rot.shape[0]
        self.d, self.bits = d, bits
        self.variant = L.TQ_PROD if variant == "prod" else L.TQ_MSE
        self.bm = bits - 1 if self.variant == L.TQ_PROD else bits
        c, t, self.mse_unit = L.tq_codebook(d - 32 if self.split else d, self.bm)
        self.centroids64, self.boundaries64 = c, t
        dev = torch.device(device)
        self.rot = None if self.split else torch.as_tensor(np.ascontiguousarray(rot, np.float32)).to(dev)
        self.proj = self.proj_o = self.proj_r = None
        if self.variant == L.TQ_PROD and not self.split:
            if proj is None:
                raise ValueError("prod quantizer needs a projection")
            self.proj = torch.as_tensor(np.ascontiguousarray(proj, np.float32)).to(dev)
        self.centroids = torch.as_tensor(c.astype(np.float32)).to(dev)
        self.boundaries = torch.as_tensor(np.concatenate([t, [0.0]]).astype(np.float32)).to(dev)
        self.prep = torch.empty(L.tq_prep_bytes(), dtype=torch.uint8, device=dev)
        self.rotation = {"dense": L.TQ_ROT_DENSE, "hadamard": L.TQ_ROT_HADAMARD}[rotation]
        self.centroids_o = self.boundaries_o = self.rot_o = self.rot_r = None
        self.channels_o = None
        if self.split:
            rot_o, rot_r, channels = split[:3]
            if np.shape(rot_o) != (32, 32) or np.shape(rot_r) != (96, 96) or np.size(channels) != 32:
                raise ValueError("the split takes a 32x32 and a 96x96 rotation and 32 outlier channels")
            if self.variant == L.TQ_PROD:
                if len(split) != 5 or np.shape(split[3]) != (32, 32) or np.shape(split[4]) != (96, 96):
                    raise ValueError("a prod split also takes the groups' 32x32 and 96x96 sketch matrices")
                self.proj_o = torch.as_tensor(np.ascontiguousarray(split[3], np.float32)).to(dev)
                self.proj_r = torch.as_tensor(np.ascontiguousarray(split[4], np.float32)).to(dev)
            self.rot_o = torch.as_tensor(np.ascontiguousarray(rot_o, np.float32)).to(dev)
            self.rot_r = torch.as_tensor(np.ascontiguousarray(rot_r, np.float32)).to(dev)
            # host memory: read by tq_prepare only
            self.channels_o = np.ascontiguousarray(np.asarray(channels).reshape(32), np.int32)
            co, to, self.mse_unit_o = L.tq_codebook(32, self.bm + 1)
            self.centroids64_o, self.boundaries64_o = co, to
            self.centroids_o = torch.as_tensor(co.astype(np.float32)).to(dev)
            self.boundaries_o = torch.as_tensor(np.concatenate([to, [0.0]]).astype(np.float32)).to(dev)
        self.c = L.tq_quantizer(d, bits, self.variant, _ptr(self.rot), _ptr(self.proj),
                                _ptr(self.centroids), _ptr(self.boundaries), _ptr(self.prep), self.rotation,
                                L.TQ_SPLIT_OUTLIER32 if self.split else L.TQ_SPLIT_NONE,
                                _ptr(self.centroids_o), _ptr(self.boundaries_o), _ptr(self.rot_o),
                                _ptr(self.rot_r),
                                None if self.channels_o is None else self.channels_o.ctypes.data,
                                _ptr(self.proj_o), _ptr(self.proj_r))
        L.tq_prepare(self.c, _stream())

    @property
    def code_bytes(self) -> int:
        return 16 * self.bm + 4 if self.split else self.d * self.bm // 8

    @property
    def norms_per_vector(self) -> int:
        return 2 if self.split else 1


class Packed:
    """Packed vectors for n slots (see tq_packed in include/tq.h)."""

    def __init__(self, q: Quantizer, n: int, device: str = "cuda"):
        dev = torch.device(device)
        self.n = n
        self.codes = torch.zeros((n, q.code_bytes), dtype=torch.uint8, device=dev)
        self.norms = torch.zeros((n, 2) if q.split else n, dtype=torch.float32, device=dev)
        self.qjl = self.gammas = None
        if q.variant == L.TQ_PROD:
            self.qjl = torch.zeros((n, q.d // 8), dtype=torch.uint8, device=dev)
            self.gammas = torch.zeros((n, 2) if q.split else n, dtype=torch.float32, device=dev)
        self.c = L.tq_packed(_ptr(self.codes) if q.code_bytes else None, _ptr(self.norms),
                             _ptr(self.qjl), _ptr(self.gammas))


def encode(q: Quantizer, x: torch.Tensor, out: Packed | None = None,
           slots: torch.Tensor | None = None) -> Packed:
    """Encode rows of x ([n, d], float32 or bfloat16, on the GPU); with `slots`
    (int64[n] on the GPU) row i goes to slot slots[i] of `out`."""
    if x.dim() != 2 or x.shape[1] != q.d or x.stride(1) != 1:
        raise ValueError("x must be [n, d] with unit column stride")
    dt = {torch.float32: L.TQ_F32, torch.bfloat16: L.TQ_BF16}[x.dtype]
    n = x.shape[0]
    if slots is not None and (slots.dtype != torch.int64 or slots.numel() != n or out is None):
        raise ValueError("slots must be int64[n] and come with an output buffer")
    out = out if out is not None else Packed(q, n, x.device)
    L.tq_encode(q.c, x.data_ptr(), dt, n, x.stride(0), out.c, _ptr(slots), _stream())
    return out


class Decoder:
    """Reusable decode-attention call for one cache shape (owns the workspace)."""

    def __init__(self, B: int, Hq: int, Hkv: int, max_ctx: int, device: str = "cuda"):
        self.B, self.Hq, self.Hkv, self.max_ctx = B, Hq, Hkv, max_ctx
        self.ws_bytes = L.tq_attn_decode_workspace(B, Hq, Hkv, max_ctx)
        if self.ws_bytes == 0:
            raise ValueError("invalid decode shape")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=torch.device(device))

    def __call__(self, kq: Quantizer, vq: Quantizer, query: torch.Tensor, kc: Packed, vc: Packed,
                 ctx_lens: torch.Tensor | None = None, scale: float | None = None,
                 out: torch.Tensor | None = None, phase: int = 0) -> torch.Tensor:
        B, Hq, d = query.shape
        if (B, Hq) != (self.B, self.Hq) or query.dtype != torch.float32 or not query.is_contiguous():
            raise ValueError("query must be contiguous float32 [B, Hq, d] of the decoder's shape")
        if ctx_lens is not None and (ctx_lens.dtype != torch.int32 or ctx_lens.numel() != B):
            raise ValueError("ctx_lens must be int32[B]")
        out = out if out is not None else torch.empty_like(query)
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        args = (kq.c, vq.c, query.data_ptr(), B, Hq, self.Hkv, _ptr(ctx_lens), self.max_ctx,
                kc.c, vc.c, scale, out.data_ptr(), self.ws.data_ptr(), self.ws_bytes, _stream())
        if phase == 0:
            L.tq_attn_decode(*args)
        else:
            L.tq_attn_decode_phase(phase, *args)
        return out

    def step(self, kq: Quantizer, vq: Quantizer, k_new: torch.Tensor, v_new: torch.Tensor,
             query: torch.Tensor, kc: Packed, vc: Packed, ctx_lens: torch.Tensor | None = None,
             scale: float | None = None, out: torch.Tensor | None = None, phase: int = 0) -> torch.Tensor:
        """One decode step: append k_new/v_new ([B, Hkv, d] or [B*Hkv, d], float32
        or bfloat16, unit column stride) at token ctx_lens[b] - 1 of each cache,
        then attend (tq_decode_step)."""
        B, Hq, d = query.shape
        if (B, Hq) != (self.B, self.Hq) or query.dtype != torch.float32 or not query.is_contiguous():
            raise ValueError("query must be contiguous float32 [B, Hq, d] of the decoder's shape")
        if ctx_lens is not None and (ctx_lens.dtype != torch.int32 or ctx_lens.numel() != B):
            raise ValueError("ctx_lens must be int32[B]")
        rows = []
        for x in (k_new, v_new):
            x2 = x.reshape(-1, x.shape[-1])
            if x2.shape != (B * self.Hkv, d) or x2.stride(1) != 1 or x.dtype != k_new.dtype:
                raise ValueError("new rows must be [B*Hkv, d] with unit column stride and one dtype")
            rows.append(x2)
        if rows[0].stride(0) != rows[1].stride(0):
            raise ValueError("k_new and v_new must share a row stride")
        dt = {torch.float32: L.TQ_F32, torch.bfloat16: L.TQ_BF16}[k_new.dtype]
        out = out if out is not None else torch.empty_like(query)
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        args = (kq.c, vq.c, rows[0].data_ptr(), rows[1].data_ptr(), dt, rows[0].stride(0), query.data_ptr(),
                B, Hq, self.Hkv, _ptr(ctx_lens), self.max_ctx, kc.c, vc.c, scale, out.data_ptr(),
                self.ws.data_ptr(), self.ws_bytes, _stream())
        if phase == 0:
            L.tq_decode_step(*args)
        else:
            L.tq_decode_step_phase(phase, *args)
        return out


def search(q: Quantizer, queries: torch.Tensor, db: Packed, k: int, n: int | None = None,
           workspace: torch.Tensor | None = None):
    """Inner-product top-k of each query row over the first n vectors of the
    packed database `db` (tq_search). Returns (scores [nq, k] float32,
    index [nq, k] int64), best first."""
    if queries.dim() != 2 or queries.dtype != torch.float32 or not queries.is_contiguous():
        raise ValueError("queries must be contiguous float32 [nq, d]")
    nq = queries.shape[0]
    n = db.n if n is None else n
    ws_bytes = L.tq_search_workspace(nq, n, k)
    if ws_bytes == 0:
        raise ValueError("invalid search sizes")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=queries.device)
    scores = torch.empty((nq, k), dtype=torch.float32, device=queries.device)
    index = torch.empty((nq, k), dtype=torch.int64, device=queries.device)
    L.tq_search(q.c, queries.data_ptr(), nq, db.c, n, k, scores.data_ptr(), index.data_ptr(),
                workspace.data_ptr(), ws_bytes, _stream())
    return scores, index


def encode_chunked(q: Quantizer, x: torch.Tensor, chunks: int, out: Packed | None = None) -> Packed:
    """Encode rows of x ([n, >= chunks·128], zero beyond each vector's length)
    as chunks of 128 coordinates (tq_encode_chunked): chunk c of row i goes to
    slot c·n + i of `out` (a Packed of chunks·n slots)."""
    if x.dim() != 2 or x.shape[1] < chunks * q.d or x.stride(1) != 1:
        raise ValueError("x must be [n, >= chunks*d] with unit column stride")
    dt = {torch.float32: L.TQ_F32, torch.bfloat16: L.TQ_BF16}[x.dtype]
    n = x.shape[0]
    out = out if out is not None else Packed(q, chunks * n, x.device)
    if out.n < chunks * n:
        raise ValueError("out holds fewer than chunks*n slots")
    L.tq_encode_chunked(q.c, x.data_ptr(), dt, n, chunks, x.stride(0), out.c, _stream())
    return out


def search_chunked(q: Quantizer, queries: torch.Tensor, db: Packed, chunks: int, k: int, n: int | None = None,
                   workspace: torch.Tensor | None = None):
    """Inner-product top-k over n chunked vectors (tq_search_chunked): queries
    are contiguous float32 [nq, chunks·128], db chunk-major. Returns
    (scores [nq, k] float32, index [nq, k] int64), best first."""
    if (queries.dim() != 2 or queries.dtype != torch.float32 or not queries.is_contiguous()
            or queries.shape[1] != chunks * q.d):
        raise ValueError("queries must be contiguous float32 [nq, chunks*d]")
    nq = queries.shape[0]
    n = db.n // chunks if n is None else n
    ws_bytes = L.tq_search_chunked_workspace(nq, n, k, chunks)
    if ws_bytes == 0:
        raise ValueError("invalid search sizes")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=queries.device)
    scores = torch.empty((nq, k), dtype=torch.float32, device=queries.device)
    index = torch.empty((nq, k), dtype=torch.int64, device=queries.device)
    L.tq_search_chunked(q.c, queries.data_ptr(), nq, chunks, db.c, n, k, scores.data_ptr(), index.data_ptr(),
                        workspace.data_ptr(), ws_bytes, _stream())
    return scores, index


def read_probe(buf: torch.Tensor, xor_out: torch.Tensor) -> None:
    """One plain read of the contiguous device tensor `buf` (tq_read_probe):
    the XOR of its 32-bit words is XORed into the int32 tensor `xor_out`."""
    if not buf.is_contiguous() or xor_out.dtype != torch.int32 or xor_out.numel() < 1:
        raise ValueError("buf must be contiguous and xor_out an int32 tensor")
    L.tq_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), xor_out.data_ptr(), _stream())
