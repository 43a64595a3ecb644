"""MI355X (gfx950) weight-streaming decode engine: Python binding.

Argument marshalling only.  Every step of the decode path runs in the HIP
kernels of ``libwsg.so`` behind the C ABI of ``include/wsg.h``; PyTorch is
used to allocate device memory and to provide a stream.  Importing this
package fails if the library has not been built, and the GPU entry points
fail if no GPU is present -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import _abi
from ._abi import (WSG_F16, WSG_F32, WSG_GEMV_NONTEMPORAL, WSG_GEMV_SPLIT2, WSG_OPT_TIMED_STAGE, WSG_OPT_USE_GRAPH,
                   WSG_STAGE_ATTN, WSG_STAGE_DOWN, WSG_STAGE_GATEUP, WSG_STAGE_HEAD, WSG_STAGE_O,
                   WSG_STAGE_QKV, WsgError, check, wsg_config, wsg_host_weights)

__all__ = ["Model", "make_config", "gemv", "gemv_q4g64", "gemm_nt", "gemm_swiglu", "argmax", "WsgError", "WSG_F32", "WSG_F16",
           "WSG_STAGE_QKV", "WSG_STAGE_ATTN", "WSG_STAGE_O", "WSG_STAGE_GATEUP", "WSG_STAGE_DOWN",
           "WSG_STAGE_HEAD", "WSG_OPT_USE_GRAPH", "WSG_OPT_TIMED_STAGE", "WSG_GEMV_NONTEMPORAL", "WSG_GEMV_SPLIT2", "stream_read", "lib"]

try:
    # torch first: libwsg.so then binds to the HIP runtime torch already
    # loaded (loading the library first would bring in a second runtime,
    # under which its launches find no device)
    import torch as _torch_module  # noqa: F401
except ImportError:
    pass

lib = _abi.lib
lib()  # fail loudly at import when libwsg.so is missing


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("weight_streaming_gemv_amd needs a ROCm GPU (torch.cuda.is_available() is False)")
    return torch


def _stream_handle(stream) -> int:
    return 0 if stream is None else int(stream.cuda_stream)


# ----------------------------------------------------------------- GEMV
def gemv(W, X, rows_per_wave: int = 0, Y=None, stream=None, grid_blocks: int = 0, flags: int = 0):
    """``Y[T, M] = X[T, K] @ W[M, K]^T`` on the GPU (torch tensors, FP32 or FP16 W/X, FP32 Y)."""
    torch = _torch()
    M, K = W.shape
    T = X.shape[0]
    dt = {torch.float32: WSG_F32, torch.float16: WSG_F16}[W.dtype]
    if X.dtype != W.dtype or not (W.is_contiguous() and X.is_contiguous()):
        raise ValueError("W and X must be contiguous and share a dtype")
    if Y is None:
        Y = torch.empty((T, M), dtype=torch.float32, device=W.device)
    check(_abi.lib().wsg_gemv_ex(dt, M, K, T, rows_per_wave, grid_blocks, flags, W.data_ptr(), X.data_ptr(),
                                 Y.data_ptr(), _stream_handle(stream)))
    return Y


def gemv_q4g64(Wq, S, X, rows_per_wave: int = 0, Y=None, stream=None, grid_blocks: int = 0, flags: int = 0):
    """int4 group-64 GEMV: ``Wq`` int32/uint32 [M, K/8], ``S`` fp16 [M, K/64], ``X`` fp16 [T, K]."""
    torch = _torch()
    M = Wq.shape[0]
    K = Wq.shape[1] * 8
    T = X.shape[0]
    if Y is None:
        Y = torch.empty((T, M), dtype=torch.float32, device=Wq.device)
    check(_abi.lib().wsg_gemv_q4g64_ex(M, K, T, rows_per_wave, grid_blocks, flags, Wq.data_ptr(), S.data_ptr(),
                                       X.data_ptr(), Y.data_ptr(), _stream_handle(stream)))
    return Y


def gemm_nt(A, B, C=None, accumulate: bool = False, stream=None):
    """``C[M, N] (+)= A[M, K] @ B[N, K]^T`` on FP32 MFMA (torch FP32 device tensors)."""
    torch = _torch()
    M, K = A.shape
    N = B.shape[0]
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    check(_abi.lib().wsg_gemm_nt_f32(M, N, K, A.data_ptr(), B.data_ptr(), C.data_ptr(), int(accumulate),
                                     _stream_handle(stream)))
    return C


def gemm_swiglu(A, Wgu, ACT=None, stream=None):
    """``ACT[M, I] = silu(A @ Wg^T) * (A @ Wu^T)`` for ``Wgu = [Wg; Wu]`` ([2I, K]) on FP32 MFMA."""
    torch = _torch()
    M, K = A.shape
    I = Wgu.shape[0] // 2
    if ACT is None:
        ACT = torch.empty((M, I), dtype=torch.float32, device=A.device)
    check(_abi.lib().wsg_gemm_swiglu_f32(M, I, K, A.data_ptr(), Wgu.data_ptr(), ACT.data_ptr(), _stream_handle(stream)))
    return ACT


def argmax(logits, out=None, stream=None):
    """Lowest-index argmax of each row of ``logits`` ([rows, n] or [n], FP32 or FP16 device
    tensor) on the GPU; returns an int32 device tensor [rows] (scratch from torch)."""
    torch = _torch()
    lg = logits if logits.dim() == 2 else logits.view(1, -1)
    if not lg.is_contiguous():
        raise ValueError("logits must be contiguous")
    dt = {torch.float32: WSG_F32, torch.float16: WSG_F16}[lg.dtype]
    rows, n = lg.shape
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=lg.device)
    nb = C.c_size_t()
    check(_abi.lib().wsg_argmax_workspace_bytes(rows, n, C.byref(nb)))
    ws = torch.empty(nb.value, dtype=torch.uint8, device=lg.device)
    check(_abi.lib().wsg_argmax(dt, rows, n, lg.data_ptr(), out.data_ptr(), ws.data_ptr(), nb.value,
                                _stream_handle(stream)))
    if stream is not None:
        ws.record_stream(stream)   # the scratch stays reserved until the stream's work is done
    return out


def stream_read(buf, out=None, stream=None):
    """Read every byte of a 16-byte-aligned device tensor once (streaming reference)."""
    torch = _torch()
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=buf.device)
    check(_abi.lib().wsg_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(),
                                     _stream_handle(stream)))
    return out


# ---------------------------------------------------------------- model
def make_config(shape, max_context: int, dtype: int = WSG_F32, prefill_chunk: int = 0,
                lossless_pack: bool = False, weight_format: int = 0) -> wsg_config:
    """C config from a ``synth.ModelShape``-like object."""
    return wsg_config(shape.n_layers, shape.hidden, shape.intermediate, shape.n_q_heads, shape.n_kv_heads,
                      shape.head_dim, shape.vocab, max_context, prefill_chunk, shape.rms_eps, shape.rope_theta,
                      dtype, int(lossless_pack), int(weight_format))


def is_q4(weights: Dict[str, object]) -> bool:
    """True for int4 weight sets: each decode matrix a (words uint32, scales float16) pair."""
    return weights.get("format") == "q4g64"


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def pack_weights(cfg: wsg_config, weights: Dict[str, object]) -> np.ndarray:
    """Host packing through ``wsg_pack_weights`` (a bit-for-bit copy into the packed layout)."""
    want = np.float16 if cfg.dtype == WSG_F16 else np.float32
    keep = []

    def arr(a):
        a = np.ascontiguousarray(a)
        if a.dtype != want:
            raise ValueError(f"weight dtype {a.dtype} does not match the config dtype {np.dtype(want)}")
        keep.append(a)
        return _ptr(a)

    layers = weights["layers"]
    L = cfg.n_layers
    if len(layers) != L:
        raise ValueError("layer count mismatch")

    def plist(name):
        P = (C.c_void_p * L)(*[arr(lw[name]) for lw in layers])
        keep.append(P)
        return C.cast(P, C.POINTER(C.c_void_p))

    hw = wsg_host_weights(arr(weights["embed"]), arr(weights["final_norm"]), plist("in_norm"), plist("wq"),
                          plist("wk"), plist("wv"), plist("q_norm"), plist("k_norm"), plist("wo"),
                          plist("post_norm"), plist("wg"), plist("wu"), plist("wd"))
    n = C.c_size_t()
    check(_abi.lib().wsg_packed_weight_bytes(C.byref(cfg), C.byref(n)))
    out = np.empty(n.value, dtype=np.uint8)
    check(_abi.lib().wsg_pack_weights(C.byref(cfg), C.byref(hw), _ptr(out), n.value))
    return out


def pack_weights_q4(cfg: wsg_config, weights: Dict[str, object]) -> np.ndarray:
    """Host packing of an int4 model through ``wsg_pack_weights_q4`` (bit-for-bit copies)."""
    keep = []

    def arr(a, dt):
        a = np.ascontiguousarray(a)
        if a.dtype != dt:
            raise ValueError(f"array dtype {a.dtype}, expected {np.dtype(dt)}")
        keep.append(a)
        return _ptr(a)

    def q4(m):
        words, scales = m
        return _abi.wsg_q4_matrix(arr(words, np.uint32), arr(scales, np.float16))

    layers = weights["layers"]
    L = cfg.n_layers
    if len(layers) != L:
        raise ValueError("layer count mismatch")

    def glist(name):
        P = (C.c_void_p * L)(*[arr(lw[name], np.float16) for lw in layers])
        keep.append(P)
        return C.cast(P, C.POINTER(C.c_void_p))

    def qlist(name):
        P = (_abi.wsg_q4_matrix * L)(*[q4(lw[name]) for lw in layers])
        keep.append(P)
        return C.cast(P, C.POINTER(_abi.wsg_q4_matrix))

    none = C.POINTER(C.c_void_p)()
    norms = wsg_host_weights(None, arr(weights["final_norm"], np.float16), glist("in_norm"), none, none, none,
                             glist("q_norm"), glist("k_norm"), none, glist("post_norm"), none, none, none)
    qw = _abi.wsg_host_q4_weights(q4(weights["embed"]), qlist("wq"), qlist("wk"), qlist("wv"), qlist("wo"),
                                  qlist("wg"), qlist("wu"), qlist("wd"))
    n = C.c_size_t()
    check(_abi.lib().wsg_packed_weight_bytes(C.byref(cfg), C.byref(n)))
    out = np.empty(n.value, dtype=np.uint8)
    check(_abi.lib().wsg_pack_weights_q4(C.byref(cfg), C.byref(norms), C.byref(qw), _ptr(out), n.value))
    return out


class Model:
    """A decode model on the GPU; weights and workspace are torch device tensors it owns."""

    def __init__(self, shape, weights: Dict[str, object], max_context: int, dtype: int = WSG_F32,
                 prefill_chunk: int = 0, stream=None, packed: Optional[np.ndarray] = None,
                 lossless_pack: bool = False):
        torch = _torch()
        self.torch = torch
        self.shape = shape
        q4 = is_q4(weights)
        self.cfg = make_config(shape, max_context, dtype, prefill_chunk, lossless_pack,
                               _abi.WSG_W_Q4G64 if q4 else _abi.WSG_W_DENSE)
        self.np_dtype = np.float16 if dtype == WSG_F16 else np.float32
        self.t_dtype = torch.float16 if dtype == WSG_F16 else torch.float32
        if packed is not None:
            host = packed
        else:
            host = pack_weights_q4(self.cfg, weights) if q4 else pack_weights(self.cfg, weights)
        self.d_packed = torch.from_numpy(host).to("cuda")
        n = C.c_size_t()
        check(_abi.lib().wsg_workspace_bytes(C.byref(self.cfg), C.byref(n)))
        self.ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
        self.stream = stream if stream is not None else torch.cuda.Stream()
        torch.cuda.synchronize()
        h = C.c_void_p()
        check(_abi.lib().wsg_model_create(C.byref(self.cfg), self.d_packed.data_ptr(), self.d_packed.numel(),
                                          self.ws.data_ptr(), self.ws.numel(), _stream_handle(self.stream),
                                          C.byref(h)))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            _abi.lib().wsg_model_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- calls
    def reset(self) -> None:
        check(_abi.lib().wsg_reset_cache(self.h))

    def prefill(self, ids: Sequence[int]) -> int:
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        tok = C.c_int32()
        lp = C.c_void_p()
        check(_abi.lib().wsg_prefill(self.h, a.ctypes.data_as(C.POINTER(C.c_int32)), a.size, C.byref(tok),
                                     C.byref(lp)))
        self._logits_ptr = lp.value
        self._logits_rows = 1
        return tok.value

    def step(self, in_token: int = -1) -> int:
        tok = C.c_int32()
        lp = C.c_void_p()
        check(_abi.lib().wsg_step(self.h, int(in_token), C.byref(tok), C.byref(lp)))
        self._logits_ptr = lp.value
        self._logits_rows = 1
        return tok.value

    def generate(self, n: int) -> List[int]:
        """``n`` greedy steps from the last output, enqueued back to back with one wait
        at the end; the same tokens as ``n`` calls of ``step()``."""
        toks = (C.c_int32 * max(int(n), 1))()
        check(_abi.lib().wsg_generate(self.h, int(n), toks))
        if n > 0:
            self._logits_rows = 1
        return list(toks[:max(int(n), 0)])

    def step2(self, draft: int, in_token: int = -1) -> Tuple[Tuple[int, int], int]:
        """Two-token step: ``in_token`` (default: the last output) at p, ``draft`` at p + 1.

        Returns ((token after row 0, token after row 1), tokens emitted): 2 when the
        draft equals the first token, else 1 (the second token is then meaningless).
        """
        toks = (C.c_int32 * 2)()
        n = C.c_int32()
        lp = C.c_void_p()
        check(_abi.lib().wsg_step2(self.h, int(in_token), int(draft), toks, C.byref(n), C.byref(lp)))
        self._logits_ptr = lp.value
        self._logits_rows = 2
        return (toks[0], toks[1]), n.value

    @property
    def position(self) -> int:
        return _abi.lib().wsg_position(self.h)

    def rewind(self, pos: int) -> None:
        """Keep the first ``pos`` tokens; ``step()`` then re-processes the token at slot ``pos``."""
        check(_abi.lib().wsg_rewind(self.h, pos))

    def set_prefill_chunk(self, rows: int) -> None:
        check(_abi.lib().wsg_set_prefill_chunk(self.h, rows))

    def set_option(self, option: int, value: int) -> None:
        check(_abi.lib().wsg_set_option(self.h, option, value))

    def stage_time(self) -> Tuple[float, int, int]:
        ms, n, b = C.c_double(), C.c_int64(), C.c_int64()
        check(_abi.lib().wsg_stage_time(self.h, C.byref(ms), C.byref(n), C.byref(b)))
        return ms.value, n.value, b.value

    # -- views into the workspace (validation)
    def _view(self, ptr: int, count: int):
        off = ptr - self.ws.data_ptr()
        es = 2 if self.t_dtype == self.torch.float16 else 4
        assert 0 <= off and off + count * es <= self.ws.numel()
        return self.ws[off:off + count * es].view(self.t_dtype)

    def storage(self) -> Dict[str, int]:
        """Decode weight storage: packed matrices, decode matrices, decode weight bytes per token."""
        pk, tot, b = C.c_int32(), C.c_int32(), C.c_int64()
        check(_abi.lib().wsg_weight_storage(self.h, C.byref(pk), C.byref(tot), C.byref(b)))
        return {"packed_matrices": pk.value, "decode_matrices": tot.value, "decode_weight_bytes": b.value}

    def time_stage(self, stage: int, reps: int = 10) -> Tuple[float, int]:
        """(microseconds per launch, weight bytes per launch) of a per-layer stage, from
        ``wsg_time_stage`` (a graph of the stage's launches over all layers, replayed)."""
        us, b = C.c_double(), C.c_int64()
        check(_abi.lib().wsg_time_stage(self.h, stage, reps, C.byref(us), C.byref(b)))
        return us.value, b.value

    def describe(self) -> dict:
        """The model's launch shapes (``wsg_describe``) as a dict."""
        import json
        need = C.c_size_t()
        check(_abi.lib().wsg_describe(self.h, None, 0, C.byref(need)))
        buf = C.create_string_buffer(need.value)
        check(_abi.lib().wsg_describe(self.h, buf, need.value, C.byref(need)))
        return json.loads(buf.value.decode())

    def logits(self):
        """Last logits (device tensor view, storage dtype): [vocab] after prefill/step,
        [2, vocab] after step2."""
        rows = getattr(self, "_logits_rows", 1)
        v = self._view(self._logits_ptr, rows * self.shape.vocab)
        return v if rows == 1 else v.view(rows, self.shape.vocab)

    def kv(self, layer: int):
        """(K, V, valid_len): device views [n_kv, max_context, head_dim] with the strides
        the library reports."""
        k, v, n = C.c_void_p(), C.c_void_p(), C.c_int32()
        st = (C.c_int64 * 3)()
        check(_abi.lib().wsg_kv_view(self.h, layer, C.byref(k), C.byref(v), C.byref(n), st))
        sh = (self.shape.n_kv_heads, self.cfg.max_context, self.shape.head_dim)
        strides = tuple(st)
        cnt = (sh[0] - 1) * strides[0] + (sh[1] - 1) * strides[1] + (sh[2] - 1) * strides[2] + 1
        return (self._view(k.value, cnt).as_strided(sh, strides), self._view(v.value, cnt).as_strided(sh, strides),
                n.value)
