"""Plain forward pass of the Qwen3-0.6B-shaped decoder with a KV cache.

Test infrastructure (see the package docstring).  The structure follows
Megakernels, "What runs in the DSL" (the layer recipe) and "GPU-wide
end-to-end generation" (the eight stages per layer, each stage's output
stored in the model dtype):

  1 input RMSNorm            a   = rms(x, g_in)
  2 QKV projection           q,k,v = Wq a, Wk a, Wv a
  3 Q/K norm + RoPE + cache  q_h = rope(rms(q_h, g_q)), k_j = rope(rms(k_j, g_k)),
                             K[j][p] = k_j, V[j][p] = v_j
  4 attention                o_h = softmax(q_h K_j^T / sqrt(D)) V_j, j = h // group
  5 output proj + residual   x = x + Wo o
  6 post-attention RMSNorm   b = rms(x, g_post)
  7 gate/up + SwiGLU         act = silu(Wg b) * (Wu b)
  8 down proj + residual     x = x + Wd act
  then h = rms(x, g_f) and logits = E h (tied head), token = lowest argmax.

Int4 weights: a weight set with ``format`` "q4g64" gives each decode matrix
(and the tied embedding) as int4 words and FP16 group scales; the oracle
dequantises them once on the CPU to the exact values q * s (Our Kernel
Benchmark Was Measuring the System Cache, "Summary": 4-bit weights) and
then runs the same forward pass.  The embedding gather stores q * s in the
model dtype, like every stage output; the head multiplies by the exact
values.

Rows: ``forward_rows`` runs a block of consecutive positions as one causal
row matrix per layer.  Each row's arithmetic is the same as running the
positions one at a time (the pages' chunked prefill keeps each row's full
causal prefix), and a single-row call is one decode step.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from .gemv import dequant_q4g64
from .prims import (argmax_lowest, gqa_attention, rms_norm, rope_angles, rope_apply,
                    silu, store)

F64 = np.float64


class OracleModel:
    """Float64-reduction, storage-rounded reference decoder.

    ``shape`` is a ``synth.ModelShape``; ``weights`` the dict from
    ``synth.model_weights`` (its arrays' dtype is the storage dtype unless
    ``dtype`` is given).  ``max_context`` sizes the KV cache.
    """

    def __init__(self, shape, weights: Dict[str, object], max_context: int,
                 dtype: Optional[np.dtype] = None):
        self.shape = shape
        q4 = weights.get("format") == "q4g64"
        self.dtype = np.dtype(dtype if dtype is not None else weights["final_norm" if q4 else "embed"].dtype)
        self.cap = int(max_context)

        def mat(v):
            """A stored matrix as float64: exact int4 values q * s, or the stored dense values."""
            if q4:
                words, scales = v
                return dequant_q4g64(words, scales, 8 * np.asarray(words).shape[1]).astype(F64)
            return np.asarray(v, dtype=self.dtype).astype(F64)

        # float64 copies of the stored weights, made once (setup, untimed)
        self.E64 = mat(weights["embed"])
        self.E = store(self.E64, self.dtype)          # the gathered rows, as stored
        self.g_f = np.asarray(weights["final_norm"], dtype=self.dtype).astype(F64)
        self.layers: List[Dict[str, np.ndarray]] = []
        for lw in weights["layers"]:
            self.layers.append({k: (mat(v) if k.startswith("w") else np.asarray(v, dtype=self.dtype).astype(F64))
                                for k, v in lw.items()})
        L, hkv, d = shape.n_layers, shape.n_kv_heads, shape.head_dim
        self.k_cache = np.zeros((L, hkv, self.cap, d), dtype=self.dtype)
        self.v_cache = np.zeros((L, hkv, self.cap, d), dtype=self.dtype)
        # float64 copies of the stored cache entries (exact), written with them, so
        # attention does not widen the whole prefix again at every step
        self._k64 = np.zeros((L, hkv, self.cap, d), dtype=F64)
        self._v64 = np.zeros((L, hkv, self.cap, d), dtype=F64)
        self.pos = 0

    def reset(self) -> None:
        """Empty the cache (valid length 0); stale slots are never read."""
        self.pos = 0

    def forward_rows(self, ids, want_logits: bool = True) -> Optional[np.ndarray]:
        """Process tokens ``ids`` at positions pos .. pos+n-1 and advance.

        Returns the logits of the last row (storage dtype) if ``want_logits``;
        earlier rows skip the final norm and vocabulary projection, as the
        pages' prefill does.
        """
        sh, dt = self.shape, self.dtype
        ids = np.asarray(ids, dtype=np.int64).reshape(-1)
        n = ids.size
        if n == 0:
            raise ValueError("empty row block")
        if np.any(ids < 0) or np.any(ids >= sh.vocab):
            raise ValueError("token id out of range")
        p0 = self.pos
        if p0 + n > self.cap:
            raise ValueError("context capacity exceeded")
        positions = np.arange(p0, p0 + n)
        hq, hkv, d = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
        ang = rope_angles(positions, d, sh.rope_theta)[:, None, :]      # [n, 1, D/2]
        eps = sh.rms_eps

        x = self.E[ids]                                                 # [n, H] stored
        for l, w in enumerate(self.layers):
            a = store(rms_norm(x, w["in_norm"], eps), dt)               # stage 1
            a64 = a.astype(F64)
            q = store(a64 @ w["wq"].T, dt).reshape(n, hq, d)            # stage 2
            k = store(a64 @ w["wk"].T, dt).reshape(n, hkv, d)
            v = store(a64 @ w["wv"].T, dt).reshape(n, hkv, d)
            q = store(rope_apply(rms_norm(q, w["q_norm"], eps), ang), dt)   # stage 3
            k = store(rope_apply(rms_norm(k, w["k_norm"], eps), ang), dt)
            self.k_cache[l, :, p0:p0 + n] = np.transpose(k, (1, 0, 2))
            self.v_cache[l, :, p0:p0 + n] = np.transpose(v, (1, 0, 2))
            self._k64[l, :, p0:p0 + n] = self.k_cache[l, :, p0:p0 + n]
            self._v64[l, :, p0:p0 + n] = self.v_cache[l, :, p0:p0 + n]
            o = store(gqa_attention(q, self._k64[l], self._v64[l], positions), dt)  # stage 4
            o64 = o.reshape(n, hq * d).astype(F64)
            x = store(x.astype(F64) + o64 @ w["wo"].T, dt)              # stage 5
            b = store(rms_norm(x, w["post_norm"], eps), dt)             # stage 6
            b64 = b.astype(F64)
            act = store(silu(b64 @ w["wg"].T) * (b64 @ w["wu"].T), dt)  # stage 7
            x = store(x.astype(F64) + act.astype(F64) @ w["wd"].T, dt)  # stage 8
        self.pos = p0 + n
        if not want_logits:
            return None
        h = store(rms_norm(x[-1], self.g_f, eps), dt)
        return store(self.E64 @ h.astype(F64), dt)

    def logits_margin(self, logits) -> float:
        """Top-1 minus top-2 logit (how close the greedy choice was to a tie)."""
        v = np.sort(np.asarray(logits, dtype=F64))
        return float(v[-1] - v[-2])

    def generate(self, prompt, n_out: int, record: bool = False):
        """Greedy generation: reset, prefill ``prompt``, then ``n_out`` tokens.

        The first output comes from the last prompt row; each later output is
        one single-row forward of the previous output (EOS ignored).  With
        ``record`` the per-output logits are returned too.
        """
        self.reset()
        logits = self.forward_rows(prompt)
        out, rec = [argmax_lowest(logits)], [logits]
        for _ in range(1, n_out):
            logits = self.forward_rows([out[-1]])
            out.append(argmax_lowest(logits))
            rec.append(logits)
        return (out, rec) if record else out
