"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np

import oracle

U32 = 2.0 ** -24   # FP32 unit roundoff


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash still says what ran."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def gemv_bound(abs_prod_sum: np.ndarray, k: int, factor: float = 2.0) -> np.ndarray:
    """Rigorous summation bound gamma_n * sum|w x| for an n-term FP32 dot product (any order)."""
    n = factor * (k + 2)
    gamma = n * U32 / (1 - n * U32)
    return gamma * abs_prod_sum + 1e-30


def close_rel(got, ref, rtol, atol):
    """Elementwise |got - ref| <= atol + rtol |ref|, a non-finite value never passing;
    returns (ok, max_abs_err, worst_index)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    err = np.abs(g - r)
    lim = atol + rtol * np.abs(r)
    bad = ~(err <= lim)            # NaN compares false: counted as bad
    if not err.size:
        return True, 0.0, -1
    worst = int(np.argmax(np.where(np.isnan(err), np.inf, err - lim)))
    return (not bad.any()), float(np.nanmax(err) if not np.isnan(err).all() else np.nan), worst


def _np(t):
    return t.float().cpu().numpy()


class Checker:
    def __init__(self, model, orc, rtol, atol, label):
        self.m, self.o, self.rtol, self.atol, self.label = model, orc, rtol, atol, label
        self.max_logit_err = 0.0
        self.max_kv_err = 0.0

    def logits(self, ref, step):
        ok, err, worst = close_rel(_np(self.m.logits()), ref, self.rtol, self.atol)
        self.max_logit_err = max(self.max_logit_err, err)
        assert ok, f"{self.label} step {step}: logits off by {err:.3e} at {worst}"

    def kv(self, lo, hi, step):
        for l in range(self.o.shape.n_layers):
            k, v, n = self.m.kv(l)
            assert n == self.o.pos, (n, self.o.pos)
            for got, ref, nm in ((k, self.o.k_cache[l], "K"), (v, self.o.v_cache[l], "V")):
                ok, err, worst = close_rel(_np(got[:, lo:hi]), ref[:, lo:hi], self.rtol, self.atol)
                self.max_kv_err = max(self.max_kv_err, err)
                assert ok, f"{self.label} step {step}: layer {l} {nm}[{lo}:{hi}] off by {err:.3e}"


def lockstep(model, orc, prompt, n_out, rtol=1e-3, atol=1e-3, teacher=False, label=""):
    """Generate on both sides; returns (gpu tokens, oracle tokens, checker)."""
    ck = Checker(model, orc, rtol, atol, label)
    model.reset()
    orc.reset()
    announce(f"{label}: prefill {len(prompt)} rows")
    tok = model.prefill(prompt)
    ref = orc.forward_rows(prompt)
    rtok = oracle.argmax_lowest(ref)
    ck.logits(ref, 0)
    ck.kv(0, orc.pos, 0)
    toks, rtoks = [tok], [rtok]
    if not teacher:
        assert tok == rtok, (f"{label}: first token {tok} != {rtok} (oracle margin {orc.logits_margin(ref):.3e}; "
                             f"argmax of the GPU logits {int(np.argmax(_np(model.logits())))})")
    for s in range(1, n_out):
        p = orc.pos
        tok = model.step(rtoks[-1] if teacher else -1)
        ref = orc.forward_rows([rtoks[-1]])
        rtok = oracle.argmax_lowest(ref)
        ck.logits(ref, s)
        ck.kv(p, p + 1, s)
        if not teacher:
            assert tok == rtok, (f"{label}: step {s} token {tok} != {rtok} (margin {orc.logits_margin(ref):.3e}; "
                                 f"argmax of the GPU logits {int(np.argmax(_np(model.logits())))})")
        toks.append(tok)
        rtoks.append(rtok)
    ck.kv(0, orc.pos, n_out)
    return toks, rtoks, ck


