"""The benchmark's validation gate on the CPU: a run whose logits, K/V entries or tokens
leave the tolerance publishes no timing (Benchmark methodology, "Long-document chunked
prefill": a failed check discards the run's timings).

The "model" here is a stand-in computed by its own oracle instance, so it agrees with the
reference exactly until a slip is planted: a logit, a cached key or a token moved just past
rtol = atol = 1e-3.  Each slip must raise ValidationError from the section that checks it,
and ``bench.main`` turns that into exit status 3 with nothing on stdout.
"""
import numpy as np
import pytest
import torch

import bench
from oracle import OracleModel, argmax_lowest
from synth import MINI, model_weights, prompt_ids

TOL = 1e-3


def _past_tol(v):
    """A value moved 1.5x the allowed distance from v."""
    return v + 1.5 * (TOL + TOL * abs(v))


class OracleStub:
    """Decode-model interface of the HIP binding, computed on the CPU by an oracle, with
    one planted slip: ``slip = (kind, position, occurrence)`` fires on the given occurrence of
    a forward whose last row is at ``position``: "logit" (one logit moved past the
    tolerance), "token" (the next id returned instead of the greedy one) or "kv" (a key of
    slot position - 8 of layer 1, written long before, moved past the tolerance)."""

    def __init__(self, shape, w, cap, slip=None):
        self.o = OracleModel(shape, w, cap)
        self.shape = shape
        self.slip = slip
        self.seen = {}
        self._lg = None
        self._last = None

    def reset(self):
        self.o.reset()

    def set_prefill_chunk(self, rows):
        pass

    def close(self):
        pass

    @property
    def position(self):
        return self.o.pos

    def prefill(self, ids):
        return self._emit(self.o.forward_rows(ids))

    def step(self, in_token=-1):
        return self._emit(self.o.forward_rows([self._last if in_token < 0 else in_token]))

    def generate(self, n):
        return [self.step() for _ in range(n)]

    def _emit(self, lg):
        lg = lg.copy()
        tok = argmax_lowest(lg)
        p = self.o.pos - 1
        self.seen[p] = self.seen.get(p, 0) + 1
        if self.slip and self.slip[1] == p and self.slip[2] == self.seen[p]:
            kind = self.slip[0]
            if kind == "logit":
                i = int(np.argmin(lg))             # not the greedy token: only the logit check sees it
                lg[i] = _past_tol(float(lg[i]))
            elif kind == "token":
                tok = (tok + 1) % self.shape.vocab
            elif kind == "kv":
                self.o.k_cache[1, 0, p - 8, 5] = _past_tol(float(self.o.k_cache[1, 0, p - 8, 5]))
        self._lg, self._last = lg, tok
        return tok

    def logits(self):
        return torch.from_numpy(self._lg)

    def kv(self, layer):
        return torch.from_numpy(self.o.k_cache[layer]), torch.from_numpy(self.o.v_cache[layer]), self.o.pos


@pytest.fixture(scope="module")
def w():
    return model_weights(MINI, seed=0)


def test_validate_passes_an_exact_model(w):
    prompt = prompt_ids(2, 8, MINI.vocab)
    toks, ml, mk, _ = bench.validate(OracleStub(MINI, w, 32), OracleModel(MINI, w, 32), prompt, 8)
    assert len(toks) == 8 and ml == 0.0 and mk == 0.0


@pytest.mark.parametrize("kind,what", [("logit", "logits"), ("token", "token"), ("kv", "K ")])
def test_validate_rejects_a_slip(w, kind, what):
    prompt = prompt_ids(2, 8, MINI.vocab)
    stub = OracleStub(MINI, w, 32, slip=(kind, 11, 1))
    with pytest.raises(bench.ValidationError, match=what):
        bench.validate(stub, OracleModel(MINI, w, 32), prompt, 8)


def _long(w, slip=None):
    make = lambda cap, chunk: OracleStub(MINI, w, cap, slip)   # noqa: E731
    return bench.long_context(torch, None, MINI, w, trials=1, warmup=1, tune_len=40, held_len=48, n_out=20,
                              chunks=(16, 32), prefix_every=8, make_model=make)


def test_long_context_passes_an_exact_model(w):
    r = _long(w)
    v = r["validation"]
    assert v["oracle_checked_outputs"] == 20 and v["max_abs_logit_err"] == 0.0 and v["max_abs_kv_err"] == 0.0
    assert v["whole_prefix_checks"] == [48, 55, 63, 67]
    assert v["chunk_boundary_prefix_checks"][-1] == 48


@pytest.mark.parametrize("slip,what", [
    (("logit", 58, 1), "held-out logits at output 12"),       # a late output, in lockstep
    (("token", 60, 1), "held-out output 14: token"),
    (("kv", 60, 1), "held-out prefix at output 16"),          # an old slot: only the periodic prefix check sees it
    (("token", 50, 2), "held-out timed tokens differ"),       # the first timed run
    (("logit", 44, 1), "chunk 16 logits at output 6"),        # the chunk-selection prompt's generation
    (("kv", 46, 1), "chunk 16 prefix after 8 outputs"),     # a prompt slot, after the 8th output
    (("kv", 31, 1), "held-out chunk boundary 32"),            # a held-out prompt slot, at the next boundary
])
def test_long_context_rejects_a_slip(w, slip, what):
    with pytest.raises(bench.ValidationError, match=what):
        _long(w, slip)


def test_main_publishes_nothing_on_a_failed_check(monkeypatch, capsys):
    def failing(argv=None):
        raise bench.ValidationError("validation failed: planted")
    monkeypatch.setattr(bench, "_main", failing)
    assert bench.main([]) == 3
    assert capsys.readouterr().out == ""


def test_sweep_summary_reads_split_configurations():
    """The cold sweep's best-configuration table: keys T{T}_R{R}_G{G}, where R = "1s" is an FP32
    row over two waves; the fastest key per shape and T wins, and its rows per wave, waves per
    row and grid are read back from the key."""
    sw = {"f32_1024x3072": {"bytes": 1024 * 3072 * 4,
                            "T1_R1_G0": {"us": 7.9}, "T1_R2_G0": {"us": 4.5}, "T1_R1s_G0": {"us": 3.9},
                            "T2_R1_G0": {"us": 4.4}, "T2_R1s_G256": {"us": 4.5},
                            "ceiling": {"us": 3.3, "gbps": 1024 * 3072 * 4 / 3.3 / 1e3}},
          "q4g64_4096x4096": {"bytes": 4096 * 2048 + 4096 * 64 * 2,
                              "T1_R1_G0": {"us": 3.9}, "T1_R2_G512": {"us": 4.4}}}
    best, _ = bench.sweep_summary(sw)
    b = best["f32_1024x3072_T1"]
    assert (b["R"], b["waves_per_row"], b["grid"], b["us"]) == (1, 2, 0, 3.9)
    assert b["frac_of_stream_ceiling"] == pytest.approx(3.3 / 3.9, abs=1e-4)
    b = best["f32_1024x3072_T2"]
    assert (b["R"], b["waves_per_row"], b["grid"], b["us"]) == (1, 1, 0, 4.4)
    b = best["q4g64_4096x4096_T1"]
    assert (b["R"], b["waves_per_row"], b["grid"]) == (1, 1, 0) and "frac_of_stream_ceiling" not in b
    assert "q4g64_4096x4096_T2" not in best
