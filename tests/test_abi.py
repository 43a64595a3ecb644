"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, validates arguments and packs weights -- no GPU needed."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wsg.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(wsg_\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def abi():
    from weight_streaming_gemv_amd import _abi
    return _abi


def test_library_exports_every_declared_symbol(abi):
    L = abi.lib()
    names = declared_functions()
    assert len(names) >= 19
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(abi.EXPORTED)
    assert b"gfx950" in L.wsg_version()


def test_gemv_argument_validation(abi):
    L = abi.lib()
    # bad dtype, bad T, bad rows, null pointers, misalignment: all rejected before any launch
    assert L.wsg_gemv(7, 8, 8, 1, 1, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemv(0, 8, 8, 3, 1, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemv(0, 8, 8, 1, 3, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemv(0, 0, 8, 1, 1, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemv(0, 8, 8, 1, 1, None, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemv(0, 8, 8, 1, 1, 18, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert b"aligned" in L.wsg_last_error()
    assert L.wsg_gemv_q4g64(8, 100, 1, 1, 16, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemv_q4g64(8, 128, 1, 1, 16, 17, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    # streaming reference: null, size not a multiple of 16, misaligned buffer
    assert L.wsg_stream_read(None, 64, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_stream_read(16, 64, None, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_stream_read(16, 60, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_stream_read(16, 0, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_stream_read(24, 64, 16, None) == abi.WSG_ERR_INVALID_ARG


def _cfg(abi, shape, cap=16, dtype=0, chunk=0):
    return abi.wsg_config(shape.n_layers, shape.hidden, shape.intermediate, shape.n_q_heads,
                          shape.n_kv_heads, shape.head_dim, shape.vocab, cap, chunk, shape.rms_eps,
                          shape.rope_theta, dtype)


def test_config_validation(abi):
    from synth import MINI, QWEN3_0_6B
    L = abi.lib()
    n = C.c_size_t()
    assert L.wsg_packed_weight_bytes(C.byref(_cfg(abi, MINI)), C.byref(n)) == 0
    bad = _cfg(abi, MINI)
    bad.head_dim = 64
    assert L.wsg_packed_weight_bytes(C.byref(bad), C.byref(n)) == abi.WSG_ERR_UNSUPPORTED
    bad = _cfg(abi, MINI)
    bad.n_kv_heads = 3
    assert L.wsg_packed_weight_bytes(C.byref(bad), C.byref(n)) == abi.WSG_ERR_INVALID_ARG
    bad = _cfg(abi, MINI, dtype=5)
    assert L.wsg_workspace_bytes(C.byref(bad), C.byref(n)) == abi.WSG_ERR_INVALID_ARG
    bad = _cfg(abi, MINI, chunk=5000)
    assert L.wsg_workspace_bytes(C.byref(bad), C.byref(n)) == abi.WSG_ERR_INVALID_ARG
    # packed bytes of the 28-layer FP32 model: the weights plus norm gains, 256-byte aligned
    assert L.wsg_packed_weight_bytes(C.byref(_cfg(abi, QWEN3_0_6B)), C.byref(n)) == 0
    assert QWEN3_0_6B.weight_bytes_per_token(4) <= n.value < QWEN3_0_6B.weight_bytes_per_token(4) + 2 ** 20
    # workspace holds at least the KV cache
    assert L.wsg_workspace_bytes(C.byref(_cfg(abi, QWEN3_0_6B, cap=5120)), C.byref(n)) == 0
    assert n.value >= 28 * 2 * 8 * 5120 * 128 * 4


def test_model_create_rejects_bad_buffers(abi):
    from synth import MINI
    L = abi.lib()
    h = C.c_void_p()
    cfg = _cfg(abi, MINI)
    assert L.wsg_model_create(C.byref(cfg), None, 0, None, 0, None, C.byref(h)) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_model_create(C.byref(cfg), 256, 10, 512, 10, None, C.byref(h)) == abi.WSG_ERR_INVALID_ARG
    assert b"packed buffer" in L.wsg_last_error()
    assert L.wsg_model_create(C.byref(cfg), 100, 1 << 40, 512, 1 << 40, None, C.byref(h)) == abi.WSG_ERR_INVALID_ARG
    assert b"aligned" in L.wsg_last_error()


def test_pack_weights_layout_is_bit_copy(abi):
    """The packer concatenates Wq|Wk|Wv and Wg|Wu and copies every value bit for bit."""
    from synth import MINI, model_weights
    from weight_streaming_gemv_amd import pack_weights
    sh = MINI.with_layers(1)
    w = model_weights(sh, seed=3)
    cfg = _cfg(abi, sh)
    img = pack_weights(cfg, w)
    f = img.view(np.float32)
    E = w["embed"].reshape(-1)
    assert np.array_equal(f[:E.size], E)        # embedding first
    lw = w["layers"][0]
    qkv = np.concatenate([lw["wq"], lw["wk"], lw["wv"]]).reshape(-1)
    gu = np.concatenate([lw["wg"], lw["wu"]]).reshape(-1)
    for block in (qkv, gu, lw["wo"].reshape(-1), lw["wd"].reshape(-1)):
        # each block appears contiguously at a 256-byte aligned offset
        starts = np.flatnonzero(f == block[0])
        assert any((s * 4) % 256 == 0 and np.array_equal(f[s:s + block.size], block) for s in starts)
    with pytest.raises(Exception):
        pack_weights(cfg, model_weights(sh, seed=3, dtype=np.float16))
