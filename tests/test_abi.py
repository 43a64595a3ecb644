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
    # launch flags: unknown bits, and the two-waves-per-row form outside FP32, one row per wave,
    # K in {1024, 2048, 3072}; a valid split request gets past the flag checks (to the null pointer)
    split = abi.WSG_GEMV_SPLIT2
    assert L.wsg_gemv_ex(0, 8, 1024, 1, 1, 0, 4, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert b"unknown flags" in L.wsg_last_error()
    for dt, R, K in ((1, 1, 1024), (0, 2, 1024), (0, 1, 4096), (0, 1, 512)):
        assert L.wsg_gemv_ex(dt, 8, K, 1, R, 0, split, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
        assert b"WSG_GEMV_SPLIT2" in L.wsg_last_error()
    assert L.wsg_gemv_ex(0, 8, 3072, 2, 0, 0, split | 1, None, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert b"null pointer" in L.wsg_last_error()
    assert L.wsg_gemv_q4g64_ex(8, 128, 1, 1, 0, 2, 16, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert b"unknown flags" in L.wsg_last_error()
    # streaming reference: null, size not a multiple of 16, misaligned buffer
    assert L.wsg_stream_read(None, 64, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_stream_read(16, 64, None, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_stream_read(16, 60, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_stream_read(16, 0, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_stream_read(24, 64, 16, None) == abi.WSG_ERR_INVALID_ARG
    # matrix-core products: bad shapes, null and misaligned pointers
    assert L.wsg_gemm_nt_f32(4, 48, 64, 16, 16, 16, 0, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemm_nt_f32(4, 64, 64, 16, 16, 16, 2, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemm_nt_f32(4, 64, 64, 16, None, 16, 0, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemm_swiglu_f32(0, 64, 64, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemm_swiglu_f32(4, 48, 64, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemm_swiglu_f32(4, 64, 48, 16, 16, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemm_swiglu_f32(4, 64, 64, 16, 16, None, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_gemm_swiglu_f32(4, 64, 64, 16, 20, 16, None) == abi.WSG_ERR_INVALID_ARG
    assert b"aligned" in L.wsg_last_error()


def test_argmax_argument_validation(abi):
    L = abi.lib()
    n = C.c_size_t()
    assert L.wsg_argmax_workspace_bytes(2, 151936, C.byref(n)) == 0
    assert n.value == 2 * 38 * 8                       # one key per 4096 logits and row
    assert L.wsg_argmax_workspace_bytes(1, 1, C.byref(n)) == 0 and n.value == 8
    assert L.wsg_argmax_workspace_bytes(0, 8, C.byref(n)) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax_workspace_bytes(1, 0, C.byref(n)) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax_workspace_bytes(1, (1 << 30) + 1, C.byref(n)) == abi.WSG_ERR_INVALID_ARG
    # bad dtype, sizes, null / misaligned pointers, small workspace: rejected before any launch
    assert L.wsg_argmax(2, 1, 8, 16, 16, 16, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(0, 0, 8, 16, 16, 16, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(0, 1, 0, 16, 16, 16, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(0, 1, 8, None, 16, 16, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(0, 1, 8, 16, None, 16, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(0, 1, 8, 18, 16, 16, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(1, 1, 8, 17, 16, 16, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(0, 1, 8, 16, 16, None, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(0, 1, 8, 16, 16, 20, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(0, 2, 8, 16, 16, 16, 8, None) == abi.WSG_ERR_INVALID_ARG
    assert b"workspace" in L.wsg_last_error()


def _cfg(abi, shape, cap=16, dtype=0, chunk=0, pack=0):
    return abi.wsg_config(shape.n_layers, shape.hidden, shape.intermediate, shape.n_q_heads,
                          shape.n_kv_heads, shape.head_dim, shape.vocab, cap, chunk, shape.rms_eps,
                          shape.rope_theta, dtype, pack)


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
    bad = _cfg(abi, MINI, pack=2)
    assert L.wsg_packed_weight_bytes(C.byref(bad), C.byref(n)) == abi.WSG_ERR_INVALID_ARG
    bad = _cfg(abi, MINI, dtype=1, pack=1)
    assert L.wsg_packed_weight_bytes(C.byref(bad), C.byref(n)) == abi.WSG_ERR_UNSUPPORTED
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


def test_model_calls_reject_null(abi):
    """Model entry points validate their pointers before touching the device."""
    L = abi.lib()
    toks = (C.c_int32 * 2)()
    n = C.c_int32()
    lp = C.c_void_p()
    assert L.wsg_step2(None, -1, 0, toks, C.byref(n), C.byref(lp)) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_step(None, -1, C.byref(n), C.byref(lp)) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_generate(None, 4, toks) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_rewind(None, 0) == abi.WSG_ERR_INVALID_ARG
    assert L.wsg_position(None) == -1
    k, v = C.c_void_p(), C.c_void_p()
    st = (C.c_int64 * 3)()
    assert L.wsg_kv_view(None, 0, C.byref(k), C.byref(v), C.byref(n), st) == abi.WSG_ERR_INVALID_ARG
    need = C.c_size_t()
    assert L.wsg_describe(None, None, 0, C.byref(need)) == abi.WSG_ERR_INVALID_ARG
    us, b = C.c_double(), C.c_int64()
    assert L.wsg_time_stage(None, 3, 1, C.byref(us), C.byref(b)) == abi.WSG_ERR_INVALID_ARG


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


def _align256(v):
    return (v + 255) & ~255


def _lossless_image(abi, shape, w):
    """(packed image, offset of the lossless header) for weights w."""
    from weight_streaming_gemv_amd import pack_weights
    n0 = C.c_size_t()
    assert abi.lib().wsg_packed_weight_bytes(C.byref(_cfg(abi, shape)), C.byref(n0)) == 0
    img = pack_weights(_cfg(abi, shape, pack=1), w)
    return img, n0.value   # the lossless region follows the FP32 image


def _flags(img, hdr, shape):
    magic, count = np.frombuffer(img[hdr:hdr + 8].tobytes(), dtype=np.uint32)
    assert magic == 0x50475357 and count == 1 + 4 * shape.n_layers
    return img[hdr + 8:hdr + 8 + count]


def test_lossless_pack_eligible_weights(abi):
    """BF16-representable FP32 weights: every decode matrix gets a packed copy holding the
    high 16 bits of each value (Megakernels, "Lossless decode-weight storage")."""
    from synth import MINI, model_weights_bf16
    sh = MINI.with_layers(2)
    w = model_weights_bf16(sh, seed=3)
    img, hdr = _lossless_image(abi, sh, w)
    assert list(_flags(img, hdr, sh)) == [1] * (1 + 4 * sh.n_layers)
    n = C.c_size_t()
    assert abi.lib().wsg_packed_weight_bytes(C.byref(_cfg(abi, sh, pack=1)), C.byref(n)) == 0
    assert n.value == img.size
    # the packed embedding follows the header: element i = high half of E's i-th FP32 value
    e_off = _align256(hdr + 8 + 1 + 4 * sh.n_layers)
    E = w["embed"].reshape(-1)
    got = np.frombuffer(img[e_off:e_off + 2 * E.size].tobytes(), dtype=np.uint16)
    assert np.array_equal(got, (E.view(np.uint32) >> 16).astype(np.uint16))
    # reconstruction is exact
    assert np.array_equal((got.astype(np.uint32) << 16).view(np.float32), E)


def test_lossless_pack_ineligible_weights(abi):
    """Plain FP32 weights (nonzero low bits), a single stray low bit, or a non-finite
    value keep FP32 storage for that matrix only."""
    from synth import MINI, model_weights, model_weights_bf16
    sh = MINI.with_layers(2)
    img, hdr = _lossless_image(abi, sh, model_weights(sh, seed=3))
    assert list(_flags(img, hdr, sh)) == [0] * (1 + 4 * sh.n_layers)
    w = model_weights_bf16(sh, seed=3)
    wk = w["layers"][1]["wk"].copy()
    wk.view(np.uint32)[3, 7] |= 1           # layer 1 W_qkv
    w["layers"][1]["wk"] = wk
    wd = w["layers"][0]["wd"].copy()
    wd[5, 5] = np.inf                        # layer 0 W_d
    w["layers"][0]["wd"] = wd
    img, hdr = _lossless_image(abi, sh, w)
    # order: embedding, then per layer W_qkv, W_o, W_gu, W_d
    assert list(_flags(img, hdr, sh)) == [1, 1, 1, 1, 0, 0, 1, 1, 1]


def test_bf16_rounding_matches_torch():
    """The synthetic BF16-representable weights use round-to-nearest-even, as torch's
    float32 -> bfloat16 conversion does (ties included)."""
    import torch
    from synth import bf16_representable
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * 0.02).astype(np.float32)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 1.5 * 2 ** -8], np.float32)
    a = np.concatenate([a, ties])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    got = bf16_representable(a)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert not np.any(got.view(np.uint32) & 0xFFFF)


def _q4_cfg(abi, shape, cap=16, dtype=1, chunk=0):
    c = _cfg(abi, shape, cap=cap, dtype=dtype, chunk=chunk)
    c.weight_format = abi.WSG_W_Q4G64
    return c


def test_q4_config_validation(abi):
    from synth import MINI, ModelShape
    L = abi.lib()
    n = C.c_size_t()
    sh = ModelShape(n_layers=1, hidden=1024, intermediate=2048, n_q_heads=8, n_kv_heads=4, head_dim=128, vocab=50)
    assert L.wsg_packed_weight_bytes(C.byref(_q4_cfg(abi, sh)), C.byref(n)) == abi.WSG_OK
    # int4 rows: k/2 bytes of words + k/32 bytes of scales
    rb = lambda k: k // 2 + k // 32
    al = lambda v: (v + 255) // 256 * 256
    exp = al(50 * rb(1024)) + al(1024 * 2)
    exp += 2 * al(1024 * 2) + 2 * al(128 * 2)
    exp += al((1024 + 2 * 512) * rb(1024)) + al(1024 * rb(1024)) + al(2 * 2048 * rb(1024)) + al(1024 * rb(2048))
    assert n.value == exp
    assert L.wsg_packed_weight_bytes(C.byref(_q4_cfg(abi, sh, dtype=0)), C.byref(n)) == abi.WSG_ERR_UNSUPPORTED
    assert b"FP16" in L.wsg_last_error()
    assert L.wsg_packed_weight_bytes(C.byref(_q4_cfg(abi, MINI)), C.byref(n)) == abi.WSG_ERR_UNSUPPORTED
    bad = _q4_cfg(abi, sh)
    bad.weight_format = 7
    assert L.wsg_packed_weight_bytes(C.byref(bad), C.byref(n)) == abi.WSG_ERR_INVALID_ARG


def test_q4_pack_layout_is_row_interleaved_copy(abi):
    """Each packed int4 row is the row's words followed by its scales, bit for bit;
    W_qkv stacks wq, wk, wv and W_gu stacks wg, wu; the dense packer refuses int4."""
    from synth import ModelShape, model_weights_q4
    from weight_streaming_gemv_amd import pack_weights, pack_weights_q4
    sh = ModelShape(n_layers=1, hidden=1024, intermediate=1024, n_q_heads=8, n_kv_heads=4, head_dim=128, vocab=40)
    w = model_weights_q4(sh, seed=2)
    cfg = _q4_cfg(abi, sh)
    img = pack_weights_q4(cfg, w)
    rb = 1024 // 2 + 1024 // 32

    def row(off, r):
        return img[off + r * rb: off + (r + 1) * rb]

    def expect(m, r):
        return np.concatenate([m[0][r].view(np.uint8), m[1][r].view(np.uint8)])

    E = w["embed"]
    for r in (0, 17, 39):
        assert np.array_equal(row(0, r), expect(E, r))
    al = lambda v: (v + 255) // 256 * 256
    off = al(40 * rb)
    assert np.array_equal(img[off:off + 2048].view(np.float16), w["final_norm"])
    off += al(2048) + 2 * al(2048) + 2 * al(256)          # final_norm, in/post norm, q/k norm
    lw = w["layers"][0]
    for r, (m, rr) in {0: (lw["wq"], 0), 1023: (lw["wq"], 1023), 1024: (lw["wk"], 0),
                       1536: (lw["wv"], 0), 2047: (lw["wv"], 511)}.items():
        assert np.array_equal(row(off, r), expect(m, rr))
    from synth import model_weights
    with pytest.raises(Exception, match="INVALID_ARG"):
        pack_weights(cfg, model_weights(sh, seed=2, dtype=np.float16))   # int4 config, dense packer
