"""The allocation-free argmax entry point (wsg_argmax_noalloc) against wsg_argmax.

(Named to be collected last: it shares nothing with the other tests, and a
failure here under ``pytest -x`` then hides none of them.)

wsg_argmax_noalloc keeps its span keys in a library-owned device array instead of a
caller workspace.  Checked through the C ABI: two calls in a row (the second on a
smaller input, so stale keys of the first call sit in the array), FP32 and FP16,
planted ties and random rows, each result equal to wsg_argmax's on the same input;
requests beyond the array's size are refused before any launch.
"""
import numpy as np
import pytest

from gpu_util import announce, gpu_available
import oracle

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _lib():
    from weight_streaming_gemv_amd import _abi
    return _abi.lib(), _abi


def _noalloc(L, abi, lg, dtype_flag, stream):
    import torch
    rows, n = lg.shape
    out = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    st = L.wsg_argmax_noalloc(dtype_flag, rows, n, lg.data_ptr(), out.data_ptr(), stream.cuda_stream)
    assert st == abi.WSG_OK, L.wsg_last_error()
    return out


def _inputs(rows, n, dtype, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, n)).astype(dtype)
    v[0, [n // 3, n - 1]] = 9.0          # a planted tie in row 0: the lower index wins
    if rows > 1:
        v[1, :] = 0.25                   # an all-equal row: index 0
    return v


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_noalloc_matches_workspace_entry_twice(dtype):
    import torch
    import weight_streaming_gemv_amd as wsg
    L, abi = _lib()
    flag = abi.WSG_F16 if dtype == np.float16 else abi.WSG_F32
    stream = torch.cuda.Stream()
    # first call: 300 rows of 151936 logits (300 * 38 = 11400 keys); second: 3 rows of 5000
    for rows, n, seed in ((300, 151936, 1), (3, 5000, 2)):
        host = _inputs(rows, n, dtype, seed)
        lg = torch.from_numpy(host).to("cuda")
        torch.cuda.synchronize()
        announce(f"noalloc argmax {np.dtype(dtype).name} rows={rows} n={n}")
        got = _noalloc(L, abi, lg, flag, stream)
        ref = wsg.argmax(lg, stream=stream)
        stream.synchronize()
        got, ref = got.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got, ref)
        assert got[0] == n // 3
        if rows > 1:
            assert got[1] == 0
        for r in (0, rows - 1):
            assert got[r] == oracle.argmax_lowest(host[r])


def test_noalloc_refuses_requests_beyond_its_scratch():
    import torch
    L, abi = _lib()
    lg = torch.zeros(16, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    # 16385 keys: one row of 16385 * 4096 logits (only the size is checked, nothing is read)
    st = L.wsg_argmax_noalloc(abi.WSG_F32, 1, 16385 * 4096, lg.data_ptr(), out.data_ptr(), None)
    assert st == abi.WSG_ERR_INVALID_ARG
    assert b"scratch" in L.wsg_last_error()
    st = L.wsg_argmax_noalloc(abi.WSG_F32, 2, 8193 * 4096, lg.data_ptr(), out.data_ptr(), None)
    assert st == abi.WSG_ERR_INVALID_ARG
