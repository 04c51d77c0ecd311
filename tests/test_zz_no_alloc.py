"""qmm_gemv_argmax_noalloc: the greedy argmax with its scratch in the
library's static device array instead of a caller's work buffer.

Through the C ABI, against qmm_gemv_argmax (the same kernels with a work
buffer): the index and the value bits must be equal.  Two calls in a row,
the second with a smaller matrix (fewer workgroup candidates, so stale slots
of the first call stay in the array and must not be read), for several
dtypes and for the int8-free f32 path; then the first shape again.
"""
import numpy as np
import pytest
import torch

import gguf_block_quant_qmm_amd as q
from qmm_inputs import make_blob, make_x, rng_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def with_work(dt, bd, M, K, xd):
    work = torch.empty(q.QMM_ARGMAX_WORK_BYTES, dtype=torch.uint8, device="cuda")
    idx = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    val = torch.full((1,), float("nan"), device="cuda")
    q.qmm_gemv_argmax(bd, dt, M, K, xd, work, idx, val)
    torch.cuda.synchronize()
    return int(idx.item()), val.cpu().numpy().view(np.uint32)[0]


def no_alloc(dt, bd, M, K, xd):
    idx = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    val = torch.full((1,), float("nan"), device="cuda")
    q.qmm_gemv_argmax_noalloc(bd, dt, M, K, xd, idx, val)
    torch.cuda.synchronize()
    return int(idx.item()), val.cpu().numpy().view(np.uint32)[0]


# (dtype, [(M, K) of successive calls]): the second call is smaller; the
# 128256-row head gives the most workgroup candidates
CASES = [
    (q.QMM_Q6_K, [(128256, 4096), (3001, 4096), (128256, 4096)]),
    (q.QMM_Q4_0, [(40001, 4096), (77, 4096)]),
    (q.QMM_Q4_K, [(14336, 8192), (300, 8192)]),
    (q.QMM_Q8_0, [(20000, 2048), (9, 2048)]),
]


@pytest.mark.parametrize("dt,calls", CASES, ids=lambda v: str(v) if isinstance(v, int) else "")
def test_noalloc_matches_work_buffer_form(dt, calls):
    for c, (M, K) in enumerate(calls):
        blob = make_blob(dt, M, K, rng_for(1400 + dt, c))
        x = make_x(1, K, rng_for(1400 + dt, 100 + c))
        bd, xd = to_dev(blob), to_dev(x.reshape(-1))
        got = no_alloc(dt, bd, M, K, xd)
        want = with_work(dt, bd, M, K, xd)
        assert got == want, f"dtype {dt} call {c} M={M} K={K}: no-alloc {got}, with work buffer {want}"
        assert 0 <= got[0] < M


def test_noalloc_value_optional_and_rejects():
    dt, M, K = q.QMM_Q4_0, 513, 4096
    blob = make_blob(dt, M, K, rng_for(1450, 0))
    x = make_x(1, K, rng_for(1450, 1))
    bd, xd = to_dev(blob), to_dev(x.reshape(-1))
    idx = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    q.qmm_gemv_argmax_noalloc(bd, dt, M, K, xd, idx)  # value = NULL
    torch.cuda.synchronize()
    assert int(idx.item()) == with_work(dt, bd, M, K, xd)[0]
    L = q.lib()
    assert L.qmm_gemv_argmax_noalloc(bd.data_ptr(), dt, M, K, 0, idx.data_ptr(), None, None) == q.QMM_ERR_NULL
    assert L.qmm_gemv_argmax_noalloc(bd.data_ptr(), dt, M, K, xd.data_ptr() + 4, idx.data_ptr(), None,
                                     None) == q.QMM_ERR_ALIGN
    assert L.qmm_gemv_argmax_noalloc(bd.data_ptr(), dt, M, 96, xd.data_ptr(), idx.data_ptr(), None,
                                     None) == q.QMM_ERR_SHAPE
