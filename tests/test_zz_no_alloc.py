"""The allocation-free Q8_0 linear (qwen3_q8_0_linear_noalloc) against the
entry point it varies (qwen3_q8_0_linear, caller scratch), through the C ABI.

Both run the same kernels on the same rows, so their outputs are bitwise
equal; both are also within one f32 ulp of the oracle's exact sum rounded
once ("Model files and quantization", section 11.9).  Two calls in a row,
the second smaller, show the fixed scratch is rewritten, not reused stale;
a size over the limit is refused before any launch."""

import ctypes as C

import numpy as np
import pytest
import torch

from oracle import q8_0 as oq
from synthetic import gen_normal_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _ulps(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def _weights(n, k, seed):
    from quantized_q8_dequant_amd import encode_q8_0, repack_q8_0

    w = gen_normal_rows((n, k), seed=seed, scale=0.02)
    qs, sc = repack_q8_0(encode_q8_0(torch.from_numpy(w).to(DEV)), n, k)
    return oq.Q8Weight(w), qs, sc


def _noalloc(x, qs, sc):
    from quantized_q8_dequant_amd import _lib
    from quantized_q8_dequant_amd.model import _stream

    m, k = x.shape
    n = qs.shape[0]
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    rc = _lib.lib().qwen3_q8_0_linear_noalloc(
        x.data_ptr(), m, k, qs.data_ptr(), sc.data_ptr(), n, y.data_ptr(), _stream()
    )
    _lib.check(rc)
    return y


# (m, k, n): the MFMA GEMM path, then a smaller small-M GEMM call, then one
# row (the GEMV, which needs no scratch), then the GEMM again
CASES = [(300, 3072, 512), (20, 1024, 384), (1, 2048, 1000), (130, 1024, 256)]


def test_noalloc_linear_equals_the_scratch_taking_entry():
    from quantized_q8_dequant_amd import q8_0_linear

    outs = []
    for i, (m, k, n) in enumerate(CASES):
        x = torch.from_numpy(gen_normal_rows((m, k), seed=900 + i)).to(DEV)
        ow, qs, sc = _weights(n, k, seed=910 + i)
        y = _noalloc(x, qs, sc)
        outs.append((x, ow, qs, sc, y))
    torch.cuda.synchronize()
    for x, ow, qs, sc, y in outs:
        want = q8_0_linear(x, qs, sc)
        assert torch.equal(y, want), "differs from qwen3_q8_0_linear"
        ref = oq.linear(x.cpu().numpy(), ow)
        u = _ulps(y.cpu().numpy(), ref)
        assert u.max() <= 1 and (u == 0).mean() >= 0.999


def test_noalloc_linear_refuses_sizes_over_the_limit():
    from quantized_q8_dequant_amd import _lib

    L = _lib.lib()
    limit = 16 << 20
    m, k = 8192, 2048  # 8192 * 2048 * 1.125 bytes > 16 MiB
    assert L.qwen3_linear_work_bytes(m, k) > limit
    y = torch.empty(1, dtype=torch.float32, device=DEV)
    rc = L.qwen3_q8_0_linear_noalloc(0x1000, m, k, 0x2000, 0x3000, 64, y.data_ptr(), None)
    assert rc == -1 and "scratch" in _lib.last_error()
    # the largest size that fits still runs
    m_ok = 64
    assert L.qwen3_linear_work_bytes(m_ok, 12288) <= limit
