"""Kernel-boundary parity of the HIP library against the CPU oracle.

Bit-exact: the Q8_0 encoder (codes and f16 scales), the repack, the
activation quantisation inside the linears and every integer block dot.
Within one f32 ulp: the Q8_0 linear (GEMV for one row, the small-M GEMM for
2-64 rows, the MFMA GEMM for more).  Every kernel widens each block term
d_w * d_a * S exactly to f64, sums in f64 and rounds once, as the oracle
does ("Model files and quantization", section 11.9, the block dot and its
rescale); only the f64 summation order differs, so a result can leave the
oracle's only by an f32 rounding that the f64 sums land on opposite sides
of.  A wrong integer dot or a dropped block moves a result by far more.
"""

import numpy as np
import pytest
import torch

from oracle import q8_0 as oq
from synthetic import gen_normal_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _special_rows(k):
    rows = [np.zeros(k, np.float32)]
    spike = np.zeros(k, np.float32)
    spike[5] = 3.25
    spike[k - 1] = -1e-3
    rows.append(spike)
    ties = np.zeros(k, np.float32)
    ties[:11] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, -1.5, 126.5, -126.5]
    rows.append(ties)
    tiny = np.full(k, 1e-30, np.float32)  # subnormal-range scale -> f16 flush
    rows.append(tiny)
    big = gen_normal_rows((k,), seed=77, scale=1e4)
    rows.append(big)
    return np.stack(rows)


@pytest.mark.parametrize("k", [256, 1024, 3072])
def test_encode_bit_exact(k):
    from quantized_q8_dequant_amd import encode_q8_0

    x = np.concatenate([gen_normal_rows((300, k), seed=k, scale=0.02), _special_rows(k)])
    got = encode_q8_0(torch.from_numpy(x).to(DEV)).cpu().numpy()
    want = oq.to_gguf(*oq.encode(x))
    assert got.shape == want.shape
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:5]}"


def test_repack_round_trip():
    from quantized_q8_dequant_amd import encode_q8_0, repack_q8_0

    x = gen_normal_rows((77, 768), seed=5, scale=0.02)
    blocks = encode_q8_0(torch.from_numpy(x).to(DEV))
    qs, sc = repack_q8_0(blocks, 77, 768)
    wq, wd = oq.encode(x)
    assert np.array_equal(qs.cpu().numpy(), wq)
    assert np.array_equal(sc.cpu().numpy().view(np.float16), wd)


def _weights(n, k, seed):
    from quantized_q8_dequant_amd import encode_q8_0, repack_q8_0

    w = gen_normal_rows((n, k), seed=seed, scale=0.02)
    qs, sc = repack_q8_0(encode_q8_0(torch.from_numpy(w).to(DEV)), n, k)
    return w, oq.Q8Weight(w), qs, sc


@pytest.mark.parametrize("m,k,n", [(1, 256, 64), (3, 1024, 96), (2, 3072, 40), (5, 768, 33)])
def test_block_dots_bit_exact(m, k, n):
    from quantized_q8_dequant_amd import q8_0_block_dots

    x = gen_normal_rows((m, k), seed=m * 1000 + k, scale=1.3)
    _, ow, qs, _ = _weights(n, k, seed=k + n)
    qa, da, S = q8_0_block_dots(torch.from_numpy(x).to(DEV), qs)
    oqa, oda = oq.encode(x)
    assert np.array_equal(qa.cpu().numpy(), oqa)
    assert np.array_equal(da.cpu().numpy().view(np.float16), oda)
    assert np.array_equal(S.cpu().numpy().astype(np.int64), oq.block_dots(oqa, ow.qs))


def _ulps(a, b):
    """Distance in f32 units in the last place (same-sign finite values)."""
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


@pytest.mark.parametrize(
    "m,k,n",
    [(1, 1024, 4096), (1, 3072, 1024), (1, 2048, 1024), (1, 256, 512), (1, 768, 256), (1, 4096, 384),
     (1, 12288, 256), (1, 4096, 4100), (1, 12288, 1400), (2, 1024, 256), (7, 1024, 256), (128, 1024, 512),
     (300, 3072, 384), (129, 256, 128),
     # small-M GEMM: 16/32/64-row tilings, K slices of 4/8/16, ragged N, 64-row units
     (16, 1024, 4096), (17, 2048, 1024), (33, 3072, 1000), (64, 4096, 520), (20, 12288, 256), (5, 768, 4100),
     (32, 256, 65600), (64, 256, 96),
     # 33..64 rows on narrow matrices (64 workgroups; two and three chunks per K slice, a ragged M)
     (64, 2048, 1024), (40, 3072, 1024), (64, 3072, 1000)],
)
def test_linear_matches_oracle(m, k, n):
    from quantized_q8_dequant_amd import q8_0_linear

    x = gen_normal_rows((m, k), seed=7 * m + k, scale=1.0)
    _, ow, qs, sc = _weights(n, k, seed=3 * k + n)
    y = q8_0_linear(torch.from_numpy(x).to(DEV), qs, sc).cpu().numpy()
    ref = oq.linear(x, ow)
    ulps = _ulps(y, ref)
    assert ulps.max() <= 1, f"max {ulps.max()} ulps at {np.unravel_index(ulps.argmax(), ulps.shape)}"
    assert (ulps == 0).mean() >= 0.999, f"{(ulps == 0).mean():.5f} bit-identical"


@pytest.mark.parametrize(
    "m,k,n",
    [(1, 1024, 4096), (7, 256, 64), (64, 1024, 1024), (64, 2048, 1000), (130, 3072, 320), (200, 1024, 151)],
)
def test_bf16_linear_matches_oracle(m, k, n):
    """bf16 weights x f32 activations: products and sum in f64, rounded once,
    as the oracle does; only the f64 summation order differs, so results
    agree exactly but for a rounding tie (at most one f32 ulp)."""
    from oracle import ops
    from quantized_q8_dequant_amd import bf16_linear, encode_bf16

    x = gen_normal_rows((m, k), seed=11 * m + k, scale=1.0)
    w = gen_normal_rows((n, k), seed=13 * n + k, scale=0.02)
    wb = encode_bf16(torch.from_numpy(w).to(DEV))
    y = bf16_linear(torch.from_numpy(x).to(DEV), wb).cpu().numpy()
    ref = ops.bf16_linear(x, ops.bf16_round(w))
    ulps = np.abs(y.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, f"max {ulps.max()} ulps"
    assert (ulps == 0).mean() >= 0.999


def test_peak_probes_compute_what_they_claim():
    """The copy probe copies and the read probe sums (a ragged multiple of 16
    bytes included); the MFMA probe's accumulators hold 32 * b * b per MFMA
    element."""
    from quantized_q8_dequant_amd import peak_copy, peak_mfma_i8, peak_read, peak_read_partials

    for nbytes in (1 << 20, 16 * 1_000_003):
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV)
        dst = torch.zeros_like(src)
        peak_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
        parts = torch.zeros(peak_read_partials(), dtype=torch.int32, device=DEV)
        peak_read(src, parts)
        words = src.cpu().numpy().view(np.uint32)
        assert int(parts.cpu().numpy().view(np.uint32).sum(dtype=np.uint64)) % 2**32 == int(
            words.sum(dtype=np.uint64)) % 2**32
    out = torch.zeros(256 * 3, dtype=torch.int32, device=DEV)
    ops = peak_mfma_i8(out, 3, 7, fill=0x1FD)  # low byte 0xFD = -3
    torch.cuda.synchronize()
    assert ops == 3 * 4 * 4 * 7 * 65536
    assert bool((out == 2048 * 9 * 7).all())
