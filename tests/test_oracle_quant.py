"""Pins for the oracle's quantizers (CPU only).

The quantizers are pinned against exact-rational brute force (correctly
rounded fp32 scale and scaled value, nearest code with ties to even), against
numpy's IEEE float32 division, and against properties any correct per-token or
per-group quantizer has.
"""
import numpy as np
import pytest

import synthetic
from tests import exact


@pytest.mark.parametrize("is_int8", [True, False])
def test_group_brute_force_random(oracle_mod, is_int8):
    rng = np.random.default_rng(11 if is_int8 else 12)
    for trial in range(12):
        n = int(rng.integers(1, 200))
        scale = 10.0 ** rng.uniform(-3, 3)
        x = (rng.standard_normal(n) * scale).astype(np.float32)
        q, s = oracle_mod.quantize_group(x, is_int8)
        want_q, want_s = exact.quantize_group_exact(x, is_int8)
        assert float(s) == float(want_s)
        assert list(q) == want_q, trial


def test_group_constructed_ties(oracle_mod):
    # amax = 127 gives s = 1 exactly, so x/s = x and the halves are exact ties.
    x = np.array([127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -126.5], dtype=np.float32)
    q, s = oracle_mod.quantize_group(x, True)
    assert s == 1.0
    assert list(q.view(np.int8)) == [127, 2, 4, -2, 0, 0, 2, -126]
    # amax = 448 gives s = 1 for E4M3FN; 1.0625 ties to 1.0, 1.1875 to 1.25.
    x = np.array([448, 1.0625, -1.1875, 0.0], dtype=np.float32)
    q, s = oracle_mod.quantize_group(x, False)
    assert s == 1.0
    assert list(q) == [0x7E, 0x38, 0xBA, 0x00]


@pytest.mark.parametrize("is_int8", [True, False])
def test_group_scale_is_ieee_division(oracle_mod, is_int8):
    rng = np.random.default_rng(5)
    qmax = np.float32(127 if is_int8 else 448)
    for _ in range(200):
        x = (rng.standard_normal(64) * 10.0 ** rng.uniform(-4, 4)).astype(np.float32)
        _, s = oracle_mod.quantize_group(x, is_int8)
        assert s == np.abs(x).max() / qmax          # numpy float32 division is IEEE


def test_group_all_zero(oracle_mod):
    for is_int8 in (True, False):
        q, s = oracle_mod.quantize_group(np.zeros(37, dtype=np.float32), is_int8)
        assert s == 1.0 and (q == 0).all()


@pytest.mark.parametrize("is_int8", [True, False])
def test_group_properties(oracle_mod, is_int8):
    rng = np.random.default_rng(21)
    qmax = 127 if is_int8 else 448
    for _ in range(50):
        x = (rng.standard_normal(300) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32)
        q, s = oracle_mod.quantize_group(x, is_int8)
        if is_int8:
            dq = q.view(np.int8).astype(np.float64)
        else:
            dq = oracle_mod.e4m3_decode(q)
        i = np.argmax(np.abs(x))
        assert abs(dq[i]) == qmax                   # the amax element lands on +-Qmax
        assert np.abs(dq).max() == qmax
        assert (np.sign(dq[dq != 0]) == np.sign(x[dq != 0])).all()
        if is_int8:
            err = np.abs(dq * float(s) - x.astype(np.float64))
            assert (err <= float(s) * (0.5 + 1e-5)).all()


def test_act_token_formats_brute_force(oracle_mod):
    M, K = 3, 160
    x = synthetic.activations("FP8_Dynamic", M, 7, K)
    xf = synthetic.bf16_bits_to_fp32(x)
    for fmt, is_int8 in (("FP8_Dynamic", False), ("W8A8_INT8", True)):
        xq, sx = oracle_mod.quantize_act(fmt, x)
        assert sx.shape == (M,)
        for m in range(M):
            want_q, want_s = exact.quantize_group_exact(xf[m], is_int8)
            assert float(sx[m]) == float(want_s)
            assert list(xq[m]) == want_q


def test_act_block_fp8_brute_force_and_group_locality(oracle_mod):
    M, K = 2, 384
    x = synthetic.activations("Block_FP8", M, 7, K)
    xf = synthetic.bf16_bits_to_fp32(x)
    xq, sx = oracle_mod.quantize_act("Block_FP8", x)
    assert sx.shape == (M, K // 128)
    for m in range(M):
        for g in range(K // 128):
            want_q, want_s = exact.quantize_group_exact(xf[m, 128 * g:128 * (g + 1)], False)
            assert float(sx[m, g]) == float(want_s)
            assert list(xq[m, 128 * g:128 * (g + 1)]) == want_q
    # changing one group leaves every other group's codes and scale unchanged
    x2 = x.copy()
    x2[0, 130] = synthetic.fp32_to_bf16_bits(np.array([50.0], np.float32))[0]
    xq2, sx2 = oracle_mod.quantize_act("Block_FP8", x2)
    assert (xq2[:, :128] == xq[:, :128]).all() and (xq2[:, 256:] == xq[:, 256:]).all()
    assert (xq2[1] == xq[1]).all()
    assert sx2[0, 1] != sx[0, 1] and sx2[0, 0] == sx[0, 0] and sx2[0, 2] == sx[0, 2]


def test_act_one_group_row_equals_token_fp8(oracle_mod):
    # with K = 128 a Block_FP8 group is the whole row: same codes, same scale
    x = synthetic.activations("Block_FP8", 5, 1, 128)
    a_q, a_s = oracle_mod.quantize_act("Block_FP8", x)
    b_q, b_s = oracle_mod.quantize_act("FP8_Dynamic", x)
    assert (a_q == b_q).all() and (a_s[:, 0] == b_s).all()


def test_act_zero_row_and_rejects_ragged_block_k(oracle_mod):
    x = synthetic.activations("W8A8_INT8", 3, 1, 256)
    x[1] = 0
    for fmt in ("W8A8_INT8", "FP8_Dynamic", "Block_FP8"):
        xq, sx = oracle_mod.quantize_act(fmt, x)
        assert (xq[1] == 0).all()
        assert (sx[1] == 1.0).all()
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.quantize_act("Block_FP8", synthetic.activations("Block_FP8", 1, 1, 200))


def test_weight_fp8_dynamic_per_row(oracle_mod):
    w = synthetic.fp32_weights("FP8_Dynamic", 1, 3, 96)
    wq, sw = oracle_mod.quantize_weight("FP8_Dynamic", w)
    assert sw.shape == (3,)
    for n in range(3):
        want_q, want_s = exact.quantize_group_exact(w[n], False)
        assert float(sw[n]) == float(want_s) and list(wq[n]) == want_q


def test_weight_block_fp8_blocks(oracle_mod):
    # N = 130 leaves a ragged two-row block at the bottom; K = 256 is two blocks
    N, K = 130, 256
    w = synthetic.fp32_weights("Block_FP8", 1, N, K)
    w[3, 5] = 40.0                                   # an outlier in block (0, 0) only
    wq, sw = oracle_mod.quantize_weight("Block_FP8", w)
    assert sw.shape == (2, 2)
    for bn, bk in ((0, 0), (1, 1), (1, 0)):
        blk = w[128 * bn:128 * (bn + 1), 128 * bk:128 * (bk + 1)]
        q, s = oracle_mod.quantize_group(blk.ravel(), False)
        assert sw[bn, bk] == s
        assert (wq[128 * bn:128 * (bn + 1), 128 * bk:128 * (bk + 1)].ravel() == q).all()
    assert sw[0, 0] == np.float32(40.0) / np.float32(448)
    # brute force on the ragged block
    blk = w[128:130, 0:128]
    want_q, want_s = exact.quantize_group_exact(blk.ravel(), False)
    assert float(sw[1, 0]) == float(want_s)
    assert list(wq[128:130, 0:128].ravel()) == want_q
