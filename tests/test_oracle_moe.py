"""Pins for the oracle's MoE grouped GEMM (CPU only).

Each routed entry is recomputed on its own, without the oracle's GEMM: numpy
int64 matmul for W8A8_INT8, and float64 matmul of the E4M3FN values from
PyTorch's own code table (exact at these sizes) for the FP8 formats, with
Block_FP8's per-group scaling written out.  The entry's expert comes from the
offsets by binary search.  Special cases: empty experts, one expert with
identity routing (= the dense GEMM), a token routed to several experts.
"""
import numpy as np
import pytest

import synthetic
from tests import exact

G = 128


def _case(oracle_mod, fmt, T, E, N, K, topk, seed, max_m=32):
    bits = synthetic.activations(fmt, T, N, K)
    xq, sx = oracle_mod.quantize_act(fmt, bits)
    w, sw = synthetic.moe_weights(fmt, E, N, K)
    if fmt == "W8A8_INT8":
        wq = w.view(np.uint8)
    else:
        qs = [oracle_mod.quantize_weight(fmt, w[e]) for e in range(E)]
        wq = np.stack([q for q, _ in qs])
        sw = np.stack([s for _, s in qs])
    offsets, rows = synthetic.moe_routing(T, E, topk, seed, max_m)
    return xq, sx, wq, sw, offsets, rows


def _entry(fmt, xq, sx, wq, sw, t, e):
    """Y of token row t with expert e, from first principles."""
    if fmt == "W8A8_INT8":
        c = xq[t].view(np.int8).astype(np.int64) @ wq[e].view(np.int8).astype(np.int64).T
        return c.astype(np.float64) * float(sx[t]) * sw[e].astype(np.float64)
    tab = exact.torch_e4m3_table()
    x, w = tab[xq[t]], tab[wq[e]]
    if fmt == "FP8_Dynamic":
        return (w @ x) * float(sx[t]) * sw[e].astype(np.float64)
    K = x.shape[0]
    y = np.zeros(w.shape[0])
    for g in range(K // G):
        part = w[:, g * G:(g + 1) * G] @ x[g * G:(g + 1) * G]
        y += part * float(sx[t, g]) * sw[e][np.arange(w.shape[0]) // G, g].astype(np.float64)
    return y


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
def test_moe_entries_from_first_principles(oracle_mod, fmt):
    T, E, N, K = 7, 5, 150, 256
    xq, sx, wq, sw, offsets, rows = _case(oracle_mod, fmt, T, E, N, K, topk=2, seed=3)
    Y = oracle_mod.moe_gemm(fmt, xq, sx, offsets, rows, wq, sw)
    assert Y.shape == (T * 2, N)
    for i in range(len(rows)):
        e = int(np.searchsorted(offsets, i, side="right") - 1)
        want = _entry(fmt, xq, sx, wq, sw, int(rows[i]), e)
        assert np.allclose(Y[i], want, rtol=1e-12, atol=0), (fmt, i, e)


def test_moe_special_cases(oracle_mod):
    fmt, T, N, K = "W8A8_INT8", 6, 64, 128
    xq, sx, wq, sw, _, _ = _case(oracle_mod, fmt, T, 3, N, K, topk=1, seed=1)
    # one expert, identity routing: the dense GEMM
    Y = oracle_mod.moe_gemm(fmt, xq, sx, [0, T], np.arange(T), wq[:1], sw[:1])
    assert np.array_equal(Y, oracle_mod.gemm(fmt, xq, sx, wq[0], sw[0]))
    # empty experts contribute no rows; a token routed to every expert
    offsets = np.array([0, 0, 2, 2])
    rows = np.array([4, 4])
    Y = oracle_mod.moe_gemm(fmt, xq, sx, offsets, rows, wq, sw)
    assert Y.shape == (2, N)
    assert np.array_equal(Y[0], Y[1])
    assert np.array_equal(Y[0], oracle_mod.gemm(fmt, xq[4:5], sx[4:5], wq[1], sw[1])[0])
    # swapping two experts' weights moves their rows' results
    offsets = np.array([0, 1, 2, 3])
    rows = np.array([0, 0, 0])
    Y = oracle_mod.moe_gemm(fmt, xq, sx, offsets, rows, wq, sw)
    Ys = oracle_mod.moe_gemm(fmt, xq, sx, offsets, rows, wq[[1, 0, 2]], sw[[1, 0, 2]])
    assert np.array_equal(Y[0], Ys[1]) and np.array_equal(Y[1], Ys[0])
    assert not np.array_equal(Y[0], Y[1])


def test_moe_routing_generator():
    offsets, rows = synthetic.moe_routing(32, 128, 8, seed=7)
    assert offsets[0] == 0 and offsets[-1] == 32 * 8 and (np.diff(offsets) >= 0).all()
    for e in range(128):
        r = rows[offsets[e]:offsets[e + 1]]
        assert (np.diff(r) > 0).all()          # distinct tokens, ascending
    # every token appears topk times, at most once per expert
    assert (np.bincount(rows, minlength=32) == 8).all()
    o2, _ = synthetic.moe_routing(32, 4, 4, seed=7, max_m=32)
    assert (np.diff(o2) == 32).all()           # 4 experts, 4 per token: all full
