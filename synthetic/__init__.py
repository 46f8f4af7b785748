"""Seeded synthetic inputs for the small-M 8-bit GEMM.

Shared by the tests, the benchmark and the smoke check, on both sides of every
parity comparison.  This module holds none of the method's arithmetic: it only
draws random numbers and rounds fp32 samples to bf16 (the activation dtype).
Quantization of activations and weights is done separately by each side.

Workload recipe (stand-in for decode-time linear layers under serving, which
the pages benchmark on ShareGPT with Qwen3 models; neither is used here):
  - activations X: bf16, N(0, 1) samples rounded to nearest-even bf16, [M, K];
  - W8A8_INT8 weights: int8 codes uniform in [-127, 127], [N, K], with
    per-output-channel fp32 scales uniform in [0.001, 0.01);
  - FP8_Dynamic weights: fp32 N(0, 0.02) samples, [N, K], quantized per row;
  - Block_FP8 weights: fp32 N(0, 1) samples, [N, K], quantized per 128x128 block.
Inputs are dense; no outlier channels are modelled.
Seeds: crc32 of "fmt|M|N|K|tensor", numpy PCG64.
"""
import zlib

import numpy as np
import torch

FORMAT_NAMES = ("FP8_Dynamic", "W8A8_INT8", "Block_FP8")
WEIGHT_SIGMA = {"FP8_Dynamic": 0.02, "Block_FP8": 1.0}


def seed_for(fmt: str, M: int, N: int, K: int, tensor: str) -> int:
    return zlib.crc32(f"{fmt}|{M}|{N}|{K}|{tensor}".encode())


def rng(fmt: str, M: int, N: int, K: int, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_for(fmt, M, N, K, tensor)))


def fp32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest-even bf16 (torch's CPU conversion); uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(fmt: str, M: int, N: int, K: int) -> np.ndarray:
    """bf16 X [M, K] as uint16 bits, from N(0, 1)."""
    x = rng(fmt, M, N, K, "x").standard_normal((M, K), dtype=np.float32)
    return fp32_to_bf16_bits(x)


def int8_weights(fmt: str, M: int, N: int, K: int):
    """int8 codes [N, K] uniform in [-127, 127] and fp32 scales [N] in U(0.001, 0.01)."""
    wq = rng(fmt, M, N, K, "w").integers(-127, 128, size=(N, K), dtype=np.int8)
    sw = rng(fmt, M, N, K, "sw").uniform(0.001, 0.01, size=(N,)).astype(np.float32)
    return wq, sw


def fp32_weights(fmt: str, M: int, N: int, K: int) -> np.ndarray:
    """fp32 W [N, K] from N(0, sigma), sigma 0.02 (FP8_Dynamic) or 1 (Block_FP8)."""
    sigma = WEIGHT_SIGMA[fmt]
    w = rng(fmt, M, N, K, "w").standard_normal((N, K), dtype=np.float32)
    return (w * np.float32(sigma)).astype(np.float32)


# The shape sweep: the (N, K) pairs of the FlashInfer mm_fp4 tuning table
# (flashinfer PR 3948, "Performance Data measured on B200", tuning testlist)
# that fall on the N x K grid {512, 896, 1792, 3584, 4608, 5120} x
# {640, 1024, 2048, 5120, 7168, 8192}, each at the page's M values, plus
# M = 32 (the top of the small-M window) for the three pairs that have
# M in {1, 4, 16} rows.
SWEEP = (
    (1, 512, 7168), (4, 512, 7168), (16, 512, 7168), (32, 512, 7168),
    (1, 896, 1024), (4, 896, 1024), (16, 896, 1024), (32, 896, 1024),
    (1, 4608, 7168), (4, 4608, 7168), (16, 4608, 7168), (32, 4608, 7168),
    (1, 896, 5120), (8, 896, 5120),
    (1, 1792, 5120), (8, 1792, 5120),
    (1, 3584, 5120), (8, 3584, 5120),
    (1, 5120, 640), (8, 5120, 640),
    (1, 5120, 2048), (8, 5120, 2048),
    (1, 5120, 8192), (8, 5120, 8192),
)


# MoE layers of the Qwen3 family's MoE models (the pages measure Qwen3
# models): 128 experts, top-8 routing, hidden size 2048 and expert width 768,
# i.e. the experts' gate/up projection (N = 1536, K = 2048) and down
# projection (N = 2048, K = 768), at decode token counts.
MOE_E, MOE_TOPK = 128, 8
MOE_SHAPES = (("gate_up", 1536, 2048), ("down", 2048, 768))
MOE_TOKENS = (1, 4, 16, 32)


def activations_extreme(fmt: str, M: int, K: int) -> np.ndarray:
    """bf16 X [M, K] whose rows span the magnitudes an activation quantizer
    meets at the edges of bf16: row r is N(0, 1) scaled by 2^e with e cycling
    through -124, -96, -90, -86, 0, 60, 120, and every third row (from row 1) has a
    quarter of its entries replaced by subnormal bf16 values (down to 2^-133)
    and an eighth by negative zeros."""
    g = rng(fmt, M, 0, K, "x_extreme")
    exps = (-124, -96, -90, -86, 0, 60, 120)
    x = g.standard_normal((M, K)).astype(np.float64)
    for r in range(M):
        x[r] *= 2.0 ** exps[r % len(exps)]
        if r % 3 == 1:
            idx = g.permutation(K)
            sub = idx[:K // 4]
            x[r, sub] = g.uniform(-1, 1, len(sub)) * 2.0 ** -126
            x[r, idx[K // 4:K // 4 + K // 8]] = -0.0
    bits = fp32_to_bf16_bits(x.astype(np.float32))
    return bits


def moe_routing(T: int, E: int, topk: int, seed: int, max_m: int = 32):
    """Top-k routing of T tokens to E experts: each token picks topk distinct
    experts uniformly at random (seeded), no expert takes more than max_m
    tokens.  Returns (offsets int32 [E + 1], rows int32 [T * topk]): the
    entries grouped by expert in expert order, tokens ascending within one."""
    g = np.random.Generator(np.random.PCG64(seed))
    per = [[] for _ in range(E)]
    for t in range(T):
        choices = [e for e in g.permutation(E) if len(per[e]) < max_m][:topk]
        for e in choices:
            per[e].append(t)
    counts = np.array([len(p) for p in per], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    rows = np.array([t for p in per for t in p], dtype=np.int32)
    return offsets, rows


def moe_weights(fmt: str, E: int, N: int, K: int):
    """Per-expert weights in the dense GEMM's distributions: W8A8_INT8 codes
    and scales ([E, N, K], [E, N]), else fp32 weights [E, N, K] to quantize."""
    if fmt == "W8A8_INT8":
        g = rng(fmt, E, N, K, "moe_w")
        wq = g.integers(-127, 128, size=(E, N, K), dtype=np.int8)
        sw = g.uniform(0.001, 0.01, size=(E, N)).astype(np.float32)
        return wq, sw
    g = rng(fmt, E, N, K, "moe_w")
    sd = 0.02 if fmt == "FP8_Dynamic" else 1.0
    return (g.standard_normal((E, N, K)) * sd).astype(np.float32), None
