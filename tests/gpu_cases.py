"""Shared helpers for the GPU parity tests: build one seeded case on both
sides (GPU library and CPU oracle) from the same synthetic inputs.

Weights of the FP8 formats are quantized independently on each side (GPU
kernel vs oracle); int8 weights come straight from the generator.  Nothing
computed by the GPU is ever fed to the oracle.
"""
import numpy as np
import torch

import oracle
import synthetic

DEV = torch.device("cuda:0")


def to_bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8(t):
    return t.view(torch.uint8).cpu().numpy()


class Case:
    def __init__(self, fmt, M, N, K):
        import bit_quantized_gemm_token_amd as w8
        self.fmt, self.M, self.N, self.K = fmt, M, N, K
        print(f"[case] {fmt} M={M} N={N} K={K}", flush=True)
        self.x_bits = synthetic.activations(fmt, M, N, K)
        self.x = to_bf16_tensor(self.x_bits)
        if fmt == "W8A8_INT8":
            wq, sw = synthetic.int8_weights(fmt, M, N, K)
            self.wq = torch.from_numpy(wq).to(DEV)
            self.sw = torch.from_numpy(sw).to(DEV)
            self.wq_ref, self.sw_ref = wq.view(np.uint8), sw
        else:
            w = synthetic.fp32_weights(fmt, M, N, K)
            self.wq, self.sw = w8.quantize_weight(fmt, torch.from_numpy(w).to(DEV))
            self.wq_ref, self.sw_ref = oracle.quantize_weight(fmt, w)
        self.xq_ref, self.sx_ref = oracle.quantize_act(fmt, self.x_bits)
        self._Y = None

    @property
    def Y(self):
        """Oracle fp64 output from the oracle's own codes and scales."""
        if self._Y is None:
            self._Y = oracle.gemm(self.fmt, self.xq_ref, self.sx_ref, self.wq_ref, self.sw_ref)
        return self._Y

    _memo = None

    def memo(self, key, fn):
        if self._memo is None:
            self._memo = {}
        if key not in self._memo:
            self._memo[key] = fn()
        return self._memo[key]

    def acc_ref(self):
        """Exact accumulators from the oracle: int64 sums (W8A8_INT8), exact
        E4M3FN dot products (FP8_Dynamic) or the fp64 result (Block_FP8)."""
        if self.fmt == "W8A8_INT8":
            return self.memo("acc", lambda: oracle.acc_int8(self.xq_ref, self.wq_ref))
        if self.fmt == "FP8_Dynamic":
            return self.memo("acc", lambda: oracle.acc_fp8(self.xq_ref, self.wq_ref))
        return self.Y

    def acc_bound(self):
        """Error bound of the GPU's E4M3FN accumulators: 2^-14 times the sum of
        |products|.  The gfx950 fp8 MFMA does not sum its products as IEEE
        fp32 (measured: up to 2^-16.8 of the sum of |products| for one K=16
        dot product, e.g. 3936 against the exact 3932); the bound allows that
        with margin and still fails any indexing or scaling mistake, whose
        error is of the order of the sum itself."""
        if self.fmt == "W8A8_INT8":
            return 0
        def mag():
            if self.fmt == "FP8_Dynamic":
                return fp8_abs_sum(self.xq_ref, self.wq_ref)
            out = np.zeros((self.M, self.N))
            for g in range(self.K // 128):
                s = (np.abs(self.sx_ref[:, g]).astype(np.float64)[:, None] *
                     np.abs(self.sw_ref[np.arange(self.N) // 128, g]).astype(np.float64)[None, :])
                out += s * oracle.acc_fp8(self.xq_ref & 0x7F, self.wq_ref & 0x7F,
                                          128 * g, 128 * g + 128)
            return out
        return self.memo("bound", lambda: 2.0 ** -14 * mag() + 1e-30)

    def packed(self):
        """The GPU weights in the packed layout (packed on the GPU)."""
        import bit_quantized_gemm_token_amd as w8
        return self.memo("packed", lambda: w8.pack_weight(self.fmt, self.wq))

    def weights(self, packed):
        return self.packed() if packed else self.wq

    def gpu_act(self):
        import bit_quantized_gemm_token_amd as w8
        return w8.quantize_act(self.fmt, self.x)


def assert_bf16_close(y, Y, what=""):
    """The output bar: |y - Y| <= 1e-2 + 1e-2 |Y| elementwise, Y the fp64 oracle."""
    got = y.float().cpu().numpy().astype(np.float64)
    assert got.shape == Y.shape
    excess = np.abs(got - Y) - (1e-2 + 1e-2 * np.abs(Y))
    bad = np.argwhere(excess > 0)
    assert bad.size == 0, (f"{what}: {len(bad)} of {Y.size} outside tolerance; first "
                           f"{[(tuple(i), got[tuple(i)], Y[tuple(i)]) for i in bad[:5]]}")
    return float(np.abs(got - Y).max())


def fp8_abs_sum(xq_ref, wq_ref):
    """Sum of |products| of each dot product (rounding scale of an fp32 sum)."""
    return oracle.acc_fp8(xq_ref & 0x7F, wq_ref & 0x7F)
