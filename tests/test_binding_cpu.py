"""Python binding checks that need no GPU: caller-supplied buffers of the
wrong size are refused with ValueError before any pointer reaches the
library (a short output or scale buffer would otherwise be written or read
past its end by the kernel), and a workspace never grows under capture."""
import pytest
import torch


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


M, N, K = 4, 256, 512


def _codes(m, k):
    return torch.zeros((m, k), dtype=torch.uint8)


@pytest.mark.parametrize("fmt", ["FP8_Dynamic", "W8A8_INT8", "Block_FP8"])
def test_gemm_refuses_short_buffers(w8, fmt):
    block = fmt == "Block_FP8"
    nsx = M * (K // 128) if block else M
    nsw = (N // 128) * (K // 128) if block else N
    xq, wq = _codes(M, K), _codes(N, K)
    sx, sw = torch.ones(nsx), torch.ones(nsw)
    y = torch.empty((M, N), dtype=torch.bfloat16)
    bad = [dict(sx=torch.ones(nsx - 1)), dict(sw=torch.ones(nsw - 1)),
           dict(sw=torch.ones(nsw + 1)), dict(y=torch.empty((M - 1, N), dtype=torch.bfloat16)),
           dict(y=torch.empty((M, N - 16), dtype=torch.bfloat16)),
           dict(sx=torch.ones(2 * nsx)[::2])]        # right count, not contiguous
    for b in bad:
        args = dict(sx=sx, sw=sw, y=y)
        args.update(b)
        with pytest.raises(ValueError):
            w8.gemm_w8a8(fmt, xq, args["sx"], wq, args["sw"], y=args["y"])
    acc_dt = torch.int32 if fmt == "W8A8_INT8" else torch.float32
    with pytest.raises(ValueError):
        w8.gemm_w8a8_acc(fmt, xq, sx, wq, sw, out=torch.empty((M, N // 2), dtype=acc_dt))


@pytest.mark.parametrize("fmt", ["FP8_Dynamic", "Block_FP8"])
def test_linear_and_quantize_refuse_short_buffers(w8, fmt):
    block = fmt == "Block_FP8"
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    wq = _codes(N, K)
    nsw = (N // 128) * (K // 128) if block else N
    with pytest.raises(ValueError):
        w8.linear(fmt, x, wq, torch.ones(nsw), y=torch.empty((M, N - 1), dtype=torch.bfloat16),
                  fused=True)
    with pytest.raises(ValueError):
        w8.linear(fmt, x, wq, torch.ones(nsw - 1), fused=True)
    with pytest.raises(ValueError):
        w8.quantize_act(fmt, x, xq=_codes(M - 1, K))
    with pytest.raises(ValueError):
        w8.quantize_act(fmt, x, sx=torch.ones(M * (K // 128) - 1 if block else M - 1))


def test_workspace_does_not_grow_under_capture(w8, monkeypatch):
    ws = w8.Workspace("cpu")
    ws.buf = torch.zeros(1024, dtype=torch.uint8)
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    assert ws.reserve(512) is ws.buf          # fits: no allocation, allowed under capture
    with pytest.raises(RuntimeError, match="capture"):
        ws.reserve(4096)
    assert ws.buf.numel() == 1024 and ws._retired == []
