"""Graph replay of the tuned table on the whole sweep: the page's deployment
(ai-radar.it, "Helion nel backend vLLM", paragraph 4: the tuned kernels run
for small token counts under graph replay), checked output by output.

For every (format, shape) of the 24-shape sweep, for the GEMM and the linear
op, and for the row-major, the packed and the fastest layout of the table
(K-segmented at small M), with the config the library resolves from
its shipped table: two calls on two distinct copies of the weights, each into
its own output, are captured into one HIP graph; the graph is replayed twice
(outputs cleared before each replay, eager work in between), and every
replayed output must be bit-equal to the eager call with the same config and
within rtol = atol = 1e-2 of the fp64 oracle.
"""
import pytest
import torch

import synthetic
from tests.gpu_cases import DEV, Case, assert_bf16_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("fmt", ["FP8_Dynamic", "W8A8_INT8", "Block_FP8"])
@pytest.mark.parametrize("M,N,K", synthetic.SWEEP)
def test_sweep_graph_replay(w8, fmt, M, N, K):
    cs = Case(fmt, M, N, K)
    xq, sx = cs.gpu_act()
    # row-major, packed, and the layout the table times best (a K-segmented
    # one at small M)
    for packed in sorted({0, 1, w8.best_layout(fmt, M, N, K)}):
        if packed > 1:
            w0 = cs.memo(("seg", packed), lambda: w8.pack_weight(fmt, cs.wq, layout=packed))
        else:
            w0 = cs.weights(bool(packed))
        if packed:
            w1 = w8.PackedWeight(fmt, N, K, w0.data.clone(), packed)
        else:
            w1 = w0.clone()
        for op in ("gemm", "linear"):
            cfg, hit = w8.resolve_config(fmt, M, N, K, packed=packed, op=op)
            assert hit == 1, f"{fmt} {M}x{N}x{K} {op} packed={packed}: no table entry"
            ws = w8.Workspace(DEV, max(256, w8.workspace_size(fmt, M, N, K, cfg, packed=packed,
                                                              op=op)))

            def call(w, y):
                if op == "gemm":
                    return w8.gemm_w8a8(fmt, xq, sx, w, cs.sw, cfg=cfg, y=y, workspace=ws)
                return w8.linear(fmt, cs.x, w, cs.sw, cfg=cfg, y=y, workspace=ws, fused=True)

            eager = [call(w, None).clone() for w in (w0, w1)]
            torch.cuda.synchronize()
            assert torch.equal(_bits(eager[0]), _bits(eager[1]))
            ys = [torch.empty_like(eager[0]) for _ in range(2)]
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):          # warm the capture stream
                call(w0, ys[0])
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call(w0, ys[0])
                call(w1, ys[1])
            what = f"{fmt} {M}x{N}x{K} {op} packed={packed} {cfg}"
            for rep in range(2):
                for y in ys:
                    y.fill_(float("nan"))
                g.replay()
                torch.cuda.synchronize()
                for i, y in enumerate(ys):
                    assert torch.equal(_bits(y), _bits(eager[i])), f"{what}: replay {rep} call {i}"
                junk = torch.randn(256, 256, device=DEV) @ torch.randn(256, 256, device=DEV)
                del junk
            assert_bf16_close(ys[1], cs.Y, what)
            del g
