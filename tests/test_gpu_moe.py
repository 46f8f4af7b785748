"""The MoE grouped GEMM on the GPU against the oracle's moe_gemm, and bit for
bit against the dense GEMM run per expert on the gathered rows with the same
config: every format, both weight layouts, split-K, stream-K, x_lds, Swap-AB,
empty experts, one expert holding every token, one-row tokens, and graph
replay with a shared-tile workspace."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_cases import DEV, assert_bf16_close, to_bf16_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


class MoeCase:
    def __init__(self, w8, fmt, T, E, N, K, topk=None, seed=0, routing=None, max_m=32):
        print(f"[moe] {fmt} T={T} E={E} N={N} K={K} topk={topk}", flush=True)
        self.fmt, self.T, self.E, self.N, self.K = fmt, T, E, N, K
        bits = synthetic.activations(fmt, T, N, K)
        self.xq, self.sx = w8.quantize_act(fmt, to_bf16_tensor(bits))
        xq_ref, sx_ref = oracle.quantize_act(fmt, bits)
        w, sw = synthetic.moe_weights(fmt, E, N, K)
        if fmt == "W8A8_INT8":
            self.wq = torch.from_numpy(w).to(DEV)
            self.sw = torch.from_numpy(sw).to(DEV)
            wq_ref, sw_ref = w.view(np.uint8), sw
        else:
            qs = [w8.quantize_weight(fmt, torch.from_numpy(w[e]).to(DEV)) for e in range(E)]
            self.wq = torch.stack([q for q, _ in qs])
            self.sw = torch.stack([s for _, s in qs]).contiguous()
            rq = [oracle.quantize_weight(fmt, w[e]) for e in range(E)]
            wq_ref = np.stack([q for q, _ in rq])
            sw_ref = np.stack([s for _, s in rq])
        if routing is None:
            routing = synthetic.moe_routing(T, E, topk, seed, max_m)
        self.offsets_np, self.rows_np = routing
        self.offsets = torch.from_numpy(np.asarray(self.offsets_np, np.int32)).to(DEV)
        self.rows = torch.from_numpy(np.asarray(self.rows_np, np.int32)).to(DEV)
        self.packed = w8.pack_experts(fmt, self.wq)
        self.Y = oracle.moe_gemm(fmt, xq_ref, sx_ref, self.offsets_np, self.rows_np, wq_ref,
                                 sw_ref)

    def weights(self, packed):
        return self.packed if packed else self.wq

    def per_expert(self, w8, cfg, packed):
        """The dense GEMM per expert on its gathered rows."""
        out = torch.empty((len(self.rows_np), self.N), dtype=torch.bfloat16, device=DEV)
        for e in range(self.E):
            a, b = int(self.offsets_np[e]), int(self.offsets_np[e + 1])
            if b == a:
                continue
            r = self.rows[a:b].long()
            xq, sx = self.xq[r].contiguous(), self.sx[r].contiguous()
            if packed:
                wq = w8.PackedWeight(self.fmt, self.N, self.K, self.packed.data[e])
            else:
                wq = self.wq[e]
            out[a:b] = w8.gemm_w8a8(self.fmt, xq, sx, wq, self.sw[e], cfg=cfg)
        return out


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


CFGS = (dict(tile_n=16, waves_k=4, unroll=2, split_k=1),
        dict(tile_n=32, waves_k=2, unroll=1, split_k=4, swap_ab=1),
        dict(tile_n=16, waves_k=1, waves_n=8, unroll=1, split_k=2, x_lds=1),
        dict(tile_n=64, waves_k=1, unroll=1, split_k=1),
        dict(tile_n=16, waves_k=8, unroll=1, split_k=16),
        dict(tile_n=16, waves_k=2, unroll=2, grid=40))


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
def test_moe_matches_oracle_and_per_expert_gemm(w8, fmt):
    # 9 experts' routing with an empty expert inserted at index 3
    off9, rows = synthetic.moe_routing(24, 9, 6, 5)
    offsets = np.insert(off9, 3, off9[3]).astype(np.int32)
    cs = MoeCase(w8, fmt, T=24, E=10, N=300, K=1024, routing=(offsets, rows))
    counts = np.diff(cs.offsets_np)
    assert counts.max() > 16 and counts[3] == 0
    for packed in (False, True):
        y = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.weights(packed), cs.sw)
        torch.cuda.synchronize()
        assert_bf16_close(y, cs.Y, f"moe default {fmt} packed={packed}")
        for kw in CFGS:
            cfg = w8.Config.make(**kw)
            y = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.weights(packed), cs.sw,
                            cfg=cfg)
            ref = cs.per_expert(w8, cfg, packed)
            torch.cuda.synchronize()
            assert same_bits(y, ref), f"{fmt} {kw} packed={packed}"
            assert_bf16_close(y, cs.Y, f"moe {fmt} {kw} packed={packed}")


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "Block_FP8"])
def test_moe_edge_routings(w8, fmt):
    T, E, N, K = 32, 4, 200, 512
    # every token to expert 2; the others empty
    routing = (np.array([0, 0, 0, 32, 32], np.int32), np.arange(32, dtype=np.int32))
    cs = MoeCase(w8, fmt, T, E, N, K, routing=routing)
    for packed in (False, True):
        y = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.weights(packed), cs.sw,
                        cfg=w8.Config.make(tile_n=16, waves_k=4, unroll=1, split_k=2))
        torch.cuda.synchronize()
        assert_bf16_close(y, cs.Y, f"moe one expert {fmt}")
    # one token, routed to three experts out of order of their ids; max_m = 1
    routing = (np.array([0, 1, 1, 2, 3], np.int32), np.array([0, 0, 0], np.int32))
    cs = MoeCase(w8, fmt, 1, E, N, K, routing=routing)
    y = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.wq, cs.sw, max_m=1)
    torch.cuda.synchronize()
    assert_bf16_close(y, cs.Y, f"moe one token {fmt}")
    # E = 1, identity routing: the dense GEMM
    routing = (np.array([0, 12], np.int32), np.arange(12, dtype=np.int32))
    cs = MoeCase(w8, fmt, 12, 1, N, K, routing=routing)
    cfg = w8.Config.make(tile_n=32, waves_k=2, unroll=2, split_k=2)
    y = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.wq, cs.sw, max_m=16, cfg=cfg)
    ref = w8.gemm_w8a8(fmt, cs.xq, cs.sx, cs.wq[0], cs.sw[0], cfg=cfg)
    torch.cuda.synchronize()
    assert same_bits(y, ref)


def test_moe_routing_is_clamped(w8):
    """Routing that breaks the preconditions stays inside the buffers: offsets
    beyond the row list are clamped to it, row ids beyond the tokens to the
    last token, and an expert over max_m computes its first 16 * ceil(max_m/16)
    rows.  The rows it does compute equal the oracle on the clamped routing."""
    fmt, T, E, N, K = "W8A8_INT8", 8, 3, 96, 256
    rows = np.array([0, 1, 2, 3, 4, 5, 7, 6], np.int32)
    cs = MoeCase(w8, fmt, T, E, N, K, routing=(np.array([0, 5, 8, 8], np.int32), rows))
    bad_off = torch.tensor([0, 5, 100, 100], dtype=torch.int32, device=DEV)
    bad_rows = cs.rows.clone()
    bad_rows[7] = 1000                      # clamped to token T - 1 = 7
    y = torch.full((8, N), 7.0, dtype=torch.bfloat16, device=DEV)
    w8.moe_gemm(fmt, cs.xq, cs.sx, bad_off, bad_rows, cs.wq, cs.sw, y=y, max_m=16)
    want_rows = rows.copy()
    want_rows[7] = T - 1
    Y = oracle.moe_gemm(fmt, *[np.asarray(v) for v in (
        oracle.quantize_act(fmt, synthetic.activations(fmt, T, N, K)))],
        np.array([0, 5, 8, 8]), want_rows,
        synthetic.moe_weights(fmt, E, N, K)[0].view(np.uint8), synthetic.moe_weights(fmt, E, N, K)[1])
    torch.cuda.synchronize()
    assert_bf16_close(y, Y, "clamped routing")
    # an expert over max_m = 2: only its first 16 rows (one block) exist; with
    # 5 entries and max_m 2 all 5 fit in the block, so all are computed
    y2 = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.wq, cs.sw, max_m=2)
    torch.cuda.synchronize()
    assert_bf16_close(y2, cs.Y, "count above max_m within one block")


def test_moe_many_experts_and_graph_replay(w8):
    """128 experts (N = 512, K = 1024, top-8 of 16 tokens) under split-K,
    eager and replayed from a HIP graph."""
    fmt = "FP8_Dynamic"
    cs = MoeCase(w8, fmt, T=16, E=128, N=512, K=1024, topk=8, seed=11)
    cfg = w8.Config.make(tile_n=16, waves_k=4, unroll=1, split_k=4)
    ws = w8.Workspace(DEV, w8.moe_workspace_size(fmt, 128, 16, 512, 1024, 32, cfg, packed=True))
    eager = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.packed, cs.sw, cfg=cfg,
                        workspace=ws).clone()
    torch.cuda.synchronize()
    assert_bf16_close(eager, cs.Y, "moe E=128")
    y = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.packed, cs.sw, cfg=cfg, y=y,
                    workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.packed, cs.sw, cfg=cfg, y=y,
                    workspace=ws)
    for i in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(y, eager), f"replay {i}"


@pytest.mark.parametrize("proj,N,K", [("gate_up", 1536, 2048), ("down", 2048, 768)])
def test_moe_bench_size_sampled(w8, proj, N, K):
    """The benchmark's MoE layers at full size (128 experts, top-8 of 32
    tokens, packed weights, the default config): W8A8_INT8, whose weight codes
    are given, against the oracle on a sample of routed entries (every entry
    of 6 experts)."""
    fmt, T, E = "W8A8_INT8", 32, 128
    print(f"[moe] bench size {proj} {N}x{K}", flush=True)
    g = np.random.Generator(np.random.PCG64(77))
    wq = g.integers(-127, 128, size=(E, N, K), dtype=np.int8)
    sw = g.uniform(0.001, 0.01, size=(E, N)).astype(np.float32)
    bits = synthetic.activations(fmt, T, N, K)
    xq, sx = w8.quantize_act(fmt, to_bf16_tensor(bits))
    xq_ref, sx_ref = oracle.quantize_act(fmt, bits)
    offsets, rows = synthetic.moe_routing(T, E, 8, seed=3)
    packed = w8.pack_experts(fmt, torch.from_numpy(wq).to(DEV))
    y = w8.moe_gemm(fmt, xq, sx, torch.from_numpy(offsets).to(DEV),
                    torch.from_numpy(rows).to(DEV), packed, torch.from_numpy(sw).to(DEV))
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()
    active = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    for e in active[::max(1, len(active) // 6)][:6]:
        a, b = int(offsets[e]), int(offsets[e + 1])
        r = rows[a:b]
        Y = oracle.gemm(fmt, xq_ref[r], sx_ref[r], wq[e].view(np.uint8), sw[e])
        assert_bf16_close(torch.from_numpy(got[a:b]), Y, f"moe bench size expert {e}")


def test_moe_tune_inserts_a_validated_entry(w8):
    """The grouped GEMM's tuner: candidates validated against the fallback
    config (one forced to fail is dropped), the winner inserted as the "moe"
    entry for (T, N, K), and picked up by moe_gemm's cfg=None path, whose
    output then matches the oracle."""
    fmt, E, T, N, K, topk = "FP8_Dynamic", 16, 4, 512, 1024, 2
    w8.clear_config_table()
    try:
        best, stats = w8.moe_tune(fmt, E, T, N, K, topk, warmup=1, replays=3,
                                  rotate_bytes=64 << 20, packed=True, fail_candidate=0)
        print(f"[moe] tune: {stats}", flush=True)
        assert stats["candidates"] > 10 and stats["rejected"] >= 1
        assert stats["validated"] + stats["rejected"] == stats["candidates"]
        assert stats["best_index"] != 0 and stats["best_us_bank2"] > 0
        cfg, hit = w8.moe_config(fmt, E, T, N, K, T, packed=True)
        assert hit == 1 and cfg == best
        cs = MoeCase(w8, fmt, T=T, E=E, N=N, K=K, topk=topk, seed=9, max_m=T)
        y = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.packed, cs.sw, max_m=T)
        torch.cuda.synchronize()
        assert_bf16_close(y, cs.Y, "moe with the tuned entry")
    finally:
        w8.clear_config_table()
        w8.load_default_table()


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "Block_FP8"])
def test_moe_compact_expert_grid(w8, fmt):
    """Fewer routed entries than experts (E <= 256): the launch holds one slot
    per entry and slot j runs the j-th expert with entries.  Routings that put
    entries at the edges of every 64-expert chunk of E = 256, a single entry
    among 200 experts, and E = 300 (above the compact bound: one slot per
    expert) all equal the per-expert GEMM bit for bit and the oracle."""
    N, K = 160, 512
    experts = [0, 63, 64, 127, 128, 191, 192, 255]
    per = {e: [i % 3] for i, e in enumerate(experts)}      # 8 entries of 3 tokens
    per[64].append(2)
    off = np.zeros(257, np.int32)
    for e in range(256):
        off[e + 1] = off[e] + len(per.get(e, []))
    rows = np.array([t for e in range(256) for t in per.get(e, [])], np.int32)
    cases = [dict(T=3, E=256, routing=(off, rows)),
             dict(T=1, E=200, routing=(np.r_[np.zeros(138, np.int32),
                                             np.ones(63, np.int32)], np.zeros(1, np.int32))),
             dict(T=2, E=300, topk=2, seed=4)]
    for kw in cases:
        cs = MoeCase(w8, fmt, N=N, K=K, **kw)
        assert len(cs.rows_np) < cs.E
        for packed in (False, True):
            for ckw in (CFGS[0], CFGS[1], CFGS[2]):
                cfg = w8.Config.make(**ckw)
                y = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.weights(packed),
                                cs.sw, max_m=cs.T, cfg=cfg)
                ref = cs.per_expert(w8, cfg, packed)
                torch.cuda.synchronize()
                assert same_bits(y, ref), f"{fmt} E={cs.E} {ckw} packed={packed}"
                assert_bf16_close(y, cs.Y, f"compact {fmt} E={cs.E} {ckw}")


FUSED_CFGS = (dict(tile_n=16, waves_k=1, waves_n=8, unroll=2, split_k=1, x_lds=1),
              dict(tile_n=32, waves_k=1, waves_n=4, unroll=1, split_k=4, swap_ab=1, x_lds=1),
              dict(tile_n=16, waves_k=1, waves_n=8, unroll=1, split_k=2, x_lds=1),
              dict(tile_n=64, waves_k=1, waves_n=4, unroll=1, split_k=1, x_lds=1),
              dict(tile_n=16, waves_k=1, waves_n=4, unroll=2, grid=40, x_lds=1))


def unfused_twin(w8, kw):
    """The grouped config on quantized activations that runs the same MFMA
    sequence: the unfused kernel stages activations in LDS only with waves
    along N, and reads them in the K loop (same fragments, same order)
    otherwise."""
    return w8.Config.make(**dict(kw, x_lds=1 if kw.get("waves_n", 1) > 1 else 0))


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
def test_moe_linear_equals_quantize_then_moe_gemm(w8, fmt):
    """moe_linear, fused quantization in the grouped kernel and quantize
    launch + grouped kernel: bit-identical to quantize_act followed by
    moe_gemm with the same tiling (every format, both layouts,
    split-K, stream-K, waves along N, Swap-AB, an empty expert, experts above
    16 tokens), within the bar of the oracle, and the compact grid with one
    token among 200 experts."""
    off9, rows = synthetic.moe_routing(24, 9, 6, 5)
    offsets = np.insert(off9, 3, off9[3]).astype(np.int32)
    N, K = 300, 1280 if fmt != "Block_FP8" else 1024
    cs = MoeCase(w8, fmt, T=24, E=10, N=N, K=K, routing=(offsets, rows))
    x = to_bf16_tensor(synthetic.activations(fmt, 24, N, K))
    for packed in (False, True):
        y = w8.moe_linear(fmt, x, cs.offsets, cs.rows, cs.weights(packed), cs.sw)
        torch.cuda.synchronize()
        assert_bf16_close(y, cs.Y, f"moe_linear default {fmt} packed={packed}")
        for kw in FUSED_CFGS:
            cfg = w8.Config.make(**kw)
            y = w8.moe_linear(fmt, x, cs.offsets, cs.rows, cs.weights(packed), cs.sw, cfg=cfg)
            ref = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.weights(packed), cs.sw,
                              cfg=unfused_twin(w8, kw))
            torch.cuda.synchronize()
            assert same_bits(y, ref), f"{fmt} {kw} packed={packed}"
            assert_bf16_close(y, cs.Y, f"moe_linear {fmt} {kw} packed={packed}")
        # quantize launch + the grouped kernel (codes in the workspace, after
        # the shared tiles of split-K / stream-K configs)
        for kw in CFGS[:3] + CFGS[5:]:
            cfg = w8.Config.make(**dict(kw, quant_launch=1))
            y = w8.moe_linear(fmt, x, cs.offsets, cs.rows, cs.weights(packed), cs.sw, cfg=cfg)
            ref = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.weights(packed), cs.sw,
                              cfg=w8.Config.make(**kw))
            torch.cuda.synchronize()
            assert same_bits(y, ref), f"quant_launch {fmt} {kw} packed={packed}"
    # one token among 200 experts (compact grid), max_m = 1
    one = MoeCase(w8, fmt, T=1, E=200, N=N, K=K,
                  routing=(np.r_[np.zeros(138, np.int32), np.ones(63, np.int32)],
                           np.zeros(1, np.int32)))
    x1 = to_bf16_tensor(synthetic.activations(fmt, 1, N, K))
    for kw in FUSED_CFGS[:3]:
        cfg = w8.Config.make(**kw)
        y = w8.moe_linear(fmt, x1, one.offsets, one.rows, one.packed, one.sw, max_m=1, cfg=cfg)
        ref = w8.moe_gemm(fmt, one.xq, one.sx, one.offsets, one.rows, one.packed, one.sw,
                          max_m=1, cfg=unfused_twin(w8, kw))
        torch.cuda.synchronize()
        assert same_bits(y, ref), f"compact {fmt} {kw}"


def test_moe_linear_extreme_rows_and_graph(w8):
    """Token rows at the edges of bf16 (subnormal, -0, 2^120 magnitudes)
    quantized inside the grouped kernel give the standalone quantizer's
    codes (outputs bit-identical to quantize_act + moe_gemm); replayed from a
    HIP graph with a split-K workspace, every replay equals the eager call."""
    fmt, T, E, N, K = "W8A8_INT8", 14, 6, 128, 512
    cs = MoeCase(w8, fmt, T=T, E=E, N=N, K=K, topk=3, seed=21, max_m=16)
    x = to_bf16_tensor(synthetic.activations_extreme(fmt, T, K))
    xq, sx = w8.quantize_act(fmt, x)
    kw = dict(tile_n=16, waves_k=1, waves_n=4, unroll=1, split_k=4, x_lds=1)
    cfg = w8.Config.make(**kw)
    ws = w8.Workspace(DEV, w8.moe_workspace_size(fmt, E, T, N, K, 16, cfg, packed=True))
    ref = w8.moe_gemm(fmt, xq, sx, cs.offsets, cs.rows, cs.packed, cs.sw, max_m=16,
                      cfg=unfused_twin(w8, kw), workspace=ws)
    eager = w8.moe_linear(fmt, x, cs.offsets, cs.rows, cs.packed, cs.sw, max_m=16, cfg=cfg,
                          workspace=ws).clone()
    torch.cuda.synchronize()
    assert same_bits(eager, ref)
    y = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w8.moe_linear(fmt, x, cs.offsets, cs.rows, cs.packed, cs.sw, max_m=16, cfg=cfg, y=y,
                      workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.moe_linear(fmt, x, cs.offsets, cs.rows, cs.packed, cs.sw, max_m=16, cfg=cfg, y=y,
                      workspace=ws)
    for i in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(y, eager), f"replay {i}"


def test_moe_linear_tune(w8):
    """The fused grouped GEMM's tuner inserts a "moe_linear" entry that
    moe_linear then uses; output within the bar of the oracle."""
    fmt, E, T, N, K, topk = "Block_FP8", 16, 4, 512, 1024, 2
    w8.clear_config_table()
    try:
        best, stats = w8.moe_tune(fmt, E, T, N, K, topk, warmup=1, replays=3,
                                  rotate_bytes=64 << 20, packed=True, fused=True)
        print(f"[moe] fused tune: {stats}", flush=True)
        assert stats["validated"] >= 1
        assert best.quant_launch == 1 or (best.x_lds == 1 and best.waves_k <= 4)
        cfg, hit = w8.moe_linear_config(fmt, E, T, N, K, T, packed=True)
        assert hit == 1 and cfg == best
        assert w8.moe_config(fmt, E, T, N, K, T, packed=True)[1] == 0   # the unfused op's key
        cs = MoeCase(w8, fmt, T=T, E=E, N=N, K=K, topk=topk, seed=9, max_m=T)
        x = to_bf16_tensor(synthetic.activations(fmt, T, N, K))
        y = w8.moe_linear(fmt, x, cs.offsets, cs.rows, cs.packed, cs.sw, max_m=T)
        torch.cuda.synchronize()
        assert_bf16_close(y, cs.Y, "moe_linear with the tuned entry")
    finally:
        w8.clear_config_table()
        w8.load_default_table()


@pytest.mark.parametrize("T", [4, 32])
@pytest.mark.parametrize("proj,N,K", [("gate_up", 1536, 2048), ("down", 2048, 768)])
def test_moe_linear_bench_size(w8, proj, N, K, T):
    """The benchmark's MoE layers at full size from bf16 tokens (128 experts,
    top-8, packed weights, the shipped moe_linear entries -- the fused kernel
    at 4 tokens on the down projection, a quantize launch elsewhere): bit for
    bit the quantize_act + moe_gemm result with the same tiling."""
    fmt, E = "Block_FP8", 128
    print(f"[moe] linear bench size {proj} {N}x{K} T={T}", flush=True)
    g = np.random.Generator(np.random.PCG64(91))
    codes = g.integers(0, 256, size=(E, N, K), dtype=np.int64).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    wq = torch.from_numpy(codes).to(DEV).view(torch.float8_e4m3fn)
    sw = torch.from_numpy(g.uniform(0.5, 2.0, size=(E, (N + 127) // 128, K // 128))
                          .astype(np.float32)).to(DEV)
    packed = w8.pack_experts(fmt, wq)
    offsets, rows = synthetic.moe_routing(T, E, 8, seed=7)
    off_t, rows_t = torch.from_numpy(offsets).to(DEV), torch.from_numpy(rows).to(DEV)
    x = to_bf16_tensor(synthetic.activations(fmt, T, N, K))
    cfg, hit = w8.moe_linear_config(fmt, E, T, N, K, T, packed=True)
    assert hit == 1
    y = w8.moe_linear(fmt, x, off_t, rows_t, packed, sw, max_m=T)
    xq, sx = w8.quantize_act(fmt, x)
    twin = cfg.as_dict()
    fused = not twin.pop("quant_launch")
    ref = w8.moe_gemm(fmt, xq, sx, off_t, rows_t, packed, sw, max_m=T,
                      cfg=unfused_twin(w8, twin) if fused else w8.Config.make(**twin))
    torch.cuda.synchronize()
    assert same_bits(y, ref), f"{proj} T={T} {cfg}"


def test_moe_empty_routing(w8):
    """No routed entry (all offsets 0, an empty row list): both grouped entry
    points return an empty output without launching, with the default and a
    split-K config."""
    fmt, T, E, N, K = "FP8_Dynamic", 3, 8, 64, 256
    cs = MoeCase(w8, fmt, T=T, E=E, N=N, K=K, routing=(np.zeros(E + 1, np.int32),
                                                       np.zeros(0, np.int32)))
    x = to_bf16_tensor(synthetic.activations(fmt, T, N, K))
    sk = w8.Config.make(tile_n=16, waves_k=4, unroll=1, split_k=4)
    for packed in (False, True):
        y = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.weights(packed), cs.sw)
        y2 = w8.moe_gemm(fmt, cs.xq, cs.sx, cs.offsets, cs.rows, cs.weights(packed), cs.sw,
                         cfg=sk, workspace=w8.Workspace(DEV, 256))
        y3 = w8.moe_linear(fmt, x, cs.offsets, cs.rows, cs.weights(packed), cs.sw)
        torch.cuda.synchronize()
        assert y.shape == y2.shape == y3.shape == (0, N)
