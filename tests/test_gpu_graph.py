"""The candidate step captured in a HIP graph (torch.cuda.CUDAGraph): the
library's calls allocate nothing and never synchronise, so the whole step
records into one graph.  Every replay (with eager work and synchronisations
between replays) must reproduce the eager results bit for bit."""
import numpy as np
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_candidate_amd as B
    B.lib()
    return B


def test_step_in_a_graph(B):
    import torch
    from tests.gpu_common import dev, dev_bf16
    d = WL.candidate_inputs("mid")
    a = WL.attention_inputs("attn", requests=8)
    Rq, S, k, R = d["requests"], d["steps"], d["top_k"], d["rank"]
    T, V, Hd = Rq * S, d["vocab"], d["hidden"]
    H, W, Wp = dev_bf16(d["H"]), dev_bf16(d["W"]), dev_bf16(d["Wp"])
    P, Sc, anchor = dev_bf16(d["P"]), dev_bf16(d["S"]), dev(d["anchor"])
    D = a["head_dim"]
    qkv, qw, kw = dev_bf16(a["qkv"]), dev_bf16(a["q_w"]), dev_bf16(a["k_w"])
    pos, slots, tables, seq = dev(a["positions"]), dev(a["slots"]), dev(a["block_tables"]), dev(a["seq_lens"])
    cache0 = dev_bf16(a["cache"])
    cs = B.rope_cos_sin(a["max_pos"], D, a["theta"], "cuda")
    # outputs and workspaces made outside the graph
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    logits = torch.empty((T, k), dtype=torch.float32, device="cuda")
    hp = torch.empty((T, R), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.lm_topk_workspace_size(T, V, Hd, k), dtype=torch.uint8, device="cuda")
    edges = torch.empty((Rq, S, k, k), dtype=torch.float32, device="cuda")
    cache = cache0.clone()
    q_out = torch.empty((qkv.shape[0], a["hq"], D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q_out)

    def step(stream=None):
        B.lm_topk_proj(H, W, k, d["multiplier"], d["softcap"], Wp, ids, logits, hp, ws, stream=stream)
        B.candidate_edges_hp(P, Sc, ids.view(Rq, S, k), logits.view(Rq, S, k), hp, anchor, edges, stream=stream)
        B.qk_norm_rope_cache(qkv, a["hq"], a["hkv"], D, qw, kw, a["eps"], pos, cs, slots, cache, q_out=q_out,
                             want_k=False, stream=stream)
        B.block_attn(q_out, cache, tables, seq, a["query_len"], a["window"], out=out, stream=stream)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (ids, logits, hp, edges, cache, out)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        step(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(s)
    for rep in range(3):
        for t in (ids, logits, hp, edges, out):
            t.zero_()                       # eager work between replays
        cache.copy_(cache0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("ids", "logits", "hp", "edges", "cache", "out"), (ids, logits, hp, edges, cache, out),
                              ref):
            assert torch.equal(t, r), f"replay {rep}: {name} differs from the eager result"


def test_streaming_lm_topk_in_a_graph(B):
    """The LM head at 16 rows (the streaming kernel and the ranking merge) captured
    in a graph: every replay equals the eager call bit for bit."""
    import torch
    from tests.gpu_common import dev_bf16
    rng = np.random.default_rng(5)
    T, V, Hd, k = 16, 20000, 1024, 16
    H = dev_bf16(WL.to_bf16_bits(rng.standard_normal((T, Hd), dtype=np.float32)))
    W = dev_bf16(WL.to_bf16_bits(rng.standard_normal((V, Hd), dtype=np.float32) * np.float32(0.1)))
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    logits = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.lm_topk_workspace_size(T, V, Hd, k), dtype=torch.uint8, device="cuda")
    B.lm_topk(H, W, k, 0.5, 30.0, ids, logits, ws)
    torch.cuda.synchronize()
    ref = (ids.clone(), logits.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.lm_topk(H, W, k, 0.5, 30.0, ids, logits, ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.lm_topk(H, W, k, 0.5, 30.0, ids, logits, ws, stream=s)
    for rep in range(3):
        ids.zero_()
        logits.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref[0]) and torch.equal(logits, ref[1]), f"replay {rep} differs from the eager call"
