"""Two candidate steps on two streams at once, each with its own outputs and
workspaces: the library keeps no state between calls (beyond the no-alloc
entry point's documented array), so the concurrent results must equal the
serial ones bit for bit."""
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


def test_two_streams_match_serial(B):
    import torch
    from tests.gpu_common import dev, dev_bf16, say
    d = WL.candidate_inputs("mid")
    a = WL.attention_inputs("attn", requests=8)
    Rq, S, k, R = d["requests"], d["steps"], d["top_k"], d["rank"]
    T, V, Hd = Rq * S, d["vocab"], d["hidden"]
    W, Wp = dev_bf16(d["W"]), dev_bf16(d["Wp"])
    P, Sc, anchor = dev_bf16(d["P"]), dev_bf16(d["S"]), dev(d["anchor"])
    D = a["head_dim"]
    qw, kw = dev_bf16(a["q_w"]), dev_bf16(a["k_w"])
    pos, slots, tables, seq = dev(a["positions"]), dev(a["slots"]), dev(a["block_tables"]), dev(a["seq_lens"])
    cache0 = dev_bf16(a["cache"])
    cs = B.rope_cos_sin(a["max_pos"], D, a["theta"], "cuda")
    # two problem instances: the workload's hidden states and qkv rows, and the same rows reversed
    Hs = [dev_bf16(d["H"]), dev_bf16(np.ascontiguousarray(d["H"][::-1]))]
    qkvs = [dev_bf16(a["qkv"]), dev_bf16(np.ascontiguousarray(a["qkv"][::-1]))]

    def buffers():
        return {
            "ids": torch.empty((T, k), dtype=torch.int32, device="cuda"),
            "logits": torch.empty((T, k), dtype=torch.float32, device="cuda"),
            "hp": torch.empty((T, R), dtype=torch.float32, device="cuda"),
            "ws": torch.empty(B.lm_topk_workspace_size(T, V, Hd, k), dtype=torch.uint8, device="cuda"),
            "edges": torch.empty((Rq, S, k, k), dtype=torch.float32, device="cuda"),
            "cache": cache0.clone(),
            "q": torch.empty((qkvs[0].shape[0], a["hq"], D), dtype=torch.bfloat16, device="cuda"),
            "out": torch.empty((qkvs[0].shape[0], a["hq"], D), dtype=torch.bfloat16, device="cuda"),
        }

    def step(i, o, stream=None):
        B.lm_topk_proj(Hs[i], W, k, d["multiplier"], d["softcap"], Wp, o["ids"], o["logits"], o["hp"], o["ws"],
                       stream=stream)
        B.candidate_edges_hp(P, Sc, o["ids"].view(Rq, S, k), o["logits"].view(Rq, S, k), o["hp"], anchor,
                             o["edges"], stream=stream)
        B.qk_norm_rope_cache(qkvs[i], a["hq"], a["hkv"], D, qw, kw, a["eps"], pos, cs, slots, o["cache"],
                             q_out=o["q"], want_k=False, stream=stream)
        B.block_attn(o["q"], o["cache"], tables, seq, a["query_len"], a["window"], out=o["out"], stream=stream)

    names = ("ids", "logits", "hp", "edges", "cache", "out")
    ref = []
    for i in range(2):
        o = buffers()
        step(i, o)
        torch.cuda.synchronize()
        ref.append({n: o[n].clone() for n in names})
    # the two instances really differ
    assert not torch.equal(ref[0]["ids"], ref[1]["ids"])

    bufs = [buffers(), buffers()]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for rep in range(3):
        for o in bufs:
            for n in ("ids", "logits", "hp", "edges", "out"):
                o[n].zero_()
            o["cache"].copy_(cache0)
        torch.cuda.synchronize()
        for i in range(2):
            streams[i].wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(streams[i]):
                step(i, bufs[i], stream=streams[i])
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(2):
            for n in names:
                assert torch.equal(bufs[i][n], ref[i][n]), f"round {rep}, stream {i}: {n} differs from the serial run"
    say("[streams] two concurrent steps equal the serial ones, 3 rounds")
