"""GPU parity of dflash_linear (the draft layer's bias-free qkv_proj / o_proj)
and of one whole draft attention sublayer built from the library's calls
(qkv_proj -> q/k norm + RoPE + cache write -> block attention -> o_proj)
against the oracle."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL
from tests.parity import assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_candidate_amd as B
    B.lib()
    return B


def _bf(rng, shape, s=1.0):
    return WL.to_bf16_bits((rng.standard_normal(shape) * s).astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(300, 200, 328), (1, 8, 8), (513, 1024, 4096), (2048, 6144, 4096),
                                   (2048, 4096, 4096),
                                   # 192-wide tiles with a ragged last row tile, a ragged last
                                   # column tile and a K tail
                                   (2000, 6104, 200)])
def test_linear(B, M, N, K):
    import torch
    from tests.gpu_common import dev_bf16, host_bf16, say
    rng = np.random.default_rng(M * 7 + N + K)
    X, W = _bf(rng, (M, K)), _bf(rng, (N, K), 0.02)
    Y = host_bf16(B.linear(dev_bf16(X), dev_bf16(W)))
    torch.cuda.synchronize()
    ref = O.linear(X, W)
    assert_close(O.bf16_to_f64(Y), O.bf16_to_f64(ref), f"linear {M}x{N}x{K}")
    say(f"[linear {M}x{N}x{K}] outputs differing from the oracle by rounding: {int((Y != ref).sum())} of {Y.size}")


def test_linear_into_wider_output_leaves_other_columns(B):
    import torch
    from tests.gpu_common import dev_bf16, host_bf16
    rng = np.random.default_rng(3)
    X, W = _bf(rng, (260, 136)), _bf(rng, (120, 136), 0.1)
    out = torch.full((260, 200), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    B.linear(dev_bf16(X), dev_bf16(W), out=out)
    torch.cuda.synchronize()
    got = host_bf16(out)
    assert np.all(got[:, 120:] == 0xFFFF)
    assert_close(O.bf16_to_f64(got[:, :120]), O.bf16_to_f64(O.linear(X, W)), "linear into a wider row")


@pytest.mark.parametrize("requests", [8, 20])
def test_draft_attention_sublayer(B, requests):
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16, say
    d = WL.draft_layer_inputs(requests=requests)
    D, Hq, Hkv, Lq = d["head_dim"], d["hq"], d["hkv"], d["query_len"]
    cs = B.rope_cos_sin(d["max_pos"], D, d["theta"], "cuda")
    cache = dev_bf16(d["cache"])
    out = B.draft_attention(dev_bf16(d["hidden_states"]), dev_bf16(d["W_qkv"]), dev_bf16(d["W_o"]), Hq, Hkv, D,
                            dev_bf16(d["q_w"]), dev_bf16(d["k_w"]), d["eps"], dev(d["positions"]), cs,
                            dev(d["slots"]), cache, dev(d["block_tables"]), dev(d["seq_lens"]), Lq, d["window"])
    torch.cuda.synchronize()
    got = host_bf16(out)
    ref, rcache = O.draft_attention(d["hidden_states"], d["W_qkv"], d["W_o"], Hq, Hkv, D, d["q_w"], d["k_w"],
                                    d["eps"], d["positions"], d["theta"], d["slots"], d["cache"],
                                    d["block_tables"], d["seq_lens"], Lq, d["block_size"], d["window"])
    g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
    assert_close(g, r, f"draft attention sublayer ({requests} requests)")
    # the output is small (~0.1 RMS): also bound the error relative to its RMS
    rel = np.abs(g - r).max() / np.sqrt(np.mean(r * r))
    assert rel < 0.05, rel
    gc = host_bf16(cache)
    written = np.any(gc != d["cache"], axis=-1)
    assert np.array_equal(written, np.any(rcache != d["cache"], axis=-1)), "written cache rows"
    assert_close(O.bf16_to_f64(gc), O.bf16_to_f64(rcache), "cache after the sublayer")
    say(f"[draft attention {requests} requests] max|d|/rms(ref) = {rel:.4f}")
