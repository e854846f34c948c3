"""GPU parity of the RoPE options (dflash_qk_norm_rope_cache_ex,
dflash_context_kv_ex: partial rotary dim, GPT-J pairing, bf16 cos/sin table)
against the oracle, and of the plain calls against the _ex calls' defaults."""
import ctypes

import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL
from tests.parity import assert_close

pytestmark = pytest.mark.gpu

VARIANTS = [(False, 128, False), (True, 64, False), (False, 32, True), (True, 128, True), (True, 16, False),
            (False, 8, True), (False, 72, False)]


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_candidate_amd as B
    B.lib()
    return B


def _table(B, max_pos, rot, theta, bf16):
    import torch
    return B.rope_cos_sin(max_pos, rot, theta, "cuda", dtype=torch.bfloat16 if bf16 else torch.float32)


@pytest.mark.parametrize("neox,rot,bf16", VARIANTS)
def test_qk_rope_variants(B, neox, rot, bf16):
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    d = WL.qk_inputs("mid", pad_fraction=0.1)
    D = d["head_dim"]
    cs = _table(B, d["max_pos"], rot, d["theta"], bf16)
    cache0 = np.full_like(d["cache"], 0xFFFF)
    cache = dev_bf16(cache0)
    q, k = B.qk_norm_rope_cache(dev_bf16(d["qkv"]), d["hq"], d["hkv"], D, dev_bf16(d["q_w"]), dev_bf16(d["k_w"]),
                                d["eps"], dev(d["positions"]), cs, dev(d["slots"]), cache, rotary_dim=rot,
                                is_neox=neox)
    torch.cuda.synchronize()
    rq, rk, rc = O.qk_norm_rope_cache(d["qkv"], d["hq"], d["hkv"], D, d["q_w"], d["k_w"], d["eps"], d["positions"],
                                      d["theta"], d["slots"], cache0, d["block_size"], rotary_dim=rot, neox=neox,
                                      table="bf16" if bf16 else "f64")
    tag = f"neox={neox} rot={rot} bf16={bf16}"
    assert_close(O.bf16_to_f64(host_bf16(q)), O.bf16_to_f64(rq), tag + " q")
    assert_close(O.bf16_to_f64(host_bf16(k)), O.bf16_to_f64(rk), tag + " k")
    gc = host_bf16(cache)
    assert np.array_equal(np.any(gc != 0xFFFF, axis=-1), np.any(rc != 0xFFFF, axis=-1)), tag + " written rows"
    assert np.array_equal(gc[..., D:], rc[..., D:]), tag + " V bits"
    # the unrotated tail is the plain norm: equal to position 0's output there
    if rot < D:
        q0, _ = B.qk_norm_rope_cache(dev_bf16(d["qkv"]), d["hq"], d["hkv"], D, dev_bf16(d["q_w"]),
                                     dev_bf16(d["k_w"]), d["eps"], torch.zeros_like(dev(d["positions"])), cs,
                                     rotary_dim=rot, is_neox=neox)
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16(q)[..., rot:], host_bf16(q0)[..., rot:]), tag + " tail"


def test_bf16_table_matches_the_oracle_rounding(B):
    import torch
    from tests.gpu_common import host_bf16
    pos = np.arange(0, 9000, 7)
    t = host_bf16(_table(B, 9000, 64, 1e6, True))[pos]
    torch.cuda.synchronize()
    c, s = O.rope_cos_sin(pos, 64, 1e6, "bf16")
    assert np.array_equal(O.bf16_to_f64(t[:, :32]), c)
    assert np.array_equal(O.bf16_to_f64(t[:, 32:]), s)


@pytest.mark.parametrize("neox,rot,bf16", [(False, 128, True), (True, 64, False), (False, 24, False)])
def test_context_kv_rope_variants(B, neox, rot, bf16):
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    d = WL.context_kv_inputs("ctx_small", pad_fraction=0.1)
    L, D, Hkv = d["layers"], d["head_dim"], d["hkv"]
    cs = _table(B, d["max_pos"], rot, d["theta"], bf16)
    shape = (d["num_blocks"], Hkv, d["block_size"], 2 * D)
    caches = [torch.full(shape, -1, dtype=torch.int16, device="cuda").view(torch.bfloat16) for _ in range(L)]
    kv = B.context_kv(dev_bf16(d["ctx_states"]), dev_bf16(d["hidden_norm_w"]), d["eps"], dev_bf16(d["W_kv"]), L,
                      Hkv, D, dev_bf16(d["k_norm_w"]), d["eps"], dev(d["positions"]), cs, dev(d["slots"]), caches,
                      want_kv=True, rotary_dim=rot, is_neox=neox)
    torch.cuda.synchronize()
    kvh = host_bf16(kv)
    # the K path on exactly the GPU's linear output
    c0 = [np.full(shape, 0xFFFF, np.uint16) for _ in range(L)]
    ref = O.store_context_kv(kvh, d["k_norm_w"], d["eps"], d["positions"], d["theta"], d["slots"], c0,
                             d["block_size"], rotary_dim=rot, neox=neox, table="bf16" if bf16 else "f64")
    tag = f"neox={neox} rot={rot} bf16={bf16}"
    for l in range(L):
        g = host_bf16(caches[l])
        w = np.any(g != 0xFFFF, axis=-1)
        assert np.array_equal(w, np.any(ref[l] != 0xFFFF, axis=-1)), tag + " written rows"
        assert np.array_equal(g[..., D:], ref[l][..., D:]), tag + " V bits"
        assert_close(O.bf16_to_f64(g[..., :D][w]), O.bf16_to_f64(ref[l][..., :D][w]), f"{tag} K layer {l}")


def test_plain_calls_equal_the_ex_defaults(B):
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    d = WL.qk_inputs("mid")
    D = d["head_dim"]
    cs = B.rope_cos_sin(d["max_pos"], D, d["theta"], "cuda")
    qkv, qw, kw, pos = dev_bf16(d["qkv"]), dev_bf16(d["q_w"]), dev_bf16(d["k_w"]), dev(d["positions"])
    q1, k1 = B.qk_norm_rope_cache(qkv, d["hq"], d["hkv"], D, qw, kw, d["eps"], pos, cs)
    q2 = torch.empty_like(q1)
    k2 = torch.empty_like(k1)
    st = B.lib().dflash_qk_norm_rope_cache(qkv.data_ptr(), qkv.stride(0), qkv.shape[0], d["hq"], d["hkv"], D,
                                           qw.data_ptr(), kw.data_ptr(), ctypes.c_float(d["eps"]), pos.data_ptr(),
                                           cs.data_ptr(), cs.shape[0], None, None, 0, 0, q2.data_ptr(),
                                           k2.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert np.array_equal(host_bf16(q1), host_bf16(q2)) and np.array_equal(host_bf16(k1), host_bf16(k2))
