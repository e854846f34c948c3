"""GPU parity of dflash_context_kv against the oracle (DFlash2BeamModel
precompute_and_store_context_kv: hidden_norm RMSNorm, the stacked K/V linear of
every draft layer, then each layer's K-norm + NeoX RoPE and the slot-mapped
write of K and V into that layer's cache)."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL
from tests.parity import assert_close

pytestmark = pytest.mark.gpu

SENTINEL = 0xFFFF  # a bf16 NaN pattern no write produces


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_candidate_amd as B
    B.lib()
    return B


def _cache_shape(d):
    return (d["num_blocks"], d["hkv"], d["block_size"], 2 * d["head_dim"])


def _run(B, d, with_cache=True, want_kv=True):
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    L, D = d["layers"], d["head_dim"]
    cs = B.rope_cos_sin(d["max_pos"], D, d["theta"], "cuda")
    caches = None
    if with_cache:
        caches = [torch.full(_cache_shape(d), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
                  for _ in range(L)]
    kv = B.context_kv(dev_bf16(d["ctx_states"]), dev_bf16(d["hidden_norm_w"]), d["eps"], dev_bf16(d["W_kv"]),
                      L, d["hkv"], D, dev_bf16(d["k_norm_w"]), d["eps"], dev(d["positions"]), cs,
                      dev(d["slots"]) if with_cache else None, caches, want_kv=want_kv)
    torch.cuda.synchronize()
    return (None if kv is None else host_bf16(kv),
            None if caches is None else [host_bf16(c) for c in caches])


def _oracle_caches(d, kv):
    c0 = [np.full(_cache_shape(d), SENTINEL, np.uint16) for _ in range(d["layers"])]
    return O.store_context_kv(kv, d["k_norm_w"], d["eps"], d["positions"], d["theta"], d["slots"], c0,
                              d["block_size"])


def _check(B, d, label):
    from tests.gpu_common import say
    D = d["head_dim"]
    kv, caches = _run(B, d)
    ref_kv = O.context_kv(d["ctx_states"], d["hidden_norm_w"], d["eps"], d["W_kv"], d["layers"], d["hkv"], D)
    assert kv.shape == ref_kv.shape
    assert_close(O.bf16_to_f64(kv), O.bf16_to_f64(ref_kv), label + " kv (stacked linear)")
    ref_caches = _oracle_caches(d, ref_kv)
    # the same K path on exactly the GPU's linear output: isolates the norm/RoPE
    own_caches = _oracle_caches(d, kv)
    k_ulps = 0
    for l in range(d["layers"]):
        g, r, o = caches[l], ref_caches[l], own_caches[l]
        written = np.any(g != SENTINEL, axis=-1)
        assert np.array_equal(written, np.any(r != SENTINEL, axis=-1)), f"{label}: written rows of layer {l}"
        w = written
        assert_close(O.bf16_to_f64(g[..., :D][w]), O.bf16_to_f64(r[..., :D][w]), f"{label} K layer {l}")
        assert_close(O.bf16_to_f64(g[..., D:][w]), O.bf16_to_f64(r[..., D:][w]), f"{label} V layer {l}")
        assert np.array_equal(g[..., D:], o[..., D:]), f"{label}: V payload != the linear's output (layer {l})"
        assert_close(O.bf16_to_f64(g[..., :D][w]), O.bf16_to_f64(o[..., :D][w]),
                     f"{label} K layer {l} (same linear output)")
        k_ulps += int(np.count_nonzero(g[..., :D][w] != o[..., :D][w]))
    n_kv = int(np.count_nonzero(kv != ref_kv))
    say(f"[context_kv {label}] linear outputs differing from the oracle by rounding: {n_kv} of {kv.size}; "
        f"K differing on equal linear outputs: {k_ulps}")
    return kv, caches


def test_context_kv_small(B):
    _check(B, WL.context_kv_inputs("ctx_small"), "small")


def test_context_kv_small_with_padding_slots(B):
    d = WL.context_kv_inputs("ctx_small", pad_fraction=0.1)
    assert (d["slots"] < 0).sum() > 0
    _check(B, d, "small+pad")


def test_context_kv_without_cache(B):
    # no slots / caches: the linear alone (the pages' profiling run); kv_out is
    # still the stacked output
    d = WL.context_kv_inputs("ctx_small")
    kv, caches = _run(B, d, with_cache=False)
    assert caches is None
    ref_kv = O.context_kv(d["ctx_states"], d["hidden_norm_w"], d["eps"], d["W_kv"], d["layers"], d["hkv"],
                          d["head_dim"])
    assert_close(O.bf16_to_f64(kv), O.bf16_to_f64(ref_kv), "kv without cache")


def test_context_kv_single_token_one_layer(B):
    d = WL.context_kv_inputs("ctx_small")
    n = 1
    D, Hkv = d["head_dim"], d["hkv"]
    d = dict(d, ctx_states=d["ctx_states"][:n], positions=d["positions"][:n], slots=d["slots"][:n],
             layers=1, W_kv=d["W_kv"][:2 * Hkv * D], k_norm_w=d["k_norm_w"][:1])
    _check(B, d, "n=1,L=1")


def test_context_kv_wide_tiles(B):
    # 4096 tokens x 8192 columns: the 256-column tile variant (with the K tail)
    _check(B, WL.context_kv_inputs("ctx_wide", pad_fraction=0.05), "wide")


def test_context_kv_full_workload(B):
    # 128 requests x 16 context tokens, hidden 4096, 5 layers of 8 kv heads
    d = WL.context_kv_inputs("ctx")
    kv, caches = _check(B, d, "full")
    # without kv_out the cache contents are the same bits
    _, caches2 = _run(B, d, want_kv=False)
    for l in range(d["layers"]):
        assert np.array_equal(caches[l], caches2[l]), f"layer {l}: cache differs without kv_out"


@pytest.mark.parametrize("Hd", [6144, 8200])
def test_context_kv_wide_hidden(B, Hd):
    # hidden sizes past the 2-chunk-per-thread norm path (4 chunks; the general loop)
    rng = np.random.default_rng(Hd)
    n, L, Hkv, D = 37, 1, 1, 128
    d = dict(ctx_states=WL.to_bf16_bits(rng.standard_normal((n, Hd)).astype(np.float32)),
             hidden_norm_w=WL.to_bf16_bits((1 + 0.1 * rng.standard_normal(Hd)).astype(np.float32)),
             W_kv=WL.to_bf16_bits((0.02 * rng.standard_normal((L * 2 * Hkv * D, Hd))).astype(np.float32)),
             k_norm_w=WL.to_bf16_bits((1 + 0.1 * rng.standard_normal((L, D))).astype(np.float32)),
             positions=rng.integers(0, 5000, n).astype(np.int64), slots=rng.permutation(64 * 16)[:n].astype(np.int64),
             num_ctx=n, hidden=Hd, layers=L, hkv=Hkv, head_dim=D, block_size=16, num_blocks=64, eps=1e-6,
             theta=1e6, max_pos=5000)
    _check(B, d, f"hidden {Hd}")
