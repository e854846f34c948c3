"""The seeded input generators: fixed bits for a given seed, independent of the
thread count, and prefix-stable when a workload is shrunk."""
import numpy as np

import workloads as WL


def test_normal_is_thread_count_independent(monkeypatch):
    a = WL.normal_f32(7, 1, (1 << 23) + 5)
    monkeypatch.setattr(WL, "_threads", lambda: 1)
    b = WL.normal_f32(7, 1, (1 << 23) + 5)
    assert np.array_equal(a, b)
    assert abs(float(a.mean())) < 1e-3 and abs(float(a.std()) - 1) < 1e-3


def test_bf16_normal_matches_float_draws():
    x = WL.normal_f32(3, 2, 1000, 0.02)
    b = WL.bf16_normal(3, 2, (10, 100), 0.02)
    back = (b.astype(np.uint32) << 16).view(np.float32).reshape(-1)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)


def test_candidate_inputs_prefix_and_shapes():
    a = WL.candidate_inputs("tiny")
    b = WL.candidate_inputs("tiny", requests=1)
    assert a["H"].shape == (8, 256) and a["W"].shape == (1024, 256)
    assert np.array_equal(a["H"][:4], b["H"]) and np.array_equal(a["ids"][:1], b["ids"])
    for row in a["ids"].reshape(-1, a["top_k"]):
        assert len(set(row)) == len(row)


def test_mantissa_rounding():
    bits = np.array([0x3F80, 0x3F81, 0x3F84, 0x3F8C, 0x3FFF, 0xBF84], dtype=np.uint16)
    r = WL.keep_mantissa_bits(bits, 4)
    # keep 4 of 7 mantissa bits: step 8 in the low bits, ties to even
    assert list(r) == [0x3F80, 0x3F80, 0x3F80, 0x3F90, 0x4000, 0xBF80]


def test_attention_layout():
    d = WL.attention_inputs("attn", requests=4)
    bs = d["block_size"]
    assert np.all(d["seq_lens"] == d["ctx"] + d["query_len"])
    # slots of the query block point into the request's own blocks
    r = np.repeat(np.arange(4), d["query_len"])
    assert np.all(d["slots"] // bs == d["block_tables"][r, d["positions"] // bs])


def test_context_kv_inputs_layout():
    d = WL.context_kv_inputs("ctx_small", pad_fraction=0.1)
    n, bs = d["num_ctx"], d["block_size"]
    s = d["slots"]
    live = s[s >= 0]
    assert len(set(live.tolist())) == live.size                    # one token per slot
    assert live.max() < d["num_blocks"] * bs
    assert np.array_equal(live % bs, d["positions"][s >= 0] % bs)  # offset in block = position % bs
    assert (s < 0).any()
    assert d["W_kv"].shape == (d["layers"] * 2 * d["hkv"] * d["head_dim"], d["hidden"])
    assert d["k_norm_w"].shape == (d["layers"], d["head_dim"])
    assert d["hidden"] % 64 != 0                                   # the K-tail case
    assert n % 256 != 0 and n > 256                                # a ragged second row tile
