"""The C ABI without a GPU: libdflash.so loads, exports every entry point that
include/dflash.h declares, and rejects bad arguments on the host before any
launch (the error paths a test can force from the host)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


@pytest.fixture(scope="module")
def L():
    import block_draft_candidate_amd as B
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libdflash.so not built")
    return B.lib()


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(6):
        assert L.dflash_status_string(code)
    assert L.dflash_status_string(99) == b"unknown status"
    assert L.dflash_version() >= 100


FAKE = 1 << 20  # an aligned, never dereferenced address: only host checks run


@pytest.fixture(autouse=True)
def _no_gpu_for_fake_pointers(request):
    # The validation tests pass fake device addresses; they must never reach a
    # real launch, so they run only where no GPU is visible.
    if "validation" in request.node.name:
        import torch
        if torch.cuda.device_count() > 0:
            pytest.skip("fake-pointer validation tests run on a host without a GPU")


def test_lm_topk_host_validation(L):
    f = L.dflash_lm_topk
    ok = dict(H=FAKE, W=FAKE, T=8, V=1024, Hd=256, k=4, s=1.0, c=0.0, ids=FAKE, lg=FAKE, ws=FAKE)
    ws = L.dflash_lm_topk_workspace_size(8, 1024, 256, 4)
    assert ws > 0

    def call(**o):
        a = dict(ok, **o)
        return f(a["H"], a["W"], a["T"], a["V"], a["Hd"], a["k"], a["s"], a["c"], a["ids"], a["lg"],
                 a["ws"], a.get("wsb", 0), None)

    assert call(H=None, wsb=ws) == 1
    assert call(H=FAKE + 2, wsb=ws) == 1          # misaligned
    assert call(k=0, wsb=ws) == 1
    assert call(k=2000, wsb=ws) == 1              # k > V
    assert call(s=0.0, wsb=ws) == 1               # multiplier must be > 0
    assert call(s=float("inf"), wsb=ws) == 1
    assert call(c=float("nan"), wsb=ws) == 1
    assert call(k=65, V=4096, wsb=ws) == 2        # k > 64 unsupported
    assert call(Hd=260, wsb=ws) == 2              # Hd % 8
    assert call(Hd=1 << 22, wsb=ws) == 2          # 256 rows of Hd bf16 overflow an int32 byte count
    assert call(wsb=ws - 1) == 3                  # workspace too small
    assert L.dflash_lm_topk_workspace_size(0, 1, 1, 1) == 0


def test_lm_topk_noalloc_host_validation(L):
    """The no-alloc call checks its arguments like dflash_lm_topk and rejects a
    problem whose partial lists exceed the library's 16 MiB scratch, all on the
    host before any HIP call."""
    f = L.dflash_lm_topk_noalloc

    def call(T=8, V=1024, Hd=256, k=4, ids=FAKE):
        return f(FAKE, FAKE, T, V, Hd, k, 1.0, 0.0, ids, FAKE, None)

    assert call(ids=None) == 1
    assert call(k=0) == 1
    assert call(Hd=260) == 2
    assert L.dflash_lm_topk_workspace_size(8192, 20000, 64, 32) == 16 << 20   # fits exactly
    assert L.dflash_lm_topk_workspace_size(8193, 20000, 64, 32) > 16 << 20
    assert call(T=8193, V=20000, Hd=64, k=32) == 5                             # DFLASH_ERR_SCRATCH


def test_edges_host_validation(L):
    f = L.dflash_candidate_edges
    ws = L.dflash_candidate_edges_workspace_size(8, 16, 256)
    assert ws > 0

    def call(**o):
        a = dict(Rq=2, S=4, k=4, V=1024, R=16, Hd=256, wsb=ws, anchor=FAKE)
        a.update(o)
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["anchor"], a["Rq"], a["S"], a["k"], a["V"], a["R"],
                 a["Hd"], FAKE, FAKE, a["wsb"], None)

    assert call(anchor=None) == 1
    assert call(k=0) == 1
    assert call(R=24) == 2          # R % 16
    assert call(R=512) == 2         # R > 256
    assert call(k=65, V=4096) == 2
    assert call(Hd=1 << 22) == 2    # 256 rows of Hd bf16 overflow an int32 byte count
    assert call(wsb=ws - 4) == 3


def test_qk_host_validation(L):
    f = L.dflash_qk_norm_rope_cache

    def call(slots=FAKE, cache=FAKE, kout=FAKE, D=128, stride=24 * 128, eps=1e-6):
        return f(FAKE, stride, 288, 16, 4, D, FAKE, FAKE, eps, FAKE, FAKE, 4096, slots, cache, 256, 16,
                 FAKE, kout, None)

    assert call(slots=None) == 1            # exactly one of slots / cache
    assert call(slots=None, cache=None, kout=None) == 1  # nothing to write K to
    assert call(D=64) == 2
    assert call(stride=100) == 1
    assert call(eps=-1.0) == 1
    assert L.dflash_rope_cos_sin(None, 10, 128, 1e6, None) == 1
    assert L.dflash_rope_cos_sin(FAKE, 10, 127, 1e6, None) == 1


def test_attn_host_validation(L):
    f = L.dflash_block_attn

    def call(Lq=16, Hq=32, Hkv=8, D=128, bs=16, window=2048, scale=0.088):
        return f(FAKE, FAKE, 100, FAKE, 10, FAKE, 4, Lq, Hq, Hkv, D, bs, window, scale, FAKE, None, 0, None)

    assert call(Hq=30) == 1          # Hq % Hkv
    assert call(window=0) == 1
    assert call(scale=0.0) == 1
    assert call(Lq=17) == 2
    assert call(D=64) == 2
    assert call(bs=32) == 2
    assert call(Hq=24, Hkv=2) == 2   # group of 12 heads
    assert L.dflash_block_attn_workspace_size(4, 16, 32, 128) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import block_draft_candidate_amd as B
    monkeypatch.setattr(B, "_LIB", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(B.DFlashError):
        B.lib()


def test_lm_topk_proj_host_validation(L):
    f = L.dflash_lm_topk_proj
    ws = L.dflash_lm_topk_workspace_size(8, 1024, 256, 4)

    def call(Wp=FAKE, R=16, hp=FAKE, wsb=ws, k=4):
        return f(FAKE, FAKE, 8, 1024, 256, k, 1.0, 0.0, Wp, R, FAKE, FAKE, hp, FAKE, wsb, None)

    assert call(Wp=None) == 1
    assert call(hp=None) == 1
    assert call(hp=FAKE + 4) == 1    # misaligned
    assert call(R=0) == 1
    assert call(R=5000) == 2
    assert call(k=0) == 1            # the LM-head checks still apply
    assert call(wsb=ws - 1) == 3


def test_edges_hp_host_validation(L):
    f = L.dflash_candidate_edges_hp

    def call(hp=FAKE, k=4, V=1024, R=16):
        return f(FAKE, FAKE, FAKE, FAKE, hp, FAKE, 2, 4, k, V, R, FAKE, None)

    assert call(hp=None) == 1
    assert call(k=0) == 1
    assert call(R=24) == 2          # R % 16
    assert call(R=512) == 2         # R > 256
    assert call(k=65, V=4096) == 2


def test_context_kv_host_validation(L):
    f = L.dflash_context_kv
    n, Hd, Lyr, Hkv, D = 300, 320, 2, 2, 128
    ws = L.dflash_context_kv_workspace_size(n, Hd)
    assert ws == n * Hd * 2
    assert L.dflash_context_kv_workspace_size(0, Hd) == 0
    caches = (ctypes.c_void_p * 64)(*([FAKE] * 64))
    bad = (ctypes.c_void_p * 2)(FAKE, FAKE + 8)

    def call(ctx=FAKE, slots=FAKE, cp=caches, Lyr=Lyr, D=D, Hd=Hd, wsb=ws, eps=1e-6, kvo=None, nblk=64):
        return f(ctx, FAKE, eps, FAKE, n, Hd, Lyr, Hkv, D, FAKE, 1e-6, FAKE, FAKE, 4096, slots,
                 ctypes.cast(cp, ctypes.c_void_p) if cp is not None else None, nblk, 16, kvo, FAKE, wsb, None)

    assert call(ctx=None) == 1
    assert call(ctx=FAKE + 2) == 1        # misaligned
    assert call(slots=None) == 1          # exactly one of slots / caches
    assert call(cp=None) == 1
    assert call(cp=bad) == 1              # a misaligned layer cache
    assert call(nblk=0) == 1
    assert call(eps=-1.0) == 1
    assert call(kvo=FAKE + 4) == 1
    assert call(D=64) == 2
    assert call(Hd=324) == 2              # Hd % 8
    assert call(Lyr=65) == 2
    assert call(wsb=ws - 1) == 3


def test_linear_host_validation(L):
    f = L.dflash_linear

    def call(X=FAKE, M=300, N=200, K=328, ldy=200, Y=FAKE):
        return f(X, FAKE, M, N, K, Y, ldy, None)

    assert call(X=None) == 1
    assert call(Y=FAKE + 2) == 1
    assert call(M=0) == 1
    assert call(ldy=192) == 1        # ldy < N
    assert call(N=201, ldy=208) == 2  # N % 8
    assert call(K=330) == 2          # K % 8
    assert call(ldy=204) == 2        # ldy % 8


def test_rope_options_host_validation(L):
    f = L.dflash_qk_norm_rope_cache_ex

    def call(rot=128, neox=1, tb=0, f8=0, sc=None):
        return f(FAKE, 24 * 128, 288, 16, 4, 128, FAKE, FAKE, 1e-6, FAKE, FAKE, 4096, rot, neox, tb, FAKE, FAKE,
                 256, 16, f8, sc, FAKE, None, None)

    assert call(rot=127) == 1        # odd
    assert call(rot=0) == 1
    assert call(rot=256) == 1        # > D
    assert call(tb=2) == 1
    assert call(neox=3) == 1
    assert call(rot=24) == 2         # NeoX needs a multiple of 16
    assert call(rot=20, neox=0) == 2  # GPT-J needs a multiple of 8
    assert call(f8=3) == 1           # cache dtype code
    assert call(f8=1) == 1           # fp8 without scales
    assert call(f8=2, sc=FAKE + 2) == 1  # misaligned scales
    g = L.dflash_context_kv_ex
    caches = (ctypes.c_void_p * 2)(FAKE, FAKE)
    ws = L.dflash_context_kv_workspace_size(300, 328)

    def callc(rot=128, neox=1, tb=0, f8=0, sc=None):
        return g(FAKE, FAKE, 1e-6, FAKE, 300, 328, 2, 2, 128, FAKE, 1e-6, FAKE, FAKE, 4096, rot, neox, tb, FAKE,
                 ctypes.cast(caches, ctypes.c_void_p), 64, 16, f8, sc, None, FAKE, ws, None)

    assert callc(rot=130) == 1
    assert callc(tb=-1) == 1
    assert callc(rot=40) == 2
    assert callc(f8=-1) == 1
    assert callc(f8=1) == 1          # fp8 without scales
    assert L.dflash_rope_cos_sin_bf16(None, 10, 64, 1e6, None) == 1


def test_attn_fp8_host_validation(L):
    f = L.dflash_block_attn_ex

    def call(f8=1, sc=FAKE):
        return f(FAKE, FAKE, 100, FAKE, 10, FAKE, 4, 16, 32, 8, 128, 16, 2048, 0.088, f8, sc, FAKE, None, 0, None)

    assert call(f8=3) == 1
    assert call(sc=None) == 1
    assert call(sc=FAKE + 2) == 1
