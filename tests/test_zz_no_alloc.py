"""dflash_lm_topk_noalloc (partial lists in the library's static device
scratch, no workspace argument) against dflash_lm_topk with a caller workspace,
through the C ABI: the same kernels, so ids and logits must be bit-identical.
Two calls in a row, the second smaller, reuse the same scratch."""
import ctypes

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


def _case(seed, T, V, Hd):
    rng = np.random.default_rng(seed)
    H = WL.to_bf16_bits(rng.standard_normal((T, Hd), dtype=np.float32))
    W = WL.to_bf16_bits(rng.standard_normal((V, Hd), dtype=np.float32) * np.float32(0.05))
    return H, W


def _both(B, H, W, k, s, c):
    import torch
    from tests.gpu_common import dev_bf16, say
    Hd_, Wd_ = dev_bf16(H), dev_bf16(W)
    T, Hd = H.shape
    V = W.shape[0]
    ids0, lg0 = B.lm_topk(Hd_, Wd_, k, s, c)
    ids1 = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    lg1 = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    st = B.lib().dflash_lm_topk_noalloc(Hd_.data_ptr(), Wd_.data_ptr(), T, V, Hd, k, s, c, ids1.data_ptr(),
                                        lg1.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().dflash_status_string(st)
    torch.cuda.synchronize()
    a0, a1 = ids0.cpu().numpy(), ids1.cpu().numpy()
    assert np.array_equal(a0, a1), "ids differ from dflash_lm_topk"
    assert np.array_equal(lg0.cpu().numpy().view(np.uint32), lg1.cpu().numpy().view(np.uint32)), \
        "logits differ from dflash_lm_topk"
    ws = B.lm_topk_workspace_size(T, V, Hd, k)
    say(f"[noalloc] T={T} V={V} Hd={Hd} k={k}: {ws / 2**20:.2f} MiB of scratch, outputs identical")
    return ws


def test_noalloc_equals_the_workspace_call_twice(B):
    # first call: the largest problem the 16 MiB scratch holds (8192 rows, k = 32),
    # then a smaller ragged one that reuses what the first left there
    H, W = _case(1, 8192, 20000, 64)
    assert _both(B, H, W, 32, 0.5, 30.0) == 16 << 20
    H, W = _case(2, 300, 5003, 200)
    assert _both(B, H, W, 7, 1.0, 0.0) < 16 << 20


def test_noalloc_full_workload_then_mid(B):
    from tests.gpu_common import candidate
    d = candidate("full")
    _both(B, d["H"], d["W"], d["top_k"], d["multiplier"], d["softcap"])
    m = WL.candidate_inputs("mid")
    _both(B, m["H"], m["W"], m["top_k"], m["multiplier"], m["softcap"])


def test_noalloc_rejects_a_problem_beyond_the_scratch(B):
    import torch
    T, V, Hd, k = 8193, 20000, 64, 32
    H = torch.zeros((T, Hd), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((V, Hd), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    lg = torch.empty((T, k), dtype=torch.float32, device="cuda")
    st = B.lib().dflash_lm_topk_noalloc(H.data_ptr(), W.data_ptr(), T, V, Hd, k, 1.0, 0.0, ids.data_ptr(),
                                        lg.data_ptr(), None)
    assert st == 5 and b"scratch" in B.lib().dflash_status_string(st)
    with pytest.raises(B.DFlashError):
        B.lm_topk_noalloc(H, W, k)
