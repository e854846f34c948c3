#!/usr/bin/env python3
"""Benchmark of the DFlash2 block-draft candidate step on one MI355X.

One step = the whole hot path over one synthetic batch, inputs resident in HBM:
  1. dflash_lm_topk_proj       256 requests x 16 steps, vocab 151936, hidden 4096, top_k 16,
                               output_multiplier 0.5, softcap 30, and the selector's rank-128
                               projection of the same hidden states in the same pass
  2. dflash_candidate_edges_hp edge scores of the same rows from step 1's ids, logits and
                               projection
  3. dflash_qk_norm_rope_cache draft-layer query block, 128 requests x 16 tokens, 32/8 heads
  4. dflash_block_attn         the same block over the paged cache, window 2048,
                               context lengths uniform in [512, 8192]
With --two-kernel-edges, steps 1-2 are dflash_lm_topk and dflash_candidate_edges
(projection and edges in their own two kernels).

Also timed, on its own and outside the step: dflash_context_kv, the context
K/V precompute of 2048 context tokens for 5 draft layers (reported under
kernels.context_kv), and dflash_linear as the draft layer's qkv_proj (2048 x
6144 x 4096) and o_proj (2048 x 4096 x 4096) (kernels.linear_*).

Prints one JSON line.  `value` is edge scores per second of the whole step.
Per-kernel times come from HIP events on the stream the kernels run on; the
roofline object is for the dominant kernel (the LM-head top-k, MFMA-bound).

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline]
    python bench.py --copy-probe-mib 1024     # plain copy, for counter calibration
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "edge scores/s + LM-head top-k GB/s as % of HBM peak, 256 reqs×16 steps"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
LM_SOURCES = [os.path.join(ROOT, "block_draft_candidate_amd", "csrc", f) for f in ("lm_topk.hip", "common.h")]


def kernel_fingerprint():
    """SHA-256 of the LM-head kernel's code (its source and the shared header)
    with comments and whitespace removed: a comment edit keeps stored counter
    figures valid, any code change invalidates them."""
    import re
    h = hashlib.sha256()
    for path in LM_SOURCES:
        src = open(path).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(re.sub(r"\s+", "", src).encode())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def lm_bytes(T, V, Hd, k, R=0):
    """W, H, ids + logits; with the rank projection (R > 0) also W_proj and hp."""
    return V * Hd * 2 + T * Hd * 2 + T * k * 8 + R * Hd * 2 + T * R * 4


def lm_flops(T, V, Hd, R=0):
    return 2 * T * (V + R) * Hd


def edge_bytes(Rq, S, k, R, Hd, from_hp=False):
    """Gathered codebook rows, ids, unary logits, anchors, edges, and either H +
    W_proj (projection inside) or hp (given)."""
    T = Rq * S
    gathers = Rq * (1 + (S - 1) * k) * R * 2 + Rq * S * k * R * 2
    proj = T * R * 4 if from_hp else T * Hd * 2 + R * Hd * 2
    return proj + gathers + T * k * 4 * 2 + Rq * 4 + T * k * k * 4


def qk_bytes(Tq, Hq, Hkv, D):
    return (Tq * (Hq + 2 * Hkv) * D * 2 + 2 * D * 2 + Tq * 8 * 2 + Tq * D * 4
            + Tq * Hq * D * 2 + Tq * Hkv * 2 * D * 2)


def attn_work(seq_lens, Lq, Hq, Hkv, D, window):
    """Algorithmic bytes (each visible K/V row once per kv head, q, out) and flops."""
    import numpy as np
    L = np.asarray(seq_lens, np.int64)
    lo0 = np.maximum(0, L - Lq - window + 1)
    keys = L - lo0
    nbytes = int(keys.sum()) * Hkv * 2 * D * 2 + 2 * len(L) * Lq * Hq * D * 2
    vis = 0
    for i in range(Lq):
        lo = np.maximum(0, L - Lq + i - window + 1)
        vis += int((L - lo).sum())
    flops = 4 * D * Hq * vis
    return nbytes, flops


def context_kv_work(n, Hd, L, Hkv, D):
    """Algorithmic bytes (context states, hidden_norm and K-norm weights, W_kv,
    positions, slots, the tokens' RoPE rows, K and V written to every layer's
    cache) and flops of the stacked linear."""
    N = L * 2 * Hkv * D
    nbytes = n * Hd * 2 + Hd * 2 + N * Hd * 2 + L * D * 2 + n * 8 * 2 + n * D * 4 + n * N * 2
    return nbytes, 2 * n * N * Hd


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, key):
    """Reduce rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) of
    this benchmark and of --copy-probe-mib to HBM bytes per LM-head call (its
    tile kernel plus its merge), each counter scaled by what it reads for the
    plain copy of known size, and store them under `key` in
    profiles/traffic.json (lm_topk_proj_full: the benchmark's default path,
    lm_topk_full: --two-kernel-edges)."""
    import csv

    def per_kernel(d, counter):
        out = {}
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    def copy_kib(d, counter):
        vals = [max(v) for k, v in per_kernel(d, counter).items() if "copyBuffer" in k]
        return max(vals)

    expect = copy_mib * 1024.0  # KiB the copy reads and writes
    f_fetch = expect / copy_kib(copy_fetch_dir, "FETCH_SIZE")
    f_write = expect / copy_kib(copy_write_dir, "WRITE_SIZE")

    def lm_kib(d, counter):
        tot = 0.0
        for k, v in per_kernel(d, counter).items():
            if "lm_topk_tiles" in k or "lm_topk_merge" in k:
                tot += sum(v) / len(v)
        return tot

    fetch = lm_kib(fetch_dir, "FETCH_SIZE") * f_fetch * 1024
    write = lm_kib(write_dir, "WRITE_SIZE") * f_write * 1024
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[key] = {
        "code_sha256": kernel_fingerprint(),
        "hbm_bytes_per_launch": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
        "fetch_scale": f_fetch, "write_scale": f_write,
        "note": "FETCH_SIZE and WRITE_SIZE per dispatch of the tile and merge kernels (KiB), scaled by "
                f"the counters' reading for a plain {copy_mib} MiB device copy"}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def traffic_for(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
        if rec and rec.get("code_sha256") == kernel_fingerprint():
            return rec.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_step_sample(cand, attn, nr, na):
    """The oracle over nr candidate-head requests (LM-head top-k + edges) and na
    attention requests (q/k norm + RoPE + cache, then attention); seconds."""
    import numpy as np
    from oracle import dflash_oracle as O
    S, k = cand["steps"], cand["top_k"]
    rows = np.arange(nr * S)
    t0 = time.perf_counter()
    ids, vals = O.lm_topk(cand["H"], cand["W"], k, cand["multiplier"], cand["softcap"], rows=rows)
    O.candidate_edges(cand["P"], cand["S"], ids.reshape(nr, S, k), vals.reshape(nr, S, k), cand["H"][rows],
                      cand["Wp"], cand["anchor"][:nr])
    Lq, D = attn["query_len"], attn["head_dim"]
    q, _, c2 = O.qk_norm_rope_cache(attn["qkv"][:na * Lq], attn["hq"], attn["hkv"], D, attn["q_w"], attn["k_w"],
                                    attn["eps"], attn["positions"][:na * Lq], attn["theta"],
                                    attn["slots"][:na * Lq], attn["cache"], attn["block_size"])
    O.block_attn(q, c2, attn["block_tables"][:na], attn["seq_lens"][:na], Lq, attn["hq"], attn["hkv"], D,
                 attn["block_size"], attn["window"], D ** -0.5)
    return time.perf_counter() - t0


def cpu_baseline(cand, attn, edges_per_step, frac):
    """The oracle timed on a bounded sample of the step: 1/frac of its
    candidate-head requests and of its attention requests (64 of 256 and 32 of
    128 at the default 1/4), scaled to a whole step, with every host core; and
    on 1/64 of the step (4 and 2 requests) with one thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        cores = len(os.sched_getaffinity(0))
    nr = max(1, cand["requests"] // frac)
    na = max(1, attn["requests"] // frac)
    dt = oracle_step_sample(cand, attn, nr, na)
    single = None
    if threadpool_limits is not None:
        f1 = 64
        nr1, na1 = max(1, cand["requests"] // f1), max(1, attn["requests"] // f1)
        with threadpool_limits(limits=1):
            dt1 = oracle_step_sample(cand, attn, nr1, na1)
        s1 = cand["requests"] / nr1  # the sample is 1/s1 of the step's candidate head (and attention)
        single = {"value": edges_per_step / (dt1 * s1), "unit": "edge scores/s", "cores": 1,
                  "sample": f"{nr1} candidate-head and {na1} attention requests = 1/{s1:g} of a step, one BLAS "
                            f"thread: {dt1:.1f} s, scaled to a whole step"}
    scale = cand["requests"] / nr
    return {"value": edges_per_step / (dt * scale), "unit": "edge scores/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{nr} of {cand['requests']} candidate-head requests ({nr * cand['steps']} rows: LM-head "
                      f"top-k + edges) and {na} of {attn['requests']} attention requests (qk-norm/RoPE/cache + "
                      f"attention) = 1/{scale:g} of a step; {dt:.1f} s on the host with {cores} BLAS threads, scaled "
                      "to a whole step",
            "single_thread": single}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-kernel-edges", action="store_true",
                    help="LM head and edges as dflash_lm_topk + dflash_candidate_edges (projection in the edge "
                         "call) instead of dflash_lm_topk_proj + dflash_candidate_edges_hp")
    ap.add_argument("--no-context-kv", action="store_true",
                    help="skip the separately timed context K/V precompute (dflash_context_kv)")
    ap.add_argument("--no-draft-layer", action="store_true",
                    help="skip the separately timed draft-layer projections (dflash_linear qkv_proj / o_proj)")
    ap.add_argument("--no-hbm-regime", action="store_true",
                    help="skip the LM-head top-k at 256 rows (mid workload; full vocabulary, one position per "
                         "request), where it is HBM-bound")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the edge call at the tiny / mid / full / large configurations and the LM-head "
                         "top-k at tiny / large (context lines, not part of the step)")
    ap.add_argument("--cpu-sample", type=int, default=4,
                    help="the oracle baseline runs 1/N of the step's requests (default 4: about 10-20 s on 16 cores)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB three times and exit "
                         "(the reference point that scales the HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="reduce rocprofv3 counter directories to profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, copy_mib=1024,
                      key="lm_topk_full" if args.two_kernel_edges else "lm_topk_proj_full")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the LM head would shard by vocabulary "
              "and the other kernels by request, but no multi-GPU path is implemented.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_draft_candidate_amd as B
    import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib > 0:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_probe_mib} MiB three times")
        return
    B.lib()

    def dbf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    log("generating inputs ...")
    cand = WL.candidate_inputs("full")
    attn = WL.attention_inputs("attn")
    Rq, S, k, V, Hd, R = (cand["requests"], cand["steps"], cand["top_k"], cand["vocab"], cand["hidden"],
                          cand["rank"])
    T = Rq * S
    H, W = dbf(cand["H"]), dbf(cand["W"])
    P, Sc, Wp = dbf(cand["P"]), dbf(cand["S"]), dbf(cand["Wp"])
    anchor = torch.from_numpy(cand["anchor"]).to(dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    logits = torch.empty((T, k), dtype=torch.float32, device=dev)
    edges = torch.empty((Rq, S, k, k), dtype=torch.float32, device=dev)
    ws_lm = torch.empty(B.lm_topk_workspace_size(T, V, Hd, k), dtype=torch.uint8, device=dev)
    ws_e = torch.empty(B.candidate_edges_workspace_size(T, R, Hd), dtype=torch.uint8, device=dev)
    hp = torch.empty((T, R), dtype=torch.float32, device=dev)
    fused = not args.two_kernel_edges

    Lq, Hq, Hkv, D = attn["query_len"], attn["hq"], attn["hkv"], attn["head_dim"]
    Rq_a = attn["requests"]
    qkv = dbf(attn["qkv"])
    q_w, k_w = dbf(attn["q_w"]), dbf(attn["k_w"])
    positions = torch.from_numpy(attn["positions"]).to(dev)
    slots = torch.from_numpy(attn["slots"]).to(dev)
    cache = dbf(attn["cache"])
    tables = torch.from_numpy(attn["block_tables"]).to(dev)
    seq_lens = torch.from_numpy(attn["seq_lens"]).to(dev)
    cos_sin = B.rope_cos_sin(attn["max_pos"], D, attn["theta"], dev)
    q_out = torch.empty((Rq_a * Lq, Hq, D), dtype=torch.bfloat16, device=dev)
    a_out = torch.empty_like(q_out)
    torch.cuda.synchronize()

    names = ["lm_topk", "edges", "qk", "attn"]
    ev = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
    acc_ms = {n: [] for n in names}

    def step(timed):
        def call(n, fn):
            if timed:
                ev[n][0].record()
            fn()
            if timed:
                ev[n][1].record()
        if fused:
            call("lm_topk", lambda: B.lm_topk_proj(H, W, k, cand["multiplier"], cand["softcap"], Wp, ids, logits,
                                                   hp, ws_lm))
            call("edges", lambda: B.candidate_edges_hp(P, Sc, ids.view(Rq, S, k), logits.view(Rq, S, k), hp,
                                                       anchor, edges))
        else:
            call("lm_topk", lambda: B.lm_topk(H, W, k, cand["multiplier"], cand["softcap"], ids, logits, ws_lm))
            call("edges", lambda: B.candidate_edges(P, Sc, ids.view(Rq, S, k), logits.view(Rq, S, k), H, Wp,
                                                    anchor, edges, ws_e))
        call("qk", lambda: B.qk_norm_rope_cache(qkv, Hq, Hkv, D, q_w, k_w, attn["eps"], positions, cos_sin,
                                                slots, cache, q_out=q_out, want_k=False))
        call("attn", lambda: B.block_attn(q_out, cache, tables, seq_lens, Lq, attn["window"], out=a_out))
        if timed:
            torch.cuda.synchronize()
            for n in names:
                acc_ms[n].append(ev[n][0].elapsed_time(ev[n][1]))

    log(f"warmup {args.warmup} ...")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # whole-step wall clock, K steps back to back
    log(f"timing {args.steps} steps ...")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-kernel HIP-event times over the same number of steps
    for _ in range(args.steps):
        step(True)
    kms = {n: sum(acc_ms[n]) / len(acc_ms[n]) for n in names}
    kstat = {n: {"ms_median": sorted(acc_ms[n])[len(acc_ms[n]) // 2], "ms_min": min(acc_ms[n])} for n in names}

    edges_per_step = Rq * S * k * k
    value = edges_per_step / (ms_per_step / 1e3)

    # the context K/V precompute that precedes a draft step (every draft
    # layer's K/V of the step's new context tokens), timed on its own: it is
    # not part of the step above
    ctx_kernel = None
    if not args.no_context_kv:
        log("context K/V precompute ...")
        cx = WL.context_kv_inputs("ctx")
        n_c, Hd_c, L_c, Hkv_c, D_c = cx["num_ctx"], cx["hidden"], cx["layers"], cx["hkv"], cx["head_dim"]
        c_states, c_hw, c_W, c_kw = dbf(cx["ctx_states"]), dbf(cx["hidden_norm_w"]), dbf(cx["W_kv"]), dbf(cx["k_norm_w"])
        c_pos = torch.from_numpy(cx["positions"]).to(dev)
        c_slots = torch.from_numpy(cx["slots"]).to(dev)
        c_cs = B.rope_cos_sin(cx["max_pos"], D_c, cx["theta"], dev)
        c_caches = [torch.zeros((cx["num_blocks"], Hkv_c, cx["block_size"], 2 * D_c), dtype=torch.bfloat16,
                                device=dev) for _ in range(L_c)]
        c_ws = torch.empty(B.context_kv_workspace_size(n_c, Hd_c), dtype=torch.uint8, device=dev)

        def ctx_call():
            B.context_kv(c_states, c_hw, cx["eps"], c_W, L_c, Hkv_c, D_c, c_kw, cx["eps"], c_pos, c_cs, c_slots,
                         c_caches, workspace=c_ws)
        for _ in range(args.warmup):
            ctx_call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c_ms = 0.0
        for _ in range(args.steps):
            e0.record()
            ctx_call()
            e1.record()
            torch.cuda.synchronize()
            c_ms += e0.elapsed_time(e1)
        c_ms /= args.steps
        cb, cf = context_kv_work(n_c, Hd_c, L_c, Hkv_c, D_c)
        ctx_kernel = {"ms": c_ms, "TFLOP_per_s": cf / (c_ms * 1e-3) / 1e12,
                      "mfma_frac": cf / (c_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                      "GB_per_s": cb / (c_ms * 1e-3) / 1e9, "hbm_frac": cb / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "algorithmic_bytes": cb, "flops": cf,
                      "workload": f"{n_c} context tokens (128 requests x 16), hidden {Hd_c}, {L_c} draft layers x "
                                  f"{Hkv_c} kv heads x head_dim {D_c}; hidden_norm + stacked K/V linear + K-norm/RoPE "
                                  "+ cache writes (not part of the step)"}

    Rp = R if fused else 0
    lmb, lmf = lm_bytes(T, V, Hd, k, Rp), lm_flops(T, V, Hd, Rp)
    eb = edge_bytes(Rq, S, k, R, Hd, from_hp=fused)
    qb = qk_bytes(Rq_a * Lq, Hq, Hkv, D)
    ab, af = attn_work(attn["seq_lens"], Lq, Hq, Hkv, D, attn["window"])
    lm_tflops = lmf / (kms["lm_topk"] * 1e-3) / 1e12
    lm_gbs = lmb / (kms["lm_topk"] * 1e-3) / 1e9

    # the attention of step 4 over an fp8 (E4M3) copy of the same cache, per-tensor
    # scales from the cache's maxima; not part of the step
    attn_fp8 = {}
    if not args.no_draft_layer:
        log("block attention over an fp8 cache ...")
        Dh = attn["head_dim"]
        cf = cache.float()
        ks = float(cf[..., :Dh].abs().max()) / 448.0
        vs = float(cf[..., Dh:].abs().max()) / 448.0
        del cf
        # synthetic fp8 codes of the same cache (torch's cast: input plumbing only)
        cache8 = torch.empty(cache.shape, dtype=torch.uint8, device=dev)
        cache8[..., :Dh] = (cache[..., :Dh].float() / ks).to(torch.float8_e4m3fn).view(torch.uint8)
        cache8[..., Dh:] = (cache[..., Dh:].float() / vs).to(torch.float8_e4m3fn).view(torch.uint8)
        sc8 = torch.tensor([ks, vs], dtype=torch.float32, device=dev)
        o8 = torch.empty_like(q_out)
        for _ in range(args.warmup):
            B.block_attn(q_out, cache8, tables, seq_lens, Lq, attn["window"], out=o8, cache_fp8="e4m3", kv_scale=sc8)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ms = 0.0
        for _ in range(args.steps):
            e0.record()
            B.block_attn(q_out, cache8, tables, seq_lens, Lq, attn["window"], out=o8, cache_fp8="e4m3", kv_scale=sc8)
            e1.record()
            torch.cuda.synchronize()
            a_ms += e0.elapsed_time(e1)
        a_ms /= args.steps
        ab8 = (ab - 2 * Rq_a * Lq * Hq * D * 2) // 2 + 2 * Rq_a * Lq * Hq * D * 2  # K/V bytes halved
        attn_fp8["block_attn_fp8_e4m3"] = {
            "ms": a_ms, "GB_per_s": ab8 / (a_ms * 1e-3) / 1e9, "hbm_frac": ab8 / (a_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": ab8,
            "workload": "step 4's attention over an E4M3 copy of its cache (per-tensor scales); not part of the step"}
        del cache8

    # the draft layer's projections around steps 3-4 (qkv_proj before the
    # q/k norm, o_proj after the attention), timed on their own at the
    # attention workload's 2048 query tokens; not part of the step
    lin_kernels = {}
    if not args.no_draft_layer:
        log("draft-layer projections ...")
        dl = WL.draft_layer_inputs(attn=attn)
        x_h, w_qkv, w_o = dbf(dl["hidden_states"]), dbf(dl["W_qkv"]), dbf(dl["W_o"])
        y_qkv = torch.empty((x_h.shape[0], w_qkv.shape[0]), dtype=torch.bfloat16, device=dev)
        x_o = torch.empty((x_h.shape[0], w_o.shape[1]), dtype=torch.bfloat16, device=dev).normal_()
        y_o = torch.empty((x_h.shape[0], w_o.shape[0]), dtype=torch.bfloat16, device=dev)
        for name, (X_, W_, Y_) in (("qkv_proj", (x_h, w_qkv, y_qkv)), ("o_proj", (x_o, w_o, y_o))):
            for _ in range(args.warmup):
                B.linear(X_, W_, out=Y_)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            l_ms = 0.0
            for _ in range(args.steps):
                e0.record()
                B.linear(X_, W_, out=Y_)
                e1.record()
                torch.cuda.synchronize()
                l_ms += e0.elapsed_time(e1)
            l_ms /= args.steps
            Mx, Kx = X_.shape
            Nx = W_.shape[0]
            lf = 2 * Mx * Nx * Kx
            lb = (Mx * Kx + Nx * Kx + Mx * Nx) * 2
            lin_kernels["linear_" + name] = {
                "ms": l_ms, "TFLOP_per_s": lf / (l_ms * 1e-3) / 1e12,
                "mfma_frac": lf / (l_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "GB_per_s": lb / (l_ms * 1e-3) / 1e9, "algorithmic_bytes": lb, "flops": lf,
                "workload": f"dflash_linear {Mx} x {Nx} x {Kx} (draft layer {name}; not part of the step)"}

    # the LM-head top-k where it is bandwidth-bound: 256 rows (the mid
    # workload, and the full vocabulary / hidden size with one position per
    # request) and 16 rows (one request's block); a 512 MiB scrub write between the timed calls (outside the
    # events) keeps the weight out of the 256 MB last-level cache
    hbm_kernels = {}
    if not args.no_hbm_regime:
        log("LM-head top-k at 256 and 16 rows ...")
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        mid = WL.candidate_inputs("mid")
        cases = [("lm_topk_mid", dbf(mid["H"]), dbf(mid["W"]), mid["top_k"], mid["multiplier"], mid["softcap"],
                  "mid workload: 256 rows (32 requests x 8 steps), vocab 32768, hidden 2048, top_k 8, softcap 30"),
                 ("lm_topk_full_vocab_256_rows", H[:256].contiguous(), W, k, cand["multiplier"], cand["softcap"],
                  "256 rows (one position of 256 requests), vocab 151936, hidden 4096, top_k 16, multiplier 0.5, "
                  "softcap 30"),
                 ("lm_topk_full_vocab_16_rows", H[:16].contiguous(), W, k, cand["multiplier"], cand["softcap"],
                  "16 rows (one request's 16 steps), vocab 151936, hidden 4096, top_k 16, multiplier 0.5, "
                  "softcap 30; the streaming kernel")]
        for name, Hx, Wx, kx, sx, cx, desc in cases:
            Tx, Hdx = Hx.shape
            Vx = Wx.shape[0]
            idsx = torch.empty((Tx, kx), dtype=torch.int32, device=dev)
            lgx = torch.empty((Tx, kx), dtype=torch.float32, device=dev)
            wsx = torch.empty(max(16, B.lm_topk_workspace_size(Tx, Vx, Hdx, kx)), dtype=torch.uint8, device=dev)
            for _ in range(args.warmup):
                B.lm_topk(Hx, Wx, kx, sx, cx, idsx, lgx, wsx)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            tms = []
            for _ in range(max(args.steps // 2, 5)):
                scrub.fill_(1)
                e0.record()
                B.lm_topk(Hx, Wx, kx, sx, cx, idsx, lgx, wsx)
                e1.record()
                torch.cuda.synchronize()
                tms.append(e0.elapsed_time(e1))
            tms.sort()
            ms = tms[len(tms) // 2]
            xb, xf = lm_bytes(Tx, Vx, Hdx, kx), lm_flops(Tx, Vx, Hdx)
            floor_ms = max(xb / (HBM_PEAK_GBS * 1e9), xf / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
            hbm_kernels[name] = {
                "ms": ms, "GB_per_s": xb / (ms * 1e-3) / 1e9, "hbm_frac": xb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "TFLOP_per_s": xf / (ms * 1e-3) / 1e12,
                "mfma_frac": xf / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "binding_roofline_frac": floor_ms / ms, "algorithmic_bytes": xb, "flops": xf,
                "workload": desc + " (median of the timed calls, cache scrubbed before each; not part of the step)"}
        del scrub

    # the other configurations, as context: dflash_candidate_edges (projection
    # inside the call, as the edge metric counts it) at every configuration and
    # dflash_lm_topk at the two not timed above, each against its binding
    # roofline; median of the timed calls, a 512 MiB scrub write before each
    other_kernels = {}
    if not args.no_other_configs:
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def on_dev(x, bf=False):
            return dbf(x) if bf else torch.from_numpy(x).to(dev)

        def median_ms(fn, reps):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            tms = []
            for _ in range(reps):
                scrub.fill_(1)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                tms.append(e0.elapsed_time(e1))
            tms.sort()
            return tms[len(tms) // 2]

        for name in ("tiny", "mid", "full", "large"):
            log(f"edges (and LM head) at the {name} configuration ...")
            d = cand if name == "full" else WL.candidate_inputs(name)
            Rx, Sx, kx, Vx, Hdx, Rkx = (d["requests"], d["steps"], d["top_k"], d["vocab"], d["hidden"],
                                        d["rank"])
            Tx = Rx * Sx
            Hx = H if name == "full" else on_dev(d["H"], True)
            Px, Sx_cb, Wpx = (P, Sc, Wp) if name == "full" else (on_dev(d["P"], True), on_dev(d["S"], True),
                                                                  on_dev(d["Wp"], True))
            idsx, ux, anx = on_dev(d["ids"]), on_dev(d["U"]), on_dev(d["anchor"])
            ex = torch.empty((Rx, Sx, kx, kx), dtype=torch.float32, device=dev)
            wsx = torch.empty(max(16, B.candidate_edges_workspace_size(Tx, Rkx, Hdx)), dtype=torch.uint8,
                              device=dev)
            ms = median_ms(lambda: B.candidate_edges(Px, Sx_cb, idsx, ux, Hx, Wpx, anx, ex, wsx), 20)
            xb = edge_bytes(Rx, Sx, kx, Rkx, Hdx)
            xf = 2 * Tx * Rkx * Hdx + Tx * (kx * Rkx + 2 * kx * kx * Rkx)
            floor_ms = max(xb / (HBM_PEAK_GBS * 1e9), xf / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
            other_kernels[f"edges_{name}"] = {
                "ms": ms, "edge_scores_per_s": Tx * kx * kx / (ms * 1e-3),
                "GB_per_s": xb / (ms * 1e-3) / 1e9, "hbm_frac": xb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "binding_roofline_frac": floor_ms / ms, "algorithmic_bytes": xb, "flops": xf,
                "workload": f"dflash_candidate_edges (projection in the call) at the {name} configuration: "
                            f"{Rx} requests x {Sx} steps, top_k {kx}, vocab {Vx}, rank {Rkx}, hidden {Hdx} "
                            "(not part of the step)"}
            if name in ("tiny", "large"):
                Wx = on_dev(d["W"], True)
                idl = torch.empty((Tx, kx), dtype=torch.int32, device=dev)
                lgl = torch.empty((Tx, kx), dtype=torch.float32, device=dev)
                wsl = torch.empty(max(16, B.lm_topk_workspace_size(Tx, Vx, Hdx, kx)), dtype=torch.uint8,
                                  device=dev)
                ms = median_ms(lambda: B.lm_topk(Hx, Wx, kx, d["multiplier"], d["softcap"], idl, lgl, wsl),
                               9 if name == "large" else 20)
                xb, xf = lm_bytes(Tx, Vx, Hdx, kx), lm_flops(Tx, Vx, Hdx)
                floor_ms = max(xb / (HBM_PEAK_GBS * 1e9), xf / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
                other_kernels[f"lm_topk_{name}"] = {
                    "ms": ms, "GB_per_s": xb / (ms * 1e-3) / 1e9,
                    "hbm_frac": xb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "TFLOP_per_s": xf / (ms * 1e-3) / 1e12,
                    "mfma_frac": xf / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                    "binding_roofline_frac": floor_ms / ms, "algorithmic_bytes": xb, "flops": xf,
                    "workload": f"dflash_lm_topk at the {name} configuration: {Tx} rows, vocab {Vx}, hidden "
                                f"{Hdx}, top_k {kx}, multiplier {d['multiplier']}, softcap {d['softcap']} "
                                "(not part of the step)"}
                del Wx
            del d
        del scrub

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "edge scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/N(0,0.02) bf16, random paged cache)",
        "config": {
            "workload": "DFlash2 candidate step: LM-head top-k + candidate edges at 256 requests x 16 steps "
                        "(vocab 151936, hidden 4096, top_k 16, rank 128, multiplier 0.5, softcap 30), then "
                        "draft-layer q/k-norm+RoPE+cache write and block attention at 128 requests x 16 "
                        "queries (32 q / 8 kv heads, head_dim 128, window 2048, context 512..8192)",
            "requests": Rq, "steps": S, "top_k": k, "vocab": V, "hidden": Hd, "rank": R,
            "attn_requests": Rq_a, "attn_queries": Lq, "heads": [Hq, Hkv], "head_dim": D,
            "window": attn["window"],
            "lm_head_and_edges": ("dflash_lm_topk_proj (rank projection in the LM-head pass) + "
                                  "dflash_candidate_edges_hp" if fused else
                                  "dflash_lm_topk + dflash_candidate_edges (projection in the edge call)"),
        },
        "roofline": {
            "kernel": ("dflash_lm_topk_proj (tile GEMM + top-k + rank projection, and its merge)" if fused
                       else "dflash_lm_topk (tile GEMM + top-k, and its merge)"),
            "bound": "mfma",
            "achieved": lm_tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": lm_tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": traffic_for("lm_topk_proj_full" if fused else "lm_topk_full"),
        },
        "kernels": {
            "lm_topk": {"ms": kms["lm_topk"], "GB_per_s": lm_gbs, "hbm_frac": lm_gbs / HBM_PEAK_GBS,
                        "TFLOP_per_s": lm_tflops, "mfma_frac": lm_tflops / MFMA_BF16_PEAK_TFLOPS,
                        "algorithmic_bytes": lmb, "flops": lmf},
            "edges": {"ms": kms["edges"], "edge_scores_per_s": edges_per_step / (kms["edges"] * 1e-3),
                      "GB_per_s": eb / (kms["edges"] * 1e-3) / 1e9,
                      "hbm_frac": eb / (kms["edges"] * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": eb},
            "qk_norm_rope_cache": {"ms": kms["qk"], "GB_per_s": qb / (kms["qk"] * 1e-3) / 1e9,
                                   "hbm_frac": qb / (kms["qk"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                   "algorithmic_bytes": qb},
            "block_attn": {"ms": kms["attn"], "GB_per_s": ab / (kms["attn"] * 1e-3) / 1e9,
                           "hbm_frac": ab / (kms["attn"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "TFLOP_per_s": af / (kms["attn"] * 1e-3) / 1e12, "algorithmic_bytes": ab,
                           "flops": af},
        },
        "cpu_baseline": None,
    }
    # the step's four calls: mean (the figures above), median and min over the event-timed steps
    for key, n in (("lm_topk", "lm_topk"), ("edges", "edges"), ("qk_norm_rope_cache", "qk"), ("block_attn", "attn")):
        result["kernels"][key].update(kstat[n])
    if ctx_kernel is not None:
        result["kernels"]["context_kv"] = ctx_kernel
    result["kernels"].update(lin_kernels)
    result["kernels"].update(hbm_kernels)
    result["kernels"].update(attn_fp8)
    result["kernels"].update(other_kernels)
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(cand, attn, edges_per_step, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
