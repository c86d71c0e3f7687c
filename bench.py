#!/usr/bin/env python3
"""Throughput of the trie-packed tree-attention hot path on one MI355X.

One step is one pass of the whole path over one synthetic rollout batch:
  host   tree_pack (C++ FFD trie build, compression, pre-order layout)
  H2D    subtree ends of every trie (pinned, async)
  device tree_meta, tree_attn_fwd, tree_attn_bwd (dQ with Delta, then dK/dV)
Q, K, V and dO are resident in HBM before the timed region.  The loop is a
steady-state pipeline: step k's device work is enqueued, then the host packs
step k+1 while the GPU runs (the trie-count all-reduce of a data-parallel
run would sit at the same point); each timed iteration holds one step's
device work and one pack.  Each kernel phase is bracketed by HIP events on
the stream the library launches on.

Prints ONE JSON line.  ``value`` is real packed tokens per second through
fwd+bwd; useful TFLOP/s counts 14 * D * Hq per visible (query, key) pair
(forward 4D, backward 10D including the score recompute, the FlashAttention
convention) and is compared with MI355X's dense bf16 MFMA peak.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--config 4a]
                    [--sweep L,b] [--no-cpu-baseline]
    python bench.py --logprobs [--vocab 151936] [--config 4a]   (the
                    tree log-probability gather, its own JSON line, with
                    --logprob-chunk 1024 times the chunked form beside it)
    python bench.py --partition K [--config 2]   (the host-side DFS-order
                    split over K workers, its own JSON line)
    python bench.py --rope [--config 4a]   (rotary embedding of Q and K by
                    tree position ids, its own JSON line)
    python bench.py --rope-fused [--config 4a]   (fwd+bwd with the rotation
                    fused into the kernels vs separate passes)
    python bench.py --dfs [--config 4a] [--chunk 2048]   (depth-first
                    execution per trie vs the packed path)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PHASES = ("meta", "fwd", "dq", "dkdv")  # in launch order; "dq" forms Delta too
PHASE_KERNEL = {"meta": "meta_lists", "fwd": "fwd_bf16_kernel", "dkdv": "dkdv_bf16_kernel", "dq": "dq_bf16_kernel"}
PHASE_SOURCE = {"meta": "meta.hip", "fwd": "fwd_bf16.hip", "dkdv": "bwd_bf16.hip", "dq": "bwd_bf16.hip"}
# algorithmic FLOPs per visible pair and query head, in units of D
PHASE_FLOPS_PER_PAIR_D = {"fwd": 4, "dkdv": 8, "dq": 6}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="4a", help="workload: 2, 3, 4a, 4b")
    ap.add_argument("--sweep", default=None, help="L,b of a sweep point (overrides --config)")
    ap.add_argument("--pack", default="ffd", choices=["ffd", "prefix"],
                    help="trie assignment: the pages' first-fit decreasing, or prefix (lexicographic next-fit) order")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=1, help="query heads in the oracle sample")
    ap.add_argument("--logprobs", action="store_true",
                    help="time the tree log-probability / entropy gather (logits_stats + gather) instead")
    ap.add_argument("--vocab", type=int, default=151936, help="vocabulary size of the --logprobs logits")
    ap.add_argument("--partition", type=int, default=0,
                    help="time the DFS-order load-balanced split of the batch over this many workers instead")
    ap.add_argument("--rope", action="store_true",
                    help="time the rotary embedding of Q and K by tree position ids instead")
    ap.add_argument("--rope-fused", action="store_true",
                    help="time fwd+bwd with the rotary embedding fused into the kernels against separate passes")
    ap.add_argument("--dfs", action="store_true",
                    help="time the depth-first (DTA) execution of every trie against the packed path")
    ap.add_argument("--chunk", type=int, default=2048, help="query chunk of the depth-first execution")
    ap.add_argument("--logprob-chunk", type=int, default=0,
                    help="with --logprobs, also time the chunked form with this many rows per chunk "
                         "(the guide's chunk_size is 1024)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB elementwise copy kernel 3x (HBM counter calibration)")
    return ap.parse_args(argv)


def copy_calibration():
    """A plain elementwise copy of 1 GiB (read 1 GiB, write 1 GiB), three
    launches: the reference reading of the FETCH_SIZE / WRITE_SIZE counters
    for a kernel of known traffic."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n}), flush=True)
    return 0


# device headers every kernel source compiles in
KERNEL_HEADERS = ("device.h", "mfma.h", "tile.h")


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed (string
    literals in these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha(name: str) -> str:
    """Hash of the code of a kernel source and of the device headers it
    compiles in (comments and layout ignored): a traffic summary counts only
    while none of them has changed."""
    h = hashlib.sha256()
    for n in (name, *KERNEL_HEADERS):
        with open(os.path.join(ROOT, "prefix_tree_attention_amd", "csrc", n)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, phase: str):
    """HBM bytes per launch of a kernel from a committed rocprofv3 PMC
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{PHASE_KERNEL[phase]}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_sha(PHASE_SOURCE[phase]):
        return None
    return float(t["bytes_per_launch"])


def cpu_baseline(w, p_oracle_input, n_heads: int):
    """The oracle (dense ancestor mask, naive fp32 attention and closed-form
    gradients) on trie 0 of the workload, restricted to `n_heads` query heads
    of key/value head 0; scaled to all heads."""
    import numpy as np
    import torch
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    ids, mask, M = p_oracle_input
    t0 = time.perf_counter()
    po = oracle.pack(ids, mask, M)[0]
    m = oracle.dense_ancestor_mask(po)
    t_pack = time.perf_counter() - t0
    q, k, v, do = workloads.attention_inputs(po.L, w.hq, w.hkv, w.d, "bf16", w.qkv_std, 4242)
    Q = q[:, :n_heads].float().numpy()
    K = k[:, :1].float().numpy()
    V = v[:, :1].float().numpy()
    G = do[:, :n_heads].float().numpy()
    scale = 1.0 / math.sqrt(w.d)
    t1 = time.perf_counter()
    o, lse = oracle.attention_forward(Q, K, V, m, scale, dtype=np.float32)
    oracle.attention_backward(Q, K, V, o, lse, G, m, scale, dtype=np.float32)
    t_attn = time.perf_counter() - t1
    per_trie = t_pack + t_attn * (w.hq / n_heads)
    del torch
    return {
        "value": po.n_tokens / per_trie,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"trie 0 ({po.n_tokens} tokens, L={po.L}): oracle pack + dense mask "
                   f"({t_pack:.1f} s) and fp32 fwd+bwd of {n_heads} of {w.hq} query heads "
                   f"({t_attn:.1f} s), attention time scaled x{w.hq // n_heads}"),
    }


def main(argv=None):
    a = parse(argv)
    if a.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": a.gpus}), flush=True)
        log("bench.py: multi-GPU runs are not implemented: the path runs one GPU's share of a batch, and the batch "
            "would be split over data-parallel ranks by tree_partition.")
        return 2
    if a.copy_calibration:
        return copy_calibration()
    if a.logprobs:
        return bench_logprobs(a)
    if a.partition:
        return bench_partition(a)
    if a.rope:
        return bench_rope(a)
    if a.rope_fused:
        return bench_rope_fused(a)
    if a.dfs:
        return bench_dfs(a)
    import numpy as np
    import torch
    import workloads
    import prefix_tree_attention_amd as pta

    if a.sweep:
        L_, b = (int(x) for x in a.sweep.split(","))
        w = workloads.sweep_workload(L_, b)
    else:
        w = workloads.make_workload(a.config)
    if w.dtype != "bf16" or not w.backward:
        raise SystemExit("bench.py times the bf16 forward+backward path; config 1 is a parity case")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---------------- untimed setup ----------------
    # All tries of the batch are laid end to end (tree_pack_concat) and run
    # as one launch: no attention crosses tries, so the concatenation is a
    # packed layout of its own, and one launch avoids per-trie launch and
    # tail costs on batches of many small tries.
    tries, stats = pta.pack(w.ids, w.mask, w.max_tokens_per_mb, order=a.pack)
    se_cat, lengths, _ = pta.pack_concat(w.ids, w.mask, w.max_tokens_per_mb, order=a.pack)
    log(f"workload {w.name}: {len(tries)} tries, L={lengths}, one launch of L={len(se_cat)}, tree tokens "
        f"{stats['tree_tokens']}, pairs {stats['n_pairs']}, unpacked pairs {stats['unpacked_pairs']}")
    if len(se_cat) > (1 << 20):
        raise SystemExit(f"batch of {len(se_cat)} packed tokens exceeds one launch (2^20)")
    bufs = []
    pairs_per_trie = []
    for i, tr in enumerate(tries):
        se_i64 = tr.subtree_end.astype(np.int64)
        real = se_i64 >= 0
        pairs_per_trie.append(int((se_i64[real] - np.arange(tr.L)[real] + 1).sum()))
    q, k, v, do = workloads.batch_attention_inputs(lengths, w.hq, w.hkv, w.d, "bf16", w.qkv_std)
    L = len(se_cat)
    nb = L // 128
    bufs.append({
        "L": L,
        "q": q.to(dev), "k": k.to(dev), "v": v.to(dev), "do": do.to(dev),
        "o": torch.empty((L, w.hq, w.d), dtype=torch.bfloat16, device=dev),
        "lse": torch.empty((w.hq, L), dtype=torch.float32, device=dev),
        "dq": torch.empty((L, w.hq, w.d), dtype=torch.bfloat16, device=dev),
        "dk": torch.empty((L, w.hkv, w.d), dtype=torch.bfloat16, device=dev),
        "dv": torch.empty((L, w.hkv, w.d), dtype=torch.bfloat16, device=dev),
        "se": torch.empty(L, dtype=torch.int32, device=dev),
        "pos": torch.empty(L, dtype=torch.int32, device=dev),
        "tc": torch.empty((nb, nb), dtype=torch.uint8, device=dev),
        "mws": torch.empty(pta.meta_workspace_bytes(L), dtype=torch.uint8, device=dev),
        "bws": torch.empty(pta.bwd_workspace_bytes(L, w.hq, w.d), dtype=torch.uint8, device=dev),
        "pinned": [torch.empty(L, dtype=torch.int32).pin_memory() for _ in range(2)],
        "copied": [None, None],
    })
    assert sum(pairs_per_trie) == stats["n_pairs"]
    torch.cuda.synchronize()
    lib = pta.lib()
    from prefix_tree_attention_amd.api import _ptr  # argument marshalling helper
    import ctypes
    sptr = ctypes.c_void_p(stream.cuda_stream)
    scale = 1.0 / math.sqrt(w.d)

    def launch(k_step, cur, events):
        """Enqueue one step's device work for the packed layout `cur`."""
        slot = k_step % 2
        for i, se_host in enumerate([cur]):
            b = bufs[i]
            assert len(se_host) == b["L"]
            if b["copied"][slot] is not None:
                b["copied"][slot].synchronize()  # the copy that last read this pinned buffer is done
            b["pinned"][slot].numpy()[:] = se_host
            b["se"].copy_(b["pinned"][slot], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(stream)
            b["copied"][slot] = ev
            L = b["L"]
            E = [torch.cuda.Event(enable_timing=True) for _ in range(len(PHASES) + 1)] if events is not None else None
            if E:
                E[0].record(stream)
            pta._lib.check(lib.tree_meta(_ptr(b["se"]), L, _ptr(b["pos"]), _ptr(b["tc"]), _ptr(b["mws"]),
                                         b["mws"].numel(), sptr))
            if E:
                E[1].record(stream)
            pta._lib.check(lib.tree_attn_fwd(_ptr(b["q"]), _ptr(b["k"]), _ptr(b["v"]), _ptr(b["o"]), _ptr(b["lse"]),
                                             _ptr(b["se"]), _ptr(b["mws"]), L, w.hq, w.hkv, w.d, scale, 0, sptr))
            if E:
                E[2].record(stream)
            for j, ph in enumerate((pta.BWD_DQ_DELTA, pta.BWD_DKDV)):
                pta._lib.check(lib.tree_attn_bwd_phase(
                    ph, _ptr(b["q"]), _ptr(b["k"]), _ptr(b["v"]), _ptr(b["o"]), _ptr(b["lse"]), _ptr(b["do"]),
                    _ptr(b["dq"]), _ptr(b["dk"]), _ptr(b["dv"]), _ptr(b["se"]), _ptr(b["mws"]), _ptr(b["bws"]),
                    b["bws"].numel(), L, w.hq, w.hkv, w.d, scale, 0, sptr))
                if E:
                    E[3 + j].record(stream)
            if events is not None:
                events.append((i, E))

    def pack_host():
        cur, _, _ = pta.pack_concat(w.ids, w.mask, w.max_tokens_per_mb, order=a.pack)
        return cur

    # Steady-state pipeline: the device work of step k is enqueued, then the
    # host packs step k+1 while the GPU runs.  Each timed iteration holds one
    # step's device work and one pack.
    pending = pack_host()
    for k_step in range(a.warmup):
        launch(k_step, pending, None)
        pending = pack_host()
    torch.cuda.synchronize()
    log(f"warmup done ({a.warmup} steps)")

    events = []
    t_pack = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k_step in range(a.steps):
        launch(a.warmup + k_step, pending, events)
        tp = time.perf_counter()
        pending = pack_host()
        t_pack += time.perf_counter() - tp
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_per_step = (t1 - t0) / a.steps

    # per-phase kernel time (ms per launch) from the events
    tot = {p: 0.0 for p in PHASES}
    for i, E in events:
        for j, p in enumerate(PHASES):
            tot[p] += E[j].elapsed_time(E[j + 1])
    n_launch = len(events)
    avg = {p: tot[p] / n_launch for p in PHASES}
    gpu_ms_per_step = sum(tot.values()) / a.steps
    log("per-launch ms: " + ", ".join(f"{p} {avg[p]:.3f}" for p in PHASES)
        + f" | gpu ms/step {gpu_ms_per_step:.3f} | wall ms/step {sec_per_step * 1e3:.3f}")

    n_pairs = stats["n_pairs"]
    tokens = stats["tree_tokens"]
    # 128x128 tile accounting: the packer's host counts (tree_pack_stats),
    # cross-checked against the classes tree_meta wrote on the device for the
    # last step; the skip rate is against dense causal attention of each trie
    tc = bufs[0]["tc"]
    dev_full, dev_partial = int((tc == 2).sum()), int((tc == 1).sum())
    if (dev_full, dev_partial) != (stats["tiles_full"], stats["tiles_partial"]):
        raise SystemExit(f"tile classes on the device ({dev_full} full, {dev_partial} partial) differ from the "
                         f"packer's counts ({stats['tiles_full']}, {stats['tiles_partial']})")
    causal = stats["tiles_causal"]
    tiles = {"full": stats["tiles_full"], "partial": stats["tiles_partial"],
             "empty": causal - stats["tiles_full"] - stats["tiles_partial"], "dense_causal": causal,
             "skip_rate_vs_causal": round(1.0 - (stats["tiles_full"] + stats["tiles_partial"]) / causal, 4),
             "visible_fraction_of_nonempty_area": round(n_pairs / (128.0 * 128.0 * (stats["tiles_full"]
                                                                                 + stats["tiles_partial"])), 4)}
    log(f"tiles: {tiles}")
    useful_flop = 14.0 * w.d * w.hq * n_pairs
    useful_tflops = useful_flop / sec_per_step / 1e12
    dom = max(PHASES, key=lambda p: avg[p])
    if dom in PHASE_FLOPS_PER_PAIR_D:
        alg = PHASE_FLOPS_PER_PAIR_D[dom] * w.d * w.hq * n_pairs / n_launch * a.steps  # per launch
        achieved = alg / (avg[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:  # HBM-bound phase
        per = 2 * sum(b["L"] for b in bufs) * w.hq * w.d * 2 / len(bufs)
        achieved = per / (avg[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = PHASE_KERNEL[dom]
    roof["traffic"] = load_traffic(w.name, dom)

    result = {
        "metric": "tree-attn fwd+bwd tokens/s + useful TFLOP/s (% of bf16 MFMA peak), 1 GPU",
        "value": round(tokens / sec_per_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(sec_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "useful_tflops": round(useful_tflops, 2),
        "pct_of_bf16_peak": round(100.0 * useful_tflops / PEAK_BF16_TFLOPS, 2),
        "effective_tokens_per_s": round(stats["original_tokens"] / sec_per_step, 1),
        "flop_reduction_vs_unpacked": round(stats["unpacked_pairs"] / n_pairs, 3),
        "tree_token_ratio": round(stats["tree_token_ratio"], 4),
        "gpu_ms_per_step": round(gpu_ms_per_step, 3),
        "host_pack_ms_per_step": round(t_pack / a.steps * 1e3, 3),
        "kernel_ms_per_launch": {p: round(avg[p], 4) for p in PHASES},
        "config": {"workload": w.name, "tries": len(tries), "L": lengths, "launch_L": bufs[0]["L"], "hq": w.hq,
                   "hkv": w.hkv, "head_dim": w.d, "max_tokens_per_mb": w.max_tokens_per_mb,
                   "tree_tokens": tokens, "pairs": n_pairs, "pack": a.pack, "parallelism": "single-gpu"},
        "roofline": roof,
        "tiles": tiles,
    }
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        sub = _first_trie_rows(w, tries[0])
        result["cpu_baseline"] = cpu_baseline(w, sub, a.cpu_heads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def bench_logprobs(a):
    """Tree log-probabilities and entropies of one batch's packed logits
    (bf16 [L, V], resident in HBM): tree_logits_stats over every packed row,
    then tree_gather_logprobs into [B, S].  One JSON line; its roofline is the
    HBM-bound row-statistics pass, whose algorithmic traffic is the logits
    read once (2 L V bytes) plus 8 L bytes of output."""
    import numpy as np
    import torch
    import workloads
    import prefix_tree_attention_amd as pta

    w = workloads.sweep_workload(*(int(x) for x in a.sweep.split(","))) if a.sweep else workloads.make_workload(a.config)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    se, tok, rp, lengths, stats = pta.pack_batch(w.ids, w.mask, w.max_tokens_per_mb)
    L, V = len(se), int(a.vocab)
    n_pred = int((w.mask.astype(bool).sum(1) - 1).sum())
    log(f"logprobs {w.name}: L={L}, V={V}, {n_pred} predictions, logits {2 * L * V / 1e9:.1f} GB bf16")
    g = torch.Generator(device=dev).manual_seed(2024)
    x = torch.empty((L, V), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, L, 2048):
        x[r0:r0 + 2048] = (torch.randn((min(2048, L - r0), V), generator=g, device=dev) * 2.0).to(torch.bfloat16)
    tok_d = torch.from_numpy(tok).to(dev)
    rp_d = torch.from_numpy(rp).to(dev)
    torch.cuda.synchronize()
    for _ in range(a.warmup):
        pta.tree_logprobs(x, tok_d, rp_d)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    t0 = time.perf_counter()
    for i in range(a.steps):
        ev[i][0].record(stream)
        lse, ent = pta.logits_stats(x)
        ev[i][1].record(stream)
        pta.gather_logprobs(x, lse, ent, tok_d, rp_d)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / a.steps
    t_stats = sum(e[0].elapsed_time(e[1]) for e in ev) / a.steps
    t_gather = sum(e[1].elapsed_time(e[2]) for e in ev) / a.steps
    # the chunked form: stats and the gather window per chunk of rows, as
    # after an LM head run chunk by chunk (here the chunks are row slices of
    # the resident logits, so only the per-chunk launches are added)
    ch = int(a.logprob_chunk)
    chunked = None
    if ch > 0:
        pta.tree_logprobs_chunked(lambda r0, r1: x[r0:r1], L, tok_d, rp_d, ch)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(a.steps):
            pta.tree_logprobs_chunked(lambda r0, r1: x[r0:r1], L, tok_d, rp_d, ch)
        e1.record(stream)
        torch.cuda.synchronize()
        t_chunked = e0.elapsed_time(e1) / a.steps
        chunked = {"rows_per_chunk": ch, "chunks": -(-L // ch), "gpu_ms_per_step": round(t_chunked, 4),
                   "logits_bytes_per_chunk": 2 * ch * V}
        log(f"stats {t_stats:.3f} ms, gather {t_gather:.3f} ms; chunked ({ch} rows, {-(-L // ch)} chunks) "
            f"{t_chunked:.3f} ms per step")
    alg = 2.0 * L * V + 8.0 * L
    achieved = alg / (t_stats * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "kernel": "logits_stats_kernel",
            "traffic": _load_traffic_file(f"traffic_logits_stats_kernel_{w.name}-V{V}.json", "logprob.hip")}
    result = {
        "metric": "tree log-probability + entropy gather: predictions/s and HBM GB/s of the row-statistics pass",
        "value": round(n_pred / sec, 1), "unit": "predictions/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(sec * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "kernel_ms_per_launch": {"logits_stats": round(t_stats, 4), "gather": round(t_gather, 4)},
        "chunked": chunked,
        "config": {"workload": w.name, "L": L, "vocab": V, "batch": list(w.ids.shape), "predictions": n_pred},
        "roofline": roof,
    }
    if not a.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"]
                        or [1])
        except Exception:  # pragma: no cover
            cores = 1
        rng = np.random.default_rng(1)
        picks = [(int(r), int(rng.integers(int(w.mask[r].sum()) - 1)))
                 for r in rng.integers(w.ids.shape[0], size=4096)]
        idx = torch.tensor([int(rp[r, j]) for r, j in picks], device=dev)
        rows = x[idx].float().cpu().numpy()  # one copy of the sampled rows
        t1 = time.perf_counter()
        for (r, j), row in zip(picks, rows):
            oracle.prediction_logprob_entropy(row, int(tok[rp[r, j + 1]]))
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": len(picks) / dt, "unit": "predictions/s", "cores": cores, "kind": "oracle",
                                  "sample": f"{len(picks)} predictions of the batch at V={V}, one float64 "
                                            f"log-softmax and entropy each ({dt:.2f} s); the oracle's node cache "
                                            f"would reuse shared rows, so this rate is per packed row"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def bench_partition(a):
    """Host-side DFS-order load-balanced split of one batch over K workers
    (tree_partition): time per call, the largest per-worker tree (the
    objective), the tokens the split duplicates relative to one tree, and,
    for contrast, a structure-blind split: the rows in a seeded random order
    cut into K runs of balanced token count."""
    import numpy as np
    import workloads
    import prefix_tree_attention_amd as pta

    w = workloads.sweep_workload(*(int(x) for x in a.sweep.split(","))) if a.sweep else workloads.make_workload(a.config)
    K = int(a.partition)
    _, one, _ = pta.partition(w.ids, w.mask, 1)
    for _ in range(max(1, a.warmup)):
        pta.partition(w.ids, w.mask, K)
    t0 = time.perf_counter()
    for _ in range(a.steps):
        g, tau, costs = pta.partition(w.ids, w.mask, K)
    sec = (time.perf_counter() - t0) / a.steps
    lens = w.mask.astype(bool).sum(1)
    # structure-blind contrast: rows in a seeded random order (the batch
    # generators emit prompt groups contiguously, which is not blind), cut
    # at balanced token counts
    perm = np.random.default_rng(12345).permutation(len(lens))
    cum = np.cumsum(lens[perm])
    blind = np.empty(len(lens), dtype=np.int64)
    blind[perm] = np.minimum((cum - 1) * K // cum[-1], K - 1)
    blind_costs = []
    for j in range(K):
        rows = np.nonzero(blind == j)[0]
        if len(rows) == 0:
            blind_costs.append(0)
            continue
        _, c, _ = pta.partition(w.ids[rows], w.mask[rows], 1)
        blind_costs.append(c)
    result = {
        "metric": "DFS-order load-balanced partition: host ms per batch, largest per-worker tree tokens",
        "value": round(sec * 1e3, 4), "unit": "ms", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "higher_is_better": False, "data": "synthetic",
        "config": {"workload": w.name, "rows": int(w.ids.shape[0]), "workers": K, "tokens": int(lens.sum())},
        "single_tree_tokens": one, "max_worker_tree_tokens": tau, "worker_tree_tokens": [int(c) for c in costs],
        "duplicated_tokens": int(costs.sum() - one), "duplication_bound": int((K - 1) * lens.max()),
        "balance": round(tau / (one / K), 4),
        "structure_blind": {"max_worker_tree_tokens": int(max(blind_costs)),
                            "duplicated_tokens": int(sum(blind_costs) - one),
                            "balance": round(max(blind_costs) / (one / K), 4)},
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_rope(a):
    """Rotary embedding of the step's Q [L, Hq, D] and K [L, Hkv, D] (bf16,
    resident) by the tree position ids of tree_meta: one tree_rope per
    tensor, timed with HIP events; HBM-bound, algorithmic traffic = each
    tensor read and written once."""
    import numpy as np
    import torch
    import workloads
    import prefix_tree_attention_amd as pta

    w = workloads.sweep_workload(*(int(x) for x in a.sweep.split(","))) if a.sweep else workloads.make_workload(a.config)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    se, _, _, _, _ = pta.pack_batch(w.ids, w.mask, w.max_tokens_per_mb)
    L = len(se)
    meta = pta.tree_meta(se)
    q, k, _, _ = workloads.attention_inputs(L, w.hq, w.hkv, w.d, "bf16", w.qkv_std, 77)
    q, k = q.to(dev), k.to(dev)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    for _ in range(a.warmup):
        pta.rope(q, meta.pos, 1e6, out=qo)
        pta.rope(k, meta.pos, 1e6, out=ko)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        pta.rope(q, meta.pos, 1e6, out=qo)
        pta.rope(k, meta.pos, 1e6, out=ko)
        e1.record(stream)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / a.steps
    ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / a.steps
    alg = 2.0 * 2 * L * (w.hq + w.hkv) * w.d
    achieved = alg / (ms * 1e-3) / 1e9
    result = {
        "metric": "rotary embedding of Q and K by tree position ids: tokens/s and HBM GB/s",
        "value": round(L / sec, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic", "kernel_ms_per_step": round(ms, 4),
        "config": {"workload": w.name, "L": L, "hq": w.hq, "hkv": w.hkv, "head_dim": w.d, "base": 1e6},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "kernel": "rope_kernel", "traffic": None},
    }
    if not a.no_cpu_baseline:
        import oracle
        n = min(L, 4096)
        pos = meta.pos[:n].cpu().numpy()
        qs, ks = q[:n].float().cpu().numpy(), k[:n].float().cpu().numpy()
        t1 = time.perf_counter()
        oracle.rope(qs, pos, 1e6)
        oracle.rope(ks, pos, 1e6)
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the first {n} tokens of Q and K, float64 numpy ({dt:.2f} s)"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def bench_rope_fused(a):
    """Attention with the rotary embedding by tree position ids, forward and
    backward, two ways on the same resident inputs: the rotation fused into
    the kernels (tree_attn_fwd_rope / tree_attn_bwd_rope: Q rotated at the
    forward's register load, K by one table pass, dQ / dK rotated back in the
    backward epilogues), and as separate passes (tree_rope of Q and K, the
    plain forward and backward, tree_rope inverse of dQ and dK).  value =
    packed tokens/s of the fused step."""
    import torch
    import workloads
    import prefix_tree_attention_amd as pta

    w = workloads.sweep_workload(*(int(x) for x in a.sweep.split(","))) if a.sweep else workloads.make_workload(a.config)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    se, lengths, stats = pta.pack_concat(w.ids, w.mask, w.max_tokens_per_mb)
    L = len(se)
    meta = pta.tree_meta(se)
    q, k, v, do = workloads.batch_attention_inputs(lengths, w.hq, w.hkv, w.d, "bf16", w.qkv_std)
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    tab = pta.rope_table(L, w.d, 1e6)
    o, lse = torch.empty_like(q), torch.empty((w.hq, L), dtype=torch.float32, device=dev)
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(pta.bwd_workspace_bytes(L, w.hq, w.d), dtype=torch.uint8, device=dev)

    def fused():
        pta.attn_fwd_rope(q, k, v, meta, tab, o=o, lse=lse)
        pta.attn_bwd_rope(qr, kr, v, o, lse, do, meta, tab, dq=dq, dk=dk, dv=dv, workspace=ws)

    def separate():
        pta.rope(q, meta.pos, 1e6, out=qr)
        pta.rope(k, meta.pos, 1e6, out=kr)
        pta.attn_fwd(qr, kr, v, meta, o=o, lse=lse)
        pta.attn_bwd(qr, kr, v, o, lse, do, meta, workspace=ws, dq=dq, dk=dk, dv=dv)
        pta.rope(dq, meta.pos, 1e6, inverse=True, out=dq)
        pta.rope(dk, meta.pos, 1e6, inverse=True, out=dk)

    def timed(fn):
        for _ in range(a.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(a.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps

    # the fused forward writes q_rot / k_rot into qr / kr for its backward
    _o, _l, qr0, kr0 = pta.attn_fwd_rope(q, k, v, meta, tab, o=o, lse=lse)
    qr.copy_(qr0)
    kr.copy_(kr0)
    t_sep = timed(separate)
    t_fused = timed(fused)
    useful = 14.0 * w.d * w.hq * stats["n_pairs"]
    result = {
        "metric": "tree-attn fwd+bwd with rotary embedding by tree position ids, fused vs separate passes",
        "value": round(stats["tree_tokens"] / (t_fused * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(t_fused, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "fused_ms_per_step": round(t_fused, 4), "separate_ms_per_step": round(t_sep, 4),
        "useful_tflops": round(useful / (t_fused * 1e-3) / 1e12, 2),
        "pct_of_bf16_peak": round(100.0 * useful / (t_fused * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": w.name, "launch_L": L, "hq": w.hq, "hkv": w.hkv, "head_dim": w.d, "base": 1e6},
        "cpu_baseline": None,
    }
    log(f"fused {t_fused:.3f} ms, separate passes {t_sep:.3f} ms per step")
    print(json.dumps(result), flush=True)
    return 0


def bench_dfs(a):
    """Depth-first (DTA) execution of every trie of the batch (tree_attn_dfs,
    forward and backward, chunk a.chunk) against the packed-trie path on the
    same resident inputs, per trie.  value = packed tokens/s of the
    depth-first step; also its device memory (the frame workspace, bounded
    by the longest path) against the packed path's per-trie tensors."""
    import torch
    import workloads
    import prefix_tree_attention_amd as pta

    w = workloads.sweep_workload(*(int(x) for x in a.sweep.split(","))) if a.sweep else workloads.make_workload(a.config)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    tries, stats = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    items = []
    for t, tr in enumerate(tries):
        q, k, v, do = (x.to(dev) for x in workloads.attention_inputs(tr.L, w.hq, w.hkv, w.d, "bf16", w.qkv_std,
                                                                      1_000_000 + t))
        meta = pta.tree_meta(tr.subtree_end)
        plan = pta.dfs_plan(tr, a.chunk)
        outs = dict(o=torch.empty_like(q), lse=torch.empty((w.hq, tr.L), dtype=torch.float32, device=dev),
                    dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v))
        ws = torch.empty(pta.dfs_workspace_bytes(plan, w.hq, w.hkv, w.d), dtype=torch.uint8, device=dev)
        items.append((tr, q, k, v, do, meta, plan, outs, ws))

    def dfs():
        for tr, q, k, v, do, meta, plan, outs, ws in items:
            pta.attn_dfs(tr, q, k, v, do, meta, chunk=a.chunk, workspace=ws, **outs)

    def packed():
        for tr, q, k, v, do, meta, plan, outs, ws in items:
            o, lse = pta.attn_fwd(q, k, v, meta, o=outs["o"], lse=outs["lse"])
            pta.attn_bwd(q, k, v, o, lse, do, meta, dq=outs["dq"], dk=outs["dk"], dv=outs["dv"])

    def timed(fn):
        for _ in range(a.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(a.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps, (time.perf_counter() - t0) / a.steps * 1e3

    t_dfs, wall_dfs = timed(dfs)
    t_packed, _ = timed(packed)
    # the whole walk of every trie holds only kernel launches: captured once
    # into a HIP graph, a replay removes the per-launch host cost
    s2 = torch.cuda.Stream()
    s2.wait_stream(stream)
    with torch.cuda.stream(s2):
        dfs()
    stream.wait_stream(s2)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dfs()
    t_graph, wall_graph = timed(g.replay)
    useful = 14.0 * w.d * w.hq * stats["n_pairs"]
    per_trie_tensors = max(tr.L for tr in tries) * (4 * w.hq + 4 * w.hkv) * w.d * 2
    result = {
        "metric": "depth-first (DTA) tree-attn fwd+bwd tokens/s and useful TFLOP/s, 1 GPU",
        "value": round(stats["tree_tokens"] / (wall_dfs * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(wall_dfs, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "gpu_ms_per_step": round(t_dfs, 4), "packed_path_ms_per_step": round(t_packed, 4),
        "graph_replay_ms_per_step": round(wall_graph, 4),
        "useful_tflops": round(useful / (wall_dfs * 1e-3) / 1e12, 2),
        "pct_of_bf16_peak": round(100.0 * useful / (wall_dfs * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "frame_workspace_bytes": max(int(x[8].numel()) for x in items),
        "packed_trie_tensor_bytes": per_trie_tensors,
        "plans": [x[6] for x in items][:8],
        "config": {"workload": w.name, "tries": len(tries), "L": [tr.L for tr in tries], "chunk": a.chunk,
                   "hq": w.hq, "hkv": w.hkv, "head_dim": w.d},
        "cpu_baseline": None,
    }
    log(f"dfs {t_dfs:.3f} ms (wall {wall_dfs:.3f}, graph replay {wall_graph:.3f}), packed {t_packed:.3f} ms per step")
    print(json.dumps(result), flush=True)
    return 0


def _load_traffic_file(name: str, source: str):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    return float(t["bytes_per_launch"]) if t.get("source_sha") == source_sha(source) else None


def _first_trie_rows(w, tr0):
    """The batch rows packed into trie 0, as an input the oracle packs into
    exactly that trie."""
    rows = sorted(int(r) for r in tr0.seq_ids)
    return w.ids[rows], w.mask[rows], w.max_tokens_per_mb


if __name__ == "__main__":
    sys.exit(main())
