#!/usr/bin/env python3
"""Benchmark of the QSA hot path on one MI355X.

Default workload: the 1M-token context configuration. One step =
  prefill chunk: compress the chunk's 4096 new blocks, index + causal top-k for
                 16384 queries at positions 1,032,192 .. 1,048,575, sparse
                 attention over their kept tokens (Q [16384,32,128],
                 K/V [1M,4,128], indexer 8 x 64, r = 4, budget 2048 tokens);
  decode step:   index + top-k and sparse attention for 4 sequences whose
                 query sits at position 1,048,575 (caches [4,1M,4,128], block
                 keys precomputed).
All inputs are seeded synthetic tensors resident in HBM before timing starts.
Prints one JSON line: the metric and its value, per-phase times, the roofline
of the dominant kernel (achieved over peak, and the HBM traffic its counters
measured), the oracle's rate on a bounded sample of the same workload, and
the sampled parity of the timed outputs.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c5|c3|c4|c6]
  python bench.py --gdn | --kl       # gated delta rule; distillation loss
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA prefill tokens/s @256K–1M ctx; decode µs/step; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
PAGES_SPEEDUP = {"prefill": 7.6, "decode": 4.9, "context": "1M tokens, QSA vs GQA attention, hardware not stated"}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# --------------------------------------------------------------- work model --
def prefill_work(W, q_pos0, n_q):
    """Algorithmic bytes / flops of one prefill chunk (what the method must touch)."""
    t = np.arange(q_pos0, q_pos0 + n_q, dtype=np.int64)
    b = t // W.r
    m = np.minimum(W.k - 1, b)
    ntok = m * W.r + (t - b * W.r) + 1
    new_blocks = (q_pos0 + n_q) // W.r - q_pos0 // W.r
    row_kv = W.Hkv * W.D * 2
    w = {}
    w["compress_bytes"] = new_blocks * (W.r * W.di * 2 + W.di * 2)
    w["index_pairs"] = int(b.sum())
    w["index_flops"] = int(b.sum()) * W.Hi * W.di * 2
    w["index_bytes"] = n_q * W.Hi * W.di * 2 + int(b.max()) * W.di * 2 + n_q * (W.k + 1) * 4
    w["attn_tokens"] = int(ntok.sum())
    w["attn_flops"] = int(ntok.sum()) * W.Hq * W.D * 4
    w["attn_bytes"] = int(ntok.sum()) * row_kv * 2 + 2 * n_q * W.Hq * W.D * 2 + n_q * (W.k + 1) * 4
    w["dense_flops"] = int((t + 1).sum()) * W.Hq * W.D * 4
    return w


def decode_work(W):
    t = W.L - 1
    b = t // W.r
    m = min(W.k - 1, b)
    ntok = m * W.r + (t - b * W.r) + 1
    B = W.batch
    w = {}
    w["index_flops"] = B * b * W.Hi * W.di * 2
    w["index_bytes"] = B * (b * W.di * 2 + W.Hi * W.di * 2 + (W.k + 1) * 4)
    w["attn_bytes"] = B * (ntok * W.Hkv * W.D * 2 * 2 + 2 * W.Hq * W.D * 2 + (W.k + 1) * 4)
    w["dense_bytes"] = B * ((t + 1) * W.Hkv * W.D * 2 * 2 + 2 * W.Hq * W.D * 2)
    return w


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_sparse_long_09_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, sha):
    """Counter-derived HBM bytes per launch from the committed profile summary,
    if it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(kernel_key)
    if not e or e.get("source_sha") != sha:
        return None
    return e.get("bytes_per_launch")


# ------------------------------------------------------------------ timing --
class PhaseTimer:
    def __init__(self, torch, names):
        self.torch = torch
        self.names = names
        self.acc = {n: [] for n in names}

    def run(self, fns):
        T = self.torch
        evs = [T.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        evs[0].record()
        for i, f in enumerate(fns):
            f()
            evs[i + 1].record()
        return evs

    def collect(self, evs):
        for i, n in enumerate(self.names):
            self.acc[n].append(evs[i].elapsed_time(evs[i + 1]))

    def mean_ms(self):
        return {n: float(np.mean(v)) if v else None for n, v in self.acc.items()}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c5", choices=["c5", "c3", "c4", "c6"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="default workload only: skip the 256K prefill and 128K decode sections")
    ap.add_argument("--cpu-sample", type=int, default=256, help="queries in the oracle's timed sample")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration runs)")
    ap.add_argument("--kl", action="store_true",
                    help="time the indexer's dense-distillation loss forward on the config's prefill instead")
    ap.add_argument("--gdn", action="store_true",
                    help="time the recurrent layers' gated delta rule instead: 32K-token prefill of one layer "
                         "and one decode step of 64 sequences")
    ap.add_argument("--block-size", type=int, default=0,
                    help="micro-block size r of a variant run (default: the workload's, 4)")
    ap.add_argument("--budget", type=int, default=0,
                    help="token budget k*r of a variant run (default: the workload's, 2048)")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "KEY"),
                    help="write profiles/traffic.json entries KEY (c5, c3 or c4) from two rocprofv3 --pmc "
                         "output folders (FETCH_SIZE, WRITE_SIZE) of a run with --calibrate-copy-mib")
    args = ap.parse_args()
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by sequence or query chunk; no multi-GPU run exists)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_long_09_amd as qsa
    from block_sparse_long_09_amd.pipeline import DecodePath, PrefillPath
    from gen.configs import CONFIGS
    from gen.device import idx_keys_to_device, normal_to_device

    torch.cuda.set_device(0)
    if args.config == "c6":
        return run_paged_batch(args, torch, qsa)
    if args.kl:
        return run_distill_kl(args, torch, qsa)
    if args.gdn:
        return run_gdn(args, torch, qsa)
    if args.config == "c5":
        Wp, Wd = CONFIGS["c5a"], CONFIGS["c5b"]
    elif args.config == "c3":
        Wp, Wd = CONFIGS["c3"], None
    else:
        Wp, Wd = None, CONFIGS["c4"]
    if args.block_size or args.budget:
        import dataclasses
        base = Wp or Wd
        r = args.block_size or base.r
        budget = args.budget or base.k * base.r
        if r not in (1, 2, 4, 8, 16, 32) or budget % r or not 1 <= budget // r <= 1024:
            print(f"bench.py: need r in {{1, 2, 4, 8, 16, 32}} and budget a multiple of r with "
                  f"1 <= budget / r <= 1024 (r = {r}, budget = {budget})",
                  file=sys.stderr)
            sys.exit(2)

        def variant(W):
            return dataclasses.replace(W, name=f"{W.name}_r{r}_budget{budget}", r=r, k=budget // r) if W else None
        Wp, Wd = variant(Wp), variant(Wd)

    out = measure(Wp, Wd, args, torch, qsa, args.steps, args.warmup, headline=True)
    if args.config == "c5" and not (args.block_size or args.budget) and not args.no_extra:
        # the rest of the metric: the 256K chunked prefill and the 128K decode batch
        out["extra"] = {}
        for key, (Wp2, Wd2, steps) in {"c3": (CONFIGS["c3"], None, 2), "c4": (None, CONFIGS["c4"], 10)}.items():
            torch.cuda.empty_cache()
            r = measure(Wp2, Wd2, args, torch, qsa, steps, 1, headline=False)
            out["extra"][key] = {k: r[k] for k in ("config", "ms_per_step", "prefill_ms", "prefill_tokens_per_s",
                                                   "prefill_schedule", "decode_us_per_step", "phase_ms", "roofline",
                                                   "rooflines", "cpu_baseline", "sample_parity") if k in r}
    print(json.dumps(out), flush=True)


def measure(Wp, Wd, args, torch, qsa, steps, warmup, headline):
    """One prefill workload (Wp, chunked as it says) and/or one decode workload
    (Wd): inputs generated into HBM, `warmup` untimed steps, `steps` timed
    ones; returns the fields of the JSON line."""
    from block_sparse_long_09_amd.pipeline import DecodePath, PrefillPath
    from gen.device import idx_keys_to_device, normal_to_device
    dev = "cuda"

    t_setup = time.time()
    # ------------------------------------------------------------- inputs --
    P = {}
    if Wp is not None:
        W = Wp
        log(f"generating prefill inputs {W.name}")
        P["K"] = normal_to_device(W.seed, 2, (W.L, W.Hkv, W.D))
        P["V"] = normal_to_device(W.seed, 3, (W.L, W.Hkv, W.D))
        P["Q"] = normal_to_device(W.seed, 1, (W.n_q, W.Hq, W.D))
        P["iq"] = normal_to_device(W.seed, 4, (W.n_q, W.Hi, W.di))
        P["ik"] = idx_keys_to_device(W.seed, 1, W.L, W.di, W.needle_window, W.r)[0]
        P["cmp"] = torch.zeros((W.n_blk, W.di), dtype=torch.bfloat16, device=dev)
        chunk = W.chunk if W.chunk else W.n_q
        P["chunk"] = chunk
        # blocks before the first query are cached (as the prefix KV is)
        if W.q_pos0 // W.r:
            qsa.qsa_compress_keys(P["ik"], P["cmp"], W.r, 0, W.q_pos0 // W.r)
        P["path"] = PrefillPath(W.Hq, W.Hkv, W.Hi, W.r, W.k, n_q_max=chunk, max_len=W.q_pos0 + W.n_q,
                                D=W.D, di=W.di, device=dev)
    D = {}
    if Wd is not None:
        W = Wd
        log(f"generating decode inputs {W.name}")
        D["Kc"] = normal_to_device(W.seed, 2, (W.batch, W.L, W.Hkv, W.D))
        D["Vc"] = normal_to_device(W.seed, 3, (W.batch, W.L, W.Hkv, W.D))
        D["Q"] = normal_to_device(W.seed, 1, (W.batch, W.Hq, W.D))
        D["iq"] = normal_to_device(W.seed, 4, (W.batch, W.Hi, W.di))
        ik = idx_keys_to_device(W.seed, W.batch, W.L, W.di, W.needle_window, W.r)
        D["cmp"] = torch.empty((W.batch, W.n_blk, W.di), dtype=torch.bfloat16, device=dev)
        qsa.qsa_compress_keys(ik, D["cmp"], W.r, 0, W.n_blk)  # precomputed block keys
        torch.cuda.synchronize()
        del ik
        D["kv_len"] = torch.full((W.batch,), W.L, dtype=torch.int32, device=dev)
        D["q_pos"] = D["kv_len"] - 1
        D["path"] = DecodePath(W.Hq, W.Hkv, W.Hi, W.batch, W.L, r=W.r, k=W.k, D=W.D, di=W.di, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s")

    # ------------------------------------------------------------ the step --
    names = []
    fns = []
    if Wp is not None:
        W, path = Wp, P["path"]
        chunk = P["chunk"]
        for c0 in range(0, W.n_q, chunk):
            q0 = W.q_pos0 + c0
            sfx = f"_{c0 // chunk}" if chunk != W.n_q else ""
            names += [f"compress{sfx}", f"index_prefill{sfx}", f"attn_prefill{sfx}"]
            fns += [
                (lambda q0=q0: path.compress(P["ik"], P["cmp"], q0, chunk)),
                (lambda q0=q0, c0=c0: path.select(P["iq"][c0:c0 + chunk], P["cmp"], q0, chunk)),
                (lambda q0=q0, c0=c0: path.attend(P["Q"][c0:c0 + chunk], P["K"], P["V"], q0, chunk)),
            ]
    if Wd is not None:
        dp = D["path"]
        names += ["index_decode", "attn_decode"]
        fns += [lambda: dp.select(D["iq"], D["cmp"], D["q_pos"]),
                lambda: dp.attend(D["Q"], D["Kc"], D["Vc"], D["kv_len"])]
    timer = PhaseTimer(torch, names)

    for _ in range(warmup):
        timer.run(fns)
    torch.cuda.synchronize()
    # phase timing (events between launches, on the launch stream)
    recorded = [timer.run(fns) for _ in range(steps)]
    torch.cuda.synchronize()
    for evs in recorded:
        timer.collect(evs)
    # whole-step wall clock over exactly `steps` steps. A prefill in several
    # chunks runs chunk c's attention beside chunk c + 1's compression and
    # indexer on two streams (ChunkedPrefill); the phase times above come
    # from the chunks run one after the other and attribute the time per
    # kernel.
    step = lambda: [f() for f in fns]
    schedule = None
    if Wp is not None and Wd is None and P["chunk"] < Wp.n_q:
        from block_sparse_long_09_amd.pipeline import ChunkedPrefill
        W = Wp
        cp = ChunkedPrefill(W.Hq, W.Hkv, W.Hi, W.r, W.k, chunk=P["chunk"], max_len=W.q_pos0 + W.n_q,
                            D=W.D, di=W.di, device=dev)
        full_out = torch.empty((W.n_q, W.Hq, W.D), dtype=torch.bfloat16, device=dev)
        full_lse = torch.empty((W.n_q, W.Hq), dtype=torch.float32, device=dev)
        step = lambda: cp(P["Q"], P["K"], P["V"], P["iq"], P["ik"], P["cmp"], W.q_pos0, W.n_q, full_out, full_lse)
        step()
        schedule = "chunk c's attention beside chunk c+1's compress + indexer (two streams)"
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    phase = timer.mean_ms()

    def ssum(prefix):
        v = [x for n, x in phase.items() if n.startswith(prefix)]
        return sum(v) if v else 0.0

    prefill_ms = ssum("compress") + ssum("index_prefill") + ssum("attn_prefill")
    decode_ms = ssum("index_decode") + ssum("attn_decode")

    # --------------------------------------------------------------- roofline --
    roof = {}
    sha_attn = source_sha("sparse_attn.hip")
    sha_idx = source_sha("index_topk.hip")
    if Wp is not None:
        W = Wp
        work = {"compress_bytes": 0, "index_flops": 0, "index_bytes": 0, "attn_bytes": 0, "attn_flops": 0,
                "attn_tokens": 0, "index_pairs": 0, "dense_flops": 0}
        chunk = P["chunk"]
        for c0 in range(0, W.n_q, chunk):
            wk = prefill_work(W, W.q_pos0 + c0, chunk)
            for key in work:
                work[key] += wk[key]
        n_ch = W.n_q // chunk
        ms_attn, ms_idx = ssum("attn_prefill"), ssum("index_prefill")
        wkey = "c5" if Wp.name.startswith("c5a") else Wp.name.split("_")[0]
        roof["attn_prefill"] = {
            "bound": "hbm", "achieved": work["attn_bytes"] / (ms_attn * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "traffic": load_traffic(f"attn_prefill_{wkey}", sha_attn),
            "bytes_per_launch": work["attn_bytes"] // n_ch, "avg_launch_ms": ms_attn / n_ch,
            "mfma_tflops": work["attn_flops"] / (ms_attn * 1e-3) / 1e12}
        roof["index_prefill"] = {
            "bound": "mfma", "achieved": work["index_flops"] / (ms_idx * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s", "traffic": load_traffic(f"index_prefill_{wkey}", sha_idx),
            "flops_per_launch": work["index_flops"] // n_ch, "avg_launch_ms": ms_idx / n_ch}
        P["work"] = work
    if Wd is not None:
        W = Wd
        wd = decode_work(W)
        ms = decode_ms
        roof["decode"] = {"bound": "hbm", "achieved": (wd["index_bytes"] + wd["attn_bytes"]) / (ms * 1e-3) / 1e9,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "traffic": decode_traffic(args.config if headline else "c4", sha_idx, sha_attn),
                          "bytes_per_step": wd["index_bytes"] + wd["attn_bytes"]}
        D["work"] = wd
    for v in roof.values():
        v["frac"] = v["achieved"] / v["peak"]
    # the dominant kernel: the phase with the largest total time
    totals = {"attn_prefill": ssum("attn_prefill"), "index_prefill": ssum("index_prefill"), "decode": decode_ms}
    dom = max((n for n in roof), key=lambda n: totals[n]) if roof else None

    # -------------------------------------------------------------- dense ----
    dense = None
    if not args.no_dense and headline:
        dense = {}
        if Wd is not None:
            W = Wd
            desc = qsa.attn_desc(W.Hq, W.Hkv, W.D)
            ws = qsa.workspace(qsa.qsa_dense_attn_workspace_size(desc, W.batch, 1, W.L))
            dout = torch.empty((W.batch, W.Hq, W.D), dtype=torch.bfloat16, device=dev)
            f = lambda: qsa.qsa_dense_attn_decode(desc, D["Q"], D["Kc"], D["Vc"], D["kv_len"], dout, None, ws)
            for _ in range(2):
                f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                f()
            e1.record()
            torch.cuda.synchronize()
            dms = e0.elapsed_time(e1) / 5
            dense["decode_us"] = dms * 1e3
            dense["decode_GBps"] = D["work"]["dense_bytes"] / (dms * 1e-3) / 1e9
            dense["decode_speedup_sparse_vs_dense"] = dms / decode_ms
        if Wp is not None:
            W = Wp
            desc = qsa.attn_desc(W.Hq, W.Hkv, W.D)
            dout = torch.empty((P["chunk"], W.Hq, W.D), dtype=torch.bfloat16, device=dev)
            chunk = P["chunk"]

            def fd():
                for c0 in range(0, W.n_q, chunk):
                    qsa.qsa_dense_attn_prefill(desc, P["Q"][c0:c0 + chunk], P["K"][:W.q_pos0 + c0 + chunk],
                                               P["V"][:W.q_pos0 + c0 + chunk], W.q_pos0 + c0, dout)
            fd()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fd()
            e1.record()
            torch.cuda.synchronize()
            pms = e0.elapsed_time(e1)
            dense["prefill_ms"] = pms
            dense["prefill_TFLOPs"] = P["work"]["dense_flops"] / (pms * 1e-3) / 1e12
            dense["prefill_speedup_sparse_vs_dense"] = pms / prefill_ms
            dense["prefill_attention_only_speedup"] = pms / ssum("attn_prefill")

    # --------------------------------------------------------- calibration ---
    if args.calibrate_copy_mib and headline:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    # ---------------------------------------------------------- CPU oracle ---
    cpu = None
    sample_parity = None
    if not args.no_cpu_baseline and Wp is not None:
        cpu, sample_parity = cpu_baseline(Wp, P, args.cpu_sample if headline else 128)
    if not args.no_cpu_baseline and Wd is not None:
        dcpu, dpar = decode_cpu_baseline(Wd, D, Wd.batch if Wd.batch <= 8 else 2)
        if cpu is None:
            cpu, sample_parity = dcpu, dpar
        else:
            cpu = dict(cpu, decode=dcpu)
            sample_parity = dict(sample_parity, decode=dpar)

    W = Wp if Wp is not None else Wd
    value = (Wp.n_q if Wp is not None else Wd.batch) / wall
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (Wp.name + " + " + Wd.name) if (Wp and Wd) else W.name,
                   "prefill_queries": Wp.n_q if Wp else 0, "context": W.L, "budget_tokens": W.k * W.r,
                   "block_size": W.r, "heads_q_kv_idx": [W.Hq, W.Hkv, W.Hi],
                   "decode_batch": Wd.batch if Wd else 0},
        "prefill_ms": prefill_ms if Wp else None,
        # a chunked prefill's phases overlap: its rate is the wall clock's
        "prefill_tokens_per_s": (Wp.n_q / (wall if schedule else prefill_ms * 1e-3)) if Wp else None,
        "prefill_schedule": schedule,
        "decode_us_per_step": decode_ms * 1e3 if Wd else None,
        "phase_ms": phase,
        "roofline": dict(roof[dom], kernel=dom) if dom else None,
        "rooflines": roof,
        "dense": dense,
        "pages_speedup_context": PAGES_SPEEDUP,
        "cpu_baseline": cpu,
        "sample_parity": sample_parity,
    }
    return out


def paged_work(W):
    """Algorithmic work of one packed step (each sequence's new rows)."""
    work = {"index_flops": 0, "attn_bytes": 0, "attn_flops": 0, "rows": 0}
    for p0, n in zip(W.prefix, W.new):
        t = np.arange(p0, p0 + n, dtype=np.int64)
        b = t // W.r
        ntok = np.minimum(W.k - 1, b) * W.r + (t - b * W.r) + 1
        work["index_flops"] += int(b.sum()) * W.Hi * W.di * 2
        work["attn_bytes"] += int(ntok.sum()) * W.Hkv * W.D * 2 * 2 + 2 * n * W.Hq * W.D * 2 + n * (W.k + 1) * 4
        work["attn_flops"] += int(ntok.sum()) * W.Hq * W.D * 4
        work["rows"] += n
    return work


def run_paged_batch(args, torch, qsa):
    """Packed variable-length batch over a paged K/V pool (config 6)."""
    from block_sparse_long_09_amd.pipeline import PagedBatchPath
    from gen.configs import PAGED
    from gen.device import paged_batch_to_device
    W = PAGED[args.config]
    dev = "cuda"
    B = W.batch
    t_setup = time.time()
    log(f"generating paged pool {W.name}")
    I = paged_batch_to_device(W, dev)
    kpool, vpool, table_d, Q, iq, ik, cu, p0 = (I[n] for n in ("kpool", "vpool", "table", "Q", "iq", "ik", "cu",
                                                              "q_pos0"))
    total, max_len = I["total"], I["max_len"]
    cmp = torch.zeros((B, max_len // W.r, W.di), dtype=torch.bfloat16, device=dev)
    for b in range(B):  # the cached prefixes' block keys
        qsa.qsa_compress_keys(ik[b], cmp[b], W.r, 0, W.prefix[b] // W.r)
    path = PagedBatchPath(W.Hq, W.Hkv, W.Hi, B, max(W.new), max_len, r=W.r, k=W.k, D=W.D, di=W.di, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s")
    names = ["compress", "index_varlen", "attn_paged"]
    fns = [lambda: path.compress(ik, cmp, W.prefix, W.new),
           lambda: path.select(iq, cmp, cu, p0, total),
           lambda: path.attend(Q, kpool, vpool, table_d, cu, p0, total)]
    timer = PhaseTimer(torch, names)
    for _ in range(args.warmup):
        timer.run(fns)
    torch.cuda.synchronize()
    recorded = [timer.run(fns) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for evs in recorded:
        timer.collect(evs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for f in fns:
            f()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    phase = timer.mean_ms()
    work = paged_work(W)
    roof = {
        "attn_paged": {"bound": "hbm", "achieved": work["attn_bytes"] / (phase["attn_paged"] * 1e-3) / 1e9,
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None, "bytes_per_launch": work["attn_bytes"],
                       "avg_launch_ms": phase["attn_paged"],
                       "mfma_tflops": work["attn_flops"] / (phase["attn_paged"] * 1e-3) / 1e12},
        "index_varlen": {"bound": "mfma", "achieved": work["index_flops"] / (phase["index_varlen"] * 1e-3) / 1e12,
                         "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "traffic": None,
                         "flops_per_launch": work["index_flops"], "avg_launch_ms": phase["index_varlen"]},
    }
    for v in roof.values():
        v["frac"] = v["achieved"] / v["peak"]
    dom = max(roof, key=lambda n: phase[n])
    step_ms = sum(phase.values())
    out = {
        "metric": METRIC,
        "value": work["rows"] / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": W.name, "sequences": B, "cached_prefix": list(W.prefix), "new_rows": list(W.new),
                   "page_size": W.page_size, "budget_tokens": W.k * W.r, "block_size": W.r,
                   "heads_q_kv_idx": [W.Hq, W.Hkv, W.Hi]},
        "phase_ms": phase,
        "phase_sum_ms": step_ms,
        "roofline": dict(roof[dom], kernel=dom),
        "rooflines": roof,
        "dense": None,
        "pages_speedup_context": PAGES_SPEEDUP,
        "cpu_baseline": None,
        "sample_parity": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["sample_parity"] = paged_cpu_baseline(W, I["table_host"], path, total)
    print(json.dumps(out), flush=True)


def paged_cpu_baseline(W, table, path, total):
    """The oracle (select + attend) on two or three new rows of every sequence
    of a packed paged batch, on the host cores, and the parity of those rows
    against the GPU's outputs (selections bit-exact or inside the near-tie
    band, outputs within 2e-2 max / 1e-3 mean, lse within 2e-4)."""
    import gen
    import oracle
    from gen.device import paged_batch_layout, paged_sequence_host
    g_sel = path.sel[:total].cpu().numpy()
    g_cnt = path.cnt[:total].cpu().numpy()
    g_out = path.out[:total].float().cpu().numpy()
    g_lse = path.lse[:total].cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(W.new)])
    key_len = paged_batch_layout(W)[2]
    rng = np.random.default_rng(17)
    t_or = 0.0
    n_rows = same = 0
    err = lerr = 0.0
    for b in range(W.batch):
        n = W.new[b]
        loc = sorted({0, n - 1} | ({int(rng.integers(0, n))} if n > 2 else set()))
        L_b = W.prefix[b] + n
        ik = gen.idx_keys(W.seed, b, key_len, 0, L_b, W.di, W.needle_window, W.r)
        Kb = paged_sequence_host(W, table, b, 2, L_b)
        Vb = paged_sequence_host(W, table, b, 3, L_b)
        tc = time.perf_counter()
        blocks = oracle.compress(ik, W.r)
        for i in loc:
            row = int(cu[b] + i)
            t = W.prefix[b] + i
            q = gen.normal(W.seed, 1, (1, W.Hq, W.D), e0=row * W.Hq * W.D)
            iqr = gen.normal(W.seed, 4, (1, W.Hi, W.di), e0=row * W.Hi * W.di)
            s, c, _, _ = oracle.select(iqr, blocks, t, W.r, W.k, W.w)
            o, lo = oracle.sparse_attn(q, Kb, Vb, t, W.r, s, c)
            n_rows += 1
            if np.array_equal(g_sel[row], s[0]) and g_cnt[row] == c[0]:
                same += 1
                err = max(err, float(np.abs(g_out[row] - o[0]).max()))
                lerr = max(lerr, float(np.abs(g_lse[row] - lo[0]).max()))
        t_or += time.perf_counter() - tc
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    cpu = {"value": n_rows / t_or, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{n_rows} of {total} new rows (first, last and one random row of each sequence) of {W.name}: "
                     f"block compression of each sequence's keys, selection and attention ({t_or:.2f}s)"}
    return cpu, {"rows": n_rows, "selection_identical_rows": same, "out_max_abs": err, "lse_max_abs": lerr}


def run_distill_kl(args, torch, qsa):
    """Forward of the indexer's dense-distillation KL over a prefill workload."""
    from gen.configs import CONFIGS
    from gen.device import idx_keys_to_device, normal_to_device
    W = CONFIGS["c2" if args.config == "c5" else args.config]
    if W.mode != "prefill":
        print("bench.py: --kl needs a prefill workload (c2, c3 or the default)", file=sys.stderr)
        sys.exit(2)
    dev = "cuda"
    t_setup = time.time()
    n_q = W.chunk or W.n_q
    q0 = W.q_pos0 + W.n_q - n_q  # the last chunk: the longest rows
    K = normal_to_device(W.seed, 2, (W.L, W.Hkv, W.D))
    Q = normal_to_device(W.seed, 1, (W.n_q, W.Hq, W.D))[W.n_q - n_q:]
    iq = normal_to_device(W.seed, 4, (W.n_q, W.Hi, W.di))[W.n_q - n_q:]
    ik = idx_keys_to_device(W.seed, 1, W.L, W.di, W.needle_window, W.r)[0]
    cmp = torch.zeros((W.n_blk, W.di), dtype=torch.bfloat16, device=dev)
    qsa.qsa_compress_keys(ik, cmp, W.r, 0, W.n_blk)
    adesc = qsa.attn_desc(W.Hq, W.Hkv, W.D)
    idesc = qsa.index_desc(W.r, W.k, W.Hi, W.di)
    kl = torch.empty(n_q, dtype=torch.float32, device=dev)
    ws = qsa.workspace(qsa.qsa_distill_kl_workspace_size(adesc, n_q))
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s")
    f = lambda: qsa.qsa_distill_kl_prefill(adesc, idesc, Q, K, iq, cmp, q0, kl, ws)
    for _ in range(args.warmup):
        f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        f()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    t = np.arange(q0, q0 + n_q, dtype=np.int64)
    # two passes of Q K^T over every (query, token <= t) pair, plus the indexer scores of the candidates
    flops = 2 * int((t + 1).sum()) * W.Hq * W.D * 2 + int((t // W.r).sum()) * W.Hi * W.di * 2
    roof = {"bound": "mfma", "achieved": flops / wall / 1e12, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "traffic": None, "flops_per_launch": flops, "avg_launch_ms": wall * 1e3}
    roof["frac"] = roof["achieved"] / roof["peak"]
    out = {
        "metric": METRIC, "value": n_q / wall, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": W.name + "_distill_kl_forward", "queries": n_q, "first_position": q0,
                   "context": W.L, "block_size": W.r, "heads_q_kv_idx": [W.Hq, W.Hkv, W.Hi]},
        "kl_mean": float(kl.mean().item()),
        "roofline": dict(roof, kernel="distill_kl"), "dense": None, "cpu_baseline": None, "sample_parity": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["sample_parity"] = distill_cpu_baseline(W, q0, n_q, kl)
    print(json.dumps(out), flush=True)


def distill_cpu_baseline(W, q0, n_q, kl):
    """The oracle's loss on 16 rows of the timed call (the first rows, rows
    near the end, random rows), timed on the host cores, and their parity
    (1e-4 absolute + 1e-4 relative)."""
    import gen
    import oracle
    g = kl.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, 4, n_q // 2, n_q - 2, n_q - 1], rng.integers(n_q - 1024, n_q, 6),
                                     rng.integers(0, n_q, 5)]))
    K = gen.normal(W.seed, 2, (W.L, W.Hkv, W.D))
    blocks = oracle.compress(gen.idx_keys(W.seed, 0, W.L, 0, W.L, W.di, W.needle_window, W.r), W.r)
    first = W.n_q - n_q  # row of the generated tensors that the call's row 0 is
    worst = 0.0
    ok = 0
    tc = time.perf_counter()
    for i in rows:
        i = int(i)
        gi = first + i
        q = gen.normal(W.seed, 1, (1, W.Hq, W.D), e0=gi * W.Hq * W.D)
        iqr = gen.normal(W.seed, 4, (1, W.Hi, W.di), e0=gi * W.Hi * W.di)
        o = float(oracle.distill_kl(q, K, iqr, blocks, q0 + i, W.r, W.w)[0])
        e = abs(g[i] - o)
        worst = max(worst, e)
        ok += int(e <= 1e-4 + 1e-4 * abs(o))
    el = time.perf_counter() - tc
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    cpu = {"value": len(rows) / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(rows)} of {n_q} query rows of {W.name} (first rows, rows near the end, random rows), "
                     f"loss per row ({el:.2f}s)"}
    return cpu, {"rows": int(len(rows)), "within_tolerance_rows": ok, "kl_max_abs_err": worst}


def gdn_work(W):
    """Algorithmic HBM bytes of one prefill call (inputs read once, outputs
    written once) and of one decode step (the fp32 state read and written)."""
    tok = W.batch * W.T
    prefill = tok * (2 * W.Hqk * W.dk * 2 + W.Hv * W.dv * 2 * 2 + 2 * W.Hv * 4)
    return {"prefill_bytes": prefill}


def run_gdn(args, torch, qsa):
    import gen
    from gen.configs import GDN
    t_setup = time.time()
    Wp, Wd = GDN["g1"], GDN["g2"]
    dev = "cuda"

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    hq, hk, hv, hg, hb = gen.gdn_inputs(Wp.seed, Wp.batch, Wp.T, Wp.Hqk, Wp.Hv, Wp.dk, Wp.dv)
    q, k, v, g, beta = (up(a) for a in (hq, hk, hv, hg, hb))
    desc = qsa.gdn_desc(Wp.Hqk, Wp.Hv, Wp.dk, Wp.dv)
    out = torch.empty((Wp.batch, Wp.T, Wp.Hv, Wp.dv), dtype=torch.bfloat16, device=dev)
    Sf = torch.empty((Wp.batch, Wp.Hv, Wp.dv, Wp.dk), dtype=torch.float32, device=dev)
    ws = qsa.workspace(qsa.qsa_gdn_prefill_workspace_size(desc, Wp.batch, Wp.T))
    # decode: 64 sequences, one token each, on carried states
    dq, dk_, dv_, dg, db = gen.gdn_inputs(Wd.seed, Wd.batch, 1, Wd.Hqk, Wd.Hv, Wd.dk, Wd.dv)
    Dq, Dk, Dv, Dg, Db = (up(a[:, 0]) for a in (dq, dk_, dv_, dg, db))
    state = up(gen.gdn_state(Wd.seed, Wd.batch, Wd.Hv, Wd.dv, Wd.dk))
    dout = torch.empty((Wd.batch, Wd.Hv, Wd.dv), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s")
    fp = lambda: qsa.qsa_gdn_prefill(desc, q, k, v, g, beta, out, final_state=Sf, workspace=ws)
    fd = lambda: qsa.qsa_gdn_decode(desc, Dq, Dk, Dv, Dg, Db, state, dout)
    for _ in range(args.warmup):
        fp()
        fd()
    torch.cuda.synchronize()
    timer = PhaseTimer(torch, ["prefill", "decode"])
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        evs.append(timer.run([fp, fd]))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    for e in evs:
        timer.collect(e)
    ms = timer.mean_ms()
    work = gdn_work(Wp)
    dec_bytes = Wd.batch * Wd.Hv * (2 * Wd.dv * Wd.dk * 4 + 2 * Wd.dv * 2) + Wd.batch * Wd.Hqk * Wd.dk * 2 * 2
    roof_p = {"bound": "hbm", "achieved": work["prefill_bytes"] / (ms["prefill"] * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
              "unit": "GB/s", "traffic": None, "bytes_per_launch": work["prefill_bytes"],
              "avg_launch_ms": ms["prefill"]}
    roof_p["frac"] = roof_p["achieved"] / roof_p["peak"]
    roof_d = {"bound": "hbm", "achieved": dec_bytes / (ms["decode"] * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
              "unit": "GB/s", "traffic": None, "bytes_per_launch": dec_bytes, "avg_launch_ms": ms["decode"]}
    roof_d["frac"] = roof_d["achieved"] / roof_d["peak"]
    cpu = None
    sample = None
    if not args.no_cpu_baseline:
        import oracle
        heads = [0, Wp.Hv - 1]
        log(f"cpu baseline: the oracle over value heads {heads}, all {Wp.T} tokens")
        tc = time.perf_counter()
        o_ref, s_ref = oracle.gdn(hq[0], hk[0], hv[0], hg[0], hb[0], heads=heads)
        el = time.perf_counter() - tc
        cpu = {"value": Wp.T * len(heads) / Wp.Hv / el, "unit": "tokens/s", "cores": os.cpu_count(),
               "kind": "oracle",
               "sample": f"value heads {heads} of {Wp.Hv} over all {Wp.T} tokens of {Wp.name} "
                         f"({el:.2f}s), scaled to the whole layer"}
        go = out.float().cpu().numpy().astype(np.float64)
        gs = Sf.cpu().numpy().astype(np.float64)
        rel = []
        for h in heads:
            e = np.abs(go[0, :, h] - o_ref[:, h])
            rel.append((e.max() / np.abs(o_ref[:, h]).max(), e.mean() / np.sqrt((o_ref[:, h] ** 2).mean()),
                        np.abs(gs[0, h] - s_ref[h]).max() / np.sqrt((s_ref[h] ** 2).mean())))
        sample = {"heads": heads, "out_max_err_rel_max": max(r[0] for r in rel),
                  "out_mean_err_rel_rms": max(r[1] for r in rel), "state_max_err_rel_rms": max(r[2] for r in rel)}
    res = {
        "metric": "GDN (gated delta rule) prefill tokens/s, one layer; decode us/step; % of HBM roofline",
        "value": Wp.batch * Wp.T / (ms["prefill"] * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": Wp.name + " + " + Wd.name, "tokens": Wp.T, "heads_qk_v": [Wp.Hqk, Wp.Hv],
                   "head_dims": [Wp.dk, Wp.dv], "decode_batch": Wd.batch},
        "prefill_ms": ms["prefill"], "decode_us_per_step": ms["decode"] * 1e3,
        "roofline": dict(roof_p, kernel="gdn_prefill (prep + scan)"),
        "rooflines": {"prefill": roof_p, "decode": roof_d},
        "cpu_baseline": cpu, "sample_parity": sample,
    }
    print(json.dumps(res), flush=True)


def cpu_baseline(W, P, n_sample):
    """Time the oracle on a bounded sample of the prefill chunk's queries (plus
    the chunk's block compression) on the host cores; also compare the GPU
    outputs of those rows."""
    import torch

    import gen
    import oracle

    # the path's buffers hold the last chunk's outputs: sample its rows
    n_q = P["chunk"]
    first = W.n_q - n_q  # generated row of the chunk's row 0
    q0 = W.q_pos0 + first
    run = 32  # consecutive queries per oracle call (OpenMP parallelises over them)
    n_runs = max(1, n_sample // run)
    starts = np.unique(np.linspace(0, n_q - run, n_runs).astype(np.int64))
    rows = np.concatenate([np.arange(s0, s0 + run) for s0 in starts])
    log(f"cpu baseline: generating host inputs, {len(rows)} sampled queries")
    ik = gen.idx_keys(W.seed, 0, W.L, 0, W.L, W.di, W.needle_window, W.r)
    K = gen.normal(W.seed, 2, (W.L, W.Hkv, W.D))
    V = gen.normal(W.seed, 3, (W.L, W.Hkv, W.D))
    Qr = [gen.normal(W.seed, 1, (run, W.Hq, W.D), e0=(first + int(s0)) * W.Hq * W.D) for s0 in starts]
    iqr = [gen.normal(W.seed, 4, (run, W.Hi, W.di), e0=(first + int(s0)) * W.Hi * W.di) for s0 in starts]
    n_prefix = q0 // W.r
    blocks = np.empty(((q0 + n_q) // W.r, W.di), np.uint16)
    blocks[:n_prefix] = oracle.compress(ik[:n_prefix * W.r], W.r)  # cached prefix, like the GPU's
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    blocks[n_prefix:] = oracle.compress(ik[n_prefix * W.r:(q0 + n_q) // W.r * W.r], W.r)
    t_comp = time.perf_counter() - t0
    sels, cnts = [], []
    t1 = time.perf_counter()
    for i, s0 in enumerate(starts):
        s, c, _, _ = oracle.select(iqr[i], blocks, q0 + int(s0), W.r, W.k, W.w)
        sels.append(s)
        cnts.append(c)
    t_sel = time.perf_counter() - t1
    t2 = time.perf_counter()
    outs, lses = [], []
    for i, s0 in enumerate(starts):
        o, l = oracle.sparse_attn(Qr[i], K, V, q0 + int(s0), W.r, sels[i], cnts[i])
        outs.append(o)
        lses.append(l)
    t_att = time.perf_counter() - t2
    sel = np.concatenate(sels)
    outs = list(zip(np.concatenate(outs), np.concatenate(lses)))
    # per-query time of the sample, plus the chunk compression amortised over all queries
    per_q = (t_sel + t_att) / len(rows) + t_comp / n_q
    what = f"{n_q} queries of the last chunk" if n_q != W.n_q else f"{n_q} prefill queries"
    cpu = {"value": 1.0 / per_q, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"{len(rows)} of {what} ({len(starts)} runs of {run} consecutive, evenly "
                     f"spaced) of {W.name}, plus the chunk's block compression; select {t_sel:.2f}s, "
                     f"attend {t_att:.2f}s, compress {t_comp:.2f}s"}
    # parity of the sampled rows (the GPU ran the same inputs)
    path = P["path"]
    g_sel = path.sel.cpu().numpy()
    g_cnt = path.cnt.cpu().numpy()
    g_out = path.out.float().cpu().numpy()
    g_lse = path.lse.cpu().numpy()
    same_sel = sum(int(np.array_equal(g_sel[r_], sel[i])) for i, r_ in enumerate(rows))
    err = max(float(np.abs(g_out[r_] - outs[i][0]).max()) for i, r_ in enumerate(rows)
              if np.array_equal(g_sel[r_], sel[i]))
    lerr = max(float(np.abs(g_lse[r_] - outs[i][1]).max()) for i, r_ in enumerate(rows)
               if np.array_equal(g_sel[r_], sel[i]))
    return cpu, {"rows": len(rows), "selection_identical_rows": same_sel, "out_max_abs": err, "lse_max_abs": lerr}


def summarize_traffic(fetch_dir, write_dir, key):
    """Per-launch HBM bytes of the step's kernels from the counters of two
    rocprofv3 runs of bench.py (FETCH_SIZE, then WRITE_SIZE, both with
    --calibrate-copy-mib N), scaled by what the same counters read for the
    plain device copy of N MiB in the same run; merged into
    profiles/traffic.json under names ending in _KEY, each with the source
    hash of its kernel file."""
    import csv
    import glob

    def read(d, counter):
        rows = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                wgs = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
                k = (r["Kernel_Name"], wgs)
                rows.setdefault(k, []).append(float(r["Counter_Value"]))
        return rows

    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    # the calibration copy: the non-library kernel that writes the most
    copies = [(k, v) for k, v in write.items() if "qsa::" not in k[0]]
    (ck, cw) = max(copies, key=lambda kv: max(kv[1]))
    w_kib = max(cw)
    f_kib = max(fetch.get(ck, [0.0]))
    copy_bytes = round(w_kib * 1024 / (1 << 20)) << 20  # the copy writes its size once
    roles = [("index_prefill_kernel", "index_prefill", "index_topk.hip"),
             ("index_select_kernel", "index_select", "index_topk.hip"),
             ("index_decode_scan_kernel", "decode_scan", "index_topk.hip"),
             ("index_decode_select_kernel", "decode_merge", "index_topk.hip"),
             ("attn_merge_kernel", "decode_attn_merge", "sparse_attn.hip"),
             ("compress_kernel", "compress", "compress.hip")]
    path = os.path.join(ROOT, "profiles", "traffic.json")
    d = json.load(open(path)) if os.path.exists(path) else {}
    d["calibration"] = {"copy_bytes": copy_bytes, "fetch_kib": f_kib, "write_kib": w_kib,
                        "fetch_factor": copy_bytes / (f_kib * 1024), "write_factor": copy_bytes / (w_kib * 1024)}
    ff, wf = d["calibration"]["fetch_factor"], d["calibration"]["write_factor"]
    for (name, wgs), fv in fetch.items():
        if "qsa::" not in name:
            continue
        role = None
        for pat, r, src in roles:
            if pat in name:
                role, file = r, src
        if "attn_gather_kernel" in name:
            role, file = ("attn_prefill" if wgs >= 1024 else "decode_attn"), "sparse_attn.hip"
        if role is None:
            continue
        wv = write.get((name, wgs), [0.0])
        fk, wk = float(np.mean(fv)), float(np.mean(wv))
        d[f"{role}_{key}"] = {"kernel": name.split("(")[0], "workgroups": wgs, "source_sha": source_sha(file),
                              "fetch_kib_raw": fk, "write_kib_raw": wk, "fetch_bytes": fk * 1024 * ff,
                              "write_bytes": wk * 1024 * wf, "bytes_per_launch": fk * 1024 * ff + wk * 1024 * wf}
    with open(path, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps({k: v.get("bytes_per_launch") for k, v in d.items() if k.endswith(key)}, indent=1))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def decode_cpu_baseline(W, D, n_seq):
    """The oracle's whole decode step (block keys of the cache compressed,
    selection over every candidate, attention over the kept tokens) for the
    first n_seq sequences, timed on the host cores, and the parity of those
    sequences against the GPU's selection and output."""
    import gen
    import oracle
    path = D["path"]
    g_sel = path.sel[:, 0].cpu().numpy()
    g_cnt = path.cnt[:, 0].cpu().numpy()
    g_out = path.out.float().cpu().numpy()
    g_lse = path.lse.cpu().numpy()
    t = W.L - 1
    t_or = 0.0
    same = 0
    err = lerr = 0.0
    for b in range(n_seq):
        ik = gen.idx_keys(W.seed, b, W.L, 0, W.L, W.di, W.needle_window, W.r)
        Kb = gen.normal(W.seed, 2, (W.L, W.Hkv, W.D), e0=b * W.L * W.Hkv * W.D)
        Vb = gen.normal(W.seed, 3, (W.L, W.Hkv, W.D), e0=b * W.L * W.Hkv * W.D)
        qb = gen.normal(W.seed, 1, (1, W.Hq, W.D), e0=b * W.Hq * W.D)
        iqb = gen.normal(W.seed, 4, (1, W.Hi, W.di), e0=b * W.Hi * W.di)
        tc = time.perf_counter()
        blocks = oracle.compress(ik, W.r)
        s, c, _, _ = oracle.select(iqb, blocks, t, W.r, W.k, W.w)
        o, lo = oracle.sparse_attn(qb, Kb, Vb, t, W.r, s, c)
        t_or += time.perf_counter() - tc
        if np.array_equal(g_sel[b], s[0]) and g_cnt[b] == c[0]:
            same += 1
            err = max(err, float(np.abs(g_out[b] - o[0]).max()))
            lerr = max(lerr, float(np.abs(g_lse[b] - lo[0]).max()))
        del Kb, Vb, ik
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    cpu = {"value_us_per_step": t_or / n_seq * W.batch * 1e6, "unit": "us/step", "cores": threads,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"{n_seq} of {W.batch} sequences of {W.name}, whole step each (compress the cache's "
                     f"{W.n_blk} block keys, select, attend: {t_or:.2f}s), scaled to the batch"}
    return cpu, {"sequences": n_seq, "selection_identical": same, "out_max_abs": err, "lse_max_abs": lerr}


def decode_traffic(key, sha_idx, sha_attn):
    """Counter-derived HBM bytes of one decode step (every decode kernel of
    the step), if the counters were taken on the current sources."""
    parts = [load_traffic(f"decode_scan_{key}", sha_idx), load_traffic(f"decode_merge_{key}", sha_idx),
             load_traffic(f"decode_attn_{key}", sha_attn), load_traffic(f"decode_attn_merge_{key}", sha_attn)]
    return None if any(p is None for p in parts) else sum(parts)


if __name__ == "__main__":
    main()
