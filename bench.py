#!/usr/bin/env python3
"""Throughput of TreeWY verify + commit through one Gated DeltaNet layer on one
MI355X, with the store_all (full-state snapshotting) baseline and the CPU
oracle measured beside it in the same run.

One step = the commit of one step's accepted node plus the verification of a
draft tree (path gates, S0 . [K;Q] and gram on MFMA, tree-WY solve, outputs),
over one batch of synthetic inputs already resident in HBM.  Per workload, the
step is timed in several forms:

* ``fused`` (the headline): one ``treewy_commit_verify`` per step, which
  commits the previous step's accepted node into the state in place and
  verifies the new draft from it -- the serving loop in steady state;
* ``separate``: ``treewy_verify`` then ``treewy_commit`` of its accepted node;
* ``fused_pool``: ``treewy_commit_verify_pool``, the fused loop with each
  request's state in a slot-indexed pool;
* ``fused_pool_trees``: ``treewy_commit_verify_pool_trees``, the same with a
  tree per request (every request on the workload's tree);
* ``fused_bf16_state``: ``treewy_commit_verify_bf16state``, the fused loop
  with the state stored as bf16 (half the state bytes);
* ``fused_bf16_state_pool`` / ``fused_bf16_state_pool_trees``: the bf16
  state in a slot-indexed pool, with the workload's tree or a tree per
  request.

Inputs are rotated over several device copies (>= 2 GiB of state) so that
consecutive steps do not find the state in the 256 MB Infinity Cache.

Prints one JSON line.  The headline workload is the wide (3,3,3) tree (batch
512, 32 value heads, N = 40 nodes, the largest single-GPU tree workload);
the 35B-like chain and (2,2,2) tree and the 397B-like chain and (2,2,2) tree
follow in ``workloads``, each with its own roofline entry, store_all baseline
and CPU oracle baseline.  The CPU oracle runs first, before the GPU is
initialised, in one worker process per available core.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "verified draft nodes/s + HBM GB/s (% roofline), tree verify+commit, 1 GPU"
HEADLINE = "wide-tree333"
WORKLOADS = ["wide-tree333", "35b-chain4", "35b-tree222", "397b-chain4", "397b-tree222"]


def byte_model(cfg_B, H, N, ib, accepted_depths):
    """Algorithmic (minimum) HBM bytes per launch.
    commit_verify:       commit + verify - 65536 per (b,h) (the state is read once)
    verify, per (b,h):   S0 65536 + N*(q,k,v 3*128*ib + alpha,beta 2*ib + out 512 + vtilde 512 + gamma 4)
    commit, per (b,h):   S0 read + S_out write 131072 + L*(vtilde 512 + k 128*ib + gamma 4), L = depth(a)+1
    store_all, per (b,h): S0 65536 + N*(3*128*ib + 2*ib + out 512) + (N+1)*65536 snapshots
    select, per (b,h):   131072
    commit_verify_pool:  commit_verify + 4 per sequence (its slot index)
    commit_verify_bf16state: commit_verify - 65536 per (b,h) (state read and
                         written as bf16: 32 KiB each way)
    commit_verify_pool_trees: commit_verify_pool + per sequence its tree's node
                         count and N parents (4 + N) and the previous tree's
                         count and the accepted node's ancestor mask (4 + 8)
    the bf16-state pool forms: their fp32-state forms - 65536 per (b,h)"""
    heads = cfg_B * H
    verify = heads * (65536 + N * (3 * 128 * ib + 2 * ib + 512 + 512 + 4))
    L_total = sum(int(d) + 1 for d in accepted_depths)
    commit = H * (cfg_B * 131072 + L_total * (512 + 128 * ib + 4)) + cfg_B * 4
    store_all = heads * (65536 + N * (3 * 128 * ib + 2 * ib + 512) + (N + 1) * 65536)
    select = heads * 131072 + cfg_B * 4
    # commit-then-verify: the state read once and written once, the previous
    # step's path rows, and the new step's rows and outputs
    fused = commit + verify - heads * 65536
    return dict(treewy_verify=verify, treewy_commit=commit, treewy_store_all=store_all,
                treewy_store_all_select=select, treewy_commit_verify=fused,
                treewy_commit_verify_pool=fused + cfg_B * 4,
                treewy_commit_verify_pool_trees=fused + cfg_B * (4 + 4 + N + 4 + 8),
                treewy_commit_verify_bf16state=fused - heads * 65536,
                treewy_commit_verify_bf16state_pool=fused + cfg_B * 4 - heads * 65536,
                treewy_commit_verify_bf16state_pool_trees=(fused + cfg_B * (4 + 4 + N + 4 + 8)
                                                           - heads * 65536))


def prefill_bench(dev, H, B=256, T=256, chunk=16, reps=20, warmup=30):
    """Prefill of a batch of prompts: B sequences x T tokens x H heads, bf16
    inputs drawn like the workloads (alpha in [0.9, 1)).  Times treewy_prefill
    (one launch, the state on chip) and, beside it, treewy_prefill_chain (the
    verify/commit kernels, one launch per chunk).  Minimum bytes per head: the
    state read and written once (131072) + T tokens of q, k, v (3*256), alpha,
    beta (4) and out (512)."""
    import numpy as np
    import torch
    from gated_deltanet_tree_03_amd import abi
    g = torch.Generator(device=dev).manual_seed(7)
    rnd = lambda *shape: torch.randn(shape, generator=g, device=dev)
    unit = lambda x: torch.nn.functional.normalize(x, dim=-1)
    q = unit(rnd(B, T, H, 128)).to(torch.bfloat16)
    k = unit(rnd(B, T, H, 128)).to(torch.bfloat16)
    v = rnd(B, T, H, 128).to(torch.bfloat16)
    a = (0.9 + 0.1 * torch.rand((B, T, H), generator=g, device=dev)).to(torch.bfloat16)
    b = torch.sigmoid(rnd(B, T, H)).to(torch.bfloat16)
    S = rnd(B, H, 128, 128) * 0.02
    out = torch.empty((B, T, H, 128), dtype=torch.float32, device=dev)
    work = abi.prefill_workspace(B, H, chunk, dev)
    min_bytes = B * H * (131072 + T * (3 * 256 + 4 + 512))
    stream = torch.cuda.current_stream()

    def timed(fn, launches):
        # warm-up launches (launch times of this work settle over the first
        # ~20 ms: 1.14 ms for the first launch, up to 1.53 ms, then down to
        # ~1.2 ms by the 13th), then an event pair around each repetition; the
        # median (a host stall between enqueues only lengthens the gap between
        # repetitions)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
        gbps = min_bytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 3), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
                "algorithmic_bytes": min_bytes, "GBps": round(gbps, 1),
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "launches": launches}

    one = timed(lambda: abi.prefill(S, q, k, v, a, b, out=out, stream=stream), 1)
    # HBM bytes per launch from the rocprofv3 counters (profiles/traffic_prefill-256x256.md),
    # when taken on the current kernel sources at this size
    from gated_deltanet_tree_03_amd import profiling
    one["traffic"] = (profiling.read_traffic("treewy_prefill", "prefill-256x256")
                      if (B, T, H) == (256, 256, 32) else None)
    chunked = timed(lambda: abi.prefill_chain(S, q, k, v, a, b, chunk=chunk, out=out, work=work,
                                              stream=stream),
                    -(-T // chunk) + 1)
    return {"workload": f"batched prompt prefill: {B} sequences x {T} tokens x {H} heads, bf16",
            "entry": "treewy_prefill (one launch, chunks of 16 on chip)", **one,
            "chunked": {"entry": f"treewy_prefill_chain (chunks of {chunk})", **chunked}}


# ---------------------------------------------------------------------------
# CPU oracle baseline: one worker process per available core
# ---------------------------------------------------------------------------

_CPU_INPUTS = {}  # workload name -> synth.Inputs, set before the workers fork


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_worker(name, seqs, budget, sub, barrier, results):
    """Runs the fp64 oracle (closed form + commit) single-threaded over this
    worker's sequences, `sub` sequences per call, cycling until `budget`
    seconds of compute have run (at least one call).  The widening of each
    call's inputs to fp64 is not timed."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import treewy_oracle as orc
    inp = _CPU_INPUTS[name]
    H, N = inp.H, inp.N
    done = calls = 0
    elapsed = 0.0
    with threadpool_limits(limits=1):
        barrier.wait()
        while elapsed < budget or calls == 0:
            i0 = (calls * sub) % len(seqs)
            bs = seqs[i0:i0 + sub]
            G = len(bs) * H
            S0 = inp.S0[bs].reshape(G, 128, 128).astype(np.float64)
            tok = lambda x: np.ascontiguousarray(x[bs].transpose(0, 2, 1, 3)).reshape(G, N, 128).astype(np.float64)
            gate = lambda x: np.ascontiguousarray(x[bs].transpose(0, 2, 1)).reshape(G, N).astype(np.float64)
            q, k, v = tok(inp.q), tok(inp.k), tok(inp.v)
            a, bt = gate(inp.alpha), gate(inp.beta)
            acc = np.repeat(inp.accepted[bs], H)
            t0 = time.perf_counter()
            cf = orc.closed_form(S0, q, k, v, a, bt, inp.parent)
            orc.commit(S0, cf.vtilde, k, cf.gamma, inp.parent, acc)
            elapsed += time.perf_counter() - t0
            done += len(bs) * N  # verified nodes: one per (sequence, node), all heads
            calls += 1
    results.put((done, elapsed, calls))


def cpu_baseline(name, budget_s: float):
    """The fp64 oracle over the workload's batch on every core available to this
    process: one single-threaded worker per core (BLAS limited to one thread in
    each, so the thread count equals the core count), each on its own share of
    the sequences.  value = total nodes / the longest worker's compute time.
    Must run before anything initialises the GPU (the workers are forked)."""
    import multiprocessing as mp

    import numpy as np
    inp = _CPU_INPUTS[name]
    B, H, N = inp.B, inp.H, inp.N
    cores = len(os.sched_getaffinity(0))
    P = max(1, min(cores, B))
    shares = [s for s in np.array_split(np.arange(B), P) if len(s)]
    sub = max(1, 600 // N)  # sequences per call: ~0.5 s of fp64 oracle work
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(len(shares))
    results = ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker, args=(name, s, budget_s, sub, barrier, results))
             for s in shares]
    for p in procs:
        p.start()
    # (a worker that dies never reports: give up after a generous limit)
    got = [results.get(timeout=10 * budget_s + 300) for _ in procs]
    for p in procs:
        p.join()
    if any(p.exitcode != 0 for p in procs):
        raise RuntimeError("a CPU oracle worker failed")
    nodes = sum(g[0] for g in got)
    wall = max(g[1] for g in got)
    calls = sum(g[2] for g in got)
    return dict(value=round(nodes / wall, 1), unit="nodes/s", cores=len(shares), kind="oracle",
                sample=f"{nodes // N} sequences x {H} heads x {N} nodes "
                       f"({nodes / (B * N):.3g} passes over the batch of {B}), fp64 "
                       f"closed form + commit, {calls} calls over {len(shares)} single-threaded "
                       f"worker processes (one per available core, BLAS 1 thread each), "
                       f"longest worker {wall:.1f} s of compute ({cpu_model()})")


# ---------------------------------------------------------------------------
# GPU legs of one workload
# ---------------------------------------------------------------------------

def gpu_workload(inp, cfg, K, W, args, dev, stream):
    """Times every form of the step on one workload; returns its JSON block
    (without the CPU baseline)."""
    import numpy as np
    import torch

    from gated_deltanet_tree_03_amd import abi, accounting, profiling, synth

    B, H, N = inp.B, inp.H, inp.N
    ib = 2 if inp.dtype == "bf16" else 4
    dcode = abi.TREEWY_BF16 if inp.dtype == "bf16" else abi.TREEWY_F32
    depths = synth.node_depths(inp.parent)
    model = byte_model(B, H, N, ib, depths[inp.accepted])

    def upload():
        d = {"S0": torch.from_numpy(inp.S0).to(dev)}
        for name in ("q", "k", "v", "alpha", "beta"):
            if inp.dtype == "bf16":
                d[name] = torch.from_numpy(inp.bits[name].view(np.int16)).to(dev).view(torch.bfloat16)
            else:
                d[name] = torch.from_numpy(getattr(inp, name)).to(dev)
        d["accepted"] = torch.from_numpy(inp.accepted.astype(np.int32)).to(dev)
        return d

    base = upload()
    s0_bytes = B * H * 65536
    R = max(2, math.ceil(2 * 2 ** 30 / s0_bytes))
    sets = []
    for r in range(R):
        d = {k: (v if r == 0 else v.clone()) for k, v in base.items()}
        d["out"] = torch.empty((B, N, H, 128), dtype=torch.float32, device=dev)
        d["vt"] = [torch.empty((B, H, N, 128), dtype=torch.float32, device=dev) for _ in range(2)]
        d["gm"] = [torch.empty((B, H, N), dtype=torch.float32, device=dev) for _ in range(2)]
        d["S_out"] = torch.empty((B, H, 128, 128), dtype=torch.float32, device=dev)
        if inp.dtype == "bf16":
            d["S16"] = torch.empty((B, H, 128, 128), dtype=torch.bfloat16, device=dev)
        sets.append(d)
    # the state pool of the pool paths: R*B slots, each set's sequences on a
    # random slot subset.  Every buffer is allocated here, before anything is
    # timed: a state buffer allocated between timed paths has measured several
    # times slower on some runs, whichever path it served.
    n_slots = R * B
    pool = torch.empty((n_slots, H, 128, 128), dtype=torch.float32, device=dev)
    pool16 = (torch.empty((n_slots, H, 128, 128), dtype=torch.bfloat16, device=dev)
              if inp.dtype == "bf16" else None)
    perm = torch.from_numpy(np.random.default_rng(12345).permutation(n_slots).astype(np.int32))
    for r, d in enumerate(sets):
        d["slots"] = perm[r * B:(r + 1) * B].to(dev)
    torch.cuda.synchronize()
    parent = inp.parent

    def timed(step, names):
        """W untimed steps, then K timed ones, bracketed by synchronize.
        Returns (ms per step, {kernel: (ms per launch, min ms or None)}), GPU
        time from HIP events on the launch stream.
        - One kernel per step: two events span the K back-to-back launches, and
          the kernel's average duration is that span / K (its own time plus
          the gap between launches).  Every launch is a pre-bound call, so the
          host enqueues all K within about a millisecond, far ahead of the
          GPU.  (With the arguments converted per call, the host took about as
          long per launch as the shortest kernels, and a host hiccup then
          showed up as GPU idle time.)  Events inside the loop cost GPU
          time of their own: one every 10 launches measured ~4% on the
          117 us (2,2,2)-tree kernel.
        - Several kernels per step: events around each kernel; the median over
          the K steps of each kernel's span (each event costs a few
          microseconds of stream time, so those figures are a bit
          pessimistic), and the step time is their sum."""
        for i in range(W):
            step(i, None)
        torch.cuda.synchronize()
        per = {}
        if len(names) == 1:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(K):
                step(W + i, None)
            e1.record(stream)
            torch.cuda.synchronize()
            per[names[0]] = (e0.elapsed_time(e1) / K, None)
            return per[names[0]][0], per
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(K)]
        for i in range(K):
            step(W + i, evs[i])
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            ts = [e[j].elapsed_time(e[j + 1]) for e in evs]
            per[n] = (float(np.median(ts)), float(np.min(ts)))
        return sum(v[0] for v in per.values()), per

    # Every launch below is a call bound once (abi.bind: arguments converted
    # ahead), one per (input set, buffer parity), so the host enqueues far
    # faster than the kernels run.
    bind = lambda name, *a: abi.bind(name, *a, stream=stream)

    def looped(calls, first):
        """Step function over calls[set][parity], continuing the step count
        from `first` (so that the pseudo-value buffer parity carries over)."""
        def step(i, evs):
            j = first + i
            if evs is not None:
                evs[0].record(stream)
            calls[j % R][(j // R) % 2]()
            if evs is not None:
                evs[1].record(stream)
        return step

    def prime(first):
        """Before a loop that starts at step `first`: verify each set's draft
        from its current state into the pseudo-value / gate buffers its first
        step of the loop will commit."""
        for r, d in enumerate(sets):
            j = first + (r - first) % R
            p = (j // R) % 2
            abi.treewy_verify(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], parent, B, H,
                              N, d["out"], d["vt"][p], d["gm"][p], dcode, stream)

    # fused serving loop (the headline form, timed first): each set's state is
    # committed in place for its previous step and the next draft is verified
    # from it; the pseudo-values and gates of consecutive steps alternate
    # between two buffers
    prime(0)
    fused_calls = [[bind("treewy_commit_verify", d["S0"], d["S0"], d["vt"][p], d["k"], d["gm"][p],
                         d["accepted"], parent, N, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                         parent, B, H, N, d["out"], d["vt"][1 - p], d["gm"][1 - p], dcode)
                    for p in (0, 1)] for d in sets]
    fus_ms, fus_k = timed(looped(fused_calls, 0), ["treewy_commit_verify"])
    step0 = W + K  # later loops continue the step count (pseudo-value buffer parity)

    # separate calls: verify, then commit of its accepted node into S_out
    # (the input state is not modified)
    sep_calls = [(bind("treewy_verify", d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                       parent, B, H, N, d["out"], d["vt"][0], d["gm"][0], dcode),
                  bind("treewy_commit", d["S0"], d["vt"][0], d["k"], d["gm"][0], d["accepted"],
                       parent, B, H, N, d["S_out"], dcode)) for d in sets]

    def step_separate(i, evs):
        ver, com = sep_calls[i % R]
        if evs is not None:
            evs[0].record(stream)
        ver()
        if evs is not None:
            evs[1].record(stream)
        com()
        if evs is not None:
            evs[2].record(stream)

    sep_ms, sep_k = timed(step_separate, ["treewy_verify", "treewy_commit"])

    # the same serving loop with the states in the slot-indexed pool (one
    # block per request)
    prime(step0)
    for d in sets:
        pool[d["slots"].long()] = d["S0"]
    pool_calls = [[bind("treewy_commit_verify_pool", pool, n_slots, d["slots"], d["vt"][p], d["k"],
                        d["gm"][p], d["accepted"], parent, N, d["q"], d["k"], d["v"], d["alpha"],
                        d["beta"], parent, B, H, N, d["out"], d["vt"][1 - p], d["gm"][1 - p],
                        dcode) for p in (0, 1)] for d in sets]
    pool_ms, pool_k = timed(looped(pool_calls, step0), ["treewy_commit_verify_pool"])

    # the pool loop with a tree per request (every request on this workload's
    # tree): what the per-request descriptors cost
    desc, _, depth = abi.pack_trees([parent] * B)
    desc = torch.from_numpy(desc.copy()).to(dev)
    step2 = step0 + W + K
    ptr_calls = [[bind("treewy_commit_verify_pool_trees", pool, n_slots, d["slots"], d["vt"][p],
                       d["k"], d["gm"][p], d["accepted"], desc, N, depth, d["q"], d["k"], d["v"],
                       d["alpha"], d["beta"], desc, N, depth, B, H, d["out"], d["vt"][1 - p],
                       d["gm"][1 - p], dcode) for p in (0, 1)] for d in sets]
    ptr_ms, ptr_k = timed(looped(ptr_calls, step2), ["treewy_commit_verify_pool_trees"])

    # the same serving loop with the state stored as bf16 (bf16 inputs only)
    s16_ms = s16_k = p16_ms = p16_k = t16_ms = t16_k = None
    if inp.dtype == "bf16":
        for d in sets:
            d["S16"].copy_(d["S0"])
        step1 = step2 + W + K
        s16_calls = [[bind("treewy_commit_verify_bf16state", d["S16"], d["S16"], d["vt"][p],
                           d["k"], d["gm"][p], d["accepted"], parent, N, d["q"], d["k"], d["v"],
                           d["alpha"], d["beta"], parent, B, H, N, d["out"], d["vt"][1 - p],
                           d["gm"][1 - p], dcode) for p in (0, 1)] for d in sets]
        s16_ms, s16_k = timed(looped(s16_calls, step1), ["treewy_commit_verify_bf16state"])
        # ... and in the slot-indexed bf16 pool, with the workload's tree and
        # with a descriptor per request
        step3 = step1 + W + K
        prime(step3)
        for d in sets:
            pool16[d["slots"].long()] = d["S0"].to(torch.bfloat16)
        p16_calls = [[bind("treewy_commit_verify_bf16state_pool", pool16, n_slots, d["slots"],
                           d["vt"][p], d["k"], d["gm"][p], d["accepted"], parent, N, d["q"], d["k"],
                           d["v"], d["alpha"], d["beta"], parent, B, H, N, d["out"],
                           d["vt"][1 - p], d["gm"][1 - p], dcode) for p in (0, 1)] for d in sets]
        p16_ms, p16_k = timed(looped(p16_calls, step3), ["treewy_commit_verify_bf16state_pool"])
        step4 = step3 + W + K
        t16_calls = [[bind("treewy_commit_verify_bf16state_pool_trees", pool16, n_slots,
                           d["slots"], d["vt"][p], d["k"], d["gm"][p], d["accepted"], desc, N,
                           depth, d["q"], d["k"], d["v"], d["alpha"], d["beta"], desc, N, depth, B,
                           H, d["out"], d["vt"][1 - p], d["gm"][1 - p], dcode) for p in (0, 1)]
                     for d in sets]
        t16_ms, t16_k = timed(looped(t16_calls, step4),
                              ["treewy_commit_verify_bf16state_pool_trees"])
    del pool, pool16, desc
    for d in sets:
        d.pop("S16", None)

    def kernel_entry(name, avg_min):
        avg, mn = avg_min
        gbps = model[name] / (avg * 1e-3) / 1e9
        return {"avg_us": round(avg * 1e3, 2), "min_us": None if mn is None else round(mn * 1e3, 2),
                "algorithmic_bytes": model[name], "GBps": round(gbps, 1),
                "frac": round(gbps / HBM_PEAK_GBPS, 4)}

    def path_entry(ms, per):
        step_bytes = sum(model[k] for k in per)
        gbps = step_bytes / (ms * 1e-3) / 1e9
        return {"value": round(B * N / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
                "step_bytes": step_bytes, "hbm_GBps": round(gbps, 1),
                "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                "kernels": {k: kernel_entry(k, v) for k, v in per.items()}}

    paths = {"fused": path_entry(fus_ms, fus_k), "separate": path_entry(sep_ms, sep_k),
             "fused_pool": path_entry(pool_ms, pool_k),
             "fused_pool_trees": path_entry(ptr_ms, ptr_k)}
    if s16_ms is not None:
        paths["fused_bf16_state"] = path_entry(s16_ms, s16_k)
        paths["fused_bf16_state_pool"] = path_entry(p16_ms, p16_k)
        paths["fused_bf16_state_pool_trees"] = path_entry(t16_ms, t16_k)
    head_ms, head_k = (fus_ms, fus_k) if args.mode == "fused" else (sep_ms, sep_k)
    head = paths[args.mode]
    dom = max(head_k, key=lambda k: head_k[k][0])
    dom_avg = head_k[dom][0]
    achieved = model[dom] / (dom_avg * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": profiling.read_traffic(dom, cfg.name),
                "algorithmic_bytes_per_launch": model[dom], "avg_launch_us": round(dom_avg * 1e3, 2)}
    block = {
        "workload": f"{cfg.name}: {cfg.description}, d_k=d_v=128",
        "B": B, "H": H, "N": N, "tree_widths": list(cfg.widths), "input_dtype": inp.dtype,
        "state_dtype": "f32",
        "path": ("treewy_commit_verify (commit of the previous step fused into the verify)"
                 if args.mode == "fused" else "treewy_verify + treewy_commit"),
        "rotating_input_sets": R,
        "value": head["value"], "unit": "nodes/s", "ms_per_step": head["ms_per_step"],
        "draft_nodes_per_s": round(B * (N - 1) / (head_ms * 1e-3), 1),
        "hbm_GBps": head["hbm_GBps"], "hbm_frac": head["hbm_frac"],
        "roofline": roofline, "paths": paths,
        "resident_state_blocks": {"treewy": accounting.treewy_state_blocks(N),
                                  "store_all_buffer": accounting.store_all_buffer_blocks(N),
                                  "store_all_pages_count": accounting.snapshot_blocks_per_request(N)},
        "transient_vtilde_bytes_per_head": accounting.pseudo_value_bytes(N),
    }

    if not args.no_store_all:
        d = sets[0]
        snaps = torch.empty((B, H, N + 1, 128, 128), dtype=torch.float32, device=dev)
        sa_out = torch.empty((B, N, H, 128), dtype=torch.float32, device=dev)
        S_sel = torch.empty((B, H, 128, 128), dtype=torch.float32, device=dev)
        sK = max(5, K // 4)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(sK)]
        for i in range(2 + sK):
            e = sev[i - 2] if i >= 2 else None
            if e is not None:
                e[0].record(stream)
            abi.treewy_store_all(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], parent,
                                 B, H, N, sa_out, snaps, dcode, stream)
            if e is not None:
                e[1].record(stream)
            abi.treewy_store_all_select(snaps, d["accepted"], B, H, N, S_sel, stream)
            if e is not None:
                e[2].record(stream)
        torch.cuda.synchronize()
        sa_ms = float(np.median([e[0].elapsed_time(e[1]) for e in sev]))
        sel_ms = float(np.median([e[1].elapsed_time(e[2]) for e in sev]))
        # the part's write ceiling on the same buffer: a plain device fill of
        # the whole snapshot buffer (torch's fill kernel), median of 3
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(4)]
        for e0, e1 in fev:
            e0.record(stream)
            snaps.fill_(0.0)
            e1.record(stream)
        torch.cuda.synchronize()
        fill_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in fev[1:]]))
        snap_bytes = B * H * (N + 1) * 65536
        sa_gbps = model["treewy_store_all"] / (sa_ms * 1e-3) / 1e9
        fill_gbps = snap_bytes / (fill_ms * 1e-3) / 1e9
        block["store_all"] = {
            "store_all_us": round(sa_ms * 1e3, 2), "select_us": round(sel_ms * 1e3, 2),
            "nodes_per_s": round(B * N / ((sa_ms + sel_ms) * 1e-3), 1),
            "snapshot_bytes": snap_bytes,
            "algorithmic_bytes": model["treewy_store_all"],
            "GBps": round(sa_gbps, 1), "frac": round(sa_gbps / HBM_PEAK_GBPS, 4),
            "traffic": profiling.read_traffic("treewy_store_all", cfg.name),
            "write_ceiling": {"kernel": "torch fill_ of the snapshot buffer",
                              "bytes": snap_bytes, "us": round(fill_ms * 1e3, 2),
                              "GBps": round(fill_gbps, 1)},
            "snapshot_write_GBps": round(snap_bytes / (sa_ms * 1e-3) / 1e9, 1),
            "snapshot_write_frac_of_ceiling": round(snap_bytes / (sa_ms * 1e-3) / 1e9 / fill_gbps, 4),
            "resident_blocks_per_head": N + 1,
            "treewy_speedup": round((sa_ms + sel_ms) / head_ms, 3),
        }
        del snaps, sa_out, S_sel
    del sets, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return block


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=HEADLINE, choices=WORKLOADS,
                    help="the headline workload (default: the wide (3,3,3) tree)")
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload alone (no other workloads)")
    ap.add_argument("--mode", default="fused", choices=["fused", "separate"],
                    help="which path gives the headline figures (both are timed)")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle compute per worker, headline workload")
    ap.add_argument("--cpu-budget-other", type=float, default=3.0,
                    help="seconds of oracle compute per worker, each other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-store-all", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy, three times (the "
                         "reference that scales the HBM byte counters), and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: only one GPU is measured here (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); every (sequence, head) is independent, so the path "
              f"shards with no exchange and the per-GPU figure is the 1-GPU figure.",
              file=sys.stderr)
        sys.exit(2)

    names = [args.config] + ([] if args.only else [w for w in WORKLOADS if w != args.config])
    inputs = {}
    cpu = {}
    if not args.calibrate_copy:
        from gated_deltanet_tree_03_amd import synth
        for n in names:
            inputs[n] = synth.make_inputs(synth.CONFIGS[n])
            print(f"bench: inputs of {n} drawn", file=sys.stderr, flush=True)
        # the CPU oracle runs before anything touches the GPU: its workers are
        # forked from this process
        if not args.no_cpu_baseline:
            _CPU_INPUTS.update(inputs)
            for n in names:
                cpu[n] = cpu_baseline(n, args.cpu_budget if n == args.config else args.cpu_budget_other)
                print(f"bench: CPU oracle on {n}: {cpu[n]['value']:.4g} nodes/s on "
                      f"{cpu[n]['cores']} cores", file=sys.stderr, flush=True)
            _CPU_INPUTS.clear()

    import numpy as np  # noqa: F401
    import torch

    from gated_deltanet_tree_03_amd import abi, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    abi.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
        n = 2 ** 28  # 1 GiB of fp32: 1 GiB read + 1 GiB written per copy
        src = torch.empty(n, dtype=torch.float32, device=dev)
        src.fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes_read": n * 4, "calibration_copy_bytes_written": n * 4,
                          "copies": 3}), flush=True)
        return

    K, W = args.steps, args.warmup
    blocks = {}
    for n in names:
        blocks[n] = gpu_workload(inputs[n], synth.CONFIGS[n], K, W, args, dev, stream)
        blocks[n]["cpu_baseline"] = cpu.get(n)
        inputs[n] = None
        print(f"bench: {n}: {blocks[n]['value']:.4g} nodes/s, "
              f"{blocks[n]['roofline']['frac']:.3f} of HBM peak", file=sys.stderr, flush=True)

    hb = blocks[args.config]
    result = {
        "metric": METRIC,
        "value": hb["value"],
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": hb["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {k: hb[k] for k in ("workload", "B", "H", "N", "tree_widths", "input_dtype",
                                      "state_dtype", "path", "rotating_input_sets")},
        "draft_nodes_per_s": hb["draft_nodes_per_s"],
        "hbm_GBps": hb["hbm_GBps"],
        "hbm_frac": hb["hbm_frac"],
        "kernels": hb["paths"][args.mode]["kernels"],
        "roofline": hb["roofline"],
        "cpu_baseline": hb["cpu_baseline"],
        "paths": hb["paths"],
        "store_all": hb.get("store_all"),
        "resident_state_blocks": hb["resident_state_blocks"],
        "transient_vtilde_bytes_per_head": hb["transient_vtilde_bytes_per_head"],
        "workloads": {n: blocks[n] for n in names if n != args.config},
    }
    if not args.no_prefill:
        result["prefill"] = prefill_bench(dev, hb["H"])

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
