#!/usr/bin/env python3
"""Benchmark of paged GQA decode attention on one MI355X (gfx950).

One *step* is one decode step of the whole batch through every layer of the
workload: one libkvdecode decode call per layer, each streaming that layer's
cached K/V once.  The headline workload is the Llama-3.1-8B-shaped single
layer (b = 1, 32 query / 8 KV heads, head dim 128, s = 32,768); the
Llama-3-70B-shaped long-context step (b = 4, 80 layers, s = 131,072, about
172 GB of resident KV) is reported beside it, and the ragged 8B batch, the
FP8 + fused-score batch, a context shard of the 70B step, a shared-prefix
batch and a 256-request serving batch as further entries of the same line.

Reported:
* value       -- algorithmic KV GB/s of the whole step (bytes the method must
                 move, see ``algorithmic_step_bytes``) over wall time of
                 exactly K steps bracketed by device synchronisation;
* seq-steps/s -- sequences x steps per second; % of the 8 TB/s HBM peak;
* roofline    -- the decode kernel alone: algorithmic bytes per launch over
                 its mean duration, from a HIP event pair around a run of
                 back-to-back launches of it;
* cpu_baseline-- the float64 oracle timed on a bounded sample on the host;
* hbm_context -- context for the roofline: a plain streaming read of the
                 headline launch's bytes with the decode kernels' own loads
                 (the practical ceiling of a launch that size), and torch's
                 copy and sum rates over 1 GiB.

Timing details: inputs are resident in HBM before the timed region; the step
sequence is captured in HIP graphs (one launch per layer call) and replayed,
so host launch overhead does not pace the ~20 us single-layer step; when one
step's bytes would fit the 256 MB Infinity Cache, several replicas of the
pool are stepped through in turn so that every step reads from HBM.
"""
from __future__ import annotations

import argparse
import ctypes

import numpy as np
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s (% of HBM peak) + seq-steps/s, 8B & 70B GQA shapes"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
INFINITY_CACHE_BYTES = 256 << 20
HEADLINE = "8b_layer"
SECONDARY = "70b_long"
DECODE_SOURCES = ["decode.hip", "device_common.h", "kv_store.h", "kvd_internal.h"]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_step_bytes(lens, layers, n_q, n_kv, head_dim, kv_bytes, fp8, scores) -> int:
    """Bytes one step must move (per layer: every cached K/V element once, q in
    and the bf16 output out, one 4-byte block id per block, two fp32 scales per
    (block, KV head) for FP8; a score update reads and writes 4 bytes per token
    once per step).  Implementation scratch (partials, score scratch) and the
    unused rows of a partly filled last block are not counted."""
    total = 0
    for s in lens:
        s = int(s)
        nblk = -(-s // 16)
        per_layer = 2 * n_kv * head_dim * kv_bytes * s + 2 * n_q * head_dim * 2 + 4 * nblk
        if fp8:
            per_layer += 2 * n_kv * 4 * nblk
        total += layers * per_layer + (8 * s if scores else 0)
    return total


class Workload:
    """A workload resident in HBM, ready to be stepped (eagerly or from graphs)."""

    def __init__(self, name: str, chunk: int, replicas: int, layers: int = 0):
        import torch
        import decode_attention_paged_04_amd as kvd
        import workloads as W

        self.kvd, self.torch = kvd, torch
        self.w = w = W.WORKLOADS[name] if not layers else W.WORKLOADS[name].with_(layers=layers)
        self.fp8 = w.kv_dtype == "fp8"
        self.lens = W.context_lengths(w)
        self.table, self.num_blocks = W.block_tables(w, self.lens)
        self.max_ctx = int(self.lens.max())
        self.kv_bytes = 1 if self.fp8 else 2
        self.step_bytes = algorithmic_step_bytes(self.lens, w.layers, w.n_q, w.n_kv, w.head_dim,
                                                 self.kv_bytes, self.fp8, w.scores)
        self.launch_bytes = algorithmic_step_bytes(self.lens, 1, w.n_q, w.n_kv, w.head_dim,
                                                   self.kv_bytes, self.fp8, False)
        if replicas <= 0:
            replicas = max(1, math.ceil(4 * INFINITY_CACHE_BYTES / self.step_bytes))
        self.R = replicas
        dev = "cuda"
        self.lens_t = torch.from_numpy(self.lens).to(dev)
        self.table_t = torch.from_numpy(self.table).to(dev)
        # a shared prefix is stored once, by sequence 0: rows are generated for the stored tokens only
        first, _, n_tok = W.stored_rows(w, self.lens)
        slots = kvd.kvd_slot_mapping(self.table_t, self.lens_t, first_token=torch.from_numpy(first).to(dev))
        self.unique_step_bytes = self.step_bytes - w.layers * (w.b - 1) * w.shared_prefix * (
            2 * w.n_kv * w.head_dim * self.kv_bytes)
        dt = kvd.KVD_FP8_E4M3 if self.fp8 else kvd.KVD_BF16
        t0 = time.time()
        self.pools = [kvd.allocate_pool(w.layers, self.num_blocks, w.n_kv, w.head_dim, dt)
                      for _ in range(self.R)]
        self.q = []
        for layer in range(w.layers):
            K, V = W.keys_values(w, layer, n_tok, dev)
            for p in self.pools:
                kvd.kvd_write_kv(p, layer, K, V, slots)
            self.q.append(W.query(w, layer, dev))
            del K, V
        torch.cuda.synchronize()
        log(f"{w.name}: {self.R} pool(s) of {self.pools[0].kv.numel() / 1e9:.2f} GB filled in "
            f"{time.time() - t0:.1f}s")
        self.out = [torch.empty_like(q) for q in self.q]
        self.score = None
        if w.scores:
            self.score0 = W.initial_scores(w, self.max_ctx, dev)
            self.score = self.score0.clone()
        # a batch behind one shared prompt reads it mostly from the L2: even chunks
        # (KVD_FLAG_EVEN_CHUNKS), as a caller that knows of the sharing would ask for
        self.even = w.shared_prefix > 0
        self.chunk_arg = chunk
        probe = kvd.make_args(self.q[0], self.table_t, self.lens_t, self.max_ctx, self.out[0],
                              chunk_tokens=chunk, score=self.score,
                              score_weight=1.0 / w.layers, pool=self.pools[0], even_chunks=self.even)
        self.chunk, self.n_chunks = kvd.kvd_decode_plan(self.pools[0], probe)
        ws_bytes = kvd.kvd_decode_workspace_bytes(self.pools[0], probe)
        self.ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.args = [[kvd.make_args(self.q[l], self.table_t, self.lens_t, self.max_ctx, self.out[l],
                                    chunk_tokens=chunk, workspace=self.ws, score=self.score,
                                    score_weight=1.0 / w.layers, pool=self.pools[r], even_chunks=self.even)
                      for l in range(w.layers)] for r in range(self.R)]
        self.fn = kvd.lib.kvd_decode_attn_fp8 if self.fp8 else kvd.lib.kvd_decode_attn
        # the decode kernel on its own: per-chunk partials into separate buffers
        b, n_q, d = w.b, w.n_q, w.head_dim
        self.part_o = torch.empty((b, n_q, self.n_chunks, d), dtype=torch.float32, device=dev)
        self.part_lse = torch.empty((b, n_q, self.n_chunks), dtype=torch.float32, device=dev)
        self.pargs = [[kvd.make_args(self.q[l], self.table_t, self.lens_t, self.max_ctx, None,
                                     chunk_tokens=chunk, pool=self.pools[r], need_out=False,
                                     even_chunks=self.even)
                       for l in range(w.layers)] for r in range(self.R)]

    def call(self, r: int, layer: int, stream: int):
        st = self.fn(self.pools[r].handle, layer, ctypes.byref(self.args[r][layer]), stream)
        if st != 0:
            raise RuntimeError(f"decode call failed: {self.kvd.kvd_status_string(st)}")

    def call_partials(self, r: int, layer: int, stream: int):
        st = self.kvd.lib.kvd_decode_partials(self.pools[r].handle, layer, ctypes.byref(self.pargs[r][layer]),
                                              self.part_o.data_ptr(), self.part_lse.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"partials call failed: {self.kvd.kvd_status_string(st)}")

    def step(self, r: int):
        stream = int(self.torch.cuda.current_stream().cuda_stream)
        for layer in range(self.w.layers):
            self.call(r, layer, stream)

    def capture(self):
        """One graph per replica (one step each) and one graph stepping all replicas."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in range(self.R):
                self.step(r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.single = []
        for r in range(self.R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(r)
            self.single.append(g)
        self.all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.all):
            for r in range(self.R):
                self.step(r)
        torch.cuda.synchronize()

    def run_steps(self, k: int):
        """Exactly k steps: full rotations from one graph, the rest one by one."""
        full, rest = divmod(k, self.R)
        for _ in range(full):
            self.all.replay()
        for r in range(rest):
            self.single[r].replay()

    def time_steps(self, steps: int, warmup: int) -> float:
        torch = self.torch
        self.run_steps(warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.run_steps(steps)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def time_launches(self, n: int) -> float:
        """Mean duration (s) of the decode kernel: n back-to-back launches of it
        (kvd_decode_partials calls, each exactly one launch), cycling through
        replicas and layers, between one HIP event pair on their stream."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        h = int(stream.cuda_stream)
        for k in range(min(n, 8)):                       # warm
            self.call_partials(k % self.R, (k // self.R) % self.w.layers, h)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for k in range(n):
            self.call_partials(k % self.R, (k // self.R) % self.w.layers, h)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n / 1e3

    def restrict(self, seed: int, t0_frac: float, t1_frac: float):
        """Restrict every layer's decode to the T0 and T1 tiers of a plan made
        from seeded block scores (first block and last two protected); the
        algorithmic bytes become those of the kept blocks."""
        kvd, torch, w = self.kvd, self.torch, self.w
        rng = np.random.default_rng(seed)
        table = self.table.copy()
        kept_tokens = []
        for i, s in enumerate(self.lens):
            nb = -(-int(s) // 16)
            plan = kvd.tier_plan(rng.random(nb), 1, 2, int(nb * t0_frac), int(nb * t1_frac))
            table[i, :nb] = kvd.tier_restrict(self.table[i, :nb], plan)
            kept = sum(min(16, int(s) - 16 * b) for b in range(nb) if plan[b] != kvd.KVD_TIER_T3)
            kept_tokens.append(kept)
        self.kept_fraction = sum(kept_tokens) / float(self.lens.sum())
        self.table_t = torch.from_numpy(table).cuda()
        per_tok = 2 * w.n_kv * w.head_dim * self.kv_bytes
        ids = sum(-(-int(s) // 16) for s in self.lens)
        self.launch_bytes = (per_tok * sum(kept_tokens) + w.b * 2 * w.n_q * w.head_dim * 2 + 4 * ids
                             + (2 * w.n_kv * 4 * sum(-(-k // 16) for k in kept_tokens) if self.fp8 else 0))
        self.step_bytes = w.layers * self.launch_bytes
        self.args = [[kvd.make_args(self.q[l], self.table_t, self.lens_t, self.max_ctx, self.out[l],
                                    chunk_tokens=self.chunk_arg, workspace=self.ws, pool=self.pools[r],
                                    even_chunks=self.even)
                      for l in range(w.layers)] for r in range(self.R)]
        self.pargs = [[kvd.make_args(self.q[l], self.table_t, self.lens_t, self.max_ctx, None,
                                     chunk_tokens=self.chunk_arg, pool=self.pools[r], need_out=False,
                                     even_chunks=self.even)
                       for l in range(w.layers)] for r in range(self.R)]

    def time_append(self, n: int):
        """Mean duration (s) of one kvd_write_kv call storing one token per
        sequence -- what a decode step writes per layer -- into each
        sequence's last block (a partly filled block re-quantises under FP8):
        (eager calls from Python, calls replayed from a HIP graph, the decode
        call alone and the decode call with the append fused, both replayed
        from graphs)."""
        torch, kvd, w = self.torch, self.kvd, self.w
        slots = kvd.kvd_slot_mapping(self.table_t, self.lens_t, first_token=self.lens_t - 1)
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed)
        K = torch.randn((w.b, w.n_kv, w.head_dim), generator=g, device="cuda").to(torch.bfloat16)
        V = torch.randn((w.b, w.n_kv, w.head_dim), generator=g, device="cuda").to(torch.bfloat16)
        stream = torch.cuda.current_stream()
        for k in range(4):
            kvd.kvd_write_kv(self.pools[0], k % w.layers, K, V, slots)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for k in range(n):
            kvd.kvd_write_kv(self.pools[0], k % w.layers, K, V, slots)
        b.record(stream)
        torch.cuda.synchronize()
        eager = a.elapsed_time(b) / n / 1e3
        per_graph = 16
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            kvd.kvd_write_kv(self.pools[0], 0, K, V, slots)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(per_graph):
                kvd.kvd_write_kv(self.pools[0], k % w.layers, K, V, slots)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, n // per_graph)
        a.record(stream)
        for _ in range(reps):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        graphed = a.elapsed_time(b) / (reps * per_graph) / 1e3

        # the same appends fused into the decode calls (kvd_decode_attn_append),
        # against the decode calls alone, both replayed from graphs
        args = self.args[0][0]

        def here():                           # the stream being captured, or the current one
            return int(torch.cuda.current_stream().cuda_stream)

        def decode_only():
            self.call(0, 0, here())

        def fused():
            st = kvd.lib.kvd_decode_attn_append(self.pools[0].handle, 0, ctypes.byref(args), K.data_ptr(),
                                                V.data_ptr(), here())
            if st != 0:
                raise RuntimeError(f"fused append failed: {kvd.kvd_status_string(st)}")

        per_call = {}
        for name, fn in (("decode", decode_only), ("fused", fused)):
            fn()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(per_graph):
                    fn()
            gr.replay()
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(reps):
                gr.replay()
            b.record(stream)
            torch.cuda.synchronize()
            per_call[name] = a.elapsed_time(b) / (reps * per_graph) / 1e3
        return eager, graphed, per_call["decode"], per_call["fused"]

    def config(self):
        w = self.w
        ctx = (str(int(w.ctx[1])) if w.ctx[0] == "fixed"
               else f"U[{w.ctx[1]},{w.ctx[2]}] (sum {int(self.lens.sum())})")
        return {"workload": w.name, "b": w.b, "layers": w.layers, "n_q": w.n_q, "n_kv": w.n_kv,
                "head_dim": w.head_dim, "context": ctx, "block_size": 16,
                "kv_dtype": w.kv_dtype, "fused_scores": bool(w.scores), "shared_prefix": w.shared_prefix,
                "chunk_tokens": self.chunk, "n_chunks": self.n_chunks, "even_chunks": self.even,
                "pool_replicas": self.R,
                "num_blocks": self.num_blocks, "hip_graphs": True}

    def free(self):
        torch = self.torch
        del self.pools, self.args, self.pargs, self.q, self.out, self.ws, self.part_o, self.part_lse
        if hasattr(self, "single"):
            del self.single, self.all
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def source_digest() -> str:
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_paged_04_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current decode kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_kernel_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"decode kernel source digest:\s*`?([0-9a-f]+)", txt)
    m_b = re.search(r"HBM bytes per launch \(calibrated\):\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != source_digest():
        return None
    return float(m_b.group(1))


def host_threads():
    """(os.cpu_count(), CPUs in this process's affinity mask, BLAS threads)."""
    aff = len(os.sched_getaffinity(0))
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [0]) or None
    except Exception:
        pass
    return os.cpu_count(), aff, blas


def measured_l2(workload: str):
    """L2 hit rate and L2 read requests per launch from the committed rocprofv3
    counter summary of a workload, if it was taken on the current decode kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_kernel_{workload}_l2_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"decode kernel source digest:\s*`?([0-9a-f]+)", txt)
    m_hit = re.search(r"L2 hit rate:\s*([0-9.]+)", txt)
    m_rd = re.search(r"L2 read bytes per launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_hit or m_src.group(1) != source_digest():
        return None
    return {"hit_rate": float(m_hit.group(1)), "read_bytes_per_launch": float(m_rd.group(1)) if m_rd else None}


def cpu_baseline(w, lens, budget_s: float):
    """The float64 oracle as it stands, timed on the host on a bounded sample of
    the workload: every sequence of the first layer and of the last layer (the
    one layer of a one-layer workload, repeated), sequence by sequence until each
    layer's share of the budget is spent; FP8 pools time the decoding of the
    stored codes too, a fused score the score increment.  The rate is the
    algorithmic bytes of the sampled (layer, sequence) units over their time;
    seq-steps/s extrapolates the sampled layers' time per byte to the whole step.
    BLAS threads are set to the CPUs of this process's affinity mask."""
    import numpy as np
    import torch
    import workloads as W
    from oracle import attention, e4m3, scores
    from threadpoolctl import threadpool_limits

    def fp8_codes(x):
        """E4M3 codes [s][n_kv][d] (uint8) and per-(block, KV head) scales of a
        bf16 sequence -- input for timing the oracle's decoding, made with
        torch's cast (quicker than the oracle's own quantiser)."""
        s_, n_kv, d = x.shape
        nb = -(-s_ // 16)
        t = torch.zeros((nb * 16, n_kv, d), dtype=torch.float32)
        t[:s_] = x.float()
        t = t.view(nb, 16, n_kv, d)
        sc = t.abs().amax(dim=(1, 3)) / 448.0
        y = (t / torch.where(sc == 0, torch.ones_like(sc), sc)[:, None, :, None]).clamp(-448, 448)
        codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(nb * 16, n_kv, d)[:s_]
        return codes.numpy(), sc.numpy()

    fp8 = w.kv_dtype == "fp8"
    kvb = 1 if fp8 else 2
    cpu_count, aff, _ = host_threads()
    sample_layers = [0] if w.layers == 1 else [0, w.layers - 1]
    per_layer_budget = budget_s / len(sample_layers)
    _, start, n_tok = W.stored_rows(w, lens)
    P = w.shared_prefix
    done_bytes, secs, units, reps_total = 0, 0.0, 0, 0
    layer_bytes = algorithmic_step_bytes(lens, 1, w.n_q, w.n_kv, w.head_dim, kvb, fp8, False)
    with threadpool_limits(limits=aff):
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [0]) or None
        dev = "cuda" if torch.cuda.is_available() else "cpu"
        for layer in sample_layers:
            K, V = W.keys_values(w, layer, n_tok, dev)
            Kc, Vc = K.cpu(), V.cpu()
            del K, V
            qf = W.query(w, layer, dev).cpu().to(torch.float64).numpy()
            spent = 0.0
            for i, s in enumerate(lens):
                a = int(start[i])
                if P and i:                         # the shared prompt is stored once, by sequence 0
                    e = a + int(s) - P
                    Ki, Vi = torch.cat([Kc[:P], Kc[a:e]]), torch.cat([Vc[:P], Vc[a:e]])
                else:
                    Ki, Vi = Kc[a:a + int(s)], Vc[a:a + int(s)]
                # inputs in the oracle's form (bf16 -> float64 is exact); not timed
                Kf, Vf = Ki.to(torch.float64).numpy(), Vi.to(torch.float64).numpy()
                if fp8:                             # stored codes and scales of the sequence
                    ck, sk = fp8_codes(Ki)
                    cv, sv = fp8_codes(Vi)
                reps, t0 = 0, time.perf_counter()
                while True:
                    if fp8:
                        Kd, Vd = e4m3.dequantize_sequence(ck, sk), e4m3.dequantize_sequence(cv, sv)
                    else:
                        Kd, Vd = Kf, Vf
                    attention.decode_sequence(qf[i], Kd, Vd)
                    if w.scores and int(s):
                        scores.layer_increment(attention.attention_weights_sequence(qf[i], Kd), 1.0 / w.layers)
                    reps += 1
                    # a one-sequence layer is repeated to fill its budget
                    if len(lens) > 1 or time.perf_counter() - t0 >= per_layer_budget:
                        break
                dt = time.perf_counter() - t0
                secs += dt
                spent += dt
                units += 1
                reps_total += reps
                done_bytes += reps * algorithmic_step_bytes([s], 1, w.n_q, w.n_kv, w.head_dim, kvb, fp8, False)
                if spent >= per_layer_budget:
                    break
    rate = done_bytes / secs                        # bytes per second of oracle time
    step_s = w.layers * layer_bytes / rate + (8 * int(np.sum(lens)) / rate if w.scores else 0.0)
    full = units * 1 >= len(lens) * len(sample_layers)
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": int(aff), "kind": "oracle",
            "os_cpu_count": cpu_count, "affinity_cpus": aff, "blas_threads": blas,
            "sample": (f"float64 numpy oracle (decode{' + FP8 decoding' if fp8 else ''}"
                       f"{' + score increment' if w.scores else ''}) on {units} (layer, sequence) units of "
                       f"layers {sample_layers} ({reps_total} calls, {secs:.1f} s)"
                       + ("" if full else ", the first sequences of each layer until its budget was spent")
                       + (f"; extrapolated to all {w.layers} layers" if w.layers > 1 else "")),
            "extrapolated": w.layers > 1 or not full,
            "seq_steps_per_s": round(len(lens) / step_s, 4)}


def measure(name: str, chunk: int, replicas: int, steps: int, warmup: int, launches: int):
    wl = Workload(name, chunk, replicas)
    wl.capture()
    secs = wl.time_steps(steps, warmup)
    ms = secs / steps * 1e3
    launch_s = wl.time_launches(launches)
    achieved = wl.launch_bytes / launch_s / 1e9
    value = wl.step_bytes / (secs / steps) / 1e9
    res = {"value": value, "ms_per_step": ms, "seq_steps_per_s": wl.w.b * steps / secs,
           "pct_of_hbm_peak": 100.0 * value / PEAK_HBM_GBS, "step_bytes": wl.step_bytes,
           "launch_bytes": wl.launch_bytes, "launch_us": launch_s * 1e6, "achieved": achieved,
           "config": wl.config()}
    log(f"{name}: {ms:.4f} ms/step, {value:.1f} GB/s ({res['pct_of_hbm_peak']:.1f}% of peak), "
        f"decode launch {launch_s * 1e6:.2f} us -> {achieved:.1f} GB/s")
    return wl, res


def extra_entry(name: str, steps: int, cpu_seconds: float = 0.0):
    """A further workload in the same line: step rate, kernel roofline, the
    oracle baseline and, for a shared prefix, the rates over the bytes actually
    stored (each shared block once).  A shared prefix's blocks are read by every
    request but fetched from HBM about once (the requests behind it read them
    together, from L2), so its roofline is taken over the unique stored bytes --
    what HBM has to deliver -- and the rate over every request's logical bytes
    is reported beside it."""
    wl, r = measure(name, 0, 0, steps, 2, 40)
    e = {"workload": r["config"]["workload"], "value": round(r["value"], 2), "unit": "GB/s",
         "ms_per_step": round(r["ms_per_step"], 4), "steps": steps,
         "seq_steps_per_s": round(r["seq_steps_per_s"], 3), "pct_of_hbm_peak": round(r["pct_of_hbm_peak"], 2),
         "config": r["config"],
         "roofline": {"bound": "hbm", "achieved": round(r["achieved"], 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(r["achieved"] / PEAK_HBM_GBS, 4), "traffic": measured_traffic(name),
                      "launch_us": round(r["launch_us"], 2)}}
    if wl.w.shared_prefix:
        unique_launch = wl.unique_step_bytes // wl.w.layers
        ach = unique_launch / (r["launch_us"] / 1e6) / 1e9
        e["unique_bytes_per_step"] = wl.unique_step_bytes
        e["unique_GBs"] = round(wl.unique_step_bytes / (r["ms_per_step"] / 1e3) / 1e9, 1)
        e["pct_of_hbm_peak"] = round(100.0 * e["unique_GBs"] / PEAK_HBM_GBS, 2)
        e["logical_GBs"] = e["value"]
        e["roofline"].update({"basis": "unique stored bytes (each shared block once)", "achieved": round(ach, 2),
                              "frac": round(ach / PEAK_HBM_GBS, 4), "bytes_per_launch": unique_launch,
                              "logical_GBs": round(r["achieved"], 2), "l2": measured_l2(name)})
    w, lens = wl.w, wl.lens
    wl.free()
    if cpu_seconds > 0:
        e["cpu_baseline"] = cpu_baseline(w, lens, cpu_seconds)
        log(f"{name} cpu baseline: {e['cpu_baseline']['value']} GB/s ({e['cpu_baseline']['sample']})")
    return e


def tiered_entry(name: str, layers: int, steps: int):
    """The same batch decoded in full and restricted to T0 + T1 (about half the
    blocks): the restricted step should cost about its kept bytes."""
    out = {}
    for label in ("full", "tiered"):
        wl = Workload(name, 0, 1, layers=layers)
        if label == "tiered":
            wl.restrict(seed=11, t0_frac=0.25, t1_frac=0.25)
        wl.capture()
        secs = wl.time_steps(steps, 2)
        launch_s = wl.time_launches(40)
        out[label] = {"ms_per_step": round(secs / steps * 1e3, 4),
                      "GBs": round(wl.step_bytes / (secs / steps) / 1e9, 1),
                      "launch_us": round(launch_s * 1e6, 2),
                      "launch_GBs": round(wl.launch_bytes / launch_s / 1e9, 1)}
        if label == "tiered":
            out[label]["kept_fraction"] = round(wl.kept_fraction, 4)
        log(f"{name} {label}: {out[label]}")
        wl.free()
    out["workload"] = f"{name} ({layers} layers), full vs restricted to T0+T1"
    return out


def mixed_entry(name: str, layers: int, steps: int, fp8_share: float = 0.5):
    """The batch with a seeded share of its blocks stored as FP8 (kvd_decode_attn_mixed):
    rate over the bytes the two pools actually hold for it."""
    import torch
    import decode_attention_paged_04_amd as kvd
    import workloads as W
    w = W.WORKLOADS[name].with_(layers=layers)
    lens = W.context_lengths(w)
    rng = np.random.default_rng(w.seed + 77)
    prec = [rng.random(-(-int(s) // 16)) < fp8_share for s in lens]
    n8 = int(sum(p.sum() for p in prec))
    n16 = int(sum(len(p) for p in prec)) - n8
    pools = {False: kvd.allocate_pool(layers, max(n16, 1), w.n_kv, w.head_dim, kvd.KVD_BF16),
             True: kvd.allocate_pool(layers, max(n8, 1), w.n_kv, w.head_dim, kvd.KVD_FP8_E4M3)}
    phys = {False: rng.permutation(max(n16, 1)), True: rng.permutation(max(n8, 1))}
    nxt = {False: 0, True: 0}
    ids = []                                    # per sequence: physical id of each logical block
    for p in prec:
        row = []
        for f8 in p:
            row.append(int(phys[bool(f8)][nxt[bool(f8)]]))
            nxt[bool(f8)] += 1
        ids.append(row)
    n_tok = int(lens.sum())
    # per pool, the logical block table of its own blocks (-1 elsewhere: slot -1, not stored)
    nbmax = max(len(p) for p in prec)
    lens_t = torch.from_numpy(lens).cuda()
    slot_t = {}
    for f8 in (False, True):
        tab = np.full((w.b, nbmax), -1, np.int32)
        for i, p in enumerate(prec):
            for b in range(len(p)):
                if bool(p[b]) == f8:
                    tab[i, b] = ids[i][b]
        slot_t[f8] = kvd.kvd_slot_mapping(torch.from_numpy(tab).cuda(), lens_t)
    qs = []
    for layer in range(layers):
        K, V = W.keys_values(w, layer, n_tok, "cuda")
        for f8 in (False, True):
            kvd.kvd_write_kv(pools[f8], layer, K, V, slot_t[f8])
        qs.append(W.query(w, layer, "cuda"))
        del K, V
    rows, ctx = [], []
    for i, s in enumerate(lens):
        nb = len(prec[i])
        r, c = kvd.mixed_row([ids[i][b] for b in range(nb) if not prec[i][b]],
                             [ids[i][b] for b in range(nb) if prec[i][b]],
                             bool(prec[i][nb - 1]), int(s) - 16 * (nb - 1))
        rows.append(r)
        ctx.append(c)
    mb = max(len(r) for r in rows)
    table = np.full((w.b, mb), -1, np.int32)
    for i, r in enumerate(rows):
        table[i, :len(r)] = r
    table_t = torch.from_numpy(table).cuda()
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    outs = [torch.empty_like(q) for q in qs]
    probe = kvd.make_args(qs[0], table_t, ctx_t, max(ctx), outs[0], pool=pools[False])
    ws = kvd.allocate_workspace(pools[False], probe)
    args = [kvd.make_args(qs[l], table_t, ctx_t, max(ctx), outs[l], workspace=ws, pool=pools[False])
            for l in range(layers)]
    def step():
        h = int(torch.cuda.current_stream().cuda_stream)     # the capture stream inside a graph
        for l in range(layers):
            kvd.kvd_decode_attn_mixed(pools[False], pools[True], l, args[l], h)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    secs = (time.perf_counter() - t0) / steps
    tok8 = sum(min(16, int(s) - 16 * b) for i, s in enumerate(lens) for b in range(len(prec[i])) if prec[i][b])
    tok16 = n_tok - tok8
    per_layer = (tok16 * 2 * w.n_kv * w.head_dim * 2 + tok8 * 2 * w.n_kv * w.head_dim
                 + 2 * w.n_kv * 4 * n8 + 4 * (n16 + n8) + w.b * 2 * w.n_q * w.head_dim * 2)
    res = {"workload": f"{w.name} ({layers} layers), {tok8 / n_tok:.1%} of tokens in FP8 blocks",
           "ms_per_step": round(secs * 1e3, 4), "GBs": round(layers * per_layer / secs / 1e9, 1),
           "bytes_per_step": layers * per_layer}
    log(f"mixed: {res}")
    del graph, pools, args, ws, outs, qs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def append_entry(name: str, calls: int):
    """Cost of the decode step's own write: one token per sequence per layer."""
    wl = Workload(name, 0, 1, layers=1)
    eager, graphed, dec, fused = wl.time_append(calls)
    w = wl.w
    e = {"workload": f"{w.name} (1 layer)", "kv_dtype": w.kv_dtype, "tokens_per_call": w.b,
         "us_per_call": round(graphed * 1e6, 2), "us_per_call_eager": round(eager * 1e6, 2),
         "decode_us": round(dec * 1e6, 2), "fused_append_decode_us": round(fused * 1e6, 2),
         "stored_bytes_per_call": w.b * 2 * w.n_kv * w.head_dim * wl.kv_bytes}
    wl.free()
    return e


def hbm_context(launch_bytes: int, secondary_bytes: int = 0, nbytes: int = 1 << 30, reps: int = 20):
    """The box's own read and copy rates, as context for the roofline (not a
    bound the decode must meet):
    * stream_read -- libkvdecode's plain streaming read (the decode kernels'
      own 16-byte non-temporal loads and nothing else) of launch_bytes, the
      headline decode launch's size, cycling through 8 buffers (more than the
      256 MB Infinity Cache) at several grid sizes: the best is the practical
      ceiling of a launch that size; stream_read_secondary likewise for the
      secondary workload's launch (one buffer, already beyond the cache);
    * copy, read_torch -- torch's device-to-device copy (read + write counted)
      and torch's sum (read only) over nbytes of fp32.
    Each is timed with HIP events over repeated calls after a warm-up."""
    import torch
    import decode_attention_paged_04_amd as kvd
    st = torch.cuda.current_stream()

    def timed(fn, n):
        for k in range(3):
            fn(k)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for k in range(n):
            fn(k)
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3          # us per call

    def stream_read(nb: int, nbuf: int, n: int):
        sb = nb // 16 * 16
        if sb >= (1 << 32):                      # beyond one buffer resource: not measured
            return None
        bufs = [torch.empty(sb, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
        by_grid = {}
        for grid in (256, 512, 1024, 2048):
            sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
            by_grid[grid] = timed(lambda k: kvd.kvd_debug_stream_read(bufs[k % nbuf], sink, grid), n)
        best = min(by_grid, key=by_grid.get)
        del bufs
        torch.cuda.empty_cache()
        return {"bytes": sb, "buffers": nbuf, "grid": best, "us": round(by_grid[best], 2),
                "GBs": round(sb / by_grid[best] / 1e3, 1),
                "us_by_grid": {str(g): round(u, 2) for g, u in by_grid.items()},
                "kernel": "kvd_debug_stream_read (the decode kernels' loads only)"}

    out = {"stream_read": stream_read(launch_bytes, 8, 200)}
    if secondary_bytes and secondary_bytes < (1 << 32):
        out["stream_read_secondary"] = stream_read(secondary_bytes, 1, 20)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    copy_us = timed(lambda k: dst.copy_(src), reps)
    read_us = timed(lambda k: torch.sum(src, dim=0, out=acc), reps)
    del src, dst
    torch.cuda.empty_cache()
    out["copy"] = {"bytes": nbytes, "us": round(copy_us, 2), "GBs_read_plus_write": round(2 * nbytes / copy_us / 1e3, 1),
                   "kernel": "torch copy_ (device to device)"}
    out["read_torch"] = {"bytes": nbytes, "us": round(read_us, 2), "GBs": round(nbytes / read_us / 1e3, 1),
                         "kernel": "torch sum over fp32"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--secondary", default=SECONDARY, help="second workload in the same line, or 'none'")
    ap.add_argument("--secondary-steps", type=int, default=10)
    ap.add_argument("--chunk", type=int, default=0, help="chunk_tokens (0 = the library's choice)")
    ap.add_argument("--replicas", type=int, default=0, help="pool replicas (0 = enough to exceed the cache)")
    ap.add_argument("--launches", type=int, default=200, help="event-timed launches for the roofline")
    ap.add_argument("--extras", default="8b_ragged,8b_fp8_scores,70b_shard,8b_prefix,8b_prefix256,8b_prefix1024,"
                    "8b_batch256",
                    help="further workloads reported in the same line (comma list), or 'none'")
    ap.add_argument("--no-append", action="store_true", help="skip the append-cost entries")
    ap.add_argument("--no-tiered", action="store_true", help="skip the tier-restricted entry")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed-precision entry")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle budget of the headline entry")
    ap.add_argument("--extra-cpu-seconds", type=float, default=6.0,
                    help="oracle budget of each further entry (two layers, extrapolated)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the decode step "
              f"shards by sequence or KV head with no exchange, so N GPUs run N independent copies).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.copy_probe:
        # A plain copy of known size: under rocprofv3 --pmc its FETCH_SIZE and
        # WRITE_SIZE per dispatch calibrate the counters against known bytes.
        n = args.copy_probe
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 10
        print(json.dumps({"copy_bytes": n, "us_per_copy": round(dt * 1e6, 2),
                          "GBs_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)
        return

    wl, head = measure(args.workload, args.chunk, args.replicas, args.steps, args.warmup, args.launches)
    w_head, lens_head = wl.w, wl.lens
    wl.free()
    del wl
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w_head, lens_head, args.cpu_seconds)
        log(f"cpu baseline: {cpu['value']} GB/s on {cpu['cores']} thread(s) ({cpu['sample']})")

    secondary = None
    if args.secondary != "none" and args.secondary != args.workload:
        wl2, sec = measure(args.secondary, 0, 0, args.secondary_steps, 2, 80)
        w2, lens2 = wl2.w, wl2.lens
        wl2.free()
        del wl2
        traffic2 = measured_traffic(args.secondary)
        secondary = {"workload": sec["config"]["workload"], "value": round(sec["value"], 2), "unit": "GB/s",
                     "ms_per_step": round(sec["ms_per_step"], 4), "steps": args.secondary_steps,
                     "seq_steps_per_s": round(sec["seq_steps_per_s"], 3),
                     "pct_of_hbm_peak": round(sec["pct_of_hbm_peak"], 2), "config": sec["config"],
                     "roofline": {"bound": "hbm", "achieved": round(sec["achieved"], 2),
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(sec["achieved"] / PEAK_HBM_GBS, 4),
                                  "traffic": traffic2, "launch_us": round(sec["launch_us"], 2)}}
        if not args.no_cpu_baseline:
            secondary["cpu_baseline"] = cpu_baseline(w2, lens2, args.extra_cpu_seconds)
            log(f"secondary cpu baseline: {secondary['cpu_baseline']['value']} GB/s "
                f"({secondary['cpu_baseline']['sample']})")

    extras = []
    if args.extras != "none":
        for name in args.extras.split(","):
            extras.append(extra_entry(name, 10, 0.0 if args.no_cpu_baseline else args.extra_cpu_seconds))
    tiered = None
    if not args.no_tiered:
        tiered = tiered_entry("8b_ragged", 8, 10)
    mixed = None
    if not args.no_mixed:
        mixed = mixed_entry("8b_ragged", 8, 10)
    appends = []
    if not args.no_append:
        for name in ("8b_ragged", "8b_fp8_scores"):
            appends.append(append_entry(name, 200))

    traffic = measured_traffic(args.workload)
    try:
        context = hbm_context(head["launch_bytes"], sec["launch_bytes"] if secondary else 0)
        if context["stream_read"]:
            context["decode_launch_vs_stream_read"] = round(context["stream_read"]["us"] / head["launch_us"], 4)
        if context.get("stream_read_secondary"):
            context["secondary_launch_vs_stream_read"] = round(
                context["stream_read_secondary"]["us"] / sec["launch_us"], 4)
        log(f"hbm context: {context}")
    except Exception as e:                     # context only: never costs the line
        log(f"hbm context not measured: {e}")
        context = None
    line = {
        "metric": METRIC,
        "value": round(head["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/K/V, per-channel K/V magnitudes U[0.5,2], shuffled block pool)",
        "config": head["config"],
        "seq_steps_per_s": round(head["seq_steps_per_s"], 1),
        "pct_of_hbm_peak": round(head["pct_of_hbm_peak"], 2),
        "roofline": {"bound": "hbm", "achieved": round(head["achieved"], 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(head["achieved"] / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "launch_us": round(head["launch_us"], 3),
                     "bytes_per_launch": head["launch_bytes"]},
        "cpu_baseline": cpu,
        "hbm_context": context,
        "secondary": secondary,
        "extra": extras,
        "tiered": tiered,
        "mixed": mixed,
        "append": appends,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
