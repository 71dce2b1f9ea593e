#!/usr/bin/env python3
"""Benchmark of the CSA2 FP4 sparse-attention decode hot path on one MI355X.

Default workload: the 1M-context decoder stack, batch 8, four layers in roles
[Full, Reindex, Reuse, Reuse] with a 16,384-candidate pool, Top-K 2,048, 64
heads and a 128-token window (the scale the DeepSeek-V4.1-Flash write-ups
describe).  One step = pack the current token's latent row into the FP4 cache,
then every layer's indexer / selection / sparse attention / window merge.

Prints ONE JSON line: query-tokens/s over the timed steps, the step's
algorithmic HBM GB/s, the roofline of the dominant kernel (the Full-layer
index scan) timed with HIP events on the launch stream, and the CPU oracle
timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W]
                  [--workload stack_1m_b8|full_decode_b64|tiny_decode|pack_1m|prefill_4k_256k]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "decode query-tokens/s + achieved HBM GB/s, CSA2 FP4 sparse attn @1M ctx"
HBM_PEAK_GBPS = 8000.0
SIGMA = 1.0 / math.sqrt(128)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="stack_1m_b8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--cpu-sample", type=int, default=0, help="sequences in the CPU-baseline sample (0 = auto)")
    ap.add_argument("--input-sets", type=int, default=4,
                    help="decode: query sets replayed in turn (different selections, different gathered rows)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    return ap.parse_args()


def kernel_source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, "fp4_sparse_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(name, digest, workload):
    """HBM bytes per launch from committed counter runs (FETCH_SIZE / WRITE_SIZE), if taken on this kernel
    source and workload; profiles/<name>_traffic.json holds one record or a list of them."""
    path = os.path.join(HERE, "profiles", f"{name}_traffic.json")
    try:
        with open(path) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    for rec in recs if isinstance(recs, list) else [recs]:
        if rec.get("kernel_source_sha256") == digest and rec.get("workload") == workload:
            return rec.get("hbm_bytes_per_launch")
    return None


def decode_step_bytes(B, T, H, K, P, modes, W=128, streams=True):
    """Compulsory bytes of one decode step (each call's inputs read once, outputs written once).
    streams: the Full layer's selection runs during its scan (csa2_index_full_pool_streams)."""
    C = 512
    total = B * (2 * C + 288)                          # pack the current token's row
    total += B * 2 * 64 + B * len(modes) * 3 * 2 * C  # its key copied; each layer's window row into both ring slots
    for mode in modes:
        if mode == "full":
            if P:
                # keys + query read; pool (positions + scores) and Top-K written: the streaming selection
                # needs no score array
                total += B * T * 64 + B * 64 + B * P * 8 + B * K * 4
            elif streams:
                # the streaming selection cuts the Top-K during the scan: keys + query read, Top-K written
                total += B * T * 64 + B * 64 + B * K * 4
            else:
                # short rows: keys + query, scores written and read back by the selection, Top-K written
                total += B * T * (64 + 4) + B * 64 + B * T * 4 + B * K * 4
        elif mode == "reindex":
            total += B * P * (4 + 64 + 4) + B * 64      # pool ids, gathered keys, scores
            total += B * P * 8 + B * K * 4
        # sparse attention: idx, gathered FP4 rows, queries, o + lse
        total += B * K * (4 + 288) + B * H * C * 2 + B * H * (C + 1) * 4
        # window merge: window rows, queries, sparse o/lse in, o/lse out
        total += B * W * C * 2 + B * H * C * 2 + 2 * B * H * (C + 1) * 4
    return total


def cpu_baseline_decode(wl, cfg, n_seq):
    """Time the CPU oracle on n_seq sequences of the same decode step."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info
    from oracle import formats as OF, indexer as OI, topk as OT, attention as OA

    cores = len(os.sched_getaffinity(0))
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max(blas) if blas else 1
    modes = cfg.modes
    P = cfg.pool if "reindex" in modes else 0
    elapsed = 0.0
    for b in range(n_seq):
        # inputs (generator data), copied to the host outside the timed region
        k_host = wl.k_idx[b].cpu().numpy()
        layers = [(io.q_idx[b].cpu().numpy(), io.q_lat[b].to(torch.float64).cpu().numpy(),
                   io.swa[b].to(torch.float64).cpu().numpy()) for io in wl.layers]
        new_row = wl.new_rows[b:b + 1].to(torch.float64).cpu().numpy()
        t0 = time.perf_counter()
        OF.fp4_pack(new_row)
        pool = None
        prev = None
        needed = []
        for mode, (q_idx, q_lat, swa) in zip(modes, layers):
            if mode == "full":
                s = OI.full_scores(q_idx, k_host)
                if P:
                    pool = OT.candidate_pool(s, P)
                    idx = OT.topk(np.where(pool >= 0, s[np.clip(pool, 0, None)], -np.inf), cfg.topk, index_map=pool)
                else:
                    idx = OT.topk(s, cfg.topk)
            elif mode == "reindex":
                idx = OT.topk(OI.reindex_scores(q_idx, k_host, pool), cfg.topk, index_map=pool)
            else:
                idx = prev
            prev = idx
            needed.append(idx)
        elapsed += time.perf_counter() - t0
        # the oracle packs the latent rows it attends over; drawing them is input generation
        rows_by_layer = []
        for idx in needed:
            pos = idx[idx >= 0]
            rows_by_layer.append(wl.latent_host(b, pos))
        t0 = time.perf_counter()
        for (q_idx, q_lat, swa), lat in zip(layers, rows_by_layer):
            c, s_ = OF.fp4_pack(lat)
            rows = OF.fp4_unpack(c, s_)
            o_s, l_s = OA.attend(q_lat, rows, SIGMA)
            o_w, l_w = OA.attend(q_lat, OA.window_rows(swa, 0, cfg.window), SIGMA)
            OA.merge(o_s, l_s, o_w, l_w)
        elapsed += time.perf_counter() - t0
    return {"value": n_seq / elapsed, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_seq} of {cfg.batch} sequences of one {len(modes)}-layer step "
                      f"(numpy; BLAS pool {threads} threads of {cores} allowed cores; index scan single-threaded int64)",
            "seconds": elapsed}


class Workload:
    """Seeded decode inputs on the GPU; the FP4 cache is packed by the library."""

    def __init__(self, cfg, dev, chunk_rows=65536, n_sets=1):
        import torch
        import workloads as W
        from fp4_sparse_attention_amd.decode import StackIO, pack_cache
        B, T = cfg.batch, cfg.context
        self.T = T
        self.cfg = cfg
        self.dev = dev
        self.chunk_rows = min(chunk_rows, T)
        self.n_chunks = (T + self.chunk_rows - 1) // self.chunk_rows
        self.outliers = W.outlier_channels(cfg.seed)
        self.codes = torch.empty((B, T, 256), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((B, T, 32), dtype=torch.uint8, device=dev)
        pack_cache(self.codes, self.scales, self.latent_chunk, self.chunk_rows)
        self.k_idx = torch.stack([W.fp8_normal(cfg.seed, (T, 64), device=dev, chunk_index=b) for b in range(B)])
        L = len(cfg.modes)
        # each layer's window is a mirrored ring of 2 x 128 rows (the decode-time append writes the current
        # token's window row into it every step)
        ds = [W.decode_layer_inputs(cfg.seed, li, B, cfg.heads, 2 * cfg.window, B, device=dev, outliers=self.outliers)
              for li in range(L)]
        self.layers = StackIO(torch.stack([d["q_lat"] for d in ds]), torch.stack([d["q_idx"] for d in ds]),
                              torch.stack([d["swa"] for d in ds]), torch.zeros((L, B), dtype=torch.int32, device=dev),
                              torch.full((L, B), min(cfg.window, T), dtype=torch.int32, device=dev))
        # the current token: its latent row, indexer key and per-layer window rows, appended at position T-1
        # by every step
        self.new_rows = self.latent_chunk_rows_at(T - 1)
        self.new_keys = self.k_idx[:, T - 1].clone()
        self.new_window = W.bf16_normal(cfg.seed, (L, B, 512), device=dev, chunk_index=7919)
        # further query sets (latent and indexer queries of every layer), so that consecutive steps select
        # different positions and gather different rows; they share the cache, keys and window rings
        self.layer_sets = [self.layers]
        for s in range(1, n_sets):
            self.layer_sets.append(StackIO(
                W.bf16_normal(cfg.seed, (L, B, cfg.heads, 512), std=0.5, device=dev, role=4, chunk_index=1000 + s),
                W.fp8_normal(cfg.seed, (L, B, 64), device=dev, role=3, chunk_index=1000 + s),
                self.layers.swa, self.layers.swa_start, self.layers.swa_len))
        torch.cuda.synchronize()

    def latent_chunk(self, b, c):
        import workloads as W
        n = min(self.chunk_rows, self.T - c * self.chunk_rows)
        return W.latent_rows(self.cfg.seed, n, device=self.dev, outliers=self.outliers,
                             chunk_index=b * self.n_chunks + c)

    def latent_chunk_rows_at(self, pos):
        import torch
        c = pos // self.chunk_rows
        return torch.stack([self.latent_chunk(b, c)[pos - c * self.chunk_rows] for b in range(self.cfg.batch)])

    def latent_host(self, b, positions):
        import numpy as np
        import torch
        positions = np.asarray(positions, dtype=np.int64)
        out = np.empty((positions.shape[0], 512))
        chunk = positions // self.chunk_rows
        for c in np.unique(chunk):
            sel = chunk == c
            local = torch.from_numpy(positions[sel] - c * self.chunk_rows).to(self.dev)
            out[sel] = self.latent_chunk(b, int(c))[local].to(torch.float64).cpu().numpy()
        return out


def attention_layer_bytes(B, H, K, W=128, C=512):
    """Compulsory bytes of one layer of the stacked attention launch: its index slice, the K gathered FP4 rows
    (288 B each), the latent queries, the window rows, o and lse written."""
    return B * K * (4 + 288) + B * H * C * 2 + B * W * C * 2 + B * H * (C + 1) * 4


def time_absorb(cfg, dev, reps):
    """Per-step time of the absorption helpers: one csa2_absorb_q and one csa2_unabsorb_o per layer, each
    layer with its own W_UK / W_UV (bf16 [H, 128, 512])."""
    import torch
    import workloads as W
    import fp4_sparse_attention_amd as F
    L, B, H = len(cfg.modes), cfg.batch, cfg.heads
    w = [W.absorb_weights(cfg.seed, l, H, device=dev) for l in range(L)]
    q = [W.head_queries(cfg.seed, l, B, H, device=dev) for l in range(L)]
    q_lat = torch.empty((L, B, H, 512), dtype=torch.bfloat16, device=dev)
    o_lat = torch.randn((L, B, H, 512), device=dev)
    out = torch.empty((L, B, H, 128), dtype=torch.float32, device=dev)

    def absorb():
        for l in range(L):
            F.csa2_absorb_q(q[l], w[l][0], q_lat[l])

    def unabsorb():
        for l in range(L):
            F.csa2_unabsorb_o(o_lat[l], w[l][1], out[l])

    res = {}
    for name, fn, per_layer in (("absorb_q", absorb, H * 128 * 512 * 2 + B * H * (128 + 512) * 2),
                                ("unabsorb_o", unabsorb, H * 128 * 512 * 2 + B * H * (512 + 128) * 4)):
        # `inner` repetitions of the L calls captured into one graph and replayed, so that neither host
        # launch overhead nor the per-replay gap is timed
        inner = 10
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(inner):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * inner)
        res[name] = {"us_per_step": us, "calls_per_step": L, "bytes_per_step": L * per_layer,
                     "gbps": L * per_layer / (us * 1e-6) / 1e9, "launch": "hip graph replay"}
    return res


def bench_decode(args, cfg):
    import torch
    import fp4_sparse_attention_amd as F
    from fp4_sparse_attention_amd.decode import Csa2DecodeStack
    dev = torch.device("cuda:0")
    n_sets = max(1, args.input_sets)
    wl = Workload(cfg, dev, n_sets=n_sets)
    stack = Csa2DecodeStack(cfg.batch, cfg.context, cfg.heads, cfg.topk, cfg.modes,
                            pool_size=cfg.pool if cfg.pool else 16384)

    def step(i, **kw):
        stack.step(wl.codes, wl.scales, wl.k_idx, wl.layer_sets[i % n_sets], SIGMA, new_rows=wl.new_rows,
                   new_keys=wl.new_keys, new_window=wl.new_window, **kw)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # eager steps, with events around the Full-layer scan and the attention launch for their roofline figures
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    index_ev, attn_ev = [], []
    t_start.record()
    for i in range(args.steps):
        step(i, time_index=True, time_attention=True)
        index_ev.append(stack.index_events)
        attn_ev.append(stack.attention_events)
    t_end.record()
    torch.cuda.synchronize()
    ms_eager = t_start.elapsed_time(t_end) / args.steps
    idx_ms = sum(a.elapsed_time(b) for a, b in index_ev) / len(index_ev)
    attn_ms = sum(a.elapsed_time(b) for a, b in attn_ev) / len(attn_ev)
    ms = ms_eager
    graphs = None
    if not args.no_graph:
        # each query set's step captured once into a HIP graph and the graphs replayed in turn: every kernel
        # of every step still runs; only the per-launch host overhead goes
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for i in range(n_sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        # one pass over the query sets (n_sets consecutive steps) in one graph, so that a short step is not
        # timed against the host's per-replay launch cost; K steps = K // n_sets passes + the single-step
        # graphs of the first K % n_sets sets
        rotation = torch.cuda.CUDAGraph()
        with torch.cuda.graph(rotation):
            for i in range(n_sets):
                step(i)
        for i in range(args.warmup):
            graphs[i % n_sets].replay()
        rotation.replay()
        torch.cuda.synchronize()
        t_start.record()
        for _ in range(args.steps // n_sets):
            rotation.replay()
        for i in range(args.steps % n_sets):
            graphs[i].replay()
        t_end.record()
        torch.cuda.synchronize()
        ms = t_start.elapsed_time(t_end) / args.steps
    B, T, H, K = cfg.batch, cfg.context, cfg.heads, cfg.topk
    L = len(cfg.modes)
    P = min(cfg.pool, T) if "reindex" in cfg.modes else 0
    # the Full-layer scan: 64-byte keys per position and the query; when the library selects during the scan
    # no score array is written, otherwise 4 bytes of score per position
    streams = F.csa2_index_full_pool_streams(B, T)
    step_bytes = decode_step_bytes(B, T, H, K, P, cfg.modes, cfg.window, streams)
    idx_bytes = B * T * (64 if streams else 64 + 4) + B * 64
    achieved = idx_bytes / (idx_ms * 1e-3) / 1e9
    digest = kernel_source_digest(["index.hip", "tile.hpp", "internal.hpp", "common.hpp"])
    attn_bytes = L * attention_layer_bytes(B, H, K, cfg.window)
    attn_achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    attn_digest = kernel_source_digest(["attention.hip", "internal.hpp", "common.hpp"])
    rec = {
        "metric": METRIC,
        "value": B / (ms * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_eager": ms_eager,
        "launch": (f"hip graph replay: one graph per pass over the {n_sets} query sets ({n_sets} steps)" if graphs is not None
                   else f"eager, {n_sets} query sets in turn"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1/e4m3 storage; e4m3xe4m3->f32 index; f16xf16->f32 sparse attention, bf16xbf16->f32 window",
        "data": "synthetic (seeded torch normal draws; FP4 cache packed by the library)",
        "config": {"workload": cfg.name, "batch": B, "context": T, "heads": H, "topk": K,
                   "layers": list(cfg.modes), "pool": P, "window": cfg.window, "latent_channels": 512},
        "achieved_hbm_gbps": step_bytes / (ms * 1e-3) / 1e9,
        "step_algorithmic_bytes": step_bytes,
        "roofline": {"kernel": ("csa2_index_full_pool scan (index_stream_kernel<true>, no score output)" if streams
                               else "csa2_index_full_pool scoring pass (scores written)"), "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic("index_full", digest, cfg.name),
                     "launch_ms": idx_ms, "bytes_per_launch": idx_bytes},
        "roofline_attention": {"kernel": f"csa2_sparse_swa_decode_layers ({L} layers: chunk + combine kernels)",
                               "bound": "hbm", "achieved": attn_achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                               "frac": attn_achieved / HBM_PEAK_GBPS,
                               "traffic": measured_traffic("attention", attn_digest, cfg.name),
                               "launch_ms": attn_ms, "bytes_per_launch": attn_bytes},
        "absorb_helpers": time_absorb(cfg, dev, max(args.steps, 5)),
    }
    if not args.no_cpu_baseline:
        n_seq = args.cpu_sample or (4 if T >= (1 << 20) else 8)
        rec["cpu_baseline"] = cpu_baseline_decode(wl, cfg, min(n_seq, B))
    else:
        rec["cpu_baseline"] = None
    return rec


class PrefillWorkload:
    """Seeded chunked-prefill inputs on the GPU: one sequence's FP4 cache and indexer keys, and the
    last `queries` positions as causal query rows with their indexer queries, absorbed queries and
    sliding-window rows (row i sees positions <= T - queries + i and the 128 window rows before it)."""

    def __init__(self, cfg, dev, chunk_rows=65536):
        import torch
        import workloads as W
        from fp4_sparse_attention_amd.decode import pack_cache
        T, Q, H = cfg.context, cfg.queries, cfg.heads
        self.T, self.cfg, self.dev = T, cfg, dev
        self.chunk_rows = min(chunk_rows, T)
        self.n_chunks = (T + self.chunk_rows - 1) // self.chunk_rows
        self.outliers = W.outlier_channels(cfg.seed)
        self.codes = torch.empty((1, T, 256), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((1, T, 32), dtype=torch.uint8, device=dev)
        pack_cache(self.codes, self.scales, self.latent_chunk, self.chunk_rows)
        self.k_idx = W.fp8_normal(cfg.seed, (T, 64), device=dev, chunk_index=0)[None]
        self.q_idx = W.fp8_normal(cfg.seed, (Q, 64), device=dev, role=3, chunk_index=100)
        self.q_lat = W.bf16_normal(cfg.seed, (Q, H, 512), std=0.5, device=dev, role=4, chunk_index=100)
        self.swa = W.bf16_normal(cfg.seed, (1, Q + cfg.window - 1, 512), device=dev, role=5, chunk_index=100)
        self.row_seq = torch.zeros(Q, dtype=torch.int32, device=dev)
        self.limit = torch.arange(T - Q, T, dtype=torch.int64, device=dev)
        self.swa_start = torch.arange(Q, dtype=torch.int32, device=dev)
        self.swa_len = torch.full((Q,), cfg.window, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()

    latent_chunk = Workload.latent_chunk
    latent_host = Workload.latent_host


def cpu_baseline_prefill(wl, cfg, n_rows):
    """Time the CPU oracle on n_rows of the prefill rows (scores over the row's visible positions,
    Top-K, FP4 round trip of the selected rows, sparse and window attention, merge)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info
    from oracle import formats as OF, indexer as OI, topk as OT, attention as OA

    cores = len(os.sched_getaffinity(0))
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max(blas) if blas else 1
    Q, T = cfg.queries, cfg.context
    k_host = wl.k_idx[0].cpu().numpy()
    swa_host = wl.swa[0].to(torch.float64).cpu().numpy()
    rows = np.linspace(0, Q - 1, n_rows).astype(np.int64)
    elapsed = 0.0
    for r in rows:
        q_idx = wl.q_idx[r].cpu().numpy()
        q_lat = wl.q_lat[r].to(torch.float64).cpu().numpy()
        t0 = time.perf_counter()
        idx = OT.topk(OI.full_scores(q_idx, k_host, limit=T - Q + int(r)), cfg.topk)
        elapsed += time.perf_counter() - t0
        lat = wl.latent_host(0, idx[idx >= 0])            # regenerating the rows is input generation
        t0 = time.perf_counter()
        c, s_ = OF.fp4_pack(lat)
        o_s, l_s = OA.attend(q_lat, OF.fp4_unpack(c, s_), SIGMA)
        o_w, l_w = OA.attend(q_lat, OA.window_rows(swa_host, int(r), cfg.window), SIGMA)
        OA.merge(o_s, l_s, o_w, l_w)
        elapsed += time.perf_counter() - t0
    return {"value": n_rows / elapsed, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_rows} of {Q} prefill rows (numpy; BLAS pool {threads} threads of {cores} allowed cores; "
                      f"index scan single-threaded int64)",
            "seconds": elapsed}


def bench_prefill(args, cfg):
    """One chunked-prefill layer per step: the Full-layer scores and Top-K of every query row
    (csa2_index_full_pool, the streaming selection over the query-block scan, no score array), then
    the sparse + window attention of every row (csa2_sparse_swa_decode)."""
    import torch
    import fp4_sparse_attention_amd as F
    dev = torch.device("cuda:0")
    wl = PrefillWorkload(cfg, dev)
    T, Q, H, K = cfg.context, cfg.queries, cfg.heads, cfg.topk
    idx = torch.empty((Q, K), dtype=torch.int32, device=dev)
    twin = torch.empty((Q, K), dtype=torch.int32, device=dev)
    o = torch.empty((Q, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((Q, H), dtype=torch.float32, device=dev)
    # the selection's workspace for all rows in one batch (8.6 GB here: 288 GB of HBM holds it); the minimal
    # size (below 1 GB) would run the rows in ten batches, +0.7 ms per step
    ws_p = torch.empty(F.csa2_index_full_pool_batch_workspace_size(Q, T, K), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(F.csa2_sparse_swa_decode_workspace_size(Q, H, K), dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(timed=False):
        F.csa2_index_full_pool(wl.q_idx, wl.k_idx, None, K, K, idx, twin, row_seq=wl.row_seq, row_limit=wl.limit,
                               workspace=ws_p)
        if timed:
            ev[0].record()
        F.csa2_sparse_swa_decode(wl.q_lat, wl.codes, wl.scales, idx, wl.swa, wl.swa_start, wl.swa_len, SIGMA, o,
                                 lse, row_seq=wl.row_seq, workspace=ws_a)
        if timed:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    attn_ms = 0.0
    ev[2].record()
    for _ in range(args.steps):
        step(timed=True)
        torch.cuda.synchronize()
        attn_ms += ev[0].elapsed_time(ev[1])
    ev[3].record()
    torch.cuda.synchronize()
    # the steps' time without the host synchronisations: a second run, untimed per call
    ev[2].record()
    for _ in range(args.steps):
        step()
    ev[3].record()
    torch.cuda.synchronize()
    ms = ev[2].elapsed_time(ev[3]) / args.steps
    attn_ms /= args.steps
    n_pos = K + cfg.window
    attn_flops = Q * H * n_pos * 512 * 2 * 2                 # q.x and p.x per head and position
    index_bytes = T * 64 + Q * 64 + 2 * Q * K * 4            # keys and queries read, two index arrays written
    rec = {
        "metric": METRIC,
        "value": Q / (ms * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "launch": "eager",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1/e4m3 storage; e4m3xe4m3->f32 index; f16xf16->f32 sparse attention, bf16xbf16->f32 window",
        "data": "synthetic (seeded torch normal draws; FP4 cache packed by the library)",
        "config": {"workload": cfg.name, "queries": Q, "context": T, "heads": H, "topk": K, "window": cfg.window,
                   "latent_channels": 512},
        "index_algorithmic_bytes": index_bytes,
        "roofline": {"kernel": "csa2_sparse_swa_decode (attn_chunk_kernel: one chunk per row, o and lse written "
                               "directly)", "bound": "mfma",
                     "achieved": attn_flops / (attn_ms * 1e-3) / 1e12, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": attn_flops / (attn_ms * 1e-3) / 2.5e15, "traffic": None, "launch_ms": attn_ms,
                     "flops_per_launch": attn_flops},
    }
    rec["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_prefill(wl, cfg, args.cpu_sample or 16)
    return rec


def bench_pack(args, cfg):
    import torch
    import workloads as W
    import fp4_sparse_attention_amd as F
    dev = torch.device("cuda:0")
    n, C = cfg.rows, cfg.channels
    x = W.latent_rows(cfg.seed, n, device=dev, outliers=W.outlier_channels(cfg.seed))
    codes = torch.empty((n, C // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, C // 16), dtype=torch.uint8, device=dev)
    xb = torch.empty_like(x)
    for _ in range(args.warmup):
        F.csa2_fp4_pack(x, codes, scales)
        F.csa2_fp4_unpack(codes, scales, xb)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
    for i in range(args.steps):
        ev[3 * i].record()
        F.csa2_fp4_pack(x, codes, scales)
        ev[3 * i + 1].record()
        F.csa2_fp4_unpack(codes, scales, xb)
        ev[3 * i + 2].record()
    torch.cuda.synchronize()
    pack_ms = sum(ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(args.steps)) / args.steps
    unpack_ms = sum(ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(args.steps)) / args.steps
    bytes_dir = n * (2 * C + C // 2 + C // 16)
    achieved = bytes_dir / (pack_ms * 1e-3) / 1e9
    digest = kernel_source_digest(["pack.hip", "common.hpp"])
    ms = pack_ms + unpack_ms
    rec = {
        "metric": "FP4 pack+unpack rows/s (memory-bound stream)", "value": n / (ms * 1e-3), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 <-> e2m1 + e4m3", "data": "synthetic",
        "config": {"workload": cfg.name, "rows": n, "channels": C},
        "achieved_hbm_gbps": 2 * bytes_dir / (ms * 1e-3) / 1e9,
        "unpack_gbps": bytes_dir / (unpack_ms * 1e-3) / 1e9,
        "roofline": {"kernel": "csa2_fp4_pack", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic("fp4_pack", digest, cfg.name), "launch_ms": pack_ms,
                     "bytes_per_launch": bytes_dir},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import formats as OF
        sample = 65536
        xs = x[:sample].to(torch.float64).cpu().numpy()
        t0 = time.perf_counter()
        c, s = OF.fp4_pack(xs)
        OF.fp4_unpack(c, s)
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": sample / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {sample} rows, pack then unpack (numpy, single thread)",
                               "seconds": dt}
    return rec


def copy_calibration():
    """A plain 1 GiB device-to-device copy (read 1 GiB, write 1 GiB), run 3 times:
    the reference for scaling the FETCH_SIZE / WRITE_SIZE hardware counters."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.full((1 << 28,), 1.0, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": 1 << 30, "copies": 3}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only (there is no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import fp4_sparse_attention_amd as F
    F.lib()                       # fail loudly if the HIP library is missing
    if args.copy_calibration:
        copy_calibration()
        return
    import workloads as W
    cfg = W.by_name(args.workload)
    print(f"# workload {cfg.name}: building inputs", file=sys.stderr, flush=True)
    if isinstance(cfg, W.PackStream):
        rec = bench_pack(args, cfg)
    elif isinstance(cfg, W.ChunkedPrefill):
        rec = bench_prefill(args, cfg)
    else:
        rec = bench_decode(args, cfg)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
