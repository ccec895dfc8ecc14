"""Benchmark of the DLRM hot path on one MI355X.

Default workload ("forward"): batch 32768, 13 log-normal dense features,
bottom MLP 13-512-256-128, 26 fp32 tables of d = 128 with log-uniform
cardinalities in [100, 4e7] (about 2e8 rows, about 100 GB in HBM), one
Zipf(1.1) index per bag, 351-pair interaction, top MLP
479-1024-1024-512-256-1, bf16 MLPs with fp32 accumulation.  A step is one
full forward pass over one batch (bottom MLP, pooled lookups, interaction,
top MLP with sigmoid); inputs are resident in HBM before timing starts.

Prints one JSON line: samples/s, the roofline of the dominant kernel (the
fused pooled lookup + interaction kernel, or the gather alone in the
gather microbench: algorithmic bytes per launch over its average launch
time, measured with HIP events on its stream), the matrix-core fraction of
every MLP layer (algorithmic 2*M*N*K flops over its HIP-event time over the
2.5 PFLOP/s bf16 peak), and the CPU oracle timed on a bounded sample (about
10 s) of the same workload, with all threads and with one.

An event record costs a few microseconds of GPU time, so the timed steps
carry only the two events around the dominant kernel.  The per-call
breakdown (medians; the forward top MLP layer by layer through
dlrm_linear_fwd, the same kernels dlrm_mlp_fwd launches) comes from an
untimed pass of at least --breakdown-seconds that runs before the warm-up
and timed steps; it also brings the GPU to its steady clock, which a few
warm-up steps alone do not (20 steps from a cold start read about 10% low).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "DLRM fwd samples/s at 1 GPU; EmbeddingBag HBM GB/s as % of peak"


ROW_BYTES = {"f32": lambda d: 4 * d, "bf16": lambda d: 2 * d, "int8": lambda d: d + 8}  # int8: + (scale, bias)


def gather_bytes(K, B, d, nnz, table_dtype="f32"):
    """Algorithmic bytes of one pooled-lookup launch: every looked-up row
    (with its scale and bias for int8 rows), the int64 indices and offsets,
    and the fp32 pooled output."""
    return ROW_BYTES[table_dtype](d) * nnz + 8 * nnz + 8 * (K * B + 1) + 4 * K * B * d


def measured_traffic(key, kernel):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (profiles/hbm_traffic.json, scaled
    by the counters' reading for a copy of known size), or None when there is
    no record for this workload or the kernel's sources changed since."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("workloads", {}).get(key)
    if not rec or rec.get("kernel") != kernel:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--breakdown-steps", type=int, default=20,
                   help="least number of untimed steps before the warm-up with every call bracketed by events (the "
                        "per-call breakdown; the timed steps carry only the dominant kernel's pair of events)")
    p.add_argument("--breakdown-seconds", type=float, default=1.0,
                   help="the breakdown pass runs at least this long (0 with --breakdown-steps 0 skips it)")
    p.add_argument("--workload", default="forward", choices=["forward", "embbag", "interaction", "train", "tiny"])
    p.add_argument("--batches", type=int, default=2, help="distinct input batches rotated over the steps")
    p.add_argument("--uniform", action="store_true", help="uniform indices instead of Zipf (control run)")
    p.add_argument("--table-dtype", default="f32", choices=["f32", "bf16", "int8"],
                   help="forward workloads: table rows stored as fp32, bf16, or int8 with a per-row scale "
                        "and bias (dlrm_embbag_fwd_lp, dlrm_embbag_interact_fwd_lp)")
    p.add_argument("--path", default="auto", choices=["auto", "fused", "two-call"],
                   help="pooled lookup + interaction: one fused call, two calls (X materialised), or auto (fused "
                        "for short bags)")
    p.add_argument("--chain", action="store_true",
                   help="training workload only: the whole backward from the BCE loss (top MLP input gradient, "
                        "interaction backward, bottom MLP and sparse update from the real X gradient) instead of "
                        "the synthetic upstream gradient G")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-samples", type=int, default=0, help="oracle sample size (0: automatic)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB five times (a known-size kernel for "
                        "calibrating hardware byte counters), then exit")
    return p.parse_args()


class Timer:
    """HIP events recorded on the stream that runs the kernel."""

    def __init__(self):
        self.pairs = []

    def start(self, stream):
        import torch

        e0 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        return e0

    def stop(self, e0, stream):
        import torch

        e1 = torch.cuda.Event(enable_timing=True)
        e1.record(stream)
        self.pairs.append((e0, e1))

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) if self.pairs else float("nan")


def cpu_baseline(w, batches, bottom, top, n_samples, chain=False, min_seconds=10.0, table_dtype="f32"):
    """The oracle (as it stands) on the first n_samples of batch 0: forward
    for forward-type workloads, pooled lookups for the gather microbench,
    forward plus the sparse update for the training step (with ``chain``:
    forward with saved activations, the BCE seed, both MLP backwards, the
    interaction backward and the sparse update from its X gradient).  The pass is
    repeated until min_seconds of CPU work have run (a bounded sample);
    row regeneration and input slicing are excluded from the timed region.
    Returns (samples processed, seconds, threads, passes)."""
    import oracle
    from synth import workloads as W

    dense, idx, off = batches[0][:3]
    S = min(n_samples, w.B)
    samples = np.arange(S)
    sidx, soff = W.sub_bags(idx, off, w.K, w.B, samples)
    ws = w.scaled(B=S)
    tabs, local, row_ids = W.compact_rows(ws, sidx, soff)
    lp = table_dtype
    if lp != "f32":
        from synth import rng as R
        if lp == "bf16":
            tabs, sbs = [R.table_rows_bf16(w.seed, k, w.rows[k], row_ids[k], w.d) for k in range(w.K)], None
        else:
            pairs = [R.table_rows_i8(w.seed, k, w.rows[k], row_ids[k], w.d) for k in range(w.K)]
            tabs, sbs = [p[0] for p in pairs], [p[1] for p in pairs]
    quant = w.mlp_dtype == "bf16"
    G = batches[0][3].reshape(w.B, -1)[:S] if w.train else None
    y = batches[0][4][:S] if w.train else None

    def chain_pass():
        E = oracle.embbag_fwd(tabs, local, soff, S)
        Wb, bb = [p[0] for p in bottom], [p[2] for p in bottom]
        Wt, bt = [p[0] for p in top], [p[2] for p in top]
        x0, _, acts_b = oracle.mlp_fwd(dense[:S], Wb, bb, quant, True, save_acts=True)
        X = np.concatenate([x0, E], axis=1).reshape(S, w.n, w.d)
        top_in = oracle.interact_fwd(X)
        _, prob, acts_t = oracle.mlp_fwd(top_in, Wt, bt, quant, False, save_acts=True)
        dY = ((prob - y) / S).astype(np.float32).reshape(-1, 1)
        _, _, g_top = oracle.mlp_bwd(Wt, acts_t, dY, False, want_dx=True)
        GX = oracle.interact_bwd(X, g_top).reshape(S, -1)
        oracle.mlp_bwd(Wb, acts_b, GX[:, :w.d], True)
        oracle.embbag_bwd_sgd(tabs, local, soff, S, GX, w.d, w.lr)

    def one_pass():
        if chain:
            return chain_pass()
        if lp != "f32":
            E = oracle.embbag_fwd_lp(tabs, lp, local, soff, S, scale_bias=sbs)
        else:
            E = oracle.embbag_fwd(tabs, local, soff, S)
        if w.name != "embbag":
            x0, _, _ = oracle.mlp_fwd(dense[:S], [p[0] for p in bottom], [p[2] for p in bottom], quant, True)
            X = np.concatenate([x0, E], axis=1).reshape(S, w.n, w.d)
            top_in = oracle.interact_fwd(X)
            oracle.mlp_fwd(top_in, [p[0] for p in top], [p[2] for p in top], quant, False)
            if w.train:
                oracle.embbag_bwd_sgd(tabs, local, soff, S, G, w.d, w.lr)

    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return S * passes, dt, oracle.num_threads(), passes


def cpu_baseline_single(w, batches, bottom, top, n_samples, chain=False, min_seconds=4.0, table_dtype="f32"):
    """The same oracle pass with one thread on a smaller sample."""
    import oracle

    threads = oracle.num_threads()
    oracle.set_threads(1)
    try:
        return cpu_baseline(w, batches, bottom, top, n_samples, chain=chain, min_seconds=min_seconds,
                            table_dtype=table_dtype)
    finally:
        oracle.set_threads(threads)


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def mlp_layer_flops(B, dims):
    return [2.0 * B * i * o for i, o in zip(dims[:-1], dims[1:])]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): this build has no multi-GPU path; the "
              "sharding design is documented but not built.", file=sys.stderr)
        sys.exit(1)
    import torch

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}), flush=True)
        return

    import deep_learning_recommendation_amd as D
    from deep_learning_recommendation_amd import pipeline as PL
    from synth import device as SD
    from synth import workloads as W
    import dataclasses

    w = W.get(args.workload)
    if args.chain and not w.train:
        print("--chain applies to the training workload only", file=sys.stderr)
        sys.exit(1)
    if args.uniform:
        w = dataclasses.replace(w, index_dist="uniform")
    lp = args.table_dtype
    if lp != "f32" and w.train:
        print("--table-dtype applies to forward workloads (the sparse update needs fp32 rows)", file=sys.stderr)
        sys.exit(1)
    t_setup = time.perf_counter()
    dev = "cuda"
    if lp == "f32":
        tables, sbs = SD.make_tables(w), None
    else:
        tables, sbs = SD.make_tables_lp(w, lp)
    bf16 = w.mlp_dtype == "bf16"
    bottom = W.mlp_params(w, "bottom") if w.bottom else None
    top = W.mlp_params(w, "top") if w.top else None
    batches = []
    for bi in range(args.batches):
        idx, off = W.indices_offsets(w, bi)
        dense = W.dense(w, bi) if w.dense_dim else None
        G = W.upstream_grad(w, bi) if w.train else None
        y = W.labels(w, bi) if w.train else None
        batches.append((dense, idx, off, G, y))
    dbatches = []
    for (dense, idx, off, G, y) in batches:
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
        dbatches.append((t(dense), t(idx), t(off), t(G), t(y), int(off[-1])))
    model = None
    if w.bottom:
        bp = PL.make_mlp(w.bottom, [p[0] for p in bottom], [p[2] for p in bottom], bf16)
        tp = PL.make_mlp(w.top, [p[0] for p in top], [p[2] for p in top], bf16)
        fused = {"auto": "auto", "fused": True, "two-call": False}[args.path]
        if args.chain and fused is True:
            print("--chain needs X: use --path auto or two-call", file=sys.stderr)
            sys.exit(1)
        model = PL.DLRM(w.B, w.K, w.d, w.rows, tables, bp, tp, train=w.train, fused=fused, table_dtype=lp,
                        scale_bias=sbs)
        if w.train:
            model.sparse_workspace(max(b[5] for b in dbatches))
    else:
        ptrs = D.device_pointer_array(tables)
        sbp = D.device_pointer_array(sbs) if sbs is not None else None
        lp_code = {"bf16": D.DLRM_BF16, "int8": D.DLRM_I8}.get(lp)
        out = torch.empty((w.B, w.K * w.d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    stream = torch.cuda.current_stream()
    # training: the sparse update runs on a second stream: the index half
    # (keys, sort, segments) from the start of the step (it reads only the
    # indices), then, once the lookup has finished reading the tables, the
    # sums and the update (the synthetic gradient is an input), whose short
    # segments take a third stream; the interaction, top MLP and dense
    # backward run on the first stream meanwhile, and the step ends when all
    # three are done.
    # (The per-call breakdown runs the calls one after another on the first
    # stream instead, so that each interval holds one call.)
    prep_stream = torch.cuda.Stream() if w.train else None
    light_stream = torch.cuda.Stream() if w.train else None
    gather_t = Timer()
    call_t = {}   # per-call event pairs of the breakdown steps
    dom_t = {}    # the dominant kernel's event pairs over the timed steps
    DOMINANT = ("embbag", "embbag_interact")

    def step(i, mode):
        """One step; mode None (warm-up), "timed" (events around the dominant
        kernel only: each event record costs a few microseconds of GPU time)
        or "breakdown" (events around every call)."""
        timed = mode == "timed"
        dense, idx, off, G, y, nnz = dbatches[i % len(dbatches)]
        if model is None:
            e0 = gather_t.start(stream) if timed else None
            if lp == "f32":
                D.dlrm_embbag_fwd(ptrs, w.K, w.d, idx, off, w.B, out, w.K * w.d, 0, nnz=nnz)
            else:
                D.dlrm_embbag_fwd_lp(ptrs, lp_code, sbp, w.K, w.d, idx, off, w.B, out, w.K * w.d, 0, nnz=nnz)
            if timed:
                gather_t.stop(e0, stream)
            return
        n, d = model.n, model.d
        ev = {}
        overlap = w.train and mode != "breakdown"

        def mark(name):
            # timed steps: the dominant kernel's mark and the next one (its end)
            if mode == "breakdown" or (timed and (name in DOMINANT or len(ev) == 1)):
                ev[name] = gather_t.start(stream)

        def fork_prepare():
            # the index half reads only the indices: it starts with the step,
            # beside the bottom MLP and the lookup (the sort is on the path to
            # the update, the lookup is not); the breakdown pass runs it alone
            # on the first stream after the lookup instead
            if mode == "breakdown":
                return
            prep_stream.wait_stream(stream)
            with torch.cuda.stream(prep_stream):
                D.dlrm_embbag_bwd_sgd_prepare(w.K, w.rows, idx, off, w.B, nnz, model.ws_sparse)

        def after_lookup():
            # the update writes rows the lookup reads: it waits for the lookup
            if mode == "breakdown":
                mark("sparse_prepare")
                D.dlrm_embbag_bwd_sgd_prepare(w.K, w.rows, idx, off, w.B, nnz, model.ws_sparse)
            prep_stream.wait_stream(stream)

        def sparse_apply(Gs, on_side):
            """The sums and the update: long segments on the stream that ran
            the prepare (or the first one), short ones on the third stream."""
            s0 = prep_stream if on_side else stream
            if not on_side:
                stream.wait_stream(prep_stream)
            light_stream.wait_stream(s0)
            D.dlrm_embbag_bwd_sgd_apply(model.table_ptrs, w.K, d, w.rows, w.B, nnz, Gs, n * d, d, w.lr,
                                        model.ws_sparse, stream=s0, side=light_stream)
            s0.wait_stream(light_stream)

        if w.train:
            fork_prepare()
        if args.chain:
            return chain_step(model, dense, idx, off, y, nnz, mark, ev, mode, after_lookup, sparse_apply, overlap)
        mark("bottom_mlp")
        D.dlrm_mlp_fwd(dense, dense.shape[1], w.B, model.bottom.dims, model.bottom.Ws, model.bottom.w_ld,
                       model.bottom.biases, model.bottom.w_dtype, D.DLRM_ACT_RELU, model.x0, model.x0_ld, None,
                       model.ws_bot, w.train)
        if model.use_fused(nnz):
            mark("embbag_interact")
            if lp == "f32":
                D.dlrm_embbag_interact_fwd(model.x0, model.x0_ld, model.table_ptrs, w.K, d, idx, off, w.B,
                                           model.top_in, model.top_ld)
            else:
                D.dlrm_embbag_interact_fwd_lp(model.x0, model.x0_ld, model.table_ptrs, model.table_code, model.sb_ptrs,
                                              w.K, d, idx, off, w.B, model.top_in, model.top_ld)
            if w.train:
                after_lookup()
        else:
            mark("embbag")
            if lp == "f32":
                D.dlrm_embbag_fwd(model.table_ptrs, w.K, d, idx, off, w.B, model.X, n * d, d, nnz=nnz)
            else:
                D.dlrm_embbag_fwd_lp(model.table_ptrs, model.table_code, model.sb_ptrs, w.K, d, idx, off, w.B, model.X,
                                     n * d, d, nnz=nnz)
            if w.train:
                after_lookup()
            mark("interact")
            D.dlrm_interact_fwd(model.X, w.B, n, d, n * d, model.top_in, model.top_ld)
        if mode == "breakdown" and not w.train and bf16:
            top_layers(model, mark)
        else:
            mark("top_mlp")
            D.dlrm_mlp_fwd(model.top_in, model.top_ld, w.B, model.top.dims, model.top.Ws, model.top.w_ld,
                           model.top.biases, model.top.w_dtype, D.DLRM_ACT_NONE, model.logit, 1, model.prob,
                           model.ws_top, w.train)
        if w.train:
            if overlap:
                sparse_apply(G, True)  # needs only the prepared segments and G
            mark("dense_bwd")
            D.dlrm_bce_grad(model.logit, 1, y, w.B, model.dlogit)
            D.dlrm_mlp_bwd(w.B, model.top.dims, model.top.Ws, model.top.w_ld, D.DLRM_ACT_NONE, model.ws_top,
                           model.logit, 1, model.dlogit, 1, model.dW_top, model.db_top, None, 0, model.ws_top_bwd)
            D.dlrm_mlp_bwd(w.B, model.bottom.dims, model.bottom.Ws, model.bottom.w_ld, D.DLRM_ACT_RELU,
                           model.ws_bot, model.x0, model.x0_ld, G, n * d, model.dW_bot, model.db_bot, None, 0,
                           model.ws_bot_bwd)
            if not overlap:
                mark("sparse_bwd_sgd")
                sparse_apply(G, False)
            else:
                stream.wait_stream(prep_stream)
        mark("end")
        record(ev, mode)

    layer_bufs = {}

    LAYER_REPS = 4

    def fused_pair_at(dims):
        """Index of the hidden layer that dlrm_mlp_fwd runs together with the
        single-output layer (at most 256 hidden outputs), or None."""
        L = len(dims) - 1
        return L - 2 if L >= 2 and dims[L] == 1 and dims[L - 1] <= 256 else None

    def top_layers(m, mark):
        """The forward top MLP one layer at a time (dlrm_linear_fwd: the
        kernels dlrm_mlp_fwd launches for it; the last hidden layer and the
        single-output layer together through dlrm_mlp_fwd, which runs them as
        one launch), each launched LAYER_REPS times back to back between two
        marks (a layer only reads its input, so every launch does the same
        work), which spreads the cost of an event record over several
        launches."""
        dims = m.top.dims
        pair = fused_pair_at(dims)
        if not layer_bufs:
            for l in range(1, len(dims) - 1):
                ld = (dims[l] + 7) // 8 * 8
                layer_bufs[l] = (torch.empty((w.B, ld), dtype=torch.bfloat16, device=dev), ld)
            if pair is not None:
                sub = dims[pair:]
                layer_bufs["ws"] = torch.empty((max(256, D.dlrm_mlp_workspace_size(w.B, sub, D.DLRM_BF16, False)),),
                                               dtype=torch.uint8, device=dev)
        src, ld_src = m.top_in, m.top_ld
        for l in range(len(dims) - 1):
            mark(f"top_l{l}")
            if l == pair:
                for _ in range(LAYER_REPS):
                    D.dlrm_mlp_fwd(src, ld_src, w.B, dims[l:], m.top.Ws[l:], m.top.w_ld[l:], m.top.biases[l:],
                                   D.DLRM_BF16, D.DLRM_ACT_NONE, m.logit, 1, m.prob, layer_bufs["ws"], False)
                break
            last = l == len(dims) - 2
            dst, ld_dst = (m.logit, 1) if last else layer_bufs[l + 1]
            for _ in range(LAYER_REPS):
                D.dlrm_linear_fwd(src, ld_src, m.top.Ws[l], m.top.w_ld[l], m.top.biases[l], dst, ld_dst, w.B,
                                  dims[l + 1], dims[l], D.DLRM_ACT_NONE if last else D.DLRM_ACT_RELU)
            src, ld_src = dst, ld_dst

    def record(ev, mode):
        if mode is not None:
            names = list(ev)
            for a, b in zip(names[:-1], names[1:]):
                (call_t if mode == "breakdown" else dom_t).setdefault(a, []).append((ev[a], ev[b]))

    def chain_step(m, dense, idx, off, y, nnz, mark, ev, mode, after_lookup, sparse_apply, overlap):
        """Forward with X materialised, then the backward from the loss (the
        sparse update, once the X gradient exists, beside the bottom MLP's
        backward)."""
        n, d, B = m.n, m.d, w.B
        mark("bottom_mlp")
        D.dlrm_mlp_fwd(dense, dense.shape[1], B, m.bottom.dims, m.bottom.Ws, m.bottom.w_ld, m.bottom.biases,
                       m.bottom.w_dtype, D.DLRM_ACT_RELU, m.x0, m.x0_ld, None, m.ws_bot, True)
        mark("embbag")
        D.dlrm_embbag_fwd(m.table_ptrs, w.K, d, idx, off, B, m.X, n * d, d, nnz=nnz)
        after_lookup()
        mark("interact")
        D.dlrm_interact_fwd(m.X, B, n, d, n * d, m.top_in, m.top_ld)
        mark("top_mlp")
        D.dlrm_mlp_fwd(m.top_in, m.top_ld, B, m.top.dims, m.top.Ws, m.top.w_ld, m.top.biases, m.top.w_dtype,
                       D.DLRM_ACT_NONE, m.logit, 1, m.prob, m.ws_top, True)
        mark("top_bwd")
        D.dlrm_bce_grad(m.logit, 1, y, B, m.dlogit)
        D.dlrm_mlp_bwd(B, m.top.dims, m.top.Ws, m.top.w_ld, D.DLRM_ACT_NONE, m.ws_top, m.logit, 1, m.dlogit, 1,
                       m.dW_top, m.db_top, m.g_top, m.top_w, m.ws_top_bwd)
        mark("interact_bwd")
        D.dlrm_interact_bwd(m.X, B, n, d, n * d, m.g_top, m.top_w, m.G, n * d)
        if overlap:
            prep_stream.wait_stream(stream)  # the X gradient
            sparse_apply(m.G, True)
        mark("bottom_bwd")
        D.dlrm_mlp_bwd(B, m.bottom.dims, m.bottom.Ws, m.bottom.w_ld, D.DLRM_ACT_RELU, m.ws_bot, m.x0, m.x0_ld,
                       m.G, n * d, m.dW_bot, m.db_bot, None, 0, m.ws_bot_bwd)
        if overlap:
            stream.wait_stream(prep_stream)
        else:
            mark("sparse_bwd_sgd")
            sparse_apply(m.G, False)
        mark("end")
        record(ev, mode)

    breakdown_done = 0
    if model is not None and args.breakdown_steps > 0:
        # the per-call breakdown pass (untimed): two plain steps first, so
        # the host is ahead of the GPU when the first bracketed call starts
        for i in range(2):
            step(i, None)
        tb = time.perf_counter()
        while breakdown_done < args.breakdown_steps or time.perf_counter() - tb < args.breakdown_seconds:
            step(2 + breakdown_done, "breakdown")
            breakdown_done += 1
            if breakdown_done % 50 == 0:
                torch.cuda.synchronize()  # keep the host within 50 steps of the GPU
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, "timed")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_per_step = 1e3 * elapsed / args.steps
    value = w.B * args.steps / elapsed
    breakdown = {k: float(np.median([a.elapsed_time(b) for a, b in v])) / (LAYER_REPS if k.startswith("top_l") else 1)
                 for k, v in call_t.items()}
    nnz_mean = float(np.mean([b[5] for b in dbatches]))
    dom_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in dom_t.items()}
    if model is None or "embbag" in dom_ms:
        kname, key = "embbag_fwd_kernel", None
        gbytes = gather_bytes(w.K, w.B, w.d, nnz_mean, lp)
        g_ms = gather_t.mean_ms() if model is None else dom_ms["embbag"]
    else:
        # fused pooled lookup + interaction: every looked-up row, indices and
        # offsets, the dense rows it reads and the packed top-MLP rows it writes
        kname, key = "fused_kernel", "embbag_interact"
        esz = model.top_in.element_size()
        # the kernel writes d + P values and zeros up to the next multiple of 8
        row_out = min((model.top_w + 7) // 8 * 8, model.top_ld)
        gbytes = (gather_bytes(w.K, w.B, w.d, nnz_mean, lp) - 4 * w.K * w.B * w.d + 4 * w.B * w.d +
                  esz * w.B * row_out)
        g_ms = dom_ms[key]
    achieved = gbytes / (g_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name + ("_uniform" if args.uniform else "") + ("_chain" if args.chain else "") +
                               ("" if lp == "f32" else "_" + lp), kname)
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": int(gbytes), "avg_launch_ms": round(g_ms, 4)}
    if traffic is not None:
        # the bytes HBM really moved (Zipf rows repeat and hit in cache)
        roofline["hbm_measured_GBs"] = round(traffic / (g_ms * 1e-3) / 1e9, 1)
        roofline["hbm_measured_frac"] = round(traffic / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    # matrix cores: algorithmic MLP flops over the HIP-event time of the calls
    mfma = None
    if model is not None and w.mlp_dtype == "bf16":
        def frac(flops, ms):
            tf = flops / (ms * 1e-3) / 1e12
            return {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        mfma = {"peak_tflops": BF16_PEAK_TFLOPS}
        bflops = mlp_layer_flops(w.B, w.bottom)
        if "bottom_mlp" in breakdown:
            mfma["bottom_mlp"] = dict(frac(sum(bflops), breakdown["bottom_mlp"]), dims="-".join(map(str, w.bottom)))
        tdims = model.top.dims
        tflops = mlp_layer_flops(w.B, w.top)  # the model's own widths (a padded first layer's zero columns excluded)
        layers = []
        pair = fused_pair_at(tdims)
        for l in range(len(tdims) - 1):
            if f"top_l{l}" in breakdown:
                if l == pair:  # the last hidden layer and the logit layer in one launch
                    layers.append(dict(frac(tflops[l] + tflops[l + 1], breakdown[f"top_l{l}"]),
                                       layer=f"{w.top[l]}->{w.top[l + 1]}->{w.top[l + 2]}", k_run=tdims[l]))
                else:
                    layers.append(dict(frac(tflops[l], breakdown[f"top_l{l}"]), layer=f"{w.top[l]}->{w.top[l + 1]}",
                                       k_run=tdims[l]))
        if layers:
            mfma["top_layers"] = layers
            tot = sum(breakdown[k] for k in breakdown if k.startswith("top_l"))
            mfma["top_mlp"] = frac(sum(tflops), tot)
        elif "top_mlp" in breakdown:
            mfma["top_mlp"] = frac(sum(tflops), breakdown["top_mlp"])
        if "dense_bwd" in breakdown:
            # weight gradients of every layer, input gradients of every layer but the first of each MLP
            fl = 2 * sum(bflops) - bflops[0] + 2 * sum(tflops) - tflops[0]
            mfma["dense_bwd"] = frac(fl, breakdown["dense_bwd"])

    cpu = None
    if not args.no_cpu_baseline:
        ns = args.cpu_samples or {"forward": 16384, "embbag": 16384, "interaction": 512, "train": 1024,
                                  "tiny": 128}[w.name]
        S, dt, thr, passes = cpu_baseline(w, batches, bottom, top, ns, chain=args.chain, table_dtype=lp)
        S1, dt1, _, passes1 = cpu_baseline_single(w, batches, bottom, top, max(1, ns // max(thr, 1)),
                                                  chain=args.chain, table_dtype=lp)
        what = {"forward": "forward pass", "embbag": "pooled lookups", "interaction": "forward pass",
                "train": "forward pass and sparse SGD update", "tiny": "forward pass"}[w.name]
        if args.chain:
            what = "forward pass and the whole backward from the loss with the sparse SGD update"
        if lp != "f32":
            what += f" from {lp} rows"
        cpu = {"value": round(S / dt, 2), "unit": "samples/s", "cores": thr, "kind": "oracle",
               "sample": f"{what} of the first {S // passes} samples of batch 0, repeated {passes} times "
                         f"({dt:.1f} s; tables regenerated for the touched rows only, outside the timed region)",
               "threads": thr, "host_cores": host_cores(),
               "single_thread": {"value": round(S1 / dt1, 2), "unit": "samples/s",
                                 "sample": f"the first {S1 // passes1} samples, repeated {passes1} times "
                                           f"({dt1:.1f} s, one thread)"}}

    cfg = {"workload": w.name, "batch": w.B, "tables": w.K, "d": w.d, "rows_total": int(sum(w.rows)),
           "bag": f"{w.bag}:{w.bag_len}", "index": f"{w.index_dist}" + (f"({w.alpha})" if w.index_dist == "zipf" else ""),
           "bottom_mlp": "-".join(map(str, w.bottom)), "top_mlp": "-".join(map(str, w.top)),
           "mlp_dtype": w.mlp_dtype, "table_dtype": lp, "batches_rotated": args.batches}
    if w.train:
        cfg["upstream_grad"] = "from the loss (interaction backward)" if args.chain else "synthetic G"
    res = {"metric": METRIC, "value": round(value, 1), "unit": "samples/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32+bf16" if w.mlp_dtype == "bf16" else "f32", "data": "synthetic",
           "config": cfg, "roofline": roofline, "mfma": mfma, "cpu_baseline": cpu,
           "breakdown_ms": {k: round(v, 4) for k, v in breakdown.items()},
           "breakdown_steps": breakdown_done, "setup_s": round(t_setup, 1)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
