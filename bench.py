#!/usr/bin/env python3
"""MLA decode throughput on one MI355X: tokens/s and achieved latent-cache
HBM bandwidth.

One step is the whole hot path over one batch: append the new tokens' rows
to the paged latent cache, fold the queries into latent space, split-KV
attention over the cache, merge the splits and project out through W_uv.
Inputs are synthetic and seeded, already resident in HBM when timing starts.
R copies of {cache, folded weights} (>= 1 GiB together) are used in turn so
that the 256 MB last-level cache cannot serve a step from the previous one.

Workloads of kind "extend" (long new chunks: chunked extend, prefill) time
append + mla_extend instead, by the form --path names (default: the
library's choice) and report matrix-core throughput.

Prints one JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--path P]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode tokens/s and achieved latent-cache HBM GB/s (% of peak), 1 GPU"
EXTEND_METRIC = "MLA chunked-extend / prefill query tokens/s and matrix-core TFLOP/s, 1 GPU"

# HBM bytes per split-KV launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled
# by the same counters on a 256 MiB device copy (x2.000 and x1.000), keyed by
# the kernel source they were taken on and the workload (profiles/ holds the
# runs).  A changed kernel reports null until counters are taken again.
MEASURED_TRAFFIC = {
    ("8d4c951127b547e1", "dsv2_b32_ctx4096"): {"fetch_bytes": 155951825, "write_bytes": 16842763},
    ("8d4c951127b547e1", "llama2_7b_mla_b64_ctx8192"): {"fetch_bytes": 606661307, "write_bytes": 8421376},
    ("8d4c951127b547e1", "dsv2_b8_ctx131072"): {"fetch_bytes": 1210617024, "write_bytes": 35258368},
    ("8d4c951127b547e1", "dsv2_ragged_paged_256"): {"fetch_bytes": 5128679836, "write_bytes": 124757703},
    ("8d4c951127b547e1", "dsv2_b32_ctx4096_fp8"): {"fetch_bytes": 89418305, "write_bytes": 16842865},
}


ATTENTION_SOURCES = ("attn_tile.hpp", "splitkv.hip", "splitkv_x8.hip", "splitkv_r128.hip")


EXTEND_SOURCES = ("attn_tile.hpp", "extend.hip")
# HBM bytes of one mla_extend call (both expanded kernels), measured as above.
EXTEND_TRAFFIC = {
    ("ebb2cf6b8e183b98", "dsv2_extend_b4_p3072_c1024"): {
        "fetch_bytes": 2560137011, "write_bytes": 1207989350,
        "per_kernel": {"expand_kv": {"fetch_bytes": 1248185549, "write_bytes": 1073741824},
                       "extend_attn": {"fetch_bytes": 1311951462, "write_bytes": 134247526}}},
}


def extend_source_id():
    """Hash of the expanded extend kernels' sources."""
    import hashlib
    h = hashlib.sha256()
    for name in EXTEND_SOURCES:
        with open(os.path.join(ROOT, "mla_compressed_latent_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def splitkv_source_id():
    """Hash of the attention kernels' sources (the counters below are valid
    for exactly this code)."""
    import hashlib
    h = hashlib.sha256()
    for name in ATTENTION_SOURCES:
        with open(os.path.join(ROOT, "mla_compressed_latent_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix throughput, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv2_b32_ctx4096")
    ap.add_argument("--kv-chunk", type=int, default=0, help="tokens per split (0 = library's choice)")
    ap.add_argument("--rotate", type=int, default=0, help="buffer copies (0 = enough for >= 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mall-warm", action="store_true",
                    help="also time steps that all reuse cache copy 0 (last-level cache may hold it)")
    ap.add_argument("--attention-rows", type=int, default=0, choices=(0, 64, 128),
                    help="split-KV rows per workgroup (0 = the library's choice by shape)")
    ap.add_argument("--separate", action="store_true",
                    help="decode workloads: time mla_append_latent + mla_decode instead of mla_decode_step")
    ap.add_argument("--path", choices=("auto", "absorbed", "expanded"), default="auto",
                    help="form of mla_extend for extend workloads")
    ap.add_argument("--form", choices=("auto", "unfolded", "folded"), default="auto",
                    help="output projection form (project workloads) or query projection form (hidden)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_state(wl, kv_chunk, rotate, path="auto", form="auto", attention_rows=0):
    import numpy as np
    import torch

    import mla_compressed_latent_amd as mla

    s = wl.shape
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    dev = "cuda"

    def up(a, dtype=dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dtype)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).to(dev)

    cfg = mla.config_from_shape(s)
    w_dkv, w_uk, w_uv = up(wl.w_dkv()), up(wl.w_uk()), up(wl.w_uv())
    pool = None
    if wl.layers:
        # a layer stack: one host page pool assigns every sequence's pages, and
        # its table serves all layers' caches
        npg = wl.pages_per_seq()
        num_pages = int(npg.sum())
        pool = mla.PagePool(num_pages, s.page_size, wl.batch, int(npg.max()))
        for b, L in enumerate(wl.seq_lens()):
            pool.reserve(b, int(L))
        table_np = pool.page_table(list(range(wl.batch)))
    else:
        table_np, num_pages = wl.page_table()
    table = i32(table_np)
    prefix = wl.prefix_lens()
    q_lens = wl.q_lens()
    seq_lens_np = wl.seq_lens()
    B = wl.batch
    if s.cache_format == "fp8":   # pages of 640-byte rows, then the rows' fp32 scales
        cache0 = torch.empty((num_pages, s.page_size * s.cache_token_bytes), dtype=torch.uint8, device=dev)
    else:
        cache0 = torch.empty((num_pages, s.page_size, s.row_width), dtype=dt, device=dev)
    layer0 = mla.mla_fold_weights(cfg, w_dkv, w_uk, w_uv)

    t0 = time.time()
    ps = s.page_size
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        if wl.prefix_source == "hidden":
            group = 8
            for b0 in range(0, B, group):
                bs = list(range(b0, min(B, b0 + group)))
                xs = list(ex.map(wl.prefix_hidden, bs))
                cu = np.zeros(B + 1, np.int64)
                for j, b in enumerate(bs):
                    cu[b + 1] = xs[j].shape[0]
                x = up(np.concatenate(xs, axis=0))
                mla.mla_append_latent(layer0, x, i32(np.cumsum(cu)), i32(np.zeros(B)), table, cache0)
                torch.cuda.synchronize()
                del x, xs
        else:
            assert s.cache_format != "fp8", "fp8 caches are filled through the append path"
            futs = {b: ex.submit(wl.prefix_latent, b) for b in range(min(B, 16))}
            for b in range(B):
                if b + 16 < B:
                    futs[b + 16] = ex.submit(wl.prefix_latent, b + 16)
                rows = up(futs.pop(b).result())
                P = rows.shape[0]
                npg = (P + ps - 1) // ps
                if npg:
                    pages = torch.from_numpy(table_np[b, :npg].astype(np.int64)).to(dev)
                    padded = torch.zeros((npg * ps, s.row_width), dtype=dt, device=dev)
                    padded[:P] = rows
                    cache0[pages] = padded.view(npg, ps, s.row_width)
    torch.cuda.synchronize()
    log(f"prefix cache filled in {time.time() - t0:.1f}s ({wl.prefix_source} prefixes)")

    cache_bytes = cache0.numel() * cache0.element_size()
    folded_bytes = layer0.folded.numel()
    R = wl.layers or rotate or max(1, math.ceil((1 << 30) / (cache_bytes + folded_bytes)))
    layers, caches = [layer0], [cache0]
    for _ in range(R - 1):
        layers.append(mla.mla_fold_weights(cfg, w_dkv, w_uk, w_uv))
        caches.append(cache0.clone())
    if attention_rows:
        for layer in layers:
            mla.mla_layer_set_attention_rows(layer, attention_rows)
    out_form = q_form = None
    if wl.kind == "hidden":
        q_form = {"auto": mla.mla_query_choose_form(cfg, int(wl.q_lens().sum())),
                  "unfolded": mla.MLA_QUERY_UNFOLDED, "folded": mla.MLA_QUERY_FOLDED}[form]
        w_q = up(wl.w_q())
        for layer in layers:
            mla.mla_fold_query(layer, w_q, w_uk, q_form)
        del w_q
    if wl.kind == "project":
        out_form = {"auto": mla.mla_output_choose_form(cfg, int(wl.q_lens().sum())),
                    "unfolded": mla.MLA_OUTPUT_UNFOLDED, "folded": mla.MLA_OUTPUT_FOLDED}[form]
        w_o = up(wl.w_o())
        for layer in layers:
            mla.mla_fold_output(layer, w_uv, w_o, out_form)
        del w_o
    del w_dkv, w_uk, w_uv
    torch.cuda.synchronize()

    Tq = int(q_lens.sum())
    st = dict(
        mla=mla, s=s, dt=dt, layers=layers, caches=caches, R=R, table=table, B=B, Tq=Tq,
        q=up(wl.queries()), x_new=up(wl.new_hidden()), cu_q=i32(wl.cu_q()), prefix=i32(prefix),
        seq_lens=i32(seq_lens_np), seq_lens_np=seq_lens_np, max_q_len=int(q_lens.max()),
        max_seq_len=int(seq_lens_np.max()), kv_chunk=kv_chunk,
        out=torch.empty((Tq, s.H, s.d_v), dtype=dt, device=dev),
        cache_bytes=cache_bytes, folded_bytes=folded_bytes, cfg=cfg, pool=pool, out_form=out_form,
        q_form=q_form,
    )
    st["chunk"] = mla.mla_decode_kv_chunk(layer0, B, st["max_q_len"], st["max_seq_len"], kv_chunk)
    st["aws"] = torch.empty(max(1, mla.mla_append_workspace_bytes(layer0, Tq)), dtype=torch.uint8, device=dev)
    st["extend"] = wl.kind == "extend"
    st["hidden"] = wl.kind == "hidden"
    st["project"] = wl.kind in ("project", "hidden")   # both: graph replay of append + one call
    if st["hidden"]:
        st["dws"] = torch.empty(max(1, mla.mla_decode_hidden_workspace_bytes(
            layer0, B, Tq, st["max_q_len"], st["max_seq_len"])), dtype=torch.uint8, device=dev)
    elif st["project"]:
        st["y"] = torch.empty((Tq, s.d_model), dtype=dt, device=dev)
        st["dws"] = torch.empty(max(1, mla.mla_decode_project_workspace_bytes(
            layer0, B, Tq, st["max_q_len"], st["max_seq_len"])), dtype=torch.uint8, device=dev)
    elif st["extend"]:
        chosen = mla.mla_extend_choose_path(cfg, B, Tq, st["max_q_len"], st["max_seq_len"])
        st["auto_path"] = chosen
        st["path"] = {"auto": chosen, "absorbed": mla.MLA_EXTEND_ABSORBED,
                      "expanded": mla.MLA_EXTEND_EXPANDED}[path]
        n = max(mla.mla_extend_workspace_bytes(layer0, B, Tq, st["max_q_len"], st["max_seq_len"], p)
                for p in (mla.MLA_EXTEND_ABSORBED, mla.MLA_EXTEND_EXPANDED))
        st["dws"] = torch.empty(max(1, n), dtype=torch.uint8, device=dev)
    else:
        st["dws"] = torch.empty(max(1, mla.mla_decode_workspace_bytes(layer0, B, Tq, st["max_q_len"],
                                                                      st["max_seq_len"], kv_chunk)),
                                dtype=torch.uint8, device=dev)
        st["sws"] = torch.empty(max(1, mla.mla_decode_step_workspace_bytes(
            layer0, B, Tq, Tq, st["max_q_len"], st["max_seq_len"], kv_chunk)), dtype=torch.uint8, device=dev)
    return st


def run_step(st, i, ev=None, path=None):
    mla = st["mla"]
    r = i % st["R"]
    layer, cache = st["layers"][r], st["caches"][r]
    if st["project"]:
        if ev is not None:
            ev[0].record()
        mla.mla_append_latent(layer, st["x_new"], st["cu_q"], st["prefix"], st["table"], cache,
                              workspace=st["aws"])
        if ev is not None:
            ev[1].record()
        if st["hidden"]:
            mla.mla_decode_hidden(layer, st["x_new"], st["cu_q"], st["seq_lens"], st["table"], cache, st["out"],
                                  st["max_q_len"], st["max_seq_len"], workspace=st["dws"])
        else:
            mla.mla_decode_project(layer, st["q"], st["cu_q"], st["seq_lens"], st["table"], cache, st["y"],
                                   st["max_q_len"], st["max_seq_len"], workspace=st["dws"])
        if ev is not None:
            ev[2].record()
        return
    if st["extend"]:
        if ev is not None:
            ev[0].record()
        mla.mla_append_latent(layer, st["x_new"], st["cu_q"], st["prefix"], st["table"], cache,
                              workspace=st["aws"])
        if ev is not None:
            ev[1].record()
        mla.mla_extend(layer, st["q"], st["cu_q"], st["seq_lens"], st["table"], cache, st["out"],
                       st["max_q_len"], st["max_seq_len"], path=st["path"] if path is None else path,
                       workspace=st["dws"])
        if ev is not None:
            ev[2].record()
        return
    if ev is None and not st["separate"]:
        # the whole step in one call: the query absorb shares a launch with the append finish
        mla.mla_decode_step(layer, st["x_new"], st["cu_q"], st["prefix"], st["q"], st["cu_q"], st["seq_lens"],
                            st["table"], cache, st["out"], st["max_q_len"], st["max_seq_len"], st["kv_chunk"],
                            workspace=st["sws"])
        return
    args = (layer, st["q"], st["cu_q"], st["seq_lens"], st["table"], cache, st["out"], st["max_q_len"],
            st["max_seq_len"], st["kv_chunk"], st["dws"])
    if ev is not None:
        ev[0].record()
    mla.mla_append_latent(layer, st["x_new"], st["cu_q"], st["prefix"], st["table"], cache, workspace=st["aws"])
    if ev is not None:
        ev[1].record()
    mla.mla_decode_phases(*args, phases=mla.MLA_PHASE_ABSORB)
    if ev is not None:
        ev[2].record()
    mla.mla_decode_phases(*args, phases=mla.MLA_PHASE_ATTEND)
    if ev is not None:
        ev[3].record()
    mla.mla_decode_phases(*args, phases=mla.MLA_PHASE_OUTPUT)
    if ev is not None:
        ev[4].record()


def extend_flops(wl, seq_lens, expanded):
    """Matrix-core flops of one mla_extend call: causal key counts per query;
    the expanded form builds K and V for every cached token of every head and
    scores at width d_nope + d_rope + d_v, the absorbed form folds each query
    in and out of latent space and scores at width 2 d_c + d_rope."""
    s = wl.shape
    keys = 0.0
    for L, lq in zip(seq_lens, wl.q_lens()):
        L, lq = int(L), int(lq)
        keys += lq * (L - lq) + lq * (lq + 1) / 2.0
    Tq = float(wl.q_lens().sum())
    if expanded:
        expand = 2.0 * s.H * s.d_c * (s.d_nope + s.d_v) * float(sum(int(L) for L in seq_lens))
        return expand, 2.0 * s.H * (s.d_nope + s.d_rope + s.d_v) * keys
    fold = 2.0 * s.H * s.d_c * (s.d_nope + s.d_v) * Tq
    return fold, 2.0 * s.H * (2 * s.d_c + s.d_rope) * keys


def cpu_baseline(wl, budget_s):
    """The float64 oracle on whole sequences of the same workload, as many as
    fit in the time budget (at least one)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import fp8, mla_oracle

    s = wl.shape
    w_dkv, w_uk, w_uv = wl.w_dkv(), wl.w_uk(), wl.w_uv()
    scale = mla_oracle.default_scale(s.d_nope, s.d_rope)
    cores = min(16, os.cpu_count() or 1)
    done_q = 0
    elapsed = 0.0
    seqs = 0
    flops = 0.0
    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        for b in range(wl.batch):
            P = int(wl.prefix_lens()[b])
            if wl.prefix_source == "hidden":
                pre = mla_oracle.latent_rows(wl.prefix_hidden(b), w_dkv, np.arange(P), s.d_c, s.rope_base)
            else:
                pre = wl.prefix_latent(b).astype(np.float64)
            x_new, q = wl.new_hidden(b), wl.queries(b)
            t0 = time.perf_counter()
            new = mla_oracle.latent_rows(x_new, w_dkv, P + np.arange(x_new.shape[0]), s.d_c, s.rope_base)
            cache = np.concatenate([pre, new], axis=0)
            if s.cache_format == "fp8":
                cache = fp8.fp8_rows(cache, s.d_c)
            mla_oracle.attend_sequence(q, cache, w_uk, w_uv, s.H, s.d_nope, s.d_v, s.rope_base, scale)
            elapsed += time.perf_counter() - t0
            done_q += q.shape[0]
            seqs += 1
            # float64 work of that sample: latent rows of the new tokens, per-head
            # K and V materialised over the whole sequence, scores and sums
            L, lq = cache.shape[0], q.shape[0]
            flops += 2.0 * lq * s.d_model * (s.d_c + s.d_rope)
            flops += 2.0 * s.H * L * s.d_c * (s.d_nope + s.d_v)
            flops += 2.0 * lq * s.H * L * (s.d_nope + s.d_rope + s.d_v)
            if elapsed >= budget_s:
                break
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    blas = sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                   for i in threadpool_info() if i.get("user_api") == "blas"})
    return {
        "value": done_q / elapsed, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{seqs} of {wl.batch} sequences ({done_q} query tokens, all {s.H} heads), "
                  f"append + unabsorbed float64 attention, {elapsed:.1f}s",
        "seconds": elapsed, "fp64_gflop": flops / 1e9, "fp64_gflops_per_s": flops / elapsed / 1e9,
        "cpu_model": cpu_model, "host_cpus": os.cpu_count(), "blas": blas,
    }


def run_phase(st, r, phase):
    """One decode phase (mla_decode_phases) on rotated copy r."""
    mla = st["mla"]
    mla.mla_decode_phases(st["layers"][r], st["q"], st["cu_q"], st["seq_lens"], st["table"], st["caches"][r],
                          st["out"], st["max_q_len"], st["max_seq_len"], st["kv_chunk"], st["dws"], phases=phase)


def graph_phase_us(st, phase, replays):
    """Average launch time of one decode phase: a HIP graph holding the phase
    once on each of the R rotated copies, replayed back to back, timed with
    HIP events on the replay stream (the stream the kernels run on)."""
    import torch
    R = st["R"]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for r in range(R):
                run_phase(st, r, phase)
    torch.cuda.current_stream().wait_stream(cap)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * R)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the decode step runs on a single MI355X and multi-GPU runs are not part of this build.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from mla_synth import WORKLOADS

    wl = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    log(f"workload {wl.name}: {wl.description}")
    st = build_state(wl, args.kv_chunk, args.rotate, args.path, args.form, args.attention_rows)
    st["separate"] = args.separate
    if st["extend"] or st["project"]:
        return main_extend(args, wl, st)
    log(f"kv_chunk {st['chunk']}, {st['R']} rotated copies of cache ({st['cache_bytes'] / 1e6:.1f} MB) "
        f"+ folded weights ({st['folded_bytes'] / 1e6:.1f} MB)")

    for i in range(args.warmup):
        run_step(st, i)
    torch.cuda.synchronize()
    K = args.steps

    # Per-phase times, eager launches, HIP events on the launch stream.
    KP = min(K, 20)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(KP)]
    t_e0, t_e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_e0.record()
    for i in range(KP):
        run_step(st, args.warmup + i, evs[i])
    t_e1.record()
    torch.cuda.synchronize()
    eager_ms = t_e0.elapsed_time(t_e1) / KP
    phase = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / KP for j in range(4)]
    attend_each = sorted(e[2].elapsed_time(e[3]) for e in evs)

    # The timed steps run as HIP graphs, as a serving loop runs a decode
    # forward: the R rotated copies of {cache, folded weights} are R distinct
    # layers, and one graph holds one step of each, back to back (a graph
    # launch costs several microseconds, paid once per R steps here as it is
    # once per forward there).  Single-step graphs of the first copies make up
    # K when R does not divide it.  (One stream: running the append beside the
    # absorb phase on a second stream measured slower, the cross-queue
    # dependencies of the replayed graph costing more than the overlap gains.)
    R = st["R"]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all, stream=cap):
            for r in range(R):
                run_step(st, r)
        singles = []
        for r in range(K % R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                run_step(st, r)
            singles.append(g)
    torch.cuda.current_stream().wait_stream(cap)
    for i in range(max(1, args.warmup // R)):
        g_all.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(K // R + 1)]
    start.record()
    marks[0].record()
    for i in range(K // R):
        g_all.replay()
        marks[i + 1].record()
    for g in singles:
        g.replay()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) / R for i in range(K // R))

    def pct(v, q):
        return v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))] if v else None

    # With --mall-warm, the same steps with every step on copy 0: the 256 MB
    # last-level cache may then serve part of the cache from the previous
    # step.  Off by default, so that every kernel launch of a default run
    # (and of a profiler run of it) streams its cache copy from HBM.
    warm_ms_step = None
    if args.mall_warm:
        with torch.cuda.stream(cap):
            g_warm = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_warm, stream=cap):
                for r in range(R):
                    run_step(st, 0)
        torch.cuda.current_stream().wait_stream(cap)
        g_warm.replay()
        torch.cuda.synchronize()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        for i in range(max(1, K // R)):
            g_warm.replay()
        w1.record()
        torch.cuda.synchronize()
        warm_ms_step = w0.elapsed_time(w1) / (max(1, K // R) * R)
    # The attention kernel and the combine + output kernels on their own:
    # back-to-back launches in a graph, each on its own cache copy.
    mla = st["mla"]
    replays = max(2, K // R)
    attend_us = graph_phase_us(st, mla.MLA_PHASE_ATTEND, replays)
    output_us = graph_phase_us(st, mla.MLA_PHASE_OUTPUT, replays)
    s = st["s"]
    latent_bytes = int(st["seq_lens_np"].astype("int64").sum()) * s.cache_token_bytes
    attend_s = attend_us * 1e-6
    achieved = latent_bytes / attend_s / 1e9
    grading = latent_bytes / ((attend_us + output_us) * 1e-6) / 1e9
    # scores (K = d_c + d_rope) and value sums (K = d_c) per query row and cached token
    q_lens = wl.q_lens()
    traffic = MEASURED_TRAFFIC.get((splitkv_source_id(), wl.name))
    traffic_bytes = None if traffic is None else traffic["fetch_bytes"] + traffic["write_bytes"]
    flops = 2.0 * s.H * (2 * s.d_c + s.d_rope) * float(
        sum(int(L) * int(lq) for L, lq in zip(st["seq_lens_np"], q_lens)))
    res = {
        "metric": METRIC,
        "value": st["Tq"] * K / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded Gaussian hidden states / latent rows and weights)",
        "config": {
            "workload": wl.name, "batch": wl.batch, "query_tokens": st["Tq"],
            "max_context": st["max_seq_len"], "heads": s.H, "kv_lora_rank": s.d_c,
            "qk_rope_head_dim": s.d_rope, "kv_chunk": st["chunk"], "rotated_copies": st["R"],
            "attention_rows": args.attention_rows or "by shape",
        },
        "latent_cache_GBps": achieved,
        "latent_cache_frac_of_hbm_peak": achieved / HBM_PEAK_GBPS,
        "timing": ("HIP graph replay of whole steps ("
                   + ("mla_append_latent + mla_decode" if st["separate"] else
                      "mla_decode_step: append + decode, the query absorb and the append finish in one launch")
                   + "); one graph holds one step on each of the R rotated layer copies; phase_us and "
                   "eager_ms_per_step time the separate calls"),
        "ms_per_step_p10_p50_p90": [pct(per_step, 0.1), pct(per_step, 0.5), pct(per_step, 0.9)],
        "mall_warm_ms_per_step": warm_ms_step,
        "end_to_end_latent_GBps": latent_bytes / (ms_step * 1e-3) / 1e9,
        "eager_ms_per_step": eager_ms,
        "attend_us_p10_p50_p90": [pct(attend_each, q) * 1e3 for q in (0.1, 0.5, 0.9)],
        "phase_us": {"append": phase[0] * 1e3, "absorb": phase[1] * 1e3, "attend": phase[2] * 1e3,
                     "combine_and_output": phase[3] * 1e3},
        "kernel_us": {"attend": attend_us, "combine_and_output": output_us},
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic_bytes,
            "traffic_detail": traffic,
            "kernel": "split-KV attention (MLA_PHASE_ATTEND)",
            "timing": ("HIP events around a graph of back-to-back MLA_PHASE_ATTEND launches, one per rotated "
                       "copy (kernel_us.attend); phase_us are eager event times including launch gaps"),
            "grading_achieved": grading,
            "grading_frac": grading / HBM_PEAK_GBPS,
            "grading": "latent bytes / (split-KV attention + combine and W_uv output), both graph-timed",
            "algorithmic_bytes_per_launch": latent_bytes,
            "mfma_tflops": flops / attend_s / 1e12,
            "mfma_frac_of_bf16_peak": flops / attend_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        },
    }
    log(f"{ms_step * 1e3:.1f} us/step (graph), {eager_ms * 1e3:.1f} us/step eager, attend "
        f"{attend_us:.1f} us -> {achieved:.0f} GB/s ({100 * achieved / HBM_PEAK_GBPS:.1f}% of HBM peak); "
        f"attend + output {attend_us + output_us:.1f} us -> {100 * grading / HBM_PEAK_GBPS:.1f}%")
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    props = torch.cuda.get_device_properties(0)
    res["hardware"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                       "compute_units": props.multi_processor_count,
                       "memory_GB": round(props.total_memory / 1e9, 1)}
    if wl.layers:
        # one graph replay is one decode forward through every layer
        mla = st["mla"]
        fwd_ms = ms_step * wl.layers
        weights = st["folded_bytes"] * wl.layers
        res["stack"] = {
            "layers": wl.layers, "forward_ms": fwd_ms, "forward_tokens_per_s": wl.batch / (fwd_ms * 1e-3),
            "cache_GB": st["cache_bytes"] * wl.layers / 1e9, "folded_weights_GB": weights / 1e9,
            "page_table": "host page pool (mla_pool_*), one table for all layers",
            # sequences of this context the planner fits in the device memory left
            # after the folded weights (cache alone, as the capacity argument counts it)
            "planner_max_sequences": mla.mla_plan_max_sequences(
                st["cfg"], wl.layers, int(props.total_memory - weights), st["max_seq_len"]),
        }
    print(json.dumps(res), flush=True)


def main_project(args, wl, st):
    """Decode + output projection: graph replay of append + mla_decode_project."""
    import torch

    mla = st["mla"]
    s = st["s"]
    K = args.steps
    n = min(K, 10)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        run_step(st, i, evs[i])
    torch.cuda.synchronize()
    phase = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / n for j in range(2)]
    R = st["R"]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all, stream=cap):
            for r in range(R):
                run_step(st, r)
    torch.cuda.current_stream().wait_stream(cap)
    g_all.replay()
    torch.cuda.synchronize()
    reps = max(1, K // R)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(reps):
        g_all.replay()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / (reps * R)
    H, dc, dv, dm, dn, dr = s.H, s.d_c, s.d_v, s.d_model, s.d_nope, s.d_rope
    hidden = st["hidden"]
    if hidden:
        # query projection (with the absorb through W_uk when unfolded), then W_uv
        folded = st["q_form"] == mla.MLA_QUERY_FOLDED
        w_bytes = 2 * H * (dc + dr) * dm if folded else 2 * H * ((dn + dr) * dm + dn * dc)
        other = 2 * H * dc * dv
        call, form_key = "mla_decode_hidden", "query_form"
    else:
        folded = st["out_form"] == mla.MLA_OUTPUT_FOLDED
        w_bytes = 2 * H * dc * dm if folded else 2 * H * dv * (dc + dm)
        other = 2 * H * dc * dn
        call, form_key = "mla_decode_project", "output_form"
    latent = int(st["seq_lens_np"].astype("int64").sum()) * s.cache_token_bytes
    call_s = phase[1] * 1e-3
    achieved = (latent + w_bytes + other) / call_s / 1e9
    res = {
        "metric": ("MLA decode from the layer input tokens/s, 1 GPU" if hidden else
                   "MLA decode + output projection tokens/s, 1 GPU"), "value": st["Tq"] / (ms_step * 1e-3),
        "unit": "tokens/s", "n_gpus": 1, "steps": reps * R, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": s.dtype,
        "data": "synthetic (seeded Gaussian hidden states and weights)",
        "config": {"workload": wl.name, "batch": wl.batch, "query_tokens": st["Tq"],
                   "max_context": st["max_seq_len"], "heads": H, "d_model": dm,
                   form_key: "folded" if folded else "unfolded", "rotated_copies": R},
        "timing": f"HIP graph replay of whole steps (append + {call})",
        "phase_ms": {"append": phase[0], call[4:]: phase[1]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": f"{call} (all its kernels, HIP events around the call)",
                     "algorithmic_bytes_per_launch": latent + w_bytes + other,
                     "weights_streamed_bytes": w_bytes},
    }
    log(f"{ms_step * 1e3:.1f} us/step (graph); {call[4:]} {phase[1] * 1e3:.1f} us "
        f"({'folded' if folded else 'unfolded'}, weights {w_bytes / 1e6:.0f} MB)")
    print(json.dumps(res), flush=True)


def main_extend(args, wl, st):
    """Chunked extend / prefill: HIP-graph replay of append + mla_extend."""
    import torch

    mla = st["mla"]
    s = st["s"]
    names = {mla.MLA_EXTEND_ABSORBED: "absorbed", mla.MLA_EXTEND_EXPANDED: "expanded"}
    for i in range(args.warmup):
        run_step(st, i)
    torch.cuda.synchronize()
    K = args.steps
    if st["project"]:
        return main_project(args, wl, st)
    # eager per-phase times of both forms (the choice's evidence)
    path_ms = {}
    phase = None
    for p in (mla.MLA_EXTEND_ABSORBED, mla.MLA_EXTEND_EXPANDED):
        run_step(st, 0, path=p)
        n = min(K, 5)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            run_step(st, i, evs[i], path=p)
        torch.cuda.synchronize()
        ph = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / n for j in range(2)]
        path_ms[names[p]] = ph[1]
        if p == st["path"]:
            phase = ph
    R = st["R"]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all, stream=cap):
            for r in range(R):
                run_step(st, r)
        singles = []
        for r in range(K % R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                run_step(st, r)
            singles.append(g)
    torch.cuda.current_stream().wait_stream(cap)
    g_all.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K // R):
        g_all.replay()
    for g in singles:
        g.replay()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K
    expanded = st["path"] == mla.MLA_EXTEND_EXPANDED
    f_side, f_attn = extend_flops(wl, st["seq_lens_np"], expanded)
    ext_s = phase[1] * 1e-3
    tflops = (f_side + f_attn) / ext_s / 1e12
    res = {
        "metric": EXTEND_METRIC,
        "value": st["Tq"] * K / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded Gaussian hidden states and weights)",
        "config": {
            "workload": wl.name, "batch": wl.batch, "query_tokens": st["Tq"],
            "max_context": st["max_seq_len"], "heads": s.H, "kv_lora_rank": s.d_c,
            "path": names[st["path"]], "auto_path": names[st["auto_path"]], "rotated_copies": R,
        },
        "timing": "HIP graph replay of whole steps (append + mla_extend); one graph holds one step on "
                  "each of the R rotated layer copies",
        "phase_ms": {"append": phase[0], "extend": phase[1]},
        "extend_ms_by_path": path_ms,
        "roofline": {
            "bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": (None if not expanded or (extend_source_id(), wl.name) not in EXTEND_TRAFFIC else
                        EXTEND_TRAFFIC[(extend_source_id(), wl.name)]["fetch_bytes"] +
                        EXTEND_TRAFFIC[(extend_source_id(), wl.name)]["write_bytes"]),
            "traffic_detail": EXTEND_TRAFFIC.get((extend_source_id(), wl.name)) if expanded else None,
            "kernel": f"mla_extend ({names[st['path']]}: both of its kernels, HIP events around the call)",
            "algorithmic_flops_per_launch": f_side + f_attn,
            "flops_split": {"expand_or_fold": f_side, "attention": f_attn},
        },
    }
    log(f"{ms_step:.3f} ms/step (graph); extend {phase[1]:.3f} ms by the {names[st['path']]} form "
        f"-> {tflops:.0f} TFLOP/s ({100 * tflops / MFMA_BF16_PEAK_TFLOPS:.1f}% of bf16 peak); "
        f"by form: {path_ms}")
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    props = torch.cuda.get_device_properties(0)
    res["hardware"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                       "compute_units": props.multi_processor_count,
                       "memory_GB": round(props.total_memory / 1e9, 1)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
