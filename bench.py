#!/usr/bin/env python3
"""LOCKS decode-step benchmark on one MI355X.

One step = the whole decode hot path for every layer: page scoring from the
summaries, GQA-shared top-k selection and split-K sparse attention, replayed
from one HIP graph.  The default workload is the 1M-token, 32-layer
Llama-3.1-8B-shaped cache (batch 1, 32 query / 8 KV heads, 2048-token
budget); the 32K single-layer workload is timed beside it.  Inputs are
synthetic and resident in HBM before timing starts.

Printed: one JSON line with microseconds per decode step per layer (the
headline), the scorer's and the attention kernel's achieved HBM bandwidth
(algorithmic bytes / kernel time, HIP events on the launch stream), the
dense-attention comparator on the same KV, summary-build throughput and the
CPU oracle timed on a bounded sample.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LOCKS decode-step µs/layer + achieved HBM GB/s (% of peak), 32K–1M ctx"
PEAK_HBM_GBS = 8000.0                 # MI355X HBM3E
SCORE_BYTES_PER_PAGE_HEAD = 832 + 16  # record read + 4 fp32 page LSEs written
ATTEND_BYTES_PER_PAGE_HEAD = 8192     # 16 tokens x 128 dims x bf16, K and V
EXACT_BYTES_PER_PAGE_HEAD = 4096 + 16 # keys of a page-head read + 4 fp32 page LSEs written
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_llama8b-1m_traffic.json")
SCORE_SRC = os.path.join(ROOT, "kv_cache_page_int4_amd", "csrc", "score.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b-1m")
    ap.add_argument("--small-workload", default="llama8b-32k")
    ap.add_argument("--large-workload", default="llama8b-256k-b16",
                    help="large-batch configuration reported beside the main one")
    ap.add_argument("--no-large", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (128K x 8, shuffled tables, seeds)")
    ap.add_argument("--no-finalize", action="store_true",
                    help="skip the finalization-inclusive step timing")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads for the all-core oracle timing (0: this process's cores, "
                         "at most 16)")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--shuffled", action="store_true",
                    help="main workload with a shuffled block table (pages at random blocks)")
    ap.add_argument("--seed", type=int, default=None, help="override the workload seed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the layer-wide selection-table variant")
    ap.add_argument("--no-small", action="store_true")
    ap.add_argument("--no-build", action="store_true", help="skip the summary-build timing")
    ap.add_argument("--no-quality", action="store_true",
                    help="skip the read-every-key comparator and the quality report")
    ap.add_argument("--quality-layers", type=int, default=4,
                    help="layers sampled for the quality report")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="also run a plain 1 GiB copy kernel (byte-counter calibration)")
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="timed replays of the graph of per-layer scorer / attention launches "
                         "(median reported)")
    return ap.parse_args()


def warm_graph(g, min_reps=3, min_seconds=0.025):
    """Replay a freshly captured graph until at least `min_reps` replays and
    `min_seconds` of wall time have passed.  The first replays of a new graph
    run slower before the launches settle (the scorer's 32 launches at 1M:
    77-83 us per launch over the first 5 to 9 replays, then 74-75 us), so
    timing starts after that."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < min_reps or time.perf_counter() - t0 < min_seconds:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    return n


def timed(fn, reps):
    """Average ms of fn() replayed from a captured graph (device time, not host
    launch rate), HIP events on the launch stream, after warm_graph."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    warm_graph(g)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / reps


def timed_replays(fn, reps):
    """ms of each of `reps` replays of fn() captured in one graph, each replay
    between its own pair of HIP events on the launch stream, after
    warm_graph."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    warm_graph(g)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    del g
    return [a.elapsed_time(b) for a, b in ev]


def replay_times(step, n):
    """ms of each of n graph replays, each bracketed by its own pair of events."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        a.record()
        step.replay()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def setup(w, build=True):
    import torch
    from kv_cache_page_int4_amd import locks as L
    from kv_cache_page_int4_amd.step import build_all_layers
    from synth.device import generate_device

    t0 = time.time()
    inp = generate_device(w)
    torch.cuda.synchronize()
    log(f"[{w.name}] inputs on device in {time.time() - t0:.1f}s "
        f"(KV {2 * inp.k.numel() * 2 / 2**30:.1f} GiB)")
    d = L.dims(w.hq, w.hkv)
    summ = torch.empty((w.layers, w.hkv, w.num_blocks, L.summary_bytes(d)), dtype=torch.uint8,
                       device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    build_all_layers(d, inp.k, summ)
    e1.record()
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    log(f"[{w.name}] summaries built: {w.layers * w.num_blocks * w.hkv} page-heads in {build_ms:.1f} ms")
    return d, inp, summ, build_ms


def time_step(step, steps, warmup):
    import torch
    step.capture()
    for _ in range(warmup):
        step.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, summ, budget, threads):
    """The oracle on every KV head of sequence 0 in layer 0, scaled to a layer
    by the number of sequences (exact for batch 1), timed twice: on one core
    and with one thread per KV head on up to `threads` cores (numpy releases
    the interpreter lock inside its array operations).  Each KV head: score
    its summary records, the GQA share, the top-k, then attention over the
    selected pages (their keys and values copied from the device between the
    two timed phases)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle as O

    n = w.pages
    G = w.group
    blk = inp.block_table[0, :n].cpu().numpy()
    blk_t = inp.block_table[0, :n].long()
    recs = [summ[0, g].index_select(0, blk_t).cpu().numpy() for g in range(w.hkv)]
    qbits = [inp.q[0, 0, g * G:(g + 1) * G].contiguous().view(torch.int16).cpu().numpy()
             .view(np.uint16) for g in range(w.hkv)]

    def select(g):
        q = O.bf16_to_f64(qbits[g])
        s = O.score_records(q, recs[g])
        _, log_m, _ = O.group_mass(s)
        return O.select_top_pages(log_m, budget)

    def gather(sels):
        out = []
        for g, sel in enumerate(sels):
            ids = torch.as_tensor(blk[sel], device="cuda").long()
            kb = inp.k[0][ids, g:g + 1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            vb = inp.v[0][ids, g:g + 1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            row = np.full(n + 1, -1, dtype=np.int64)
            row[sel] = np.arange(len(sel))
            out.append((kb, vb, row, sel))
        return out

    def attend(g, kv):
        kb, vb, row, sel = kv
        O.sparse_attention(O.bf16_to_f64(qbits[g]), kb, vb, row, 0, sel, n * w.page)

    def run(nthreads):
        with threadpool_limits(1):
            t = time.perf_counter()
            if nthreads == 1:
                sels = [select(g) for g in range(w.hkv)]
            else:
                with ThreadPoolExecutor(nthreads) as ex:
                    sels = list(ex.map(select, range(w.hkv)))
            t_sel = time.perf_counter() - t
        kvs = gather(sels)
        with threadpool_limits(1):
            t = time.perf_counter()
            if nthreads == 1:
                for g in range(w.hkv):
                    attend(g, kvs[g])
            else:
                with ThreadPoolExecutor(nthreads) as ex:
                    list(ex.map(attend, range(w.hkv), kvs))
            t_att = time.perf_counter() - t
        return t_sel + t_att, sum(len(x) for x in sels)

    t1, n_att = run(1)
    threads = min(threads, w.hkv)     # one task per KV head: more threads would sit idle
    tn, _ = run(threads) if threads > 1 else (t1, n_att)
    scale = f", scaled x{w.batch} (sequences) to one layer" if w.batch > 1 else ""
    sample = (f"layer 0, sequence 0, all {w.hkv} KV heads of {w.name}: score {n} summary "
              f"records per KV head, GQA share, top-{budget}, attend {n_att} pages in all; "
              f"{tn:.2f} s on {threads} threads (one KV head each), {t1:.2f} s on one core"
              f"{scale}")
    return {"value": tn * w.batch * 1e6, "unit": "us/layer", "cores": threads, "kind": "oracle",
            "sample": sample, "cpu_model": _cpu_model(),
            "one_core": {"value": t1 * w.batch * 1e6, "unit": "us/layer", "cores": 1}}


def cpu_build_baseline(w, inp, threads, n_sample=16384):
    """The oracle's summary build (bf16 decode, page spectrum, quantization,
    packing) on the first n_sample pages of KV head 0, layer 0, sequence 0,
    timed on one core and split into equal runs of pages over `threads`
    threads.  Returns page-heads per second for both."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle as O

    n = min(n_sample, w.pages)
    blk = inp.block_table[0, :n].long()
    kb = inp.k[0][blk, 0].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def build(lo_hi):
        lo, hi = lo_hi
        O.build_records(O.bf16_to_f64(kb[lo:hi]), w.rank)

    with threadpool_limits(1):
        t = time.perf_counter()
        build((0, n))
        t1 = time.perf_counter() - t
        edges = np.linspace(0, n, threads + 1).astype(int)
        t = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(build, zip(edges[:-1], edges[1:])))
        tn = time.perf_counter() - t
    return {"page_heads_per_s": n / tn, "cores": threads,
            "one_core_page_heads_per_s": n / t1,
            "sample": (f"{n} page-heads (layer 0, sequence 0, KV head 0 of {w.name}): "
                       f"{tn:.2f} s on {threads} threads ({n // threads} pages each), "
                       f"{t1:.2f} s on one core")}


def quality_report(w, d, inp, summ, step, budget, n_layers, kernel_reps, light=False):
    """The read-every-key comparator and the selection quality of LOCKS
    against it: exact page LSE from the true keys (locks_exact_page_lse),
    the exact top-k from it (locks_select_pages), recall of the LOCKS page
    sets, retention of the planted carrier pages by both selectors, and the
    key-deviation energy captured by the rank-r bases (GPU builder's
    unquantized output on sampled page-heads).  light=True leaves out the
    shared-basis selector."""
    import torch
    from kv_cache_page_int4_amd import locks as L

    P = inp.block_table.shape[1]
    lse = torch.empty((w.batch, w.hq, P), dtype=torch.float32, device="cuda")

    def exact_all_layers():
        for layer in range(w.layers):
            L.exact_page_lse(d, inp.q[layer], inp.k[layer], inp.block_table, inp.seq_lens, lse)

    exact_ms = timed(exact_all_layers, kernel_reps) / w.layers
    page_heads = w.batch * w.hkv * w.pages
    exact_gbs = page_heads * EXACT_BYTES_PER_PAGE_HEAD / (exact_ms * 1e-3) / 1e9

    ws = torch.empty(L.score_workspace_bytes(d, w.batch, P, budget), dtype=torch.uint8,
                     device="cuda")
    sel_x = torch.empty((w.batch, w.hkv, budget), dtype=torch.int32, device="cuda")
    cnt_x = torch.empty((w.batch, w.hkv), dtype=torch.int32, device="cuda")
    layers = sorted(set(int(round(i * (w.layers - 1) / max(1, n_layers - 1)))
                        for i in range(min(n_layers, w.layers))))
    inter = tot = inter_sh = 0
    car_locks = car_exact = car_both = car_n = 0
    # the shared-basis selector: one pooled basis per (layer, KV head) over
    # every finalized page, summaries in it, then the same scorer and selection
    if not light:
        fin = torch.cat([inp.block_table[b, :int(inp.seq_lens[b]) // w.page]
                         for b in range(w.batch)]).unique().to(torch.int32)
        basis = torch.empty((w.hkv, 8, 128), dtype=torch.float32, device="cuda")
        eig = torch.empty((w.hkv, 128), dtype=torch.float32, device="cuda")
        summ_sh = torch.empty((w.hkv, w.num_blocks, L.summary_bytes(d)), dtype=torch.uint8,
                              device="cuda")
    sel_sh = torch.empty_like(sel_x)
    cnt_sh = torch.empty_like(cnt_x)
    energy_sh = []
    shared_ms = []
    # exact attention mass captured, at the configured budget and at others:
    # the page shares m_j of the true-key page LSE (each query head's softmax
    # over pages, averaged over its group), summed over the pages LOCKS
    # selects and over the exact top-k pages (the most any k pages hold)
    budgets = sorted({bb for bb in (16, 32, 64, 128, 256, 512, budget) if bb <= w.pages})
    ws_b = torch.empty(L.score_workspace_bytes(d, w.batch, P, max(budgets)), dtype=torch.uint8,
                       device="cuda")
    mass = {bb: [0.0, 0.0, 0, 0] for bb in budgets}   # locks mass, exact mass, overlap, exact count

    def share_of_pages(sel_t, cnt_t, m_t):
        idx = sel_t.long().clamp_min(0)
        keep = torch.arange(sel_t.shape[-1], device="cuda")[None, None, :] < cnt_t[..., None]
        return (m_t.gather(2, idx) * keep).sum(dim=2)

    for layer in layers:
        L.exact_page_lse(d, inp.q[layer], inp.k[layer], inp.block_table, inp.seq_lens, lse)
        L.select_pages(d, lse, inp.seq_lens, budget, sel_x, cnt_x, ws)
        m_ex = torch.softmax(lse.double().view(w.batch, w.hkv, w.group, P), dim=-1).mean(dim=2)
        for bb in budgets:
            s_l = torch.empty((w.batch, w.hkv, bb), dtype=torch.int32, device="cuda")
            c_l = torch.empty((w.batch, w.hkv), dtype=torch.int32, device="cuda")
            s_e, c_e = torch.empty_like(s_l), torch.empty_like(c_l)
            L.score_select(d, inp.q[layer], summ[layer], w.num_blocks, inp.block_table,
                           inp.seq_lens, bb, s_l, c_l, ws_b)
            L.select_pages(d, lse, inp.seq_lens, bb, s_e, c_e, ws_b)
            mass[bb][0] += float(share_of_pages(s_l, c_l, m_ex).sum())
            mass[bb][1] += float(share_of_pages(s_e, c_e, m_ex).sum())
            for b in range(w.batch):
                for g in range(w.hkv):
                    a = set(s_l[b, g, :int(c_l[b, g])].tolist())
                    e = set(s_e[b, g, :int(c_e[b, g])].tolist())
                    mass[bb][2] += len(a & e)
                    mass[bb][3] += len(e)
        del m_ex
        torch.cuda.synchronize()
        if not light:
            t0 = time.perf_counter()
            L.shared_basis(d, inp.k[layer], fin, basis, eigvals=eig)
            torch.cuda.synchronize()
            shared_ms.append((time.perf_counter() - t0) * 1e3)
            L.build_summaries_basis(d, inp.k[layer], fin, basis, summ_sh)
            L.score_select(d, inp.q[layer], summ_sh, w.num_blocks, inp.block_table, inp.seq_lens,
                           budget, sel_sh, cnt_sh, ws)
            ev = eig.double()
            energy_sh.append(float((ev[:, :8].sum(dim=1) / ev.clamp_min(0).sum(dim=1)).mean()))
        sl = step.sel[layer].cpu().numpy()
        cl = step.cnt[layer].cpu().numpy()
        sx = sel_x.cpu().numpy()
        cx = cnt_x.cpu().numpy()
        ss = sel_sh.cpu().numpy() if not light else None
        cs = cnt_sh.cpu().numpy() if not light else None
        for b in range(w.batch):
            for g in range(w.hkv):
                a = set(sl[b, g, :cl[b, g]].tolist())
                e = set(sx[b, g, :cx[b, g]].tolist())
                inter += len(a & e)
                tot += len(e)
                if not light:
                    inter_sh += len(set(ss[b, g, :cs[b, g]].tolist()) & e)
        for (lay, b, g, page, _slot, _head) in inp.carriers:
            if lay != layer:
                continue
            car_n += 1
            in_l = page in set(sl[b, g, :cl[b, g]].tolist())
            in_x = page in set(sx[b, g, :cx[b, g]].tolist())
            car_locks += int(in_l)
            car_exact += int(in_x)
            car_both += int(in_l and in_x)
    # energy captured on sampled page-heads of layer 0
    n_smp = min(w.num_blocks, 2048)
    blocks = torch.randperm(w.num_blocks, device="cuda")[:n_smp].to(torch.int32)
    raw = torch.empty((n_smp, w.hkv, 1280), dtype=torch.float32, device="cuda")
    tmp = torch.empty((w.hkv, w.num_blocks, L.summary_bytes(d)), dtype=torch.uint8, device="cuda")
    L.build_summaries(d, inp.k[0], blocks, tmp, raw_debug=raw)
    K = inp.k[0].index_select(0, blocks.long()).float()              # [n, hkv, 16, 128]
    X = K - raw[:, :, None, :128]
    C = raw[:, :, 1152:].reshape(n_smp, w.hkv, 16, 8)
    energy = float(((C * C).sum(dim=(2, 3)) / (X * X).sum(dim=(2, 3)).clamp_min(1e-30)).mean())
    del tmp, raw, K, X
    rep = {"exact_us_per_layer": round(exact_ms * 1e3, 3),
           "exact_scorer_gbs": round(exact_gbs, 1),
           "exact_scorer_frac": round(exact_gbs / PEAK_HBM_GBS, 4),
           "recall_vs_exact": inter / max(tot, 1),
           "carrier_retention_locks": car_locks / max(car_n, 1),
           "carrier_retention_exact": car_exact / max(car_n, 1),
           "carriers_kept_by_both": car_both, "carriers_kept_by_exact": car_exact,
           "carriers": car_n, "layers_sampled": layers,
           "energy_captured_rank8": round(energy, 4),
           "by_budget": {str(bb): {"recall_vs_exact": round(v[2] / max(v[3], 1), 4),
                                   "exact_mass_captured": round(v[0] / max(v[1], 1e-300), 4),
                                   "exact_mass_of_exact_topk": round(v[1] / (len(layers) * w.batch * w.hkv), 4)}
                         for bb, v in mass.items()},
           "note": ("exact = top-k from the true-key page LSE (reads every key); recall = "
                    "fraction of the exact page set LOCKS also selects; carriers kept by exact "
                    "selection are the ones LOCKS can be asked to keep; by_budget (pages): "
                    "exact_mass_captured = the true-key attention mass (page shares averaged "
                    "over a group's query heads) on the pages LOCKS selects, over the mass on "
                    "the exact top-k pages; exact_mass_of_exact_topk = the latter per (sequence, "
                    "KV head), out of 1")}
    if not light:
        del summ_sh
        rep["shared_basis"] = {
            "recall_vs_exact": inter_sh / max(tot, 1),
            "energy_captured_rank8": round(sum(energy_sh) / len(energy_sh), 4),
            "basis_ms_per_layer": round(sum(shared_ms) / len(shared_ms), 2),
            "note": ("one rank-8 basis per (layer, KV head) from the pooled page deviations, "
                     "same record size, scorer and selection")}
    return rep


def traffic_if_current(workload):
    """Counter-measured HBM bytes per scorer launch, when the stored counters
    were taken on this workload and on the current score.hip."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
        sha = hashlib.sha256(open(SCORE_SRC, "rb").read()).hexdigest()
        if rec.get("score_hip_sha256") != sha:
            return None
        if str(rec.get("workload", "")).split(" ")[0] != workload:
            return None
        return rec.get("hbm_bytes_per_launch")
    except Exception:
        return None


def kernel_rates(w, d, inp, summ, step, budget, reps):
    """The scorer and the stand-alone attention (with its split merge), each
    timed in isolation from one captured graph of every layer's launch, back
    to back (each layer's launch repeated so that a graph holds at least 16
    launches), on its launch stream: `reps` replays, each between its own
    pair of HIP events.  Returns a dict: the mean microseconds per launch
    over all replays (and p10 / p50 / p90 of the replays' own means), GB/s
    from the algorithmic bytes (848 per scored page-head, 8192 per attended
    page-head), and the selected page-heads per layer."""
    import torch
    from kv_cache_page_int4_amd import locks as L

    P = inp.block_table.shape[1]
    lse_buf = torch.empty((w.batch, w.hq, P), dtype=torch.float32, device="cuda")

    rounds = -(-16 // w.layers)   # passes over the layers per replay
    launches = rounds * w.layers

    def score_all_layers():
        for _ in range(rounds):
            for layer in range(w.layers):
                L.score_pages(d, inp.q[layer], summ[layer], w.num_blocks, inp.block_table,
                              inp.seq_lens, lse_buf, step.ws_score)

    def attend_all_layers():
        for _ in range(rounds):
            for layer in range(w.layers):
                L.sparse_attend(d, inp.q[layer], inp.k[layer], inp.v[layer], inp.block_table,
                                inp.seq_lens, step.sel[layer], step.cnt[layer], budget,
                                step.out[layer], step.ws_att)

    def per_launch_us(fn):
        import numpy as np
        us = np.array(timed_replays(fn, reps)) * 1e3 / launches
        p10, p50, p90 = np.percentile(us, [10, 50, 90])
        return float(us.mean()), [round(float(x), 3) for x in (p10, p50, p90)]

    score_us, score_pct = per_launch_us(score_all_layers)
    attend_us, attend_pct = per_launch_us(attend_all_layers)
    page_heads = w.batch * w.hkv * w.pages
    att_units = int(step.cnt.sum().item()) / w.layers
    del lse_buf
    return {"score_us": score_us, "score_us_p10_p50_p90": score_pct,
            "score_gbs": page_heads * SCORE_BYTES_PER_PAGE_HEAD / (score_us * 1e-6) / 1e9,
            "attend_us": attend_us, "attend_us_p10_p50_p90": attend_pct,
            "attend_gbs": att_units * ATTEND_BYTES_PER_PAGE_HEAD / (attend_us * 1e-6) / 1e9,
            "att_units": att_units, "launches": launches * reps}


def finalize_timing(w, d, inp, summ, budget, steps, ms_plain):
    """The step with incremental finalization, in both forms: "step" (the
    pages the step's token completed are summarized after the step, all
    layers in one launch, with the newest page pending during it) and "layer"
    (each layer's page is summarized before that layer is scored).  Each is
    timed with the sequence lengths a multiple of 16 (every layer builds one
    page per sequence and KV head: a step in which a page completes) and one
    token shorter (nothing to build: the other 15 steps of 16).  The
    amortized cost is (completing + 15 x other) / 16 against the plain step."""
    import torch
    from kv_cache_page_int4_amd.step import DecodeStep

    short = (inp.seq_lens - 1).contiguous()
    plain2 = DecodeStep(d, inp.k, inp.v, summ, inp.q, inp.block_table, short, budget)
    ms_plain2 = time_step(plain2, steps, 2)
    del plain2
    base = (ms_plain + 15 * ms_plain2) / 16
    res = {"plain_step_us_per_layer": round(ms_plain * 1e3 / w.layers, 3),
           "plain_step_one_token_short_us_per_layer": round(ms_plain2 * 1e3 / w.layers, 3)}
    for mode in ("step", "layer"):
        fin = DecodeStep(d, inp.k, inp.v, summ, inp.q, inp.block_table, inp.seq_lens, budget,
                         finalize=mode)
        ms_done = time_step(fin, steps, 2)
        del fin
        fin2 = DecodeStep(d, inp.k, inp.v, summ, inp.q, inp.block_table, short, budget,
                          finalize=mode)
        ms_other = time_step(fin2, steps, 2)
        del fin2
        torch.cuda.synchronize()
        amort = (ms_done + 15 * ms_other) / 16
        res["after_step" if mode == "step" else "per_layer"] = {
            "completing_step_us_per_layer": round(ms_done * 1e3 / w.layers, 3),
            "other_step_us_per_layer": round(ms_other * 1e3 / w.layers, 3),
            "amortized_extra_us_per_step": round((amort - base) * 1e3, 3)}
    res["note"] = ("after_step: the pages a step's token completes are summarized after the "
                   "step, every layer in one launch, and the step runs with the newest page "
                   "pending (attended in full); per_layer: each layer's page is summarized "
                   "after the layer's newest key and before its scorer.  completing = every "
                   "sequence's newest token completes a page (one page per sequence, KV head "
                   "and layer is summarized), other = nothing to build")
    return res


def config_entry(name, args, dense=False, quality_layers=0, finalize=False, cpu=False,
                 **overrides):
    """Step time, scorer and attention bandwidth (and optionally the dense
    comparator, the quality report and the finalization cost) of one more
    configuration, set up after the previous one's buffers are freed."""
    import torch
    from kv_cache_page_int4_amd.step import DecodeStep
    from synth import get_workload

    wl = get_workload(name, **overrides)
    d3, inp3, summ3, _ = setup(wl)
    st3 = DecodeStep(d3, inp3.k, inp3.v, summ3, inp3.q, inp3.block_table, inp3.seq_lens,
                     wl.budget_pages)
    ms3 = time_step(st3, max(10, args.steps // 2), 2)
    kr = kernel_rates(wl, d3, inp3, summ3, st3, wl.budget_pages, args.kernel_reps)
    sc_us, sc_gbs, at_us, at_gbs = kr["score_us"], kr["score_gbs"], kr["attend_us"], kr["attend_gbs"]
    entry = {"us_per_layer": round(ms3 * 1e3 / wl.layers, 3),
             "scorer_us": round(sc_us, 3), "scorer_gbs": round(sc_gbs, 1),
             "scorer_frac": round(sc_gbs / PEAK_HBM_GBS, 4),
             "attention_us": round(at_us, 3), "attention_gbs": round(at_gbs, 1),
             "attention_frac": round(at_gbs / PEAK_HBM_GBS, 4),
             "batch": wl.batch, "ctx": wl.ctx, "layers": wl.layers, "seed": wl.seed,
             "shuffled_blocks": wl.shuffled_blocks}
    log(f"[{wl.name}{' shuffled' if wl.shuffled_blocks else ''} seed {wl.seed}] decode step "
        f"{entry['us_per_layer']:.2f} us/layer; scorer {sc_us:.2f} us = {sc_gbs:.0f} GB/s; "
        f"attention {at_us:.2f} us = {at_gbs:.0f} GB/s")
    if dense:
        dn3 = DecodeStep(d3, inp3.k, inp3.v, summ3, inp3.q, inp3.block_table, inp3.seq_lens,
                         1, dense=True)
        dms3 = time_step(dn3, max(2, min(args.steps, 20)), 1)
        entry["dense_us_per_layer"] = round(dms3 * 1e3 / wl.layers, 3)
        entry["speedup_vs_dense"] = round(dms3 / ms3, 3)
        log(f"[{wl.name}] dense {dms3 * 1e3 / wl.layers:.2f} us/layer, "
            f"speedup {dms3 / ms3:.2f}x")
        del dn3
    if finalize:
        entry["finalize"] = finalize_timing(wl, d3, inp3, summ3, wl.budget_pages,
                                            max(10, args.steps // 2), ms3)
        log(f"[{wl.name}] finalization: { {k: v for k, v in entry['finalize'].items() if k != 'note'} }")
    if quality_layers:
        entry["quality"] = quality_report(wl, d3, inp3, summ3, st3, wl.budget_pages,
                                          quality_layers, args.kernel_reps, light=True)
        q = entry["quality"]
        log(f"[{wl.name}] recall vs exact {q['recall_vs_exact']:.4f}; carriers kept: LOCKS "
            f"{q['carrier_retention_locks']:.3f}, exact {q['carrier_retention_exact']:.3f}, both "
            f"{q['carriers_kept_by_both']}/{q['carriers_kept_by_exact']} of those exact keeps")
    if cpu and not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
        entry["cpu_baseline"] = cpu_baseline(wl, inp3, summ3, wl.budget_pages, threads)
        c = entry["cpu_baseline"]
        log(f"[{wl.name}] oracle {c['value']:.0f} us/layer on {c['cores']} threads, "
            f"{c['one_core']['value']:.0f} us/layer on one core")
    del st3, inp3, summ3
    torch.cuda.empty_cache()
    return entry


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: the LOCKS decode path here runs on a single MI355X.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from kv_cache_page_int4_amd import locks as L
    from kv_cache_page_int4_amd.step import DecodeStep
    from synth import get_workload

    torch.cuda.set_device(0)
    w = get_workload(args.workload)
    if args.layers:
        w = w.with_(layers=args.layers)
    if args.shuffled:
        w = w.with_(shuffled_blocks=True)
    if args.seed is not None:
        w = w.with_(seed=args.seed)
    d, inp, summ, build_ms = setup(w)
    budget = w.budget_pages

    step = DecodeStep(d, inp.k, inp.v, summ, inp.q, inp.block_table, inp.seq_lens, budget)
    torch.cuda.synchronize()
    ms_step = time_step(step, args.steps, args.warmup)
    us_layer = ms_step * 1e3 / w.layers
    log(f"[{w.name}] decode step {ms_step:.3f} ms = {us_layer:.2f} us/layer "
        f"({args.steps} timed replays)")
    # spread of single replays, each between its own pair of events (after the
    # timed region, so that the value above is untouched by the extra events)
    per_replay = replay_times(step, args.steps)
    pct = np.percentile(np.array(per_replay) * 1e3 / w.layers, [10, 50, 90])
    step_spread = {"p10": round(float(pct[0]), 3), "p50": round(float(pct[1]), 3),
                   "p90": round(float(pct[2]), 3), "replays": len(per_replay)}
    log(f"[{w.name}] single replays: p10 {pct[0]:.2f}, median {pct[1]:.2f}, p90 {pct[2]:.2f} us/layer")

    # --- dominant kernel: the scorer, timed in isolation on the launch stream ---
    kr = kernel_rates(w, d, inp, summ, step, budget, args.kernel_reps)
    score_us, score_gbs = kr["score_us"], kr["score_gbs"]
    attend_us, attend_gbs, att_units = kr["attend_us"], kr["attend_gbs"], kr["att_units"]
    page_heads = w.batch * w.hkv * w.pages
    log(f"[{w.name}] scorer {score_us:.2f} us/launch = {score_gbs:.0f} GB/s; "
        f"attention {attend_us:.2f} us/launch = {attend_gbs:.0f} GB/s")

    extra = {}
    if not args.no_finalize:
        extra["finalize"] = finalize_timing(w, d, inp, summ, budget, max(10, args.steps // 2),
                                            ms_step)
        log(f"[{w.name}] finalization: { {k: v for k, v in extra['finalize'].items() if k != 'note'} }")

    if not args.no_dense:
        dense = DecodeStep(d, inp.k, inp.v, summ, inp.q, inp.block_table, inp.seq_lens, 1,
                           dense=True)
        dense_ms = time_step(dense, max(2, min(args.steps, 20)), 1)
        extra["dense_us_per_layer"] = dense_ms * 1e3 / w.layers
        extra["speedup_vs_dense"] = dense_ms / ms_step
        dense_bytes = w.batch * w.hkv * w.pages * ATTEND_BYTES_PER_PAGE_HEAD
        extra["dense_attention_gbs"] = dense_bytes / (dense_ms * 1e-3 / w.layers) / 1e9
        locks_bytes = page_heads * 832 + att_units * ATTEND_BYTES_PER_PAGE_HEAD
        extra["kv_bytes_ratio_dense_over_locks"] = dense_bytes / locks_bytes
        log(f"[{w.name}] dense {extra['dense_us_per_layer']:.2f} us/layer, "
            f"speedup {extra['speedup_vs_dense']:.2f}x")
        del dense

    # variant: one selection table for the whole layer (all query heads share
    # one page set) -- its step time and how much of each KV head's own page
    # set it keeps
    if not args.no_variants:
        wide = DecodeStep(d, inp.k, inp.v, summ, inp.q, inp.block_table, inp.seq_lens, budget,
                          n_tables=1)
        wide_ms = time_step(wide, max(2, args.steps // 2), 1)
        keep = []
        for layer in range(w.layers):
            for b in range(w.batch):
                c1 = int(wide.cnt[layer, b, 0])
                s1 = set(wide.sel[layer, b, 0, :c1].tolist())
                for g in range(w.hkv):
                    c = int(step.cnt[layer, b, g])
                    own = set(step.sel[layer, b, g, :c].tolist())
                    keep.append(len(own & s1) / max(len(own), 1))
        extra["variants"] = {"layer_wide_table": {
            "us_per_layer": round(wide_ms * 1e3 / w.layers, 3),
            "own_pages_kept": round(sum(keep) / len(keep), 4),
            "note": ("one table per layer over all query heads (the wider reading of the "
                     "group-shared table); "
                     "own_pages_kept = mean fraction of a KV head's own top-k pages that the "
                     "layer-wide table also selects")}}
        log(f"[{w.name}] layer-wide table {wide_ms * 1e3 / w.layers:.2f} us/layer; keeps "
            f"{extra['variants']['layer_wide_table']['own_pages_kept']:.3f} of each KV head's "
            f"own pages")
        del wide

    # variant: summary ranks 4 and 16 (the same step at other state sizes) on
    # the first layers: step time per layer and recall against exact selection
    if not args.no_variants:
        nl = min(w.layers, 4)
        P = inp.block_table.shape[1]
        lse_x = torch.empty((w.batch, w.hq, P), dtype=torch.float32, device="cuda")
        ws_x = torch.empty(L.score_workspace_bytes(d, w.batch, P, budget), dtype=torch.uint8,
                           device="cuda")
        sel_x = torch.empty((nl, w.batch, w.hkv, budget), dtype=torch.int32, device="cuda")
        cnt_x = torch.empty((nl, w.batch, w.hkv), dtype=torch.int32, device="cuda")
        for layer in range(nl):
            L.exact_page_lse(d, inp.q[layer], inp.k[layer], inp.block_table, inp.seq_lens, lse_x)
            L.select_pages(d, lse_x, inp.seq_lens, budget, sel_x[layer], cnt_x[layer], ws_x)
        ranks = {}
        for r in (4, 16):
            dr = L.dims(w.hq, w.hkv, rank=r)
            summ_r = torch.empty((nl, w.hkv, w.num_blocks, L.summary_bytes(dr)),
                                 dtype=torch.uint8, device="cuda")
            blocks = torch.arange(w.num_blocks, dtype=torch.int32, device="cuda")
            for layer in range(nl):
                L.build_summaries(dr, inp.k[layer], blocks, summ_r[layer])
            st_r = DecodeStep(dr, inp.k[:nl], inp.v[:nl], summ_r, inp.q[:nl], inp.block_table,
                              inp.seq_lens, budget)
            ms_r = time_step(st_r, max(4, args.steps // 2), 2)
            inter = tot = 0
            for layer in range(nl):
                for b in range(w.batch):
                    for g in range(w.hkv):
                        c = int(st_r.cnt[layer, b, g])
                        cx = int(cnt_x[layer, b, g])
                        a = set(st_r.sel[layer, b, g, :c].tolist())
                        e = set(sel_x[layer, b, g, :cx].tolist())
                        inter += len(a & e)
                        tot += len(e)
            ranks[f"rank{r}"] = {"us_per_layer": round(ms_r * 1e3 / nl, 3),
                                 "record_bytes": L.summary_bytes(dr),
                                 "recall_vs_exact": inter / max(tot, 1), "layers": nl}
            log(f"[{w.name}] rank {r}: {ms_r * 1e3 / nl:.2f} us/layer, recall vs exact "
                f"{inter / max(tot, 1):.4f} ({L.summary_bytes(dr)} B records)")
            del st_r, summ_r
        extra.setdefault("variants", {}).update(ranks)
        del lse_x, ws_x

    # achievable streaming-read bandwidth (context for the roofline)
    from synth.device import device_read
    rbuf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4 * 8192, dtype=torch.int32, device="cuda")
    read_ms = timed(lambda: device_read(rbuf, sink), 5)
    stream_read_gbs = rbuf.numel() / (read_ms * 1e-3) / 1e9
    del rbuf, sink
    log(f"streaming read of 2 GiB: {stream_read_gbs:.0f} GB/s")

    if args.copy_calibrate:
        from synth.device import device_copy
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        device_copy(dst, src)
        torch.cuda.synchronize()
        del src, dst

    quality = None
    if not args.no_quality:
        quality = quality_report(w, d, inp, summ, step, budget, args.quality_layers,
                                 args.kernel_reps)
        log(f"[{w.name}] read-every-key scorer {quality['exact_us_per_layer']:.1f} us/layer = "
            f"{quality['exact_scorer_gbs']:.0f} GB/s; recall vs exact "
            f"{quality['recall_vs_exact']:.4f}; carriers kept: LOCKS "
            f"{quality['carrier_retention_locks']:.3f}, exact {quality['carrier_retention_exact']:.3f}; "
            f"energy captured {quality['energy_captured_rank8']:.3f}; shared basis: recall "
            f"{quality['shared_basis']['recall_vs_exact']:.4f}, energy "
            f"{quality['shared_basis']['energy_captured_rank8']:.3f}")

    cpu = None
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
        cpu = cpu_baseline(w, inp, summ, budget, threads)
        log(f"[{w.name}] oracle {cpu['value']:.0f} us/layer on {cpu['cores']} threads, "
            f"{cpu['one_core']['value']:.0f} us/layer on one core ({cpu['cpu_model']})")
        cpu["build"] = cpu_build_baseline(w, inp, threads)
        log(f"[{w.name}] oracle build {cpu['build']['page_heads_per_s']:.0f} page-heads/s on "
            f"{threads} threads, {cpu['build']['one_core_page_heads_per_s']:.0f} on one core")

    also = {}
    del step, inp, summ
    torch.cuda.empty_cache()
    if not args.no_configs:
        # the main workload with a shuffled block table (records and K/V pages
        # at random physical blocks), then seeds 1 and 2
        also[f"{w.name}-shuffled"] = config_entry(args.workload, args, shuffled_blocks=True)
        for seed in (1, 2):
            also[f"{w.name}-seed{seed}"] = config_entry(args.workload, args, seed=seed)
    if not args.no_large and args.large_workload:
        also[args.large_workload] = config_entry(
            args.large_workload, args, dense=not args.no_dense,
            quality_layers=0 if args.no_quality else 2, cpu=True)
    if not args.no_configs:
        also["llama8b-128k-b8"] = config_entry("llama8b-128k-b8", args,
                                               quality_layers=0 if args.no_quality else 2,
                                               cpu=True)
    if not args.no_small and args.small_workload:
        ent = config_entry(args.small_workload, args, dense=not args.no_dense,
                           quality_layers=0 if args.no_quality else 1,
                           finalize=not args.no_finalize, cpu=True)
        ent["note"] = "working set fits the 256 MB Infinity Cache; latency-bound"
        also[args.small_workload] = ent
        if not args.no_configs:
            for seed in (1, 2):
                also[f"{args.small_workload}-seed{seed}"] = config_entry(
                    args.small_workload, args, quality_layers=0 if args.no_quality else 1,
                    seed=seed)

    traffic = traffic_if_current(w.name)
    result = {
        "metric": METRIC,
        "value": round(us_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "us_per_layer_single_replays": step_spread,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "batch": w.batch, "ctx": w.ctx,
                   "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d, "page": w.page,
                   "rank": w.rank, "budget_tokens": w.budget_tokens,
                   "carriers_per_kv_head": w.carriers, "seed": w.seed,
                   "shuffled_blocks": w.shuffled_blocks,
                   "graph": "one hipGraph per step"},
        "roofline": {"bound": "hbm", "achieved": round(score_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(score_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": "score_kernel",
                     "traffic_gbs": (round(traffic / (score_us * 1e-6) / 1e9, 1)
                                     if traffic else None),
                     "kernel_us": round(score_us, 3),
                     "kernel_us_replays_p10_p50_p90": kr["score_us_p10_p50_p90"],
                     "launches_timed": kr["launches"],
                     "bytes_per_launch": page_heads * SCORE_BYTES_PER_PAGE_HEAD,
                     "timing": ("mean over graph replays of every layer's "
                                "locks_score_pages launch, back to back, each replay between "
                                "its own HIP events on the launch stream, after at least 25 ms "
                                "of warm-up replays of the same graph")},
        "attention": {"achieved": round(attend_gbs, 1), "unit": "GB/s",
                      "frac": round(attend_gbs / PEAK_HBM_GBS, 4),
                      "kernel_us": round(attend_us, 3),
                      "kernel_us_replays_p10_p50_p90": kr["attend_us_p10_p50_p90"],
                      "note": ("attention + split merge, selected K/V bytes only; "
                               f"{att_units * ATTEND_BYTES_PER_PAGE_HEAD / 2**20:.1f} MiB per "
                               "layer is latency-bound, see also.*.attention_gbs for the "
                               "large-batch rate")},
        "stream_read_gbs": round(stream_read_gbs, 1),
        "pages_scored_per_s": page_heads / (score_us * 1e-6),
        "build_page_heads_per_s": w.layers * w.num_blocks * w.hkv / (build_ms * 1e-3),
        "cpu_baseline": cpu,
        "quality": quality,
    }
    result.update(extra)
    if also:
        result["also"] = also
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
