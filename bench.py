"""Decode-step benchmark of the sparse paged MLA layer on one MI355X.

One step = dsa_indexer_scores -> topk_select -> mla_paged_decode -> lse_merge
(dense workloads: decode -> merge) on one HIP stream, every input resident in
HBM.  The default workload is the 64-request 32K-128K FP8 decode (c3f).

Timing: W untimed warm-up steps, then exactly K timed steps.  Before each
timed step a 512 MiB buffer is read (outside the timed events) so the step
starts with L2 and MALL holding unrelated clean lines, as after the other
layers of a model.  (An overwriting flush would leave dirty lines whose
write-back competes with the timed step.)  Each kernel is bracketed by HIP events on
the stream it runs on; the step time is the sum of its kernels' spans (start
of the first to end of the last).  `value` = requests / mean step time.
A warm number (K steps back to back, no flush) is reported beside it.

Prints ONE JSON line (rank 0).  Other workloads: --config c2|c3|c4|c5.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="c3f")
    ap.add_argument("--splits", type=int, default=0, help="KV splits (0: per-workload default)")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=-1,
                    help="requests in the CPU-oracle sample (-1: auto, 0: skip)")
    ap.add_argument("--profile-only", action="store_true",
                    help="no CPU baseline; adds one plain 256 MiB device copy (counter calibration) for rocprofv3")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE "
                         "rocprofv3 run of --profile-only into profiles/counters.json entries for --config, "
                         "and print them as a markdown table")
    return ap.parse_args()


# Kernel-name fragment -> source file whose HBM traffic it measures.
COUNTER_SOURCES = [("indexer_kernel", "indexer.hip"), ("topk_", "topk.hip"), ("mla_decode_f8ws", "mla_decode_f8.hip"),
                   ("mla_decode_bf16ws", "mla_decode_bf16.hip"), ("mla_decode_kernel", "mla_decode.hip"),
                   ("lse_merge", "lse_merge.hip"),
                   ("cache_append", "cache_append.hip")]
CALIB_BYTES = 256 << 20  # the plain device copy --profile-only adds


def summarize_counters(fetch_csv, write_csv, workload):
    """HBM bytes per launch of each kernel source from two rocprofv3 counter
    runs of `bench.py --profile-only` (FETCH_SIZE, then WRITE_SIZE, in KiB per
    dispatch), scaled by what the same counters read for the plain 256 MiB
    device copy; a source with several kernels per call (top-k) sums them."""
    import csv
    per = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                per.setdefault(r["Kernel_Name"], {}).setdefault(counter, []).append(float(r["Counter_Value"]))
    copies = per.get("__amd_rocclr_copyBuffer", {})
    rf = CALIB_BYTES / (max(copies["FETCH_SIZE"]) * 1024)
    wf = CALIB_BYTES / (max(copies["WRITE_SIZE"]) * 1024)
    recs = {}
    for name, c in per.items():
        src = next((f for frag, f in COUNTER_SOURCES if frag in name), None)
        if src is None or "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        fk, wk = statistics.fmean(c["FETCH_SIZE"]), statistics.fmean(c["WRITE_SIZE"])
        r = recs.setdefault(src, dict(fetch_kib=0.0, write_kib=0.0, kernels=[]))
        r["fetch_kib"] += fk
        r["write_kib"] += wk
        r["kernels"].append((name, fk, wk))
    p = os.path.join(ROOT, "profiles", "counters.json")
    allrec = json.load(open(p)) if os.path.exists(p) else {}
    w = allrec.setdefault(workload, {})
    print("| Kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | Calibrated HBM MB/launch |")
    print("|---|---|---|---|")
    print(f"| `__amd_rocclr_copyBuffer` (256 MiB calibration copy) | {max(copies['FETCH_SIZE']):.0f} | "
          f"{max(copies['WRITE_SIZE']):.0f} | {2 * CALIB_BYTES / 1e6:.1f} |")
    for src, r in sorted(recs.items()):
        for name, fk, wk in r["kernels"]:
            print(f"| `{name.split('(')[0]}` | {fk:.0f} | {wk:.0f} | {(fk * 1024 * rf + wk * 1024 * wf) / 1e6:.1f} |")
        w[src] = dict(source_sha=kernel_source_sha(src),
                      hbm_bytes_per_launch=int(r["fetch_kib"] * 1024 * rf + r["write_kib"] * 1024 * wf),
                      fetch_kib=r["fetch_kib"], write_kib=r["write_kib"], read_factor=rf, write_factor=wf,
                      summary=f"profiles/{workload}_step_hbm_traffic.md")
    print(f"\nread factor {rf:.3f}, write factor {wf:.3f}")
    json.dump(allrec, open(p, "w"), indent=1)


def algorithmic(cfg, lens):
    """Per-kernel algorithmic bytes and FLOPs of one step (what the method must move / compute)."""
    B, H, D, dc = cfg.batch, cfg.n_heads, cfg.dim, cfg.d_latent
    sumL = int(lens.sum())
    e_c = {0: 4, 1: 2, 2: 1}[cfg.cache_dtype]
    s_c = 4 if cfg.cache_dtype == 2 else 0
    e_q = {0: 4, 1: 2}[cfg.q_dtype]
    out = {}
    if cfg.dense:
        n_sel = sumL
        k = 0
    else:
        k = cfg.topk
        HI, dI = cfg.idx_heads, cfg.idx_dim
        e_k = {0: 4, 1: 2, 2: 1}[cfg.idx_dtype]
        s_k = 4 if cfg.idx_dtype == 2 else 0
        out["indexer"] = dict(bytes=sumL * (dI * e_k + s_k) + B * HI * (dI * e_q + 4) + 4 * sumL,
                              flops=2 * HI * dI * sumL)
        out["topk"] = dict(bytes=4 * sumL + 4 * B * k, flops=0)
        n_sel = int(sum(min(k, int(L)) for L in lens))
    out["decode"] = dict(bytes=n_sel * (D * e_c + s_c) + B * H * D * e_q + 4 * B * H * (dc + 1) + 4 * B * k,
                         flops=2 * H * (D + dc) * n_sel)
    out["merge"] = dict(bytes=0, flops=0)
    return out


def roofline_time_s(a):
    return sum(max(v["bytes"] / (HBM_PEAK_GBS * 1e9), v["flops"] / (BF16_PEAK_TFLOPS * 1e12)) for v in a.values())


def kernel_source_sha(name):
    """Hash of a kernel source together with the compiler flags it is built with."""
    from sparse_paged_mla_amd.build import FLAGS
    p = os.path.join(ROOT, "sparse_paged_mla_amd", "csrc", name)
    h = hashlib.sha256(open(p, "rb").read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_file, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this kernel source."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(workload, {}).get(kernel_file)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_sha(kernel_file):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_cache_append(cfg, db, inp, steps, flush, run_flush):
    """The step before the path: each request's new token row appended to the
    latent pool and its indexer key to the key pool, both quantised to FP8 on
    write (one kv_cache_append_pair launch, timed with HIP events on the
    launch stream, cold like the step).  Writes the requests' last slots."""
    import numpy as np
    import torch
    import spmla_gen as gen
    import sparse_paged_mla_amd as spm
    B = cfg.batch
    lat = np.stack([gen.normals32(cfg.seed, gen.T_NEW_KV, b, cfg.dim) for b in range(B)])
    key = np.stack([gen.normals32(cfg.seed, gen.T_NEW_KIDX, b, cfg.idx_dim) for b in range(B)])
    lat_t = torch.from_numpy(gen.to_bf16_bits(lat).view(np.int16)).view(torch.bfloat16).cuda()
    key_t = torch.from_numpy(gen.to_bf16_bits(key).view(np.int16)).view(torch.bfloat16).cuda()
    pos = (db.lens - 1).to(torch.int32)
    status = torch.zeros(B, dtype=torch.int32, device="cuda")

    def both():
        spm.kv_cache_append_pair(lat_t, db.kv, db.kv_scale, key_t, db.k_idx, db.k_idx_scale, db.block_table, pos,
                                 status)

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for _ in range(3):
        both()
    ts = []
    for e0, e1 in evs:
        if flush:
            run_flush()
        e0.record()
        both()
        e1.record()
    torch.cuda.synchronize()
    assert not status.cpu().numpy().any(), "append flagged a request on clean inputs"
    us = statistics.fmean(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3
    # Algorithmic bytes: the bf16 rows read, codes and scales written, and one
    # position and block-table entry read per request, for both pools.
    nbytes = B * (cfg.dim * 3 + 4 + cfg.idx_dim * 3 + 4 + 2 * 8)
    return {"us_per_step": round(us, 2), "calls": 1, "algorithmic_bytes": nbytes,
            "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 2),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 6),
            "note": "one launch of a few hundred bytes per request: launch- and latency-bound"}


def time_page_check(cfg, db, inp, steps, flush, run_flush, step=None):
    """The KV-page integrity check a server may run with the step (one
    kv_page_check call over every covered block-table entry), timed cold like
    the step: alone, and (with `step`) on a second stream of default priority
    beside the step, started when the indexer is done (the top-k launches
    leave most compute units idle; beside the indexer, whose grid fills the
    GPU, it added twice its own time) and waited for at the step's end (the
    check reads only block tables and tags, nothing the step writes, and its
    status bits mark the requests whose outputs to discard).  On c3f it still
    adds a little more than its own time (8.0 against 6.6 us): the
    cross-stream hand-off costs about what the overlap hides.  Tags: page p carries
    p * 0x9E3779B97F4A7C15 mod 2^64 (distinct for every page) and every entry
    records its page's tag."""
    import numpy as np
    import torch
    import sparse_paged_mla_amd as spm
    P = cfg.page_size
    page_tags = np.arange(inp.num_pages, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)
    bt = inp.block_table
    bt_tags = np.where(bt >= 0, page_tags[np.clip(bt, 0, None)], np.uint64(0)).astype(np.uint64)
    pt_t = torch.from_numpy(page_tags.view(np.int64)).cuda()
    bt_tags_t = torch.from_numpy(bt_tags.view(np.int64)).cuda()
    status = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")

    def check():
        spm.kv_page_check(db.block_table, bt_tags_t, db.lens, db.max_len, pt_t, P, status)

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for _ in range(3):
        check()
    for e0, e1 in evs:
        if flush:
            run_flush()
        e0.record()
        check()
        e1.record()
    torch.cuda.synchronize()
    assert not status.cpu().numpy().any(), "page check flagged a request on clean inputs"
    us = statistics.fmean(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3
    entries = int(((inp.lens + P - 1) // P).sum())
    nbytes = entries * (4 + 8 + 8) + 4 * cfg.batch
    out = {"us": round(us, 2), "entries": entries, "algorithmic_bytes": nbytes,
           "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    if step is None:
        return out
    side = torch.cuda.Stream()  # default priority, like the step's stream
    marks = [(torch.cuda.Event(), torch.cuda.Event()) for _ in range(steps)]
    pair = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            for _ in range(2)]
    main = torch.cuda.current_stream()

    def with_check(i):
        go, done = marks[i]
        if step.sparse:
            step.indexer()
        go.record(main)
        with torch.cuda.stream(side):
            side.wait_event(go)
            check()
            done.record(side)
        if step.sparse:
            step.select()
        step.attend()
        step.merge()
        main.wait_event(done)

    for i in range(3):
        with_check(i)
    torch.cuda.synchronize()
    for i in range(steps):  # interleaved: the step alone, then with the check beside it
        for mode in (0, 1):
            if flush:
                run_flush()
            e0, e1 = pair[mode][i]
            e0.record()
            step.run() if mode == 0 else with_check(i)
            e1.record()
    torch.cuda.synchronize()
    assert not status.cpu().numpy().any(), "page check flagged a request on clean inputs"
    alone, beside = (statistics.fmean(e0.elapsed_time(e1) for e0, e1 in pair[m]) * 1e3 for m in (0, 1))
    out.update(step_us_alone=round(alone, 1), step_us_with_check_on_a_second_stream=round(beside, 1),
               added_us=round(beside - alone, 2), added_frac_of_step=round((beside - alone) / alone, 4))
    return out


def time_multi_query(cfg, db, inp, n_q, splits, steps, flush, run_flush):
    """A verification step over n_q new tokens per request (query i attends
    causally, with its own scores and top-k): mq_expand_requests and the four
    calls on the expanded batch, timed cold like the step."""
    import numpy as np
    import torch
    import spmla_gen as gen
    from spmla_gen.torch_io import tensor
    from sparse_paged_mla_amd.step import MultiQueryStep
    q, qi, w = gen.make_mq_queries(inp, n_q)
    st = MultiQueryStep(db, tensor(q, "cuda"), tensor(qi, "cuda"), torch.from_numpy(w).cuda(), num_splits=splits)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for _ in range(5):
        st.run()
    for e0, e1 in evs:
        if flush:
            run_flush()
        e0.record()
        st.run()
        e1.record()
    torch.cuda.synchronize()
    assert not st.status.cpu().numpy().any(), "multi-query step flagged a request on clean inputs"
    us = statistics.fmean(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3
    # Roofline of the method: every query's scores, top-k and attention, with
    # the indexer keys read once for all n_q queries (as the two-query
    # indexer reads them) and one score row written per query.
    alg = algorithmic(cfg, inp.lens)
    sumL = int(inp.lens.sum())
    t_star = (max((alg["indexer"]["bytes"] + (n_q - 1) * 4 * sumL) / (HBM_PEAK_GBS * 1e9),
                  n_q * alg["indexer"]["flops"] / (BF16_PEAK_TFLOPS * 1e12))
              + n_q * alg["topk"]["bytes"] / (HBM_PEAK_GBS * 1e9)
              + max(n_q * alg["decode"]["bytes"] / (HBM_PEAK_GBS * 1e9),
                    n_q * alg["decode"]["flops"] / (BF16_PEAK_TFLOPS * 1e12)))
    return {"n_q": n_q, "us_per_step": round(us, 2), "verified_tokens_per_s": round(cfg.batch * n_q / (us * 1e-6), 1),
            "t_star_us": round(t_star * 1e6, 2), "frac": round(t_star / (us * 1e-6), 4), "num_splits": splits,
            "note": "indexer scores both queries per key read; top-k, decode and merge run on the expanded "
                    "batch of batch*n_q requests"}


def time_prefill_chunk(cfg, db, inp, n_req, n_q, blocks, steps, flush, run_flush):
    """Attention of a prefill chunk: n_q new tokens at the end of each of the
    first n_req requests, each attending densely and causally to its context,
    computed in `blocks` KV blocks merged by the online-softmax algebra."""
    import dataclasses
    import numpy as np
    import torch
    import spmla_gen as gen
    from spmla_gen.torch_io import tensor
    from sparse_paged_mla_amd.step import PrefillChunkStep
    q = gen.make_chunk_queries(inp, n_req, n_q)
    sub = dataclasses.replace(db, q=db.q[:n_req], block_table=db.block_table[:n_req], lens=db.lens[:n_req])
    st = PrefillChunkStep(sub, tensor(q, "cuda"), num_blocks=blocks)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for _ in range(2):
        st.run()
    for e0, e1 in evs:
        if flush:
            run_flush()
        e0.record()
        st.run()
        e1.record()
    torch.cuda.synchronize()
    assert not st.status.cpu().numpy().any(), "prefill chunk flagged a request on clean inputs"
    us = statistics.fmean(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3
    lens = inp.lens[:n_req].astype(np.int64)
    vis = (lens[:, None] - n_q + 1 + np.arange(n_q)[None, :]).sum()
    flops = 2.0 * int(vis) * cfg.n_heads * (cfg.dim + cfg.d_latent)
    e_c = {0: 4, 1: 2, 2: 1}[cfg.cache_dtype] * cfg.dim + (4 if cfg.cache_dtype == 2 else 0)
    nbytes = int(lens.sum()) * e_c + n_req * n_q * cfg.n_heads * (cfg.dim * 2 + 4 * (cfg.d_latent + 1))
    t_star = max(flops / (BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9))
    return {"requests": n_req, "n_q": n_q, "kv_blocks": blocks, "context_tokens": int(lens.sum()),
            "us_per_step": round(us, 1), "prefill_tokens_per_s": round(n_req * n_q / (us * 1e-6), 1),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1), "t_star_us": round(t_star * 1e6, 1),
            "frac": round(t_star / (us * 1e-6), 4), "bound": "mfma (bf16 peak)",
            "note": "each chunk query runs as its own request through the decode kernel: its KV is re-read per query "
                    "(from L2/MALL)"}


def _host_cpu():
    """CPU model name and the core counts this process may use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, os.cpu_count() or 1, usable


def _oracle_step(inp, reqs):
    """The fp64 oracle, as it stands, on the requests `reqs` of the inputs:
    indexer scores, top-k and attention (dense workloads: attention only)."""
    import numpy as np
    import oracle
    cfg = inp.cfg
    sel = np.asarray(reqs, np.int32)
    lens = inp.lens[sel]
    idx = s = None
    if not cfg.dense:
        s, _, _ = oracle.indexer_scores(inp.q_idx[sel], inp.w[sel], inp.k_idx, inp.k_idx_scale,
                                        inp.block_table[sel], lens, max_len=inp.max_len,
                                        score_stride=int(lens.max()))
        idx = oracle.topk(s, lens, cfg.topk)
    o, lse, _ = oracle.mla_attention(inp.q[sel], inp.kv, inp.kv_scale, inp.block_table[sel], lens, idx, cfg.n_heads,
                                     cfg.d_latent, cfg.d_rope, cfg.softmax_scale, max_len=inp.max_len)
    return s, idx, o


def _oracle_pass(inp, reqs, threads):
    """Wall time of the oracle over `reqs`: one request per task, `threads`
    tasks at a time (the oracle's C code runs outside the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    if threads == 1:
        out = [_oracle_step(inp, [b]) for b in reqs]
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            out = list(ex.map(lambda b: _oracle_step(inp, [b]), reqs))
    return time.perf_counter() - t0, out


def cpu_baseline(inp, n_single, n_multi, gpu_pass, step):
    """The fp64 oracle timed on the host beside the GPU: three rounds, each a
    single-thread pass over the first n_single requests, a pass over the
    first n_multi requests with one thread per usable core (at most 16), and
    a GPU pass of the timed step (A/B interleaving).  Medians of the three
    rounds.  The single-thread pass's outputs also give the end-to-end
    diagnostic: the oracle's own fp64 selection and attention against what
    the GPU step selected and produced for the same requests."""
    import numpy as np
    cfg = inp.cfg
    model, n_logical, usable = _host_cpu()
    threads = max(1, min(16, usable, n_multi))
    single_s, multi_s, gpu_ms = [], [], []
    out_single = None
    for _ in range(3):
        dt, out_single = _oracle_pass(inp, list(range(n_single)), 1)
        single_s.append(dt)
        dt, _ = _oracle_pass(inp, list(range(n_multi)), threads)
        multi_s.append(dt)
        gpu_ms.append(gpu_pass())
    t1 = statistics.median(single_s)
    tm = statistics.median(multi_s)
    sample_tokens = int(np.sum(inp.lens[:n_single]))
    multi_tokens = int(np.sum(inp.lens[:n_multi]))
    # End-to-end diagnostic on the single-thread sample (nothing asserted).
    e2e = None
    if not cfg.dense:
        idx_gpu = step.idx.cpu().numpy()
        o_gpu = step.o.cpu().numpy()
        swaps = sel_total = 0
        d_o = 0.0
        num = den = 0.0
        for b, (_, idx_ref, o_ref) in enumerate(out_single):
            a = set(int(x) for x in idx_gpu[b] if x >= 0)
            r = set(int(x) for x in idx_ref[0] if x >= 0)
            swaps += len(a - r)
            sel_total += len(r)
            diff = o_gpu[b].astype(np.float64) - o_ref[0]
            d_o = max(d_o, float(np.abs(diff).max()))
            num += float(np.sum(diff ** 2))
            den += float(np.sum(o_ref[0] ** 2))
        e2e = {"requests": n_single, "selected": sel_total, "swaps": swaps, "max_abs_do": d_o,
               "rel_rms_o": (num / den) ** 0.5 if den > 0 else None,
               "note": "oracle's own fp64 scores and top-k, then its attention, against the GPU step: selected "
                       "tokens that differ from the fp64 ranking (fp32 score rounding at the selection boundary) "
                       "and the resulting output difference"}
    return dict(value=n_multi / tm, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{cfg.name}: full step (" + ("attention" if cfg.dense else "indexer + top-k + attention")
                       + f", fp64) over the first {n_multi} of {cfg.batch} requests ({multi_tokens} context tokens), "
                         f"one request per thread on {threads} threads; median of 3 passes interleaved with GPU passes",
                single_thread={"value": n_single / t1, "cores": 1, "requests": n_single,
                               "context_tokens": sample_tokens, "median_s": round(t1, 3),
                               "runs_s": [round(x, 3) for x in single_s]},
                all_threads={"value": n_multi / tm, "cores": threads, "requests": n_multi,
                             "context_tokens": multi_tokens, "median_s": round(tm, 3),
                             "runs_s": [round(x, 3) for x in multi_s]},
                host={"cpu_model": model, "logical_cpus": n_logical, "usable_cpus": usable},
                gpu_passes_ms_per_step=[round(x, 4) for x in gpu_ms],
                end_to_end=e2e)


def main():
    args = parse()
    if args.counters:
        summarize_counters(*args.counters, args.config)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import spmla_gen as gen
    from spmla_gen.torch_io import device_batch
    from sparse_paged_mla_amd.step import DecodeStep, default_splits
    import sparse_paged_mla_amd as spm

    spm.load_library()
    cfg = gen.CONFIGS[args.config]
    t_gen = time.perf_counter()
    inp = gen.make_inputs(cfg)
    db = device_batch(inp, "cuda")
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: inputs ready in {time.perf_counter() - t_gen:.1f} s "
          f"(sum L = {int(inp.lens.sum())}, pool {inp.num_pages} pages)", file=sys.stderr, flush=True)
    splits, split_tokens = default_splits(cfg.name, inp.lens, cfg.n_heads, args.splits)
    step = DecodeStep(db, num_splits=splits, split_tokens=split_tokens)
    stages = ["indexer", "select", "attend", "merge"] if step.sparse else ["attend", "merge"]
    if splits == 1:
        stages.remove("merge")
    flush_buf = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    flush_sink = torch.zeros((), dtype=torch.float32, device="cuda")

    # Every event the timed region records is created (and recorded once)
    # up front: creating events while timing costs the steps measurable time.
    ev_sets = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    ev_sets_k = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    for evs in ev_sets + ev_sets_k:
        for e in evs:
            e.record()
    torch.cuda.synchronize()

    def run_timed(flush, evs, per_kernel):
        """One step between evs[0] and evs[-1]; with per_kernel, an event after
        every stage as well (each such event costs the step 2-3 us, so the
        step time that gives `value` is taken without them)."""
        if flush:
            flush_sink.copy_(flush_buf.amax())
        evs[0].record()
        for i, name in enumerate(stages):
            getattr(step, name)()
            if per_kernel or i == len(stages) - 1:
                evs[i + 1].record()
        return evs

    # Warm-up steps are the timed steps' twins (cache sweep included).
    flush = not args.no_flush
    for i in range(args.warmup):
        run_timed(flush, ev_sets[i % args.steps], i % 2 == 1)
    torch.cuda.synchronize()
    assert not step.status.cpu().numpy().any(), "device status flags set on clean inputs"

    # The K timed steps: whole-step events only.
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    recs = [run_timed(flush, evs, False) for evs in ev_sets]
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [evs[0].elapsed_time(evs[-1]) for evs in recs]
    mean_ms = statistics.fmean(step_ms)
    # K more steps with an event after every kernel: per-kernel times.
    recs_k = [run_timed(flush, evs, True) for evs in ev_sets_k]
    torch.cuda.synchronize()
    per_stage = {n: [evs[i].elapsed_time(evs[i + 1]) for evs in recs_k] for i, n in enumerate(stages)}
    step_k_ms = statistics.fmean(evs[0].elapsed_time(evs[-1]) for evs in recs_k)

    # Warm: K steps back to back (skipped under --profile-only so that a
    # profiler's per-kernel averages cover the same launches as the events).
    warm_ms = float("nan")
    if not args.profile_only:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step.run()
        e1.record()
        torch.cuda.synchronize()
        warm_ms = e0.elapsed_time(e1) / args.steps

    # The legs of the next rows (skipped under --profile-only, so that a
    # profile's per-kernel figures cover the step's launches only).
    legs = not args.profile_only
    app = None if not legs or cfg.dense or cfg.cache_dtype != gen.FP8 else time_cache_append(cfg, db, inp, args.steps, flush,
                                                                                 run_flush=lambda: flush_sink.copy_(
                                                                                     flush_buf.amax()))

    # The expanded batch has n_q times the requests, so the same workgroup
    # count comes from n_q times fewer KV splits.
    mq = None if not legs or cfg.dense else time_multi_query(cfg, db, inp, 2, max(1, splits // 2), args.steps, flush,
                                                 run_flush=lambda: flush_sink.copy_(flush_buf.amax()))
    n_pre = min(2, cfg.batch)
    pre = None if not legs else time_prefill_chunk(cfg, db, inp, n_pre, min(64, int(inp.lens[:n_pre].min())), 2,
                                                   min(args.steps, 10), flush,
                                                   run_flush=lambda: flush_sink.copy_(flush_buf.amax()))
    chk = None
    if legs:
        chk = time_page_check(cfg, db, inp, args.steps, flush, run_flush=lambda: flush_sink.copy_(flush_buf.amax()),
                              step=step)
        chk["overhead_frac_of_step"] = round(chk["us"] / (mean_ms * 1e3), 4)

    alg = algorithmic(cfg, inp.lens)
    t_star = roofline_time_s(alg)
    kname = {"indexer": "indexer", "select": "topk", "attend": "decode", "merge": "merge"}
    kernel_ms = {kname[n]: statistics.fmean(v) for n, v in per_stage.items()}
    # Dominant kernel: the one with the largest roofline time.
    dom = max((k for k in kernel_ms if k in alg),
              key=lambda k: max(alg[k]["bytes"] / HBM_PEAK_GBS, alg[k]["flops"] / BF16_PEAK_TFLOPS * 1e-3))
    dk = alg[dom]
    t_dom = kernel_ms[dom] * 1e-3
    hbm_bound = dk["bytes"] / (HBM_PEAK_GBS * 1e9) >= dk["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    src = {"indexer": "indexer.hip", "topk": "topk.hip",
           "decode": ("mla_decode.hip" if cfg.q_dtype != 1 else
                      "mla_decode_f8.hip" if cfg.cache_dtype == 2 else "mla_decode_bf16.hip"),
           "merge": "lse_merge.hip"}[dom]
    traffic = measured_traffic(src, cfg.name)
    if hbm_bound:
        achieved = dk["bytes"] / t_dom / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic, kernel=dom,
                    algorithmic_bytes=int(dk["bytes"]), avg_launch_us=round(t_dom * 1e6, 2))
    else:
        achieved = dk["flops"] / t_dom / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / BF16_PEAK_TFLOPS, 4), traffic=traffic, kernel=dom,
                    algorithmic_flops=int(dk["flops"]), avg_launch_us=round(t_dom * 1e6, 2))
    roof["scope"] = (f"one kernel ({dom}, the largest roofline time of the step), not the whole step: "
                     f"the whole step's fraction of its roofline is step_roofline.frac")

    if args.profile_only:
        # A plain device-to-device copy of known size: the HBM counters read for
        # it calibrate the counters read for the kernels.
        src = torch.ones(256 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    n_cpu = args.cpu_requests
    if n_cpu < 0:
        n_cpu = {"c1": 2, "c2": 32, "c3": 2, "c3f": 2, "c4": 8, "c5": 1}.get(cfg.name, 1)

    def gpu_pass():
        recs = [run_timed(flush, evs, False) for evs in ev_sets]
        torch.cuda.synchronize()
        return statistics.median(evs[0].elapsed_time(evs[-1]) for evs in recs)

    cpu = None
    if not args.profile_only and n_cpu > 0:
        n_multi = min(cfg.batch, max(n_cpu, min(16, _host_cpu()[2])))
        cpu = cpu_baseline(inp, min(n_cpu, cfg.batch), n_multi, gpu_pass, step)

    value = cfg.batch / (mean_ms * 1e-3)
    line = {
        "metric": "decode tokens/s for sparse paged MLA attention (one layer, one decode step)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(mean_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded generator)",
        "config": {
            "workload": f"{cfg.name}: {cfg.batch} requests, context {cfg.lens}, sum L {int(inp.lens.sum())}, "
                        f"{cfg.n_heads} heads, latent {cfg.d_latent}+{cfg.d_rope}, "
                        + ("dense attention" if cfg.dense else
                           f"indexer {cfg.idx_heads}x{cfg.idx_dim} {gen.DTYPE_NAMES[cfg.idx_dtype]}, top-k {cfg.topk}")
                        + f", cache {gen.DTYPE_NAMES[cfg.cache_dtype]}, page {cfg.page_size}",
            "global_batch": cfg.batch, "seq_len": int(inp.max_len), "num_splits": splits,
            "split_tokens": split_tokens,
            "parallelism": "single GPU", "cache_flush_between_steps": flush},
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_roofline": {"t_star_us": round(t_star * 1e6, 2), "t_step_us": round(mean_ms * 1e3, 2),
                          "frac": round(t_star / (mean_ms * 1e-3), 4),
                          "note": "T* = sum over the step's kernels of max(algorithmic bytes / 8 TB/s, "
                                  "FLOPs / 2.5 PFLOP/s); frac = T* / measured step time (the gate is 0.60)"},
        "kernel_us": {k: round(v * 1e3, 2) for k, v in kernel_ms.items()},
        "ms_per_step_with_kernel_events": round(step_k_ms, 4),
        "cache_append": app,
        "page_check": chk,
        "multi_query": mq,
        "prefill_chunk": pre,
        "step_ms_median_min_max": [round(statistics.median(step_ms), 4), round(min(step_ms), 4),
                                   round(max(step_ms), 4)],
        "warm_ms_per_step": None if warm_ms != warm_ms else round(warm_ms, 4),
        "warm_value": None if warm_ms != warm_ms else round(cfg.batch / (warm_ms * 1e-3), 1),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
