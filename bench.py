"""Throughput of the MSA hot path on one MI355X.

Default workload (the headline metric): routed decode at a 1M-token bank --
2048 documents x 512 tokens, bf16, 8 router heads, 32 query / 8 KV heads,
d = 128, batch 16, top-16, 4096-token local context.  One step = route ->
top-k -> gather -> split-K attention (msa_step) for one batch of 16 queries.
Independent batches rotate over --batches query sets (so the 256 MB MALL
cannot hold a step's data) and alternate over --streams HIP streams.

Prints one JSON line: queries/s, the dominant kernel's roofline (decode
attention, timed with HIP events around each launch on its stream), and the
fp64 oracle timed on this host on a bounded sample of the same workload.
"""
import argparse
import ctypes
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed decode queries/sec at 1M-token bank; % peak HBM GB/s; prefill MFMA %"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
TIMER_PERIOD = 5  # two-stream decode legs: HIP events bracket every 5th launch


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _code_tokens(text):
    """Source text without comments, whitespace collapsed: what the compiler
    sees, so that a comment edit does not count as a kernel change."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def _sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_tokens(f.read()).encode())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    record profiles/<name>.json (FETCH_SIZE and WRITE_SIZE per dispatch, each
    scaled by the same counter's reading on a plain copy of known size), or
    None when there is no record or the kernel's sources changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if _sources_sha256(rec["sources"]) != rec["sources_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def measured_read_rate(n_bytes=1 << 30, reps=20):
    """HBM rate of the library's read-only stream over a 1 GiB buffer (four
    times the last-level cache): what a kernel that only reads reaches on
    this device, next to the datasheet's 8 TB/s."""
    import torch
    from long_context_memory_amd import msa
    buf = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(msa.MSA_STREAM_READ_BLOCKS, dtype=torch.int32, device="cuda")
    for _ in range(3):
        msa.stream_read(buf, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        msa.stream_read(buf, out)
    e1.record()
    e1.synchronize()
    rate = n_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, out
    torch.cuda.empty_cache()
    return rate


def calibrate_copy(n_bytes=1 << 30, reps=10):
    """A plain device copy of known size (reads and writes n_bytes each), run
    under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to scale those counters."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n_bytes, "copy_bytes_written": n_bytes, "reps": reps}))


def cpu_baseline(w, r_dev, k_raw_dev, v_raw_dev, batch_inputs, budget_s=12.0):
    """The fp64 oracle on one 16-query decode step of the same bank.  Bank
    build (pooling, document RoPE) and the local context's RoPE are set-up,
    as on the GPU; the timed part is routing over every chunk, top-k, the
    gather and the attention."""
    import numpy as np
    import torch
    from oracle import msa_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    limits = threadpool_limits(limits=cores, user_api="blas")  # BLAS on every allowed core
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
            for i in threadpool_info() if i.get("user_api") == "blas"]
    try:
        deps = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas_build = f"{deps.get('name')} {deps.get('version')}"
    except Exception:  # pragma: no cover
        blas_build = None

    f64 = lambda t: t.detach().to("cpu", torch.float32).double().numpy()  # noqa: E731
    off = np.concatenate([[0], np.cumsum(w.doc_len)])
    keys = []
    for n0 in range(0, w.n_docs, 256):
        n1 = min(w.n_docs, n0 + 256)
        keys.append(O.chunk_mean_pool(f64(r_dev[off[n0]:off[n1]]), w.doc_len[n0:n1]))
    kr = O.round_to_storage(np.concatenate(keys), w.dtype)
    inv = O.inverse_norms(kr)
    q, q_route, lk, lv = batch_inputs
    qn, qrn = f64(q), f64(q_route)
    scores = O.cosine_doc_scores(qrn, kr, inv, w.doc_len)
    ids, _ = O.select_topk(scores, w.k)
    doc_kv = {}
    for n in set(ids.ravel().tolist()):
        a, b = off[n], off[n + 1]
        doc_kv[n] = (O.bank_keys_rotated(f64(k_raw_dev[a:b]), [b - a], w.rope_base, w.dtype),
                     f64(v_raw_dev[a:b]))
    L = w.L_loc
    lkr = [O.round_to_storage(O.rope_rotate(f64(lk[b]), (w.P0 + np.arange(L))[:, None],
                                            w.rope_base), w.dtype) for b in range(w.B)]
    lvn = [f64(lv[b]) for b in range(w.B)]

    def one_step():
        s = O.cosine_doc_scores(qrn, kr, inv, w.doc_len)
        sel, _ = O.select_topk(s, w.k)
        for b in range(w.B):
            K = np.concatenate([doc_kv[n][0] for n in sel[b]] + [lkr[b]])
            V = np.concatenate([doc_kv[n][1] for n in sel[b]] + [lvn[b]])
            qr = O.rope_rotate(qn[b][None], np.full((1, w.h_q), w.q_pos), w.rope_base)
            O.gqa_attention(qr, K, V)

    n, t0 = 0, time.perf_counter()
    while True:
        one_step()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or n >= 50:
            break
    limits.restore_original_limits()
    return {"value": w.B * n / dt, "unit": "queries/s", "cores": int(cores), "kind": "oracle",
            "blas": blas, "blas_build": blas_build,
            "sample": f"{n} full 16-query decode step(s) of the 1M-token bank: cosine routing "
                      "over all 4096 chunks x 8 heads, top-16, gather, GQA attention over "
                      "12,288 tokens x 32 heads per query (bank build and local RoPE are "
                      "set-up, as on the GPU)",
            "seconds": dt, "processor": platform.processor() or platform.machine()}


def prefill_bench(steps, warmup, splits=0):
    """Blocked prefill on the 8M-token bank (4096 docs x 2048 tokens): 2048
    query tokens in 32 blocks of 64, top-16 per block, causal 2048-token local
    context, 32 query / 8 KV heads.  Returns tokens/s and the attention
    kernel's roofline (algorithmic bytes and flops / event-timed duration)."""
    import torch
    from long_context_memory_amd import msa, synth as S

    dev = "cuda"
    w = S.workload("prefill_8m")
    log(f"prefill: building {w.name}: {w.n_docs} docs, {w.T} tokens")
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, dev, rope_base=w.rope_base)
    step_docs = 1024
    off = S.doc_token_offsets(w)
    for n0 in range(0, w.n_docs, step_docs):
        n1 = min(w.n_docs, n0 + step_docs)
        r = S.route_vectors(w, dev, int(off[n0]), int(off[n1]))
        k_raw, v_raw = S.kv_raw(w, dev, int(off[n0]), int(off[n1]))
        bank.build(n0, n1, r, k_raw, v_raw)
        torch.cuda.synchronize()
        del r, k_raw, v_raw
    q = S.queries(w, dev)
    rt = S.prefill_route_tokens(w, dev)
    lk, lv = S.local_raw(w, dev)
    k_loc, v_loc, L = bank.prepare_local(lk[None], lv[None], w.P0)
    q_pos = w.P0 + (w.L_loc - w.B)
    ws = bank.workspace(msa.MSA_PREFILL, w.B, w.h_q, w.k, w.block, splits=splits)
    nb = w.B // w.block
    outs = (torch.empty((1, nb, w.k), dtype=torch.int32, device=dev),
            torch.empty((1, nb, w.k), dtype=torch.float32, device=dev),
            torch.empty((1, w.B, w.h_q, 128), dtype=torch.float32, device=dev))

    def step():
        bank.step(q, q_pos, w.k, k_loc, v_loc, L, route_tokens=rt, mode=msa.MSA_PREFILL,
                  block=w.block, ws=ws, outputs=outs, splits=splits)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    msa.timer_reserve(2 * steps)  # attention + routing intervals, events made up front
    msa.timer_enable(True)
    msa.timer_read(msa.MSA_TIMER_ATTENTION)
    msa.timer_read(msa.MSA_TIMER_ROUTE)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    att_ms, att_n = msa.timer_read(msa.MSA_TIMER_ATTENTION)
    msa.timer_read(msa.MSA_TIMER_ROUTE)
    msa.timer_enable(False)
    # algorithmic flops: QK^T and PV over every unmasked (query, key) pair
    doc_pairs = w.B * w.k * 2048
    causal_pairs = sum(range(w.L_loc - w.B + 1, w.L_loc + 1))
    flops = (doc_pairs + causal_pairs) * w.h_q * 128 * 4
    # bytes: each block's selected documents' K/V once + the causal local prefix
    kv_bytes = (nb * w.k * 2048 + sum(min(w.L_loc, (b + 1) * w.block) for b in range(nb))) \
        * w.h_kv * 128 * 2 * 2
    att_s = att_ms * 1e-3 / max(att_n, 1)
    return {"workload": "blocked prefill: 8M-token bank (4096 docs x 2048 tokens), 2048 query "
                        "tokens in 32 blocks of 64, top-16 per block, causal 2048-token local "
                        "context, h_q=32, h_kv=8, d=128, bf16",
            "tokens_per_s": w.B * steps / dt, "ms_per_step": dt * 1e3 / steps, "steps": steps,
            "attention": prefill_roofline(flops, kv_bytes, att_s)}


def prefill_roofline(flops, kv_bytes, att_s):
    """The blocked prefill's roofline.  Each block's K/V tiles are read once
    and meet 256 query rows (64 queries x 4 heads of a KV head): 256 flop per
    byte, under the 2.5 PFLOP/s / 8 TB/s = 312 ridge, so the binding bound is
    HBM (bytes / 8 TB/s exceeds flops / 2.5 PFLOP/s).  Both fractions are
    reported."""
    t_hbm = kv_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS * 1e12)
    gbs, tfs = kv_bytes / att_s / 1e9, flops / att_s / 1e12
    hbm_bound = t_hbm >= t_mfma
    return {"bound": "hbm" if hbm_bound else "mfma",
            "achieved": gbs if hbm_bound else tfs,
            "peak": HBM_PEAK_GBS if hbm_bound else MFMA_PEAK_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": max(t_hbm, t_mfma) / att_s,
            "traffic": measured_traffic("prefill_8m_counters"),
            "bytes_per_launch": kv_bytes, "flops_per_launch": flops,
            "avg_launch_us": att_s * 1e6,
            "hbm_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "mfma_TFLOPs": tfs, "mfma_frac": tfs / MFMA_PEAK_TFLOPS}


CACHE_MARGIN_BYTES = 16 << 30  # HBM left free beside an automatically sized document cache


def host_bank_bench(steps, warmup, cache_gb=0.0, window=4):
    """The 100M-token host-resident bank (12,207 x 8192 + one 256-token
    document; routing keys in HBM, K/V in pinned host memory backed by 384
    document slots): 8-query decode steps, each reading its selected
    documents' K/V from host memory.  Two runs on one bank: (1) every
    selected document copied into device staging each step; (2) a device
    document cache of cache_gb (0: all the HBM left free, less a 16 GiB
    margin) with a prefetch window: batch i + window is routed and its
    documents copied into the cache while batch i steps.
    Reports queries/s, the host-to-device rate of the copies, a plain pinned
    1 GiB copy's rate in the same run, and the routing scan's HBM rate."""
    import torch
    from long_context_memory_amd import msa, synth as S

    dev = "cuda"
    w = S.workload("host_100m")
    log(f"host bank: {w.n_docs} docs, {w.T} tokens, {w.host_slots} slots")
    slot_len, kv_off = S.host_slot_layout(w)
    kr = S.keys_direct(w, dev).to(w.torch_dtype).permute(1, 0, 2).contiguous()
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, dev, kv_loc="host", kv_off=kv_off,
                    kv_tokens=int(sum(slot_len)), rope_base=w.rope_base, kr=kr)
    bank.build(0, w.n_docs)
    msa.fill_host_store(bank, slot_len, lambda t0, t1: S.host_kv_raw(w, dev, t0, t1),
                        slots_per_pass=32)
    q = S.queries(w, dev)
    lk, lv = S.local_raw(w, dev)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    main, side, cs = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    ws = bank.workspace(msa.MSA_DECODE, w.B, w.h_q, w.k)
    ws_side = bank.workspace(msa.MSA_DECODE, w.B, w.h_q, w.k)
    rt_bytes = w.C * w.h_r * (128 * 2 + 4)  # every routing key (bf16) and its norm

    # plain pinned host -> device copies of 1 GiB, for the link's own rate:
    # one 1 GiB copy, and the same bytes as 64 copies of 16 MiB (the size of
    # one 8192-token document's K or V), each a hipMemcpyAsync on the copy
    # stream as the step issues them (torch's copy_ of a pinned slice adds
    # host work per copy and reaches about half the rate at this size)
    hsrc = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    ddst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    hip.hipMemcpyAsync.restype = ctypes.c_int
    host_to_device = 1

    def copy_rate(chunks):
        n = (1 << 30) // chunks

        def issue():
            for c in range(chunks):
                rc = hip.hipMemcpyAsync(ddst.data_ptr() + c * n, hsrc.data_ptr() + c * n, n,
                                        host_to_device, cs.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"hipMemcpyAsync failed ({rc})")
        issue()
        torch.cuda.synchronize()
        tc = time.perf_counter()
        for _ in range(5):
            issue()
        torch.cuda.synchronize()
        return 5 * (1 << 30) / (time.perf_counter() - tc) / 1e9

    link_one, link_chunked = copy_rate(1), copy_rate(64)
    link = max(link_one, link_chunked)
    del hsrc, ddst

    def run(n_warm, n_steps, cached):
        total = n_warm + n_steps
        qrs = [S.route_queries(w, dev, batch=i) for i in range(total + window)]
        # staging: steps alternate over two streams, each with its own staging
        # buffer, so one step's copies queue behind the previous step's while
        # that step's attention and this step's routing run (one staging
        # buffer on one stream leaves the link idle for that time); cached:
        # steps on one stream, the prefetch window on the side stream
        stg = None if cached else [bank.staging(w.B, w.k) for _ in range(2)]
        wss = [ws, ws_side]
        step_streams = [main] if cached else [main, side]
        copied = [0, 0, 0]  # bytes, documents copied, documents found cached

        def count(st):
            copied[0] += st.bytes_copied
            copied[1] += st.docs_copied
            copied[2] += st.docs_cached

        if cached:
            for i in range(window):
                bank.prefetch(qrs[i], w.k, ws=ws_side, stream=side, copy_stream=cs)
        t0 = None
        for i in range(total):
            if i == n_warm:
                torch.cuda.synchronize()
                msa.timer_reserve(2 * n_steps)
                msa.timer_enable(True)
                msa.timer_read(msa.MSA_TIMER_ATTENTION)
                msa.timer_read(msa.MSA_TIMER_ROUTE)
                copied[:] = [0, 0, 0]
                t0 = time.perf_counter()
            if cached:
                count(bank.prefetch(qrs[i + window], w.k, ws=ws_side, stream=side,
                                    copy_stream=cs))
            j = i % len(step_streams)
            _, _, _, st = bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=qrs[i], ws=wss[j],
                                    staging=None if cached else stg[j], stream=step_streams[j],
                                    copy_stream=cs)
            count(st)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        msa.timer_read(msa.MSA_TIMER_ATTENTION)
        rt_ms, rt_n = msa.timer_read(msa.MSA_TIMER_ROUTE)
        msa.timer_enable(False)
        return {"queries_per_s": w.B * n_steps / dt, "ms_per_step": dt * 1e3 / n_steps,
                "steps": n_steps, "h2d_GBs": copied[0] / dt / 1e9,
                "h2d_frac_of_pinned_copy": copied[0] / dt / 1e9 / link,
                "h2d_frac_of_16MiB_copies": copied[0] / dt / 1e9 / link_chunked,
                "docs_copied_per_step": copied[1] / n_steps,
                "bytes_copied_per_step": copied[0] / n_steps,
                "docs_cached_per_step": copied[2] / n_steps,
                "routing_avg_launch_us": rt_ms * 1e3 / max(rt_n, 1),
                "routing_GBs": rt_bytes / (rt_ms * 1e-3 / max(rt_n, 1)) / 1e9}

    log(f"host bank: staging path, {warmup} + {steps} steps")
    plain = run(warmup, steps, False)
    slot = bank.cache_slot_bytes()
    if cache_gb > 0:
        cache_bytes = int(cache_gb * 1e9)
    else:  # the HBM left free, less a margin for the leg's own allocations
        torch.cuda.empty_cache()
        free, _ = torch.cuda.mem_get_info()
        cache_bytes = free - CACHE_MARGIN_BYTES
    slots = min(w.n_docs, max(0, cache_bytes) // slot)
    cache = None
    for _ in range(4):  # an allocation the free-memory figure promised but cannot place
        if slots < (window + 2) * w.B * w.k:
            raise RuntimeError(f"host bank: {slots} cache slots cannot hold a {window}-batch window")
        try:
            cache = torch.empty(slots * slot, dtype=torch.uint8, device=dev)
            break
        except torch.OutOfMemoryError:
            torch.cuda.empty_cache()
            slots -= CACHE_MARGIN_BYTES // slot
    if cache is None:
        raise RuntimeError("host bank: no room for the document cache")
    bank.set_cache(cache)
    del cache
    # each step routes fresh queries: hits come from the cache holding a share
    # of the bank, so the cache is filled before the timed steps
    fill = -(-slots // (w.B * w.k)) + 4
    log(f"host bank: cache of {slots} slots, prefetch window {window}, {fill} + {steps} steps")
    cached = run(fill, steps, True)
    bank.set_cache(None)
    cached.update({"cache_slots": slots, "cache_bytes": slots * slot,
                   "cache_share_of_documents": slots / w.n_docs, "prefetch_window": window,
                   "hit_rate": cached["docs_cached_per_step"] /
                   max(1e-9, cached["docs_cached_per_step"] + cached["docs_copied_per_step"])})
    return {"workload": "100M-token host-resident bank: 12,207 docs x 8192 + one 256-token doc "
                        "(390,625 chunks, bf16 keys in HBM), K/V in pinned host memory (384 "
                        "document slots), B=8, top-16, local 4096",
            "pinned_copy_GBs": link, "pinned_copy_1GiB_GBs": link_one,
            "pinned_copy_16MiB_GBs": link_chunked, "staging": plain, "cached_prefetch": cached,
            "routing": {"bound": "hbm", "bytes_per_launch": rt_bytes,
                        "avg_launch_us": plain["routing_avg_launch_us"],
                        "achieved": plain["routing_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": plain["routing_GBs"] / HBM_PEAK_GBS}}


def interleave_bench(steps, warmup):
    """Three Memory Interleave hops over a 32 Mi-token bank of lognormal
    documents (K/V resident in HBM), 64 queries, top-8 per hop.  Reports
    queries/s per 3-hop step and the attention launches' HBM rate from the
    bytes of the documents actually selected."""
    import numpy as np
    import torch
    from long_context_memory_amd import msa, synth as S

    dev = "cuda"
    w = S.workload("interleave_32m")
    log(f"interleave: building {w.n_docs} docs, {w.T} tokens")
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, dev, rope_base=w.rope_base)
    off = S.doc_token_offsets(w)
    for n0 in range(0, w.n_docs, 256):
        n1 = min(w.n_docs, n0 + 256)
        a, b = int(off[n0]), int(off[n1])
        bank.build(n0, n1, S.route_vectors(w, dev, a, b), *S.kv_raw(w, dev, a, b))
        torch.cuda.synchronize()
    q = S.queries(w, dev)
    q_route = S.route_queries(w, dev)
    lk, lv = S.local_raw(w, dev)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    wp = S.interleave_projection(w, dev)
    ws = bank.workspace(msa.MSA_DECODE, w.B, w.h_q, w.k, hops=w.hops)
    outs = (torch.empty((w.hops, w.B, w.k), dtype=torch.int32, device=dev),
            torch.empty((w.hops, w.B, w.k), dtype=torch.float32, device=dev),
            torch.empty((w.hops, w.B, w.h_q, 128), dtype=torch.float32, device=dev))

    def step():
        bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=q_route, hops=w.hops, w_proj=wp,
                  ws=ws, outputs=outs)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    msa.timer_reserve(2 * steps * w.hops)  # attention + routing intervals, events made up front
    msa.timer_enable(True)
    msa.timer_read(msa.MSA_TIMER_ATTENTION)
    msa.timer_read(msa.MSA_TIMER_ROUTE)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    att_ms, att_n = msa.timer_read(msa.MSA_TIMER_ATTENTION)
    rt_ms, rt_n = msa.timer_read(msa.MSA_TIMER_ROUTE)
    msa.timer_enable(False)
    rt_bytes = w.C * w.h_r * (128 * 2 + 4)
    # the scan's arithmetic: 64 queries x every key x 128 channels, multiply-add
    rt_flops = 2 * w.B * w.C * w.h_r * 128
    ids = outs[0].cpu().numpy()
    lens = np.asarray(w.doc_len, dtype=np.int64)
    tok = int(lens[ids].sum()) + w.hops * w.B * w.L_loc  # union tokens over the 3 hops
    att_bytes = tok * w.h_kv * 128 * 2 * 2
    att_s = att_ms * 1e-3 / max(att_n, 1) * w.hops
    return {"workload": "Memory Interleave x3 over a 32 Mi-token bank (lognormal document "
                        "lengths, median 4096, 1024..65536), B=64, top-8 per hop, h_r=1, "
                        "local 4096",
            "queries_per_s": w.B * steps / dt, "ms_per_step": dt * 1e3 / steps, "steps": steps,
            "attention": {"bound": "hbm", "bytes_per_step": att_bytes,
                          "avg_launch_us": att_s / w.hops * 1e6,
                          "achieved": att_bytes / att_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": att_bytes / att_s / 1e9 / HBM_PEAK_GBS},
            "routing": {"kernel": "routing scan on the matrix cores (64 queries per pass)",
                        "bytes_per_launch": rt_bytes, "flops_per_launch": rt_flops,
                        "avg_launch_us": rt_ms * 1e3 / max(rt_n, 1),
                        "achieved_GBs": rt_bytes / (rt_ms * 1e-3 / max(rt_n, 1)) / 1e9,
                        "peak_GBs": HBM_PEAK_GBS}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first (about 0.15 s: the chip reaches its steady state)")
    ap.add_argument("--batches", type=int, default=4, help="rotating query batches")
    ap.add_argument("--streams", type=int, default=2, help="HIP streams batches alternate over")
    ap.add_argument("--splits", type=int, default=0, help="attention splits (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=20, help="0 skips the prefill leg")
    ap.add_argument("--prefill-splits", type=int, default=0, help="token splits (0: automatic)")
    ap.add_argument("--pooled-steps", type=int, default=0,
                    help="also time compressed-memory decode on the same bank (0 skips it)")
    ap.add_argument("--single-stream-steps", type=int, default=300,
                    help="decode steps on one stream, timed once without events (the step) "
                         "and once with every launch event-timed (the kernel's isolated "
                         "duration); 0 skips it")
    ap.add_argument("--host-bank-steps", type=int, default=8,
                    help="timed steps of each 100M-token host-bank run (0 skips the leg)")
    ap.add_argument("--host-cache-gb", type=float, default=0.0,
                    help="device document cache of the host-bank leg's second run, GB "
                         "(0: the free HBM less 16 GiB)")
    ap.add_argument("--prefetch-window", type=int, default=4,
                    help="batches routed and prefetched ahead in the cached host-bank run")
    ap.add_argument("--interleave-steps", type=int, default=3,
                    help="timed 3-hop steps over the 32 Mi-token bank (0 skips the leg)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported here "
              "(the path would shard by document range across GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_memory_amd import msa, synth as S

    dev = "cuda"
    w = S.workload("decode_1m")
    log(f"building {w.name}: {w.n_docs} docs, {w.T} tokens")
    r = S.route_vectors(w, dev)
    k_raw, v_raw = S.kv_raw(w, dev)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, dev, rope_base=w.rope_base)
    torch.cuda.synchronize()
    tb = time.perf_counter()
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - tb
    batches, raw0 = [], None
    for i in range(args.batches):
        q = S.queries(w, dev, batch=i)
        q_route = S.route_queries(w, dev, batch=i)
        lk, lv = S.local_raw(w, dev, batch=i)
        k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
        if i == 0:
            raw0 = (q, q_route, lk, lv)
        batches.append((q, q_route, k_loc, v_loc, L))
    streams = [torch.cuda.Stream() for _ in range(max(1, args.streams))]
    ws = [bank.workspace(msa.MSA_DECODE, w.B, w.h_q, w.k) for _ in streams]
    outs = [(torch.empty((1, w.B, w.k), dtype=torch.int32, device=dev),
             torch.empty((1, w.B, w.k), dtype=torch.float32, device=dev),
             torch.empty((1, w.B, w.h_q, 128), dtype=torch.float32, device=dev))
            for _ in range(args.batches)]
    torch.cuda.synchronize()

    def step(i):
        si = i % len(streams)
        q, q_route, k_loc, v_loc, L = batches[i % args.batches]
        bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=q_route, ws=ws[si],
                  outputs=outs[i % args.batches], stream=streams[si], splits=args.splits)

    single = None
    if args.single_stream_steps > 0:
        # one stream, every launch bracketed: the decode kernel's own duration
        # with nothing overlapping it, and the serial route -> top-k ->
        # attention -> merge chain of a step (this also brings the chip to its
        # steady clock before the timed region)
        log("single-stream leg")
        n1 = args.single_stream_steps
        def sstep(i):
            q, q_route, k_loc, v_loc, L = batches[i % args.batches]
            bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=q_route, ws=ws[0],
                      outputs=outs[i % args.batches], stream=streams[0], splits=args.splits)
        for i in range(n1):
            sstep(i)
        torch.cuda.synchronize()
        # the step as a caller sees it: no events on the stream
        t1 = time.perf_counter()
        for i in range(n1):
            sstep(i)
        hdt = time.perf_counter() - t1  # the host's time to issue the steps
        torch.cuda.synchronize()
        sdt = time.perf_counter() - t1
        # the same steps again with every launch bracketed by events: the
        # kernels' own durations (events on a single stream serialise its
        # launches, so this pass's wall time is not the step's)
        msa.timer_reserve(2 * n1)
        msa.timer_enable(True, 1)
        msa.timer_read(msa.MSA_TIMER_ATTENTION)
        msa.timer_read(msa.MSA_TIMER_ROUTE)
        t2 = time.perf_counter()
        for i in range(n1):
            sstep(i)
        torch.cuda.synchronize()
        edt = time.perf_counter() - t2
        s_att_ms, s_att_n = msa.timer_read(msa.MSA_TIMER_ATTENTION)
        s_rt_ms, s_rt_n = msa.timer_read(msa.MSA_TIMER_ROUTE)
        msa.timer_enable(False)
        dec_us = s_att_ms * 1e3 / max(s_att_n, 1)
        single = {"steps": n1, "ms_per_step": sdt * 1e3 / n1, "queries_per_s": w.B * n1 / sdt,
                  "decode_avg_launch_us": dec_us,
                  "routing_avg_launch_us": s_rt_ms * 1e3 / max(s_rt_n, 1),
                  "step_over_decode": sdt * 1e6 / n1 / dec_us,
                  "ms_per_step_with_events": edt * 1e3 / n1,
                  "host_issue_ms_per_step": hdt * 1e3 / n1,
                  "note": "ms_per_step from a pass with no events; launch durations from a "
                          "second pass of the same steps with every launch event-timed"}

    log("warmup")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("timed")
    msa.timer_reserve(2 * args.steps)  # attention + routing intervals, events made up front
    # events bracket every TIMER_PERIOD-th launch of the timed region (an odd
    # period samples both streams); bracketing every launch costs the step
    # about 2% (four event records per step on the streams)
    msa.timer_enable(True, TIMER_PERIOD)
    msa.timer_read(msa.MSA_TIMER_ATTENTION)
    msa.timer_read(msa.MSA_TIMER_ROUTE)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    att_ms, att_n = msa.timer_read(msa.MSA_TIMER_ATTENTION)
    rt_ms, rt_n = msa.timer_read(msa.MSA_TIMER_ROUTE)
    msa.timer_enable(False)
    log("done")
    ms = dt * 1e3 / args.steps
    qps = w.B * args.steps / dt

    # algorithmic bytes: every K and V element of each query's union once
    kv_bytes = w.B * (w.k * 512 + w.L_loc) * w.h_kv * 128 * 2 * 2
    att_avg_us = att_ms * 1e3 / max(att_n, 1)
    achieved = kv_bytes / (att_avg_us * 1e-6) / 1e9
    res = {
        "metric": METRIC, "value": qps, "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "1M-token bank decode: 2048 docs x 512 tokens (4096 chunks), "
                   "B=16, top-16, h_r=8 router heads, h_q=32, h_kv=8, d=128, local 4096, bf16",
                   "batch": w.B, "bank_tokens": w.T, "streams": len(streams),
                   "rotating_batches": args.batches},
        "roofline": {"kernel": "decode attention (split-K)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("decode_1m_counters"),
                     "bytes_per_launch": kv_bytes, "avg_launch_us": att_avg_us,
                     "launches": att_n,
                     # the two streams' launches overlap, so a launch's duration
                     # includes time shared with the other stream's launch; the
                     # whole-run rate counts every byte once over the wall clock
                     "aggregate_GBs": kv_bytes * args.steps / dt / 1e9,
                     "aggregate_frac": kv_bytes * args.steps / dt / 1e9 / HBM_PEAK_GBS,
                     "note": "frac: bytes per launch over the average event-timed launch, "
                             "each launch overlapped by the other stream's; aggregate_frac: "
                             "every launch's bytes over the timed wall clock; isolated: the "
                             "same launches on one stream, none overlapping"},
        # the routing scan streams every routing key and its norm once per step;
        # timed inside the two-stream step, where it overlaps the other
        # stream's attention
        "routing": {"kernel": "cosine routing scan (overlapped with attention)", "bound": "hbm",
                    "bytes_per_launch": w.C * w.h_r * (128 * 2 + 4),
                    "traffic": measured_traffic("route_1m_counters"),
                    "avg_launch_us": rt_ms * 1e3 / max(rt_n, 1), "launches": rt_n,
                    "achieved": w.C * w.h_r * (128 * 2 + 4) / (rt_ms * 1e-3 / max(rt_n, 1)) / 1e9,
                    "unit": "GB/s", "peak": HBM_PEAK_GBS},
        "hbm_read_stream_GBs": measured_read_rate(),
        "tokens_attended_per_s": qps * (w.k * 512 + w.L_loc),
        "bank_build_s": build_s,
    }
    if single is not None:
        iso = kv_bytes / (single["decode_avg_launch_us"] * 1e-6) / 1e9
        single.update({"decode_achieved_GBs": iso, "decode_frac": iso / HBM_PEAK_GBS})
        res["roofline"]["isolated"] = {"achieved": iso, "frac": iso / HBM_PEAK_GBS,
                                       "avg_launch_us": single["decode_avg_launch_us"],
                                       "launches": single["steps"],
                                       "source": "single-stream leg"}
        res["single_stream"] = single
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(w, r, k_raw, v_raw, raw0)
    if args.pooled_steps > 0:
        # compressed memory on the same bank: per-chunk means of the selected
        # documents' K/V (one log-weighted entry per 256 tokens) + local tokens
        log("pooled-memory decode")
        bank.attach_pooled()
        torch.cuda.synchronize()
        tb = time.perf_counter()
        bank.build_pooled(0, w.n_docs)
        torch.cuda.synchronize()
        pool_build_s = time.perf_counter() - tb

        def pstep(i):
            si = i % len(streams)
            q, q_route, k_loc, v_loc, L = batches[i % args.batches]
            bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=q_route, ws=ws[si],
                      outputs=outs[i % args.batches], stream=streams[si],
                      memory=msa.MSA_MEMORY_POOLED)

        for i in range(args.warmup):
            pstep(i)
        torch.cuda.synchronize()
        msa.timer_reserve(2 * args.pooled_steps)
        msa.timer_enable(True, TIMER_PERIOD)
        msa.timer_read(msa.MSA_TIMER_ATTENTION)
        msa.timer_read(msa.MSA_TIMER_ROUTE)
        t0 = time.perf_counter()
        for i in range(args.pooled_steps):
            pstep(i)
        torch.cuda.synchronize()
        pdt = time.perf_counter() - t0
        pms, pn = msa.timer_read(msa.MSA_TIMER_ATTENTION)
        msa.timer_read(msa.MSA_TIMER_ROUTE)
        msa.timer_enable(False)
        entries = w.k * (512 // 256)
        # bytes: the pooled K rows and V entries of 16 documents + the local K/V
        pbytes = w.B * (entries + w.L_loc) * w.h_kv * 128 * 2 * 2
        patt = pms * 1e-3 / max(pn, 1)
        res["pooled"] = {"workload": "compressed-memory decode on the 1M-token bank: the 16 "
                                     "selected documents as 2 chunk-mean entries each "
                                     "(log-weighted) + 4096 local tokens, B=16",
                         "queries_per_s": w.B * args.pooled_steps / pdt,
                         "ms_per_step": pdt * 1e3 / args.pooled_steps,
                         "pooled_build_s": pool_build_s,
                         "attention": {"bound": "hbm", "bytes_per_launch": pbytes,
                                       "avg_launch_us": patt * 1e6,
                                       "achieved": pbytes / patt / 1e9, "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": pbytes / patt / 1e9 / HBM_PEAK_GBS}}
    if args.prefill_steps > 0:
        del bank, batches, ws, outs, r, k_raw, v_raw, raw0
        torch.cuda.empty_cache()
        res["prefill"] = prefill_bench(args.prefill_steps, 3, args.prefill_splits)
    if args.host_bank_steps > 0:
        torch.cuda.empty_cache()
        res["host_bank"] = host_bank_bench(args.host_bank_steps, 2, args.host_cache_gb,
                                           args.prefetch_window)
    if args.interleave_steps > 0:
        torch.cuda.empty_cache()
        res["interleave"] = interleave_bench(args.interleave_steps, 1)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
