"""Throughput of the MSA hot path on one MI355X.

Default workload: routed decode at a 1M-token bank (2048 documents x 512
tokens, bf16, 8 router heads, 32 query / 8 KV heads, d = 128), batch 16,
top-16, 4096-token local context.  One step = route -> top-k -> gather ->
split-K attention for one batch of 16 queries, through msa_step.  Prints one
JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed decode queries/sec at 1M-token bank; % peak HBM GB/s; prefill MFMA %"
HBM_PEAK_GBS = 8000.0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--batches", type=int, default=4, help="rotating query batches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by document range; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_memory_amd import msa, synth as S

    dev = "cuda"
    w = S.workload("c2")
    print(f"[bench] building {w.name}: {w.n_docs} docs, {w.T} tokens", file=sys.stderr, flush=True)
    r = S.route_vectors(w, dev)
    k_raw, v_raw = S.kv_raw(w, dev)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, dev, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    del r, k_raw, v_raw
    batches = []
    for i in range(args.batches):
        q = S.queries(w, dev, batch=i)
        q_route = S.route_queries(w, dev, batch=i)
        lk, lv = S.local_raw(w, dev, batch=i)
        k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
        del lk, lv
        batches.append((q, q_route, k_loc, v_loc, L))
    ws = bank.workspace(msa.MSA_DECODE, w.B, w.h_q, w.k)
    outs = [(torch.empty((1, w.B, w.k), dtype=torch.int32, device=dev),
             torch.empty((1, w.B, w.k), dtype=torch.float32, device=dev),
             torch.empty((1, w.B, w.h_q, 128), dtype=torch.float32, device=dev))
            for _ in range(args.batches)]
    torch.cuda.synchronize()

    def step(i):
        q, q_route, k_loc, v_loc, L = batches[i % args.batches]
        bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=q_route, ws=ws,
                  outputs=outs[i % args.batches])

    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print("[bench] timed", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    qps = w.B * args.steps / dt
    kv_bytes = w.B * (w.k * 512 + w.L_loc) * w.h_kv * 128 * 2 * 2
    step_bytes = kv_bytes + w.C * w.h_r * 128 * 2 + w.C * w.h_r * 4
    res = {
        "metric": METRIC, "value": qps, "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "1M-token bank decode: 2048 docs x 512 tokens, B=16, top-16, "
                   "h_r=8, h_q=32, h_kv=8, d=128, local 4096, bf16", "batch": w.B,
                   "bank_tokens": w.T},
        "step_hbm_frac": step_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
