"""HIP graph capture of device-bank calls through the C ABI.

The kernel launches of one call are captured once and replayed.
- Calls covered: msa_step (multi-hop decode with exclusion, whose bitmap is
  cleared at the start of every call, and the blocked prefill) and
  msa_attend.
- Every replay must reproduce the eager call bit for bit: the same kernels
  run on the same inputs. Between replays the test runs eager calls of its
  own and synchronises.
- A replay after the inputs are changed in place must match an eager call
  on the new inputs.
"""
import pytest
import torch

from long_context_memory_amd import synth as S

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPLAYS = 3


@pytest.fixture(scope="module")
def msa():
    from long_context_memory_amd import msa as m
    return m


def capture(fn):
    """Warm up on a side stream (first-call set-up stays out of the graph),
    then capture fn's launches."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def poison(outs):
    for t in outs:
        t.fill_(-5 if t.dtype == torch.int32 else float("nan"))


def replay_and_compare(g, outs, expect, eager_between, what, names=("ids", "scores", "out")):
    for r in range(REPLAYS):
        poison(outs)
        eager_between()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(names, outs, expect):
            assert torch.equal(got, ref), f"{what}: replay {r}: {name} differs from the eager call"


def bank_of(msa, w):
    r = S.route_vectors(w, DEV)
    k_raw, v_raw = S.kv_raw(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    return bank


def test_graph_interleave_step_with_exclusion(msa):
    w = S.workload("interleave_small")
    bank = bank_of(msa, w)
    q = S.queries(w, DEV)
    q_route = S.route_queries(w, DEV).clone()
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    wp = S.interleave_projection(w, DEV)
    ws = bank.workspace(msa.MSA_DECODE, w.B, w.h_q, w.k, hops=w.hops)
    shape = (w.hops, w.B, w.k)
    outs = (torch.empty(shape, dtype=torch.int32, device=DEV),
            torch.empty(shape, dtype=torch.float32, device=DEV),
            torch.empty((w.hops, w.B, w.h_q, 128), dtype=torch.float32, device=DEV))

    def call(qr, outputs, ws_=ws):
        return bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=qr, hops=w.hops, w_proj=wp,
                         exclude_selected=True, ws=ws_, outputs=outputs)

    def fresh():
        return tuple(torch.empty_like(t) for t in outs)

    eager = fresh()
    call(q_route, eager)
    torch.cuda.synchronize()
    # the exclusion is live: no document repeats across a row's hops
    ids = eager[0].cpu()
    for b in range(w.B):
        sel = ids[:, b].flatten().tolist()
        assert len(set(sel)) == len(sel)

    g = capture(lambda: call(q_route, outs))
    other_q = torch.flip(q_route, dims=[0]).contiguous()
    other_ws = torch.empty_like(ws)
    other = fresh()
    replay_and_compare(g, outs, eager, lambda: call(other_q, other, other_ws),
                       "interleave step")

    # new router queries written in place: the graph reads them
    q_route.copy_(other_q)
    eager2 = fresh()
    call(q_route, eager2, other_ws)
    torch.cuda.synchronize()
    assert not torch.equal(eager2[0], eager[0])
    replay_and_compare(g, outs, eager2, lambda: None, "interleave step, new inputs")


def test_graph_prefill_step(msa):
    w = S.workload("prefill_small")
    bank = bank_of(msa, w)
    q = S.queries(w, DEV).clone()
    rt = S.prefill_route_tokens(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk[None], lv[None], w.P0)
    q_pos = w.P0 + (w.L_loc - w.B)
    n_groups = w.B // w.block
    ws = bank.workspace(msa.MSA_PREFILL, w.B, w.h_q, w.k, block=w.block)
    outs = (torch.empty((1, n_groups, w.k), dtype=torch.int32, device=DEV),
            torch.empty((1, n_groups, w.k), dtype=torch.float32, device=DEV),
            torch.empty((1, w.B, w.h_q, 128), dtype=torch.float32, device=DEV))

    def call(outputs, ws_=ws):
        return bank.step(q, q_pos, w.k, k_loc, v_loc, L, route_tokens=rt,
                         mode=msa.MSA_PREFILL, block=w.block, ws=ws_, outputs=outputs)

    def fresh():
        return tuple(torch.empty_like(t) for t in outs)

    eager = fresh()
    call(eager)
    torch.cuda.synchronize()
    g = capture(lambda: call(outs))
    other_ws = torch.empty_like(ws)
    other = fresh()
    replay_and_compare(g, outs, eager, lambda: call(other, other_ws), "prefill step")

    q.mul_(-1.0)  # new attention queries, same routing
    eager2 = fresh()
    call(eager2, other_ws)
    torch.cuda.synchronize()
    assert torch.equal(eager2[0], eager[0]) and not torch.equal(eager2[2], eager[2])
    replay_and_compare(g, outs, eager2, lambda: None, "prefill step, new inputs")


def test_graph_attend(msa):
    w = S.workload("decode_small")
    bank = bank_of(msa, w)
    q = S.queries(w, DEV).clone()
    q_route = S.route_queries(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    ids, scores = bank.route(q_route, w.k)
    ws = bank.workspace(msa.MSA_DECODE, w.B, w.h_q, w.k)
    out = torch.empty((w.B, w.h_q, 128), dtype=torch.float32, device=DEV)

    def call(o, ws_=ws):
        return bank.attend(q, w.q_pos, ids, k_loc, v_loc, L, ws=ws_, out=o)

    eager = torch.empty_like(out)
    call(eager)
    torch.cuda.synchronize()
    g = capture(lambda: call(out))
    other_ws = torch.empty_like(ws)
    other = torch.empty_like(out)
    replay_and_compare(g, (out,), (eager,), lambda: call(other, other_ws), "attend",
                       names=("out",))
