"""Exact ties in routing, on the GPU through the C ABI: documents whose
routing vectors are bit-identical get bit-identical scores, and top-k keeps
the lower document id (ties broken toward the lower id, output in rank
order).  The bank holds copies of documents

  - across a 64-chunk routing tile boundary (document 21 spans chunks 63-65,
    its copy, document 5, sits inside the first tile),
  - inside the selected set (documents 30, 33 and 37 are one document three
    times), and
  - at the k-cut, where only some members of a tied group fit.

Router queries are planted on the documents' pooled keys (computed by the
oracle) with weights that put each tied group where the case wants it; the
oracle's own exact ties are asserted first, so the case is what it says.
"""
import numpy as np
import pytest
import torch

from long_context_memory_amd import synth as S
from oracle import msa_oracle as O
import msa_cases as M

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (copy source, copy destination): destination rows := source rows
COPIES = [(21, 5), (30, 33), (30, 37), (44, 50)]
# per query: [(document, weight)] planted into the router query
PLANTS = [
    # 0: every tied group inside the top-8 (30/33/37 and 5/21), plus 1, 2, 3
    [(30, 1.0), (21, 1.0), (1, 1.0), (2, 1.0), (3, 1.0)],
    # 1: 44/50 tie at the cut: seven strong targets, the pair weaker
    [(1, 1.0), (2, 1.0), (3, 1.0), (4, 1.0), (6, 1.0), (7, 1.0), (8, 1.0), (44, 0.6)],
    # 2: the tile-straddling pair 5/21 at the cut
    [(10, 1.0), (11, 1.0), (12, 1.0), (13, 1.0), (14, 1.0), (15, 1.0), (16, 1.0), (21, 0.6)],
    # 3: a three-way tie (30/33/37) for the last two places
    [(10, 1.0), (11, 1.0), (12, 1.0), (13, 1.0), (14, 1.0), (15, 1.0), (30, 0.6)],
]


@pytest.fixture(scope="module")
def msa():
    from long_context_memory_amd import msa as m
    return m


def tie_workload(dtype):
    # 40 documents of 3 chunks, then 16 of 2: 152 chunks in tiles of 64
    # (the last one ragged); document 21 covers chunks 63, 64 and 65
    return S.Workload("ties_" + dtype, dtype, [768] * 40 + [512] * 16, h_r=8, h_kv=8, h_q=32,
                      k=8, B=len(PLANTS), L_loc=100, seed=2101)


def planted_queries(w, kr_o):
    off = O.chunk_offsets(w.doc_len)
    q = np.zeros((w.B, w.h_r, w.d_r))
    for b, plant in enumerate(PLANTS):
        for n, wt in plant:
            q[b] += wt * kr_o[off[n]]  # the document's first chunk key, every head
    return torch.tensor(q, dtype=torch.float32, device=DEV)


def build_case(msa, dtype):
    w = tie_workload(dtype)
    off = S.doc_token_offsets(w)
    r = S.route_vectors(w, DEV).clone()
    for src, dst in COPIES:
        assert w.doc_len[src] == w.doc_len[dst]
        r[off[dst]:off[dst + 1]] = r[off[src]:off[src + 1]]
    k_raw, v_raw = S.kv_raw(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    kr_o, inv_o = M.pool_oracle(w, r)
    qr = planted_queries(w, kr_o)
    torch.cuda.synchronize()
    so = O.cosine_doc_scores(M.np64(qr), kr_o, inv_o, w.doc_len)
    return w, bank, r, k_raw, v_raw, kr_o, inv_o, qr, so


def assert_designed_ties(w, so):
    """The oracle sees the ties the case plants (so the GPU check below
    tests what it claims to)."""
    for src, dst in COPIES:
        assert np.array_equal(so[:, src], so[:, dst]), (src, dst)
    o_ids, o_vals = O.select_topk(so, w.k + 2)
    k = w.k
    # query 0: all tied groups inside the top-k
    assert {30, 33, 37, 5, 21} <= set(o_ids[0, :k].tolist())
    # query 1: 44 and 50 straddle the cut, and nothing else is near it
    assert o_ids[1, k - 1] == 44 and o_ids[1, k] == 50 and o_vals[1, k - 1] == o_vals[1, k]
    # query 2: 5 and 21 straddle the cut
    assert o_ids[2, k - 1] == 5 and o_ids[2, k] == 21 and o_vals[2, k - 1] == o_vals[2, k]
    # query 3: three tied documents for the last two places
    assert list(o_ids[3, k - 2:k + 1]) == [30, 33, 37]
    for b in (1, 2, 3):  # clear gaps around the tied group at the cut
        s = o_vals[b, k - 1]
        others = so[b][so[b] != s]
        assert np.min(np.abs(others - s)) > 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_ties_go_to_the_lower_id(msa, dtype):
    w, bank, *_rest, kr_o, inv_o, qr, so = build_case(msa, dtype)
    assert_designed_ties(w, so)
    ids, scores = bank.route(qr, w.k)
    torch.cuda.synchronize()
    ids, scores = ids.cpu().numpy(), scores.cpu().numpy()
    M.check_topk(ids, scores, so, w.k)
    o_ids, _ = O.select_topk(so, w.k)
    for b in range(w.B):
        row = ids[b].tolist()
        # bit-identical documents get bit-identical GPU scores
        for src, dst in COPIES:
            if src in row and dst in row:
                assert scores[b, row.index(src)] == scores[b, row.index(dst)]
        # tied groups: consecutive, in increasing id order; at the cut only
        # the lowest ids get in
        for grp in ([5, 21], [30, 33, 37], [44, 50]):
            got = [n for n in row if n in grp]
            want = [n for n in o_ids[b].tolist() if n in grp]
            assert got == want, f"query {b}: tied group {grp}: got {got}, oracle {want}"
            if len(got) > 1:
                pos = [row.index(n) for n in got]
                assert pos == list(range(pos[0], pos[0] + len(pos))), f"query {b}: {row}"
    assert 44 in ids[1] and 50 not in ids[1]
    assert 5 in ids[2] and 21 not in ids[2]
    assert 30 in ids[3] and 33 in ids[3] and 37 not in ids[3]


def test_exact_ties_through_a_full_step(msa):
    """The same selections inside msa_step, and attention over them against
    the oracle."""
    w, bank, r, k_raw, v_raw, kr_o, inv_o, qr, so = build_case(msa, "bf16")
    q = S.queries(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    ids, scores, out, _ = bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=qr)
    torch.cuda.synchronize()
    ids_np = ids[0].cpu().numpy()
    M.check_topk(ids_np, scores[0].cpu().numpy(), so, w.k)
    o_ids, _ = O.select_topk(so, w.k)
    for b in range(w.B):  # clear gaps and exact ties: the oracle's set
        assert set(ids_np[b].tolist()) == set(o_ids[b].tolist()), f"query {b}"
    doc_kv = {n: M.oracle_doc_kv(w, k_raw, v_raw, n) for n in set(o_ids.ravel().tolist())}
    qn, lkn, lvn = M.np64(q), M.np64(lk), M.np64(lv)
    ref = np.stack([M.oracle_attend_decode(w, qn[b], w.q_pos, o_ids[b], doc_kv, lkn[b], lvn[b],
                                           w.P0) for b in range(w.B)])
    M.check_out(out[0].cpu().numpy(), ref, w.dtype, "ties step")
