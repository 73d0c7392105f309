"""Test helpers: build a workload on the GPU through the C ABI and compute
the fp64 oracle's answer for the same inputs.

Inputs come from long_context_memory_amd.synth; expected values come from
oracle/ only.  Nothing here feeds a GPU result into the oracle except the
selection a GPU run made when it is a valid alternative under a near-tie
(then the oracle recomputes attention for that selection).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from long_context_memory_amd import synth as S
from oracle import msa_oracle as O

TOPK_TIE = 1e-4          # near-tie window on document scores
SCORE_TOL = 1e-4         # cosine document scores
OUT_TOL = {"bf16": 1e-2, "f32": 1e-5}   # max abs error of attention outputs
REL_RMS_TOL = {"bf16": 1e-2, "f32": 1e-6}


def np64(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).double().numpy()


def pool_oracle(w, r, slice_docs=256):
    """Oracle routing keys [C, h_r, 128] (rounded to storage) and inverse
    norms, pooled document slice by document slice to bound host memory."""
    off = S.doc_token_offsets(w)
    keys = []
    for n0 in range(0, w.n_docs, slice_docs):
        n1 = min(w.n_docs, n0 + slice_docs)
        rs = np64(r[off[n0]:off[n1]])
        keys.append(O.chunk_mean_pool(rs, w.doc_len[n0:n1]))
    kr = O.round_to_storage(np.concatenate(keys), w.dtype)
    return kr, O.inverse_norms(kr)


def check_topk(ids_gpu, scores_gpu, oracle_scores, k, tie=TOPK_TIE, score_tol=SCORE_TOL):
    """Top-k acceptance: ids equal the oracle's (order may differ only between
    documents whose oracle scores are within `tie` but not equal), except
    where the oracle's k-th and (k+1)-th scores are within `tie` but not
    equal: then every returned document must score >= s_k - tie and every
    document above s_k + tie must be returned.  Exact ties follow the lower-id
    rule everywhere: when the k-th and (k+1)-th oracle scores are equal the
    ids and their order must be the oracle's exactly, no document may be
    passed over for a higher id of exactly the same oracle score, and
    returned documents of equal oracle score come in increasing id order.
    Returned scores match the oracle's within `score_tol`.
    Returns the number of rows that fell in the near-tie case."""
    ids_gpu = np.asarray(ids_gpu)
    scores_gpu = np.asarray(scores_gpu, dtype=np.float64)
    B, N = oracle_scores.shape
    near = 0
    for b in range(B):
        o_ids, o_vals = O.select_topk(oracle_scores[b:b + 1], min(k + 1, N))
        o_ids, o_vals = o_ids[0], o_vals[0]
        g = ids_gpu[b]
        assert len(set(g.tolist())) == k, f"row {b}: repeated ids {g}"
        assert g.min() >= 0 and g.max() < N, f"row {b}: id out of range"
        sg = oracle_scores[b, g]
        np.testing.assert_allclose(scores_gpu[b], sg, atol=score_tol, rtol=0,
                                   err_msg=f"row {b}: document scores")
        # returned in rank order (by the GPU's own scores, ties to lower id)
        for r in range(k - 1):
            assert (scores_gpu[b, r] > scores_gpu[b, r + 1]) or (
                scores_gpu[b, r] == scores_gpu[b, r + 1] and g[r] < g[r + 1]), f"row {b}: order"
        # exact ties, anywhere: a returned document never outranks (or
        # displaces) a lower id of exactly the same oracle score
        for r in range(k):
            same = np.nonzero(oracle_scores[b] == sg[r])[0]
            lower = same[same < g[r]]
            assert set(lower.tolist()) <= set(g[:r].tolist()), \
                f"row {b}: id {g[r]} taken before a lower id of equal score {lower}"
        s_k = o_vals[k - 1]
        s_k1 = o_vals[k] if N > k else -np.inf
        # the cut inside an exact tie (identical documents) with no other
        # score near it: the lower-id rule fixes the set, as a clear gap does
        vals = oracle_scores[b]
        exact_cut = s_k == s_k1 and not np.any((np.abs(vals - s_k) < tie) & (vals != s_k))
        if exact_cut or s_k - s_k1 >= tie:
            assert set(g.tolist()) == set(o_ids[:k].tolist()), f"row {b}: ids {g} vs {o_ids[:k]}"
            for r in range(k - 1):  # order differs from the oracle's only inside a near-tie
                if g[r] != o_ids[r]:
                    s_o = oracle_scores[b, o_ids[r]]
                    assert abs(sg[r] - s_o) < tie and sg[r] != s_o, f"row {b}: rank {r}"
        else:
            near += 1
            assert np.all(sg >= s_k - tie), f"row {b}: below the near-tie window"
            must = np.nonzero(oracle_scores[b] > s_k + tie)[0]
            assert set(must.tolist()) <= set(g.tolist()), f"row {b}: missing a clear winner"
    return near


def check_out(out_gpu, out_ref, dtype, what=""):
    o = np.asarray(out_gpu, dtype=np.float64)
    err = np.abs(o - out_ref)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.sqrt(np.mean(err ** 2)) / max(np.sqrt(np.mean(out_ref ** 2)), 1e-30)) if err.size else 0.0
    assert mx <= OUT_TOL[dtype], f"{what}: max abs err {mx} > {OUT_TOL[dtype]}"
    assert rel <= REL_RMS_TOL[dtype], f"{what}: rel RMS err {rel} > {REL_RMS_TOL[dtype]}"
    return mx, rel


def doc_rows(w, n):
    off = S.doc_token_offsets(w)
    return int(off[n]), int(off[n + 1])


def oracle_doc_kv(w, k_raw, v_raw, n):
    """Oracle's stored K (document-RoPE'd, rounded) and V of document n, from
    the raw per-token K/V, natural layout [L, h_kv, 128]."""
    a, b = doc_rows(w, n)
    kr = O.bank_keys_rotated(np64(k_raw[a:b]), [b - a], w.rope_base, w.dtype)
    return kr, np64(v_raw[a:b])


def oracle_attend_decode(w, q_b, q_pos, ids_b, doc_kv, lk_raw_b, lv_b, pos0):
    """Oracle attention of one decode query over its selected documents
    (given as a dict id -> (K_rot, V)) and its local context."""
    L = lk_raw_b.shape[0]
    lk = O.round_to_storage(O.rope_rotate(lk_raw_b, (pos0 + np.arange(L))[:, None], w.rope_base),
                            w.dtype)
    Ks = [doc_kv[n][0] for n in ids_b] + [lk]
    Vs = [doc_kv[n][1] for n in ids_b] + [lv_b]
    K, V = np.concatenate(Ks), np.concatenate(Vs)
    qr = O.rope_rotate(q_b[None], np.full((1, q_b.shape[0]), q_pos), w.rope_base)
    return O.gqa_attention(qr, K, V)[0]


def natural_from_store_k(bank, n, kv_off=None):
    """Read document n's K from the bank store back into [L, h_kv, 128]."""
    L = bank.doc_len[n]
    o = (int(kv_off[n]) if kv_off is not None else sum(bank.doc_len[:n])) * bank.h_kv * 128
    blk = bank.k_store[o:o + L * bank.h_kv * 128].view(bank.h_kv, L, 128)
    return blk.permute(1, 0, 2)


def natural_from_store_v(bank, n, kv_off=None):
    """Read document n's V from the tile-blocked store back into [L, h_kv, 128]."""
    L = bank.doc_len[n]
    o = (int(kv_off[n]) if kv_off is not None else sum(bank.doc_len[:n])) * bank.h_kv * 128
    blk = bank.v_store[o:o + L * bank.h_kv * 128].view(bank.h_kv, L // 64, 128, 64)
    return blk.permute(1, 3, 0, 2).reshape(L, bank.h_kv, 128)


def local_v_natural(v_loc_seq):
    """One sequence of prepared local V [h_kv, Tp, 128, 64] -> [Tp*64, h_kv, 128]."""
    h, tp = v_loc_seq.shape[0], v_loc_seq.shape[1]
    return v_loc_seq.permute(1, 3, 0, 2).reshape(tp * 64, h, 128)


def ulp_diff_bf16(a, b):
    """Distance in bf16 units in the last place between two bf16 tensors."""
    ia = a.contiguous().view(torch.int16).to(torch.int32)
    ib = b.contiguous().view(torch.int16).to(torch.int32)
    # map to a monotone integer line
    ia = torch.where(ia < 0, -(ia & 0x7fff), ia)
    ib = torch.where(ib < 0, -(ib & 0x7fff), ib)
    return (ia - ib).abs()


def seeded_subset(n, m, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=min(m, n), replace=False))


def math_isclose(a, b, tol):
    return math.isclose(a, b, abs_tol=tol)


def pool_oracle_sliced(w, rows, slice_docs=64):
    """Like pool_oracle, with the routing vectors of documents [n0, n1)
    produced on demand by rows(t0, t1) (so 8M+ token banks need not be held
    in memory at once)."""
    off = S.doc_token_offsets(w)
    keys = []
    for n0 in range(0, w.n_docs, slice_docs):
        n1 = min(w.n_docs, n0 + slice_docs)
        rs = np64(rows(int(off[n0]), int(off[n1])))
        keys.append(O.chunk_mean_pool(rs, w.doc_len[n0:n1]))
        del rs
    kr = O.round_to_storage(np.concatenate(keys), w.dtype)
    return kr, O.inverse_norms(kr)


def doc_kv_from_rows(w, rows, n):
    """Oracle K (document-RoPE'd, rounded) and V of document n, the raw rows
    produced on demand by rows(t0, t1) -> (k_raw, v_raw)."""
    off = S.doc_token_offsets(w)
    a, b = int(off[n]), int(off[n + 1])
    k_raw, v_raw = rows(a, b)
    return (O.bank_keys_rotated(np64(k_raw), [b - a], w.rope_base, w.dtype), np64(v_raw))


def oracle_prefill_rows(w, q, lk, lv, doc_kv, sel, blk, queries):
    """Oracle prefill outputs of the given queries (indices inside block
    blk) attending to the documents `sel` (ids; doc_kv[id] = (K_rot, V)) and
    the causal local context.  q: [B, h_q, d] raw; lk, lv: [L_loc, h_kv, d]."""
    L, Lq, bsz = w.L_loc, w.B, w.block
    lkr = O.round_to_storage(O.rope_rotate(lk, (w.P0 + np.arange(L))[:, None], w.rope_base),
                             w.dtype)
    K = np.concatenate([doc_kv[n][0] for n in sel] + [lkr])
    V = np.concatenate([doc_kv[n][1] for n in sel] + [lv])
    n_doc = K.shape[0] - L
    outs = []
    for i in queries:
        qi = blk * bsz + i
        li = L - Lq + qi
        mask = np.ones((1, K.shape[0]), dtype=bool)
        mask[0, n_doc:] = np.arange(L) <= li
        qr = O.rope_rotate(q[qi][None], np.full((1, w.h_q), w.P0 + li), w.rope_base)
        outs.append(O.gqa_attention(qr, K, V, mask)[0])
    return np.stack(outs)



def check_decode_step(w, ids, scores, out, q, q_route, lk, lv, kr_o, inv_o, doc_kv, what=""):
    """A GPU decode step (ids, scores [B, k]; out [B, h_q, d]) against the
    oracle for the same inputs: top-k acceptance on the oracle's document
    scores, then attention over the oracle's selection (the GPU's where it is
    a valid alternative inside a near-tie).  doc_kv(n) gives the oracle's
    stored (K_rot, V) of document n.  Returns (max abs, rel RMS) error."""
    ids, scores = np.asarray(ids), np.asarray(scores)
    so = O.cosine_doc_scores(np64(q_route), kr_o, inv_o, w.doc_len)
    check_topk(ids, scores, so, w.k)
    o_ids, _ = O.select_topk(so, w.k)
    qn, lkn, lvn = np64(q), np64(lk), np64(lv)
    refs = []
    for b in range(ids.shape[0]):
        sel = o_ids[b] if set(o_ids[b].tolist()) == set(ids[b].tolist()) else ids[b]
        kv = {int(n): doc_kv(int(n)) for n in sel}
        refs.append(oracle_attend_decode(w, qn[b], w.q_pos, sel, kv, lkn[b], lvn[b], w.P0))
    return check_out(np.asarray(out), np.stack(refs), w.dtype, what)


def memo(fn):
    """fn(n) cached per argument (oracle document K/V are reused across steps)."""
    cache = {}

    def get(n):
        if n not in cache:
            cache[n] = fn(n)
        return cache[n]
    return get
