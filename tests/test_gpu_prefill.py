"""GPU parity of the blocked prefill (block-mean routing, shared top-k per
block, causal local context, MFMA attention) against the fp64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

from long_context_memory_amd import synth as S
from oracle import msa_oracle as O
import msa_cases as M

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def msa():
    from long_context_memory_amd import msa as m
    return m


def run_prefill(msa, w, splits=0):
    r = S.route_vectors(w, DEV)
    k_raw, v_raw = S.kv_raw(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    q = S.queries(w, DEV)
    rt = S.prefill_route_tokens(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk[None], lv[None], w.P0)
    q_pos = w.P0 + (w.L_loc - w.B)  # position of query 0
    ids, scores, out, _ = bank.step(q, q_pos, w.k, k_loc, v_loc, L, route_tokens=rt,
                                    mode=msa.MSA_PREFILL, block=w.block, splits=splits)
    torch.cuda.synchronize()
    return dict(w=w, r=r, k_raw=k_raw, v_raw=v_raw, q=q, rt=rt, lk=lk, lv=lv, ids=ids[0],
                scores=scores[0], out=out[0], bank=bank, k_loc=k_loc, v_loc=v_loc)


def oracle_block(c, kr_o, inv_o, blk, ids_gpu, queries=None, sel=None):
    """Oracle outputs of block `blk` (optionally a subset of its queries) with
    the oracle's own selection, or the GPU's when it is a valid near-tie, or
    the documents `sel` when given (no routing)."""
    w = c["w"]
    L, Lq, bsz = w.L_loc, w.B, w.block
    so = None
    if sel is None:
        qb = O.block_mean_queries(M.np64(c["rt"][blk * bsz:(blk + 1) * bsz]), bsz)
        so = O.cosine_doc_scores(qb, kr_o, inv_o, w.doc_len)
        o_ids, _ = O.select_topk(so, w.k)
        sel = o_ids[0] if set(o_ids[0].tolist()) == set(ids_gpu.tolist()) else ids_gpu
    kv = [M.oracle_doc_kv(w, c["k_raw"], c["v_raw"], n) for n in sel]
    lk = O.round_to_storage(O.rope_rotate(M.np64(c["lk"]), (w.P0 + np.arange(L))[:, None],
                                          w.rope_base), w.dtype)
    lv = M.np64(c["lv"])
    K = np.concatenate([x[0] for x in kv] + [lk])
    V = np.concatenate([x[1] for x in kv] + [lv])
    n_doc = K.shape[0] - L
    qs = range(bsz) if queries is None else queries
    outs = []
    for i in qs:
        qi = blk * bsz + i
        li = L - Lq + qi
        mask = np.ones((1, K.shape[0]), dtype=bool)
        mask[0, n_doc:] = np.arange(L) <= li
        qr = O.rope_rotate(M.np64(c["q"][qi])[None], np.full((1, w.h_q), w.P0 + li), w.rope_base)
        outs.append(O.gqa_attention(qr, K, V, mask)[0])
    return np.stack(outs), so


def test_prefill_small_matches_oracle(msa):
    w = S.workload("prefill_small")
    c = run_prefill(msa, w)
    kr_o, inv_o = M.pool_oracle(w, c["r"])
    nb = w.B // w.block
    qb = O.block_mean_queries(M.np64(c["rt"]), w.block)
    so = O.cosine_doc_scores(qb, kr_o, inv_o, w.doc_len)
    M.check_topk(c["ids"].cpu().numpy(), c["scores"].cpu().numpy(), so, w.k)
    out = c["out"].cpu().numpy()
    for blk in range(nb):
        ref, _ = oracle_block(c, kr_o, inv_o, blk, c["ids"][blk].cpu().numpy())
        mx, rel = M.check_out(out[blk * w.block:(blk + 1) * w.block], ref, w.dtype, f"block {blk}")
        print(f"block {blk}: max abs {mx:.3e} rel rms {rel:.3e}")


@pytest.mark.parametrize("g", [4, 2])
def test_prefill_skips_empty_id_slots(msa, g):
    # -1 and out-of-range ids select nothing: each block attends to its
    # remaining documents (block 2: none, the causal local context only);
    # G = 4 runs the matrix-core kernel, G = 2 the vector kernel
    w = S.workload("prefill_small")
    if w.h_q != g * w.h_kv:
        w = dataclasses.replace(w, h_q=g * w.h_kv, name=f"prefill_small_g{g}")
    c = run_prefill(msa, w)
    ids = c["ids"].clone()
    ids[0, -1] = -1
    ids[1, 0] = w.n_docs + 3
    ids[2, :] = -1
    k_loc, v_loc = c["k_loc"], c["v_loc"]
    q_pos = w.P0 + (w.L_loc - w.B)
    out = c["bank"].attend(c["q"], q_pos, ids, k_loc, v_loc, w.L_loc, mode=msa.MSA_PREFILL,
                           block=w.block)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ids_np = ids.cpu().numpy()
    for blk in range(w.B // w.block):
        sel = [int(n) for n in ids_np[blk] if 0 <= n < w.n_docs]
        ref, _ = oracle_block(c, None, None, blk, None, sel=sel)
        M.check_out(out[blk * w.block:(blk + 1) * w.block], ref, w.dtype, f"block {blk}")


def test_prefill_splits_agree(msa):
    w = S.workload("prefill_small")
    a = run_prefill(msa, w, splits=1)["out"]
    scale = float(a.abs().max())
    # 200 splits exceed a block's ~100 tiles: empty splits merge as nothing
    for s in (5, 200):
        b = run_prefill(msa, w, splits=s)["out"]
        assert float((a - b).abs().max()) <= 2.0 ** -8 * scale, s


def test_prefill_vector_path_g2(msa):
    # h_q / h_kv = 2 takes the per-query vector kernel
    w = dataclasses.replace(S.workload("prefill_small"), h_q=16, name="prefill_small_g2")
    c = run_prefill(msa, w)
    kr_o, inv_o = M.pool_oracle(w, c["r"])
    out = c["out"].cpu().numpy()
    for blk in range(w.B // w.block):
        ref, _ = oracle_block(c, kr_o, inv_o, blk, c["ids"][blk].cpu().numpy())
        M.check_out(out[blk * w.block:(blk + 1) * w.block], ref, w.dtype, f"g2 block {blk}")


def test_prefill_float32_bank(msa):
    # float32 storage takes the per-query vector kernel; outputs within the
    # float32 tolerance
    w = dataclasses.replace(S.workload("prefill_small"), dtype="f32", doc_len=[2048] * 6, B=128,
                            L_loc=150, name="prefill_small_f32")
    c = run_prefill(msa, w)
    kr_o, inv_o = M.pool_oracle(w, c["r"])
    qb = O.block_mean_queries(M.np64(c["rt"]), w.block)
    so = O.cosine_doc_scores(qb, kr_o, inv_o, w.doc_len)
    M.check_topk(c["ids"].cpu().numpy(), c["scores"].cpu().numpy(), so, w.k)
    out = c["out"].cpu().numpy()
    for blk in range(w.B // w.block):
        ref, _ = oracle_block(c, kr_o, inv_o, blk, c["ids"][blk].cpu().numpy())
        mx, rel = M.check_out(out[blk * w.block:(blk + 1) * w.block], ref, w.dtype, f"f32 block {blk}")
        print(f"f32 block {blk}: max abs {mx:.3e} rel rms {rel:.3e}")
