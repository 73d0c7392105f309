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
                scores=scores[0], out=out[0], bank=bank, k_loc=k_loc, v_loc=v_loc, L=L,
                q_pos=q_pos)


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


@pytest.mark.parametrize("cached", [False, True])
def test_prefill_on_a_host_resident_bank(msa, tmp_path, cached):
    """The blocked prefill on a host-resident copy of the bank (saved, then
    loaded into pinned host memory): the blocks' selections are read back
    and their documents copied -- into staging, or into a device cache --
    before the MFMA attention.  Ids, scores and outputs are bit-identical to
    the device bank's; with a cache, a second step finds every document
    resident and copies nothing."""
    w = S.workload("prefill_small")
    c = run_prefill(msa, w)
    path = str(tmp_path / "prefill_bank.safetensors")
    msa.save_bank(c["bank"], path)
    host = msa.load_bank(path, DEV, kv_loc="host")
    n_sel = (w.B // w.block) * w.k  # selections of one step
    if cached:
        host.set_cache(torch.empty((n_sel + 2) * host.cache_slot_bytes(), dtype=torch.uint8,
                                   device=DEV))
    args = (c["q"], c["q_pos"], w.k, c["k_loc"], c["v_loc"], c["L"])
    kw = dict(route_tokens=c["rt"], mode=msa.MSA_PREFILL, block=w.block)
    try:
        for rep in range(2 if cached else 1):
            ids, scores, out, st = host.step(*args, **kw)
            torch.cuda.synchronize()
            assert torch.equal(ids[0], c["ids"]) and torch.equal(scores[0], c["scores"])
            assert torch.equal(out[0], c["out"]), f"step {rep}"
            distinct = len(set(c["ids"].cpu().numpy().ravel().tolist()) - {-1})
            assert st.docs_copied + st.docs_cached == distinct
            if rep == 1:
                assert st.docs_copied == 0 and st.docs_cached == distinct
    finally:
        if cached:
            host.set_cache(None)


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


# channels of the rotary pairs (i, i + 64) with i >= 40: their angle moves
# by under 0.31 rad across the 192 query positions of the small prefill
LOWF = np.zeros(128, dtype=bool)
LOWF[40:64] = LOWF[104:128] = True


def dominant_token_case(w):
    """Queries and raw K with one key (document n_docs - 1, token 777, every
    KV head) aligned with query heads 0 and 1 of each group: about 300 log2
    units above every other score of theirs.  Heads 2 and 3 have no
    component along that key (zero in its channels), so their rows stay
    ordinary.  Returns (q, k_raw, v_raw, big document, token offset)."""
    big, pk = w.n_docs - 1, 777
    q = S.queries(w, DEV).clone()
    k_raw, v_raw = S.kv_raw(w, DEV)
    k_raw = k_raw.clone()
    lowf = torch.tensor(LOWF, device=DEV)
    spike_head = torch.arange(w.h_q, device=DEV) % w.G < 2
    q0 = torch.where(lowf, q[0, 0], torch.zeros_like(q[0, 0]))
    rest = q[:, ~spike_head]
    rest[..., lowf] = 0
    q[:, ~spike_head] = rest
    q[:, spike_head] = q0
    # the key q0 takes at the middle query position, expressed at the
    # document-local position pk; scaled so q0 . k ~ 300 log2 units
    p_mid = w.P0 + (w.L_loc - w.B) + w.B // 2
    q0n = M.np64(q0)
    k = O.rope_rotate(q0n, p_mid - pk, w.rope_base)
    k *= 300.0 * np.sqrt(w.d) / np.log2(np.e) / float(q0n @ q0n)
    t = int(S.doc_token_offsets(w)[big]) + pk
    k_raw[t] = torch.tensor(k, dtype=k_raw.dtype, device=DEV)
    return q, k_raw, v_raw, big, t


@pytest.mark.parametrize("splits", [1, 0])
def test_prefill_late_dominant_token(msa, splits):
    """A document ranked last holds a key that outscores everything the
    block's first tiles gave query heads 0 and 1 by far more than a softmax
    kept relative to the first tile's maximum can hold (2^300 overflows
    float32): the kernel must notice and recompute with each row's true
    maximum.  Heads 2 and 3 share the workgroups and keep ordinary scores.
    One split, and the automatic split count (partials merged)."""
    w = S.workload("prefill_small")
    q, k_raw, v_raw, big, t_big = dominant_token_case(w)
    r = S.route_vectors(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk[None], lv[None], w.P0)
    nb = w.B // w.block
    ids = torch.tensor([[b, b + 4, big] for b in range(nb)], dtype=torch.int32, device=DEV)
    q_pos = w.P0 + (w.L_loc - w.B)
    out = bank.attend(q, q_pos, ids, k_loc, v_loc, L, mode=msa.MSA_PREFILL, block=w.block,
                      splits=splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    c = dict(w=w, q=q, k_raw=k_raw, v_raw=v_raw, lk=lk, lv=lv)
    # the case is what it says: for every row of heads 0 and 1 the key
    # exceeds the first tile's maximum by over 128 log2 units
    kb = M.oracle_doc_kv(w, k_raw, v_raw, big)[0]
    spike_heads = [h for h in range(w.h_q) if h % w.G < 2]
    t0 = t_big - int(S.doc_token_offsets(w)[big])
    for blk in range(nb):
        k_first = M.oracle_doc_kv(w, k_raw, v_raw, blk)[0][:64]
        for i in (0, w.block - 1):
            qi = blk * w.block + i
            pos = w.P0 + (w.L_loc - w.B) + qi
            qr = O.rope_rotate(M.np64(q[qi]), np.full((w.h_q,), pos), w.rope_base)
            for h in spike_heads:
                g = h // w.G
                s_big = qr[h] @ kb[t0, g] / np.sqrt(w.d) * np.log2(np.e)
                s_first = np.max(k_first[:, g] @ qr[h]) / np.sqrt(w.d) * np.log2(np.e)
                assert s_big - s_first > 128, (blk, i, h, s_big, s_first)
    v_big = M.np64(v_raw[t_big])
    for blk in range(nb):
        ref, _ = oracle_block(c, None, None, blk, None, sel=ids[blk].tolist())
        got = out[blk * w.block:(blk + 1) * w.block]
        # heads 0 and 1: all weight on the one token
        for h in spike_heads:
            assert np.allclose(ref[:, h], v_big[h // w.G], atol=1e-12)
        mx, rel = M.check_out(got, ref, w.dtype, f"block {blk} splits {splits}")
        print(f"block {blk}: max abs {mx:.3e} rel rms {rel:.3e}")
