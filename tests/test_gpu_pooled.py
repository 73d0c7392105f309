"""GPU parity of the compressed memory (per-chunk means of the selected
documents' K/V, each entry log-weighted by the 256 tokens it stands for)
against the fp64 oracle, through the C ABI."""
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


_CACHE = {}


def pooled_case(msa, name):
    if name in _CACHE:
        return _CACHE[name]
    w = S.workload(name)
    r = S.route_vectors(w, DEV)
    k_raw, v_raw = S.kv_raw(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    bank.attach_pooled()
    bank.build_pooled(0, w.n_docs)
    kr_o, inv_o = M.pool_oracle(w, r)
    if w.plant == "pooled_key":
        _, ch = S.pooled_key_target(w)
        q_route = S.pooled_key_query(w, kr_o[ch], DEV)
    else:
        q_route = S.route_queries(w, DEV)
    q = S.queries(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    torch.cuda.synchronize()
    c = dict(w=w, r=r, k_raw=k_raw, v_raw=v_raw, bank=bank, kr_o=kr_o, inv_o=inv_o,
             q_route=q_route, q=q, lk=lk, lv=lv, k_loc=k_loc, v_loc=v_loc, L=L)
    _CACHE[name] = c
    return c


def oracle_pooled(c):
    """The oracle's compressed memory [C, h_kv, d] x 2, from its own stored
    (rotated, rounded) K and V, document by document."""
    w = c["w"]
    off = S.doc_token_offsets(w)
    pk, pv = [], []
    for n in range(w.n_docs):
        a, b = int(off[n]), int(off[n + 1])
        kr = O.bank_keys_rotated(M.np64(c["k_raw"][a:b]), [b - a], w.rope_base, w.dtype)
        k_, v_ = O.pooled_kv(kr, M.np64(c["v_raw"][a:b]), [b - a], w.dtype)
        pk.append(k_)
        pv.append(v_)
    return np.concatenate(pk), np.concatenate(pv)


def gpu_pooled(bank):
    """The GPU's pooled stores read back into [C, h_kv, d] x 2."""
    h, pk, pv, voff = bank.h_kv, [], [], 0
    koff = 0
    for L in bank.doc_len:
        P = L // 256
        Pp = (P + 63) // 64 * 64
        pk.append(bank.pool_k[koff * h * 128:(koff + P) * h * 128].view(h, P, 128).permute(1, 0, 2))
        blk = bank.pool_v[voff * h * 128:(voff + Pp) * h * 128].view(h, Pp // 64, 128, 64)
        full = blk.permute(1, 3, 0, 2).reshape(Pp, h, 128)
        assert float(full[P:].abs().max()) == 0.0 if Pp > P else True  # zero padding
        pv.append(full[:P])
        koff += P
        voff += Pp
    return torch.cat(pk), torch.cat(pv)


@pytest.mark.parametrize("name", ["tiny_f32_small", "decode_small", "decode_1m"])
def test_pooled_stores_match_oracle(msa, name):
    c = pooled_case(msa, name)
    w = c["w"]
    pk_g, pv_g = gpu_pooled(c["bank"])
    pk_o, pv_o = oracle_pooled(c) if name != "decode_1m" else (None, None)
    if pk_o is None:  # full size: a seeded sample of documents
        off = S.doc_token_offsets(w)
        coff = np.concatenate([[0], np.cumsum(np.asarray(w.doc_len) // 256)])
        for n in M.seeded_subset(w.n_docs, 16, 9):
            a, b = int(off[n]), int(off[n + 1])
            kr = O.bank_keys_rotated(M.np64(c["k_raw"][a:b]), [b - a], w.rope_base, w.dtype)
            ko, vo = O.pooled_kv(kr, M.np64(c["v_raw"][a:b]), [b - a], w.dtype)
            kg, vg = pk_g[coff[n]:coff[n + 1]], pv_g[coff[n]:coff[n + 1]]
            np.testing.assert_array_equal(M.np64(vg), vo)
            assert int(M.ulp_diff_bf16(kg.cpu(), torch.from_numpy(ko).to(kg.dtype)).max()) <= 1
        return
    np.testing.assert_array_equal(M.np64(pv_g), pv_o)  # V: exact sums, one rounding
    if w.dtype == "bf16":
        ud = M.ulp_diff_bf16(pk_g.cpu(), torch.from_numpy(pk_o).to(pk_g.dtype))
        assert int(ud.max()) <= 1 and float((ud > 0).float().mean()) < 1e-2
    else:
        np.testing.assert_allclose(M.np64(pk_g), pk_o, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("name", ["tiny_f32_small", "decode_small", "decode_1m"])
def test_pooled_decode_matches_oracle(msa, name):
    c = pooled_case(msa, name)
    w = c["w"]
    ids, scores, out, st = c["bank"].step(c["q"], w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"],
                                          q_route=c["q_route"], memory=msa.MSA_MEMORY_POOLED)
    torch.cuda.synchronize()
    ids_np = ids[0].cpu().numpy()
    so = O.cosine_doc_scores(M.np64(c["q_route"]), c["kr_o"], c["inv_o"], w.doc_len)
    M.check_topk(ids_np, scores[0].cpu().numpy(), so, w.k)
    pk_o, pv_o = oracle_pooled(c)
    q, lk, lv = M.np64(c["q"]), M.np64(c["lk"]), M.np64(c["lv"])
    o_ids, _ = O.select_topk(so, w.k)
    coff = np.concatenate([[0], np.cumsum(np.asarray(w.doc_len) // 256)])
    refs = []
    for b in range(w.B):
        sel = o_ids[b] if set(o_ids[b].tolist()) == set(ids_np[b].tolist()) else ids_np[b]
        L = lk.shape[1]
        lkr = O.round_to_storage(O.rope_rotate(lk[b], (w.P0 + np.arange(L))[:, None], w.rope_base),
                                 w.dtype)
        K = np.concatenate([pk_o[coff[n]:coff[n + 1]] for n in sel] + [lkr])
        V = np.concatenate([pv_o[coff[n]:coff[n + 1]] for n in sel] + [lv[b]])
        n_pool = K.shape[0] - L
        bias = np.concatenate([np.full(n_pool, np.log(256.0)), np.zeros(L)])
        qr = O.rope_rotate(q[b][None], np.full((1, w.h_q), w.q_pos), w.rope_base)
        refs.append(O.gqa_attention(qr, K, V, None, bias)[0])
    mx, rel = M.check_out(out[0].cpu().numpy(), np.stack(refs), w.dtype, f"pooled {name}")
    print(f"pooled {name}: max abs {mx:.3e} rel rms {rel:.3e}")
    # the composed oracle agrees with this per-query assembly
    if name == "decode_small":
        full_o, _, _ = O.pooled_decode_step(q, w.q_pos, M.np64(c["q_route"]), c["kr_o"], c["inv_o"],
                                            pk_o, pv_o, w.doc_len, lk, lv, w.P0, w.k, w.rope_base,
                                            w.dtype)
        M.check_out(out[0].cpu().numpy(), full_o, w.dtype, "pooled_decode_step")


def test_pooled_attend_equals_step(msa):
    c = pooled_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    ids, _, out, _ = bank.step(c["q"], w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"],
                               q_route=c["q_route"], memory=msa.MSA_MEMORY_POOLED)
    out2 = bank.attend(c["q"], w.q_pos, ids[0], c["k_loc"], c["v_loc"], c["L"],
                       memory=msa.MSA_MEMORY_POOLED)
    torch.cuda.synchronize()
    assert torch.equal(out[0], out2)


def test_pooled_on_host_bank_needs_no_copies(msa):
    """A host-resident bank answers from pooled stores built on its device
    twin: no host->device copies, results identical to the twin's."""
    w = S.workload("host_small")
    slot_len, kv_off = S.host_slot_layout(w)
    kr = S.keys_direct(w, DEV).to(w.torch_dtype).permute(1, 0, 2).contiguous()
    hb = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, kv_loc="host", kv_off=kv_off,
                  kv_tokens=int(sum(slot_len)), rope_base=w.rope_base, kr=kr)
    hb.build(0, w.n_docs)
    msa.fill_host_store(hb, slot_len, lambda t0, t1: S.host_kv_raw(w, DEV, t0, t1))
    db = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, kv_off=kv_off, kv_tokens=hb.kv_tokens,
                  rope_base=w.rope_base, kr=kr, k_store=hb.k_store.to(DEV), v_store=hb.v_store.to(DEV))
    db.build(0, w.n_docs)
    db.attach_pooled()
    db.build_pooled(0, w.n_docs)
    hb.use_pooled(db.pool_k, db.pool_v)
    q, qr = S.queries(w, DEV), S.route_queries(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = hb.prepare_local(lk, lv, w.P0)
    a = db.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=qr, memory=msa.MSA_MEMORY_POOLED)
    b = hb.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=qr, memory=msa.MSA_MEMORY_POOLED)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])
    assert b[3].docs_copied == 0 and b[3].bytes_copied == 0


def test_pooled_errors(msa):
    c = pooled_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    plain = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    plain.build(0, w.n_docs, c["r"], c["k_raw"], c["v_raw"])
    with pytest.raises(msa.MSAError, match="pooled"):
        plain.step(c["q"], w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"], q_route=c["q_route"],
                   memory=msa.MSA_MEMORY_POOLED)
    pw = S.workload("prefill_small")
    with pytest.raises(msa.MSAError):
        bank.attend(S.queries(pw, DEV)[:64], 0, torch.zeros((1, w.k), dtype=torch.int32, device=DEV),
                    c["k_loc"][:1], c["v_loc"][:1], c["L"], mode=msa.MSA_PREFILL,
                    memory=msa.MSA_MEMORY_POOLED)
