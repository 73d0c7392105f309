"""GPU tests of bank growth and persistence through the C ABI: a bank grown
by appending documents (and building only the new ones) matches the oracle
and is bit-identical to one built in one go; so is a host-resident store the
caller grows (keys built by the library, K/V written by the caller at
offsets of its choice); capacity errors are reported; a bank saved to a file
and loaded again -- into device or pinned host memory -- matches the oracle
and gives identical results."""
import numpy as np
import pytest
import torch

from long_context_memory_amd import synth as S
import msa_cases as M

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def msa():
    from long_context_memory_amd import msa as m
    return m


def full_and_grown(msa, w, n_first):
    off = S.doc_token_offsets(w)
    r = S.route_vectors(w, DEV)
    k_raw, v_raw = S.kv_raw(w, DEV)
    full = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    full.build(0, w.n_docs, r, k_raw, v_raw)
    t1 = int(off[n_first])
    grown = msa.Bank(w.doc_len[:n_first], w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base,
                     chunk_cap=w.C, kv_tokens=w.T)
    grown.build(0, n_first, r[:t1], k_raw[:t1], v_raw[:t1])
    grown.append(w.doc_len[n_first:])
    grown.build(n_first, w.n_docs, r[t1:], k_raw[t1:], v_raw[t1:])
    torch.cuda.synchronize()
    return full, grown


def step_case(w, bank):
    q = S.queries(w, DEV)
    qr = S.route_queries(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    return bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=qr)


_ORACLE = {}


def oracle_check(w, res, what):
    """A decode step's (ids, scores, out, stats) on the workload's batch-0
    inputs against the oracle (keys pooled from the raw routing vectors, K/V
    rotated from the raw K/V: nothing from the GPU)."""
    if w.name not in _ORACLE:
        r = S.route_vectors(w, DEV)
        k_raw, v_raw = S.kv_raw(w, DEV)
        kr_o, inv_o = M.pool_oracle(w, r)
        _ORACLE[w.name] = (kr_o, inv_o, M.memo(lambda n: M.oracle_doc_kv(w, k_raw, v_raw, n)))
    kr_o, inv_o, doc_kv = _ORACLE[w.name]
    q = S.queries(w, DEV)
    qr = S.route_queries(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    ids, scores, out, _ = res
    torch.cuda.synchronize()
    return M.check_decode_step(w, ids[0].cpu(), scores[0].cpu(), out[0].cpu(), q, qr, lk, lv,
                               kr_o, inv_o, doc_kv, what)


def test_append_matches_full_build(msa):
    w = S.workload("decode_small")
    full, grown = full_and_grown(msa, w, 17)
    C = w.C
    assert torch.equal(grown.kr[:, :C], full.kr) and torch.equal(grown.inv_norm[:, :C], full.inv_norm)
    assert torch.equal(grown.k_store, full.k_store) and torch.equal(grown.v_store, full.v_store)
    a = step_case(w, full)
    b = step_case(w, grown)
    torch.cuda.synchronize()
    oracle_check(w, b, "grown bank")
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    # unfilled capacity rows are never read: poison them and route again
    g2 = msa.Bank(w.doc_len[:17], w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base,
                  chunk_cap=w.C + 64, kv_tokens=w.T)
    g2.kr.fill_(float("nan"))
    g2.inv_norm.fill_(float("nan"))
    off = S.doc_token_offsets(w)
    t1 = int(off[17])
    r = S.route_vectors(w, DEV)
    k_raw, v_raw = S.kv_raw(w, DEV)
    g2.build(0, 17, r[:t1], k_raw[:t1], v_raw[:t1])
    g2.append(w.doc_len[17:])
    g2.build(17, w.n_docs, r[t1:], k_raw[t1:], v_raw[t1:])
    c = step_case(w, g2)
    torch.cuda.synchronize()
    oracle_check(w, c, "grown bank with spare capacity")
    for x, y in zip(a[:3], c[:3]):
        assert torch.equal(x, y)


def test_append_to_a_host_resident_store(msa):
    """A host-resident bank grows as its owner writes K/V: the library pools
    the new documents' keys, the caller writes their K/V (store layout) at
    offsets it chooses -- here in reverse order after the first documents."""
    w = S.workload("decode_small")
    off = S.doc_token_offsets(w)
    n0 = 17
    t1 = int(off[n0])
    full, _ = full_and_grown(msa, w, n0)  # its stores give the caller's K/V blocks
    r = S.route_vectors(w, DEV)
    host = msa.Bank(w.doc_len[:n0], w.h_r, w.h_kv, w.dtype, DEV, kv_loc="host",
                    kv_tokens=w.T, chunk_cap=w.C, rope_base=w.rope_base)
    host.build(0, n0, r[:t1])
    per_tok = w.h_kv * 128

    def write(n, dst_tok):
        a, L = int(off[n]) * per_tok, w.doc_len[n] * per_tok
        host.k_store[dst_tok * per_tok:dst_tok * per_tok + L].copy_(full.k_store[a:a + L])
        host.v_store[dst_tok * per_tok:dst_tok * per_tok + L].copy_(full.v_store[a:a + L])

    for n in range(n0):
        write(n, int(off[n]))
    new = list(range(n0, w.n_docs))
    kv_off, t = [], w.T  # the first new document at the end of the store
    for n in new:
        t -= w.doc_len[n]
        kv_off.append(t)
    host.append([w.doc_len[n] for n in new], kv_off=kv_off)
    host.build(n0, w.n_docs, r[t1:])
    for n, o in zip(new, kv_off):
        write(n, o)
    torch.cuda.synchronize()
    assert torch.equal(host.kr, full.kr) and torch.equal(host.inv_norm, full.inv_norm)
    res = step_case(w, host)
    oracle_check(w, res, "host store after append")
    ref = step_case(w, full)
    torch.cuda.synchronize()
    for x, y in zip(ref[:3], res[:3]):
        assert torch.equal(x, y)
    assert res[3].docs_copied > 0


def test_append_capacity_errors(msa):
    w = S.workload("decode_small")
    b = msa.Bank(w.doc_len[:10], w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base,
                 chunk_cap=w.C, kv_tokens=sum(w.doc_len[:12]))
    with pytest.raises(msa.MSAError, match="kv_tokens"):
        b.append(w.doc_len[10:20])  # K/V store too small
    assert b.n_docs == 10 and b.info().n_docs == 10
    b.append(w.doc_len[10:12])
    assert b.info().n_docs == 12
    nocap = msa.Bank(w.doc_len[:10], w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base,
                     kv_tokens=w.T)
    with pytest.raises(msa.MSAError, match="chunk_cap"):
        nocap.append(w.doc_len[10:12])
    with pytest.raises(msa.MSAError):
        b.append([300])  # not a multiple of 256


def test_save_load_roundtrip(msa, tmp_path):
    w = S.workload("decode_small")
    full, _ = full_and_grown(msa, w, 30)
    ref = step_case(w, full)
    path = str(tmp_path / "bank.safetensors")
    msa.save_bank(full, path)
    dev = msa.load_bank(path, DEV)
    host = msa.load_bank(path, DEV, kv_loc="host")
    a = step_case(w, dev)
    b = step_case(w, host)
    torch.cuda.synchronize()
    oracle_check(w, a, "loaded into device memory")
    oracle_check(w, b, "loaded into pinned host memory")
    for x, y, z in zip(ref[:3], a[:3], b[:3]):
        assert torch.equal(x, y) and torch.equal(x, z)
    # a loaded bank with room to grow accepts more documents
    grow = msa.load_bank(path, DEV, chunk_cap=w.C + 8, kv_tokens=w.T + 2048)
    grow.append([1024, 1024])
    assert grow.info().n_docs == w.n_docs + 2
