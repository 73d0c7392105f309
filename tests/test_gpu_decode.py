"""GPU parity of the decode path (bank build, routing, top-k, gather, split-K
decode attention) against the fp64 oracle, through the C ABI."""
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


_CACHE = {}


def decode_case(msa, name):
    """Bank, inputs and oracle keys of a named workload (or a Workload)."""
    w = S.workload(name) if isinstance(name, str) else name
    name = w.name
    if name in _CACHE:
        return _CACHE[name]
    r = S.route_vectors(w, DEV)
    k_raw, v_raw = S.kv_raw(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    kr_o, inv_o = M.pool_oracle(w, r)
    if w.plant == "pooled_key":
        doc, ch = S.pooled_key_target(w)
        q_route = S.pooled_key_query(w, kr_o[ch], DEV)
    else:
        doc = None
        q_route = S.route_queries(w, DEV)
    q = S.queries(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    torch.cuda.synchronize()
    c = dict(w=w, r=r, k_raw=k_raw, v_raw=v_raw, bank=bank, kr_o=kr_o, inv_o=inv_o,
             q_route=q_route, q=q, lk=lk, lv=lv, k_loc=k_loc, v_loc=v_loc, L=L,
             target_doc=doc)
    _CACHE[name] = c
    return c


SMALL = ["tiny_f32_small", "decode_small", "tiny_f32_64k"]


@pytest.mark.parametrize("name", SMALL + ["decode_1m"])
def test_bank_build_matches_oracle(msa, name):
    c = decode_case(msa, name)
    w, bank = c["w"], c["bank"]
    kr = M.np64(bank.kr.permute(1, 0, 2))
    np.testing.assert_array_equal(kr, c["kr_o"])  # float64 mean, one rounding: bit-exact
    inv = M.np64(bank.inv_norm.t())
    np.testing.assert_allclose(inv, c["inv_o"], rtol=2e-7, atol=0)
    for n in M.seeded_subset(w.n_docs, 6, 7):
        k_o, v_o = M.oracle_doc_kv(w, c["k_raw"], c["v_raw"], n)
        kg = M.natural_from_store_k(bank, n)
        vg = M.natural_from_store_v(bank, n)
        np.testing.assert_array_equal(M.np64(vg), v_o)
        kt = torch.from_numpy(k_o).to(kg.dtype)
        if w.dtype == "bf16":
            ud = M.ulp_diff_bf16(kg.cpu(), kt)
            assert int(ud.max()) <= 1 and float((ud > 0).float().mean()) < 1e-3
        else:
            np.testing.assert_allclose(M.np64(kg), k_o, rtol=2.5e-7, atol=1e-30)


@pytest.mark.parametrize("name", ["tiny_f32_small", "decode_small"])
def test_prepare_local_matches_oracle(msa, name):
    c = decode_case(msa, name)
    w = c["w"]
    L = c["L"]
    for b in range(w.B):
        lk_o = O.round_to_storage(O.rope_rotate(M.np64(c["lk"][b]), (w.P0 + np.arange(L))[:, None],
                                                w.rope_base), w.dtype)
        # local K takes the bank K's bar: one rounding of a float64 rotation
        kg = c["k_loc"][b].permute(1, 0, 2)
        if w.dtype == "bf16":
            ud = M.ulp_diff_bf16(kg.cpu(), torch.from_numpy(lk_o).to(kg.dtype))
            assert int(ud.max()) <= 1 and float((ud > 0).float().mean()) < 1e-3
        else:
            np.testing.assert_allclose(M.np64(kg), lk_o, rtol=2.5e-7, atol=1e-30)
        vg = M.local_v_natural(c["v_loc"][b])  # [Tp*64, h_kv, 128]
        np.testing.assert_array_equal(M.np64(vg[:L]), M.np64(c["lv"][b]))
        assert float(vg[L:].abs().max()) == 0.0 if vg.shape[0] > L else True


def oracle_scores(c, exclude=None):
    w = c["w"]
    return O.cosine_doc_scores(M.np64(c["q_route"]), c["kr_o"], c["inv_o"], w.doc_len, exclude)


@pytest.mark.parametrize("name", SMALL + ["decode_1m"])
def test_route_matches_oracle(msa, name):
    c = decode_case(msa, name)
    w = c["w"]
    ids, scores = c["bank"].route(c["q_route"], w.k)
    torch.cuda.synchronize()
    so = oracle_scores(c)
    M.check_topk(ids.cpu().numpy(), scores.cpu().numpy(), so, w.k)
    if w.plant == "direction":
        tgt, _ = S.planted_targets(w)
        for b in range(w.B):
            assert set(ids[b].tolist()) == set(tgt[b].tolist())
    if w.plant == "pooled_key":
        assert all(int(ids[b, 0]) == c["target_doc"] for b in range(w.B))


@pytest.mark.parametrize("B", [1, 7, 32, 40, 64, 70])
def test_route_large_batches_match_oracle(msa, B):
    # bf16 keys take the matrix-core scan at every batch size (a pass holds up
    # to 64 queries: 70 is a pass of 64 and a pass of 6; 1 and 7 leave most of
    # each 32-query block empty); the bank's last tile is ragged
    c = decode_case(msa, "decode_small")
    w = c["w"]
    g = torch.Generator(device=DEV)
    g.manual_seed(7000 + B)
    qr = torch.randn((B, w.h_r, 128), generator=g, device=DEV)
    ids, scores = c["bank"].route(qr, w.k)
    torch.cuda.synchronize()
    so = O.cosine_doc_scores(M.np64(qr), c["kr_o"], c["inv_o"], w.doc_len)
    M.check_topk(ids.cpu().numpy(), scores.cpu().numpy(), so, w.k)


def test_zero_query_batches(msa):
    # empty batches are valid calls that launch nothing
    c = decode_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    ids, scores = bank.route(torch.empty((0, w.h_r, 128), device=DEV), w.k)
    assert ids.shape == (0, w.k) and scores.shape == (0, w.k)
    q0 = c["q"][:0]
    out = bank.attend(q0, w.q_pos, ids, c["k_loc"][:0], c["v_loc"][:0], c["L"])
    assert out.shape == (0, w.h_q, 128)
    ids, scores, out, st = bank.step(q0, w.q_pos, w.k, c["k_loc"][:0], c["v_loc"][:0], c["L"],
                                     q_route=c["q_route"][:0])
    torch.cuda.synchronize()
    assert out.shape[1] == 0 and st.docs_copied == 0


def test_timer_brackets_every_period_th_launch(msa):
    c = decode_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    ids, _ = bank.route(c["q_route"], w.k)
    torch.cuda.synchronize()
    msa.timer_reserve(8)
    msa.timer_enable(True, 3)
    for _ in range(7):  # launches 0, 3 and 6 are bracketed
        bank.attend(c["q"], w.q_pos, ids, c["k_loc"], c["v_loc"], c["L"])
    ms, n = msa.timer_read(msa.MSA_TIMER_ATTENTION)
    msa.timer_enable(False)
    assert n == 3 and ms > 0.0
    bank.attend(c["q"], w.q_pos, ids, c["k_loc"], c["v_loc"], c["L"])  # disabled: not timed
    ms, n = msa.timer_read(msa.MSA_TIMER_ATTENTION)
    assert n == 0 and ms == 0.0


def test_misaligned_arrays_are_rejected(msa):
    # a contiguous view that starts 2 bytes into its storage: refused before
    # any launch, and the output is left as it was
    c = decode_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    flat = torch.empty(c["q"].numel() + 8, dtype=c["q"].dtype, device=DEV)
    q_bad = flat[1:1 + c["q"].numel()].view(c["q"].shape)
    q_bad.copy_(c["q"])
    ids, _ = bank.route(c["q_route"], w.k)
    out = torch.full((w.B, w.h_q, 128), 3.0, device=DEV)
    with pytest.raises(msa.MSAError) as e:
        bank.attend(q_bad, w.q_pos, ids, c["k_loc"], c["v_loc"], c["L"], out=out)
    assert e.value.status == msa.MSA_EINVAL
    assert "aligned" in msa.lib.msa_last_error().decode()
    with pytest.raises(msa.MSAError):
        bank.step(q_bad, w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"], q_route=c["q_route"])
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


@pytest.mark.parametrize("B", [5, 70])
def test_route_float32_keys_match_oracle(msa, B):
    # float32 keys take the vector scan (70: a pass of 64 and a pass of 6)
    c = decode_case(msa, "tiny_f32_small")
    w = c["w"]
    g = torch.Generator(device=DEV)
    g.manual_seed(7100 + B)
    qr = torch.randn((B, w.h_r, 128), generator=g, device=DEV)
    ids, scores = c["bank"].route(qr, w.k)
    torch.cuda.synchronize()
    so = O.cosine_doc_scores(M.np64(qr), c["kr_o"], c["inv_o"], w.doc_len)
    M.check_topk(ids.cpu().numpy(), scores.cpu().numpy(), so, w.k)


@pytest.mark.parametrize("h_r", [1, 16])
def test_route_router_head_counts(msa, h_r):
    # one and sixteen router heads (the pooling kernel's and the scan's
    # extremes) on a bf16 bank of the small decode shape
    w = dataclasses.replace(S.workload("decode_small"), h_r=h_r, name=f"decode_small_hr{h_r}")
    r = S.route_vectors(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    k_raw, v_raw = S.kv_raw(w, DEV)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    kr_o, inv_o = M.pool_oracle(w, r)
    np.testing.assert_array_equal(M.np64(bank.kr.permute(1, 0, 2)), kr_o)
    g = torch.Generator(device=DEV)
    g.manual_seed(7200 + h_r)
    qr = torch.randn((9, h_r, 128), generator=g, device=DEV)
    ids, scores = bank.route(qr, w.k)
    torch.cuda.synchronize()
    so = O.cosine_doc_scores(M.np64(qr), kr_o, inv_o, w.doc_len)
    M.check_topk(ids.cpu().numpy(), scores.cpu().numpy(), so, w.k)


@pytest.mark.parametrize("name", ["decode_small"])
def test_route_exclusion_and_k_equals_n(msa, name):
    c = decode_case(msa, name)
    w = c["w"]
    N = w.n_docs
    rng = np.random.default_rng(5)
    excl = rng.random((w.B, N)) < 0.3
    words = np.zeros((w.B, (N + 31) // 32), dtype=np.uint32)
    for b in range(w.B):
        for n in np.nonzero(excl[b])[0]:
            words[b, n // 32] |= np.uint32(1 << (n % 32))
    ex = torch.from_numpy(words.view(np.int32)).to(DEV)
    kk = min(w.k, int((~excl).sum(axis=1).min()))
    ids, scores = c["bank"].route(c["q_route"], kk, exclude=ex)
    so = oracle_scores(c, excl)
    M.check_topk(ids.cpu().numpy(), scores.cpu().numpy(), so, kk)
    # more requested than remain: the tail is -1 / -inf
    ids, scores = c["bank"].route(c["q_route"], N, exclude=ex)
    for b in range(w.B):
        nv = int((~excl[b]).sum())
        assert (ids[b, nv:] == -1).all() and torch.isinf(scores[b, nv:]).all()
        assert set(ids[b, :nv].tolist()) == set(np.nonzero(~excl[b])[0].tolist())
    # k = N without exclusion: every document, in score order
    ids, scores = c["bank"].route(c["q_route"], N)
    so = oracle_scores(c)
    M.check_topk(ids.cpu().numpy(), scores.cpu().numpy(), so, N)
    # a query with every document excluded selects nothing; the others are
    # unaffected
    words_all = np.zeros_like(words)
    words_all[0, :] = np.uint32(0xFFFFFFFF)
    ex_all = torch.from_numpy(words_all.view(np.int32)).to(DEV)
    ids0, sc0 = c["bank"].route(c["q_route"], w.k)
    ids, scores = c["bank"].route(c["q_route"], w.k, exclude=ex_all)
    assert (ids[0] == -1).all() and torch.isinf(scores[0]).all() and (scores[0] < 0).all()
    assert torch.equal(ids[1:], ids0[1:]) and torch.equal(scores[1:], sc0[1:])


def oracle_decode(c, ids_gpu, so):
    """Oracle outputs for every query; the oracle's own top-k unless the GPU
    chose a valid alternative inside a near-tie."""
    w = c["w"]
    o_ids, _ = O.select_topk(so, w.k)
    q = M.np64(c["q"])
    lk, lv = M.np64(c["lk"]), M.np64(c["lv"])
    outs = []
    cache = {}
    for b in range(w.B):
        sel = o_ids[b] if set(o_ids[b].tolist()) == set(ids_gpu[b].tolist()) else ids_gpu[b]
        for n in sel:
            if n not in cache:
                cache[n] = M.oracle_doc_kv(w, c["k_raw"], c["v_raw"], n)
        outs.append(M.oracle_attend_decode(w, q[b], w.q_pos, sel, cache, lk[b], lv[b], w.P0))
    return np.stack(outs)


@pytest.mark.parametrize("name", SMALL + ["decode_1m"])
def test_decode_step_matches_oracle(msa, name):
    c = decode_case(msa, name)
    w = c["w"]
    ids, scores, out, _ = c["bank"].step(c["q"], w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"],
                                         q_route=c["q_route"])
    torch.cuda.synchronize()
    so = oracle_scores(c)
    ids_np = ids[0].cpu().numpy()
    M.check_topk(ids_np, scores[0].cpu().numpy(), so, w.k)
    ref = oracle_decode(c, ids_np, so)
    mx, rel = M.check_out(out[0].cpu().numpy(), ref, w.dtype, name)
    print(f"{name}: max abs {mx:.3e} rel rms {rel:.3e}")


@pytest.mark.parametrize("form", ["torch", "int", "ctypes"])
def test_binding_calls_on_a_side_stream(msa, form):
    """The binding's route and step on a stream other than the current one,
    given as a torch stream, an int handle or a ctypes pointer, with the
    workspace and outputs the binding allocates itself (it records the
    stream on them, so their memory is not handed out again while the
    stream still uses it): the same bits as on the current stream."""
    import ctypes
    c = decode_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    ref_ids, ref_sc = bank.route(c["q_route"], w.k)
    ref = bank.step(c["q"], w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"], q_route=c["q_route"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    s = {"torch": side, "int": side.cuda_stream,
         "ctypes": ctypes.c_void_p(side.cuda_stream)}[form]
    for _ in range(3):  # dropped temporaries reallocated while the stream runs
        ids, sc = bank.route(c["q_route"], w.k, stream=s)
        got = bank.step(c["q"], w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"],
                        q_route=c["q_route"], stream=s)
        scratch = torch.full((1 << 20,), 7.0, device=DEV)  # on the current stream
        del scratch
        side.synchronize()
        assert torch.equal(ids, ref_ids) and torch.equal(sc, ref_sc)
        for a, b in zip(got[:3], ref[:3]):
            assert torch.equal(a, b)


def test_attend_over_a_caller_source(msa):
    """msa_attend with a source override: the selected documents' K and V
    blocks copied out of the bank's stores into compact caller-owned arrays
    (the layout a host-resident bank's staging has), in an order of their
    own, and the ids remapped to that table: bit-identical to attention
    over the bank itself."""
    c = decode_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    ids, _ = bank.route(c["q_route"], w.k)
    ref = bank.attend(c["q"], w.q_pos, ids, c["k_loc"], c["v_loc"], c["L"])
    ids_np = ids.cpu().numpy()
    docs = sorted(set(ids_np.ravel().tolist()) - {-1}, reverse=True)
    tok = S.doc_token_offsets(w)
    per_tok = w.h_kv * 128
    total = sum(int(w.doc_len[n]) for n in docs)
    sk = torch.empty(total * per_tok, dtype=w.torch_dtype, device=DEV)
    sv = torch.empty_like(sk)
    off, t = [], 0
    for n in docs:
        a, m = int(tok[n]) * per_tok, int(w.doc_len[n]) * per_tok
        sk[t * per_tok:t * per_tok + m] = bank.k_store[a:a + m]
        sv[t * per_tok:t * per_tok + m] = bank.v_store[a:a + m]
        off.append(t)
        t += int(w.doc_len[n])
    so = torch.tensor(off, dtype=torch.int64, device=DEV)
    sl = torch.tensor([int(w.doc_len[n]) for n in docs], dtype=torch.int32, device=DEV)
    slot = {n: i for i, n in enumerate(docs)}
    ids_c = torch.tensor([[slot.get(int(x), -1) for x in row] for row in ids_np],
                         dtype=torch.int32, device=DEV)
    out = bank.attend(c["q"], w.q_pos, ids_c, c["k_loc"], c["v_loc"], c["L"], src=(sk, sv, so, sl))
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("name", ["tiny_f32_small", "decode_small"])
@pytest.mark.parametrize("cached", [False, True])
def test_host_resident_copy_of_the_bank(msa, tmp_path, name, cached):
    """A decode step on a host-resident copy of the bank (saved, then loaded
    into pinned host memory), float32 and bf16 stores: the selected
    documents are copied (into staging, or into a device cache) and the
    results are bit-identical to the device bank's."""
    c = decode_case(msa, name)
    w = c["w"]
    path = str(tmp_path / f"{name}.safetensors")
    msa.save_bank(c["bank"], path)
    host = msa.load_bank(path, DEV, kv_loc="host")
    if cached:
        host.set_cache(torch.empty((w.B * w.k + 1) * host.cache_slot_bytes(), dtype=torch.uint8,
                                   device=DEV))
    args = (c["q"], w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"])
    try:
        ref = c["bank"].step(*args, q_route=c["q_route"])
        got = host.step(*args, q_route=c["q_route"])
        torch.cuda.synchronize()
        for name_, a, b in zip(("ids", "scores", "out"), got[:3], ref[:3]):
            assert torch.equal(a, b), name_
        distinct = len(set(ref[0].cpu().numpy().ravel().tolist()) - {-1})
        assert got[3].docs_copied == distinct
    finally:
        if cached:
            host.set_cache(None)


@pytest.mark.parametrize("h_q,k,n_docs", [(8, 4, 48), (16, 4, 48), (64, 4, 48), (32, 64, 72)])
def test_decode_gqa_groups_and_max_k(msa, h_q, k, n_docs):
    # one, two and eight query heads per KV head, and the largest k (64
    # selected documents, 32K document tokens per query), on the small bf16
    # decode shape with unplanted router queries
    base = S.workload("decode_small")
    w = dataclasses.replace(base, h_q=h_q, k=k, doc_len=[512] * n_docs, plant=None,
                            name=f"decode_small_hq{h_q}_k{k}")
    c = decode_case(msa, w)
    ids, scores, out, _ = c["bank"].step(c["q"], w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"],
                                         q_route=c["q_route"])
    torch.cuda.synchronize()
    so = oracle_scores(c)
    ids_np = ids[0].cpu().numpy()
    M.check_topk(ids_np, scores[0].cpu().numpy(), so, w.k)
    ref = oracle_decode(c, ids_np, so)
    mx, rel = M.check_out(out[0].cpu().numpy(), ref, w.dtype, w.name)
    print(f"{w.name}: max abs {mx:.3e} rel rms {rel:.3e}")


def test_decode_power_wrong_document_is_caught(msa):
    # the tolerance is tight enough to see one swapped document
    c = decode_case(msa, "decode_small")
    w = c["w"]
    ids, scores, out, _ = c["bank"].step(c["q"], w.q_pos, w.k, c["k_loc"], c["v_loc"], c["L"],
                                         q_route=c["q_route"])
    ids_np = ids[0].cpu().numpy().copy()
    so = oracle_scores(c)
    bad = ids_np.copy()
    bad[0, -1] = [n for n in range(w.n_docs) if n not in bad[0]][0]
    ref_bad = oracle_decode(c, bad, so)  # union with one document replaced
    with pytest.raises(AssertionError):
        M.check_out(out[0].cpu().numpy(), ref_bad, w.dtype, "power")


def test_decode_skips_empty_id_slots(msa):
    # -1 (an empty top-k slot) and ids outside [0, n_docs) select nothing:
    # the output is the oracle's over the remaining documents
    c = decode_case(msa, "decode_small")
    w = c["w"]
    ids, _ = c["bank"].route(c["q_route"], w.k)
    ids = ids.clone()
    ids[0::2, -1] = -1
    ids[1, 0] = w.n_docs + 5
    ids[2, :] = -1  # local context only
    out = c["bank"].attend(c["q"], w.q_pos, ids, c["k_loc"], c["v_loc"], c["L"])
    torch.cuda.synchronize()
    q, lk, lv = M.np64(c["q"]), M.np64(c["lk"]), M.np64(c["lv"])
    ids_np = ids.cpu().numpy()
    cache = {}
    for b in range(w.B):
        sel = [int(n) for n in ids_np[b] if 0 <= n < w.n_docs]
        for n in sel:
            if n not in cache:
                cache[n] = M.oracle_doc_kv(w, c["k_raw"], c["v_raw"], n)
        ref = M.oracle_attend_decode(w, q[b], w.q_pos, sel, cache, lk[b], lv[b], w.P0)
        M.check_out(out[b].cpu().numpy(), ref, w.dtype, f"query {b}")


@pytest.mark.parametrize("name", ["tiny_f32_small", "decode_small"])
def test_decode_splits_and_determinism(msa, name):
    c = decode_case(msa, name)
    w = c["w"]
    ids, _ = c["bank"].route(c["q_route"], w.k)
    # 256 (the maximum) exceeds the tiles of every union: empty splits merge as nothing
    outs = [c["bank"].attend(c["q"], w.q_pos, ids, c["k_loc"], c["v_loc"], c["L"], splits=s)
            for s in (4, 8, 64, 256)]
    again = c["bank"].attend(c["q"], w.q_pos, ids, c["k_loc"], c["v_loc"], c["L"], splits=8)
    torch.cuda.synchronize()
    assert torch.equal(outs[1], again)  # deterministic
    # different splits see different running maxima; fp32 agrees to rounding,
    # bf16 to the bf16 rounding of the probabilities (2^-8 relative)
    scale = float(outs[0].abs().max())
    tol = 2e-6 if w.dtype == "f32" else 2.0 ** -8
    for o in outs[1:]:
        assert float((o - outs[0]).abs().max()) <= tol * scale


def test_decode_workspace_reuse(msa):
    # the split merge counters live in the workspace: a poisoned workspace and
    # one reused call after call give the same bits as a fresh one
    c = decode_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    ids, _ = bank.route(c["q_route"], w.k)
    ref = bank.attend(c["q"], w.q_pos, ids, c["k_loc"], c["v_loc"], c["L"])
    ws = bank.workspace(msa.MSA_DECODE, w.B, w.h_q, w.k)
    ws.fill_(255)
    outs = [bank.attend(c["q"], w.q_pos, ids, c["k_loc"], c["v_loc"], c["L"], ws=ws)
            for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


@pytest.mark.parametrize("L_loc", [0, 1, 63, 64, 65, 130])
def test_decode_ragged_and_empty_local(msa, L_loc):
    c = decode_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    lk, lv = c["lk"][:, :L_loc].contiguous(), c["lv"][:, :L_loc].contiguous()
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    ids, _ = bank.route(c["q_route"], w.k)
    out = bank.attend(c["q"], w.P0 + max(L_loc, 1) - 1, ids, k_loc, v_loc, L)
    torch.cuda.synchronize()
    so = oracle_scores(c)
    ids_np = ids.cpu().numpy()
    q = M.np64(c["q"])
    cache = {}
    for b in range(w.B):
        for n in ids_np[b]:
            cache.setdefault(n, M.oracle_doc_kv(w, c["k_raw"], c["v_raw"], n))
        ref = M.oracle_attend_decode(w, q[b], w.P0 + max(L_loc, 1) - 1, ids_np[b], cache,
                                     M.np64(lk[b]), M.np64(lv[b]), w.P0)
        M.check_out(out[b].cpu().numpy(), ref, w.dtype, f"L_loc={L_loc}")
    del so


def test_decode_local_only_and_docs_only(msa):
    c = decode_case(msa, "decode_small")
    w, bank = c["w"], c["bank"]
    q = M.np64(c["q"])
    # k = 0: attention over the local context alone
    out = bank.attend(c["q"], w.q_pos, None, c["k_loc"], c["v_loc"], c["L"])
    torch.cuda.synchronize()
    for b in range(w.B):
        ref = M.oracle_attend_decode(w, q[b], w.q_pos, [], {}, M.np64(c["lk"][b]),
                                     M.np64(c["lv"][b]), w.P0)
        M.check_out(out[b].cpu().numpy(), ref, w.dtype, "local only")
    # one document, some ids -1 (skipped)
    ids = torch.full((w.B, 3), -1, dtype=torch.int32, device=DEV)
    ids[:, 1] = torch.arange(w.B, dtype=torch.int32, device=DEV) + 5
    e = torch.empty((w.B, 0, w.h_kv, 128), dtype=c["lk"].dtype, device=DEV)
    k0, v0, L0 = bank.prepare_local(e, e, w.P0)
    out = bank.attend(c["q"], w.q_pos, ids, k0, v0, L0)
    torch.cuda.synchronize()
    for b in range(w.B):
        n = b + 5
        kv = {n: M.oracle_doc_kv(w, c["k_raw"], c["v_raw"], n)}
        ref = M.oracle_attend_decode(w, q[b], w.q_pos, [n], kv, np.zeros((0, w.h_kv, 128)),
                                     np.zeros((0, w.h_kv, 128)), w.P0)
        M.check_out(out[b].cpu().numpy(), ref, w.dtype, "docs only")
    # no key at all (every id empty, no local tokens): the output is 0, with
    # one split and with the most splits
    ids = torch.full((w.B, 3), -1, dtype=torch.int32, device=DEV)
    for splits in (4, 256):
        out = bank.attend(c["q"], w.q_pos, ids, k0, v0, L0, splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out, torch.zeros_like(out)), splits


def test_stream_read_probe_reads_every_word(msa):
    # the HBM read-rate probe's checksum is the XOR of every 32-bit word it
    # read: check it over a single word, a ragged size and several grid strides
    g = torch.Generator().manual_seed(7)
    out = torch.empty(msa.MSA_STREAM_READ_BLOCKS, dtype=torch.int32, device=DEV)
    for n_words in (4, 4 * 12345, 4 * 4096 * 256 * 3 + 36):
        host = torch.randint(-2**31, 2**31 - 1, (n_words,), dtype=torch.int32, generator=g)
        msa.stream_read(host.to(DEV), out)
        got = np.bitwise_xor.reduce(out.cpu().numpy())
        assert got == np.bitwise_xor.reduce(host.numpy()), n_words


# channels of the rotary pairs (i, i + 64) with i >= 40
LOWF = np.zeros(128, dtype=bool)
LOWF[40:64] = LOWF[104:128] = True


def dominant_key_case(w):
    """Queries and raw K where one key of document n_docs - 1 (token 100,
    every KV head) is aligned with query heads 0 and 1 of each group, about
    300 log2 units above any other score of theirs; heads 2 and 3 are zero
    in that key's channels.  Returns (q, k_raw, v_raw, big document, token
    row of the key)."""
    big, pk = w.n_docs - 1, 100
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
    q0n = M.np64(q0)
    k = O.rope_rotate(q0n, w.q_pos - pk, w.rope_base)  # rotated at pk it equals q0 at q_pos
    k *= 300.0 * np.sqrt(w.d) / np.log2(np.e) / float(q0n @ q0n)
    t = int(S.doc_token_offsets(w)[big]) + pk
    k_raw[t] = torch.tensor(k, dtype=k_raw.dtype, device=DEV)
    return q, k_raw, v_raw, big, t


@pytest.mark.parametrize("splits", [1, 0])
def test_decode_late_dominant_key(msa, splits):
    """A key ranked last that outscores everything before it by far more
    than float32 can hold as a ratio (2^300): the online softmax must move
    its reference there, and the earlier probabilities must vanish rather
    than overflow.  Query heads 2 and 3 share the key heads with ordinary
    scores.  One split and the automatic split count (partials merged)."""
    w = S.workload("decode_small")
    q, k_raw, v_raw, big, t_big = dominant_key_case(w)
    r = S.route_vectors(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    sel = [[(5 * b + j) % (w.n_docs - 1) for j in range(w.k - 1)] + [big] for b in range(w.B)]
    ids = torch.tensor(sel, dtype=torch.int32, device=DEV)
    out = bank.attend(q, w.q_pos, ids, k_loc, v_loc, L, splits=splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    qn, lkn, lvn = M.np64(q), M.np64(lk), M.np64(lv)
    doc_kv = {n: M.oracle_doc_kv(w, k_raw, v_raw, n) for n in set(sum(sel, []))}
    spike_heads = [h for h in range(w.h_q) if h % w.G < 2]
    v_big = M.np64(v_raw[t_big])
    # the case is what it says: the key leads every other document score of
    # heads 0 and 1 by more than 128 log2 units (query 0)
    to_log2 = np.log2(np.e) / np.sqrt(w.d)
    qr = O.rope_rotate(qn[0], np.full((w.h_q,), w.q_pos), w.rope_base)
    kb = doc_kv[big][0][t_big - int(S.doc_token_offsets(w)[big])]
    for h in spike_heads:
        g = h // w.G
        s_big = float(qr[h] @ kb[g]) * to_log2
        others = max(float(np.max(doc_kv[n][0][:, g] @ qr[h])) for n in sel[0][:-1]) * to_log2
        assert s_big - others > 128, (h, s_big, others)
    for b in range(w.B):
        ref = M.oracle_attend_decode(w, qn[b], w.q_pos, sel[b], doc_kv, lkn[b], lvn[b], w.P0)
        for h in spike_heads:
            assert np.allclose(ref[h], v_big[h // w.G], atol=1e-12)
        M.check_out(out[b], ref, w.dtype, f"query {b} splits {splits}")
