"""msa_step_static, the entry point for callers that cannot allocate: the
same step as msa_step with the workspace taken from the library's own
per-device scratch.  Checked through the C ABI against msa_step with a
caller workspace (bit for bit: the same kernels on the same inputs) and
against the oracle, on two calls in a row, the second smaller; and a request
beyond the scratch's size is refused before anything runs."""
import ctypes as C

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


def step_args(msa, bank, q, q_pos, k, k_loc, v_loc, L, q_route, outs, hops=1, w_proj=None,
              exclude_selected=False):
    ids, scores, out = outs
    return msa.StepArgs(msa.MSA_DECODE, int(q.shape[0]), int(q.shape[1]), k, q.data_ptr(),
                        int(q_pos), q_route.data_ptr(), None, 64, k_loc.data_ptr(),
                        v_loc.data_ptr(), int(L), hops, None if w_proj is None else w_proj.data_ptr(),
                        int(exclude_selected), None, ids.data_ptr(), scores.data_ptr(),
                        out.data_ptr(), None, 0, None, 0, 0, msa.MSA_MEMORY_TOKENS)


def outputs(n_groups, k, n_q, h_q, hops=1):
    return (torch.full((hops, n_groups, k), -7, dtype=torch.int32, device=DEV),
            torch.full((hops, n_groups, k), 7.0, dtype=torch.float32, device=DEV),
            torch.full((hops, n_q, h_q, 128), 7.0, dtype=torch.float32, device=DEV))


def test_static_step_equals_step_on_two_calls(msa):
    w = S.workload("decode_small")
    r = S.route_vectors(w, DEV)
    k_raw, v_raw = S.kv_raw(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    kr_o, inv_o = M.pool_oracle(w, r)
    doc_kv = M.memo(lambda n: M.oracle_doc_kv(w, k_raw, v_raw, n))
    q = S.queries(w, DEV)
    qr = S.route_queries(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    stream = torch.cuda.current_stream().cuda_stream
    # call 1: the whole batch, k = 4; call 2: two queries, k = 3 (smaller)
    for n_q, k in ((w.B, w.k), (2, 3)):
        ref = bank.step(q[:n_q].contiguous(), w.q_pos, k, k_loc[:n_q].contiguous(),
                        v_loc[:n_q].contiguous(), L, q_route=qr[:n_q].contiguous())
        outs = outputs(n_q, k, n_q, w.h_q)
        qq, qrr = q[:n_q].contiguous(), qr[:n_q].contiguous()
        kl, vl = k_loc[:n_q].contiguous(), v_loc[:n_q].contiguous()
        a = step_args(msa, bank, qq, w.q_pos, k, kl, vl, L, qrr, outs)
        st = msa.lib.msa_step_static(bank.handle, C.byref(a), C.c_void_p(stream))
        assert st == msa.MSA_OK, msa.lib.msa_last_error()
        torch.cuda.synchronize()
        for x, y in zip(ref[:3], outs):
            assert torch.equal(x, y), f"n_q={n_q} k={k}"
        wk = S.Workload(w.name, w.dtype, w.doc_len, h_r=w.h_r, h_kv=w.h_kv, h_q=w.h_q, k=k, B=n_q,
                        L_loc=w.L_loc, seed=w.seed)
        M.check_decode_step(wk, outs[0][0].cpu(), outs[1][0].cpu(), outs[2][0].cpu(), qq, qrr,
                            lk[:n_q], lv[:n_q], kr_o, inv_o, doc_kv, f"static n_q={n_q}")


def test_static_step_multi_hop_with_exclusion(msa):
    """The exclusion bitmap lives in the scratch: it must start cleared on
    every call, whatever the previous call left there."""
    w = S.workload("interleave_small")
    r = S.route_vectors(w, DEV)
    k_raw, v_raw = S.kv_raw(w, DEV)
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    bank.build(0, w.n_docs, r, k_raw, v_raw)
    q = S.queries(w, DEV)
    qr = S.route_queries(w, DEV)
    lk, lv = S.local_raw(w, DEV)
    k_loc, v_loc, L = bank.prepare_local(lk, lv, w.P0)
    wp = S.interleave_projection(w, DEV)
    stream = torch.cuda.current_stream().cuda_stream
    ref = bank.step(q, w.q_pos, w.k, k_loc, v_loc, L, q_route=qr, hops=w.hops, w_proj=wp,
                    exclude_selected=True)
    for _ in range(2):
        outs = outputs(w.B, w.k, w.B, w.h_q, w.hops)
        a = step_args(msa, bank, q, w.q_pos, w.k, k_loc, v_loc, L, qr, outs, w.hops, wp, True)
        assert msa.lib.msa_step_static(bank.handle, C.byref(a), C.c_void_p(stream)) == msa.MSA_OK
        torch.cuda.synchronize()
        for x, y in zip(ref[:3], outs):
            assert torch.equal(x, y)


def test_static_step_refuses_oversized_requests_and_host_banks(msa):
    w = S.workload("decode_small")
    bank = msa.Bank(w.doc_len, w.h_r, w.h_kv, w.dtype, DEV, rope_base=w.rope_base)
    # 4096 queries with 256 splits: the attention partials alone are about
    # 17 GB, far beyond the scratch; refused before any launch (the buffers
    # are real and of the declared sizes all the same)
    n_q, k = 4096, 4
    q = torch.zeros((n_q, w.h_q, 128), dtype=torch.bfloat16, device=DEV)
    qr = torch.zeros((n_q, w.h_r, 128), dtype=torch.float32, device=DEV)
    outs = outputs(n_q, k, n_q, w.h_q)
    a = step_args(msa, bank, q, 0, k, q, q, 0, qr, outs)
    a.k_loc = None
    a.v_loc = None
    a.splits = 256
    stream = torch.cuda.current_stream().cuda_stream
    st = msa.lib.msa_step_static(bank.handle, C.byref(a), C.c_void_p(stream))
    assert st == msa.MSA_ENOMEM
    assert b"scratch" in msa.lib.msa_last_error()
    torch.cuda.synchronize()
    assert int((outs[0] != -7).sum()) == 0  # nothing was written
    hw = S.workload("host_small")
    slot_len, kv_off = S.host_slot_layout(hw)
    host = msa.Bank(hw.doc_len, hw.h_r, hw.h_kv, hw.dtype, DEV, kv_loc="host", kv_off=kv_off,
                    kv_tokens=int(sum(slot_len)), rope_base=hw.rope_base)
    assert msa.lib.msa_step_static(host.handle, C.byref(a), C.c_void_p(stream)) == \
        msa.MSA_EUNSUPPORTED
