"""Arrays shorter than their stated shapes are refused at the C ABI, before
any kernel runs: the library checks each array's extent against the
allocation that holds it.  The binding checks tensors itself, so these
tests call the C entry points directly, with buffers from hipMalloc of an
exact size (the short ones a multiple of 2 MiB, so no rounding of the
allocation hides the shortfall)."""
import ctypes as C

import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"
MIB = 1 << 20


@pytest.fixture(scope="module")
def msa():
    from long_context_memory_amd import msa as m
    return m


@pytest.fixture(scope="module")
def hip():
    torch.zeros(1, device=DEV)  # the runtime is up on this device
    lib = C.CDLL("libamdhip64.so")
    lib.hipMalloc.argtypes = [C.POINTER(C.c_void_p), C.c_size_t]
    lib.hipFree.argtypes = [C.c_void_p]
    bufs = []

    def alloc(nbytes):
        p = C.c_void_p()
        assert lib.hipMalloc(C.byref(p), nbytes) == 0
        bufs.append(p)
        return p.value

    yield alloc
    torch.cuda.synchronize()
    for p in bufs:
        lib.hipFree(p)


def desc(msa, doc_len, kr, inv, ks, vs, h_r=8, h_kv=8):
    dl = (C.c_int64 * len(doc_len))(*doc_len)
    d = msa.BankDesc(msa.MSA_BF16, len(doc_len), dl, None, sum(doc_len), h_r, 128, h_kv, 128,
                     10000.0, msa.MSA_KV_DEVICE, kr, inv, ks, vs, 0)
    return d, dl


def test_bank_arrays_shorter_than_the_bank_are_refused(msa, hip):
    doc_len = [4096] * 128  # 2048 chunks: kr needs 8 x 2048 x 128 x 2 B = 4 MiB
    kv = 128 * 4096 * 8 * 128 * 2  # 1 GiB
    ks, vs = hip(kv), hip(kv)
    inv = hip(8 * 2048 * 4)
    for kr_bytes, ok in ((2 * MIB, False), (4 * MIB, True)):
        kr = hip(kr_bytes)
        d, _dl = desc(msa, doc_len, kr, inv, ks, vs)
        h = C.c_void_p()
        st = msa.lib.msa_bank_create(C.byref(d), C.byref(h))
        if ok:
            assert st == msa.MSA_OK, msa.lib.msa_last_error()
            msa.lib.msa_bank_destroy(h)
        else:
            assert st == msa.MSA_EINVAL and not h.value
            assert b"kr is shorter" in msa.lib.msa_last_error()
    d, _dl = desc(msa, doc_len, hip(4 * MIB), inv, hip(kv - 2 * MIB), vs)  # K store 2 MiB short
    h = C.c_void_p()
    assert msa.lib.msa_bank_create(C.byref(d), C.byref(h)) == msa.MSA_EINVAL
    assert b"k_store is shorter" in msa.lib.msa_last_error()


def test_build_and_local_inputs_shorter_than_their_shapes_are_refused(msa, hip):
    doc_len = [512] * 8  # 4096 tokens, 1 MiB of routing vectors per 512 tokens
    n_tok = sum(doc_len)
    kv = n_tok * 8 * 128 * 2  # 8 MiB
    d, _dl = desc(msa, doc_len, hip(8 * 16 * 128 * 2), hip(8 * 16 * 4), hip(kv), hip(kv))
    h = C.c_void_p()
    assert msa.lib.msa_bank_create(C.byref(d), C.byref(h)) == msa.MSA_OK
    try:
        rv_ok, rv_short = hip(8 * MIB), hip(6 * MIB)
        k_raw, v_raw = hip(kv), hip(kv)
        st = msa.lib.msa_build_bank(h, 0, 8, rv_short, k_raw, v_raw, None)
        assert st == msa.MSA_EINVAL and b"route_vec is shorter" in msa.lib.msa_last_error()
        # a shorter document range needs fewer rows: the same buffer fits
        assert msa.lib.msa_build_bank(h, 0, 6, rv_short, k_raw, v_raw, None) == msa.MSA_OK
        assert msa.lib.msa_build_bank(h, 0, 8, rv_ok, k_raw, v_raw, None) == msa.MSA_OK
        # local context: 1 sequence of 4000 tokens, V tiles padded to 4032
        L = 4000
        k_bytes, v_bytes = L * 8 * 128 * 2, 4032 * 8 * 128 * 2
        lk, lv, k_loc = hip(k_bytes), hip(k_bytes), hip(k_bytes)
        st = msa.lib.msa_prepare_local(h, lk, lv, 1, L, 4096, k_loc, hip(6 * MIB), None)
        assert st == msa.MSA_EINVAL and b"v_loc is shorter" in msa.lib.msa_last_error()
        st = msa.lib.msa_prepare_local(h, hip(6 * MIB), lv, 1, L, 4096, k_loc, hip(v_bytes), None)
        assert st == msa.MSA_EINVAL and b"k_raw is shorter" in msa.lib.msa_last_error()
        assert msa.lib.msa_prepare_local(h, lk, lv, 1, L, 4096, k_loc, hip(v_bytes),
                                         None) == msa.MSA_OK
        torch.cuda.synchronize()
    finally:
        msa.lib.msa_bank_destroy(h)
    x = torch.ones(4, device=DEV)  # no error left behind for the next call
    assert float((x + 1).sum()) == 8.0
