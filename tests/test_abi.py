"""The C ABI library loads and exports every symbol include/msa.h declares;
host-side argument validation rejects bad requests before touching HIP.
No compute call runs here (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def msa():
    from long_context_memory_amd import msa as m
    return m


def test_header_declares_the_boundary():
    f = header_functions()
    for name in ("msa_build_bank", "msa_route", "msa_attend", "msa_step"):
        assert name in f


def test_library_exports_every_declared_symbol(msa):
    for name in header_functions():
        assert hasattr(msa.lib, name), name
    assert sorted(msa.EXPORTS) == header_functions()


def test_status_strings(msa):
    for s in range(5):
        assert msa.lib.msa_status_string(s)
    assert msa.lib.msa_version() >= 10000


def _desc(msa, **kw):
    n = kw.pop("n_docs", 2)
    dl = (C.c_int64 * n)(*kw.pop("doc_len", [256] * n))
    d = msa.BankDesc(kw.pop("dtype", msa.MSA_BF16), n, dl, None, kw.pop("kv_tokens", 512),
                     kw.pop("h_r", 8), kw.pop("d_r", 128), kw.pop("h_kv", 8), kw.pop("d", 128),
                     kw.pop("rope_base", 10000.0), kw.pop("kv_loc", msa.MSA_KV_DEVICE),
                     kw.pop("kr", 16), kw.pop("inv_norm", 16), kw.pop("k_store", 16),
                     kw.pop("v_store", 16))
    return d, dl


@pytest.mark.parametrize("bad,code", [
    (dict(doc_len=[300, 256]), 1),
    (dict(doc_len=[0, 256]), 1),
    (dict(n_docs=0, doc_len=[]), 1),
    (dict(dtype=7), 1),
    (dict(d=64), 4),
    (dict(d_r=96), 4),
    (dict(h_r=3), 4),
    (dict(h_kv=0), 4),
    (dict(rope_base=0.5), 1),
    (dict(kr=None), 1),
    (dict(k_store=None), 1),
    (dict(kv_tokens=100), 1),
    (dict(kv_loc=5), 1),
    (dict(kr=24), 1),  # arrays must start on a 16-byte boundary
    (dict(inv_norm=20), 1),
    (dict(k_store=8), 1),
    (dict(v_store=40), 1),
])
def test_bank_create_rejects_bad_descriptors(msa, bad, code):
    d, _keep = _desc(msa, **bad)
    h = C.c_void_p()
    st = msa.lib.msa_bank_create(C.byref(d), C.byref(h))
    assert st == code, msa.lib.msa_last_error()
    assert not h.value
    assert msa.lib.msa_last_error()


def test_null_arguments(msa):
    h = C.c_void_p()
    assert msa.lib.msa_bank_create(None, C.byref(h)) == msa.MSA_EINVAL
    assert msa.lib.msa_bank_destroy(None) == msa.MSA_OK
    assert msa.lib.msa_route(None, None, 1, 1, None, None, None, None, 0, None) == msa.MSA_EINVAL
    assert msa.lib.msa_attend(None, None, None) == msa.MSA_EINVAL
    assert msa.lib.msa_step(None, None, None, None, None) == msa.MSA_EINVAL
    assert msa.lib.msa_workspace_bytes(None, 0, 1, 32, 16, 64, 1, 0) == 0
    assert msa.lib.msa_build_bank(None, 0, 1, None, None, None, None) == msa.MSA_EINVAL
    ms, n = C.c_double(), C.c_int64()
    assert msa.lib.msa_timer_read(2, C.byref(ms), C.byref(n)) == msa.MSA_EINVAL
    assert msa.lib.msa_timer_read(0, None, None) == msa.MSA_EINVAL
    assert msa.lib.msa_timer_reserve(-1) == msa.MSA_EINVAL
    assert msa.lib.msa_timer_reserve(0) == msa.MSA_OK  # nothing to create: no device needed
    with pytest.raises(ValueError):
        msa.timer_enable(True, 0)
    assert msa.lib.msa_timer_enable(0) == msa.MSA_OK  # disabling needs no device
    # the read-rate probe validates before any launch (these pointers are never read)
    out = C.c_void_p(4096)
    assert msa.lib.msa_stream_read(None, 1 << 20, out, None) == msa.MSA_EINVAL
    assert msa.lib.msa_stream_read(C.c_void_p(4096), 1 << 20, None, None) == msa.MSA_EINVAL
    assert msa.lib.msa_stream_read(C.c_void_p(4096), 1000, out, None) == msa.MSA_EINVAL
    assert msa.lib.msa_stream_read(C.c_void_p(4096), 0, out, None) == msa.MSA_EINVAL
    assert msa.lib.msa_stream_read(C.c_void_p(4104), 1 << 20, out, None) == msa.MSA_EINVAL


def test_build_script_flags():
    from long_context_memory_amd import build
    assert "--offload-arch=gfx950" in build.FLAGS
    joined = " ".join(build.FLAGS)
    assert "-packed-fp32-ops" in joined
