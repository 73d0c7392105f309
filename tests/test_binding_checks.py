"""The binding refuses tensors whose shape, dtype or layout differ from what
the C call would read or write: the library sees only pointers and sizes, so
a short tensor would be read out of bounds on the device.  Every check runs
before the library is called, so these tests need no GPU."""
import pytest
import torch

from long_context_memory_amd import msa


def fake_bank(h_r=1, h_kv=8, dtype=torch.bfloat16, n_docs=4, doc_len=512):
    b = msa.Bank.__new__(msa.Bank)  # no device tables: only the checks run
    b.h_r, b.h_kv, b.d = h_r, h_kv, 128
    b.dtype = dtype
    b.device = torch.device("cpu")
    b.n_docs = n_docs
    b.doc_len = [doc_len] * n_docs
    b.kv_host = False
    return b


def test_prepare_local_refuses_a_local_context_without_batch_dimension():
    b = fake_bank()
    lk = torch.zeros((250, 8, 128), dtype=torch.bfloat16)  # [L, h_kv, d]: no n_seq
    with pytest.raises(ValueError, match="k_raw"):
        b.prepare_local(lk, lk, 1024)


def test_prepare_local_refuses_wrong_heads_dtype_and_mismatched_v():
    b = fake_bank()
    with pytest.raises(ValueError, match="shape"):
        b.prepare_local(torch.zeros((2, 64, 4, 128), dtype=torch.bfloat16),
                        torch.zeros((2, 64, 4, 128), dtype=torch.bfloat16), 0)
    with pytest.raises(ValueError, match="dtype"):
        b.prepare_local(torch.zeros((2, 64, 8, 128)), torch.zeros((2, 64, 8, 128)), 0)
    with pytest.raises(ValueError, match="v_raw"):
        b.prepare_local(torch.zeros((2, 64, 8, 128), dtype=torch.bfloat16),
                        torch.zeros((2, 32, 8, 128), dtype=torch.bfloat16), 0)


def test_build_refuses_token_counts_that_do_not_match_the_documents():
    b = fake_bank(n_docs=4, doc_len=512)
    short = torch.zeros((1024 - 256, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_raw"):
        b.build(0, 2, None, short, short)
    with pytest.raises(ValueError, match="range"):
        b.build(3, 5)


def test_attend_refuses_local_context_of_another_length_and_non_contiguous_q():
    b = fake_bank()
    q = torch.zeros((2, 32, 128), dtype=torch.bfloat16)
    ids = torch.zeros((2, 4), dtype=torch.int32)
    k_loc = torch.zeros((2, 8, 100, 128), dtype=torch.bfloat16)
    v_loc = torch.zeros((2, 8, 2, 128, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_loc"):
        b.attend(q, 0, ids, k_loc, v_loc, 128)
    qt = torch.zeros((32, 2, 128), dtype=torch.bfloat16).transpose(0, 1)
    with pytest.raises(ValueError, match="contiguous"):
        b.attend(qt, 0, ids, k_loc, v_loc, 100)
    with pytest.raises(ValueError, match="ids"):
        b.attend(q, 0, torch.zeros((3, 4), dtype=torch.int32), k_loc, v_loc, 100)


def test_step_refuses_outputs_and_router_queries_of_the_wrong_shape():
    b = fake_bank(h_r=2)
    q = torch.zeros((2, 32, 128), dtype=torch.bfloat16)
    k_loc = torch.zeros((2, 8, 64, 128), dtype=torch.bfloat16)
    v_loc = torch.zeros((2, 8, 1, 128, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q_route"):
        b.step(q, 0, 4, k_loc, v_loc, 64, q_route=torch.zeros((2, 1, 128)))
    outs = (torch.zeros((1, 2, 3), dtype=torch.int32), torch.zeros((1, 2, 4)),
            torch.zeros((1, 2, 32, 128)))
    with pytest.raises(ValueError, match="ids"):
        b.step(q, 0, 4, k_loc, v_loc, 64, q_route=torch.zeros((2, 2, 128)), outputs=outs,
               ws=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="w_proj"):
        b.step(q, 0, 4, k_loc, v_loc, 64, q_route=torch.zeros((2, 2, 128)), hops=2,
               w_proj=torch.zeros((128, 128)))


def test_route_refuses_exclusion_masks_of_the_wrong_width():
    b = fake_bank(h_r=2, n_docs=100)
    qr = torch.zeros((3, 2, 128))
    with pytest.raises(ValueError, match="exclude"):
        b.route(qr, 4, exclude=torch.zeros((3, 3), dtype=torch.int32))


def test_buffers_of_too_few_bytes_are_refused():
    with pytest.raises(ValueError, match="need"):
        msa._expect_bytes(torch.zeros(10, dtype=torch.uint8), 11, "ws")
    msa._expect_bytes(torch.zeros(3, dtype=torch.float32), 12, "ws")


def test_bank_refuses_caller_arrays_of_the_wrong_extent_type_or_place():
    # every check runs before the library is called (CPU tensors never reach it)
    kw = dict(h_r=2, h_kv=8, dtype="bf16", device="cpu")
    docs = [512] * 4  # 8 chunks, 2048 tokens
    with pytest.raises(ValueError, match="kr"):
        msa.Bank(docs, kr=torch.zeros((2, 7, 128), dtype=torch.bfloat16), **kw)
    with pytest.raises(ValueError, match="kr"):
        msa.Bank(docs, kr=torch.zeros((2, 8, 128)), **kw)  # float32 keys for a bf16 bank
    with pytest.raises(ValueError, match="inv_norm"):
        msa.Bank(docs, inv_norm=torch.zeros((2, 8), dtype=torch.float64), **kw)
    with pytest.raises(ValueError, match="inv_norm"):
        msa.Bank(docs, chunk_cap=16, inv_norm=torch.zeros((2, 8)), **kw)  # capacity rows
    short = torch.zeros(2048 * 8 * 128 - 1, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_store"):
        msa.Bank(docs, k_store=short, v_store=short, **kw)
    full = torch.zeros(2048 * 8 * 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="together"):
        msa.Bank(docs, k_store=full, **kw)
    with pytest.raises(ValueError, match="v_store"):
        msa.Bank(docs, k_store=full, v_store=full.float(), **kw)
    with pytest.raises(ValueError, match="pinned"):  # pageable memory for a host-resident store
        msa.Bank(docs, kv_loc="host", k_store=full, v_store=full, **kw)
