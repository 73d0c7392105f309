"""Top-k selection on both of its paths, through msa_route: banks of up to
2048 documents take the single-launch kernel (one workgroup per query),
larger ones the multi-level kernel (two levels up to 65,536 documents, three
beyond).  Routing keys are drawn directly (one
256-token chunk per document, no K/V needed: every document shares one
K/V block), so banks just either side of the boundary stay small; the
selections are checked against the oracle's cosine scores, with exclusion
masks (down to a query that excludes every document) and the largest k."""
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


@pytest.mark.parametrize("n_docs,k", [(2048, 16), (2048, 64), (2049, 16), (2049, 64),
                                     (9000, 64), (100, 64)])
def test_topk_paths_match_oracle(msa, n_docs, k):
    w = S.Workload(f"topk_{n_docs}", "bf16", [256] * n_docs, h_r=8, h_kv=1, h_q=4, k=k, B=5,
                   keys_given=True, seed=2201)
    kr = S.keys_direct(w, DEV).to(w.torch_dtype)  # [C, h_r, 128]
    bank = msa.Bank(w.doc_len, w.h_r, 1, "bf16", DEV, kv_off=[0] * n_docs, kv_tokens=256,
                    kr=kr.permute(1, 0, 2).contiguous())
    bank.build(0, n_docs)  # inverse norms of the given keys
    qr = S.route_queries(w, DEV)
    # exclusion: query 1 excludes every third document, query 3 all but 70,
    # query 4 every document
    W = (n_docs + 31) // 32
    ex = np.zeros((w.B, n_docs), dtype=bool)
    ex[1, ::3] = True
    ex[3, 70:] = True
    ex[4, :] = True
    words = np.zeros((w.B, W), dtype=np.uint32)
    for b in range(w.B):
        for n in np.nonzero(ex[b])[0]:
            words[b, n >> 5] |= np.uint32(1) << np.uint32(n & 31)
    excl = torch.from_numpy(words.view(np.int32)).to(DEV)
    ids, scores = bank.route(qr, k, exclude=excl)
    torch.cuda.synchronize()
    kr_o = M.np64(kr)
    so = O.cosine_doc_scores(M.np64(qr), kr_o, O.inverse_norms(kr_o), w.doc_len, ex)
    ids, scores = ids.cpu().numpy(), scores.cpu().numpy()
    valid = [b for b in range(w.B) if (~ex[b]).sum() >= k]
    M.check_topk(ids[valid], scores[valid], so[valid], k)
    for b in range(w.B):
        assert not ex[b, ids[b][ids[b] >= 0]].any(), f"query {b} selected an excluded document"
    # query 3 keeps only 70 documents: with k = 64 all of them but 6, else k
    assert (ids[3] >= 0).sum() == min(k, 70)
    # query 4 keeps none: every slot empty
    assert (ids[4] == -1).all() and np.isneginf(scores[4]).all()
