"""Pins of the fp64 oracle to things other than itself.

Each test checks an oracle function against a closed form, an invariant, a
library routine, a hand-derived special case or a brute-force loop written
with plain Python arithmetic, chosen so that a dropped term, a wrong sign,
a swapped pairing or a transposed operand fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- rounding
def test_bf16_rounding_matches_torch():
    x = (RNG.standard_normal(20000) * np.exp(RNG.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(x.astype(np.float64)), ref)


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour is 1.
    assert O.round_to_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert O.round_to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert O.round_to_bf16(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    assert O.round_to_bf16(0.0) == 0.0
    # just above the tie rounds up
    assert O.round_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7


def test_f32_storage_rounding():
    x = RNG.standard_normal(100)
    np.testing.assert_array_equal(O.round_to_storage(x, "f32"),
                                  x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- pooling
def test_chunk_mean_closed_form():
    # r[t] = c * 1 + (t mod 256 - 127.5) * e_j: every chunk mean is exactly c * 1.
    doc_len = [512, 256, 768]
    T, H, d = sum(doc_len), 2, 8
    r = np.zeros((T, H, d))
    cvals = RNG.integers(-8, 8, size=(T // 256, H)).astype(np.float64)
    for t in range(T):
        for h in range(H):
            r[t, h, :] = cvals[t // 256, h]
            r[t, h, (t // 256 + h) % d] += (t % 256) - 127.5
    kr = O.chunk_mean_pool(r, doc_len)
    expect = np.repeat(cvals[:, :, None], d, axis=2)
    np.testing.assert_array_equal(kr, expect)


def test_chunk_mean_brute_force():
    doc_len = [256, 512]
    r = RNG.standard_normal((768, 1, 3))
    kr = O.chunk_mean_pool(r, doc_len)
    for c in range(3):
        for j in range(3):
            s = math.fsum(r[c * 256 + t, 0, j] for t in range(256)) / 256
            assert abs(kr[c, 0, j] - s) < 1e-15


def test_chunk_rejects_ragged_documents():
    with pytest.raises(ValueError):
        O.chunk_mean_pool(np.zeros((300, 1, 4)), [300])


def test_inverse_norms():
    v = np.array([[3.0, 4.0, 0.0], [0.0, 0.0, 0.0], [1.0, 2.0, 2.0]])
    np.testing.assert_allclose(O.inverse_norms(v), [0.2, 0.0, 1.0 / 3.0], rtol=0, atol=1e-16)


# ---------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    x = RNG.standard_normal((5, 128))
    np.testing.assert_array_equal(O.rope_rotate(x, np.zeros(5), 10000.0), x)


def test_rope_preserves_norm():
    x = RNG.standard_normal((7, 128))
    y = O.rope_rotate(x, RNG.integers(0, 70000, 7), 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rope_relative_position_identity():
    q, k = RNG.standard_normal(128), RNG.standard_normal(128)
    for m, n in [(5, 3), (1000, 17), (65535, 4096), (3, 900)]:
        lhs = O.rope_rotate(q, m, 10000.0) @ O.rope_rotate(k, n, 10000.0)
        rhs = O.rope_rotate(q, m - n, 10000.0) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(lhs))


def test_rope_d2_is_complex_multiplication():
    # d = 2: theta_0 = 1, so (x0 + i x1) is multiplied by exp(i p).
    x = np.array([0.3, -1.7])
    for p in [0.0, 1.0, 2.5, 1234.0]:
        z = complex(x[0], x[1]) * np.exp(1j * p)
        y = O.rope_rotate(x, p, 10000.0)
        assert abs(y[0] - z.real) < 1e-12 and abs(y[1] - z.imag) < 1e-12


def test_rope_pairing_sign_and_frequencies():
    # Hand-derived: for d = 128, base = 10000, theta_16 = 10000^(-1/4) = 0.1 and
    # theta_32 = 10000^(-1/2) = 0.01; theta_0 = 1.  A unit vector e_i is
    # carried to cos(a) e_i + sin(a) e_{i+64}.
    for i, p in [(0, 1.0), (16, 10.0), (32, 100.0)]:
        e = np.zeros(128)
        e[i] = 1.0
        y = O.rope_rotate(e, p, 10000.0)
        expect = np.zeros(128)
        expect[i], expect[i + 64] = math.cos(1.0), math.sin(1.0)
        np.testing.assert_allclose(y, expect, atol=1e-12)
        # the partner component turns the other way
        e2 = np.zeros(128)
        e2[i + 64] = 1.0
        y2 = O.rope_rotate(e2, p, 10000.0)
        expect2 = np.zeros(128)
        expect2[i], expect2[i + 64] = -math.sin(1.0), math.cos(1.0)
        np.testing.assert_allclose(y2, expect2, atol=1e-12)


def test_document_positions_restart():
    assert list(O.document_positions([3, 2, 4])) == [0, 1, 2, 0, 1, 0, 1, 2, 3]


def test_bank_rope_restarts_per_document():
    # the same raw document at different places in the bank gives identical
    # rotated keys
    doc = RNG.standard_normal((256, 2, 128))
    other = RNG.standard_normal((512, 2, 128))
    a = O.bank_keys_rotated(np.concatenate([doc, other]), [256, 512], 10000.0, "bf16")
    b = O.bank_keys_rotated(np.concatenate([other, doc]), [512, 256], 10000.0, "bf16")
    np.testing.assert_array_equal(a[:256], b[512:])
    # and differs from rotating it at bank-global positions
    g = O.round_to_storage(O.rope_rotate(doc, (512 + np.arange(256))[:, None], 10000.0), "bf16")
    assert np.abs(g - b[512:]).max() > 0.1


# ---------------------------------------------------------------- routing
def _brute_scores(q, kr, doc_len):
    B, H, d = q.shape
    off = np.concatenate([[0], np.cumsum(np.array(doc_len) // 256)])
    out = np.zeros((B, len(doc_len)))
    for b in range(B):
        for n in range(len(doc_len)):
            acc = 0.0
            for h in range(H):
                best = -math.inf
                for c in range(off[n], off[n + 1]):
                    dot = math.fsum(q[b, h, i] * kr[c, h, i] for i in range(d))
                    nq = math.sqrt(math.fsum(v * v for v in q[b, h]))
                    nk = math.sqrt(math.fsum(v * v for v in kr[c, h]))
                    best = max(best, dot / (nq * nk))
                acc += best
            out[b, n] = acc / H
    return out


def test_cosine_scores_brute_force():
    doc_len = [256, 768, 512]
    kr = RNG.standard_normal((9, 3, 6))
    q = RNG.standard_normal((2, 3, 6))
    got = O.cosine_doc_scores(q, kr, O.inverse_norms(kr), doc_len)
    np.testing.assert_allclose(got, _brute_scores(q, kr, doc_len), atol=1e-14)


def test_cosine_scale_invariance_and_self_match():
    doc_len = [512, 512, 256]
    kr = RNG.standard_normal((5, 1, 16))
    inv = O.inverse_norms(kr)
    q = kr[3:4].copy()  # chunk 3 belongs to document 1
    s = O.cosine_doc_scores(q, kr, inv, doc_len)
    assert abs(s[0, 1] - 1.0) < 1e-14 and s[0].argmax() == 1
    s2 = O.cosine_doc_scores(q * 37.0, kr * 0.01, O.inverse_norms(kr * 0.01), doc_len)
    np.testing.assert_allclose(s, s2, atol=1e-14)


def test_cosine_zero_query_and_exclusion():
    doc_len = [256, 256]
    kr = RNG.standard_normal((2, 1, 8))
    s = O.cosine_doc_scores(np.zeros((1, 1, 8)), kr, O.inverse_norms(kr), doc_len)
    np.testing.assert_array_equal(s, [[0.0, 0.0]])
    q = RNG.standard_normal((1, 1, 8))
    s = O.cosine_doc_scores(q, kr, O.inverse_norms(kr), doc_len, exclude=[[False, True]])
    assert s[0, 1] == -np.inf and np.isfinite(s[0, 0])


def test_mean_over_heads_of_max_over_chunks():
    # two heads, one document of two chunks: head 0 prefers chunk 0, head 1
    # prefers chunk 1; the score averages the two per-head maxima.
    kr = np.zeros((2, 2, 2))
    kr[0, 0] = [1, 0]; kr[1, 0] = [0, 1]
    kr[0, 1] = [0, 1]; kr[1, 1] = [1, 1]
    q = np.array([[[1.0, 0.0], [1.0, 1.0]]])
    s = O.cosine_doc_scores(q, kr, O.inverse_norms(kr), [512])
    assert abs(s[0, 0] - 1.0) < 1e-15  # (max(1, 0) + max(1/sqrt2, 1)) / 2


def test_topk_brute_force_with_ties():
    for _ in range(20):
        N = int(RNG.integers(3, 40))
        k = int(RNG.integers(1, N + 1))
        s = RNG.integers(0, 5, size=(3, N)).astype(np.float64)  # many ties
        ids, vals = O.select_topk(s, k)
        for b in range(3):
            expect = sorted(range(N), key=lambda n: (-s[b, n], n))[:k]
            assert list(ids[b]) == expect
            assert list(vals[b]) == [s[b, n] for n in expect]


def test_duplicate_documents_lower_id_wins():
    doc_len = [256] * 6
    kr = RNG.standard_normal((6, 1, 8))
    kr[4] = kr[1]  # identical documents 1 and 4
    q = kr[1:2] + 0.01 * RNG.standard_normal((1, 1, 8))
    s = O.cosine_doc_scores(q, kr, O.inverse_norms(kr), doc_len)
    ids, _ = O.select_topk(s, 2)
    assert list(ids[0]) == [1, 4]


# ---------------------------------------------------------------- attention
def _brute_attention(q, K, V, scale, mask=None):
    M, L = q.shape[0], K.shape[0]
    out = np.zeros((M, V.shape[1]))
    for i in range(M):
        s = [math.fsum(q[i, a] * K[j, a] for a in range(q.shape[1])) * scale
             if (mask is None or mask[i, j]) else -math.inf for j in range(L)]
        mx = max(s)
        w = [math.exp(v - mx) for v in s]
        z = math.fsum(w)
        for c in range(V.shape[1]):
            out[i, c] = math.fsum(w[j] * V[j, c] for j in range(L)) / z
    return out


def test_softmax_attention_brute_force():
    q, K, V = RNG.standard_normal((3, 8)), RNG.standard_normal((11, 8)), RNG.standard_normal((11, 5))
    np.testing.assert_allclose(O.softmax_attention(q, K, V, 0.3),
                               _brute_attention(q, K, V, 0.3), atol=1e-14)
    mask = RNG.random((3, 11)) < 0.6
    mask[:, 0] = True
    np.testing.assert_allclose(O.softmax_attention(q, K, V, 0.3, mask),
                               _brute_attention(q, K, V, 0.3, mask), atol=1e-14)


def test_softmax_rows_sum_to_one():
    q, K = RNG.standard_normal((4, 16)) * 5, RNG.standard_normal((50, 16))
    out = O.softmax_attention(q, K, np.ones((50, 3)), 1.0)
    np.testing.assert_allclose(out, 1.0, atol=1e-14)


def test_single_key_returns_its_value():
    v = RNG.standard_normal((1, 7))
    out = O.softmax_attention(RNG.standard_normal((2, 4)), RNG.standard_normal((1, 4)), v, 1.0)
    np.testing.assert_allclose(out, np.repeat(v, 2, 0), atol=1e-15)


def test_gqa_equals_mha_with_repeated_heads():
    M, Hq, Hkv, d, L = 3, 8, 2, 16, 20
    q = RNG.standard_normal((M, Hq, d))
    K, V = RNG.standard_normal((L, Hkv, d)), RNG.standard_normal((L, Hkv, d))
    got = O.gqa_attention(q, K, V)
    Kr, Vr = np.repeat(K, Hq // Hkv, axis=1), np.repeat(V, Hq // Hkv, axis=1)
    for hq in range(Hq):
        ref = _brute_attention(q[:, hq], Kr[:, hq], Vr[:, hq], 1.0 / math.sqrt(d))
        np.testing.assert_allclose(got[:, hq], ref, atol=1e-13)


def _tiny_bank(doc_len, Hr=1, Hkv=2, d=128, seed=0):
    g = np.random.default_rng(seed)
    T = sum(doc_len)
    r = g.standard_normal((T, Hr, d))
    kr = O.round_to_storage(O.chunk_mean_pool(r, doc_len), "f32")
    k_raw, v = g.standard_normal((T, Hkv, d)), g.standard_normal((T, Hkv, d))
    k_rot = O.bank_keys_rotated(k_raw, doc_len, 10000.0, "f32")
    return kr, O.inverse_norms(kr), k_raw, k_rot, v


def test_decode_with_k_equal_n_is_dense_attention():
    doc_len = [256, 512, 256]
    kr, inv, k_raw, k_rot, v = _tiny_bank(doc_len)
    B, Hq, d, L = 2, 8, 128, 40
    q = RNG.standard_normal((B, Hq, d))
    qr_route = RNG.standard_normal((B, 1, d))
    lk, lv = RNG.standard_normal((B, L, 2, d)), RNG.standard_normal((B, L, 2, d))
    P0 = 512
    out, ids, _ = O.decode_step(q, P0 + L - 1, qr_route, kr, inv, k_rot, v, doc_len,
                                lk, lv, P0, len(doc_len), 10000.0, "f32")
    for b in range(B):
        # dense attention over documents in their own order, then local
        lkr = O.round_to_storage(O.rope_rotate(lk[b], (P0 + np.arange(L))[:, None], 10000.0), "f32")
        K = np.concatenate([k_rot, lkr])
        V = np.concatenate([v, lv[b]])
        qrot = O.rope_rotate(q[b], P0 + L - 1, 10000.0)
        for hq in range(Hq):
            ref = _brute_attention(qrot[hq:hq + 1], K[:, hq // 4], V[:, hq // 4], 1 / math.sqrt(d))
            np.testing.assert_allclose(out[b, hq], ref[0], atol=1e-12)


def test_prefill_causal_mask_brute_force():
    doc_len = [256, 256, 512]
    kr, inv, k_raw, k_rot, v = _tiny_bank(doc_len, Hr=2, seed=3)
    Lq, L, block, Hq, d = 8, 12, 4, 8, 128
    q = RNG.standard_normal((Lq, Hq, d))
    route = RNG.standard_normal((Lq, 2, d))
    lk, lv = RNG.standard_normal((L, 2, d)), RNG.standard_normal((L, 2, d))
    P0 = 512
    out, ids, _ = O.prefill(q, route, kr, inv, k_rot, v, doc_len, lk, lv, P0, 2, block,
                            10000.0, "f32")
    starts = np.concatenate([[0], np.cumsum(doc_len)])
    lkr = O.round_to_storage(O.rope_rotate(lk, (P0 + np.arange(L))[:, None], 10000.0), "f32")
    for i in range(Lq):
        blk = i // block
        # routing of the block: brute-force mean of its router vectors
        qb = np.array([[[math.fsum(route[blk * block + t, h, a] for t in range(block)) / block
                         for a in range(d)] for h in range(2)]])
        s = _brute_scores(qb, kr, doc_len)[0]
        top = sorted(range(len(doc_len)), key=lambda n: (-s[n], n))[:2]
        assert list(ids[blk]) == top
        li = L - Lq + i  # local index of query i
        K = np.concatenate([k_rot[starts[n]:starts[n + 1]] for n in top] + [lkr[:li + 1]])
        V = np.concatenate([v[starts[n]:starts[n + 1]] for n in top] + [lv[:li + 1]])
        qrot = O.rope_rotate(q[i], P0 + li, 10000.0)
        for hq in range(Hq):
            ref = _brute_attention(qrot[hq:hq + 1], K[:, hq // 4], V[:, hq // 4], 1 / math.sqrt(d))
            np.testing.assert_allclose(out[i, hq], ref[0], atol=1e-12)


def test_block_mean_and_projection_brute_force():
    r = RNG.standard_normal((6, 2, 3))
    bm = O.block_mean_queries(r, 3)
    for b in range(2):
        for h in range(2):
            for a in range(3):
                assert abs(bm[b, h, a] - math.fsum(r[b * 3 + t, h, a] for t in range(3)) / 3) < 1e-15
    out = RNG.standard_normal((2, 4, 5))
    w = RNG.standard_normal((3, 20))
    p = O.interleave_project(out, w)
    assert p.shape == (2, 1, 3)
    for b in range(2):
        flat = [out[b, h, a] for h in range(4) for a in range(5)]
        for j in range(3):
            assert abs(p[b, 0, j] - math.fsum(w[j, i] * flat[i] for i in range(20))) < 1e-13


# ---------------------------------------------------------------- compressed memory
def test_pooled_kv_brute_force():
    rng = np.random.default_rng(71)
    doc_len = [512, 256]
    k = rng.standard_normal((768, 2, 4))
    v = rng.standard_normal((768, 2, 4))
    pk, pv = O.pooled_kv(k, v, doc_len, "f64")
    assert pk.shape == (3, 2, 4)
    for c in range(3):
        for h in range(2):
            for i in range(4):
                assert math.isclose(pk[c, h, i], math.fsum(k[256 * c:256 * (c + 1), h, i]) / 256,
                                    rel_tol=0, abs_tol=1e-15)
                assert math.isclose(pv[c, h, i], math.fsum(v[256 * c:256 * (c + 1), h, i]) / 256,
                                    rel_tol=0, abs_tol=1e-15)


def test_pooled_attention_equals_full_when_chunks_are_constant():
    """If every token of a chunk has the same key and value, one pooled
    entry with log-weight ln 256 is exactly the chunk's 256 tokens."""
    rng = np.random.default_rng(72)
    C, H, d = 3, 2, 8
    kc = rng.standard_normal((C, H, d))
    vc = rng.standard_normal((C, H, d))
    K = np.repeat(kc, 256, axis=0)
    V = np.repeat(vc, 256, axis=0)
    q = rng.standard_normal((5, 4, d))
    full = O.gqa_attention(q, K, V)
    pk, pv = O.pooled_kv(K, V, [256 * C], "f64")
    np.testing.assert_allclose(pk, kc, rtol=1e-14, atol=0)  # a few ulps of summation
    pooled = O.gqa_attention(q, pk, pv, None, np.full(C, np.log(256)))
    np.testing.assert_allclose(pooled, full, rtol=0, atol=1e-12)
    # without the log-weight the local tokens would be over-weighted
    loc_k = rng.standard_normal((7, H, d))
    loc_v = rng.standard_normal((7, H, d))
    full2 = O.gqa_attention(q, np.concatenate([K, loc_k]), np.concatenate([V, loc_v]))
    pooled2 = O.gqa_attention(q, np.concatenate([pk, loc_k]), np.concatenate([pv, loc_v]), None,
                              np.concatenate([np.full(C, np.log(256)), np.zeros(7)]))
    np.testing.assert_allclose(pooled2, full2, rtol=0, atol=1e-12)
    unweighted = O.gqa_attention(q, np.concatenate([pk, loc_k]), np.concatenate([pv, loc_v]))
    assert np.abs(unweighted - full2).max() > 1e-3


def test_attention_bias_is_a_log_weight():
    """A bias of ln n on a key equals n copies of it."""
    rng = np.random.default_rng(73)
    q = rng.standard_normal((3, 6))
    K = rng.standard_normal((4, 6))
    V = rng.standard_normal((4, 5))
    rep = O.softmax_attention(q, np.concatenate([K, np.repeat(K[1:2], 4, axis=0)]),
                              np.concatenate([V, np.repeat(V[1:2], 4, axis=0)]), 0.3)
    b = np.zeros(4)
    b[1] = np.log(5)
    np.testing.assert_allclose(O.softmax_attention(q, K, V, 0.3, None, b), rep, rtol=0, atol=1e-12)


def test_pooled_decode_step_reduces_to_decode_step_on_constant_chunks():
    """End to end: with chunk-constant bank K/V, the compressed decode step
    equals the per-token decode step (routing identical, attention equal)."""
    rng = np.random.default_rng(74)
    doc_len = [512, 256, 768]
    T, C = sum(doc_len), sum(doc_len) // 256
    H_kv, H_q, d, L = 2, 4, 8, 5
    kc = rng.standard_normal((C, H_kv, d))
    vc = rng.standard_normal((C, H_kv, d))
    bank_k = np.repeat(kc, 256, axis=0)
    bank_v = np.repeat(vc, 256, axis=0)
    keys = rng.standard_normal((C, 1, d))
    inv = O.inverse_norms(keys)
    q = rng.standard_normal((2, H_q, d))
    qr = rng.standard_normal((2, 1, d))
    lk = rng.standard_normal((2, L, H_kv, d))
    lv = rng.standard_normal((2, L, H_kv, d))
    a, ia, _ = O.decode_step(q, 900, qr, keys, inv, bank_k, bank_v, doc_len, lk, lv, 890, 2,
                             10000.0, "f64")
    pk, pv = O.pooled_kv(bank_k, bank_v, doc_len, "f64")
    b, ib, _ = O.pooled_decode_step(q, 900, qr, keys, inv, pk, pv, doc_len, lk, lv, 890, 2,
                                    10000.0, "f64")
    np.testing.assert_array_equal(ia, ib)
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)



# ---------------------------------------------------------------- helpers, pinned directly
def test_chunk_offsets_hand_values():
    # documents of 1, 2 and 3 chunks own chunks [0,1), [1,3), [3,6)
    np.testing.assert_array_equal(O.chunk_offsets([256, 512, 768]), [0, 1, 3, 6])
    with pytest.raises(ValueError):
        O.chunk_offsets([256, 300])
    with pytest.raises(ValueError):
        O.chunk_offsets([0])


def test_rope_frequencies_closed_form():
    # theta_0 = 1, theta_{d/2-1} = base^(-(d-2)/d), a constant ratio base^(-2/d)
    d, base = 128, 10000.0
    th = O.rope_frequencies(d, base)
    assert th.shape == (64,) and th[0] == 1.0
    assert math.isclose(th[-1], base ** (-(d - 2) / d), rel_tol=1e-15)
    np.testing.assert_allclose(th[1:] / th[:-1], base ** (-2.0 / d), rtol=1e-14)
    # d = 4: angles 1 and base^-1/2, by hand
    np.testing.assert_allclose(O.rope_frequencies(4, 100.0), [1.0, 0.1], rtol=1e-15)


def test_union_kv_order_and_rows():
    # rows tagged by (document, token): the union holds the selected
    # documents' rows in rank order, then the local rows
    doc_len = [2, 3, 1]
    T = sum(doc_len)
    bank_k = np.arange(T, dtype=np.float64).reshape(T, 1, 1) * np.ones((1, 1, 4))
    bank_v = -bank_k
    loc_k = np.full((2, 1, 4), 100.0)
    loc_v = np.full((2, 1, 4), 200.0)
    K, V = O.union_kv([2, 0], bank_k, bank_v, doc_len, loc_k, loc_v)
    np.testing.assert_array_equal(K[:, 0, 0], [5, 0, 1, 100, 100])
    np.testing.assert_array_equal(V[:, 0, 0], [-5, 0, -1, 200, 200])
    K, V = O.union_kv([], bank_k, bank_v, doc_len, loc_k, loc_v)
    assert K.shape == (2, 1, 4)
