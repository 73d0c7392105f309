"""Plain float64 CPU oracle for the Memory Sparse Attention (MSA) hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library under ``long_context_memory_amd/csrc``.

Every function is a direct, slow statement of what the method computes, in
float64 numpy, in the natural (token-major) layouts a model would produce.
Rounding happens only where the method *stores* a tensor (the routing keys,
the rotated document keys, the rotated local keys), to the storage dtype.

Sources (the pages' text; no formulas are printed there, so each step is the
plainest reading of the prose):

* "MSA架构：突破大模型记忆瓶颈的稀疏注意力技术" (intelliparadigm.com),
  section 2.1 (router by latent cosine top-k; 256-token chunk-mean pooling)
  and section 3.1 (the ``chunk_mean_pooling`` snippet: a view into
  256-row chunks followed by a mean over the chunk axis).
* "MSA" card (robocikowo.com), section "Komponenty":
  the MSA layer picks the top-k documents of a compressed bank and appends
  their K/V to the local context; the router key Kr is matched to the query
  by cosine similarity; document-wise RoPE resets the position counter to 0
  at each document; global RoPE with an offset for the active context;
  "Memory Interleave" alternates document-id generation and context
  expansion.  "Paradygmat wykonania": only the k selected blocks take part.
* the MLA/CSA attention article (mlqm.cn), section 6.2: the attention scale
  1/sqrt(head_dim).

Readings where the pages are silent:
rotate-half RoPE pairing (i, i + d/2) with theta_i = base^(-2i/d); no RoPE on
routing keys; a document's score is the mean over router heads of the max
cosine over its chunks; ties in top-k go to the lower document id; query
head hq reads KV head hq // G; the cosine of a zero vector is 0.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` (closed forms, invariants, brute force, library
routines).  The end-to-end composition has no worked example on the pages.
"""
from __future__ import annotations

import numpy as np

CHUNK = 256  # routing-key chunk length (intelliparadigm.com, section 2.1 / 3.1)


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------
def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    bfloat16 keeps 8 significant bits.  frexp writes x = m * 2**e with
    |m| in [0.5, 1); x * 2**(8 - e) then has its 8 significant bits in the
    integer part, and ``np.rint`` rounds half to even.  Magnitudes in this
    path stay far from bfloat16's overflow and subnormal ranges.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    scaled = np.ldexp(m, 8)  # |scaled| in [128, 256)
    return np.ldexp(np.rint(scaled), e - 8)


def round_to_storage(x, dtype: str):
    """Round to the bank's storage dtype ("f32" or "bf16"; "f64" keeps the
    value, for exact identities in the pins); float64 out."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# a1: chunk-mean pooling into routing keys
# --------------------------------------------------------------------------
def chunk_offsets(doc_len, chunk: int = CHUNK):
    """Prefix offsets of each document's chunks: doc n owns chunks
    [off[n], off[n+1]).  Every document length is a whole number of chunks."""
    doc_len = np.asarray(doc_len, dtype=np.int64)
    if np.any(doc_len <= 0) or np.any(doc_len % chunk):
        raise ValueError("document lengths must be positive multiples of the chunk")
    return np.concatenate([[0], np.cumsum(doc_len // chunk)])


def chunk_mean_pool(route_vec, doc_len, chunk: int = CHUNK):
    """Routing keys: the mean of each run of ``chunk`` consecutive per-token
    routing vectors (intelliparadigm.com, section 3.1 snippet).

    route_vec: [T, H_r, d_r].  Documents are laid end to end and each length
    is a multiple of ``chunk``, so no chunk straddles two documents.
    Returns float64 [C, H_r, d_r], C = T / chunk, before storage rounding.
    """
    r = np.asarray(route_vec, dtype=np.float64)
    chunk_offsets(doc_len, chunk)
    T, H, d = r.shape
    if T != int(np.sum(doc_len)):
        raise ValueError("route_vec rows must equal the total document length")
    return r.reshape(T // chunk, chunk, H, d).mean(axis=1)


def inverse_norms(keys):
    """1 / ||key|| over the last axis; 0 for a zero key."""
    k = np.asarray(keys, dtype=np.float64)
    n = np.sqrt(np.sum(k * k, axis=-1))
    out = np.zeros_like(n)
    nz = n > 0
    out[nz] = 1.0 / n[nz]
    return out


# --------------------------------------------------------------------------
# a2 / a3: rotary position embedding
# --------------------------------------------------------------------------
def rope_frequencies(d: int, base: float):
    """theta_i = base ** (-2 i / d) for i in [0, d/2)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def rope_rotate(x, pos, base: float):
    """Rotate-half RoPE: pairs (i, i + d/2) turned by angle pos * theta_i.

    x: [..., d]; pos: broadcastable to x.shape[:-1] (any real positions).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_frequencies(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def document_positions(doc_len):
    """Document-wise positions: 0, 1, ..., L_n - 1 restarting at every
    document ("MSA" card, robocikowo.com, section "Komponenty", Document-wise RoPE)."""
    return np.concatenate([np.arange(int(L), dtype=np.int64) for L in doc_len])


def bank_keys_rotated(k_raw, doc_len, base: float, dtype: str):
    """Document K rotated at document-local positions, rounded to storage.

    k_raw: [T, H_kv, d].  Returns float64 [T, H_kv, d]."""
    pos = document_positions(doc_len)
    k = rope_rotate(np.asarray(k_raw, dtype=np.float64), pos[:, None], base)
    return round_to_storage(k, dtype)


# --------------------------------------------------------------------------
# a4 / a5: cosine routing and top-k
# --------------------------------------------------------------------------
def cosine_doc_scores(q_route, keys, inv_norm, doc_len, exclude=None):
    """Document scores for each router query.

    cos[b, h, c] = (q[b,h] . Kr[c,h]) * inv_norm[c,h] / ||q[b,h]||  (0 when a
    norm is 0); score[b, n] = mean over h of max over the chunks c of
    document n.  exclude: optional bool [B, N]; excluded documents score -inf.

    q_route: [B, H_r, d_r]; keys: [C, H_r, d_r]; inv_norm: [C, H_r].
    Returns float64 [B, N].
    """
    q = np.asarray(q_route, dtype=np.float64)
    kr = np.asarray(keys, dtype=np.float64)
    inv = np.asarray(inv_norm, dtype=np.float64)
    off = chunk_offsets(doc_len)
    B, H, _ = q.shape
    qn = np.sqrt(np.sum(q * q, axis=-1))
    inv_q = np.where(qn > 0, 1.0 / np.where(qn > 0, qn, 1.0), 0.0)
    dots = np.einsum("bhd,chd->bhc", q, kr)
    cos = dots * inv.T[None, :, :] * inv_q[:, :, None]
    N = len(off) - 1
    per_head = np.empty((B, H, N))
    for n in range(N):
        per_head[:, :, n] = cos[:, :, off[n]:off[n + 1]].max(axis=2)
    score = per_head.mean(axis=1)
    if exclude is not None:
        score = np.where(np.asarray(exclude, dtype=bool), -np.inf, score)
    return score


def select_topk(scores, k: int):
    """The k highest scores per row, ordered by (score descending, id
    ascending); equal scores go to the lower document id.

    Returns (ids int64 [B, k], values float64 [B, k])."""
    s = np.asarray(scores, dtype=np.float64)
    B, N = s.shape
    ids = np.empty((B, k), dtype=np.int64)
    for b in range(B):
        order = np.lexsort((np.arange(N), -s[b]))
        ids[b] = order[:k]
    return ids, np.take_along_axis(s, ids, axis=1)


# --------------------------------------------------------------------------
# a7 / a8: softmax attention over the union
# --------------------------------------------------------------------------
def softmax_attention(q, keys, values, scale, mask=None, bias=None):
    """out[i] = sum_j softmax_j(q[i] . keys[j] * scale + bias[j]) values[j].

    q: [M, d]; keys: [L, d]; values: [L, dv]; mask: optional bool [M, L]
    (True = attend); bias: optional [L] log-weights of the keys (a key that
    stands for n identical tokens has bias ln n).  Max-subtracted float64
    softmax."""
    q = np.asarray(q, dtype=np.float64)
    s = (q @ np.asarray(keys, dtype=np.float64).T) * scale
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[None, :]
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ np.asarray(values, dtype=np.float64)


def gqa_attention(q, keys, values, mask=None, bias=None):
    """Grouped-query attention with the 1/sqrt(d) scale.

    q: [M, H_q, d]; keys/values: [L, H_kv, d]; query head hq reads KV head
    hq // (H_q / H_kv).  mask: optional bool [M, L]; bias: optional [L]
    key log-weights (see softmax_attention).  Returns [M, H_q, d]."""
    q = np.asarray(q, dtype=np.float64)
    M, Hq, d = q.shape
    Hkv = keys.shape[1]
    G = Hq // Hkv
    out = np.empty((M, Hq, values.shape[2]))
    for hq in range(Hq):
        h = hq // G
        out[:, hq, :] = softmax_attention(q[:, hq, :], keys[:, h, :], values[:, h, :],
                                          1.0 / np.sqrt(d), mask, bias)
    return out


def union_kv(ids, bank_k_rot, bank_v, doc_len, local_k_rot, local_v):
    """The attended context of one query: the selected documents' K/V in
    rank order followed by the local context ("MSA" card, robocikowo.com, section "Komponenty", the MSA
    layer).  bank_*: [T, H_kv, d] in document order; local_*: [L_loc, H_kv, d]."""
    starts = np.concatenate([[0], np.cumsum(doc_len)])
    ks = [bank_k_rot[starts[n]:starts[n + 1]] for n in ids] + [local_k_rot]
    vs = [bank_v[starts[n]:starts[n + 1]] for n in ids] + [local_v]
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


# --------------------------------------------------------------------------
# composites: one decode step, one blocked prefill, memory interleave
# --------------------------------------------------------------------------
def decode_step(q, q_pos, q_route, keys, inv_norm, bank_k_rot, bank_v, doc_len,
                local_k_raw, local_v, local_pos0, k, base, dtype, exclude=None):
    """Route, select, gather and attend for a batch of decode queries.

    q: [B, H_q, d] (pre-RoPE); q_route: [B, H_r, d_r]; keys/inv_norm: the
    stored routing keys; bank_k_rot/bank_v: [T, H_kv, d] stored bank K (already
    document-RoPE'd) and V; local_k_raw/local_v: [B, L_loc, H_kv, d] with local
    token j at global position local_pos0 + j.  The query sits at q_pos.

    Returns (out [B, H_q, d], ids [B, k], scores [B, k])."""
    scores = cosine_doc_scores(q_route, keys, inv_norm, doc_len, exclude)
    ids, vals = select_topk(scores, k)
    B = q.shape[0]
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(B):
        L = local_k_raw.shape[1]
        lk = round_to_storage(
            rope_rotate(local_k_raw[b], (local_pos0 + np.arange(L))[:, None], base), dtype)
        K, V = union_kv(ids[b], bank_k_rot, bank_v, doc_len, lk, local_v[b])
        qr = rope_rotate(q[b][None], np.full((1, q.shape[1]), q_pos), base)
        out[b] = gqa_attention(qr, K, V)[0]
    return out, ids, vals


def block_mean_queries(route_tokens, block: int):
    """Per-block router query: the arithmetic mean of the block's per-token
    router vectors.  route_tokens: [L_q, H_r, d_r] -> [L_q / block, H_r, d_r]."""
    r = np.asarray(route_tokens, dtype=np.float64)
    L, H, d = r.shape
    return r.reshape(L // block, block, H, d).mean(axis=1)


def prefill(q, route_tokens, keys, inv_norm, bank_k_rot, bank_v, doc_len,
            local_k_raw, local_v, pos0, k, block, base, dtype):
    """Blocked prefill: each block of ``block`` queries routes with its mean
    router vector, shares one top-k document set, and every query attends
    to all selected document tokens plus the local tokens at or before its
    own position.  The L_q queries are the last L_q local tokens.

    q: [L_q, H_q, d] pre-RoPE; local_*: [L_loc, H_kv, d]; local token j at
    position pos0 + j.  Returns (out [L_q, H_q, d], ids [nb, k], scores)."""
    Lq = q.shape[0]
    L = local_k_raw.shape[0]
    qb = block_mean_queries(route_tokens, block)
    scores = cosine_doc_scores(qb, keys, inv_norm, doc_len)
    ids, vals = select_topk(scores, k)
    lpos = pos0 + np.arange(L)
    lk = round_to_storage(rope_rotate(local_k_raw, lpos[:, None], base), dtype)
    qpos = lpos[L - Lq:]
    qr = rope_rotate(q, qpos[:, None], base)
    out = np.empty(q.shape, dtype=np.float64)
    for blk in range(Lq // block):
        rows = slice(blk * block, (blk + 1) * block)
        K, V = union_kv(ids[blk], bank_k_rot, bank_v, doc_len, lk, local_v)
        n_doc = K.shape[0] - L
        qi = np.arange(blk * block, (blk + 1) * block) + (L - Lq)  # local index
        mask = np.ones((block, K.shape[0]), dtype=bool)
        mask[:, n_doc:] = np.arange(L)[None, :] <= qi[:, None]
        out[rows] = gqa_attention(qr[rows], K, V, mask)
    return out, ids, vals


def interleave_project(out, w):
    """Next hop's router query: W times the concatenation of the previous
    hop's per-head outputs.  out: [B, H_q, d]; w: [d_r, H_q * d].
    Returns [B, 1, d_r]."""
    o = np.asarray(out, dtype=np.float64).reshape(out.shape[0], -1)
    return (o @ np.asarray(w, dtype=np.float64).T)[:, None, :]


# --------------------------------------------------------------------------
# compressed (pooled) memory: attention over chunk means of the selected
# documents' K/V
# --------------------------------------------------------------------------
def pooled_kv(k_rot, v, doc_len, dtype: str):
    """The compressed memory of a bank: each 256-token chunk of every document
    becomes one entry, the mean of its stored (document-RoPE'd) keys and the
    mean of its values, rounded to the storage dtype -- the chunk-mean
    pooling of the intelliparadigm.com article (section 3.1, "KV cache
    compression") applied to K and V.

    k_rot, v: [T, H_kv, d] stored K (rotated, rounded) and V; returns
    ([C, H_kv, d], [C, H_kv, d])."""
    return (round_to_storage(chunk_mean_pool(k_rot, doc_len), dtype),
            round_to_storage(chunk_mean_pool(v, doc_len), dtype))


def pooled_decode_step(q, q_pos, q_route, keys, inv_norm, pool_k, pool_v, doc_len,
                       local_k_raw, local_v, local_pos0, k, base, dtype, exclude=None):
    """Decode with a compressed memory: route and select as decode_step, then
    attend over the selected documents' pooled entries (rank order, each
    with the log-weight ln 256 of the 256 tokens it stands for) followed by
    the local context's tokens.

    pool_k, pool_v: [C, H_kv, d] from pooled_kv.  Other arguments as in
    decode_step.  Returns (out [B, H_q, d], ids [B, k], scores [B, k])."""
    scores = cosine_doc_scores(q_route, keys, inv_norm, doc_len, exclude)
    ids, vals = select_topk(scores, k)
    off = chunk_offsets(doc_len)
    B = q.shape[0]
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(B):
        L = local_k_raw.shape[1]
        lk = round_to_storage(
            rope_rotate(local_k_raw[b], (local_pos0 + np.arange(L))[:, None], base), dtype)
        pk = [pool_k[off[n]:off[n + 1]] for n in ids[b] if n >= 0]
        pv = [pool_v[off[n]:off[n + 1]] for n in ids[b] if n >= 0]
        n_pool = sum(x.shape[0] for x in pk)
        K = np.concatenate(pk + [lk])
        V = np.concatenate(pv + [local_v[b]])
        bias = np.concatenate([np.full(n_pool, np.log(CHUNK)), np.zeros(L)])
        qr = rope_rotate(q[b][None], np.full((1, q.shape[1]), q_pos), base)
        out[b] = gqa_attention(qr, K, V, None, bias)[0]
    return out, ids, vals
