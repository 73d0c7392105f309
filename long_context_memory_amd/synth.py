"""Seeded synthetic inputs for the MSA hot path.

This module draws random inputs only: it holds none of the method's
arithmetic (no pooling, no RoPE, no cosine, no softmax).  Both the HIP path
and the fp64 oracle consume what it produces.  Tensors come out in the
natural token-major layouts a model would emit; arranging them into the
bank's storage layout is the library's job.

Every array is drawn with its own ``torch.Generator`` seeded from
(workload seed, array name), on the device the caller asks for; a given
(seed, name, device) always gives the same values.  Values are N(0, 1) in
float32 unless stated otherwise, then rounded to bfloat16 (round to nearest
even, torch's conversion) for bf16 workloads.

The workloads mirror the five configurations the method is measured on:
a tiny fp32 decode, a 1M-token bf16 decode, an 8M-token blocked prefill, a
100M-token bank with host-resident K/V, and a 32M-token, 3-hop Memory
Interleave; plus small siblings of each for fast parity runs.
"""
from __future__ import annotations

import dataclasses
import math
import zlib
from typing import List, Optional

import numpy as np
import torch

CHUNK = 256


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16": bank storage and activations
    doc_len: List[int]              # tokens per document (multiples of 256)
    h_r: int = 1                    # router heads
    d_r: int = 128
    h_kv: int = 8
    h_q: int = 32
    d: int = 128
    k: int = 16
    B: int = 1                      # decode queries (prefill: query tokens)
    L_loc: int = 0                  # local-context tokens
    pos0: Optional[int] = None      # first local position; None = longest document
    mode: str = "decode"            # "decode" | "prefill" | "interleave"
    plant: Optional[str] = None     # "pooled_key" | "direction" | None
    plant_strength: float = 0.1
    plant_batches: int = 1          # "direction": query batches with planted targets
    block: int = 64                 # prefill routing block
    hops: int = 1
    exclude_selected: bool = False
    keys_given: bool = False        # routing keys drawn directly (no pooling input)
    kv_host: bool = False           # K/V live in pinned host memory
    host_slots: int = 0             # physical document slots backing a host bank
    rope_base: float = 10000.0
    seed: int = 0

    @property
    def n_docs(self) -> int:
        return len(self.doc_len)

    @property
    def T(self) -> int:
        return int(sum(self.doc_len))

    @property
    def C(self) -> int:
        return self.T // CHUNK

    @property
    def G(self) -> int:
        return self.h_q // self.h_kv

    @property
    def P0(self) -> int:
        return int(max(self.doc_len)) if self.pos0 is None else int(self.pos0)

    @property
    def q_pos(self) -> int:
        """Decode query position: the last local token."""
        return self.P0 + self.L_loc - 1

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def lognormal_doc_lengths(total_tokens: int, median: int, sigma: float, lo: int, hi: int,
                          seed: int) -> List[int]:
    """Document lengths drawn lognormally (median ``median``), clipped to
    [lo, hi], rounded up to whole 256-token chunks, until ``total_tokens``;
    the last document is cut so the lengths sum to exactly ``total_tokens``."""
    g = np.random.default_rng(seed)
    out, acc = [], 0
    while acc < total_tokens:
        x = float(np.clip(g.lognormal(math.log(median), sigma), lo, hi))
        L = int(math.ceil(x / CHUNK)) * CHUNK
        L = min(L, total_tokens - acc)
        out.append(L)
        acc += L
    return out


def workload(name: str) -> Workload:
    """The named workload: tiny_f32_64k, decode_1m, prefill_8m, host_100m,
    interleave_32m (full size) and their small siblings (*_small)."""
    if name == "tiny_f32_64k":
        return Workload("tiny_f32_64k", "f32", [1024] * 64, h_r=1, h_kv=2, h_q=8, k=4, B=1, L_loc=512,
                        pos0=1024, plant="pooled_key", seed=1001)
    if name == "decode_1m":
        return Workload("decode_1m", "bf16", [512] * 2048, h_r=8, h_kv=8, h_q=32, k=16, B=16,
                        L_loc=4096, plant="direction", plant_batches=4, seed=1002)
    if name == "prefill_8m":
        return Workload("prefill_8m", "bf16", [2048] * 4096, h_r=8, h_kv=8, h_q=32, k=16, B=2048,
                        L_loc=2048, mode="prefill", block=64, seed=1003)
    if name == "host_100m":
        return Workload("host_100m", "bf16", [8192] * 12207 + [256], h_r=8, h_kv=8, h_q=32, k=16, B=8,
                        L_loc=4096, keys_given=True, kv_host=True, host_slots=384, seed=1004)
    if name == "interleave_32m":
        lens = lognormal_doc_lengths(32 * 2 ** 20, 4096, 1.0, 1024, 65536, seed=1005)
        return Workload("interleave_32m", "bf16", lens, h_r=1, h_kv=8, h_q=32, k=8, B=64, L_loc=4096,
                        mode="interleave", hops=3, seed=1005)
    # small siblings: same structure, sizes the oracle finishes in seconds,
    # ragged local contexts
    if name == "tiny_f32_small":
        return Workload("tiny_f32_small", "f32", [1024] * 8, h_r=1, h_kv=2, h_q=8, k=4, B=2,
                        L_loc=77, pos0=1024, plant="pooled_key", seed=2001)
    if name == "decode_small":
        return Workload("decode_small", "bf16", [512] * 48, h_r=8, h_kv=8, h_q=32, k=4, B=3,
                        L_loc=300, plant="direction", seed=2002)
    if name == "prefill_small":
        return Workload("prefill_small", "bf16", [2048] * 12, h_r=8, h_kv=8, h_q=32, k=3, B=192,
                        L_loc=250, mode="prefill", block=64, seed=2003)
    if name == "host_small":
        return Workload("host_small", "bf16", [1024] * 23 + [256], h_r=8, h_kv=8, h_q=32, k=4,
                        B=2, L_loc=200, keys_given=True, kv_host=True, host_slots=5, seed=2004)
    if name == "interleave_small":
        lens = lognormal_doc_lengths(40 * 1024, 1024, 1.0, 256, 8192, seed=2005)
        return Workload("interleave_small", "bf16", lens, h_r=1, h_kv=8, h_q=32, k=3, B=4, L_loc=129,
                        mode="interleave", hops=3, seed=2005)
    raise KeyError(name)


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------
def array_seed(seed: int, name: str) -> int:
    return (int(seed) * 1_000_003 + zlib.crc32(name.encode())) % (2 ** 63)


def normal(shape, seed: int, name: str, device="cpu", dtype=torch.float32, std: float = 1.0):
    g = torch.Generator(device=device)
    g.manual_seed(array_seed(seed, name))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def integers(n: int, high: int, seed: int, name: str) -> np.ndarray:
    return np.random.default_rng(array_seed(seed, name)).integers(0, high, size=n)


def permutation(n: int, seed: int, name: str) -> np.ndarray:
    return np.random.default_rng(array_seed(seed, name)).permutation(n)


GEN_ELEMS = 1 << 24  # elements per independently seeded generation slice


def token_rows(w: Workload, what: str, width, t0: int, t1: int, device="cpu",
               dtype=None, std: float = 1.0, total: Optional[int] = None):
    """Rows [t0, t1) of a per-row array of shape [total, *width] (total
    defaults to the bank's token count), drawn in fixed slices of about
    GEN_ELEMS elements so that any row range is reproducible on its own."""
    dtype = w.torch_dtype if dtype is None else dtype
    width = tuple(width)
    total = w.T if total is None else int(total)
    per = max(1, GEN_ELEMS // int(np.prod(width)))
    parts = []
    s = t0 // per
    while s * per < t1:
        a, b = s * per, min((s + 1) * per, total)
        lo, hi = max(a, t0), min(b, t1)
        full = normal((b - a,) + width, w.seed, f"{what}/{s}", device, torch.float32, std)
        parts.append(full[lo - a:hi - a].to(dtype))
        del full
        s += 1
    return torch.cat(parts, 0) if len(parts) > 1 else parts[0]


def doc_token_offsets(w: Workload) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(w.doc_len, dtype=np.int64))])


def host_slot_layout(w: Workload):
    """Physical layout of a host-resident bank backed by w.host_slots document
    slots (a stand-in for a store too large for host memory: the bytes each
    step copies are those of the full bank, the contents repeat).  Documents
    of the longest length share the first slots round-robin; every shorter
    document has a slot of its own after them.

    Returns (slot_len [S] tokens, kv_off [n_docs] token offset of each
    document's slot)."""
    L = np.asarray(w.doc_len, dtype=np.int64)
    lmax = int(L.max())
    short = np.nonzero(L != lmax)[0]
    long_ids = np.nonzero(L == lmax)[0]
    n_long = int(w.host_slots) - len(short)
    if n_long < 1:
        raise ValueError("host_slots must exceed the number of shorter documents")
    slot_len = [lmax] * n_long + [int(L[n]) for n in short]
    starts = np.concatenate([[0], np.cumsum(np.asarray(slot_len, dtype=np.int64))])
    kv_off = np.empty(len(L), dtype=np.int64)
    kv_off[long_ids] = starts[np.arange(len(long_ids)) % n_long]
    kv_off[short] = starts[n_long + np.arange(len(short))]
    return slot_len, kv_off


def host_kv_raw(w: Workload, device="cpu", t0: int = 0, t1: Optional[int] = None):
    """Raw (pre-RoPE) K and V of the host slots' tokens [t0, t1) (token
    indices of the slot store), [t1 - t0, h_kv, d] each."""
    slot_len, _ = host_slot_layout(w)
    total = int(sum(slot_len))
    t1 = total if t1 is None else t1
    return (token_rows(w, "host_k", (w.h_kv, w.d), t0, t1, device, total=total),
            token_rows(w, "host_v", (w.h_kv, w.d), t0, t1, device, total=total))


def planted_targets(w: Workload, batch: int = 0):
    """For "direction" planting: query b's k target documents in query batch
    `batch` (< w.plant_batches; disjoint across every planted batch's
    queries) and, for each, the chunk inside it that carries the planted
    direction.  Returns (targets [B, k], chunk_in_doc [B, k])."""
    n = w.B * w.k
    perm = permutation(w.n_docs, w.seed, "targets")[batch * n:(batch + 1) * n].reshape(w.B, w.k)
    nch = np.asarray(w.doc_len)[perm] // CHUNK
    name = "target_chunk" if batch == 0 else f"target_chunk/{batch}"
    pick = integers(n, 1 << 30, w.seed, name).reshape(w.B, w.k) % nch
    return perm, pick


def route_vectors(w: Workload, device="cpu", t0: int = 0, t1: Optional[int] = None):
    """Per-token routing vectors [t1 - t0, h_r, d_r].  With "direction"
    planting, every row of query b's chosen chunk in each of its target
    documents gets strength * u_b added (u_b is the query's router vector,
    see ``route_queries``) before rounding."""
    t1 = w.T if t1 is None else t1
    r = token_rows(w, "route", (w.h_r, w.d_r), t0, t1, device, torch.float32)
    if w.plant == "direction":
        if w.plant_batches * w.B * w.k > w.n_docs:
            raise ValueError("planted targets must be disjoint: too few documents")
        off = doc_token_offsets(w)
        for i in range(w.plant_batches):
            tgt, pick = planted_targets(w, i)
            u = route_queries(w, device, batch=i)
            for b in range(w.B):
                for j in range(w.k):
                    s = int(off[tgt[b, j]] + pick[b, j] * CHUNK)
                    lo, hi = max(s, t0), min(s + CHUNK, t1)
                    if lo < hi:
                        r[lo - t0:hi - t0] += w.plant_strength * u[b]
    return r.to(w.torch_dtype)


def route_queries(w: Workload, device="cpu", batch: int = 0):
    """Decode router queries [B, h_r, d_r], float32, N(0, 1).  With
    "direction" planting, a batch below w.plant_batches is the planted
    directions themselves (its targets' chunks carry them); other batches
    are fresh draws.  ("pooled_key" planting needs the pooled key of the
    target chunk, which the caller supplies to ``pooled_key_query``.)"""
    name = "route_query" if batch == 0 else f"route_query/{batch}"
    return normal((w.B, w.h_r, w.d_r), w.seed, name, device)


def pooled_key_target(w: Workload):
    """For "pooled_key" planting: (target document, chunk index in the bank)."""
    doc = int(integers(1, w.n_docs, w.seed, "pk_doc")[0])
    off = np.concatenate([[0], np.cumsum(np.asarray(w.doc_len) // CHUNK)])
    ch = int(off[doc] + integers(1, w.doc_len[doc] // CHUNK, w.seed, "pk_chunk")[0])
    return doc, ch


def pooled_key_query(w: Workload, key, device="cpu"):
    """Router query = a given pooled key [h_r, d_r] plus N(0, 0.1^2) noise,
    for every query of the batch (each its own noise)."""
    noise = normal((w.B, w.h_r, w.d_r), w.seed, "pk_noise", device, std=0.1)
    return (torch.as_tensor(key, dtype=torch.float32, device=device)[None] + noise).float()


def kv_raw(w: Workload, device="cpu", t0: int = 0, t1: Optional[int] = None):
    """Raw (pre-RoPE) document K and V, [t1 - t0, h_kv, d] each."""
    t1 = w.T if t1 is None else t1
    return (token_rows(w, "k", (w.h_kv, w.d), t0, t1, device),
            token_rows(w, "v", (w.h_kv, w.d), t0, t1, device))


def keys_direct(w: Workload, device="cpu"):
    """Routing keys drawn directly, [C, h_r, d_r]: N(0, 1/256) per element,
    the distribution of a mean of 256 N(0, 1) rows."""
    return token_rows(w, "keys", (w.h_r, w.d_r), 0, w.C, device, std=1.0 / 16.0, total=w.C)


def local_raw(w: Workload, device="cpu", batch: int = 0):
    """Raw local-context K and V.  decode/interleave: [B, L_loc, h_kv, d];
    prefill: [L_loc, h_kv, d] (the prefill tokens are its last B tokens)."""
    sfx = "" if batch == 0 else f"/{batch}"
    shape = (w.L_loc, w.h_kv, w.d) if w.mode == "prefill" else (w.B, w.L_loc, w.h_kv, w.d)
    return (normal(shape, w.seed, "local_k" + sfx, device).to(w.torch_dtype),
            normal(shape, w.seed, "local_v" + sfx, device).to(w.torch_dtype))


def queries(w: Workload, device="cpu", batch: int = 0):
    """Raw (pre-RoPE) attention queries [B, h_q, d]."""
    sfx = "" if batch == 0 else f"/{batch}"
    return normal((w.B, w.h_q, w.d), w.seed, "q" + sfx, device).to(w.torch_dtype)


def prefill_route_tokens(w: Workload, device="cpu"):
    """Per-token router vectors of the prefill queries [B, h_r, d_r]."""
    return normal((w.B, w.h_r, w.d_r), w.seed, "prefill_route", device).to(w.torch_dtype)


def interleave_projection(w: Workload, device="cpu"):
    """Fixed projection [d_r, h_q * d], N(0, 1/(h_q * d)), float32."""
    n = w.h_q * w.d
    return normal((w.d_r, n), w.seed, "w_proj", device, std=1.0 / math.sqrt(n))
