/*
 * msa.h -- C ABI of libmsa.so, the MI355X (gfx950) hot path of Memory Sparse
 * Attention (MSA).
 *
 * The method (sources are web pages; each call cites the passage that
 * defines what it computes):
 *   - "MSA架构：突破大模型记忆瓶颈的稀疏注意力技术" (intelliparadigm.com),
 *     sections 2.1 and 3.1: a router picks documents by cosine top-k over
 *     routing keys made by 256-token chunk-mean pooling.
 *   - "MSA" card (robocikowo.com), sections "Komponenty", "Pułapki
 *     implementacyjne", "Równoległość": the MSA layer appends the top-k
 *     documents' K/V to the local context; document-wise RoPE restarts
 *     positions at every document, global RoPE with an offset covers the
 *     active context; routing keys live in GPU memory and full K/V may live
 *     in host memory (pinned, copied asynchronously); top-k and the
 *     following K/V fetch are sequential within a decode step; Memory
 *     Interleave alternates document selection and context expansion.
 *   - the MLA/CSA attention article (mlqm.cn), section 6.2: 1/sqrt(d) scale.
 *
 * Conventions for every call
 *   - Every pointer is caller-owned.  "device" pointers are HIP device
 *     memory on the current device; "host" pointers are ordinary CPU memory.
 *     The library allocates only in msa_bank_create (small per-bank tables;
 *     for a host-resident bank also pinned id buffers for 4096 selections and
 *     65 events) and frees them in msa_bank_destroy.  The one exception on
 *     the hot path: msa_step or msa_prefetch on a host-resident bank regrows
 *     those pinned id buffers once when a call selects more documents than
 *     they hold.
 *   - A host-resident K/V store (MSA_KV_HOST) must be pinned host memory
 *     (hipHostMalloc, or torch's pin_memory) over its whole extent;
 *     msa_bank_create refuses pageable memory with MSA_EINVAL.
 *   - Every data array (device, or pinned host for a host-resident store)
 *     starts on a 16-byte boundary, as hipMalloc, hipHostMalloc and torch
 *     allocations do; a misaligned array is MSA_EINVAL.
 *   - msa_bank_create, msa_build_bank and msa_prepare_local check each
 *     device array they are given against the allocation that holds it
 *     (hipMemGetAddressRange): an array that would end past its allocation
 *     for the shape the call implies is MSA_EINVAL, nothing launched.  Memory
 *     the runtime cannot place (another allocator's) is not checked; an
 *     array carved from a larger allocation passes if it ends inside it.
 *   - No call records a memset: the library clears device memory with a
 *     kernel, so the kernel launches of a device-bank call can be captured
 *     into a HIP graph (a host-resident bank's msa_step synchronises and
 *     cannot).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls are asynchronous on that stream unless stated; results are valid
 *     once the stream has completed the work.
 *   - Return value: msa_status.  Argument and shape errors are detected on
 *     the host before anything is launched (MSA_EINVAL / MSA_EUNSUPPORTED,
 *     nothing written).  A failed HIP launch or copy returns MSA_EHIP.
 *     msa_last_error() gives a human-readable reason for the last failure
 *     on the calling thread.
 *   - An empty batch (B or n_q = 0) is a valid call that launches nothing;
 *     its data pointers may then be NULL.
 *   - Head size d and routing-key size d_r are 128.  Routing chunks are 256
 *     tokens; every document length is a positive multiple of 256.
 *   - dtype: MSA_F32 or MSA_BF16, the storage type of routing keys, document
 *     K/V, local K/V and attention queries.  Router queries and attention
 *     outputs are always float32.  Arithmetic accumulates in float32 (the
 *     routing-key pooling and norms in float64).
 *   - A bank handle is immutable after msa_bank_create; calls on one bank may
 *     run concurrently on different streams if their workspaces (and staging
 *     buffers) differ.  On a host-resident bank the host part of msa_step
 *     (id readback, copy issue) runs one call at a time under a lock held in
 *     the bank.
 *
 * Layouts (row-major; the last index is contiguous)
 *   Routing keys      kr       [h_r][C_cap][d_r]    (C = total chunks in use,
 *                                                    C_cap >= C the capacity)
 *   Key norms         inv_norm [h_r][C_cap] float32 (1/||key||, 0 for a zero key)
 *   Document K store  per document n at token offset kv_off[n]:
 *                     k_store + kv_off[n]*h_kv*d  ->  [h_kv][L_n][d]
 *                     (rotated at document-local positions 0..L_n-1)
 *   Document V store  v_store + kv_off[n]*h_kv*d  ->  [h_kv][L_n/64][d][64]
 *                     (tile-blocked: each 64-token tile is stored channel-major,
 *                     one contiguous 16 KiB block per head in bf16)
 *   Local K           [n_seq][h_kv][L][d]            (rotated at pos0 + j)
 *   Local V           [n_seq][h_kv][ceil(L/64)][d][64]  (tile-blocked, tokens past
 *                     L in the last tile are zero)
 *   Raw per-token inputs (what a model emits): [tokens][heads][128].
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_EINVAL = 1,        /* bad argument, shape or pointer */
  MSA_ENOMEM = 2,        /* workspace/staging too small, or bank tables could not be allocated */
  MSA_EHIP = 3,          /* a HIP launch, copy or synchronisation failed */
  MSA_EUNSUPPORTED = 4   /* valid request outside what this build supports */
} msa_status;

typedef enum { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype;
typedef enum { MSA_KV_DEVICE = 0, MSA_KV_HOST = 1 } msa_kv_loc;
typedef enum { MSA_DECODE = 0, MSA_PREFILL = 1 } msa_mode;
/* What the attention reads of each selected document: its per-token K/V,
 * or its compressed memory (one log-weighted entry per 256-token chunk, see
 * msa_bank_set_pooled). */
typedef enum { MSA_MEMORY_TOKENS = 0, MSA_MEMORY_POOLED = 1 } msa_memory;

typedef struct msa_bank msa_bank;

/* Description of a memory bank ("MSA" card, robocikowo.com, "Komponenty":
 * the KV-cache memory store keeps the routing keys Kr in GPU memory and the
 * full K/V of every document, possibly in CPU memory). */
typedef struct {
  msa_dtype dtype;
  int32_t n_docs;            /* N >= 1 */
  const int64_t* doc_len;    /* host [N]: tokens per document, > 0, % 256 == 0 */
  const int64_t* kv_off;     /* host [N] or NULL: token offset of each document in the
                                K/V stores (NULL = documents packed in order).  Several
                                documents may share storage. */
  int64_t kv_tokens;         /* tokens the K/V stores hold: >= max(kv_off[n] + doc_len[n]) */
  int32_t h_r;               /* router heads, 1..16 */
  int32_t d_r;               /* 128 */
  int32_t h_kv;              /* KV heads, 1..64 */
  int32_t d;                 /* 128 */
  double rope_base;          /* RoPE base (10000) */
  msa_kv_loc kv_loc;         /* where k_store / v_store live */
  void* kr;                  /* device [h_r][C_cap][d_r], dtype (rows [0, C) in use) */
  float* inv_norm;           /* device [h_r][C_cap] */
  void* k_store;             /* device or pinned host, kv_tokens*h_kv*d elements */
  void* v_store;             /* device or pinned host, kv_tokens*h_kv*d elements */
  int64_t chunk_cap;         /* C_cap, routing-key rows per head the kr / inv_norm
                                allocations hold (room for msa_bank_append);
                                0 = exactly the chunks of the initial documents */
} msa_bank_desc;

typedef struct {
  int64_t n_chunks;          /* C */
  int64_t n_tokens;          /* sum of doc_len */
  int64_t max_doc_len;
  int32_t n_docs;
  int32_t n_pieces;          /* routing partial slots per (query, head) */
} msa_bank_info;

/* Per-call knobs of the attention kernels. */
typedef struct {
  int32_t mode;              /* MSA_DECODE or MSA_PREFILL */
  int32_t n_q;               /* decode: queries B; prefill: query tokens L_q */
  int32_t h_q;               /* query heads, a multiple of h_kv with h_q/h_kv in {1,2,4,8} */
  const void* q;             /* device [n_q][h_q][d], dtype, before RoPE */
  int32_t q_pos;             /* decode: position of every query;
                                prefill: position of query 0 (query i at q_pos + i) */
  const int32_t* ids;        /* device [n_groups][k]: selected document ids (or source ids
                                when src_len is set); ids outside [0, N) (resp. [0, n_src))
                                are skipped, so -1 marks an empty slot.
                                decode: n_groups = n_q; prefill: n_groups = n_q / block */
  int32_t k;                 /* documents per group, >= 0 */
  int32_t block;             /* prefill: queries per routing group (n_q % block == 0) */
  const void* k_loc;         /* device local K [n_seq][h_kv][L_loc][d] (prepared) */
  const void* v_loc;         /* device local V [n_seq][h_kv][ceil(L_loc/64)][d][64] (prepared) */
  int32_t L_loc;             /* local tokens, >= 0 (decode: n_seq = n_q; prefill: n_seq = 1) */
  float* out;                /* device [n_q][h_q][d] float32 */
  void* ws;                  /* device workspace */
  size_t ws_bytes;
  int32_t splits;            /* decode: work splits per (query, KV head); 0 = automatic */
  /* Optional source override (host-resident banks copy selected documents
   * into a staging area; ids then index this table).  All NULL = the bank. */
  const void* src_k;         /* device K store of the sources, layout as the bank's */
  const void* src_v;         /* device V store of the sources */
  const int64_t* src_off;    /* device [n_src] token offsets */
  const int32_t* src_len;    /* device [n_src] token lengths */
  int32_t n_src;             /* entries in src_off / src_len */
  int32_t memory;            /* msa_memory: MSA_MEMORY_TOKENS, or MSA_MEMORY_POOLED (decode) */
} msa_attend_args;

/* One step of the path: route -> top-k -> gather -> attend, repeated for
 * `hops` hops (Memory Interleave). */
typedef struct {
  int32_t mode;              /* MSA_DECODE or MSA_PREFILL */
  int32_t n_q;               /* decode: B; prefill: L_q */
  int32_t h_q;
  int32_t k;                 /* top-k documents, 1 <= k <= N */
  const void* q;             /* device [n_q][h_q][d] dtype, before RoPE */
  int32_t q_pos;             /* as in msa_attend_args */
  const float* q_route;      /* decode: device [n_q][h_r][d_r] float32, hop-1 router query */
  const void* route_tokens;  /* prefill: device [n_q][h_r][d_r] dtype per-token router vectors */
  int32_t block;             /* prefill routing block (64) */
  const void* k_loc;         /* prepared local context, as in msa_attend_args */
  const void* v_loc;
  int32_t L_loc;
  int32_t hops;              /* >= 1; > 1 needs h_r == 1 and w_proj (decode only) */
  const float* w_proj;       /* device [d_r][h_q*d] float32: next hop's router query is
                                w_proj times the concatenated per-head outputs */
  int32_t exclude_selected;  /* nonzero: documents selected in earlier hops are excluded */
  uint32_t* exclude;         /* device [n_groups][ceil(N/32)] bit mask of excluded documents
                                (bit n%32 of word n/32), or NULL.  With exclude_selected the
                                call ORs each hop's selections into it. */
  int32_t* ids;              /* device [hops][n_groups][k] */
  float* scores;             /* device [hops][n_groups][k] */
  float* out;                /* device [hops][n_q][h_q][d] float32 */
  void* ws;
  size_t ws_bytes;
  void* staging;             /* host banks: device staging for copied documents */
  size_t staging_bytes;
  int32_t splits;
  int32_t memory;            /* msa_memory, as in msa_attend_args; pooled memory needs no
                                host->device copies, so staging is unused */
} msa_step_args;

typedef struct {
  int64_t docs_copied;       /* host banks: distinct documents copied host->device */
  int64_t bytes_copied;      /* host banks: bytes copied host->device */
  int64_t docs_cached;       /* host banks with a device cache: distinct selected
                                documents found in the cache (no copy) */
} msa_step_stats;

const char* msa_status_string(int status);
const char* msa_last_error(void);
int msa_version(void);

/* Validate `desc`, build the bank's routing tables (document and chunk
 * offsets, the chunk->document map, RoPE frequencies) and upload them.
 * Does not touch kr / inv_norm / the K/V stores.  Synchronous. */
int msa_bank_create(const msa_bank_desc* desc, msa_bank** out);
int msa_bank_destroy(msa_bank* bank);

/* Incremental bank growth ("MSA" card, "Pułapki implementacyjne": the memory
 * bank is built ahead of inference; new documents join it without rebuilding
 * the rest).  Appends n_new documents after the current ones (ids N ..
 * N + n_new - 1): doc_len (host, each a positive multiple of 256) and
 * kv_off (host, or NULL = packed after the current tokens) as in the
 * descriptor.  The routing-key and K/V allocations must already hold them
 * (chunk_cap, kv_tokens), else MSA_EINVAL.  Their keys and K/V are then
 * written by msa_build_bank(bank, N, N + n_new, ...) (a device-resident
 * store) or by the caller (a host-resident store).  Workspace and staging
 * sizes may grow: query them again.  A document longer than an attached
 * cache's slots is refused (detach the cache first).  Not to be called
 * concurrently with other calls on this bank.  Synchronous. */
int msa_bank_append(msa_bank* bank, int32_t n_new, const int64_t* doc_len,
                    const int64_t* kv_off);
int msa_bank_get_info(const msa_bank* bank, msa_bank_info* info);

/* Offline bank build for documents [doc_begin, doc_end) ("MSA" card,
 * robocikowo.com, "Pułapki implementacyjne", cold start: encode documents
 * ahead of time, store routing keys and K/V, pool by chunk means).
 *   route_vec: device [T_s][h_r][d_r] dtype, the per-token routing vectors of
 *     those documents in order (T_s = their total length).  Writes kr rows
 *     as the mean of each 256-token chunk (intelliparadigm.com, section 3.1),
 *     rounded to dtype, and inv_norm from the rounded keys.  NULL: kr is
 *     taken as given and only inv_norm of those chunks is computed.
 *   k_raw, v_raw: device [T_s][h_kv][d] dtype, or both NULL.  K is rotated at
 *     document-local positions (document-wise RoPE, "MSA" card,
 *     "Komponenty") and both are written into the device K/V stores in the
 *     layouts above.  Host-resident stores are not written (MSA_EUNSUPPORTED).
 */
int msa_build_bank(const msa_bank* bank, int32_t doc_begin, int32_t doc_end,
                   const void* route_vec, const void* k_raw, const void* v_raw, void* stream);

/* Local (active) context: rotate raw K at global positions pos0 + j ("MSA"
 * card, "Pułapki implementacyjne": global RoPE with an offset for the
 * active context) and lay K and V out for the attention kernels.
 *   k_raw, v_raw: device [n_seq][L][h_kv][d] dtype.
 *   k_loc: device [n_seq][h_kv][L][d];
 *   v_loc: device [n_seq][h_kv][ceil(L/64)][d][64], tokens past L zero-filled. */
int msa_prepare_local(const msa_bank* bank, const void* k_raw, const void* v_raw,
                      int32_t n_seq, int32_t L, int32_t pos0,
                      void* k_loc, void* v_loc, void* stream);

/* Workspace bytes msa_route / msa_attend / msa_step need for these sizes.
 * mode: MSA_DECODE or MSA_PREFILL; n_q, h_q, k as in the args; hops >= 1. */
size_t msa_workspace_bytes(const msa_bank* bank, int32_t mode, int32_t n_q, int32_t h_q,
                           int32_t k, int32_t block, int32_t hops, int32_t splits);

/* Staging bytes msa_step needs for a host-resident bank. */
size_t msa_staging_bytes(const msa_bank* bank, int32_t n_groups, int32_t k);

/* Routing ("MSA" card, "Komponenty", router; intelliparadigm.com, 2.1):
 *   cos[b,h,c] = q_route[b,h] . kr[h,c] * inv_norm[h,c] / ||q_route[b,h]||
 *   score[b,n] = mean over h of max over document n's chunks of cos
 * then the k best documents per query, ordered by score (descending) with
 * ties to the lower id.  Excluded documents (bit set in `exclude`, may be
 * NULL) are never chosen; if fewer than k remain, the tail is id -1, score
 * -inf.
 *   q_route: device [B][h_r][d_r] float32.  ids: device [B][k] int32;
 *   scores: device [B][k] float32 (the document scores).  1 <= k <= N. */
int msa_route(const msa_bank* bank, const float* q_route, int32_t B, int32_t k,
              const uint32_t* exclude, int32_t* ids, float* scores,
              void* ws, size_t ws_bytes, void* stream);

/* GQA softmax attention of each query over the union of its selected
 * documents' K/V (rank order) and the local context ("MSA" card,
 * "Komponenty", the MSA layer; "Paradygmat wykonania": only the selected
 * blocks take part), scale 1/sqrt(d) (mlqm.cn article, 6.2).  Query head
 * hq reads KV head hq / (h_q/h_kv).  Queries are rotated at their global
 * positions.  Decode: each query sees all L_loc local tokens.  Prefill:
 * query i of group g = i / block sees group g's documents and local tokens
 * j <= L_loc - n_q + i (the queries are the last n_q local tokens).  A
 * query with no key at all (every id slot empty and L_loc = 0) gets 0. */
int msa_attend(const msa_bank* bank, const msa_attend_args* args, void* stream);

/* Compressed memory (intelliparadigm.com, section 3.1: chunk-mean pooling
 * as KV-cache compression; "MSA" card, "Komponenty": a compressed memory
 * bank).  Each 256-token chunk of a document becomes one entry: the mean of
 * its stored (document-RoPE'd) K and the mean of its V, rounded to dtype.
 * With memory = MSA_MEMORY_POOLED a decode attends over its selected
 * documents' entries -- each scored with an extra ln 256, the log of the 256
 * tokens it stands for -- followed by the local context's tokens.
 *   msa_pooled_sizes: elements (of dtype) the two pooled stores hold.
 *   msa_bank_set_pooled: attach caller-owned device stores (NULL detaches):
 *     pool_k per document n at entry chunk_first(n): [h_kv][P_n][d]
 *     (P_n = doc_len[n] / 256); pool_v per document [h_kv][ceil(P_n/64)][d][64]
 *     (tile-blocked, zero-padded) at the running sum of 64-padded P.
 *     msa_bank_append detaches them (sizes grow).
 *   msa_build_pooled: fill the pooled stores of documents [doc0, doc1) from
 *     the bank's device K/V stores (device-resident banks).  Asynchronous. */
int msa_pooled_sizes(const msa_bank* bank, int64_t* k_elems, int64_t* v_elems);
int msa_bank_set_pooled(msa_bank* bank, void* pool_k, void* pool_v);
int msa_build_pooled(const msa_bank* bank, int32_t doc_begin, int32_t doc_end, void* stream);

/* Device (HBM) document cache of a host-resident bank (intelliparadigm.com,
 * section 5.2: keep frequently used memory in HBM; "MSA" card, "Pułapki
 * implementacyjne": the CPU-GPU link is the bottleneck of large banks).
 *   cache: device memory the caller owns (NULL detaches), cache_bytes of it,
 *     divided into n = cache_bytes / msa_cache_slot_bytes() slots, each
 *     holding one document's K and V in the store layouts: slot s's K at
 *     s * S and its V at n * S + s * S, with S = msa_cache_slot_bytes() / 2.
 * While a cache is attached, msa_step keeps recently selected documents
 * resident: a selected document already in a slot is read from there, any
 * other is copied from the host store into the least recently used slot
 * that the same hop does not need (its `staging` is then unused and may be
 * NULL).  A copy into a slot waits, on the copy stream, for the last
 * attention that read the slot and for its previous fill; an attention
 * waits for the fills of the slots it reads.  Results are identical with and
 * without a cache.
 * Errors: MSA_EINVAL for a device-resident bank; MSA_ENOMEM if no slot
 * fits; msa_step fails with MSA_ENOMEM when one hop selects more distinct
 * documents than there are slots.  Resets the cache's contents; not to be
 * called while an msa_step on this bank is running.  Synchronous. */
int msa_bank_set_cache(msa_bank* bank, void* cache, size_t cache_bytes);
size_t msa_cache_slot_bytes(const msa_bank* bank);

/* Route + top-k + gather + attend for one batch, `hops` times ("MSA" card,
 * "Równoległość": top-k then K/V fetch, sequential in each decode step;
 * "Komponenty": Memory Interleave).  Prefill: each block of `block` query
 * tokens routes with the mean of its router vectors and shares one top-k set.
 * Host-resident banks: after top-k the ids are read back (the call blocks
 * once per hop on `stream`, i.e. until the stream's earlier work is done),
 * each distinct selected document is copied into `staging` -- or, with a
 * device cache attached, found in the cache or copied into a cache slot --
 * on `copy_stream` (NULL = `stream`), and attention waits, on the device,
 * for the copies it reads (including a cached document's copy that an
 * earlier call or msa_prefetch left in flight).  A document copied into a
 * cache slot has its K copied on `copy_stream` and its V on a second copy
 * stream the bank owns (created with a host-resident bank, default
 * priority), which starts after the work already on `copy_stream` and which
 * `copy_stream` waits for after the call's last copy: seen from
 * `copy_stream`, every copy of the call is on it, and two copies in flight
 * keep the link busy through each copy's start-up.  Copies into `staging`
 * all run on `copy_stream`.  The call returns once the attention is
 * enqueued; `staging` may be reused by the next call on the same `stream`.
 * `stats` (host, may be NULL) receives copy and cache-hit counts. */
int msa_step(const msa_bank* bank, const msa_step_args* args, void* stream,
             void* copy_stream, msa_step_stats* stats);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): msa_step
 * on a device-resident bank with its workspace taken from scratch memory the
 * library holds on each device -- a 64 MiB device-code array, created with
 * the library's code on that device and kept until the process ends.
 * args->ws and args->ws_bytes are not read (staging and the copy stream do
 * not apply to a device-resident bank).  Nothing is allocated.  Every call
 * on one device shares that device's scratch, which keeps the last call's
 * contents (the call clears what must start at zero, the exclusion bitmap
 * of a multi-hop step): calls that overlap in time on one device race, so
 * issue them on one stream or order them.
 * Errors: as msa_step; MSA_ENOMEM (nothing launched) when the request needs
 * more workspace than the scratch holds (msa_workspace_bytes with the
 * splits it resolves to: a 16-query decode of a 1M-token bank needs about
 * 2.4 MB, an 8M-token 2048-token prefill about 36 MB); MSA_EUNSUPPORTED on a
 * host-resident bank. */
int msa_step_static(const msa_bank* bank, const msa_step_args* args, void* stream);

/* Asynchronous prefetch into the device cache of a host-resident bank
 * (intelliparadigm.com, section 5.2: prefetch memory ahead of its use so that
 * IO overlaps compute, over a window of upcoming requests; "MSA" card,
 * "Pułapki implementacyjne": pinned memory and asynchronous copies against
 * the CPU-GPU bandwidth bottleneck).  Routes B router queries exactly as
 * msa_route does (q_route: device [B][h_r][d_r] float32; exclude as there),
 * on `stream`, reads the selection back (blocking once on `stream`), and
 * makes every distinct selected document resident: a document already in
 * the cache is marked recently used, any other is copied into the least
 * recently used slot on `copy_stream` (NULL = `stream`; V copies on the
 * bank's second copy stream, joined back as in msa_step).  The copies are
 * left in flight: a later msa_step that selects these documents finds them
 * in the cache and its attention waits for them on the device.  Running
 * route + prefetch for batch i + W while batch i steps keeps the host link
 * busy without gaps.
 *   ws: device workspace of at least msa_workspace_bytes(bank, MSA_DECODE,
 *     B, h_kv, k, 1, 1, 0) bytes (must not be in use by another call).
 *   stats (host, may be NULL): copies issued and documents already cached.
 * Errors: MSA_EINVAL without an attached cache or on a device-resident bank;
 * MSA_ENOMEM when the selection has more distinct documents than the cache
 * has slots; k and B as in msa_route. */
int msa_prefetch(const msa_bank* bank, const float* q_route, int32_t B, int32_t k,
                 const uint32_t* exclude, void* ws, size_t ws_bytes, void* stream,
                 void* copy_stream, msa_step_stats* stats);

/* Kernel timing for measurement.  While enabled on the calling thread, the
 * library brackets launches of the kernel class `which` with a pair of HIP
 * events on the stream it launches on: every `period`-th launch of each
 * class, counted from the enabling call (period 1 = every launch; a larger
 * period keeps the events' own cost on the stream small).  msa_timer_read
 * synchronises those events, returns the accumulated milliseconds and the
 * number of bracketed launches since the last read, and clears them.
 *   which: MSA_TIMER_ATTENTION (decode or prefill attention kernel),
 *          MSA_TIMER_ROUTE (routing scan: the scan launches of one call,
 *          as one interval).
 *   period: <= 0 disables the timer. */
enum { MSA_TIMER_ATTENTION = 0, MSA_TIMER_ROUTE = 1 };
int msa_timer_enable(int period);
int msa_timer_read(int which, double* total_ms, int64_t* launches);
/* Create the events for `launches` timed launches ahead of a timed region
 * (events are otherwise created on first use, on the host, inside it).
 * Synchronous; MSA_EINVAL if launches < 0, MSA_EHIP if HIP cannot create
 * an event. */
int msa_timer_reserve(int64_t launches);

/* HBM read-rate probe, for measurement: streams `bytes` of the device buffer
 * `buf` once (every byte read, nothing else touched) on `stream`, so that
 * the rate a kernel which only reads can reach on this device can be timed
 * by the caller and set beside the datasheet's peak.  `buf`: device, 16-byte
 * aligned; `bytes`: a positive multiple of 16; `out`: device array of
 * MSA_STREAM_READ_BLOCKS uint32 words that receives a checksum per
 * workgroup (its only purpose is to keep every load).  Asynchronous;
 * MSA_EINVAL on a null pointer, misalignment or a bad size, MSA_EHIP if the
 * launch fails.  Buffers are the caller's. */
enum { MSA_STREAM_READ_BLOCKS = 4096 };
int msa_stream_read(const void* buf, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
