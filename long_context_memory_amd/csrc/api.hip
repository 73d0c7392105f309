// C ABI entry points: argument validation, bank tables, workspace layout and
// the orchestration of msa_step (route -> top-k -> gather -> attend, hops,
// host-resident banks).  See include/msa.h for the contract of each call.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "msa_internal.h"

namespace msa {

static thread_local std::string g_last_error;
void set_error(const std::string& msg) { g_last_error = msg; }

// ---- kernel timing (measurement only; off by default)
struct TimerState {
  bool on = false;
  int64_t period = 1;         // bracket every period-th launch of a class
  int64_t seq[2] = {0, 0};    // launches of each class since enabling
  bool skipping[2] = {false, false};  // the open launch is not bracketed
  std::vector<std::pair<hipEvent_t, hipEvent_t>> done[2];
  std::vector<hipEvent_t> pool;
  hipEvent_t open[2] = {nullptr, nullptr};
};
static thread_local TimerState g_timer;

static hipEvent_t timer_event() {
  if (!g_timer.pool.empty()) {
    hipEvent_t e = g_timer.pool.back();
    g_timer.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void timer_mark(int which, bool begin, hipStream_t s) {
  if (!g_timer.on || which < 0 || which > 1) return;
  if (begin) g_timer.skipping[which] = g_timer.seq[which]++ % g_timer.period != 0;
  if (g_timer.skipping[which]) return;
  hipEvent_t e = timer_event();
  if (!e) return;
  (void)hipEventRecord(e, s);
  if (begin) {
    g_timer.open[which] = e;
  } else if (g_timer.open[which]) {
    g_timer.done[which].emplace_back(g_timer.open[which], e);
    g_timer.open[which] = nullptr;
  }
}

namespace {

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

#define MSA_CHECK_HIP(expr)                                                          \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess)                                                            \
      return fail(MSA_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_));      \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// The kernels move 16-byte vectors: every data array starts on a 16-byte
// boundary (NULL passes; its own check comes first)
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
template <typename... P>
bool all_al16(P... p) {
  return (al16(p) && ...);
}

// Workspace layout shared by msa_workspace_bytes and the entry points.
struct WsLayout {
  size_t piecemax = 0, keys = 0, route_end = 0, qroute = 0, qrot = 0, part = 0, srcids = 0, srcoff = 0,
         srclen = 0, excl = 0, total = 0;
};

WsLayout ws_layout(const Bank& bk, int mode, int n_q, int h_q, int k, int block, int hops,
                   int splits) {
  WsLayout L;
  const int n_groups = mode == MSA_PREFILL ? n_q / std::max(block, 1) : n_q;
  const size_t esz = dtype_size(bk.desc.dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.piecemax = take((size_t)bk.desc.h_r * bk.n_pieces * n_groups * sizeof(float));
  L.keys = take((size_t)n_groups * topk_scratch_keys(bk.desc.n_docs, std::max(k, 1)) *
                sizeof(uint64_t));
  L.route_end = off;  // msa_route uses the workspace up to here
  L.qroute = take((size_t)n_groups * bk.desc.h_r * kD * sizeof(float));
  L.qrot = take((size_t)n_q * h_q * kD * esz);
  const int G = std::max(1, h_q / bk.desc.h_kv);
  L.part = take(decode_partial_floats(n_q, bk.desc.h_kv, G, splits) * sizeof(float));
  L.srcids = take((size_t)n_groups * k * sizeof(int32_t));
  L.srcoff = take((size_t)n_groups * k * sizeof(int64_t));
  L.srclen = take((size_t)n_groups * k * sizeof(int32_t));
  L.excl = take((size_t)n_groups * ((bk.desc.n_docs + 31) / 32) * sizeof(uint32_t));
  (void)hops;
  L.total = off;
  return L;
}

constexpr int kMaxSplits = 256;

// Splits of the attention kernels: the MFMA prefill takes any count, the
// split-K decode kernel (and the vector prefill) multiples of 4.
int resolve_splits(const Bank& bk, int mode, int splits, int n_q, int h_q, int block, int k,
                   int L_loc, bool pooled = false) {
  if (mode == MSA_PREFILL && prefill_mfma_supported(bk, n_q, h_q, block))
    return splits > 0 ? splits : prefill_auto_splits(bk, n_q, k, L_loc);
  if (splits > 0) return ((splits + 3) / 4) * 4;
  const double avg_doc = (double)bk.n_tokens / bk.desc.n_docs;
  // expected 64-entry tiles per selected document
  const double doc_tiles = pooled ? std::ceil(avg_doc / kChunk / kAttnTile) : avg_doc / kAttnTile;
  int s = decode_auto_splits(bk, n_q, k, L_loc, doc_tiles);
  if (pooled) {
    // compressed unions are short and mostly ragged tiles (a document's few
    // entries fill one tile): about 5 tiles per wave, which also gives two
    // waves per SIMD, measured best on the 1M-token bank on a single stream
    // (61 us per launch against 72 us at the per-token rule's 8 splits; two
    // streams' overlapping launches hide the difference)
    const double tiles = k * doc_tiles + (L_loc + kAttnTile - 1) / kAttnTile;
    const int t5 = (int)std::min(tiles, std::ceil(tiles / 5.0));
    s = std::min(kMaxSplits, std::max(s, ((t5 + 3) / 4) * 4));
  }
  return s;
}

// The compressed-memory sources: pooled entries, 64-padded V, ln 256 each
AttnSources pooled_sources(const Bank& bk) {
  AttnSources src{bk.pool_k, bk.pool_v, bk.d_pool_off, bk.d_pool_len, bk.desc.n_docs};
  src.voff = bk.d_pool_voff;
  src.bias = 8.0f;  // log2(256): scores are in log2 units
  return src;
}

const Bank* as_bank(const msa_bank* b) { return reinterpret_cast<const Bank*>(b); }

int check_attend_common(const Bank& bk, int mode, int n_q, int h_q, int k, int block, int L_loc,
                        const void* k_loc, const void* v_loc) {
  if (mode != MSA_DECODE && mode != MSA_PREFILL) return fail(MSA_EINVAL, "mode");
  if (n_q < 0) return fail(MSA_EINVAL, "n_q < 0");
  if (h_q <= 0 || h_q % bk.desc.h_kv) return fail(MSA_EINVAL, "h_q must be a multiple of h_kv");
  const int G = h_q / bk.desc.h_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(MSA_EUNSUPPORTED, "h_q / h_kv must be 1, 2, 4 or 8");
  if (k < 0 || k > kMaxK) return fail(MSA_EUNSUPPORTED, "k must be in [0, 64]");
  if (mode == MSA_PREFILL && (block <= 0 || n_q % block))
    return fail(MSA_EINVAL, "prefill: n_q must be a positive multiple of block");
  if (L_loc < 0) return fail(MSA_EINVAL, "L_loc < 0");
  // (an empty batch reads nothing: its local K/V may be NULL)
  if (L_loc > 0 && n_q > 0 && (!k_loc || !v_loc))
    return fail(MSA_EINVAL, "local K/V pointers are NULL");
  if (!all_al16(k_loc, v_loc)) return fail(MSA_EINVAL, "local K/V must be 16-byte aligned");
  if (mode == MSA_PREFILL && L_loc < n_q)
    return fail(MSA_EINVAL, "prefill: the queries are the last n_q local tokens (L_loc >= n_q)");
  return MSA_OK;
}

}  // namespace

hipError_t host_buffers_reserve(Bank& bk, size_t cap) {
  if (bk.h_ids_cap >= cap) return hipSuccess;
  if (bk.h_ids) (void)hipHostFree(bk.h_ids);
  if (bk.h_src) (void)hipHostFree(bk.h_src);
  if (bk.h_src_off) (void)hipHostFree(bk.h_src_off);
  bk.h_ids = nullptr;
  bk.h_src = nullptr;
  bk.h_src_off = nullptr;
  bk.h_ids_cap = 0;
  hipError_t e = hipHostMalloc((void**)&bk.h_ids, cap * 4, 0);
  if (e == hipSuccess) e = hipHostMalloc((void**)&bk.h_src, cap * 8, 0);
  if (e == hipSuccess) e = hipHostMalloc((void**)&bk.h_src_off, cap * 8, 0);
  if (e == hipSuccess) bk.h_ids_cap = cap;
  return e;
}

// initial capacity of a host-resident bank's pinned id buffers (selections
// per msa_step); a larger step regrows them once
constexpr size_t kHostIdsInitial = 4096;

// ---- ordering events of a host-resident bank (host_mu held)
// Record the next ring event on stream s and return its tag (sequence + 1).
// The entry's previous record is synchronised first, so a tag older than
// the ring always names completed work.
hipError_t ring_record(Bank& bk, hipStream_t s, uint64_t* tag) {
  const uint64_t q = bk.ring_seq;
  hipEvent_t e = bk.ring[q % Bank::kRing];
  if (q >= (uint64_t)Bank::kRing) {
    const hipError_t r = hipEventSynchronize(e);
    if (r != hipSuccess) return r;
  }
  const hipError_t r = hipEventRecord(e, s);
  if (r != hipSuccess) return r;
  bk.ring_seq = q + 1;
  *tag = q + 1;
  return hipSuccess;
}

// True while the work a tag names may still be running (its ring entry has
// not been recorded again since).
bool ring_live(const Bank& bk, uint64_t tag) {
  return tag != 0 && bk.ring_seq - (tag - 1) <= (uint64_t)Bank::kRing;
}

// Make stream s wait, on the device, for the work a tag names.
hipError_t ring_wait(Bank& bk, hipStream_t s, uint64_t tag) {
  if (!ring_live(bk, tag)) return hipSuccess;
  return hipStreamWaitEvent(s, bk.ring[(tag - 1) % Bank::kRing], 0);
}

// Wait on the host for every recorded ring event.
hipError_t ring_drain(Bank& bk) {
  const uint64_t n = std::min<uint64_t>(bk.ring_seq, Bank::kRing);
  for (uint64_t q = bk.ring_seq - n; q < bk.ring_seq; ++q) {
    const hipError_t r = hipEventSynchronize(bk.ring[q % Bank::kRing]);
    if (r != hipSuccess) return r;
  }
  return hipSuccess;
}

// A host-resident store must be pinned host memory from its first to its
// last byte: copies from pageable memory would run synchronously (and
// through a bounce buffer).
bool pinned_host_range(const void* p, size_t bytes) {
  for (const char* q : {(const char*)p, (const char*)p + (bytes ? bytes - 1 : 0)}) {
    hipPointerAttribute_t at{};
    const hipError_t e = hipPointerGetAttributes(&at, q);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // leave no error behind for the next call to report
      return false;
    }
    if (at.type != hipMemoryTypeHost) return false;
  }
  return true;
}

// Whether [p, p + bytes) lies inside the allocation that holds p, as the
// runtime records it (hipMemGetAddressRange).  The library sees only
// pointers, so this is where an array shorter than its stated shape is
// caught before a kernel runs past its end.  A pointer the runtime cannot
// place (memory from another allocator) passes: nothing can be checked.
// A caching allocator's array passes if it ends inside its segment.
bool extent_ok(const void* p, size_t bytes) {
  if (!p || bytes == 0) return true;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the next call to report
    return true;
  }
  return (const char*)p + bytes <= (const char*)base + size;
}

int extent_fail(const char* what, size_t bytes) {
  return fail(MSA_EINVAL, std::string(what) + " is shorter than its shape says (" +
                              std::to_string(bytes) + " bytes, past the end of its allocation)");
}

}  // namespace msa

using namespace msa;

extern "C" {

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_EINVAL: return "invalid argument";
    case MSA_ENOMEM: return "not enough memory (workspace, staging or tables)";
    case MSA_EHIP: return "HIP runtime error";
    case MSA_EUNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

int msa_version(void) { return 10200; }

int msa_timer_enable(int period) {
  g_timer.on = period > 0;
  g_timer.period = std::max(1, period);
  g_timer.seq[0] = g_timer.seq[1] = 0;
  g_timer.skipping[0] = g_timer.skipping[1] = false;
  return MSA_OK;
}

int msa_timer_reserve(int64_t launches) {
  if (launches < 0) return fail(MSA_EINVAL, "timer_reserve: launches < 0");
  while ((int64_t)g_timer.pool.size() < 2 * launches) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return fail(MSA_EHIP, "hipEventCreate");
    g_timer.pool.push_back(e);
  }
  return MSA_OK;
}

int msa_stream_read(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
  static_assert(MSA_STREAM_READ_BLOCKS == kStreamReadBlocks, "probe grid");
  if (!buf || !out || bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return fail(MSA_EINVAL, "stream_read: null pointer, misaligned buffer or bytes not a "
                            "positive multiple of 16");
  MSA_CHECK_HIP(launch_stream_read(buf, bytes, out, static_cast<hipStream_t>(stream)));
  return MSA_OK;
}

int msa_timer_read(int which, double* total_ms, int64_t* launches) {
  if (which < 0 || which > 1 || !total_ms || !launches) return fail(MSA_EINVAL, "timer_read");
  double tot = 0.0;
  int64_t n = 0;
  for (auto& pr : g_timer.done[which]) {
    float ms = 0.f;
    if (hipEventSynchronize(pr.second) != hipSuccess ||
        hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess)
      return fail(MSA_EHIP, "timer events");
    tot += ms;
    ++n;
    g_timer.pool.push_back(pr.first);
    g_timer.pool.push_back(pr.second);
  }
  g_timer.done[which].clear();
  *total_ms = tot;
  *launches = n;
  return MSA_OK;
}

namespace {

// Append documents to the bank's host tables (document and token/chunk
// offsets), checking the store capacities.  On error nothing is changed.
int bank_add_docs(Bank* bk, int n_new, const int64_t* doc_len, const int64_t* kv_off) {
  const int N0 = (int)bk->doc_len.size();
  if ((int64_t)N0 + n_new >= ((int64_t)1 << 31)) return fail(MSA_EUNSUPPORTED, "too many documents");
  int64_t tok = bk->n_tokens, lmax = bk->max_doc_len;
  std::vector<int64_t> kvo(n_new);
  for (int i = 0; i < n_new; ++i) {
    const int64_t L = doc_len[i];
    if (L <= 0 || L % kChunk || L > (int64_t)1 << 30)
      return fail(MSA_EINVAL, "doc_len[" + std::to_string(N0 + i) + "] must be a positive multiple of 256");
    const int64_t o = kv_off ? kv_off[i] : tok;
    if (o < 0 || o + L > bk->desc.kv_tokens)
      return fail(MSA_EINVAL, "kv_off[" + std::to_string(N0 + i) + "] + doc_len exceeds kv_tokens");
    kvo[i] = o;
    tok += L;
    lmax = std::max(lmax, L);
  }
  if (tok / kChunk > bk->chunk_stride)
    return fail(MSA_EINVAL, "documents exceed the routing-key capacity (chunk_cap)");
  if (tok / kChunk >= ((int64_t)1 << 31)) return fail(MSA_EUNSUPPORTED, "too many chunks");
  if (bk->cache && lmax > bk->max_doc_len)
    return fail(MSA_EINVAL, "a document longer than the cache slots: detach the cache first");
  if (bk->tok_off.empty()) {
    bk->tok_off.push_back(0);
    bk->chunk_off.push_back(0);
  }
  for (int i = 0; i < n_new; ++i) {
    bk->doc_len.push_back(doc_len[i]);
    bk->kv_off.push_back(kvo[i]);
    bk->tok_off.push_back(bk->tok_off.back() + doc_len[i]);
    bk->chunk_off.push_back((int32_t)(bk->tok_off.back() / kChunk));
  }
  bk->n_tokens = tok;
  bk->n_chunks = tok / kChunk;
  bk->max_doc_len = lmax;
  bk->desc.n_docs = (int32_t)bk->doc_len.size();
  return MSA_OK;
}

// (Re)build the device tables from the host tables: document lengths and
// offsets, the chunk -> document map, the routing tiles' pieces (document x
// 64-chunk tile overlaps) and the RoPE frequencies, in one allocation.
int bank_upload_tables(Bank* bk) {
  const int N = bk->desc.n_docs;
  const int64_t C = bk->n_chunks;
  const int32_t n_tiles = (int32_t)((C + kRouteTile - 1) / kRouteTile);
  std::vector<int32_t> chunk_doc(C), tile_piece0(n_tiles + 1), doc_piece0(N + 1);
  for (int n = 0; n < N; ++n)
    for (int64_t c = bk->chunk_off[n]; c < bk->chunk_off[n + 1]; ++c) chunk_doc[c] = n;
  int32_t piece = 0;
  int last_doc = -1;
  for (int t = 0; t < n_tiles; ++t) {
    tile_piece0[t] = piece;
    const int64_t c0 = (int64_t)t * kRouteTile, c1 = std::min(C, c0 + kRouteTile);
    for (int64_t c = c0; c < c1; ++c) {
      const int n = chunk_doc[c];
      if (c == c0 || n != chunk_doc[c - 1]) {
        if (n != last_doc) {
          for (int m = last_doc + 1; m <= n; ++m) doc_piece0[m] = piece;
          last_doc = n;
        }
        ++piece;
      }
    }
  }
  tile_piece0[n_tiles] = piece;
  for (int m = last_doc + 1; m <= N; ++m) doc_piece0[m] = piece;
  std::vector<int32_t> dl32(N), plen(N);
  std::vector<int64_t> poff(N), pvoff(N + 1);
  pvoff[0] = 0;
  for (int n = 0; n < N; ++n) {
    dl32[n] = (int32_t)bk->doc_len[n];
    plen[n] = (int32_t)(bk->doc_len[n] / kChunk);
    poff[n] = bk->chunk_off[n];
    pvoff[n + 1] = pvoff[n] + (plen[n] + kAttnTile - 1) / kAttnTile * kAttnTile;
  }
  double inv_freq[kD / 2];
  for (int i = 0; i < kD / 2; ++i) inv_freq[i] = std::pow(bk->desc.rope_base, -2.0 * i / kD);

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t o_dl = take(N * 4), o_kv = take(N * 8), o_tok = take((N + 1) * 8),
               o_cd = take(C * 4), o_tp = take((n_tiles + 1) * 4),
               o_dp = take((N + 1) * 4), o_if = take(sizeof(inv_freq)),
               o_po = take(N * 8), o_pl = take(N * 4), o_pv = take(N * 8);
  void* mem = nullptr;
  if (hipMalloc(&mem, off) != hipSuccess) return fail(MSA_ENOMEM, "hipMalloc of bank tables failed");
  char* base = (char*)mem;
  hipError_t e = hipMemcpy(base + o_dl, dl32.data(), N * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_kv, bk->kv_off.data(), N * 8, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_tok, bk->tok_off.data(), (N + 1) * 8, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_cd, chunk_doc.data(), C * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(base + o_tp, tile_piece0.data(), (n_tiles + 1) * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_dp, doc_piece0.data(), (N + 1) * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_if, inv_freq, sizeof(inv_freq), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_po, poff.data(), N * 8, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_pl, plen.data(), N * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_pv, pvoff.data(), N * 8, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(mem);
    return fail(MSA_EHIP, std::string("uploading bank tables: ") + hipGetErrorString(e));
  }
  if (bk->dev_mem) (void)hipFree(bk->dev_mem);
  bk->dev_mem = mem;
  bk->n_tiles = n_tiles;
  bk->n_pieces = piece;
  bk->d_doc_len = (int32_t*)(base + o_dl);
  bk->d_kv_off = (int64_t*)(base + o_kv);
  bk->d_tok_off = (int64_t*)(base + o_tok);
  bk->d_chunk_doc = (int32_t*)(base + o_cd);
  bk->d_tile_piece0 = (int32_t*)(base + o_tp);
  bk->d_doc_piece0 = (int32_t*)(base + o_dp);
  bk->d_inv_freq = (double*)(base + o_if);
  bk->d_pool_off = (int64_t*)(base + o_po);
  bk->d_pool_len = (int32_t*)(base + o_pl);
  bk->d_pool_voff = (int64_t*)(base + o_pv);
  bk->pool_voff.swap(pvoff);
  return MSA_OK;
}

}  // namespace

int msa_bank_create(const msa_bank_desc* d, msa_bank** out) {
  if (!d || !out) return fail(MSA_EINVAL, "NULL descriptor or output");
  *out = nullptr;
  if (d->dtype != MSA_F32 && d->dtype != MSA_BF16) return fail(MSA_EINVAL, "dtype");
  if (d->n_docs <= 0 || !d->doc_len) return fail(MSA_EINVAL, "n_docs / doc_len");
  if (d->d_r != kD || d->d != kD) return fail(MSA_EUNSUPPORTED, "d and d_r must be 128");
  const int vmax = d->dtype == MSA_BF16 ? 16 : 8;
  if (!is_pow2(d->h_r) || d->h_r > vmax)
    return fail(MSA_EUNSUPPORTED, "h_r must be a power of two <= 16 (bf16) or 8 (f32)");
  if (d->h_kv <= 0 || d->h_kv > 64) return fail(MSA_EUNSUPPORTED, "h_kv must be in [1, 64]");
  if (!(d->rope_base > 1.0)) return fail(MSA_EINVAL, "rope_base must be > 1");
  if (d->kv_loc != MSA_KV_DEVICE && d->kv_loc != MSA_KV_HOST) return fail(MSA_EINVAL, "kv_loc");
  if (!d->kr || !d->inv_norm) return fail(MSA_EINVAL, "kr / inv_norm are NULL");
  if (!d->k_store || !d->v_store) return fail(MSA_EINVAL, "k_store / v_store are NULL");
  if (!all_al16(d->kr, d->inv_norm, d->k_store, d->v_store))
    return fail(MSA_EINVAL, "kr, inv_norm, k_store and v_store must be 16-byte aligned");
  if (d->chunk_cap < 0) return fail(MSA_EINVAL, "chunk_cap < 0");

  Bank* bk = new Bank();
  bk->desc = *d;
  bk->desc.doc_len = nullptr;
  bk->desc.kv_off = nullptr;
  bk->desc.n_docs = 0;
  int64_t chunks = 0;
  for (int n = 0; n < d->n_docs; ++n) chunks += std::max<int64_t>(0, d->doc_len[n]) / kChunk;
  bk->chunk_stride = d->chunk_cap > 0 ? d->chunk_cap : chunks;
  int st = bank_add_docs(bk, d->n_docs, d->doc_len, d->kv_off);
  if (st == MSA_OK && hipGetDevice(&bk->device) != hipSuccess) st = fail(MSA_EHIP, "hipGetDevice");
  if (st == MSA_OK) st = bank_upload_tables(bk);
  if (st != MSA_OK) {
    delete bk;
    return st;
  }
  {
    const size_t dsz = dtype_size(d->dtype);
    const size_t kr_bytes = (size_t)d->h_r * bk->chunk_stride * kD * dsz;
    const size_t in_bytes = (size_t)d->h_r * bk->chunk_stride * sizeof(float);
    const size_t kv_bytes = (size_t)d->kv_tokens * d->h_kv * kD * dsz;
    const char* bad = !extent_ok(d->kr, kr_bytes)         ? "kr"
                      : !extent_ok(d->inv_norm, in_bytes) ? "inv_norm"
                      : d->kv_loc == MSA_KV_DEVICE && !extent_ok(d->k_store, kv_bytes) ? "k_store"
                      : d->kv_loc == MSA_KV_DEVICE && !extent_ok(d->v_store, kv_bytes) ? "v_store"
                                                                                        : nullptr;
    if (bad) {
      msa_bank_destroy(reinterpret_cast<msa_bank*>(bk));
      return extent_fail(bad, !strcmp(bad, "kr") ? kr_bytes
                              : !strcmp(bad, "inv_norm") ? in_bytes : kv_bytes);
    }
  }
  if (d->kv_loc == MSA_KV_HOST) {
    const size_t store_bytes = (size_t)d->kv_tokens * d->h_kv * kD * dtype_size(d->dtype);
    if (!pinned_host_range(d->k_store, store_bytes) || !pinned_host_range(d->v_store, store_bytes)) {
      msa_bank_destroy(reinterpret_cast<msa_bank*>(bk));
      return fail(MSA_EINVAL, "a host-resident K/V store must be pinned host memory "
                              "(hipHostMalloc) over its whole kv_tokens extent");
    }
    hipError_t e = host_buffers_reserve(*bk, kHostIdsInitial);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&bk->tables_done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&bk->copy_fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&bk->copy_join, hipEventDisableTiming);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&bk->copy2, hipStreamNonBlocking);
    for (int i = 0; i < Bank::kRing && e == hipSuccess; ++i)
      e = hipEventCreateWithFlags(&bk->ring[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      msa_bank_destroy(reinterpret_cast<msa_bank*>(bk));
      return fail(MSA_EHIP, std::string("host-bank buffers: ") + hipGetErrorString(e));
    }
  }
  *out = reinterpret_cast<msa_bank*>(bk);
  return MSA_OK;
}

int msa_bank_append(msa_bank* b, int32_t n_new, const int64_t* doc_len, const int64_t* kv_off) {
  if (!b) return fail(MSA_EINVAL, "NULL bank");
  if (n_new < 0 || (n_new > 0 && !doc_len)) return fail(MSA_EINVAL, "n_new / doc_len");
  if (n_new == 0) return MSA_OK;
  Bank* bk = reinterpret_cast<Bank*>(b);
  std::lock_guard<std::mutex> lock(bk->host_mu);
  Bank saved_tables;  // roll back the host tables if the upload fails
  saved_tables.doc_len = bk->doc_len;
  saved_tables.kv_off = bk->kv_off;
  saved_tables.tok_off = bk->tok_off;
  saved_tables.chunk_off = bk->chunk_off;
  const int64_t tok0 = bk->n_tokens, lmax0 = bk->max_doc_len;
  const int32_t n0 = bk->desc.n_docs;
  int st = bank_add_docs(bk, n_new, doc_len, kv_off);
  if (st != MSA_OK) return st;
  const std::vector<int64_t> pool_voff0 = bk->pool_voff;
  st = bank_upload_tables(bk);
  if (st == MSA_OK) {
    bk->pool_k = nullptr;  // the pooled stores' sizes grow: attach them again
    bk->pool_v = nullptr;
  } else {
    bk->pool_voff = pool_voff0;
    bk->doc_len.swap(saved_tables.doc_len);
    bk->kv_off.swap(saved_tables.kv_off);
    bk->tok_off.swap(saved_tables.tok_off);
    bk->chunk_off.swap(saved_tables.chunk_off);
    bk->n_tokens = tok0;
    bk->n_chunks = tok0 / kChunk;
    bk->max_doc_len = lmax0;
    bk->desc.n_docs = n0;
  }
  return st;
}

int msa_bank_destroy(msa_bank* b) {
  if (!b) return MSA_OK;
  Bank* bk = reinterpret_cast<Bank*>(b);
  if (bk->tables_pending) (void)hipEventSynchronize(bk->tables_done);
  if (bk->tables_done) (void)hipEventDestroy(bk->tables_done);
  if (bk->ring[0]) (void)ring_drain(*bk);
  if (bk->copy2) {
    (void)hipStreamSynchronize(bk->copy2);
    (void)hipStreamDestroy(bk->copy2);
  }
  if (bk->copy_fork) (void)hipEventDestroy(bk->copy_fork);
  if (bk->copy_join) (void)hipEventDestroy(bk->copy_join);
  for (hipEvent_t e : bk->ring)
    if (e) (void)hipEventDestroy(e);
  if (bk->dev_mem) (void)hipFree(bk->dev_mem);
  if (bk->h_ids) (void)hipHostFree(bk->h_ids);
  if (bk->h_src) (void)hipHostFree(bk->h_src);
  if (bk->h_src_off) (void)hipHostFree(bk->h_src_off);
  delete bk;
  return MSA_OK;
}

int msa_bank_get_info(const msa_bank* b, msa_bank_info* info) {
  if (!b || !info) return fail(MSA_EINVAL, "NULL bank or info");
  const Bank& bk = *as_bank(b);
  info->n_chunks = bk.n_chunks;
  info->n_tokens = bk.n_tokens;
  info->max_doc_len = bk.max_doc_len;
  info->n_docs = bk.desc.n_docs;
  info->n_pieces = bk.n_pieces;
  return MSA_OK;
}

int msa_build_bank(const msa_bank* b, int32_t doc0, int32_t doc1, const void* route_vec,
                   const void* k_raw, const void* v_raw, void* stream) {
  if (!b) return fail(MSA_EINVAL, "NULL bank");
  const Bank& bk = *as_bank(b);
  if (doc0 < 0 || doc1 > bk.desc.n_docs || doc0 > doc1) return fail(MSA_EINVAL, "document range");
  if ((k_raw == nullptr) != (v_raw == nullptr))
    return fail(MSA_EINVAL, "k_raw and v_raw must both be given or both be NULL");
  if (k_raw && bk.desc.kv_loc != MSA_KV_DEVICE)
    return fail(MSA_EUNSUPPORTED, "K/V of a host-resident store are not written by the library");
  if (!all_al16(route_vec, k_raw, v_raw))
    return fail(MSA_EINVAL, "route_vec, k_raw and v_raw must be 16-byte aligned");
  {
    const size_t rows = (size_t)(bk.tok_off[doc1] - bk.tok_off[doc0]);
    const size_t dsz = dtype_size(bk.desc.dtype);
    const size_t rv_bytes = rows * bk.desc.h_r * kD * dsz, kv_bytes = rows * bk.desc.h_kv * kD * dsz;
    if (!extent_ok(route_vec, rv_bytes)) return extent_fail("route_vec", rv_bytes);
    if (!extent_ok(k_raw, kv_bytes)) return extent_fail("k_raw", kv_bytes);
    if (!extent_ok(v_raw, kv_bytes)) return extent_fail("v_raw", kv_bytes);
  }
  hipStream_t s = (hipStream_t)stream;
  if (route_vec) MSA_CHECK_HIP(launch_pool_keys(bk, doc0, doc1, route_vec, s));
  else MSA_CHECK_HIP(launch_key_norms(bk, doc0, doc1, s));
  if (k_raw) MSA_CHECK_HIP(launch_store_kv(bk, doc0, doc1, k_raw, v_raw, s));
  return MSA_OK;
}

int msa_prepare_local(const msa_bank* b, const void* k_raw, const void* v_raw, int32_t n_seq,
                      int32_t L, int32_t pos0, void* k_loc, void* v_loc, void* stream) {
  if (!b) return fail(MSA_EINVAL, "NULL bank");
  if (n_seq < 0 || L < 0) return fail(MSA_EINVAL, "n_seq / L");
  if (pos0 < 0) return fail(MSA_EINVAL, "pos0 < 0");
  if (n_seq == 0 || L == 0) return MSA_OK;
  if (!k_loc || !v_loc || !k_raw || !v_raw) return fail(MSA_EINVAL, "NULL pointer");
  if (!all_al16(k_loc, v_loc, k_raw, v_raw)) return fail(MSA_EINVAL, "16-byte alignment");
  {
    const Bank& bk = *as_bank(b);
    const size_t dsz = dtype_size(bk.desc.dtype);
    const size_t k_bytes = (size_t)n_seq * L * bk.desc.h_kv * kD * dsz;
    const size_t v_bytes = (size_t)n_seq * bk.desc.h_kv * ((L + 63) / 64) * 64 * kD * dsz;
    if (!extent_ok(k_raw, k_bytes)) return extent_fail("k_raw", k_bytes);
    if (!extent_ok(v_raw, k_bytes)) return extent_fail("v_raw", k_bytes);
    if (!extent_ok(k_loc, k_bytes)) return extent_fail("k_loc", k_bytes);
    if (!extent_ok(v_loc, v_bytes)) return extent_fail("v_loc", v_bytes);
  }
  MSA_CHECK_HIP(launch_prepare_local(*as_bank(b), k_raw, v_raw, n_seq, L, pos0, k_loc, v_loc,
                                     (hipStream_t)stream));
  return MSA_OK;
}

size_t msa_workspace_bytes(const msa_bank* b, int32_t mode, int32_t n_q, int32_t h_q, int32_t k,
                           int32_t block, int32_t hops, int32_t splits) {
  if (!b || n_q < 0 || h_q <= 0 || k < 0) return 0;
  const Bank& bk = *as_bank(b);
  if (splits <= 0) splits = 256;  // covers any automatic choice
  splits = ((splits + 3) / 4) * 4;
  return ws_layout(bk, mode, n_q, h_q, k, block, hops, splits).total;
}

size_t msa_staging_bytes(const msa_bank* b, int32_t n_groups, int32_t k) {
  if (!b || n_groups < 0 || k < 0) return 0;
  const Bank& bk = *as_bank(b);
  return (size_t)2 * n_groups * k * bk.max_doc_len * bk.desc.h_kv * kD *
         dtype_size(bk.desc.dtype);
}

size_t msa_cache_slot_bytes(const msa_bank* b) {
  if (!b) return 0;
  const Bank& bk = *as_bank(b);
  return (size_t)2 * bk.max_doc_len * bk.desc.h_kv * kD * dtype_size(bk.desc.dtype);
}

int msa_bank_set_cache(msa_bank* b, void* cache, size_t cache_bytes) {
  if (!b) return fail(MSA_EINVAL, "NULL bank");
  Bank& bk = *reinterpret_cast<Bank*>(b);
  if (bk.desc.kv_loc != MSA_KV_HOST) return fail(MSA_EINVAL, "a device cache needs a host-resident bank");
  if (!al16(cache)) return fail(MSA_EINVAL, "the cache must be 16-byte aligned");
  std::lock_guard<std::mutex> lock(bk.host_mu);
  // earlier steps' copies and attention may still use the old cache (the
  // second copy stream too, should a call have failed before tagging its
  // copies)
  MSA_CHECK_HIP(ring_drain(bk));
  if (bk.copy2) MSA_CHECK_HIP(hipStreamSynchronize(bk.copy2));
  bk.cache = nullptr;
  bk.cache_slots = 0;
  bk.cache_doc.clear();
  bk.cache_epoch.clear();
  bk.slot_fill.clear();
  bk.slot_read.clear();
  bk.cache_lru.clear();
  bk.cache_pos.clear();
  bk.cache_slot_of.clear();
  if (!cache) return MSA_OK;
  const size_t slot = msa_cache_slot_bytes(b);
  const int64_t n = (int64_t)(cache_bytes / slot);
  if (n < 1) return fail(MSA_ENOMEM, "cache smaller than one document slot");
  bk.cache = (char*)cache;
  bk.cache_slots = n;
  bk.cache_doc.assign(n, -1);
  bk.cache_epoch.assign(n, 0);
  bk.slot_fill.assign(n, 0);
  bk.slot_read.assign(n, 0);
  bk.cache_pos.resize(n);
  for (int64_t i = 0; i < n; ++i) bk.cache_pos[i] = bk.cache_lru.insert(bk.cache_lru.end(), (int32_t)i);
  return MSA_OK;
}

int msa_pooled_sizes(const msa_bank* b, int64_t* k_elems, int64_t* v_elems) {
  if (!b || !k_elems || !v_elems) return fail(MSA_EINVAL, "NULL argument");
  const Bank& bk = *as_bank(b);
  *k_elems = bk.n_chunks * bk.desc.h_kv * kD;
  *v_elems = bk.pool_voff.back() * bk.desc.h_kv * kD;
  return MSA_OK;
}

int msa_bank_set_pooled(msa_bank* b, void* pool_k, void* pool_v) {
  if (!b) return fail(MSA_EINVAL, "NULL bank");
  if ((pool_k == nullptr) != (pool_v == nullptr)) return fail(MSA_EINVAL, "pool_k and pool_v");
  if (!all_al16(pool_k, pool_v)) return fail(MSA_EINVAL, "pool_k / pool_v must be 16-byte aligned");
  Bank& bk = *reinterpret_cast<Bank*>(b);
  bk.pool_k = pool_k;
  bk.pool_v = pool_v;
  return MSA_OK;
}

int msa_build_pooled(const msa_bank* b, int32_t doc0, int32_t doc1, void* stream) {
  if (!b) return fail(MSA_EINVAL, "NULL bank");
  const Bank& bk = *as_bank(b);
  if (doc0 < 0 || doc1 > bk.desc.n_docs || doc0 > doc1) return fail(MSA_EINVAL, "document range");
  if (!bk.pool_k || !bk.pool_v) return fail(MSA_EINVAL, "no pooled stores attached");
  if (bk.desc.kv_loc != MSA_KV_DEVICE)
    return fail(MSA_EUNSUPPORTED, "pooled stores are built from a device-resident store");
  MSA_CHECK_HIP(launch_pool_kv(bk, doc0, doc1, (hipStream_t)stream));
  return MSA_OK;
}

}  // extern "C"

namespace {

// Where one hop's distinct selected documents of a host-resident bank sit on
// the device, and what the attention must wait for before reading them.
struct Resident {
  char* kbase = nullptr;         // K of compact index j at kbase + off[j] * token bytes
  char* vbase = nullptr;         // V likewise
  std::vector<uint64_t> waits;   // ring tags of copies the attention waits for
  std::vector<int32_t> slots;    // cache slots in use (with a cache)
};

// Make the distinct documents `docs` resident on the device (host_mu held):
// with a cache, documents already in a slot stay (hits) and the others are
// copied from the host store into least recently used slots; without one,
// every document is copied into `staging`, in order.  Copies go on stream
// cs.  A copy into a slot first waits, on cs, for the slot's last reader and
// its previous fill.  slot_off / slot_len receive each compact index's token
// offset from the bases and its length.
int make_resident(Bank& bk, const std::vector<int32_t>& docs, void* staging, size_t staging_bytes,
                  hipStream_t cs, msa_step_stats* stats, int64_t* slot_off, int32_t* slot_len,
                  Resident* r) {
  const int32_t n = (int32_t)docs.size();
  const size_t tok_bytes = (size_t)bk.desc.h_kv * kD * dtype_size(bk.desc.dtype);
  // Copies into cache slots: K on cs, V on the bank's second copy stream,
  // forked from cs before the first copy (after every wait placed on cs)
  // and joined back into cs after the last.  Copies into staging stay on cs
  // alone: into staging, two streams measured faster in the first process
  // to use a device but slower in every later process (about 95 against 102
  // queries/s at 100M tokens), while copies into slots gained in all of them.
  const bool two = bk.cache != nullptr;
  bool forked = false;
  auto fork = [&]() -> hipError_t {
    if (forked) return hipSuccess;
    forked = true;
    hipError_t e = hipEventRecord(bk.copy_fork, cs);
    return e == hipSuccess ? hipStreamWaitEvent(bk.copy2, bk.copy_fork, 0) : e;
  };
  auto join = [&]() -> hipError_t {
    if (!forked) return hipSuccess;
    forked = false;
    hipError_t e = hipEventRecord(bk.copy_join, bk.copy2);
    return e == hipSuccess ? hipStreamWaitEvent(cs, bk.copy_join, 0) : e;
  };
  struct JoinOnExit {  // an early error return still orders cs after the V copies
    decltype(join)& f;
    ~JoinOnExit() { (void)f(); }
  } join_on_exit{join};
  auto copy_doc = [&](int32_t id, char* kdst, char* vdst) -> hipError_t {
    const size_t bytes = (size_t)bk.doc_len[id] * tok_bytes;
    const size_t src_o = (size_t)bk.kv_off[id] * tok_bytes;
    hipError_t e = two ? fork() : hipSuccess;
    if (e == hipSuccess)
      e = hipMemcpyAsync(kdst, (const char*)bk.desc.k_store + src_o, bytes, hipMemcpyHostToDevice, cs);
    if (e == hipSuccess)
      e = hipMemcpyAsync(vdst, (const char*)bk.desc.v_store + src_o, bytes, hipMemcpyHostToDevice,
                         two ? bk.copy2 : cs);
    if (stats) {
      stats->docs_copied += 1;
      stats->bytes_copied += (int64_t)(2 * bytes);
    }
    return e;
  };
  std::vector<int32_t> filled;
  if (bk.cache) {
    if (n > bk.cache_slots)
      return fail(MSA_ENOMEM, "one hop selects more distinct documents than the cache has slots");
    const size_t slot_k = (size_t)bk.max_doc_len * tok_bytes;
    r->kbase = bk.cache;
    r->vbase = bk.cache + (size_t)bk.cache_slots * slot_k;
    const uint64_t ep = ++bk.hop_epoch;
    auto touch = [&](int32_t slot) {
      bk.cache_lru.splice(bk.cache_lru.begin(), bk.cache_lru, bk.cache_pos[slot]);
      bk.cache_epoch[slot] = ep;
    };
    r->slots.assign(n, -1);
    // hits first: they move to the front, so no miss of this hop evicts them;
    // a hit whose fill may still be in flight is waited for
    for (int32_t j = 0; j < n; ++j) {
      auto h = bk.cache_slot_of.find(docs[j]);
      if (h == bk.cache_slot_of.end()) continue;
      r->slots[j] = h->second;
      touch(h->second);
      if (ring_live(bk, bk.slot_fill[h->second])) r->waits.push_back(bk.slot_fill[h->second]);
      if (stats) stats->docs_cached += 1;
    }
    std::vector<uint64_t> before;  // what cs waits for before overwriting victims
    std::vector<int32_t> victims;
    for (int32_t j = 0; j < n; ++j) {
      if (r->slots[j] >= 0) continue;
      const int32_t victim = bk.cache_lru.back();
      if (bk.cache_epoch[victim] == ep) return fail(MSA_ENOMEM, "cache slots exhausted");
      if (bk.cache_doc[victim] >= 0) bk.cache_slot_of.erase(bk.cache_doc[victim]);
      bk.cache_doc[victim] = docs[j];
      bk.cache_slot_of[docs[j]] = victim;
      touch(victim);
      r->slots[j] = victim;
      victims.push_back(j);
      for (uint64_t t : {bk.slot_read[victim], bk.slot_fill[victim]})
        if (ring_live(bk, t)) before.push_back(t);
    }
    std::sort(before.begin(), before.end());
    before.erase(std::unique(before.begin(), before.end()), before.end());
    for (uint64_t t : before) MSA_CHECK_HIP(ring_wait(bk, cs, t));
    for (int32_t j : victims) {
      const int32_t v = r->slots[j];
      MSA_CHECK_HIP(copy_doc(docs[j], r->kbase + (size_t)v * slot_k, r->vbase + (size_t)v * slot_k));
      filled.push_back(v);
    }
    for (int32_t j = 0; j < n; ++j) {
      slot_off[j] = (int64_t)r->slots[j] * bk.max_doc_len;
      slot_len[j] = (int32_t)bk.doc_len[docs[j]];
    }
  } else {
    const size_t half = staging_bytes / 2;
    r->kbase = (char*)staging;
    r->vbase = r->kbase + half;
    int64_t tok = 0;
    for (int32_t j = 0; j < n; ++j) {
      slot_off[j] = tok;
      slot_len[j] = (int32_t)bk.doc_len[docs[j]];
      MSA_CHECK_HIP(copy_doc(docs[j], r->kbase + (size_t)tok * tok_bytes,
                             r->vbase + (size_t)tok * tok_bytes));
      tok += bk.doc_len[docs[j]];
    }
    if (n > 0) filled.push_back(-1);
  }
  MSA_CHECK_HIP(join());
  if (!filled.empty()) {
    uint64_t tag = 0;
    MSA_CHECK_HIP(ring_record(bk, cs, &tag));
    for (int32_t v : filled)
      if (v >= 0) bk.slot_fill[v] = tag;
    r->waits.push_back(tag);
  }
  std::sort(r->waits.begin(), r->waits.end());
  r->waits.erase(std::unique(r->waits.begin(), r->waits.end()), r->waits.end());
  return MSA_OK;
}

// Read one hop's selected ids back and reduce them to distinct documents:
// docs[j] is compact index j's document, slot_ids[i] selection i's compact
// index (-1 for an empty slot).  Blocks on stream s.
int read_back_ids(Bank& bk, const int32_t* ids, size_t n_sel, hipStream_t s,
                  std::vector<int32_t>* docs, int32_t* slot_ids) {
  MSA_CHECK_HIP(hipMemcpyAsync(bk.h_ids, ids, n_sel * 4, hipMemcpyDeviceToHost, s));
  MSA_CHECK_HIP(hipStreamSynchronize(s));
  std::unordered_map<int32_t, int32_t> slot_of;  // document -> compact index
  const int N = bk.desc.n_docs;
  for (size_t i = 0; i < n_sel; ++i) {
    const int32_t id = bk.h_ids[i];
    if (id < 0 || id >= N) {
      if (slot_ids) slot_ids[i] = -1;
      continue;
    }
    auto it = slot_of.find(id);
    if (it == slot_of.end()) {
      it = slot_of.emplace(id, (int32_t)docs->size()).first;
      docs->push_back(id);
    }
    if (slot_ids) slot_ids[i] = it->second;
  }
  return MSA_OK;
}

}  // namespace

extern "C" {

int msa_route(const msa_bank* b, const float* q_route, int32_t B, int32_t k,
              const uint32_t* exclude, int32_t* ids, float* scores, void* ws, size_t ws_bytes,
              void* stream) {
  if (!b) return fail(MSA_EINVAL, "NULL bank");
  const Bank& bk = *as_bank(b);
  if (B < 0) return fail(MSA_EINVAL, "B < 0");
  if (k < 1 || k > bk.desc.n_docs) return fail(MSA_EINVAL, "k must be in [1, n_docs]");
  if (k > kMaxK) return fail(MSA_EUNSUPPORTED, "k must be <= 64");
  if (B == 0) return MSA_OK;
  if (!q_route || !ids || !scores || !ws) return fail(MSA_EINVAL, "NULL pointer");
  if (!all_al16(q_route, ws)) return fail(MSA_EINVAL, "q_route and ws must be 16-byte aligned");
  const WsLayout L = ws_layout(bk, MSA_DECODE, B, bk.desc.h_kv, k, 1, 1, 4);
  const size_t need = L.route_end;
  if (ws_bytes < need) return fail(MSA_ENOMEM, "workspace too small for msa_route");
  char* w = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  MSA_CHECK_HIP(launch_route_scan(bk, q_route, B, (float*)(w + L.piecemax), s));
  MSA_CHECK_HIP(launch_topk(bk, (const float*)(w + L.piecemax), B, k, exclude, nullptr, ids,
                            scores, (uint64_t*)(w + L.keys), s));
  return MSA_OK;
}

int msa_attend(const msa_bank* b, const msa_attend_args* a, void* stream) {
  if (!b || !a) return fail(MSA_EINVAL, "NULL bank or args");
  const Bank& bk = *as_bank(b);
  int st = check_attend_common(bk, a->mode, a->n_q, a->h_q, a->k, a->block, a->L_loc, a->k_loc,
                               a->v_loc);
  if (st) return st;
  if (a->n_q == 0) return MSA_OK;
  if (!a->q || !a->out || !a->ws || (a->k > 0 && !a->ids)) return fail(MSA_EINVAL, "NULL pointer");
  if (!all_al16(a->q, a->out, a->ws, a->src_k, a->src_v))
    return fail(MSA_EINVAL, "q, out, ws and source K/V must be 16-byte aligned");
  if (a->q_pos < 0) return fail(MSA_EINVAL, "q_pos < 0");
  AttnSources src{bk.desc.k_store, bk.desc.v_store, bk.d_kv_off, bk.d_doc_len, bk.desc.n_docs};
  const bool pooled = a->memory == MSA_MEMORY_POOLED;
  if (a->memory != MSA_MEMORY_TOKENS && !pooled) return fail(MSA_EINVAL, "memory");
  if (pooled) {
    if (a->mode != MSA_DECODE) return fail(MSA_EUNSUPPORTED, "pooled memory is a decode mode");
    if (!bk.pool_k || !bk.pool_v) return fail(MSA_EINVAL, "no pooled stores attached");
    if (a->src_len || a->src_off || a->src_k || a->src_v)
      return fail(MSA_EINVAL, "pooled memory takes no source override");
    src = pooled_sources(bk);
  } else if (a->src_len || a->src_off || a->src_k || a->src_v) {
    if (!a->src_len || !a->src_off || !a->src_k || !a->src_v || a->n_src < 0)
      return fail(MSA_EINVAL, "source override needs src_k, src_v, src_off, src_len and n_src");
    src = AttnSources{a->src_k, a->src_v, a->src_off, a->src_len, a->n_src};
  } else if (bk.desc.kv_loc != MSA_KV_DEVICE && a->k > 0) {
    return fail(MSA_EUNSUPPORTED, "host-resident bank: use msa_step or a source override");
  }
  if (a->splits < 0 || a->splits > kMaxSplits) return fail(MSA_EINVAL, "splits must be in [0, 256]");
  const int splits =
      resolve_splits(bk, a->mode, a->splits, a->n_q, a->h_q, a->block, a->k, a->L_loc, pooled);
  const WsLayout L = ws_layout(bk, a->mode, a->n_q, a->h_q, a->k, a->block, 1, splits);
  if (a->ws_bytes < L.total) return fail(MSA_ENOMEM, "workspace too small for msa_attend");
  char* w = (char*)a->ws;
  hipStream_t s = (hipStream_t)stream;
  const bool prefill = a->mode == MSA_PREFILL;
  // decode rotates the queries inside the attention kernel
  if (prefill) {
    MSA_CHECK_HIP(launch_rope_queries(bk, a->q, a->n_q, a->h_q, a->q_pos, 1, w + L.qrot, s));
    MSA_CHECK_HIP(launch_prefill(bk, w + L.qrot, a->n_q, a->h_q, a->ids, a->k, a->block, src,
                                 a->k_loc, a->v_loc, a->L_loc, splits, (float*)(w + L.part),
                                 a->out, s));
  } else {
    MSA_CHECK_HIP(launch_decode(bk, a->q, a->q_pos, a->n_q, a->h_q, a->ids, a->k, src,
                                a->k_loc, a->v_loc, a->L_loc, splits, (float*)(w + L.part),
                                a->out, s));
  }
  return MSA_OK;
}

}  // extern "C"

namespace {

// Scratch of msa_step_static: device memory the library owns, one copy per
// GPU (a file-scope device array), for callers that cannot allocate.  Host
// code never uses the array's name as an address: the address comes from
// hipGetSymbolAddress on each device, kept per device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = 0;
  MSA_CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(MSA_EUNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MSA_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(MSA_EHIP, "hipGetSymbolAddress returned no address for the scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

// msa_step with the workspace taken from the arguments (ws_override NULL) or
// from ws_override / ws_override_bytes (the static scratch).
int step_impl(const msa_bank* b, const msa_step_args* a, void* stream, void* copy_stream,
              msa_step_stats* stats, void* ws_override, size_t ws_override_bytes) {
  if (!b || !a) return fail(MSA_EINVAL, "NULL bank or args");
  Bank& bk = *const_cast<Bank*>(as_bank(b));
  void* const ws_ptr = ws_override ? ws_override : a->ws;
  const size_t ws_bytes = ws_override ? ws_override_bytes : a->ws_bytes;
  const int N = bk.desc.n_docs;
  int st = check_attend_common(bk, a->mode, a->n_q, a->h_q, a->k, a->block, a->L_loc, a->k_loc,
                               a->v_loc);
  if (st) return st;
  if (a->k < 1 || a->k > N) return fail(MSA_EINVAL, "k must be in [1, n_docs]");
  if (a->hops < 1) return fail(MSA_EINVAL, "hops must be >= 1");
  const bool prefill = a->mode == MSA_PREFILL;
  if (a->hops > 1 && (prefill || bk.desc.h_r != 1 || !a->w_proj))
    return fail(MSA_EINVAL, "hops > 1 needs decode mode, h_r == 1 and w_proj");
  if (stats) {
    stats->docs_copied = 0;
    stats->bytes_copied = 0;
    stats->docs_cached = 0;
  }
  if (a->n_q == 0) return MSA_OK;
  if (!a->q || !a->ids || !a->scores || !a->out || !ws_ptr) return fail(MSA_EINVAL, "NULL pointer");
  if (prefill ? !a->route_tokens : !a->q_route) return fail(MSA_EINVAL, "router input is NULL");
  if (!all_al16(a->q, a->out, ws_ptr, a->q_route, a->route_tokens, a->staging, a->w_proj))
    return fail(MSA_EINVAL, "q, out, ws, router input, w_proj and staging must be 16-byte aligned");
  if (a->q_pos < 0) return fail(MSA_EINVAL, "q_pos < 0");
  const bool pooled = a->memory == MSA_MEMORY_POOLED;
  if (a->memory != MSA_MEMORY_TOKENS && !pooled) return fail(MSA_EINVAL, "memory");
  if (pooled && a->mode != MSA_DECODE) return fail(MSA_EUNSUPPORTED, "pooled memory is a decode mode");
  if (pooled && (!bk.pool_k || !bk.pool_v)) return fail(MSA_EINVAL, "no pooled stores attached");
  // pooled memory lives on the device: no host copies even for a host-resident bank
  const bool host = bk.desc.kv_loc == MSA_KV_HOST && !pooled;
  const int n_groups = prefill ? a->n_q / a->block : a->n_q;
  const int k = a->k;
  if (a->splits < 0 || a->splits > kMaxSplits) return fail(MSA_EINVAL, "splits must be in [0, 256]");
  const int splits =
      resolve_splits(bk, a->mode, a->splits, a->n_q, a->h_q, a->block, k, a->L_loc, pooled);
  const WsLayout L = ws_layout(bk, a->mode, a->n_q, a->h_q, k, a->block, a->hops, splits);
  if (ws_bytes < L.total) {
    if (ws_override)
      return fail(MSA_ENOMEM, "msa_step_static: this request needs " + std::to_string(L.total) +
                                  " bytes of scratch, more than the " +
                                  std::to_string(kStaticScratchBytes) + " the library holds per device");
    return fail(MSA_ENOMEM, "workspace too small for msa_step");
  }
  // The host part of a host-resident bank's step (id readback, copy issue,
  // remap tables) uses the bank's pinned buffers: one step at a time.
  std::unique_lock<std::mutex> host_lock;
  if (host) {
    host_lock = std::unique_lock<std::mutex>(bk.host_mu);
    // the previous step's remap tables must have left the pinned buffers
    if (bk.tables_pending) {
      MSA_CHECK_HIP(hipEventSynchronize(bk.tables_done));
      bk.tables_pending = false;
    }
    if (host_buffers_reserve(bk, (size_t)n_groups * k) != hipSuccess)
      return fail(MSA_ENOMEM, "pinned id buffers");
    if (!bk.cache) {
      if (!a->staging) return fail(MSA_EINVAL, "host-resident bank needs a staging buffer");
      if (a->staging_bytes < msa_staging_bytes(b, n_groups, k))
        return fail(MSA_ENOMEM, "staging buffer too small");
    }
  }
  char* w = (char*)ws_ptr;
  hipStream_t s = (hipStream_t)stream;
  hipStream_t cs = copy_stream ? (hipStream_t)copy_stream : s;
  const int W = (N + 31) / 32;
  uint32_t* excl = a->exclude;
  if (a->exclude_selected && !excl) {
    excl = (uint32_t*)(w + L.excl);
    MSA_CHECK_HIP(launch_fill_zero(excl, (size_t)n_groups * W * 4, s));
  }
  float* q_route = (float*)(w + L.qroute);
  if (prefill) {
    MSA_CHECK_HIP(launch_block_mean(bk, a->route_tokens, a->n_q, a->block, q_route, s));
  }
  const float* qr = prefill ? q_route : a->q_route;
  const size_t out_stride = (size_t)a->n_q * a->h_q * kD;
  // decode rotates the queries inside the attention kernel
  if (prefill)
    MSA_CHECK_HIP(launch_rope_queries(bk, a->q, a->n_q, a->h_q, a->q_pos, 1, w + L.qrot, s));
  for (int hop = 0; hop < a->hops; ++hop) {
    int32_t* ids = a->ids + (size_t)hop * n_groups * k;
    float* scores = a->scores + (size_t)hop * n_groups * k;
    float* out = a->out + (size_t)hop * out_stride;
    MSA_CHECK_HIP(launch_route_scan(bk, qr, n_groups, (float*)(w + L.piecemax), s));
    MSA_CHECK_HIP(launch_topk(bk, (const float*)(w + L.piecemax), n_groups, k, excl,
                              a->exclude_selected ? excl : nullptr, ids, scores,
                              (uint64_t*)(w + L.keys), s));
    AttnSources src = pooled ? pooled_sources(bk)
                             : AttnSources{bk.desc.k_store, bk.desc.v_store, bk.d_kv_off,
                                           bk.d_doc_len, N};
    const int32_t* att_ids = ids;
    Resident res;
    if (host) {
      // top-k -> K/V fetch is sequential: read the ids back, then make each
      // distinct selected document resident on the device (a cache hit, or
      // a copy into a cache slot or into staging) and remap the ids to a
      // compact table of those documents
      std::vector<int32_t> docs;
      int32_t* slot_ids = bk.h_src;                        // [n_groups*k]
      int32_t* slot_len = bk.h_src + (size_t)n_groups * k;  // [n_slots]
      int64_t* slot_off = bk.h_src_off;                    // [n_slots]
      st = read_back_ids(bk, ids, (size_t)n_groups * k, s, &docs, slot_ids);
      if (st) return st;
      const int32_t n_slots = (int32_t)docs.size();
      st = make_resident(bk, docs, a->staging, a->staging_bytes, cs, stats, slot_off, slot_len, &res);
      if (st) return st;
      int32_t* d_ids = (int32_t*)(w + L.srcids);
      int64_t* d_off = (int64_t*)(w + L.srcoff);
      int32_t* d_len = (int32_t*)(w + L.srclen);
      MSA_CHECK_HIP(hipMemcpyAsync(d_ids, slot_ids, (size_t)n_groups * k * 4,
                                   hipMemcpyHostToDevice, s));
      if (n_slots > 0) {
        MSA_CHECK_HIP(hipMemcpyAsync(d_off, slot_off, (size_t)n_slots * 8, hipMemcpyHostToDevice, s));
        MSA_CHECK_HIP(hipMemcpyAsync(d_len, slot_len, (size_t)n_slots * 4, hipMemcpyHostToDevice, s));
      }
      MSA_CHECK_HIP(hipEventRecord(bk.tables_done, s));
      bk.tables_pending = true;
      for (uint64_t t : res.waits) MSA_CHECK_HIP(ring_wait(bk, s, t));
      src = AttnSources{res.kbase, res.vbase, d_off, d_len, n_slots};
      att_ids = d_ids;
    }
    if (prefill)
      MSA_CHECK_HIP(launch_prefill(bk, w + L.qrot, a->n_q, a->h_q, att_ids, k, a->block, src,
                                   a->k_loc, a->v_loc, a->L_loc, splits, (float*)(w + L.part), out,
                                   s));
    else
      MSA_CHECK_HIP(launch_decode(bk, a->q, a->q_pos, a->n_q, a->h_q, att_ids, k, src,
                                  a->k_loc, a->v_loc, a->L_loc, splits, (float*)(w + L.part),
                                  out, s));
    if (host && bk.cache) {  // no later copy overwrites these slots before this attention ends
      uint64_t tag = 0;
      MSA_CHECK_HIP(ring_record(bk, s, &tag));
      for (int32_t v : res.slots) bk.slot_read[v] = tag;
    }
    if (hop + 1 < a->hops) {
      MSA_CHECK_HIP(launch_project(out, a->w_proj, a->n_q, a->h_q * kD, kD, q_route, s));
      qr = q_route;
    }
  }
  return MSA_OK;
}

}  // namespace

extern "C" {

int msa_step(const msa_bank* b, const msa_step_args* a, void* stream, void* copy_stream,
             msa_step_stats* stats) {
  return step_impl(b, a, stream, copy_stream, stats, nullptr, 0);
}

int msa_step_static(const msa_bank* b, const msa_step_args* a, void* stream) {
  if (!b || !a) return fail(MSA_EINVAL, "NULL bank or args");
  const Bank& bk = *as_bank(b);
  if (bk.desc.kv_loc != MSA_KV_DEVICE)
    return fail(MSA_EUNSUPPORTED, "msa_step_static: device-resident banks only (a host-resident "
                                  "step reads ids back into pinned buffers it may have to grow)");
  void* p = nullptr;
  const int st = static_scratch(&p);
  if (st) return st;
  return step_impl(b, a, stream, nullptr, nullptr, p, kStaticScratchBytes);
}

int msa_prefetch(const msa_bank* b, const float* q_route, int32_t B, int32_t k,
                 const uint32_t* exclude, void* ws, size_t ws_bytes, void* stream,
                 void* copy_stream, msa_step_stats* stats) {
  if (!b) return fail(MSA_EINVAL, "NULL bank");
  Bank& bk = *const_cast<Bank*>(as_bank(b));
  if (bk.desc.kv_loc != MSA_KV_HOST || !bk.cache)
    return fail(MSA_EINVAL, "prefetch needs a host-resident bank with a device cache attached");
  if (B < 0) return fail(MSA_EINVAL, "B < 0");
  if (k < 1 || k > bk.desc.n_docs) return fail(MSA_EINVAL, "k must be in [1, n_docs]");
  if (k > kMaxK) return fail(MSA_EUNSUPPORTED, "k must be <= 64");
  if (stats) {
    stats->docs_copied = 0;
    stats->bytes_copied = 0;
    stats->docs_cached = 0;
  }
  if (B == 0) return MSA_OK;
  if (!q_route || !ws) return fail(MSA_EINVAL, "NULL pointer");
  if (!all_al16(q_route, ws)) return fail(MSA_EINVAL, "q_route and ws must be 16-byte aligned");
  const WsLayout L = ws_layout(bk, MSA_DECODE, B, bk.desc.h_kv, k, 1, 1, 4);
  if (ws_bytes < L.total) return fail(MSA_ENOMEM, "workspace too small for msa_prefetch");
  char* w = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  hipStream_t cs = copy_stream ? (hipStream_t)copy_stream : s;
  // the selection lands in the workspace's remap-table area
  int32_t* ids = (int32_t*)(w + L.srcids);
  float* scores = (float*)(w + L.srcoff);
  MSA_CHECK_HIP(launch_route_scan(bk, q_route, B, (float*)(w + L.piecemax), s));
  MSA_CHECK_HIP(launch_topk(bk, (const float*)(w + L.piecemax), B, k, exclude, nullptr, ids,
                            scores, (uint64_t*)(w + L.keys), s));
  std::lock_guard<std::mutex> lock(bk.host_mu);
  if (bk.tables_pending && (size_t)B * k > bk.h_ids_cap) {  // regrowing frees the table buffers
    MSA_CHECK_HIP(hipEventSynchronize(bk.tables_done));
    bk.tables_pending = false;
  }
  if (host_buffers_reserve(bk, (size_t)B * k) != hipSuccess) return fail(MSA_ENOMEM, "pinned id buffers");
  std::vector<int32_t> docs;
  int st = read_back_ids(bk, ids, (size_t)B * k, s, &docs, nullptr);
  if (st) return st;
  std::vector<int64_t> off(docs.size());
  std::vector<int32_t> len(docs.size());
  Resident res;
  return make_resident(bk, docs, nullptr, 0, cs, stats, off.data(), len.data(), &res);
}

}  // extern "C"
