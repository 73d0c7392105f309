// Internal declarations of libmsa: the bank object, device helpers shared by
// the kernels, and the launchers each translation unit exports to the API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <string>
#include <list>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/msa.h"

namespace msa {

constexpr int kChunk = 256;     // routing-key chunk (tokens)
constexpr int kD = 128;         // head size and routing-key size
constexpr int kRouteTile = 64;  // chunks per routing wave
constexpr int kAttnTile = 64;   // tokens per attention wave step
constexpr int kMaxK = 64;       // documents per query the attention kernels accept

struct Bank {
  msa_bank_desc desc;  // host pointers inside are not retained
  int device = 0;
  int64_t n_tokens = 0, n_chunks = 0, max_doc_len = 0;
  int64_t chunk_stride = 0;  // rows per head of kr / inv_norm (the chunk capacity)
  int32_t n_tiles = 0, n_pieces = 0;
  std::vector<int64_t> doc_len, kv_off, tok_off;  // host copies; tok_off has N+1 entries
  std::vector<int32_t> chunk_off;                 // N+1
  // device tables, one allocation
  void* dev_mem = nullptr;
  int32_t* d_doc_len = nullptr;      // [N]
  int64_t* d_kv_off = nullptr;       // [N]
  int64_t* d_tok_off = nullptr;      // [N+1]
  int32_t* d_chunk_doc = nullptr;    // [C]
  int32_t* d_tile_piece0 = nullptr;  // [n_tiles + 1]
  int32_t* d_doc_piece0 = nullptr;   // [N + 1]
  double* d_inv_freq = nullptr;      // [64]
  // compressed memory (msa_bank_set_pooled): per document its pooled K
  // offset (= its first chunk), entry count (chunks) and padded V offset
  int64_t* d_pool_off = nullptr;     // [N]
  int32_t* d_pool_len = nullptr;     // [N]
  int64_t* d_pool_voff = nullptr;    // [N]
  std::vector<int64_t> pool_voff;    // N+1, host copy (entries, 64-padded per document)
  void* pool_k = nullptr;            // [C][h_kv][d] in per-document [h_kv][P][d] blocks
  void* pool_v = nullptr;            // per document [h_kv][ceil(P/64)][d][64], zero-padded
  // host-resident banks: pinned buffers for reading back selected ids and
  // staging the remap tables, and the events that order the copies.  The
  // host part of msa_step / msa_prefetch holds host_mu while it uses them.
  int32_t* h_ids = nullptr;
  size_t h_ids_cap = 0;
  int32_t* h_src = nullptr;  // pinned [2 * cap] remap table staging
  int64_t* h_src_off = nullptr;
  hipEvent_t tables_done = nullptr;  // remap tables read out of h_src / h_src_off
  bool tables_pending = false;
  // A second copy stream (default priority) that takes the V copy of each
  // document copied into a cache slot while the caller's copy stream takes
  // its K: two copies in flight keep the link busy through each copy's
  // start-up.  copy_fork orders it after the caller's copy stream,
  // copy_join orders the copy stream after it, so callers see every copy
  // of a call on their copy stream.
  hipStream_t copy2 = nullptr;
  hipEvent_t copy_fork = nullptr, copy_join = nullptr;
  // Ordering events: a ring of kRing events, recorded in sequence.  An
  // entry is synchronised before it is recorded again, so work tagged with a
  // sequence number older than the ring has completed.  Tags are stored as
  // sequence + 1 (0 = nothing to wait for).
  static constexpr int kRing = 64;
  hipEvent_t ring[kRing] = {};
  uint64_t ring_seq = 0;  // sequence number of the next record
  // device document cache of a host-resident bank (msa_bank_set_cache):
  // slot s holds one document's K at cache + s * slot K bytes and its V in
  // the second half; an LRU list of slots, most recently used first
  char* cache = nullptr;
  int64_t cache_slots = 0;
  std::vector<int32_t> cache_doc;     // [slots] document in the slot, or -1
  std::vector<uint64_t> cache_epoch;  // [slots] last hop that used the slot
  std::vector<uint64_t> slot_fill;    // [slots] tag of the copy that filled the slot
  std::vector<uint64_t> slot_read;    // [slots] tag of the last attention that read it
  std::list<int32_t> cache_lru;
  std::vector<std::list<int32_t>::iterator> cache_pos;
  std::unordered_map<int32_t, int32_t> cache_slot_of;  // document -> slot
  uint64_t hop_epoch = 0;
  std::mutex host_mu;
};

// (Re)allocate a host-resident bank's pinned id/table buffers for `cap`
// selections.  Called with host_mu held (or before the bank is published).
hipError_t host_buffers_reserve(Bank& bk, size_t cap);

// thread-local last error message
void set_error(const std::string& msg);

// optional event timing of one kernel class (see msa_timer_enable)
void timer_mark(int which, bool begin, hipStream_t s);

inline size_t dtype_size(msa_dtype t) { return t == MSA_BF16 ? 2 : 4; }

// --------------------------------------------------------------------------
// device helpers
// --------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// 16-byte global load with the nontemporal hint, for data a kernel streams
// once: on a 2 GiB read-only stream it raises the sustained HBM read rate
// from about 6.2 to 7.0 TB/s.  Used for the routing keys and decode's K
// tiles; where a kernel interleaves other streams the effect has to be
// measured per stream (on decode's V tiles it was a loss).
__device__ __forceinline__ uint4 ld_nt(const void* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// float -> bfloat16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// double -> bfloat16, round to nearest even, directly from the 64-bit pattern
// (no intermediate float rounding).  Normal-range finite inputs; zero maps to
// signed zero.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint64_t sign = u >> 63;
  if ((u & 0x7fffffffffffffffull) == 0) return (uint16_t)(sign << 15);
  u += 0xfffffffffffull + ((u >> 45) & 1ull);  // add half-ulp - 1 (+1 if odd): RNE at bit 45
  const int64_t e = (int64_t)((u >> 52) & 0x7ff) - 1023 + 127;
  const uint32_t mant = (uint32_t)((u >> 45) & 0x7f);
  return (uint16_t)((sign << 15) | ((uint64_t)e << 7) | mant);
}

// storage element <-> float64 (bf16 stores round to nearest even)
template <typename T> struct St;
template <> struct St<float> {
  static __device__ __forceinline__ float store(double x) { return (float)x; }
  static __device__ __forceinline__ double load(float x) { return (double)x; }
};
template <> struct St<uint16_t> {
  static __device__ __forceinline__ uint16_t store(double x) { return f64_to_bf16(x); }
  static __device__ __forceinline__ double load(uint16_t x) { return (double)bf16_to_f32(x); }
};

// fp32 accumulate of a bf16 pair dot product: c + a.lo*b.lo + a.hi*b.hi
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP lane exchanges inside groups of 8 lanes (all sources valid)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4e;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each 8 lanes

constexpr int kDppRowMirror = 0x140;  // lane i <-> 15 - i within each 16 lanes

// Wave-wide reductions (result in every lane): four DPP steps leave each
// 16-lane row's result in all of its lanes, then the four row values are
// read into scalars.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppRowMirror>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Order-preserving map of a float onto uint32 (larger float -> larger code).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// --------------------------------------------------------------------------
// launchers (each returns hipError_t of the launch)
// --------------------------------------------------------------------------
// bank build
hipError_t launch_pool_keys(const Bank& bk, int doc0, int doc1, const void* route_vec,
                            hipStream_t s);
hipError_t launch_key_norms(const Bank& bk, int doc0, int doc1, hipStream_t s);
hipError_t launch_pool_kv(const Bank& bk, int doc0, int doc1, hipStream_t s);
hipError_t launch_store_kv(const Bank& bk, int doc0, int doc1, const void* k_raw,
                           const void* v_raw, hipStream_t s);
hipError_t launch_prepare_local(const Bank& bk, const void* k_raw, const void* v_raw, int n_seq,
                                int L, int pos0, void* k_loc, void* v_loc, hipStream_t s);
// queries: rotate at positions (pos0 + i*pos_step) and pre-scale by log2(e)/sqrt(d)
hipError_t launch_rope_queries(const Bank& bk, const void* q, int n_q, int h_q, int pos0,
                               int pos_step, void* q_rot, hipStream_t s);

// routing
hipError_t launch_route_scan(const Bank& bk, const float* q_route, int B, float* piecemax,
                             hipStream_t s);
// HBM read-rate probe: kStreamReadBlocks workgroups; out holds one word each
constexpr int kStreamReadBlocks = 4096;
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s);
// zero `bytes` (a multiple of 4) at a 4-byte-aligned device address with a
// kernel (no memset node if the caller captures the stream into a graph)
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_topk(const Bank& bk, const float* piecemax, int B, int k,
                       const uint32_t* exclude, uint32_t* exclude_out, int32_t* ids,
                       float* scores, uint64_t* keys, hipStream_t s);
size_t topk_scratch_keys(int N, int k);  // u64 keys per query launch_topk needs
hipError_t launch_block_mean(const Bank& bk, const void* route_tokens, int n_tok, int block,
                             float* q_out, hipStream_t s);
hipError_t launch_project(const float* out, const float* w, int B, int n_in, int d_r,
                          float* q_next, hipStream_t s);

// attention
struct AttnSources {
  const void* k;
  const void* v;
  const int64_t* off;
  const int32_t* len;
  int n;                          // entries in off / len
  const int64_t* voff = nullptr;  // V offsets (entries) when V rows are padded to
                                  // whole 64-entry tiles; NULL: V shares off
  float bias = 0.f;               // score bias of these entries, log2 units
};
// q: the raw queries [B][h_q][128] (dtype), rotated at q_pos inside the
// kernel, exactly as launch_rope_queries would
hipError_t launch_decode(const Bank& bk, const void* q, int q_pos, int B, int h_q,
                         const int32_t* ids, int k, const AttnSources& src, const void* k_loc,
                         const void* v_loc, int L_loc, int splits, float* part, float* out,
                         hipStream_t s);
hipError_t launch_prefill(const Bank& bk, const void* q_rot, int n_q, int h_q, const int32_t* ids,
                          int k, int block, const AttnSources& src, const void* k_loc,
                          const void* v_loc, int L_loc, int splits, float* part, float* out,
                          hipStream_t s);

// sizes of the attention partial buffers
size_t decode_partial_floats(int B, int h_kv, int G, int splits);
int decode_auto_splits(const Bank& bk, int B, int k, int L_loc, double doc_tiles);
size_t prefill_partial_floats(int n_q, int h_kv, int splits);
int prefill_auto_splits(const Bank& bk, int n_q, int k, int L_loc);
bool prefill_mfma_supported(const Bank& bk, int n_q, int h_q, int block);

}  // namespace msa
