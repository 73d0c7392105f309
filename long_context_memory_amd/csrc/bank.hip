// Bank build and position handling:
//   - routing keys: mean of every 256-token chunk of the per-token routing
//     vectors ("MSA架构" article, intelliparadigm.com, sections 2.1 and 3.1),
//     accumulated in float64, rounded once to the storage type, plus the
//     inverse norm of the rounded key;
//   - document K/V store: K rotated at document-local positions (document-wise
//     RoPE, "MSA" card, robocikowo.com, "Komponenty"), V laid out as
//     channel-major 64-token tiles, the blocks the attention kernels stream;
//   - local context: K rotated at global positions pos0 + j (global RoPE with
//     an offset, same card, "Pułapki implementacyjne");
//   - queries: rotated at their positions and pre-scaled by log2(e)/sqrt(d) so
//     the attention kernels can use exp2.
// RoPE is rotate-half: channel pairs (i, i + 64), angle pos * base^(-2i/128);
// angles and rotations are computed in float64.
#include "msa_internal.h"

namespace msa {
namespace {

// ---------------------------------------------------------------- pooling
// One workgroup per chunk.  Thread t owns 16-byte vector (t % NV) of every
// token row (NV vectors per row of h_r*128 elements) and tokens t/NV,
// t/NV + S, ... (S = 256/NV streams); float64 partial sums are combined in a
// fixed order through LDS.
template <typename T>
__global__ __launch_bounds__(256) void pool_keys_kernel(
    const T* __restrict__ rv, int64_t chunk_first, int h_r, int64_t C,
    T* __restrict__ kr, float* __restrict__ inv_norm) {
  constexpr int VE = 16 / sizeof(T);
  const int E = h_r * kD;
  const int NV = E / VE;
  const int S = 256 / NV;
  const int tid = threadIdx.x;
  const int v = tid % NV, stream = tid / NV;
  const int64_t c = chunk_first + blockIdx.x;
  const T* base = rv + (size_t)blockIdx.x * kChunk * E;

  double acc[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) acc[i] = 0.0;
  for (int t = stream; t < kChunk; t += S) {
    const T* p = base + (size_t)t * E + v * VE;
    T buf[VE];
    *reinterpret_cast<uint4*>(buf) = ld_nt(p);
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] += St<T>::load(buf[i]);
  }
  __shared__ double sums[256 * (16 / sizeof(uint16_t))];  // S * E <= 256 * VE doubles
  __shared__ double rnd[16 * kD];                          // rounded keys, h_r <= 16
#pragma unroll
  for (int i = 0; i < VE; ++i) sums[stream * E + v * VE + i] = acc[i];
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    double tot = 0.0;
    for (int s = 0; s < S; ++s) tot += sums[s * E + e];
    const T q = St<T>::store(tot / (double)kChunk);
    const int h = e / kD, i = e % kD;
    kr[((size_t)h * C + c) * kD + i] = q;
    rnd[e] = St<T>::load(q);
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  for (int h = wave; h < h_r; h += 4) {
    const double a = rnd[h * kD + lane], b = rnd[h * kD + 64 + lane];
    double ss = a * a + b * b;
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) inv_norm[(size_t)h * C + c] = ss > 0.0 ? (float)(1.0 / sqrt(ss)) : 0.0f;
  }
}

// inverse norms of given keys: one thread per (head, chunk) row
template <typename T>
__global__ __launch_bounds__(256) void key_norms_kernel(const T* __restrict__ kr, int64_t c0,
                                                        int64_t nc, int h_r, int64_t C,
                                                        float* __restrict__ inv_norm) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nc * h_r) return;
  const int h = (int)(idx / nc);
  const int64_t c = c0 + idx % nc;
  const T* row = kr + ((size_t)h * C + c) * kD;
  double ss = 0.0;
  for (int i = 0; i < kD; ++i) {
    const double x = St<T>::load(row[i]);
    ss += x * x;
  }
  inv_norm[(size_t)h * C + c] = ss > 0.0 ? (float)(1.0 / sqrt(ss)) : 0.0f;
}

// ---------------------------------------------------------------- K rotation
// Tiles of 64 tokens.  Bank mode: the input slice starts at a document start
// and documents are multiples of 256 tokens, so a tile lies inside one
// document; its document is found by binary search.  Local mode: tile ->
// (sequence, offset) with sequences of L tokens.
struct KLayout {
  int mode;                 // 0 bank, 1 local
  // bank
  const int64_t* tok_off;   // device [N+1]
  const int64_t* kv_off;    // device [N]
  const int32_t* doc_len;   // device [N]
  int doc0, doc1;
  int64_t slice_tok0;       // tok_off[doc0]
  // local
  int L, pos0, tiles_per_seq;
  int h_kv;
};

struct TileInfo {
  int64_t in_row0;   // first input row of the tile
  int64_t out_base;  // element offset of [0][0][0] of the segment in the output
  int seg_len;       // tokens in the segment (output row length)
  int t0;            // token offset of the tile inside the segment
  int pos_base;      // position of token 0 of the segment
  int n_valid;       // valid tokens in this tile
};

__device__ __forceinline__ TileInfo tile_info(const KLayout& ly, int tile) {
  TileInfo ti;
  if (ly.mode == 0) {
    const int64_t tok = ly.slice_tok0 + (int64_t)tile * kAttnTile;
    int lo = ly.doc0, hi = ly.doc1 - 1;  // last doc with tok_off <= tok
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ly.tok_off[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    ti.in_row0 = tok - ly.slice_tok0;
    ti.seg_len = ly.doc_len[lo];
    ti.t0 = (int)(tok - ly.tok_off[lo]);
    ti.out_base = ly.kv_off[lo] * ly.h_kv * kD;
    ti.pos_base = 0;
    ti.n_valid = kAttnTile;
  } else {
    const int s = tile / ly.tiles_per_seq;
    ti.t0 = (tile % ly.tiles_per_seq) * kAttnTile;
    ti.seg_len = ly.L;
    ti.in_row0 = (int64_t)s * ly.L + ti.t0;
    ti.out_base = (int64_t)s * ly.h_kv * ly.L * kD;
    ti.pos_base = ly.pos0;
    ti.n_valid = min(kAttnTile, ly.L - ti.t0);
  }
  return ti;
}

// One workgroup per tile.  Thread (token t, channel group g) holds the sines
// and cosines of pairs 8g .. 8g+7 at t's position (computed once, used for
// every head) and moves 16-byte vectors: channels 8g.. and 64 + 8g.. of each
// head's row.  A wave's 64 lanes cover 8 tokens x 8 groups.
template <typename T>
__global__ __launch_bounds__(256) void rotate_k_kernel(const T* __restrict__ in,
                                                       T* __restrict__ out, KLayout ly,
                                                       const double* __restrict__ inv_freq) {
  constexpr int VE = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int NG = 64 / VE;         // vectors per half row
  const TileInfo ti = tile_info(ly, blockIdx.x);
  for (int u = threadIdx.x; u < kAttnTile * NG; u += 256) {
    const int tt = u / NG, g = u % NG;
    if (tt >= ti.n_valid) break;  // u grows with tt
    const int t = ti.t0 + tt;
    double cs[VE], sn[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) sincos((double)(ti.pos_base + t) * inv_freq[g * VE + e], &sn[e], &cs[e]);
    const T* src = in + (size_t)(ti.in_row0 + tt) * ly.h_kv * kD + g * VE;
    T* dst0 = out + ti.out_base + (size_t)t * kD + g * VE;
    for (int h = 0; h < ly.h_kv; ++h) {
      T x1[VE], x2[VE], y1[VE], y2[VE];
      *reinterpret_cast<uint4*>(x1) = *reinterpret_cast<const uint4*>(src + h * kD);
      *reinterpret_cast<uint4*>(x2) = *reinterpret_cast<const uint4*>(src + h * kD + 64);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const double a = St<T>::load(x1[e]), b = St<T>::load(x2[e]);
        y1[e] = St<T>::store(a * cs[e] - b * sn[e]);
        y2[e] = St<T>::store(b * cs[e] + a * sn[e]);
      }
      T* dst = dst0 + (size_t)h * ti.seg_len * kD;
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(y1);
      *reinterpret_cast<uint4*>(dst + 64) = *reinterpret_cast<const uint4*>(y2);
    }
  }
}

// ---------------------------------------------------------------- V transpose
// One workgroup per (tile of 64 tokens, head): [64 tokens][128] -> the tile's
// channel-major block [128][64] (tokens past the end of a local sequence are
// written as zeros).  16-byte vectors in and out: rows are read as 16
// vectors of 8 (bf16) channels, staged in LDS token-major, and each output
// vector gathers 8 consecutive tokens of one channel.
template <typename T>
__global__ __launch_bounds__(256) void transpose_v_kernel(const T* __restrict__ in,
                                                          T* __restrict__ out, KLayout ly) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int NV = kD / VE;  // vectors per token row
  const int h = blockIdx.y;
  const TileInfo ti = tile_info(ly, blockIdx.x);
  size_t blk;  // element offset of the tile block
  if (ly.mode == 0) {
    blk = (size_t)ti.out_base + ((size_t)h * ti.seg_len + ti.t0) * kD;
  } else {
    const int s = blockIdx.x / ly.tiles_per_seq, m = blockIdx.x % ly.tiles_per_seq;
    blk = (((size_t)s * ly.h_kv + h) * ly.tiles_per_seq + m) * kAttnTile * kD;
  }
  __shared__ __attribute__((aligned(16))) T tile[kAttnTile][kD + VE];
  for (int u = threadIdx.x; u < kAttnTile * NV; u += 256) {
    const int t = u / NV, c = u % NV;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < ti.n_valid)
      v = *reinterpret_cast<const uint4*>(in + (size_t)(ti.in_row0 + t) * ly.h_kv * kD + h * kD +
                                          c * VE);
    *reinterpret_cast<uint4*>(&tile[t][c * VE]) = v;
  }
  __syncthreads();
  T* dst = out + blk;
  constexpr int NT = kAttnTile / VE;  // output vectors per channel row
  for (int u = threadIdx.x; u < kD * NT; u += 256) {
    const int i = u / NT, t0 = (u % NT) * VE;
    T w[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) w[e] = tile[t0 + e][i];
    *reinterpret_cast<uint4*>(dst + (size_t)i * kAttnTile + t0) = *reinterpret_cast<const uint4*>(w);
  }
}

// ---------------------------------------------------------------- queries
// Workgroup = kRopeRows query rows.  First the rows' angles: one (row, pair)
// per thread, sine and cosine in float64 into LDS; then every (row, head,
// group of pairs) moves 16-byte vectors of channels 8g.. and 64 + 8g.. (bf16).
constexpr int kRopeRows = 4;  // 4 rows x 64 pairs = one angle per thread

template <typename T>
__global__ __launch_bounds__(256) void rope_queries_kernel(const T* __restrict__ q, int n_q,
                                                           int h_q, int pos0, int pos_step,
                                                           const double* __restrict__ inv_freq,
                                                           double scale, T* __restrict__ out) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int NG = 64 / VE;
  __shared__ double s_cs[kRopeRows][64], s_sn[kRopeRows][64];
  const int r0 = blockIdx.x * kRopeRows;
  {
    const int r = threadIdx.x >> 6, pair = threadIdx.x & 63;
    const int i = min(r0 + r, n_q - 1);
    sincos((double)(pos0 + (int64_t)i * pos_step) * inv_freq[pair], &s_sn[r][pair], &s_cs[r][pair]);
  }
  __syncthreads();
  const int rows = min(kRopeRows, n_q - r0);
  for (int u = threadIdx.x; u < rows * h_q * NG; u += 256) {
    const int g = u % NG, h = (u / NG) % h_q, r = u / (NG * h_q);
    const size_t o = ((size_t)(r0 + r) * h_q + h) * kD + g * VE;
    T x1[VE], x2[VE], y1[VE], y2[VE];
    *reinterpret_cast<uint4*>(x1) = *reinterpret_cast<const uint4*>(q + o);
    *reinterpret_cast<uint4*>(x2) = *reinterpret_cast<const uint4*>(q + o + 64);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const double cs = s_cs[r][g * VE + e], sn = s_sn[r][g * VE + e];
      const double a = St<T>::load(x1[e]), b = St<T>::load(x2[e]);
      y1[e] = St<T>::store((a * cs - b * sn) * scale);
      y2[e] = St<T>::store((b * cs + a * sn) * scale);
    }
    *reinterpret_cast<uint4*>(out + o) = *reinterpret_cast<const uint4*>(y1);
    *reinterpret_cast<uint4*>(out + o + 64) = *reinterpret_cast<const uint4*>(y2);
  }
}

KLayout bank_layout(const Bank& bk, int doc0, int doc1) {
  KLayout ly{};
  ly.mode = 0;
  ly.tok_off = bk.d_tok_off;
  ly.kv_off = bk.d_kv_off;
  ly.doc_len = bk.d_doc_len;
  ly.doc0 = doc0;
  ly.doc1 = doc1;
  ly.slice_tok0 = bk.tok_off[doc0];
  ly.h_kv = bk.desc.h_kv;
  return ly;
}

}  // namespace

hipError_t launch_pool_keys(const Bank& bk, int doc0, int doc1, const void* rv, hipStream_t s) {
  const int64_t c0 = bk.chunk_off[doc0], nc = bk.chunk_off[doc1] - c0;
  if (nc == 0) return hipSuccess;
  if (bk.desc.dtype == MSA_BF16)
    hipLaunchKernelGGL(pool_keys_kernel<uint16_t>, dim3((unsigned)nc), dim3(256), 0, s,
                       (const uint16_t*)rv, c0, bk.desc.h_r, bk.chunk_stride,
                       (uint16_t*)bk.desc.kr, bk.desc.inv_norm);
  else
    hipLaunchKernelGGL(pool_keys_kernel<float>, dim3((unsigned)nc), dim3(256), 0, s,
                       (const float*)rv, c0, bk.desc.h_r, bk.chunk_stride, (float*)bk.desc.kr,
                       bk.desc.inv_norm);
  return hipGetLastError();
}

hipError_t launch_key_norms(const Bank& bk, int doc0, int doc1, hipStream_t s) {
  const int64_t c0 = bk.chunk_off[doc0], nc = bk.chunk_off[doc1] - c0;
  if (nc == 0) return hipSuccess;
  const int64_t rows = nc * bk.desc.h_r;
  const unsigned grid = (unsigned)((rows + 255) / 256);
  if (bk.desc.dtype == MSA_BF16)
    hipLaunchKernelGGL(key_norms_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                       (const uint16_t*)bk.desc.kr, c0, nc, bk.desc.h_r, bk.chunk_stride,
                       bk.desc.inv_norm);
  else
    hipLaunchKernelGGL(key_norms_kernel<float>, dim3(grid), dim3(256), 0, s,
                       (const float*)bk.desc.kr, c0, nc, bk.desc.h_r, bk.chunk_stride,
                       bk.desc.inv_norm);
  return hipGetLastError();
}

namespace {

// Compressed memory: entry j of document n is the mean of the document's
// chunk j of stored K (already rotated at document positions) and of V
// (intelliparadigm.com, section 3.1: chunk-mean pooling of the KV cache),
// accumulated in float64 and rounded once.  One workgroup per (chunk, KV
// head).  K rows are read as 16-byte vectors: thread (vector column, token
// group) sums every 16th token of the chunk; V (channel-major 64-token
// tiles) as 16-byte runs of 8 tokens: thread (channel, half) sums two of the
// chunk's four tiles.  Partial sums are combined in a fixed order in LDS.
template <typename T>
__global__ __launch_bounds__(256) void pool_kv_kernel(
    const T* __restrict__ ks, const T* __restrict__ vs, const int32_t* __restrict__ chunk_doc,
    const int32_t* __restrict__ doc_len, const int64_t* __restrict__ kv_off,
    const int64_t* __restrict__ tok_off, const int64_t* __restrict__ pool_voff, int h_kv,
    int64_t c0, T* __restrict__ pk, T* __restrict__ pv) {
  constexpr int VE = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int NV = kD / VE;         // vectors per K row
  constexpr int NTG = 256 / NV;       // token groups
  const int64_t c = c0 + blockIdx.x;
  const int h = blockIdx.y;
  const int n = chunk_doc[c];
  const int64_t L = doc_len[n];
  const int64_t P = L / kChunk;
  const int64_t cfirst = tok_off[n] / kChunk;
  const int64_t j = c - cfirst;  // entry (chunk) within the document
  const int tid = threadIdx.x;
  const int64_t base = (kv_off[n] * h_kv + (int64_t)h * L) * kD;  // this head's block
  const int64_t tok0 = j * kChunk;  // first token of the chunk within the document

  const int cv = tid % NV, tg = tid / NV;
  double ak[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) ak[e] = 0.0;
  const T* kb = ks + base + tok0 * kD + cv * VE;
  for (int t = tg; t < kChunk; t += NTG) {
    T x[VE];
    *reinterpret_cast<uint4*>(x) = ld_nt(kb + (size_t)t * kD);
#pragma unroll
    for (int e = 0; e < VE; ++e) ak[e] += St<T>::load(x[e]);
  }
  const int d = tid & (kD - 1), half = tid >> 7;
  double av = 0.0;
  for (int q = 2 * half; q < 2 * half + 2; ++q) {
    const T* vb = vs + base + (tok0 / kAttnTile + q) * kD * kAttnTile + d * kAttnTile;
    for (int w = 0; w < kAttnTile / VE; ++w) {
      T x[VE];
      *reinterpret_cast<uint4*>(x) = ld_nt(vb + w * VE);
#pragma unroll
      for (int e = 0; e < VE; ++e) av += St<T>::load(x[e]);
    }
  }
  __shared__ double s_k[NTG][kD];
  __shared__ double s_v[2][kD];
#pragma unroll
  for (int e = 0; e < VE; ++e) s_k[tg][cv * VE + e] = ak[e];
  s_v[half][d] = av;
  __syncthreads();
  if (tid < kD) {
    double sk = 0.0;
    for (int g = 0; g < NTG; ++g) sk += s_k[g][tid];
    const double sv = s_v[0][tid] + s_v[1][tid];
    pk[(cfirst * h_kv + (int64_t)h * P + j) * kD + tid] = St<T>::store(sk / (double)kChunk);
    const int64_t Pp = (P + kAttnTile - 1) / kAttnTile * kAttnTile;
    pv[(pool_voff[n] * h_kv + (int64_t)h * Pp) * kD + (j / kAttnTile) * kD * kAttnTile +
       tid * kAttnTile + j % kAttnTile] = St<T>::store(sv / (double)kChunk);
  }
}

}  // namespace

hipError_t launch_pool_kv(const Bank& bk, int doc0, int doc1, hipStream_t s) {
  const int64_t c0 = bk.chunk_off[doc0], nc = bk.chunk_off[doc1] - c0;
  if (nc == 0) return hipSuccess;
  const size_t esz = dtype_size(bk.desc.dtype);
  const size_t row = (size_t)bk.desc.h_kv * kD * esz;
  // V rows past a document's last entry (tile padding) are zero
  hipError_t e = launch_fill_zero((char*)bk.pool_v + (size_t)bk.pool_voff[doc0] * row,
                                 (size_t)(bk.pool_voff[doc1] - bk.pool_voff[doc0]) * row, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)nc, (unsigned)bk.desc.h_kv);
  if (bk.desc.dtype == MSA_BF16)
    hipLaunchKernelGGL(pool_kv_kernel<uint16_t>, grid, dim3(256), 0, s,
                       (const uint16_t*)bk.desc.k_store, (const uint16_t*)bk.desc.v_store,
                       bk.d_chunk_doc, bk.d_doc_len, bk.d_kv_off, bk.d_tok_off, bk.d_pool_voff,
                       bk.desc.h_kv, c0, (uint16_t*)bk.pool_k, (uint16_t*)bk.pool_v);
  else
    hipLaunchKernelGGL(pool_kv_kernel<float>, grid, dim3(256), 0, s,
                       (const float*)bk.desc.k_store, (const float*)bk.desc.v_store,
                       bk.d_chunk_doc, bk.d_doc_len, bk.d_kv_off, bk.d_tok_off, bk.d_pool_voff,
                       bk.desc.h_kv, c0, (float*)bk.pool_k, (float*)bk.pool_v);
  return hipGetLastError();
}

hipError_t launch_store_kv(const Bank& bk, int doc0, int doc1, const void* k_raw,
                           const void* v_raw, hipStream_t s) {
  const int64_t ntok = bk.tok_off[doc1] - bk.tok_off[doc0];
  if (ntok == 0) return hipSuccess;
  const unsigned tiles = (unsigned)(ntok / kAttnTile);
  const KLayout ly = bank_layout(bk, doc0, doc1);
  if (bk.desc.dtype == MSA_BF16) {
    hipLaunchKernelGGL(rotate_k_kernel<uint16_t>, dim3(tiles), dim3(256), 0, s,
                       (const uint16_t*)k_raw, (uint16_t*)bk.desc.k_store, ly, bk.d_inv_freq);
    hipLaunchKernelGGL(transpose_v_kernel<uint16_t>, dim3(tiles, bk.desc.h_kv), dim3(256), 0, s,
                       (const uint16_t*)v_raw, (uint16_t*)bk.desc.v_store, ly);
  } else {
    hipLaunchKernelGGL(rotate_k_kernel<float>, dim3(tiles), dim3(256), 0, s,
                       (const float*)k_raw, (float*)bk.desc.k_store, ly, bk.d_inv_freq);
    hipLaunchKernelGGL(transpose_v_kernel<float>, dim3(tiles, bk.desc.h_kv), dim3(256), 0, s,
                       (const float*)v_raw, (float*)bk.desc.v_store, ly);
  }
  return hipGetLastError();
}

hipError_t launch_prepare_local(const Bank& bk, const void* k_raw, const void* v_raw, int n_seq,
                                int L, int pos0, void* k_loc, void* v_loc, hipStream_t s) {
  KLayout ly{};
  ly.mode = 1;
  ly.L = L;
  ly.pos0 = pos0;
  ly.tiles_per_seq = (L + kAttnTile - 1) / kAttnTile;
  ly.h_kv = bk.desc.h_kv;
  const unsigned tiles = (unsigned)(n_seq * ly.tiles_per_seq);
  if (tiles == 0) return hipSuccess;
  if (bk.desc.dtype == MSA_BF16) {
    hipLaunchKernelGGL(rotate_k_kernel<uint16_t>, dim3(tiles), dim3(256), 0, s,
                       (const uint16_t*)k_raw, (uint16_t*)k_loc, ly, bk.d_inv_freq);
    hipLaunchKernelGGL(transpose_v_kernel<uint16_t>, dim3(tiles, bk.desc.h_kv), dim3(256), 0, s,
                       (const uint16_t*)v_raw, (uint16_t*)v_loc, ly);
  } else {
    hipLaunchKernelGGL(rotate_k_kernel<float>, dim3(tiles), dim3(256), 0, s,
                       (const float*)k_raw, (float*)k_loc, ly, bk.d_inv_freq);
    hipLaunchKernelGGL(transpose_v_kernel<float>, dim3(tiles, bk.desc.h_kv), dim3(256), 0, s,
                       (const float*)v_raw, (float*)v_loc, ly);
  }
  return hipGetLastError();
}

hipError_t launch_rope_queries(const Bank& bk, const void* q, int n_q, int h_q, int pos0,
                               int pos_step, void* q_rot, hipStream_t s) {
  if (n_q == 0) return hipSuccess;
  const double scale = 1.4426950408889634 / sqrt((double)kD);  // log2(e) / sqrt(d)
  const unsigned grid = (unsigned)((n_q + kRopeRows - 1) / kRopeRows);
  if (bk.desc.dtype == MSA_BF16)
    hipLaunchKernelGGL(rope_queries_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                       (const uint16_t*)q, n_q, h_q, pos0, pos_step, bk.d_inv_freq, scale,
                       (uint16_t*)q_rot);
  else
    hipLaunchKernelGGL(rope_queries_kernel<float>, dim3(grid), dim3(256), 0, s,
                       (const float*)q, n_q, h_q, pos0, pos_step, bk.d_inv_freq, scale,
                       (float*)q_rot);
  return hipGetLastError();
}

}  // namespace msa
