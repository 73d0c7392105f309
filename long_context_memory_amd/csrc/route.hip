// Routing: cosine scoring of router queries against every routing key, the
// per-document max over chunks and mean over router heads, and top-k
// document selection ("MSA" card, robocikowo.com, "Komponenty", router;
// "MSA架构" article, intelliparadigm.com, section 2.1).  Also the block-mean
// router queries of the blocked prefill and the Memory Interleave projection
// that forms the next hop's router query.
//
// route_scan produces, per (query, router head), the maximum cosine of every
// "piece" -- a run of one document's chunks inside a tile of 64 chunks.
// top-k later takes the max over a document's pieces and the mean over
// heads, so no atomics and no initialisation are needed.
#include <algorithm>
#include <atomic>

#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kQPerWave = 16;    // queries a wave scores per pass (64 per workgroup pass)
constexpr int kScanWgPerCu = 3;  // resident matrix-core scan workgroups per compute unit
// LDS buffer of the matrix-core scan's piece maxima, written out in bulk so
// that no store waits inside the tile loop (sized so that three workgroups
// fit in 160 KiB of LDS)
constexpr int kScanOutFloats = 4608, kScanOutTiles = 128;
static_assert(kScanOutFloats >= 64 * 64, "one tile's block must fit");

// Workgroup barrier that waits for this wave's LDS operations only (a
// __syncthreads() would also wait for every global load in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Routing scan for float32 keys.  Workgroup = one (tile of 64 chunks, router
// head); the tile's key rows are staged once through LDS and every wave takes
// all 64 rows, one per lane.  The batch's router queries for this head are
// staged in LDS and read back as broadcasts.  Every global load of the
// workgroup (key rows, queries, chunk table) is issued before the first LDS
// store, so a launch costs one memory round trip.  Wave w scores queries w,
// w+4, ... with fp32 FMAs; for each, lane c holds the cosine of chunk c and a
// segmented max across lanes folds the tile's runs of equal documents
// ("pieces") into per-document maxima, written by the lane that starts each
// run.
__global__ __launch_bounds__(256) void route_scan_kernel(
    const float* __restrict__ kr, const float* __restrict__ inv_norm, const float* __restrict__ q,
    int B, int bg, int h_r, int64_t C, int64_t Cs, const int32_t* __restrict__ chunk_doc,
    const int32_t* __restrict__ tile_piece0, int P, float* __restrict__ piecemax) {
  // queries bg .. bg + min(64, B - bg) - 1 (one launch per group of 64)
  constexpr int RowF = kD + 4;  // 32-bit words per staged row (+16 B pad)
  constexpr int QW = kD;        // words per staged query
  __shared__ __attribute__((aligned(16))) uint32_t s_rows[64 * RowF];
  __shared__ __attribute__((aligned(16))) uint32_t s_q[64 * QW];
  __shared__ float s_iq[64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x, h = blockIdx.y;
  const int64_t c0 = (int64_t)tile * kRouteTile;
  const int nc = (int)min((int64_t)kRouteTile, C - c0);
  const int npass = min(64, B - bg);
  const float* rows = kr + ((size_t)h * Cs + c0) * kD;  // Cs: rows per head (capacity)

  // ---- every global load first: the tile (64 rows x VPR 16-byte vectors;
  // rows past the end of the bank read the last row and are stored as zero),
  // this pass's queries (64 x 32 float4, rows past the pass skipped) and the
  // tile's chunk table
  constexpr int VPR = kD / 4;
  constexpr int NLD = 64 * VPR / 256;
  uint4 v[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int f = u * 256 + threadIdx.x;
    const int row = f / VPR, col = f % VPR;
    v[u] = *reinterpret_cast<const uint4*>(rows + ((size_t)min(row, nc - 1) * VPR + col) * 4);
  }
  // query slice u covers queries 8u .. 8u + 7 (workgroup-uniform bound)
  const int nslice = (npass + 7) / 8;
  float4 qv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (u >= nslice) break;
    const int f = u * 256 + threadIdx.x;
    const int qi = f / (kD / 4), col = f % (kD / 4);
    qv[u] = qi < npass ? *reinterpret_cast<const float4*>(q + ((size_t)(bg + qi) * h_r + h) * kD +
                                                          col * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int my_doc = lane < nc ? chunk_doc[c0 + lane] : -1;
  const float inv_k = lane < nc ? inv_norm[(size_t)h * Cs + c0 + lane] : 0.0f;
  const int piece0 = tile_piece0[tile];

#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int f = u * 256 + threadIdx.x;
    const int row = f / VPR, col = f % VPR;
    *reinterpret_cast<uint4*>(s_rows + row * RowF + col * 4) =
        row < nc ? v[u] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (u >= nslice) break;
    const int f = u * 256 + threadIdx.x;
    const int qi = f / (kD / 4), col = f % (kD / 4);
    *reinterpret_cast<float4*>(s_q + qi * QW + col * 4) = qv[u];
    // partial squared norm of the float32 query
    float ss = qv[u].x * qv[u].x + qv[u].y * qv[u].y + qv[u].z * qv[u].z + qv[u].w * qv[u].w;
    // 32 consecutive threads hold one query row: reduce within the 32
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    ss += __shfl_xor(ss, 8, 64);
    ss += __shfl_xor(ss, 16, 64);
    if (col == 0) s_iq[qi] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.0f;
  }

  // document runs inside the tile (same for every wave): this lane's run
  // ends before lane `end`; a run's first lane writes piece piece0 + seg
  const int prev_doc = __shfl_up(my_doc, 1, 64);
  const bool start = lane < nc && (lane == 0 || my_doc != prev_doc);
  const uint64_t starts = __ballot(start);
  const uint64_t later = lane == 63 ? 0 : starts & (~0ull << (lane + 1));
  const int end = later ? __builtin_ctzll(later) : nc;
  const int seg = __builtin_popcountll(starts & ((1ull << lane) - 1));
  __syncthreads();

  // this lane's key row (32 x uint4)
  uint4 kw[VPR];
#pragma unroll
  for (int c = 0; c < VPR; ++c) kw[c] = *reinterpret_cast<const uint4*>(s_rows + lane * RowF + c * 4);

  // this wave's queries: bg + wave + 4*j, j < nq
  const int nq = max(0, min(kQPerWave, (npass - wave + 3) / 4));
#pragma unroll 1
  for (int j = 0; j < nq; ++j) {
    const int qi = wave + 4 * j;
    const uint32_t* qj = s_q + qi * QW;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int c = 0; c < 32; c += 2) {
      const float4 x0 = *reinterpret_cast<const float4*>(qj + c * 4);
      const float4 x1 = *reinterpret_cast<const float4*>(qj + c * 4 + 4);
      a0 = fmaf(__uint_as_float(kw[c].x), x0.x, a0); a1 = fmaf(__uint_as_float(kw[c].y), x0.y, a1);
      a0 = fmaf(__uint_as_float(kw[c].z), x0.z, a0); a1 = fmaf(__uint_as_float(kw[c].w), x0.w, a1);
      a2 = fmaf(__uint_as_float(kw[c + 1].x), x1.x, a2); a3 = fmaf(__uint_as_float(kw[c + 1].y), x1.y, a3);
      a2 = fmaf(__uint_as_float(kw[c + 1].z), x1.z, a2); a3 = fmaf(__uint_as_float(kw[c + 1].w), x1.w, a3);
    }
    // segmented max over [lane, end): after the step with offset o a lane
    // holds the max of [lane, min(lane + 2o, end)); then the query norm
    // (x -> x * s with s > 0 is monotone, so it commutes with the max)
    float m = ((a0 + a1) + (a2 + a3)) * inv_k;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float u = __shfl_down(m, o, 64);
      if (lane + o < end) m = fmaxf(m, u);
    }
    if (start) piecemax[((size_t)(bg + qi) * h_r + h) * P + piece0 + seg] = m * s_iq[qi];
  }
}

// Routing scan on the matrix cores, for bf16 keys: the scan is a dense
// contraction ([queries x 128] times [128 x chunks]) that would otherwise be
// VALU-bound, and even a pass of a few queries leaves the matrix cores far
// from their limit.  v_mfma_f32_32x32x16_bf16 with the float32 query split
// into two bfloat16 terms, q = hi + lo + r with |r| <= 2^-17 |q| (two MFMAs
// per 16-channel step, fp32 accumulation): the products are those of the
// bf16 key with the float32 query up to that remainder.
//
// Persistent workgroups: grid (g, router head), workgroup x takes tiles x,
// x + g, x + 2g, ...; its query fragments are loaded and split once, and the next
// tile's key rows, chunk table entries, norms and first piece are loaded into
// registers while the current tile is scored, so the key stream stays in
// flight.  Per tile: the rows go to LDS; wave w computes one 32x32 block of
// cosines (chunks 32*(w&1).., queries 32*(w>>1)..) into LDS as [query][chunk]
// rows; then wave w folds queries w, w+4, ...: lane c holds chunk c's cosine
// times 1/||k_c||, and a segmented max over the tile's runs of equal
// documents ("pieces") -- DPP shifts inside each 16-lane row, then the three
// later rows' leading values read into scalars -- leaves each piece's maximum
// in the run's first lane.  Scaled by 1/||q||, it goes to an LDS buffer that
// is written out once per workgroup (earlier only if it fills), so that no
// store is in flight when a wave waits for the next tile's keys.
typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x16_t __attribute__((ext_vector_type(16)));

// lane i takes lane i+O's value within its row of 16 lanes (0 past the row);
// every lane of the wave must execute it, since a move reads its source
// lane's register
template <int O>
__device__ __forceinline__ float row_down(float m) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x100 + O, 0xf, 0xf, true));
}

__global__ __launch_bounds__(256) void route_scan_mfma_kernel(
    const uint16_t* __restrict__ kr, const float* __restrict__ inv_norm,
    const float* __restrict__ q, int B, int bg, int h_r,
    int64_t C, int64_t Cs, const int32_t* __restrict__ chunk_doc,
    const int32_t* __restrict__ tile_piece0, int P, float* __restrict__ piecemax) {
  constexpr int RowF = kD / 2 + 4;  // 32-bit words per staged key row (+16 B pad)
  constexpr int NLD = 64 * 16 / 256;  // 16-byte vectors of a tile per thread
  __shared__ __attribute__((aligned(16))) uint32_t s_rows[64 * RowF];
  __shared__ float s_cos[64 * 65];  // [query][chunk], rows padded to 65
  __shared__ float s_iq[64];
  // piece maxima of the tiles scored since the last flush: tile b's block is
  // [query][piece], its first piece and piece count are in the table
  __shared__ float s_out[kScanOutFloats];
  __shared__ int s_tp0[kScanOutTiles], s_tnp[kScanOutTiles];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
  const int h = blockIdx.y;
  const int ntiles = (int)((C + kRouteTile - 1) / kRouteTile);
  const int npass = min(64, B - bg);
  const int cb = wave & 1, qb = wave >> 1;
  const bool busy = 32 * qb < npass;  // wave-uniform
  const uint16_t* head = kr + (size_t)h * Cs * kD;  // Cs: rows per head (capacity)
  const float* head_ik = inv_norm + (size_t)h * Cs;

  // this wave's query fragments: query 32*qb + l32, channels 16*kk + 8*hl ..
  // +7, as bfloat16 pairs of the hi terms and of the lo terms; and the
  // pass's 1/||q|| (this lane's 64 squares plus its partner half's)
  uint4 qh[8], ql[8];
  {
    const int qi = 32 * qb + l32;
    const bool qok = busy && qi < npass;
    const float* qrow = q + ((size_t)(bg + (qok ? qi : 0)) * h_r + h) * kD + 8 * hl;
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const float4 a = qok ? *reinterpret_cast<const float4*>(qrow + 16 * kk) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 b = qok ? *reinterpret_cast<const float4*>(qrow + 16 * kk + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t h0 = f32_to_bf16(x[2 * e]), h1 = f32_to_bf16(x[2 * e + 1]);
        hi[e] = h0 | (h1 << 16);
        lo[e] = f32_to_bf16(x[2 * e] - __uint_as_float(h0 << 16)) |
                (f32_to_bf16(x[2 * e + 1] - __uint_as_float(h1 << 16)) << 16);
        ss = fmaf(x[2 * e], x[2 * e], ss);
        ss = fmaf(x[2 * e + 1], x[2 * e + 1], ss);
      }
      qh[kk] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      ql[kk] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    ss += __shfl_xor(ss, 32, 64);
    if (cb == 0 && hl == 0 && qok) s_iq[qi] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.0f;
  }

  // tile t's loads: 64 rows x 16 vectors (rows past the bank's end read the
  // last row and are stored as zero), lane's chunk table entry and norm
  uint4 v[NLD];
  int nd = -1, np0 = 0;
  float nik = 0.f;
  auto load = [&](int t) __attribute__((always_inline)) {
    const int64_t c0 = (int64_t)t * kRouteTile;
    const int nc = (int)min((int64_t)kRouteTile, C - c0);
    const uint16_t* rows = head + c0 * kD;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int f = u * 256 + threadIdx.x;
      const int row = f / 16, col = f % 16;
      v[u] = ld_nt(rows + ((size_t)min(row, nc - 1) * 16 + col) * 8);
    }
    nd = lane < nc ? chunk_doc[c0 + lane] : -1;
    nik = lane < nc ? head_ik[c0 + lane] : 0.f;
    np0 = tile_piece0[t];
  };
  // write the buffered piece maxima to their rows (each tile's block is a
  // contiguous run of pieces per query); every thread runs it, after a barrier
  int n_buf = 0, off_buf = 0;  // buffered tiles and floats (workgroup-uniform)
  auto flush = [&]() __attribute__((always_inline)) {
    int off = 0;
    for (int b = 0; b < n_buf; ++b) {
      const int p0 = s_tp0[b], np = s_tnp[b], n = npass * np;
      for (int i = threadIdx.x; i < n; i += 256) {
        const int qi = i / np;
        piecemax[((size_t)(bg + qi) * h_r + h) * P + p0 + (i - qi * np)] = s_out[off + i];
      }
      off += n;
    }
    n_buf = 0;
    off_buf = 0;
  };
  int tile = blockIdx.x;
  if (tile < ntiles) load(tile);
  while (tile < ntiles) {  // workgroup-uniform
    const int nc = (int)min((int64_t)kRouteTile, C - (int64_t)tile * kRouteTile);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int f = u * 256 + threadIdx.x;
      const int row = f / 16, col = f % 16;
      *reinterpret_cast<uint4*>(s_rows + row * RowF + col * 4) = row < nc ? v[u] : make_uint4(0, 0, 0, 0);
    }
    const int my_doc = nd, piece0 = np0;
    const float inv_k = nik;
    const int next = tile + (int)gridDim.x;
    if (next < ntiles) load(next);

    // document runs inside the tile (same for every wave): this lane's run
    // ends before lane `end`; a run's first lane writes piece piece0 + seg
    const int prev_doc = __shfl_up(my_doc, 1, 64);
    const bool start = lane < nc && (lane == 0 || my_doc != prev_doc);
    const uint64_t starts = __ballot(start);
    const uint64_t later = lane == 63 ? 0 : starts & (~0ull << (lane + 1));
    const int end = later ? __builtin_ctzll(later) : nc;
    const int seg = __builtin_popcountll(starts & ((1ull << lane) - 1));
    const int np = __builtin_popcountll(starts);  // pieces in this tile
    // (the barriers wait for LDS only: the next tile's loads stay in flight)
    lds_barrier();
    // the previous tiles' folds are complete: flush if this tile's block
    // would not fit (a tile's block, at most 64 x 64 floats, always fits)
    if (n_buf == kScanOutTiles || off_buf + npass * np > kScanOutFloats) flush();

    // ---- wave w: cosines of chunks 32*cb + row by queries 32*qb + column
    if (busy) {
      rf32x16_t acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
      const uint32_t* krow = s_rows + (32 * cb + l32) * RowF + 4 * hl;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const rbf16x8_t a = __builtin_bit_cast(rbf16x8_t, *reinterpret_cast<const uint4*>(krow + 8 * kk));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(rbf16x8_t, qh[kk]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(rbf16x8_t, ql[kk]), acc, 0, 0, 0);
      }
      // element e: chunk row 8*(e/4) + 4*hl + e%4 of the block, query column l32
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 32 * cb + 8 * (e >> 2) + 4 * hl + (e & 3);
        s_cos[(32 * qb + l32) * 65 + c] = acc[e];
      }
    }
    lds_barrier();

    // ---- wave w folds queries w, w+4, ...  In-row stage: after the shift
    // by o a lane holds the max over [lane, min(lane + 2o, end, row end));
    // then the rows after this lane's that its run reaches add their first
    // lane's value (x -> x / ||q|| is monotone, so it is applied last).
    const int lim = min(end, (lane | 15) + 1);
    const bool c1 = lane + 1 < lim, c2 = lane + 2 < lim, c4 = lane + 4 < lim, c8 = lane + 8 < lim;
    const bool x1 = lane < 16 && 16 < end, x2 = lane < 32 && 32 < end, x3 = lane < 48 && 48 < end;
    const int nq = max(0, min(16, (npass - wave + 3) / 4));
    for (int j = 0; j < nq; ++j) {
      const int qi = wave + 4 * j;
      float m = s_cos[qi * 65 + lane] * inv_k;
      float t = row_down<1>(m);
      m = c1 && t > m ? t : m;
      t = row_down<2>(m);
      m = c2 && t > m ? t : m;
      t = row_down<4>(m);
      m = c4 && t > m ? t : m;
      t = row_down<8>(m);
      m = c8 && t > m ? t : m;
      const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16));
      const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32));
      const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48));
      m = x1 && r1 > m ? r1 : m;
      m = x2 && r2 > m ? r2 : m;
      m = x3 && r3 > m ? r3 : m;
      if (start) s_out[off_buf + qi * np + seg] = m * s_iq[qi];
    }
    if (threadIdx.x == 0) {
      s_tp0[n_buf] = piece0;
      s_tnp[n_buf] = np;
    }
    ++n_buf;
    off_buf += npass * np;
    tile = next;
  }
  lds_barrier();
  flush();
}

// ---------------------------------------------------------------- top-k
// Document n's score is the mean over router heads of the max over its
// pieces; its key is (order-preserving score bits << 32 | ~n): a larger key
// is a higher score, and among equal scores the lower id.  Key 0 marks an
// excluded document (or no document).  Keys are unique, so a key's rank is
// the number of larger keys.
//
// Selection runs in levels of the same kernel: every workgroup takes 256
// keys (level 0: computed from the routing partials; later levels: the
// previous level's lists), ranks each key by counting the larger keys of its
// group in LDS, and writes the k best in rank order.  Each level shrinks the
// candidates by 256/k; the level that sees at most 256 keys writes the ids.
constexpr int kTopkGroup = 256;

__device__ __forceinline__ uint64_t doc_key(const float* __restrict__ pm, int h_r, int P,
                                            const int32_t* __restrict__ doc_piece0,
                                            const uint32_t* excl_row, int n) {
  if (excl_row && ((excl_row[n >> 5] >> (n & 31)) & 1u)) return 0;
  const int p0 = doc_piece0[n], p1 = doc_piece0[n + 1];
  float m[16];
#pragma unroll
  for (int h = 0; h < 16; ++h)  // independent loads (heads past h_r re-read head 0)
    m[h] = pm[(size_t)(h < h_r ? h : 0) * P + p0];
  for (int p = p0 + 1; p < p1; ++p)
#pragma unroll
    for (int h = 0; h < 16; ++h) m[h] = fmaxf(m[h], pm[(size_t)(h < h_r ? h : 0) * P + p]);
  float s = 0.f;
#pragma unroll
  for (int h = 0; h < 16; ++h)
    if (h < h_r) s += m[h];
  return ((uint64_t)float_order_key(s / (float)h_r) << 32) | (uint64_t)(~(uint32_t)n);
}

struct TopkLevel {
  // level 0 input (keys from routing partials)
  const float* piecemax;
  int h_r, N, P;
  const int32_t* doc_piece0;
  const uint32_t* exclude;
  int W;
  // later levels: candidate lists [B][M_in]
  const uint64_t* in;
  int M_in;
  int k;
  // output: next lists [B][groups * k], or ids/scores when final
  uint64_t* out;
  int final_level;
  int32_t* ids;
  float* scores;
  uint32_t* exclude_out;
};

__global__ __launch_bounds__(kTopkGroup) void topk_level_kernel(TopkLevel a) {
  __shared__ __attribute__((aligned(16))) uint64_t s_key[kTopkGroup];
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int groups = gridDim.x;
  const int i = g * kTopkGroup + t;
  uint64_t key = 0;
  if (a.in == nullptr) {
    if (i < a.N)
      key = doc_key(a.piecemax + (size_t)b * a.h_r * a.P, a.h_r, a.P, a.doc_piece0,
                    a.exclude ? a.exclude + (size_t)b * a.W : nullptr, i);
  } else if (i < a.M_in) {
    key = a.in[(size_t)b * a.M_in + i];
  }
  s_key[t] = key;
  if (a.final_level) {
    if (t < a.k) {
      a.ids[(size_t)b * a.k + t] = -1;
      a.scores[(size_t)b * a.k + t] = -INFINITY;
    }
  } else if (t < a.k) {
    a.out[((size_t)b * groups + g) * a.k + t] = 0;
  }
  __syncthreads();
  if (key == 0) return;
  int rank = 0;
#pragma unroll 8
  for (int j = 0; j < kTopkGroup; j += 2) {
    const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(s_key + j);
    rank += (v.x > key) + (v.y > key);
  }
  if (rank >= a.k) return;
  if (a.final_level) {
    const int n = (int)(~(uint32_t)(key & 0xffffffffu));
    a.ids[(size_t)b * a.k + rank] = n;
    a.scores[(size_t)b * a.k + rank] = float_from_order_key((uint32_t)(key >> 32));
    if (a.exclude_out) atomicOr(&a.exclude_out[(size_t)b * a.W + (n >> 5)], 1u << (n & 31));
  } else {
    a.out[((size_t)b * groups + g) * a.k + rank] = key;
  }
}

// Single-launch top-k for banks of up to kFusedDocs documents: one workgroup
// of 1024 threads per query, two documents per thread.  A threshold select:
// the valid scores' range [lo, hi] is cut into 256 equal bins, an LDS
// histogram finds the bin holding the k-th best score, and only the keys in
// that bin or above survive (bins are monotone in the score, so every key
// below lies under at least k survivors).  The survivors -- about k, or
// all of them in a degenerate range -- are ranked exactly by their 64-bit
// keys and the k best written in rank order.  The keys are those of the
// level kernel, so both select the same documents in the same order.
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kFusedDocs = 2 * kFusedThreads;
constexpr int kBins = 256;

__device__ __forceinline__ int score_bin(float s, float lo, float scale) {
  return min(kBins - 1, max(0, (int)((s - lo) * scale)));
}

__global__ __launch_bounds__(kFusedThreads) void topk_fused_kernel(TopkLevel a) {
  __shared__ __attribute__((aligned(16))) uint64_t s_surv[kFusedDocs];
  __shared__ int s_hist[kBins];
  __shared__ float s_lo[kFusedWaves], s_hi[kFusedWaves];
  __shared__ int s_cnt[kFusedWaves];
  __shared__ int s_cut, s_n;
  const int b = blockIdx.x, t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int k = a.k;
  const float* pm = a.piecemax + (size_t)b * a.h_r * a.P;
  const uint32_t* excl = a.exclude ? a.exclude + (size_t)b * a.W : nullptr;
  const int n0 = t, n1 = t + kFusedThreads;
  const uint64_t k0 = n0 < a.N ? doc_key(pm, a.h_r, a.P, a.doc_piece0, excl, n0) : 0;
  const uint64_t k1 = n1 < a.N ? doc_key(pm, a.h_r, a.P, a.doc_piece0, excl, n1) : 0;
  const float s0 = float_from_order_key((uint32_t)(k0 >> 32));
  const float s1 = float_from_order_key((uint32_t)(k1 >> 32));
  // the valid scores' range and count, per wave
  float lo = INFINITY, hi = -INFINITY;
  if (k0) lo = fminf(lo, s0), hi = fmaxf(hi, s0);
  if (k1) lo = fminf(lo, s1), hi = fmaxf(hi, s1);
  lo = -wave_max(-lo);
  hi = wave_max(hi);
  const int cnt = __builtin_popcountll(__ballot(k0 != 0)) + __builtin_popcountll(__ballot(k1 != 0));
  if (lane == 0) {
    s_lo[wave] = lo;
    s_hi[wave] = hi;
    s_cnt[wave] = cnt;
  }
  if (t < kBins) s_hist[t] = 0;
  if (t == 0) s_n = 0;
  if (t < k) {
    a.ids[(size_t)b * k + t] = -1;
    a.scores[(size_t)b * k + t] = -INFINITY;
  }
  __syncthreads();
  int valid = 0;
  lo = INFINITY;
  hi = -INFINITY;
#pragma unroll
  for (int w = 0; w < kFusedWaves; ++w) {
    lo = fminf(lo, s_lo[w]);
    hi = fmaxf(hi, s_hi[w]);
    valid += s_cnt[w];
  }
  if (valid == 0) return;
  const float scale = hi > lo ? (float)kBins / (hi - lo) : 0.f;
  if (k0) atomicAdd(&s_hist[score_bin(s0, lo, scale)], 1);
  if (k1) atomicAdd(&s_hist[score_bin(s1, lo, scale)], 1);
  __syncthreads();
  // the bin holding the k-th best score: wave 0, four bins per lane counted
  // from the top
  if (wave == 0) {
    const int top = kBins - 1 - 4 * lane;
    const int c = s_hist[top] + s_hist[top - 1] + s_hist[top - 2] + s_hist[top - 3];
    int incl = c;  // inclusive prefix over lanes (bins from the top down)
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    const int need = min(k, valid);
    const uint64_t reach = __ballot(incl >= need);  // lanes whose bins reach k
    if (lane == __builtin_ctzll(reach)) {
      int acc = incl - c, bin = top;
      for (;; --bin) {
        acc += s_hist[bin];
        if (acc >= need) break;
      }
      s_cut = bin;
    }
  }
  __syncthreads();
  const int cut = s_cut;
  if (k0 && score_bin(s0, lo, scale) >= cut) s_surv[atomicAdd(&s_n, 1)] = k0;
  if (k1 && score_bin(s1, lo, scale) >= cut) s_surv[atomicAdd(&s_n, 1)] = k1;
  __syncthreads();
  const int S = s_n;
  for (int i = t; i < S; i += kFusedThreads) {
    const uint64_t key = s_surv[i];
    int rank = 0;
    for (int j = 0; j < S; ++j) rank += s_surv[j] > key;
    if (rank >= k) continue;
    const int n = (int)(~(uint32_t)(key & 0xffffffffu));
    a.ids[(size_t)b * k + rank] = n;
    a.scores[(size_t)b * k + rank] = float_from_order_key((uint32_t)(key >> 32));
    if (a.exclude_out) atomicOr(&a.exclude_out[(size_t)b * a.W + (n >> 5)], 1u << (n & 31));
  }
}

// ---------------------------------------------------------------- prefill routing
// block-mean router query per (block, head): mean of the block's rows
template <typename T>
__global__ __launch_bounds__(128) void block_mean_kernel(const T* __restrict__ rt, int h_r,
                                                         int block, float* __restrict__ qo) {
  const int g = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
  double s = 0.0;
  int t = 0;
  // eight loads in flight ahead of the (sequential) float64 sum
  for (; t + 8 <= block; t += 8) {
    T x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = rt[((size_t)(g * block + t + u) * h_r + h) * kD + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += St<T>::load(x[u]);
  }
  for (; t < block; ++t) s += St<T>::load(rt[((size_t)(g * block + t) * h_r + h) * kD + i]);
  qo[((size_t)g * h_r + h) * kD + i] = (float)(s / (double)block);
}

// ---------------------------------------------------------------- interleave
// q_next[b][j] = sum_i w[j][i] * out[b][i]; one wave per (b, j)
__global__ __launch_bounds__(256) void project_kernel(const float* __restrict__ out,
                                                      const float* __restrict__ w, int B,
                                                      int n_in, int d_r,
                                                      float* __restrict__ qn) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + wave;
  if (idx >= B * d_r) return;
  const int b = idx / d_r, j = idx % d_r;
  const float* o = out + (size_t)b * n_in;
  const float* wr = w + (size_t)j * n_in;
  float s = 0.f;
  for (int i = lane * 4; i < n_in; i += 256) {
    const float4 a = *reinterpret_cast<const float4*>(o + i);
    const float4 c = *reinterpret_cast<const float4*>(wr + i);
    s = fmaf(a.x, c.x, s); s = fmaf(a.y, c.y, s); s = fmaf(a.z, c.z, s); s = fmaf(a.w, c.w, s);
  }
  s = wave_sum(s);
  if (lane == 0) qn[(size_t)b * d_r + j] = s;
}

}  // namespace


// compute units of the current device (queried once per device)
static int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_route_scan(const Bank& bk, const float* q_route, int B, float* piecemax,
                             hipStream_t s) {
  timer_mark(1, true, s);
  if (bk.desc.dtype == MSA_BF16) {
    // persistent: about kScanWgPerCu workgroups per compute unit in all
    const int gx = std::max(1, std::min(bk.n_tiles, (kScanWgPerCu * device_cus() + bk.desc.h_r - 1) /
                                                        bk.desc.h_r));
    for (int bg = 0; bg < B; bg += 64)
      hipLaunchKernelGGL(route_scan_mfma_kernel, dim3((unsigned)gx, (unsigned)bk.desc.h_r),
                         dim3(256), 0, s, (const uint16_t*)bk.desc.kr, bk.desc.inv_norm, q_route, B,
                         bg, bk.desc.h_r, bk.n_chunks, bk.chunk_stride, bk.d_chunk_doc,
                         bk.d_tile_piece0, bk.n_pieces, piecemax);
  } else {
    const dim3 grid((unsigned)bk.n_tiles, (unsigned)bk.desc.h_r);
    for (int bg = 0; bg < B; bg += 64)
      hipLaunchKernelGGL(route_scan_kernel, grid, dim3(256), 0, s, (const float*)bk.desc.kr,
                         bk.desc.inv_norm, q_route, B, bg, bk.desc.h_r, bk.n_chunks,
                         bk.chunk_stride, bk.d_chunk_doc, bk.d_tile_piece0, bk.n_pieces, piecemax);
  }
  timer_mark(1, false, s);
  return hipGetLastError();
}

size_t topk_scratch_keys(int N, int k) {
  // two ping-pong candidate buffers of (ceil(N/256) * k) keys per query
  return 2 * (size_t)std::max(1, (N + kTopkGroup - 1) / kTopkGroup) * std::max(k, 1);
}

hipError_t launch_topk(const Bank& bk, const float* piecemax, int B, int k,
                       const uint32_t* exclude, uint32_t* exclude_out, int32_t* ids,
                       float* scores, uint64_t* cand, hipStream_t s) {
  const int N = bk.desc.n_docs;
  TopkLevel a{};
  a.piecemax = piecemax;
  a.h_r = bk.desc.h_r;
  a.N = N;
  a.P = bk.n_pieces;
  a.doc_piece0 = bk.d_doc_piece0;
  a.exclude = exclude;
  a.W = (N + 31) / 32;
  a.k = k;
  a.ids = ids;
  a.scores = scores;
  a.exclude_out = exclude_out;
  if (N <= kFusedDocs && k <= kMaxK) {
    a.final_level = 1;
    hipLaunchKernelGGL(topk_fused_kernel, dim3((unsigned)B), dim3(kFusedThreads), 0, s, a);
    return hipGetLastError();
  }
  const size_t half = topk_scratch_keys(N, k) / 2;
  uint64_t* bufs[2] = {cand, cand + (size_t)B * half};
  int M = N, lvl = 0;
  for (;;) {
    const int groups = (M + kTopkGroup - 1) / kTopkGroup;
    a.final_level = groups == 1;
    a.out = bufs[lvl & 1];
    hipLaunchKernelGGL(topk_level_kernel, dim3((unsigned)groups, (unsigned)B), dim3(kTopkGroup), 0,
                       s, a);
    if (a.final_level) break;
    a.in = a.out;
    a.M_in = groups * k;
    M = a.M_in;
    ++lvl;
  }
  return hipGetLastError();
}

hipError_t launch_block_mean(const Bank& bk, const void* rt, int n_tok, int block, float* q_out,
                             hipStream_t s) {
  const dim3 grid((unsigned)(n_tok / block), (unsigned)bk.desc.h_r);
  if (bk.desc.dtype == MSA_BF16)
    hipLaunchKernelGGL(block_mean_kernel<uint16_t>, grid, dim3(128), 0, s, (const uint16_t*)rt,
                       bk.desc.h_r, block, q_out);
  else
    hipLaunchKernelGGL(block_mean_kernel<float>, grid, dim3(128), 0, s, (const float*)rt,
                       bk.desc.h_r, block, q_out);
  return hipGetLastError();
}

hipError_t launch_project(const float* out, const float* w, int B, int n_in, int d_r,
                          float* q_next, hipStream_t s) {
  const unsigned grid = (unsigned)((B * d_r + 3) / 4);
  hipLaunchKernelGGL(project_kernel, dim3(grid), dim3(256), 0, s, out, w, B, n_in, d_r, q_next);
  return hipGetLastError();
}

}  // namespace msa
