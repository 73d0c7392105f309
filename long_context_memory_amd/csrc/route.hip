// Routing: cosine scoring of router queries against every routing key, the
// per-document max over chunks and mean over router heads, and top-k
// document selection ("MSA" card, robocikowo.com, "Komponenty", router;
// "MSA架构" article, intelliparadigm.com, section 2.1).  Also the block-mean
// router queries of the blocked prefill and the Memory Interleave projection
// that forms the next hop's router query.
//
// route_scan: one wave per (router head, tile of 64 chunks).  The wave stages
// its 64 key rows (16 KiB of bf16, coalesced 1 KiB loads) through LDS, each
// lane takes one row into registers (float32), and dots it with every query
// of the batch (query values are wave-uniform, so they arrive as scalar
// loads).  Cosines go back through LDS transposed, and lane b folds its
// query's cosines into per-document maxima over the tile's chunks: one
// "piece" per (document, tile) it overlaps.  top-k later takes the max over a
// document's pieces, so no atomics and no initialisation are needed.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kRowPad = 68;      // floats per staged row (256 B of bf16 + 16 B pad)
constexpr int kCosStride = 65;   // floats per query row of staged cosines

template <typename T>
__device__ __forceinline__ void load_row_f32(const T* __restrict__ rows, int nc, int lane,
                                             float* lds_w, float (&kf)[kD]);

template <>
__device__ __forceinline__ void load_row_f32<uint16_t>(const uint16_t* __restrict__ rows, int nc,
                                                       int lane, float* lds_w,
                                                       float (&kf)[kD]) {
  // 64 rows x 16 vectors of 16 B; flat vector f = i*64 + lane -> row f/16
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int f = i * 64 + lane;
    const int row = f >> 4, col = f & 15;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < nc) v = *reinterpret_cast<const uint4*>(rows + (size_t)f * 8);
    *reinterpret_cast<uint4*>(lds_w + row * kRowPad + col * 4) = v;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint4 v = *reinterpret_cast<const uint4*>(lds_w + lane * kRowPad + j * 4);
    kf[j * 8 + 0] = bf16_lo(v.x); kf[j * 8 + 1] = bf16_hi(v.x);
    kf[j * 8 + 2] = bf16_lo(v.y); kf[j * 8 + 3] = bf16_hi(v.y);
    kf[j * 8 + 4] = bf16_lo(v.z); kf[j * 8 + 5] = bf16_hi(v.z);
    kf[j * 8 + 6] = bf16_lo(v.w); kf[j * 8 + 7] = bf16_hi(v.w);
  }
}

template <>
__device__ __forceinline__ void load_row_f32<float>(const float* __restrict__ rows, int nc,
                                                    int lane, float* lds_w, float (&kf)[kD]) {
  // float32 keys: each lane reads its own 512 B row directly
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < nc) v = *reinterpret_cast<const float4*>(rows + (size_t)lane * kD + j * 4);
    kf[j * 4 + 0] = v.x; kf[j * 4 + 1] = v.y; kf[j * 4 + 2] = v.z; kf[j * 4 + 3] = v.w;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void route_scan_kernel(
    const T* __restrict__ kr, const float* __restrict__ inv_norm, const float* __restrict__ q,
    int B, int h_r, int64_t C, int n_tiles, const int32_t* __restrict__ chunk_doc,
    const int32_t* __restrict__ tile_piece0, int P, float* __restrict__ piecemax) {
  __shared__ float lds[4][64 * kRowPad];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + wave;
  const int h = blockIdx.y;
  // a wave past the last tile keeps taking part in the workgroup barriers
  const bool active = tile < n_tiles;
  float* lds_w = lds[wave];
  const int64_t c0 = (int64_t)(active ? tile : 0) * kRouteTile;
  const int nc = active ? (int)min((int64_t)kRouteTile, C - c0) : 0;
  const T* rows = kr + ((size_t)h * C + c0) * kD;

  float kf[kD];
  load_row_f32<T>(rows, nc, lane, lds_w, kf);
  const float inv_k = lane < nc ? inv_norm[(size_t)h * C + c0 + lane] : 0.0f;
  __syncthreads();  // every lane holds its row before LDS is reused for cosines

  const int piece0 = active ? tile_piece0[tile] : 0;
  const int doc_first = active ? chunk_doc[c0] : 0;
  for (int bg = 0; bg < B; bg += 64) {
    const int nb = min(64, B - bg);
    // lane b's own query norm (applied after the max: x -> x * s is monotone)
    float iq = 0.0f;
    if (lane < nb) {
      const float* qb = q + ((size_t)(bg + lane) * h_r + h) * kD;
      float s = 0.f;
      for (int i = 0; i < kD; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(qb + i);
        s = fmaf(v.x, v.x, s); s = fmaf(v.y, v.y, s); s = fmaf(v.z, v.z, s); s = fmaf(v.w, v.w, s);
      }
      iq = s > 0.f ? 1.0f / sqrtf(s) : 0.0f;
    }
    // dot products of this lane's key row with queries bg .. bg+nb-1, four at
    // a time (query values are wave-uniform)
    for (int bb = 0; bb < nb; bb += 4) {
      const float* q0 = q + ((size_t)(bg + bb) * h_r + h) * kD;
      const float* q1 = q + ((size_t)(bg + min(bb + 1, nb - 1)) * h_r + h) * kD;
      const float* q2 = q + ((size_t)(bg + min(bb + 2, nb - 1)) * h_r + h) * kD;
      const float* q3 = q + ((size_t)(bg + min(bb + 3, nb - 1)) * h_r + h) * kD;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int i = 0; i < kD; ++i) {
        a0 = fmaf(kf[i], q0[i], a0);
        a1 = fmaf(kf[i], q1[i], a1);
        a2 = fmaf(kf[i], q2[i], a2);
        a3 = fmaf(kf[i], q3[i], a3);
      }
      lds_w[(bb + 0) * kCosStride + lane] = a0 * inv_k;
      if (bb + 1 < nb) lds_w[(bb + 1) * kCosStride + lane] = a1 * inv_k;
      if (bb + 2 < nb) lds_w[(bb + 2) * kCosStride + lane] = a2 * inv_k;
      if (bb + 3 < nb) lds_w[(bb + 3) * kCosStride + lane] = a3 * inv_k;
    }
    __syncthreads();
    // lane b: per-document max over the tile's chunks (document runs are
    // wave-uniform), then the query norm
    int c = 0;
    while (c < nc) {
      const int d = chunk_doc[c0 + c];
      float m = -INFINITY;
      while (c < nc && chunk_doc[c0 + c] == d) {
        if (lane < nb) m = fmaxf(m, lds_w[lane * kCosStride + c]);
        ++c;
      }
      if (lane < nb)
        piecemax[((size_t)h * P + piece0 + (d - doc_first)) * B + bg + lane] = m * iq;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- top-k
// One workgroup per query.  Each document's score is turned into a 64-bit
// key (order-preserving score bits << 32 | ~id): the larger key is the higher
// score, and among equal scores the lower id.  Key 0 marks an excluded or
// taken document.  k rounds of a block-wide max pick the winners in rank
// order; only the winner's owner rescans its strided share.
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ piecemax, int B, int h_r, int N, int P,
    const int32_t* __restrict__ doc_piece0, const uint32_t* exclude, int W,
    uint32_t* exclude_out, int k, int32_t* __restrict__ ids,
    float* __restrict__ scores, uint64_t* __restrict__ keys) {
  const int b = blockIdx.x, tid = threadIdx.x;
  uint64_t* kb = keys + (size_t)b * N;
  uint64_t best = 0;
  for (int n = tid; n < N; n += 256) {
    uint64_t key = 0;
    const bool excl = exclude && ((exclude[(size_t)b * W + (n >> 5)] >> (n & 31)) & 1u);
    if (!excl) {
      const int p0 = doc_piece0[n], p1 = doc_piece0[n + 1];
      float s = 0.f;
      for (int h = 0; h < h_r; ++h) {
        float m = -INFINITY;
        for (int p = p0; p < p1; ++p) m = fmaxf(m, piecemax[((size_t)h * P + p) * B + b]);
        s += m;
      }
      s = s / (float)h_r;
      key = ((uint64_t)float_order_key(s) << 32) | (uint64_t)(~(uint32_t)n);
    }
    kb[n] = key;
    best = umax64(best, key);
  }
  __shared__ uint64_t red[4];
  const int wave = tid >> 6, lane = tid & 63;
  for (int r = 0; r < k; ++r) {
    uint64_t m = best;
    for (int o = 32; o >= 1; o >>= 1) m = umax64(m, (uint64_t)__shfl_xor((long long)m, o, 64));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    const uint64_t win = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
    __syncthreads();
    if (win == 0) {
      if (tid == 0) {
        ids[(size_t)b * k + r] = -1;
        scores[(size_t)b * k + r] = -INFINITY;
      }
      continue;
    }
    const int n = (int)(~(uint32_t)(win & 0xffffffffu));
    if (tid == 0) {
      ids[(size_t)b * k + r] = n;
      scores[(size_t)b * k + r] = float_from_order_key((uint32_t)(win >> 32));
      if (exclude_out) atomicOr(&exclude_out[(size_t)b * W + (n >> 5)], 1u << (n & 31));
    }
    if ((n & 255) == tid) {
      kb[n] = 0;
      best = 0;
      for (int j = tid; j < N; j += 256) best = umax64(best, kb[j]);
    }
  }
}

// ---------------------------------------------------------------- prefill routing
// block-mean router query per (block, head): mean of the block's rows
template <typename T>
__global__ __launch_bounds__(128) void block_mean_kernel(const T* __restrict__ rt, int h_r,
                                                         int block, float* __restrict__ qo) {
  const int g = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
  double s = 0.0;
  for (int t = 0; t < block; ++t) {
    const T x = rt[((size_t)(g * block + t) * h_r + h) * kD + i];
    if constexpr (sizeof(T) == 2) s += (double)bf16_to_f32(x);
    else s += (double)x;
  }
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

hipError_t launch_route_scan(const Bank& bk, const float* q_route, int B, float* piecemax,
                             hipStream_t s) {
  const dim3 grid((unsigned)((bk.n_tiles + 3) / 4), (unsigned)bk.desc.h_r);
  if (bk.desc.dtype == MSA_BF16)
    hipLaunchKernelGGL(route_scan_kernel<uint16_t>, grid, dim3(256), 0, s,
                       (const uint16_t*)bk.desc.kr, bk.desc.inv_norm, q_route, B, bk.desc.h_r,
                       bk.n_chunks, bk.n_tiles, bk.d_chunk_doc, bk.d_tile_piece0, bk.n_pieces,
                       piecemax);
  else
    hipLaunchKernelGGL(route_scan_kernel<float>, grid, dim3(256), 0, s,
                       (const float*)bk.desc.kr, bk.desc.inv_norm, q_route, B, bk.desc.h_r,
                       bk.n_chunks, bk.n_tiles, bk.d_chunk_doc, bk.d_tile_piece0, bk.n_pieces,
                       piecemax);
  return hipGetLastError();
}

hipError_t launch_topk(const Bank& bk, const float* piecemax, int B, int k,
                       const uint32_t* exclude, uint32_t* exclude_out, int32_t* ids,
                       float* scores, uint64_t* keys, hipStream_t s) {
  const int N = bk.desc.n_docs;
  const int W = (N + 31) / 32;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)B), dim3(256), 0, s, piecemax, B,
                     bk.desc.h_r, N, bk.n_pieces, bk.d_doc_piece0, exclude, W, exclude_out, k,
                     ids, scores, keys);
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
