// Blocked prefill attention on the matrix cores.
//
// Each block of `block` consecutive query tokens shares one set of selected
// documents ("MSA" card, robocikowo.com, "Komponenty": the MSA layer appends
// the top-k documents' K/V to the local context); query i attends to every
// token of its block's documents and to local tokens j <= its own local index
// (causal), with the 1/sqrt(d) scale (mlqm.cn MLA/CSA article, section 6.2).
//
// One workgroup = (block of 64 queries, KV head, token split): 256 rows
// (64 queries x 4 query heads of the KV head), 4 waves of 64 rows.  Each
// 64-token K/V tile is staged once in LDS (double-buffered, XOR-swizzled
// 16-byte chunks) and shared by all 256 rows: 256 flop per byte of K/V.
// Both contractions use v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// Scores are computed transposed, S^T = K . Q^T (tokens x rows), so the
// accumulator layout of S^T is exactly the B-operand layout P^T needs for
// O^T = V^T . P^T (the contraction order over the tile's tokens is permuted
// consistently in both operands): probabilities never leave registers.
// Online softmax in base 2 (queries are pre-scaled by log2 e / sqrt(d)).
#include <algorithm>

#include "msa_internal.h"

namespace msa {

hipError_t launch_prefill_vector(const Bank& bk, const void* q_rot, int n_q, int h_q,
                                 const int32_t* ids, int k, int block, const AttnSources& src,
                                 const void* k_loc, const void* v_loc, int L_loc, int splits,
                                 float* part, float* out, hipStream_t s);

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRows = 256;          // rows per workgroup (64 queries x 4 heads)
constexpr int kQBlock = 64;         // queries per routing block handled here
constexpr int kPG = 4;              // query heads per KV head handled here
constexpr int kTileB = 64 * kD * 2;  // bytes of one K (or V) tile in bf16

struct PrefillP {
  const uint16_t* q;  // [n_q][h_q][128] rotated, pre-scaled
  const int32_t* ids;  // [n_blocks][k]
  const uint16_t* ks;
  const uint16_t* vs;
  const int64_t* soff;
  const int32_t* slen;
  int n_src;
  const uint16_t* kl;  // [h_kv][L_loc][128]
  const uint16_t* vl;  // [h_kv][Tp][128][64]
  int k, L_loc, n_q, h_kv, h_q, S;
  float* part;  // [n_blocks][h_kv][S][256][130]
};

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b,
                                           const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }

__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillP p) {
  const int split = blockIdx.x, h = blockIdx.y, blk = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int k = p.k;
  const int causal_base = p.L_loc - p.n_q;  // local index of query 0

  __shared__ int64_t s_koff[kMaxK + 1], s_voff[kMaxK + 1];
  __shared__ int s_len[kMaxK + 1], s_tile0[kMaxK + 2];
  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][kTileB];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][kTileB];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[kRows * kD * 2];  // [row][16 chunks], swizzled

  if (tid < k) {
    const int id = p.ids[(size_t)blk * k + tid];
    int L = 0;
    int64_t off = 0;
    if (id >= 0 && id < p.n_src) {
      L = p.slen[id];
      off = p.soff[id];
    }
    const int64_t o = (off * p.h_kv + (int64_t)h * L) * kD;
    s_len[tid] = L;
    s_koff[tid] = o;
    s_voff[tid] = o;
  } else if (tid == k) {
    const int64_t tp = (p.L_loc + 63) / 64;
    s_len[k] = min(p.L_loc, causal_base + kQBlock * (blk + 1));
    s_koff[k] = (int64_t)h * p.L_loc * kD;
    s_voff[k] = (int64_t)h * tp * 64 * kD;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int r = 0; r <= k; ++r) {
      s_tile0[r] = acc;
      acc += (s_len[r] + 63) / 64;
    }
    s_tile0[k + 1] = acc;
  }
  __syncthreads();
  const int NT = __builtin_amdgcn_readfirstlane(s_tile0[k + 1]);
  const int u0 = (int)((int64_t)NT * split / p.S);
  const int u1 = (int)((int64_t)NT * (split + 1) / p.S);

  // ---- Q rows of the workgroup staged in LDS: row R = 64*wave + n ->
  // query 16*wave + n/4, head n%4; 16-byte chunk c at (c ^ (R & 15)).
  const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int f = tid + 256 * i;  // 256 rows x 16 chunks
    const int R = f >> 4, c = f & 15;
    const int qi = blk * kQBlock + (R >> 2);
    const uint16_t* qrow = p.q + ((size_t)qi * p.h_q + (size_t)h * kPG + (R & 3)) * kD;
    *reinterpret_cast<uint4*>(&s_q[R * 256 + ((c ^ (R & 15)) << 4)]) =
        *reinterpret_cast<const uint4*>(qrow + 8 * c);
  }
  // Q^T B operand for row tile nt, k-step kk: row 32*nt + l32 of this wave,
  // channels 16*kk + 8*hl .. +7
  auto qfrag = [&](int nt, int kk) {
    const int R = 64 * wave + 32 * nt + l32, c = 2 * kk + hl;
    return __builtin_bit_cast(bf16x8_t,
                              *reinterpret_cast<const uint4*>(&s_q[R * 256 + ((c ^ (R & 15)) << 4)]));
  };
  // local (causal) index of each of this lane's two rows; the wave's smallest
  const int li_wave_min = causal_base + blk * kQBlock + 16 * wave;
  int li[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) li[nt] = causal_base + blk * kQBlock + 16 * wave + ((32 * nt + l32) >> 2);

  f32x16_t o[4][2];  // O^T: [channel tile 0..3][row tile 0..1]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][nt][e] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  // ---- tile staging: 256 threads x (4 K + 4 V) 16-byte chunks
  int r = 0;
  struct Tile {
    const uint16_t* kb;
    const uint16_t* vb;
    int nvalid;
    int t0;     // token offset inside the segment
    bool local;
  };
  auto tile_at = [&](int u) {
    while (u >= __builtin_amdgcn_readfirstlane(s_tile0[r + 1])) ++r;
    Tile t;
    t.t0 = (u - __builtin_amdgcn_readfirstlane(s_tile0[r])) * 64;
    t.nvalid = min(64, __builtin_amdgcn_readfirstlane(s_len[r]) - t.t0);
    t.local = r == k;
    const int64_t koff = ((int64_t)__builtin_amdgcn_readfirstlane((int)(s_koff[r] >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)s_koff[r]);
    const int64_t voff = ((int64_t)__builtin_amdgcn_readfirstlane((int)(s_voff[r] >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)s_voff[r]);
    t.kb = (t.local ? p.kl : p.ks) + koff + (size_t)t.t0 * kD;
    t.vb = (t.local ? p.vl : p.vs) + voff + (size_t)t.t0 * kD;
    return t;
  };
  uint4 stg[8];
  auto fetch = [&](const Tile& t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + 256 * i;
      const int row = f >> 4, c = f & 15;  // K: 64 rows x 16 chunks
      stg[i] = row < t.nvalid ? *reinterpret_cast<const uint4*>(t.kb + row * kD + c * 8)
                              : make_uint4(0, 0, 0, 0);
      const int d = f >> 3, cv = f & 7;  // V^T: 128 rows x 8 chunks (zero-padded tiles)
      stg[4 + i] = *reinterpret_cast<const uint4*>(t.vb + d * 64 + cv * 8);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + 256 * i;
      const int row = f >> 4, c = f & 15;
      *reinterpret_cast<uint4*>(&s_k[buf][row * 256 + ((c ^ (row & 15)) << 4)]) = stg[i];
      const int d = f >> 3, cv = f & 7;
      *reinterpret_cast<uint4*>(&s_v[buf][d * 128 + ((cv ^ (d & 7)) << 4)]) = stg[4 + i];
    }
  };

  Tile cur{};
  if (u0 < u1) {
    cur = tile_at(u0);
    fetch(cur);
    stash(0);
  }
  __syncthreads();
  for (int u = u0; u < u1; ++u) {
    const int buf = (u - u0) & 1;
    const bool has_next = u + 1 < u1;
    Tile nxt{};
    if (has_next) {
      nxt = tile_at(u + 1);
      fetch(nxt);  // in flight during this tile's math
    }
    const uint8_t* sk = s_k[buf];
    const uint8_t* sv = s_v[buf];

    // ---- two halves of 32 tokens (mt).  Each half: S^T = K . Q^T for the 2
    // row tiles, mask, lazy-rescaled softmax, then O^T += V^T . P^T over the
    // half's two 16-token k-steps.  Lazy rescaling: probabilities are taken
    // relative to a per-row reference m_run that only moves (rescaling O and
    // l) when a row max exceeds it by more than 8 in log2 units, so p <= 256;
    // O otherwise stays untouched in the accumulators.
    // Element e of s[nt]: token 32*mt + 8*(e/4) + 4*hl + (e%4), row 32*nt + l32.
    const bool need_mask = cur.nvalid < 64 || (cur.local && cur.t0 + 63 > li_wave_min);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16_t s[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[nt][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int row = 32 * mt + l32, c = 2 * kk + hl;
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(&sk[row * 256 + ((c ^ (row & 15)) << 4)]));
        s[0] = mfma32(a, qfrag(0, kk), s[0]);
        s[1] = mfma32(a, qfrag(1, kk), s[1]);
      }
      float mx[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float m = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float v = s[nt][e];
          if (need_mask) {
            const int t = 32 * mt + 8 * (e >> 2) + 4 * hl + (e & 3);
            const bool ok = t < cur.nvalid && (!cur.local || cur.t0 + t <= li[nt]);
            v = ok ? v : -INFINITY;
            s[nt][e] = v;
          }
          m = fmaxf(m, v);
        }
        mx[nt] = fmaxf(m, __shfl_xor(m, 32, 64));
      }
      const bool grow = mx[0] > m_run[0] + 8.f || mx[1] > m_run[1] + 8.f;
      if (__builtin_amdgcn_readfirstlane((int)(__ballot(grow) != 0))) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float m_new = mx[nt] > m_run[nt] + 8.f ? mx[nt] : m_run[nt];
          const float alpha =
              m_new == m_run[nt] ? 1.f : __builtin_amdgcn_exp2f(m_run[nt] - m_new);
          m_run[nt] = m_new;
          l_run[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][nt][e] *= alpha;
        }
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float m_use = m_run[nt] == -INFINITY ? 0.f : m_run[nt];
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pe = __builtin_amdgcn_exp2f(s[nt][e] - m_use);
          s[nt][e] = pe;
          ls += pe;
        }
        l_run[nt] += ls;
      }
      // O^T += V^T . P^T: k-step hh covers tokens 32mt+16hh+4hl+[0..3], +8+[0..3]
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8_t pb[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          uint4 w;
          w.x = pack2(s[nt][8 * hh + 0], s[nt][8 * hh + 1]);
          w.y = pack2(s[nt][8 * hh + 2], s[nt][8 * hh + 3]);
          w.z = pack2(s[nt][8 * hh + 4], s[nt][8 * hh + 5]);
          w.w = pack2(s[nt][8 * hh + 6], s[nt][8 * hh + 7]);
          pb[nt] = __builtin_bit_cast(bf16x8_t, w);
        }
        const int tk = 32 * mt + 16 * hh + 4 * hl;
        const int c0 = tk >> 3, c1 = (tk + 8) >> 3, half = (tk >> 2) & 1;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d = 32 * dt + l32;
          const uint2 lo =
              *reinterpret_cast<const uint2*>(&sv[d * 128 + ((c0 ^ (d & 7)) << 4) + 8 * half]);
          const uint2 hi =
              *reinterpret_cast<const uint2*>(&sv[d * 128 + ((c1 ^ (d & 7)) << 4) + 8 * half]);
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          o[dt][0] = mfma32(a, pb[0], o[dt][0]);
          o[dt][1] = mfma32(a, pb[1], o[dt][1]);
        }
      }
    }

    if (has_next) stash(buf ^ 1);
    __syncthreads();
    cur = nxt;
  }

  // ---- partials: row n of this wave (lane holds row 32*nt + l32)
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) l_run[nt] += __shfl_xor(l_run[nt], 32, 64);
  const size_t pbase = ((((size_t)blk * p.h_kv + h) * p.S + split) * kRows + 64 * wave) * (kD + 2);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float* pr = p.part + pbase + (size_t)(32 * nt + l32) * (kD + 2);
    if (hl == 0) {
      pr[0] = m_run[nt];
      pr[1] = l_run[nt];
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) pr[2 + 32 * dt + 8 * (e >> 2) + 4 * hl + (e & 3)] = o[dt][nt][e];
  }
}

// merge the S partials of each (block, KV head): base-2 log-sum-exp per row
__global__ __launch_bounds__(256) void prefill_combine_kernel(const float* __restrict__ part,
                                                              int S, int h_kv, int h_q,
                                                              float* __restrict__ out) {
  const int h = blockIdx.y, blk = blockIdx.z;
  const int row = blockIdx.x * 2 + (threadIdx.x >> 7), d = threadIdx.x & 127;
  const float* pb = part + (((size_t)blk * h_kv + h) * S * kRows + row) * (kD + 2);
  const size_t sstride = (size_t)kRows * (kD + 2);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pb[s * sstride]);
  float L = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float* ps = pb + s * sstride;
      const float w = exp2f(ps[0] - M);
      L = fmaf(w, ps[1], L);
      acc = fmaf(w, ps[2 + d], acc);
    }
  }
  const int wave = row >> 6, n = row & 63;
  const int qi = blk * kQBlock + 16 * wave + (n >> 2);
  out[((size_t)qi * h_q + (size_t)h * kPG + (n & 3)) * kD + d] = L > 0.f ? acc / L : 0.f;
}

}  // namespace

size_t prefill_partial_floats(int n_q, int h_kv, int splits) {
  return (size_t)(n_q / kQBlock) * h_kv * splits * kRows * (kD + 2);
}

int prefill_auto_splits(const Bank& bk, int n_q, int k, int L_loc) {
  // enough workgroups to cover the GPU twice over
  const int n_blocks = std::max(1, n_q / kQBlock);
  const int64_t wg = (int64_t)n_blocks * bk.desc.h_kv;
  const double avg_doc = (double)bk.n_tokens / bk.desc.n_docs;
  const int tiles = (int)std::max(1.0, k * avg_doc / 64 + (L_loc + 63) / 64);
  int s = (int)((512 + wg - 1) / wg);
  return std::max(1, std::min({s, tiles, 64}));
}

bool prefill_mfma_supported(const Bank& bk, int n_q, int h_q, int block) {
  return bk.desc.dtype == MSA_BF16 && block == kQBlock && h_q == bk.desc.h_kv * kPG &&
         n_q % kQBlock == 0;
}

hipError_t launch_prefill(const Bank& bk, const void* q_rot, int n_q, int h_q, const int32_t* ids,
                          int k, int block, const AttnSources& src, const void* k_loc,
                          const void* v_loc, int L_loc, int splits, float* part, float* out,
                          hipStream_t s) {
  if (!prefill_mfma_supported(bk, n_q, h_q, block))
    return launch_prefill_vector(bk, q_rot, n_q, h_q, ids, k, block, src, k_loc, v_loc, L_loc,
                                 splits, part, out, s);
  PrefillP p;
  p.q = (const uint16_t*)q_rot;
  p.ids = ids;
  p.ks = (const uint16_t*)src.k;
  p.vs = (const uint16_t*)src.v;
  p.soff = src.off;
  p.slen = src.len;
  p.n_src = src.n;
  p.kl = (const uint16_t*)k_loc;
  p.vl = (const uint16_t*)v_loc;
  p.k = k;
  p.L_loc = L_loc;
  p.n_q = n_q;
  p.h_kv = bk.desc.h_kv;
  p.h_q = h_q;
  p.S = splits;
  p.part = part;
  const int n_blocks = n_q / kQBlock;
  timer_mark(0, true, s);
  hipLaunchKernelGGL(prefill_mfma_kernel, dim3((unsigned)splits, (unsigned)p.h_kv, (unsigned)n_blocks),
                     dim3(256), 0, s, p);
  timer_mark(0, false, s);
  hipLaunchKernelGGL(prefill_combine_kernel, dim3(kRows / 2, (unsigned)p.h_kv, (unsigned)n_blocks),
                     dim3(256), 0, s, part, splits, p.h_kv, h_q, out);
  return hipGetLastError();
}

}  // namespace msa
