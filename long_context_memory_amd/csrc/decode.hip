// Split-K decode attention over the union of the selected documents and the
// local context ("MSA" card, robocikowo.com, "Komponenty", the MSA layer:
// the top-k documents' K/V are appended to the local context; "Paradygmat
// wykonania": only the selected blocks take part), GQA with G query heads per
// KV head, scale 1/sqrt(d) (mlqm.cn MLA/CSA article, section 6.2).
//
// HBM-bound: every K/V byte of the union is read once and feeds G query
// heads (4 flop per byte at G = 4), so the kernel is built around streaming:
//   - workgroup = 4 independent waves; grid = (splits/4, h_kv, B).  Each wave
//     owns a contiguous range of 64-token tiles of its (query, KV head) union
//     and keeps its own online-softmax state; partials are merged by
//     combine_kernel.
//   - K tile [64 tok][128] (row-major): 8 lanes per token row, 16 channels per
//     lane, fully used 128-byte lines; bf16 pair dots (v_dot2_f32_bf16, fp32
//     accumulate) against register-resident query fragments, then a three-step
//     DPP transpose-reduce leaves lane l with the G scores of one token.
//   - V tile [128 ch][64 tok] (channel-major store): 4 lanes per channel row,
//     16 tokens per lane; each lane keeps its 8 rows x G accumulators for the
//     whole range and contracts over its 16 tokens with bf16 pair dots against
//     probabilities staged (as bf16) in a per-wave LDS slot.  The 4-lane
//     reduction of the accumulators happens once, at the end.
//   - the "gather" is an indirection: per (query, head) the workgroup reads
//     the k selected ids and the document table and walks the tiles in place.
//   - decode queries arrive raw: the prologue rotates them at q_pos (float64,
//     one (head, pair) per thread, into LDS), so no separate RoPE launch
//     precedes the kernel.
#include <algorithm>
#include <cmath>

#include "msa_internal.h"

namespace msa {
namespace {

struct DecodeP {
  const void* q;       // [B][h_q][128]: rotated and pre-scaled by log2(e)/sqrt(d), or raw
                       // when inv_freq is set
  const double* inv_freq;  // NULL, or [64]: rotate the raw queries at q_pos in the prologue
  int q_pos;
  const int32_t* ids;  // [B][k]
  const void* ks;
  const void* vs;
  const int64_t* soff;
  const int32_t* slen;
  int n_src;
  const void* kl;
  const void* vl;
  int k, L_loc, h_kv, S, h_q;
  int id_div;      // queries per id row (decode 1; prefill: the routing block)
  int loc_shared;  // 1: every query reads local sequence 0 (prefill)
  int causal_off;  // < 0: none; else query b sees local tokens j < causal_off + b + 1
  const int64_t* svoff;  // NULL, or V offsets of padded (64-entry tile) V blocks
  float doc_bias;        // added to the scores of document entries (log2 units)
  float* part;     // [B][h_kv][S][G][130]: m (log2 units), l, o[128]
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// one transpose-reduce step over lane pairs chosen by CTRL: the lane with
// `upper` set keeps the upper half of its N values, its partner the lower.
template <int CTRL, int N>
__device__ __forceinline__ void treduce(float (&a)[N], int n, bool upper) {
  const int half = n / 2;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    if (i < half) {
      float lo = a[i], hi = a[i + half];
      // opaque copies: keeps the compiler from turning the selects below
      // into a lane-varying index into a[] (a compare/select chain)
      asm volatile("" : "+v"(lo), "+v"(hi));
      const float send = upper ? lo : hi;
      const float keep = upper ? hi : lo;
      a[i] = keep + dpp_f<CTRL>(send);
    }
  }
}

template <int N>
__device__ __forceinline__ void treduce8(float (&a)[N], int j) {
  treduce<kDppHalfMirror, N>(a, N, (j & 4) != 0);
  treduce<kDppXor2, N>(a, N / 2, (j & 2) != 0);
  treduce<kDppXor1, N>(a, N / 4, (j & 1) != 0);
}

template <typename T, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeP p) {
  constexpr bool kBF = sizeof(T) == 2;
  const int b = blockIdx.z, h = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int split = blockIdx.x * 4 + wave;

  __shared__ int64_t s_koff[kMaxK + 1], s_voff[kMaxK + 1];
  __shared__ int s_len[kMaxK + 1], s_tile0[kMaxK + 2];
  __shared__ __attribute__((aligned(16))) T s_p[4][G][kAttnTile];
  __shared__ double s_cs[64], s_sn[64];  // RoPE of the queries: pair i at q_pos
  __shared__ __attribute__((aligned(16))) T s_q[G * kD];  // the rotated queries of (b, h)

  const int k = p.k;
  if (p.inv_freq && threadIdx.x >= 192)
    sincos((double)p.q_pos * p.inv_freq[threadIdx.x - 192], &s_sn[threadIdx.x - 192],
           &s_cs[threadIdx.x - 192]);
  if ((int)threadIdx.x < k) {
    const int id = p.ids[(size_t)(b / p.id_div) * k + threadIdx.x];
    int L = 0;
    int64_t off = 0, voff = 0;
    if (id >= 0 && id < p.n_src) {
      L = p.slen[id];
      off = p.soff[id];
      voff = p.svoff ? p.svoff[id] : off;
    }
    const int64_t Lp = p.svoff ? (L + kAttnTile - 1) / kAttnTile * kAttnTile : L;
    s_len[threadIdx.x] = L;
    s_koff[threadIdx.x] = (off * p.h_kv + (int64_t)h * L) * kD;
    s_voff[threadIdx.x] = (voff * p.h_kv + (int64_t)h * Lp) * kD;
  } else if ((int)threadIdx.x == k) {
    const int64_t seq = p.loc_shared ? 0 : b;
    const int64_t tp = (p.L_loc + kAttnTile - 1) / kAttnTile;  // padded local tiles
    s_len[k] = p.causal_off < 0 ? p.L_loc : min(p.L_loc, p.causal_off + b + 1);
    s_koff[k] = (seq * p.h_kv + h) * p.L_loc * kD;
    s_voff[k] = (seq * p.h_kv + h) * tp * kAttnTile * kD;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int r = 0; r <= k; ++r) {
      s_tile0[r] = acc;
      acc += (s_len[r] + kAttnTile - 1) / kAttnTile;
    }
    s_tile0[k + 1] = acc;
  }
  if (p.inv_freq) {
    // rotate-half RoPE at q_pos and the log2(e)/sqrt(d) scale, in float64
    // and rounded once, as the query RoPE kernel does; one (head, pair) per
    // thread, into LDS
    const double scale = 1.4426950408889634 / sqrt((double)kD);
    const T* qraw = (const T*)p.q + ((size_t)b * p.h_q + (size_t)h * G) * kD;
    for (int t = threadIdx.x; t < G * 64; t += 256) {
      const int g = t >> 6, pair = t & 63;
      const double x1 = St<T>::load(qraw[g * kD + pair]), x2 = St<T>::load(qraw[g * kD + 64 + pair]);
      const double cs = s_cs[pair], sn = s_sn[pair];
      s_q[g * kD + pair] = St<T>::store((x1 * cs - x2 * sn) * scale);
      s_q[g * kD + 64 + pair] = St<T>::store((x2 * cs + x1 * sn) * scale);
    }
  }
  __syncthreads();

  const int NT = __builtin_amdgcn_readfirstlane(s_tile0[k + 1]);
  const int u0 = (int)((int64_t)NT * split / p.S);
  const int u1 = (int)((int64_t)NT * (split + 1) / p.S);
  const int j = lane & 7, g8 = lane >> 3;
  const int tau = 8 * j + g8;  // token this lane scores after the reduction
  const T* qrow = (const T*)p.q + ((size_t)b * p.h_q + (size_t)h * G) * kD;

  // query fragments: 16 channels per lane (bf16: chunks j and j+8 of 8;
  // fp32: chunks j, j+8, j+16, j+24 of 4)
  constexpr int QV = kBF ? 2 : 4;  // 16-byte vectors per lane per head
  uint4 qf[G][QV];
  const T* qsrc = p.inv_freq ? s_q : qrow;
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < QV; ++c)
      qf[g][c] = *reinterpret_cast<const uint4*>(qsrc + (size_t)g * kD +
                                                 (kBF ? (c * 64 + 8 * j) : (c * 32 + 4 * j)));

  float m_run[G], l_run[G], o[8 * G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 8 * G; ++i) o[i] = 0.f;
  const int c4 = lane & 3, r0 = lane >> 2;  // PV: token chunk c4 (16 tokens), row r0

  int r = 0;
  for (int u = u0; u < u1; ++u) {
    while (u >= __builtin_amdgcn_readfirstlane(s_tile0[r + 1])) ++r;
    const int t0 = (u - __builtin_amdgcn_readfirstlane(s_tile0[r])) * kAttnTile;
    const int nvalid = min(kAttnTile, __builtin_amdgcn_readfirstlane(s_len[r]) - t0);
    const bool loc = r == k;
    const int64_t koff = ((int64_t)__builtin_amdgcn_readfirstlane((int)(s_koff[r] >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)s_koff[r]);
    const int64_t voff = ((int64_t)__builtin_amdgcn_readfirstlane((int)(s_voff[r] >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)s_voff[r]);
    const T* kb = (const T*)(loc ? p.kl : p.ks) + koff + (size_t)t0 * kD;
    const T* vb = (const T*)(loc ? p.vl : p.vs) + voff + (size_t)t0 * kD;  // [128][64] block

    // ---- loads: K 8 token rows x QV vectors; V 8 channel rows x VV vectors.
    // Document tiles are always full (lengths are multiples of 256); only a
    // ragged local tail takes the guarded path.  K loads carry the
    // nontemporal hint; V loads do not (measured: the hint on K raised the
    // 1M-token decode by 6-9% and the 3-hop interleave's attention by 3-6%,
    // while on V it slowed the interleave's long-document attention).
    constexpr int VV = kBF ? 2 : 4;  // 16-byte vectors per lane per row (16 tokens)
    uint4 kv[8][QV];
    uint4 vv[8][VV];
    const bool vok = 16 * c4 < nvalid;
    if (nvalid == kAttnTile) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int c = 0; c < QV; ++c)
          kv[s][c] = ld_nt(kb + (size_t)(8 * s + g8) * kD + (kBF ? (c * 64 + 8 * j) : (c * 32 + 4 * j)));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < VV; ++c)
          vv[i][c] = *reinterpret_cast<const uint4*>(vb + (16 * i + r0) * kAttnTile + 16 * c4 +
                                                     c * (16 / (int)sizeof(T)));
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int tt = 8 * s + g8;
#pragma unroll
        for (int c = 0; c < QV; ++c) {
          kv[s][c] = make_uint4(0, 0, 0, 0);
          if (tt < nvalid)
            kv[s][c] = ld_nt(kb + (size_t)tt * kD + (kBF ? (c * 64 + 8 * j) : (c * 32 + 4 * j)));
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < VV; ++c) {
          vv[i][c] = make_uint4(0, 0, 0, 0);
          if (vok)
            vv[i][c] = *reinterpret_cast<const uint4*>(vb + (16 * i + r0) * kAttnTile +
                                                       16 * c4 + c * (16 / (int)sizeof(T)));
        }
    }

    // ---- scores: partial dots over this lane's 16 channels
    float acc[8 * G];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < QV; ++c) {
          if constexpr (kBF) {
            a = dot2_bf16(kv[s][c].x, qf[g][c].x, a);
            a = dot2_bf16(kv[s][c].y, qf[g][c].y, a);
            a = dot2_bf16(kv[s][c].z, qf[g][c].z, a);
            a = dot2_bf16(kv[s][c].w, qf[g][c].w, a);
          } else {
            a = fmaf(__uint_as_float(kv[s][c].x), __uint_as_float(qf[g][c].x), a);
            a = fmaf(__uint_as_float(kv[s][c].y), __uint_as_float(qf[g][c].y), a);
            a = fmaf(__uint_as_float(kv[s][c].z), __uint_as_float(qf[g][c].z), a);
            a = fmaf(__uint_as_float(kv[s][c].w), __uint_as_float(qf[g][c].w), a);
          }
        }
        acc[s * G + g] = a;
      }
    treduce8<8 * G>(acc, j);  // lane now holds token tau's G scores in acc[0..G)

    // ---- online softmax (base 2; scores are pre-scaled by log2 e)
    const bool tv = tau < nvalid;
    const float bias = loc ? 0.f : p.doc_bias;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sc = tv ? acc[g] + bias : -INFINITY;
      const float m_new = fmaxf(m_run[g], wave_max(sc));
      const float alpha = exp2f(m_run[g] - m_new);
      const float pe = exp2f(sc - m_new);
      float pq;
      if constexpr (kBF) {
        const uint16_t pb = (uint16_t)f32_to_bf16(pe);
        s_p[wave][g][tau] = pb;
        pq = bf16_to_f32(pb);
      } else {
        s_p[wave][g][tau] = pe;
        pq = pe;
      }
      l_run[g] = l_run[g] * alpha + pq;
      m_run[g] = m_new;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i * G + g] *= alpha;
    }
    wave_lds_sync();

    // ---- values: zero tokens past the end of a ragged tail
    if (nvalid < kAttnTile && vok && nvalid - 16 * c4 < 16) {
      const int nv = nvalid - 16 * c4;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < VV; ++c) {
          uint32_t* w = reinterpret_cast<uint32_t*>(&vv[i][c]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (kBF) {
              const int t = c * 8 + 2 * e;
              if (t >= nv) w[e] = 0;
              else if (t + 1 >= nv) w[e] &= 0xffffu;
            } else {
              if (c * 4 + e >= nv) w[e] = 0;
            }
          }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint4 pp[VV];
#pragma unroll
      for (int c = 0; c < VV; ++c)
        pp[c] = *reinterpret_cast<const uint4*>(&s_p[wave][g][16 * c4 + c * (16 / (int)sizeof(T))]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = o[i * G + g];
#pragma unroll
        for (int c = 0; c < VV; ++c) {
          if constexpr (kBF) {
            a = dot2_bf16(vv[i][c].x, pp[c].x, a);
            a = dot2_bf16(vv[i][c].y, pp[c].y, a);
            a = dot2_bf16(vv[i][c].z, pp[c].z, a);
            a = dot2_bf16(vv[i][c].w, pp[c].w, a);
          } else {
            a = fmaf(__uint_as_float(vv[i][c].x), __uint_as_float(pp[c].x), a);
            a = fmaf(__uint_as_float(vv[i][c].y), __uint_as_float(pp[c].y), a);
            a = fmaf(__uint_as_float(vv[i][c].z), __uint_as_float(pp[c].z), a);
            a = fmaf(__uint_as_float(vv[i][c].w), __uint_as_float(pp[c].w), a);
          }
        }
        o[i * G + g] = a;
      }
    }
    wave_lds_sync();  // probabilities consumed before the next tile overwrites them
  }

  // ---- wave epilogue: total l, 4-lane reduction of the accumulators
  float l_tot[G];
#pragma unroll
  for (int g = 0; g < G; ++g) l_tot[g] = wave_sum(l_run[g]);
  treduce<kDppXor2, 8 * G>(o, 8 * G, (c4 & 2) != 0);
  treduce<kDppXor1, 8 * G>(o, 4 * G, (c4 & 1) != 0);  // lane keeps o indices [2G*c4, 2G*c4 + 2G)
  const size_t pbase = (((size_t)b * p.h_kv + h) * p.S + split) * G;
#pragma unroll
  for (int e = 0; e < 2 * G; ++e) {
    const int idx = 2 * G * c4 + e;
    const int i = idx / G, g = idx % G;
    p.part[(pbase + g) * (kD + 2) + 2 + 16 * i + r0] = o[e];
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
    if (lane == g) {
      p.part[(pbase + g) * (kD + 2) + 0] = m_run[g];
      p.part[(pbase + g) * (kD + 2) + 1] = l_tot[g];
    }
}

// merge the S partials of each (query, KV head): log-sum-exp in base 2.
// One workgroup per (KV head, query); the (split, head) weights go through
// LDS, then each thread owns (head, channel) outputs and streams the splits.
template <int G>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part, int S,
                                                      int h_kv, int h_q, float* __restrict__ out) {
  constexpr int kMaxSG = 2048;
  __shared__ float s_w[kMaxSG];
  __shared__ float s_l[kMaxSG];
  __shared__ float s_M[G], s_L[G];
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const float* pb = part + ((size_t)b * h_kv + h) * S * G * (kD + 2);
  const int SG = S * G;
  for (int i = t; i < SG; i += 256) {
    s_w[i] = pb[(size_t)i * (kD + 2)];
    s_l[i] = pb[(size_t)i * (kD + 2) + 1];
  }
  __syncthreads();
  if (t < G) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, s_w[s * G + t]);
    s_M[t] = M;
  }
  __syncthreads();
  for (int i = t; i < SG; i += 256) {
    const float M = s_M[i % G];
    s_w[i] = M == -INFINITY ? 0.f : exp2f(s_w[i] - M);
  }
  __syncthreads();
  if (t < G) {
    float L = 0.f;
    for (int s = 0; s < S; ++s) L = fmaf(s_w[s * G + t], s_l[s * G + t], L);
    s_L[t] = L;
  }
  __syncthreads();
  for (int e = t; e < G * kD; e += 256) {
    const int g = e / kD, d = e % kD;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 8 <= S; s += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pb[((size_t)(s + u) * G + g) * (kD + 2) + 2 + d];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = fmaf(s_w[(s + u) * G + g], v[u], a[u]);
    }
    for (; s < S; ++s) a[0] = fmaf(s_w[s * G + g], pb[((size_t)s * G + g) * (kD + 2) + 2 + d], a[0]);
    const float acc = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    const float L = s_L[g];
    out[((size_t)b * h_q + (size_t)h * G + g) * kD + d] = L > 0.f ? acc / L : 0.f;
  }
}

template <typename T, int G>
hipError_t run_decode(const DecodeP& p, int B, float* out, hipStream_t s) {
  const dim3 grid((unsigned)(p.S / 4), (unsigned)p.h_kv, (unsigned)B);
  timer_mark(0, true, s);
  hipLaunchKernelGGL((decode_kernel<T, G>), grid, dim3(256), 0, s, p);
  timer_mark(0, false, s);
  hipLaunchKernelGGL((combine_kernel<G>), dim3((unsigned)p.h_kv, (unsigned)B), dim3(256), 0, s,
                     p.part, p.S, p.h_kv, p.h_q, out);
  return hipGetLastError();
}

}  // namespace

size_t decode_partial_floats(int B, int h_kv, int G, int splits) {
  return (size_t)B * h_kv * splits * G * (kD + 2);
}

int decode_auto_splits(const Bank& bk, int B, int k, int L_loc, double doc_tiles) {
  // At least one long-running wave per SIMD (1024 waves on 256 CUs): each
  // wave walks a long contiguous run of tiles, which streams best when the
  // unions are of equal length.  With documents of mixed lengths the unions
  // differ from query to query, and a wave per about 32 tiles of the
  // expected union lets short unions' waves finish and make room for the
  // rest of the long ones.  Splits come in multiples of 4 (one workgroup =
  // 4 waves) and never exceed the tiles.
  const double tiles = k * doc_tiles + (L_loc + kAttnTile - 1) / kAttnTile;
  const int64_t pairs = std::max<int64_t>(1, (int64_t)B * bk.desc.h_kv);
  int s = (int)((1024 + pairs - 1) / pairs);
  s = std::max(s, (int)std::ceil(tiles / 32.0));
  s = (int)std::min<double>(s, std::max(4.0, tiles));
  s = std::max(4, ((s + 3) / 4) * 4);
  return std::min(s, 256);
}

hipError_t launch_decode(const Bank& bk, const void* q, int q_pos, int B, int h_q,
                         const int32_t* ids, int k, const AttnSources& src, const void* k_loc,
                         const void* v_loc, int L_loc, int splits, float* part, float* out,
                         hipStream_t s) {
  DecodeP p;
  p.q = q;
  p.inv_freq = bk.d_inv_freq;
  p.q_pos = q_pos;
  p.ids = ids;
  p.ks = src.k;
  p.vs = src.v;
  p.soff = src.off;
  p.slen = src.len;
  p.n_src = src.n;
  p.svoff = src.voff;
  p.doc_bias = src.bias;
  p.kl = k_loc;
  p.vl = v_loc;
  p.k = k;
  p.L_loc = L_loc;
  p.h_kv = bk.desc.h_kv;
  p.S = splits;
  p.h_q = h_q;
  p.part = part;
  p.id_div = 1;
  p.loc_shared = 0;
  p.causal_off = -1;
  const int G = h_q / bk.desc.h_kv;
  const bool bf = bk.desc.dtype == MSA_BF16;
#define MSA_DEC(GG)                                                              \
  case GG:                                                                       \
    return bf ? run_decode<uint16_t, GG>(p, B, out, s) : run_decode<float, GG>(p, B, out, s);
  switch (G) {
    MSA_DEC(1)
    MSA_DEC(2)
    MSA_DEC(4)
    MSA_DEC(8)
    default:
      return hipErrorInvalidValue;
  }
#undef MSA_DEC
}

}  // namespace msa

namespace msa {

// Blocked prefill on the decode kernel: every query token is its own split-K
// job that reads its block's document set and a causal prefix of the shared
// local context.  Exact, but each block's documents are re-read per query;
// the MFMA kernel in prefill.hip shares them across the block.
hipError_t launch_prefill_vector(const Bank& bk, const void* q_rot, int n_q, int h_q,
                                 const int32_t* ids, int k, int block, const AttnSources& src,
                                 const void* k_loc, const void* v_loc, int L_loc, int splits,
                                 float* part, float* out, hipStream_t s) {
  DecodeP p;
  p.q = q_rot;
  p.inv_freq = nullptr;
  p.q_pos = 0;
  p.ids = ids;
  p.ks = src.k;
  p.vs = src.v;
  p.soff = src.off;
  p.slen = src.len;
  p.n_src = src.n;
  p.svoff = src.voff;
  p.doc_bias = src.bias;
  p.kl = k_loc;
  p.vl = v_loc;
  p.k = k;
  p.L_loc = L_loc;
  p.h_kv = bk.desc.h_kv;
  p.S = splits;
  p.h_q = h_q;
  p.part = part;
  p.id_div = block;
  p.loc_shared = 1;
  p.causal_off = L_loc - n_q;
  const int G = h_q / bk.desc.h_kv;
  const bool bf = bk.desc.dtype == MSA_BF16;
#define MSA_DEC(GG)                                                                   \
  case GG:                                                                            \
    return bf ? run_decode<uint16_t, GG>(p, n_q, out, s) : run_decode<float, GG>(p, n_q, out, s);
  switch (G) {
    MSA_DEC(1)
    MSA_DEC(2)
    MSA_DEC(4)
    MSA_DEC(8)
    default:
      return hipErrorInvalidValue;
  }
#undef MSA_DEC
}

}  // namespace msa
