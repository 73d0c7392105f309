// Blocked prefill attention on the matrix cores.
//
// Each block of `block` consecutive query tokens shares one set of selected
// documents ("MSA" card, robocikowo.com, "Komponenty": the MSA layer appends
// the top-k documents' K/V to the local context); query i attends to every
// token of its block's documents and to local tokens j <= its own local index
// (causal), with the 1/sqrt(d) scale (mlqm.cn MLA/CSA article, section 6.2).
//
// One workgroup = (block of 64 queries, KV head, token split): 256 rows
// (64 queries x 4 query heads of the KV head) in 8 waves of 32 rows, two
// waves per SIMD so one wave's softmax overlaps the other's matrix work.
// Each 64-token K/V tile is staged once in LDS and shared by all 256 rows:
// 256 flop per byte of K/V.  Tiles stream through a 4-stage LDS ring filled
// by direct global->LDS loads through buffer descriptors (no register
// staging), three tiles in flight while one is consumed.  Both contractions use v_mfma_f32_32x32x16_bf16 with
// fp32 accumulation.  Scores are computed transposed, S^T = K . Q^T (tokens
// x rows), so the accumulator of S^T is already laid out as the B operand
// P^T of O^T = V^T . P^T; K rows are permuted inside each 16-row group when
// staged so that every lane's 8 probabilities of a 16-token k-step are 8
// consecutive tokens, i.e. one 16-byte V^T read.  Online softmax in base 2
// (queries are pre-scaled by log2 e / sqrt(d)).  With a single token split
// the kernel writes the normalised output; otherwise per-split partials
// that prefill_combine_kernel merges.
#include <algorithm>
#include <type_traits>

#include "msa_internal.h"

namespace msa {

hipError_t launch_prefill_vector(const Bank& bk, const void* q_rot, int n_q, int h_q,
                                 const int32_t* ids, int k, int block, const AttnSources& src,
                                 const void* k_loc, const void* v_loc, int L_loc, int splits,
                                 float* part, float* out, hipStream_t s);

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kRows = 256;           // rows per workgroup (64 queries x 4 heads)
constexpr int kQBlock = 64;          // queries per routing block handled here
constexpr int kPG = 4;               // query heads per KV head handled here
constexpr int kWaves = 8;            // 32 rows each
constexpr int kThreads = 64 * kWaves;
constexpr int kTileB = 64 * kD * 2;  // bytes of one K (or V) tile in bf16
constexpr int kStages = 4;           // LDS ring depth (K + V tile per stage)

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
  float* out;   // [n_q][h_q][128]: written directly when S == 1
};

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b,
                                           const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// hardware round-to-nearest-even pack of two floats into a bf16 pair
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// One 16-byte global->LDS copy per lane through a buffer descriptor: lane l
// reads bytes [voff, voff + 16) of the buffer (zeros past its range) and they
// land at lds_wave_base + 16*l (the base is wave-uniform).  The buffer form,
// unlike the flat-encoded global one, leaves the compiler's count of
// outstanding LDS reads exact, so fragment reads can be pipelined while ring
// loads are in flight.
constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufWord3);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base,
                                           16, voff, 0, 0, 0);
}

// max over lanes l and l ^ 32: a swap of the wave's halves (one VALU op, no
// LDS round trip); with the same register as both operands, the two results
// hold this lane's value and its partner's in some order
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// LDS row r of a staged K tile holds token perm16(r): bits 2 and 3 swapped.
__device__ __forceinline__ int perm16(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// s_waitcnt immediates that wait on the vector-memory counter only
// (vmcnt in bits 3:0, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
constexpr int kWaitVm0 = 0xF70, kWaitVm4 = 0xF74, kWaitVm8 = 0xF78;

// Workgroup barrier after waiting until at most WAIT_IMM's count of this
// lane's ring loads are in flight.  No memory fence: the loads being waited
// for write LDS only, and a fence's wait for every outstanding load would
// drain the ring.  The wait goes through the builtin (not asm) so the
// compiler's own wait insertion sees it and adds none of its own.
template <int WAIT_IMM>
__device__ __forceinline__ void wait_ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(WAIT_IMM);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct Tile {
  const uint16_t* kb;
  const uint16_t* vb;
  int nvalid;
  int t0;  // token offset inside the segment
  bool local;
};

__global__ __launch_bounds__(kThreads) void prefill_mfma_kernel(PrefillP p) {
  const int split = blockIdx.x, h = blockIdx.y, blk = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int k = p.k;
  const int causal_base = p.L_loc - p.n_q;  // local index of query 0

  __shared__ int64_t s_koff[kMaxK + 1], s_voff[kMaxK + 1];
  __shared__ int s_len[kMaxK + 1], s_tile0[kMaxK + 2];
  // the ring: one array per stage (K tile, then V^T tile), so the compiler
  // can tell the stages apart and wait only on the loads that fill a stage
  __shared__ __attribute__((aligned(1024))) uint8_t s_kv0[2 * kTileB];
  __shared__ __attribute__((aligned(1024))) uint8_t s_kv1[2 * kTileB];
  __shared__ __attribute__((aligned(1024))) uint8_t s_kv2[2 * kTileB];
  __shared__ __attribute__((aligned(1024))) uint8_t s_kv3[2 * kTileB];
  static_assert(kStages == 4, "one array per ring stage");
  auto stage_buf = [&](auto st) -> uint8_t* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? s_kv0 : S == 1 ? s_kv1 : S == 2 ? s_kv2 : s_kv3;
  };

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

  // ---- this lane's row: R = 32*wave + l32 -> query 8*wave + l32/4, head l32%4.
  // Q^T B operand of k-step kk: channels 16*kk + 8*hl .. +7 of that row.
  bf16x8_t qf[8];
  {
    const int qi = blk * kQBlock + 8 * wave + (l32 >> 2);
    const uint16_t* qrow = p.q + ((size_t)qi * p.h_q + (size_t)h * kPG + (l32 & 3)) * kD + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + 16 * kk));
  }
  // Q must have landed before the ring starts: its wait counts assume
  // nothing else in flight (an asm use makes the compiler wait here).
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) asm volatile("" ::"v"(qf[kk]));
  const int li_wave_min = causal_base + blk * kQBlock + 8 * wave;
  const int li = li_wave_min + (l32 >> 2);  // local (causal) index of this lane's row

  f32x16_t o[4];  // O^T: [channel tile 0..3], column = this lane's row
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  // -ref_of(m_run) in every element: the accumulator a score tile starts
  // from, so scores come out relative to the row's reference
  f32x16_t negm;
#pragma unroll
  for (int e = 0; e < 16; ++e) negm[e] = 0.f;

  // Tile cursors.  Tile u of the split walks the segments (the selected
  // documents in rank order, then the local context) 64 tokens at a time; a
  // cursor keeps its segment's values in scalar registers and reads the
  // segment table only when it crosses into the next segment.
  auto rfl = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  auto rfl64 = [&](int64_t v) {
    return (int64_t)(((uint64_t)(uint32_t)rfl((int)(v >> 32)) << 32) | (uint32_t)rfl((int)v));
  };
  struct Cursor {
    int u, r, end, t0, len;
    const uint16_t* kb;  // segment's K rows for this KV head
    const uint16_t* vb;  // segment's V^T tiles for this KV head
  };
  auto load_seg = [&](Cursor& c) __attribute__((always_inline)) {
    c.end = rfl(s_tile0[c.r + 1]);
    c.len = rfl(s_len[c.r]);
    c.kb = (c.r == k ? p.kl : p.ks) + rfl64(s_koff[c.r]);
    c.vb = (c.r == k ? p.vl : p.vs) + rfl64(s_voff[c.r]);
  };
  auto seek = [&](Cursor& c, int u) __attribute__((always_inline)) {
    c.u = u;
    c.r = 0;
    while (u >= rfl(s_tile0[c.r + 1])) ++c.r;
    load_seg(c);
    c.t0 = (u - rfl(s_tile0[c.r])) * 64;
  };
  // next tile, or stay on the split's last tile
  auto advance = [&](Cursor& c, int u_stop) __attribute__((always_inline)) {
    if (c.u >= u_stop) return;
    ++c.u;
    if (c.u < c.end) {
      c.t0 += 64;
      return;
    }
    do ++c.r;
    while (c.u >= rfl(s_tile0[c.r + 1]));
    load_seg(c);
    c.t0 = 0;
  };
  auto tile_of = [&](const Cursor& c) __attribute__((always_inline)) {
    Tile t;
    t.t0 = c.t0;
    t.nvalid = min(64, c.len - c.t0);
    t.local = c.r == k;
    t.kb = c.kb + (size_t)c.t0 * kD;
    t.vb = c.vb + (size_t)c.t0 * kD;
    return t;
  };
  // Stage a tile: wave w's load i fills 1 KB j = w + 8*i of the K tile (LDS
  // rows 4j..4j+3, 16-byte chunk c of row r at slot c ^ (r & 15)) and 1 KB j
  // of the V^T tile (channel rows 8j..8j+7, chunk cv of row d at slot
  // cv ^ ((d >> 1) & 7)).  The LDS has 64 four-byte banks and serves a
  // 16-byte-per-lane read 16 lanes at a time: K rows are 256 bytes, so 16
  // consecutive rows must use 16 different slots; V^T rows are 128 bytes, so
  // rows d and d + 1 already sit in different halves of the banks and the
  // slot must differ across rows of equal parity.  V^T tiles are
  // zero-padded in memory.
  int kofs[2], vofs[2];  // byte offsets of this lane's loads in each half of a tile
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = wave + kWaves * i;
    const int r = 4 * j + (lane >> 4);
    kofs[i] = perm16(r) * 256 + 16 * ((lane & 15) ^ (r & 15));
    const int d = 8 * j + (lane >> 3);
    vofs[i] = d * 128 + 16 * ((lane & 7) ^ ((d >> 1) & 7));
  }
  // The K buffer ends at the tile's last valid token, so rows past it load
  // as zeros (their scores are masked).
  auto issue = [&](const Tile& t, uint8_t* base) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(t.kb, t.nvalid * 256);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(t.vb, kTileB);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(rk, kofs[i], base + 1024 * (wave + kWaves * i));
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(rv, vofs[i], base + kTileB + 1024 * (wave + kWaves * i));
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // K fragment (A operand) of the staged tile for token half mt, k-step kk:
  // LDS row 32*mt + l32, channels 16*kk + 8*hl .. +7
  auto kfrag = [&](const uint8_t* sk, int mt, int kk) __attribute__((always_inline)) {
    const int row = 32 * mt + l32, c = 2 * kk + hl;
    return __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const uint4*>(&sk[row * 256 + ((c ^ (row & 15)) << 4)]));
  };
  // V^T fragment (A operand) for channel tile dt, 16-token k-step ks: channel
  // 32*dt + l32, tokens 16*ks + 8*hl .. +7
  auto vfrag = [&](const uint8_t* sv, int ks, int dt) __attribute__((always_inline)) {
    const int d = 32 * dt + l32, cv = 2 * ks + hl;
    return __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const uint4*>(&sv[d * 128 + ((cv ^ ((d >> 1) & 7)) << 4)]));
  };
  auto ref_of = [](float m) { return m == -INFINITY ? 0.f : m; };

  // Scores of a tile, sc = S^T - m_ref, as two 32-token halves (mt).
  // Element e of sc[mt] is token 32*mt + 16*(e/8) + 8*hl + e%8 (the staged
  // row permutation), column = this lane's row.
  //
  // Before a tile's probabilities: mask, row max and the lazy rescale.
  // Probabilities are relative to a per-row reference m_run that moves
  // (rescaling O and l) only when a row max exceeds it by more than 8 in log2
  // units, so p <= 256 and O is rarely touched.  The scores were taken
  // relative to ref_of(m_run), which has not moved since.
  auto softmax_pre = [&](const Tile& cur, f32x16_t(&sc)[2]) __attribute__((always_inline)) {
    const float m_use = ref_of(m_run);
    // Tile tokens past the segment's end, and local tokens after this row's
    // own position, are masked: token t is kept iff t < lim.
    if (cur.nvalid < 64 || (cur.local && cur.t0 + 63 > li_wave_min)) {
      const int lim = (cur.local ? min(cur.nvalid, li - cur.t0 + 1) : cur.nvalid) - 8 * hl;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sc[mt][e] = 32 * mt + 16 * (e >> 3) + (e & 7) < lim ? sc[mt][e] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[mt][e]);
    mx = max_xor32(mx);  // relative to m_use
    const bool grow = mx + m_use > m_run + 8.f;
    if (__builtin_amdgcn_readfirstlane((int)(__ballot(grow) != 0))) {
      if (grow) {
        const float m_new = mx + m_use;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) sc[mt][e] -= mx;
#pragma unroll
        for (int e = 0; e < 16; ++e) negm[e] = -m_new;
      }
    }
  };

  // Software pipeline: the scores of tile u + 1 go onto the matrix cores in
  // the same straight-line block as tile u's exponentials and P.V, so the
  // matrix and vector units overlap.  Every ring step issues exactly one
  // tile (past the split's end the cursors stay on its last tile, and a
  // score pass past the end is discarded), so the ring's wait counts are the
  // same on every path.  Score tiles alternate between two register sets.
  const int u_last = u1 - 1;
  f32x16_t sA[2], sB[2];
  Tile cur{};
  Cursor ci{}, cc{};  // issue cursor (three tiles ahead) and compute cursor
  if (u0 < u1) {
    seek(ci, u0);
    cc = ci;
    issue(tile_of(ci), stage_buf(I0{}));
    advance(ci, u_last);
    issue(tile_of(ci), stage_buf(I1{}));
    advance(ci, u_last);
    issue(tile_of(ci), stage_buf(I2{}));
    advance(ci, u_last);
    wait_ring_barrier<kWaitVm8>();  // tile u0 landed
    cur = tile_of(cc);
    const uint8_t* sk = stage_buf(I0{});
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sA[mt] = mfma32(kfrag(sk, mt, 0), qf[0], negm);
#pragma unroll
      for (int kk = 1; kk < 8; ++kk) sA[mt] = mfma32(kfrag(sk, mt, kk), qf[kk], sA[mt]);
    }
  }

  // ring step for tile u in stage st: tile u + 1 (stage st + 1) must have
  // landed; tile u + 3 goes to stage st + 3, which held tile u - 1
  auto step = [&](auto st, int u, f32x16_t(&sc)[2], f32x16_t(&sn)[2]) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    wait_ring_barrier<kWaitVm4>();
    issue(tile_of(ci), stage_buf(std::integral_constant<int, (S + kStages - 1) % kStages>{}));
    advance(ci, u_last);
    if (u >= u1) return;
    softmax_pre(cur, sc);
    advance(cc, u_last);
    const Tile nxt = tile_of(cc);
    const uint8_t* sk = stage_buf(std::integral_constant<int, (S + 1) % kStages>{});
    const uint8_t* sv = stage_buf(st) + kTileB;
    // k-step ks: 4 score MFMAs of tile u + 1 (half ks/2, k-steps
    // 4*(ks%2) .. +3), then tile u's probabilities for tokens 16*ks + 8*hl
    // .. +7 (elements 8*(ks%2) .. +7 of sc[ks/2]) as bf16 and their 4 P.V
    // MFMAs.  The row sum takes the rounded p.
    const uint32_t ones = 0x3f803f80u;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int mt = ks >> 1, kk = 4 * (ks & 1) + j;
        sn[mt] = mfma32(kfrag(sk, mt, kk), qf[kk], kk == 0 ? negm : sn[mt]);
      }
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 8 * (ks & 1) + 2 * i;
        w[i] = cvt_pk_bf16(__builtin_amdgcn_exp2f(sc[ks >> 1][e]),
                           __builtin_amdgcn_exp2f(sc[ks >> 1][e + 1]));
        l_run = dot2_bf16(w[i], ones, l_run);
      }
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(vfrag(sv, ks, dt), pb, o[dt]);
    }
    cur = nxt;
  };
  for (int u = u0; u < u1; u += kStages) {
    // all four steps run on every pass, so every wave meets the same
    // barriers and the wait counts hold on every path
    step(I0{}, u, sA, sB);
    step(I1{}, u + 1, sB, sA);
    step(I2{}, u + 2, sA, sB);
    step(I3{}, u + 3, sB, sA);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no load may still write LDS after the workgroup ends

  // ---- this lane's row (both lane halves hold half the tokens' l)
  l_run += __shfl_xor(l_run, 32, 64);
  if (p.S == 1) {
    // one split: the merge reduces to o / l, so write the output directly
    // (row R -> query R/4, head R%4 of this KV head)
    const int R = 32 * wave + l32;
    float* orow = p.out + ((size_t)(blk * kQBlock + (R >> 2)) * p.h_q + (size_t)h * kPG + (R & 3)) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        orow[32 * dt + 8 * (e >> 2) + 4 * hl + (e & 3)] = l_run > 0.f ? o[dt][e] / l_run : 0.f;
    return;
  }
  float* pr = p.part + ((((size_t)blk * p.h_kv + h) * p.S + split) * kRows + 32 * wave + l32) * (kD + 2);
  if (hl == 0) {
    pr[0] = m_run;
    pr[1] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) pr[2 + 32 * dt + 8 * (e >> 2) + 4 * hl + (e & 3)] = o[dt][e];
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
  // row R -> query R/4, head R%4 of this KV head
  const int qi = blk * kQBlock + (row >> 2);
  out[((size_t)qi * h_q + (size_t)h * kPG + (row & 3)) * kD + d] = L > 0.f ? acc / L : 0.f;
}

}  // namespace

size_t prefill_partial_floats(int n_q, int h_kv, int splits) {
  return (size_t)(n_q / kQBlock) * h_kv * splits * kRows * (kD + 2);
}

int prefill_auto_splits(const Bank& bk, int n_q, int k, int L_loc) {
  // one workgroup per compute unit (a workgroup holds 128 KiB of LDS)
  const int n_blocks = std::max(1, n_q / kQBlock);
  const int64_t wg = (int64_t)n_blocks * bk.desc.h_kv;
  const double avg_doc = (double)bk.n_tokens / bk.desc.n_docs;
  const int tiles = (int)std::max(1.0, k * avg_doc / 64 + (L_loc + 63) / 64);
  int s = (int)((256 + wg - 1) / wg);
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
  p.out = out;
  const int n_blocks = n_q / kQBlock;
  timer_mark(0, true, s);
  hipLaunchKernelGGL(prefill_mfma_kernel, dim3((unsigned)splits, (unsigned)p.h_kv, (unsigned)n_blocks),
                     dim3(kThreads), 0, s, p);
  timer_mark(0, false, s);
  if (splits > 1)
    hipLaunchKernelGGL(prefill_combine_kernel, dim3(kRows / 2, (unsigned)p.h_kv, (unsigned)n_blocks),
                       dim3(256), 0, s, part, splits, p.h_kv, h_q, out);
  return hipGetLastError();
}

}  // namespace msa
