// Device code of the decode kernel, shared by the decode launch (decode.hip)
// and the fused mixed-step launch (mixed.hip).
#pragma once

// Batched GQA decode over a paged KV cache (FlashInferDecodeWrapper.run on the
// mstar attn.wrappers page; split-KV partials in the workspace, attn.workspace).
//
// Work comes as a worker table: worker w is num_kv_heads wavefronts, one per KV
// head, that run the key-range pieces [work[w], work[w + 1]) in order; the
// planner gives every worker about the same number of pages, so the waves of a
// launch finish together.  A piece is a contiguous key range of one row.
//
// A key row of one KV head is head_dim bf16 = D*2 bytes, contiguous in the
// cache; it is spread over LPK = D/8 lanes, 16 bytes each, so one wave-wide load
// fetches KPL = 64/LPK whole key rows with fully used 16-byte lane accesses.  An
// iteration issues U such loads for K and U for V (KB = KPL*U keys) and the
// next iteration's loads go out before the current one is computed.  K and V
// are streamed once, so they are loaded non-temporal.
//
// Scores: each lane forms the partial dot product of its 8 dimensions with the
// group's G query heads (bf16 dot2).  With D = 128 and G of 4 or 8 a block
// holds 16 (key, head) pairs per 16-lane key row; a DPP reduce-scatter leaves
// one whole score per lane, so each exponential is taken once, and the
// probabilities return to the lanes by row broadcasts.  Other shapes use a DPP
// allreduce over the LPK lanes of a key.
// Softmax: the KPL lane groups of a wave each keep their own running max, sum
// and output accumulator (fp32, in registers) over the keys they see; the
// groups are combined once, at the end of the piece, by log-sum-exp.  The
// running max moves only when a block exceeds it by more than 2^8, and P.V
// takes two keys per v_dot2_f32_bf16 with P rounded to bf16, so the vector ALU
// work per byte stays well below what the stream leaves room for.  Only blocks
// that cross a piece's first or last key mask keys.
//
// Memory traffic is one read of every visible K and V byte: the kernel is
// bound by HBM bandwidth.
#include <type_traits>

#include "common.cuh"
#include "kernels.h"

namespace pkv {
namespace dec {

constexpr int kWaves = 4;  // waves per workgroup

// Loads per iteration (each for K and V).  With 8 query heads per KV head the
// accumulators take twice the registers, so the load buffers are halved to
// keep every value in registers.
constexpr int decode_loads(int G) { return G == 8 ? 2 : 4; }

// One piece (keys [kv_start, kv_end) of one row) for KV head hk, by one wave.
template <int D, int G, bool ONE_PAGE_PER_ITER>
__device__ __forceinline__ void decode_piece(const DecodeArgs& a, int piece, int hk, int lane) {
  constexpr int LPK = D / 8;       // lanes per key row
  constexpr int KPL = 64 / LPK;    // key rows per wave load
  constexpr int U = decode_loads(G);  // loads per iteration (each for K and V)
  constexpr int KB = KPL * U;      // keys per iteration

  // Plan metadata is read-only for the launch: scalar loads.
  const auto tp = as_const4(a.pieces + piece);
  const int row_ref = tp->row;
  const int chunk = tp->chunk;
  const int ks = tp->kv_start;
  const int ke = tp->kv_end;
  const auto rp = as_const4(a.rows + row_ref);
  const int page_base = rp->page_base;
  const int q_index = rp->q_index;
  const int n_chunks = rp->n_chunks;
  const int out_slot = rp->slot0 >= 0 ? rp->slot0 + hk * n_chunks + chunk : -1;

  const int Hq = a.num_qo_heads;
  const int Hk = a.num_kv_heads;
  const int ps = a.page_size;
  const int ps_log2 = __builtin_ctz(ps);
  const int row_elems = Hk * D;                      // one token slot, all KV heads
  const int64_t page_elems = 2LL * ps * row_elems;   // K half + V half
  const int v_off = ps * row_elems;

  const int lk = lane / LPK;   // key row within a load
  const int ld = lane % LPK;   // 8-element segment of head_dim
  const uint32_t lane_off = hk * D + ld * 8;
  const_as4_ptr<int32_t> cidx = as_const4(a.indices);

  // Query heads hk*G .. hk*G+G-1, this lane's 8 dimensions, as packed bf16 pairs.
  uint32_t qw[G][4];
  {
    const uint16_t* qp = a.q + ((int64_t)q_index * Hq + hk * G) * D + ld * 8;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + h * D);
      qw[h][0] = v.x; qw[h][1] = v.y; qw[h][2] = v.z; qw[h][3] = v.w;
    }
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -1e30f;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  // Scattered softmax (D 128, 16 (key, head) pairs per block): lane li of a key
  // row's 16 lanes owns pair li, i.e. head li % G of key row kt_u(li); it keeps
  // its head's running max and its own share of the sum.
  constexpr bool kScatter = LPK == 16 && U * G == 16;
  const int li = lane & 15;
  float m_own = -1e30f, lsum = 0.f;

  // Key blocks of KB keys: block b starts at kb0 + b*KB; the last one holds key ke-1.
  const int kb0 = ks & ~(KB - 1);
  const int nb = (((ke - 1) & ~(KB - 1)) - kb0) / KB + 1;

  // Physical page of block b (one page per block): a uniform load through the
  // scalar unit, fetched one block ahead of the loads that use it.
  uint32_t lane_byte[U];  // byte offset of this lane's 16 bytes within a block
#pragma unroll
  for (int u = 0; u < U; ++u) lane_byte[u] = ((u * KPL + lk) * (uint32_t)row_elems + lane_off) * 2u;
  auto page_of = [&](int b) -> int {
    b = b < nb ? b : nb - 1;
    return cidx[page_base + ((kb0 + b * KB) >> ps_log2)];
  };

  // Issue the K and V loads of block b (clamped to the last block, so the
  // number of loads in flight is the same on every path).
  auto issue = [&](int b, int phys, uint4 (&kk)[U], uint4 (&vv)[U]) {
    b = b < nb ? b : nb - 1;
    const int kb = kb0 + b * KB;
    if constexpr (ONE_PAGE_PER_ITER) {
      // Uniform base (page and slot, scalar registers) + a loop-invariant 32-bit
      // byte offset per lane: no address arithmetic per block in vector registers.
      const char* kbase = reinterpret_cast<const char*>(a.cache) +
                          ((int64_t)phys * page_elems + (int64_t)(kb & (ps - 1)) * row_elems) * 2;
      const char* vbase = kbase + (int64_t)v_off * 2;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kk[u] = load_nt16(kbase + lane_byte[u]);
        vv[u] = load_nt16(vbase + lane_byte[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int j = kb + u * KPL + lk;
        j = j < ke ? j : ke - 1;  // keys past the chunk are masked; keep the address valid
        const int pg = a.indices[page_base + (j >> ps_log2)];
        const uint16_t* p = a.cache + (int64_t)pg * page_elems + (j & (ps - 1)) * row_elems +
                            lane_off;
        kk[u] = load_nt16(p);
        vv[u] = load_nt16(p + v_off);
      }
    }
  };

  const float sc = a.scale_log2;  // log2(e) / sqrt(D): scores in log2 units
  // Pair q of a block: key row u and head h with q = h + G * pair_u(u), where
  // for G = 4 the key rows 0, 1, 2, 3 sit at 0, 8, 4, 12 (and for G = 8 rows 0,
  // 1 at 0, 8), so the two keys of a P.V pair are 8 lanes apart (row_ror:8).
  auto pair_of = [](int u) { return G == 4 ? ((u & 1) << 3) | ((u >> 1) << 2) : u << 3; };
  auto scatter_blk = [&](const uint4 (&kk)[U], const uint4 (&vv)[U], int kb, auto edge_c) {
    constexpr bool kEdge = decltype(edge_c)::value;
    // Partial dot products of this lane's 8 dimensions, all 16 pairs.
    float v[16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = dot2_bf16(qw[h][0], kk[u].x, 0.f);
        acc = dot2_bf16(qw[h][1], kk[u].y, acc);
        acc = dot2_bf16(qw[h][2], kk[u].z, acc);
        acc = dot2_bf16(qw[h][3], kk[u].w, acc);
        v[pair_of(u) + h] = acc;
      }
    }
    // Reduce-scatter over the 16 lanes: each step halves the values a lane
    // holds; a lane keeps the half its lane bit selects, sends the other half to
    // the partner that differs in that bit and adds what it receives.  After
    // the four steps lane li holds the full score of pair li.
    const bool b3 = (li & 8) != 0, b2 = (li & 4) != 0, b1 = (li & 2) != 0, b0 = (li & 1) != 0;
    float w8[8], w4[4], w2[2];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w8[k] = (b3 ? v[k + 8] : v[k]) + dpp<kDppRowRor8>(b3 ? v[k] : v[k + 8]);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w4[k] = (b2 ? w8[k + 4] : w8[k]) + dpp<kDppRowHalfMirror>(b2 ? w8[k] : w8[k + 4]);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      w2[k] = (b1 ? w4[k + 2] : w4[k]) + dpp<kDppQuadXor2>(b1 ? w4[k] : w4[k + 2]);
    float sv = (b0 ? w2[1] : w2[0]) + dpp<kDppQuadXor1>(b0 ? w2[0] : w2[1]);
    if constexpr (kEdge) {
      const int ul = G == 4 ? ((li >> 3) & 1) | (((li >> 2) & 1) << 1) : li >> 3;
      const int j = kb + ul * KPL + lk;
      sv = (j >= ks && j < ke) ? sv : -INFINITY;
    }
    // The block's maximum of this lane's head (its lanes are li mod G apart).
    float mx = sv;
    if constexpr (G == 4) mx = fmaxf(mx, dpp<kDppRowRor4>(mx));
    mx = fmaxf(mx, dpp<kDppRowRor8>(mx));
    const float mxs = mx * sc;
    if (__builtin_amdgcn_ballot_w64(mxs > m_own + 8.f) != 0) {
      const float mn = fmaxf(m_own, mxs);
      const float alpha = fast_exp2(m_own - mn);
      m_own = mn;
      lsum *= alpha;
#pragma unroll
      for (int h = 0; h < G; ++h) {  // lane h holds head h
        const float ah = bcast16(alpha, h);
        m[h] = bcast16(m_own, h);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= ah;
      }
    }
    const float p = fast_exp2(fmaf(sv, sc, -m_own));
    lsum += p;
    // (p of key row u, p of key row u + 1) of one head, on the lanes of row u.
    const uint32_t pk = cvt_bf16x2(p, dpp<kDppRowRor8>(p));
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      uint32_t w0[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
      uint32_t w1[4] = {vv[u + 1].x, vv[u + 1].y, vv[u + 1].z, vv[u + 1].w};
      if constexpr (kEdge) {  // stale slots may hold NaN
        const bool ok0 = kb + u * KPL + lk >= ks && kb + u * KPL + lk < ke;
        const bool ok1 = kb + (u + 1) * KPL + lk >= ks && kb + (u + 1) * KPL + lk < ke;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w0[i] = ok0 ? w0[i] : 0u;
          w1[i] = ok1 ? w1[i] : 0u;
        }
      }
      uint32_t vp[8];  // vp[e] = (v0[e], v1[e]) as a bf16 pair
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vp[2 * i] = __builtin_amdgcn_perm(w1[i], w0[i], 0x05040100u);
        vp[2 * i + 1] = __builtin_amdgcn_perm(w1[i], w0[i], 0x07060302u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t pp = bcast16u(pk, pair_of(u) + h);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = dot2_bf16(pp, vp[e], o[h][e]);
      }
    }
  };
  auto compute_blk = [&](const uint4 (&kk)[U], const uint4 (&vv)[U], int b, auto edge_c) {
    constexpr bool kEdge = decltype(edge_c)::value;
    const int kb = kb0 + b * KB;
    if constexpr (kScatter) {
      scatter_blk(kk, vv, kb, edge_c);
      return;
    } else {
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = dot2_bf16(qw[h][0], kk[u].x, 0.f);
        acc = dot2_bf16(qw[h][1], kk[u].y, acc);
        acc = dot2_bf16(qw[h][2], kk[u].z, acc);
        acc = dot2_bf16(qw[h][3], kk[u].w, acc);
        s[u][h] = group_sum<LPK>(acc);  // unscaled: the scale is folded into exp2 below
      }
    }
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = kb + u * KPL + lk;
      ok[u] = !kEdge || (j >= ks && j < ke);
      if constexpr (kEdge) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[u][h] = ok[u] ? s[u][h] : -INFINITY;
      }
    }
    // Running max per head, in scaled (log2) units, moved lazily: only when a
    // block's maximum exceeds it by more than 8 (probabilities then stay below
    // 2^8), and then for every head of the wave at once behind a uniform branch.
    float mxs[G];
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][h]);
      mxs[h] = mx * sc;
      grow = grow || mxs[h] > m[h] + 8.f;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], mxs[h]);
        const float alpha = fast_exp2(m[h] - mn);
        m[h] = mn;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
      }
    }
    // Two key rows at a time: their V, interleaved per dimension into bf16
    // pairs, and each head's two probabilities rounded to a bf16 pair give
    // o += p0*v0 + p1*v1 in one v_dot2_f32_bf16 per dimension.  The sum l
    // takes the fp32 probabilities.
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      uint32_t w0[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
      uint32_t w1[4] = {vv[u + 1].x, vv[u + 1].y, vv[u + 1].z, vv[u + 1].w};
      if constexpr (kEdge) {  // stale slots may hold NaN
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w0[i] = ok[u] ? w0[i] : 0u;
          w1[i] = ok[u + 1] ? w1[i] : 0u;
        }
      }
      uint32_t vp[8];  // vp[e] = (v0[e], v1[e]) as a bf16 pair
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vp[2 * i] = __builtin_amdgcn_perm(w1[i], w0[i], 0x05040100u);
        vp[2 * i + 1] = __builtin_amdgcn_perm(w1[i], w0[i], 0x07060302u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p0 = fast_exp2(fmaf(s[u][h], sc, -m[h]));
        const float p1 = fast_exp2(fmaf(s[u + 1][h], sc, -m[h]));
        l[h] += p0 + p1;
        const uint32_t pp = cvt_bf16x2(p0, p1);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = dot2_bf16(pp, vp[e], o[h][e]);
      }
    }
    }
  };
  // A block that crosses the piece's first or last key masks per key; the
  // others (all but at most two per piece) skip the masks.  Uniform branch.
  // With 8 query heads per KV head the second copy of the block code would
  // not fit the registers of two waves per SIMD: every block masks.
  auto compute = [&](const uint4 (&kk)[U], const uint4 (&vv)[U], int b) {
    const int kb = kb0 + b * KB;
    if (G == 8 || kb < ks || kb + KB > ke)
      compute_blk(kk, vv, b, std::true_type{});
    else
      compute_blk(kk, vv, b, std::false_type{});
  };

  // Two register buffers: one block's loads are in flight while the other is
  // computed.  Each trip computes two blocks and has a single exit at the top (a
  // mid-loop exit would give the loop head a path with other loads in flight,
  // and the compiler would then wait for all of them there).  The scheduling
  // barriers keep compute from being hoisted above the loads.
  uint4 ka[U], va[U], kbuf[U], vbuf[U];
  issue(0, ONE_PAGE_PER_ITER ? page_of(0) : 0, ka, va);
  // Let q land before the key loop starts, so every path into the loop has the
  // same loads in flight (otherwise the loop head waits for everything): an
  // empty asm that reads the q registers makes the compiler wait for them here,
  // behind the first block's loads, which stay in flight.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < G; ++h) asm volatile("" ::"v"(qw[h][0]), "v"(qw[h][1]), "v"(qw[h][2]), "v"(qw[h][3]));
  __builtin_amdgcn_sched_barrier(0);
  int pid = ONE_PAGE_PER_ITER ? page_of(1) : 0;
  int b = 0;
  for (; b + 1 < nb; b += 2) {
    issue(b + 1, pid, kbuf, vbuf);
    pid = ONE_PAGE_PER_ITER ? page_of(b + 2) : 0;
    __builtin_amdgcn_sched_barrier(0);
    compute(ka, va, b);
    issue(b + 2, pid, ka, va);  // past the end: a clamped, cached reload, never computed
    pid = ONE_PAGE_PER_ITER ? page_of(b + 3) : 0;
    __builtin_amdgcn_sched_barrier(0);
    compute(kbuf, vbuf, b + 1);
  }
  if (b < nb) compute(ka, va, b);  // odd block count: the last block is in A

  if constexpr (kScatter) {  // each head's sum from its lanes' shares
    float t = lsum;
    if constexpr (G == 4) t += dpp<kDppRowRor4>(t);
    t += dpp<kDppRowRor8>(t);
#pragma unroll
    for (int h = 0; h < G; ++h) l[h] = bcast16(t, h);
  }
  // Combine the KPL lane groups (lanes that differ in bits >= log2(LPK)).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = m[h];
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float sc = fast_exp2(m[h] - M);
    l[h] *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] *= sc;
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
      l[h] += __shfl_xor(l[h], off);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] += __shfl_xor(o[h][e], off);
    }
    m[h] = M;
  }

  if (lk == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = 1.f / l[h];
      const float lse_nat = (m[h] + log2f(l[h])) * kLn2;
      const int qh = hk * G + h;
      if (out_slot < 0) {
        uint4 pk;
        pk.x = pack_bf16x2(o[h][0] * inv, o[h][1] * inv);
        pk.y = pack_bf16x2(o[h][2] * inv, o[h][3] * inv);
        pk.z = pack_bf16x2(o[h][4] * inv, o[h][5] * inv);
        pk.w = pack_bf16x2(o[h][6] * inv, o[h][7] * inv);
        *reinterpret_cast<uint4*>(a.out + ((int64_t)q_index * Hq + qh) * D + ld * 8) = pk;
        if (a.lse != nullptr && ld == 0) a.lse[(int64_t)q_index * Hq + qh] = lse_nat;
      } else {  // split-KV partial, combined by the merge kernel
        float* po = a.part_o + ((int64_t)out_slot * G + h) * D + ld * 8;
        *reinterpret_cast<float4*>(po) = make_float4(o[h][0] * inv, o[h][1] * inv, o[h][2] * inv, o[h][3] * inv);
        *reinterpret_cast<float4*>(po + 4) = make_float4(o[h][4] * inv, o[h][5] * inv, o[h][6] * inv, o[h][7] * inv);
        if (ld == 0) a.part_lse[(int64_t)out_slot * G + h] = lse_nat;
      }
    }
  }
}

// Wave gw of the decode grid: worker gw / Hk, KV head gw % Hk, runs its
// worker's pieces in order.
template <int D, int G, bool ONE_PAGE_PER_ITER>
__device__ __forceinline__ void decode_wave(const DecodeArgs& a, int gw, int lane) {
  const int worker = gw / a.num_kv_heads;
  if (worker >= a.n_workers) return;
  const int hk = gw - worker * a.num_kv_heads;
  const auto wp = as_const4(a.work + worker);
  const int p0 = wp[0], p1 = wp[1];
  for (int p = p0; p < p1; ++p) decode_piece<D, G, ONE_PAGE_PER_ITER>(a, p, hk, lane);
}

}  // namespace dec
}  // namespace pkv
