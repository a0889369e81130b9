// Device code of the prefill kernel, shared by the prefill launch
// (prefill.hip) and the fused mixed-step launch (mixed.hip).
#pragma once

// Causal ragged prefill over a paged KV cache (FlashInferPrefillWrapper.run on
// the mstar attn.wrappers page; the [cached prefix | fresh tokens] sequence of
// attn.dense).  A dense contraction, so both products run on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
// A workgroup (4 waves) owns one tile: a row, a KV head and a block of BT =
// 128/group query tokens, i.e. 128 (query head, token) pairs that all read the
// same K/V.  Wave w takes pairs 32w..32w+31.  Keys are consumed 64 at a time:
// the workgroup gathers the 64 key rows of K and V from their pages into LDS,
// both as rows [key][d], and every wave then computes
//   S^T (64 keys x 32 queries) = K . Q^T       (A = K from LDS, B = Q in registers)
//   P = exp2(S*scale*log2e - m)                (online softmax, fp32, per query column)
//   O^T (D x 32 queries)     += V^T . P^T      (A = V^T, read transposed from LDS
//                                                by ds_read_b64_tr_b16; B = P as bf16)
// With S^T a lane holds one query column, so the row max needs a single
// cross-half exchange and the per-query rescale is a per-lane scalar.
//
// The running max is only moved when some query's new maximum exceeds it by
// more than 2^8 (in exp2 units): P stays <= 256, harmless in fp32 and bf16,
// and the O rescale (64 multiplies per lane) is skipped on most key tiles.
#include <type_traits>

#include "common.cuh"
#include "kernels.h"

namespace pkv {
namespace pre {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kRescaleSlack = 8.f;  // log2 units: P may reach 2^8 before O is rescaled
#ifndef PKV_PREFILL_AHEAD
#define PKV_PREFILL_AHEAD 3
#endif
#ifndef PKV_PREFILL_VALU_QK
#define PKV_PREFILL_VALU_QK 7
#endif
#ifndef PKV_PREFILL_VALU_PV
#define PKV_PREFILL_VALU_PV 2
#endif
constexpr int kAhead = PKV_PREFILL_AHEAD;      // LDS fragments in flight ahead of the MFMAs
constexpr int kValuQK = PKV_PREFILL_VALU_QK;   // VALU slots per MFMA while S is formed
constexpr int kValuPV = PKV_PREFILL_VALU_PV;   // VALU slots per MFMA while O is updated

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: in each group of 16 lanes, lane L receives element L%4 of
// the 4-element (8-byte) rows addressed by lanes L/4, L/4+4, L/4+8, L/4+12, in
// that order.  With lane a of the group pointing at row (key0 + a/4) and column
// (d0 + 4*(a%4)) of a [key][d] tile, lane 4m+j receives column d0 + 4m + j at
// keys key0 .. key0+3: a column of V, four keys long.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  // p points into __shared__ memory; the C-style cast converts it to an LDS address.
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(u32x2_t, v);
}

// WAVE_PAGE: page_size >= 16, so the 16 keys a wave stages per tile lie in one
// page -- its id is a scalar load and the loads use a scalar base.
// DENSE (with WAVE_PAGE): the keys are contiguous rows of k_dense / v_dense
// starting at the tile's page_base; the row acts as one page.
// Tile `tile` of the prefill tile list, by a workgroup of 256 threads.
template <int D, bool WAVE_PAGE, bool DENSE>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int tile) {
  constexpr int BN = 64;              // keys per tile
  constexpr int KSTEPS = D / 16;      // MFMA steps over head_dim for S
  constexpr int DBLK = D / 32;        // 32-row output blocks over head_dim
  constexpr int SEGS = D / 8;         // 16-byte segments of a key row
  constexpr int KPT = BN * SEGS / 256;  // key rows each thread stages per tile
  // LDS row strides (elements), chosen free of bank conflicts (64 banks of 4
  // bytes): the 16 lanes of a K row read start 4 (D=128) or 36 (D=64) banks
  // apart; a transposed V read serves 32 lanes at once, 4 rows x 2 column
  // groups of 8 banks, with rows 16 (D=128) or 48 (D=64) banks apart, so the
  // 32 lanes touch each bank once.
  constexpr int KS = D + 8;
  constexpr int VS = D + 32;
  constexpr int KBUF = BN * KS, VBUF = BN * VS;
  // Two LDS buffers: tile t lives in buffer t % 2.
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2 * VBUF];

  if (a.counts != nullptr && (int64_t)tile >= as_const4(a.counts)[2]) return;
  const pkv_prefill_tile* tp = a.tiles + tile;
  const int hk = tp->kv_head;
  const int q_start = tp->q_start;
  const int q_count = tp->q_count;
  const int kv_lo = tp->kv_lo;
  const int kv_hi = tp->kv_hi;
  const int page_base = tp->page_base;
  const int q_base = tp->q_base;
  const int kv_len = tp->kv_len;
  const int q_len = tp->q_len;

  const int Hq = a.num_qo_heads;
  const int g = a.group;
  const int BT = 128 / g;
  const int ps = a.page_size;
  const int ps_log2 = __builtin_ctz(ps);
  const int row_elems = a.num_kv_heads * D;
  const int64_t page_elems = 2LL * ps * row_elems;
  const int v_off = ps * row_elems;
  const bool causal = a.causal != 0;
  const int wl = a.window_left;
  const float c = a.scale_log2;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int jcol = lane & 31;
  const int half = lane >> 5;
  const int mrow = wave * 32 + jcol;
  const int hl = mrow / BT;
  const int tl = mrow - hl * BT;
  const int qh = hk * g + hl;
  const bool qvalid = tl < q_count;
  const int token = q_base + q_start + tl;
  const int pos = kv_len - q_len + q_start + tl;  // sequence position of this query
  const int hi_j = causal ? (pos < kv_len - 1 ? pos : kv_len - 1) : kv_len - 1;
  const int lo_j = wl >= 0 ? pos - wl : 0;

  // Q^T operand: k-step s uses d = 16 s + 8 half .. +7 of this lane's query.
  u32x4_t qreg[KSTEPS];
  {
    const uint16_t* qp = a.q + ((int64_t)token * Hq + qh) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (qvalid) qreg[s] = *reinterpret_cast<const u32x4_t*>(qp + 16 * s);
      else qreg[s] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  f32x16_t oacc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) oacc[b] = f32x16_t{};
  float m_run = -1e30f, l_run = 0.f;  // m_run in exp2 units (scaled)

  // Block-wide query position bounds, for deciding which key tiles need masks.
  const int p_first = kv_len - q_len + q_start;
  const int p_last = p_first + q_count - 1;

  // Staging map: thread -> (segment, key group of KPT keys).  The 16 keys of a
  // wave are [16*wave, 16*wave + 16) of the tile.
  const int seg = threadIdx.x % SEGS;
  const int kg = threadIdx.x / SEGS;
  const int kstart = kv_lo & ~(BN - 1);
  const int kend = kv_hi + 1;
  const int ntiles = (kend - kstart + BN - 1) / BN;
  const_as4_ptr<int32_t> cidx = as_const4(a.indices);
  const uint32_t row_bytes = (uint32_t)row_elems * 2u;
  const int64_t head_bytes = (int64_t)hk * D * 2;

  // Key i of this thread in tile t (clamped to the last tile and the last key,
  // so addresses stay inside the row; keys past the row are masked later).
  auto key_of = [&](int t, int i) {
    t = t < ntiles ? t : ntiles - 1;
    const int key = kstart + t * BN + kg * KPT + i;
    return key < kv_len ? key : kv_len - 1;
  };
  // WAVE_PAGE: the wave's 16 keys k0 .. k0+15 (k0 a multiple of 16) lie in
  // one page; the first is clamped to the row's last key to choose the page.
  auto wave_key0 = [&](int t) {
    t = t < ntiles ? t : ntiles - 1;
    return kstart + t * BN + 16 * wave;
  };
  auto load_pids = [&](int t, int (&pid)[KPT]) {
    if constexpr (DENSE) {
      pid[0] = 0;  // no page table
    } else if constexpr (WAVE_PAGE) {
      const int k0 = wave_key0(t);
      const int k0c = k0 < kv_len ? k0 : kv_len - 1;
      pid[0] = cidx[page_base + (k0c >> ps_log2)];  // uniform: scalar load
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) pid[i] = cidx[page_base + (key_of(t, i) >> ps_log2)];
    }
  };
  // WAVE_PAGE byte offsets inside a page: key k0 + tk + i sits at slot
  // (k0 - page start) + tk + i, clamped to the slot of the row's last key; the
  // per-thread part is fixed, the rest is uniform.
  const int tk = kg * KPT - 16 * wave;  // this thread's first key within the wave's 16
  uint32_t toff[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) toff[i] = (uint32_t)(tk + i) * row_bytes + seg * 16u;
  u32x4_t gk[KPT], gv[KPT];
  // Global loads of tile t into registers: K (kv = 0) into gk, V (kv = 1) into gv.
  auto gload = [&](int t, const int (&pid)[KPT], int kv, u32x4_t (&dst)[KPT]) {
    if constexpr (DENSE) {
      // key k0 + tk + i of the row at byte (k0 + tk + i) * row_bytes, clamped to
      // the row's last key
      const char* base_p = reinterpret_cast<const char*>(kv ? a.v_dense : a.k_dense) +
                           (int64_t)page_base * row_bytes + head_bytes;
      const int k0 = wave_key0(t);
      const uint32_t base = (uint32_t)k0 * row_bytes;
      const uint32_t lim = (uint32_t)(kv_len - 1) * row_bytes + seg * 16u;
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        dst[i] = *reinterpret_cast<const u32x4_t*>(base_p + min(base + toff[i], lim));
    } else if constexpr (WAVE_PAGE) {
      const char* base_p = reinterpret_cast<const char*>(a.cache) +
                           (int64_t)pid[0] * page_elems * 2 + head_bytes +
                           (kv ? (int64_t)v_off * 2 : 0);
      const int k0 = wave_key0(t);
      const int pstart = (k0 < kv_len ? k0 : kv_len - 1) & ~(ps - 1);
      const uint32_t base = (uint32_t)(k0 - pstart) * row_bytes;
      const uint32_t lim = (uint32_t)(kv_len - 1 - pstart) * row_bytes + seg * 16u;
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        dst[i] = *reinterpret_cast<const u32x4_t*>(base_p + min(base + toff[i], lim));
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int key = key_of(t, i);
        const uint16_t* p = a.cache + (int64_t)pid[i] * page_elems +
                            (key & (ps - 1)) * row_elems + hk * D + seg * 8 + (kv ? v_off : 0);
        dst[i] = *reinterpret_cast<const u32x4_t*>(p);
      }
    }
  };
  auto swrite_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      *reinterpret_cast<u32x4_t*>(&sK[buf * KBUF + (kg * KPT + i) * KS + seg * 8]) = gk[i];
  };
  auto swrite_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      *reinterpret_cast<u32x4_t*>(&sV[buf * VBUF + (kg * KPT + i) * VS + seg * 8]) = gv[i];
  };

  // S^T (64 keys x 32 queries) of the tile in buffer buf.
  // sacc[kb2][r] is key 32 kb2 + 8 (r/4) + 4 half + r%4 of the tile, query jcol.
  auto qk = [&](int buf, f32x16_t (&sacc)[2]) {
    const uint16_t* kp = sK + buf * KBUF + jcol * KS + 8 * half;
    sacc[0] = f32x16_t{};
    sacc[1] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kp + kb2 * 32 * KS + 16 * s);
        sacc[kb2] = mfma32(kf, qreg[s], sacc[kb2]);
      }
    }
  };
  // Does the tile at kbase cross the causal diagonal, the window edge or the
  // row end?  (uniform)
  auto needs_mask = [&](int kbase) {
    return (kbase + BN - 1 > (causal ? p_first : kv_len - 1)) || (kbase + BN > kv_len) ||
           (wl >= 0 && kbase < p_last - wl);
  };
  // Scores of keys outside [lo_j, hi_j] become -inf.
  auto apply_mask = [&](f32x16_t (&sacc)[2], int kbase) {
    const int k0 = kbase + 4 * half;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * kb2 + 8 * (r >> 2) + (r & 3);
        sacc[kb2][r] = (key > hi_j || key < lo_j) ? -INFINITY : sacc[kb2][r];
      }
  };
  // Max of the raw scores of this lane's query column (both halves).
  auto colmax = [&](const f32x16_t (&sacc)[2]) {
    // Three-input maxima (v_max3_f32): 32 values in 16 instructions.
    float m3[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x16_t& v = sacc[k >> 2];
      const int r = 4 * (k & 3);
      m3[k] = fmaxf(fmaxf(v[r], v[r + 1]), fmaxf(v[r + 2], v[r + 3]));
    }
    const float a = fmaxf(fmaxf(m3[0], m3[1]), m3[2]);
    const float b = fmaxf(fmaxf(m3[3], m3[4]), m3[5]);
    const float mr = fmaxf(fmaxf(m3[6], m3[7]), fmaxf(a, b));
    return fmaxf(mr, __shfl_xor(mr, 32));
  };
  // Move the running max (and rescale O, l) only when some query's new maximum
  // exceeds it by more than the slack (uniform branch).
  auto update_max = [&](float mr) {
    const float mt = mr * c;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DBLK; ++b) oacc[b] *= alpha;
    }
  };
  // P = exp2(S*c - m) as the bf16 P^T operand; step s = 2 kb2 + t holds keys
  // 16 s + {0..3, 8..11} + 4 half.
  auto expsum = [&](const f32x16_t (&sacc)[2], u32x4_t (&pb)[4]) {
    const float neg_m = -m_run;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(sacc[kb2][8 * t + e], c, neg_m));
          l_run += p[e];  // fp32 P: a sum of the bf16-rounded P misses the LSE bound
        }
        pb[2 * kb2 + t] = u32x4_t{cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]),
                                  cvt_pk_bf16(p[4], p[5]), cvt_pk_bf16(p[6], p[7])};
      }
    }
  };
  // O^T += V^T . P^T for the tile in buffer buf; the transposed reads deliver
  // column 32 b + jcol at the keys of pb[s].
  const int grp = lane >> 4, ga = lane & 15;
  const int v_lane = (4 * (grp >> 1) + (ga >> 2)) * VS + 16 * (grp & 1) + 4 * (ga & 3);
  auto pv = [&](int buf, const u32x4_t (&pb)[4]) {
    const uint16_t* vb = sV + buf * VBUF + v_lane;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int b = 0; b < DBLK; ++b) {
        const uint16_t* vp = vb + 16 * s * VS + 32 * b;
        const u32x2_t v0 = lds_read_tr16(vp);
        const u32x2_t v1 = lds_read_tr16(vp + 8 * VS);
        oacc[b] = mfma32(u32x4_t{v0[0], v0[1], v1[0], v1[1]}, pb[s], oacc[b]);
      }
    }
  };

  // ---- pipeline ----
  // K runs two tiles ahead of the softmax and V one: at step i the registers
  // hold K(i+2) and V(i+1), which go to the K buffer of tile i (last read by
  // the scores of tile i in step i-1) and the V buffer of tile i-1 (last read
  // by step i-1's O update).  So one barrier per step separates every LDS
  // write from the reads before and after it.
  int pid_k[KPT], pid_v[KPT];
  {
    int pid0[KPT];
    load_pids(0, pid0);
    load_pids(1, pid_k);
    gload(0, pid0, 0, gk);
    gload(0, pid0, 1, gv);
  }
  swrite_k(0);
  swrite_v(0);
  gload(1, pid_k, 0, gk);
  load_pids(2, pid_k);
  load_pids(1, pid_v);
  swrite_k(1);
  gload(2, pid_k, 0, gk);
  gload(1, pid_v, 1, gv);
  load_pids(3, pid_k);
  load_pids(2, pid_v);
  __syncthreads();
  f32x16_t sa[2], sb[2];
  qk(0, sa);
  if (needs_mask(kstart)) apply_mask(sa, kstart);
  update_max(colmax(sa));
  __syncthreads();  // step 0 overwrites the K buffer just read

  // One step: softmax and O update for tile i (scores in cur), scores of tile
  // i+1 into nxt.  Past the last tile the clamped loads repeat it; those
  // scores are never used.
  auto step = [&](f32x16_t (&cur)[2], f32x16_t (&nxt)[2], int i) {
    const int buf = i & 1;
    u32x4_t pb[4];
    // S of the next tile on the matrix cores while the VALU turns the current
    // scores into P.
    qk(buf ^ 1, nxt);
    expsum(cur, pb);
    // LDS reads run kAhead fragments ahead of the MFMA that consumes them.
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int k = 0; k < 2 * KSTEPS; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (k + kAhead < 2 * KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x002, kValuQK, 0);  // VALU
    }
    // Pin P here: without a use the compiler would sink its computation past
    // the masking branch below, out of reach of the matrix-core work above.
#pragma unroll
    for (int k = 0; k < 4; ++k) asm volatile("" ::"v"(pb[k]));
    // Stage K(i+2) and V(i+1); issue the loads of K(i+3) and V(i+2).
    swrite_k(buf);
    swrite_v(buf ^ 1);
    gload(i + 3, pid_k, 0, gk);
    gload(i + 2, pid_v, 1, gv);
    load_pids(i + 4, pid_k);
    load_pids(i + 3, pid_v);
    const int knext = kstart + (i + 1) * BN;
    if (needs_mask(knext)) apply_mask(nxt, knext);
    // O += P V for the current tile on the matrix cores while the VALU finds
    // the next tile's column maxima.
    pv(buf, pb);
    const float mr = colmax(nxt);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 1);
#pragma unroll
    for (int k = 0; k < 4 * DBLK; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      if (k + kAhead < 4 * DBLK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // two DS reads
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPV, 1);  // VALU
    }
    update_max(mr);
    __syncthreads();
  };

  int i = 0;
  for (; i + 1 < ntiles; i += 2) {
    step(sa, sb, i);
    step(sb, sa, i + 1);
  }
  if (i < ntiles) step(sa, sb, i);

  // ---- normalise and store ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qvalid) {
    const float inv = 1.f / l_tot;
    uint16_t* op = a.out + ((int64_t)token * Hq + qh) * D;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * b + 8 * rq + 4 * half;
        u32x2_t w2 = {cvt_pk_bf16(oacc[b][4 * rq + 0] * inv, oacc[b][4 * rq + 1] * inv),
                      cvt_pk_bf16(oacc[b][4 * rq + 2] * inv, oacc[b][4 * rq + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(op + d0) = w2;
      }
    }
    if (a.lse != nullptr && half == 0)
      a.lse[(int64_t)token * Hq + qh] = (m_run + log2f(l_tot)) * kLn2;
  }
}

}  // namespace pre
}  // namespace pkv
