// Device code of the prefill kernel, shared by the prefill launch
// (prefill.hip) and the fused mixed-step launch (mixed.hip).
#pragma once

// Causal ragged prefill over a paged KV cache (FlashInferPrefillWrapper.run on
// the mstar attn.wrappers page; the [cached prefix | fresh tokens] sequence of
// attn.dense).  A dense contraction, so both products run on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with fp32 accumulation.
//
// A workgroup (4 waves) owns one tile: a row, a KV head and a block of
// BT = 64*NQB/group query tokens, i.e. 64*NQB (query head, token) pairs that
// all read the same K/V.  Wave w takes NQB blocks of 16 pairs.  Keys are
// consumed 32 at a time: the workgroup gathers the 32 key rows of K and V from
// their pages into LDS, both as rows [key][d], and every wave computes, per
// query block,
//   S^T (32 keys x 16 queries) = K . Q^T       (A = K from LDS, B = Q in registers)
//   P = exp2(S*scale*log2e - m)                (online softmax, fp32, per query column)
//   O^T (D x 16 queries)     += V^T . P^T      (A = V^T, read transposed from LDS
//                                                by ds_read_b64_tr_b16; B = P as bf16)
// Each K or V fragment read from LDS feeds NQB matrix instructions, so the LDS
// read traffic per FLOP falls as 1/NQB.  NQB = 3 (48 queries per wave) fits at
// two waves per SIMD because K and V are copied from memory straight into LDS
// (global_load_lds_dwordx4), NBUF-1 steps ahead into a ring of NBUF buffers,
// with no registers held for the copies in flight.
//
// In the 16x16x32 layouts a lane holds one query column (lane % 16) and four
// keys 4*(lane/16) .. +3 of every 16-key block; the column max and sum need two
// cross-row exchanges (v_permlane16_swap, v_permlane32_swap).
//
// The running max is only moved when some query's new maximum exceeds it by
// more than 2^8 (in exp2 units): P stays <= 256, harmless in fp32 and bf16,
// and the O rescale is skipped on most key tiles.
#include <type_traits>

#include "common.cuh"
#include "kernels.h"

namespace pkv {
namespace pre {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTilePairs = kPrefillTilePairs;  // (query head, token) pairs per tile
constexpr int kNqb = kTilePairs / 64;          // 16-pair query blocks per wave
static_assert(kTilePairs % 64 == 0, "tile pairs must be a multiple of 64");

constexpr float kRescaleSlack = 8.f;  // log2 units: P may reach 2^8 before O is rescaled
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float max3f(float x, float y, float z) { return fmaxf(fmaxf(x, y), z); }

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

// x combined with the same register of lane ^ 16 (v_permlane16_swap: odd and
// even rows of 16 lanes trade places) or of lane ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float max_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

#ifndef PKV_PREFILL_KA
#define PKV_PREFILL_KA 2
#endif
#ifndef PKV_PREFILL_NBUF
#define PKV_PREFILL_NBUF 4
#endif

// One 16-byte-per-lane copy from memory straight into LDS: lane l's 16 bytes
// at sbase + voff go to LDS byte m0 + 16 l (global_load_lds_dwordx4; the LDS
// base is bound to m0 as an operand, so the compiler sets m0 and knows it).
// The compiler does not see these copies as memory accesses; their completion
// is awaited with wait_copies (vmcnt counts them with the wave's other vector
// memory reads, which return in issue order).
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma16_flat(const void* p, uint32_t m0) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(p), "{m0}"(m0) : "memory");
}
// Wait until at most N of this wave's vector memory reads are outstanding.
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

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

// WAVE_PAGE: page_size >= 16, so the 8 keys a wave stages per step lie in one
// page -- its id is a scalar load and the loads use a scalar base.
// DENSE (with WAVE_PAGE): the keys are contiguous rows of k_dense / v_dense
// starting at the tile's page_base; the row acts as one page.
// Tile `tile` of the prefill tile list, by a workgroup of 256 threads.
// PRIO: raise the wave's priority for the softmax and the copy issue (the
// prefill launch, where both waves of a SIMD run prefill tiles); off in the
// fused mixed-step launch, where it would hold back the decode waves.
template <int D, bool WAVE_PAGE, bool DENSE, bool PRIO = true>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int tile) {
  constexpr int NQB = kNqb;
  constexpr int BN = 32;              // keys per step
  constexpr int KSTEPS = D / 32;      // MFMA steps over head_dim for S
  constexpr int DBLK = D / 16;        // 16-row output blocks over head_dim
  constexpr int SEGS = D / 8;         // 16-byte segments of a key row
  constexpr int KW = BN / 4;          // keys each wave copies per step
  constexpr int NI = KW * D * 2 / 1024; // 1 KB copies per wave per step, per tensor
  constexpr int RPI = 1024 / (2 * D); // key rows per 1 KB copy
  constexpr int ROWB = 2 * D;         // LDS row bytes (no padding)
  constexpr int BUFB = BN * ROWB;     // bytes of one step's K (or V)
  constexpr int NBUF = PKV_PREFILL_NBUF;
  constexpr int PF = NBUF - 1;        // steps a copy runs ahead of its first read
  static_assert(NBUF >= 3, "the scores of step i+1 are read in step i");
  // K and V reach LDS straight from memory (global_load_lds_dwordx4: a wave's
  // copy fills 1 KB of LDS, 16 bytes per lane in lane order), so rows cannot
  // be padded; instead the 16-byte segments of a row are XOR-swizzled.
  //  K, row r: segment c at c ^ kswz(r).  The 16 lanes reading one column of a
  //    16-key block (rows r0 .. r0+15) then touch 16 different segments.
  //  V, row r: segment c at c ^ vswz(r).  A transposed read serves 32 lanes,
  //    8 rows x 2 segments; the swizzle moves the 8 rows' segment pairs apart.
  // (D=64 rows are half the 64 banks, so row pairs share the swizzle.)
  auto kswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };
  // NBUF LDS buffers: step t lives in buffer t % NBUF.
  __shared__ __attribute__((aligned(1024))) uint8_t sK[NBUF * BUFB];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[NBUF * BUFB];

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
  const int BT = kTilePairs / g;
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
  const int li = lane & 15;   // query column inside a block; key row of a K fragment
  const int lg = lane >> 4;   // row group: keys 4 lg .. 4 lg + 3 of each 16-key block

  // Query blocks of this wave: pair m = 16 (NQB wave + b) + li is query head
  // hk*g + m / BT at token m % BT of the tile.
  auto pair_of = [&](int b, int& qh, int& tl) {
    const int m = 16 * (NQB * wave + b) + li;
    const int hl = m / BT;
    tl = m - hl * BT;
    qh = hk * g + hl;
  };
  // Sequence position of query block b of this lane; keys [pos - wl, pos]
  // (causal) are visible.  Recomputed where needed (masked steps only).
  auto pos_of = [&](int b) {
    int qh, tl;
    pair_of(b, qh, tl);
    return kv_len - q_len + q_start + tl;
  };

  // Q^T operand: k-step s uses d = 32 s + 8 lg .. +7 of this lane's query.
  u32x4_t qreg[NQB][KSTEPS];
#pragma unroll
  for (int b = 0; b < NQB; ++b) {
    int qh, tl;
    pair_of(b, qh, tl);
    const uint16_t* qp = a.q + ((int64_t)(q_base + q_start + tl) * Hq + qh) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (tl < q_count) qreg[b][s] = *reinterpret_cast<const u32x4_t*>(qp + 32 * s);
      else qreg[b][s] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  f32x4_t oacc[NQB][DBLK];
#pragma unroll
  for (int b = 0; b < NQB; ++b)
#pragma unroll
    for (int d = 0; d < DBLK; ++d) oacc[b][d] = f32x4_t{};
  // Running max per query in exp2 units, kept negated (nm = -m, the exponent's
  // offset), and the raw-score threshold above which it must move:
  // th = (m + slack) / c.
  const float inv_c = 1.f / a.scale_log2;
  float nm[NQB], th[NQB], l_run[NQB];
#pragma unroll
  for (int b = 0; b < NQB; ++b) {
    nm[b] = 1e30f;
    th[b] = -1e30f;
    l_run[b] = 0.f;
  }

  // Block-wide query position bounds, for deciding which key tiles need masks.
  const int p_first = kv_len - q_len + q_start;
  const int p_last = p_first + q_count - 1;

  const int kstart = kv_lo & ~(BN - 1);
  const int kend = kv_hi + 1;
  const int ntiles = (kend - kstart + BN - 1) / BN;
  const_as4_ptr<int32_t> cidx = as_const4(a.indices);
  const uint32_t row_bytes = (uint32_t)row_elems * 2u;
  const uint32_t head_bytes = (uint32_t)hk * D * 2u;
  const uint32_t page_bytes = (uint32_t)(page_elems * 2);  // < 4 GiB: ps <= 256
  const uint64_t v_bytes = (uint64_t)v_off * 2u;
  const uint32_t lane_row_bytes = (uint32_t)(lane / SEGS) * row_bytes;  // lane's row in a copy

  // Copy map: copy j of wave w fills rows KW*w + RPI*j + lane/SEGS of the step,
  // physical segment lane % SEGS, with the source segment that the swizzle
  // puts there; copy_src gives the lane's byte offset inside a key row.  (On
  // the steps whose keys all lie in the row the lanes' offsets do not change,
  // so they stay in registers; the row-end steps clamp them.)
  auto copy_src = [&](int j, bool v, int& rwj) -> uint32_t {
    rwj = RPI * j + lane / SEGS;
    const int r = KW * wave + rwj;
    return head_bytes + 16u * (uint32_t)((lane % SEGS) ^ (v ? vswz(r) : kswz(r)));
  };
  const uint32_t lds_k = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(sK);
  const uint32_t lds_v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(sV);

  // Issue the copies of step t (clamped to the last step, and each key to the
  // row's last key, so addresses stay inside the row; keys past the row are
  // masked later) into the buffer at byte offset boff (t % NBUF times BUFB) of
  // the K and V rings.  Every call issues exactly 2*NI copies per wave: the
  // waits below count on it.
  auto issue = [&](int t, uint32_t boff) {
    const uint32_t mk = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(lds_k + boff + KW * wave * ROWB));
    const uint32_t mv = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(lds_v + boff + KW * wave * ROWB));
    if constexpr (DENSE || WAVE_PAGE) {
      // The wave's KW keys lie in one page (or one dense row): a uniform base.
      const int kw0 = kstart + t * BN + KW * wave;
      if (kw0 + KW <= kv_len) {
        // All KW keys are in the row (every step but the row's last): no
        // clamping, and the key's offset inside the page goes into the base.
        // (A step past the tile's last reads keys of the row that no score
        // uses.)
        const char* kbase;
        if constexpr (DENSE) {
          kbase = reinterpret_cast<const char*>(a.k_dense) +
                  (uint64_t)(uint32_t)(page_base + kw0) * row_bytes;
        } else {
          const uint32_t ib = ((uint32_t)page_base + ((uint32_t)kw0 >> ps_log2)) << 2;
          const uint32_t pid = *reinterpret_cast<const_as4_ptr<uint32_t>>(
              reinterpret_cast<const_as4_ptr<char>>(cidx) + ib);  // scalar load
          kbase = reinterpret_cast<const char*>(a.cache) + (uint64_t)pid * page_bytes +
                  (uint32_t)(kw0 & (ps - 1)) * row_bytes;
        }
        const char* vbase = DENSE ? reinterpret_cast<const char*>(a.v_dense) +
                                        (uint64_t)(uint32_t)(page_base + kw0) * row_bytes
                                  : kbase + v_bytes;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          int rwj;
          const uint32_t src = copy_src(j, false, rwj);
          dma16(lane_row_bytes + (uint32_t)(RPI * j) * row_bytes + src, kbase, mk + 1024u * j);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          int rwj;
          const uint32_t src = copy_src(j, true, rwj);
          dma16(lane_row_bytes + (uint32_t)(RPI * j) * row_bytes + src, vbase, mv + 1024u * j);
        }
        return;
      }
      t = t < ntiles ? t : ntiles - 1;
      const int k0 = kstart + t * BN + KW * wave;        // multiple of KW
      const int kb0 = k0 < kv_len ? k0 : kv_len - 1;    // first key actually read
      const int room = kv_len - 1 - kb0;                // keys after kb0 in the row
      const char* kbase;
      if constexpr (DENSE) {
        kbase = reinterpret_cast<const char*>(a.k_dense) + ((int64_t)page_base + kb0) * row_bytes;
      } else {
        const int pid = cidx[page_base + (kb0 >> ps_log2)];  // uniform: scalar load
        kbase = reinterpret_cast<const char*>(a.cache) + (int64_t)pid * page_elems * 2 +
                (int64_t)(kb0 & (ps - 1)) * row_bytes;
      }
      const char* vbase = DENSE ? reinterpret_cast<const char*>(a.v_dense) +
                                      ((int64_t)page_base + kb0) * row_bytes
                                : kbase + (int64_t)v_off * 2;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        int rwj;
        const uint32_t src = copy_src(j, false, rwj);
        dma16((uint32_t)min(rwj, room) * row_bytes + src, kbase, mk + 1024u * j);
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        int rwj;
        const uint32_t src = copy_src(j, true, rwj);
        dma16((uint32_t)min(rwj, room) * row_bytes + src, vbase, mv + 1024u * j);
      }
    } else {
      // Pages shorter than the wave's keys: a page id per lane.
      t = t < ntiles ? t : ntiles - 1;
      const int k0 = kstart + t * BN + KW * wave;        // multiple of KW
      const int kb0 = k0 < kv_len ? k0 : kv_len - 1;    // first key actually read
      const int room = kv_len - 1 - kb0;                // keys after kb0 in the row
#pragma unroll
      for (int kv = 0; kv < 2; ++kv)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          int rwj;
          const uint32_t src = copy_src(j, kv != 0, rwj);
          const int key = kb0 + min(rwj, room);
          const int pid = cidx[page_base + (key >> ps_log2)];
          const char* p = reinterpret_cast<const char*>(a.cache) + (int64_t)pid * page_elems * 2 +
                          (int64_t)(key & (ps - 1)) * row_bytes + (kv ? (int64_t)v_off * 2 : 0);
          dma16_flat(p + src, (kv ? mv : mk) + 1024u * j);
        }
    }
  };

  // S^T (32 keys x 16 queries per block) of the step in buffer buf.
  // sacc[b][kb][r] is key 16 kb + 4 lg + r of the step, query li of block b.
  auto qk = [&](int buf, f32x4_t (&sacc)[NQB][2]) {
    const uint8_t* kp = sK + buf * BUFB + li * ROWB;
#pragma unroll
    for (int b = 0; b < NQB; ++b) {
      sacc[b][0] = f32x4_t{};
      sacc[b][1] = f32x4_t{};
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        // logical segment 4 s + lg of row 16 kb + li (kswz(16 kb + li) = kswz(li))
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(
            kp + kb * 16 * ROWB + 16 * ((4 * s + lg) ^ kswz(li)));
#pragma unroll
        for (int b = 0; b < NQB; ++b) sacc[b][kb] = mfma16(kf, qreg[b][s], sacc[b][kb]);
      }
    }
  };
  // Does step t cross the causal diagonal, the row end (both from step t_a
  // on) or the window edge (steps before t_b)?  A step at key kbase needs
  // masks when kbase + BN - 1 passes the first query's last visible key or
  // kbase + BN passes the row end, or kbase is below the last query's window.
  // (uniform; kstart <= the first visible key, so mask_x >= -BN)
  const int mask_x = min((causal ? p_first : kv_len - 1) - kstart - (BN - 1), kv_len - kstart - BN);
  const int t_a = (mask_x + BN) / BN;
  const int mask_y = wl >= 0 ? p_last - wl - kstart : 0;
  const int t_b = mask_y > 0 ? (mask_y + BN - 1) / BN : 0;
  // Steps in [t_b, t_a) need no mask: one unsigned compare per step.
  const uint32_t t_span = t_a > t_b ? (uint32_t)(t_a - t_b) : 0u;
  auto needs_mask = [&](int t) { return (uint32_t)(t - t_b) >= t_span; };
  // Scores of keys outside [lo_j, hi_j] become -inf.
  auto apply_mask = [&](f32x4_t (&sacc)[NQB][2], int kbase) {
    const int k0 = kbase + 4 * lg;
#pragma unroll
    for (int b = 0; b < NQB; ++b) {
      const int pos = pos_of(b);
      const int hi_j = causal ? min(pos, kv_len - 1) : kv_len - 1;
      const int lo_j = wl >= 0 ? pos - wl : 0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 16 * kb + r;
          sacc[b][kb][r] = (key > hi_j || key < lo_j) ? -INFINITY : sacc[b][kb][r];
        }
    }
  };
  // Max of the raw scores of each query block held by this lane (its 8 keys
  // of the step; the other three row groups hold the rest of the column).
  auto lanemax = [&](const f32x4_t (&sacc)[NQB][2], float (&lm)[NQB]) {
#pragma unroll
    for (int b = 0; b < NQB; ++b) {
      lm[b] = max3f(max3f(sacc[b][0][0], sacc[b][0][1], sacc[b][0][2]),
                    max3f(sacc[b][0][3], sacc[b][1][0], sacc[b][1][1]),
                    fmaxf(sacc[b][1][2], sacc[b][1][3]));
    }
  };
  // Move the running maxima (and rescale O, l) only when some raw score
  // exceeds its query's threshold, i.e. the running max by more than the
  // slack after scaling.  Each lane tests its own scores, so the column
  // maxima across the four row groups (two exchanges per block) are formed
  // only on that rare branch (uniform over the wave); there every query's max
  // moves to its column max, which is always exact.
  auto update_max = [&](const float (&lm)[NQB]) {
    bool need = false;
#pragma unroll
    for (int b = 0; b < NQB; ++b) need |= lm[b] > th[b];
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int b = 0; b < NQB; ++b) {
        const float mr = max_x32(max_x16(lm[b]));
        const float mn = fmaxf(-nm[b], mr * c);
        const float alpha = fast_exp2(-nm[b] - mn);
        nm[b] = -mn;
        th[b] = (mn + kRescaleSlack) * inv_c;
        l_run[b] *= alpha;
#pragma unroll
        for (int d = 0; d < DBLK; ++d) oacc[b][d] *= alpha;
      }
    }
  };
  // Lane (li, lg) points at row 4 lg + li/4 (and 16 more), columns
  // 16 db + 4 (li % 4) .. +3: logical segment 2 db + (li % 4) / 2, half li % 2.
  const int v_row = 4 * lg + (li >> 2);
  const int v_z = vswz(v_row);  // equal for v_row + 16
  const int v_h = ((li & 3) >> 1) * 16 + (li & 1) * 8;
  // Per-lane byte offsets inside a buffer of the K fragments (by k-step) and
  // the V fragments (by 16-row block of head_dim), row base included: a step
  // adds only its buffer's offset.
  uint32_t k_ofs[KSTEPS], v_ofs[DBLK];
#pragma unroll
  for (int st = 0; st < KSTEPS; ++st)
    k_ofs[st] = (uint32_t)(li * ROWB + 16 * ((4 * st + lg) ^ kswz(li)));
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
    v_ofs[db] = (uint32_t)(v_row * ROWB + v_h + 16 * ((2 * db) ^ v_z));
  // ---- pipeline ----
  // Step t's K and V are copied PF steps ahead, into buffer t % NBUF.  Step i
  // reads K(i+1) and V(i) and issues the copies of step i+PF, into the buffer
  // of step i-1, whose last reads (K in step i-2, V in step i-1) precede the
  // barrier that ends step i-1.  Before that barrier every wave waits for its
  // copies of step i+1 (copies land in issue order), leaving PF-2 steps of
  // copies in flight.
  constexpr int NL = 2 * NI;  // copies per wave per step
#pragma unroll
  for (int t = 0; t < PF; ++t) issue(t, t * BUFB);
  wait_copies<(PF - 1) * NL>();
  __syncthreads();
  f32x4_t sa[NQB][2], sb[NQB][2];
  {
    qk(0, sa);
    if (needs_mask(0)) apply_mask(sa, kstart);
    float lm[NQB];
    lanemax(sa, lm);
    update_max(lm);
  }
  wait_copies<(PF - 2) * NL>();
  __syncthreads();

  // One step: softmax and O update for step i (scores in cur), scores of step
  // i+1 into nxt.  Past the last step the clamped copies repeat it; those
  // scores are never used.  The instruction order is written out: LDS
  // fragments are read KA groups ahead of the MFMAs that use them, and
  // scheduling fences keep that order for the score MFMAs (the output
  // update, with the lane maxima between its MFMAs, is left to the compiler's
  // scheduler: about 1 % faster than fenced).
  constexpr int NG = 2 * KSTEPS;         // K fragments per step (16 keys x 32 d)
  constexpr int NEA = 8 * NQB;           // exponentials per lane per step
  constexpr int KA = PKV_PREFILL_KA;     // fragment groups read ahead
  // bo = (i % NBUF) * BUFB, carried from step to step; NBUF is a power of
  // two, so the ring wraps with a mask.
  static_assert((NBUF & (NBUF - 1)) == 0, "ring offsets wrap with a mask");
  constexpr uint32_t RING = NBUF * BUFB - 1;
  auto step = [&](f32x4_t (&cur)[NQB][2], f32x4_t (&nxt)[NQB][2], int i, uint32_t bo) {
    const uint32_t bn = (bo + BUFB) & RING;              // buffer of step i + 1
    const uint32_t bp = (bo + (NBUF - 1) * BUFB) & RING;  // of step i + PF = i - 1 (mod NBUF)
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(2);
    issue(i + PF, bp);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    u32x4_t pb[NQB];
    // ---- S(i+1) on the matrix cores while the VALU turns S(i) into P ----
    {
      const uint8_t* kp = sK + bn;
      // fragment g: keys 16 (g / KSTEPS) + li, logical segment 4 (g % KSTEPS) + lg
      auto kread = [&](int gi) {
        return *reinterpret_cast<const u32x4_t*>(kp + k_ofs[gi % KSTEPS] +
                                                 (gi / KSTEPS) * 16 * ROWB);
      };
      u32x4_t kf[KA + 1];
#pragma unroll
      for (int gi = 0; gi < KA; ++gi) kf[gi] = kread(gi);
      float pe[NQB][2][4];
      // exponential e of the lane's 8 * NQB: block (e / 4) % NQB, key block
      // e / (4 NQB), element e % 4
      auto expo = [&](int e) {
        const int b = (e / 4) % NQB, kb = e / (4 * NQB), r = e % 4;
        const float p = fast_exp2(fmaf(cur[b][kb][r], c, nm[b]));
        pe[b][kb][r] = p;
        l_run[b] += p;  // fp32 P: a sum of the bf16-rounded P misses the LSE bound
        if (r & 1) {
          pb[b][2 * kb + r / 2] = cvt_pk_bf16(pe[b][kb][r - 1], p);
          // keep the softmax here, inside the raised-priority window below,
          // instead of letting the compiler sink it past the mask branch
          asm volatile("" : "+v"(pb[b][2 * kb + r / 2]), "+v"(l_run[b]));
        }
      };
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        if (gi + KA < NG) kf[(gi + KA) % (KA + 1)] = kread(gi + KA);
        const int kb = gi / KSTEPS, st = gi % KSTEPS;
#pragma unroll
        for (int b = 0; b < NQB; ++b) {
          nxt[b][kb] = mfma16(kf[gi % (KA + 1)], qreg[b][st], st == 0 ? f32x4_t{} : nxt[b][kb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P of step i.  On the VALU, after the matrix work above is issued: the
      // other wave on the SIMD (another workgroup, at another phase) keeps
      // the matrix cores busy meanwhile.  With PRIO the wave's priority is
      // raised for this vector work (and for the copy issue), so that when both
      // waves of a SIMD are ready the softmax goes first and the other wave's
      // MFMAs fill the matrix pipe behind it (about 1 % faster, alternated on
      // one box).
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int e = 0; e < NEA; ++e) expo(e);
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    }
    if (needs_mask(i + 1)) apply_mask(nxt, kstart + (i + 1) * BN);
    // ---- O += P V on the matrix cores while the VALU finds S(i+1)'s maxima ----
    float lm[NQB];
    {
      const uint8_t* vb = sV + bo;
      auto vread = [&](int db) {
        const uint8_t* vp = vb + v_ofs[db];
        const u32x2_t v0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vp));
        const u32x2_t v1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vp + 16 * ROWB));
        return u32x4_t{v0[0], v0[1], v1[0], v1[1]};
      };
      u32x4_t vf[KA + 1];
#pragma unroll
      for (int db = 0; db < KA; ++db) vf[db] = vread(db);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        if (db + KA < DBLK) vf[(db + KA) % (KA + 1)] = vread(db + KA);
#pragma unroll
        for (int b = 0; b < NQB; ++b) {
          const int k = db * NQB + b;
          oacc[b][db] = mfma16(vf[db % (KA + 1)], pb[b], oacc[b][db]);
          // the lane's maxima of S(i+1) in the first NQB slots
          if (k < NQB)
            lm[k] = max3f(max3f(nxt[k][0][0], nxt[k][0][1], nxt[k][0][2]),
                          max3f(nxt[k][0][3], nxt[k][1][0], nxt[k][1][1]),
                          fmaxf(nxt[k][1][2], nxt[k][1][3]));
        }
      }
    }
    update_max(lm);
    wait_copies<(PF - 2) * NL>();
    __syncthreads();
  };

  int i = 0;
  uint32_t bo = 0;
  for (; i + 1 < ntiles; i += 2) {
    step(sa, sb, i, bo);
    bo = (bo + BUFB) & RING;
    step(sb, sa, i + 1, bo);
    bo = (bo + BUFB) & RING;
  }
  if (i < ntiles) step(sa, sb, i, bo);
  // Copies of the clamped steps past the end may still be in flight: let them
  // land before the workgroup ends and its LDS goes to another.
  wait_copies<0>();

  // ---- normalise and store ----
#pragma unroll
  for (int b = 0; b < NQB; ++b) {
    const float l_tot = sum_x32(sum_x16(l_run[b]));
    int qh, tl;
    pair_of(b, qh, tl);
    // recomputed here rather than kept from the q loads across the key loop
    // (which would hold 64-bit addresses in scratch)
    asm volatile("" : "+v"(tl), "+v"(qh));
    const int64_t qi = (int64_t)(q_base + q_start + tl) * Hq + qh;
    if (tl < q_count) {
      const float inv = 1.f / l_tot;
      uint16_t* op = a.out + qi * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        u32x2_t w2 = {cvt_pk_bf16(oacc[b][db][0] * inv, oacc[b][db][1] * inv),
                      cvt_pk_bf16(oacc[b][db][2] * inv, oacc[b][db][3] * inv)};
        *reinterpret_cast<u32x2_t*>(op + 16 * db) = w2;
      }
      if (a.lse != nullptr && lg == 0)
        a.lse[qi] = (log2f(l_tot) - nm[b]) * kLn2;
    }
  }
}

}  // namespace pre
}  // namespace pkv
