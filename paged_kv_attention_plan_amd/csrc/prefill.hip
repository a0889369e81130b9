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
#include "common.cuh"
#include "kernels.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kRescaleSlack = 8.f;  // log2 units: P may reach 2^8 before O is rescaled

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
template <int D, bool WAVE_PAGE>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int BN = 64;              // keys per iteration
  constexpr int KSTEPS = D / 16;      // MFMA steps over head_dim for S
  constexpr int DBLK = D / 32;        // 32-row output blocks over head_dim
  constexpr int SEGS = D / 8;         // 16-byte segments of a key row
  constexpr int KPT = BN * SEGS / 256;  // key rows each thread stages per iteration
  constexpr int KS = D + 8;           // LDS row stride of K (elements): 16-byte row reads
  constexpr int VS = D + 16;          // LDS row stride of V (elements): the four rows a
                                      // transposed read touches start 8 banks apart
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BN * VS];

  const pkv_prefill_tile* tp = a.tiles + blockIdx.x;
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
  auto load_pids = [&](int t, int (&pid)[KPT]) {
    if constexpr (WAVE_PAGE) {
      const int tt = t < ntiles ? t : ntiles - 1;
      int k0 = kstart + tt * BN + 16 * wave;
      k0 = k0 < kv_len ? k0 : kv_len - 1;
      pid[0] = cidx[page_base + (k0 >> ps_log2)];  // uniform: scalar load
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) pid[i] = cidx[page_base + (key_of(t, i) >> ps_log2)];
    }
  };
  u32x4_t gk[KPT], gv[KPT];
  auto gload = [&](int t, const int (&pid)[KPT]) {
    if constexpr (WAVE_PAGE) {
      const char* kb = reinterpret_cast<const char*>(a.cache) + (int64_t)pid[0] * page_elems * 2 +
                       head_bytes;
      const char* vb = kb + (int64_t)v_off * 2;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t off = (uint32_t)(key_of(t, i) & (ps - 1)) * row_bytes + seg * 16u;
        gk[i] = *reinterpret_cast<const u32x4_t*>(kb + off);
        gv[i] = *reinterpret_cast<const u32x4_t*>(vb + off);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int key = key_of(t, i);
        const uint16_t* p = a.cache + (int64_t)pid[i] * page_elems +
                            (key & (ps - 1)) * row_elems + hk * D + seg * 8;
        gk[i] = *reinterpret_cast<const u32x4_t*>(p);
        gv[i] = *reinterpret_cast<const u32x4_t*>(p + v_off);
      }
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      *reinterpret_cast<u32x4_t*>(&sK[(kg * KPT + i) * KS + seg * 8]) = gk[i];
      *reinterpret_cast<u32x4_t*>(&sV[(kg * KPT + i) * VS + seg * 8]) = gv[i];
    }
  };

  // Pipeline: the data of tile it+1 is loaded while tile it is computed, and
  // the page ids of tile it+2 one tile earlier still, so no page-id load sits
  // in front of a data load.
  int pid_next[KPT];
  {
    int pid0[KPT];
    load_pids(0, pid0);
    gload(0, pid0);
  }
  load_pids(1, pid_next);
  for (int it = 0; it < ntiles; ++it) {
    const int kbase = kstart + it * BN;
    __syncthreads();  // every wave is done reading the previous tile
    swrite();
    gload(it + 1, pid_next);  // clamped past the end: the loads in flight are the same every trip
    load_pids(it + 2, pid_next);
    __syncthreads();

    // ---- S^T = K . Q^T ----
    f32x16_t sacc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sacc[kb2] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const u32x4_t kf =
            *reinterpret_cast<const u32x4_t*>(&sK[(kb2 * 32 + jcol) * KS + 16 * s + 8 * half]);
        sacc[kb2] = mfma32(kf, qreg[s], sacc[kb2]);
      }
    }

    // ---- mask, online softmax ----
    // sacc[kb2][r] is key kbase + 32 kb2 + 8 (r/4) + 4 half + r%4 for query jcol.
    const bool need_mask = (kbase + BN - 1 > (causal ? p_first : kv_len - 1)) ||
                           (kbase + BN > kv_len) || (wl >= 0 && kbase < p_last - wl);
    if (need_mask) {  // uniform: the tile crosses the diagonal, the window edge or the row end
      const int k0 = kbase + 4 * half;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb2 + 8 * (r >> 2) + (r & 3);
          sacc[kb2][r] = (key > hi_j || key < lo_j) ? -INFINITY : sacc[kb2][r];
        }
    }
    // Max over the raw scores (the scale is positive, so order is kept), then scaled.
    float mr = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mr = fmaxf(mr, fmaxf(sacc[0][r], sacc[0][r + 1]));
#pragma unroll
    for (int r = 0; r < 16; r += 2) mr = fmaxf(mr, fmaxf(sacc[1][r], sacc[1][r + 1]));
    mr = fmaxf(mr, __shfl_xor(mr, 32));
    const float mt = mr * c;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0) {  // uniform
      const float mn = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DBLK; ++b) oacc[b] *= alpha;
    }
    const float neg_m = -m_run;
    u32x4_t pb[4];  // P^T operand per 16-key step s = 2 kb2 + t
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(sacc[kb2][8 * t + e], c, neg_m));
          l_run += p[e];
        }
        pb[2 * kb2 + t] = u32x4_t{cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]),
                                  cvt_pk_bf16(p[4], p[5]), cvt_pk_bf16(p[6], p[7])};
      }
    }

    // ---- O^T += V^T . P^T ----
    // Step s covers keys 16 s + {0..3, 8..11} + 4 half, matching pb[s]'s element
    // order; the transposed reads deliver column 32 b + jcol at those keys.
    {
      const int grp = lane >> 4, ga = lane & 15;
      const int key_l = 4 * (grp >> 1) + (ga >> 2);
      const int d_l = 16 * (grp & 1) + 4 * (ga & 3);
#pragma unroll
      for (int b = 0; b < DBLK; ++b) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint16_t* vp = &sV[(16 * s + key_l) * VS + 32 * b + d_l];
          const u32x2_t v0 = lds_read_tr16(vp);
          const u32x2_t v1 = lds_read_tr16(vp + 8 * VS);
          oacc[b] = mfma32(u32x4_t{v0[0], v0[1], v1[0], v1[1]}, pb[s], oacc[b]);
        }
      }
    }
  }

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

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_tiles), block(256);
  if (a.page_size >= 16)
    hipLaunchKernelGGL((prefill_kernel<D, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.n_tiles <= 0) return hipSuccess;
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
