// Causal ragged prefill over a paged KV cache (FlashInferPrefillWrapper.run on
// the mstar attn.wrappers page; the [cached prefix | fresh tokens] sequence of
// attn.dense).  A dense contraction, so both products run on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
// A workgroup (4 waves) owns one tile: a row, a KV head and a block of BT =
// 128/group query tokens, i.e. 128 (query head, token) pairs that all read the
// same K/V.  Wave w takes pairs 32w..32w+31.  Keys are consumed 64 at a time:
// the workgroup gathers the 64 key rows from their pages into LDS -- K as rows
// [key][d], V transposed [d][key] -- and every wave then computes
//   S^T (64 keys x 32 queries) = K . Q^T       (A = K from LDS, B = Q in registers)
//   P = exp2(S*scale*log2e - m)                (online softmax, fp32, per query column)
//   O^T (D x 32 queries)     += V^T . P^T      (A = V^T from LDS, B = P as bf16)
// With S^T a lane holds one query column, so the row max needs a single
// cross-half exchange and the per-query rescale is a per-lane scalar.
#include "common.cuh"
#include "kernels.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

// Two bf16 of different keys at the same dimension, packed (key a low, key b high).
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int BN = 64;              // keys per iteration
  constexpr int KSTEPS = D / 16;      // MFMA steps over head_dim for S
  constexpr int DBLK = D / 32;        // 32-row output blocks over head_dim
  constexpr int SEGS = D / 8;         // 16-byte segments of a key row
  constexpr int KPT = BN * SEGS / 256;  // key rows each thread stages per iteration
  constexpr int KS = D + 8;           // LDS row stride of K (elements)
  constexpr int VS = BN + 4;          // LDS row stride of V^T (elements)
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VS];

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
  float m_run = -1e30f, l_run = 0.f;

  // Block-wide query position bounds, for deciding which key tiles need masks.
  const int p_first = kv_len - q_len + q_start;
  const int p_last = p_first + q_count - 1;

  // Staging map: thread -> (segment, key group of KPT keys).
  const int seg = threadIdx.x % SEGS;
  const int kg = threadIdx.x / SEGS;
  u32x4_t gk[KPT], gv[KPT];
  auto gload = [&](int kbase) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int key = kbase + kg * KPT + i;
      key = key < kv_len ? key : kv_len - 1;  // past the row: masked later, address kept valid
      const int phys = a.indices[page_base + (key >> ps_log2)];
      const uint16_t* p = a.cache + (int64_t)phys * page_elems + (key & (ps - 1)) * row_elems +
                          hk * D + seg * 8;
      gk[i] = *reinterpret_cast<const u32x4_t*>(p);
      gv[i] = *reinterpret_cast<const u32x4_t*>(p + v_off);
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      *reinterpret_cast<u32x4_t*>(&sK[(kg * KPT + i) * KS + seg * 8]) = gk[i];
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // dword w of a key row holds d = seg*8 + 2w, 2w+1
      if constexpr (KPT == 4) {
        const uint32_t x0 = gv[0][w], x1 = gv[1][w], x2 = gv[2][w], x3 = gv[3][w];
        const u32x2_t lo = {lo_halves(x0, x1), lo_halves(x2, x3)};
        const u32x2_t hi = {hi_halves(x0, x1), hi_halves(x2, x3)};
        *reinterpret_cast<u32x2_t*>(&sV[(seg * 8 + 2 * w) * VS + kg * 4]) = lo;
        *reinterpret_cast<u32x2_t*>(&sV[(seg * 8 + 2 * w + 1) * VS + kg * 4]) = hi;
      } else {
        const uint32_t x0 = gv[0][w], x1 = gv[1][w];
        *reinterpret_cast<uint32_t*>(&sV[(seg * 8 + 2 * w) * VS + kg * 2]) = lo_halves(x0, x1);
        *reinterpret_cast<uint32_t*>(&sV[(seg * 8 + 2 * w + 1) * VS + kg * 2]) = hi_halves(x0, x1);
      }
    }
  };

  const int kstart = kv_lo & ~(BN - 1);
  const int kend = kv_hi + 1;
  const int ntiles = (kend - kstart + BN - 1) / BN;

  gload(kstart);
  for (int it = 0; it < ntiles; ++it) {
    const int kbase = kstart + it * BN;
    __syncthreads();  // every wave is done reading the previous tile
    swrite();
    __syncthreads();
    if (it + 1 < ntiles) gload(kbase + BN);

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
    float sv[2][16];
    float mt = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[kb2][r] * a.scale_log2;
        if (need_mask) {
          const int key = kbase + 32 * kb2 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > hi_j || key < lo_j) x = -INFINITY;
        }
        sv[kb2][r] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - mn);
    m_run = mn;
    l_run *= alpha;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) oacc[b] *= alpha;
    u32x4_t pb[4];  // P^T operand per 16-key step s = 2 kb2 + t
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(sv[kb2][8 * t + e] - mn);
          l_run += p[e];
        }
        pb[2 * kb2 + t] = u32x4_t{cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]),
                                  cvt_pk_bf16(p[4], p[5]), cvt_pk_bf16(p[6], p[7])};
      }
    }

    // ---- O^T += V^T . P^T ----
    // Step s covers keys 16 s + {0..3, 8..11} + 4 half, matching pb[s]'s element order.
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint16_t* vrow = &sV[(32 * b + jcol) * VS + 16 * s + 4 * half];
        const u32x2_t v0 = *reinterpret_cast<const u32x2_t*>(vrow);
        const u32x2_t v1 = *reinterpret_cast<const u32x2_t*>(vrow + 8);
        oacc[b] = mfma32(u32x4_t{v0[0], v0[1], v1[0], v1[1]}, pb[s], oacc[b]);
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

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.n_tiles <= 0) return hipSuccess;
  const dim3 grid(a.n_tiles), block(256);
  if (a.head_dim == 128) hipLaunchKernelGGL(prefill_kernel<128>, grid, block, 0, stream, a);
  else if (a.head_dim == 64) hipLaunchKernelGGL(prefill_kernel<64>, grid, block, 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
