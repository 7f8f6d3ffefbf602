// Attention backward main pass for grouped-query attention (key/value
// stationary), gfx950.
//
// Per (query tile i, key tile j) the pass recomputes S = Q K^T and
// P = exp(S * scale - lse), then forms dV += P^T dO, dP = dO V^T,
// dS = P o (dP - Delta) * scale, dK += dS^T Q and the dQ partial dS K
// (tilelang-ascend PR "GQA Sink Backward BHSD": review thread listing kernels
// k1-k5, fused here into one loop body as in its single-kernel revision).
//
// Work decomposition: one workgroup (4 waves) owns one (sequence, kv head g,
// key block of 128 rows); wave w owns keys [32w, 32w + 32) of the block.
//  * K and V rows of the wave live in registers as MFMA B operands for the
//    S and dP products; K is also staged transposed in LDS for dQ.
//  * The loop runs over every query head of the group and, per head, over
//    every query block (64 rows) that can see the key block under the causal
//    / window masks.  dK and dV accumulate in fp32 registers across the whole
//    loop and are written once at the end, with no atomics (tilelang PR
//    "[GQA] Add regional atomic add": review comment on accumulating dK/dV
//    fragments across the loop and writing once).
//  * S and dP are computed with the key index in the lane (MFMA column), so P
//    and dS feed the dV / dK products straight from registers.  dS is stored
//    once to LDS (query-major) for dQ = dS K, whose 64 x D result is split
//    over the 4 waves.
//  * dQ partials leave through fp32 atomic adds issued directly from the
//    MFMA C layout: one register = two query rows x 32 consecutive
//    dimensions, i.e. two fully used 128-byte segments per wave instruction
//    (tilelang PR: one region-wide atomic per tile instead of per-element
//    loops; triton issue "atomic_add slows down attention backwards": avoid a
//    layout conversion before the atomics and vectorise them).
//
// The sink needs no term here: it only enters through lse.
#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kBM = 64;   // query rows per step
constexpr int kBN = 128;  // key rows per workgroup (4 waves x 32)

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* delta;
  const int32_t* cu;
  float* dq_accum;
  void* dk;
  void* dv;
  int num_seqs, max_seqlen, total, hq, hkv, window;
  bool causal;
  float scale, scale_log2;
};

template <typename T, int D>
struct BwdSmem {
  alignas(16) T q[kBM][D + 8];     // Q_i, query-major
  alignas(16) T dout[kBM][D + 8];  // dO_i, query-major
  alignas(16) T qt[D][kBM + 8];    // Q_i transposed
  alignas(16) T dot[D][kBM + 8];   // dO_i transposed
  alignas(16) T ds[kBM][kBN + 8];  // dS, query-major
  alignas(16) T kt[D][kBN + 8];    // K_j transposed
  float lse2[kBM];                 // lse * log2(e); +inf outside the sequence
  float delta[kBM];
};

// Stage a [kBM x D] tile (rows r0.., zero-filled past `L`) into a row-major
// and a transposed LDS copy.  A unit is 4 rows x 8 dims: four 16-byte global
// loads, four 16-byte row-major stores and eight 8-byte transposed stores.
template <typename T, int D>
__device__ __forceinline__ void stage_tile(const T* __restrict__ src, size_t row_stride,
                                           int r0, int L, T (*rm)[D + 8], T (*tr)[kBM + 8],
                                           int tid) {
  using T8 = typename V8<T>::type;
  using T4 = typename V8<T>::half_type;
  for (int u = tid; u < (kBM / 4) * (D / 8); u += 256) {
    const int rg = u / (D / 8), dc = u % (D / 8);
    T8 rows[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + 4 * rg + e;
      rows[e] = r < L ? ld16<T>(src + (size_t)r * row_stride + 8 * dc) : zero8<T>();
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) st16<T>(&rm[4 * rg + e][8 * dc], rows[e]);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      T4 col;
#pragma unroll
      for (int e = 0; e < 4; ++e) col[e] = rows[e][dd];
      st8<T>(&tr[8 * dc + dd][4 * rg], col);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdArgs p) {
  using T8 = typename V8<T>::type;
  using T4 = typename V8<T>::half_type;
  __shared__ BwdSmem<T, D> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n = lane & 31, c = lane >> 5;

  // Block order: key-block index slowest, so every (sequence, kv head) gets
  // its largest causal workload (key block 0) first, and the blocks of one
  // (sequence, kv head) are a multiple of 8 apart whenever num_seqs * Hkv is,
  // which keeps them on one XCD and its L2.
  const int nsg = p.num_seqs * p.hkv;
  const int jb = blockIdx.x / nsg;
  const int rem = blockIdx.x % nsg;
  const int s = rem / p.hkv, g = rem % p.hkv;
  int a, b;
  seq_bounds(p.cu, s, p.max_seqlen, p.total, a, b);
  const int L = b - a;
  const int kv0 = jb * kBN;
  if (kv0 >= L) return;
  const int G = p.hq / p.hkv;

  const T* __restrict__ qp = static_cast<const T*>(p.q);
  const T* __restrict__ kp = static_cast<const T*>(p.k);
  const T* __restrict__ vp = static_cast<const T*>(p.v);
  const T* __restrict__ dop = static_cast<const T*>(p.dout);
  const size_t kv_stride = (size_t)p.hkv * D;
  const size_t q_stride = (size_t)p.hq * D;

  // Keys of this lane: B-operand column n of wave w.
  const int kj = kv0 + 32 * w + n;
  T8 kreg[D / 16], vreg[D / 16];
  {
    const size_t off = (size_t)(a + kj) * kv_stride + (size_t)g * D + 8 * c;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kreg[ks] = kj < L ? ld16<T>(kp + off + 16 * ks) : zero8<T>();
      vreg[ks] = kj < L ? ld16<T>(vp + off + 16 * ks) : zero8<T>();
    }
  }
  // K_j transposed into LDS (a unit is 4 keys x 8 dims).
  for (int u = tid; u < (kBN / 4) * (D / 8); u += 256) {
    const int rg = u / (D / 8), dc = u % (D / 8);
    T8 rows[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = kv0 + 4 * rg + e;
      rows[e] = j < L ? ld16<T>(kp + (size_t)(a + j) * kv_stride + (size_t)g * D + 8 * dc)
                      : zero8<T>();
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      T4 col;
#pragma unroll
      for (int e = 0; e < 4; ++e) col[e] = rows[e][dd];
      st8<T>(&sm.kt[8 * dc + dd][4 * rg], col);
    }
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    dk[t] = f32x16{};
    dv[t] = f32x16{};
  }

  // Query blocks that can see any key of this block.
  const int kv_last = min(L, kv0 + kBN) - 1;
  const int ib0 = p.causal ? kv0 / kBM : 0;
  int ib1 = (L + kBM - 1) / kBM;
  if (p.window > 0) ib1 = min(ib1, (kv_last + p.window - 1) / kBM + 1);
  const int wk_lo = kv0 + 32 * w, wk_hi = wk_lo + 31;

  // dQ tiles of this wave: D = 128 -> column tile w, both row tiles;
  // D = 64 -> row tile w / 2, column tile w % 2.
  constexpr int kDqTiles = D / 64;
  const int dq_nt = D == 128 ? w : (w & 1);
  const int dq_mt0 = D == 128 ? 0 : (w >> 1);

  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const T* qh = qp + (size_t)a * q_stride + (size_t)h * D;
    const T* doh = dop + (size_t)a * q_stride + (size_t)h * D;
    for (int ib = ib0; ib < ib1; ++ib) {
      const int q0 = ib * kBM;
      __syncthreads();  // the previous step is done with every LDS tile
      stage_tile<T, D>(qh, q_stride, q0, L, sm.q, sm.qt, tid);
      stage_tile<T, D>(doh, q_stride, q0, L, sm.dout, sm.dot, tid);
      if (tid < kBM) {
        const int r = q0 + tid;
        const size_t idx = (size_t)h * p.total + a + r;
        const float l = r < L ? p.lse[idx] : -INFINITY;
        // Rows outside the sequence, and rows that saw nothing (lse = -inf),
        // get P = 0 through lse2 = +inf.
        sm.lse2[tid] = l == -INFINITY ? INFINITY : l * kLog2e;
        sm.delta[tid] = r < L ? p.delta[idx] : 0.0f;
      }
      __syncthreads();

      // S = Q K^T and dP = dO V^T for 64 queries x this wave's 32 keys.
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      f32x16 pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          sacc[mt] = mfma32(ld16<T>(&sm.q[32 * mt + n][16 * ks + 8 * c]), kreg[ks], sacc[mt]);
          pacc[mt] = mfma32(ld16<T>(&sm.dout[32 * mt + n][16 * ks + 8 * c]), vreg[ks], pacc[mt]);
        }
      }

      // P = exp2(S * scale * log2e - lse * log2e); dS = P (dP - Delta) scale.
      const bool full = (q0 + kBM <= L) && (wk_hi < L) && (!p.causal || wk_hi <= q0) &&
                        (p.window <= 0 || wk_lo > q0 + kBM - 1 - p.window);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 32 * mt + (r >> 2) * 8 + 4 * c + (r & 3);
          float x = sacc[mt][r] * p.scale_log2 - sm.lse2[qr];
          if (!full && (kj >= L || !visible(q0 + qr, kj, p.causal, p.window))) x = -INFINITY;
          const float pv = fast_exp2(x);
          sacc[mt][r] = pv;
          pacc[mt][r] = pv * (pacc[mt][r] - sm.delta[qr]) * p.scale;
        }
      }

      // dV += P^T dO and dK += dS^T Q over the 64 queries (four 16-query
      // steps).  Slot (c, e) of step ks holds query 16 ks + (e / 4) * 8 +
      // 4 c + e % 4, where the C layout of S keeps it.
#pragma unroll
      for (int ks = 0; ks < kBM / 16; ++ks) {
        const T8 pa = pack8<T>(sacc[ks >> 1], 8 * (ks & 1));
        const T8 sa = pack8<T>(pacc[ks >> 1], 8 * (ks & 1));
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const T* dor = &sm.dot[32 * t + n][16 * ks + 4 * c];
          const T* qr = &sm.qt[32 * t + n][16 * ks + 4 * c];
          dv[t] = mfma32(pa, cat8<T>(ld8<T>(dor), ld8<T>(dor + 8)), dv[t]);
          dk[t] = mfma32(sa, cat8<T>(ld8<T>(qr), ld8<T>(qr + 8)), dk[t]);
        }
      }

      // dS to LDS, query-major, for dQ = dS K.
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sm.ds[32 * mt + (r >> 2) * 8 + 4 * c + (r & 3)][32 * w + n] = to16<T>(pacc[mt][r]);
      }
      __syncthreads();

      // dQ partial = dS K over all 128 keys of the block.
      f32x16 qacc[kDqTiles];
#pragma unroll
      for (int t = 0; t < kDqTiles; ++t) qacc[t] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kBN / 16; ++ks) {
        const T8 kb = ld16<T>(&sm.kt[32 * dq_nt + n][16 * ks + 8 * c]);
#pragma unroll
        for (int t = 0; t < kDqTiles; ++t)
          qacc[t] = mfma32(ld16<T>(&sm.ds[32 * (dq_mt0 + t) + n][16 * ks + 8 * c]), kb, qacc[t]);
      }
      // Region-wide fp32 atomics straight from the C layout.
      float* dqh = p.dq_accum + (size_t)a * q_stride + (size_t)h * D + 32 * dq_nt + n;
#pragma unroll
      for (int t = 0; t < kDqTiles; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = q0 + 32 * (dq_mt0 + t) + (r >> 2) * 8 + 4 * c + (r & 3);
          if (qrow < L)
            __hip_atomic_fetch_add(dqh + (size_t)qrow * q_stride, qacc[t][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  // Single write of dK and dV (C layout: column = dim, row = key).
  T* dkp = static_cast<T*>(p.dk) + (size_t)a * kv_stride + (size_t)g * D;
  T* dvp = static_cast<T*>(p.dv) + (size_t)a * kv_stride + (size_t)g * D;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kv0 + 32 * w + (r >> 2) * 8 + 4 * c + (r & 3);
      if (j < L) {
        const size_t off = (size_t)j * kv_stride + 32 * t + n;
        dkp[off] = to16<T>(dk[t][r]);
        dvp[off] = to16<T>(dv[t][r]);
      }
    }
  }
}

template <typename T, int D>
hipError_t bwd_t(const BwdArgs& args, int nkb, hipStream_t stream) {
  const unsigned blocks = (unsigned)nkb * args.num_seqs * args.hkv;
  hipLaunchKernelGGL((bwd_kernel<T, D>), dim3(blocks), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const void* dout, const float* lse, const float* delta,
                      const int32_t* cu, float* dq_accum, void* dk, void* dv,
                      hipStream_t stream) {
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.cu = cu;
  a.dq_accum = dq_accum;
  a.dk = dk;
  a.dv = dv;
  a.num_seqs = p.num_seqs;
  a.max_seqlen = p.max_seqlen;
  a.total = p.total;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.window = p.window;
  a.causal = p.causal;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  const int nkb = (p.max_seqlen + kBN - 1) / kBN;
  if (p.bf16) return p.d == 64 ? bwd_t<__bf16, 64>(a, nkb, stream) : bwd_t<__bf16, 128>(a, nkb, stream);
  return p.d == 64 ? bwd_t<_Float16, 64>(a, nkb, stream) : bwd_t<_Float16, 128>(a, nkb, stream);
}

}  // namespace attn
