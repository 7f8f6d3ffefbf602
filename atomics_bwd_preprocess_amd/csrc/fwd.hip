// Attention forward with online softmax, attention sink, causal / sliding-window
// masks and varlen packing (tilelang-ascend PR "GQA Sink Backward BHSD":
// forward kernel of its 2-kernel architecture, producing O and lse).
//
// gfx950 design: one workgroup = 4 waves = 128 query rows of one (sequence,
// query head); wave w owns rows [32w, 32w + 32).  Its Q rows stay in
// registers as the MFMA B operand.  The loop walks 64-key blocks staged in LDS
// (K row-major, V transposed) and computes, per wave,
//     S^T = K Q^T      (32x32x16 MFMA, K from LDS, Q^T from registers)
//     O^T += V^T P^T   (P^T is consumed directly from the MFMA C layout)
// so the softmax statistics of one query live in one lane pair (l, l ^ 32).
// The sink initialises the running max and sum (m = sink, l = 1), which adds
// exp(sink) to the denominator without a value vector.
#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kFwdBM = 128;  // query rows per workgroup
constexpr int kFwdBN = 64;   // keys per block

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu;
  const float* sink;
  void* o;
  float* lse;
  int num_seqs, max_seqlen, total, hq, hkv, window, nqb;
  bool causal;
  float scale_log2;
};

template <typename T, int D>
struct FwdSmem {
  alignas(16) T k[kFwdBN][D + 8];
  alignas(16) T vt[D][kFwdBN + 8];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs p) {
  using T8 = typename V8<T>::type;
  using T4 = typename V8<T>::half_type;
  __shared__ FwdSmem<T, D> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n = lane & 31, c = lane >> 5;

  // Longest work first: the largest query-block index of every (seq, head)
  // is dispatched before smaller ones.
  const int nsh = p.num_seqs * p.hq;
  const int qb = p.nqb - 1 - (int)(blockIdx.x / nsh);
  const int rem = blockIdx.x % nsh;
  const int s = rem / p.hq, h = rem % p.hq;
  int a, b;
  seq_bounds(p.cu, s, p.max_seqlen, p.total, a, b);
  const int L = b - a;
  const int q0 = qb * kFwdBM;
  if (q0 >= L) return;
  const int g = h / (p.hq / p.hkv);
  const T* __restrict__ qp = static_cast<const T*>(p.q);
  const T* __restrict__ kp = static_cast<const T*>(p.k);
  const T* __restrict__ vp = static_cast<const T*>(p.v);

  // This lane's query (B-operand column n of wave w).
  const int qi = q0 + 32 * w + n;
  const bool qvalid = qi < L;
  T8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qreg[ks] = qvalid ? ld16<T>(qp + ((size_t)(a + qi) * p.hq + h) * D + 16 * ks + 8 * c)
                      : zero8<T>();

  float m_run, l_run;
  if (p.sink) {
    m_run = p.sink[h] * kLog2e;
    l_run = 1.0f;
  } else {
    m_run = -INFINITY;
    l_run = 0.0f;
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};

  // Key range visible to any row of this workgroup.
  const int qlast = min(L, q0 + kFwdBM) - 1;
  int k_lo = 0, k_hi = L;
  if (p.causal) k_hi = qlast + 1;
  if (p.window > 0) k_lo = max(0, q0 - p.window + 1);
  k_lo = (k_lo / kFwdBN) * kFwdBN;
  // Rows of this wave (for the mask decision).
  const int wq_lo = q0 + 32 * w, wq_hi = min(q0 + 32 * w + 31, L - 1);

  for (int kb = k_lo; kb < k_hi; kb += kFwdBN) {
    __syncthreads();
    // K block, row-major: 64 rows x D / 8 chunks of 16 bytes.
    for (int u = tid; u < kFwdBN * (D / 8); u += 256) {
      const int r = u / (D / 8), dc = u % (D / 8);
      const int j = kb + r;
      st16<T>(&sm.k[r][8 * dc],
              j < L ? ld16<T>(kp + ((size_t)(a + j) * p.hkv + g) * D + 8 * dc) : zero8<T>());
    }
    // V block, transposed through registers: a unit is 4 keys x 8 dims.
    for (int u = tid; u < (kFwdBN / 4) * (D / 8); u += 256) {
      const int rg = u / (D / 8), dc = u % (D / 8);
      T8 rows[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = kb + 4 * rg + e;
        rows[e] = j < L ? ld16<T>(vp + ((size_t)(a + j) * p.hkv + g) * D + 8 * dc) : zero8<T>();
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        T4 col;
#pragma unroll
        for (int e = 0; e < 4; ++e) col[e] = rows[e][dd];
        st8<T>(&sm.vt[8 * dc + dd][4 * rg], col);
      }
    }
    __syncthreads();
    if (wq_lo > wq_hi) continue;  // wave entirely past the sequence end

    // S^T for keys [kb, kb + 64) (two 32-row tiles) against this wave's queries.
    f32x16 st[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        st[mt] = mfma32(ld16<T>(&sm.k[32 * mt + n][16 * ks + 8 * c]), qreg[ks], st[mt]);
    }

    // Mask only blocks that are not fully visible to every row of this wave.
    const int kb_last = kb + kFwdBN - 1;
    const bool full = (kb_last < L) && (!p.causal || kb_last <= wq_lo) &&
                      (p.window <= 0 || kb > wq_hi - p.window);
    float mloc = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = st[mt][r] * p.scale_log2;
        if (!full) {
          const int j = kb + 32 * mt + (r >> 2) * 8 + 4 * c + (r & 3);
          if (j >= L || !visible(qi, j, p.causal, p.window)) x = -INFINITY;
        }
        st[mt][r] = x;
        mloc = fmaxf(mloc, x);
      }
    }
    mloc = fmaxf(mloc, xor32(mloc));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float lsum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(st[mt][r] - m_use);
        st[mt][r] = pv;
        lsum += pv;
      }
    }
    lsum += xor32(lsum);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;

    // O^T += V^T P^T over the 64 keys in four 16-key steps.  Slot (c, e) of
    // step ks holds key 16 ks + (e / 4) * 8 + 4 c + e % 4, which is where the
    // C layout of S^T already keeps it.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const T8 pb = pack8<T>(st[ks >> 1], 8 * (ks & 1));
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const T* row = &sm.vt[32 * t + n][16 * ks + 4 * c];
        oacc[t] = mfma32(cat8<T>(ld8<T>(row), ld8<T>(row + 8)), pb, oacc[t]);
      }
    }
  }

  if (!qvalid) return;
  const bool any = l_run > 0.0f;
  const float inv = any ? 1.0f / l_run : 0.0f;
  T* __restrict__ op = static_cast<T*>(p.o) + ((size_t)(a + qi) * p.hq + h) * D;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      T4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = to16<T>(oacc[t][4 * rg + e] * inv);
      st8<T>(op + 32 * t + 8 * rg + 4 * c, out);
    }
  }
  if (c == 0)
    p.lse[(size_t)h * p.total + a + qi] = any ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
}

template <typename T, int D>
hipError_t fwd_t(const FwdArgs& args, hipStream_t stream) {
  const unsigned blocks = (unsigned)args.nqb * args.num_seqs * args.hq;
  hipLaunchKernelGGL((fwd_kernel<T, D>), dim3(blocks), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const Problem& p, const void* q, const void* k, const void* v,
                      const int32_t* cu, const float* sink, void* o, float* lse,
                      hipStream_t stream) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu = cu;
  a.sink = sink;
  a.o = o;
  a.lse = lse;
  a.num_seqs = p.num_seqs;
  a.max_seqlen = p.max_seqlen;
  a.total = p.total;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.window = p.window;
  a.causal = p.causal;
  a.nqb = (p.max_seqlen + kFwdBM - 1) / kFwdBM;
  a.scale_log2 = p.scale * kLog2e;
  if (p.bf16) return p.d == 64 ? fwd_t<__bf16, 64>(a, stream) : fwd_t<__bf16, 128>(a, stream);
  return p.d == 64 ? fwd_t<_Float16, 64>(a, stream) : fwd_t<_Float16, 128>(a, stream);
}

}  // namespace attn
