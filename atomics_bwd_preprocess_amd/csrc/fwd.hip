// Attention forward with online softmax, attention sink, causal / sliding-window
// masks and varlen packing (tilelang-ascend PR "GQA Sink Backward BHSD":
// forward kernel of its 2-kernel architecture, producing O and lse).
//
// gfx950 design: one workgroup = 4 waves = 128 query rows of one (sequence,
// query head), two workgroups per CU; wave w owns rows [32w, 32w + 32) and
// keeps its Q rows in registers as the MFMA B operand.  The loop walks
// 64-key blocks.  Each block's K and V tiles are copied from memory straight
// into LDS (buffer loads with an LDS destination; row-major tiles with
// XOR-swizzled 16-byte chunks, double-buffered, issued one block ahead), and
// per wave
//     S^T = K Q^T      (32x32x16 MFMA, K rows from LDS, Q^T from registers)
//     O^T += V^T P^T   (V^T from the transposing LDS read, P^T straight from
//                       the MFMA C layout of S^T)
// so the softmax statistics of one query live in one lane pair (l, l ^ 32).
// The running maximum is taken over raw scores (the scale is positive) and
// the scale folds into the exponent's FMA.  The sink initialises the running
// max and sum (m = sink, l = 1), which adds exp(sink) to the denominator
// without a value vector.  A wave skips the blocks that are masked for all
// of its rows, masks are applied only on blocks that need them, and there is
// one workgroup barrier per block.
#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kFwdBM = 128;  // query rows per workgroup
constexpr int kFwdBN = 64;   // keys per block
constexpr int kFwdNW = 4;    // waves per workgroup
constexpr int kFwdThreads = 64 * kFwdNW;

template <int D>
struct FwdCfg {
  static constexpr int CH = D / 8;                               // 16-byte chunks per row
  static constexpr int TILE = kFwdBN * D * 2;                    // bytes of a K or V tile
  static constexpr int STAGE = 2 * TILE;                         // K tile, then V tile
  static constexpr int BYTES = 2 * STAGE;                        // two stages
  static constexpr int NDMA = 2 * kFwdBN * CH / kFwdThreads;     // 16-byte copies per thread per block
  static_assert(kFwdBN * CH % 64 == 0 && NDMA * kFwdThreads == 2 * kFwdBN * CH, "copy split");
  // Workgroups per CU: four at D = 64 (about 120 registers per wave), two at
  // D = 128.
  static constexpr int WGS = D == 64 ? 4 : 2;
  static_assert(WGS * BYTES <= 160 * 1024, "LDS for WGS workgroups per CU");
};

// acc + the sum of the 8 values, two per v_dot2_f32_{f16,bf16} (products
// with 1 are exact; accumulation in fp32).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sum8(f16x8 v, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 pr = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float sum8(bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}

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

// BHSD: [B, H, S, D] tensors instead of packed [T, H, D].  WIN: sliding
// windows, where a wave also skips the products of the 32-key halves of a
// block that none of its rows can see (their scores are -inf, their P zero).
template <typename T, int D, bool BHSD, bool WIN>
__global__ __launch_bounds__(kFwdThreads, FwdCfg<D>::WGS) void fwd_kernel(FwdArgs p) {
  using C = FwdCfg<D>;
  using T8 = typename V8<T>::type;
  using T4 = typename V8<T>::half_type;
  __shared__ __attribute__((aligned(16))) char smem[C::BYTES];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n = lane & 31, c = lane >> 5;
  const int l16 = lane & 15, g16 = (lane >> 4) & 1;

  // Longest work first: the largest query-block index of every (seq, head)
  // is dispatched before smaller ones.  Within one query-block index the kv
  // group varies fastest, so (with Hkv a multiple of 8) every head of a group
  // lands on the same XCD -- workgroups are dealt round-robin over the 8
  // XCDs -- and the group's K / V blocks are shared through one L2.
  const int nsh = p.num_seqs * p.hq;
  const int G = p.hq / p.hkv;
  const int qb = p.nqb - 1 - (int)(blockIdx.x / nsh);
  const int rem = blockIdx.x % nsh;
  const int s = rem / p.hq;
  const int h = (rem % p.hkv) * G + (rem % p.hq) / p.hkv;
  int a, b;
  seq_bounds(p.cu, s, p.max_seqlen, p.total, a, b);
  const int L = b - a;
  const int q0 = qb * kFwdBM;
  if (q0 >= L) return;
  const int g = h / G;
  const uint32_t kv_row = BHSD ? (uint32_t)D : (uint32_t)p.hkv * D;  // elements between key rows
  const uint32_t q_row = BHSD ? (uint32_t)D : (uint32_t)p.hq * D;     // elements between query rows

  // This lane's query (B-operand column n of wave w); rows past the sequence
  // end read as zero.
  const int qi = q0 + 32 * w + n;
  const int qrows = uni(min(L - q0, kFwdBM));
  const rsrc_t qr = make_rsrc(static_cast<const T*>(p.q) + row_off<D, BHSD>(a, q0, h, p.hq, p.max_seqlen),
                              qrows * q_row * 2);
  T8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qreg[ks] = __builtin_bit_cast(T8, buf_load16(qr, ((32 * w + n) * q_row + 16 * ks + 8 * c) * 2));

  float m_run, l_run;  // running max (scaled, log2 units) and sum
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
  // Rows of this wave (for the skip and mask decisions).
  const int wq_lo = q0 + 32 * w, wq_hi = min(q0 + 32 * w + 31, L - 1);

  // Copy keys [kb, kb + 64) of K and V into stage `stage`.  Lane l of wave w
  // fills physical chunk 64 (w + 4 u) + l of the K tile followed by the V
  // tile: row P / CH, logical chunk (P % CH) ^ swz(row).  Rows past the
  // sequence end repeat its last key (finite values; masked below).
  const T* kp = static_cast<const T*>(p.k);
  const T* vp = static_cast<const T*>(p.v);
  // Per-lane source offsets within a full block (loop-invariant).
  uint32_t coff[C::NDMA];
#pragma unroll
  for (int u = 0; u < C::NDMA; ++u) {
    const int Pt = (64 * (w + kFwdNW * u)) % (kFwdBN * C::CH);
    const int P = Pt + lane;
    const int r = P / C::CH, ch = (P % C::CH) ^ chunk_swz<D>(r);
    coff[u] = ((uint32_t)r * kv_row + 8 * ch) * 2;
  }
  // Copy u of a block fills the K tile for u < NDMA / 2 and the V tile
  // otherwise; its wave-uniform LDS address is this wave's base plus
  // constants, formed once.
  const uint32_t lds_w = lds_addr(smem) + 1024u * (uint32_t)uni(w);
  auto issue = [&](int kb, int stage) {
    const int nk = uni(min(L - kb, kFwdBN));
    const size_t base = row_off<D, BHSD>(a, kb, g, p.hkv, p.max_seqlen);
    const rsrc_t kr = make_rsrc(kp + base, nk * kv_row * 2);
    const rsrc_t vr = make_rsrc(vp + base, nk * kv_row * 2);
    const uint32_t lds_s = lds_w + (uint32_t)uni(stage) * C::STAGE;
    constexpr int kHalf = C::NDMA / 2;
    if (nk == kFwdBN) {
#pragma unroll
      for (int u = 0; u < C::NDMA; ++u) {
        const bool isv = u >= kHalf;
        const int uu = isv ? u - kHalf : u;
        lds_dma16(isv ? vr : kr, lds_s + (isv ? C::TILE : 0) + 1024u * kFwdNW * uu, coff[u]);
      }
    } else {  // tail block: rows past the end repeat the last key
#pragma unroll
      for (int u = 0; u < C::NDMA; ++u) {
        const bool isv = u >= kHalf;
        const int uu = isv ? u - kHalf : u;
        const int P = 64 * (w + kFwdNW * uu) + lane;
        const int r = P / C::CH, ch = (P % C::CH) ^ chunk_swz<D>(r);
        const uint32_t off = ((uint32_t)min(r, nk - 1) * kv_row + 8 * ch) * 2;
        lds_dma16(isv ? vr : kr, lds_s + (isv ? C::TILE : 0) + 1024u * kFwdNW * uu, off);
      }
    }
  };

  issue(k_lo, 0);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  int stage = 0;
  for (int kb = k_lo; kb < k_hi; kb += kFwdBN, stage ^= 1) {
    // The other stage was last read before the previous barrier.
    if (kb + kFwdBN < k_hi) issue(kb + kFwdBN, stage ^ 1);

    const bool skip = wq_lo > wq_hi || (p.causal && kb > wq_hi) ||
                      (p.window > 0 && kb + kFwdBN - 1 <= wq_lo - p.window);
    if (!skip) {
      const char* kt = smem + stage * C::STAGE;
      const char* vt = kt + C::TILE;

      // S^T for keys [kb, kb + 64) (two 32-row tiles) against this wave's queries.
      f32x16 st[2] = {f32x16{}, f32x16{}};
      bool hvis[2] = {true, true};  // WIN: some row of the wave sees the half
      if constexpr (WIN) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int h_lo = kb + 32 * mt, h_hi = h_lo + 31;
          hvis[mt] = !(h_lo >= L || (p.causal && h_lo > wq_hi) || h_hi <= wq_lo - p.window);
          if (hvis[mt]) {
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
              st[mt] = mfma32(lds16<T>(kt, rm_off<D>(32 * mt + n, 16 * ks + 8 * c)), qreg[ks], st[mt]);
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) st[mt][r] = -INFINITY;
          }
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            st[mt] = mfma32(lds16<T>(kt, rm_off<D>(32 * mt + n, 16 * ks + 8 * c)), qreg[ks], st[mt]);
      }

      // Hidden keys -> -inf, only on blocks not fully visible to every row of
      // the wave.  The empty asm keeps this a real branch.
      const int kb_last = kb + kFwdBN - 1;
      const bool full = (kb_last < L) && (!p.causal || kb_last <= wq_lo) &&
                        (p.window <= 0 || kb > wq_hi - p.window);
      if (!full) {
        asm volatile("");
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kb + 32 * mt + (r >> 2) * 8 + 4 * c + (r & 3);
            if (j >= L || !visible(qi, j, p.causal, p.window)) st[mt][r] = -INFINITY;
          }
      }

      // Online softmax over raw scores: the maximum is scaled afterwards.
      float mraw = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, st[mt][r]);
      mraw = fmaxf(mraw, xor32(mraw));
      const float m_new = fmaxf(m_run, mraw * p.scale_log2);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[mt][r] = fast_exp2(st[mt][r] * p.scale_log2 - m_use);
      // alpha is exactly 1 on lanes whose maximum did not move; skip the
      // rescale when that holds for the whole wave.
      if (!__all(m_new == m_run)) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;
      }
      m_run = m_new;

      // O^T += V^T P^T over the 64 keys in four 16-key steps.  Slot (c, e)
      // of step ks holds key 16 ks + (e / 4) * 8 + 4 c + e % 4, which is
      // where the C layout of S^T already keeps it; the transposing read of
      // the row-major V tile delivers the A operand in the same order.  The
      // row sum is taken over the same rounded P (two per dot2 instruction,
      // fp32 accumulation), so the weights of O sum to one.
      float lsum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kFwdBN / 16; ++ks) {
        if (WIN && !hvis[ks >> 1]) continue;  // P = 0 there
        const T8 pb = pack8<T>(st[ks >> 1], 8 * (ks & 1));
        lsum = sum8(pb, lsum);
        const int row = 16 * ks + 4 * c + (l16 >> 2);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const int col = 32 * t + 16 * g16 + 4 * (lane & 3);
          oacc[t] = mfma32(tr_pair<T>(vt, rm_off<D>(row, col), rm_off<D>(row + 8, col)), pb, oacc[t]);
        }
      }
      lsum += xor32(lsum);
      l_run = l_run * alpha + lsum;
    }
    // The next block's copies have landed and every wave is done with this
    // stage before it is overwritten.
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
  }

  if (qi >= L) return;
  const bool any = l_run > 0.0f;
  const float inv = any ? 1.0f / l_run : 0.0f;
  T* __restrict__ op = static_cast<T*>(p.o) + row_off<D, BHSD>(a, qi, h, p.hq, p.max_seqlen);
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
hipError_t fwd_t(const FwdArgs& args, bool bhsd, hipStream_t stream) {
  const unsigned blocks = (unsigned)args.nqb * args.num_seqs * args.hq;
  const dim3 grid(blocks), block(kFwdThreads);
  if (args.window > 0) {
    if (bhsd)
      hipLaunchKernelGGL((fwd_kernel<T, D, true, true>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, false, true>), grid, block, 0, stream, args);
  } else {
    if (bhsd)
      hipLaunchKernelGGL((fwd_kernel<T, D, true, false>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, false, false>), grid, block, 0, stream, args);
  }
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
  if (p.bf16)
    return p.d == 64 ? fwd_t<__bf16, 64>(a, p.bhsd, stream) : fwd_t<__bf16, 128>(a, p.bhsd, stream);
  return p.d == 64 ? fwd_t<_Float16, 64>(a, p.bhsd, stream) : fwd_t<_Float16, 128>(a, p.bhsd, stream);
}

}  // namespace attn
