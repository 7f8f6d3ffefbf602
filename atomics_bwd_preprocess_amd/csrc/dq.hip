// Query-stationary dQ pass: dQ accumulated on chip, written once, no atomics
// (tilelang-ascend PR "GQA Sink Backward BHSD": its backward keeps dQ in the
// matrix unit's accumulator over the key loop -- the query-stationary
// orientation -- while the key/value-stationary main pass of this library
// sends dQ through fp32 atomics).  Together with the main pass built without
// its dQ product (dK / dV only) it forms a backward whose every output is
// bitwise reproducible.
//
// Per (query tile, key block) the pass recomputes
//     S = Q K^T,  P = exp(S scale - lse),  dP = dO V^T,  dS = P o (dP - Delta)
// and accumulates dQ += dS K; the score scale is applied once at the end.
//
// gfx950 design (the forward's layout): one workgroup = 4 waves = 128 query
// rows of one (sequence, query head), two workgroups per CU; wave w owns rows
// [32w, 32w + 32) and holds its Q and dO rows in registers as MFMA B
// operands, so the lse and Delta of a lane's query are two registers.  The
// loop walks 64-key blocks whose K and V tiles are copied from memory straight
// into LDS (double-buffered, one block ahead, XOR-swizzled row-major tiles),
// and per wave and 32-key half
//     S^T  = K  Q^T     (K rows from LDS)
//     dP^T = V  dO^T    (V rows from LDS)
//     dS^T = P^T o (dP^T - Delta)        in the MFMA C layout
//     dQ^T += K^T dS^T  (K^T from the transposing LDS read; dS^T is already
//                        in the B-operand order)
// Waves skip blocks that are hidden from all of their rows; masks are applied
// only on blocks that need them; one workgroup barrier per block.
#include "common.h"
#include "delta_dot.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kDqBM = 128;  // query rows per workgroup
constexpr int kDqBN = 64;   // keys per block
constexpr int kDqNW = 4;    // waves per workgroup
constexpr int kDqThreads = 64 * kDqNW;

template <int D>
struct DqCfg {
  static constexpr int CH = D / 8;                            // 16-byte chunks per row
  static constexpr int TILE = kDqBN * D * 2;                  // bytes of a K or V tile
  static constexpr int STAGE = 2 * TILE;                      // K tile, then V tile
  static constexpr int BYTES = 2 * STAGE;                     // two stages
  static constexpr int NDMA = 2 * kDqBN * CH / kDqThreads;    // 16-byte copies per thread per block
  static_assert(kDqBN * CH % 64 == 0 && NDMA * kDqThreads == 2 * kDqBN * CH, "copy split");
  // Workgroups per CU: three at D = 64 (about 150 registers per wave), two
  // at D = 128.
  static constexpr int WGS = D == 64 ? 3 : 2;
  static_assert(WGS * BYTES <= 160 * 1024, "LDS for WGS workgroups per CU");
};

struct DqArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* delta;
  const int32_t* cu;
  void* dq;
  // Optional: O, to form Delta here instead of reading it (written to
  // delta_out), in the preprocess's arithmetic and summation order.
  const void* o;
  float* delta_out;
  int num_seqs, max_seqlen, total, hq, hkv, window, nqb;
  bool causal;
  float scale, scale_log2;
};

// BHSD: [B, H, S, D] tensors instead of packed [T, H, D].  WIN: sliding
// windows, where a wave also skips the 32-key halves of a block that none of
// its rows can see (measured 8 % faster at W = 128, 2 % slower on long
// causal problems, hence only here).
template <typename T, int D, bool BHSD, bool WIN>
__global__ __launch_bounds__(kDqThreads, DqCfg<D>::WGS) void dq_kernel(DqArgs p) {
  using C = DqCfg<D>;
  using T8 = typename V8<T>::type;
  using T4 = typename V8<T>::half_type;
  __shared__ __attribute__((aligned(16))) char smem[C::BYTES];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n = lane & 31, c = lane >> 5;
  const int l16 = lane & 15, g16 = (lane >> 4) & 1;

  // Longest work first (largest query-block index of every (seq, head));
  // within one index the kv group varies fastest, so with Hkv a multiple of 8
  // the heads of a group share an XCD and read the group's K / V through one L2.
  const int nsh = p.num_seqs * p.hq;
  const int G = p.hq / p.hkv;
  const int qb = p.nqb - 1 - (int)(blockIdx.x / nsh);
  const int rem = blockIdx.x % nsh;
  const int s = rem / p.hq;
  const int h = (rem % p.hkv) * G + (rem % p.hq) / p.hkv;
  int a, b;
  seq_bounds(p.cu, s, p.max_seqlen, p.total, a, b);
  const int L = b - a;
  const int q0 = qb * kDqBM;
  if (q0 >= L) return;
  const int g = h / G;
  const uint32_t kv_row = BHSD ? (uint32_t)D : (uint32_t)p.hkv * D;  // elements between key rows
  const uint32_t q_row = BHSD ? (uint32_t)D : (uint32_t)p.hq * D;     // elements between query rows

  // This lane's query (B-operand column n of wave w): its Q and dO rows, lse
  // and Delta.  Rows past the sequence end read as zero and get P = 0.
  const int qi = q0 + 32 * w + n;
  const int qrows = uni(min(L - q0, kDqBM));
  const size_t qbase = row_off<D, BHSD>(a, q0, h, p.hq, p.max_seqlen);
  const rsrc_t qr = make_rsrc(static_cast<const T*>(p.q) + qbase, qrows * q_row * 2);
  const rsrc_t dr = make_rsrc(static_cast<const T*>(p.dout) + qbase, qrows * q_row * 2);
  T8 qreg[D / 16], dreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint32_t off = ((32 * w + n) * q_row + 16 * ks + 8 * c) * 2;
    qreg[ks] = __builtin_bit_cast(T8, buf_load16(qr, off));
    dreg[ks] = __builtin_bit_cast(T8, buf_load16(dr, off));
  }
  float l2 = INFINITY, dlt = 0.0f;  // lse * log2(e) and Delta of query qi
  if (p.o) {
    // Delta of this lane's row from O and dO, bit for bit as the preprocess
    // forms it: dot8 per 8-element chunk, then the chunks summed in its
    // butterfly order.  Chunk j of the row sits in lane c = j % 2, slot
    // ks = j / 2, so the butterfly steps over chunk distances D/16 .. 2 stay
    // inside the lane (slot distance D/32 .. 1) and the last one, distance 1,
    // pairs the two lanes (xor 32).
    const rsrc_t orr = make_rsrc(static_cast<const T*>(p.o) + qbase, qrows * q_row * 2);
    float v[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const uint32_t off = ((32 * w + n) * q_row + 16 * ks + 8 * c) * 2;
      v[ks] = dot8(__builtin_bit_cast(T8, buf_load16(orr, off)), dreg[ks], 0.0f);
    }
#pragma unroll
    for (int hs = D / 32; hs >= 1; hs >>= 1) {
      float u[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) u[ks] = v[ks] + v[ks ^ hs];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) v[ks] = u[ks];
    }
    const float dfull = v[0] + xor32(v[0]);
    if (qi < L) {
      const size_t idx = (size_t)h * p.total + a + qi;
      l2 = p.lse[idx] * kLog2e;
      dlt = dfull;
      if (c == 0) p.delta_out[idx] = dfull;
    }
  } else if (qi < L) {
    const size_t idx = (size_t)h * p.total + a + qi;
    l2 = p.lse[idx] * kLog2e;
    dlt = p.delta[idx];
  }

  f32x16 qacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) qacc[t] = f32x16{};

  // Key range visible to any row of this workgroup.
  const int qlast = min(L, q0 + kDqBM) - 1;
  int k_lo = 0, k_hi = L;
  if (p.causal) k_hi = qlast + 1;
  if (p.window > 0) k_lo = max(0, q0 - p.window + 1);
  k_lo = (k_lo / kDqBN) * kDqBN;
  const int wq_lo = q0 + 32 * w, wq_hi = min(q0 + 32 * w + 31, L - 1);

  // Copy keys [kb, kb + 64) of K and V into stage `stage`.  Lane l of wave w
  // fills physical chunk 64 (w + 4 u) + l of the K tile followed by the V
  // tile: row P / CH, logical chunk (P % CH) ^ swz(row).  Rows past the
  // sequence end repeat its last key (finite values; masked below).
  const T* kp = static_cast<const T*>(p.k);
  const T* vp = static_cast<const T*>(p.v);
  uint32_t coff[C::NDMA];  // per-lane source offsets within a full block
#pragma unroll
  for (int u = 0; u < C::NDMA; ++u) {
    const int P = (64 * (w + kDqNW * u)) % (kDqBN * C::CH) + lane;
    const int r = P / C::CH, ch = (P % C::CH) ^ chunk_swz<D>(r);
    coff[u] = ((uint32_t)r * kv_row + 8 * ch) * 2;
  }
  // Copy u of a block fills the K tile for u < NDMA / 2 and the V tile
  // otherwise; its wave-uniform LDS address is this wave's base plus
  // constants, formed once.
  const uint32_t lds_w = lds_addr(smem) + 1024u * (uint32_t)uni(w);
  auto issue = [&](int kb, int stage) {
    const int nk = uni(min(L - kb, kDqBN));
    const size_t base = row_off<D, BHSD>(a, kb, g, p.hkv, p.max_seqlen);
    const rsrc_t kr = make_rsrc(kp + base, nk * kv_row * 2);
    const rsrc_t vr = make_rsrc(vp + base, nk * kv_row * 2);
    const uint32_t lds_s = lds_w + (uint32_t)uni(stage) * C::STAGE;
    constexpr int kHalf = C::NDMA / 2;
    if (nk == kDqBN) {
#pragma unroll
      for (int u = 0; u < C::NDMA; ++u) {
        const bool isv = u >= kHalf;
        const int uu = isv ? u - kHalf : u;
        lds_dma16(isv ? vr : kr, lds_s + (isv ? C::TILE : 0) + 1024u * kDqNW * uu, coff[u]);
      }
    } else {  // tail block: rows past the end repeat the last key
#pragma unroll
      for (int u = 0; u < C::NDMA; ++u) {
        const bool isv = u >= kHalf;
        const int uu = isv ? u - kHalf : u;
        const int P = 64 * (w + kDqNW * uu) + lane;
        const int r = P / C::CH, ch = (P % C::CH) ^ chunk_swz<D>(r);
        const uint32_t off = ((uint32_t)min(r, nk - 1) * kv_row + 8 * ch) * 2;
        lds_dma16(isv ? vr : kr, lds_s + (isv ? C::TILE : 0) + 1024u * kDqNW * uu, off);
      }
    }
  };

  issue(k_lo, 0);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  int stage = 0;
  for (int kb = k_lo; kb < k_hi; kb += kDqBN, stage ^= 1) {
    if (kb + kDqBN < k_hi) issue(kb + kDqBN, stage ^ 1);

    const bool skip = wq_lo > wq_hi || (p.causal && kb > wq_hi) ||
                      (p.window > 0 && kb + kDqBN - 1 <= wq_lo - p.window);
    if (!skip) {
      const char* kt = smem + stage * C::STAGE;
      const char* vt = kt + C::TILE;
      const int kb_last = kb + kDqBN - 1;
      bool full = (kb_last < L) && (!p.causal || kb_last <= wq_lo) &&
                  (p.window <= 0 || kb > wq_hi - p.window);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        if constexpr (WIN) {
          // Keys [h_lo, h_lo + 32): skipped when hidden from every row of
          // the wave, masked only when hidden from some.
          const int h_lo = kb + 32 * mt, h_hi = h_lo + 31;
          if (h_lo >= L || (p.causal && h_lo > wq_hi) || h_hi <= wq_lo - p.window) continue;
          full = (h_hi < L) && (!p.causal || h_hi <= wq_lo) && h_lo > wq_hi - p.window;
        }
        // S^T and dP^T for keys [kb + 32 mt, +32) against this wave's queries.
        f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int o = rm_off<D>(32 * mt + n, 16 * ks + 8 * c);
          st = mfma32(lds16<T>(kt, o), qreg[ks], st);
          dpt = mfma32(lds16<T>(vt, o), dreg[ks], dpt);
        }
        // Operand reads run ahead of the products (AHEAD reads first, then
        // product / read pairs, then the last products) instead of one
        // product ahead: 4 x 32k 6.45 -> 6.30 ms at D = 64.  At D = 128 only
        // with windows: without them the read-ahead spills (7-14 registers).
        if constexpr (D == 64 || WIN) {
          constexpr int AHEAD = D == 64 ? 3 : 2, NPROD = 2 * (D / 16);
          __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
          for (int u = 0; u < NPROD - AHEAD; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
        }
        // dS^T = P^T o (dP^T - Delta); register r holds key
        // kb + 32 mt + (r / 4) * 8 + 4 c + r % 4 of query qi.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(st[r] * p.scale_log2 - l2);
          dpt[r] = pv * (dpt[r] - dlt);
        }
        // Hidden keys -> 0 (selected, so whatever the unmasked exponent gave
        // is discarded); the empty asm keeps this a real branch.
        if (!full) {
          asm volatile("");
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kb + 32 * mt + (r >> 2) * 8 + 4 * c + (r & 3);
            dpt[r] = (j < L && visible(qi, j, p.causal, p.window)) ? dpt[r] : 0.0f;
          }
        }
        // dQ^T += K^T dS^T over these 32 keys in two 16-key steps.  Slot
        // (c, e) of step ks holds key 16 ks + (e / 4) * 8 + 4 c + e % 4 of the
        // half, where the C layout of dP^T keeps it; the transposing read of
        // the row-major K tile delivers K^T in the same order.
        if constexpr (D == 128) {
          // The transposed K operands are read kAh (key step, dim tile)
          // steps before their products, through a ring of kAh + 1 buffers;
          // the scheduling groups pin that order (the compiler otherwise
          // waited for each step's reads right before its product).
          constexpr int NS = 2 * (D / 32), kAh = 2;
          const T8 sbv[2] = {pack8<T>(dpt, 0), pack8<T>(dpt, 8)};
          T8 ka[kAh + 1];
          auto load_a = [&](int i) {
            const int ks = i / (D / 32), t = i % (D / 32);
            const int row = 32 * mt + 16 * ks + 4 * c + (l16 >> 2);
            const int col = 32 * t + 16 * g16 + 4 * (lane & 3);
            ka[i % (kAh + 1)] = tr_pair<T>(kt, rm_off<D>(row, col), rm_off<D>(row + 8, col));
          };
#pragma unroll
          for (int i = 0; i < kAh; ++i) load_a(i);
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAh, 2);
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            if (i + kAh < NS) load_a(i + kAh);
            const int t = i % (D / 32);
            qacc[t] = mfma32(ka[i % (kAh + 1)], sbv[i / (D / 32)], qacc[t]);
            if (i + kAh < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const T8 sb = pack8<T>(dpt, 8 * ks);
            const int row = 32 * mt + 16 * ks + 4 * c + (l16 >> 2);
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
              const int col = 32 * t + 16 * g16 + 4 * (lane & 3);
              qacc[t] = mfma32(tr_pair<T>(kt, rm_off<D>(row, col), rm_off<D>(row + 8, col)), sb, qacc[t]);
            }
          }
        }
      }
    }
    // The next block's copies have landed and every wave is done with this
    // stage before it is overwritten.
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
  }

  if (qi >= L) return;
  // C layout of dQ^T: register 4 rg + e of tile t = dim 32 t + 8 rg + 4 c + e.
  T* __restrict__ op = static_cast<T*>(p.dq) + row_off<D, BHSD>(a, qi, h, p.hq, p.max_seqlen);
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      T4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = to16<T>(qacc[t][4 * rg + e] * p.scale);
      st8<T>(op + 32 * t + 8 * rg + 4 * c, out);
    }
  }
}

template <typename T, int D>
hipError_t dq_t(const DqArgs& args, bool bhsd, hipStream_t stream) {
  const unsigned blocks = (unsigned)args.nqb * args.num_seqs * args.hq;
  const dim3 grid(blocks), block(kDqThreads);
  if (args.window > 0) {
    if (bhsd)
      hipLaunchKernelGGL((dq_kernel<T, D, true, true>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((dq_kernel<T, D, false, true>), grid, block, 0, stream, args);
  } else {
    if (bhsd)
      hipLaunchKernelGGL((dq_kernel<T, D, true, false>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((dq_kernel<T, D, false, false>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const Problem& p, const void* q, const void* k, const void* v,
                         const void* dout, const float* lse, const float* delta,
                         const int32_t* cu, void* dq, const void* o, float* delta_out,
                         hipStream_t stream) {
  DqArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.cu = cu;
  a.dq = dq;
  a.o = o;
  a.delta_out = delta_out;
  a.num_seqs = p.num_seqs;
  a.max_seqlen = p.max_seqlen;
  a.total = p.total;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.window = p.window;
  a.causal = p.causal;
  a.nqb = (p.max_seqlen + kDqBM - 1) / kDqBM;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  if (p.bf16)
    return p.d == 64 ? dq_t<__bf16, 64>(a, p.bhsd, stream) : dq_t<__bf16, 128>(a, p.bhsd, stream);
  return p.d == 64 ? dq_t<_Float16, 64>(a, p.bhsd, stream) : dq_t<_Float16, 128>(a, p.bhsd, stream);
}

}  // namespace attn
