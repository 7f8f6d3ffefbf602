// Attention backward main pass for grouped-query attention (key/value
// stationary), gfx950.
//
// Per (query tile, key tile) the pass recomputes S = Q K^T and
// P = exp(S * scale - lse), then forms dV += P^T dO, dP = dO V^T,
// dS = P o (dP - Delta) * scale, dK += dS^T Q and the dQ partial dS K
// (tilelang-ascend PR "GQA Sink Backward BHSD": review thread listing kernels
// k1-k5, fused here into one loop body as in its single-kernel revision).
//
// Work decomposition.  One workgroup (8 waves, two per SIMD) owns one
// (sequence, kv head g, block of 256 keys); wave w owns keys [32w, 32w + 32)
// as one 32-key MFMA tile.  The loop runs over every query head of the
// group and every query block that can see the key block under the causal /
// window masks ("pairs"): head by head in the atomic pass, query block by
// query block (from the sequence end) in the passes without dQ atomics.
//  * dK and dV of the wave's 32 keys accumulate in fp32 registers over the
//    whole loop -- every query block of every head of the group -- and are
//    written once at the end, with no atomics (tilelang PR "[GQA] Add
//    regional atomic add": review comment on accumulating dK/dV fragments
//    across the loop and writing once).
//  * dQ partials leave through fp32 atomic adds issued straight from the
//    MFMA C layout, one sweep per pair: each wave owns two 16 x 16 tiles of
//    the pair's dQ block, and one register of a tile = four query rows x 16
//    consecutive dims, four fully used 64-byte segments per wave instruction
//    (tilelang PR: one region-wide atomic per tile instead of per-element
//    loops; triton issue "atomic_add slows down attention backwards": no
//    layout conversion before the atomics, vectorised updates).
//    Device-scope fp32 atomics resolve at the memory side on this part, so
//    their bytes per FLOP (4 * BM * D per 10 * BM * BN * D) set a ceiling;
//    256 keys per workgroup halve them relative to 128.  At D = 64 the
//    atomics of a pair are issued during the next pair's tile rather than in
//    one burst, which keeps the memory-side queue fed more evenly.
//
// Data movement.  K is staged once into LDS (needed as the dQ operand); V
// (and K for D = 64) of the wave live in registers as MFMA B operands.  At
// D = 128 the register file is short: the last three V k-steps of each wave
// sit in LDS instead, and lse / Delta are copied raw into LDS rather than
// passing through registers.
// Q / dO tiles of a pair (row-major, XOR-swizzled 16-byte chunks) and their
// lse / Delta rows are double-buffered in LDS.  Right after pair i's barrier
// the Q / dO tiles of pair i + 2 are copied from memory straight into the
// buffer pair i has released (buffer loads with an LDS destination, so no
// registers are held for them); at D = 64 lse / Delta pass through
// registers.  All of them go out before the atomics of pair i, so they never
// queue behind them.
// Transposed operands (dO, Q for dV / dK; dS, K for dQ) come from gfx950's
// transposing LDS read, and dS is stored key-major with 8-byte writes.  All
// LDS patterns are bank-conflict free under the measured bank model
// (row-major swizzle in common.h, dS swizzle below).
// One workgroup barrier per pair.
//
// The sink needs no term here: it only enters through lse.
//
// Variants (template parameters): WIN for sliding windows; DQ = false drops
// the dQ product and its atomics (the dK / dV pass of the deterministic
// backward, paired with the query-stationary dQ pass in dq.hip); BHSD for
// [B, H, S, D] tensors (row and head strides swapped, see row_off); SPLIT
// divides the pair loop of every key block over nsplit workgroups, each of
// which writes its fp32 dK / dV partial to a workspace slot of its own (no
// atomics; a reduce pass sums the slots in a fixed order and casts), for
// problems whose longest key block would otherwise set the critical path.
// The dK / dV-only variants (split or not) run four waves (128 keys) per
// workgroup, two workgroups per CU (see nw_of).
#include <limits.h>

#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kKT = 1;  // 32-key MFMA tiles per wave
// Waves per workgroup: eight (two per SIMD, one workgroup per CU), except in
// the dK / dV-only passes, which run four, two workgroups per CU.
// Where only some of a key block's 32-key tiles see a query block (the
// causal diagonal; under a narrow window about five of eight on every
// pair), eight waves leave SIMDs idle at the pair's barrier while one SIMD
// holds two busy waves; two four-wave workgroups share each SIMD without a
// common barrier, so one fills the other's idle pairs, and short sequences
// get twice as many workgroups; a split part of a 128-key block also holds
// half the pairs of a 256-key part in about the same time per pair, so
// splitting shortens the critical path twice as much.  The atomic passes
// (split or not) keep 256 keys per workgroup: their atomic bytes scale with
// 1 / keys per workgroup.
constexpr int nw_of(bool dq, bool /*split*/) { return dq ? 8 : 4; }
constexpr int kNW = 8;  // the atomic pass

template <int D, int NW = kNW, bool DQ = true>
struct Cfg {
  static constexpr int THREADS = 64 * NW;
  static constexpr int BN = NW * 32 * kKT;       // keys per workgroup
  static constexpr int BM = D == 128 ? 32 : 64;  // query rows per pair
  static constexpr int MT = BM / 32;             // 32-row query tiles
  static constexpr int NT = D / 32;              // 32-wide dim tiles
  static constexpr bool KREG = D == 64;          // K of the wave also in registers
  // LDS map (bytes)
  static constexpr int K_OFF = 0;
  static constexpr int QT = BM * D * 2;
  static constexpr int Q_OFF = K_OFF + BN * D * 2;
  static constexpr int DO_OFF = Q_OFF + 2 * QT;
  static constexpr int DST = BN * BM * 2;
  static constexpr int DS_OFF = DO_OFF + 2 * QT;
  // lse / Delta rows of a pair: at D = 128 they are copied raw into LDS
  // (64 floats per buffer, one wave each); otherwise they pass through
  // registers and are stored as lse * log2(e) (+inf on rows past the end)
  // and -Delta, which then seeds the dP accumulator.
  static constexpr bool LSE_DMA = D == 128;
  // (the four-wave dK / dV-only pass has no dS tiles and leaves no room for them)
  static constexpr int LSE_OFF = DS_OFF + (DQ || NW == 8 ? 2 * DST : 0);
  static constexpr int DLT_OFF = LSE_OFF + 2 * 64 * 4;
  // The last VLDS k-steps of each wave's V operand live in LDS (16 bytes per
  // lane per step, lane-linear) instead of registers: at D = 128 the
  // register file is otherwise a dozen registers short.
  static constexpr int VLDS = D == 128 ? 3 : 0;
  static constexpr int VREG = D / 16 - VLDS;  // V k-steps held in registers
  static constexpr int V_OFF = DLT_OFF + 2 * 64 * 4;
  static constexpr int BYTES = V_OFF + VLDS * NW * 1024;
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int PF = BM * CH / THREADS;       // prefetch chunks per thread per tensor
  static constexpr int NQT = BM / 16, NDT = D / 16;  // 16x16 dQ tiles
  static_assert(!DQ || NQT * NDT == 2 * NW, "two 16x16 dQ tiles per wave");
  static_assert(PF >= 1 && BM * CH % THREADS == 0, "prefetch split");
  static_assert(BYTES * (8 / NW) <= 160 * 1024, "LDS budget (8 / NW workgroups per CU)");
  static_assert(BYTES >= 4 * (8 * THREADS + 1), "LDS holds the fused cast's list");
};

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
  float* dkv_part;  // SPLIT: fp32 partials [nsplit][2][dk-shaped]
  int nsplit;
  int lpt;  // rank the (sequence, key block) items longest first (ragged batches)
  // Fused dQ cast (causal problems, unsplit atomic pass): arrival counters
  // per (sequence, query head, query block), zeroed before the launch, and
  // the 16-bit dQ the last contributing workgroup of a block casts into.
  int* counters;
  void* dq;
};

// Number of key-block workgroups whose pair loop contains query block qb of
// a causal sequence of length L: key blocks jb with jb * BN / BM <= qb (the
// loop starts at the block's first key) and qb below the loop's end, which a
// window places at (last key of jb + W - 1) / BM + 1.  The same bounds the
// loop uses, evaluated from the query side.
__device__ __forceinline__ int cast_contributors(int qb, int L, int BM, int BN, int window) {
  const int jb_hi = (qb * BM) / BN;
  if (window <= 0) return jb_hi + 1;
  const int nqb = (L + BM - 1) / BM;
  int cnt = 0;
  for (int jb = jb_hi; jb >= 0; --jb) {
    const int kv_last = min(L, jb * BN + BN) - 1;
    if (qb >= min(nqb, (kv_last + window - 1) / BM + 1)) break;  // the end only moves down
    ++cnt;
  }
  return cnt;
}

// Longest-first order for ragged batches.  Key-block index slowest is
// longest first only when every sequence has the same length; otherwise a
// long sequence's later key blocks (still many query blocks) would start
// after every short sequence's first one and form the tail.  Every
// workgroup ranks the num_seqs * nkb (sequence, key block) items by their
// number of query blocks under the masks (ties: lower item first; empty
// items last) and takes the item of rank r.  All threads take part; it uses
// the start of LDS and ends with a barrier.  At most one item per thread
// (64 NW for NW waves), then a scan of LDS broadcasts.
template <int BM, int NW>
__device__ int lpt_item(const BwdArgs& p, int nkb, int r, char* smem) {
  constexpr int BN = NW * 32 * kKT;
  int* work = reinterpret_cast<int*>(smem);
  int* found = work + 64 * NW;
  const int n = p.num_seqs * nkb, i = threadIdx.x;
  int wi = -1;
  if (i < n) {
    const int s = i / nkb, kv0 = (i % nkb) * BN;
    int a, b;
    seq_bounds(p.cu, s, p.max_seqlen, p.total, a, b);
    const int L = b - a;
    wi = 0;
    if (kv0 < L) {
      const int ib0 = p.causal ? kv0 / BM : 0;
      int ib1 = (L + BM - 1) / BM;
      if (p.window > 0) ib1 = min(ib1, (min(L, kv0 + BN) - 1 + p.window - 1) / BM + 1);
      wi = ib1 - ib0;
    }
    work[i] = wi;
  }
  __syncthreads();
  if (i < n) {
    int rank = 0;
    for (int k = 0; k < n; ++k) {
      const int wk = work[k];
      rank += (wk > wi) | ((wk == wi) & (k < i));
    }
    if (rank == r) found[0] = i;
  }
  __syncthreads();
  const int item = found[0];
  __syncthreads();
  return item;
}

// Scheduling groups for the S / dP products of one pair (D = 128, dK / dV
// only): the operand reads of k-step ks + AH (K, Q, dO, and V where that
// k-step is held in LDS) go out before the two products of k-step ks.
template <int NKS, int VREG, int AH, int KS = 0>
__device__ __forceinline__ void sdp_groups() {
  if constexpr (KS == 0) {
    constexpr int pre = 3 * AH + (AH > VREG ? AH - VREG : 0);
    __builtin_amdgcn_sched_group_barrier(0x100, pre, 1);
  }
  if constexpr (KS < NKS) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
    if constexpr (KS + AH < NKS)
      __builtin_amdgcn_sched_group_barrier(0x100, 3 + (KS + AH >= VREG ? 1 : 0), 1);
    sdp_groups<NKS, VREG, AH, KS + 1>();
  }
}

// Key-major dS tile (BM queries per row): 8-byte slot s of row r lives at
// slot s ^ slot_swz(r).  The 8-byte stores resolve 16 lanes (16 consecutive
// rows) at a time over 32 banks, so slot_swz is a bijection on the low row
// bits; the transposing reads need its top two bits to separate rows r,
// r + 2, r + 8 and r + 10 (both measured on MI355X).
template <int BM>
__device__ __forceinline__ int slot_swz(int r) {
  return BM == 32 ? ((((r >> 3) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 1) & 1))
                  : ((((r >> 3) & 1) << 3) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | (r & 1));
}
template <int BM>
__device__ __forceinline__ int dst_off(int r, int q) {  // q: multiple of 4
  return r * (BM * 2) + (((q >> 2) ^ slot_swz<BM>(r)) << 3);
}

// WIN: sliding-window problems, where most key tiles of a query block are
// invisible; the dQ product then runs only over the visible key tiles.
// DQ: false builds the pass without its dQ product (dK / dV only, for use
// with the query-stationary dQ pass): no dS tile in LDS, no atomics.
// BHSD: [B, H, S, D] tensors instead of packed [T, H, D].
// SPLIT: pairs of a key block split over p.nsplit workgroups (see above).
// CAST: the fused dQ cast epilogue (p.counters, p.dq; causal, unsplit, packed).
template <typename T, int D, bool WIN, bool DQ, bool BHSD, bool SPLIT, bool CAST = false>
__global__ __launch_bounds__(64 * nw_of(DQ, SPLIT), 8 / nw_of(DQ, SPLIT)) void bwd_kernel(BwdArgs p) {
  constexpr int NW = nw_of(DQ, SPLIT);
  using C = Cfg<D, NW, DQ>;
  constexpr int kThreads = C::THREADS, kBN = C::BN;
  using T8 = typename V8<T>::type;
  using T4 = typename V8<T>::half_type;
  constexpr int BM = C::BM, MT = C::MT, NT = C::NT;
  __shared__ __attribute__((aligned(16))) char smem[C::BYTES];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n = lane & 31, c = lane >> 5;
  const int l16 = lane & 15, g16 = (lane >> 4) & 1;

  // Key-block index slowest: every (sequence, kv head) starts with its
  // largest causal workload, and the blocks of one (sequence, kv head) stay
  // a multiple of 8 apart whenever num_seqs * Hkv is (same XCD and L2).
  // With SPLIT the part index sits between the key block and (seq, kv head).
  // Ragged batches rank their (sequence, key block) items instead (lpt_item);
  // the kv head stays fastest, so with Hkv a multiple of 8 kv head g runs on
  // XCD g either way.
  const int nsg = p.num_seqs * p.hkv;
  int jb, s, g, part = 0;
  if (p.lpt) {
    const int nkb = (p.max_seqlen + kBN - 1) / kBN;
    const int r = blockIdx.x / (p.hkv * (SPLIT ? p.nsplit : 1));
    if constexpr (SPLIT) part = (blockIdx.x / p.hkv) % p.nsplit;
    g = blockIdx.x % p.hkv;
    const int item = uni(lpt_item<BM, NW>(p, nkb, r, smem));
    s = item / nkb;
    jb = item % nkb;
  } else {
    int rem;
    if constexpr (SPLIT) {
      jb = blockIdx.x / (nsg * p.nsplit);
      const int r2 = blockIdx.x % (nsg * p.nsplit);
      part = r2 / nsg;
      rem = r2 % nsg;
    } else {
      jb = blockIdx.x / nsg;
      rem = blockIdx.x % nsg;
    }
    s = rem / p.hkv;
    g = rem % p.hkv;
  }
  int a, b;
  seq_bounds(p.cu, s, p.max_seqlen, p.total, a, b);
  const int L = b - a;
  const int kv0 = jb * kBN;
  if (kv0 >= L) return;
  const int G = p.hq / p.hkv;
  const uint32_t kv_row = BHSD ? (uint32_t)D : (uint32_t)p.hkv * D;  // elements between key rows
  const uint32_t q_row = BHSD ? (uint32_t)D : (uint32_t)p.hq * D;     // elements between query rows
  const int nkeys = uni(min(L - kv0, kBN));     // valid keys of this block

  // Buffer resources over this block's keys: rows past the sequence end read
  // as zero and their stores are dropped.
  const size_t kv_base = row_off<D, BHSD>(a, kv0, g, p.hkv, p.max_seqlen);
  const rsrc_t kr = make_rsrc(static_cast<const T*>(p.k) + kv_base, nkeys * kv_row * 2);
  const rsrc_t vr = make_rsrc(static_cast<const T*>(p.v) + kv_base, nkeys * kv_row * 2);

  // ---- K block into LDS (the dQ operand, and the S operand at D = 128) -------
  if constexpr (DQ || !C::KREG) {
#pragma unroll 4
    for (int u = tid; u < kBN * C::CH; u += kThreads) {
      const int r = u / C::CH, ch = u % C::CH;
      *reinterpret_cast<u32x4*>(smem + C::K_OFF + rm_off<D>(r, 8 * ch)) =
          buf_load16(kr, (r * kv_row + 8 * ch) * 2);
    }
  }
  // LDS address of the tile buffers (direct-to-LDS copies) and this wave's index, formed once.
  const uint32_t lds0 = lds_addr(smem);
  const int wu = uni(w);
  // ---- V (and K for D = 64) of this wave's keys as MFMA B operands ---------
  T8 vreg[kKT][C::VREG];
  T8 kreg[C::KREG ? kKT : 1][C::KREG ? D / 16 : 1];
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt) {
    const uint32_t row = 32 * kKT * w + 32 * kt + n;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const uint32_t off = (row * kv_row + 16 * ks + 8 * c) * 2;
      if (ks < C::VREG)
        vreg[kt][ks] = __builtin_bit_cast(T8, buf_load16(vr, off));
      else
        lds_dma16(vr, lds0 + C::V_OFF + ((kt * C::VLDS + ks - C::VREG) * NW + wu) * 1024, off);
      if constexpr (C::KREG) kreg[kt][ks] = __builtin_bit_cast(T8, buf_load16(kr, off));
    }
  }

  f32x16 dk[kKT][NT], dv[kKT][NT];
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      dk[kt][t] = f32x16{};
      dv[kt][t] = f32x16{};
    }

  // ---- pairs: (query head of the group) x (query blocks that see the keys)
  const int kv_last = kv0 + nkeys - 1;
  const int ib0 = p.causal ? kv0 / BM : 0;
  int ib1 = (L + BM - 1) / BM;
  if (p.window > 0) ib1 = min(ib1, (kv_last + p.window - 1) / BM + 1);
  const int nq = ib1 - ib0;
  const int npairs = G * nq;
  // This workgroup's pairs: i_lo + [0, np), all of them or part `part` of
  // nsplit (possibly none).  The loop counts from zero in either case.
  int i_lo = 0, np = npairs;
  if constexpr (SPLIT) {
    i_lo = (int)((long long)part * npairs / p.nsplit);
    np = (int)((long long)(part + 1) * npairs / p.nsplit) - i_lo;
  }
  const int wk_lo = kv0 + 32 * kKT * w;

  // Prefetch: Q / dO of a pair go straight into LDS (buffer_load ... lds);
  // lse / Delta too at D = 128, through registers otherwise.
  float plse = 0.0f, pdlt = 0.0f;
  int prows = 0;
  // Pair i = (query head g G + hi, query block ib0 + qi).  The atomic pass
  // walks head by head, i = hi nq + qi.  The passes without dQ atomics walk
  // query blocks from the sequence end down, every head of a block in turn,
  // i = (nq - 1 - qi) G + hi: all key blocks of a (sequence, kv head) start
  // at the same query block, and those running on one XCD then read the same
  // Q / dO tiles at about the same time, so one L2 serves them (in the atomic
  // pass that order would aim their atomics at the same rows at once).
  // The loop steps (hi, qi) instead of dividing (a runtime integer division
  // costs dozens of scalar instructions, twice per pair).
  constexpr bool QMAJOR = !DQ;
  struct PairPos {
    int hi, qi;
  };
  auto step_pos = [&](PairPos& pp) {
    if constexpr (QMAJOR) {
      if (++pp.hi == G) {
        pp.hi = 0;
        --pp.qi;
      }
    } else if (++pp.qi == nq) {
      pp.qi = 0;
      ++pp.hi;
    }
  };
  auto load_pair = [&](PairPos pp, int buf) {
    const int h = g * G + pp.hi;
    const int q0 = (ib0 + pp.qi) * BM;
    const int rows = uni(min(L - q0, BM));  // >= 1: query blocks start inside the sequence
    const size_t qb = row_off<D, BHSD>(a, q0, h, p.hq, p.max_seqlen);
    const rsrc_t qr = make_rsrc(static_cast<const T*>(p.q) + qb, rows * q_row * 2);
    const rsrc_t dr = make_rsrc(static_cast<const T*>(p.dout) + qb, rows * q_row * 2);
#pragma unroll
    for (int u = 0; u < C::PF; ++u) {
      // Lane l of wave w fills physical chunk P = 64 (w + NW u) + l of the
      // swizzled tile, i.e. row P / CH, logical chunk (P % CH) ^ swz(row).
      // Rows past the sequence end repeat the last row; P = dS = 0 there
      // whatever Q / dO hold (their lse is stored as +inf, or, when lse is
      // copied raw, the edge-tile pass masks them).
      const int P0 = 64 * (wu + NW * u);  // wave-uniform
      const int P = P0 + lane;
      const int r = P / C::CH, ch = (P % C::CH) ^ chunk_swz<D>(r);
      const uint32_t off = ((uint32_t)min(r, rows - 1) * q_row + 8 * ch) * 2;
      const uint32_t lds = lds0 + (uint32_t)(buf * C::QT + 16 * P0);
      lds_dma16(qr, lds + C::Q_OFF, off);
      lds_dma16(dr, lds + C::DO_OFF, off);
    }
    // lse / Delta of the pair's rows.
    if constexpr (C::LSE_DMA) {
      // Waves 0 and 1 copy 64 floats each (lanes past the rows read out of
      // range); rows past the sequence end are masked in the edge-tile pass.
      const size_t idx = (size_t)h * p.total + a + q0;
      if (wu < 2)
        lds_dma4(make_rsrc((wu == 0 ? p.lse : p.delta) + idx, rows * 4),
                 lds0 + (wu == 0 ? C::LSE_OFF : C::DLT_OFF) + buf * 256, lane_here() * 4);
    } else {
      // every thread issues the loads (threads past the block read out of
      // range, i.e. zero) so the number of outstanding memory operations is
      // the same in every lane.
      const size_t idx = (size_t)h * p.total + a + q0;
      const uint32_t off = (uint32_t)(tid & (BM - 1)) * 4 + (tid < BM ? 0u : 0x40000000u);
      plse = buf_load_f32(make_rsrc(p.lse + idx, rows * 4), off);
      pdlt = buf_load_f32(make_rsrc(p.delta + idx, rows * 4), off);
      prows = rows;
    }
  };
  auto store_pair = [&](int buf) {
    if (!C::LSE_DMA && tid < BM) {
      // rows outside the sequence (or that saw nothing) get P = 0
      const float l2 = (tid >= prows || plse == -INFINITY) ? INFINITY : plse * kLog2e;
      reinterpret_cast<float*>(smem + C::LSE_OFF)[buf * 64 + tid] = l2;
      reinterpret_cast<float*>(smem + C::DLT_OFF)[buf * 64 + tid] = -pdlt;
    }
  };

  // Positions of the pair being computed and of the pair two ahead (the one
  // whose copies go out after this pair's barrier).
  PairPos cur = QMAJOR ? PairPos{i_lo % G, nq - 1 - i_lo / G} : PairPos{i_lo / nq, i_lo % nq};
  PairPos ahead = cur;
  if (!SPLIT || np > 0) {  // workgroup-uniform; unsplit blocks always have pairs
    load_pair(ahead, 0);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    store_pair(0);
    step_pos(ahead);
    if (np > 1) load_pair(ahead, 1);
    step_pos(ahead);
    __syncthreads();
  }

  // dQ tiles of this wave (16x16x32 MFMA): query tile dq_qt, dim tiles dq_dt
  // and dq_dt + 1.  C layout: lane l holds dim l % 16 of rows 4 (l / 16) + r.
  const int dq_qt = (2 * w) / C::NDT, dq_dt = (2 * w) % C::NDT;
  const int g64 = lane >> 4;  // 16-lane group = k-slot group of the 16x16x32 operands
  const uint32_t dq_lane_off = ((16 * dq_qt + 4 * g64) * q_row + 16 * dq_dt + l16) * 4;

  // D = 64: the atomics of pair i leave during the tile of pair i + 1 (half
  // after its S / dP products, half after the exponentials) instead of as
  // one burst after the dQ product.
  constexpr bool TRICKLE = DQ && D == 64 && !WIN;
  f32x4 pend0 = f32x4{}, pend1 = f32x4{};
  rsrc_t pend_r = make_rsrc(p.dq_accum, 0);
  auto flush = [&](int lo, int hi) {
#pragma unroll
    for (int r = lo; r < hi; ++r) {
      buf_atomic_add(pend_r, dq_lane_off + r * q_row * 4, pend0[r]);
      buf_atomic_add(pend_r, dq_lane_off + r * q_row * 4 + 64, pend1[r]);
    }
  };

  for (int j = 0; j < np; ++j, step_pos(cur)) {
    const int buf = j & 1;
    const int h = g * G + cur.hi;
    const int q0 = (ib0 + cur.qi) * BM;
    const char* qs = smem + C::Q_OFF + buf * C::QT;
    const char* dos = smem + C::DO_OFF + buf * C::QT;
    char* dss = smem + C::DS_OFF + buf * C::DST;
    const float* lse2 = reinterpret_cast<const float*>(smem + C::LSE_OFF) + buf * 64;
    const float* dlt = reinterpret_cast<const float*>(smem + C::DLT_OFF) + buf * 64;

#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
      // Keys [tk_lo, tk_lo + 32) of this wave's tile kt against queries [q0, q0 + BM).
      const int tk_lo = wk_lo + 32 * kt, tk_hi = tk_lo + 31;
      // Every path through the tile issues all 8 pending atomics of the
      // previous pair (the barrier's wait count relies on it).  On the first
      // pair they hold zeros aimed at an empty range and are dropped; issuing
      // them anyway keeps the products and the exponentials in one block.
      if constexpr (TRICKLE) {
        if (kt == 0) flush(0, 2);
      }
      const bool empty = tk_lo >= L || q0 >= L || (p.causal && tk_lo > q0 + BM - 1) ||
                         (p.window > 0 && tk_hi <= q0 - p.window);
      if (empty) {
        if constexpr (TRICKLE) {
          if (kt == 0) flush(2, 4);
        }
        // With WIN the dQ product below skips exactly the key tiles that no
        // query of the block can see, so their dS rows are never read;
        // otherwise they are zeroed.
        if constexpr (DQ && !WIN) {
          const u32x2 z = {0u, 0u};
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              *reinterpret_cast<u32x2*>(dss + dst_off<BM>(32 * kKT * w + 32 * kt + n, 32 * mt + 8 * g4 + 4 * c)) = z;
        }
        continue;
      }
      // -- S = Q K^T and dP = dO V^T: [BM queries] x [32 keys]
      // With -Delta in LDS (register path) the dP accumulator starts from it,
      // so the products leave dP - Delta without a subtraction per element.
      // Register 4 g4 + e of a tile holds query row 32 mt + 8 g4 + 4 c + e.
      f32x16 sacc[MT], pacc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        sacc[mt] = f32x16{};
        if constexpr (C::LSE_DMA) {
          pacc[mt] = f32x16{};
        } else {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 nd = *reinterpret_cast<const f32x4*>(dlt + 32 * mt + 8 * g4 + 4 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) pacc[mt][4 * g4 + e] = nd[e];
          }
        }
      }
      auto prod_step = [&](int mt, int ks) {
        T8 kb;
        if constexpr (C::KREG)
          kb = kreg[kt][ks];
        else
          kb = lds16<T>(smem, C::K_OFF + rm_off<D>(32 * kKT * w + 32 * kt + n, 16 * ks + 8 * c));
        const int o = rm_off<D>(32 * mt + n, 16 * ks + 8 * c);
        sacc[mt] = mfma32(lds16<T>(qs, o), kb, sacc[mt]);
        const T8 vb = ks < C::VREG
                          ? vreg[kt][ks]
                          : lds16<T>(smem, C::V_OFF + ((kt * C::VLDS + ks - C::VREG) * NW + w) * 1024 + 16 * lane);
        pacc[mt] = mfma32(lds16<T>(dos, o), vb, pacc[mt]);
      };
      // -- P = exp2(S scale log2e - lse log2e); dS' = P (dP - Delta) for the
      //    four rows of group g4 of query tile mt.  The factor `scale` of dS
      //    is applied once to dK (epilogue) and to dQ (postprocess), not per
      //    element.
      auto expq = [&](int mt, int g4) {
        const int qr = 32 * mt + 8 * g4 + 4 * c;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + qr);
        f32x4 d4 = {0.f, 0.f, 0.f, 0.f};  // Delta still to subtract (raw copies only)
        if constexpr (C::LSE_DMA) d4 = *reinterpret_cast<const f32x4*>(dlt + qr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          const float l2 = C::LSE_DMA ? l4[e] * kLog2e : l4[e];
          const float pv = fast_exp2(sacc[mt][r] * p.scale_log2 - l2);
          sacc[mt][r] = pv;
          pacc[mt][r] = C::LSE_DMA ? pv * (pacc[mt][r] - d4[e]) : pv * pacc[mt][r];
        }
      };
      if constexpr (MT == 2) {
        // Two query tiles (D = 64): the second tile's S / dP products run
        // under the first tile's exponentials (an LDS-read-only scheduling
        // barrier per k-step keeps them interleaved), with the wave at raised
        // priority from there to the dV / dK products, so the two waves
        // sharing a SIMD also drift apart and one's matrix work overlaps the
        // other's exponentials.  Measured on the dK / dV-only pass: 4-7 %
        // faster than the products of both tiles first (atomic pass
        // unchanged, atomic-bound).  Interleaving the second tile's
        // exponentials with the first tile's dV / dK products as well was
        // slower, at both head dims.
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) prod_step(0, ks);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          prod_step(1, ks);
          expq(0, ks);
          __builtin_amdgcn_sched_barrier(0x100);
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) expq(1, g4);
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) prod_step(mt, ks);
        if constexpr (D == 128 && !DQ) sdp_groups<D / 16, C::VREG, 1>();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) expq(mt, g4);
      }
      if constexpr (TRICKLE) {
        if (kt == 0) {
          __builtin_amdgcn_sched_barrier(0);
          flush(2, 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // Edge tiles: zero P and dS where the key is hidden (visible iff
      // lo <= q - k <= hi, k < L and q < L).  Selecting (not multiplying)
      // discards whatever the unmasked exponent produced there.  The empty asm
      // keeps this a real branch: if-converted, its compares and selects would
      // run on every tile.
      const bool full = (q0 + BM <= L) && (tk_hi < L) && (!p.causal || tk_hi <= q0) &&
                        (p.window <= 0 || tk_lo > q0 + BM - 1 - p.window);
      if (!full) {
        asm volatile("");
        const int kj = tk_lo + n;
        const int dlo = p.causal ? 0 : INT_MIN;
        const int dhi = p.window > 0 ? p.window - 1 : INT_MAX;
        const int kin = kj < L ? 1 : 0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = q0 + 32 * mt + 8 * (r >> 2) + 4 * c + (r & 3);
            const int dd = q - kj;
            const bool vis = kin & (q < L) & (dd >= dlo) & (dd <= dhi);
            sacc[mt][r] = vis ? sacc[mt][r] : 0.0f;
            pacc[mt][r] = vis ? pacc[mt][r] : 0.0f;
          }
      }

      if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
      // -- dV += P^T dO, dK += dS^T Q over the BM queries (16 per step).
      // Slot (c, e) of step qs holds query 16 qs + (e / 4) * 8 + 4 c + e % 4,
      // where the C layout of S keeps it; the B operands are read transposed.
      if constexpr (D == 128 && !DQ) {
        // The (query step, dim tile) steps' transposed operands are read
        // kAhead steps before their products, through a ring of kAhead + 1
        // buffers per tensor; the scheduling groups pin that order (left to
        // itself the compiler issued each step's reads right before its
        // products and waited for them there, one LDS round trip per step).
        // Only in the dK / dV-only pass: with the dQ product's registers
        // live the ring spills, and that pass is bound by its atomics.
        constexpr int NS = (BM / 16) * NT, kAhead = 2;
        T8 pa[BM / 16], sa[BM / 16];
#pragma unroll
        for (int qs2 = 0; qs2 < BM / 16; ++qs2) {
          pa[qs2] = pack8<T>(sacc[qs2 >> 1], 8 * (qs2 & 1));
          sa[qs2] = pack8<T>(pacc[qs2 >> 1], 8 * (qs2 & 1));
        }
        T8 bo[kAhead + 1], bq[kAhead + 1];
        auto load_b = [&](int i) {
          const int qs2 = i / NT, t = i % NT;
          const int row = 16 * qs2 + 4 * c + (l16 >> 2);
          const int col = 32 * t + 16 * g16 + 4 * (lane & 3);
          const int o0 = rm_off<D>(row, col), o1 = rm_off<D>(row + 8, col);
          bo[i % (kAhead + 1)] = tr_pair<T>(dos, o0, o1);
          bq[i % (kAhead + 1)] = tr_pair<T>(qs, o0, o1);
        };
#pragma unroll
        for (int i = 0; i < kAhead; ++i) load_b(i);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * kAhead, 0);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          if (i + kAhead < NS) load_b(i + kAhead);
          const int qs2 = i / NT, t = i % NT;
          dv[kt][t] = mfma32(pa[qs2], bo[i % (kAhead + 1)], dv[kt][t]);
          dk[kt][t] = mfma32(sa[qs2], bq[i % (kAhead + 1)], dk[kt][t]);
          if (i + kAhead < NS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
      } else {
#pragma unroll
        for (int qs2 = 0; qs2 < BM / 16; ++qs2) {
          const int mt = qs2 >> 1, rb = 8 * (qs2 & 1);
          const T8 pa = pack8<T>(sacc[mt], rb);
          const T8 sa = pack8<T>(pacc[mt], rb);
          const int row = 16 * qs2 + 4 * c + (l16 >> 2);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int col = 32 * t + 16 * g16 + 4 * (lane & 3);
            const int o0 = rm_off<D>(row, col), o1 = rm_off<D>(row + 8, col);
            dv[kt][t] = mfma32(pa, tr_pair<T>(dos, o0, o1), dv[kt][t]);
            dk[kt][t] = mfma32(sa, tr_pair<T>(qs, o0, o1), dk[kt][t]);
          }
        }
      }

      // -- dS to LDS, key-major: 4 consecutive queries per 8-byte write.
      if constexpr (DQ) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            T4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = to16<T>(pacc[mt][4 * g4 + e]);
            *reinterpret_cast<u32x2*>(dss + dst_off<BM>(32 * kKT * w + 32 * kt + n, 32 * mt + 8 * g4 + 4 * c)) =
                __builtin_bit_cast(u32x2, v4);
          }
      }
    }

    // -- next pair's lse / Delta into the other buffer (register path); the
    //    copies for the pair after it go out before this pair's atomics.
    if (j + 1 < np) store_pair(buf ^ 1);
    // The copies for pair i + 1 must have landed: after them this wave
    // issued the two lse / Delta register loads (unless those are copies
    // too) and, except on the first pair, the 8 atomics of pair i - 1
    // (memory operations complete in order).
    {
      constexpr int after = C::LSE_DMA ? 0 : 2;
      if (j == 0 || !DQ)
        __builtin_amdgcn_s_waitcnt(kVmcnt0 + after);
      else
        __builtin_amdgcn_s_waitcnt(kVmcnt0 + after + 8);
    }
    __syncthreads();
    if (j + 2 < np) {
      load_pair(ahead, buf);
      step_pos(ahead);
    }

    if constexpr (DQ) {
      // -- dQ partial = dS K for this wave's two 16 x 16 tiles.  Slot (g, e)
      //    of the 16x16x32 operands holds key 32 ks + 8 g + e; k-step ks covers
      //    the keys of wave ks.  With WIN only the key tiles some query of the
      //    block can see are visited (exactly the tiles not "empty" above).
      f32x4 qacc0 = f32x4{}, qacc1 = f32x4{};
      {
        int ks_lo = 0, ks_hi = kBN / 32;
        if constexpr (WIN) {
          ks_hi = min(ks_hi, (nkeys + 31) / 32);
          ks_hi = min(ks_hi, (q0 + BM - 1 - kv0) / 32 + 1);  // windows are causal
          // tile ks is visible iff 32 ks + 31 > q0 - W - kv0, i.e.
          // ks >= floor((q0 - W + 1 - kv0) / 32) (arithmetic shift = floor).
          ks_lo = max(0, (q0 - p.window + 1 - kv0) >> 5);
        }
        const int qcol = 16 * dq_qt + 4 * (lane & 3);
        const int dcol = 16 * dq_dt + 4 * (lane & 3);
        auto step = [&](int ks) {
          const int key = 32 * ks + 8 * g64 + (l16 >> 2);
          const T8 as = tr_pair<T>(dss, dst_off<BM>(key, qcol), dst_off<BM>(key + 4, qcol));
          const T8 b0 = tr_pair<T>(smem, C::K_OFF + rm_off<D>(key, dcol),
                                   C::K_OFF + rm_off<D>(key + 4, dcol));
          const T8 b1 = tr_pair<T>(smem, C::K_OFF + rm_off<D>(key, dcol + 16),
                                   C::K_OFF + rm_off<D>(key + 4, dcol + 16));
          qacc0 = mfma16(as, b0, qacc0);
          qacc1 = mfma16(as, b1, qacc1);
        };
        // Full unrolling fits the register budget only at D = 64; elsewhere
        // the loop stays rolled (the compiler's own partial unrolling of it
        // costs registers the pair loop does not have).
        if constexpr (WIN || D == 128) {
#pragma unroll 1
          for (int ks = ks_lo; ks < ks_hi; ++ks) step(ks);
        } else {
#pragma unroll
          for (int ks = 0; ks < kBN / 32; ++ks) step(ks);
        }
      }
      // -- region-wide fp32 atomics straight from the C layout; rows past the
      //    sequence end fall outside the resource and are dropped.
      {
        const int rows = uni(min(L - q0, BM));
        const rsrc_t dq = make_rsrc(p.dq_accum + row_off<D, BHSD>(a, q0, h, p.hq, p.max_seqlen),
                                    rows * q_row * 4);
        if constexpr (TRICKLE) {
          pend0 = qacc0;
          pend1 = qacc1;
          pend_r = dq;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            buf_atomic_add(dq, dq_lane_off + r * q_row * 4, qacc0[r]);
            buf_atomic_add(dq, dq_lane_off + r * q_row * 4 + 64, qacc1[r]);
          }
        }
      }
    }
  }
  if constexpr (TRICKLE) flush(0, 4);

  // ---- single write of dK and dV (C layout: column = dim, row = key) -------
  if constexpr (SPLIT) {
    // fp32 partials into slot `part` (dK already scaled); rows past the
    // sequence end fall outside the resource and are dropped.
    const size_t n_kv = (size_t)p.total * p.hkv * D;
    float* slot = p.dkv_part + (size_t)part * 2 * n_kv + kv_base;
    const rsrc_t pkr = make_rsrc(slot, nkeys * kv_row * 4);
    const rsrc_t pvr = make_rsrc(slot + n_kv, nkeys * kv_row * 4);
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t row = 32 * kKT * w + 32 * kt + (r >> 2) * 8 + 4 * c + (r & 3);
          const uint32_t off = (row * kv_row + 32 * t + n) * 4;
          buf_store_f32(pkr, off, dk[kt][t][r] * p.scale);
          buf_store_f32(pvr, off, dv[kt][t][r]);
        }
    return;
  }
  const rsrc_t dkr = make_rsrc(static_cast<T*>(p.dk) + kv_base, nkeys * kv_row * 2);
  const rsrc_t dvr = make_rsrc(static_cast<T*>(p.dv) + kv_base, nkeys * kv_row * 2);
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t row = 32 * kKT * w + 32 * kt + (r >> 2) * 8 + 4 * c + (r & 3);
        const uint32_t off = (row * kv_row + 32 * t + n) * 2;
        buf_store_b16(dkr, off, bits16(to16<T>(dk[kt][t][r] * p.scale)));
        buf_store_b16(dvr, off, bits16(to16<T>(dv[kt][t][r])));
      }

  // ---- fused dQ cast (causal problems): count this workgroup's arrival at
  // every (query head, query block) it sent atomics to, once all of them are
  // performed; the last contributor of a block casts it.  Workgroup-uniform.
  if constexpr (CAST) {
    {
      // Release at device scope (wait for this thread's atomics, write back
      // L2), not __threadfence(): its acquire half would invalidate this
      // XCD's whole L2 at every workgroup end and throw away the other CUs'
      // cached Q / dO (measured: +8 % on the long causal problems).
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();  // ... for every thread of the workgroup
      // The thread index from values the pair loop keeps live anyway (keeping
      // threadIdx.x live across the loop costs the loop a register).
      const int ti = (wu << 6) + lane;
      int* count = reinterpret_cast<int*>(smem);  // the pair loop is done with LDS
      int* list = count + 1;
      constexpr int kPer = 8;  // counter atomics in flight per thread
      const int nqb_max = (p.max_seqlen + BM - 1) / BM;
      for (int base = 0; base < npairs; base += kPer * kThreads) {
        if (ti == 0) *count = 0;
        __syncthreads();
        int old[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int i = base + u * kThreads + ti;
          old[u] = -1;
          if (i < npairs) {
            const int hh = g * G + i / nq, qb = ib0 + i % nq;
            old[u] = atomicAdd(p.counters + ((size_t)s * p.hq + hh) * nqb_max + qb, 1);
          }
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int i = base + u * kThreads + ti;
          if (i < npairs && old[u] + 1 == cast_contributors(ib0 + i % nq, L, BM, kBN, p.window))
            list[atomicAdd(count, 1)] = i;
        }
        __syncthreads();
        const int ncast = *count;
        if (ncast > 0) {
          // Every listed block's BM x D elements as one flat range.  The
          // loads are device-coherent (agent-scope atomic loads skip the
          // caches that other XCDs' atomics bypass), issued after the counter
          // that saw every contributor's release.
          constexpr int kTile = BM * (D / 4);
#pragma unroll 4
          for (int e = ti; e < ncast * kTile; e += kThreads) {
            const int it = list[e / kTile], r = (e % kTile) / (D / 4), c4 = e % (D / 4);
            const int hh = g * G + it / nq, q = (ib0 + it % nq) * BM + r;
            if (q < L) {  // rows past the sequence end of its last block
              const size_t off = row_off<D, BHSD>(a, q, hh, p.hq, p.max_seqlen) + 4 * c4;
              T4 o4;
#pragma unroll
              for (int u = 0; u < 4; ++u)
                o4[u] = to16<T>(__hip_atomic_load(p.dq_accum + off + u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT) * p.scale);
              st8<T>(static_cast<T*>(p.dq) + off, o4);
            }
          }
        }
        __syncthreads();  // the list is rewritten next round
      }
    }
  }
}

template <typename T, int D, bool DQ, bool BHSD>
hipError_t bwd_t2(const BwdArgs& args, unsigned blocks, int threads, hipStream_t stream) {
  const dim3 grid(blocks), block(threads);
  if constexpr (DQ && !BHSD) {
    if (args.counters) {
      if (args.window > 0)
        hipLaunchKernelGGL((bwd_kernel<T, D, true, true, false, false, true>), grid, block, 0,
                           stream, args);
      else
        hipLaunchKernelGGL((bwd_kernel<T, D, false, true, false, false, true>), grid, block, 0,
                           stream, args);
      return hipGetLastError();
    }
  }
  if (args.counters) return hipErrorInvalidValue;  // no fused cast for this variant
  // The split kernel is built without the window specialisation (it is
  // still correct for windows, whose key blocks are short anyway).
  if (args.dkv_part)
    hipLaunchKernelGGL((bwd_kernel<T, D, false, DQ, BHSD, true>), grid, block, 0, stream, args);
  else if (args.window > 0)
    hipLaunchKernelGGL((bwd_kernel<T, D, true, DQ, BHSD, false>), grid, block, 0, stream, args);
  else
    hipLaunchKernelGGL((bwd_kernel<T, D, false, DQ, BHSD, false>), grid, block, 0, stream, args);
  return hipGetLastError();
}

template <typename T, int D, bool DQ>
hipError_t bwd_t(const BwdArgs& args, int nkb, int threads, bool bhsd, hipStream_t stream) {
  const unsigned blocks = (unsigned)nkb * args.num_seqs * args.hkv * (unsigned)args.nsplit;
  return bhsd ? bwd_t2<T, D, DQ, true>(args, blocks, threads, stream)
              : bwd_t2<T, D, DQ, false>(args, blocks, threads, stream);
}

template <bool DQ>
hipError_t bwd_dispatch(const Problem& p, const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, const float* delta,
                        const int32_t* cu, float* dq_accum, void* dk, void* dv,
                        float* dkv_part, int nsplit, hipStream_t stream,
                        int* counters = nullptr, void* dq = nullptr) {
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
  a.dkv_part = dkv_part;
  a.nsplit = nsplit;
  a.counters = counters;
  a.dq = dq;
  // The variant bwd_t2 picks fixes the workgroup: nw_of waves, 32 keys each.
  const int nw = nw_of(DQ, dkv_part != nullptr);
  const int bn = nw * 32 * kKT;
  const int nkb = (p.max_seqlen + bn - 1) / bn;
  // Packed sequences of unknown (device-side) lengths are ranked in the
  // kernel (one item per thread at most); a dense batch's formula order is
  // already longest first.
  a.lpt = (cu != nullptr && p.num_seqs > 1 && (long long)p.num_seqs * nkb <= 64LL * nw) ? 1 : 0;
  if (p.bf16)
    return p.d == 64 ? bwd_t<__bf16, 64, DQ>(a, nkb, 64 * nw, p.bhsd, stream)
                     : bwd_t<__bf16, 128, DQ>(a, nkb, 64 * nw, p.bhsd, stream);
  return p.d == 64 ? bwd_t<_Float16, 64, DQ>(a, nkb, 64 * nw, p.bhsd, stream)
                   : bwd_t<_Float16, 128, DQ>(a, nkb, 64 * nw, p.bhsd, stream);
}

}  // namespace

hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const void* dout, const float* lse, const float* delta,
                      const int32_t* cu, float* dq_accum, void* dk, void* dv,
                      hipStream_t stream) {
  return bwd_dispatch<true>(p, q, k, v, dout, lse, delta, cu, dq_accum, dk, dv, nullptr, 1, stream);
}

hipError_t launch_bwd_fused_cast(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dout, const float* lse, const float* delta,
                                const int32_t* cu, float* dq_accum, int* counters, void* dq,
                                void* dk, void* dv, hipStream_t stream) {
  return bwd_dispatch<true>(p, q, k, v, dout, lse, delta, cu, dq_accum, dk, dv, nullptr, 1, stream,
                            counters, dq);
}

hipError_t launch_bwd_dkdv(const Problem& p, const void* q, const void* k, const void* v,
                           const void* dout, const float* lse, const float* delta,
                           const int32_t* cu, void* dk, void* dv, hipStream_t stream) {
  return bwd_dispatch<false>(p, q, k, v, dout, lse, delta, cu, nullptr, dk, dv, nullptr, 1, stream);
}

hipError_t launch_bwd_split(const Problem& p, const void* q, const void* k, const void* v,
                            const void* dout, const float* lse, const float* delta,
                            const int32_t* cu, float* dq_accum, float* dkv_part, int nsplit,
                            hipStream_t stream) {
  if (dq_accum)
    return bwd_dispatch<true>(p, q, k, v, dout, lse, delta, cu, dq_accum, nullptr, nullptr,
                              dkv_part, nsplit, stream);
  return bwd_dispatch<false>(p, q, k, v, dout, lse, delta, cu, nullptr, nullptr, nullptr,
                             dkv_part, nsplit, stream);
}

}  // namespace attn
