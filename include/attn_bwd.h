/*
 * attn_bwd.h -- C ABI of the MI355X (gfx950) GQA attention backward library.
 *
 * The library computes the FlashAttention-style backward pass of grouped-query
 * attention over packed variable-length sequences, with causal and
 * sliding-window masks and a per-head attention sink, plus the forward pass
 * that produces the O and lse the backward consumes.  Sources for the
 * operations are given per call below; "the pages" are
 *   [TL]  tilelang PR "[GQA] Add regional atomic add to slightly boost performance",
 *   [ASC] tilelang-ascend PR "GQA Sink Backward BHSD",
 *   [TRI] triton issue "atomic_add slows down attention backwards due to layout conversions".
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are packed "THD" by default (shape->layout = ATTN_LAYOUT_THD):
 *    all tokens of all sequences along one axis, heads next, head_dim
 *    innermost and contiguous.
 *      q, o, dout, dq      [T, Hq,  D]   storage dtype (fp16 or bf16)
 *      k, v, dk, dv        [T, Hkv, D]   storage dtype
 *      lse, delta          [Hq, T]       fp32 (lse: natural log)
 *      dq_accum            [T, Hq, D]    fp32 workspace for dQ accumulation
 *      sink, dsink         [Hq]          fp32
 *      cu_seqlens          [num_seqs+1]  int32, sequence s spans tokens
 *                                        [cu_seqlens[s], cu_seqlens[s+1])
 *  - With shape->layout = ATTN_LAYOUT_BHSD (the [ASC] kernels' "BHSD" layout)
 *    the batch is dense (B = num_seqs sequences of S = max_seqlen tokens,
 *    cu_seqlens NULL) and the 16-bit tensors and dq_accum are [B, H, S, D]
 *    (each head's rows contiguous): q, o, dout, dq, dq_accum [B, Hq, S, D],
 *    k, v, dk, dv [B, Hkv, S, D].  lse / delta stay [Hq, T] with token
 *    t = b * S + s.  Results are the same as for the same data packed THD.
 *  - All pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees or retains them and keeps no state between calls.
 *  - Every call only enqueues work on `stream` (NULL = the default stream) and
 *    never synchronises; buffers must stay alive until that work completes.
 *  - Query head h reads kv head h / (Hq/Hkv) (contiguous groups, [TL] review
 *    comment on the single dK/dV write).
 *  - Masks (per sequence, query position i, key position j, both local):
 *      causal:      j <= i
 *      window W>0:  i - W < j <= i  (requires causal; at most W keys per query)
 *  - Sink ([ASC] forward with online softmax + sink + window): one logit per
 *    query head in the units of scaled scores; it joins the softmax
 *    denominator and has no value vector, so
 *      lse_i = log(sum_{visible j} exp(scale*q_i.k_j) + exp(sink_h)).
 *  - Alignment: q, k, v, o, dout, dq, dk, dv and dq_accum must be 16-byte
 *    aligned; lse, delta, sink, dsink and cu_seqlens 4-byte aligned.
 *  - Errors: argument problems are reported by the return code before any
 *    work is enqueued (nothing is launched on error); a launch failure returns
 *    ATTN_ERR_HIP.  attn_last_error() gives a message for the calling thread.
 *    Device-side faults surface at the caller's next synchronisation.
 *  - Device-data preconditions (documented, not checked because the data is
 *    device-resident): cu_seqlens[0] = 0, non-decreasing, last entry =
 *    total_tokens, every length <= max_seqlen.  Kernels clamp sequence bounds
 *    to [0, total_tokens], so a violation gives wrong results, never an
 *    out-of-bounds access.  A NULL cu_seqlens means a dense batch:
 *    sequence s spans [s*max_seqlen, (s+1)*max_seqlen) and
 *    total_tokens must equal num_seqs*max_seqlen.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 7
#define ATTN_MAX_SPLIT 16 /* largest nsplit of attn_bwd_split */
/* Bytes of the library-owned scratch array attn_bwd_static accumulates dQ in
   (64 MiB per GPU the library runs on). */
#define ATTN_STATIC_SCRATCH_BYTES (64u * 1024u * 1024u)

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, misalignment, bad dims, Hq % Hkv != 0,
                               window without causal, sink/dsink mismatch */
  ATTN_ERR_UNSUPPORTED = 2, /* head_dim not in {64, 128}, unknown dtype */
  ATTN_ERR_HIP = 3          /* a HIP launch reported an error */
} attn_status_t;

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Layout of the 16-bit tensors (q, k, v, o, dout, dq, dk, dv) and of dq_accum. */
typedef enum {
  ATTN_LAYOUT_THD = 0, /* packed [T, H, D] (varlen via cu_seqlens, or a dense batch) */
  ATTN_LAYOUT_BHSD = 1 /* [B, H, S, D] dense batch: B = num_seqs, S = max_seqlen,
                          T = B * S, cu_seqlens must be NULL */
} attn_layout_t;

/* Problem description shared by every call. */
typedef struct {
  int32_t num_seqs;     /* number of packed sequences (>= 1) */
  int32_t max_seqlen;   /* upper bound on every sequence length (>= 1) */
  int32_t total_tokens; /* T: rows of q/k/v (>= 0) */
  int32_t hq;           /* query heads */
  int32_t hkv;          /* key/value heads; hq % hkv == 0 */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t causal;       /* 0 or 1 */
  int32_t window;       /* 0: none; W > 0: sliding window (requires causal) */
  float scale;          /* score scale, typically 1/sqrt(D); finite and > 0 */
  int32_t dtype;        /* attn_dtype_t of q/k/v/o/dout/dq/dk/dv */
  int32_t layout;       /* attn_layout_t (0 = packed THD) */
} attn_shape_t;

/*
 * Forward ([ASC] forward kernel: online softmax with sink and window).
 * Writes O [T,Hq,D] (storage dtype, RNE from fp32) and lse [Hq,T] (fp32,
 * natural log).  sink may be NULL (no sink).  A row with no visible key and
 * no sink gets O = 0 and lse = -inf (cannot happen with causal masks, where a
 * query always sees itself).
 */
attn_status_t attn_fwd(const attn_shape_t* shape, const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens, const float* sink, void* o, float* lse,
                       hipStream_t stream);

/*
 * Backward preprocess ([ASC] merged "flashattn_bwd_preprocess" with the dsink
 * kernel; Phase 0 of its single backward kernel computes Delta as the row sum
 * of O*dO; the Dsink kernel computes dsink = -sum exp(sink - lse) * Delta).
 *   delta[h][t]  = sum_d o[t][h][d] * dout[t][h][d]   (fp32 accumulation)
 *   dq_accum     := 0 (all T*Hq*D entries; skipped when dq_accum is NULL,
 *                   as the deterministic path below needs no accumulator)
 *   dsink[h]     = -sum_t exp(sink[h] - lse[h][t]) * delta[h][t]
 * sink and dsink must both be NULL or both non-NULL.  dsink is written (not
 * accumulated) and its reduction order is fixed, so it is deterministic.
 */
attn_status_t attn_bwd_preprocess(const attn_shape_t* shape, const void* o, const void* dout,
                                  const float* lse, const int32_t* cu_seqlens,
                                  const float* sink, float* delta, float* dq_accum,
                                  float* dsink, hipStream_t stream);

/*
 * dsink alone ([ASC] Dsink kernel): dsink[h] = -sum_t exp(sink[h] - lse[h][t])
 * * delta[h][t] over all T tokens, written (not accumulated), fixed reduction
 * order.  The same values attn_bwd_preprocess writes when given sink and
 * dsink.  For callers that run the preprocess without sink (Delta only) and
 * the reduction later, off the path of the main passes; it needs delta
 * complete.
 */
attn_status_t attn_bwd_dsink(const attn_shape_t* shape, const float* lse, const float* delta,
                             const float* sink, float* dsink, hipStream_t stream);

/*
 * Backward main pass.  Recomputes S = Q K^T and P = exp(S*scale - lse) per
 * tile, then dV = P^T dO, dP = dO V^T, dS = P o (dP - Delta) * scale,
 * dK = dS^T Q and dQ = dS K ([ASC] review thread, kernels k1-k5 fused).
 *  - lse must be finite on every row of every sequence, as attn_fwd
 *    produces it whenever each query sees at least one key (always the case
 *    under causal and window masks); rows with lse = -inf are not supported.
 *  - dq_accum (zeroed by attn_bwd_preprocess) receives dQ / scale through
 *    fp32 atomic adds issued once per (query tile, key tile) as one
 *    coalesced region-wide sweep ([TL] regional atomic add; [TRI] atomics
 *    issued from the matrix-core layout).  The score scale is applied by
 *    attn_bwd_postprocess.  Summation order varies run to run.
 *  - dk, dv are WRITTEN once per key row after accumulating, in fp32
 *    registers, over every query block and every query head of the group
 *    ([TL] review: accumulate locally, write once).  They are deterministic.
 * The sink enters only through lse.
 */
attn_status_t attn_bwd(const attn_shape_t* shape, const void* q, const void* k, const void* v,
                       const void* dout, const float* lse, const float* delta,
                       const int32_t* cu_seqlens, float* dq_accum, void* dk, void* dv,
                       hipStream_t stream);

/*
 * Number of int32 arrival counters attn_bwd_fused_cast needs: one per
 * (sequence, query head, block of 32 query rows), rounded up to a multiple
 * of 4.
 */
#define ATTN_FUSED_CAST_COUNTERS(num_seqs, hq, max_seqlen) \
  (((long long)(num_seqs) * (hq) * (((max_seqlen) + 31) / 32) + 3) / 4 * 4)

/*
 * attn_bwd and attn_bwd_postprocess in one pass, for causal problems
 * ([ASC] names the separate postprocess, and the host-side cast of its fp32
 * dK/dV atomics, as costs it could not remove; on this part the cast needs
 * no host sync and can live in the main pass).  dq_accum is zeroed by
 * attn_bwd_preprocess as for attn_bwd.  The call zeroes `counters`
 * (int32[ATTN_FUSED_CAST_COUNTERS(...)], caller-owned, 16-byte aligned) and
 * runs the main pass; every key-block workgroup, after its last dQ atomics
 * are performed device-wide, counts one arrival at each (query head, query
 * block) it contributed to, and the workgroup whose arrival completes a
 * block's count (the number of key blocks whose loop contains it, known in
 * closed form) reads that block's rows of dq_accum and writes
 * dq = RNE(scale * dq_accum).  dk and dv are written as by attn_bwd.
 * Non-causal problems (where the last finisher of a sequence would cast all
 * of it alone) and the [B, H, S, D] layout run attn_bwd followed by the
 * separate cast instead; the results are the same either way.  dq_accum
 * holds dQ / scale afterwards.
 */
attn_status_t attn_bwd_fused_cast(const attn_shape_t* shape, const void* q, const void* k,
                                  const void* v, const void* dout, const float* lse,
                                  const float* delta, const int32_t* cu_seqlens, float* dq_accum,
                                  int32_t* counters, void* dq, void* dk, void* dv,
                                  hipStream_t stream);

/*
 * Deterministic backward, pass 1 of 2: the main pass above without its dQ
 * product.  Writes the dk and dv of attn_bwd up to fp32 summation order: it
 * sums the same products query block by query block from the sequence end
 * (every head of a block in turn), where attn_bwd goes head by head.  The
 * result is bitwise reproducible run to run; issues no atomics and needs no
 * dq_accum.
 */
attn_status_t attn_bwd_dkdv(const attn_shape_t* shape, const void* q, const void* k,
                            const void* v, const void* dout, const float* lse,
                            const float* delta, const int32_t* cu_seqlens, void* dk, void* dv,
                            hipStream_t stream);

/*
 * Deterministic backward, pass 2 of 2: query-stationary dQ ([ASC] backward
 * keeps dQ in the matrix unit's accumulator over its key loop).  Per query
 * tile it walks the visible key blocks, recomputes S, P, dP and
 * dS = P o (dP - Delta), accumulates dQ = scale * sum_j dS_ij k_j in fp32
 * registers and writes dq [T,Hq,D] once (storage dtype, RNE).  No atomics,
 * no workspace, a fixed summation order: bitwise reproducible.  Same lse
 * precondition as attn_bwd.  Independent of attn_bwd_dkdv (the two may run
 * concurrently on different streams).
 */
attn_status_t attn_bwd_dq(const attn_shape_t* shape, const void* q, const void* k, const void* v,
                          const void* dout, const float* lse, const float* delta,
                          const int32_t* cu_seqlens, void* dq, hipStream_t stream);

/*
 * attn_bwd_dq that also forms Delta: [ASC]'s single-kernel revision folds
 * the preprocess into its backward kernel as Phase 0; here the
 * query-stationary dQ pass reads O beside dO and computes
 *   delta[h][t] = sum_d o[t][h][d] * dout[t][h][d]
 * for its own rows, writes it (every row of every sequence exactly once) and
 * uses it.  The arithmetic and summation order are those of
 * attn_bwd_preprocess, so delta is bitwise the same.  For a deterministic
 * backward without the preprocess:
 * attn_bwd_dq_delta, then attn_bwd_dkdv (which reads delta), then
 * attn_bwd_dsink if there is a sink.  dq_accum is not used.
 */
attn_status_t attn_bwd_dq_delta(const attn_shape_t* shape, const void* q, const void* k,
                                const void* v, const void* o, const void* dout, const float* lse,
                                const int32_t* cu_seqlens, float* delta, void* dq,
                                hipStream_t stream);

/*
 * Main backward pass (as attn_bwd, or as attn_bwd_dkdv when dq_accum is NULL)
 * with the query loop of every key block split over `nsplit` workgroups
 * (1..ATTN_MAX_SPLIT), for problems whose longest key block sets the
 * critical path (ragged varlen batches).  Part p of a key block covers an
 * equal share of its (query head, query block) pairs and WRITES its dK / dV
 * partial, summed in fp32 registers over that share, into slot p of
 * dkv_partial: fp32 [nsplit][2][dk-shaped] (slot p holds dK * scale, then
 * dV, each in the layout of dk).  Every row of every slot is written once,
 * so no zeroing is needed.  dQ is accumulated into dq_accum exactly as in
 * attn_bwd.  attn_bwd_dkv_reduce then forms dk and dv.
 */
attn_status_t attn_bwd_split(const attn_shape_t* shape, const void* q, const void* k,
                             const void* v, const void* dout, const float* lse,
                             const float* delta, const int32_t* cu_seqlens, float* dq_accum,
                             float* dkv_partial, int32_t nsplit, hipStream_t stream);

/*
 * dk = RNE(sum_p dkv_partial[p][0]), dv = RNE(sum_p dkv_partial[p][1]), the
 * sum taken in fp32 over p = 0 .. nsplit-1 in that order (deterministic).
 */
attn_status_t attn_bwd_dkv_reduce(const attn_shape_t* shape, const float* dkv_partial,
                                  int32_t nsplit, void* dk, void* dv, hipStream_t stream);

/*
 * attn_bwd followed by attn_bwd_postprocess, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the fp32 dQ accumulator is not a caller workspace but a
 * library-owned device array of ATTN_STATIC_SCRATCH_BYTES per GPU, held from
 * library load until the process ends.  The call zeroes that accumulator
 * with a fill kernel, runs the main pass into it and casts it into dq
 * (storage dtype, RNE of scale * accumulator), all on `stream`; it allocates
 * nothing and calls no allocating routine.  Inputs and outputs are the
 * caller's as for attn_bwd (delta from attn_bwd_preprocess, which may be
 * called with dq_accum = NULL); dq, dk, dv are written.
 *  - Size limit: total_tokens * hq * head_dim * 4 bytes must not exceed
 *    ATTN_STATIC_SCRATCH_BYTES, else ATTN_ERR_INVALID_ARG before any launch.
 *  - Every call on one GPU uses that GPU's single array: calls that overlap
 *    on one GPU (different streams, or host threads) race and give wrong dQ.
 *    Serialise them (one stream, or events).
 *  - The first call on a device looks up the array's device address (no
 *    allocation); a failure there is ATTN_ERR_HIP.
 * Results equal attn_bwd + attn_bwd_postprocess (dQ within the atomic
 * summation-order variation; dk, dv bitwise).
 */
attn_status_t attn_bwd_static(const attn_shape_t* shape, const void* q, const void* k,
                              const void* v, const void* dout, const float* lse,
                              const float* delta, const int32_t* cu_seqlens, void* dq, void* dk,
                              void* dv, hipStream_t stream);

/*
 * Backward postprocess ([ASC] postprocess kernel casting the fp32 gradient
 * accumulator): dq[t][h][d] = RNE cast of (scale * dq_accum[t][h][d]) to the
 * storage dtype, the multiplication done in fp32.
 */
attn_status_t attn_bwd_postprocess(const attn_shape_t* shape, const float* dq_accum, void* dq,
                                   hipStream_t stream);

/* Static text for a status code. */
const char* attn_status_string(attn_status_t status);
/* Detail of the calling thread's most recent error ("" if none). */
const char* attn_last_error(void);
/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
