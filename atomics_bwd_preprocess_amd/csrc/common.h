// Device helpers shared by the gfx950 attention kernels: vector types, MFMA
// wrappers, 16-bit conversions and small wave-level primitives.
//
// MFMA 32x32x16 (v_mfma_f32_32x32x16_{f16,bf16}) register layout used
// throughout (wave64, lane l, c = l / 32, n = l % 32):
//   A (32 x 16): lane l holds row n, k-slots (c, e), e = 0..7   (8 x 16-bit)
//   B (16 x 32): lane l holds column n, k-slots (c, e)          (8 x 16-bit)
//   C (32 x 32): lane l, register r = 0..15 holds
//                row (r / 4) * 8 + 4 * c + (r % 4), column n.
// A and B pair the same slot (c, e) in the contraction, so any assignment of
// k indices to slots is valid as long as both operands use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct V8;
template <> struct V8<_Float16> { typedef f16x8 type; typedef f16x4 half_type; };
template <> struct V8<__bf16> { typedef bf16x8 type; typedef bf16x4 half_type; };

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// MFMA 16x16x32 (v_mfma_f32_16x16x32_{f16,bf16}): lane l, g = l / 16, i = l % 16:
//   A (16 x 32): row i, k-slots (g, e); B (32 x 16): column i, k-slots (g, e);
//   C (16 x 16): register r = 0..3 holds row 4 g + r, column i.
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even conversion of fp32 to the 16-bit storage type.
template <typename T> __device__ __forceinline__ T to16(float x) { return static_cast<T>(x); }

// 16-byte loads / stores and 8-byte stores (global or LDS, by address space
// inference).
template <typename T> __device__ __forceinline__ typename V8<T>::type ld16(const T* p) {
  return __builtin_bit_cast(typename V8<T>::type, *reinterpret_cast<const u32x4*>(p));
}
template <typename T> __device__ __forceinline__ void st16(T* p, typename V8<T>::type v) {
  *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}
template <typename T> __device__ __forceinline__ void st8(T* p, typename V8<T>::half_type v) {
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v);
}

// Pack registers [base, base + 8) of an MFMA C tile into an operand.
template <typename T>
__device__ __forceinline__ typename V8<T>::type pack8(const f32x16& v, int base) {
  typename V8<T>::type r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = to16<T>(v[base + i]);
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Raw buffer resources (gfx9 descriptor: stride 0, num_records in bytes).
// Loads beyond num_records return zero and stores / atomics beyond it are
// dropped by the hardware, which is how the kernels handle tile tails.  The
// whole offset is passed in the VGPR operand (soffset = 0).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store_b16(rsrc_t r, uint32_t off, unsigned short v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store_f32(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_atomic_add(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, off, 0, 0);
}
template <typename T> __device__ __forceinline__ unsigned short bits16(T x) {
  return __builtin_bit_cast(unsigned short, x);
}

// ---- LDS tiles, transposing reads and direct-to-LDS copies --------------

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS bank model (measured on MI355X): 64 banks of 4 bytes; 16-byte accesses
// resolve in passes of 16 lanes, 8-byte and transposing accesses in passes of
// 32 lanes.  The swizzles of the kernels make every access pattern they issue
// conflict-free under that model (checked exhaustively by the host model of
// the LDS layouts in the tests).
//
// Row-major tiles (D columns): 16-byte chunk c of row r lives at chunk
// c ^ chunk_swz(r): 16 consecutive rows hit 16 distinct chunks (16-byte operand
// reads), and 4 consecutive rows spread a 64-byte column block over the whole
// bank range (transposing reads).
template <int D>
__device__ __forceinline__ int chunk_swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int rm_off(int r, int col) {  // col: multiple of 4
  return r * (D * 2) + (((col >> 3) ^ chunk_swz<D>(r)) << 4) + ((col & 7) << 1);
}

template <typename T>
__device__ __forceinline__ typename V8<T>::type lds16(const char* smem, int off) {
  return __builtin_bit_cast(typename V8<T>::type, *reinterpret_cast<const u32x4*>(smem + off));
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// i receives element (i % 4) of the 8-byte pieces addressed by lanes
// 4e + i / 4, e = 0..3.  Lanes address row k0 + p / 4, columns n0 + 4 (p % 4)
// (p = lane % 16) of a row-major matrix; lane i then holds rows k0..k0+3 of
// column n0 + i.
__device__ __forceinline__ u32x2 tr_read(const char* smem, int off) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + off));
  return __builtin_bit_cast(u32x2, v);
}
template <typename T>
__device__ __forceinline__ typename V8<T>::type tr_pair(const char* smem, int off_lo, int off_hi) {
  const u32x2 lo = tr_read(smem, off_lo), hi = tr_read(smem, off_hi);
  const u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(typename V8<T>::type, r);
}

// LDS byte address of a location in a __shared__ array: the value M0 takes
// for a direct-to-LDS copy.  Formed once per kernel (the conversion from a
// generic pointer costs a null check and the aperture base in scalar code).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes bytes
// [16 l, 16 l + 16) after the wave-uniform LDS address `lds` (lds_addr plus
// uniform offsets).  Issued as inline assembly so the compiler's wait-count
// bookkeeping does not follow it (it would otherwise wait for the load before
// the next LDS access); the kernel waits for it explicitly before the barrier
// that publishes it.  M0 (which supplies the LDS address) is saved and
// restored around it.
__device__ __forceinline__ void lds_dma16(rsrc_t r, uint32_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(r)
      : "memory");
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8) that wait on vector memory only.
// kVmcnt0 + n (n < 16) waits until at most n are outstanding.
constexpr int kVmcnt0 = 0x0F70;

// Same for 4 bytes per lane: lane l writes bytes [4 l, 4 l + 4) after `lds`.
__device__ __forceinline__ void lds_dma4(rsrc_t r, uint32_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(r)
      : "memory");
}

// This lane's index within the wave, computed where it is used.  The asm is
// volatile so the value is not hoisted out of a loop and held in a register
// across it (in register-bound loops the compiler would rather spill it).
__device__ __forceinline__ uint32_t lane_here() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Wave-uniform integer kept in a scalar register (buffer descriptor fields
// must be scalar; clamps otherwise tend to land in vector registers).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Sequence bounds [a, b) clamped to [0, total]; cu == nullptr means a dense batch.
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int s, int max_seqlen, int total,
                                           int& a, int& b) {
  long long lo, hi;
  if (cu) {
    lo = cu[s];
    hi = cu[s + 1];
  } else {
    lo = (long long)s * max_seqlen;
    hi = lo + max_seqlen;
  }
  lo = lo < 0 ? 0 : (lo > total ? total : lo);
  hi = hi < lo ? lo : (hi > total ? total : hi);
  a = (int)lo;
  b = (int)hi;
}

// Visibility of key position j to query position i (local to one sequence).
__device__ __forceinline__ bool visible(int i, int j, bool causal, int window) {
  return (!causal || j <= i) && (window <= 0 || j > i - window);
}

}  // namespace attn
