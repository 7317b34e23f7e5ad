// Shared pieces of the gfx950 attention kernels: vector types, MFMA and
// LDS-transpose wrappers, the LDS swizzle, work decomposition helpers and the
// launch parameter block.  Host code includes it for the parameter block and
// the tile-count helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "attn_sched.h"
#include <stdint.h>

namespace attn {

// ---------------------------------------------------------------- params

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // may be null
  const int32_t* cu;       // varlen prefix sums (device) or null
  float* ws_o;             // split partial outputs [B,H,S,d] (decode path)
  float* ws_lse;           // split base-2 LSEs [B,H,S]
  int B, H, Hkv, Sq, Skv, d;
  int group;               // H / Hkv
  int causal;
  float scale;             // softmax scale s
  float scale_log2;        // s * log2(e): scores enter exp2 through one FMA
  int num_splits;          // decode path
  int split_len;           // keys per split: ceil(Skv / num_splits)
  int tiles_per_head;      // query tiles per (b, h) (varlen: upper bound per head)
  int work_items;          // real work items; the grid may be padded to 8k
  int persist_c;           // > 0: persistent grid of 8 x persist_c workgroups (see the kernel)
  // paged KV cache (decode): k and v are [num_pages, Hkv, page_size, d]
  const int32_t* block_table;  // [B, max_pages] physical page of each logical block, or null
  const int32_t* seqlens_k;    // [B] keys per sequence
  int page_shift;              // log2(page_size)
  int max_pages;               // row length of block_table
  int num_pages;               // pages in the cache (table entries are clamped into range)
  // layout: row strides (elements) of q/o and k/v; bshd selects the
  // [B, S, H, d] (varlen [T, H, d]) offsets instead of [B, H, S, d]
  int q_rs, kv_rs;
  int bshd;
  // sliding window and attention sinks (causal paths only)
  int window;                  // > 0: keys j with i + off - window < j <= i + off
  const float* sinks;          // [H] per-head sink logits (scaled-score units), or null
};

// ---------------------------------------------------------------- helpers

// Keys a causal query block [q_lo, q_hi) may see (bottom-right alignment:
// key j visible to row i iff j <= i + off).
__host__ __device__ inline int causal_kv_end(int q_hi, int off, int skv) {
  long e = (long)q_hi + off;
  if (e < 0) e = 0;
  return e < skv ? (int)e : skv;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 32x32x16 bf16 MFMA.  Lane l: A[l%32][8(l/32)+j], B[8(l/32)+j][l%32],
// D[8(r/4)+4(l/32)+r%4][l%32] (layout checked on gfx950).
__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16 MFMA.  Lane l: A[l%16][8(l/16)+j], B[8(l/16)+j][l%16],
// D[4(l/16)+i][l%16].
__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read of four 16-bit values.  Inside each group of 16 lanes,
// lane i receives element i%4 of the 8-byte words addressed by lanes
// i/4, 4+i/4, 8+i/4, 12+i/4 (element j from lane 4j+i/4).
__device__ inline s16x4 lds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      LDS_PTR(s16x4, const_cast<void*>(lds_addr)));
}

__device__ inline bf16x8 join_tr(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return __builtin_bit_cast(bf16x8, r);
}

// Eight fp32 -> bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ inline bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                   float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

__device__ inline float shfl_xor_f(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Value of lane l ^ 32 combined with lane l's own, through v_permlane32_swap
// (no LDS round trip): returns max / sum over the lane pair (l, l ^ 32).
__device__ inline float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3).
// Loads whose offset falls outside [0, bytes) return zero.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

#pragma clang diagnostic push
// m0 is written by these loads only; no other instruction in the kernel reads it
#pragma clang diagnostic ignored "-Winline-asm"
// HBM -> LDS without registers: 16 bytes per lane at LDS address m0 + 16 *
// lane (out-of-range bytes arrive as zeros).  Issued as inline assembly so
// that the compiler, which cannot tell which LDS bytes they write, does not
// wait for them before every LDS read; a kernel waits for them itself
// (vmcnt) before the barrier that publishes the buffer they fill.  lds_addr
// must be wave-uniform.
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, int voff, int soff, unsigned lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(r), "s"(soff), "s"(lds_addr)
      : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ inline int64_t uniform64(int64_t x) {
  const uint64_t u = (uint64_t)x;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// buffer descriptor of a wave-uniform base and size, kept in scalar registers
// (the loads above take it as a scalar operand)
__device__ inline __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const int64_t b = uniform64((int64_t)(uintptr_t)base);
  return make_rsrc((const void*)(uintptr_t)b, __builtin_amdgcn_readfirstlane(bytes));
}

__device__ inline unsigned lds_u32(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N-1>), expanded at
// compile time (every index a constant, so arrays indexed by it stay in
// registers however long the sequence)
template <typename F, int... I>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------- LDS swizzle
//
// A K or V tile sits in LDS row-major (one key per row, d contiguous) with
// its 16-byte chunks permuted per row: chunk c of row r lives at chunk
// c ^ swz(r).  Rows are 128 B (d = 64) or 256 B (d = 128) wide and the LDS
// has 64 four-byte banks.  The permutation keeps two access patterns free of
// bank conflicts:
//   * the QK^T operand read: 16 consecutive rows, same logical chunk;
//   * the transposed V read: 8 consecutive rows x 4 consecutive chunks, the
//     minimum (two-way) for 512 bytes.
template <int D>
__host__ __device__ constexpr int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    // two rows per 256-byte bank sweep: the row parity picks the half
    const int b = r >> 1;
    return ((b & 1) << 2) | ((b >> 1) & 3);
  }
}

template <int D>
__host__ __device__ constexpr int lds_off(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ swz<D>(row)) << 4);
}

}  // namespace attn
