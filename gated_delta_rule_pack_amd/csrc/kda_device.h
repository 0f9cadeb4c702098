// Device helpers for the gfx950 kernels: vector types, conversions, MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16. Operand lane layout (lane l, g = l / 16):
//   A (16 x 32): row l % 16, k = 8g + j for element j of the bf16x8;
//   B (32 x 16): column l % 16, k = 8g + j;
//   C/D (16 x 16, fp32): column l % 16, rows 4g + i for element i.
// The k order inside an operand is free as long as A and B agree; the kernels use that
// to feed MFMA outputs straight back in as operands without any transposition.
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ float from_bf16(__bf16 x) { return (float)x; }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Split x into hi + lo, both bf16, with hi + lo = x to ~16 significant bits.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - from_bf16(hi));
}

__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
  bf16x8 r;
  r[0] = to_bf16(a[0]); r[1] = to_bf16(a[1]); r[2] = to_bf16(a[2]); r[3] = to_bf16(a[3]);
  r[4] = to_bf16(b[0]); r[5] = to_bf16(b[1]); r[6] = to_bf16(b[2]); r[7] = to_bf16(b[3]);
  return r;
}

// Eight fp32 values (a then b) as bf16 hi + lo operands.
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
  hi = pack8(a, b);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = to_bf16(a[i] - from_bf16(hi[i]));
    lo[4 + i] = to_bf16(b[i] - from_bf16(hi[4 + i]));
  }
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Logistic function with the fast exponential; -inf -> 0, +inf -> 1.
__device__ __forceinline__ float sigmoidf_fast(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ------------------------------------------------------------------ scan-side helpers
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer resource word 3 for gfx9-family untyped loads.
constexpr int kBufWord3 = 0x00020000;

// Cache policy of loads whose data is used once and should not displace what the call
// reads again: the non-temporal hint. When a call's chunk records fit the memory-side
// cache, prep streams its inputs (q, k, v, the raw gate) with it, so that the records it
// writes stay there for the segment-map and scan passes (1 x 16384 at H = 12: 217 MB of
// records next to 252 MB of inputs; the scan phase takes 107 instead of 120 us). Records
// that cannot fit (the 128-sequence batch: 1.7 GB) gain nothing, and its scan measured
// 5 % slower with the hint.
constexpr int kStreamLoad = 2;

__device__ __forceinline__ bf16x8 bload8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <int SDT>
__device__ __forceinline__ f32x4 load_state4(const void* plane, size_t off) {
  if constexpr (SDT == kF32) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(plane) + off);
  } else if constexpr (SDT == kF16) {
    const _Float16* s = reinterpret_cast<const _Float16*>(plane) + off;
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 v = *reinterpret_cast<const h4*>(s);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    const __bf16* s = reinterpret_cast<const __bf16*>(plane) + off;
    bf16x4 v = *reinterpret_cast<const bf16x4*>(s);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
}

template <int SDT>
__device__ __forceinline__ void store_state4(void* plane, size_t off, f32x4 x) {
  if constexpr (SDT == kF32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(plane) + off) = x;
  } else if constexpr (SDT == kF16) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 v = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
    *reinterpret_cast<h4*>(reinterpret_cast<_Float16*>(plane) + off) = v;
  } else {
    bf16x4 v = {to_bf16(x[0]), to_bf16(x[1]), to_bf16(x[2]), to_bf16(x[3])};
    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(plane) + off) = v;
  }
}

template <int SDT>
__device__ __forceinline__ size_t elem_size() {
  return SDT == kF32 ? 4 : 2;
}

template <int SDT>
__device__ __forceinline__ float load_state1(const void* plane, size_t off) {
  if constexpr (SDT == kF32) return reinterpret_cast<const float*>(plane)[off];
  else if constexpr (SDT == kF16) return (float)reinterpret_cast<const _Float16*>(plane)[off];
  else return (float)reinterpret_cast<const __bf16*>(plane)[off];
}

template <int SDT>
__device__ __forceinline__ void store_state1(void* plane, size_t off, float x) {
  if constexpr (SDT == kF32) reinterpret_cast<float*>(plane)[off] = x;
  else if constexpr (SDT == kF16) reinterpret_cast<_Float16*>(plane)[off] = (_Float16)x;
  else reinterpret_cast<__bf16*>(plane)[off] = to_bf16(x);
}

// State elements (v, k .. k+3) of a plane in either layout: V-first [V][K] holds them
// in one 16/8-byte run; K-first [K][V] holds them K elements apart (the lanes of a row
// group, consecutive v, then read consecutive addresses).
template <int SDT>
__device__ __forceinline__ f32x4 load_state4_vk(const void* plane, int v, int k, bool kfirst) {
  if (!kfirst) return load_state4<SDT>(plane, (size_t)v * kHead + k);
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = load_state1<SDT>(plane, (size_t)(k + i) * kHead + v);
  return r;
}

template <int SDT>
__device__ __forceinline__ void store_state4_vk(void* plane, int v, int k, f32x4 x, bool kfirst) {
  if (!kfirst) {
    store_state4<SDT>(plane, (size_t)v * kHead + k, x);
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) store_state1<SDT>(plane, (size_t)(k + i) * kHead + v, x[i]);
}

// The (sequence n, head h) state plane to read at the start (null: start from zero) and
// the one to write at the end (null: not written).
template <int SDT>
__device__ __forceinline__ const void* state_in_plane(const Plan& p, int n, int h) {
  if (p.in_mode == kStateDense)
    return reinterpret_cast<const char*>(p.state_in) + ((size_t)n * p.stride0 + (size_t)h * kHead * kHead) * elem_size<SDT>();
  if (p.in_mode == kStatePaged && p.flags[n])
    return reinterpret_cast<const char*>(p.state_in) +
           ((size_t)p.indices[n] * p.stride0 + (size_t)h * kHead * kHead) * elem_size<SDT>();
  return nullptr;
}

template <int SDT>
__device__ __forceinline__ void* state_out_plane(const Plan& p, int n, int h) {
  if (p.out_mode == kStateDense)
    return reinterpret_cast<char*>(p.state_out) + ((size_t)n * p.stride0 + (size_t)h * kHead * kHead) * elem_size<SDT>();
  if (p.out_mode == kStatePaged)
    return reinterpret_cast<char*>(p.state_out) +
           ((size_t)p.indices[n] * p.stride0 + (size_t)h * kHead * kHead) * elem_size<SDT>();
  return nullptr;
}

// Position of element (k, k') of a segment map's A^T plane (A^T[k][k'] = A[k'][k]) in the
// segment combine kernel's MFMA operand fragment order: fragment (k / 16) * 4 + k' / 32 of
// 64 lanes x 8 bf16, lane (k % 16) + 16 ((k' % 32) / 8), element k' % 8. One fragment is
// 1 KB of contiguous bytes, which the combine streams into LDS with one direct load.
__device__ __forceinline__ int map_frag_index(int k, int kp) {
  return ((k >> 4) * 4 + (kp >> 5)) * 512 + ((k & 15) + 16 * ((kp & 31) >> 3)) * 8 + (kp & 7);
}

// Barrier for waves that touch LDS only with ds instructions: their LDS writes are
// complete (lgkmcnt) before it and no LDS read moves above it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt bits
// [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most k chunks of L loads each are still in flight (k <= KMAX).
template <int L, int KMAX>
__device__ __forceinline__ void wait_chunks(int k) {
  if constexpr (KMAX == 0) {
    wait_vmcnt<0>();
  } else {
    if (k >= KMAX) wait_vmcnt<KMAX * L>();
    else wait_chunks<L, KMAX - 1>(k);
  }
}

}  // namespace kda
