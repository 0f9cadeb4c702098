// Decode kernel: the recurrent step for calls in which every sequence has at most one
// token. Decode goes through a fused update kernel rather than the chunked path (aiter
// PR 4741, Performance), and it is bound by state bandwidth, with the state read and
// written at its storage dtype and accumulated in fp32 (aiter PR 5249, Why).
//
// Per (sequence, head), with the token's q-hat, k-hat, v, g = lb * sigmoid(g_raw) and
// beta = sigmoid(beta_raw), and S the V x K state:
//
//   D = S Diag(e^g)                     decay
//   u = D k-hat                         (V)
//   S = D + beta (v - u) k-hat^T        delta update with the token's own gate
//   o = scale * S q-hat                 read-out from the updated state
//
// A sequence with no token leaves its state unchanged, and the state is still written
// back: a flagged paged slot round-trips bit for bit and an unflagged one becomes zero,
// as in the chunked path.
//
// It is bound by the state traffic (one read and one write of V x K elements per
// sequence and head), so it is a single pass over the state rows in fp32: a workgroup
// per (sequence, head); wave w owns value rows 32w .. 32w+31, four rows at a time with
// sixteen lanes per row and eight keys per lane (one or two 16-byte accesses). Every
// row's loads are issued before any of its arithmetic, the rows stay packed at the
// storage dtype until they are used, and the two row reductions (u and o) are 16-lane
// sums on DPP lane permutes.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kRowsPerWave = 32;
constexpr int kIters = kRowsPerWave / 4;  // four rows per wave per iteration

// Sum over the 16 lanes of a row group (lanes 16r .. 16r+15), left in every lane of the
// group. Each step adds a lane permutation of the partial sums on the vector ALU (DPP, no
// LDS round trip): quad partners at distance 1 and 2, then lane i with 7 - i of its eight
// (the two quads of a half-row), then the two half-rows (row rotate by 8).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xb1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4e>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x128>(x);  // row_ror:8
  return x;
}

// x plus its copy in lane l ^ 8, l ^ 16 or l ^ 32 (row rotate by 8; the row and half-wave
// register swaps of gfx950, which here swap a register with itself).
__device__ __forceinline__ float add_xor8(float x) { return x + dpp<0x128>(x); }
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum over all 64 lanes, left in every lane.
__device__ __forceinline__ float sum64(float x) { return add_xor32(add_xor16(sum16(x))); }

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Eight state elements of one row, as stored: 32 bytes of fp32 or 16 bytes of fp16/bf16,
// each moved with 16-byte accesses.
template <int SDT>
struct Row8 {
  uint4 w[SDT == kF32 ? 2 : 1];
};

template <int SDT>
__device__ __forceinline__ Row8<SDT> load_row8(const void* plane, size_t off) {
  Row8<SDT> r;
  const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(plane) + off * elem_size<SDT>());
#pragma unroll
  for (int i = 0; i < (SDT == kF32 ? 2 : 1); ++i) r.w[i] = src[i];
  return r;
}

template <int SDT>
__device__ __forceinline__ float row8_get(const Row8<SDT>& r, int j) {
  if constexpr (SDT == kF32) {
    const uint32_t x = j < 4 ? (&r.w[0].x)[j] : (&r.w[1].x)[j - 4];
    return __uint_as_float(x);
  } else {
    const uint32_t x = (&r.w[0].x)[j >> 1];
    const uint16_t b = (j & 1) ? (uint16_t)(x >> 16) : (uint16_t)(x & 0xffffu);
    if constexpr (SDT == kF16) return (float)__builtin_bit_cast(_Float16, b);
    else return __uint_as_float((uint32_t)b << 16);
  }
}

template <int SDT>
__device__ __forceinline__ void store_row8(void* plane, size_t off, const float* x) {
  uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(plane) + off * elem_size<SDT>());
  if constexpr (SDT == kF32) {
    dst[0] = uint4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    dst[1] = uint4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])};
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t lo, hi;
      if constexpr (SDT == kF16) {
        lo = __builtin_bit_cast(uint16_t, (_Float16)x[2 * i]);
        hi = __builtin_bit_cast(uint16_t, (_Float16)x[2 * i + 1]);
      } else {
        lo = __builtin_bit_cast(uint16_t, to_bf16(x[2 * i]));
        hi = __builtin_bit_cast(uint16_t, to_bf16(x[2 * i + 1]));
      }
      w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    dst[0] = uint4{w[0], w[1], w[2], w[3]};
  }
}

template <int SDT, bool GF32>
__global__ __launch_bounds__(256) void decode_kernel(Plan p) {
  const int n = blockIdx.x / p.H;
  const int h = blockIdx.x - n * p.H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rg = lane >> 4;       // row of the group of four
  const int k0 = 8 * (lane & 15);  // this lane's eight keys
  const int hqk = __builtin_amdgcn_readfirstlane(h / p.group);  // q/k head of value head h
  const int t0 = __builtin_amdgcn_readfirstlane(p.d_cu[n]);
  const bool has_token = __builtin_amdgcn_readfirstlane(p.d_cu[n + 1]) > t0;

  // State rows of this wave, all loads first, kept as stored until used.
  const void* in_plane = state_in_plane<SDT>(p, n, h);
  Row8<SDT> raw[kIters];
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    const size_t off = (size_t)(kRowsPerWave * wave + 4 * i + rg) * kHead + k0;
    if (in_plane) raw[i] = load_row8<SDT>(in_plane, off);
    else raw[i] = Row8<SDT>{};
  }
  void* out_plane = state_out_plane<SDT>(p, n, h);

  float o_rows[kIters];
  if (has_token) {
    const size_t tok = ((size_t)t0 * p.H + h) * kHead;
    const size_t tqk = ((size_t)t0 * p.H_qk + hqk) * kHead;
    // q, k (bf16), the raw gate, beta and this lane's value rows.
    const uint4 qw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.q) + tqk + k0);
    const uint4 kw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.k) + tqk + k0);
    float gr[8];
    if constexpr (GF32) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.g_raw) + tok + k0);
      const f32x4 b = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.g_raw) + tok + k0 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gr[j] = a[j];
        gr[4 + j] = b[j];
      }
    } else {
      const uint4 gw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.g_raw) + tok + k0);
      const uint32_t g32[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gr[2 * j] = __uint_as_float(g32[j] << 16);
        gr[2 * j + 1] = __uint_as_float(g32[j] & 0xffff0000u);
      }
    }
    const size_t bidx = (size_t)t0 * p.H + h;
    const float braw = p.beta_dtype == kF32 ? reinterpret_cast<const float*>(p.beta_raw)[bidx]
                                            : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.beta_raw)[bidx]);
    float vr[kIters];
#pragma unroll
    for (int i = 0; i < kIters; ++i)
      vr[i] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.v)[tok + kRowsPerWave * wave + 4 * i + rg]);

    const uint32_t q32[4] = {qw.x, qw.y, qw.z, qw.w}, k32[4] = {kw.x, kw.y, kw.z, kw.w};
    float qh[8], kh[8], eg[8];
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qh[2 * j] = __uint_as_float(q32[j] << 16);
      qh[2 * j + 1] = __uint_as_float(q32[j] & 0xffff0000u);
      kh[2 * j] = __uint_as_float(k32[j] << 16);
      kh[2 * j + 1] = __uint_as_float(k32[j] & 0xffff0000u);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sq += qh[j] * qh[j];
      sk += kh[j] * kh[j];
      eg[j] = __expf(p.lower_bound * sigmoid(gr[j]));
    }
    const float rq = rsqrtf(sum16(sq) + 1e-6f) * p.scale;  // scale folded into q-hat
    const float rk = rsqrtf(sum16(sk) + 1e-6f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qh[j] *= rq;
      kh[j] *= rk;
    }
    const float beta = sigmoid(braw);

    // Each row is stored as soon as it is updated.
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      float d[8];
      float pu = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        d[j] = row8_get<SDT>(raw[i], j) * eg[j];
        pu += d[j] * kh[j];
      }
      const float c = beta * (vr[i] - sum16(pu));
      float po = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        d[j] += c * kh[j];
        po += d[j] * qh[j];
      }
      o_rows[i] = sum16(po);
      if (out_plane) store_row8<SDT>(out_plane, (size_t)(kRowsPerWave * wave + 4 * i + rg) * kHead + k0, d);
    }
  } else if (out_plane) {
    // No token: the state is written back as read (zero when nothing was read).
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(out_plane) +
                                            ((size_t)(kRowsPerWave * wave + 4 * i + rg) * kHead + k0) * elem_size<SDT>());
#pragma unroll
      for (int w = 0; w < (SDT == kF32 ? 2 : 1); ++w) dst[w] = raw[i].w[w];
    }
  }
  if (has_token && (lane & 15) == 0) {
    __bf16* o = reinterpret_cast<__bf16*>(p.out) + ((size_t)t0 * p.H + h) * kHead + kRowsPerWave * wave + rg;
#pragma unroll
    for (int i = 0; i < kIters; ++i) o[4 * i] = to_bf16(o_rows[i]);
  }
}

// K-first planes [K][V]. Wave w owns value columns 32w .. 32w+31; lane (ko = lane & 15,
// vo = lane >> 4) holds S[k][v] for keys k = 16i + ko (i = 0..7) and the eight columns
// v = 32w + 8vo .. 32w + 8vo + 7, one or two 16-byte accesses per key. The sums over k
// (u and o) run over the lane's eight keys, then over the 16 lanes of its group, which
// hold all 128 keys of the same columns.
template <int SDT, bool GF32>
__global__ __launch_bounds__(256) void decode_kfirst_kernel(Plan p) {
  const int n = blockIdx.x / p.H;
  const int h = blockIdx.x - n * p.H;
  const int hqk = __builtin_amdgcn_readfirstlane(h / p.group);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ko = lane & 15;
  const int v0 = kRowsPerWave * wave + 8 * (lane >> 4);
  const int t0 = __builtin_amdgcn_readfirstlane(p.d_cu[n]);
  const bool has_token = __builtin_amdgcn_readfirstlane(p.d_cu[n + 1]) > t0;

  const void* in_plane = state_in_plane<SDT>(p, n, h);
  Row8<SDT> raw[kIters];
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    if (in_plane) raw[i] = load_row8<SDT>(in_plane, (size_t)(16 * i + ko) * kHead + v0);
    else raw[i] = Row8<SDT>{};
  }
  void* out_plane = state_out_plane<SDT>(p, n, h);

  if (has_token) {
    const size_t tok = ((size_t)t0 * p.H + h) * kHead;
    const size_t tqk = ((size_t)t0 * p.H_qk + hqk) * kHead;
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(p.q) + tqk;
    const uint16_t* k16 = reinterpret_cast<const uint16_t*>(p.k) + tqk;
    float qh[kIters], kh[kIters], eg[kIters];
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int kk = 16 * i + ko;
      qh[i] = bf16_bits_to_f32(q16[kk]);
      kh[i] = bf16_bits_to_f32(k16[kk]);
      const float gr = GF32 ? reinterpret_cast<const float*>(p.g_raw)[tok + kk]
                            : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.g_raw)[tok + kk]);
      eg[i] = __expf(p.lower_bound * sigmoid(gr));
      sq += qh[i] * qh[i];
      sk += kh[i] * kh[i];
    }
    const size_t bidx = (size_t)t0 * p.H + h;
    const float braw = p.beta_dtype == kF32 ? reinterpret_cast<const float*>(p.beta_raw)[bidx]
                                            : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.beta_raw)[bidx]);
    const uint4 vw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.v) + tok + v0);
    const uint32_t v32[4] = {vw.x, vw.y, vw.z, vw.w};
    const float rq = rsqrtf(sum16(sq) + 1e-6f) * p.scale;  // scale folded into q-hat
    const float rk = rsqrtf(sum16(sk) + 1e-6f);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      qh[i] *= rq;
      kh[i] *= rk;
    }
    const float beta = sigmoid(braw);

    // u = D k-hat for the lane's eight columns.
    float pu[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const float w = eg[i] * kh[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) pu[j] += row8_get<SDT>(raw[i], j) * w;
    }
    float c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float vj = __uint_as_float((j & 1) ? (v32[j >> 1] & 0xffff0000u) : (v32[j >> 1] << 16));
      c[j] = beta * (vj - sum16(pu[j]));
    }
    // Update, store each key row as soon as it is done, and accumulate o = S q-hat.
    float po[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = row8_get<SDT>(raw[i], j) * eg[i] + c[j] * kh[i];
        po[j] += x[j] * qh[i];
      }
      if (out_plane) store_row8<SDT>(out_plane, (size_t)(16 * i + ko) * kHead + v0, x);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) po[j] = sum16(po[j]);
    if (ko == 0) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)__builtin_bit_cast(uint16_t, to_bf16(po[2 * j])) |
               ((uint32_t)__builtin_bit_cast(uint16_t, to_bf16(po[2 * j + 1])) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + tok + v0) = uint4{w[0], w[1], w[2], w[3]};
    }
  } else if (out_plane) {
    // No token: the state is written back as read (zero when nothing was read).
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(out_plane) +
                                            ((size_t)(16 * i + ko) * kHead + v0) * elem_size<SDT>());
#pragma unroll
      for (int w = 0; w < (SDT == kF32 ? 2 : 1); ++w) dst[w] = raw[i].w[w];
    }
  }
}

// K-first planes with a 2-byte state. A 128-byte line holds 64 columns of one key row, so
// eight lanes cover a line and every load reads eight whole rows. Wave w owns columns
// 64 (w & 1) .. +63 and key rows 64 (w >> 1) .. +63; lane (vo = lane & 7, ko = lane >> 3)
// holds the eight columns 64 (w & 1) + 8 vo .. +7 of rows 64 (w >> 1) + 8 i + ko
// (i = 0..7). The sums over k (u and o) run over the lane's eight rows, then over the
// eight lanes of its column group, then over the two waves of its column half (LDS).
template <int SDT, bool GF32>
__global__ __launch_bounds__(256) void decode_kfirst2_kernel(Plan p) {
  static_assert(SDT != kF32, "2-byte states only");
  __shared__ float part[2][2][kHead];  // [u, o][key half][column]
  const int n = blockIdx.x / p.H;
  const int h = blockIdx.x - n * p.H;
  const int hqk = __builtin_amdgcn_readfirstlane(h / p.group);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int vo = lane & 7, ko = lane >> 3;
  const int half = wave >> 1;                        // key half of this wave
  const int c0 = 64 * (wave & 1) + 8 * vo;           // first of the lane's columns
  const int r0 = 64 * half + ko;                     // the lane's rows are r0 + 8 i
  const int t0 = __builtin_amdgcn_readfirstlane(p.d_cu[n]);
  const bool has_token = __builtin_amdgcn_readfirstlane(p.d_cu[n + 1]) > t0;

  const void* in_plane = state_in_plane<SDT>(p, n, h);
  Row8<SDT> raw[kIters];
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    if (in_plane) raw[i] = load_row8<SDT>(in_plane, (size_t)(r0 + 8 * i) * kHead + c0);
    else raw[i] = Row8<SDT>{};
  }
  void* out_plane = state_out_plane<SDT>(p, n, h);

  if (has_token) {  // the same for the whole workgroup: its barriers are reached by all
    const size_t tok = ((size_t)t0 * p.H + h) * kHead;
    const size_t tqk = ((size_t)t0 * p.H_qk + hqk) * kHead;
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(p.q) + tqk;
    const uint16_t* k16 = reinterpret_cast<const uint16_t*>(p.k) + tqk;
    // Norms over all 128 keys: two keys per lane, summed over the wave.
    const uint32_t qw = *reinterpret_cast<const uint32_t*>(q16 + 2 * lane);
    const uint32_t kw = *reinterpret_cast<const uint32_t*>(k16 + 2 * lane);
    float sq = bf16_bits_to_f32(qw & 0xffffu) * bf16_bits_to_f32(qw & 0xffffu) +
               bf16_bits_to_f32(qw >> 16) * bf16_bits_to_f32(qw >> 16);
    float sk = bf16_bits_to_f32(kw & 0xffffu) * bf16_bits_to_f32(kw & 0xffffu) +
               bf16_bits_to_f32(kw >> 16) * bf16_bits_to_f32(kw >> 16);
    sq = sum64(sq);
    sk = sum64(sk);
    const float rq = rsqrtf(sq + 1e-6f) * p.scale;  // scale folded into q-hat
    const float rk = rsqrtf(sk + 1e-6f);
    float qh[kIters], kh[kIters], eg[kIters];
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int r = r0 + 8 * i;
      qh[i] = bf16_bits_to_f32(q16[r]) * rq;
      kh[i] = bf16_bits_to_f32(k16[r]) * rk;
      const float gr = GF32 ? reinterpret_cast<const float*>(p.g_raw)[tok + r]
                            : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.g_raw)[tok + r]);
      eg[i] = __expf(p.lower_bound * sigmoid(gr));
    }
    const size_t bidx = (size_t)t0 * p.H + h;
    const float braw = p.beta_dtype == kF32 ? reinterpret_cast<const float*>(p.beta_raw)[bidx]
                                            : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.beta_raw)[bidx]);
    const float beta = sigmoid(braw);
    const uint4 vw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.v) + tok + c0);
    const uint32_t v32[4] = {vw.x, vw.y, vw.z, vw.w};

    // u = D k-hat for the lane's columns: own rows, the column group, the two key halves.
    float pu[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const float w = eg[i] * kh[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) pu[j] += row8_get<SDT>(raw[i], j) * w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) pu[j] = add_xor32(add_xor16(add_xor8(pu[j])));
    if (ko == 0)
#pragma unroll
      for (int j = 0; j < 8; ++j) part[0][half][c0 + j] = pu[j];
    __syncthreads();
    float c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float vj = __uint_as_float((j & 1) ? (v32[j >> 1] & 0xffff0000u) : (v32[j >> 1] << 16));
      c[j] = beta * (vj - (part[0][0][c0 + j] + part[0][1][c0 + j]));
    }
    // Update, store each key row as soon as it is done, and accumulate o = S q-hat.
    float po[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = row8_get<SDT>(raw[i], j) * eg[i] + c[j] * kh[i];
        po[j] += x[j] * qh[i];
      }
      if (out_plane) store_row8<SDT>(out_plane, (size_t)(r0 + 8 * i) * kHead + c0, x);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) po[j] = add_xor32(add_xor16(add_xor8(po[j])));
    if (ko == 0)
#pragma unroll
      for (int j = 0; j < 8; ++j) part[1][half][c0 + j] = po[j];
    __syncthreads();
    if (half == 0 && ko == 0) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = part[1][0][c0 + 2 * j] + part[1][1][c0 + 2 * j];
        const float b = part[1][0][c0 + 2 * j + 1] + part[1][1][c0 + 2 * j + 1];
        w[j] = (uint32_t)__builtin_bit_cast(uint16_t, to_bf16(a)) |
               ((uint32_t)__builtin_bit_cast(uint16_t, to_bf16(b)) << 16);
      }
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + tok + c0) = uint4{w[0], w[1], w[2], w[3]};
    }
  } else if (out_plane) {
    // No token: the state is written back as read (zero when nothing was read).
#pragma unroll
    for (int i = 0; i < kIters; ++i)
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(out_plane) +
                                ((size_t)(r0 + 8 * i) * kHead + c0) * elem_size<SDT>()) = raw[i].w[0];
  }
}

template <int SDT>
int launch_sdt(const Plan& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(p.N * p.H);
  if (p.kfirst) {
    if constexpr (SDT == kF32) {  // four lanes already cover a line
      if (p.g_dtype == kF32)
        hipExtLaunchKernelGGL((decode_kfirst_kernel<SDT, true>), grid, dim3(256), 0, s, e0, e1, 0, p);
      else
        hipExtLaunchKernelGGL((decode_kfirst_kernel<SDT, false>), grid, dim3(256), 0, s, e0, e1, 0, p);
    } else if (p.g_dtype == kF32) {
      hipExtLaunchKernelGGL((decode_kfirst2_kernel<SDT, true>), grid, dim3(256), 0, s, e0, e1, 0, p);
    } else {
      hipExtLaunchKernelGGL((decode_kfirst2_kernel<SDT, false>), grid, dim3(256), 0, s, e0, e1, 0, p);
    }
  } else if (p.g_dtype == kF32) {
    hipExtLaunchKernelGGL((decode_kernel<SDT, true>), grid, dim3(256), 0, s, e0, e1, 0, p);
  } else {
    hipExtLaunchKernelGGL((decode_kernel<SDT, false>), grid, dim3(256), 0, s, e0, e1, 0, p);
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_decode(const Plan& p, void* stream, void* start, void* stop) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t e0 = reinterpret_cast<hipEvent_t>(start), e1 = reinterpret_cast<hipEvent_t>(stop);
  switch (p.state_dtype) {
    case kF16: return launch_sdt<kF16>(p, s, e0, e1);
    case kBF16: return launch_sdt<kBF16>(p, s, e0, e1);
    default: return launch_sdt<kF32>(p, s, e0, e1);
  }
}

}  // namespace kda
