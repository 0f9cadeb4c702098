// Chunk-parallel prep kernel for chunkwise KDA prefill on gfx950.
//
// Each (chunk, head) item fuses the pre-processing the pages describe as a separate pack
// pass (aiter PR 4741, Optimizations Applied: q/k L2 norm, lower-bounded sigmoid gate,
// beta sigmoid, zero padding as an exact no-op) with the chunk-parallel prep (same page,
// Summary: the first of its two kernels, one program per chunk):
//
//   G      inclusive in-chunk cumsum of g = lb * sigmoid(g_raw), per key channel;
//          padding rows have g = 0 so they carry the last valid row's G
//   A      A[r,i] = beta_r sum_c k_r k_i e^{G_r - G_i}          (i < r)
//   P      P[r,i] = scale sum_c q_r k_i e^{G_r - G_i}           (i <= r)
//   T      (I + A)^{-1}, unit lower triangular, fp32: diagonal 16x16 blocks by forward
//          substitution, the off-diagonal block -T11 A10 T00 on fp32 MFMA
//   W, U   T diag(beta) (k * e^G),  T diag(beta) v; the record holds -W, so that the
//          scan's Delta = U - W S^T is an MFMA accumulation started from U
//   Q, K   scale * q * e^G,  k * e^{G_C - G};  E = e^{G_C}
//
// A and P use a bounded factorisation of the decay (same page, Optimizations Applied:
// the split path's bounded construction, NaN-free to 640 nats): rows are grouped in
// blocks of REF rows and row r of block b uses the block's first row m_b as reference,
// e^{G_r - G_i} = e^{G_r - G_{m_b}} e^{G_{m_b} - G_i}. REF is chosen on the host so
// that (REF - 1) |lower_bound| <= 80, which keeps every factor inside e^{+-80} and so
// inside fp32/bf16 range; factors of earlier rows are <= 1 and may only underflow.
// The products run on bf16 MFMA with hi/lo operand splits and fp32 accumulation.
//
// Organisation: a persistent grid (two workgroups per CU) walks the items; each
// workgroup loads the next item's inputs while it computes the current one. Eight waves
// share an item, so each SIMD holds four waves to cover the latency of the item's phases.
// Thread (wave w, lane l) owns rows 4w .. 4w+3 and key/value channels 2l, 2l+1, so the
// in-chunk cumsum is mostly in registers and transposed tiles are written 8 bytes at a
// time. Output: one record per (head, chunk) in the scan's MFMA fragment order.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int LDA = 136;   // bf16 per row of a [32][128] operand tile (16-byte pad)
constexpr int LDT = 40;    // bf16 per row of a transposed [128][32] tile
constexpr int LDF = 36;    // fp32 per row of the [32][32] A / P / T tiles

constexpr int kWaves = kThreadsPrep / 64;  // waves per item
constexpr int kRows = kChunk / kWaves;      // rows per wave
static_assert(kRows == 4, "the thread layout below is written for four rows per wave");

// Region A: small per-item tiles.
constexpr int kOffBeta = 0;                     // fp32 [32]
constexpr int kOffA = kOffBeta + 32 * 4;        // fp32 [32][LDF]
constexpr int kOffTot = kOffA;                  // fp32 [8][128] per-wave cumsum totals,
                                                // dead before A is written
constexpr int kOffP = kOffA + 32 * LDF * 4;     // fp32 [32][LDF]
constexpr int kOffT = kOffP + 32 * LDF * 4;     // fp32 [32][LDF] T = (I + A)^{-1}
constexpr int kOffM = kOffT + 32 * LDF * 4;     // fp32 [16][LDF] scratch of the block solve
constexpr int kOffGref = kOffM + 16 * LDF * 4;  // fp32 [32/REF + 1][128] reference rows, then G_C
// Region X (after Gref): two views.
constexpr int kTileA = 32 * LDA * 2;            // 8704 B
constexpr int kTileT = 128 * LDT * 2;           // 10240 B
constexpr int kTileTT = 32 * LDT * 2;           // 2560 B
constexpr int kFactorBytes = 6 * kTileA;        // L_k hi/lo, L_q hi/lo, R hi/lo
constexpr int kProductBytes = 4 * kTileT + kTileA + 2 * kTileTT;  // KG hi/lo, K^T, v^T, Q, T' hi/lo

// REF = 16 (two row blocks) builds both blocks' right factors at once: block 1 over all
// 32 rows, block 0 over rows 0..15 (half a tile), next to the left factors.
constexpr int factor_bytes(int ref) { return ref == 16 ? 7 * kTileA : kFactorBytes; }
constexpr int gref_bytes(int ref) { return (32 / ref + 1) * 128 * 4; }
constexpr int off_x(int ref) { return (kOffGref + gref_bytes(ref) + 255) / 256 * 256; }
constexpr int lds_bytes(int ref) {
  return off_x(ref) + (factor_bytes(ref) > kProductBytes ? factor_bytes(ref) : kProductBytes);
}
static_assert(2 * lds_bytes(16) <= 160 * 1024, "two workgroups per CU at the default block");
static_assert(kWaves * 128 * 4 <= 32 * LDF * 4, "the cumsum totals fit the A tile");

// Offsets inside region X.
constexpr int xLKh = 0, xLKl = xLKh + kTileA, xLQh = xLKl + kTileA, xLQl = xLQh + kTileA, xRh = xLQl + kTileA,
              xRl = xRh + kTileA;
// REF = 16: R of block 1 at xRh / xRl (32 rows), R of block 0 (16 rows each) after them.
constexpr int xR0h = xRl + kTileA, xR0l = xR0h + kTileA / 2;
constexpr int xKGh = 0, xKGl = xKGh + kTileT, xKt = xKGl + kTileT, xVt = xKt + kTileT, xQs = xVt + kTileT,
              xTh = xQs + kTileA, xTl = xTh + kTileTT;

// Inputs of one item held by one thread: rows 4w .. 4w+3, channels 2l, 2l+1. The words
// are kept as loaded and widened where they are used: arithmetic on a loaded value makes
// the compiler wait for that load (and for every load issued before it) right there.
struct Inputs {
  uint32_t q[4], k[4], v[4];  // two bf16 each
  uint32_t g[4][2];           // raw gate: two fp32, or two bf16 in word 0
  uint32_t bhi, blo;          // raw beta of row 4w + (lane & 3) (lanes 0..3 meaningful):
                              // upper and lower 16 bits of an fp32 value, or the bf16 twice
};

template <bool GF32>
__device__ __forceinline__ float2 gate_of(const uint32_t* g) {
  if constexpr (GF32) return make_float2(__uint_as_float(g[0]), __uint_as_float(g[1]));
  return make_float2(__uint_as_float(g[0] << 16), __uint_as_float(g[0] & 0xffff0000u));
}

struct Item {
  int cid, h, seq, t0, len;
};

__device__ __forceinline__ Item item_of(const Plan& p, int item) {
  Item it;
  it.cid = item / p.H;
  it.h = item - it.cid * p.H;
  // Uniform metadata, kept in scalar registers (see the scan's unit lookup).
  it.seq = __builtin_amdgcn_readfirstlane(p.d_table[2 * it.cid]);
  const int jc = __builtin_amdgcn_readfirstlane(p.d_table[2 * it.cid + 1]);
  it.t0 = __builtin_amdgcn_readfirstlane(p.d_cu[it.seq]) + kChunk * jc;
  it.len = min(kChunk, __builtin_amdgcn_readfirstlane(p.d_cu[it.seq + 1]) - it.t0);
  return it;
}

// Buffer descriptor over rows t0 .. t0 + len - 1 of head h of a [T][H][128] tensor with
// elem-byte elements: loads from rows past the sequence fall outside the range and return
// zero, which is the padding the method needs for q, k and v. The loads never depend on a
// branch, so the next item's loads stay in flight during compute.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, const Item& it, int H, int h, int elem) {
  const char* b = reinterpret_cast<const char*>(base) + ((size_t)it.t0 * H + h) * kHead * elem;
  const int bytes = it.len > 0 ? (it.len - 1) * H * kHead * elem + kHead * elem : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b), (short)0, bytes, kBufWord3);
}

// GVA: q and k have H_qk < H heads and value head h reads q/k head h / (H / H_qk). It is
// a separate instantiation so that the one-to-one case keeps a single set of row offsets
// (the prep kernel has no registers to spare).
template <bool GF32, bool GVA>
__device__ __forceinline__ void load_inputs(const Plan& p, const Item& it, int w, int lane, Inputs& in) {
  const int H = p.H, Hqk = GVA ? p.H_qk : H;
  const int hqk = GVA ? __builtin_amdgcn_readfirstlane(it.h / p.group) : it.h;
  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(p.q, it, Hqk, hqk, 2), rk = rows_rsrc(p.k, it, Hqk, hqk, 2),
                               rv = rows_rsrc(p.v, it, H, it.h, 2), rg = rows_rsrc(p.g_raw, it, H, it.h, GF32 ? 4 : 2);
  const int row2 = H * kHead * 2;  // bytes per token row of a 2-byte [T][H][128] tensor
  // The whole offset goes in the vector operand: the range check covers only that part.
  // The cache policy is an instruction immediate: one copy of the loads per policy, chosen
  // by a uniform branch (both copies issue the same loads, so no wait is forced at the join).
  auto issue = [&](auto policy) {
    constexpr int kPolicy = decltype(policy)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vo = (4 * w + i) * row2 + lane * 4;
      const int vqk = GVA ? (4 * w + i) * Hqk * kHead * 2 + lane * 4 : vo;
      in.q[i] = __builtin_amdgcn_raw_buffer_load_b32(rq, vqk, 0, kPolicy);
      in.k[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, vqk, 0, kPolicy);
      in.v[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo, 0, kPolicy);
      if constexpr (GF32) {
        const auto g = __builtin_amdgcn_raw_buffer_load_b64(rg, 2 * vo, 0, kPolicy);
        in.g[i][0] = g[0];
        in.g[i][1] = g[1];
      } else {
        in.g[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rg, vo, 0, kPolicy);
      }
    }
  };
  if (p.stream_inputs) issue(std::integral_constant<int, kStreamLoad>{});
  else issue(std::integral_constant<int, 0>{});
  // Raw beta of row 4w + (lane & 3) as two 2-byte loads (the upper and lower halves of
  // an fp32 value, or the bf16 value twice), so no branch holds the loads back and no
  // byte outside the element is read.
  const int brow = min(it.t0 + 4 * w + (lane & 3), p.T - 1);
  const size_t bidx = (size_t)brow * H + it.h;
  const bool bf = p.beta_dtype != kF32;
  const char* bb = reinterpret_cast<const char*>(p.beta_raw);
  in.bhi = *reinterpret_cast<const uint16_t*>(bb + (bf ? bidx * 2 : bidx * 4 + 2));
  in.blo = *reinterpret_cast<const uint16_t*>(bb + (bf ? bidx * 2 : bidx * 4));
}

__device__ __forceinline__ float lo16(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi16(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
// The gate cumsum is kept in base 2 (G2 = G log2 e), so every decay factor e^{G_a - G_b}
// is one subtraction and the hardware's 2^x. Its results below the fp32 normal range
// may flush to zero, which only drops terms smaller than 2^-126 of their sum.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float sigm(float x) { return rcp(1.0f + ex2(-kLog2e * x)); }

// Two floats to packed bf16 (round to nearest even; a in the low half).
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
// Two floats split into packed bf16 hi and lo words, x = hi + lo to about 2^-17 |x|.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt_pk(a, b);
  lo = cvt_pk(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ bf16x8 ld_frag(const char* lds, int off) {
  return *reinterpret_cast<const bf16x8*>(lds + off);
}

__device__ __forceinline__ bf16x8 ld_frag_2x4(const char* lds, int off0, int off1) {
  const uint2 a = *reinterpret_cast<const uint2*>(lds + off0);
  const uint2 b = *reinterpret_cast<const uint2*>(lds + off1);
  const uint4 r = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, r);
}

// Write channels 2l and 2l + 1 (rows 4w .. 4w+3 each, packed two rows a word) to a
// transposed [128][LDT] tile. Lanes with bit 3 set write the odd channel first, so that
// the 16 lanes an 8-byte store serves at once spread over twice as many LDS banks.
__device__ __forceinline__ void st_cols(char* lds, int off, int lane, int w, const uint32_t* a, const uint32_t* b) {
  const int sw = (lane >> 3) & 1;
  const int c = 2 * lane;
  const uint2 x = sw ? uint2{b[0], b[1]} : uint2{a[0], a[1]};
  const uint2 y = sw ? uint2{a[0], a[1]} : uint2{b[0], b[1]};
  *reinterpret_cast<uint2*>(lds + off + ((c + sw) * LDT + 4 * w) * 2) = x;
  *reinterpret_cast<uint2*>(lds + off + ((c + 1 - sw) * LDT + 4 * w) * 2) = y;
}

// Sum 8 per-lane values over the 64 lanes of a wave. Each of the first three steps keeps
// half of the values and adds the partner's copy of that half; every exchange is a lane
// permutation on the vector ALU (no LDS round trip). Steps over lane bits 5 and 4 swap a
// pair of registers between half-waves (v_permlane32_swap) and between 16-lane rows
// (v_permlane16_swap), which moves both halves at once; bit 3 pairs lanes across each row
// (row rotate by 8). The last three steps sum each group of eight lanes: lane i with
// 7 - i (half-row mirror), then the quad permutes. Lane L ends up holding the total of
// value index 4*b5 + 2*b4 + b3 (b = bits of L).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuadXor2 = 0x4e;  // quad_perm [2, 3, 0, 1]
constexpr int kDppQuadXor1 = 0xb1;  // quad_perm [1, 0, 3, 2]

__device__ __forceinline__ float wave_sum8(const float* x, int lane) {
  const bool b3 = lane & 8;
  float y[4], z[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // Lanes 0..31 keep value j, lanes 32..63 value 4 + j.
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]), __float_as_uint(x[4 + j]), false, false);
    y[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // Even rows keep y[j], odd rows y[2 + j].
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[j]), __float_as_uint(y[2 + j]), false, false);
    z[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const float keep = b3 ? z[1] : z[0];
  const float send = b3 ? z[0] : z[1];
  float s = keep + dpp<kDppRowRor8>(send);
  s += dpp<kDppRowHalfMirror>(s);
  s += dpp<kDppQuadXor2>(s);
  s += dpp<kDppQuadXor1>(s);
  return s;
}

__device__ __forceinline__ float bcast(float x, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}

__device__ __forceinline__ int lane_of_sum(int v) { return ((v >> 2) & 1) * 32 + ((v >> 1) & 1) * 16 + (v & 1) * 8; }

// Processes item it from its inputs in, and once they are dead (after staging) loads
// the inputs of item next into in.
template <int REF, bool GF32, bool GVA>
__device__ void process_item(const Plan& p, const Item& it, Inputs& in, const Item& next, char* lds, int w_in,
                             int lane) {
  // The wave index is uniform, so everything derived from it (fragment and tile choices,
  // LDS offsets, branch masks) is scalar. Redefining it here for the compiler keeps those
  // values from being hoisted out of the item loop, where they would stay live across
  // the whole kernel and spill scalar registers into vector lanes.
  int w = w_in;
  asm volatile("" : "+s"(w));
  constexpr int NB = 32 / REF;
  constexpr int OX = off_x(REF);
  float* tot = reinterpret_cast<float*>(lds + kOffTot);
  float* betas = reinterpret_cast<float*>(lds + kOffBeta);
  float* As = reinterpret_cast<float*>(lds + kOffA);
  float* Ps = reinterpret_cast<float*>(lds + kOffP);
  float* Ts = reinterpret_cast<float*>(lds + kOffT);
  float* Ms = reinterpret_cast<float*>(lds + kOffM);
  float* Gref = reinterpret_cast<float*>(lds + kOffGref);
  char* X = lds + OX;
  const int tid = threadIdx.x;
  const int c0 = 2 * lane;
  const int len = it.len;
  char* rec = reinterpret_cast<char*>(p.ws) + ((size_t)it.h * p.n_chunks + it.cid) * kRecBytes;

  // ---------------------------------------------------------------- elementwise
  float qn[4][2], kn[4][2], G[4][2];
  {
    float sq[8];
    // Rows past the sequence were loaded as zeros.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qn[i][0] = lo16(in.q[i]);
      qn[i][1] = hi16(in.q[i]);
      kn[i][0] = lo16(in.k[i]);
      kn[i][1] = hi16(in.k[i]);
      sq[i] = qn[i][0] * qn[i][0] + qn[i][1] * qn[i][1];
      sq[4 + i] = kn[i][0] * kn[i][0] + kn[i][1] * kn[i][1];
    }
    // Each lane takes the inverse norm of the row sum it holds; rows read theirs back.
    const float rs = __builtin_amdgcn_rsqf(wave_sum8(sq, lane) + 1e-6f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float rq = bcast(rs, lane_of_sum(i));
      const float rk = bcast(rs, lane_of_sum(4 + i));
      qn[i][0] *= rq; qn[i][1] *= rq;
      kn[i][0] *= rk; kn[i][1] *= rk;
    }
    // Gate per key channel and its cumsum over this wave's rows (padding rows: g = 0),
    // in base 2.
    const float lb2 = p.lower_bound * kLog2e;
    float run0 = 0.f, run1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = 4 * w + i < len;
      const float2 g = gate_of<GF32>(in.g[i]);
      run0 += valid ? lb2 * sigm(g.x) : 0.f;
      run1 += valid ? lb2 * sigm(g.y) : 0.f;
      G[i][0] = run0;
      G[i][1] = run1;
    }
    *reinterpret_cast<float2*>(tot + w * 128 + c0) = make_float2(run0, run1);
    const float braw = __uint_as_float((in.bhi << 16) | (p.beta_dtype != kF32 ? 0u : in.blo));
    if (lane < 4) betas[4 * w + lane] = (4 * w + lane < len) ? sigm(braw) : 0.f;
  }
  __syncthreads();
  {
    // Add the totals of the earlier waves (in wave order), then publish reference rows.
    float o0 = 0.f, o1 = 0.f;
    for (int ww = 0; ww < w; ++ww) {
      const float2 t = *reinterpret_cast<const float2*>(tot + ww * 128 + c0);
      o0 += t.x;
      o1 += t.y;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      G[i][0] += o0;
      G[i][1] += o1;
      const int r = 4 * w + i;
      if (r % REF == 0) *reinterpret_cast<float2*>(Gref + (r / REF) * 128 + c0) = make_float2(G[i][0], G[i][1]);
    }
    if (w == kWaves - 1) *reinterpret_cast<float2*>(Gref + NB * 128 + c0) = make_float2(G[3][0], G[3][1]);  // G_C
  }
  __syncthreads();

  // ---------------------------------------------------------------- A and P on MFMA
  // At REF = 16 the record's Q, K and KG tiles are formed here from the decay factors
  // (e^{G_r} = e^{G_r - G_m} e^{G_m}, e^{G_C - G_r} = e^{G_C - G_16} e^{G_16 - G_r}, every
  // factor inside the fp32 range) and kept packed until staging.
  [[maybe_unused]] uint32_t qs[4], kg0h[2], kg0l[2], kg1h[2], kg1l[2], kt0[2], kt1[2];
  {
    [[maybe_unused]] float kgv[4][2];
    // At REF = 16 the wave's 4 rows share one reference row (0 or 16).
    const float2 gw = *reinterpret_cast<const float2*>(Gref + (REF == 16 ? w / 4 : 0) * 128 + c0);
    [[maybe_unused]] float em0 = 0.f, em1 = 0.f;
    if constexpr (REF == 16) {
      em0 = ex2(gw.x);  // e^{G_m}, m = 0 or 16: inside the fp32 range at REF = 16
      em1 = ex2(gw.y);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * w + i;
      // Below REF = 16 the rows of the lower half first take row 16 as their reference
      // (the pivot of the off-diagonal tile, see below).
      const int gi = REF == 16 ? 0 : (w >= kWaves / 2 ? 16 / REF : r / REF);
      const float2 gm = REF == 16 ? gw : *reinterpret_cast<const float2*>(Gref + gi * 128 + c0);
      const float e0 = ex2(G[i][0] - gm.x), e1 = ex2(G[i][1] - gm.y);  // in [e^-80, 1]
      uint32_t kh, kl, qh, ql;
      split2(kn[i][0] * e0, kn[i][1] * e1, kh, kl);
      split2(qn[i][0] * e0, qn[i][1] * e1, qh, ql);
      const int o = (r * LDA + c0) * 2;
      *reinterpret_cast<uint32_t*>(X + xLKh + o) = kh;
      *reinterpret_cast<uint32_t*>(X + xLKl + o) = kl;
      *reinterpret_cast<uint32_t*>(X + xLQh + o) = qh;
      *reinterpret_cast<uint32_t*>(X + xLQl + o) = ql;
      if constexpr (REF == 16) {
        const float eg0 = e0 * em0, eg1 = e1 * em1;  // e^{G_r}
        qs[i] = cvt_pk(p.scale * qn[i][0] * eg0, p.scale * qn[i][1] * eg1);
        kgv[i][0] = kn[i][0] * eg0;
        kgv[i][1] = kn[i][1] * eg1;
      }
    }
    if constexpr (REF == 16) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        split2(kgv[2 * j][0], kgv[2 * j + 1][0], kg0h[j], kg0l[j]);
        split2(kgv[2 * j][1], kgv[2 * j + 1][1], kg1h[j], kg1l[j]);
      }
    }
  }
  const int l16 = lane & 15, g4 = lane >> 4;
  // One tile job for each of waves 0..5: (row tile jr, column tile jc, matrix A = 0 or
  // P = 1): wave 0 (0,0,A), 1 (0,0,P), 2 (1,1,A), 3 (1,1,P), 4 (1,0,A), 5 (1,0,P). Waves 6
  // and 7 write the zero tile (0,1) of A and of P.
  const bool has_job = w < 6;
  const int jr = w >= 2 ? 1 : 0;
  const int jc = (w == 2 || w == 3) ? 1 : 0;
  const int mat = w & 1;
  f32x4 acc = zero4();
  if constexpr (REF == 16) {
    // Both row blocks at once. Row tile t is exactly row block t (reference row 16t),
    // so every job's rows are inside its block and no row masking is needed. Right
    // factors: block 1 over all rows (k_i e^{G_16 - G_i}), block 0 over rows 0..15
    // (k_i e^{G_0 - G_i}); the exponent is minus the left factor's for the rows of the
    // factor's own block, and for block 1 on rows 0..15 it is block 0's plus G_16 - G_0.
    {
      const float2 g0 = *reinterpret_cast<const float2*>(Gref + c0);
      const float2 g16 = *reinterpret_cast<const float2*>(Gref + 128 + c0);
      const float2 gc = *reinterpret_cast<const float2*>(Gref + NB * 128 + c0);
      const float d0 = ex2(g16.x - g0.x), d1 = ex2(g16.y - g0.y);  // e^{G_16 - G_0} <= 1
      const float c0e = ex2(gc.x - g16.x), c1e = ex2(gc.y - g16.y);  // e^{G_C - G_16} >= e^-80
      const bool upper = w < kWaves / 2;  // rows 0..15
      float ktv[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * w + i;
        const float2 gm = upper ? g0 : g16;
        const float r0 = ex2(gm.x - G[i][0]), r1 = ex2(gm.y - G[i][1]);  // own block, <= e^80
        uint32_t h, l;
        const int o = (r * LDA + c0) * 2;
        float b0 = r0, b1 = r1;  // e^{G_16 - G_r}
        if (upper) {
          split2(kn[i][0] * r0, kn[i][1] * r1, h, l);
          *reinterpret_cast<uint32_t*>(X + xR0h + o) = h;
          *reinterpret_cast<uint32_t*>(X + xR0l + o) = l;
          b0 = r0 * d0;  // <= 1
          b1 = r1 * d1;
        }
        split2(kn[i][0] * b0, kn[i][1] * b1, h, l);
        *reinterpret_cast<uint32_t*>(X + xRh + o) = h;
        *reinterpret_cast<uint32_t*>(X + xRl + o) = l;
        ktv[i][0] = kn[i][0] * (b0 * c0e);  // k e^{G_C - G_r}
        ktv[i][1] = kn[i][1] * (b1 * c1e);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        kt0[j] = cvt_pk(ktv[2 * j][0], ktv[2 * j + 1][0]);
        kt1[j] = cvt_pk(ktv[2 * j][1], ktv[2 * j + 1][1]);
      }
    }
    __syncthreads();
    if (has_job) {
      const int row = 16 * jr + l16;
      const int col = 16 * jc + l16;
      const int rb_h = (jr == 0) ? xR0h : xRh;  // right factors of the row tile's block
      const int rb_l = (jr == 0) ? xR0l : xRl;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ea = (row * LDA + 32 * kk + 8 * g4) * 2;
        const int eb = (col * LDA + 32 * kk + 8 * g4) * 2;
        const bf16x8 bh = ld_frag(X, rb_h + eb), bl = ld_frag(X, rb_l + eb);
        const bf16x8 ah = ld_frag(X, (mat ? xLQh : xLKh) + ea), al = ld_frag(X, (mat ? xLQl : xLKl) + ea);
        acc = mfma(ah, bh, acc);
        acc = mfma(ah, bl, acc);
        acc = mfma(al, bh, acc);
      }
    }
    __syncthreads();
  } else {
    // Below REF = 16 the two diagonal 16 x 16 tiles are built from REF-row sub-blocks and
    // the off-diagonal tile (rows 16..31, columns 0..15) through row 16: for r >= 16 > i,
    // e^{G_r - G_i} = e^{G_r - G_16} e^{G_16 - G_i}, both factors <= 1 whatever the decay.
    // The diagonal jobs (waves 0..3) accumulate over the sub-block rounds; the
    // off-diagonal jobs (waves 4 and 5) take one round first.
    const float2 g16 = *reinterpret_cast<const float2*>(Gref + (16 / REF) * 128 + c0);
    if (w < kWaves / 2) {  // right factors of the off-diagonal tile: rows 0..15, through row 16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * w + i;
        uint32_t h, l;
        split2(kn[i][0] * ex2(g16.x - G[i][0]), kn[i][1] * ex2(g16.y - G[i][1]), h, l);  // <= 1
        const int o = (r * LDA + c0) * 2;
        *reinterpret_cast<uint32_t*>(X + xRh + o) = h;
        *reinterpret_cast<uint32_t*>(X + xRl + o) = l;
      }
    }
    __syncthreads();
    if (w == 4 || w == 5) {
      const int row = 16 + l16, col = l16;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ea = (row * LDA + 32 * kk + 8 * g4) * 2;
        const int eb = (col * LDA + 32 * kk + 8 * g4) * 2;
        const bf16x8 bh = ld_frag(X, xRh + eb), bl = ld_frag(X, xRl + eb);
        const bf16x8 ah = ld_frag(X, (mat ? xLQh : xLKh) + ea), al = ld_frag(X, (mat ? xLQl : xLKl) + ea);
        acc = mfma(ah, bh, acc);
        acc = mfma(ah, bl, acc);
        acc = mfma(al, bh, acc);
      }
    }
    __syncthreads();
    if (w >= kWaves / 2) {  // left factors of the lower half with their own sub-block references
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * w + i;
        const float2 gm = *reinterpret_cast<const float2*>(Gref + (r / REF) * 128 + c0);
        const float e0 = ex2(G[i][0] - gm.x), e1 = ex2(G[i][1] - gm.y);  // in [e^-80, 1]
        uint32_t kh, kl, qh, ql;
        split2(kn[i][0] * e0, kn[i][1] * e1, kh, kl);
        split2(qn[i][0] * e0, qn[i][1] * e1, qh, ql);
        const int o = (r * LDA + c0) * 2;
        *reinterpret_cast<uint32_t*>(X + xLKh + o) = kh;
        *reinterpret_cast<uint32_t*>(X + xLKl + o) = kl;
        *reinterpret_cast<uint32_t*>(X + xLQh + o) = qh;
        *reinterpret_cast<uint32_t*>(X + xLQl + o) = ql;
      }
    }
    // Round b: sub-block b of both halves at once (rows 16t + b REF .. + REF - 1).
    const int th = w >= kWaves / 2 ? 1 : 0;  // the half this wave's rows are in
    for (int b = 0; b < 16 / REF; ++b) {
      {
        const int mb = 16 * th + b * REF;
        const int lim = mb + REF - 1;  // right factors past the sub-block are 0
        const float2 gm = *reinterpret_cast<const float2*>(Gref + (mb / REF) * 128 + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * w + i;
          float x0 = 0.f, x1 = 0.f;
          if (r <= lim) {
            x0 = kn[i][0] * ex2(gm.x - G[i][0]);  // <= e^80
            x1 = kn[i][1] * ex2(gm.y - G[i][1]);
          }
          uint32_t h, l;
          split2(x0, x1, h, l);
          const int o = (r * LDA + c0) * 2;
          *reinterpret_cast<uint32_t*>(X + xRh + o) = h;
          *reinterpret_cast<uint32_t*>(X + xRl + o) = l;
        }
      }
      __syncthreads();
      if (w < 4) {  // the diagonal jobs: tile (jr, jr)
        const int mb = 16 * jr + b * REF;
        const int lim = mb + REF - 1;
        const int row = 16 * jr + l16;
        const bool rowin = (row >= mb) && (row <= lim);
        const int col = 16 * jr + l16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int ea = (row * LDA + 32 * kk + 8 * g4) * 2;
          const int eb = (col * LDA + 32 * kk + 8 * g4) * 2;
          const bf16x8 bh = ld_frag(X, xRh + eb), bl = ld_frag(X, xRl + eb);
          bf16x8 ah = ld_frag(X, (mat ? xLQh : xLKh) + ea), al = ld_frag(X, (mat ? xLQl : xLKl) + ea);
          if (!rowin) { ah = bf16x8{}; al = bf16x8{}; }
          acc = mfma(ah, bh, acc);
          acc = mfma(ah, bl, acc);
          acc = mfma(al, bh, acc);
        }
      }
      __syncthreads();
    }
  }
  // Masked, scaled tiles: A strictly lower times beta_r, P lower with diagonal. The tile
  // above the diagonal is written as zeros.
  if (has_job) {
    const int col = 16 * jc + l16;
    float* dst = mat ? Ps : As;
    const int diag = mat;  // P keeps its diagonal, A does not
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * jr + 4 * g4 + i;
      const float sc = mat ? p.scale : betas[row];
      dst[row * LDF + col] = (col < row + diag) ? sc * acc[i] : 0.f;
    }
  } else {  // upper tile (0,1) of A (wave 6) and of P (wave 7)
    float* dst = (w == 6) ? As : Ps;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(4 * g4 + i) * LDF + 16 + l16] = 0.f;
  }

  // ---------------------------------------------------------------- staging
  // (the factor tiles are dead after the last barrier of the A and P phase)
  {
    const float2 gc = *reinterpret_cast<const float2*>(Gref + NB * 128 + c0);
    // Transposed tiles take rows in pairs: word j of a channel holds rows 2j, 2j + 1.
    uint32_t v0[2], v1[2];
    if constexpr (REF != 16) {
      float eg[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        eg[i][0] = ex2(G[i][0]);  // e^{G_r} <= 1
        eg[i][1] = ex2(G[i][1]);
        qs[i] = cvt_pk(p.scale * qn[i][0] * eg[i][0], p.scale * qn[i][1] * eg[i][1]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = 2 * j;
        split2(kn[i][0] * eg[i][0], kn[i + 1][0] * eg[i + 1][0], kg0h[j], kg0l[j]);
        split2(kn[i][1] * eg[i][1], kn[i + 1][1] * eg[i + 1][1], kg1h[j], kg1l[j]);
        // e^{G_C - G_r} <= 1
        kt0[j] = cvt_pk(kn[i][0] * ex2(gc.x - G[i][0]), kn[i + 1][0] * ex2(gc.x - G[i + 1][0]));
        kt1[j] = cvt_pk(kn[i][1] * ex2(gc.y - G[i][1]), kn[i + 1][1] * ex2(gc.y - G[i + 1][1]));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(X + xQs + ((4 * w + i) * LDA + c0) * 2) = qs[i];
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // padding rows of v were loaded as zeros
      const int i = 2 * j;
      v0[j] = (in.v[i] & 0xffffu) | (in.v[i + 1] << 16);
      v1[j] = (in.v[i] >> 16) | (in.v[i + 1] & 0xffff0000u);
    }
    st_cols(X, xKGh, lane, w, kg0h, kg1h);
    st_cols(X, xKGl, lane, w, kg0l, kg1l);
    st_cols(X, xKt, lane, w, kt0, kt1);
    st_cols(X, xVt, lane, w, v0, v1);
    if (w == kWaves - 1) *reinterpret_cast<float2*>(rec + kRecE + c0 * 4) = make_float2(ex2(gc.x), ex2(gc.y));
    // This item's inputs are dead: the next item's loads overlap the solve and W/U.
    load_inputs<GF32, GVA>(p, next, w, lane, in);
  }
  __syncthreads();

  // ---------------------------------------------------------------- solve + stores
  if (w == 0) {
    if (lane < 32) {
      // Diagonal 16x16 blocks of T = (I + A)^{-1}: lane -> (block, column j). Forward
      // substitution T[i][j] = [i == j] - sum_{j <= k < i} A[i][k] T[k][j], with the sum
      // split over four accumulators to shorten the dependent chain.
      const int blk = lane >> 4, j = lane & 15, base = 16 * blk;
      float tc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* Ai = As + (base + i) * LDF + base;
        float s0 = (i == j) ? 1.f : 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
        for (int k = 0; k < i; k += 4) {
          s0 = fmaf(-Ai[k], tc[k], s0);
          if (k + 1 < i) s1 = fmaf(-Ai[k + 1], tc[k + 1], s1);
          if (k + 2 < i) s2 = fmaf(-Ai[k + 2], tc[k + 2], s2);
          if (k + 3 < i) s3 = fmaf(-Ai[k + 3], tc[k + 3], s3);
        }
        tc[i] = (s0 + s1) + (s2 + s3);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) Ts[(base + i) * LDF + base + j] = tc[i];
    }
    // Off-diagonal block T10 = -T11 (A10 T00) on fp32 MFMA (16x16x4: lane l holds A[l%16]
    // [l/16] and B[l/16][l%16], D rows 4*(l/16) + i of column l%16). The diagonal blocks
    // were written by lanes 0..31 of this wave: wait for those LDS writes, and keep the
    // compiler from moving LDS accesses across the wait (the lanes exchange data).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    f32x4 m = zero4();
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      m = __builtin_amdgcn_mfma_f32_16x16x4f32(As[(16 + l16) * LDF + 4 * s4 + g4], Ts[(4 * s4 + g4) * LDF + l16], m,
                                               0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) Ms[(4 * g4 + i) * LDF + l16] = m[i];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    f32x4 t10 = zero4();
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      t10 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ts[(16 + l16) * LDF + 16 + 4 * s4 + g4], Ms[(4 * s4 + g4) * LDF + l16],
                                                 t10, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) Ts[(16 + 4 * g4 + i) * LDF + l16] = -t10[i];
  } else if (w <= 6) {
    // 18 fragments (Q: 8, K: 8, P: 2), three per wave on waves 1..6.
    for (int f = (w - 1) * 3; f < w * 3; ++f) {
      bf16x8 val;
      size_t dst;
      if (f < 8) {
        const int t = f >> 2, m = f & 3;
        const int row = 16 * t + l16;
        const int o0 = xQs + (row * LDA + 32 * m + 4 * g4) * 2;
        val = ld_frag_2x4(X, o0, o0 + 32);
        dst = kRecQ + (size_t)f * kFrag;
      } else if (f < 16) {
        const int kt = f - 8;
        const int krow = 16 * kt + l16;
        const int o0 = xKt + (krow * LDT + 4 * g4) * 2;
        val = ld_frag_2x4(X, o0, o0 + 32);
        dst = kRecK + (size_t)kt * kFrag;
      } else {
        const int t = f - 16;
        const float* Pr = Ps + (16 * t + l16) * LDF;
        const f32x4 a = {Pr[4 * g4], Pr[4 * g4 + 1], Pr[4 * g4 + 2], Pr[4 * g4 + 3]};
        const f32x4 b = {Pr[16 + 4 * g4], Pr[16 + 4 * g4 + 1], Pr[16 + 4 * g4 + 2], Pr[16 + 4 * g4 + 3]};
        val = pack8(a, b);
        dst = kRecP + (size_t)t * kFrag;
      }
      *reinterpret_cast<bf16x8*>(rec + dst + lane * 16) = val;
    }
  }
  __syncthreads();
  // T diag(beta) as hi/lo bf16 (rows r, column r'), zero above the diagonal.
  {
    // Thread: columns j, j + 1 of row i.
    const int i = tid >> 4, j = 2 * (tid & 15);
    const float x0 = (j <= i) ? Ts[i * LDF + j] * betas[j] : 0.f;
    const float x1 = (j + 1 <= i) ? Ts[i * LDF + j + 1] * betas[j + 1] : 0.f;
    uint32_t hi, lo;
    split2(x0, x1, hi, lo);
    *reinterpret_cast<uint32_t*>(X + xTh + (i * LDT + j) * 2) = hi;
    *reinterpret_cast<uint32_t*>(X + xTl + (i * LDT + j) * 2) = lo;
  }
  __syncthreads();

  // ---------------------------------------------------------------- W and U on MFMA
  // Wave w produces the W fragment (row tile t = w / 4, key block m = w % 4) and the U
  // fragment of value tile w.
  {
    const int t = w >> 2, m = w & 3;
    bf16x8 th[2], tl[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int rrow = 16 * tt + l16;
      th[tt] = ld_frag(X, xTh + (rrow * LDT + 8 * g4) * 2);
      tl[tt] = ld_frag(X, xTl + (rrow * LDT + 8 * g4) * 2);
    }
    // Row tile t's fragments read again by address: indexing th/tl with the wave's t
    // would become a chain of selects.
    const bf16x8 tht = ld_frag(X, xTh + ((16 * t + l16) * LDT + 8 * g4) * 2);
    const bf16x8 tlt = ld_frag(X, xTl + ((16 * t + l16) * LDT + 8 * g4) * 2);
    f32x4 dw[2];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int crow = 16 * (2 * m + q2) + l16;
      // W^T tile (key tile 2m + q2, t) = (k e^G)^T (T diag beta)^T: A = KG^T rows c,
      // B = T' rows r.
      const bf16x8 kh = ld_frag(X, xKGh + (crow * LDT + 8 * g4) * 2);
      const bf16x8 kl = ld_frag(X, xKGl + (crow * LDT + 8 * g4) * 2);
      f32x4 a = zero4();
      a = mfma(kh, tht, a);
      a = mfma(kh, tlt, a);
      a = mfma(kl, tht, a);
      dw[q2] = a;
    }
    // U tile (tt, w) = T' v: A = T' rows r, B = v columns.
    f32x4 du[2];
    {
      const bf16x8 vt = ld_frag(X, xVt + ((16 * w + l16) * LDT + 8 * g4) * 2);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 uu = zero4();
        uu = mfma(th[tt], vt, uu);
        uu = mfma(tl[tt], vt, uu);
        du[tt] = uu;
      }
    }
    *reinterpret_cast<bf16x8*>(rec + kRecW + (size_t)(t * 4 + m) * kFrag + lane * 16) = pack8(-dw[0], -dw[1]);
    *reinterpret_cast<bf16x8*>(rec + kRecU + (size_t)w * kFrag + lane * 16) = pack8(du[0], du[1]);
  }
}

template <int REF, bool GF32, bool GVA>
__global__ __launch_bounds__(kThreadsPrep, kThreadsPrep / 128) void prep_kernel(Plan p, int n_items) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int step = gridDim.x;
  int item = blockIdx.x;
  if (item >= n_items) return;
  // One input buffer: each item loads the next item's inputs once its own are dead.
  // Those loads are unconditional (clamped to the last item), so no branch holds them
  // back and the wait before each item covers only its own inputs.
  Inputs in;
  Item cur = item_of(p, item);
  load_inputs<GF32, GVA>(p, cur, w, lane, in);
  for (;;) {
    const Item nxt = item_of(p, min(item + step, n_items - 1));
    process_item<REF, GF32, GVA>(p, cur, in, nxt, lds, w, lane);
    item += step;
    if (item >= n_items) break;
    cur = nxt;
  }
}

template <int REF, bool GF32, bool GVA>
int launch_ref(const Plan& p, hipStream_t s, int grid, hipEvent_t start, hipEvent_t stop) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<REF, GF32, GVA>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes(REF));
    if (e != hipSuccess) return (int)e;
    attr_set = true;
  }
  const int n_items = p.n_chunks * p.H;
  hipExtLaunchKernelGGL((prep_kernel<REF, GF32, GVA>), dim3(min(grid, n_items)), dim3(kThreadsPrep), lds_bytes(REF), s,
                        start, stop, 0, p, n_items);
  return (int)hipGetLastError();
}

template <bool GF32, bool GVA>
int launch_gate(const Plan& p, hipStream_t s, int grid, hipEvent_t e0, hipEvent_t e1) {
  switch (p.ref_block) {
    case 16: return launch_ref<16, GF32, GVA>(p, s, grid, e0, e1);
    case 8: return launch_ref<8, GF32, GVA>(p, s, grid, e0, e1);
    case 4: return launch_ref<4, GF32, GVA>(p, s, grid, e0, e1);
    case 2: return launch_ref<2, GF32, GVA>(p, s, grid, e0, e1);
    default: return launch_ref<1, GF32, GVA>(p, s, grid, e0, e1);
  }
}

}  // namespace

int launch_prep(const Plan& p, void* stream, void* start, void* stop) {
  if (p.n_chunks == 0) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t e0 = reinterpret_cast<hipEvent_t>(start), e1 = reinterpret_cast<hipEvent_t>(stop);
  const int grid = 2 * p.cu_count;  // persistent: two resident workgroups per CU
  if (p.group > 1)
    return p.g_dtype == kF32 ? launch_gate<true, true>(p, s, grid, e0, e1) : launch_gate<false, true>(p, s, grid, e0, e1);
  return p.g_dtype == kF32 ? launch_gate<true, false>(p, s, grid, e0, e1) : launch_gate<false, false>(p, s, grid, e0, e1);
}

}  // namespace kda
