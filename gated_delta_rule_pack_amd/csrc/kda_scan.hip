// Serial scan kernel for chunkwise KDA prefill on gfx950.
//
// The state walk over each sequence's chunks (aiter PR 4741, Summary: "scan, the serial
// state walk"), with paged or dense state read and written in-kernel (aiter PR 5754,
// Technical Details) and fp16/bf16 state storage up-cast to fp32 on load and rounded to
// nearest even on store (aiter PR 5249, What). Per chunk, with S the V x K state at the
// chunk start and the prep tiles W, U, Q, K, P, E of the chunk:
//
//   Delta = U - W S^T                    (the chunk's delta rows)
//   O     = Q S^T + P Delta              (scale folded into Q and P in prep)
//   S     = S Diag(E) + Delta^T K
//
// Work split: one workgroup per (sequence, head, value slice of 16*NT channels); the
// slice count is the occupancy-aware dv_split chosen on the host. Each of the two waves
// holds the fp32 state for half of the key channels (S^T rows 64w .. 64w+63) in MFMA
// accumulator layout, so the state never leaves registers between chunks. The key
// reduction of W S^T and Q S^T is split across the two waves and combined through LDS
// (one barrier per chunk, double-buffered by chunk parity). The next chunk's operand
// fragments are loaded while the current chunk computes.

#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <int NT>
struct Frags {
  bf16x8 w[2][2];   // W fragments: row tile t, key block 2*wave + mm
  bf16x8 q[2][2];   // Q fragments, same order
  bf16x8 k[4];      // K fragments: key tiles 4*wave .. 4*wave + 3
  bf16x8 u[NT];     // U fragments of this workgroup's value tiles
  bf16x8 p;         // P fragment of row tile = wave
  f32x4 e[4];       // exp(G_C) for this lane's key rows in each key tile
};

template <int NT>
__device__ __forceinline__ void load_frags(Frags<NT>& f, const char* rec, int wave, int lane, int g4,
                                           int vtile0) {
  const char* lp = rec + lane * 16;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int fi = t * 4 + 2 * wave + mm;
      f.w[t][mm] = *reinterpret_cast<const bf16x8*>(lp + kRecW + fi * kFrag);
      f.q[t][mm] = *reinterpret_cast<const bf16x8*>(lp + kRecQ + fi * kFrag);
    }
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
    f.k[tt] = *reinterpret_cast<const bf16x8*>(lp + kRecK + (4 * wave + tt) * kFrag);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    f.u[nt] = *reinterpret_cast<const bf16x8*>(lp + kRecU + (vtile0 + nt) * kFrag);
  f.p = *reinterpret_cast<const bf16x8*>(lp + kRecP + wave * kFrag);
  const float* E = reinterpret_cast<const float*>(rec + kRecE);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
    f.e[tt] = *reinterpret_cast<const f32x4*>(E + 16 * (4 * wave + tt) + 4 * g4);
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
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 v = *reinterpret_cast<const b4*>(s);
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
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 v = {to_bf16(x[0]), to_bf16(x[1]), to_bf16(x[2]), to_bf16(x[3])};
    *reinterpret_cast<b4*>(reinterpret_cast<__bf16*>(plane) + off) = v;
  }
}

template <int SDT>
__device__ __forceinline__ size_t elem_size() {
  return SDT == kF32 ? 4 : 2;
}

template <int NT, int SDT>
__global__ __launch_bounds__(kThreadsScan, 1) void scan_kernel(Plan p, int units, int groups) {
  // Partial sums exchanged between the two waves: [parity][wave][X: 2*NT, Y: NT][lane].
  extern __shared__ __attribute__((aligned(16))) f32x4 xch[];
  const int bidx = blockIdx.x;
  const int xcd = bidx & 7;  // workgroups are dealt round-robin to the 8 XCDs
  const int slot = bidx >> 3;
  const int local = slot / groups;
  const int grp = slot - local * groups;
  const int u = local * 8 + xcd;  // all value slices of one (sequence, head) share an XCD
  if (u >= units) return;
  const int n = u / p.H;
  const int h = u - n * p.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  const int vtile0 = grp * NT;  // first 16-channel value tile of this workgroup

  // ---- initial state: lane holds S^T[k][v] for k = 16*(4*wave+tt) + 4*g4 + i,
  //      v = 16*(vtile0 + nt) + l16.
  f32x4 S[NT][4];
  const void* in_plane = nullptr;
  if (p.in_mode == kStateDense) {
    in_plane = reinterpret_cast<const char*>(p.state_in) +
               ((size_t)n * p.stride0 + (size_t)h * kHead * kHead) * elem_size<SDT>();
  } else if (p.in_mode == kStatePaged && p.flags[n]) {
    in_plane = reinterpret_cast<const char*>(p.state_in) +
               ((size_t)p.indices[n] * p.stride0 + (size_t)h * kHead * kHead) * elem_size<SDT>();
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (in_plane) {
        const size_t off = (size_t)(16 * (vtile0 + nt) + l16) * kHead + 16 * (4 * wave + tt) + 4 * g4;
        S[nt][tt] = load_state4<SDT>(in_plane, off);
      } else {
        S[nt][tt] = zero4();
      }
    }

  const int cu0 = p.d_cu[n], cu1 = p.d_cu[n + 1];
  const int nc = (cu1 - cu0 + kChunk - 1) / kChunk;
  const char* rec0 = reinterpret_cast<const char*>(p.ws) + ((size_t)h * p.n_chunks + p.d_co[n]) * kRecBytes;
  __bf16* outp = reinterpret_cast<__bf16*>(p.out);
  const size_t row_stride = (size_t)p.H * kHead;

  auto step = [&](const Frags<NT>& f, int c) {
    // State as B operand per key block (2 blocks of 32 keys per wave).
    bf16x8 Sb[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) Sb[nt][mm] = pack8(S[nt][2 * mm], S[nt][2 * mm + 1]);
    // Partial W S^T and Q S^T over this wave's 64 keys.
    f32x4 X[2][NT], Y[2][NT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 a = zero4(), b = zero4();
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          a = mfma(f.w[t][mm], Sb[nt][mm], a);
          b = mfma(f.q[t][mm], Sb[nt][mm], b);
        }
        X[t][nt] = a;
        Y[t][nt] = b;
      }
    // Exchange: both X tiles, and the Y tile the other wave finishes.
    const int par = c & 1;
    f32x4* mine = xch + ((par * 2 + wave) * 3 * NT) * 64;
    const f32x4* other = xch + ((par * 2 + (1 - wave)) * 3 * NT) * 64;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mine[(0 * NT + nt) * 64 + lane] = X[0][nt];
      mine[(1 * NT + nt) * 64 + lane] = X[1][nt];
      mine[(2 * NT + nt) * 64 + lane] = Y[1 - wave][nt];
    }
    __syncthreads();
    const int t0 = cu0 + kChunk * c;
    const int len = min(kChunk, cu1 - t0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // Full key sums (a + b == b + a, so both waves get identical bits).
      const f32x4 x0 = X[0][nt] + other[(0 * NT + nt) * 64 + lane];
      const f32x4 x1 = X[1][nt] + other[(1 * NT + nt) * 64 + lane];
      const bf16x8 uu = f.u[nt];
      f32x4 d0, d1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0[i] = from_bf16(uu[i]) - x0[i];
        d1[i] = from_bf16(uu[4 + i]) - x1[i];
      }
      const bf16x8 Db = pack8(d0, d1);  // Delta rows {4g..4g+3, 16+4g..16+4g+3} as B operand
      // Output rows of tile = wave.
      f32x4 o = Y[wave][nt] + other[(2 * NT + nt) * 64 + lane];
      o = mfma(f.p, Db, o);
      const int v = 16 * (vtile0 + nt) + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * wave + 4 * g4 + i;
        if (rr < len) outp[(size_t)(t0 + rr) * row_stride + (size_t)h * kHead + v] = to_bf16(o[i]);
      }
      // State update: S^T = Diag(E) S^T + K^T Delta over this wave's key tiles.
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) S[nt][tt] = mfma(f.k[tt], Db, S[nt][tt] * f.e[tt]);
    }
  };

  if (nc > 0) {
    Frags<NT> fa, fb;
    load_frags<NT>(fa, rec0, wave, lane, g4, vtile0);
    for (int c = 0; c < nc; c += 2) {
      if (c + 1 < nc) load_frags<NT>(fb, rec0 + (size_t)(c + 1) * kRecBytes, wave, lane, g4, vtile0);
      step(fa, c);
      if (c + 1 >= nc) break;
      if (c + 2 < nc) load_frags<NT>(fa, rec0 + (size_t)(c + 2) * kRecBytes, wave, lane, g4, vtile0);
      step(fb, c + 1);
    }
  }

  // ---- final state
  void* out_plane = nullptr;
  if (p.out_mode == kStateDense) {
    out_plane = reinterpret_cast<char*>(p.state_out) +
                ((size_t)n * p.stride0 + (size_t)h * kHead * kHead) * elem_size<SDT>();
  } else if (p.out_mode == kStatePaged) {
    out_plane = reinterpret_cast<char*>(p.state_out) +
                ((size_t)p.indices[n] * p.stride0 + (size_t)h * kHead * kHead) * elem_size<SDT>();
  }
  if (out_plane) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const size_t off = (size_t)(16 * (vtile0 + nt) + l16) * kHead + 16 * (4 * wave + tt) + 4 * g4;
        store_state4<SDT>(out_plane, off, S[nt][tt]);
      }
  }
}

template <int NT, int SDT>
int launch_nt(const Plan& p, hipStream_t s) {
  const int groups = 8 / NT;
  const int units = p.N * p.H;
  const int per_xcd = (units + 7) / 8;
  const int nblocks = 8 * per_xcd * groups;
  const size_t lds = (size_t)2 * 2 * 3 * NT * 64 * sizeof(f32x4);
  hipLaunchKernelGGL((scan_kernel<NT, SDT>), dim3(nblocks), dim3(kThreadsScan), lds, s, p, units, groups);
  return (int)hipGetLastError();
}

template <int SDT>
int launch_dt(const Plan& p, hipStream_t s) {
  switch (p.dv_split) {
    case 8: return launch_nt<1, SDT>(p, s);
    case 4: return launch_nt<2, SDT>(p, s);
    default: return launch_nt<4, SDT>(p, s);
  }
}

}  // namespace

int launch_scan(const Plan& p, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (p.state_dtype) {
    case kF16: return launch_dt<kF16>(p, s);
    case kBF16: return launch_dt<kBF16>(p, s);
    default: return launch_dt<kF32>(p, s);
  }
}

}  // namespace kda
