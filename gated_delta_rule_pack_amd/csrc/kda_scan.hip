// Serial scan kernel for chunkwise KDA prefill on gfx950.
//
// The serial pass over each sequence's chunks that carries the state (aiter PR 4741,
// Summary: the second of its two kernels), with paged or dense state read and written
// in-kernel (aiter PR 5754,
// Technical Details) and fp16/bf16 state storage up-cast to fp32 on load and rounded to
// nearest even on store (aiter PR 5249, What). Per chunk, with S the V x K state at the
// chunk start and the prep tiles W, U, Q, K, P, E of the chunk:
//
//   Delta = U - W S^T                    (the chunk's delta rows)
//   O     = Q S^T + P Delta              (scale folded into Q and P in prep)
//   S     = S Diag(E) + Delta^T K
//
// Work split: one workgroup per (sequence, head, value slice of 16*NT channels); the
// slice count is the occupancy-aware dv_split chosen on the host. The workgroup has
// four waves with two roles:
//   * state waves 0 and 1 each hold the fp32 state for half of the key channels
//     (S^T rows 64w .. 64w+63) in MFMA accumulator layout and run only the recurrence:
//     partial W S^T, exchange through LDS, Delta, and the state update;
//   * output waves 2 and 3 each own one 16-row tile of the chunk's output. After the
//     chunk's barrier they read the state snapshot (bf16, as the state waves used it) and
//     the W S^T partials from LDS, rebuild Delta bit for bit, and form O^T = S Q^T +
//     Delta^T P^T, one 8-byte store per lane.
// The serial chain therefore carries no output work. One barrier per chunk; LDS buffers
// are double-buffered by chunk parity. Each wave loads only the fragments it consumes,
// one chunk ahead, through buffer loads with uniform offsets.

#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource word 3 for gfx9-family untyped loads.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ bf16x8 bload8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Fragments a state wave consumes per chunk.
template <int NT>
struct StateFrags {
  bf16x8 w[2][2];  // W fragments: row tile t, key block 2*wave + mm
  bf16x8 k[4];     // K fragments: key tiles 4*wave .. 4*wave + 3
  bf16x8 u[NT];    // U fragments of this workgroup's value tiles
  float e;         // exp(G_C) of key 64*wave + lane
};

template <int NT>
__device__ __forceinline__ void load_state_frags(StateFrags<NT>& f, __amdgpu_buffer_rsrc_t rs, int coff, int vo,
                                                 int wave, int vtile0) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
      f.w[t][mm] = bload8(rs, vo, coff + (int)kRecW + (t * 4 + 2 * wave + mm) * (int)kFrag);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) f.k[tt] = bload8(rs, vo, coff + (int)kRecK + (4 * wave + tt) * (int)kFrag);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) f.u[nt] = bload8(rs, vo, coff + (int)kRecU + (vtile0 + nt) * (int)kFrag);
  // One float per lane (256 bytes per wave), redistributed through LDS.
  f.e = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo >> 2, coff + (int)kRecE + 256 * wave, 0));
}

// Fragments an output wave consumes per chunk (its row tile t).
template <int NT>
struct OutFrags {
  bf16x8 q[4];   // Q fragments (t, key block m)
  bf16x8 p;      // P fragment of row tile t
  bf16x8 u[NT];  // U fragments (to rebuild Delta)
};

template <int NT>
__device__ __forceinline__ void load_out_frags(OutFrags<NT>& f, __amdgpu_buffer_rsrc_t rs, int coff, int vo, int t,
                                               int vtile0) {
#pragma unroll
  for (int m = 0; m < 4; ++m) f.q[m] = bload8(rs, vo, coff + (int)kRecQ + (t * 4 + m) * (int)kFrag);
  f.p = bload8(rs, vo, coff + (int)kRecP + t * (int)kFrag);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) f.u[nt] = bload8(rs, vo, coff + (int)kRecU + (vtile0 + nt) * (int)kFrag);
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

// LDS layout per chunk parity, in rows of 64 lanes x 16 bytes:
//   Sb  [2 state waves][NT][2 key blocks]   state snapshot (bf16 operand registers)
//   X   [2 state waves][2 row tiles][NT]    partial W S^T
//   E   [2 state waves]                     exp(G_C), 64 floats each
template <int NT>
struct Lds {
  static constexpr int kSb = 0;
  static constexpr int kX = kSb + 2 * NT * 2;
  static constexpr int kE = kX + 2 * 2 * NT;
  static constexpr int kPerParity = kE + 2;
  static constexpr size_t kBytes = (size_t)2 * kPerParity * 64 * 16;
  __device__ static int sb(int par, int w, int nt, int mm) { return (par * kPerParity + kSb + (w * NT + nt) * 2 + mm) * 64; }
  __device__ static int x(int par, int w, int t, int nt) { return (par * kPerParity + kX + (w * 2 + t) * NT + nt) * 64; }
  __device__ static int e(int par, int w) { return (par * kPerParity + kE + w) * 64; }
};

template <int NT, int SDT>
__global__ __launch_bounds__(kThreadsScan, 1) void scan_kernel(Plan p, int units, int groups) {
  extern __shared__ __attribute__((aligned(16))) u32x4 lds[];
  typedef Lds<NT> L;
  const int bidx = blockIdx.x;
  const int xcd = bidx & 7;  // workgroups are dealt round-robin to the 8 XCDs
  const int slot = bidx >> 3;
  const int local = slot / groups;
  const int grp = slot - local * groups;
  const int u = local * 8 + xcd;  // all value slices of one (sequence, head) share an XCD
  if (u >= units) return;
  const int n = u / p.H;
  const int h = u - n * p.H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  const int vtile0 = grp * NT;  // first 16-channel value tile of this workgroup

  const int cu0 = p.d_cu[n], cu1 = p.d_cu[n + 1];
  const int nc = (cu1 - cu0 + kChunk - 1) / kChunk;
  const char* rec0 = reinterpret_cast<const char*>(p.ws) + ((size_t)h * p.n_chunks + p.d_co[n]) * kRecBytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rec0), (short)0, nc * (int)kRecBytes, kBufWord3);
  const int vo = lane * 16;  // lane offset inside a fragment

  if (wave < 2) {
    // ============================================================ state waves
    // Lane holds S^T[k][v] for k = 16*(4*wave+tt) + 4*g4 + i, v = 16*(vtile0 + nt) + l16.
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

    auto step = [&](const StateFrags<NT>& f, int c) {
      const int par = c & 1;
      bf16x8 Sb[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          Sb[nt][mm] = pack8(S[nt][2 * mm], S[nt][2 * mm + 1]);
          lds[L::sb(par, wave, nt, mm) + lane] = __builtin_bit_cast(u32x4, Sb[nt][mm]);
        }
      // Partial W S^T over this wave's 64 keys, both row tiles.
      f32x4 X[2][NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 a = mfma(f.w[t][0], Sb[nt][0], zero4());
          a = mfma(f.w[t][1], Sb[nt][1], a);
          X[t][nt] = a;
          lds[L::x(par, wave, t, nt) + lane] = __builtin_bit_cast(u32x4, a);
        }
      reinterpret_cast<float*>(lds + L::e(par, wave))[lane] = f.e;
      __syncthreads();
      // exp(G_C) of this lane's key rows (lane k of the wave loaded key 64*wave + k).
      const float* eb = reinterpret_cast<const float*>(lds + L::e(par, wave));
      f32x4 E[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) E[tt] = *reinterpret_cast<const f32x4*>(eb + 16 * tt + 4 * g4);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // Full key sums; a + b == b + a, so every wave rebuilds identical bits.
        const f32x4 x0 = X[0][nt] + __builtin_bit_cast(f32x4, lds[L::x(par, wave ^ 1, 0, nt) + lane]);
        const f32x4 x1 = X[1][nt] + __builtin_bit_cast(f32x4, lds[L::x(par, wave ^ 1, 1, nt) + lane]);
        const bf16x8 uu = f.u[nt];
        f32x4 d0, d1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          d0[i] = from_bf16(uu[i]) - x0[i];
          d1[i] = from_bf16(uu[4 + i]) - x1[i];
        }
        const bf16x8 Db = pack8(d0, d1);  // Delta rows {4g..4g+3, 16+4g..16+4g+3}
        // S^T = Diag(E) S^T + K^T Delta over this wave's key tiles.
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) S[nt][tt] = mfma(f.k[tt], Db, S[nt][tt] * E[tt]);
      }
    };

    if (nc > 0) {
      // Next chunk's loads are unconditional (clamped to the last chunk) so the wait
      // before each step covers only the current chunk's fragments.
      StateFrags<NT> fa, fb;
      load_state_frags<NT>(fa, rs, 0, vo, wave, vtile0);
      for (int c = 0; c < nc; c += 2) {
        load_state_frags<NT>(fb, rs, min(c + 1, nc - 1) * (int)kRecBytes, vo, wave, vtile0);
        step(fa, c);
        if (c + 1 >= nc) break;
        load_state_frags<NT>(fa, rs, min(c + 2, nc - 1) * (int)kRecBytes, vo, wave, vtile0);
        step(fb, c + 1);
      }
    }

    // Final state.
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
  } else {
    // ============================================================ output waves
    const int t = wave - 2;  // row tile
    const size_t row_stride = (size_t)p.H * kHead;
    // Lane holds O^T rows v = 16*(vtile0+nt) + 4*g4 .. +3 of token row 16*t + l16.
    const int orow = 16 * t + l16;
    const size_t ooff = (size_t)orow * row_stride + (size_t)h * kHead + 16 * vtile0 + 4 * g4;

    auto step = [&](const OutFrags<NT>& f, int c) {
      const int par = c & 1;
      __syncthreads();  // the state waves have published chunk c's snapshot and partials
      const int t0 = cu0 + kChunk * c;
      const int len = min(kChunk, cu1 - t0);
      __bf16* out_c = reinterpret_cast<__bf16*>(p.out) + (size_t)t0 * row_stride + ooff;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x4 x0 = __builtin_bit_cast(f32x4, lds[L::x(par, 0, 0, nt) + lane]) +
                         __builtin_bit_cast(f32x4, lds[L::x(par, 1, 0, nt) + lane]);
        const f32x4 x1 = __builtin_bit_cast(f32x4, lds[L::x(par, 0, 1, nt) + lane]) +
                         __builtin_bit_cast(f32x4, lds[L::x(par, 1, 1, nt) + lane]);
        const bf16x8 uu = f.u[nt];
        f32x4 d0, d1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          d0[i] = from_bf16(uu[i]) - x0[i];
          d1[i] = from_bf16(uu[4 + i]) - x1[i];
        }
        const bf16x8 Db = pack8(d0, d1);
        // (Q S^T)^T = S Q^T over all 128 keys: key block m lives in state wave m / 2.
        f32x4 o = zero4();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8 sb = __builtin_bit_cast(bf16x8, lds[L::sb(par, m >> 1, nt, m & 1) + lane]);
          o = mfma(sb, f.q[m], o);
        }
        o = mfma(Db, f.p, o);  // + Delta^T P^T
        if (orow < len) {
          const bf16x4 ov = {to_bf16(o[0]), to_bf16(o[1]), to_bf16(o[2]), to_bf16(o[3])};
          *reinterpret_cast<bf16x4*>(out_c + 16 * nt) = ov;
        }
      }
    };

    if (nc > 0) {
      OutFrags<NT> fa, fb;
      load_out_frags<NT>(fa, rs, 0, vo, t, vtile0);
      for (int c = 0; c < nc; c += 2) {
        load_out_frags<NT>(fb, rs, min(c + 1, nc - 1) * (int)kRecBytes, vo, t, vtile0);
        step(fa, c);
        if (c + 1 >= nc) break;
        load_out_frags<NT>(fa, rs, min(c + 2, nc - 1) * (int)kRecBytes, vo, t, vtile0);
        step(fb, c + 1);
      }
    }
  }
}

template <int NT, int SDT>
int launch_nt(const Plan& p, hipStream_t s) {
  const int groups = 8 / NT;
  const int units = p.N * p.H;
  const int per_xcd = (units + 7) / 8;
  const int nblocks = 8 * per_xcd * groups;
  hipLaunchKernelGGL((scan_kernel<NT, SDT>), dim3(nblocks), dim3(kThreadsScan), Lds<NT>::kBytes, s, p, units,
                     groups);
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
