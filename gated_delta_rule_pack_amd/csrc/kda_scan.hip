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
//
// The serial chain is issue-bound, so the step is written for a small instruction count:
// fragments come in through buffer loads whose chunk offset is uniform (no per-load
// address arithmetic), and no register array is indexed by the wave number.

#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <int NT>
struct Frags {
  bf16x8 w[2][2];   // W fragments: row tile t, key block 2*wave + mm
  bf16x8 qo[2];     // Q fragments of row tile = wave (key blocks 2*wave + mm)
  bf16x8 qx[2];     // Q fragments of the other row tile
  bf16x8 k[4];      // K fragments: key tiles 4*wave .. 4*wave + 3
  bf16x8 u[NT];     // U fragments of this workgroup's value tiles
  bf16x8 p;         // P fragment of row tile = wave
  float e;          // exp(G_C) of key 64*wave + lane
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource word 3 for gfx9-family untyped loads.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// One chunk's fragments through buffer loads: the per-lane offset is one VGPR for every
// fragment and the chunk/fragment offset is uniform (SGPR), so no per-load address math.
// Fragments whose row tile depends on the wave are selected by address, never by
// indexing a register array with the wave number.
template <int NT>
__device__ __forceinline__ void load_frags(Frags<NT>& f, __amdgpu_buffer_rsrc_t rs, int chunk_off, int vo,
                                           int wave, int vtile0) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
      f.w[t][mm] = __builtin_bit_cast(bf16x8, bload(rs, vo, chunk_off + (int)kRecW + (t * 4 + 2 * wave + mm) * (int)kFrag));
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    f.qo[mm] = __builtin_bit_cast(bf16x8, bload(rs, vo, chunk_off + (int)kRecQ + (wave * 4 + 2 * wave + mm) * (int)kFrag));
    f.qx[mm] = __builtin_bit_cast(bf16x8, bload(rs, vo, chunk_off + (int)kRecQ + ((wave ^ 1) * 4 + 2 * wave + mm) * (int)kFrag));
  }
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
    f.k[tt] = __builtin_bit_cast(bf16x8, bload(rs, vo, chunk_off + (int)kRecK + (4 * wave + tt) * (int)kFrag));
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    f.u[nt] = __builtin_bit_cast(bf16x8, bload(rs, vo, chunk_off + (int)kRecU + (vtile0 + nt) * (int)kFrag));
  f.p = __builtin_bit_cast(bf16x8, bload(rs, vo, chunk_off + (int)kRecP + wave * (int)kFrag));
  // One float per lane (256 bytes per wave): redistributed through LDS in the step.
  f.e = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo >> 2, chunk_off + (int)kRecE + 256 * wave, 0));
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

// L2 prefetch role: stream the records of one (sequence, head) through this XCD's L2
// ahead of the scan workgroups, staying at most prefetch_ahead chunks in front of the
// published progress. Purely a cache hint: nothing waits on it, and its own wait is
// bounded.
__device__ void prefetch_records(const Plan& p, int u, int n, int h, int pf_index) {
  const int cu0 = p.d_cu[n], cu1 = p.d_cu[n + 1];
  const int nc = (cu1 - cu0 + kChunk - 1) / kChunk;
  const char* rec0 = reinterpret_cast<const char*>(p.ws) + ((size_t)h * p.n_chunks + p.d_co[n]) * kRecBytes;
  const uint32_t* prog = p.progress + u;
  uint32_t acc = 0;
  uint32_t seen = 0;
  int idle = 0;
  for (int c = pf_index; c < nc; c += p.prefetchers) {
    while ((int)seen + p.prefetch_ahead <= c) {
      const uint32_t now = __hip_atomic_load(prog, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (now != seen) {
        seen = now;
        idle = 0;
      } else {
        if (++idle > (1 << 16)) return;  // the scan stalled or finished: stop hinting
        __builtin_amdgcn_s_sleep(8);
      }
    }
    const uint4* src = reinterpret_cast<const uint4*>(rec0 + (size_t)c * kRecBytes);
    constexpr int kVec = (int)(kRecBytes / 16);
#pragma unroll 6
    for (int i = threadIdx.x; i < kVec; i += kThreadsScan) {
      const uint4 v = src[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  // Keeps the loads alive; threadIdx.x never reaches 1023 in a 128-thread workgroup.
  if (acc == 0x9e3779b9u && threadIdx.x == 1023) p.progress[u] = acc;
}

template <int NT, int SDT>
__global__ __launch_bounds__(kThreadsScan, 1) void scan_kernel(Plan p, int units, int groups) {
  // LDS: partial sums exchanged between the two waves [parity][wave][X: 2*NT, Y: NT][lane],
  // then exp(G_C) broadcast areas [parity][wave][64 floats].
  extern __shared__ __attribute__((aligned(16))) f32x4 xch[];
  const int bidx = blockIdx.x;
  const int xcd = bidx & 7;  // workgroups are dealt round-robin to the 8 XCDs
  const int slot = bidx >> 3;
  const int per_unit = groups + p.prefetchers;
  const int local = slot / per_unit;
  const int grp = slot - local * per_unit;
  const int u = local * 8 + xcd;  // all workgroups of one (sequence, head) share an XCD
  if (u >= units) return;
  const int n = u / p.H;
  const int h = u - n * p.H;
  if (grp >= groups) {
    prefetch_records(p, u, n, h, grp - groups);
    return;
  }
  const bool publish = (grp == 0) && (threadIdx.x == 0) && p.prefetchers > 0;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
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
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rec0), (short)0, nc * (int)kRecBytes, kBufWord3);
  const int vo = lane * 16;  // lane offset inside a fragment
  const size_t row_stride = (size_t)p.H * kHead;  // elements between tokens in q/k/v/out
  // Output: lane holds O^T rows v = 4*g4 .. 4*g4+3 (consecutive value channels) of token
  // row 16*wave + l16, so each lane stores 8 contiguous bytes per value tile.
  const int orow = 16 * wave + l16;
  const size_t ooff = (size_t)orow * row_stride + (size_t)h * kHead + 16 * vtile0 + 4 * g4;
  // LDS: exchange area, then per-wave exp(G_C) broadcast areas [parity][wave][64].
  float* ebuf = reinterpret_cast<float*>(xch + 2 * 2 * 3 * NT * 64);

  auto step = [&](const Frags<NT>& f, int c) {
    const int par = c & 1;
    f32x4* mine = xch + ((par * 2 + wave) * 3 * NT) * 64 + lane;
    const f32x4* other = xch + ((par * 2 + (wave ^ 1)) * 3 * NT) * 64 + lane;
    // State as MFMA operand per key block (2 blocks of 32 keys per wave).
    bf16x8 Sb[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) Sb[nt][mm] = pack8(S[nt][2 * mm], S[nt][2 * mm + 1]);
    // Partial W S^T over this wave's 64 keys (the critical path): both row tiles.
    f32x4 X[2][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 a = mfma(f.w[t][0], Sb[nt][0], zero4());
        a = mfma(f.w[t][1], Sb[nt][1], a);
        X[t][nt] = a;
        mine[(t * NT + nt) * 64] = a;
      }
    // Partial (Q S^T)^T = S Q^T for the other wave's row tile (exchanged) and this one.
    f32x4 Yo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 b = mfma(Sb[nt][0], f.qx[0], zero4());
      b = mfma(Sb[nt][1], f.qx[1], b);
      mine[((2 * NT) + nt) * 64] = b;
      f32x4 o = mfma(Sb[nt][0], f.qo[0], zero4());
      Yo[nt] = mfma(Sb[nt][1], f.qo[1], o);
    }
    // exp(G_C) of this wave's keys: lane k holds key 64*wave + k; broadcast via LDS.
    float* eb = ebuf + (par * 2 + wave) * 64;
    eb[lane] = f.e;
    __syncthreads();
    f32x4 E[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) E[tt] = *reinterpret_cast<const f32x4*>(eb + 16 * tt + 4 * g4);
    const int t0 = cu0 + kChunk * c;
    const int len = min(kChunk, cu1 - t0);
    __bf16* out_c = reinterpret_cast<__bf16*>(p.out) + (size_t)t0 * row_stride + ooff;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // Full key sums; a + b == b + a, so both waves hold identical bits.
      const f32x4 x0 = X[0][nt] + other[(0 * NT + nt) * 64];
      const f32x4 x1 = X[1][nt] + other[(1 * NT + nt) * 64];
      const bf16x8 uu = f.u[nt];
      f32x4 d0, d1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0[i] = from_bf16(uu[i]) - x0[i];
        d1[i] = from_bf16(uu[4 + i]) - x1[i];
      }
      const bf16x8 Db = pack8(d0, d1);  // Delta rows {4g..4g+3, 16+4g..16+4g+3}
      // State update: S^T = Diag(E) S^T + K^T Delta over this wave's key tiles.
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) S[nt][tt] = mfma(f.k[tt], Db, S[nt][tt] * E[tt]);
      // O^T of row tile = wave: (S Q^T) + Delta^T P^T, then one 8-byte store per lane.
      f32x4 o = Yo[nt] + other[(2 * NT + nt) * 64];
      o = mfma(Db, f.p, o);
      if (orow < len) {
        typedef __bf16 b4 __attribute__((ext_vector_type(4)));
        const b4 ov = {to_bf16(o[0]), to_bf16(o[1]), to_bf16(o[2]), to_bf16(o[3])};
        *reinterpret_cast<b4*>(out_c + 16 * nt) = ov;
      }
    }
    if (publish) __hip_atomic_store(p.progress + u, (uint32_t)(c + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  if (nc > 0) {
    // The next chunk's loads are issued unconditionally (clamped to the last chunk) so
    // that the wait before each step only covers the current chunk's fragments: a load
    // under a branch makes the compiler wait for every outstanding load instead.
    Frags<NT> fa, fb;
    load_frags<NT>(fa, rs, 0, vo, wave, vtile0);
    for (int c = 0; c < nc; c += 2) {
      load_frags<NT>(fb, rs, min(c + 1, nc - 1) * (int)kRecBytes, vo, wave, vtile0);
      step(fa, c);
      if (c + 1 >= nc) break;
      load_frags<NT>(fa, rs, min(c + 2, nc - 1) * (int)kRecBytes, vo, wave, vtile0);
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
  const int nblocks = 8 * per_xcd * (groups + p.prefetchers);
  const size_t lds = (size_t)2 * 2 * 3 * NT * 64 * sizeof(f32x4) + 2 * 2 * 64 * sizeof(float);
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
