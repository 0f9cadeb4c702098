// Serial scan kernels for chunkwise KDA prefill on gfx950.
//
// The serial pass over each sequence's chunks that carries the state (aiter PR 4741,
// Summary: the second of its two kernels), with paged or dense state read and written
// in-kernel (aiter PR 5754, Technical Details) and fp16/bf16 state storage up-cast to
// fp32 on load and rounded to nearest even on store (aiter PR 5249, What). Per chunk,
// with S the V x K state at the chunk start and the prep tiles W, U, Q, K, P, E:
//
//   Delta = U - W S^T                    (the chunk's delta rows; the record holds -W,
//                                         so this is an MFMA accumulation from U)
//   O     = Q S^T + P Delta              (scale folded into Q and P in prep)
//   S     = S Diag(E) + Delta^T K
//
// One workgroup per (segment, head, value slice of 16*NT channels); a segment is a whole
// sequence unless the call is segmented, then it starts from the state the combine
// kernel computed and only a sequence's last segment writes the final state. The slice
// count is the host's occupancy-aware dv_split. Every slice of a (sequence, head) needs the whole
// W, K, Q and P of each chunk, so a step costs about the same number of bytes through
// one CU's vector-memory path whatever the slice width; at one workgroup per CU that
// path, and the dependent MFMA/LDS chain of the state update, bound a step.
//
// Narrow slices (16 or 32 channels; long sequences, few units), 4 waves:
//   * wave 0 holds the fp32 state of the slice for all 128 keys in MFMA accumulator
//     layout and runs only the recurrence. It publishes each chunk's bf16 state copy
//     and bf16 Delta to LDS for the output waves, then updates the state;
//   * waves 1 and 2 each own one 16-row tile of the output: O^T = S Q^T + Delta^T P^T
//     from the published copies, with their own Q and P fragments loaded from the
//     record several chunks ahead;
//   * wave 3 is a loader: it copies W, K, U and E of each chunk into a ring of LDS
//     slots with direct-to-LDS buffer loads, several chunks ahead, so that the state
//     wave never waits on a global load or on issuing one.
//   One barrier per chunk orders the publication and the ring.
// Wide slices (64 channels; many units), 4 waves, two workgroups per CU:
//   * waves 0 and 1 each hold the state for half of the keys and exchange partial
//     W S^T through LDS (64 value channels do not fit one wave's registers);
//   * waves 2 and 3 add up Delta from the partials and form the output;
//   every wave loads its own fragments, a few chunks ahead.

#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// Which (segment, head, value group) a workgroup serves. Workgroups are dealt
// round-robin to the 8 XCDs; all value groups of one (segment, head) land on one XCD,
// so its records are fetched into that XCD's L2 once. A segment is a run of one
// sequence's chunks (the whole sequence unless the call is segmented).
struct Unit {
  int n, h, grp;
  int c0, nch;         // first chunk within the sequence, chunks
  int m_prev, m_self;  // start-state map slot (-1: initial state), own map slot (-1: last)
};

__device__ __forceinline__ bool unit_of(const Plan& p, int units, int groups, Unit& u) {
  const int bidx = blockIdx.x;
  const int xcd = bidx & 7;
  const int slot8 = bidx >> 3;
  const int local = slot8 / groups;
  u.grp = slot8 - local * groups;
  const int id = local * 8 + xcd;
  if (id >= units) return false;
  const int s = id / p.H;
  u.h = id - s * p.H;
  const int32_t* e = p.d_seg + (size_t)kSegInts * s;
  u.n = e[0];
  u.c0 = e[1];
  u.nch = e[2];
  u.m_prev = e[3];
  u.m_self = e[4];
  return true;
}

// One state row group of four: the segment's start state (fp32, from the combine
// kernel), the call's initial state, or zero.
template <int SDT>
__device__ __forceinline__ f32x4 load_start4(const Plan& p, const Unit& u, const void* in_plane, size_t off) {
  if (u.m_prev >= 0) return load_state4<kF32>(p.starts + ((size_t)u.m_prev * p.H + u.h) * kHead * kHead, off);
  return in_plane ? load_state4<SDT>(in_plane, off) : zero4();
}

// Output-tile fragments one output wave consumes per chunk (row tile t).
struct OutFrags {
  bf16x8 q[4];  // Q fragments (t, key block m)
  bf16x8 p;     // P fragment of row tile t
};

__device__ __forceinline__ void load_out_frags(OutFrags& f, __amdgpu_buffer_rsrc_t rs, int coff, int vo, int t) {
#pragma unroll
  for (int m = 0; m < 4; ++m) f.q[m] = bload8(rs, vo, coff + (int)kRecQ + (t * 4 + m) * (int)kFrag);
  f.p = bload8(rs, vo, coff + (int)kRecP + t * (int)kFrag);
}

// Runs step(f[j], c) for every chunk c < nc with DEPTH chunks of fragments in flight:
// before step c the loads of chunk c + DEPTH - 1 go into the buffer step c - 1 used.
// The prologue is issued chunk by chunk (the compiler's wait before the first step
// counts only loads issued after chunk 0's). Full groups of DEPTH chunks run without
// an early exit, because a path from a partial group back to the loop head would make
// the compiler wait there for every load in flight; the last nc % DEPTH chunks are
// already loaded into f[0 ..].
template <int DEPTH, typename Frags, typename LoadF, typename StepF>
__device__ __forceinline__ void pipelined_chunks(int nc, LoadF&& load, StepF&& step) {
  Frags f[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH - 1; ++j) {
    load(f[j], min(j, nc - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  const int nfull = nc - nc % DEPTH;
  for (int c = 0; c < nfull; c += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      load(f[(j + DEPTH - 1) % DEPTH], min(c + j + DEPTH - 1, nc - 1));
      step(f[j], c + j);
    }
  }
#pragma unroll
  for (int j = 0; j < DEPTH - 1; ++j)
    if (nfull + j < nc) step(f[j], nfull + j);
}

// ====================================================================== narrow slices
// LDS: a ring of RING slots with the state wave's fragments of one chunk each (W 8, K 8,
// U NT fragments of 1 KB, E 128 fp32), then, per chunk parity, the published bf16 state
// copy Sb [NT][4 key blocks] and Delta Db [NT] as 1 KB operand rows.
template <int NT, int RING>
struct NarrowLds {
  static constexpr int kSlotW = 0;
  static constexpr int kSlotK = 8 * 1024;
  static constexpr int kSlotU = 16 * 1024;
  static constexpr int kSlotE = (16 + NT) * 1024;
  static constexpr int kSlot = kSlotE + 512;
  static constexpr int kRing = RING * kSlot;
  static constexpr int kPerParity = 5 * NT * 1024;
  static constexpr size_t kBytes = (size_t)kRing + 2 * (size_t)kPerParity;
  __device__ static int sb(int par, int nt, int m) { return kRing + par * kPerParity + (nt * 4 + m) * 1024; }
  __device__ static int db(int par, int nt) { return kRing + par * kPerParity + (4 * NT + nt) * 1024; }
};

template <int NT, int SDT, int RING, int DOUT>
__global__ __launch_bounds__(256, 1) void scan_narrow(Plan p, int units, int groups) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  typedef NarrowLds<NT, RING> L;
  Unit un;
  if (!unit_of(p, units, groups, un)) return;
  const int n = un.n, h = un.h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  const int vtile0 = un.grp * NT;  // first 16-channel value tile of this workgroup
  const int cu0 = p.d_cu[n] + kChunk * un.c0, cu1 = p.d_cu[n + 1];  // segment start, sequence end
  const int nc = un.nch;
  const char* rec0 =
      reinterpret_cast<const char*>(p.ws) + ((size_t)h * p.n_chunks + p.d_co[n] + un.c0) * kRecBytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rec0), (short)0, nc * (int)kRecBytes, kBufWord3);
  const int vo = lane * 16;  // lane offset inside a fragment

  if (wave == 3) {
    // ------------------------------------------------------------ loader wave
    // Chunk c goes to slot c mod RING, RING - 1 chunks ahead. Before barrier c (and
    // before the first barrier, for chunk 0) it waits until chunk c + 1 has landed.
    // The slot it refills during step c held chunk c - 1, which the state wave read
    // before barrier c - 1. Only chunks < nc are loaded. Its barriers carry no fence:
    // a fence would wait for every direct-to-LDS load in flight.
    constexpr int kLoads = 8 + 8 + NT + 2;
    auto issue = [&](int c, int slot) {
      char* base = lds + slot * L::kSlot;
      const int soff = c * (int)kRecBytes;
#pragma unroll
      for (int f = 0; f < 8; ++f)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotW + f * 1024), 16, vo,
                                                 soff + (int)kRecW + f * (int)kFrag, 0, 0);
#pragma unroll
      for (int f = 0; f < 8; ++f)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotK + f * 1024), 16, vo,
                                                 soff + (int)kRecK + f * (int)kFrag, 0, 0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotU + nt * 1024), 16, vo,
                                                 soff + (int)kRecU + (vtile0 + nt) * (int)kFrag, 0, 0);
#pragma unroll
      for (int half = 0; half < 2; ++half)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotE + half * 256), 4, lane * 4,
                                                 soff + (int)kRecE + half * 256, 0, 0);
    };
    if (nc > 0) {
      const int pre = min(RING - 1, nc);
      for (int c = 0; c < pre; ++c) issue(c, c);
      wait_chunks<kLoads, RING - 2>(pre - 1);  // chunk 0 has landed
      __builtin_amdgcn_s_barrier();
      int fill = RING - 1;  // slot of chunk c + RING - 1
      for (int c = 0; c < nc; ++c) {
        if (c + RING - 1 < nc) issue(c + RING - 1, fill);
        fill = (fill + 1 == RING) ? 0 : fill + 1;
        // Still in flight behind chunk c + 1: chunks c + 2 .. min(c + RING - 1, nc - 1).
        wait_chunks<kLoads, RING - 2>(min(RING - 2, nc - 2 - c));
        __builtin_amdgcn_s_barrier();
      }
    }
  } else if (wave == 0) {
    // ------------------------------------------------------------ state wave
    // Lane holds S^T[k][v] for k = 16*tt + 4*g4 + i (key tile tt = 0..7),
    // v = 16*(vtile0 + nt) + l16.
    f32x4 S[NT][8];
    const void* in_plane = state_in_plane<SDT>(p, n, h);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const size_t off = (size_t)(16 * (vtile0 + nt) + l16) * kHead + 16 * tt + 4 * g4;
        S[nt][tt] = load_start4<SDT>(p, un, in_plane, off);
      }

    // One chunk's fragments, read from its ring slot.
    // Issued together, in order of first use and pinned in that order (the scheduler
    // would otherwise sink each read to its use or permute them): the LDS counter can
    // name at most 15 reads in flight, so the wait before the first MFMA then covers
    // only W, U and little else.
    struct Frags {
      bf16x8 w[2][4];  // -W (row tile t, key block m)
      bf16x8 u[NT];    // U of this workgroup's value tiles
      bf16x8 k[8];     // K (key tile)
      f32x4 e[8];      // exp(G_C) of this lane's keys 16*tt + 4*g4 + i
    };
    auto read = [&](Frags& f, int slot) {
      const char* sl = lds + slot * L::kSlot;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f.w[t][m] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotW + (t * 4 + m) * 1024 + vo);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f.u[nt] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotU + nt * 1024 + vo);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        f.k[tt] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotK + tt * 1024 + vo);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        f.e[tt] = *reinterpret_cast<const f32x4*>(sl + L::kSlotE + (16 * tt + 4 * g4) * 4);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    if (nc > 0) {
      barrier_lds();  // the loader has chunk 0 in slot 0
      Frags f;
      read(f, 0);
      int slot = 0;
      for (int c = 0; c < nc; ++c) {
        const int par = c & 1;
        // bf16 copy of the state: key block m holds key tiles 2m, 2m+1 (the record's
        // W and Q fragments use the same key order).
        bf16x8 Sb[NT][4];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int m = 0; m < 4; ++m) Sb[nt][m] = pack8(S[nt][2 * m], S[nt][2 * m + 1]);
        // Delta = U + (-W) S^T, accumulated from U; rows {4g..4g+3, 16+4g..16+4g+3} of
        // the chunk per lane.
        f32x4 x[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            f32x4 a;
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = from_bf16(f.u[nt][4 * t + i]);
#pragma unroll
            for (int m = 0; m < 4; ++m) a = mfma(f.w[t][m], Sb[nt][m], a);
            x[nt][t] = a;
          }
        // Publish the state copy after the MFMAs are issued (they need only registers).
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int m = 0; m < 4; ++m) *reinterpret_cast<bf16x8*>(lds + L::sb(par, nt, m) + vo) = Sb[nt][m];
        // Diag(E) S^T while the MFMAs above run.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) S[nt][tt] = S[nt][tt] * f.e[tt];
        bf16x8 Db[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          Db[nt] = pack8(x[nt][0], x[nt][1]);
          *reinterpret_cast<bf16x8*>(lds + L::db(par, nt) + vo) = Db[nt];
        }
        // S^T = Diag(E) S^T + K^T Delta.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) S[nt][tt] = mfma(f.k[tt], Db[nt], S[nt][tt]);
        barrier_lds();  // publishes Sb, Db; the loader has chunk c + 1 in the next slot
        slot = (slot + 1 == RING) ? 0 : slot + 1;
        if (c + 1 < nc) read(f, slot);
      }
    }

    void* out_plane = un.m_self < 0 ? state_out_plane<SDT>(p, n, h) : nullptr;
    if (out_plane) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const size_t off = (size_t)(16 * (vtile0 + nt) + l16) * kHead + 16 * tt + 4 * g4;
          store_state4<SDT>(out_plane, off, S[nt][tt]);
        }
    }
  } else {
    // ------------------------------------------------------------ output waves
    const int t = wave - 1;  // row tile
    const size_t row_stride = (size_t)p.H * kHead;
    // Lane holds O^T rows v = 16*(vtile0+nt) + 4*g4 .. +3 of token row 16*t + l16.
    const int orow = 16 * t + l16;
    const size_t ooff = (size_t)orow * row_stride + (size_t)h * kHead + 16 * vtile0 + 4 * g4;
    typedef OutFrags F;
    if (nc > 0) {
      barrier_lds();  // pairs with the first barrier of the other waves
      pipelined_chunks<DOUT, F>(
          nc, [&](F& f, int c) { load_out_frags(f, rs, c * (int)kRecBytes, vo, t); },
          [&](const F& f, int c) {
            const int par = c & 1;
            barrier_lds();  // the state wave has published chunk c's Sb and Db
            const int t0 = cu0 + kChunk * c;
            const int len = min(kChunk, cu1 - t0);
            __bf16* out_c = reinterpret_cast<__bf16*>(p.out) + (size_t)t0 * row_stride + ooff;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              // (Q S^T)^T = S Q^T, then + Delta^T P^T.
              f32x4 o = zero4();
#pragma unroll
              for (int m = 0; m < 4; ++m)
                o = mfma(*reinterpret_cast<const bf16x8*>(lds + L::sb(par, nt, m) + vo), f.q[m], o);
              o = mfma(*reinterpret_cast<const bf16x8*>(lds + L::db(par, nt) + vo), f.p, o);
              if (orow < len) {
                const bf16x4 ov = {to_bf16(o[0]), to_bf16(o[1]), to_bf16(o[2]), to_bf16(o[3])};
                *reinterpret_cast<bf16x4*>(out_c + 16 * nt) = ov;
              }
            }
          });
    }
  }
}

// ====================================================================== wide slices
// LDS per chunk parity, in rows of 64 lanes x 16 bytes:
//   Sb [2 state waves][NT][2 key blocks]   state copy (bf16 operand registers)
//   X  [2 state waves][2 row tiles][NT]    partial (-W) S^T, wave 0's started from U
//   E  [2 state waves]                     exp(G_C), 64 floats each
template <int NT>
struct WideLds {
  static constexpr int kSb = 0;
  static constexpr int kX = kSb + 2 * NT * 2;
  static constexpr int kE = kX + 2 * 2 * NT;
  static constexpr int kPerParity = kE + 2;
  static constexpr size_t kBytes = (size_t)2 * kPerParity * 64 * 16;
  __device__ static int sb(int par, int w, int nt, int mm) { return (par * kPerParity + kSb + (w * NT + nt) * 2 + mm) * 64; }
  __device__ static int x(int par, int w, int t, int nt) { return (par * kPerParity + kX + (w * 2 + t) * NT + nt) * 64; }
  __device__ static int e(int par, int w) { return (par * kPerParity + kE + w) * 64; }
};

// Fragments a state wave of the wide kernel consumes per chunk.
template <int NT>
struct WideStateFrags {
  bf16x8 w[2][2];  // -W fragments: row tile t, key block 2*wave + mm
  bf16x8 k[4];     // K fragments: key tiles 4*wave .. 4*wave + 3
  float e;         // exp(G_C) of key 64*wave + lane
  bf16x8 u[NT];    // U fragments of this workgroup's value tiles (wave 0 only)
};

template <int NT>
__device__ __forceinline__ void load_wide_state_frags(WideStateFrags<NT>& f, __amdgpu_buffer_rsrc_t rs, int coff,
                                                      int vo, int wave, int vtile0) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
      f.w[t][mm] = bload8(rs, vo, coff + (int)kRecW + (t * 4 + 2 * wave + mm) * (int)kFrag);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) f.k[tt] = bload8(rs, vo, coff + (int)kRecK + (4 * wave + tt) * (int)kFrag);
  // One float per lane (256 bytes per wave), redistributed through LDS.
  f.e = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo >> 2, coff + (int)kRecE + 256 * wave, 0));
  // Last, so that the other loads' wait counts do not depend on whether U was loaded.
  if (wave == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) f.u[nt] = bload8(rs, vo, coff + (int)kRecU + (vtile0 + nt) * (int)kFrag);
  }
}

template <int NT, int SDT, int DEPTH>
__global__ __launch_bounds__(256, 2) void scan_wide(Plan p, int units, int groups) {
  extern __shared__ __attribute__((aligned(16))) u32x4 wlds[];
  typedef WideLds<NT> L;
  Unit un;
  if (!unit_of(p, units, groups, un)) return;
  const int n = un.n, h = un.h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  const int vtile0 = un.grp * NT;
  const int cu0 = p.d_cu[n] + kChunk * un.c0, cu1 = p.d_cu[n + 1];  // segment start, sequence end
  const int nc = un.nch;
  const char* rec0 =
      reinterpret_cast<const char*>(p.ws) + ((size_t)h * p.n_chunks + p.d_co[n] + un.c0) * kRecBytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rec0), (short)0, nc * (int)kRecBytes, kBufWord3);
  const int vo = lane * 16;

  if (wave < 2) {
    // ------------------------------------------------------------ state waves
    // Lane holds S^T[k][v] for k = 16*(4*wave+tt) + 4*g4 + i, v = 16*(vtile0 + nt) + l16.
    f32x4 S[NT][4];
    const void* in_plane = state_in_plane<SDT>(p, n, h);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const size_t off = (size_t)(16 * (vtile0 + nt) + l16) * kHead + 16 * (4 * wave + tt) + 4 * g4;
        S[nt][tt] = load_start4<SDT>(p, un, in_plane, off);
      }
    typedef WideStateFrags<NT> F;
    if (nc > 0) {
      pipelined_chunks<DEPTH, F>(
          nc, [&](F& f, int c) { load_wide_state_frags<NT>(f, rs, c * (int)kRecBytes, vo, wave, vtile0); },
          [&](const F& f, int c) {
            const int par = c & 1;
            bf16x8 Sb[NT][2];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int mm = 0; mm < 2; ++mm) {
                Sb[nt][mm] = pack8(S[nt][2 * mm], S[nt][2 * mm + 1]);
                wlds[L::sb(par, wave, nt, mm) + lane] = __builtin_bit_cast(u32x4, Sb[nt][mm]);
              }
            // Partial (-W) S^T over this wave's 64 keys, both row tiles; wave 0 starts
            // from U, so the two partials add up to Delta.
            f32x4 X[2][NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int t = 0; t < 2; ++t) {
                f32x4 a = zero4();
                if (wave == 0) {
#pragma unroll
                  for (int i = 0; i < 4; ++i) a[i] = from_bf16(f.u[nt][4 * t + i]);
                }
                a = mfma(f.w[t][0], Sb[nt][0], a);
                a = mfma(f.w[t][1], Sb[nt][1], a);
                X[t][nt] = a;
                wlds[L::x(par, wave, t, nt) + lane] = __builtin_bit_cast(u32x4, a);
              }
            reinterpret_cast<float*>(wlds + L::e(par, wave))[lane] = f.e;
            barrier_lds();
            // exp(G_C) of this lane's key rows (lane k of the wave loaded key 64*wave + k).
            const float* eb = reinterpret_cast<const float*>(wlds + L::e(par, wave));
            f32x4 E[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) E[tt] = *reinterpret_cast<const f32x4*>(eb + 16 * tt + 4 * g4);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              // Delta: a + b == b + a, so every wave rebuilds identical bits.
              const f32x4 d0 = X[0][nt] + __builtin_bit_cast(f32x4, wlds[L::x(par, wave ^ 1, 0, nt) + lane]);
              const f32x4 d1 = X[1][nt] + __builtin_bit_cast(f32x4, wlds[L::x(par, wave ^ 1, 1, nt) + lane]);
              const bf16x8 Db = pack8(d0, d1);
#pragma unroll
              for (int tt = 0; tt < 4; ++tt) S[nt][tt] = mfma(f.k[tt], Db, S[nt][tt] * E[tt]);
            }
          });
    }
    void* out_plane = un.m_self < 0 ? state_out_plane<SDT>(p, n, h) : nullptr;
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
    // ------------------------------------------------------------ output waves
    const int t = wave - 2;
    const size_t row_stride = (size_t)p.H * kHead;
    const int orow = 16 * t + l16;
    const size_t ooff = (size_t)orow * row_stride + (size_t)h * kHead + 16 * vtile0 + 4 * g4;
    typedef OutFrags F;
    if (nc > 0) {
      pipelined_chunks<DEPTH, F>(
          nc, [&](F& f, int c) { load_out_frags(f, rs, c * (int)kRecBytes, vo, t); },
          [&](const F& f, int c) {
            const int par = c & 1;
            barrier_lds();  // the state waves have published chunk c's copies and partials
            const int t0 = cu0 + kChunk * c;
            const int len = min(kChunk, cu1 - t0);
            __bf16* out_c = reinterpret_cast<__bf16*>(p.out) + (size_t)t0 * row_stride + ooff;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const f32x4 d0 = __builtin_bit_cast(f32x4, wlds[L::x(par, 0, 0, nt) + lane]) +
                               __builtin_bit_cast(f32x4, wlds[L::x(par, 1, 0, nt) + lane]);
              const f32x4 d1 = __builtin_bit_cast(f32x4, wlds[L::x(par, 0, 1, nt) + lane]) +
                               __builtin_bit_cast(f32x4, wlds[L::x(par, 1, 1, nt) + lane]);
              const bf16x8 Db = pack8(d0, d1);
              // (Q S^T)^T = S Q^T over all 128 keys: key block m lives in state wave m / 2.
              f32x4 o = zero4();
#pragma unroll
              for (int m = 0; m < 4; ++m)
                o = mfma(__builtin_bit_cast(bf16x8, wlds[L::sb(par, m >> 1, nt, m & 1) + lane]), f.q[m], o);
              o = mfma(Db, f.p, o);  // + Delta^T P^T
              if (orow < len) {
                const bf16x4 ov = {to_bf16(o[0]), to_bf16(o[1]), to_bf16(o[2]), to_bf16(o[3])};
                *reinterpret_cast<bf16x4*>(out_c + 16 * nt) = ov;
              }
            }
          });
    }
  }
}

// ====================================================================== launch
template <typename KernelT>
int set_lds_limit(KernelT* kernel, size_t bytes, bool& done) {
  if (done) return 0;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)bytes);
  if (e != hipSuccess) return (int)e;
  done = true;
  return 0;
}

template <int NT, int SDT>
int launch_nt(const Plan& p, hipStream_t s) {
  const int groups = 8 / NT;
  const int units = p.n_seg * p.H;
  const int nblocks = 8 * ((units + 7) / 8) * groups;
  if constexpr (NT <= 2) {
    constexpr int R = 5;                 // ring slots: the loader runs 4 chunks ahead
    constexpr int DO = NT == 1 ? 4 : 3;  // output-wave fragment depth
    constexpr size_t bytes = NarrowLds<NT, R>::kBytes;
    static_assert(bytes <= 160 * 1024, "fits one CU's LDS");
    static bool done = false;
    if (int e = set_lds_limit(&scan_narrow<NT, SDT, R, DO>, bytes, done)) return e;
    hipLaunchKernelGGL((scan_narrow<NT, SDT, R, DO>), dim3(nblocks), dim3(kThreadsScan), bytes, s, p, units, groups);
  } else {
    constexpr int D = 2;
    constexpr size_t bytes = WideLds<NT>::kBytes;
    static_assert(2 * bytes <= 160 * 1024, "two workgroups per CU");
    static bool done = false;
    if (int e = set_lds_limit(&scan_wide<NT, SDT, D>, bytes, done)) return e;
    hipLaunchKernelGGL((scan_wide<NT, SDT, D>), dim3(nblocks), dim3(kThreadsScan), bytes, s, p, units, groups);
  }
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
