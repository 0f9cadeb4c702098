// Serial scan kernel for chunkwise KDA prefill on gfx950, and the segment-map pass that
// shares its machinery.
//
// The serial pass over each sequence's chunks that carries the state (aiter PR 4741,
// Summary: the second of its two kernels), with paged or dense state read and written
// in-kernel (aiter PR 5754, Technical Details) and fp16/bf16 state storage up-cast to
// fp32 on load and rounded to nearest even on store (aiter PR 5249, What). Per chunk,
// with S the V x K state at the chunk start and the prep tiles W, U, Q, K, P, E:
//
//   Delta = U - W S^T      (the record holds -W: an MFMA accumulation started from U)
//   O     = Q S^T + P Delta              (scale folded into Q and P in prep)
//   S     = S Diag(E) + Delta^T K
//
// One workgroup per (segment, head[, half of the value channels]); a segment is a whole
// sequence unless the call is segmented, then it starts from the state the combine
// kernel computed and only a sequence's last segment writes the final state.
//
// Every value channel of a head needs the whole W, K, Q and P of each chunk, and a
// CU takes in only so many bytes per cycle, so the kernel serves as many value channels
// per workgroup as the registers allow: five waves,
//   * waves 0..3 (state waves) each hold the fp32 state of 16*NTW value channels for all
//     128 keys in MFMA accumulator layout and run the recurrence and the output of
//     those channels: Delta (accumulated from U), the state update, and
//     O^T = S Q^T + Delta^T P^T from the bf16 state copy and Delta the step used;
//   * wave 4 (loader) copies W, K, U, Q, P and E of each chunk into a ring of LDS slots
//     with direct-to-LDS buffer loads, so the state waves never issue a global load.
// One barrier per chunk orders the ring.
//
// The segment-map pass (for the segmented scan) is the same recurrence without output
// on 256 rows of an augmented state: 128 rows that start as the identity with U = 0
// (they end as the segment's transition A) and 128 rows that start at zero with the
// chunk's U (they end as the state C the segment reaches from zero); one workgroup per
// half.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// Loader modes: the scan, and the two halves of the map pass.
enum { kModeScan = 0, kModeMapA = 1, kModeMapC = 2 };
// Kernel modes: the scan, or the map pass (both halves in one grid).
enum { kKernelScan = 0, kKernelMap = 1 };

// LDS ring of kRing chunk slots: W 8, K 8, U 4*NTW, Q 8 and P 2 fragments of 1 KB, then
// E (128 fp32).
template <int NTW>
struct HeadLds {
  static constexpr int kRing = 4;
  static constexpr int kSlotW = 0;
  static constexpr int kSlotK = 8 * 1024;
  static constexpr int kSlotU = 16 * 1024;
  static constexpr int kSlotQ = kSlotU + 4 * NTW * 1024;
  static constexpr int kSlotP = kSlotQ + 8 * 1024;
  static constexpr int kSlotE = kSlotP + 2 * 1024;
  static constexpr int kSlot = kSlotE + 512;
  static constexpr size_t kBytes = (size_t)kRing * kSlot;
};

// What one workgroup serves: a (segment, head) and a group of value channels.
struct Unit {
  int n, h, grp;
  int c0, nch;         // first chunk within the sequence, chunks
  int m_prev, m_self;  // scan: start-state slot (-1: the caller's initial state), own map slot
                       // (-1: last segment); map: the map slot
};

// The chunk's decay exp(G_C) for the state rows a lane holds. A lane's rows are keys
// k = 16*tt + 4*g4 + i (key tile tt, register i), so the 16 lanes of a row g4 all need
// the same 32 keys and the wave only 128. Each lane reads two of its row's keys,
// 16*(j/4) + 4*g4 + j%4 and the same + 64 (j = lane within the row), and the decay of
// key tile tt, register i is broadcast along the row from lane 4*(tt%4) + i, register
// tt/4 (DPP row_newbcast, folded into the multiply): one two-word LDS read per step in
// place of eight 16-byte ones, and no more VALU instructions.
__device__ __forceinline__ void read_decay(float (&e)[2], const char* slot_e, int g4, int l16) {
  const float* E = reinterpret_cast<const float*>(slot_e) + 16 * (l16 >> 2) + 4 * g4 + (l16 & 3);
  e[0] = E[0];
  e[1] = E[64];
}

template <int J>
__device__ __forceinline__ float row_bcast(float x) {
  // Every lane's source (lane J of its row) exists, so bound_ctrl does not matter; set,
  // it lets the compiler fold the move into the multiply.
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + J, 0xf, 0xf, true));
}


// S^T[k][v] *= exp(G_C)[k] for key tile TT alone.
template <int TT>
__device__ __forceinline__ void decay_tile(f32x4& s, const float (&e)[2]) {
  constexpr int J = 4 * (TT & 3);
  s[0] *= row_bcast<J + 0>(e[TT >> 2]);
  s[1] *= row_bcast<J + 1>(e[TT >> 2]);
  s[2] *= row_bcast<J + 2>(e[TT >> 2]);
  s[3] *= row_bcast<J + 3>(e[TT >> 2]);
}

// S^T[k][v] *= exp(G_C)[k] for key tiles TT..7.
template <int TT = 0>
__device__ __forceinline__ void decay_state(f32x4 (&S)[8], const float (&e)[2]) {
  if constexpr (TT < 8) {
    decay_tile<TT>(S[TT], e);
    decay_state<TT + 1>(S, e);
  }
}

// S^T = Diag(E) S^T + K^T Delta, key tile by key tile, for a state whose tiles 0 and 1
// are already decayed: the decay of tile TT + 2 is issued next to the update MFMA of
// tile TT, so that its multiplies run while the matrix unit works (the schedule is fixed
// by the group barriers in update_groups).
template <int TT = 0>
__device__ __forceinline__ void update_interleaved(f32x4 (&S)[8], const bf16x8 (&k)[8], bf16x8 db, const float (&e)[2]) {
  if constexpr (TT < 8) {
    S[TT] = mfma(k[TT], db, S[TT]);
    if constexpr (TT + 2 < 8) decay_tile<TT + 2>(S[TT + 2], e);
    update_interleaved<TT + 1>(S, k, db, e);
  }
}

// Issue order of one update_interleaved: each update MFMA, then the four multiplies of
// a later tile's decay.
template <int TT = 0>
__device__ __forceinline__ void update_groups() {
  if constexpr (TT < 8) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
    if constexpr (TT + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
    update_groups<TT + 1>();
  }
}

// A operand that copies U into the Delta accumulators on the matrix unit instead of
// widening it on the vector ALU. The U fragment, taken as a B operand, holds in element
// j of lane group g the chunk row 16*(j/4) + 4g + j%4 (the accumulator rows of both row
// tiles). Row m of u_select(t) has a single 1, at the element that holds row 16t + m, so
// mfma(u_select(t), U, 0) is rows 16t..16t+15 of U, exactly and in accumulator layout;
// the W products then accumulate onto the same fp32 values as before.
__device__ __forceinline__ bf16x8 u_select(int t, int g4, int l16) {
  const int d = l16 - 4 * g4;  // row l16 sits in element d + 4t of group g4 if 0 <= d < 4
  bf16x8 a;
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = to_bf16(d >= 0 && d < 4 && j == d + 4 * t ? 1.f : 0.f);
  return a;
}

// Workgroups are dealt round-robin to the 8 XCDs; all groups of one unit land on one
// XCD, so its records are fetched into that XCD's L2 once. Scan: units are (segment,
// head), groups the value-channel halves. Map: units are (map slot, head), groups the
// halves A and C.
template <int KMODE>
__device__ __forceinline__ bool unit_of(const Plan& p, int units, int groups, Unit& u) {
  // Every field is uniform. readfirstlane keeps each in a scalar register: the integer
  // divisions below run on vector ALUs, and the compiler cannot always prove the loads
  // unclobbered; a buffer descriptor built from vector registers would make every load
  // that uses it loop over the lanes.
  const int bidx = blockIdx.x;
  const int xcd = bidx & 7;
  const int slot8 = bidx >> 3;
  const int local = __builtin_amdgcn_readfirstlane(slot8 / groups);
  u.grp = __builtin_amdgcn_readfirstlane(slot8 - local * groups);
  const int id = local * 8 + xcd;
  if (id >= units) return false;
  const int q = __builtin_amdgcn_readfirstlane(id / p.H);
  u.h = __builtin_amdgcn_readfirstlane(id - q * p.H);
  const int s = KMODE == kKernelScan ? q : __builtin_amdgcn_readfirstlane(p.d_m2s[q]);
  const int32_t* e = p.d_seg + (size_t)kSegInts * s;
  u.n = __builtin_amdgcn_readfirstlane(e[0]);
  u.c0 = __builtin_amdgcn_readfirstlane(e[1]);
  u.nch = __builtin_amdgcn_readfirstlane(e[2]);
  u.m_prev = __builtin_amdgcn_readfirstlane(e[3]);
  u.m_self = KMODE == kKernelScan ? __builtin_amdgcn_readfirstlane(e[4]) : q;
  return true;
}

// Loader wave. Chunk c goes to slot c mod kRing. Before barrier c (and the first
// barrier, for chunk 0) chunk c + 1 has landed; right after that wait it issues chunk
// c + 3 into the slot of chunk c - 1, which the state waves finished reading before
// barrier c - 1. Only chunks < nc are loaded. Its barriers carry no fence (a fence
// would wait for every direct-to-LDS load in flight).
template <int NTW, int MODE>
__device__ __forceinline__ void loader(char* lds, __amdgpu_buffer_rsrc_t rs, int nc, int lane, int u0) {
  typedef HeadLds<NTW> L;
  constexpr int kU = MODE == kModeScan ? 4 * NTW : (MODE == kModeMapC ? 8 : 0);
  constexpr bool kOut = MODE == kModeScan;
  constexpr int kLoads = 8 + 8 + kU + (kOut ? 10 : 0) + 2;
  static_assert(kLoads < 64, "one chunk of loads fits the wait counter");
  static_assert(L::kRing == 4, "the schedule below keeps at most one chunk behind the awaited one");
  const int vo = lane * 16;
  auto issue = [&](int c) {
    char* base = lds + (c & (L::kRing - 1)) * L::kSlot;
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
    for (int f = 0; f < kU; ++f)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotU + f * 1024), 16, vo,
                                               soff + (int)kRecU + (u0 + f) * (int)kFrag, 0, 0);
    if constexpr (kOut) {
#pragma unroll
      for (int f = 0; f < 8; ++f)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotQ + f * 1024), 16, vo,
                                                 soff + (int)kRecQ + f * (int)kFrag, 0, 0);
#pragma unroll
      for (int f = 0; f < 2; ++f)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotP + f * 1024), 16, vo,
                                                 soff + (int)kRecP + f * (int)kFrag, 0, 0);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotE + half * 256), 4, lane * 4,
                                               soff + (int)kRecE + half * 256, 0, 0);
  };
  issue(0);
  if (nc > 1) issue(1);
  wait_chunks<kLoads, 1>(min(1, nc - 1));  // chunk 0 has landed
  if (nc > 2) issue(2);
  __builtin_amdgcn_s_barrier();
  for (int c = 0; c < nc; ++c) {
    // Issued so far: chunks up to min(c + 2, nc - 1); only chunk c + 2 may stay in flight.
    wait_chunks<kLoads, 1>(min(1, nc - 2 - c));
    if (c + 3 < nc) issue(c + 3);
    __builtin_amdgcn_s_barrier();
  }
}

// KF: the caller's state planes are K-first [K][V] (state I/O only; the map mode reads
// and writes no caller state and uses KF = false).
template <int NTW, int SDT, int KMODE, bool KF>
__global__ __launch_bounds__(320, 1) void head_kernel(Plan p, int units, int groups) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  typedef HeadLds<NTW> L;
  Unit un;
  if (!unit_of<KMODE>(p, units, groups, un)) return;
  constexpr bool kScan = KMODE == kKernelScan;
  const bool part_a = !kScan && un.grp == 0;  // map half A: identity start, U = 0
  const int n = un.n, h = un.h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  const int vo = lane * 16;  // lane offset inside a fragment
  const int nc = un.nch;
  const int cu0 = __builtin_amdgcn_readfirstlane(p.d_cu[n]) + kChunk * un.c0;  // segment start
  const int cu1 = __builtin_amdgcn_readfirstlane(p.d_cu[n + 1]);              // sequence end
  const int co = __builtin_amdgcn_readfirstlane(p.d_co[n]);
  const char* rec0 = reinterpret_cast<const char*>(p.ws) + ((size_t)h * p.n_chunks + co + un.c0) * kRecBytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rec0), (short)0, nc * (int)kRecBytes, kBufWord3);
  // Value tiles of the workgroup start at u0 (scan: its half; map: all 8).
  const int u0 = kScan ? un.grp * 4 * NTW : 0;

  if (wave == 4) {
    if (nc > 0) {
      if (kScan) loader<NTW, kModeScan>(lds, rs, nc, lane, u0);
      else if (part_a) loader<NTW, kModeMapA>(lds, rs, nc, lane, u0);
      else loader<NTW, kModeMapC>(lds, rs, nc, lane, u0);
    }
    return;
  }

  // State wave: value tiles vt = vt0 + nt; lane holds S^T[k][v] for k = 16*tt + 4*g4 + i
  // (key tile tt = 0..7), v = 16*vt + l16.
  const int vt0 = u0 + NTW * wave;
  f32x4 S[NTW][8];
  if constexpr (kScan) {
    const void* in_plane = state_in_plane<SDT>(p, n, h);
    const float* start = un.m_prev >= 0 ? p.starts + ((size_t)un.m_prev * p.H + h) * kHead * kHead : nullptr;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int v = 16 * (vt0 + nt) + l16, k = 16 * tt + 4 * g4;
        S[nt][tt] = start ? load_state4<kF32>(start, (size_t)v * kHead + k)
                          : (in_plane ? load_state4_vk<SDT>(in_plane, v, k, KF) : zero4());
      }
  } else {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[nt][tt][i] = (part_a && 16 * tt + 4 * g4 + i == 16 * (vt0 + nt) + l16) ? 1.f : 0.f;
  }

  // Ring reads, issued together in order of first use and pinned in that order (the
  // scheduler would otherwise sink each read to its use or permute them): the LDS
  // counter can name at most 15 reads in flight, so the wait before the first MFMA then
  // covers W, U and little else. (Reading U first, as the narrow kernel does, measured
  // slower in this kernel.)
  struct Frags {
    bf16x8 w[2][4];  // -W (row tile t, key block m)
    bf16x8 u[NTW];   // U of this wave's value tiles
    bf16x8 k[8];     // K (key tile)
    float e[2];      // exp(G_C), two keys of this lane's row (read_decay)
  };
  auto read = [&](Frags& f, const char* sl) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f.w[t][m] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotW + (t * 4 + m) * 1024 + vo);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      // (Half A loads no U: its slot area holds stale bytes, replaced by zero.)
      const bf16x8 u = *reinterpret_cast<const bf16x8*>(sl + L::kSlotU + (vt0 + nt - u0) * 1024 + vo);
      f.u[nt] = part_a ? bf16x8{} : u;
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      f.k[tt] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotK + tt * 1024 + vo);
      __builtin_amdgcn_sched_barrier(0);
    }
    read_decay(f.e, sl + L::kSlotE, g4, l16);
    __builtin_amdgcn_sched_barrier(0);
  };

  const size_t row_stride = (size_t)p.H * kHead;
  const bf16x8 usel[2] = {u_select(0, g4, l16), u_select(1, g4, l16)};
  if (nc > 0) {
    barrier_lds();  // the loader has chunk 0 in slot 0
    Frags f;
    read(f, lds);
    for (int c = 0; c < nc; ++c) {
      const char* sl = lds + (c & (L::kRing - 1)) * L::kSlot;
      // bf16 copy of the state: key block m holds key tiles 2m, 2m+1 (the record's W
      // and Q fragments use the same key order).
      bf16x8 Sb[NTW][4];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int m = 0; m < 4; ++m) Sb[nt][m] = pack8(S[nt][2 * m], S[nt][2 * m + 1]);
      // Delta = U + (-W) S^T, accumulated from U (copied in by an MFMA); rows
      // {4g..4g+3, 16+4g..16+4g+3}.
      f32x4 x[NTW][2];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 a = mfma(usel[t], f.u[nt], zero4());
#pragma unroll
          for (int m = 0; m < 4; ++m) a = mfma(f.w[t][m], Sb[nt][m], a);
          x[nt][t] = a;
        }
      // Diag(E) S^T while the MFMAs above run.
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) decay_state(S[nt], f.e);
      bf16x8 Db[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) Db[nt] = pack8(x[nt][0], x[nt][1]);
      // S^T = Diag(E) S^T + K^T Delta.
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) S[nt][tt] = mfma(f.k[tt], Db[nt], S[nt][tt]);
      if constexpr (kScan) {
        // O^T = S Q^T + Delta^T P^T for row tile t: lane holds rows v = 16*vt + 4*g4 ..
        // + 3 of token row 16*t + l16.
        const int t0 = cu0 + kChunk * c;
        const int len = min(kChunk, cu1 - t0);
        __bf16* out_c = reinterpret_cast<__bf16*>(p.out) + (size_t)t0 * row_stride + (size_t)h * kHead + 4 * g4;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16x8 q[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) q[m] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotQ + (t * 4 + m) * 1024 + vo);
          const bf16x8 pf = *reinterpret_cast<const bf16x8*>(sl + L::kSlotP + t * 1024 + vo);
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
            f32x4 o = zero4();
#pragma unroll
            for (int m = 0; m < 4; ++m) o = mfma(Sb[nt][m], q[m], o);
            o = mfma(Db[nt], pf, o);
            const int row = 16 * t + l16;
            if (row < len) {
              const bf16x4 ov = {to_bf16(o[0]), to_bf16(o[1]), to_bf16(o[2]), to_bf16(o[3])};
              *reinterpret_cast<bf16x4*>(out_c + (size_t)row * row_stride + 16 * (vt0 + nt)) = ov;
            }
          }
        }
      }
      barrier_lds();  // the loader has chunk c + 1 in its slot
      if (c + 1 < nc) read(f, lds + ((c + 1) & (L::kRing - 1)) * L::kSlot);
    }
  }

  if constexpr (kScan) {
    void* out_plane = un.m_self < 0 ? state_out_plane<SDT>(p, n, h) : nullptr;
    if (out_plane) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
          store_state4_vk<SDT>(out_plane, 16 * (vt0 + nt) + l16, 16 * tt + 4 * g4, S[nt][tt], KF);
    }
  } else {
    // Map slot layout (kMapBytes): A^T as bf16 hi and lo planes in the combine kernel's
    // MFMA operand fragment order (map_frag_index), then C in fp32 in S order (element
    // (v, k) at [v][k]).
    char* base = reinterpret_cast<char*>(p.maps) + (size_t)(un.m_self * p.H + h) * kMapBytes;
    if (part_a) {
      // Wave w holds input keys k' = 32w .. 32w + 31 (NTW = 2), i.e. key block w of every
      // fragment: it transposes them through its own LDS region (the ring is no longer
      // read once every chunk is done) and writes each fragment row as 16 bytes.
      static_assert(NTW == 2, "one key block of 32 input keys per wave");
      constexpr int kLdT = 40;  // bf16 per LDS row: 32 input keys + pad
      __bf16* th = reinterpret_cast<__bf16*>(lds) + wave * 2 * kHead * kLdT;
      __bf16* tl = th + kHead * kLdT;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int at = (16 * tt + 4 * g4 + i) * kLdT + 16 * nt + l16;
            split_bf16(S[nt][tt][i], th[at], tl[at]);
          }
      __bf16* hi = reinterpret_cast<__bf16*>(base);
      __bf16* lo = hi + kHead * kHead;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        // Fragment (kt, kb = wave), lane (l16, g4): A^T[16 kt + l16][32 wave + 8 g4 .. + 7].
        const int src = (16 * kt + l16) * kLdT + 8 * g4;
        const int dst = map_frag_index(16 * kt + l16, 32 * wave + 8 * g4);
        *reinterpret_cast<bf16x8*>(hi + dst) = *reinterpret_cast<const bf16x8*>(th + src);
        *reinterpret_cast<bf16x8*>(lo + dst) = *reinterpret_cast<const bf16x8*>(tl + src);
      }
    } else {
      float* dst = reinterpret_cast<float*>(base + kHead * kHead * 4);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
          *reinterpret_cast<f32x4*>(dst + (size_t)(16 * (vt0 + nt) + l16) * kHead + 16 * tt + 4 * g4) = S[nt][tt];
    }
  }
}

// One state row group of four: the segment's start state (fp32, from the combine
// kernel), the call's initial state, or zero.
template <int SDT, bool KF>
__device__ __forceinline__ f32x4 load_start4(const Plan& p, const Unit& u, const void* in_plane, int v, int k) {
  if (u.m_prev >= 0) return load_state4<kF32>(p.starts + ((size_t)u.m_prev * p.H + u.h) * kHead * kHead, (size_t)v * kHead + k);
  return in_plane ? load_state4_vk<SDT>(in_plane, v, k, KF) : zero4();
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
// For few (segment, head) units, where per-chunk latency rather than the chip's total
// load bandwidth bounds the call: 16*NT value channels per workgroup, one state wave,
// one output wave (both row tiles, so the published state copy and Delta are read once
// per chunk) and a loader, so that the state wave's chain carries no output work and
// reads only W, K, U and E.
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

template <int NT, int SDT, int RING, int DOUT, bool KF>
__global__ __launch_bounds__(192, 1) void scan_narrow(Plan p, int units, int groups) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  typedef NarrowLds<NT, RING> L;
  Unit un;
  if (!unit_of<kKernelScan>(p, units, groups, un)) return;
  const int n = un.n, h = un.h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  const int vtile0 = un.grp * NT;  // first 16-channel value tile of this workgroup
  const int cu0 = __builtin_amdgcn_readfirstlane(p.d_cu[n]) + kChunk * un.c0;  // segment start
  const int cu1 = __builtin_amdgcn_readfirstlane(p.d_cu[n + 1]);              // sequence end
  const int nc = un.nch;
  const int co = __builtin_amdgcn_readfirstlane(p.d_co[n]);
  const char* rec0 = reinterpret_cast<const char*>(p.ws) + ((size_t)h * p.n_chunks + co + un.c0) * kRecBytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rec0), (short)0, nc * (int)kRecBytes, kBufWord3);
  const int vo = lane * 16;  // lane offset inside a fragment

  if (wave == 2) {
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
      for (int g = 0; g < 8; ++g) {  // the workgroups of a head start at different fragments
        const int f = (g + un.grp) & 7;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotW + f * 1024), 16, vo,
                                                 soff + (int)kRecW + f * (int)kFrag, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int f = (g + un.grp) & 7;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotK + f * 1024), 16, vo,
                                                 soff + (int)kRecK + f * (int)kFrag, 0, 0);
      }
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
      for (int tt = 0; tt < 8; ++tt) S[nt][tt] = load_start4<SDT, KF>(p, un, in_plane, 16 * (vtile0 + nt) + l16, 16 * tt + 4 * g4);

    // One chunk's fragments, read from its ring slot.
    // Issued together, in order of first use and pinned in that order (the scheduler
    // would otherwise sink each read to its use or permute them): U, which the first
    // MFMA of each Delta chain copies, then W by key block, both row tiles' fragments of
    // a block together, so that both chains start while the rest of W, K and E land.
    struct Frags {
      bf16x8 w[2][4];  // -W (row tile t, key block m)
      bf16x8 u[NT];    // U of this workgroup's value tiles
      bf16x8 k[8];     // K (key tile)
      float e[2];      // exp(G_C), two keys of this lane's row (read_decay)
    };
    auto read = [&](Frags& f, int slot) {
      const char* sl = lds + slot * L::kSlot;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f.u[nt] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotU + nt * 1024 + vo);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f.w[t][m] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotW + (t * 4 + m) * 1024 + vo);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        f.k[tt] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotK + tt * 1024 + vo);
        __builtin_amdgcn_sched_barrier(0);
      }
      read_decay(f.e, sl + L::kSlotE, g4, l16);
      __builtin_amdgcn_sched_barrier(0);
    };

    const bf16x8 usel[2] = {u_select(0, g4, l16), u_select(1, g4, l16)};
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
        // Delta = U + (-W) S^T, accumulated from U (copied in by an MFMA); rows
        // {4g..4g+3, 16+4g..16+4g+3} of the chunk per lane.
        f32x4 x[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            f32x4 a = mfma(usel[t], f.u[nt], zero4());
#pragma unroll
            for (int m = 0; m < 4; ++m) a = mfma(f.w[t][m], Sb[nt][m], a);
            x[nt][t] = a;
          }
        // Publish the state copy after the MFMAs are issued (they need only registers).
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int m = 0; m < 4; ++m) *reinterpret_cast<bf16x8*>(lds + L::sb(par, nt, m) + vo) = Sb[nt][m];
        // Diag(E) S^T for key tiles 0 and 1 while the last Delta MFMAs run; the other
        // tiles' decay goes between the update MFMAs below.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          decay_tile<0>(S[nt][0], f.e);
          decay_tile<1>(S[nt][1], f.e);
        }
        bf16x8 Db[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          Db[nt] = pack8(x[nt][0], x[nt][1]);
          *reinterpret_cast<bf16x8*>(lds + L::db(par, nt) + vo) = Db[nt];
        }
        // Every LDS write of the step is issued before the update MFMAs, and the barrier
        // after them (below), so that the MFMAs cover the writes' latency; sunk below the
        // MFMAs, or the barrier hoisted above them, the writes would hold its wait.
        __builtin_amdgcn_sched_barrier(0);
        // S^T = Diag(E) S^T + K^T Delta.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) update_interleaved(S[nt], f.k, Db[nt], f.e);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) update_groups();
        __builtin_amdgcn_sched_barrier(0);
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
        for (int tt = 0; tt < 8; ++tt)
          store_state4_vk<SDT>(out_plane, 16 * (vtile0 + nt) + l16, 16 * tt + 4 * g4, S[nt][tt], KF);
    }
  } else {
    // ------------------------------------------------------------ output wave
    // Both row tiles, so that the published Sb and Db are read from LDS once per chunk.
    const size_t row_stride = (size_t)p.H * kHead;
    // Lane holds O^T rows v = 16*(vtile0+nt) + 4*g4 .. +3 of token row 16*t + l16.
    const size_t ooff = (size_t)l16 * row_stride + (size_t)h * kHead + 16 * vtile0 + 4 * g4;
    struct F {
      OutFrags t[2];
    };
    if (nc > 0) {
      barrier_lds();  // pairs with the first barrier of the other waves
      pipelined_chunks<DOUT, F>(
          nc,
          [&](F& f, int c) {
            load_out_frags(f.t[0], rs, c * (int)kRecBytes, vo, 0);
            load_out_frags(f.t[1], rs, c * (int)kRecBytes, vo, 1);
          },
          [&](const F& f, int c) {
            const int par = c & 1;
            barrier_lds();  // the state wave has published chunk c's Sb and Db
            const int t0 = cu0 + kChunk * c;
            const int len = min(kChunk, cu1 - t0);
            __bf16* out_c = reinterpret_cast<__bf16*>(p.out) + (size_t)t0 * row_stride + ooff;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              bf16x8 sb[4];
#pragma unroll
              for (int m = 0; m < 4; ++m) sb[m] = *reinterpret_cast<const bf16x8*>(lds + L::sb(par, nt, m) + vo);
              const bf16x8 db = *reinterpret_cast<const bf16x8*>(lds + L::db(par, nt) + vo);
#pragma unroll
              for (int t = 0; t < 2; ++t) {
                // (Q S^T)^T = S Q^T, then + Delta^T P^T.
                f32x4 o = zero4();
#pragma unroll
                for (int m = 0; m < 4; ++m) o = mfma(sb[m], f.t[t].q[m], o);
                o = mfma(db, f.t[t].p, o);
                if (16 * t + l16 < len) {
                  const bf16x4 ov = {to_bf16(o[0]), to_bf16(o[1]), to_bf16(o[2]), to_bf16(o[3])};
                  *reinterpret_cast<bf16x4*>(out_c + (size_t)16 * t * row_stride + 16 * nt) = ov;
                }
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

template <int NTW, int SDT, bool KF>
int launch_scan_ntw(const Plan& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr size_t bytes = HeadLds<NTW>::kBytes;
  static_assert(bytes <= 160 * 1024, "fits one CU's LDS");
  static bool done = false;
  if (int e = set_lds_limit(&head_kernel<NTW, SDT, kKernelScan, KF>, bytes, done)) return e;
  const int groups = 2 / NTW;  // value-channel halves per (segment, head)
  const int units = p.n_seg * p.H;
  const int nblocks = 8 * ((units + 7) / 8) * groups;
  hipExtLaunchKernelGGL((head_kernel<NTW, SDT, kKernelScan, KF>), dim3(nblocks), dim3(320), bytes, s, e0, e1, 0, p, units,
                        groups);
  return (int)hipGetLastError();
}

template <int NT, int SDT, bool KF>
int launch_narrow(const Plan& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int R = 5;                 // ring slots: the loader runs 4 chunks ahead
  constexpr int DO = NT == 1 ? 4 : 3;  // output-wave fragment depth
  constexpr size_t bytes = NarrowLds<NT, R>::kBytes;
  static_assert(bytes <= 160 * 1024, "fits one CU's LDS");
  static bool done = false;
  if (int e = set_lds_limit(&scan_narrow<NT, SDT, R, DO, KF>, bytes, done)) return e;
  const int groups = 8 / NT;
  const int units = p.n_seg * p.H;
  const int nblocks = 8 * ((units + 7) / 8) * groups;
  hipExtLaunchKernelGGL((scan_narrow<NT, SDT, R, DO, KF>), dim3(nblocks), dim3(192), bytes, s, e0, e1, 0, p, units, groups);
  return (int)hipGetLastError();
}

template <int SDT, bool KF>
int launch_scan_kf(const Plan& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (p.dv_split) {
    case 8: return launch_narrow<1, SDT, KF>(p, s, e0, e1);
    case 4: return launch_narrow<2, SDT, KF>(p, s, e0, e1);
    case 2: return launch_scan_ntw<1, SDT, KF>(p, s, e0, e1);
    default: return launch_scan_ntw<2, SDT, KF>(p, s, e0, e1);
  }
}

template <int SDT>
int launch_scan_dt(const Plan& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return p.kfirst ? launch_scan_kf<SDT, true>(p, s, e0, e1) : launch_scan_kf<SDT, false>(p, s, e0, e1);
}

}  // namespace

int launch_scan(const Plan& p, void* stream, void* start, void* stop) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t e0 = reinterpret_cast<hipEvent_t>(start), e1 = reinterpret_cast<hipEvent_t>(stop);
  switch (p.state_dtype) {
    case kF16: return launch_scan_dt<kF16>(p, s, e0, e1);
    case kBF16: return launch_scan_dt<kBF16>(p, s, e0, e1);
    default: return launch_scan_dt<kF32>(p, s, e0, e1);
  }
}

int launch_segmap(const Plan& p, void* stream, void* start, void* stop) {
  if (p.n_maps == 0) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t e0 = reinterpret_cast<hipEvent_t>(start), e1 = reinterpret_cast<hipEvent_t>(stop);
  constexpr size_t bytes = HeadLds<2>::kBytes;
  static bool done = false;
  if (int e = set_lds_limit(&head_kernel<2, kF32, kKernelMap, false>, bytes, done)) return e;
  const int units = p.n_maps * p.H;
  const int nblocks = 8 * ((units + 7) / 8) * 2;  // halves A and C
  hipExtLaunchKernelGGL((head_kernel<2, kF32, kKernelMap, false>), dim3(nblocks), dim3(320), bytes, s, e0, e1, 0, p, units, 2);
  return (int)hipGetLastError();
}

}  // namespace kda
