// Segment kernels of the segmented scan on gfx950.
//
// Long sequences are split into segments of seg_len chunks and the serial walk runs in
// two levels, as the pages' segmented prefill does (a pass that composes each segment,
// then a scan over segments; aiter PR 5754, Technical Details and Test Result; the
// segment kernels up-cast a 2-byte initial state as the seg-scan does, aiter PR 5249,
// What). Every chunk acts on the V x K state as an affine map
//
//   S -> S M + B,   M = Diag(E) - W^T K,   B = U^T K        (K x K and V x K)
//
// so a segment of chunks composes to S_end = S_start A + C with A the product of its
// M's and C the state it reaches from zero.
//
//   segmap:     for every segment but a sequence's last, A and C by running the state
//               recurrence on an augmented state: 128 rows that start as the identity
//               with U = 0 give A, 128 rows that start at zero with the chunk's U give
//               C. One workgroup per (segment, head, half); 4 state waves of 32 rows
//               and a loader wave that stages W, K, E (and U) through an LDS ring.
//   segcombine: per (sequence, head, 32 value rows), S_{g+1} = S_g A_g + C_g over the
//               sequence's segments, from the call's initial state, in fp32 (bf16 hi/lo
//               operand splits on MFMA); the results are the segments' start states.
//
// The scan kernel then runs every segment from its start state in parallel.

#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// ====================================================================== segment maps
// LDS ring slot: W 8, K 8 and U 8 fragments of 1 KB, then E (128 fp32).
struct MapLds {
  static constexpr int kRing = 4;
  static constexpr int kSlotW = 0;
  static constexpr int kSlotK = 8 * 1024;
  static constexpr int kSlotU = 16 * 1024;
  static constexpr int kSlotE = 24 * 1024;
  static constexpr int kSlot = kSlotE + 512;
  static constexpr size_t kBytes = (size_t)kRing * kSlot;
};

// Loader wave: chunk c of the segment into slot c mod kRing, kRing - 1 chunks ahead;
// before barrier c (and the first barrier, for chunk 0) chunk c + 1 has landed. The
// slot it refills during step c held chunk c - 1, read by the state waves before
// barrier c - 1. Barriers carry no fence (a fence would wait for every direct-to-LDS
// load in flight).
template <bool WITH_U>
__device__ __forceinline__ void map_loader(char* lds, __amdgpu_buffer_rsrc_t rs, int nc, int lane) {
  typedef MapLds L;
  constexpr int kLoads = 8 + 8 + 2 + (WITH_U ? 8 : 0);
  const int vo = lane * 16;
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
    if constexpr (WITH_U) {
#pragma unroll
      for (int f = 0; f < 8; ++f)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotU + f * 1024), 16, vo,
                                                 soff + (int)kRecU + f * (int)kFrag, 0, 0);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + L::kSlotE + half * 256), 4, lane * 4,
                                               soff + (int)kRecE + half * 256, 0, 0);
  };
  const int pre = min(L::kRing - 1, nc);
  for (int c = 0; c < pre; ++c) issue(c, c);
  wait_chunks<kLoads, L::kRing - 2>(pre - 1);
  __builtin_amdgcn_s_barrier();
  int fill = L::kRing - 1;
  for (int c = 0; c < nc; ++c) {
    if (c + L::kRing - 1 < nc) issue(c + L::kRing - 1, fill);
    fill = (fill + 1 == L::kRing) ? 0 : fill + 1;
    wait_chunks<kLoads, L::kRing - 2>(min(L::kRing - 2, nc - 2 - c));
    __builtin_amdgcn_s_barrier();
  }
}

__global__ __launch_bounds__(320, 1) void segmap_kernel(Plan p, int units) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  typedef MapLds L;
  // (map slot, head) units dealt round-robin to the XCDs; both halves of a unit share one.
  const int bidx = blockIdx.x;
  const int xcd = bidx & 7;
  const int slot8 = bidx >> 3;
  const int part = slot8 & 1;  // 0: A (identity start, U = 0), 1: C (zero start, U)
  const int id = (slot8 >> 1) * 8 + xcd;
  if (id >= units) return;
  const int m = id / p.H;
  const int h = id - m * p.H;
  const int32_t* e = p.d_seg + (size_t)kSegInts * p.d_m2s[m];
  const int n = e[0], c0 = e[1], nc = e[2];
  const char* rec0 = reinterpret_cast<const char*>(p.ws) + ((size_t)h * p.n_chunks + p.d_co[n] + c0) * kRecBytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rec0), (short)0, nc * (int)kRecBytes, kBufWord3);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  const int vo = lane * 16;

  if (wave == 4) {
    if (part) map_loader<true>(lds, rs, nc, lane);
    else map_loader<false>(lds, rs, nc, lane);
    return;
  }

  // State wave: rows v of value tiles 2*wave + nt (nt = 0, 1); lane holds S^T[k][v] for
  // k = 16*tt + 4*g4 + i, v = 16*(2*wave + nt) + l16.
  f32x4 S[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[nt][tt][i] = (part == 0 && 16 * tt + 4 * g4 + i == 16 * (2 * wave + nt) + l16) ? 1.f : 0.f;

  struct Frags {
    bf16x8 w[2][4];  // -W (row tile t, key block m)
    bf16x8 u[2];     // U of value tiles 2*wave + nt
    bf16x8 k[8];     // K (key tile)
    f32x4 e[8];      // exp(G_C) of this lane's keys
  };
  auto read = [&](Frags& f, int slot) {
    const char* sl = lds + slot * L::kSlot;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        f.w[t][mb] = *reinterpret_cast<const bf16x8*>(sl + L::kSlotW + (t * 4 + mb) * 1024 + vo);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f.u[nt] = part ? *reinterpret_cast<const bf16x8*>(sl + L::kSlotU + (2 * wave + nt) * 1024 + vo) : bf16x8{};
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

  barrier_lds();  // the loader has chunk 0 in slot 0
  Frags f;
  read(f, 0);
  int slot = 0;
  for (int c = 0; c < nc; ++c) {
    bf16x8 Sb[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) Sb[nt][mb] = pack8(S[nt][2 * mb], S[nt][2 * mb + 1]);
    // Delta = U + (-W) S^T.
    f32x4 x[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 a;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = from_bf16(f.u[nt][4 * t + i]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) a = mfma(f.w[t][mb], Sb[nt][mb], a);
        x[nt][t] = a;
      }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) S[nt][tt] = S[nt][tt] * f.e[tt];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const bf16x8 Db = pack8(x[nt][0], x[nt][1]);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) S[nt][tt] = mfma(f.k[tt], Db, S[nt][tt]);
    }
    barrier_lds();  // the loader has chunk c + 1 in the next slot
    slot = (slot + 1 == L::kRing) ? 0 : slot + 1;
    if (c + 1 < nc) read(f, slot);
  }

  // A or C in S^T layout: element (k, v) at [k][v].
  float* dst = p.maps + ((size_t)(m * p.H + h) * 2 + part) * kHead * kHead;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(size_t)(16 * tt + 4 * g4 + i) * kHead + 16 * (2 * wave + nt) + l16] = S[nt][tt][i];
}

// ====================================================================== combine
// LDS: the current state rows of this workgroup's 32 value rows, fp32 [32][kLdS].
constexpr int kLdS = kHead + 4;

template <int SDT>
__global__ __launch_bounds__(256) void segcombine_kernel(Plan p) {
  __shared__ __attribute__((aligned(16))) float Sv[32 * kLdS];
  const int slice = blockIdx.x & 3;  // value rows 32*slice .. 32*slice + 31
  const int rest = blockIdx.x >> 2;
  const int h = rest % p.H;
  const int k = rest / p.H;
  const int32_t* cb = p.d_comb + 4 * k;
  const int n = cb[0], m0 = cb[1], cnt = cb[2];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;

  // Initial state rows (the call's initial state, or zero).
  const void* in_plane = state_in_plane<SDT>(p, n, h);
  for (int q = threadIdx.x; q < 32 * 32; q += 256) {
    const int r = q >> 5, c4 = (q & 31) * 4;
    const f32x4 x = in_plane ? load_state4<SDT>(in_plane, (size_t)(32 * slice + r) * kHead + c4) : zero4();
    *reinterpret_cast<f32x4*>(&Sv[r * kLdS + c4]) = x;
  }
  __syncthreads();

  // Wave w forms columns k = 32*w + 16*kt + l16 (kt = 0, 1) of the 32 rows; output
  // tile (vt, kt): lane holds rows v = 32*slice + 16*vt + 4*g4 + i. Every map is ready
  // when the kernel starts, so step j + 1's map loads are issued before step j's MFMAs.
  struct MapFrags {
    f32x4 b[2][4][2];  // A[k'][k]: column tile kt, key block kb, k' = 32*kb + 8*g4 + (0..3, 4..7)
    f32x4 c[2][2];     // C[v][k]: value tile vt, column tile kt
  };
  auto load_map = [&](MapFrags& f, int m) {
    const float* A = p.maps + ((size_t)(m * p.H + h) * 2 + 0) * kHead * kHead;  // [k][k'] = A[k'][k]
    const float* C = p.maps + ((size_t)(m * p.H + h) * 2 + 1) * kHead * kHead;  // [k][v]  = C[v][k]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const float* row = A + (size_t)(32 * wave + 16 * kt + l16) * kHead + 8 * g4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f.b[kt][kb][0] = *reinterpret_cast<const f32x4*>(row + 32 * kb);
        f.b[kt][kb][1] = *reinterpret_cast<const f32x4*>(row + 32 * kb + 4);
      }
    }
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        f.c[vt][kt] =
            *reinterpret_cast<const f32x4*>(C + (size_t)(32 * wave + 16 * kt + l16) * kHead + 32 * slice + 16 * vt + 4 * g4);
  };
  auto step = [&](const MapFrags& f, int m) {
    f32x4 acc[2][2];
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc[vt][kt] = f.c[vt][kt];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 bh[2], bl[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) split8(f.b[kt][kb][0], f.b[kt][kb][1], bh[kt], bl[kt]);
      // A operand: S[v][k'], v = 16*vt + l16 (local row), k' = 32*kb + 8*g4 + jj.
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        const float* src = &Sv[(16 * vt + l16) * kLdS + 32 * kb + 8 * g4];
        bf16x8 ah, al;
        split8(*reinterpret_cast<const f32x4*>(src), *reinterpret_cast<const f32x4*>(src + 4), ah, al);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          acc[vt][kt] = mfma(ah, bh[kt], acc[vt][kt]);
          acc[vt][kt] = mfma(ah, bl[kt], acc[vt][kt]);
          acc[vt][kt] = mfma(al, bh[kt], acc[vt][kt]);
        }
      }
    }
    // Start state of the segment after map slot m, [v][k].
    float* dst = p.starts + ((size_t)m * p.H + h) * kHead * kHead;
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(size_t)(32 * slice + 16 * vt + 4 * g4 + i) * kHead + 32 * wave + 16 * kt + l16] = acc[vt][kt][i];
    __syncthreads();  // every wave has read the previous rows
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) Sv[(16 * vt + 4 * g4 + i) * kLdS + 32 * wave + 16 * kt + l16] = acc[vt][kt][i];
    __syncthreads();
  };
  MapFrags fa, fb;
  load_map(fa, m0);
  for (int j = 0; j < cnt; j += 2) {
    load_map(fb, m0 + min(j + 1, cnt - 1));
    step(fa, m0 + j);
    if (j + 1 >= cnt) break;
    load_map(fa, m0 + min(j + 2, cnt - 1));
    step(fb, m0 + j + 1);
  }
}

}  // namespace

int launch_segmap(const Plan& p, void* stream) {
  if (p.n_maps == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&segmap_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)MapLds::kBytes);
    if (e != hipSuccess) return (int)e;
    attr_set = true;
  }
  const int units = p.n_maps * p.H;
  const int nblocks = 8 * ((units + 7) / 8) * 2;
  hipLaunchKernelGGL(segmap_kernel, dim3(nblocks), dim3(320), MapLds::kBytes, s, p, units);
  return (int)hipGetLastError();
}

int launch_segcombine(const Plan& p, void* stream) {
  if (p.n_multi == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(p.n_multi * p.H * 4);
  switch (p.state_dtype) {
    case kF16: hipLaunchKernelGGL(segcombine_kernel<kF16>, grid, dim3(256), 0, s, p); break;
    case kBF16: hipLaunchKernelGGL(segcombine_kernel<kBF16>, grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL(segcombine_kernel<kF32>, grid, dim3(256), 0, s, p); break;
  }
  return (int)hipGetLastError();
}

}  // namespace kda
