// Segment combine kernel of the segmented scan on gfx950.
//
// Long sequences are split into segments of seg_len chunks and the serial walk runs in
// two levels, as the pages' segmented prefill does (a pass that composes each segment,
// then a scan over segments; aiter PR 5754, Technical Details and Test Result; the
// segment kernels up-cast a 2-byte initial state as the seg-scan does, aiter PR 5249,
// What). Every chunk acts on the V x K state as an affine map
//
//   S -> S M + B,   M = Diag(E) - W^T K,   B = U^T K        (K x K and V x K)
//
// so a segment of chunks composes to S_end = S_start A + C, with A the product of its
// M's and C the state it reaches from zero. The segment-map pass in the scan kernel's
// file forms A and C for every segment but a sequence's last. This kernel walks, per
// (sequence, head, 32 value rows), S_{g+1} = S_g A_g + C_g over the sequence's segments
// from the call's initial state, in fp32 (bf16 hi/lo operand splits on MFMA: hi*hi +
// hi*lo + lo*hi), and stores the results: the start states the scan runs the segments
// from, the first segment's included (a copy of the initial state).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// ====================================================================== combine
// One workgroup per (sequence, head, 32 value rows): four compute waves and a loader wave.
//
// A step S_{g+1} = S_g A_g + C_g is computed transposed, S_{g+1}^T = A_g^T S_g^T + C_g^T:
// the map is the left MFMA operand (rows k, reduction over k'), the state the right one
// (reduction k', columns v), so each lane's accumulator holds four consecutive keys of one
// value row. Those go to the start-state store, the next step's operand rows in LDS and
// the C initialisation as 16-byte (8-byte) vectors. Compute wave w forms keys
// 32w .. 32w + 31 of the 32 rows.
//
// The loader wave streams each step's A^T (hi and lo planes, 64 KB) into a two-slot LDS
// ring with direct-to-LDS loads, one MFMA operand fragment (64 lanes x 16 bytes) per
// load, so the compute waves issue no map loads: step j + 2 goes into the slot step j
// used, once every wave is past step j's reads, while the compute waves run step j + 1.
constexpr int kLdS = kHead + 8;        // bf16 per row of the state operand rows [32][kLdS]
constexpr int kSlotA = 64 * 1024;      // one step: A^T hi, then lo, 32 fragments of 1 KB each
constexpr int kOffS = 2 * kSlotA;      // state rows: hi [32][kLdS], then lo
constexpr size_t kCombineLds = (size_t)kOffS + 2 * 32 * kLdS * 2;
static_assert(kCombineLds <= 160 * 1024, "fits one CU's LDS");

// Fragment f = (kt, kb) of a plane (kt = key tile 0..7, kb = key' block 0..3): lane
// (l16, g4) holds A^T[16 kt + l16][32 kb + 8 g4 .. + 7]; the maps store each plane in
// this order (map_frag_index), 1 KB per fragment.
__device__ __forceinline__ int frag_of(int kt, int kb) { return kt * 4 + kb; }

template <int SDT>
__global__ __launch_bounds__(320) void segcombine_kernel(Plan p, int units) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  // Workgroup b runs on XCD b mod 8; all four of a unit's workgroups have b = u mod 8, so
  // they share one L2 for the unit's maps.
  const int u = (blockIdx.x >> 5) * 8 + (blockIdx.x & 7);
  if (u >= units) return;
  const int slice = (blockIdx.x >> 3) & 3;  // value rows 32*slice .. 32*slice + 31
  const int h = __builtin_amdgcn_readfirstlane(u % p.H);
  const int k = __builtin_amdgcn_readfirstlane(u / p.H);
  const int32_t* cb = p.d_comb + 4 * k;
  const int n = __builtin_amdgcn_readfirstlane(cb[0]);
  const int m0 = __builtin_amdgcn_readfirstlane(cb[1]);
  const int cnt = __builtin_amdgcn_readfirstlane(cb[2]);
  const int first_slot = __builtin_amdgcn_readfirstlane(cb[3]);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  __bf16* Shi = reinterpret_cast<__bf16*>(lds + kOffS);
  __bf16* Slo = Shi + 32 * kLdS;

  if (wave == 4) {
    // ---------------------------------------------------------------- loader wave
    // Per step 64 fragment loads: at most 63 may be in flight, so each wait is for all of
    // them (vmcnt 0), taken before the next step's loads are issued.
    const int voff = lane * 16;  // lane's bytes in a fragment
    auto issue = [&](int j, int slot) {
      const char* base = reinterpret_cast<const char*>(p.maps) + (size_t)((m0 + j) * p.H + h) * kMapBytes;
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)(kHead * kHead * 4), kBufWord3);
      char* dst = lds + slot * kSlotA;
#pragma unroll
      for (int plane = 0; plane < 2; ++plane)
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_ptr_t)(dst + (plane * 32 + frag_of(kt, kb)) * 1024), 16, voff,
                (plane * 32 + frag_of(kt, kb)) * 1024, 0, 0);
    };
    issue(0, 0);
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // Y(-1): step 0's operands and the initial rows are ready
    if (cnt > 1) issue(1, 1);
    for (int j = 0; j < cnt; ++j) {
      __builtin_amdgcn_s_barrier();  // X(j): every wave is past step j's reads of slot j & 1
      wait_vmcnt<0>();               // step j + 1 has landed
      __builtin_amdgcn_s_barrier();  // Y(j)
      // Issued while the compute waves run step j + 1 (from the other slot), so that the
      // issue does not hold up barrier Y(j).
      if (j + 2 < cnt) issue(j + 2, j & 1);
    }
    return;
  }

  // ------------------------------------------------------------------ compute waves
  // Initial state rows (the call's initial state, or zero). They are also stored, in fp32
  // (exact for every storage dtype), as the start state of the sequence's first segment:
  // the scan must not read the caller's plane for a sequence whose last segment writes
  // the final state into it from another workgroup of the same launch.
  const void* in_plane = state_in_plane<SDT>(p, n, h);
  float* first = p.starts + ((size_t)first_slot * p.H + h) * kHead * kHead;
  for (int q = threadIdx.x; q < 32 * 32; q += 256) {
    const int r = q >> 5, c4 = (q & 31) * 4;
    const f32x4 x = in_plane ? load_state4_vk<SDT>(in_plane, 32 * slice + r, c4, p.kfirst) : zero4();
    *reinterpret_cast<f32x4*>(first + (size_t)(32 * slice + r) * kHead + c4) = x;
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16(x[i], Shi[r * kLdS + c4 + i], Slo[r * kLdS + c4 + i]);
  }
  // C^T tiles of this lane: value tile vt, key tile kt = 2w + t; lane holds keys
  // 16 kt + 4 g4 .. + 3 of value row 32 slice + 16 vt + l16 (C is stored [v][k]).
  auto load_c = [&](f32x4 (&c)[2][2], int j) {
    const float* C = reinterpret_cast<const float*>(reinterpret_cast<const char*>(p.maps) +
                                                    (size_t)((m0 + j) * p.H + h) * kMapBytes + kHead * kHead * 4);
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        c[vt][t] = *reinterpret_cast<const f32x4*>(C + (size_t)(32 * slice + 16 * vt + l16) * kHead +
                                                   16 * (2 * wave + t) + 4 * g4);
  };
  f32x4 c0[2][2], c1[2][2];
  load_c(c0, 0);
  barrier_lds();  // Y(-1)
  auto step = [&](const f32x4 (&c)[2][2], int j) {
    const char* sl = lds + (j & 1) * kSlotA;
    f32x4 acc[2][2];
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[vt][t] = c[vt][t];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 sh[2], sl8[2];
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        const int at = (16 * vt + l16) * kLdS + 32 * kb + 8 * g4;
        sh[vt] = *reinterpret_cast<const bf16x8*>(&Shi[at]);
        sl8[vt] = *reinterpret_cast<const bf16x8*>(&Slo[at]);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int f = frag_of(2 * wave + t, kb);
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(sl + f * 1024 + lane * 16);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(sl + (32 + f) * 1024 + lane * 16);
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
          acc[vt][t] = mfma(ah, sh[vt], acc[vt][t]);
          acc[vt][t] = mfma(ah, sl8[vt], acc[vt][t]);
          acc[vt][t] = mfma(al, sh[vt], acc[vt][t]);
        }
      }
    }
    // Start state of the segment after map slot m0 + j, [v][k].
    float* dst = p.starts + ((size_t)(m0 + j) * p.H + h) * kHead * kHead;
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        *reinterpret_cast<f32x4*>(dst + (size_t)(32 * slice + 16 * vt + l16) * kHead + 16 * (2 * wave + t) + 4 * g4) =
            acc[vt][t];
    barrier_lds();  // X(j): every wave has read the rows and slot j & 1
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int at = (16 * vt + l16) * kLdS + 16 * (2 * wave + t) + 4 * g4;
        bf16x4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = to_bf16(acc[vt][t][i]);
          lo[i] = to_bf16(acc[vt][t][i] - from_bf16(hi[i]));
        }
        *reinterpret_cast<bf16x4*>(&Shi[at]) = hi;
        *reinterpret_cast<bf16x4*>(&Slo[at]) = lo;
      }
    barrier_lds();  // Y(j): the new rows are written; step j + 1's operands have landed
  };
  // Pairs of steps with the next step's C loaded ahead, without an early exit inside a
  // pair (a path from a partial pair back to the loop head would make the compiler wait
  // there for every load in flight); an odd last step follows with its C in c0.
  for (int j = 0; j + 1 < cnt; j += 2) {
    load_c(c1, j + 1);
    step(c0, j);
    load_c(c0, min(j + 2, cnt - 1));
    step(c1, j + 1);
  }
  if (cnt & 1) step(c0, cnt - 1);
}

}  // namespace

int launch_segcombine(const Plan& p, void* stream, void* start, void* stop) {
  if (p.n_multi == 0) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t e0 = reinterpret_cast<hipEvent_t>(start), e1 = reinterpret_cast<hipEvent_t>(stop);
  const int units = p.n_multi * p.H;
  const dim3 grid(32 * ((units + 7) / 8));
  static bool done[3] = {false, false, false};
  auto run = [&](auto kernel, int dt) -> int {
    if (!done[dt]) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kCombineLds);
      if (e != hipSuccess) return (int)e;
      done[dt] = true;
    }
    hipExtLaunchKernelGGL(kernel, grid, dim3(320), kCombineLds, s, e0, e1, 0, p, units);
    return (int)hipGetLastError();
  };
  switch (p.state_dtype) {
    case kF16: return run(segcombine_kernel<kF16>, kF16);
    case kBF16: return run(segcombine_kernel<kBF16>, kBF16);
    default: return run(segcombine_kernel<kF32>, kF32);
  }
}

}  // namespace kda
