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
// from the call's initial state, in fp32 (bf16 hi/lo operand splits on MFMA), and stores
// the results: the start states the scan runs the segments from, the first segment's
// included (a copy of the initial state).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// ====================================================================== combine
// LDS: the current state rows of this workgroup's 32 value rows as bf16 hi and lo
// planes [32][kLdS] (the MFMA A operand, already split).
constexpr int kLdS = kHead + 8;

template <int SDT>
__global__ __launch_bounds__(256) void segcombine_kernel(Plan p) {
  __shared__ __attribute__((aligned(16))) __bf16 Shi[32 * kLdS];
  __shared__ __attribute__((aligned(16))) __bf16 Slo[32 * kLdS];
  const int slice = blockIdx.x & 3;  // value rows 32*slice .. 32*slice + 31
  const int rest = blockIdx.x >> 2;
  const int h = rest % p.H;
  const int k = rest / p.H;
  const int32_t* cb = p.d_comb + 4 * k;
  const int n = cb[0], m0 = cb[1], cnt = cb[2];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;

  // Initial state rows (the call's initial state, or zero). They are also stored, in fp32
  // (exact for every storage dtype), as the start state of the sequence's first segment:
  // the scan must not read the caller's plane for a sequence whose last segment writes
  // the final state into it from another workgroup of the same launch.
  const void* in_plane = state_in_plane<SDT>(p, n, h);
  float* first = p.starts + ((size_t)cb[3] * p.H + h) * kHead * kHead;
  for (int q = threadIdx.x; q < 32 * 32; q += 256) {
    const int r = q >> 5, c4 = (q & 31) * 4;
    const f32x4 x = in_plane ? load_state4_vk<SDT>(in_plane, 32 * slice + r, c4, p.kfirst) : zero4();
    *reinterpret_cast<f32x4*>(first + (size_t)(32 * slice + r) * kHead + c4) = x;
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16(x[i], Shi[r * kLdS + c4 + i], Slo[r * kLdS + c4 + i]);
  }
  __syncthreads();

  // Wave w forms columns k = 32*w + 16*kt + l16 (kt = 0, 1) of the 32 rows; output tile
  // (vt, kt): lane holds rows v = 32*slice + 16*vt + 4*g4 + i. Every map is ready when
  // the kernel starts, so step j + 1's map loads are issued before step j's MFMAs.
  struct MapFrags {
    bf16x8 bh[2][4], bl[2][4];  // A[k'][k] hi, lo: column tile kt, key block kb
    f32x4 c[2][2];              // C[v][k]: value tile vt, column tile kt
  };
  auto load_map = [&](MapFrags& f, int m) {
    const char* base = reinterpret_cast<const char*>(p.maps) + (size_t)(m * p.H + h) * kMapBytes;
    const __bf16* Ahi = reinterpret_cast<const __bf16*>(base);  // [k][k'] = A[k'][k]
    const __bf16* Alo = Ahi + kHead * kHead;
    const float* C = reinterpret_cast<const float*>(base + kHead * kHead * 4);  // [k][v] = C[v][k]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const size_t row = (size_t)(32 * wave + 16 * kt + l16) * kHead + 8 * g4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f.bh[kt][kb] = *reinterpret_cast<const bf16x8*>(Ahi + row + 32 * kb);
        f.bl[kt][kb] = *reinterpret_cast<const bf16x8*>(Alo + row + 32 * kb);
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
      // A operand: S[v][k'], v = 16*vt + l16 (local row), k' = 32*kb + 8*g4 + jj.
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        const int at = (16 * vt + l16) * kLdS + 32 * kb + 8 * g4;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Shi[at]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Slo[at]);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          acc[vt][kt] = mfma(ah, f.bh[kt][kb], acc[vt][kt]);
          acc[vt][kt] = mfma(ah, f.bl[kt][kb], acc[vt][kt]);
          acc[vt][kt] = mfma(al, f.bh[kt][kb], acc[vt][kt]);
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
        for (int i = 0; i < 4; ++i) {
          const int at = (16 * vt + 4 * g4 + i) * kLdS + 32 * wave + 16 * kt + l16;
          split_bf16(acc[vt][kt][i], Shi[at], Slo[at]);
        }
    __syncthreads();
  };
  // Pairs of steps run without an early exit (a path from a partial pair back to the loop
  // head would make the compiler wait there for every load in flight); an odd last step
  // follows with its maps already in fa.
  // The next step's loads are pinned ahead of this step's MFMAs (the scheduler would
  // otherwise sink them to the end of the step and expose their latency every step).
  MapFrags fa, fb;
  load_map(fa, m0);
  for (int j = 0; j + 1 < cnt; j += 2) {
    load_map(fb, m0 + j + 1);
    __builtin_amdgcn_sched_barrier(0);
    step(fa, m0 + j);
    load_map(fa, m0 + min(j + 2, cnt - 1));
    __builtin_amdgcn_sched_barrier(0);
    step(fb, m0 + j + 1);
  }
  if (cnt & 1) step(fa, m0 + cnt - 1);
}

}  // namespace

int launch_segcombine(const Plan& p, void* stream, void* start, void* stop) {
  if (p.n_multi == 0) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t e0 = reinterpret_cast<hipEvent_t>(start), e1 = reinterpret_cast<hipEvent_t>(stop);
  const dim3 grid(p.n_multi * p.H * 4);
  switch (p.state_dtype) {
    case kF16: hipExtLaunchKernelGGL(segcombine_kernel<kF16>, grid, dim3(256), 0, s, e0, e1, 0, p); break;
    case kBF16: hipExtLaunchKernelGGL(segcombine_kernel<kBF16>, grid, dim3(256), 0, s, e0, e1, 0, p); break;
    default: hipExtLaunchKernelGGL(segcombine_kernel<kF32>, grid, dim3(256), 0, s, e0, e1, 0, p); break;
  }
  return (int)hipGetLastError();
}

}  // namespace kda
