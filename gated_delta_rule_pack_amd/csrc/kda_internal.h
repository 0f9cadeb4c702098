// Internal declarations shared by the host orchestration and the kernel launchers.
// Not part of the public ABI (include/kda.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 32;    // tokens per chunk
constexpr int kHead = 128;    // K = V = 128
constexpr int kThreadsPrep = 512;

// Per (head, chunk) workspace record written by prep and read by scan. Every tile is
// stored in the exact per-lane order the scan's MFMA operands use, so the scan issues
// one contiguous 16-byte load per lane per fragment.
//   W  : 8 fragments (row tile t in 0..1, key block m in 0..3), bf16, stored negated (-W)
//   Q  : 8 fragments, same order, bf16 (scale folded in)
//   K  : 8 fragments (key tile 0..7), bf16
//   U  : 8 fragments (value slice 0..7 of 16 channels), bf16
//   P  : 2 fragments (row tile 0..1), bf16 (scale folded in)
//   E  : 128 fp32, exp(G_C) per key channel
constexpr size_t kFrag = 64 * 16;  // one fragment: 64 lanes x 16 bytes
constexpr size_t kRecW = 0;
constexpr size_t kRecQ = kRecW + 8 * kFrag;
constexpr size_t kRecK = kRecQ + 8 * kFrag;
constexpr size_t kRecU = kRecK + 8 * kFrag;
constexpr size_t kRecP = kRecU + 8 * kFrag;
constexpr size_t kRecE = kRecP + 2 * kFrag;
constexpr size_t kRecBytes = kRecE + kHead * 4;  // 35328 = 138 * 256
static_assert(kRecBytes % 256 == 0, "records stay 256-byte aligned");

// Segmented scan. A sequence of nc chunks is split into segments of seg_len chunks (the
// last one shorter). Each chunk acts on the state as the affine map S -> S M + B
// (M = Diag(e^{G_C}) - W^T K, B = U^T K); each segment but a sequence's last gets its
// composed map (A, C) from the segment-map kernel, the combine kernel walks the maps to
// every segment's start state, and the scan then runs all segments in parallel.
constexpr int kSegMin = 8;        // shortest segment (chunks)
constexpr int kSegInts = 8;       // segment table record: sequence, first chunk, chunks,
                                  // start-state slot (-1: the caller's initial state, read
                                  // only by a sequence's single segment),
                                  // own map slot (-1: last segment, writes the final state)
constexpr size_t kMapBytes = (size_t)2 * kHead * kHead * 4;  // A (bf16 hi, lo; [k][k']), C (fp32; [v][k])
constexpr size_t kStartBytes = (size_t)kHead * kHead * 4;    // start state, fp32, [v][k]

enum StateMode : int { kStateNone = 0, kStateDense = 1, kStatePaged = 2 };
enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Everything one launch needs; filled by the host orchestration.
struct Plan {
  int T, N, H, n_chunks;
  int H_qk, group;  // q/k heads and value heads per q/k head (H = H_qk * group)
  int kfirst;       // state planes are [K][V] (1) or [V][K] (0)
  float scale, lower_bound;
  int ref_block;  // reference-row block of the bounded decay construction
  int dv_split;   // value-channel split of the scan (8, 4 or 2)
  const void* q;
  const void* k;
  const void* v;
  const void* g_raw;
  const void* beta_raw;
  int g_dtype, beta_dtype;
  const int32_t* d_cu;     // [N+1] token bounds (device)
  const int32_t* d_co;     // [N+1] chunk offsets (device)
  const int32_t* d_table;  // [n_chunks][2] (sequence, chunk within sequence) (device)
  int n_seg, n_maps, n_multi, seg_len;
  const int32_t* d_seg;    // [n_seg][kSegInts] segment table (device)
  const int32_t* d_m2s;    // [n_maps] segment of each map slot (device)
  const int32_t* d_comb;   // [n_multi][4] (sequence, first map slot, maps, start slot of
                           // the first segment) (device)
  int state_dtype;
  const void* state_in;
  int in_mode;
  void* state_out;
  int out_mode;
  int64_t stride0;  // elements between sequence/slot planes
  const int32_t* indices;
  const uint8_t* flags;
  void* out;
  void* ws;             // first chunk record (256-byte aligned)
  float* maps;          // [n_maps][H] segment maps: A as bf16 hi and lo planes [k][k'] (A^T),
                        // then C fp32 [v][k]
  float* starts;        // [n_maps + n_multi][H][V][K] fp32 start states: slot m < n_maps
                        // starts the segment after map slot m, slot n_maps + k the first
                        // segment of multi-segment sequence k (its initial state)
  int cu_count;         // compute units of the device (persistent grid sizing)
  int stream_inputs;    // prep reads its inputs with the non-temporal hint (the call's chunk
                        // records fit the memory-side cache)
};

// Fixed device workspace of the allocation-free call (kda_noalloc.hip): 64 MiB per device,
// enough for the records of one 4096-token call with 12 heads (54.3 MB) and for any call
// that takes the decode kernel (which needs none).
constexpr size_t kScratchBytes = size_t(64) << 20;
// Memory-side cache of an MI355X (256 MB): a call whose chunk records fit it streams
// prep's inputs past it, so that the records stay there for the passes that read them.
constexpr size_t kMallBytes = size_t(256) << 20;
// Device address of that device's copy of the workspace, resolved once per device with the
// device current (0 on success, else a HIP error code).
int scratch_address(int device, void** ptr);

// Launchers (defined in the .hip files). Return 0 on success, nonzero HIP error code.
// start / stop, when not null, are HIP events the launch itself records when the kernel
// starts and when it completes (no separate marker in the stream). Each launcher is
// called only when its kernel has work: prep when n_chunks > 0, the segment kernels when
// n_maps > 0; the scan always has at least one (segment, head) unit.
int launch_prep(const Plan& p, void* stream, void* start, void* stop);
int launch_scan(const Plan& p, void* stream, void* start, void* stop);
int launch_segmap(const Plan& p, void* stream, void* start, void* stop);
int launch_segcombine(const Plan& p, void* stream, void* start, void* stop);
int launch_decode(const Plan& p, void* stream, void* start, void* stop);
// Copies bytes (a multiple of 16, both pointers 16-byte aligned) from device-readable
// pinned host memory to device memory with a kernel on the stream.
// done, when not null, is an event the launch records when the copy has completed.
int launch_meta_copy(const void* host_src, void* dst, size_t bytes, void* stream, void* done);

}  // namespace kda
