/*
 * kda.h: C ABI of the MI355X (gfx950) chunkwise Kimi Delta Attention prefill library.
 *
 * Operation (aiter PR 4741, "[FlyDSL] Add gfx950 Kimi Delta Attention prefill kernel",
 * Summary and Optimizations Applied): for every token t of sequence n and head h, with
 * a V-first state S in R^{V x K} (K = V = 128),
 *
 *     q^ = q / sqrt(|q|^2 + 1e-6),  k^ = k / sqrt(|k|^2 + 1e-6)
 *     g  = lower_bound * sigmoid(g_raw)        (one value per key channel)
 *     b  = sigmoid(beta_raw)                   (one value per token-head)
 *     S  = S Diag(exp g) (I - b k^ k^T) + b v k^T
 *     o  = scale * S q^
 *
 * computed chunkwise (32-token chunks) by three stages on the caller's stream: host
 * metadata, a chunk-parallel prep kernel (L2-norm, gate, beta, in-chunk gate cumsum,
 * bounded intra-chunk tiles, the unit-lower-triangular solve and the w/u products) and
 * a serial scan kernel over each sequence's chunks that carries the fp32 state.
 *
 * State I/O follows aiter PR 5754 (FlashKDA paged state_cache, Technical Details): a
 * dense initial/final state, or a paged pool [slots, H, V, K] whose slot planes are
 * dense and whose stride(0) may be padded, addressed by int32 state_indices with a
 * per-sequence has_initial_state flag. Stored state may be fp32, fp16 or bf16 and is
 * accumulated in fp32 (aiter PR 5249, What). Host bounds (cu_seqlens_host) let the
 * call build and upload its metadata without any synchronising call (aiter PR 6912,
 * Changes).
 *
 * Conventions for every function below:
 *  - Pointers are device memory owned by the caller unless marked "host".
 *  - The library never allocates or frees caller memory. It owns only its context: a
 *    pinned staging arena and a device arena for the metadata cache, both made when the
 *    context is created and freed only when it is destroyed.
 *  - Tensors are contiguous row-major with the shapes stated; "[T, H, D]" means
 *    element (t, h, d) sits at offset (t * H + h) * D + d.
 *  - A failed call returns before enqueuing any work: nothing is written.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1,  /* null required pointer, N < 1, T < 0, bad bounds, non-finite scale */
  KDA_ERR_UNSUPPORTED = 2,  /* K or V != 128, dtype not allowed, lower_bound > 0, not gfx950,
                               T * H > 2^31 / 128, or a scan walk over more than 2^31 bytes of
                               chunk records (over 60 786 chunks in one segment: only with
                               H = 1 and a sequence of more than about 15.5 M tokens) */
  KDA_ERR_STATE_MODE = 3,   /* dense and paged state both given, or final_state with a pool */
  KDA_ERR_STRIDE = 4,       /* state_cache_stride0 < H*V*K */
  KDA_ERR_ALIAS = 5,        /* the byte ranges of out and v overlap */
  KDA_ERR_WORKSPACE = 6,    /* workspace null or smaller than kda_chunk_fwd_workspace_bytes() */
  KDA_ERR_CAPTURE_MISS = 7, /* metadata-cache miss while the stream is being captured */
  KDA_ERR_HIP = 8,          /* a HIP runtime call or a kernel launch failed */
  KDA_ERR_NO_SPACE = 9      /* a call that may not allocate: its workspace or metadata does not
                               fit the fixed memory it must use */
} kda_status;

/* Element types accepted by the arguments that allow a choice. */
typedef enum kda_dtype { KDA_F32 = 0, KDA_F16 = 1, KDA_BF16 = 2 } kda_dtype;

/* Arguments of one forward call. Zero-initialise, then fill. */
typedef struct kda_fwd_args {
  int32_t T; /* total tokens over all sequences (batch 1, packed varlen); may be 0 */
  int32_t N; /* number of sequences, >= 1 */
  int32_t H; /* heads, >= 1 */
  int32_t K; /* key head size, must be 128 */
  int32_t V; /* value head size, must be 128 */
  float scale;       /* read-out scale, finite; 1/sqrt(K) is the usual value */
  float lower_bound; /* gate lower bound, finite and <= 0 (the pages use -5) */

  const void* q;        /* bf16 [T, H, K] ([T, H_qk, K] with grouped value heads) */
  const void* k;        /* bf16 [T, H, K] ([T, H_qk, K] with grouped value heads) */
  const void* v;        /* bf16 [T, H, V] */
  const void* g_raw;    /* [T, H, K], dtype g_dtype (KDA_F32 or KDA_BF16): raw gate */
  const void* beta_raw; /* [T, H], dtype beta_dtype (KDA_F32 or KDA_BF16): raw beta */
  kda_dtype g_dtype;
  kda_dtype beta_dtype;

  const int32_t* cu_seqlens;      /* [N+1] device sequence bounds, cu[0] = 0, cu[N] = T */
  const int32_t* cu_seqlens_host; /* [N+1] host copy, nullable. Trusted to equal the device
                                     copy and never compared with it. With it the call makes
                                     no synchronising call; without it the bounds are read
                                     back once (one counted stream synchronisation). */

  /* State, exactly one of three modes:
   *   none : all state pointers null -> zero initial state, no final state;
   *   dense: initial_state and/or final_state set (state_cache null);
   *   paged: state_cache set (initial_state and final_state null). */
  kda_dtype state_dtype;     /* element type of whichever state tensors are given */
  const void* initial_state; /* dense [N, H, V, K] ([N, H, K, V] when state_k_first),
                                nullable (null -> zero) */
  void* final_state;         /* dense, laid out as initial_state, nullable (null -> not written) */
  void* state_cache;         /* paged pool: slot s plane at state_cache + s*stride0 elements,
                                laid out [H, V, K] ([H, K, V] when state_k_first); read and
                                written in place */
  int64_t num_slots;          /* slots in the pool (>= 1 when paged) */
  int64_t state_cache_stride0; /* elements between consecutive slots, >= H*V*K */
  const int32_t* state_indices;      /* [N] device: slot of each sequence. Not validated on the
                                        device (that would need a sync): out-of-range or
                                        duplicate indices are undefined behaviour. */
  const uint8_t* has_initial_state;  /* [N] device bools: 0 -> the sequence starts from zero
                                        and its slot is not read */

  void* out; /* bf16 [T, H, V], required; must not overlap v */

  /* Grouped value heads (GVA; the default pipeline's head layout, aiter PR 5754, Technical
   * Details). 0 means H (one q/k head per value head). Otherwise 1 <= H_qk <= H and H_qk
   * divides H: q and k are then bf16 [T, H_qk, K], and value head h reads q/k head
   * h / (H / H_qk). v, g_raw, beta_raw, out and the state keep H heads. Anything else
   * returns KDA_ERR_INVALID_ARG. */
  int32_t H_qk;
  /* State plane layout for the dense tensors and the pool alike (same passage): 0 =
   * V-first [V, K] (element (v, k) at v * K + k), 1 = K-first [K, V] (element (v, k) at
   * k * V + v). Any other value returns KDA_ERR_INVALID_ARG. */
  int32_t state_k_first;
} kda_fwd_args;

/* Counters kept per context. */
typedef struct kda_stats {
  uint64_t calls;          /* successful kda_chunk_fwd calls */
  uint64_t cache_hits;     /* metadata found in the cache (no upload) */
  uint64_t cache_misses;   /* metadata built and uploaded */
  uint64_t blocking_syncs; /* host waits on the device: bounds read-backs, and (calls that may
                              not allocate) waits for arena ranges still being read */
  uint64_t d2h_reads;      /* bounds read back because cu_seqlens_host was null */
  uint64_t h2d_uploads;    /* asynchronous metadata uploads */
  int32_t last_dv_split;   /* value-channel split used by the last scan launch */
  int32_t last_ref_block;  /* reference-row block used by the last prep launch */
  int64_t last_n_chunks;   /* chunks (over all sequences) in the last call */
  int32_t last_seg_len;    /* segment length (chunks) of the last call's scan, 0 = unsegmented */
  int32_t last_n_segments; /* segments (over all sequences) in the last call */
  int32_t last_path;       /* kernels of the last call: 0 = prep + scan, 1 = decode */
  int32_t reserved;        /* zero */
  uint64_t arena_grows;        /* blocks added to the metadata arenas after context creation */
  uint64_t arena_device_bytes; /* device memory the metadata arena holds (not reset) */
  uint64_t arena_host_bytes;   /* pinned host memory the staging arena holds (not reset) */
} kda_stats;

typedef struct kda_ctx kda_ctx;

/* ---- Host-runtime seam (for tests). ----------------------------------------------
 * Every HIP runtime call and kernel launch of the host orchestration goes through this
 * table. kda_ctx_create() installs the real HIP runtime. A test can install a fake with
 * kda_ctx_create_with_runtime() to run the host logic (validation, metadata, cache,
 * uploads, synchronisation accounting, launch sequence) on a machine without a GPU.
 * Each function returns 0 on success and nonzero on failure; event_query returns 0 when
 * the event has completed, 1 while it is pending and a negative value on failure. */
typedef struct kda_runtime {
  void* user;
  int (*memcpy_h2d_async)(void* user, void* dst, const void* src, size_t bytes, void* stream);
  int (*memcpy_d2h_async)(void* user, void* dst, const void* src, size_t bytes, void* stream);
  int (*stream_synchronize)(void* user, void* stream);
  int (*stream_is_capturing)(void* user, void* stream, int* capturing);
  int (*event_create)(void* user, void** event);
  int (*event_destroy)(void* user, void* event);
  int (*event_record)(void* user, void* event, void* stream);
  int (*event_query)(void* user, void* event);
  int (*event_synchronize)(void* user, void* event);
  int (*stream_wait_event)(void* user, void* stream, void* event);
  int (*host_alloc_pinned)(void* user, void** ptr, size_t bytes);
  int (*host_free_pinned)(void* user, void* ptr);
  int (*device_alloc)(void* user, void** ptr, size_t bytes);
  int (*device_free)(void* user, void* ptr);
  /* kernel: 0 = prep (only when the call has chunks), 1 = scan, 2 = segment maps,
   * 3 = segment combine (2 and 3 only for a segmented call, between prep and scan),
   * 4 = decode (alone, when no sequence of the call has more than one token). plan
   * is internal launch data, opaque to the runtime. start and stop, when not NULL, are
   * events the launch itself records when the kernel starts and when it completes
   * (hipExtLaunchKernel), with no separate marker in the stream. */
  int (*launch)(void* user, int kernel, const void* plan, void* stream, void* start, void* stop);
  /* Timing events (used only while profiling is enabled). */
  int (*event_create_timed)(void* user, void** event);
  int (*event_elapsed_ms)(void* user, float* ms, void* start, void* end);
  /* Completion events: they only tell the host that a launch has finished (they track the
   * last use of a cached metadata buffer) and carry no memory fence. */
  int (*event_create_completion)(void* user, void** event);
  /* Metadata upload (optional; null means memcpy_h2d_async followed by event_record): copies
   * bytes from pinned host memory to device memory on stream and records done_event when the
   * copy has completed, with no separate marker in the stream. */
  int (*upload)(void* user, void* dst, const void* src, size_t bytes, void* stream, void* done_event);
} kda_runtime;

/* Context (aiter PR 6912, Changes: metadata built from host bounds, uploaded with one
 * non-blocking copy from pinned memory and cached on the bounds' contents; a hit from
 * another stream waits on the uploading stream; a buffer used under graph capture lives
 * as long as its owner). It holds the device properties (CU count), a content-keyed cache
 * of up to 64 metadata buffers, the arenas they and their pinned staging are sub-allocated
 * from, and the stats. kda_ctx_create makes a 4 MiB device block and a 4 MiB pinned block;
 * a call whose metadata does not fit in their free ranges adds a block (arena_grows in
 * kda_stats), and no call frees memory (hipFree and hipHostFree synchronise the device):
 * a range is reused once the work that reads it has completed. device is a HIP device
 * ordinal. Returns KDA_ERR_UNSUPPORTED on a device that is not gfx950 and KDA_ERR_HIP if
 * an allocation fails. One context may be used from one host thread at a time (the Python
 * binding serialises its calls on a shared context). */
kda_status kda_ctx_create(int device, kda_ctx** out);
kda_status kda_ctx_create_with_runtime(const kda_runtime* rt, int cu_count, kda_ctx** out);
/* Waits for every event the context still tracks (uploads, the launches that read its
 * metadata buffers), then frees the arenas and everything else it owns. Null is a no-op. */
void kda_ctx_destroy(kda_ctx* ctx);

/* Host-only, pure: bytes of caller workspace one call with these shapes needs. The pages
 * keep the prefill's intermediates in one workspace pool (aiter PR 4741, Optimizations
 * Applied); here it holds one 35 328-byte record per (head, chunk) that prep writes and
 * the scan reads, and, when N*H <= 96 (a call that may be segmented), room for segment maps
 * (128 KiB per map and head) and fp32 start states (64 KiB per segment start and head). It
 * depends on T, N and H only. 0 when the arguments are invalid (kda_chunk_fwd_validate). */
size_t kda_chunk_fwd_workspace_bytes(const kda_fwd_args* args);

/* Host-only: every argument check kda_chunk_fwd makes, touching no device memory (aiter PR
 * 5754, Technical Details and its review thread: a pool slot plane must be dense and
 * stride(0) may pad but not be smaller than one H*V*K plane, KDA_ERR_STRIDE; out must not
 * alias v, KDA_ERR_ALIAS; dense and paged state are mutually exclusive and a pool returns
 * no final_state, KDA_ERR_STATE_MODE; state_indices are not checked, since that would need
 * the device). Also: K = V = 128, the dtypes above, finite scale, lower_bound <= 0, 16-byte
 * aligned token tensors and state planes, H_qk dividing H, and host bounds (when given)
 * that start at 0, end at T and never decrease. Returns the first failing check's code. */
kda_status kda_chunk_fwd_validate(const kda_fwd_args* args);

/* Forward call. Validates, resolves metadata (cache hit, or one asynchronous upload from
 * pinned memory), then enqueues prep, the segment kernels when the call is segmented,
 * and scan on stream (a hipStream_t; null = default
 * stream) and returns without waiting. When no sequence of the call has more than one
 * token, a single fused decode kernel replaces prep and scan (aiter PR 4741,
 * Performance: decode runs a fused update, not the chunked path). The workspace
 * (caller-owned device memory of at least kda_chunk_fwd_workspace_bytes(args) bytes,
 * 256-byte aligned) must stay allocated and unused by anything else until the stream
 * work completes.
 *
 * Graph capture (aiter PR 6912, Changes): while stream is being captured the call needs
 * its metadata already cached. A miss, or a call without cu_seqlens_host (whose
 * read-back cannot be captured), returns KDA_ERR_CAPTURE_MISS and enqueues nothing. A hit
 * marks the cached entry as retained: it is never evicted, so the graph can be launched
 * for as long as the context lives. Captured launches carry no events. The call that
 * filled the cache entry must have completed before the graph is first launched. */
kda_status kda_chunk_fwd(kda_ctx* ctx, const kda_fwd_args* args, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Allocation-free forward call, for callers that cannot allocate memory around a call
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, checks and results as kda_chunk_fwd, with no workspace argument: the
 * workspace is a fixed array of kda_noalloc_scratch_bytes() bytes (64 MiB) that the
 * library's code object holds on every device it runs on until the process ends. The
 * call allocates and frees nothing (no hipMalloc, hipHostMalloc or frees; the metadata
 * arenas do not grow): when the call's exact workspace (35 328 bytes per chunk and head,
 * plus segment maps and start states for a segmented call; none for a decode call)
 * exceeds the array, or its metadata does not fit the arenas' free ranges even after
 * waiting for the ranges still being read (a counted blocking wait), it returns
 * KDA_ERR_NO_SPACE before enqueuing anything. 1 x 4096 tokens at H = 12 needs 54.3 MB.
 * The caller passes every input and output (out, final_state) as for kda_chunk_fwd.
 * Every call on a GPU uses that GPU's one array, which keeps the last call's contents:
 * calls that overlap in time on one GPU (other streams, other contexts, other threads)
 * race on it and must be ordered by the caller. KDA_ERR_UNSUPPORTED on a context made
 * with kda_ctx_create_with_runtime (it has no device array). */
kda_status kda_chunk_fwd_noalloc(kda_ctx* ctx, const kda_fwd_args* args, void* stream);
size_t kda_noalloc_scratch_bytes(void);

/* Host-only chunk table (aiter PR 6912, Changes and Tests): for host bounds
 * cu_host[0..n_seqs], writes pairs (sequence, chunk-within-sequence) of every chunk of
 * `chunk` tokens, sequences in cu order, an empty sequence contributing none.
 * pairs_out has room for cap pairs (2*cap int32); *n_out receives the pair count even
 * when it exceeds cap (then KDA_ERR_INVALID_ARG is returned and nothing is written). */
kda_status kda_prepare_chunk_indices(const int32_t* cu_host, int32_t n_seqs, int32_t chunk,
                                     int32_t* pairs_out, int64_t cap, int64_t* n_out);

/* Value-channel split the scan uses for n_seqs scan units (sequences, or segments of a
 * segmented call) of H heads on cu_count compute units (host-only, pure; aiter PR 4741,
 * Optimizations Applied: occupancy-aware dv_split): the finest split in {8, 4, 2} with
 * n_seqs*H*split <= cu_count, else 1. Every split of a head rereads the chunk's whole W,
 * K, Q and P: fine splits shorten the serial chain of few units, the whole head per
 * workgroup (1) spends the chip's load bandwidth best when there are many. */
int32_t kda_dv_split(int32_t n_seqs, int32_t H, int32_t cu_count);

/* Segment length (chunks) of the segmented scan for n_seqs sequences of H heads whose
 * longest sequence has max_chunks chunks, on cu_count compute units (host-only, pure);
 * 0 = not segmented. The pages split long sequences into segments (a pass that composes
 * each segment, then a scan over segments; aiter PR 5754, Technical Details and Test
 * Result; segment tables built from host bounds in the one metadata upload, aiter PR
 * 6912, Changes). Here: only when n_seqs*H <= 96 and max_chunks >= 256; about 8 segments
 * for the longest sequence, at least 8 chunks each, or 10 when 8 would already take
 * 64-channel slices (kda_dv_split 2) and 10 still do (n_seqs*H*10*2 <= cu_count <
 * n_seqs*H*8*4). cu_count = 0 gives the 8-segment length. */
int32_t kda_seg_len(int32_t n_seqs, int32_t H, int64_t max_chunks, int32_t cu_count);

/* Reference-row block the prep kernel uses for a gate lower bound (host-only, pure): the
 * largest s in {16, 8, 4, 2, 1} with (s - 1) * |lower_bound| <= 80, so that every factor
 * of the intra-chunk decay construction stays within e^{+-80} (aiter PR 4741,
 * Optimizations Applied: bounded construction, NaN-free to 640 nats). */
int32_t kda_ref_block(float lower_bound);

/* Per-kernel timing, off by default. While enabled, each kda_chunk_fwd attaches timing
 * events to its kernel launches (start and end of prep; start of the first scan-phase
 * kernel and end of the scan; for a decode call, start and end of the decode kernel), so
 * the durations are the kernels' own, with no marker in the stream. kda_profile_read
 * waits for the recorded events, adds up the prep and scan durations in milliseconds (a
 * decode call adds nothing to prep and its decode kernel to scan), reports how many
 * calls they cover, and clears them.
 * kda_profile_calls (call it before kda_profile_read) writes, in call order, up to cap
 * per-call durations in milliseconds, from the start of the call's first kernel to the
 * end of its scan, sets *n to the number of recorded calls and clears nothing.
 * Both return KDA_ERR_INVALID_ARG for null pointers (call_ms may be null when cap is 0)
 * and KDA_ERR_HIP if an event query fails. */
kda_status kda_profile_enable(kda_ctx* ctx, int enable);
kda_status kda_profile_read(kda_ctx* ctx, double* prep_ms, double* scan_ms, int64_t* calls);
kda_status kda_profile_calls(kda_ctx* ctx, float* call_ms, int64_t cap, int64_t* n);

/* sizeof(kda_fwd_args) and sizeof(kda_stats), so a binding can check its mirrors of
 * the structs. */
size_t kda_fwd_args_size(void);
size_t kda_stats_size(void);

/* A static string naming a status code ("unknown status" for other values): the error
 * conventions the codes carry follow aiter PR 5754, Technical Details (rejected stride,
 * aliasing out, conflicting state modes) and aiter PR 6912, Changes (a metadata miss under
 * graph capture is an error). */
const char* kda_status_str(kda_status status);
/* Copies the context's counters (aiter PR 6912, Tests: a call with host bounds makes no
 * synchronising call on a metadata-cache miss, the same call with device bounds does;
 * blocking_syncs and d2h_reads count exactly those waits). KDA_ERR_INVALID_ARG for null
 * pointers. kda_reset_stats zeroes every counter except the arena sizes. */
kda_status kda_get_stats(const kda_ctx* ctx, kda_stats* out);
kda_status kda_reset_stats(kda_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
