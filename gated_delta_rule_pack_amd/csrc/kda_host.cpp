// Host side of the KDA prefill library: argument validation, chunk metadata, the
// content-keyed metadata cache with asynchronous uploads from pinned memory, and the
// launch sequence (prep; for few long sequences the segment maps and their combination;
// then the scan) on the caller's stream.
//
// Metadata handling follows aiter PR 6912 (Changes): tables are built from host bounds
// when the caller has them (no read-back), otherwise the bounds are read back once;
// chunks are numbered by their sequence's position in cu_seqlens (an empty sequence
// contributes none); the tables share one int32 buffer whose blocks start 16-byte
// aligned and go up with one non-blocking copy from pinned memory; the buffer is cached
// on the bounds' contents; a hit from another stream waits on the uploading stream; a
// miss while the stream is being captured is an error; a buffer a captured stream has
// used is kept for the context's lifetime.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <new>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

using kda::kChunk;
using kda::kHead;

namespace {

// ------------------------------------------------------------------ real HIP runtime
// The only host-to-device copies are metadata uploads from the pinned staging arena
// (16-byte aligned, multiples of 16 bytes): a copy kernel on the stream reads them.
int rt_h2d(void*, void* dst, const void* src, size_t n, void* s) { return kda::launch_meta_copy(src, dst, n, s, nullptr); }
int rt_upload(void*, void* dst, const void* src, size_t n, void* s, void* done) {
  return kda::launch_meta_copy(src, dst, n, s, done);
}
int rt_d2h(void*, void* dst, const void* src, size_t n, void* s) {
  return (int)hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToHost, (hipStream_t)s);
}
int rt_sync(void*, void* s) { return (int)hipStreamSynchronize((hipStream_t)s); }
int rt_capturing(void*, void* s, int* cap) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing((hipStream_t)s, &st);
  *cap = (st == hipStreamCaptureStatusActive) ? 1 : 0;
  return (int)e;
}
int rt_ev_create(void*, void** ev) {
  return (int)hipEventCreateWithFlags(reinterpret_cast<hipEvent_t*>(ev), hipEventDisableTiming);
}
int rt_ev_destroy(void*, void* ev) { return (int)hipEventDestroy((hipEvent_t)ev); }
int rt_ev_record(void*, void* ev, void* s) { return (int)hipEventRecord((hipEvent_t)ev, (hipStream_t)s); }
int rt_ev_query(void*, void* ev) {
  hipError_t e = hipEventQuery((hipEvent_t)ev);
  if (e == hipSuccess) return 0;
  if (e == hipErrorNotReady) return 1;
  return -1;
}
int rt_ev_sync(void*, void* ev) { return (int)hipEventSynchronize((hipEvent_t)ev); }
int rt_wait(void*, void* s, void* ev) { return (int)hipStreamWaitEvent((hipStream_t)s, (hipEvent_t)ev, 0); }
int rt_host_alloc(void*, void** p, size_t n) { return (int)hipHostMalloc(p, n, hipHostMallocDefault); }
int rt_host_free(void*, void* p) { return (int)hipHostFree(p); }
int rt_dev_alloc(void*, void** p, size_t n) { return (int)hipMalloc(p, n); }
int rt_dev_free(void*, void* p) { return (int)hipFree(p); }
int rt_launch(void*, int kernel, const void* plan, void* s, void* start, void* stop) {
  const kda::Plan& p = *reinterpret_cast<const kda::Plan*>(plan);
  switch (kernel) {
    case 0: return kda::launch_prep(p, s, start, stop);
    case 1: return kda::launch_scan(p, s, start, stop);
    case 2: return kda::launch_segmap(p, s, start, stop);
    case 4: return kda::launch_decode(p, s, start, stop);
    default: return kda::launch_segcombine(p, s, start, stop);
  }
}
// Timing and completion-only events skip the system-scope fence: nothing the host reads
// depends on them, and the fence's cache write-back would idle the GPU between calls.
int rt_ev_create_timed(void*, void** ev) {
  return (int)hipEventCreateWithFlags(reinterpret_cast<hipEvent_t*>(ev), hipEventDisableSystemFence);
}
int rt_ev_create_completion(void*, void** ev) {
  return (int)hipEventCreateWithFlags(reinterpret_cast<hipEvent_t*>(ev),
                                      hipEventDisableTiming | hipEventDisableSystemFence);
}
int rt_ev_elapsed(void*, float* ms, void* a, void* b) {
  return (int)hipEventElapsedTime(ms, (hipEvent_t)a, (hipEvent_t)b);
}

const kda_runtime kHipRuntime = {nullptr,    rt_h2d,        rt_d2h,         rt_sync,     rt_capturing,
                                 rt_ev_create, rt_ev_destroy, rt_ev_record, rt_ev_query, rt_ev_sync,
                                 rt_wait,    rt_host_alloc, rt_host_free,   rt_dev_alloc, rt_dev_free,
                                 rt_launch,  rt_ev_create_timed, rt_ev_elapsed, rt_ev_create_completion,
                                 rt_upload};

// ------------------------------------------------------------------ metadata
inline size_t align4(size_t n) { return (n + 3) & ~size_t(3); }  // int32 count -> 16-byte blocks

struct Meta {
  int N = 0;
  int64_t n_chunks = 0;
  int seg_len = 0;  // chunks per segment of the segmented scan, 0 = one segment per sequence
  int n_seg = 0, n_maps = 0, n_multi = 0;
  size_t off_cu = 0, off_co = 0, off_table = 0, off_seg = 0, off_m2s = 0, off_comb = 0, words = 0;  // int32 units
};

int64_t count_chunks(const int32_t* cu, int N) {
  int64_t n = 0;
  for (int i = 0; i < N; ++i) n += (cu[i + 1] - cu[i] + kChunk - 1) / kChunk;
  return n;
}

int32_t max_seq_len(const int32_t* cu, int N) {
  int32_t m = 0;
  for (int i = 0; i < N; ++i) m = std::max(m, cu[i + 1] - cu[i]);
  return m;
}

int64_t max_seq_chunks(const int32_t* cu, int N) {
  int64_t m = 0;
  for (int i = 0; i < N; ++i) m = std::max<int64_t>(m, (cu[i + 1] - cu[i] + kChunk - 1) / kChunk);
  return m;
}

// Segments of one sequence of nc chunks (an empty sequence has one empty segment).
inline int segments_of(int64_t nc, int seg_len) {
  if (seg_len <= 0 || nc <= seg_len) return 1;
  return (int)((nc + seg_len - 1) / seg_len);
}

// Layout of the single int32 metadata buffer: token bounds [N+1], chunk offsets [N+1],
// chunk table [n_chunks][2], segment table [n_seg][kSegInts], map-slot -> segment
// [n_maps], multi-segment sequences [n_multi][4] (sequence, first map slot, maps, slot of
// the first segment's start state).
Meta meta_layout(const int32_t* cu, int N, int seg_len) {
  Meta m;
  m.N = N;
  m.n_chunks = count_chunks(cu, N);
  m.seg_len = seg_len;
  for (int i = 0; i < N; ++i) {
    const int g = segments_of((cu[i + 1] - cu[i] + kChunk - 1) / kChunk, seg_len);
    m.n_seg += g;
    m.n_maps += g - 1;
    m.n_multi += g > 1;
  }
  m.off_cu = 0;
  m.off_co = align4(N + 1);
  m.off_table = m.off_co + align4(N + 1);
  m.off_seg = m.off_table + align4((size_t)2 * m.n_chunks);
  m.off_m2s = m.off_seg + align4((size_t)kda::kSegInts * m.n_seg);
  m.off_comb = m.off_m2s + align4(m.n_maps);
  m.words = m.off_comb + align4((size_t)4 * m.n_multi);
  return m;
}

void build_meta(const int32_t* cu, const Meta& m, int32_t* buf) {
  std::memset(buf, 0, m.words * sizeof(int32_t));
  int32_t* co = buf + m.off_co;
  int32_t* table = buf + m.off_table;
  int32_t* seg = buf + m.off_seg;
  int32_t* m2s = buf + m.off_m2s;
  int32_t* comb = buf + m.off_comb;
  int64_t c = 0;
  int s = 0, mbase = 0, k = 0;
  for (int i = 0; i <= m.N; ++i) buf[m.off_cu + i] = cu[i];
  if (m.seg_len <= 0) {
    // One segment per sequence, listed longest first: the scan deals its units in table
    // order, so the longest walks start first and the short ones fill in behind them
    // (which workgroup takes which sequence changes nothing in the results).
    std::vector<int> order(m.N);
    for (int i = 0; i < m.N; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cu[a + 1] - cu[a] > cu[b + 1] - cu[b]; });
    for (int i = 0; i < m.N; ++i) {
      co[i] = (int32_t)c;
      const int nc = (cu[i + 1] - cu[i] + kChunk - 1) / kChunk;
      for (int j = 0; j < nc; ++j, ++c) {
        table[2 * c] = i;
        table[2 * c + 1] = j;
      }
    }
    for (int r = 0; r < m.N; ++r) {
      const int i = order[r];
      int32_t* e = seg + (size_t)kda::kSegInts * r;
      e[0] = i;
      e[1] = 0;
      e[2] = (cu[i + 1] - cu[i] + kChunk - 1) / kChunk;
      e[3] = -1;
      e[4] = -1;
    }
    co[m.N] = (int32_t)c;
    return;
  }
  for (int i = 0; i < m.N; ++i) {
    co[i] = (int32_t)c;
    const int nc = (cu[i + 1] - cu[i] + kChunk - 1) / kChunk;
    for (int j = 0; j < nc; ++j, ++c) {
      table[2 * c] = i;
      table[2 * c + 1] = j;
    }
    const int G = segments_of(nc, m.seg_len);
    // Start-state slots: slot j < n_maps holds the state after map slot j; slot n_maps + k
    // holds the initial state of the k-th multi-segment sequence, copied there (fp32) by
    // the combine kernel. A multi-segment sequence's last segment writes the final state
    // into the caller's plane (its slot, for a pool) from another workgroup of the scan
    // launch than its first segment, so no segment of such a sequence reads that plane.
    for (int g = 0; g < G; ++g, ++s) {
      int32_t* e = seg + (size_t)kda::kSegInts * s;
      e[0] = i;                                              // sequence
      e[1] = g * m.seg_len;                                  // first chunk (within the sequence)
      e[2] = G == 1 ? nc : std::min(m.seg_len, nc - g * m.seg_len);  // chunks
      e[3] = g > 0 ? mbase + g - 1 : (G > 1 ? m.n_maps + k : -1);  // start-state slot (-1: the caller's)
      e[4] = g == G - 1 ? -1 : mbase + g;                    // map slot this segment produces
      if (g < G - 1) m2s[mbase + g] = s;
    }
    if (G > 1) {
      comb[4 * k] = i;
      comb[4 * k + 1] = mbase;
      comb[4 * k + 2] = G - 1;
      comb[4 * k + 3] = m.n_maps + k;  // start-state slot of the sequence's first segment
      ++k;
    }
    mbase += G - 1;
  }
  co[m.N] = (int32_t)c;
}

uint64_t hash_bounds(const int32_t* cu, int N) {
  uint64_t h = 1469598103934665603ull ^ (uint64_t)N;
  for (int i = 0; i <= N; ++i) {
    h ^= (uint32_t)cu[i];
    h *= 1099511628211ull;
  }
  return h;
}

bool bounds_ok(const int32_t* cu, int N, int T) {
  if (cu[0] != 0 || cu[N] != T) return false;
  for (int i = 0; i < N; ++i)
    if (cu[i + 1] < cu[i]) return false;
  return true;
}

// Value-channel split of the scan: the finest split in {8, 4, 2} whose workgroups all
// get a CU of their own, else the whole head per workgroup (1). Few units are bound by
// the per-chunk latency (narrow slices shorten it); many by the chip's load bandwidth
// (every split rereads the chunk's shared tiles, so coarse is cheaper).
int32_t dv_split_for(int32_t units_n, int32_t H, int32_t cus) {
  const int64_t units = (int64_t)units_n * H;
  for (int s : {8, 4, 2})
    if (units * s <= (int64_t)cus) return s;
  return 1;
}

// Segment length of the segmented scan: only few, long sequences are split (many
// (sequence, head) units already fill the chip, and below 256 chunks the maps and their
// combination cost more than the shorter walk saves); about 8 segments for the longest
// sequence, at least kSegMin chunks each. Where 8 segments would already put the scan on
// 64-channel slices (dv_split 2) and 10 still fit them on cus CUs, 10: the map and scan
// walks shorten by a fifth for two more combine steps. cus = 0 gives the 8-segment length
// (the longest walk, as validation checks it).
int32_t seg_len_for(int32_t N, int32_t H, int64_t max_chunks, int32_t cus) {
  if ((int64_t)N * H > 96 || max_chunks < 256) return 0;
  const int64_t u = (int64_t)N * H;
  const int64_t n = (u * 10 * 2 <= cus && u * 8 * 4 > cus) ? 10 : 8;
  return (int32_t)std::max<int64_t>(kda::kSegMin, (max_chunks + n - 1) / n);
}

// The scan addresses one segment's chunk records through a buffer descriptor with a
// 32-bit size: a segment may span at most INT32_MAX bytes of records (60 786 chunks).
// Segmentation keeps every sequence of a call with N * H <= 96 far below that unless
// H = 1 and a sequence has more than about 15.5 M tokens.
bool walk_fits(int64_t seg_chunks) { return seg_chunks * (int64_t)kda::kRecBytes <= (int64_t)INT32_MAX; }

int32_t ref_block_for(float lb) {
  const float a = std::fabs(lb);
  for (int s : {16, 8, 4, 2})
    if ((float)(s - 1) * a <= 80.0f) return s;
  return 1;
}

bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return an && bn && a0 < b0 + bn && b0 < a0 + an;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

// ------------------------------------------------------------------ context
// First-fit sub-allocator over blocks of device or pinned host memory. The context makes
// one block of each kind when it is created. A request that fits nowhere, even after the
// completed releases have been taken back, adds a block, except in an allocation-free
// call. Blocks are freed only when the context is destroyed: hipFree and hipHostFree
// synchronise the device, so no call frees memory.
struct Arena {
  struct Block {
    char* base = nullptr;
    size_t bytes = 0;
    std::map<size_t, size_t> free;  // offset -> length of each free range, coalesced
  };
  bool device = true;
  std::vector<Block> blocks;
  size_t total = 0;
};

// A range that goes back to its arena once every event in it has completed, i.e. once
// the work that reads it (an upload, the kernels of the calls that used an evicted
// metadata buffer) has finished.
struct Release {
  Arena* arena = nullptr;
  void* ptr = nullptr;
  size_t bytes = 0;
  Arena* arena2 = nullptr;  // a second range released with the first (null: none)
  void* ptr2 = nullptr;
  size_t bytes2 = 0;
  std::vector<void*> events;       // plain events, back to their pool afterwards
  std::vector<void*> completions;  // launch-attached completion events, back to their pool
};

struct CacheEntry {
  std::vector<int32_t> bounds;  // key: the full bounds array and the segment length
  int seg_len = 0;
  uint64_t hash = 0;
  void* dev = nullptr;          // device metadata buffer (a range of the device arena)
  void* stage = nullptr;        // its pinned staging copy (a range of the pinned arena), kept
                                // with the entry, so that no event of its own tracks the upload
  size_t bytes = 0;
  Meta meta;
  void* upload_event = nullptr;  // recorded right after the upload
  void* upload_stream = nullptr;
  std::vector<std::pair<void*, void*>> uses;  // (stream, completion event of the last launch there)
  bool retained = false;                      // used under graph capture: never evicted
  uint64_t tick = 0;
};

struct ProfileMarks {
  void* ev[4];        // prep start, prep end, scan phase start (segment kernels or scan), scan end
  bool prep = false;  // the call launched prep
};

struct kda_ctx {
  kda_runtime rt{};
  int dv_split_override = 0;  // tuning only (KDA_DV_SPLIT), 0 = policy
  int seg_len_override = -1;  // tuning only (KDA_SEG_LEN), -1 = policy, 0 = never segment
  bool decode_off = false;    // testing only (KDA_DECODE=0): one-token calls take the chunked path
  bool cache_off = false;     // measurement only (KDA_META_CACHE=0): every call builds and uploads
                              // its metadata, as a call with new bounds does
  bool profiling = false;
  std::vector<ProfileMarks> marks;       // recorded, not yet read
  std::vector<ProfileMarks> marks_free;  // reusable
  int cu_count = 0;
  std::vector<CacheEntry*> cache;
  Arena dev_arena, host_arena;
  std::vector<Release> releases;  // in release order
  std::vector<void*> ev_pool, cev_pool;  // idle plain and completion events
  std::vector<int32_t> bounds_tmp;       // bounds read back from the device
  void* scratch = nullptr;  // this device's fixed workspace for allocation-free calls (null: none)
  size_t scratch_bytes = 0;
  uint64_t tick = 0;
  kda_stats stats{};
};

namespace {

constexpr size_t kCacheCap = 64;
constexpr size_t kArenaAlign = 256;
constexpr size_t kDevArenaBytes = size_t(4) << 20;   // first device block (metadata buffers)
constexpr size_t kHostArenaBytes = size_t(4) << 20;  // first pinned block (upload staging)

kda_status hip_fail() { return KDA_ERR_HIP; }

inline size_t round_arena(size_t n) { return (n + kArenaAlign - 1) / kArenaAlign * kArenaAlign; }

void* arena_take(Arena& a, size_t bytes) {
  bytes = round_arena(bytes);
  for (auto& b : a.blocks)
    for (auto it = b.free.begin(); it != b.free.end(); ++it) {
      if (it->second < bytes) continue;
      const size_t off = it->first, len = it->second;
      b.free.erase(it);
      if (len > bytes) b.free.emplace(off + bytes, len - bytes);
      return b.base + off;
    }
  return nullptr;
}

void arena_give(Arena& a, void* p, size_t bytes) {
  bytes = round_arena(bytes);
  char* c = static_cast<char*>(p);
  for (auto& b : a.blocks) {
    if (c < b.base || c >= b.base + b.bytes) continue;
    size_t off = (size_t)(c - b.base);
    auto next = b.free.lower_bound(off);
    if (next != b.free.end() && off + bytes == next->first) {
      bytes += next->second;
      next = b.free.erase(next);
    }
    if (next != b.free.begin()) {
      auto prev = std::prev(next);
      if (prev->first + prev->second == off) {
        prev->second += bytes;
        return;
      }
    }
    b.free.emplace(off, bytes);
    return;
  }
}

kda_status arena_add_block(kda_ctx* ctx, Arena& a, size_t want) {
  const size_t last = a.blocks.empty() ? 0 : a.blocks.back().bytes;
  const size_t bytes = round_arena(std::max(want, 2 * last));
  void* p = nullptr;
  const int rc = a.device ? ctx->rt.device_alloc(ctx->rt.user, &p, bytes)
                          : ctx->rt.host_alloc_pinned(ctx->rt.user, &p, bytes);
  if (rc || !p) return hip_fail();
  Arena::Block b;
  b.base = static_cast<char*>(p);
  b.bytes = bytes;
  b.free.emplace(0, bytes);
  a.blocks.push_back(std::move(b));
  a.total += bytes;
  return KDA_OK;
}

kda_status ev_get(kda_ctx* ctx, bool completion, void** ev) {
  auto& pool = completion ? ctx->cev_pool : ctx->ev_pool;
  if (!pool.empty()) {
    *ev = pool.back();
    pool.pop_back();
    return KDA_OK;
  }
  const int rc = completion ? ctx->rt.event_create_completion(ctx->rt.user, ev) : ctx->rt.event_create(ctx->rt.user, ev);
  return rc ? hip_fail() : KDA_OK;
}

bool release_done(kda_ctx* ctx, const Release& r) {
  for (void* e : r.events)
    if (ctx->rt.event_query(ctx->rt.user, e) != 0) return false;
  for (void* e : r.completions)
    if (ctx->rt.event_query(ctx->rt.user, e) != 0) return false;
  return true;
}

void finish_release(kda_ctx* ctx, Release& r) {
  arena_give(*r.arena, r.ptr, r.bytes);
  if (r.arena2) arena_give(*r.arena2, r.ptr2, r.bytes2);
  ctx->ev_pool.insert(ctx->ev_pool.end(), r.events.begin(), r.events.end());
  ctx->cev_pool.insert(ctx->cev_pool.end(), r.completions.begin(), r.completions.end());
}

// Take back every range whose readers have completed (queries only, never waits).
void sweep(kda_ctx* ctx) {
  auto& rs = ctx->releases;
  size_t w = 0;
  for (size_t i = 0; i < rs.size(); ++i) {
    if (release_done(ctx, rs[i])) {
      finish_release(ctx, rs[i]);
    } else {
      if (w != i) rs[w] = std::move(rs[i]);  // (a self-move would empty the event lists)
      ++w;
    }
  }
  rs.resize(w);
}

// Allocation-free calls only: wait for the oldest pending release that returns a range of
// arena a (one counted blocking wait) and take it back. *waited is false when none is pending.
kda_status wait_oldest(kda_ctx* ctx, Arena& a, bool* waited) {
  *waited = false;
  auto& rs = ctx->releases;
  for (size_t i = 0; i < rs.size(); ++i) {
    if (rs[i].arena != &a && rs[i].arena2 != &a) continue;
    for (void* e : rs[i].events)
      if (ctx->rt.event_synchronize(ctx->rt.user, e)) return hip_fail();
    for (void* e : rs[i].completions)
      if (ctx->rt.event_synchronize(ctx->rt.user, e)) return hip_fail();
    ctx->stats.blocking_syncs++;
    finish_release(ctx, rs[i]);
    rs.erase(rs.begin() + i);
    *waited = true;
    return KDA_OK;
  }
  return KDA_OK;
}

bool evict_one(kda_ctx* ctx);

// A range of `bytes` from arena a. may_grow: add a block when nothing fits (never waits).
// Otherwise (allocation-free calls) wait for pending releases, evicting cached metadata
// (whose device buffer and staging copy hold both arenas) when they are full of it;
// KDA_ERR_NO_SPACE when the request cannot fit.
kda_status arena_alloc(kda_ctx* ctx, Arena& a, size_t bytes, bool may_grow, void** out) {
  for (;;) {
    if ((*out = arena_take(a, bytes))) return KDA_OK;
    sweep(ctx);
    if ((*out = arena_take(a, bytes))) return KDA_OK;
    if (may_grow) {
      if (kda_status st = arena_add_block(ctx, a, bytes)) return st;
      ctx->stats.arena_grows++;
      continue;
    }
    bool waited = false;
    if (kda_status st = wait_oldest(ctx, a, &waited)) return st;
    if (waited) continue;
    if (evict_one(ctx)) continue;  // an entry's device buffer and staging copy come back together
    return KDA_ERR_NO_SPACE;
  }
}

// Move the least recently used entry that is not retained to the release list; false when
// every entry is retained (or the cache is empty).
bool evict_one(kda_ctx* ctx) {
  int victim = -1;
  for (size_t i = 0; i < ctx->cache.size(); ++i) {
    if (ctx->cache[i]->retained) continue;
    if (victim < 0 || ctx->cache[i]->tick < ctx->cache[victim]->tick) victim = (int)i;
  }
  if (victim < 0) return false;
  CacheEntry* e = ctx->cache[victim];
  Release r;
  r.arena = &ctx->dev_arena;
  r.ptr = e->dev;
  r.bytes = e->bytes;
  r.arena2 = &ctx->host_arena;
  r.ptr2 = e->stage;
  r.bytes2 = e->bytes;
  if (e->upload_event) r.events.push_back(e->upload_event);
  for (auto& u : e->uses) r.completions.push_back(u.second);
  ctx->releases.push_back(std::move(r));
  ctx->cache.erase(ctx->cache.begin() + victim);
  delete e;
  return true;
}

// The completion event that tracks this entry's last use on a stream (taken on the first
// use there). The call's last kernel records it on completion, so an evicted buffer is
// reused only after every launch that read it has finished.
kda_status use_event(kda_ctx* ctx, CacheEntry* e, void* stream, void** ev) {
  for (auto& u : e->uses)
    if (u.first == stream) {
      *ev = u.second;
      return KDA_OK;
    }
  if (kda_status st = ev_get(ctx, true, ev)) return st;
  e->uses.push_back({stream, *ev});
  return KDA_OK;
}

// Find or upload the metadata for these bounds. may_grow: the arenas may add blocks
// (false in allocation-free calls).
kda_status get_meta(kda_ctx* ctx, const int32_t* cu, int N, int seg_len, void* stream, bool may_grow,
                    CacheEntry** out, int& capturing) {
  capturing = 0;
  if (ctx->rt.stream_is_capturing(ctx->rt.user, stream, &capturing)) return hip_fail();
  const uint64_t hsh = hash_bounds(cu, N);
  for (CacheEntry* e : ctx->cache) {
    if (ctx->cache_off && !capturing) break;
    if (e->hash == hsh && e->seg_len == seg_len && (int)e->bounds.size() == N + 1 &&
        std::memcmp(e->bounds.data(), cu, (N + 1) * sizeof(int32_t)) == 0) {
      // A hit from another stream waits for the upload. Under capture the wait would
      // join an event recorded outside the graph, which capture does not allow: the
      // caller guarantees instead that the call that filled the entry has completed
      // before the graph is launched.
      if (!capturing && e->upload_stream != stream && e->upload_event) {
        if (ctx->rt.stream_wait_event(ctx->rt.user, stream, e->upload_event)) return hip_fail();
      }
      if (capturing) e->retained = true;
      e->tick = ++ctx->tick;
      ctx->stats.cache_hits++;
      *out = e;
      return KDA_OK;
    }
  }
  if (capturing) return KDA_ERR_CAPTURE_MISS;

  sweep(ctx);
  while (ctx->cache.size() >= kCacheCap)
    if (!evict_one(ctx)) break;  // everything retained
  const Meta m = meta_layout(cu, N, seg_len);
  const size_t bytes = m.words * sizeof(int32_t);

  // Pinned staging and the device buffer, both sub-allocated; the staging range goes back
  // once its copy has completed.
  void* stage = nullptr;
  if (kda_status st = arena_alloc(ctx, ctx->host_arena, bytes, may_grow, &stage)) return st;
  CacheEntry* e = new (std::nothrow) CacheEntry();
  if (!e) {
    arena_give(ctx->host_arena, stage, bytes);
    return KDA_ERR_HIP;
  }
  if (kda_status st = arena_alloc(ctx, ctx->dev_arena, bytes, may_grow, &e->dev)) {
    arena_give(ctx->host_arena, stage, bytes);
    delete e;
    return st;
  }
  build_meta(cu, m, reinterpret_cast<int32_t*>(stage));
  e->bounds.assign(cu, cu + N + 1);
  e->seg_len = seg_len;
  e->hash = hsh;
  e->meta = m;
  e->bytes = bytes;
  e->stage = stage;
  // One upload whose completion the copy itself records (no marker in the stream); the
  // staging range stays with the entry and goes back with its device buffer.
  int rc = ev_get(ctx, false, &e->upload_event) != KDA_OK;
  if (!rc) {
    if (ctx->rt.upload) {
      rc = ctx->rt.upload(ctx->rt.user, e->dev, stage, bytes, stream, e->upload_event);
    } else {
      rc = ctx->rt.memcpy_h2d_async(ctx->rt.user, e->dev, stage, bytes, stream) ||
           ctx->rt.event_record(ctx->rt.user, e->upload_event, stream);
    }
  }
  if (rc) {
    // Nothing reads the ranges if the copy was not enqueued; if it was, they stay held
    // (the copy may still run) until the context is destroyed.
    if (e->upload_event) ctx->ev_pool.push_back(e->upload_event);
    delete e;
    return hip_fail();
  }
  e->upload_stream = stream;
  e->tick = ++ctx->tick;
  ctx->cache.push_back(e);
  ctx->stats.cache_misses++;
  ctx->stats.h2d_uploads++;
  *out = e;
  return KDA_OK;
}

size_t elem_bytes(kda_dtype d) { return d == KDA_F32 ? 4 : 2; }

}  // namespace

// ================================================================== public API
extern "C" {

const char* kda_status_str(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported shape, dtype or device";
    case KDA_ERR_STATE_MODE: return "conflicting state arguments (dense vs paged)";
    case KDA_ERR_STRIDE: return "state_cache_stride0 smaller than one H*V*K plane";
    case KDA_ERR_ALIAS: return "out overlaps v";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_CAPTURE_MISS: return "metadata cache miss during stream capture";
    case KDA_ERR_HIP: return "HIP runtime error";
    case KDA_ERR_NO_SPACE: return "the call does not fit the fixed memory it may use";
  }
  return "unknown status";
}

int32_t kda_dv_split(int32_t n_seqs, int32_t H, int32_t cu_count) { return dv_split_for(n_seqs, H, cu_count); }

int32_t kda_ref_block(float lower_bound) { return ref_block_for(lower_bound); }

int32_t kda_seg_len(int32_t n_seqs, int32_t H, int64_t max_chunks, int32_t cu_count) {
  return seg_len_for(n_seqs, H, max_chunks, cu_count);
}

kda_status kda_chunk_fwd_validate(const kda_fwd_args* a) {
  if (!a) return KDA_ERR_INVALID_ARG;
  if (a->N < 1 || a->T < 0 || a->H < 1) return KDA_ERR_INVALID_ARG;
  if (a->K != kHead || a->V != kHead) return KDA_ERR_UNSUPPORTED;
  if (!std::isfinite(a->scale) || !std::isfinite(a->lower_bound)) return KDA_ERR_INVALID_ARG;
  if (a->lower_bound > 0.f) return KDA_ERR_UNSUPPORTED;
  if (a->g_dtype != KDA_F32 && a->g_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (a->beta_dtype != KDA_F32 && a->beta_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (a->state_dtype != KDA_F32 && a->state_dtype != KDA_F16 && a->state_dtype != KDA_BF16)
    return KDA_ERR_UNSUPPORTED;
  if (!a->cu_seqlens) return KDA_ERR_INVALID_ARG;
  if (a->H_qk < 0 || a->H_qk > a->H || (a->H_qk > 0 && a->H % a->H_qk != 0)) return KDA_ERR_INVALID_ARG;
  if (a->state_k_first != 0 && a->state_k_first != 1) return KDA_ERR_INVALID_ARG;
  if ((int64_t)a->T * a->H > (int64_t)INT32_MAX / kHead) return KDA_ERR_UNSUPPORTED;
  if (a->T > 0) {
    if (!a->q || !a->k || !a->v || !a->g_raw || !a->beta_raw || !a->out) return KDA_ERR_INVALID_ARG;
    // 16-byte vector accesses on every token tensor.
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->g_raw, 16) ||
        !aligned(a->out, 16) || !aligned(a->beta_raw, elem_bytes(a->beta_dtype)))
      return KDA_ERR_INVALID_ARG;
  }
  const bool dense = a->initial_state || a->final_state;
  const bool paged = a->state_cache != nullptr;
  if (dense && paged) return KDA_ERR_STATE_MODE;
  const size_t plane = (size_t)a->H * kHead * kHead;
  const size_t sz = elem_bytes(a->state_dtype);
  if (paged) {
    if (!a->state_indices || !a->has_initial_state || a->num_slots < 1) return KDA_ERR_INVALID_ARG;
    if (a->state_cache_stride0 < (int64_t)plane) return KDA_ERR_STRIDE;
    // Every slot plane must keep the 16/8-byte alignment of the state accesses.
    if (!aligned(a->state_cache, 16) || ((size_t)a->state_cache_stride0 * sz) % 16 != 0)
      return KDA_ERR_INVALID_ARG;
  }
  if (dense) {
    if ((a->initial_state && !aligned(a->initial_state, 16)) || (a->final_state && !aligned(a->final_state, 16)))
      return KDA_ERR_INVALID_ARG;
  }
  if (a->T > 0) {
    const size_t tok_bytes = (size_t)a->T * a->H * kHead * 2;
    if (ranges_overlap(a->out, tok_bytes, a->v, tok_bytes)) return KDA_ERR_ALIAS;
  }
  if (a->cu_seqlens_host) {
    if (!bounds_ok(a->cu_seqlens_host, a->N, a->T)) return KDA_ERR_INVALID_ARG;
    const int64_t mc = max_seq_chunks(a->cu_seqlens_host, a->N);
    const int32_t L = seg_len_for(a->N, a->H, mc, 0);  // the longest walk any device would take
    if (!walk_fits(L > 0 ? L : mc)) return KDA_ERR_UNSUPPORTED;
  }
  return KDA_OK;
}

kda_status kda_chunk_fwd_validate(const kda_fwd_args* a);

namespace {

// Workspace: chunk records, then the segment maps, then the segment start states (one
// per map, for the segment after it, and one per multi-segment sequence, for its first
// segment).
struct WsLayout {
  size_t records = 0, maps = 0, starts = 0, total = 0;
};

WsLayout ws_layout_for(int H, int64_t records, int64_t maps, int64_t multi) {
  WsLayout w;
  w.records = (size_t)H * (size_t)records * kda::kRecBytes;
  w.maps = w.records;
  w.starts = w.maps + (size_t)maps * H * kda::kMapBytes;
  w.total = w.starts + (size_t)(maps + multi) * H * kda::kStartBytes;
  return w;
}

// The caller's workspace, from T, N and H alone: chunks over all sequences are at most
// ceil(T / 32) + N; only a call with N * H <= 96 may be segmented, with at most
// max_chunks / kSegMin maps and no more multi-segment sequences than maps.
WsLayout ws_layout(const kda_fwd_args* a) {
  const int64_t max_chunks = ((int64_t)a->T + kChunk - 1) / kChunk + a->N;
  const int64_t max_maps = (int64_t)a->N * a->H <= 96 ? max_chunks / kda::kSegMin : 0;
  return ws_layout_for(a->H, max_chunks, max_maps, max_maps);
}

}  // namespace

size_t kda_chunk_fwd_workspace_bytes(const kda_fwd_args* a) {
  if (kda_chunk_fwd_validate(a) != KDA_OK) return 0;
  return ws_layout(a).total;
}

kda_status kda_prepare_chunk_indices(const int32_t* cu_host, int32_t n_seqs, int32_t chunk, int32_t* pairs_out,
                                     int64_t cap, int64_t* n_out) {
  if (!cu_host || n_seqs < 0 || chunk < 1 || !n_out) return KDA_ERR_INVALID_ARG;
  int64_t total = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int32_t len = cu_host[i + 1] - cu_host[i];
    if (len < 0) return KDA_ERR_INVALID_ARG;
    total += (len + chunk - 1) / chunk;
  }
  *n_out = total;
  if (total > cap || (total > 0 && !pairs_out)) return KDA_ERR_INVALID_ARG;
  int64_t c = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int32_t nc = (cu_host[i + 1] - cu_host[i] + chunk - 1) / chunk;
    for (int32_t j = 0; j < nc; ++j, ++c) {
      pairs_out[2 * c] = i;
      pairs_out[2 * c + 1] = j;
    }
  }
  return KDA_OK;
}

kda_status kda_ctx_create_with_runtime(const kda_runtime* rt, int cu_count, kda_ctx** out) {
  if (!rt || !out || cu_count < 1) return KDA_ERR_INVALID_ARG;
  kda_ctx* ctx = new (std::nothrow) kda_ctx();
  if (!ctx) return KDA_ERR_HIP;
  ctx->rt = *rt;
  ctx->cu_count = cu_count;
  // Tuning overrides, read once per context; the defaults are the documented policy.
  if (const char* e = std::getenv("KDA_DV_SPLIT")) {
    const int v = std::atoi(e);
    if (v == 1 || v == 2 || v == 4 || v == 8) ctx->dv_split_override = v;
  }
  if (const char* e = std::getenv("KDA_DECODE")) ctx->decode_off = e[0] == '0';
  if (const char* e = std::getenv("KDA_META_CACHE")) ctx->cache_off = e[0] == '0';
  if (const char* e = std::getenv("KDA_SEG_LEN")) {
    const int v = std::atoi(e);
    if (v == 0 || v >= kda::kSegMin) ctx->seg_len_override = v;
  }
  ctx->dev_arena.device = true;
  ctx->host_arena.device = false;
  if (arena_add_block(ctx, ctx->dev_arena, kDevArenaBytes) || arena_add_block(ctx, ctx->host_arena, kHostArenaBytes)) {
    kda_ctx_destroy(ctx);
    return KDA_ERR_HIP;
  }
  *out = ctx;
  return KDA_OK;
}

kda_status kda_ctx_create(int device, kda_ctx** out) {
  if (!out) return KDA_ERR_INVALID_ARG;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return KDA_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return KDA_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  if (kda::scratch_address(device, &scratch)) return KDA_ERR_HIP;
  kda_status st = kda_ctx_create_with_runtime(&kHipRuntime, prop.multiProcessorCount, out);
  if (st == KDA_OK) {
    (*out)->scratch = scratch;
    (*out)->scratch_bytes = kda::kScratchBytes;
  }
  return st;
}

void kda_ctx_destroy(kda_ctx* ctx) {
  if (!ctx) return;
  auto& rt = ctx->rt;
  std::vector<void*> evs = ctx->ev_pool, cevs = ctx->cev_pool;
  for (CacheEntry* e : ctx->cache) {
    if (e->upload_event) evs.push_back(e->upload_event);
    for (auto& u : e->uses) cevs.push_back(u.second);
    delete e;
  }
  for (auto& r : ctx->releases) {
    evs.insert(evs.end(), r.events.begin(), r.events.end());
    cevs.insert(cevs.end(), r.completions.begin(), r.completions.end());
  }
  for (auto* v : {&ctx->marks, &ctx->marks_free})
    for (auto& m : *v)
      for (void* e : m.ev) evs.push_back(e);
  // Every event is waited for before the memory its work reads is freed.
  for (auto* v : {&evs, &cevs})
    for (void* e : *v) rt.event_synchronize(rt.user, e);
  for (auto* v : {&evs, &cevs})
    for (void* e : *v) rt.event_destroy(rt.user, e);
  for (auto& b : ctx->dev_arena.blocks) rt.device_free(rt.user, b.base);
  for (auto& b : ctx->host_arena.blocks) rt.host_free_pinned(rt.user, b.base);
  delete ctx;
}

kda_status kda_get_stats(const kda_ctx* ctx, kda_stats* out) {
  if (!ctx || !out) return KDA_ERR_INVALID_ARG;
  *out = ctx->stats;
  out->arena_device_bytes = ctx->dev_arena.total;
  out->arena_host_bytes = ctx->host_arena.total;
  return KDA_OK;
}

kda_status kda_reset_stats(kda_ctx* ctx) {
  if (!ctx) return KDA_ERR_INVALID_ARG;
  ctx->stats = kda_stats{};
  return KDA_OK;
}

}  // extern "C"

namespace {

// One forward call. alloc_free: ws is a fixed device area of ws_bytes that must hold the
// call's exact workspace (else KDA_ERR_NO_SPACE), and the metadata arenas may not grow;
// otherwise ws is the caller's workspace of at least kda_chunk_fwd_workspace_bytes().
kda_status chunk_fwd_impl(kda_ctx* ctx, const kda_fwd_args* a, void* ws, size_t ws_bytes, void* stream,
                          bool alloc_free) {
  if (!ctx) return KDA_ERR_INVALID_ARG;
  kda_status st = kda_chunk_fwd_validate(a);
  if (st != KDA_OK) return st;
  if (!alloc_free) {
    const size_t need = ws_layout(a).total;
    if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256))) return KDA_ERR_WORKSPACE;
  }
  auto& rt = ctx->rt;

  // Host bounds: given, or read back once (one counted synchronisation) into a range of
  // the pinned arena, taken back right after the wait.
  const int32_t* cu = a->cu_seqlens_host;
  if (!cu) {
    int capturing = 0;
    if (rt.stream_is_capturing(rt.user, stream, &capturing)) return hip_fail();
    if (capturing) return KDA_ERR_CAPTURE_MISS;  // a read-back cannot run under capture
    const size_t bytes = (size_t)(a->N + 1) * sizeof(int32_t);
    void* land = nullptr;
    if ((st = arena_alloc(ctx, ctx->host_arena, bytes, !alloc_free, &land)) != KDA_OK) return st;
    if (rt.memcpy_d2h_async(rt.user, land, a->cu_seqlens, bytes, stream) || rt.stream_synchronize(rt.user, stream))
      return hip_fail();  // the range stays held: the copy may not have completed
    ctx->stats.blocking_syncs++;
    ctx->stats.d2h_reads++;
    ctx->bounds_tmp.assign(reinterpret_cast<const int32_t*>(land), reinterpret_cast<const int32_t*>(land) + a->N + 1);
    arena_give(ctx->host_arena, land, bytes);
    cu = ctx->bounds_tmp.data();
    if (!bounds_ok(cu, a->N, a->T)) return KDA_ERR_INVALID_ARG;
  }

  const bool decode = max_seq_len(cu, a->N) <= 1 && !ctx->decode_off;
  int seg_len = seg_len_for(a->N, a->H, max_seq_chunks(cu, a->N), ctx->cu_count);
  if (ctx->seg_len_override >= 0 && (int64_t)a->N * a->H <= 96) seg_len = ctx->seg_len_override;
  if (!decode && !walk_fits(seg_len > 0 ? seg_len : max_seq_chunks(cu, a->N))) return KDA_ERR_UNSUPPORTED;
  WsLayout wl;
  if (alloc_free) {
    // The exact workspace of this call (a decode call needs none).
    if (!decode) {
      const Meta m = meta_layout(cu, a->N, seg_len);
      wl = ws_layout_for(a->H, m.n_chunks, m.n_maps, m.n_multi);
    }
    if (wl.total > ws_bytes || (wl.total > 0 && (!ws || !aligned(ws, 256)))) return KDA_ERR_NO_SPACE;
  } else {
    wl = ws_layout(a);
  }
  CacheEntry* e = nullptr;
  int capturing = 0;
  st = get_meta(ctx, cu, a->N, seg_len, stream, !alloc_free, &e, capturing);
  if (st != KDA_OK) return st;

  kda::Plan p{};
  p.T = a->T;
  p.N = a->N;
  p.H = a->H;
  p.H_qk = a->H_qk > 0 ? a->H_qk : a->H;
  p.group = a->H / p.H_qk;
  p.kfirst = a->state_k_first;
  p.n_chunks = (int)e->meta.n_chunks;
  p.scale = a->scale;
  p.lower_bound = a->lower_bound;
  p.ref_block = ref_block_for(a->lower_bound);
  p.n_seg = e->meta.n_seg;
  p.n_maps = e->meta.n_maps;
  p.n_multi = e->meta.n_multi;
  p.seg_len = e->meta.seg_len;
  p.dv_split = ctx->dv_split_override ? ctx->dv_split_override : dv_split_for(p.n_seg, a->H, ctx->cu_count);
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.g_raw = a->g_raw;
  p.beta_raw = a->beta_raw;
  p.g_dtype = a->g_dtype == KDA_F32 ? kda::kF32 : kda::kBF16;
  p.beta_dtype = a->beta_dtype == KDA_F32 ? kda::kF32 : kda::kBF16;
  const int32_t* base = reinterpret_cast<const int32_t*>(e->dev);
  p.d_cu = base + e->meta.off_cu;
  p.d_co = base + e->meta.off_co;
  p.d_table = base + e->meta.off_table;
  p.d_seg = base + e->meta.off_seg;
  p.d_m2s = base + e->meta.off_m2s;
  p.d_comb = base + e->meta.off_comb;
  p.state_dtype = a->state_dtype == KDA_F32 ? kda::kF32 : (a->state_dtype == KDA_F16 ? kda::kF16 : kda::kBF16);
  const int64_t plane = (int64_t)a->H * kHead * kHead;
  if (a->state_cache) {
    p.state_in = a->state_cache;
    p.in_mode = kda::kStatePaged;
    p.state_out = a->state_cache;
    p.out_mode = kda::kStatePaged;
    p.stride0 = a->state_cache_stride0;
  } else {
    p.state_in = a->initial_state;
    p.in_mode = a->initial_state ? kda::kStateDense : kda::kStateNone;
    p.state_out = a->final_state;
    p.out_mode = a->final_state ? kda::kStateDense : kda::kStateNone;
    p.stride0 = plane;
  }
  p.indices = a->state_indices;
  p.flags = a->has_initial_state;
  p.out = a->out;
  p.ws = ws;
  p.maps = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + wl.maps);
  p.starts = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + wl.starts);
  p.cu_count = ctx->cu_count;
  p.stream_inputs = (size_t)a->H * (size_t)p.n_chunks * kda::kRecBytes <= kda::kMallBytes;

  // Launches. Under capture the entry is retained (never evicted), so no completion event
  // is attached, and no timing events are recorded.
  const bool prof = ctx->profiling && !capturing;
  void* use_ev = nullptr;
  if (!capturing && (st = use_event(ctx, e, stream, &use_ev)) != KDA_OK) return st;
  ProfileMarks pm{};
  if (prof) {
    if (!ctx->marks_free.empty()) {
      pm = ctx->marks_free.back();
      ctx->marks_free.pop_back();
    } else {
      for (void*& ev : pm.ev)
        if (rt.event_create_timed(rt.user, &ev)) return hip_fail();
    }
    pm.prep = p.n_chunks > 0;
  }
  if (decode) {
    // Every sequence has at most one token: the fused recurrent step alone.
    pm.prep = false;
    if (rt.launch(rt.user, 4, &p, stream, pm.ev[2], prof ? pm.ev[3] : use_ev)) return hip_fail();
  } else {
    if (p.n_chunks > 0 && rt.launch(rt.user, 0, &p, stream, pm.ev[0], pm.ev[1])) return hip_fail();
    if (p.n_maps > 0) {
      if (rt.launch(rt.user, 2, &p, stream, pm.ev[2], nullptr)) return hip_fail();
      if (rt.launch(rt.user, 3, &p, stream, nullptr, nullptr)) return hip_fail();
    }
    if (rt.launch(rt.user, 1, &p, stream, p.n_maps > 0 ? nullptr : pm.ev[2], prof ? pm.ev[3] : use_ev))
      return hip_fail();
  }
  if (prof) {
    ctx->marks.push_back(pm);
    if (use_ev && rt.event_record(rt.user, use_ev, stream)) return hip_fail();
  }
  ctx->stats.calls++;
  ctx->stats.last_dv_split = p.dv_split;
  ctx->stats.last_ref_block = p.ref_block;
  ctx->stats.last_n_chunks = e->meta.n_chunks;
  ctx->stats.last_seg_len = e->meta.seg_len;
  ctx->stats.last_n_segments = e->meta.n_seg;
  ctx->stats.last_path = decode ? 1 : 0;
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(kda_ctx* ctx, const kda_fwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  return chunk_fwd_impl(ctx, a, ws, ws_bytes, stream, false);
}

kda_status kda_chunk_fwd_noalloc(kda_ctx* ctx, const kda_fwd_args* a, void* stream) {
  if (!ctx) return KDA_ERR_INVALID_ARG;
  if (!ctx->scratch) return KDA_ERR_UNSUPPORTED;  // a context without a device (test runtime)
  return chunk_fwd_impl(ctx, a, ctx->scratch, ctx->scratch_bytes, stream, true);
}

size_t kda_noalloc_scratch_bytes(void) { return kda::kScratchBytes; }

kda_status kda_profile_enable(kda_ctx* ctx, int enable) {
  if (!ctx) return KDA_ERR_INVALID_ARG;
  ctx->profiling = enable != 0;
  return KDA_OK;
}

kda_status kda_profile_read(kda_ctx* ctx, double* prep_ms, double* scan_ms, int64_t* calls) {
  if (!ctx || !prep_ms || !scan_ms || !calls) return KDA_ERR_INVALID_ARG;
  auto& rt = ctx->rt;
  double a = 0.0, b = 0.0;
  for (auto& m : ctx->marks) {
    if (rt.event_synchronize(rt.user, m.ev[3])) return hip_fail();
    float x = 0.f, y = 0.f;
    if ((m.prep && rt.event_elapsed_ms(rt.user, &x, m.ev[0], m.ev[1])) || rt.event_elapsed_ms(rt.user, &y, m.ev[2], m.ev[3]))
      return hip_fail();
    a += x;
    b += y;
  }
  *prep_ms = a;
  *scan_ms = b;
  *calls = (int64_t)ctx->marks.size();
  ctx->marks_free.insert(ctx->marks_free.end(), ctx->marks.begin(), ctx->marks.end());
  ctx->marks.clear();
  return KDA_OK;
}

kda_status kda_profile_calls(kda_ctx* ctx, float* call_ms, int64_t cap, int64_t* n) {
  if (!ctx || !n || (cap > 0 && !call_ms)) return KDA_ERR_INVALID_ARG;
  auto& rt = ctx->rt;
  int64_t i = 0;
  for (auto& m : ctx->marks) {
    if (i < cap) {
      if (rt.event_synchronize(rt.user, m.ev[3])) return hip_fail();
      float x = 0.f;
      if (rt.event_elapsed_ms(rt.user, &x, m.prep ? m.ev[0] : m.ev[2], m.ev[3])) return hip_fail();
      call_ms[i] = x;
    }
    ++i;
  }
  *n = i;
  return KDA_OK;
}

size_t kda_fwd_args_size(void) { return sizeof(kda_fwd_args); }
size_t kda_stats_size(void) { return sizeof(kda_stats); }

}  // extern "C"
