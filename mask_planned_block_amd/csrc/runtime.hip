// Host runtime of libmpb: the C ABI declared in include/mpb.h.
//
// mask_plan_build follows the stage order of "Flex Attention Mask Plan
// Design" §4: host structural validation and consumer resolution (§4.1) with
// no elementwise work on the host; on the GPU the Varlen geometry, the Q2K
// classification whose last workgroup computes the offsets and publishes the
// 8-value header (§4.3, §4.5), and the forward schedule (§4.8); one header
// read-back (host-mapped memory, no copy command, no stream wait) that both
// sizes the exact allocation and reports device-side validation errors; then
// materialisation (§4.6), which also moves the staged plan metadata into the
// plan's block.
//
// Memory: the build workspace is a per-(host thread, device) arena reused by
// every build; each plan owns one exactly sized block carved from device
// chunks the library keeps, released in its build stream's order.  A build
// therefore makes no device allocation in the steady state and no
// device-wide synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>
#include <new>
#include <string>

#include "../../include/mpb.h"
#include "mpb_internal.h"

using namespace mpb;

// HIP events recorded on the build stream around each planner launch when
// the build asks for stage times: stage k between ev[2k] and ev[2k+1].
struct StageEvents {
  static constexpr int kStages = 6;   // geometry, classify, schedule, materialize, K2Q x2
  hipEvent_t ev[2 * kStages] = {};
  bool used[kStages] = {};
  int first = -1;                     // stage launched first
  int last = -1;                      // stage launched last
  bool on = false;
  hipError_t create() {
    on = true;
    for (hipEvent_t& e : ev) {
      const hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
  void destroy() {
    for (hipEvent_t& e : ev)
      if (e) {
        hipEventDestroy(e);
        e = nullptr;
      }
    on = false;
  }
  template <class F>
  hipError_t timed(int stage, hipStream_t s, F&& launch) {
    hipError_t r = on ? hipEventRecord(ev[2 * stage], s) : hipSuccess;
    if (r == hipSuccess) r = launch();
    if (r == hipSuccess && on) {
      r = hipEventRecord(ev[2 * stage + 1], s);
      used[stage] = true;
      if (first < 0) first = stage;
      last = stage;
    }
    return r;
  }
};

struct mpb_plan {
  int device;
  mpb_problem prob;        // binding, with the resolved tile
  mpb_signature sig;
  PlanGeo geo;
  PlanDev dev;
  K2QDev kdev;             // backward view (has_k2q)
  bool has_k2q;
  int32_t rows_total;
  int32_t num_tasks;
  int64_t header[8];
  void* block;             // every device array of the plan, one allocation
  size_t bytes;
  int blk_chunk;           // where the block sits in the device's plan heap
  size_t blk_off;
  hipStream_t stream;
  StageEvents tev;         // build stage events (time_stages)
  int build_mode;          // kBuildExact, kBuildInPlace or kBuildSinglePass
  int32_t pack;            // PackGQA: Q heads per plan row (1 = unpacked)
  // Deferred header (mpb_build_options.defer_header): the build returned
  // without reading the header back.  Until the first call that needs it
  // reads it from the plan block (resolve_header), header, rows_total and
  // num_tasks are unknown, the block keeps its upper-bound layout and a
  // forward covers tasks_upper workgroups that read the task count on the
  // device.
  std::atomic<bool> pending{false};
  std::mutex resolve_mu;
  mpb_status resolve_status = MPB_OK;
  std::string resolve_detail;
  int64_t rows_upper = 0;
  int64_t tiles_upper = 0;
  int32_t tasks_upper = 0;
};

namespace {

thread_local std::string g_detail;

mpb_status fail(mpb_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return s;
}

mpb_status ok() {
  g_detail.clear();
  return MPB_OK;
}

// ---- per-device plan memory
//
// Plan blocks are carved from device chunks the library keeps (never
// returned while the process runs), best fit with coalescing, so a build
// pays no allocator call on the device.  A destroyed plan's block is reused
// only after an event recorded on its build stream has completed, which
// gives the same ordering as a stream-ordered free on that stream.

struct PlanHeap {
  struct Chunk { char* base; size_t size; };
  struct Pending { int chunk; size_t off, size; hipEvent_t ev; };
  std::mutex mu;
  std::vector<Chunk> chunks;
  std::map<std::pair<int, size_t>, size_t> free_at;    // (chunk, offset) -> size
  std::multimap<size_t, std::pair<int, size_t>> by_size; // size -> (chunk, offset)
  std::vector<Pending> pending;
  std::vector<hipEvent_t> idle_events;

  void insert_free(int c, size_t off, size_t size) {
    // coalesce with the neighbours in the same chunk
    auto next = free_at.lower_bound({c, off});
    if (next != free_at.end() && next->first.first == c && next->first.second == off + size) {
      size += next->second;
      erase_by_size(c, next->first.second, next->second);
      next = free_at.erase(next);
    }
    if (next != free_at.begin()) {
      auto prev = std::prev(next);
      if (prev->first.first == c && prev->first.second + prev->second == off) {
        off = prev->first.second;
        size += prev->second;
        erase_by_size(c, prev->first.second, prev->second);
        free_at.erase(prev);
      }
    }
    free_at[{c, off}] = size;
    by_size.insert({size, {c, off}});
  }
  void erase_by_size(int c, size_t off, size_t size) {
    auto range = by_size.equal_range(size);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second.first == c && it->second.second == off) {
        by_size.erase(it);
        return;
      }
  }
  void reap() {
    size_t k = 0;
    for (size_t i = 0; i < pending.size(); ++i) {
      Pending& q = pending[i];
      if (hipEventQuery(q.ev) == hipSuccess) {
        insert_free(q.chunk, q.off, q.size);
        idle_events.push_back(q.ev);
      } else {
        pending[k++] = q;
      }
    }
    pending.resize(k);
  }
  hipError_t alloc(size_t bytes, void** out, int* chunk_out, size_t* off_out) {
    std::lock_guard<std::mutex> lk(mu);
    bytes = (bytes + 255) & ~(size_t)255;
    if (!pending.empty()) reap();
    auto it = by_size.lower_bound(bytes);
    if (it == by_size.end()) {
      const size_t want = std::max(bytes, (size_t)64 << 20);
      void* p = nullptr;
      hipError_t e = hipMalloc(&p, want);
      if (e != hipSuccess) return e;
      chunks.push_back({(char*)p, want});
      insert_free((int)chunks.size() - 1, 0, want);
      it = by_size.lower_bound(bytes);
    }
    const int c = it->second.first;
    const size_t off = it->second.second, size = it->first;
    by_size.erase(it);
    free_at.erase({c, off});
    if (size > bytes) insert_free(c, off + bytes, size - bytes);
    *out = chunks[c].base + off;
    *chunk_out = c;
    *off_out = off;
    return hipSuccess;
  }
  // Returns the block once everything enqueued on `stream` so far is done.
  // The event only tells the host when the stream has passed this point; no
  // memory has to become visible to the host with it, so it is recorded
  // without the system-scope fence (a fence would write back and invalidate
  // the caches between the work before it and the work after it).
  hipError_t release(int c, size_t off, size_t bytes, hipStream_t stream) {
    std::lock_guard<std::mutex> lk(mu);
    bytes = (bytes + 255) & ~(size_t)255;
    hipEvent_t ev = nullptr;
    if (!idle_events.empty()) {
      ev = idle_events.back();
      idle_events.pop_back();
    } else {
      hipError_t e =
          hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
      if (e != hipSuccess) return e;
    }
    hipError_t e = hipEventRecord(ev, stream);
    if (e != hipSuccess) {
      idle_events.push_back(ev);
      return e;
    }
    pending.push_back({c, off, bytes, ev});
    return hipSuccess;
  }
};

std::mutex g_heap_mu;
PlanHeap* g_heaps[64];

PlanHeap* plan_heap(int dev) {
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_heap_mu);
  if (!g_heaps[dev]) g_heaps[dev] = new (std::nothrow) PlanHeap;
  return g_heaps[dev];
}

// ---- per-thread host-mapped header slot and arrival counters
//
// The classify kernel's last workgroup writes the 8-value header straight
// into this pinned, coherent, device-mapped host memory and then the build's
// sequence number; the host spins on the sequence number, so the header
// read-back needs neither a copy command nor a wait for the kernel to retire.
// Builds issued from one host thread are sequential (each returns only after
// its header arrived), so one slot and one arrival counter per (thread,
// device) are never shared by two builds in flight.

// The build workspace of a (thread, device) is one arena reused by every
// build: the previous build's kernels that still read it are ordered before
// the next build's by the stream, and a build on another stream first waits
// for the stream of the previous one.
struct Arena {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipStream_t last = nullptr;
  bool used = false;
};

struct ThreadSlot {
  int32_t* pinned = nullptr;
  int32_t* pinned_dev = nullptr;
  uint32_t seq = 0;
  int32_t* arrive[64] = {};   // [64] counters: classify, K2Q count, (spare)
  Arena arena[64];
  Arena lookback[64];         // look-back words of single-pass builds
};
thread_local ThreadSlot g_slot;

hipError_t thread_slot(int dev, ThreadSlot** out) {
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!g_slot.pinned) {
    hipError_t e = hipHostMalloc((void**)&g_slot.pinned, kHostSlotInts * sizeof(int32_t),
                                 hipHostMallocMapped | hipHostMallocCoherent);
    if (e == hipSuccess) e = hipHostGetDevicePointer((void**)&g_slot.pinned_dev, g_slot.pinned, 0);
    if (e != hipSuccess) {
      if (g_slot.pinned) hipHostFree(g_slot.pinned);
      g_slot.pinned = nullptr;
      g_slot.pinned_dev = nullptr;
      return e;
    }
    for (int i = 0; i < kHostSlotInts; ++i) g_slot.pinned[i] = 0;
  }
  if (!g_slot.arrive[dev]) {
    int32_t* a = nullptr;
    hipError_t e = hipMalloc((void**)&a, 256);
    if (e == hipSuccess) e = hipMemset(a, 0, 256);
    if (e != hipSuccess) {
      if (a) hipFree(a);
      return e;
    }
    g_slot.arrive[dev] = a;
  }
  *out = &g_slot;
  return hipSuccess;
}

// An arena of at least `bytes` that no earlier build's kernels still read.
hipError_t arena_acquire(Arena& a, size_t bytes, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.used && a.last != stream && (e = hipStreamSynchronize(a.last)) != hipSuccess) return e;
  if (a.bytes < bytes) {
    if (a.ptr && ((e = hipDeviceSynchronize()) != hipSuccess || (e = hipFree(a.ptr)) != hipSuccess))
      return e;
    a.ptr = nullptr;
    a.bytes = 0;
    const size_t want = std::max(bytes + bytes / 2, (size_t)1 << 20);
    if ((e = hipMalloc(&a.ptr, want)) != hipSuccess) return e;
    a.bytes = want;
  }
  a.last = stream;
  a.used = true;
  return hipSuccess;
}

// Look-back words of single-pass builds, per (thread, device).  The buffer
// holds nothing else and is zeroed when allocated, so every word in it
// carries the tag of an earlier build of this thread, or 0.  `clear`: zero it
// again (the sequence numbers wrapped round).
hipError_t lookback_acquire(Arena& a, size_t bytes, hipStream_t stream, bool clear) {
  hipError_t e = hipSuccess;
  if (a.used && a.last != stream && (e = hipStreamSynchronize(a.last)) != hipSuccess) return e;
  if (a.bytes < bytes) {
    if (a.ptr && ((e = hipDeviceSynchronize()) != hipSuccess || (e = hipFree(a.ptr)) != hipSuccess))
      return e;
    a.ptr = nullptr;
    a.bytes = 0;
    const size_t want = std::max(bytes + bytes / 2, (size_t)1 << 16);
    if ((e = hipMalloc(&a.ptr, want)) != hipSuccess) return e;
    a.bytes = want;
    clear = true;
  }
  if (clear && (e = hipMemsetAsync(a.ptr, 0, a.bytes, stream)) != hipSuccess) return e;
  a.last = stream;
  a.used = true;
  return hipSuccess;
}

// The THD geometry launch, timed as stage 0; fixed-length plans have no
// geometry launch and no stage 0.
hipError_t geometry_stage(StageEvents& tev, const PlanGeo& g, const int32_t* cq,
                          const int32_t* ck, const PlanDev& d, const PlanWork& w, hipStream_t s) {
  if (g.layout != MPB_LAYOUT_THD) return hipSuccess;
  return tev.timed(0, s, [&] { return launch_plan_geometry(g, cq, ck, d, w, s); });
}

// Wait until the header of build `seq` has landed in the slot.  Now and then
// (every few hundred microseconds) the stream is queried: if all its work has
// completed and the sequence number is still not there, the header was never
// written.
hipError_t wait_header(ThreadSlot* slot, hipStream_t stream, uint32_t seq, bool* published,
                       int seq_index = kHeaderSeq) {
  volatile int32_t* sq = slot->pinned + seq_index;
  *published = false;
  for (uint32_t spin = 1;; ++spin) {
    if ((uint32_t)*sq == seq) break;
    if ((spin & 4095u) == 0) {
      const hipError_t e = hipStreamQuery(stream);
      if (e == hipSuccess) {
        if ((uint32_t)*sq == seq) break;
        return hipSuccess;   // the stream drained without publishing
      }
      if (e != hipErrorNotReady) return e;
    }
    __builtin_ia32_pause();
  }
  std::atomic_thread_fence(std::memory_order_acquire);
  *published = true;
  return hipSuccess;
}

// ---- layout of a device block carved into 256-byte aligned arrays

struct Carver {
  size_t off = 0;
  template <class T>
  size_t take(int64_t count) {
    const size_t o = off;
    const size_t bytes = (size_t)(count > 0 ? count : 1) * sizeof(T);
    off += (bytes + 255) & ~(size_t)255;
    return o;
  }
};

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// Arrays of one plan block for `rows` plan rows, `pnnz` partial and `fnnz`
// full tiles (exact counts, or upper bounds for a block allocated before the
// header is known).
struct BlockLayout {
  size_t header, seqdesc, cu_rows, cu_q, cu_k, work_desc, sec, rec, p_off, f_off, p_idx, f_idx,
      masks, k_cu, k_p_off, k_f_off, k_p_idx, k_f_idx, k_masks, k_order, bytes;
};
// Counts of the backward K2Q view (all zero: none).
struct K2QCounts {
  int64_t krows = 0, pnnz = 0, fnnz = 0;
  bool on = false;
};
// lists_last (single-pass builds): the payload comes before the two index
// lists, so its place does not depend on the counts and the block can be
// allocated at the upper bound and cut back to the exact size.
BlockLayout block_layout(const mpb_problem& p, int tq, int tk, int64_t rows, int64_t pnnz,
                         int64_t fnnz, const K2QCounts& kc = K2QCounts(),
                         bool lists_last = false) {
  const int64_t n_off = p.mask_heads * rows + 1;
  const int64_t tasks = rows * p.heads_q;
  const bool thd = p.layout == MPB_LAYOUT_THD;
  Carver c;
  BlockLayout L;
  L.header = c.take<int32_t>(8);
  L.seqdesc = c.take<int32_t>(8 * (int64_t)p.batch);
  L.cu_rows = c.take<int32_t>(p.batch + 1);
  L.cu_q = c.take<int32_t>(thd ? p.batch + 1 : 0);
  L.cu_k = c.take<int32_t>(thd ? p.batch + 1 : 0);
  L.work_desc = c.take<int32_t>(4 * tasks);
  L.sec = c.take<int32_t>(kNumQueues + 1);
  L.rec = c.take<int32_t>(kTaskRecInts * tasks);
  L.p_off = c.take<int32_t>(n_off);
  L.f_off = c.take<int32_t>(n_off);
  if (lists_last) {
    L.masks = c.take<uint32_t>(pnnz * tq * (tk / 32));
    L.p_idx = c.take<int32_t>(pnnz);
    L.f_idx = c.take<int32_t>(fnnz);
  } else {
    L.p_idx = c.take<int32_t>(pnnz);
    L.f_idx = c.take<int32_t>(fnnz);
    L.masks = c.take<uint32_t>(pnnz * tq * (tk / 32));
  }
  if (kc.on) {
    const int64_t nk_off = p.mask_heads * kc.krows + 1;
    L.k_cu = c.take<int32_t>(p.batch + 1);
    L.k_p_off = c.take<int32_t>(nk_off);
    L.k_f_off = c.take<int32_t>(nk_off);
    L.k_p_idx = c.take<int32_t>(kc.pnnz);
    L.k_f_idx = c.take<int32_t>(kc.fnnz);
    L.k_masks = c.take<uint32_t>(kc.pnnz * tk * (tq / 32));
    L.k_order = c.take<int32_t>(kc.krows);
  } else {
    L.k_cu = L.k_p_off = L.k_f_off = L.k_p_idx = L.k_f_idx = L.k_masks = L.k_order = 0;
  }
  L.bytes = c.off;
  return L;
}
K2QDev bind_k2q(void* block, const BlockLayout& L, bool on) {
  K2QDev k;
  std::memset(&k, 0, sizeof(k));
  if (!on) return k;
  k.cu_krows = at<int32_t>(block, L.k_cu);
  k.p_off = at<int32_t>(block, L.k_p_off);
  k.f_off = at<int32_t>(block, L.k_f_off);
  k.p_idx = at<int32_t>(block, L.k_p_idx);
  k.f_idx = at<int32_t>(block, L.k_f_idx);
  k.p_masks = at<uint32_t>(block, L.k_masks);
  k.order = at<int32_t>(block, L.k_order);
  return k;
}
PlanDev bind_block(void* block, const BlockLayout& L, bool thd) {
  PlanDev d;
  d.header = at<int32_t>(block, L.header);
  d.seqdesc = at<int32_t>(block, L.seqdesc);
  d.cu_rows = at<int32_t>(block, L.cu_rows);
  d.cu_q = thd ? at<int32_t>(block, L.cu_q) : nullptr;
  d.cu_k = thd ? at<int32_t>(block, L.cu_k) : nullptr;
  d.work_desc = at<int32_t>(block, L.work_desc);
  d.section_off = at<int32_t>(block, L.sec);
  d.task_rec = at<int32_t>(block, L.rec);
  d.p_off = at<int32_t>(block, L.p_off);
  d.f_off = at<int32_t>(block, L.f_off);
  d.p_idx = at<int32_t>(block, L.p_idx);
  d.f_idx = at<int32_t>(block, L.f_idx);
  d.p_masks = at<uint32_t>(block, L.masks);
  return d;
}

// Plans whose block at the upper bound of every count stays under this size
// are built in one pass: the block is allocated before the header is known
// and every planner kernel writes its part in place, so the launches follow
// each other with no host round trip and no staging copy.
constexpr size_t kInPlaceBlockBytes = (size_t)32 << 20;

// Forward plans whose block at the upper bound of every count, plus the list
// workspace at that bound, stays under this size are built in a single pass
// (plan_single_pass_kernel): the block is allocated at the upper bound, every
// array is written in place, and once the header is back the block is cut to
// its exact size (the payload and the lists end it), so the plan keeps no
// padding of its lists or payload.
constexpr size_t kSinglePassBytes = (size_t)2 << 30;

enum BuildMode {
  kBuildExact = MPB_BUILD_EXACT,
  kBuildInPlace = MPB_BUILD_IN_PLACE,
  kBuildSinglePass = MPB_BUILD_SINGLE_PASS,
  kBuildSinglePassDeferred = MPB_BUILD_SINGLE_PASS_DEFERRED
};

int device_cus(int dev) {
  // fixed-size cache (no allocation on any call path)
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices];
  if (dev >= 0 && dev < kDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  if (dev >= 0 && dev < kDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int default_tile_q(const mpb_problem& p) { return p.dtype == MPB_DTYPE_BF16 ? 128 : 64; }

// Physical K-tile width when the caller leaves it to the library ([TESS]:
// the physical tile is chosen for the hardware, independently of the mask's
// logical blocks).  For bf16 d = 128 with 128-row tiles both 64- and 32-wide
// K tiles exist: the 32-wide kernel holds three workgroups per CU (two for
// the 64-wide one) and halves the tile granularity, so it executes fewer
// masked score entries, but it pays a barrier and an index read per 32
// columns.  Measured on MI355X (the two tiles' forwards interleaved, medians
// of seven rounds), it is faster once the plan has at least as many tasks
// (Q tiles x heads) as the GPU holds resident 32-wide workgroups (3 per CU):
// block-sparse 362 against 467 us, causal documents 170 against 184,
// prefix-LM 712 against 742; below that (the long-K chunk's 128 tasks) each
// workgroup's own speed decides and the 64-wide kernel wins.  The task count
// is known from the geometry (for THD, total_q / 128 rows, the lower bound).
// A plan built for the backward keeps 64-wide tiles: its dK/dV consumer
// streams the Q and dO tiles of every pair once per K tile, so 32-wide K
// tiles double that traffic and cost far more in the backward than they save
// in the forward.
int default_tile_k(const mpb_problem& p, int tq, bool backward) {
  if (p.dtype == MPB_DTYPE_FP32) return p.head_dim > 64 ? 32 : 64;
  if (p.head_dim == 128 && tq == 128 && !backward) {
    const int64_t rows = p.layout == MPB_LAYOUT_BSHD
                             ? (int64_t)p.batch * ((p.seqlen_q + tq - 1) / tq)
                             : (int64_t)p.total_q / tq;
    int dev = 0;
    const int cus = hipGetDevice(&dev) == hipSuccess ? device_cus(dev) : 256;
    return rows * p.heads_q >= 3 * (int64_t)cus ? 32 : 64;
  }
  return 64;
}

mpb_signature consumer_signature(const mpb_problem& p, int tq, int tk, int pack) {
  mpb_signature s;
  s.arch = 950;
  s.direction = 0;
  s.kernel_family = p.dtype == MPB_DTYPE_BF16 ? 1 : 2;
  s.tile_q = tq;
  s.tile_k = tk;
  s.head_dim = p.head_dim;
  s.dtype = p.dtype;
  s.payload_layout = 1;
  s.scheduler = 2;
  s.pack_gqa = pack;
  return s;
}

// PackGQA ([MPD §4.1]: the consumer resolution fixes the PackGQA mapping):
// the G = heads_q / heads_k Q heads that share a K/V head fill one tile of
// T_Q / G tokens each, so the plan's rows hold T_Q / G tokens and its tasks
// are (row, K/V head).  Possible when every Q head of a group sees the same
// mask (mask_heads = 1), G is a power of two (the kernel splits a tile row
// into token and head with a shift) and the plan rows keep at least 16
// tokens, and only for forward-only plans (the backward consumers read
// unpacked tiles).  Returns the reason it is not possible, or nullptr.
const char* pack_gqa_refusal(const mpb_problem& p, int tq, bool backward) {
  const int grp = p.heads_q / p.heads_k;
  if (grp < 2) return "heads_q == heads_k (nothing to pack)";
  if (p.mask_heads != 1) return "the Q heads of a K/V group have masks of their own";
  if (grp & (grp - 1)) return "heads_q / heads_k is not a power of two";
  if (tq / grp < 16) return "tile_q / (heads_q / heads_k) < 16";
  if (backward) return "a packed plan has no backward view";
  return nullptr;
}

// Packing when the caller leaves it to the library: whenever it is
// possible.  Measured on MI355X (bf16, d = 128, forward medians, unpacked
// against packed): 16-token chunks against 8192 keys with G = 4, 118 against
// 61 us, against 32768 keys with G = 8, 216 against 84 us (a one-head tile
// leaves most rows past the chunk's end, a packed one fills them with the
// group's heads and loads every K/V tile once for all of them); 512 queries
// against 32768 keys 302 against 275 us; and with full-length sequences and
// G = 4 still ahead, as the narrower token blocks skip more of a local
// mask: window + sink 28.2 against 25.4 us, causal documents 187 against
// 165, prefix-LM + softcap + ALiBi 749 against 708.
bool pack_gqa_default(const mpb_problem&, int) { return true; }

// §4.5: what a planner header says about the build: the device error bits
// (first set of: look-back time-out, prefixes, endpoint range, endpoint
// order) or counts outside their upper bounds.
mpb_status header_status(const int64_t (&header)[8], int64_t rows_upper, int64_t tiles_upper) {
  const uint32_t err = (uint32_t)header[7];
  if (err) {
    if (err & kDevErrLookback)
      return fail(MPB_ERR_DEVICE, "a single-pass planner workgroup waited too long for the "
                                  "offsets of the rows before it");
    if (err & MPB_DEVERR_SEQLENS)
      return fail(MPB_ERR_SEQLENS,
                  "cu_seqlens must start at 0, end at total_q/total_k, be nondecreasing and "
                  "respect max_seqlen");
    if (err & MPB_DEVERR_RANGE)
      return fail(MPB_ERR_ENDPOINT_RANGE, "an endpoint is < 0 or > its sample's k_len");
    return fail(MPB_ERR_ENDPOINT_ORDER, "endpoints of some row are not nondecreasing");
  }
  const int64_t rows_total = header[0], pnnz = header[1], fnnz = header[2];
  if (rows_total < 0 || rows_total > rows_upper || pnnz < 0 || fnnz < 0 ||
      pnnz > tiles_upper || fnnz > tiles_upper)
    return fail(MPB_ERR_DEVICE, "inconsistent plan header");
  return MPB_OK;
}

// §4.1: structural validation only (no element is read on the host).
mpb_status validate_problem(const mpb_problem* p, int* tq_out, int* tk_out,
                            bool backward = false) {
  if (!p) return fail(MPB_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->layout != MPB_LAYOUT_BSHD && p->layout != MPB_LAYOUT_THD)
    return fail(MPB_ERR_INVALID_ARGUMENT, "layout %d is neither BSHD (0) nor THD (1)", p->layout);
  if (p->dtype != MPB_DTYPE_BF16 && p->dtype != MPB_DTYPE_FP32)
    return fail(MPB_ERR_INVALID_ARGUMENT, "dtype %d is neither bf16 (0) nor fp32 (1)", p->dtype);
  if (p->batch < 1) return fail(MPB_ERR_INVALID_ARGUMENT, "batch %d < 1", p->batch);
  if (p->seqlen_q < 0 || p->seqlen_k < 0)
    return fail(MPB_ERR_INVALID_ARGUMENT, "negative sequence length");
  if (p->total_q < 0 || p->total_k < 0)
    return fail(MPB_ERR_INVALID_ARGUMENT, "negative token total");
  if (p->layout == MPB_LAYOUT_BSHD) {
    if ((int64_t)p->batch * p->seqlen_q != p->total_q)
      return fail(MPB_ERR_INVALID_ARGUMENT, "BSHD total_q %d != batch*seqlen_q", p->total_q);
    if ((int64_t)p->batch * p->seqlen_k != p->total_k)
      return fail(MPB_ERR_INVALID_ARGUMENT, "BSHD total_k %d != batch*seqlen_k", p->total_k);
  }
  if (p->heads_q < 1 || p->heads_k < 1)
    return fail(MPB_ERR_INVALID_ARGUMENT, "heads_q/heads_k must be >= 1");
  if (p->heads_q % p->heads_k != 0)
    return fail(MPB_ERR_INVALID_ARGUMENT, "heads_q %d is not a multiple of heads_k %d", p->heads_q,
                p->heads_k);
  if (p->head_dim < 1) return fail(MPB_ERR_INVALID_ARGUMENT, "head_dim %d < 1", p->head_dim);
  if (p->mask_heads != 1 && p->mask_heads != p->heads_q)
    return fail(MPB_ERR_INVALID_ARGUMENT, "mask_heads %d is neither 1 nor heads_q %d",
                p->mask_heads, p->heads_q);
  if (p->nfunc < 1 || (p->nfunc % 2) == 0)
    return fail(MPB_ERR_INVALID_ARGUMENT, "nfunc %d is not a positive odd integer", p->nfunc);
  if (p->nfunc > 4095) return fail(MPB_ERR_UNSUPPORTED, "nfunc %d > 4095", p->nfunc);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(MPB_ERR_UNSUPPORTED, "head_dim %d: gfx950 consumers exist for 64 and 128",
                p->head_dim);
  const int tq = p->tile_q ? p->tile_q : default_tile_q(*p);
  if (tq != 32 && tq != 64 && tq != 128 && tq != 256)
    return fail(MPB_ERR_UNSUPPORTED, "tile_q %d not in {32,64,128,256}", tq);
  const int tk = p->tile_k ? p->tile_k : default_tile_k(*p, tq, backward);
  if (tk < 32 || tk % 32 != 0 || tk > 256)
    return fail(MPB_ERR_UNSUPPORTED, "tile_k %d is not a multiple of 32 in [32,256]", tk);
  if (!attn_variant_exists(p->dtype, p->head_dim, tq, tk))
    return fail(MPB_ERR_UNSUPPORTED,
                "no gfx950 forward consumer for dtype %d, head_dim %d, tile %dx%d", p->dtype,
                p->head_dim, tq, tk);
  const int64_t elems = (int64_t)p->total_q * p->heads_q * p->head_dim;
  if (elems > ((int64_t)1 << 40)) return fail(MPB_ERR_UNSUPPORTED, "problem too large");
  *tq_out = tq;
  *tk_out = tk;
  return MPB_OK;
}

mpb_status device_status(hipError_t e, const char* what) {
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
    return fail(MPB_ERR_OUT_OF_MEMORY, "%s: %s", what, hipGetErrorString(e));
  return fail(MPB_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// The header of a deferred plan, read from its block by the first call that
// needs it (after the build stream has drained); the outcome, the counts or
// the build's error, is kept and returned to every later call.  A plan built
// with its header read back returns MPB_OK at once.
mpb_status resolve_header(const mpb_plan* cplan) {
  mpb_plan* plan = const_cast<mpb_plan*>(cplan);
  if (plan->pending.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lk(plan->resolve_mu);
    if (plan->pending.load(std::memory_order_relaxed)) {
      int cur = 0;
      hipGetDevice(&cur);
      if (cur != plan->device) hipSetDevice(plan->device);
      int32_t h32[8] = {};
      hipError_t e = hipStreamSynchronize(plan->stream);
      if (e == hipSuccess)
        e = hipMemcpy(h32, plan->dev.header, sizeof(h32), hipMemcpyDeviceToHost);
      if (cur != plan->device) hipSetDevice(cur);
      mpb_status st;
      if (e != hipSuccess) {
        st = device_status(e, "deferred header read-back");
      } else {
        int64_t header[8];
        for (int i = 0; i < 8; ++i) header[i] = (i >= 3 && i < 7) ? 0 : h32[i];
        st = header_status(header, plan->rows_upper, plan->tiles_upper);
        if (st == MPB_OK) {
          for (int i = 0; i < 8; ++i) plan->header[i] = header[i];
          plan->rows_total = (int32_t)header[0];
          plan->num_tasks = (int32_t)(header[0] * (plan->prob.heads_q / plan->pack));
        }
      }
      plan->resolve_status = st;
      plan->resolve_detail = st == MPB_OK ? std::string() : g_detail;
      plan->pending.store(false, std::memory_order_release);
    }
  }
  if (plan->resolve_status != MPB_OK)
    return fail(plan->resolve_status, "%s", plan->resolve_detail.c_str());
  return MPB_OK;
}

}  // namespace

extern "C" {

int32_t mpb_version(void) { return 100; }

const char* mpb_status_string(mpb_status s) {
  switch (s) {
    case MPB_OK: return "MPB_OK";
    case MPB_ERR_INVALID_ARGUMENT: return "MPB_ERR_INVALID_ARGUMENT";
    case MPB_ERR_ENDPOINT_RANGE: return "MPB_ERR_ENDPOINT_RANGE";
    case MPB_ERR_ENDPOINT_ORDER: return "MPB_ERR_ENDPOINT_ORDER";
    case MPB_ERR_SEQLENS: return "MPB_ERR_SEQLENS";
    case MPB_ERR_SIGNATURE_MISMATCH: return "MPB_ERR_SIGNATURE_MISMATCH";
    case MPB_ERR_WORKSPACE: return "MPB_ERR_WORKSPACE";
    case MPB_ERR_UNSUPPORTED: return "MPB_ERR_UNSUPPORTED";
    case MPB_ERR_OUT_OF_MEMORY: return "MPB_ERR_OUT_OF_MEMORY";
    case MPB_ERR_DEVICE: return "MPB_ERR_DEVICE";
  }
  return "MPB_ERR_UNKNOWN";
}

const char* mpb_last_error_detail(void) { return g_detail.c_str(); }

mpb_status mask_plan_build(const mpb_problem* problem, const int32_t* mask_func,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* stream,
                           mpb_plan** out) {
  return mask_plan_build_ex(problem, nullptr, mask_func, cu_seqlens_q, cu_seqlens_k, stream, out);
}

mpb_status mask_plan_build_ex(const mpb_problem* problem, const mpb_build_options* options,
                              const int32_t* mask_func, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* stream, mpb_plan** out) {
  if (!out) return fail(MPB_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  const bool bwd = options && options->build_backward;
  if (options && (options->build_backward != 0 && options->build_backward != 1))
    return fail(MPB_ERR_INVALID_ARGUMENT, "build_backward must be 0 or 1");
  if (options && (options->time_stages != 0 && options->time_stages != 1))
    return fail(MPB_ERR_INVALID_ARGUMENT, "time_stages must be 0 or 1");
  const bool time_stages = options && options->time_stages;
  const int pack_opt = options ? options->pack_gqa : 0;
  if (pack_opt < 0 || pack_opt > 2)
    return fail(MPB_ERR_INVALID_ARGUMENT, "pack_gqa must be 0 (library's choice), 1 or 2");
  if (options && options->defer_header != 0 && options->defer_header != 1)
    return fail(MPB_ERR_INVALID_ARGUMENT, "defer_header must be 0 or 1");
  int tq = 0, tk = 0;
  mpb_status st = validate_problem(problem, &tq, &tk, bwd);
  if (st != MPB_OK) return st;
  const char* no_pack = pack_gqa_refusal(*problem, tq, bwd);
  if (pack_opt == 2 && no_pack) return fail(MPB_ERR_UNSUPPORTED, "PackGQA: %s", no_pack);
  const int pack = (pack_opt == 2 || (pack_opt == 0 && !no_pack &&
                                      pack_gqa_default(*problem, tq)))
                       ? problem->heads_q / problem->heads_k
                       : 1;
  // The planner's view of the problem: a packed plan's rows hold tq / pack
  // tokens and its tasks run one per K/V head.
  mpb_problem pp = *problem;
  const int tq_tile = tq;
  if (pack > 1) {
    pp.heads_q = problem->heads_k;
    tq /= pack;
    pp.tile_q = tq;
  }
  const mpb_problem& p = pp;
  if (!mask_func && p.total_q > 0) return fail(MPB_ERR_INVALID_ARGUMENT, "mask_func is NULL");
  if (p.layout == MPB_LAYOUT_THD && (!cu_seqlens_q || !cu_seqlens_k))
    return fail(MPB_ERR_INVALID_ARGUMENT, "THD layout needs cu_seqlens_q and cu_seqlens_k");

  PlanGeo g;
  g.layout = p.layout;
  g.batch = p.batch;
  g.seqlen_q = p.seqlen_q;
  g.seqlen_k = p.seqlen_k;
  g.total_q = p.total_q;
  g.total_k = p.total_k;
  g.heads_q = p.heads_q;
  g.heads_k = p.heads_k;
  g.mask_heads = p.mask_heads;
  g.nfunc = p.nfunc;
  g.tile_q = tq;
  g.tile_k = tk;
  const int64_t upper = p.layout == MPB_LAYOUT_BSHD
                            ? (int64_t)p.batch * ((p.seqlen_q + tq - 1) / tq)
                            : ((int64_t)p.total_q + (int64_t)p.batch * (tq - 1)) / tq;
  const int64_t nk_max = ((int64_t)p.seqlen_k + tk - 1) / tk;
  const int64_t words_k = nk_max > 0 ? (nk_max + 31) / 32 : 1;
  if (nk_max > kMaxKTiles)
    return fail(MPB_ERR_UNSUPPORTED, "seqlen_k %d spans more than %d K tiles of %d", p.seqlen_k,
                kMaxKTiles, tk);
  if (upper * p.mask_heads >= ((int64_t)1 << 31) || upper * p.heads_q >= ((int64_t)1 << 31) ||
      upper * p.mask_heads * words_k >= ((int64_t)1 << 31) ||
      upper * p.mask_heads * nk_max >= ((int64_t)1 << 31))
    return fail(MPB_ERR_UNSUPPORTED, "too many plan rows");
  g.upper_rows = (int32_t)upper;
  g.nk_max = (int32_t)nk_max;
  g.words_k = (int32_t)words_k;
  g.words_tile = tk / 32;

  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  PlanHeap* heap = plan_heap(dev);
  if (!heap) return fail(MPB_ERR_OUT_OF_MEMORY, "plan heap");
  ThreadSlot* slot = nullptr;
  if ((e = thread_slot(dev, &slot)) != hipSuccess) return device_status(e, "host slot");

  // Build workspace and the staged plan metadata, in the thread's arena.
  const int64_t items_upper = upper * p.mask_heads;
  const int64_t tasks_upper = upper * p.heads_q;
  const int64_t nchunks = (items_upper + 63) / 64;
  const int64_t cnt_len = (nk_max + 1) * nchunks;
  // The schedule's [cost][chunk] count matrix lives in LDS when it fits.
  const bool cnt_in_lds = cnt_len * 4 <= 60 * 1024;
  const int64_t tiles_upper = items_upper * nk_max;
  // Single pass: forward plans whose upper-bound block (lists last) and list
  // workspace fit kSinglePassBytes.
  const BlockLayout L_sp = block_layout(p, tq, tk, upper, tiles_upper, tiles_upper, K2QCounts(),
                                        true);
  const bool single = !bwd && L_sp.bytes + (size_t)tiles_upper * 8 <= kSinglePassBytes;
  // Deferred header: single-pass builds only; the single pass then writes the
  // lists straight into the block (upper-bound layout, kept as it is).
  const bool defer = single && options && options->defer_header;
  Carver cw;
  const size_t o_vis = cw.take<uint32_t>(items_upper * words_k);
  const size_t o_full = cw.take<uint32_t>(items_upper * words_k);
  const size_t o_pcnt = cw.take<int32_t>(items_upper);
  const size_t o_fcnt = cw.take<int32_t>(items_upper);
  const size_t o_first = cw.take<int32_t>(items_upper);
  const size_t o_poff = cw.take<int32_t>(items_upper + 1);
  const size_t o_foff = cw.take<int32_t>(items_upper + 1);
  const size_t o_ierr = cw.take<int32_t>(items_upper);
  const size_t o_gerr = cw.take<int32_t>(1);
  const size_t o_lrank = cw.take<int32_t>(items_upper);
  const size_t o_order = cw.take<int32_t>(items_upper);
  const size_t o_base = cw.take<int32_t>(items_upper * kNumQueues);
  const size_t o_cnt = cw.take<int32_t>(cnt_in_lds ? 1 : cnt_len);
  const size_t o_header = cw.take<int32_t>(8);
  const size_t o_seqdesc = cw.take<int32_t>(8 * (int64_t)p.batch);
  const size_t o_cu_rows = cw.take<int32_t>(p.batch + 1);
  const size_t o_cu_q = cw.take<int32_t>(p.batch + 1);
  const size_t o_cu_k = cw.take<int32_t>(p.batch + 1);
  const size_t o_work_desc = cw.take<int32_t>(4 * tasks_upper);
  const size_t o_sec = cw.take<int32_t>(kNumQueues + 1);
  const size_t o_rec = cw.take<int32_t>(kTaskRecInts * tasks_upper);
  // backward K2Q view: counts padded per sample, compact offsets, K rows
  const int64_t kpad = bwd ? (int64_t)p.mask_heads * p.batch * nk_max : 0;
  const size_t o_kpc = cw.take<int32_t>(kpad);
  const size_t o_kfc = cw.take<int32_t>(kpad);
  const size_t o_kcu = cw.take<int32_t>(bwd ? p.batch + 1 : 0);
  const size_t o_kpo = cw.take<int32_t>(bwd ? kpad + 1 : 0);
  const size_t o_kfo = cw.take<int32_t>(bwd ? kpad + 1 : 0);
  const size_t o_kin = cw.take<int32_t>(4);
  const size_t o_kord = cw.take<int32_t>(bwd ? (int64_t)p.batch * nk_max : 0);
  const size_t o_plist = cw.take<int32_t>(single ? tiles_upper : 0);
  const size_t o_flist = cw.take<int32_t>(single ? tiles_upper : 0);
  Arena& arena = slot->arena[dev];
  if ((e = arena_acquire(arena, cw.off, s)) != hipSuccess)
    return device_status(e, "planner workspace");
  void* wb = arena.ptr;

  PlanDev sg;   // staged: geometry, header and schedule before the exact allocation
  std::memset(&sg, 0, sizeof(sg));
  sg.header = at<int32_t>(wb, o_header);
  sg.seqdesc = at<int32_t>(wb, o_seqdesc);
  sg.cu_rows = at<int32_t>(wb, o_cu_rows);
  sg.cu_q = p.layout == MPB_LAYOUT_THD ? at<int32_t>(wb, o_cu_q) : nullptr;
  sg.cu_k = p.layout == MPB_LAYOUT_THD ? at<int32_t>(wb, o_cu_k) : nullptr;
  sg.work_desc = at<int32_t>(wb, o_work_desc);
  sg.section_off = at<int32_t>(wb, o_sec);
  sg.task_rec = at<int32_t>(wb, o_rec);
  PlanWork w;
  w.vis_bits = at<uint32_t>(wb, o_vis);
  w.full_bits = at<uint32_t>(wb, o_full);
  w.pcnt = at<int32_t>(wb, o_pcnt);
  w.fcnt = at<int32_t>(wb, o_fcnt);
  w.first_tile = at<int32_t>(wb, o_first);
  w.p_off_tmp = at<int32_t>(wb, o_poff);
  w.f_off_tmp = at<int32_t>(wb, o_foff);
  w.item_err = at<int32_t>(wb, o_ierr);
  w.geo_err = at<int32_t>(wb, o_gerr);
  w.lrank = at<int32_t>(wb, o_lrank);
  w.order = at<int32_t>(wb, o_order);
  w.row_base = at<int32_t>(wb, o_base);
  w.chunk_cnt = cnt_in_lds ? nullptr : at<int32_t>(wb, o_cnt);
  w.nchunks = (int32_t)nchunks;
  K2QWork kw;
  kw.pcnt = at<int32_t>(wb, o_kpc);
  kw.fcnt = at<int32_t>(wb, o_kfc);
  kw.cu_krows = at<int32_t>(wb, o_kcu);
  kw.p_off = at<int32_t>(wb, o_kpo);
  kw.f_off = at<int32_t>(wb, o_kfo);
  kw.info = at<int32_t>(wb, o_kin);
  kw.order = at<int32_t>(wb, o_kord);
  {
    // a K row's cost is at most mask_heads x the Q tiles of its sample
    const int64_t rps_max = ((int64_t)p.seqlen_q + tq - 1) / tq;
    const int64_t mc = (int64_t)p.mask_heads * rps_max;
    kw.max_cost = (int32_t)(mc < (int64_t)kK2QOrderBuckets ? mc : (int64_t)kK2QOrderBuckets);
  }

  const int32_t* cq = p.layout == MPB_LAYOUT_THD ? cu_seqlens_q : nullptr;
  const int32_t* ck = p.layout == MPB_LAYOUT_THD ? cu_seqlens_k : nullptr;
  const bool thd = p.layout == MPB_LAYOUT_THD;
  StageEvents tev;
  struct EventGuard {
    StageEvents* t;
    ~EventGuard() {
      if (t) t->destroy();
    }
  } tev_guard{&tev};
  if (time_stages && (e = tev.create()) != hipSuccess) return device_status(e, "stage events");
  uint32_t seq = ++slot->seq;
  if (seq == 0) seq = ++slot->seq;   // 0 is the slot's initial value

  // In place (small plans): the block at the upper bound of every count,
  // allocated now; every kernel writes the plan directly and the header is
  // read back only to report errors and the exact counts.
  K2QCounts kc_up;
  kc_up.on = bwd;
  if (bwd) {
    kc_up.krows = (int64_t)p.batch * nk_max;
    kc_up.pnnz = kc_up.fnnz = tiles_upper;
  }
  const BlockLayout L_up = block_layout(p, tq, tk, upper, tiles_upper, tiles_upper, kc_up);
  const bool in_place =
      !single && L_up.bytes <= kInPlaceBlockBytes && plan_finish_fits(g, cnt_in_lds, nchunks);
  void* block = nullptr;
  int blk_chunk = 0;
  size_t blk_off = 0, blk_bytes = 0;
  PlanDev d;
  std::memset(&d, 0, sizeof(d));
  K2QDev kd;
  std::memset(&kd, 0, sizeof(kd));
  if (single) {
    if ((e = lookback_acquire(slot->lookback[dev], (size_t)items_upper * kLbWords * 8, s,
                              seq == 1)) !=
        hipSuccess)
      return device_status(e, "look-back words");
    if ((e = heap->alloc(L_sp.bytes, &block, &blk_chunk, &blk_off)) != hipSuccess)
      return device_status(e, "plan allocation");
    blk_bytes = L_sp.bytes;
    d = bind_block(block, L_sp, thd);
    SinglePass sp;
    sp.lb = static_cast<uint64_t*>(slot->lookback[dev].ptr);
    sp.tag = seq;
    sp.host_slot = slot->pinned_dev;
    sp.deferred = defer ? 1 : 0;   // deferred: the header goes to the block only
    // small deferred builds: the last item schedules too (no tail launch)
    sp.fused = defer && items_upper <= kFusedMaxItems ? 1 : 0;
    sp.seq = (int32_t)seq;
    sp.p_list = defer ? d.p_idx : at<int32_t>(wb, o_plist);
    sp.f_list = defer ? d.f_idx : at<int32_t>(wb, o_flist);
    // endpoints staged in LDS when [nfunc + 6][T_Q] takes at most 48 KiB:
    // as int32 loaded straight into LDS (whole wavefronts of rows, 32-bit
    // offsets) while that takes at most 16 KiB, else as int16 when the
    // longest sample (seqlen_k) has at most kShortEpMaxLen keys (half the
    // LDS, so twice the items fit a CU, for loads through registers)
    const int64_t ep32_bytes = ((int64_t)p.nfunc + 6) * tq * 4;
    const bool short_ep = p.seqlen_k <= kShortEpMaxLen && ep32_bytes > 16 * 1024;
    const bool stage_ep = (short_ep ? ep32_bytes / 2 : ep32_bytes) <= 48 * 1024;
    sp.stage = !stage_ep ? 0
               : short_ep ? 3
               : (tq >= 64 && (int64_t)p.nfunc * p.total_q * 4 < ((int64_t)1 << 31)) ? 2
                                                                                      : 1;
    PlanWork ws = w;   // the schedule reads the plan's own offsets
    ws.p_off_tmp = d.p_off;
    ws.f_off_tmp = d.f_off;
    if ((e = geometry_stage(tev, g, cq, ck, d, w, s)) !=
            hipSuccess ||
        (e = tev.timed(1, s, [&] {
           return launch_plan_single_pass(g, mask_func, d, w, sp, thd ? -1 : (int32_t)upper, s);
         })) != hipSuccess ||
        (!sp.fused && (e = tev.timed(2, s, [&] {
           return launch_plan_single_pass_tail(g, d, ws, sp, tiles_upper, !defer, s);
         })) != hipSuccess)) {
      heap->release(blk_chunk, blk_off, blk_bytes, s);
      return device_status(e, "planner launch");
    }
  } else if (in_place) {
    if ((e = heap->alloc(L_up.bytes, &block, &blk_chunk, &blk_off)) != hipSuccess)
      return device_status(e, "plan allocation");
    blk_bytes = L_up.bytes;
    d = bind_block(block, L_up, thd);
    kd = bind_k2q(block, L_up, bwd);
    if ((e = geometry_stage(tev, g, cq, ck, d, w, s)) !=
            hipSuccess ||
        (e = tev.timed(1, s, [&] {
           return launch_plan_classify(g, mask_func, d, w, slot->arrive[dev], slot->pinned_dev,
                                       (int32_t)seq, s);
         })) != hipSuccess ||
        (e = tev.timed(2, s, [&] {
           return launch_plan_finish(g, mask_func, d, w, thd ? -1 : (int32_t)upper, s);
         })) != hipSuccess ||
        (bwd && ((e = tev.timed(4, s, [&] {
                    return launch_plan_k2q_count(g, d, w, kw, slot->arrive[dev] + 16,
                                                 slot->pinned_dev, (int32_t)seq, s);
                  })) != hipSuccess ||
                 (e = tev.timed(5, s, [&] {
                    return launch_plan_k2q_materialize(g, d, w, kw, kd, -1, s);
                  })) != hipSuccess))) {
      heap->release(blk_chunk, blk_off, blk_bytes, s);
      return device_status(e, "planner launch");
    }
  } else {
    if ((e = geometry_stage(tev, g, cq, ck, sg, w, s)) !=
            hipSuccess ||
        (e = tev.timed(1, s, [&] {
           return launch_plan_classify(g, mask_func, sg, w, slot->arrive[dev], slot->pinned_dev,
                                       (int32_t)seq, s);
         })) != hipSuccess ||
        (e = tev.timed(2, s, [&] { return launch_plan_schedule(g, sg, w, s); })) != hipSuccess ||
        (bwd && (e = tev.timed(4, s, [&] {
                   return launch_plan_k2q_count(g, sg, w, kw, slot->arrive[dev] + 16,
                                                slot->pinned_dev, (int32_t)seq, s);
                 })) != hipSuccess))
      return device_status(e, "planner launch");
  }
  auto drop_block = [&]() {
    if (block) heap->release(blk_chunk, blk_off, blk_bytes, s);
  };
  auto new_plan = [&]() -> mpb_plan* {
    mpb_plan* plan = new (std::nothrow) mpb_plan;
    if (!plan) return nullptr;
    plan->device = dev;
    plan->prob = *problem;
    plan->prob.tile_q = tq_tile;
    plan->prob.tile_k = tk;
    plan->sig = consumer_signature(*problem, tq_tile, tk, pack);
    plan->pack = pack;
    plan->geo = g;
    plan->dev = d;
    plan->kdev = kd;
    plan->has_k2q = bwd;
    plan->block = block;
    plan->bytes = blk_bytes;
    plan->blk_chunk = blk_chunk;
    plan->blk_off = blk_off;
    plan->stream = s;
    plan->tev = tev;
    plan->rows_upper = upper;
    plan->tiles_upper = tiles_upper;
    plan->tasks_upper = (int32_t)tasks_upper;
    plan->build_mode = single ? kBuildSinglePass : in_place ? kBuildInPlace : kBuildExact;
    return plan;
  };
  if (defer) {
    mpb_plan* plan = new_plan();
    if (!plan) {
      drop_block();
      return fail(MPB_ERR_OUT_OF_MEMORY, "host allocation of the plan");
    }
    plan->rows_total = 0;
    plan->num_tasks = 0;
    for (int i = 0; i < 8; ++i) plan->header[i] = 0;
    plan->build_mode = kBuildSinglePassDeferred;
    plan->pending.store(true, std::memory_order_release);
    tev_guard.t = nullptr;   // the plan owns the events now
    *out = plan;
    return ok();
  }
  // §4.5: the single header read-back of the build.
  bool published = false;
  if ((e = wait_header(slot, s, seq, &published)) != hipSuccess) {
    drop_block();
    return device_status(e, "header read-back");
  }
  if (!published) {
    drop_block();
    return fail(MPB_ERR_DEVICE, "the planner did not publish its header");
  }
  if (bwd) {   // the K2Q count publishes slots 3..6 with its own sequence number
    if ((e = wait_header(slot, s, seq, &published, kHeaderSeq2)) != hipSuccess) {
      drop_block();
      return device_status(e, "header read-back");
    }
    if (!published) {
      drop_block();
      return fail(MPB_ERR_DEVICE, "the K2Q count did not publish its header");
    }
  }
  int64_t header[8];
  for (int i = 0; i < 8; ++i) header[i] = ((volatile int32_t*)slot->pinned)[i];
  if (!bwd)
    for (int i = 3; i < 7; ++i) header[i] = 0;
  if ((st = header_status(header, upper, tiles_upper)) != MPB_OK) {
    drop_block();
    return st;
  }
  const int64_t rows_total = header[0], pnnz = header[1], fnnz = header[2];
  const int64_t tasks = rows_total * p.heads_q;
  K2QCounts kc;
  kc.on = bwd;
  if (bwd) {
    kc.krows = header[4];
    kc.pnnz = header[5];
    kc.fnnz = header[6];
    if (header[3] != rows_total || kc.krows < 0 || kc.krows > (int64_t)p.batch * nk_max ||
        kc.pnnz != pnnz || kc.fnnz != fnnz) {
      // the same block relation read K-major: its totals equal the Q2K ones
      drop_block();
      return fail(MPB_ERR_DEVICE, "inconsistent K2Q header");
    }
  }

  if (single) {
    // The exact layout keeps every place but those of the two lists (which the
    // tail launch has written behind the payload); the rest of the block goes
    // back to the heap in stream order.
    const BlockLayout L = block_layout(p, tq, tk, upper, pnnz, fnnz, K2QCounts(), true);
    d.p_idx = at<int32_t>(block, L.p_idx);
    d.f_idx = at<int32_t>(block, L.f_idx);
    if (L.bytes < blk_bytes) {
      if ((e = heap->release(blk_chunk, blk_off + L.bytes, blk_bytes - L.bytes, s)) !=
          hipSuccess) {
        drop_block();
        return device_status(e, "plan trim");
      }
      blk_bytes = L.bytes;
    }
  } else if (!in_place) {
    // Exact allocation: every retained array sized by the header, no
    // capacity padding (§4.5); one block per plan.
    const BlockLayout L = block_layout(p, tq, tk, rows_total, pnnz, fnnz, kc);
    if ((e = heap->alloc(L.bytes, &block, &blk_chunk, &blk_off)) != hipSuccess)
      return device_status(e, "plan allocation");
    blk_bytes = L.bytes;
    d = bind_block(block, L, thd);
    kd = bind_k2q(block, L, bwd);
    if ((e = tev.timed(3, s, [&] {
           return launch_plan_materialize(g, mask_func, sg, d, w, (int32_t)rows_total, s);
         })) != hipSuccess ||
        (bwd && (e = tev.timed(5, s, [&] {
                   return launch_plan_k2q_materialize(g, d, w, kw, kd, (int32_t)kc.krows, s);
                 })) != hipSuccess)) {
      drop_block();
      return device_status(e, "materialize launch");
    }
  }

  mpb_plan* plan = new_plan();
  if (!plan) {
    drop_block();
    return fail(MPB_ERR_OUT_OF_MEMORY, "host allocation of the plan");
  }
  plan->rows_total = (int32_t)rows_total;
  plan->num_tasks = (int32_t)tasks;
  for (int i = 0; i < 8; ++i) plan->header[i] = header[i];
  tev_guard.t = nullptr;   // the plan owns the events now
  *out = plan;
  return ok();
}

mpb_status mask_plan_destroy(mpb_plan* plan) {
  if (!plan) return ok();
  int cur = 0;
  hipGetDevice(&cur);
  if (cur != plan->device) hipSetDevice(plan->device);
  if (PlanHeap* heap = plan_heap(plan->device))
    heap->release(plan->blk_chunk, plan->blk_off, plan->bytes, plan->stream);
  plan->tev.destroy();
  if (cur != plan->device) hipSetDevice(cur);
  delete plan;
  return ok();
}

mpb_status mask_plan_info(const mpb_plan* plan, mpb_plan_info* info) {
  if (!plan || !info) return fail(MPB_ERR_INVALID_ARGUMENT, "plan or info is NULL");
  const mpb_status rs = resolve_header(plan);
  if (rs != MPB_OK) return rs;
  for (int i = 0; i < 8; ++i) info->header[i] = plan->header[i];
  info->rows_total = plan->rows_total;
  info->nk_max = plan->geo.nk_max;
  info->words_per_row = plan->geo.words_tile;
  info->num_tasks = plan->num_tasks;
  info->num_sections = kNumQueues;
  info->device = plan->device;
  info->problem = plan->prob;
  info->signature = plan->sig;
  info->device_bytes = (int64_t)plan->bytes;
  info->build_mode = plan->build_mode;
  info->reserved = 0;
  return ok();
}

mpb_status mask_plan_export(const mpb_plan* plan, int32_t* cu_rows, int32_t* seqdesc,
                            int32_t* p_off, int32_t* p_idx, uint32_t* p_masks, int32_t* f_off,
                            int32_t* f_idx, int32_t* work_desc, int32_t* section_off) {
  if (!plan) return fail(MPB_ERR_INVALID_ARGUMENT, "plan is NULL");
  const mpb_status rs = resolve_header(plan);
  if (rs != MPB_OK) return rs;
  int cur = 0;
  hipGetDevice(&cur);
  if (cur != plan->device) hipSetDevice(plan->device);
  hipError_t e = hipStreamSynchronize(plan->stream);
  const int64_t B = plan->prob.batch;
  const int64_t n_off = (int64_t)plan->prob.mask_heads * plan->rows_total + 1;
  const int64_t words =
      plan->header[1] * (plan->prob.tile_q / plan->pack) * (plan->prob.tile_k / 32);
  struct Copy { void* dst; const void* src; size_t bytes; } copies[] = {
      {cu_rows, plan->dev.cu_rows, (size_t)(B + 1) * 4},
      {seqdesc, plan->dev.seqdesc, (size_t)B * 32},
      {p_off, plan->dev.p_off, (size_t)n_off * 4},
      {p_idx, plan->dev.p_idx, (size_t)plan->header[1] * 4},
      {p_masks, plan->dev.p_masks, (size_t)words * 4},
      {f_off, plan->dev.f_off, (size_t)n_off * 4},
      {f_idx, plan->dev.f_idx, (size_t)plan->header[2] * 4},
      {work_desc, plan->dev.work_desc, (size_t)plan->num_tasks * 16},
      {section_off, plan->dev.section_off, (size_t)(kNumQueues + 1) * 4},
  };
  for (const Copy& c : copies) {
    if (e != hipSuccess) break;
    if (c.dst && c.bytes) e = hipMemcpy(c.dst, c.src, c.bytes, hipMemcpyDeviceToHost);
  }
  if (cur != plan->device) hipSetDevice(cur);
  if (e != hipSuccess) return device_status(e, "plan export");
  return ok();
}

mpb_status mask_plan_export_k2q(const mpb_plan* plan, int32_t* cu_krows, int32_t* p_off,
                                int32_t* p_idx, uint32_t* p_masks, int32_t* f_off,
                                int32_t* f_idx) {
  if (!plan) return fail(MPB_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!plan->has_k2q) return fail(MPB_ERR_INVALID_ARGUMENT, "the plan has no K2Q view");
  int cur = 0;
  hipGetDevice(&cur);
  if (cur != plan->device) hipSetDevice(plan->device);
  hipError_t e = hipStreamSynchronize(plan->stream);
  const int64_t B = plan->prob.batch;
  const int64_t n_off = (int64_t)plan->prob.mask_heads * plan->header[4] + 1;
  const int64_t words = plan->header[5] * plan->prob.tile_k * (plan->prob.tile_q / 32);
  struct Copy { void* dst; const void* src; size_t bytes; } copies[] = {
      {cu_krows, plan->kdev.cu_krows, (size_t)(B + 1) * 4},
      {p_off, plan->kdev.p_off, (size_t)n_off * 4},
      {p_idx, plan->kdev.p_idx, (size_t)plan->header[5] * 4},
      {p_masks, plan->kdev.p_masks, (size_t)words * 4},
      {f_off, plan->kdev.f_off, (size_t)n_off * 4},
      {f_idx, plan->kdev.f_idx, (size_t)plan->header[6] * 4},
  };
  for (const Copy& c : copies) {
    if (e != hipSuccess) break;
    if (c.dst && c.bytes) e = hipMemcpy(c.dst, c.src, c.bytes, hipMemcpyDeviceToHost);
  }
  if (cur != plan->device) hipSetDevice(cur);
  if (e != hipSuccess) return device_status(e, "K2Q export");
  return ok();
}

mpb_status mask_plan_export_k2q_order(const mpb_plan* plan, int32_t* order) {
  if (!plan || !order) return fail(MPB_ERR_INVALID_ARGUMENT, "plan or order is NULL");
  if (!plan->has_k2q) return fail(MPB_ERR_INVALID_ARGUMENT, "the plan has no K2Q view");
  int cur = 0;
  hipGetDevice(&cur);
  if (cur != plan->device) hipSetDevice(plan->device);
  hipError_t e = hipStreamSynchronize(plan->stream);
  if (e == hipSuccess && plan->header[4] > 0)
    e = hipMemcpy(order, plan->kdev.order, (size_t)plan->header[4] * 4, hipMemcpyDeviceToHost);
  if (cur != plan->device) hipSetDevice(cur);
  if (e != hipSuccess) return device_status(e, "K2Q order export");
  return ok();
}

mpb_status mask_plan_stage_times(const mpb_plan* plan, float* us) {
  if (!plan || !us) return fail(MPB_ERR_INVALID_ARGUMENT, "plan or us is NULL");
  const StageEvents& t = plan->tev;
  if (!t.on || t.last < 0)
    return fail(MPB_ERR_INVALID_ARGUMENT, "the plan was built without time_stages");
  int cur = 0;
  hipGetDevice(&cur);
  if (cur != plan->device) hipSetDevice(plan->device);
  hipError_t e = hipEventSynchronize(t.ev[2 * t.last + 1]);
  for (int k = 0; k < StageEvents::kStages && e == hipSuccess; ++k) {
    us[k] = -1.0f;
    float ms = 0.0f;
    if (t.used[k] && (e = hipEventElapsedTime(&ms, t.ev[2 * k], t.ev[2 * k + 1])) == hipSuccess)
      us[k] = ms * 1e3f;
  }
  float span = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&span, t.ev[2 * t.first], t.ev[2 * t.last + 1]);
  if (e == hipSuccess) us[StageEvents::kStages] = span * 1e3f;
  if (cur != plan->device) hipSetDevice(cur);
  if (e != hipSuccess) return device_status(e, "stage times");
  return ok();
}

mpb_status mask_plan_export_launch_order(const mpb_plan* plan, int32_t* records) {
  if (!plan || !records) return fail(MPB_ERR_INVALID_ARGUMENT, "plan or records is NULL");
  const mpb_status rs = resolve_header(plan);
  if (rs != MPB_OK) return rs;
  int cur = 0;
  hipGetDevice(&cur);
  if (cur != plan->device) hipSetDevice(plan->device);
  hipError_t e = hipStreamSynchronize(plan->stream);
  if (e == hipSuccess && plan->num_tasks > 0)
    e = hipMemcpy(records, plan->dev.task_rec, (size_t)plan->num_tasks * kTaskRecInts * 4,
                  hipMemcpyDeviceToHost);
  if (cur != plan->device) hipSetDevice(cur);
  if (e != hipSuccess) return device_status(e, "launch order export");
  return ok();
}

size_t flex_attn_fwd_workspace_size(const mpb_plan* plan) {
  (void)plan;
  return 0;  // the forward launches one workgroup per task: no scheduler state
}

// ---- Split-K ----
constexpr int32_t kMaxSplits = 64;

// Splits per task when the caller leaves the choice to the library: enough
// workgroups to give every CU its resident share (two 4-wavefront or four
// 2-wavefront workgroups) when the plan has fewer tasks, but no split shorter
// than four tiles on average (each split pays its own Q load, prologue and
// partial-state write).
static int32_t choose_splits(const mpb_plan* plan) {
  const mpb_problem& b = plan->prob;
  if (resolve_header(plan) != MPB_OK || plan->num_tasks <= 0) return 1;
  const int64_t wg_per_cu = b.tile_q >= 128 ? 2 : 4;
  const int64_t slots = (int64_t)device_cus(plan->device) * wg_per_cu;
  if (plan->num_tasks >= slots) return 1;
  const int64_t tiles =
      (plan->header[1] + plan->header[2]) * (b.heads_q / plan->pack / b.mask_heads);
  const int64_t avg = tiles / plan->num_tasks;
  int64_t sp = (slots + plan->num_tasks - 1) / plan->num_tasks;
  sp = std::min<int64_t>(sp, avg / 4);
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(sp, kMaxSplits));
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
static size_t splitk_o_bytes(const mpb_plan* plan, int32_t sp) {
  return round256((size_t)sp * plan->prob.total_q * plan->prob.heads_q * plan->prob.head_dim *
                  sizeof(float));
}
static size_t splitk_lse_bytes(const mpb_plan* plan, int32_t sp) {
  return round256((size_t)sp * plan->prob.heads_q * plan->prob.total_q * sizeof(float));
}

// Paged K/V arguments of flex_attn_fwd_paged.
struct PagedArgs {
  const int32_t* page_table;
  int32_t page_size, pages_per_seq, num_pages;
  int32_t remap;   // 0: the workspace already holds this plan's remapped lists
};

// Workspace of the paged forward: the pool tile of every listed K tile,
// partial list then full list, each area rounded to 256 bytes.
static size_t paged_remap_bytes(const mpb_plan* plan) {
  if (resolve_header(plan) != MPB_OK) return 0;
  return round256((size_t)plan->header[1] * 4) + round256((size_t)plan->header[2] * 4);
}

static mpb_status attn_common(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                              const void* k, const void* v, void* o, float* lse, float scale,
                              const mpb_score_mod* mod, void* workspace, size_t workspace_bytes,
                              void* stream, int32_t ablate, int32_t num_splits,
                              const PagedArgs* paged = nullptr) {
  if (!plan) return fail(MPB_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!problem) return fail(MPB_ERR_INVALID_ARGUMENT, "problem is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(MPB_ERR_SIGNATURE_MISMATCH, "plan built on device %d used on device %d",
                plan->device, dev);
  // A deferred plan's header is read here unless the launch can take the task
  // count on the device (the plain forward); Split-K and paged forwards size
  // their work from the counts on the host.
  const bool lazy = plan->pending.load(std::memory_order_acquire) && num_splits <= 1 && !paged;
  if (!lazy) {
    const mpb_status rs = resolve_header(plan);
    if (rs != MPB_OK) return rs;
  }
  const int32_t ntasks = lazy ? plan->tasks_upper : plan->num_tasks;
  // §7 / §8: the call's geometry must equal the plan binding field by field.
  const mpb_problem& a = *problem;
  const mpb_problem& b = plan->prob;
#define MPB_CMP(f)                                                                           \
  if (a.f != b.f)                                                                            \
    return fail(MPB_ERR_SIGNATURE_MISMATCH, "field " #f ": call has %d, plan has %d", a.f, b.f);
  MPB_CMP(layout) MPB_CMP(dtype) MPB_CMP(batch) MPB_CMP(seqlen_q) MPB_CMP(seqlen_k)
  MPB_CMP(total_q) MPB_CMP(total_k) MPB_CMP(heads_q) MPB_CMP(heads_k) MPB_CMP(head_dim)
  MPB_CMP(mask_heads) MPB_CMP(nfunc)
#undef MPB_CMP
  if ((a.tile_q && a.tile_q != b.tile_q) || (a.tile_k && a.tile_k != b.tile_k))
    return fail(MPB_ERR_SIGNATURE_MISMATCH, "tile %dx%d requested, plan has %dx%d", a.tile_q,
                a.tile_k, b.tile_q, b.tile_k);
  const mpb_signature want = consumer_signature(b, b.tile_q, b.tile_k, plan->pack);
  if (std::memcmp(&want, &plan->sig, sizeof(want)) != 0 ||
      !attn_variant_exists(b.dtype, b.head_dim, b.tile_q, b.tile_k))
    return fail(MPB_ERR_SIGNATURE_MISMATCH, "plan payload/scheduler signature does not match "
                                            "this forward consumer");
  // k and v are never read when there are no keys (every row is then empty)
  if (ntasks > 0 && (!q || !o || !lse || (b.total_k > 0 && (!k || !v))))
    return fail(MPB_ERR_INVALID_ARGUMENT, "q, k, v, o and lse must be non-NULL");
  const size_t remap_bytes = paged ? paged_remap_bytes(plan) : 0;
  const size_t ws_need =
      remap_bytes + (num_splits > 1 ? flex_attn_fwd_splitk_workspace_size(plan, num_splits)
                                    : flex_attn_fwd_workspace_size(plan));
  if (workspace_bytes < ws_need || (ws_need > 0 && !workspace))
    return fail(MPB_ERR_WORKSPACE, "workspace of %zu bytes needed", ws_need);
  if ((num_splits > 1 || paged) && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(MPB_ERR_WORKSPACE, "split-K and paged workspaces must be 256-byte aligned");
  if (paged) {
    if (b.dtype != MPB_DTYPE_BF16)
      return fail(MPB_ERR_UNSUPPORTED, "paged K/V is implemented for bf16 plans only");
    if (!paged->page_table)
      return fail(MPB_ERR_INVALID_ARGUMENT, "page_table is NULL");
    if (paged->page_size < b.tile_k || paged->page_size % b.tile_k != 0)
      return fail(MPB_ERR_UNSUPPORTED, "page_size %d must be a positive multiple of the plan's "
                  "tile_k %d", paged->page_size, b.tile_k);
    if (paged->pages_per_seq < 1 || paged->num_pages < 1)
      return fail(MPB_ERR_INVALID_ARGUMENT, "pages_per_seq and num_pages must be >= 1");
    if ((int64_t)paged->pages_per_seq * paged->page_size < b.seqlen_k)
      return fail(MPB_ERR_INVALID_ARGUMENT, "pages_per_seq * page_size = %lld < seqlen_k %d",
                  (long long)paged->pages_per_seq * paged->page_size, b.seqlen_k);
    if ((int64_t)paged->num_pages * (paged->page_size / b.tile_k) >= ((int64_t)1 << 31) ||
        (int64_t)b.batch * paged->pages_per_seq >= ((int64_t)1 << 31))
      return fail(MPB_ERR_UNSUPPORTED, "page pool or page table too large");
  }
  if (num_splits > 1 && (reinterpret_cast<uintptr_t>(o) & 15))
    return fail(MPB_ERR_INVALID_ARGUMENT, "split-K output o must be 16-byte aligned");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(MPB_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  // The kernel addresses one sample's rows of one head through 32-bit buffer
  // offsets (including one tile of overshoot past the sample end).
  const int64_t esz = b.dtype == MPB_DTYPE_BF16 ? 2 : 4;
  const int64_t qspan = ((int64_t)b.seqlen_q + b.tile_q) * b.heads_q * b.head_dim * esz;
  const int64_t kspan = paged ? 0 : ((int64_t)b.seqlen_k + b.tile_k) * b.heads_k * b.head_dim * esz;
  if (qspan >= ((int64_t)1 << 31) || kspan >= ((int64_t)1 << 31))
    return fail(MPB_ERR_UNSUPPORTED, "one sample spans >= 2 GiB of Q/K/V; not supported");
  // partial states are fp32 rows addressed like O
  if (num_splits > 1 && ((int64_t)b.seqlen_q + b.tile_q) * b.heads_q * b.head_dim * 4 >=
                            ((int64_t)1 << 31))
    return fail(MPB_ERR_UNSUPPORTED, "one sample's fp32 partial output spans >= 2 GiB");
  const bool sc = mod && mod->softcap_enabled;
  const bool al = mod && mod->alibi_enabled;
  if (sc && !(std::isfinite(mod->softcap) && mod->softcap > 0.0f))
    return fail(MPB_ERR_INVALID_ARGUMENT, "softcap must be finite and > 0");
  if (al && !mod->alibi_slopes) return fail(MPB_ERR_INVALID_ARGUMENT, "alibi_slopes is NULL");
  int32_t kind = kModNone;
  if (sc && al) kind = mod->alibi_before_softcap ? kModAlibiSoftcap : kModSoftcapAlibi;
  else if (sc) kind = kModSoftcap;
  else if (al) kind = kModAlibi;

  AttnParams prm = {};
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.lse = lse;
  prm.seqdesc = plan->dev.seqdesc;
  prm.cu_rows = plan->dev.cu_rows;
  prm.p_off = plan->dev.p_off;
  prm.p_idx = plan->dev.p_idx;
  prm.f_off = plan->dev.f_off;
  prm.f_idx = plan->dev.f_idx;
  prm.p_masks = plan->dev.p_masks;
  prm.task_rec = plan->dev.task_rec;
  prm.slopes = al ? mod->alibi_slopes : nullptr;
  prm.heads_q = b.heads_q;
  prm.heads_k = b.heads_k;
  prm.group = b.heads_q / b.heads_k;
  prm.mask_heads = b.mask_heads;
  prm.rows_total = plan->rows_total;
  prm.total_q = b.total_q;
  prm.force_partial = (ablate & MPB_ABLATE_FULL_AS_PARTIAL) ? 1 : 0;
  prm.no_skip = (ablate & MPB_ABLATE_NO_SKIP) ? 1 : 0;
  prm.pack_shift = __builtin_ctz((unsigned)plan->pack);
  prm.dev_header = lazy ? plan->dev.header : nullptr;
  prm.task_heads = b.heads_q / plan->pack;
  const float log2e = 1.4426950408889634f;
  prm.scale_log2 = scale * log2e;
  prm.softcap_k = sc ? 2.0f * scale * log2e / mod->softcap : 0.0f;
  prm.softcap_c2 = sc ? mod->softcap * log2e : 0.0f;
  prm.alibi_k = sc ? 2.0f * log2e / mod->softcap : 0.0f;
  // the bound of full tiles' softcapped scores serves as their reference max
  // while weights within 2c of it stay far from underflow (c <= 31.8)
  prm.cap_bounded = sc && 2.0f * prm.softcap_c2 + 8.0f <= 100.0f ? 1 : 0;
  if (ntasks == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (paged) {
    RemapParams rp;
    rp.cu_rows = plan->dev.cu_rows;
    rp.p_off = plan->dev.p_off;
    rp.f_off = plan->dev.f_off;
    rp.p_idx = plan->dev.p_idx;
    rp.f_idx = plan->dev.f_idx;
    rp.page_table = paged->page_table;
    rp.phys_p = static_cast<int32_t*>(workspace);
    rp.phys_f = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                           round256((size_t)plan->header[1] * 4));
    rp.rows_total = plan->rows_total;
    rp.rows_flat = b.mask_heads * plan->rows_total;
    rp.batch = b.batch;
    rp.tile_k = b.tile_k;
    rp.page_size = paged->page_size;
    rp.pages_per_seq = paged->pages_per_seq;
    rp.num_pages = paged->num_pages;
    if (paged->remap && (e = launch_page_remap(rp, s)) != hipSuccess)
      return device_status(e, "page remap launch");
    prm.paged = 1;
    prm.phys_p = rp.phys_p;
    prm.phys_f = rp.phys_f;
    workspace = static_cast<char*>(workspace) + remap_bytes;
  }
  if (num_splits <= 1) {
    if ((e = launch_attn_fwd(b.dtype, b.head_dim, b.tile_q, b.tile_k, kind, ntasks, prm, s)) !=
        hipSuccess)
      return device_status(e, "attention launch");
    return ok();
  }
  // Split-K: the splits of a task are tasks_padded workgroups apart; with
  // tasks_padded a multiple of the 8 XCDs every split of a task runs on the
  // XCD its launch slot maps to (the plan's section for that slot).
  prm.num_tasks = plan->num_tasks;
  prm.num_splits = num_splits;
  prm.tasks_padded = (plan->num_tasks + kNumSections - 1) / kNumSections * kNumSections;
  prm.o_part = static_cast<float*>(workspace);
  prm.lse_part =
      reinterpret_cast<float*>(static_cast<char*>(workspace) + splitk_o_bytes(plan, num_splits));
  if ((e = launch_attn_fwd_split(b.dtype, b.head_dim, b.tile_q, b.tile_k, kind, prm, s)) !=
      hipSuccess)
    return device_status(e, "split-K attention launch");
  MergeParams mp;
  mp.o_part = prm.o_part;
  mp.lse_part = prm.lse_part;
  mp.o = o;
  mp.lse = lse;
  mp.rows = (int64_t)b.total_q * b.heads_q;
  mp.parts = num_splits;
  mp.heads_q = b.heads_q;
  mp.total_q = b.total_q;
  if ((e = launch_attn_merge(b.dtype, b.head_dim, mp, s)) != hipSuccess)
    return device_status(e, "split-K merge launch");
  return ok();
}

int32_t flex_attn_fwd_num_splits(const mpb_plan* plan) {
  return plan ? choose_splits(plan) : 1;
}

size_t flex_attn_fwd_splitk_workspace_size(const mpb_plan* plan, int32_t num_splits) {
  if (!plan || num_splits < 0 || num_splits > kMaxSplits) return 0;
  const int32_t sp = num_splits == 0 ? choose_splits(plan) : num_splits;
  if (sp <= 1) return flex_attn_fwd_workspace_size(plan);
  return splitk_o_bytes(plan, sp) + splitk_lse_bytes(plan, sp);
}

mpb_status flex_attn_fwd_splitk(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                                const void* k, const void* v, void* o, float* lse, float scale,
                                const mpb_score_mod* mod, int32_t num_splits, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MPB_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(MPB_ERR_INVALID_ARGUMENT, "num_splits must be in [0, %d]", kMaxSplits);
  const int32_t sp = num_splits == 0 ? choose_splits(plan) : num_splits;
  return attn_common(plan, problem, q, k, v, o, lse, scale, mod, workspace, workspace_bytes,
                     stream, 0, sp);
}

}  // extern "C"

// Scratch of flex_attn_fwd_splitk_noalloc: the Split-K partial states live
// in this file-scope device array instead of a caller workspace.  Every GPU
// the library runs on holds its own copy until the process ends; host code
// reaches it only through the address hipGetSymbolAddress returns for the
// current device (the array's name is a host-side stand-in).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// Device address of this device's scratch, looked up once per device with
// that device current.
mpb_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MPB_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kScratchDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return device_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MPB_OK;
}
}  // namespace

extern "C" {

mpb_status flex_attn_fwd_splitk_noalloc(const mpb_plan* plan, const mpb_problem* problem,
                                        const void* q, const void* k, const void* v, void* o,
                                        float* lse, float scale, const mpb_score_mod* mod,
                                        int32_t num_splits, void* stream) {
  if (!plan) return fail(MPB_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(MPB_ERR_INVALID_ARGUMENT, "num_splits must be in [0, %d]", kMaxSplits);
  const int32_t sp = num_splits == 0 ? choose_splits(plan) : num_splits;
  const size_t need = sp > 1 ? splitk_o_bytes(plan, sp) + splitk_lse_bytes(plan, sp) : 0;
  if (need > kNoAllocScratchBytes)
    return fail(MPB_ERR_WORKSPACE, "%d parts need %zu bytes of partial states; the static "
                "scratch holds %zu (use flex_attn_fwd_splitk with a workspace)", sp, need,
                kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, "hipGetDevice");
    const mpb_status st = scratch_address(dev, &ws);
    if (st != MPB_OK) return st;
  }
  return attn_common(plan, problem, q, k, v, o, lse, scale, mod, ws, need, stream, 0, sp);
}

size_t flex_attn_fwd_paged_workspace_size(const mpb_plan* plan, int32_t num_splits) {
  if (!plan || num_splits < 0 || num_splits > kMaxSplits) return 0;
  const int32_t sp = num_splits == 0 ? choose_splits(plan) : num_splits;
  return paged_remap_bytes(plan) +
         (sp > 1 ? splitk_o_bytes(plan, sp) + splitk_lse_bytes(plan, sp) : 0);
}

mpb_status flex_attn_fwd_paged(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                               const void* k_pages, const void* v_pages,
                               const int32_t* page_table, int32_t page_size,
                               int32_t pages_per_seq, int32_t num_pages, void* o, float* lse,
                               float scale, const mpb_score_mod* mod, int32_t num_splits,
                               int32_t remap, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!plan) return fail(MPB_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(MPB_ERR_INVALID_ARGUMENT, "num_splits must be in [0, %d]", kMaxSplits);
  if (remap != 0 && remap != 1) return fail(MPB_ERR_INVALID_ARGUMENT, "remap must be 0 or 1");
  const int32_t sp = num_splits == 0 ? choose_splits(plan) : num_splits;
  const PagedArgs pg = {page_table, page_size, pages_per_seq, num_pages, remap};
  return attn_common(plan, problem, q, k_pages, v_pages, o, lse, scale, mod, workspace,
                     workspace_bytes, stream, 0, sp, &pg);
}

mpb_status flex_attn_fwd_merge(int32_t num_parts, int32_t total_q, int32_t heads_q,
                               int32_t head_dim, int32_t dtype, const float* o_parts,
                               const float* lse_parts, void* o, float* lse, void* stream) {
  if (num_parts < 1 || total_q < 0 || heads_q < 1)
    return fail(MPB_ERR_INVALID_ARGUMENT, "need num_parts >= 1, total_q >= 0, heads_q >= 1");
  if (head_dim != 64 && head_dim != 128)
    return fail(MPB_ERR_UNSUPPORTED, "merge supports head_dim 64 and 128, got %d", head_dim);
  if (dtype != MPB_DTYPE_BF16 && dtype != MPB_DTYPE_FP32)
    return fail(MPB_ERR_INVALID_ARGUMENT, "dtype must be MPB_DTYPE_BF16 or MPB_DTYPE_FP32");
  const int64_t rows = (int64_t)total_q * heads_q;
  if (rows == 0) return ok();
  if (!o_parts || !lse_parts || !o || !lse)
    return fail(MPB_ERR_INVALID_ARGUMENT, "o_parts, lse_parts, o and lse must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(o_parts) & 15) || (reinterpret_cast<uintptr_t>(o) & 15))
    return fail(MPB_ERR_INVALID_ARGUMENT, "o_parts and o must be 16-byte aligned");
  MergeParams mp;
  mp.o_part = o_parts;
  mp.lse_part = lse_parts;
  mp.o = o;
  mp.lse = lse;
  mp.rows = rows;
  mp.parts = num_parts;
  mp.heads_q = heads_q;
  mp.total_q = total_q;
  const hipError_t e = launch_attn_merge(dtype, head_dim, mp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_status(e, "merge launch");
  return ok();
}

// Two fp32 vectors per (head, Q row): dO . O and the LSE in log2 units.
static size_t bwd_vec_bytes(const mpb_plan* plan) {
  const size_t bytes = (size_t)plan->prob.heads_q * plan->prob.total_q * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

size_t flex_attn_bwd_workspace_size(const mpb_plan* plan) {
  if (!plan) return 0;
  return 2 * bwd_vec_bytes(plan);
}

static mpb_status bwd_common(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                             const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, float scale,
                             const mpb_score_mod* mod, void* workspace, size_t workspace_bytes,
                             void* stream, int32_t ablate) {
  if (!plan) return fail(MPB_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!problem) return fail(MPB_ERR_INVALID_ARGUMENT, "problem is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(MPB_ERR_SIGNATURE_MISMATCH, "plan built on device %d used on device %d",
                plan->device, dev);
  const mpb_problem& a = *problem;
  const mpb_problem& b = plan->prob;
#define MPB_CMP(f)                                                                           \
  if (a.f != b.f)                                                                            \
    return fail(MPB_ERR_SIGNATURE_MISMATCH, "field " #f ": call has %d, plan has %d", a.f, b.f);
  MPB_CMP(layout) MPB_CMP(dtype) MPB_CMP(batch) MPB_CMP(seqlen_q) MPB_CMP(seqlen_k)
  MPB_CMP(total_q) MPB_CMP(total_k) MPB_CMP(heads_q) MPB_CMP(heads_k) MPB_CMP(head_dim)
  MPB_CMP(mask_heads) MPB_CMP(nfunc)
#undef MPB_CMP
  if ((a.tile_q && a.tile_q != b.tile_q) || (a.tile_k && a.tile_k != b.tile_k))
    return fail(MPB_ERR_SIGNATURE_MISMATCH, "tile %dx%d requested, plan has %dx%d", a.tile_q,
                a.tile_k, b.tile_q, b.tile_k);
  // §8: a training call needs a plan built with its backward view.
  if (!plan->has_k2q)
    return fail(MPB_ERR_INVALID_ARGUMENT, "the plan was built without the backward K2Q view");
  if (!attn_bwd_variant_exists(b.dtype, b.head_dim, b.tile_q, b.tile_k))
    return fail(MPB_ERR_UNSUPPORTED, "no gfx950 backward consumer for dtype %d, head_dim %d, "
                "tile %dx%d", b.dtype, b.head_dim, b.tile_q, b.tile_k);
  // tensors of an empty side are never touched (no Q rows: dK = dV = 0 only;
  // no keys: dQ = 0 only)
  if ((b.total_q > 0 && (!q || !o || !lse || !dout || !dq)) ||
      (b.total_k > 0 && (!k || !v || !dk || !dv)))
    return fail(MPB_ERR_INVALID_ARGUMENT, "q, k, v, o, lse, dout, dq, dk and dv must be non-NULL");
  if (workspace_bytes < flex_attn_bwd_workspace_size(plan) ||
      (flex_attn_bwd_workspace_size(plan) > 0 && !workspace))
    return fail(MPB_ERR_WORKSPACE, "workspace of %zu bytes needed",
                flex_attn_bwd_workspace_size(plan));
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(MPB_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  const int64_t qspan = ((int64_t)b.seqlen_q + b.tile_q) * b.heads_q * b.head_dim * 2;
  const int64_t kspan = ((int64_t)b.seqlen_k + b.tile_k) * b.heads_k * b.head_dim * 2;
  if (qspan >= ((int64_t)1 << 31) || kspan >= ((int64_t)1 << 31))
    return fail(MPB_ERR_UNSUPPORTED, "one sample spans >= 2 GiB of Q/K/V; not supported");
  const bool sc = mod && mod->softcap_enabled;
  const bool al = mod && mod->alibi_enabled;
  if (sc && !(std::isfinite(mod->softcap) && mod->softcap > 0.0f))
    return fail(MPB_ERR_INVALID_ARGUMENT, "softcap must be finite and > 0");
  if (al && !mod->alibi_slopes) return fail(MPB_ERR_INVALID_ARGUMENT, "alibi_slopes is NULL");
  int32_t kind = kModNone;
  if (sc && al) kind = mod->alibi_before_softcap ? kModAlibiSoftcap : kModSoftcapAlibi;
  else if (sc) kind = kModSoftcap;
  else if (al) kind = kModAlibi;

  BwdParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.dout = dout;
  prm.dq = dq;
  prm.dk = dk;
  prm.dv = dv;
  prm.lse = lse;
  prm.dvec = static_cast<float*>(workspace);
  prm.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_vec_bytes(plan));
  prm.seqdesc = plan->dev.seqdesc;
  prm.task_rec = plan->dev.task_rec;
  prm.p_idx = plan->dev.p_idx;
  prm.f_idx = plan->dev.f_idx;
  prm.p_masks = plan->dev.p_masks;
  prm.k_cu = plan->kdev.cu_krows;
  prm.k_p_off = plan->kdev.p_off;
  prm.k_f_off = plan->kdev.f_off;
  prm.k_p_idx = plan->kdev.p_idx;
  prm.k_f_idx = plan->kdev.f_idx;
  prm.k_masks = plan->kdev.p_masks;
  prm.k_order = plan->kdev.order;
  prm.slopes = al ? mod->alibi_slopes : nullptr;
  prm.batch = b.batch;
  prm.heads_q = b.heads_q;
  prm.heads_k = b.heads_k;
  prm.group = b.heads_q / b.heads_k;
  prm.mask_heads = b.mask_heads;
  prm.total_q = b.total_q;
  prm.krows_total = (int32_t)plan->header[4];
  prm.scale = scale;
  const float log2e = 1.4426950408889634f;
  prm.scale_log2 = scale * log2e;
  prm.softcap_k = sc ? 2.0f * scale * log2e / mod->softcap : 0.0f;
  prm.softcap_c2 = sc ? mod->softcap * log2e : 0.0f;
  prm.alibi_k = sc ? 2.0f * log2e / mod->softcap : 0.0f;
  prm.no_skip = (ablate & MPB_ABLATE_NO_SKIP) ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((e = launch_attn_bwd(b.head_dim, b.tile_q, b.tile_k, kind, plan->num_tasks, prm, s)) !=
      hipSuccess)
    return device_status(e, "backward launch");
  return ok();
}

mpb_status flex_attn_bwd(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                         const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float scale,
                         const mpb_score_mod* mod, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return bwd_common(plan, problem, q, k, v, o, lse, dout, dq, dk, dv, scale, mod, workspace,
                    workspace_bytes, stream, 0);
}

mpb_status flex_attn_bwd_ablation(const mpb_plan* plan, const mpb_problem* problem,
                                  const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk,
                                  void* dv, float scale, const mpb_score_mod* mod,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  int32_t flags) {
  if (flags & ~MPB_ABLATE_NO_SKIP)
    return fail(MPB_ERR_INVALID_ARGUMENT, "backward ablation flags must be 0 or %d",
                MPB_ABLATE_NO_SKIP);
  return bwd_common(plan, problem, q, k, v, o, lse, dout, dq, dk, dv, scale, mod, workspace,
                    workspace_bytes, stream, flags);
}

mpb_status flex_attn_fwd(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                         const void* k, const void* v, void* o, float* lse, float scale,
                         const mpb_score_mod* mod, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return attn_common(plan, problem, q, k, v, o, lse, scale, mod, workspace, workspace_bytes,
                     stream, 0, 1);
}

mpb_status flex_attn_fwd_ablation(const mpb_plan* plan, const mpb_problem* problem,
                                  const void* q, const void* k, const void* v, void* o,
                                  float* lse, float scale, const mpb_score_mod* mod,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  int32_t flags) {
  if (flags & ~(MPB_ABLATE_FULL_AS_PARTIAL | MPB_ABLATE_NO_SKIP))
    return fail(MPB_ERR_INVALID_ARGUMENT, "unknown ablation flags 0x%x", flags);
  return attn_common(plan, problem, q, k, v, o, lse, scale, mod, workspace, workspace_bytes,
                     stream, flags, 1);
}

}  // extern "C"
