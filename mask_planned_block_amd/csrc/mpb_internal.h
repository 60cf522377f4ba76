// Internal declarations shared by the host runtime and the HIP kernels of
// libmpb.  Nothing here is part of the public ABI (include/mpb.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpb {

// Forward schedule: positive-cost tasks are split into kNumSections sections,
// one per XCD of the MI355X (8 XCDs, each with its own L2).  Tasks of one
// (batch, K/V head) pair share a section.  Workgroups are handed to the XCDs
// round-robin in launch order, so the launch order interleaves the sections
// (launch slot 8r+x holds the r-th task of section x while every section still
// has tasks): each XCD then runs one section's tasks in descending cost and
// keeps that section's K/V in its L2.  This is this library's reading of the
// "L2 section" of the mask plan design page, §4.8.  Zero-cost tasks (rows
// with nothing visible) come last.
constexpr int kNumSections = 8;
constexpr int kNumQueues = kNumSections + 1;

// One 64-byte record per forward task, in launch order: workgroup i runs
// record i.  Fields (int32):
enum TaskRecField {
  kRecMBlock = 0, kRecHead, kRecBatch, kRecQValid,
  kRecQOff, kRecKOff, kRecQLen, kRecKLen,
  kRecPBeg, kRecPCnt, kRecFBeg, kRecFCnt,
  kRecFirstTile,   // K tile of the first listed block, -1 if none
  kRecMaskHead, kRecKvHead, kRecSection,
  kTaskRecInts
};

// Planner geometry, passed by value to every planner kernel.
struct PlanGeo {
  int32_t layout;       // 0 BSHD, 1 THD
  int32_t batch;
  int32_t seqlen_q, seqlen_k;   // BSHD: Sq, Sk ; THD: max lengths
  int32_t total_q, total_k;
  int32_t heads_q, heads_k, mask_heads, nfunc;
  int32_t tile_q, tile_k;
  int32_t upper_rows;   // upper bound of Q plan rows (exact for BSHD)
  int32_t nk_max;       // upper bound of K tiles per sample
  int32_t words_k;      // ceil(nk_max / 32): bitset words per (hm, row)
  int32_t words_tile;   // tile_k / 32: payload words per tile row
};

// Device arrays of a plan.
struct PlanDev {
  int32_t* header;       // [8]
  int32_t* seqdesc;      // [B][8]
  int32_t* cu_rows;      // [B+1]
  int32_t* cu_q;         // [B+1] clone (THD) or nullptr
  int32_t* cu_k;
  int32_t* work_desc;    // [upper_rows*Hq][4] section-major schedule
  int32_t* section_off;  // [kNumQueues+1]
  int32_t* task_rec;     // [upper_rows*Hq][kTaskRecInts] launch order (sections interleaved)
  int32_t* p_off;        // [Hmask*rows+1]
  int32_t* f_off;
  int32_t* p_idx;
  int32_t* f_idx;
  uint32_t* p_masks;
};

// Build-time workspace (freed when the build finishes).
struct PlanWork {
  uint32_t* vis_bits;    // [Hmask][upper_rows][words_k]
  uint32_t* full_bits;
  int32_t* pcnt;         // [Hmask][upper_rows]
  int32_t* fcnt;
  int32_t* first_tile;   // [Hmask][upper_rows] first listed K tile (partial list first), -1 if none
  int32_t* p_off_tmp;    // [Hmask*upper_rows+1] (compact head-major order)
  int32_t* f_off_tmp;
  int32_t* item_err;     // [Hmask][upper_rows] endpoint error bits per classified row
  int32_t* geo_err;      // [1] cu_seqlens error bit (THD)
  int32_t* lrank;        // [Hmask*upper_rows] rank among equal costs within its 64-row chunk
  int32_t* order;        // [Hmask*upper_rows] rows sorted by descending cost
  int32_t* row_base;     // [Hmask*upper_rows][kNumQueues] first in-section position of each row's tasks
  int32_t* chunk_cnt;    // [nk_max+1][nchunks] counts, then first positions (when not in LDS)
  int32_t nchunks;       // ceil(Hmask*upper_rows / 64)
};

// Longest sample the planner handles, in K tiles: bounds the cost range of
// the schedule's counting sort.
constexpr int kMaxKTiles = 8191;

// Host-mapped slot the classify kernel publishes the header into: values
// [0, 8) and, last, the build's sequence number at kHeaderSeq.
constexpr int kHeaderSeq = 8;
constexpr int kHostSlotInts = 16;

// Backward K2Q view: plan arrays and build workspace.
struct K2QDev {
  int32_t* cu_krows;   // [B+1] K plan rows per sample, prefix
  int32_t* p_off;      // [Hmask*krows+1]
  int32_t* f_off;
  int32_t* p_idx;      // sample-local Q tiles, ascending per K row
  int32_t* f_idx;
  uint32_t* p_masks;   // [pnnz][tile_k][tile_q/32]
  int32_t* order;      // [krows] K rows by descending cost over mask heads (launch order)
};
struct K2QWork {
  int32_t* pcnt;       // [Hmask][B][nk_max] (padded by sample)
  int32_t* fcnt;
  int32_t* cu_krows;   // [B+1]
  int32_t* p_off;      // [Hmask*B*nk_max+1] compact exclusive offsets
  int32_t* f_off;
  int32_t* info;       // [4]: K rows total, partial nnz, full nnz, 0
  int32_t* order;      // [B*nk_max] launch order staged for the plan
  int32_t max_cost;    // upper bound of a K row's cost (mask heads x Q tiles of a sample)
};
// Costs up to this bound are sorted in LDS; above it the K rows keep their
// natural order (any permutation is a valid launch order).
constexpr int kK2QOrderBuckets = 4096;
constexpr int kHeaderSeq2 = 9;   // host slot index of the K2Q header's sequence number

// ---- planner launchers (plan_kernels.hip) ----
hipError_t launch_plan_geometry(const PlanGeo& g, const int32_t* cu_q_in, const int32_t* cu_k_in,
                                const PlanDev& d, const PlanWork& w, hipStream_t s);
// `arrive` is a device counter that is 0 on entry and left 0 on exit; the last
// workgroup to finish computes the offsets and publishes the header (with
// `seq`) to `host_slot` (host-mapped).
hipError_t launch_plan_classify(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                                const PlanWork& w, int32_t* arrive, int32_t* host_slot,
                                int32_t seq, hipStream_t s);
hipError_t launch_plan_schedule(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                hipStream_t s);
// Segments of plan metadata copied from the staging arrays into the plan
// block by the materialize launch: segment i covers flat elements
// [end[i-1], end[i]).
struct MetaCopy {
  const int32_t* src[8];
  int32_t* dst[8];
  int64_t end[8];
  int64_t total;
};
hipError_t launch_plan_materialize(const PlanGeo& g, const int32_t* mask_func, const PlanDev& st,
                                   const PlanDev& d, const PlanWork& w, int32_t rows_total,
                                   hipStream_t s);

// In-place builds: the schedule and the rows' lists and payload in one launch
// on the plan block itself (rows_total < 0: read from the device header).
hipError_t launch_plan_finish(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                              const PlanWork& w, int32_t rows_total, hipStream_t s);
// Whether that launch's LDS fits (count matrix in LDS or not, its chunks).
bool plan_finish_fits(const PlanGeo& g, bool cnt_in_lds, int64_t nchunks);

// Single-pass builds (forward plans whose block at the upper bound of every
// count fits the library's cap): classification, offsets by decoupled
// look-back, lists and payload in one launch, then the schedule and the
// placement of the lists in a second one.
struct SinglePass {
  uint64_t* lb;          // [Hmask * upper_rows][kLbWords] look-back words {aggregate,
                         // inclusive partial, inclusive full, done}, each (tag << 32) | value
  uint32_t tag;          // this build's tag (nonzero; words of earlier builds differ)
  int32_t* host_slot;    // host-mapped header slot
  int32_t deferred;      // 1: deferred read-back: the header goes to the plan block only,
                         // after the last item's own lists and payload
  int32_t seq;           // the build's sequence number (published last)
  int32_t* p_list;       // [Hmask * upper_rows * nk_max] partial lists, flat CSR order
                         // (workspace, or the plan block's own lists when deferred)
  int32_t* f_list;       // full lists
  int32_t stage;         // endpoints: 0 read from HBM; staged in LDS as int32 (1 through
                         // registers, 2 loaded straight into LDS) or int16 (3)
  int32_t fused;         // 1 (deferred builds of at most kFusedMaxItems upper-bound items):
                         // every item also ranks its row and writes its tasks, and there is
                         // no tail launch
};
// Look-back words per item.
constexpr int kLbWords = 8;
// Largest Hmask * upper_rows for which a deferred single-pass build also runs
// the schedule: every item reads every item's cost, so all of them must be
// resident at once, and each item's ranking pass grows with their number.
constexpr int kFusedMaxItems = 256;
// Row keys of that schedule: a row's tasks per queue depend on its key alone
// (16 layouts of a sample's KV heads over the sections, and empty rows).
constexpr int kKeys = 17;
// Longest sample (seqlen_k) whose endpoints a single-pass build stages as
// int16: every column it compares, up to seqlen_k plus a tile and a word,
// stays below the int16 sentinel 32767.
constexpr int kShortEpMaxLen = 32000;
// Header error bit of a single-pass build whose look-back wait ran out.
constexpr uint32_t kDevErrLookback = 1u << 8;
// rows_total < 0: THD, rows counted on the device (the grid covers the upper
// bound).
hipError_t launch_plan_single_pass(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                                   const PlanWork& w, const SinglePass& sp, int32_t rows_total,
                                   hipStream_t s);
// place_lists: copy the lists from the workspace behind the payload (exact
// layout); false when the single pass wrote them into the block itself.
hipError_t launch_plan_single_pass_tail(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                        const SinglePass& sp, int64_t tiles_upper,
                                        bool place_lists, hipStream_t s);

// Backward K2Q view (same tile geometry as the forward plan): count from the
// classifier's bitsets, then (last workgroup) offsets and header values 3..6
// published with `seq` at kHeaderSeq2; materialize lists and K-major payload
// (the transpose of the Q2K payload: d is the finished forward plan).
hipError_t launch_plan_k2q_count(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                 const K2QWork& kw, int32_t* arrive, int32_t* host_slot,
                                 int32_t seq, hipStream_t s);
// krows_total < 0: read from kw.info (launch before the header is back).
hipError_t launch_plan_k2q_materialize(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                       const K2QWork& kw, const K2QDev& kd, int32_t krows_total,
                                       hipStream_t s);

// ---- attention ----
enum ModKind : int32_t {
  kModNone = 0,
  kModSoftcap = 1,
  kModAlibi = 2,
  kModSoftcapAlibi = 3,   // softcap, then ALiBi
  kModAlibiSoftcap = 4,   // ALiBi, then softcap
};

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seqdesc;
  const int32_t* cu_rows;
  const int32_t* p_off;
  const int32_t* p_idx;
  const int32_t* f_off;
  const int32_t* f_idx;
  const uint32_t* p_masks;
  const int32_t* task_rec;  // [num_tasks][kTaskRecInts]
  const float* slopes;
  int32_t heads_q, heads_k, group, mask_heads, rows_total, total_q;
  int32_t force_partial;     // full tiles through the predicate path (ablation)
  int32_t no_skip;           // compute tiles and blocks whose weights are all exactly 0 (ablation)
  // PackGQA: a task's tile row r is token r >> pack_shift of its plan row and
  // Q head (task head) * 2^pack_shift + (r & (2^pack_shift - 1)); 0 = unpacked
  // (the task head is then the Q head).
  int32_t pack_shift;
  // A plan whose header the host has not read (deferred build): the launch
  // covers the upper bound of tasks and workgroup i runs only while
  // i < dev_header[0] * task_heads and dev_header[7] (device error bits) is
  // 0.  nullptr: the launch covers exactly the plan's tasks.
  const int32_t* dev_header;
  int32_t task_heads;
  // Softcap score_mods: full tiles take the reference max from the closed-form
  // bound of their scores (c plus the tile's largest ALiBi bias) instead of the
  // scores' maximum; set when 2c*log2(e) plus the rescale slack stays under
  // 100, so weights within 2c of the bound stay normal floats.
  int32_t cap_bounded;
  float scale_log2;         // scale * log2(e)
  float softcap_k;          // 2*scale*log2(e)/c  (exp2 argument factor of tanh)
  float softcap_c2;         // c * log2(e)
  float alibi_k;            // ALiBi-first: 2*log2(e)/c multiplier of slope*(k-q)
  // Split-K (launch_attn_fwd_split only): workgroup i runs split i / tasks_padded
  // of task i % tasks_padded; split s covers positions [s*n/S, (s+1)*n/S) of
  // the task's tile list (partial tiles, then full tiles, n of them) and
  // writes O normalized over those tiles into o_part [S][total_q][heads_q][D]
  // (fp32) and its LSE into lse_part [S][heads_q][total_q].
  int32_t num_tasks, num_splits, tasks_padded;
  float* o_part;
  float* lse_part;
  // Paged K/V: k and v are pools of token rows ([pool rows][heads_k][D]);
  // phys_p / phys_f hold, beside p_idx / f_idx, the pool tile (tile_k rows)
  // of every listed K tile, -1 for an entry whose page is out of range.
  int32_t paged;
  const int32_t* phys_p;
  const int32_t* phys_f;
};

// Page remap of a plan's K-tile lists (the forward's paged mode).
struct RemapParams {
  const int32_t* cu_rows;    // [batch+1]
  const int32_t* p_off;      // [rows_flat+1]
  const int32_t* f_off;
  const int32_t* p_idx;
  const int32_t* f_idx;
  const int32_t* page_table; // [batch][pages_per_seq]
  int32_t* phys_p;
  int32_t* phys_f;
  int32_t rows_total, rows_flat, batch, tile_k, page_size, pages_per_seq, num_pages;
};

// Merge of Split-K partial states into O (input dtype) and LSE.
struct MergeParams {
  const float* o_part;       // [parts][rows][D], rows = total_q * heads_q (token-major)
  const float* lse_part;     // [parts][heads_q][total_q]
  void* o;                   // [rows][D]
  float* lse;                // [heads_q][total_q]
  int64_t rows;
  int32_t parts, heads_q, total_q;
};

// Backward: Q2K launch records and payload (dQ), K2Q lists and payload
// (dK, dV), the forward's O and LSE, the incoming dO and a Dq workspace.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const float* lse;          // [heads_q][total_q], natural log
  float* dvec;               // workspace [heads_q][total_q]: -(dO . O) per row
  float* lse2;               // workspace [heads_q][total_q]: LSE in log2 units, +inf if empty
  const int32_t* seqdesc;
  const int32_t* task_rec;
  const int32_t* p_idx;
  const int32_t* f_idx;
  const uint32_t* p_masks;
  const int32_t* k_cu;       // K2Q: cu_krows [batch+1]
  const int32_t* k_p_off;
  const int32_t* k_f_off;
  const int32_t* k_p_idx;
  const int32_t* k_f_idx;
  const uint32_t* k_masks;
  const int32_t* k_order;    // K2Q launch order of the K rows
  const float* slopes;
  int32_t batch, heads_q, heads_k, group, mask_heads, total_q, krows_total;
  float scale;
  float scale_log2, softcap_k, softcap_c2, alibi_k;   // as in AttnParams
  int32_t no_skip;           // compute blocks whose weights are all exactly 0 (ablation)
};

bool attn_bwd_variant_exists(int32_t dtype, int32_t head_dim, int32_t tile_q, int32_t tile_k);
hipError_t launch_attn_bwd(int32_t head_dim, int32_t tile_q, int32_t tile_k, int32_t mod_kind,
                           int32_t num_tasks, const BwdParams& p, hipStream_t s);

// Attention kernel variants known to this build (the consumers a plan can be
// resolved to).  Returns false if (dtype, head_dim, tile_q, tile_k) has none.
bool attn_variant_exists(int32_t dtype, int32_t head_dim, int32_t tile_q, int32_t tile_k);
hipError_t launch_attn_fwd(int32_t dtype, int32_t head_dim, int32_t tile_q, int32_t tile_k,
                           int32_t mod_kind, int32_t num_tasks, const AttnParams& p,
                           hipStream_t s);
// Split-K forward: p.num_splits * p.tasks_padded workgroups writing partial
// states (p.o_part, p.lse_part); the merge follows with launch_attn_merge.
hipError_t launch_attn_fwd_split(int32_t dtype, int32_t head_dim, int32_t tile_q, int32_t tile_k,
                                 int32_t mod_kind, const AttnParams& p, hipStream_t s);
// Physical pool tiles of every listed K tile (one wavefront per flat row).
hipError_t launch_page_remap(const RemapParams& p, hipStream_t s);
// Merge kernel for head_dim 64 or 128, output bf16 (dtype 0) or fp32 (1).
hipError_t launch_attn_merge(int32_t dtype, int32_t head_dim, const MergeParams& p,
                             hipStream_t s);

}  // namespace mpb
