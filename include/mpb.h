/*
 * mpb.h -- C ABI of the interval-mask flex attention library (libmpb.so).
 *
 * Two operations, both hand-written HIP kernels for gfx950 (MI355X):
 *
 *   mask_plan_build  turns per-Q-row interval endpoints into a MaskPlan: per
 *                    (mask head, Q tile) the K tiles classed partial or full
 *                    (empty tiles are absent), a packed predicate for every
 *                    partial tile, and a forward task schedule.
 *   flex_attn_fwd    consumes a plan: S = Q K^T * scale, optional score_mod
 *                    (tanh softcap, ALiBi), online softmax over the listed K
 *                    tiles, O = P V and a per-row log-sum-exp.
 *
 * Sources (cited by page title and section):
 *   [MPD]  "Flex Attention Mask Plan Design", cuDNN frontend documentation.
 *   [FLEX] "FlexAttention" (Dong et al.), Eq. 1 and the BlockMask section.
 *   [TESS] "Decoupling Logical Masks from GPU Execution for Dynamic
 *          Block-Sparse Attention" (Tessera), physical tile vs logical block.
 *   [PYG]  cuDNN "pygraph and execution backends" page, sections "Handle,
 *          stream, and device" and "Accept means run".
 *
 * Conventions for every entry point:
 *   - Every call returns an mpb_status; nothing throws across the ABI.  On
 *     failure mpb_last_error_detail() (thread-local) names the violated rule.
 *   - Device pointers are plain HIP device addresses (e.g. torch tensor
 *     data_ptr()).  `stream` is a hipStream_t passed as void*; NULL is the
 *     null stream.  There is no ambient stream or device state [PYG].
 *   - The caller owns every buffer it passes in; the plan owns every array it
 *     creates (including device copies of cu_seqlens) [MPD §3.2, §8].
 */
#ifndef MPB_H_
#define MPB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MPB_OK = 0,
  MPB_ERR_INVALID_ARGUMENT = 1,   /* host-decidable shape/pointer/enum error */
  MPB_ERR_ENDPOINT_RANGE = 2,     /* an endpoint < 0 or > its sample's k_len [MPD §2, §4.3] */
  MPB_ERR_ENDPOINT_ORDER = 3,     /* F(i) > F(i+1) for some row [MPD §2, §4.3] */
  MPB_ERR_SEQLENS = 4,            /* cu_seqlens not 0..total, decreasing, or > max_seqlen [MPD §3.2] */
  MPB_ERR_SIGNATURE_MISMATCH = 5, /* plan used with another geometry/consumer/device [MPD §7] */
  MPB_ERR_WORKSPACE = 6,          /* workspace missing or too small */
  MPB_ERR_UNSUPPORTED = 7,        /* legal but not implemented (head_dim, tile, nfunc > 4095) */
  MPB_ERR_OUT_OF_MEMORY = 8,
  MPB_ERR_DEVICE = 9              /* a HIP runtime call failed */
} mpb_status;

enum { MPB_LAYOUT_BSHD = 0, MPB_LAYOUT_THD = 1 };
enum { MPB_DTYPE_BF16 = 0, MPB_DTYPE_FP32 = 1 };

/* Device error bits, OR-ed into header[7] by the planner kernels. */
enum { MPB_DEVERR_SEQLENS = 1, MPB_DEVERR_RANGE = 2, MPB_DEVERR_ORDER = 4 };

/* Problem geometry = the plan binding [MPD §8].
 *   BSHD: Q is [batch, seqlen_q, heads_q, head_dim], K/V [batch, seqlen_k,
 *         heads_k, head_dim], contiguous; total_q = batch*seqlen_q,
 *         total_k = batch*seqlen_k.
 *   THD : Q is [total_q, heads_q, head_dim], K/V [total_k, heads_k, head_dim];
 *         seqlen_q/seqlen_k are max_seqlen_q/k; sample b owns tokens
 *         [cu_seqlens[b], cu_seqlens[b+1]).
 *   mask_heads (Hmask) is 1 (one mask shared by all Q heads) or heads_q
 *   [MPD §2].  nfunc is odd, 1 <= nfunc <= 4095.  heads_q % heads_k == 0; the
 *   K/V head of Q head h is h / (heads_q / heads_k).  tile_q/tile_k are the
 *   physical tile, chosen independently of any logical block size [TESS
 *   "logical blocks and physical tiles"].  0 = the library's choice: tile_q
 *   128 (bf16) or 64 (fp32); tile_k for bf16 head_dim 128 with 128-row
 *   tiles is 32 when the plan has at least 3 tasks (Q tiles x heads_q; THD:
 *   total_q/128 rows) per compute unit of the current device and is built
 *   without the backward view, else 64 (the 32-wide forward kernel keeps
 *   three workgroups per CU and executes fewer masked entries, the 64-wide
 *   one is faster per workgroup, and the backward's dK/dV consumer reads
 *   every Q and dO tile once per K tile); otherwise 64 (fp32 head_dim 128:
 *   32).  mask_plan_info reports the resolved tile. */
typedef struct mpb_problem {
  int32_t layout;
  int32_t dtype;
  int32_t batch;
  int32_t seqlen_q, seqlen_k;
  int32_t total_q, total_k;
  int32_t heads_q, heads_k, head_dim;
  int32_t mask_heads, nfunc;
  int32_t tile_q, tile_k;
} mpb_problem;

typedef struct mpb_plan mpb_plan; /* opaque, immutable after build [MPD §8] */

/* Consumer signature recorded in a plan and compared field by field before
 * every launch; a mismatch is an error, never a fallback [MPD §7, §9.9]. */
typedef struct mpb_signature {
  int32_t arch;            /* 950 = gfx950 */
  int32_t direction;       /* 0 = forward */
  int32_t kernel_family;   /* 1 = bf16 MFMA 32x32x16, 2 = fp32 MFMA 32x32x2 */
  int32_t tile_q, tile_k, head_dim, dtype;
  int32_t payload_layout;  /* 1 = row-major, 32-column uint32 words (see below) */
  int32_t scheduler;       /* 2 = one workgroup per task, section-interleaved launch order */
  int32_t pack_gqa;        /* Q heads per plan row in the consumer tile: 1, or heads_q/heads_k
                            * when the plan is packed (PackGQA, see mpb_build_options) */
} mpb_signature;

typedef struct mpb_plan_info {
  int64_t header[8];       /* fwd Q rows, fwd partial nnz, fwd full nnz, then (K2Q view only,
                            * else 0) Q rows, K rows, K2Q partial nnz, K2Q full nnz; error bits */
  int32_t rows_total;      /* Q plan rows over all samples */
  int32_t nk_max;          /* K tiles of the longest sample */
  int32_t words_per_row;   /* tile_k / 32 */
  int32_t num_tasks;       /* rows_total * heads_q (packed: rows_total * heads_k) */
  int32_t num_sections;    /* schedule sections (8 XCD sections + the zero-cost tail) */
  int32_t device;
  mpb_problem problem;
  mpb_signature signature;
  int64_t device_bytes;    /* bytes of device memory the plan holds */
  int32_t build_mode;      /* how the plan was built: MPB_BUILD_EXACT (header read back, then the
                            * exact block and the materialisation), MPB_BUILD_IN_PLACE (small
                            * plans: the upper-bound block, schedule and materialisation in one
                            * launch) or MPB_BUILD_SINGLE_PASS (forward plans: one pass over the
                            * endpoints, block cut to its exact size after the header) */
  int32_t reserved;
} mpb_plan_info;
enum {
  MPB_BUILD_EXACT = 0,
  MPB_BUILD_IN_PLACE = 1,
  MPB_BUILD_SINGLE_PASS = 2,
  MPB_BUILD_SINGLE_PASS_DEFERRED = 3   /* single pass, header read lazily (defer_header) */
};

/* score_mod of [FLEX] Eq. 1, applied to t = scale * (q . k):
 *   softcap:  t <- softcap * tanh(t / softcap)
 *   ALiBi:    t <- t + alibi_slopes[h] * (k - q), sample-local positions
 * Default order is softcap, then ALiBi; alibi_before_softcap = 1 swaps it.
 * alibi_slopes is a device float array [heads_q]. */
typedef struct mpb_score_mod {
  int32_t softcap_enabled;
  float softcap;
  int32_t alibi_enabled;
  const float* alibi_slopes;
  int32_t alibi_before_softcap;
} mpb_score_mod;

/* mask_plan_build [MPD §4]: host structural validation and consumer
 * resolution (§4.1), then GPU stages: Varlen geometry (§4.2), Q2K
 * classification with endpoint validation (§4.3), count scan and header
 * (§4.5), the forward schedule (§4.8), one 8-value header read-back (the
 * call waits on the host until the header has landed in host-mapped memory,
 * not for the stream to drain), allocation, and Q2K materialisation of the
 * partial/full CSR and the packed predicates (§4.6, §5).  Three build
 * modes (mask_plan_info's build_mode):
 *   single pass  forward plans (no backward view) whose block at the upper
 *                bound of every count, with the list workspace, is at most
 *                2 GiB: that block is allocated before the launches; one
 *                launch classifies every (mask head, Q row), takes its CSR
 *                offsets by decoupled look-back and writes its lists and
 *                payload (the endpoints are read once), a second runs the
 *                schedule and places the lists; after the header the block is
 *                cut to its exact size (nothing padded is kept).
 *   in place     backward plans whose upper-bound block is at most 32 MiB:
 *                that block is allocated first and kept; schedule and
 *                materialisation run in one launch.
 *   exact        the rest: the block is allocated after the header, sized by
 *                it, and the materialisation runs after that.
 *
 *   mask_func    device int32 [mask_heads][nfunc][total_q]; column t holds the
 *                endpoints F0..F(nfunc-1) of Q token t, sample-local K
 *                positions; row t sees [0,F0) U [F1,F2) U ... [MPD §2].
 *                Work enqueued on `stream` still reads it after the call
 *                returns: release it in stream order (as torch's caching
 *                allocator does) or after synchronising the stream.
 *   cu_seqlens_q/k  device int32 [batch+1] for THD; ignored (may be NULL) for
 *                BSHD.  Validated on the GPU [MPD §3.2].  Same lifetime rule.
 *   stream       work is enqueued here.  The plan's arrays are complete in
 *                this stream's order: a forward on another stream must be
 *                ordered after it (event or synchronisation).  Builds of one
 *                host thread share a device workspace; a build on a stream
 *                other than the previous build's first waits for that stream.
 *   out          receives the plan, or NULL on any failure (nothing leaks).
 * Errors: host-decidable problems return MPB_ERR_INVALID_ARGUMENT or
 * MPB_ERR_UNSUPPORTED before any launch; endpoint and prefix violations found
 * on the GPU return MPB_ERR_SEQLENS, then MPB_ERR_ENDPOINT_RANGE, then
 * MPB_ERR_ENDPOINT_ORDER (first set bit in that order).
 *
 * Plan layout (device, read with mask_plan_export):
 *   rows are Q tiles of T_Q tokens per sample (a packed plan: T_Q/G tokens,
 *   G = signature.pack_gqa; see mpb_build_options); row r of sample b is global row
 *   cu_rows[b] + r; CSR rows are flattened head-major, flat = hm*rows_total +
 *   row.  p_off/f_off [mask_heads*rows_total + 1] are exclusive offsets into
 *   p_idx/f_idx (sample-local K-tile indices, ascending).  Partial tile n
 *   owns payload words p_masks[n][T_Q/G][tile_k/32]: bit c%32 of word
 *   [r][c/32] is 1 iff score (row r, column c) of the tile is visible and in
 *   bounds [MPD §5].  In the attention kernel each lane owns one Q row and 16
 *   K columns of every 32-column block, all in one such word, so it reads its
 *   predicate with a single dword load (the packed-bit select of [MPD §5.1]). */
mpb_status mask_plan_build(const mpb_problem* problem, const int32_t* mask_func,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           void* stream, mpb_plan** out);

/* Releases the plan's device memory in stream order on its build stream.
 * The caller must order every use of the plan on other streams before this
 * call (e.g. synchronise them).  NULL is accepted. */
mpb_status mask_plan_destroy(mpb_plan* plan);

/* Header, geometry and signature of a plan (host struct).  No device access,
 * except for a plan built with defer_header whose header has not been read
 * yet: the call then waits for the build stream, reads the header and returns
 * the build's error (MPB_ERR_SEQLENS, MPB_ERR_ENDPOINT_RANGE, ...) if the
 * GPU checks failed, else fills *info. */
mpb_status mask_plan_info(const mpb_plan* plan, mpb_plan_info* info);

/* Copies plan arrays to host memory [MPD §8 debug_snapshot]; any pointer may
 * be NULL.  Sizes: cu_rows [batch+1], seqdesc [batch][8] = {q_offset,
 * k_offset, q_len, k_len, row_begin, row_count, k_tiles, 0}, p_off/f_off
 * [mask_heads*rows_total+1], p_idx [header[1]], f_idx [header[2]], p_masks
 * [header[1]*(tile_q/pack_gqa)*tile_k/32], work_desc [num_tasks][4] =
 * {m_block, head, batch, q_valid_rows} in schedule order (a packed plan's
 * tasks are (row, K/V head): head is the K/V head and q_valid_rows counts
 * tokens of the row), section_off [num_sections+1].
 * Synchronises the plan's build stream. */
mpb_status mask_plan_export(const mpb_plan* plan, int32_t* cu_rows, int32_t* seqdesc,
                            int32_t* p_off, int32_t* p_idx, uint32_t* p_masks, int32_t* f_off,
                            int32_t* f_idx, int32_t* work_desc, int32_t* section_off);

/* Launch order of the forward tasks: records [num_tasks][16] int32, record i
 * run by workgroup i: {m_block, head, batch, q_valid_rows, q_offset, k_offset,
 * q_len, k_len, partial_begin, partial_count, full_begin, full_count,
 * first_k_tile (-1 if none), mask_head, kv_head, section}.  The order
 * interleaves the schedule's sections (one per XCD): while every section has
 * tasks left, slot 8r+x holds the r-th task of section x [MPD §4.8, read for
 * MI355X's round-robin workgroup-to-XCD dispatch].  Synchronises the plan's
 * build stream. */
mpb_status mask_plan_export_launch_order(const mpb_plan* plan, int32_t* records);

/* Build options.  build_backward = 1 adds the backward K2Q view [MPD §4.4
 * K2Q counting, §4.7 K2Q materialization] at the plan's own tile geometry
 * (read from the forward classification; a different backward geometry is
 * not built).  For every mask head and K plan row (one T_KV tile of one
 * sample's K; K rows flattened head-major, flat = hm*krows_total + krow,
 * krow = cu_krows[b] + j) it holds the sample-local Q tiles whose pair with
 * that K tile is partial and, independently, full, each list ascending, and
 * for every partial pair a K-major predicate: word [r][c/32], bit c%32, is 1
 * iff score (Q row c, K row r) of the pair is in bounds and visible
 * (consumer layout chosen for a K-major backward: one word row per K row).
 * The header then also holds {Q rows, K rows, K2Q partial nnz, K2Q full nnz}
 * in slots 3..6, read back like the forward values.  NULL options = all
 * zero. */
typedef struct {
  int32_t build_backward;  /* 0 or 1: also build the K2Q view */
  int32_t time_stages;     /* 0 or 1: record HIP events around each planner launch
                            * (mask_plan_stage_times); adds event records to the
                            * build stream, for measurement only */
  int32_t pack_gqa;        /* PackGQA [MPD §4.1 consumer resolution, §6.2]: 0 = the
                            * library's choice, 1 = off, 2 = on.  A packed forward tile
                            * holds T_Q/G tokens x the G = heads_q/heads_k Q heads that
                            * share one K/V head (tile row r: token r/G of the row, Q
                            * head G*kv_head + r%G), so one K/V tile load serves all G
                            * heads and the payload keeps one word row per token (T_Q/G
                            * payload rows: the same block relation and predicate as an
                            * unpacked plan with T_Q/G-token rows).  Needs mask_heads = 1
                            * (every Q head of a group sees the same mask), G a power of
                            * two with T_Q/G >= 16, and no backward view; 2 with any of
                            * these unmet is MPB_ERR_UNSUPPORTED.  The library packs
                            * whenever it may (measured faster on every shape tried:
                            * short query chunks most, by filling the tile's rows). */
  int32_t defer_header;    /* 0 or 1.  1: a single-pass build returns as soon as its
                            * launches are enqueued, without the header read-back
                            * (and with at most 256 (mask head, Q row) items at the upper
                            * bound, the single pass also runs the schedule in the
                            * workgroup that publishes the header: one launch in all)
                            * (other builds ignore the flag and read it back as usual).
                            * The block keeps its upper-bound layout (the lists are
                            * written into it directly; nothing is cut off), and the
                            * endpoint / prefix checks done on the GPU are reported by
                            * the first call that reads the header: mask_plan_info, the
                            * exports, flex_attn_fwd_num_splits and the Split-K and
                            * paged forwards read it (waiting for the build stream) and
                            * return the build's error if it failed.  flex_attn_fwd and
                            * flex_attn_fwd_ablation do not wait: they launch the upper
                            * bound of workgroups, which read the task count and the
                            * error word on the device; on a plan that failed its checks
                            * they write nothing (O and LSE keep their contents). */
} mpb_build_options;

/* mask_plan_build with options; same arguments, errors and lifetime rules. */
mpb_status mask_plan_build_ex(const mpb_problem* problem, const mpb_build_options* options,
                              const int32_t* mask_func, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* stream, mpb_plan** out);

/* Copies the K2Q view to host memory; any pointer may be NULL.  Sizes:
 * cu_krows [batch+1], p_off/f_off [mask_heads*header[4]+1], p_idx
 * [header[5]], f_idx [header[6]], p_masks [header[5]*tile_k*tile_q/32].
 * MPB_ERR_INVALID_ARGUMENT if the plan was built without it.  Synchronises
 * the plan's build stream. */
mpb_status mask_plan_export_k2q(const mpb_plan* plan, int32_t* cu_krows, int32_t* p_off,
                                int32_t* p_idx, uint32_t* p_masks, int32_t* f_off,
                                int32_t* f_idx);

/* Copies the K2Q view's launch order to host memory: order[header[4]], the
 * K rows sorted by descending cost (partial + full Q tiles summed over mask
 * heads), ties by K row (the backward dK/dV consumer starts the heaviest K
 * rows first).  MPB_ERR_INVALID_ARGUMENT if the plan was built without the
 * view.  Synchronises the plan's build stream. */
mpb_status mask_plan_export_k2q_order(const mpb_plan* plan, int32_t* order);

/* GPU time of each planner stage of a build made with time_stages = 1, in
 * microseconds, from the HIP events around its launches [MPD §4.2-§4.7
 * stages]; us must hold 7 floats, -1 for a stage the build did not launch:
 * us[0] THD geometry (none for BSHD), us[1] classify (a single-pass build:
 * classification, offsets, lists and payload in one launch), us[2] schedule
 * (in place: schedule and materialization in one launch; single pass:
 * schedule and list placement; -1 for a deferred build of at most 256
 * (mask head, Q row) items, whose single pass also schedules: each item
 * ranks and writes its own row's tasks),
 * us[3] materialization (exact builds only),
 * us[4] K2Q count, us[5] K2Q materialization (backward view only), us[6]
 * first event to last (for an exact build this includes the host's header
 * wait).  Waits for the build's last event.
 * MPB_ERR_INVALID_ARGUMENT if the plan was built without time_stages. */
mpb_status mask_plan_stage_times(const mpb_plan* plan, float* us);

/* Bytes of caller-provided device workspace flex_attn_fwd needs.  The
 * forward launches one workgroup per task in the plan's launch order, so no
 * scheduler state is needed and this returns 0; the argument is kept for
 * consumers that need call-local state [MPD §4.8]. */
size_t flex_attn_fwd_workspace_size(const mpb_plan* plan);

/* flex_attn_fwd [MPD §6.1; FLEX Eq. 1]: block-sparse attention forward.
 *   problem   geometry of q/k/v/o as the caller sees it; must equal the plan's
 *             binding field by field (tile_q/tile_k may be 0) and the current
 *             device must be the plan's, else MPB_ERR_SIGNATURE_MISMATCH.
 *   q,k,v     device, layout per `problem` (bf16 or fp32 per dtype); k and
 *             v may be NULL when total_k is 0 (nothing is then read).
 *   o         device, same layout and dtype as q.
 *   lse       device float32 [heads_q][total_q], natural log of the sum of
 *             exp(score) over visible keys (scores after score_mod).  A row
 *             with nothing visible gets O = 0 and LSE = -inf [MPD §6.1].
 *   scale     multiplies q.k before score_mod; finite and > 0 (usually
 *             1/sqrt(head_dim)), else MPB_ERR_INVALID_ARGUMENT.
 *   mod       NULL for no score_mod.
 *   workspace device, >= flex_attn_fwd_workspace_size(plan) bytes (may be
 *             NULL when that is 0).
 * Partial tiles apply their predicate; full tiles skip it; empty tiles are
 * never touched.  Enqueue only; no synchronisation.  Every refusal happens
 * before the launch [PYG "Accept means run"]. */
mpb_status flex_attn_fwd(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                         const void* k, const void* v, void* o, float* lse, float scale,
                         const mpb_score_mod* mod, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Ablation hooks: same contracts as flex_attn_fwd / flex_attn_bwd, with
 * flags selecting slower paths whose results are identical bit for bit:
 *   MPB_ABLATE_FULL_AS_PARTIAL (forward only): every full tile runs through
 *     the partial-tile code path with an all-ones predicate, which measures
 *     what the full-tile fast path saves ([FLEX] "full block optimization";
 *     [MPD §6.1]);
 *   MPB_ABLATE_NO_SKIP: the kernels compute every listed tile and block,
 *     including those they otherwise skip because every weight in them is
 *     exactly zero in fp32 (a predicate that hides a block from all of a
 *     wavefront's rows; scores bounded 200 log2 units below the running max
 *     or the row's LSE), which checks that those skips change nothing (given
 *     finite V: a skipped 0 * inf would have been NaN).
 * Unknown flag bits return MPB_ERR_INVALID_ARGUMENT. */
enum { MPB_ABLATE_FULL_AS_PARTIAL = 1, MPB_ABLATE_NO_SKIP = 2 };
mpb_status flex_attn_fwd_ablation(const mpb_plan* plan, const mpb_problem* problem,
                                  const void* q, const void* k, const void* v, void* o,
                                  float* lse, float scale, const mpb_score_mod* mod,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  int32_t flags);

/* Split-K forward [TESS "Split-K", Figure 5; MPD §6.1]: for plans with too
 * few tasks to fill the GPU (short Q against a long K, few heads or
 * samples), every task's tile list (partial tiles, then full tiles, n of
 * them) is cut into num_splits contiguous parts; part s covers list
 * positions [s*n/S, (s+1)*n/S) and runs in its own workgroup, writing the
 * softmax output normalized over its tiles (fp32) and their log-sum-exp to
 * the workspace; a merge kernel then rescales the parts to a common maximum,
 * sums and normalizes them into o and lse (flex_attn_fwd_merge).  Results
 * equal flex_attn_fwd's up to fp32 rounding order; o is rounded to its
 * dtype once, after the merge.
 *
 * flex_attn_fwd_num_splits: the library's choice for a plan: 1 when the
 * plan has at least as many tasks as the GPU holds resident workgroups,
 * else enough parts to fill it, with at least four tiles per part on
 * average, at most 64.
 * flex_attn_fwd_splitk_workspace_size: bytes needed for num_splits parts
 * (0 = the library's choice): per part, fp32 O [total_q][heads_q][head_dim]
 * and fp32 LSE [heads_q][total_q], each area rounded up to 256 bytes; 0 when
 * the resolved split count is 1.
 * flex_attn_fwd_splitk: arguments as flex_attn_fwd, plus num_splits in
 * [0, 64] (0 = library's choice; 1 = flex_attn_fwd itself).  With more than
 * one part the workspace must be 256-byte aligned and o 16-byte aligned.
 * Enqueues the split launch and the merge launch on `stream`; the
 * workspace is in use until the merge has run.  Errors as flex_attn_fwd,
 * MPB_ERR_INVALID_ARGUMENT for num_splits out of range. */
int32_t flex_attn_fwd_num_splits(const mpb_plan* plan);
size_t flex_attn_fwd_splitk_workspace_size(const mpb_plan* plan, int32_t num_splits);
mpb_status flex_attn_fwd_splitk(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                                const void* k, const void* v, void* o, float* lse, float scale,
                                const mpb_score_mod* mod, int32_t num_splits, void* workspace,
                                size_t workspace_bytes, void* stream);

/* flex_attn_fwd_splitk without allocation, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results
 * and errors as flex_attn_fwd_splitk minus the workspace: the partial states
 * live in a static device array of the library (64 MiB, one per GPU the
 * library runs on, held until the process ends), so a call whose resolved
 * parts need more than that (flex_attn_fwd_splitk_workspace_size) returns
 * MPB_ERR_WORKSPACE before any launch.  No device or host memory is
 * allocated.  Every call overwrites the partial states it reads (nothing
 * needs clearing), and all calls on one GPU share the array: calls that
 * overlap on one GPU (several streams or host threads) race and must be
 * ordered by the caller.  A resolved split count of 1 runs flex_attn_fwd. */
mpb_status flex_attn_fwd_splitk_noalloc(const mpb_plan* plan, const mpb_problem* problem,
                                        const void* q, const void* k, const void* v, void* o,
                                        float* lse, float scale, const mpb_score_mod* mod,
                                        int32_t num_splits, void* stream);

/* flex_attn_fwd_merge [TESS "Split-K"]: merges num_parts partial attention
 * states of the same rows, e.g. the parts of a Split-K forward or the
 * outputs of attention over disjoint key ranges.  Row r = token*heads_q + h.
 *   o_parts   device fp32 [num_parts][total_q][heads_q][head_dim], part s's
 *             output normalized over its own keys (16-byte aligned).
 *   lse_parts device fp32 [num_parts][heads_q][total_q], part s's natural
 *             log-sum-exp; -inf = the part holds no key of the row (its O
 *             is then not read).  Finite or -inf values only.
 *   o         device [total_q][heads_q][head_dim] in dtype (bf16 or fp32),
 *             16-byte aligned:  O = sum_s exp(L_s - LSE) O_s.
 *   lse       device fp32 [heads_q][total_q]:  LSE = M + ln sum_s exp(L_s - M),
 *             M = max_s L_s.  A row whose parts are all empty gets O = 0,
 *             LSE = -inf.
 * head_dim 64 or 128 (else MPB_ERR_UNSUPPORTED).  Enqueue only. */
mpb_status flex_attn_fwd_merge(int32_t num_parts, int32_t total_q, int32_t heads_q,
                               int32_t head_dim, int32_t dtype, const float* o_parts,
                               const float* lse_parts, void* o, float* lse, void* stream);

/* Paged K/V forward [FLEX paged attention: the page table is folded into
 * the block indices, physical = page_table[batch][logical]; MPD §6.1]:
 * flex_attn_fwd (or, with num_splits != 1, flex_attn_fwd_splitk) with K and
 * V read from page pools instead of contiguous BSHD/THD tensors.
 *   k_pages, v_pages  device pools of token rows, [num_pages * page_size]
 *             [heads_k][head_dim] in the plan's dtype: logical K position
 *             kk of sample b lives in pool row
 *             page_table[b][kk / page_size] * page_size + kk % page_size.
 *   page_table device int32 [batch][pages_per_seq]; entries must lie in
 *             [0, num_pages) for every page a sample's k_len reaches (an
 *             entry outside it is read as zeros, never dereferenced).
 *   page_size a positive multiple of the plan's tile_k (a K tile never
 *             straddles pages), else MPB_ERR_UNSUPPORTED.
 *   pages_per_seq * page_size >= seqlen_k (the longest sample).
 *   q, o, lse, problem, scale, mod: as flex_attn_fwd (problem describes the
 *             logical K: seqlen_k / total_k / cu_seqlens as for the plan).
 *   num_splits as flex_attn_fwd_splitk (1 = one workgroup per task).
 *   remap     1: a remap launch first writes the pool tile of every listed K
 *             tile into the workspace; 0: the workspace already holds them
 *             from an earlier call with remap = 1 on the same plan, page
 *             table contents and page_size, and they are reused (e.g. the
 *             layers of one model step share one page table).
 *   workspace >= flex_attn_fwd_paged_workspace_size(plan, num_splits) bytes,
 *             256-byte aligned: the remapped lists, then the Split-K area.
 * Pool rows past a sample's k_len are never read (loads there return
 * zero), so unused pool rows may hold anything.  Results are identical to
 * flex_attn_fwd (or flex_attn_fwd_splitk) on the same logical K/V.  bf16
 * plans only (fp32: MPB_ERR_UNSUPPORTED). */
size_t flex_attn_fwd_paged_workspace_size(const mpb_plan* plan, int32_t num_splits);
mpb_status flex_attn_fwd_paged(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                               const void* k_pages, const void* v_pages,
                               const int32_t* page_table, int32_t page_size,
                               int32_t pages_per_seq, int32_t num_pages, void* o, float* lse,
                               float scale, const mpb_score_mod* mod, int32_t num_splits,
                               int32_t remap, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Bytes of caller-provided device workspace flex_attn_bwd needs: two fp32
 * per (Q row, head), dO . O and the LSE in log2 units, each vector rounded
 * up to 256 bytes. */
size_t flex_attn_bwd_workspace_size(const mpb_plan* plan);

/* flex_attn_bwd [MPD §6.3, §8; FLEX Eq. 1 and its automatic backward]:
 * gradients of O = softmax(mod(Q K^T * scale)) V for an incoming dO.
 *   plan      built with build_backward = 1 (else MPB_ERR_INVALID_ARGUMENT:
 *             a training call needs the backward view [MPD §8]); problem,
 *             device and tile checked as for flex_attn_fwd.  bf16 only, at
 *             the forward's bf16 tile geometries (else MPB_ERR_UNSUPPORTED).
 *   q,k,v     device bf16, the forward's inputs, layout per `problem`.
 *             Tensors of an empty side may be NULL: q, o, lse, dout, dq when
 *             total_q is 0; k, v, dk, dv when total_k is 0.
 *   o, lse    the forward's outputs for these inputs (flex_attn_fwd).
 *   dout      device bf16, layout of o: the gradient of the loss w.r.t. O.
 *   dq        device bf16, layout of q (overwritten).
 *   dk, dv    device bf16, layout of k and v (overwritten): for grouped
 *             heads, summed over the Q heads of each KV head.
 *   scale,mod exactly as given to the forward; the score_mod contributes its
 *             derivative (softcap: 1 - tanh^2 of its argument; ALiBi: 1).
 *   workspace device, >= flex_attn_bwd_workspace_size(plan) bytes.
 * The dQ consumer walks the Q2K view, the dK/dV consumer the K2Q view;
 * partial entries apply their predicate, full entries none, empty pairs are
 * never touched [MPD §6.3].  A row with nothing visible contributes nothing;
 * a K row that no Q row sees gets dK = dV = 0.  Every buffer must be 16-byte
 * aligned.  Enqueue only; every refusal happens before any launch. */
mpb_status flex_attn_bwd(const mpb_plan* plan, const mpb_problem* problem, const void* q,
                         const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float scale,
                         const mpb_score_mod* mod, void* workspace, size_t workspace_bytes,
                         void* stream);

/* flex_attn_bwd with ablation flags (see flex_attn_fwd_ablation; only
 * MPB_ABLATE_NO_SKIP applies to the backward). */
mpb_status flex_attn_bwd_ablation(const mpb_plan* plan, const mpb_problem* problem,
                                  const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk,
                                  void* dv, float scale, const mpb_score_mod* mod,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  int32_t flags);

const char* mpb_status_string(mpb_status status);
const char* mpb_last_error_detail(void);

/* Library ABI version (major*100 + minor). */
int32_t mpb_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MPB_H_ */
