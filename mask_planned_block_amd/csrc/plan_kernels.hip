// MaskPlan builder kernels for gfx950.
//
// Stages follow "Flex Attention Mask Plan Design" (cuDNN frontend docs):
//   plan_geometry_kernel    §4.2 Varlen geometry (THD only): validates
//                           cu_seqlens, builds the per-sample descriptor and
//                           the compact Q plan-row prefix.  Fixed-length
//                           geometry is closed form (written by the scan).
//   plan_classify_kernel    §4.3 Q2K classification: one wavefront per
//                           (mask head, Q plan row).  Each lane reads its
//                           row's intervals once (coalesced across lanes),
//                           validates them (§2 order and bounds), merges
//                           touching intervals and records the K tiles each
//                           run touches / fully covers in LDS difference
//                           arrays; a wavefront prefix scan then gives, per
//                           tile, how many rows see it at all and how many see
//                           all of it: any > 0 is visible, all == T_Q is full.
//   plan_index_kernel       one workgroup: §4.5 exact exclusive CSR offsets
//                           and the 8-value allocation header (device errors
//                           OR-ed in, published to host-mapped memory), then
//                           §4.8 the forward schedule as a stable counting sort
//                           and the section-interleaved launch records.
//   plan_materialize_kernel §4.6 / §5 Q2K materialisation: ascending partial
//                           and full K-tile indices, and one predicate word per
//                           (row, 32 columns) of each partial tile.
//
// Visibility used throughout: with sorted endpoints F, column k is visible iff
// an even number of endpoints are <= k (k < F0: none; F0 <= k < F1: one, ...),
// which is the union [0,F0) U [F1,F2) U ... of §2; columns >= F(nfunc-1)
// (hence >= k_len) see an odd count and are masked.
#include "mpb_internal.h"
#include "../../include/mpb.h"

namespace mpb {

namespace {

__device__ inline int sample_of_row(const int32_t* cu_rows, int batch, int row) {
  // Largest b with cu_rows[b] <= row; empty samples share their prefix value
  // with the next sample and are skipped by taking the largest such b.
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_rows[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline int wave_lane() { return threadIdx.x & 63; }

__device__ inline uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Geometry of one Q plan row: sample, tile row within the sample, bounds.
struct RowGeo {
  int b, i, q_off, q_len, k_off, k_len, nk, row_begin;
};

__device__ inline RowGeo row_geometry(const PlanGeo& g, const PlanDev& d, int row) {
  RowGeo r;
  if (g.layout == MPB_LAYOUT_BSHD) {
    const int rps = (g.seqlen_q + g.tile_q - 1) / g.tile_q;
    r.b = row / rps;
    r.i = row - r.b * rps;
    r.q_off = r.b * g.seqlen_q;
    r.q_len = g.seqlen_q;
    r.k_off = r.b * g.seqlen_k;
    r.k_len = g.seqlen_k;
    r.row_begin = r.b * rps;
  } else {
    r.b = sample_of_row(d.cu_rows, g.batch, row);
    const int32_t* sd = d.seqdesc + 8 * r.b;
    r.q_off = sd[0];
    r.k_off = sd[1];
    r.q_len = sd[2];
    r.k_len = sd[3];
    r.row_begin = sd[4];
    r.i = row - r.row_begin;
  }
  r.nk = (r.k_len + g.tile_k - 1) / g.tile_k;
  return r;
}

__device__ inline int rows_total_of(const PlanGeo& g, const PlanDev& d) {
  return g.layout == MPB_LAYOUT_BSHD ? g.upper_rows : d.cu_rows[g.batch];
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

}  // namespace

// ---------------------------------------------------------------- geometry

__global__ __launch_bounds__(1024) void plan_geometry_kernel(PlanGeo g, const int32_t* cu_q,
                                                             const int32_t* cu_k, PlanDev d,
                                                             PlanWork w) {
  __shared__ int s_bad;
  __shared__ int s_carry;
  __shared__ int s_scan[1024];
  const int tid = threadIdx.x;
  const int B = g.batch;
  if (tid == 0) {
    s_bad = 0;
    s_carry = 0;
  }
  __syncthreads();
  // §3.2: prefixes start at 0, end at the totals, never decrease and no
  // sample exceeds max_seqlen.  The plan keeps its own copy of both.
  for (int b = tid; b <= B; b += blockDim.x) {
    int bad = 0;
    const int q1 = cu_q[b], k1 = cu_k[b];
    if (b == 0 && (q1 != 0 || k1 != 0)) bad = 1;
    if (b == B && (q1 != g.total_q || k1 != g.total_k)) bad = 1;
    if (b < B) {
      const int q2 = cu_q[b + 1], k2 = cu_k[b + 1];
      if (q2 < q1 || k2 < k1) bad = 1;
      if ((int64_t)q2 - q1 > g.seqlen_q || (int64_t)k2 - k1 > g.seqlen_k) bad = 1;
    }
    d.cu_q[b] = q1;
    d.cu_k[b] = k1;
    if (bad) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  // With a bad prefix every sample is given zero length, so later stages see
  // no rows and touch nothing; the error bit makes the build fail.
  for (int base = 0; base < B; base += blockDim.x) {
    const int b = base + tid;
    int q_off = 0, q_len = 0, k_off = 0, k_len = 0;
    if (b < B && !bad) {
      q_off = cu_q[b];
      q_len = cu_q[b + 1] - q_off;
      k_off = cu_k[b];
      k_len = cu_k[b + 1] - k_off;
    }
    const int rows_b = (q_len + g.tile_q - 1) / g.tile_q;
    s_scan[tid] = rows_b;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int incl = s_scan[tid] + s_carry;
    if (b < B) {
      d.cu_rows[b + 1] = incl;
      int32_t* sd = d.seqdesc + 8 * b;
      sd[0] = q_off;
      sd[1] = k_off;
      sd[2] = q_len;
      sd[3] = k_len;
      sd[4] = incl - rows_b;
      sd[5] = rows_b;
      sd[6] = (k_len + g.tile_k - 1) / g.tile_k;
      sd[7] = 0;
    }
    __syncthreads();
    if (tid == (int)blockDim.x - 1) s_carry = incl;
    __syncthreads();
  }
  if (tid == 0) {
    d.cu_rows[0] = 0;
    w.geo_err[0] = bad ? MPB_DEVERR_SEQLENS : 0;
  }
}

// ---------------------------------------------------------------- classify

namespace {

// bits [lo, hi) of a 32-bit word, 0 <= lo < hi <= 32
__device__ inline uint32_t range_bits(int lo, int hi) {
  const uint32_t upto = hi >= 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u);
  return upto & ~((1u << lo) - 1u);
}

// OR tiles [t0, t1) into a 128-tile window starting at tile tg.
__device__ inline void set_tiles(uint32_t (&m)[4], int t0, int t1, int tg) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int w0 = tg + 32 * x;
    const int lo = max(t0, w0), hi = min(t1, w0 + 32);
    if (hi > lo) m[x] |= range_bits(lo - w0, hi - w0);
  }
}

__device__ inline uint32_t wave_or(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x |= (uint32_t)__shfl_xor((int)x, off);
  return x;
}
__device__ inline uint32_t wave_and(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x &= (uint32_t)__shfl_xor((int)x, off);
  return x;
}

}  // namespace

// One wavefront per (mask head, Q plan row); lanes own rows lane + 64t.
// Tiles are handled in windows of 128 (four 32-bit words): for each window a
// lane walks its row's intervals (read 8 at a time, coalesced across lanes),
// merges touching intervals into runs, and ORs the tiles each run touches
// ("any") or fully covers ("full") into its words.  Across the wavefront the
// "any" words are OR-ed and the "full" words AND-ed: a tile is visible if any
// row sees part of it and full if every one of the T_Q rows covers it, which
// needs every row in bounds (rows past q_len contribute nothing) and the tile
// inside k_len (no run extends past k_len).  §2 order and bounds of every
// endpoint are checked on the way.
template <int RPL>
__global__ __launch_bounds__(256) void plan_classify_kernel(PlanGeo g,
                                                            const int32_t* __restrict__ mf,
                                                            PlanDev d, PlanWork w) {
  const int lane = wave_lane();
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  // Side job: clear the schedule's [bucket][chunk] count matrix (read only
  // by the schedule kernels, which run after this kernel).
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < w.chunk_cnt_len;
       x += (int64_t)gridDim.x * blockDim.x)
    w.chunk_cnt[x] = 0;
  const int hm = item / g.upper_rows;
  const int row = item - hm * g.upper_rows;
  if (hm >= g.mask_heads) return;
  if (row >= rows_total_of(g, d)) return;
  const RowGeo rg = row_geometry(g, d, row);
  const int nk = rg.nk;
  const int T = g.tile_k;
  const int nint = (g.nfunc + 1) >> 1;

  bool valid[RPL], exists[RPL];
  const int32_t* col[RPL];
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int rho = lane + 64 * t;
    exists[t] = rho < g.tile_q;
    valid[t] = exists[t] && rg.i * g.tile_q + rho < rg.q_len;
    col[t] = mf + (int64_t)hm * g.nfunc * g.total_q + rg.q_off + (int64_t)rg.i * g.tile_q +
             (valid[t] ? rho : 0);
  }

  uint32_t err = 0;
  int pc = 0, fc = 0;
  const int64_t wbase = ((int64_t)hm * g.upper_rows + row) * g.words_k;
  for (int tg = 0; tg < nk; tg += 128) {
    uint32_t any_m[4] = {0u, 0u, 0u, 0u};
    uint32_t full_m[4] = {~0u, ~0u, ~0u, ~0u};   // AND identity
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
      if (!exists[t]) continue;                    // not a row of the tile
      uint32_t rf[4] = {0u, 0u, 0u, 0u};
      if (valid[t]) {
        // A run [a, b) touches tiles a/T .. (b-1)/T and fully covers
        // ceil(a/T) .. b/T - 1 (clamped to [0, nk] for malformed input).
        auto flush = [&](int a, int b) {
          if (b <= a) return;
          const int t0 = min(max(a / T, 0), nk), t1 = min(max((b - 1) / T + 1, 0), nk);
          set_tiles(any_m, t0, t1, tg);
          const int f0 = min(max((a + T - 1) / T, 0), nk), f1 = min(max(b / T, 0), nk);
          set_tiles(rf, f0, f1, tg);
        };
        int run_a = 0, run_b = 0;  // open run, empty when run_b <= run_a
        int prev = 0;
        constexpr int kBatch = 8;
        for (int p0 = 0; p0 < nint; p0 += kBatch) {
          int sv[kBatch], ev[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int p = p0 + u;
            sv[u] = 0;
            ev[u] = 0;
            if (p < nint) {
              if (p > 0) sv[u] = col[t][(int64_t)(2 * p - 1) * g.total_q];
              ev[u] = col[t][(int64_t)(2 * p) * g.total_q];
            }
          }
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int p = p0 + u;
            if (p >= nint) break;
            const int s = sv[u], e = ev[u];
            if (tg == 0) {
              if (p > 0) {
                if (s < prev) err |= MPB_DEVERR_ORDER;
                if (s < 0 || s > rg.k_len) err |= MPB_DEVERR_RANGE;
              }
              if (e < s) err |= MPB_DEVERR_ORDER;
              if (e < 0 || e > rg.k_len) err |= MPB_DEVERR_RANGE;
            }
            prev = e;
            if (e <= s) continue;                 // empty interval
            if (run_b > run_a && s == run_b) {
              run_b = e;                          // touching: extend the run
            } else {
              flush(run_a, run_b);
              run_a = s;
              run_b = e;
            }
          }
        }
        flush(run_a, run_b);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) full_m[x] &= rf[x];
    }
    uint32_t vis_w[4], full_w[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      vis_w[x] = wave_or(any_m[x]);
      full_w[x] = wave_and(full_m[x]);
      const int w0 = tg + 32 * x;
      const uint32_t live = w0 >= nk ? 0u : (nk - w0 >= 32 ? ~0u : ((1u << (nk - w0)) - 1u));
      vis_w[x] &= live;
      full_w[x] &= vis_w[x];
      pc += __popc(vis_w[x] & ~full_w[x]);
      fc += __popc(full_w[x]);
    }
    if (lane < 4) {
      const int x = lane;
      const int w0 = tg + 32 * x;
      if (w0 < nk) {
        w.vis_bits[wbase + (w0 >> 5)] = x == 0 ? vis_w[0] : x == 1 ? vis_w[1] : x == 2 ? vis_w[2] : vis_w[3];
        w.full_bits[wbase + (w0 >> 5)] = x == 0 ? full_w[0] : x == 1 ? full_w[1] : x == 2 ? full_w[2] : full_w[3];
      }
    }
  }
  const uint64_t er = __ballot((err & MPB_DEVERR_RANGE) != 0);
  const uint64_t eo = __ballot((err & MPB_DEVERR_ORDER) != 0);
  if (lane == 0) {
    const int64_t it = (int64_t)hm * g.upper_rows + row;
    w.pcnt[it] = pc;
    w.fcnt[it] = fc;
    w.item_err[it] = (er ? MPB_DEVERR_RANGE : 0) | (eo ? MPB_DEVERR_ORDER : 0);
  }
}

// ---------------------------------------------------------------- scan, header, schedule

namespace {

__device__ inline void block_incl_scan2(int* sa, int* sb, int tid, int n) {
  for (int off = 1; off < n; off <<= 1) {
    const int va = tid >= off ? sa[tid - off] : 0;
    const int vb = tid >= off ? sb[tid - off] : 0;
    __syncthreads();
    sa[tid] += va;
    sb[tid] += vb;
    __syncthreads();
  }
}

// In-place exclusive scan of n ints (LDS or global) by one workgroup of 1024
// threads: four consecutive values per thread, a wavefront shuffle scan of
// the thread sums and one scan of the 16 wavefront totals -- two barriers per
// 4096 values.  Returns the total (valid in every thread).
__device__ inline int block_exclusive_scan_inplace(int32_t* a, int64_t n, int* s_wave,
                                                   int* s_carry) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) *s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < n; base += 4096) {
    const int64_t i0 = base + 4 * (int64_t)tid;
    int v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i0 + u < n ? a[i0 + u] : 0;
    const int tsum = v[0] + v[1] + v[2] + v[3];
    const int incl = wave_incl_scan(tsum, lane);
    if (lane == 63) s_wave[wv] = incl;
    __syncthreads();
    if (wv == 0) {
      const int t = lane < 16 ? s_wave[lane] : 0;
      const int ti = wave_incl_scan(t, lane);
      if (lane < 16) s_wave[16 + lane] = ti - t;   // exclusive prefix of wave totals
      if (lane == 15) s_wave[32] = ti;             // block total
    }
    __syncthreads();
    int run = *s_carry + s_wave[16 + wv] + incl - tsum;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + u < n) a[i0 + u] = run;
      run += v[u];
    }
    __syncthreads();
    if (tid == 0) *s_carry += s_wave[32];
    __syncthreads();
  }
  return *s_carry;
}

struct TaskInfo {
  int b, h, i, rows_b, row;
};

__device__ inline TaskInfo decode_task(const PlanGeo& g, const PlanDev& d, int t) {
  // Canonical tie order: t = Hq*cu_rows[b] + h*rows_b + i.
  TaskInfo r;
  r.b = sample_of_row(d.cu_rows, g.batch, t / g.heads_q);
  const int r0 = d.cu_rows[r.b];
  r.rows_b = d.cu_rows[r.b + 1] - r0;
  const int rel = t - g.heads_q * r0;
  r.h = rel / r.rows_b;
  r.i = rel - r.h * r.rows_b;
  r.row = r0 + r.i;
  return r;
}

__device__ inline int task_cost(const PlanGeo& g, const PlanWork& w, int h, int row) {
  const int hm = g.mask_heads == 1 ? 0 : h;
  const int64_t src = (int64_t)hm * g.upper_rows + row;
  return w.pcnt[src] + w.fcnt[src];
}

__device__ inline int task_section(const PlanGeo& g, int b, int h, int cost) {
  if (cost == 0) return kNumSections;
  const int group = g.heads_q / g.heads_k;
  return (b * g.heads_k + h / group) % kNumSections;
}

// Launch slot of the r-th task of section s: sections interleaved while they
// last; zero-cost tasks after all positive-cost ones.
__device__ inline int launch_slot(const PlanDev& d, int s, int r) {
  if (s >= kNumSections) return d.section_off[kNumSections] + r;
  int slot = 0;
#pragma unroll
  for (int s2 = 0; s2 < kNumSections; ++s2) {
    const int n2 = d.section_off[s2 + 1] - d.section_off[s2];
    slot += min(r, n2) + ((s2 < s && n2 > r) ? 1 : 0);
  }
  return slot;
}

__device__ inline void write_task(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                  const TaskInfo& ti, int s, int pos, int rows_total) {
  const int32_t* sd = d.seqdesc + 8 * ti.b;
  const int qvalid = min(g.tile_q, sd[2] - ti.i * g.tile_q);
  int32_t* wd = d.work_desc + 4 * (int64_t)pos;
  wd[0] = ti.i;
  wd[1] = ti.h;
  wd[2] = ti.b;
  wd[3] = qvalid;
  const int hm = g.mask_heads == 1 ? 0 : ti.h;
  const int64_t flat = (int64_t)hm * rows_total + ti.row;
  const int64_t src = (int64_t)hm * g.upper_rows + ti.row;
  const int p_beg = w.p_off_tmp[flat], np = w.p_off_tmp[flat + 1] - p_beg;
  const int f_beg = w.f_off_tmp[flat], nf = w.f_off_tmp[flat + 1] - f_beg;
  int first = -1;
  if (np + nf > 0) {
    const int nwords = (sd[6] + 31) >> 5;
    for (int ww = 0; ww < nwords && first < 0; ++ww) {
      const uint32_t vw = w.vis_bits[src * g.words_k + ww];
      const uint32_t fw = w.full_bits[src * g.words_k + ww];
      const uint32_t pick = np > 0 ? (vw & ~fw) : fw;  // partial list first (§6.1)
      if (pick) first = 32 * ww + __ffs(pick) - 1;
    }
  }
  int32_t* rec = d.task_rec + (int64_t)launch_slot(d, s, pos - d.section_off[s]) * kTaskRecInts;
  rec[kRecMBlock] = ti.i;
  rec[kRecHead] = ti.h;
  rec[kRecBatch] = ti.b;
  rec[kRecQValid] = qvalid;
  rec[kRecQOff] = sd[0];
  rec[kRecKOff] = sd[1];
  rec[kRecQLen] = sd[2];
  rec[kRecKLen] = sd[3];
  rec[kRecPBeg] = p_beg;
  rec[kRecPCnt] = np;
  rec[kRecFBeg] = f_beg;
  rec[kRecFCnt] = nf;
  rec[kRecFirstTile] = first;
  rec[kRecMaskHead] = hm;
  rec[kRecKvHead] = ti.h / (g.heads_q / g.heads_k);
  rec[kRecSection] = s;
}

}  // namespace

// One workgroup after classification:
//  1. §4.5 exact exclusive CSR offsets over rows flattened head-major
//     (flat = hm * rows_total + row), off[0] = 0, off[i+1] = off[i] + cnt[i];
//     the fixed-length geometry in closed form; the 8-value header with the
//     OR of every device error bit, published to host-mapped memory so the
//     host reads it with no copy command.
//  2. §4.8 the forward schedule: section ascending, cost descending, ties in
//     canonical order t = Hq*cu_rows[b] + h*rows_b + i; zero-cost tasks form
//     the last section.  A stable counting sort: tasks are cut into chunks
//     of 64 (one wavefront each) that yield each task's bucket key, its rank
//     among equal keys of the chunk and the chunk's bucket counts; one
//     exclusive scan of the counts laid out [bucket][chunk] gives, per
//     (bucket, chunk), the position of the chunk's first task of that bucket.
//     Each task is then written to the section-major schedule and, as a
//     launch record, at its section-interleaved launch slot.
__global__ __launch_bounds__(1024) void plan_index_kernel(PlanGeo g, PlanDev d, PlanWork w,
                                                          int32_t* host_header, int cnt_in_lds) {
  extern __shared__ int dyn[];
  __shared__ int sa[1024], sb[1024];
  __shared__ int carry_p, carry_f;
  __shared__ uint32_t s_err;
  __shared__ int s_wave[33];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int rows_total = rows_total_of(g, d);
  const int n = g.mask_heads * rows_total;
  if (tid == 0) {
    carry_p = 0;
    carry_f = 0;
    s_err = g.layout == MPB_LAYOUT_THD ? (uint32_t)w.geo_err[0] : 0u;
  }
  // Fixed-length geometry in closed form (§4.2: rectangular upper bound).
  if (g.layout == MPB_LAYOUT_BSHD) {
    const int rps = (g.seqlen_q + g.tile_q - 1) / g.tile_q;
    for (int b = tid; b < g.batch; b += 1024) {
      int32_t* sd = d.seqdesc + 8 * b;
      sd[0] = b * g.seqlen_q;
      sd[1] = b * g.seqlen_k;
      sd[2] = g.seqlen_q;
      sd[3] = g.seqlen_k;
      sd[4] = b * rps;
      sd[5] = rps;
      sd[6] = (g.seqlen_k + g.tile_k - 1) / g.tile_k;
      sd[7] = 0;
      d.cu_rows[b + 1] = (b + 1) * rps;
    }
    if (tid == 0) d.cu_rows[0] = 0;
  }
  __syncthreads();
  uint32_t err = 0;
  for (int base = 0; base < n; base += 1024) {
    const int idx = base + tid;
    int a = 0, c = 0;
    if (idx < n) {
      const int hm = idx / rows_total;
      const int r = idx - hm * rows_total;
      const int64_t it = (int64_t)hm * g.upper_rows + r;
      a = w.pcnt[it];
      c = w.fcnt[it];
      err |= (uint32_t)w.item_err[it];
    }
    sa[tid] = a;
    sb[tid] = c;
    __syncthreads();
    block_incl_scan2(sa, sb, tid, 1024);
    if (idx < n) {
      w.p_off_tmp[idx] = carry_p + sa[tid] - a;
      w.f_off_tmp[idx] = carry_f + sb[tid] - c;
    }
    __syncthreads();
    if (tid == 1023) {
      carry_p += sa[1023];
      carry_f += sb[1023];
    }
    __syncthreads();
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  if (tid == 0) {
    w.p_off_tmp[n] = carry_p;
    w.f_off_tmp[n] = carry_f;
    const int32_t hdr[8] = {rows_total, carry_p, carry_f, 0, 0, 0, 0, (int32_t)s_err};
    for (int i = 0; i < 8; ++i) {
      d.header[i] = hdr[i];
      __hip_atomic_store(&host_header[i], hdr[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    __threadfence_system();
  }
  if (s_err) return;  // no plan will be built (uniform: read after the barrier)

  // ---- schedule
  const int ntasks = rows_total * g.heads_q;
  const int per = g.nk_max + 1;
  const int nc = w.nchunks;
  int32_t* cnt = cnt_in_lds ? dyn : w.chunk_cnt;
  if (cnt_in_lds)
    for (int64_t x = tid; x < w.chunk_cnt_len; x += 1024) cnt[x] = 0;  // global copy: zeroed by classify
  __syncthreads();
  const uint64_t lt = lanes_below(lane);
  for (int chunk = wv; chunk * 64 < ntasks; chunk += 16) {
    const int t = chunk * 64 + lane;
    int key = -1;
    if (t < ntasks) {
      const TaskInfo ti = decode_task(g, d, t);
      const int cost = task_cost(g, w, ti.h, ti.row);
      key = task_section(g, ti.b, ti.h, cost) * per + (g.nk_max - cost);
      w.keys[t] = key;
    }
    bool todo = t < ntasks;
    while (true) {  // one pass per distinct key of the chunk
      const uint64_t m = __ballot(todo);
      if (m == 0) break;
      const int leader = __ffsll((unsigned long long)m) - 1;
      const int k0 = __shfl(key, leader);
      const bool same = todo && key == k0;
      const uint64_t match = __ballot(same);
      if (same) {
        w.lrank[t] = __popcll(match & lt);
        todo = false;
      }
      if (lane == leader) cnt[(int64_t)k0 * nc + chunk] = __popcll(match);
    }
  }
  __syncthreads();
  const int total = block_exclusive_scan_inplace(cnt, w.chunk_cnt_len, s_wave, &s_carry);
  const int64_t per_section = (int64_t)per * nc;
  if (tid < kNumQueues) d.section_off[tid] = cnt[(int64_t)tid * per_section];
  if (tid == 0) d.section_off[kNumQueues] = total;
  __syncthreads();
  for (int t = tid; t < ntasks; t += 1024) {
    const int key = w.keys[t];
    const int pos = cnt[(int64_t)key * nc + t / 64] + w.lrank[t];
    write_task(g, d, w, decode_task(g, d, t), key / per, pos, rows_total);
  }
}

// ---------------------------------------------------------------- materialize

// One workgroup per (mask head, Q plan row), one thread per Q row of the
// tile.
//  * §4.6: exact offsets and the ascending partial and full K-tile indices
//    (sample-local), partial and full kept apart; the partial list is also
//    staged in LDS for the payload loop.
//  * §5: payload word [r][c/32] bit c%32 is 1 iff column c is visible for row
//    r.  A column is visible iff an even number of the row's endpoints are
//    <= it, so a word starts from that parity at its first column and each
//    endpoint inside the word flips the bits from its column on.  The
//    thread's endpoints are staged in LDS (when [nfunc][T_Q] ints fit) and
//    its pointer (endpoints <= current column) only moves forward, because
//    partial tiles are listed in ascending order.  Rows past q_len write 0.
__global__ __launch_bounds__(256) void plan_materialize_kernel(PlanGeo g,
                                                               const int32_t* __restrict__ mf,
                                                               PlanDev d, PlanWork w,
                                                               int rows_total, int stage_ep) {
  extern __shared__ int lds[];
  int* tiles = lds;                     // [nk_max] partial K tiles of this row
  int* ep = lds + g.nk_max;             // [nfunc][T_Q] endpoints when staged
  const int item = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = g.mask_heads * rows_total;
  if (item == 0 && tid == 0) {
    d.p_off[n] = w.p_off_tmp[n];
    d.f_off[n] = w.f_off_tmp[n];
  }
  if (item >= n) return;
  const int hm = item / rows_total;
  const int row = item - hm * rows_total;
  const int64_t src = (int64_t)hm * g.upper_rows + row;
  const int p_begin = w.p_off_tmp[item];
  const int f_begin = w.f_off_tmp[item];
  const int np = w.p_off_tmp[item + 1] - p_begin;
  const RowGeo rg = row_geometry(g, d, row);
  if (tid == 0) {
    d.p_off[item] = p_begin;
    d.f_off[item] = f_begin;
  }
  if (tid < 64) {
    const int nwords = (rg.nk + 31) >> 5;
    int pb = 0, fb = f_begin;
    for (int ww = 0; ww < nwords; ++ww) {
      const uint32_t vw = w.vis_bits[src * g.words_k + ww];
      const uint32_t fw = w.full_bits[src * g.words_k + ww];
      const uint32_t pw = vw & ~fw;
      if (tid < 32) {
        const uint32_t bit = 1u << tid;
        const uint32_t below = bit - 1u;
        if (pw & bit) {
          const int k = pb + __popc(pw & below);
          d.p_idx[p_begin + k] = 32 * ww + tid;
          tiles[k] = 32 * ww + tid;
        }
        if (fw & bit) d.f_idx[fb + __popc(fw & below)] = 32 * ww + tid;
      }
      pb += __popc(pw);
      fb += __popc(fw);
    }
  }
  if (np == 0) return;  // uniform; no payload
  const int rho = tid;
  const bool is_row = rho < g.tile_q;
  const bool valid = is_row && rg.i * g.tile_q + rho < rg.q_len;
  const int32_t* col = mf + (int64_t)hm * g.nfunc * g.total_q + rg.q_off +
                       (int64_t)rg.i * g.tile_q + (valid ? rho : 0);
  if (stage_ep && valid)
    for (int f = 0; f < g.nfunc; ++f) ep[f * g.tile_q + rho] = col[(int64_t)f * g.total_q];
  __syncthreads();  // the partial tile list is complete
  auto E = [&](int f) -> int {
    return stage_ep ? ep[f * g.tile_q + rho] : col[(int64_t)f * g.total_q];
  };
  int ptr = 0;
  for (int k = 0; k < np; ++k) {
    const int c0 = tiles[k] * g.tile_k;
    uint32_t* dst = d.p_masks + ((int64_t)(p_begin + k) * g.tile_q + rho) * g.words_tile;
    for (int x = 0; x < g.words_tile; ++x) {
      uint32_t word = 0u;
      if (valid) {
        const int c = c0 + 32 * x;
        while (ptr < g.nfunc && E(ptr) <= c) ++ptr;
        word = (ptr & 1) ? 0u : 0xFFFFFFFFu;
        for (int f = ptr; f < g.nfunc; ++f) {
          const int e = E(f);
          if (e >= c + 32) break;
          word ^= 0xFFFFFFFFu << (e - c);
        }
      }
      if (is_row) dst[x] = word;
    }
  }
}

// ---------------------------------------------------------------- launchers

static inline int rows_per_lane(int tile_q) { return tile_q <= 64 ? 1 : tile_q / 64; }

hipError_t launch_plan_geometry(const PlanGeo& g, const int32_t* cu_q_in, const int32_t* cu_k_in,
                                const PlanDev& d, const PlanWork& w, hipStream_t s) {
  if (g.layout != MPB_LAYOUT_THD) return hipSuccess;
  hipLaunchKernelGGL(plan_geometry_kernel, dim3(1), dim3(1024), 0, s, g, cu_q_in, cu_k_in, d, w);
  return hipGetLastError();
}

hipError_t launch_plan_classify(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                                const PlanWork& w, hipStream_t s) {
  const int64_t items = (int64_t)g.mask_heads * g.upper_rows;
  if (items == 0) return hipSuccess;
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
  switch (rows_per_lane(g.tile_q)) {
    case 1: hipLaunchKernelGGL(plan_classify_kernel<1>, grid, block, 0, s, g, mask_func, d, w); break;
    case 2: hipLaunchKernelGGL(plan_classify_kernel<2>, grid, block, 0, s, g, mask_func, d, w); break;
    case 4: hipLaunchKernelGGL(plan_classify_kernel<4>, grid, block, 0, s, g, mask_func, d, w); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t index_kernel_lds(const PlanWork& w) {
  const size_t bytes = (size_t)w.chunk_cnt_len * 4;
  return bytes <= 40 * 1024 ? bytes : 0;
}

hipError_t launch_plan_index(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                             int32_t* host_header, hipStream_t s) {
  const size_t lds = index_kernel_lds(w);
  hipLaunchKernelGGL(plan_index_kernel, dim3(1), dim3(1024), lds, s, g, d, w, host_header,
                     lds > 0 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_plan_materialize(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                                   const PlanWork& w, int32_t rows_total, hipStream_t s) {
  const int64_t items = (int64_t)g.mask_heads * rows_total;
  const int threads = g.tile_q < 64 ? 64 : g.tile_q;
  const size_t ep_bytes = (size_t)g.nfunc * g.tile_q * 4;
  const int stage = ep_bytes <= 32 * 1024 ? 1 : 0;
  const size_t lds = (size_t)g.nk_max * 4 + (stage ? ep_bytes : 0);
  hipLaunchKernelGGL(plan_materialize_kernel, dim3((unsigned)(items > 0 ? items : 1)),
                     dim3(threads), lds, s, g, mask_func, d, w, rows_total, stage);
  return hipGetLastError();
}

}  // namespace mpb
