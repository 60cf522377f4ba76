// MaskPlan builder kernels for gfx950.
//
// Stages follow "Flex Attention Mask Plan Design" (cuDNN frontend docs):
//   plan_geometry_kernel    §4.2 Varlen geometry: validates cu_seqlens, builds
//                           the per-sample descriptor and the compact Q plan
//                           row prefix; fixed-length geometry is closed form.
//   plan_classify_kernel    §4.3 Q2K classification: one wavefront per
//                           (mask head, Q plan row); each lane owns Q rows and
//                           sweeps that row's sorted intervals; the per-tile
//                           any/all reduction is a wavefront ballot.  Also
//                           validates every endpoint (§2 order and bounds).
//   plan_scan_kernel        §4.5 count scan into exact exclusive offsets plus
//                           the 8-value allocation header.
//   plan_sched_*_kernel     §4.8 forward schedule by bounded counting:
//                           histogram over (section, cost), one-workgroup
//                           scan of bucket offsets, one wavefront per section
//                           scattering its tasks in tie order, then the
//                           section-interleaved launch order with one record
//                           per task.
//   plan_materialize_kernel §4.6 / §5 Q2K materialisation: ascending partial
//                           and full K-tile indices plus one packed predicate
//                           per partial tile.
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

__device__ inline uint32_t range_bits(int lo, int hi) {
  // bits [lo, hi) of a 32-bit word, 0 <= lo < hi <= 32
  uint32_t upto = hi >= 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u);
  return upto & ~((1u << lo) - 1u);
}

// Reads interval p of one row: p = 0 is [0, F0); p >= 1 is [F(2p-1), F(2p)).
struct RowIntervals {
  const int32_t* col;   // &mask_func[hm][0][token]
  int64_t stride;       // total_q
  __device__ inline void get(int p, int& s, int& e) const {
    if (p == 0) {
      s = 0;
      e = col[0];
    } else {
      s = col[(int64_t)(2 * p - 1) * stride];
      e = col[(int64_t)(2 * p) * stride];
    }
  }
};

// Monotone sweep over one row's intervals: count(x) = number of visible k < x.
struct CountSweep {
  int p, cum, s, e;
  __device__ inline void init(const RowIntervals& r, int nint) {
    p = 0;
    cum = 0;
    r.get(0, s, e);
    (void)nint;
  }
  __device__ inline int count_below(const RowIntervals& r, int nint, int x) {
    while (p < nint && e <= x) {
      cum += max(0, e - s);
      ++p;
      if (p < nint) r.get(p, s, e);
    }
    int v = cum;
    if (p < nint) v += min(max(x - s, 0), max(0, e - s));
    return v;
  }
};

}  // namespace

// ---------------------------------------------------------------- geometry

__global__ __launch_bounds__(1024) void plan_geometry_kernel(PlanGeo g, const int32_t* cu_q,
                                                             const int32_t* cu_k, PlanDev d) {
  __shared__ int s_bad;
  __shared__ int s_carry;
  __shared__ int s_scan[1024];
  const int tid = threadIdx.x;
  const int B = g.batch;
  if (tid < 8) d.header[tid] = 0;
  if (tid == 0) {
    s_bad = 0;
    s_carry = 0;
  }
  __syncthreads();
  if (g.layout == MPB_LAYOUT_THD) {
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
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  // With a bad prefix every sample is given zero length, so later stages see
  // no rows and touch nothing; the error bit makes the build fail.
  for (int base = 0; base < B; base += blockDim.x) {
    const int b = base + tid;
    int q_off = 0, q_len = 0, k_off = 0, k_len = 0;
    if (b < B && !bad) {
      if (g.layout == MPB_LAYOUT_BSHD) {
        q_off = b * g.seqlen_q;
        q_len = g.seqlen_q;
        k_off = b * g.seqlen_k;
        k_len = g.seqlen_k;
      } else {
        q_off = cu_q[b];
        q_len = cu_q[b + 1] - q_off;
        k_off = cu_k[b];
        k_len = cu_k[b + 1] - k_off;
      }
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
    if (bad) d.header[7] = MPB_DEVERR_SEQLENS;
  }
}

// ---------------------------------------------------------------- classify

template <int RPL>
__global__ __launch_bounds__(256) void plan_classify_kernel(PlanGeo g,
                                                            const int32_t* __restrict__ mf,
                                                            PlanDev d, PlanWork w) {
  const int lane = wave_lane();
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int hm = item / g.upper_rows;
  const int row = item - hm * g.upper_rows;
  if (hm >= g.mask_heads) return;
  const int rows_total = d.cu_rows[g.batch];
  if (row >= rows_total) return;
  const int b = sample_of_row(d.cu_rows, g.batch, row);
  const int32_t* sd = d.seqdesc + 8 * b;
  const int q_off = sd[0], q_len = sd[2], k_len = sd[3], nk = sd[6];
  const int i = row - sd[4];
  const int nint = (g.nfunc + 1) >> 1;

  bool valid[RPL];
  RowIntervals ri[RPL];
  for (int t = 0; t < RPL; ++t) {
    const int rho = lane + 64 * t;
    valid[t] = rho < g.tile_q && i * g.tile_q + rho < q_len;
    const int64_t tok = (int64_t)q_off + (int64_t)i * g.tile_q + rho;
    ri[t].col = mf + (int64_t)hm * g.nfunc * g.total_q + (valid[t] ? tok : 0);
    ri[t].stride = g.total_q;
  }

  // §2 / §4.3: every endpoint in [0, k_len] and nondecreasing.  Loads are
  // coalesced: all lanes read endpoint f of consecutive tokens.
  uint32_t err = 0;
  {
    int prev[RPL];
    for (int f = 0; f < g.nfunc; ++f) {
      for (int t = 0; t < RPL; ++t) {
        if (!valid[t]) continue;
        const int F = ri[t].col[(int64_t)f * g.total_q];
        if (F < 0 || F > k_len) err |= MPB_DEVERR_RANGE;
        if (f > 0 && F < prev[t]) err |= MPB_DEVERR_ORDER;
        prev[t] = F;
      }
    }
  }
  const uint64_t any_range = __ballot((err & MPB_DEVERR_RANGE) != 0);
  const uint64_t any_order = __ballot((err & MPB_DEVERR_ORDER) != 0);
  if (lane == 0 && (any_range | any_order)) {
    atomicOr(&d.header[7], (any_range ? MPB_DEVERR_RANGE : 0) | (any_order ? MPB_DEVERR_ORDER : 0));
  }

  // §4.3 three states per (row tile, K tile).  A lane's visible count in
  // tile j is count(c1) - count(c0) of its row; a tile is full only if the
  // whole T_Q x T_KV tile is in bounds and every element is visible.
  CountSweep sw[RPL];
  int prevc[RPL];
  for (int t = 0; t < RPL; ++t) {
    if (valid[t]) sw[t].init(ri[t], nint);
    prevc[t] = 0;
  }
  const bool rows_in_bounds = (i + 1) * g.tile_q <= q_len;
  uint32_t vword = 0, fword = 0;
  int pc = 0, fc = 0;
  const int64_t wbase = ((int64_t)hm * g.upper_rows + row) * g.words_k;
  for (int j = 0; j < nk; ++j) {
    const int c0 = j * g.tile_k;
    const int c1 = min(c0 + g.tile_k, k_len);
    bool any_vis = false, all_vis = true;
    for (int t = 0; t < RPL; ++t) {
      if (!valid[t]) continue;
      const int c = sw[t].count_below(ri[t], nint, c1);
      const int cnt = c - prevc[t];
      prevc[t] = c;
      any_vis |= cnt > 0;
      all_vis &= cnt == g.tile_k;
    }
    const bool tile_any = __ballot(any_vis) != 0;
    const bool tile_full = tile_any && rows_in_bounds && (c0 + g.tile_k <= k_len) &&
                           __ballot(!all_vis) == 0;
    vword |= (uint32_t)tile_any << (j & 31);
    fword |= (uint32_t)tile_full << (j & 31);
    pc += (tile_any && !tile_full) ? 1 : 0;
    fc += tile_full ? 1 : 0;
    if ((j & 31) == 31 || j == nk - 1) {
      if (lane == 0) {
        w.vis_bits[wbase + (j >> 5)] = vword;
        w.full_bits[wbase + (j >> 5)] = fword;
      }
      vword = 0;
      fword = 0;
    }
  }
  if (lane == 0) {
    w.pcnt[(int64_t)hm * g.upper_rows + row] = pc;
    w.fcnt[(int64_t)hm * g.upper_rows + row] = fc;
  }
}

// ---------------------------------------------------------------- scan + header

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

__global__ __launch_bounds__(1024) void plan_scan_kernel(PlanGeo g, PlanDev d, PlanWork w) {
  __shared__ int sa[1024], sb[1024];
  __shared__ int carry_p, carry_f;
  const int tid = threadIdx.x;
  const int rows_total = d.cu_rows[g.batch];
  const int n = g.mask_heads * rows_total;
  if (tid == 0) {
    carry_p = 0;
    carry_f = 0;
  }
  __syncthreads();
  // §4.5: off[0] = 0, off[i+1] = off[i] + cnt[i], over rows flattened
  // head-major (flat = hm * rows_total + row).
  for (int base = 0; base < n; base += 1024) {
    const int idx = base + tid;
    int a = 0, c = 0;
    if (idx < n) {
      const int hm = idx / rows_total;
      const int r = idx - hm * rows_total;
      a = w.pcnt[(int64_t)hm * g.upper_rows + r];
      c = w.fcnt[(int64_t)hm * g.upper_rows + r];
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
  if (tid == 0) {
    w.p_off_tmp[n] = carry_p;
    w.f_off_tmp[n] = carry_f;
    d.header[0] = rows_total;
    d.header[1] = carry_p;
    d.header[2] = carry_f;
  }
  const int nbins = kNumQueues * (g.nk_max + 1);
  for (int x = tid; x < nbins; x += 1024) w.bins[x] = 0;
}

// ---------------------------------------------------------------- schedule

namespace {

struct TaskInfo {
  int b, h, i, rows_b, cost;
};

__device__ inline TaskInfo decode_task(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                       int t) {
  // Canonical tie order: t = Hq*cu_rows[b] + h*rows_b + i.
  TaskInfo r;
  r.b = sample_of_row(d.cu_rows, g.batch, t / g.heads_q);
  const int r0 = d.cu_rows[r.b];
  r.rows_b = d.cu_rows[r.b + 1] - r0;
  const int rel = t - g.heads_q * r0;
  r.h = rel / r.rows_b;
  r.i = rel - r.h * r.rows_b;
  const int hm = g.mask_heads == 1 ? 0 : r.h;
  const int64_t src = (int64_t)hm * g.upper_rows + r0 + r.i;
  r.cost = w.pcnt[src] + w.fcnt[src];
  return r;
}

__device__ inline int task_section(const PlanGeo& g, int b, int h, int cost) {
  if (cost == 0) return kNumSections;
  const int group = g.heads_q / g.heads_k;
  return (b * g.heads_k + h / group) % kNumSections;
}

__device__ inline int task_bin(const PlanGeo& g, int sec, int cost) {
  // Buckets in final order: section ascending, then cost descending.
  return sec * (g.nk_max + 1) + (g.nk_max - cost);
}

}  // namespace

__global__ __launch_bounds__(256) void plan_sched_hist_kernel(PlanGeo g, PlanDev d, PlanWork w) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int ntasks = d.cu_rows[g.batch] * g.heads_q;
  if (t >= ntasks) return;
  const TaskInfo ti = decode_task(g, d, w, t);
  atomicAdd(&w.bins[task_bin(g, task_section(g, ti.b, ti.h, ti.cost), ti.cost)], 1);
}

__global__ __launch_bounds__(1024) void plan_sched_offsets_kernel(PlanGeo g, PlanDev d,
                                                                  PlanWork w) {
  __shared__ int sa[1024], sb[1024];
  __shared__ int carry;
  const int tid = threadIdx.x;
  const int per = g.nk_max + 1;
  const int nbins = kNumQueues * per;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nbins; base += 1024) {
    const int x = base + tid;
    const int c = x < nbins ? w.bins[x] : 0;
    sa[tid] = c;
    sb[tid] = 0;
    __syncthreads();
    block_incl_scan2(sa, sb, tid, 1024);
    const int excl = carry + sa[tid] - c;
    if (x < nbins) {
      w.bins[x] = excl;  // becomes the bucket's write cursor
      if (x % per == 0) d.section_off[x / per] = excl;
    }
    __syncthreads();
    if (tid == 1023) carry += sa[1023];
    __syncthreads();
  }
  if (tid == 0) d.section_off[kNumQueues] = carry;
}

// One wavefront per queue.  Section s walks the (batch, head) pairs that map
// to it in canonical order and scatters each 64-task chunk: lanes with equal
// buckets are grouped by ballot, ranked by lane order, and reserve their slots
// with one atomic on the bucket cursor, so each bucket keeps tie order.
__global__ __launch_bounds__(64) void plan_sched_scatter_kernel(PlanGeo g, PlanDev d,
                                                                PlanWork w) {
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const int group = g.heads_q / g.heads_k;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int zero_cursor = (s == kNumSections) ? d.section_off[kNumSections] : 0;
  for (int b = 0; b < g.batch; ++b) {
    const int r0 = d.cu_rows[b];
    const int rows_b = d.cu_rows[b + 1] - r0;
    if (rows_b == 0) continue;
    const int32_t* sd = d.seqdesc + 8 * b;
    const int q_len = sd[2];
    for (int h = 0; h < g.heads_q; ++h) {
      if (s < kNumSections && (b * g.heads_k + h / group) % kNumSections != s) continue;
      const int hm = g.mask_heads == 1 ? 0 : h;
      for (int i0 = 0; i0 < rows_b; i0 += 64) {
        const int i = i0 + lane;
        int cost = 0;
        if (i < rows_b) {
          const int64_t src = (int64_t)hm * g.upper_rows + r0 + i;
          cost = w.pcnt[src] + w.fcnt[src];
        }
        const int qvalid = min(g.tile_q, q_len - i * g.tile_q);
        if (s == kNumSections) {
          const bool mine = i < rows_b && cost == 0;
          const uint64_t m = __ballot(mine);
          if (mine) {
            int32_t* wd = d.work_desc + 4 * (int64_t)(zero_cursor + __popcll(m & lt));
            wd[0] = i; wd[1] = h; wd[2] = b; wd[3] = qvalid;
          }
          zero_cursor += __popcll(m);
        } else {
          bool mine = i < rows_b && cost > 0;
          const int key = task_bin(g, s, cost);
          while (true) {
            const uint64_t m = __ballot(mine);
            if (m == 0) break;
            const int leader = __ffsll((unsigned long long)m) - 1;
            const int k0 = __shfl(key, leader);
            const bool same = mine && key == k0;
            const uint64_t match = __ballot(same);
            int base = 0;
            if (lane == leader) base = atomicAdd(&w.bins[k0], __popcll(match));
            base = __shfl(base, leader);
            if (same) {
              int32_t* wd = d.work_desc + 4 * (int64_t)(base + __popcll(match & lt));
              wd[0] = i; wd[1] = h; wd[2] = b; wd[3] = qvalid;
              mine = false;
            }
          }
        }
      }
    }
  }
}

// Launch order and task records.  Task t of the section-major schedule has
// rank r in its section s; its launch slot interleaves the sections:
// slot = sum_s' min(r, n_s') + #{s' < s : n_s' > r}; zero-cost tasks follow
// all positive-cost ones.  Each record carries everything a forward
// workgroup needs (see TaskRecField), so the attention kernel starts its
// Q and first K/V loads after a single record read.
__global__ __launch_bounds__(256) void plan_sched_records_kernel(PlanGeo g, PlanDev d,
                                                                 PlanWork w) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int rows_total = d.cu_rows[g.batch];
  const int ntasks = rows_total * g.heads_q;
  if (t >= ntasks) return;
  int s = 0;
  while (s < kNumSections && t >= d.section_off[s + 1]) ++s;
  const int r = t - d.section_off[s];
  int slot;
  if (s < kNumSections) {
    slot = 0;
    for (int s2 = 0; s2 < kNumSections; ++s2) {
      const int n2 = d.section_off[s2 + 1] - d.section_off[s2];
      slot += min(r, n2) + ((s2 < s && n2 > r) ? 1 : 0);
    }
  } else {
    slot = d.section_off[kNumSections] + r;
  }
  const int32_t* wd = d.work_desc + 4 * (int64_t)t;
  const int m_block = wd[0], h = wd[1], b = wd[2];
  const int32_t* sd = d.seqdesc + 8 * b;
  const int row = sd[4] + m_block;
  const int hm = g.mask_heads == 1 ? 0 : h;
  const int64_t flat = (int64_t)hm * rows_total + row;
  const int64_t src = (int64_t)hm * g.upper_rows + row;
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
  int32_t* rec = d.task_rec + (int64_t)slot * kTaskRecInts;
  rec[kRecMBlock] = m_block;
  rec[kRecHead] = h;
  rec[kRecBatch] = b;
  rec[kRecQValid] = wd[3];
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
  rec[kRecKvHead] = h / (g.heads_q / g.heads_k);
  rec[kRecSection] = s;
}

// ---------------------------------------------------------------- materialize

namespace {

// Predicate word of one row for columns [x0, x0+32): OR over the row's
// intervals of their overlap with the window; columns >= k_len stay 0.
struct WordSweep {
  int p, s, e;
  __device__ inline void init(const RowIntervals& r) {
    p = 0;
    r.get(0, s, e);
  }
  __device__ inline uint32_t word(const RowIntervals& r, int nint, int x0, int k_len) {
    const int x1 = min(x0 + 32, k_len);
    if (x1 <= x0) return 0u;
    while (p < nint && e <= x0) {
      ++p;
      if (p < nint) r.get(p, s, e);
    }
    uint32_t wbits = 0u;
    int q = p, qs = s, qe = e;
    while (q < nint && qs < x1) {
      const int lo = max(qs, x0), hi = min(qe, x1);
      if (hi > lo) wbits |= range_bits(lo - x0, hi - x0);
      ++q;
      if (q < nint) r.get(q, qs, qe);
    }
    return wbits;
  }
};

}  // namespace

template <int RPL>
__global__ __launch_bounds__(256) void plan_materialize_kernel(PlanGeo g,
                                                               const int32_t* __restrict__ mf,
                                                               PlanDev d, PlanWork w,
                                                               int rows_total) {
  const int lane = wave_lane();
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = g.mask_heads * rows_total;
  if (item == 0 && lane == 0) {
    d.p_off[n] = w.p_off_tmp[n];
    d.f_off[n] = w.f_off_tmp[n];
  }
  if (item >= n) return;
  const int hm = item / rows_total;
  const int row = item - hm * rows_total;
  const int b = sample_of_row(d.cu_rows, g.batch, row);
  const int32_t* sd = d.seqdesc + 8 * b;
  const int q_off = sd[0], q_len = sd[2], k_len = sd[3], nk = sd[6];
  const int i = row - sd[4];
  const int nint = (g.nfunc + 1) >> 1;
  const int64_t src = (int64_t)hm * g.upper_rows + row;
  const int p_begin = w.p_off_tmp[item];
  const int f_begin = w.f_off_tmp[item];
  if (lane == 0) {
    d.p_off[item] = p_begin;
    d.f_off[item] = f_begin;
  }
  // §4.6: sample-local K-tile indices, ascending, partial and full apart.
  const int nwords = (nk + 31) >> 5;
  int pb = p_begin, fb = f_begin;
  for (int ww = 0; ww < nwords; ++ww) {
    const uint32_t vw = w.vis_bits[src * g.words_k + ww];
    const uint32_t fw = w.full_bits[src * g.words_k + ww];
    const uint32_t pw = vw & ~fw;
    if (lane < 32) {
      const uint32_t bit = 1u << lane;
      const uint32_t below = bit - 1u;
      if (pw & bit) d.p_idx[pb + __popc(pw & below)] = 32 * ww + lane;
      if (fw & bit) d.f_idx[fb + __popc(fw & below)] = 32 * ww + lane;
    }
    pb += __popc(pw);
    fb += __popc(fw);
  }
  // §5: one predicate bit per score element of each partial tile; word
  // [r][c/32], bit c%32; rows past q_len and columns past k_len are 0.
  bool valid[RPL];
  RowIntervals ri[RPL];
  WordSweep sw[RPL];
  for (int t = 0; t < RPL; ++t) {
    const int rho = lane + 64 * t;
    valid[t] = rho < g.tile_q && i * g.tile_q + rho < q_len;
    const int64_t tok = (int64_t)q_off + (int64_t)i * g.tile_q + rho;
    ri[t].col = mf + (int64_t)hm * g.nfunc * g.total_q + (valid[t] ? tok : 0);
    ri[t].stride = g.total_q;
    if (valid[t]) sw[t].init(ri[t]);
  }
  int pos = p_begin;
  for (int ww = 0; ww < nwords; ++ww) {
    uint32_t pw = w.vis_bits[src * g.words_k + ww] & ~w.full_bits[src * g.words_k + ww];
    while (pw) {
      const int jb = __ffs(pw) - 1;
      pw &= pw - 1u;
      const int c0 = (32 * ww + jb) * g.tile_k;
      uint32_t* dst = d.p_masks + (int64_t)pos * g.tile_q * g.words_tile;
      for (int t = 0; t < RPL; ++t) {
        const int rho = lane + 64 * t;
        if (rho >= g.tile_q) continue;
        for (int x = 0; x < g.words_tile; ++x) {
          const uint32_t word = valid[t] ? sw[t].word(ri[t], nint, c0 + 32 * x, k_len) : 0u;
          dst[(int64_t)rho * g.words_tile + x] = word;
        }
      }
      ++pos;
    }
  }
}

// ---------------------------------------------------------------- launchers

static inline int rows_per_lane(int tile_q) { return tile_q <= 64 ? 1 : tile_q / 64; }

hipError_t launch_plan_geometry(const PlanGeo& g, const int32_t* cu_q_in, const int32_t* cu_k_in,
                                const PlanDev& d, hipStream_t s) {
  hipLaunchKernelGGL(plan_geometry_kernel, dim3(1), dim3(1024), 0, s, g, cu_q_in, cu_k_in, d);
  return hipGetLastError();
}

hipError_t launch_plan_classify(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                                const PlanWork& w, hipStream_t s) {
  const int64_t items = (int64_t)g.mask_heads * g.upper_rows;
  if (items == 0) return hipSuccess;
  const dim3 grid((unsigned)((items + 3) / 4));
  switch (rows_per_lane(g.tile_q)) {
    case 1: hipLaunchKernelGGL(plan_classify_kernel<1>, grid, dim3(256), 0, s, g, mask_func, d, w); break;
    case 2: hipLaunchKernelGGL(plan_classify_kernel<2>, grid, dim3(256), 0, s, g, mask_func, d, w); break;
    case 4: hipLaunchKernelGGL(plan_classify_kernel<4>, grid, dim3(256), 0, s, g, mask_func, d, w); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_plan_scan(const PlanGeo& g, const PlanDev& d, const PlanWork& w, hipStream_t s) {
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, s, g, d, w);
  return hipGetLastError();
}

hipError_t launch_plan_schedule(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                int32_t upper_tasks, hipStream_t s) {
  if (upper_tasks > 0) {
    hipLaunchKernelGGL(plan_sched_hist_kernel, dim3((upper_tasks + 255) / 256), dim3(256), 0, s,
                       g, d, w);
  }
  hipLaunchKernelGGL(plan_sched_offsets_kernel, dim3(1), dim3(1024), 0, s, g, d, w);
  hipLaunchKernelGGL(plan_sched_scatter_kernel, dim3(kNumQueues), dim3(64), 0, s, g, d, w);
  if (upper_tasks > 0) {
    hipLaunchKernelGGL(plan_sched_records_kernel, dim3((upper_tasks + 255) / 256), dim3(256), 0,
                       s, g, d, w);
  }
  return hipGetLastError();
}

hipError_t launch_plan_materialize(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                                   const PlanWork& w, int32_t rows_total, hipStream_t s) {
  const int64_t items = (int64_t)g.mask_heads * rows_total;
  const dim3 grid((unsigned)((items > 0 ? items + 3 : 4) / 4));
  switch (rows_per_lane(g.tile_q)) {
    case 1: hipLaunchKernelGGL(plan_materialize_kernel<1>, grid, dim3(256), 0, s, g, mask_func, d, w, rows_total); break;
    case 2: hipLaunchKernelGGL(plan_materialize_kernel<2>, grid, dim3(256), 0, s, g, mask_func, d, w, rows_total); break;
    case 4: hipLaunchKernelGGL(plan_materialize_kernel<4>, grid, dim3(256), 0, s, g, mask_func, d, w, rows_total); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mpb
