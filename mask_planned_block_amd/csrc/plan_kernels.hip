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
//                           touching intervals and ORs / ANDs the K tiles each
//                           run touches / fully covers across the wavefront:
//                           any row touching a tile makes it visible, all T_Q
//                           rows covering it make it full.  The workgroup
//                           that finishes last then computes the §4.5 exact
//                           CSR offsets and the 8-value allocation header
//                           (device errors OR-ed in) and publishes the header
//                           to host-mapped memory.
//   plan_schedule_kernel    one workgroup: §4.8 the forward schedule by
//                           bounded counting (cost ranks, per-section scans)
//                           and the section-interleaved launch records; runs
//                           while the host reads the header and allocates.
//   plan_materialize_kernel §4.6 / §5 Q2K materialisation: ascending partial
//                           and full K-tile indices, and one predicate word per
//                           (row, 32 columns) of each partial tile.
//
// Visibility used throughout: with sorted endpoints F, column k is visible iff
// an even number of endpoints are <= k (k < F0: none; F0 <= k < F1: one, ...),
// which is the union [0,F0) U [F1,F2) U ... of §2; columns >= F(nfunc-1)
// (hence >= k_len) see an odd count and are masked.
#include <algorithm>
#include <climits>

#include "mpb_internal.h"
#include "../../include/mpb.h"

namespace mpb {

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// LDS-typed pointers: code that chooses between an LDS copy and the HBM
// original at run time takes one branch per type, so neither becomes a flat
// access.
typedef __attribute__((address_space(3))) int32_t* lds_ptr;
typedef __attribute__((address_space(3))) const int32_t* lds_cptr;

template <class P>
__device__ inline int sample_of_row(P cu_rows, int batch, int row) {
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

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP moves:
// shifts by 1, 2, 4, 8 inside each row of 16 lanes, then row 0's last lane
// is broadcast into row 1 and row 2's into row 3, then lane 31 into rows 2
// and 3.  Lanes a move has no source for receive 0.
__device__ inline int wave_incl_scan(int v, int /*lane*/) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Sum over the wavefront, in every lane.
__device__ inline int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v, 0), 63);
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

// OR tiles [t0, t1) into the window of WW 32-bit words starting at tile tg.
template <int WW>
__device__ inline void set_tiles(uint32_t (&m)[WW], int t0, int t1, int tg) {
#pragma unroll
  for (int x = 0; x < WW; ++x) {
    const int w0 = tg + 32 * x;
    const int lo = max(t0, w0), hi = min(t1, w0 + 32);
    if (hi > lo) m[x] |= range_bits(lo - w0, hi - w0);
  }
}

// OR / AND over the wavefront (same DPP pattern as the scan; lanes without a
// source receive the identity), in every lane.
__device__ inline uint32_t wave_or(uint32_t x) {
  int v = (int)x;
  v |= __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v |= __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v |= __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v |= __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v |= __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v |= __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}
__device__ inline int wave_min(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x111, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x112, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x114, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x118, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x142, 0xa, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ inline uint32_t wave_and(uint32_t x) {
  int v = (int)x;
  v &= __builtin_amdgcn_update_dpp(-1, v, 0x111, 0xf, 0xf, false);
  v &= __builtin_amdgcn_update_dpp(-1, v, 0x112, 0xf, 0xf, false);
  v &= __builtin_amdgcn_update_dpp(-1, v, 0x114, 0xf, 0xf, false);
  v &= __builtin_amdgcn_update_dpp(-1, v, 0x118, 0xf, 0xf, false);
  v &= __builtin_amdgcn_update_dpp(-1, v, 0x142, 0xa, 0xf, false);
  v &= __builtin_amdgcn_update_dpp(-1, v, 0x143, 0xc, 0xf, false);
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

// Classification of one (mask head, Q plan row): one wavefront, lanes own rows
// lane + 64t.  Tiles are handled in windows of 32*WW (WW 32-bit words; 4 when
// a sample has at most 128 K tiles, else 8, so the 256 tiles of an 8192-key
// sample at 32-wide tiles take one pass over the endpoints): for
// each window a lane walks its rows' intervals, 64/RPL at a time with the
// loads of all its rows issued together (coalesced across lanes, so a row's
// intervals cost one memory round trip per batch), merges touching
// intervals into runs, and ORs the tiles each run touches ("any") or fully
// covers ("full") into its words.  Across the wavefront the "any" words are
// OR-ed and the "full" words AND-ed: a tile is visible if any row sees part
// of it and full if every one of the T_Q rows covers it, which needs every
// row in bounds (rows past q_len contribute nothing) and the tile inside
// k_len (no run extends past k_len).  §2 order and bounds of every endpoint
// are checked on the way.
template <int RPL, int WW>
__device__ inline void classify_row(const PlanGeo& g, const int32_t* __restrict__ mf,
                                    const PlanDev& d, const PlanWork& w, int hm, int row,
                                    int lane) {
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
  int pc = 0, fc = 0, first_p = -1, first_f = -1;
  const int64_t wbase = ((int64_t)hm * g.upper_rows + row) * g.words_k;
  for (int tg = 0; tg < nk; tg += 32 * WW) {
    uint32_t any_m[WW], rf[RPL][WW];
#pragma unroll
    for (int x = 0; x < WW; ++x) {
      any_m[x] = 0u;
#pragma unroll
      for (int t = 0; t < RPL; ++t) rf[t][x] = 0u;
    }
    // open run per row, empty when run_b <= run_a; last endpoint seen
    int run_a[RPL], run_b[RPL], prev[RPL];
#pragma unroll
    for (int t = 0; t < RPL; ++t) run_a[t] = run_b[t] = prev[t] = 0;
    // A run [a, b) touches tiles a/T .. (b-1)/T and fully covers
    // ceil(a/T) .. b/T - 1 (clamped to [0, nk] for malformed input).
    auto flush = [&](int t, int a, int b) {
      if (b <= a) return;
      const int t0 = min(max(a / T, 0), nk), t1 = min(max((b - 1) / T + 1, 0), nk);
      set_tiles(any_m, t0, t1, tg);
      const int f0 = min(max((a + T - 1) / T, 0), nk), f1 = min(max(b / T, 0), nk);
      set_tiles(rf[t], f0, f1, tg);
    };
    constexpr int kBatch = 16 / RPL;   // intervals per lane in flight
    for (int p0 = 0; p0 < nint; p0 += kBatch) {
      int sv[RPL][kBatch], ev[RPL][kBatch];
#pragma unroll
      for (int t = 0; t < RPL; ++t)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int p = p0 + u;
          sv[t][u] = 0;
          ev[t][u] = 0;
          if (valid[t] && p < nint) {
            if (p > 0) sv[t][u] = col[t][(int64_t)(2 * p - 1) * g.total_q];
            ev[t][u] = col[t][(int64_t)(2 * p) * g.total_q];
          }
        }
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        if (!valid[t]) continue;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int p = p0 + u;
          if (p >= nint) break;
          const int s = sv[t][u], e = ev[t][u];
          if (tg == 0) {
            if (p > 0) {
              if (s < prev[t]) err |= MPB_DEVERR_ORDER;
              if (s < 0 || s > rg.k_len) err |= MPB_DEVERR_RANGE;
            }
            if (e < s) err |= MPB_DEVERR_ORDER;
            if (e < 0 || e > rg.k_len) err |= MPB_DEVERR_RANGE;
          }
          prev[t] = e;
          if (e <= s) continue;                 // empty interval
          if (run_b[t] > run_a[t] && s == run_b[t]) {
            run_b[t] = e;                       // touching: extend the run
          } else {
            flush(t, run_a[t], run_b[t]);
            run_a[t] = s;
            run_b[t] = e;
          }
        }
      }
    }
    uint32_t full_m[WW];
#pragma unroll
    for (int x = 0; x < WW; ++x) full_m[x] = ~0u;   // AND identity
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
      if (!exists[t]) continue;                 // not a row of the tile
      if (valid[t]) flush(t, run_a[t], run_b[t]);
#pragma unroll
      for (int x = 0; x < WW; ++x) full_m[x] &= rf[t][x];
    }
    uint32_t vis_w[WW], full_w[WW];
#pragma unroll
    for (int x = 0; x < WW; ++x) {
      vis_w[x] = wave_or(any_m[x]);
      full_w[x] = wave_and(full_m[x]);
      const int w0 = tg + 32 * x;
      const uint32_t live = w0 >= nk ? 0u : (nk - w0 >= 32 ? ~0u : ((1u << (nk - w0)) - 1u));
      vis_w[x] &= live;
      full_w[x] &= vis_w[x];
      const uint32_t part = vis_w[x] & ~full_w[x];
      pc += __popc(part);
      fc += __popc(full_w[x]);
      if (first_p < 0 && part) first_p = w0 + __ffs(part) - 1;
      if (first_f < 0 && full_w[x]) first_f = w0 + __ffs(full_w[x]) - 1;
    }
    // lane x < WW stores word x of the window (values are uniform)
    uint32_t my_vis = 0, my_full = 0;
#pragma unroll
    for (int x = 0; x < WW; ++x) {
      my_vis = lane == x ? vis_w[x] : my_vis;
      my_full = lane == x ? full_w[x] : my_full;
    }
    if (lane < WW && tg + 32 * lane < nk) {
      w.vis_bits[wbase + ((tg + 32 * lane) >> 5)] = my_vis;
      w.full_bits[wbase + ((tg + 32 * lane) >> 5)] = my_full;
    }
  }
  const uint64_t er = __ballot((err & MPB_DEVERR_RANGE) != 0);
  const uint64_t eo = __ballot((err & MPB_DEVERR_ORDER) != 0);
  if (lane == 0) {
    const int64_t it = (int64_t)hm * g.upper_rows + row;
    w.pcnt[it] = pc;
    w.fcnt[it] = fc;
    w.first_tile[it] = pc > 0 ? first_p : first_f;   // the partial list is traversed first
    w.item_err[it] = (er ? MPB_DEVERR_RANGE : 0) | (eo ? MPB_DEVERR_ORDER : 0);
  }
}

// §4.5 after classification, by the last workgroup of the classify launch:
// exact exclusive CSR offsets over rows flattened head-major
// (flat = hm * rows_total + row; off[0] = 0, off[i+1] = off[i] + cnt[i]) and
// the 8-value allocation header {rows, partial blocks, full blocks, 0, 0, 0,
// 0, OR of every device error bit}.  The header goes to the plan and to the
// host-mapped slot, its values first and the build's sequence number last,
// so the host can read it the moment it lands.  Four values per thread, a
// wavefront scan of the thread sums and a pass over the NT/64 wavefront
// totals in LDS.
template <int NT>
__device__ inline void publish_offsets(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                       int32_t* host_slot, int32_t seq, int* s_wp, int* s_wf,
                                       uint32_t* s_err) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rows_total = rows_total_of(g, d);
  const int n = g.mask_heads * rows_total;
  uint32_t err = 0;
  int carry_p = 0, carry_f = 0;
  for (int base = 0; base < n; base += 4 * NT) {
    const int i0 = base + 4 * tid;
    int vp[4], vf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u;
      vp[u] = 0;
      vf[u] = 0;
      if (i < n) {
        const int hm = i / rows_total;
        const int64_t src = (int64_t)hm * g.upper_rows + (i - hm * rows_total);
        vp[u] = w.pcnt[src];
        vf[u] = w.fcnt[src];
        err |= (uint32_t)w.item_err[src];
      }
    }
    const int tp = vp[0] + vp[1] + vp[2] + vp[3];
    const int tf = vf[0] + vf[1] + vf[2] + vf[3];
    const int ip = wave_incl_scan(tp, lane);
    const int jf = wave_incl_scan(tf, lane);
    if (lane == 63) {
      s_wp[wv] = ip;
      s_wf[wv] = jf;
    }
    __syncthreads();
    int pre_p = 0, pre_f = 0, tot_p = 0, tot_f = 0;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      const int a = s_wp[x], c = s_wf[x];
      if (x < wv) {
        pre_p += a;
        pre_f += c;
      }
      tot_p += a;
      tot_f += c;
    }
    int run_p = carry_p + pre_p + ip - tp, run_f = carry_f + pre_f + jf - tf;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + u < n) {
        w.p_off_tmp[i0 + u] = run_p;
        w.f_off_tmp[i0 + u] = run_f;
      }
      run_p += vp[u];
      run_f += vf[u];
    }
    carry_p += tot_p;
    carry_f += tot_f;
    __syncthreads();  // s_wp / s_wf are reused
  }
  if (tid == 0 && g.layout == MPB_LAYOUT_THD) err |= (uint32_t)w.geo_err[0];
  if (err) atomicOr(s_err, err);
  __syncthreads();
  if (tid == 0) {
    w.p_off_tmp[n] = carry_p;
    w.f_off_tmp[n] = carry_f;
    const int32_t hdr[8] = {rows_total, carry_p, carry_f, 0, 0, 0, 0, (int32_t)*s_err};
    for (int i = 0; i < 8; ++i) {
      d.header[i] = hdr[i];
      __hip_atomic_store(&host_slot[i], hdr[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    __hip_atomic_store(&host_slot[kHeaderSeq], seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace

// §4.3 Q2K classification, one wavefront per (mask head, Q plan row), then
// §4.5 offsets and header by whichever workgroup finishes last: every
// workgroup makes its results visible device-wide and takes a ticket from
// `arrive`; the one that draws the last ticket resets the counter, sees
// every other workgroup's results and runs publish_offsets.  No workgroup
// waits for another, so the grid always drains.
template <int RPL, int WW>
__global__ __launch_bounds__(256) void plan_classify_kernel(PlanGeo g,
                                                            const int32_t* __restrict__ mf,
                                                            PlanDev d, PlanWork w, int32_t* arrive,
                                                            int32_t* host_slot, int32_t seq) {
  __shared__ int s_last;
  __shared__ int s_wp[4], s_wf[4];
  __shared__ uint32_t s_err;
  const int lane = wave_lane();
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g.upper_rows > 0) {
    const int hm = item / g.upper_rows;
    const int row = item - hm * g.upper_rows;
    if (hm < g.mask_heads && row < rows_total_of(g, d))
      classify_row<RPL, WW>(g, mf, d, w, hm, row, lane);
  }

  // Every wavefront waits for its stores to complete; the workgroup's ticket
  // is then taken with release semantics (writing the device caches back
  // once per workgroup), and only the last workgroup acquires.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (int)gridDim.x - 1 ? 1 : 0;
    s_err = 0;
  }
  __syncthreads();
  if (!s_last) return;
  __atomic_thread_fence(__ATOMIC_ACQUIRE);   // agent scope: sees every workgroup's results
  if (threadIdx.x == 0) __hip_atomic_store(arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  publish_offsets<256>(g, d, w, host_slot, seq, s_wp, s_wf, &s_err);
}

// ---------------------------------------------------------------- schedule

namespace {

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

struct SampleGeo {
  int b, row_begin, q_off, k_off, q_len, k_len;
};

// Sample of a plan row; `s_cu` is an LDS copy of cu_rows (THD) or nullptr.
__device__ inline SampleGeo sample_geo(const PlanGeo& g, const PlanDev& d, const int* s_cu,
                                       int row) {
  SampleGeo r;
  if (g.layout == MPB_LAYOUT_BSHD) {
    const int rps = (g.seqlen_q + g.tile_q - 1) / g.tile_q;
    r.b = row / rps;
    r.row_begin = r.b * rps;
    r.q_off = r.b * g.seqlen_q;
    r.k_off = r.b * g.seqlen_k;
    r.q_len = g.seqlen_q;
    r.k_len = g.seqlen_k;
  } else {
    r.b = s_cu ? sample_of_row((lds_cptr)s_cu, g.batch, row)
               : sample_of_row(d.cu_rows, g.batch, row);
    const int32_t* sd = d.seqdesc + 8 * r.b;
    r.q_off = sd[0];
    r.k_off = sd[1];
    r.q_len = sd[2];
    r.k_len = sd[3];
    r.row_begin = sd[4];
  }
  return r;
}

__device__ inline int row_cost(const PlanWork& w, int i) {
  return (w.p_off_tmp[i + 1] - w.p_off_tmp[i]) + (w.f_off_tmp[i + 1] - w.f_off_tmp[i]);
}

// Sections deal the (sample, KV head) pairs to the eight XCDs in snake
// order: with x = b*Hk + hk, block x / 8 goes 0..7 when even and 7..0 when
// odd, so consecutive heads (whose ALiBi slopes, and with them the work the
// exact-zero skips leave, fall with the head index) spread over all XCDs.
// The pattern repeats every 16, so only x mod 16 matters: x0 = (b*Hk) mod 16
// from the low bits (unsigned arithmetic, exact whatever the product's size).
__device__ inline int snake_section(uint32_t x) {
  const int lo = (int)(x & (kNumSections - 1));
  return (x >> 3) & 1u ? kNumSections - 1 - lo : lo;
}
__device__ inline int section_of(int b, int heads_k, int hk) {
  return snake_section(((uint32_t)b * (uint32_t)heads_k & 15u) + (uint32_t)hk);
}
// Targets of section s up to X (X >= -1): blocks 2k and 2k+1 hold it at 16k + s
// and 16k + 15 - s.
__device__ inline int section_targets_upto(int s, int X) {
  const int n = X + 1, m = n & 15;
  return 2 * (n >> 4) + (m > s ? 1 : 0) + (m > kNumSections * 2 - 1 - s ? 1 : 0);
}
// Number of KV heads hk in [0, Hk) of section s for a sample whose first KV
// head has snake index x0, and (rank_hk >= 0) the number of those below
// rank_hk.
__device__ inline int kv_heads_in_section_at(int x0, int heads_k, int s, int rank_hk = -1) {
  const int below = section_targets_upto(s, x0 - 1);
  const int end = rank_hk >= 0 ? x0 + rank_hk : x0 + heads_k;
  return section_targets_upto(s, end - 1) - below;
}
// The same for sample b: its first KV head takes snake index (b * Hk) mod 16.
__device__ inline int kv_heads_in_section(int b, int heads_k, int s, int rank_hk = -1) {
  return kv_heads_in_section_at((int)((uint32_t)b * (uint32_t)heads_k & 15u), heads_k, s,
                                rank_hk);
}

// Launch slot of the r-th task of section s: sections interleaved while they
// last; zero-cost tasks after all positive-cost ones.
__device__ inline int launch_slot(const int* secoff, int s, int r) {
  if (s >= kNumSections) return secoff[kNumSections] + r;
  int slot = 0;
#pragma unroll
  for (int s2 = 0; s2 < kNumSections; ++s2) {
    const int n2 = secoff[s2 + 1] - secoff[s2];
    slot += min(r, n2) + ((s2 < s && n2 > r) ? 1 : 0);
  }
  return slot;
}

}  // namespace

// §4.8 the forward schedule, one workgroup, after the header is known.
// Tasks are (plan row, Q head).  Order: section ascending (section of
// (b, h) = (b*Hk + h/group) % 8, zero-cost tasks last), then the cost of the
// task's mask row descending, ties by flat row index then head.  Bounded
// counting, no general sort:
//  1. rows (flat, head-major) are ranked by descending cost with a stable
//     counting sort: per 64-row chunk (one wavefront) the rows with an equal
//     cost are found with one ballot per cost bit, giving each row its rank
//     among them and the chunk's per-cost counts; one exclusive scan of the
//     counts laid out [cost][chunk] gives every row its sorted position.  The
//     same pass totals the tasks of each section.
//  2. over the sorted rows, an exclusive scan of each row's per-section task
//     counts (eight sections and the zero-cost queue) gives the in-section
//     position of the row's first task in each queue.
//  3. every task is written to the section-major schedule and, as a launch
//     record, at its section-interleaved launch slot (slot 8r+x holds the r-th
//     task of section x while every section still has tasks).
// Up to kSchedLdsRows rows, the row data (offsets, first tiles, the sorted
// order) live in LDS, and their nine first positions too while they fit
// (sched_rows_in_lds); past that in the build workspace.
constexpr int kSchedLdsRows = 4096;

namespace {

// Tasks of one row in each of the nine queues.
__device__ inline void row_queue_counts(const PlanGeo& g, int b, int hm, int cost,
                                        int (&v)[kNumQueues]) {
  const int group = g.heads_q / g.heads_k;
#pragma unroll
  for (int s = 0; s < kNumQueues; ++s) v[s] = 0;
  if (cost == 0) {
    v[kNumSections] = g.mask_heads == 1 ? g.heads_q : 1;
  } else if (g.mask_heads == 1) {
#pragma unroll
    for (int s = 0; s < kNumSections; ++s) v[s] = group * kv_heads_in_section(b, g.heads_k, s);
  } else {
    const int sec = section_of(b, g.heads_k, hm / group);
#pragma unroll
    for (int s = 0; s < kNumSections; ++s) v[s] = s == sec ? 1 : 0;
  }
}

// Tasks of one row in queue q alone.
__device__ inline int row_queue_count(const PlanGeo& g, int b, int hm, int cost, int q) {
  const int group = g.heads_q / g.heads_k;
  if (cost == 0) return q == kNumSections ? (g.mask_heads == 1 ? g.heads_q : 1) : 0;
  if (q == kNumSections) return 0;
  if (g.mask_heads == 1) return group * kv_heads_in_section(b, g.heads_k, q);
  return q == section_of(b, g.heads_k, hm / group) ? 1 : 0;
}

__device__ inline void write_task(const PlanGeo& g, const PlanDev& d, const int* secoff,
                                  const SampleGeo& sg, int il, int h, int hm, int s, int pos_s,
                                  int p_beg, int np, int f_beg, int nf, int first) {
  const int qvalid = min(g.tile_q, sg.q_len - il * g.tile_q);
  *reinterpret_cast<int4*>(d.work_desc + 4 * (int64_t)(secoff[s] + pos_s)) =
      make_int4(il, h, sg.b, qvalid);
  int4* rec = reinterpret_cast<int4*>(d.task_rec +
                                      (int64_t)launch_slot(secoff, s, pos_s) * kTaskRecInts);
  rec[0] = make_int4(il, h, sg.b, qvalid);                         // kRecMBlock ..
  rec[1] = make_int4(sg.q_off, sg.k_off, sg.q_len, sg.k_len);      // kRecQOff ..
  rec[2] = make_int4(p_beg, np, f_beg, nf);                        // kRecPBeg ..
  rec[3] = make_int4(first, hm, h / (g.heads_q / g.heads_k), s);   // kRecFirstTile ..
}

}  // namespace

namespace {

// Records of task (row i, Q head h): its queue and its rank among the row's
// tasks in that queue give its section-major slot and its launch slot.  rb:
// the row's first in-queue position per queue; so: queue offsets; cu: an LDS
// copy of cu_rows or nullptr.
template <class RP>
__device__ __attribute__((always_inline)) inline void place_task(
    const PlanGeo& g, const PlanDev& d, RP rb, const int* cu,
    const int (&so)[kNumQueues + 1], int rows_total, int i, int h, int p_beg, int np, int f_beg,
    int nf, int first) {
  const int group = g.heads_q / g.heads_k;
  const int hm = g.mask_heads == 1 ? 0 : h;
  const int row = i - hm * rows_total;
  const SampleGeo sg = sample_geo(g, d, cu, row);
  int s, rank;
  if (np + nf == 0) {
    s = kNumSections;
    rank = g.mask_heads == 1 ? h : 0;
  } else {
    const int hk = h / group;
    s = section_of(sg.b, g.heads_k, hk);
    if (g.mask_heads == 1) {
      rank = kv_heads_in_section(sg.b, g.heads_k, s, hk) * group + (h - hk * group);
    } else {
      rank = 0;
    }
  }
  write_task(g, d, so, sg, row - sg.row_begin, h, hm, s, rb[s] + rank, p_beg, np, f_beg, nf,
             first);
}
// §4.8 step 3: tasks t = t0, t0 + stride, ... (t < rows_total * Hq) to the
// section-major schedule and, as launch records, to their interleaved launch
// slots.  P, F: the rows' CSR offsets; FT: first listed K tile per
// (hm * upper_rows + row); rbase: first in-queue position of each row's
// tasks; so: queue offsets; cu: an LDS copy of cu_rows or nullptr.
template <class PP, class RP>
__device__ __attribute__((always_inline)) inline void write_tasks(
    const PlanGeo& g, const PlanDev& d, PP P, PP F, PP FT, RP rbase, const int* cu,
    const int (&so)[kNumQueues + 1], int rows_total, int t0, int stride) {
  const int Hq = g.heads_q;
  const int ntasks = rows_total * Hq;
  for (int t = t0; t < ntasks; t += stride) {
    int i, h;
    if (g.mask_heads == 1) {
      i = t / Hq;
      h = t - i * Hq;
    } else {
      i = t;
      h = t / rows_total;
    }
    const int hm = g.mask_heads == 1 ? 0 : h;
    const int row = i - hm * rows_total;
    const int p_beg = P[i], f_beg = F[i];
    place_task(g, d, rbase + (int64_t)i * kNumQueues, cu, so, rows_total, i, h, p_beg,
               P[i + 1] - p_beg, f_beg, F[i + 1] - f_beg, FT[(int64_t)hm * g.upper_rows + row]);
  }
}

}  // namespace

// The schedule, run by one workgroup of 1024 threads; `dyn` is its dynamic
// LDS.  CNT_LDS: the count matrix is in LDS; ROWS: 0 row data read from the
// workspace, 1 in LDS, 2 their first positions in LDS too.  (Compile-time, so
// that every access is ds_* or global_*: a pointer that may point to either
// memory becomes a flat access.)
struct SchedShared {
  int secoff[kNumQueues + 1];
  int run[kNumQueues];
  int tot[kNumQueues];
  int vec[16][kNumQueues];
  int wave[33];
  int carry;
  int cu[1025];
};

// rank / nranks: several workgroups may run the schedule together, each
// sorting the rows itself (the sort only writes LDS: CNT_LDS and ROWS == 2)
// and writing every nranks-th block of 1024 tasks; rank 0 also writes the
// section offsets and the fixed-length geometry.
template <bool CNT_LDS, int ROWS>
__device__ __attribute__((always_inline)) inline void schedule_block(
    const PlanGeo& g, const PlanDev& d, const PlanWork& w, int* dyn, SchedShared& sh, int rank,
    int nranks) {
  constexpr bool cnt_in_lds = CNT_LDS;
  constexpr int rows_in_lds = ROWS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_up = g.mask_heads * g.upper_rows;

  // LDS carve, sized for the upper bound of rows so the row data can be
  // fetched in the same round trip as the header:
  // [count matrix][p_off n_up+1][f_off n_up+1][first n_up][order n_up][bases]
  int32_t* cnt = cnt_in_lds ? dyn : w.chunk_cnt;
  int* lds_rows = dyn + (cnt_in_lds ? (int64_t)(g.nk_max + 1) * w.nchunks : 0);
  const int32_t* P = w.p_off_tmp;
  const int32_t* F = w.f_off_tmp;
  const int32_t* FT = w.first_tile;   // indexed hm * upper_rows + row
  int32_t* order = w.order;
  // header first, so that its load and the row loads are in flight together
  const int hdr_err = d.header[7];
  const int hdr_rows = d.header[0];
  if constexpr (rows_in_lds != 0) {
    int* lp = lds_rows;
    int* lf = lp + n_up + 1;
    int* lt = lf + n_up + 1;
    order = lt + n_up;
    for (int i = tid; i <= n_up; i += 1024) {
      lp[i] = w.p_off_tmp[i];
      lf[i] = w.f_off_tmp[i];
      if (i < n_up) lt[i] = w.first_tile[i];
    }
    P = lp;
    F = lf;
    FT = lt;
  }
  if (hdr_err != 0) return;  // the build failed: no plan is made
  const int rows_total = hdr_rows;
  const int n = g.mask_heads * rows_total;
  const int nc = (n + 63) >> 6;
  const int64_t cnt_len = (int64_t)(g.nk_max + 1) * nc;
  auto cost_of = [&](int i) -> int { return (P[i + 1] - P[i]) + (F[i + 1] - F[i]); };

  const int* cu = nullptr;
  if (g.layout == MPB_LAYOUT_BSHD) {
    // Fixed-length geometry in closed form (§4.2: rectangular upper bound).
    const int rps = (g.seqlen_q + g.tile_q - 1) / g.tile_q;
    for (int b = tid; b < g.batch && rank == 0; b += 1024) {
      int4* sd = reinterpret_cast<int4*>(d.seqdesc + 8 * b);
      sd[0] = make_int4(b * g.seqlen_q, b * g.seqlen_k, g.seqlen_q, g.seqlen_k);
      sd[1] = make_int4(b * rps, rps, (g.seqlen_k + g.tile_k - 1) / g.tile_k, 0);
      d.cu_rows[b + 1] = (b + 1) * rps;
    }
    if (tid == 0 && rank == 0) d.cu_rows[0] = 0;
  } else if (g.batch < 1025) {
    for (int b = tid; b <= g.batch; b += 1024) sh.cu[b] = d.cu_rows[b];
    cu = sh.cu;
  }
  if (tid < kNumQueues) {
    sh.run[tid] = 0;
    sh.tot[tid] = 0;
  }
  for (int64_t x = tid; x < cnt_len; x += 1024) cnt[x] = 0;
  __syncthreads();

  // 1. stable counting sort of the rows by descending cost; queue totals
  const int nbits = 32 - __clz(g.nk_max);
  const uint64_t below = lanes_below(lane);
  int lr[kSchedLdsRows / 1024];
  int tot[kNumQueues];
#pragma unroll
  for (int s = 0; s < kNumQueues; ++s) tot[s] = 0;
  // With one chunk of rows, wavefront 0 ranks them while wavefronts 1..9 each
  // total one queue; otherwise every wavefront does both for its chunks.
  const bool one_chunk = nc == 1;
  if (one_chunk && wv >= 1 && wv <= kNumQueues) {
    const int q = wv - 1;
    int v = 0;
    if (lane < n) {
      const int hm = lane / rows_total;
      v = row_queue_count(g, sample_geo(g, d, cu, lane - hm * rows_total).b, hm, cost_of(lane), q);
    }
    const int t = wave_sum(v);
    if (lane == 0) sh.tot[q] = t;
  }
  for (int c = wv, k = 0; c < nc && !(one_chunk && wv > 0); c += 16, ++k) {
    const int i = c * 64 + lane;
    const bool live = i < n;
    int key = 0;
    if (live) {
      const int cost = cost_of(i);
      key = g.nk_max - cost;
      if (!one_chunk) {
        const int hm = i / rows_total;
        int v[kNumQueues];
        row_queue_counts(g, sample_geo(g, d, cu, i - hm * rows_total).b, hm, cost, v);
#pragma unroll
        for (int s = 0; s < kNumQueues; ++s) tot[s] += v[s];
      }
    }
    uint64_t eq = __ballot(live);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (key >> bit) & 1;
      const uint64_t m = __ballot(on);
      eq &= on ? m : ~m;
    }
    if (live) {
      const int rank = __popcll(eq & below);
      if constexpr (rows_in_lds != 0) {
#pragma unroll
        for (int u = 0; u < kSchedLdsRows / 1024; ++u)
          if (u == k) lr[u] = rank;
      } else {
        w.lrank[i] = rank;
      }
      if ((eq & below) == 0) cnt[(int64_t)key * nc + c] = __popcll(eq);
    }
  }
  if (!one_chunk && wv < nc) {   // wavefronts that classified rows
#pragma unroll
    for (int s = 0; s < kNumQueues; ++s) {
      const int t = wave_sum(tot[s]);
      if (lane == 0 && t) atomicAdd(&sh.tot[s], t);
    }
  }
  __syncthreads();
  if (cnt_len <= 64) {   // one wavefront scans the whole count matrix
    if (wv == 0) {
      const int v = lane < cnt_len ? cnt[lane] : 0;
      const int incl = wave_incl_scan(v, lane);
      if (lane < cnt_len) cnt[lane] = incl - v;
    }
    __syncthreads();
  } else {
    block_exclusive_scan_inplace(cnt, cnt_len, sh.wave, &sh.carry);
  }
  for (int c = wv, k = 0; c < nc; c += 16, ++k) {   // same row-to-thread map as above
    const int i = c * 64 + lane;
    if (i >= n) continue;
    int rank = 0;
    if constexpr (rows_in_lds != 0) {
#pragma unroll
      for (int u = 0; u < kSchedLdsRows / 1024; ++u)
        if (u == k) rank = lr[u];
    } else {
      rank = w.lrank[i];
    }
    order[cnt[(int64_t)(g.nk_max - cost_of(i)) * nc + c] + rank] = i;
  }
  if (tid == 0) {
    sh.secoff[0] = 0;
    for (int s = 0; s < kNumQueues; ++s) sh.secoff[s + 1] = sh.secoff[s] + sh.tot[s];
    if (rank == 0)
      for (int s = 0; s <= kNumQueues; ++s) d.section_off[s] = sh.secoff[s];
  }
  __syncthreads();

  // 2. in-section position of each row's first task, over the sorted rows
  // (one chunk: wavefront q scans queue q)
  int32_t* rbase = rows_in_lds == 2 ? order + n_up : w.row_base;
  if (one_chunk) {
    if (wv < kNumQueues) {
      int v = 0, i = 0;
      if (lane < n) {
        i = order[lane];
        const int hm = i / rows_total;
        v = row_queue_count(g, sample_geo(g, d, cu, i - hm * rows_total).b, hm, cost_of(i), wv);
      }
      const int incl = wave_incl_scan(v, lane);
      if (lane < n) rbase[(int64_t)i * kNumQueues + wv] = incl - v;
    }
    __syncthreads();
  }
  for (int base = 0; base < n && !one_chunk; base += 1024) {
    const int pos = base + tid;
    int v[kNumQueues];
    int i = 0;
    if (pos < n) {
      i = order[pos];
      const int hm = i / rows_total;
      row_queue_counts(g, sample_geo(g, d, cu, i - hm * rows_total).b, hm, cost_of(i), v);
    } else {
#pragma unroll
      for (int s = 0; s < kNumQueues; ++s) v[s] = 0;
    }
    int first_pos[kNumQueues];
#pragma unroll
    for (int s = 0; s < kNumQueues; ++s) {
      const int incl = wave_incl_scan(v[s], lane);
      first_pos[s] = incl - v[s];
      if (lane == 63) sh.vec[wv][s] = incl;
    }
    __syncthreads();
    if (tid < kNumQueues) {   // queue tid: exclusive prefix of the wavefront totals
      int run = sh.run[tid];
      for (int x = 0; x < 16; ++x) {
        const int t = sh.vec[x][tid];
        sh.vec[x][tid] = run;
        run += t;
      }
      sh.run[tid] = run;
    }
    __syncthreads();
    if (pos < n) {
#pragma unroll
      for (int s = 0; s < kNumQueues; ++s)
        rbase[(int64_t)i * kNumQueues + s] = sh.vec[wv][s] + first_pos[s];
    }
    __syncthreads();   // sh.vec is reused
  }

  // 3. every task, one per thread
  int so[kNumQueues + 1];
#pragma unroll
  for (int s = 0; s <= kNumQueues; ++s) so[s] = sh.secoff[s];
  write_tasks(g, d, P, F, FT, rbase, cu, so, rows_total, tid + 1024 * rank, 1024 * nranks);
}

__device__ __attribute__((always_inline)) inline void schedule_any(
    const PlanGeo& g, const PlanDev& d, const PlanWork& w, int cnt_in_lds, int rows_in_lds,
    int* dyn, int rank = 0, int nranks = 1) {
  __shared__ SchedShared sh;
  if (cnt_in_lds) {
    if (rows_in_lds == 2) schedule_block<true, 2>(g, d, w, dyn, sh, rank, nranks);
    else if (rows_in_lds == 1) schedule_block<true, 1>(g, d, w, dyn, sh, 0, 1);
    else schedule_block<true, 0>(g, d, w, dyn, sh, 0, 1);
  } else {
    if (rows_in_lds == 2) schedule_block<false, 2>(g, d, w, dyn, sh, 0, 1);
    else if (rows_in_lds == 1) schedule_block<false, 1>(g, d, w, dyn, sh, 0, 1);
    else schedule_block<false, 0>(g, d, w, dyn, sh, 0, 1);
  }
}

__global__ __launch_bounds__(1024) void plan_schedule_kernel(PlanGeo g, PlanDev d, PlanWork w,
                                                             int cnt_in_lds, int rows_in_lds) {
  extern __shared__ int dyn[];
  schedule_any(g, d, w, cnt_in_lds, rows_in_lds, dyn);
}

// ---------------------------------------------------------------- materialize

// Payload words of one row for its np partial K tiles (ascending, in
// `tiles`), written from pair p_begin on.  Word [r][c/32] of a pair starts
// from the parity of the row's endpoints < c and flips at each endpoint
// inside the word.  Words come in ascending column order, so every endpoint
// is read once: `ptr` counts the endpoints below the current word and `nxt`
// holds the next one (INT_MAX past the last), and a word with no endpoint
// inside costs one compare.  STAGED: the endpoints were staged in LDS as
// [nfunc][T_Q]; else read from HBM through `col`.  (One instance per source
// keeps LDS reads ds_read: a pointer that may point to either memory would
// become a flat load.)
// E(f): the row's endpoint f, INT_MAX past the last.
template <class EF>
__device__ __attribute__((always_inline)) inline void row_payload_e(
    const PlanGeo& g, const int* tiles, int np, EF&& E, int rho, bool valid, bool is_row,
    uint32_t* p_masks, int p_begin) {
  // e0..e3: endpoints ptr..ptr+3, each loaded three steps before it is
  // needed, so the walk does not wait on one load per endpoint
  int ptr = 0;
  int e0 = valid ? E(0) : INT_MAX, e1 = valid ? E(1) : INT_MAX;
  int e2 = valid ? E(2) : INT_MAX, e3 = valid ? E(3) : INT_MAX;
  auto advance = [&]() {
    ++ptr;
    e0 = e1;
    e1 = e2;
    e2 = e3;
    e3 = E(ptr + 3);
  };
  auto word_at = [&](int c) -> uint32_t {
    if (!valid) return 0u;
    while (e3 < c) {   // all four below c: skip them with one round of loads
      ptr += 4;
      e0 = E(ptr);
      e1 = E(ptr + 1);
      e2 = E(ptr + 2);
      e3 = E(ptr + 3);
    }
    while (e0 < c) advance();
    uint32_t word = (ptr & 1) ? 0u : 0xFFFFFFFFu;
    while (e0 < c + 32) {
      word ^= 0xFFFFFFFFu << (e0 - c);
      advance();
    }
    return word;
  };
  int t_next = np > 0 ? tiles[0] : 0;   // the list is read one tile ahead
  for (int k = 0; k < np; ++k) {
    const int c0 = t_next * g.tile_k;
    if (k + 1 < np) t_next = tiles[k + 1];
    uint32_t* dst = p_masks + ((int64_t)(p_begin + k) * g.tile_q + rho) * g.words_tile;
    if (g.words_tile == 2) {
      const uint32_t w0 = word_at(c0);
      const uint32_t w1 = word_at(c0 + 32);
      if (is_row) *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
    } else {
      for (int x = 0; x < g.words_tile; ++x) {
        const uint32_t wd = word_at(c0 + 32 * x);
        if (is_row) dst[x] = wd;
      }
    }
  }
}

// The payload walk of a staged row, kept to a few instructions per word: the
// tile's column is uniform (read once for the wavefront), the words go out
// by buffer stores whose per-tile offset is a scalar add, and a word with no
// endpoint inside costs two compares.  E(f) must hold a sentinel above every
// column at f = nfunc.  Rows past q_len write 0.
template <class EF>
__device__ __attribute__((always_inline)) inline void row_payload_tight(
    const PlanGeo& g, const int* tiles, int k_begin, int k_end, EF&& E, int rho, bool valid,
    bool is_row, uint32_t* p_masks, int p_begin) {
  const int W = g.words_tile;
  const int64_t cap = (int64_t)g.mask_heads * g.upper_rows * g.nk_max * g.tile_q * W * 4;
  const rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      p_masks, (short)0, (int)(cap < 0x7FFFFFFF ? cap : 0x7FFFFFFF), 0x00020000);
  const uint32_t step = (uint32_t)g.tile_q * W * 4;
  uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(p_begin + k_begin) * step;   // uniform
  const uint32_t voff = (uint32_t)rho * W * 4;
  // the walk starts at the first endpoint not below the first tile's column
  // (binary search; a row past q_len is invisible everywhere)
  int ptr = 1, e0 = INT_MAX;
  if (valid) {
    const int c_first = __builtin_amdgcn_readfirstlane(tiles[k_begin]) * g.tile_k;
    int lo = 0, hi = g.nfunc;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (E(mid) < c_first) lo = mid + 1;
      else hi = mid;
    }
    ptr = lo;
    e0 = E(ptr);
  }
  for (int k = k_begin; k < k_end; ++k, soff += step) {
    const int c0 = __builtin_amdgcn_readfirstlane(tiles[k]) * g.tile_k;
    for (int x = 0; x < W; ++x) {
      const int c = c0 + 32 * x;
      while (e0 < c) e0 = E(++ptr);
      uint32_t word = (ptr & 1) ? 0u : 0xFFFFFFFFu;
      while (e0 < c + 32) {
        word ^= 0xFFFFFFFFu << (e0 - c);
        e0 = E(++ptr);
      }
      if (is_row) __builtin_amdgcn_raw_buffer_store_b32(word, rm, (int)(voff + 4 * x), (int)soff, 0);
    }
  }
}

template <bool STAGED>
__device__ __attribute__((always_inline)) inline void row_payload(
    const PlanGeo& g, const int* tiles, int np, const int* ep, const int32_t* col, int rho,
    bool valid, bool is_row, uint32_t* p_masks, int p_begin) {
  auto E = [&](int f) -> int {
    if (f >= g.nfunc) return INT_MAX;
    if constexpr (STAGED) return ep[f * g.tile_q + rho];
    else return col[(int64_t)f * g.total_q];
  };
  row_payload_e(g, tiles, np, E, rho, valid, is_row, p_masks, p_begin);
}

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
                                                               PlanDev st, PlanDev d, PlanWork w,
                                                               int rows_total, int stage_ep,
                                                               MetaCopy mc) {
  extern __shared__ int lds[];
  int* tiles = lds;                     // [nk_max] partial K tiles of this row
  int* ep = lds + g.nk_max;             // [nfunc][T_Q] endpoints when staged
  const int item = blockIdx.x;
  const int tid = threadIdx.x;
  if (rows_total < 0) {
    // launched before the header was read back (Varlen rows counted on the
    // device): nothing to do for a failed build
    if (d.header[7] != 0) return;
    rows_total = d.header[0];
  }
  const int n = g.mask_heads * rows_total;
  const bool has_row = item < n;
  // This row's loads are issued first; the metadata copy below runs while
  // they are in flight.
  const int hm = has_row ? item / rows_total : 0;
  const int row = has_row ? item - hm * rows_total : 0;
  const int64_t src = (int64_t)hm * g.upper_rows + row;
  int p_begin = 0, f_begin = 0, np = 0;
  RowGeo rg = {};
  bool valid = false;
  const bool is_row = tid < g.tile_q;
  const int rho = tid;
  const int32_t* col = mf;
  if (has_row) {
    p_begin = w.p_off_tmp[item];
    f_begin = w.f_off_tmp[item];
    np = w.p_off_tmp[item + 1] - p_begin;
    rg = row_geometry(g, st, row);
    valid = is_row && rg.i * g.tile_q + rho < rg.q_len;
    col = mf + (int64_t)hm * g.nfunc * g.total_q + rg.q_off + (int64_t)rg.i * g.tile_q +
          (valid ? rho : 0);
    if (stage_ep == 2) {
      // straight into LDS: lane l of wavefront v loads row 64v + l of every
      // endpoint column (rows past q_len load values nobody reads)
      const int wv = tid >> 6, ln = tid & 63;
      if (64 * wv < g.tile_q) {
        const rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t*>(mf + (int64_t)hm * g.nfunc * g.total_q), (short)0,
            (int)((int64_t)g.nfunc * g.total_q * 4), 0x00020000);
        const uint32_t base = (uint32_t)(rg.q_off + rg.i * g.tile_q + 64 * wv + ln) * 4u;
        for (int f = 0; f < g.nfunc; ++f)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rm, (__attribute__((address_space(3))) void*)&ep[f * g.tile_q + 64 * wv], 4,
              (int)(base + (uint32_t)f * (uint32_t)g.total_q * 4u), 0, 0, 0);
      }
    } else if (stage_ep && valid) {
      for (int f = 0; f < g.nfunc; ++f) ep[f * g.tile_q + rho] = col[(int64_t)f * g.total_q];
    }
  }
  // Plan metadata staged in the workspace (header, geometry, schedule and
  // launch records), copied into the plan block a slice per workgroup.
  {
    const int64_t per = (mc.total + gridDim.x - 1) / gridDim.x;
    const int64_t lo = per * blockIdx.x, hi = min(mc.total, lo + per);
    for (int64_t x = lo + tid; x < hi; x += blockDim.x) {
      int seg = 0;
      while (x >= mc.end[seg]) ++seg;
      const int64_t off = x - (seg ? mc.end[seg - 1] : 0);
      mc.dst[seg][off] = mc.src[seg][off];
    }
  }
  if (item == 0 && tid == 0) {
    d.p_off[n] = w.p_off_tmp[n];
    d.f_off[n] = w.f_off_tmp[n];
  }
  if (!has_row) return;
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
  __builtin_amdgcn_s_waitcnt(0);   // this wavefront's loads into LDS have landed
  __syncthreads();  // the partial tile list and the staged endpoints are complete
  if (stage_ep)
    row_payload<true>(g, tiles, np, ep, col, rho, valid, is_row, d.p_masks, p_begin);
  else
    row_payload<false>(g, tiles, np, ep, col, rho, valid, is_row, d.p_masks, p_begin);
}


// In-place builds: the schedule (workgroup 0) and every row's lists and
// payload (the other workgroups, 1024 / SG rows each with SG = max(64, T_Q)
// threads per row) in one launch -- both follow from the classification and
// its offsets, neither needs the other.  The per-row work is the one of
// plan_materialize_kernel; the metadata is already in place.
__global__ __launch_bounds__(1024) void plan_finish_kernel(PlanGeo g,
                                                           const int32_t* __restrict__ mf,
                                                           PlanDev d, PlanWork w, int rows_total,
                                                           int stage_ep, int cnt_in_lds,
                                                           int rows_in_lds) {
  extern __shared__ int dyn[];
  if (blockIdx.x == 0) {
    schedule_any(g, d, w, cnt_in_lds, rows_in_lds, dyn);
    return;
  }
  if (rows_total < 0) {   // Varlen: rows counted on the device; nothing for a failed build
    if (d.header[7] != 0) return;
    rows_total = d.header[0];
  }
  const int SG = g.tile_q < 64 ? 64 : g.tile_q;
  const int G = 1024 / SG;
  const int sub = threadIdx.x / SG;
  const int tid = threadIdx.x - sub * SG;
  int* tiles = dyn + sub * (g.nk_max + (stage_ep ? g.nfunc * g.tile_q : 0));
  int* ep = tiles + g.nk_max;
  const int item = (blockIdx.x - 1) * G + sub;
  const int n = g.mask_heads * rows_total;
  const bool has_row = item < n;
  const int hm = has_row ? item / rows_total : 0;
  const int row = has_row ? item - hm * rows_total : 0;
  const int64_t src = (int64_t)hm * g.upper_rows + row;
  int p_begin = 0, f_begin = 0, np = 0;
  RowGeo rg = {};
  bool valid = false;
  const bool is_row = tid < g.tile_q;
  const int rho = tid;
  const int32_t* col = mf;
  if (has_row) {
    p_begin = w.p_off_tmp[item];
    f_begin = w.f_off_tmp[item];
    np = w.p_off_tmp[item + 1] - p_begin;
    rg = row_geometry(g, d, row);
    valid = is_row && rg.i * g.tile_q + rho < rg.q_len;
    col = mf + (int64_t)hm * g.nfunc * g.total_q + rg.q_off + (int64_t)rg.i * g.tile_q +
          (valid ? rho : 0);
    if (stage_ep == 2) {
      const int wv = tid >> 6, ln = tid & 63;
      if (64 * wv < g.tile_q) {
        const rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t*>(mf + (int64_t)hm * g.nfunc * g.total_q), (short)0,
            (int)((int64_t)g.nfunc * g.total_q * 4), 0x00020000);
        const uint32_t base = (uint32_t)(rg.q_off + rg.i * g.tile_q + 64 * wv + ln) * 4u;
        for (int f = 0; f < g.nfunc; ++f)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rm, (__attribute__((address_space(3))) void*)&ep[f * g.tile_q + 64 * wv], 4,
              (int)(base + (uint32_t)f * (uint32_t)g.total_q * 4u), 0, 0, 0);
      }
    } else if (stage_ep && valid) {
      for (int f = 0; f < g.nfunc; ++f) ep[f * g.tile_q + rho] = col[(int64_t)f * g.total_q];
    }
    if (item == 0 && tid == 0) {
      d.p_off[n] = w.p_off_tmp[n];
      d.f_off[n] = w.f_off_tmp[n];
    }
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
  }
  __builtin_amdgcn_s_waitcnt(0);   // this wavefront's loads into LDS have landed
  __syncthreads();  // every row's partial tile list and staged endpoints are complete
  if (!has_row || np == 0) return;
  if (stage_ep)
    row_payload<true>(g, tiles, np, ep, col, rho, valid, is_row, d.p_masks, p_begin);
  else
    row_payload<false>(g, tiles, np, ep, col, rho, valid, is_row, d.p_masks, p_begin);
}


// ---------------------------------------------------------------- single pass
//
// Forward plans whose block at the upper bound of every count fits the
// library's cap are built in one pass over the endpoints: one workgroup per
// (mask head, Q plan row) item classifies its row (§4.3), takes the exact CSR
// offsets of its lists by decoupled look-back over the items before it
// (§4.5), and writes its lists and payload (§4.6, §5) while its endpoints are
// still in LDS, so the endpoints are read from HBM once.
//  * Workgroup t handles item t of the flat head-major order and waits only
//    for items before it.  Workgroups go to the XCDs round-robin and each XCD
//    starts its own in index order, so the lowest unfinished item either runs
//    (everything it waits for is done) or waits for a slot on its XCD that
//    only finished or foreign work holds: the waits end.  (A ticket counter
//    drawn by every workgroup gave the same guarantee without the dispatch
//    order, but its atomics on one address serialized the starts: 19 us for
//    1536 items.)
//  * Look-back words are tagged with the build's sequence number, so nothing
//    has to be cleared between builds: a word is valid when its tag is this
//    build's.  Item t publishes its aggregate (tile counts) as soon as it is
//    classified, then its inclusive prefix and a "done" word with its error
//    bits once its look-back ends.  A wavefront reads 64 predecessors at a
//    time and stops at the nearest inclusive prefix.  Every wait is bounded
//    (kLookbackSpins polls); a wait that runs out marks the build failed
//    (kDevErrLookback).
//  * The item that ends the flat order publishes the header after every
//    item's "done" word has landed, with the OR of their error bits.
//  * The lists go to workspace arrays in flat CSR order; the tail launch
//    (schedule plus list placement) copies them behind the payload once the
//    total partial count fixes their place in the exact block.
namespace {

constexpr uint32_t kLookbackSpins = 1u << 20;
// Sentinel rows after a staged row's endpoints (the walks read up to
// nfunc + 5) and the int16 sentinel: above every column of a sample short
// enough for int16 endpoints (seqlen_k <= kShortEpMaxLen).
constexpr int kEpPad = 6;
constexpr short kEpSentinel16 = 32767;

__device__ inline uint64_t lb_word(uint32_t tag, uint32_t v) { return ((uint64_t)tag << 32) | v; }

__device__ inline uint64_t lb_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void lb_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Header of a finished single-pass build, to the plan and the host slot
// (values first, then the sequence number with release semantics).
__device__ inline void sp_publish(const PlanDev& d, const SinglePass& sp, int rows_total,
                                  int pnnz, int fnnz, uint32_t err) {
  const int32_t hdr[8] = {rows_total, pnnz, fnnz, 0, 0, 0, 0, (int32_t)err};
  for (int i = 0; i < 8; ++i) d.header[i] = hdr[i];
  if (sp.deferred) return;   // the host reads d.header later
  for (int i = 0; i < 8; ++i)
    __hip_atomic_store(&sp.host_slot[i], hdr[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(&sp.host_slot[kHeaderSeq], sp.seq, __ATOMIC_RELEASE,
                     __HIP_MEMORY_SCOPE_SYSTEM);
}

// §4.8 tasks that a row of key k puts in queue s, for the fused schedule
// below.  Key kKeys - 1: an empty row, all its tasks in the empty queue;
// keys 0..15 for one mask row shared by the Q heads: (b * Hk) mod 16, which
// fixes how its sample's KV heads fall on the sections; for a per-head mask
// row, the section of its KV head.
__device__ inline int fused_queue_weight(const PlanGeo& g, int k, int s) {
  if (k == kKeys - 1) return s == kNumSections ? (g.mask_heads == 1 ? g.heads_q : 1) : 0;
  if (s == kNumSections) return 0;
  if (g.mask_heads == 1)
    return (g.heads_q / g.heads_k) * kv_heads_in_section_at(k, g.heads_k, s);
  return k == s ? 1 : 0;
}
// §4.8 queue positions of one row of a fused single-pass build, computed by
// one whole wavefront beside the look-back.  The schedule ranks the rows by
// descending cost (partial plus full tiles), ties by flat index.  A row's
// tasks per queue follow from its key alone (fused_queue_weight), so the
// row's first position in each queue is a sum over the keys of (rows of that
// key ranked before it) x (tasks such a row puts in the queue), and the queue
// starts are the same sums over all rows; no item sorts.  The costs come from
// the items' aggregate words, which every item publishes right after its
// classification.  ci: this item's cost; wts[kKeys * kNumQueues]: the
// weights.  Out: rb[kNumQueues] this row's first position per queue,
// sec[kNumQueues + 1] the queue starts; cnt[kKeys] and red[kNumQueues] are
// scratch.  Returns false when some item's word never came (the positions
// are then in bounds but not meaningful).
__device__ bool fused_row_positions(const PlanGeo& g, const PlanDev& d, const SinglePass& sp,
                                    int n, int rows_total, int item, int ci, const int* wts,
                                    int* cnt, int* red, int* rb, int* sec) {
  const int lane = threadIdx.x & 63;
  const int group = g.heads_q / g.heads_k;
  // one wavefront: its LDS operations complete in order; the fences keep
  // the compiler from moving them across the points between the steps
  auto wave_sync = []() __attribute__((always_inline)) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (lane < kKeys) cnt[lane] = 0;
  wave_sync();
  bool late = false;
  for (int j = lane; j < n; j += 64) {
    int c = ci;
    if (j != item) {
      const uint64_t* wj = sp.lb + kLbWords * (int64_t)j;
      uint64_t ag = lb_load(wj);
      uint32_t spins = 0;
      while ((uint32_t)(ag >> 32) != sp.tag) {
        if (++spins > kLookbackSpins) {
          late = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        ag = lb_load(wj);
      }
      c = (int)((uint32_t)ag >> 16) + (int)((uint32_t)ag & 0xFFFFu);
    }
    const int hm = j / rows_total;
    const int b = sample_geo(g, d, nullptr, j - hm * rows_total).b;
    const int key = c == 0 ? kKeys - 1
                    : g.mask_heads == 1 ? (int)((uint32_t)b * (uint32_t)g.heads_k & 15u)
                                        : section_of(b, g.heads_k, hm / group);
    const bool before = c > ci || (c == ci && j < item);
    // rows of the key in the low half, those ranked before this one in the
    // high half (at most kFusedMaxItems of each)
    atomicAdd(&cnt[key], before ? 0x10001 : 1);
  }
  wave_sync();
  // lanes 0..8: this row's first position per queue; 9..17: queue totals
  if (lane < 2 * kNumQueues) {
    const bool tot = lane >= kNumQueues;
    const int s = tot ? lane - kNumQueues : lane;
    int acc = 0;
    for (int k = 0; k < kKeys; ++k) {
      const int v = cnt[k];
      acc += wts[k * kNumQueues + s] * (tot ? (v & 0xFFFF) : (v >> 16));
    }
    if (tot)
      red[s] = acc;
    else
      rb[s] = acc;
  }
  wave_sync();
  if (lane == 0) {
    sec[0] = 0;
    for (int s = 0; s < kNumQueues; ++s) sec[s + 1] = sec[s] + red[s];
  }
  return __ballot(late) == 0;
}

// Exclusive prefix over the workgroup's threads of (a, b); totals in ta, tb.
__device__ inline void block_scan2(int a, int b, int* pa, int* pb, int* ta, int* tb, int* s_a,
                                   int* s_b) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int ia = wave_incl_scan(a, lane), ib = wave_incl_scan(b, lane);
  if (lane == 63) {
    s_a[wv] = ia;
    s_b[wv] = ib;
  }
  __syncthreads();
  int ra = 0, rb = 0, sa = 0, sb = 0;
  for (int x = 0; x < nw; ++x) {
    if (x < wv) {
      ra += s_a[x];
      rb += s_b[x];
    }
    sa += s_a[x];
    sb += s_b[x];
  }
  *pa = ra + ia - a;
  *pb = rb + ib - b;
  *ta = sa;
  *tb = sb;
}

}  // namespace

// One workgroup per item: one or two groups of max(64, T_Q) threads, thread
// rho of a group owning Q row rho of the tile.  EPM, where the item's
// endpoints [nfunc][T_Q] are read from:
// 1 LDS as int32 (sp.stage 2: loaded straight into LDS, whole wavefronts of
// rows; 1: through registers), 2 LDS as int16 (every sample has k_len below
// 2^15; loaded through registers and checked at full width on the way, half
// the LDS, so twice the workgroups fit a CU), 0 HBM in both passes.
template <int EPM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6)))
void plan_single_pass_kernel(PlanGeo g,
                                                               const int32_t* __restrict__ mf,
                                                               PlanDev d, PlanWork w,
                                                               SinglePass sp) {
  extern __shared__ int lds[];
  __shared__ int s_item, s_err, s_err2, s_pbeg, s_fbeg, s_ffirst;
  __shared__ int s_a[4], s_b[4];
  // fused builds: this row's queue positions, the queue starts, scratch
  __shared__ int s_frb[kNumQueues], s_fsec[kNumQueues + 1], s_fok;
  __shared__ int s_fcnt[kKeys], s_fred[kNumQueues], s_fwts[kKeys * kNumQueues];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // ng groups of sg threads: thread rho of every group owns Q row rho of the
  // tile; the groups split the endpoint loads, the K-tile range of the
  // classification and the partial tiles of the payload
  const int sg = g.tile_q < 64 ? 64 : g.tile_q;
  const int ng = (int)blockDim.x / sg;
  const int grp = tid / sg;
  const int nwr = sg >> 6;            // wavefronts per group
  const int wr = (tid - grp * sg) >> 6;   // this wavefront's 64-row block
  if (tid == 0) {
    s_item = blockIdx.x;
    s_err = 0;
    s_ffirst = -1;
    s_err2 = 0;
  }
  __syncthreads();
  const int item = s_item;
  const int rows_total = rows_total_of(g, d);
  const int n = g.mask_heads * rows_total;
  if (item >= n) {
    // no rows at all (empty THD batch or a failed prefix check): item 0
    // publishes the empty header
    if (item == 0 && tid == 0) {
      d.p_off[0] = 0;
      d.f_off[0] = 0;
      const uint32_t err = g.layout == MPB_LAYOUT_THD ? (uint32_t)w.geo_err[0] : 0u;
      sp_publish(d, sp, rows_total, 0, 0, err);
    }
    return;
  }
  const int hm = item / rows_total;
  const int row = item - hm * rows_total;
  const RowGeo rg = row_geometry(g, d, row);
  const int rho = tid - grp * sg;
  const bool is_row = rho < g.tile_q;
  const bool valid = is_row && rg.i * g.tile_q + rho < rg.q_len;
  const int32_t* col = mf + (int64_t)hm * g.nfunc * g.total_q + rg.q_off +
                       (int64_t)rg.i * g.tile_q + (valid ? rho : 0);
  // [nfunc + kEpPad][T_Q] when staged; the pad rows hold a sentinel above
  // every column, so reads past the last endpoint need no bound check
  const int ep_rows = g.nfunc + kEpPad;
  int* ep = lds;
  short* ep16 = reinterpret_cast<short*>(lds);
  const int ep_ints = EPM == 1 ? ep_rows * g.tile_q : EPM == 2 ? (ep_rows * g.tile_q + 1) / 2 : 0;
  uint32_t* s_any = reinterpret_cast<uint32_t*>(lds + ep_ints);
  uint32_t* s_nfull = s_any + nwr * g.words_k;              // [nwr][words_k] each
  int* ptiles = reinterpret_cast<int*>(s_nfull + nwr * g.words_k);   // [nk_max]

  // §2 order and bounds of every endpoint of the row (EPM 2: while staging)
  uint32_t err = 0;
  if constexpr (EPM == 2) {
    // group grp loads endpoints grp, grp + ng, ...; bounds are checked on
    // the full int32 values, order once the whole row is staged
    for (int f0 = grp; f0 < g.nfunc; f0 += 32 * ng) {
      int v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int f = f0 + u * ng;
        v[u] = valid && f < g.nfunc ? col[(int64_t)f * g.total_q] : 0;
      }
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int f = f0 + u * ng;
        if (valid && f < g.nfunc) {
          const int e = v[u];
          if (e < 0 || e > rg.k_len) err |= MPB_DEVERR_RANGE;
          ep16[f * g.tile_q + rho] = (short)e;
        }
      }
    }
    if (is_row && grp == 0)
      for (int f = g.nfunc; f < ep_rows; ++f) ep16[f * g.tile_q + rho] = kEpSentinel16;
    __syncthreads();
  } else if constexpr (EPM == 1) {
    if (sp.stage == 2) {
      // lane l of wavefront v loads row 64v + l of every endpoint column
      // (rows past q_len load values nobody reads)
      const rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<int32_t*>(mf + (int64_t)hm * g.nfunc * g.total_q), (short)0,
          (int)((int64_t)g.nfunc * g.total_q * 4), 0x00020000);
      const uint32_t base = (uint32_t)(rg.q_off + rg.i * g.tile_q + 64 * wr + lane) * 4u;
      for (int f = grp; f < g.nfunc; f += ng)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rm, (__attribute__((address_space(3))) void*)&ep[f * g.tile_q + 64 * wr], 4,
            (int)(base + (uint32_t)f * (uint32_t)g.total_q * 4u), 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(0);
    } else if (valid) {
      for (int f = grp; f < g.nfunc; f += ng) ep[f * g.tile_q + rho] = col[(int64_t)f * g.total_q];
    }
    if (is_row && grp == 0)
      for (int f = g.nfunc; f < ep_rows; ++f) ep[f * g.tile_q + rho] = INT_MAX;
    __syncthreads();
  }
  // E(f): endpoint f of the row, a value above every column past the last
  // (staged: f < nfunc + kEpPad without a check)
  auto E = [&](int f) -> int {
    if constexpr (EPM == 2) return (int)ep16[f * g.tile_q + rho];
    else if constexpr (EPM == 1) return ep[f * g.tile_q + rho];
    else return f >= g.nfunc ? INT_MAX : col[(int64_t)f * g.total_q];
  };

  // §2: every endpoint in [0, k_len] (EPM 2: checked while staging) and no
  // endpoint below the one before it; group grp takes endpoints grp, grp + ng, ...
  if (valid) {
    for (int f = grp; f < g.nfunc; f += ng) {
      const int e = E(f);
      if (EPM != 2 && (e < 0 || e > rg.k_len)) err |= MPB_DEVERR_RANGE;
      if (f > 0 && e < E(f - 1)) err |= MPB_DEVERR_ORDER;
    }
  }

  // Pass 1 (§4.3): each lane merges its row's touching intervals into runs
  // and ORs the tiles each run touches into an "any" word and the tiles it
  // fully covers into a "full" word, one 32-tile word at a time.  Across the
  // wavefront "any" is OR-ed and "full" AND-ed: a tile is visible if some row
  // sees part of it and full if every one of the T_Q rows covers it, which
  // needs every row in bounds (rows past q_len cover nothing; lanes past T_Q
  // are not rows) and the tile inside k_len (no run passes k_len).
  const int nk = rg.nk, T = g.tile_k;
  const int wk = (nk + 31) >> 5;
  if constexpr (EPM != 0) {
    // Endpoints in LDS: the lane walks its runs along the words, so a run
    // costs one mask per word it touches.  [ra, rb) is the lane's current
    // run ([INT_MAX, INT_MAX) once they are used up).
    const int nint = (g.nfunc + 1) >> 1;
    const int hw = (wk + ng - 1) / ng;
    const int g_w0 = min(grp * hw, wk), g_w1 = min(g_w0 + hw, wk);
    const int sh = 31 - __builtin_clz((uint32_t)T);   // T is a power of two
    int p = 0, ra = INT_MAX, rb = INT_MAX;
    auto advance = [&]() __attribute__((always_inline)) {
      int a = INT_MAX, b = INT_MAX;
      while (p < nint) {   // the next nonempty interval
        const int s = p > 0 ? E(2 * p - 1) : 0, e = E(2 * p);
        ++p;
        if (e > s) {
          a = s;
          b = e;
          break;
        }
      }
      while (p < nint && b != INT_MAX) {   // intervals touching it: one run
        const int s = E(2 * p - 1), e = E(2 * p);
        if (s != b) break;
        b = e;
        ++p;
      }
      ra = a;
      rb = b;
    };
    if (valid && g_w0 < g_w1) {
      // enter at the first interval that ends past the group's first key
      // (binary search; a run that started before it is clipped to the word
      // anyway, so its earlier intervals are not needed)
      const int k0 = (32 * g_w0) << sh;
      int lo = 0, hi = nint;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (E(2 * mid) > k0) hi = mid;
        else lo = mid + 1;
      }
      p = lo;
      advance();
    }
    for (int x = g_w0; x < g_w1; ++x) {
      const int t_lo = 32 * x;
      const int k_lo = t_lo << sh, k_hi = (t_lo + 32) << sh;
      uint32_t any = 0u, full = 0u;
      while (rb <= k_lo) advance();   // runs that end before this word
      while (ra < k_hi) {
        const int t0 = max(ra >> sh, t_lo) - t_lo;
        const int t1 = min(((rb - 1) >> sh) + 1, t_lo + 32) - t_lo;
        any |= range_bits(t0, t1);
        const int f0 = max((ra + T - 1) >> sh, t_lo) - t_lo;
        const int f1 = min(rb >> sh, t_lo + 32) - t_lo;
        if (f1 > f0) full |= range_bits(f0, f1);
        if (rb > k_hi) break;         // the run goes on into the next word
        advance();
      }
      const uint32_t va = wave_or(any);
      const uint32_t vf = wave_and(is_row ? full : 0xFFFFFFFFu);
      if (lane == 0) {
        s_any[wr * g.words_k + x] = va;
        s_nfull[wr * g.words_k + x] = ~vf;
      }
    }
  } else {
    // Endpoints read from HBM: runs in windows of 256 tiles (eight words per
    // lane), the endpoints loaded four intervals at a time.
    {
      const int nint = (g.nfunc + 1) >> 1;
      // group grp: words [g_w0, g_w1) of the item, tiles [32 g_w0, t_end)
      const int hw = (wk + ng - 1) / ng;
      const int g_w0 = min(grp * hw, wk), g_w1 = min(g_w0 + hw, wk);
      const int t_end = min(32 * g_w1, nk);
      for (int tg = 32 * g_w0; tg < t_end; tg += 256) {
        uint32_t am[8], fm[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) am[x] = fm[x] = 0u;
        // tiles [lo, hi) of the window into m; a range inside one word (most
        // runs) costs one mask and a select per word
        auto set_range = [&](uint32_t (&m)[8], int lo, int hi) {
          lo = max(lo, 0);
          hi = min(hi, 256);
          if (hi <= lo) return;
          const int w0 = lo >> 5;
          if (w0 == ((hi - 1) >> 5)) {
            const uint32_t bits = range_bits(lo - 32 * w0, hi - 32 * w0);
#pragma unroll
            for (int x = 0; x < 8; ++x) m[x] |= x == w0 ? bits : 0u;
            return;
          }
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int l = min(max(lo - 32 * x, 0), 32), h = min(max(hi - 32 * x, 0), 32);
            const uint32_t from_l = l >= 32 ? 0u : (0xFFFFFFFFu << l);
            const uint32_t from_h = h >= 32 ? 0u : (0xFFFFFFFFu << h);
            m[x] |= from_l & ~from_h;
          }
        };
        const int w_lo = tg * T, w_hi = min(tg + 256, t_end) * T;
        auto flush = [&](int a, int b) {
          if (b <= a || b <= w_lo || a >= w_hi) return;
          set_range(am, a / T - tg, (b - 1) / T + 1 - tg);
          const int f0 = (a + T - 1) / T - tg, f1 = b / T - tg;
          if (f1 > f0) set_range(fm, f0, f1);
        };
        if (valid) {
          int ra = 0, rb = 0;   // open run [ra, rb), empty while rb <= ra
          for (int p0 = 0; p0 < nint; p0 += 4) {
            int sv[4], ev[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int p = p0 + u;
              sv[u] = p > 0 ? E(2 * p - 1) : 0;
              ev[u] = E(2 * p);   // INT_MAX past the last interval
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              if (p0 + u >= nint) break;
              if (ev[u] <= sv[u]) continue;             // empty interval
              if (rb > ra && sv[u] == rb) {
                rb = ev[u];                             // touching: extend the run
              } else {
                flush(ra, rb);
                ra = sv[u];
                rb = ev[u];
              }
            }
          }
          flush(ra, rb);
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int wd = (tg >> 5) + x;
          if (wd < g_w1) {
            const uint32_t va = wave_or(am[x]);
            const uint32_t vf = wave_and(is_row ? fm[x] : 0xFFFFFFFFu);
            if (lane == 0) {
              s_any[wr * g.words_k + wd] = va;
              s_nfull[wr * g.words_k + wd] = ~vf;
            }
          }
        }
      }
    }
  }
  {
    const uint64_t er = __ballot((err & MPB_DEVERR_RANGE) != 0);
    const uint64_t eo = __ballot((err & MPB_DEVERR_ORDER) != 0);
    if (lane == 0 && (er | eo))
      atomicOr(&s_err, (er ? MPB_DEVERR_RANGE : 0) | (eo ? MPB_DEVERR_ORDER : 0));
  }
  __syncthreads();

  // Words of the item: visible = OR over the wavefronts, full = visible and
  // no wavefront has a row that misses a bit.  Thread tid takes words
  // [per*tid, per*tid + per).
  const int per = (wk + (int)blockDim.x - 1) / (int)blockDim.x;   // at most 4
  const int x0 = per * tid;
  uint32_t pw[4], fw[4];
  int cp = 0, cf = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    pw[u] = fw[u] = 0u;
    const int x = x0 + u;
    if (u < per && x < wk) {
      uint32_t vis = 0u, nfull = 0u;
      for (int v = 0; v < nwr; ++v) {
        vis |= s_any[v * g.words_k + x];
        nfull |= s_nfull[v * g.words_k + x];
      }
      vis &= nk - 32 * x >= 32 ? 0xFFFFFFFFu : ((1u << (nk - 32 * x)) - 1u);   // tiles < nk
      fw[u] = vis & ~nfull;
      pw[u] = vis & ~fw[u];
      cp += __popc(pw[u]);
      cf += __popc(fw[u]);
    }
  }
  // fused builds: the schedule's weights (the scan's barrier publishes them)
  if (sp.fused != 0 && sp.deferred != 0)
    for (int x = tid; x < kKeys * kNumQueues; x += blockDim.x)
      s_fwts[x] = fused_queue_weight(g, x / kNumQueues, x % kNumQueues);
  int pp, pf, pc, fc;
  block_scan2(cp, cf, &pp, &pf, &pc, &fc, s_a, s_b);
  // the ascending partial list into LDS (the payload loop reads it); the
  // first full tile for the schedule
  {
    int k = pp;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t m = pw[u];
      while (m) {
        ptiles[k++] = 32 * (x0 + u) + __ffs(m) - 1;
        m &= m - 1u;
      }
    }
    if (cf > 0 && pf == 0) {
#pragma unroll
      for (int u = 3; u >= 0; --u)
        if (fw[u]) s_ffirst = 32 * (x0 + u) + __ffs(fw[u]) - 1;
    }
  }

  // §4.5 offsets by decoupled look-back (wavefront 0).  Only relaxed atomics:
  // every word carries its whole value, so no other memory has to be made
  // visible with it (a release or acquire at agent scope would write back or
  // invalidate the L2 on every publish).
  if (wv == 0) {
    const uint32_t tag = sp.tag;
    uint64_t* lb = sp.lb;
    if (lane == 0) lb_store(&lb[kLbWords * (int64_t)item], lb_word(tag, ((uint32_t)pc << 16) | (uint32_t)fc));
    int acc_p = 0, acc_f = 0;
    int base = item - 1;
    uint32_t spins = 0;
    bool timeout = false;
    while (true) {
      const int j = base - lane;
      int st = 2, vp = 0, vf = 0;   // before item 0: an inclusive prefix of 0
      if (j >= 0) {
        // the three words in one round of loads
        const uint64_t ag = lb_load(&lb[kLbWords * (int64_t)j]);
        const uint64_t ip = lb_load(&lb[kLbWords * (int64_t)j + 1]);
        const uint64_t iq = lb_load(&lb[kLbWords * (int64_t)j + 2]);
        if ((uint32_t)(ip >> 32) == tag && (uint32_t)(iq >> 32) == tag) {
          vp = (int)(uint32_t)ip;
          vf = (int)(uint32_t)iq;
        } else {
          if ((uint32_t)(ag >> 32) == tag) {
            st = 1;
            vp = (int)((uint32_t)ag >> 16);
            vf = (int)((uint32_t)ag & 0xFFFFu);
          } else {
            st = 0;
          }
        }
      }
      const uint64_t m2 = __ballot(st == 2);
      const int L = m2 ? (int)__ffsll((unsigned long long)m2) - 1 : 64;
      const uint64_t upto = L >= 63 ? ~0ull : ((2ull << L) - 1ull);   // lanes 0..L
      if (__ballot(st == 0) & upto) {   // a needed predecessor has not published
        if (++spins > kLookbackSpins) {
          timeout = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        continue;
      }
      const bool take = lane <= L;
      acc_p += wave_sum(take ? vp : 0);
      acc_f += wave_sum(take ? vf : 0);
      if (L < 64) break;
      base -= 64;
    }
    if (lane == 0) {
      lb_store(&lb[kLbWords * (int64_t)item + 1], lb_word(tag, (uint32_t)(acc_p + pc)));
      lb_store(&lb[kLbWords * (int64_t)item + 2], lb_word(tag, (uint32_t)(acc_f + fc)));
      // offsets fixed: this item's error bits (and a wait that ran out)
      lb_store(&lb[kLbWords * (int64_t)item + 3],
               lb_word(tag, (uint32_t)s_err | (timeout ? kDevErrLookback : 0u)));
      s_pbeg = acc_p;
      s_fbeg = acc_f;
    }
  }
  // fused builds: this row's queue positions, by the second wavefront while
  // the first looks back (by the only one, after it)
  const bool fuse = sp.fused != 0 && sp.deferred != 0;
  if (fuse && wv == ((int)blockDim.x > 64 ? 1 : 0)) {
    const bool ok = fused_row_positions(g, d, sp, n, rows_total, item, pc + fc, s_fwts, s_fcnt,
                                        s_fred, s_frb, s_fsec);
    if (lane == 0) s_fok = ok ? 1 : 0;
  }
  __syncthreads();
  const int p_begin = s_pbeg, f_begin = s_fbeg;
  if (tid == 0) {
    const int first = pc > 0 ? ptiles[0] : s_ffirst;
    d.p_off[item] = p_begin;
    d.f_off[item] = f_begin;
    w.first_tile[(int64_t)hm * g.upper_rows + row] = first;
  }
  // §4.5 header: with a host read-back it goes out before this item's own
  // lists and payload (the host waits for it); deferred, after them (only
  // the kernel's end matters then).
  const bool deferred = sp.deferred != 0;
  auto publish = [&]() __attribute__((always_inline)) {
    if (item == n - 1) {
      // The header waits until every item has fixed its offsets (each did so
      // from its predecessors' words alone, so these waits end), and carries
      // the OR of their error bits.
      const uint32_t tag = sp.tag;
      uint32_t err_all = 0;
      for (int j = tid; j < n; j += blockDim.x) {
        const uint64_t* wj = sp.lb + kLbWords * (int64_t)j;
        uint32_t spins = 0;
        uint64_t v = lb_load(wj + 3);
        while ((uint32_t)(v >> 32) != tag) {
          if (++spins > kLookbackSpins) {
            v = lb_word(tag, kDevErrLookback);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          v = lb_load(wj + 3);
        }
        err_all |= (uint32_t)v;
      }
      if (err_all) atomicOr(&s_err2, err_all);
      __syncthreads();
      uint32_t e = (uint32_t)s_err2;
      if (g.layout == MPB_LAYOUT_THD) e |= (uint32_t)w.geo_err[0];
      if (tid == 0) {
        d.p_off[n] = p_begin + pc;
        d.f_off[n] = f_begin + fc;
        sp_publish(d, sp, rows_total, p_begin + pc, f_begin + fc, e);
      }
      // fused builds: the queue starts and the fixed-length geometry (§4.2,
      // in closed form)
      if (fuse && e == 0) {
        if (tid <= kNumQueues) d.section_off[tid] = s_fsec[tid];
        if (g.layout == MPB_LAYOUT_BSHD) {
          const int rps = (g.seqlen_q + g.tile_q - 1) / g.tile_q;
          for (int b = tid; b < g.batch; b += blockDim.x) {
            int4* sd = reinterpret_cast<int4*>(d.seqdesc + 8 * b);
            sd[0] = make_int4(b * g.seqlen_q, b * g.seqlen_k, g.seqlen_q, g.seqlen_k);
            sd[1] = make_int4(b * rps, rps, (g.seqlen_k + g.tile_k - 1) / g.tile_k, 0);
            d.cu_rows[b + 1] = (b + 1) * rps;
          }
          if (tid == 0) d.cu_rows[0] = 0;
        }
      }
    }
    // fused builds: every item writes its own row's tasks (one per Q head, or
    // the one task of a per-head mask row).  Their slots stay in bounds
    // whatever other items found, and a failed build's header keeps the
    // forward from reading them.
    if (fuse && s_fok != 0 && (g.layout != MPB_LAYOUT_THD || w.geo_err[0] == 0)) {
      int so[kNumQueues + 1];
#pragma unroll
      for (int s = 0; s <= kNumQueues; ++s) so[s] = s_fsec[s];
      const int first = pc > 0 ? ptiles[0] : s_ffirst;
      const int h_lo = g.mask_heads == 1 ? 0 : hm;
      const int h_hi = g.mask_heads == 1 ? g.heads_q : hm + 1;
      for (int h = h_lo + tid; h < h_hi; h += blockDim.x)
        place_task(g, d, (const int*)s_frb, nullptr, so, rows_total, item, h, p_begin, pc,
                   f_begin, fc, first);
    }
  };
  if (!deferred) publish();
  // §4.6 lists, flat CSR order, to the workspace
  for (int k = tid; k < pc; k += blockDim.x) sp.p_list[p_begin + k] = ptiles[k];
  {
    int k = f_begin + pf;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t m = fw[u];
      while (m) {
        sp.f_list[k++] = 32 * (x0 + u) + __ffs(m) - 1;
        m &= m - 1u;
      }
    }
  }
  // §5 payload of every partial tile
  if (pc > 0) {
    if constexpr (EPM != 0) {
      // group grp writes partial tiles [k0, k1)
      const int k0 = (pc * grp) / ng, k1 = (pc * (grp + 1)) / ng;
      if (k1 > k0)
        row_payload_tight(g, ptiles, k0, k1, E, rho, valid, is_row, d.p_masks, p_begin);
    } else {
      if (grp == 0) row_payload_e(g, ptiles, pc, E, rho, valid, is_row, d.p_masks, p_begin);
    }
  }
  if (deferred) publish();
}

// The tail of a single-pass build: workgroup 0 runs the schedule (§4.8) on
// the finished offsets; the others place the partial and full lists behind
// the payload, where the exact block has them: the payload holds
// pnnz * T_Q * words_tile words, then come pnnz partial and fnnz full
// indices, each array starting on a 256-byte boundary (the host binds the
// same places once it has read the header).
__global__ __launch_bounds__(1024) void plan_single_pass_tail_kernel(PlanGeo g, PlanDev d,
                                                                     PlanWork w, SinglePass sp,
                                                                     int cnt_in_lds,
                                                                     int rows_in_lds,
                                                                     int place_lists) {
  extern __shared__ int dyn[];
  // With the sort in LDS every workgroup sorts and writes its share of the
  // tasks (after its share of the lists); else workgroup 0 alone schedules.
  const bool shared_sort = cnt_in_lds && rows_in_lds == 2;
  if (blockIdx.x == 0 && !shared_sort) {
    schedule_any(g, d, w, cnt_in_lds, rows_in_lds, dyn);
    return;
  }
  if (d.header[7] != 0) return;   // failed build: nothing to place
  if (!place_lists) {   // the lists are in place already: schedule only
    schedule_any(g, d, w, cnt_in_lds, rows_in_lds, dyn, blockIdx.x, gridDim.x);
    return;
  }
  const int64_t pn = d.header[1], fn = d.header[2];
  auto padded = [](int64_t bytes) -> int64_t { return (bytes + 255) & ~(int64_t)255; };
  const int64_t mask_words = pn * g.tile_q * g.words_tile;
  const int64_t mask_bytes = padded((mask_words > 0 ? mask_words : 1) * 4);
  int32_t* p_dst = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(d.p_masks) + mask_bytes);
  int32_t* f_dst = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(p_dst) +
                                              padded((pn > 0 ? pn : 1) * 4));
  const int copiers = shared_sort ? (int)gridDim.x : (int)gridDim.x - 1;
  const int me = shared_sort ? (int)blockIdx.x : (int)blockIdx.x - 1;
  const int64_t stride = (int64_t)copiers * blockDim.x;
  for (int64_t x = (int64_t)me * blockDim.x + threadIdx.x; x < pn + fn; x += stride) {
    if (x < pn) p_dst[x] = sp.p_list[x];
    else f_dst[x - pn] = sp.f_list[x - pn];
  }
  if (shared_sort) schedule_any(g, d, w, cnt_in_lds, rows_in_lds, dyn, blockIdx.x, gridDim.x);
}


// ---------------------------------------------------------------- backward K2Q view

namespace {

// Q rows [row_begin, row_begin + nrows) and K tiles nk of sample b.
struct SampleRows {
  int row_begin, nrows, nk, q_off, q_len, k_len;
};
__device__ inline SampleRows sample_rows(const PlanGeo& g, const PlanDev& d, int b) {
  SampleRows r;
  if (g.layout == MPB_LAYOUT_BSHD) {
    const int rps = (g.seqlen_q + g.tile_q - 1) / g.tile_q;
    r.row_begin = b * rps;
    r.nrows = rps;
    r.nk = (g.seqlen_k + g.tile_k - 1) / g.tile_k;
    r.q_off = b * g.seqlen_q;
    r.q_len = g.seqlen_q;
    r.k_len = g.seqlen_k;
  } else {
    const int32_t* sd = d.seqdesc + 8 * b;
    r.q_off = sd[0];
    r.q_len = sd[2];
    r.k_len = sd[3];
    r.row_begin = sd[4];
    r.nrows = sd[5];
    r.nk = sd[6];
  }
  return r;
}

}  // namespace

// §4.4 K2Q counting, the count phase of a sparse transpose of the
// classifier's bitsets: one wavefront per (mask head, sample, 32-tile word
// of K tiles).  For every 64 Q rows of the sample the lanes load their row's
// word; one ballot per K tile and class counts the partial and full Q
// contributors, kept by lane j for K tile 32w + j.  The last workgroup (same
// ticket protocol as the classifier) lays the K rows out per sample
// (cu_krows), scans the counts into compact head-major exclusive offsets and
// publishes the header's backward values {Q rows, K rows, partial nnz, full
// nnz} (slots 3..6) with its own sequence number.
__global__ __launch_bounds__(256) void plan_k2q_count_kernel(PlanGeo g, PlanDev d, PlanWork w,
                                                             K2QWork kw, int32_t* arrive,
                                                             int32_t* host_slot, int32_t seq) {
  __shared__ int s_last;
  __shared__ int s_wp[4], s_wf[4];
  __shared__ int s_cu[1025];
  __shared__ int s_hist[kK2QOrderBuckets];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t items = (int64_t)g.mask_heads * g.batch * g.words_k;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  // a failed classification (bad endpoints or prefixes) leaves the geometry
  // and bitsets meaningless: count nothing, publish zeros
  const bool failed = d.header[7] != 0;
  if (item < items && !failed) {
    const int wi = (int)(item % g.words_k);
    const int64_t hb = item / g.words_k;
    const int b = (int)(hb % g.batch);
    const int hm = (int)(hb / g.batch);
    const SampleRows sr = sample_rows(g, d, b);
    int mp = 0, mf = 0;
    for (int r0 = 0; r0 < sr.nrows; r0 += 64) {
      uint32_t vis = 0u, full = 0u;
      if (r0 + lane < sr.nrows && sr.row_begin + r0 + lane < g.upper_rows) {
        const int64_t src = ((int64_t)hm * g.upper_rows + sr.row_begin + r0 + lane) * g.words_k + wi;
        vis = w.vis_bits[src];
        full = w.full_bits[src];
      }
      const uint32_t part = vis & ~full;
#pragma unroll 4
      for (int j = 0; j < 32; ++j) {
        const int cp = __popcll(__ballot((part >> j) & 1u));
        const int cf = __popcll(__ballot((full >> j) & 1u));
        if (lane == j) {
          mp += cp;
          mf += cf;
        }
      }
    }
    const int kt = 32 * wi + lane;
    if (lane < 32 && kt < sr.nk) {
      const int64_t dst = ((int64_t)hm * g.batch + b) * g.nk_max + kt;
      kw.pcnt[dst] = mp;
      kw.fcnt[dst] = mf;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (int)gridDim.x - 1 ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __atomic_thread_fence(__ATOMIC_ACQUIRE);
  if (threadIdx.x == 0) __hip_atomic_store(arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // K rows per sample: cu_krows (one thread per sample, then a serial pass
  // over the wavefront totals; B <= 1024 samples are kept in LDS)
  const int tid = threadIdx.x;
  auto offsets = [&](auto cu) {
  for (int b = tid; b < g.batch; b += 256) cu[b + 1] = failed ? 0 : sample_rows(g, d, b).nk;
  __syncthreads();
  if (tid == 0) {
    cu[0] = 0;
    for (int b = 0; b < g.batch; ++b) cu[b + 1] += cu[b];
  }
  __syncthreads();
  const int krows = cu[g.batch];
  for (int b = tid; b <= g.batch; b += 256) kw.cu_krows[b] = cu[b];
  const int n = g.mask_heads * krows;
  // compact exclusive offsets over flat = hm * krows + krow: thread t scans
  // the contiguous segment [t*per, (t+1)*per) (its loads all in flight, the
  // sample advanced along the segment instead of searched per element),
  // then the 256 segment totals are scanned
  const int per = (n + 255) / 256;
  const int f0 = min(n, tid * per), f1 = min(n, f0 + per);
  auto walk = [&](auto&& visit) {
    if (f0 >= f1) return;
    int hm = f0 / krows, kr = f0 - hm * krows;
    int b = sample_of_row(cu, g.batch, kr);
    for (int f = f0; f < f1; ++f) {
      while (kr >= cu[b + 1]) ++b;
      visit(f, ((int64_t)hm * g.batch + b) * g.nk_max + (kr - cu[b]));
      if (++kr == krows) {
        kr = 0;
        b = 0;
        ++hm;
      }
    }
  };
  int sp = 0, sf = 0;
  walk([&](int, int64_t src) {
    sp += kw.pcnt[src];
    sf += kw.fcnt[src];
  });
  const int ip = wave_incl_scan(sp, lane);
  const int jf = wave_incl_scan(sf, lane);
  if (lane == 63) {
    s_wp[wv] = ip;
    s_wf[wv] = jf;
  }
  __syncthreads();
  int carry_p = ip - sp, carry_f = jf - sf, tot_p = 0, tot_f = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    if (x < wv) {
      carry_p += s_wp[x];
      carry_f += s_wf[x];
    }
    tot_p += s_wp[x];
    tot_f += s_wf[x];
  }
  walk([&](int f, int64_t src) {
    kw.p_off[f] = carry_p;
    kw.f_off[f] = carry_f;
    carry_p += kw.pcnt[src];
    carry_f += kw.fcnt[src];
  });
  carry_p = tot_p;
  carry_f = tot_f;

  // Launch order of the K rows for a backward consumer: descending cost
  // summed over mask heads (partial + full Q tiles), ties by K row, by a
  // counting sort (histogram in LDS, then one wavefront places the rows in
  // order, ranking equal keys by one ballot per key bit).  Heavy K rows then
  // start first instead of forming the tail of the grid.
  auto cost = [&](int k) -> int {
    int b2 = sample_of_row(cu, g.batch, k);
    const int jj = k - cu[b2];
    int c = 0;
    for (int hm = 0; hm < g.mask_heads; ++hm) {
      const int64_t src = ((int64_t)hm * g.batch + b2) * g.nk_max + jj;
      c += kw.pcnt[src] + kw.fcnt[src];
    }
    return c;
  };
  const int maxc = kw.max_cost;
  if (maxc < kK2QOrderBuckets) {
    for (int x = tid; x <= maxc; x += 256) s_hist[x] = 0;
    __syncthreads();
    for (int k = tid; k < krows; k += 256) atomicAdd(&s_hist[maxc - min(cost(k), maxc)], 1);
    __syncthreads();
    if (wv == 0) {
      int run = 0;
      for (int x0 = 0; x0 <= maxc; x0 += 64) {
        const int x = x0 + lane;
        const int v = x <= maxc ? s_hist[x] : 0;
        const int inc = wave_incl_scan(v, lane);
        if (x <= maxc) s_hist[x] = run + inc - v;
        run += __builtin_amdgcn_readlane(inc, 63);
      }
      const uint64_t below = lanes_below(lane);
      for (int k0 = 0; k0 < krows; k0 += 64) {
        const int k = k0 + lane;
        const bool valid = k < krows;
        const int key = valid ? maxc - min(cost(k), maxc) : 0;
        uint64_t same = __ballot(valid);
        for (int bit = 0; (1 << bit) <= maxc; ++bit) {
          const uint64_t ones = __ballot(valid && ((key >> bit) & 1));
          same &= ((key >> bit) & 1) ? ones : ~ones;
        }
        const int pos = valid ? s_hist[key] + __popcll(same & below) : 0;
        const bool leader = valid && (same & below) == 0;
        if (valid) kw.order[pos] = k;
        __builtin_amdgcn_wave_barrier();
        if (leader) s_hist[key] += __popcll(same);
        __builtin_amdgcn_wave_barrier();
      }
    }
  } else {
    for (int k = tid; k < krows; k += 256) kw.order[k] = k;
  }
  if (tid == 0) {
    kw.p_off[n] = carry_p;
    kw.f_off[n] = carry_f;
    kw.info[0] = krows;
    kw.info[1] = carry_p;
    kw.info[2] = carry_f;
    kw.info[3] = 0;
    const int32_t vals[4] = {d.header[0], krows, carry_p, carry_f};
    for (int i = 0; i < 4; ++i) {
      d.header[3 + i] = vals[i];
      __hip_atomic_store(&host_slot[3 + i], vals[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    __hip_atomic_store(&host_slot[kHeaderSeq2], seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  };
  if (g.batch < 1025) offsets((lds_ptr)s_cu);
  else offsets(kw.cu_krows);
}

namespace {

// Lanes L and L ^ J of a wavefront swap one dword: DPP quad permutes for
// J = 1, 2, a swizzle within 32 lanes for J = 4, 8, 16, a lane permute
// across the halves for J = 32.
template <int J>
__device__ inline uint32_t xor_lane(uint32_t v) {
  if constexpr (J == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  else if constexpr (J == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  else if constexpr (J < 32) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (J << 10));
  else return (uint32_t)__shfl_xor((int)v, 32);
}

// One butterfly stage of a 64 x 64 bit transpose: between lanes L and L ^ J
// swap the bits b with (b & J) != 0 of the lower lane and (b & J) == 0 of
// the upper one (M: the bits with (b & J) == 0 of a dword).
template <int J, uint32_t M>
__device__ inline void butterfly(uint32_t& lo, uint32_t& hi, int lane) {
  const uint32_t plo = xor_lane<J>(lo), phi = xor_lane<J>(hi);
  if ((lane & J) == 0) {
    lo = (lo & M) | ((plo & M) << J);
    hi = (hi & M) | ((phi & M) << J);
  } else {
    lo = (lo & ~M) | ((plo & ~M) >> J);
    hi = (hi & ~M) | ((phi & ~M) >> J);
  }
}

// Transposes the 64 x 64 bit matrix whose row c is lane c's (lo, hi): on
// return lane r holds column r, bit c = old bit r of lane c (recursive
// block transpose: swap the off-diagonal halves, then recurse in place).
__device__ inline void transpose_bits64(uint32_t& lo, uint32_t& hi, int lane) {
  const bool top = lane < 32;
  const uint32_t got = xor_lane<32>(top ? hi : lo);
  if (top) hi = got; else lo = got;
  butterfly<16, 0x0000FFFFu>(lo, hi, lane);
  butterfly<8, 0x00FF00FFu>(lo, hi, lane);
  butterfly<4, 0x0F0F0F0Fu>(lo, hi, lane);
  butterfly<2, 0x33333333u>(lo, hi, lane);
  butterfly<1, 0x55555555u>(lo, hi, lane);
}

}  // namespace

// §4.7 K2Q materialization, one workgroup of 256 threads per (mask head, K
// plan row).  The Q tiles of the K row's sample are read from the bitsets in
// ascending order, ranked with one ballot per wavefront and written to the
// partial and full lists.  The K-major predicate of a partial pair is the
// transpose of the same pair's Q2K payload, already in the plan: the thread
// that found pair (i, j) also locates it in row i's Q2K list (row offset plus
// the partial tiles of the row before j, counted in the bitsets) and keeps
// the list and that position in LDS (lds_list = 1: the longest sample's Q
// tiles fit; otherwise both are read back or recounted).  Then the
// wavefronts take the pairs in turn: a lane per Q row loads its row's
// T_KV-bit word(s), each 64-row half is transposed across the wavefront and
// lane r writes K row r's T_Q/32 words with one store.
__global__ __launch_bounds__(256) void plan_k2q_materialize_kernel(
    PlanGeo g, PlanDev d, PlanWork w, K2QWork kw, K2QDev kd, int krows_total, int lds_list) {
  extern __shared__ int qlds[];   // [rps_max] partial Q tiles, then [rps_max] Q2K positions
  __shared__ int s_wp[4], s_wf[4];
  __shared__ int s_cu[1025];
  if (krows_total < 0) {   // launched before the header was read back
    if (d.header[7] != 0) return;
    krows_total = kw.info[0];
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int item = blockIdx.x;
  const int n = g.mask_heads * krows_total;
  if (item == 0) {   // also when there are no K rows at all
    for (int x = tid; x <= g.batch; x += 256) kd.cu_krows[x] = kw.cu_krows[x];
    if (tid == 0) {
      kd.p_off[n] = kw.p_off[n];
      kd.f_off[n] = kw.f_off[n];
    }
  }
  if (item < krows_total && threadIdx.x == 0) kd.order[item] = kw.order[item];
  if (item >= n) return;
  const int hm = item / krows_total, kr = item - hm * krows_total;
  int b, j;
  if (g.batch < 1025) {
    for (int x = tid; x <= g.batch; x += 256) s_cu[x] = kw.cu_krows[x];
    __syncthreads();
    b = sample_of_row((lds_cptr)s_cu, g.batch, kr);
    j = kr - ((lds_cptr)s_cu)[b];
  } else {
    b = sample_of_row(kw.cu_krows, g.batch, kr);
    j = kr - kw.cu_krows[b];
  }
  const SampleRows sr = sample_rows(g, d, b);
  const int p_begin = kw.p_off[item], f_begin = kw.f_off[item];
  const int rows_total = d.header[0];
  if (tid == 0) {
    kd.p_off[item] = p_begin;
    kd.f_off[item] = f_begin;
  }
  const int rps_max = (g.seqlen_q + g.tile_q - 1) / g.tile_q;
  int* qlist = qlds;
  int* qpos = qlds + rps_max;
  const int jw = j >> 5;
  const uint32_t jbit = 1u << (j & 31);
  // position of pair (i, j) in Q row i's partial list
  auto q2k_pos = [&](int i, uint32_t part_j) -> int {
    const int64_t rs = ((int64_t)hm * g.upper_rows + sr.row_begin + i) * g.words_k;
    int below = __popc(part_j & (jbit - 1u));
    for (int x = 0; x < jw; ++x) below += __popc(w.vis_bits[rs + x] & ~w.full_bits[rs + x]);
    return d.p_off[(int64_t)hm * rows_total + sr.row_begin + i] + below;
  };

  // lists, ascending Q tile
  const uint64_t below = lanes_below(lane);
  int base_p = 0, base_f = 0;
  for (int i0 = 0; i0 < sr.nrows; i0 += 256) {
    const int i = i0 + tid;
    bool isp = false, isf = false;
    uint32_t part = 0u;
    if (i < sr.nrows) {
      const int64_t src = ((int64_t)hm * g.upper_rows + sr.row_begin + i) * g.words_k + jw;
      const uint32_t vis = w.vis_bits[src], full = w.full_bits[src];
      part = vis & ~full;
      isf = (full & jbit) != 0u;
      isp = (part & jbit) != 0u;
    }
    const uint64_t bp = __ballot(isp), bf = __ballot(isf);
    if (lane == 0) {
      s_wp[wv] = __popcll(bp);
      s_wf[wv] = __popcll(bf);
    }
    __syncthreads();
    int pre_p = base_p, pre_f = base_f;
    for (int x = 0; x < wv; ++x) {
      pre_p += s_wp[x];
      pre_f += s_wf[x];
    }
    if (isp) {
      const int rk = pre_p + __popcll(bp & below);
      kd.p_idx[p_begin + rk] = i;
      if (lds_list) {
        qlist[rk] = i;
        qpos[rk] = q2k_pos(i, part);
      }
    }
    if (isf) kd.f_idx[f_begin + pre_f + __popcll(bf & below)] = i;
    for (int x = 0; x < 4; ++x) {
      base_p += s_wp[x];
      base_f += s_wf[x];
    }
    __syncthreads();
  }
  const int np = base_p;

  // payload, K-major: [pair][T_KV][T_Q/32]; wavefront wv takes pairs wv, wv + 4, ...
  const int wt = g.tile_k >> 5;     // words of a Q2K row (1 or 2)
  const int wq = g.tile_q >> 5;     // words of a K2Q row
  const int halves = (g.tile_q + 63) >> 6;
  auto pos_of = [&](int x) -> int {
    if (lds_list) return qpos[x];
    const int i = kd.p_idx[p_begin + x];   // written above by this workgroup
    const int64_t src = ((int64_t)hm * g.upper_rows + sr.row_begin + i) * g.words_k + jw;
    return q2k_pos(i, w.vis_bits[src] & ~w.full_bits[src]);
  };
  for (int x = wv; x < np; x += 4) {
    const int64_t pos = pos_of(x);
    uint32_t lo[2], hi[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      lo[h] = hi[h] = 0u;
      const int c = 64 * h + lane;   // Q row of the tile
      if (h < halves && c < g.tile_q) {
        const uint32_t* src = d.p_masks + (pos * g.tile_q + c) * wt;
        lo[h] = src[0];
        if (wt == 2) hi[h] = src[1];
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (h < halves) transpose_bits64(lo[h], hi[h], lane);
    if (lane < g.tile_k) {
      uint32_t* dst = kd.p_masks + ((int64_t)(p_begin + x) * g.tile_k + lane) * wq;
      if (wq == 4) *reinterpret_cast<uint4*>(dst) = make_uint4(lo[0], hi[0], lo[1], hi[1]);
      else if (wq == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(lo[0], hi[0]);
      else dst[0] = lo[0];
    }
  }
}

// ---------------------------------------------------------------- launchers

static inline int rows_per_lane(int tile_q) { return tile_q <= 64 ? 1 : tile_q / 64; }

// Where the schedule keeps its row data: 2 offsets, first tiles, order and
// first positions in LDS, 1 all but the first positions, 0 none -- as much
// as fits 120 KiB beside the count matrix (cnt_bytes of LDS, 0 when it is in
// the workspace); at most kSchedLdsRows rows either way.
static inline int sched_rows_in_lds(int64_t rows, size_t cnt_bytes) {
  if (rows > kSchedLdsRows) return 0;
  const size_t two = cnt_bytes + (size_t)(4 * rows + 2 + kNumQueues * rows) * 4;
  const size_t one = cnt_bytes + (size_t)(4 * rows + 2) * 4;
  return two <= 120 * 1024 ? 2 : one <= 120 * 1024 ? 1 : 0;
}

hipError_t launch_plan_geometry(const PlanGeo& g, const int32_t* cu_q_in, const int32_t* cu_k_in,
                                const PlanDev& d, const PlanWork& w, hipStream_t s) {
  if (g.layout != MPB_LAYOUT_THD) return hipSuccess;
  hipLaunchKernelGGL(plan_geometry_kernel, dim3(1), dim3(1024), 0, s, g, cu_q_in, cu_k_in, d, w);
  return hipGetLastError();
}

hipError_t launch_plan_classify(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                                const PlanWork& w, int32_t* arrive, int32_t* host_slot,
                                int32_t seq, hipStream_t s) {
  const int64_t items = (int64_t)g.mask_heads * g.upper_rows;
  // At least one workgroup, so the header is always published.
  const dim3 grid((unsigned)(items > 0 ? (items + 3) / 4 : 1)), block(256);
  // 128-tile windows when every sample fits in one, else 256-tile windows
  const bool wide = g.nk_max > 128;
#define MPB_CLASSIFY(R, WW_) \
  hipLaunchKernelGGL((plan_classify_kernel<R, WW_>), grid, block, 0, s, g, mask_func, d, w, arrive, host_slot, seq)
  switch (rows_per_lane(g.tile_q)) {
    case 1: if (wide) MPB_CLASSIFY(1, 8); else MPB_CLASSIFY(1, 4); break;
    case 2: if (wide) MPB_CLASSIFY(2, 8); else MPB_CLASSIFY(2, 4); break;
    case 4: if (wide) MPB_CLASSIFY(4, 8); else MPB_CLASSIFY(4, 4); break;
    default: return hipErrorInvalidValue;
  }
#undef MPB_CLASSIFY
  return hipGetLastError();
}

hipError_t launch_plan_schedule(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                hipStream_t s) {
  const int64_t rows = (int64_t)g.mask_heads * g.upper_rows;
  const size_t cnt_bytes = w.chunk_cnt ? 0 : (size_t)(g.nk_max + 1) * w.nchunks * 4;
  // 0: row data in the workspace; 1: in LDS; 2: their first positions too
  const int rows_in_lds = sched_rows_in_lds(rows, cnt_bytes);
  const size_t row_bytes =
      rows_in_lds ? (size_t)(4 * rows + 2 + (rows_in_lds == 2 ? kNumQueues * rows : 0)) * 4 : 0;
  hipLaunchKernelGGL(plan_schedule_kernel, dim3(1), dim3(1024), cnt_bytes + row_bytes, s, g, d,
                     w, w.chunk_cnt ? 0 : 1, rows_in_lds);
  return hipGetLastError();
}

hipError_t launch_plan_materialize(const PlanGeo& g, const int32_t* mask_func, const PlanDev& st,
                                   const PlanDev& d, const PlanWork& w, int32_t rows_total,
                                   hipStream_t s) {
  // rows_total < 0: rows counted on the device, one workgroup per row of the
  // upper bound; st == d: the metadata is already in place, nothing to copy
  const int64_t items = (int64_t)g.mask_heads * (rows_total >= 0 ? rows_total : g.upper_rows);
  const int64_t tasks = (int64_t)(rows_total >= 0 ? rows_total : 0) * g.heads_q;
  MetaCopy mc;
  int nseg = 0;
  int64_t run = 0;
  auto seg = [&](const int32_t* src, int32_t* dst, int64_t count) {
    mc.src[nseg] = src;
    mc.dst[nseg] = dst;
    run += count;
    mc.end[nseg++] = run;
  };
  if (st.header != d.header) {
    seg(st.header, d.header, 8);
    seg(st.seqdesc, d.seqdesc, 8 * (int64_t)g.batch);
    seg(st.cu_rows, d.cu_rows, g.batch + 1);
    seg(st.cu_q, d.cu_q, g.layout == MPB_LAYOUT_THD ? g.batch + 1 : 0);
    seg(st.cu_k, d.cu_k, g.layout == MPB_LAYOUT_THD ? g.batch + 1 : 0);
    seg(st.work_desc, d.work_desc, 4 * tasks);
    seg(st.section_off, d.section_off, kNumQueues + 1);
    seg(st.task_rec, d.task_rec, kTaskRecInts * tasks);
  }
  mc.total = run;
  const int threads = g.tile_q < 64 ? 64 : g.tile_q;
  const size_t ep_bytes = (size_t)g.nfunc * g.tile_q * 4;
  // 0: endpoints read from HBM as needed; 1: staged in LDS through registers;
  // 2: staged with loads straight into LDS (whole wavefronts of rows, and a
  // mask head's endpoints addressable with 32-bit offsets)
  int stage = ep_bytes <= 32 * 1024 ? 1 : 0;
  if (stage && g.tile_q >= 64 && (int64_t)g.nfunc * g.total_q * 4 < ((int64_t)1 << 31)) stage = 2;
  const size_t lds = (size_t)g.nk_max * 4 + (stage ? ep_bytes : 0);
  hipLaunchKernelGGL(plan_materialize_kernel, dim3((unsigned)(items > 0 ? items : 1)),
                     dim3(threads), lds, s, g, mask_func, st, d, w, rows_total, stage, mc);
  return hipGetLastError();
}


namespace {
struct FinishShape {
  int rows_in_lds, stage, per_wg;
  size_t lds;
};
FinishShape finish_shape(const PlanGeo& g, bool cnt_in_lds, int64_t nchunks) {
  FinishShape f;
  const int64_t rows = (int64_t)g.mask_heads * g.upper_rows;
  const size_t cnt_bytes = cnt_in_lds ? (size_t)(g.nk_max + 1) * nchunks * 4 : 0;
  f.rows_in_lds = sched_rows_in_lds(rows, cnt_bytes);
  const size_t row_bytes =
      f.rows_in_lds ? (size_t)(4 * rows + 2 + (f.rows_in_lds == 2 ? kNumQueues * rows : 0)) * 4
                    : 0;
  const int sg = g.tile_q < 64 ? 64 : g.tile_q;
  f.per_wg = 1024 / sg;
  const size_t ep_bytes = (size_t)g.nfunc * g.tile_q * 4;
  // endpoints staged in LDS when every row of a workgroup fits in 96 KiB
  f.stage = (size_t)f.per_wg * ((size_t)g.nk_max * 4 + ep_bytes) <= 96 * 1024 ? 1 : 0;
  if (f.stage && g.tile_q >= 64 && (int64_t)g.nfunc * g.total_q * 4 < ((int64_t)1 << 31))
    f.stage = 2;
  const size_t mat_bytes = (size_t)f.per_wg * ((size_t)g.nk_max * 4 + (f.stage ? ep_bytes : 0));
  f.lds = std::max(cnt_bytes + row_bytes, mat_bytes);
  return f;
}
}  // namespace

bool plan_finish_fits(const PlanGeo& g, bool cnt_in_lds, int64_t nchunks) {
  return finish_shape(g, cnt_in_lds, nchunks).lds <= 120 * 1024;
}

hipError_t launch_plan_finish(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                              const PlanWork& w, int32_t rows_total, hipStream_t s) {
  const FinishShape f = finish_shape(g, w.chunk_cnt == nullptr, w.nchunks);
  const int rows_in_lds = f.rows_in_lds, stage = f.stage, per_wg = f.per_wg;
  const size_t lds = f.lds;
  const int64_t items = (int64_t)g.mask_heads * (rows_total >= 0 ? rows_total : g.upper_rows);
  const unsigned grid = (unsigned)(1 + (items + per_wg - 1) / per_wg);
  hipLaunchKernelGGL(plan_finish_kernel, dim3(grid), dim3(1024), lds, s, g, mask_func, d, w,
                     rows_total, stage, w.chunk_cnt ? 0 : 1, rows_in_lds);
  return hipGetLastError();
}


hipError_t launch_plan_single_pass(const PlanGeo& g, const int32_t* mask_func, const PlanDev& d,
                                   const PlanWork& w, const SinglePass& sp, int32_t rows_total,
                                   hipStream_t s) {
  const int64_t items = (int64_t)g.mask_heads * (rows_total >= 0 ? rows_total : g.upper_rows);
  // two groups of T_Q threads per item when the endpoints are staged and
  // T_Q is 64 or 128 (twice the wavefronts to hide the walks' latency)
  const int sg = g.tile_q < 64 ? 64 : g.tile_q;
  const int threads = (sp.stage != 0 && sg <= 128) ? 2 * sg : sg;
  const int nw = sg / 64;
  const size_t ep_rows = (size_t)g.nfunc + kEpPad;
  const size_t ep_ints = sp.stage == 3   ? (ep_rows * g.tile_q + 1) / 2
                         : sp.stage != 0 ? ep_rows * g.tile_q
                                         : 0;
  size_t lds = ep_ints * 4 + (size_t)2 * nw * g.words_k * 4 + (size_t)g.nk_max * 4;
  // at least one workgroup, so the header is always published
  const dim3 grid((unsigned)(items > 0 ? items : 1)), block(threads);
  if (sp.stage == 3)
    hipLaunchKernelGGL(plan_single_pass_kernel<2>, grid, block, lds, s, g, mask_func, d, w, sp);
  else if (sp.stage != 0)
    hipLaunchKernelGGL(plan_single_pass_kernel<1>, grid, block, lds, s, g, mask_func, d, w, sp);
  else
    hipLaunchKernelGGL(plan_single_pass_kernel<0>, grid, block, lds, s, g, mask_func, d, w, sp);
  return hipGetLastError();
}

hipError_t launch_plan_single_pass_tail(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                        const SinglePass& sp, int64_t tiles_upper,
                                        bool place_lists, hipStream_t s) {
  const int64_t rows = (int64_t)g.mask_heads * g.upper_rows;
  const size_t cnt_bytes = w.chunk_cnt ? 0 : (size_t)(g.nk_max + 1) * w.nchunks * 4;
  const int rows_in_lds = sched_rows_in_lds(rows, cnt_bytes);
  const size_t row_bytes =
      rows_in_lds ? (size_t)(4 * rows + 2 + (rows_in_lds == 2 ? kNumQueues * rows : 0)) * 4 : 0;
  // list placement (four indices per thread) and, with the sort in LDS,
  // tasks (one per thread): up to 256 more workgroups of 1024 threads
  const int64_t tasks = (int64_t)g.upper_rows * g.heads_q;
  const bool shared_sort = !w.chunk_cnt && rows_in_lds == 2;
  int64_t copy_wgs = place_lists ? (2 * tiles_upper + 4095) / 4096 : 0;
  if (shared_sort) copy_wgs = std::max(copy_wgs, (tasks + 1023) / 1024 - 1);
  copy_wgs = copy_wgs < (place_lists ? 1 : 0) ? 1 : (copy_wgs > 256 ? 256 : copy_wgs);
  // without list placement and without the shared sort, workgroup 0 alone
  // schedules (the kernel then returns from every other workgroup at once)
  if (!place_lists && !shared_sort) copy_wgs = 0;
  hipLaunchKernelGGL(plan_single_pass_tail_kernel, dim3((unsigned)(1 + copy_wgs)), dim3(1024),
                     cnt_bytes + row_bytes, s, g, d, w, sp, w.chunk_cnt ? 0 : 1, rows_in_lds,
                     place_lists ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_plan_k2q_count(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                 const K2QWork& kw, int32_t* arrive, int32_t* host_slot,
                                 int32_t seq, hipStream_t s) {
  const int64_t items = (int64_t)g.mask_heads * g.batch * g.words_k;
  const dim3 grid((unsigned)(items > 0 ? (items + 3) / 4 : 1)), block(256);
  hipLaunchKernelGGL(plan_k2q_count_kernel, grid, block, 0, s, g, d, w, kw, arrive, host_slot,
                     seq);
  return hipGetLastError();
}

hipError_t launch_plan_k2q_materialize(const PlanGeo& g, const PlanDev& d, const PlanWork& w,
                                       const K2QWork& kw, const K2QDev& kd, int32_t krows_total,
                                       hipStream_t s) {
  const int64_t upper = (int64_t)g.mask_heads * g.batch * g.nk_max;
  const int64_t items = krows_total >= 0 ? (int64_t)g.mask_heads * krows_total : upper;
  const int64_t rps_max = (g.seqlen_q + (int64_t)g.tile_q - 1) / g.tile_q;   // longest sample
  const int lds_list = rps_max <= 4096 ? 1 : 0;
  const size_t lds = lds_list ? (size_t)(rps_max > 0 ? rps_max : 1) * 8 : 0;
  hipLaunchKernelGGL(plan_k2q_materialize_kernel, dim3((unsigned)(items > 0 ? items : 1)),
                     dim3(256), lds, s, g, d, w, kw, kd, krows_total, lds_list);
  return hipGetLastError();
}

}  // namespace mpb
