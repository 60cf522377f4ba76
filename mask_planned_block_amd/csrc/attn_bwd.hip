// Block-sparse flex attention backward for gfx950 (MI355X).
//
// Gradients of FlexAttention's Eq. 1 (O = softmax(mod(Q K^T * scale)) V)
// for an incoming dO, consuming the plan as "Flex Attention Mask Plan
// Design" §6.3 prescribes: the Q-major dQ kernel walks the Q2K view and the
// K-major dK/dV kernel walks the K2Q view; partial entries apply their packed
// predicate, full entries none; empty pairs are never touched.  Softmax
// weights are recomputed from the forward's LSE (FlexAttention: the backward
// recomputes the forward softmax from saved statistics), and the score_mod
// contributes its derivative (softcap: 1 - tanh^2 of its argument; ALiBi: 1).
//
// With x = scale * q.k, t = mod(x), P = exp(t - LSE) and Dq = dO . O:
//   dP = dO . V,  dS = P (dP - Dq) dt/dx,
//   dQ = scale * sum_k dS K,  dK = scale * sum_q dS Q,  dV = sum_q P dO.
//
// Three launches:
//  * attn_bwd_dot_kernel: -Dq per (row, head), fp32 [Hq][total_q].
//  * attn_bwd_dq_kernel: one workgroup per task of the plan's launch order
//    (as the forward), a wavefront per 32 Q rows.  S^T = K Q^T and
//    dP^T = V dO^T put one Q row in each lane (its LSE and Dq are scalars),
//    dS^T feeds dQ^T += K^T dS^T from registers; K^T is read from the
//    row-major K tile with ds_read_b64_tr_b16.  K and V are double buffered
//    in LDS and fetched one tile ahead straight from HBM.
//  * attn_bwd_dkdv_kernel: one workgroup per (KV head, K plan row), a
//    wavefront per 32 K rows, looping over the heads of the KV group and the
//    Q tiles that the K2Q view lists for the K row.  S = Q K^T and
//    dP = dO V^T put one K row in each lane, with K and V held in registers
//    for the whole workgroup; P and dS feed dV^T += dO^T P and dK^T += Q^T dS
//    from registers, dO^T and Q^T read transposed from the Q/dO tiles in LDS.
//    dK and dV of the K row are summed over the group in registers, so no
//    atomics and a deterministic result.
// All products on v_mfma_f32_32x32x16_bf16 (P and dS rounded to bf16),
// statistics and accumulators in fp32; outputs in bf16.
#include <type_traits>

#include "mpb_internal.h"
#include "../../include/mpb.h"

namespace mpb {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void* lds_vptr;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPosInf = __builtin_huge_valf();

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ inline u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// MFMA 32x32x16 bf16 operand layouts used below (D = A B, 32x32 outputs):
//   A: lane l holds A[l % 32][8 (l / 32) + i], i = 0..7
//   B: lane l holds B[8 (l / 32) + i][l % 32]
//   D: lane l holds D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32], v = 0..15
// A tile in LDS is row-major with D bf16 per row, its 16-byte chunk c of row
// r stored at position c ^ swz(r).  Every tile here is read both ways: as
// rows (8 lanes reading one chunk of 8 consecutive rows) and transposed (16
// lanes reading two neighbouring chunks of 4 consecutive rows), and
// swz(r) = 2 ((r / rp) % (CH / 2)), rp = rows per 256 bytes, puts both
// groups on distinct banks (the forward's K-only swizzle serves one pattern).
template <int D>
__device__ constexpr int swz(int r) {
  constexpr int CH = D / 8, RP = 256 / (2 * D);
  return 2 * ((r / RP) % (CH / 2));
}

// 16 bytes of row `row`, logical chunk `c`.
template <int D>
__device__ inline bf16x8 lds_chunk(const __bf16* tile, int row, int c) {
  return *(const bf16x8*)(tile + row * D + ((c ^ swz<D>(row)) << 3));
}

// A operand X^T (rows of the LDS tile X are the MFMA k index, its columns the
// m index) for the k-step over X rows [kb, kb + 16) and columns [32 db, +32):
// two ds_read_b64_tr_b16, each giving lane L the column 32 db + L % 32 of
// four consecutive rows, in the k-slot order of the D layout above (slots
// 0..3: rows kb + 4 (L / 32) + j, slots 4..7: the same + 8).
template <int D>
__device__ inline bf16x8 lds_tr_frag(const __bf16* tile, int kb, int db, int lane) {
  const int r = lane & 15, g2 = (lane >> 4) & 1, kg = lane >> 5;
  const int row = kb + 4 * kg + (r >> 2);
  const int dcol = 32 * db + 16 * g2 + 4 * (r & 3);
  const int c = dcol >> 3, e = dcol & 7;
  const __bf16* p0 = tile + row * D + (((c ^ swz<D>(row)) << 3) + e);
  const __bf16* p1 = tile + (row + 8) * D + (((c ^ swz<D>(row + 8)) << 3) + e);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p0);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p1);
  const v4i16 both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, both);
}

// Rows [0, R) of a row-major bf16 tile at byte tile_off of `src` (rs bytes
// per row) straight into LDS `dst` with the chunk swizzle above; NWAVES
// wavefronts share the rows.  Rows past the resource's range land as zeros.
template <int D, int R, int NWAVES>
__device__ inline void dma_tile(__bf16* dst, rsrc_t src, uint32_t tile_off, uint32_t rs,
                                int wave, int lane) {
  constexpr int CH = D / 8, RPI = 1024 / (D * 2);
  static_assert(R % (RPI * NWAVES) == 0, "tile rows must split evenly over wavefronts");
#pragma unroll
  for (int c = 0; c < R / RPI / NWAVES; ++c) {
    const int r0 = (c * NWAVES + wave) * RPI;
    const int r = r0 + lane / CH;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src, (lds_vptr)&dst[r0 * D], 16, (int)(tile_off + r * rs + ((lane % CH) ^ swz<D>(r)) * 16),
        0, 0, 0);
  }
}

// B operand fragments of one token row (d = 16 s + 8 (lane / 32) + i).
template <int D>
__device__ inline void load_row_frags(bf16x8 (&f)[D / 16], rsrc_t r, uint32_t row_off, int g) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    f[s] = __builtin_bit_cast(bf16x8, bload16(r, row_off + (16 * s + 8 * g) * 2));
}

// Stores a D^T accumulator set (lane: one token row, d = 32 db + 8 a + 4 g + c)
// times `mul` as bf16; stores past the resource's range are dropped.
template <int D>
__device__ inline void store_rows(rsrc_t r, uint32_t row_off, const f32x16 (&acc)[D / 32],
                                  float mul, int g) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 v;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = (__bf16)(acc[db][4 * a + c] * mul);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r,
                                            (int)(row_off + (db * 32 + 8 * a + 4 * g) * 2), 0, 0);
    }
}

// score_mod of a raw dot product s in log2 units, log2(e) * mod(s * scale),
// and its derivative with respect to x = s * scale.  kq = k - q.
// softcap: c tanh(u / c) = c (1 - 2 r) with r = 1 / (1 + e^{2u/c}), whose
// derivative 1 - tanh^2 is 4 r (1 - r).
template <int MOD>
__device__ inline float mod_fwd_bwd(float s, float kq, const BwdParams& p, float slope,
                                    float& grad) {
  if constexpr (MOD == kModNone) {
    grad = 1.0f;
    return s * p.scale_log2;
  } else if constexpr (MOD == kModAlibi) {
    grad = 1.0f;
    return fmaf(s, p.scale_log2, slope * kq);          // slope = slope_h * log2e
  } else if constexpr (MOD == kModSoftcap || MOD == kModSoftcapAlibi) {
    const float r = rcp_fast(1.0f + exp2_fast(s * p.softcap_k));
    grad = 4.0f * r * (1.0f - r);
    float u = fmaf(-2.0f * p.softcap_c2, r, p.softcap_c2);
    if constexpr (MOD == kModSoftcapAlibi) u = fmaf(slope, kq, u);
    return u;
  } else {   // kModAlibiSoftcap: slope = slope_h * 2 log2e / c
    const float r = rcp_fast(1.0f + exp2_fast(fmaf(s, p.softcap_k, slope * kq)));
    grad = 4.0f * r * (1.0f - r);
    return fmaf(-2.0f * p.softcap_c2, r, p.softcap_c2);
  }
}

template <int MOD>
__device__ inline float head_slope(const BwdParams& p, int h) {
  if constexpr (MOD == kModAlibi || MOD == kModSoftcapAlibi) return p.slopes[h] * kLog2e;
  else if constexpr (MOD == kModAlibiSoftcap) return p.slopes[h] * p.alibi_k;
  else return 0.0f;
}

// LSE in log2 units for the exponent; +inf for a row with nothing visible
// (its weights are then exactly 0) and for rows past the sample.
__device__ inline float lse_log2(float lse) { return lse == -kPosInf ? kPosInf : lse * kLog2e; }

// A weight exp2(t - lse2) with t - lse2 below -200 is exactly 0 in fp32 (the
// smallest denormal is 2^-149), and so is its dS.  With the softcap applied
// before ALiBi, t <= c2 + slope * (k - q) (c2 = the cap in log2 units), so a
// block whose every element has that bound 200 below its row's LSE adds
// nothing to dQ, dK or dV and is skipped before its scores.
constexpr float kNegligibleLog2 = 200.0f;

// Upper bound of t over the K - Q offsets [k_lo, k_lo + 27] a lane holds in
// one 32 x 32 block; fmaf rounds the bound the way t itself is rounded, and
// monotonically, so t never exceeds it.
__device__ inline float softcap_alibi_bound(float c2, float slope, float k_lo) {
  return fmaxf(fmaf(slope, k_lo, c2), fmaf(slope, k_lo + 27.0f, c2));
}

// Weight and dS of one score element; lse2 is the row's LSE in log2 units
// (+inf for a row that sees nothing), ndq is -Dq of the row.  Full tiles
// (MASKED = false) keep every element.
template <int MOD, bool MASKED>
__device__ inline void weight_and_ds(float s, float dp, float kq, uint32_t mw, int pos,
                                     float lse2, float ndq, const BwdParams& p, float slope,
                                     float& P, float& dS) {
  float grad;
  const float t = mod_fwd_bwd<MOD>(s, kq, p, slope, grad);
  P = exp2_fast(t - lse2);
  if constexpr (MASKED) P = ((mw >> pos) & 1u) ? P : 0.0f;
  dS = P * (dp + ndq) * grad;
}

}  // namespace

// ------------------------------------------------------------------ Dq

// -Dq[h][t] = -(dO[t][h] . O[t][h]) in fp32, and the row's LSE in log2 units
// (+inf for a row that sees nothing, whose weights are then exactly 0);
// D / 8 lanes per (token, head) row.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dot_kernel(BwdParams p) {
  constexpr int L = D / 8;
  const int64_t rows = (int64_t)p.total_q * p.heads_q;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / L;
  const int part = (int)(gid % L);
  float s = 0.0f;
  if (row < rows) {
    const bf16x8 a = *(const bf16x8*)((const __bf16*)p.o + row * D + part * 8);
    const bf16x8 b = *(const bf16x8*)((const __bf16*)p.dout + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf((float)a[i], (float)b[i], s);
  }
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && part == 0) {
    const int64_t t = row / p.heads_q;
    const int h = (int)(row % p.heads_q);
    const int64_t x = (int64_t)h * p.total_q + t;
    p.dvec[x] = -s;
    p.lse2[x] = lse_log2(p.lse[x]);
  }
}

// ------------------------------------------------------------------ dQ

// Stage index of a double buffer: an int, or a compile-time constant where
// the loop is unrolled by two.  With one LDS array per stage and compile-time
// stages, the compiler sees that the loads landing in the next stage cannot
// alias this stage's reads and does not wait for them.
using S0 = std::integral_constant<int, 0>;
using S1 = std::integral_constant<int, 1>;
template <class St>
__device__ constexpr auto flip(St) {
  return std::integral_constant<int, St::value ^ 1>{};
}

template <int D, int TQ, int TKV, int MOD>
__global__ __launch_bounds__(TQ * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(BwdParams p) {
  constexpr int NW = TQ / 32, NKB = TKV / 32, DS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 k_s0[TKV * D];
  __shared__ __attribute__((aligned(16))) __bf16 k_s1[TKV * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_s0[TKV * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_s1[TKV * D];
  auto kbuf = [&](auto st) -> __bf16* {
    if constexpr (decltype(st)::value == 0) return k_s0; else return k_s1;
  };
  auto vbuf = [&](auto st) -> __bf16* {
    if constexpr (decltype(st)::value == 0) return v_s0; else return v_s1;
  };
  __shared__ float s_min[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lq = lane & 31;

  const int32_t* rec = p.task_rec + (int64_t)blockIdx.x * kTaskRecInts;
  const int m_block = __builtin_amdgcn_readfirstlane(rec[kRecMBlock]);
  const int h = __builtin_amdgcn_readfirstlane(rec[kRecHead]);
  const int q_off = __builtin_amdgcn_readfirstlane(rec[kRecQOff]);
  const int k_off = __builtin_amdgcn_readfirstlane(rec[kRecKOff]);
  const int q_len = __builtin_amdgcn_readfirstlane(rec[kRecQLen]);
  const int k_len = __builtin_amdgcn_readfirstlane(rec[kRecKLen]);
  int p_beg = __builtin_amdgcn_readfirstlane(rec[kRecPBeg]);
  int np = __builtin_amdgcn_readfirstlane(rec[kRecPCnt]);
  int f_beg = __builtin_amdgcn_readfirstlane(rec[kRecFBeg]);
  int nf = __builtin_amdgcn_readfirstlane(rec[kRecFCnt]);
  const int kvh = __builtin_amdgcn_readfirstlane(rec[kRecKvHead]);
  const int qloc = m_block * TQ + 32 * wave + lq;   // this lane's sample-local Q row
  const bool row_in = qloc < q_len;
  const int64_t stat = (int64_t)h * p.total_q + q_off + qloc;
  const float lse2 = row_in ? p.lse2[stat] : kPosInf;
  if (MOD == kModSoftcapAlibi && !p.no_skip) {
    // The tile's least LSE; the K tiles whose every weight in this tile is
    // negligible (softcap_alibi_bound below the least LSE by 200) are cut
    // from the ends of both ascending lists before anything is loaded.  With
    // slope >= 0 the bound grows with the K tile, so such tiles lead the
    // lists (trail them for slope < 0); only whole leading and trailing runs
    // are cut.
    float v = lse2;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off));
    if (lane == 0) s_min[wave] = v;
    __syncthreads();
    float tm = s_min[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) tm = fminf(tm, s_min[w]);
    const float slope = head_slope<MOD>(p, h);
    const float thr = tm - kNegligibleLog2;
    const int q0 = m_block * TQ;
    auto negligible = [&](int j) {
      const float lo = (float)(j * TKV - (q0 + TQ - 1)), hi = (float)(j * TKV + TKV - 1 - q0);
      return fmaxf(fmaf(slope, lo, p.softcap_c2), fmaf(slope, hi, p.softcap_c2)) < thr;
    };
    auto trim = [&](const int32_t* idx, int& beg, int& cnt) {
      for (int front = 1; front >= 0; --front)
        while (cnt > 0) {
          bool f = false;
          if (lane < cnt) f = negligible(idx[front ? beg + lane : beg + cnt - 1 - lane]);
          const uint64_t m = __builtin_amdgcn_ballot_w64(f);
          const int run = ~m == 0 ? 64 : __builtin_ctzll(~m);
          if (front) beg += run;
          cnt -= run;
          if (run < 64) break;
        }
      beg = __builtin_amdgcn_readfirstlane(beg);
      cnt = __builtin_amdgcn_readfirstlane(cnt);
    };
    trim(p.p_idx, p_beg, np);
    trim(p.f_idx, f_beg, nf);
  }
  const int ntiles = np + nf;

  const uint32_t q_rs = (uint32_t)p.heads_q * D * 2;
  const uint32_t kv_rs = (uint32_t)p.heads_k * D * 2;
  const int64_t qh = (int64_t)q_off * q_rs + (int64_t)h * D * 2;
  const int64_t kh = (int64_t)k_off * kv_rs + (int64_t)kvh * D * 2;
  const rsrc_t rq = make_rsrc((const char*)p.q + qh, (uint32_t)q_len * q_rs);
  const rsrc_t rdo = make_rsrc((const char*)p.dout + qh, (uint32_t)q_len * q_rs);
  const rsrc_t rdq = make_rsrc((char*)p.dq + qh, (uint32_t)q_len * q_rs);
  const rsrc_t rk = make_rsrc((const char*)p.k + kh, (uint32_t)k_len * kv_rs);
  const rsrc_t rv = make_rsrc((const char*)p.v + kh, (uint32_t)k_len * kv_rs);

  const uint32_t q_row_off = (uint32_t)qloc * q_rs;
  // Tile t of the row: the partial list, then the full list; without ALiBi
  // the full list first, as in the forward (the tasks of a head begin on the
  // tiles they share)
  constexpr bool kFullFirst = MOD == kModNone || MOD == kModSoftcap;
  const int nfl = ntiles - np;
  auto is_partial = [&](int t) { return kFullFirst ? t >= nfl : t < np; };
  auto list_pos = [&](int t) {
    return kFullFirst ? (t < nfl ? f_beg + t : p_beg + t - nfl)
                      : (t < np ? p_beg + t : f_beg + t - np);
  };
  auto tile_raw = [&](int t) { return is_partial(t) ? p.p_idx[list_pos(t)] : p.f_idx[list_pos(t)]; };
  auto tile_j = [&](int t) {
    return __builtin_amdgcn_readfirstlane(tile_raw(t));
  };
  auto load_masks = [&](int t, uint32_t (&mw)[NKB]) {
    if (is_partial(t)) {
      const uint32_t* src = p.p_masks + ((int64_t)list_pos(t) * TQ + 32 * wave + lq) * NKB;
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) mw[kk] = src[kk];
    } else {
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) mw[kk] = 0xFFFFFFFFu;
    }
  };
  auto load_kv = [&](int j, __bf16* kd, __bf16* vd) {
    const uint32_t off = (uint32_t)j * TKV * kv_rs;
    dma_tile<D, TKV, NW>(kd, rk, off, kv_rs, wave, lane);
    dma_tile<D, TKV, NW>(vd, rv, off, kv_rs, wave, lane);
  };

  int j_cur = 0, j_next = 0;
  uint32_t mw_cur[NKB], mw_next[NKB];
  if (ntiles > 0) {
    j_cur = tile_j(0);
    load_kv(j_cur, k_s0, v_s0);
    load_masks(0, mw_cur);
    if (ntiles > 1) j_next = tile_j(1);
  }
  bf16x8 qf[DS], df[DS];
  load_row_frags<D>(qf, rq, q_row_off, g);
  load_row_frags<D>(df, rdo, q_row_off, g);
  const float ndq = row_in ? p.dvec[stat] : 0.0f;   // -Dq
  const float slope = head_slope<MOD>(p, h);

  f32x16 acc_dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_dq[db] = f32x16{};

  int t = 0;
  // One K tile: per 32-row K block kk, S^T = K Q^T and dP^T = V dO^T on MFMA
  // (lane holds Q row lq, K rows 32kk+8(v/4)+4g+v%4), the weights and dS^T
  // on the VALU, then dQ^T += K^T dS^T (K^T read transposed from LDS).
  auto step = [&](auto masked, auto stage) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
    const auto nx = flip(stage);
    const __bf16* ks = kbuf(stage);
    const __bf16* vs = vbuf(stage);
    const bool more = t + 1 < ntiles;
    // the K tile after next, read before the next tile's fill so that
    // waiting for it (after this tile's products) does not wait for the fill
    int j2 = 0;
    if (t + 2 < ntiles) j2 = tile_raw(t + 2);
    if (more) {
      load_kv(j_next, kbuf(nx), vbuf(nx));
      load_masks(t + 1, mw_next);
    }
    const float kq0 = (float)(j_cur * TKV + 4 * g - qloc);
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      // a 32-row K block that the predicate hides from all of this
      // wavefront's Q rows contributes nothing (every weight is exactly 0)
      if constexpr (kMasked)
        if (!p.no_skip && __builtin_amdgcn_ballot_w64(mw_cur[kk] != 0) == 0) continue;
      // ... and so does one whose weights are all negligible
      if constexpr (MOD == kModSoftcapAlibi) {
        const float bound = softcap_alibi_bound(p.softcap_c2, slope, kq0 + (float)(32 * kk));
        if (!p.no_skip && __builtin_amdgcn_ballot_w64(!(bound < lse2 - kNegligibleLog2)) == 0)
          continue;
      }
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
      // operand rows read from LDS one k-step ahead of the MFMAs using them
      bf16x8 ak[2], av[2];
      ak[0] = lds_chunk<D>(ks, 32 * kk + lq, g);
      av[0] = lds_chunk<D>(vs, 32 * kk + lq, g);
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const int c = s & 1;
        if (s + 1 < DS) {
          ak[c ^ 1] = lds_chunk<D>(ks, 32 * kk + lq, 2 * (s + 1) + g);
          av[c ^ 1] = lds_chunk<D>(vs, 32 * kk + lq, 2 * (s + 1) + g);
        }
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[c], qf[s], s_acc, 0, 0, 0);
        dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[c], df[s], dp_acc, 0, 0, 0);
      }
      const uint32_t mw = mw_cur[kk] >> (4 * g);
      // per-lane part of the exponent (element offsets pos are added per
      // element); softcap derivatives as r (1 - r), the factor 4 in dQ's scale
      const float kqb = kq0 + (float)(32 * kk);
      float base;
      if constexpr (MOD == kModAlibi || MOD == kModAlibiSoftcap) base = slope * kqb;
      else if constexpr (MOD == kModSoftcapAlibi) base = fmaf(slope, kqb, p.softcap_c2);
      else if constexpr (MOD == kModSoftcap) base = p.softcap_c2;
      else base = 0.0f;
      bf16x8 dsb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int pos = 8 * (v / 4) + v % 4;
        const float s = s_acc[v];
        float tt, grad = 1.0f;
        if constexpr (MOD == kModNone) {
          tt = fmaf(s, p.scale_log2, -lse2);
        } else if constexpr (MOD == kModAlibi) {
          tt = fmaf(s, p.scale_log2, fmaf(slope, (float)pos, base)) - lse2;
        } else if constexpr (MOD == kModAlibiSoftcap) {
          const float r =
              rcp_fast(1.0f + exp2_fast(fmaf(s, p.softcap_k, fmaf(slope, (float)pos, base))));
          grad = fmaf(-r, r, r);
          tt = fmaf(-2.0f * p.softcap_c2, r, p.softcap_c2) - lse2;
        } else {   // softcap, then ALiBi for kModSoftcapAlibi (in base)
          const float r = rcp_fast(1.0f + exp2_fast(s * p.softcap_k));
          grad = fmaf(-r, r, r);
          float u = fmaf(-2.0f * p.softcap_c2, r, base);
          if constexpr (MOD == kModSoftcapAlibi) u = fmaf(slope, (float)pos, u);
          tt = u - lse2;
        }
        float P = exp2_fast(tt);
        if constexpr (kMasked) {
          int keep;   // the predicate bit sign-extended to an all-ones or all-zeros mask
          asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(keep) : "v"(mw), "i"(pos));
          P = __int_as_float(__float_as_int(P) & keep);
        }
        float dS = P * (dp_acc[v] + ndq);
        if constexpr (MOD != kModNone && MOD != kModAlibi) dS *= grad;
        dsb[v / 8][v % 8] = (__bf16)dS;
      }
      // dQ^T += K^T dS^T, transposed operands read one step ahead
      bf16x8 fk[2];
      fk[0] = lds_tr_frag<D>(ks, 32 * kk, 0, lane);
#pragma unroll
      for (int x = 0; x < 2 * DB; ++x) {
        const int c = x & 1, db = x % DB, m = x / DB;
        if (x + 1 < 2 * DB)
          fk[c ^ 1] = lds_tr_frag<D>(ks, 32 * kk + 16 * ((x + 1) / DB), (x + 1) % DB, lane);
        acc_dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[c], dsb[m], acc_dq[db], 0, 0, 0);
      }
    }
    asm volatile("" : "+v"(j2));   // used from here on only
    if (more) {
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) mw_cur[kk] = mw_next[kk];
      j_cur = j_next;
      j_next = __builtin_amdgcn_readfirstlane(j2);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wavefront's loads of the next tile have landed
    __syncthreads();                 // ... and everyone's; this tile's reads are done
    ++t;
  };
  // partial tiles with their predicate, then full tiles without (§6.3)
  auto run = [&](auto masked, int t_end) __attribute__((always_inline)) {
    if (t < t_end && (t & 1)) step(masked, S1{});
    while (t + 1 < t_end) {
      step(masked, S0{});
      step(masked, S1{});
    }
    if (t < t_end) step(masked, S0{});
  };
  if (ntiles > 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (kFullFirst) {
      run(std::false_type{}, nfl);
      run(std::true_type{}, ntiles);
    } else {
      run(std::true_type{}, np);
      run(std::false_type{}, ntiles);
    }
  }
  constexpr bool kSoftcap =
      MOD == kModSoftcap || MOD == kModSoftcapAlibi || MOD == kModAlibiSoftcap;
  store_rows<D>(rdq, q_row_off, acc_dq, kSoftcap ? 4.0f * p.scale : p.scale, g);
}

// ------------------------------------------------------------------ dK, dV

// One workgroup per (KV head, K plan row): wavefront w takes K block
// w % NKW (32 K rows) and Q half w / NKW of every Q tile, so dK and dV of a K
// block are summed by two wavefronts and added through LDS at the end.  The
// Q tiles of all heads of the group (partial list, then full list, per head)
// stream through a double buffer: item n + 1 (Q, dO, LSE and Dq rows) is
// fetched straight into LDS while item n is computed.
template <int D, int TQ, int TKV, int MOD>
__global__ __launch_bounds__(TKV * 4) void attn_bwd_dkdv_kernel(BwdParams p) {
  constexpr int NKW = TKV / 32, NW = 2 * NKW, NQB = TQ / 32, QBW = NQB / 2;
  constexpr int DS = D / 16, DB = D / 32;
  static_assert(NQB % 2 == 0, "Q tile must split into two halves of whole 32-row blocks");
  __shared__ __attribute__((aligned(16))) __bf16 q_s0[TQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 q_s1[TQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 do_s0[TQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 do_s1[TQ * D];
  __shared__ __attribute__((aligned(16))) float lse_s0[TQ];
  __shared__ __attribute__((aligned(16))) float lse_s1[TQ];
  __shared__ __attribute__((aligned(16))) float dd_s0[TQ];
  __shared__ __attribute__((aligned(16))) float dd_s1[TQ];
  auto qbuf = [&](auto st) -> __bf16* {
    if constexpr (decltype(st)::value == 0) return q_s0; else return q_s1;
  };
  auto dobuf = [&](auto st) -> __bf16* {
    if constexpr (decltype(st)::value == 0) return do_s0; else return do_s1;
  };
  auto lsebuf = [&](auto st) -> float* {
    if constexpr (decltype(st)::value == 0) return lse_s0; else return lse_s1;
  };
  auto ddbuf = [&](auto st) -> float* {
    if constexpr (decltype(st)::value == 0) return dd_s0; else return dd_s1;
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lq = lane & 31;
  const int kb = wave % NKW, qh = wave / NKW;

  // K rows in the plan's launch order (heaviest first), all KV heads of a
  // K row next to each other
  const int kvh = blockIdx.x % p.heads_k;
  const int kr = __builtin_amdgcn_readfirstlane(p.k_order[blockIdx.x / p.heads_k]);
  // sample of the K row (largest b with cu_krows[b] <= kr)
  int lo = 0, hi = p.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.k_cu[mid] <= kr) lo = mid; else hi = mid - 1;
  }
  const int b = __builtin_amdgcn_readfirstlane(lo);
  const int j = kr - p.k_cu[b];
  const int32_t* sd = p.seqdesc + 8 * b;
  const int q_off = __builtin_amdgcn_readfirstlane(sd[0]);
  const int k_off = __builtin_amdgcn_readfirstlane(sd[1]);
  const int q_len = __builtin_amdgcn_readfirstlane(sd[2]);
  const int k_len = __builtin_amdgcn_readfirstlane(sd[3]);

  const uint32_t q_rs = (uint32_t)p.heads_q * D * 2;
  const uint32_t kv_rs = (uint32_t)p.heads_k * D * 2;
  const int64_t kh = (int64_t)k_off * kv_rs + (int64_t)kvh * D * 2;
  const rsrc_t rk = make_rsrc((const char*)p.k + kh, (uint32_t)k_len * kv_rs);
  const rsrc_t rv = make_rsrc((const char*)p.v + kh, (uint32_t)k_len * kv_rs);
  const rsrc_t rdk = make_rsrc((char*)p.dk + kh, (uint32_t)k_len * kv_rs);
  const rsrc_t rdv = make_rsrc((char*)p.dv + kh, (uint32_t)k_len * kv_rs);

  // Items: (head of the group, Q tile) pairs, per head its partial list then
  // its full list.  pair >= 0 is the partial pair's payload index.
  struct Item { int h, i, pair; };
  auto lists = [&](int hh, int& pb, int& np, int& fb, int& nf) {
    const int h = kvh * p.group + hh;
    const int64_t flat = (int64_t)(p.mask_heads == 1 ? 0 : h) * p.krows_total + kr;
    pb = __builtin_amdgcn_readfirstlane(p.k_p_off[flat]);
    np = __builtin_amdgcn_readfirstlane(p.k_p_off[flat + 1]) - pb;
    fb = __builtin_amdgcn_readfirstlane(p.k_f_off[flat]);
    nf = __builtin_amdgcn_readfirstlane(p.k_f_off[flat + 1]) - fb;
  };
  int n_items = 0;
  for (int hh = 0; hh < p.group; ++hh) {
    int pb, np, fb, nf;
    lists(hh, pb, np, fb, nf);
    n_items += np + nf;
  }
  auto item_at = [&](int n) -> Item {
    for (int hh = 0; hh < p.group; ++hh) {
      int pb, np, fb, nf;
      lists(hh, pb, np, fb, nf);
      const int h = kvh * p.group + hh;
      if (n < np) return Item{h, __builtin_amdgcn_readfirstlane(p.k_p_idx[pb + n]), pb + n};
      n -= np;
      if (n < nf) return Item{h, __builtin_amdgcn_readfirstlane(p.k_f_idx[fb + n]), -1};
      n -= nf;
    }
    return Item{0, 0, -1};
  };

  // Q, dO, LSE and Dq rows of an item into one stage (rows past q_len land as
  // zeros and are never kept: their predicate bits are 0 and tail Q tiles
  // are never full).
  auto load_item = [&](const Item& it, __bf16* qd, __bf16* dod, float* ld, float* dd) {
    const int64_t qh64 = (int64_t)q_off * q_rs + (int64_t)it.h * D * 2;
    const rsrc_t rq = make_rsrc((const char*)p.q + qh64, (uint32_t)q_len * q_rs);
    const rsrc_t rdo = make_rsrc((const char*)p.dout + qh64, (uint32_t)q_len * q_rs);
    const uint32_t off = (uint32_t)it.i * TQ * q_rs;
    dma_tile<D, TQ, NW>(qd, rq, off, q_rs, wave, lane);
    dma_tile<D, TQ, NW>(dod, rdo, off, q_rs, wave, lane);
    const int64_t st = (int64_t)it.h * p.total_q + q_off;
    if (wave < TQ / 64) {
      const rsrc_t rl = make_rsrc(p.lse2 + st, (uint32_t)q_len * 4);
      const rsrc_t rd = make_rsrc(p.dvec + st, (uint32_t)q_len * 4);
      const int q = it.i * TQ + 64 * wave + lane;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_vptr)&ld[64 * wave], 4, q * 4, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_vptr)&dd[64 * wave], 4, q * 4, 0, 0, 0);
    }
  };
  auto load_masks = [&](const Item& it, uint32_t (&mw)[QBW]) {
    if (it.pair >= 0) {
      const uint32_t* src =
          p.k_masks + ((int64_t)it.pair * TKV + 32 * kb + lq) * NQB + qh * QBW;
#pragma unroll
      for (int w = 0; w < QBW; ++w) mw[w] = src[w];
    } else {
#pragma unroll
      for (int w = 0; w < QBW; ++w) mw[w] = 0xFFFFFFFFu;
    }
  };

  const int kloc = j * TKV + 32 * kb + lq;   // this lane's sample-local K row
  const uint32_t k_row_off = (uint32_t)kloc * kv_rs;
  Item cur = Item{0, 0, -1}, nxt = Item{0, 0, -1};
  uint32_t mw_cur[QBW], mw_next[QBW];
  if (n_items > 0) {
    cur = item_at(0);
    load_item(cur, q_s0, do_s0, lse_s0, dd_s0);
    load_masks(cur, mw_cur);
    if (n_items > 1) nxt = item_at(1);
  }
  bf16x8 kf[DS], vf[DS];
  load_row_frags<D>(kf, rk, k_row_off, g);
  load_row_frags<D>(vf, rv, k_row_off, g);

  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_dk[db] = acc_dv[db] = f32x16{};

  int n = 0;
  auto step = [&](auto stage) __attribute__((always_inline)) {
    const auto nx = flip(stage);
    const __bf16* qs = qbuf(stage);
    const __bf16* dos = dobuf(stage);
    const float* ls = lsebuf(stage);
    const float* ds = ddbuf(stage);
    const bool more = n + 1 < n_items;
    if (more) {
      load_item(nxt, qbuf(nx), dobuf(nx), lsebuf(nx), ddbuf(nx));
      load_masks(nxt, mw_next);
    }
    const float slope = head_slope<MOD>(p, cur.h);
    const float kq0 = (float)(kloc - cur.i * TQ - 4 * g);
    // Phases per 32-row Q block qb: S = Q K^T and dP = dO V^T on MFMA (lane
    // holds K row lq, Q rows 32qb+8(v/4)+4g+v%4), the weights and dS on the
    // VALU, then dV^T += dO^T P and dK^T += Q^T dS on MFMA.  With two blocks
    // per wavefront they are issued as S(0) S(1) W(0) V(0) W(1) V(1): the
    // VALU work of one block sits between MFMAs of the other.
    f32x16 s_acc[QBW], dp_acc[QBW];
    bf16x8 pb8[QBW][2], dsb[QBW][2];
    auto scores = [&](int w) __attribute__((always_inline)) {
      const int qb = qh * QBW + w;
      s_acc[w] = f32x16{};
      dp_acc[w] = f32x16{};
      // operand rows read from LDS one k-step ahead of the MFMAs using them
      bf16x8 aq[2], ad[2];
      aq[0] = lds_chunk<D>(qs, 32 * qb + lq, g);
      ad[0] = lds_chunk<D>(dos, 32 * qb + lq, g);
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const int c = s & 1;
        if (s + 1 < DS) {
          aq[c ^ 1] = lds_chunk<D>(qs, 32 * qb + lq, 2 * (s + 1) + g);
          ad[c ^ 1] = lds_chunk<D>(dos, 32 * qb + lq, 2 * (s + 1) + g);
        }
        s_acc[w] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[c], kf[s], s_acc[w], 0, 0, 0);
        dp_acc[w] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad[c], vf[s], dp_acc[w], 0, 0, 0);
      }
    };
    auto weights = [&](int w, auto masked) __attribute__((always_inline)) {
      constexpr bool kMasked = decltype(masked)::value;
      const int qb = qh * QBW + w;
      const uint32_t mw = mw_cur[w] >> (4 * g);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        // rows 32qb + 8a + 4g + 0..3 of the LSE and Dq vectors: one 16-byte read each
        const int q4 = 32 * qb + 8 * a + 4 * g;
        const float4 l4 = *(const float4*)&ls[q4];
        const float4 d4 = *(const float4*)&ds[q4];
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int v = 4 * a + c, pos = 8 * a + c;
          float P, dS;
          weight_and_ds<MOD, kMasked>(s_acc[w][v], dp_acc[w][v], kq0 - (float)(32 * qb + pos), mw,
                                      pos, lv[c], dv[c], p, slope, P, dS);
          pb8[w][v / 8][v % 8] = (__bf16)P;
          dsb[w][v / 8][v % 8] = (__bf16)dS;
        }
      }
    };
    auto grads = [&](int w) __attribute__((always_inline)) {
      const int qb = qh * QBW + w;
      // transposed operands read one step ahead; consecutive MFMAs update
      // different accumulators
      constexpr int NS = 2 * DB;
      bf16x8 fd[2], fq[2];
      fd[0] = lds_tr_frag<D>(dos, 32 * qb, 0, lane);
      fq[0] = lds_tr_frag<D>(qs, 32 * qb, 0, lane);
#pragma unroll
      for (int x = 0; x < NS; ++x) {
        const int c = x & 1, m = x / DB, db = x % DB;
        if (x + 1 < NS) {
          const int m1 = (x + 1) / DB, db1 = (x + 1) % DB;
          fd[c ^ 1] = lds_tr_frag<D>(dos, 32 * qb + 16 * m1, db1, lane);
          fq[c ^ 1] = lds_tr_frag<D>(qs, 32 * qb + 16 * m1, db1, lane);
        }
        acc_dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fd[c], pb8[w][m], acc_dv[db], 0, 0, 0);
        acc_dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[c], dsb[w][m], acc_dk[db], 0, 0, 0);
      }
    };
    auto item = [&](auto masked) __attribute__((always_inline)) {
      // a pair whose predicate hides the wavefront's Q half from all of its
      // K rows contributes nothing (every weight is exactly 0)
      uint32_t any_bit = 0;
#pragma unroll
      for (int w = 0; w < QBW; ++w) any_bit |= mw_cur[w];
      if (!p.no_skip && __builtin_amdgcn_ballot_w64(any_bit != 0) == 0) return;
      // ... and so does one whose weights are all negligible: the bound over
      // the lane's 16 elements of each block against its 16 rows' least LSE
      if constexpr (MOD == kModSoftcapAlibi) {
        bool need = p.no_skip != 0;
#pragma unroll
        for (int w = 0; w < QBW; ++w) {
          const int qb = qh * QBW + w;
          float lmin = kPosInf;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float4 l4 = *(const float4*)&ls[32 * qb + 8 * a + 4 * g];
            lmin = fminf(lmin, fminf(fminf(l4.x, l4.y), fminf(l4.z, l4.w)));
          }
          const float bound =
              softcap_alibi_bound(p.softcap_c2, slope, kq0 - (float)(32 * qb + 27));
          need |= !(bound < lmin - kNegligibleLog2);
        }
        if (__builtin_amdgcn_ballot_w64(need) == 0) return;
      }
      if constexpr (QBW == 2) {
        scores(0);
        scores(1);
        weights(0, masked);
        grads(0);
        weights(1, masked);
        grads(1);
      } else {
#pragma unroll
        for (int w = 0; w < QBW; ++w) {
          scores(w);
          weights(w, masked);
          grads(w);
        }
      }
    };
    // (one code path: a full pair's predicate words are all ones; two paths
    // would not fit the register file together)
    item(std::true_type{});
    if (more) {
#pragma unroll
      for (int w = 0; w < QBW; ++w) mw_cur[w] = mw_next[w];
      cur = nxt;
      if (n + 2 < n_items) nxt = item_at(n + 2);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wavefront's loads of the next item have landed
    __syncthreads();                 // ... and everyone's; this item's reads are done
    ++n;
  };
  if (n_items > 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    while (n + 1 < n_items) {
      step(S0{});
      step(S1{});
    }
    if (n < n_items) step(S0{});
  }

  // The two Q halves of each K block: the upper half's wavefronts hand their
  // sums over through LDS (the Q buffers, free now), the lower half adds and
  // stores.
  // K block kb uses stage kb's Q buffer for dK and its dO buffer for dV.
  static_assert(NKW <= 2 && DB * 16 * 64 * 4 <= TQ * D * 2, "reduction buffer");
  float* red = reinterpret_cast<float*>(kb == 0 ? q_s0 : q_s1);
  float* red_v = reinterpret_cast<float*>(kb == 0 ? do_s0 : do_s1);
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        red[(db * 16 + v) * 64 + lane] = acc_dk[db][v];
        red_v[(db * 16 + v) * 64 + lane] = acc_dv[db][v];
      }
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc_dk[db][v] += red[(db * 16 + v) * 64 + lane];
        acc_dv[db][v] += red_v[(db * 16 + v) * 64 + lane];
      }
    store_rows<D>(rdk, k_row_off, acc_dk, p.scale, g);
    store_rows<D>(rdv, k_row_off, acc_dv, 1.0f, g);
  }
}

// Inclusive prefix sum over the wavefront's lanes.
__device__ inline int wave_prefix_sum(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Byte offsets inside a swizzled tile for the split kernel's fixed reads,
// each an XOR and an immediate away from a per-lane base: with swz even,
// chunk 2 s + g of row r sits at row_base(r, g) ^ 32 s, and the transposed
// fragment (rows 16 m + 8 p + the lane's row, columns 32 db + the lane's) at
// (tr_base ^ 64 db) + (16 m + 8 p) 2 D for rows that start a multiple of 8.
template <int D>
__device__ inline int row_base(int row, int g) {
  constexpr int CH = D / 8, RP = 256 / (2 * D);
  return row * 2 * D + 16 * g + 32 * ((row / RP) % (CH / 2));
}
template <int D>
__device__ inline int tr_base(int lane) {
  const int r = lane & 15, g2 = (lane >> 4) & 1, kg = lane >> 5;
  const int row = 4 * kg + (r >> 2);
  const int dcol = 16 * g2 + 4 * (r & 3);
  return row * 2 * D + (((dcol >> 3) ^ swz<D>(row)) << 4) + 2 * (dcol & 7);
}
__device__ inline bf16x8 lds_at(const __bf16* tile, int off) {
  return *(const bf16x8*)((const char*)tile + off);
}
// the A operand of lds_tr_frag from the byte offset of its first four rows
template <int D>
__device__ inline bf16x8 lds_tr_at(const __bf16* tile, int off) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const char* b = (const char*)tile + off;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)b);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(b + 8 * 2 * D));
  const v4i16 both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, both);
}

// dK and dV with one wavefront per 32 x 32 block of a (K plan row, Q tile)
// pair: for 128-row Q tiles and 64-row K tiles, eight wavefronts, two per
// SIMD, so one wavefront's weights (VALU) run beside the other's products
// (MFMA).  Wavefront w takes K block w % 2 and Q block w / 2 of every item;
// V stays in its registers (a lane per K row), K sits in LDS for the whole
// workgroup, and Q, dO, LSE and Dq stream through the double buffer of the
// kernel above.  The four wavefronts of a K block add their sums through LDS
// at the end (two rounds).  Softcap weights use r (1 - r) for the derivative
// 4 r (1 - r) and dK's scale takes the factor 4 (exact in bf16).
template <int D, int TQ, int TKV, int MOD>
__global__ __launch_bounds__(TQ * TKV / 16) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_split_kernel(BwdParams p) {
  constexpr int NKW = TKV / 32, NQB = TQ / 32, NW = NKW * NQB;
  constexpr int DS = D / 16, DB = D / 32;
  static_assert(NW == 8 && NQB == 4, "eight wavefronts: two K blocks by four Q blocks");
  __shared__ __attribute__((aligned(16))) __bf16 q_s0[TQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 q_s1[TQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 do_s0[TQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 do_s1[TQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 k_s[TKV * D];
  __shared__ __attribute__((aligned(16))) float lse_s0[TQ];
  __shared__ __attribute__((aligned(16))) float lse_s1[TQ];
  __shared__ __attribute__((aligned(16))) float dd_s0[TQ];
  __shared__ __attribute__((aligned(16))) float dd_s1[TQ];
  __shared__ int s_lists[5][64];   // per head of the group: partial begin, count, full begin, running total, full count
  auto qbuf = [&](auto st) -> __bf16* {
    if constexpr (decltype(st)::value == 0) return q_s0; else return q_s1;
  };
  auto dobuf = [&](auto st) -> __bf16* {
    if constexpr (decltype(st)::value == 0) return do_s0; else return do_s1;
  };
  auto lsebuf = [&](auto st) -> float* {
    if constexpr (decltype(st)::value == 0) return lse_s0; else return lse_s1;
  };
  auto ddbuf = [&](auto st) -> float* {
    if constexpr (decltype(st)::value == 0) return dd_s0; else return dd_s1;
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lq = lane & 31;
  const int kb = wave % NKW, qb = wave / NKW;
  constexpr bool kSoftcap =
      MOD == kModSoftcap || MOD == kModSoftcapAlibi || MOD == kModAlibiSoftcap;

  // KV head: workgroup i runs on XCD i % 8, so with Hk a multiple of 8 the
  // heads r, r + 8, r + 16, ... would share an XCD; dealing the heads out in
  // snake order (0..7, then 15..8, ...) mixes the steep and flat ALiBi slopes
  // (whose exact zero skips leave very different work) on every XCD
  int kvh = blockIdx.x % p.heads_k;
  if (p.heads_k % 8 == 0 && ((kvh >> 3) & 1)) kvh ^= 7;
  const int kr = __builtin_amdgcn_readfirstlane(p.k_order[blockIdx.x / p.heads_k]);
  // Everything the K row's setup reads is issued at once: the group's list
  // bounds (lane hh: head hh) and, for up to 64 samples, every sample's K
  // row start and descriptor (lane b: sample b), so the setup waits for one
  // round of reads instead of a chain of them.
  // (the reads land in plain registers, used only after all are issued)
  int p0 = 0, p1 = 0, f0 = 0, f1 = 0;
  if (lane < p.group) {
    const int64_t flat =
        (int64_t)(p.mask_heads == 1 ? 0 : kvh * p.group + lane) * p.krows_total + kr;
    p0 = p.k_p_off[flat];
    p1 = p.k_p_off[flat + 1];
    f0 = p.k_f_off[flat];
    f1 = p.k_f_off[flat + 1];
  }
  int cu = 0;
  int4 sdl = int4{0, 0, 0, 0};
  if (p.batch <= 64 && lane < p.batch) {
    cu = p.k_cu[lane];
    sdl = *(const int4*)(p.seqdesc + 8 * lane);   // 32-byte records, 256-byte aligned array
  }
  const int l_pb = p0, l_np = p1 - p0, l_fb = f0, l_nf = f1 - f0;
  int b, j, q_off, k_off, q_len, k_len;
  if (p.batch <= 64) {
    // the largest b with cu_krows[b] <= kr (the starts ascend)
    b = __popcll(__builtin_amdgcn_ballot_w64(lane < p.batch && cu <= kr)) - 1;
    j = kr - __builtin_amdgcn_readlane(cu, b);
    q_off = __builtin_amdgcn_readlane(sdl.x, b);
    k_off = __builtin_amdgcn_readlane(sdl.y, b);
    q_len = __builtin_amdgcn_readlane(sdl.z, b);
    k_len = __builtin_amdgcn_readlane(sdl.w, b);
  } else {
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.k_cu[mid] <= kr) lo = mid; else hi = mid - 1;
    }
    b = __builtin_amdgcn_readfirstlane(lo);
    j = kr - p.k_cu[b];
    const int32_t* sd = p.seqdesc + 8 * b;
    q_off = __builtin_amdgcn_readfirstlane(sd[0]);
    k_off = __builtin_amdgcn_readfirstlane(sd[1]);
    q_len = __builtin_amdgcn_readfirstlane(sd[2]);
    k_len = __builtin_amdgcn_readfirstlane(sd[3]);
  }

  const uint32_t q_rs = (uint32_t)p.heads_q * D * 2;
  const uint32_t kv_rs = (uint32_t)p.heads_k * D * 2;
  const int64_t kh = (int64_t)k_off * kv_rs + (int64_t)kvh * D * 2;
  const rsrc_t rk = make_rsrc((const char*)p.k + kh, (uint32_t)k_len * kv_rs);
  const rsrc_t rv = make_rsrc((const char*)p.v + kh, (uint32_t)k_len * kv_rs);
  const rsrc_t rdk = make_rsrc((char*)p.dk + kh, (uint32_t)k_len * kv_rs);
  const rsrc_t rdv = make_rsrc((char*)p.dv + kh, (uint32_t)k_len * kv_rs);

  // Items: (head of the group, Q tile) pairs, per head its partial list then
  // its full list (without ALiBi the full list first, as in the forward).
  // Lane hh < group holds head hh's list bounds and the running item count,
  // so locating item n needs no memory access; only its Q tile index is read
  // (pair >= 0: the partial pair's payload index).
  struct Item { int h, i, pair; };
  constexpr bool kFullFirst = MOD == kModNone || MOD == kModSoftcap;
  const int l_cum = wave_prefix_sum(l_np + l_nf, lane);
  const int n_items = __builtin_amdgcn_readlane(l_cum, 63);
  // head, list slot and payload index of item n (n < n_items), from the
  // lanes' registers (first items) or from their copy in LDS (the loop)
  auto locate = [&](int n, int& h, const int32_t*& src, int& pair) {
    const int hh = __popcll(__builtin_amdgcn_ballot_w64(lane < p.group && l_cum <= n));
    const int r = n - (hh ? __builtin_amdgcn_readlane(l_cum, hh - 1) : 0);
    const int np = __builtin_amdgcn_readlane(l_np, hh), nf = __builtin_amdgcn_readlane(l_nf, hh);
    h = kvh * p.group + hh;
    if (kFullFirst ? r >= nf : r < np) {
      pair = __builtin_amdgcn_readlane(l_pb, hh) + (kFullFirst ? r - nf : r);
      src = p.k_p_idx + pair;
    } else {
      pair = -1;
      src = p.k_f_idx + __builtin_amdgcn_readlane(l_fb, hh) + (kFullFirst ? r : r - np);
    }
  };
  auto locate_lds = [&](int n, int& h, const int32_t*& src, int& pair) {
    const int cum = lane < p.group ? s_lists[3][lane] : n + 1;
    const int hh = __popcll(__builtin_amdgcn_ballot_w64(cum <= n));
    const int r = n - (hh ? __builtin_amdgcn_readfirstlane(s_lists[3][hh - 1]) : 0);
    const int np = __builtin_amdgcn_readfirstlane(s_lists[1][hh]);
    const int nf = __builtin_amdgcn_readfirstlane(s_lists[4][hh]);
    h = kvh * p.group + hh;
    if (kFullFirst ? r >= nf : r < np) {
      pair = __builtin_amdgcn_readfirstlane(s_lists[0][hh]) + (kFullFirst ? r - nf : r);
      src = p.k_p_idx + pair;
    } else {
      pair = -1;
      src = p.k_f_idx + __builtin_amdgcn_readfirstlane(s_lists[2][hh]) + (kFullFirst ? r : r - np);
    }
  };
  if (wave == 0) {
    s_lists[0][lane] = l_pb;
    s_lists[1][lane] = l_np;
    s_lists[2][lane] = l_fb;
    s_lists[3][lane] = l_cum;
    s_lists[4][lane] = l_nf;
  }
  auto slope_of = [&](int h) -> float {
    if constexpr (MOD == kModAlibi || MOD == kModSoftcapAlibi || MOD == kModAlibiSoftcap)
      return p.slopes[h];
    else
      return 0.0f;
  };
  // the raw slope in the units the weights use
  auto slope_units = [&](float s) -> float {
    if constexpr (MOD == kModAlibi || MOD == kModSoftcapAlibi) return s * kLog2e;
    else if constexpr (MOD == kModAlibiSoftcap) return s * p.alibi_k;
    else return 0.0f;
  };
  auto load_item = [&](const Item& it, __bf16* qd, __bf16* dod, float* ld, float* dd) {
    const int64_t qh64 = (int64_t)q_off * q_rs + (int64_t)it.h * D * 2;
    const rsrc_t rq = make_rsrc((const char*)p.q + qh64, (uint32_t)q_len * q_rs);
    const rsrc_t rdo = make_rsrc((const char*)p.dout + qh64, (uint32_t)q_len * q_rs);
    const uint32_t off = (uint32_t)it.i * TQ * q_rs;
    dma_tile<D, TQ, NW>(qd, rq, off, q_rs, wave, lane);
    dma_tile<D, TQ, NW>(dod, rdo, off, q_rs, wave, lane);
    const int64_t st = (int64_t)it.h * p.total_q + q_off;
    if (wave < TQ / 64) {
      const rsrc_t rl = make_rsrc(p.lse2 + st, (uint32_t)q_len * 4);
      const rsrc_t rd = make_rsrc(p.dvec + st, (uint32_t)q_len * 4);
      const int q = it.i * TQ + 64 * wave + lane;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_vptr)&ld[64 * wave], 4, q * 4, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_vptr)&dd[64 * wave], 4, q * 4, 0, 0, 0);
    }
  };
  // this lane's predicate word: K row 32 kb + lq against the 32 rows of Q block qb
  auto load_mask = [&](const Item& it) -> uint32_t {
    return it.pair >= 0 ? p.k_masks[((int64_t)it.pair * TKV + 32 * kb + lq) * NQB + qb]
                        : 0xFFFFFFFFu;
  };

  const int kloc = j * TKV + 32 * kb + lq;   // this lane's sample-local K row
  const uint32_t k_row_off = (uint32_t)kloc * kv_rs;
  const int qa0 = row_base<D>(32 * qb + lq, g), ka0 = row_base<D>(32 * kb + lq, g);
  const int ta0 = tr_base<D>(lane) + 32 * qb * 2 * D;
  Item cur = Item{0, 0, -1}, nxt = Item{0, 0, -1};
  uint32_t mw_cur = 0, mw_next = 0;
  float slope_cur = 0.0f;
  if (n_items > 0) {   // the first two items' Q tiles, read before any fill
    const int32_t* src;
    int i0 = 0, i1 = 0;
    locate(0, cur.h, src, cur.pair);
    i0 = *src;
    if (n_items > 1) {
      locate(1, nxt.h, src, nxt.pair);
      i1 = *src;
    }
    const float s0 = slope_of(cur.h);
    cur.i = __builtin_amdgcn_readfirstlane(i0);
    nxt.i = __builtin_amdgcn_readfirstlane(i1);
    slope_cur = slope_units(s0);
  }
  dma_tile<D, TKV, NW>(k_s, rk, (uint32_t)j * TKV * kv_rs, kv_rs, wave, lane);
  if (n_items > 0) {
    load_item(cur, q_s0, do_s0, lse_s0, dd_s0);
    mw_cur = load_mask(cur);
  }
  bf16x8 vf[DS];
  load_row_frags<D>(vf, rv, k_row_off, g);

  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_dk[db] = acc_dv[db] = f32x16{};

  int n = 0;
  auto step = [&](auto stage) __attribute__((always_inline)) {
    const auto nx = flip(stage);
    const __bf16* qs = qbuf(stage);
    const __bf16* dos = dobuf(stage);
    const float* ls = lsebuf(stage);
    const float* ds = ddbuf(stage);
    const bool more = n + 1 < n_items;
    // the Q tile of the item after next and the next item's slope, read
    // before the next item's fill so that waiting for them (after this
    // item's block) does not wait for the fill
    Item after = Item{0, 0, -1};
    int after_i = 0;
    float slope_nxt = 0.0f;
    if (n + 2 < n_items) {
      const int32_t* src;
      locate_lds(n + 2, after.h, src, after.pair);
      after_i = *src;
    }
    if (more) {
      slope_nxt = slope_of(nxt.h);
      load_item(nxt, qbuf(nx), dobuf(nx), lsebuf(nx), ddbuf(nx));
      mw_next = load_mask(nxt);
    }
    // read bases, opaque per item so that the addresses derived from them
    // are formed inside the item rather than held across the loop
    int qa = qa0, ka = ka0, ta = ta0;
    asm volatile("" : "+v"(qa), "+v"(ka), "+v"(ta));
    const float slope = slope_cur;
    // k - q of this lane's K row and the block's Q row 4 g (element offsets
    // 8 (v / 4) + v % 4 are subtracted per element)
    const float kq0 = (float)(kloc - cur.i * TQ - 32 * qb - 4 * g);
    auto block = [&]() __attribute__((always_inline)) {
      // S = Q K^T and dP = dO V^T (lane: K row lq; element v: Q row
      // 8 (v / 4) + 4 g + v % 4 of the block); dP starts from the rows' -Dq,
      // so its accumulator ends as dP - Dq
      f32x16 s_acc = f32x16{}, dp_acc;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 d4 = *(const float4*)&ds[32 * qb + 8 * a + 4 * g];
        dp_acc[4 * a] = d4.x;
        dp_acc[4 * a + 1] = d4.y;
        dp_acc[4 * a + 2] = d4.z;
        dp_acc[4 * a + 3] = d4.w;
      }
      // (operands are not read ahead: the registers are full, and a spill
      // reloaded after the next item's fill would wait for the whole fill)
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 aq = lds_at(qs, qa ^ (32 * s));
        const bf16x8 ad = lds_at(dos, qa ^ (32 * s));
        const bf16x8 ak = lds_at(k_s, ka ^ (32 * s));
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, ak, s_acc, 0, 0, 0);
        dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vf[s], dp_acc, 0, 0, 0);
      }
      // weights and dS, rounded to bf16 as the B operands of the gradients
      bf16x8 pb8[2], dsb[2];
      const uint32_t mw = mw_cur >> (4 * g);
      float base;   // per-lane part of the exponent that does not depend on the element
      if constexpr (MOD == kModAlibi) base = slope * kq0;
      else if constexpr (MOD == kModSoftcapAlibi) base = fmaf(slope, kq0, p.softcap_c2);
      else if constexpr (MOD == kModSoftcap) base = p.softcap_c2;
      else base = 0.0f;
      auto elem = [&](int v) __attribute__((always_inline)) {
        const int pos = 8 * (v / 4) + v % 4;
        const float s = s_acc[v];
        const float lse = ls[32 * qb + 4 * g + pos];
        float t, grad = 1.0f;
        if constexpr (MOD == kModNone) {
          t = fmaf(s, p.scale_log2, -lse);
        } else if constexpr (MOD == kModAlibi) {
          t = fmaf(s, p.scale_log2, fmaf(-slope, (float)pos, base)) - lse;
        } else if constexpr (MOD == kModAlibiSoftcap) {
          const float r =
              rcp_fast(1.0f + exp2_fast(fmaf(s, p.softcap_k, slope * (kq0 - (float)pos))));
          grad = fmaf(-r, r, r);
          t = fmaf(-2.0f * p.softcap_c2, r, p.softcap_c2) - lse;
        } else {   // softcap, then ALiBi for kModSoftcapAlibi (in base)
          const float r = rcp_fast(1.0f + exp2_fast(s * p.softcap_k));
          grad = fmaf(-r, r, r);
          float u = fmaf(-2.0f * p.softcap_c2, r, base);
          if constexpr (MOD == kModSoftcapAlibi) u = fmaf(-slope, (float)pos, u);
          t = u - lse;
        }
        // the predicate bit sign-extended to an all-ones or all-zeros mask
        int keep;
        asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(keep) : "v"(mw), "i"(pos));
        const float P = __int_as_float(__float_as_int(exp2_fast(t)) & keep);
        float dS = P * dp_acc[v];
        if constexpr (kSoftcap) dS *= grad;
        pb8[v / 8][v % 8] = (__bf16)P;
        dsb[v / 8][v % 8] = (__bf16)dS;
      };
      // dV^T += dO^T P and dK^T += Q^T dS over the block's Q rows 16 m ..
      // 16 m + 15: the products of rows 0..15 run while the weights of rows
      // 16..31 are formed
      // transposed operands of product x (rows 16 (x / DB), columns block x % DB)
      bf16x8 fd[2], fq[2];
      auto tr_read = [&](int x, int c) __attribute__((always_inline)) {
        const int off = (ta ^ (64 * (x % DB))) + 16 * (x / DB) * 2 * D;
        fd[c] = lds_tr_at<D>(dos, off);
        fq[c] = lds_tr_at<D>(qs, off);
      };
#pragma unroll
      for (int v = 0; v < 8; ++v) elem(v);
#pragma unroll
      for (int x = 0; x < 2 * DB; ++x) {
        const int c = x & 1, m = x / DB, db = x % DB;
        tr_read(x, c);
        acc_dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fd[c], pb8[m], acc_dv[db], 0, 0, 0);
        if (m == 0) elem(8 + 2 * db);
        acc_dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[c], dsb[m], acc_dk[db], 0, 0, 0);
        if (m == 0) elem(9 + 2 * db);
        if (x == DB - 1) {
#pragma unroll
          for (int v = 8 + 2 * DB; v < 16; ++v) elem(v);
        }
      }
    };
    // a block whose predicate hides all of its Q rows from all of the
    // wavefront's K rows contributes nothing (every weight is exactly 0) ...
    bool need = p.no_skip != 0 || __builtin_amdgcn_ballot_w64(mw_cur != 0) != 0;
    // ... and so does one whose weights are all negligible: the bound of
    // every exponent over the lane's 16 elements against its rows' least LSE
    // (the 200 margin covers the rounding of the exponent's terms)
    if constexpr (MOD == kModSoftcapAlibi) {
      if (need && !p.no_skip) {
        float lmin = kPosInf;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float4 l4 = *(const float4*)&ls[32 * qb + 8 * a + 4 * g];
          lmin = fminf(lmin, fminf(fminf(l4.x, l4.y), fminf(l4.z, l4.w)));
        }
        const float bound = softcap_alibi_bound(p.softcap_c2, slope, kq0 - 27.0f);
        need = __builtin_amdgcn_ballot_w64(!(bound < lmin - kNegligibleLog2)) != 0;
      }
    }
    // (one code path: a full pair's predicate words are all ones; two paths
    // would not fit the register file together)
    if (need) block();
    asm volatile("" : "+v"(after_i), "+v"(slope_nxt));   // used from here on only
    if (more) {
      mw_cur = mw_next;
      cur = nxt;
      slope_cur = slope_units(slope_nxt);
      after.i = __builtin_amdgcn_readfirstlane(after_i);
      nxt = after;
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wavefront's loads of the next item have landed
    __syncthreads();                 // ... and everyone's; this item's reads are done
    ++n;
  };
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n_items > 0) {
    while (n + 1 < n_items) {
      step(S0{});
      step(S1{});
    }
    if (n < n_items) step(S0{});
  }

  // The four Q blocks of each K block add their sums in two rounds through
  // the Q and dO buffers (free now): blocks 2 and 3 hand over to 0 and 1,
  // then 1 to 0, which stores.
  static_assert(2 * DB * 16 * 64 * 4 <= TQ * D * 2, "reduction slot");
  auto slot = [&](int i) -> float* {
    __bf16* s = i == 0 ? q_s0 : i == 1 ? q_s1 : i == 2 ? do_s0 : do_s1;
    return reinterpret_cast<float*>(s);
  };
  auto put = [&](float* r) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const float4 a = {acc_dk[db][4 * v4], acc_dk[db][4 * v4 + 1], acc_dk[db][4 * v4 + 2],
                          acc_dk[db][4 * v4 + 3]};
        const float4 c = {acc_dv[db][4 * v4], acc_dv[db][4 * v4 + 1], acc_dv[db][4 * v4 + 2],
                          acc_dv[db][4 * v4 + 3]};
        *(float4*)&r[((db * 4 + v4) * 64 + lane) * 4] = a;
        *(float4*)&r[((DB * 4 + db * 4 + v4) * 64 + lane) * 4] = c;
      }
  };
  auto take = [&](const float* r) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const float4 a = *(const float4*)&r[((db * 4 + v4) * 64 + lane) * 4];
        const float4 c = *(const float4*)&r[((DB * 4 + db * 4 + v4) * 64 + lane) * 4];
        acc_dk[db][4 * v4] += a.x; acc_dk[db][4 * v4 + 1] += a.y;
        acc_dk[db][4 * v4 + 2] += a.z; acc_dk[db][4 * v4 + 3] += a.w;
        acc_dv[db][4 * v4] += c.x; acc_dv[db][4 * v4 + 1] += c.y;
        acc_dv[db][4 * v4 + 2] += c.z; acc_dv[db][4 * v4 + 3] += c.w;
      }
  };
  if (qb >= 2) put(slot((qb - 2) * NKW + kb));
  __syncthreads();
  if (qb < 2) take(slot(qb * NKW + kb));
  __syncthreads();
  if (qb == 1) put(slot(kb));
  __syncthreads();
  if (qb == 0) {
    take(slot(kb));
    store_rows<D>(rdk, k_row_off, acc_dk, kSoftcap ? 4.0f * p.scale : p.scale, g);
    store_rows<D>(rdv, k_row_off, acc_dv, 1.0f, g);
  }
}

// ------------------------------------------------------------------ dispatch

namespace {

template <int D, int TQ, int TKV, int MOD>
hipError_t launch_bwd_mod(int num_tasks, const BwdParams& p, hipStream_t s) {
  if (num_tasks > 0)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, TQ, TKV, MOD>), dim3(num_tasks), dim3(TQ * 2), 0, s,
                       p);
  const int64_t items = (int64_t)p.heads_k * p.krows_total;
  if (items > 0) {
    bool split = false;
    if constexpr (TQ / 32 * (TKV / 32) == 8) {   // eight 32 x 32 blocks per pair
      split = p.group <= 64;   // the split kernel keeps a group's lists in one wavefront
      if (split)
        hipLaunchKernelGGL((attn_bwd_dkdv_split_kernel<D, TQ, TKV, MOD>),
                           dim3((unsigned)items), dim3(TQ * TKV / 16), 0, s, p);
    }
    if (!split)
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, TQ, TKV, MOD>), dim3((unsigned)items),
                         dim3(TKV * 4), 0, s, p);
  }
  return hipGetLastError();
}

template <int D, int TQ, int TKV>
hipError_t launch_bwd(int mod, int num_tasks, const BwdParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.total_q * p.heads_q;
  if (rows > 0)
    hipLaunchKernelGGL((attn_bwd_dot_kernel<D>), dim3((unsigned)((rows * (D / 8) + 255) / 256)),
                       dim3(256), 0, s, p);
  switch (mod) {
    case kModNone: return launch_bwd_mod<D, TQ, TKV, kModNone>(num_tasks, p, s);
    case kModSoftcap: return launch_bwd_mod<D, TQ, TKV, kModSoftcap>(num_tasks, p, s);
    case kModAlibi: return launch_bwd_mod<D, TQ, TKV, kModAlibi>(num_tasks, p, s);
    case kModSoftcapAlibi: return launch_bwd_mod<D, TQ, TKV, kModSoftcapAlibi>(num_tasks, p, s);
    case kModAlibiSoftcap: return launch_bwd_mod<D, TQ, TKV, kModAlibiSoftcap>(num_tasks, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// The backward consumers: bf16 at the forward's bf16 tile geometries.
#define MPB_BWD_VARIANTS(X) \
  X(128, 128, 64) X(128, 64, 64) X(128, 128, 32) X(128, 64, 32) X(64, 128, 64) X(64, 64, 64)

bool attn_bwd_variant_exists(int32_t dtype, int32_t head_dim, int32_t tile_q, int32_t tile_k) {
  if (dtype != MPB_DTYPE_BF16) return false;
#define X(D_, TQ_, TKV_) \
  if (head_dim == D_ && tile_q == TQ_ && tile_k == TKV_) return true;
  MPB_BWD_VARIANTS(X)
#undef X
  return false;
}

hipError_t launch_attn_bwd(int32_t head_dim, int32_t tile_q, int32_t tile_k, int32_t mod_kind,
                           int32_t num_tasks, const BwdParams& p, hipStream_t s) {
#define X(D_, TQ_, TKV_) \
  if (head_dim == D_ && tile_q == TQ_ && tile_k == TKV_) return launch_bwd<D_, TQ_, TKV_>(mod_kind, num_tasks, p, s);
  MPB_BWD_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace mpb
