// Block-sparse flex attention forward for gfx950 (MI355X).
//
// Computes FlexAttention's Eq. 1, softmax(mod(Q K^T * scale)) V, over the K
// tiles a MaskPlan lists ("Flex Attention Mask Plan Design" §6.1): partial
// tiles first with their packed predicate, then full tiles without it; empty
// tiles are never touched; a row with nothing visible gets O = 0, LSE = -inf.
//
// Design (gfx950 native, not a port of any CUDA kernel):
//  * One workgroup = NW wavefronts = one Q tile of 32*NW rows; a persistent
//    grid pulls tasks from per-section work queues (one per XCD) through
//    atomic counters held in caller workspace (§4.8 dynamic scheduler).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator a lane holds one Q
//    column (q = lane%32) and 16 K rows {8a + 4*(lane/32) + c}.  So the
//    softmax row max/sum is 16 in-lane values plus one exchange with lane^32,
//    the packed predicate of a 32-column block is one dword per lane, and P
//    feeds the P.V MFMA straight from registers: O^T = V^T P^T, where the V
//    operand is read from an LDS copy of V stored transposed with its K order
//    permuted (bits 2 and 3 swapped) so each lane reads 8 contiguous values.
//  * K and V^T tiles are staged in LDS (double buffered, padded rows) from
//    coalesced 16-byte HBM loads issued one tile ahead.
//  * Online softmax in base 2 (scale*log2e folded into one multiply), fp32
//    statistics, P rounded to bf16 for the second MFMA.
//  * fp32 inputs use v_mfma_f32_32x32x2_f32 with the same accumulator layout
//    and keep P in fp32.
#include "mpb_internal.h"
#include "../../include/mpb.h"

namespace mpb {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// Position of K index k inside a permuted V^T row: bits 2 and 3 swapped.
__device__ constexpr int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// ----------------------------------------------------------------- bf16 tiles

template <int D_, int NW_, int TKV_>
struct Bf16Ops {
  using T = __bf16;
  static constexpr int D = D_, NW = NW_, TKV = TKV_;
  static constexpr int NT = NW * 64, TQ = 32 * NW, NKB = TKV / 32;
  static constexpr int KP = D + 8;    // K row pitch (elements): 16 B pad, conflict-free b128 reads
  static constexpr int VP = TKV + 8;  // V^T row pitch (elements)
  static constexpr int KCH = TKV * D / 8 / NT;          // 16-byte K chunks per thread
  static constexpr int VCH = (TKV / 2) * (D / 8) / NT;  // V row-pair chunks per thread
  static_assert(KCH * NT * 8 == TKV * D, "K tile must split evenly over threads");
  static_assert(VCH * NT * 16 == TKV * D, "V tile must split evenly over threads");
  static_assert(D % 32 == 0 && TKV % 32 == 0, "tile shape");

  struct Smem {
    __bf16 k[2][TKV * KP];
    __bf16 vt[2][D * VP];
  };
  struct QFrag { bf16x8 q[D / 16]; };
  struct Stage { u32x4 k[KCH]; u32x4 v0[VCH]; u32x4 v1[VCH]; };
  struct PFrag { bf16x8 p[NKB][2]; };

  // Tile rows >= rows_valid (past the sample's k_len) are zero-filled, so
  // no stale or foreign value can reach P.V.
  static __device__ inline void load(Stage& st, const __bf16* kg, const __bf16* vg, int64_t rs,
                                     int rows_valid, int tid) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      st.k[c] = r < rows_valid ? *(const u32x4*)(kg + r * rs + c8 * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = tid + c * NT;
      const int pr = idx % (TKV / 2), c8 = idx / (TKV / 2);
      const int r0 = 2 * pr;
      st.v0[c] = r0 < rows_valid ? *(const u32x4*)(vg + r0 * rs + c8 * 8) : u32x4{0, 0, 0, 0};
      st.v1[c] = r0 + 1 < rows_valid ? *(const u32x4*)(vg + (r0 + 1) * rs + c8 * 8)
                                     : u32x4{0, 0, 0, 0};
    }
  }

  static __device__ inline void store(const Stage& st, Smem& sm, int stage, int tid) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      *(u32x4*)&sm.k[stage][r * KP + c8 * 8] = st.k[c];
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = tid + c * NT;
      const int pr = idx % (TKV / 2), c8 = idx / (TKV / 2);
      const int pos = vt_pos(2 * pr);  // rows 2pr, 2pr+1 stay adjacent
      __bf16* dst = &sm.vt[stage][(c8 * 8) * VP + pos];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = st.v0[c][w], b = st.v1[c][w];
        *(uint32_t*)(dst + (2 * w) * VP) = (a & 0xFFFFu) | (b << 16);
        *(uint32_t*)(dst + (2 * w + 1) * VP) = (a >> 16) | (b & 0xFFFF0000u);
      }
    }
  }

  static __device__ inline void load_q(QFrag& qf, const __bf16* qrow, int b2) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if (qrow) {
        qf.q[s] = *(const bf16x8*)(qrow + 16 * s + 8 * b2);
      } else {
        u32x4 z = {0, 0, 0, 0};
        qf.q[s] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }

  static __device__ inline void qk(f32x16 (&acc)[NKB], const QFrag& qf, const Smem& sm, int stage,
                                   int lane) {
    const __bf16* kb = &sm.k[stage][(lane & 31) * KP + 8 * (lane >> 5)];
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) acc[kk] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const bf16x8 a = *(const bf16x8*)(kb + kk * 32 * KP + 16 * s);
        acc[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.q[s], acc[kk], 0, 0, 0);
      }
    }
  }

  static __device__ inline void to_p(PFrag& pf, const f32x16 (&acc)[NKB]) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf.p[kk][m][e] = (__bf16)acc[kk][8 * m + e];
  }

  static __device__ inline void pv(f32x16 (&o)[D / 32], const PFrag& pf, const Smem& sm,
                                   int stage, int lane) {
    const __bf16* vb = &sm.vt[stage][(lane & 31) * VP + 8 * (lane >> 5)];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const bf16x8 a = *(const bf16x8*)(vb + db * 32 * VP + kk * 32 + 16 * m);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf.p[kk][m], o[db], 0, 0, 0);
        }
  }

  static __device__ inline void store_o(__bf16* orow, const f32x16 (&o)[D / 32], float inv,
                                        int b2) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (__bf16)(o[db][4 * a + c] * inv);
        *(bf16x4*)(orow + db * 32 + 8 * a + 4 * b2) = v;
      }
  }
};

// ----------------------------------------------------------------- fp32 tiles

template <int D_, int NW_, int TKV_>
struct F32Ops {
  using T = float;
  static constexpr int D = D_, NW = NW_, TKV = TKV_;
  static constexpr int NT = NW * 64, TQ = 32 * NW, NKB = TKV / 32;
  static constexpr int KP = D + 4;   // 16-byte reads of 32 rows: banks 4r, conflict-free
  static constexpr int VP = D + 8;   // lanes 32..63 read row k+4: +32 banks
  static constexpr int KCH = TKV * D / 4 / NT;
  static constexpr int VCH = TKV * D / 4 / NT;
  static_assert(KCH * NT * 4 == TKV * D, "tile must split evenly over threads");

  struct Smem {
    float k[2][TKV * KP];
    float v[2][TKV * VP];
  };
  struct QFrag { float q[D / 2]; };
  struct Stage { f32x4 k[KCH]; f32x4 v[VCH]; };
  struct PFrag { f32x16 p[NKB]; };

  static __device__ inline void load(Stage& st, const float* kg, const float* vg, int64_t rs,
                                     int rows_valid, int tid) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      st.k[c] = r < rows_valid ? *(const f32x4*)(kg + r * rs + c4 * 4) : f32x4{};
      st.v[c] = r < rows_valid ? *(const f32x4*)(vg + r * rs + c4 * 4) : f32x4{};
    }
  }

  static __device__ inline void store(const Stage& st, Smem& sm, int stage, int tid) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      *(f32x4*)&sm.k[stage][r * KP + c4 * 4] = st.k[c];
      *(f32x4*)&sm.v[stage][r * VP + c4 * 4] = st.v[c];
    }
  }

  static __device__ inline void load_q(QFrag& qf, const float* qrow, int b2) {
#pragma unroll
    for (int s = 0; s < D / 2; s += 4) {
      const f32x4 x = qrow ? *(const f32x4*)(qrow + b2 * (D / 2) + s) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf.q[s + e] = x[e];
    }
  }

  static __device__ inline void qk(f32x16 (&acc)[NKB], const QFrag& qf, const Smem& sm, int stage,
                                   int lane) {
    const float* kb = &sm.k[stage][(lane & 31) * KP + (lane >> 5) * (D / 2)];
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) acc[kk] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 2; s += 4) {
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const f32x4 a = *(const f32x4*)(kb + kk * 32 * KP + s);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[kk] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf.q[s + e], acc[kk], 0, 0, 0);
      }
    }
  }

  static __device__ inline void to_p(PFrag& pf, const f32x16 (&acc)[NKB]) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) pf.p[kk] = acc[kk];
  }

  static __device__ inline void pv(f32x16 (&o)[D / 32], const PFrag& pf, const Smem& sm,
                                   int stage, int lane) {
    const int b2 = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int k = kk * 32 + 8 * (v / 4) + 4 * b2 + (v % 4);
          const float a = sm.v[stage][k * VP + db * 32 + (lane & 31)];
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pf.p[kk][v], o[db], 0, 0, 0);
        }
  }

  static __device__ inline void store_o(float* orow, const f32x16 (&o)[D / 32], float inv, int b2) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = o[db][4 * a + c] * inv;
        *(f32x4*)(orow + db * 32 + 8 * a + 4 * b2) = v;
      }
  }
};

// ----------------------------------------------------------------- scheduling

__device__ inline int fetch_task(const AttnParams& p, int home, int& qpos) {
  // Home section first, then the others in rotation, then the zero-cost
  // queue.  Every counter only grows, so each workgroup leaves after at most
  // (tasks it ran + kNumQueues) atomics.
  while (qpos < kNumQueues) {
    const int q = qpos < kNumSections ? (home + qpos) % kNumSections : kNumSections;
    const int beg = p.section_off[q];
    const int size = p.section_off[q + 1] - beg;
    if (size > 0) {
      const int idx = atomicAdd(&p.counters[q], 1);
      if (idx < size) return beg + idx;
    }
    ++qpos;
  }
  return -1;
}

// score_mod in log2 units: returns log2(e) * mod(s * scale).  kq = k - q.
template <int MOD>
__device__ inline float mod_score(float s, float kq, const AttnParams& p, float slope) {
  if constexpr (MOD == kModNone) {
    return s * p.scale_log2;
  } else if constexpr (MOD == kModAlibi) {
    return fmaf(s, p.scale_log2, slope * kq);            // slope = slope_h * log2e
  } else if constexpr (MOD == kModSoftcap || MOD == kModSoftcapAlibi) {
    // c*tanh(x) = c - 2c / (1 + e^{2x}),  e^{2x} = exp2(s * 2*scale*log2e/c)
    const float e = exp2_fast(s * p.softcap_k);
    float u = fmaf(-2.0f * p.softcap_c2, rcp_fast(1.0f + e), p.softcap_c2);
    if constexpr (MOD == kModSoftcapAlibi) u = fmaf(slope, kq, u);
    return u;
  } else {  // kModAlibiSoftcap: tanh of (s*scale + slope_h*(k-q)) / c
    const float e = exp2_fast(fmaf(s, p.softcap_k, slope * kq));  // slope = slope_h*2*log2e/c
    return fmaf(-2.0f * p.softcap_c2, rcp_fast(1.0f + e), p.softcap_c2);
  }
}

template <class Ops, int MOD>
__global__ __launch_bounds__(Ops::NT) void attn_fwd_kernel(AttnParams p) {
  using T = typename Ops::T;
  constexpr int D = Ops::D, TQ = Ops::TQ, TKV = Ops::TKV, NKB = Ops::NKB;
  __shared__ typename Ops::Smem sm;
  __shared__ int s_task;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b2 = lane >> 5;
  const int lq = lane & 31;
  const int home = blockIdx.x % kNumSections;
  int qpos = 0;

  const T* __restrict__ Qg = (const T*)p.q;
  const T* __restrict__ Kg = (const T*)p.k;
  const T* __restrict__ Vg = (const T*)p.v;
  T* __restrict__ Og = (T*)p.o;
  const int64_t q_rs = (int64_t)p.heads_q * D;
  const int64_t kv_rs = (int64_t)p.heads_k * D;

  while (true) {
    if (tid == 0) s_task = fetch_task(p, home, qpos);
    __syncthreads();
    const int task = s_task;
    __syncthreads();
    if (task < 0) break;

    const int32_t* wd = p.work_desc + 4 * (int64_t)task;
    const int m_block = wd[0], h = wd[1], b = wd[2];
    const int32_t* sd = p.seqdesc + 8 * b;
    const int q_off = sd[0], k_off = sd[1], q_len = sd[2], k_len = sd[3];
    const int g = h / p.group;
    const int hm = p.mask_heads == 1 ? 0 : h;
    const int64_t flat = (int64_t)hm * p.rows_total + sd[4] + m_block;
    const int p_beg = p.p_off[flat];
    const int np = p.p_off[flat + 1] - p_beg;
    const int f_beg = p.f_off[flat];
    const int ntiles = np + (p.f_off[flat + 1] - f_beg);

    const int qloc = m_block * TQ + 32 * wave + lq;  // sample-local Q row of this lane
    const bool qvalid = qloc < q_len;
    typename Ops::QFrag qf;
    Ops::load_q(qf, qvalid ? Qg + (q_off + (int64_t)qloc) * q_rs + (int64_t)h * D : nullptr, b2);

    float slope = 0.0f;
    if constexpr (MOD == kModAlibi || MOD == kModSoftcapAlibi) slope = p.slopes[h] * kLog2e;
    if constexpr (MOD == kModAlibiSoftcap) slope = p.slopes[h] * p.alibi_k;

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;

    const T* kbase = Kg + (int64_t)k_off * kv_rs + (int64_t)g * D;
    const T* vbase = Vg + (int64_t)k_off * kv_rs + (int64_t)g * D;
    // tile t of the task: partial list first, then full list (§6.1)
    auto tile_j = [&](int t) { return t < np ? p.p_idx[p_beg + t] : p.f_idx[f_beg + t - np]; };
    auto load_masks = [&](int t, uint32_t (&mw)[NKB]) {
      if (t < np) {
        const uint32_t* src = p.p_masks + ((int64_t)(p_beg + t) * TQ + 32 * wave + lq) * NKB;
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) mw[kk] = src[kk] >> (4 * b2);
      } else {
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) mw[kk] = 0xFFFFFFFFu;
      }
    };

    if (ntiles > 0) {
      typename Ops::Stage st;
      uint32_t mw_cur[NKB], mw_next[NKB];
      int j_cur = tile_j(0);
      Ops::load(st, kbase + (int64_t)j_cur * TKV * kv_rs, vbase + (int64_t)j_cur * TKV * kv_rs,
                kv_rs, min(TKV, k_len - j_cur * TKV), tid);
      load_masks(0, mw_cur);
      Ops::store(st, sm, 0, tid);
      __syncthreads();

      for (int t = 0; t < ntiles; ++t) {
        const int stage = t & 1;
        const bool partial = t < np || p.force_partial;
        const bool more = t + 1 < ntiles;
        int j_next = 0;
        if (more) {
          j_next = tile_j(t + 1);
          Ops::load(st, kbase + (int64_t)j_next * TKV * kv_rs,
                    vbase + (int64_t)j_next * TKV * kv_rs, kv_rs,
                    min(TKV, k_len - j_next * TKV), tid);
          load_masks(t + 1, mw_next);
        }

        f32x16 acc[NKB];
        Ops::qk(acc, qf, sm, stage, lane);

        // score_mod, predicate, running max
        const float kq0 = (float)(j_cur * TKV + 4 * b2 - qloc);
        float mt = kNegInf;
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float kq = kq0 + (float)(kk * 32 + 8 * (v / 4) + (v % 4));
            float u = mod_score<MOD>(acc[kk][v], kq, p, slope);
            if (partial && !((mw_cur[kk] >> (8 * (v / 4) + (v % 4))) & 1u)) u = kNegInf;
            acc[kk][v] = u;
            mt = fmaxf(mt, u);
          }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        float rs = 0.0f;
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float e = exp2_fast(acc[kk][v] - m_use);
            acc[kk][v] = e;
            rs += e;
          }
        l_run = fmaf(l_run, alpha, rs);
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;

        typename Ops::PFrag pf;
        Ops::to_p(pf, acc);
        Ops::pv(o, pf, sm, stage, lane);

        if (more) {
          Ops::store(st, sm, stage ^ 1, tid);
#pragma unroll
          for (int kk = 0; kk < NKB; ++kk) mw_cur[kk] = mw_next[kk];
          j_cur = j_next;
        }
        __syncthreads();
      }
    }

    // epilogue: O = acc / l, LSE = m + ln l (natural log); empty rows 0 / -inf
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qvalid) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      Ops::store_o(Og + (q_off + (int64_t)qloc) * q_rs + (int64_t)h * D, o, inv, b2);
      if (b2 == 0) {
        p.lse[(int64_t)h * p.total_q + q_off + qloc] =
            l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
      }
    }
  }
}

__global__ void reset_counters_kernel(int32_t* c) {
  if (threadIdx.x <= kNumQueues) c[threadIdx.x] = 0;
}

// ----------------------------------------------------------------- dispatch

template <class Ops>
hipError_t launch_ops(int mod, int grid, const AttnParams& p, hipStream_t s) {
  const dim3 g(grid), blk(Ops::NT);
  switch (mod) {
    case kModNone: hipLaunchKernelGGL((attn_fwd_kernel<Ops, kModNone>), g, blk, 0, s, p); break;
    case kModSoftcap: hipLaunchKernelGGL((attn_fwd_kernel<Ops, kModSoftcap>), g, blk, 0, s, p); break;
    case kModAlibi: hipLaunchKernelGGL((attn_fwd_kernel<Ops, kModAlibi>), g, blk, 0, s, p); break;
    case kModSoftcapAlibi: hipLaunchKernelGGL((attn_fwd_kernel<Ops, kModSoftcapAlibi>), g, blk, 0, s, p); break;
    case kModAlibiSoftcap: hipLaunchKernelGGL((attn_fwd_kernel<Ops, kModAlibiSoftcap>), g, blk, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class Ops>
int occupancy_grid(int num_tasks, int device) {
  static int cached[16] = {0};
  int& per_cu = cached[device & 15];
  if (per_cu == 0) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_fwd_kernel<Ops, kModNone>,
                                                     Ops::NT, 0) != hipSuccess || blocks < 1)
      blocks = 1;
    per_cu = blocks;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus < 1)
    cus = 256;
  const int g = per_cu * cus;
  return num_tasks < g ? num_tasks : g;
}

// The consumer table: (dtype, head_dim, tile_q, tile_k) -> kernel family.
#define MPB_VARIANTS(X)                         \
  X(MPB_DTYPE_BF16, 128, 128, 64, Bf16Ops<128, 4, 64>) \
  X(MPB_DTYPE_BF16, 128, 64, 64, Bf16Ops<128, 2, 64>)  \
  X(MPB_DTYPE_BF16, 128, 128, 32, Bf16Ops<128, 4, 32>) \
  X(MPB_DTYPE_BF16, 128, 64, 32, Bf16Ops<128, 2, 32>)  \
  X(MPB_DTYPE_BF16, 64, 128, 64, Bf16Ops<64, 4, 64>)   \
  X(MPB_DTYPE_BF16, 64, 64, 64, Bf16Ops<64, 2, 64>)    \
  X(MPB_DTYPE_FP32, 64, 64, 64, F32Ops<64, 2, 64>)     \
  X(MPB_DTYPE_FP32, 64, 64, 32, F32Ops<64, 2, 32>)     \
  X(MPB_DTYPE_FP32, 128, 64, 32, F32Ops<128, 2, 32>)

}  // namespace

bool attn_variant_exists(int32_t dtype, int32_t head_dim, int32_t tile_q, int32_t tile_k) {
#define X(DT, HD, TQ_, TK_, ...) \
  if (dtype == DT && head_dim == HD && tile_q == TQ_ && tile_k == TK_) return true;
  MPB_VARIANTS(X)
#undef X
  return false;
}

hipError_t launch_attn_fwd(int32_t dtype, int32_t head_dim, int32_t tile_q, int32_t tile_k,
                           int32_t mod_kind, int32_t grid, const AttnParams& p, hipStream_t s) {
#define X(DT, HD, TQ_, TK_, ...) \
  if (dtype == DT && head_dim == HD && tile_q == TQ_ && tile_k == TK_) return launch_ops<__VA_ARGS__>(mod_kind, grid, p, s);
  MPB_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

int32_t attn_grid_size(int32_t dtype, int32_t head_dim, int32_t tile_q, int32_t tile_k,
                       int32_t num_tasks, int device) {
#define X(DT, HD, TQ_, TK_, ...) \
  if (dtype == DT && head_dim == HD && tile_q == TQ_ && tile_k == TK_) return occupancy_grid<__VA_ARGS__>(num_tasks, device);
  MPB_VARIANTS(X)
#undef X
  return 0;
}

hipError_t launch_reset_counters(int32_t* counters, hipStream_t s) {
  hipLaunchKernelGGL(reset_counters_kernel, dim3(1), dim3(64), 0, s, counters);
  return hipGetLastError();
}

}  // namespace mpb
