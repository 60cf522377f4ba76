// Block-sparse flex attention forward for gfx950 (MI355X).
//
// Computes FlexAttention's Eq. 1, softmax(mod(Q K^T * scale)) V, over the K
// tiles a MaskPlan lists ("Flex Attention Mask Plan Design" §6.1): partial
// tiles first with their packed predicate, then full tiles without it; empty
// tiles are never touched; a row with nothing visible gets O = 0, LSE = -inf.
//
// Design (gfx950 native, not a port of any CUDA kernel):
//  * One workgroup = NW wavefronts = one Q tile of 32*NW rows = one task of
//    the plan's launch order (§4.8): workgroup i reads record i, which holds
//    the task's geometry, CSR ranges and first K tile, so its Q and first K/V
//    loads issue after one record read.  Sections are interleaved in the
//    launch order because workgroups reach the XCDs round-robin; the hardware
//    dispatcher balances the load (cost-descending order within a section).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator a lane holds one Q
//    column (q = lane%32) and 16 K rows {8a + 4*(lane/32) + c}.  So the
//    softmax row max/sum is 16 in-lane values plus one exchange with lane^32,
//    the packed predicate of a 32-column block is one dword per lane, and P
//    feeds the P.V MFMA straight from registers: O^T = V^T P^T, where the
//    V^T operand is read from the row-major V tile with ds_read_b64_tr_b16.
//  * Q, K, V and O are addressed through buffer resources bounded by the
//    task's sample: loads past k_len/q_len return zero and stores past q_len
//    are dropped by the hardware range check, so the tail protection of the
//    plan design (§4.3, §4.8) costs no branch; offsets are 32-bit.
//  * bf16 K and V tiles go straight from HBM into LDS (16-byte buffer loads
//    with the LDS flag, swizzled rows), double buffered in separate LDS
//    arrays and fetched one tile ahead; fp32 tiles pass through registers.
//  * Online softmax in base 2 with lazy rescaling: the running max used for
//    the exponent only moves when a row's max grows by more than 2^8, and the
//    O rescale is skipped by the whole wavefront when no lane moved.
//    Statistics in fp32, P rounded to bf16 for the second MFMA.
//  * fp32 inputs use v_mfma_f32_32x32x2_f32 with the same accumulator layout
//    and keep P in fp32.
#include <type_traits>

#include "mpb_internal.h"
#include "../../include/mpb.h"

namespace mpb {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();
// Lazy rescale threshold in log2 units: P values stay <= 2^8.
constexpr float kRescaleSlack = 8.0f;
// A weight exp2(u - m) with u more than this far below the reference max m
// is exactly 0 in fp32 (anything below 2^-149 underflows past the smallest
// denormal), so a tile whose scores all lie that far below it adds nothing to
// O or to the row sum and leaves the max alone: skipping it changes no bit of
// the result.
constexpr float kNegligibleLog2 = 200.0f;

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// Raw (stride 0) buffer descriptor over [base, base + bytes); gfx9 word 3.
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ inline u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}


// ----------------------------------------------------------------- bf16 tiles

// QB 32-row Q blocks per wavefront: every K or V^T fragment read from LDS
// feeds QB MFMAs, and one block's softmax can run while the other block's
// MFMAs are in flight.  QB = 2 needs one wavefront per SIMD.
//
// K goes straight from HBM into LDS (buffer_load ... lds: lane l of a
// wavefront writes LDS bytes [16 l, 16 l + 16) of the instruction's 1 KiB),
// rows unpadded, the 16-byte chunk c of row r stored at chunk position
// c ^ (r % CH): 8 or 16 consecutive lanes reading one logical chunk of
// consecutive rows then hit distinct banks.  V passes through registers to be
// stored transposed.
template <int D_, int NW_, int TKV_, int QB_>
struct Bf16Ops {
  using T = __bf16;
  static constexpr int D = D_, NW = NW_, TKV = TKV_, QB = QB_;
  static constexpr int NT = NW * 64, TQ = 32 * QB * NW, NKB = TKV / 32;
  static constexpr int WPE = QB == 1 ? (TKV == 32 ? 3 : 2) : 1;   // wavefronts per SIMD
  static constexpr int ESZ = 2;
  static constexpr int CH = D / 8;              // 16-byte chunks per K row
  static constexpr int RPI = 1024 / (D * 2);    // K rows per wavefront load instruction
  static constexpr int KI = TKV / RPI / NW;     // K load instructions per wavefront per tile
  static_assert(KI * RPI * NW == TKV, "K tile must split evenly over wavefronts");
  static_assert(D % 32 == 0 && TKV % 32 == 0 && CH <= 16 && CH >= 8, "tile shape");

  static constexpr int KELEMS = TKV * D, VELEMS = TKV * D;   // LDS elements per stage
  static constexpr bool kDirectLds = true;   // tiles land in LDS without registers
  struct QFrag { bf16x8 q[QB][D / 16]; };
  struct Stage {};
  typedef bf16x8 PBlock[NKB][2];
  struct PFrag { PBlock p[QB]; };

  // Swizzles of the 16-byte chunk positions inside a row: K is read as MFMA
  // operands by 32 lanes holding 32 consecutive rows (chunk c of row r at
  // c ^ (r % CH)); V by transposing reads whose 16-lane groups hold 4
  // consecutive rows and 2 neighbouring chunks (chunk c of row r at
  // c ^ 2 (r % 4)).  Either way the lanes serviced together hit distinct banks.
  static __device__ constexpr int kswz(int r) { return r % CH; }
  static __device__ constexpr int vswz(int r) { return 2 * (r % 4); }

  // tile_off = byte offset of the tile's first row; rs = bytes per token row.
  // K and V land in kdst / vdst (one stage's LDS buffers) when the issuing
  // wavefront's loads complete.
  static __device__ inline void load(Stage&, T* kdst, T* vdst, rsrc_t rk, rsrc_t rv,
                                     uint32_t tile_off, uint32_t rs, int tid) {
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int c = 0; c < KI; ++c) {
      const int r0 = (c * NW + wave) * RPI;
      const int r = r0 + lane / CH;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)&kdst[r0 * D], 16,
          (int)(tile_off + r * rs + ((lane % CH) ^ kswz(r)) * 16), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)&vdst[r0 * D], 16,
          (int)(tile_off + r * rs + ((lane % CH) ^ vswz(r)) * 16), 0, 0, 0);
    }
  }

  static __device__ inline void store(const Stage&, T*, T*, int) {}
  // Loads of one operand (K: kv = 0, V: kv = 1) of a tile by NW wavefronts,
  // with the tile's offset folded into the descriptor (built on the scalar
  // unit) so the per-lane offsets stay loop invariant: lane_off(kv, c, ...)
  // is the lane's byte offset within the tile for load instruction c of
  // wavefront `wave`.
  static __device__ inline uint32_t lane_off(int kv, int c, int wave, int lane, uint32_t rs) {
    const int r = (c * NW + wave) * RPI + lane / CH;
    return (uint32_t)r * rs + (uint32_t)(((lane % CH) ^ (kv ? vswz(r) : kswz(r))) * 16);
  }
  static __device__ inline void load_op(T* dst, rsrc_t r, const uint32_t (&voff)[KI], int wave) {
#pragma unroll
    for (int c = 0; c < KI; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)&dst[(c * NW + wave) * RPI * D], 16,
          (int)voff[c], 0, 0, 0);
  }

  static __device__ inline void load_q(QFrag& qf, rsrc_t rq, const uint32_t (&row_off)[QB],
                                       int b2) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        qf.q[qb][s] =
            __builtin_bit_cast(bf16x8, bload16(rq, row_off[qb] + (16 * s + 8 * b2) * ESZ));
  }

  // K fragments are read from LDS two k-steps ahead of the MFMAs using them.
  static __device__ inline void qk(f32x16 (&acc)[QB][NKB], const QFrag& qf, const T* kst,
                                   int lane) {
    // row kk*32 + lane%32, logical chunk 2s + lane/32, at chunk (2s) ^ x
    const __bf16* kb = &kst[(lane & 31) * D];
    const int x = (lane >> 5) ^ kswz(lane & 31);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) acc[qb][kk] = f32x16{};
    // ring of PF + 1 K-steps: step s + PF is requested while step s computes
    constexpr int PF = 2, NS = D / 16;
    bf16x8 a[PF + 1][NKB];
    auto fetch = [&](int s, bf16x8 (&dst)[NKB]) {
      const int off = ((2 * s) ^ x) * 8;
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) dst[kk] = *(const bf16x8*)(kb + kk * 32 * D + off);
    };
#pragma unroll
    for (int s = 0; s < PF; ++s) fetch(s, a[s]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + PF < NS) fetch(s + PF, a[(s + PF) % (PF + 1)]);
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s % (PF + 1)][kk], qf.q[qb][s],
                                                                acc[qb][kk], 0, 0, 0);
    }
  }

  static __device__ inline void to_p(PBlock& pb, const f32x16 (&acc)[NKB]) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kk][m][e] = (__bf16)acc[kk][8 * m + e];
  }

  // Sum of the bf16-rounded weights (the values P.V uses), two per
  // v_dot2_f32_bf16 against (1, 1).
  static __device__ inline float row_sum(const PBlock& pb, const f32x16 (&)[NKB]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    float s = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pb[kk][m][e], pb[kk][m][e + 1]};
          s = __builtin_amdgcn_fdot2_f32_bf16(pr, one, s, false);
        }
    return s;
  }

  // O^T += V^T P^T.  The V^T operand of MFMA (db, kk, m) is read from the
  // row-major V tile with two ds_read_b64_tr_b16: in each 16-lane group, lane
  // i receives element i % 4 of the rows addressed by lanes i/4 + 4j
  // (j = 0..3).  Lane r of the group addresses row kb + 4 kg + r/4 at
  // columns 32 db + 16 ((lane/16) % 2) + 4 (r % 4), so lane L receives
  // V[kb + 4 kg + j][32 db + L % 32] for j = 0..3: the 4 K slots of one
  // MFMA operand half, in the K order of the P registers (kb = 32 kk +
  // 16 m, then + 8 for slots 4..7).  Reads run three MFMAs ahead.
  static __device__ inline void pv(f32x16 (&o)[QB][D / 32], const PFrag& pf, const T* vst,
                                   int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int r = lane & 15, g2 = (lane >> 4) & 1, kg = lane >> 5;
    const int krow = 4 * kg + (r >> 2);            // lane part of the row
    const __bf16* vb = &vst[krow * D];
    int coff[D / 32];                              // lane part of the column, per db
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dcol = 32 * db + 16 * g2 + 4 * (r & 3);
      coff[db] = (((dcol >> 3) ^ vswz(krow)) << 3) + (dcol & 7);
    }
    constexpr int NS = (D / 32) * NKB * 2;
    auto frag = [&](int i) {
      const int db = i / (NKB * 2), kk = (i / 2) % NKB, m = i % 2;
      const __bf16* p0 = vb + (32 * kk + 16 * m) * D + coff[db];
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)p0);
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(p0 + 8 * D));
      const v4i16 both[2] = {lo, hi};
      return __builtin_bit_cast(bf16x8, both);
    };
    constexpr int PF = 3;
    bf16x8 a[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) a[i] = frag(i);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + PF < NS) a[(i + PF) % (PF + 1)] = frag(i + PF);
      const int db = i / (NKB * 2), kk = (i / 2) % NKB, m = i % 2;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % (PF + 1)], pf.p[qb][kk][m],
                                                            o[qb][db], 0, 0, 0);
    }
  }

  static __device__ inline void store_o(rsrc_t ro, uint32_t row_off, const f32x16 (&o)[D / 32],
                                        float inv, int b2) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (__bf16)(o[db][4 * a + c] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), ro,
                                              (int)(row_off + (db * 32 + 8 * a + 4 * b2) * ESZ),
                                              0, 0);
      }
  }
};

// ----------------------------------------------------------------- fp32 tiles

template <int D_, int NW_, int TKV_>
struct F32Ops {
  using T = float;
  static constexpr int D = D_, NW = NW_, TKV = TKV_;
  static constexpr int QB = 1;
  static constexpr int NT = NW * 64, TQ = 32 * NW, NKB = TKV / 32;
  static constexpr int WPE = 2;
  static constexpr int ESZ = 4;
  static constexpr int KP = D + 4;   // 16-byte reads of 32 rows: banks 4r, conflict-free
  static constexpr int VP = D + 8;   // lanes 32..63 read row k+4: +32 banks
  static constexpr int KCH = TKV * D / 4 / NT;
  static_assert(KCH * NT * 4 == TKV * D, "tile must split evenly over threads");

  static constexpr int KELEMS = TKV * KP, VELEMS = TKV * VP;   // LDS elements per stage
  static constexpr bool kDirectLds = false;  // tiles pass through registers
  static constexpr int KI = 1;               // (lane offsets of direct LDS loads: unused)
  struct QFrag { float q[QB][D / 2]; };
  struct Stage { u32x4 k[KCH]; u32x4 v[KCH]; };
  typedef f32x16 PBlock[NKB];
  struct PFrag { PBlock p[QB]; };

  static __device__ inline void load(Stage& st, T*, T*, rsrc_t rk, rsrc_t rv,
                                     uint32_t tile_off, uint32_t rs, int tid) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      st.k[c] = bload16(rk, tile_off + r * rs + c4 * 16);
      st.v[c] = bload16(rv, tile_off + r * rs + c4 * 16);
    }
  }

  static __device__ inline void store(const Stage& st, T* kdst, T* vdst, int tid) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      *(u32x4*)&kdst[r * KP + c4 * 4] = st.k[c];
      *(u32x4*)&vdst[r * VP + c4 * 4] = st.v[c];
    }
  }

  static __device__ inline void load_q(QFrag& qf, rsrc_t rq, const uint32_t (&row_off)[QB],
                                       int b2) {
#pragma unroll
    for (int s = 0; s < D / 2; s += 4) {
      const f32x4 x =
          __builtin_bit_cast(f32x4, bload16(rq, row_off[0] + (b2 * (D / 2) + s) * ESZ));
#pragma unroll
      for (int e = 0; e < 4; ++e) qf.q[0][s + e] = x[e];
    }
  }

  static __device__ inline void qk(f32x16 (&acc)[QB][NKB], const QFrag& qf, const T* kst,
                                   int lane) {
    const float* kb = &kst[(lane & 31) * KP + (lane >> 5) * (D / 2)];
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) acc[0][kk] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 2; s += 4) {
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const f32x4 a = *(const f32x4*)(kb + kk * 32 * KP + s);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[0][kk] =
              __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf.q[0][s + e], acc[0][kk], 0, 0, 0);
      }
    }
  }

  static __device__ inline void to_p(PBlock& pb, const f32x16 (&acc)[NKB]) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) pb[kk] = acc[kk];
  }

  static __device__ inline float row_sum(const PBlock&, const f32x16 (&acc)[NKB]) {
    float s = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[kk][v];
    return s;
  }

  static __device__ inline void pv(f32x16 (&o)[QB][D / 32], const PFrag& pf, const T* vst,
                                   int lane) {
    const int b2 = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int k = kk * 32 + 8 * (v / 4) + 4 * b2 + (v % 4);
          const float a = vst[k * VP + db * 32 + (lane & 31)];
          o[0][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pf.p[0][kk][v], o[0][db], 0, 0, 0);
        }
  }

  static __device__ inline void store_o(rsrc_t ro, uint32_t row_off, const f32x16 (&o)[D / 32],
                                        float inv, int b2) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = o[db][4 * a + c] * inv;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro,
                                               (int)(row_off + (db * 32 + 8 * a + 4 * b2) * ESZ),
                                               0, 0);
      }
  }
};

// ----------------------------------------------------------------- helpers

// Reduction over the two lanes that own one Q row (lane and lane ^ 32):
// v_permlane32_swap exchanges the wavefront halves in one VALU op.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Packed predicate select (§5.1): bit `pos` of the lane's word keeps the
// score, a 0 bit turns it into -inf.  sbfe yields 0 or all-ones.
__device__ inline float keep_or_neginf(float u, uint32_t word, int pos) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)word, pos, 1);
  return __uint_as_float((__float_as_uint(u) & m) | (~m & 0xFF800000u));
}

// score_mod in log2 units: returns log2(e) * mod(s * scale).  kq = k - q.
template <int MOD>
__device__ inline float mod_score(float s, float kq, const AttnParams& p, float slope) {
  if constexpr (MOD == kModAlibi) {
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

// Running softmax state of one lane (one Q row, shared with lane ^ 32).
struct RowState {
  float m;   // reference max (log2 units) used by the exponents so far
  float l;   // this lane's partial sum of the weights
};

// Softmax of one 32-row Q block over one K tile under a softcap score_mod,
// with the reference max taken from a bound instead of the scores: every
// softcapped score is at most c (log2 units: c2), plus, for softcap then
// ALiBi, the largest bias slope * (k - q) over the row's visible keys of the
// tile.  The row sees the key of that largest bias, whose score is at least
// -c2 plus the bias, so the row's true maximum is within 2 c2 of the bound,
// and with 2 c2 + kRescaleSlack <= 100 (cap_bounded) no weight that matters
// leaves the normal range.  Per score this leaves the cap's exponential and
// reciprocal, one FMA for the bias and one for the exponent, and the weight's
// exponential (MASKED: and the predicate's select): no maximum, no
// subtraction.  A full tile's bound comes from its last (or, for a negative
// slope, first) column; a partial tile's from the row's last (first) visible
// column, found from its predicate words -- the same column and the same
// arithmetic when the predicate is all ones, so a full tile run through the
// predicate path gives the same bits.  Lazy rescale and the exact zero skip
// work on the bound as on the maximum.
template <class Ops, int MOD, bool MASKED>
__device__ __attribute__((always_inline)) inline bool softmax_block_capped(
    const AttnParams& p, f32x16 (&acc)[Ops::NKB], const uint32_t (&mw)[Ops::NKB], float kq0,
    float slope, f32x16 (&o)[Ops::D / 32], RowState& rs, typename Ops::PBlock& pb) {
  constexpr int NKB = Ops::NKB, D = Ops::D;
  const float c2 = p.softcap_c2;
  float bound = c2;
  if constexpr (MOD == kModSoftcapAlibi) {
    // the lane's column of element v of block kk is kk*32 + 8(v/4) + v%4 past
    // kq0; its predicate bit sits at the same position of word kk
    int col;                                    // the lane's extreme visible column, or -1
    if constexpr (MASKED) {
      col = -1;
      if (slope > 0.0f) {
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) {
          const uint32_t m = mw[kk] & 0x0F0F0F0Fu;
          if (m) col = kk * 32 + 31 - __builtin_clz(m);
        }
      } else {
#pragma unroll
        for (int kk = NKB - 1; kk >= 0; --kk) {
          const uint32_t m = mw[kk] & 0x0F0F0F0Fu;
          if (m) col = kk * 32 + __builtin_ctz(m);
        }
      }
    } else {
      col = slope > 0.0f ? (NKB - 1) * 32 + 27 : 0;
    }
    const float bias = col < 0 ? kNegInf : slope * (kq0 + (float)col);
    bound = c2 + pair_max(bias);                // the row's two lanes agree
  }
  if (!p.no_skip && __builtin_amdgcn_ballot_w64(!(bound < rs.m - kNegligibleLog2)) == 0) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) acc[kk] = f32x16{};
    Ops::to_p(pb, acc);
    return false;
  }
  const bool bump = bound > rs.m + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(bump)) {
    const float alpha = bump ? exp2_fast(rs.m - bound) : 1.0f;
    rs.m = bump ? bound : rs.m;
    rs.l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
  }
  const float m2 = -2.0f * c2;
  if constexpr (MOD == kModSoftcap) {
    const float x = c2 - rs.m;
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = exp2_fast(acc[kk][v] * p.softcap_k);
        acc[kk][v] = exp2_fast(fmaf(m2, rcp_fast(1.0f + e), x));
      }
  } else if constexpr (MOD == kModSoftcapAlibi) {
    const float base = fmaf(slope, kq0, c2 - rs.m);
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float x = fmaf(slope, (float)(kk * 32 + 8 * (v / 4) + (v % 4)), base);
        const float e = exp2_fast(acc[kk][v] * p.softcap_k);
        acc[kk][v] = exp2_fast(fmaf(m2, rcp_fast(1.0f + e), x));
      }
  } else {   // ALiBi inside the cap: tanh of (s*scale + slope_h*(k-q)) / c
    const float x = c2 - rs.m, sb = slope * kq0;
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float t = fmaf(slope, (float)(kk * 32 + 8 * (v / 4) + (v % 4)), sb);
        const float e = exp2_fast(fmaf(acc[kk][v], p.softcap_k, t));
        acc[kk][v] = exp2_fast(fmaf(m2, rcp_fast(1.0f + e), x));
      }
  }
  if constexpr (MASKED) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t keep =
            (uint32_t)__builtin_amdgcn_sbfe((int)mw[kk], 8 * (v / 4) + v % 4, 1);
        acc[kk][v] = __uint_as_float(__float_as_uint(acc[kk][v]) & keep);
      }
  }
  Ops::to_p(pb, acc);
  rs.l += Ops::row_sum(pb, acc);
  return true;
}

// Softmax of one 32-row Q block over one K tile: score_mod and (MASKED) the
// predicate, online max with lazy rescale of the block's O, exponentials,
// P in the MFMA operand type and the row sum.  Returns false, with P zero and
// the state untouched, when every weight of the block would be exactly 0
// (all scores kNegligibleLog2 below the reference max, or all masked).
// CAPPED: a softcap score_mod's kernel takes its reference max from the
// scores' bound (softmax_block_capped).
template <class Ops, int MOD, bool MASKED, bool CAPPED>
__device__ __attribute__((always_inline)) inline bool softmax_block(const AttnParams& p, f32x16 (&acc)[Ops::NKB],
                                     const uint32_t (&mw)[Ops::NKB], float kq0, float slope,
                                     f32x16 (&o)[Ops::D / 32], RowState& rs,
                                     typename Ops::PBlock& pb) {
  constexpr int NKB = Ops::NKB, D = Ops::D;
  if constexpr (CAPPED)
    return softmax_block_capped<Ops, MOD, MASKED>(p, acc, mw, kq0, slope, o, rs, pb);
  // Without a score_mod the max is taken on the raw dot products (scale > 0)
  // and scaled once; the exponent is then one FMA per element.
  float mt = kNegInf;
  if constexpr (MOD == kModNone) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if constexpr (MASKED) acc[kk][v] = keep_or_neginf(acc[kk][v], mw[kk], 8 * (v / 4) + v % 4);
        mt = fmaxf(mt, acc[kk][v]);
      }
    mt = pair_max(mt) * p.scale_log2;
  } else {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float kq = kq0 + (float)(kk * 32 + 8 * (v / 4) + (v % 4));
        float u = mod_score<MOD>(acc[kk][v], kq, p, slope);
        if constexpr (MASKED) u = keep_or_neginf(u, mw[kk], 8 * (v / 4) + v % 4);
        acc[kk][v] = u;
        mt = fmaxf(mt, u);
      }
    mt = pair_max(mt);
  }
  // Only a predicate (a fully masked 32-row block) or an ALiBi bias (keys far
  // from the row) makes a whole block negligible often; elsewhere the check
  // is compiled out.
  constexpr bool kCheck = MASKED || MOD == kModAlibi || MOD == kModSoftcapAlibi ||
                          MOD == kModAlibiSoftcap;
  if constexpr (kCheck) {
    const bool negligible = mt == kNegInf || mt < rs.m - kNegligibleLog2;
    if (!p.no_skip && __builtin_amdgcn_ballot_w64(!negligible) == 0) {
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) acc[kk] = f32x16{};
      Ops::to_p(pb, acc);
      return false;
    }
  }
  // Lazy rescale: the reference max only moves when the row max grows by more
  // than kRescaleSlack, and the wavefront skips the O rescale if no lane
  // moved.  Both lanes of a row see the same mt, so they stay in step.
  const bool bump = mt > rs.m + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(bump)) {
    const float alpha = bump ? exp2_fast(rs.m - mt) : 1.0f;
    rs.m = bump ? mt : rs.m;
    rs.l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
  }
  const float m_use = rs.m == kNegInf ? 0.0f : rs.m;
  if constexpr (MOD == kModNone) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[kk][v] = exp2_fast(fmaf(acc[kk][v], p.scale_log2, -m_use));
  } else {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[kk][v] = exp2_fast(acc[kk][v] - m_use);
  }
  Ops::to_p(pb, acc);
  rs.l += Ops::row_sum(pb, acc);
  return true;
}

// One K tile for the wavefront's QB Q blocks: scores on MFMA, softmax per
// block, P.V on MFMA.  Tiles whose weights are all exactly 0 for this
// wavefront's rows are skipped: before the scores when the predicate hides
// the whole tile from them or the score_mod bounds the scores (softcap, then
// ALiBi: a score is at most the cap plus the tile's largest ALiBi bias), else
// after the scores.
template <class Ops, int MOD, bool MASKED, bool CAPPED>
__device__ __attribute__((always_inline)) inline void tile_step(const AttnParams& p, const typename Ops::QFrag& qf,
                                 const typename Ops::T* kst, const typename Ops::T* vst,
                                 int lane,
                                 const uint32_t (&mw)[Ops::QB][Ops::NKB],
                                 const float (&kq0)[Ops::QB], const float (&slope)[Ops::QB],
                                 f32x16 (&o)[Ops::QB][Ops::D / 32], RowState (&rs)[Ops::QB]) {
  constexpr int QB = Ops::QB, NKB = Ops::NKB, TKV = Ops::TKV;
  if constexpr (MASKED) {
    // no predicate bit set for any of this wavefront's rows: nothing visible
    uint32_t any_bit = 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) any_bit |= mw[qb][kk];
    if (!p.no_skip && __builtin_amdgcn_ballot_w64(any_bit != 0) == 0) return;
  }
  if constexpr (MOD == kModSoftcapAlibi) {
    bool need = p.no_skip != 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // the lane's row spans k - q in [kq0 - 4, kq0 + TKV) over this tile
      const float bias =
          fmaxf(slope[qb] * (kq0[qb] - 4.0f), slope[qb] * (kq0[qb] + (float)TKV));
      need |= !(p.softcap_c2 + bias < rs[qb].m - kNegligibleLog2);
    }
    if (__builtin_amdgcn_ballot_w64(need) == 0) return;
  }
  f32x16 acc[QB][NKB];
  // Wavefront priority: high while issuing MFMAs, low during the softmax, so
  // that of the wavefronts sharing a SIMD the one with matrix work issues
  // first and the other fills the VALU meanwhile.
  __builtin_amdgcn_s_setprio(1);
  Ops::qk(acc, qf, kst, lane);
  __builtin_amdgcn_s_setprio(0);
  typename Ops::PFrag pf;
  bool any = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
    any |= softmax_block<Ops, MOD, MASKED, CAPPED>(p, acc[qb], mw[qb], kq0[qb], slope[qb], o[qb],
                                                   rs[qb], pf.p[qb]);
  if (!any) return;
  __builtin_amdgcn_s_setprio(1);
  Ops::pv(o, pf, vst, lane);
  __builtin_amdgcn_s_setprio(0);
}

// Normalized fp32 O of one 32-row block (a Split-K partial state): lane
// stores four consecutive columns per 32-column group, as store_o does.
template <int D>
__device__ inline void store_o_f32(rsrc_t ro, uint32_t row_off, const f32x16 (&o)[D / 32],
                                   float inv, int b2) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 v;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = o[db][4 * a + c] * inv;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro,
                                             (int)(row_off + (db * 32 + 8 * a + 4 * b2) * 4), 0,
                                             0);
    }
}

// One task of the plan's launch order (or one Split-K part of it): the
// geometry and tile-list ranges of its record, scalar in every lane.
struct TaskCtx {
  int m_block, h, g, q_off, k_off, q_len, k_len;
  int p_beg, np, f_beg, ntiles, j_first;
  int split;
};

// Reads record blockIdx.x (SPLIT: record blockIdx.x % tasks_padded, part
// blockIdx.x / tasks_padded, cut to positions [s*n/S, (s+1)*n/S) of the
// list).  Returns false for the padding workgroups of a Split-K launch.
template <bool SPLIT>
__device__ inline bool read_task(const AttnParams& p, TaskCtx& c) {
  int task = blockIdx.x;
  c.split = 0;
  if constexpr (SPLIT) {
    c.split = blockIdx.x / p.tasks_padded;
    task = blockIdx.x - c.split * p.tasks_padded;
    if (task >= p.num_tasks) return false;   // padding of the last task row (whole workgroup)
  } else {
    if (p.dev_header) {   // deferred header: the plan's task count is on the device
      const int rows = __builtin_amdgcn_readfirstlane(p.dev_header[0]);
      const int err = __builtin_amdgcn_readfirstlane(p.dev_header[7]);
      if (err != 0 || task >= rows * p.task_heads) return false;
    }
  }
  const int32_t* rec = p.task_rec + (int64_t)task * kTaskRecInts;
  c.m_block = __builtin_amdgcn_readfirstlane(rec[kRecMBlock]);
  c.h = __builtin_amdgcn_readfirstlane(rec[kRecHead]);
  c.q_off = __builtin_amdgcn_readfirstlane(rec[kRecQOff]);
  c.k_off = __builtin_amdgcn_readfirstlane(rec[kRecKOff]);
  c.q_len = __builtin_amdgcn_readfirstlane(rec[kRecQLen]);
  c.k_len = __builtin_amdgcn_readfirstlane(rec[kRecKLen]);
  c.p_beg = __builtin_amdgcn_readfirstlane(rec[kRecPBeg]);
  c.np = __builtin_amdgcn_readfirstlane(rec[kRecPCnt]);
  c.f_beg = __builtin_amdgcn_readfirstlane(rec[kRecFBeg]);
  c.ntiles = c.np + __builtin_amdgcn_readfirstlane(rec[kRecFCnt]);
  c.j_first = __builtin_amdgcn_readfirstlane(rec[kRecFirstTile]);
  c.g = __builtin_amdgcn_readfirstlane(rec[kRecKvHead]);
  if constexpr (SPLIT) {
    // positions [t0, t1) of the list: partial positions [t0, min(t1, np)),
    // full positions [max(t0, np), t1)
    const int t0 = c.split * c.ntiles / p.num_splits;
    const int t1 = (c.split + 1) * c.ntiles / p.num_splits;
    const int f0 = t0 > c.np ? t0 : c.np;
    const int np_s = (t1 < c.np ? t1 : c.np) - t0;
    c.p_beg += t0;
    c.f_beg += f0 - c.np;
    c.np = np_s > 0 ? np_s : 0;
    c.ntiles = t1 - t0;
    c.j_first = __builtin_amdgcn_readfirstlane(
        c.ntiles == 0 ? -1 : (c.np > 0 ? p.p_idx[c.p_beg] : p.f_idx[c.f_beg]));
  }
  return true;
}

// Buffer descriptor of pool tile `phys` holding logical K tile j of a paged
// sample: it covers only the rows below the sample's k_len, so loads past it
// read zero as in the contiguous case; an unmapped entry (phys < 0) gets an
// empty descriptor, its rows read zero.
template <int TKV>
__device__ inline rsrc_t paged_tile_rsrc(const char* pool, int j, int phys, int k_len,
                                         uint32_t kv_rs) {
  const int rows = k_len - j * TKV;
  const uint32_t n = phys < 0 ? 0u : (uint32_t)(rows < TKV ? rows : TKV) * kv_rs;
  return make_rsrc(pool + (int64_t)(phys < 0 ? 0 : phys) * TKV * kv_rs, n);
}

// Epilogue of a task: O = acc / l, LSE = m + ln l (natural log); empty rows
// get 0 / -inf.  Rows past q_len are dropped by the O descriptor's range
// check.  A Split-K part writes the same for its tiles, in fp32, into its
// partial-state slice.
// hq0 is the task's first Q head, hs the lane's head within the task
// (PackGQA; 0 when unpacked).
template <class Ops, bool SPLIT>
__device__ inline void write_rows(const AttnParams& p, const TaskCtx& c, rsrc_t ro, int hq0,
                                  const uint32_t (&q_row_off)[Ops::QB], const int (&qloc)[Ops::QB],
                                  const int (&hs)[Ops::QB],
                                  const f32x16 (&o)[Ops::QB][Ops::D / 32],
                                  const RowState (&rs)[Ops::QB], int b2) {
  constexpr int D = Ops::D;
  rsrc_t rout = ro;
  float* lse_out = p.lse;
  if constexpr (SPLIT) {
    const int64_t fq_rs = (int64_t)p.heads_q * D;   // floats per token row
    float* ob = p.o_part + (int64_t)c.split * p.total_q * fq_rs + (int64_t)c.q_off * fq_rs +
                (int64_t)hq0 * D;
    rout = make_rsrc(ob, (uint32_t)(c.q_len * fq_rs * 4));
    lse_out = p.lse_part + (int64_t)c.split * p.heads_q * p.total_q;
  }
#pragma unroll
  for (int qb = 0; qb < Ops::QB; ++qb) {
    const float l_tot = pair_sum(rs[qb].l);
    const float inv = l_tot > 0.0f ? rcp_fast(l_tot) : 0.0f;
    if constexpr (SPLIT)
      store_o_f32<D>(rout, ((uint32_t)qloc[qb] * p.heads_q + hs[qb]) * D * 4, o[qb], inv, b2);
    else
      Ops::store_o(rout, q_row_off[qb], o[qb], inv, b2);
    if (b2 == 0 && qloc[qb] < c.q_len) {
      lse_out[(int64_t)(hq0 + hs[qb]) * p.total_q + c.q_off + qloc[qb]] =
          l_tot > 0.0f ? (rs[qb].m + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
    }
  }
}

// One workgroup per task, in the plan's launch order (record blockIdx.x).
// SPLIT: one workgroup per (split, task), the splits of the Tessera page's
// Split-K: workgroup i runs split i / tasks_padded of task i % tasks_padded
// over a contiguous part of the task's tile list and writes its partial state.
// PAGED: K and V are page pools addressed through the remapped tile lists.
template <class Ops, int MOD, bool SPLIT, bool PAGED, bool CAPPED>
__global__ __launch_bounds__(Ops::NT) __attribute__((amdgpu_waves_per_eu(Ops::WPE, Ops::WPE)))
void attn_fwd_kernel(AttnParams p) {
  constexpr int D = Ops::D, TQ = Ops::TQ, TKV = Ops::TKV, NKB = Ops::NKB, ESZ = Ops::ESZ;
  constexpr int QB = Ops::QB;
  using T = typename Ops::T;
  // One LDS array per stage and operand, each a separate object: the compiler
  // then knows that the loads landing in the next stage's buffers cannot
  // alias this stage's operand reads and does not wait for them.
  __shared__ __attribute__((aligned(16))) T k_s0[Ops::KELEMS];
  __shared__ __attribute__((aligned(16))) T k_s1[Ops::KELEMS];
  __shared__ __attribute__((aligned(16))) T v_s0[Ops::VELEMS];
  __shared__ __attribute__((aligned(16))) T v_s1[Ops::VELEMS];
  // A stage is an int or, where the loop is unrolled, a compile-time constant.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto kbuf = [&](auto st) -> T* {
    if constexpr (std::is_integral_v<decltype(st)>) return st ? k_s1 : k_s0;
    else if constexpr (decltype(st)::value == 0) return k_s0;
    else return k_s1;
  };
  auto vbuf = [&](auto st) -> T* {
    if constexpr (std::is_integral_v<decltype(st)>) return st ? v_s1 : v_s0;
    else if constexpr (decltype(st)::value == 0) return v_s0;
    else return v_s1;
  };
  auto flip = [](auto st) {
    if constexpr (std::is_integral_v<decltype(st)>) return st ^ 1;
    else return std::integral_constant<int, decltype(st)::value ^ 1>{};
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b2 = lane >> 5;
  const int lq = lane & 31;

  TaskCtx c;
  if (!read_task<SPLIT>(p, c)) return;
  const int m_block = c.m_block, h = c.h, g = c.g, q_off = c.q_off, k_off = c.k_off;
  const int q_len = c.q_len, k_len = c.k_len;
  const int p_beg = c.p_beg, np = c.np, f_beg = c.f_beg, ntiles = c.ntiles;
  const int j_first = c.j_first;
  // PackGQA: the task covers Q heads [hq0, hq0 + 2^psh) (the task head is
  // the K/V head) and TQ >> psh tokens; tile row r is token r >> psh, head
  // hq0 + (r & (2^psh - 1)).  Unpacked: psh = 0, hq0 = h.
  const int psh = p.pack_shift;
  const int hq0 = h << psh;

  const uint32_t q_rs = (uint32_t)p.heads_q * D * ESZ;   // bytes per Q/O token row
  const uint32_t kv_rs = (uint32_t)p.heads_k * D * ESZ;  // bytes per K/V token row
  // Sample-bounded views: [q_off, q_off+q_len) rows from head hq0 on in Q
  // and O, [k_off, k_off+k_len) rows of K/V head g.
  const char* qbase = (const char*)p.q + (int64_t)q_off * q_rs + (int64_t)hq0 * D * ESZ;
  char* obase = (char*)p.o + (int64_t)q_off * q_rs + (int64_t)hq0 * D * ESZ;
  const char* kbase = (const char*)p.k + (int64_t)k_off * kv_rs + (int64_t)g * D * ESZ;
  const char* vbase = (const char*)p.v + (int64_t)k_off * kv_rs + (int64_t)g * D * ESZ;
  const rsrc_t rq = make_rsrc(qbase, (uint32_t)q_len * q_rs);
  const rsrc_t ro = make_rsrc(obase, (uint32_t)q_len * q_rs);
  const rsrc_t rk = make_rsrc(kbase, (uint32_t)k_len * kv_rs);
  const rsrc_t rv = make_rsrc(vbase, (uint32_t)k_len * kv_rs);
  // Paged K/V: tile t's rows live in pool tile phys (tile_k rows of the pool,
  // starting at row phys * TKV).
  const char* kpool = (const char*)p.k + (int64_t)g * D * ESZ;
  const char* vpool = (const char*)p.v + (int64_t)g * D * ESZ;
  auto tile_rsrc = [&](const char* pool, int j, int phys) {
    return paged_tile_rsrc<TKV>(pool, j, phys, k_len, kv_rs);
  };
  // bf16 tiles go straight to LDS: each lane's offsets within a tile are
  // fixed for the task and the tile's own offset is folded into a
  // descriptor built on the scalar unit (listed tiles start below k_len)
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t kv_bytes = (uint32_t)k_len * kv_rs;
  uint32_t koff[Ops::KI], voff[Ops::KI];
  if constexpr (Ops::kDirectLds) {
#pragma unroll
    for (int i = 0; i < Ops::KI; ++i) {
      koff[i] = Ops::lane_off(0, i, wave_u, tid & 63, kv_rs);
      voff[i] = Ops::lane_off(1, i, wave_u, tid & 63, kv_rs);
    }
  }
  auto load_tile = [&](typename Ops::Stage& stg, T* kd, T* vd, int j, int phys)
      __attribute__((always_inline)) {
    if constexpr (Ops::kDirectLds) {
      const uint32_t off = (uint32_t)j * TKV * kv_rs;
      const rsrc_t a = PAGED ? tile_rsrc(kpool, j, phys) : make_rsrc(kbase + off, kv_bytes - off);
      const rsrc_t b = PAGED ? tile_rsrc(vpool, j, phys) : make_rsrc(vbase + off, kv_bytes - off);
      Ops::load_op(kd, a, koff, wave_u);
      Ops::load_op(vd, b, voff, wave_u);
    } else if constexpr (PAGED) {
      Ops::load(stg, kd, vd, tile_rsrc(kpool, j, phys), tile_rsrc(vpool, j, phys), 0u, kv_rs, tid);
    } else {
      Ops::load(stg, kd, vd, rk, rv, (uint32_t)j * TKV * kv_rs, kv_rs, tid);
    }
  };

  // Sample-local Q token (qloc), head within the task (hs) and payload word
  // row (prow) of this lane's tile row in each of the wavefront's blocks.
  int qloc[QB], hs[QB], prow[QB];
  uint32_t q_row_off[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = 32 * (QB * wave + qb) + lq;
    prow[qb] = r >> psh;
    hs[qb] = r & ((1 << psh) - 1);
    qloc[qb] = m_block * (TQ >> psh) + prow[qb];
    q_row_off[qb] = (uint32_t)qloc[qb] * q_rs + (uint32_t)hs[qb] * D * ESZ;
  }
  const int tq_plan = TQ >> psh;   // payload word rows per partial tile

  // Tile t of the task: the partial list first, then the full list (§6.1);
  // without ALiBi (whose bias peaks where the partial tiles are) the full
  // list first, so that the tasks of a (sample, head) begin on the tiles they
  // share (window + sink: the sink tile, an L2 hit) rather than on a tile of
  // their own.  Split-K parts keep the plan's order (their ranges are cut
  // from it).
  constexpr bool kFullFirst = !SPLIT && (MOD == kModNone || MOD == kModSoftcap);
  const int nf = ntiles - np;
  auto is_partial = [&](int t) { return kFullFirst ? t >= nf : t < np; };
  auto list_pos = [&](int t) {   // position in the partial or the full list
    return kFullFirst ? (t < nf ? f_beg + t : p_beg + t - nf)
                      : (t < np ? p_beg + t : f_beg + t - np);
  };
  auto tile_j = [&](int t) {
    return __builtin_amdgcn_readfirstlane(is_partial(t) ? p.p_idx[list_pos(t)]
                                                        : p.f_idx[list_pos(t)]);
  };
  auto tile_phys = [&](int t) {
    return __builtin_amdgcn_readfirstlane(is_partial(t) ? p.phys_p[list_pos(t)]
                                                        : p.phys_f[list_pos(t)]);
  };
  auto load_masks = [&](int t, uint32_t (&mw)[QB][NKB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (is_partial(t)) {
        const uint32_t* src = p.p_masks + ((int64_t)list_pos(t) * tq_plan + prow[qb]) * NKB;
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) mw[qb][kk] = src[kk];
      } else {
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) mw[qb][kk] = 0xFFFFFFFFu;
      }
    }
  };

  typename Ops::Stage st;
  uint32_t mw_cur[QB][NKB], mw_next[QB][NKB];
  // (the record's first tile is the first listed one, partial first)
  int j_cur = kFullFirst && ntiles > 0 && nf > 0 && np > 0 ? tile_j(0) : j_first;
  // K-tile index of tile t+1, read one tile ahead of its use so that no
  // tile waits on the index load before issuing its prefetch.
  int j_ahead = 0, ph_ahead = 0;
  if (ntiles > 0) {
    load_tile(st, k_s0, v_s0, j_cur, PAGED ? tile_phys(0) : 0);
    load_masks(0, mw_cur);
    if (ntiles > 1) {
      j_ahead = tile_j(1);
      if constexpr (PAGED) ph_ahead = tile_phys(1);
    }
  }
  typename Ops::QFrag qf;
  Ops::load_q(qf, rq, q_row_off, b2);

  float slope[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    slope[qb] = 0.0f;
    if constexpr (MOD == kModAlibi || MOD == kModSoftcapAlibi)
      slope[qb] = p.slopes[hq0 + hs[qb]] * kLog2e;
    if constexpr (MOD == kModAlibiSoftcap) slope[qb] = p.slopes[hq0 + hs[qb]] * p.alibi_k;
  }

  f32x16 o[QB][D / 32];
  RowState rs[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[qb][db] = f32x16{};
    rs[qb] = RowState{kNegInf, 0.0f};
  }

  // Two loops, as in §6.1: the partial list with its predicate, then the full
  // list without one.  The K/V prefetch runs one tile ahead across both, the
  // tile-index read two tiles ahead.  Tile t uses stage t % 2; with tiles
  // loaded straight into LDS the stage is a compile-time constant in every
  // step (the loops step two tiles at a time).
  int t = 0;
  int j_pending = 0;   // index of tile t+2, in flight during tile t
  int ph_pending = 0;  // its pool tile (paged K/V)
  auto step = [&](auto masked, auto stage) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
    const auto next = flip(stage);
    const bool more = t + 1 < ntiles;
    const int j_next = j_ahead;
    if (more) {
      load_tile(st, kbuf(next), vbuf(next), j_next, ph_ahead);
      load_masks(t + 1, mw_next);
    }
    if (t + 2 < ntiles) {
      j_pending = is_partial(t + 2) ? p.p_idx[list_pos(t + 2)] : p.f_idx[list_pos(t + 2)];
      if constexpr (PAGED)
        ph_pending = is_partial(t + 2) ? p.phys_p[list_pos(t + 2)] : p.phys_f[list_pos(t + 2)];
    }
    float kq0[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) kq0[qb] = (float)(j_cur * TKV + 4 * b2 - qloc[qb]);
    tile_step<Ops, MOD, kMasked, CAPPED>(p, qf, kbuf(stage), vbuf(stage), lane, mw_cur, kq0, slope,
                                         o, rs);
    if (more) {
      Ops::store(st, kbuf(next), vbuf(next), tid);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) mw_cur[qb][kk] = mw_next[qb][kk] >> (4 * b2);
      j_cur = j_next;
    }
    // this wavefront's loads straight into LDS have landed; the barrier
    // publishes them and the stores above to the whole workgroup
    __builtin_amdgcn_s_waitcnt(0);
    if (t + 2 < ntiles) {
      j_ahead = __builtin_amdgcn_readfirstlane(j_pending);
      if constexpr (PAGED) ph_ahead = __builtin_amdgcn_readfirstlane(ph_pending);
    }
    __syncthreads();
    ++t;
  };
  // tiles [t, t_end) with the predicate or without it
  auto run = [&](auto masked, int t_end) __attribute__((always_inline)) {
    if constexpr (Ops::kDirectLds) {
      if (t < t_end && (t & 1)) step(masked, S1{});
      while (t + 1 < t_end) {
        step(masked, S0{});
        step(masked, S1{});
      }
      if (t < t_end) step(masked, S0{});
    } else {
      while (t < t_end) step(masked, t & 1);
    }
  };
  if (ntiles > 0) {
    Ops::store(st, k_s0, v_s0, tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // mask words are kept as loaded until their tile starts (a shift right at
    // the load would make it wait for every load in flight); lanes 32..63 hold
    // the columns 4 above those of lanes 0..31
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) mw_cur[qb][kk] >>= 4 * b2;
    if constexpr (kFullFirst) {
      if (p.force_partial) {
        run(std::true_type{}, ntiles);
      } else {
        run(std::false_type{}, nf);
        run(std::true_type{}, ntiles);
      }
    } else {
      run(std::true_type{}, p.force_partial ? ntiles : np);
      run(std::false_type{}, ntiles);
    }
  }

  write_rows<Ops, SPLIT>(p, c, ro, hq0, q_row_off, qloc, hs, o, rs, b2);
}

// Page-table remap of the plan's K-tile lists (FlexAttention page, paged
// attention: the page table is folded into the block indices, physical =
// page_table[batch][logical]): one wavefront per flat mask row finds the
// row's sample, then its lanes map every listed K tile j to the pool tile
// page * (page_size / tile_k) + (j * tile_k mod page_size) / tile_k, or -1
// when the page entry is outside [0, num_pages).
__global__ __launch_bounds__(256) void page_remap_kernel(RemapParams p) {
  const int flat = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (flat >= p.rows_flat) return;
  const int r = flat % p.rows_total;
  // sample b with cu_rows[b] <= r < cu_rows[b+1] (largest such b)
  int lo = 0, hi = p.batch;              // invariant: cu_rows[lo] <= r < cu_rows[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.cu_rows[mid] <= r) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int tiles_per_page = p.page_size / p.tile_k;
  const int32_t* pt = p.page_table + (int64_t)b * p.pages_per_seq;
  auto map = [&](int j) {
    const int lp = j / tiles_per_page;
    if (lp >= p.pages_per_seq) return -1;
    const int pg = pt[lp];
    if (pg < 0 || pg >= p.num_pages) return -1;
    return pg * tiles_per_page + (j - lp * tiles_per_page);
  };
  for (int e = p.p_off[flat] + lane; e < p.p_off[flat + 1]; e += 64) p.phys_p[e] = map(p.p_idx[e]);
  for (int e = p.f_off[flat] + lane; e < p.f_off[flat + 1]; e += 64) p.phys_f[e] = map(p.f_idx[e]);
}

// Merge of Split-K partial states (Tessera page, "Split-K"): per (token, head)
// row, LSE = M + ln sum_s exp(L_s - M) with M = max_s L_s, and
// O = sum_s exp(L_s - LSE) O_s; parts with L_s = -inf are not read; a row
// with every part empty gets O = 0, LSE = -inf.  D/8 lanes per row, eight
// columns each (two 16-byte loads per part); HBM-bound.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (row >= p.rows) return;
  const int64_t tok = row / p.heads_q;
  const int h = (int)(row - tok * p.heads_q);
  const int64_t lstride = (int64_t)p.heads_q * p.total_q;
  const float* lp = p.lse_part + (int64_t)h * p.total_q + tok;
  float m = kNegInf;
  for (int s = 0; s < p.parts; ++s) m = fmaxf(m, lp[s * lstride]);
  float acc[8] = {};
  float lsum = 0.0f;
  if (m != kNegInf) {
    const int64_t ostride = p.rows * D;
    const float* op = p.o_part + row * D + c * 8;
    for (int s = 0; s < p.parts; ++s) {
      const float ls = lp[s * lstride];
      if (ls == kNegInf) continue;
      const float w = exp2_fast((ls - m) * kLog2e);
      lsum += w;
      const f32x4 x0 = *(const f32x4*)(op + s * ostride);
      const f32x4 x1 = *(const f32x4*)(op + s * ostride + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(w, x0[e], acc[e]);
        acc[4 + e] = fmaf(w, x1[e], acc[4 + e]);
      }
    }
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
  }
  OutT* out = (OutT*)p.o + row * D + c * 8;
  if constexpr (std::is_same_v<OutT, float>) {
    *(f32x4*)out = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)(out + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)acc[e];
    *(bf16x8*)out = v;
  }
  if (c == 0) p.lse[(int64_t)h * p.total_q + tok] = m == kNegInf ? kNegInf : m + logf(lsum);
}

// ----------------------------------------------------------------- dispatch

template <class Ops, bool SPLIT, bool PAGED>
hipError_t launch_mods(int mod, int num_blocks, const AttnParams& p, hipStream_t s) {
  const dim3 g(num_blocks), blk(Ops::NT);
  auto go = [&](auto m) {
    hipLaunchKernelGGL((attn_fwd_kernel<Ops, decltype(m)::value, SPLIT, PAGED, false>), g, blk, 0,
                       s, p);
    return hipGetLastError();
  };
  // softcap score_mods: the bound-max kernel where the cap allows it
  auto go_cap = [&](auto m) {
    if (!p.cap_bounded) return go(m);
    hipLaunchKernelGGL((attn_fwd_kernel<Ops, decltype(m)::value, SPLIT, PAGED, true>), g, blk, 0,
                       s, p);
    return hipGetLastError();
  };
  switch (mod) {
    case kModNone: return go(std::integral_constant<int, kModNone>{});
    case kModSoftcap: return go_cap(std::integral_constant<int, kModSoftcap>{});
    case kModAlibi: return go(std::integral_constant<int, kModAlibi>{});
    case kModSoftcapAlibi: return go_cap(std::integral_constant<int, kModSoftcapAlibi>{});
    case kModAlibiSoftcap: return go_cap(std::integral_constant<int, kModAlibiSoftcap>{});
    default: return hipErrorInvalidValue;
  }
}

// Paged K/V kernels exist for the bf16 consumers only.
template <class Ops, bool SPLIT>
hipError_t launch_ops(int mod, int num_blocks, const AttnParams& p, hipStream_t s) {
  if (p.paged) {
    if constexpr (std::is_same_v<typename Ops::T, __bf16>)
      return launch_mods<Ops, SPLIT, true>(mod, num_blocks, p, s);
    else
      return hipErrorInvalidValue;
  }
  return launch_mods<Ops, SPLIT, false>(mod, num_blocks, p, s);
}

// The consumer table: (dtype, head_dim, tile_q, tile_k) -> kernel family.
#define MPB_VARIANTS(X)                         \
  X(MPB_DTYPE_BF16, 128, 128, 64, Bf16Ops<128, 4, 64, 1>) \
  X(MPB_DTYPE_BF16, 128, 64, 64, Bf16Ops<128, 2, 64, 1>)  \
  X(MPB_DTYPE_BF16, 128, 128, 32, Bf16Ops<128, 4, 32, 1>) \
  X(MPB_DTYPE_BF16, 128, 64, 32, Bf16Ops<128, 2, 32, 1>)  \
  X(MPB_DTYPE_BF16, 64, 128, 64, Bf16Ops<64, 4, 64, 1>)   \
  X(MPB_DTYPE_BF16, 64, 64, 64, Bf16Ops<64, 2, 64, 1>)    \
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
                           int32_t mod_kind, int32_t num_tasks, const AttnParams& p,
                           hipStream_t s) {
#define X(DT, HD, TQ_, TK_, ...) \
  if (dtype == DT && head_dim == HD && tile_q == TQ_ && tile_k == TK_) return launch_ops<__VA_ARGS__, false>(mod_kind, num_tasks, p, s);
  MPB_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_split(int32_t dtype, int32_t head_dim, int32_t tile_q, int32_t tile_k,
                                 int32_t mod_kind, const AttnParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.num_splits * p.tasks_padded;
  if (p.num_splits < 1 || p.tasks_padded < p.num_tasks || blocks > 0x7FFFFFFF)
    return hipErrorInvalidValue;
#define X(DT, HD, TQ_, TK_, ...) \
  if (dtype == DT && head_dim == HD && tile_q == TQ_ && tile_k == TK_) return launch_ops<__VA_ARGS__, true>(mod_kind, (int)blocks, p, s);
  MPB_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_page_remap(const RemapParams& p, hipStream_t s) {
  if (p.rows_flat == 0) return hipSuccess;
  hipLaunchKernelGGL(page_remap_kernel, dim3((p.rows_flat + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_merge(int32_t dtype, int32_t head_dim, const MergeParams& p,
                             hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const int rpb = 256 / (head_dim / 8);
  const int64_t blocks = (p.rows + rpb - 1) / rpb;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), blk(256);
  if (dtype == MPB_DTYPE_BF16 && head_dim == 128)
    hipLaunchKernelGGL((attn_merge_kernel<128, __bf16>), g, blk, 0, s, p);
  else if (dtype == MPB_DTYPE_BF16 && head_dim == 64)
    hipLaunchKernelGGL((attn_merge_kernel<64, __bf16>), g, blk, 0, s, p);
  else if (dtype == MPB_DTYPE_FP32 && head_dim == 128)
    hipLaunchKernelGGL((attn_merge_kernel<128, float>), g, blk, 0, s, p);
  else if (dtype == MPB_DTYPE_FP32 && head_dim == 64)
    hipLaunchKernelGGL((attn_merge_kernel<64, float>), g, blk, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mpb
