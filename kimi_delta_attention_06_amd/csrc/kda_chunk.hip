// Chunkwise-parallel KDA forward for gfx950 (MI355X).
//
// KDA is computed chunk-wise: parallel inside a chunk of C tokens, recurrent
// across chunks ("Kimi K3 technical report summary", section 1, pre-training
// table, KDA row).  The per-token transition (I - b k k^T) Diag(a) is diagonal
// plus rank one, so a chunk folds into a WY/UT form ("DPLR chunk kernel",
// "Kimi K3 NPU Training", section "NPU operator support").  For one chunk with
// entering state S, rows r = 0..C-1 and per-channel cumulative log-decay
// g_r = sum_{i<=r} log a_i (the algebra follows from unrolling the recurrence):
//
//   A[r,i] = b_r sum_c k_rc k_ic e^{g_rc - g_ic}   (i < r)      key Gram, decay-scaled
//   M[r,i] =     sum_c q_rc k_ic e^{g_rc - g_ic}   (i <= r)     query-key Gram
//   T      = (I + A)^-1                                         UT lower-triangular inverse
//   U      = T Diag(b) (V - (K * e^G) S)                        pseudo-values
//   O      = (Q * e^G) S + M U
//   S     <- Diag(e^{g_last}) S + (K * e^{g_last - G})^T U
//
// U equals the WY form T Diag(b) V - (T Diag(b) (K * e^G)) S; with the entering state at
// hand the pseudo-key product T Diag(b) (K * e^G) is never formed, and (K * e^G) S does
// not wait for T, so it runs beside the inverse.
//
// One workgroup (512 threads, 8 waves, one per CU) owns one (sequence, head,
// tile of BV value columns) and walks that sequence's chunks in order, resetting
// the state at the sequence start (packed-sequence state reset, "Kimi K3 NPU
// Training", section "TND is not a layout switch", item 2).  The fp32 master
// state lives in MFMA accumulator registers; a 16-bit copy in LDS feeds the
// next chunk's matrix products.  The next chunk's inputs are loaded into
// registers while the current chunk is computed, in three groups issued after
// different barriers (a single burst stalls instruction issue on the CU's memory
// pipeline), and the next chunk's gate stage (part a) runs at the end of the
// current iteration, so no loaded register is live across the loop back-edge.
//
// Gate stage in matrix-core layout.  Waves (R, p) own 16-row sub-block R and
// half p of the key channels; lane l holds token 16R + (l & 15) and DK/8
// consecutive channels.  That is the MFMA operand layout of the Gram products
// (the channel order inside a k-step is the same permutation for both
// operands), so the 16x16 diagonal sub-blocks of A and M are formed from
// registers; the in-block cumulative decay is a DPP scan across the 16 lanes
// of a row.  Each channel half gives a partial Gram tile; the two are summed
// through LDS.
//
// Overflow-safe decay.  With c the in-block cumulative decay and s the block
// total (both <= 0) every operand is a value times an exponential:
//   * diagonal sub-block R: left X_r e^{c_r - s/2}, right k_i e^{s/2 - c_i},
//     each bounded by e^{|s|/2}: finite while a 16-token block decays by less
//     than ~170 nats per channel (the documented precondition);
//   * sub-block pair R > I: left X_r e^{c_r} e^{G_{R-1} - G_I}, right
//     k_i e^{s_I - c_i}, all <= 1 (G_J: cumulative decay at the end of block J).
// Entries above the diagonal are removed with a select, never a multiply.
//
// Precision policies:
//   Mixed (bf16 inputs): fp16 MFMA operands.  The diagonal Gram sub-blocks use fp16
//     too when every channel of the wave decays by less than 8 nats over the 16-token
//     block (the balanced operands then stay within e^{+-4} of the inputs); otherwise
//     A's are bf16 (range) and M's go on the fp32 matrix core (range and precision).
//     The diagonal of M (q_r . k_r) multiplies U in fp32 outside the MFMA.
//   F32 (fp32 inputs): every product on the fp32 MFMA (16x16x4).
#include <atomic>
#include <type_traits>

#include "kda_common.hpp"
#include "kda_launch.hpp"

// The host code below is in two parts, each built into its own object so that each
// can take its own instruction-scheduling flags: the fused forward (every PREP = false
// instantiation) and the split path (the in-chunk, pipelined and state passes).  A
// plain compile builds both.
#ifndef KDA_CHUNK_FUSED
#define KDA_CHUNK_FUSED 1
#endif
#ifndef KDA_CHUNK_SPLIT
#define KDA_CHUNK_SPLIT 1
#endif

namespace kda {
namespace chunkk {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 8;
static_assert((NW & (NW - 1)) == 0, "wave indices are masked with NW - 1");
constexpr int NT = NW * kWave;

enum class Prec { Mixed, F32 };

template <Prec P> struct Op;
template <> struct Op<Prec::Mixed> {
  using T = _Float16;
  static constexpr int KS = 32, PAD = 8;
};
template <> struct Op<Prec::F32> {
  using T = float;
  static constexpr int KS = 16, PAD = 4;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <typename T> __device__ __forceinline__ T cvt(float x);
template <> __device__ __forceinline__ _Float16 cvt<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ float cvt<float>(float x) { return x; }

__device__ __forceinline__ void store4(_Float16* p, float a, float b, float c, float d) {
  *reinterpret_cast<half4*>(p) = half4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ float4 load4(const _Float16* p) {
  const half4 h = *reinterpret_cast<const half4*>(p);
  return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
}
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// One lane's operand fragment of one MMA k-step, loaded from LDS.
__device__ __forceinline__ half8 ld_frag(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }
__device__ __forceinline__ float4 ld_frag(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void mma_frag(f32x4& acc, const half8& a, const half8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_frag(f32x4& acc, const float4& a, const float4& b) {
  // four fp32 MFMAs on k = 4*(lane>>4) + j: the same k permutation for A and B
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
}
// One MMA step from LDS operands: `a`, `b` point at the lane's first k element.
template <typename T>
__device__ __forceinline__ void mma_step(f32x4& acc, const T* a, const T* b) {
  mma_frag(acc, ld_frag(a), ld_frag(b));
}

// acc (+)= A[16 rows, K] * B[16 rows, K]^T, both row-major with k contiguous, K = NST*KS.
template <typename T, int KS, int NST>
__device__ __forceinline__ void mma_lds(f32x4& acc, const T* A, int lda, const T* B, int ldb) {
  const int l = lane_id();
  const T* a = A + (l & 15) * lda + (l >> 4) * (KS / 4);
  const T* b = B + (l & 15) * ldb + (l >> 4) * (KS / 4);
#pragma unroll
  for (int s = 0; s < NST; ++s) mma_step(acc, a + s * KS, b + s * KS);
}

// f(std::integral_constant<int, I>{}) for I = B .. E-1, each I a compile-time constant
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// every lane of a 16-lane row receives lane N of that row (DPP row_newbcast).  Every lane is
// written, so the move takes no old value (update_dpp with an old value of 0 made the
// compiler set each destination to 0 first: one extra move per broadcast).
template <int N>
__device__ __forceinline__ float row_bcast16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, false));
}


// lane i of each 16-lane row receives lane i - N (0 for i < N): a step of the row scan
template <int N>
__device__ __forceinline__ float shr16(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | N, 0xf, 0xf, false));
}
__device__ __forceinline__ float scan16(float x) {
  x += shr16<1>(x);
  x += shr16<2>(x);
  x += shr16<4>(x);
  x += shr16<8>(x);
  return x;
}

constexpr size_t al16(size_t x) { return (x + 15) & ~size_t(15); }
constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// In log2 units: the balanced factors of a diagonal 16-token sub-block stay finite in fp32
// while the block decays by at most 160 nats in every channel (see the gate stage).
constexpr float kBalancedLimit = -230.83f;  // -160 nats
// Per-token decay floor for the exact path, log2 units (about -111 nats): 2^-160 is 0 in fp32,
// like 2^x for every x below it, so the floor changes nothing an fp32 recurrence can represent;
// it keeps sums of 16 steps finite for any finite log alpha, and small enough that differences
// of nearby sums keep their precision.
constexpr float kStepFloor = -160.f;

// Exact diagonal Gram sub-block for one channel part, for blocks whose decay is too wide for
// the balanced factorisation.  Lane (column token i = lr, channel group lg) holds its token's q,
// k and in-block cumulative decay cx (log2 units) for GC channels; every entry
// X[r][i] = sum_c x_rc k_ic 2^{cx_rc - cx_ic} (i <= r) has a factor <= 1.  Row r's values come
// from lane r of the same 16-lane row (same channels) by a DPP broadcast; the four channel
// groups are then summed across rows, and each lane adds rows 4 lg .. 4 lg + 3 of column lr to
// its accumulators (the 16x16 MFMA accumulator layout).  Rows go in two halves of 8 to bound
// the live registers.
template <int GC>
__device__ __forceinline__ void gram_exact(const float* q, const float* k, const float* cx, int lr, int lg,
                                           f32x4& accM, f32x4& accA) {
  static_for<0, 2>([&](auto hc) {
    constexpr int r0 = 8 * decltype(hc)::value;
    float pm[8], pa[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) pm[r] = pa[r] = 0.f;
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      const float ci = cx[j], ki = k[j];
      static_for<0, 8>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const float cr = row_bcast16<r0 + r>(cx[j]);
        const float qr = row_bcast16<r0 + r>(q[j]);
        const float kr = row_bcast16<r0 + r>(k[j]);
        // r == lr gives cr - ci = 0 exactly; entries above the diagonal are selected away
        const float t = (r0 + r >= lr) ? ki * __builtin_amdgcn_exp2f(cr - ci) : 0.f;
        pm[r] = fmaf(qr, t, pm[r]);
        pa[r] = fmaf(kr, t, pa[r]);
      });
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      pm[r] += __shfl_xor(pm[r], 16, kWave);
      pm[r] += __shfl_xor(pm[r], 32, kWave);
      pa[r] += __shfl_xor(pa[r], 16, kWave);
      pa[r] += __shfl_xor(pa[r], 32, kWave);
    }
    // lanes of groups 2 hc and 2 hc + 1 own rows r0 .. r0 + 3 and r0 + 4 .. r0 + 7
    const bool lo = lg == 2 * decltype(hc)::value, hi = lg == 2 * decltype(hc)::value + 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      accM[u] += lo ? pm[u] : (hi ? pm[4 + u] : 0.f);
      accA[u] += lo ? pa[u] : (hi ? pa[4 + u] : 0.f);
    }
  });
}

// ---------------------------------------------------------------------------
// Range of the 16-bit state-step operands.  The state S and the values V enter the fp16
// matrix products of a chunk (Y = V - Kg S, U = T Diag(b) Y, O = Qg S + M U, S' = g S + Kd^T U),
// all linear in (V, S) jointly; a chunk whose largest |S| or |V| is outside [2^-6, 2^6) is
// computed on copies scaled by a power of two 2^-e that brings it into [2^4, 2^5), and its o
// and state update are scaled back by 2^e (exact in fp32).  So any finite v and h0 are taken,
// and tiny ones keep their precision instead of flushing in fp16.
// ---------------------------------------------------------------------------
// |x| as a bit pattern: ordered like the magnitudes (NaN above inf above every finite value)
__device__ __forceinline__ uint32_t mag_bits(float x) { return __float_as_uint(x) << 1; }
// The largest mag_bits over fp32 values: the signed maximum of the raw patterns is the largest
// non-negative value (if any), the unsigned maximum the negative value of largest magnitude (if
// any); one integer max per value.
template <int N>
__device__ __forceinline__ uint32_t mag_max(const float* x) {
  int32_t smax = INT32_MIN;
  uint32_t umax = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    smax = max(smax, (int32_t)__float_as_uint(x[i]));
    umax = max(umax, __float_as_uint(x[i]));
  }
  const uint32_t pos = smax < 0 ? 0u : (uint32_t)smax;
  const uint32_t neg = (umax >> 31) ? (umax & 0x7fffffffu) : 0u;
  return max(pos, neg) << 1;
}
// The largest mag_bits over the bf16 values packed in n 32-bit words: packed 16-bit maxima of the
// magnitudes, then the larger half, as an fp32 pattern.
__device__ __forceinline__ uint32_t mag_max_bf16(const uint32_t* w, int n) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7fff7fffu);
  for (int i = 1; i < n; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
  return (uint32_t)max(m[0], m[1]) << 17;
}
// A mag_bits pattern of an unscaled value, expressed in units scaled by 2^-e (saturating; zero,
// inf and NaN unchanged).
__device__ __forceinline__ uint32_t mag_scaled(uint32_t m, int e) {
  const int E = (int)(m >> 24);
  if (m == 0 || E == 255) return m;
  const int Es = E - e < 1 ? 1 : (E - e > 254 ? 254 : E - e);
  return ((uint32_t)Es << 24) | (m & 0xffffffu);
}
// largest of the wave's lanes (each lane's value >= 0 as an unsigned pattern)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
  const uint32_t a = __builtin_amdgcn_readlane(x, 15), b = __builtin_amdgcn_readlane(x, 31);
  const uint32_t c = __builtin_amdgcn_readlane(x, 47), d = __builtin_amdgcn_readlane(x, 63);
  return max(max(a, b), max(c, d));
}
// Range exponent e of a chunk from the largest |S| and |v| (pattern m, in the previous chunk's
// scaled units 2^-e_prev): 0 while the largest true magnitude is inside [2^-6, 2^6) or zero;
// otherwise the scaled largest magnitude lands in [2^4, 2^5), with 2^e and 2^-e kept normal.
// With an inf or NaN present nothing can be kept in range (it propagates) and e_prev is kept.
__device__ __forceinline__ int range_exponent(uint32_t m, int e_prev) {
  const int Em = (int)(m >> 24);  // biased exponent
  if (Em == 255) return e_prev;
  if (m == 0) return 0;
  const int E = Em - 127 + e_prev;
  if (E >= -6 && E < 6) return 0;
  const int e = E - 4;
  return e < -125 ? -125 : (e > 125 ? 125 : e);
}
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// ---------------------------------------------------------------------------
// LDS layout (bytes).  Regions with disjoint lifetimes share memory:
//   RB (gate stage -> off-diagonal Gram) with YT (T stage -> U),
//   PT (partial Gram tiles) with TB (T stage -> U) and UT (U -> state update).
// ---------------------------------------------------------------------------
template <int C, int DK, int BV, Prec P>
struct Lay {
  using T = typename Op<P>::T;
  static constexpr int KS = Op<P>::KS, PD = Op<P>::PAD;
  static constexpr int NB = C / 16;
  static constexpr int CK = ((C + KS - 1) / KS) * KS;   // token k-extent rounded to the MMA step
  static constexpr int LDD = DK + PD;                   // [*][DK] rows (k = channel)
  static constexpr int LDC = CK + PD;                   // [*][CK] rows (k = token)
  static constexpr int LDA = C + 4;                     // fp32 [C][C] rows
  static constexpr int NPAIR = NB * (NB - 1) / 2;       // off-diagonal sub-block pairs
  static constexpr int NPALL = NB * (NB + 1) / 2;
  // persistent
  static constexpr size_t BH = 0;                                         // e^{s_J/2} [NB][DK] f32
  static constexpr size_t ST = BH + al16(size_t(NB) * DK * 4);            // S^T [BV][LDD]
  static constexpr size_t AK = ST + al16(size_t(BV) * LDD * sizeof(T));   // A then T, f32 [C][LDA]
  static constexpr size_t AQ = AK + al16(size_t(C) * LDA * 4);            // strict M [C][LDC]
  // off-diagonal A tiles, f32 [NPAIR][16][AOR]: rows padded to 20 floats so the float4 row
  // reads of eight consecutive rows fall on distinct LDS bank groups
  static constexpr int AOR = 20;
  static constexpr size_t AO = AQ + al16(size_t(C) * LDC * sizeof(T));
  static constexpr size_t BE = AO + al16(size_t(NPAIR) * 16 * AOR * 4);   // beta [C]
  static constexpr size_t DQ = BE + al16(size_t(C) * 4);                  // q_r . k_r [C]
  static constexpr size_t GM = DQ + al16(size_t(C) * 4);                  // e^{g_last} [DK]
  // per-wave words: largest |S|, largest |v|, exact-path vote [3][NW]
  static constexpr size_t MX = GM + al16(size_t(DK) * 4);
  // per chunk
  static constexpr int LDV = BV + PD;                   // [C][BV] rows (value columns)
  static constexpr size_t QG = MX + al16(size_t(3 * NW) * 4);             // Qg [C][LDD]
  static constexpr size_t KG = QG + al16(size_t(C) * LDD * sizeof(T));    // Kg [C][LDD]
  static constexpr size_t KDT = KG + al16(size_t(C) * LDD * sizeof(T));   // Kd^T [DK][LDC]
  static constexpr size_t VR = KDT + al16(size_t(DK) * LDC * sizeof(T));  // V [C][LDV]
  static constexpr size_t X1 = VR + al16(size_t(C) * LDV * sizeof(T));    // RB | YT
  static constexpr size_t RB = X1;                                        // right base [C][LDD]
  static constexpr size_t YT = X1;                                        // (V - Kg S)^T [BV][LDC]
  static constexpr size_t X2 = X1 + cmax(al16(size_t(C) * LDD * sizeof(T)), al16(size_t(BV) * LDC * sizeof(T)));
  static constexpr size_t PT = X2;                                        // partial tiles f32 [2*NPALL][64][4]
  static constexpr size_t TB = X2;                                        // T Diag(b) [C][LDC]
  static constexpr size_t UT = TB + al16(size_t(C) * LDC * sizeof(T));    // U^T [BV][LDC]
  static constexpr size_t X2END = cmax(PT + al16(size_t(2 * NPALL) * 1024),
                                       UT + al16(size_t(BV) * LDC * sizeof(T)));
  static constexpr size_t TOTAL = X2END;
};

template <int C, int DK, int BV, Prec P>
constexpr size_t lds_bytes() { return Lay<C, DK, BV, P>::TOTAL; }

// index of the off-diagonal block pair (R, I), R > I
__host__ __device__ constexpr int pair_index(int R, int I) { return R * (R - 1) / 2 + I; }

// Gate-stage row block of wave w (two waves per block, channel half = w & 1).  Waves w and
// w + 4 share a SIMD; with four blocks they take blocks R and 3 - R, so each SIMD carries
// the same number of off-diagonal sub-block pairs (block R has R of them).
template <int NB>
__device__ __forceinline__ int row_block_of(int w) {
  return (NB == 4 && w >= 4) ? 5 - (w >> 1) : (w >> 1);
}
// The channel half whose wave inverts the diagonal block R of A (the other half finishes the
// rest of the Gram reduction); chosen so the four inverting waves sit on four SIMDs.
__device__ __forceinline__ int inv_half(int R) { return ((R >> 1) & 1) ^ 1; }

// Raw global loads of one lane's inputs, held in registers one chunk ahead.
template <typename InT, int CPL>
struct GateRegs {
  static constexpr int QW = CPL * (int)sizeof(InT) / 16;  // 16-byte words for q or k
  uint4 q[QW], k[QW];
  float4 la[CPL / 4];
  float b;
};
template <typename InT>
struct VRegs {
  static constexpr int VW = 8 * (int)sizeof(InT) / 16;
  uint4 v[VW];
};

// Raw buffer loads (gfx9 descriptor: stride 0, 32-bit data format); an access at or past
// `nbytes` from `base` returns zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ float buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// An empty use of every loaded register on every path: the memory counter is waited on
// here, where the data has long arrived, instead of before the next loads into the same
// registers (a wave that skipped a conditional use would otherwise carry the pending load
// into the next chunk and wait for every load in flight when it reloads the register).
__device__ __forceinline__ void retire(const uint4& x) {
  asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}
__device__ __forceinline__ void retire(const float4& x) {
  asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}
__device__ __forceinline__ void retire(float x) { asm volatile("" ::"v"(x)); }

template <typename InT>
__device__ __forceinline__ void unpack(const uint4* w, float* out, int n) {
  if constexpr (sizeof(InT) == 2) {
    for (int i = 0; i < n / 8; ++i) {
      const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 f = bf16x2_to_f32x2(ww[j]);
        out[8 * i + 2 * j] = f.x;
        out[8 * i + 2 * j + 1] = f.y;
      }
    }
  } else {
    for (int i = 0; i < n / 4; ++i) {
      out[4 * i] = __uint_as_float(w[i].x);
      out[4 * i + 1] = __uint_as_float(w[i].y);
      out[4 * i + 2] = __uint_as_float(w[i].z);
      out[4 * i + 3] = __uint_as_float(w[i].w);
    }
  }
}

// ---------------------------------------------------------------------------
// Workspace tile of the split path: one chunk's state-free operands for one head, in
// 16-byte units.  The fp16 matrices are stored in matrix-core fragment order: for a
// [rows][K] matrix (K padded to a multiple of 32 with zeros), unit
// ((rb * K/32 + s) * 64 + lane) holds row 16 rb + (lane & 15), elements
// 32 s + 8 (lane >> 4) .. +7, so that the operand of one k-step for one 16-row block is
// 1 KB of consecutive units, one per lane.  The two token-by-token matrices (strict M and
// T Diag(beta), both lower triangular) keep only the fragments that reach their row block:
// fragment (R, s) for s < tri(R), at index tri_base(R) + s (6 of 8 at C = 64).  The two
// fp32 vectors follow in plain order.
// ---------------------------------------------------------------------------
template <int C, int DK>
struct WsTile {
  static constexpr int CK = ((C + 31) / 32) * 32;                    // token k-extent
  static constexpr int NSD = DK / 32, NSC = CK / 32;                 // k-steps over channels / tokens
  static constexpr int NB = C / 16;                                  // 16-row token blocks
  // k-steps of a lower-triangular token operand that reach row block R, and the index of
  // block R's first fragment
  __host__ __device__ static constexpr int tri(int R) { return (16 * R + 15) / 32 + 1; }  // = R / 2 + 1
  __host__ __device__ static constexpr int tri_base(int R) { return R + ((R - 1) / 2) * (R / 2); }
  static constexpr int NTRI = tri_base(NB);
  static_assert(tri_base(1) == tri(0) && tri_base(2) == tri_base(1) + tri(1) && tri_base(3) == tri_base(2) + tri(2) &&
                    tri_base(4) == tri_base(3) + tri(3),
                "closed form of the fragment prefix sums");
  static_assert(tri(NB - 1) <= NSC, "the last row block's fragments cover the token extent");
  static constexpr int QG = 0;                                       // Qg   [C][DK]
  static constexpr int KG = QG + C * DK / 8;                         // Kg   [C][DK]
  static constexpr int KDT = KG + C * DK / 8;                        // Kd^T [DK][CK]
  static constexpr int AQ = KDT + DK * CK / 8;                       // strict M, NTRI fragments
  static constexpr int TB = AQ + 64 * NTRI;                          // T Diag(beta), NTRI fragments
  static constexpr int DQ = TB + 64 * NTRI;                          // q.k [C] fp32
  static constexpr int GM = DQ + C / 4;                              // e^{g_last} [DK] fp32
  static constexpr int NU = GM + DK / 4;
};

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
// PREP = false: the fused forward.  PREP = true: the intra-chunk part only, for a group of
// `cpg` consecutive chunks of one (sequence, head) per workgroup, over chunks [in_ch0,
// in_ch_end) of every sequence (in_ch_end = 0: to the sequence's end); each chunk's
// state-free operands go to workspace slot (sequence start / C + sequence + chunk) (see
// write_ws).  Pipelined split (PIPE_BV > 0, in-chunk mode only): the first n_state_blocks
// workgroups run the state pass over chunks [ch_begin, ch_end) with value tiles of PIPE_BV
// columns (chunk_state_wave_body, defined below), the others the in-chunk pass.
struct PipeArgs {
  int n_state_blocks;
  int64_t in_ch0, in_ch_end;
  int64_t ch_begin, ch_end;
  const float* h0;
  float *o, *hT, *carry;
};

// What one workgroup of the state pass does beyond its chunk loop (chunk_state_body and
// chunk_state_wave_body take the same job).
struct StateJob {
  int chain, j0;             // chain, and the first state column of its tile
  int64_t ch_begin, ch_end;  // chunk range (clipped to the chain's chunks)
  const float* s_in;         // entering state ([n_chains][DK][DV], true units) or null for zeros
  float* end_out;            // final state when the range reaches the chain's end ([n_chains][DK][DV]) or null
  float* mid_out;            // final state otherwise ([n_chains][DK][mid_ld]) or null
  int mid_ld;
  bool map;                  // segment-map mode (see chunk_state_body)
};

// The (chain, value tile) of state-pass workgroup `bid` over n_chains chains of `ntile` tiles:
// the tiles of one chain take indices of one residue mod 8, so they run on one XCD and read
// each workspace fragment through one L2.  False for a padding workgroup (the grid covers a
// multiple of 8 chains).
__device__ __forceinline__ bool state_block(int bid, int n_chains, int ntile, int& chain, int& tile) {
  const int xcd = bid & 7, qd = bid >> 3;
  tile = qd % ntile;
  chain = (qd / ntile) * 8 + xcd;
  return chain < n_chains;
}

template <int C, int DK, int BV, typename InT>
__device__ __forceinline__ void chunk_state_body(const uint4* __restrict__ ws, const InT* __restrict__ v,
                                                 const int32_t* __restrict__ cu_seqlens, float* __restrict__ o,
                                                 int H, int DV, int64_t seq_len, const StateJob& job);
template <int C, int DK, int NCW, typename InT>
__device__ __forceinline__ void chunk_state_wave_body(const uint4* __restrict__ ws, const InT* __restrict__ v,
                                                      const int32_t* __restrict__ cu_seqlens, float* __restrict__ o,
                                                      int H, int DV, int64_t seq_len, const StateJob& job);

template <int C, int DK, int BV, Prec P, typename InT, bool PREP, int PIPE_BV = 0>
__global__ __launch_bounds__(NT, 1) void chunk_fwd_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, const float* h0,
    const int32_t* __restrict__ cu_seqlens, float* __restrict__ o, float* hT, float* __restrict__ ckpt,
    int ckpt_every, int n_chains, int H, int DV, int64_t seq_len, void* __restrict__ ws, int cpg, PipeArgs pa) {
  static_assert(PIPE_BV == 0 || PREP, "the pipelined mode pairs the state pass with the in-chunk pass");
  if constexpr (PIPE_BV > 0) {
    if ((int)blockIdx.x < pa.n_state_blocks) {
      StateJob job;
      if (!state_block((int)blockIdx.x, n_chains, DV / PIPE_BV, job.chain, job.j0)) return;
      job.j0 *= PIPE_BV;
      job.ch_begin = pa.ch_begin;
      job.ch_end = pa.ch_end;
      job.s_in = pa.ch_begin > 0 ? pa.carry : pa.h0;
      job.end_out = pa.hT;
      job.mid_out = pa.carry;
      job.mid_ld = DV;
      job.map = false;
      chunk_state_wave_body<C, DK, PIPE_BV / 16, InT>(reinterpret_cast<const uint4*>(ws), v, cu_seqlens, pa.o, H, DV,
                                                      seq_len, job);
      return;
    }
  }
  using L = Lay<C, DK, BV, P>;
  using T = typename L::T;
  constexpr int KS = L::KS, NB = L::NB, CK = L::CK;
  constexpr int LDD = L::LDD, LDC = L::LDC, LDA = L::LDA, LDV = L::LDV;
  constexpr int NPAIR = L::NPAIR;
  constexpr int NA = DK / 16;   // channel tiles
  constexpr int NJ = BV / 16;   // value-column tiles
  constexpr int CPL = DK / 8;   // gate-stage channels per lane
  constexpr int VPR = BV / 8;   // value loads: lanes per row (8 columns each)
  static_assert(C % 16 == 0 && C <= 64 && (DK == 64 || DK == 128) && BV % 16 == 0 && BV <= 64, "shape");
  static_assert(2 * NB <= NW, "two waves per 16-row sub-block");
  static_assert(C * VPR <= NT, "value load map");
  static_assert(P == Prec::F32 || CPL % 8 == 0, "k-step");
  static_assert((2 * NB + NPAIR) * DK <= C * LDA, "factor table fits the A/T region");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* sBH = reinterpret_cast<float*>(smem + L::BH);
  T* sST = reinterpret_cast<T*>(smem + L::ST);
  float* sAK = reinterpret_cast<float*>(smem + L::AK);
  T* sAQ = reinterpret_cast<T*>(smem + L::AQ);
  float* sAO = reinterpret_cast<float*>(smem + L::AO);
  float* sBE = reinterpret_cast<float*>(smem + L::BE);
  float* sDQ = reinterpret_cast<float*>(smem + L::DQ);
  float* sGM = reinterpret_cast<float*>(smem + L::GM);
  uint32_t* sMX = reinterpret_cast<uint32_t*>(smem + L::MX);
  T* sQG = reinterpret_cast<T*>(smem + L::QG);
  T* sKG = reinterpret_cast<T*>(smem + L::KG);
  T* sKDT = reinterpret_cast<T*>(smem + L::KDT);
  T* sV = reinterpret_cast<T*>(smem + L::VR);
  T* sRB = reinterpret_cast<T*>(smem + L::RB);
  T* sYT = reinterpret_cast<T*>(smem + L::YT);
  float4* sPT = reinterpret_cast<float4*>(smem + L::PT);
  T* sTB = reinterpret_cast<T*>(smem + L::TB);
  T* sUT = reinterpret_cast<T*>(smem + L::UT);

  // ---- (sequence, head, value tile); the value tiles of one chain share an XCD
  // (prep: (sequence, head, chunk group))
  const int bid = (int)blockIdx.x - (PIPE_BV > 0 ? pa.n_state_blocks : 0);
  int chain, tile = 0, grp = 0;
  if constexpr (PREP) {
    chain = bid % n_chains;
    grp = bid / n_chains;
  } else {
    const int ntile = DV / BV;
    const int xcd = bid & 7, qd = bid >> 3;
    tile = qd % ntile;
    chain = (qd / ntile) * 8 + xcd;
  }
  if (chain >= n_chains) return;
  const int n = chain / H, h = chain - n * H;
  const int j0 = tile * BV;
  int64_t t_begin, t_end;
  if (cu_seqlens) {
    t_begin = cu_seqlens[n];
    t_end = cu_seqlens[n + 1];
  } else {
    t_begin = (int64_t)n * seq_len;
    t_end = t_begin + seq_len;
  }

  int tid = threadIdx.x;
  const int wave0 = __builtin_amdgcn_readfirstlane(tid / kWave);
  int wave = wave0;
  // Masking the opaque wave index with NW - 1 (an identity) hands the compiler its range
  // back, so wave-dependent LDS offsets use 24-bit multiplies instead of 32- and 64-bit
  // ones (quarter rate): 1.4% off the BV = 64 tiles; the BV = 16 tiles lose 4% under
  // the changed schedule and BV = 32 gains nothing, so they keep the unmasked index.
  constexpr bool kMaskWave = BV >= 64;
  int l = lane_id();
  int lr = l & 15, lg = l >> 4;
  // A lane index the compiler cannot see through: lane-derived addresses are recomputed
  // where they are used instead of being held (or spilled) across the chunk loop.
  auto fresh_lane = [&]() {
    int x = lane_id();
    asm volatile("" : "+v"(x));
    return x & (kWave - 1);  // keeps the known range (24-bit multiplies, shifts)
  };
  auto refresh_lane = [&]() {
    l = fresh_lane();
    lr = l & 15;
    lg = l >> 4;
    tid = wave0 * kWave + l;
  };

  // one-time zero fill of the persistent strictly-lower operands' upper parts
  for (int i = tid; i < C * LDA; i += NT) sAK[i] = 0.f;
  for (int i = tid; i < C * LDC; i += NT) sAQ[i] = cvt<T>(0.f);

  // ---- fp32 master state: tiles (a, j), id = a + NA*j owned by wave id % NW
  constexpr int S_SLOTS = (NA * NJ + NW - 1) / NW;
  f32x4 Sacc[S_SLOTS];
  const float* h0p = h0 ? h0 + (size_t)chain * DK * DV : nullptr;
#pragma unroll
  for (int s = 0; s < S_SLOTS; ++s) {
    const int id = wave + NW * s;
    Sacc[s] = zero4();
    if (!PREP && id < NA * NJ && h0p) {
      const int a = id % NA, j = id / NA;
#pragma unroll
      for (int i = 0; i < 4; ++i) Sacc[s][i] = h0p[(size_t)(16 * a + 4 * lg + i) * DV + j0 + 16 * j + lr];
    }
  }
  // The 16-bit copy of the state for the chunk's products.  In the 16-bit precision the fp32
  // state is held in the chunk's scaled units 2^-e (see range_exponent): it is rescaled when e
  // changes, and o, hT and the checkpoints are scaled back by 2^e.
  auto write_ST = [&]() {
#pragma unroll
    for (int s = 0; s < S_SLOTS; ++s) {
      const int id = wave + NW * s;
      if ((NA * NJ) % NW == 0 || id < NA * NJ) {
        const int a = id % NA, j = id / NA;
        store4(sST + (16 * j + lr) * LDD + 16 * a + 4 * lg, Sacc[s][0], Sacc[s][1], Sacc[s][2], Sacc[s][3]);
      }
    }
  };
  // Range exponent of the chunk in flight (16-bit operands only).
  constexpr bool kRanged = P == Prec::Mixed && !PREP;
  int sc_e = 0;
  float sc_dn = 1.f, sc_up = 1.f;  // 2^-e and 2^e
  // largest |v| of this thread's values of the next chunk, as a mag_bits pattern
  uint32_t v_mag = 0;
  auto publish_range = [&]() {
    if constexpr (kRanged) {
      float sv[4 * S_SLOTS];
#pragma unroll
      for (int s = 0; s < S_SLOTS; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * s + i] = ((NA * NJ) % NW == 0 || wave + NW * s < NA * NJ) ? Sacc[s][i] : 0.f;
      uint32_t m = mag_max<4 * S_SLOTS>(sv);
      m = max(m, sc_e == 0 ? v_mag : mag_scaled(v_mag, sc_e));
      m = wave_max_u32(m);
      if (lane_id() == 0) sMX[wave0] = m;
    }
  };

  // ---- gate-stage map: waves (R = wave/2, p = wave%2) for 2*NB waves
  const bool e_act = 2 * NB >= NW || wave0 < 2 * NB;
  // gate-stage load map: lane (r, g) of wave (R, p) loads row 16R + r, channels p*DK/2 + CPL*g ..
  // value-load map: thread t < C*VPR loads 8 columns of one row
  const bool v_act = C * VPR >= NT || tid < C * VPR;
  int v_row = tid / VPR, v_c0 = 8 * (tid % VPR);

  // U / O tiles (R, j), held transposed: lane (token 16R + (l & 15), columns
  // 16j + 4 (l >> 4) .. +3)
  constexpr int U_SLOTS = (NB * NJ + NW - 1) / NW;
  // With 4 row blocks, 4 value tiles and 8 waves, slot s of wave w holds row block
  // 2s + w/4: slot 0 only ever sees tokens below 32 and slot 1 below 64, so products
  // over tokens whose token operand is block-lower-triangular (T Diag(beta), M) stop
  // at a compile-time k-step.
  constexpr bool UO_SPLIT = NB == 4 && NJ == 4 && NW == 8;
  auto uo_tile = [&](int s, int& R, int& j) {
    if constexpr (UO_SPLIT) {
      R = 2 * s + (wave >> 2);
      j = wave & 3;
    } else {
      const int id = wave + NW * s;
      R = id % NB;
      j = id / NB;
    }
  };

  const int64_t nchunks = (t_end - t_begin + C - 1) / C;
  int64_t ch_lo = 0, ch_hi = nchunks;
  if constexpr (PREP) {
    const int64_t lim = pa.in_ch_end > 0 && pa.in_ch_end < nchunks ? pa.in_ch_end : nchunks;
    ch_lo = pa.in_ch0 + (int64_t)grp * cpg;
    ch_hi = ch_lo + cpg < lim ? ch_lo + cpg : lim;
    if (ch_lo >= ch_hi) return;
  }

  using GR = GateRegs<InT, CPL>;
  using VR = VRegs<InT>;
  // Global addressing: a chunk-uniform 64-bit base plus a 32-bit per-lane element offset
  // (the scalar-base form of the global loads and stores; no 64-bit lane arithmetic).
  auto gate_map = [&](int& row, int& elem) {
    const int x = fresh_lane();
    row = 16 * (e_act ? row_block_of<NB>(wave0) : 0) + (x & 15);
    elem = row * H * DK + (wave0 & 1) * (DK / 2) + CPL * (x >> 4);
  };
  GR gbuf;
  VR vbuf;
  // The next chunk's inputs are loaded in four groups (q; k; the log-decay; v and beta),
  // issued in different stages: every CU runs the same stage at about the same time, and
  // one large group per chunk would be a device-wide burst that saturates HBM and stalls
  // instruction issue while the rest of the chunk leaves it idle.
  // Each group is a raw buffer load whose descriptor covers the chunk's valid rows of this
  // head: rows past the chunk's length (and every row past the last chunk) read as zero
  // in hardware, so the loads need no branch and no zero fill.
  auto row_bytes = [&](int Lc, uint32_t bytes_per_row) -> uint32_t {
    return (e_act && Lc > 0) ? (uint32_t)Lc * bytes_per_row : 0u;
  };
  auto load_qk1 = [&](const InT* src, uint4 (&dst)[GR::QW], int64_t cb, int Lc) {
    int ld_row, el;
    gate_map(ld_row, el);
    const uint32_t ld_off = (uint32_t)el * (uint32_t)sizeof(InT);
    const auto rs = make_rsrc(src + ((size_t)cb * H + h) * DK, row_bytes(Lc, (uint32_t)(H * DK * sizeof(InT))));
#pragma unroll
    for (int i = 0; i < GR::QW; ++i) dst[i] = buf_load16(rs, ld_off + 16 * i);
  };
  auto load_la = [&](int64_t cb, int Lc) {
    int ld_row, el;
    gate_map(ld_row, el);
    const uint32_t ld_off_f = (uint32_t)el * 4u;
    const auto rs = make_rsrc(log_alpha + ((size_t)cb * H + h) * DK, row_bytes(Lc, (uint32_t)(H * DK * 4)));
#pragma unroll
    for (int i = 0; i < CPL / 4; ++i) gbuf.la[i] = __builtin_bit_cast(float4, buf_load16(rs, ld_off_f + 16 * i));
  };
  auto load_vb = [&](int64_t cb, int Lc) {
    int ld_row, el;
    gate_map(ld_row, el);
    const uint32_t ld_off_b = (uint32_t)(ld_row * H) * 4u;
    const int t = wave0 * kWave + fresh_lane();
    // lanes past the C * VPR value loads have v_row >= C, past every chunk's valid rows
    const int v_row = t / VPR, v_c0 = 8 * (t % VPR);
    const uint32_t v_off = (uint32_t)(v_row * H * DV + v_c0) * (uint32_t)sizeof(InT);
    const auto rb_ = make_rsrc(beta + (size_t)cb * H + h, row_bytes(Lc, (uint32_t)(H * 4)));
    const auto rv = make_rsrc(v + ((size_t)cb * H + h) * DV + j0,
                              Lc > 0 ? (uint32_t)Lc * (uint32_t)(H * DV * sizeof(InT)) : 0u);
    gbuf.b = buf_load4(rb_, ld_off_b);
#pragma unroll
    for (int i = 0; i < VR::VW; ++i) vbuf.v[i] = PREP ? make_uint4(0, 0, 0, 0) : buf_load16(rv, v_off + 16 * i);
  };
  auto load_chunk = [&](int64_t cb, int Lc) {
    load_qk1(q, gbuf.q, cb, Lc);
    load_qk1(k, gbuf.k, cb, Lc);
    load_la(cb, Lc);
    load_vb(cb, Lc);
  };
  auto chunk_len = [&](int64_t ch) -> int {
    const int64_t rem = t_end - (t_begin + ch * C);
    return (int)(rem < C ? rem : C);
  };
  f32x4 Opend[U_SLOTS];
  int64_t o_begin = 0;
  int o_len = 0;
  // the fp32 master state of this value tile into a [DK][DV] row-major state
  // (from the chunk's scaled units back to the state's own)
  auto store_state = [&](float* sp) {
#pragma unroll
    for (int s = 0; s < S_SLOTS; ++s) {
      const int id = wave + NW * s;
      if ((NA * NJ) % NW == 0 || id < NA * NJ) {
        const int a = id % NA, j = id / NA;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sp[(size_t)(16 * a + 4 * lg + i) * DV + j0 + 16 * j + lr] = kRanged ? Sacc[s][i] * sc_up : Sacc[s][i];
      }
    }
  };
  // Workspace tile of one (chunk, head), 16-byte units in this order: Qg [C][DK], Kg [C][DK],
  // Kd^T [DK][C], strict M [C][C], T Diag(beta) [C][C] (all T), then q.k [C] and e^{g_last}
  // [DK] (fp32).  Slot of chunk j of the sequence starting at token t0: t0 / C + n + j.
  auto write_ws = [&](int64_t chn) {
    using W = WsTile<C, DK>;
    static_assert(!PREP || sizeof(T) == 2, "fp16 operands");
    const int64_t slot = t_begin / C + n + chn;
    uint4* dst = reinterpret_cast<uint4*>(ws) + ((size_t)slot * H + h) * W::NU;
    // Unrolled over blocks of NT units with the thread index the compiler can see (its range
    // is the launch bound): all but the last two blocks lie in one region each, so their
    // region tests fold and the fragment, row and column of a unit reduce to a per-thread
    // constant plus an immediate (a rolled loop recomputed them for every unit: 6% of the
    // varlen batch's split time).
#pragma unroll
    for (int m = 0; m < (W::NU + NT - 1) / NT; ++m) {
      const int i = (int)threadIdx.x + NT * m;
      if (W::NU % NT != 0 && i >= W::NU) break;
      // byte offset in LDS of unit i's source
      uint32_t off;
      bool pad = false;  // a k-unit past the chunk's tokens: zero
      if (i < W::KDT) {
        // Qg, Kg: rows are tokens, k runs over the key channels
        const int ii = i < W::KG ? i : i - W::KG, f = ii >> 6, ln = ii & 63;
        const int row = 16 * (f / W::NSD) + (ln & 15), k0 = 32 * (f % W::NSD) + 8 * (ln >> 4);
        off = (uint32_t)(i < W::KG ? L::QG : L::KG) + (uint32_t)(row * LDD + k0) * 2u;
      } else if (i < W::DQ) {
        // Kd^T (rows: channels), M and T Diag(beta) (rows: tokens, the fragments that reach
        // each row block); k runs over the tokens
        const int ii = i < W::AQ ? i - W::KDT : (i < W::TB ? i - W::AQ : i - W::TB), f = ii >> 6, ln = ii & 63;
        int rb = f / W::NSC, st = f % W::NSC;
        if (i >= W::AQ) {
          rb = 0;
#pragma unroll
          for (int r = 1; r < W::NB; ++r) rb += f >= W::tri_base(r) ? 1 : 0;
          st = f - W::tri_base(rb);
        }
        const int row = 16 * rb + (ln & 15), k0 = 32 * st + 8 * (ln >> 4);
        pad = k0 >= C;
        off = (uint32_t)(i < W::AQ ? L::KDT : (i < W::TB ? L::AQ : L::TB)) + (uint32_t)(row * LDC + (pad ? 0 : k0)) * 2u;
      } else if (i < W::GM) {
        off = (uint32_t)L::DQ + (uint32_t)(i - W::DQ) * 16u;
      } else {
        off = (uint32_t)L::GM + (uint32_t)(i - W::GM) * 16u;
      }
      // written once, read once by the state pass much later: a streaming store
      typedef unsigned int u32x4w __attribute__((ext_vector_type(4)));
      u32x4w val = *reinterpret_cast<const u32x4w*>(smem + off);
      if (pad) val = u32x4w{0u, 0u, 0u, 0u};
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4w*>(dst) + i);
    }
  };
  auto store_pending = [&]() {
    char* ob = reinterpret_cast<char*>(o + ((size_t)o_begin * H + h) * DV + j0);
#pragma unroll
    for (int s = 0; s < U_SLOTS; ++s) {
      const int id = wave + NW * s;
      if ((NB * NJ) % NW == 0 || id < NB * NJ) {
        int R, j;
        uo_tile(s, R, j);
        const uint32_t hdv = (uint32_t)(H * DV);
        // lane (token lr, column group lg) holds o[16R + lr][16j + 4lg .. +3]
        const int r = 16 * R + lr;
        const uint32_t off = ((uint32_t)r * hdv + (uint32_t)(16 * j + 4 * lg)) * 4u;
        if (r < o_len)
          *reinterpret_cast<float4*>(ob + off) = make_float4(Opend[s][0], Opend[s][1], Opend[s][2], Opend[s][3]);
      }
    }
  };
  __syncthreads();

  // Software pipeline: the inputs of chunk c+1 are loaded during iteration c and its gate
  // stage (part a) runs beside iteration c's state products, so loaded registers never
  // cross the loop back-edge (only computed gate values do).  The right base it computes
  // shares LDS with Y^T and is stored only after Y^T's last use.
  float qL[CPL], kL[CPL], kR[CPL], rbv[CPL];
  f32x4 accQd, accKd;
  bool wide_ext = false;  // this wave's gate stage of the next chunk needs the exact path
  // Gate stage, part a, in GH channel parts of GC channels (each a whole number of the
  // diagonal Gram's MMA k-steps), then the value / beta part.  The parts of chunk c+1 run
  // beside chunk c's latency-bound MMA stages: part 0 with the inverse levels, the rest
  // with the U / O products.
  constexpr int GH = ((P == Prec::Mixed ? CPL >= 16 : CPL >= 8) && (CPL / 2) * (int)sizeof(InT) % 16 == 0) ? 2 : 1;
  constexpr int GC = CPL / GH;
  static_assert(GC * (int)sizeof(InT) % 16 == 0, "a gate part unpacks whole 16-byte input words");
  auto gate_part = [&](auto hc) {
    constexpr int hh = decltype(hc)::value;
    // Wave-dependent LDS offsets are cheap scalar arithmetic; an opaque copy of the
    // wave index keeps the compiler from hoisting (and spilling) them out of the loop.
    wave = wave0;
    asm volatile("" : "+s"(wave));
    if constexpr (kMaskWave) wave &= NW - 1;
    refresh_lane();
    const int eR = e_act ? row_block_of<NB>(wave) : 0;
    const int e_cb = (wave & 1) * (DK / 2) + CPL * lg + hh * GC;
    if constexpr (hh == 0) {
      accQd = zero4();
      accKd = zero4();
      wide_ext = false;
    }
    float* const qh_ = qL + hh * GC;
    float* const kh_ = kL + hh * GC;
    float* const rh_ = kR + hh * GC;
    float* const bh_ = rbv + hh * GC;
    unpack<InT>(gbuf.q + hh * (GR::QW / GH), qh_, GC);
    unpack<InT>(gbuf.k + hh * (GR::QW / GH), kh_, GC);
    float la[GC];
#pragma unroll
    for (int i = 0; i < GC / 4; ++i) {
      const float4 x = gbuf.la[hh * (GC / 4) + i];
      la[4 * i] = x.x; la[4 * i + 1] = x.y; la[4 * i + 2] = x.z; la[4 * i + 3] = x.w;
    }
    if (e_act) {
      // in-block cumulative decay c and block total s, in log2 units; every phase
      // runs across all channels so the DPP and permute latencies overlap
      float cc[GC], ss[GC];
#pragma unroll
      for (int j = 0; j < GC; ++j) cc[j] = la[j] * 1.4426950408889634f;
#pragma unroll
      for (int j = 0; j < GC; ++j) cc[j] += shr16<1>(cc[j]);
#pragma unroll
      for (int j = 0; j < GC; ++j) cc[j] += shr16<2>(cc[j]);
#pragma unroll
      for (int j = 0; j < GC; ++j) cc[j] += shr16<4>(cc[j]);
#pragma unroll
      for (int j = 0; j < GC; ++j) cc[j] += shr16<8>(cc[j]);
#pragma unroll
      for (int j = 0; j < GC; ++j) ss[j] = row_bcast16<15>(cc[j]);
      // When every channel of this part decays by less than 8 nats over the block, the
      // balanced operands stay within e^{+-4} of the inputs and fp16 represents them as
      // well as the off-diagonal operands; otherwise the part's diagonal products take
      // the wide path.  The vote is wave-uniform.
      float smin = ss[0];
#pragma unroll
      for (int j = 1; j < GC; ++j) smin = fminf(smin, ss[j]);
      [[maybe_unused]] const bool fast16 = __builtin_amdgcn_ballot_w64(!(smin > -11.5415603f)) == 0;  // 8 nats in log2 units
      // Past 160 nats over the block the balanced factors overflow: the wave redoes its gate stage
      // on the exact path (fix_exact) after the next barrier, out of this code's way.
      wide_ext |= __builtin_amdgcn_ballot_w64(!(smin > kBalancedLimit)) != 0;
#pragma unroll
      for (int j = 0; j < GC; ++j) {
        const float x = cc[j] - 0.5f * ss[j];
        const float eL = __builtin_amdgcn_exp2f(x);  // e^{c - s/2} <= e^{|s|/2}
        const float eRt = __builtin_amdgcn_exp2f(-x);
        // e^{s/2} <= 1 is e^{c - s/2} at the block's last row (c = s there, and s - s/2
        // is exact), so lane 15 of the row supplies it (below 2^-126 it flushes to 0)
        const float bh = row_bcast16<15>(eL);
        const float kk = kh_[j];
        qh_[j] *= eL;
        kh_[j] = kk * eL;
        rh_[j] = kk * eRt;
        bh_[j] = rh_[j] * bh;                                    // right base k e^{s - c} <= |k|
        ss[j] = bh;
      }
      if (lr == 15) {
#pragma unroll
        for (int j = 0; j < GC; j += 4) store4(sBH + eR * DK + e_cb + j, ss[j], ss[j + 1], ss[j + 2], ss[j + 3]);
      }
      // diagonal Gram sub-block partials over this part's channels
      if constexpr (P == Prec::Mixed) {
        if (fast16) {
          // narrow decay: fp16 operands, one MFMA per 8 channels for each of M and A
#pragma unroll
          for (int t = 0; t < GC / 8; ++t) {
            half8 qh, kh, rh;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              qh[j] = (_Float16)qh_[8 * t + j];
              kh[j] = (_Float16)kh_[8 * t + j];
              rh[j] = (_Float16)rh_[8 * t + j];
            }
            accQd = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh, rh, accQd, 0, 0, 0);
            accKd = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, rh, accKd, 0, 0, 0);
          }
        } else {
            // wide decay: M on the fp32 matrix core; A in bf16 (range), one MFMA per 8 channels
#pragma unroll
            for (int j = 0; j < GC; ++j) accQd = __builtin_amdgcn_mfma_f32_16x16x4f32(qh_[j], rh_[j], accQd, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < GC / 8; ++t) {
              bf16x8 kh, bh8;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                kh[j] = (__bf16)kh_[8 * t + j];
                bh8[j] = (__bf16)rh_[8 * t + j];
              }
              accKd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, bh8, accKd, 0, 0, 0);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < GC; ++j) {
            accQd = __builtin_amdgcn_mfma_f32_16x16x4f32(qh_[j], rh_[j], accQd, 0, 0, 0);
            accKd = __builtin_amdgcn_mfma_f32_16x16x4f32(kh_[j], rh_[j], accKd, 0, 0, 0);
          }
        }
    }
  };
  // the value / beta part; it also retires every loaded register of the chunk
  auto gate_v = [&]() {
    wave = wave0;
    asm volatile("" : "+s"(wave));
    if constexpr (kMaskWave) wave &= NW - 1;
    refresh_lane();
    v_row = tid / VPR;
    v_c0 = 8 * (tid % VPR);
    const int eR = e_act ? row_block_of<NB>(wave) : 0;
    if (!PREP && v_act) {
      if constexpr (kRanged) {
        // the next chunk's values to LDS as they are (bf16): the chunk's range factor is
        // applied where Y is formed, after its exponent is known
        static_assert(sizeof(InT) == 2 && sizeof(T) == 2 && VR::VW == 1, "8 bf16 values per thread");
        *reinterpret_cast<uint4*>(sV + v_row * LDV + v_c0) = vbuf.v[0];
      } else {
        float vv[8];
        unpack<InT>(vbuf.v, vv, 8);
        store4(sV + v_row * LDV + v_c0, vv[0], vv[1], vv[2], vv[3]);
        store4(sV + v_row * LDV + v_c0 + 4, vv[4], vv[5], vv[6], vv[7]);
      }
      if constexpr (kRanged) {
        uint32_t w[4 * VR::VW];
#pragma unroll
        for (int i = 0; i < VR::VW; ++i) {
          w[4 * i] = vbuf.v[i].x; w[4 * i + 1] = vbuf.v[i].y; w[4 * i + 2] = vbuf.v[i].z; w[4 * i + 3] = vbuf.v[i].w;
        }
        v_mag = mag_max_bf16(w, 4 * VR::VW);
      }
    }
    if (e_act && (wave & 1) == 0 && lg == 0) sBE[16 * eR + lr] = gbuf.b;
#pragma unroll
    for (int i = 0; i < GR::QW; ++i) {
      retire(gbuf.q[i]);
      retire(gbuf.k[i]);
    }
#pragma unroll
    for (int i = 0; i < CPL / 4; ++i) retire(gbuf.la[i]);
    retire(gbuf.b);
#pragma unroll
    for (int i = 0; i < VR::VW; ++i) retire(vbuf.v[i]);
  };
  auto gate_a = [&]() {
    static_for<0, GH>(gate_part);
    gate_v();
  };
  // The gate stage of one part on the exact path, from the raw inputs in gbuf: operands
  // referenced to the block start instead of its middle (left q e^{c}, k e^{c} <= 1, right base
  // k e^{s - c} <= 1), the diagonal Gram from per-element factors.  The block's own factor in the
  // chunk tables is then 1, which the stored decay e^{s} says by its sign bit (stored negated;
  // -0 when it underflows).
  auto exact_part = [&](auto hc) {
    constexpr int hh = decltype(hc)::value;
    const int eR = row_block_of<NB>(wave0);
    const int e_cb = (wave0 & 1) * (DK / 2) + CPL * lg + hh * GC;
    if constexpr (hh == 0) {
      accQd = zero4();
      accKd = zero4();
    }
    float* const qh_ = qL + hh * GC;
    float* const kh_ = kL + hh * GC;
    float* const rh_ = kR + hh * GC;
    float* const bh_ = rbv + hh * GC;
    unpack<InT>(gbuf.q + hh * (GR::QW / GH), qh_, GC);
    unpack<InT>(gbuf.k + hh * (GR::QW / GH), kh_, GC);
    float la[GC];
#pragma unroll
    for (int i = 0; i < GC / 4; ++i) {
      const float4 x = gbuf.la[hh * (GC / 4) + i];
      la[4 * i] = x.x; la[4 * i + 1] = x.y; la[4 * i + 2] = x.z; la[4 * i + 3] = x.w;
    }
    float cx[GC], ss[GC];
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      const float x = la[j] * 1.4426950408889634f;
      cx[j] = x < kStepFloor ? kStepFloor : x;  // (a NaN stays NaN)
    }
#pragma unroll
    for (int j = 0; j < GC; ++j) cx[j] += shr16<1>(cx[j]);
#pragma unroll
    for (int j = 0; j < GC; ++j) cx[j] += shr16<2>(cx[j]);
#pragma unroll
    for (int j = 0; j < GC; ++j) cx[j] += shr16<4>(cx[j]);
#pragma unroll
    for (int j = 0; j < GC; ++j) cx[j] += shr16<8>(cx[j]);
    gram_exact<GC>(qh_, kh_, cx, lr, lg, accQd, accKd);
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      const float sx = row_bcast16<15>(cx[j]);
      const float eq = __builtin_amdgcn_exp2f(cx[j]);
      const float kk = kh_[j];
      qh_[j] *= eq;
      kh_[j] = kk * eq;
      rh_[j] = kk * __builtin_amdgcn_exp2f(sx - cx[j]);
      bh_[j] = rh_[j];
      ss[j] = -__builtin_amdgcn_exp2f(sx);
    }
    if (lr == 15) {
#pragma unroll
      for (int j = 0; j < GC; j += 4) store4(sBH + eR * DK + e_cb + j, ss[j], ss[j + 1], ss[j + 2], ss[j + 3]);
    }
  };
  auto store_rb = [&]() {
    const int x = fresh_lane();
    const int eR = e_act ? row_block_of<NB>(wave0) : 0;
    if (e_act && eR < NB - 1) {
      T* dst = sRB + (16 * eR + (x & 15)) * LDD + (wave0 & 1) * (DK / 2) + CPL * (x >> 4);
#pragma unroll
      for (int j = 0; j < CPL; j += 4) store4(dst + j, rbv[j], rbv[j + 1], rbv[j + 2], rbv[j + 3]);
    }
  };
  // A wave whose gate stage voted for the exact path reloads the chunk's q, k and log-decay and
  // redoes its gate stage on that path (every part, so its partial Gram sums are consistent).
  auto fix_exact = [&](int64_t cb, int Lc) {
    refresh_lane();
    load_qk1(q, gbuf.q, cb, Lc);
    load_qk1(k, gbuf.k, cb, Lc);
    load_la(cb, Lc);
    static_for<0, GH>(exact_part);
#pragma unroll
    for (int i = 0; i < GR::QW; ++i) {
      retire(gbuf.q[i]);
      retire(gbuf.k[i]);
    }
#pragma unroll
    for (int i = 0; i < CPL / 4; ++i) retire(gbuf.la[i]);
    store_rb();
  };
  if (ch_hi > ch_lo) {
    load_chunk(t_begin + ch_lo * C, chunk_len(ch_lo));
    gate_a();
    store_rb();
    publish_range();
    if (lane_id() == 0) sMX[2 * NW + wave0] = wide_ext;
  }
  for (int64_t ch = ch_lo; ch < ch_hi; ++ch) {
    const int64_t c_begin = t_begin + ch * C;
    const int Lc = chunk_len(ch);
    // Wave-dependent LDS offsets are cheap scalar arithmetic; an opaque copy of the
    // wave index keeps the compiler from hoisting (and spilling) them out of the loop.
    wave = wave0;
    asm volatile("" : "+s"(wave));
    if constexpr (kMaskWave) wave &= NW - 1;
    refresh_lane();
    v_row = tid / VPR;
    v_c0 = 8 * (tid % VPR);
    const int eR = e_act ? row_block_of<NB>(wave) : 0, ep = wave & 1;
    const int e_row = 16 * eR + lr;
    const int e_cb = ep * (DK / 2) + CPL * lg;

    __syncthreads();  // ------------------------------------------------------------- B_a

    // ================= the exact path for blocks of extreme decay (rare) =================
    {
      static_assert(NW == 8, "16-byte reads of the per-wave words");
      const uint4 f0 = *reinterpret_cast<const uint4*>(sMX + 2 * NW), f1 = *reinterpret_cast<const uint4*>(sMX + 2 * NW + 4);
      if (__builtin_amdgcn_readfirstlane(f0.x | f0.y | f0.z | f0.w | f1.x | f1.y | f1.z | f1.w)) {
        if (wide_ext) fix_exact(c_begin, Lc);
        __syncthreads();
      }
    }

    // ================= the chunk's range exponent and its 16-bit state copy =================
    if constexpr (kRanged) {
      static_assert(NW == 8, "16-byte reads of the per-wave maxima");
      const uint4 a0 = *reinterpret_cast<const uint4*>(sMX), a1 = *reinterpret_cast<const uint4*>(sMX + 4);
      const uint32_t m = max(max(max(a0.x, a0.y), max(a0.z, a0.w)), max(max(a1.x, a1.y), max(a1.z, a1.w)));
      const int e = range_exponent(__builtin_amdgcn_readfirstlane(m), sc_e);
      if (e != sc_e) {
        // rescale the held state to the new units, in two steps (the shift may exceed 2^126)
        const int d = sc_e - e, d1 = d / 2;
        const float f1 = pow2i(d1), f2 = pow2i(d - d1);
#pragma unroll
        for (int s = 0; s < S_SLOTS; ++s) Sacc[s] = (Sacc[s] * f1) * f2;
        sc_e = e;
        sc_dn = pow2i(-e);
        sc_up = pow2i(e);
      }
    }
    // (waves past the factor stage's DK threads write their copy now, the others after it)
    auto write_copies = [&]() {
      if constexpr (!PREP) write_ST();
    };
    if (tid >= DK) write_copies();

    // ================= per-channel block factors (once per chunk) =================
    // With bh_J = e^{s_J/2} (<= 1), for row block R and channel c:
    //   pre_R  = bh_R prod_{J<R} bh_J^2 = e^{G_{R-1} + s_R/2}      Qg = qL pre, Kg = kL pre
    //   post_R = bh_R prod_{J>R} bh_J^2 = e^{g_last - G_R + s_R/2} Kd = kR post
    //   f_RI   = bh_R prod_{I<J<R} bh_J^2                          off-diagonal left factor (I < R)
    //   gamma  = prod_J bh_J^2 = e^{g_last}
    // A block on the exact path stores -e^{s_J} instead: its operands are referenced to the
    // block start, so its own factor is 1 and its squared factor is e^{s_J}.
    // Stored in the A/T region, which is free from the previous chunk's WY stage until
    // this chunk's Gram reduction.
    float* sFT = sAK;
    if (tid < DK) {
      float bh[NB], b2[NB];
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        const float x = sBH[J * DK + tid];
        const bool exact = __float_as_uint(x) >> 31;
        bh[J] = exact ? 1.f : x;
        b2[J] = exact ? -x : x * x;
      }
      float g = 1.f;
#pragma unroll
      for (int R = 0; R < NB; ++R) {
        float pre = bh[R], post = bh[R];
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J < R) pre *= b2[J];
          if (J > R) post *= b2[J];
        }
        sFT[R * DK + tid] = pre;
        sFT[(NB + R) * DK + tid] = post;
        float f = bh[R];
#pragma unroll
        for (int I = R - 1; I >= 0; --I) {
          sFT[(2 * NB + pair_index(R, I)) * DK + tid] = f;
          f *= b2[I];
        }
        g *= b2[R];
      }
      sGM[tid] = g;
      write_copies();
    }
    // Next-chunk loads (and the next gate stage) run unconditionally: past the last chunk
    // the length is <= 0 and every load reads zero.  Each group is issued as a wave finishes
    // a stage's work rather than right after a barrier, so the device's requests spread out.
    load_qk1(q, gbuf.q, c_begin + C, chunk_len(ch + 1));
    __syncthreads();  // ------------------------------------------------------------- B_f1

    // ================= gate stage, part b: off-diagonal Gram, state operands =================
    f32x4 accQo[NB > 1 ? NB - 1 : 1], accKo[NB > 1 ? NB - 1 : 1];
#pragma unroll
    for (int I = 0; I < NB - 1; ++I) accQo[I] = accKo[I] = zero4();
    if (e_act) {
      {
        const float* fpre = sFT + eR * DK + e_cb;
        const float* fpost = sFT + (NB + eR) * DK + e_cb;
#pragma unroll
        for (int j4 = 0; j4 < CPL; j4 += 4) {
          const float4 pr = *reinterpret_cast<const float4*>(fpre + j4);
          const float4 po = *reinterpret_cast<const float4*>(fpost + j4);
          const float pre[4] = {pr.x, pr.y, pr.z, pr.w}, post[4] = {po.x, po.y, po.z, po.w};
          store4(sQG + e_row * LDD + e_cb + j4, qL[j4] * pre[0], qL[j4 + 1] * pre[1], qL[j4 + 2] * pre[2],
                 qL[j4 + 3] * pre[3]);
          store4(sKG + e_row * LDD + e_cb + j4, kL[j4] * pre[0], kL[j4 + 1] * pre[1], kL[j4 + 2] * pre[2],
                 kL[j4 + 3] * pre[3]);
#pragma unroll
          for (int u = 0; u < 4; ++u) sKDT[(e_cb + j4 + u) * LDC + e_row] = cvt<T>(kR[j4 + u] * post[u]);
        }
      }
      // off-diagonal pairs (eR, I), I < eR: left X e^{c} e^{G_{R-1} - G_I} = X{L} f_RI,
      // right = the stored right base of block I
#pragma unroll
      for (int I = 0; I < NB - 1; ++I) {
        if (I < eR) {
          const float* ff = sFT + (2 * NB + pair_index(eR, I)) * DK + e_cb;
          if constexpr (P == Prec::Mixed) {
#pragma unroll
            for (int t = 0; t < CPL / 8; ++t) {
              const float4 f0 = *reinterpret_cast<const float4*>(ff + 8 * t);
              const float4 f1 = *reinterpret_cast<const float4*>(ff + 8 * t + 4);
              const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
              half8 aq, ak;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                aq[j] = (_Float16)(qL[8 * t + j] * f[j]);
                ak[j] = (_Float16)(kL[8 * t + j] * f[j]);
              }
              const half8 b = *reinterpret_cast<const half8*>(sRB + (16 * I + lr) * LDD + e_cb + 8 * t);
              accQo[I] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, b, accQo[I], 0, 0, 0);
              accKo[I] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, b, accKo[I], 0, 0, 0);
            }
          } else {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
              const float f = ff[j];
              const float b = (float)sRB[(16 * I + lr) * LDD + e_cb + j];
              accQo[I] = __builtin_amdgcn_mfma_f32_16x16x4f32(qL[j] * f, b, accQo[I], 0, 0, 0);
              accKo[I] = __builtin_amdgcn_mfma_f32_16x16x4f32(kL[j] * f, b, accKo[I], 0, 0, 0);
            }
          }
        }
      }
      // Partial tiles change hands: the inverting half gives its M tiles and off-diagonal A
      // tiles to the other half, which gives back its diagonal A tile.
      const int base = eR * (eR + 1);  // tiles of row block eR: diag Q, diag K, then (Q, K) per I < eR
      if (ep == inv_half(eR)) {
        sPT[(base + 0) * 64 + l] = make_float4(accQd[0], accQd[1], accQd[2], accQd[3]);
#pragma unroll
        for (int I = 0; I < NB - 1; ++I) {
          if (I < eR) {
            sPT[(base + 2 + 2 * I) * 64 + l] = make_float4(accQo[I][0], accQo[I][1], accQo[I][2], accQo[I][3]);
            sPT[(base + 3 + 2 * I) * 64 + l] = make_float4(accKo[I][0], accKo[I][1], accKo[I][2], accKo[I][3]);
          }
        }
      } else {
        sPT[(base + 1) * 64 + l] = make_float4(accKd[0], accKd[1], accKd[2], accKd[3]);
      }
    }
    load_qk1(k, gbuf.k, c_begin + C, chunk_len(ch + 1));
    __syncthreads();  // ------------------------------------------------------------- B_b

    // ===== Gram reduction by one wave of each row block, in parallel with the inverse of
    //       that block's diagonal sub-block of A by the other =====
    if (e_act) {
      const int base = eR * (eR + 1);
      const float4 bet4 = *reinterpret_cast<const float4*>(sBE + 16 * eR + 4 * lg);
      const float bet[4] = {bet4.x, bet4.y, bet4.z, bet4.w};
      if (ep != inv_half(eR)) {
        const float4 pq = sPT[(base + 0) * 64 + l];
        accQd[0] += pq.x; accQd[1] += pq.y; accQd[2] += pq.z; accQd[3] += pq.w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ri = 4 * lg + i;
          const int r = 16 * eR + ri, cc = 16 * eR + lr;
          sAQ[r * LDC + cc] = cvt<T>(ri > lr ? accQd[i] : 0.f);
          if (ri == lr) sDQ[r] = accQd[i];
        }
#pragma unroll
        for (int I = 0; I < NB - 1; ++I) {
          if (I < eR) {
            const float4 xq = sPT[(base + 2 + 2 * I) * 64 + l], xk = sPT[(base + 3 + 2 * I) * 64 + l];
            accQo[I][0] += xq.x; accQo[I][1] += xq.y; accQo[I][2] += xq.z; accQo[I][3] += xq.w;
            accKo[I][0] += xk.x; accKo[I][1] += xk.y; accKo[I][2] += xk.z; accKo[I][3] += xk.w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ri = 4 * lg + i;
              sAQ[(16 * eR + ri) * LDC + 16 * I + lr] = cvt<T>(accQo[I][i]);
              sAO[(pair_index(eR, I) * 16 + ri) * L::AOR + lr] = bet[i] * accKo[I][i];
            }
          }
        }
      } else {
        const float4 pk = sPT[(base + 1) * 64 + l];
        accKd[0] += pk.x; accKd[1] += pk.y; accKd[2] += pk.z; accKd[3] += pk.w;
        // A_RR (strict lower, rows scaled by beta), row-major into the diagonal tile of the
        // A/T region; each lane then reads back one row (one wave's LDS operations complete
        // in order, so no barrier is needed).
        float* blk = sAK + 16 * eR * LDA + 16 * eR;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * lg + u;
          blk[r * LDA + lr] = r > lr ? bet[u] * accKd[u] : 0.f;
        }
        __builtin_amdgcn_wave_barrier();  // the rows read below were written by other lanes
        float ar[16];  // A[lr][0..15]
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = *reinterpret_cast<const float4*>(blk + lr * LDA + 4 * q4);
          ar[4 * q4] = v4.x; ar[4 * q4 + 1] = v4.y; ar[4 * q4 + 2] = v4.z; ar[4 * q4 + 3] = v4.w;
        }
        // T_RR = (I + A_RR)^-1 by right-looking forward substitution over its rows: lane
        // (row r = lane & 15, group g) holds T[r][4g .. 4g+3].  Row i is final once pivots
        // < i are folded in; it reaches every lane of the 16-lane row through a DPP row
        // broadcast from lane i, and A[r][i] = 0 for r <= i, so the update needs no mask.
        float xr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xr[u] = (lr == 4 * lg + u) ? 1.f : 0.f;
        static_for<0, 15>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
#pragma unroll
          for (int u = 0; u < 4; ++u) xr[u] -= ar[i] * row_bcast16<i>(xr[u]);
        });
        // T_RR row-major over A (all reads of A precede these writes)
        store4(blk + lr * LDA + 4 * lg, xr[0], xr[1], xr[2], xr[3]);
      }
    }
    load_la(c_begin + C, chunk_len(ch + 1));
    __syncthreads();  // ------------------------------------------------------------- B_c
    load_vb(c_begin + C, chunk_len(ch + 1));

    // ===== T off-diagonal blocks, one block column per wave (wave I): for R = I+1 .. NB-1,
    //       T_RI = -T_RR sum_{J=I}^{R-1} A_RJ T_JI, with T_JI (J > I) kept in registers.
    //       The accumulator layout of a 16x16 fp32 MFMA tile is the B-operand layout
    //       (k = 4*(lane>>4) + i), so results feed the next block without LDS. =====
    if (wave < NB - 1) {
      const int kq = 4 * lg;
      const float bcol = sBE[16 * wave + lr];
#pragma unroll
      for (int I0 = 0; I0 < NB - 1; ++I0) {
        if (I0 == wave) {
          // operands first: T_II, T_RR and A_RJ for I0 <= J < R
          float tb[NB][4];
#pragma unroll
          for (int u = 0; u < 4; ++u) tb[I0][u] = sAK[(16 * I0 + kq + u) * LDA + 16 * I0 + lr];
          float4 a[NB][NB], tr[NB];
#pragma unroll
          for (int R = I0 + 1; R < NB; ++R) {
            tr[R] = *reinterpret_cast<const float4*>(sAK + (16 * R + lr) * LDA + 16 * R + kq);
#pragma unroll
            for (int J = I0; J < R; ++J)
              a[R][J] = *reinterpret_cast<const float4*>(sAO + (pair_index(R, J) * 16 + lr) * L::AOR + kq);
          }
          // one accumulator per term A_RJ T_JI: the J = I0 terms of every R start at once,
          // and each later term waits only for its own T_JI
          f32x4 Xp[NB][NB];
          // one 16x16x16 product: fp16 operands for bf16 inputs (rounding at the level of the
          // fp16 T Diag(beta) the WY products use anyway), four fp32 steps for fp32 inputs
          auto prod = [&](const float4& x, const float (&y)[4]) {
            f32x4 acc = zero4();
            if constexpr (P == Prec::Mixed) {
              const half4 xh = {(_Float16)x.x, (_Float16)x.y, (_Float16)x.z, (_Float16)x.w};
              const half4 yh = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
              acc = __builtin_amdgcn_mfma_f32_16x16x16f16(xh, yh, acc, 0, 0, 0);
            } else {
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, y[0], acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, y[1], acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, y[2], acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, y[3], acc, 0, 0, 0);
            }
            return acc;
          };
          auto term = [&](int R, int J) { return prod(a[R][J], tb[J]); };
#pragma unroll
          for (int R = I0 + 1; R < NB; ++R) Xp[R][I0] = term(R, I0);
#pragma unroll
          for (int R = I0 + 1; R < NB; ++R) {
#pragma unroll
            for (int J = I0 + 1; J < R; ++J) Xp[R][J] = term(R, J);
            f32x4 X = Xp[R][I0];
#pragma unroll
            for (int J = I0 + 1; J < R; ++J) X += Xp[R][J];
            const float xv[4] = {X[0], X[1], X[2], X[3]};
            const f32x4 Y = prod(tr[R], xv);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              tb[R][i] = -Y[i];
              sTB[(16 * R + kq + i) * LDC + 16 * I0 + lr] = cvt<T>(-Y[i] * bcol);
            }
          }
        }
      }
    }
    if (wave >= NB - 1) {
      // the other waves: Y = V - Kg S (does not need T), T Diag(beta) on the diagonal
      // blocks, zero upper tiles and padding
      constexpr int NH = NW - (NB - 1);
      const int hw = wave - (NB - 1);
      // Y tile (R, j): lane (token 16R + (l & 15), columns 16j + 4 (l >> 4) .. +3), stored
      // transposed (token contiguous) as the operand of U = T Diag(beta) Y.  With even tile
      // counts a wave takes a 2x2 block of tiles, so each operand fragment feeds two products.
      auto y_store = [&](int R, int j, const f32x4& ks) {
        if constexpr (kRanged) {
#pragma clang fp contract(off)
          // v (bf16 in LDS) in the chunk's scaled units; Y rounded to fp32, then to fp16 (no
          // fused multiply-add: the product is exact, and one rounding straight to fp16 is
          // what contraction would give)
          const uint2 w = *reinterpret_cast<const uint2*>(sV + (16 * R + lr) * LDV + 16 * j + 4 * lg);
          const float2 v01 = bf16x2_to_f32x2(w.x), v23 = bf16x2_to_f32x2(w.y);
          const float vv[4] = {v01.x, v01.y, v23.x, v23.y};
#pragma unroll
          for (int i = 0; i < 4; ++i) sYT[(16 * j + 4 * lg + i) * LDC + 16 * R + lr] = (T)(vv[i] * sc_dn - ks[i]);
        } else {
          const float4 v4 = load4(sV + (16 * R + lr) * LDV + 16 * j + 4 * lg);
          const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) sYT[(16 * j + 4 * lg + i) * LDC + 16 * R + lr] = cvt<T>(vv[i] - ks[i]);
        }
      };
      if constexpr (PREP) {
        // no state here: Y is formed by the state kernel
      } else if constexpr (NB % 2 == 0 && NJ % 2 == 0) {
        constexpr int NYB = (NB / 2) * (NJ / 2);
        static_for<0, (NYB + NH - 1) / NH>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          const int id = hw + NH * s;
          if (NYB % NH == 0 || id < NYB) {
            const int R0 = 2 * (id % (NB / 2)), j0 = 2 * (id / (NB / 2));
            f32x4 ks[2][2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
              for (int b = 0; b < 2; ++b) ks[a][b] = zero4();
            const T* pa = sST + (16 * j0 + lr) * LDD + lg * (KS / 4);
            const T* pb = sKG + (16 * R0 + lr) * LDD + lg * (KS / 4);
#pragma unroll
            for (int st = 0; st < DK / KS; ++st) {
              const auto a0 = ld_frag(pa + st * KS), a1 = ld_frag(pa + 16 * LDD + st * KS);
              const auto b0 = ld_frag(pb + st * KS), b1 = ld_frag(pb + 16 * LDD + st * KS);
              mma_frag(ks[0][0], a0, b0);
              mma_frag(ks[0][1], a0, b1);
              mma_frag(ks[1][0], a1, b0);
              mma_frag(ks[1][1], a1, b1);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
              for (int b = 0; b < 2; ++b) y_store(R0 + b, j0 + a, ks[a][b]);
          }
        });
      } else {
        static_for<0, (NB * NJ + NH - 1) / NH>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          const int id = hw + NH * s;
          if ((NB * NJ) % NH == 0 || id < NB * NJ) {
            const int R = id % NB, j = id / NB;
            f32x4 ks = zero4();
            mma_lds<T, KS, DK / KS>(ks, sST + 16 * j * LDD, LDD, sKG + 16 * R * LDD, LDD);
            y_store(R, j, ks);
          }
        });
      }
      for (int idx = hw * kWave + l; idx < C * 4; idx += NH * kWave) {
        const int r = idx >> 2, c = 16 * (r >> 4) + 4 * (idx & 3);  // 4 columns of row r's diagonal block
        const float4 tv = *reinterpret_cast<const float4*>(sAK + r * LDA + c);
        const float4 bv = *reinterpret_cast<const float4*>(sBE + c);
        store4(sTB + r * LDC + c, tv.x * bv.x, tv.y * bv.y, tv.z * bv.z, tv.w * bv.w);
      }
      // strictly-upper tiles (Tb shares memory with the partial tiles)
      for (int t = hw; t < NPAIR; t += NH) {
        int I = 1;
        while (I * (I + 1) / 2 <= t) ++I;
        const int R = t - I * (I - 1) / 2;  // upper tile (row block R, column block I > R)
        store4(sTB + (16 * R + (l >> 2)) * LDC + 16 * I + 4 * (l & 3), 0.f, 0.f, 0.f, 0.f);
      }
      if constexpr (CK > C) {
        // padded token columns of Kd^T, Y^T, U^T and Tb (Y^T shares memory with the right
        // base, U^T and Tb with the partials)
        for (int idx = hw * kWave + l; idx < (DK + 2 * BV + C) * (CK - C); idx += NH * kWave) {
          const int rowi = idx / (CK - C), col = C + idx % (CK - C);
          T* base = rowi < DK            ? sKDT + rowi * LDC
                    : rowi < DK + BV     ? sYT + (rowi - DK) * LDC
                    : rowi < DK + 2 * BV ? sUT + (rowi - DK - BV) * LDC
                                         : sTB + (rowi - DK - 2 * BV) * LDC;
          base[col] = cvt<T>(0.f);
        }
      }
    }
    // first part of the next chunk's gate stage (writes only BH, read after the next barrier)
    if constexpr (GH > 1) gate_part(std::integral_constant<int, 0>{});
    __syncthreads();  // ------------------------------------------------------------- B_e

    if constexpr (PREP) {
      // the chunk's state-free operands to its workspace slot, beside the next gate stage
      write_ws(ch);
      gate_part(std::integral_constant<int, GH - 1>{});  // the only part when GH == 1
      gate_v();
      __syncthreads();  // (prep) the right base is stored after this barrier
      store_rb();
      if (lane_id() == 0) sMX[2 * NW + wave0] = wide_ext;
    } else {
      // ================= U = Tb Y ; O = Qg S ; next chunk's gate stage =================
      // The products are issued first; the next chunk's gate stage (vector ALU) runs while
      // they complete.  It writes V, BH and beta, none of which is read after the barrier
      // above; the loads it consumes were issued two stages ago.
      f32x4 Uacc[U_SLOTS], Oacc[U_SLOTS];
      static_for<0, U_SLOTS>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int steps = UO_SPLIT ? ((32 * (s + 1) + KS - 1) / KS < CK / KS ? (32 * (s + 1) + KS - 1) / KS : CK / KS)
                                       : CK / KS;
        const int id = wave + NW * s;
        Uacc[s] = zero4();
        Oacc[s] = zero4();
        if ((NB * NJ) % NW == 0 || id < NB * NJ) {
          int R, j;
          uo_tile(s, R, j);
          mma_lds<T, KS, steps>(Uacc[s], sYT + 16 * j * LDC, LDC, sTB + 16 * R * LDC, LDC);
          mma_lds<T, KS, DK / KS>(Oacc[s], sST + 16 * j * LDD, LDD, sQG + 16 * R * LDD, LDD);
        }
      });
      gate_part(std::integral_constant<int, GH - 1>{});  // the only part when GH == 1
      gate_v();
  #pragma unroll
      for (int s = 0; s < U_SLOTS; ++s) {
        const int id = wave + NW * s;
        if ((NB * NJ) % NW == 0 || id < NB * NJ) {
          int R, j;
          uo_tile(s, R, j);
  #pragma unroll
          for (int i = 0; i < 4; ++i) sUT[(16 * j + 4 * lg + i) * LDC + 16 * R + lr] = cvt<T>(Uacc[s][i]);
        }
      }
      __syncthreads();  // ------------------------------------------------------------- B_f
      store_rb();

      // ================= O += M U ; S <- e^{g} S + Kd^T U =================
      static_for<0, U_SLOTS>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int steps = UO_SPLIT ? ((32 * (s + 1) + KS - 1) / KS < CK / KS ? (32 * (s + 1) + KS - 1) / KS : CK / KS)
                                       : CK / KS;
        const int id = wave + NW * s;
        if ((NB * NJ) % NW == 0 || id < NB * NJ) {
          int R, j;
          uo_tile(s, R, j);
          mma_lds<T, KS, steps>(Oacc[s], sUT + 16 * j * LDC, LDC, sAQ + 16 * R * LDC, LDC);
          const float dq = sDQ[16 * R + lr];
  #pragma unroll
          for (int i = 0; i < 4; ++i) Opend[s][i] = (Oacc[s][i] + dq * Uacc[s][i]) * (kRanged ? sc_up : 1.f);
        }
      });
  #pragma unroll
      for (int s = 0; s < S_SLOTS; ++s) {
        const int id = wave + NW * s;
        if ((NA * NJ) % NW == 0 || id < NA * NJ) {
          const int a = id % NA, j = id / NA;
  #pragma unroll
          for (int i = 0; i < 4; ++i) Sacc[s][i] *= sGM[16 * a + 4 * lg + i];
          mma_lds<T, KS, CK / KS>(Sacc[s], sKDT + 16 * a * LDC, LDC, sUT + 16 * j * LDC, LDC);
        }
      }
      o_begin = c_begin;
      o_len = Lc;
      store_pending();
      publish_range();
      if (lane_id() == 0) sMX[2 * NW + wave0] = wide_ext;
      // prefix-cache checkpoint: the state after p tokens of this sequence, p a multiple of
      // ckpt_every, goes to slot (sequence start + p) / ckpt_every - 1 (distinct for every
      // checkpoint of every packed sequence)
      if (ckpt && (c_begin + Lc - t_begin) % ckpt_every == 0) {
        const int64_t slot = (c_begin + Lc) / ckpt_every - 1;
        store_state(ckpt + ((size_t)slot * H + h) * DK * DV);
      }
    }
  }

  if (!PREP && hT) store_state(hT + (size_t)chain * DK * DV);
}

// ---------------------------------------------------------------------------
// State-only kernel of the split path.  Per (sequence, head, value tile) it walks the
// chunks in order with the fp32 master state in accumulator registers:
//   Y = V - Kg S,  U = (T Diag beta) Y,  O = Qg S + M U + diag(q.k) U,  S <- Diag(gamma) S + Kd^T U,
// reading each chunk's state-free operands from the workspace tile the prep pass wrote.
// Those operands go from memory straight into the registers of the matrix-core products
// (each wave loads the fragments of its own row blocks, one chunk ahead, right after the
// products of this chunk that used the same registers); only the operands that depend on
// the state (S^T, Y^T, U^T) pass through LDS.  Three barriers per chunk; the values go
// from memory straight to registers in the layout of the Y product.  Each fragment is
// loaded by exactly one wave (see the wave roles below): the vector memory path of the CU,
// not its matrix cores, bounds this loop.
// ---------------------------------------------------------------------------
template <int C, int DK, int BV>
struct SLay {
  static constexpr int KS = 32, PD = 8, NB = C / 16;
  static constexpr int CK = WsTile<C, DK>::CK;
  static constexpr int LDD = DK + PD, LDC = CK + PD;
  static constexpr size_t ST = 0;                                   // S^T [BV][LDD]
  static constexpr size_t YT = ST + al16(size_t(BV) * LDD * 2);     // Y^T [BV][LDC]
  static constexpr size_t UT = YT + al16(size_t(BV) * LDC * 2);     // U^T [BV][LDC]
  static constexpr size_t MX = UT + al16(size_t(BV) * LDC * 2);     // per-wave largest |S|, |v| [NW]
  static constexpr size_t TOTAL = MX + al16(size_t(NW) * 4);
};

// The row-role state pass (the non-pipelined split path's; the pipelined and segmented forms
// run chunk_state_wave_body below, which takes the same job).
// Chunks [job.ch_begin, job.ch_end) of one chain (clipped to its length), value columns
// job.j0 .. + BV.  The state enters from job.s_in (or zeros) and leaves to job.end_out when the
// chain's last chunk is in the range, else to job.mid_out (either may be null: not stored).
// Segment-map mode (job.map) runs the same recurrence on a DK x (DK + DV) state whose first DK
// columns start at the identity with zero values and whose last DV start at zero with the
// chain's values (state column j0 >= DK is value column j0 - DK): its final state [M | B] is
// the range's affine map S_out = M S_in + B.  It writes no o, and a range that reaches the
// chain's end (whose map no later range needs) does nothing.
template <int C, int DK, int BV, typename InT>
__device__ __forceinline__ void chunk_state_body(
    const uint4* __restrict__ ws, const InT* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
    float* __restrict__ o, int H, int DV, int64_t seq_len, const StateJob& job) {
  using L = SLay<C, DK, BV>;
  using W = WsTile<C, DK>;
  using T = _Float16;
  constexpr int NB = L::NB, LDD = L::LDD, LDC = L::LDC, NSD = W::NSD, NSC = W::NSC;
  constexpr int NA = DK / 16, NJ = BV / 16;
  static_assert(sizeof(InT) == 2, "bf16 values");
  static_assert(NW % NA == 0, "the state tiles of a wave share one row block of Kd^T");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sST = reinterpret_cast<T*>(smem + L::ST);
  T* sYT = reinterpret_cast<T*>(smem + L::YT);
  T* sUT = reinterpret_cast<T*>(smem + L::UT);
  uint32_t* sMX = reinterpret_cast<uint32_t*>(smem + L::MX);

  const int chain = job.chain, j0 = job.j0;
  const int64_t ch_begin = job.ch_begin, ch_end = job.ch_end;
  const int n = chain / H, h = chain - n * H;
  // value column of the tile (map mode: none for the identity columns)
  const int vj0 = job.map ? (j0 >= DK ? j0 - DK : -1) : j0;
  int64_t t_begin, t_end;
  if (cu_seqlens) {
    t_begin = cu_seqlens[n];
    t_end = cu_seqlens[n + 1];
  } else {
    t_begin = (int64_t)n * seq_len;
    t_end = t_begin + seq_len;
  }
  const int64_t nchunks = (t_end - t_begin + C - 1) / C;
  if (ch_begin > 0 && ch_begin >= nchunks) return;  // the chain ended in an earlier range
  const int64_t ch_stop = ch_end < nchunks ? ch_end : nchunks;
  if (job.map && ch_stop == nchunks) return;        // no later range of the chain needs this map
  auto chunk_len = [&](int64_t ch) -> int {
    const int64_t rem = t_end - (t_begin + ch * C);
    return (int)(rem < C ? rem : C);
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = lane_id(), lr = l & 15, lg = l >> 4;

  // zero once: the padded token columns (C .. CK) of Y^T and U^T stay zero
  for (int i = tid; i < int(L::TOTAL / 16); i += NT) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);

  constexpr int S_SLOTS = (NA * NJ + NW - 1) / NW;
  f32x4 Sacc[S_SLOTS];
  const float* h0p = (!job.map && job.s_in) ? job.s_in + (size_t)chain * DK * DV : nullptr;
  auto s_active = [&](int s) { return (NA * NJ) % NW == 0 || wave + NW * s < NA * NJ; };
  const int sa = wave % NA;  // row block of every state tile of this wave: tile (sa, (wave + NW s) / NA)
#pragma unroll
  for (int s = 0; s < S_SLOTS; ++s) {
    const int j = (wave + NW * s) / NA;
    Sacc[s] = zero4();
    if (s_active(s) && h0p) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Sacc[s][i] = h0p[(size_t)(16 * sa + 4 * lg + i) * DV + j0 + 16 * j + lr];
    }
    if (s_active(s) && job.map) {  // the identity in the map's first DK columns
#pragma unroll
      for (int i = 0; i < 4; ++i) Sacc[s][i] = (16 * sa + 4 * lg + i == j0 + 16 * j + lr) ? 1.f : 0.f;
    }
  }
  // The 16-bit state copy.  The fp32 state is held in the chunk's scaled units 2^-e (see
  // range_exponent); o, hT and the hand-over state are scaled back by 2^e.
  auto write_ST = [&]() {
#pragma unroll
    for (int s = 0; s < S_SLOTS; ++s)
      if (s_active(s)) {
        const int j = (wave + NW * s) / NA;
        store4(sST + (16 * j + lr) * LDD + 16 * sa + 4 * lg, Sacc[s][0], Sacc[s][1], Sacc[s][2], Sacc[s][3]);
      }
  };
  auto store_state = [&](float* sp, int ld, float f) {
#pragma unroll
    for (int s = 0; s < S_SLOTS; ++s)
      if (s_active(s)) {
        const int j = (wave + NW * s) / NA;
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[(size_t)(16 * sa + 4 * lg + i) * ld + j0 + 16 * j + lr] = Sacc[s][i] * f;
      }
  };

  // Wave roles: wave R < NB (an "O wave") owns token row block R of Qg S, U and O over all
  // NJ value tiles; wave NB + R (a "K wave") owns row block R of Kg S and Y.  Every operand
  // fragment of the workspace tile is then loaded by one wave only.
  static_assert(2 * NB <= NW, "two waves per token row block");
  const bool o_wave = wave < NB, k_wave = wave >= NB && wave < 2 * NB;
  const int R = o_wave ? wave : wave - NB;
  const int tri = (16 * R + 15) / 32 + 1;  // k-steps of T Diag(beta) and M that reach row block R

  // ---- the chunk's operand fragments, loaded into the registers of the products: Qg (O
  // waves) or Kg (K waves) rows of block R; T Diag(beta), M and q.k rows of block R (O waves);
  // Kd^T rows of block sa and e^{g_last} (every wave with a state tile).
  // Every wave issues the same memory instructions in the same order; an access a wave does
  // not need goes through a descriptor of no bytes (or past its end) and returns zero without
  // touching memory, and a store there is dropped.  The memory counter then has one count on
  // every path, so each wait covers exactly the loads of the chunk before.  Each load group is
  // fenced off from the instruction scheduler (sched_barrier 0 before and after it), so the
  // loads are issued where they are written, each right after the last use of its registers:
  // left free, the scheduler gathers them ahead of the barriers and the products then wait on
  // more of the memory counter than their own operands (1M tokens x 32 heads: 38.5 -> 35.7 ms).
  half8 gq[NSD], tb[NSC], aq[NSC], kdt[NSC];
  float dq = 0.f;
  float4 gm = make_float4(0.f, 0.f, 0.f, 0.f);
  auto tile_rsrc = [&](int64_t chn, bool mine) {
    const bool ok = chn < ch_stop && mine;
    const int64_t slot = t_begin / C + n + chn;
    return make_rsrc(ws + ((size_t)(chn < ch_stop ? slot : 0) * H + h) * W::NU, ok ? (uint32_t)W::NU * 16u : 0u);
  };
  auto frag = [&](__amdgpu_buffer_rsrc_t rs, int region, int f) {
    return __builtin_bit_cast(half8, buf_load16(rs, (uint32_t)(region + 64 * f + l) * 16u));
  };
  constexpr uint32_t kPast = 0x7ffffff0u;  // an offset past the end of any tile
  const int Rl = (o_wave || k_wave) ? R : 0;
  auto load_gq = [&](int64_t chn) {
    __builtin_amdgcn_sched_barrier(0);
    const auto rs = tile_rsrc(chn, o_wave || k_wave);
    const int region = o_wave ? W::QG : W::KG;
#pragma unroll
    for (int st = 0; st < NSD; ++st) gq[st] = frag(rs, region, Rl * NSD + st);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_tb = [&](int64_t chn) {
    __builtin_amdgcn_sched_barrier(0);
    const auto rs = tile_rsrc(chn, o_wave);
#pragma unroll
    for (int st = 0; st < NSC; ++st)
      tb[st] = __builtin_bit_cast(half8, buf_load16(rs, st < tri ? (uint32_t)(W::TB + 64 * (W::tri_base(Rl) + st) + l) * 16u : kPast));
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_aq = [&](int64_t chn) {
    __builtin_amdgcn_sched_barrier(0);
    const auto rs = tile_rsrc(chn, o_wave);
#pragma unroll
    for (int st = 0; st < NSC; ++st)
      aq[st] = __builtin_bit_cast(half8, buf_load16(rs, st < tri ? (uint32_t)(W::AQ + 64 * (W::tri_base(Rl) + st) + l) * 16u : kPast));
    dq = buf_load4(rs, (uint32_t)W::DQ * 16u + (uint32_t)(16 * Rl + lr) * 4u);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_kd = [&](int64_t chn) {
    __builtin_amdgcn_sched_barrier(0);
    const auto rs = tile_rsrc(chn, s_active(0));
#pragma unroll
    for (int st = 0; st < NSC; ++st) kdt[st] = frag(rs, W::KDT, sa * NSC + st);
    gm = __builtin_bit_cast(float4, buf_load16(rs, (uint32_t)W::GM * 16u + (uint32_t)(16 * sa + 4 * lg) * 4u));
    __builtin_amdgcn_sched_barrier(0);
  };
  // (every wave issues the loads; the descriptor of a wave other than a K wave has no bytes, so
  // its loads return zeros without touching memory and need no branch)
  uint2 vnx[NJ];
  auto load_v = [&](int64_t chn) {
    __builtin_amdgcn_sched_barrier(0);
    const bool ok = chn < ch_stop;
    const int Lc = ok ? chunk_len(chn) : 0;
    const auto rv = make_rsrc(v + ((size_t)(t_begin + (ok ? chn : 0) * C) * H + h) * DV + (vj0 >= 0 ? vj0 : 0),
                              (k_wave && Lc > 0 && vj0 >= 0) ? (uint32_t)Lc * (uint32_t)(H * DV * 2) : 0u);
    const int Rv = k_wave ? R : 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      typedef int i32x2 __attribute__((ext_vector_type(2)));
      const i32x2 x = __builtin_amdgcn_raw_buffer_load_b64(
          rv, (int)(((uint32_t)(16 * Rv + lr) * (uint32_t)(H * DV) + (uint32_t)(16 * j + 4 * lg)) * 2u), 0, 0);
      vnx[j] = make_uint2((uint32_t)x[0], (uint32_t)x[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int sc_e = 0;
  float sc_dn = 1.f, sc_up = 1.f;
  // largest |S| and |v| of the next chunk (in the chunk's scaled units) over the wave, to LDS
  auto publish_range = [&]() {
    uint32_t w[2 * NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      w[2 * j] = vnx[j].x;
      w[2 * j + 1] = vnx[j].y;
    }
    const uint32_t mv = mag_max_bf16(w, 2 * NJ);
    float sv[4 * S_SLOTS];
#pragma unroll
    for (int s = 0; s < S_SLOTS; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * s + i] = s_active(s) ? Sacc[s][i] : 0.f;
    uint32_t m = max(mag_max<4 * S_SLOTS>(sv), sc_e == 0 ? mv : mag_scaled(mv, sc_e));
    m = wave_max_u32(m);
    if (l == 0) sMX[wave] = m;
  };
  // after the barrier that follows publish_range: the next chunk's range exponent from every
  // wave's figure.  When it changes (rarely) the held state is rescaled to the new units and
  // its 16-bit copy, already written in the old units, is written again.
  auto settle_range = [&]() {
    static_assert(NW == 8, "16-byte reads of the per-wave maxima");
    const uint4 a0 = *reinterpret_cast<const uint4*>(sMX), a1 = *reinterpret_cast<const uint4*>(sMX + 4);
    const uint32_t m = max(max(max(a0.x, a0.y), max(a0.z, a0.w)), max(max(a1.x, a1.y), max(a1.z, a1.w)));
    const int e = range_exponent(__builtin_amdgcn_readfirstlane(m), sc_e);
    if (e != sc_e) {
      const int d = sc_e - e, d1 = d / 2;
      const float f1 = pow2i(d1), f2 = pow2i(d - d1);
#pragma unroll
      for (int s = 0; s < S_SLOTS; ++s) Sacc[s] = (Sacc[s] * f1) * f2;
      sc_e = e;
      sc_dn = pow2i(-e);
      sc_up = pow2i(e);
      write_ST();
      __syncthreads();
    }
  };

  load_gq(ch_begin);
  load_tb(ch_begin);
  load_aq(ch_begin);
  load_kd(ch_begin);
  load_v(ch_begin);
  __syncthreads();  // zero fill before the first state copy
  write_ST();
  publish_range();
  __syncthreads();
  settle_range();

  // acc: Qg S, then O (O waves) or Kg S (K waves); Uacc: U (O waves)
  f32x4 acc[NJ], Uacc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = Uacc[j] = zero4();
  for (int64_t ch = ch_begin; ch < ch_stop; ++ch) {
    const int64_t c_begin = t_begin + ch * C;
    const int Lc = chunk_len(ch);
    // this chunk's values (loaded during the previous chunk); the next chunk's are loaded now
    uint2 vcur[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) vcur[j] = vnx[j];
    load_v(ch + 1);

    // Qg S (O waves) or Kg S (K waves), then Y = V - Kg S (to Y^T)
    if (o_wave || k_wave) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = zero4();
#pragma unroll
      for (int st = 0; st < NSD; ++st)
#pragma unroll
        for (int j = 0; j < NJ; ++j) mma_frag(acc[j], ld_frag(sST + (16 * j + lr) * LDD + 8 * lg + 32 * st), gq[st]);
    }
    load_gq(ch + 1);
    if (k_wave) {
#pragma clang fp contract(off)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float2 v01 = bf16x2_to_f32x2(vcur[j].x), v23 = bf16x2_to_f32x2(vcur[j].y);
        const float vv[4] = {v01.x, v01.y, v23.x, v23.y};
        // rounded to fp32, then to fp16, as in the fused forward (not in one step)
#pragma unroll
        for (int i = 0; i < 4; ++i) sYT[(16 * j + 4 * lg + i) * LDC + 16 * R + lr] = (T)(vv[i] * sc_dn - acc[j][i]);
      }
    }
    __syncthreads();

    // U = (T Diag beta) Y (to U^T)
    if (o_wave) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) Uacc[j] = zero4();
#pragma unroll
      for (int st = 0; st < NSC; ++st)
        if (st < tri) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) mma_frag(Uacc[j], ld_frag(sYT + (16 * j + lr) * LDC + 8 * lg + 32 * st), tb[st]);
        }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) sUT[(16 * j + 4 * lg + i) * LDC + 16 * R + lr] = (T)Uacc[j][i];
    }
    load_tb(ch + 1);
    __syncthreads();

    // O = Qg S + M U + diag(q.k) U, stored (O waves); S <- Diag(gamma) S + Kd^T U (in the
    // chunk's scaled units)
    if (o_wave) {
#pragma unroll
      for (int st = 0; st < NSC; ++st)
        if (st < tri) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) mma_frag(acc[j], ld_frag(sUT + (16 * j + lr) * LDC + 8 * lg + 32 * st), aq[st]);
        }
    }
    {
      // o rows of the chunk (O waves; a store past the chunk's rows, or by another wave, is dropped)
      const uint32_t hdv = (uint32_t)(H * DV);
      const auto ro = job.map ? make_rsrc(o, 0u)
                              : make_rsrc(o + ((size_t)c_begin * H + h) * DV + j0, o_wave ? (uint32_t)Lc * hdv * 4u : 0u);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));
        f32x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = (acc[j][i] + dq * Uacc[j][i]) * sc_up;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4s, ov), ro,
                                               (int)(((uint32_t)(16 * Rl + lr) * hdv + (uint32_t)(16 * j + 4 * lg)) * 4u),
                                               0, 0);
      }
    }
    load_aq(ch + 1);
#pragma unroll
    for (int s = 0; s < S_SLOTS; ++s) {
      if (s_active(s)) {
        const int j = (wave + NW * s) / NA;
        Sacc[s][0] *= gm.x;
        Sacc[s][1] *= gm.y;
        Sacc[s][2] *= gm.z;
        Sacc[s][3] *= gm.w;
        const T* pb = sUT + (16 * j + lr) * LDC + 8 * lg;
#pragma unroll
        for (int st = 0; st < NSC; ++st) mma_frag(Sacc[s], kdt[st], ld_frag(pb + 32 * st));
      }
    }
    load_kd(ch + 1);
    // S^T for the next chunk: every read of this chunk's S^T was before the first barrier
    write_ST();
    publish_range();
    __syncthreads();  // S^T, every read of Y^T / U^T and the per-wave maxima
    settle_range();
  }
  if (ch_stop == nchunks) {
    if (job.end_out) store_state(job.end_out + (size_t)chain * DK * DV, DV, sc_up);
  } else if (job.mid_out) {
    store_state(job.mid_out + (size_t)chain * DK * job.mid_ld, job.mid_ld, sc_up);
  }
}

// ---------------------------------------------------------------------------
// Wave-parallel state pass.  The value columns of the state are independent chains given the
// chunk's operands, so one wave can carry 16 of them through a whole chunk step on its own:
// in the 16x16 matrix-core layout a product's accumulator (lane (j, g): rows 4g .. 4g+3 of
// column j) is the B operand of the next product whose k runs over those rows, once each
// 32-wide k-step takes its 32 rows in the order {4g .. 4g+3 of the first 16-row block, then of
// the second} and the A operand (read from LDS) takes its columns in the same order.  So
//   S (channels x 16) -> Kg S, Qg S;  Y = V - Kg S -> U = (T Diag beta) Y -> M U, Kd^T U;
//   S' = Diag(gamma) S + Kd^T U;  O = Qg S + M U + diag(q.k) U
// run in one wave's registers with no exchange and no barrier inside the step.  NCW such
// waves take 16 NCW columns of one chain and load their values straight from memory, one
// chunk ahead; the other NW - NCW waves of the workgroup stage each chunk's workspace tile in
// LDS (two buffers, loaded two chunks ahead through two register sets), and all waves meet at
// one barrier per chunk.  The operand precisions and
// rounding points are the split path's (fp16 operands, fp32 accumulation; Y rounded to fp32,
// then to fp16); the range exponent (see range_exponent) is taken per wave, over its columns.
// ---------------------------------------------------------------------------
template <int C, int DK, int NCW>
struct WLay {
  using W = WsTile<C, DK>;
  static constexpr int WBV = 16 * NCW;                       // value columns per workgroup
  static constexpr size_t TILE = al16(size_t(W::NU) * 16);
  static constexpr size_t T0 = 0, T1 = T0 + TILE;
  static constexpr size_t TOTAL = T1 + TILE;
};

// The A operand of one 32-wide k-step in the accumulator k order: lane (r, g) takes
// X[r][4g .. 4g+3] and X[r][16+4g .. 16+4g+3].  The workspace holds each fragment in the
// matrix core's own order (lane (r, g') of the stored fragment holds X[r][8g' .. 8g'+7]),
// so lane (r, g) needs half of stored unit (r, g >> 1) and half of unit (r, (g >> 1) + 2).
// The loader waves put them together when they stage a tile in LDS: from stored units
// (r, g') and (r, g' + 2) they write staged units (r, 2g') = both low halves and (r, 2g' + 1)
// = both high halves, so each compute lane reads its operand as 16 consecutive bytes (one
// conflict-free 128-bit LDS read; two 64-bit reads at a 16-byte lane stride hit each bank
// twice).
__device__ __forceinline__ void stage_pair(uint4* dst_lo, uint4* dst_hi, const uint4& n1, const uint4& n2) {
  *dst_lo = uint4{n1.x, n1.y, n2.x, n2.y};
  *dst_hi = uint4{n1.z, n1.w, n2.z, n2.w};
}
// The B operand of one 32-wide k-step from the accumulators of its two 16-row blocks.
__device__ __forceinline__ half8 pack_b(const f32x4& lo, const f32x4& hi) {
  return half8{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
               (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
}

// The A operands of one chunk step in the order of their products: Kg (k-step outer, row block
// inner: four independent accumulators in turn), T Diag(beta) (k-step outer), Kd^T (k-step
// outer, channel block inner), Qg, strict M.
template <int C, int DK>
struct WOrder {
  using W = WsTile<C, DK>;
  static constexpr int NB = W::NB, NSD = W::NSD, NSC = W::NSC, NCB = DK / 16;
  static constexpr int nA = NB * NSD, nB = W::NTRI, nC = NCB * NSC, nD = NB * NSD, nE = W::NTRI;
  static constexpr int NFR = nA + nB + nC + nD + nE;
  // (row block, k-step) of the j-th stored fragment of a lower-triangular token operand, k-step outer
  __host__ __device__ static constexpr int tri_pair(int j, bool st_of) {
    for (int st = 0; st < NSC; ++st)
      for (int R = 0; R < NB; ++R)
        if (st < W::tri(R)) {
          if (j == 0) return st_of ? st : R;
          --j;
        }
    return 0;
  }
  __host__ __device__ static constexpr int tri_R(int j) { return tri_pair(j, false); }
  __host__ __device__ static constexpr int tri_st(int j) { return tri_pair(j, true); }
  // first 16-byte unit of the k-th fragment
  __host__ __device__ static constexpr int unit(int k) {
    if (k < nA) return W::KG + 64 * ((k % NB) * NSD + k / NB);
    k -= nA;
    if (k < nB) return W::TB + 64 * (W::tri_base(tri_R(k)) + tri_st(k));
    k -= nB;
    if (k < nC) return W::KDT + 64 * ((k % NCB) * NSC + k / NCB);
    k -= nC;
    if (k < nD) return W::QG + 64 * ((k % NB) * NSD + k / NB);
    k -= nD;
    return W::AQ + 64 * (W::tri_base(tri_R(k)) + tri_st(k));
  }
};

template <int C, int DK, int NCW, typename InT>
__device__ __forceinline__ void chunk_state_wave_body(
    const uint4* __restrict__ ws, const InT* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
    float* __restrict__ o, int H, int DV, int64_t seq_len, const StateJob& job) {
  using L = WLay<C, DK, NCW>;
  using W = WsTile<C, DK>;
  using Ord = WOrder<C, DK>;
  constexpr int NB = W::NB, NSD = W::NSD, NSC = W::NSC, NCB = DK / 16;
  constexpr int kAhead = 8;  // fragments in flight
  constexpr int NL = NW - NCW, NLL = NL * kWave;
  // the tile's fragments [0, DQ) are staged in unit pairs (see stage_pair), the fp32 tail
  // (q.k, gamma) [DQ, NU) unit by unit
  constexpr int NPR = W::DQ / 2, NTL = W::NU - W::DQ;
  static_assert(W::DQ % 64 == 0, "whole fragments before the fp32 tail");
  constexpr int PPL = (NPR + NLL - 1) / NLL;    // unit pairs per loader lane
  constexpr int TLL = (NTL + NLL - 1) / NLL;    // tail units per loader lane
  constexpr int TPL = 2 * PPL + TLL;            // loaded 16-byte units per loader lane
  static_assert(sizeof(InT) == 2, "bf16 values");
  static_assert(NCW >= 1 && NCW < NW, "compute and loader waves");
  static_assert(2 * NSD == NCB && 2 * NSC >= NB, "k-steps pair 16-row blocks");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int chain = job.chain, j0 = job.j0;
  const int64_t ch_begin = job.ch_begin, ch_end = job.ch_end;
  const int n = chain / H, h = chain - n * H;
  const int vj0 = job.map ? (j0 >= DK ? j0 - DK : -1) : j0;  // first value column (-1: identity columns)
  int64_t t_begin, t_end;
  if (cu_seqlens) {
    t_begin = cu_seqlens[n];
    t_end = cu_seqlens[n + 1];
  } else {
    t_begin = (int64_t)n * seq_len;
    t_end = t_begin + seq_len;
  }
  const int64_t nchunks = (t_end - t_begin + C - 1) / C;
  if (ch_begin > 0 && ch_begin >= nchunks) return;  // the chain ended in an earlier range
  const int64_t ch_stop = ch_end < nchunks ? ch_end : nchunks;
  if (job.map && ch_stop == nchunks) return;        // no later range of the chain needs this map
  auto chunk_len = [&](int64_t ch) -> int {
    const int64_t rem = t_end - (t_begin + ch * C);
    return (int)(rem < C ? rem : C);
  };
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = lane_id(), lr = l & 15, lg = l >> 4;

  if (wave >= NCW) {
    // ================= loader waves =================
    const int li = tid - NCW * kWave;
    uint4 ra[TPL], rb[TPL];
    auto fetch = [&](int64_t chn, uint4* r) {
      const bool ok = chn < ch_stop;
      const int64_t slot = t_begin / C + n + chn;
      const auto rs = make_rsrc(ws + ((size_t)(ok ? slot : 0) * H + h) * W::NU, ok ? (uint32_t)W::NU * 16u : 0u);
#pragma unroll
      for (int m = 0; m < PPL; ++m) {
        // pair p: stored units (r, g') and (r, g' + 2) of fragment p / 32, r = p % 16, g' = (p / 16) % 2
        // (past the tile the loads return zero and the pair is not staged)
        const int p = li + NLL * m;
        const uint32_t u1 = (uint32_t)(64 * (p >> 5) + (p & 15) + 16 * ((p >> 4) & 1));
        r[2 * m] = buf_load16(rs, u1 * 16u);
        r[2 * m + 1] = buf_load16(rs, (u1 + 32u) * 16u);
      }
#pragma unroll
      for (int m = 0; m < TLL; ++m) r[2 * PPL + m] = buf_load16(rs, (uint32_t)(W::DQ + li + NLL * m) * 16u);
    };
    auto stage = [&](const uint4* r, int buf) {
      uint4* dt = reinterpret_cast<uint4*>(smem + (buf ? L::T1 : L::T0));
#pragma unroll
      for (int m = 0; m < PPL; ++m) {
        const int p = li + NLL * m;
        if (NPR % NLL == 0 || p < NPR) {
          const int d = 64 * (p >> 5) + (p & 15) + 32 * ((p >> 4) & 1);  // staged unit (r, 2g')
          stage_pair(dt + d, dt + d + 16, r[2 * m], r[2 * m + 1]);
        }
      }
#pragma unroll
      for (int m = 0; m < TLL; ++m) {
        const int u = li + NLL * m;
        if (NTL % NLL == 0 || u < NTL) dt[W::DQ + u] = r[2 * PPL + m];
      }
    };
    fetch(ch_begin, ra);
    stage(ra, 0);
    fetch(ch_begin + 1, rb);
    fetch(ch_begin + 2, ra);
    __syncthreads();  // buffer 0 holds the first chunk
    for (int64_t ch = ch_begin; ch < ch_stop; ch += 2) {
      // step ch: buffer 1 <- chunk ch + 1 (set b), then set b <- chunk ch + 3
      stage(rb, 1);
      fetch(ch + 3, rb);
      __syncthreads();
      if (ch + 1 >= ch_stop) break;
      // step ch + 1: buffer 0 <- chunk ch + 2 (set a), then set a <- chunk ch + 4
      stage(ra, 0);
      fetch(ch + 4, ra);
      __syncthreads();
    }
    return;
  }

  // ================= compute waves: columns j0 + 16 wave + (0 .. 15) =================
  const int col = j0 + 16 * wave + lr;        // state column of this lane
  const int vcol = vj0 >= 0 ? vj0 + 16 * wave : 0;  // first value column of this wave
  const int aoff = 16 * l;  // this lane's staged unit of a fragment
  f32x4 Sacc[NCB];
  const float* h0p = (!job.map && job.s_in) ? job.s_in + (size_t)chain * DK * DV : nullptr;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * cb + 4 * lg + i;
      Sacc[cb][i] = h0p ? h0p[(size_t)row * DV + col] : (job.map ? (row == col ? 1.f : 0.f) : 0.f);
    }
  }
  int sc_e = 0;
  float sc_dn = 1.f, sc_up = 1.f;
  // this wave's values of a chunk straight from memory, one chunk ahead: lane (lr, lg) takes
  // rows 16 R + 4 lg .. + 3 of column lr (rows past the chunk read as zero)
  uint2 vnx[NB];
  auto load_vw = [&](int64_t chn) {
    const bool ok = chn < ch_stop;
    const int Lc = ok ? chunk_len(chn) : 0;
    const uint32_t hdv = (uint32_t)(H * DV);
    const auto rv = make_rsrc(v + ((size_t)(t_begin + (ok ? chn : 0) * C) * H + h) * DV + (vj0 >= 0 ? vj0 + 16 * wave : 0),
                              (Lc > 0 && vj0 >= 0) ? (uint32_t)Lc * hdv * 2u : 0u);
#pragma unroll
    for (int R = 0; R < NB; ++R) {
      uint32_t e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        e[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rv, (int)(((uint32_t)(16 * R + 4 * lg + i) * hdv + (uint32_t)lr) * 2u), 0, 0);
      vnx[R] = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
    }
  };
  load_vw(ch_begin);
  __syncthreads();  // buffer 0 holds the first chunk
  for (int64_t ch = ch_begin; ch < ch_stop; ++ch) {
    const int p = (int)((ch - ch_begin) & 1);
    const unsigned char* tile = smem + (p ? L::T1 : L::T0);
    const int64_t c_begin = t_begin + ch * C;
    const int Lc = chunk_len(ch);

    // this chunk's values: rows 16 R + 4 lg .. + 3 of column lr (bf16 pairs)
    uint2 vv[NB];
#pragma unroll
    for (int R = 0; R < NB; ++R) vv[R] = vnx[R];
    load_vw(ch + 1);
    // the A operands of the step's products, kAhead products ahead of their use
    half8 fb[kAhead];
    auto fetch = [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k < Ord::NFR) fb[k % kAhead] = *reinterpret_cast<const half8*>(tile + 16 * Ord::unit(k) + aoff);
    };
    static_for<0, kAhead>(fetch);
    // the chunk's range exponent from the largest |S| and |v| of this wave's columns
    {
      uint32_t w[2 * NB];
#pragma unroll
      for (int R = 0; R < NB; ++R) {
        w[2 * R] = vv[R].x;
        w[2 * R + 1] = vv[R].y;
      }
      const uint32_t mv = mag_max_bf16(w, 2 * NB);
      float sv[4 * NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * cb + i] = Sacc[cb][i];
      const uint32_t m = wave_max_u32(max(mag_max<4 * NCB>(sv), sc_e == 0 ? mv : mag_scaled(mv, sc_e)));
      const int e = range_exponent(__builtin_amdgcn_readfirstlane(m), sc_e);
      if (e != sc_e) {
        const int d = sc_e - e, d1 = d / 2;
        const float f1 = pow2i(d1), f2 = pow2i(d - d1);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) Sacc[cb] = (Sacc[cb] * f1) * f2;
        sc_e = e;
        sc_dn = pow2i(-e);
        sc_up = pow2i(e);
      }
    }
    // S as the B operand of the products over channels
    half8 Sb[NSD];
#pragma unroll
    for (int st = 0; st < NSD; ++st) Sb[st] = pack_b(Sacc[2 * st], Sacc[2 * st + 1]);
    // product k of the step: its fragment is used, and the one kAhead later read into its
    // registers; the fence keeps the reads where they are written
    auto product = [&](auto kc, f32x4& d, const half8& b) {
      constexpr int k = decltype(kc)::value;
      mma_frag(d, fb[k % kAhead], b);
      fetch(std::integral_constant<int, k + kAhead>{});
      __builtin_amdgcn_sched_barrier(0);
    };

    // Kg S, then Y = V - Kg S
    f32x4 acc[NB];
#pragma unroll
    for (int R = 0; R < NB; ++R) acc[R] = zero4();
    static_for<0, Ord::nA>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      product(jc, acc[j % NB], Sb[j / NB]);
    });
    float4 gm[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) gm[cb] = *reinterpret_cast<const float4*>(tile + 16 * W::GM + 4 * (16 * cb + 4 * lg));
    f32x4 Y[2 * NSC];
#pragma unroll
    for (int R = 0; R < 2 * NSC; ++R) Y[R] = zero4();
    {
#pragma clang fp contract(off)
#pragma unroll
      for (int R = 0; R < NB; ++R) {
        const float2 v01 = bf16x2_to_f32x2(vv[R].x), v23 = bf16x2_to_f32x2(vv[R].y);
        const float x[4] = {v01.x, v01.y, v23.x, v23.y};
        // rounded to fp32 here, to fp16 in the operand
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[R][i] = x[i] * sc_dn - acc[R][i];
      }
    }
    half8 Yb[NSC];
#pragma unroll
    for (int st = 0; st < NSC; ++st) Yb[st] = pack_b(Y[2 * st], Y[2 * st + 1]);

    // U = (T Diag beta) Y
    f32x4 U[2 * NSC];
#pragma unroll
    for (int R = 0; R < 2 * NSC; ++R) U[R] = zero4();
    static_for<0, Ord::nB>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      product(std::integral_constant<int, Ord::nA + j>{}, U[Ord::tri_R(j)], Yb[Ord::tri_st(j)]);
    });
    float4 dq[NB];
#pragma unroll
    for (int R = 0; R < NB; ++R) dq[R] = *reinterpret_cast<const float4*>(tile + 16 * W::DQ + 4 * (16 * R + 4 * lg));
    half8 Ub[NSC];
#pragma unroll
    for (int st = 0; st < NSC; ++st) Ub[st] = pack_b(U[2 * st], U[2 * st + 1]);

    // S <- Diag(gamma) S + Kd^T U (in the chunk's scaled units)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      Sacc[cb][0] *= gm[cb].x;
      Sacc[cb][1] *= gm[cb].y;
      Sacc[cb][2] *= gm[cb].z;
      Sacc[cb][3] *= gm[cb].w;
    }
    static_for<0, Ord::nC>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      product(std::integral_constant<int, Ord::nA + Ord::nB + j>{}, Sacc[j % NCB], Ub[j / NCB]);
    });

    // O = Qg S + M U + diag(q.k) U, stored (map mode: no o)
    f32x4 O[NB];
#pragma unroll
    for (int R = 0; R < NB; ++R) O[R] = zero4();
    static_for<0, Ord::nD>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      product(std::integral_constant<int, Ord::nA + Ord::nB + Ord::nC + j>{}, O[j % NB], Sb[j / NB]);
    });
    static_for<0, Ord::nE>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      product(std::integral_constant<int, Ord::nA + Ord::nB + Ord::nC + Ord::nD + j>{}, O[Ord::tri_R(j)],
              Ub[Ord::tri_st(j)]);
    });
    {
      const uint32_t hdv = (uint32_t)(H * DV);
      const auto ro = job.map ? make_rsrc(o, 0u) : make_rsrc(o + ((size_t)c_begin * H + h) * DV + vcol, (uint32_t)Lc * hdv * 4u);
#pragma unroll
      for (int R = 0; R < NB; ++R) {
        const float d[4] = {dq[R].x, dq[R].y, dq[R].z, dq[R].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, (O[R][i] + d[i] * U[R][i]) * sc_up), ro,
                                                (int)(((uint32_t)(16 * R + 4 * lg + i) * hdv + (uint32_t)lr) * 4u), 0, 0);
      }
    }
    __syncthreads();  // every read of this chunk's buffers is done; the next chunk's are written
  }
  auto store_state = [&](float* sp, int ld) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sp[(size_t)(16 * cb + 4 * lg + i) * ld + col] = Sacc[cb][i] * sc_up;
  };
  if (ch_stop == nchunks) {
    if (job.end_out) store_state(job.end_out + (size_t)chain * DK * DV, DV);
  } else if (job.mid_out) {
    store_state(job.mid_out + (size_t)chain * DK * job.mid_ld, job.mid_ld);
  }
}

template <int C, int DK, int BV, typename InT>
__global__ __launch_bounds__(NT, 1) void chunk_state_kernel(
    const uint4* __restrict__ ws, const InT* __restrict__ v, const float* h0,
    const int32_t* __restrict__ cu_seqlens, float* __restrict__ o, float* hT,
    int n_chains, int H, int DV, int64_t seq_len) {
  StateJob job;
  if (!state_block((int)blockIdx.x, n_chains, DV / BV, job.chain, job.j0)) return;
  job.j0 *= BV;
  job.ch_begin = 0;
  job.ch_end = INT64_MAX;
  job.s_in = h0;
  job.end_out = hT;
  job.mid_out = nullptr;
  job.mid_ld = DV;
  job.map = false;
  chunk_state_body<C, DK, BV, InT>(ws, v, cu_seqlens, o, H, DV, seq_len, job);
}

// ---------------------------------------------------------------------------
// Segmented state pass (in-device context parallelism for few long chains).  Each chain's
// chunks are cut into n_seg segments of rl chunks.  Over a segment the chunk recurrence is
// affine in the entering state, S_out = M S_in + B ("Kimi K3 model structure (7)", context
// parallelism through an associative prefix scan, because KDA states cannot simply be
// added): the map pass finds [M | B] of every segment but each chain's last, all in parallel;
// the scan composes them in order, S_in(r + 1) = M_r S_in(r) + B_r, from h0; the rerun then
// walks every segment in parallel from its entering state and writes o (and hT from the
// chain's last segment).  Map and rerun workgroups take virtual chains u = r * n_chains +
// chain (segment r), mapped like the state pass's chains.
// ---------------------------------------------------------------------------
template <int C, int DK, int BV, typename InT>
__global__ __launch_bounds__(NT, 1) void chunk_seg_kernel(
    const uint4* __restrict__ ws, const InT* __restrict__ v, const float* h0,
    const int32_t* __restrict__ cu_seqlens, float* __restrict__ o, float* hT, const float* seg_in, float* maps,
    int n_chains, int n_vchains, int64_t rl, int H, int DV, int64_t seq_len, int map) {
  const int width = map ? DK + DV : DV;
  int u = 0, tile = 0;
  if (!state_block((int)blockIdx.x, n_vchains, width / BV, u, tile)) return;
  const int r = u / n_chains;
  StateJob job;
  job.chain = u - r * n_chains;
  job.j0 = tile * BV;
  job.ch_begin = (int64_t)r * rl;
  job.ch_end = (int64_t)(r + 1) * rl;
  job.map = map != 0;
  if (job.map) {
    job.s_in = nullptr;
    job.end_out = nullptr;
    job.mid_out = maps + (size_t)r * n_chains * DK * (DK + DV);
    job.mid_ld = DK + DV;
  } else {
    // (segment 0 too reads the copy of h0 the scan made: hT may alias h0, and the chain's last
    // segment writes hT in the same launch)
    job.s_in = seg_in + (size_t)r * n_chains * DK * DV;
    job.end_out = hT;
    job.mid_out = nullptr;
    job.mid_ld = DV;
  }
  chunk_state_wave_body<C, DK, BV / 16, InT>(ws, v, cu_seqlens, o, H, DV, seq_len, job);
}

// The scan: one workgroup of 256 threads per (chain, 32 value columns), fp32; it copies
// S_in(0) = h0 to the workspace, then thread t forms row t / 2, columns 16 (t & 1) .. + 15 of
// S_in(r + 1) = M_r S_in(r) + B_r (the sum over k in order), the tile of S_in(r) in LDS.  It
// stops at the chain's last segment.
template <int C, int DK>
__global__ __launch_bounds__(256) void chunk_seg_scan_kernel(const float* h0, const int32_t* __restrict__ cu_seqlens,
                                                             const float* __restrict__ maps, float* __restrict__ seg_in,
                                                             int n_chains, int n_seg, int64_t rl, int H, int DV,
                                                             int64_t seq_len) {
  __shared__ float sS[DK][32];
  const int ntile = DV / 32;
  const int chain = blockIdx.x / ntile, c0 = (blockIdx.x - chain * ntile) * 32;
  const int n = chain / H;
  int64_t len;
  if (cu_seqlens) len = (int64_t)cu_seqlens[n + 1] - cu_seqlens[n];
  else len = seq_len;
  const int64_t nchunks = (len + C - 1) / C;
  const int t = threadIdx.x, row = t >> 1, cb = 16 * (t & 1);
  const bool act = row < DK;
  for (int e = t; e < DK * 32; e += 256) {  // S_in(0): h0 (or zeros), also to the workspace
    const int rr = e >> 5, cc = e & 31;
    const float x = h0 ? h0[((size_t)chain * DK + rr) * DV + c0 + cc] : 0.f;
    sS[rr][cc] = x;
    seg_in[((size_t)chain * DK + rr) * DV + c0 + cc] = x;
  }
  const int W = DK + DV;
  for (int r = 0; r + 1 < n_seg && nchunks > (int64_t)(r + 1) * rl; ++r) {
    __syncthreads();  // S_in(r) in LDS
    const float* mr = maps + ((size_t)r * n_chains + chain) * DK * W;
    float acc[16];
    if (act) {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) acc[jj] = mr[(size_t)row * W + DK + c0 + cb + jj];
      for (int kk = 0; kk < DK; ++kk) {
        const float m = mr[(size_t)row * W + kk];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) acc[jj] = fmaf(m, sS[kk][cb + jj], acc[jj]);
      }
    }
    __syncthreads();  // every read of S_in(r)
    if (act) {
      float* dst = seg_in + (((size_t)(r + 1) * n_chains + chain) * DK + row) * DV + c0 + cb;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        sS[row][cb + jj] = acc[jj];
        dst[jj] = acc[jj];
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
// The dynamic-LDS limit is a per-device attribute of each kernel: set it once per device
// (one bit each in the kernel's own flag word, thread-safe); devices past the 64th set it
// on every launch.
static hipError_t set_lds_limit(const void* kern, size_t lds, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
  if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (bit) done.fetch_or(bit, std::memory_order_release);
  }
  return hipSuccess;
}

#if KDA_CHUNK_FUSED
template <int C, int DK, int BV, Prec P, typename InT>
static hipError_t launch_one(const ChunkArgs& a) {
  constexpr size_t lds = lds_bytes<C, DK, BV, P>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = chunk_fwd_kernel<C, DK, BV, P, InT, false>;
  static std::atomic<uint64_t> attr_done{0};
  hipError_t e = set_lds_limit((const void*)kern, lds, attr_done);
  if (e != hipSuccess) return e;
  const int n_chains = a.n_seqs * a.n_heads;
  const int ntile = a.dv / BV;
  const int grid = ((n_chains + 7) / 8) * 8 * ntile;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), lds, (hipStream_t)a.stream, (const InT*)a.q, (const InT*)a.k,
                     (const InT*)a.v, a.log_alpha, a.beta, a.h0, a.cu_seqlens, a.o, a.hT, a.ckpt, a.ckpt_every,
                     n_chains, a.n_heads, a.dv, a.seq_len, nullptr, 0, PipeArgs{});
  return hipGetLastError();
}

#endif  // KDA_CHUNK_FUSED
static int pick_bv(int n_chains, int dv, int max_bv);

// ---- split path: prep pass (intra-chunk operands to the workspace), then the state pass
#if KDA_CHUNK_SPLIT
template <int C, int DK>
constexpr size_t split_tile_bytes() { return size_t(WsTile<C, DK>::NU) * 16; }

// upper bound on chunks per sequence, known on the host without reading cu_seqlens
static int64_t max_chunks_per_seq(const ChunkArgs& a) {
  const int64_t len = a.cu_seqlens ? a.total_tokens : a.seq_len;
  return (len + a.chunk_size - 1) / a.chunk_size;
}

// Pipelined split (chunk_fwd_kernel with PIPE_BV): value tiles of 32 columns, so that a few
// chains' state pass takes at most 128 CUs.  Launch r runs the state pass over chunk range r
// beside the in-chunk pass over range r + 1 on the other CUs; the in-chunk pass over the
// first range runs alone before, the state pass over the last alone after.  On the other
// half of the CUs the in-chunk pass takes nearly as long per chunk as the wave-parallel
// state pass, so each range is kRangeGrowth times the one before it: every launch stays
// about balanced, while the first range (its in-chunk pass not hidden) is short and the
// last (its state pass alone) is long.  Ranges in multiples of 16 chunks, the first at
// least 64, as many as that allows (at most 48).
constexpr int kPipeBV = 32;
constexpr double kRangeGrowth = 1.10;
struct PipeRanges {
  static constexpr int kMax = 48;
  int n = 0;
  int64_t b[kMax + 1];  // range r: chunks [b[r], b[r + 1])
};
static bool pipe_ranges(int64_t mc, PipeRanges& pr) {
  // the most ranges n whose geometric sizes f, g f, g^2 f, .. (g = kRangeGrowth, summing to
  // mc) start at f >= 64
  int n = 1;
  double f = (double)mc, qk = kRangeGrowth;
  for (int k = 2; k <= PipeRanges::kMax; ++k) {
    qk *= kRangeGrowth;  // g^k
    const double fk = (double)mc * (kRangeGrowth - 1.0) / (qk - 1.0);
    if (fk < 64.0) break;
    n = k;
    f = fk;
  }
  if (n < 2) return false;
  pr.n = n;
  pr.b[0] = 0;
  double s = f;
  for (int r = 0; r < n - 1; ++r) {
    int64_t sz = (int64_t)(s / 16.0 + 0.5) * 16;
    pr.b[r + 1] = pr.b[r] + (sz < 64 ? 64 : sz);
    s *= kRangeGrowth;
  }
  pr.b[n] = mc;  // the last range takes the rest (within a few chunks of f g^(n-1))
  return pr.b[n - 1] < mc;
}
static bool split_pipelined(const ChunkArgs& a, int64_t max_chunks, PipeRanges& pr) {
  const int64_t state_blocks = (int64_t)((a.n_seqs * a.n_heads + 7) / 8) * 8 * (a.dv / kPipeBV);
  return state_blocks <= 128 && pipe_ranges(max_chunks, pr);
}

template <int C, int DK, typename InT>
static hipError_t launch_split_pipelined(const ChunkArgs& a, void* ws, float* carry, const PipeRanges& pr) {
  const int n_chains = a.n_seqs * a.n_heads;
  const int state_blocks = ((n_chains + 7) / 8) * 8 * (a.dv / kPipeBV);
  // the in-chunk pass over range r: groups of cpg chunks, about 16 per sequence and range
  auto cpg_of = [&](int r) -> int64_t {
    const int64_t c = (pr.b[r + 1] - pr.b[r] + 15) / 16;
    return c < 4 ? 4 : (c > 64 ? 64 : c);
  };
  auto groups_of = [&](int r) -> int64_t { return (pr.b[r + 1] - pr.b[r] + cpg_of(r) - 1) / cpg_of(r); };
  for (int r = 0; r < pr.n; ++r)
    if ((int64_t)n_chains * groups_of(r) + state_blocks > 0x7fffffff) return hipErrorInvalidValue;
  // first range's in-chunk pass on its own
  {
    constexpr size_t lds = lds_bytes<C, DK, 16, Prec::Mixed>();
    auto kern = chunk_fwd_kernel<C, DK, 16, Prec::Mixed, InT, true>;
    static std::atomic<uint64_t> attr_done{0};
    hipError_t e = set_lds_limit((const void*)kern, lds, attr_done);
    if (e != hipSuccess) return e;
    PipeArgs p0{};
    p0.in_ch0 = 0;
    p0.in_ch_end = pr.b[1];
    hipLaunchKernelGGL(kern, dim3((unsigned)(n_chains * groups_of(0))), dim3(NT), lds, (hipStream_t)a.stream,
                       (const InT*)a.q, (const InT*)a.k, (const InT*)a.v, a.log_alpha, a.beta, nullptr, a.cu_seqlens,
                       nullptr, nullptr, nullptr, 0, n_chains, a.n_heads, a.dv, a.seq_len, ws, (int)cpg_of(0), p0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // then per range r: the state pass over range r beside the in-chunk pass over range r + 1
  constexpr size_t lds_p = lds_bytes<C, DK, 16, Prec::Mixed>(), lds_s = WLay<C, DK, kPipeBV / 16>::TOTAL;
  constexpr size_t lds = lds_p > lds_s ? lds_p : lds_s;
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = chunk_fwd_kernel<C, DK, 16, Prec::Mixed, InT, true, kPipeBV>;
  static std::atomic<uint64_t> attr_done{0};
  hipError_t e = set_lds_limit((const void*)kern, lds, attr_done);
  if (e != hipSuccess) return e;
  for (int r = 0; r < pr.n; ++r) {
    const bool next = r + 1 < pr.n;
    const int64_t grid = state_blocks + (next ? (int64_t)n_chains * groups_of(r + 1) : 0);
    PipeArgs pa{};
    pa.n_state_blocks = state_blocks;
    pa.in_ch0 = next ? pr.b[r + 1] : 0;
    pa.in_ch_end = next ? pr.b[r + 2] : 0;
    pa.ch_begin = pr.b[r];
    pa.ch_end = next ? pr.b[r + 1] : INT64_MAX;
    pa.h0 = a.h0;
    pa.o = a.o;
    pa.hT = a.hT;
    pa.carry = carry;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, (hipStream_t)a.stream, (const InT*)a.q,
                       (const InT*)a.k, (const InT*)a.v, a.log_alpha, a.beta, nullptr, a.cu_seqlens, nullptr, nullptr,
                       nullptr, 0, n_chains, a.n_heads, a.dv, a.seq_len, ws, (int)(next ? cpg_of(r + 1) : 4), pa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int C, int DK, int BV, typename InT>
static hipError_t launch_split(const ChunkArgs& a, void* ws) {
  const int n_chains = a.n_seqs * a.n_heads;
  {
    constexpr size_t lds = lds_bytes<C, DK, 16, Prec::Mixed>();
    auto kern = chunk_fwd_kernel<C, DK, 16, Prec::Mixed, InT, true>;
    static std::atomic<uint64_t> attr_done{0};
    hipError_t e = set_lds_limit((const void*)kern, lds, attr_done);
    if (e != hipSuccess) return e;
    // chunks per workgroup: about 8 workgroups per CU over the whole input, 4 to 64 chunks
    const int64_t mc = max_chunks_per_seq(a);
    int64_t cpg = ((int64_t)n_chains * mc) / 2048;
    cpg = cpg < 4 ? 4 : (cpg > 64 ? 64 : cpg);
    const int64_t groups = (mc + cpg - 1) / cpg;
    const int64_t grid = (int64_t)n_chains * (groups > 0 ? groups : 1);
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, (hipStream_t)a.stream, (const InT*)a.q,
                       (const InT*)a.k, (const InT*)a.v, a.log_alpha, a.beta, nullptr, a.cu_seqlens, nullptr, nullptr,
                       nullptr, 0, n_chains, a.n_heads, a.dv, a.seq_len, ws, (int)cpg, PipeArgs{});
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    constexpr size_t lds = SLay<C, DK, BV>::TOTAL;
    static_assert(lds <= 160 * 1024, "LDS budget");
    auto kern = chunk_state_kernel<C, DK, BV, InT>;
    static std::atomic<uint64_t> attr_done{0};
    hipError_t e = set_lds_limit((const void*)kern, lds, attr_done);
    if (e != hipSuccess) return e;
    const int ntile = a.dv / BV;
    const int grid = ((n_chains + 7) / 8) * 8 * ntile;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), lds, (hipStream_t)a.stream, (const uint4*)ws, (const InT*)a.v,
                       a.h0, a.cu_seqlens, a.o, a.hT, n_chains, a.n_heads, a.dv, a.seq_len);
    return hipGetLastError();
  }
}

// Segments for the segmented state pass: taken for at most 64 state tiles of 32 columns
// (n_chains x dv / 32; 16 chains at dv = 128 would leave 3/4 of the CUs idle in the state pass)
// and at least 512 chunks in the longest sequence, with as many segments as keep the map pass
// near 512 workgroups of 32 columns (two per CU; at most 64 segments, each at least 64 chunks)
// and at least 4 (with fewer the pipelined form, which hides the in-chunk pass, is as fast).
// 1M tokens at dk = dv = 128: 1 head 2.5 ms, 4 heads 6.6 ms, 8 heads 13.0 ms, against
// 32-34 ms for the pipelined form (256 workgroups: 2.8, 9.8, 19.5 ms).
static constexpr int kMaxSeg = 64;
static bool split_segments(int n_chains, int dk, int dv, int64_t mc, int& n_seg, int64_t& rl) {
  if (n_chains <= 0 || (int64_t)n_chains * (dv / 32) > 64 || mc < 512) return false;
  int64_t sgs = 512 / ((int64_t)n_chains * ((dk + dv) / 32));
  if (sgs > kMaxSeg) sgs = kMaxSeg;
  if (sgs > mc / 64) sgs = mc / 64;
  if (sgs < 4) return false;
  rl = (mc + sgs - 1) / sgs;
  n_seg = (int)((mc + rl - 1) / rl);
  return n_seg >= 4;
}
// The most segments the segmented form can take for these sizes, known on the host from the
// token total (the longest sequence has at most ceil(total / C) chunks), or 0 when it cannot
// be taken; its workspace holds that many maps [n_chains][DK][DK + DV] (one fewer) and
// entering states [n_chains][DK][DV] (fp32).
static int split_seg_max(int n_chains, int dv, int64_t total_tokens, int chunk_size) {
  const int64_t mc = (total_tokens + chunk_size - 1) / chunk_size;
  if (n_chains <= 0 || (int64_t)n_chains * (dv / 32) > 64 || mc < 512) return 0;
  return (int)(mc / 64 < kMaxSeg ? mc / 64 : kMaxSeg);
}
static size_t split_seg_bytes(int n_chains, int dk, int dv, int64_t total_tokens, int chunk_size) {
  const int sm = split_seg_max(n_chains, dv, total_tokens, chunk_size);
  if (sm == 0) return 0;
  return ((size_t)(sm - 1) * dk * (dk + dv) + (size_t)sm * dk * dv) * (size_t)n_chains * sizeof(float);
}

template <int C, int DK, typename InT>
static hipError_t launch_split_segmented(const ChunkArgs& a, void* ws, float* seg, int n_seg, int64_t rl) {
  const int n_chains = a.n_seqs * a.n_heads;
  const int sm = split_seg_max(n_chains, a.dv, a.total_tokens, a.chunk_size);
  if (n_seg > sm) return hipErrorInvalidValue;  // (the workspace holds sm segments)
  float* maps = seg;
  float* seg_in = seg + (size_t)(sm - 1) * n_chains * DK * (DK + a.dv);
  {  // the in-chunk pass over every chunk (as launch_split)
    constexpr size_t lds = lds_bytes<C, DK, 16, Prec::Mixed>();
    auto kern = chunk_fwd_kernel<C, DK, 16, Prec::Mixed, InT, true>;
    static std::atomic<uint64_t> attr_done{0};
    hipError_t e = set_lds_limit((const void*)kern, lds, attr_done);
    if (e != hipSuccess) return e;
    const int64_t mc = max_chunks_per_seq(a);
    int64_t cpg = ((int64_t)n_chains * mc) / 2048;
    cpg = cpg < 4 ? 4 : (cpg > 64 ? 64 : cpg);
    const int64_t groups = (mc + cpg - 1) / cpg;
    const int64_t grid = (int64_t)n_chains * (groups > 0 ? groups : 1);
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, (hipStream_t)a.stream, (const InT*)a.q,
                       (const InT*)a.k, (const InT*)a.v, a.log_alpha, a.beta, nullptr, a.cu_seqlens, nullptr, nullptr,
                       nullptr, 0, n_chains, a.n_heads, a.dv, a.seq_len, ws, (int)cpg, PipeArgs{});
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr size_t lds = WLay<C, DK, kPipeBV / 16>::TOTAL;
  auto kern = chunk_seg_kernel<C, DK, kPipeBV, InT>;
  static std::atomic<uint64_t> attr_done{0};
  hipError_t e = set_lds_limit((const void*)kern, lds, attr_done);
  if (e != hipSuccess) return e;
  {  // the maps of segments 0 .. n_seg - 2
    const int nv = (n_seg - 1) * n_chains;
    const int64_t grid = (int64_t)((nv + 7) / 8) * 8 * ((DK + a.dv) / kPipeBV);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, (hipStream_t)a.stream, (const uint4*)ws,
                       (const InT*)a.v, a.h0, a.cu_seqlens, a.o, a.hT, (const float*)seg_in, maps, n_chains, nv, rl,
                       a.n_heads, a.dv, a.seq_len, 1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((chunk_seg_scan_kernel<C, DK>), dim3((unsigned)(n_chains * (a.dv / 32))), dim3(256), 0,
                     (hipStream_t)a.stream, a.h0, a.cu_seqlens, (const float*)maps, seg_in, n_chains, n_seg, rl,
                     a.n_heads, a.dv, a.seq_len);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {  // every segment from its entering state
    const int nv = n_seg * n_chains;
    const int64_t grid = (int64_t)((nv + 7) / 8) * 8 * (a.dv / kPipeBV);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, (hipStream_t)a.stream, (const uint4*)ws,
                       (const InT*)a.v, a.h0, a.cu_seqlens, a.o, a.hT, (const float*)seg_in, maps, n_chains, nv, rl,
                       a.n_heads, a.dv, a.seq_len, 0);
    return hipGetLastError();
  }
}

template <int C, int DK, typename InT>
static hipError_t dispatch_split_bv(const ChunkArgs& a, void* ws, float* carry) {
  const int64_t mc = max_chunks_per_seq(a);
  int n_seg = 0;
  int64_t rl = 0;
  if (split_segments(a.n_seqs * a.n_heads, DK, a.dv, mc, n_seg, rl))
    return launch_split_segmented<C, DK, InT>(a, ws, carry + (size_t)a.n_seqs * a.n_heads * DK * a.dv, n_seg, rl);
  PipeRanges pr;
  if (split_pipelined(a, mc, pr)) return launch_split_pipelined<C, DK, InT>(a, ws, carry, pr);
  // (a value tile as wide as dv when the chains alone fill the CUs: the state pass then runs
  // in one round of workgroups instead of two)
  const int bv = pick_bv(a.n_seqs * a.n_heads, a.dv, 128);
  if (bv == 128) return launch_split<C, DK, 128, InT>(a, ws);
  if (bv == 64) return launch_split<C, DK, 64, InT>(a, ws);
  if (bv == 32) return launch_split<C, DK, 32, InT>(a, ws);
  return launch_split<C, DK, 16, InT>(a, ws);
}

#endif  // KDA_CHUNK_SPLIT
// value-tile width: the widest that still gives at least one workgroup per CU
static int pick_bv(int n_chains, int dv, int max_bv) {
  for (int bv = max_bv; bv >= 16; bv /= 2)
    if (dv % bv == 0 && (int64_t)n_chains * (dv / bv) >= 256) return bv;
  return 16;
}

#if KDA_CHUNK_FUSED
template <int C, int DK, int MAXBV, Prec P, typename InT>
static hipError_t dispatch_bv(const ChunkArgs& a) {
  const int bv = pick_bv(a.n_seqs * a.n_heads, a.dv, MAXBV);
  if constexpr (MAXBV >= 64) {
    if (bv == 64) return launch_one<C, DK, 64, P, InT>(a);
  }
  if constexpr (MAXBV >= 32) {
    if (bv == 32) return launch_one<C, DK, 32, P, InT>(a);
  }
  return launch_one<C, DK, 16, P, InT>(a);
}

template <int DK, Prec P, typename InT>
static hipError_t dispatch_c(const ChunkArgs& a) {
  if constexpr (P == Prec::Mixed) {
    if (a.chunk_size == 64) return dispatch_bv<64, DK, 64, P, InT>(a);
    if (a.chunk_size == 32) return dispatch_bv<32, DK, 64, P, InT>(a);
    if (a.chunk_size == 16) return dispatch_bv<16, DK, 64, P, InT>(a);
  } else {
    if (a.chunk_size == 16) return dispatch_bv<16, DK, 64, P, InT>(a);
    if (a.chunk_size == 32) return dispatch_bv<32, DK, (DK == 128 ? 32 : 64), P, InT>(a);
    if constexpr (DK == 64) {
      if (a.chunk_size == 64) return dispatch_bv<64, DK, 32, P, InT>(a);
    } else {
      // fp32 operands of a 64-token chunk at dk = 128 (Qg, Kg, Kd^T, the right base: 32 KB each)
      // do not fit the 160 KB of LDS beside the rest; the recurrence does not depend on the
      // chunk size, so these run as 32-token chunks (checkpoint spacings, multiples of 64, are
      // multiples of 32 as well)
      if (a.chunk_size == 64) return dispatch_bv<32, DK, 32, P, InT>(a);
    }
  }
  return hipErrorInvalidValue;
}

#endif  // KDA_CHUNK_FUSED
}  // namespace chunkk

#if KDA_CHUNK_FUSED
bool chunk_fwd_supported(int dk, int dv, int chunk_size, bool bf16) {
  if (!((dk == 64 || dk == 128) && (dv == 64 || dv == 128))) return false;
  if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return false;
  return true;
}

#endif  // KDA_CHUNK_FUSED

#if KDA_CHUNK_SPLIT
// per-chunk tiles, then one fp32 state per chain for the pipelined path's hand-over between ranges
static size_t split_tiles_bytes(int64_t total_tokens, int n_seqs, int n_heads, int dk, int chunk_size) {
  using namespace chunkk;
  size_t tile = 0;
  if (dk == 128) {
    tile = chunk_size == 64 ? split_tile_bytes<64, 128>() : chunk_size == 32 ? split_tile_bytes<32, 128>()
                                                                             : split_tile_bytes<16, 128>();
  } else {
    tile = chunk_size == 64 ? split_tile_bytes<64, 64>() : chunk_size == 32 ? split_tile_bytes<32, 64>()
                                                                            : split_tile_bytes<16, 64>();
  }
  // slots: sequence start / C + sequence index + chunk index < total_tokens / C + n_seqs + 1
  const size_t slots = (size_t)(total_tokens / chunk_size) + (size_t)n_seqs + 1;
  return slots * (size_t)n_heads * tile;
}

size_t chunk_split_workspace_bytes(int64_t total_tokens, int n_seqs, int n_heads, int dk, int dv, int chunk_size) {
  return split_tiles_bytes(total_tokens, n_seqs, n_heads, dk, chunk_size) +
         (size_t)n_seqs * n_heads * dk * dv * sizeof(float) +
         chunkk::split_seg_bytes(n_seqs * n_heads, dk, dv, total_tokens, chunk_size);
}

// Which forward path is faster for a bf16 input of this shape (measured on MI355X at dk = 128,
// dv in {64, 128}, chunks of 16-64 tokens).  The fused kernel cuts each chain's dv columns
// into the widest value tiles that still give every CU a workgroup (pick_bv, at most 64) and
// redoes the chunk's in-chunk work once per tile; the split path does it once per chunk and
// head, at the price of the workspace round trip.  So the split path is taken when the fused
// kernel would repeat the in-chunk work (two or more tiles per chain) and either its tiles
// take two or more rounds of workgroups or the sequences are long enough (16 chunks on
// average) to repay the split path's extra launch.  Measured: 1M tokens x 32 heads split
// 35.3 ms, fused 96 ms; 8 x 4,096 tokens x 32 heads, dv 128, split 0.79 ms, fused 0.93 ms;
// 4 x 4,096 x 32 heads, dv 128, split 0.42 ms, fused 0.47 ms; 16 x 4,096 x 32 heads, dv 64
// (one 64-column tile per chain): fused 0.94 ms, split 1.42 ms.  Sequences shorter than 4
// chunks on average stay on the fused kernel.
bool chunk_fwd_prefers_split(int n_seqs, int n_heads, int dv, int chunk_size, int64_t total_tokens) {
  if (n_seqs <= 0 || total_tokens <= 0) return false;
  const int64_t chunks = total_tokens / n_seqs / chunk_size;  // per sequence, on average
  if (chunks < 4) return false;
  const int chains = n_seqs * n_heads;
  const int64_t tiles = dv / chunkk::pick_bv(chains, dv, 64);  // fused value tiles per chain
  if (tiles < 2) return false;
  return (int64_t)chains * tiles > 256 || chunks >= 16;
}

hipError_t launch_chunk_fwd_split(const ChunkArgs& a, void* ws) {
  using namespace chunkk;
  if (!a.bf16 || !chunk_fwd_supported(a.dk, a.dv, a.chunk_size, a.bf16)) return hipErrorInvalidValue;
  float* carry = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) +
                                          split_tiles_bytes(a.total_tokens, a.n_seqs, a.n_heads, a.dk, a.chunk_size));
  if (a.dk == 128) {
    if (a.chunk_size == 64) return dispatch_split_bv<64, 128, bf16_t>(a, ws, carry);
    if (a.chunk_size == 32) return dispatch_split_bv<32, 128, bf16_t>(a, ws, carry);
    return dispatch_split_bv<16, 128, bf16_t>(a, ws, carry);
  }
  if (a.chunk_size == 64) return dispatch_split_bv<64, 64, bf16_t>(a, ws, carry);
  if (a.chunk_size == 32) return dispatch_split_bv<32, 64, bf16_t>(a, ws, carry);
  return dispatch_split_bv<16, 64, bf16_t>(a, ws, carry);
}

#endif  // KDA_CHUNK_SPLIT

#if KDA_CHUNK_FUSED
hipError_t launch_chunk_fwd(const ChunkArgs& a) {
  using namespace chunkk;
  if (!chunk_fwd_supported(a.dk, a.dv, a.chunk_size, a.bf16)) return hipErrorInvalidValue;
  if (a.bf16) {
    return a.dk == 128 ? dispatch_c<128, Prec::Mixed, bf16_t>(a) : dispatch_c<64, Prec::Mixed, bf16_t>(a);
  }
  return a.dk == 128 ? dispatch_c<128, Prec::F32, float>(a) : dispatch_c<64, Prec::F32, float>(a);
}

#endif  // KDA_CHUNK_FUSED

}  // namespace kda
