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
//   W      = T Diag(b) (K * e^G),  Ut = T Diag(b) V             WY pseudo-keys / values
//   U      = Ut - W S                                           (serial part starts here)
//   O      = (Q * e^G) S + M U
//   S     <- Diag(e^{g_last}) S + (K * e^{g_last - G})^T U
//
// One workgroup (256 threads, 4 waves) owns one (sequence, head, dv-tile of BV
// value columns) and walks the sequence's chunks in order, resetting the state at
// the sequence start (packed-sequence state reset, "Kimi K3 NPU Training",
// section "TND is not a layout switch", item 2).  The fp32 master state lives in
// MFMA accumulator registers; a 16-bit copy in LDS feeds the next chunk's MFMAs.
//
// Overflow-safe decay.  Every MFMA operand is a product of a value and an
// exponential <= 1, except inside the 16x16 diagonal sub-blocks of A and M:
//   * sub-block pair (R > I): left = X_r e^{c_r}, right = k_i e^{s_I - c_i}
//     scaled by e^{G_{R-1} - G_I} (all <= 1), where c is the in-block cumulative
//     decay, s_I the block total and G_J the cumulative decay at the end of block J;
//   * diagonal sub-block R: left = X_r e^{c_r - s_R/2}, right = k_i e^{s_R/2 - c_i},
//     each bounded by e^{|s_R|/2}; finite when a 16-token block decays by less
//     than ~170 nats per channel (the documented precondition).
// Entries above the diagonal are removed with a select, never a multiply.
//
// Precision policies:
//   Mixed (bf16 inputs): fp16 MFMA operands for all products except the diagonal
//     sub-blocks of the Gram matrices, which use bf16 (range) and, for M, a hi/lo
//     bf16 split (three MFMAs).  The diagonal of M (q_r . k_r) is applied to U in
//     fp32 outside the MFMA.  Accumulation is fp32 throughout.
//   F32 (fp32 inputs): every product on the fp32 MFMA (16x16x4).
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace chunkk {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int NW = NT / kWave;

enum class Prec { Mixed, F32 };

// ---------------------------------------------------------------------------
// MFMA operand types.  T: element type of the LDS operand matrices.
// KS: k-extent of one MMA step; each lane holds KS/4 consecutive k values.
// ---------------------------------------------------------------------------
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

// acc += A(16 x KS) * B(16 x KS)^T for one MMA step.  `a` and `b` point at the
// lane's first k element (row (lane & 15), k offset (lane >> 4) * KS/4).
__device__ __forceinline__ void mma_step(f32x4& acc, const _Float16* a, const _Float16* b) {
  const half8 av = *reinterpret_cast<const half8*>(a);
  const half8 bv = *reinterpret_cast<const half8*>(b);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_step(f32x4& acc, const float* a, const float* b) {
  // The four fp32 MFMAs take k = 4*(lane>>4) + j, j = 0..3: a permutation of the
  // 16 k values that is the same for A and B, so the product is unchanged.
  const float4 av = *reinterpret_cast<const float4*>(a);
  const float4 bv = *reinterpret_cast<const float4*>(b);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, acc, 0, 0, 0);
}

// C[16x16] (+)= A[m0.., k0..k0+K) * B[n0.., same k]^T with row-major operands.
template <typename T, int KS>
__device__ __forceinline__ void mma_tile(f32x4& acc, const T* A, int lda, const T* B, int ldb, int nsteps) {
  const int l = lane_id();
  const T* a = A + (l & 15) * lda + (l >> 4) * (KS / 4);
  const T* b = B + (l & 15) * ldb + (l >> 4) * (KS / 4);
  for (int s = 0; s < nsteps; ++s) mma_step(acc, a + s * KS, b + s * KS);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <typename T> __device__ __forceinline__ T cvt(float x);
template <> __device__ __forceinline__ _Float16 cvt<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ float cvt<float>(float x) { return x; }

// Four consecutive elements from fp32.
__device__ __forceinline__ void store4(_Float16* p, float a, float b, float c, float d) {
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<half4*>(p) = half4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

constexpr size_t al16(size_t x) { return (x + 15) & ~size_t(15); }
constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------
// LDS layout (bytes).  Region 1 is time-shared: the fp32 decay-scaled q/k
// operands of the Gram stage, then the 16-bit operands of the WY and state
// stages.  The other regions persist.
// ---------------------------------------------------------------------------
template <int C, int DK, int BV, Prec P>
struct Lay {
  using T = typename Op<P>::T;
  static constexpr int KS = Op<P>::KS, PD = Op<P>::PAD;
  static constexpr int NB = C / 16;                      // 16-row sub-blocks per chunk
  static constexpr int CK = ((C + KS - 1) / KS) * KS;    // token k-extent rounded to the MMA step
  static constexpr int LDF = DK + 4;                     // fp32 [C][DK] rows
  static constexpr int LDD = DK + PD;                    // T [*][DK] rows (k = channel)
  static constexpr int LDC = CK + PD;                    // T [*][CK] rows (k = token)
  static constexpr int LDA = C + 4;                      // fp32 [C][C] rows
  static constexpr int NPAIR = NB * (NB - 1) / 2;
  // region 1, Gram view
  static constexpr size_t LQ = 0;
  static constexpr size_t LK = LQ + al16(size_t(C) * LDF * 4);
  static constexpr size_t RK = LK + al16(size_t(C) * LDF * 4);
  static constexpr size_t END_G = RK + al16(size_t(C) * LDF * 4);
  // region 1, WY / state view
  static constexpr size_t QG = 0;                                          // [C][LDD]
  static constexpr size_t KGT = QG + al16(size_t(C) * LDD * sizeof(T));    // [DK][LDC]
  static constexpr size_t KDT = KGT + al16(size_t(DK) * LDC * sizeof(T));  // [DK][LDC]
  static constexpr size_t WM = KDT + al16(size_t(DK) * LDC * sizeof(T));   // [C][LDD]
  static constexpr size_t TB = WM + al16(size_t(C) * LDD * sizeof(T));     // [C][LDC]
  static constexpr size_t UT = TB + al16(size_t(C) * LDC * sizeof(T));     // [BV][LDC]
  static constexpr size_t VT = UT + al16(size_t(BV) * LDC * sizeof(T));    // [BV][LDC]
  static constexpr size_t END_W = VT + al16(size_t(BV) * LDC * sizeof(T));
  static constexpr size_t R1 = al16(cmax(END_G, END_W));
  // persistent
  static constexpr size_t ST = R1;                                          // S^T [BV][LDD] (T)
  static constexpr size_t AK = ST + al16(size_t(BV) * LDD * sizeof(T));      // A then T, fp32 [C][LDA]
  static constexpr size_t AQ = AK + al16(size_t(C) * LDA * 4);              // strict M, T [C][LDC]
  static constexpr size_t AO = AQ + al16(size_t(C) * LDC * sizeof(T));      // off-diag A tiles, T [NPAIR][16][16]
  static constexpr size_t SB = AO + al16(size_t(NPAIR) * 256 * sizeof(T));  // block totals s [NB][DK] f32
  static constexpr size_t BB = SB + al16(size_t(NB) * DK * 4);              // e^{s_J} [NB][DK]
  static constexpr size_t PS = BB + al16(size_t(NB) * DK * 4);              // e^{-s_J/2} [NB][DK]
  static constexpr size_t GM = PS + al16(size_t(NB) * DK * 4);              // e^{g_last} [DK]
  static constexpr size_t BE = GM + al16(size_t(DK) * 4);                   // beta [C]
  static constexpr size_t DQ = BE + al16(size_t(C) * 4);                    // q_r . k_r [C]
  static constexpr size_t TOTAL = DQ + al16(size_t(C) * 4);
};

template <int C, int DK, int BV, Prec P>
constexpr size_t lds_bytes() { return Lay<C, DK, BV, P>::TOTAL; }

// index of the off-diagonal block pair (R, I), R > I, in row-major lower order
__host__ __device__ constexpr int pair_index(int R, int I) { return R * (R - 1) / 2 + I; }

// bf16 hi/lo split of eight fp32 values (hi = RNE(x), lo = RNE(x - hi)).
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)x[j];
    hi[j] = h;
    lo[j] = (__bf16)(x[j] - (float)h);
  }
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int C, int DK, int BV, Prec P, typename InT>
__global__ __launch_bounds__(NT, 1) void chunk_fwd_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, const float* h0,
    const int32_t* __restrict__ cu_seqlens, float* __restrict__ o, float* hT, int n_chains, int H, int DV,
    int64_t seq_len) {
  using L = Lay<C, DK, BV, P>;
  using T = typename L::T;
  constexpr int KS = L::KS, NB = L::NB, CK = L::CK;
  constexpr int LDF = L::LDF, LDD = L::LDD, LDC = L::LDC, LDA = L::LDA;
  constexpr int NA = DK / 16;   // channel tiles
  constexpr int NJ = BV / 16;   // value-column tiles
  constexpr int LPR = DK / 4;   // elementwise lanes per row (4 channels each)
  constexpr int HB = C / 8;     // half-blocks of 8 rows
  static_assert(C % 16 == 0 && C <= 64 && DK % 64 == 0 && BV % 16 == 0, "shape");
  static_assert(NB <= NW, "one wave per diagonal sub-block");
  static_assert(HB * LPR <= NT, "elementwise map");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* sLQ = reinterpret_cast<float*>(smem + L::LQ);
  float* sLK = reinterpret_cast<float*>(smem + L::LK);
  float* sRK = reinterpret_cast<float*>(smem + L::RK);
  T* sQG = reinterpret_cast<T*>(smem + L::QG);
  T* sKGT = reinterpret_cast<T*>(smem + L::KGT);
  T* sKDT = reinterpret_cast<T*>(smem + L::KDT);
  T* sW = reinterpret_cast<T*>(smem + L::WM);
  T* sTB = reinterpret_cast<T*>(smem + L::TB);
  T* sUT = reinterpret_cast<T*>(smem + L::UT);
  T* sVT = reinterpret_cast<T*>(smem + L::VT);
  T* sST = reinterpret_cast<T*>(smem + L::ST);
  float* sAK = reinterpret_cast<float*>(smem + L::AK);
  T* sAQ = reinterpret_cast<T*>(smem + L::AQ);
  T* sAO = reinterpret_cast<T*>(smem + L::AO);
  float* sSB = reinterpret_cast<float*>(smem + L::SB);
  float* sBB = reinterpret_cast<float*>(smem + L::BB);
  float* sPS = reinterpret_cast<float*>(smem + L::PS);
  float* sGM = reinterpret_cast<float*>(smem + L::GM);
  float* sBE = reinterpret_cast<float*>(smem + L::BE);
  float* sDQ = reinterpret_cast<float*>(smem + L::DQ);

  // ---- which (sequence, head, value tile): dv tiles of one chain share an XCD
  const int ntile = DV / BV;
  const int b = blockIdx.x;
  const int xcd = b & 7, qd = b >> 3;
  const int tile = qd % ntile;
  const int chain = (qd / ntile) * 8 + xcd;
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

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int l = lane_id();

  // ---- one-time zero fill of the persistent triangular operands
  for (int i = tid; i < C * LDA; i += NT) sAK[i] = 0.f;
  for (int i = tid; i < C * LDC; i += NT) sAQ[i] = cvt<T>(0.f);

  // ---- state: fp32 master tiles (a, j) in MFMA accumulator layout.
  // Tile id = a + NA*j, owned by wave id % NW, slot id / NW.
  constexpr int S_SLOTS = (NA * NJ + NW - 1) / NW;
  f32x4 Sacc[S_SLOTS];
  const float* h0p = h0 ? h0 + (size_t)chain * DK * DV : nullptr;
#pragma unroll
  for (int s = 0; s < S_SLOTS; ++s) {
    const int id = wave + NW * s;
    Sacc[s] = zero4();
    if (id < NA * NJ && h0p) {
      const int a = id % NA, j = id / NA;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Sacc[s][i] = h0p[(size_t)(16 * a + 4 * (l >> 4) + i) * DV + j0 + 16 * j + (l & 15)];
    }
  }
  // 16-bit copy S^T [BV][DK] for the MFMAs
  auto write_ST = [&]() {
#pragma unroll
    for (int s = 0; s < S_SLOTS; ++s) {
      const int id = wave + NW * s;
      if (id < NA * NJ) {
        const int a = id % NA, j = id / NA;
        store4(sST + (16 * j + (l & 15)) * LDD + 16 * a + 4 * (l >> 4), Sacc[s][0], Sacc[s][1], Sacc[s][2],
               Sacc[s][3]);
      }
    }
  };
  write_ST();

  // ---- elementwise thread map: 8 rows x 4 channels per thread
  const int e_hb = tid / LPR, e_cg = tid % LPR;
  const bool e_act = e_hb < HB;
  const int e_r0 = 8 * e_hb, e_c0 = 4 * e_cg;
  const int e_R = e_hb >> 1;
  const bool e_second = (e_hb & 1) != 0;
  // value-tile map: 2 rows x 8 columns per thread
  constexpr int VLPR = BV / 8;
  const int v_p = tid / VLPR, v_c0 = 8 * (tid % VLPR);
  const bool v_act = v_p < C / 2;

  // U / O tiles (R, j): id = R + NB*j, owned by wave id % NW
  constexpr int U_SLOTS = (NB * NJ + NW - 1) / NW;

  const int64_t nchunks = (t_end - t_begin + C - 1) / C;
  __syncthreads();

  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t c_begin = t_begin + ch * C;
    const int Lc = (int)((t_end - c_begin) < C ? (t_end - c_begin) : C);

    // ================= E1: load the chunk, in-block cumulative decay =================
    float eq[8][4], ek[8][4], ec[8][4];
    float vv[2][8];
    {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = e_r0 + i;
        const bool ok = e_act && r < Lc;
        const size_t off = ((size_t)(c_begin + r) * H + h) * DK + e_c0;
        if (ok) {
          const float4 la = *reinterpret_cast<const float4*>(log_alpha + off);
          ec[i][0] = la.x; ec[i][1] = la.y; ec[i][2] = la.z; ec[i][3] = la.w;
          if constexpr (sizeof(InT) == 2) {
            const uint2 qw = *reinterpret_cast<const uint2*>(q + off);
            const uint2 kw = *reinterpret_cast<const uint2*>(k + off);
            float2 a0 = bf16x2_to_f32x2(qw.x), a1 = bf16x2_to_f32x2(qw.y);
            float2 b0 = bf16x2_to_f32x2(kw.x), b1 = bf16x2_to_f32x2(kw.y);
            eq[i][0] = a0.x; eq[i][1] = a0.y; eq[i][2] = a1.x; eq[i][3] = a1.y;
            ek[i][0] = b0.x; ek[i][1] = b0.y; ek[i][2] = b1.x; ek[i][3] = b1.y;
          } else {
            const float4 qa = *reinterpret_cast<const float4*>(q + off);
            const float4 ka = *reinterpret_cast<const float4*>(k + off);
            eq[i][0] = qa.x; eq[i][1] = qa.y; eq[i][2] = qa.z; eq[i][3] = qa.w;
            ek[i][0] = ka.x; ek[i][1] = ka.y; ek[i][2] = ka.z; ek[i][3] = ka.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) ec[i][c] = eq[i][c] = ek[i][c] = 0.f;
        }
      }
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int r = 2 * v_p + rr;
        const bool ok = v_act && r < Lc;
        const size_t off = ((size_t)(c_begin + r) * H + h) * DV + j0 + v_c0;
        if (ok) {
          if constexpr (sizeof(InT) == 2) {
            const uint4 w = *reinterpret_cast<const uint4*>(v + off);
            float2 x0 = bf16x2_to_f32x2(w.x), x1 = bf16x2_to_f32x2(w.y), x2 = bf16x2_to_f32x2(w.z),
                   x3 = bf16x2_to_f32x2(w.w);
            vv[rr][0] = x0.x; vv[rr][1] = x0.y; vv[rr][2] = x1.x; vv[rr][3] = x1.y;
            vv[rr][4] = x2.x; vv[rr][5] = x2.y; vv[rr][6] = x3.x; vv[rr][7] = x3.y;
          } else {
            const float4 w0 = *reinterpret_cast<const float4*>(v + off);
            const float4 w1 = *reinterpret_cast<const float4*>(v + off + 4);
            vv[rr][0] = w0.x; vv[rr][1] = w0.y; vv[rr][2] = w0.z; vv[rr][3] = w0.w;
            vv[rr][4] = w1.x; vv[rr][5] = w1.y; vv[rr][6] = w1.z; vv[rr][7] = w1.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) vv[rr][c] = 0.f;
        }
      }
      // in-half cumulative sum, then combine the two halves of the 16-row block
      float tot[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          acc += ec[i][c];
          ec[i][c] = acc;
        }
        tot[c] = acc;
      }
      float s_blk[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float other = wave_xor(tot[c], LPR);
        s_blk[c] = tot[c] + other;
        if (e_second) {
#pragma unroll
          for (int i = 0; i < 8; ++i) ec[i][c] += other;
        }
      }
      if (e_act && e_second)
        *reinterpret_cast<float4*>(sSB + e_R * DK + e_c0) = make_float4(s_blk[0], s_blk[1], s_blk[2], s_blk[3]);
      if (tid < C) sBE[tid] = tid < Lc ? beta[(size_t)(c_begin + tid) * H + h] : 0.f;

      __syncthreads();  // ---------------------------------------------------------- B1

      // ================= E2: decay-scaled operands (fp32) =================
      if (e_act) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float sR = sSB[e_R * DK + e_c0 + c];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float e = __expf(ec[i][c]);           // e^{c_r} <= 1
            const float rgt = __expf(sR - ec[i][c]);    // e^{s_R - c_r} <= 1
            ec[i][c] = rgt;
            eq[i][c] *= e;
            const float kk = ek[i][c];
            ek[i][c] = kk * e;
            // reuse: eq = q e^{c}, ek = k e^{c}, ec = e^{s-c} (k applied at the store)
            ec[i][c] = kk * rgt;
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = e_r0 + i;
          *reinterpret_cast<float4*>(sLQ + r * LDF + e_c0) = make_float4(eq[i][0], eq[i][1], eq[i][2], eq[i][3]);
          *reinterpret_cast<float4*>(sLK + r * LDF + e_c0) = make_float4(ek[i][0], ek[i][1], ek[i][2], ek[i][3]);
          *reinterpret_cast<float4*>(sRK + r * LDF + e_c0) = make_float4(ec[i][0], ec[i][1], ec[i][2], ec[i][3]);
        }
        // per-channel block vectors, written once (by the first half-block's threads)
        if (e_hb == 0) {
          float gl[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
          for (int J = 0; J < NB; ++J) {
            float bj[4], pj[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float sJ = sSB[J * DK + e_c0 + c];
              bj[c] = __expf(sJ);
              pj[c] = __expf(-0.5f * sJ);
              gl[c] *= bj[c];
            }
            *reinterpret_cast<float4*>(sBB + J * DK + e_c0) = make_float4(bj[0], bj[1], bj[2], bj[3]);
            *reinterpret_cast<float4*>(sPS + J * DK + e_c0) = make_float4(pj[0], pj[1], pj[2], pj[3]);
          }
          *reinterpret_cast<float4*>(sGM + e_c0) = make_float4(gl[0], gl[1], gl[2], gl[3]);
        }
      }
    }
    __syncthreads();  // ---------------------------------------------------------------- B2

    // ================= Gram stage: A (key-key) and M (query-key) =================
    {
      const int row = l & 15;
      const int kof = (l >> 4) * 8;  // Mixed: 8 k values per lane per 32-wide step
      constexpr int NPAIRS_ALL = NB * (NB + 1) / 2;
      // pairs enumerated as: diagonal R = 0..NB-1 first (one per wave), then off-diagonal
      for (int pidx = wave; pidx < NPAIRS_ALL; pidx += NW) {
        int R, I;
        if (pidx < NB) {
          R = I = pidx;
        } else {
          int o2 = pidx - NB;
          R = 1;
          while (o2 >= R) { o2 -= R; ++R; }
          I = o2;
        }
        const bool diag = R == I;
        f32x4 accQ = zero4(), accK = zero4();
        const float* lq = sLQ + (16 * R + row) * LDF;
        const float* lk = sLK + (16 * R + row) * LDF;
        const float* rk = sRK + (16 * I + row) * LDF;
        if constexpr (P == Prec::Mixed) {
          for (int ks = 0; ks < DK / 32; ++ks) {
            const int c0 = ks * 32 + kof;
            float a[8], ak[8], bq[8], f[8];
            *reinterpret_cast<float4*>(&a[0]) = *reinterpret_cast<const float4*>(lq + c0);
            *reinterpret_cast<float4*>(&a[4]) = *reinterpret_cast<const float4*>(lq + c0 + 4);
            *reinterpret_cast<float4*>(&ak[0]) = *reinterpret_cast<const float4*>(lk + c0);
            *reinterpret_cast<float4*>(&ak[4]) = *reinterpret_cast<const float4*>(lk + c0 + 4);
            *reinterpret_cast<float4*>(&bq[0]) = *reinterpret_cast<const float4*>(rk + c0);
            *reinterpret_cast<float4*>(&bq[4]) = *reinterpret_cast<const float4*>(rk + c0 + 4);
            if (diag) {
              *reinterpret_cast<float4*>(&f[0]) = *reinterpret_cast<const float4*>(sPS + R * DK + c0);
              *reinterpret_cast<float4*>(&f[4]) = *reinterpret_cast<const float4*>(sPS + R * DK + c0 + 4);
#pragma unroll
              for (int j = 0; j < 8; ++j) { a[j] *= f[j]; ak[j] *= f[j]; bq[j] *= f[j]; }
              bf16x8 ah, al, bh, bl, kh;
              split8(a, ah, al);
              split8(bq, bh, bl);
#pragma unroll
              for (int j = 0; j < 8; ++j) kh[j] = (__bf16)ak[j];
              accQ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, accQ, 0, 0, 0);
              accQ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, accQ, 0, 0, 0);
              accQ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, accQ, 0, 0, 0);
              accK = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, bh, accK, 0, 0, 0);
            } else {
#pragma unroll
              for (int j = 0; j < 8; ++j) f[j] = 1.f;
              for (int J = I + 1; J < R; ++J) {
                float g[8];
                *reinterpret_cast<float4*>(&g[0]) = *reinterpret_cast<const float4*>(sBB + J * DK + c0);
                *reinterpret_cast<float4*>(&g[4]) = *reinterpret_cast<const float4*>(sBB + J * DK + c0 + 4);
#pragma unroll
                for (int j = 0; j < 8; ++j) f[j] *= g[j];
              }
              half8 ah, kh, bh;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                ah[j] = (_Float16)a[j];
                kh[j] = (_Float16)ak[j];
                bh[j] = (_Float16)(bq[j] * f[j]);
              }
              accQ = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, accQ, 0, 0, 0);
              accK = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, bh, accK, 0, 0, 0);
            }
          }
        } else {
          const int kf = (l >> 4) * 4;
          for (int ks = 0; ks < DK / 16; ++ks) {
            const int c0 = ks * 16 + kf;
            float4 a = *reinterpret_cast<const float4*>(lq + c0);
            float4 ak = *reinterpret_cast<const float4*>(lk + c0);
            float4 bq = *reinterpret_cast<const float4*>(rk + c0);
            float4 f;
            if (diag) {
              f = *reinterpret_cast<const float4*>(sPS + R * DK + c0);
              a.x *= f.x; a.y *= f.y; a.z *= f.z; a.w *= f.w;
              ak.x *= f.x; ak.y *= f.y; ak.z *= f.z; ak.w *= f.w;
            } else {
              f = make_float4(1.f, 1.f, 1.f, 1.f);
              for (int J = I + 1; J < R; ++J) {
                const float4 g = *reinterpret_cast<const float4*>(sBB + J * DK + c0);
                f.x *= g.x; f.y *= g.y; f.z *= g.z; f.w *= g.w;
              }
            }
            bq.x *= f.x; bq.y *= f.y; bq.z *= f.z; bq.w *= f.w;
            accQ = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, bq.x, accQ, 0, 0, 0);
            accQ = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, bq.y, accQ, 0, 0, 0);
            accQ = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, bq.z, accQ, 0, 0, 0);
            accQ = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, bq.w, accQ, 0, 0, 0);
            accK = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.x, bq.x, accK, 0, 0, 0);
            accK = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.y, bq.y, accK, 0, 0, 0);
            accK = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.z, bq.z, accK, 0, 0, 0);
            accK = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.w, bq.w, accK, 0, 0, 0);
          }
        }
        // write out: lane holds rows 4*(l>>4)+i, column l&15 of the 16x16 tile
        const int ci = l & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ri = 4 * (l >> 4) + i;
          const int r = 16 * R + ri, cc = 16 * I + ci;
          const bool strict = !diag || ri > ci;
          const float akv = strict ? sBE[r] * accK[i] : 0.f;
          sAK[r * LDA + cc] = akv;
          sAQ[r * LDC + cc] = cvt<T>(strict ? accQ[i] : 0.f);
          if (diag && ri == ci) sDQ[r] = accQ[i];
          if (!diag) sAO[pair_index(R, I) * 256 + ri * 16 + ci] = cvt<T>(akv);
        }
      }
    }
    __syncthreads();  // ---------------------------------------------------------------- B3

    // ================= E3 (read) + UT inverse of the diagonal sub-blocks =================
    float qg[8][4], kg[8][4], kd[8][4];
    if (e_act) {
      float es[4], ee[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float pre = 1.f, post = 1.f;
        for (int J = 0; J < NB; ++J) {
          const float bj = sBB[J * DK + e_c0 + c];
          if (J < e_R) pre *= bj;
          if (J > e_R) post *= bj;
        }
        es[c] = pre;   // e^{G_{R-1}}
        ee[c] = post;  // e^{g_last - G_R}
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = e_r0 + i;
        const float4 a = *reinterpret_cast<const float4*>(sLQ + r * LDF + e_c0);
        const float4 b2 = *reinterpret_cast<const float4*>(sLK + r * LDF + e_c0);
        const float4 c2 = *reinterpret_cast<const float4*>(sRK + r * LDF + e_c0);
        qg[i][0] = a.x * es[0]; qg[i][1] = a.y * es[1]; qg[i][2] = a.z * es[2]; qg[i][3] = a.w * es[3];
        kg[i][0] = b2.x * es[0]; kg[i][1] = b2.y * es[1]; kg[i][2] = b2.z * es[2]; kg[i][3] = b2.w * es[3];
        kd[i][0] = c2.x * ee[0]; kd[i][1] = c2.y * ee[1]; kd[i][2] = c2.z * ee[2]; kd[i][3] = c2.w * ee[3];
      }
    }
    // diagonal 16x16 blocks of T = (I + A)^-1 by forward substitution: wave R,
    // lane (column j = l & 15, part p = l >> 4) keeps T[p + 4m][j], m = 0..3.
    if (wave < NB) {
      const int R = wave, j = l & 15, p = l >> 4;
      const float* Ab = sAK + (16 * R) * LDA + 16 * R;
      float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float sum = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int i = p + 4 * m;
          if (i < r) sum += Ab[r * LDA + i] * x[m];
        }
        sum += wave_xor(sum, 16);
        sum += wave_xor(sum, 32);
        const float t = (r == j ? 1.f : 0.f) - sum;
        if ((r & 3) == p) x[r >> 2] = t;
      }
      // in place: every lane has read all of its block's A rows above
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = p + 4 * m;
        sAK[(16 * R + i) * LDA + 16 * R + j] = x[m];
        sTB[(16 * R + i) * LDC + 16 * R + j] = cvt<T>(x[m] * sBE[16 * R + j]);
      }
    }
    __syncthreads();  // ---------------------------------------------------------------- B4

    // ================= E3 (write) + off-diagonal blocks of T, level 1 =================
    if (e_act) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        store4(sQG + (e_r0 + i) * LDD + e_c0, qg[i][0], qg[i][1], qg[i][2], qg[i][3]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        T* pg = sKGT + (e_c0 + c) * LDC + e_r0;
        T* pd = sKDT + (e_c0 + c) * LDC + e_r0;
        store4(pg, kg[0][c], kg[1][c], kg[2][c], kg[3][c]);
        store4(pg + 4, kg[4][c], kg[5][c], kg[6][c], kg[7][c]);
        store4(pd, kd[0][c], kd[1][c], kd[2][c], kd[3][c]);
        store4(pd + 4, kd[4][c], kd[5][c], kd[6][c], kd[7][c]);
      }
    }
    if (v_act) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        T* p = sVT + (v_c0 + c) * LDC + 2 * v_p;
        p[0] = cvt<T>(vv[0][c]);
        p[1] = cvt<T>(vv[1][c]);
      }
    }
    if constexpr (NB > 1) {
      // Tb lives in region 1: its strictly-upper 16x16 tiles hold stale bytes and
      // are read by the MMA steps that round the token range up to KS.
      for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) sTB[r * LDC + c] = cvt<T>(0.f);
      }
    }
    if constexpr (CK > C) {
      // zero the padded token columns [C, CK) of the token-k operands in region 1
      for (int idx = tid; idx < (2 * DK + C + 2 * BV) * (CK - C); idx += NT) {
        const int rowi = idx / (CK - C), col = C + idx % (CK - C);
        T* base;
        int rr;
        if (rowi < DK) { base = sKGT; rr = rowi; }
        else if (rowi < 2 * DK) { base = sKDT; rr = rowi - DK; }
        else if (rowi < 2 * DK + C) { base = sTB; rr = rowi - 2 * DK; }
        else if (rowi < 2 * DK + C + BV) { base = sUT; rr = rowi - 2 * DK - C; }
        else { base = sVT; rr = rowi - 2 * DK - C - BV; }
        base[rr * LDC + col] = cvt<T>(0.f);
      }
    }
    // off-diagonal blocks: T_RI = -T_RR sum_{J=I}^{R-1} A_RJ T_JI, level d = R - I
    for (int d = 1; d < NB; ++d) {
      const int R = d + wave, I = wave;
      if (R < NB) {
        f32x4 X = zero4();
        const int kq = 4 * (l >> 4), nn = l & 15, mm = l & 15;
        for (int J = I; J < R; ++J) {
          const T* Aj = sAO + pair_index(R, J) * 256;
          float a4[4], b4[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            a4[jj] = (float)Aj[mm * 16 + kq + jj];
            b4[jj] = sAK[(16 * J + kq + jj) * LDA + 16 * I + nn];
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) X = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[jj], b4[jj], X, 0, 0, 0);
        }
        // Y = T_RR X ; the accumulator layout of X is the B operand layout (k = 4(l>>4)+i)
        f32x4 Y = zero4();
        const float4 tr = *reinterpret_cast<const float4*>(sAK + (16 * R + mm) * LDA + 16 * R + kq);
        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tr.x, X[0], Y, 0, 0, 0);
        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tr.y, X[1], Y, 0, 0, 0);
        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tr.z, X[2], Y, 0, 0, 0);
        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tr.w, X[3], Y, 0, 0, 0);
        const float bcol = sBE[16 * I + nn];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * R + kq + i;
          sAK[r * LDA + 16 * I + nn] = -Y[i];
          sTB[r * LDC + 16 * I + nn] = cvt<T>(-Y[i] * bcol);
        }
      }
      __syncthreads();  // ------------------------------------------------------ B5 (per level)
    }
    if (NB == 1) __syncthreads();

    // ================= WY stage: W^T = Kg^T Tb^T ; Ut = Tb V =================
    {
#pragma unroll
      for (int s = 0; s < (NA * NB + NW - 1) / NW; ++s) {
        const int id = wave + NW * s;
        if (id < NA * NB) {
          const int a = id % NA, R = id / NA;
          f32x4 acc = zero4();
          const int nst = (16 * R + 16 + KS - 1) / KS;
          mma_tile<T, KS>(acc, sKGT + 16 * a * LDC, LDC, sTB + 16 * R * LDC, LDC, nst);
          // acc rows = channels 16a + 4(l>>4) + i, column = token 16R + (l&15)
          store4(sW + (16 * R + (l & 15)) * LDD + 16 * a + 4 * (l >> 4), acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
    f32x4 Uacc[U_SLOTS], Oacc[U_SLOTS];
#pragma unroll
    for (int s = 0; s < U_SLOTS; ++s) {
      const int id = wave + NW * s;
      Uacc[s] = zero4();
      Oacc[s] = zero4();
      if (id < NB * NJ) {
        const int R = id % NB, j = id / NB;
        const int nst = (16 * R + 16 + KS - 1) / KS;
        mma_tile<T, KS>(Uacc[s], sTB + 16 * R * LDC, LDC, sVT + 16 * j * LDC, LDC, nst);
      }
    }
    __syncthreads();  // ---------------------------------------------------------------- B6

    // ================= state stage 1: U = Ut - W S ; O = Qg S =================
#pragma unroll
    for (int s = 0; s < U_SLOTS; ++s) {
      const int id = wave + NW * s;
      if (id < NB * NJ) {
        const int R = id % NB, j = id / NB;
        f32x4 ws = zero4();
        mma_tile<T, KS>(ws, sW + 16 * R * LDD, LDD, sST + 16 * j * LDD, LDD, DK / KS);
        mma_tile<T, KS>(Oacc[s], sQG + 16 * R * LDD, LDD, sST + 16 * j * LDD, LDD, DK / KS);
#pragma unroll
        for (int i = 0; i < 4; ++i) Uacc[s][i] -= ws[i];
        // U^T [BV][CK]: lane holds U[token 16R + 4(l>>4) + i][column 16j + (l&15)]
        store4(sUT + (16 * j + (l & 15)) * LDC + 16 * R + 4 * (l >> 4), Uacc[s][0], Uacc[s][1], Uacc[s][2],
               Uacc[s][3]);
      }
    }
    __syncthreads();  // ---------------------------------------------------------------- B7

    // ================= state stage 2: O += M U ; S <- e^{g} S + Kd^T U =================
#pragma unroll
    for (int s = 0; s < U_SLOTS; ++s) {
      const int id = wave + NW * s;
      if (id < NB * NJ) {
        const int R = id % NB, j = id / NB;
        const int nst = (16 * R + 16 + KS - 1) / KS;
        mma_tile<T, KS>(Oacc[s], sAQ + 16 * R * LDC, LDC, sUT + 16 * j * LDC, LDC, nst);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * R + 4 * (l >> 4) + i;
          const float ov = Oacc[s][i] + sDQ[r] * Uacc[s][i];
          if (r < Lc) o[((size_t)(c_begin + r) * H + h) * DV + j0 + 16 * j + (l & 15)] = ov;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < S_SLOTS; ++s) {
      const int id = wave + NW * s;
      if (id < NA * NJ) {
        const int a = id % NA, j = id / NA;
#pragma unroll
        for (int i = 0; i < 4; ++i) Sacc[s][i] *= sGM[16 * a + 4 * (l >> 4) + i];
        mma_tile<T, KS>(Sacc[s], sKDT + 16 * a * LDC, LDC, sUT + 16 * j * LDC, LDC, CK / KS);
      }
    }
    write_ST();
    // the next chunk's first barrier (B1) orders these reads/writes against region 1 reuse
  }

  if (hT) {
    float* hp = hT + (size_t)chain * DK * DV;
#pragma unroll
    for (int s = 0; s < S_SLOTS; ++s) {
      const int id = wave + NW * s;
      if (id < NA * NJ) {
        const int a = id % NA, j = id / NA;
#pragma unroll
        for (int i = 0; i < 4; ++i) hp[(size_t)(16 * a + 4 * (l >> 4) + i) * DV + j0 + 16 * j + (l & 15)] = Sacc[s][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
template <int C, int DK, int BV, Prec P, typename InT>
static hipError_t launch_one(const ChunkArgs& a) {
  constexpr size_t lds = lds_bytes<C, DK, BV, P>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = chunk_fwd_kernel<C, DK, BV, P, InT>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_chains = a.n_seqs * a.n_heads;
  const int ntile = a.dv / BV;
  const int grid = ((n_chains + 7) / 8) * 8 * ntile;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), lds, (hipStream_t)a.stream, (const InT*)a.q, (const InT*)a.k,
                     (const InT*)a.v, a.log_alpha, a.beta, a.h0, a.cu_seqlens, a.o, a.hT, n_chains, a.n_heads, a.dv,
                     a.seq_len);
  return hipGetLastError();
}

// value-tile width: the widest that still gives at least one workgroup per CU
static int pick_bv(int n_chains, int dv, int max_bv) {
  for (int bv = max_bv; bv >= 16; bv /= 2)
    if (dv % bv == 0 && (int64_t)n_chains * (dv / bv) >= 256) return bv;
  return 16;
}

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
      if (a.chunk_size == 64) return dispatch_bv<64, DK, 16, P, InT>(a);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace chunkk

bool chunk_fwd_supported(int dk, int dv, int chunk_size, bool bf16) {
  if (!((dk == 64 || dk == 128) && (dv == 64 || dv == 128))) return false;
  if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return false;
  if (!bf16 && dk == 128 && chunk_size == 64) return false;
  return true;
}

hipError_t launch_chunk_fwd(const ChunkArgs& a) {
  using namespace chunkk;
  if (!chunk_fwd_supported(a.dk, a.dv, a.chunk_size, a.bf16)) return hipErrorInvalidValue;
  if (a.bf16) {
    return a.dk == 128 ? dispatch_c<128, Prec::Mixed, bf16_t>(a) : dispatch_c<64, Prec::Mixed, bf16_t>(a);
  }
  return a.dk == 128 ? dispatch_c<128, Prec::F32, float>(a) : dispatch_c<64, Prec::F32, float>(a);
}

}  // namespace kda
