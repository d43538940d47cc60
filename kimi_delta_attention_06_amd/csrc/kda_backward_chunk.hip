// Chunkwise backward pass of KDA on gfx950: the reverse mode of the chunk form,
// every product on the fp32 matrix core.
//
// Training needs the gradients of KDA beyond the published inference forward
// ("Kimi K3 NPU Training", conclusions, item 1, and the NPU operator-support table,
// KDA backward row).  The forward is chunkwise ("Kimi K3 technical report summary",
// section 1, pre-training table, KDA row; the DPLR chunk kernel of "Kimi K3 NPU
// Training", section "NPU operator support"), and so is its reverse mode here.  For
// one chunk of C = 16 tokens with entering state S, rows i = 0..C-1, per-channel
// cumulative log-decay g_i and g_L = g_{C-1} (rows past a sequence end have zero
// inputs and zero decay):
//
//   Qg = Q * e^G,  Kg = K * e^G,  Kc = K * e^{g_L - G},  e_L = e^{g_L}
//   A[i][j] = sum_c k_ic k_jc e^{g_ic - g_jc}  (j < i),   M[i][j] = same with q_i (j <= i)
//   T = (I + Diag(b) A)^-1,   Y = V - Kg S,   U = T Diag(b) Y
//   O = Qg S + M U,           S' = Diag(e_L) S + Kc^T U
//
// and for the cotangents dO and dS' of the outputs (the adjoint of each line above,
// taken in reverse order):
//
//   dU = M^T dO + Kc dS',   lambda = T^T dU,   dY = Diag(b) lambda  (= dV)
//   dS = Diag(e_L) dS' + Qg^T dO - Kg^T dY              (cotangent of the entering state)
//   db_i = lambda_i . (Y - A U)_i
//   dM = tril(dO U^T),  dA = -strict_tril(dY U^T),  dQg = dO S^T,  dKg = -dY S^T,  dKc = U dS'^T
//
// then the chain rule through the decay factors: for the Gram terms, with
// P = (dM o E) K, R = (dM o E)^T Q, P' = (dA o E) K, R' = (dA o E)^T K (E the decay
// e^{g_i - g_j} per channel),
//   dq = dQg e^G + P
//   dk = dKg e^G + dKc e^{g_L - G} + R + P' + R'
//   dg = q (dQg e^G + P) + k (dKg e^G - dKc e^{g_L - G} - R + P' - R')
//        + [last row] (e_L sum_v S dS' + sum_i k_i dKc_i e^{g_L - g_i})
//   dlog a_t = sum_{i >= t} dg_i                     (g is the prefix sum of log a)
//
// Decay balancing.  Gram products take their decay from the chunk midpoint m = g_L / 2:
// left operands x_i e^{g_i - m}, right operands k_j e^{m - g_j}, each at most e^{|g_L|/2},
// on the matrix core.  A chunk that decays by more than 64 nats in some channel (where those
// operands, times the values they scale, could leave the fp32 range) forms the Gram terms from
// per-element factors e^{g_i - g_j} <= 1 instead, so any finite log a is taken.
//
// Three launches: (1) the forward chunk kernel in fp32 stores the state entering every
// chunk (its checkpoint output at a 16-token spacing); (2) `bwd_ds_kernel` walks each
// (sequence, head, value tile) backwards over its chunks, keeping dS in registers and
// storing the dS' of every chunk; (3) `bwd_grad_kernel` takes one (chunk, head) per
// workgroup, all in parallel, and forms every gradient of the chunk from its S and dS'.
#include <atomic>

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace bwdc {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 16;        // tokens per chunk
constexpr int NT = 512;      // threads per workgroup (8 waves)
constexpr int LDC = C + 4;   // row stride of the 16 x 16 tiles

__device__ __forceinline__ int lane() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// acc += A B^T over k in [0, 16 NS): A(i, k) = A[i*AI + k*AK], B(j, k) = B[j*BJ + k*BK].
// Lane l supplies row i = j = l & 15 and k = 16 s + 4 (l >> 4) + e (e = 0..3, one fp32
// MFMA each: the same k permutation for both operands).  acc[r] is C[4 (l >> 4) + r][l & 15].
template <int NS, int AI, int AK, int BJ, int BK>
__device__ __forceinline__ void mma(f32x4& acc, const float* A, const float* B) {
  const int l = lane();
  const float* a = A + (l & 15) * AI + 4 * (l >> 4) * AK;
  const float* b = B + (l & 15) * BJ + 4 * (l >> 4) * BK;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float4 fa, fb;
    if constexpr (AK == 1) {
      fa = *reinterpret_cast<const float4*>(a + 16 * s);
    } else {
      fa = make_float4(a[(16 * s) * AK], a[(16 * s + 1) * AK], a[(16 * s + 2) * AK], a[(16 * s + 3) * AK]);
    }
    if constexpr (BK == 1) {
      fb = *reinterpret_cast<const float4*>(b + 16 * s);
    } else {
      fb = make_float4(b[(16 * s) * BK], b[(16 * s + 1) * BK], b[(16 * s + 2) * BK], b[(16 * s + 3) * BK]);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.x, fb.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.y, fb.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.z, fb.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.w, fb.w, acc, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_tile(float* p, int ld, const f32x4& acc) {
  const int l = lane();
#pragma unroll
  for (int r = 0; r < 4; ++r) p[(4 * (l >> 4) + r) * ld + (l & 15)] = acc[r];
}
__device__ __forceinline__ void add_tile(f32x4& acc, const float* p, int ld) {
  const int l = lane();
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] += p[(4 * (l >> 4) + r) * ld + (l & 15)];
}

template <typename InT> struct Vec;
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(float* d, const float* s) {
    const float4 x = *reinterpret_cast<const float4*>(s);
    d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
  }
};
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ static void load(float* d, const bf16_t* s) {
    const uint4 x = *reinterpret_cast<const uint4*>(s);
    float2 f;
    f = bf16x2_to_f32x2(x.x); d[0] = f.x; d[1] = f.y;
    f = bf16x2_to_f32x2(x.y); d[2] = f.x; d[3] = f.y;
    f = bf16x2_to_f32x2(x.z); d[4] = f.x; d[5] = f.y;
    f = bf16x2_to_f32x2(x.w); d[6] = f.x; d[7] = f.y;
  }
};

// 16 bytes of input (8 bf16 or 4 fp32 values), widened to fp32 at d
__device__ __forceinline__ void widen16(float* d, const uint4& x, bf16_t) {
  float2 f;
  f = bf16x2_to_f32x2(x.x); d[0] = f.x; d[1] = f.y;
  f = bf16x2_to_f32x2(x.y); d[2] = f.x; d[3] = f.y;
  f = bf16x2_to_f32x2(x.z); d[4] = f.x; d[5] = f.y;
  f = bf16x2_to_f32x2(x.w); d[6] = f.x; d[7] = f.y;
}
__device__ __forceinline__ void widen16(float* d, const uint4& x, float) {
  d[0] = __uint_as_float(x.x); d[1] = __uint_as_float(x.y); d[2] = __uint_as_float(x.z); d[3] = __uint_as_float(x.w);
}

// The per-chunk operands both kernels form (LDS, fp32).
template <int DK>
struct Intra {
  static constexpr int LDK = DK + 4;
  static constexpr int FLOATS = 9 * C * LDK + 4 * C * LDC + C + DK;
  float *q, *k, *g, *ql, *kl, *kr, *qg, *kg, *kc;  // [C][LDK]; g holds log a until the prefix sum
  float *A, *M, *T, *TB;                           // [C][LDC]; TB = T Diag(b)
  float *b;                                        // [C]
  float *el;                                       // [DK], e^{g_L}
  __device__ explicit Intra(float* s) {
    q = s; k = q + C * LDK; g = k + C * LDK; ql = g + C * LDK; kl = ql + C * LDK; kr = kl + C * LDK;
    qg = kr + C * LDK; kg = qg + C * LDK; kc = kg + C * LDK;
    A = kc + C * LDK; M = A + C * LDC; T = M + C * LDC; TB = T + C * LDC;
    b = TB + C * LDC; el = b + C;
  }

  // q, k, log a and b of rows t0 .. t0 + Lc - 1 (zeros past Lc)
  template <typename InT>
  __device__ void load(const InT* __restrict__ qp, const InT* __restrict__ kp, const float* __restrict__ lap,
                       const float* __restrict__ bp, int64_t t0, int Lc, int H, int h) {
    constexpr int VE = Vec<InT>::N, NV = C * DK / VE;
    for (int e = threadIdx.x; e < 2 * NV; e += NT) {
      const int which = e / NV, ee = e - which * NV;
      const int i = ee / (DK / VE), c = (ee - i * (DK / VE)) * VE;
      float x[VE];
      if (i < Lc) {
        Vec<InT>::load(x, (which ? kp : qp) + ((size_t)(t0 + i) * H + h) * DK + c);
      } else {
#pragma unroll
        for (int u = 0; u < VE; ++u) x[u] = 0.f;
      }
      float* d = (which ? k : q) + i * LDK + c;
#pragma unroll
      for (int u = 0; u < VE; u += 4) *reinterpret_cast<float4*>(d + u) = make_float4(x[u], x[u + 1], x[u + 2], x[u + 3]);
    }
    for (int e = threadIdx.x; e < C * DK / 4; e += NT) {
      const int i = e / (DK / 4), c = (e - i * (DK / 4)) * 4;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < Lc) x = *reinterpret_cast<const float4*>(lap + ((size_t)(t0 + i) * H + h) * DK + c);
      *reinterpret_cast<float4*>(g + i * LDK + c) = x;
    }
    if (threadIdx.x < C) b[threadIdx.x] = (int)threadIdx.x < Lc ? bp[(size_t)(t0 + threadIdx.x) * H + h] : 0.f;
  }

  // Prefix sum of log a over the rows (one thread per channel) and e^{g_L}.  Each step is
  // floored at -110 nats: e^{-110} is 0 in fp32 like e^{x} for every x below it, so the floor
  // changes nothing an fp32 evaluation can represent, the sums stay finite for any finite log a,
  // and differences of nearby sums keep their precision.  Returns true for a channel whose
  // chunk decays by more than kBalancedNats.
  static constexpr float kBalancedNats = 64.f;
  __device__ bool prefix() {
    const int c = threadIdx.x;
    bool wide = false;
    if (c < DK) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const float x = g[i * LDK + c];
        s += x < -110.f ? -110.f : x;  // (a NaN stays NaN)
        g[i * LDK + c] = s;
      }
      el[c] = expf(s);
      wide = !(s >= -kBalancedNats);
    }
    return wide;
  }

  // Decay-scaled operands, every element.  `exact` (a chunk decaying by more than kBalancedNats
  // in some channel): the midpoint-balanced Gram operands ql, kl, kr would overflow, so they are
  // not formed and the Gram terms take their per-element factors instead (gram_exact and the
  // exact branch of the gradient pass).
  __device__ void scale(bool exact) {
    for (int e = threadIdx.x; e < C * DK; e += NT) {
      const int i = e / DK, c = e - i * DK, o = i * LDK + c;
      const float gi = g[o], gl = g[(C - 1) * LDK + c], m = 0.5f * gl;
      const float eg = expf(gi), ec = expf(gl - gi);
      const float qv = q[o], kv = k[o];
      if (!exact) {
        const float e1 = expf(gi - m), e2 = expf(m - gi);
        ql[o] = qv * e1;
        kl[o] = kv * e1;
        kr[o] = kv * e2;
      }
      qg[o] = qv * eg;
      kg[o] = kv * eg;
      kc[o] = kv * ec;
    }
  }

  // A and M from per-element decay factors e^{g_ic - g_jc} <= 1 (j <= i): one thread per
  // (i, j) pair, threads 0 .. 255
  __device__ void gram_exact() {
    const int t = threadIdx.x, i = t >> 4, j = t & 15;
    float a = 0.f, m = 0.f;
    if (j <= i) {
      for (int c = 0; c < DK; ++c) {
        const float kj = k[j * LDK + c] * expf(fminf(g[i * LDK + c] - g[j * LDK + c], 0.f));
        a = fmaf(k[i * LDK + c], kj, a);
        m = fmaf(q[i * LDK + c], kj, m);
      }
    }
    A[i * LDC + j] = j < i ? a : 0.f;
    M[i * LDC + j] = m;
  }

  // wave 0: A (strictly lower), wave 1: M (lower with the diagonal)
  __device__ void gram(int w) {
    f32x4 acc = zero4();
    mma<DK / 16, LDK, 1, LDK, 1>(acc, w == 0 ? kl : ql, kr);
    const int l = lane(), j = l & 15;
    float* dst = w == 0 ? A : M;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * (l >> 4) + r;
      dst[i * LDC + j] = (w == 0 ? j < i : j <= i) ? acc[r] : 0.f;
    }
  }

  // one wave: T = (I + Diag(b) A)^-1 by forward substitution, lane j owning column j
  __device__ void inverse() {
    const int j = lane() & 15;
    float tc[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      float s = 0.f;
#pragma unroll
      for (int kk = 0; kk < i; ++kk) s += A[i * LDC + kk] * tc[kk];
      tc[i] = i == j ? 1.f : (i > j ? -b[i] * s : 0.f);
    }
    if (lane() < 16) {
      const float bj = b[j];
#pragma unroll
      for (int i = 0; i < C; ++i) {
        T[i * LDC + j] = tc[i];
        TB[i * LDC + j] = tc[i] * bj;
      }
    }
  }
};

__device__ __forceinline__ void seq_range(const int32_t* cu, int n, int64_t seq_len, int64_t& start, int64_t& len) {
  if (cu) {
    start = cu[n];
    len = (int64_t)cu[n + 1] - cu[n];
  } else {
    start = (int64_t)n * seq_len;
    len = seq_len;
  }
}

// ---------------------------------------------------------------------------------------------
// dS pass: one workgroup per (sequence, head, BV value columns), chunks in reverse order.
// dS (DK x BV) lives in MFMA accumulators: wave w owns tiles tt = w + 8 u, c-tile tt % (DK/16),
// v-tile tt / (DK/16).  Stores dS' of chunk j at workspace slot start/16 + n + j.
template <int DK, int BV, typename InT>
__global__ __launch_bounds__(NT) void bwd_ds_kernel(const InT* __restrict__ q, const InT* __restrict__ k,
                                                    const float* __restrict__ la, const float* __restrict__ beta,
                                                    const int32_t* __restrict__ cu, const float* __restrict__ dout,
                                                    const float* __restrict__ dhT, float* __restrict__ dsw,
                                                    float* __restrict__ dh0, int H, int DV, int64_t seq_len) {
  using In = Intra<DK>;
  constexpr int LDK = In::LDK, LDO = BV + 4;
  constexpr int NVT = BV / 16, NCT = DK / 16, NTL = NCT * NVT, TPW = NTL / 8;
  constexpr int KSPLIT = 8 / NVT, KR = DK / KSPLIT;
  static_assert(NTL % 8 == 0 && 8 % NVT == 0 && KR % 16 == 0, "tiling");

  extern __shared__ __attribute__((aligned(16))) float smem[];
  In in(smem);
  float* sDO = smem + In::FLOATS;     // [C][LDO]
  float* sDST = sDO + C * LDO;        // [BV][LDK]: dS' transposed
  float* sPart = sDST + BV * LDK;     // [8][C][LDC]
  float* sDU = sPart + 8 * C * LDC;   // [C][LDO]
  float* sNDY = sDU + C * LDO;        // [C][LDO]: -dY

  const int ntile = DV / BV;
  const int chain = blockIdx.x / ntile, tile = blockIdx.x - chain * ntile;
  const int n = chain / H, h = chain - n * H, v0 = tile * BV;
  int64_t start, len;
  seq_range(cu, n, seq_len, start, len);
  const int64_t nch = (len + C - 1) / C;
  const int w = threadIdx.x / kWave, l = lane();

  f32x4 ds[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tt = w + 8 * u, ct = tt % NCT, vt = tt / NCT;
    const int crow = 16 * ct + 4 * (l >> 4), vcol = 16 * vt + (l & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      ds[u][r] = dhT ? dhT[((size_t)chain * DK + crow + r) * DV + v0 + vcol] : 0.f;
    *reinterpret_cast<float4*>(sDST + vcol * LDK + crow) = make_float4(ds[u][0], ds[u][1], ds[u][2], ds[u][3]);
  }
  const int64_t slot0 = start / C + n;

  // The inputs of the next chunk (in reverse order) are loaded into registers while the
  // current one is processed: q, k (16 bytes per item), log a and dO (float4), beta.
  constexpr int VE = Vec<InT>::N, NV = C * DK / VE;
  constexpr int IQK = (2 * NV + NT - 1) / NT, ILA = (C * DK / 4 + NT - 1) / NT, IDO = (C * BV / 4 + NT - 1) / NT;
  uint4 rqk[IQK];
  float4 rla[ILA], rdo[IDO];
  float rb = 0.f;
  auto fetch = [&](int64_t jj) {
    const int64_t t0 = start + C * jj;
    const int Lc = (int)(len - C * jj < C ? len - C * jj : C);
#pragma unroll
    for (int it = 0; it < IQK; ++it) {
      const int e = threadIdx.x + NT * it, which = e / NV, ee = e - which * NV;
      const int i = ee / (DK / VE), c = (ee - i * (DK / VE)) * VE;
      rqk[it] = make_uint4(0u, 0u, 0u, 0u);
      if (e < 2 * NV && i < Lc)
        rqk[it] = *reinterpret_cast<const uint4*>((which ? k : q) + ((size_t)(t0 + i) * H + h) * DK + c);
    }
#pragma unroll
    for (int it = 0; it < ILA; ++it) {
      const int e = threadIdx.x + NT * it, i = e / (DK / 4), c = (e - i * (DK / 4)) * 4;
      rla[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < C * DK / 4 && i < Lc) rla[it] = *reinterpret_cast<const float4*>(la + ((size_t)(t0 + i) * H + h) * DK + c);
    }
#pragma unroll
    for (int it = 0; it < IDO; ++it) {
      const int e = threadIdx.x + NT * it, i = e / (BV / 4), c = (e - i * (BV / 4)) * 4;
      rdo[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < C * BV / 4 && i < Lc)
        rdo[it] = *reinterpret_cast<const float4*>(dout + ((size_t)(t0 + i) * H + h) * DV + v0 + c);
    }
    rb = (int)threadIdx.x < Lc ? beta[(size_t)(t0 + threadIdx.x) * H + h] : 0.f;
  };
  auto put = [&]() {
#pragma unroll
    for (int it = 0; it < IQK; ++it) {
      const int e = threadIdx.x + NT * it, which = e / NV, ee = e - which * NV;
      const int i = ee / (DK / VE), c = (ee - i * (DK / VE)) * VE;
      if (e < 2 * NV) widen16((which ? in.k : in.q) + i * LDK + c, rqk[it], InT{});
    }
#pragma unroll
    for (int it = 0; it < ILA; ++it) {
      const int e = threadIdx.x + NT * it, i = e / (DK / 4), c = (e - i * (DK / 4)) * 4;
      if (e < C * DK / 4) *reinterpret_cast<float4*>(in.g + i * LDK + c) = rla[it];
    }
#pragma unroll
    for (int it = 0; it < IDO; ++it) {
      const int e = threadIdx.x + NT * it, i = e / (BV / 4), c = (e - i * (BV / 4)) * 4;
      if (e < C * BV / 4) *reinterpret_cast<float4*>(sDO + i * LDO + c) = rdo[it];
    }
    if (threadIdx.x < C) in.b[threadIdx.x] = rb;
  };
  if (nch > 0) fetch(nch - 1);

  for (int64_t j = nch - 1; j >= 0; --j) {
    put();
    if (j > 0) fetch(j - 1);
    {
      float* dst = dsw + ((size_t)(slot0 + j) * H + h) * DK * DV;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tt = w + 8 * u, ct = tt % NCT, vt = tt / NCT;
        const int crow = 16 * ct + 4 * (l >> 4), vcol = 16 * vt + (l & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(size_t)(crow + r) * DV + v0 + vcol] = ds[u][r];
      }
    }
    __syncthreads();
    const bool exact = __syncthreads_or(in.prefix());
    in.scale(exact);
    __syncthreads();
    if (exact) {
      if (w < 4) in.gram_exact();
    } else if (w < 2) {
      in.gram(w);
    }
    {  // partial Kc dS' over one k-range: job w = (v-tile w % NVT, k-range w / NVT)
      const int vt = w % NVT, kq = w / NVT;
      f32x4 acc = zero4();
      mma<KR / 16, LDK, 1, LDK, 1>(acc, in.kc + kq * KR, sDST + 16 * vt * LDK + kq * KR);
      store_tile(sPart + w * C * LDC, LDC, acc);
    }
    __syncthreads();
    if (w == 0) in.inverse();
    if (w >= 8 - NVT) {  // dU = M^T dO + Kc dS'
      const int vt = w - (8 - NVT);
      f32x4 acc = zero4();
      mma<1, 1, LDC, 1, LDO>(acc, in.M, sDO + 16 * vt);
#pragma unroll
      for (int kq = 0; kq < KSPLIT; ++kq) add_tile(acc, sPart + (vt + kq * NVT) * C * LDC, LDC);
      store_tile(sDU + 16 * vt, LDO, acc);
    }
    __syncthreads();
    if (w >= 8 - NVT) {  // lambda = T^T dU; -dY = -b lambda
      const int vt = w - (8 - NVT);
      f32x4 acc = zero4();
      mma<1, 1, LDC, 1, LDO>(acc, in.T, sDU + 16 * vt);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        sNDY[i * LDO + 16 * vt + (l & 15)] = -in.b[i] * acc[r];
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TPW; ++u) {  // dS = Diag(e_L) dS' + Qg^T dO - Kg^T dY
      const int tt = w + 8 * u, ct = tt % NCT, vt = tt / NCT;
      const int crow = 16 * ct + 4 * (l >> 4), vcol = 16 * vt + (l & 15);
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = in.el[crow + r] * ds[u][r];
      mma<1, 1, LDK, 1, LDO>(acc, in.qg + 16 * ct, sDO + 16 * vt);
      mma<1, 1, LDK, 1, LDO>(acc, in.kg + 16 * ct, sNDY + 16 * vt);
      ds[u] = acc;
      *reinterpret_cast<float4*>(sDST + vcol * LDK + crow) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();
  }
  if (dh0) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + 8 * u, ct = tt % NCT, vt = tt / NCT;
      const int crow = 16 * ct + 4 * (l >> 4), vcol = 16 * vt + (l & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) dh0[((size_t)chain * DK + crow + r) * DV + v0 + vcol] = ds[u][r];
    }
  }
}

template <int DK, int BV>
constexpr size_t ds_lds_bytes() {
  constexpr int LDK = Intra<DK>::LDK, LDO = BV + 4;
  return sizeof(float) * ((size_t)Intra<DK>::FLOATS + 3 * C * LDO + (size_t)BV * LDK + 8 * C * LDC);
}

// ---------------------------------------------------------------------------------------------
// Gradient pass: one workgroup per (chunk slot, head).  Value columns in tiles of BV = 32:
// per tile, S and dS' columns are staged in LDS and the dv-reductions (dQg, dKg, dKc, dM, dA,
// db and sum_v S dS') accumulate in registers.
template <int DK, int DV, typename InT>
__global__ __launch_bounds__(NT) void bwd_grad_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v, const float* __restrict__ la,
    const float* __restrict__ beta, const float* __restrict__ h0, const int32_t* __restrict__ cu,
    const float* __restrict__ dout, const float* __restrict__ ckpt, const float* __restrict__ dsw,
    float* __restrict__ dq, float* __restrict__ dk_out, float* __restrict__ dv_out, float* __restrict__ dla,
    float* __restrict__ dbeta, int H, int64_t seq_len, int n_seqs) {
  using In = Intra<DK>;
  constexpr int BV = 32, LDK = In::LDK, LDO = DV + 4, LDB = BV + 4, LDY = BV + 4;
  constexpr int NCT = DK / 16, NTV = DV / BV, UPT = DK * BV / 4 / NT;
  constexpr int XW0 = NCT % 8, XW1 = (NCT + 1) % 8, XW2 = (NCT + 2) % 8;
  static_assert(NCT <= 8 && UPT >= 1 && DK * BV / 4 % NT == 0, "tiling");

  extern __shared__ __attribute__((aligned(16))) float smem[];
  In in(smem);
  float* sDO = smem + In::FLOATS;  // [C][LDO]
  float* sS = sDO + C * LDO;       // [DK][LDB]
  float* sD = sS + DK * LDB;       // [DK][LDB]
  float* sPart = sD + DK * LDB;    // [8][C][LDC]
  float* sY = sPart + 8 * C * LDC; // [C][LDY]
  float* sDU = sY + C * LDY;
  float* sU = sDU + C * LDY;
  float* sL = sU + C * LDY;        // lambda
  float* sDY = sL + C * LDY;
  float* sDM = sDY + C * LDY;      // [C][LDC]
  float* sDA = sDM + C * LDC;
  float* sGS = sDA + C * LDC;      // [DK]: sum_v S dS'

  const int slot = blockIdx.x / H, h = blockIdx.x - slot * H;
  // the sequence of this slot: the last n with start(n) / C + n <= slot
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t st = cu ? (int64_t)cu[mid] : (int64_t)mid * seq_len;
    if (st / C + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  const int n = lo;
  int64_t start, len;
  seq_range(cu, n, seq_len, start, len);
  const int64_t j = (int64_t)slot - (start / C + n);
  if (j < 0 || C * j >= len) return;  // a slot no chunk maps to (whole workgroup)
  const int64_t t0 = start + C * j;
  const int Lc = (int)(len - C * j < C ? len - C * j : C);
  const int chain = n * H + h;
  const float* S0 = j == 0 ? (h0 ? h0 + (size_t)chain * DK * DV : nullptr)
                           : ckpt + ((size_t)((start + C * j) / C - 1) * H + h) * DK * DV;
  const float* dSC = dsw + ((size_t)slot * H + h) * DK * DV;
  const int w = threadIdx.x / kWave, l = lane();

  // S and dS' columns of value tile tv, in registers: the next tile's are in flight while
  // the current one is worked on (the first tile's beside the chunk's input loads)
  float4 pS[UPT], pD[UPT];
  auto fetch = [&](int tv) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int e = threadIdx.x + NT * u, c = e / (BV / 4), c4 = (e - c * (BV / 4)) * 4;
      pS[u] = S0 ? *reinterpret_cast<const float4*>(S0 + (size_t)c * DV + tv * BV + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
      pD[u] = *reinterpret_cast<const float4*>(dSC + (size_t)c * DV + tv * BV + c4);
    }
  };
  fetch(0);
  in.load(q, k, la, beta, t0, Lc, H, h);
  for (int e = threadIdx.x; e < C * DV / 4; e += NT) {
    const int i = e / (DV / 4), c = (e - i * (DV / 4)) * 4;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < Lc) x = *reinterpret_cast<const float4*>(dout + ((size_t)(t0 + i) * H + h) * DV + c);
    *reinterpret_cast<float4*>(sDO + i * LDO + c) = x;
  }
  __syncthreads();
  const bool exact = __syncthreads_or(in.prefix());
  in.scale(exact);
  __syncthreads();
  if (exact) {
    if (w < 4) in.gram_exact();
  } else if (w < 2) {
    in.gram(w);
  }
  __syncthreads();
  if (w == 0) in.inverse();

  f32x4 aQ = zero4(), aK = zero4(), aC = zero4(), aX = zero4(), db = zero4();
  float gs[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) gs[u] = 0.f;

  for (int tv = 0; tv < NTV; ++tv) {
    const int vb = tv * BV;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {  // stage S and dS' columns [vb, vb + BV)
      const int e = threadIdx.x + NT * u, c = e / (BV / 4), c4 = (e - c * (BV / 4)) * 4;
      const float4 s4 = pS[u], d4 = pD[u];
      *reinterpret_cast<float4*>(sS + c * LDB + c4) = s4;
      *reinterpret_cast<float4*>(sD + c * LDB + c4) = d4;
      gs[u] += s4.x * d4.x + s4.y * d4.y + s4.z * d4.z + s4.w * d4.w;
    }
    if (tv + 1 < NTV) fetch(tv + 1);
    __syncthreads();
    {  // partial Kg S (waves 0-3) and Kc dS' (waves 4-7) over one half of the channels
      const int vt = w & 1, kh = (w >> 1) & 1;
      f32x4 acc = zero4();
      if (w < 4) mma<DK / 32, LDK, 1, 1, LDB>(acc, in.kg + kh * (DK / 2), sS + kh * (DK / 2) * LDB + 16 * vt);
      else mma<DK / 32, LDK, 1, 1, LDB>(acc, in.kc + kh * (DK / 2), sD + kh * (DK / 2) * LDB + 16 * vt);
      store_tile(sPart + w * C * LDC, LDC, acc);
    }
    __syncthreads();
    if (w < 2) {  // Y = V - Kg S
      const int vt = w;
      f32x4 acc = zero4();
      add_tile(acc, sPart + vt * C * LDC, LDC);
      add_tile(acc, sPart + (vt + 2) * C * LDC, LDC);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        float vv = 0.f;
        if (i < Lc) vv = to_f32(v[((size_t)(t0 + i) * H + h) * DV + vb + 16 * vt + (l & 15)]);
        sY[i * LDY + 16 * vt + (l & 15)] = vv - acc[r];
      }
    } else if (w < 4) {  // dU = M^T dO + Kc dS'
      const int vt = w - 2;
      f32x4 acc = zero4();
      mma<1, 1, LDC, 1, LDO>(acc, in.M, sDO + vb + 16 * vt);
      add_tile(acc, sPart + (4 + vt) * C * LDC, LDC);
      add_tile(acc, sPart + (6 + vt) * C * LDC, LDC);
      store_tile(sDU + 16 * vt, LDY, acc);
    }
    __syncthreads();
    if (w < 2) {  // U = T Diag(b) Y
      const int vt = w;
      f32x4 acc = zero4();
      mma<1, LDC, 1, 1, LDY>(acc, in.TB, sY + 16 * vt);
      store_tile(sU + 16 * vt, LDY, acc);
    } else if (w < 4) {  // lambda = T^T dU, dV = dY = b lambda
      const int vt = w - 2;
      f32x4 acc = zero4();
      mma<1, 1, LDC, 1, LDY>(acc, in.T, sDU + 16 * vt);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r, col = 16 * vt + (l & 15);
        const float dy = in.b[i] * acc[r];
        sL[i * LDY + col] = acc[r];
        sDY[i * LDY + col] = dy;
        if (i < Lc) dv_out[((size_t)(t0 + i) * H + h) * DV + vb + col] = dy;
      }
    }
    __syncthreads();
    if (w < NCT) {  // dQg += dO S^T, sum dY S^T (= -dKg), dKc += U dS'^T
      const int ct = w;
      mma<BV / 16, LDO, 1, LDB, 1>(aQ, sDO + vb, sS + 16 * ct * LDB);
      mma<BV / 16, LDY, 1, LDB, 1>(aK, sDY, sS + 16 * ct * LDB);
      mma<BV / 16, LDY, 1, LDB, 1>(aC, sU, sD + 16 * ct * LDB);
    }
    if (w == XW0) mma<BV / 16, LDO, 1, LDY, 1>(aX, sDO + vb, sU);  // dO U^T
    if (w == XW1) mma<BV / 16, LDY, 1, LDY, 1>(aX, sDY, sU);       // dY U^T
    if (w == XW2) {                                                // db += lambda . (Y - A U)
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        f32x4 au = zero4();
        mma<1, LDC, 1, 1, LDY>(au, in.A, sU + 16 * vt);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * (l >> 4) + r, col = 16 * vt + (l & 15);
          db[r] += (sY[i * LDY + col] - au[r]) * sL[i * LDY + col];
        }
      }
    }
    __syncthreads();
  }

  // dM, dA, db, sum_v S dS'
  {
    const int jj = l & 15;
    if (w == XW0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        sDM[i * LDC + jj] = jj <= i ? aX[r] : 0.f;
      }
    }
    if (w == XW1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        sDA[i * LDC + jj] = jj < i ? -aX[r] : 0.f;
      }
    }
    if (w == XW2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        const float s = row_sum16(db[r]);
        if (jj == 0 && i < Lc) dbeta[(size_t)(t0 + i) * H + h] = s;
      }
    }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {  // the BV/4 threads of one channel are consecutive lanes
      float s = gs[u];
#pragma unroll
      for (int m = 1; m < BV / 4; m <<= 1) s += wave_xor(s, m);
      const int e = threadIdx.x + NT * u, c = e / (BV / 4);
      if ((e & (BV / 4 - 1)) == 0) sGS[c] = s;
    }
  }
  __syncthreads();

  float* sDG = sS;   // [C][LDK]: dg per row (sS and sD are free now)
  float* sKCT = sD;  // [C][LDK]: k dKc e^{g_L - g}
  if (w < NCT) {
    const int ct = w;
    // Gram terms through the decay: P = (dM o E) K, R = (dM o E)^T Q, P' = (dA o E) K,
    // R' = (dA o E)^T K, on the matrix core from the balanced operands, or per element
    float pfa[4], rfa[4], ppfa[4], rpfa[4];
    if (!exact) {
      f32x4 P = zero4(), R = zero4(), Pp = zero4(), Rp = zero4();
      mma<1, LDC, 1, 1, LDK>(P, sDM, in.kr + 16 * ct);
      mma<1, 1, LDC, 1, LDK>(R, sDM, in.ql + 16 * ct);
      mma<1, LDC, 1, 1, LDK>(Pp, sDA, in.kr + 16 * ct);
      mma<1, 1, LDC, 1, LDK>(Rp, sDA, in.kl + 16 * ct);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r, c = 16 * ct + (l & 15), o = i * LDK + c;
        const float gi = in.g[o], m = 0.5f * in.g[(C - 1) * LDK + c];
        const float e1 = expf(gi - m), e2 = expf(m - gi);
        pfa[r] = e1 * P[r];
        rfa[r] = e2 * R[r];
        ppfa[r] = e1 * Pp[r];
        rpfa[r] = e2 * Rp[r];
      }
    } else {
      // dM is lower and dA strictly lower, so the factor of every entry they keep is <= 1 (the
      // exponent is clamped at 0 where they are zero, so no inf meets a zero)
      const int c = 16 * ct + (l & 15);
      float gi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gi[r] = in.g[(4 * (l >> 4) + r) * LDK + c];
        pfa[r] = rfa[r] = ppfa[r] = rpfa[r] = 0.f;
      }
      for (int y = 0; y < C; ++y) {
        const float gy = in.g[y * LDK + c], ky = in.k[y * LDK + c], qy = in.q[y * LDK + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * (l >> 4) + r;
          const float ef = expf(fminf(gi[r] - gy, 0.f)) * ky;  // row i, column y <= i
          const float eb = expf(fminf(gy - gi[r], 0.f));       // row y >= i, column i
          pfa[r] = fmaf(sDM[i * LDC + y], ef, pfa[r]);
          ppfa[r] = fmaf(sDA[i * LDC + y], ef, ppfa[r]);
          rfa[r] = fmaf(sDM[y * LDC + i] * eb, qy, rfa[r]);
          rpfa[r] = fmaf(sDA[y * LDC + i] * eb, ky, rpfa[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * (l >> 4) + r, c = 16 * ct + (l & 15), o = i * LDK + c;
      const float gi = in.g[o], gl = in.g[(C - 1) * LDK + c];
      const float eg = expf(gi), ec = expf(gl - gi);
      const float qv = in.q[o], kv = in.k[o];
      const float pf = pfa[r], rf = rfa[r], ppf = ppfa[r], rpf = rpfa[r];
      const float dqg = aQ[r], dkg = -aK[r], dkc = aC[r];
      const float dqv = dqg * eg + pf;
      const float dkv = dkg * eg + dkc * ec + rf + ppf + rpf;
      const float dgv = qv * dqv + kv * (dkg * eg - dkc * ec - rf + ppf - rpf);
      if (i < Lc) {
        const size_t go = ((size_t)(t0 + i) * H + h) * DK + c;
        dq[go] = dqv;
        dk_out[go] = dkv;
      }
      sDG[o] = dgv;
      sKCT[o] = kv * dkc * ec;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < DK) {  // dlog a: suffix sums of dg, the last-row terms entering every row
    const int c = threadIdx.x;
    float run = in.el[c] * sGS[c];
#pragma unroll
    for (int i = 0; i < C; ++i) run += sKCT[i * LDK + c];
#pragma unroll
    for (int i = C - 1; i >= 0; --i) {
      run += sDG[i * LDK + c];
      if (i < Lc) dla[((size_t)(t0 + i) * H + h) * DK + c] = run;
    }
  }
}

template <int DK, int DV>
constexpr size_t grad_lds_bytes() {
  constexpr int BV = 32, LDO = DV + 4, LDB = BV + 4, LDY = BV + 4;
  return sizeof(float) * ((size_t)Intra<DK>::FLOATS + C * LDO + 2 * DK * LDB + 8 * C * LDC + 5 * C * LDY +
                          2 * C * LDC + DK);
}

static hipError_t set_lds(const void* kern, size_t lds, std::atomic<uint64_t>& done) {
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

// value-tile width of the dS pass: 64 when that still gives a workgroup per CU
static int ds_bv(int n_chains, int dv) { return ((int64_t)n_chains * (dv / 64) >= 256) ? 64 : 32; }

template <int DK, int BV, typename InT>
static hipError_t launch_ds(const BwdArgs& a, float* dsw) {
  constexpr size_t lds = ds_lds_bytes<DK, BV>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = bwd_ds_kernel<DK, BV, InT>;
  static std::atomic<uint64_t> done{0};
  hipError_t e = set_lds((const void*)kern, lds, done);
  if (e != hipSuccess) return e;
  const int64_t grid = (int64_t)a.n_seqs * a.n_heads * (a.dv_dim / BV);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, (hipStream_t)a.stream, (const InT*)a.q,
                     (const InT*)a.k, a.log_alpha, a.beta, a.cu_seqlens, a.dout, a.dhT, dsw, a.dh0, a.n_heads,
                     a.dv_dim, a.seq_len);
  return hipGetLastError();
}

template <int DK, int DV, typename InT>
static hipError_t launch_grad(const BwdArgs& a, const float* ckpt, const float* dsw) {
  constexpr size_t lds = grad_lds_bytes<DK, DV>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = bwd_grad_kernel<DK, DV, InT>;
  static std::atomic<uint64_t> done{0};
  hipError_t e = set_lds((const void*)kern, lds, done);
  if (e != hipSuccess) return e;
  const int64_t slots = a.total_tokens / C + a.n_seqs + 1;
  const int64_t grid = slots * a.n_heads;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, (hipStream_t)a.stream, (const InT*)a.q,
                     (const InT*)a.k, (const InT*)a.v, a.log_alpha, a.beta, a.h0, a.cu_seqlens, a.dout, ckpt, dsw,
                     a.dq, a.dk, a.dv, a.dlog_alpha, a.dbeta, a.n_heads, a.seq_len, a.n_seqs);
  return hipGetLastError();
}

template <int DK, int DV, typename InT>
static hipError_t run(const BwdArgs& a) {
  const size_t sd = (size_t)DK * DV;
  const int64_t nck = a.total_tokens / C;
  float* ckpt = (float*)a.ws;
  float* dsw = ckpt + (size_t)nck * a.n_heads * sd;
  // (1) forward states entering every chunk; o goes to dv, which the gradient pass overwrites
  ChunkArgs f{};
  f.q = a.q; f.k = a.k; f.v = a.v; f.log_alpha = a.log_alpha; f.beta = a.beta; f.h0 = a.h0;
  f.cu_seqlens = a.cu_seqlens; f.o = a.dv; f.hT = nullptr; f.ckpt = nck > 0 ? ckpt : nullptr;
  f.ckpt_every = C; f.n_seqs = a.n_seqs; f.n_heads = a.n_heads; f.dk = DK; f.dv = DV; f.chunk_size = C;
  f.total_tokens = a.total_tokens; f.seq_len = a.seq_len; f.bf16 = a.bf16; f.stream = a.stream;
  hipError_t e = launch_chunk_fwd_f32(f);
  if (e != hipSuccess) return e;
  // (2) dS' of every chunk, dh0
  if (ds_bv(a.n_seqs * a.n_heads, DV) == 64) e = launch_ds<DK, 64, InT>(a, dsw);
  else e = launch_ds<DK, 32, InT>(a, dsw);
  if (e != hipSuccess) return e;
  // (3) the gradients of every chunk
  return launch_grad<DK, DV, InT>(a, ckpt, dsw);
}

template <typename InT>
static hipError_t dispatch(const BwdArgs& a) {
  if (a.dk_dim == 128 && a.dv_dim == 128) return run<128, 128, InT>(a);
  if (a.dk_dim == 64 && a.dv_dim == 64) return run<64, 64, InT>(a);
  if (a.dk_dim == 128 && a.dv_dim == 64) return run<128, 64, InT>(a);
  if (a.dk_dim == 64 && a.dv_dim == 128) return run<64, 128, InT>(a);
  return hipErrorInvalidValue;
}

}  // namespace bwdc

size_t bwd_chunk_workspace_bytes(int64_t total_tokens, int n_seqs, int n_heads, int dk, int dv) {
  const size_t sd = (size_t)dk * dv * sizeof(float);
  const size_t nck = (size_t)(total_tokens / bwdc::C);
  return (2 * nck + (size_t)n_seqs + 1) * (size_t)n_heads * sd;
}

hipError_t launch_bwd_chunk(const BwdArgs& a) {
  if (a.n_seqs == 0) return hipSuccess;
  return a.bf16 ? bwdc::dispatch<bf16_t>(a) : bwdc::dispatch<float>(a);
}

}  // namespace kda
