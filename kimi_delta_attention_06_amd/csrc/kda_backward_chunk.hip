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
// Four launches: (1) `bwd_prep_kernel`, one (chunk, head) per workgroup, all in parallel,
// forms the chunk's state-free operands (g, Qg, Kg, Kc, A, M, T, T Diag(b), e_L) once and
// writes them to the workspace; (2) `bwd_states_kernel` walks each (sequence, head, value
// tile) forwards over its chunks with S in registers and stores the state entering every
// chunk; (3) `bwd_ds_kernel` walks them backwards with dS in registers and stores the dS'
// of every chunk; (4) `bwd_grad_kernel`, one (chunk, head) per workgroup, forms every
// gradient of the chunk from its S, dS' and operands.  The two serial passes only run the
// state-dependent products; every per-chunk operand they need is read, one chunk ahead.
#include <atomic>
#include <mutex>
#include <type_traits>

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

// e^x through the hardware base-2 exponential: the rounding of x log2(e) adds a relative
// error of at most |x| 2^-24 (7e-6 for the |x| <= 120 nats these factors take off the exact
// path), against roughly ten instructions for expf.  Used for the per-element decay factors;
// the per-channel chunk decay and the exact path's factors keep expf.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

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

  // q, k, log a and b of rows t0 .. t0 + Lc - 1 (zeros past Lc): every load issued before the
  // first is stored
  template <typename InT>
  __device__ void load(const InT* __restrict__ qp, const InT* __restrict__ kp, const float* __restrict__ lap,
                       const float* __restrict__ bp, int64_t t0, int Lc, int H, int h) {
    constexpr int VE = (int)(16 / sizeof(InT)), NQK = 2 * C * DK / VE, IQK = (NQK + NT - 1) / NT;
    constexpr int NLA = C * DK / 4, ILA = (NLA + NT - 1) / NT;
    const int tid = threadIdx.x;
    uint4 rqk[IQK];
    float4 rla[ILA];
#pragma unroll
    for (int it = 0; it < IQK; ++it) {
      const int e = tid + NT * it, which = e / (NQK / 2), ee = e - which * (NQK / 2);
      const int i = ee / (DK / VE), c = (ee - i * (DK / VE)) * VE;
      rqk[it] = make_uint4(0u, 0u, 0u, 0u);
      if (e < NQK && i < Lc) rqk[it] = *reinterpret_cast<const uint4*>((which ? kp : qp) + ((size_t)(t0 + i) * H + h) * DK + c);
    }
#pragma unroll
    for (int it = 0; it < ILA; ++it) {
      const int e = tid + NT * it, i = e / (DK / 4), c = (e - i * (DK / 4)) * 4;
      rla[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < NLA && i < Lc) rla[it] = *reinterpret_cast<const float4*>(lap + ((size_t)(t0 + i) * H + h) * DK + c);
    }
    const float rb = tid < Lc ? bp[(size_t)(t0 + tid) * H + h] : 0.f;
#pragma unroll
    for (int it = 0; it < IQK; ++it) {
      const int e = tid + NT * it, which = e / (NQK / 2), ee = e - which * (NQK / 2);
      const int i = ee / (DK / VE), c = (ee - i * (DK / VE)) * VE;
      if (e < NQK) widen16((which ? k : q) + i * LDK + c, rqk[it], InT{});
    }
#pragma unroll
    for (int it = 0; it < ILA; ++it) {
      const int e = tid + NT * it, i = e / (DK / 4), c = (e - i * (DK / 4)) * 4;
      if (e < NLA) *reinterpret_cast<float4*>(g + i * LDK + c) = rla[it];
    }
    if (tid < C) b[tid] = rb;
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
      const float eg = exp_hw(gi), ec = exp_hw(gl - gi);
      const float qv = q[o], kv = k[o];
      if (!exact) {
        const float e1 = exp_hw(gi - m), e2 = exp_hw(m - gi);
        ql[o] = qv * e1;
        kl[o] = kv * e1;
        kr[o] = kv * e2;
      }
      qg[o] = qv * eg;
      kg[o] = kv * eg;
      kc[o] = kv * ec;
    }
  }

  // The midpoint-balanced operands ql, kl, kr alone (the same values as scale), from q, k, g
  __device__ void scale_balanced() {
    for (int e = threadIdx.x; e < C * DK; e += NT) {
      const int i = e / DK, c = e - i * DK, o = i * LDK + c;
      const float gi = g[o], m = 0.5f * g[(C - 1) * LDK + c];
      const float e1 = exp_hw(gi - m), e2 = exp_hw(m - gi);
      const float qv = q[o], kv = k[o];
      ql[o] = qv * e1;
      kl[o] = kv * e1;
      kr[o] = kv * e2;
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

// The chunk slot of chunk j of sequence n is start_n / C + n + j: distinct for every chunk of
// every packed sequence, below total_tokens / C + n_seqs + 1.  For a slot: its sequence (the
// last n with start_n / C + n <= slot) and chunk; false for a slot no chunk maps to.
__device__ __forceinline__ bool slot_chunk(const int32_t* cu, int n_seqs, int64_t seq_len, int slot, int& n,
                                           int64_t& start, int64_t& len, int64_t& j) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t st = cu ? (int64_t)cu[mid] : (int64_t)mid * seq_len;
    if (st / C + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  n = lo;
  seq_range(cu, n, seq_len, start, len);
  j = (int64_t)slot - (start / C + n);
  return j >= 0 && C * j < len;
}

// The operands the prep pass forms once per (chunk slot, head), fp32, in floats: Qg, Kg, Kc
// and g (the floored prefix sums of log a) [C][DK]; A, M, T and T Diag(b) [C][C]; b [C];
// e^{g_L} [DK]; the exact-path flag (0 or 1) padded to 16 bytes.  65 DK + 1044 floats.
template <int DK>
struct OpTile {
  static constexpr int QG = 0, KG = QG + C * DK, KC = KG + C * DK, G = KC + C * DK;
  static constexpr int A = G + C * DK, M = A + C * C, T = M + C * C, TB = T + C * C;
  static constexpr int B = TB + C * C, EL = B + C, FLAG = EL + DK;
  static constexpr int FLOATS = FLAG + 4;
  static_assert(FLOATS == 65 * DK + 1044 && FLOATS % 4 == 0, "layout");
};

// States and state cotangents in the workspace are in matrix-core fragment order: the dk x dv
// matrix is cut into 16 x 16 tiles (channel block ct, value block vt), tile vt * (DK / 16) + ct
// at 256 floats each, in which lane l's four floats (channels 16 ct + 4 (l >> 4) + r, r = 0..3,
// value 16 vt + (l & 15)) are consecutive at 4 l.  A wave moves a tile with one 16-byte access
// per lane, and the tiles of a run of value blocks are contiguous.
__device__ __forceinline__ size_t frag_off(int ct, int vt, int nct) {
  return ((size_t)vt * nct + ct) * 256 + 4 * lane();
}

// An LDS tile written by some lanes of a wave and read by others of the same wave: the wave's
// LDS accesses complete in order, so only the compiler must keep them in place.
__device__ __forceinline__ void wave_lds_order() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------------------------
// Prep pass: one workgroup per (chunk slot, head), all in parallel.  Qg, Kg, Kc and g go from
// registers to the workspace as they are formed; only what the Gram products and the inverse
// read stays in LDS, with the balanced operands ql, kl formed over q, k (about 39 KB at
// dk = 128: four workgroups per CU, so one workgroup's single-wave inverse overlaps the
// others' work).
template <int DK>
struct PrepLay {
  static constexpr int LDK = DK + 4;
  static constexpr int FLOATS = 4 * C * LDK + 4 * C * LDC + C + DK;  // q|ql, k|kl, g, kr; A, M, T, TB; b; e_L
};

template <int DK, typename InT>
__global__ __launch_bounds__(NT) void bwd_prep_kernel(const InT* __restrict__ q, const InT* __restrict__ k,
                                                      const float* __restrict__ la, const float* __restrict__ beta,
                                                      const int32_t* __restrict__ cu, float* __restrict__ ops, int H,
                                                      int64_t seq_len, int n_seqs) {
  using In = Intra<DK>;
  using O = OpTile<DK>;
  constexpr int LDK = In::LDK, R4 = DK / 4;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  In in(smem);
  // (Intra's layout re-pointed: the balanced left operands over q and k, the decayed forms
  // not held; A, M, T, TB, b, e_L as in Intra, after four [C][LDK] matrices)
  in.kr = in.g + C * LDK;
  in.ql = in.q;
  in.kl = in.k;
  in.qg = in.kg = in.kc = nullptr;
  in.A = in.kr + C * LDK;
  in.M = in.A + C * LDC;
  in.T = in.M + C * LDC;
  in.TB = in.T + C * LDC;
  in.b = in.TB + C * LDC;
  in.el = in.b + C;
  const int slot = blockIdx.x / H, h = blockIdx.x - slot * H;
  int n;
  int64_t start, len, j;
  if (!slot_chunk(cu, n_seqs, seq_len, slot, n, start, len, j)) return;  // (whole workgroup)
  const int64_t t0 = start + C * j;
  const int Lc = (int)(len - C * j < C ? len - C * j : C);
  const int w = threadIdx.x / kWave;
  float* dst = ops + ((size_t)slot * H + h) * O::FLOATS;

  in.load(q, k, la, beta, t0, Lc, H, h);
  __syncthreads();
  const bool exact = __syncthreads_or(in.prefix());
  // decayed operands to the workspace, balanced ones (not on the exact path) in place
  for (int e = threadIdx.x; e < C * R4; e += NT) {
    const int i = e / R4, c = (e - i * R4) * 4, o = i * LDK + c;
    const float4 gi = *reinterpret_cast<const float4*>(in.g + o);
    const float4 gl = *reinterpret_cast<const float4*>(in.g + (C - 1) * LDK + c);
    const float4 qv = *reinterpret_cast<const float4*>(in.q + o), kv = *reinterpret_cast<const float4*>(in.k + o);
    const float g4[4] = {gi.x, gi.y, gi.z, gi.w}, l4[4] = {gl.x, gl.y, gl.z, gl.w};
    const float q4[4] = {qv.x, qv.y, qv.z, qv.w}, k4[4] = {kv.x, kv.y, kv.z, kv.w};
    float qg[4], kg[4], kc[4], ql[4], kl[4], kr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float eg = exp_hw(g4[u]), ec = exp_hw(l4[u] - g4[u]), m = 0.5f * l4[u];
      qg[u] = q4[u] * eg;
      kg[u] = k4[u] * eg;
      kc[u] = k4[u] * ec;
      if (!exact) {
        const float e1 = exp_hw(g4[u] - m), e2 = exp_hw(m - g4[u]);
        ql[u] = q4[u] * e1;
        kl[u] = k4[u] * e1;
        kr[u] = k4[u] * e2;
      }
    }
    const int go = i * DK + c;
    *reinterpret_cast<float4*>(dst + O::QG + go) = make_float4(qg[0], qg[1], qg[2], qg[3]);
    *reinterpret_cast<float4*>(dst + O::KG + go) = make_float4(kg[0], kg[1], kg[2], kg[3]);
    *reinterpret_cast<float4*>(dst + O::KC + go) = make_float4(kc[0], kc[1], kc[2], kc[3]);
    *reinterpret_cast<float4*>(dst + O::G + go) = gi;
    if (!exact) {
      *reinterpret_cast<float4*>(in.ql + o) = make_float4(ql[0], ql[1], ql[2], ql[3]);
      *reinterpret_cast<float4*>(in.kl + o) = make_float4(kl[0], kl[1], kl[2], kl[3]);
      *reinterpret_cast<float4*>(in.kr + o) = make_float4(kr[0], kr[1], kr[2], kr[3]);
    }
  }
  __syncthreads();
  if (exact) {
    if (w < 4) in.gram_exact();
  } else if (w < 2) {
    in.gram(w);
  }
  __syncthreads();
  if (w == 0) in.inverse();
  __syncthreads();
  const int e = threadIdx.x;
  if (e < 4 * C * C / 4) {  // A, M, T, T Diag(b)
    const int m = e / (C * C / 4), i = (e / 4) % C, c = (e % 4) * 4;
    *reinterpret_cast<float4*>(dst + O::A + m * C * C + i * C + c) =
        *reinterpret_cast<const float4*>(in.A + m * C * LDC + i * LDC + c);
  } else if (e < 4 * C * C / 4 + C / 4 + R4) {  // b, e^{g_L} (consecutive in both)
    const int f = e - 4 * C * C / 4;
    *reinterpret_cast<float4*>(dst + O::B + 4 * f) = *reinterpret_cast<const float4*>(in.b + 4 * f);
  } else if (e == 4 * C * C / 4 + C / 4 + R4) {
    *reinterpret_cast<float4*>(dst + O::FLAG) = make_float4(exact ? 1.f : 0.f, 0.f, 0.f, 0.f);
  }
}

// ---------------------------------------------------------------------------------------------
// Serial passes: one workgroup per (sequence, head, BV value columns).  The DK x BV state (or
// its cotangent) lives in MFMA accumulators: wave w owns tiles tt = w + 8 u, channel block
// tt % (DK/16), value block tt / (DK/16).  A chunk's operands are read from its prep tile into
// registers while the chunk before is processed, and put in LDS at the top of the chunk.
// Block -> (chain, value tile) of a serial pass.  Workgroups go to the 8 XCDs round-robin by
// index, so the tiles of one chain take indices of one residue mod 8: they run on one XCD and
// read each chunk's operand tile through one L2 (the grid is padded to a multiple of 8 chains).
__device__ __forceinline__ bool serial_block(int n_chains, int ntile, int& chain, int& tile) {
  const int xcd = blockIdx.x & 7, qd = blockIdx.x >> 3;
  tile = qd % ntile;
  chain = (qd / ntile) * 8 + xcd;
  return chain < n_chains;
}

template <int DK, int BV>
struct SerialShape {
  static constexpr int LDK = DK + 4, LDO = BV + 4;
  static constexpr int NVT = BV / 16, NCT = DK / 16, NTL = NCT * NVT, TPW = NTL / 8;
  static constexpr int KSPLIT = 8 / NVT, KR = DK / KSPLIT;  // the k-split of the DK-long products
  static constexpr int R4 = DK / 4;
  static_assert(NTL % 8 == 0 && 8 % NVT == 0 && KR % 16 == 0, "tiling");
};

// Forward states pass: S <- Diag(e_L) S + Kc^T U with U = T Diag(b) (V - Kg S), chunks in
// order; stores the state entering chunk j (h0 or zeros for j = 0) at slot start/C + n + j.
template <int DK, int BV, typename InT>
__global__ __launch_bounds__(NT) void bwd_states_kernel(const InT* __restrict__ v, const float* __restrict__ h0,
                                                        const int32_t* __restrict__ cu, const float* __restrict__ ops,
                                                        float* __restrict__ sw, int n_chains, int H, int DV,
                                                        int64_t seq_len) {
  using O = OpTile<DK>;
  using Sh = SerialShape<DK, BV>;
  constexpr int LDK = Sh::LDK, LDO = Sh::LDO, NVT = Sh::NVT, NCT = Sh::NCT, TPW = Sh::TPW;
  constexpr int KSPLIT = Sh::KSPLIT, KR = Sh::KR, R4 = Sh::R4;
  constexpr int NKK = 2 * C * R4, IKK = (NKK + NT - 1) / NT;  // float4 of Kg and Kc (consecutive)
  constexpr int NSM = C * C / 4 + R4;                          // T Diag(b), then e^{g_L}
  constexpr int VE = (int)(16 / sizeof(InT)), NVI = C * BV / VE; // 16-byte items of the value tile
  static_assert(NSM <= NT && NVI <= NT, "one small item per thread");

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* sKG = smem;                   // [C][LDK]
  float* sKC = sKG + C * LDK;          // [C][LDK]
  float* sTB = sKC + C * LDK;          // [C][LDC]
  float* sEL = sTB + C * LDC;          // [DK]
  float* sV = sEL + DK;                // [C][LDO]
  float* sST = sV + C * LDO;           // [BV][LDK]: S transposed
  float* sPart = sST + BV * LDK;       // [8][C][LDC]
  float* sY = sV;                      // Y = V - Kg S over V (each element read, then written, by one lane)
  float* sU = sPart + 8 * C * LDC;     // [C][LDO]

  int chain, tile;
  if (!serial_block(n_chains, DV / BV, chain, tile)) return;
  const int n = chain / H, h = chain - n * H, v0 = tile * BV;
  int64_t start, len;
  seq_range(cu, n, seq_len, start, len);
  const int64_t nch = (len + C - 1) / C;
  const int64_t slot0 = start / C + n;
  const int tid = threadIdx.x, w = tid / kWave, l = lane();

  f32x4 S[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tt = w + 8 * u, ct = tt % NCT, vt = tt / NCT;
    const int crow = 16 * ct + 4 * (l >> 4), vcol = 16 * vt + (l & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) S[u][r] = h0 ? h0[((size_t)chain * DK + crow + r) * DV + v0 + vcol] : 0.f;
    *reinterpret_cast<float4*>(sST + vcol * LDK + crow) = make_float4(S[u][0], S[u][1], S[u][2], S[u][3]);
  }

  float4 rkk[IKK], rsm = make_float4(0.f, 0.f, 0.f, 0.f);
  uint4 rv = make_uint4(0u, 0u, 0u, 0u);
  auto fetch = [&](int64_t jj) {
    const float* op = ops + ((size_t)(slot0 + jj) * H + h) * O::FLOATS;
    const int64_t t0 = start + C * jj;
    const int Lc = (int)(len - C * jj < C ? len - C * jj : C);
#pragma unroll
    for (int it = 0; it < IKK; ++it) {
      const int e = tid + NT * it;
      rkk[it] = e < NKK ? *reinterpret_cast<const float4*>(op + O::KG + 4 * e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < C * C / 4) rsm = *reinterpret_cast<const float4*>(op + O::TB + 4 * tid);
    else if (tid < NSM) rsm = *reinterpret_cast<const float4*>(op + O::EL + 4 * (tid - C * C / 4));
    rv = make_uint4(0u, 0u, 0u, 0u);
    if (tid < NVI) {
      const int i = tid / (BV / VE), c = (tid - i * (BV / VE)) * VE;
      if (i < Lc) rv = *reinterpret_cast<const uint4*>(v + ((size_t)(t0 + i) * H + h) * DV + v0 + c);
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int it = 0; it < IKK; ++it) {
      const int e = tid + NT * it;
      if (e < NKK) {
        const int m = e / (C * R4), ee = e - m * (C * R4), i = ee / R4, c = (ee - i * R4) * 4;
        *reinterpret_cast<float4*>((m ? sKC : sKG) + i * LDK + c) = rkk[it];
      }
    }
    if (tid < C * C / 4) *reinterpret_cast<float4*>(sTB + (tid / 4) * LDC + (tid % 4) * 4) = rsm;
    else if (tid < NSM) *reinterpret_cast<float4*>(sEL + 4 * (tid - C * C / 4)) = rsm;
    if (tid < NVI) {
      const int i = tid / (BV / VE), c = (tid - i * (BV / VE)) * VE;
      widen16(sV + i * LDO + c, rv, InT{});
    }
  };
  if (nch > 0) fetch(0);

  for (int64_t j = 0; j < nch; ++j) {
    put();
    if (j + 1 < nch) fetch(j + 1);
    {  // the state entering chunk j
      float* dst = sw + ((size_t)(slot0 + j) * H + h) * DK * DV;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tt = w + 8 * u, ct = tt % NCT, vt = tt / NCT;
        *reinterpret_cast<float4*>(dst + frag_off(ct, v0 / 16 + vt, NCT)) = make_float4(S[u][0], S[u][1], S[u][2], S[u][3]);
      }
    }
    __syncthreads();
    {  // partial Kg S over one k-range: job w = (value block w % NVT, k-range w / NVT)
      const int vt = w % NVT, kq = w / NVT;
      f32x4 acc = zero4();
      mma<KR / 16, LDK, 1, LDK, 1>(acc, sKG + kq * KR, sST + 16 * vt * LDK + kq * KR);
      store_tile(sPart + w * C * LDC, LDC, acc);
    }
    __syncthreads();
    if (w >= 8 - NVT) {  // Y = V - Kg S, then U = T Diag(b) Y, one value block per wave
      const int vt = w - (8 - NVT);
      f32x4 acc = zero4();
#pragma unroll
      for (int kq = 0; kq < KSPLIT; ++kq) add_tile(acc, sPart + (vt + kq * NVT) * C * LDC, LDC);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r, col = 16 * vt + (l & 15);
        sY[i * LDO + col] = sV[i * LDO + col] - acc[r];
      }
      wave_lds_order();
      f32x4 u = zero4();
      mma<1, LDC, 1, 1, LDO>(u, sTB, sY + 16 * vt);
      store_tile(sU + 16 * vt, LDO, u);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TPW; ++u) {  // S <- Diag(e_L) S + Kc^T U
      const int tt = w + 8 * u, ct = tt % NCT, vt = tt / NCT;
      const int crow = 16 * ct + 4 * (l >> 4), vcol = 16 * vt + (l & 15);
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sEL[crow + r] * S[u][r];
      mma<1, 1, LDK, 1, LDO>(acc, sKC + 16 * ct, sU + 16 * vt);
      S[u] = acc;
      *reinterpret_cast<float4*>(sST + vcol * LDK + crow) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();
  }
}

template <int DK, int BV>
constexpr size_t states_lds_bytes() {
  using Sh = SerialShape<DK, BV>;
  return sizeof(float) * ((size_t)2 * C * Sh::LDK + C * LDC + DK + 2 * C * Sh::LDO + (size_t)BV * Sh::LDK +
                          8 * C * LDC);
}

// dS pass: chunks in reverse order; stores dS' of chunk j (the cotangent of the state leaving
// it) at slot start/C + n + j, and dh0.
//   dU = M^T dO + Kc dS',  lambda = T^T dU,  dS = Diag(e_L) dS' + Qg^T dO - Kg^T Diag(b) lambda
template <int DK, int BV>
__global__ __launch_bounds__(NT) void bwd_ds_kernel(const int32_t* __restrict__ cu, const float* __restrict__ dout,
                                                    const float* __restrict__ dhT, const float* __restrict__ ops,
                                                    float* __restrict__ dsw, float* __restrict__ dh0, int n_chains,
                                                    int H, int DV, int64_t seq_len) {
  using O = OpTile<DK>;
  using Sh = SerialShape<DK, BV>;
  constexpr int LDK = Sh::LDK, LDO = Sh::LDO, NVT = Sh::NVT, NCT = Sh::NCT, TPW = Sh::TPW;
  constexpr int KSPLIT = Sh::KSPLIT, KR = Sh::KR, R4 = Sh::R4;
  constexpr int NBIG = 3 * C * R4, IBIG = (NBIG + NT - 1) / NT;  // float4 of Qg, Kg, Kc (consecutive)
  constexpr int NMT = 2 * C * C / 4, NSM = NMT + C / 4 + R4;      // M, T (consecutive), then b, e^{g_L}
  constexpr int NDO = C * BV / 4;
  static_assert(NSM <= NT && NDO <= NT, "one small item per thread");

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* sQG = smem;                   // [C][LDK]
  float* sKG = sQG + C * LDK;
  float* sKC = sKG + C * LDK;
  float* sM = sKC + C * LDK;           // [C][LDC]
  float* sT = sM + C * LDC;            // [C][LDC]
  float* sB = sT + C * LDC;            // [C]
  float* sEL = sB + C;                 // [DK]
  float* sDO = sEL + DK;               // [C][LDO]
  float* sDST = sDO + C * LDO;         // [BV][LDK]: dS' transposed
  float* sPart = sDST + BV * LDK;      // [8][C][LDC]
  float* sDU = sPart + 8 * C * LDC;    // [C][LDO]
  float* sNDY = sDU + C * LDO;         // [C][LDO]: -dY

  int chain, tile;
  if (!serial_block(n_chains, DV / BV, chain, tile)) return;
  const int n = chain / H, h = chain - n * H, v0 = tile * BV;
  int64_t start, len;
  seq_range(cu, n, seq_len, start, len);
  const int64_t nch = (len + C - 1) / C;
  const int64_t slot0 = start / C + n;
  const int tid = threadIdx.x, w = tid / kWave, l = lane();

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

  float4 rbig[IBIG], rsm = make_float4(0.f, 0.f, 0.f, 0.f), rdo = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fetch = [&](int64_t jj) {
    const float* op = ops + ((size_t)(slot0 + jj) * H + h) * O::FLOATS;
    const int64_t t0 = start + C * jj;
    const int Lc = (int)(len - C * jj < C ? len - C * jj : C);
#pragma unroll
    for (int it = 0; it < IBIG; ++it) {
      const int e = tid + NT * it;
      rbig[it] = e < NBIG ? *reinterpret_cast<const float4*>(op + O::QG + 4 * e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < NMT) rsm = *reinterpret_cast<const float4*>(op + O::M + 4 * tid);
    else if (tid < NSM) rsm = *reinterpret_cast<const float4*>(op + O::B + 4 * (tid - NMT));
    rdo = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < NDO) {
      const int i = tid / (BV / 4), c = (tid - i * (BV / 4)) * 4;
      if (i < Lc) rdo = *reinterpret_cast<const float4*>(dout + ((size_t)(t0 + i) * H + h) * DV + v0 + c);
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int it = 0; it < IBIG; ++it) {
      const int e = tid + NT * it;
      if (e < NBIG) {
        const int m = e / (C * R4), ee = e - m * (C * R4), i = ee / R4, c = (ee - i * R4) * 4;
        *reinterpret_cast<float4*>(sQG + m * C * LDK + i * LDK + c) = rbig[it];
      }
    }
    if (tid < NMT) *reinterpret_cast<float4*>(sM + (tid / (C * C / 4)) * C * LDC + ((tid / 4) % C) * LDC + (tid % 4) * 4) = rsm;
    else if (tid < NSM) *reinterpret_cast<float4*>(sB + 4 * (tid - NMT)) = rsm;
    if (tid < NDO) {
      const int i = tid / (BV / 4), c = (tid - i * (BV / 4)) * 4;
      *reinterpret_cast<float4*>(sDO + i * LDO + c) = rdo;
    }
  };
  if (nch > 0) fetch(nch - 1);

  for (int64_t j = nch - 1; j >= 0; --j) {
    put();
    if (j > 0) fetch(j - 1);
    {  // dS' of chunk j
      float* dst = dsw + ((size_t)(slot0 + j) * H + h) * DK * DV;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tt = w + 8 * u, ct = tt % NCT, vt = tt / NCT;
        *reinterpret_cast<float4*>(dst + frag_off(ct, v0 / 16 + vt, NCT)) =
            make_float4(ds[u][0], ds[u][1], ds[u][2], ds[u][3]);
      }
    }
    __syncthreads();
    {  // partial Kc dS' over one k-range: job w = (value block w % NVT, k-range w / NVT)
      const int vt = w % NVT, kq = w / NVT;
      f32x4 acc = zero4();
      mma<KR / 16, LDK, 1, LDK, 1>(acc, sKC + kq * KR, sDST + 16 * vt * LDK + kq * KR);
      store_tile(sPart + w * C * LDC, LDC, acc);
    }
    __syncthreads();
    if (w >= 8 - NVT) {  // dU = M^T dO + Kc dS', then lambda = T^T dU and -dY = -b lambda
      const int vt = w - (8 - NVT);
      f32x4 acc = zero4();
      mma<1, 1, LDC, 1, LDO>(acc, sM, sDO + 16 * vt);
#pragma unroll
      for (int kq = 0; kq < KSPLIT; ++kq) add_tile(acc, sPart + (vt + kq * NVT) * C * LDC, LDC);
      store_tile(sDU + 16 * vt, LDO, acc);
      wave_lds_order();
      f32x4 lam = zero4();
      mma<1, 1, LDC, 1, LDO>(lam, sT, sDU + 16 * vt);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        sNDY[i * LDO + 16 * vt + (l & 15)] = -sB[i] * lam[r];
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TPW; ++u) {  // dS = Diag(e_L) dS' + Qg^T dO - Kg^T dY
      const int tt = w + 8 * u, ct = tt % NCT, vt = tt / NCT;
      const int crow = 16 * ct + 4 * (l >> 4), vcol = 16 * vt + (l & 15);
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sEL[crow + r] * ds[u][r];
      mma<1, 1, LDK, 1, LDO>(acc, sQG + 16 * ct, sDO + 16 * vt);
      mma<1, 1, LDK, 1, LDO>(acc, sKG + 16 * ct, sNDY + 16 * vt);
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
  using Sh = SerialShape<DK, BV>;
  return sizeof(float) * ((size_t)3 * C * Sh::LDK + 2 * C * LDC + C + DK + 3 * C * Sh::LDO + (size_t)BV * Sh::LDK +
                          8 * C * LDC);
}

// ---------------------------------------------------------------------------------------------
// Gradient pass: one workgroup of 4 waves per (chunk slot, head), two per CU (about 76 KB of
// LDS each), so one workgroup's memory phases overlap the other's matrix-core work.  Value
// columns in tiles of BV = 16: per tile, the columns of S, dS', V and dO are staged in LDS and
// the dv-reductions (dQg, dKg, dKc, dM, dA, db and sum_v S dS') accumulate in registers; then
// the chain rule through the decay factors.  What only the tile loop reads (Kg, Kc, the staged
// columns and products) and what only the chain-rule step reads (q, k, g, the balanced
// operands, dg) share LDS.
constexpr int NTG = 256;  // threads per gradient workgroup

template <int DK, int DV>
struct GradLay {
  static constexpr int BV = 16, LDK = DK + 4, LDB = BV + 4, LDY = BV + 4;
  // persistent: A, M, T, T Diag(b) [C][LDC]; b [C], e^{g_L} [DK]; dM, dA [C][LDC]; sum_v S dS' [DK]
  static constexpr int A = 0, M = A + C * LDC, T = M + C * LDC, TB = T + C * LDC;
  static constexpr int B = TB + C * LDC, EL = B + C, DM = EL + DK, DA = DM + C * LDC, GS = DA + C * LDC;
  // R1: Kg, Kc [C][LDK] in the tile loop; then the dQg tiles (float4 [NCT][64]), then dg and
  // k dKc e^{g_L - g} [C][LDK]
  static constexpr int R1 = GS + DK, KG = R1, KC = KG + C * LDK, QX = R1, DG = R1, KCT = DG + C * LDK;
  // R2, tile loop: S, dS' [DK][LDB]; partial Kg S and Kc dS' [2][4][C][LDC]; Y, dU, U, lambda,
  // dY, V, dO [C][LDY]
  static constexpr int R2 = KCT + C * LDK, SS = R2, SD = SS + DK * LDB, PART = SD + DK * LDB;
  static constexpr int SY = PART + 8 * C * LDC, SDU = SY + C * LDY, SU = SDU + C * LDY, SL = SU + C * LDY;
  static constexpr int SDY = SL + C * LDY, SV = SDY + C * LDY, SDO = SV + C * LDY, LOOP_END = SDO + C * LDY;
  //     chain-rule step: q, k, g, ql, kl, kr [C][LDK]
  static constexpr int Q = R2, K = Q + C * LDK, G = K + C * LDK, QL = G + C * LDK, KL = QL + C * LDK;
  static constexpr int KR = KL + C * LDK, TAIL_END = KR + C * LDK;
  static constexpr int FLOATS = LOOP_END > TAIL_END ? LOOP_END : TAIL_END;
  static_assert(A % 4 == 0 && B % 4 == 0 && EL % 4 == 0 && DM % 4 == 0 && GS % 4 == 0 && R1 % 4 == 0 &&
                    KC % 4 == 0 && R2 % 4 == 0 && SD % 4 == 0 && PART % 4 == 0 && SY % 4 == 0 && SDO % 4 == 0 &&
                    K % 4 == 0 && G % 4 == 0 && QL % 4 == 0 && KR % 4 == 0,
                "16-byte aligned regions");
  static_assert(2 * C * LDK >= 4 * (DK / 16) * 64, "the dQg tiles fit in R1");
};

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(NTG) void bwd_grad_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v, const int32_t* __restrict__ cu,
    const float* __restrict__ dout, const float* __restrict__ ops, const float* __restrict__ sw,
    const float* __restrict__ dsw, float* __restrict__ dq, float* __restrict__ dk_out, float* __restrict__ dv_out,
    float* __restrict__ dla, float* __restrict__ dbeta, int H, int64_t seq_len, int n_seqs) {
  using O = OpTile<DK>;
  using L = GradLay<DK, DV>;
  constexpr int BV = L::BV, LDK = L::LDK, LDB = L::LDB, LDY = L::LDY, R4 = DK / 4;
  constexpr int NCT = DK / 16, NTV = DV / BV, UPT = DK * BV / 4 / NTG, KQ = DK / 4;
  constexpr int VE = (int)(16 / sizeof(InT)), NVI = C * BV / VE, NDI = C * BV / 4;
  constexpr int NQH = (NCT + 1) / 2;  // dQg channel blocks per accumulating wave (waves 2, 3)
  static_assert(NCT <= 8 && UPT >= 1 && DK * BV / 4 % NTG == 0 && NVI <= NTG && NDI <= NTG && KQ % 16 == 0,
                "tiling");

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float *sA = smem + L::A, *sM = smem + L::M, *sT = smem + L::T, *sTB = smem + L::TB, *sB = smem + L::B;
  float *sEL = smem + L::EL, *sDM = smem + L::DM, *sDA = smem + L::DA, *sGS = smem + L::GS;
  float *sKG = smem + L::KG, *sKC = smem + L::KC, *sDG = smem + L::DG, *sKCT = smem + L::KCT;
  float4* sQX = reinterpret_cast<float4*>(smem + L::QX);
  float *sS = smem + L::SS, *sD = smem + L::SD, *sPart = smem + L::PART, *sY = smem + L::SY, *sDU = smem + L::SDU;
  float *sU = smem + L::SU, *sL = smem + L::SL, *sDY = smem + L::SDY, *sV = smem + L::SV, *sDO = smem + L::SDO;
  float *sQ = smem + L::Q, *sK = smem + L::K, *sG = smem + L::G, *sQL = smem + L::QL, *sKL = smem + L::KL;
  float* sKR = smem + L::KR;

  const int slot = blockIdx.x / H, h = blockIdx.x - slot * H;
  int n;
  int64_t start, len, j;
  if (!slot_chunk(cu, n_seqs, seq_len, slot, n, start, len, j)) return;  // (whole workgroup)
  const int64_t t0 = start + C * j;
  const int Lc = (int)(len - C * j < C ? len - C * j : C);
  const float* S0 = sw + ((size_t)slot * H + h) * DK * DV;
  const float* dSC = dsw + ((size_t)slot * H + h) * DK * DV;
  const float* op = ops + ((size_t)slot * H + h) * O::FLOATS;
  const int tid = threadIdx.x, w = tid / kWave, l = lane();

  // The columns of value tile tv, in registers (two sets, by the tile's parity): the tile two
  // ahead is in flight while the current one is worked on.  S and dS' (fragment order): item
  // e = tid + NTG u is lane l of channel block e / 64 of value block tv.  V and dO: row
  // tid / (BV / VE) (resp. / (BV / 4)).
  static_assert(NTV % 2 == 0, "value tiles in pairs");
  float4 pS[2][UPT], pD[2][UPT], pdo[2];
  uint4 pv[2];
  auto fetch = [&](int tv, auto pc) {
    constexpr int P = decltype(pc)::value;
    const size_t base = (size_t)tv * NCT * 256;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const size_t o4 = base + 4 * (size_t)(tid + NTG * u);
      pS[P][u] = *reinterpret_cast<const float4*>(S0 + o4);
      pD[P][u] = *reinterpret_cast<const float4*>(dSC + o4);
    }
    pv[P] = make_uint4(0u, 0u, 0u, 0u);
    if (tid < NVI) {
      const int i = tid / (BV / VE), c = (tid - i * (BV / VE)) * VE;
      if (i < Lc) pv[P] = *reinterpret_cast<const uint4*>(v + ((size_t)(t0 + i) * H + h) * DV + tv * BV + c);
    }
    pdo[P] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < NDI) {
      const int i = tid / (BV / 4), c = (tid - i * (BV / 4)) * 4;
      if (i < Lc) pdo[P] = *reinterpret_cast<const float4*>(dout + ((size_t)(t0 + i) * H + h) * DV + tv * BV + c);
    }
  };
  fetch(0, std::integral_constant<int, 0>{});
  fetch(1, std::integral_constant<int, 1>{});
  // the tile loop's operands from the prep tile (Kg, Kc; A, M, T, T Diag(b); b, e^{g_L}):
  // every load issued before the first is stored
  constexpr int NOP = 2 * C * R4, IOP = (NOP + NTG - 1) / NTG;
  constexpr int NSM = 4 * C * C / 4 + C / 4 + R4, ISM = (NSM + NTG - 1) / NTG;
  float4 rop[IOP], rsm[ISM];
#pragma unroll
  for (int it = 0; it < IOP; ++it) {
    const int e = tid + NTG * it;
    rop[it] = e < NOP ? *reinterpret_cast<const float4*>(op + O::KG + 4 * e) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int it = 0; it < ISM; ++it) {
    const int e = tid + NTG * it;
    rsm[it] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e < 4 * C * C / 4) rsm[it] = *reinterpret_cast<const float4*>(op + O::A + 4 * e);
    else if (e < NSM) rsm[it] = *reinterpret_cast<const float4*>(op + O::B + 4 * (e - 4 * C * C / 4));
  }
  const bool exact = op[O::FLAG] != 0.f;
#pragma unroll
  for (int it = 0; it < IOP; ++it) {
    const int e = tid + NTG * it;
    if (e < NOP) {
      const int m = e / (C * R4), ee = e - m * (C * R4), i = ee / R4, c = (ee - i * R4) * 4;
      *reinterpret_cast<float4*>((m ? sKC : sKG) + i * LDK + c) = rop[it];
    }
  }
#pragma unroll
  for (int it = 0; it < ISM; ++it) {
    const int e = tid + NTG * it;
    if (e < 4 * C * C / 4) {  // A, M, T, T Diag(b): consecutive [C][LDC] regions
      const int m = e / (C * C / 4), i = (e / 4) % C, c = (e % 4) * 4;
      *reinterpret_cast<float4*>(sA + m * C * LDC + i * LDC + c) = rsm[it];
    } else if (e < NSM) {  // b, e^{g_L}: consecutive
      *reinterpret_cast<float4*>(sB + 4 * (e - 4 * C * C / 4)) = rsm[it];
    }
  }

  f32x4 aQ[NQH], aK[2], aC[2], aX = zero4(), db = zero4();
#pragma unroll
  for (int u = 0; u < NQH; ++u) aQ[u] = zero4();
  aK[0] = aK[1] = aC[0] = aC[1] = zero4();
  float gs[UPT][4];
#pragma unroll
  for (int u = 0; u < UPT; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) gs[u][r] = 0.f;
  // the chain-rule step's inputs (q, k, g), loaded two value tiles before the last
  constexpr int NQK = 2 * C * DK / VE, IQK = (NQK + NTG - 1) / NTG, IG = (C * R4 + NTG - 1) / NTG;
  uint4 rqk[IQK];
  float4 rg[IG];

  auto tile = [&](int tv, auto pc) {
    constexpr int P = decltype(pc)::value;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {  // stage S and dS' columns of value block tv
      const int c = 16 * ((tid + NTG * u) / 64) + 4 * (l >> 4), col = l & 15;
      const float sv[4] = {pS[P][u].x, pS[P][u].y, pS[P][u].z, pS[P][u].w};
      const float dv[4] = {pD[P][u].x, pD[P][u].y, pD[P][u].z, pD[P][u].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sS[(c + r) * LDB + col] = sv[r];
        sD[(c + r) * LDB + col] = dv[r];
        gs[u][r] += sv[r] * dv[r];
      }
    }
    if (tid < NVI) {
      const int i = tid / (BV / VE), c = (tid - i * (BV / VE)) * VE;
      widen16(sV + i * LDY + c, pv[P], InT{});
    }
    if (tid < NDI) {
      const int i = tid / (BV / 4), c = (tid - i * (BV / 4)) * 4;
      *reinterpret_cast<float4*>(sDO + i * LDY + c) = pdo[P];
    }
    if (tv + 2 < NTV) {
      fetch(tv + 2, pc);
    } else if (tv + 2 == NTV) {
#pragma unroll
      for (int it = 0; it < IQK; ++it) {
        const int e = tid + NTG * it, which = e / (NQK / 2), ee = e - which * (NQK / 2);
        const int i = ee / (DK / VE), c = (ee - i * (DK / VE)) * VE;
        rqk[it] = make_uint4(0u, 0u, 0u, 0u);
        if (e < NQK && i < Lc)
          rqk[it] = *reinterpret_cast<const uint4*>((which ? k : q) + ((size_t)(t0 + i) * H + h) * DK + c);
      }
#pragma unroll
      for (int it = 0; it < IG; ++it) {
        const int e = tid + NTG * it;
        rg[it] = e < C * R4 ? *reinterpret_cast<const float4*>(op + O::G + 4 * e) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    __syncthreads();
    {  // partial Kg S and Kc dS' over channel quarter w
      f32x4 pk = zero4(), pc = zero4();
      mma<KQ / 16, LDK, 1, 1, LDB>(pk, sKG + w * KQ, sS + w * KQ * LDB);
      mma<KQ / 16, LDK, 1, 1, LDB>(pc, sKC + w * KQ, sD + w * KQ * LDB);
      store_tile(sPart + w * C * LDC, LDC, pk);
      store_tile(sPart + (4 + w) * C * LDC, LDC, pc);
    }
    __syncthreads();
    if (w == 0) {  // Y = V - Kg S, then U = T Diag(b) Y
      f32x4 acc = zero4();
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) add_tile(acc, sPart + kq * C * LDC, LDC);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        sY[i * LDY + (l & 15)] = sV[i * LDY + (l & 15)] - acc[r];
      }
      wave_lds_order();
      f32x4 u = zero4();
      mma<1, LDC, 1, 1, LDY>(u, sTB, sY);
      store_tile(sU, LDY, u);
    } else if (w == 1) {  // dU = M^T dO + Kc dS', then lambda = T^T dU and dY = Diag(b) lambda
      f32x4 acc = zero4();
      mma<1, 1, LDC, 1, LDY>(acc, sM, sDO);
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) add_tile(acc, sPart + (4 + kq) * C * LDC, LDC);
      store_tile(sDU, LDY, acc);
      wave_lds_order();
      f32x4 lam = zero4();
      mma<1, 1, LDC, 1, LDY>(lam, sT, sDU);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r, col = l & 15;
        const float dy = sB[i] * lam[r];
        sL[i * LDY + col] = lam[r];
        sDY[i * LDY + col] = dy;
        if (i < Lc) dv_out[((size_t)(t0 + i) * H + h) * DV + tv * BV + col] = dy;
      }
    } else {  // dQg += dO S^T over channel blocks (w - 2) NQH ..
#pragma unroll
      for (int u = 0; u < NQH; ++u) {
        const int ct = (w - 2) * NQH + u;
        if (ct < NCT) mma<1, LDY, 1, LDB, 1>(aQ[u], sDO, sS + 16 * ct * LDB);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // sum dY S^T (= -dKg), dKc += U dS'^T over channel blocks w, w + 4
      const int ct = w + 4 * u;
      if (ct < NCT) {
        mma<1, LDY, 1, LDB, 1>(aK[u], sDY, sS + 16 * ct * LDB);
        mma<1, LDY, 1, LDB, 1>(aC[u], sU, sD + 16 * ct * LDB);
      }
    }
    if (w == 0) mma<1, LDY, 1, LDY, 1>(aX, sDO, sU);  // dO U^T
    if (w == 1) mma<1, LDY, 1, LDY, 1>(aX, sDY, sU);  // dY U^T
    if (w == 2) {                                     // db += lambda . (Y - A U)
      f32x4 au = zero4();
      mma<1, LDC, 1, 1, LDY>(au, sA, sU);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        db[r] += (sY[i * LDY + (l & 15)] - au[r]) * sL[i * LDY + (l & 15)];
      }
    }
    __syncthreads();
  };
  for (int tv = 0; tv < NTV; tv += 2) {
    tile(tv, std::integral_constant<int, 0>{});
    tile(tv + 1, std::integral_constant<int, 1>{});
  }

  // dQg tiles (waves 2, 3) to the shared tiles, q, k, g to LDS, dM, dA, db, sum_v S dS'
  if (w >= 2) {
#pragma unroll
    for (int u = 0; u < NQH; ++u) {
      const int ct = (w - 2) * NQH + u;
      if (ct < NCT) sQX[ct * 64 + l] = make_float4(aQ[u][0], aQ[u][1], aQ[u][2], aQ[u][3]);
    }
  }
#pragma unroll
  for (int it = 0; it < IQK; ++it) {
    const int e = tid + NTG * it, which = e / (NQK / 2), ee = e - which * (NQK / 2);
    const int i = ee / (DK / VE), c = (ee - i * (DK / VE)) * VE;
    if (e < NQK) widen16((which ? sK : sQ) + i * LDK + c, rqk[it], InT{});
  }
#pragma unroll
  for (int it = 0; it < IG; ++it) {
    const int e = tid + NTG * it;
    if (e < C * R4) *reinterpret_cast<float4*>(sG + (e / R4) * LDK + (e % R4) * 4) = rg[it];
  }
  {
    const int jj = l & 15;
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        sDM[i * LDC + jj] = jj <= i ? aX[r] : 0.f;
      }
    }
    if (w == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        sDA[i * LDC + jj] = jj < i ? -aX[r] : 0.f;
      }
    }
    if (w == 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r;
        const float s = row_sum16(db[r]);
        if (jj == 0 && i < Lc) dbeta[(size_t)(t0 + i) * H + h] = s;
      }
    }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {  // over the 16 value columns of a lane row
      const int c = 16 * ((tid + NTG * u) / 64) + 4 * (l >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = row_sum16(gs[u][r]);
        if (jj == 0) sGS[c + r] = s;
      }
    }
  }
  __syncthreads();
  // the balanced operands for the Gram terms' chain rule (not on the exact path), and each
  // wave's dQg tiles into registers (their LDS is reused below)
  if (!exact) {
    for (int e = tid; e < C * DK; e += NTG) {
      const int i = e / DK, c = e - i * DK, o = i * LDK + c;
      const float gi = sG[o], m = 0.5f * sG[(C - 1) * LDK + c];
      const float e1 = exp_hw(gi - m), e2 = exp_hw(m - gi);
      const float qv = sQ[o], kv = sK[o];
      sQL[o] = qv * e1;
      sKL[o] = kv * e1;
      sKR[o] = kv * e2;
    }
  }
  float4 dq4[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) dq4[u] = w + 4 * u < NCT ? sQX[(w + 4 * u) * 64 + l] : make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();

#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ct = w + 4 * u;
    if (ct >= NCT) continue;
    const float dqt[4] = {dq4[u].x, dq4[u].y, dq4[u].z, dq4[u].w};
    // Gram terms through the decay: P = (dM o E) K, R = (dM o E)^T Q, P' = (dA o E) K,
    // R' = (dA o E)^T K, on the matrix core from the balanced operands, or per element
    float pfa[4], rfa[4], ppfa[4], rpfa[4];
    if (!exact) {
      f32x4 P = zero4(), R = zero4(), Pp = zero4(), Rp = zero4();
      mma<1, LDC, 1, 1, LDK>(P, sDM, sKR + 16 * ct);
      mma<1, 1, LDC, 1, LDK>(R, sDM, sQL + 16 * ct);
      mma<1, LDC, 1, 1, LDK>(Pp, sDA, sKR + 16 * ct);
      mma<1, 1, LDC, 1, LDK>(Rp, sDA, sKL + 16 * ct);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (l >> 4) + r, c = 16 * ct + (l & 15), o = i * LDK + c;
        const float gi = sG[o], m = 0.5f * sG[(C - 1) * LDK + c];
        const float e1 = exp_hw(gi - m), e2 = exp_hw(m - gi);
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
        gi[r] = sG[(4 * (l >> 4) + r) * LDK + c];
        pfa[r] = rfa[r] = ppfa[r] = rpfa[r] = 0.f;
      }
      for (int y = 0; y < C; ++y) {
        const float gy = sG[y * LDK + c], ky = sK[y * LDK + c], qy = sQ[y * LDK + c];
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
      const float gi = sG[o], gl = sG[(C - 1) * LDK + c];
      const float eg = exp_hw(gi), ec = exp_hw(gl - gi);
      const float qv = sQ[o], kv = sK[o];
      const float pf = pfa[r], rf = rfa[r], ppf = ppfa[r], rpf = rpfa[r];
      const float dqg = dqt[r], dkg = -aK[u][r], dkc = aC[u][r];
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
    float run = sEL[c] * sGS[c];
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
constexpr size_t grad_lds_bytes() { return sizeof(float) * (size_t)GradLay<DK, DV>::FLOATS; }

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

// chunk slots (see slot_chunk) and the workspace: the prep tiles, then the states entering
// every chunk, then the state cotangents leaving every chunk
static int64_t n_slots(int64_t total_tokens, int n_seqs) { return total_tokens / C + n_seqs + 1; }



template <int DK, typename InT>
static hipError_t launch_prep(const BwdArgs& a, float* ops) {
  constexpr size_t lds = sizeof(float) * (size_t)PrepLay<DK>::FLOATS;
  auto kern = bwd_prep_kernel<DK, InT>;
  static std::atomic<uint64_t> done{0};
  hipError_t e = set_lds((const void*)kern, lds, done);
  if (e != hipSuccess) return e;
  const int64_t grid = n_slots(a.total_tokens, a.n_seqs) * a.n_heads;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, (hipStream_t)a.stream, (const InT*)a.q,
                     (const InT*)a.k, a.log_alpha, a.beta, a.cu_seqlens, ops, a.n_heads, a.seq_len, a.n_seqs);
  return hipGetLastError();
}

// A second stream per device on which the reverse pass runs beside the forward-states pass
// (created on first use, default priority, kept until the process ends).  Each call forks
// to it and joins back through events of its own, so concurrent calls stay ordered on their
// own streams and the pair can be captured into a HIP graph like any fork and join.
static hipError_t side_stream(hipStream_t& out) {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev]) {
    e = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking);
    if (e != hipSuccess) return e;
  }
  out = streams[dev];
  return hipSuccess;
}

// The two serial passes.  `concurrent`: the reverse pass on the side stream beside the
// forward-states pass (64-column tiles: 71 + 86 KB of LDS, one workgroup of each per CU).
template <int DK, int BV, typename InT>
static hipError_t launch_serial(const BwdArgs& a, const float* ops, float* sw, float* dsw, bool concurrent) {
  const int n_chains = a.n_seqs * a.n_heads;
  const int64_t grid = (int64_t)((n_chains + 7) / 8) * 8 * (a.dv_dim / BV);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipStream_t main = (hipStream_t)a.stream, ds_stream = main;
  hipEvent_t fork = nullptr, join = nullptr;
  if (concurrent) {
    hipError_t e = side_stream(ds_stream);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&join, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(fork, main);
    if (e == hipSuccess) e = hipStreamWaitEvent(ds_stream, fork, 0);
    if (e != hipSuccess) {
      if (fork) (void)hipEventDestroy(fork);
      if (join) (void)hipEventDestroy(join);
      return e;
    }
  }
  auto finish = [&](hipError_t e) {  // join the side stream (also after a failed launch)
    if (concurrent) {
      hipError_t e2 = hipEventRecord(join, ds_stream);
      if (e2 == hipSuccess) e2 = hipStreamWaitEvent(main, join, 0);
      (void)hipEventDestroy(fork);
      (void)hipEventDestroy(join);
      if (e == hipSuccess) e = e2;
    }
    return e;
  };
  {
    constexpr size_t lds = ds_lds_bytes<DK, BV>();
    static_assert(lds <= 160 * 1024, "LDS budget");
    auto kern = bwd_ds_kernel<DK, BV>;
    static std::atomic<uint64_t> done{0};
    hipError_t e = set_lds((const void*)kern, lds, done);
    if (e != hipSuccess) return finish(e);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, ds_stream, a.cu_seqlens, a.dout, a.dhT, ops, dsw,
                       a.dh0, n_chains, a.n_heads, a.dv_dim, a.seq_len);
    e = hipGetLastError();
    if (e != hipSuccess) return finish(e);
  }
  {
    constexpr size_t lds = states_lds_bytes<DK, BV>();
    static_assert(lds <= 160 * 1024, "LDS budget");
    static_assert(BV != 64 || lds + ds_lds_bytes<DK, BV>() <= 160 * 1024, "one workgroup of each pass per CU");
    auto kern = bwd_states_kernel<DK, BV, InT>;
    static std::atomic<uint64_t> done{0};
    hipError_t e = set_lds((const void*)kern, lds, done);
    if (e != hipSuccess) return finish(e);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, main, (const InT*)a.v, a.h0, a.cu_seqlens, ops,
                       sw, n_chains, a.n_heads, a.dv_dim, a.seq_len);
    return finish(hipGetLastError());
  }
}

template <int DK, int DV, typename InT>
static hipError_t launch_grad(const BwdArgs& a, const float* ops, const float* sw, const float* dsw) {
  constexpr size_t lds = grad_lds_bytes<DK, DV>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = bwd_grad_kernel<DK, DV, InT>;
  static std::atomic<uint64_t> done{0};
  hipError_t e = set_lds((const void*)kern, lds, done);
  if (e != hipSuccess) return e;
  const int64_t grid = n_slots(a.total_tokens, a.n_seqs) * a.n_heads;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NTG), lds, (hipStream_t)a.stream, (const InT*)a.q,
                     (const InT*)a.k, (const InT*)a.v, a.cu_seqlens, a.dout, ops, sw, dsw, a.dq, a.dk, a.dv,
                     a.dlog_alpha, a.dbeta, a.n_heads, a.seq_len, a.n_seqs);
  return hipGetLastError();
}

template <int DK, int DV, typename InT>
static hipError_t run(const BwdArgs& a) {
  const size_t per = (size_t)n_slots(a.total_tokens, a.n_seqs) * a.n_heads;
  float* ops = (float*)a.ws;
  float* sw = ops + per * OpTile<DK>::FLOATS;
  float* dsw = sw + per * DK * DV;
  // (1) every chunk's operands
  hipError_t e = launch_prep<DK, InT>(a, ops);
  if (e != hipSuccess) return e;
  // (2) the states entering every chunk, (3) the cotangents of the states leaving them and dh0.
  // The two passes are independent: when one workgroup of each fits on every CU at once
  // (64-column tiles, chains x dv/64 <= 256) they run side by side; otherwise one after the
  // other in 32-column tiles, two or three workgroups of one pass per CU
  if ((int64_t)a.n_seqs * a.n_heads * (DV / 64) <= 256) e = launch_serial<DK, 64, InT>(a, ops, sw, dsw, true);
  else e = launch_serial<DK, 32, InT>(a, ops, sw, dsw, false);
  if (e != hipSuccess) return e;
  // (4) the gradients of every chunk
  return launch_grad<DK, DV, InT>(a, ops, sw, dsw);
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
  const size_t per_slot = ((size_t)65 * dk + 1044 + 2 * (size_t)dk * dv) * sizeof(float);
  return (size_t)bwdc::n_slots(total_tokens, n_seqs) * (size_t)n_heads * per_slot;
}

hipError_t launch_bwd_chunk(const BwdArgs& a) {
  if (a.n_seqs == 0) return hipSuccess;
  return a.bf16 ? bwdc::dispatch<bf16_t>(a) : bwdc::dispatch<float>(a);
}

}  // namespace kda
