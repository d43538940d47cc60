// Decode / draft-replay state update for KDA on gfx950.
//
// One workgroup owns one (sequence, head) state S [DK][DV] fp32 and keeps it in
// registers for the whole call: read once from HBM, n_tokens updates, written
// once (replay of cached projected inputs instead of per-draft snapshots,
// "Kimi K3 model structure (7)", section "KDA state rollback").  Per token, with
// S' = Diag(alpha) S (decay of the key rows):
//   u = S'^T k,  w = S'^T q          (reductions over the dk rows)
//   d = beta (v - u)
//   o = w + (q . k) d                (= S_new^T q)
//   S = S' + k d^T
// which is the recurrence S_new = (I - beta k k^T) S' + beta k v^T, o = S_new^T q
// regrouped so the state is traversed once per token.
//
// Replay + verify (same section: the cached inputs of accepted drafts are replayed
// onto the committed state, fused with verifying the new drafts): with a per-sequence
// commit count c, every token produces o, but the state is written back as it stands
// after token c - 1 (not at all for c = 0); later tokens are drafts whose updates are
// dropped.  Without counts, every token is committed.
//
// Thread map: a group of G = 8 consecutive lanes shares four value columns
// [4 cg, 4 cg + 4); lane rg of the group holds the DK / G contiguous key rows
// [rg DK/G, (rg + 1) DK/G) as float4s, DV/4 groups (256 threads for DV = 128).  The
// per-row inputs are read from LDS as float4s, and a reduction over dk is in-lane,
// then a 3-step DPP butterfly (quad swaps, half-row mirror) that leaves the sum in
// every lane of the group, so the token loop has no barrier.  Every HBM access of S is
// a float4 per lane, read and written non-temporally: each state tile is touched once
// per call, and streaming stores keep the written tiles from occupying the caches
// (measured on 256 x 32 states of 128 x 128: 245 -> 215 us at 8 tokens).
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kMaxReplay = 8;

// State tiles are read once and written once per call: streaming (non-temporal) accesses.
typedef float f32x4nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_state(const float* p) {
  const f32x4nt x = __builtin_nontemporal_load(reinterpret_cast<const f32x4nt*>(p));
  return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void st_state(float* p, const float4& v) {
  const f32x4nt x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4nt*>(p));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// sum over the aligned group of RG lanes, the same value (bit for bit) in every lane of the group
template <int RG>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<0xB1>(x);     // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);     // quad_perm [2,3,0,1]
  if constexpr (RG >= 8) x += dpp_f32<0x141>(x);   // row_half_mirror: the other quad of the 8
  if constexpr (RG >= 16) x += dpp_f32<0x140>(x);  // row_mirror: the other half of the 16
  return x;
}

template <typename InT> struct Stage;
template <> struct Stage<float> {
  static constexpr int VE = 4;
  __device__ static void load(float* d, const float* s) {
    *reinterpret_cast<float4*>(d) = *reinterpret_cast<const float4*>(s);
  }
};
template <> struct Stage<bf16_t> {
  static constexpr int VE = 8;
  __device__ static void load(float* d, const bf16_t* s) {
    const uint4 x = *reinterpret_cast<const uint4*>(s);
    const float2 a = bf16x2_to_f32x2(x.x), b = bf16x2_to_f32x2(x.y), c = bf16x2_to_f32x2(x.z),
                 e = bf16x2_to_f32x2(x.w);
    *reinterpret_cast<float4*>(d) = make_float4(a.x, a.y, b.x, b.y);
    *reinterpret_cast<float4*>(d + 4) = make_float4(c.x, c.y, e.x, e.y);
  }
};

template <int DK, int DV, int RG, typename InT>
__global__ __launch_bounds__(DV / 4 * RG) void recurrent_group_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, float* __restrict__ S,
    float* __restrict__ o, const int32_t* __restrict__ n_commit, int n_tokens, int H) {
  constexpr int NTH = DV / 4 * RG;
  constexpr int RPL = DK / RG;
  constexpr int VE = Stage<InT>::VE;
  static_assert(RG == 4 || RG == 8 || RG == 16, "group size");
  static_assert(RPL % 4 == 0 && DK % VE == 0 && DV % VE == 0, "thread map");

  __shared__ __attribute__((aligned(16))) float s_q[kMaxReplay][DK];
  __shared__ __attribute__((aligned(16))) float s_k[kMaxReplay][DK];
  __shared__ __attribute__((aligned(16))) float s_a[kMaxReplay][DK];
  __shared__ __attribute__((aligned(16))) float s_v[kMaxReplay][DV];
  __shared__ float s_b[kMaxReplay];
  __shared__ float s_qk[kMaxReplay];

  const int nh = blockIdx.x;  // sequence * H + head
  const int n = nh / H, h = nh - n * H;
  const int t = threadIdx.x;
  const int lane = t % kWave, wave = t / kWave;
  const int rg = t % RG, cg = t / RG;
  const int r0 = rg * RPL;  // the lane's rows are r0 .. r0 + RPL - 1

  // tokens whose updates reach the stored state (clamped to [0, n_tokens])
  int commit = n_tokens;
  if (n_commit) commit = min(max(n_commit[n], 0), n_tokens);

  float* Sp = S + (size_t)nh * DK * DV + (size_t)r0 * DV + cg * 4;
  float4 st[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) st[i] = ld_state(Sp + (size_t)i * DV);

  // Stage the token inputs (the state loads above are still in flight).
  for (int idx = t; idx < n_tokens * (DK / VE); idx += NTH) {
    const int tok = idx / (DK / VE), c = (idx - tok * (DK / VE)) * VE;
    const size_t off = ((size_t)(n * n_tokens + tok) * H + h) * DK + c;
    Stage<InT>::load(&s_q[tok][c], q + off);
    Stage<InT>::load(&s_k[tok][c], k + off);
  }
  for (int idx = t; idx < n_tokens * (DK / 4); idx += NTH) {
    const int tok = idx / (DK / 4), c = (idx - tok * (DK / 4)) * 4;
    const float4 la = *reinterpret_cast<const float4*>(log_alpha + ((size_t)(n * n_tokens + tok) * H + h) * DK + c);
    *reinterpret_cast<float4*>(&s_a[tok][c]) = make_float4(expf(la.x), expf(la.y), expf(la.z), expf(la.w));
  }
  for (int idx = t; idx < n_tokens * (DV / VE); idx += NTH) {
    const int tok = idx / (DV / VE), j = (idx - tok * (DV / VE)) * VE;
    Stage<InT>::load(&s_v[tok][j], v + ((size_t)(n * n_tokens + tok) * H + h) * DV + j);
  }
  if (t < n_tokens) s_b[t] = beta[(size_t)(n * n_tokens + t) * H + h];
  __syncthreads();
  // q . k per token: wave w reduces tokens w, w + waves, ...
  for (int tok = wave; tok < n_tokens; tok += NTH / kWave) {
    float p = 0.f;
    for (int c = lane; c < DK; c += kWave) p += s_q[tok][c] * s_k[tok][c];
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) p += wave_xor(p, m);
    if (lane == 0) s_qk[tok] = p;
  }
  __syncthreads();

  for (int tok = 0; tok < n_tokens; ++tok) {
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f), w = u;
#pragma unroll
    for (int i4 = 0; i4 < RPL; i4 += 4) {
      const float4 a4 = *reinterpret_cast<const float4*>(&s_a[tok][r0 + i4]);
      const float4 k4 = *reinterpret_cast<const float4*>(&s_k[tok][r0 + i4]);
      const float4 q4 = *reinterpret_cast<const float4*>(&s_q[tok][r0 + i4]);
      const float av[4] = {a4.x, a4.y, a4.z, a4.w}, kv[4] = {k4.x, k4.y, k4.z, k4.w},
                  qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float4& x = st[i4 + e];
        const float a = av[e], kr = kv[e], qr = qv[e];
        x.x *= a; x.y *= a; x.z *= a; x.w *= a;
        u.x += x.x * kr; u.y += x.y * kr; u.z += x.z * kr; u.w += x.w * kr;
        w.x += x.x * qr; w.y += x.y * qr; w.z += x.z * qr; w.w += x.w * qr;
      }
    }
    u.x = group_sum<RG>(u.x); u.y = group_sum<RG>(u.y); u.z = group_sum<RG>(u.z); u.w = group_sum<RG>(u.w);
    w.x = group_sum<RG>(w.x); w.y = group_sum<RG>(w.y); w.z = group_sum<RG>(w.z); w.w = group_sum<RG>(w.w);
    const float b = s_b[tok], qk = s_qk[tok];
    const float4 vv = *reinterpret_cast<const float4*>(&s_v[tok][cg * 4]);
    float4 d;
    d.x = b * (vv.x - u.x); d.y = b * (vv.y - u.y); d.z = b * (vv.z - u.z); d.w = b * (vv.w - u.w);
    if (rg == 0) {
      float4 ot;
      ot.x = w.x + qk * d.x; ot.y = w.y + qk * d.y; ot.z = w.z + qk * d.z; ot.w = w.w + qk * d.w;
      *reinterpret_cast<float4*>(o + ((size_t)(n * n_tokens + tok) * H + h) * DV + cg * 4) = ot;
    }
#pragma unroll
    for (int i4 = 0; i4 < RPL; i4 += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(&s_k[tok][r0 + i4]);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float4& x = st[i4 + e];
        const float kr = kv[e];
        x.x += kr * d.x; x.y += kr * d.y; x.z += kr * d.z; x.w += kr * d.w;
      }
    }
    if (tok + 1 == commit) {
#pragma unroll
      for (int i = 0; i < RPL; ++i) st_state(Sp + (size_t)i * DV, st[i]);
    }
  }
}

template <int DK, int DV, typename InT>
static hipError_t launch_rec(const RecurrentArgs& a) {
  const dim3 grid((unsigned)((int64_t)a.n_seqs * a.n_heads));
  constexpr int G = 8;
  hipLaunchKernelGGL((recurrent_group_kernel<DK, DV, G, InT>), grid, dim3(DV / 4 * G), 0, (hipStream_t)a.stream,
                     (const InT*)a.q, (const InT*)a.k, (const InT*)a.v, a.log_alpha, a.beta, a.S, a.o, a.n_commit,
                     a.n_tokens, a.n_heads);
  return hipGetLastError();
}

template <typename InT>
static hipError_t dispatch_rec_dims(const RecurrentArgs& a) {
  if (a.dk == 128 && a.dv == 128) return launch_rec<128, 128, InT>(a);
  if (a.dk == 64 && a.dv == 64) return launch_rec<64, 64, InT>(a);
  if (a.dk == 128 && a.dv == 64) return launch_rec<128, 64, InT>(a);
  if (a.dk == 64 && a.dv == 128) return launch_rec<64, 128, InT>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_recurrent_step(const RecurrentArgs& a) {
  if (a.n_seqs == 0) return hipSuccess;
  return a.bf16 ? dispatch_rec_dims<bf16_t>(a) : dispatch_rec_dims<float>(a);
}

}  // namespace kda
