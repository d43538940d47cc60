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
// Thread map: each wave owns 16 value columns and all DK rows, so the dk reductions
// never leave the wave and the token loop has no barrier.  Lane l of wave w holds
// row group rg = l & 15 (RPT = DK/16 rows: rg, rg + 16, ...) and columns
// [4 cg, 4 cg + 4) with cg = 4 w + (l >> 4); DV/16 waves per workgroup.  A
// reduction is in-lane over RPT rows, then a DPP scan across the 16 lanes of a row
// and a DPP broadcast of lane 15.  Every HBM access of S is a float4 per lane.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kMaxReplay = 8;

template <typename InT>
__device__ __forceinline__ float ld_in(const InT* p, size_t i) {
  return to_f32(p[i]);
}

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(DV * 4) void recurrent_step_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, float* __restrict__ S,
    float* __restrict__ o, const int32_t* __restrict__ n_commit, int n_tokens, int H) {
  constexpr int NTH = DV * 4;  // DV/16 waves
  constexpr int RPT = DK / 16;
  static_assert(DV % 16 == 0 && DK % 16 == 0, "thread map");

  __shared__ float s_q[kMaxReplay][DK];
  __shared__ float s_k[kMaxReplay][DK];
  __shared__ float s_a[kMaxReplay][DK];
  __shared__ float s_v[kMaxReplay][DV];
  __shared__ float s_b[kMaxReplay];
  __shared__ float s_qk[kMaxReplay];

  const int nh = blockIdx.x;  // sequence * H + head
  const int n = nh / H, h = nh - n * H;
  const int t = threadIdx.x;
  const int lane = t % kWave, wave = t / kWave;
  const int rg = lane & 15, cg = 4 * wave + (lane >> 4);

  // tokens whose updates reach the stored state (clamped to [0, n_tokens])
  int commit = n_tokens;
  if (n_commit) commit = min(max(n_commit[n], 0), n_tokens);

  float* Sp = S + (size_t)nh * DK * DV;
  float4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    st[i] = *reinterpret_cast<const float4*>(Sp + (size_t)(rg + 16 * i) * DV + cg * 4);

  // Stage the token inputs (the state loads above are still in flight).
  for (int idx = t; idx < n_tokens * DK; idx += NTH) {
    const int tok = idx / DK, c = idx - tok * DK;
    const size_t off = ((size_t)(n * n_tokens + tok) * H + h) * DK + c;
    s_q[tok][c] = ld_in(q, off);
    s_k[tok][c] = ld_in(k, off);
    s_a[tok][c] = expf(log_alpha[off]);
  }
  for (int idx = t; idx < n_tokens * DV; idx += NTH) {
    const int tok = idx / DV, j = idx - tok * DV;
    s_v[tok][j] = ld_in(v, ((size_t)(n * n_tokens + tok) * H + h) * DV + j);
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
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + 16 * i;
      const float a = s_a[tok][r], kr = s_k[tok][r], qr = s_q[tok][r];
      st[i].x *= a; st[i].y *= a; st[i].z *= a; st[i].w *= a;
      u.x += st[i].x * kr; u.y += st[i].y * kr; u.z += st[i].z * kr; u.w += st[i].w * kr;
      w.x += st[i].x * qr; w.y += st[i].y * qr; w.z += st[i].z * qr; w.w += st[i].w * qr;
    }
    u.x = row_sum16(u.x); u.y = row_sum16(u.y); u.z = row_sum16(u.z); u.w = row_sum16(u.w);
    w.x = row_sum16(w.x); w.y = row_sum16(w.y); w.z = row_sum16(w.z); w.w = row_sum16(w.w);
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
    for (int i = 0; i < RPT; ++i) {
      const float kr = s_k[tok][rg + 16 * i];
      st[i].x += kr * d.x; st[i].y += kr * d.y; st[i].z += kr * d.z; st[i].w += kr * d.w;
    }
    if (tok + 1 == commit) {
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        *reinterpret_cast<float4*>(Sp + (size_t)(rg + 16 * i) * DV + cg * 4) = st[i];
    }
  }
}

template <int DK, int DV, typename InT>
static hipError_t launch_rec(const RecurrentArgs& a) {
  dim3 grid((unsigned)((int64_t)a.n_seqs * a.n_heads)), block(DV * 4);
  hipLaunchKernelGGL((recurrent_step_kernel<DK, DV, InT>), grid, block, 0, (hipStream_t)a.stream,
                     (const InT*)a.q, (const InT*)a.k, (const InT*)a.v, a.log_alpha, a.beta, a.S, a.o,
                     a.n_commit, a.n_tokens, a.n_heads);
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
