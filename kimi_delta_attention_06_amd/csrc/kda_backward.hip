// Backward pass of the KDA recurrence on gfx950 (token-recurrent, fp32).
//
// The recurrence (S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t) is differentiated token by token in reverse: with
// P = Diag(a_t) S_{t-1}, u = P^T k_t, d = b_t (v_t - u), S_t = P + k_t d^T and the adjoint
// dS of S_t (dS_L = dhT),
//   dS      += q_t do_t^T
//   dq_t     = S_t do_t
//   dd       = dS^T k_t,   dv_t = b_t dd,   db_t = dd . (v_t - u),   du = -b_t dd
//   dk_t     = dS d + P du
//   dP       = dS + k_t du^T,   dlog a_t[c] = sum_j dP[c][j] P[c][j]
//   dS       = Diag(a_t) dP            (the adjoint of S_{t-1}; dh0 is the last one)
// (the reverse mode of the forward written out in order).  The backward pass and its
// gradients dq, dk, dv, dbeta, the gate gradient and the state gradient are what
// training needs beyond the published inference forward ("Kimi K3 NPU Training",
// conclusions, item 1, and the NPU operator-support table, KDA backward row).
//
// Two workgroups per (sequence, head), each owning half of the value columns (the
// columns of S evolve independently), DV/32 waves each, with the decode kernel's thread
// map: lane l of wave w holds rows rg = l & 15, rg + 16, ... and value columns
// [j0 + 16 w + 4 (l >> 4), +4).  The row gradients of the second half go to the
// workspace and are added to the first half's by a small kernel (a two-term sum, so the
// result does not depend on which half finishes first).  Column reductions (over rows: u, dd) stay in the wave
// (in-lane, then a DPP row sum); row reductions (over columns: dq, dk, dlog a, db) are
// summed across the wave's four column groups with lane shuffles and across waves
// through LDS once per batch of kB tokens.
//
// The reverse sweep needs every S_{t-1}.  Phase 1 runs the forward once and keeps the
// state at the start of every kL-token segment (workspace, `ckpt`); phase 2 walks the
// segments backwards, recomputes the segment's per-token states into a per-chain
// scratch (`tok`), then runs the adjoint over the segment.  Every thread reads back only
// the state entries it wrote itself.
#include <atomic>

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kBwdB = 8;    // tokens per staged batch
constexpr int kBwdL = 64;   // tokens per recomputed segment (a multiple of kBwdB)

template <int DK, int DV, typename InT>
__global__ __launch_bounds__(DV * 2) void bwd_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, const float* __restrict__ h0,
    const int32_t* __restrict__ cu_seqlens, const float* __restrict__ dout, const float* __restrict__ dhT,
    float* __restrict__ dq, float* __restrict__ dk_out, float* __restrict__ dv_out, float* __restrict__ dla,
    float* __restrict__ dbeta, float* __restrict__ dh0, float* __restrict__ ckpt, float* __restrict__ tok,
    float* __restrict__ part, int H, int64_t seq_len, int64_t total_tokens) {
  constexpr int NTH = DV * 2, NWV = DV / 32, RPT = DK / 16;
  constexpr int B = kBwdB, L = kBwdL;
  static_assert(DV % 16 == 0 && DK % 16 == 0 && L % B == 0, "thread map");

  // dynamic LDS: staged token inputs, then the per-wave row partials of dq, dk, dlog a and db
  extern __shared__ __attribute__((aligned(16))) float smem_b[];
  float(*s_q)[DK] = reinterpret_cast<float(*)[DK]>(smem_b);
  float(*s_k)[DK] = reinterpret_cast<float(*)[DK]>(smem_b + B * DK);
  float(*s_a)[DK] = reinterpret_cast<float(*)[DK]>(smem_b + 2 * B * DK);
  float(*s_v)[DV] = reinterpret_cast<float(*)[DV]>(smem_b + 3 * B * DK);
  float(*s_do)[DV] = reinterpret_cast<float(*)[DV]>(smem_b + 3 * B * DK + B * DV);
  float* s_b = smem_b + 3 * B * DK + 2 * B * DV;
  float(*s_red)[NWV][3][DK] = reinterpret_cast<float(*)[NWV][3][DK]>(smem_b + 3 * B * DK + 2 * B * DV + B);
  float(*s_redb)[NWV] = reinterpret_cast<float(*)[NWV]>(smem_b + 3 * B * DK + 2 * B * DV + B + B * NWV * 3 * DK);

  const int chain = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int n = chain / H, h = chain - n * H;
  // the second half's row gradients: partial dq, dk, dlog a [3][T][H][DK] and db [T][H]
  if (half) {
    const size_t TH = (size_t)total_tokens * H;
    dq = part;
    dk_out = part + TH * DK;
    dla = part + 2 * TH * DK;
    dbeta = part + 3 * TH * DK;
  }
  int64_t t_begin, t_end;
  if (cu_seqlens) {
    t_begin = cu_seqlens[n];
    t_end = cu_seqlens[n + 1];
  } else {
    t_begin = (int64_t)n * seq_len;
    t_end = t_begin + seq_len;
  }
  const int64_t len = t_end - t_begin;
  const int64_t nseg = (len + L - 1) / L;

  const int t = threadIdx.x;
  const int lane = t % kWave, wave = t / kWave;
  const int rg = lane & 15, c0 = half * (DV / 2) + 16 * wave + 4 * (lane >> 4);
  constexpr size_t SD = (size_t)DK * DV;

  // state at the start of segment s: slot t_begin / L + n + s (distinct for any packing)
  auto ckpt_at = [&](int64_t s) { return ckpt + ((size_t)(t_begin / L + n + s) * H + h) * SD; };
  float* tok_base = tok + (size_t)chain * L * SD;  // per-token states of the current segment

  float4 S[RPT];
  auto store_state = [&](float* p, const float4 (&X)[RPT]) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) *reinterpret_cast<float4*>(p + (size_t)(rg + 16 * i) * DV + c0) = X[i];
  };
  auto load_state = [&](const float* p, float4 (&X)[RPT]) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) X[i] = *reinterpret_cast<const float4*>(p + (size_t)(rg + 16 * i) * DV + c0);
  };
  // tokens [t0, t0 + cnt) into slots 0 .. cnt-1 (q and do only for the reverse sweep)
  auto stage = [&](int64_t t0, int cnt, bool rev) {
    for (int idx = t; idx < cnt * DK; idx += NTH) {
      const int j = idx / DK, c = idx - j * DK;
      const size_t off = ((size_t)(t0 + j) * H + h) * DK + c;
      s_k[j][c] = to_f32(k[off]);
      s_a[j][c] = expf(log_alpha[off]);
      if (rev) s_q[j][c] = to_f32(q[off]);
    }
    for (int idx = t; idx < cnt * (DV / 2); idx += NTH) {
      const int j = idx / (DV / 2), c = half * (DV / 2) + idx - j * (DV / 2);
      const size_t off = ((size_t)(t0 + j) * H + h) * DV + c;
      s_v[j][c] = to_f32(v[off]);
      if (rev) s_do[j][c] = dout[off];
    }
    if (t < cnt) s_b[t] = beta[(size_t)(t0 + t) * H + h];
  };
  // one forward token on the state S (staged slot j)
  auto fwd_token = [&](int j) {
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + 16 * i;
      const float a = s_a[j][r], kr = s_k[j][r];
      S[i].x *= a; S[i].y *= a; S[i].z *= a; S[i].w *= a;
      u.x += S[i].x * kr; u.y += S[i].y * kr; u.z += S[i].z * kr; u.w += S[i].w * kr;
    }
    u.x = row_sum16(u.x); u.y = row_sum16(u.y); u.z = row_sum16(u.z); u.w = row_sum16(u.w);
    const float b = s_b[j];
    const float4 vv = *reinterpret_cast<const float4*>(&s_v[j][c0]);
    const float4 d = make_float4(b * (vv.x - u.x), b * (vv.y - u.y), b * (vv.z - u.z), b * (vv.w - u.w));
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float kr = s_k[j][rg + 16 * i];
      S[i].x += kr * d.x; S[i].y += kr * d.y; S[i].z += kr * d.z; S[i].w += kr * d.w;
    }
  };

  // ---- phase 1: forward, keeping the state at every segment start
  const float* h0p = h0 ? h0 + (size_t)chain * SD : nullptr;
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    S[i] = h0p ? *reinterpret_cast<const float4*>(h0p + (size_t)(rg + 16 * i) * DV + c0) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t s = 0; s < nseg; ++s) {
    store_state(ckpt_at(s), S);
    const int64_t sb = t_begin + s * L, se = sb + L < t_end ? sb + L : t_end;
    for (int64_t t0 = sb; t0 < se; t0 += B) {
      const int cnt = (int)(se - t0 < B ? se - t0 : B);
      __syncthreads();
      stage(t0, cnt, false);
      __syncthreads();
      for (int j = 0; j < cnt; ++j) fwd_token(j);
    }
  }

  // ---- phase 2: adjoint, segments in reverse
  float4 dS[RPT];
  const float* dhTp = dhT ? dhT + (size_t)chain * SD : nullptr;
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    dS[i] = dhTp ? *reinterpret_cast<const float4*>(dhTp + (size_t)(rg + 16 * i) * DV + c0) : make_float4(0.f, 0.f, 0.f, 0.f);
  __threadfence();  // phase 1's checkpoint stores before their loads (the same thread's data)

  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t sb = t_begin + s * L, se = sb + L < t_end ? sb + L : t_end;
    // (a) recompute the segment's states S_t, stored per token
    load_state(ckpt_at(s), S);
    for (int64_t t0 = sb; t0 < se; t0 += B) {
      const int cnt = (int)(se - t0 < B ? se - t0 : B);
      __syncthreads();
      stage(t0, cnt, false);
      __syncthreads();
      for (int j = 0; j < cnt; ++j) {
        fwd_token(j);
        store_state(tok_base + (size_t)(t0 + j - sb) * SD, S);
      }
    }
    __threadfence();
    // (b) the adjoint over the segment; S holds S_t for the token being processed
    const int64_t nb = (se - sb + B - 1) / B;
    for (int64_t bi = nb - 1; bi >= 0; --bi) {
      const int64_t t0 = sb + bi * B;
      const int cnt = (int)(se - t0 < B ? se - t0 : B);
      __syncthreads();
      stage(t0, cnt, true);
      __syncthreads();
      float4 Sn[RPT];  // S_{t-1} of the batch's last token, loaded ahead
      {
        const int64_t it = t0 + cnt - 1 - sb;
        load_state(it > 0 ? tok_base + (size_t)(it - 1) * SD : ckpt_at(s), Sn);
      }
      for (int j = cnt - 1; j >= 0; --j) {
        const int64_t it = t0 + j - sb;  // token index inside the segment
        float4 Sp[RPT];                  // S_{t-1}; P = Diag(a_t) S_{t-1} is formed on the fly
#pragma unroll
        for (int i = 0; i < RPT; ++i) Sp[i] = Sn[i];
        // the next (earlier) token's S_{t-2}, in flight during this token's work
        if (j > 0) load_state(it > 1 ? tok_base + (size_t)(it - 2) * SD : ckpt_at(s), Sn);
        float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int r = rg + 16 * i;
          const float ak = s_a[j][r] * s_k[j][r];
          u.x += Sp[i].x * ak; u.y += Sp[i].y * ak; u.z += Sp[i].z * ak; u.w += Sp[i].w * ak;
        }
        u.x = row_sum16(u.x); u.y = row_sum16(u.y); u.z = row_sum16(u.z); u.w = row_sum16(u.w);
        const float b = s_b[j];
        const float4 vv = *reinterpret_cast<const float4*>(&s_v[j][c0]);
        const float4 dov = *reinterpret_cast<const float4*>(&s_do[j][c0]);
        const float4 d = make_float4(b * (vv.x - u.x), b * (vv.y - u.y), b * (vv.z - u.z), b * (vv.w - u.w));
        // read-out: dS += q do^T, dq = S_t do (this lane's four columns)
        float pq[RPT];
        float4 dd = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int r = rg + 16 * i;
          const float qr = s_q[j][r], kr = s_k[j][r];
          dS[i].x += qr * dov.x; dS[i].y += qr * dov.y; dS[i].z += qr * dov.z; dS[i].w += qr * dov.w;
          pq[i] = S[i].x * dov.x + S[i].y * dov.y + S[i].z * dov.z + S[i].w * dov.w;
          dd.x += dS[i].x * kr; dd.y += dS[i].y * kr; dd.z += dS[i].z * kr; dd.w += dS[i].w * kr;
        }
        dd.x = row_sum16(dd.x); dd.y = row_sum16(dd.y); dd.z = row_sum16(dd.z); dd.w = row_sum16(dd.w);
        if (rg == 0) {
          *reinterpret_cast<float4*>(dv_out + ((size_t)(t0 + j) * H + h) * DV + c0) =
              make_float4(b * dd.x, b * dd.y, b * dd.z, b * dd.w);
        }
        float pb = dd.x * (vv.x - u.x) + dd.y * (vv.y - u.y) + dd.z * (vv.z - u.z) + dd.w * (vv.w - u.w);
        const float4 du = make_float4(-b * dd.x, -b * dd.y, -b * dd.z, -b * dd.w);
        float pk[RPT], pl[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int r = rg + 16 * i;
          const float kr = s_k[j][r], a = s_a[j][r];
          pk[i] = dS[i].x * d.x + dS[i].y * d.y + dS[i].z * d.z + dS[i].w * d.w +
                  a * (Sp[i].x * du.x + Sp[i].y * du.y + Sp[i].z * du.z + Sp[i].w * du.w);
          const float4 dP = make_float4(dS[i].x + kr * du.x, dS[i].y + kr * du.y, dS[i].z + kr * du.z,
                                        dS[i].w + kr * du.w);
          pl[i] = a * (dP.x * Sp[i].x + dP.y * Sp[i].y + dP.z * Sp[i].z + dP.w * Sp[i].w);
          dS[i] = make_float4(a * dP.x, a * dP.y, a * dP.z, a * dP.w);
          S[i] = Sp[i];  // the earlier token's own state
        }
        // Row partials: sum over this wave's four column groups (lanes rg, rg+16, rg+32, rg+48).
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          pq[i] += wave_xor(pq[i], 16); pq[i] += wave_xor(pq[i], 32);
          pk[i] += wave_xor(pk[i], 16); pk[i] += wave_xor(pk[i], 32);
          pl[i] += wave_xor(pl[i], 16); pl[i] += wave_xor(pl[i], 32);
        }
        pb += wave_xor(pb, 16);
        pb += wave_xor(pb, 32);
        if (lane < 16) {
#pragma unroll
          for (int i = 0; i < RPT; ++i) {
            const int r = rg + 16 * i;
            s_red[j][wave][0][r] = pq[i];
            s_red[j][wave][1][r] = pk[i];
            s_red[j][wave][2][r] = pl[i];
          }
        }
        if (lane == 0) s_redb[j][wave] = pb;
      }
      __syncthreads();
      // sum the batch's row partials over waves: dq, dk, dlog a per (token, row), db per token
      for (int idx = t; idx < cnt * 3 * DK; idx += NTH) {
        const int j = idx / (3 * DK), rem = idx - j * 3 * DK, kind = rem / DK, r = rem - kind * DK;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) acc += s_red[j][w][kind][r];
        float* dst = kind == 0 ? dq : kind == 1 ? dk_out : dla;
        dst[((size_t)(t0 + j) * H + h) * DK + r] = acc;
      }
      if (t < cnt) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) acc += s_redb[t][w];
        dbeta[(size_t)(t0 + t) * H + h] = acc;
      }
    }
  }
  if (dh0) store_state(dh0 + (size_t)chain * SD, dS);
}

// second-half row gradients added to the first half's: x[i] += p[i]
__global__ void bwd_add_kernel(float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dla,
                               float* __restrict__ db, const float* __restrict__ part, int64_t nk, int64_t nb) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = i; j < nk; j += stride) {
    dq[j] += part[j];
    dk[j] += part[nk + j];
    dla[j] += part[2 * nk + j];
  }
  for (int64_t j = i; j < nb; j += stride) db[j] += part[3 * nk + j];
}

size_t bwd_workspace_bytes(int64_t total_tokens, int n_seqs, int n_heads, int dk, int dv) {
  const size_t sd = (size_t)dk * dv * sizeof(float);
  const size_t ck = ((size_t)(total_tokens / kBwdL) + (size_t)n_seqs + 1) * (size_t)n_heads * sd;
  const size_t tk = (size_t)n_seqs * n_heads * kBwdL * sd;
  const size_t th = (size_t)total_tokens * n_heads;
  const size_t pt = (3 * th * dk + th) * sizeof(float);
  return ck + tk + ((pt + 15) & ~size_t(15));
}

template <int DK, int DV, typename InT>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  float* ck = (float*)a.ws;
  float* tk = ck + ((size_t)(a.total_tokens / kBwdL) + (size_t)a.n_seqs + 1) * a.n_heads * DK * DV;
  float* pt = tk + (size_t)a.n_seqs * a.n_heads * kBwdL * DK * DV;
  constexpr int NWV = DV / 32;
  constexpr size_t lds = sizeof(float) * ((size_t)3 * kBwdB * DK + 2 * kBwdB * DV + kBwdB + (size_t)kBwdB * NWV * 3 * DK +
                                          kBwdB * NWV);
  static std::atomic<uint64_t> attr_done{0};
  {
    int dev = 0;
    hipError_t e0 = hipGetDevice(&dev);
    if (e0 != hipSuccess) return e0;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
    if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
      e0 = hipFuncSetAttribute((const void*)bwd_kernel<DK, DV, InT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds);
      if (e0 != hipSuccess) return e0;
      if (bit) attr_done.fetch_or(bit, std::memory_order_release);
    }
  }
  hipLaunchKernelGGL((bwd_kernel<DK, DV, InT>), dim3((unsigned)((int64_t)a.n_seqs * a.n_heads * 2)), dim3(DV * 2), lds,
                     (hipStream_t)a.stream, (const InT*)a.q, (const InT*)a.k, (const InT*)a.v, a.log_alpha, a.beta,
                     a.h0, a.cu_seqlens, a.dout, a.dhT, a.dq, a.dk, a.dv, a.dlog_alpha, a.dbeta, a.dh0, ck, tk, pt,
                     a.n_heads, a.seq_len, a.total_tokens);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nk = a.total_tokens * a.n_heads * DK, nb = a.total_tokens * a.n_heads;
  const int64_t blocks = (nk + 255) / 256 < 4096 ? (nk + 255) / 256 : 4096;
  hipLaunchKernelGGL(bwd_add_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, (hipStream_t)a.stream,
                     a.dq, a.dk, a.dlog_alpha, a.dbeta, (const float*)pt, nk, nb);
  return hipGetLastError();
}

template <typename InT>
static hipError_t dispatch_bwd(const BwdArgs& a) {
  if (a.dk_dim == 128 && a.dv_dim == 128) return launch_bwd_t<128, 128, InT>(a);
  if (a.dk_dim == 64 && a.dv_dim == 64) return launch_bwd_t<64, 64, InT>(a);
  if (a.dk_dim == 128 && a.dv_dim == 64) return launch_bwd_t<128, 64, InT>(a);
  if (a.dk_dim == 64 && a.dv_dim == 128) return launch_bwd_t<64, 128, InT>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.n_seqs == 0) return hipSuccess;
  return a.bf16 ? dispatch_bwd<bf16_t>(a) : dispatch_bwd<float>(a);
}

}  // namespace kda
