// C ABI of the KDA library: argument validation on the host, then dispatch.
// Every argument error is caught here, before any launch, and leaves no side
// effects.  See include/kda.h for the contract of each entry point.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_launch.hpp"

// The workspace of kda_chunk_fwd_split_noalloc: one array per GPU in the library's device
// memory.  Host code never uses its name as an address: each device's address is looked up
// once with hipGetSymbolAddress (scratch_address) and that pointer goes to the kernels.
static __device__ __attribute__((aligned(256))) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dims_ok(int32_t d) { return d == 64 || d == 128; }

// a byte range of one buffer (n == 0: absent)
struct Range {
  const void* p;
  size_t n;
};
bool overlap(const Range& a, const Range& b) {
  const char* pa = (const char*)a.p;
  const char* pb = (const char*)b.p;
  return a.n && b.n && pa < pb + b.n && pb < pa + a.n;
}

// The device address of `scratch` on the current device: looked up on the first call per device
// (devices past the 64th look it up on every call).
std::mutex scratch_mu;
void* scratch_ptr[64] = {};
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (dev >= 0 && dev < 64 && scratch_ptr[dev]) {
    *out = scratch_ptr[dev];
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  if (dev >= 0 && dev < 64) scratch_ptr[dev] = p;
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

static kda_status chunk_common(const void* q, const void* k, const void* v, const float* log_alpha,
                               const float* beta, const float* h0, const int32_t* cu_seqlens, int32_t n_seqs,
                               int64_t total_tokens, int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk_size,
                               kda_dtype qkv_dtype, float* o, float* hT, int32_t ckpt_every, float* ckpt,
                               bool split, void* ws, size_t ws_bytes, void* stream, bool noalloc = false) {
  if (n_seqs < 0 || total_tokens < 0 || n_heads <= 0 || dk <= 0 || dv <= 0 || chunk_size <= 0)
    return KDA_ERR_INVALID_ARGUMENT;
  // checkpoints: ckpt_every > 0 and a multiple of the chunk size; ckpt holds
  // total_tokens / ckpt_every slots and may be NULL only when that is zero
  int64_t n_slots = 0;
  if (ckpt_every != 0 || ckpt) {
    if (ckpt_every <= 0 || ckpt_every % chunk_size != 0) return KDA_ERR_INVALID_ARGUMENT;
    n_slots = total_tokens / ckpt_every;
    if (n_slots > 0 && (!ckpt || !aligned16(ckpt))) return KDA_ERR_INVALID_ARGUMENT;
    if (n_slots == 0) ckpt = nullptr;
  }
  if (ckpt) {
    // the checkpoints are outputs: they must not overlap any input or other output
    const char* cb = (const char*)ckpt;
    const char* ce = cb + (size_t)n_slots * n_heads * dk * dv * sizeof(float);
    const size_t esz = qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4;
    struct R { const void* p; size_t n; } bufs[] = {
        {q, (size_t)total_tokens * n_heads * dk * esz}, {k, (size_t)total_tokens * n_heads * dk * esz},
        {v, (size_t)total_tokens * n_heads * dv * esz}, {log_alpha, (size_t)total_tokens * n_heads * dk * 4},
        {beta, (size_t)total_tokens * n_heads * 4}, {o, (size_t)total_tokens * n_heads * dv * 4},
        {h0, h0 ? (size_t)n_seqs * n_heads * dk * dv * 4 : 0}, {hT, hT ? (size_t)n_seqs * n_heads * dk * dv * 4 : 0},
        {cu_seqlens, cu_seqlens ? (size_t)(n_seqs + 1) * 4 : 0}};
    for (const R& r : bufs) {
      const char* b = (const char*)r.p;
      if (r.n && b < ce && cb < b + r.n) return KDA_ERR_INVALID_ARGUMENT;
    }
  }
  if (qkv_dtype != KDA_DTYPE_F32 && qkv_dtype != KDA_DTYPE_BF16) return KDA_ERR_INVALID_ARGUMENT;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_INVALID_ARGUMENT;
  if (n_seqs == 0 && total_tokens != 0) return KDA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {q, k, v, log_alpha, beta, h0, cu_seqlens, o, hT};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_INVALID_ARGUMENT;
  int64_t seq_len = 0;
  if (!cu_seqlens && n_seqs > 0) {
    if (total_tokens % n_seqs != 0) return KDA_ERR_INVALID_ARGUMENT;
    seq_len = total_tokens / n_seqs;
  }
  // o must not overlap the inputs it is computed from (checked on the byte ranges)
  if (o && total_tokens > 0) {
    const char* ob = (const char*)o;
    const char* oe = ob + (size_t)total_tokens * n_heads * dv * sizeof(float);
    const size_t esz = qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4;
    struct R { const void* p; size_t n; } ins[] = {
        {q, (size_t)total_tokens * n_heads * dk * esz}, {k, (size_t)total_tokens * n_heads * dk * esz},
        {v, (size_t)total_tokens * n_heads * dv * esz}, {log_alpha, (size_t)total_tokens * n_heads * dk * 4},
        {beta, (size_t)total_tokens * n_heads * 4}};
    for (const R& r : ins) {
      const char* b = (const char*)r.p;
      if (b < oe && ob < b + r.n) return KDA_ERR_INVALID_ARGUMENT;
    }
  }
  // hT is an output: it must not overlap o or an input, except that it may be h0 itself
  // (in-place advance: every workgroup reads its h0 tile before it writes that hT tile)
  if (hT && n_seqs > 0) {
    const size_t esz = qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const size_t T = (size_t)total_tokens, Hh = (size_t)n_heads;
    const Range h{hT, (size_t)n_seqs * n_heads * dk * dv * sizeof(float)};
    const Range others[] = {{q, T * Hh * dk * esz}, {k, T * Hh * dk * esz}, {v, T * Hh * dv * esz},
                            {log_alpha, T * Hh * dk * 4}, {beta, T * Hh * 4}, {o, T * Hh * dv * 4},
                            {cu_seqlens, cu_seqlens ? (size_t)(n_seqs + 1) * 4 : 0},
                            {h0 == hT ? nullptr : h0, h0 && h0 != hT ? h.n : 0}};
    for (const Range& r : others)
      if (overlap(h, r)) return KDA_ERR_INVALID_ARGUMENT;
  }
  if (total_tokens > INT32_MAX) return KDA_ERR_UNSUPPORTED;  // cu_seqlens is int32
  if ((int64_t)n_seqs * n_heads * 8 > INT32_MAX) return KDA_ERR_UNSUPPORTED;  // grid: chains x value tiles
  if (!dims_ok(dk) || !dims_ok(dv)) return KDA_ERR_UNSUPPORTED;
  const bool bf16 = qkv_dtype == KDA_DTYPE_BF16;
  if (!kda::chunk_fwd_supported(dk, dv, chunk_size, bf16)) return KDA_ERR_UNSUPPORTED;
  if (split) {
    if (!bf16) return KDA_ERR_UNSUPPORTED;
    const size_t need = kda::chunk_split_workspace_bytes(total_tokens, n_seqs, n_heads, dk, dv, chunk_size);
    if (noalloc && n_seqs > 0 && total_tokens > 0) {
      // the library's own array in place of a caller workspace
      if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_UNSUPPORTED;
      if (scratch_address(&ws) != hipSuccess) return KDA_ERR_LAUNCH;
      ws_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    }
    if (n_seqs > 0 && total_tokens > 0) {
      if (!ws || !aligned16(ws) || ws_bytes < need) return KDA_ERR_INVALID_ARGUMENT;
      // the workspace must not overlap any input or output
      const char* wb = (const char*)ws;
      const char* we = wb + need;
      const size_t esz = 2;
      struct R { const void* p; size_t n; } bufs[] = {
          {q, (size_t)total_tokens * n_heads * dk * esz}, {k, (size_t)total_tokens * n_heads * dk * esz},
          {v, (size_t)total_tokens * n_heads * dv * esz}, {log_alpha, (size_t)total_tokens * n_heads * dk * 4},
          {beta, (size_t)total_tokens * n_heads * 4}, {o, (size_t)total_tokens * n_heads * dv * 4},
          {h0, h0 ? (size_t)n_seqs * n_heads * dk * dv * 4 : 0}, {hT, hT ? (size_t)n_seqs * n_heads * dk * dv * 4 : 0},
          {cu_seqlens, cu_seqlens ? (size_t)(n_seqs + 1) * 4 : 0}};
      for (const R& r : bufs) {
        const char* b = (const char*)r.p;
        if (r.n && b < we && wb < b + r.n) return KDA_ERR_INVALID_ARGUMENT;
      }
    }
  }
  if (n_seqs == 0) return KDA_OK;

  kda::ChunkArgs a;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.h0 = h0;
  a.cu_seqlens = cu_seqlens; a.o = o; a.hT = hT; a.ckpt = ckpt; a.ckpt_every = ckpt ? ckpt_every : 1;
  a.n_seqs = n_seqs; a.n_heads = n_heads; a.dk = dk; a.dv = dv; a.chunk_size = chunk_size;
  a.total_tokens = total_tokens; a.seq_len = seq_len; a.bf16 = bf16; a.stream = stream;
  if (split) {
    if (total_tokens == 0) return kda::launch_chunk_fwd(a) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;  // hT only
    return kda::launch_chunk_fwd_split(a, ws) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
  }
  return kda::launch_chunk_fwd(a) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* h0, const int32_t* cu_seqlens,
                         int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                         int32_t dv, int32_t chunk_size, kda_dtype qkv_dtype, float* o, float* hT,
                         void* stream) {
  return chunk_common(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens, n_heads, dk, dv, chunk_size,
                      qkv_dtype, o, hT, 0, nullptr, false, nullptr, 0, stream);
}

kda_status kda_chunk_fwd_split_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                                              int32_t dv, int32_t chunk_size, kda_dtype qkv_dtype, size_t* bytes) {
  if (!bytes || n_seqs < 0 || total_tokens < 0 || n_heads <= 0 || dk <= 0 || dv <= 0 || chunk_size <= 0)
    return KDA_ERR_INVALID_ARGUMENT;
  if (qkv_dtype != KDA_DTYPE_F32 && qkv_dtype != KDA_DTYPE_BF16) return KDA_ERR_INVALID_ARGUMENT;
  if (!dims_ok(dk) || !dims_ok(dv) || qkv_dtype != KDA_DTYPE_BF16 ||
      !kda::chunk_fwd_supported(dk, dv, chunk_size, true))
    return KDA_ERR_UNSUPPORTED;
  *bytes = kda::chunk_split_workspace_bytes(total_tokens, n_seqs, n_heads, dk, dv, chunk_size);
  return KDA_OK;
}

kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, const float* log_alpha,
                               const float* beta, const float* h0, const int32_t* cu_seqlens, int32_t n_seqs,
                               int64_t total_tokens, int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk_size,
                               kda_dtype qkv_dtype, float* o, float* hT, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return chunk_common(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens, n_heads, dk, dv, chunk_size,
                      qkv_dtype, o, hT, 0, nullptr, true, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_auto(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, const float* h0, const int32_t* cu_seqlens, int32_t n_seqs,
                              int64_t total_tokens, int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk_size,
                              kda_dtype qkv_dtype, float* o, float* hT, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const bool split = qkv_dtype == KDA_DTYPE_BF16 && n_heads > 0 && dv > 0 &&
                     kda::chunk_fwd_prefers_split(n_seqs, n_heads, dv, chunk_size, total_tokens);
  return chunk_common(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens, n_heads, dk, dv, chunk_size,
                      qkv_dtype, o, hT, 0, nullptr, split, split ? workspace : nullptr, split ? workspace_bytes : 0,
                      stream);
}

kda_status kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                       const float* beta, const float* h0, const int32_t* cu_seqlens,
                                       int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                                       int32_t dv, int32_t chunk_size, kda_dtype qkv_dtype, float* o, float* hT,
                                       void* stream) {
  return chunk_common(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens, n_heads, dk, dv, chunk_size,
                      qkv_dtype, o, hT, 0, nullptr, true, nullptr, 0, stream, true);
}

kda_status kda_chunk_fwd_checkpointed(const void* q, const void* k, const void* v, const float* log_alpha,
                                      const float* beta, const float* h0, const int32_t* cu_seqlens,
                                      int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                                      int32_t dv, int32_t chunk_size, kda_dtype qkv_dtype, float* o, float* hT,
                                      int32_t ckpt_every, float* ckpt, void* stream) {
  if (ckpt_every <= 0) return KDA_ERR_INVALID_ARGUMENT;
  return chunk_common(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens, n_heads, dk, dv, chunk_size,
                      qkv_dtype, o, hT, ckpt_every, ckpt, false, nullptr, 0, stream);
}

static size_t bwd_ws_bytes(bool chunk, int64_t total_tokens, int n_seqs, int n_heads, int dk, int dv) {
  return chunk ? kda::bwd_chunk_workspace_bytes(total_tokens, n_seqs, n_heads, dk, dv)
               : kda::bwd_workspace_bytes(total_tokens, n_seqs, n_heads, dk, dv);
}

static kda_status bwd_ws_common(bool chunk, int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                                int32_t dv, size_t* bytes) {
  if (!bytes || n_seqs < 0 || total_tokens < 0 || n_heads <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARGUMENT;
  if (!dims_ok(dk) || !dims_ok(dv)) return KDA_ERR_UNSUPPORTED;
  *bytes = bwd_ws_bytes(chunk, total_tokens, n_seqs, n_heads, dk, dv);
  return KDA_OK;
}

kda_status kda_bwd_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk, int32_t dv,
                                  size_t* bytes) {
  return bwd_ws_common(true, n_seqs, total_tokens, n_heads, dk, dv, bytes);
}

kda_status kda_bwd_recurrent_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                                            int32_t dv, size_t* bytes) {
  return bwd_ws_common(false, n_seqs, total_tokens, n_heads, dk, dv, bytes);
}

static kda_status bwd_common(bool chunk, const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const float* h0, const int32_t* cu_seqlens, int32_t n_seqs,
                             int64_t total_tokens, int32_t n_heads, int32_t dk, int32_t dv, kda_dtype qkv_dtype,
                             const float* dout, const float* dhT, float* dq, float* dk_out, float* dv_out,
                             float* dlog_alpha, float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (n_seqs < 0 || total_tokens < 0 || n_heads <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARGUMENT;
  if (qkv_dtype != KDA_DTYPE_F32 && qkv_dtype != KDA_DTYPE_BF16) return KDA_ERR_INVALID_ARGUMENT;
  if (n_seqs == 0 && total_tokens != 0) return KDA_ERR_INVALID_ARGUMENT;
  if (total_tokens > 0 &&
      (!q || !k || !v || !log_alpha || !beta || !dout || !dq || !dk_out || !dv_out || !dlog_alpha || !dbeta))
    return KDA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {q, k, v, log_alpha, beta, h0, cu_seqlens, dout, dhT, dq, dk_out, dv_out, dlog_alpha,
                        dbeta, dh0, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_INVALID_ARGUMENT;
  int64_t seq_len = 0;
  if (!cu_seqlens && n_seqs > 0) {
    if (total_tokens % n_seqs != 0) return KDA_ERR_INVALID_ARGUMENT;
    seq_len = total_tokens / n_seqs;
  }
  if (total_tokens > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)n_seqs * n_heads > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if (!dims_ok(dk) || !dims_ok(dv)) return KDA_ERR_UNSUPPORTED;
  if (n_seqs == 0) return KDA_OK;
  const size_t need = bwd_ws_bytes(chunk, total_tokens, n_seqs, n_heads, dk, dv);
  if (!workspace || workspace_bytes < need) return KDA_ERR_INVALID_ARGUMENT;
  // every output (and the workspace) must not overlap any input or any other output
  const size_t esz = qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4;
  const size_t T = (size_t)total_tokens, Hh = (size_t)n_heads, st = (size_t)n_seqs * n_heads * dk * dv * 4;
  struct R { const void* p; size_t n; };
  const R ins[] = {{q, T * Hh * dk * esz}, {k, T * Hh * dk * esz}, {v, T * Hh * dv * esz},
                   {log_alpha, T * Hh * dk * 4}, {beta, T * Hh * 4}, {h0, h0 ? st : 0},
                   {cu_seqlens, cu_seqlens ? (size_t)(n_seqs + 1) * 4 : 0}, {dout, T * Hh * dv * 4},
                   {dhT, dhT ? st : 0}};
  const R outs[] = {{dq, T * Hh * dk * 4}, {dk_out, T * Hh * dk * 4}, {dv_out, T * Hh * dv * 4},
                    {dlog_alpha, T * Hh * dk * 4}, {dbeta, T * Hh * 4}, {dh0, dh0 ? st : 0},
                    {workspace, need}};
  auto overlap = [](const R& a, const R& b) {
    const char* pa = (const char*)a.p;
    const char* pb = (const char*)b.p;
    return a.n && b.n && pa < pb + b.n && pb < pa + a.n;
  };
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const R& r : ins)
      if (overlap(outs[i], r)) return KDA_ERR_INVALID_ARGUMENT;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j])) return KDA_ERR_INVALID_ARGUMENT;
  }
  kda::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.h0 = h0; a.cu_seqlens = cu_seqlens;
  a.dout = dout; a.dhT = dhT; a.dq = dq; a.dk = dk_out; a.dv = dv_out; a.dlog_alpha = dlog_alpha;
  a.dbeta = dbeta; a.dh0 = dh0; a.ws = workspace; a.n_seqs = n_seqs; a.n_heads = n_heads; a.dk_dim = dk;
  a.dv_dim = dv; a.total_tokens = total_tokens; a.seq_len = seq_len; a.bf16 = qkv_dtype == KDA_DTYPE_BF16;
  a.stream = stream;
  return (chunk ? kda::launch_bwd_chunk(a) : kda::launch_bwd(a)) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status kda_bwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                   const float* h0, const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens, int32_t n_heads,
                   int32_t dk, int32_t dv, kda_dtype qkv_dtype, const float* dout, const float* dhT, float* dq,
                   float* dk_out, float* dv_out, float* dlog_alpha, float* dbeta, float* dh0, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return bwd_common(true, q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens, n_heads, dk, dv, qkv_dtype,
                    dout, dhT, dq, dk_out, dv_out, dlog_alpha, dbeta, dh0, workspace, workspace_bytes, stream);
}

kda_status kda_bwd_recurrent(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                             const float* h0, const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                             int32_t n_heads, int32_t dk, int32_t dv, kda_dtype qkv_dtype, const float* dout,
                             const float* dhT, float* dq, float* dk_out, float* dv_out, float* dlog_alpha,
                             float* dbeta, float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(false, q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens, n_heads, dk, dv,
                    qkv_dtype, dout, dhT, dq, dk_out, dv_out, dlog_alpha, dbeta, dh0, workspace, workspace_bytes,
                    stream);
}

static kda_status recurrent_common(const void* q, const void* k, const void* v, const float* log_alpha,
                                   const float* beta, float* S_inout, const int32_t* n_commit, bool need_commit,
                                   int32_t n_seqs, int32_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv,
                                   kda_dtype qkv_dtype, float* o, void* stream) {
  if (n_seqs < 0 || n_tokens <= 0 || n_heads <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARGUMENT;
  if (qkv_dtype != KDA_DTYPE_F32 && qkv_dtype != KDA_DTYPE_BF16) return KDA_ERR_INVALID_ARGUMENT;
  if (n_seqs > 0 && (!q || !k || !v || !log_alpha || !beta || !S_inout || !o)) return KDA_ERR_INVALID_ARGUMENT;
  if (n_seqs > 0 && need_commit && !n_commit) return KDA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {q, k, v, log_alpha, beta, S_inout, o};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_INVALID_ARGUMENT;
  if (n_commit && ((uintptr_t)n_commit & 3)) return KDA_ERR_INVALID_ARGUMENT;
  if (!dims_ok(dk) || !dims_ok(dv) || n_tokens > 8) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)n_seqs * n_heads > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if (n_seqs == 0) return KDA_OK;
  // the state is read and written in place: it must not overlap the token inputs or the commit
  // counts (o is checked below)
  {
    const size_t ntok = (size_t)n_seqs * n_tokens * n_heads;
    const size_t esz = qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const Range st{S_inout, (size_t)n_seqs * n_heads * dk * dv * 4};
    const Range ins[] = {{q, ntok * dk * esz}, {k, ntok * dk * esz}, {v, ntok * dv * esz}, {log_alpha, ntok * dk * 4},
                         {beta, ntok * 4}, {n_commit, n_commit ? (size_t)n_seqs * 4 : 0}};
    for (const Range& r : ins)
      if (overlap(st, r)) return KDA_ERR_INVALID_ARGUMENT;
  }
  // o must not overlap the state, the token inputs or the commit counts
  {
    const bool bf16 = qkv_dtype == KDA_DTYPE_BF16;
    const size_t ntok = (size_t)n_seqs * n_tokens * n_heads;
    const char* ob = (const char*)o;
    const char* oe = ob + ntok * dv * sizeof(float);
    const size_t esz = bf16 ? 2 : 4;
    struct R { const void* p; size_t n; } ins[] = {
        {q, ntok * dk * esz}, {k, ntok * dk * esz}, {v, ntok * dv * esz},
        {log_alpha, ntok * dk * 4}, {beta, ntok * 4}, {S_inout, (size_t)n_seqs * n_heads * dk * dv * 4},
        {n_commit, n_commit ? (size_t)n_seqs * 4 : 0}};
    for (const R& r : ins) {
      const char* b = (const char*)r.p;
      if (r.n && b < oe && ob < b + r.n) return KDA_ERR_INVALID_ARGUMENT;
    }
  }
  kda::RecurrentArgs a;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.S = S_inout; a.o = o;
  a.n_commit = n_commit;
  a.n_seqs = n_seqs; a.n_tokens = n_tokens; a.n_heads = n_heads; a.dk = dk; a.dv = dv;
  a.bf16 = qkv_dtype == KDA_DTYPE_BF16; a.stream = stream;
  return kda::launch_recurrent_step(a) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, float* S_inout, int32_t n_seqs, int32_t n_tokens,
                              int32_t n_heads, int32_t dk, int32_t dv, kda_dtype qkv_dtype, float* o,
                              void* stream) {
  return recurrent_common(q, k, v, log_alpha, beta, S_inout, nullptr, false, n_seqs, n_tokens, n_heads, dk, dv,
                          qkv_dtype, o, stream);
}

kda_status kda_recurrent_verify(const void* q, const void* k, const void* v, const float* log_alpha,
                                const float* beta, float* S_inout, const int32_t* n_commit, int32_t n_seqs,
                                int32_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv, kda_dtype qkv_dtype,
                                float* o, void* stream) {
  return recurrent_common(q, k, v, log_alpha, beta, S_inout, n_commit, true, n_seqs, n_tokens, n_heads, dk, dv,
                          qkv_dtype, o, stream);
}

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH";
  }
  return "KDA_ERR_UNKNOWN";
}

int32_t kda_version(void) { return 10200; }

}  // extern "C"
