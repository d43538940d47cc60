// Internal launch interface between the C ABI (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct RecurrentArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  float* S;
  float* o;
  const int32_t* n_commit;  // may be null: every token is committed
  int n_seqs, n_tokens, n_heads, dk, dv;
  bool bf16;
  void* stream;
};

struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  const float* h0;          // may be null
  const int32_t* cu_seqlens; // may be null (equal lengths)
  float* o;
  float* hT;                // may be null
  float* ckpt;              // may be null: no checkpoints
  int ckpt_every;           // checkpoint spacing in tokens (a multiple of chunk_size)
  int n_seqs, n_heads, dk, dv, chunk_size;
  int64_t total_tokens;
  int64_t seq_len;          // used when cu_seqlens is null
  bool bf16;
  void* stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  const float* h0;           // may be null
  const int32_t* cu_seqlens; // may be null (equal lengths)
  const float* dout;         // cotangent of o
  const float* dhT;          // cotangent of hT, may be null
  float* dq;
  float* dk;
  float* dv;
  float* dlog_alpha;
  float* dbeta;
  float* dh0;                // may be null
  void* ws;                  // bwd_workspace_bytes(...) bytes
  int n_seqs, n_heads, dk_dim, dv_dim;
  int64_t total_tokens;
  int64_t seq_len;
  bool bf16;
  void* stream;
};

hipError_t launch_recurrent_step(const RecurrentArgs& a);
// Backward pass (token-recurrent, fp32 state and gradients).
hipError_t launch_bwd(const BwdArgs& a);
size_t bwd_workspace_bytes(int64_t total_tokens, int n_seqs, int n_heads, int dk, int dv);
// Backward pass (chunkwise, fp32 matrix core): per-chunk operands, forward states and reverse
// dS passes, per-chunk gradients.
hipError_t launch_bwd_chunk(const BwdArgs& a);
size_t bwd_chunk_workspace_bytes(int64_t total_tokens, int n_seqs, int n_heads, int dk, int dv);
hipError_t launch_chunk_fwd(const ChunkArgs& a);
// Split path (bf16 only): intra-chunk pass into `ws`, then the state pass.
hipError_t launch_chunk_fwd_split(const ChunkArgs& a, void* ws);
// Workspace bytes the split path needs for these sizes.
size_t chunk_split_workspace_bytes(int64_t total_tokens, int n_seqs, int n_heads, int dk, int dv, int chunk_size);
// whether kda_chunk_fwd_auto takes the split path for a bf16 input of this shape
bool chunk_fwd_prefers_split(int n_seqs, int n_heads, int dv, int chunk_size, int64_t total_tokens);
// True if the chunk kernel has an instantiation for these parameters.
bool chunk_fwd_supported(int dk, int dv, int chunk_size, bool bf16);

}  // namespace kda
