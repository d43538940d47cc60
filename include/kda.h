/*
 * kda.h - C ABI of the KDA (Kimi Delta Attention) operator library for AMD
 * Instinct MI355X (gfx950).  Plain pointers and sizes only.
 *
 * The operator.  KDA is a delta-rule linear-attention recurrence with a
 * channel-wise forget gate ("Kimi K3 technical report summary", section 1,
 * pre-training table, KDA row; "Kimi K3 NPU Training", section "confirmed
 * skeleton": unlike the scalar gate per head of Gated DeltaNet, KDA gates every
 * channel).  For each sequence n and head h it carries a dk x dv matrix state S
 * (rows: key channels, columns: value channels) and, for each token t in order,
 *
 *     S <- (I - beta_t k_t k_t^T) Diag(alpha_t) S + beta_t k_t v_t^T,
 *     o_t = S^T q_t,          alpha_t = exp(log_alpha_t) (one gate per key channel).
 *
 * q and k are expected L2-normalised per (token, head) by the caller (the layer
 * normalises them before the recurrence, "Kimi K3 NPU Training", section
 * "confirmed skeleton", list item 3); the kernels take them as stored.  There is
 * no 1/sqrt(dk) scale: fold any scale into q.
 *
 * Memory layouts (all dense, row-major, element strides as listed):
 *   q, k       [T_total, H, dk]   token-major, heads inner (a fixed-length
 *                                  [B, T, H, d] tensor is the same memory)
 *   v          [T_total, H, dv]
 *   log_alpha  [T_total, H, dk]   fp32, <= 0 (a gate in [0, 1]); any finite value
 *   beta       [T_total, H]       fp32, in [0, 1]
 *   o          [T_total, H, dv]   fp32 output
 *   h0, hT     [N, H, dk, dv]     fp32 states
 *   cu_seqlens [N + 1]            int32 offsets of packed sequences
 *
 * Ownership and threading.  The caller allocates and frees every buffer.  The
 * library allocates no memory at run time and is safe to call from several host
 * threads.  Its only mutable global state is set up once and never read back:
 * one word per kernel that records, thread-safely, on which devices the kernel's
 * LDS limit was raised, the per-device address of the fixed device array of
 * kda_chunk_fwd_split_noalloc (looked up under a lock), and one non-blocking
 * side stream per device that kda_bwd creates under a lock on first use and
 * keeps until the process ends (each kda_bwd call that forks to it creates and
 * destroys its own two events).  All pointers except
 * cu_seqlens-for-fixed-length, h0 and hT are required.  Device pointers must be
 * 16-byte aligned.
 *
 * Asynchrony and errors.  Calls enqueue kernels on `stream` (a hipStream_t;
 * NULL is the default stream) and return at once; results are valid once the
 * stream is synchronised.  Argument errors are detected on the host before any
 * launch and return a status with no side effects.  A launch failure reported
 * by the HIP runtime returns KDA_ERR_LAUNCH.  Nothing is printed and no C++
 * exception crosses this interface.  The fused chunked-forward kernels
 * (kda_chunk_fwd, kda_chunk_fwd_checkpointed
 * and kda_chunk_fwd_split on zero tokens) are built for XNACK off, the MI355X
 * default; in a process with XNACK on they do not load and those calls return
 * KDA_ERR_LAUNCH.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, negative size, misalignment */
  KDA_ERR_UNSUPPORTED = 2,      /* valid but outside the compiled shape / dtype set */
  KDA_ERR_LAUNCH = 3            /* the HIP runtime rejected a kernel launch */
} kda_status;

typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype;

/*
 * kda_chunk_fwd - chunkwise-parallel forward (training / prefill).
 *
 * Computes the recurrence above over packed sequences, parallel inside each
 * chunk of `chunk_size` tokens and recurrent across chunks ("Kimi K3 technical
 * report summary", section 1, pre-training table, KDA row: chunk-wise parallel
 * form).  The state is reset at every sequence boundary of cu_seqlens (state
 * reset at packed boundaries: "Kimi K3 NPU Training", section "TND is not a
 * layout switch", item 2); chunks never span two sequences and the last chunk
 * of a sequence may be partial.
 *
 *   q, k, v      device, qkv_dtype (KDA_DTYPE_BF16: bfloat16; KDA_DTYPE_F32: float)
 *   log_alpha    device fp32 [total_tokens, n_heads, dk]
 *   beta         device fp32 [total_tokens, n_heads]
 *   h0           device fp32 [n_seqs, n_heads, dk, dv], or NULL for zero states
 *   cu_seqlens   device int32 [n_seqs + 1] with cu[0] = 0, non-decreasing,
 *                cu[n_seqs] = total_tokens; or NULL for n_seqs equal sequences of
 *                total_tokens / n_seqs tokens (total_tokens must divide evenly)
 *   o            device fp32 [total_tokens, n_heads, dv], written for every token
 *   hT           device fp32 [n_seqs, n_heads, dk, dv], the state after each
 *                sequence's last token (h0 for an empty sequence), or NULL to skip.
 *                hT may alias h0 (in-place advance); o must not alias any input.
 *
 * Supported: dk, dv in {64, 128}; chunk_size in {16, 32, 64}; qkv_dtype F32 or
 * BF16 (F32 with dk = 128 and chunk_size 64 runs in chunks of 32 tokens, which
 * changes only the rounding).  Other shapes return KDA_ERR_UNSUPPORTED.
 *
 * Range.  Any finite log_alpha <= 0 and any bf16 magnitude of q, k, v and h0 are
 * taken.  A token's log_alpha below -110.9 nats (-160 in base 2) counts as -110.9
 * (a factor of 6.6e-49 is already 0 against any other term in fp32).  A 16-token
 * block whose decay spread exceeds 160 nats forms its decayed Gram products
 * element by element, exactly, instead of from factors balanced around the
 * block's middle.  With BF16 inputs the state and values of each chunk are
 * scaled by a power of two chosen per chunk to fit the fp16 matrix-core operands;
 * o and hT are scaled back.  NaN inputs give NaN outputs where they reach.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* h0, const int32_t* cu_seqlens,
                         int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                         int32_t dv, int32_t chunk_size, kda_dtype qkv_dtype, float* o, float* hT,
                         void* stream);

/*
 * kda_chunk_fwd_checkpointed - kda_chunk_fwd that also stores periodic states.
 *
 * For prefix-cache reuse the state is kept only at the ends of fixed-size hash
 * blocks of 512 tokens ("Kimi K3 model structure (7)", section "Prefix cache:
 * decoupled granularity, 512-token reuse").  Same arguments and results as
 * kda_chunk_fwd, plus:
 *
 *   ckpt_every   checkpoint spacing in tokens, > 0 and a multiple of chunk_size
 *                (512 for 512-token hash blocks)
 *   ckpt         device fp32 [total_tokens / ckpt_every, n_heads, dk, dv]; the
 *                state of sequence n after its first p tokens, for every positive
 *                multiple p of ckpt_every up to the sequence length, is written to
 *                slot (cu_seqlens[n] + p) / ckpt_every - 1 (n * seq_len in place
 *                of cu_seqlens[n] for equal lengths).  These slots are distinct;
 *                slots that no checkpoint maps to are left untouched.  May be NULL
 *                only when total_tokens < ckpt_every.  Must not overlap any other
 *                buffer.
 *
 * Errors: as kda_chunk_fwd, plus KDA_ERR_INVALID_ARGUMENT for ckpt_every <= 0,
 * ckpt_every not a multiple of chunk_size, a NULL or misaligned ckpt when slots
 * exist, or ckpt overlapping another buffer.
 */
kda_status kda_chunk_fwd_checkpointed(const void* q, const void* k, const void* v, const float* log_alpha,
                                      const float* beta, const float* h0, const int32_t* cu_seqlens,
                                      int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                                      int32_t dv, int32_t chunk_size, kda_dtype qkv_dtype, float* o, float* hT,
                                      int32_t ckpt_every, float* ckpt, void* stream);

/*
 * kda_chunk_fwd_split - kda_chunk_fwd in two passes, for inputs with few
 * (sequence, head) chains such as one long sequence.
 *
 * The chunkwise form separates work inside a chunk (decay, Gram matrices, the
 * UT inverse) from the propagation of the state across chunks ("Kimi K3 model
 * structure (7)", Q&A on the training/prefill kernel; the same page lists
 * in-device context parallelism among KDA's execution forms).  Pass 1 does the
 * in-chunk work for every chunk of every head at once, in parallel over the
 * whole sequence, and writes each chunk's state-free operands to `workspace`;
 * pass 2 walks the chunks of each chain with the state, reading them.  When the
 * state pass fits on half of the CUs (chains x dv/32 <= 128) and the longest
 * sequence has at least 135 chunks, the chunks are cut into 2 to 48 ranges, each
 * about 1.1 times the size of the one before it, and each launch runs pass 2 over one range
 * beside pass 1 over the next, with the state handed between ranges through the
 * workspace.  With fewer chains still
 * (chains x dv/32 <= 64: 16 at dv = 128) and at least 512 chunks in the longest
 * sequence, pass 2 itself runs in parallel over S = 4 to 64 segments of each
 * chain (in-device context parallelism, the same page: KDA states cannot simply
 * be added, so they are composed by an associative scan): the affine map
 * S_out = M S_in + B of every segment but the last is found in parallel (the
 * recurrence run on a dk x (dk + dv) state [I | 0] with values [0 | v]), the maps
 * are composed in fp32 from h0 in order, and every segment is then rerun from
 * its entering state (1M tokens at dk = dv = 128: 1 head 2.5 ms, 8 heads 13.3 ms
 * on MI355X, against 32-34 ms without segments).  Results equal kda_chunk_fwd's
 * up to rounding (the same operand precisions; the segmented form also rounds
 * each segment's map).
 *
 * Same arguments and results as kda_chunk_fwd, plus:
 *
 *   workspace        device scratch of at least the size that
 *                    kda_chunk_fwd_split_workspace_size returns for the same
 *                    sizes; 16-byte aligned; must not overlap any other buffer.
 *                    Its contents are undefined before and after the call.
 *   workspace_bytes  its size in bytes
 *
 * Supported: as kda_chunk_fwd with qkv_dtype BF16 only (KDA_ERR_UNSUPPORTED
 * otherwise).  Errors: as kda_chunk_fwd, plus KDA_ERR_INVALID_ARGUMENT for a
 * NULL, misaligned, too small or overlapping workspace when tokens exist.
 */
kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, const float* log_alpha,
                               const float* beta, const float* h0, const int32_t* cu_seqlens, int32_t n_seqs,
                               int64_t total_tokens, int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk_size,
                               kda_dtype qkv_dtype, float* o, float* hT, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * kda_chunk_fwd_auto - the chunked forward on whichever path is faster for the
 * input's shape: kda_chunk_fwd_split or kda_chunk_fwd (same results up to
 * rounding).  The fused kernel cuts each chain's dv columns into the widest value
 * tiles (at most 64 columns) that still give every CU a workgroup and redoes each
 * chunk's in-chunk work once per tile; the split path does that work once per
 * chunk and head but writes it to the workspace and reads it back.  With bf16
 * inputs and sequences of at least 4 chunks on average, the split path is taken
 * when the fused kernel would use two or more tiles per chain and either those
 * tiles need more than one round of 256 workgroups or the sequences average at
 * least 16 chunks; otherwise, and for fp32 inputs, the fused kernel.  Measured on
 * MI355X at dk = 128, chunk 64: 1M tokens x 32 heads (dv 128) 35 ms split vs 96
 * ms fused; 8 x 4,096 tokens x 32 heads 0.79 vs 0.93 ms; 4 x 4,096 x 32 heads
 * 0.42 vs 0.47 ms; 16 x 4,096 x 32 heads at dv = 64 (one tile per chain) 0.94 ms
 * fused vs 1.42 ms split.
 *
 * Same arguments as kda_chunk_fwd_split.  The workspace is used only when the
 * split path is taken (it may be NULL with workspace_bytes 0 otherwise); a caller
 * that always passes kda_chunk_fwd_split_workspace_size bytes is always valid.
 * Errors: as the path taken.
 */
kda_status kda_chunk_fwd_auto(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, const float* h0, const int32_t* cu_seqlens, int32_t n_seqs,
                              int64_t total_tokens, int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk_size,
                              kda_dtype qkv_dtype, float* o, float* hT, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * kda_chunk_fwd_split_noalloc - kda_chunk_fwd_split for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Instead of a caller workspace it uses a
 * fixed array of KDA_NOALLOC_SCRATCH_BYTES in the library's device memory, one
 * per GPU, held until the process ends; nothing is allocated on any call.
 * Calls on one GPU share that array and the contents of the last call stay in
 * it, so calls that overlap in time on one GPU (several streams or host
 * threads) race and must not be made.  The first call on a device looks up that
 * device's array address.
 *
 * Same arguments and results as kda_chunk_fwd_split without workspace and
 * workspace_bytes.  Errors: as kda_chunk_fwd_split, plus KDA_ERR_UNSUPPORTED when
 * the workspace these sizes need (kda_chunk_fwd_split_workspace_size) exceeds
 * KDA_NOALLOC_SCRATCH_BYTES, and KDA_ERR_LAUNCH when the array's address cannot
 * be obtained.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
kda_status kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                       const float* beta, const float* h0, const int32_t* cu_seqlens,
                                       int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                                       int32_t dv, int32_t chunk_size, kda_dtype qkv_dtype, float* o, float* hT,
                                       void* stream);

/*
 * kda_chunk_fwd_split_workspace_size - bytes of workspace kda_chunk_fwd_split
 * needs: (total_tokens / chunk_size + n_seqs + 1) * n_heads tiles of the
 * per-chunk operands (62,208 B each for dk = 128, chunk 64), then
 * n_seqs * n_heads fp32 dk x dv states; then, when n_seqs * n_heads * dv / 32
 * <= 64 and m = ceil(total_tokens / chunk_size) >= 512, for S = min(64, m / 64)
 * segments, (S - 1) * n_seqs * n_heads fp32 dk x (dk + dv) segment maps and
 * S * n_seqs * n_heads fp32 dk x dv segment states.  Writes *bytes.
 * Errors: KDA_ERR_INVALID_ARGUMENT (NULL bytes, negative or zero sizes, bad
 * dtype), KDA_ERR_UNSUPPORTED (a combination kda_chunk_fwd_split does not take).
 */
kda_status kda_chunk_fwd_split_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                                              int32_t dv, int32_t chunk_size, kda_dtype qkv_dtype, size_t* bytes);

/*
 * kda_bwd - backward pass of the recurrence (reverse mode), chunkwise.
 *
 * Training needs the gradients of KDA beyond the published inference forward
 * ("Kimi K3 NPU Training", conclusions, item 1, and the NPU operator-support
 * table, KDA backward row).  For the same inputs as kda_chunk_fwd and the
 * cotangents `dout` of o and `dhT` of the final states, writes the gradients of
 *     sum_t o_t . dout_t + sum_n hT_n . dhT_n
 * with respect to q, k, v, log_alpha, beta and h0.  Reverse mode of the chunk
 * form in 16-token chunks, every product in fp32: a parallel pass forms every
 * chunk's state-free operands into `workspace`, a forward pass over each
 * sequence's chunks stores the state entering every chunk, a reverse pass stores
 * the cotangent of the state leaving every chunk, and a parallel pass forms each
 * chunk's gradients from the three.  When n_seqs * n_heads * dv / 64 <= 256 the
 * reverse pass runs beside the forward pass on a second stream the library keeps
 * per device, forked from and joined back to `stream` through events, so the call
 * is still ordered on `stream` and can be captured into a HIP graph.
 *
 *   q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens, n_heads,
 *   dk, dv, qkv_dtype    as kda_chunk_fwd (the chunk size is fixed at 16)
 *   dout        device fp32 [total_tokens, n_heads, dv]
 *   dhT         device fp32 [n_seqs, n_heads, dk, dv] or NULL (zeros)
 *   dq, dk_out, dlog_alpha   device fp32 [total_tokens, n_heads, dk]
 *   dv_out      device fp32 [total_tokens, n_heads, dv]
 *   dbeta       device fp32 [total_tokens, n_heads]
 *   dh0         device fp32 [n_seqs, n_heads, dk, dv] or NULL (not written)
 *   workspace   device scratch of at least kda_bwd_workspace_size bytes; contents
 *               undefined before and after the call
 *
 * Outputs and the workspace must not overlap any input or each other.  All
 * pointers 16-byte aligned.  Supported: dk, dv in {64, 128}; qkv_dtype F32 or
 * BF16.  Any finite log_alpha <= 0: a token's log_alpha below -110 nats counts
 * as -110, and a 16-token chunk that decays by more than 64 nats in some channel
 * forms its decay factors element by element (exactly) instead of balanced
 * around the chunk's middle.  Errors as kda_chunk_fwd, plus
 * KDA_ERR_INVALID_ARGUMENT for a missing, small or overlapping workspace or
 * overlapping outputs.
 */
kda_status kda_bwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                   const float* h0, const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens, int32_t n_heads,
                   int32_t dk, int32_t dv, kda_dtype qkv_dtype, const float* dout, const float* dhT, float* dq,
                   float* dk_out, float* dv_out, float* dlog_alpha, float* dbeta, float* dh0, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * kda_bwd_workspace_size - bytes of workspace kda_bwd needs:
 * (total_tokens / 16 + n_seqs + 1) * n_heads * (2 * dk * dv + 65 * dk + 1044) * 4.
 * Errors: KDA_ERR_INVALID_ARGUMENT (NULL bytes, bad sizes), KDA_ERR_UNSUPPORTED (dk, dv).
 */
kda_status kda_bwd_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk, int32_t dv,
                                  size_t* bytes);

/*
 * kda_bwd_recurrent - the same gradients as kda_bwd, token by token.
 *
 * Differentiates the recurrence one token at a time in fp32 (the reverse mode of
 * the per-token update, the same passage as kda_bwd): the state at the start of
 * every 64-token segment is kept in `workspace`, each segment's per-token states are
 * recomputed into it, and the adjoint runs backwards over them.  It shares none of
 * kda_bwd's chunk algebra (a cross-check of it) and is
 * much slower than kda_bwd on long sequences.  Arguments, outputs and errors as
 * kda_bwd, with kda_bwd_recurrent_workspace_size bytes of workspace.
 */
kda_status kda_bwd_recurrent(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                             const float* h0, const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                             int32_t n_heads, int32_t dk, int32_t dv, kda_dtype qkv_dtype, const float* dout,
                             const float* dhT, float* dq, float* dk_out, float* dv_out, float* dlog_alpha,
                             float* dbeta, float* dh0, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_bwd_recurrent_workspace_size - bytes of workspace kda_bwd_recurrent needs:
 * (total_tokens / 64 + n_seqs + 1 + 64 * n_seqs) * n_heads * dk * dv * 4 (states)
 * + (3 * dk + 1) * total_tokens * n_heads * 4 rounded up to 16 (partial gradients).
 * Errors: KDA_ERR_INVALID_ARGUMENT (NULL bytes, bad sizes), KDA_ERR_UNSUPPORTED (dk, dv).
 */
kda_status kda_bwd_recurrent_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t n_heads, int32_t dk,
                                            int32_t dv, size_t* bytes);

/*
 * kda_recurrent_step - decode / draft-replay state update.
 *
 * For each of n_seqs sequences, applies n_tokens consecutive tokens to the
 * state S_inout in place and writes one output per token (decode updates each
 * head's fixed matrix state per token: "Kimi K3 NPU Training", section
 * "confirmed skeleton", list item 4; replay rebuilds the state from cached
 * projected inputs of accepted draft tokens instead of restoring snapshots:
 * "Kimi K3 model structure (7)", section "KDA state rollback").  The state is
 * read once and written once per call for any n_tokens.
 *
 *   q, k, v      device, qkv_dtype, [n_seqs, n_tokens, n_heads, dk | dv]
 *   log_alpha    device fp32 [n_seqs, n_tokens, n_heads, dk]
 *   beta         device fp32 [n_seqs, n_tokens, n_heads]
 *   S_inout      device fp32 [n_seqs, n_heads, dk, dv], updated in place
 *   o            device fp32 [n_seqs, n_tokens, n_heads, dv]; must not alias inputs
 *
 * Supported: dk, dv in {64, 128}; n_tokens in [1, 8]; qkv_dtype F32 or BF16.
 */
kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, float* S_inout, int32_t n_seqs, int32_t n_tokens,
                              int32_t n_heads, int32_t dk, int32_t dv, kda_dtype qkv_dtype, float* o,
                              void* stream);

/*
 * kda_recurrent_verify - replay accepted drafts and verify new ones in one pass.
 *
 * Speculative decoding keeps only the projected inputs of accepted draft tokens
 * and replays them onto the committed state on-chip, fused with the verification
 * of the next drafts ("Kimi K3 model structure (7)", section "KDA state
 * rollback").  For sequence n the n_tokens tokens are applied in order to the
 * state read from S_inout[n] and every token writes its output, exactly as
 * kda_recurrent_step; but S_inout[n] is overwritten with the state as it stands
 * after the first n_commit[n] tokens (left untouched when n_commit[n] == 0).
 * The later tokens are drafts: their outputs see the continued state, their
 * updates are dropped.  State traffic is one read and at most one write.
 *
 *   q, k, v, log_alpha, beta, S_inout, o   as for kda_recurrent_step
 *   n_commit     device int32 [n_seqs], caller-owned; values are clamped to
 *                [0, n_tokens] on the device (the host cannot read them)
 *
 * Errors: as kda_recurrent_step, plus KDA_ERR_INVALID_ARGUMENT for a NULL or
 * misaligned n_commit when n_seqs > 0, or for o overlapping n_commit.
 */
kda_status kda_recurrent_verify(const void* q, const void* k, const void* v, const float* log_alpha,
                                const float* beta, float* S_inout, const int32_t* n_commit, int32_t n_seqs,
                                int32_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv, kda_dtype qkv_dtype,
                                float* o, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* kda_status_string(kda_status s);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
