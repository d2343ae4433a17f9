/*
 * ssd.h - C ABI of the MI355X (gfx950) Mamba-2 SSD layer core.
 *
 * The operation is the multi-head selective state-space transform with a
 * scalar-times-identity transition per head:
 *
 *     a_t = exp(dt_t * A_h)
 *     h_t = a_t * h_{t-1} + (dt_t * x_t) B_t^T          (state: headdim x dstate per head)
 *     y_t = h_t C_t + D_h * x_t
 *
 * (the recurrence of the "Mamba-2" wiki note, section "Question"; the
 * discretised decay of "Mamba-2: State Space Models and Linear-Time
 * Sequence Modeling Without Attention", section "State Space Models: The
 * Core Abstraction", where the continuous system also carries the D x
 * term; the dt-scaled input of that page's multi-head block, section
 * "Architecture: Multi-Head SSM"; one decay scalar per head, "Transformers
 * are SSMs" paper card, section "How It Works").  B and C are shared by the
 * heads of a group: head h reads group h / (nheads / ngroups).
 *
 * Two modes compute it ("Mamba-2" wiki note, section "Algorithmic Lesson";
 * mohakchugh blog, section "Why This Matters for Hardware"):
 *   ssd_forward - the chunked (dual) mode over a whole sequence: quadratic,
 *                 matmul-shaped work inside chunks of chunk_size tokens and
 *                 the recurrent state passed between chunks (mohakchugh blog,
 *                 section "Block Decomposition"; ql.gl, "The Core of SSD").
 *                 It runs the four stage kernels below in order.
 *   ssd_step    - the recurrent mode: one token per call, O(1) in the
 *                 sequence length (crackai.dev paper card, "Why It Matters").
 *
 * For comparison the library also runs the layer SSD replaces, the Mamba-1
 * selective scan with a diagonal transition per channel
 * (ssd_selective_scan, at the end of this header).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers (current HIP device) to dense,
 *     row-major arrays in the layouts given per call.  The caller owns every
 *     buffer, including the workspace; the library allocates nothing, keeps
 *     no mutable global state and is safe to call from several threads
 *     (except ssd_forward_noalloc, whose static scratch is shared: see there).
 *   - "T" is the storage type of x, B, C, y and of the chunk-entry states:
 *     dtype SSD_F32 (float) or SSD_BF16 (bfloat16, 2 bytes).  dt, A, D,
 *     initial/final/step states and the fp32 workspace arrays are float.
 *     Arithmetic accumulates in fp32; bf16 operands of the matrix-core
 *     products are rounded to nearest even.
 *   - dt must already be positive (softplus applied by the caller) and A
 *     negative (or zero); neither is clamped.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without synchronising.  SSD_OK means
 *     "enqueued"; completion is the stream's business.
 *   - Arguments are validated on the host before anything is enqueued: an
 *     error status means no device memory was read or written.  A launch
 *     failure reported by the runtime returns SSD_ERR_HIP.  No C++
 *     exception crosses this interface.
 *   - Shape limits: 0 <= batch <= 65535; seqlen >= 0; 1 <= nheads <= 65535
 *     with nheads * headdim <= 2^20; headdim in {16, 32, 64, 128}; dstate a
 *     multiple of 16 in [16, 256]; ngroups >= 1 dividing nheads, with
 *     ngroups * dstate <= 2^20; chunk_size
 *     a multiple of 16 in [16, 256].  seqlen need not be a multiple of
 *     chunk_size: the last chunk is then shorter.
 *   - Outputs must not overlap inputs (the step state is the one in/out
 *     argument); overlap is reported as SSD_ERR_ALIAS.
 *   - Non-finite inputs: in the recurrence a NaN or Inf in x at token t of
 *     head h reaches y only from token t on (in that head and head-dimension
 *     column).  The chunked forwards reach it from the first token of t's
 *     32-token block within its chunk (the block's masked scores are zero
 *     and zero times NaN is NaN on the matrix cores), up to 31 tokens
 *     earlier, still only in that column of that head.  Non-finite dt, B or
 *     C values reach y from their own token on.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,      /* a required pointer is NULL */
    SSD_ERR_SHAPE = -2,     /* a size is out of the supported range */
    SSD_ERR_DTYPE = -3,     /* dtype is not SSD_F32 or SSD_BF16 */
    SSD_ERR_WORKSPACE = -4, /* workspace smaller than ssd_forward_workspace_bytes */
    SSD_ERR_HIP = -5,       /* the HIP runtime reported an error at launch */
    SSD_ERR_ALIAS = -6,     /* an output overlaps an input */
    SSD_ERR_SCRATCH = -7    /* ssd_forward_noalloc: one batch row needs more than the static scratch */
} ssd_status;

/* Human-readable text of a status code (static storage; never NULL). */
const char* ssd_status_string(int status);

/* Version of this interface: 100 * major + minor. */
int ssd_abi_version(void);

/* Number of chunks ceil(seqlen / chunk_size) (0 for seqlen 0); -1 on bad sizes. */
int64_t ssd_num_chunks(int64_t seqlen, int64_t chunk_size);

/* ---------------------------------------------------------------------------------------------
 * Chunked (dual) mode.
 * ------------------------------------------------------------------------------------------- */

/* Bytes of device workspace ssd_forward needs for these sizes: at least 256
 * for valid sizes, 0 when the sizes or dtype are invalid.
 * Layout (each part 256-byte aligned, nc = number of chunks):
 *   dA_cs      float (batch, nheads, nc, chunk_size)
 *   dt_chunked float (batch, nheads, nc, chunk_size)
 *   chunk_states float (batch, nc, nheads, headdim, dstate)
 *   entry_states T   (batch, nc, nheads, headdim, dstate)          */
size_t ssd_forward_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                   int64_t dstate, int64_t chunk_size, int dtype);

/* y, final_states = SSD(x, dt, A, B, C, D, init_states) in chunks of chunk_size.
 *   x            T     (batch, seqlen, nheads, headdim)
 *   dt           float (batch, seqlen, nheads)
 *   A, D         float (nheads)
 *   B, C         T     (batch, seqlen, ngroups, dstate)
 *   init_states  float (batch, nheads, headdim, dstate), the state before
 *                token 0 (h_{-1}); NULL means zeros
 *   y            T     (batch, seqlen, nheads, headdim), written
 *   final_states float (batch, nheads, headdim, dstate), written: the state
 *                after the last token (equal to init_states when seqlen = 0)
 *   workspace    device buffer of at least ssd_forward_workspace_bytes()
 * Runs ssd_dA_cumsum, ssd_chunk_state, ssd_state_passing, ssd_chunk_scan. */
int ssd_forward(const void* x, const float* dt, const float* A, const void* B, const void* C,
                const float* D, const float* init_states, void* y, float* final_states,
                int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                int64_t ngroups, int64_t chunk_size, int dtype, void* workspace,
                size_t workspace_bytes, void* stream);

/* ssd_forward for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments, results and errors, with no
 * workspace argument.  The workspace is a static scratch array in the library's device code
 * (ssd_forward_noalloc_scratch_bytes() = 64 MiB), one copy per GPU, held from the library's load
 * until the process ends; the call allocates nothing.  Batch rows are independent, so the forward
 * runs on slices of batch rows whose workspace (ssd_forward_workspace_bytes of the slice) fits the
 * scratch, one slice after another on `stream`; the results equal ssd_forward's bit for bit.
 * Returns SSD_ERR_SCRATCH, before any device work, when one batch row's workspace exceeds the
 * scratch (for example 65536 tokens x 80 heads of 64 x 256 states).  Every call on a GPU shares
 * that GPU's scratch: calls that overlap in time on one GPU (on different streams, or from
 * different threads without ordering) race and give wrong results.  Nothing in the scratch needs
 * to start at zero: every byte a call reads was written by the same call. */
size_t ssd_forward_noalloc_scratch_bytes(void);
int ssd_forward_noalloc(const void* x, const float* dt, const float* A, const void* B, const void* C,
                        const float* D, const float* init_states, void* y, float* final_states, int64_t batch,
                        int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                        int64_t chunk_size, int dtype, void* stream);

/* Gradients of ssd_forward (the training pass) for dL/dy = dy and dL/d(final_states) = dfinal
 * (NULL = 0), by the adjoint of the recurrence: the adjoint state runs backwards in time as an SSD
 * of its own (dy as input, C in the role of B), computed with the same stage kernels on
 * time-reversed and role-swapped arrays; the log-decay gradient is the suffix sum over tokens of
 * dy.(y - D x) - (dt x).(dL/d(dt x)), summed within each chunk from its end (bf16 inputs: the mean
 * of the sums from both ends), where the gradient is the inner product of the adjoint and forward
 * states at the chunk boundary (so rounding does not accumulate across chunks).  Arguments as for
 * ssd_forward, plus
 *   dy T (batch, seqlen, nheads, headdim); dfinal float (batch, nheads, headdim, dstate) or NULL
 *   dx T like x; ddt float like dt; dA, dD float (nheads); dB, dC T like B, C;
 *   dinit float (batch, nheads, headdim, dstate): the gradient of the initial state (written
 *     also when init_states is NULL)
 *   workspace of at least ssd_backward_workspace_bytes() bytes
 * dstate must be one of 16, 32, 64, 128, 256 and nheads * dstate <= 2^20.  The decay gradients
 * cancel too much for bf16 operands: fp32 inputs take the fp32 matrix cores for the recompute, the
 * adjoint states and the readouts; with bf16 inputs each fp32 operand there is carried as a pair of
 * bf16 values (hi + lo, the fp32 value to 2^-18) and multiplied on the bf16 matrix cores with fp32
 * sums; dx, dB, dC are rounded to bf16 once. */
size_t ssd_backward_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                                    int64_t ngroups, int64_t chunk_size, int dtype);
int ssd_backward(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                 const float* init_states, const void* dy, const float* dfinal, void* dx, float* ddt, float* dA,
                 void* dB, void* dC, float* dD, float* dinit, int64_t batch, int64_t seqlen, int64_t nheads,
                 int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk_size, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

/* The same forward as one pass over the sequence per (batch, head), the state kept on chip (the
 * chunk-ordered walk of the mohakchugh blog's block-decomposition outline, section "Block
 * Decomposition: The Hardware-Aware Algorithm"): a workgroup per (batch, head, slice of the head dimension) steps through the tokens
 * in blocks of 32, so no chunk size and no workspace.  Arguments, layouts, results and errors as for ssd_forward (y and
 * final_states to the same tolerance; the sums run in another order), plus SSD_ERR_SHAPE when
 * headdim x (dstate rounded up to 32, 64, 128 or 256) exceeds 16384 (headdim 128 with dstate > 128).
 * The sequential walk leaves little parallelism on a large GPU: ssd_forward is the fast path. */
int ssd_forward_fused(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                      const float* init_states, void* y, float* final_states, int64_t batch, int64_t seqlen,
                      int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups, int dtype, void* stream);

/* Packed variable-length batch: nseq sequences stored back to back on one token axis of
 * total_tokens tokens, sequence k being tokens cu_seqlens[k] .. cu_seqlens[k+1]-1 (the padding-free
 * variable-length batches of the ql.gl page, section "Mamba-2 Changes More Than the Algorithm").
 * Every sequence starts from a zero state: the recurrence is reset at each sequence start, so y
 * equals running ssd_forward on every sequence alone.  Chunks of chunk_size tokens are laid over the
 * packed axis (a chunk may hold parts of several sequences).
 *   x T (total_tokens, nheads, headdim); dt float (total_tokens, nheads); A, D float (nheads)
 *   B, C T (total_tokens, ngroups, dstate)
 *   cu_seqlens int32 (nseq + 1), DEVICE memory, non-decreasing from 0 to total_tokens (empty
 *     sequences allowed).  Its content is not checked on the host; other content yields
 *     unspecified values but no access outside the buffers.
 *   y T (total_tokens, nheads, headdim), written
 *   final_states float (nseq, nheads, headdim, dstate), written: each sequence's state after its
 *     last token (zeros for an empty sequence)
 *   workspace of at least ssd_forward_varlen_workspace_bytes() bytes:
 *     dA_cs, dt_chunked float (nheads, nc, chunk_size); chunk states float (nc, nheads, headdim,
 *     dstate); entry states T (same shape); int32 per-token sequence starts (total_tokens) and
 *     int32 x 4 per-chunk boundary records (nc)
 * Limits as for ssd_forward with batch 1; 0 <= nseq <= 2^24 (nseq 0 only with no tokens). */
size_t ssd_forward_varlen_workspace_bytes(int64_t total_tokens, int64_t nheads, int64_t headdim, int64_t dstate,
                                          int64_t chunk_size, int dtype);
int ssd_forward_varlen(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                       const int32_t* cu_seqlens, int64_t nseq, void* y, float* final_states, int64_t total_tokens,
                       int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk_size, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Stage 1 (segment decays).  For every chunk c and position l inside it:
 *   dA_cs[b,h,c,l]      = sum_{j = cQ .. cQ+l} dt[b,j,h] * A[h]
 *   dt_chunked[b,h,c,l] = dt[b, cQ+l, h]
 * so that exp(dA_cs[l] - dA_cs[s]) is the decay product prod_{j=s+1..l} a_j
 * of the matrix-mixer entries ("Mamba-2" wiki note, "Matrix Mixer View").
 * Positions past seqlen in a short last chunk get dt 0 (the sum stays flat).
 *   dt float (batch, seqlen, nheads); A float (nheads)
 *   dA_cs, dt_chunked float (batch, nheads, nc, chunk_size), written */
int ssd_dA_cumsum(const float* dt, const float* A, float* dA_cs, float* dt_chunked, int64_t batch,
                  int64_t seqlen, int64_t nheads, int64_t chunk_size, void* stream);

/* Stage 2 (chunk states).  The state each chunk reaches from a zero state,
 * the rank-dstate factor of the off-diagonal blocks of the mixing matrix
 * ("Mamba-2" wiki note, "Structured Semiseparable Matrices"):
 *   chunk_states[b,c,h,p,n] = sum_l x[b,cQ+l,h,p] * dt_l * exp(dA_cs[Q-1] - dA_cs[l]) * B[b,cQ+l,g(h),n]
 *   x T (batch, seqlen, nheads, headdim); B T (batch, seqlen, ngroups, dstate)
 *   dt_chunked, dA_cs float (batch, nheads, nc, chunk_size) as written by stage 1
 *   chunk_states float (batch, nc, nheads, headdim, dstate), written */
int ssd_chunk_state(const void* x, const void* B, const float* dt_chunked, const float* dA_cs,
                    float* chunk_states, int64_t batch, int64_t seqlen, int64_t nheads,
                    int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk_size, int dtype,
                    void* stream);

/* Stage 3 (state passing).  The recurrence between chunks (ql.gl, "The Core
 * of SSD"; mohakchugh blog, "Block Decomposition"), sequential over chunks:
 *   S = init (or 0); for c: entry_states[b,c] = S; S = exp(dA_cs[b,h,c,Q-1]) * S + chunk_states[b,c]
 *   final_states = S
 *   chunk_states float (batch, nc, nheads, headdim, dstate); dA_cs float (batch, nheads, nc, chunk_size)
 *   init_states float (batch, nheads, headdim, dstate) or NULL (zeros)
 *   entry_states T (batch, nc, nheads, headdim, dstate), written (rounded to T)
 *   final_states float (batch, nheads, headdim, dstate), written */
int ssd_state_passing(const float* chunk_states, const float* dA_cs, const float* init_states,
                      void* entry_states, float* final_states, int64_t batch, int64_t seqlen,
                      int64_t nheads, int64_t headdim, int64_t dstate, int64_t chunk_size,
                      int dtype, void* stream);

/* Stage 4 (chunk scan).  The output of every chunk: the masked quadratic
 * (attention-like) form inside the chunk plus the entering state read out
 * by C, plus the skip term (mohakchugh blog, "Block Decomposition" and "The
 * Tensor Core Connection"):
 *   y[l,p] = sum_{s<=l} (C_l . B_s) exp(dA_cs[l] - dA_cs[s]) dt_s x[s,p]
 *          + exp(dA_cs[l]) * sum_n C_l[n] entry_states[c,p,n] + D[h] x[l,p]
 *   x, y T (batch, seqlen, nheads, headdim); B, C T (batch, seqlen, ngroups, dstate)
 *   dt_chunked, dA_cs float (batch, nheads, nc, chunk_size); entry_states T (batch, nc, nheads, headdim, dstate)
 *   D float (nheads) */
int ssd_chunk_scan(const void* x, const void* B, const void* C, const float* dt_chunked,
                   const float* dA_cs, const void* entry_states, const float* D, void* y,
                   int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                   int64_t ngroups, int64_t chunk_size, int dtype, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Recurrent mode.
 * ------------------------------------------------------------------------------------------- */

/* One token: a = exp(dt*A); state = a*state + (dt*x) B^T; y = state C + D x.
 *   state float (batch, nheads, headdim, dstate), read and written IN PLACE
 *   x T (batch, nheads, headdim); dt float (batch, nheads); A, D float (nheads)
 *   B, C T (batch, ngroups, dstate); y T (batch, nheads, headdim), written */
int ssd_step(float* state, const void* x, const float* dt, const float* A, const void* B,
             const void* C, const float* D, void* y, int64_t batch, int64_t nheads,
             int64_t headdim, int64_t dstate, int64_t ngroups, int dtype, void* stream);

/* ---------------------------------------------------------------------------------------------
 * The Mamba-1 selective scan (mohakchugh blog, section "Mamba-1: Selective State Spaces"): each
 * channel d of the input has its own diagonal transition, one decay per state entry, and B, C
 * are per token, shared by all channels:
 *
 *     h_t[d, n] = exp(delta_t[d] A[d, n]) h_{t-1}[d, n] + (delta_t[d] x_t[d]) B_t[n]
 *     y_t[d]    = sum_n C_t[n] h_t[d, n] + D[d] x_t[d]
 *
 * The input enters as delta * B * x, as in ssd_forward.  It runs as a sequential scan on the
 * vector units (one kernel); there is no workspace.
 *   x T (batch, seqlen, dim); delta float (batch, seqlen, dim), positive
 *   A float (dim, dstate), negative or zero; D float (dim)
 *   B, C T (batch, seqlen, dstate)
 *   init_states float (batch, dim, dstate) or NULL (zeros)
 *   y T (batch, seqlen, dim), written; final_states float (batch, dim, dstate), written
 * Shape limits: 0 <= batch <= 65535; 0 <= seqlen < 2^31; dim a multiple of 8 in [8, 2^20];
 * dstate in {4, 8, 16, 32, 64}.  x, delta and y must be 16-byte aligned; with seqlen 0 the
 * token arrays (x, delta, B, C, y) may be NULL and final_states receives the initial state.  Errors as above
 * (SSD_ERR_SHAPE for a bad size or alignment, SSD_ERR_ALIAS when an output overlaps an input
 * or the other output). */
int ssd_selective_scan(const void* x, const float* delta, const float* A, const void* B, const void* C,
                       const float* D, const float* init_states, void* y, float* final_states, int64_t batch,
                       int64_t seqlen, int64_t dim, int64_t dstate, int dtype, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSD_MI355X_H */
