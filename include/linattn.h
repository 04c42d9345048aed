/*
 * linattn.h - C ABI of a gfx950 (MI355X) library for kernelised linear
 * attention over video latent tokens, in its global form and its
 * block-causal (chunk-wise, constant-memory state) form.
 *
 * Sources, cited by page title and section:
 *  [TR] "Nvidia, MIT ve diğerleri video yapay zeka devrimini başlattı"
 *       (aihaber.org), section "Sabit Bellekli KV önbelleğe alma
 *       mekanizması": a video is cut into blocks; later blocks fuse earlier
 *       blocks' features and never the reverse; the computation splits along
 *       token order with identical results; KV1 is cached, KV2 added to give
 *       KV1-2, and after the last block the global KV matrix results; each
 *       block costs only the accumulated KVsum plus its own KV.
 *  [ZH] sd114.wiki article on SANA-Video, section "1. 线性 DiT" (kernel
 *       mapping then global aggregation, no N x N matrix) and section
 *       "2. 块线性注意力 + 恒定内存 KV 缓存" (one accumulated state per chunk,
 *       constant memory, no stored history of keys and values).
 *  [EN] "SANA-Video: Efficient Video Generation with Block Linear Diffusion
 *       Transformer", abstract, designs (1) and (2).
 *
 * What is computed (per batch b and head h; phi(x) = max(x, 0)):
 *   KV  = phi(K)^T V          (d x d, row a = key feature, column c = value feature)
 *   k   = phi(K)^T 1          (d)
 *   S_out = S_in + KV,  z_out = z_in + k
 *   o_i = phi(q_i)^T S_out / (phi(q_i) . z_out + eps)   for every query i of the call
 * The pages do not write the normaliser; the eps-regularised row sum above,
 * and phi = ReLU, are this library's fixed choices.  Inside one call every
 * query sees every key of the call (bidirectional within a block); across
 * calls the state carries only earlier blocks (causal across blocks).
 *
 * Layouts (all contiguous, row-major):
 *   q, k, v : [B][H][L][d] of in_dt      (token-major per head)
 *   out     : [B][H][L][d] of out_dt
 *   state   : [B][H][d*d + d] float32    S[a][c] at a*d + c, then z[a] at d*d + a
 * d is 32, 64 or 128.  in_dt is LA_F32 or LA_BF16; out_dt is LA_F32 or
 * LA_BF16; the state and all accumulation are float32.
 *
 * Ownership: the caller allocates every buffer (device memory) and owns it.
 * The library allocates nothing and keeps no state between calls.  While a
 * forward call runs, the front of `out` serves as scratch for per-split
 * partial KV sums; `out` is completely overwritten with the result before
 * the call's last kernel ends.
 *
 * Streams and errors: every call only enqueues work on `stream` (0 = the
 * null stream) and returns at once.  Arguments are checked before anything
 * is enqueued; a rejected call enqueues nothing and returns:
 *   LA_E_INVAL        null pointer where L > 0, B/H <= 0 or > 65535, L < 0,
 *                     L * d >= 2^31, eps < 0 or not finite, or a tensor of 2^40
 *                     bytes or more (B*H*L*d at 4 bytes an element, or the
 *                     float32 states of every block): beyond any one GPU
 *   LA_E_UNSUPPORTED  d not in {32, 64, 128}, or an unknown dtype code
 *   LA_E_ALIGN        a pointer not 16-byte aligned
 *   LA_E_ALIAS        `out` overlaps an input or a state, or state_out overlaps
 *                     q/k/v/out, or state_out partially overlaps state_in
 *   LA_E_HIP          a kernel launch failed (hipGetLastError after launch)
 *   LA_E_SCRATCH      the allocation-free backward call needs more device
 *                     scratch than its static buffer holds
 * Faults inside kernels surface at the caller's next synchronisation.
 * Calls are thread-safe; calls on different streams may run concurrently
 * as long as their buffers are disjoint.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_OK 0
#define LA_E_INVAL 1
#define LA_E_UNSUPPORTED 2
#define LA_E_ALIGN 3
#define LA_E_ALIAS 4
#define LA_E_HIP 5
#define LA_E_SCRATCH 6

#define LA_F32 0
#define LA_BF16 1

/*
 * la_state_reset - start of a video: S = 0, z = 0 ([TR]: the cache is empty
 * before KV1 is put in it).
 *   state : [B][H][d*d + d] float32, device memory, written.
 * Clears with a fill kernel (no memset node), so it may be graph-captured.
 */
int la_state_reset(float* state, int B, int H, int d, hipStream_t stream);

/*
 * la_chunk_forward - one block of the block-causal form ([TR]: each block
 * reads KVsum plus its own KV; [ZH] section 2: one accumulated state, no
 * key/value history).
 *   q, k, v   : [B][H][L][d] in_dt, read.  The block's tokens.
 *   state_in  : [B][H][d*d+d] float32, read only.  The state after the
 *               previous block (zeros for the first block).
 *   out       : [B][H][L][d] out_dt, written (and used as scratch).
 *   state_out : [B][H][d*d+d] float32, written: state_in + this block's KV.
 *               May be the same pointer as state_in (in-place commit).
 *   eps       : added to every denominator; >= 0 and finite.
 * L = 0 is allowed: state_out = state_in and q/k/v/out may be NULL.
 * Because state_in is never written (unless it is state_out), a diffusion
 * sampler may call this repeatedly against one committed state.
 */
int la_chunk_forward(const void* q, const void* k, const void* v,
                     const float* state_in, void* out, float* state_out,
                     int B, int H, int L, int d, int in_dt, int out_dt,
                     float eps, hipStream_t stream);

/*
 * la_global_forward - global (non-causal) linear attention over N tokens
 * ([ZH] section 1; [EN] design (1)): la_chunk_forward with a zero state_in.
 *   state_out receives the global (S, z) ([TR]: the global KV matrix).
 * N = 0 is allowed: state_out = 0.
 */
int la_global_forward(const void* q, const void* k, const void* v,
                      void* out, float* state_out,
                      int B, int H, int N, int d, int in_dt, int out_dt,
                      float eps, hipStream_t stream);

/*
 * la_blockcausal_forward - a whole sequence in the block-causal form, in one
 * call (the form a block-wise autoregressive model is trained with; [TR]:
 * the video is cut into blocks, block n reads KVsum of blocks 1..n-1 plus
 * its own KV, and the computation splits along token order).  The N tokens
 * of every (b, h) are cut into C = ceil(N / T) blocks of T tokens (the last
 * may be shorter); block n's queries read S_in + KV_1 + ... + KV_n.  The
 * result equals C calls of la_chunk_forward in order with the state carried
 * (up to float32 summation order).
 *   q, k, v   : [B][H][N][d] in_dt, read.
 *   state_in  : [B][H][d*d+d] float32, read; NULL means zeros.  Must not
 *               overlap `states`.
 *   out       : [B][H][N][d] out_dt, written (and used as scratch).
 *   states    : [B][H][C][d*d+d] float32, written: the state after every
 *               block; states[..][C-1] is the state after the sequence.
 *   T         : tokens per block, >= 1 (T >= N: one block, the global form
 *               plus state_in).
 * N = 0 is allowed and does nothing.  Errors as for la_chunk_forward
 * (T <= 0 gives LA_E_INVAL).
 */
int la_blockcausal_forward(const void* q, const void* k, const void* v,
                           const float* state_in, void* out, float* states,
                           int B, int H, int N, int T, int d, int in_dt, int out_dt,
                           float eps, hipStream_t stream);

/*
 * Launch options for the _ex variants (same computation, same rules):
 *   kv_splits     : token splits per (b, h) and block for the KV reduction; 0
 *                   lets the library choose.  A request is clamped to [1,
 *                   the number of 64-token tiles] and to what the scratch in
 *                   `out` holds.
 *                   Results differ between split counts only by float32
 *                   summation order.
 *   readout_workgroups: workgroups of the readout grid; 0 lets the library
 *                   choose.  At d <= 64 with bfloat16 inputs every wave
 *                   sweeps 32-token tiles of all heads, and the request is
 *                   clamped to one wave per tile; at d = 128 with bfloat16
 *                   inputs the request sets the number of work items (whole
 *                   items per (b, h, block)) of a persistent grid; with
 *                   float32 inputs it is rounded to whole workgroups per
 *                   (b, h).  Results do not depend on it.
 *   stage_events  : NULL, or 4 caller-created events recorded on `stream`
 *                   before the KV reduction, before the split reduce (or the
 *                   prefix over blocks), before the readout, and after the
 *                   readout (for timing).
 */
typedef struct la_launch_opts {
  int kv_splits;
  int readout_workgroups;
  hipEvent_t* stage_events;
} la_launch_opts;

int la_chunk_forward_ex(const void* q, const void* k, const void* v,
                        const float* state_in, void* out, float* state_out,
                        int B, int H, int L, int d, int in_dt, int out_dt,
                        float eps, const la_launch_opts* opts, hipStream_t stream);

int la_global_forward_ex(const void* q, const void* k, const void* v,
                         void* out, float* state_out,
                         int B, int H, int N, int d, int in_dt, int out_dt,
                         float eps, const la_launch_opts* opts, hipStream_t stream);

int la_blockcausal_forward_ex(const void* q, const void* k, const void* v,
                              const float* state_in, void* out, float* states,
                              int B, int H, int N, int T, int d, int in_dt, int out_dt,
                              float eps, const la_launch_opts* opts, hipStream_t stream);

/*
 * Rotary position embedding ([ZH] section 1: the Linear DiT adds rotary
 * position encoding for relative positions in space and time; the pages say
 * nothing of where it enters linear attention, so the following is this
 * library's reading).
 *   Positions: token i of a (b, h) sequence (for la_chunk_forward_rope, of
 *   the block) sits at frame frame0 + i / (grid_h * grid_w), row
 *   (i / grid_w) % grid_h and column i % grid_w: the latent frames of the
 *   video, each grid_h x grid_w tokens in row-major order.
 *   Rotation R_i: feature pair m = (2m, 2m + 1) turns by p * theta^(-2j/d_a)
 *   radians, (x, y) -> (x cos - y sin, x sin + y cos), where the first d_t/2
 *   pairs use the frame (p = frame, j = m, d_a = d_t), the next d_h/2 the row
 *   and the last d_w/2 the column; d_h = d_w = 2 * (d / 6) and d_t = d - d_h
 *   - d_w (d = 64: 24, 20, 20).
 *   Placement: the linear-attention form of RoPE (Su et al., "RoFormer",
 *   2021, section 3.4.3), on the numerator only:
 *     S_out = S_in + sum_j R_j phi(k_j) v_j^T,   z_out = z_in + sum_j phi(k_j),
 *     o_i = (R_i phi(q_i))^T S_out / (phi(q_i) . z_out + eps).
 *   The state layout is unchanged; its S holds keys turned by their absolute
 *   positions, so a stream carries it from block to block when every call
 *   passes the absolute frame0 of its first token (whole frames per block).
 *   A state from the plain calls and one from these calls are not
 *   interchangeable.
 * Arguments and rules are those of la_chunk_forward / la_blockcausal_forward
 * plus frame0, grid_h, grid_w and theta (10000 in RoFormer); with T >= N and
 * state_in NULL, la_blockcausal_forward_rope is the global form.  Extra
 * errors (LA_E_INVAL): grid_h or grid_w <= 0, grid_h * grid_w >= 2^22,
 * N >= 2^22 - 64, |frame0| >= 2^22, theta not positive and finite.
 * bfloat16 inputs take sin and cos from the hardware's v_sin_f32 /
 * v_cos_f32 (absolute error near 1e-6 at the angles used); float32 inputs
 * from sincospif.
 */
int la_chunk_forward_rope(const void* q, const void* k, const void* v,
                          const float* state_in, void* out, float* state_out,
                          int B, int H, int L, int d, int in_dt, int out_dt, float eps,
                          int frame0, int grid_h, int grid_w, float theta,
                          hipStream_t stream);

int la_blockcausal_forward_rope(const void* q, const void* k, const void* v,
                                const float* state_in, void* out, float* states,
                                int B, int H, int N, int T, int d, int in_dt, int out_dt,
                                float eps, int frame0, int grid_h, int grid_w, float theta,
                                hipStream_t stream);

int la_blockcausal_forward_rope_ex(const void* q, const void* k, const void* v,
                                   const float* state_in, void* out, float* states,
                                   int B, int H, int N, int T, int d, int in_dt, int out_dt,
                                   float eps, int frame0, int grid_h, int grid_w, float theta,
                                   const la_launch_opts* opts, hipStream_t stream);

/* la_global_forward_rope - the global form with the rotation: as
 * la_global_forward (one block of all N tokens, no state input; state_out
 * receives S with every key turned by its position, and z), token 0 at
 * frame frame0.  Arguments and errors as la_global_forward plus the grid's. */
int la_global_forward_rope(const void* q, const void* k, const void* v, void* out,
                           float* state_out, int B, int H, int N, int d, int in_dt, int out_dt,
                           float eps, int frame0, int grid_h, int grid_w, float theta,
                           hipStream_t stream);

/*
 * Gradients (training uses the same attention: [EN] abstract; [TR] trains
 * with block-causal attention over the blocks of a video).  For a loss L,
 * given dO = dL/dO and optionally dL/dS_n, dL/dz_n for the state after every
 * block, the backward calls return dL/dQ, dL/dK, dL/dV and optionally the
 * gradient of the state before the first block.  They are the chain rule of
 * the forward above (den_i = phi(q_i) . z_n + eps, S_n the state block n's
 * queries read):
 *   dq_i = (S_n do_i - (t_i / den_i) z_n) / den_i * [q_i > 0],
 *          t_i = phi(q_i) . (S_n do_i)
 *   R_m  = sum over blocks n >= m of ( sum_{i in n} phi(q_i) do_i^T / den_i + dL/dS_n )
 *   r_m  = sum over blocks n >= m of ( -sum_{i in n} t_i / den_i^2 phi(q_i) + dL/dz_n )
 *   dk_j = (R_m v_j + r_m) * [k_j > 0],   dv_j = R_m^T phi(k_j)   (j in block m)
 *   dS_in = R_1, dz_in = r_1
 * with [x > 0] the derivative of max(x, 0), taken as 0 at 0.
 *
 * Common arguments:
 *   q, k, v    : the forward's inputs, [B][H][N][d] in_dt, read.
 *   dout       : dL/dO, [B][H][N][d] grad_dt, read.
 *   dq, dk, dv : [B][H][N][d] grad_dt, written.
 *   grad_dt    : LA_F32 or LA_BF16, the type of dout and of dq, dk, dv.
 *   workspace  : device memory of at least la_backward_workspace_size() bytes
 *                (caller-owned, contents need not be initialised, clobbered).
 * Outputs (dq, dk, dv, dstate_in, workspace) must not overlap each other or
 * any input (LA_E_ALIAS); inputs may overlap each other.  A workspace that is
 * NULL or too small gives LA_E_INVAL.  Other errors as for the forward calls.
 * Results are bitwise reproducible run to run.
 *
 * Streams.  A call with bfloat16 inputs and at least 2^20 token-heads (B H N)
 * whose key-gradient kernel works on items (d = 128, and the rotary calls at
 * every d; at d <= 64 the plain calls take the key-gradient sweep, which
 * fills the GPU by itself) runs the two halves of its (b, h) pairs at once:
 * the first on `stream`, the
 * second on a stream the library creates on the device at the first such call
 * (default priority, held until the process ends).  The call forks that
 * stream from `stream` and joins it back, so everything it does is ordered on
 * `stream` as for any other call.  Calls from several host threads share the
 * second stream (their halves run there one after another).  Under stream
 * capture, with stage events (la_launch_opts), in the allocation-free entry
 * point, or if the second stream cannot be created, a call runs on `stream`
 * alone.  The results are bitwise the same either way, and the workspace
 * size does not change.
 */

/* Bytes of workspace a backward call with these arguments needs (T as for
 * la_blockcausal_backward; L or N for the chunk and global calls). */
int la_backward_workspace_size(int B, int H, int N, int T, int d, int in_dt, size_t* bytes);

/* Streams (1 or 2, in *count) a backward call with these arguments runs its
 * kernels on when it may use two (see "Streams" above); rotary != 0 asks for
 * la_blockcausal_backward_rope.  Errors as for la_backward_workspace_size. */
int la_backward_stream_count(int B, int H, int N, int T, int d, int in_dt, int rotary,
                             int* count);

/*
 * la_backward_plan - the launch shape a backward call with these arguments
 * would use on one stream, with no device work (the two halves of a
 * two-stream call keep its query splits).  query_splits_request and
 * key_workgroups_request are the kv_splits and readout_workgroups fields of
 * la_launch_opts in the _ex calls (0: the library's choice); workspace_bytes
 * is the size of the workspace the call is given (0: as much as it needs,
 * la_backward_workspace_size); rotary != 0 asks for the RoPE'd backward.
 * Errors as for la_backward_workspace_size, plus LA_E_INVAL for a negative
 * request, a workspace too small for any plan (as the call itself), or, with
 * rotary != 0, a sequence the rotary calls refuse (N >= 2^22 - 64).
 */
typedef struct la_backward_shape {
  int blocks;           /* blocks of T tokens (0 when N = 0) */
  int query_splits;     /* query-gradient items per (b, h, block); above 1, each
                           writes a partial state gradient to the workspace */
  int query_workgroups; /* the query-gradient kernel's workgroups */
  int key_items;        /* key-gradient items per (b, h, block); 0 with the sweep */
  int key_workgroups;   /* the key-gradient kernel's workgroups */
  int key_sweep_units;  /* the key-gradient sweep's 128-token units per block
                           (bf16 inputs at d <= 64 without rotary or a key
                           request); 0 when the key gradients take work items */
} la_backward_shape;

int la_backward_plan(int B, int H, int N, int T, int d, int in_dt, int rotary,
                     int query_splits_request, int key_workgroups_request,
                     size_t workspace_bytes, la_backward_shape* shape);

/*
 * la_blockcausal_backward - gradients of la_blockcausal_forward.
 *   states    : [B][H][C][d*d+d] float32, read: the forward's `states`.
 *   dstates   : [B][H][C][d*d+d] float32, read, or NULL (zero): dL/dS_n, dL/dz_n.
 *   dstate_in : [B][H][d*d+d] float32, written (NULL: not wanted): the gradient
 *               of the forward's state_in (R_1, r_1).
 * N = 0 writes zeros to dstate_in (if given) and nothing else.
 */
int la_blockcausal_backward(const void* q, const void* k, const void* v, const float* states,
                            const void* dout, const float* dstates, void* dq, void* dk, void* dv,
                            float* dstate_in, int B, int H, int N, int T, int d, int in_dt,
                            int grad_dt, float eps, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* As above, with launch options: kv_splits = workgroups per block of the
 * query-gradient kernel (clamped as the forward's, and to the workspace),
 * readout_workgroups = workgroups of the key-gradient kernel, stage_events =
 * 4 events around its three kernels. */
int la_blockcausal_backward_ex(const void* q, const void* k, const void* v, const float* states,
                               const void* dout, const float* dstates, void* dq, void* dk,
                               void* dv, float* dstate_in, int B, int H, int N, int T, int d,
                               int in_dt, int grad_dt, float eps, void* workspace,
                               size_t workspace_bytes, const la_launch_opts* opts,
                               hipStream_t stream);

/*
 * la_blockcausal_backward_noalloc - la_blockcausal_backward for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and results.  Its workspace is a static device
 * array of LA_NOALLOC_SCRATCH_BYTES (32 MiB) in the library's code object,
 * one per GPU, held until the process ends; the call allocates nothing and
 * fits the query-gradient split count to that size.  A call whose smallest
 * plan needs more (the suffix states alone, B*H*ceil(N/T)*(d*d+d)*4 bytes,
 * exceed it) returns LA_E_SCRATCH and enqueues nothing.  The array keeps the
 * last call's contents; every byte a call reads from it, that call wrote
 * first.  All calls on one GPU share the array: two such calls that overlap
 * in time on one GPU (concurrent streams, or threads) race and give wrong
 * results; serialise them.  Other arguments, rules and errors as
 * la_blockcausal_backward.
 */
#define LA_NOALLOC_SCRATCH_BYTES (32u << 20)
int la_blockcausal_backward_noalloc(const void* q, const void* k, const void* v,
                                    const float* states, const void* dout, const float* dstates,
                                    void* dq, void* dk, void* dv, float* dstate_in, int B, int H,
                                    int N, int T, int d, int in_dt, int grad_dt, float eps,
                                    hipStream_t stream);

/*
 * la_chunk_backward - gradients of one la_chunk_forward call.
 *   state_out  : the forward's state_out (the state the queries read), read.
 *   dstate_out : dL/d state_out, [B][H][d*d+d] float32, read, or NULL (zero).
 *   dstate_in  : dL/d state_in, written, or NULL.
 * L = 0: dstate_in = dstate_out (or zeros); q, k, v, dout, dq, dk, dv may be NULL.
 */
int la_chunk_backward(const void* q, const void* k, const void* v, const float* state_out,
                      const void* dout, const float* dstate_out, void* dq, void* dk, void* dv,
                      float* dstate_in, int B, int H, int L, int d, int in_dt, int grad_dt,
                      float eps, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * la_global_backward - gradients of la_global_forward (no state gradient).
 *   state : the forward's state_out (the global S, z), read.
 */
int la_global_backward(const void* q, const void* k, const void* v, const float* state,
                       const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                       int in_dt, int grad_dt, float eps, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * la_blockcausal_backward_rope - gradients of la_blockcausal_forward_rope
 * (training with the rotary form; the chain rule of the forward stated with
 * la_chunk_forward_rope, q~ = R phi(q), k~ = R phi(k), R^T the turn by the
 * opposite angles):
 *   u_i  = R_i^T (S_n do_i),  t_i = phi(q_i) . u_i
 *   dq_i = (u_i - (t_i / den_i) z_n) / den_i * [q_i > 0]
 *   G_m  = sum over blocks n >= m of ( sum_{i in n} q~_i do_i^T / den_i + dL/dS_n )
 *   g_m  = sum over blocks n >= m of ( -sum_{i in n} t_i / den_i^2 phi(q_i) + dL/dz_n )
 *   dk_j = (R_j^T (G_m v_j) + g_m) * [k_j > 0],   dv_j = G_m^T k~_j
 *   dS_in = G_1, dz_in = g_1
 * Arguments and rules as la_blockcausal_backward (the same workspace size,
 * la_backward_workspace_size) plus frame0, grid_h, grid_w, theta and their
 * checks as la_chunk_forward_rope; `states` is what the rotary forward
 * returned.
 */
int la_blockcausal_backward_rope(const void* q, const void* k, const void* v,
                                 const float* states, const void* dout, const float* dstates,
                                 void* dq, void* dk, void* dv, float* dstate_in, int B, int H,
                                 int N, int T, int d, int in_dt, int grad_dt, float eps,
                                 void* workspace, size_t workspace_bytes, int frame0, int grid_h,
                                 int grid_w, float theta, hipStream_t stream);

/* As la_blockcausal_backward_rope, with launch options as
 * la_blockcausal_backward_ex. */
int la_blockcausal_backward_rope_ex(const void* q, const void* k, const void* v,
                                    const float* states, const void* dout, const float* dstates,
                                    void* dq, void* dk, void* dv, float* dstate_in, int B, int H,
                                    int N, int T, int d, int in_dt, int grad_dt, float eps,
                                    void* workspace, size_t workspace_bytes, int frame0,
                                    int grid_h, int grid_w, float theta,
                                    const la_launch_opts* opts, hipStream_t stream);

/*
 * la_chunk_backward_rope - gradients of one la_chunk_forward_rope call, as
 * la_chunk_backward is of la_chunk_forward: state_out (the state the
 * queries read, keys rotated by absolute position) read, dstate_out read or
 * NULL (zero), dstate_in written or NULL; frame0, grid_h, grid_w and theta
 * as the forward call took them.  L = 0: dstate_in = dstate_out (or zeros).
 */
int la_chunk_backward_rope(const void* q, const void* k, const void* v, const float* state_out,
                           const void* dout, const float* dstate_out, void* dq, void* dk,
                           void* dv, float* dstate_in, int B, int H, int L, int d, int in_dt,
                           int grad_dt, float eps, void* workspace, size_t workspace_bytes,
                           int frame0, int grid_h, int grid_w, float theta, hipStream_t stream);

/* la_global_backward_rope - gradients of la_global_forward_rope, as
 * la_global_backward is of la_global_forward (state: the forward's
 * state_out; no state gradient). */
int la_global_backward_rope(const void* q, const void* k, const void* v, const float* state,
                            const void* dout, void* dq, void* dk, void* dv, int B, int H, int N,
                            int d, int in_dt, int grad_dt, float eps, void* workspace,
                            size_t workspace_bytes, int frame0, int grid_h, int grid_w,
                            float theta, hipStream_t stream);

/*
 * Temporal convolution of the Spatial-Temporal Mix-FFN with its
 * chunk-boundary cache ([TR] section "Verimli doğrusal DiT": the MLP
 * alternates 1x3x3 spatial and 3x1x1 temporal convolutions; [ZH] section 1:
 * a temporal convolution module).  The pages do not give its streaming
 * treatment; this library's reading: the 3x1x1 convolution is depthwise
 * (one 3-tap filter per channel along latent frames), and it follows the
 * block-causal attention's visibility rule ([TR]: a block reads earlier
 * blocks, never later ones), so per batch b, frame f, position p, channel c:
 *   y[f] = w[c][0] x[f-1] + w[c][1] x[f] + w[c][2] x[f+1] + bias[c]
 * with x[f+1] = 0 when frame f+1 is in a later chunk or past the end, and
 * x[-1] = the cache (the previous chunk's last frame; NULL = zeros, the start
 * of a video).  A stream therefore carries one frame, constant in memory.
 *   x, y      : [B][F][P][C] (frames, positions per frame, channels),
 *               x_dt / y_dt each LA_F32 or LA_BF16; C a multiple of 8.
 *   cache_in  : [B][P][C] x_dt, read; NULL = zeros.
 *   weight    : [C][3] float32 (taps for f-1, f, f+1); bias: [C] float32 or NULL.
 *   cache_out : [B][P][C] x_dt, written with the last frame (NULL: not
 *               wanted); F = 0 copies cache_in (or zeros) into it.
 * Errors: LA_E_INVAL (B, P, C <= 0, F < 0, Tf <= 0, a needed pointer NULL,
 * more than 65535 chunks, B*F*P*C*4 >= 2^40), LA_E_UNSUPPORTED (C not a multiple of 8, dtype),
 * LA_E_ALIGN, LA_E_ALIAS (y overlapping anything else; cache_out overlapping
 * x, weight, bias, or cache_in unless it is cache_in itself and the call has
 * one chunk).
 */

/* One chunk of F frames.  cache_out may be cache_in (in-place update). */
int la_temporal_conv_chunk(const void* x, const void* cache_in, const float* weight,
                           const float* bias, void* y, void* cache_out, int B, int F, int P, int C,
                           int x_dt, int y_dt, hipStream_t stream);

/* A whole sequence of F frames in chunks of Tf frames (the training form):
 * equals la_temporal_conv_chunk over the chunks in order with the cache
 * carried.  With more than one chunk, cache_out must not overlap cache_in. */
int la_temporal_conv_blockcausal(const void* x, const void* cache_in, const float* weight,
                                 const float* bias, void* y, void* cache_out, int B, int F, int Tf,
                                 int P, int C, int x_dt, int y_dt, hipStream_t stream);

/*
 * la_plan - the launch shape a forward call with these arguments (and the
 * given kv_splits / readout_workgroups requests, 0 = library's choice) would
 * use, with no device work: *kv_splits receives the split count (1 = the KV
 * kernel writes state_out directly and the split reduce is skipped),
 * *readout_workgroups the readout grid size.  Returns a status code.
 */
int la_plan(int B, int H, int L, int d, int in_dt, int out_dt, int kv_splits_request,
            int readout_workgroups_request, int* kv_splits, int* readout_workgroups);

/* Static text for a status code. */
const char* la_status_string(int status);

/* ABI version of this header (increases whenever a call is added or a call's
 * arguments or behaviour change). */
int la_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
