/*
 * gdn.h — C ABI of the MI355X (gfx950) gated-delta-rule library (libgdn.so).
 *
 * The operation.  Per (batch b, head h) the library carries an fp32 state
 * S in R^{dv x dk} (row i = value index, column j = key index) through the
 * gated delta rule
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 *
 * i.e. per token: decay the state by alpha_t, read r = S k_t, form the
 * delta-rule error u = beta_t (v_t - r), add u k_t^T, and read o_t from the
 * updated state.  Sources (web pages, by title and section):
 *   [P1] "Gated DeltaNet GPU并行实现：拆解线性注意力循环的两种高效方案"
 *        §2.1 the delta rule S_t = S_{t-1} - beta_t (S_{t-1} k_t - v_t) k_t^T and
 *        its affine-map form; §2.2 a scalar forgetting gate multiplying the old
 *        state; §3.2-§3.3 the chunked evaluation (matmuls inside a chunk, the
 *        state carried serially from chunk to chunk, one workgroup carrying all
 *        chunks of a sequence); §4.1 inputs in (batch, head, seq_len, d) with d
 *        contiguous; §4.4 state kept in fp32 while matmul inputs are bf16 with
 *        fp32 accumulation; §5.2 (second pitfall) non-contiguous or misaligned
 *        inputs must not be taken silently.
 *   [P3] "线性注意力机制与Gated DeltaNet的优化实践" §2.1 the output of token i
 *        includes token i (o_t is read after the update); §3.1 a single-step
 *        in-place state update kernel on global fp32 memory (the decode step
 *        below adds the erase term and the output).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises.  Work is enqueued on
 *     `hip_stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns once it is enqueued.  The library holds no state between calls
 *     (except the per-GPU scratch of gdn_chunk_fwd_split_noalloc, below) and
 *     is safe to call from several host threads on different streams.
 *   - Layouts are dense row-major exactly as written (no strides).  Every
 *     tensor pointer must be 16-byte aligned.
 *   - Arguments are validated before anything is launched; on any error no
 *     device work is enqueued and the call returns a nonzero code.  Faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - Values are not inspected: NaN/Inf propagate.  There is no 1/sqrt(d)
 *     query scaling and no normalisation of q or k inside the library.
 *   - Size limits: the number of sequences (B*H, or N*H for the decode step)
 *     and T are each at most 2^31 - 1, and B*H*T at most 2^48; larger sizes
 *     return GDN_ERR_UNSUPPORTED (the workspace queries return 0).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define GDN_OK 0
#define GDN_ERR_INVALID_ARG 1 /* NULL pointer, negative size, aliasing, bad dtype */
#define GDN_ERR_UNSUPPORTED 2 /* shape/chunk size the library does not handle     */
#define GDN_ERR_ALIGNMENT 3   /* a tensor pointer is not 16-byte aligned           */
#define GDN_ERR_HIP 4         /* the HIP runtime reported an error on launch       */

/* Element type of q, k, v and o.  alpha, beta and every state are fp32. */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/*
 * gdn_chunk_fwd — chunked forward pass over T tokens for B*H independent
 * sequences ([P1] §3.2-§3.3).
 *
 *   q, k           [B,H,T,dk]  dtype   queries and keys, d contiguous
 *   v              [B,H,T,dv]  dtype   values
 *   alpha          [B,H,T]     fp32    forgetting gate in [0,1]
 *   beta           [B,H,T]     fp32    write strength (the pages draw it from
 *                                      (0,1); any finite value is accepted)
 *   initial_state  [B,H,dv,dk] fp32    S_0, or NULL for a zero state
 *   o              [B,H,T,dv]  dtype   OUT: o_t = S_t q_t
 *   final_state    [B,H,dv,dk] fp32    OUT: S_T, or NULL to skip it.
 *                                      May be initial_state itself (each
 *                                      workgroup reads its part of S_0 before
 *                                      writing); otherwise it must not overlap
 *                                      initial_state or any input.
 *   chunk_size     tokens per chunk: 64 (the pipelined bf16 kernel; the fast
 *                  path), or 32 (the 32-token kernel, bf16 or fp32).  T need
 *                  not be a multiple: the missing tokens of the last chunk act
 *                  as identity maps (alpha = 1, beta = 0) and produce no
 *                  output.  (fp32 inputs are evaluated 32 tokens at a time for
 *                  either size: 64-token fp32 buffers exceed the LDS at
 *                  d = 128.  The result does not depend on the chunk size
 *                  beyond rounding.)  Other sizes return GDN_ERR_UNSUPPORTED.
 *   dk, dv         64 or 128, dk == dv, for bf16 and fp32.
 *   T              >= 0.  T == 0 writes final_state = initial_state (or zeros).
 *                  For bf16, one sequence's q, k or v (T * d * 2 bytes) must be
 *                  under 2^31 bytes, else GDN_ERR_UNSUPPORTED.
 *
 * `o` must not overlap any input.  The chunk form works with log2(alpha),
 * clamped below at -200: a gate under 2^-200 (alpha == 0 included) acts as
 * 2^-200, which wipes the state up to that factor.
 */
int gdn_chunk_fwd(const void* q, const void* k, const void* v,
                  const float* alpha, const float* beta,
                  const float* initial_state, void* o, float* final_state,
                  int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                  int64_t chunk_size, gdn_dtype dtype, void* hip_stream);

/*
 * gla_chunk_fwd — chunked forward pass of gated linear attention without the
 * delta rule ([P3] §2.3: the state decays by a gate and gains the key-value
 * outer product, with no erase term; [P3] §2.1 inclusive output):
 *
 *     S_t = alpha_t S_{t-1} + beta_t v_t k_t^T,      o_t = S_t q_t,
 *
 * with the same state orientation (S is d_v x d_k) as gdn_chunk_fwd.  Same
 * arguments, layouts, dtypes (bf16 and fp32), chunk sizes (64, or 32 through
 * the 32-token kernel; fp32 is evaluated 32 tokens at a time), aliasing and
 * error codes as gdn_chunk_fwd.
 */
int gla_chunk_fwd(const void* q, const void* k, const void* v,
                  const float* alpha, const float* beta,
                  const float* initial_state, void* o, float* final_state,
                  int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                  int64_t chunk_size, gdn_dtype dtype, void* hip_stream);

/*
 * gdn_scan_fwd — the same recurrence as gdn_chunk_fwd by the other route of
 * [P1]: a (blocked) parallel scan over the per-token affine maps
 * S -> S A_t + B_t, A_t = alpha_t (I - beta_t k_t k_t^T), B_t = beta_t v_t k_t^T
 * ([P1] §2.3 maps compose associatively, §3.1 scan route, §3.4/§5.1 the
 * routes compared).  Each block of L tokens is reduced to its map by a
 * per-token loop, the block start states follow from the maps in order, and
 * every block replays its tokens from its start state.  fp32 state and
 * arithmetic; bf16 or fp32 q/k/v; d 64 or 128 for both dtypes.
 *
 *   workspace   caller-owned device memory of at least
 *               gdn_scan_fwd_workspace(...) bytes (never 0 for B*H > 0),
 *               16-byte aligned, overlapping no other argument.  Calls that
 *               share a workspace must not overlap in time.
 * Other arguments, layouts, aliasing and errors as for gdn_chunk_fwd (no
 * chunk size); a missing or too small workspace returns GDN_ERR_INVALID_ARG.
 */
int gdn_scan_fwd(const void* q, const void* k, const void* v,
                 const float* alpha, const float* beta,
                 const float* initial_state, void* o, float* final_state,
                 int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                 gdn_dtype dtype, void* workspace, size_t workspace_bytes,
                 void* hip_stream);

/*
 * gdn_recurrent_fwd — the forward pass evaluated token by token ([P1] §1.2:
 * each token's state follows from the previous one): one launch walks every
 * sequence's tokens in order with the state in registers, reading the
 * initial state once and writing the final state once.  For many short
 * sequences (a few tokens each, e.g. several new tokens per sequence while
 * decoding) this is much cheaper than the chunked pass, whose per-chunk work
 * does not shrink with T; for long sequences use gdn_chunk_fwd.  Arguments,
 * layouts, dtypes (bf16 and fp32), aliasing and errors as for gdn_chunk_fwd
 * (no chunk size).  alpha is used as given (no clamp).
 */
int gdn_recurrent_fwd(const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta,
                      const float* initial_state, void* o, float* final_state,
                      int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                      gdn_dtype dtype, void* hip_stream);

/* gdn_recurrent_fwd with the per-dimension gate of gdn_scan_fwd_vecgate
 * (alpha [B,H,T,dk] fp32). */
int gdn_recurrent_fwd_vecgate(const void* q, const void* k, const void* v,
                              const float* alpha, const float* beta,
                              const float* initial_state, void* o, float* final_state,
                              int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                              gdn_dtype dtype, void* hip_stream);

/*
 * gdn_scan_fwd_vecgate — gdn_scan_fwd with a per-dimension gate ([P1] §2.2
 * allows a vector gate): alpha is [B,H,T,dk] fp32, each entry in [0,1], and
 * decays the key columns of the state,
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
 * Everything else, the workspace size included, as for gdn_scan_fwd.
 */
int gdn_scan_fwd_vecgate(const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta,
                         const float* initial_state, void* o, float* final_state,
                         int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                         gdn_dtype dtype, void* workspace, size_t workspace_bytes,
                         void* hip_stream);

/*
 * gdn_chunk_fwd_vecgate — the per-dimension gate of gdn_scan_fwd_vecgate on
 * the chunked route ([P1] §2.2 vector gate, §3.2 chunked evaluation): alpha
 * is [B,H,T,dk] fp32, each entry in [0,1], decaying the key columns of the
 * state,
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
 * The per-column decay is folded into the chunk's key and query operands, so
 * the chunk products stay dense MFMA products (bf16 or fp32, as q/k/v).
 * chunk_size must be 32 (this route's chunk: its per-token, per-column decay
 * table and the scaled operand copies fit the LDS at that size); otherwise
 * GDN_ERR_UNSUPPORTED.  Other arguments, layouts, aliasing and errors as for
 * gdn_chunk_fwd.  A gate under 2^-200 acts as 2^-200, as on the scalar path.
 */
int gdn_chunk_fwd_vecgate(const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta,
                          const float* initial_state, void* o, float* final_state,
                          int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                          int64_t chunk_size, gdn_dtype dtype, void* hip_stream);

/*
 * gdn_chunk_fwd_vecgate_split — gdn_chunk_fwd_vecgate for workloads with few
 * sequences: every sequence is cut into G segments that run in parallel and
 * are joined by composing their affine maps ([P1] §2.3, §3.3), exactly as in
 * gdn_chunk_fwd_split (the per-token maps stay affine with a per-dimension
 * gate): the segments' states from a zero start and their transitions, then
 * the segments' start states (fp32), then every segment from its start state.
 * G is chosen from B*H, T, the device's CU count and the kernel's occupancy;
 * when fewer than 3 segments would do, G is 1 and this is
 * gdn_chunk_fwd_vecgate itself (the workspace is not touched).
 *
 *   workspace        device memory owned by the caller, at least
 *                    gdn_chunk_fwd_vecgate_split_workspace(...) bytes (0 when
 *                    no split is planned; NULL is then accepted), 16-byte
 *                    aligned, overlapping no other argument; its contents on
 *                    entry do not matter.  Calls sharing a workspace must not
 *                    overlap in time.
 * Other arguments, layouts, aliasing and errors as for gdn_chunk_fwd_vecgate;
 * a missing or too small workspace returns GDN_ERR_INVALID_ARG.
 */
int gdn_chunk_fwd_vecgate_split(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta,
                                const float* initial_state, void* o, float* final_state,
                                int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                int64_t chunk_size, gdn_dtype dtype, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

/* Workspace bytes gdn_chunk_fwd_vecgate_split needs on the current device
 * (0: no split).  Host-only; also 0 for arguments the entry point rejects. */
size_t gdn_chunk_fwd_vecgate_split_workspace(int64_t B, int64_t H, int64_t T, int64_t dk,
                                             int64_t dv, int64_t chunk_size, gdn_dtype dtype);

/*
 * gdn_chunk_fwd_vecgate_2pass — the result of gdn_chunk_fwd_vecgate
 * ([P1] §2.2 per-dimension gate, §3.2 chunked evaluation; bit for bit for
 * fp32, up to the order of the bf16 products' fp32 sums for bf16), in two
 * passes over tiles of at most 256 chunks (8192 tokens) per sequence:
 *   1. per chunk, once: the gate prefix, the scaled operand copies of q and
 *      k, L, (I+L)^-1 and P, written to a record in the workspace;
 *   2. per 16-row value slice: the state-dependent products of every chunk
 *      of the tile, from the records.
 * The single-pass kernel repeats step 1 in the workgroup of every value
 * slice; here it is done once per chunk, at the cost of writing and reading
 * the records.  The state passes from tile to tile through the workspace.
 * With few sequences (B*H*dv/16 small against the CU count) and a workspace
 * that holds the records of whole sequences, step 2 splits every sequence
 * into segments as gdn_chunk_fwd_split does ([P1] §3.3), joined through their
 * affine state maps; the result then differs from the unsplit one by
 * rounding only.
 *
 *   workspace        device memory owned by the caller, at least
 *                    B*H*(dk*dv*4 + R) bytes for a record size R (one chunk
 *                    per tile); gdn_chunk_fwd_vecgate_2pass_workspace(...)
 *                    gives the size for the largest tile, and a larger
 *                    workspace is not used beyond it.  16-byte aligned,
 *                    overlapping no other argument; its contents on entry do
 *                    not matter.  Calls sharing a workspace must not overlap
 *                    in time.
 * Other arguments, layouts, aliasing (final_state may be initial_state) and
 * errors as for gdn_chunk_fwd_vecgate (chunk_size 32); a missing or too
 * small workspace returns GDN_ERR_INVALID_ARG.
 */
int gdn_chunk_fwd_vecgate_2pass(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta,
                                const float* initial_state, void* o, float* final_state,
                                int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                int64_t chunk_size, gdn_dtype dtype, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

/* Workspace bytes with which gdn_chunk_fwd_vecgate_2pass uses its best plan
 * for these sizes on the current device (the sequence split where one is
 * planned, else the largest tile).  Host-only; 0 for arguments it rejects. */
size_t gdn_chunk_fwd_vecgate_2pass_workspace(int64_t B, int64_t H, int64_t T, int64_t dk,
                                             int64_t dv, int64_t chunk_size, gdn_dtype dtype);

/* Workspace bytes gdn_scan_fwd needs for these sizes.  Host-only. */
size_t gdn_scan_fwd_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                              gdn_dtype dtype);

/*
 * gdn_chunk_fwd_split — the same result as gdn_chunk_fwd, for workloads with
 * few sequences (B*H small against the number of CUs), by splitting every
 * sequence into G segments that run in parallel ([P1] §3.3 splitting a long
 * sequence into parts, joined by composing their affine maps, §2.3):
 *   1. for each of the first G-1 segments, its state from a zero start and
 *      its transition matrix M (the state map S -> S M + tilde), in one launch;
 *   2. the start state of every segment, start_{g+1} = start_g M_g + tilde_g
 *      (fp32);
 *   3. every segment from its start state, writing o and (last segment)
 *      final_state.
 * The work is about (3G-2)/G times that of gdn_chunk_fwd, spread over G
 * times as many workgroups.  G is chosen from B*H, T and the device's CU
 * count; when fewer than 3 segments would do (enough sequences, or T under
 * 1536 tokens: two segments take as long as the plain pass), G is 1, this
 * is gdn_chunk_fwd itself and the workspace is not touched.  bf16 only
 * (fp32 inputs always take gdn_chunk_fwd).
 *
 *   workspace        device memory owned by the caller, at least
 *                    gdn_chunk_fwd_split_workspace(...) bytes, 16-byte
 *                    aligned, overlapping no other argument; its contents
 *                    on entry do not matter.  Calls that share a workspace
 *                    must not overlap in time.
 * Other arguments, errors and aliasing as for gdn_chunk_fwd; a missing or too
 * small workspace (when G > 1) returns GDN_ERR_INVALID_ARG.
 */
int gdn_chunk_fwd_split(const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta,
                        const float* initial_state, void* o, float* final_state,
                        int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                        int64_t chunk_size, gdn_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes gdn_chunk_fwd_split needs for these sizes on the current
 * device (0: it would not split).  A host-side query; launches nothing. */
size_t gdn_chunk_fwd_split_workspace(int64_t B, int64_t H, int64_t T, int64_t dk,
                                     int64_t dv, int64_t chunk_size, gdn_dtype dtype);

/*
 * gdn_chunk_fwd_split_noalloc — gdn_chunk_fwd_split for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result, aliasing and
 * errors as gdn_chunk_fwd_split, without the workspace: the segment states live
 * in a static scratch array of GDN_SPLIT_NOALLOC_SCRATCH_BYTES that the library
 * keeps in the memory of each GPU it runs on until the process ends.  The call
 * allocates and frees nothing (on its first call on a device it only looks up
 * that device's scratch address, with hipGetSymbolAddress).
 *   - It uses the scratch of the device current on the calling thread;
 *     hip_stream must belong to that device.
 *   - A plan that needs more scratch than GDN_SPLIT_NOALLOC_SCRATCH_BYTES
 *     returns GDN_ERR_UNSUPPORTED before anything is launched.  (With 256
 *     compute units every plan fits: the workspace is bounded by about
 *     (B*H + 3 * CUs / 8) * dk * dk * 4 bytes for dk = 128.)
 *   - Every call on one GPU shares that GPU's scratch; its contents on entry
 *     do not matter (each call writes every part it reads), but calls that
 *     overlap in time on one GPU race and give wrong results: serialise them
 *     (one stream, or events).
 *   - When no split is planned (G = 1) the scratch is not touched and this is
 *     gdn_chunk_fwd.
 */
#define GDN_SPLIT_NOALLOC_SCRATCH_BYTES (8u << 20)
int gdn_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta,
                                const float* initial_state, void* o, float* final_state,
                                int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                int64_t chunk_size, gdn_dtype dtype, void* hip_stream);

/*
 * gdn_recurrent_step — one decode step: one new token for each of N*H
 * sequences, applied to the state IN PLACE ([P3] §3.1 analog, with the
 * erase term of [P1] §2.1 and the output of [P3] §2.1).
 *
 *   q, k    [N,H,dk] dtype     v [N,H,dv] dtype
 *   alpha, beta [N,H] fp32
 *   state   [N,H,dv,dk] fp32   IN: S_{t-1}, OUT: S_t (updated in place)
 *   o       [N,H,dv] dtype     OUT: S_t q_t
 *   dk, dv  64 or 128, dk == dv.  N, H >= 0 (N*H == 0 is a no-op).
 *
 * `o` must not overlap any input or the state, and the state must not overlap
 * q, k, v, alpha or beta (GDN_ERR_INVALID_ARG).
 */
int gdn_recurrent_step(const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, float* state,
                       void* o, int64_t N, int64_t H, int64_t dk, int64_t dv,
                       gdn_dtype dtype, void* hip_stream);

/*
 * gdn_recurrent_step_vecgate — gdn_recurrent_step with a per-dimension gate
 * ([P1] §2.2 vector gate): alpha is [N,H,dk] fp32, each entry in [0,1], and
 * decays the key columns of the state,
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * the token update of gdn_chunk_fwd_vecgate (alpha is used as given; nothing
 * clamps it).  Other arguments, layouts, dtypes and errors as for
 * gdn_recurrent_step; `o` must not overlap any input (alpha's dk entries per
 * head included) or the state.
 */
int gdn_recurrent_step_vecgate(const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta, float* state,
                               void* o, int64_t N, int64_t H, int64_t dk, int64_t dv,
                               gdn_dtype dtype, void* hip_stream);

/*
 * gla_recurrent_step — one decode step of gated linear attention without the
 * delta rule ([P3] §2.3), the token update of gla_chunk_fwd:
 *     S_t = alpha_t S_{t-1} + beta_t v_t k_t^T,      o_t = S_t q_t.
 * Arguments, layouts, dtypes (bf16 and fp32) and errors as for
 * gdn_recurrent_step.
 */
int gla_recurrent_step(const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, float* state,
                       void* o, int64_t N, int64_t H, int64_t dk, int64_t dv,
                       gdn_dtype dtype, void* hip_stream);

/* Static, human-readable text for a return code (never NULL). */
const char* gdn_strerror(int code);

/* Version of the library as "major.minor.patch" (static string). */
const char* gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
