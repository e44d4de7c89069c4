/*
 * moe.h — C ABI of one rank's MoE expert-layer forward on an AMD Instinct
 * MI355X (gfx950): router top-k, token dispatch, grouped expert GEMM with
 * SwiGLU, and the weighted combine.
 *
 * Sources of the operations (page title, then section):
 *   [EP] "Paralelismo de especialistas" (transformers v5.23.0 docs, pt), with
 *        the tr ("Uzman paralelliği") and zh ("专家并行") pages of transformers main;
 *   [TP] "Paralelismo de tensor para inferência" (transformers main docs, pt).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer to a dense row-major array that
 *     the caller allocates and owns. The library allocates nothing. Its only
 *     process-wide state is a per-device cache of the compute-unit count (read
 *     once per device with hipDeviceGetAttribute, filled atomically, never
 *     changed afterwards), which sizes the persistent GEMM grids, and the
 *     per-device array of moe_dispatch_indices_noalloc with its address cache.
 *     Calls on different streams may run concurrently when they write disjoint
 *     buffers (moe_dispatch_indices_noalloc excepted: see there).
 *   - Every call validates its arguments on the host, enqueues its kernels on
 *     `stream` and returns without synchronising. Invalid arguments return
 *     MOE_EINVAL (or MOE_EUNSUPPORTED for a valid but unsupported shape) before
 *     anything is enqueued, so no output is touched on error. A failed kernel
 *     launch returns MOE_EHIP. Faults inside kernels surface at the caller's
 *     next synchronisation.
 *   - Shapes: T tokens on this rank (T = 0 is a valid no-op call), hidden size
 *     d, expert FFN width d_ff, E global experts, top-k k, and this rank's
 *     contiguous block of local experts [e_begin, e_end) with
 *     E_loc = e_end - e_begin. A flat pair index is p = t*k + j.
 *     N_max = T * min(k, E_loc) bounds the number of local pairs N_loc, so every
 *     buffer can be sized on the host without reading any device value (the
 *     layer needs no host synchronisation).
 *   - Limits: 1 <= k <= E <= 1024; T*k < 2^31; d and d_ff are multiples of 8
 *     (16-byte rows of bf16); 1 <= E_loc.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* invalid argument (null pointer, bad shape, bad range) */
  MOE_EUNSUPPORTED = 2, /* valid but unsupported (e.g. E > 1024) */
  MOE_EHIP = 3          /* a HIP launch failed */
} moe_status;

/* Element type of activations, weights, H, Y and outputs. Router logits and
 * routing weights are always fp32; indices are always int32. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef struct {
  int64_t T;        /* tokens in this call, >= 0 */
  int32_t d;        /* hidden size, > 0, multiple of 8 */
  int32_t d_ff;     /* expert FFN width, > 0, multiple of 8 */
  int32_t E;        /* global experts */
  int32_t k;        /* experts per token, 1 <= k <= E */
  int32_t e_begin;  /* first local expert (global id) */
  int32_t e_end;    /* one past the last local expert; 0 <= e_begin < e_end <= E */
} moe_shape;

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status status);

/* Local expert block of `rank` under expert parallelism of size `ep`:
 * [EP] "Como os tamanhos se combinam": ep_size cuts the expert list into
 * ep_size contiguous blocks, each rank computes E/ep experts and ep_size
 * consecutive ranks hold a full set, so the block of rank r is
 * [(r % ep) * E/ep, (r % ep + 1) * E/ep). Host-only; writes *e_begin, *e_end.
 * MOE_EINVAL unless E >= 1, ep >= 1, E % ep == 0, rank >= 0 and both output
 * pointers are non-null. */
moe_status moe_expert_range(int32_t E, int32_t ep, int32_t rank,
                            int32_t* e_begin, int32_t* e_end);

/* Router top-k ([EP] "Adicionando uma implementação": the implementation is
 * called with top_k_index / top_k_weights; [EP] intro: each token activates
 * only a few experts).
 *   logits   [T, E] fp32, read only.
 *   topk_idx [T, k] int32, written: the k largest logits of each token in
 *            descending order; equal logits go to the lower expert id and
 *            -0.0 equals +0.0. Global expert ids.
 *   topk_w   [T, k] fp32, written: softmax over the k selected logits (they
 *            sum to 1 per token), computed in fp32.
 * Logits must be finite; NaN/Inf give unspecified ids but never a fault.
 * Uses s->T, s->E, s->k only. */
moe_status moe_route_topk(const moe_shape* s, const float* logits,
                          int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* Bytes of device workspace moe_dispatch needs for this shape (may be 0). */
size_t moe_dispatch_workspace_bytes(const moe_shape* s);

/* Token dispatch on one rank ([EP] "Despacho de tokens": every (token, expert)
 * pair goes to the rank owning the expert and only local experts compute;
 * [EP] "Como os tamanhos se combinam": ownership is one contiguous block, so
 * this rank's pairs form one contiguous segment of the expert-sorted list;
 * [TP] EpRouterParallel row: local experts are addressed by local ids).
 *   x        [T, d] dt, read only: hidden states.
 *   topk_idx [T, k] int32, read only: global expert ids. An id outside [0, E)
 *            is dropped: not counted, pair_pos = -1, and the perm slots it
 *            would take (past offsets[E]) are left unwritten.
 *   counts   [E]   int32, written: pairs per expert over ALL experts.
 *   offsets  [E+1] int32, written: exclusive prefix sum of counts.
 *   perm     [T*k] int32, written: sorted slot -> flat pair p, pairs sorted by
 *            expert id, stable in p inside each expert.
 *   pair_pos [T*k] int32, written: flat pair -> row in x_perm of this rank
 *            (slot - offsets[e_begin]) for a local pair, -1 otherwise.
 *   x_perm   [N_max, d] dt, written: rows [0, N_loc) hold x[perm[offsets
 *            [e_begin] + r] / k]; rows past N_loc are left unwritten.
 *   workspace moe_dispatch_workspace_bytes(s) bytes of device memory (may be
 *            NULL when that is 0); contents on entry do not matter.
 * T = 0 still writes counts and offsets (all zero). MOE_EINVAL if workspace is
 * NULL while moe_dispatch_workspace_bytes(s) > 0. */
moe_status moe_dispatch(const moe_shape* s, moe_dtype dt, const void* x,
                        const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* pair_pos, void* x_perm,
                        void* workspace, hipStream_t stream);

/* Debug builds. The library compiled with MOE_DEBUG defined (libmoe_debug.so,
 * built beside libmoe.so) also checks on the device the expert ids that
 * moe_dispatch and moe_dispatch_indices receive, where the release build drops
 * an id outside [0, E) without a trace ("Paralelismo de especialistas",
 * "Sobrescrevendo os planos": invalid input is refused rather than sharded).
 * Each call then writes an int32 error word into its workspace, at byte offset
 * moe_dispatch_debug_word_offset(): the number of ids outside [0, E) in
 * topk_idx, 0 when every id is valid (T = 0 writes 0). It is rewritten by every
 * call; read it once the stream has passed the call. The outputs are those of
 * the release build. Returns SIZE_MAX in release builds (no error word). */
size_t moe_dispatch_debug_word_offset(void);

/* moe_dispatch without the row gather: counts, offsets, perm and pair_pos as
 * moe_dispatch writes them, and no x_perm. For the fused path, in which
 * moe_grouped_gemm_gather reads each local row straight from x. Same sources,
 * arguments and errors as moe_dispatch (x, x_perm and dt are not taken); the
 * workspace size is moe_dispatch_workspace_bytes(s). */
moe_status moe_dispatch_indices(const moe_shape* s, const int32_t* topk_idx,
                                int32_t* counts, int32_t* offsets, int32_t* perm,
                                int32_t* pair_pos, void* workspace, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): moe_dispatch_indices
 * with its workspace taken from an array of MOE_DISPATCH_SCRATCH_BYTES bytes
 * that the library holds in each GPU's device memory until the process ends.
 * Same outputs, bit for bit, and same errors as moe_dispatch_indices, plus
 * MOE_EUNSUPPORTED when moe_dispatch_workspace_bytes(s) exceeds
 * MOE_DISPATCH_SCRATCH_BYTES (8 MiB: for example up to about 1M pairs at
 * E = 256, or 2M pairs at E = 128), and MOE_EHIP if the array's address cannot
 * be found. No memory is allocated or freed. Every call on one GPU uses that
 * GPU's one array, so calls that overlap on one GPU (from several streams or
 * host threads) race and give undefined results; calls in one stream are safe.
 * The array needs no clearing between calls. The stream must belong to the
 * current device. */
#define MOE_DISPATCH_SCRATCH_BYTES ((size_t)8 << 20)
moe_status moe_dispatch_indices_noalloc(const moe_shape* s, const int32_t* topk_idx,
                                        int32_t* counts, int32_t* offsets, int32_t* perm,
                                        int32_t* pair_pos, hipStream_t stream);

/* Bytes of device workspace the grouped GEMM calls take for this shape (may be
 * 0). moe_grouped_gemm_gather(_save) use it for a copy of the gathered rows in
 * 32-column blocks ([d/32][N_max][32]), whose K = 32 stages the gate/up loads
 * read as contiguous runs, followed by 1 KB of per-XCD tile counts that pace the
 * gate/up launch's workgroups (cleared by the call itself): N_max * d * 2 + 1024
 * bytes for bf16 when each row is read by at least 20 gate/up column tiles
 * (d_ff / 128 >= 20) and the local experts average at least 128 rows
 * (N_max / E_loc >= 128), 0 otherwise. Passing NULL instead makes those calls
 * read the rows straight from x (same results, bit for bit). Calls that overlap
 * on one workspace race. moe_grouped_gemm takes no workspace. */
size_t moe_grouped_gemm_workspace_bytes(const moe_shape* s, moe_dtype dt);

/* Grouped expert FFN over this rank's local experts: experts_forward of
 * [EP] "Adicionando uma implementação", with the weights sharded along the
 * expert dimension ([EP] GroupedGemmParallel) and the packed gate/up layout of
 * [TP] "Estratégias empacotadas" (gate = first d_ff columns, up = the rest).
 * For each local expert e with rows R (its segment of x_perm):
 *     H_R = silu(R @ Wgu[e][:, :d_ff]) * (R @ Wgu[e][:, d_ff:])
 *     Y_R = H_R @ Wdn[e]
 * with fp32 accumulation; for dt = MOE_BF16, H and Y are rounded to bf16 (RNE).
 *   x_perm    [N_max, d] dt, read only (rows [0, N_loc) are used).
 *   offsets   [E+1] int32 DEVICE array from moe_dispatch; the row counts are
 *             read on the device, never on the host.
 *   w_gate_up [E_loc, d, 2*d_ff] dt, read only. Empty experts are not read.
 *   w_down    [E_loc, d_ff, d] dt, read only.
 *   h         [N_max, d_ff] dt, written (intermediate activations).
 *   y         [N_max, d] dt, written: rows [0, N_loc).
 *   workspace not used (may be NULL).
 * Uses s->T, d, d_ff, k, e_begin, e_end. */
moe_status moe_grouped_gemm(const moe_shape* s, moe_dtype dt, const void* x_perm,
                            const int32_t* offsets, const void* w_gate_up,
                            const void* w_down, void* h, void* y, void* workspace,
                            hipStream_t stream);

/* moe_grouped_gemm with the dispatch's row gather folded into the gate/up
 * loads: the activation rows of local row r are x[perm[offsets[e_begin] + r] / k]
 * read directly from x (or, with a workspace of moe_grouped_gemm_workspace_bytes
 * > 0 bytes, from a blocked copy of them made first), so x_perm is never written
 * or read. Results (h, y) are bit-identical to moe_dispatch + moe_grouped_gemm.
 * Same sources as those two.
 *   x         [T, d] dt, read only: hidden states.
 *   perm      [T*k] int32 DEVICE array from moe_dispatch or moe_dispatch_indices.
 *   offsets, w_gate_up, w_down, h, y, workspace: as for moe_grouped_gemm
 *             (workspace size moe_grouped_gemm_workspace_bytes(s, dt)).
 * MOE_EUNSUPPORTED unless dt = MOE_BF16, d and d_ff are multiples of 32 and
 * T * d * 2 bytes fit in 31 bits; use moe_dispatch + moe_grouped_gemm then. */
moe_status moe_grouped_gemm_gather(const moe_shape* s, moe_dtype dt, const void* x,
                                   const int32_t* perm, const int32_t* offsets,
                                   const void* w_gate_up, const void* w_down, void* h,
                                   void* y, void* workspace, hipStream_t stream);

/* Weighted combine back to token order ([EP] "Despacho de tokens": results are
 * combined with the routing weights; "Adicionando uma implementação": the
 * output is the weighted expert output of every token this rank holds):
 *     out[t] = sum over j = 0..k-1 with pair_pos[t*k+j] >= 0 of
 *              topk_w[t, j] * y[pair_pos[t*k+j]]
 * accumulated in fp32 in slot order, rounded once to dt. A token with no local
 * pair gets a zero row; every one of the T rows is written.
 *   y        [N_max, d] dt, read only.
 *   pair_pos [T*k] int32, read only: a local row in [0, N_max), or -1; any other
 *            value (negative or >= N_max) is treated as -1 and contributes nothing.
 *   topk_w   [T, k] fp32, read only.
 *   out      [T, d] dt, written. */
moe_status moe_combine(const moe_shape* s, moe_dtype dt, const void* y,
                       const int32_t* pair_pos, const float* topk_w, void* out,
                       hipStream_t stream);

/* ------------------------------------------------------------------ backward
 * The gradient of the forward above, step by step in reverse order. The pages
 * ask for it as the training use of the layer ("Paralelismo de especialistas":
 * gradients return to every rank that holds a token; the masking variant's
 * partial outputs are summed across ranks, so are their gradients) and give no
 * formula: each call is the chain rule through the forward call of the same
 * name. On one rank every gradient is that rank's partial gradient; their sum
 * over ranks is the full one. Gradients arrive and leave in dt (d_topk_w and
 * d_logits in fp32) and accumulate in fp32. */

/* Gradient of moe_combine:
 *     d_y[r]        = topk_w[t, j] * d_out[t]    for the local pair (t, j) at row r
 *     d_topk_w[t, j] = <d_out[t], y[r]>           (0 when pair (t, j) is not local)
 *   d_out    [T, d] dt, read only: gradient of the layer output.
 *   y, pair_pos, topk_w: as passed to moe_combine.
 *   d_y      [N_max, d] dt, written: rows [0, N_loc).
 *   d_topk_w [T, k] fp32, written. */
moe_status moe_combine_backward(const moe_shape* s, moe_dtype dt, const void* d_out,
                                const void* y, const int32_t* pair_pos, const float* topk_w,
                                void* d_y, float* d_topk_w, hipStream_t stream);

/* Bytes of device workspace moe_grouped_gemm_backward needs (0 unless dt is
 * MOE_BF16): the gathered rows, a copy of d_y, and the gate/up pre-activations
 * and their gradient, each for N_max rows. */
size_t moe_grouped_gemm_backward_workspace_bytes(const moe_shape* s, moe_dtype dt);

/* Gradient of the grouped expert FFN (moe_grouped_gemm / _gather). For each local
 * expert e with rows R, [G | U] = X_R @ W_gu[e] (recomputed here), H = silu(G) * U:
 *     dH = d_y @ W_dn[e]^T;  dG = dH * U * silu'(G);  dU = dH * silu(G)
 *     d_x_perm = [dG | dU] @ W_gu[e]^T
 *     d_w_down[e]    = H^T @ d_y
 *     d_w_gate_up[e] = X_R^T @ [dG | dU]
 *   x, perm   the hidden states [T, d] and the dispatch's perm (as for
 *             moe_grouped_gemm_gather; X_R are the gathered rows).
 *   offsets, w_gate_up, w_down: as for the forward.
 *   h         [N_max, d_ff] dt, read only: the forward's h.
 *   d_y       [N_max, d] dt, read only: from moe_combine_backward.
 *   d_x_perm  [N_max, d] dt, written: rows [0, N_loc).
 *   d_w_gate_up [E_loc, d, 2*d_ff] dt, d_w_down [E_loc, d_ff, d] dt, written in
 *             full (zero for an expert with no rows).
 *   workspace moe_grouped_gemm_backward_workspace_bytes(s, dt) bytes.
 * MOE_EUNSUPPORTED unless dt = MOE_BF16, d and d_ff are multiples of 32, and the
 * activation blocks (N_max rows of max(d, 2*d_ff)) and x fit 31-bit byte offsets. */
moe_status moe_grouped_gemm_backward(const moe_shape* s, moe_dtype dt, const void* x,
                                     const int32_t* perm, const int32_t* offsets,
                                     const void* w_gate_up, const void* w_down, const void* h,
                                     const void* d_y, void* d_x_perm, void* d_w_gate_up,
                                     void* d_w_down, void* workspace, hipStream_t stream);

/* Gradient of the dispatch's row gather: d_x[t] = sum over t's local pairs (slot
 * order, fp32) of d_x_perm[pair_pos[t*k + j]]; zero rows for tokens without one.
 *   d_x_perm [N_max, d] dt, read only.  pair_pos: as from moe_dispatch.
 *   d_x      [T, d] dt, written (every row). */
moe_status moe_dispatch_backward(const moe_shape* s, moe_dtype dt, const void* d_x_perm,
                                 const int32_t* pair_pos, void* d_x, hipStream_t stream);

/* Training pair: a forward that keeps the gate/up pre-activations and a
 * backward that takes them instead of recomputing them (one grouped GEMM of
 * 4 N_loc d d_ff FLOP fewer, for 2 N_max d_ff elements of device memory).
 * Same computation and sources as moe_grouped_gemm_gather and
 * moe_grouped_gemm_backward above.
 *
 * moe_grouped_gemm_gather_save: moe_grouped_gemm_gather (same h and y, bit for
 * bit), and also
 *   gu        [N_max, 2*d_ff] dt, written: rows [0, N_loc) hold [G | U] = X_R @
 *             W_gu[e] for each local row (G in columns [0, d_ff), U after it),
 *             rounded to dt from the fp32 accumulators that h is formed from.
 * MOE_EINVAL if gu is NULL with T > 0; otherwise as moe_grouped_gemm_gather. */
moe_status moe_grouped_gemm_gather_save(const moe_shape* s, moe_dtype dt, const void* x,
                                        const int32_t* perm, const int32_t* offsets,
                                        const void* w_gate_up, const void* w_down, void* h, void* y,
                                        void* gu, void* workspace, hipStream_t stream);

/* moe_grouped_gemm_backward with [G | U] read from gu (as written by
 * moe_grouped_gemm_gather_save for the same x, perm, offsets and w_gate_up)
 * rather than recomputed: the same gradients, bit for bit. Arguments as for
 * moe_grouped_gemm_backward, plus
 *   gu        [N_max, 2*d_ff] dt, read only.
 * The workspace is the same size (its [G | U] part goes unused).
 * MOE_EINVAL if gu is NULL with T > 0; otherwise as moe_grouped_gemm_backward. */
moe_status moe_grouped_gemm_backward_saved(const moe_shape* s, moe_dtype dt, const void* x,
                                           const int32_t* perm, const int32_t* offsets,
                                           const void* w_gate_up, const void* w_down,
                                           const void* h, const void* gu, const void* d_y,
                                           void* d_x_perm, void* d_w_gate_up, void* d_w_down,
                                           void* workspace, hipStream_t stream);

/* Gradient of the combine weights of moe_route_topk w.r.t. the logits (softmax
 * over the selected logits; the selection passes no gradient):
 *     d_logits[t, topk_idx[t, j]] = topk_w[t, j] * (d_topk_w[t, j] - sum_i topk_w[t, i] * d_topk_w[t, i])
 * and 0 for every other expert.
 *   topk_idx, topk_w [T, k]: from moe_route_topk (ids of a token distinct).
 *   d_topk_w [T, k] fp32, read only.   d_logits [T, E] fp32, written (every entry). */
moe_status moe_route_topk_backward(const moe_shape* s, const int32_t* topk_idx,
                                   const float* topk_w, const float* d_topk_w, float* d_logits,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
