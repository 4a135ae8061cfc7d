/*
 * ggq.h -- C ABI of the MI355X (gfx950) library for matrix products over GGUF
 * block-quantized weights.
 *
 * What the calls compute, and the passages they follow:
 *  - Phobos README (githubhelp mirror), section "Inference": quantized GGUF models
 *    (Q8_0, Q4_K_M) run their products on the GPU at decode time; the engine
 *    fuses kernels ("Kernel fusion, memory management" under "Components").
 *  - Same README, opening paragraph: a mixture-of-experts layer sends each token
 *    to a few experts and only those experts' weights are used.
 *  - Same README, "Command-Line Tools" / phobos-bench: prompt processing is
 *    measured at pp<N> (N-token prompts); prompt batches are matrix-matrix work.
 *  - Kernel-cache page (phobos-lang.dev, section "Kernel cache"): one kernel per
 *    shape and format.
 * The pages define neither block format; this library reads them as the GGUF
 * on-disk layout:
 *    Q8_0: 34-byte blocks of 32 weights: fp16 d, then 32 int8 q.  w = d*q.
 *    Q4_K: 144-byte super-blocks of 256 weights: fp16 d, fp16 dmin, 12 bytes of
 *          packed 6-bit sub-block scales sc[8] and mins m[8], then 128 bytes of
 *          4-bit quants.  w = d*sc*q - dmin*m.
 *
 * Conventions for every call:
 *  - A quantized matrix W is N x K, row-major: row r is K/32 Q8_0 blocks
 *    (K*34/32 bytes) or K/256 Q4_K super-blocks (K*144/256 bytes); rows are
 *    contiguous.  Activations X are fp32 [B][K] with row stride ldx (elements);
 *    outputs Y are fp32 [B][N] with row stride ldy.
 *  - Every pointer is a device pointer owned by the caller (e.g. a torch tensor's
 *    data_ptr()).  The library allocates nothing, keeps no pointer after return
 *    and never synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL
 *    is the default stream).
 *  - Arguments are validated on the host before any HIP call; an invalid call
 *    returns a negative ggq_status and enqueues nothing.  A launch failure returns
 *    GGQ_ERR_LAUNCH.  Device faults surface at the caller's next synchronisation.
 *  - Results are deterministic: the same inputs give the same bits.  Floating-
 *    point atomics appear in two places, both as two adds onto an output that
 *    an earlier kernel of the same call zeroed: the matrix-core decode GEMV
 *    (quant_gemv and friends with a workspace, batch >= 2) when a row tile's K
 *    range is cut in two, and quant_gemm at 17..128 rows when K is cut in two.
 *    0 + a + b gives the same bits in either order, so the result does not
 *    depend on which half lands first; deeper K cuts keep per-part sums in the
 *    workspace and add them in part order.
 *  - Outputs never alias inputs or the workspace: y (or c, h) must not overlap
 *    w, x (or a) or ws.
 *  - Workspaces of quant_gemv, quant_gemv_grouped, quant_gemv_swiglu,
 *    quant_gemm and moe_layer_gemv begin with a control block of
 *    GGQ_CTRL_BYTES: counters through which the workgroups of one launch learn
 *    which of them finishes last (the one that adds up a tile's K parts, or
 *    makes the expert selection).  It must be zero before a workspace is
 *    first used (allocate it zeroed, or clear those bytes once); every call
 *    leaves it zero, and the rest of the workspace may hold anything.  These
 *    calls can therefore share one workspace; a workspace that served other
 *    calls (moe_*) or a call that failed on the device must be cleared again.
 *  - Nothing throws across this interface.
 */
#ifndef GGQ_H
#define GGQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GGQ_CTRL_BYTES 4096u

/* Block formats, numbered as GGUF tensor types. */
enum ggq_type { GGQ_Q8_0 = 8, GGQ_Q4_K = 12 };

enum ggq_status {
    GGQ_OK = 0,
    GGQ_ERR_ARG = -1,         /* null pointer, bad size, K not a multiple of the block */
    GGQ_ERR_UNSUPPORTED = -2, /* unknown format or mode */
    GGQ_ERR_ALIGN = -3,       /* a pointer or leading dimension breaks the alignment rules */
    GGQ_ERR_WORKSPACE = -4,   /* workspace missing or smaller than the size query says */
    GGQ_ERR_LAUNCH = -5,      /* the HIP runtime refused a launch */
    GGQ_ERR_SCRATCH = -6      /* quant_gemv_noalloc: the call needs more than its fixed scratch */
};

/* Arithmetic of the prompt GEMM.  Only bf16 operands with fp32 accumulation are
 * built; an int8 mode (per-32-column activation quantisation) would take the
 * value 1 and is refused as GGQ_ERR_UNSUPPORTED. */
enum ggq_gemm_mode { GGQ_GEMM_BF16 = 0 };

/* Short English text for a status code; never NULL. */
const char *ggq_status_string(int status);

/* Library ABI version (major*10000 + minor*100 + patch). */
int ggq_version(void);

/*
 * quant_dequantize -- out[r][c] = w[r][c] as fp32 for an N x K quantized matrix.
 * Follows the block definitions above.  The result is exact: Q8_0 d*q and Q4_K
 * d*sc*q, dmin*m are exact in fp32 and the Q4_K difference is rounded once, so
 * any correct implementation gives the same bits.
 *   type  GGQ_Q8_0 (K % 32 == 0) or GGQ_Q4_K (K % 256 == 0)
 *   w     device, N rows of K/32*34 or K/256*144 bytes, 16-byte aligned
 *   out   device, N*K floats, row-major, 16-byte aligned
 * N == 0 is a no-op.  Errors: GGQ_ERR_ARG, GGQ_ERR_UNSUPPORTED, GGQ_ERR_ALIGN.
 */
int quant_dequantize(int type, const void *w, int64_t n, int64_t k, float *out, void *stream);

/*
 * quant_gemv -- decode matrix-vector product, batch 1..16:
 *     y[b][r] = sum_c w[r][c] * x[b][c]   for b < batch, r < N
 * with the weights decoded on the fly (never materialised) and one read of W
 * serving every batch row (README "Inference": the decode-time product).
 * The result is within 1e-5 * sum_c |w x| of the exact value.
 *   w     device, 16-byte aligned
 *   x     device fp32 [batch][ldx], ldx >= K, 16-byte aligned, ldx % 4 == 0
 *   y     device fp32 [batch][ldy], ldy >= N
 *   batch 1..16
 *   ws    NULL, or device workspace of at least quant_gemv_workspace_size(type, K,
 *         batch) bytes, 256-byte aligned, control block zero (see above), not
 *         shared with a call running at the same time.  With a workspace the
 *         activations are split into exact fp16 pairs and the products run on
 *         the matrix cores (fp32 accumulation): for one matrix, when the
 *         workspace also holds the K-part sums (quant_gemv_split_workspace_size),
 *         in a single launch that splits the activations itself; otherwise
 *         (batch >= 2) after a pass that splits them.  At batch 1 only that
 *         single launch uses the workspace, and only for Q4_K matrices that
 *         take more workgroups than the device has compute units and whose
 *         rows are few and long (fewer than 16 per compute unit, K above
 *         6144); other batch-1 calls run on the vector units.  With NULL every batch row
 *         costs one fp32 FMA per weight on the vector units.  All paths meet the
 *         same tolerance.
 * A matrix may hold at most 4 GiB ((N + 64) * row bytes < 2^32) and an activation
 * block batch * ldx * 4 < 2^32 bytes.
 * N == 0 is a no-op.  Errors: GGQ_ERR_ARG (null, K not a multiple of the block,
 * batch out of range, ld too small, size limits), GGQ_ERR_ALIGN, GGQ_ERR_WORKSPACE
 * (ws given but too small), GGQ_ERR_UNSUPPORTED.
 */
int quant_gemv(int type, const void *w, int64_t n, int64_t k, const float *x, int64_t ldx,
               float *y, int64_t ldy, int batch, void *ws, size_t ws_bytes, void *stream);

/*
 * quant_gemv_noalloc -- quant_gemv for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same product, arguments and tolerance as quant_gemv
 * with a workspace, but the workspace is a fixed array of
 * GGQ_NOALLOC_SCRATCH_BYTES in device memory that the library holds on each GPU
 * it runs on until the process ends.  The call allocates and frees nothing.
 *   batch 1 runs on the vector units and uses no scratch.  batch >= 2 runs on
 *   the matrix cores with the activation fragments in the scratch, and also
 *   cuts K across workgroups when the partial-sum planes
 *   (quant_gemv_split_workspace_size) fit; with the same workspace size
 *   quant_gemv gives the same bits.
 * Calls on one GPU share its scratch, and each call leaves its contents behind:
 * the scratch starts zeroed when the library loads and every call leaves its
 * control block zero (the rest is rewritten by each call before use).  Calls
 * that can overlap on one GPU (several streams or host threads) race and must
 * be serialised by the caller.  The stream must belong to the current device; the scratch address
 * of a device is looked up on the first call made with that device current.
 * Errors: as quant_gemv, and GGQ_ERR_SCRATCH when
 * quant_gemv_workspace_size(type, K, batch) exceeds the scratch (nothing is
 * launched); GGQ_ERR_LAUNCH if the scratch address cannot be obtained.
 */
#define GGQ_NOALLOC_SCRATCH_BYTES (16u << 20)

int quant_gemv_noalloc(int type, const void *w, int64_t n, int64_t k, const float *x,
                       int64_t ldx, float *y, int64_t ldy, int batch, void *stream);

/* Workspace bytes one matrix of K columns needs in quant_gemv at this batch
 * (control block included); 0 on bad arguments. */
size_t quant_gemv_workspace_size(int type, int64_t k, int batch);

/* Larger workspace for a matrix of N rows and K columns: with at least this
 * many bytes (summed over the descriptors of a grouped call) the matrix-core
 * path may also cut each row tile into K parts, run them on separate
 * workgroups and keep their fp32 partial sums in the workspace, added in part
 * order (by the last workgroup of the tile, or by a second launch) -- for
 * short, long-K matrices, whose row tiles alone leave most of the chip idle.
 * The result is as deterministic and within the same tolerance as without.
 * With less (but at least quant_gemv_workspace_size) nothing changes.  0 on
 * bad arguments. */
size_t quant_gemv_split_workspace_size(int type, int64_t n, int64_t k, int batch);

/*
 * quant_gemv_grouped -- several decode products of the same format and batch in
 * one launch: for each descriptor i,
 *     descs[i].y[b][r] = sum_c descs[i].w[r][c] * descs[i].x[b][c]
 * with the same rules and tolerance as quant_gemv.  Meant for the projections of
 * a decoder layer (README "Components": kernel fusion), so that small matrices
 * share one launch instead of each paying its own start-up.  The descriptor
 * array is read on the host during the call and may be reused afterwards.
 *   count  1..16;  descriptors with n == 0 are skipped
 *   ws     NULL, or at least GGQ_CTRL_BYTES plus, per descriptor,
 *          quant_gemv_workspace_size(type, descs[i].k, batch) - GGQ_CTRL_BYTES
 *          bytes (the plain sum of quant_gemv_workspace_size always suffices);
 *          control block zero
 * Errors: as quant_gemv, for any descriptor; nothing is launched on error.
 */
typedef struct ggq_gemv_desc {
    const void *w;     /* N x K quantized matrix, 16-byte aligned */
    int64_t n;
    int64_t k;
    const float *x;    /* [batch][ldx], 16-byte aligned, ldx % 4 == 0, ldx >= k */
    int64_t ldx;
    float *y;          /* [batch][ldy], ldy >= n */
    int64_t ldy;
} ggq_gemv_desc;

int quant_gemv_grouped(int type, const ggq_gemv_desc *descs, int count, int batch, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * quant_gemv_swiglu -- the gate and up projections of a dense gated
 * feed-forward in one pass, fused with its activation (README "Components":
 * kernel fusion):
 *     h[b][r] = silu(sum_c wg[r][c] x[b][c]) * (sum_c wu[r][c] x[b][c]),
 *     silu(g) = g / (1 + exp(-g)),
 * for b < batch, r < N -- the first half of a routed expert's feed-forward
 * (moe_expert_gemv) for one expert and every token.  A workgroup holds the
 * same rows of both matrices, so neither product is written out.  Each product
 * is within the quant_gemv tolerance before the activation.
 *   wg, wu  N x K quantized matrices, 16-byte aligned; K % 256 == 0
 *   x       device fp32 [batch][ldx], 16-byte aligned, ldx % 4 == 0, ldx >= K
 *   h       device fp32 [batch][ldh], ldh >= N
 *   batch   1..16
 *   ws      batch >= 2: device workspace of at least
 *           quant_gemv_workspace_size(type, K, batch) bytes, 256-byte aligned,
 *           control block zero (the activation fragments follow it); batch 1:
 *           may be NULL
 * N == 0 is a no-op.  Errors: as quant_gemv; GGQ_ERR_ARG for K % 256 != 0;
 * GGQ_ERR_WORKSPACE for batch >= 2 without the workspace.
 */
int quant_gemv_swiglu(int type, const void *wg, const void *wu, int64_t n, int64_t k,
                      const float *x, int64_t ldx, float *h, int64_t ldh, int batch,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * quant_gemm_workspace_size -- bytes of device workspace quant_gemm needs for
 * these sizes (the bf16 copy of A plus tile bookkeeping; for M <= 16 at least
 * the split-K GEMV workspace).  0 on bad arguments.
 */
size_t quant_gemm_workspace_size(int type, int64_t m, int64_t n, int64_t k, int mode);

/*
 * quant_gemm -- prompt-batch product (phobos-bench pp<N>):
 *     c[i][r] = sum_c a[i][c] * w[r][c]   for i < M, r < N
 * Activations are rounded to bf16 and weight tiles decoded to bf16 in LDS; the
 * products accumulate in fp32 on the matrix cores.  Result within
 * 8e-3 * sum_c |a w| of the exact value.  Up to 16 rows (M <= 16) the product
 * runs as quant_gemv instead (one read of W; within its tighter 1e-5 bound).
 * From 17 to 128 rows, when K is a multiple of 256 and the 64-row column tiles
 * cover the device, all rows of a 64-row block share each weight read (A in
 * bf16 staged through LDS, weights decoded straight into matrix-core operands;
 * c is first zeroed when K is cut in two).
 *   a     device fp32 [M][lda], lda >= K, lda % 4 == 0, 16-byte aligned
 *   c     device fp32 [M][ldc], ldc >= N
 *   mode  GGQ_GEMM_BF16
 *   ws    device workspace of at least quant_gemm_workspace_size() bytes,
 *         256-byte aligned, control block zero; the rest may hold anything
 * M == 0 or N == 0 is a no-op.  Errors: GGQ_ERR_ARG, GGQ_ERR_ALIGN,
 * GGQ_ERR_WORKSPACE, GGQ_ERR_UNSUPPORTED.
 */
int quant_gemm(int type, const void *w, int64_t n, int64_t k, const float *a, int64_t lda,
               int64_t m, float *c, int64_t ldc, int mode, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_route -- router of a mixture-of-experts layer (README opening paragraph):
 *     logits[t][e] = sum_h wr[e][h] * x[t][h]   (fp32)
 * then the top_k experts by softmax probability (equivalently by logit), in
 * rank order, equal logits ranking the lower expert index first, and their
 * probabilities renormalised over the selected set:
 *     probs[t][s] = exp(l_s - l_max) / sum_{s'} exp(l_s' - l_max).
 *   wr     device fp32 [E][H], 16-byte aligned, H % 4 == 0
 *   x      device fp32 [T][H], 16-byte aligned
 *   idx    device int32 [T][top_k]
 *   probs  device fp32 [T][top_k]
 *   logits device fp32 [T][E], required (not NULL): always written, and the
 *          selection is made on these stored values
 *   1 <= top_k <= min(E, 32), 1 <= E <= 1024, H % 4 == 0, H <= 2^24.
 *   T == 0 is a no-op.
 * Logits must be finite for the selection to be meaningful.
 * Errors: GGQ_ERR_ARG, GGQ_ERR_ALIGN.
 */
int moe_route(const float *wr, int64_t e, int64_t h, const float *x, int64_t t, int top_k,
              int32_t *idx, float *probs, float *logits, void *stream);

/*
 * moe_workspace_size -- device workspace bytes moe_expert_gemv needs:
 * per-expert token lists, the hidden state h [T*top_k][F] and the per-slot
 * down-projection outputs [T*top_k][H].  0 on bad arguments.
 */
size_t moe_workspace_size(int64_t e, int64_t t, int top_k, int64_t h, int64_t f);

/*
 * moe_expert_gemv -- routed expert feed-forward for T tokens:
 *     for each token t and slot s with expert e = idx[t][s]:
 *         g = Wg[e] x_t,  u = Wu[e] x_t,  h = silu(g) * u,  d = Wd[e] h
 *     y[t] = sum_s probs[t][s] * d_(t,s)      (summed in slot order)
 * silu(g) = g / (1 + exp(-g)).  Only the selected experts' bytes are read: the
 * (token, slot) pairs are grouped by expert so each selected expert's gate, up
 * and down matrices are read once for all the tokens routed to it.
 * Stacked expert tensors: expert e of Wg/Wu (each F x H) starts at byte
 * e*F*(H/256)*144, expert e of Wd (H x F) at byte e*H*(F/256)*144.
 *   type   GGQ_Q4_K or GGQ_Q8_0; H and F multiples of 256; T*top_k <= 65536;
 *          T*H, T*top_k*F and T*top_k*H each below 2^30 (32-bit byte offsets)
 *   x      device fp32 [T][H];  y device fp32 [T][H]
 *   idx    device int32 [T][top_k], each in [0, E).  An out-of-range entry is
 *          grouped with expert 0 (so expert 0's matrices may be read for it,
 *          never anything out of bounds) and its term is left out of the sum,
 *          whatever expert 0 holds.
 *   probs  device fp32 [T][top_k]
 *   ws     device workspace >= moe_workspace_size(E, T, top_k, H, F) bytes,
 *          256-byte aligned.  On return ws holds h at byte offset
 *          moe_workspace_h_offset(E, T, top_k) as fp32 [T*top_k][F].
 * Errors: GGQ_ERR_ARG, GGQ_ERR_ALIGN, GGQ_ERR_WORKSPACE, GGQ_ERR_UNSUPPORTED.
 */
int moe_expert_gemv(int type, const void *wg, const void *wu, const void *wd, int64_t e,
                    int64_t h, int64_t f, const float *x, int64_t t, const int32_t *idx,
                    const float *probs, int top_k, float *y, void *ws, size_t ws_bytes,
                    void *stream);

/* Byte offset of the hidden-state array h inside the moe_expert_gemv workspace. */
size_t moe_workspace_h_offset(int64_t e, int64_t t, int top_k);

/*
 * moe_layer_workspace_size -- device workspace bytes moe_layer_gemv needs: the
 * GGQ_CTRL_BYTES control block, then a moe_expert_gemv workspace.  0 on bad
 * arguments.
 */
size_t moe_layer_workspace_size(int64_t e, int64_t t, int top_k, int64_t h, int64_t f);

/*
 * moe_layer_gemv -- moe_route followed by moe_expert_gemv on the same
 * arguments (README opening paragraph: the router picks a few experts per
 * token and only they take part), with identical results bit for bit: logits,
 * idx, probs and y are what the two calls would write.  For one token the
 * layer is three launches: up to 256 experts the router, then the gate/up
 * stage, each of whose workgroups makes the selection from the logits (the
 * first one also stores idx and probs), then down and combine; beyond 256
 * experts the router and the selection are one launch (the last router
 * workgroup to finish, counted in the control block, makes the selection),
 * then gate/up, then down and combine.  For 2 to 31 tokens the router and the
 * split of the tokens for the matrix-core stages share one launch.
 *   type, e, h, f, x, t, top_k, y, wg, wu, wd   as for moe_expert_gemv
 *   wr, logits, idx, probs                       as for moe_route (written)
 *   ws     device workspace >= moe_layer_workspace_size(E, T, top_k, H, F)
 *          bytes, 256-byte aligned, control block zero before the first call
 *          (every call leaves it zero; the rest may hold anything); h is at
 *          byte offset GGQ_CTRL_BYTES + moe_workspace_h_offset(E, T, top_k) on
 *          return
 * Calls that share a workspace must not overlap.  T == 0 is a no-op.
 * Errors: GGQ_ERR_ARG, GGQ_ERR_ALIGN, GGQ_ERR_WORKSPACE, GGQ_ERR_UNSUPPORTED.
 */
int moe_layer_gemv(int type, const float *wr, const void *wg, const void *wu, const void *wd,
                   int64_t e, int64_t h, int64_t f, const float *x, int64_t t, int top_k,
                   float *logits, int32_t *idx, float *probs, float *y, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * moe_gemm_workspace_size -- device workspace bytes moe_expert_gemm needs:
 * per-expert slot lists and tiles, x in bf16, h in bf16 (one row per padded
 * slot) and the per-pair down-projection outputs [T*top_k][H] fp32.  0 on bad
 * arguments.
 */
size_t moe_gemm_workspace_size(int64_t e, int64_t t, int top_k, int64_t h, int64_t f);

/*
 * moe_expert_gemm -- the routed expert feed-forward of moe_expert_gemv at
 * prompt batch (phobos-bench pp<N> through a mixture-of-experts layer): the
 * same function of the same arguments,
 *     y[t] = sum_s probs[t][s] * Wd[e] (silu(Wg[e] x_t) * (Wu[e] x_t)),
 *     e = idx[t][s],  summed in slot order,
 * computed as grouped products on the matrix cores: the (token, slot) pairs
 * are grouped by expert and each selected expert's matrices are read once per
 * 64 of its pairs.  x and h are rounded to bf16 and the weights decoded to bf16;
 * products accumulate in fp32.  Each of the three products is within
 * 8e-3 * sum |a w| of its exact value on its own (rounded) input, as for
 * quant_gemm; use moe_expert_gemv for the tighter decode tolerance.  The result
 * does not depend on the order in which pairs of one expert are processed, and
 * repeated calls give identical results.
 *   type, e, h, f, x, idx, probs, top_k, y   as for moe_expert_gemv
 *          (T*top_k <= 65536; out-of-range idx entries are grouped with
 *          expert 0 and their terms left out of the sum)
 *   ws     device workspace >= moe_gemm_workspace_size(E, T, top_k, H, F) bytes,
 *          256-byte aligned; its contents on entry do not matter
 * T == 0 is a no-op.  Errors: GGQ_ERR_ARG (also when a bf16 copy of x or h
 * would exceed 2 GiB), GGQ_ERR_ALIGN, GGQ_ERR_WORKSPACE, GGQ_ERR_UNSUPPORTED.
 */
int moe_expert_gemm(int type, const void *wg, const void *wu, const void *wd, int64_t e,
                    int64_t h, int64_t f, const float *x, int64_t t, const int32_t *idx,
                    const float *probs, int top_k, float *y, void *ws, size_t ws_bytes,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GGQ_H */
