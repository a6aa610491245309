/*
 * qknr.h -- C ABI of the fused QK-Norm + RoPE prologue for AMD MI355X (gfx950).
 *
 * The operation, per token t and per head of Q [tokens, hq, head_dim] and of
 * K [tokens, hkv, head_dim] (a "row" is one head_dim vector x):
 *
 *   1. RMSNorm with a static [head_dim] weight w and one inverse-RMS scalar per
 *      row ("QK-Normed MLA: QK normalization without full key caching",
 *      abstract: RMSNorm splits into a static affine weight and a dynamic
 *      inverse-RMS scalar), applied per head (QG-MIL abstract, "per-head QK
 *      normalization"; HobbyLM abstract, grouped-query attention with per-head
 *      QK-normalization).  Q rows use wq, K rows use wk:
 *          r = 1 / sqrt(mean_j(x_j^2) + eps),   n_j = w_j * x_j * r
 *   2. Rotary position embedding of the first rotary_dim channels ("Fractional
 *      Rotation, Full Potential? Investigating Performance and Convergence of
 *      Partial RoPE", abstract: rotating only a fraction of the dimensions),
 *      pairs (i, i + rotary_dim/2), angle position_ids[t] * theta^(-2i/rotary_dim)
 *      evaluated in fp64, cos and sin rounded to fp32:
 *          y_i = n_i c_i - n_{i+h} s_i,   y_{i+h} = n_{i+h} c_i + n_i s_i,
 *          y_j = n_j for j >= rotary_dim.
 *   Fusing the two into one pass over memory is the "QK-RoPE" fusion of
 *   "Chronicals: A High-Performance Framework for LLM Fine-Tuning with 3.51x
 *   Speedup over Unsloth" (abstract, contribution (1)); position ids restart
 *   at 0 at each document boundary of a packed buffer (same abstract,
 *   contribution (4): Best-Fit-Decreasing sequence packing).
 *
 * Conventions shared by every entry point:
 *   - All tensors are dense, row-major and live in device memory; the caller
 *     allocates and owns them.  The library allocates no device memory; on
 *     the host it only caches, per device, how many workgroups stay resident.
 *   - q, k, the weights, the outputs and the weight gradients share one
 *     element type (qknr_dtype); arithmetic is fp32 with one round-to-nearest-
 *     even rounding at each store.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream).  The return value reports argument validation (done on the host
 *     before any HIP call; nothing is launched on error) and the launch status.
 *     Faults during execution surface at the caller's next synchronisation.
 *   - Tensor pointers must be 16-byte aligned; position_ids 4-byte aligned.
 *   - head_dim is 64, 128 or 256; rotary_dim is a multiple of 16 in
 *     [0, head_dim] (0 gives plain per-head RMSNorm); hq >= 1, hkv >= 1;
 *     eps > 0 and finite; theta > 0 and finite.
 *   - tokens == 0 is a valid no-op (pointers are not inspected).
 *   - position_ids may hold any int32 value (any order; restarts per document).
 */
#ifndef QKNR_H
#define QKNR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qknr_status {
    QKNR_OK = 0,
    QKNR_ERR_INVALID_ARG = 1,  /* null pointer, negative size, eps/theta out of range */
    QKNR_ERR_UNSUPPORTED = 2,  /* head_dim or rotary_dim outside the supported set */
    QKNR_ERR_MISALIGNED = 3,   /* a pointer is not 16-byte (positions: 4-byte) aligned */
    QKNR_ERR_WORKSPACE = 4,    /* workspace null or smaller than required */
    QKNR_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed */
} qknr_status;

typedef enum qknr_dtype {
    QKNR_F32 = 0,
    QKNR_BF16 = 1
} qknr_dtype;

/*
 * Forward: q_out = RoPE(RMSNorm_wq(q)), k_out = RoPE(RMSNorm_wk(k)).
 *   q            [tokens, hq, head_dim]           input
 *   k            [tokens, hkv, head_dim]          input
 *   wq, wk       [head_dim] each                  norm weights
 *   position_ids [tokens] int32                   rotary position of each token
 *   eps          added to the mean square inside the root (used as fp32)
 *   theta        RoPE base; frequencies theta^(-2i/rotary_dim), i < rotary_dim/2
 *   q_out, k_out same shapes as q, k.  q_out may be q itself and k_out may be
 *                k itself (in place); any other overlap is undefined.
 */
qknr_status qknr_fwd(const void *q, const void *k, const void *wq, const void *wk,
                     const int32_t *position_ids, int64_t tokens, int32_t hq,
                     int32_t hkv, int32_t head_dim, int32_t rotary_dim, float eps,
                     double theta, qknr_dtype dtype, void *q_out, void *k_out,
                     void *stream);

/*
 * Bytes of device workspace qknr_bwd needs for these sizes (per-workgroup
 * partial sums of the weight gradients).  Pure host function; 0 for
 * tokens <= 0 or unsupported sizes.  The value does not depend on rotary_dim.
 */
size_t qknr_bwd_workspace_bytes(int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                                qknr_dtype dtype);

/*
 * Backward of the forward above for L = <dq_out, q_out> + <dk_out, k_out>:
 *   dq_out, dk_out  upstream gradients, shapes of q and k
 *   dq, dk          gradients w.r.t. q and k (written).  dq may be dq_out or q
 *                   itself and dk may be dk_out or k itself; other overlap is
 *                   undefined.
 *   dwq, dwk        [head_dim] gradients w.r.t. wq and wk, summed over all rows
 *                   of their tensor and OVERWRITTEN (not accumulated).
 *   workspace       device memory of at least qknr_bwd_workspace_bytes(...)
 *                   bytes, 16-byte aligned; contents need no initialisation and
 *                   are clobbered.  Calls that may run concurrently (other
 *                   streams) need separate workspaces.
 * The inverse RMS of every row is recomputed, not stored by the forward.  The
 * weight gradients are summed per workgroup in registers and LDS, then a
 * second small kernel adds the workgroup partials in a fixed order; no
 * floating-point atomics, so results are bit-identical from run to run on a
 * given device.
 */
qknr_status qknr_bwd(const void *q, const void *k, const void *wq, const void *wk,
                     const int32_t *position_ids, int64_t tokens, int32_t hq,
                     int32_t hkv, int32_t head_dim, int32_t rotary_dim, float eps,
                     double theta, qknr_dtype dtype, const void *dq_out,
                     const void *dk_out, void *dq, void *dk, void *dwq, void *dwk,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Static, human-readable name of a status code. */
const char *qknr_status_string(qknr_status s);

/*
 * qknr_bwd without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Arguments and results as qknr_bwd; the weight-gradient
 * partials live in a static device array of the library (2 MiB per GPU, held
 * until the process ends), which covers every size qknr_bwd supports: a size
 * whose partials would not fit returns QKNR_ERR_WORKSPACE.  The call allocates
 * nothing; its first call on a device looks up the array's address there.
 * Every call on a GPU shares that GPU's array, so calls that may overlap on
 * one GPU (other streams, other host threads) race: serialise them, or use
 * qknr_bwd with separate workspaces.
 */
qknr_status qknr_bwd_noalloc(const void *q, const void *k, const void *wq, const void *wk,
                             const int32_t *position_ids, int64_t tokens, int32_t hq,
                             int32_t hkv, int32_t head_dim, int32_t rotary_dim, float eps,
                             double theta, qknr_dtype dtype, const void *dq_out,
                             const void *dk_out, void *dq, void *dk, void *dwq, void *dwk,
                             void *stream);

/* ---- Extended entry points: strided views, paged K output, conventions ------
 *
 * The same operation as qknr_fwd / qknr_bwd with three kinds of options.
 *
 * Layout (qknr_layout; NULL means every tensor dense).  Each tensor is a
 * sequence of token slices; a token's heads are contiguous (head stride =
 * head_dim) and consecutive tokens are `*_stride` ELEMENTS apart.  This takes
 * Q and K as views of a fused projection output, e.g. qkv [tokens,
 * (hq + 2 hkv) * head_dim]: q = qkv, k = qkv + hq * head_dim, both strides
 * (hq + 2 hkv) * head_dim, and q_out = q, k_out = k for in place.  Every stride
 * is at least heads * head_dim of its tensor, at most 2^40, and a multiple of
 * 16 bytes' worth of elements (4 for fp32, 8 for bf16).  Outputs may coincide
 * with their own input (same pointer and stride); other overlap is undefined.
 *
 * Paged K output (forward only).  With k_out_slots (device, [tokens] int64),
 * token t's K heads are written at row k_out_slots[t] of k_out, i.e. at
 * k_out + k_out_slots[t] * k_out_stride, instead of row t.  k_out_rows (>= 1)
 * is the number of rows k_out holds: a slot outside [0, k_out_rows) skips that
 * token's K write (a negative slot marks padding), so a bad slot is never
 * written.  The slots live in device memory and are not read on the host, so
 * such a slot gives no status code; two tokens must not share a slot.  This
 * writes the rotated keys straight into a KV cache laid out [blocks,
 * block_size, hkv, head_dim] (slot = block * block_size + offset, k_out_stride =
 * hkv * head_dim, k_out_rows = blocks * block_size), for decode steps.  Q is
 * written at row t as usual.
 *
 * Convention flags (bitwise OR of qknr_flag), for the conventions the RoPE
 * literature leaves open (Rope to Nope and Back Again, abstract: RoPE and its
 * extensions; Partial RoPE abstract: rotated fraction of the head):
 *   QKNR_FLAG_INTERLEAVED    pairs (2i, 2i+1) for i < rotary_dim/2:
 *                              y_2i = n_2i c_i - n_2i+1 s_i,  y_2i+1 = n_2i+1 c_i + n_2i s_i
 *   QKNR_FLAG_FREQ_HEAD_DIM  frequencies theta^(-2i/head_dim) (i < rotary_dim/2)
 *                            instead of theta^(-2i/rotary_dim)
 *   QKNR_FLAG_NO_WEIGHT      parameter-free norm, w = 1: wq and wk are not read
 *                            (may be NULL); the backward neither reads nor
 *                            writes dwq, dwk (may be NULL)
 *   QKNR_FLAG_LAYERNORM      QK-LayerNorm ("Nyonic Technical Report", abstract:
 *                            RoPE with QK-LayerNorm): the row mean m is
 *                            subtracted first,
 *                              r = 1 / sqrt(mean_j((x_j - m)^2) + eps),
 *                              n_j = w_j (x_j - m) r
 *   QKNR_FLAG_HEAD_WEIGHTS   per-head weights: wq is [hq, head_dim] and wk
 *                            [hkv, head_dim] (biases and all their gradients
 *                            likewise) instead of one [head_dim] vector each.
 *                            qknr_fwd_opt / qknr_bwd_opt only.
 * Unknown flag bits are rejected with QKNR_ERR_INVALID_ARG.
 */
typedef enum qknr_flag {
    QKNR_FLAG_INTERLEAVED = 1,
    QKNR_FLAG_FREQ_HEAD_DIM = 2,
    QKNR_FLAG_NO_WEIGHT = 4,
    QKNR_FLAG_LAYERNORM = 8,
    QKNR_FLAG_HEAD_WEIGHTS = 16
} qknr_flag;

typedef struct qknr_layout {
    int64_t q_stride;            /* q */
    int64_t k_stride;            /* k */
    int64_t q_out_stride;        /* q_out (forward) or dq (backward) */
    int64_t k_out_stride;        /* k_out (forward) or dk (backward) */
    int64_t dq_out_stride;       /* dq_out (backward only) */
    int64_t dk_out_stride;       /* dk_out (backward only) */
    const int64_t *k_out_slots;  /* forward only; NULL = row t.  Must be NULL in the backward. */
    int64_t k_out_rows;          /* rows of k_out; >= 1 with k_out_slots, else unused */
} qknr_layout;

/* Forward with layout and flags; other arguments as qknr_fwd.  With slots,
 * k_out must not overlap q or k; k_out_rows < 1 with slots gives
 * QKNR_ERR_INVALID_ARG. */
qknr_status qknr_fwd_ex(const void *q, const void *k, const void *wq, const void *wk,
                        const int32_t *position_ids, int64_t tokens, int32_t hq,
                        int32_t hkv, int32_t head_dim, int32_t rotary_dim, float eps,
                        double theta, qknr_dtype dtype, uint32_t flags,
                        const qknr_layout *layout, void *q_out, void *k_out, void *stream);

/* Backward with layout and flags; other arguments as qknr_bwd (same workspace
 * size).  Gradients are those of the forward with the same flags. */
qknr_status qknr_bwd_ex(const void *q, const void *k, const void *wq, const void *wk,
                        const int32_t *position_ids, int64_t tokens, int32_t hq,
                        int32_t hkv, int32_t head_dim, int32_t rotary_dim, float eps,
                        double theta, qknr_dtype dtype, uint32_t flags,
                        const qknr_layout *layout, const void *dq_out, const void *dk_out,
                        void *dq, void *dk, void *dwq, void *dwk, void *workspace,
                        size_t workspace_bytes, void *stream);

/* ---- Entry points with every option ------------------------------------------
 *
 * The same operation as qknr_fwd_ex / qknr_bwd_ex, plus the options that RoPE
 * and QK-norm variants in the literature add:
 *   - biases: n_j = w_j x_j r + b_j (or with the LayerNorm centring), one [head_dim]
 *     bias per tensor, added after the weight and before the rotation;
 *   - a caller frequency table: the rotary_dim/2 frequencies theta_i replace
 *     theta^(-2i/d) (RoPE "extensions" such as position interpolation or
 *     NTK/YaRN-style rescaling change these frequencies: Rope to Nope and Back
 *     Again, abstract); theta is then unused but must still be valid;
 *   - an attention factor a: c_i = fp32(a cos phi_i), s_i = fp32(a sin phi_i),
 *     the product taken in fp64 before the fp32 rounding; unrotated channels
 *     are not scaled.
 *   - norm groups: norm_group_q consecutive q heads (norm_group_k k heads) of a
 *     token share the mean and the inverse RMS, taken over their
 *     norm_group * head_dim values ("QK-Normed MLA: QK normalization without
 *     full key caching", abstract: one dynamic inverse-RMS scalar per token and
 *     head group; a group of every head is the layerwise QK-Norm of the
 *     "SwiftQK" abstract); RoPE still rotates each head on its own.
 * Norm groups above 1 or QKNR_FLAG_HEAD_WEIGHTS run the norm-group kernels: a
 * wave-level one when every group lies within one stage of 2 * 64 / (head_dim /
 * (16 / elem_bytes)) consecutive rows of a token (its hq q rows, then its hkv k
 * rows), else one that keeps whole tokens in a workgroup.  Both need
 * (hq + hkv) * head_dim * elem_bytes <= 32 KiB in the forward and, in the
 * backward, 24 KiB (bf16) or 16 KiB (fp32); otherwise the call returns
 * QKNR_ERR_UNSUPPORTED.  With k_out_slots it writes
 * K as qknr_fwd_ex does (decode steps with group norms into a paged cache).
 * A zero-filled qknr_options (or a NULL pointer) means: dense tensors, no flags,
 * no biases, the theta formula, no attention factor, per-head norm; results
 * are then bit-identical to qknr_fwd / qknr_bwd.
 */
typedef struct qknr_options {
    uint32_t flags;               /* qknr_flag bits */
    const qknr_layout *layout;    /* NULL: dense tensors */
    const void *bq, *bk;          /* [head_dim] device biases of q's dtype, 16-byte
                                     aligned; both or neither (NULL: none).  Read
                                     by the forward only. */
    const double *inv_freq;       /* HOST array of rotary_dim/2 finite frequencies,
                                     read during the call; NULL: the theta formula */
    double attention_factor;      /* finite; 0 means 1 (no scaling) */
    int32_t norm_group_q;         /* q heads sharing one inverse RMS (and mean); must
                                     divide hq; 0 or 1: per head; hq: the layerwise
                                     norm over the token's whole q vector */
    int32_t norm_group_k;         /* the same for k and hkv */
} qknr_options;

/* Forward with options; other arguments as qknr_fwd_ex.  Errors as
 * qknr_fwd_ex, plus QKNR_ERR_INVALID_ARG for a single bias, a non-finite
 * frequency or factor, and QKNR_ERR_MISALIGNED for misaligned biases.
 * head_dim, rotary_dim and dtype are checked (QKNR_ERR_UNSUPPORTED) before the
 * frequency table is read, so it is never read past rotary_dim / 2 entries of
 * a supported rotary_dim. */
qknr_status qknr_fwd_opt(const void *q, const void *k, const void *wq, const void *wk,
                         const int32_t *position_ids, int64_t tokens, int32_t hq, int32_t hkv,
                         int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                         qknr_dtype dtype, const qknr_options *options, void *q_out, void *k_out,
                         void *stream);

/* Bytes of workspace qknr_bwd_opt needs with these options (at least
 * qknr_bwd_workspace_bytes; more with norm groups or per-head weights).  Pure
 * host function; 0 for invalid or unsupported arguments. */
size_t qknr_bwd_opt_workspace_bytes(int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                                    int32_t rotary_dim, qknr_dtype dtype,
                                    const qknr_options *options);

/* Backward of qknr_fwd_opt with the same options.  The biases do not enter dq
 * or dk; dbq, dbk (the weights' shape, both or neither, 16-byte aligned)
 * receive the bias gradients, sums over rows of R^T dy, overwritten, when
 * non-NULL.  Workspace: qknr_bwd_opt_workspace_bytes. */
qknr_status qknr_bwd_opt(const void *q, const void *k, const void *wq, const void *wk,
                         const int32_t *position_ids, int64_t tokens, int32_t hq, int32_t hkv,
                         int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                         qknr_dtype dtype, const qknr_options *options, const void *dq_out,
                         const void *dk_out, void *dq, void *dk, void *dwq, void *dwk, void *dbq,
                         void *dbk, void *workspace, size_t workspace_bytes, void *stream);

/* ---- Best-Fit-Decreasing sequence packing -------------------------------------
 *
 * The data step that produces the packed position ids: documents are packed
 * into buffers of `capacity` tokens with Best-Fit Decreasing ("Chronicals: A
 * High-Performance Framework for LLM Fine-Tuning with 3.51x Speedup over
 * Unsloth", abstract, contribution (4): BFD sequence packing in place of
 * padding).  Tie-breaks (the abstract fixes none): documents in order of
 * length, longest first, equal lengths in input order; each into the open bin
 * with the least room that fits it, the lowest bin index among equals; else a
 * new bin, numbered in opening order.  Bin b occupies tokens [b * capacity,
 * (b + 1) * capacity) of the packed buffers; its documents follow each other in
 * placement order and the rest of the bin, if any, is one filler segment.
 *
 *   lengths       [ndocs] int32, device: document lengths, each in [1, capacity]
 *   doc_start     [ndocs] int32, device, written: first token of each document
 *   position_ids  [max_bins * capacity] int32, device, written for the first
 *                 bins * capacity tokens: 0, 1, ... from the start of every
 *                 segment (document or filler); the rest is left alone
 *   cu_seqlens    [ndocs + max_bins + 1] int32, device, written: the first token
 *                 of every segment in token order, then bins * capacity
 *   counts        [2] int32, device, written: {bins, segments}
 *   status        [1] int32, device, written: 0 ok; 1 more than max_bins bins
 *                 would be needed; 2 a length outside [1, capacity].  With a
 *                 non-zero status counts are {0, 0} and the other outputs are
 *                 unspecified (nothing is written past their extents).
 * 0 <= ndocs <= 2^22, capacity >= 1, 1 <= max_bins <= 4096, max_bins * capacity
 * < 2^31; int32 arrays 4-byte aligned; workspace of qknr_bfd_workspace_bytes
 * (16-byte aligned, no initialisation needed).  The sort is one workgroup's
 * bitonic sort and the placement one wave scanning the open bins per document:
 * sized for the documents of a batch (thousands), not millions.
 */
size_t qknr_bfd_workspace_bytes(int32_t ndocs, int32_t max_bins);

qknr_status qknr_bfd_pack(const int32_t *lengths, int32_t ndocs, int32_t capacity,
                          int32_t max_bins, int32_t *doc_start, int32_t *position_ids,
                          int32_t *cu_seqlens, int32_t *counts, int32_t *status, void *workspace,
                          size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QKNR_H */
