/*
 * moe.h - C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer library.
 *
 * The layer (Red Lite "Architecture" page, section "Qwen3-Next shape"; the
 * routing step of "Research notes, October 2026", section 1, "Metal"):
 *
 *   l_e   = W_r[e] . x (+ b_e)                      router logits, e < E
 *   ids   = the K experts with the largest l, ordered by (l desc, id asc)
 *   w_k   = exp(l_ids[k] - l_max) / sum_j exp(l_ids[j] - l_max)   (renormalized)
 *   g     = 1 / (1 + exp(-w_g . x))                 shared-expert gate
 *   h^e   = silu(G_e x) * (U_e x),  silu(a) = a / (1 + exp(-a))
 *   y     = sum_k w_k D_ids[k] h^ids[k] + g * D_s h^s
 *
 * Every call is per row of x and rows are independent. y is overwritten.
 *
 * Conventions for every entry point:
 *   - All pointers are raw. "device" means memory of the current HIP device
 *     (hipMalloc or a framework allocator), "host" means ordinary CPU memory.
 *   - The caller owns every buffer; the library never allocates or frees
 *     device memory and keeps no device state between calls. Its only
 *     global state is a host-side, mutex-guarded memo of occupancy queries
 *     (workgroups a kernel keeps resident per device), which does not change
 *     results.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *     GPU work of a call is enqueued on it, in order, and the call returns
 *     without waiting. Calls on different streams with different workspaces
 *     are independent.
 *   - Arguments are validated on the host before any launch; a failed check
 *     returns a negative moe_status and enqueues nothing. Device-side faults
 *     surface at the caller's next synchronization.
 *   - Device inputs are not checked for finiteness; non-finite inputs give
 *     undefined outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3u

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* null/invalid argument, bad shape, T < 0, K > E, K > 16 */
    MOE_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. a size limit) */
    MOE_EWORKSPACE = -3,    /* workspace (or packer destination) too small */
    MOE_EALIGN = -4,        /* a pointer is not 16-byte aligned */
    MOE_EHIP = -5,          /* a HIP launch or runtime call failed */
    MOE_ENONFINITE = -6     /* packer: NaN/Inf input, or a block out of fp16 range */
} moe_status;

/* How router_bias enters the routing. */
typedef enum {
    MOE_BIAS_SELECT_AND_WEIGH = 0,  /* l_e + b_e for the selection and the softmax weights */
    MOE_BIAS_SELECT_ONLY = 1        /* l_e + b_e for the selection; weights from the unbiased l_e */
} moe_bias_mode;

/* Weight storage formats. */
typedef enum {
    MOE_F32 = 0,            /* IEEE binary32 */
    MOE_BF16 = 1,           /* bfloat16 bit patterns (uint16) */
    MOE_Q2B32 = 2,          /* 2-bit block format, see moe_qb_pack (routed experts only) */
    MOE_Q3B32 = 3,          /* 3-bit block format, see moe_qb_pack (routed experts only) */
    MOE_Q4B32 = 4           /* 4-bit block format, see moe_qb_pack (routed experts only) */
} moe_wtype;

/*
 * One layer. Dimensions: H = hidden, E = n_experts, K = top_k, I = inter,
 * Is = shared_inter. Limits: H, I, Is multiples of 32; 1 <= K <= min(E, 16);
 * E <= 1024; H <= 8192; I, Is <= 4096.
 *
 * All weight pointers are device pointers, 16-byte aligned, row-major:
 *   router_w       [E][H]   router_t (MOE_F32 or MOE_BF16)
 *   router_bias    [E]      fp32, or NULL for no bias; bias_mode says whether
 *                           it enters the softmax weights too (see below)
 *   shared_gate_w  [H]      router_t (the vector w_g)
 *   exp_gate       E stacked [I][H] matrices, expert_t
 *   exp_up         E stacked [I][H] matrices, expert_t
 *   exp_down       E stacked [H][I] matrices, expert_t
 *   sh_gate        [Is][H]  shared_t (MOE_F32 or MOE_BF16)
 *   sh_up          [Is][H]  shared_t
 *   sh_down        [H][Is]  shared_t
 * For the b-bit block formats (MOE_Q2B32, MOE_Q3B32, MOE_Q4B32: b = 2, 3, 4)
 * each stacked matrix is one moe_qb_pack(b, ...) result and occupies
 * moe_qb_packed_bytes(b, rows, cols) bytes; expert e starts at
 * e * moe_qb_packed_bytes(b, rows, cols). The expert dimension is outermost and
 * every expert is one contiguous byte range (the merged routed tensors of the
 * "Red Lite v0.3 streaming development" page, section "Implemented in dev1").
 *
 * renormalize: 1 = softmax over the K selected logits (the Qwen3-Next case),
 * 0 = the full softmax over all E, taken at the K selected experts.
 *
 * bias_mode (with router_bias): MOE_BIAS_SELECT_AND_WEIGH adds b_e to the
 * logits for the selection and the weights (a skewed router);
 * MOE_BIAS_SELECT_ONLY adds it for the selection only and weighs the chosen
 * experts by their unbiased logits: the opt-in cache-aware routing
 * z + lambda * Delta * cached of "Research notes, October 2026", section 4,
 * with router_bias[e] = lambda * Delta * cached_e (cached_e = 1 for experts
 * resident in the caller's expert cache, else 0).
 *
 * Multi-layer stacks ("Architecture" page, "Qwen3-Next shape": 48 MoE layers,
 * each preceded by an RMS norm; RMS_NORM+SCALE and the tail fused into the
 * MoE step, "Research notes, October 2026", section 4, MoE-fusions row):
 *   norm_w    [H] fp32 gamma (device), or NULL: the layer's input u is x.
 *             Otherwise, per row, r = 1 / sqrt(sum_h x_h^2 / H + eps) in
 *             double and u_h = fp32(x_h * r * gamma_h); routing and experts
 *             read u.
 *   norm_eps  eps of that norm (fp32, >= 0).
 *   residual  1: y = x + MoE(u) (x un-normalized); 0: y = MoE(u).
 */
typedef struct moe_layer_desc {
    int32_t hidden, n_experts, top_k, inter, shared_inter;
    int32_t renormalize;
    int32_t router_t, expert_t, shared_t;
    int32_t bias_mode;                 /* moe_bias_mode */
    const void *router_w;
    const float *router_bias;
    const void *shared_gate_w;
    const void *exp_gate, *exp_up, *exp_down;
    const void *sh_gate, *sh_up, *sh_down;
    const float *norm_w;               /* pre-MoE RMS norm gamma [H], or NULL */
    float norm_eps;
    int32_t residual;                  /* 0 or 1 */
    int64_t reserved;                  /* must be 0 */
} moe_layer_desc;

/* MOE_ABI_VERSION of the loaded library. */
uint32_t moe_abi_version(void);

/* Static text for a moe_status value. */
const char *moe_strerror(int status);

/*
 * Bytes of device workspace moe_route / moe_forward need for T rows (0 on an
 * invalid descriptor). The workspace needs no initialization and holds no
 * state between calls; calls that run at the same time (different streams)
 * need different workspaces.
 */
size_t moe_workspace_bytes(const moe_layer_desc *d, int32_t T);

/*
 * Routing only (router logits, top-K, softmax weights, shared gate): the
 * single routing step of "Research notes, October 2026", section 1 ("Metal"
 * bullet: router, top-k and shared gate computed together), with the tie
 * rule (lower expert id first) that settles the exact router tie reported on
 * the "Red Lite dev18" page, section "Scope boundary".
 *   x     [T][H]  fp32 device, 16-byte aligned
 *   ids   [T][K]  int32 device (out), ordered by logit desc, id asc
 *   wts   [T][K]  fp32 device (out)
 *   gate  [T]     fp32 device (out)
 *   ws    device workspace of ws_bytes >= moe_workspace_bytes(d, T)
 * Logits are accumulated in double so that the selection is exact up to
 * summation order. T == 0 is a no-op returning MOE_OK.
 */
int moe_route(const moe_layer_desc *d, const float *x, int32_t T,
              int32_t *ids, float *wts, float *gate,
              void *ws, size_t ws_bytes, void *stream);

/*
 * The whole layer for T rows (the Qwen3-Next MoE block of the "Architecture"
 * page, section "Qwen3-Next shape"; the shared expert as one more slot of
 * the expert pass and the weighted reduce of "Research notes, October 2026",
 * sections 1 and 4; several rows reading each selected expert once: the
 * same page, section 1, MTP "Verify" bullet; prefill chunks: the "DwarfStar
 * Red Lite" guide, section "Chat defaults").
 *   x [T][H] fp32 device (in), y [T][H] fp32 device (out, overwritten).
 *   If ids_in != NULL, the routing ids_in [T][K], wts_in [T][K] and
 *   gate_in [T] (device) is used as given (wts_in/gate_in must then be
 *   non-NULL) and no routing is computed; ids outside [0, E) contribute
 *   nothing (no expert is read for them). Otherwise routing is computed and,
 *   for each of ids_out / wts_out / gate_out that is non-NULL, written out.
 * Path by T: T == 1 decode; 2 <= T <= 4 few-row (the selected experts'
 * union is read once for all rows); 5 <= T <= 12 few-row launches of three
 * rows (a remainder of one joins the last launch as four) when the layer's
 * shapes allow 4-row launches; larger T the prefill path (rows grouped by
 * expert, grouped bf16 MFMA GEMMs), in chunks of rows whose workspace stays
 * below 1.5 GiB (consecutive chunks reuse the workspace). The environment
 * variable MOE_FORCE_PATH (decode | fewrow | prefill) overrides the choice;
 * decode/fewrow then run in such groups (one launch when T fits one).
 */
int moe_forward(const moe_layer_desc *d, const float *x, int32_t T, float *y,
                const int32_t *ids_in, const float *wts_in, const float *gate_in,
                int32_t *ids_out, float *wts_out, float *gate_out,
                void *ws, size_t ws_bytes, void *stream);

/*
 * moe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The library keeps one scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU (a static device array, held until the
 * process ends) and runs moe_forward on it; this call itself allocates
 * nothing. Arguments and results are those of moe_forward. Calls whose
 * workspace (moe_workspace_bytes(d, T)) exceeds the scratch return
 * MOE_EWORKSPACE and enqueue nothing: every decode and few-row call of any
 * supported shape fits (at most 0.35 MiB), prefill calls only while their
 * workspace does (about 20 rows at hidden 2048, 512 experts, top-10). All calls on one GPU share its scratch array: calls
 * that overlap on one GPU (two streams, two host threads) race and must be
 * ordered by the caller. The scratch needs no initialization.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_forward_noalloc(const moe_layer_desc *d, const float *x, int32_t T, float *y,
                        const int32_t *ids_in, const float *wts_in, const float *gate_in,
                        int32_t *ids_out, float *wts_out, float *gate_out, void *stream);

/*
 * Prefill grouping step on its own (rows grouped by expert before the
 * batched prefill GEMMs; "DwarfStar Red Lite" guide, "Chat defaults"): a
 * stable counting sort of the T*K
 * (row, slot) pairs of ids [T][K] (device int32, values in [0, E)) by expert.
 *   counts  [E]    int32 device (out): pairs per expert
 *   offsets [E+1]  int32 device (out): exclusive prefix sum of counts
 *   perm    [T*K]  int32 device (out): pair index t*K+k, grouped by expert in
 *                  increasing expert order, increasing t*K+k within a group
 * ids outside [0, E) are skipped (their pairs are not placed).
 * ws: device workspace of at least moe_sort_workspace_bytes(T, K, E) bytes
 * (per-chunk histograms; no initialization needed).
 */
size_t moe_sort_workspace_bytes(int32_t T, int32_t K, int32_t E);
int moe_sort_by_expert(const int32_t *ids, int32_t T, int32_t K, int32_t E,
                       int32_t *counts, int32_t *offsets, int32_t *perm,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * b-bit block formats (b = 2: MOE_Q2B32, 3: MOE_Q3B32, 4: MOE_Q4B32). The
 * 32-weight block is that of the quantized matvec kernels' 32-weight chunks
 * ("Research notes, October 2026", section 4, narrow-row row); the 2-bit
 * width, fp16 scale and fp16 minimum are the layer's 2-bit configuration,
 * and the 3- and 4-bit widths stand for the higher-precision expert files
 * of the same model ("DwarfStar Red Lite" guide, the IQ3_XXS file; the
 * weight type a constant of the kernels, "Research notes", section 1).
 * Logical content of a [rows][cols] fp32 matrix (cols % 32 == 0): each run
 * of 32 consecutive weights of a row is a block with b-bit codes c
 * (0 .. 2^b - 1), an fp16 scale s and an fp16 minimum m; the weight is
 * fp32(c * s + m).
 * Quantizer (IEEE binary32, round to nearest even, no fused operations):
 *   lo, hi = min, max of the block;  m = fp16(lo);
 *   s = fp16((hi - float(m)) / (2^b - 1));
 *   c = 0 if float(s) == 0, else clamp(nearbyint((w - float(m)) / float(s)), 0, 2^b - 1).
 * Physical layout written by moe_qb_pack (little-endian), nb = cols / 32:
 *   bytes [0, rows*cols*b/8)               codes: block b' of row r holds 4b
 *                                          bytes at (r*nb + b')*4b, read as
 *                                          one little-endian integer with
 *                                          weight j at bits b*j .. b*j+b-1
 *   bytes [rows*cols*b/8, rows*cols*(b+1)/8)  per block, row-major: uint16
 *                                          scale bits then uint16 min bits
 *   then zero padding up to moe_qb_packed_bytes(b, rows, cols).
 */

/* Bytes of one packed matrix (a multiple of 256), or 0 if bits is not 2, 3
 * or 4, rows <= 0, cols <= 0 or cols % 32 != 0. */
size_t moe_qb_packed_bytes(int32_t bits, int64_t rows, int64_t cols);

/* Host-only packer (the quantizer above, applied block by block): src
 * [rows][cols] fp32 (host) -> dst (host, dst_bytes >= moe_qb_packed_bytes).
 * Returns MOE_EINVAL for a bits, shape or pointer outside the above,
 * MOE_ENONFINITE if an input is NaN/Inf or a block's min or scale does not
 * fit fp16, MOE_EWORKSPACE if dst is too small. */
int moe_qb_pack(int32_t bits, const float *src, int64_t rows, int64_t cols, void *dst, size_t dst_bytes);

/* Device unpack of one packed matrix to fp32 [rows][cols] (device), bit-exact
 * with the format definition (w = fp32(c * s + m) above). packed: device,
 * 16-byte aligned; dst: device, 16-byte aligned. Enqueued on `stream`. */
int moe_qb_unpack(int32_t bits, const void *packed, int64_t rows, int64_t cols, float *dst, void *stream);

/* The 2-bit instances: moe_qb_*(2, ...). */
size_t moe_q2_packed_bytes(int64_t rows, int64_t cols);
int moe_q2_pack(const float *src, int64_t rows, int64_t cols, void *dst, size_t dst_bytes);
int moe_q2_unpack(const void *packed, int64_t rows, int64_t cols, float *dst, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
