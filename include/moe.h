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
 *     device memory and keeps no device state between calls. Its global
 *     state is host-side and mutex-guarded: a cache of occupancy queries per
 *     kernel and device, and per device one side stream with two events,
 *     created by the first prefill call outside a stream capture and kept
 *     until the process ends.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). GPU
 *     work is enqueued on it and the call returns without waiting. A prefill
 *     call (moe_forward with many rows) forks the shared expert's GEMMs onto
 *     the side stream after an event on `stream` and joins them back with a
 *     second event before its last kernel, so all of its work is still
 *     ordered after earlier work on `stream` and before later work; inside a
 *     stream capture this is a fork and join of the captured graph.
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

#define MOE_ABI_VERSION 1u

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* null/invalid argument, bad shape, T < 0, K > E, K > 16 */
    MOE_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. a size limit) */
    MOE_EWORKSPACE = -3,    /* workspace (or packer destination) too small */
    MOE_EALIGN = -4,        /* a pointer is not 16-byte aligned */
    MOE_EHIP = -5,          /* a HIP launch or runtime call failed */
    MOE_ENONFINITE = -6     /* packer: NaN/Inf input, or a block out of fp16 range */
} moe_status;

/* Weight storage formats. */
typedef enum {
    MOE_F32 = 0,            /* IEEE binary32 */
    MOE_BF16 = 1,           /* bfloat16 bit patterns (uint16) */
    MOE_Q2B32 = 2           /* 2-bit block format, see moe_q2_pack (routed experts only) */
} moe_wtype;

/*
 * One layer. Dimensions: H = hidden, E = n_experts, K = top_k, I = inter,
 * Is = shared_inter. Limits: H, I, Is multiples of 32; 1 <= K <= min(E, 16);
 * E <= 1024; H <= 8192; I, Is <= 4096.
 *
 * All weight pointers are device pointers, 16-byte aligned, row-major:
 *   router_w       [E][H]   router_t (MOE_F32 or MOE_BF16)
 *   router_bias    [E]      fp32, or NULL for no bias (added to the logits
 *                           before selection and softmax)
 *   shared_gate_w  [H]      router_t (the vector w_g)
 *   exp_gate       E stacked [I][H] matrices, expert_t
 *   exp_up         E stacked [I][H] matrices, expert_t
 *   exp_down       E stacked [H][I] matrices, expert_t
 *   sh_gate        [Is][H]  shared_t (MOE_F32 or MOE_BF16)
 *   sh_up          [Is][H]  shared_t
 *   sh_down        [H][Is]  shared_t
 * For MOE_Q2B32 experts each stacked matrix is one moe_q2_pack() result and
 * occupies moe_q2_packed_bytes(rows, cols) bytes; expert e starts at
 * e * moe_q2_packed_bytes(rows, cols). The expert dimension is outermost and
 * every expert is one contiguous byte range (the merged routed tensors of the
 * "Red Lite v0.3 streaming development" page, section "Implemented in dev1").
 *
 * renormalize: 1 = softmax over the K selected logits (the Qwen3-Next case),
 * 0 = the full softmax over all E, taken at the K selected experts.
 */
typedef struct moe_layer_desc {
    int32_t hidden, n_experts, top_k, inter, shared_inter;
    int32_t renormalize;
    int32_t router_t, expert_t, shared_t;
    int32_t reserved;                  /* must be 0 */
    const void *router_w;
    const float *router_bias;
    const void *shared_gate_w;
    const void *exp_gate, *exp_up, *exp_down;
    const void *sh_gate, *sh_up, *sh_down;
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
 * Routing only (router logits, top-K, softmax weights, shared gate).
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
 * The whole layer for T rows.
 *   x [T][H] fp32 device (in), y [T][H] fp32 device (out, overwritten).
 *   If ids_in != NULL, the routing ids_in [T][K], wts_in [T][K] and
 *   gate_in [T] (device) is used as given (wts_in/gate_in must then be
 *   non-NULL) and no routing is computed; ids outside [0, E) contribute
 *   nothing. Otherwise routing is computed and,
 *   for each of ids_out / wts_out / gate_out that is non-NULL, written out.
 * Path by T: T == 1 decode; 2 <= T <= 4 few-row (the selected experts'
 * union is read once for all rows); 5 <= T <= 12 few-row launches of three
 * rows (a remainder of one joins the last launch as four) when the layer's
 * shapes allow 4-row launches; larger T the prefill path (rows grouped by
 * expert, grouped bf16 MFMA GEMMs). The environment variable MOE_FORCE_PATH
 * (decode | fewrow | prefill) overrides the choice; decode/fewrow then run
 * in such groups (one launch when T fits one).
 */
int moe_forward(const moe_layer_desc *d, const float *x, int32_t T, float *y,
                const int32_t *ids_in, const float *wts_in, const float *gate_in,
                int32_t *ids_out, float *wts_out, float *gate_out,
                void *ws, size_t ws_bytes, void *stream);

/*
 * Prefill grouping step on its own: a stable counting sort of the T*K
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
 * 2-bit block format (MOE_Q2B32). The logical content of a [rows][cols] fp32
 * matrix (cols % 32 == 0): each run of 32 consecutive weights of a row is a
 * block with 2-bit codes c (0..3), an fp16 scale s and an fp16 minimum m;
 * the weight is fp32(c * s + m).
 * Quantizer (IEEE binary32, round to nearest even, no fused operations):
 *   lo, hi = min, max of the block;  m = fp16(lo);
 *   s = fp16((hi - float(m)) / 3);
 *   c = 0 if float(s) == 0, else clamp(nearbyint((w - float(m)) / float(s)), 0, 3).
 * Physical layout written by moe_q2_pack (little-endian):
 *   bytes [0, rows*cols/4)                 codes; weight j of block b of row r
 *                                          is at byte r*cols/4 + b*8 + j/4,
 *                                          bits 2*(j%4) .. 2*(j%4)+1
 *   bytes [rows*cols/4, rows*cols*3/8)     per block, row-major: uint16 scale
 *                                          bits then uint16 min bits
 *   then zero padding up to moe_q2_packed_bytes(rows, cols).
 */

/* Bytes of one packed matrix (a multiple of 256), or 0 if rows <= 0 or
 * cols <= 0 or cols % 32 != 0. */
size_t moe_q2_packed_bytes(int64_t rows, int64_t cols);

/* Host-only packer: src [rows][cols] fp32 (host) -> dst (host, dst_bytes >=
 * moe_q2_packed_bytes). Returns MOE_ENONFINITE if an input is NaN/Inf or a
 * block's min or scale does not fit fp16, MOE_EWORKSPACE if dst is too small. */
int moe_q2_pack(const float *src, int64_t rows, int64_t cols, void *dst, size_t dst_bytes);

/* Device unpack of one packed matrix to fp32 [rows][cols] (device), bit-exact
 * with the format definition. packed: device, 16-byte aligned. */
int moe_q2_unpack(const void *packed, int64_t rows, int64_t cols, float *dst, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
