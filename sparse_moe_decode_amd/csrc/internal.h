// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// decode / few-row path (R rows, 1 <= R <= 4)
size_t gateup_lds_bytes(int R, int H, int E);
// Bound on the static LDS of the decode kernels (the routing state).
constexpr size_t kDecodeStaticLds = 12288;
int decode_ws_size(const moe_layer_desc *d, int R);
int launch_decode_route(const moe_layer_desc *d, const float *x, int R, int32_t *ids, float *wts, float *gate,
                        void *ws, hipStream_t s);
int launch_decode_forward(const moe_layer_desc *d, const float *x, int R, float *y, const int32_t *ids_in,
                          const float *wts_in, const float *gate_in, int32_t *ids_out, float *wts_out,
                          float *gate_out, void *ws, hipStream_t s);

// b-bit block unpack (bits 2, 3, 4)
int launch_qb_unpack(int bits, const void *packed, int64_t rows, int64_t cols, float *dst, hipStream_t s);

// stable counting sort of (row, slot) pairs by expert
size_t sort_ws_bytes_tke(int64_t n, int E);
int launch_sort_by_expert(const int32_t *ids, int T, int K, int E, int32_t *counts, int32_t *offsets,
                          int32_t *perm, void *ws, hipStream_t s, int32_t *inv = nullptr, int bm = 0,
                          int max_tiles = 0, int4 *tiles = nullptr);

// prefill path (any number of rows; rows grouped by expert, MFMA GEMMs)
size_t prefill_ws_bytes(const moe_layer_desc *d, int T);
int launch_prefill_route(const moe_layer_desc *d, const float *x, int T, int32_t *ids, float *wts, float *gate,
                         void *ws, hipStream_t s);
int launch_prefill_forward(const moe_layer_desc *d, const float *x, int T, float *y, const int32_t *ids_in,
                           const float *wts_in, const float *gate_in, int32_t *ids_out, float *wts_out,
                           float *gate_out, void *ws, hipStream_t s);

}  // namespace moe
