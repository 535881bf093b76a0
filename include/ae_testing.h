/*
 * ae_testing.h -- test-only entry points of the action-expert library.
 *
 * Not part of the denoise path: these run single pieces of the fp8 e4m3
 * projection path (MolmoBot PR "Inference optimization for MolmoBot VLA",
 * Part 3: per-tensor dynamic fp8, amax -> cast -> scaled matmul; LoongForge
 * blog "How to Speed Up VLA Training Step by Step", section 7: inputs and
 * weights quantised, the product restored with both scales) on inputs a test
 * chooses, so the GPU's codes and products can be compared element by
 * element with a reference on identical e4m3 codes and scales, without the
 * amplification a whole denoise loop adds.
 *
 * Each call validates its sizes (AE_ERR_INVALID_ARGUMENT / AE_ERR_UNSUPPORTED
 * before any HIP call), allocates its own scratch, runs on `stream`, waits
 * for it and frees the scratch before returning (so, unlike ae.h, these
 * calls synchronise the host and allocate).  Pointers are device memory;
 * weights are bf16 bit patterns [K][N] row-major (y = x W).  Rows are grouped
 * into requests of T consecutive rows, each with its own activation scale.
 */
#ifndef AE_TESTING_H
#define AE_TESTING_H

#include <stdint.h>

#include "ae.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The activation quantiser of the down projection's input: x [M][K] fp32
 * (K a multiple of 64, M a multiple of T) -> codes [M][K] e4m3 bytes with
 * the request's scale; sx_row [M] = amax / 448 of the row's request (the
 * amax taken over every element of the request's T rows, floored at 1e-12),
 * each code e4m3(x * (448 / amax)) decided in fp32. */
ae_status aetest_fp8_quantize(const float* x, int M, int K, int T, uint8_t* codes,
                              float* sx_row, void* stream);

/* The adaRMS input of a QKV / gate-up product and its codes: per row
 * r = 1 / sqrt(mean(h^2) + eps), u = h r (1 + scale) + shift, then codes of
 * u as aetest_fp8_quantize does (K = D a multiple of 64). r_out [M].  T = 1
 * is the row-wise recipe (each row its own scale), which runs the one-pass
 * per-row kernel. */
ae_status aetest_fp8_norm_quantize(const float* h, int M, int D, int T, const float* scale,
                                   const float* shift, float eps, uint8_t* codes, float* sx_row,
                                   float* r_out, void* stream);

/* The down projection: y [M][N] fp32 = (codes . e4m3(W / s_w)) * sx_row * s_w
 * with s_w = amax|W| / 448 (one scale for the tensor), written to sw[0];
 * per_column = 1: the row-wise variant, s_w per output column j (amax of
 * column j), sw[0..N).  K and N multiples of 128. */
ae_status aetest_fp8_down(const uint8_t* codes, const float* sx_row, int M, int K,
                          const uint16_t* w, int N, float* y, float* sw, int per_column, void* stream);

/* The merged gate/up projection: act [M][F] fp32 = gelu_tanh(g) * u with
 * g = (codes . e4m3(Wg / s_g)) * sx_row * s_g and u likewise with W_u and its
 * own scale s_u; sw[0] = s_g, sw[1] = s_u (per_column = 1: a scale per
 * column, sw = [gate columns | up columns], 2F values).  K and 2F multiples
 * of 128. */
ae_status aetest_fp8_gate_up(const uint8_t* codes, const float* sx_row, int M, int K,
                             const uint16_t* wg, const uint16_t* wu, int F, float* act, float* sw,
                             int per_column, void* stream);

/* The merged q|k|v projection of one request of M rows, through the
 * product's own epilogue (scatter of q, and of k and v into a key-block
 * cache) with identity rotation tables (cos 1, sin 0), so the products come
 * back unrotated: q [M][Hq dh], k and v [M][Hkv dh] fp32 holding the bf16
 * values the kernel stores, each (codes . e4m3(W / s)) * sx_row * s with the
 * tensor's own scale; sw[0..2] = s_q, s_k, s_v (per_column = 1: a scale per
 * column, sw = [q columns | k columns | v columns]).
 * K and (Hq + 2 Hkv) dh multiples of 128, dh in {64, 128, 256}. */
ae_status aetest_fp8_qkv(const uint8_t* codes, const float* sx_row, int M, int K,
                         const uint16_t* wq, const uint16_t* wk, const uint16_t* wv, int Hq,
                         int Hkv, int dh, float* q, float* k, float* v, float* sw, int per_column,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AE_TESTING_H */
