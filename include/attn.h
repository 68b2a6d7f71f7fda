/*
 * attn.h - C ABI of libmoe's attention forward on AMD Instinct MI355X (gfx950): the X-Stage
 * paper's second fused workload ("X-Stage: An Overlooked Pipeline Stage for Communication-
 * Computation Overlap in DiT Inference", Section 4.3, FlashAttention-A2A, and Figure 6).
 *
 * After the first Ulysses all-to-all each GPU holds every token of its share of the heads and
 * runs full, non-causal attention (the DiT setting): O = softmax(Q K^T / sqrt(d)) V per (batch,
 * head). The page's kernel computes it tile by tile and issues each b_m x d output tile at the
 * tile boundary, before the next tile's Q-loop over all key tiles; this is that forward on one
 * GPU, each output tile stored to local memory at its boundary (the post-attention all-to-all
 * needs more than one GPU). Conventions as in moe.h: bf16 as uint16_t bits, caller-owned device
 * buffers, asynchronous on `stream`, host-side validation before any launch, no global state.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_HEAD_DIM 128      /* the head dimension this implementation supports (the page's d) */
#define ATTN_TILE_QUERIES 128  /* queries per output tile (b_m)                                  */
#define ATTN_WORKGROUPS_PER_CU 2 /* persistent workgroups per CU (one tile each at a time)       */

typedef struct attn_config {
  int32_t B;              /* batch (>= 1)                                                    */
  int32_t heads;          /* heads on this GPU (>= 1)                                         */
  int32_t M;              /* sequence length, every token (>= 1; M * d * 2 < 2^31)            */
  int32_t d;              /* head dimension: ATTN_HEAD_DIM                                    */
  int32_t num_workgroups; /* persistent grid; 0 or more than fits = one workgroup per CU      */
  int32_t reserved[3];    /* must be 0                                                        */
} attn_config;

/* Attention forward, full and non-causal, scale 1/sqrt(d) (X-Stage paper, Section 4.3).
 *   q, k, v [B, heads, M, d] bf16 in; o [B, heads, M, d] bf16 out;
 *   lse [B, heads, M] float32 out, or NULL: log(sum_j exp(q . k_j / sqrt(d))) of each query.
 * A persistent grid walks (batch, head, 128-query tile) items; each tile's output is stored at
 * the end of its loop over all key tiles. Scores and the softmax in fp32, P rounded to bf16 for
 * the second product, fp32 accumulation, O rounded to bf16 once.
 * Errors: MOE_ERR_INVALID_ARG (NULL pointer, a size below 1, reserved not 0),
 * MOE_ERR_UNSUPPORTED (d other than 128, a head larger than 2^31 bytes, more than 2^31 tiles),
 * MOE_ERR_HIP (a launch failed). */
moe_status attn_forward(const attn_config* cfg, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
