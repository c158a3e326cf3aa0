/*
 * csmla_indexer.h — C ABI of the lightning-indexer top-k producer for AMD
 * Instinct MI355X (gfx950), the step that writes the cmp_sparse_indices the
 * attention in csmla.h consumes.
 *
 * The operation (QuantLightningIndexerV2 page, 功能说明 formula and steps
 * 1-3), for quant_mode 1 (fp8 e4m3 query and key, fp32 dequant scales, fp32
 * weights; 约束说明 for Ascend 950): for query row t with g index heads and
 * each compressed index key s the row may see,
 *
 *     score[t, s] = sum_h W[t, h] * ReLU(scale_q[t, h] * scale_k[s] * (q[t, h, :] . k[s, :]))
 *
 * and sparse_indices[t, :] holds the key positions of the topk largest
 * scores.  Readings of what the page leaves open:
 *   - key positions are counted within the batch (0 = the batch's first
 *     compressed key), as the attention's cmp_sparse_indices expects;
 *   - a row sees keys as the attention page's right-down causal cmp mask
 *     says: with L = n * cmp_ratio + cmp_residual_k (n = the batch's key
 *     count) row i of S1 sits at p = L - S1 + i and, under mask_mode 3, sees
 *     the first floor((p + 1) / cmp_ratio) keys (clamped to [0, n]);
 *     mask_mode 0 sees all n;
 *   - equal scores prefer the lower position; the chosen positions are
 *     written in ascending order and the rest of the row is -1 (a row that
 *     sees fewer than topk keys lists them all);
 *   - query rows past seqused_q are all -1 (约束说明, TND padding).
 * Scores are ranked in float32.  The dequant scales must be finite and >= 0
 * (they scale a ReLU argument; the kernel applies them outside the ReLU).
 *
 * Call flow, as for the attention: csmla_indexer_plan() on the host (the
 * counterpart of QuantLightningIndexerV2Metadata, 参数说明 metadata: the work
 * split), then csmla_indexer_forward() enqueues two kernels on the caller's
 * stream.  Conventions are those of csmla.h: plain C types, caller-owned
 * device memory, no allocation, no synchronisation, csmla_status results
 * and csmla_last_error() for the message.
 */
#ifndef CSMLA_INDEXER_H
#define CSMLA_INDEXER_H

#include "csmla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Words of the indexer plan (host int32). */
#define CSMLA_INDEXER_METADATA_WORDS 32

/* Shapes and attributes (QuantLightningIndexerV2, 参数说明); host values.
 * Field order is part of the ABI. */
typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t g;           /* query heads (N of query), 1..64 (约束说明) */
  int32_t n2;          /* key heads: must be 1 (约束说明) */
  int32_t d;           /* head width: must be 128 */
  int32_t layout_q;    /* CSMLA_LAYOUT_BSND or CSMLA_LAYOUT_TND */
  int32_t layout_k;    /* CSMLA_LAYOUT_BSND, _TND or _PA_BBND */
  int32_t q_s;         /* BSND query: S1 (rows per batch); TND: ignored */
  int32_t t1;          /* rows of query: TND T, BSND B * S1 */
  int32_t k_s;         /* BSND key: S (dim 1 of key); TND key: rows of key; PA: ignored */
  int32_t block_size;  /* PA: keys per block, 1..1024 */
  int32_t num_blocks;  /* PA: dim 0 of key */
  int32_t table_cols;  /* PA: dim 1 of block_table */
  int32_t topk;        /* 1..8192 (约束说明) */
  int32_t mask_mode;   /* 0 (every key) or 3 (right-down causal over compressed keys) */
  int32_t cmp_ratio;   /* 1..128 */
  int32_t quant_mode;  /* must be 1 (fp8 e4m3 + fp32 scales); 2..5 are CSMLA_ERR_UNSUPPORTED */
} csmla_indexer_problem;

/* Host copies of the length tensors; any pointer may be NULL (the planner
 * then sizes the work from the shapes).  They must hold the values the device
 * tensors hold: rows or keys past what the plan covers are not scored. */
typedef struct {
  const int32_t* cu_seqlens_q;   /* [B+1] (TND query) */
  const int32_t* seqused_q;      /* [B] */
  const int32_t* cu_seqlens_k;   /* [B+1] (TND key) */
  const int32_t* seqused_k;      /* [B] */
  const int32_t* cmp_residual_k; /* [B] */
} csmla_indexer_host_lengths;

/* Device pointers; contiguous row-major tensors in the page's layouts.
 *   query                 fp8 e4m3 bytes [t1, g, 128]  (BSND [B, S1, g, 128] is the same memory)
 *   key                   fp8 e4m3 bytes: PA [blocks, block_size, 1, 128]; TND [rows, 1, 128];
 *                         BSND [B, S, 1, 128]
 *   weights               f32 [t1, g]
 *   query_dequant_scale   f32 [t1, g]
 *   key_dequant_scale     f32: PA [blocks, block_size]; TND [rows]; BSND [B, S]
 *   cu_seqlens_q          int32 [B+1]: required for TND query, must be NULL for BSND
 *   cu_seqlens_k          int32 [B+1]: required for TND key, must be NULL otherwise
 *   seqused_q             int32 [B] or NULL (rows per batch actually used)
 *   seqused_k             int32 [B]: required for PA, optional for BSND (default S), NULL for TND
 *   cmp_residual_k        int32 [B] or NULL (0): 0 <= value < cmp_ratio
 *   block_table           int32 [B, table_cols] (PA)
 *   sparse_indices        int32 [t1, 1, topk] output
 *   workspace             device scratch of the size the plan reports, 256-byte aligned; after
 *                         the call it holds the float32 scores, row t at t * stride floats
 *                         (stride = metadata word 9), valid for the keys row t sees.
 *                         Calls that overlap in time must not share it. */
typedef struct {
  const void*    query;
  const void*    key;
  const float*   weights;
  const float*   query_dequant_scale;
  const float*   key_dequant_scale;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* seqused_q;
  const int32_t* seqused_k;
  const int32_t* cmp_residual_k;
  const int32_t* block_table;
  int32_t*       sparse_indices;
  void*          workspace;
  size_t         workspace_bytes;
} csmla_indexer_tensors;

/* Words the plan needs: CSMLA_INDEXER_METADATA_WORDS. */
size_t csmla_indexer_metadata_words(void);

/* Host-side check against the page's constraints (QuantLightningIndexerV2,
 * 约束说明 for Ascend 950): query N in [1, 64], key N = 1, topk in [1, 8192],
 * the layouts and which length tensors they take (参数说明), block sizes
 * 1..1024, cmp_ratio 1..128, mask_mode 0 or 3, no empty tensors.
 * CSMLA_ERR_UNSUPPORTED for quant_mode != 1 and d != 128. */
csmla_status csmla_indexer_validate(const csmla_indexer_problem* problem);

/* Work split, the counterpart of QuantLightningIndexerV2Metadata.  Host only.
 *   metadata         host int32[metadata_words] (>= CSMLA_INDEXER_METADATA_WORDS); written
 *   workspace_bytes  host; written: the device scratch the forward needs (> 0) */
csmla_status csmla_indexer_plan(const csmla_indexer_problem* problem, const csmla_indexer_host_lengths* lengths,
                                int32_t* metadata, size_t metadata_words, size_t* workspace_bytes);

/* The indexer (QuantLightningIndexerV2, 参数说明 inputs; output sparse_indices).
 *   metadata   host int32 plan from csmla_indexer_plan for this problem (required)
 *   stream     hipStream_t as void*
 * Writes sparse_indices (and the scores into the workspace) on `stream`. */
csmla_status csmla_indexer_forward(const csmla_indexer_problem* problem, const csmla_indexer_tensors* tensors,
                                   const int32_t* metadata, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSMLA_INDEXER_H */
