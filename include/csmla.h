/*
 * csmla.h — C ABI of the quantized sparse shared-KV MLA attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (QuantSparseFlashMla page, 功能说明 formula, with a per-head
 * sink logit added to the softmax):
 *
 *     O = softmax(Q K~^T * softmax_scale + sink) V~,     K~ = V~
 *
 * K~ joins the sliding-window / causal band of the original KV (ori_kv) with
 * compressed KV (cmp_kv): every causally visible compressed token (HCA), or
 * the entries of cmp_sparse_indices (CSA); with no cmp_kv it is window-only
 * attention (SWA).  All query heads share one 512-wide fp8 e4m3 KV head
 * (QuantSparseFlashMla, 约束说明: N2 = 1, D = 512).
 *
 * Call flow (QuantSparseFlashMla page, 功能说明: the metadata op runs before
 * the main op and its output is a mandatory input):
 *   1. csmla_plan()     host only: validates the problem and writes the
 *                       int32[1024] split plan plus the workspace size.
 *   2. csmla_forward()  enqueues the kernels on the caller's HIP stream.
 *
 * Conventions for every entry point
 *   - Plain C types only.  "device" pointers are HIP device memory owned by
 *     the caller; "host" pointers are read during the call only.
 *   - The library never allocates or frees memory and never synchronises:
 *     csmla_forward() is asynchronous on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream) and can be captured into a HIP graph.
 *   - Validation is synchronous and returns a csmla_status; nothing throws
 *     across the ABI.  csmla_last_error() gives a message for the calling
 *     thread's last failure.
 *   - Block-table entries and index values are not validated (as on the
 *     fused infer-attention page, 约束说明: block ids are the caller's
 *     responsibility).  An index outside [0, visible) is skipped, not an error.
 *   - Device results are NaN where an input row the method reads is NaN.
 */
#ifndef CSMLA_H
#define CSMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSMLA_ABI_VERSION 2
/* Size of the split plan (QuantSparseFlashMla, 约束说明: metadata shape [1024]). */
#define CSMLA_METADATA_WORDS 1024

typedef enum {
  CSMLA_OK = 0,
  CSMLA_ERR_INVALID_ARG = 1,      /* a value the pages' constraints reject */
  CSMLA_ERR_UNSUPPORTED = 2,      /* allowed by the pages, not built here */
  CSMLA_ERR_WORKSPACE = 3,        /* workspace missing or too small */
  CSMLA_ERR_METADATA_MISMATCH = 4,/* plan made for another problem */
  CSMLA_ERR_HIP = 5               /* a HIP runtime call failed */
} csmla_status;

/* layout_q / layout_kv (QuantSparseFlashMla, 参数说明: layout_q, layout_kv) */
enum { CSMLA_LAYOUT_BSND = 0, CSMLA_LAYOUT_TND = 1, CSMLA_LAYOUT_PA_BBND = 2 };
/* ori_mask_mode / cmp_mask_mode (QuantSparseFlashMla, 参数说明) */
enum { CSMLA_MASK_NONE = 0, CSMLA_MASK_RIGHT_DOWN_CAUSAL = 3, CSMLA_MASK_BAND = 4 };
/* KV descale granularity: one fp32 per KV row (QuantSparseFlashMla quant_mode 1,
 * per-token) or one per 64-wide slice of D (KvQuantSparseAttnSharedkv,
 * kv_quant_mode 1 per-tile with tile_size 64, here with fp32 scales). */
enum { CSMLA_KV_SCALE_PER_TOKEN = 0, CSMLA_KV_SCALE_PER_TILE64 = 1 };
/* q_dtype: fp8 e4m3 codes with fp32 q_descale (QuantSparseFlashMla), or bf16
 * without a descale (KvQuantSparseAttnSharedkv and SparseCompressedFlashAttention,
 * 参数说明: q BFLOAT16). */
enum { CSMLA_Q_FP8 = 0, CSMLA_Q_BF16 = 1 };
/* kv_dtype: rows of ori_kv / cmp_kv.
 *   CSMLA_KV_FP8        d fp8 e4m3 codes per row, fp32 descales beside (kv_scale_mode)
 *   CSMLA_KV_BF16       d bf16 values per row, no descales
 *                       (SparseCompressedFlashAttention, 参数说明: ori_kv / cmp_kv bfloat16)
 *   CSMLA_KV_PACKED640  640 bytes per row: 64 bf16 rope values, 448 e4m3 nope codes,
 *                       7 e8m0 scales (one per 64 nope columns: value = code * 2^(E - 127),
 *                       E = 255 is NaN), 57 pad bytes; the row's 512 logical columns are
 *                       rope then nope (KvQuantSparseAttnSharedkv, 约束说明: D 640;
 *                       参数说明: kv_quant_mode 1, tile_size 64, rope_head_dim 64)
 * bf16 and packed rows need q_dtype CSMLA_Q_BF16 (the pages pair them with bf16 q);
 * q's 512 columns pair with the logical columns in that order. */
enum { CSMLA_KV_FP8 = 0, CSMLA_KV_BF16 = 1, CSMLA_KV_PACKED640 = 2 };

/* Shapes and attributes; host values.  Field order is part of the ABI. */
typedef struct {
  int32_t batch;              /* B >= 1 */
  int32_t n1;                 /* query heads: 64 (SparseCompressedFlashAttention: N1 = 64) or 128
                                 (KvQuantSparseAttnSharedkv, 约束说明); 128 runs as two 64-head
                                 launches on the stream, sharing the plan and the workspace */
  int32_t n2;                 /* KV heads; must be 1 */
  int32_t d;                  /* head dim; must be 512 */
  int32_t layout_q;           /* CSMLA_LAYOUT_BSND or _TND */
  int32_t layout_kv;          /* BSND/BSND, TND/TND, BSND/PA_BBND or TND/PA_BBND */
  int32_t q_s;                /* BSND: Q_S (rows per batch); TND: ignored */
  int32_t t1;                 /* rows of q: TND T1, BSND B*Q_S */
  int32_t ori_s;              /* BSND kv: S2 (dim 1 of ori_kv); TND kv: rows of ori_kv; PA: ignored */
  int32_t cmp_s;              /* the same for cmp_kv */
  int32_t ori_block_size;     /* PA: 1..1024 */
  int32_t cmp_block_size;     /* PA: 1..1024 */
  int32_t ori_num_blocks;     /* PA: dim 0 of ori_kv */
  int32_t cmp_num_blocks;     /* PA: dim 0 of cmp_kv */
  int32_t ori_table_cols;     /* PA: dim 1 of ori_block_table */
  int32_t cmp_table_cols;     /* PA: dim 1 of cmp_block_table */
  int32_t has_cmp;            /* 0: SWA (no cmp_kv); 1: cmp_kv given */
  int32_t topk;               /* K2 = slots per row of cmp_sparse_indices; 0: no indices (HCA/SWA) */
  float   softmax_scale;      /* multiplies Q K^T before the softmax */
  int32_t cmp_ratio;          /* 1..128; must be 1 without cmp_kv */
  int32_t ori_mask_mode;      /* 0, 3 or 4 */
  int32_t cmp_mask_mode;      /* 0 or 3 */
  int32_t ori_win_left;       /* -1 (unbounded) or >= 0 (only with ori_mask_mode 4) */
  int32_t ori_win_right;      /* -1 (unbounded) or >= 0 (only with ori_mask_mode 4) */
  int32_t kv_scale_mode;      /* CSMLA_KV_SCALE_PER_TOKEN or _PER_TILE64 */
  int32_t q_descale_per_head; /* 1: q_descale [t1, n1]; 0: q_descale [t1] */
  int32_t topk_value_mode;    /* only 0: an index is a token position within its batch */
  int32_t return_softmax_lse; /* 1: write softmax_lse */
  int32_t q_dtype;            /* CSMLA_Q_FP8 or CSMLA_Q_BF16 */
  int32_t kv_dtype;           /* CSMLA_KV_FP8, CSMLA_KV_BF16 or CSMLA_KV_PACKED640 */
  int32_t ori_topk;           /* K1 = slots per row of ori_sparse_indices; 0: no ori indices (the
                                 whole window).  With them the ori keys are the listed positions
                                 in slot order that the ori mask and window admit (-1 and
                                 out-of-range slots skipped, duplicates kept); ori_topk + topk
                                 <= 1024 (QuantSparseFlashMla, 参数说明: ori_sparse_indices,
                                 ori_topk_length) */
} csmla_problem;

/* Host copies of the length tensors, used by csmla_plan to balance work.
 * Any pointer may be NULL; the planner then uses shape-derived upper bounds. */
typedef struct {
  const int32_t* cu_seqlens_q;      /* [B+1] (TND q) */
  const int32_t* seqused_q;         /* [B] */
  const int32_t* seqused_ori_kv;    /* [B] */
  const int32_t* cu_seqlens_ori_kv; /* [B+1] (TND kv) */
  const int32_t* seqused_cmp_kv;    /* [B] */
  const int32_t* cu_seqlens_cmp_kv; /* [B+1] (TND kv) */
  const int32_t* cmp_residual_kv;   /* [B] */
  const int32_t* cmp_topk_length;   /* [t1] */
  const int32_t* ori_topk_length;   /* [t1] */
} csmla_host_lengths;

/* Device pointers; contiguous row-major tensors in the pages' layouts.
 *   q                 fp8 e4m3 bytes [t1, n1, d] (bf16 [t1, n1, d] with CSMLA_Q_BF16)
 *                     (BSND [B, Q_S, n1, d] is the same memory)
 *   q_descale         f32 [t1, n1] or [t1]; unused (may be NULL) with CSMLA_Q_BF16
 *   ori_kv / cmp_kv   fp8 e4m3 bytes: PA [blocks, block_size, 1, d]; TND [rows, 1, d];
 *                     BSND [B, S, 1, d]
 *   *_kv_descale      f32 per-token: PA [blocks, block_size], TND [rows], BSND [B, S];
 *                     per-tile64: the same with a trailing [d/64]; unused (may be NULL) with
 *                     bf16 or packed rows (rows of 2 d or 640 bytes instead of d)
 *   cmp_sparse_indices int32 [t1, 1, topk]  (BSND [B, Q_S, 1, topk])
 *   *_block_table     int32 [B, *_table_cols] (PA)
 *   cu_seqlens_*      int32 [B+1]; seqused_*, cmp_residual_kv int32 [B];
 *   cmp_topk_length   int32 [t1]
 *   ori_sparse_indices int32 [t1, 1, ori_topk] (listed logical ori positions; -1 invalid)
 *   ori_topk_length   int32 [t1] (slots in effect per row; NULL: all ori_topk)
 *   sinks             f32 [n1] (NULL: no sink)
 *   attn_out          bf16 [t1, n1, d]
 *   softmax_lse       f32 [t1, n1] (TND [1, t1, n1]; BSND [B, 1, Q_S, n1])
 *   workspace         device scratch of the size csmla_plan reports (may be NULL if 0),
 *                     256-byte aligned and zero-filled before its first use: its first
 *                     8.25 MiB hold sync words and the exchange slots of in-kernel
 *                     merges, which every call leaves ready for the next (so one buffer
 *                     serves any sequence of plans); after them, with splits, the
 *                     partial outputs and their (max, sum).  Calls that overlap in time
 *                     must not share it.
 * Descales must be finite and >= 0 (a zero descale is treated as 2^-126). */
typedef struct {
  const void*    q;
  const float*   q_descale;
  const void*    ori_kv;
  const float*   ori_kv_descale;
  const void*    cmp_kv;
  const float*   cmp_kv_descale;
  const int32_t* cmp_sparse_indices;
  const int32_t* ori_block_table;
  const int32_t* cmp_block_table;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_ori_kv;
  const int32_t* cu_seqlens_cmp_kv;
  const int32_t* seqused_q;
  const int32_t* seqused_ori_kv;
  const int32_t* seqused_cmp_kv;
  const int32_t* cmp_residual_kv;
  const int32_t* cmp_topk_length;
  const float*   sinks;
  void*          attn_out;
  float*         softmax_lse;
  void*          workspace;
  size_t         workspace_bytes;
  const int32_t* ori_sparse_indices;
  const int32_t* ori_topk_length;
} csmla_tensors;

/* ABI version of the loaded library (CSMLA_ABI_VERSION). */
int csmla_abi_version(void);

/* Static text for a status code. */
const char* csmla_status_string(int status);

/* Message of the calling thread's last failing call ("" if none). */
const char* csmla_last_error(void);

/* Words of metadata csmla_plan writes: CSMLA_METADATA_WORDS. */
size_t csmla_metadata_words(void);

/* Host-side check of a problem against the pages' constraints
 * (QuantSparseFlashMla, 约束说明): N2 = 1 and D = 512; cmp_ratio 1..128 and
 * 1 without cmp_kv; mask modes {0,3,4}/{0,3}; windows -1 or >= 0, and >= 0
 * only with band mode; the allowed layout pairs; block sizes 1..1024; no
 * empty tensors.  Returns CSMLA_OK, CSMLA_ERR_INVALID_ARG or
 * CSMLA_ERR_UNSUPPORTED (n1 other than 64 or 128, topk_value_mode != 0). */
csmla_status csmla_validate(const csmla_problem* problem);

/* Split planner, the counterpart of QuantSparseFlashMlaMetadata
 * (QuantSparseFlashMla, 功能说明 and 约束说明: int32 metadata of shape [1024]
 * generated before the main op).  Host only; no device work.
 *   metadata         host int32[metadata_words], metadata_words >= 1024; written
 *   workspace_bytes  host; written: device scratch csmla_forward needs (may be 0)
 * The plan depends on the problem fields and on the host lengths given;
 * csmla_forward rejects a plan made for a different problem, and
 * csmla_plan_check also one made for other host lengths. */
csmla_status csmla_plan(const csmla_problem* problem, const csmla_host_lengths* lengths,
                        int32_t* metadata, size_t metadata_words, size_t* workspace_bytes);

/* Whether `metadata` is csmla_plan's output for this problem and these host
 * lengths (the plan records hashes of both; QuantSparseFlashMla, 功能说明:
 * the metadata is made for the main op's inputs).  Host only.  Returns
 * CSMLA_OK or CSMLA_ERR_METADATA_MISMATCH.  csmla_forward checks the problem
 * hash itself but, having no host lengths, cannot see a plan made for other
 * lengths: a caller that keeps a plan across steps whose lengths may change
 * calls this first (or plans again). */
csmla_status csmla_plan_check(const csmla_problem* problem, const csmla_host_lengths* lengths,
                              const int32_t* metadata);

/* The attention forward (QuantSparseFlashMla, 参数说明 inputs and outputs).
 *   metadata   host int32[1024] from csmla_plan for this problem (required)
 *   stream     hipStream_t as void*
 * Writes attn_out (and softmax_lse when problem->return_softmax_lse) on
 * `stream`.  Query rows past seqused_q get O = 0 and lse = -inf; a row with
 * no visible key gets O = 0 and lse = sink (-inf without sinks). */
csmla_status csmla_forward(const csmla_problem* problem, const csmla_tensors* tensors,
                           const int32_t* metadata, void* stream);

/* csmla_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, with tensors->workspace / workspace_bytes ignored and the
 * split partials kept in the library's static device scratch instead, 64 MiB
 * per GPU (CSMLA_NOALLOC_SCRATCH_BYTES), held from the first call on a device
 * until the process ends.  A plan needing more workspace than that returns
 * CSMLA_ERR_WORKSPACE before any device work.  Allocates nothing and records
 * no memset.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (two streams, two threads) race and must be
 * serialised by the caller. */
#define CSMLA_NOALLOC_SCRATCH_BYTES (64u << 20)
csmla_status csmla_forward_noalloc(const csmla_problem* problem, const csmla_tensors* tensors,
                                   const int32_t* metadata, void* stream);

/* Resolved key list of every query row (QuantSparseFlashMla, 参数说明: the
 * band window, cmp_sparse_indices with -1 skipped, the block tables), as the
 * key-split and head-split kernels resolve it: their resolution functions
 * (key position, block position, table entry, row) run on every key.  For
 * row t, keys[t*max_keys + k] for k < counts[2t] + counts[2t+1] holds the
 * physical cache row of the k-th key — ori band rows in position order first
 * (counts[2t] of them), then cmp rows in index-slot order (counts[2t+1]);
 * entries past max_keys are not written (counts are exact).
 *   keys    device int32 [t1, max_keys]
 *   counts  device int32 [t1, 2]
 * Used to check the gather sets bit for bit. */
csmla_status csmla_debug_resolve(const csmla_problem* problem, const csmla_tensors* tensors,
                                 int32_t* keys, int32_t* counts, int32_t max_keys, void* stream);

/* The same export through the whole-token (prefill) kernel's own resolution:
 * its token entry (lengths, index compaction), per-tile key resolution and
 * row-address functions, with the row recovered from the address its LDS-DMA
 * would read.  Same arguments and output as csmla_debug_resolve;
 * CSMLA_ERR_UNSUPPORTED when topk > 1024 (that kernel's index-list limit). */
csmla_status csmla_debug_resolve_whole_token(const csmla_problem* problem, const csmla_tensors* tensors,
                                             int32_t* keys, int32_t* counts, int32_t max_keys, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSMLA_H */
