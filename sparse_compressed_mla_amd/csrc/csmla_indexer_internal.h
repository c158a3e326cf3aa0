// Internal definitions shared by the indexer's host side
// (csmla_indexer_host.cpp) and its HIP kernels (csmla_indexer_kernels.hip).
// Not part of the public ABI.
#pragma once
#include <stdint.h>
#include <stddef.h>

namespace csmla_idx {

constexpr int kD = 128;                 // index head width
constexpr int kMaxG = 64;               // query heads (QuantLightningIndexerV2, 约束说明: N in [1, 64])
constexpr int32_t kMagic = 0x58444943;  // "CIDX"
constexpr int kStep = 64;               // keys per wave step of the score kernel

// plan word offsets (int32[CSMLA_INDEXER_METADATA_WORDS])
enum {
  IM_MAGIC = 0, IM_VERSION = 1, IM_PROBLEM_HASH = 2, IM_LENGTHS_HASH = 3,
  IM_TW = 4,       // query rows per wave
  IM_WT = 5,       // waves of a work-group that take different rows (1 or 4)
  IM_KC = 6,       // keys per work-group
  IM_NQT = 7,      // row tiles per batch (grid y)
  IM_NKC = 8,      // key chunks (grid x)
  IM_STRIDE = 9,   // floats per score row in the workspace
  IM_TOPK_NT = 10, // threads of the top-k work-group
  IM_TOPK_C = 11,  // score chunks the top-k keeps in registers
  IM_WS_LO = 12, IM_WS_HI = 13,
};

struct IArgs {
  int32_t batch, t1, g, q_s, layout_q, layout_k, k_s, bs, bs_shift, cols;
  int32_t nrows;             // rows of the key cache (PA: blocks * block_size)
  int32_t tab_ld, tab_cols;  // block-table row stride and width as read (0 and 1 without paging)
  int32_t topk, mask, ratio;
  int32_t tw, wt, kc, nqt, nkc, stride;
  const uint8_t* q; const float* qs; const float* w;
  const uint8_t* key; const float* ks;
  const int32_t* tab; const int32_t* cu_q; const int32_t* cu_k; const int32_t* su_q; const int32_t* su_k;
  const int32_t* res;
  float* scores; int32_t* out;
};

// launchers (csmla_indexer_kernels.hip); return a hipError_t as int
int launch_indexer(const IArgs& a, int topk_nt, int topk_c, void* stream);

}  // namespace csmla_idx
