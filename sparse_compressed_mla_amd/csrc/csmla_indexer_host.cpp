// Host side of the indexer's C ABI (include/csmla_indexer.h): validation
// against the QuantLightningIndexerV2 page's constraints, the work split
// (the counterpart of QuantLightningIndexerV2Metadata), and the marshalling
// of csmla_indexer_forward into the two kernel launches.  No device memory is
// allocated here and nothing synchronises.
#include "../../include/csmla_indexer.h"
#include "csmla_indexer_internal.h"
#include "csmla_internal.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

using namespace csmla_idx;

namespace {

csmla_status fail(csmla_status st, const char* msg) {
  return (csmla_status)csmla::fail_with(st, "%s", msg);
}

template <typename... A>
csmla_status failf(csmla_status st, const char* fmt, A... args) {
  return (csmla_status)csmla::fail_with(st, fmt, args...);
}

int64_t floordiv(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}

uint32_t problem_hash(const csmla_indexer_problem* p) {
  return csmla::hash_bytes(p, sizeof(*p)) & 0x7fffffffu;
}

uint32_t lengths_hash(const csmla_indexer_problem* p, const csmla_indexer_host_lengths* hl) {
  if (!hl) return 0;
  uint32_t h = 2166136261u;
  auto mix = [&](const int32_t* a, size_t n, uint32_t tag) {
    h = csmla::hash_bytes(&tag, 4, h);
    if (a) h = csmla::hash_bytes(a, n * 4, h);
  };
  mix(hl->cu_seqlens_q, p->batch + 1, 1);
  mix(hl->seqused_q, p->batch, 2);
  mix(hl->cu_seqlens_k, p->batch + 1, 3);
  mix(hl->seqused_k, p->batch, 4);
  mix(hl->cmp_residual_k, p->batch, 5);
  return h & 0x7fffffffu;
}

int64_t key_capacity(const csmla_indexer_problem* p) {
  if (p->layout_k == CSMLA_LAYOUT_PA_BBND) return (int64_t)p->table_cols * p->block_size;
  return p->k_s;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Top-k work-group shapes built (threads, float4 chunks kept in registers).
bool topk_shape_ok(int nt, int cc) {
  return (nt == 256 && (cc == 1 || cc == 4)) || (nt == 1024 && (cc == 2 || cc == 4 || cc == 8));
}

// Most blocks a wave's `part` keys starting at a multiple of 64 can touch.
int block_span(int part, int bs) {
  int worst = 0;
  const int period = 64 * bs;
  for (int k0 = 0; k0 < period; k0 += 64)
    worst = std::max(worst, (k0 + part - 1) / bs - k0 / bs + 1);
  return worst;
}

}  // namespace

extern "C" {

size_t csmla_indexer_metadata_words(void) { return CSMLA_INDEXER_METADATA_WORDS; }

csmla_status csmla_indexer_validate(const csmla_indexer_problem* p) {
  if (!p) return fail(CSMLA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1) return fail(CSMLA_ERR_INVALID_ARG, "batch must be >= 1 (empty tensors are rejected)");
  if (p->t1 < 1) return fail(CSMLA_ERR_INVALID_ARG, "t1 must be >= 1 (empty tensors are rejected)");
  if (p->g < 1 || p->g > kMaxG) return failf(CSMLA_ERR_INVALID_ARG, "query heads g must be in 1..64, got %d", p->g);
  if (p->n2 != 1) return failf(CSMLA_ERR_INVALID_ARG, "key heads must be 1, got %d", p->n2);
  if (p->quant_mode != 1)
    return failf(CSMLA_ERR_UNSUPPORTED, "only quant_mode 1 (fp8 e4m3, fp32 scales) is built, got %d", p->quant_mode);
  if (p->d != kD) return failf(CSMLA_ERR_UNSUPPORTED, "only d = 128 is built, got %d", p->d);
  if (p->topk < 1 || p->topk > 8192) return failf(CSMLA_ERR_INVALID_ARG, "topk must be in 1..8192, got %d", p->topk);
  if (p->layout_q != CSMLA_LAYOUT_BSND && p->layout_q != CSMLA_LAYOUT_TND)
    return fail(CSMLA_ERR_INVALID_ARG, "layout_q must be BSND or TND");
  if (p->layout_k != CSMLA_LAYOUT_BSND && p->layout_k != CSMLA_LAYOUT_TND && p->layout_k != CSMLA_LAYOUT_PA_BBND)
    return fail(CSMLA_ERR_INVALID_ARG, "layout_k must be BSND, TND or PA_BBND");
  if (p->layout_q == CSMLA_LAYOUT_BSND) {
    if (p->q_s < 1) return fail(CSMLA_ERR_INVALID_ARG, "BSND query needs q_s >= 1");
    if ((int64_t)p->batch * p->q_s != p->t1) return fail(CSMLA_ERR_INVALID_ARG, "BSND query: t1 must equal batch * q_s");
  }
  if (p->layout_k == CSMLA_LAYOUT_PA_BBND) {
    if (p->block_size < 1 || p->block_size > 1024) return fail(CSMLA_ERR_INVALID_ARG, "block_size must be in 1..1024");
    if (p->num_blocks < 1 || p->table_cols < 1) return fail(CSMLA_ERR_INVALID_ARG, "key cache / block table must not be empty");
  } else if (p->k_s < 1) {
    return fail(CSMLA_ERR_INVALID_ARG, "key must not be empty");
  }
  if (p->cmp_ratio < 1 || p->cmp_ratio > 128) return fail(CSMLA_ERR_INVALID_ARG, "cmp_ratio must be in 1..128");
  if (p->mask_mode != 0 && p->mask_mode != 3) return fail(CSMLA_ERR_INVALID_ARG, "mask_mode must be 0 or 3");
  const int64_t rows = p->layout_k == CSMLA_LAYOUT_PA_BBND ? (int64_t)p->num_blocks * p->block_size
                       : p->layout_k == CSMLA_LAYOUT_BSND  ? (int64_t)p->batch * p->k_s
                                                           : (int64_t)p->k_s;
  if (rows >= ((int64_t)1 << 31)) return fail(CSMLA_ERR_UNSUPPORTED, "key caches of 2^31 rows or more are not built");
  csmla::clear_last_error();
  return CSMLA_OK;
}

csmla_status csmla_indexer_plan(const csmla_indexer_problem* p, const csmla_indexer_host_lengths* hl, int32_t* md,
                                size_t md_words, size_t* ws_bytes) {
  csmla_status st = csmla_indexer_validate(p);
  if (st != CSMLA_OK) return st;
  if (!md) return fail(CSMLA_ERR_INVALID_ARG, "metadata buffer is NULL (it is mandatory)");
  if (md_words < CSMLA_INDEXER_METADATA_WORDS)
    return failf(CSMLA_ERR_INVALID_ARG, "metadata needs %d words", CSMLA_INDEXER_METADATA_WORDS);
  const csmla_indexer_host_lengths empty{};
  const csmla_indexer_host_lengths& h = hl ? *hl : empty;
  const int B = p->batch;
  if (h.cu_seqlens_q) {
    if (p->layout_q != CSMLA_LAYOUT_TND) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_q is for TND query only");
    if (h.cu_seqlens_q[0] != 0) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_q[0] must be 0");
    for (int b = 0; b < B; ++b)
      if (h.cu_seqlens_q[b + 1] < h.cu_seqlens_q[b]) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_q must be non-decreasing");
    if (h.cu_seqlens_q[B] != p->t1) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_q[B] must equal t1");
  }
  if (h.cu_seqlens_k) {
    if (p->layout_k != CSMLA_LAYOUT_TND) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_k is for TND key only");
    if (h.cu_seqlens_k[0] != 0) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_k[0] must be 0");
    for (int b = 0; b < B; ++b)
      if (h.cu_seqlens_k[b + 1] < h.cu_seqlens_k[b]) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_k must be non-decreasing");
    if (h.cu_seqlens_k[B] > p->k_s) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_k[B] exceeds the rows of key");
  }
  for (int b = 0; b < B; ++b) {
    if (h.seqused_q && h.seqused_q[b] < 0) return fail(CSMLA_ERR_INVALID_ARG, "seqused_q must be >= 0");
    if (h.seqused_k && (h.seqused_k[b] < 0 || h.seqused_k[b] > key_capacity(p)))
      return fail(CSMLA_ERR_INVALID_ARG, "seqused_k must be in [0, key capacity]");
    if (h.cmp_residual_k && (h.cmp_residual_k[b] < 0 || h.cmp_residual_k[b] >= p->cmp_ratio))
      return fail(CSMLA_ERR_INVALID_ARG, "cmp_residual_k must be in [0, cmp_ratio)");
  }

  // rows used and keys per batch (exact from the lengths, else shape bounds)
  int64_t max_s1 = 0, max_n = 0;
  for (int b = 0; b < B; ++b) {
    int64_t span;
    if (p->layout_q == CSMLA_LAYOUT_TND) span = h.cu_seqlens_q ? h.cu_seqlens_q[b + 1] - h.cu_seqlens_q[b] : p->t1;
    else span = p->q_s;
    const int64_t s1 = h.seqused_q ? std::min<int64_t>(span, h.seqused_q[b]) : span;
    int64_t n;
    if (p->layout_k == CSMLA_LAYOUT_TND) n = h.cu_seqlens_k ? h.cu_seqlens_k[b + 1] - h.cu_seqlens_k[b] : p->k_s;
    else n = h.seqused_k ? h.seqused_k[b] : key_capacity(p);
    if (s1 < 1) continue;
    max_s1 = std::max(max_s1, s1);
    // the last row of a batch sees the most keys: floor((n r + res) / r) = n
    max_n = std::max(max_n, n);
  }
  const int64_t stride = std::max<int64_t>(kStep, (max_n + kStep - 1) / kStep * kStep);

  int tw, wt, kc;
  if (max_s1 <= 1) { tw = 1; wt = 1; }
  else if (max_s1 == 2) { tw = 2; wt = 1; }
  else if (max_s1 <= 8) { tw = 4; wt = 1; }
  else { tw = 2; wt = 4; }
  if (const char* env = std::getenv("CSMLA_IDX_TILE")) {   // tuning override "tw,wt"
    int a = 0, b = 0;
    if (std::sscanf(env, "%d,%d", &a, &b) == 2 && ((a == 1 && b == 1) || (a == 2 && (b == 1 || b == 4)) ||
                                                   (a == 4 && (b == 1 || b == 4)))) {
      tw = a;
      wt = b;
    }
  }
  if (wt == 1) kc = max_n <= 4096 ? 256 : 4096;
  else kc = 1024;
  if (const char* env = std::getenv("CSMLA_IDX_KC")) {   // tuning override: a multiple of 256
    const int f = std::atoi(env);
    if (f >= 256 && f % 256 == 0) kc = f;
  }
  // A wave reads the block-table entries of its keys with one load per lane:
  // its keys may span at most 64 blocks.
  if (p->layout_k == CSMLA_LAYOUT_PA_BBND) {
    while (block_span(kc / (4 / wt), p->block_size) > 64) {
      if (kc > 256) kc -= 256;
      else wt = 1;
    }
  }
  const int64_t rows_per_tile = (int64_t)tw * wt;
  const int64_t nqt = std::max<int64_t>(1, (max_s1 + rows_per_tile - 1) / rows_per_tile);
  const int64_t nkc = std::max<int64_t>(1, (max_n + kc - 1) / kc);
  if (nqt > 65535 || B > 65535) return fail(CSMLA_ERR_UNSUPPORTED, "too many query rows per batch or batches");
  if (nkc > ((int64_t)1 << 30)) return fail(CSMLA_ERR_UNSUPPORTED, "too many keys");

  int nt, cc;
  if (stride <= 1024) { nt = 256; cc = 1; }
  else if (stride <= 4096) { nt = 256; cc = 4; }
  else if (stride <= 8192) { nt = 1024; cc = 2; }
  else if (stride <= 16384) { nt = 1024; cc = 4; }
  else { nt = 1024; cc = 8; }

  if (const char* env = std::getenv("CSMLA_IDX_TOPK")) {   // tuning override "threads,chunks"
    int a = 0, b = 0;
    if (std::sscanf(env, "%d,%d", &a, &b) == 2 && topk_shape_ok(a, b)) {
      nt = a;
      cc = b;
    }
  }
  const size_t ws = align256((size_t)p->t1 * (size_t)stride * sizeof(float));
  std::memset(md, 0, sizeof(int32_t) * CSMLA_INDEXER_METADATA_WORDS);
  md[IM_MAGIC] = kMagic;
  md[IM_VERSION] = CSMLA_ABI_VERSION;
  md[IM_PROBLEM_HASH] = (int32_t)problem_hash(p);
  md[IM_LENGTHS_HASH] = (int32_t)lengths_hash(p, hl);
  md[IM_TW] = tw;
  md[IM_WT] = wt;
  md[IM_KC] = kc;
  md[IM_NQT] = (int32_t)nqt;
  md[IM_NKC] = (int32_t)nkc;
  md[IM_STRIDE] = (int32_t)stride;
  md[IM_TOPK_NT] = nt;
  md[IM_TOPK_C] = cc;
  md[IM_WS_LO] = (int32_t)(ws & 0x7fffffff);
  md[IM_WS_HI] = (int32_t)(ws >> 31);
  if (ws_bytes) *ws_bytes = ws;
  csmla::clear_last_error();
  return CSMLA_OK;
}

csmla_status csmla_indexer_forward(const csmla_indexer_problem* p, const csmla_indexer_tensors* t, const int32_t* md,
                                   void* stream) {
  csmla_status st = csmla_indexer_validate(p);
  if (st != CSMLA_OK) return st;
  if (!t) return fail(CSMLA_ERR_INVALID_ARG, "tensors is NULL");
  if (!md) return fail(CSMLA_ERR_INVALID_ARG, "metadata is NULL (it is mandatory)");
  if (md[IM_MAGIC] != kMagic || md[IM_VERSION] != CSMLA_ABI_VERSION)
    return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata was not written by csmla_indexer_plan");
  if (md[IM_PROBLEM_HASH] != (int32_t)problem_hash(p))
    return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata was planned for another problem");
  const int tw = md[IM_TW], wt = md[IM_WT], kc = md[IM_KC], nt = md[IM_TOPK_NT], cc = md[IM_TOPK_C];
  const bool tile_ok = (tw == 1 && wt == 1) || (tw == 2 && (wt == 1 || wt == 4)) || (tw == 4 && (wt == 1 || wt == 4));
  const bool topk_ok = topk_shape_ok(nt, cc);
  if (!tile_ok || !topk_ok || kc < 256 || kc % 256 != 0 || md[IM_NQT] < 1 || md[IM_NKC] < 1 || md[IM_STRIDE] < kStep ||
      md[IM_STRIDE] % kStep != 0)
    return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata fields are inconsistent");
  if (p->layout_k == CSMLA_LAYOUT_PA_BBND && block_span(kc / (4 / wt), p->block_size) > 64)
    return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata key chunk spans more than 64 blocks per wave");
  if (!t->query || !t->key || !t->weights || !t->query_dequant_scale || !t->key_dequant_scale || !t->sparse_indices)
    return fail(CSMLA_ERR_INVALID_ARG, "query, key, weights, both dequant scales and sparse_indices are required");
  if (p->layout_q == CSMLA_LAYOUT_TND && !t->cu_seqlens_q) return fail(CSMLA_ERR_INVALID_ARG, "TND query needs cu_seqlens_q");
  if (p->layout_q == CSMLA_LAYOUT_BSND && t->cu_seqlens_q)
    return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_q must not be given with BSND query");
  if (p->layout_k == CSMLA_LAYOUT_TND && !t->cu_seqlens_k) return fail(CSMLA_ERR_INVALID_ARG, "TND key needs cu_seqlens_k");
  if (p->layout_k != CSMLA_LAYOUT_TND && t->cu_seqlens_k)
    return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_k is for TND key only");
  if (p->layout_k == CSMLA_LAYOUT_TND && t->seqused_k) return fail(CSMLA_ERR_INVALID_ARG, "seqused_k is not used with TND key");
  if (p->layout_k == CSMLA_LAYOUT_PA_BBND && (!t->seqused_k || !t->block_table))
    return fail(CSMLA_ERR_INVALID_ARG, "PA_BBND key needs seqused_k and block_table");
  const size_t ws = (size_t)(uint32_t)md[IM_WS_LO] | ((size_t)(uint32_t)md[IM_WS_HI] << 31);
  if (!t->workspace || t->workspace_bytes < ws)
    return failf(CSMLA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", ws, t->workspace ? t->workspace_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(t->workspace) & 255) != 0)
    return fail(CSMLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  IArgs a{};
  a.batch = p->batch; a.t1 = p->t1; a.g = p->g; a.q_s = p->q_s;
  a.layout_q = p->layout_q; a.layout_k = p->layout_k; a.k_s = p->k_s;
  a.bs = p->layout_k == CSMLA_LAYOUT_PA_BBND ? p->block_size : 1;
  a.bs_shift = -1;
  for (int s = 0; s < 11; ++s)
    if (a.bs == (1 << s)) a.bs_shift = s;
  a.cols = p->table_cols;
  if (p->layout_k == CSMLA_LAYOUT_PA_BBND) {
    a.nrows = (int32_t)std::min<int64_t>((int64_t)p->num_blocks * p->block_size, INT32_MAX);
    a.tab_ld = p->table_cols;
    a.tab_cols = p->table_cols;
  } else {
    a.nrows = p->layout_k == CSMLA_LAYOUT_TND ? p->k_s
                                              : (int32_t)std::min<int64_t>((int64_t)p->batch * p->k_s, INT32_MAX);
    a.tab_ld = 0;
    a.tab_cols = 1;
  }
  a.topk = p->topk; a.mask = p->mask_mode; a.ratio = p->cmp_ratio;
  a.tw = tw; a.wt = wt; a.kc = kc; a.nqt = md[IM_NQT]; a.nkc = md[IM_NKC]; a.stride = md[IM_STRIDE];
  a.q = (const uint8_t*)t->query; a.qs = t->query_dequant_scale; a.w = t->weights;
  a.key = (const uint8_t*)t->key; a.ks = t->key_dequant_scale;
  // without paging the kernel's one table read per lane lands on the first key scale
  a.tab = t->block_table ? t->block_table : (const int32_t*)t->key_dequant_scale;
  a.cu_q = t->cu_seqlens_q; a.cu_k = t->cu_seqlens_k;
  a.su_q = t->seqused_q; a.su_k = t->seqused_k; a.res = t->cmp_residual_k;
  a.scores = (float*)t->workspace; a.out = t->sparse_indices;
  const int e = launch_indexer(a, nt, cc, stream);
  if (e != 0) return failf(CSMLA_ERR_HIP, "kernel launch failed (hipError %d)", e);
  csmla::clear_last_error();
  return CSMLA_OK;
}

}  // extern "C"
