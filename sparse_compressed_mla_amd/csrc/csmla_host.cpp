// Host side of the C ABI: validation against the pages' constraints, the
// split planner (the counterpart of QuantSparseFlashMlaMetadata), and the
// marshalling of csmla_forward / csmla_debug_resolve into kernel launches.
// No device memory is allocated here and nothing synchronises.
#include "../../include/csmla.h"
#include "csmla_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

using namespace csmla;

namespace {
constexpr int64_t kSkKeys = 2 * kTileKeys;   // keys per split-key unit (two 64-key tiles)
constexpr int64_t kSkMaxSplits = 16;
}  // namespace

static_assert(CSMLA_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "static scratch size");

namespace {

thread_local std::string g_last_error;

csmla_status fail(csmla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

uint32_t fnv1a(const void* data, size_t n, uint32_t h = 2166136261u) {
  const uint8_t* p = static_cast<const uint8_t*>(data);
  for (size_t i = 0; i < n; ++i) { h ^= p[i]; h *= 16777619u; }
  return h;
}

uint32_t problem_hash(const csmla_problem* p) {
  return fnv1a(p, sizeof(csmla_problem)) & 0x7fffffffu;
}

int64_t floordiv64(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}

// Per-token key counts from host lengths: exact band size and an upper bound
// of the compressed part (indices may be -1).  Mirrors the device resolution.
struct TokCost { int64_t n_o, n_c_up; };

std::vector<TokCost> token_costs(const csmla_problem* p, const csmla_host_lengths* hl) {
  std::vector<TokCost> out;
  out.reserve(p->t1);
  const csmla_host_lengths empty{};
  const csmla_host_lengths& h = hl ? *hl : empty;
  const int B = p->batch;
  for (int b = 0; b < B; ++b) {
    int64_t q0, span;
    if (p->layout_q == CSMLA_LAYOUT_TND) {
      if (h.cu_seqlens_q) { q0 = h.cu_seqlens_q[b]; span = h.cu_seqlens_q[b + 1] - q0; }
      else { // unknown split of t1 over batches: spread evenly (estimate only)
        q0 = (int64_t)p->t1 * b / B; span = (int64_t)p->t1 * (b + 1) / B - q0;
      }
    } else { q0 = (int64_t)b * p->q_s; span = p->q_s; }
    int64_t s1 = span;
    if (h.seqused_q) s1 = std::min<int64_t>(span, h.seqused_q[b]);
    int64_t s2;
    if (h.seqused_ori_kv) s2 = h.seqused_ori_kv[b];
    else if (h.cu_seqlens_ori_kv) s2 = h.cu_seqlens_ori_kv[b + 1] - h.cu_seqlens_ori_kv[b];
    else if (p->layout_kv == CSMLA_LAYOUT_PA_BBND) s2 = (int64_t)p->ori_table_cols * p->ori_block_size;
    else s2 = p->ori_s;
    int64_t c = 0;
    const int r = p->cmp_ratio;
    if (p->has_cmp) {
      if (h.seqused_cmp_kv) c = h.seqused_cmp_kv[b];
      else if (h.cu_seqlens_cmp_kv) c = h.cu_seqlens_cmp_kv[b + 1] - h.cu_seqlens_cmp_kv[b];
      else if (p->layout_kv == CSMLA_LAYOUT_BSND) c = p->cmp_s;
      else if (p->layout_kv == CSMLA_LAYOUT_PA_BBND) c = s2 / r;
      else c = p->cmp_s;
    }
    const int64_t res = h.cmp_residual_kv ? h.cmp_residual_kv[b] : 0;
    const int64_t L = c * r + res;
    for (int64_t i = 0; i < span; ++i) {
      TokCost tc{0, 0};
      if (i < s1) {
        const int64_t pos = s2 - s1 + i;
        int64_t lo = 0, hi = s2;
        if (p->ori_mask_mode == CSMLA_MASK_RIGHT_DOWN_CAUSAL) hi = std::max<int64_t>(0, std::min<int64_t>(s2, pos + 1));
        if (p->ori_mask_mode == CSMLA_MASK_BAND) {
          lo = p->ori_win_left < 0 ? 0 : std::max<int64_t>(0, pos - p->ori_win_left);
          hi = p->ori_win_right < 0 ? s2 : std::max<int64_t>(0, std::min<int64_t>(s2, pos + p->ori_win_right + 1));
          hi = std::max(hi, lo);
        }
        tc.n_o = hi - lo;
        if (p->ori_topk > 0) {   // listed ori positions: at most the slots in effect
          int64_t k = p->ori_topk;
          const int64_t t = q0 + i;
          if (h.ori_topk_length && t < p->t1) k = std::max<int64_t>(0, std::min<int64_t>(k, h.ori_topk_length[t]));
          tc.n_o = tc.n_o > 0 ? k : 0;   // duplicates may list a window position more than once
        }
        if (p->has_cmp) {
          int64_t vis = c;
          if (p->cmp_mask_mode == CSMLA_MASK_RIGHT_DOWN_CAUSAL)
            vis = std::max<int64_t>(0, std::min<int64_t>(c, floordiv64(L - s1 + i + 1, r)));
          if (p->topk > 0) {
            int64_t k = p->topk;
            const int64_t t = q0 + i;
            if (h.cmp_topk_length && t < p->t1) k = std::max<int64_t>(0, std::min<int64_t>(k, h.cmp_topk_length[t]));
            tc.n_c_up = std::min(k, vis);
          } else {
            tc.n_c_up = vis;
          }
        }
      }
      out.push_back(tc);
    }
  }
  if ((int)out.size() != p->t1) out.resize(p->t1, TokCost{0, 0});
  return out;
}

uint32_t lengths_hash(const csmla_problem* p, const csmla_host_lengths* hl) {
  if (!hl) return 0;
  uint32_t h = 2166136261u;
  const int B = p->batch;
  auto mix = [&](const int32_t* a, size_t n, uint32_t tag) {
    h = fnv1a(&tag, 4, h);
    if (a) h = fnv1a(a, n * 4, h);
  };
  mix(hl->cu_seqlens_q, B + 1, 1);
  mix(hl->seqused_q, B, 2);
  mix(hl->seqused_ori_kv, B, 3);
  mix(hl->cu_seqlens_ori_kv, B + 1, 4);
  mix(hl->seqused_cmp_kv, B, 5);
  mix(hl->cu_seqlens_cmp_kv, B + 1, 6);
  mix(hl->cmp_residual_kv, B, 7);
  mix(hl->cmp_topk_length, p->t1, 8);
  mix(hl->ori_topk_length, p->t1, 9);
  return h & 0x7fffffffu;
}

bool is_win(int w) { return w == -1 || w >= 0; }

}  // namespace

// Error reporting shared with the indexer's host code (csmla_indexer_host.cpp).
int csmla::fail_with(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

void csmla::clear_last_error() { g_last_error.clear(); }

uint32_t csmla::hash_bytes(const void* data, size_t n, uint32_t seed) { return fnv1a(data, n, seed); }

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Workspace of a split plan: bf16 partial outputs [units, 64, 512], then
// (max, sum) [units, 64, 2] fp32.
void csmla::workspace_offsets(int n_units, size_t* xcc, size_t* o, size_t* ml) {
  *xcc = kWsFixedBytes;
  *o = align256(*xcc + (size_t)n_units * sizeof(int32_t));
  *ml = align256(*o + (size_t)n_units * kN1 * kD * 2);
}

size_t csmla::workspace_bytes_for(int n_units, int splits, int dk_parts) {
  if (dk_parts > 1) return kWsFixedBytes;
  if (splits <= 1) return 0;
  size_t xcc, o, ml;
  workspace_offsets(n_units, &xcc, &o, &ml);
  return ml + (size_t)n_units * kN1 * 2 * sizeof(float);
}

extern "C" {

int csmla_abi_version(void) { return CSMLA_ABI_VERSION; }

const char* csmla_status_string(int status) {
  switch (status) {
    case CSMLA_OK: return "ok";
    case CSMLA_ERR_INVALID_ARG: return "invalid argument";
    case CSMLA_ERR_UNSUPPORTED: return "unsupported";
    case CSMLA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSMLA_ERR_METADATA_MISMATCH: return "metadata planned for another problem";
    case CSMLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* csmla_last_error(void) { return g_last_error.c_str(); }

size_t csmla_metadata_words(void) { return CSMLA_METADATA_WORDS; }

csmla_status csmla_validate(const csmla_problem* p) {
  if (!p) return fail(CSMLA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1) return fail(CSMLA_ERR_INVALID_ARG, "batch must be >= 1 (empty tensors are rejected)");
  if (p->t1 < 1) return fail(CSMLA_ERR_INVALID_ARG, "t1 must be >= 1 (empty tensors are rejected)");
  if (p->n2 != 1) return fail(CSMLA_ERR_INVALID_ARG, "n2 must be 1, got %d", p->n2);
  if (p->d != 512) return fail(CSMLA_ERR_INVALID_ARG, "d must be 512, got %d", p->d);
  if (p->n1 < 1) return fail(CSMLA_ERR_INVALID_ARG, "n1 must be >= 1");
  if (p->n1 != kN1 && p->n1 != 2 * kN1)
    return fail(CSMLA_ERR_UNSUPPORTED, "only n1 = 64 or 128 query heads are built, got %d", p->n1);
  if (p->layout_q != CSMLA_LAYOUT_BSND && p->layout_q != CSMLA_LAYOUT_TND)
    return fail(CSMLA_ERR_INVALID_ARG, "layout_q must be BSND or TND");
  if (p->layout_kv != CSMLA_LAYOUT_BSND && p->layout_kv != CSMLA_LAYOUT_TND && p->layout_kv != CSMLA_LAYOUT_PA_BBND)
    return fail(CSMLA_ERR_INVALID_ARG, "layout_kv must be BSND, TND or PA_BBND");
  if (p->layout_kv != CSMLA_LAYOUT_PA_BBND && p->layout_kv != p->layout_q)
    return fail(CSMLA_ERR_INVALID_ARG, "without PA_BBND, layout_q and layout_kv must match");
  if (p->layout_q == CSMLA_LAYOUT_BSND) {
    if (p->q_s < 1) return fail(CSMLA_ERR_INVALID_ARG, "BSND q needs q_s >= 1");
    if ((int64_t)p->batch * p->q_s != p->t1) return fail(CSMLA_ERR_INVALID_ARG, "BSND q: t1 must equal batch * q_s");
  }
  if (p->layout_kv == CSMLA_LAYOUT_PA_BBND) {
    if (p->ori_block_size < 1 || p->ori_block_size > 1024)
      return fail(CSMLA_ERR_INVALID_ARG, "ori_block_size must be in 1..1024");
    if (p->ori_num_blocks < 1 || p->ori_table_cols < 1)
      return fail(CSMLA_ERR_INVALID_ARG, "ori cache / block table must not be empty");
    if (p->has_cmp) {
      if (p->cmp_block_size < 1 || p->cmp_block_size > 1024)
        return fail(CSMLA_ERR_INVALID_ARG, "cmp_block_size must be in 1..1024");
      if (p->cmp_num_blocks < 1 || p->cmp_table_cols < 1)
        return fail(CSMLA_ERR_INVALID_ARG, "cmp cache / block table must not be empty");
    }
  } else {
    if (p->ori_s < 1) return fail(CSMLA_ERR_INVALID_ARG, "ori_kv must not be empty");
    if (p->has_cmp && p->cmp_s < 1) return fail(CSMLA_ERR_INVALID_ARG, "cmp_kv must not be empty");
  }
  if (p->cmp_ratio < 1 || p->cmp_ratio > 128) return fail(CSMLA_ERR_INVALID_ARG, "cmp_ratio must be in 1..128");
  if (!p->has_cmp && p->cmp_ratio != 1) return fail(CSMLA_ERR_INVALID_ARG, "cmp_ratio must be 1 without cmp_kv");
  if (!p->has_cmp && p->topk != 0) return fail(CSMLA_ERR_INVALID_ARG, "cmp_sparse_indices need cmp_kv");
  if (p->topk < 0) return fail(CSMLA_ERR_INVALID_ARG, "topk must be >= 0");
  if (p->ori_mask_mode != 0 && p->ori_mask_mode != 3 && p->ori_mask_mode != 4)
    return fail(CSMLA_ERR_INVALID_ARG, "ori_mask_mode must be 0, 3 or 4");
  if (p->cmp_mask_mode != 0 && p->cmp_mask_mode != 3) return fail(CSMLA_ERR_INVALID_ARG, "cmp_mask_mode must be 0 or 3");
  if (!is_win(p->ori_win_left) || !is_win(p->ori_win_right))
    return fail(CSMLA_ERR_INVALID_ARG, "ori_win_left/right must be -1 or >= 0");
  if (p->ori_mask_mode != CSMLA_MASK_BAND && (p->ori_win_left >= 0 || p->ori_win_right >= 0))
    return fail(CSMLA_ERR_INVALID_ARG, "ori_win_left/right may be >= 0 only with ori_mask_mode 4");
  if (p->kv_scale_mode != CSMLA_KV_SCALE_PER_TOKEN && p->kv_scale_mode != CSMLA_KV_SCALE_PER_TILE64)
    return fail(CSMLA_ERR_INVALID_ARG, "kv_scale_mode must be 0 or 1");
  if (p->topk_value_mode != 0) return fail(CSMLA_ERR_UNSUPPORTED, "only topk_value_mode 0 is built");
  if (!(std::isfinite(p->softmax_scale))) return fail(CSMLA_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (p->q_dtype != CSMLA_Q_FP8 && p->q_dtype != CSMLA_Q_BF16) return fail(CSMLA_ERR_INVALID_ARG, "q_dtype must be 0 or 1");
  if (p->kv_dtype != CSMLA_KV_FP8 && p->kv_dtype != CSMLA_KV_BF16 && p->kv_dtype != CSMLA_KV_PACKED640)
    return fail(CSMLA_ERR_INVALID_ARG, "kv_dtype must be 0, 1 or 2");
  if (p->kv_dtype != CSMLA_KV_FP8 && p->q_dtype != CSMLA_Q_BF16)
    return fail(CSMLA_ERR_INVALID_ARG, "bf16 and packed KV rows go with bf16 q");
  if (p->q_dtype == CSMLA_Q_BF16 && p->kv_dtype == CSMLA_KV_FP8)
    return fail(CSMLA_ERR_UNSUPPORTED, "bf16 q with fp8 KV and fp32 descales is not built");
  if (p->kv_dtype != CSMLA_KV_FP8 && p->kv_scale_mode != CSMLA_KV_SCALE_PER_TOKEN)
    return fail(CSMLA_ERR_INVALID_ARG, "kv_scale_mode applies to fp8 KV only (leave it 0)");
  if (p->kv_dtype != CSMLA_KV_FP8 && p->topk > kListMax)
    return fail(CSMLA_ERR_UNSUPPORTED, "bf16 / packed KV: at most %d index slots per row are built", kListMax);
  if (p->ori_topk < 0) return fail(CSMLA_ERR_INVALID_ARG, "ori_topk must be >= 0");
  if (p->ori_topk > 0 && (int64_t)p->ori_topk + p->topk > kListMax)
    return fail(CSMLA_ERR_UNSUPPORTED, "ori_topk + topk must be <= %d (one index list per row)", kListMax);
  g_last_error.clear();
  return CSMLA_OK;
}

csmla_status csmla_plan(const csmla_problem* p, const csmla_host_lengths* hl, int32_t* md, size_t md_words,
                        size_t* ws_bytes) {
  csmla_status st = csmla_validate(p);
  if (st != CSMLA_OK) return st;
  if (!md) return fail(CSMLA_ERR_INVALID_ARG, "metadata buffer is NULL (it is mandatory)");
  if (md_words < CSMLA_METADATA_WORDS) return fail(CSMLA_ERR_INVALID_ARG, "metadata needs %d words", CSMLA_METADATA_WORDS);
  if (p->layout_q == CSMLA_LAYOUT_TND && hl && hl->cu_seqlens_q) {
    if (hl->cu_seqlens_q[0] != 0) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_q[0] must be 0");
    for (int b = 0; b < p->batch; ++b)
      if (hl->cu_seqlens_q[b + 1] < hl->cu_seqlens_q[b]) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_q must be non-decreasing");
    if (hl->cu_seqlens_q[p->batch] != p->t1) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_q[B] must equal t1");
  }
  for (const int32_t* cu : {hl ? hl->cu_seqlens_ori_kv : nullptr, hl ? hl->cu_seqlens_cmp_kv : nullptr}) {
    if (!cu) continue;
    if (cu[0] != 0) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_*_kv[0] must be 0");
    for (int b = 0; b < p->batch; ++b)
      if (cu[b + 1] < cu[b]) return fail(CSMLA_ERR_INVALID_ARG, "cu_seqlens_*_kv must be non-decreasing");
  }

  const std::vector<TokCost> cost = token_costs(p, hl);
  const int T1 = p->t1;
  int64_t max_n = 0, max_c = 0, total = 0;
  for (const auto& c : cost) {
    max_n = std::max(max_n, c.n_o + c.n_c_up);
    max_c = std::max(max_c, c.n_c_up);
    total += c.n_o + c.n_c_up;
  }
  // splits per token: enough units to occupy every CU, units of >= 64 keys,
  // and at most kListMax compressed indices per unit
  int64_t s_list = 1;
  if (p->topk > 0 && max_c > kListMax) s_list = (max_n + kListMax - 1) / kListMax;
  const int64_t avg = T1 ? total / T1 : 0;
  int64_t s_par = 1;
  if (T1 < kMaxGrid) s_par = std::min<int64_t>((kMaxGrid + T1 - 1) / T1, std::max<int64_t>(1, avg / 64));
  int64_t S = std::max(s_list, s_par);
  if (const char* env = std::getenv("CSMLA_SPLITS")) {
    const int64_t f = std::atoll(env);
    if (f >= 1) S = std::max(s_list, f);
  }
  // Decode batches with per-token descales: split the heads instead of the
  // keys, so that no partial outputs need merging.  Groups of 8 heads while
  // their units fit one round of the work-groups (T1 <= 32), else groups of
  // 16 up to 128 tokens; from 129 tokens whole tokens per unit (all 64 heads,
  // hg = kN1) when the index list fits the list buffer.  Measured on MI355X
  // with 640 keys per token: 48 tokens take 17.1 us in 16-head groups and
  // 29.3 us in 8-head groups; 128 tokens 34.5 us in 16-head groups and
  // 38.2 us as whole tokens; 160 tokens 47.3 us and 39.1 us.  Long key lists
  // and per-tile descales keep the key split up to 256 tokens.
  // Prefill-sized batches (more tokens than CUs) with at most kListMax index
  // slots per token: whole tokens per unit, no splits.
  const bool pf_ok = p->topk <= kListMax && p->kv_dtype == CSMLA_KV_FP8;
  const bool bf = p->kv_dtype != CSMLA_KV_FP8;   // the bf16-q kernel: key splits of <= kBkMaxUnitKeys keys
  if (bf) S = std::max<int64_t>(S, (max_n + kBkMaxUnitKeys - 1) / kBkMaxUnitKeys);
  int hg = 0;
  if (!bf && p->kv_scale_mode == CSMLA_KV_SCALE_PER_TOKEN && avg <= 8192) {
    if (T1 * (kN1 / 8) <= kMaxGrid) hg = 8;
    else if (T1 <= 128 || (T1 <= 256 && !pf_ok)) hg = 16;
    else if (pf_ok) hg = kN1;
  }
  if (T1 > 256 && pf_ok) hg = kN1;
  // 12 to 28 tokens: 16-head groups in two key parts (below) instead of
  // 8-head groups.  Measured on MI355X with 640 keys per token (two rounds,
  // one box): 12 / 16 / 20 / 24 tokens 14.97 / 15.04 / 15.61 / 15.83 us
  // against 15.10 / 15.62 / 16.14 / 16.08 us; equal at 28 tokens, slower at
  // 4, 8 and 32 (14.61 / 14.51 / 16.62 against 14.37 / 14.44 / 16.40 us).
  // With the output rows stored non-temporally the parted plan also wins
  // from 25 to 28 tokens (four interleaved rounds, one box: 28 tokens 16.04
  // against 16.40 us).  At 32 tokens it gains only 0.8% (16.25 against
  // 16.38 us) while its exchange moves ~4 MB of tagged partials (22.8 MB
  // per launch against 14.3 MB measured), so 8-head groups over whole key
  // lists keep 29 to 32 tokens.  A kernel override (CSMLA_KERNEL) keeps its
  // own choice.
  bool h16_parts = false;
  if (hg == 8 && T1 >= 12 && T1 <= 28 && !std::getenv("CSMLA_KERNEL")) {
    hg = 16;
    h16_parts = true;
  }
  // Split-key decode kernel: all 64 heads of a token over <= 128 keys per
  // unit, the splits of a token merged inside the kernel.  It needs every
  // unit resident at once (one work-group per CU: 8 S ceil(T1 / 8) <= 256)
  // and top-k within the list buffer; S is as large as that allows.
  const int64_t t_rounds = (T1 + 7) / 8;
  const int64_t sk_min = std::max<int64_t>(1, (max_n + kSkKeys - 1) / kSkKeys);
  const int64_t sk_max = std::min<int64_t>(kMaxGrid / (8 * t_rounds), kSkMaxSplits);
  const bool sk_ok = pf_ok && T1 <= kSkMaxTokens && sk_min <= sk_max;   // (pf_ok: fp8 KV)
  bool sk = false;
  if (const char* env = std::getenv("CSMLA_KERNEL")) {   // tuning / test override
    if (!std::strcmp(env, "split")) hg = 0;
    else if (!std::strcmp(env, "heads8") && p->kv_scale_mode == CSMLA_KV_SCALE_PER_TOKEN) hg = 8;
    else if (!std::strcmp(env, "heads16") && p->kv_scale_mode == CSMLA_KV_SCALE_PER_TOKEN) hg = 16;
    else if (!std::strcmp(env, "prefill") && pf_ok) hg = kN1;
    else if (!std::strcmp(env, "splitkey") && sk_ok) { hg = 0; sk = true; }
  }
  if (sk) {
    S = sk_max;
    if (const char* env = std::getenv("CSMLA_SPLITS")) {
      const int64_t f = std::atoll(env);
      if (f >= 1) S = std::min(std::max(f, sk_min), sk_max);
    }
  }
  if (p->ori_topk > 0) {   // listed ori keys: the key-split kernels (fp8 or bf16-q) only
    hg = 0;
    sk = false;
  }
  if (bf) {   // every override keeps the bf16-q kernel (only CSMLA_SPLITS applies)
    hg = 0;
    sk = false;
    S = std::max<int64_t>(S, (max_n + kBkMaxUnitKeys - 1) / kBkMaxUnitKeys);
  }
  if (hg > 0) S = 1;
  // Key parts of the head-split kernel: each (token, head group) split into
  // P parts of whole 128-key tiles on one XCD, the last merging the others'
  // partials.  Every unit needs a work-group of its own (the grid rounded up
  // to whole XCD rounds of groups, at most one work-group per CU), and a
  // part gets at least one tile.  Two parts by default where they fit (8-head
  // groups up to 16 tokens, and the 16-head groups chosen above): measured on
  // MI355X with 640 keys per token, 4 and 8 tokens run 15.1 and 15.3 us in
  // two parts against 16.2 and 16.1 us whole; four parts lose (the merger
  // reads each writer's partial in a round trip of its own).  CSMLA_DK_PARTS
  // overrides the count.
  int parts = 1;
  if (hg == 8 || hg == 16) {
    int64_t want = (hg == 8 || h16_parts) ? 2 : 1;
    if (const char* env = std::getenv("CSMLA_DK_PARTS")) want = std::atoll(env);
    const int64_t tiles = std::max<int64_t>(1, (max_n + kDkTileKeys - 1) / kDkTileKeys);
    const int64_t groups = (int64_t)T1 * (kN1 / hg);
    while (parts * 2 <= want && parts * 2 <= kDkMaxParts && parts * 2 <= tiles &&
           round_up(groups * parts * 2, 8 * parts * 2) <= kMaxGrid)
      parts *= 2;
  }
  int dk_test = 0;
  if (parts > 1)
    if (const char* env = std::getenv("CSMLA_DK_TEST")) dk_test = std::atoi(env);
  if (S > kMaxSplits) return fail(CSMLA_ERR_UNSUPPORTED, "a token needs %lld splits; at most %d are built", (long long)S, kMaxSplits);
  const int64_t per_token = hg > 0 ? (kN1 / hg) * parts : S;   // units per query token
  const int64_t n_units64 = (int64_t)T1 * per_token;
  if (n_units64 > (int64_t)1 << 30) return fail(CSMLA_ERR_UNSUPPORTED, "too many work units");
  const int n_units = (int)n_units64;
  // the split-key kernel's grid: 8 S ceil(T1 / 8) blocks, token t's splits on XCD t mod 8
  const int G = sk ? (int)(8 * S * t_rounds)
                   : parts > 1 ? (int)round_up(n_units64, 8 * parts) : (int)std::min<int64_t>(n_units64, kMaxGrid);

  // contiguous unit ranges per work-group, balanced by estimated keys
  std::vector<double> pre(n_units + 1, 0.0);
  for (int u = 0; u < n_units; ++u) {
    const auto& c = cost[u / per_token];
    if (hg == kN1) {
      // whole-token prefill kernel: a token takes at least one 64-key tile, and
      // its first-tile reference move, output, sink and lse plus the next
      // token's set-up cost about 2.5 tiles more (swept on MI355X: 112 to 176
      // keys balance equally well; 56 runs 12% slower, 400 runs 3% slower)
      const int64_t tiles = std::max<int64_t>(1, (c.n_o + c.n_c_up + kTileKeys - 1) / kTileKeys);
      pre[u + 1] = pre[u] + (double)(tiles * kTileKeys) + 160.0;
    } else {
      pre[u + 1] = pre[u] + (double)(c.n_o + c.n_c_up) / (double)S + 48.0;
    }
  }
  std::vector<int32_t> starts(G + 1);
  starts[0] = 0;
  int u = 0;
  for (int g = 1; g < G && !sk && parts == 1; ++g) {
    const double target = pre[n_units] * g / G;
    while (u < n_units && pre[u] < target) ++u;
    int lo = starts[g - 1] + 1, hi = n_units - (G - g);
    starts[g] = std::min(std::max(u, lo), hi);
    u = starts[g];
  }
  if (sk || parts > 1)   // one unit per block; the block -> unit map lives in the kernel
    for (int g = 1; g < G; ++g) starts[g] = std::min(g, n_units);
  starts[G] = n_units;

  std::memset(md, 0, sizeof(int32_t) * CSMLA_METADATA_WORDS);
  md[MD_MAGIC] = kMagic;
  md[MD_VERSION] = CSMLA_ABI_VERSION;
  md[MD_PROBLEM_HASH] = (int32_t)problem_hash(p);
  md[MD_LENGTHS_HASH] = (int32_t)lengths_hash(p, hl);
  md[MD_T1] = T1;
  md[MD_SPLITS] = (int32_t)S;
  md[MD_UNITS] = n_units;
  md[MD_GRID] = G;
  md[MD_LIST_MAX] = kListMax;
  const size_t ws = workspace_bytes_for(n_units, (int)S, parts);
  md[MD_WS_LO] = (int32_t)(ws & 0x7fffffff);
  md[MD_WS_HI] = (int32_t)(ws >> 31);
  md[MD_FLAGS] = S > 1 ? 1 : 0;
  md[MD_HEAD_GROUP] = hg;
  md[MD_SPLIT_KEY] = sk ? 1 : 0;
  md[MD_DK_PARTS] = parts;
  md[MD_DK_TEST] = dk_test;
  for (int g = 0; g <= G; ++g) md[MD_STARTS + g] = starts[g];
  if (ws_bytes) *ws_bytes = ws;
  g_last_error.clear();
  return CSMLA_OK;
}

static csmla_status build_args(const csmla_problem* p, const csmla_tensors* t, const int32_t* md, KArgs& a,
                               bool need_plan) {
  csmla_status st = csmla_validate(p);
  if (st != CSMLA_OK) return st;
  if (!t) return fail(CSMLA_ERR_INVALID_ARG, "tensors is NULL");
  const bool fp8q = p->q_dtype == CSMLA_Q_FP8, fp8kv = p->kv_dtype == CSMLA_KV_FP8;
  if (!t->q || (fp8q && !t->q_descale)) return fail(CSMLA_ERR_INVALID_ARG, "q (and with fp8 q, q_descale) required");
  if (!t->ori_kv || (fp8kv && !t->ori_kv_descale))
    return fail(CSMLA_ERR_INVALID_ARG, "ori_kv (and with fp8 KV, ori_kv_descale) required");
  if (p->has_cmp && (!t->cmp_kv || (fp8kv && !t->cmp_kv_descale)))
    return fail(CSMLA_ERR_INVALID_ARG, "has_cmp needs cmp_kv (and with fp8 KV, cmp_kv_descale)");
  if (p->topk > 0 && !t->cmp_sparse_indices) return fail(CSMLA_ERR_INVALID_ARG, "topk > 0 needs cmp_sparse_indices");
  if (p->ori_topk > 0 && !t->ori_sparse_indices)
    return fail(CSMLA_ERR_INVALID_ARG, "ori_topk > 0 needs ori_sparse_indices");
  if (p->layout_q == CSMLA_LAYOUT_TND && !t->cu_seqlens_q) return fail(CSMLA_ERR_INVALID_ARG, "TND q needs cu_seqlens_q");
  if (p->layout_kv == CSMLA_LAYOUT_PA_BBND) {
    if (!t->seqused_ori_kv || !t->ori_block_table)
      return fail(CSMLA_ERR_INVALID_ARG, "PA_BBND needs seqused_ori_kv and ori_block_table");
    if (p->has_cmp && !t->cmp_block_table) return fail(CSMLA_ERR_INVALID_ARG, "PA_BBND cmp_kv needs cmp_block_table");
  }
  if (p->layout_kv == CSMLA_LAYOUT_TND) {
    if (!t->cu_seqlens_ori_kv) return fail(CSMLA_ERR_INVALID_ARG, "TND kv needs cu_seqlens_ori_kv");
    if (p->has_cmp && !t->cu_seqlens_cmp_kv) return fail(CSMLA_ERR_INVALID_ARG, "TND kv with cmp_kv needs cu_seqlens_cmp_kv");
  }
  if (need_plan && !t->attn_out) return fail(CSMLA_ERR_INVALID_ARG, "attn_out is required");
  if (need_plan && p->return_softmax_lse && !t->softmax_lse)
    return fail(CSMLA_ERR_INVALID_ARG, "return_softmax_lse needs softmax_lse");

  std::memset(&a, 0, sizeof(a));
  a.dk_parts = 1;
  a.batch = p->batch; a.t1 = p->t1; a.q_s = p->q_s; a.layout_q = p->layout_q; a.layout_kv = p->layout_kv;
  a.ori_s = p->ori_s; a.cmp_s = p->cmp_s; a.ori_bs = p->ori_block_size; a.cmp_bs = p->cmp_block_size;
  a.ori_cols = p->ori_table_cols; a.cmp_cols = p->cmp_table_cols;
  a.has_cmp = p->has_cmp; a.topk = p->topk; a.cmp_ratio = p->cmp_ratio;
  a.ori_mask = p->ori_mask_mode; a.cmp_mask = p->cmp_mask_mode;
  a.win_left = p->ori_mask_mode == CSMLA_MASK_BAND ? p->ori_win_left : -1;
  a.win_right = p->ori_mask_mode == CSMLA_MASK_BAND ? p->ori_win_right : -1;
  a.scale_mode = p->kv_scale_mode; a.q_ds_per_head = p->q_descale_per_head; a.ret_lse = p->return_softmax_lse;
  a.n1 = p->n1;
  a.kv_fmt = p->kv_dtype;
  a.ori_topk = p->ori_topk;
  a.ori_idx = p->ori_topk > 0 ? t->ori_sparse_indices : nullptr;
  a.ori_tkl = p->ori_topk > 0 ? t->ori_topk_length : nullptr;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.q = (const uint8_t*)t->q; a.q_ds = t->q_descale;
  a.ori_kv = (const uint8_t*)t->ori_kv; a.ori_ds = t->ori_kv_descale;
  a.cmp_kv = p->has_cmp ? (const uint8_t*)t->cmp_kv : nullptr; a.cmp_ds = p->has_cmp ? t->cmp_kv_descale : nullptr;
  a.idx = p->topk > 0 ? t->cmp_sparse_indices : nullptr;
  a.ori_tab = t->ori_block_table; a.cmp_tab = t->cmp_block_table;
  a.cu_q = t->cu_seqlens_q; a.cu_ori = t->cu_seqlens_ori_kv; a.cu_cmp = t->cu_seqlens_cmp_kv;
  a.su_q = t->seqused_q; a.su_ori = t->seqused_ori_kv; a.su_cmp = t->seqused_cmp_kv;
  a.res = t->cmp_residual_kv; a.topk_len = t->cmp_topk_length; a.sinks = t->sinks;
  a.out = (uint16_t*)t->attn_out; a.lse = p->return_softmax_lse ? t->softmax_lse : nullptr;

  if (need_plan) {
    if (!md) return fail(CSMLA_ERR_INVALID_ARG, "metadata is NULL (it is mandatory)");
    if (md[MD_MAGIC] != kMagic || md[MD_VERSION] != CSMLA_ABI_VERSION)
      return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata was not written by csmla_plan of this version");
    if ((uint32_t)md[MD_PROBLEM_HASH] != problem_hash(p) || md[MD_T1] != p->t1)
      return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata was planned for a different problem");
    const int S = md[MD_SPLITS], U = md[MD_UNITS], G = md[MD_GRID], HG = md[MD_HEAD_GROUP], SK = md[MD_SPLIT_KEY];
    const bool hg_ok = HG == 0 || (p->ori_topk == 0 && p->kv_dtype == CSMLA_KV_FP8 &&
                                   (((HG == 8 || HG == 16) && S == 1 && p->kv_scale_mode == CSMLA_KV_SCALE_PER_TOKEN) ||
                                    (HG == kN1 && S == 1 && p->topk <= kListMax)));
    const bool sk_ok = SK == 0 || (SK == 1 && HG == 0 && p->ori_topk == 0 && p->kv_dtype == CSMLA_KV_FP8 &&
                                   S <= kSkMaxSplits && p->t1 <= kSkMaxTokens &&
                                   p->topk <= kListMax && G == 8 * S * ((p->t1 + 7) / 8) && G <= kMaxGrid);
    const int PT = md[MD_DK_PARTS], DT = md[MD_DK_TEST];
    const bool parts_ok = PT == 1 || ((PT == 2 || PT == 4 || PT == 8) && (HG == 8 || HG == 16) &&
                                      G == (int)round_up(U, 8 * PT) && (DT >= 0 && DT <= 2));
    const int per_token = HG > 0 ? (kN1 / HG) * PT : S;
    if (S < 1 || !hg_ok || !sk_ok || !parts_ok || U != p->t1 * per_token || G < 1 || G > kMaxGrid ||
        (!SK && PT == 1 && G > U))
      return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata header is inconsistent");
    a.hg = HG;
    a.sk = SK;
    a.dk_parts = PT;
    a.dk_test = DT;
    a.dk_ticks = DT ? 0 : kDkWaitTicks;
    for (int g = 0; g <= G; ++g) {
      const int s0 = md[MD_STARTS + g];
      if (s0 < 0 || s0 > U || (g > 0 && s0 < md[MD_STARTS + g - 1]) || (g == 0 && s0 != 0) || (g == G && s0 != U))
        return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata work ranges are inconsistent");
      a.starts[g] = s0;
    }
    a.splits = S; a.n_units = U; a.grid = G;
    const size_t ws = workspace_bytes_for(U, S, PT);
    if (ws > 0) {
      if (!t->workspace || t->workspace_bytes < ws)
        return fail(CSMLA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", ws, t->workspace ? t->workspace_bytes : (size_t)0);
      if ((reinterpret_cast<uintptr_t>(t->workspace) & 255) != 0)
        return fail(CSMLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
      size_t o_xcc, o_o, o_ml;
      workspace_offsets(U, &o_xcc, &o_o, &o_ml);
      a.ws_sync = (int32_t*)t->workspace;
      a.ws_xcc = (int32_t*)((char*)t->workspace + o_xcc);
      a.ws_o = (uint16_t*)((char*)t->workspace + o_o);
      a.ws_ml = (float*)((char*)t->workspace + o_ml);
      a.ws_xch = (uint8_t*)t->workspace + kWsSyncBytes;
    }
  }
  return CSMLA_OK;
}

csmla_status csmla_forward(const csmla_problem* p, const csmla_tensors* t, const int32_t* md, void* stream) {
  KArgs a;
  csmla_status st = build_args(p, t, md, a, true);
  if (st != CSMLA_OK) return st;
  // The kernels cover 64 heads per launch: n1 = 128 runs the two halves one
  // after the other on the stream (same plan, same workspace), each with its
  // pointers at the half's first head and the token stride of n1 heads.
  for (int h0 = 0; h0 < p->n1; h0 += kN1) {
    KArgs ah = a;
    ah.q = a.q + (size_t)h0 * kD * (p->q_dtype == CSMLA_Q_BF16 ? 2 : 1);
    ah.out = a.out + (size_t)h0 * kD;
    if (a.lse) ah.lse = a.lse + h0;
    if (a.q_ds && a.q_ds_per_head) ah.q_ds = a.q_ds + h0;
    if (a.sinks) ah.sinks = a.sinks + h0;
    const int e = launch_forward(ah, stream);
    if (e != 0) return fail(CSMLA_ERR_HIP, "kernel launch failed (hipError %d)", e);
  }
  g_last_error.clear();
  return CSMLA_OK;
}

csmla_status csmla_plan_check(const csmla_problem* p, const csmla_host_lengths* hl, const int32_t* md) {
  csmla_status st = csmla_validate(p);
  if (st != CSMLA_OK) return st;
  if (!md) return fail(CSMLA_ERR_INVALID_ARG, "metadata is NULL");
  if (md[MD_MAGIC] != kMagic || md[MD_VERSION] != CSMLA_ABI_VERSION)
    return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata was not written by csmla_plan of this version");
  if ((uint32_t)md[MD_PROBLEM_HASH] != problem_hash(p) || md[MD_T1] != p->t1)
    return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata was planned for a different problem");
  if ((uint32_t)md[MD_LENGTHS_HASH] != lengths_hash(p, hl))
    return fail(CSMLA_ERR_METADATA_MISMATCH, "metadata was planned for other host lengths");
  g_last_error.clear();
  return CSMLA_OK;
}

csmla_status csmla_forward_noalloc(const csmla_problem* p, const csmla_tensors* t, const int32_t* md, void* stream) {
  if (!t) return fail(CSMLA_ERR_INVALID_ARG, "tensors is NULL");
  csmla_tensors ts = *t;
  ts.workspace = nullptr;
  ts.workspace_bytes = 0;
  // the plan's workspace size, checked against the static scratch before any
  // HIP call (a plan that is not csmla_plan's is rejected by csmla_forward)
  if (md && md[MD_MAGIC] == kMagic && md[MD_VERSION] == CSMLA_ABI_VERSION && md[MD_UNITS] >= 0 &&
      md[MD_SPLITS] >= 1) {
    const size_t need = workspace_bytes_for(md[MD_UNITS], md[MD_SPLITS], md[MD_DK_PARTS]);
    if (need > kNoAllocScratchBytes)
      return fail(CSMLA_ERR_WORKSPACE,
                  "the plan needs %zu bytes of workspace; csmla_forward_noalloc holds %zu (use csmla_forward with "
                  "a workspace, or a plan with fewer key splits)",
                  need, kNoAllocScratchBytes);
    if (need > 0) {
      void* ptr = nullptr;
      const int e = noalloc_scratch(&ptr, stream);
      if (e != 0) return fail(CSMLA_ERR_HIP, "static scratch lookup failed (hipError %d)", e);
      ts.workspace = ptr;
      ts.workspace_bytes = kNoAllocScratchBytes;
    }
  }
  return csmla_forward(p, &ts, md, stream);
}

static csmla_status debug_resolve(const csmla_problem* p, const csmla_tensors* t, int32_t* keys, int32_t* counts,
                                  int32_t max_keys, int whole_token, void* stream) {
  KArgs a;
  csmla_status st = build_args(p, t, nullptr, a, false);
  if (st != CSMLA_OK) return st;
  if (!keys || !counts || max_keys < 0) return fail(CSMLA_ERR_INVALID_ARG, "keys/counts buffers are required");
  if (whole_token && p->ori_topk > 0)
    return fail(CSMLA_ERR_UNSUPPORTED, "the whole-token kernel takes no ori_sparse_indices");
  if (whole_token && p->topk > kListMax)
    return fail(CSMLA_ERR_UNSUPPORTED, "the whole-token kernel keeps at most %d index slots (topk %d)", kListMax,
                p->topk);
  const int e = launch_debug_resolve(a, keys, counts, max_keys, whole_token, stream);
  if (e != 0) return fail(CSMLA_ERR_HIP, "kernel launch failed (hipError %d)", e);
  g_last_error.clear();
  return CSMLA_OK;
}

csmla_status csmla_debug_resolve(const csmla_problem* p, const csmla_tensors* t, int32_t* keys, int32_t* counts,
                                 int32_t max_keys, void* stream) {
  return debug_resolve(p, t, keys, counts, max_keys, 0, stream);
}

csmla_status csmla_debug_resolve_whole_token(const csmla_problem* p, const csmla_tensors* t, int32_t* keys,
                                             int32_t* counts, int32_t max_keys, void* stream) {
  return debug_resolve(p, t, keys, counts, max_keys, 1, stream);
}

}  // extern "C"
