// HIP kernels for gfx950 (MI355X): quantized sparse shared-KV MLA attention.
//
// One work unit = (query token t, split s): all 64 heads of t against the
// keys [kb, ke) of t's resolved key list (ori band positions, then cmp
// entries), as defined on the QuantSparseFlashMla page (功能说明: SWA / CSA /
// HCA and the formula; 参数说明: masks, windows, cmp_ratio, residual).
//
// A work-group has 4 waves; wave w owns heads [32*(w&1), +32) and output
// columns [256*(w>>1), +256).  Per 64-key tile:
//   S^T[32 keys x 32 heads] = K Q^T        v_mfma_f32_32x32x64_f8f6f4, fp8 e4m3;
//                                          each wave of a pair sums half of D,
//                                          the halves are added through LDS
//   online softmax in log2 units, the V descale folded into the exponent so
//   that P' = 2^(s + log2 vds - M) lies in (0, 2^8], the running max at 2^4
//   O^T[32 d x 32 heads] += V^T P'^T        same MFMA, P' as an fp8 hi + lo
//                                            pair (two MFMAs), V^T read with
//                                            ds_read_b64_tr_b8 (LDS transpose)
// Rows are gathered HBM -> LDS with global_load_lds_dwordx4 into an
// XOR-swizzled layout (16-byte chunk c of row r at chunk c ^ swz(r)).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "csmla_internal.h"

namespace csmla {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kPShift = 4.0f;                 // P' of the running max is 2^4
constexpr float kTau = 8.0f;                    // rescale once P' would pass 2^8 (e4m3 max 448)
constexpr float kMinDescale = 1.17549435e-38f;  // a zero descale is read as 2^-126
constexpr float kNegInf = -__builtin_huge_valf();

constexpr int kThreads = 256;
constexpr int kTileBytes = kTileKeys * kD;      // 32 KiB
constexpr int kStageRow = 2 * 256 + 16;         // bytes per head row of the output staging

// LDS layout.  Tiles: 3 buffers of 64 rows x 512 fp8 bytes (XOR-swizzled
// 16-byte chunks).  Per-key arrays of the current chunk of a unit's key list
// (row address, log2 / inverse of the row's largest V descale, descales).
template <int PER_TILE>
struct Lds {
  static constexpr int kPerTile = PER_TILE;
  static constexpr int kNT = kThreads;                     // threads of the work-group
  static constexpr int kFlag = 8;                          // misc word of the redo flag
  static constexpr int kChunk = PER_TILE ? 512 : 1024;     // keys resolved at once
  static constexpr int kNks = PER_TILE ? 8 : 1;            // descales per key
  static constexpr int kTiles = 0;                         // 3 x 32 KiB
  static constexpr int kSx = 3 * kTileBytes;               // partial scores for the partner, 4 waves x 4 KiB
  static constexpr int kPx = kSx + 4 * 4096;               // P halves for the partner, 4 waves x 4 KiB
  static constexpr int kAddr = kPx + 4 * 4096;             // uint64 [kChunk]
  static constexpr int kLam = kAddr + 8 * kChunk;          // float [kChunk]
  static constexpr int kInv = kLam + 4 * kChunk;           // float [kChunk]
  static constexpr int kKs = kInv + 4 * kChunk;            // float [kNks][kChunk]
  static constexpr int kList = kKs + 4 * kNks * kChunk;    // int [kListMax]: compacted cmp indices
  static constexpr int kMisc = kList + 4 * kListMax;       // [0..7] compaction, [8] redo flag, [64..319] pair values
  static constexpr int kBytes = kMisc + 4 * 64 + 4 * 4 * 64;
};
static_assert(Lds<0>::kBytes <= 160 * 1024 && Lds<1>::kBytes <= 160 * 1024, "LDS");

// The kernel arguments live in the kernarg segment (constant address space).
// The kernels read the header once into two VGPRs (load_hdr_regs) and the
// per-work-group unit ranges directly from the segment.
typedef const __attribute__((address_space(4))) KArgs* KArgPtr;


// Source of the rows of key slots past the end of a chunk: the gather always
// issues the same number of loads per wave, so that the pipeline can count them.
__device__ __attribute__((aligned(4096))) uint8_t g_zero_row[2 * kD];   // covers a bf16 row too

// Work-group barrier that orders LDS only: outstanding global loads (the
// next tiles' gathers, stores of a finished unit) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A copy of x that the compiler cannot see through: values derived from it
// are recomputed where they are used instead of being hoisted out of loops
// and held in registers across the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The header fields as register values.  Two vector loads bring the header
// into two VGPRs (dword i in lane i mod 64) in one round trip; each field is
// then a lane read.  A field read where it is used would be a scalar load
// that waits for every scalar load in flight, one round trip each.
// hdr_view launders the two registers first, so that the lane reads (and
// what is computed from them) stay where a loop body uses them instead of
// being hoisted to the kernel entry into spilled scalar registers.
// v combined (max or sum) with the value of lane l ^ 32, or of lane l ^ 16,
// on the vector ALU: v_permlane32_swap (v_permlane16_swap) of v with itself
// leaves lane l's own value in one result and its partner's in the other, so
// no LDS round trip (as a ds_bpermute would take) is needed.
__device__ __forceinline__ float xor32_reduce(float v, bool is_max) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return is_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float xor16_reduce(float v, bool is_max) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return is_max ? fmaxf(a, b) : a + b;
}

// A pointer known to address device (global) memory, rebuilt from its bits
// so that loads through it compile to global (not flat) loads after its
// provenance was lost in a register copy.
template <class T>
__device__ __forceinline__ T* gptr(T* p) {
  return (T*)(__attribute__((address_space(1))) void*)(uintptr_t)p;
}

struct HdrRegs {
  uint32_t v0, v1;
};

constexpr int kHdrWords = (int)(sizeof(KHdr) / 4);
static_assert(sizeof(KHdr) % 4 == 0 && kHdrWords <= 128, "header size");

__device__ __forceinline__ HdrRegs load_hdr_regs(KArgPtr ap) {
  const int lane = opaque((int)threadIdx.x & 63);
  const uint32_t* p = (const uint32_t*)ap;
  return HdrRegs{p[min(lane, kHdrWords - 1)], p[min(64 + lane, kHdrWords - 1)]};
}

__device__ __forceinline__ KHdr hdr_view(HdrRegs r) {
  asm volatile("" : "+v"(r.v0), "+v"(r.v1));
  uint32_t wd[kHdrWords];
#pragma unroll
  for (int i = 0; i < kHdrWords; ++i) wd[i] = __builtin_amdgcn_readlane(i < 64 ? r.v0 : r.v1, i & 63);
  KHdr h;
  __builtin_memcpy(&h, wd, sizeof(KHdr));
  // every tensor is device (global) memory: a pointer that went through the
  // lane reads is generic, and loads through it would be flat loads (which
  // also count against the LDS wait counter)
#define CSMLA_GLOBAL(f) h.f = gptr(h.f)
  CSMLA_GLOBAL(q); CSMLA_GLOBAL(q_ds); CSMLA_GLOBAL(ori_kv); CSMLA_GLOBAL(ori_ds);
  CSMLA_GLOBAL(cmp_kv); CSMLA_GLOBAL(cmp_ds); CSMLA_GLOBAL(idx); CSMLA_GLOBAL(ori_tab); CSMLA_GLOBAL(cmp_tab);
  CSMLA_GLOBAL(cu_q); CSMLA_GLOBAL(cu_ori); CSMLA_GLOBAL(cu_cmp); CSMLA_GLOBAL(su_q); CSMLA_GLOBAL(su_ori);
  CSMLA_GLOBAL(su_cmp); CSMLA_GLOBAL(res); CSMLA_GLOBAL(topk_len); CSMLA_GLOBAL(sinks); CSMLA_GLOBAL(out);
  CSMLA_GLOBAL(lse); CSMLA_GLOBAL(ws_o); CSMLA_GLOBAL(ws_ml); CSMLA_GLOBAL(ws_sync); CSMLA_GLOBAL(ws_xcc);
  CSMLA_GLOBAL(ori_idx); CSMLA_GLOBAL(ori_tkl); CSMLA_GLOBAL(ws_xch);
#undef CSMLA_GLOBAL
  return h;
}

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ (((r >> 3) & 1) << 2); }

__device__ __forceinline__ v16f mma(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four fp32 values as two fp8 e4m3 words: hi = RNE(x), lo = RNE(x - hi).
// hi + lo carries ~8 significant bits, so P' keeps bf16-like precision
// while both MFMA operands stay fp8.
__device__ __forceinline__ void split_fp8(float x0, float x1, float x2, float x3, int& hi, int& lo) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
  const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - f01[0], x1 - f01[1], 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - f23[0], x3 - f23[1], l, true);
  hi = h;
  lo = l;
}

__device__ __forceinline__ int floordiv(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return (int)q;
}

// Two fp32 values as packed bf16 (round to nearest even; v_cvt_pk_bf16_f32),
// the first in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// ---------------------------------------------------------------------------
// per-token context: lengths, positions, windows (QuantSparseFlashMla,
// 参数说明 cu_seqlens_* / seqused_* / cmp_residual_kv / masks / windows)
// ---------------------------------------------------------------------------
struct Tok {
  int b, i, s1, s2, c, valid;
  int lo, hi;      // visible ori positions [lo, hi)
  int vis;         // visible compressed tokens: [0, vis)
  int kv0, cmp0;   // row offsets of a TND cache
  int k_eff;       // index slots read
  int ko_eff;      // ori index slots read (listed ori keys)
};

// A token's lengths: one load per array, all issued before the first is
// used.  They are vector loads of a uniform address (the lane index is
// laundered so that the compiler keeps them in the vector memory pipe): those
// complete in order, so the unit's later loads need not have landed when the
// lengths are used, which scalar loads (completing out of order) would
// require.  An absent array reads the zero row instead.  The TND batch
// lookup (a binary search over cu_seqlens_q) stays scalar.
typedef const __attribute__((address_space(4))) int32_t* ConstI32;

__device__ __forceinline__ int ld_len(const int32_t* p, int i, int zero) {
  const int32_t* q = p ? p : reinterpret_cast<const int32_t*>(g_zero_row);
  return q[(p ? i : 0) + zero];
}

struct TokLens {
  int b, q0, span;
  int su_q, su_ori, cu_o0, cu_o1, su_cmp, cu_c0, cu_c1, res, tkl, otkl;
};

__device__ __forceinline__ TokLens token_lens(const KHdr& a, int t) {
  TokLens l;
  if (a.layout_q == 1) {  // TND: largest b with cu_q[b] <= t
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (((ConstI32)a.cu_q)[mid] <= t) lo = mid; else hi = mid;
    }
    l.b = lo;
    l.q0 = ((ConstI32)a.cu_q)[lo];
    l.span = ((ConstI32)a.cu_q)[lo + 1] - l.q0;
  } else {
    l.b = (a.q_s == 1) ? t : t / a.q_s;   // (uniform) decode rows: no division
    l.q0 = l.b * a.q_s; l.span = a.q_s;
  }
  const int z = opaque(0), b = l.b;
  l.su_q = ld_len(a.su_q, b, z); l.su_ori = ld_len(a.su_ori, b, z);
  l.cu_o0 = ld_len(a.cu_ori, b, z); l.cu_o1 = ld_len(a.cu_ori, b + 1, z);
  l.su_cmp = ld_len(a.su_cmp, b, z);
  l.cu_c0 = ld_len(a.cu_cmp, b, z); l.cu_c1 = ld_len(a.cu_cmp, b + 1, z);
  l.res = ld_len(a.res, b, z); l.tkl = ld_len(a.topk_len, t, z); l.otkl = ld_len(a.ori_tkl, t, z);
  return l;
}

__device__ __forceinline__ Tok token_ctx(const KHdr& a, int t, const TokLens& l) {
  Tok k;
  const int b = l.b, q0 = l.q0, span = l.span;
  const int v_su_q = __builtin_amdgcn_readfirstlane(l.su_q), v_su_ori = __builtin_amdgcn_readfirstlane(l.su_ori);
  const int v_cu_o0 = __builtin_amdgcn_readfirstlane(l.cu_o0), v_cu_o1 = __builtin_amdgcn_readfirstlane(l.cu_o1);
  const int v_su_cmp = __builtin_amdgcn_readfirstlane(l.su_cmp);
  const int v_cu_c0 = __builtin_amdgcn_readfirstlane(l.cu_c0), v_cu_c1 = __builtin_amdgcn_readfirstlane(l.cu_c1);
  const int v_res = __builtin_amdgcn_readfirstlane(l.res), v_tkl = __builtin_amdgcn_readfirstlane(l.tkl);
  const int i = t - q0;
  const int s1 = a.su_q ? min(span, v_su_q) : span;
  const int s2 = a.su_ori ? v_su_ori : (a.cu_ori ? v_cu_o1 - v_cu_o0 : a.ori_s);
  k.kv0 = (a.layout_kv == 1) ? v_cu_o0 : 0;
  int c = 0;
  k.cmp0 = 0;
  if (a.has_cmp) {
    if (a.su_cmp) c = v_su_cmp;
    else if (a.cu_cmp) c = v_cu_c1 - v_cu_c0;
    else if (a.layout_kv == 0) c = a.cmp_s;
    else c = s2 / a.cmp_ratio;
    if (a.layout_kv == 1) k.cmp0 = v_cu_c0;
  }
  const int64_t res = a.res ? v_res : 0;
  k.b = b; k.i = i; k.s1 = s1; k.s2 = s2; k.c = c;
  k.valid = i < s1;
  const int64_t p = (int64_t)s2 - s1 + i;  // bottom-right aligned position
  int64_t lo = 0, hi = s2;
  if (a.ori_mask == 3) hi = max((int64_t)0, min((int64_t)s2, p + 1));
  if (a.ori_mask == 4) {
    lo = a.win_left < 0 ? 0 : max((int64_t)0, p - a.win_left);
    hi = a.win_right < 0 ? (int64_t)s2 : max((int64_t)0, min((int64_t)s2, p + a.win_right + 1));
    hi = max(hi, lo);
  }
  k.lo = (int)lo; k.hi = (int)hi;
  int vis = c;
  if (a.has_cmp && a.cmp_mask == 3) {
    const int64_t L = (int64_t)c * a.cmp_ratio + res;
    vis = max(0, min(c, floordiv(L - s1 + i + 1, a.cmp_ratio)));
  }
  k.vis = a.has_cmp ? vis : 0;
  int ke = a.topk;
  if (a.topk_len) ke = max(0, min(ke, v_tkl));
  k.k_eff = ke;
  int ko = a.ori_topk;
  if (a.ori_tkl) ko = max(0, min(ko, __builtin_amdgcn_readfirstlane(l.otkl)));
  k.ko_eff = ko;
  if (!k.valid) { k.lo = k.hi = 0; k.vis = 0; k.k_eff = 0; k.ko_eff = 0; }
  return k;
}

__device__ __forceinline__ Tok token_ctx(const KHdr& a, int t) { return token_ctx(a, t, token_lens(a, t)); }

// The first kIdxPre index slots of token t, one value per thread per round
// (NT threads), loaded before the token's lengths are known (bounded by topk,
// not by the effective length), so that these loads share a round trip with
// them.
constexpr int kIdxPre = 1024;

template <int NT>
struct IdxPre {
  static constexpr int kRounds = kIdxPre / NT;
  int v[kRounds];
};

// Branch-free: slots past topk read a valid slot (or the zero row when
// there are no indices) and are then replaced by -1.
template <int NT>
__device__ __forceinline__ IdxPre<NT> load_indices(const KHdr& a, int t, int s0) {
  constexpr int R = IdxPre<NT>::kRounds;
  IdxPre<NT> p;
  const int* row = a.topk > 0 ? a.idx + (size_t)t * a.topk : reinterpret_cast<const int*>(g_zero_row);
  const int last = max(a.topk - 1, 0);
  const int tid = opaque((int)threadIdx.x);
#pragma unroll
  for (int m = 0; m < R; ++m) p.v[m] = row[min(s0 + m * NT + tid, last)];
  __builtin_amdgcn_sched_barrier(0);   // all loads in flight before the first select
#pragma unroll
  for (int m = 0; m < R; ++m) p.v[m] = (s0 + m * NT + tid < a.topk) ? p.v[m] : -1;
  return p;
}

// Compact the valid index slots of token t in slot order; entries whose
// compacted position lies in [w_lo, w_lo + kListMax) go to list[pos - w_lo].
// Returns the number of valid slots.  Whole-work-group call (NT threads);
// `first` holds the slots [0, kIdxPre), later rounds are loaded here; wtot
// holds 2 NT / 64 words.
template <int NT>
__device__ __forceinline__ int compact_indices(const KHdr& a, const Tok& k, int t, int* list, int* wtot, int w_lo,
                                               const IdxPre<NT>& first) {
  constexpr int NW = NT / 64, R = IdxPre<NT>::kRounds;
  const int tid = opaque((int)threadIdx.x);
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int base = 0, parity = 0;
  for (int s0 = 0; s0 < k.k_eff; s0 += kIdxPre) {
    const IdxPre<NT> cur = (s0 == 0) ? first : load_indices<NT>(a, t, s0);
#pragma unroll
    for (int m = 0; m < R; ++m) {
      if (s0 + m * NT >= k.k_eff) break;   // wave-uniform
      const int slot = s0 + m * NT + tid;
      const bool ok = (slot < k.k_eff) && (cur.v[m] >= 0) && (cur.v[m] < k.vis);
      const uint64_t bal = __ballot(ok);
      const int pre = __popcll(bal & ((1ull << lane) - 1ull));
      int* wt = wtot + NW * parity;   // the wave totals alternate between two slots,
      parity ^= 1;                   // so one barrier per round suffices
      if (lane == 0) wt[w] = __popcll(bal);
      lds_barrier();
      int off = 0;
      for (int j = 0; j < w; ++j) off += wt[j];
      int tot = 0;
#pragma unroll
      for (int j = 0; j < NW; ++j) tot += wt[j];
      const int pos = base + off + pre;
      if (ok && pos >= w_lo && pos < w_lo + kListMax) list[pos - w_lo] = cur.v[m];
      base += tot;
    }
  }
  lds_barrier();   // the list is complete
  return base;
}

template <int NT>
__device__ __forceinline__ int compact_indices(const KHdr& a, const Tok& k, int t, int* list, int* wtot, int w_lo) {
  return compact_indices<NT>(a, k, t, list, wtot, w_lo, load_indices<NT>(a, t, 0));
}

// The listed ori positions of token t (ori_sparse_indices, slot order) that
// lie in the token's window [lo, hi), compacted into list[0, n) the same way
// (n <= kListMax: the plan bounds ori_topk + topk by it).  Returns n.
// Whole-work-group call; ends with a barrier.
template <int NT>
__device__ __forceinline__ int compact_ori(const KHdr& a, const Tok& k, int t, int* list, int* wtot) {
  constexpr int NW = NT / 64;
  const int tid = opaque((int)threadIdx.x);
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int* row = a.ori_idx + (size_t)t * a.ori_topk;
  int base = 0, parity = 0;
  for (int s0 = 0; s0 < k.ko_eff; s0 += NT) {
    const int slot = s0 + tid;
    const int v = (slot < k.ko_eff) ? row[slot] : -1;
    const bool ok = (slot < k.ko_eff) && (v >= k.lo) && (v < k.hi);
    const uint64_t bal = __ballot(ok);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    int* wt = wtot + NW * parity;
    parity ^= 1;
    if (lane == 0) wt[w] = __popcll(bal);
    lds_barrier();
    int off = 0;
    for (int j = 0; j < w; ++j) off += wt[j];
    int tot = 0;
#pragma unroll
    for (int j = 0; j < NW; ++j) tot += wt[j];
    const int pos = base + off + pre;
    if (ok && pos < kListMax) list[pos] = v;
    base += tot;
  }
  lds_barrier();
  return base;
}

// ---------------------------------------------------------------------------
// key resolution: list position -> cache row (QuantSparseFlashMla, 参数说明:
// the block tables, the band window, cmp_sparse_indices with -1 skipped)
// ---------------------------------------------------------------------------

// Logical token position of key `key` of the token's list (ori band first,
// then cmp entries) and whether it lives in cmp_kv.
// With listed ori keys (ori_topk > 0) the list holds the ori positions first,
// then the compressed entries.
__device__ __forceinline__ int key_pos(const KHdr& a, const Tok& k, int n_o, int key, const int* list, int w_lo,
                                       bool& is_cmp) {
  is_cmp = key >= n_o;
  const bool listed = a.ori_topk > 0;
  if (!is_cmp) return listed ? list[key] : k.lo + key;
  return (a.topk > 0) ? list[(listed ? key : key - n_o) - w_lo] : key - n_o;
}

// The two caches' attributes as uniform registers.  A per-key choice
// between them is then a register select; written as a choice between
// kernel-argument fields, it compiles to a per-lane load from the argument
// segment on every key.
struct Side {
  const uint8_t* kv;
  const float* ds;
  const int32_t* tab;
  int bs, cols, s;
};
struct Sides {
  Side o, c;   // ori_kv, cmp_kv
  bool pow2;   // both block sizes are powers of two: shifts instead of divisions
  int osh, csh;
};

template <class T>
__device__ __forceinline__ T pin_s(T v) {
  asm volatile("" : "+s"(v));
  return v;
}

__device__ __forceinline__ Sides cache_sides(const KHdr& a) {
  Sides x;
  x.o.kv = gptr(pin_s(a.ori_kv)); x.o.ds = gptr(pin_s(a.ori_ds)); x.o.tab = gptr(pin_s(a.ori_tab));
  x.o.bs = pin_s(a.ori_bs); x.o.cols = pin_s(a.ori_cols); x.o.s = pin_s(a.ori_s);
  x.c.kv = gptr(pin_s(a.cmp_kv)); x.c.ds = gptr(pin_s(a.cmp_ds)); x.c.tab = gptr(pin_s(a.cmp_tab));
  x.c.bs = pin_s(a.cmp_bs); x.c.cols = pin_s(a.cmp_cols); x.c.s = pin_s(a.cmp_s);
  const bool op = x.o.bs > 0 && (x.o.bs & (x.o.bs - 1)) == 0, cp = x.c.bs > 0 && (x.c.bs & (x.c.bs - 1)) == 0;
  x.pow2 = op && cp;
  x.osh = op ? __builtin_ctz((unsigned)x.o.bs) : 0;
  x.csh = cp ? __builtin_ctz((unsigned)x.c.bs) : 0;
  return x;
}

// Block index and offset of position j in a paged cache.
struct BlockPos {
  int q, r;
};

__device__ __forceinline__ BlockPos block_pos(const Sides& sd, bool is_cmp, int j) {
  if (sd.pow2) {   // uniform
    const int sh = is_cmp ? sd.csh : sd.osh;
    return BlockPos{j >> sh, j & ((1 << sh) - 1)};
  }
  const int bs = is_cmp ? sd.c.bs : sd.o.bs;
  const int q = j / bs;
  return BlockPos{q, j - q * bs};
}

// blk: the table entry of the position's block; r: its offset in the block.
__device__ __forceinline__ int64_t row_of(const KHdr& a, const Sides& sd, const Tok& k, bool is_cmp, int j, int blk,
                                          int r) {
  if (a.layout_kv == 2) {
    const int bs = is_cmp ? sd.c.bs : sd.o.bs;
    return (int64_t)blk * bs + r;
  }
  if (a.layout_kv == 1) return (int64_t)(is_cmp ? k.cmp0 : k.kv0) + j;
  return (int64_t)k.b * (is_cmp ? sd.c.s : sd.o.s) + j;
}

__device__ __forceinline__ int block_of(const Sides& sd, const Tok& k, bool is_cmp, int q) {
  const int32_t* tab = is_cmp ? sd.c.tab : sd.o.tab;
  const int cols = is_cmp ? sd.c.cols : sd.o.cols;
  return tab[(size_t)k.b * cols + q];
}

// Row of key `key` for the debug export (same resolution code).
__device__ __forceinline__ int64_t resolve_row(const KHdr& a, const Sides& sd, const Tok& k, int n_o, int key,
                                               const int* list, int w_lo) {
  bool is_cmp;
  const int j = key_pos(a, k, n_o, key, list, w_lo, is_cmp);
  BlockPos bp{0, 0};
  if (a.layout_kv == 2) bp = block_pos(sd, is_cmp, j);
  const int blk = (a.layout_kv == 2) ? block_of(sd, k, is_cmp, bp.q) : 0;
  return row_of(a, sd, k, is_cmp, j, blk, bp.r);
}

// Resolving the keys [c0, c1) of a unit into the chunk arrays takes two
// phases.  resolve_rows: all block-table loads of the chunk at once, then
// the row addresses into LDS (slots past c1 point at the zero row) and the
// descale loads, left in flight.  resolve_scales: the descales and
// lam = log2 / inv = 1 / the row's largest descale into LDS (slots past c1:
// zero descales, lam = -inf).  In between, the caller publishes the
// addresses with a barrier and issues the first gathers, so that the rows
// and their descales travel in the same round trip.  Whole-work-group calls.
template <class L>
struct ChunkScales {
  float ds[L::kChunk / L::kNT][L::kNks];
  bool ok[L::kChunk / L::kNT];
};

template <class L>
__device__ __forceinline__ ChunkScales<L> resolve_rows(const KHdr& a, const Tok& k, int n_o, const int* list,
                                                              int w_lo, int c0, int c1, uint8_t* smem) {
  constexpr int M = L::kChunk / L::kNT, NKS = L::kNks;
  uint64_t* kaddr = reinterpret_cast<uint64_t*>(smem + L::kAddr);
  const int tid = opaque((int)threadIdx.x);
  const Sides sd = cache_sides(a);
  ChunkScales<L> cs;
  int j[M], blk[M], off[M];
  bool cmp[M];
  // Slots past the chunk end resolve the chunk's last key (a chunk holds at
  // least one) and then take the zero row: no lane-divergent branch around
  // the loads, so that they are all in flight together.
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int key = c0 + m * L::kNT + tid;
    cs.ok[m] = key < c1;
    j[m] = key_pos(a, k, n_o, cs.ok[m] ? key : c1 - 1, list, w_lo, cmp[m]);
    blk[m] = 0;
    off[m] = 0;
  }
  if (a.layout_kv == 2) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const BlockPos bp = block_pos(sd, cmp[m], j[m]);
      blk[m] = block_of(sd, k, cmp[m], bp.q);
      off[m] = bp.r;
    }
  }
  const uint8_t* zero = g_zero_row;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int64_t row = row_of(a, sd, k, cmp[m], j[m], blk[m], off[m]);
    const uint8_t* kvp = (cmp[m] ? sd.c.kv : sd.o.kv) + row * kD;
    const float* dsp = (cmp[m] ? sd.c.ds : sd.o.ds) + row * NKS;
    kvp = cs.ok[m] ? kvp : zero;
    dsp = cs.ok[m] ? dsp : reinterpret_cast<const float*>(zero);
    if constexpr (L::kPerTile) {
      const v4f x0 = *(const v4f*)dsp;
      const v4f x1 = *(const v4f*)(dsp + 4);
      cs.ds[m][0] = x0[0]; cs.ds[m][1] = x0[1]; cs.ds[m][2] = x0[2]; cs.ds[m][3] = x0[3];
      cs.ds[m][4] = x1[0]; cs.ds[m][5] = x1[1]; cs.ds[m][6] = x1[2]; cs.ds[m][7] = x1[3];
    } else {
      cs.ds[m][0] = *dsp;
    }
    kaddr[m * L::kNT + tid] = (uint64_t)(uintptr_t)kvp;
  }
  return cs;
}

template <class L>
__device__ __forceinline__ void resolve_scales(const ChunkScales<L>& cs, uint8_t* smem) {
  constexpr int M = L::kChunk / L::kNT, NKS = L::kNks;
  float* klam = reinterpret_cast<float*>(smem + L::kLam);
  float* kinv = reinterpret_cast<float*>(smem + L::kInv);
  float* kks = reinterpret_cast<float*>(smem + L::kKs);
  const int tid = opaque((int)threadIdx.x);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int slot = m * L::kNT + tid;
    float lam = kNegInf, inv = 0.f;
    if (cs.ok[m]) {
      float mx = cs.ds[m][0];
#pragma unroll
      for (int c = 1; c < NKS; ++c) mx = fmaxf(mx, cs.ds[m][c]);
#pragma unroll
      for (int c = 0; c < NKS; ++c)
        if (cs.ds[m][c] != cs.ds[m][c]) mx = cs.ds[m][c];   // a NaN descale poisons the row
      mx = (mx == 0.f) ? kMinDescale : mx;
      lam = __log2f(mx);
      inv = 1.0f / mx;
      if (mx != mx) { lam = mx; inv = mx; }
    }
    klam[slot] = lam;
    kinv[slot] = inv;
#pragma unroll
    for (int c = 0; c < NKS; ++c) kks[c * L::kChunk + slot] = cs.ds[m][c];
  }
}

// Both phases with nothing in between (ends with a barrier).
template <class L>
__device__ __forceinline__ void resolve_chunk(const KHdr& a, const Tok& k, int n_o, const int* list, int w_lo,
                                              int c0, int c1, uint8_t* smem) {
  const ChunkScales<L> cs = resolve_rows<L>(a, k, n_o, list, w_lo, c0, c1, smem);
  resolve_scales<L>(cs, smem);
  lds_barrier();
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Gather the rows of chunk tile `tile` into a tile buffer: wave w covers
// rows [16 w, +16) with 8 instructions of 2 rows each (lanes 0-31 and 32-63,
// 16 bytes per lane).  A pair with a row below `nrows` (the tile's valid
// rows) is loaded with global_load_lds_dwordx4 (M0 = LDS destination, lane l
// writes base + 16 l; a lone odd row reads the zero row); a pair past it is
// zeroed with LDS stores, so that stale bytes never reach the MFMAs.  A full
// tile issues exactly 8 vector-memory instructions per wave.  The loads are
// ordered only by the explicit waits of the pipeline, so the compiler does
// not hold the other tiles' LDS reads behind them.
__device__ __forceinline__ void gather_tile(const uint64_t* kaddr, int tile, int nrows, uint8_t* tb, int w) {
  const int lane = opaque((int)threadIdx.x & 63), g = lane >> 5, li = lane & 31;
  uint64_t src[8];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) {   // all row addresses first: one LDS wait for the tile
    const int r = 16 * w + 2 * mi + g;
    src[mi] = kaddr[tile * kTileKeys + r] + 16u * (uint32_t)(li ^ swz(r));
  }
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) {
    const int r0 = 16 * w + 2 * mi;
    if (r0 < nrows) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(tb + r0 * kD));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src[mi]) : "m0");
    } else {
      *(v4i*)(tb + (r0 + g) * kD + 16 * li) = v4i{0, 0, 0, 0};
    }
  }
}

// Valid rows of tile `tile` of a chunk holding nkeys keys.
__device__ __forceinline__ int tile_rows(int nkeys, int tile) { return min(kTileKeys, nkeys - tile * kTileKeys); }

__device__ __forceinline__ void wait_all_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Work-group barrier after which the older of the wave's gathers has landed:
// with `newer_full` set, the 8 loads of the most recent gather (a full tile)
// may still be in flight; otherwise every load is waited for.
// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt unconstrained.
constexpr int kWaitVm0 = 0x0F70;

__device__ __forceinline__ void gather_barrier(bool newer_full) {
  if (newer_full) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// attention kernel
// ---------------------------------------------------------------------------
//
// Wave w: heads [32 hh, +32) with hh = w & 1, output columns [256 dh, +256)
// with dh = w >> 1.  The pair (w, w ^ 2) shares its heads.  For a 64-key
// tile each wave of the pair computes S^T over its half of D for both
// 32-key m-tiles, hands the partner the half it does not own through LDS,
// and runs the softmax of its own 32 keys (m-tile dh); the fp8 P halves are
// swapped back, so that both waves hold P for all 64 keys.
//
// Pipelined by one tile: step i runs P V of tile i in two halves around
// S^T and the softmax of tile i+1, so that the softmax VALU work has MFMAs to
// hide under.  The keys of a chunk are resolved before its first tile; the
// gather of tile i+2 is issued at the start of step i (3 LDS tile buffers).

// Per-lane LDS byte offsets into tile buffer 0, fixed for the whole kernel
// (they include the wave's half of D).  Within a row the 16-byte chunk index
// is XOR-swizzled, so the offsets of the other chunks a lane reads differ
// from a base by an XOR: bit 4 (16-byte half of a K operand), bit 6 (K-step
// parity), bits 5-6 (d-block of a V^T read).  Per step the buffer offset is
// added and the XORs applied (qk_at / tr_at); what varies with the K-step
// pair / d-block group is a multiple of 128 bytes and goes into the ds_read
// immediate offset.
struct LaneOffsets {
  int qk[2];   // [own m-tile / other m-tile]: K row base for S^T = K Q^T
  int tr[4];   // [rho]: V^T transpose-read base
};
struct QkOff {
  int v[2][2][2];   // [own / other m-tile][K-step parity][16-byte half]
};
struct TrOff {
  int v[4][4];      // [rho][d-block mod 4]
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane, int dh) {
  LaneOffsets o;
  const int g = lane >> 5, li = lane & 31;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const int tt = which ? 1 - dh : dh;
    const int key = 32 * tt + li, f = swz(key);
    o.qk[which] = key * kD + 256 * dh + 16 * ((2 * g) ^ f);
  }
  const int trx = (lane >> 4) & 1;
#pragma unroll
  for (int rho = 0; rho < 4; ++rho) {
    const int key = 16 * rho + 8 * ((lane >> 3) & 1) + 4 * (lane >> 5) + ((lane >> 1) & 3);
    const int f = swz(key);
    o.tr[rho] = key * kD + 256 * dh + 8 * (lane & 1) + 16 * ((f & 6) + (trx ^ (f & 1)));
  }
  return o;
}

// chunk (4 sp + 2 g + x) ^ f  =  (2 g ^ f) ^ 4 sp ^ x;  the key and dh terms
// lie above bit 7, so the XOR of the chunk bits commutes with them.
__device__ __forceinline__ QkOff qk_at(const LaneOffsets& o, int boff) {
  QkOff q;
#pragma unroll
  for (int which = 0; which < 2; ++which)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int x = 0; x < 2; ++x) q.v[which][sp][x] = (o.qk[which] ^ (64 * sp + 16 * x)) + boff;
  return q;
}

// chunk ((2 b) ^ (f & 6)) + (trx ^ (f & 1))  =  ((f & 6) + (trx ^ (f & 1))) ^ 2 b
__device__ __forceinline__ TrOff tr_at(const LaneOffsets& o, int boff) {
  TrOff t;
#pragma unroll
  for (int rho = 0; rho < 4; ++rho)
#pragma unroll
    for (int b = 0; b < 4; ++b) t.v[rho][b] = (o.tr[rho] ^ (32 * b)) + boff;
  return t;
}

// K operand (32 keys x 64 d): m-tile `which`, d in [256 dh + 64 s4, +64).
__device__ __forceinline__ v8i read_k(const uint8_t* smem, const QkOff& q, int which, int s4) {
  const int a = s4 >> 1, sp = s4 & 1;
  const v4i lo = *(const v4i*)(smem + q.v[which][sp][0] + 128 * a);
  const v4i hi = *(const v4i*)(smem + q.v[which][sp][1] + 128 * a);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// V^T operand (32 d x 64 keys) of the wave's d-block j (0..7), via LDS transpose reads.
__device__ __forceinline__ v8i read_vt(const uint8_t* smem, const TrOff& t, int j) {
  const int a = j >> 2, b = j & 3;
  v8i av;
#pragma unroll
  for (int rho = 0; rho < 4; ++rho) {
    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(smem + t.v[rho][b] + 128 * a));
    av[2 * rho] = x[0];
    av[2 * rho + 1] = x[1];
  }
  return av;
}

// P of one tile as the B operand of O^T += V^T P^T: byte r of register 4 tt + q
// is key 32 tt + 8 q + 4 g + r.  Per-token descales: an fp8 hi/lo pair.  Per-tile
// descales: P' / vds_max in fp32 (16 values per m-tile), scaled per 64-wide D tile
// at use.
template <int PER_TILE>
struct PTile;
template <>
struct PTile<0> { v8i hi, lo; };
template <>
struct PTile<1> { v16f lt[2]; };

// Per-key arrays of one tile of the current chunk.
template <int PER_TILE>
struct TileView {
  const float* lam;   // [64]
  const float* inv;   // [64]
  const float* ks;    // descale c of key k at ks[c * kChunk + k]
};

template <int PER_TILE>
__device__ __forceinline__ TileView<PER_TILE> tile_view(const uint8_t* smem, int tile) {
  using L = Lds<PER_TILE>;
  TileView<PER_TILE> v;
  v.lam = reinterpret_cast<const float*>(smem + L::kLam) + tile * kTileKeys;
  v.inv = reinterpret_cast<const float*>(smem + L::kInv) + tile * kTileKeys;
  v.ks = reinterpret_cast<const float*>(smem + L::kKs) + tile * kTileKeys;
  return v;
}

// Partial S^T of both m-tiles over this wave's half of D.  Per-tile
// descales scale each 64-wide D tile's partial product before the sum.
template <int PER_TILE>
__device__ __forceinline__ void qk_partial(const uint8_t* smem, const QkOff& o, const TileView<PER_TILE>& tv,
                                           int dh, const v8i (&qreg)[4], int g, v16f& s_own, v16f& s_oth) {
  s_own = v16f{};
  s_oth = v16f{};
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const v8i k_oth = read_k(smem, o, 1, s4);
    const v8i k_own = read_k(smem, o, 0, s4);
    if constexpr (PER_TILE) {
      const v16f p_oth = mma(k_oth, qreg[s4], v16f{});
      const v16f p_own = mma(k_own, qreg[s4], v16f{});
      const float* ks = tv.ks + (4 * dh + s4) * Lds<PER_TILE>::kChunk;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const v4f ko = *(const v4f*)&ks[32 * (1 - dh) + 8 * q4 + 4 * g];
        const v4f km = *(const v4f*)&ks[32 * dh + 8 * q4 + 4 * g];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s_oth[4 * q4 + r] += ko[r] * p_oth[4 * q4 + r];
          s_own[4 * q4 + r] += km[r] * p_own[4 * q4 + r];
        }
      }
    } else {
      s_oth = mma(k_oth, qreg[s4], s_oth);
      s_own = mma(k_own, qreg[s4], s_own);
    }
  }
}

// O^T += V^T P^T for d-blocks [J0, J0 + 4) of this wave's half of D.
template <int PER_TILE, int J0>
__device__ __forceinline__ void pv_half(const uint8_t* smem, const TrOff& o, const TileView<PER_TILE>& tv,
                                        int dh, const PTile<PER_TILE>& P, int g, v16f (&oacc)[8]) {
  if constexpr (PER_TILE) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int c4 = J0 / 2 + c2;             // 64-wide D tile within the half
      const float* ks = tv.ks + (4 * dh + c4) * Lds<PER_TILE>::kChunk;
      v8i ph, pl;
#pragma unroll
      for (int rg = 0; rg < 8; ++rg) {
        const int tt = rg >> 2, q4 = rg & 3;
        const v4f kv = *(const v4f*)&ks[32 * tt + 8 * q4 + 4 * g];
        const v16f& x = P.lt[tt];
        int hv, lv;
        split_fp8(x[4 * q4] * kv[0], x[4 * q4 + 1] * kv[1], x[4 * q4 + 2] * kv[2], x[4 * q4 + 3] * kv[3], hv, lv);
        ph[rg] = hv;
        pl[rg] = lv;
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int j = 2 * c4 + h2;
        const v8i vt = read_vt(smem, o, j);
        oacc[j] = mma(vt, ph, oacc[j]);
        oacc[j] = mma(vt, pl, oacc[j]);
      }
    }
  } else {
    v8i vt = read_vt(smem, o, J0);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = J0 + jj;
      const v8i vn = (jj < 3) ? read_vt(smem, o, j + 1) : vt;   // next operand in flight during these MFMAs
      __builtin_amdgcn_sched_barrier(0);
      oacc[j] = mma(vt, P.hi, oacc[j]);
      oacc[j] = mma(vt, P.lo, oacc[j]);
      __builtin_amdgcn_sched_barrier(0);
      vt = vn;
    }
  }
}

template <int PER_TILE>
__device__ __forceinline__ void put_v16(uint8_t* smem, int off, int w, int lane, const v16f& v) {
  float* p = reinterpret_cast<float*>(smem + off) + (w * 64 + lane) * 16;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) *(v4f*)&p[4 * r4] = v4f{v[4 * r4], v[4 * r4 + 1], v[4 * r4 + 2], v[4 * r4 + 3]};
}

__device__ __forceinline__ v16f get_v16(const uint8_t* smem, int off, int w, int lane) {
  const float* p = reinterpret_cast<const float*>(smem + off) + (w * 64 + lane) * 16;
  v16f v;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const v4f x = *(const v4f*)&p[4 * r4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[4 * r4 + r] = x[r];
  }
  return v;
}

struct WaveCtx {
  int w, lane, g, dh;
  float qs;   // softmax_scale * log2(e) * q descale of the lane's head
};

// Hand the partner the partial scores of the m-tile it owns.
template <int PER_TILE>
__device__ __forceinline__ void scores_publish(uint8_t* smem, const WaveCtx& c, const v16f& s_oth) {
  put_v16<PER_TILE>(smem, Lds<PER_TILE>::kSx, c.w, c.lane, s_oth);
}

// Per-key values of the wave's own 32 keys (m-tile dh) that the softmax of a
// tile needs, loaded ahead of the score exchange.
template <int PER_TILE>
struct KeyVals {
  v4f lam[4], inv[4], kd[PER_TILE ? 1 : 4];
};

template <int PER_TILE>
__device__ __forceinline__ KeyVals<PER_TILE> key_vals(const TileView<PER_TILE>& tv, const WaveCtx& c) {
  KeyVals<PER_TILE> kv;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int kb4 = 32 * c.dh + 8 * q4 + 4 * c.g;
    kv.lam[q4] = *(const v4f*)&tv.lam[kb4];
    kv.inv[q4] = *(const v4f*)&tv.inv[kb4];
    if constexpr (!PER_TILE) kv.kd[q4] = *(const v4f*)&tv.ks[kb4];
  }
  return kv;
}

// Full scores of the own m-tile (own partial + the partner's), turned into
// exponents E = s * log2(e) + log2(vds) in place.  Slots past the end of the
// chunk need no mask: their row is zero and their lam is -inf.  Returns the
// per-head maximum of the half.
template <int PER_TILE>
__device__ __forceinline__ float scores_finish(const uint8_t* smem, const KeyVals<PER_TILE>& kv, const WaveCtx& c,
                                               v16f& s_own) {
  const v16f x = get_v16(smem, Lds<PER_TILE>::kSx, c.w ^ 2, c.lane);
  float mt = kNegInf;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sv = s_own[4 * q4 + r] + x[4 * q4 + r];
      float e;
      if constexpr (PER_TILE) e = sv * c.qs + kv.lam[q4][r];
      else e = sv * (c.qs * kv.kd[q4][r]) + kv.lam[q4][r];
      s_own[4 * q4 + r] = e;
      mt = fmaxf(mt, e);
    }
  }
  return xor32_reduce(mt, true);
}

// P' = 2^(E - Mrun) of the own half; accumulates l += P' / vds_max and
// publishes the half for the partner (fp8 hi/lo words, or fp32 P' / vds_max).
template <int PER_TILE>
__device__ __forceinline__ void probs_half(uint8_t* smem, const KeyVals<PER_TILE>& kv, const WaveCtx& c, float Mrun,
                                           const v16f& ev, float& lsum) {
  const float Ms = (Mrun == kNegInf) ? 0.f : Mrun;
  v16f pv;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(ev[4 * q4 + r] - Ms);
      const float lt = p * kv.inv[q4][r];
      lsum += lt;
      pv[4 * q4 + r] = PER_TILE ? lt : p;
    }
  }
  if constexpr (PER_TILE) {
    put_v16<PER_TILE>(smem, Lds<PER_TILE>::kPx, c.w, c.lane, pv);
  } else {
    int hv[4], lv[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) split_fp8(pv[4 * q4], pv[4 * q4 + 1], pv[4 * q4 + 2], pv[4 * q4 + 3], hv[q4], lv[q4]);
    int* px = reinterpret_cast<int*>(smem + Lds<PER_TILE>::kPx) + (c.w * 64 + c.lane) * 8;
    *(v4i*)&px[0] = v4i{hv[0], hv[1], hv[2], hv[3]};
    *(v4i*)&px[4] = v4i{lv[0], lv[1], lv[2], lv[3]};
  }
}

// P of the whole tile from both halves published by the pair (after a barrier).
template <int PER_TILE>
__device__ __forceinline__ void probs_gather(const uint8_t* smem, const WaveCtx& c, PTile<PER_TILE>& P) {
  const int w0 = c.w & 1, w1 = w0 | 2;   // the pair's waves owning m-tiles 0 and 1
  if constexpr (PER_TILE) {
    P.lt[0] = get_v16(smem, Lds<PER_TILE>::kPx, w0, c.lane);
    P.lt[1] = get_v16(smem, Lds<PER_TILE>::kPx, w1, c.lane);
  } else {
    const int* p0 = reinterpret_cast<const int*>(smem + Lds<PER_TILE>::kPx) + (w0 * 64 + c.lane) * 8;
    const int* p1 = reinterpret_cast<const int*>(smem + Lds<PER_TILE>::kPx) + (w1 * 64 + c.lane) * 8;
    const v4i h0 = *(const v4i*)&p0[0], l0 = *(const v4i*)&p0[4];
    const v4i h1 = *(const v4i*)&p1[0], l1 = *(const v4i*)&p1[4];
    P.hi = v8i{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
    P.lo = v8i{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
  }
}

// Per-head value shared by the pair (w, w ^ 2): the max or the sum of both.
__device__ __forceinline__ float pair_reduce(int* misc, int w, int lane, float v, bool is_max) {
  float* pm = reinterpret_cast<float*>(misc + 64);
  pm[w * 64 + lane] = v;
  lds_barrier();
  const float o = pm[(w ^ 2) * 64 + lane];
  lds_barrier();
  return is_max ? fmaxf(v, o) : v + o;
}

struct UnitState {
  Tok k;
  int t, n_o, w_lo, n_c, kb, ke;
};

// Slide the compacted index window so that it covers the cmp entries of the
// keys [c0, c1); only a token with more than kListMax valid indices moves it.
template <int NT>
__device__ __forceinline__ void cover_chunk(const KHdr& a, UnitState& us, int* list, int* misc, int c0, int c1) {
  if (a.topk > 0 && us.n_c > kListMax) {
    const int need_lo = max(c0 - us.n_o, 0), need_hi = max(c1 - us.n_o, 0);
    if (need_hi > need_lo && (need_lo < us.w_lo || need_hi > us.w_lo + kListMax)) {
      us.w_lo = need_lo;
      compact_indices<NT>(a, us.k, us.t, list, misc, us.w_lo);
    }
  }
}

// One step i of a chunk (tile T in buffer T % 3; bv = i % 3):
//   gather tile i+2 | P V(i), d-blocks 0-3 | barrier: tile i+1 landed
//   | S^T of tile i+1, publish | barrier | softmax of tile i+1, publish P
//   | P V(i), d-blocks 4-7 | barrier | P of tile i+1
// One code path for all three buffers (the buffer offset is added to the
// lane offsets), so that the accumulators keep their registers.
template <int PER_TILE>
__device__ __forceinline__ void pipeline_step(uint8_t* smem, const LaneOffsets& o_in, int nkeys, int tiles, int i, int bv,
                                              const WaveCtx& c, const v8i (&qreg)[4], v16f (&oacc)[8], float Mrun,
                                              float& lsum, PTile<PER_TILE>& P, int* flag) {
  using L = Lds<PER_TILE>;
  LaneOffsets o = o_in;
#pragma unroll
  for (int k = 0; k < 2; ++k) o.qk[k] = opaque(o.qk[k]);
#pragma unroll
  for (int k = 0; k < 4; ++k) o.tr[k] = opaque(o.tr[k]);
  const int bq = (bv == 2) ? 0 : bv + 1, bg = (bq == 2) ? 0 : bq + 1;
  const bool g2 = i + 2 < tiles;
  if (g2)
    gather_tile(reinterpret_cast<const uint64_t*>(smem + L::kAddr), i + 2, tile_rows(nkeys, i + 2),
                smem + L::kTiles + bg * kTileBytes, c.w);
  const TileView<PER_TILE> tv = tile_view<PER_TILE>(smem, i);
  const TrOff tro = tr_at(o, L::kTiles + bv * kTileBytes);
  pv_half<PER_TILE, 0>(smem, tro, tv, c.dh, P, c.g, oacc);
  gather_barrier(g2 && tile_rows(nkeys, i + 2) == kTileKeys);
  const bool has_next = i + 1 < tiles;
  const TileView<PER_TILE> tq = tile_view<PER_TILE>(smem, i + 1);
  v16f s_own, s_oth;
  KeyVals<PER_TILE> kv;
  if (has_next) {
    kv = key_vals<PER_TILE>(tq, c);
    qk_partial<PER_TILE>(smem, qk_at(o, L::kTiles + bq * kTileBytes), tq, c.dh, qreg, c.g, s_own, s_oth);
    scores_publish<PER_TILE>(smem, c, s_oth);
  }
  lds_barrier();
  if (has_next) {
    const float mt = scores_finish<PER_TILE>(smem, kv, c, s_own);
    if (__ballot(mt > Mrun + kTau)) *flag = 1;   // would overflow fp8: the unit is redone
    probs_half<PER_TILE>(smem, kv, c, Mrun, s_own, lsum);
  }
  pv_half<PER_TILE, 4>(smem, tro, tv, c.dh, P, c.g, oacc);
  lds_barrier();
  if (has_next) probs_gather<PER_TILE>(smem, c, P);
}

// Runs the unit's keys [kb, ke) into (oacc, lsum).  With `preset`, Mrun is the
// reference from the redo pass; otherwise the first tile sets it (the pair's
// max maps to 2^4).
template <int PER_TILE>
__device__ __forceinline__ void run_unit(HdrRegs hr, bool preset, UnitState& us, int* list, int* misc, uint8_t* smem,
                                         const LaneOffsets& o, const WaveCtx& c, const v8i (&qreg)[4],
                                         v16f (&oacc)[8], float& Mrun, float& lsum) {
  using L = Lds<PER_TILE>;
  int* flag = misc + 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) oacc[j] = v16f{};
  lsum = 0.f;
  for (int c0 = us.kb; c0 < us.ke; c0 += L::kChunk) {
    const int c1 = min(us.ke, c0 + L::kChunk);
    const KHdr a = hdr_view(hr);
    cover_chunk<kThreads>(a, us, list, misc, c0, c1);
    const int nkeys = c1 - c0, tiles = (nkeys + kTileKeys - 1) / kTileKeys;
    {
      // row addresses -> barrier -> gathers of tiles 0 and 1, then the
      // descales, whose loads were issued with the addresses
      const ChunkScales<L> cs = resolve_rows<L>(a, us.k, us.n_o, list, us.w_lo, c0, c1, smem);
      lds_barrier();
      const uint64_t* kaddr = reinterpret_cast<const uint64_t*>(smem + L::kAddr);
      gather_tile(kaddr, 0, tile_rows(nkeys, 0), smem + L::kTiles, c.w);
      if (tiles > 1) gather_tile(kaddr, 1, tile_rows(nkeys, 1), smem + L::kTiles + kTileBytes, c.w);
      resolve_scales<L>(cs, smem);
    }
    gather_barrier(tiles > 1 && tile_rows(nkeys, 1) == kTileKeys);
    // ---- P of tile 0 ----
    PTile<PER_TILE> P;
    {
      const TileView<PER_TILE> t0 = tile_view<PER_TILE>(smem, 0);
      const KeyVals<PER_TILE> kv = key_vals<PER_TILE>(t0, c);
      v16f s_own, s_oth;
      qk_partial<PER_TILE>(smem, qk_at(o, L::kTiles), t0, c.dh, qreg, c.g, s_own, s_oth);
      scores_publish<PER_TILE>(smem, c, s_oth);
      lds_barrier();
      const float mt = scores_finish<PER_TILE>(smem, kv, c, s_own);
      if (!preset && c0 == us.kb) {   // wave-uniform: every wave takes the same branch
        const float mx = pair_reduce(misc, c.w, c.lane, mt, true);
        Mrun = (mx == kNegInf) ? kNegInf : mx - kPShift;
      } else if (__ballot(mt > Mrun + kTau)) {
        *flag = 1;
      }
      probs_half<PER_TILE>(smem, kv, c, Mrun, s_own, lsum);
      lds_barrier();
      probs_gather<PER_TILE>(smem, c, P);
    }
    // ---- steady state ----
    for (int i = 0, bv = 0; i < tiles; ++i, bv = (bv == 2) ? 0 : bv + 1)
      pipeline_step<PER_TILE>(smem, o, nkeys, tiles, i, bv, c, qreg, oacc, Mrun, lsum, P, flag);
  }
}

// Per-head maximum exponent over the unit (S^T only, not pipelined), for the
// rare unit where a later tile outgrows the first tile's fp8 window.
template <int PER_TILE>
__device__ __forceinline__ float unit_max(HdrRegs hr, UnitState& us, int* list, int* misc, uint8_t* smem,
                                          const LaneOffsets& o, const WaveCtx& c, const v8i (&qreg)[4]) {
  using L = Lds<PER_TILE>;
  float mx = kNegInf;
  for (int c0 = us.kb; c0 < us.ke; c0 += L::kChunk) {
    const int c1 = min(us.ke, c0 + L::kChunk);
    const KHdr a = hdr_view(hr);
    cover_chunk<kThreads>(a, us, list, misc, c0, c1);
    resolve_chunk<L>(a, us.k, us.n_o, list, us.w_lo, c0, c1, smem);
    const int nkeys = c1 - c0, tiles = (nkeys + kTileKeys - 1) / kTileKeys;
    for (int i = 0; i < tiles; ++i) {
      gather_tile(reinterpret_cast<const uint64_t*>(smem + L::kAddr), i, tile_rows(nkeys, i), smem + L::kTiles, c.w);
      gather_barrier(false);
      const TileView<PER_TILE> tv = tile_view<PER_TILE>(smem, i);
      v16f s_own, s_oth;
      qk_partial<PER_TILE>(smem, qk_at(o, L::kTiles), tv, c.dh, qreg, c.g, s_own, s_oth);
      scores_publish<PER_TILE>(smem, c, s_oth);
      lds_barrier();
      mx = fmaxf(mx, scores_finish<PER_TILE>(smem, key_vals<PER_TILE>(tv, c), c, s_own));
      lds_barrier();
    }
  }
  return pair_reduce(misc, c.w, c.lane, mx, true);
}

template <int PER_TILE>
__device__ __forceinline__ void attn_body(KArgPtr ap, uint8_t* smem, int w) {
  using L = Lds<PER_TILE>;
  const int tid = threadIdx.x, lane = tid & 63;
  WaveCtx c;
  c.w = w;
  c.lane = lane;
  c.g = lane >> 5;
  c.dh = w >> 1;
  const int hh = w & 1, g = c.g, dh = c.dh;
  const HdrRegs hr = load_hdr_regs(ap);
  const KHdr a0 = hdr_view(hr);
  const int G = a0.grid;
  const int bid = blockIdx.x;
  const int lw = (G % 8 == 0) ? ((bid & 7) * (G >> 3) + (bid >> 3)) : bid;  // one XCD per contiguous range
  int u_begin = lw, u_end = lw + 1;
  if (a0.n_units != G) {
    u_begin = ap->starts[lw];
    u_end = ap->starts[lw + 1];
  }
  int* list = reinterpret_cast<int*>(smem + L::kList);
  int* misc = reinterpret_cast<int*>(smem + L::kMisc);
  const LaneOffsets o = lane_offsets(lane, dh);

  for (int u = u_begin; u < u_end; ++u) {
    // Settles every load of the previous unit here, where nothing of this
    // unit is in flight yet; without it the compiler guards registers reused
    // across units with a wait placed after this unit's first loads.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    const KHdr a = hdr_view(hr);
    const int h = 32 * hh + (opaque(lane) & 31);   // the lane's head, recomputed per unit
    UnitState us;
    us.t = (a.splits == 1) ? u : u / a.splits;
    const int s = u - us.t * a.splits;
    const int t = us.t;
    // every load of the unit's prologue is issued before any is used: the
    // lengths, index slots, the query fragment (B operand of S^T = K Q^T for
    // d in [256 dh + 64 s4 + 32 g, +32)) and its descale
    const TokLens tl = token_lens(a, t);
    const IdxPre<kThreads> ip = load_indices<kThreads>(a, t, 0);
    v8i qreg[4];
    {
      const uint8_t* qrow = a.q + ((size_t)t * a.n1 + h) * kD + 256 * dh + 32 * g;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const v4i x0 = *(const v4i*)(qrow + 64 * s4);
        const v4i x1 = *(const v4i*)(qrow + 64 * s4 + 16);
        qreg[s4] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
    }
    const float qd = a.q_ds[a.q_ds_per_head ? (size_t)t * a.n1 + h : (size_t)t];
    us.k = token_ctx(a, t, tl);
    c.qs = a.scale_log2 * qd;
    if (!us.k.valid) {   // padded query row: O = 0, lse = -inf
      if (a.splits == 1) {
        for (int x = opaque(lane); x < 32 * 64; x += 64) {
          const int hr = 32 * hh + x / 64, d = 256 * dh + 4 * (x % 64);
          *(uint2*)(a.out + ((size_t)t * a.n1 + hr) * kD + d) = make_uint2(0, 0);
        }
        if (a.lse && dh == 0 && g == 0) a.lse[(size_t)t * a.n1 + h] = kNegInf;
      } else {
        if (dh == 0 && g == 0) {
          a.ws_ml[((size_t)u * kN1 + h) * 2] = kNegInf;
          a.ws_ml[((size_t)u * kN1 + h) * 2 + 1] = -1.0f;   // marks a padded row for the combine
        }
      }
      continue;
    }

    us.n_o = (a.ori_topk > 0) ? compact_ori<kThreads>(a, us.k, t, list, misc) : us.k.hi - us.k.lo;
    us.n_c = 0;
    us.w_lo = 0;
    if (a.topk > 0) us.n_c = compact_indices<kThreads>(a, us.k, t, list + (a.ori_topk > 0 ? us.n_o : 0), misc, 0, ip);
    else if (a.has_cmp) us.n_c = us.k.vis;
    const int64_t n = (int64_t)us.n_o + us.n_c;
    us.kb = (int)(n * s / a.splits);
    us.ke = (int)(n * (s + 1) / a.splits);

    v16f oacc[8];
    float Mrun = kNegInf, lsum = 0.f;
    for (int pass = 0;; ++pass) {
      if (tid == 0) misc[8] = 0;
      run_unit<PER_TILE>(hr, pass > 0, us, list, misc, smem, o, c, qreg, oacc, Mrun, lsum);
      lds_barrier();
      const int redo = misc[8];
      lds_barrier();
      if (!redo || pass > 0) break;
      // recompute with the reference preset from the unit's true maximum
      const float mx = unit_max<PER_TILE>(hr, us, list, misc, smem, o, c, qreg);
      Mrun = (mx == kNegInf) ? kNegInf : mx - kPShift;
    }

    // ---------------- write: final output (one split) or partial state ----------------
    const KHdr ae = hdr_view(hr);
    float lh = xor32_reduce(lsum, false);
    lh = pair_reduce(misc, w, lane, lh, false);   // both key halves
    float sc;
    if (ae.splits == 1) {
      const float sg = ae.sinks ? ae.sinks[h] * kLog2e : kNegInf;
      const float Mf = fmaxf(Mrun, sg);
      float lse_v = kNegInf;
      sc = 0.f;
      if (Mf != kNegInf) {
        const float af = (Mrun == kNegInf) ? 0.f : exp2f(Mrun - Mf);
        const float Lf = af * lh + ((sg == kNegInf) ? 0.f : exp2f(sg - Mf));
        sc = af / Lf;
        lse_v = (Mf + __log2f(Lf)) * kLn2;
      }
      if (ae.lse && dh == 0 && g == 0) ae.lse[(size_t)t * ae.n1 + h] = lse_v;
    } else {
      sc = (lh > 0.f) ? 1.0f / lh : 0.f;
      if (dh == 0 && g == 0) {
        ae.ws_ml[((size_t)u * kN1 + h) * 2] = Mrun;
        ae.ws_ml[((size_t)u * kN1 + h) * 2 + 1] = lh;
      }
    }
    // The wave's 32 heads x 256 columns go through LDS (rows padded to 528
    // bytes), so that each half-wave stores one contiguous 512-byte row.
    lds_barrier();   // every wave is done with the tile buffers
    uint8_t* stage = smem + L::kTiles + w * (32 * kStageRow);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const v16f& ov = oacc[j];
        *(uint2*)(stage + (lane & 31) * kStageRow + 2 * (32 * j + 8 * r4 + 4 * g)) =
            pack_bf16x4(sc * ov[4 * r4], sc * ov[4 * r4 + 1], sc * ov[4 * r4 + 2], sc * ov[4 * r4 + 3]);
      }
    }
    uint16_t* dst = (ae.splits == 1) ? ae.out + (size_t)t * ae.n1 * kD : ae.ws_o + (size_t)u * kN1 * kD;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = 2 * it + g;   // head 32 hh + row
      const v4i x = *(const v4i*)(stage + row * kStageRow + 16 * (lane & 31));
      *(v4i*)(dst + (size_t)(32 * hh + row) * kD + 256 * dh + 8 * (lane & 31)) = x;
    }
  }
}

template <int PER_TILE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_kernel(const KArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Lds<PER_TILE>::kBytes];
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  attn_body<PER_TILE>((KArgPtr)__builtin_amdgcn_kernarg_segment_ptr(), smem, w);
}

// ---------------------------------------------------------------------------
// words shared by the work-groups of one XCD (workspace sync and exchange
// words).  Global atomics act in the L2, which the CUs of an XCD share.
// ---------------------------------------------------------------------------

// A read of a sync word where the atomics act (L2): an atomic add of zero
// that returns the old value, waited for in the same asm.  (A load with the
// workgroup-scope bit may be served by the CU's L1, which would keep
// returning the value it cached first.)
__device__ __forceinline__ int ws_poll(int* p) {
  int v;
  asm volatile("global_atomic_add %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p), "v"(0) : "memory");
  return v;
}
__device__ __forceinline__ int ws_atomic_add(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// The same with the address in a register the compiler cannot see into: a
// uniform-address add would be rewritten into one add per wave plus a scan of
// the lanes, which reads the result at once (and so waits for every load
// issued before it); this one is waited for only where its result is used.
__device__ __forceinline__ int ws_atomic_add_late(int* p, int v) {
  uint64_t q = (uint64_t)(uintptr_t)p;
  asm volatile("" : "+v"(q));
  return __hip_atomic_fetch_add(reinterpret_cast<int*>((uintptr_t)q), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int ws_atomic_xchg(int* p, int v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------------------
// head-split kernel (decode): one work unit = (query token, group of HG = 8
// or 16 heads, key part), over the part's share of the token's key list.
// ---------------------------------------------------------------------------
//
// For a decode batch the tokens are few, and splitting each token's keys
// over work-groups (the kernel above) leaves 64-head partial outputs that a
// second pass must merge.  Here the work-groups of one token divide its heads
// instead and read the same rows, which the XCD's L2 serves after the first.
// With P > 1 key parts, each (token, head group) is also split into P parts
// of whole 128-key tiles run by work-groups of one XCD; the last part merges
// the others' 16-head partials (a 16 KiB exchange, described before dk_body).
//
// 8 waves (two per SIMD, so that one wave's MFMAs, LDS reads and gather
// issues overlap the other's vector work; one wave alone issues at most one
// instruction every four cycles); 128-key tiles (2 LDS buffers).  With
// v_mfma_f32_16x16x128_f8f6f4 (A lane i+16g: row i, k = 32g..32g+31; B lane
// j+16g: column j; D lane j+16g, reg r: element [4g+r][j]):
//   S^T = K Q^T: wave w scores keys [16w, +16) against the HG heads over all
//   of D (4 K-steps of 128), so no score exchange;
//   P' = 2^(E - M) as an fp8 hi + lo pair goes to LDS as [head][key] bytes;
//   O^T += V^T P^T: wave w owns output columns [64w, +64) (4 blocks of 16)
//   over the tile's 128 keys, V^T from ds_read_b64_tr_b8.
// Unused head columns of an 8-head group carry zero q and are not stored.

constexpr int kDkWaves = 8;
constexpr int kDkThreads = 64 * kDkWaves;
constexpr int kDkRows = kDkTileKeys;                  // keys per tile (128)
constexpr int kDkTileBytes = kDkRows * kD;            // 64 KiB
constexpr int kDkPxRow = 144;                         // bytes per head row of P (128 keys + pad)
constexpr int kDkKB = kDkRows / 16 / kDkWaves;        // 16-key S^T blocks per wave
constexpr int kDkDB = kD / 16 / kDkWaves;             // 16-column O^T blocks per wave
constexpr int kDkGI = kDkRows / 4 / kDkWaves;         // gather instructions per wave per half tile
static_assert(kDkKB >= 1 && kDkDB >= 1 && kDkGI % 4 == 0, "wave split");

struct LdsDK {
  static constexpr int kPerTile = 0;
  static constexpr int kNT = kDkThreads;
  static constexpr int kFlag = 2 * kDkWaves;
  static constexpr int kChunk = 1024;
  static constexpr int kNks = 1;
  static constexpr int kTiles = 0;                             // 2 x 64 KiB
  static constexpr int kAddr = 2 * kDkTileBytes;               // uint64 [kChunk]
  static constexpr int kLam = kAddr + 8 * kChunk;              // float [kChunk]
  static constexpr int kInv = kLam + 4 * kChunk;               // float [kChunk]
  static constexpr int kKs = kInv + 4 * kChunk;                // float [kChunk]
  static constexpr int kPx = kKs + 4 * kChunk;                 // fp8 P: [hi, lo][16 heads][kDkPxRow]
  static constexpr int kList = kPx + 2 * 16 * kDkPxRow;        // int [kListMax]
  static constexpr int kMisc = kList + 4 * kListMax;           // [0, 2 waves) compaction, [kFlag, +2) reference flags,
  static constexpr int kBytes = kMisc + 4 * 64 + 4 * 4 * 64;   // [64, 64 + 16 waves) per-head reductions
};
static_assert(LdsDK::kBytes <= 160 * 1024, "LDS");
static_assert(LdsDK::kFlag < 64 && 64 + 16 * kDkWaves <= 64 + 4 * 64, "misc words");

__device__ __forceinline__ v4f mma16(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Gather of chunk tile `tile` (128 keys) into a tile buffer in two halves
// of 64 rows: in half `half`, wave w covers rows [64 half + 8 w, +8) with 4
// instructions of 2 rows.  Every slot of a chunk holds a row address (slots
// past the chunk end hold the zero row), so a tile is always loaded whole.
// The source addresses are formed first (DkSrc), and the instructions are
// then issued one at a time between the MFMAs of a step: the hardware holds
// back a wave's LDS-DMA loads once about a dozen are in flight, and a wave
// stalled on an issue would leave its matrix core idle.
struct DkSrc {
  uint64_t p[kDkGI];
};

// The decode tiles' swizzle: source chunk c (16 bytes) of row r sits at chunk
// c ^ dk_swz(r), a 4-bit value, so that 16 consecutive rows (the K operand
// reads of a key block) and rows 8 m + [0, 8) with 32 + 8 m + [0, 8) (the
// V^T transpose reads of two lane groups) each reach 16 distinct chunks of a
// 256-byte window: every LDS bank once.  dk_swz(r + 64) == dk_swz(r).
__device__ __forceinline__ int dk_swz(int r) { return (r & 15) ^ (((r >> 5) & 1) << 3); }

// Both halves of a tile with one LDS round trip: every read of the
// addresses is issued before the first is used.
__device__ __forceinline__ void dk_src2(const uint64_t* kaddr, int tile, int w, DkSrc& s0, DkSrc& s1) {
  const int lane = opaque((int)threadIdx.x & 63), g = lane >> 5, li = lane & 31;
  constexpr int RW = 2 * kDkGI;   // rows per wave per half
#pragma unroll
  for (int mi = 0; mi < kDkGI; ++mi) {
    s0.p[mi] = kaddr[tile * kDkRows + RW * w + 2 * mi + g];
    s1.p[mi] = kaddr[tile * kDkRows + 64 + RW * w + 2 * mi + g];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mi = 0; mi < kDkGI; ++mi) {
    const uint32_t off = 16u * (uint32_t)(li ^ dk_swz(RW * w + 2 * mi + g));   // dk_swz(r + 64) == dk_swz(r)
    s0.p[mi] += off;
    s1.p[mi] += off;
  }
}

// M0 = the wave's row block of the half, plus the pair's offset added in
// the same asm (per-instruction destinations would otherwise be formed once
// for the whole kernel and held in spilled scalar registers).
// nt (wave-uniform): the non-temporal policy, for work-groups that run one
// unit.  The work-groups of a token then read its rows at about the same
// time, and their gathers ran ~4% faster with it; a work-group that runs
// several units of a token in turn re-reads the rows a unit's time later, and
// such plans lost ~8% with it (so did the whole-token kernel, whose rows
// later tokens reuse).
__device__ __forceinline__ void dk_issue(const DkSrc& s, int mi, int half, uint8_t* tb, int w, bool nt) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(tb + (64 * half + 2 * kDkGI * w) * kD));
  const uint32_t off = (uint32_t)(2 * mi * kD);
  if (nt)
    asm volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(base), "v"(s.p[mi]),
                 "s"(off) : "m0", "scc");
  else
    asm volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(s.p[mi]),
                 "s"(off) : "m0", "scc");
}

// The whole tile at once (both halves).
__device__ __forceinline__ void dk_gather_tile(const uint64_t* kaddr, int tile, uint8_t* tb, int w, bool nt) {
  DkSrc s0, s1;
  dk_src2(kaddr, tile, w, s0, s1);
#pragma unroll
  for (int mi = 0; mi < kDkGI; ++mi) dk_issue(s0, mi, 0, tb, w, nt);
#pragma unroll
  for (int mi = 0; mi < kDkGI; ++mi) dk_issue(s1, mi, 1, tb, w, nt);
}

// Tile 0 of a unit whose keys start with a whole tile of band keys, in a
// paged ori cache with blocks of >= 128 rows (the tile then spans at most two
// blocks), gathered as soon as the token's lengths are known, before its
// index slots are compacted.  The two block-table entries come through scalar
// loads, so this waits neither for the index slots still in flight nor for
// anything queued behind them on the vector memory counter; the row
// addresses are formed in registers (no LDS round trip).
__device__ __forceinline__ void dk_band_tile(const KHdr& a, const Tok& k, uint8_t* tb, int w, bool nt) {
  const int bs = a.ori_bs, cols = a.ori_cols;
  const int b0 = k.lo / bs, split = (b0 + 1) * bs;   // the second block starts at position split
  const ConstI32 trow = (ConstI32)(a.ori_tab + (size_t)k.b * cols);
  const int e0 = trow[b0], e1 = trow[min(b0 + 1, cols - 1)];
  const uint8_t* kv = gptr(a.ori_kv);
  const int lane = opaque((int)threadIdx.x & 63), g = lane >> 5, li = lane & 31;
  constexpr int RW = 2 * kDkGI;
  DkSrc s[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int mi = 0; mi < kDkGI; ++mi) {
      const int r = RW * w + 2 * mi + g;
      const int j = k.lo + 64 * half + r;
      const bool second = j >= split;
      const int64_t row = (int64_t)(second ? e1 : e0) * bs + (j - (second ? split : b0 * bs));
      s[half].p[mi] = (uint64_t)(uintptr_t)(kv + row * kD) + 16u * (uint32_t)(li ^ dk_swz(r));
    }
#pragma unroll
  for (int mi = 0; mi < kDkGI; ++mi) dk_issue(s[0], mi, 0, tb, w, nt);
#pragma unroll
  for (int mi = 0; mi < kDkGI; ++mi) dk_issue(s[1], mi, 1, tb, w, nt);
}

// The next tile's gather: src[h] holds half h's source addresses; half 0 is
// issued between the S^T MFMAs (operator()), half 1 after the exponents.
// Inactive (no next tile) issues nothing.
struct DkFeed {
  DkSrc src[2];
  uint8_t* tb;
  int w;
  bool on, nt;
  __device__ __forceinline__ void operator()(int x) const {
    if (on) dk_issue(src[x / kDkGI], x % kDkGI, x / kDkGI, tb, w, nt);
  }
};

// Per-lane LDS offsets (tile buffer 0) of the wave's K and V^T operand reads.
// In a tile row, source chunk c (16 bytes) sits at chunk c ^ dk_swz(row).
struct DkOffsets {
  int k[kDkKB][2][2];   // [key block b][K-step parity][16-byte half]: row 16 (KB w + b) + i, chunk
                        // (8 k + 2 g + x) ^ dk_swz, + 256 per K-step pair
  int v[4][kDkDB];      // [m][d-block]: V^T transpose reads of keys 32 g + 8 m + .., columns 16 (DB w + db) + ..
};

__device__ __forceinline__ DkOffsets dk_offsets(int lane, int w) {
  DkOffsets o;
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int b = 0; b < kDkKB; ++b) {
    const int row = 16 * (kDkKB * w + b) + i, f = dk_swz(row);
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int x = 0; x < 2; ++x) o.k[b][kp][x] = row * kD + 16 * ((8 * kp + 2 * g + x) ^ f);
  }
  const int L = lane & 15;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int row = 32 * g + 8 * m + (L >> 1), f = dk_swz(row);
#pragma unroll
    for (int db = 0; db < kDkDB; ++db) o.v[m][db] = row * kD + 16 * ((kDkDB * w + db) ^ f) + 8 * (L & 1);
  }
  return o;
}

// S^T blocks (16 keys x 16 heads) of the wave's keys, full D; the next
// K-step's operands are read while the current ones multiply.
__device__ __forceinline__ v8i dk_kop(const uint8_t* tb, const DkOffsets& o, int b, int k) {
  const v4i lo = *(const v4i*)(tb + o.k[b][k & 1][0] + 256 * (k >> 1));
  const v4i hi = *(const v4i*)(tb + o.k[b][k & 1][1] + 256 * (k >> 1));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// kDkGI / 4 gather instructions of `feed` follow each K-step's MFMAs.
__device__ __forceinline__ void dk_qk(const uint8_t* tb, const DkOffsets& o, const v8i (&qreg)[4], v4f (&s)[kDkKB],
                                      const DkFeed& feed) {
  v8i a[kDkKB];
#pragma unroll
  for (int b = 0; b < kDkKB; ++b) {
    s[b] = v4f{0.f, 0.f, 0.f, 0.f};
    a[b] = dk_kop(tb, o, b, 0);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v8i n[kDkKB];
#pragma unroll
    for (int b = 0; b < kDkKB; ++b) n[b] = (k < 3) ? dk_kop(tb, o, b, k + 1) : a[b];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < kDkKB; ++b) s[b] = mma16(a[b], qreg[k], s[b]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < kDkGI / 4; ++x) feed(k * (kDkGI / 4) + x);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < kDkKB; ++b) a[b] = n[b];
  }
}

// O^T[16 (DB w + db), +16][heads] += V^T P^T over the tile's 128 keys.
__device__ __forceinline__ void dk_pv(const uint8_t* tb, const DkOffsets& o, const v8i& phi, const v8i& plo,
                                      v4f (&oacc)[kDkDB]) {
  v8i vt;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(tb + o.v[m][0]));
    vt[2 * m] = x[0];
    vt[2 * m + 1] = x[1];
  }
#pragma unroll
  for (int db = 0; db < kDkDB; ++db) {
    v8i vn = vt;
    if (db < kDkDB - 1) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(tb + o.v[m][db + 1]));
        vn[2 * m] = x[0];
        vn[2 * m + 1] = x[1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    oacc[db] = mma16(vt, phi, oacc[db]);
    oacc[db] = mma16(vt, plo, oacc[db]);
    __builtin_amdgcn_sched_barrier(0);
    vt = vn;
  }
}

// Exponents of the wave's keys (block b, reg r = key 16 (KB w + b) + 4 g + r
// of head j) in place; returns the lane's maximum.
__device__ __forceinline__ float dk_exponents(const uint8_t* smem, int tile, int w, int g, float qs,
                                              v4f (&s)[kDkKB]) {
  const float* lam = reinterpret_cast<const float*>(smem + LdsDK::kLam) + tile * kDkRows;
  const float* ks = reinterpret_cast<const float*>(smem + LdsDK::kKs) + tile * kDkRows;
  float mt = kNegInf;
#pragma unroll
  for (int b = 0; b < kDkKB; ++b) {
    const int k0 = 16 * (kDkKB * w + b) + 4 * g;
    const v4f lv = *(const v4f*)&lam[k0];
    const v4f kv = *(const v4f*)&ks[k0];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = s[b][r] * (qs * kv[r]) + lv[r];
      s[b][r] = e;
      mt = fmaxf(mt, e);
    }
  }
  return mt;
}

// P' = 2^(E - Mrun) as fp8 hi + lo into LDS ([head j][key] bytes); l += P' / vds_max.
__device__ __forceinline__ void dk_probs(uint8_t* smem, int tile, int w, int j, int g, float Mrun,
                                         const v4f (&e)[kDkKB], float& lsum) {
  const float* inv = reinterpret_cast<const float*>(smem + LdsDK::kInv) + tile * kDkRows;
  const float Ms = (Mrun == kNegInf) ? 0.f : Mrun;
  uint8_t* px = smem + LdsDK::kPx + j * kDkPxRow;
#pragma unroll
  for (int b = 0; b < kDkKB; ++b) {
    const int k0 = 16 * (kDkKB * w + b) + 4 * g;
    const v4f iv = *(const v4f*)&inv[k0];
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(e[b][r] - Ms);
      lsum += p[r] * iv[r];
    }
    int hv, lv;
    split_fp8(p[0], p[1], p[2], p[3], hv, lv);
    *(int*)(px + k0) = hv;
    *(int*)(px + 16 * kDkPxRow + k0) = lv;
  }
}

// B operands of P V: lane j+16g holds P[head j][keys 32 g .. +31] (hi, lo).
__device__ __forceinline__ void dk_pread(const uint8_t* smem, int j, int g, v8i& phi, v8i& plo) {
  const uint8_t* px = smem + LdsDK::kPx + j * kDkPxRow + 32 * g;
  const v4i h0 = *(const v4i*)px, h1 = *(const v4i*)(px + 16);
  const v4i l0 = *(const v4i*)(px + 16 * kDkPxRow), l1 = *(const v4i*)(px + 16 * kDkPxRow + 16);
  phi = v8i{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  plo = v8i{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
}

// Per-head value over the waves (lanes j, j+16, j+32, j+48 of each wave
// hold head j): the max or the sum.
__device__ __forceinline__ float dk_heads_reduce(int* misc, int w, int lane, float v, bool is_max) {
  v = xor32_reduce(xor16_reduce(v, is_max), is_max);
  float* red = reinterpret_cast<float*>(misc + 64);
  if (lane < 16) red[w * 16 + lane] = v;
  lds_barrier();
  const int j = lane & 15;
  float x[kDkWaves];
#pragma unroll
  for (int i = 0; i < kDkWaves; ++i) x[i] = red[16 * i + j];
  // No barrier after the reads: every caller passes another barrier (the P
  // barrier after the probabilities, the epilogue's staging barrier, or the
  // next unit's resolution barrier) before any wave writes these words again.
#pragma unroll
  for (int step = kDkWaves / 2; step >= 1; step /= 2)   // pairwise tree
#pragma unroll
    for (int i = 0; i < step; ++i) x[i] = is_max ? fmaxf(x[i], x[i + step]) : x[i] + x[i + step];
  return x[0];
}

// Runs the unit's keys into (oacc, lsum) against the reference Mrun, which the
// first tile sets (its maximum maps to 2^kPShift) and a later tile moves when
// one of its P' would pass 2^kTau: that tile's waves vote through a flag
// (one word per tile parity, read with the P operands after the P barrier),
// then every wave takes the new per-head maximum, rescales its accumulators
// and row sums, and rewrites the tile's P.  Flags start at zero.
__device__ __forceinline__ void dk_run(const KHdr& a, UnitState& us, int* list, int* misc, uint8_t* smem,
                                       const DkOffsets& o, int w, int lane, const v8i (&qreg)[4], float qd,
                                       v4f (&oacc)[kDkDB], float& Mrun, float& lsum, bool nt, bool band_pre) {
  using L = LdsDK;
  const int j = lane & 15, g = lane >> 4;
  int* flag = misc + L::kFlag;   // [2]: by tile parity
  int it = 0;                    // tiles run so far (over the chunks)
#pragma unroll
  for (int db = 0; db < kDkDB; ++db) oacc[db] = v4f{0.f, 0.f, 0.f, 0.f};
  lsum = 0.f;
  const uint64_t* kaddr = reinterpret_cast<const uint64_t*>(smem + L::kAddr);
  for (int c0 = us.kb; c0 < us.ke; c0 += L::kChunk) {
    const int c1 = min(us.ke, c0 + L::kChunk);
    cover_chunk<L::kNT>(a, us, list, misc, c0, c1);
    const int nkeys = c1 - c0, tiles = (nkeys + kDkRows - 1) / kDkRows;
    {
      const ChunkScales<L> cs = resolve_rows<L>(a, us.k, us.n_o, list, us.w_lo, c0, c1, smem);
      lds_barrier();
      if (!(band_pre && c0 == us.kb)) dk_gather_tile(kaddr, 0, smem + L::kTiles, w, nt);   // (else in flight)
      resolve_scales<L>(cs, smem);
    }
    // source addresses of the next tile's gather, formed a step ahead (their
    // LDS round trip overlaps the end of the previous step)
    DkFeed feed;
    feed.w = w;
    feed.nt = nt;
    if (tiles > 1) dk_src2(kaddr, 1, w, feed.src[0], feed.src[1]);
    gather_barrier(false);
    // (formed here, after the wait above, and kept here through an opaque
    // copy: hoisted out of the chunk loop, its wait for the q descale would
    // also wait for the band tile's gathers)
    const float qs = a.scale_log2 * __int_as_float(opaque(__float_as_int(qd)));
    for (int i = 0; i < tiles; ++i, ++it) {
      uint8_t* tb = smem + L::kTiles + (i & 1) * kDkTileBytes;
      const bool next = __builtin_amdgcn_readfirstlane(i + 1 < tiles ? 1 : 0) != 0;
      if (threadIdx.x == 0) flag[(it & 1) ^ 1] = 0;   // the previous tile's flag was read by all
      feed.tb = smem + L::kTiles + ((i + 1) & 1) * kDkTileBytes;
      feed.on = next;
      v4f s[kDkKB];
      dk_qk(tb, o, qreg, s, feed);   // half 0 of tile i+1 goes out between the S^T MFMAs
      const float mt = dk_exponents(smem, i, w, g, qs, s);
      if (c0 == us.kb && i == 0) {   // wave-uniform
        const float mx = dk_heads_reduce(misc, w, lane, mt, true);
        Mrun = (mx == kNegInf) ? kNegInf : mx - kPShift;
      } else if (__ballot(mt > Mrun + kTau)) {
        flag[it & 1] = 1;   // would pass the fp8 range: the reference moves
      }
      if (next) {   // half 1: in flight during the probabilities and P V
#pragma unroll
        for (int mi = 0; mi < kDkGI; ++mi) dk_issue(feed.src[1], mi, 1, feed.tb, w, nt);
      }
      const float lprev = lsum;
      dk_probs(smem, i, w, j, g, Mrun, s, lsum);
      lds_barrier();
      v8i phi, plo;
      dk_pread(smem, j, g, phi, plo);
      if (__builtin_amdgcn_readfirstlane(flag[it & 1])) {
        // every wave's P reads are done at the reduction's first barrier.  The
        // vote is shared by all heads, so a head whose tile maximum stays
        // below its reference keeps it (the reference never moves down: a
        // downward move would scale the history by 2^(Mrun - Mnew), which
        // overflows once a head's earlier maximum is far above this tile's).
        // A head with no finite exponent so far has an empty history.
        const float mx = dk_heads_reduce(misc, w, lane, mt, true);
        const float Mnew = fmaxf(Mrun, mx - kPShift);
        const float fa = (Mrun == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(Mrun - Mnew);
#pragma unroll
        for (int db = 0; db < kDkDB; ++db) oacc[db] *= fa;
        lsum = lprev * fa;
        Mrun = Mnew;
        dk_probs(smem, i, w, j, g, Mrun, s, lsum);
        lds_barrier();
        dk_pread(smem, j, g, phi, plo);
      }
      dk_pv(tb, o, phi, plo, oacc);
      if (i + 2 < tiles) dk_src2(kaddr, i + 2, w, feed.src[0], feed.src[1]);
      gather_barrier(false);   // tile i+1 landed; every wave is done with tile i and with P
    }
  }
}

// ---- key parts: exchange of partial outputs between the parts of a group ----
//
// The parts of one (token, head group) run on one XCD (consecutive units of an
// XCD's range).  Each writing part stores its partial output, normalised by
// its own row sum, as 16-byte words {bf16 pair, tag, bf16 pair, tag} into its
// unit's slot, plus the per-head (max, sum) words; every 8-byte half carries
// the tag, so a reader that sees the tag in a half has that half's data (no
// flag word and no wait for the stores to complete).  The tag is the slot's
// epoch + 1; the merging part (the group's last) bumps the epoch after each
// call, so stale words never match.  Presence word: a writer adds 1 when its
// keys are known; a merger that has waited too long adds 2 and, if the writer
// had not arrived, computes that part itself (the late writer then finds 2,
// stores nothing and clears the word); a merger that finds the writer arrived
// waits longer, then also computes the part itself.  So every wait is bounded
// and the result never depends on a writer being scheduled; the words return
// to zero by the end of every launch.

constexpr uint64_t kDkWaitTicks2 = 20000;   // s_memrealtime ticks (100 MHz) a merger waits for an arrived writer

__device__ __forceinline__ uint8_t* xch_slot(const KHdr& a, int unit) {
  return a.ws_xch + (size_t)unit * kXchSlotBytes;
}

// Keys [lo(p), lo(p + 1)) of part p of P: whole 128-key tiles, the earlier
// parts taking the larger shares.
__device__ __forceinline__ int dk_part_lo(int p, int P, int nkeys) {
  const int nt = (nkeys + kDkRows - 1) / kDkRows;
  return min(nkeys, ((p * nt + P - 1) / P) * kDkRows);
}

// A writer's slot: its partial output O / l (bf16) and (max, sum) per head.
__device__ __forceinline__ void dk_xch_write(uint8_t* slot, uint32_t tag, int w, int lane, const v4f (&o)[kDkDB],
                                             float Mrun, float lh) {
  const int j = lane & 15, g = lane >> 4;
  const float inv = (lh > 0.f) ? 1.0f / lh : 0.f;
#pragma unroll
  for (int db = 0; db < kDkDB; ++db) {
    const int quad = 4 * (kDkDB * w + db) + g;   // columns 4 quad .. +3
    const v4i x{(int)pack_bf16x2(o[db][0] * inv, o[db][1] * inv), (int)tag,
                (int)pack_bf16x2(o[db][2] * inv, o[db][3] * inv), (int)tag};
    *(v4i*)(slot + kXchData + (size_t)(quad * 16 + j) * 16) = x;
  }
  if (w == 0 && g == 0)
    *(v4i*)(slot + kXchMl + 16 * j) = v4i{__float_as_int(Mrun), (int)tag, __float_as_int(lh), (int)tag};
}

// Poll a writer's slot until every word the wave's lanes merge carries `tag`
// (true) or `limit` ticks pass (false).  The words are read as agent-scope
// atomic loads (8 bytes each, the granularity the tags cover), which the
// CU's L1 does not serve, so every round reaches the L2 the writer's stores
// went to.  (Measured on MI355X: plain loads after buffer_inv sc0 kept
// returning the first line the L1 had cached; buffer_inv sc1 before plain
// loads saw the words but cost ~5 us per round.)
__device__ __forceinline__ v4i ld_v4i_agent(const uint8_t* p) {
  uint64_t* q = (uint64_t*)(uintptr_t)p;
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v4i{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)(uint32_t)b, (int)(uint32_t)(b >> 32)};
}

__device__ __forceinline__ bool dk_xch_poll(const uint8_t* slot, uint32_t tag, int w, int lane, v4i (&d)[kDkDB],
                                            v4i& ml, uint64_t limit) {
  const int j = lane & 15, g = lane >> 4;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int db = 0; db < kDkDB; ++db) {
      const int quad = 4 * (kDkDB * w + db) + g;
      d[db] = ld_v4i_agent(slot + kXchData + (size_t)(quad * 16 + j) * 16);
    }
    ml = ld_v4i_agent(slot + kXchMl + 16 * j);
#pragma unroll
    for (int db = 0; db < kDkDB; ++db) ok = ok && (uint32_t)d[db][1] == tag && (uint32_t)d[db][3] == tag;
    ok = ok && (uint32_t)ml[1] == tag && (uint32_t)ml[3] == tag;
    if (__ballot(!ok) == 0) return true;
    if (__builtin_amdgcn_s_memrealtime() - t0 > limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// (M, L, acc) += a partial with maximum M2, row sum L2 and output x * xs
// (x unnormalised with xs = 1, or normalised with xs = L2), all in the log2
// domain of the scores.
__device__ __forceinline__ void dk_acc_merge(float& M, float& L, v4f (&acc)[kDkDB], float M2, float L2,
                                             const v4f (&x)[kDkDB], float xs) {
  const float Mn = fmaxf(M, M2);
  const float f1 = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
  const float f2 = (M2 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M2 - Mn);
  const float fx = f2 * xs;
#pragma unroll
  for (int db = 0; db < kDkDB; ++db) acc[db] = acc[db] * f1 + x[db] * fx;
  L = L * f1 + L2 * f2;
  M = Mn;
}

// All waves' flags ANDed (every wave calls; two barriers).
__device__ __forceinline__ bool wg_all(int* words, int w, bool v) {
  if ((threadIdx.x & 63) == 0) words[w] = v ? 1 : 0;
  lds_barrier();
  int all = 1;
#pragma unroll
  for (int i = 0; i < kDkWaves; ++i) all &= words[i];
  lds_barrier();
  return all != 0;
}

// NT: the gathers use the non-temporal policy (dk_issue); the host picks it
// for plans whose work-groups run one unit each.
template <int NT>
__device__ __forceinline__ void dk_body(KArgPtr ap, uint8_t* smem, int w) {
  using L = LdsDK;
  const int lane = (int)threadIdx.x & 63;
  const HdrRegs hr = load_hdr_regs(ap);
  const KHdr a0 = hdr_view(hr);
  const int G = a0.grid;
  const int bid = blockIdx.x;
  const int lw = (G % 8 == 0) ? ((bid & 7) * (G >> 3) + (bid >> 3)) : bid;  // one XCD per contiguous range
  // With as many units as work-groups the planner's ranges are [g, g + 1)
  // (any valid ranges cover each unit once, and units are independent): no
  // load of the range table then.  Key parts always take one unit per
  // work-group (the grid rounded up to whole XCD rounds of groups).
  int u_begin = lw, u_end = lw + 1;
  if (a0.dk_parts > 1) {
    if (lw >= a0.n_units) return;
  } else if (a0.n_units != G) {
    u_begin = ap->starts[lw];
    u_end = ap->starts[lw + 1];
  }
  const bool nt = NT != 0;
  int* list = reinterpret_cast<int*>(smem + L::kList);
  int* misc = reinterpret_cast<int*>(smem + L::kMisc);
  const DkOffsets o = dk_offsets(lane, w);

  for (int u = u_begin; u < u_end; ++u) {
    // Settles every load of the previous unit here, where nothing of this
    // unit is in flight yet; without it the compiler guards registers reused
    // across units with a wait placed after this unit's first loads.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    const KHdr a = hdr_view(hr);
    const int P = a.dk_parts;                    // 1, 2, 4 or 8
    const int part = u & (P - 1), ub = u - part;  // the group's first unit
    const int ug = u >> (31 - __builtin_clz(P));
    const bool writer = part < P - 1;
    const int lg = (a.hg == 8) ? 3 : 4;          // head groups of 8 or 16
    const int t = ug >> (6 - lg), h0 = (ug & ((kN1 >> lg) - 1)) << lg;
    const int j = opaque(lane) & 15, g = lane >> 4;
    const bool real = j < a.hg;                 // head column j holds a real head
    const int h = h0 + (real ? j : 0);
    // every load of the unit's prologue is issued before any is used: the
    // lengths, index slots, the q fragment (lane j+16g: q[t, h0+j, 128 k +
    // 32 g .. +31] for K-step k; every wave holds all of it), its descale and
    // the group's slot epochs (lane q: writer q's)
    const TokLens tl = token_lens(a, t);
    const IdxPre<L::kNT> ip = load_indices<L::kNT>(a, t, 0);
    // (columns j >= hg read the zero row: no branch around the loads, and no
    // select on the loaded values, which would wait for them here)
    v8i qreg[4];
    {
      const uint8_t* qrow = real ? a.q + ((size_t)t * a.n1 + h) * kD + 32 * g : g_zero_row + 32 * g;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const v4i x0 = *(const v4i*)(qrow + 128 * k);
        const v4i x1 = *(const v4i*)(qrow + 128 * k + 16);
        qreg[k] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
    }
    const float qd_h = *(real ? a.q_ds + (a.q_ds_per_head ? (size_t)t * a.n1 + h : (size_t)t)
                              : reinterpret_cast<const float*>(g_zero_row));
    int ep = 0;
    if (P > 1) ep = *(const int*)xch_slot(a, ub + min(opaque(lane), P - 2));
    UnitState us;
    us.t = t;
    us.k = token_ctx(a, t, tl);
    if (!us.k.valid) {   // padded query row: O = 0, lse = -inf (written by the merging part)
      if (writer && P > 1) continue;
      for (int x = opaque(lane); x < a.hg * 64; x += 64) {
        const int hr = h0 + x / 64, d = 8 * (x % 64);
        if (w == 0) *(v4i*)(a.out + ((size_t)t * a.n1 + hr) * kD + d) = v4i{0, 0, 0, 0};
      }
      if (a.lse && w == 0 && g == 0 && real) a.lse[(size_t)t * a.n1 + h] = kNegInf;
      continue;
    }
    us.n_o = us.k.hi - us.k.lo;
    us.n_c = 0;
    us.w_lo = 0;
    // tile 0 in flight before the index slots are compacted (dk_band_tile);
    // the first part's range starts at key 0
    const bool band_pre = a.layout_kv == 2 && a.ori_topk == 0 && part == 0 && us.n_o >= kDkRows &&
                          a.ori_bs >= kDkRows;
    if (band_pre) dk_band_tile(a, us.k, smem + L::kTiles, w, nt);
    if (a.topk > 0) us.n_c = compact_indices<L::kNT>(a, us.k, t, list, misc, 0, ip);
    else if (a.has_cmp) us.n_c = us.k.vis;
    const int nkeys = us.n_o + us.n_c;
    int run_lo = dk_part_lo(part, P, nkeys), run_hi = dk_part_lo(part + 1, P, nkeys);
    // a writer with keys announces itself (the result is read at the end)
    int pres_old = 0;
    int* pres = reinterpret_cast<int*>(xch_slot(a, u) + 64);
    if (P > 1 && writer && run_hi > run_lo && threadIdx.x == 0) {
      if (a.dk_test == 1) {   // test hook: arrive only once the merger has given up (bounded)
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (!(ws_poll(pres) & 2) && __builtin_amdgcn_s_memrealtime() - t0 < 100000) __builtin_amdgcn_s_sleep(8);
      }
      pres_old = ws_atomic_add_late(pres, 1);
    }

    // Own keys, then (a merger) the writers' partials; a writer part the
    // merger had to take over is run here too, one range per pass.
    float accM = kNegInf, accL = 0.f;
    v4f acc[kDkDB];
#pragma unroll
    for (int db = 0; db < kDkDB; ++db) acc[db] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t todo = 0;
    bool polled = false;
    for (;;) {
      us.kb = run_lo;
      us.ke = run_hi;
      v4f oacc[kDkDB];
      float Mrun = kNegInf, lsum = 0.f;
      if (threadIdx.x < 2) misc[L::kFlag + threadIdx.x] = 0;   // seen at dk_run's first barrier
      dk_run(a, us, list, misc, smem, o, w, lane, qreg, qd_h, oacc, Mrun, lsum, nt, band_pre && !polled);
      if (threadIdx.x == 0) misc[49] = pres_old;   // (after the run: its atomic is long back) seen after the reduction's barriers
      const float lh = dk_heads_reduce(misc, w, lane, lsum, false);
      if (P == 1) {
        accM = Mrun;
        accL = lh;
#pragma unroll
        for (int db = 0; db < kDkDB; ++db) acc[db] = oacc[db];
        break;
      }
      if (writer) {
        if (run_hi > run_lo) {
          if (misc[49] & 2) {   // the merger took this part over
            if (threadIdx.x == 0) ws_atomic_xchg(pres, 0);
          } else {
            dk_xch_write(xch_slot(a, u), (uint32_t)__builtin_amdgcn_readlane(ep, part) + 1u, w, lane, oacc, Mrun, lh);
          }
        }
        break;
      }
      dk_acc_merge(accM, accL, acc, Mrun, lh, oacc, 1.f);
      if (!polled) {
        polled = true;
        const uint64_t lim1 = (uint64_t)a.dk_ticks, lim2 = (a.dk_test == 2) ? 0 : kDkWaitTicks2;
        for (int q = 0; q < P - 1; ++q) {
          if (dk_part_lo(q + 1, P, nkeys) <= dk_part_lo(q, P, nkeys)) continue;   // no keys: nothing written
          uint8_t* sq = xch_slot(a, ub + q);
          int* wq = reinterpret_cast<int*>(sq + 64);
          const uint32_t eq = (uint32_t)__builtin_amdgcn_readlane(ep, q);
          v4i d[kDkDB], ml;
          bool ok = wg_all(misc + 32, w, dk_xch_poll(sq, eq + 1u, w, lane, d, ml, lim1));
          int old = 1;
          if (!ok) {
            if (threadIdx.x == 0) misc[48] = ws_atomic_add(wq, 2);
            lds_barrier();
            old = misc[48];
            lds_barrier();
            if (old & 1) ok = wg_all(misc + 32, w, dk_xch_poll(sq, eq + 1u, w, lane, d, ml, lim2));
          }
          if (ok) {
            v4f x[kDkDB];
#pragma unroll
            for (int db = 0; db < kDkDB; ++db)
              x[db] = v4f{__uint_as_float((uint32_t)d[db][0] << 16), __uint_as_float((uint32_t)d[db][0] & 0xffff0000u),
                          __uint_as_float((uint32_t)d[db][2] << 16), __uint_as_float((uint32_t)d[db][2] & 0xffff0000u)};
            const float Lq = __int_as_float(ml[2]);
            dk_acc_merge(accM, accL, acc, __int_as_float(ml[0]), Lq, x, Lq);
          } else {
            todo |= 1u << q;
          }
          if (threadIdx.x == 0) {
            if (old & 1) ws_atomic_xchg(wq, 0);   // (an absent writer clears the word when it comes)
            *(int*)sq = (int)(eq + 1u);           // the slot's next epoch
          }
        }
      }
      if (!todo) break;
      const int q = __builtin_ctz(todo);
      todo &= todo - 1u;
      run_lo = dk_part_lo(q, P, nkeys);
      run_hi = dk_part_lo(q + 1, P, nkeys);
    }
    if (P > 1 && writer) {
      if (u + 1 < u_end) lds_barrier();
      continue;
    }

    // ---------------- epilogue: normalise, add the sink, bf16 through LDS ----------------
    const KHdr& ae = a;
    const float sg = (ae.sinks && real) ? ae.sinks[h] * kLog2e : kNegInf;
    const float Mf = fmaxf(accM, sg);
    float lse_v = kNegInf, sc = 0.f;
    if (Mf != kNegInf) {
      const float af = (accM == kNegInf) ? 0.f : exp2f(accM - Mf);
      const float Lf = af * accL + ((sg == kNegInf) ? 0.f : exp2f(sg - Mf));
      sc = af / Lf;
      lse_v = (Mf + __log2f(Lf)) * kLn2;
    }
    if (ae.lse && w == 0 && g == 0 && real) ae.lse[(size_t)t * ae.n1 + h] = lse_v;
    // stage [16 heads][512 columns] bf16 (rows padded to 1040 bytes)
    constexpr int kRow = 2 * kD + 16;
#pragma unroll
    for (int db = 0; db < kDkDB; ++db) {
      const int d = 16 * (kDkDB * w + db) + 4 * g;
      *(uint2*)(smem + j * kRow + 2 * d) = pack_bf16x4(sc * acc[db][0], sc * acc[db][1], sc * acc[db][2], sc * acc[db][3]);
    }
    lds_barrier();
    // wave w stores head rows w, w + waves, ...: a row is 1 KiB = 64 lanes x 16 bytes.
    // Non-temporal: where a work-group runs several units, the rows then do
    // not push the next unit's key rows out of L2.
    for (int row = w; row < ae.hg; row += kDkWaves) {
      const v4i x = *(const v4i*)(smem + row * kRow + 16 * lane);
      __builtin_nontemporal_store(x, (v4i*)(ae.out + ((size_t)t * ae.n1 + h0 + row) * kD + 8 * lane));
    }
    if (u + 1 < u_end) lds_barrier();   // the staging area is read before the next unit's gathers
  }
}

template <int NT>
__global__ void __launch_bounds__(kDkThreads) __attribute__((amdgpu_waves_per_eu(kDkWaves / 4, kDkWaves / 4)))
dk_kernel(const KArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LdsDK::kBytes];
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  dk_body<NT>((KArgPtr)__builtin_amdgcn_kernarg_segment_ptr(), smem, w);
}

// ---------------------------------------------------------------------------
// split-KV combine: merge the sink-free partial states of every split with
// the log-sum-exp rule and add the sink logit once.  A block is (token, 8
// heads); 256 threads = 8 heads x 32 x 16 columns.  All loads of a batch of 8
// splits are issued before any is used.
//
// The partial states of a token are read on the XCD that wrote them: work-
// groups are dispatched to the 8 XCDs round-robin by block id, and the
// attention kernel gives XCD x the units of logical work-groups
// [x G/8, (x+1) G/8).  Block b serves XCD b % 8; its tokens are those whose
// first unit XCD x computed.  (Reading another XCD's fresh partials costs
// several microseconds at the kernel boundary.)
// ---------------------------------------------------------------------------

// Tokens whose first split was computed by XCD x: [t0, t1).
// With one unit per work-group the ranges are [g, g + 1) (no load of the
// range table, whose read would precede the partials' loads).
__host__ __device__ __forceinline__ void xcd_tokens(const KArgs& a, int x, int& t0, int& t1) {
  const int per = a.grid / 8;
  const bool one = a.n_units == a.grid;
  const int u0 = one ? x * per : a.starts[x * per], u1 = one ? (x + 1) * per : a.starts[(x + 1) * per];
  t0 = (u0 + a.splits - 1) / a.splits;
  t1 = (u1 + a.splits - 1) / a.splits;
}

__global__ void __launch_bounds__(256) combine_kernel(const KArgs a) {
  int t, hg;
  if (a.grid % 8 == 0) {
    const int x = blockIdx.x % 8, k = blockIdx.x / 8;
    int t0, t1;
    xcd_tokens(a, x, t0, t1);
    t = t0 + k / 8;
    hg = k % 8;
    if (t >= t1) return;
  } else {
    t = blockIdx.x / 8;
    hg = blockIdx.x % 8;
  }
  const int h = hg * 8 + (threadIdx.x >> 5);
  const int col = (threadIdx.x & 31) * 16;
  const int S = a.splits;
  uint16_t* dst = a.out + ((size_t)t * a.n1 + h) * kD + col;
  const float* ml = a.ws_ml + ((size_t)t * S * kN1 + h) * 2;   // split s at + s * kN1 * 2
  const size_t ostride = (size_t)kN1 * kD;
  const uint16_t* op = a.ws_o + ((size_t)t * S * kN1 + h) * kD + col;
  const float sg = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
  // Eight splits at a time, every load of a group (the (m, l) pairs and the
  // partial rows) issued together; the running maximum starts at the sink and
  // the sums are rescaled when a later group raises it (one group, so one
  // round trip, for up to eight splits).
  float M = sg, L = 0.f;
  bool padded = false;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float m8[8], l8[8];
    uint4 x0[8], x1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sj = min(s0 + j, S - 1);   // past S: split S - 1 again, weighed zero
      m8[j] = ml[(size_t)sj * kN1 * 2];
      l8[j] = ml[(size_t)sj * kN1 * 2 + 1];
      const uint4* src = (const uint4*)(op + (size_t)sj * ostride);
      x0[j] = src[0];
      x1[j] = src[1];
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = s0 + j < S;
      Mn = in ? fmaxf(Mn, m8[j]) : Mn;
      padded |= in && l8[j] < 0.f;
    }
    const float fa = (M == kNegInf) ? 0.f : exp2f(M - Mn);   // (the sink's own weight is added at the end)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] *= fa;
    L *= fa;
    M = Mn;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wgt = (s0 + j >= S || m8[j] == kNegInf) ? 0.f : l8[j] * exp2f(m8[j] - M);
      L += wgt;
      const uint32_t xs[8] = {x0[j].x, x0[j].y, x0[j].z, x0[j].w, x1[j].x, x1[j].y, x1[j].z, x1[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[2 * e] += wgt * __uint_as_float(xs[e] << 16);
        acc[2 * e + 1] += wgt * __uint_as_float(xs[e] & 0xffff0000u);
      }
    }
  }
  if (padded || M == kNegInf) {
    L = 0.f;
  } else if (sg != kNegInf) {
    L += exp2f(sg - M);
  }
  const float inv = (L > 0.f) ? 1.0f / L : 0.f;
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  *(uint4*)dst = make_uint4(o[0], o[1], o[2], o[3]);
  *(uint4*)(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
  if (a.lse && (threadIdx.x & 31) == 0)
    a.lse[(size_t)t * a.n1 + h] = (!padded && L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------------------
// debug export of the resolved key rows (same resolution code as above)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) debug_resolve_kernel(const KArgs a, int32_t* keys, int32_t* counts,
                                                                 int32_t max_keys) {
  __shared__ int list[kListMax];
  __shared__ int wtot[8];
  const int t = blockIdx.x;
  const Sides sd = cache_sides(a);
  const Tok k = token_ctx(a, t);
  const int n_o = (a.ori_topk > 0) ? compact_ori<kThreads>(a, k, t, list, wtot) : k.hi - k.lo;
  int n_c = 0;
  if (a.topk > 0) n_c = compact_indices<kThreads>(a, k, t, list + (a.ori_topk > 0 ? n_o : 0), wtot, 0);
  else if (a.has_cmp) n_c = k.vis;
  if (threadIdx.x == 0) { counts[2 * t] = n_o; counts[2 * t + 1] = n_c; }
  const int n = min(n_o + n_c, max_keys);
  int w_lo = 0;
  for (int c0 = 0; c0 < n; c0 += kListMax) {
    const int c1 = min(n, c0 + kListMax);
    if (a.topk > 0 && n_c > kListMax) {
      const int need_lo = max(c0 - n_o, 0), need_hi = max(c1 - n_o, 0);
      if (need_hi > need_lo && (need_lo < w_lo || need_hi > w_lo + kListMax)) {
        w_lo = need_lo;
        compact_indices<kThreads>(a, k, t, list, wtot, w_lo);
      }
    }
    for (int key = c0 + threadIdx.x; key < c1; key += kThreads)
      keys[(size_t)t * max_keys + key] = (int32_t)resolve_row(a, sd, k, n_o, key, list, w_lo);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// prefill kernel: one work unit = one query token, all 64 heads, over the
// token's whole key list (ori band positions, then the compacted cmp
// entries), so no split partials exist.  QuantSparseFlashMla, 功能说明 (the
// formula and the SWA / CSA / HCA key sets); KvQuantSparseAttnSharedkv,
// 参数说明 (per-64-column KV descales).
// ---------------------------------------------------------------------------
//
// 8 waves (two per SIMD).  The work-group walks its range of tokens as one
// stream of 64-key tiles.  Step s computes tile s from LDS only:
//   S^T = K Q^T in fp8 (v_mfma_f32_32x32x64_f8f6f4): wave w = kb + 2 hb + 4 dh
//     scores keys [32 kb, +32) against heads [32 hb, +32) over D half dh, one
//     64-wide D tile per MFMA, so that a per-tile K descale multiplies an
//     exact fp32 partial; the two D halves meet in LDS and each wave finishes
//     16 of its 32 keys,
//   the softmax in log2 units against a per-head reference that moves only
//     when a tile's maximum passes it by 2^8 (every wave then rescales its
//     accumulators by the same factor),
//   O^T += V^T P^T in f16 (v_mfma_f32_32x32x16_f16): wave w owns output
//     columns [64 w, +64), which is exactly D tile w, so each V value is
//     dequantized once, in registers, after the LDS transpose read
//     (ds_read_b64_tr_b8): V' = e4m3 value * vds[key][w] / vmax[key] in f16,
//     with log2 vmax[key] folded into the exponent of P.
// At the boundary after step s one wait covers every vector-memory access of
// the last boundary; then tile s+2 goes HBM -> LDS (global_load_lds_dwordx4
// into the buffer tile s used) with its descales, the row addresses of tile
// s+3 are formed from its block-table entries, and tile s+4's key positions
// are resolved and its block-table loads issued.  Every global load is
// consumed one boundary after it is issued.
// The K side stays fp8 (exact products); V' and P carry f16 rounding
// (relative 2^-11).
//
// MFMA operand k-slots: in the P V product, lane group g (lanes 32 g..) slot i
// of the 16-key step rho stands for key 16 rho + 8 (i >> 2) + 4 g + (i & 3):
// the byte order of the transpose read, and the order in which the S^T
// accumulator holds a wave's keys (D layout of the 32x32 MFMA: lane l, reg r
// = column l % 32, row 8 (r >> 2) + 4 (l >> 5) + (r & 3)).

constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr float kPfTau = 8.0f;   // a tile maximum above the reference + 8 moves the reference

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

struct LdsPF {
  static constexpr int kTiles = 0;                          // 2 x 32 KiB fp8 tiles (XOR-swizzled chunks)
  static constexpr int kXch = 2 * kTileBytes;               // f32 [8 waves][64 lanes][8]: S^T halves for the partner
  static constexpr int kP = kXch + kPfThreads * 32;         // f16 P [64 heads][8 groups of 8 keys], groups swizzled
  static constexpr int kSc = kP + 64 * 64 * 2;              // 2 sets of per-key scales (tile parity)
  static constexpr int kScKs = 0;                           //   f32 [8 D tiles][64 keys]: K descales (per-tile mode)
  static constexpr int kScVs = 2048;                        //   f16 [8 D tiles][64 slots]: vds / vmax (per-tile mode)
  static constexpr int kScLam = 3072;                       //   f32 [64]: log2 vmax (-inf: empty slot)
  static constexpr int kScInv = 3328;                       //   f32 [64]: 1 / vmax
  static constexpr int kScKd = 3584;                        //   f32 [64]: the key's descale (per-token mode)
  static constexpr int kScBytes = 3840;
  static constexpr int kList = kSc + 2 * kScBytes;          // int [kListMax]: compacted cmp indices (cursor token)
  static constexpr int kMax = kList + 4 * kListMax;         // f32 [8 waves][64]: tile maxima per head
  static constexpr int kL = kMax + 4 * kPfThreads;          // f32 [8 waves][64]: row sums per head (epilogue)
  static constexpr int kMisc = kL + 4 * kPfThreads;         // int: [0,16) compaction, [16,18) flags, [24,32) tiles ring
  // The cursor is at most 5 tokens ahead of the token whose successor's entry
  // is read (it resolves 4 tiles ahead and enters the next token as soon as
  // one is done), so 8 entries are never overwritten before they are read.
  static constexpr int kFlag = 16, kRing = 24, kRingMask = 7;
  static constexpr int kQ = kMisc + 4 * 64;                 // fp8 q staging [64 heads][512], swizzled like a tile
  static constexpr int kKaddr = kQ + kN1 * kD;              // u64 [2][64]: row addresses (tile parity), from wave 0
  static constexpr int kKds = kKaddr + 2 * 64 * 8;          // u64 [2][64]: descale addresses (tile parity), from wave 0
  static constexpr int kNvalid = kKds + 2 * 64 * 8;         // int [2]: keys of the tile (tile parity)
  static constexpr int kBytes = kNvalid + 16;
};
static_assert(LdsPF::kBytes <= 160 * 1024, "LDS");

__device__ __forceinline__ v16f mma_f16(h8_t a, h8_t b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Eight e4m3 codes (two dwords, byte order) as f16 (exact: every e4m3 value
// is an f16 value).
__device__ __forceinline__ h8_t e4m3x8_f16(v2i x) {
  const h2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.0f, false);
  const h2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.0f, true);
  const h2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.0f, false);
  const h2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.0f, true);
  return h8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// Slot of key k (0..63) in the P-V operand order: 16 rho + 8 g + i.
__device__ __forceinline__ int pf_slot(int k) {
  const int kk = k & 15;
  return (k & 48) + 8 * ((kk >> 2) & 1) + (kk & 3) + 4 * (kk >> 3);
}

// The resolution cursor: the token whose tiles are being resolved, and the
// prefetched lengths and first index slots of the token after it.
struct PfCursor {
  int u, tile, tiles, n_o, n_c;
  Tok k;
  TokLens nl;
  IdxPre<kPfThreads> nip;
};

// Index slots [0, kIdxPre) of token t as loaded (slots past topk read the
// last slot); pf_idx_fix replaces those by -1 where they are used, so that
// the loads stay in flight until then.
__device__ __forceinline__ IdxPre<kPfThreads> pf_idx_raw(const KHdr& a, int t) {
  IdxPre<kPfThreads> p;
  const int* row = a.topk > 0 ? a.idx + (size_t)t * a.topk : reinterpret_cast<const int*>(g_zero_row);
  const int last = max(a.topk - 1, 0);
  const int tid = opaque((int)threadIdx.x);
#pragma unroll
  for (int m = 0; m < IdxPre<kPfThreads>::kRounds; ++m) p.v[m] = row[min(m * kPfThreads + tid, last)];
  return p;
}

__device__ __forceinline__ IdxPre<kPfThreads> pf_idx_fix(const KHdr& a, IdxPre<kPfThreads> p) {
  const int tid = opaque((int)threadIdx.x);
#pragma unroll
  for (int m = 0; m < IdxPre<kPfThreads>::kRounds; ++m) p.v[m] = (m * kPfThreads + tid < a.topk) ? p.v[m] : -1;
  return p;
}

// Enter token c.u (whole-work-group call): its context, the compaction of
// its index slots into `list`, its tile count (at least one: a token with no
// keys still takes one step, which writes its output) into the tiles ring,
// and the prefetch of the next token's lengths and index slots.
__device__ __forceinline__ void pf_enter(const KHdr& a, PfCursor& c, int u_end, int* list, int* misc) {
  c.k = token_ctx(a, c.u, c.nl);
  c.n_o = c.k.hi - c.k.lo;
  c.n_c = 0;
  if (a.topk > 0) c.n_c = compact_indices<kPfThreads>(a, c.k, c.u, list, misc, 0, pf_idx_fix(a, c.nip));
  else if (a.has_cmp) c.n_c = c.k.vis;
  c.n_c = __builtin_amdgcn_readfirstlane(c.n_c);
  c.tiles = max(1, (c.n_o + c.n_c + kTileKeys - 1) / kTileKeys);
  c.tile = 0;
  if (threadIdx.x == 0) misc[LdsPF::kRing + (c.u & LdsPF::kRingMask)] = c.tiles | (c.k.valid ? 0 : 0x10000);
  if (c.u + 1 < u_end) {
    c.nl = token_lens(a, c.u + 1);
    c.nip = pf_idx_raw(a, c.u + 1);
  }
}

// Key resolution runs in wave 0 only, one key of a tile per lane: the
// block-table entry (in flight) and what locates the row.
struct PfKey {
  int blk;
  int64_t rc;   // paged: offset in the block; else the row
  bool cmp, ok;
};

// It reads only the header fields it uses (no cache_sides, which pins all of
// them in scalar registers): this runs in every step.  Lane l resolves list
// position key0 + l; positions at or past key_end are not keys (ok = false).
__device__ __forceinline__ PfKey pf_resolve_keys(const KHdr& a, const PfCursor& c, const int* list, bool live,
                                                 int key0, int key_end) {
  // Branch-free around the table load (a branch would make the compiler wait
  // for it at the join): without a paged key it reads the zero row.
  PfKey r;
  const int n = min(c.n_o + c.n_c, key_end);
  const int key = key0 + (opaque((int)threadIdx.x) & 63);
  const bool any = live && n > key0;   // uniform
  r.ok = live && key < n;
  bool is_cmp = false;
  int j = 0;
  if (any) j = key_pos(a, c.k, c.n_o, min(key, n - 1), list, 0, is_cmp);
  r.cmp = is_cmp;
  const bool paged = a.layout_kv == 2;
  int bq = 0, br = j;
  if (paged) {   // uniform
    const int bs = is_cmp ? a.cmp_bs : a.ori_bs;
    if (((a.cmp_bs & (a.cmp_bs - 1)) | (a.ori_bs & (a.ori_bs - 1))) == 0) {   // both powers of two
      bq = j >> __builtin_ctz((unsigned)bs);
      br = j & (bs - 1);
    } else {
      bq = j / bs;
      br = j - bq * bs;
    }
  }
  const int32_t* tab = is_cmp ? a.cmp_tab : a.ori_tab;
  const int cols = is_cmp ? a.cmp_cols : a.ori_cols;
  const int32_t* tp = (paged && any) ? tab + (size_t)c.k.b * cols + bq : reinterpret_cast<const int32_t*>(g_zero_row);
  r.blk = *gptr(tp);
  if (paged) r.rc = br;
  else if (a.layout_kv == 1) r.rc = (int64_t)(is_cmp ? c.k.cmp0 : c.k.kv0) + j;
  else r.rc = (int64_t)c.k.b * (is_cmp ? a.cmp_s : a.ori_s) + j;
  return r;
}

// The cursor's current tile of its token's list.
__device__ __forceinline__ PfKey pf_resolve(const KHdr& a, const PfCursor& c, const int* list, bool live) {
  return pf_resolve_keys(a, c, list, live, kTileKeys * c.tile, c.n_o + c.n_c);
}

// Move the cursor past its tile (every wave: entering a token compacts its
// index slots with the whole work-group).  The header is read only on entry.
__device__ __forceinline__ void pf_advance(HdrRegs hr, PfCursor& c, int u_end, int* list, int* misc) {
  if (c.u < u_end) {
    if (++c.tile == c.tiles) {
      if (++c.u < u_end) pf_enter(hdr_view(hr), c, u_end, list, misc);
    }
  }
}

// A key's row address and the address of its descales (per-tile: all eight),
// from its block-table entry (which must have landed).  No loads.
struct PfSrc {
  uint64_t addr;
  const float* ds;
  bool ok;
};

template <int PER_TILE>
__device__ __forceinline__ PfSrc pf_src(const KHdr& a, const PfKey& k) {
  int64_t row = k.rc;
  if (a.layout_kv == 2) row += (int64_t)k.blk * (k.cmp ? a.cmp_bs : a.ori_bs);
  const uint8_t* src = (k.cmp ? a.cmp_kv : a.ori_kv) + row * kD;
  const float* dsp = (k.cmp ? a.cmp_ds : a.ori_ds) + row * (PER_TILE ? 8 : 1);
  PfSrc r;
  r.addr = (uint64_t)(uintptr_t)(k.ok ? src : g_zero_row);
  r.ds = gptr(k.ok ? dsp : reinterpret_cast<const float*>(g_zero_row));
  r.ok = k.ok;
  return r;
}

// Swizzle of the prefill kernel's 512-byte LDS rows (key tiles, q staging):
// 16-byte chunk c of row r sits at chunk c ^ (r & 15), so 16 lanes reading
// the same chunk of 16 consecutive rows touch 16 different chunks (256 bytes).
__device__ __forceinline__ int pf_swz(int r) { return r & 15; }

// One LDS-DMA instruction: lane l's 16 (or 4) source bytes to M0 + 16 l (or 4 l).
__device__ __forceinline__ void pf_dma16(uint32_t dst, uint64_t src) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src) : "m0");
}
__device__ __forceinline__ void pf_dma4(uint32_t dst, uint64_t src) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(dst), "v"(src) : "m0");
}

// The tile's 64 rows HBM -> LDS (global_load_lds_dwordx4, M0 = LDS row pair,
// lane l writes chunk l % 32 of row 2 mi + l / 32 and reads source chunk
// (l % 32) ^ pf_swz(row)).  Wave w moves the keys [8 w, +8), whose row addresses
// wave 0 left in `kaddr`.  Not ordered by the compiler: a step boundary waits
// for every vector-memory access.
__device__ __forceinline__ void pf_issue(uint8_t* tb, const uint64_t* kaddr, int w) {
  const int lane = opaque((int)threadIdx.x & 63), g = lane >> 5, li = lane & 31;
  uint64_t src[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int row = 8 * w + 2 * mi + g;
    src[mi] = kaddr[row] + 16u * (uint32_t)(li ^ pf_swz(row));
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
    pf_dma16(__builtin_amdgcn_readfirstlane(lds_addr(tb + (8 * w + 2 * mi) * kD)), src[mi]);
}

// This thread's descale of its key (tid >> 3) of a tile (per-tile: the one of
// D tile tid & 7), from the descale address wave 0 left in `kds` (read with
// pf_scale_addr, which can go ahead of the tile's DMA issue).
__device__ __forceinline__ uint64_t pf_scale_addr(const uint64_t* kds) {
  return kds[opaque((int)threadIdx.x) >> 3];
}
template <int PER_TILE>
__device__ __forceinline__ float pf_load_scale(uint64_t addr) {
  const float* p = gptr(reinterpret_cast<const float*>(addr));
  return p[PER_TILE ? (opaque((int)threadIdx.x) & 7) : 0];
}

// The tile's per-key scales into scale set `set` (thread: key tid >> 3, part
// tid & 7; the key's 8 descales sit in 8 consecutive lanes).  Slots past the
// tile's `nvalid` keys hold zero descales and lam = -inf; a NaN descale
// poisons the key.
// Largest of 8 consecutive lanes' values (DPP: swap lanes 1 apart, 2 apart,
// then mirror within 8).
__device__ __forceinline__ uint32_t max8_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));   // row_half_mirror
  return x;
}

template <int PER_TILE>
__device__ __forceinline__ void pf_scales(uint8_t* set, float s, int nvalid) {
  using L = LdsPF;
  const int tid = opaque((int)threadIdx.x), key = tid >> 3, part = tid & 7;
  const bool ok = key < nvalid;
  // per-tile: the largest |descale| of the key's 8 (as unsigned integers the
  // magnitudes of floats order like the floats, and a NaN orders above every
  // one of them); per-token: the descale itself
  float mx = s;
  if constexpr (PER_TILE) mx = __uint_as_float(max8_u32(__float_as_uint(s) & 0x7fffffffu));
  const float mxd = (mx == 0.f) ? kMinDescale : mx;
  const float lam = ok ? __log2f(mxd) : kNegInf;
  const float inv = ok ? __builtin_amdgcn_rcpf(mxd) : 0.f;   // mxd is a normal float, NaN or inf
  if constexpr (PER_TILE) {
    reinterpret_cast<float*>(set + L::kScKs)[part * 64 + key] = s;
    reinterpret_cast<_Float16*>(set + L::kScVs)[part * 64 + pf_slot(key)] = (_Float16)(s * inv);
  }
  if (part == 0) {
    reinterpret_cast<float*>(set + L::kScLam)[key] = lam;
    reinterpret_cast<float*>(set + L::kScInv)[key] = inv;
    reinterpret_cast<float*>(set + L::kScKd)[key] = s;
  }
}

// S^T of the wave's 32 keys x 32 heads over D half dh (per-tile: each D
// tile's exact partial times that tile's K descale).
// The 32 bytes [256 dh + 64 s4 + 32 g, +32) of row r of a swizzled buffer
// (an MFMA operand of 32x32x64: lane group g holds k = 32 g .. 32 g + 31).
__device__ __forceinline__ v8i pf_op(const uint8_t* buf, int r, int dh, int s4, int g) {
  const uint8_t* row = buf + r * kD;
  const int f = pf_swz(r), c = 16 * dh + 8 * (s4 >> 1) + 4 * (s4 & 1) + 2 * g;
  const v4i lo = *(const v4i*)(row + 16 * (c ^ f));
  const v4i hi = *(const v4i*)(row + 16 * ((c + 1) ^ f));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int PER_TILE>
__device__ __forceinline__ v16f pf_qk(const uint8_t* tb, const v8i (&qf)[4], const float* ks, int kb, int dh,
                                      int lane_in) {
  const int lane = opaque(lane_in), g = lane >> 5, kr = 32 * kb + (lane & 31);
  v8i ka = pf_op(tb, kr, dh, 0, g);
  v16f S = v16f{};
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    v8i kn = ka;
    if (s4 < 3) kn = pf_op(tb, kr, dh, s4 + 1, g);
    const v8i kop = ka, qop = qf[s4];
    ka = kn;
    if constexpr (PER_TILE) {
      const v16f p = mma(kop, qop, v16f{});
      const float* kst = ks + (4 * dh + s4) * 64 + 32 * kb + 4 * g;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const v4f kv = *(const v4f*)(kst + 8 * q4);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[4 * q4 + r] += kv[r] * p[4 * q4 + r];
      }
      __builtin_amdgcn_sched_barrier(0);   // one D tile's partial live at a time
    } else {
      S = mma(kop, qop, S);
    }
  }
  return S;
}

// O^T[64 w + 32 db + .., heads] += V'^T P^T over the tile's 64 keys.
template <int PER_TILE>
__device__ __forceinline__ void pf_pv(const uint8_t* tb, const _Float16* vs, const uint8_t* pb, int w, int lane_in,
                                      v16f (&acc)[2][2]) {
  const int lane = opaque(lane_in), g = lane >> 5, trx = (lane >> 4) & 1;
  const int vkey = 8 * ((lane >> 3) & 1) + 4 * g + ((lane >> 1) & 3);
#pragma unroll
  for (int rho = 0; rho < 4; ++rho) {
    h8_t pop[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = 32 * hb + (lane & 31);
      pop[hb] = __builtin_bit_cast(h8_t, *(const v4i*)(pb + h * 128 + 16 * ((2 * rho + g) ^ (h & 7))));
    }
    h8_t vsc;
    if constexpr (PER_TILE) vsc = *(const h8_t*)(vs + w * 64 + 16 * rho + 8 * g);
    const int key = 16 * rho + vkey, f = pf_swz(key);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int J = 2 * w + db;
      const uint8_t* src = tb + key * kD + 16 * ((2 * J + trx) ^ f) + 8 * (lane & 1);
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)src);
      h8_t va = e4m3x8_f16(x);
      if constexpr (PER_TILE) va = va * vsc;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) acc[db][hb] = mma_f16(va, pop[hb], acc[db][hb]);
    }
  }
}

// Token t's query rows HBM -> the LDS staging buffer (laid out like a key
// tile): wave w moves heads [8 w, +8) by LDS-DMA.
__device__ __forceinline__ void pf_issue_q(uint8_t* qb, const uint8_t* q, int n1, int t, int w) {
  const int lane = opaque((int)threadIdx.x & 63), g = lane >> 5, li = lane & 31;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int h = 8 * w + 2 * mi + g;
    const uint64_t src = (uint64_t)(uintptr_t)(q + ((size_t)t * n1 + h) * kD) + 16u * (uint32_t)(li ^ pf_swz(h));
    pf_dma16(__builtin_amdgcn_readfirstlane(lds_addr(qb + (8 * w + 2 * mi) * kD)), src);
  }
}

// The wave's query fragments from the staging buffer: the B operands of
// S^T = K Q^T for heads [32 hb, +32), D half dh (held for the whole token).
__device__ __forceinline__ void pf_q_frag(const uint8_t* qb, int hb, int dh, int lane_in, v8i (&qf)[4]) {
  const int lane = opaque(lane_in), g = lane >> 5, hr = 32 * hb + (lane & 31);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) qf[s4] = pf_op(qb, hr, dh, s4, g);
}

// The q descale of head h of token t.
__device__ __forceinline__ float pf_qds(const KHdr& a, int t, int h) {
  return a.q_ds[a.q_ds_per_head ? (size_t)t * a.n1 + h : (size_t)t];
}

// P' = 2^(E - M) of the lane's 8 keys (M = -inf: no key seen yet, read as 0),
// written as f16 to the lane's 16-byte group of P; returns sum P' / vmax.
__device__ __forceinline__ float pf_probs(const float (&E)[8], float Mh, v4f iv0, v4f iv1, uint8_t* prow) {
  const float Mz = (Mh == kNegInf) ? 0.f : Mh;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(E[i] - Mz);
  float ls = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) ls += p[i] * iv0[i] + p[4 + i] * iv1[i];
  *(v4i*)prow = v4i{(int)pk_f16(p[0], p[1]), (int)pk_f16(p[2], p[3]), (int)pk_f16(p[4], p[5]), (int)pk_f16(p[6], p[7])};
  return ls;
}

template <int PER_TILE>
__device__ __forceinline__ void pf_body(KArgPtr ap, uint8_t* smem, int w) {
  using L = LdsPF;
  const int lane = opaque((int)threadIdx.x & 63);
  const int kb = w & 1, hb = (w >> 1) & 1, dh = w >> 2;
  const HdrRegs hr = load_hdr_regs(ap);
  const KHdr a0 = hdr_view(hr);
  const int G = a0.grid, bid = blockIdx.x;
  const int lw = (G % 8 == 0) ? ((bid & 7) * (G >> 3) + (bid >> 3)) : bid;   // one XCD per contiguous range
  int u_begin = lw, u_end = lw + 1;
  if (a0.n_units != G) {
    u_begin = ap->starts[lw];
    u_end = ap->starts[lw + 1];
  }
  if (u_begin >= u_end) return;   // uniform over the work-group
  int* list = reinterpret_cast<int*>(smem + L::kList);
  int* misc = reinterpret_cast<int*>(smem + L::kMisc);
  float* xch = reinterpret_cast<float*>(smem + L::kXch);
  float* maxb = reinterpret_cast<float*>(smem + L::kMax);
  float* lbuf = reinterpret_cast<float*>(smem + L::kL);
  uint8_t* pbuf = smem + L::kP;
  if (threadIdx.x < 2) misc[L::kFlag + threadIdx.x] = 0;

  // sink logits (log2 units) of the lane's two output heads
  float sink[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) sink[x] = a0.sinks ? a0.sinks[32 * x + (lane & 31)] * kLog2e : kNegInf;

  // ---- fill the pipeline ----
  // In the loop, every global load is issued right after a step boundary
  // (after that boundary's DMA) and consumed only at the next boundary,
  // after its wait for every vector-memory access: a compiler-placed wait
  // between the two would also wait for the DMA, which it does not count.
  PfCursor cur;
  cur.u = u_begin;
  cur.nl = token_lens(a0, u_begin);
  cur.nip = pf_idx_raw(a0, u_begin);
  pf_enter(a0, cur, u_end, list, misc);
  // Tile stages: in step s wave 0 resolves tile s+2 (block-table loads,
  // during its S^T MFMAs); at the boundary after step s it forms tile s+2's
  // row and descale addresses, then every wave starts tile s+2's DMA and
  // descale loads and turns tile s+1's descales (loaded one boundary
  // earlier) into its scale set.
  const bool w0 = w == 0;
  uint64_t* kaddr = reinterpret_cast<uint64_t*>(smem + L::kKaddr);
  uint64_t* kds = reinterpret_cast<uint64_t*>(smem + L::kKds);
  int* nvalid = reinterpret_cast<int*>(smem + L::kNvalid);
  PfKey kR;          // wave 0: tile s+2's block-table entries (in flight)
  float sB;          // tile s+1's descale of this thread (in flight)
  int nvB;           // tile s+1's key count
  {
    // tiles 0 and 1: resolved, addressed, loaded
#pragma unroll 1
    for (int x = 0; x < 2; ++x) {
      if (w0) {
        const PfKey k = pf_resolve(a0, cur, list, cur.u < u_end);
        const PfSrc r = pf_src<PER_TILE>(a0, k);
        kaddr[64 * x + lane] = r.addr;
        kds[64 * x + lane] = (uint64_t)(uintptr_t)r.ds;
        const int nv = (int)__popcll(__ballot(r.ok));   // the whole wave votes
        if (lane == 0) nvalid[x] = nv;
      }
      pf_advance(hr, cur, u_end, list, misc);
    }
    lds_barrier();
    pf_issue(smem + L::kTiles, kaddr, w);
    pf_issue(smem + L::kTiles + kTileBytes, kaddr + 64, w);
    const float s0 = pf_load_scale<PER_TILE>(pf_scale_addr(kds));
    sB = pf_load_scale<PER_TILE>(pf_scale_addr(kds + 64));
    nvB = nvalid[1];
    pf_scales<PER_TILE>(smem + L::kSc, s0, nvalid[0]);
  }
  const int hq0 = 32 * hb + (lane & 31);   // the lane's head in S^T and the softmax
  pf_issue_q(smem + L::kQ, a0.q, a0.n1, u_begin, w);
  float qc = a0.scale_log2 * pf_qds(a0, u_begin, hq0);
  float qd_next = 0.f;
  v8i qf[4];
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // tiles 0 and 1 and the first token's q landed
  lds_barrier();

  v16f acc[2][2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int x = 0; x < 2; ++x) acc[db][x] = v16f{};
  float Macc[2] = {kNegInf, kNegInf};
  float lsum = 0.f;
  int u = u_begin, ti = 0;
  int ring = __builtin_amdgcn_readfirstlane(misc[L::kRing + (u & L::kRingMask)]);
  int tiles_u = ring & 0xffff;
  bool valid_u = (ring >> 16) == 0;
  // q of a token: LDS-DMA into the staging buffer during the previous
  // token's last step (after its first barrier, when every wave holds its
  // fragments), read into registers at the token's first step

  for (int s = 0;; ++s) {
    const int buf = s & 1, par = s & 1;
    const int ln = opaque(lane), gg = ln >> 5, hq = 32 * hb + (ln & 31);
    const uint8_t* tb = smem + L::kTiles + buf * kTileBytes;
    const uint8_t* set = smem + L::kSc + buf * L::kScBytes;
    if (ti == 0) pf_q_frag(smem + L::kQ, hb, dh, ln, qf);   // a new token's q
    // ---- S^T, the D halves exchanged ----
    if (w0) {   // tile s+2: block-table loads (in flight until the boundary)
      const KHdr a = hdr_view(hr);
      kR = pf_resolve(a, cur, list, cur.u < u_end);
    }
    const v16f S = pf_qk<PER_TILE>(tb, qf, reinterpret_cast<const float*>(set + L::kScKs), kb, dh, ln);
    {
      float* dst = xch + (w * 64 + ln) * 8;
      if (dh) {
        *(v4f*)dst = v4f{S[0], S[1], S[2], S[3]};
        *(v4f*)(dst + 4) = v4f{S[4], S[5], S[6], S[7]};
      } else {
        *(v4f*)dst = v4f{S[8], S[9], S[10], S[11]};
        *(v4f*)(dst + 4) = v4f{S[12], S[13], S[14], S[15]};
      }
    }
    lds_barrier();
    if (threadIdx.x == 0) misc[L::kFlag + (par ^ 1)] = 0;   // the previous step's flag was read by all
    if (ti + 1 == tiles_u && u + 1 < u_end) {   // the next token's q (every wave holds this token's)
      const KHdr a = hdr_view(hr);
      pf_issue_q(smem + L::kQ, a.q, a.n1, u + 1, w);
      qd_next = pf_qds(a, u + 1, hq);
    }
    float E[8];
    {
      const float* src = xch + ((w ^ 4) * 64 + ln) * 8;
      const v4f x0 = *(const v4f*)src, x1 = *(const v4f*)(src + 4);
      const int kt = 32 * kb + 16 * dh + 4 * gg;
      const float* lamp = reinterpret_cast<const float*>(set + L::kScLam) + kt;
      const float* kdp = reinterpret_cast<const float*>(set + L::kScKd) + kt;
      const v4f la0 = *(const v4f*)lamp, la1 = *(const v4f*)(lamp + 8);
      v4f kd0 = v4f{1.f, 1.f, 1.f, 1.f}, kd1 = kd0;
      if constexpr (!PER_TILE) {
        kd0 = *(const v4f*)kdp;
        kd1 = *(const v4f*)(kdp + 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s0 = (dh ? S[8 + i] : S[i]) + x0[i];
        const float s1 = (dh ? S[12 + i] : S[4 + i]) + x1[i];
        E[i] = s0 * (qc * kd0[i]) + la0[i];
        E[4 + i] = s1 * (qc * kd1[i]) + la1[i];
      }
    }
    float m = E[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, E[i]);
    m = xor32_reduce(m, true);
    maxb[w * 64 + ln] = m;
    const float Ms = hb ? Macc[1] : Macc[0];
    if ((ti == 0 || __ballot(m > Ms + kPfTau)) && ln == 0) misc[L::kFlag + par] = 1;   // ti uniform
    // ---- P against the current reference; redone if any wave moves it (a
    // token's first tile has no reference yet: P is written only then) ----
    const float* invp = reinterpret_cast<const float*>(set + L::kScInv) + 32 * kb + 16 * dh + 4 * gg;
    const v4f iv0 = *(const v4f*)invp, iv1 = *(const v4f*)(invp + 8);
    const int pq = 2 * (2 * kb + dh) + gg;
    uint8_t* prow = pbuf + hq * 128 + 16 * (pq ^ (hq & 7));
    float lt = 0.f;
    if (ti != 0) lt = pf_probs(E, Ms, iv0, iv1, prow);
    lds_barrier();
    if (__builtin_amdgcn_readfirstlane(misc[L::kFlag + par])) {   // first tile of a token, or a jump
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        float mn = Macc[x];
#pragma unroll
        for (int y = 0; y < 4; ++y) mn = fmaxf(mn, maxb[((y & 1) + 2 * x + 4 * (y >> 1)) * 64 + (ln & 31)]);
        const float fa = (Macc[x] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(Macc[x] - mn);
        if (ti != 0) {   // uniform; on a token's first tile acc and lsum are zero
#pragma unroll
          for (int db = 0; db < 2; ++db) acc[db][x] *= fa;
          if (x == hb) lsum *= fa;
        }
        Macc[x] = mn;
      }
      lt = pf_probs(E, hb ? Macc[1] : Macc[0], iv0, iv1, prow);
      lds_barrier();
    }
    lsum += lt;
    // ---- O^T += V'^T P^T ----
    pf_pv<PER_TILE>(tb, reinterpret_cast<const _Float16*>(set + L::kScVs), pbuf, w, ln, acc);

    // ---- step boundary: every vector-memory access of the last boundary
    // (tile s+1's DMA, descales, table entries, q, prefetches, stores) done ----
    const bool last = ti + 1 == tiles_u;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    {
      // tile s+1 uses parity buf ^ 1, tile s+2 parity buf
      pf_scales<PER_TILE>(smem + L::kSc + (buf ^ 1) * L::kScBytes, sB, nvB);   // tile s+1
      if (w0) {                                                       // tile s+2: addresses
        const PfSrc r = pf_src<PER_TILE>(hdr_view(hr), kR);
        const int key = opaque(lane) & 63;
        kaddr[64 * buf + key] = r.addr;
        kds[64 * buf + key] = (uint64_t)(uintptr_t)r.ds;
        const int nv = (int)__popcll(__ballot(r.ok));
        if (key == 0) nvalid[buf] = nv;
      }
      if (last) lbuf[w * 64 + ln] = xor32_reduce(lsum, false);       // row sums of the ending token
      lds_barrier();                                                  // tile s is done in every wave
      const uint64_t dsa = pf_scale_addr(kds + 64 * buf);
      nvB = nvalid[buf];
      pf_issue(smem + L::kTiles + buf * kTileBytes, kaddr + 64 * buf, w);   // tile s+2 into tile s's buffer
      sB = pf_load_scale<PER_TILE>(dsa);                              // and its descales
      pf_advance(hr, cur, u_end, list, misc);
    }
    if (last) {
      // ---- epilogue of token u ----
      const KHdr ae = hdr_view(hr);
      const int t = u;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int h = 32 * x + (ln & 31);
        float Ls = 0.f;
#pragma unroll
        for (int y = 0; y < 4; ++y) Ls += lbuf[((y & 1) + 2 * x + 4 * (y >> 1)) * 64 + (ln & 31)];
        const float M = Macc[x], sg = sink[x];
        const float Mf = fmaxf(M, sg);
        float sc = 0.f, lse_v = kNegInf;
        if (valid_u && Mf != kNegInf) {
          const float af = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - Mf);
          const float Lf = af * Ls + ((sg == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sg - Mf));
          sc = af * __builtin_amdgcn_rcpf(Lf);
          lse_v = (Mf + __log2f(Lf)) * kLn2;
        }
        if (ae.lse && w == 0 && gg == 0) ae.lse[(size_t)t * ae.n1 + h] = lse_v;
        // lane (h, g) holds columns 8 q + 4 g + [0, 4) of each 32-column block;
        // v_permlane32_swap trades the upper lanes' even-q half with the lower
        // lanes' odd-q half of each q pair, so that each lane stores 16
        // contiguous bytes: columns 16 k + 8 g + [0, 8)
        uint16_t* orow = ae.out + ((size_t)t * ae.n1 + h) * kD + 64 * w + 8 * gg;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const v16f& o = acc[db][x];
            const int q0 = 2 * k2, q1 = 2 * k2 + 1;
            const uint2 A = pack_bf16x4(sc * o[4 * q0], sc * o[4 * q0 + 1], sc * o[4 * q0 + 2], sc * o[4 * q0 + 3]);
            const uint2 B = pack_bf16x4(sc * o[4 * q1], sc * o[4 * q1 + 1], sc * o[4 * q1 + 2], sc * o[4 * q1 + 3]);
            // lanes 32..63 of the first operand <-> lanes 0..31 of the second:
            // lower lanes end with (A own, A of lane + 32), upper lanes with
            // (B of lane - 32, B own)
            const auto sx = __builtin_amdgcn_permlane32_swap(A.x, B.x, false, false);
            const auto sy = __builtin_amdgcn_permlane32_swap(A.y, B.y, false, false);
            *(uint4*)(orow + 32 * db + 16 * k2) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
          }
      }
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int x = 0; x < 2; ++x) acc[db][x] = v16f{};
      Macc[0] = Macc[1] = kNegInf;
      lsum = 0.f;
      if (++u == u_end) break;
      ti = 0;
      ring = __builtin_amdgcn_readfirstlane(misc[L::kRing + (u & L::kRingMask)]);
      tiles_u = ring & 0xffff;
      valid_u = (ring >> 16) == 0;
      qc = ae.scale_log2 * qd_next;
    } else {
      ++ti;
    }
  }
  // every wave's last loads (of the stream past its end) settle before exit
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

template <int PER_TILE>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(kPfWaves / 4, kPfWaves / 4)))
pf_kernel(const KArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LdsPF::kBytes];
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  pf_body<PER_TILE>((KArgPtr)__builtin_amdgcn_kernarg_segment_ptr(), smem, w);
}

// ---------------------------------------------------------------------------
// split-key decode kernel: one work unit = (query token t, key split s), all
// 64 heads of t against at most 128 consecutive keys of t's list (ori band
// positions, then the compacted cmp entries).  QuantSparseFlashMla, 功能说明
// (the formula and the SWA / CSA / HCA key sets); fused infer-attention page,
// 输出说明 (the log-sum-exp that merges partial results).
// ---------------------------------------------------------------------------
//
// For a decode batch the tokens are few (32 here) and their key lists short
// (~640 keys), so each token's keys are split over S work-groups on one XCD
// (block b runs on XCD b mod 8; the splits of token t take block ids that are
// equal mod 8).  A work-group gathers its (at most two) 64-key tiles at once,
// right after the key resolution, and computes them with the whole-token
// kernel's step code (fp8 S^T with the D halves exchanged through LDS, f16
// P V): no tile pipeline and no online reference, because all of the unit's
// keys are in LDS together and the softmax reference is their exact maximum.
//
// Merge (S > 1): every unit writes its partial (bf16 O normalised by its own
// row sum, and fp32 (max, sum) per head) to the workspace, then arrives at the
// token's counter.  The last arriver starts a new generation of the token's
// sync words; the other units wait for that (a bounded spin: after ~40 us a
// unit leaves, and the work it would have done is claimed by the others) and
// every unit present then claims groups of 8 heads and merges them (log-sum-
// exp rule, sink added once), so the merge is spread over the token's
// work-groups.  The exchange relies on the units of a token sharing one L2:
// partial stores are complete (s_waitcnt) before the arrival atomic, the sync
// words are only touched by L2 atomics or L1-bypassing loads, and a merge
// reads the other units' partial lines for the first time in the launch (so
// its CU's L1 holds none of them).  Each unit also records the XCD it ran on
// (HW_REG_XCC_ID); a merge that finds a partial from another XCD writes NaN
// instead of a result, so a broken placement cannot pass silently.
// Sync words per token: [0] arrivals, [1] generation, [2] claims.  They must
// be zero before a workspace's first use and every call leaves the arrivals
// zero.

constexpr int kSkMaxKeys = 2 * kTileKeys;    // keys per unit: two 64-key tiles in LDS at once
constexpr int kSkHeadGroup = 8;              // heads per merge claim
constexpr int kSkSpinTicks = 4000;           // s_memrealtime ticks (100 MHz): a waiting unit leaves after ~40 us
constexpr int kSkMaxSplitsDev = 16;          // splits per token (the planner's bound)
typedef float v2f __attribute__((ext_vector_type(2)));

struct LdsSK {
  static constexpr int kTiles = 0;                          // 2 x 32 KiB fp8 tiles (whole-token kernel layout)
  static constexpr int kXch = 2 * kTileBytes;               // f32 [2 tiles][8 waves][64 lanes][8]: S^T halves
  static constexpr int kP = kXch + 2 * kPfThreads * 32;     // f16 P [2 tiles][64 heads][64 keys]
  static constexpr int kSc = kP + 2 * 64 * 64 * 2;          // 2 scale sets (LdsPF layout)
  static constexpr int kList = kSc + 2 * LdsPF::kScBytes;   // int [kListMax]: compacted cmp indices
  static constexpr int kMax = kList + 4 * kListMax;         // f32 [8 waves][64]: maxima per head
  static constexpr int kL = kMax + 4 * kPfThreads;          // f32 [8 waves][64]: row sums per head
  static constexpr int kMisc = kL + 4 * kPfThreads;         // int [64]: compaction, broadcast words
  static constexpr int kKaddr = kMisc + 4 * 64;             // u64 [2][64]: row addresses
  static constexpr int kKds = kKaddr + 2 * 64 * 8;          // u64 [2][64]: descale addresses
  static constexpr int kNvalid = kKds + 2 * 64 * 8;         // int [2]: keys of each tile
  static constexpr int kBytes = kNvalid + 16;
};
static_assert(LdsSK::kBytes <= 160 * 1024, "LDS");

__device__ __forceinline__ int sk_xcc_id() {
  int id;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
  return id & 0xf;
}

// The token's q fragments straight from global memory (the B operands of
// S^T = K Q^T for heads [32 hb, +32), D half dh, in the order pf_op reads a
// staged row: lane group g holds bytes 256 dh + 64 s4 + 32 g, +32).
__device__ __forceinline__ void sk_q_frag(const uint8_t* q, int n1, int t, int hb, int dh, int lane, v8i (&qf)[4]) {
  const uint8_t* row = q + ((size_t)t * n1 + 32 * hb + (lane & 31)) * kD + 256 * dh + 32 * (lane >> 5);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const v4i lo = *(const v4i*)(row + 64 * s4);
    const v4i hi = *(const v4i*)(row + 64 * s4 + 16);
    qf[s4] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// Merge heads [8 g, +8) of token t from its S partials (units t S .. t S + S - 1):
// thread tid takes head 8 g + tid / 64 and columns 8 (tid % 64) .. +7.  Every
// load of every split is issued before the first is used (splits past S
// read split 0 again and weigh nothing).
__device__ __forceinline__ void sk_merge(const KHdr& a, int t, int S, int grp, int my_xcc, const int* xcc) {
  constexpr int SM = kSkMaxSplitsDev;
  const int tid = opaque((int)threadIdx.x);
  const int h = kSkHeadGroup * grp + (tid >> 6), col = 8 * (tid & 63);
  const size_t u0 = (size_t)t * S;
  const float sg = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
  v2f mlv[SM];
  uint4 ov[SM];
  int xv[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    const size_t u = u0 + (s < S ? s : 0);
    mlv[s] = *(const v2f*)(a.ws_ml + (u * kN1 + h) * 2);
    ov[s] = *(const uint4*)(a.ws_o + (u * kN1 + h) * kD + col);
    xv[s] = xcc[u];
  }
  float M = sg;
  bool padded = false, foreign = false;
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    if (s < S) {
      M = fmaxf(M, mlv[s][0]);
      padded |= mlv[s][1] < 0.f;
      foreign |= xv[s] != my_xcc;
    }
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float L = 0.f;
  if (!padded && M != kNegInf) {
    L = (sg == kNegInf) ? 0.f : exp2f(sg - M);
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      const float ms = mlv[s][0], ls = mlv[s][1];
      const float wgt = (s >= S || ms == kNegInf) ? 0.f : ls * exp2f(ms - M);
      const uint32_t xs[4] = {ov[s].x, ov[s].y, ov[s].z, ov[s].w};
      L += wgt;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += wgt * __uint_as_float(xs[e] << 16);
        acc[2 * e + 1] += wgt * __uint_as_float(xs[e] & 0xffff0000u);
      }
    }
  }
  float inv = (L > 0.f) ? 1.0f / L : 0.f;
  if (foreign) inv = __builtin_nanf("");
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *(uint4*)(a.out + ((size_t)t * a.n1 + h) * kD + col) = make_uint4(o[0], o[1], o[2], o[3]);
  if (a.lse && (tid & 63) == 0) {
    float lse_v = (!padded && L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
    if (foreign) lse_v = __builtin_nanf("");
    a.lse[(size_t)t * a.n1 + h] = lse_v;
  }
}

template <int PER_TILE>
__device__ __forceinline__ void sk_body(KArgPtr ap, uint8_t* smem, int w) {
  using L = LdsSK;
  const int lane = opaque((int)threadIdx.x & 63), g = lane >> 5;
  const int kb = w & 1, hb = (w >> 1) & 1, dh = w >> 2;
  const HdrRegs hr = load_hdr_regs(ap);
  const KHdr a = hdr_view(hr);
  const int S = a.splits;
  const int bid = blockIdx.x, xq = bid & 7, kq = bid >> 3;
  const int t = xq + 8 * (kq / S), sp = kq - (kq / S) * S;
  if (t >= a.t1) return;   // uniform: an idle block of the last XCD round
  int* list = reinterpret_cast<int*>(smem + L::kList);
  int* misc = reinterpret_cast<int*>(smem + L::kMisc);
  float* maxb = reinterpret_cast<float*>(smem + L::kMax);
  float* lbuf = reinterpret_cast<float*>(smem + L::kL);
  uint64_t* kaddr = reinterpret_cast<uint64_t*>(smem + L::kKaddr);
  uint64_t* kds = reinterpret_cast<uint64_t*>(smem + L::kKds);
  int* nvalid = reinterpret_cast<int*>(smem + L::kNvalid);
  int* sync = a.ws_sync;   // [kSkMaxTokens][4]
  int* xcc = a.ws_xcc;     // [units]

  // ---- every load of the prologue in flight together: lengths, index slots,
  // q fragments and descale, the token's sync generation ----
  const TokLens tl = token_lens(a, t);
  const IdxPre<kPfThreads> ip = pf_idx_raw(a, t);
  v8i qf[4];
  sk_q_frag(a.q, a.n1, t, hb, dh, lane, qf);
  const int hq = 32 * hb + (lane & 31);   // the lane's head in S^T and the softmax
  const float qc = a.scale_log2 * pf_qds(a, t, hq);

  PfCursor c;
  c.u = t;
  c.tile = 0;
  c.k = token_ctx(a, t, tl);
  c.n_o = c.k.hi - c.k.lo;
  c.n_c = 0;
  if (a.topk > 0) c.n_c = compact_indices<kPfThreads>(a, c.k, t, list, misc, 0, pf_idx_fix(a, ip));
  else if (a.has_cmp) c.n_c = c.k.vis;
  c.n_c = __builtin_amdgcn_readfirstlane(c.n_c);
  const int n = c.n_o + c.n_c;
  const int k0 = (int)(((int64_t)n * sp) / S), k1 = (int)(((int64_t)n * (sp + 1)) / S);
  const int nk = k1 - k0;
  const bool over = nk > kSkMaxKeys;          // the plan's key bound was exceeded: poison, never drop keys
  const int ntiles = (nk > kTileKeys) ? 2 : 1;

  // ---- key resolution (waves 0 and 1: one tile each), then both tiles'
  // rows HBM -> LDS and their descales ----
  if (w < ntiles) {
    const PfKey k = pf_resolve_keys(a, c, list, c.k.valid != 0, k0 + kTileKeys * w, k1);
    const PfSrc r = pf_src<PER_TILE>(a, k);
    kaddr[64 * w + lane] = r.addr;
    kds[64 * w + lane] = (uint64_t)(uintptr_t)r.ds;
    const int nv = (int)__popcll(__ballot(r.ok));
    if (lane == 0) nvalid[w] = nv;
  }
  lds_barrier();
  float sd[2];
  for (int x = 0; x < ntiles; ++x) {
    pf_issue(smem + L::kTiles + x * kTileBytes, kaddr + 64 * x, w);
    sd[x] = pf_load_scale<PER_TILE>(pf_scale_addr(kds + 64 * x));
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // rows, descales (and the prologue loads) landed
  for (int x = 0; x < ntiles; ++x) pf_scales<PER_TILE>(smem + L::kSc + x * LdsPF::kScBytes, sd[x], nvalid[x]);
  lds_barrier();

  // ---- S^T per tile, the D halves exchanged through LDS ----
  float E[2][8];
  for (int x = 0; x < ntiles; ++x) {
    const uint8_t* set = smem + L::kSc + x * LdsPF::kScBytes;
    const v16f Sx = pf_qk<PER_TILE>(smem + L::kTiles + x * kTileBytes, qf,
                                    reinterpret_cast<const float*>(set + LdsPF::kScKs), kb, dh, lane);
    float* dst = reinterpret_cast<float*>(smem + L::kXch) + ((x * kPfWaves + w) * 64 + lane) * 8;
    if (dh) {
      *(v4f*)dst = v4f{Sx[0], Sx[1], Sx[2], Sx[3]};
      *(v4f*)(dst + 4) = v4f{Sx[4], Sx[5], Sx[6], Sx[7]};
    } else {
      *(v4f*)dst = v4f{Sx[8], Sx[9], Sx[10], Sx[11]};
      *(v4f*)(dst + 4) = v4f{Sx[12], Sx[13], Sx[14], Sx[15]};
    }
    // the wave keeps its own half of the 16 rows (dh 0: rows 0-7, dh 1: rows 8-15)
#pragma unroll
    for (int i = 0; i < 8; ++i) E[x][i] = dh ? Sx[8 + i] : Sx[i];
  }
  lds_barrier();
  float m = kNegInf;
  for (int x = 0; x < ntiles; ++x) {
    const uint8_t* set = smem + L::kSc + x * LdsPF::kScBytes;
    const float* src = reinterpret_cast<const float*>(smem + L::kXch) + ((x * kPfWaves + (w ^ 4)) * 64 + lane) * 8;
    const v4f x0 = *(const v4f*)src, x1 = *(const v4f*)(src + 4);
    const int kt = 32 * kb + 16 * dh + 4 * g;
    const float* lamp = reinterpret_cast<const float*>(set + LdsPF::kScLam) + kt;
    const float* kdp = reinterpret_cast<const float*>(set + LdsPF::kScKd) + kt;
    const v4f la0 = *(const v4f*)lamp, la1 = *(const v4f*)(lamp + 8);
    v4f kd0 = v4f{1.f, 1.f, 1.f, 1.f}, kd1 = kd0;
    if constexpr (!PER_TILE) {
      kd0 = *(const v4f*)kdp;
      kd1 = *(const v4f*)(kdp + 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s0 = E[x][i] + x0[i];
      const float s1 = E[x][4 + i] + x1[i];
      E[x][i] = s0 * (qc * kd0[i]) + la0[i];
      E[x][4 + i] = s1 * (qc * kd1[i]) + la1[i];
      m = fmaxf(m, fmaxf(E[x][i], E[x][4 + i]));
    }
  }
  m = xor32_reduce(m, true);
  maxb[w * 64 + lane] = m;
  lds_barrier();
  // the exact maximum of each head over the unit's keys (both head blocks:
  // every wave's output columns cover all 64 heads)
  float Mx[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    float mn = kNegInf;
#pragma unroll
    for (int y = 0; y < 4; ++y) mn = fmaxf(mn, maxb[((y & 1) + 2 * x + 4 * (y >> 1)) * 64 + (lane & 31)]);
    Mx[x] = mn;
  }
  // ---- P = 2^(E - M) (f16) and the row sums ----
  float lt = 0.f;
  for (int x = 0; x < ntiles; ++x) {
    const uint8_t* set = smem + L::kSc + x * LdsPF::kScBytes;
    const float* invp = reinterpret_cast<const float*>(set + LdsPF::kScInv) + 32 * kb + 16 * dh + 4 * g;
    const v4f iv0 = *(const v4f*)invp, iv1 = *(const v4f*)(invp + 8);
    const int pq = 2 * (2 * kb + dh) + g;
    uint8_t* prow = smem + L::kP + x * 8192 + hq * 128 + 16 * (pq ^ (hq & 7));
    lt += pf_probs(E[x], hb ? Mx[1] : Mx[0], iv0, iv1, prow);
  }
  lbuf[w * 64 + lane] = xor32_reduce(lt, false);
  lds_barrier();
  // ---- O^T = V'^T P^T ----
  v16f acc[2][2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int x = 0; x < 2; ++x) acc[db][x] = v16f{};
  for (int x = 0; x < ntiles; ++x) {
    const uint8_t* set = smem + L::kSc + x * LdsPF::kScBytes;
    pf_pv<PER_TILE>(smem + L::kTiles + x * kTileBytes, reinterpret_cast<const _Float16*>(set + LdsPF::kScVs),
                    smem + L::kP + x * 8192, w, lane, acc);
  }

  // ---- epilogue: the final result (one split) or the unit's partial ----
  const size_t unit = (size_t)t * S + sp;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int h = 32 * x + (lane & 31);
    float Ls = 0.f;
#pragma unroll
    for (int y = 0; y < 4; ++y) Ls += lbuf[((y & 1) + 2 * x + 4 * (y >> 1)) * 64 + (lane & 31)];
    const float M = Mx[x];
    float sc = 0.f;
    uint16_t* orow;
    if (S == 1) {
      const float sg = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
      const float Mf = fmaxf(M, sg);
      float lse_v = kNegInf;
      if (c.k.valid && Mf != kNegInf) {
        const float af = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - Mf);
        const float Lf = af * Ls + ((sg == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sg - Mf));
        sc = af * __builtin_amdgcn_rcpf(Lf);
        lse_v = (Mf + __log2f(Lf)) * kLn2;
      }
      if (over) { sc = __builtin_nanf(""); lse_v = sc; }
      if (a.lse && w == 0 && g == 0) a.lse[(size_t)t * a.n1 + h] = lse_v;
      orow = a.out + ((size_t)t * a.n1 + h) * kD;
    } else {
      // partial: O / own row sum in bf16, (max, sum) in log2 units; a padded
      // query row is marked by a negative sum
      sc = (Ls > 0.f) ? __builtin_amdgcn_rcpf(Ls) : 0.f;
      if (over) sc = __builtin_nanf("");
      if (w == 0 && g == 0) {
        float* ml = a.ws_ml + (unit * kN1 + h) * 2;
        ml[0] = c.k.valid ? M : kNegInf;
        ml[1] = c.k.valid ? Ls : -1.f;
      }
      orow = a.ws_o + (unit * kN1 + h) * kD;
    }
    // lanes l and l + 32 trade halves so each stores 16 contiguous bytes
    // (columns 64 w + 32 db + 16 k2 + 8 g + [0, 8))
    orow += 64 * w + 8 * g;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const v16f& o = acc[db][x];
        const int q0 = 2 * k2, q1 = 2 * k2 + 1;
        const uint2 A = pack_bf16x4(sc * o[4 * q0], sc * o[4 * q0 + 1], sc * o[4 * q0 + 2], sc * o[4 * q0 + 3]);
        const uint2 B = pack_bf16x4(sc * o[4 * q1], sc * o[4 * q1 + 1], sc * o[4 * q1 + 2], sc * o[4 * q1 + 3]);
        const auto sx = __builtin_amdgcn_permlane32_swap(A.x, B.x, false, false);
        const auto sy = __builtin_amdgcn_permlane32_swap(A.y, B.y, false, false);
        *(uint4*)(orow + 32 * db + 16 * k2) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
      }
  }
  if (S == 1) return;

  // ---- merge: arrive, wait for the token's last arrival, claim head groups ----
  const int my_xcc = sk_xcc_id();
  if (threadIdx.x == 0) xcc[unit] = my_xcc;
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this thread's partial stores are in L2
  __syncthreads();
  int* sy = sync + 4 * t;
  if (threadIdx.x == 0) {
    int go = 1;
    // the generation cannot move before this unit arrives
    const int gen0 = ws_poll(sy + 1);
    if (ws_atomic_add(sy, 1) == S - 1) {   // last arrival: a new generation, claims from 0
      ws_atomic_xchg(sy, 0);
      ws_atomic_xchg(sy + 2, 0);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      ws_atomic_add(sy + 1, 1);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    } else {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (ws_poll(sy + 1) == gen0) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)kSkSpinTicks) { go = 0; break; }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    misc[0] = go;
  }
  __syncthreads();
  if (!misc[0]) return;   // uniform: the others merge every group
  asm volatile("buffer_inv sc0" ::: "memory");   // (the other units' partial lines are first read here: L1 holds none)
  for (;;) {
    __syncthreads();   // misc[1] is read by every thread before it is rewritten
    if (threadIdx.x == 0) misc[1] = ws_atomic_add(sy + 2, 1);
    __syncthreads();
    const int grp = misc[1];
    if (grp >= kN1 / kSkHeadGroup) break;
    sk_merge(a, t, S, grp, my_xcc, xcc);
  }
}

template <int PER_TILE>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(kPfWaves / 4, kPfWaves / 4)))
sk_kernel(const KArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LdsSK::kBytes];
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  sk_body<PER_TILE>((KArgPtr)__builtin_amdgcn_kernarg_segment_ptr(), smem, w);
}

// ---------------------------------------------------------------------------
// bf16-q kernel: bf16 q against bf16 KV rows (SparseCompressedFlashAttention,
// 函数原型 / 参数说明: q, ori_kv, cmp_kv bfloat16, D = 512) or against packed
// 640-byte rows (KvQuantSparseAttnSharedkv, 约束说明: bf16 rope 64, e4m3 nope
// 448, seven e8m0 scales, pad; 参数说明: q bfloat16, tile_size 64).  One work
// unit = (query token, key split), all 64 heads; the split partials go to the
// split-KV combine, as with the key-split fp8 kernel.
// ---------------------------------------------------------------------------
//
// 4 waves.  Per 32-key tile: every thread loads a block of 8 keys x 8 columns
// (bf16 rows: 16 bytes per key; packed rows: the rope bytes, or 8 nope codes
// and their tile's scale byte), turns it into bf16 (nope: e4m3 x 2^(E - 127),
// exact) and writes it twice to LDS: as K [key][d] rows and, transposed in
// registers, as V^T [d][key] rows.  The next tile's loads are in flight while
// the current tile is computed.
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16: wave w scores the 32 keys against
//                 heads [32 (w & 1), +32) over D half w >> 1 (q in VGPRs); the
//                 half-1 partial is added through LDS
//   softmax       online, in log2 units, per head (the D-half-0 waves)
//   O^T += V^T P^T  same MFMA: wave w owns output columns [128 w, +128) of all
//                 64 heads; P in bf16
// LDS rows are XOR-swizzled by 16-byte chunk so that 16 lanes reading the
// same chunk of 16 rows hit different banks.

constexpr int kBkKeys = 32;          // keys per tile
constexpr int kBkMaxKeys = 1024;     // keys per unit, resolved at once
constexpr float kBkRefSlack = 16.f;  // log2 units a tile maximum may pass the reference by
constexpr int kBkThreads = 256;

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));

struct LdsBK {
  static constexpr int kK = 0;                               // bf16 [32 keys][512]: 1 KiB rows, chunk ^ bk_swz(key)
  static constexpr int kP = kK + kBkKeys * 2 * kD;           // bf16 [64 heads][32 keys]: chunk ^ ((h >> 2) & 3)
  static constexpr int kX = kP + kN1 * kBkKeys * 2;          // f32 [2 head blocks][64 lanes][16]: D-half-1 partials
  static constexpr int kAddr = kX + 2 * 64 * 16 * 4;         // u64 [kBkMaxKeys]: the unit's row addresses
  static constexpr int kList = kAddr + 8 * kBkMaxKeys;       // int [kListMax]: compacted cmp indices
  static constexpr int kAlpha = kList + 4 * kListMax;        // f32 [64]: this tile's rescale per head
  static constexpr int kM = kAlpha + 4 * kN1;                // f32 [64]: final maximum per head
  static constexpr int kL = kM + 4 * kN1;                    // f32 [64]: final row sum per head
  static constexpr int kMisc = kL + 4 * kN1;                 // int [64]: compaction
  static constexpr int kFlag = kMisc + 4 * 64;               // int [2]: a head block's reference moved this tile
  static constexpr int kRaw = (kFlag + 8 + 1023) / 1024 * 1024;   // packed rows: the tile's raw 640-byte rows
  static constexpr int kBytes = kRaw + kBkKeys * 640;
};
static_assert(LdsBK::kBytes <= 160 * 1024, "LDS");

__device__ __forceinline__ v16f mma_bf16(bf8_t a, bf8_t b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte chunk c of key row `key` sits at chunk c ^ bk_swz(key).  Reads of
// one chunk from 16 consecutive rows (S^T operands) and transpose reads of 4
// consecutive rows x 2 chunks (P V operands) both reach 16 distinct chunks,
// i.e. all 64 banks.
__device__ __forceinline__ int bk_swz(int key) { return ((key & 3) << 2) | ((key >> 2) & 3); }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// V^T operand of O^T += V^T P^T (32 d x 16 keys, 8 keys per lane) straight
// from the row-major K tile with two transpose reads: within each group of 16
// lanes, lanes 4r..4r+3 address the 8-byte pieces of key row r (columns
// dbase + 4 (j & 3) .. +3), and lane j receives column dbase + j of the four
// rows.  Lane l: d = dblk + (l % 32), keys 16 ks + 8 (l / 32) .. +7.
__device__ __forceinline__ bf8_t bk_vop(const uint8_t* kt, int dblk, int ks, int lane) {
  const int gq = lane >> 4, j = lane & 15;
  const int dbase = dblk + 16 * (gq & 1), e = dbase + 4 * (j & 3);
  v4i out;
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int row = 16 * ks + 8 * (gq >> 1) + 4 * rd + (j >> 2);
    const uint8_t* p = kt + row * 2 * kD + 16 * ((e >> 3) ^ bk_swz(row)) + 8 * ((e >> 2) & 1);
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
    const v2i y = __builtin_bit_cast(v2i, x);
    out[2 * rd] = y[0];
    out[2 * rd + 1] = y[1];
  }
  return __builtin_bit_cast(bf8_t, out);
}

// bf16 rows: the tile's bytes of one thread, keys 8 kq + j (j < 8) of the
// tile, columns 8 dq .. 8 dq + 7 (one 16-byte load per key).
struct BkRaw {
  v4i x[8];
};

__device__ __forceinline__ BkRaw bk_load(const uint64_t* kaddr, int tile, int tid) {
  const int kq = tid >> 6, dq = tid & 63;
  BkRaw r;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint8_t* row = gptr(reinterpret_cast<const uint8_t*>(kaddr[kBkKeys * tile + 8 * kq + j]));
    r.x[j] = *(const v4i*)(row + 16 * dq);
  }
  return r;
}

// The block into the K rows (P V reads them transposed, bk_vop).
__device__ __forceinline__ void bk_store(const BkRaw& r, uint8_t* smem, int tid) {
  const int kq = tid >> 6, dq = tid & 63;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int key = 8 * kq + j;
    *(v4i*)(smem + LdsBK::kK + key * 2 * kD + 16 * (dq ^ bk_swz(key))) = r.x[j];
  }
}

// Packed rows: the tile's 32 raw 640-byte rows into LDS by LDS-DMA, 16 bytes
// per lane (20 instructions of 1 KiB, 5 per wave: lane-chunk q = 64 i + lane
// of the tile is chunk q % 40 of key q / 40, written at raw + 16 q).  Narrow
// loads of the 8-byte code blocks and the scale words took 3 instructions per
// key and wave, and the CU's address unit became the bound.
__device__ __forceinline__ void bk_dma_packed(const uint64_t* kaddr, int tile, uint8_t* raw, int w) {
  const int lane = opaque((int)threadIdx.x & 63);
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int q = 64 * (5 * w + i) + lane;
    const int key = q / 40, c = q - 40 * key;
    const uint64_t src = kaddr[kBkKeys * tile + key] + 16u * (uint32_t)c;
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(raw + 1024 * (5 * w + i)));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(src)
                 : "memory", "m0");
  }
}

// bf16 of 8 e4m3 codes times 2^(E - 127) (E = 255: NaN), exact.
__device__ __forceinline__ v4i bk_nope8(v2i x, int scw, int tile) {
  const uint32_t e = ((uint32_t)scw >> (8 * (tile & 3))) & 0xffu;
  const float sc = (e == 255u) ? __builtin_nanf("") : ((e == 0u) ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23));
  const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(x[0], false);
  const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(x[0], true);
  const auto f45 = __builtin_amdgcn_cvt_pk_f32_fp8(x[1], false);
  const auto f67 = __builtin_amdgcn_cvt_pk_f32_fp8(x[1], true);
  return v4i{(int)pack_bf16x2(f01[0] * sc, f01[1] * sc), (int)pack_bf16x2(f23[0] * sc, f23[1] * sc),
             (int)pack_bf16x2(f45[0] * sc, f45[1] * sc), (int)pack_bf16x2(f67[0] * sc, f67[1] * sc)};
}

// The raw packed rows as bf16 into the K rows: thread (kq, dq) converts
// columns 8 dq .. +7 of keys 8 kq + j (rope: the row's bf16 values; nope:
// 8 codes and their tile's scale).
__device__ __forceinline__ void bk_convert_packed(const uint8_t* raw, uint8_t* smem, int tid) {
  const int kq = tid >> 6, dq = tid & 63;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int key = 8 * kq + j;
    const uint8_t* row = raw + key * 640;
    v4i v;
    if (dq < 8) {
      v = *(const v4i*)(row + 16 * dq);
    } else {
      const int nb = 8 * dq - 64;                       // nope column of the block's first value
      const v2i c = *(const v2i*)(row + 128 + nb);
      const int scw = *(const int*)(row + 576 + 4 * ((nb >> 6) >> 2));
      v = bk_nope8(c, scw, nb >> 6);
    }
    *(v4i*)(smem + LdsBK::kK + key * 2 * kD + 16 * (dq ^ bk_swz(key))) = v;
  }
}

template <int FMT>
__device__ __forceinline__ void bk_body(KArgPtr ap, uint8_t* smem, int w) {
  using L = LdsBK;
  constexpr int ROW = (FMT == 1) ? 2 * kD : 640;   // bytes per cache row
  const int lane = opaque((int)threadIdx.x & 63), g = lane >> 5;
  const int hb = w & 1, dh = w >> 1;
  const HdrRegs hr = load_hdr_regs(ap);
  const KHdr a0 = hdr_view(hr);
  const int G = a0.grid, bid = blockIdx.x;
  const int lw = (G % 8 == 0) ? ((bid & 7) * (G >> 3) + (bid >> 3)) : bid;  // one XCD per contiguous range
  int u_begin = lw, u_end = lw + 1;
  if (a0.n_units != G) {
    u_begin = ap->starts[lw];
    u_end = ap->starts[lw + 1];
  }
  int* list = reinterpret_cast<int*>(smem + L::kList);
  int* misc = reinterpret_cast<int*>(smem + L::kMisc);
  uint64_t* kaddr = reinterpret_cast<uint64_t*>(smem + L::kAddr);
  float* alpha_s = reinterpret_cast<float*>(smem + L::kAlpha);
  float* m_s = reinterpret_cast<float*>(smem + L::kM);
  float* l_s = reinterpret_cast<float*>(smem + L::kL);
  int* flag_s = reinterpret_cast<int*>(smem + L::kFlag);
  float* xch = reinterpret_cast<float*>(smem + L::kX) + (hb * 64 + lane) * 16;

  for (int u = u_begin; u < u_end; ++u) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the previous unit's stores settle here
    const KHdr a = hdr_view(hr);
    const int tid = opaque((int)threadIdx.x);
    const int S = a.splits;
    const int t = (S == 1) ? u : u / S, sp = u - t * S;
    const int hq = 32 * hb + (lane & 31);   // the lane's head in S^T and the softmax
    // prologue loads: lengths, index slots, the q fragments (B operands of
    // S^T: head hq, columns 256 dh + 16 ks + 8 g .. +7)
    const TokLens tl = token_lens(a, t);
    const IdxPre<kBkThreads> ip = load_indices<kBkThreads>(a, t, 0);
    bf8_t qf[16];
    {
      const uint8_t* qrow = a.q + (((size_t)t * a.n1 + hq) * kD + 256 * dh + 8 * g) * 2;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[ks] = __builtin_bit_cast(bf8_t, *(const v4i*)(qrow + 32 * ks));
    }
    const Tok k = token_ctx(a, t, tl);
    if (!k.valid) {   // padded query row: O = 0, lse = -inf
      if (S == 1) {
        for (int x = tid; x < kN1 * kD / 8; x += kBkThreads)
          *(v4i*)(a.out + ((size_t)t * a.n1 + x / (kD / 8)) * kD + 8 * (x % (kD / 8))) = v4i{0, 0, 0, 0};
        if (a.lse && tid < kN1) a.lse[(size_t)t * a.n1 + tid] = kNegInf;
      } else if (tid < kN1) {
        a.ws_ml[((size_t)u * kN1 + tid) * 2] = kNegInf;
        a.ws_ml[((size_t)u * kN1 + tid) * 2 + 1] = -1.0f;   // marks a padded row for the combine
      }
      continue;
    }
    const int n_o = (a.ori_topk > 0) ? compact_ori<kBkThreads>(a, k, t, list, misc) : k.hi - k.lo;
    int n_c = 0;
    if (a.topk > 0) n_c = compact_indices<kBkThreads>(a, k, t, list + (a.ori_topk > 0 ? n_o : 0), misc, 0, ip);
    else if (a.has_cmp) n_c = k.vis;
    const int64_t n = (int64_t)n_o + n_c;
    const int kb = (int)(n * sp / S), ke = (int)(n * (sp + 1) / S);
    const bool over = ke - kb > kBkMaxKeys;    // the plan's key bound was exceeded: poison, never drop keys
    const int nk = min(ke - kb, kBkMaxKeys);
    const int tiles = (nk + kBkKeys - 1) / kBkKeys;

    // ---- the unit's row addresses (the split kernels' resolution functions);
    // slots past the unit's end read the zero row ----
    {
      const Sides sd = cache_sides(a);
      for (int i = tid; i < tiles * kBkKeys; i += kBkThreads) {
        const bool ok = i < nk;
        bool is_cmp;
        const int j = key_pos(a, k, n_o, kb + (ok ? i : 0), list, 0, is_cmp);
        BlockPos bp{0, 0};
        if (a.layout_kv == 2) bp = block_pos(sd, is_cmp, j);
        const int blk = (a.layout_kv == 2) ? block_of(sd, k, is_cmp, bp.q) : 0;
        const int64_t row = row_of(a, sd, k, is_cmp, j, blk, bp.r);
        const uint8_t* src = (is_cmp ? sd.c.kv : sd.o.kv) + row * ROW;
        kaddr[i] = (uint64_t)(uintptr_t)(ok ? src : g_zero_row);
      }
    }
    lds_barrier();

    v16f acc[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int x = 0; x < 2; ++x) acc[db][x] = v16f{};
    float mrun = kNegInf, lrun = 0.f;   // the D-half-0 waves: head hq
    uint8_t* rawbuf = smem + L::kRaw;
    BkRaw raw;
    if (FMT == 2) {
      if (tiles > 0) {
        bk_dma_packed(kaddr, 0, rawbuf, w);
        gather_barrier(false);
      }
    } else if (tiles > 0) {
      raw = bk_load(kaddr, 0, tid);
    }
    for (int it = 0; it < tiles; ++it) {
      if (FMT == 2) {
        bk_convert_packed(rawbuf, smem, tid);
        lds_barrier();   // the K rows are complete and the raw rows free
        if (it + 1 < tiles) bk_dma_packed(kaddr, it + 1, rawbuf, w);   // in flight during this tile
      } else {
        bk_store(raw, smem, tid);
        if (it + 1 < tiles) raw = bk_load(kaddr, it + 1, tid);   // in flight during this tile
        lds_barrier();
      }
      // ---- S^T: keys x heads [32 hb, +32), D half dh ----
      v16f Sx = v16f{};
      {
        const int key = lane & 31;
        const uint8_t* krow = smem + L::kK + key * 2 * kD;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          const int c = 32 * dh + 2 * ks + g;
          const bf8_t av = __builtin_bit_cast(bf8_t, *(const v4i*)(krow + 16 * (c ^ bk_swz(key))));
          Sx = mma_bf16(av, qf[ks], Sx);
        }
      }
      if (dh) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) *(v4f*)(xch + 4 * q4) = v4f{Sx[4 * q4], Sx[4 * q4 + 1], Sx[4 * q4 + 2], Sx[4 * q4 + 3]};
      }
      lds_barrier();
      if (dh == 0) {
        const int nv = min(kBkKeys, nk - kBkKeys * it);
        float E[16];
        float mx = kNegInf;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const v4f o = *(const v4f*)(xch + 4 * q4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = 8 * q4 + 4 * g + r;
            E[4 * q4 + r] = (key < nv) ? (Sx[4 * q4 + r] + o[r]) * a.scale_log2 : kNegInf;
            mx = fmaxf(mx, E[4 * q4 + r]);
          }
        }
        mx = xor32_reduce(mx, true);
        // a head's reference moves only when the tile's maximum passes it
        // by more than kBkRefSlack (P <= 2^kBkRefSlack is exact enough in
        // bf16 and the sums have range to spare), so the accumulators are
        // rescaled only on such tiles; the first finite maximum sets it
        const bool move = mx > mrun + kBkRefSlack;
        const float mnew = move ? mx : mrun;
        const float al = (move && mrun != kNegInf) ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.f;
        const float mz = (mnew == kNegInf) ? 0.f : mnew;
        float ps = 0.f;
        uint8_t* prow = smem + L::kP + hq * 64;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float p[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = __builtin_amdgcn_exp2f(E[4 * q4 + r] - mz);
            ps += p[r];
          }
          *(uint2*)(prow + 16 * (q4 ^ ((hq >> 2) & 3)) + 8 * g) = pack_bf16x4(p[0], p[1], p[2], p[3]);
        }
        ps = xor32_reduce(ps, false);
        lrun = al * lrun + ps;
        mrun = mnew;
        if (g == 0) alpha_s[hq] = al;
        const bool rescale = __ballot(al != 1.f) != 0;
        if (lane == 0) flag_s[hb] = rescale ? 1 : 0;
      }
      lds_barrier();
      // ---- O^T += V^T P^T: columns [128 w, +128), all 64 heads ----
      {
        if (__builtin_amdgcn_readfirstlane(flag_s[0] | flag_s[1])) {
          float al[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) al[x] = alpha_s[32 * x + (lane & 31)];
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int x = 0; x < 2; ++x) acc[db][x] *= al[x];
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int c = 2 * ks + g;
          bf8_t pb[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int h = 32 * x + (lane & 31);
            pb[x] = __builtin_bit_cast(bf8_t, *(const v4i*)(smem + L::kP + h * 64 + 16 * (c ^ ((h >> 2) & 3))));
          }
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf8_t va = bk_vop(smem + L::kK, 128 * w + 32 * db, ks, lane);
#pragma unroll
            for (int x = 0; x < 2; ++x) acc[db][x] = mma_bf16(va, pb[x], acc[db][x]);
          }
        }
      }
      // K and P are read before the next tile overwrites them (packed rows:
      // and the next tile's raw rows have landed)
      if (FMT == 2) gather_barrier(false);
      else lds_barrier();
    }

    // ---- epilogue: the final result (one split) or the unit's partial ----
    if (dh == 0 && g == 0) {
      m_s[hq] = mrun;
      l_s[hq] = lrun;
    }
    lds_barrier();
    if constexpr (FMT == 1) {
      float scx[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int h = 32 * x + (lane & 31);
        const float M = m_s[h], Ls = l_s[h];
        float sc;
        if (S == 1) {
          const float sg = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
          const float Mf = fmaxf(M, sg);
          float lse_v = kNegInf;
          sc = 0.f;
          if (Mf != kNegInf) {
            const float af = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - Mf);
            const float Lf = af * Ls + ((sg == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sg - Mf));
            sc = af / Lf;
            lse_v = (Mf + __log2f(Lf)) * kLn2;
          }
          if (over) { sc = __builtin_nanf(""); lse_v = sc; }
          if (a.lse && w == 0 && g == 0) a.lse[(size_t)t * a.n1 + h] = lse_v;
        } else {
          sc = (Ls > 0.f) ? 1.0f / Ls : 0.f;
          if (over) sc = __builtin_nanf("");
          if (w == 0 && g == 0) {
            a.ws_ml[((size_t)u * kN1 + h) * 2] = M;
            a.ws_ml[((size_t)u * kN1 + h) * 2 + 1] = Ls;
          }
        }
        scx[x] = sc;
      }
      // The output rows go through LDS, 32 heads at a time over the K tile and
      // the P area (both free now), so that each store instruction writes one
      // whole 1 KiB head row.  Lane (h, g) holds columns 8 q + 4 g + [0, 4) of
      // each 32-column block.
      constexpr int kRow = 2 * kD + 16;   // padded: the 8-byte writes of 32 rows reach distinct banks
      static_assert(32 * kRow <= LdsBK::kX, "staging");
      uint16_t* obase = (S == 1) ? a.out + (size_t)t * a.n1 * kD : a.ws_o + (size_t)u * kN1 * kD;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        uint8_t* srow = smem + (lane & 31) * kRow + 2 * (128 * w + 4 * g);
        const float sc = scx[x];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const v16f& o = acc[db][x];
            *(uint2*)(srow + 2 * (32 * db + 8 * q4)) =
                pack_bf16x4(sc * o[4 * q4], sc * o[4 * q4 + 1], sc * o[4 * q4 + 2], sc * o[4 * q4 + 3]);
          }
        lds_barrier();
        for (int row = w; row < 32; row += kBkThreads / 64)
          *(v4i*)(obase + (size_t)(32 * x + row) * kD + 8 * lane) = *(const v4i*)(smem + row * kRow + 16 * lane);
        if (x == 0 || u + 1 < u_end) lds_barrier();   // the staged rows are read before they are overwritten
      }
    } else {
      // (the packed-row instantiation keeps direct 16-byte stores: with the
      // staged form, the compiler parked the per-lane address of the m_s /
      // l_s reads in an AGPR through a copy inside a divergent block, so
      // that every lane but 0 and 32 read head 0's values)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int h = 32 * x + (lane & 31);
        const float M = m_s[h], Ls = l_s[h];
        float sc;
        uint16_t* orow;
        if (S == 1) {
          const float sg = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
          const float Mf = fmaxf(M, sg);
          float lse_v = kNegInf;
          sc = 0.f;
          if (Mf != kNegInf) {
            const float af = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - Mf);
            const float Lf = af * Ls + ((sg == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sg - Mf));
            sc = af / Lf;
            lse_v = (Mf + __log2f(Lf)) * kLn2;
          }
          if (over) { sc = __builtin_nanf(""); lse_v = sc; }
          if (a.lse && w == 0 && g == 0) a.lse[(size_t)t * a.n1 + h] = lse_v;
          orow = a.out + ((size_t)t * a.n1 + h) * kD;
        } else {
          sc = (Ls > 0.f) ? 1.0f / Ls : 0.f;
          if (over) sc = __builtin_nanf("");
          if (w == 0 && g == 0) {
            a.ws_ml[((size_t)u * kN1 + h) * 2] = M;
            a.ws_ml[((size_t)u * kN1 + h) * 2 + 1] = Ls;
          }
          orow = a.ws_o + ((size_t)u * kN1 + h) * kD;
        }
        // lane (h, g) holds columns 8 q + 4 g + [0, 4) of each 32-column block;
        // v_permlane32_swap trades the upper lanes' even-q half with the lower
        // lanes' odd-q half of each q pair, so that each lane stores 16
        // contiguous bytes (columns 16 k + 8 g + [0, 8)): half the store
        // instructions of 8-byte pieces
        uint16_t* ocol = orow + 128 * w + 8 * g;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const v16f& o = acc[db][x];
            const int q0 = 2 * k2, q1 = 2 * k2 + 1;
            const uint2 A = pack_bf16x4(sc * o[4 * q0], sc * o[4 * q0 + 1], sc * o[4 * q0 + 2], sc * o[4 * q0 + 3]);
            const uint2 B = pack_bf16x4(sc * o[4 * q1], sc * o[4 * q1 + 1], sc * o[4 * q1 + 2], sc * o[4 * q1 + 3]);
            const auto sx = __builtin_amdgcn_permlane32_swap(A.x, B.x, false, false);
            const auto sy = __builtin_amdgcn_permlane32_swap(A.y, B.y, false, false);
            *(uint4*)(ocol + 32 * db + 16 * k2) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
          }
      }
    }
  }
}

template <int FMT>
__global__ void __launch_bounds__(kBkThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) bk_kernel(const KArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LdsBK::kBytes];
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  bk_body<FMT>((KArgPtr)__builtin_amdgcn_kernarg_segment_ptr(), smem, w);
}

}  // namespace

// ---------------------------------------------------------------------------
// debug export of the whole-token kernel's resolved key rows: the token entry
// (pf_enter: lengths, index compaction), the per-tile key resolution
// (pf_resolve) and the row address (pf_src) that feeds the tile's LDS-DMA,
// each the same function pf_kernel runs; the row is recovered from the address.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kPfThreads) pf_debug_resolve_kernel(const KArgs a, int32_t* keys, int32_t* counts,
                                                                      int32_t max_keys) {
  __shared__ int list[kListMax];
  __shared__ int misc[64];
  const int t = blockIdx.x;
  PfCursor c;
  c.u = t;
  c.nl = token_lens(a, t);
  c.nip = pf_idx_raw(a, t);
  pf_enter(a, c, t + 1, list, misc);
  if (threadIdx.x == 0) { counts[2 * t] = c.n_o; counts[2 * t + 1] = c.n_c; }
  const int n = min(c.n_o + c.n_c, max_keys);
  if (threadIdx.x >= 64) return;
  for (c.tile = 0; c.tile * kTileKeys < n; ++c.tile) {
    const PfKey k = pf_resolve(a, c, list, true);
    const PfSrc src = pf_src<0>(a, k);
    const int key = kTileKeys * c.tile + (int)threadIdx.x;
    if (key < n && src.ok) {
      const uint8_t* base = k.cmp ? a.cmp_kv : a.ori_kv;
      keys[(size_t)t * max_keys + key] = (int32_t)(((const uint8_t*)(uintptr_t)src.addr - base) / kD);
    }
  }
}

// ---------------------------------------------------------------------------
// static scratch for callers that cannot allocate (csmla_forward_noalloc):
// the split partials and their (max, sum) live here instead of in a
// caller-provided workspace.  Each GPU holds its own copy of the array at its
// own address; host code uses only the address hipGetSymbolAddress returns
// for the current device (the array's name is a host-side stand-in).
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

__global__ void zero_words_kernel(int32_t* p, int n) {
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x)) p[i] = 0;
}

int noalloc_scratch(void** ptr, void* stream) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    // the workspace's sync words and exchange slots start at zero (a fill
    // kernel on the caller's stream, ahead of the first forward that uses them)
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream, (int32_t*)p,
                       (int)(kWsFixedBytes / 4));
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

// Blocks of the split-KV combine (XCD-local token ranges when the grid is a
// multiple of 8).
static int combine_blocks(const KArgs& a) {
  int blocks = a.t1 * 8;
  if (a.grid % 8 == 0) {
    int most = 0;
    for (int x = 0; x < 8; ++x) {
      int t0, t1;
      xcd_tokens(a, x, t0, t1);
      most = std::max(most, t1 - t0);
    }
    blocks = 8 * 8 * most;
  }
  return blocks;
}

int launch_forward(const KArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (a.kv_fmt != 0) {
    if (a.kv_fmt == 1)
      hipLaunchKernelGGL(bk_kernel<1>, dim3(a.grid), dim3(kBkThreads), 0, st, a);
    else
      hipLaunchKernelGGL(bk_kernel<2>, dim3(a.grid), dim3(kBkThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return (int)e;
    hipLaunchKernelGGL(combine_kernel, dim3(combine_blocks(a)), dim3(256), 0, st, a);
    return (int)hipGetLastError();
  }
  if (a.sk) {
    if (a.scale_mode == 1)
      hipLaunchKernelGGL(sk_kernel<1>, dim3(a.grid), dim3(kPfThreads), 0, st, a);
    else
      hipLaunchKernelGGL(sk_kernel<0>, dim3(a.grid), dim3(kPfThreads), 0, st, a);
    return (int)hipGetLastError();
  }
  if (a.hg == kN1) {
    if (a.scale_mode == 1)
      hipLaunchKernelGGL(pf_kernel<1>, dim3(a.grid), dim3(kPfThreads), 0, st, a);
    else
      hipLaunchKernelGGL(pf_kernel<0>, dim3(a.grid), dim3(kPfThreads), 0, st, a);
    return (int)hipGetLastError();
  }
  if (a.hg > 0) {
    if (a.dk_parts > 1 || a.n_units <= a.grid)   // one unit per work-group
      hipLaunchKernelGGL(dk_kernel<1>, dim3(a.grid), dim3(kDkThreads), 0, st, a);
    else
      hipLaunchKernelGGL(dk_kernel<0>, dim3(a.grid), dim3(kDkThreads), 0, st, a);
    return (int)hipGetLastError();
  }
  if (a.scale_mode == 1)
    hipLaunchKernelGGL(attn_kernel<1>, dim3(a.grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(attn_kernel<0>, dim3(a.grid), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  if (a.splits > 1) {
    const int blocks = combine_blocks(a);
    if (blocks > 0) hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  return (int)e;
}

int launch_debug_resolve(const KArgs& a, int32_t* keys, int32_t* counts, int32_t max_keys, int whole_token,
                         void* stream) {
  if (whole_token)
    hipLaunchKernelGGL(pf_debug_resolve_kernel, dim3(a.t1), dim3(kPfThreads), 0, (hipStream_t)stream, a, keys, counts,
                       max_keys);
  else
    hipLaunchKernelGGL(debug_resolve_kernel, dim3(a.t1), dim3(kThreads), 0, (hipStream_t)stream, a, keys, counts,
                       max_keys);
  return (int)hipGetLastError();
}

}  // namespace csmla

