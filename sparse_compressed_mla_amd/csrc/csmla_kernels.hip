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

struct Meta {                 // per-key data of one tile, in LDS
  uint64_t addr[kTileKeys];   // byte address of the fp8 row; 0 = no row (tail)
  float lam[kTileKeys];       // log2 of the largest V descale of the row
  float inv[kTileKeys];       // 2^-lam
  float ks[8][kTileKeys];     // descales: per-token in ks[0]; per-tile in ks[0..7]
};
constexpr int kMetaBytes = 3072;
static_assert(sizeof(Meta) <= kMetaBytes, "meta");

constexpr int kOffTiles = 0;                               // 2 tile buffers
constexpr int kOffXchg = 2 * kTileBytes;                   // partial scores, 4 waves x 8 KiB
constexpr int kOffMeta = kOffXchg + 4 * 8192;              // 3 meta stages
constexpr int kOffList = kOffMeta + 3 * kMetaBytes;        // compacted cmp indices
constexpr int kOffMisc = kOffList + kListMax * 4;
constexpr int kLdsBytes = kOffMisc + 256;

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

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(bf16_rne(a) | (bf16_rne(b) << 16), bf16_rne(c) | (bf16_rne(d) << 16));
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
};

__device__ Tok token_ctx(const KArgs& a, int t) {
  Tok k;
  int b, q0, span;
  if (a.layout_q == 1) {  // TND: largest b with cu_q[b] <= t
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_q[mid] <= t) lo = mid; else hi = mid;
    }
    b = lo; q0 = a.cu_q[b]; span = a.cu_q[b + 1] - q0;
  } else {
    b = t / a.q_s; q0 = b * a.q_s; span = a.q_s;
  }
  const int i = t - q0;
  int s1 = span;
  if (a.su_q) s1 = min(span, a.su_q[b]);
  int s2;
  if (a.su_ori) s2 = a.su_ori[b];
  else if (a.cu_ori) s2 = a.cu_ori[b + 1] - a.cu_ori[b];
  else s2 = a.ori_s;
  k.kv0 = (a.layout_kv == 1) ? a.cu_ori[b] : 0;
  int c = 0;
  k.cmp0 = 0;
  if (a.has_cmp) {
    if (a.su_cmp) c = a.su_cmp[b];
    else if (a.cu_cmp) c = a.cu_cmp[b + 1] - a.cu_cmp[b];
    else if (a.layout_kv == 0) c = a.cmp_s;
    else c = s2 / a.cmp_ratio;
    if (a.layout_kv == 1) k.cmp0 = a.cu_cmp[b];
  }
  const int64_t res = a.res ? a.res[b] : 0;
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
  if (a.topk_len) ke = max(0, min(ke, a.topk_len[t]));
  k.k_eff = ke;
  if (!k.valid) { k.lo = k.hi = 0; k.vis = 0; k.k_eff = 0; }
  return k;
}

// Compact the valid index slots of token t in slot order; entries whose
// compacted position lies in [w_lo, w_lo + kListMax) go to list[pos - w_lo].
// Returns the number of valid slots.  Whole-work-group call.
__device__ int compact_indices(const KArgs& a, const Tok& k, int t, int* list, int* wtot, int w_lo) {
  const int* row = a.idx + (size_t)t * a.topk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int base = 0;
  for (int s0 = 0; s0 < k.k_eff; s0 += kThreads) {
    const int s = s0 + threadIdx.x;
    const int v = (s < k.k_eff) ? row[s] : -1;
    const bool ok = (v >= 0) && (v < k.vis);
    const uint64_t bal = __ballot(ok);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[w] = __popcll(bal);
    __syncthreads();
    int off = 0;
    for (int j = 0; j < w; ++j) off += wtot[j];
    const int tot = wtot[0] + wtot[1] + wtot[2] + wtot[3];
    const int pos = base + off + pre;
    if (ok && pos >= w_lo && pos < w_lo + kListMax) list[pos - w_lo] = v;
    base += tot;
    __syncthreads();
  }
  return base;
}

// Resolving one tile of 64 keys takes three stages, spread over pipeline
// steps so that no wave waits on a dependent load: (1) the block-table
// lookup, (2) the row address and the descale loads, (3) the descales into
// meta.  One wave, one key per lane.
struct KeyLoc {
  int j;       // logical token position in its cache
  int cmp;     // 1: the key lives in cmp_kv
  int blk;     // PA block id (loaded in stage 1)
  int valid;   // key < end of the chunk
};

template <int PER_TILE>
struct KeyScale {
  float v[PER_TILE ? 8 : 1];
};

__device__ __forceinline__ KeyLoc resolve_issue(const KArgs& a, const Tok& k, int n_o, const int* list, int w_lo,
                                                int key0, int key_end) {
  const int key = key0 + (int)(threadIdx.x & 63);
  KeyLoc kl;
  kl.valid = key < key_end;
  kl.cmp = key >= n_o;
  kl.j = 0;
  kl.blk = 0;
  if (kl.valid) {
    kl.j = !kl.cmp ? k.lo + key : ((a.topk > 0) ? list[key - n_o - w_lo] : key - n_o);
    if (a.layout_kv == 2) {
      const int bs = kl.cmp ? a.cmp_bs : a.ori_bs;
      const int* tab = kl.cmp ? a.cmp_tab : a.ori_tab;
      const int cols = kl.cmp ? a.cmp_cols : a.ori_cols;
      kl.blk = tab[(size_t)k.b * cols + kl.j / bs];
    }
  }
  return kl;
}

__device__ __forceinline__ int64_t key_row(const KArgs& a, const Tok& k, const KeyLoc& kl) {
  if (a.layout_kv == 2) {
    const int bs = kl.cmp ? a.cmp_bs : a.ori_bs;
    return (int64_t)kl.blk * bs + (kl.j % bs);
  }
  if (a.layout_kv == 1) return (int64_t)(kl.cmp ? k.cmp0 : k.kv0) + kl.j;
  return (int64_t)k.b * (kl.cmp ? a.cmp_s : a.ori_s) + kl.j;
}

template <int PER_TILE>
__device__ __forceinline__ void resolve_rows(const KArgs& a, const Tok& k, const KeyLoc& kl, Meta* m,
                                             KeyScale<PER_TILE>& sc) {
  const int lane = threadIdx.x & 63;
  uint64_t addr = 0;
#pragma unroll
  for (int c = 0; c < (PER_TILE ? 8 : 1); ++c) sc.v[c] = 0.f;
  if (kl.valid) {
    const int64_t row = key_row(a, k, kl);
    addr = (uint64_t)((kl.cmp ? a.cmp_kv : a.ori_kv) + row * kD);
    const float* ds = kl.cmp ? a.cmp_ds : a.ori_ds;
    if (PER_TILE) {
      const v4f* p = (const v4f*)(ds + row * 8);
      const v4f x0 = p[0], x1 = p[1];
      sc.v[0] = x0[0]; sc.v[1] = x0[1]; sc.v[2] = x0[2]; sc.v[3] = x0[3];
      sc.v[4] = x1[0]; sc.v[5] = x1[1]; sc.v[6] = x1[2]; sc.v[7] = x1[3];
    } else {
      sc.v[0] = ds[row];
    }
  }
  m->addr[lane] = addr;
}

template <int PER_TILE>
__device__ __forceinline__ void resolve_scales(const KeyScale<PER_TILE>& sc, int valid, Meta* m) {
  const int lane = threadIdx.x & 63;
  float lam = kNegInf, inv = 0.f;
  if (valid) {
    float mx = sc.v[0];
#pragma unroll
    for (int c = 1; c < (PER_TILE ? 8 : 1); ++c) mx = fmaxf(mx, sc.v[c]);
#pragma unroll
    for (int c = 0; c < (PER_TILE ? 8 : 1); ++c)
      if (sc.v[c] != sc.v[c]) mx = sc.v[c];   // a NaN scale poisons the row
    mx = (mx == 0.f) ? kMinDescale : mx;
    lam = __log2f(mx);
    inv = 1.0f / mx;
    if (mx != mx) { lam = mx; inv = mx; }
  }
  m->lam[lane] = lam;
  m->inv[lane] = inv;
#pragma unroll
  for (int c = 0; c < (PER_TILE ? 8 : 1); ++c) m->ks[c][lane] = valid ? sc.v[c] : 0.f;
}

// Whole-tile resolve in one go (used by the pipeline prologue).
template <int PER_TILE>
__device__ __forceinline__ void resolve_tile(const KArgs& a, const Tok& k, int n_o, const int* list, int w_lo,
                                             int key0, int key_end, Meta* m) {
  const KeyLoc kl = resolve_issue(a, k, n_o, list, w_lo, key0, key_end);
  KeyScale<PER_TILE> sc;
  resolve_rows<PER_TILE>(a, k, kl, m, sc);
  resolve_scales<PER_TILE>(sc, kl.valid, m);
}

// Row of key `key` for the debug export (same resolution code).
__device__ __forceinline__ int64_t resolve_row(const KArgs& a, const Tok& k, int n_o, int key, const int* list,
                                               int w_lo) {
  KeyLoc kl;
  kl.valid = 1;
  kl.cmp = key >= n_o;
  kl.j = !kl.cmp ? k.lo + key : ((a.topk > 0) ? list[key - n_o - w_lo] : key - n_o);
  kl.blk = 0;
  if (a.layout_kv == 2) {
    const int bs = kl.cmp ? a.cmp_bs : a.ori_bs;
    const int* tab = kl.cmp ? a.cmp_tab : a.ori_tab;
    const int cols = kl.cmp ? a.cmp_cols : a.ori_cols;
    kl.blk = tab[(size_t)k.b * cols + kl.j / bs];
  }
  return key_row(a, k, kl);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Gather the 64 rows of a tile into LDS: 4 waves x 8 instructions, each
// instruction 2 rows (lanes 0-31 and 32-63, 16 bytes per lane), issued as
// global_load_lds_dwordx4 (M0 = LDS destination, lane l writes base + 16 l).
// The loads are ordered only by the explicit waits of the pipeline barriers,
// so the compiler does not hold the other tile's LDS reads behind them.
__device__ __forceinline__ void gather_tile(const Meta* m, uint8_t* tb, int w) {
  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31;
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) {
    const int r0 = 16 * w + 2 * mi;
    const int r = r0 + g;
    const uint64_t p = m->addr[r];
    if (p) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(tb + r0 * kD));
      const uint64_t src = p + 16u * (uint32_t)(li ^ swz(r));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src) : "m0");
    } else {
      *(v4i*)(tb + r * kD + li * 16) = v4i{0, 0, 0, 0};
    }
  }
}

__device__ __forceinline__ void wait_all_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Work-group barrier that orders LDS only: outstanding global loads (the
// next tile's gather, descale prefetches) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Barrier at the end of a pipeline step: the gather into LDS must have landed;
// the wave's last NDS global loads (descale prefetches) may still be in flight.
template <int NDS>
__device__ __forceinline__ void step_barrier() {
  if (NDS == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (NDS == 1) asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// attention kernel
// ---------------------------------------------------------------------------

// Per-lane LDS byte offsets, fixed for the whole kernel.  The parts that vary
// with the K-step / d-block are multiples of 128 bytes and the buffer parity
// is 32 KiB: both go into the ds_read immediate offset.
struct LaneOffsets {
  int qk[2][2][2];   // [m-tile tt][K-step parity][16-byte half]: K row reads for S^T = K Q^T
  int tr[4][4];      // [rho][d-block mod 4]: source address of the V^T transpose reads
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
  LaneOffsets o;
  const int g = lane >> 5, li = lane & 31;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int key = 32 * tt + li, f = swz(key);
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int x = 0; x < 2; ++x) o.qk[tt][sp][x] = kOffTiles + key * kD + 16 * ((4 * sp + 2 * g + x) ^ f);
  }
  const int trx = (lane >> 4) & 1;
#pragma unroll
  for (int rho = 0; rho < 4; ++rho) {
    const int key = 16 * rho + 8 * ((lane >> 3) & 1) + 4 * (lane >> 5) + ((lane >> 1) & 3);
    const int f = swz(key);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      o.tr[rho][b] = kOffTiles + key * kD + 8 * (lane & 1) + 16 * (((2 * b) ^ (f & 6)) + (trx ^ (f & 1)));
  }
  return o;
}

// K operand (32 keys x 64 d, d in [64 s8, +64)) of m-tile tt.
template <int BUF>
__device__ __forceinline__ v8i read_k(const uint8_t* smem, const LaneOffsets& o, int tt, int s8) {
  const int a = s8 >> 1, sp = s8 & 1;
  const v4i lo = *(const v4i*)(smem + o.qk[tt][sp][0] + BUF * kTileBytes + 128 * a);
  const v4i hi = *(const v4i*)(smem + o.qk[tt][sp][1] + BUF * kTileBytes + 128 * a);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// V^T operand (32 d x 64 keys) of d-block nt, via LDS transpose reads.
template <int BUF>
__device__ __forceinline__ v8i read_vt(const uint8_t* smem, const LaneOffsets& o, int nt) {
  const int a = nt >> 2, b = nt & 3;
  v8i av;
#pragma unroll
  for (int rho = 0; rho < 4; ++rho) {
    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_v2i*)(smem + o.tr[rho][b] + BUF * kTileBytes + 128 * a));
    av[2 * rho] = x[0];
    av[2 * rho + 1] = x[1];
  }
  return av;
}

// One 64-key tile of one wave (32 heads, 256 output columns of half DH).
// The first tile with visible keys fixes each head's reference Mrun (unless
// it was preset); a later tile that would push P' past 2^8 only raises
// *flag, and the unit is then recomputed with Mrun preset from its true
// maximum (MAXONLY = 1 computes that maximum: S^T and the max, no P V).
template <int PER_TILE, int BUF, int DH, int MAXONLY>
__device__ __forceinline__ void compute_tile(uint8_t* smem, const LaneOffsets& o, const Meta* m,
                                             const v8i (&qreg)[4], float qs, int nvalid, int w, int lane,
                                             v16f (&oacc)[8], float& Mrun, float& lsum, int* flag) {
  const int g = lane >> 5;
  // ---- partial S^T over this wave's half of D ----
  v16f sacc[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    sacc[tt] = v16f{};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int s8 = 4 * DH + s4;
      const v8i av = read_k<BUF>(smem, o, tt, s8);
      if (PER_TILE) {
        const v16f part = mma(av, qreg[s4], v16f{});
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const v4f kv = *(const v4f*)&m->ks[s8][32 * tt + 8 * q4 + 4 * g];
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[tt][4 * q4 + r] += kv[r] * part[4 * q4 + r];
        }
      } else {
        sacc[tt] = mma(av, qreg[s4], sacc[tt]);
      }
    }
  }
  // ---- add the partner's half (same heads, other half of D) ----
  float* xw = reinterpret_cast<float*>(smem + kOffXchg) + w * 2048;
  const float* xp = reinterpret_cast<const float*>(smem + kOffXchg) + (w ^ 2) * 2048;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *(v4f*)&xw[((tt * 4 + r4) * 64 + lane) * 4] =
          v4f{sacc[tt][4 * r4], sacc[tt][4 * r4 + 1], sacc[tt][4 * r4 + 2], sacc[tt][4 * r4 + 3]};
  lds_barrier();
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const v4f pv = *(const v4f*)&xp[((tt * 4 + r4) * 64 + lane) * 4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[tt][4 * r4 + r] += pv[r];
    }
  // ---- exponent E = s*log2(e) + log2(vds), masked past nvalid; in place ----
  float mt = kNegInf;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int kb4 = 32 * tt + 8 * q4 + 4 * g;
      const v4f lam = *(const v4f*)&m->lam[kb4];
      v4f kd = {1.f, 1.f, 1.f, 1.f};
      if (!PER_TILE) kd = *(const v4f*)&m->ks[0][kb4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sv = sacc[tt][4 * q4 + r] * (PER_TILE ? qs : qs * kd[r]) + lam[r];
        const float ev = (kb4 + r < nvalid) ? sv : kNegInf;
        sacc[tt][4 * q4 + r] = ev;
        mt = fmaxf(mt, ev);
      }
    }
  }
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  if (MAXONLY) {
    Mrun = fmaxf(Mrun, mt);
    return;
  }
  // Mrun is the reference of P' = 2^(E - Mrun): the max maps to 2^4, and P'
  // may grow to 2^8 before the reference would have to move.
  if (Mrun == kNegInf) Mrun = mt - kPShift;          // first tile with keys: O is still zero
  else if (__ballot(mt > Mrun + kTau)) *flag = 1;    // would overflow fp8: redo with a preset reference
  const float Ms = (Mrun == kNegInf) ? 0.f : Mrun;
  // ---- P' = 2^(E - M) in (0, 2^8]; l accumulates P' / vds_max ----
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int kb4 = 32 * tt + 8 * q4 + 4 * g;
      const v4f iv = *(const v4f*)&m->inv[kb4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = __builtin_amdgcn_exp2f(sacc[tt][4 * q4 + r] - Ms);
        const float lt = pv * iv[r];
        lsum += lt;
        sacc[tt][4 * q4 + r] = PER_TILE ? lt : pv;
      }
    }
  }
  // ---- O^T += V^T P'^T over this wave's 8 d-blocks; P' = hi + lo, both fp8 ----
  if (PER_TILE) {
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int c = 4 * DH + c4;   // 64-wide D tile
      v8i ph, pl;
#pragma unroll
      for (int rg = 0; rg < 8; ++rg) {
        // P byte b = 16*tt + r  <->  key 32*tt + 8*(r/4) + 4*g + r%4
        const int tt = rg >> 2, q4 = rg & 3;
        const v4f kv = *(const v4f*)&m->ks[c][32 * tt + 8 * q4 + 4 * g];
        int hv, lv;
        split_fp8(sacc[tt][4 * q4] * kv[0], sacc[tt][4 * q4 + 1] * kv[1], sacc[tt][4 * q4 + 2] * kv[2],
                  sacc[tt][4 * q4 + 3] * kv[3], hv, lv);
        ph[rg] = hv;
        pl[rg] = lv;
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int j = 2 * c4 + h2;
        const v8i vt = read_vt<BUF>(smem, o, 8 * DH + j);
        oacc[j] = mma(vt, ph, oacc[j]);
        oacc[j] = mma(vt, pl, oacc[j]);
      }
    }
  } else {
    v8i ph, pl;
#pragma unroll
    for (int rg = 0; rg < 8; ++rg) {
      const int tt = rg >> 2, q4 = rg & 3;
      int hv, lv;
      split_fp8(sacc[tt][4 * q4], sacc[tt][4 * q4 + 1], sacc[tt][4 * q4 + 2], sacc[tt][4 * q4 + 3], hv, lv);
      ph[rg] = hv;
      pl[rg] = lv;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const v8i vt = read_vt<BUF>(smem, o, 8 * DH + j);
      oacc[j] = mma(vt, ph, oacc[j]);
      oacc[j] = mma(vt, pl, oacc[j]);
    }
  }
}

struct Chunk {
  int st, en, tiles;
};

struct UnitState {
  Tok k;
  int t, n_o, w_lo, n_c, kb, ke;
};

// One pipeline step i: gather tile i+1 | issue table loads of tile i+2 |
// compute tile i | descales of tile i+1 into meta, row addresses and
// descale loads of tile i+2 | barrier (gather landed).
template <int PER_TILE, int BUF, int DH, int MAXONLY>
__device__ __forceinline__ void pipeline_step(const KArgs& a, const UnitState& us, const int* list, uint8_t* smem,
                                              const LaneOffsets& o, Meta* mm, const Chunk& ck, int i, int w, int lane,
                                              const v8i (&qreg)[4], float qs, v16f (&oacc)[8], float& Mrun,
                                              float& lsum, KeyScale<PER_TILE>& sc_next, int& valid_next, int* flag) {
  if (i + 1 < ck.tiles) gather_tile(mm + (i + 1) % 3, smem + kOffTiles + (BUF ^ 1) * kTileBytes, w);
  KeyLoc kl2;
  const bool r2 = (w == 0) && (i + 2 < ck.tiles);
  if (r2) kl2 = resolve_issue(a, us.k, us.n_o, list, us.w_lo, ck.st + (i + 2) * kTileKeys, ck.en);
  const int nvalid = min(kTileKeys, ck.en - ck.st - i * kTileKeys);
  compute_tile<PER_TILE, BUF, DH, MAXONLY>(smem, o, mm + i % 3, qreg, qs, nvalid, w, lane, oacc, Mrun, lsum, flag);
  if (w == 0) {
    if (i + 1 < ck.tiles) resolve_scales<PER_TILE>(sc_next, valid_next, mm + (i + 1) % 3);
    if (r2) {
      resolve_rows<PER_TILE>(a, us.k, kl2, mm + (i + 2) % 3, sc_next);
      valid_next = kl2.valid;
      step_barrier<PER_TILE ? 2 : 1>();
      return;
    }
  }
  step_barrier<0>();
}

// Runs the unit's key range [kb, ke) into (oacc, Mrun, lsum); Mrun enters
// as the preset reference (-inf: set by the first tile).  With MAXONLY it
// only leaves the per-head maximum exponent in Mrun.
template <int PER_TILE, int DH, int MAXONLY>
__device__ __forceinline__ void run_unit(const KArgs& a, UnitState& us, int* list, int* misc, uint8_t* smem,
                                         const LaneOffsets& lo, int w, int lane, const v8i (&qreg)[4], float qs,
                                         v16f (&oacc)[8], float& Mrun, float& lsum) {
  Meta* mm = reinterpret_cast<Meta*>(smem + kOffMeta);
  int* flag = misc + 4;
  if (!MAXONLY) {
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[j] = v16f{};
  }
  lsum = 0.f;
  // chunks of at most kListMax keys, so that a chunk's cmp entries fit the list
  for (int c0 = us.kb; c0 < us.ke; c0 += kListMax) {
    const int c1 = min(us.ke, c0 + kListMax);
    if (a.topk > 0 && us.n_c > kListMax) {
      const int need_lo = max(c0 - us.n_o, 0), need_hi = max(c1 - us.n_o, 0);
      if (need_hi > need_lo && (need_lo < us.w_lo || need_hi > us.w_lo + kListMax)) {
        us.w_lo = need_lo;
        compact_indices(a, us.k, us.t, list, misc, us.w_lo);
      }
    }
    Chunk ck;
    ck.st = c0;
    ck.en = c1;
    ck.tiles = (c1 - c0 + kTileKeys - 1) / kTileKeys;
    KeyScale<PER_TILE> sc_next;
    int valid_next = 0;
    if (w == 0) {
      resolve_tile<PER_TILE>(a, us.k, us.n_o, list, us.w_lo, ck.st, ck.en, mm + 0);
      if (ck.tiles > 1) {
        const KeyLoc kl1 = resolve_issue(a, us.k, us.n_o, list, us.w_lo, ck.st + kTileKeys, ck.en);
        resolve_rows<PER_TILE>(a, us.k, kl1, mm + 1, sc_next);
        valid_next = kl1.valid;
      }
    }
    wait_all_and_sync();
    gather_tile(mm + 0, smem + kOffTiles, w);
    wait_all_and_sync();
    for (int i = 0; i < ck.tiles; i += 2) {
      pipeline_step<PER_TILE, 0, DH, MAXONLY>(a, us, list, smem, lo, mm, ck, i, w, lane, qreg, qs, oacc, Mrun, lsum,
                                              sc_next, valid_next, flag);
      if (i + 1 < ck.tiles)
        pipeline_step<PER_TILE, 1, DH, MAXONLY>(a, us, list, smem, lo, mm, ck, i + 1, w, lane, qreg, qs, oacc, Mrun,
                                                lsum, sc_next, valid_next, flag);
    }
  }
}

template <int PER_TILE, int DH>
__device__ __forceinline__ void attn_body(const KArgs& a, uint8_t* smem, int w) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int hh = w & 1, g = lane >> 5, li = lane & 31;
  const int h = 32 * hh + li;
  const int G = a.grid;
  const int bid = blockIdx.x;
  const int lw = (G % 8 == 0) ? ((bid & 7) * (G >> 3) + (bid >> 3)) : bid;  // one XCD per contiguous range
  const int u_begin = a.starts[lw], u_end = a.starts[lw + 1];
  int* list = reinterpret_cast<int*>(smem + kOffList);
  int* misc = reinterpret_cast<int*>(smem + kOffMisc);
  const LaneOffsets lo = lane_offsets(lane);

  for (int u = u_begin; u < u_end; ++u) {
    UnitState us;
    us.t = u / a.splits;
    const int s = u - us.t * a.splits;
    us.k = token_ctx(a, us.t);
    const int t = us.t;
    if (!us.k.valid) {   // padded query row: O = 0, lse = -inf
      if (a.splits == 1) {
        for (int x = lane; x < 32 * 64; x += 64) {
          const int hr = 32 * hh + x / 64, d = 256 * DH + 4 * (x % 64);
          *(uint2*)(a.out + ((size_t)t * kN1 + hr) * kD + d) = make_uint2(0, 0);
        }
        if (a.lse && DH == 0 && g == 0) a.lse[(size_t)t * kN1 + h] = kNegInf;
      } else if (DH == 0 && g == 0) {
        a.ws_ml[((size_t)u * kN1 + h) * 2] = kNegInf;
        a.ws_ml[((size_t)u * kN1 + h) * 2 + 1] = -1.0f;   // marks a padded row for the combine
      }
      continue;
    }

    // query fragment: B operand of S^T = K Q^T for d in [256 DH + 64 s4 + 32 g, +32)
    v8i qreg[4];
    {
      const uint8_t* qrow = a.q + ((size_t)t * kN1 + h) * kD + 256 * DH + 32 * g;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const v4i x0 = *(const v4i*)(qrow + 64 * s4);
        const v4i x1 = *(const v4i*)(qrow + 64 * s4 + 16);
        qreg[s4] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
    }
    const float qd = a.q_ds_per_head ? a.q_ds[(size_t)t * kN1 + h] : a.q_ds[t];
    const float qs = a.scale_log2 * qd;

    us.n_o = us.k.hi - us.k.lo;
    us.n_c = 0;
    us.w_lo = 0;
    if (a.topk > 0) us.n_c = compact_indices(a, us.k, t, list, misc, 0);
    else if (a.has_cmp) us.n_c = us.k.vis;
    const int64_t n = (int64_t)us.n_o + us.n_c;
    us.kb = (int)(n * s / a.splits);
    us.ke = (int)(n * (s + 1) / a.splits);

    v16f oacc[8];
    float Mrun = kNegInf, lsum = 0.f;
    for (int pass = 0;; ++pass) {
      if (tid == 0) misc[4] = 0;
      run_unit<PER_TILE, DH, 0>(a, us, list, misc, smem, lo, w, lane, qreg, qs, oacc, Mrun, lsum);
      __syncthreads();
      const int redo = misc[4];
      __syncthreads();
      if (!redo || pass > 0) break;
      // a later tile outgrew the first tile's fp8 window: find each head's
      // maximum exponent, then recompute with the reference preset from it
      float mx = kNegInf;
      run_unit<PER_TILE, DH, 1>(a, us, list, misc, smem, lo, w, lane, qreg, qs, oacc, mx, lsum);
      Mrun = (mx == kNegInf) ? kNegInf : mx - kPShift;
    }

    // ---------------- write: final output (one split) or partial state ----------------
    const float lh = lsum + __shfl_xor(lsum, 32);
    float sc;
    if (a.splits == 1) {
      const float sg = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
      const float Mf = fmaxf(Mrun, sg);
      float lse_v = kNegInf;
      sc = 0.f;
      if (Mf != kNegInf) {
        const float af = (Mrun == kNegInf) ? 0.f : exp2f(Mrun - Mf);
        const float Lf = af * lh + ((sg == kNegInf) ? 0.f : exp2f(sg - Mf));
        sc = af / Lf;
        lse_v = (Mf + __log2f(Lf)) * kLn2;
      }
      if (a.lse && DH == 0 && g == 0) a.lse[(size_t)t * kN1 + h] = lse_v;
    } else {
      sc = (lh > 0.f) ? 1.0f / lh : 0.f;
      if (DH == 0 && g == 0) {
        a.ws_ml[((size_t)u * kN1 + h) * 2] = Mrun;
        a.ws_ml[((size_t)u * kN1 + h) * 2 + 1] = lh;
      }
    }
    uint16_t* dst = (a.splits == 1) ? a.out + ((size_t)t * kN1 + h) * kD : a.ws_o + ((size_t)u * kN1 + h) * kD;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const v16f& ov = oacc[j];
        const int d = 32 * (8 * DH + j) + 8 * r4 + 4 * g;
        *(uint2*)(dst + d) = pack_bf16x4(sc * ov[4 * r4], sc * ov[4 * r4 + 1], sc * ov[4 * r4 + 2], sc * ov[4 * r4 + 3]);
      }
    }
  }
}

template <int PER_TILE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_kernel(const KArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (w >> 1) attn_body<PER_TILE, 1>(a, smem, w);
  else attn_body<PER_TILE, 0>(a, smem, w);
}

// ---------------------------------------------------------------------------
// split-KV combine: merge the sink-free partial states of every split with
// the log-sum-exp rule and add the sink logit once.
// grid (t1, 8): 8 heads per work-group; 256 threads = 8 heads x 32 x 16 cols.
// All loads of a batch of 8 splits are issued before any is used.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) combine_kernel(const KArgs a) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * 8 + (threadIdx.x >> 5);
  const int col = (threadIdx.x & 31) * 16;
  const int S = a.splits;
  uint16_t* dst = a.out + ((size_t)t * kN1 + h) * kD + col;
  const float* ml = a.ws_ml + ((size_t)t * S * kN1 + h) * 2;   // split s at + s * kN1 * 2
  const size_t ostride = (size_t)kN1 * kD;
  const uint16_t* op = a.ws_o + ((size_t)t * S * kN1 + h) * kD + col;
  const float sg = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
  float M = sg;
  bool padded = false;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float m8[8], l8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      m8[j] = (s0 + j < S) ? ml[(size_t)(s0 + j) * kN1 * 2] : kNegInf;
      l8[j] = (s0 + j < S) ? ml[(size_t)(s0 + j) * kN1 * 2 + 1] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      M = fmaxf(M, m8[j]);
      padded |= l8[j] < 0.f;
    }
  }
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  float L = 0.f;
  if (!padded && M != kNegInf) {
    L = (sg == kNegInf) ? 0.f : exp2f(sg - M);
    for (int s0 = 0; s0 < S; s0 += 8) {
      float wgt[8];
      uint4 x0[8], x1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool in = s0 + j < S;
        const float Ms = in ? ml[(size_t)(s0 + j) * kN1 * 2] : kNegInf;
        const float ls = in ? ml[(size_t)(s0 + j) * kN1 * 2 + 1] : 0.f;
        wgt[j] = (Ms == kNegInf) ? 0.f : ls * exp2f(Ms - M);
        if (in) {
          const uint4* src = (const uint4*)(op + (size_t)(s0 + j) * ostride);
          x0[j] = src[0];
          x1[j] = src[1];
        } else {
          x0[j] = make_uint4(0, 0, 0, 0);
          x1[j] = x0[j];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        L += wgt[j];
        const uint32_t xs[8] = {x0[j].x, x0[j].y, x0[j].z, x0[j].w, x1[j].x, x1[j].y, x1[j].z, x1[j].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[2 * e] += wgt[j] * __uint_as_float(xs[e] << 16);
          acc[2 * e + 1] += wgt[j] * __uint_as_float(xs[e] & 0xffff0000u);
        }
      }
    }
  }
  const float inv = (L > 0.f) ? 1.0f / L : 0.f;
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = bf16_rne(acc[2 * j] * inv) | (bf16_rne(acc[2 * j + 1] * inv) << 16);
  *(uint4*)dst = make_uint4(o[0], o[1], o[2], o[3]);
  *(uint4*)(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
  if (a.lse && (threadIdx.x & 31) == 0)
    a.lse[(size_t)t * kN1 + h] = (!padded && L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------------------
// debug export of the resolved key rows (same resolution code as above)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) debug_resolve_kernel(const KArgs a, int32_t* keys, int32_t* counts,
                                                                 int32_t max_keys) {
  __shared__ int list[kListMax];
  __shared__ int wtot[4];
  const int t = blockIdx.x;
  const Tok k = token_ctx(a, t);
  const int n_o = k.hi - k.lo;
  int n_c = 0;
  if (a.topk > 0) n_c = compact_indices(a, k, t, list, wtot, 0);
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
        compact_indices(a, k, t, list, wtot, w_lo);
      }
    }
    for (int key = c0 + threadIdx.x; key < c1; key += kThreads)
      keys[(size_t)t * max_keys + key] = (int32_t)resolve_row(a, k, n_o, key, list, w_lo);
    __syncthreads();
  }
}

}  // namespace

int launch_forward(const KArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (a.scale_mode == 1)
    hipLaunchKernelGGL(attn_kernel<1>, dim3(a.grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(attn_kernel<0>, dim3(a.grid), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  if (a.splits > 1) {
    hipLaunchKernelGGL(combine_kernel, dim3(a.t1, kN1 / 8), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  return (int)e;
}

int launch_debug_resolve(const KArgs& a, int32_t* keys, int32_t* counts, int32_t max_keys, void* stream) {
  hipLaunchKernelGGL(debug_resolve_kernel, dim3(a.t1), dim3(kThreads), 0, (hipStream_t)stream, a, keys, counts,
                     max_keys);
  return (int)hipGetLastError();
}

}  // namespace csmla

