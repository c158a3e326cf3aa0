// HIP kernels for gfx950 (MI355X): the lightning-indexer top-k
// (QuantLightningIndexerV2 page, 功能说明 formula and steps 1-3; quant_mode 1:
// fp8 e4m3 query and key, fp32 dequant scales and weights).
//
// idx_score_kernel — work-group (key chunk, row tile, batch) of 4 waves.  A
// wave holds the fp8 query operands of its TW rows in VGPRs and walks its
// keys in steps of 64, loading each key row straight from HBM (lane j + 16g
// reads bytes [32g, 32g + 32) of key j of a 16-key group: 2 KiB contiguous
// per group when the rows are).  Per row and step, 4 key groups x 4 head
// blocks of v_mfma_f32_16x16x128_f8f6f4 (A lane i+16g: head i, k = 32g..+31;
// B lane j+16g: key j; D lane j+16g, reg r: S[head 4g+r][key j]); then, in
// registers, ReLU and the per-head factor W * scale_q (16 heads per lane), a
// 3-shuffle reduce-scatter over the four lane groups that leaves lane l with
// key l of the step, the key's scale, and one coalesced 256-byte store.
// With scale_q, scale_k >= 0, W * ReLU(scale_q * scale_k * x) equals
// scale_k * (W * scale_q) * ReLU(x), so the key scale multiplies the sum once.
//
// idx_topk_kernel — one work-group per query row: up to three rounds of radix
// selection (11, 11 and 10 bits) over order-preserving integer keys of the
// float32 scores (an LDS histogram per round and a suffix scan to find the
// digit of the topk-th largest; it stops as soon as the chosen bin is taken
// whole), then one pass in index order that writes every score above the
// threshold and the lowest-positioned ties, so the output comes out in
// ascending position order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csmla.h"
#include "csmla_indexer_internal.h"

namespace csmla_idx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mma16(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const v4i x0 = *(const v4i*)p;
  const v4i x1 = *(const v4i*)(p + 16);
  return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// Lengths of batch b (QuantLightningIndexerV2, 参数说明: cu_seqlens_q/k,
// seqused_q/k, cmp_residual_k).
struct Batch {
  int q0, s1, n, res;
};

__device__ __forceinline__ Batch batch_of(const IArgs& a, int b) {
  Batch c;
  int span;
  if (a.layout_q == CSMLA_LAYOUT_TND) {
    c.q0 = a.cu_q[b];
    span = a.cu_q[b + 1] - c.q0;
  } else {
    c.q0 = b * a.q_s;
    span = a.q_s;
  }
  c.s1 = a.su_q ? max(0, min(span, a.su_q[b])) : span;
  if (a.layout_k == CSMLA_LAYOUT_TND) c.n = a.cu_k[b + 1] - a.cu_k[b];
  else if (a.su_k) c.n = a.su_k[b];
  else c.n = a.k_s;
  c.n = max(c.n, 0);
  c.res = a.res ? a.res[b] : 0;
  return c;
}

// Leading keys row i of the batch sees: all n, or under the right-down causal
// mask floor((p + 1) / ratio) with p = n * ratio + res - s1 + i; never more
// than a score row holds.
__device__ __forceinline__ int visible(const IArgs& a, const Batch& c, int i) {
  int v = c.n;
  if (a.mask == CSMLA_MASK_RIGHT_DOWN_CAUSAL) {
    const long long p1 = (long long)c.n * a.ratio + c.res - c.s1 + i + 1;
    v = p1 <= 0 ? 0 : (int)min((long long)c.n, p1 / a.ratio);
  }
  return min(v, a.stride);
}

// ---------------------------------------------------------------------------
// scores
// ---------------------------------------------------------------------------

// The fp8 key operands (4 groups of 16 keys) and the key scale of one step.
struct Step {
  v8i k[4];
  float s;
};

template <int TW, int WT>
__global__ __launch_bounds__(256) void idx_score_kernel(IArgs a) {
  constexpr int KP = 4 / WT;                 // waves of a work-group that split the keys
  const int b = blockIdx.z;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hi = lane & 15, grp = lane >> 4;
  const int part = a.kc / KP;
  const int k0 = blockIdx.x * a.kc + (w / WT) * part;
  const bool paged = a.layout_k == CSMLA_LAYOUT_PA_BBND;

  // Block-table entries of the blocks the wave's keys can touch (at most 64,
  // as planned), one per lane, read before any length is known; later rows
  // come from a lane shuffle.  Without paging the read is a harmless word.
  const int blk0 = paged ? (a.bs_shift >= 0 ? k0 >> a.bs_shift : k0 / a.bs) : 0;
  const int tabreg = a.tab[(long long)b * a.tab_ld + min(blk0 + lane, a.tab_cols - 1)];

  const Batch c = batch_of(a, b);
  const int i0 = (blockIdx.y * WT + w % WT) * TW;
  if (i0 >= c.s1) return;
  const int nt = min(TW, c.s1 - i0);
  int vis[TW];
  int vmax = 0;
#pragma unroll
  for (int r = 0; r < TW; ++r) {
    vis[r] = r < nt ? visible(a, c, i0 + r) : 0;
    vmax = max(vmax, vis[r]);
  }
  const int k1 = min(k0 + part, vmax);
  if (k0 >= k1) return;
  const int kbase = a.layout_k == CSMLA_LAYOUT_TND ? a.cu_k[b] : b * a.k_s;

  // Row of key s (k0 <= s < k1) in the cache, clamped into the cache.
  auto row_of = [&](int s) -> int {
    const int bi = a.bs_shift >= 0 ? s >> a.bs_shift : s / a.bs;
    const int blk = __shfl(tabreg, bi - blk0);
    const int pr = min(max(blk, 0) * a.bs + (s - bi * a.bs), a.nrows - 1);
    const int cr = min(kbase + s, a.nrows - 1);
    return paged ? pr : cr;
  };
  // Issue the loads of the step at `base`; keys past k1 repeat key k1 - 1.
  auto issue = [&](int base, Step& st) {
    int myrow = 0;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int row = row_of(min(base + 16 * kg + hi, k1 - 1));
      st.k[kg] = load32(a.key + (long long)row * kD + 32 * grp);
      myrow = kg == grp ? row : myrow;                   // key base + lane after the reduction
    }
    st.s = a.ks[myrow];
  };

  Step A, B;
  issue(k0, A);

  // query operands and the per-head factors W * scale_q of this lane's heads
  // (rows past the batch and heads past g read a valid row, then count zero)
  v8i qa[TW][4];
  float wq[TW][4][4];
#pragma unroll
  for (int r = 0; r < TW; ++r) {
    const long long t = c.q0 + i0 + min(r, nt - 1);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int head = 16 * hb + hi;
      const v8i x = load32(a.q + (t * a.g + min(head, a.g - 1)) * kD + 32 * grp);
      const bool on = r < nt && head < a.g;
#pragma unroll
      for (int e = 0; e < 8; ++e) qa[r][hb][e] = on ? x[e] : 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int h2 = 16 * hb + 4 * grp + e;
        const long long j = t * a.g + min(h2, a.g - 1);
        const float f = a.w[j] * a.qs[j];
        wq[r][hb][e] = (r < nt && h2 < a.g) ? f : 0.f;
      }
    }
  }

  auto compute = [&](int base, const Step& st) {
#pragma unroll
    for (int r = 0; r < TW; ++r) {
      if (r < nt) {
        float p[4];
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
          v4f acc[4];
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) acc[hb] = mma16(qa[r][hb], st.k[kg], v4f{0.f, 0.f, 0.f, 0.f});
          float s = 0.f;
#pragma unroll
          for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int e = 0; e < 4; ++e) s = fmaf(wq[r][hb][e], fmaxf(acc[hb][e], 0.f), s);
          p[kg] = s;
        }
        // reduce-scatter over lane groups g = lane / 16: afterwards lane l
        // holds the sum over all 64 heads for key 16 (l / 16) + l % 16 = l
        const bool upper = lane >= 32;
        const float a0 = (upper ? p[2] : p[0]) + __shfl_xor(upper ? p[0] : p[2], 32);
        const float a1 = (upper ? p[3] : p[1]) + __shfl_xor(upper ? p[1] : p[3], 32);
        const bool odd = (lane >> 4) & 1;
        const float tot = (odd ? a1 : a0) + __shfl_xor(odd ? a0 : a1, 16);
        const int key = base + lane;
        if (key < vis[r]) a.scores[(long long)(c.q0 + i0 + r) * a.stride + key] = st.s * tot;
      }
    }
  };

  // two buffers: the next step's keys are in flight while this one multiplies
  const int nsteps = (k1 - k0 + kStep - 1) / kStep;
  for (int st = 0; st < nsteps; st += 2) {
    issue(k0 + (st + 1) * kStep, B);
    compute(k0 + st * kStep, A);
    if (st + 1 >= nsteps) break;
    issue(k0 + (st + 2) * kStep, A);
    compute(k0 + (st + 1) * kStep, B);
  }
}

// ---------------------------------------------------------------------------
// top-k
// ---------------------------------------------------------------------------

// Unsigned key with the order of the float (-0 taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the work-group's threads; `total` gets the sum.
// `wsum` (one word per wave) must not be reused by the next call.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int j = 0; j < NT / 64; ++j) {
    const uint32_t s = wsum[j];
    if (j < w) before += s;
    total += s;
  }
  return before + x - v;
}

// Batch of query row t: t / S1 (BSND), or the last batch whose
// cu_seqlens_q entry is <= t (TND), found 64 entries per load.
__device__ __forceinline__ int batch_of_row(const IArgs& a, int t) {
  if (a.layout_q != CSMLA_LAYOUT_TND) return t / a.q_s;
  const int lane = threadIdx.x & 63;
  int b = 0;
  for (int j0 = 0; j0 < a.batch; j0 += 64) {
    const int cv = a.cu_q[min(j0 + lane, a.batch - 1)];
    const bool le = (j0 + lane < a.batch) & (cv <= t);
    b += __popcll(__ballot(le));
  }
  return b - 1;
}

template <int NT, int C>
__global__ __launch_bounds__(NT) void idx_topk_kernel(IArgs a) {
  constexpr int NB = 2048;                   // bins of an 11-bit digit
  constexpr int BPT = NB / NT;               // bins per thread in the scan
  __shared__ uint32_t hist[NB];
  __shared__ uint32_t wsum[2][NT / 64];
  __shared__ int32_t pick[3];
  constexpr int CH = 4 * NT;                 // scores per chunk; thread tid holds [4 tid, 4 tid + 4)
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* row = a.scores + (long long)t * a.stride;
  auto load = [&](int cc, uint32_t (&u)[4]) {
    const int j0 = min(cc * CH + 4 * tid, a.stride - 4);   // stays in the row; masked by vis below
    const v4f x = *(const v4f*)(row + j0);
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = order_key(x[e]);
  };
  // the cached part of the row is read before the row's length is known
  uint32_t cache[C][4];
#pragma unroll
  for (int cc = 0; cc < C; ++cc) load(cc, cache[cc]);

  const int b = batch_of_row(a, t);
  const Batch c = batch_of(a, b);
  const int i = t - c.q0;
  int32_t* out = a.out + (long long)t * a.topk;
  const int vis = (i < c.s1) ? visible(a, c, i) : 0;
  if (vis <= a.topk) {                       // every visible key, then -1
    for (int j = tid; j < a.topk; j += NT) out[j] = j < vis ? j : -1;
    return;
  }
  const int nch = (vis + CH - 1) / CH;

  // radix selection of the topk-th largest key: digits of 11, 11 and 10
  // bits; stop early once the chosen bin is taken whole
  uint32_t prefix = 0;
  int need = a.topk, sh = 0, sb = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t hmask = pass == 0 ? 0u : (pass == 1 ? 0xFFFFFFFFu << 21 : 0xFFFFFFFFu << 10);
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
#pragma unroll
    for (int j = 0; j < BPT; ++j) hist[tid * BPT + j] = 0;
    __syncthreads();
    auto count = [&](int cc, const uint32_t (&u)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = cc * CH + 4 * tid + e;
        if (idx < vis && (u[e] & hmask) == prefix) atomicAdd(&hist[(u[e] >> shift) & dmask], 1u);
      }
    };
#pragma unroll
    for (int cc = 0; cc < C; ++cc)
      if (cc < nch) count(cc, cache[cc]);
    for (int cc = C; cc < nch; ++cc) {
      uint32_t u[4];
      load(cc, u);
      count(cc, u);
    }
    __syncthreads();
    // thread tid holds digits NB-1 - (tid*BPT + j), j = 0..BPT-1 (descending)
    uint32_t hv[BPT], local = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      hv[j] = hist[NB - 1 - (tid * BPT + j)];
      local += hv[j];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan<NT>(local, wsum[sb++ & 1], total);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (run < (uint32_t)need && run + hv[j] >= (uint32_t)need) {
        pick[0] = NB - 1 - (tid * BPT + j);
        pick[1] = need - (int)run;
        pick[2] = (int)hv[j];
      }
      run += hv[j];
    }
    __syncthreads();
    prefix |= (uint32_t)pick[0] << shift;
    need = pick[1];
    sh = shift;
    if (pick[2] == need) break;              // the whole bin is taken: no finer digit matters
  }

  // index-order compaction at the resolved digits: keys above the prefix,
  // then the first `need` keys equal to it; the output position of key s is
  // (keys above before s) + min(keys equal before s, need)
  const uint32_t T = prefix >> sh;
  uint32_t GT = 0, EQ = 0;
  auto emit = [&](int cc, const uint32_t (&u)[4]) {
    uint32_t ng = 0, ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = cc * CH + 4 * tid + e;
      if (idx < vis) {
        ng += (u[e] >> sh) > T;
        ne += (u[e] >> sh) == T;
      }
    }
    uint32_t total;
    const uint32_t ex = block_exclusive_scan<NT>(ng | (ne << 16), wsum[sb++ & 1], total);
    uint32_t lg = GT + (ex & 0xFFFFu), le = EQ + (ex >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = cc * CH + 4 * tid + e;
      if (idx < vis) {
        const uint32_t v = u[e] >> sh;
        if (v > T) {
          const uint32_t pos = lg + min(le, (uint32_t)need);
          if (pos < (uint32_t)a.topk) out[pos] = idx;     // always true; keeps every store in the row
          ++lg;
        } else if (v == T) {
          if (le < (uint32_t)need && lg + le < (uint32_t)a.topk) out[lg + le] = idx;
          ++le;
        }
      }
    }
    GT += total & 0xFFFFu;
    EQ += total >> 16;
  };
#pragma unroll
  for (int cc = 0; cc < C; ++cc)
    if (cc < nch) emit(cc, cache[cc]);
  for (int cc = C; cc < nch; ++cc) {
    uint32_t u[4];
    load(cc, u);
    emit(cc, u);
  }
}

}  // namespace

int launch_indexer(const IArgs& a, int nt, int cc, void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  const dim3 g1(a.nkc, a.nqt, a.batch);
  if (a.tw == 1) hipLaunchKernelGGL((idx_score_kernel<1, 1>), g1, dim3(256), 0, s, a);
  else if (a.tw == 2 && a.wt == 1) hipLaunchKernelGGL((idx_score_kernel<2, 1>), g1, dim3(256), 0, s, a);
  else if (a.tw == 2) hipLaunchKernelGGL((idx_score_kernel<2, 4>), g1, dim3(256), 0, s, a);
  else if (a.wt == 1) hipLaunchKernelGGL((idx_score_kernel<4, 1>), g1, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((idx_score_kernel<4, 4>), g1, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  const dim3 g2(a.t1);
  if (nt == 256 && cc == 1) hipLaunchKernelGGL((idx_topk_kernel<256, 1>), g2, dim3(256), 0, s, a);
  else if (nt == 256) hipLaunchKernelGGL((idx_topk_kernel<256, 4>), g2, dim3(256), 0, s, a);
  else if (cc == 2) hipLaunchKernelGGL((idx_topk_kernel<1024, 2>), g2, dim3(1024), 0, s, a);
  else if (cc == 4) hipLaunchKernelGGL((idx_topk_kernel<1024, 4>), g2, dim3(1024), 0, s, a);
  else hipLaunchKernelGGL((idx_topk_kernel<1024, 8>), g2, dim3(1024), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace csmla_idx
