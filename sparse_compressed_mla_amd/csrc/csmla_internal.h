// Internal definitions shared by the host planner (csmla_host.cpp) and the
// HIP kernels (csmla_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stdint.h>
#include <stddef.h>

namespace csmla {

constexpr int kN1 = 64;            // query heads handled by one work unit
constexpr int kD = 512;            // head dim (QuantSparseFlashMla, 约束说明: D = 512)
constexpr int kTileKeys = 64;      // keys per LDS tile
constexpr int kListMax = 1024;     // compacted cmp indices a unit keeps in LDS
constexpr int kMaxGrid = 256;      // persistent work-groups (one per CU on MI355X)
constexpr int kMaxSplits = 4096;   // splits per token
constexpr int kHeaderWords = 16;
constexpr int32_t kMagic = 0x4C4D5343;   // "CSML"

// metadata word offsets (int32[1024])
enum {
  MD_MAGIC = 0, MD_VERSION = 1, MD_PROBLEM_HASH = 2, MD_LENGTHS_HASH = 3, MD_T1 = 4,
  MD_SPLITS = 5, MD_UNITS = 6, MD_GRID = 7, MD_LIST_MAX = 8, MD_WS_LO = 9, MD_WS_HI = 10,
  MD_FLAGS = 11, MD_HEAD_GROUP = 12, MD_SPLIT_KEY = 13, MD_DK_PARTS = 14, MD_DK_TEST = 15,
  MD_STARTS = kHeaderWords
};

// Workspace layout (every plan that needs one): a sync region of fixed size
// first (the split-key decode kernel's per-token words; zero before the
// workspace's first use, and every call leaves the arrival words zero, so one
// buffer serves plans of any size), then per-unit XCD ids, the partial
// outputs and their (max, sum).
constexpr int kSkMaxTokens = 256;                          // tokens the split-key decode kernel takes
constexpr int kBkMaxUnitKeys = 1024;                       // keys per unit of the bf16-q kernel
constexpr size_t kWsSyncBytes = (size_t)kSkMaxTokens * 4 * 4;
// The head-split kernel's key parts exchange partial outputs through one slot
// per work unit, in a region of fixed size right after the sync region (so
// that no other plan's partial outputs overlap it): [0, 4) the slot's epoch,
// [64, 68) its presence word, then [16 heads x 128 column quads] 16-byte
// words (bf16 pair, tag, bf16 pair, tag), the per-head (max, sum) words and
// the writer's XCD word.  Zero before the workspace's first use; every call
// leaves the presence words zero.
constexpr int kDkMaxParts = 8;
constexpr int kDkTileKeys = 128;                           // keys per tile of the head-split kernel
constexpr int kDkWaitTicks = 2000;                         // s_memrealtime ticks (20 us) before a merger takes a part over
constexpr size_t kXchData = 256;                           // data offset in a slot
constexpr size_t kXchMl = kXchData + (size_t)16 * 128 * 16;  // per-head (max, sum) words
constexpr size_t kXchXcc = kXchMl + 16 * 16;               // the writer's XCD word
constexpr size_t kXchSlotBytes = 33792;                    // >= kXchXcc + 16, a multiple of 256
constexpr size_t kWsXchBytes = (size_t)kMaxGrid * kXchSlotBytes;
constexpr size_t kWsFixedBytes = kWsSyncBytes + kWsXchBytes;  // zeroed before first use
static_assert(kXchXcc + 16 <= kXchSlotBytes && kXchSlotBytes % 256 == 0, "exchange slot");

// Everything one kernel launch needs, passed by value in the kernarg segment:
// the problem and tensors (KHdr), then the per-work-group unit ranges.
struct KHdr {
  // problem attributes
  int32_t batch, t1, q_s, layout_q, layout_kv;
  int32_t ori_s, cmp_s, ori_bs, cmp_bs, ori_cols, cmp_cols;
  int32_t has_cmp, topk, cmp_ratio, ori_mask, cmp_mask, win_left, win_right;
  int32_t scale_mode, q_ds_per_head, ret_lse;
  int32_t n1;                       // query heads per token: the token stride of q, q_descale, out, lse
                                    // (one launch covers 64 of them; pointers start at its first head)
  float scale_log2;                 // softmax_scale * log2(e)
  // tensors
  const uint8_t* q; const float* q_ds;
  const uint8_t* ori_kv; const float* ori_ds;
  const uint8_t* cmp_kv; const float* cmp_ds;
  const int32_t* idx; const int32_t* ori_tab; const int32_t* cmp_tab;
  const int32_t* cu_q; const int32_t* cu_ori; const int32_t* cu_cmp;
  const int32_t* su_q; const int32_t* su_ori; const int32_t* su_cmp;
  const int32_t* res; const int32_t* topk_len; const float* sinks;
  uint16_t* out; float* lse;
  uint16_t* ws_o; float* ws_ml;
  int32_t* ws_sync; int32_t* ws_xcc;
  // plan
  int32_t splits, n_units, grid;
  int32_t hg;                       // > 0: head-split kernel with groups of hg heads (8 or 16)
  int32_t sk;                       // 1: split-key decode kernel (64 heads, <= 128 keys per unit, in-kernel merge)
  int32_t kv_fmt;                   // 0: fp8 rows + descales; 1: bf16 rows; 2: packed 640-byte rows (bf16 q for 1, 2)
  int32_t ori_topk;                 // > 0: the ori keys are listed in ori_idx [t1][ori_topk]
  const int32_t* ori_idx; const int32_t* ori_tkl;
  uint8_t* ws_xch;                  // exchange slots of the head-split kernel's key parts
  int32_t dk_parts;                 // head-split kernel: key parts per (token, head group) (1: none)
  int32_t dk_ticks;                 // s_memrealtime ticks a merging unit waits before it computes a part itself
  int32_t dk_test;                  // test hook: 1 = every writing part leaves at once (as if never scheduled)
};

struct KArgs : KHdr {
  int32_t starts[kMaxGrid + 1];
};

size_t workspace_bytes_for(int n_units, int splits, int dk_parts);
// byte offsets of the workspace parts (xcc ids, partial outputs, (max, sum))
void workspace_offsets(int n_units, size_t* xcc, size_t* o, size_t* ml);

// Host helpers shared by the two halves of the library (csmla_host.cpp):
// set the calling thread's last-error message and return `status`; clear it;
// FNV-1a over bytes.
int fail_with(int status, const char* fmt, ...);
void clear_last_error();
uint32_t hash_bytes(const void* data, size_t n, uint32_t seed = 2166136261u);

// Size of the library's static device scratch (csmla_forward_noalloc's
// workspace): 64 MiB per GPU, enough for ~860 split units after the fixed
// sync and exchange regions.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

// Device address of that scratch on the current device (looked up once per
// device, then cached; the first lookup also clears its sync words with a
// fill kernel on `stream`); returns a hipError_t as int.
int noalloc_scratch(void** ptr, void* stream);

// launchers (csmla_kernels.hip); return a hipError_t as int
int launch_forward(const KArgs& a, void* stream);
int launch_debug_resolve(const KArgs& a, int32_t* keys, int32_t* counts, int32_t max_keys, int whole_token,
                         void* stream);

}  // namespace csmla
