// Internal declarations shared by the libtr sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tr.h"

namespace tr {

constexpr int kMaxNodes = 128;   // tree nodes, root included
constexpr int kMaxK = 16;        // candidates per row of M
constexpr int kHeadDim = 128;    // attention head dimension
constexpr int kDrawBucket = 512;  // ids per bucket of the sampling draw
constexpr int kMaxBuckets = 512;  // so sampling takes V <= 262144

// Tree template as kernels see it: passed by value as a kernel argument,
// so no device allocation is tied to a tree.
struct TreeDev {
  int32_t T;                     // nodes, root included
  int32_t D;                     // depth (root = 0)
  uint8_t parent[kMaxNodes];     // 0xFF for the root
  uint8_t rank[kMaxNodes];
  uint8_t depth[kMaxNodes];
  uint64_t anc[kMaxNodes][2];    // bit m of anc[n]: m lies on the path root..n (n included)
};

}  // namespace tr

struct tr_tree {
  tr::TreeDev dev;
  int32_t k;
};

namespace tr {

// ---------------------------------------------------------------- workspace
// [0, 256)             status word (TR_FLAG_* bits) + padding
// [256, kCntEnd)       counters, zero between calls (each call's last block
//                      returns the ones it used to zero)
// [kDataOff, ...)      per-call scratch (top-k partial keys, top-k ids,
//                      attention partials); calls ordered on one stream may
//                      reuse it.
constexpr size_t kSeqCntOff = 256;                    // uint32 [<= 4096]
constexpr size_t kMaxSeqCnt = 4096;
constexpr size_t kRowCntOff = kSeqCntOff + 4 * kMaxSeqCnt;   // uint32 [<= 32768]
constexpr size_t kMaxRowCnt = 32768;
// the greedy step for few rows (k_step.hip):
constexpr size_t kMailOff = kRowCntOff + 4 * kMaxRowCnt;       // uint32 [< 256 rows][k]: ids | 1 << 31
constexpr size_t kVerdictOff = kMailOff + 4 * 256 * 16;        // uint64 [<= 256 sequences]
constexpr size_t kCommitCntOff = kVerdictOff + 8 * 256;        // uint32 [<= 256 sequences]
constexpr size_t kDataOff = 256 * 1024;
static_assert(kCommitCntOff + 4 * 256 <= kDataOff, "workspace counter region");

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Top-k launch shape: rows x segments.
struct TopkPlan {
  int64_t rows;
  int32_t segs;       // segments per row (1..64)
  int64_t seg_len;    // elements per segment (multiple of 8)
  int32_t kmax;       // 8 or 16 (list length kept per thread)
  int32_t threads;    // 256 (16 vectors per lane) or 1024 (4 vectors per lane)
  int64_t seg_cap;    // the longest segment a block holds (elements)
  int64_t max_v;      // the largest row length the plan supports (segments x seg_cap)
  size_t part_off;    // uint64 [rows][segs][kmax] partial keys (segs > 1)
  size_t ids_off;     // int32  [rows][k] ids when the caller gives no buffer
  size_t stat_off;    // float2 [rows][segs] softmax statistics (sampling)
  size_t end;
};
TopkPlan plan_topk(int64_t rows, int64_t V, int32_t k, int32_t esz);

// Attention launch shape.
//  bf16: a resident grid (one block per CU) over the flat (sequence, kv
//  head, 64-key sub-block) order, cut into equal ranges on the device; the
//  query rows of a (sequence, kv head) split into nt row tiles of at most
//  16 strips of 16 rows, each tile with its own gl blocks ("lane").
//  fp32: split-K chunks per (sequence, kv head, row tile) and a combine.
struct AttnPlan {
  int32_t G;          // query heads per key/value head
  int32_t R;          // query rows per (sequence, kv head) = T * G
  int32_t tree_keys;  // the prefix pass takes the tree keys (bf16; fp32: the combine)
  // bf16
  int32_t nt;         // row tiles (lanes)
  int32_t S;          // 16-row strips per (sequence, kv head)
  int32_t tstrips;    // strips of the largest tile
  int32_t gl;         // blocks per lane
  int32_t grid;       // blocks launched (nt gl)
  int32_t xpair;      // the lanes' blocks of one index share an XCD
  int32_t split;      // 5- and 6-strip tiles split strips 4, 5 by key halves
  size_t lds_dyn;     // dynamic LDS bytes of the prefix kernel
  size_t rec_off;     // int4 [nt][gl] merge records
  // fp32
  int32_t spw;        // 16-row strips per wave
  int32_t tile_rows;  // query rows per block
  int32_t row_tiles;  // ceil(R / tile_rows)
  int32_t chunks;     // prefix chunks per (sequence, kv head)
  // both: partials (bf16 path: bf16 O [nt][2 gl][tstrips*16][128] and
  // float2 (m, l) [nt][2 gl][tstrips*16]; fp32 path: fp32 O
  // [B*Hkv][chunks][row_tiles*tile_rows][128] and (m, l) likewise)
  size_t o_off;
  size_t ml_off;
  size_t end;
};
constexpr int kMaxAttnSeq = 2048;     // sequences of one bf16 attention call
AttnPlan plan_attn(int32_t T, int32_t B, int32_t Hq, int32_t Hkv, int64_t cap, int is_bf16);

// ---------------------------------------------------------------- launchers
// Paged prefix cache: a pool [num_pages][Hkv][page_size][d] per layer and a
// block table [B][max_pages] of page ids (position p of sequence b is row
// p % page_size of page table[b][p / page_size]).
struct PagedArgs {
  const int32_t* table;
  int32_t max_pages;
  int32_t page_size;       // a power of two, at least 64
  int32_t ps_log2;
  int64_t num_pages;
};

enum TailMode : int32_t { TAIL_NONE = 0, TAIL_UPDATE = 1, TAIL_STEP = 2 };

enum UpdateMode : int32_t { UPDATE_ALL = 0, UPDATE_ACCEPTED = 1 };

struct TailArgs {
  int32_t mode;
  int32_t m_is64;
  int32_t update_mode;     // UpdateMode (TAIL_STEP only)
  int32_t sample;          // verify by sampling (TAIL_STEP only)
  float temp_scale;        // log2(e) / temperature
  const float* uniforms;   // [B][T][2]
  void* M;                 // [B][V][k]
  int32_t* tree_tok;       // [B][T]
  int32_t* root_tok;       // [B]
  int32_t* accept_len;     // [B]
  int32_t* accept_path;    // [B][D+1] or null
  int32_t* emitted;        // [B][D+1] or null
  // commit
  const uint8_t* k_tree;   // [B][T][Hkv][d] bytes
  const uint8_t* v_tree;
  uint8_t* k_cache;        // [B][Hkv][cap][d] or null
  uint8_t* v_cache;
  int32_t* prefix_len;
  int64_t cap;
  int32_t Hkv;
  int32_t row_bytes;       // d * element size
  // paged cache (k_cache/v_cache are then the pools of layer 0)
  PagedArgs paged;         // paged.table null: contiguous [B][Hkv][cap][d]
  int32_t n_layers;        // layers committed (1 for the contiguous cache)
  int64_t tree_layer_bytes;   // stride between layers of k_tree/v_tree
  int64_t cache_layer_bytes;  // stride between layers' pools
};

// Profiling hooks around each launch (no-ops unless tr_profile_enable).
void prof_begin(hipStream_t s, int32_t kernel_id);
void prof_end(hipStream_t s);

hipError_t launch_topk(const TreeDev& tree, int32_t B, const void* logits, int l_is_bf16, int64_t V,
                       int32_t k, int32_t* topk_ids, const TailArgs& tail, uint8_t* ws,
                       const TopkPlan& plan, hipStream_t s);
// The greedy step for few rows: one block per logit row, one tail block per
// sequence, `commit` commit blocks per sequence (0 without a cache), then
// M-prefetch helpers on each tail block's XCD.
constexpr int kMaxStepSeq = 256;
constexpr int64_t kStepMaxV = 32768;
struct StepPlan {
  bool use;
  int32_t rows, B, commit;
  int32_t helpers, help_base;   // M-prefetch helper blocks per sequence, first helper-region block
  int32_t grid;
};
StepPlan plan_step(int32_t B, const TreeDev& tree, int64_t V, int32_t k, int32_t esz, bool sample,
                   const TailArgs& tail);
hipError_t launch_step(const TreeDev& tree, const void* logits, int l_is_bf16, int64_t V,
                       int32_t k, int32_t* topk_ids, const TailArgs& tail, uint8_t* ws,
                       const StepPlan& plan, hipStream_t s);
// The few-row step on the LM head's slice lists (k <= 8) instead of logits.
hipError_t launch_step_lmhead(const TreeDev& tree, const uint64_t* part, int64_t V, int32_t k,
                              int32_t* topk_ids, const TailArgs& tail, uint8_t* ws,
                              const StepPlan& plan, hipStream_t s);
// Fused LM head + top-k: slices of 128 vocabulary rows, 8 keys per (row,
// slice), then one merge block per row.
struct LmheadPlan {
  int32_t nvs;        // vocabulary slices
  size_t part_off;    // uint64 [rows][nvs][8]
  size_t ids_off;     // int32 [rows][k] when the caller gives no buffer
  size_t end;
};
inline LmheadPlan plan_lmhead(int64_t rows, int64_t V, int32_t k) {
  LmheadPlan p{};
  p.nvs = int32_t((V + 127) / 128);
  p.part_off = kDataOff;
  p.ids_off = align256(p.part_off + size_t(rows) * p.nvs * 8 * 8);
  p.end = align256(p.ids_off + size_t(rows) * k * 4);
  return p;
}
hipError_t launch_lmhead(const void* h, const void* W, int32_t R, int32_t H, int64_t V,
                         uint64_t* part, int32_t nvs, hipStream_t s);
hipError_t launch_lmhead_merge(const TreeDev& tree, int64_t rows, const uint64_t* part, int32_t nvs,
                               int64_t V, int32_t k, int32_t* ids, const TailArgs& tail,
                               uint8_t* ws, hipStream_t s);
hipError_t launch_retrieve(const TreeDev& tree, int32_t B, const void* M, int m_is64, int64_t V,
                           int32_t k, const int32_t* root_tok, int32_t* tree_tok, uint8_t* ws,
                           hipStream_t s);
hipError_t launch_verify(const TreeDev& tree, int32_t B, const int32_t* topk, int32_t k,
                         const int32_t* tree_tok, int32_t* accept_len, int32_t* accept_path,
                         int32_t* bonus, int32_t* emitted, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
enum InitMode : int32_t { INIT_ZERO = 0, INIT_RANDOM = 1, INIT_PRIOR = 2 };
hipError_t launch_init_m(int mode, void* M, int m_is64, int32_t B, int64_t V, int32_t k,
                         const void* prior, int prior_is64, int prior_bcast, uint64_t seed,
                         hipStream_t s);
// ws: the scratch of the call (partials at the plan's offsets); flags: where
// the kernels raise sticky TR_FLAG_* bits (null: the status word of ws).
hipError_t launch_attn(const TreeDev& tree, int32_t B, int32_t Hq, int32_t Hkv, int is_bf16,
                       const void* q, const void* k_tree, const void* v_tree, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* prefix_len, float scale,
                       void* out, uint8_t* ws, const AttnPlan& plan, hipStream_t s,
                       const PagedArgs* paged = nullptr, uint8_t* flags = nullptr);

// Host-side helpers of the entry points (api.cpp): every check of a
// tr_tree_attn call except its workspace, and the plan; the last-error
// text of a status.
tr_status attn_prepare(const tr_tree* t, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, tr_dtype dt,
                       const void* q, const void* k_tree, const void* v_tree, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* prefix_len, float scale,
                       const void* out, AttnPlan* plan);
tr_status set_error(tr_status s, const char* what);
tr_status hip_error(hipError_t e, const char* what);

}  // namespace tr
