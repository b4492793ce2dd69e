// extern "C" entry points of libtr: argument checks on the host, then the
// kernel launches.  No call here allocates device memory.
#include <cmath>
#include <cstdlib>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "tr_internal.h"

namespace tr {

// Launch timing for tr_profile_*: a pool of event pairs, one per launch.
namespace {
constexpr int kProfMax = 16384;
struct ProfState {
  bool on = false;
  std::vector<hipEvent_t> ev;        // 2 per record, created when enabled
  std::vector<int32_t> id;
  int n = 0;                         // records since the last read
  int open = -1;                     // record begun, not ended
};
ProfState g_prof;
}  // namespace

void prof_begin(hipStream_t s, int32_t kernel_id) {
  g_prof.open = -1;
  if (!g_prof.on || g_prof.n >= kProfMax || size_t(2 * g_prof.n + 1) >= g_prof.ev.size()) return;
  const int i = g_prof.n;
  if (hipEventRecord(g_prof.ev[2 * i], s) != hipSuccess) return;
  g_prof.id[i] = kernel_id;
  g_prof.open = i;
}

void prof_end(hipStream_t s) {
  if (g_prof.open < 0) return;
  if (hipEventRecord(g_prof.ev[2 * g_prof.open + 1], s) == hipSuccess) ++g_prof.n;
  g_prof.open = -1;
}

}  // namespace tr

namespace {

thread_local char g_err[512];

tr_status fail(tr_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

tr_status ok() {
  g_err[0] = 0;
  return TR_OK;
}

tr_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define TR_CHECK(cond, status, ...) \
  do {                              \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

tr_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  TR_CHECK(ws != nullptr, TR_ERR_INVALID_ARGUMENT, "workspace is null");
  TR_CHECK((reinterpret_cast<uintptr_t>(ws) & 255) == 0, TR_ERR_INVALID_ARGUMENT,
           "workspace must be 256-byte aligned");
  TR_CHECK(ws_bytes >= need, TR_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
           ws_bytes, need);
  return TR_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Builds the template from parent/rank and checks it: root first, parents
// before children, distinct ranks below k under one parent, layer order.
tr_status build_tree(int32_t n, const int32_t* parent, const int32_t* rank, int32_t k,
                     tr_tree** out) {
  TR_CHECK(out != nullptr, TR_ERR_INVALID_ARGUMENT, "out is null");
  *out = nullptr;
  TR_CHECK(parent && rank, TR_ERR_INVALID_ARGUMENT, "parent/rank is null");
  TR_CHECK(n >= 1 && n <= tr::kMaxNodes, TR_ERR_INVALID_ARGUMENT, "n_nodes %d outside 1..%d", n,
           tr::kMaxNodes);
  TR_CHECK(k >= 1 && k <= tr::kMaxK, TR_ERR_INVALID_ARGUMENT, "k %d outside 1..%d", k, tr::kMaxK);
  TR_CHECK(parent[0] == -1 && rank[0] == -1, TR_ERR_INVALID_TREE,
           "node 0 must be the root (parent -1, rank -1)");
  tr_tree* t = new (std::nothrow) tr_tree();
  TR_CHECK(t != nullptr, TR_ERR_INVALID_ARGUMENT, "out of host memory");
  t->k = k;
  t->dev.T = n;
  t->dev.D = 0;
  t->dev.parent[0] = 0xFF;
  t->dev.rank[0] = 0xFF;
  t->dev.depth[0] = 0;
  std::memset(t->dev.anc, 0, sizeof t->dev.anc);
  t->dev.anc[0][0] = 1;
  std::vector<uint32_t> used(size_t(n), 0);   // rank bitmask per parent
  int prev_d = 0, prev_p = -1, prev_r = -1;
  for (int i = 1; i < n; ++i) {
    const int p = parent[i], r = rank[i];
    if (p < 0 || p >= i) { delete t; return fail(TR_ERR_INVALID_TREE, "node %d: parent %d must precede it", i, p); }
    if (r < 0 || r >= k) { delete t; return fail(TR_ERR_INVALID_TREE, "node %d: rank %d outside 0..k-1", i, r); }
    if (used[p] & (1u << r)) { delete t; return fail(TR_ERR_INVALID_TREE, "node %d: rank %d repeated under parent %d", i, r, p); }
    used[p] |= 1u << r;
    const int d = t->dev.depth[p] + 1;
    const bool in_order = d > prev_d || (d == prev_d && (p > prev_p || (p == prev_p && r > prev_r)));
    if (!in_order) { delete t; return fail(TR_ERR_INVALID_TREE, "node %d breaks layer order (depth, parent, rank)", i); }
    prev_d = d; prev_p = p; prev_r = r;
    t->dev.parent[i] = uint8_t(p);
    t->dev.rank[i] = uint8_t(r);
    t->dev.depth[i] = uint8_t(d);
    if (d > t->dev.D) t->dev.D = d;
    t->dev.anc[i][0] = t->dev.anc[p][0];
    t->dev.anc[i][1] = t->dev.anc[p][1];
    t->dev.anc[i][i >> 6] |= uint64_t(1) << (i & 63);
  }
  for (int i = n; i < tr::kMaxNodes; ++i) {
    t->dev.parent[i] = 0xFF;
    t->dev.rank[i] = 0xFF;
    t->dev.depth[i] = 0xFF;
  }
  *out = t;
  return ok();
}

// Limits of the bf16 attention pass: every block scans the sequences'
// prefix lengths in LDS, and the flat sub-block count fits 32 bits.
tr_status check_bf16_attn(const tr_tree* t, int32_t B, int32_t Hkv, int64_t cap) {
  TR_CHECK(B <= tr::kMaxAttnSeq, TR_ERR_UNSUPPORTED, "bf16 attention takes B <= %d", tr::kMaxAttnSeq);
  const int64_t per_seq = (cap + 63) / 64 + (t->dev.T + 63) / 64;
  TR_CHECK(int64_t(B) * per_seq * Hkv <= INT32_MAX, TR_ERR_UNSUPPORTED,
           "B x Hkv x 64-key blocks of the cache above 2^31-1");
  return TR_OK;
}

size_t topk_need(const tr_tree* t, int32_t B, int64_t V, int32_t k) {
  const int64_t rows = int64_t(B) * t->dev.T;
  const size_t a = tr::plan_topk(rows, V, k, 2).end, b = tr::plan_topk(rows, V, k, 4).end;
  return a > b ? a : b;
}

}  // namespace

namespace tr {

tr_status set_error(tr_status s, const char* what) { return fail(s, "%s", what); }

tr_status hip_error(hipError_t e, const char* what) { return hip_status(e, what); }

tr_status attn_prepare(const tr_tree* t, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, tr_dtype dt,
                       const void* q, const void* k_tree, const void* v_tree, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* prefix_len, float scale,
                       const void* out, AttnPlan* plan) {
  TR_CHECK(t != nullptr, TR_ERR_INVALID_ARGUMENT, "tree is null");
  TR_CHECK(B >= 1, TR_ERR_INVALID_ARGUMENT, "B must be >= 1");
  TR_CHECK(q && k_tree && v_tree && k_cache && v_cache && prefix_len && out,
           TR_ERR_INVALID_ARGUMENT, "null tensor");
  TR_CHECK(dt == TR_FLOAT32 || dt == TR_BFLOAT16, TR_ERR_UNSUPPORTED, "attention dtype must be float32 or bfloat16");
  TR_CHECK(d == kHeadDim, TR_ERR_UNSUPPORTED, "head dimension must be %d", kHeadDim);
  TR_CHECK(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, TR_ERR_INVALID_ARGUMENT,
           "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  TR_CHECK(cap >= 0, TR_ERR_INVALID_ARGUMENT, "negative capacity");
  TR_CHECK(scale > 0.f && scale < 1e30f, TR_ERR_INVALID_ARGUMENT, "scale must be positive and finite");
  TR_CHECK(int64_t(B) * Hkv <= 65535, TR_ERR_UNSUPPORTED, "B*Hkv above 65535");
  TR_CHECK(aligned16(q) && aligned16(k_tree) && aligned16(v_tree) && aligned16(k_cache) &&
               aligned16(v_cache) && aligned16(out), TR_ERR_INVALID_ARGUMENT,
           "attention tensors must be 16-byte aligned");
  if (dt == TR_BFLOAT16) {
    tr_status st = check_bf16_attn(t, B, Hkv, cap);
    if (st != TR_OK) return st;
  }
  *plan = plan_attn(t->dev.T, B, Hq, Hkv, cap, dt == TR_BFLOAT16);
  return ok();
}

}  // namespace tr

extern "C" {

const char* tr_status_string(tr_status s) {
  switch (s) {
    case TR_OK: return "TR_OK";
    case TR_ERR_INVALID_ARGUMENT: return "TR_ERR_INVALID_ARGUMENT";
    case TR_ERR_UNSUPPORTED: return "TR_ERR_UNSUPPORTED";
    case TR_ERR_INVALID_TREE: return "TR_ERR_INVALID_TREE";
    case TR_ERR_WORKSPACE_TOO_SMALL: return "TR_ERR_WORKSPACE_TOO_SMALL";
    case TR_ERR_HIP: return "TR_ERR_HIP";
  }
  return "TR_UNKNOWN_STATUS";
}

const char* tr_last_error(void) { return g_err; }

tr_status tr_tree_create(int32_t n_nodes, const int32_t* parent, const int32_t* rank, int32_t k,
                         tr_tree** out) {
  return build_tree(n_nodes, parent, rank, k, out);
}

tr_status tr_tree_create_levels(int32_t n_levels, const int32_t* level_len, const int32_t* counts,
                                int32_t k, tr_tree** out) {
  TR_CHECK(out != nullptr, TR_ERR_INVALID_ARGUMENT, "out is null");
  *out = nullptr;
  TR_CHECK(n_levels >= 0 && (n_levels == 0 || (level_len && counts)), TR_ERR_INVALID_ARGUMENT,
           "level arrays are null");
  std::vector<int32_t> parent{-1}, rank{-1}, layer{0};
  size_t pos = 0;
  for (int l = 0; l < n_levels; ++l) {
    TR_CHECK(level_len[l] >= 0 && size_t(level_len[l]) <= layer.size(), TR_ERR_INVALID_TREE,
             "layer %d lists %d counts for %zu nodes", l, level_len[l], layer.size());
    std::vector<int32_t> next;
    for (int i = 0; i < level_len[l]; ++i) {
      const int c = counts[pos++];
      TR_CHECK(c >= 0 && c <= k, TR_ERR_INVALID_TREE, "layer %d node %d: %d children, k = %d", l, i, c, k);
      for (int r = 0; r < c; ++r) {
        parent.push_back(layer[size_t(i)]);
        rank.push_back(r);
        next.push_back(int32_t(parent.size()) - 1);
        TR_CHECK(parent.size() <= size_t(tr::kMaxNodes), TR_ERR_INVALID_ARGUMENT,
                 "more than %d nodes", tr::kMaxNodes);
      }
    }
    layer.swap(next);
  }
  return build_tree(int32_t(parent.size()), parent.data(), rank.data(), k, out);
}

void tr_tree_destroy(tr_tree* t) { delete t; }

tr_status tr_tree_info(const tr_tree* t, int32_t* n_nodes, int32_t* depth, int32_t* k,
                       int32_t* parent_out, int32_t* rank_out, int32_t* depth_out,
                       uint64_t* anc_out) {
  TR_CHECK(t != nullptr, TR_ERR_INVALID_ARGUMENT, "tree is null");
  if (n_nodes) *n_nodes = t->dev.T;
  if (depth) *depth = t->dev.D;
  if (k) *k = t->k;
  for (int i = 0; i < t->dev.T; ++i) {
    if (parent_out) parent_out[i] = i ? t->dev.parent[i] : -1;
    if (rank_out) rank_out[i] = i ? t->dev.rank[i] : -1;
    if (depth_out) depth_out[i] = t->dev.depth[i];
    if (anc_out) {
      anc_out[2 * i] = t->dev.anc[i][0];
      anc_out[2 * i + 1] = t->dev.anc[i][1];
    }
  }
  return ok();
}

size_t tr_workspace_size(const tr_tree* t, int32_t B, int64_t V, int32_t k, int32_t Hq,
                         int32_t Hkv, int32_t d, int64_t cap) {
  if (!t || B < 1) return 0;
  size_t need = tr::kDataOff;
  if (V >= 1 && k >= 1) {
    size_t a = topk_need(t, B, V, k);
    if (a > need) need = a;
  }
  if (Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && d == tr::kHeadDim && cap >= 0) {
    for (int bf = 0; bf < 2; ++bf) {
      size_t a = tr::plan_attn(t->dev.T, B, Hq, Hkv, cap, bf).end;
      if (a > need) need = a;
    }
  }
  return need;
}

tr_status tr_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  tr_status st = check_ws(ws, ws_bytes, tr::kDataOff);
  if (st != TR_OK) return st;
  TR_CHECK(ws_bytes % 16 == 0, TR_ERR_INVALID_ARGUMENT, "workspace size must be a multiple of 16");
  return hip_status(tr::launch_fill_zero(ws, ws_bytes, hipStream_t(stream)), "tr_workspace_init");
}

tr_status tr_read_device_status(void* ws, uint32_t* flags, void* stream) {
  TR_CHECK(ws && flags, TR_ERR_INVALID_ARGUMENT, "null argument");
  hipStream_t s = hipStream_t(stream);
  hipError_t e = hipMemcpyAsync(flags, ws, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && *flags) {
    e = tr::launch_fill_zero(ws, 16, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
  }
  return hip_status(e, "tr_read_device_status");
}

tr_status tr_retrieve(const tr_tree* t, int32_t B, const void* M, tr_dtype m_dtype, int64_t V,
                      int32_t k, const int32_t* root_tok, int32_t* tree_tok, void* ws,
                      size_t ws_bytes, void* stream) {
  TR_CHECK(t != nullptr, TR_ERR_INVALID_ARGUMENT, "tree is null");
  TR_CHECK(B >= 1, TR_ERR_INVALID_ARGUMENT, "B must be >= 1");
  TR_CHECK(M && root_tok && tree_tok, TR_ERR_INVALID_ARGUMENT, "null tensor");
  TR_CHECK(m_dtype == TR_INT32 || m_dtype == TR_INT64, TR_ERR_UNSUPPORTED, "M must be int32 or int64");
  TR_CHECK(k == t->k, TR_ERR_INVALID_ARGUMENT, "k %d differs from the tree's %d", k, t->k);
  TR_CHECK(V >= 1 && V <= INT32_MAX, TR_ERR_INVALID_ARGUMENT, "V outside 1..2^31-1");
  tr_status st = check_ws(ws, ws_bytes, tr::kDataOff);
  if (st != TR_OK) return st;
  return hip_status(tr::launch_retrieve(t->dev, B, M, m_dtype == TR_INT64, V, k, root_tok, tree_tok,
                                        static_cast<uint8_t*>(ws), hipStream_t(stream)),
                    "tr_retrieve");
}

tr_status tr_tree_attn(const tr_tree* t, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, tr_dtype dt,
                       const void* q, const void* k_tree, const void* v_tree, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* prefix_len, float scale,
                       void* out, void* ws, size_t ws_bytes, void* stream) {
  tr::AttnPlan plan;
  tr_status st = tr::attn_prepare(t, B, Hq, Hkv, d, dt, q, k_tree, v_tree, k_cache, v_cache, cap,
                                  prefix_len, scale, out, &plan);
  if (st != TR_OK) return st;
  st = check_ws(ws, ws_bytes, plan.end);
  if (st != TR_OK) return st;
  return hip_status(tr::launch_attn(t->dev, B, Hq, Hkv, dt == TR_BFLOAT16, q, k_tree, v_tree, k_cache,
                                    v_cache, cap, prefix_len, scale, out, static_cast<uint8_t*>(ws),
                                    plan, hipStream_t(stream)),
                    "tr_tree_attn");
}

// A row longer than the plan's segments can hold in registers is refused
// (the scan would otherwise leave its tail unread).
// The few-row greedy step kernel (k_step.hip) is used where it applies
// unless the environment sets TR_FEW_ROW_STEP=0 (a diagnostic switch: the
// general kernel computes the same results).
static bool few_row_step_enabled() {
  const char* v = std::getenv("TR_FEW_ROW_STEP");
  return !(v && v[0] == '0' && v[1] == 0);
}

static tr_status check_topk_len(const tr::TopkPlan& plan, int64_t V) {
  TR_CHECK(plan.seg_len <= plan.seg_cap, TR_ERR_UNSUPPORTED,
           "V = %lld above the top-k limit of %lld for this logit dtype and k",
           (long long)V, (long long)plan.max_v);
  return TR_OK;
}

static tr_status check_topk_args(const tr_tree* t, int32_t B, const void* logits, tr_dtype l_dtype,
                                 int64_t V, int32_t k) {
  TR_CHECK(t != nullptr, TR_ERR_INVALID_ARGUMENT, "tree is null");
  TR_CHECK(B >= 1, TR_ERR_INVALID_ARGUMENT, "B must be >= 1");
  TR_CHECK(logits != nullptr, TR_ERR_INVALID_ARGUMENT, "logits is null");
  TR_CHECK(l_dtype == TR_FLOAT32 || l_dtype == TR_BFLOAT16, TR_ERR_UNSUPPORTED,
           "logits must be float32 or bfloat16");
  TR_CHECK(k == t->k, TR_ERR_INVALID_ARGUMENT, "k %d differs from the tree's %d", k, t->k);
  TR_CHECK(V >= k && V <= INT32_MAX, TR_ERR_INVALID_ARGUMENT, "V must be in k..2^31-1");
  TR_CHECK(int64_t(B) * t->dev.T <= int64_t(tr::kMaxRowCnt), TR_ERR_UNSUPPORTED,
           "B * nodes above %zu", tr::kMaxRowCnt);
  TR_CHECK(size_t(B) <= tr::kMaxSeqCnt, TR_ERR_UNSUPPORTED, "B above %zu", tr::kMaxSeqCnt);
  const uintptr_t esz = l_dtype == TR_BFLOAT16 ? 2 : 4;
  TR_CHECK((reinterpret_cast<uintptr_t>(logits) & (esz - 1)) == 0, TR_ERR_INVALID_ARGUMENT,
           "logits must be aligned to their element size");
  return TR_OK;
}

tr_status tr_update_topk(const tr_tree* t, int32_t B, const void* logits, tr_dtype l_dtype,
                         int64_t V, int32_t k, const int32_t* tree_tok, void* M, tr_dtype m_dtype,
                         int32_t* topk_out, void* ws, size_t ws_bytes, void* stream) {
  tr_status st = check_topk_args(t, B, logits, l_dtype, V, k);
  if (st != TR_OK) return st;
  TR_CHECK(M || topk_out, TR_ERR_INVALID_ARGUMENT, "nothing to write: M and topk_out are null");
  if (M) {
    TR_CHECK(tree_tok != nullptr, TR_ERR_INVALID_ARGUMENT, "tree_tok is null");
    TR_CHECK(m_dtype == TR_INT32 || m_dtype == TR_INT64, TR_ERR_UNSUPPORTED, "M must be int32 or int64");
  }
  const tr::TopkPlan plan = tr::plan_topk(int64_t(B) * t->dev.T, V, k, l_dtype == TR_BFLOAT16 ? 2 : 4);
  st = check_topk_len(plan, V);
  if (st != TR_OK) return st;
  st = check_ws(ws, ws_bytes, plan.end);
  if (st != TR_OK) return st;
  uint8_t* w = static_cast<uint8_t*>(ws);
  int32_t* ids = topk_out ? topk_out : reinterpret_cast<int32_t*>(w + plan.ids_off);
  tr::TailArgs tail{};
  tail.mode = M ? tr::TAIL_UPDATE : tr::TAIL_NONE;
  tail.m_is64 = m_dtype == TR_INT64;
  tail.M = M;
  tail.tree_tok = const_cast<int32_t*>(tree_tok);
  if (M && few_row_step_enabled()) {
    const tr::StepPlan sp = tr::plan_step(B, t->dev, V, k, l_dtype == TR_BFLOAT16 ? 2 : 4, false, tail);
    if (sp.use)
      return hip_status(tr::launch_step(t->dev, logits, l_dtype == TR_BFLOAT16, V, k, ids, tail, w,
                                        sp, hipStream_t(stream)),
                        "tr_update_topk");
  }
  return hip_status(tr::launch_topk(t->dev, B, logits, l_dtype == TR_BFLOAT16, V, k, ids, tail, w,
                                    plan, hipStream_t(stream)),
                    "tr_update_topk");
}

tr_status tr_verify(const tr_tree* t, int32_t B, const int32_t* topk, int32_t k,
                    const int32_t* tree_tok, int32_t* accept_len, int32_t* accept_path,
                    int32_t* bonus, int32_t* emitted, void* stream) {
  TR_CHECK(t != nullptr, TR_ERR_INVALID_ARGUMENT, "tree is null");
  TR_CHECK(B >= 1, TR_ERR_INVALID_ARGUMENT, "B must be >= 1");
  TR_CHECK(topk && tree_tok && accept_len && bonus, TR_ERR_INVALID_ARGUMENT, "null tensor");
  TR_CHECK(k == t->k, TR_ERR_INVALID_ARGUMENT, "k %d differs from the tree's %d", k, t->k);
  return hip_status(tr::launch_verify(t->dev, B, topk, k, tree_tok, accept_len, accept_path, bonus,
                                      emitted, hipStream_t(stream)),
                    "tr_verify");
}

namespace {

// LM-head input of the fused step: hidden states h [rows][H] and the output
// embedding W [V][H], bfloat16.
struct LmSrc {
  const void* h;
  const void* W;
  int32_t H;
};

tr_status check_lmhead_args(int64_t rows, int32_t H, int64_t V, int32_t k, const void* h,
                            const void* W, tr_dtype dtype) {
  TR_CHECK(rows >= 1, TR_ERR_INVALID_ARGUMENT, "rows must be >= 1");
  TR_CHECK(rows <= int64_t(tr::kMaxRowCnt), TR_ERR_UNSUPPORTED, "rows above %zu", tr::kMaxRowCnt);
  TR_CHECK(h && W, TR_ERR_INVALID_ARGUMENT, "h or W is null");
  TR_CHECK(dtype == TR_BFLOAT16, TR_ERR_UNSUPPORTED, "the LM head takes bfloat16 h and W");
  TR_CHECK(H >= 128 && H % 128 == 0, TR_ERR_UNSUPPORTED, "H must be a positive multiple of 128");
  TR_CHECK(k >= 1 && k <= 8, TR_ERR_UNSUPPORTED, "the fused LM head keeps k <= 8");
  TR_CHECK(V >= k && V <= INT32_MAX, TR_ERR_INVALID_ARGUMENT, "V must be in k..2^31-1");
  TR_CHECK(aligned16(h) && aligned16(W), TR_ERR_INVALID_ARGUMENT, "h and W must be 16-byte aligned");
  return TR_OK;
}

// The fused step; temperature 0 verifies greedily, above 0 by sampling.
tr_status step_impl(const tr_tree* t, int32_t B, int64_t V, int32_t k, const void* logits,
                    tr_dtype l_dtype, float temperature, const float* uniforms, void* M,
                    tr_dtype m_dtype, int32_t* tree_tok, int32_t* root_tok, int32_t* accept_len,
                    int32_t* accept_path, int32_t* emitted, int32_t Hkv, int32_t d,
                    tr_dtype kv_dtype, const void* k_tree, const void* v_tree, void* k_cache,
                    void* v_cache, int64_t cap, int32_t* prefix_len, int32_t* topk_out,
                    tr_update_mode mode, void* ws, size_t ws_bytes, void* stream,
                    const tr::PagedArgs* paged = nullptr, int32_t n_layers = 1,
                    int64_t tree_layer_bytes = 0, int64_t cache_layer_bytes = 0,
                    const LmSrc* lm = nullptr) {
  TR_CHECK(mode == TR_UPDATE_ALL || mode == TR_UPDATE_ACCEPTED, TR_ERR_INVALID_ARGUMENT,
           "unknown update mode %d", int(mode));
  const bool sample = temperature != 0.f;
  if (sample) {
    TR_CHECK(temperature > 0.f && std::isfinite(temperature), TR_ERR_INVALID_ARGUMENT,
             "temperature must be positive and finite");
    TR_CHECK(uniforms != nullptr, TR_ERR_INVALID_ARGUMENT, "uniforms is null");
    TR_CHECK(V <= int64_t(tr::kMaxBuckets) * tr::kDrawBucket, TR_ERR_UNSUPPORTED,
             "sampling takes V <= %d", tr::kMaxBuckets * tr::kDrawBucket);
  }
  tr_status st = lm ? check_lmhead_args(int64_t(B) * (t ? t->dev.T : 0), lm->H, V, k, lm->h, lm->W,
                                         l_dtype)
                    : check_topk_args(t, B, logits, l_dtype, V, k);
  if (st != TR_OK) return st;
  if (lm) {
    TR_CHECK(t != nullptr, TR_ERR_INVALID_ARGUMENT, "tree is null");
    TR_CHECK(k == t->k, TR_ERR_INVALID_ARGUMENT, "k %d differs from the tree's %d", k, t->k);
    TR_CHECK(size_t(B) <= tr::kMaxSeqCnt, TR_ERR_UNSUPPORTED, "B above %zu", tr::kMaxSeqCnt);
  }
  TR_CHECK(M && tree_tok && root_tok && accept_len, TR_ERR_INVALID_ARGUMENT, "null tensor");
  TR_CHECK(m_dtype == TR_INT32 || m_dtype == TR_INT64, TR_ERR_UNSUPPORTED, "M must be int32 or int64");
  int row_bytes = 0;
  if (k_cache) {
    TR_CHECK(v_cache && k_tree && v_tree && prefix_len, TR_ERR_INVALID_ARGUMENT,
             "commit needs k_tree, v_tree, v_cache and prefix_len");
    TR_CHECK(kv_dtype == TR_FLOAT32 || kv_dtype == TR_BFLOAT16, TR_ERR_UNSUPPORTED,
             "key/value dtype must be float32 or bfloat16");
    TR_CHECK(d == tr::kHeadDim, TR_ERR_UNSUPPORTED, "head dimension must be %d", tr::kHeadDim);
    TR_CHECK(Hkv >= 1 && cap >= 0, TR_ERR_INVALID_ARGUMENT, "bad Hkv or cap");
    TR_CHECK(aligned16(k_cache) && aligned16(v_cache) && aligned16(k_tree) && aligned16(v_tree),
             TR_ERR_INVALID_ARGUMENT, "key/value tensors must be 16-byte aligned");
    row_bytes = d * (kv_dtype == TR_BFLOAT16 ? 2 : 4);
  }
  const int64_t rows = int64_t(B) * t->dev.T;
  const tr::TopkPlan plan = tr::plan_topk(rows, V, k, l_dtype == TR_BFLOAT16 ? 2 : 4);
  const tr::LmheadPlan lplan = tr::plan_lmhead(rows, V, k);
  if (!lm) {
    st = check_topk_len(plan, V);
    if (st != TR_OK) return st;
  }
  st = check_ws(ws, ws_bytes, lm ? lplan.end : plan.end);
  if (st != TR_OK) return st;
  uint8_t* w = static_cast<uint8_t*>(ws);
  int32_t* ids = topk_out ? topk_out
                          : reinterpret_cast<int32_t*>(w + (lm ? lplan.ids_off : plan.ids_off));
  tr::TailArgs tail{};
  tail.mode = tr::TAIL_STEP;
  tail.m_is64 = m_dtype == TR_INT64;
  tail.update_mode = mode == TR_UPDATE_ACCEPTED ? tr::UPDATE_ACCEPTED : tr::UPDATE_ALL;
  tail.sample = sample ? 1 : 0;
  tail.temp_scale = sample ? float(1.4426950408889634 / double(temperature)) : 0.f;
  tail.uniforms = uniforms;
  tail.M = M;
  tail.tree_tok = tree_tok;
  tail.root_tok = root_tok;
  tail.accept_len = accept_len;
  tail.accept_path = accept_path;
  tail.emitted = emitted;
  tail.k_tree = static_cast<const uint8_t*>(k_tree);
  tail.v_tree = static_cast<const uint8_t*>(v_tree);
  tail.k_cache = static_cast<uint8_t*>(k_cache);
  tail.v_cache = static_cast<uint8_t*>(v_cache);
  tail.prefix_len = prefix_len;
  tail.cap = cap;
  tail.Hkv = Hkv;
  tail.row_bytes = row_bytes;
  tail.n_layers = n_layers;
  tail.tree_layer_bytes = tree_layer_bytes;
  tail.cache_layer_bytes = cache_layer_bytes;
  if (paged) tail.paged = *paged;
  if (lm) {
    uint64_t* part = reinterpret_cast<uint64_t*>(w + lplan.part_off);
    hipError_t e = tr::launch_lmhead(lm->h, lm->W, int32_t(rows), lm->H, V, part, lplan.nvs,
                                     hipStream_t(stream));
    // few rows: the few-row step kernel merges the slice lists in its row
    // blocks; else one merge block per row, the tail in the last of each
    // sequence
    const tr::StepPlan sp = few_row_step_enabled() ? tr::plan_step(B, t->dev, V, k, 2, false, tail)
                                                   : tr::StepPlan{};
    if (e == hipSuccess && sp.use)
      e = tr::launch_step_lmhead(t->dev, part, V, k, ids, tail, w, sp, hipStream_t(stream));
    else if (e == hipSuccess)
      e = tr::launch_lmhead_merge(t->dev, rows, part, lplan.nvs, V, k, ids, tail, w,
                                  hipStream_t(stream));
    return hip_status(e, "tr_step_lmhead");
  }
  if (few_row_step_enabled()) {
    const tr::StepPlan sp = tr::plan_step(B, t->dev, V, k, l_dtype == TR_BFLOAT16 ? 2 : 4, sample, tail);
    if (sp.use)
      return hip_status(tr::launch_step(t->dev, logits, l_dtype == TR_BFLOAT16, V, k, ids, tail, w,
                                        sp, hipStream_t(stream)),
                        "tr_step");
  }
  return hip_status(tr::launch_topk(t->dev, B, logits, l_dtype == TR_BFLOAT16, V, k, ids, tail, w,
                                    plan, hipStream_t(stream)),
                    "tr_step");
}

}  // namespace

tr_status tr_step_ex(const tr_tree* t, int32_t B, int64_t V, int32_t k, const void* logits,
                     tr_dtype l_dtype, void* M, tr_dtype m_dtype, int32_t* tree_tok,
                     int32_t* root_tok, int32_t* accept_len, int32_t* accept_path,
                     int32_t* emitted, int32_t Hkv, int32_t d, tr_dtype kv_dtype,
                     const void* k_tree, const void* v_tree, void* k_cache, void* v_cache,
                     int64_t cap, int32_t* prefix_len, int32_t* topk_out, tr_update_mode mode,
                     void* ws, size_t ws_bytes, void* stream) {
  return step_impl(t, B, V, k, logits, l_dtype, 0.f, nullptr, M, m_dtype, tree_tok, root_tok,
                   accept_len, accept_path, emitted, Hkv, d, kv_dtype, k_tree, v_tree, k_cache,
                   v_cache, cap, prefix_len, topk_out, mode, ws, ws_bytes, stream);
}

tr_status tr_step_sample(const tr_tree* t, int32_t B, int64_t V, int32_t k, const void* logits,
                         tr_dtype l_dtype, float temperature, const float* uniforms, void* M,
                         tr_dtype m_dtype, int32_t* tree_tok, int32_t* root_tok,
                         int32_t* accept_len, int32_t* accept_path, int32_t* emitted, int32_t Hkv,
                         int32_t d, tr_dtype kv_dtype, const void* k_tree, const void* v_tree,
                         void* k_cache, void* v_cache, int64_t cap, int32_t* prefix_len,
                         int32_t* topk_out, tr_update_mode mode, void* ws, size_t ws_bytes,
                         void* stream) {
  TR_CHECK(temperature > 0.f && std::isfinite(temperature), TR_ERR_INVALID_ARGUMENT,
           "temperature must be positive and finite");
  return step_impl(t, B, V, k, logits, l_dtype, temperature, uniforms, M, m_dtype, tree_tok,
                   root_tok, accept_len, accept_path, emitted, Hkv, d, kv_dtype, k_tree, v_tree,
                   k_cache, v_cache, cap, prefix_len, topk_out, mode, ws, ws_bytes, stream);
}

// Checks a paged cache description; fills the kernels' view of it.
static tr_status check_paged(const tr_paged_kv* kv, int32_t B, tr::PagedArgs* pa) {
  TR_CHECK(kv != nullptr, TR_ERR_INVALID_ARGUMENT, "kv is null");
  TR_CHECK(kv->n_layers >= 1 && kv->Hkv >= 1, TR_ERR_INVALID_ARGUMENT, "bad n_layers or Hkv");
  TR_CHECK(kv->d == tr::kHeadDim, TR_ERR_UNSUPPORTED, "head dimension must be %d", tr::kHeadDim);
  TR_CHECK(kv->dtype == TR_BFLOAT16, TR_ERR_UNSUPPORTED, "paged caches hold bfloat16");
  TR_CHECK(kv->page_size >= 64 && (kv->page_size & (kv->page_size - 1)) == 0,
           TR_ERR_INVALID_ARGUMENT, "page_size must be a power of two >= 64");
  TR_CHECK(kv->num_pages >= 1 && kv->max_pages >= 1, TR_ERR_INVALID_ARGUMENT,
           "num_pages and max_pages must be >= 1");
  TR_CHECK(kv->block_table && kv->k_pages && kv->v_pages && kv->k_tree && kv->v_tree &&
               kv->prefix_len, TR_ERR_INVALID_ARGUMENT, "null tensor in kv");
  TR_CHECK(aligned16(kv->k_pages) && aligned16(kv->v_pages) && aligned16(kv->k_tree) &&
               aligned16(kv->v_tree), TR_ERR_INVALID_ARGUMENT, "kv tensors must be 16-byte aligned");
  (void)B;
  pa->table = kv->block_table;
  pa->max_pages = kv->max_pages;
  pa->page_size = kv->page_size;
  pa->ps_log2 = __builtin_ctz(uint32_t(kv->page_size));
  pa->num_pages = kv->num_pages;
  return TR_OK;
}

tr_status tr_tree_attn_paged(const tr_tree* t, int32_t B, int32_t Hq, const void* q,
                             const tr_paged_kv* kv, int32_t layer, float scale, void* out,
                             void* ws, size_t ws_bytes, void* stream) {
  tr::PagedArgs pa{};
  tr_status st = check_paged(kv, B, &pa);
  if (st != TR_OK) return st;
  TR_CHECK(t != nullptr, TR_ERR_INVALID_ARGUMENT, "tree is null");
  TR_CHECK(B >= 1, TR_ERR_INVALID_ARGUMENT, "B must be >= 1");
  TR_CHECK(layer >= 0 && layer < kv->n_layers, TR_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)",
           layer, kv->n_layers);
  TR_CHECK(q && out, TR_ERR_INVALID_ARGUMENT, "null tensor");
  const int32_t Hkv = kv->Hkv;
  TR_CHECK(Hq >= 1 && Hq % Hkv == 0, TR_ERR_INVALID_ARGUMENT,
           "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  TR_CHECK(scale > 0.f && scale < 1e30f, TR_ERR_INVALID_ARGUMENT, "scale must be positive and finite");
  TR_CHECK(int64_t(B) * Hkv <= 65535, TR_ERR_UNSUPPORTED, "B*Hkv above 65535");
  TR_CHECK(aligned16(q) && aligned16(out), TR_ERR_INVALID_ARGUMENT,
           "attention tensors must be 16-byte aligned");
  const int64_t cap = int64_t(kv->max_pages) * kv->page_size;
  st = check_bf16_attn(t, B, Hkv, cap);
  if (st != TR_OK) return st;
  const tr::AttnPlan plan = tr::plan_attn(t->dev.T, B, Hq, Hkv, cap, 1);
  st = check_ws(ws, ws_bytes, plan.end);
  if (st != TR_OK) return st;
  const size_t row = size_t(Hkv) * tr::kHeadDim * 2;
  const int64_t T = t->dev.T;
  const uint8_t* kt = static_cast<const uint8_t*>(kv->k_tree) + layer * int64_t(B) * T * row;
  const uint8_t* vt = static_cast<const uint8_t*>(kv->v_tree) + layer * int64_t(B) * T * row;
  const int64_t pool = kv->num_pages * kv->page_size * int64_t(row);
  const uint8_t* kp = static_cast<const uint8_t*>(kv->k_pages) + layer * pool;
  const uint8_t* vp = static_cast<const uint8_t*>(kv->v_pages) + layer * pool;
  return hip_status(tr::launch_attn(t->dev, B, Hq, Hkv, 1, q, kt, vt, kp, vp, cap, kv->prefix_len,
                                    scale, out, static_cast<uint8_t*>(ws), plan,
                                    hipStream_t(stream), &pa),
                    "tr_tree_attn_paged");
}

tr_status tr_step_paged(const tr_tree* t, int32_t B, int64_t V, int32_t k, const void* logits,
                        tr_dtype l_dtype, void* M, tr_dtype m_dtype, int32_t* tree_tok,
                        int32_t* root_tok, int32_t* accept_len, int32_t* accept_path,
                        int32_t* emitted, const tr_paged_kv* kv, int32_t* topk_out,
                        tr_update_mode mode, void* ws, size_t ws_bytes, void* stream) {
  tr::PagedArgs pa{};
  tr_status st = check_paged(kv, B, &pa);
  if (st != TR_OK) return st;
  TR_CHECK(t != nullptr, TR_ERR_INVALID_ARGUMENT, "tree is null");
  const int64_t row = int64_t(kv->Hkv) * tr::kHeadDim * 2;
  const int64_t cap = int64_t(kv->max_pages) * kv->page_size;
  return step_impl(t, B, V, k, logits, l_dtype, 0.f, nullptr, M, m_dtype, tree_tok, root_tok,
                   accept_len, accept_path, emitted, kv->Hkv, kv->d, kv->dtype, kv->k_tree,
                   kv->v_tree, kv->k_pages, kv->v_pages, cap, kv->prefix_len, topk_out, mode, ws,
                   ws_bytes, stream, &pa, kv->n_layers, int64_t(B) * t->dev.T * row,
                   kv->num_pages * kv->page_size * row);
}

size_t tr_lmhead_workspace_size(int64_t rows, int64_t V, int32_t k) {
  if (rows < 1 || V < 1 || k < 1) return 0;
  return tr::plan_lmhead(rows, V, k).end;
}

tr_status tr_lmhead_topk(int32_t rows, int32_t H, int64_t V, int32_t k, const void* h,
                         const void* W, tr_dtype dtype, int32_t* topk_out, void* ws,
                         size_t ws_bytes, void* stream) {
  tr_status st = check_lmhead_args(rows, H, V, k, h, W, dtype);
  if (st != TR_OK) return st;
  TR_CHECK(topk_out != nullptr, TR_ERR_INVALID_ARGUMENT, "topk_out is null");
  const tr::LmheadPlan plan = tr::plan_lmhead(rows, V, k);
  st = check_ws(ws, ws_bytes, plan.end);
  if (st != TR_OK) return st;
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint64_t* part = reinterpret_cast<uint64_t*>(w + plan.part_off);
  hipError_t e = tr::launch_lmhead(h, W, rows, H, V, part, plan.nvs, hipStream_t(stream));
  if (e == hipSuccess) {
    tr::TreeDev none{};
    none.T = 1;
    tr::TailArgs tail{};
    tail.mode = tr::TAIL_NONE;
    e = tr::launch_lmhead_merge(none, rows, part, plan.nvs, V, k, topk_out, tail, w,
                                hipStream_t(stream));
  }
  return hip_status(e, "tr_lmhead_topk");
}

tr_status tr_step_lmhead(const tr_tree* t, int32_t B, int32_t H, int64_t V, int32_t k,
                         const void* h, const void* W, tr_dtype dtype, void* M, tr_dtype m_dtype,
                         int32_t* tree_tok, int32_t* root_tok, int32_t* accept_len,
                         int32_t* accept_path, int32_t* emitted, int32_t Hkv, int32_t d,
                         tr_dtype kv_dtype, const void* k_tree, const void* v_tree, void* k_cache,
                         void* v_cache, int64_t cap, int32_t* prefix_len, int32_t* topk_out,
                         tr_update_mode mode, void* ws, size_t ws_bytes, void* stream) {
  TR_CHECK(t != nullptr && B >= 1, TR_ERR_INVALID_ARGUMENT, "tree is null or B < 1");
  const LmSrc lm{h, W, H};
  return step_impl(t, B, V, k, nullptr, dtype, 0.f, nullptr, M, m_dtype, tree_tok, root_tok,
                   accept_len, accept_path, emitted, Hkv, d, kv_dtype, k_tree, v_tree, k_cache,
                   v_cache, cap, prefix_len, topk_out, mode, ws, ws_bytes, stream, nullptr, 1, 0,
                   0, &lm);
}

tr_status tr_step(const tr_tree* t, int32_t B, int64_t V, int32_t k, const void* logits,
                  tr_dtype l_dtype, void* M, tr_dtype m_dtype, int32_t* tree_tok, int32_t* root_tok,
                  int32_t* accept_len, int32_t* accept_path, int32_t* emitted, int32_t Hkv,
                  int32_t d, tr_dtype kv_dtype, const void* k_tree, const void* v_tree,
                  void* k_cache, void* v_cache, int64_t cap, int32_t* prefix_len, int32_t* topk_out,
                  void* ws, size_t ws_bytes, void* stream) {
  return tr_step_ex(t, B, V, k, logits, l_dtype, M, m_dtype, tree_tok, root_tok, accept_len,
                    accept_path, emitted, Hkv, d, kv_dtype, k_tree, v_tree, k_cache, v_cache, cap,
                    prefix_len, topk_out, TR_UPDATE_ALL, ws, ws_bytes, stream);
}

tr_status tr_init_matrix(int32_t B, int64_t V, int32_t k, void* M, tr_dtype m_dtype,
                         tr_init_mode mode, const void* prior, tr_dtype prior_dtype,
                         int32_t prior_batches, uint64_t seed, void* stream) {
  TR_CHECK(B >= 1 && V >= 1 && k >= 1, TR_ERR_INVALID_ARGUMENT, "B, V and k must be at least 1");
  TR_CHECK(V <= INT32_MAX, TR_ERR_INVALID_ARGUMENT, "V above 2^31-1");
  TR_CHECK(M && aligned16(M), TR_ERR_INVALID_ARGUMENT, "M is null or not 16-byte aligned");
  TR_CHECK(m_dtype == TR_INT32 || m_dtype == TR_INT64, TR_ERR_UNSUPPORTED, "M must be int32 or int64");
  TR_CHECK(mode == TR_INIT_ZERO || mode == TR_INIT_RANDOM || mode == TR_INIT_PRIOR,
           TR_ERR_INVALID_ARGUMENT, "unknown init mode %d", int(mode));
  int prior_is64 = 0;
  if (mode == TR_INIT_PRIOR) {
    TR_CHECK(prior && aligned16(prior), TR_ERR_INVALID_ARGUMENT,
             "prior is null or not 16-byte aligned");
    TR_CHECK(prior_dtype == TR_INT32 || prior_dtype == TR_INT64, TR_ERR_UNSUPPORTED,
             "prior must be int32 or int64");
    TR_CHECK(prior_batches == 1 || prior_batches == B, TR_ERR_INVALID_ARGUMENT,
             "prior_batches %d must be 1 or B = %d", prior_batches, B);
    prior_is64 = prior_dtype == TR_INT64;
  }
  const int mode_i = mode == TR_INIT_ZERO ? tr::INIT_ZERO
                     : mode == TR_INIT_RANDOM ? tr::INIT_RANDOM : tr::INIT_PRIOR;
  return hip_status(tr::launch_init_m(mode_i, M, m_dtype == TR_INT64, B, V, k, prior, prior_is64,
                                      prior_batches == 1 && B > 1 ? 1 : 0, seed,
                                      hipStream_t(stream)),
                    "tr_init_matrix");
}

}  // extern "C"

extern "C" {

tr_status tr_profile_enable(int32_t on) {
  auto& P = tr::g_prof;
  if (on && P.ev.empty()) {
    P.ev.resize(2 * tr::kProfMax, nullptr);
    P.id.resize(tr::kProfMax, 0);
    for (auto& e : P.ev) {
      const hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) {
        for (auto& f : P.ev)
          if (f) (void)hipEventDestroy(f);   // already failing: keep the first error
        P.ev.clear();
        P.id.clear();
        return hip_status(err, "tr_profile_enable");
      }
    }
  }
  P.on = on != 0;
  P.n = 0;
  return ok();
}

tr_status tr_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  TR_CHECK(src && sink, TR_ERR_INVALID_ARGUMENT, "null pointer");
  TR_CHECK(aligned16(src) && (reinterpret_cast<uintptr_t>(sink) & 3) == 0, TR_ERR_INVALID_ARGUMENT,
           "src must be 16-byte aligned, sink 4-byte aligned");
  TR_CHECK(bytes > 0 && bytes % 16 == 0, TR_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16");
  return hip_status(tr::launch_read_probe(src, bytes, sink, hipStream_t(stream)), "tr_read_probe");
}

int32_t tr_profile_read(tr_launch_time* out, int32_t max) {
  auto& P = tr::g_prof;
  int32_t w = 0;
  for (int i = 0; i < P.n; ++i) {
    if (hipEventSynchronize(P.ev[2 * i + 1]) != hipSuccess) continue;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, P.ev[2 * i], P.ev[2 * i + 1]) != hipSuccess) continue;
    if (out && w < max) out[w++] = tr_launch_time{P.id[i], ms};
  }
  P.n = 0;
  return w;
}

}  // extern "C"
