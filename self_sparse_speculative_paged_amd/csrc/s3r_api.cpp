// C ABI of libs3r: host-side validation (before any HIP call), workspace
// sizing and kernel dispatch on the caller's stream. See include/s3r.h for the
// contract of each entry point.
#include <math.h>

#include <atomic>

#include "s3r.h"
#include "s3r_internal.h"

namespace {

constexpr int32_t kVersion = 300;  // 0.3.0: the drafter's draws and the acceptance rate
constexpr int32_t kMaxRows = 64;   // G * n_queries per kv head (4 MFMA row blocks)
constexpr int32_t kMaxGamma = 16;
// Largest grid of a sampling pass: one block per (sequence, row, 4096-token chunk).
constexpr size_t kMaxBlocks = (size_t)1 << 31;

// The kernels move K/V rows, bounds, queries, outputs and workspace through
// 16-byte vector accesses.
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

s3r_status check_kv(const s3r_paged_kv* kv) {
  if (kv == nullptr) return S3R_ERR_INVALID_ARGUMENT;
  if (kv->num_seqs < 1 || kv->num_q_heads < 1 || kv->num_kv_heads < 1 || kv->max_pages_per_seq < 1 ||
      kv->total_pages_hint < 0 || kv->num_phys_pages < 0)
    return S3R_ERR_INVALID_ARGUMENT;
  if (kv->num_q_heads % kv->num_kv_heads != 0) return S3R_ERR_INVALID_ARGUMENT;
  if (kv->k_pool == nullptr || kv->v_pool == nullptr || kv->page_table == nullptr || kv->seq_lens == nullptr)
    return S3R_ERR_INVALID_ARGUMENT;
  if (misaligned(kv->k_pool) || misaligned(kv->v_pool)) return S3R_ERR_INVALID_ARGUMENT;
  if (kv->kv_dtype != S3R_F32 && kv->kv_dtype != S3R_BF16) return S3R_ERR_UNSUPPORTED;
  if (kv->head_dim != 64 && kv->head_dim != 128) return S3R_ERR_UNSUPPORTED;
  if (kv->page_size != 16) return S3R_ERR_UNSUPPORTED;
  if (kv->num_q_heads / kv->num_kv_heads > 8) return S3R_ERR_UNSUPPORTED;
  if ((int64_t)kv->num_seqs * kv->num_q_heads > ((int64_t)1 << 24)) return S3R_ERR_UNSUPPORTED;
  return S3R_OK;
}

s3r_status check_workspace(void* ws, size_t have, size_t need) {
  if (have < need) return S3R_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && (ws == nullptr || misaligned(ws))) return S3R_ERR_INVALID_ARGUMENT;
  return S3R_OK;
}

s3r_status from_hip(hipError_t e) { return e == hipSuccess ? S3R_OK : S3R_ERR_HIP; }

// Under S3R_DEBUG: the device data a call on kv would read, checked on the host.
s3r_status debug_kv(const s3r_paged_kv& kv, void* stream, const char* where) {
  if (!s3r::debug_checks_on()) return S3R_OK;
  return s3r::debug_check_kv(kv, static_cast<hipStream_t>(stream), where);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of one attention call: the split partials, then (ragged batches)
// the longest-first order.
size_t attn_call_workspace(const s3r_paged_kv& kv, const s3r::SplitPlan& plan) {
  const size_t ob = s3r::order_bytes(kv);
  return ob ? align256(plan.workspace_bytes) + ob : plan.workspace_bytes;
}

s3r::AttnArgs attn_args(const s3r_paged_kv* kv, const s3r::SplitPlan& plan, const void* q,
                        const int32_t* sel, int32_t ksel, int32_t n_q, float scale,
                        s3r_dtype out_dtype, void* out, void* ws);

s3r_status check_attention(const s3r_paged_kv* kv, const void* q, int32_t n_q, float scale,
                           s3r_dtype out_dtype, void* out) {
  if (s3r_status s = check_kv(kv)) return s;
  if (q == nullptr || out == nullptr || n_q < 1 || !isfinite(scale)) return S3R_ERR_INVALID_ARGUMENT;
  if (misaligned(q) || misaligned(out)) return S3R_ERR_INVALID_ARGUMENT;
  if (out_dtype != S3R_F32 && out_dtype != S3R_BF16) return S3R_ERR_UNSUPPORTED;
  const int32_t G = kv->num_q_heads / kv->num_kv_heads;
  if ((int64_t)G * n_q > kMaxRows) return S3R_ERR_UNSUPPORTED;
  return S3R_OK;
}

s3r_status run_attention(const s3r_paged_kv* kv, const void* q, const int32_t* sel, int32_t ksel,
                         int32_t n_q, float scale, s3r_dtype out_dtype, void* out, void* ws,
                         size_t ws_bytes, void* stream, const char* where) {
  if (s3r_status s = check_attention(kv, q, n_q, scale, out_dtype, out)) return s;
  const int32_t max_items = sel ? ksel : kv->max_pages_per_seq;
  const s3r::SplitPlan plan = s3r::plan_attention(*kv, n_q, max_items, sel == nullptr);
  if (s3r_status s = check_workspace(ws, ws_bytes, attn_call_workspace(*kv, plan))) return s;
  if (s3r_status s = debug_kv(*kv, stream, where)) return s;
  s3r::AttnArgs a = attn_args(kv, plan, q, sel, ksel, n_q, scale, out_dtype, out, ws);
  if (s3r::order_bytes(*kv))
    a.order = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align256(plan.workspace_bytes));
  return from_hip(s3r::launch_attention(a, kv->kv_dtype, static_cast<hipStream_t>(stream)));
}

s3r::AttnArgs attn_args(const s3r_paged_kv* kv, const s3r::SplitPlan& plan, const void* q,
                        const int32_t* sel, int32_t ksel, int32_t n_q, float scale,
                        s3r_dtype out_dtype, void* out, void* ws) {
  const int32_t G = kv->num_q_heads / kv->num_kv_heads;
  s3r::AttnArgs a{};
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.page_table = kv->page_table;
  a.seq_lens = kv->seq_lens;
  a.q = q;
  a.sel = sel;
  a.out = out;
  const size_t items = (size_t)kv->num_seqs * kv->num_kv_heads * plan.n_groups;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = ws ? a.part_o + items * plan.rows * kv->head_dim : nullptr;
  a.B = kv->num_seqs;
  a.Hq = kv->num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = G;
  a.D = kv->head_dim;
  a.max_pages = kv->max_pages_per_seq;
  a.nq = n_q;
  a.ksel = ksel;
  a.rows = plan.rows;
  a.pages_per_split = plan.pages_per_split;
  a.n_splits = plan.n_splits;
  a.waves_per_group = plan.waves_per_group;
  a.n_groups = plan.n_groups;
  a.lds_region_bytes = plan.lds_region_bytes;
  a.staged = plan.staged;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_bf16 = out_dtype == S3R_BF16;
  return a;
}

s3r::SelectArgs select_args(const s3r_paged_kv* kv, const void* bounds, const void* q,
                            int32_t budget_tokens, float scale, int32_t* selected,
                            int32_t* num_selected, void* scores) {
  s3r::SelectArgs a{};
  a.bounds = bounds;
  a.k_pool = kv->k_pool;
  a.q = q;
  a.page_table = kv->page_table;
  a.seq_lens = kv->seq_lens;
  a.scores = static_cast<float*>(scores);
  a.selected = selected;
  a.num_selected = num_selected;
  a.B = kv->num_seqs;
  a.Hq = kv->num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = kv->num_q_heads / kv->num_kv_heads;
  a.D = kv->head_dim;
  a.max_pages = kv->max_pages_per_seq;
  a.k = budget_tokens / kv->page_size;
  a.scale = scale;
  return a;
}

// kWaves waves per (sequence, kv head), the selection split evenly over them:
// the draft's plan whenever its top-k runs inside the attention workgroup.
s3r::SplitPlan wave_plan(const s3r_paged_kv& kv, int32_t k, int kWaves) {
  s3r::SplitPlan a{};
  const int32_t G = kv.num_q_heads / kv.num_kv_heads;
  a.rows = G;
  a.row_blocks = 1;
  int32_t pps = (k + kWaves - 1) / kWaves;
  pps = pps < 2 ? 2 : (pps + 1) & ~1;
  a.pages_per_split = pps;
  a.n_splits = (k + pps - 1) / pps;
  a.waves_per_group = kWaves;
  a.n_groups = 1;
  const size_t table = sizeof(int) * 4 * (size_t)((pps + 1) / 2);
  const size_t partial = sizeof(float) * (size_t)G * (kv.head_dim + 2);
  a.lds_region_bytes = (int32_t)(((table > partial ? table : partial) + 15) & ~(size_t)15);
  a.workspace_bytes = 0;
  return a;
}

// The two-kernel draft step keeps the selection list in LDS after the per-wave
// regions; it needs bf16 KV, at most 64 KB of LDS and a page table short
// enough for its in-register top-k. A selection that fits one workgroup runs
// on eight waves, so the top-k has 512 threads.
struct DraftStepPlan {
  s3r::SplitPlan attn;
  size_t select_ws;
  bool fused;
  int32_t list_offset;
  size_t order_offset;     // longest-first order in the workspace (ragged batches)
  size_t workspace_bytes;  // enough for every path the call may take
};

// Whether the rank-and-attend kernel can take plan a: eight waves (its top-k
// runs on 512 threads), the page table within that top-k, and the wave regions
// plus the list within 64 KB of LDS. Sets the list's offset.
bool rank_and_attend_fits(const s3r_paged_kv& kv, const s3r::SplitPlan& a, int32_t k, int32_t* list_offset) {
  const int32_t w = a.waves_per_group;
  const size_t regions = (size_t)a.lds_region_bytes * w;
  const size_t list = (regions + 15) & ~(size_t)15;
  *list_offset = (int32_t)list;
  return kv.kv_dtype == S3R_BF16 && w == 8 && kv.max_pages_per_seq <= s3r::fused_topk_keys(w) * 64 * w &&
         list + sizeof(int32_t) * (size_t)k <= 64 * 1024;
}

DraftStepPlan plan_draft_step(const s3r_paged_kv& kv, int32_t budget_tokens) {
  DraftStepPlan p{};
  const int32_t k = budget_tokens / kv.page_size;
  // The attention's own plan (its LDS is capped) unless eight waves are what
  // lets the step rank inside the attention kernel.
  p.attn = s3r::plan_attention(kv, 1, k, false);
  if (kv.kv_dtype == S3R_BF16 && p.attn.row_blocks == 1 && p.attn.waves_per_group < 8) {
    const s3r::SplitPlan w8 = wave_plan(kv, k, 8);
    int32_t unused = 0;
    if (rank_and_attend_fits(kv, w8, k, &unused)) p.attn = w8;
  }
  p.select_ws = s3r::select_workspace_bytes(kv.num_seqs, kv.num_kv_heads, kv.max_pages_per_seq);
  p.fused = rank_and_attend_fits(kv, p.attn, k, &p.list_offset);
  p.workspace_bytes = p.fused ? p.select_ws + p.attn.workspace_bytes
                              : (p.select_ws > p.attn.workspace_bytes ? p.select_ws : p.attn.workspace_bytes);
  if (const size_t ob = s3r::order_bytes(kv)) {
    p.order_offset = align256(p.workspace_bytes);
    p.workspace_bytes = p.order_offset + ob;
  }
  return p;
}

// Compute units of the current device, cached per device (256 if the query fails).
int32_t device_cu_count() {
  static std::atomic<int32_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int32_t v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    int n = 0;
    v = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Single-kernel draft step: one workgroup of four or eight waves per (sequence,
// kv head) that scores, ranks and attends. It pays off when those workgroups
// fill the device; each reads its whole bounds row, so it needs the row's page
// ids, its scores and the list in LDS and its keys in the top-k's registers.
struct SingleKernelPlan {
  bool ok;
  s3r::SplitPlan attn;
  int32_t pt_offset, list_offset;
};

// A four-wave workgroup runs at about half its CU's rate while it shares the
// CU. Four waves are only worth it while the longest (sequence, kv head) then
// still ends near the average CU's load. Otherwise, on a ragged batch whose
// long outliers meet few (sequence, kv head) pairs per CU, their workgroups
// would set the end of the kernel. The bytes of one item with p pages are its
// bounds (p rows) plus the K/V of min(k, p) pages. The batch total comes from
// the page hint.
bool longest_fits_half_cu(const s3r_paged_kv& kv, int32_t k, int32_t cus) {
  const double bound_bytes = 2.0 * kv.head_dim * 2, page_bytes = 2.0 * kv.page_size * kv.head_dim * 2;
  auto item = [&](double pages) { return pages * bound_bytes + (pages < k ? pages : k) * page_bytes; };
  const double total = kv.total_pages_hint > 0 ? kv.total_pages_hint
                                               : (double)kv.num_seqs * kv.max_pages_per_seq;
  const double per_cu = kv.num_kv_heads * (total * bound_bytes +
                                           kv.num_seqs * (total / kv.num_seqs < k ? total / kv.num_seqs : k) *
                                               page_bytes) / cus;
  return 2.0 * item(kv.max_pages_per_seq) <= 1.25 * per_cu;
}

SingleKernelPlan plan_single_kernel(const s3r_paged_kv& kv, int32_t k) {
  SingleKernelPlan p{};
  const int32_t G = kv.num_q_heads / kv.num_kv_heads;
  if (kv.kv_dtype != S3R_BF16 || (G != 1 && G != 2 && G != 4 && G != 8)) return p;
  const int64_t items = (int64_t)kv.num_seqs * kv.num_kv_heads;
  const int32_t cus = device_cu_count();
  if (items < cus) return p;
  // Eight waves per workgroup give one resident workgroup per CU. With at
  // least two (sequence, kv head) pairs per CU, workgroups of four waves let
  // two share each CU at once, so one's ranking overlaps the other's reads.
  // Their 256-thread top-k ranks up to kWideTopkKeys * 256 pages.
  const int kWaves =
      items >= 2 * (int64_t)cus && kv.max_pages_per_seq <= s3r::kWideTopkKeys * 64 * 4 &&
              longest_fits_half_cu(kv, k, cus)
          ? 4
          : 8;
  const int keys = kWaves == 4 ? s3r::kWideTopkKeys : s3r::fused_topk_keys(kWaves);
  if (kv.max_pages_per_seq > keys * 64 * kWaves) return p;
  const s3r::SplitPlan& a = p.attn = wave_plan(kv, k, kWaves);
  const size_t row = sizeof(int32_t) * (size_t)kv.max_pages_per_seq;
  size_t front = (size_t)a.lds_region_bytes * kWaves;
  if (front < row) front = row;  // the scores alias the wave regions
  front = (front + 15) & ~(size_t)15;
  const size_t list = (front + row + 15) & ~(size_t)15;
  if (list + sizeof(int32_t) * (size_t)k > 64 * 1024) return p;
  p.pt_offset = (int32_t)front;
  p.list_offset = (int32_t)list;
  p.ok = true;
  return p;
}

}  // namespace

extern "C" {

size_t s3r_page_select_workspace(const s3r_paged_kv* kv, int32_t budget_tokens) {
  (void)budget_tokens;
  if (check_kv(kv) != S3R_OK) return 0;
  return s3r::select_workspace_bytes(kv->num_seqs, kv->num_kv_heads, kv->max_pages_per_seq);
}

size_t s3r_attn_workspace(const s3r_paged_kv* kv, int32_t n_queries, int32_t max_pages_attended) {
  if (check_kv(kv) != S3R_OK || n_queries < 1 || max_pages_attended < 1) return 0;
  // enough for either kind of call: a dense verify or a sparse attention
  const size_t dense = attn_call_workspace(*kv, s3r::plan_attention(*kv, n_queries, max_pages_attended, true));
  const size_t sparse = attn_call_workspace(*kv, s3r::plan_attention(*kv, n_queries, max_pages_attended, false));
  return dense > sparse ? dense : sparse;
}

size_t s3r_spec_sample_workspace(int32_t num_seqs, int32_t gamma, int32_t vocab) {
  if (num_seqs < 1 || gamma < 1 || gamma > kMaxGamma || vocab < 1) return 0;
  return s3r::sample_workspace_bytes(num_seqs, gamma, vocab);
}

s3r_status s3r_page_bounds_update(const s3r_paged_kv* kv, void* bounds, const int32_t* first_pos,
                                  int32_t max_pages_touched, void* stream) {
  if (s3r_status s = check_kv(kv)) return s;
  if (bounds == nullptr || misaligned(bounds)) return S3R_ERR_INVALID_ARGUMENT;
  if (first_pos != nullptr && max_pages_touched < 1) return S3R_ERR_INVALID_ARGUMENT;
  s3r::BoundsArgs a{};
  a.k_pool = kv->k_pool;
  a.page_table = kv->page_table;
  a.seq_lens = kv->seq_lens;
  a.first_pos = first_pos;
  a.bounds = bounds;
  a.B = kv->num_seqs;
  a.Hkv = kv->num_kv_heads;
  a.D = kv->head_dim;
  a.max_pages = kv->max_pages_per_seq;
  a.span = first_pos ? (max_pages_touched < kv->max_pages_per_seq ? max_pages_touched
                                                                  : kv->max_pages_per_seq)
                     : kv->max_pages_per_seq;
  a.pages_y = a.span;
  if (s3r_status s = debug_kv(*kv, stream, "s3r_page_bounds_update")) return s;
  return from_hip(s3r::launch_bounds(a, kv->kv_dtype, static_cast<hipStream_t>(stream)));
}

s3r_status s3r_page_select(const s3r_paged_kv* kv, const void* bounds, const void* q,
                           int32_t budget_tokens, float softmax_scale, int32_t* selected,
                           int32_t* num_selected, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (s3r_status s = check_kv(kv)) return s;
  if (bounds == nullptr || q == nullptr || selected == nullptr || num_selected == nullptr)
    return S3R_ERR_INVALID_ARGUMENT;
  if (misaligned(bounds) || misaligned(q)) return S3R_ERR_INVALID_ARGUMENT;
  if (budget_tokens < kv->page_size || !isfinite(softmax_scale)) return S3R_ERR_INVALID_ARGUMENT;
  if (kv->max_pages_per_seq > s3r::select_max_pages_supported()) return S3R_ERR_UNSUPPORTED;
  const size_t need = s3r::select_workspace_bytes(kv->num_seqs, kv->num_kv_heads, kv->max_pages_per_seq);
  if (s3r_status s = check_workspace(workspace, workspace_bytes, need)) return s;
  if (s3r_status s = debug_kv(*kv, stream, "s3r_page_select")) return s;
  const s3r::SelectArgs a = select_args(kv, bounds, q, budget_tokens, softmax_scale, selected,
                                        num_selected, workspace);
  return from_hip(s3r::launch_select(a, kv->kv_dtype, static_cast<hipStream_t>(stream)));
}

s3r_status s3r_sparse_draft_attn(const s3r_paged_kv* kv, const void* q, const int32_t* selected,
                                 int32_t k, float softmax_scale, s3r_dtype out_dtype, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (selected == nullptr || k < 1) return S3R_ERR_INVALID_ARGUMENT;
  return run_attention(kv, q, selected, k, 1, softmax_scale, out_dtype, out, workspace,
                       workspace_bytes, stream, "s3r_sparse_draft_attn");
}

size_t s3r_sparse_draft_step_workspace(const s3r_paged_kv* kv, int32_t budget_tokens) {
  if (check_kv(kv) != S3R_OK || budget_tokens < kv->page_size) return 0;
  return plan_draft_step(*kv, budget_tokens).workspace_bytes;
}

}  // extern "C"

namespace {

// One draft step; round_gamma > 0 makes its selection the round's (forced
// pages kept, reused by the round's later steps).
s3r_status draft_step(const s3r_paged_kv* kv, void* bounds, const int32_t* refresh_from,
                      const void* q, int32_t budget_tokens, int32_t round_gamma,
                      float softmax_scale, int32_t* selected, int32_t* num_selected,
                      s3r_dtype out_dtype, void* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (s3r_status s = check_attention(kv, q, 1, softmax_scale, out_dtype, out)) return s;
  if (bounds == nullptr || selected == nullptr || num_selected == nullptr || misaligned(bounds))
    return S3R_ERR_INVALID_ARGUMENT;
  if (budget_tokens < kv->page_size) return S3R_ERR_INVALID_ARGUMENT;
  if (kv->max_pages_per_seq > s3r::select_max_pages_supported()) return S3R_ERR_UNSUPPORTED;
  const DraftStepPlan plan = plan_draft_step(*kv, budget_tokens);
  if (s3r_status s = check_workspace(workspace, workspace_bytes, plan.workspace_bytes)) return s;
  if (s3r_status s = debug_kv(*kv, stream, round_gamma ? "s3r_sparse_draft_round" : "s3r_sparse_draft_step"))
    return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t k = budget_tokens / kv->page_size;
  int32_t* order = s3r::order_bytes(*kv)
                       ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.order_offset)
                       : nullptr;
  s3r::SelectArgs sa = select_args(kv, bounds, q, budget_tokens, softmax_scale, selected,
                                   num_selected, workspace);
  sa.round_gamma = round_gamma;
  const SingleKernelPlan one = plan_single_kernel(*kv, k);
  if (one.ok) {
    s3r::AttnArgs a = attn_args(kv, one.attn, q, nullptr, k, 1, softmax_scale, out_dtype, out, nullptr);
    a.sel_out = selected;
    a.nsel_out = num_selected;
    a.list_offset = one.list_offset;
    a.score_here = 1;
    a.pt_offset = one.pt_offset;
    a.bounds = bounds;
    a.bounds_out = bounds;
    a.refresh_from = refresh_from;
    a.sel_scale = softmax_scale;
    a.round_gamma = round_gamma;
    a.order = order;
    return from_hip(s3r::launch_attention(a, kv->kv_dtype, st));
  }
  if (plan.fused) {
    sa.refresh_from = refresh_from;
    sa.bounds_out = bounds;
    if (hipError_t e = s3r::launch_scores(sa, kv->kv_dtype, st)) return from_hip(e);
    char* partials = static_cast<char*>(workspace) + plan.select_ws;
    s3r::AttnArgs a = attn_args(kv, plan.attn, q, nullptr, k, 1, softmax_scale, out_dtype, out,
                                plan.attn.workspace_bytes ? partials : nullptr);
    a.scores = static_cast<const float*>(workspace);
    a.sel_out = selected;
    a.nsel_out = num_selected;
    a.list_offset = plan.list_offset;
    a.round_gamma = round_gamma;
    a.order = order;
    return from_hip(s3r::launch_attention(a, kv->kv_dtype, st));
  }
  // Unfused: bounds refresh, then select, then attention (stream order makes
  // the workspace reusable between them).
  if (refresh_from) {
    s3r::BoundsArgs ba{};
    ba.k_pool = kv->k_pool;
    ba.page_table = kv->page_table;
    ba.seq_lens = kv->seq_lens;
    ba.first_pos = refresh_from;
    ba.bounds = bounds;
    ba.B = kv->num_seqs;
    ba.Hkv = kv->num_kv_heads;
    ba.D = kv->head_dim;
    ba.max_pages = kv->max_pages_per_seq;
    ba.span = kv->max_pages_per_seq;  // every page from refresh_from / P to the tail,
    ba.pages_y = 2;                   // normally just the tail page
    if (hipError_t e = s3r::launch_bounds(ba, kv->kv_dtype, st)) return from_hip(e);
  }
  if (hipError_t e = s3r::launch_select(sa, kv->kv_dtype, st)) return from_hip(e);
  s3r::AttnArgs a = attn_args(kv, plan.attn, q, selected, k, 1, softmax_scale, out_dtype, out,
                              plan.attn.workspace_bytes ? workspace : nullptr);
  a.order = order;
  return from_hip(s3r::launch_attention(a, kv->kv_dtype, st));
}

}  // namespace

extern "C" {

s3r_status s3r_sparse_draft_step(const s3r_paged_kv* kv, void* bounds, const int32_t* refresh_from,
                                 const void* q, int32_t budget_tokens, float softmax_scale,
                                 int32_t* selected, int32_t* num_selected, s3r_dtype out_dtype,
                                 void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return draft_step(kv, bounds, refresh_from, q, budget_tokens, 0, softmax_scale, selected,
                    num_selected, out_dtype, out, workspace, workspace_bytes, stream);
}

s3r_status s3r_sparse_draft_round(const s3r_paged_kv* kv, void* bounds, const int32_t* refresh_from,
                                  const void* q, int32_t budget_tokens, int32_t gamma,
                                  float softmax_scale, int32_t* selected, int32_t* num_selected,
                                  s3r_dtype out_dtype, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (s3r_status s = check_kv(kv)) return s;
  if (gamma < 1 || gamma > kMaxGamma || budget_tokens < 2 * kv->page_size) return S3R_ERR_INVALID_ARGUMENT;
  return draft_step(kv, bounds, refresh_from, q, budget_tokens, gamma, softmax_scale, selected,
                    num_selected, out_dtype, out, workspace, workspace_bytes, stream);
}

s3r_status s3r_kv_commit(const s3r_paged_kv* kv, const void* k_new, const void* v_new,
                         const int32_t* first_pos, int32_t count, void* bounds, void* stream) {
  if (s3r_status s = check_kv(kv)) return s;
  if (first_pos == nullptr || count < 0) return S3R_ERR_INVALID_ARGUMENT;
  if (count > 0 && (k_new == nullptr || v_new == nullptr)) return S3R_ERR_INVALID_ARGUMENT;
  if (misaligned(k_new) || misaligned(v_new) || misaligned(bounds))
    return S3R_ERR_INVALID_ARGUMENT;  // rows are moved as 16-byte runs
  s3r::KvCommitArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.first_pos = first_pos;
  // The struct's pool pointers are const for the read-only calls; this one
  // writes the caller's pools through them.
  a.k_pool = const_cast<void*>(kv->k_pool);
  a.v_pool = const_cast<void*>(kv->v_pool);
  a.page_table = kv->page_table;
  a.seq_lens = kv->seq_lens;
  a.bounds = bounds;
  a.B = kv->num_seqs;
  a.Hkv = kv->num_kv_heads;
  a.D = kv->head_dim;
  a.max_pages = kv->max_pages_per_seq;
  a.count = count;
  if (s3r::debug_checks_on())
    if (s3r_status s = s3r::debug_check_commit(*kv, first_pos, count, static_cast<hipStream_t>(stream),
                                                "s3r_kv_commit"))
      return s;
  return from_hip(s3r::launch_kv_commit(a, kv->kv_dtype, static_cast<hipStream_t>(stream)));
}

s3r_status s3r_dense_verify_attn(const s3r_paged_kv* kv, const void* q, int32_t n_q,
                                 float softmax_scale, s3r_dtype out_dtype, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return run_attention(kv, q, nullptr, 0, n_q, softmax_scale, out_dtype, out, workspace,
                       workspace_bytes, stream, "s3r_dense_verify_attn");
}

}  // extern "C"

namespace {

s3r_status check_spec_sample(int32_t num_seqs, int32_t gamma, int32_t vocab, const float* draft_logits,
                             const float* target_logits, const int32_t* draft_tokens, float temperature,
                             int32_t* out_tokens, int32_t* num_accepted) {
  if (num_seqs < 1 || vocab < 1 || gamma < 1 || gamma > kMaxGamma) return S3R_ERR_INVALID_ARGUMENT;
  if (!(temperature > 0.f) || !isfinite(temperature)) return S3R_ERR_INVALID_ARGUMENT;
  if (draft_logits == nullptr || target_logits == nullptr || draft_tokens == nullptr ||
      out_tokens == nullptr || num_accepted == nullptr)
    return S3R_ERR_INVALID_ARGUMENT;
  if (s3r::sample_blocks(num_seqs, 2 * gamma + 1, vocab) >= kMaxBlocks) return S3R_ERR_UNSUPPORTED;
  return S3R_OK;
}

s3r_status run_spec_sample(int32_t num_seqs, int32_t gamma, int32_t vocab, const float* draft_logits,
                           const float* target_logits, const int32_t* draft_tokens, float temperature,
                           uint64_t seed, uint64_t offset, int32_t* out_tokens, int32_t* num_accepted,
                           void* workspace, void* stream) {
  if (s3r::debug_checks_on())
    if (s3r_status s = s3r::debug_check_tokens(draft_tokens, num_seqs, gamma, vocab,
                                                static_cast<hipStream_t>(stream), "s3r_spec_sample"))
      return s;
  s3r::SampleArgs a{};
  a.draft_logits = draft_logits;
  a.target_logits = target_logits;
  a.draft_tokens = draft_tokens;
  a.out_tokens = out_tokens;
  a.num_accepted = num_accepted;
  a.workspace = workspace;
  a.B = num_seqs;
  a.gamma = gamma;
  a.V = vocab;
  a.n_chunks = s3r::sample_chunks(vocab);
  a.temperature = temperature;
  a.seed = seed;
  a.offset = offset;
  return from_hip(s3r::launch_sample(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

s3r_status s3r_spec_sample(int32_t num_seqs, int32_t gamma, int32_t vocab,
                           const float* draft_logits, const float* target_logits,
                           const int32_t* draft_tokens, float temperature, uint64_t seed,
                           uint64_t offset, int32_t* out_tokens, int32_t* num_accepted,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (s3r_status s = check_spec_sample(num_seqs, gamma, vocab, draft_logits, target_logits, draft_tokens,
                                       temperature, out_tokens, num_accepted))
    return s;
  const size_t need = s3r::sample_workspace_bytes(num_seqs, gamma, vocab);
  if (s3r_status s = check_workspace(workspace, workspace_bytes, need)) return s;
  return run_spec_sample(num_seqs, gamma, vocab, draft_logits, target_logits, draft_tokens, temperature,
                         seed, offset, out_tokens, num_accepted, workspace, stream);
}

size_t s3r_spec_sample_noalloc_max_workspace(void) { return s3r::kStaticSampleScratchBytes; }

s3r_status s3r_spec_sample_noalloc(int32_t num_seqs, int32_t gamma, int32_t vocab,
                                   const float* draft_logits, const float* target_logits,
                                   const int32_t* draft_tokens, float temperature, uint64_t seed,
                                   uint64_t offset, int32_t* out_tokens, int32_t* num_accepted,
                                   void* stream) {
  if (s3r_status s = check_spec_sample(num_seqs, gamma, vocab, draft_logits, target_logits, draft_tokens,
                                       temperature, out_tokens, num_accepted))
    return s;
  if (s3r::sample_workspace_bytes(num_seqs, gamma, vocab) > s3r::kStaticSampleScratchBytes)
    return S3R_ERR_WORKSPACE_TOO_SMALL;
  void* scratch = nullptr;
  if (hipError_t e = s3r::static_sample_scratch(&scratch)) return from_hip(e);
  return run_spec_sample(num_seqs, gamma, vocab, draft_logits, target_logits, draft_tokens, temperature,
                         seed, offset, out_tokens, num_accepted, scratch, stream);
}

size_t s3r_draft_sample_workspace(int32_t num_seqs, int32_t n_rows, int32_t vocab) {
  if (num_seqs < 1 || n_rows < 1 || vocab < 1) return 0;
  return s3r::draft_sample_workspace_bytes(num_seqs, n_rows, vocab);
}

s3r_status s3r_draft_sample(int32_t num_seqs, int32_t n_rows, int32_t vocab, const float* logits,
                            float temperature, uint64_t seed, uint64_t offset, int64_t first_slot,
                            int32_t* tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 1 || n_rows < 1 || vocab < 1 || first_slot < 0) return S3R_ERR_INVALID_ARGUMENT;
  if (!(temperature > 0.f) || !isfinite(temperature)) return S3R_ERR_INVALID_ARGUMENT;
  if (logits == nullptr || tokens == nullptr) return S3R_ERR_INVALID_ARGUMENT;
  if (s3r::sample_blocks(num_seqs, n_rows, vocab) >= kMaxBlocks) return S3R_ERR_UNSUPPORTED;
  const size_t need = s3r::draft_sample_workspace_bytes(num_seqs, n_rows, vocab);
  if (s3r_status s = check_workspace(workspace, workspace_bytes, need)) return s;
  s3r::SampleArgs a{};
  a.draft_logits = logits;
  a.out_tokens = tokens;
  a.workspace = workspace;
  a.B = num_seqs;
  a.rows = n_rows;
  a.V = vocab;
  a.n_chunks = s3r::sample_chunks(vocab);
  a.first_slot = first_slot;
  a.temperature = temperature;
  a.seed = seed;
  a.offset = offset;
  return from_hip(s3r::launch_draft_sample(a, static_cast<hipStream_t>(stream)));
}

size_t s3r_acceptance_rate_workspace(int32_t num_seqs, int32_t gamma, int32_t vocab) {
  if (num_seqs < 1 || gamma < 1 || vocab < 1) return 0;
  return s3r::acceptance_workspace_bytes(num_seqs, gamma, vocab);
}

s3r_status s3r_acceptance_rate(int32_t num_seqs, int32_t gamma, int32_t vocab,
                               const float* draft_logits, const float* target_logits,
                               float temperature, double* alpha, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (num_seqs < 1 || gamma < 1 || vocab < 1) return S3R_ERR_INVALID_ARGUMENT;
  if (!(temperature > 0.f) || !isfinite(temperature)) return S3R_ERR_INVALID_ARGUMENT;
  if (draft_logits == nullptr || target_logits == nullptr || alpha == nullptr)
    return S3R_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(alpha) & 7) != 0) return S3R_ERR_INVALID_ARGUMENT;
  if (s3r::sample_blocks(num_seqs, 2 * gamma, vocab) >= kMaxBlocks) return S3R_ERR_UNSUPPORTED;
  const size_t need = s3r::acceptance_workspace_bytes(num_seqs, gamma, vocab);
  if (s3r_status s = check_workspace(workspace, workspace_bytes, need)) return s;
  s3r::SampleArgs a{};
  a.draft_logits = draft_logits;
  a.target_logits = target_logits;
  a.alpha = alpha;
  a.workspace = workspace;
  a.B = num_seqs;
  a.gamma = gamma;
  a.V = vocab;
  a.n_chunks = s3r::sample_chunks(vocab);
  a.temperature = temperature;
  return from_hip(s3r::launch_acceptance(a, static_cast<hipStream_t>(stream)));
}

const char* s3r_status_string(s3r_status status) {
  switch (status) {
    case S3R_OK: return "S3R_OK";
    case S3R_ERR_INVALID_ARGUMENT: return "S3R_ERR_INVALID_ARGUMENT";
    case S3R_ERR_UNSUPPORTED: return "S3R_ERR_UNSUPPORTED";
    case S3R_ERR_WORKSPACE_TOO_SMALL: return "S3R_ERR_WORKSPACE_TOO_SMALL";
    case S3R_ERR_HIP: return "S3R_ERR_HIP";
    default: return "S3R_ERR_UNKNOWN";
  }
}

int32_t s3r_version(void) { return kVersion; }

}  // extern "C"
