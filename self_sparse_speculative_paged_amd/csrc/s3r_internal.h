// Internal launch interface between the C-ABI layer (s3r_api.cpp) and the
// kernels. Everything here is host-visible plain data; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "s3r.h"

namespace s3r {

// Split-KV partition of one attention call: the attended items (pages, or
// entries of a selection row) of every (sequence, kv head) are cut into
// n_splits ranges of pages_per_split items; each range is one wave's work.
struct SplitPlan {
  int32_t pages_per_split;
  int32_t n_splits;
  int32_t rows;             // G * n_queries attention rows per kv head
  int32_t row_blocks;       // ceil(rows / 16): MFMA N-blocks
  int32_t waves_per_group;  // splits merged inside one workgroup (bf16)
  int32_t n_groups;         // workgroups per (sequence, kv head)
  int32_t lds_region_bytes; // per-wave LDS region (window table, then partial)
  size_t workspace_bytes;   // global partials: only when n_groups > 1 (or fp32)
  int32_t staged;           // K/V staged through an LDS ring, one split per workgroup
};

// The LDS-staged kernel (bf16 dense verify, head dim 128, 49..64 rows): a
// ring of kStagedRing window slots of 16 KB, then the split's page pairs.
constexpr int32_t kStagedRing = 4;
inline size_t staged_lds_bytes(int32_t pages_per_split) {
  return (size_t)kStagedRing * 16384 + 8 * (size_t)((pages_per_split + 1) / 2);
}

// dense: every page of each sequence (the verify); else a selection of max_items.
SplitPlan plan_attention(const s3r_paged_kv& kv, int32_t n_queries, int32_t max_items, bool dense);

// Once-per-round selection: logical pages [f0, f1] hold the positions of the
// round's gamma draft queries, seq_len - 1 .. seq_len + gamma - 2 (seq_len at
// draft step 0), clipped below at 0 and to the table width; empty (f1 < f0)
// when gamma == 0 or no such position exists. These pages are always selected.
struct ForcedPages {
  int32_t f0, f1;
};

__host__ __device__ inline ForcedPages round_forced_pages(int32_t seq_len, int32_t gamma,
                                                          int32_t page_size, int32_t max_pages) {
  ForcedPages f{0, -1};
  if (gamma <= 0) return f;
  const int32_t lo = seq_len > 1 ? seq_len - 1 : 0;
  const int32_t hi = seq_len + gamma - 2;
  if (hi < lo) return f;
  f.f0 = lo / page_size;
  f.f1 = hi / page_size < max_pages - 1 ? hi / page_size : max_pages - 1;
  return f;
}

struct AttnArgs {
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const void* q;          // [B][nq][Hq][D]
  const int32_t* sel;     // [B][Hkv][ksel] or nullptr (dense)
  void* out;              // [B][nq][Hq][D]
  float* part_o;          // [B][Hkv][n_groups][rows][D]
  float* part_ml;         // [B][Hkv][n_groups][rows][2] (max in log2 units, sum)
  int32_t B, Hq, Hkv, G, D, max_pages, nq, ksel;
  int32_t rows, pages_per_split, n_splits;
  int32_t waves_per_group, n_groups, lds_region_bytes;
  int32_t staged;         // SplitPlan::staged
  float scale_log2;       // softmax_scale * log2(e)
  int32_t out_bf16;
  // Fused draft step only: page scores [B][Hkv][max_pages]; the selection is
  // built in LDS at list_offset and published to sel_out / nsel_out.
  const float* scores;
  int32_t* sel_out;
  int32_t* nsel_out;
  int32_t list_offset;
  // Single-kernel draft step (score_here != 0): the workgroup scores its pages
  // from the bf16 bounds (refreshing pages from refresh_from[b] / P on into
  // bounds_out) with sel_scale, keeping its page-table row in LDS at pt_offset.
  int32_t score_here;
  int32_t pt_offset;
  int32_t round_gamma;      // > 0: once-per-round selection with forced pages
  const void* bounds;
  void* bounds_out;
  const int32_t* refresh_from;
  float sel_scale;
  // Longest-first scheduling for ragged batches: when set, launch_attention
  // first ranks the sequences by length into order[B] (device scratch the
  // caller's workspace provides) and workgroup slots take sequences in that
  // order, so the longest start first and the short ones fill in behind.
  int32_t* order;
};

// Whether a batch is ragged enough for longest-first scheduling: its longest
// table is more than twice the average the caller's page hint implies.
inline bool schedule_longest_first(const s3r_paged_kv& kv) {
  return kv.total_pages_hint > 0 &&
         (int64_t)kv.max_pages_per_seq * kv.num_seqs > 2 * (int64_t)kv.total_pages_hint;
}
inline size_t order_bytes(const s3r_paged_kv& kv) {
  return schedule_longest_first(kv) ? (sizeof(int32_t) * (size_t)kv.num_seqs + 255) & ~(size_t)255 : 0;
}

hipError_t launch_attention(const AttnArgs& a, s3r_dtype kv_dtype, hipStream_t stream);

struct BoundsArgs {
  const void* k_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* first_pos;  // nullptr = all pages
  void* bounds;
  int32_t B, Hkv, D, max_pages, pages_y;  // grid rows: pages handled together per (seq, head)
  int32_t span;                           // pages from first_pos / P the call covers
};

hipError_t launch_bounds(const BoundsArgs& a, s3r_dtype kv_dtype, hipStream_t stream);

struct KvCommitArgs {
  const void* k_new;      // [B][count][Hkv][D]
  const void* v_new;      // [B][count][Hkv][D]
  const int32_t* first_pos;
  void* k_pool;           // written
  void* v_pool;           // written
  const int32_t* page_table;
  const int32_t* seq_lens;  // committed lengths after the call
  void* bounds;           // nullptr: no bounds upkeep
  int32_t B, Hkv, D, max_pages, count;
};

hipError_t launch_kv_commit(const KvCommitArgs& a, s3r_dtype kv_dtype, hipStream_t stream);

struct SelectArgs {
  const void* bounds;
  void* bounds_out;             // == bounds when refresh_from is set (bf16 only)
  const void* k_pool;
  const int32_t* refresh_from;  // [B] or nullptr: pages from refresh_from/P on are recomputed
  const void* q;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* scores;        // workspace [B][Hkv][max_pages]
  int32_t* selected;    // [B][Hkv][k]
  int32_t* num_selected;
  int32_t B, Hq, Hkv, G, D, max_pages, k;
  float scale;
  int32_t round_gamma;  // > 0: once-per-round selection with forced pages
};

hipError_t launch_select(const SelectArgs& a, s3r_dtype kv_dtype, hipStream_t stream);
// Scores only (no top-k), with the optional bounds refresh: the first half of
// the fused draft step.
hipError_t launch_scores(const SelectArgs& a, s3r_dtype kv_dtype, hipStream_t stream);
size_t select_workspace_bytes(int32_t B, int32_t Hkv, int32_t max_pages);
int32_t select_max_pages_supported();
// Page keys per thread of the fused draft step's in-register top-k: a W-wave
// workgroup ranks at most fused_topk_keys(W) * 64 * W pages per sequence
// (8192 at W = 8); longer page tables take the separate select kernel.
constexpr int fused_topk_keys(int waves) { return waves >= 8 ? 16 : 8; }
// The one-kernel step's four-wave workgroups also come with 32 keys per
// thread (8192 pages), used only for tables past fused_topk_keys(4) * 256
// pages: unused keys cost a uniform branch each, so short tables keep 8.
constexpr int kWideTopkKeys = 32;

struct SampleArgs {
  const float* draft_logits;   // [B][draft_rows][V]
  const float* target_logits;  // [B][gamma + 1][V], or nullptr (the drafter's draws)
  const int32_t* draft_tokens; // [B][gamma] (spec_sample only)
  int32_t* out_tokens;         // spec_sample: [B][gamma + 1]; the drafter's draws: [B][rows]
  int32_t* num_accepted;
  double* alpha;               // acceptance rate: [B][gamma]
  void* workspace;
  int32_t B, gamma, V, n_chunks;
  int32_t rows;                // rows per sequence of the statistics pass (set by the launchers
                               // except for the drafter's draws, where it is the caller's row count)
  int32_t draft_rows;          // rows per sequence in draft_logits (set by the launchers)
  int64_t first_slot;          // the drafter's draws: row r uses Philox slot first_slot + r
  float temperature;
  uint64_t seed, offset;
};

int32_t sample_chunks(int32_t vocab);
// Blocks of the statistics pass over `rows` rows per sequence (the largest
// grid of the sampling calls).
size_t sample_blocks(int32_t B, int32_t rows, int32_t vocab);
size_t sample_workspace_bytes(int32_t B, int32_t gamma, int32_t vocab);
size_t draft_sample_workspace_bytes(int32_t B, int32_t rows, int32_t vocab);
size_t acceptance_workspace_bytes(int32_t B, int32_t gamma, int32_t vocab);
hipError_t launch_sample(const SampleArgs& a, hipStream_t stream);
// The allocation-free sampler's scratch: a device array of this many bytes,
// and its address on the current device.
constexpr size_t kStaticSampleScratchBytes = (size_t)4 << 20;
hipError_t static_sample_scratch(void** ptr);
hipError_t launch_draft_sample(const SampleArgs& a, hipStream_t stream);
hipError_t launch_acceptance(const SampleArgs& a, hipStream_t stream);

// Checks of the device data the kernels trust, run when S3R_DEBUG is set
// (s3r_debug.cpp). Each waits for the stream and returns INVALID_ARGUMENT on a
// value a launch would read out of range, UNSUPPORTED under graph capture.
bool debug_checks_on();
// seq_lens fit a page-table row and the entries below them name pool pages.
s3r_status debug_check_kv(const s3r_paged_kv& kv, hipStream_t st, const char* where);
// The entries a KV commit reads are below num_phys_pages (negative: unallocated).
s3r_status debug_check_commit(const s3r_paged_kv& kv, const int32_t* first_pos, int32_t count,
                              hipStream_t st, const char* where);
// Draft token ids lie in [0, vocab).
s3r_status debug_check_tokens(const int32_t* tokens, int32_t num_seqs, int32_t gamma, int32_t vocab,
                              hipStream_t st, const char* where);

}  // namespace s3r
