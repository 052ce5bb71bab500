// Host-side checks of the device data the kernels trust (sequence lengths,
// page-table entries, draft token ids), run by the entry points when the
// environment variable S3R_DEBUG is set. Each check waits for the caller's
// stream, copies the data it needs to the host and tests every value the
// following launch would read; nothing here launches a kernel.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "s3r.h"
#include "s3r_internal.h"

namespace s3r {
namespace {

s3r_status not_capturing(hipStream_t st, const char* where) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return S3R_ERR_HIP;
  if (cs != hipStreamCaptureStatusNone) {
    fprintf(stderr, "libs3r S3R_DEBUG: %s: the checks synchronise the stream, which is being captured\n",
            where);
    return S3R_ERR_UNSUPPORTED;
  }
  return S3R_OK;
}

// Copies n int32 values from the device once the stream's earlier work is done.
s3r_status fetch(std::vector<int32_t>& out, const int32_t* dev, size_t n, hipStream_t st,
                 const char* where) {
  out.resize(n);
  if (n == 0) return S3R_OK;
  if (hipMemcpyAsync(out.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    fprintf(stderr, "libs3r S3R_DEBUG: %s: copying device data to the host failed\n", where);
    return S3R_ERR_HIP;
  }
  return S3R_OK;
}

int64_t pages_below(int32_t seq_len, int32_t P) { return seq_len > 0 ? ((int64_t)seq_len + P - 1) / P : 0; }

s3r_status bad_entry(const char* where, int b, int64_t j, int32_t e, int32_t n_phys) {
  if (n_phys > 0)
    fprintf(stderr, "libs3r S3R_DEBUG: %s: page_table[%d][%lld] = %d is outside the pool [0, %d)\n", where,
            b, (long long)j, e, n_phys);
  else
    fprintf(stderr, "libs3r S3R_DEBUG: %s: page_table[%d][%lld] = %d is negative\n", where, b,
            (long long)j, e);
  return S3R_ERR_INVALID_ARGUMENT;
}

}  // namespace

bool debug_checks_on() {
  const char* e = getenv("S3R_DEBUG");
  return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
}

s3r_status debug_check_kv(const s3r_paged_kv& kv, hipStream_t st, const char* where) {
  if (s3r_status s = not_capturing(st, where)) return s;
  const int B = kv.num_seqs, maxp = kv.max_pages_per_seq;
  std::vector<int32_t> lens, table;
  if (s3r_status s = fetch(lens, kv.seq_lens, (size_t)B, st, where)) return s;
  if (s3r_status s = fetch(table, kv.page_table, (size_t)B * maxp, st, where)) return s;
  for (int b = 0; b < B; ++b) {
    const int64_t n = pages_below(lens[b], kv.page_size);
    if (n > maxp) {
      fprintf(stderr, "libs3r S3R_DEBUG: %s: seq_lens[%d] = %d spans %lld pages; a page_table row holds %d\n",
              where, b, lens[b], (long long)n, maxp);
      return S3R_ERR_INVALID_ARGUMENT;
    }
    for (int64_t j = 0; j < n; ++j) {
      const int32_t e = table[(size_t)b * maxp + j];
      if (e < 0 || (kv.num_phys_pages > 0 && e >= kv.num_phys_pages))
        return bad_entry(where, b, j, e, kv.num_phys_pages);
    }
  }
  return S3R_OK;
}

s3r_status debug_check_commit(const s3r_paged_kv& kv, const int32_t* first_pos, int32_t count,
                              hipStream_t st, const char* where) {
  if (s3r_status s = not_capturing(st, where)) return s;
  const int B = kv.num_seqs, maxp = kv.max_pages_per_seq, P = kv.page_size;
  std::vector<int32_t> lens, first, table;
  if (s3r_status s = fetch(lens, kv.seq_lens, (size_t)B, st, where)) return s;
  if (s3r_status s = fetch(first, first_pos, (size_t)B, st, where)) return s;
  if (s3r_status s = fetch(table, kv.page_table, (size_t)B * maxp, st, where)) return s;
  for (int b = 0; b < B; ++b) {
    // The commit reads the entries of the pages it writes and of the pages up to
    // the committed tail, within the row; a negative entry is an unallocated page.
    const int64_t last_written = count > 0 ? ((int64_t)first[b] + count - 1) / P : -1;
    int64_t hi = pages_below(lens[b], P) - 1;
    if (last_written > hi) hi = last_written;
    if (hi > maxp - 1) hi = maxp - 1;
    for (int64_t j = 0; j <= hi; ++j) {
      const int32_t e = table[(size_t)b * maxp + j];
      if (kv.num_phys_pages > 0 && e >= kv.num_phys_pages) return bad_entry(where, b, j, e, kv.num_phys_pages);
    }
  }
  return S3R_OK;
}

s3r_status debug_check_tokens(const int32_t* tokens, int32_t num_seqs, int32_t gamma, int32_t vocab,
                              hipStream_t st, const char* where) {
  if (s3r_status s = not_capturing(st, where)) return s;
  std::vector<int32_t> t;
  if (s3r_status s = fetch(t, tokens, (size_t)num_seqs * gamma, st, where)) return s;
  for (size_t i = 0; i < t.size(); ++i) {
    if (t[i] < 0 || t[i] >= vocab) {
      fprintf(stderr, "libs3r S3R_DEBUG: %s: draft_tokens[%zu][%zu] = %d is outside the vocabulary [0, %d)\n",
              where, i / gamma, i % gamma, t[i], vocab);
      return S3R_ERR_INVALID_ARGUMENT;
    }
  }
  return S3R_OK;
}

}  // namespace s3r
