// plan_rule.h -- integer rules of the split planner, shared by the host twin
// (mla_api.cpp) and the device planner kernel (mla_kernels.hip) so that both
// produce the same plan.
//
// Range rule: the TileLang MLA guide's paged variant cuts each sequence by
// blocks_per_split / remaining_blocks ("Split-KV" item of its optimisation
// list).  Here a sequence of L rows has nb = ceil(L / 64) blocks; split k of s
// takes floor(nb / s) blocks, plus one more when k < nb mod s, in order.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define MLA_HD __host__ __device__ __forceinline__
#else
#define MLA_HD inline
#endif

namespace mla {

constexpr int kSplitBlockRows = 64;
constexpr int kMaxSplits = 1024;
constexpr int kHeadsPerGroup = 128;

MLA_HD int32_t ceil_div(int32_t a, int32_t b) { return (int32_t)(((int64_t)a + b - 1) / b); }
// ceil(a / b) for 0 <= a < 2^30 and 1 <= b < 2^30, in 32-bit unsigned
// arithmetic: the planner's inner loops run on every wave of the split kernel,
// where a 64-bit divide expands to a long instruction sequence.
MLA_HD int32_t ceil_div_small(int32_t a, int32_t b) {
  return (int32_t)(((uint32_t)a + (uint32_t)b - 1u) / (uint32_t)b);
}

MLA_HD int32_t clamp_len(int32_t L, int32_t cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

MLA_HD int32_t num_blocks(int32_t L) { return L <= 0 ? 0 : ceil_div(L, kSplitBlockRows); }

// Rows [*r0, *r1) of split k out of s for a sequence of L rows.
MLA_HD void split_range(int32_t L, int32_t s, int32_t k, int32_t* r0, int32_t* r1) {
  const int32_t nb = num_blocks(L);
  const int32_t per = nb / s, rem = nb % s;
  const int32_t first = k * per + (k < rem ? k : rem);
  const int32_t n = per + (k < rem ? 1 : 0);
  const int64_t a = (int64_t)first * kSplitBlockRows, b = (int64_t)(first + n) * kSplitBlockRows;
  *r0 = (int32_t)(a < L ? a : L);
  *r1 = (int32_t)(b < L ? b : L);
}

// Several query tokens (seqlen_q = s > 1).  Query token t sees rows
// j < L - (s - 1 - t), so the last s - 1 rows are seen by some tokens only.
// The prefix, cut by the planner's splits, ends at the last multiple of 32 at
// or below L - (s - 1) (every token sees it; a 32-row boundary keeps every
// tile inside one page); the rest, at most 31 + 15 rows, forms two tail
// splits of one tile each (the second may be empty), the only tiles whose
// rows the kernel masks per query row.
constexpr int kMaxSeqlenQ = 16;
constexpr int kTailAlign = 32;

MLA_HD int32_t tail_splits(int32_t seqlen_q) { return seqlen_q > 1 ? 2 : 0; }

MLA_HD int32_t prefix_len(int32_t L, int32_t seqlen_q) {
  if (seqlen_q <= 1) return L;
  const int32_t seen_by_all = L > seqlen_q - 1 ? L - (seqlen_q - 1) : 0;
  return seen_by_all / kTailAlign * kTailAlign;
}

// Rows [*r0, *r1) of split k of a sequence of L rows with s_pre prefix splits
// (splits s_pre and s_pre + 1, present when seqlen_q > 1, are the tails).
MLA_HD void seq_split_range(int32_t L, int32_t seqlen_q, int32_t s_pre, int32_t k, int32_t* r0, int32_t* r1) {
  const int32_t Lp = prefix_len(L, seqlen_q);
  const int32_t mid = Lp + kTailAlign < L ? Lp + kTailAlign : L;
  if (k < s_pre) {
    split_range(Lp, s_pre, k, r0, r1);
  } else if (k == s_pre) {
    *r0 = Lp;
    *r1 = mid;
  } else {
    *r0 = mid;
    *r1 = L;
  }
}

// Splits given to a sequence of nb blocks when each work item may take up to t blocks.
MLA_HD int32_t splits_for_budget(int32_t nb, int32_t t) {
  int32_t s = nb <= 0 ? 1 : ceil_div_small(nb, t);   // nb <= 2^25 blocks, 1 <= t <= nb
  return s > kMaxSplits ? kMaxSplits : s;
}

MLA_HD int32_t head_groups(int32_t heads) { return ceil_div(heads, kHeadsPerGroup); }

// Most prefix splits the planner may emit (planner mode): one work item per
// CU and head group, at least one per sequence.  The tail splits (one tile
// each) come on top, except that when they are at most a quarter of the
// budget they are taken out of it: otherwise a few of them push the
// workgroups just past one per CU, and on the XCDs where the extra one is a
// full-length prefix split it waits for a whole second round.
MLA_HD int32_t planner_cap(int32_t batch, int32_t heads, int32_t num_cus, int32_t seqlen_q) {
  int32_t per_group = ceil_div(num_cus, head_groups(heads));
  const int32_t tails = batch * tail_splits(seqlen_q);
  if (tails > 0 && 4 * tails <= per_group) per_group -= tails;
  return batch > per_group ? batch : per_group;
}

// Most work items (splits, the tails included) of a plan.
MLA_HD int64_t max_splits(int32_t batch, int32_t heads, int32_t num_split, int32_t num_cus, int32_t seqlen_q) {
  const int64_t per_seq_extra = tail_splits(seqlen_q);
  if (num_split > 0) return (int64_t)batch * (num_split + per_seq_extra);
  return (int64_t)planner_cap(batch, heads, num_cus, seqlen_q) + (int64_t)batch * per_seq_extra;
}

}  // namespace mla
