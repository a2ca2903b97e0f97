// Host-side work decomposition of the split-KV forward (fa_fwd_splitkv): how many key ranges
// each (sequence, kv head, 32-row block) is split into, the grid of the split kernel and the
// size of the partials workspace. Plain C++: no device code, so the validation layer of the
// library (this file and fa_api.cpp) also builds and runs under host sanitizers.
#include <algorithm>
#include <cstdint>

#include "fa.h"
#include "fa_launch.h"

namespace fa {

SplitPlan plan_splitkv(const fa_fwd_params& p, int32_t num_splits) {
  SplitPlan plan;
  const bool varlen = p.cu_seqlens != nullptr;
  const int64_t groups = varlen ? p.num_seqs : p.batch;
  const int64_t group = p.heads_q / p.heads_kv;
  const int64_t rows = varlen ? p.max_seqlen : p.seqlen;  // query tokens per sequence, at most
  plan.rowblocks = (group * rows + kSplitBlockRows - 1) / kSplitBlockRows;
  int64_t splits = num_splits;
  if (splits == 0) {
    // The LDS of all CUs holds three workgroups of the split kernel per CU, 768 at once. Each
    // workgroup pays a pipeline fill (its first tiles' full memory latency), so with equal
    // keys per sequence one round of equal workgroups is best (measured: 1 round 189 us, 2
    // rounds 201 us, 4 rounds 221 us for 16 sequences x 8 kv heads x 16K keys). Packed
    // sequences of unequal lengths take two rounds: the split kernel starts the longest
    // sequences' splits first and the short splits fill in behind them. At least four tiles
    // (128 keys) per split.
    constexpr int64_t kResident = 256 * 3;
    const int64_t rounds = varlen ? 2 : 1;
    const int64_t units = std::max<int64_t>(groups * p.heads_kv * plan.rowblocks, 1);
    const int64_t keys = varlen ? (int64_t(p.seqlen_k) + groups - 1) / groups : p.seqlen_k;
    const int64_t tiles = (keys + kSplitTileKeys - 1) / kSplitTileKeys;
    splits = (kResident * rounds + units - 1) / units;
    splits = std::min(splits, std::max<int64_t>(tiles / 4, 1));
    splits = std::min<int64_t>(std::max<int64_t>(splits, 1), FA_MAX_SPLITS);
  }
  plan.splits = int32_t(splits);
  plan.items = splits * p.heads_kv * groups;
  plan.grid = (plan.items + 7) / 8 * 8 * plan.rowblocks;
  plan.rows_total = int64_t(p.batch) * p.heads_q * p.seqlen;
  plan.workspace_bytes =
      splits == 1 ? 0 : uint64_t(splits) * uint64_t(plan.rows_total) * uint64_t(p.head_dim + 1) * 4u;
  return plan;
}

}  // namespace fa
