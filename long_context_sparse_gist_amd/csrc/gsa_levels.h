// Kernel arguments of the hierarchy of any depth (levels.hip).
#pragma once

#include "gsa_internal.h"

namespace gsa {

constexpr int kMaxLevels = 8;     // meta-gist levels above the gists
constexpr int kDescShift = 56;    // row descriptor: array id << 56 | element offset
constexpr int kChainCap = 8192;   // candidate rows the select chain keeps in LDS
constexpr int kChainSel = 4096;   // kept ids (all levels) the select chain keeps in LDS
constexpr int kFoldTop = 1024;    // largest top level the select chain scores itself
constexpr int kTopSplits = 64;    // workgroups per unit of the top-level pass
constexpr int kChainBt = 4096;    // block-table entries per sequence the select chain keeps in LDS

struct LvArgs {
    Args a;                       // shapes, q, caches, block table, lengths, partials, out
    int L;                        // meta-gist levels
    // per level l (index l; level 0 = the gists, whose arrays are the caches)
    const void* lk[kMaxLevels + 1];
    const void* lv[kMaxLevels + 1];
    int maxe[kMaxLevels + 1];     // entries per (batch, kv-head) row of the level's arrays
    int fan[kMaxLevels + 1];      // R_l: entries of level l-1 per entry of level l
    int topk[kMaxLevels + 1];     // k_l (topk[0]: the chunks unfolded)
    int32_t* sel[kMaxLevels + 1];   // [units][k_l] kept ids, ascending, -1 padded
    int32_t* usel[kMaxLevels + 1];  // the caller's copies, or null
    // lists
    int cap;                      // rows per (level, unit) of the key buffers
    float* keys;                  // [L+1][units][cap] routing keys of each level's list
    int32_t* cid;                 // [L+1][units][cap] entry ids of each candidate list (below the top)
    int chain_lds;                // the select chain keeps its lists in LDS (they fit)
    int fold_top;                 // the select chain scores the top level and the final list
                                  // holds its entries (no top-level launch; S_top = 0)
    int fcap;                     // rows per unit of the final list
    int64_t* fdesc;               // [units][fcap]
    int32_t* nfin;                // [units]
    unsigned* uctr;               // [units] arrival counters of the final attention's
                                  // workgroups (zero between calls), or null: merge launch
    int S_top, S_fin, NS;         // splits of the top level and the final list; partial slots
};

hipError_t launch_levels(const LvArgs& A, hipStream_t st);

}  // namespace gsa
