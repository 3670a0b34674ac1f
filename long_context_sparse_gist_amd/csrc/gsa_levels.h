// Kernel arguments of the hierarchy of any depth (levels.hip).
#pragma once

#include "gsa_internal.h"

namespace gsa {

constexpr int kMaxLevels = 8;     // meta-gist levels above the gists
constexpr int kDescShift = 56;    // row descriptor: array id << 56 | element offset

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
    int cap;                      // rows per unit of the key / candidate buffers
    float* keys;                  // [units][cap] routing keys of the current list
    int32_t* cid[2];              // [units][cap] ids of the candidate lists (ping-pong)
    int64_t* desc[2];             // [units][cap] their row descriptors
    int32_t* ncand[2];            // [units] their lengths
    int fcap;                     // rows per unit of the final list
    int64_t* fdesc;               // [units][fcap]
    int32_t* nfin;                // [units]
    int S_top, S_cand, S_fin, NS; // splits of the top level, candidate lists, final list; partial slots
};

hipError_t launch_levels(const LvArgs& A, hipStream_t st);

}  // namespace gsa
