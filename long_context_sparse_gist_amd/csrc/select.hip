// Standalone per-unit top-k select kernel (one workgroup per unit) for the
// multi-launch paths; the selection itself is block_topk.
#include "gsa_lists.h"
#include "gsa_select.h"

namespace gsa {
namespace {

constexpr int kThreads = 512;

__global__ __launch_bounds__(kThreads) void select_kernel(Args a, int mode) {
    __shared__ SelectSmem<kThreads> sh;
    const int u = blockIdx.x;
    ListCtx c;
    make_ctx(a, mode == kSelCand ? kListCand : kListGists, u, mode != kSelGists, c);
    if (mode == kSelGists) {
        // scores past the sequence's gists read -inf
        float* kw = a.keys + (size_t)u * a.key_stride;
        for (int i = c.n + threadIdx.x; i < a.num_chunks; i += kThreads) kw[i] = -INFINITY;
        block_topk<kThreads>(a.keys + (size_t)u * a.key_stride, nullptr, c.n, a.top_k,
                             a.sel + (size_t)u * a.top_k, false, sh);
    } else if (mode == kSelMeta) {
        block_topk<kThreads>(a.mkeys + (size_t)u * a.max_meta, nullptr, c.nm, a.top_k_meta,
                             a.sel_meta + (size_t)u * a.top_k_meta, false, sh);
    } else {
        block_topk<kThreads>(a.ckeys + (size_t)u * a.cand_stride,
                             a.cand + (size_t)u * a.cand_stride, c.len, a.top_k,
                             a.sel + (size_t)u * a.top_k, false, sh);
    }
}

}  // namespace

hipError_t launch_select(const Args& a, int mode, hipStream_t st) {
    hipLaunchKernelGGL(select_kernel, dim3(a.B * a.Hkv), dim3(kThreads), 0, st, a, mode);
    return hipGetLastError();
}

}  // namespace gsa
