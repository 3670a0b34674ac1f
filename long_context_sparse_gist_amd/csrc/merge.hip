// Online-softmax merge of the per-split partials of one unit into the output
// (the exact combination of softmax partials over disjoint token sets, the
// merge the Pulsar Attention page applies across hosts in its phase 2):
//     M = max_i m_i,  lambda = sum_i l_i 2^(m_i - M),
//     out = (sum_i acc_i 2^(m_i - M)) / lambda
// with m_i in the exp2 domain.  An empty attention set gives a zero output.
// One workgroup per (head, unit); 4 slot groups x 64 column pairs.
#include "gsa_lists.h"

namespace gsa {
namespace {

constexpr int kSlotGroups = 4;

template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(Args a, int hier) {
    __shared__ float2 red[kSlotGroups][64];
    __shared__ float s_m[kSlotGroups], s_l[kSlotGroups];
    const int h = blockIdx.x, u = blockIdx.y;
    ListCtx c;
    make_ctx(a, kListUnfolded, u, hier != 0, c);
    const int len1 = hier ? c.nm : ((a.flags & kFlagSelectedGists) ? 0 : c.n);
    const int n1 = (len1 + a.SL - 1) / a.SL;
    const int n2 = (c.len + a.SR - 1) / a.SR;
    const int ns = n1 + n2;
    const int G = a.G, D = a.D;
    const float2* ml = a.part_ml + (size_t)u * a.NS * G;
    const float* acc = a.part_acc + (size_t)u * a.NS * G * D;
    auto slot = [&](int i) { return i < n1 ? i : a.S1 + (i - n1); };
    const int sg = threadIdx.x >> 6, lane = threadIdx.x & 63;

    // maximum and normaliser of head h
    float m = -INFINITY;
    for (int i = threadIdx.x; i < ns; i += blockDim.x) m = fmaxf(m, ml[(size_t)slot(i) * G + h].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) s_m[sg] = m;
    __syncthreads();
    float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float l = 0.f;
    if (M != -INFINITY)
        for (int i = threadIdx.x; i < ns; i += blockDim.x) {
            float2 v = ml[(size_t)slot(i) * G + h];
            l += v.y * exp2f(v.x - M);
        }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) s_l[sg] = l;
    __syncthreads();
    const float lam = s_l[0] + s_l[1] + s_l[2] + s_l[3];

    // weighted column sums: thread (sg, lane) owns columns 2*lane, 2*lane+1
    float2 o = make_float2(0.f, 0.f);
    if (M != -INFINITY && 2 * lane < D) {
#pragma unroll 8
        for (int i = sg; i < ns; i += kSlotGroups) {
            size_t s = (size_t)slot(i);
            float sc = exp2f(ml[s * G + h].x - M);
            float2 v = *(const float2*)(acc + (s * G + h) * D + 2 * lane);
            o.x += v.x * sc;
            o.y += v.y * sc;
        }
    }
    red[sg][lane] = o;
    __syncthreads();
    if (sg == 0 && 2 * lane < D) {
        float2 t = red[0][lane];
        for (int j = 1; j < kSlotGroups; ++j) { t.x += red[j][lane].x; t.y += red[j][lane].y; }
        float inv = (M != -INFINITY) ? 1.f / lam : 0.f;
        T* out = (T*)a.out + ((size_t)c.b * a.Hq + (size_t)c.g * G + h) * D;
        out[2 * lane] = (T)(t.x * inv);
        out[2 * lane + 1] = (T)(t.y * inv);
    }
}

}  // namespace

hipError_t launch_merge(const Args& a, int hier, hipStream_t st) {
    dim3 grid(a.G, a.B * a.Hkv);
    if (a.dtype == 0)
        hipLaunchKernelGGL((merge_kernel<float>), grid, dim3(256), 0, st, a, hier);
    else
        hipLaunchKernelGGL((merge_kernel<__bf16>), grid, dim3(256), 0, st, a, hier);
    return hipGetLastError();
}

}  // namespace gsa
