// Online-softmax merge of the per-split partials of one unit into the output
// (the exact combination of softmax partials over disjoint token sets, the
// merge the Pulsar Attention page applies across hosts in its phase 2):
//     M = max_i m_i,  lambda = sum_i l_i 2^(m_i - M),
//     out = (sum_i acc_i 2^(m_i - M)) / lambda
// with m_i in the exp2 domain.  An empty attention set gives a zero output.
// One workgroup per (head, unit); 4 slot groups x 64 column pairs, each slot
// group folding its slots in one streaming pass (running maximum, rescaled).
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
    const bool col = 2 * lane < D;

    // one streaming pass per slot group (slots sg, sg + 4, ...): a running
    // maximum, normaliser and column pair, rescaled as the maximum grows (the
    // loads of consecutive slots are independent, so they are in flight
    // together); then the four groups are combined
    constexpr int kBatch = 16;  // slots of a group loaded before they are folded
    float m = -INFINITY, l = 0.f;
    float2 o = make_float2(0.f, 0.f);
    for (int i0 = sg; i0 < ns; i0 += kBatch * kSlotGroups) {
        float2 v[kBatch], x[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = i0 + kSlotGroups * k;
            v[k] = make_float2(-INFINITY, 0.f);
            x[k] = make_float2(0.f, 0.f);
            if (i < ns) {
                const size_t s = (size_t)slot(i);
                v[k] = ml[s * G + h];
                if (col) x[k] = *(const float2*)(acc + (s * G + h) * D + 2 * lane);
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (v[k].x == -INFINITY) continue;  // an empty split (or none)
            const float mn = fmaxf(m, v[k].x);
            const float fo = m == -INFINITY ? 0.f : exp2f(m - mn);
            const float fv = exp2f(v[k].x - mn);
            l = l * fo + v[k].y * fv;
            o.x = o.x * fo + x[k].x * fv;
            o.y = o.y * fo + x[k].y * fv;
            m = mn;
        }
    }
    if (lane == 0) s_m[sg] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    const float f = m == -INFINITY ? 0.f : exp2f(m - M);
    if (lane == 0) s_l[sg] = l * f;
    red[sg][lane] = make_float2(o.x * f, o.y * f);
    __syncthreads();
    if (sg == 0 && col) {
        const float lam = s_l[0] + s_l[1] + s_l[2] + s_l[3];
        float2 t = red[0][lane];
        for (int j = 1; j < kSlotGroups; ++j) {
            t.x += red[j][lane].x;
            t.y += red[j][lane].y;
        }
        const float inv = (M != -INFINITY && lam > 0.f) ? 1.f / lam : 0.f;
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
