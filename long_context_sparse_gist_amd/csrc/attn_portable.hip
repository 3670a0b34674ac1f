// Portable attention over a token list: plain fp32 VALU arithmetic, any
// dtype, GQA group size up to 16, head_dim up to 128.  It serves the fp32
// caches and is the cross-check for the MFMA kernels; it produces the same
// per-split partials (max in the exp2 domain, sum, weighted V sum).
#include "gsa_lists.h"

namespace gsa {
namespace {

constexpr int kTB = 64;  // tokens per workgroup

template <typename T> __device__ inline float ldf(const T* p, size_t i);
template <> __device__ inline float ldf<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ inline float ldf<__bf16>(const __bf16* p, size_t i) { return (float)p[i]; }

template <typename T>
__global__ __launch_bounds__(256) void attn_portable_kernel(Args a, int kind, int hier) {
    __shared__ float qs[16][128];
    __shared__ float z[16][kTB];
    __shared__ float pmax[16];
    __shared__ size_t roff[kTB];
    __shared__ int rmeta[kTB];

    const int u = blockIdx.y;
    const int split = blockIdx.x;
    ListCtx c;
    make_ctx(a, kind, u, hier != 0, c);
    const int p0 = split * kTB;
    const int count = min(kTB, c.len - p0);
    if (count <= 0) return;
    const int G = a.G, D = a.D, tid = threadIdx.x;
    const bool want_keys = kind != kListUnfolded;
    const bool want_attn = kind == kListUnfolded || kind == kListMeta ||
                           (kind == kListGists && !(a.flags & kFlagSelectedGists));

    const T* q = (const T*)a.q + ((size_t)c.b * a.Hq + (size_t)c.g * G) * D;
    for (int e = tid; e < G * D; e += blockDim.x) qs[e / D][e % D] = ldf(q, e);
    if (tid < count) {
        const void *kb, *vb;
        roff[tid] = list_row(a, kind, c, hier != 0, p0 + tid, &kb, &vb);
        rmeta[tid] = kind == kListMeta;
    }
    __syncthreads();

    for (int e = tid; e < G * count; e += blockDim.x) {
        int h = e / count, t = e - h * count;
        const T* kr = (const T*)(rmeta[t] ? a.km : a.kc) + roff[t];
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc += qs[h][d] * ldf(kr, d);
        z[h][t] = acc;
    }
    __syncthreads();

    if (want_keys && tid < count) {
        float S = 0.f;
        for (int h = 0; h < G; ++h) S += z[h][tid];
        S *= a.tau;
        int p = p0 + tid;
        if (kind == kListGists && a.hlog)  // per-head logits for the sum-of-probabilities key
            for (int h = 0; h < G; ++h) a.hlog[((size_t)u * G + h) * a.key_stride + p] = z[h][tid] * a.tau;
        if (kind == kListGists) {
            a.keys[(size_t)u * a.key_stride + p] = S;
        } else if (kind == kListMeta) {
            a.mkeys[(size_t)u * a.max_meta + p] = S;
        } else {
            a.ckeys[(size_t)u * a.cand_stride + p] = S;
            a.cand[(size_t)u * a.cand_stride + p] = cand_gist(a, c, p);
        }
    }
    if (!want_attn) return;

    if (tid < G) {
        float m = -INFINITY;
        for (int t = 0; t < count; ++t) m = fmaxf(m, z[tid][t]);
        pmax[tid] = m * a.tau_log2e;
    }
    __syncthreads();
    for (int e = tid; e < G * count; e += blockDim.x) {
        int h = e / count, t = e - h * count;
        z[h][t] = exp2f(z[h][t] * a.tau_log2e - pmax[h]);
    }
    __syncthreads();

    const int slot = partial_slot(a, kind, split);
    const size_t pbase = ((size_t)u * a.NS + slot) * G;
    for (int e = tid; e < G * D; e += blockDim.x) {
        int h = e / D, d = e - h * D;
        float acc = 0.f;
        for (int t = 0; t < count; ++t) {
            const T* vr = (const T*)(rmeta[t] ? a.vm : a.vc) + roff[t];
            acc += z[h][t] * ldf(vr, d);
        }
        a.part_acc[(pbase + h) * D + d] = acc;
    }
    if (tid < G) {
        float l = 0.f;
        for (int t = 0; t < count; ++t) l += z[tid][t];
        a.part_ml[pbase + tid] = make_float2(pmax[tid], l);
    }
}

}  // namespace

int portable_tokens_per_block() { return kTB; }

hipError_t launch_attn_portable(const Args& a, int kind, int splits, hipStream_t st) {
    dim3 grid(splits, a.B * a.Hkv);
    int hier = a.km != nullptr;
    if (a.dtype == 0)
        hipLaunchKernelGGL((attn_portable_kernel<float>), grid, dim3(256), 0, st, a, kind, hier);
    else
        hipLaunchKernelGGL((attn_portable_kernel<__bf16>), grid, dim3(256), 0, st, a, kind, hier);
    return hipGetLastError();
}

}  // namespace gsa
