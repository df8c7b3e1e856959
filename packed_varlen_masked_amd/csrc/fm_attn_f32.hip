// N4 (fp32 reference path): the same FlashMask forward in fp32 storage and
// arithmetic, one wave per work item, one lane per query row (Br <= 64),
// any Bc <= 64.  It exists for exact small-shape checks (e.g. the 16x16
// worked example of the PaddleNLP FlashMask article §2.2 with the 4x4 tiles
// of its §3.2 figure), not for speed.
//
// Per tile ([FM] §3.2): FULL tiles are skipped, PARTIAL tiles are masked
// element by element, UNMASKED tiles take no mask work; online softmax in
// base 2 with the scale folded in.
#include <algorithm>

#include "fm_common.hpp"
#include "fm_internal.h"
#include "fm_api.h"

namespace fm {

constexpr float LN2f = 0.69314718055994530942f;

template <int D>
__global__ __launch_bounds__(64) void fm_attn_f32_kernel(AttnArgs a) {
    extern __shared__ float smem[];  // K tile [Bc][D] then V tile [Bc][D]
    float* sk = smem;
    float* sv_ = smem + a.Bc * D;
    const int Br = a.Br, Bc = a.Bc, tid = threadIdx.x;
    const int n_items = *a.n_items;
    const float* __restrict__ Qp = (const float*)a.q;
    const float* __restrict__ Kp = (const float*)a.k;
    const float* __restrict__ Vp = (const float*)a.v;
    float* __restrict__ Op = (float*)a.out;
    const int64_t rs = (int64_t)a.H * D;
    const float sl2 = a.scale_log2;
    const bool no_skip = (a.flags & FM_FLAG_NO_SKIP) != 0;
    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        const int32_t* rec = a.items + (int64_t)it * ITEM_WORDS;
        const int b = rec[0], h = rec[1], qt = rec[2], kbb = rec[3], kbe = rec[4];
        const int s_b = a.cu[b], e_b = a.cu[b + 1];
        const int Tc = ceil_div(e_b - s_b, Bc);
        const int r0 = s_b + qt * Br, r1 = min(r0 + Br, e_b);
        const int i = r0 + tid;
        const bool active = tid < Br && i < r1;
        const int32_t* __restrict__ xb = a.extrema + (int64_t)a.kb_off[b] * 8;
        float q[D], o[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            q[d] = active ? Qp[(int64_t)i * rs + (int64_t)h * D + d] : 0.f;
            o[d] = 0.f;
        }
        float m_run = -INFINITY, l_run = 0.f;
        const int lo = no_skip ? 0 : kbb, hi = no_skip ? Tc : kbe;
        for (int kb = lo; kb < hi; ++kb) {
            const int c0 = s_b + kb * Bc, c1 = min(c0 + Bc, e_b);
            int x[8];
            for (int t = 0; t < 8; ++t) x[t] = xb[(int64_t)kb * 8 + t];
            const TileInfo ti = classify_tile(r0, r1, c0, c1, x, a.causal);
            if (ti.causal_full) continue;
            if (ti.cls == CLS_FULL && !no_skip) continue;
            __syncthreads();
            for (int idx = tid; idx < Bc * D; idx += 64) {
                const int key = idx / D, d = idx - key * D;
                const bool ok = c0 + key < c1;
                const int64_t g = (int64_t)(c0 + key) * rs + (int64_t)h * D + d;
                sk[idx] = ok ? Kp[g] : 0.f;
                sv_[idx] = ok ? Vp[g] : 0.f;
            }
            __syncthreads();
            if (!active) continue;
            const bool masked_tile = ti.cls != CLS_UNMASKED;
            // pass 1: scores -> tile max
            float mx = -INFINITY;
            for (int jj = 0; jj < c1 - c0; ++jj) {
                const int j = c0 + jj;
                bool msk = false;
                if (masked_tile) {
                    if (ti.need_causal) msk |= j > i;
                    if (ti.need_lt || ti.need_ut) {
                        const Vec4 f = fill_column(a.sv, a.n_vec, a.causal, a.N, j);
                        if (ti.need_lt) msk |= (f.lts <= i) && (i < f.lte);
                        if (ti.need_ut) msk |= (f.uts <= i) && (i < f.ute);
                    }
                }
                if (msk) continue;
                float dot = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) dot = __builtin_fmaf(q[d], sk[jj * D + d], dot);
                mx = fmaxf(mx, dot * sl2);
            }
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m_run - m_use);
            float rsum = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] *= alpha;
            // pass 2: probabilities and P V
            for (int jj = 0; jj < c1 - c0; ++jj) {
                const int j = c0 + jj;
                bool msk = false;
                if (masked_tile) {
                    if (ti.need_causal) msk |= j > i;
                    if (ti.need_lt || ti.need_ut) {
                        const Vec4 f = fill_column(a.sv, a.n_vec, a.causal, a.N, j);
                        if (ti.need_lt) msk |= (f.lts <= i) && (i < f.lte);
                        if (ti.need_ut) msk |= (f.uts <= i) && (i < f.ute);
                    }
                }
                if (msk) continue;
                float dot = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) dot = __builtin_fmaf(q[d], sk[jj * D + d], dot);
                const float p = exp2f(__builtin_fmaf(dot, sl2, -m_use));
                rsum += p;
#pragma unroll
                for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, sv_[jj * D + d], o[d]);
            }
            l_run = l_run * alpha + rsum;
            m_run = m_new;
        }
        if (active) {
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) Op[(int64_t)i * rs + (int64_t)h * D + d] = o[d] * inv;
            a.lse[(int64_t)h * a.N + i] = l_run > 0.f ? (m_run + log2f(l_run)) * LN2f : -INFINITY;
        }
        __syncthreads();
    }
}

hipError_t launch_attn_f32(const AttnArgs& a, int n_cu, hipStream_t s) {
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(a.items_cap, (int64_t)n_cu * 8));
    const size_t lds = (size_t)2 * a.Bc * a.D * sizeof(float);
    switch (a.D) {
        case 32: hipLaunchKernelGGL(fm_attn_f32_kernel<32>, dim3((unsigned)grid), dim3(64), lds, s, a); break;
        case 64: hipLaunchKernelGGL(fm_attn_f32_kernel<64>, dim3((unsigned)grid), dim3(64), lds, s, a); break;
        case 128: hipLaunchKernelGGL(fm_attn_f32_kernel<128>, dim3((unsigned)grid), dim3(64), lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fm
