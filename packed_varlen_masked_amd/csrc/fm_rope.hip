// Rotary position embedding of packed q and k rows, in place, one launch for
// both tensors.
//
// Method (Unsloth packing blog, unsloth.ai, fused QK RoPE section): one
// kernel rotates Q and K; positions restart at 0 in every packed sample;
// the rotation runs in place; out = x cos + rotate_half(x) sin with
// rotate_half(x) = [-x2, x1] for the halves x1 = x[:D/2], x2 = x[D/2:], the
// tables repeated over both halves, and the backward is the same map with
// sin negated.
//
// Layout (this file's own): a thread owns V consecutive channels j..j+V-1
// of the first half of one (token, head) row and their partners j+D/2.. in
// the second half, V = 16 bytes of the storage type, so every access to x
// is one 16-byte load or store.  q rows come first, then k rows.  A thread
// finds its token's sample by binary search over cu_seqlens and reads the
// cos / sin row of the position (the same row serves every head of the
// token, so it is a cache hit after the first).
#include "fm_common.hpp"
#include "fm_internal.h"
#include "fm_api.h"

namespace fm {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint32_t pack_bf16(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

template <typename T>
__global__ __launch_bounds__(256) void fm_rope_kernel(RopeArgs a) {
    constexpr int V = 16 / (int)sizeof(T);           // channels per 16-byte access
    const int half = a.D / 2, cpr = half / V;        // chunks per row
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = t / cpr;
    const int ch = (int)(t - row * cpr);
    const int64_t rows_q = a.N * a.Hq;
    if (row >= rows_q + a.N * a.Hk) return;
    int64_t tok;
    char* base;
    if (row < rows_q) {
        tok = row / a.Hq;
        base = (char*)a.q + row * a.D * (int64_t)sizeof(T);
    } else {
        const int64_t r = row - rows_q;
        tok = r / a.Hk;
        base = (char*)a.k + r * a.D * (int64_t)sizeof(T);
    }
    int lo = 0, hi = a.B;   // the sample: cu[lo] <= tok < cu[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu[mid] <= tok) lo = mid; else hi = mid;
    }
    const int64_t pos = tok - a.cu[lo];
    if (pos < 0 || pos >= a.max_pos) {   // outside the tables (or cu_seqlens invalid): row left as is
        if (a.status) atomicOr(a.status, FM_STATUS_POS);
        return;
    }
    float c[V], s[V];
    const float4* cp = (const float4*)(a.cos_t + pos * half + ch * V);
    const float4* sp = (const float4*)(a.sin_t + pos * half + ch * V);
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
        const float4 cv = cp[i], sv = sp[i];
        c[4 * i] = cv.x; c[4 * i + 1] = cv.y; c[4 * i + 2] = cv.z; c[4 * i + 3] = cv.w;
        s[4 * i] = sv.x; s[4 * i + 1] = sv.y; s[4 * i + 2] = sv.z; s[4 * i + 3] = sv.w;
    }
    if (a.inverse) {
#pragma unroll
        for (int i = 0; i < V; ++i) s[i] = -s[i];
    }
    u32x4* p1 = (u32x4*)(base + (int64_t)ch * 16);
    u32x4* p2 = (u32x4*)(base + (int64_t)half * sizeof(T) + (int64_t)ch * 16);
    const u32x4 w1 = *p1, w2 = *p2;
    float x1[V], x2[V];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x1[2 * i] = lo16(w1[i]); x1[2 * i + 1] = hi16(w1[i]);
            x2[2 * i] = lo16(w2[i]); x2[2 * i + 1] = hi16(w2[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) { x1[i] = __uint_as_float(w1[i]); x2[i] = __uint_as_float(w2[i]); }
    }
    float y1[V], y2[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        y1[i] = x1[i] * c[i] - x2[i] * s[i];   // first half:  x1 cos + (-x2) sin
        y2[i] = x2[i] * c[i] + x1[i] * s[i];   // second half: x2 cos + x1 sin
    }
    u32x4 o1, o2;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { o1[i] = pack_bf16(y1[2 * i], y1[2 * i + 1]); o2[i] = pack_bf16(y2[2 * i], y2[2 * i + 1]); }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) { o1[i] = __float_as_uint(y1[i]); o2[i] = __float_as_uint(y2[i]); }
    }
    *p1 = o1;
    *p2 = o2;
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, hipStream_t s) {
    const int V = a.dtype == FM_BF16 ? 8 : 4;
    const int64_t threads = a.N * (int64_t)(a.Hq + a.Hk) * (a.D / 2 / V);
    if (threads == 0) return hipSuccess;
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (a.dtype == FM_BF16) hipLaunchKernelGGL(fm_rope_kernel<__bf16>, dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(fm_rope_kernel<float>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace fm
