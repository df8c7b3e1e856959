// N4: FlashMask forward attention, bf16 in / fp32 accumulate, head_dim 128,
// on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Method (PaddleNLP FlashMask article, m.nxbn.cn/news/70198): FlashAttention-2
// extended with the column-wise mask (§3): for each key block the tile class
// is derived from the block extrema (§3.1, §3.2); fully masked tiles are
// skipped, partially masked tiles are masked element by element, unmasked
// tiles take the plain path.  Skipping leaves every bit of the result
// unchanged (§3.3): a skipped tile would contribute p = 0 and alpha = 1.
// Tiling: Q tiles stay on chip and K/V tiles stream through LDS, S and P
// never reach HBM (Varlen-Packing technical document, www.gsyq.cn/news/432802,
// §1.3).
//
// Layout choices (this file's own):
//   * one workgroup = 4 waves = one 128-row q tile; wave w owns rows
//     32w..32w+31.  The kernel is persistent: workgroups pull items from the
//     longest-first work list with one atomic counter.
//   * scores are computed transposed, S^T = K Q^T, so that in the MFMA
//     result each lane holds ONE query (lane & 31) and 16 keys per 32x32
//     tile.  Row max / row sum are then per-lane reductions plus one swap
//     with lane ^ 32, and the output O^T = V^T P^T keeps that ownership, so
//     the online-softmax rescale of O is a per-lane scalar.
//   * the key order inside each 16-key group is permuted when K is written
//     to LDS (swap of bits 2 and 3 of the row index) so that the 8 keys a
//     lane holds for one PV k-step are contiguous in V^T: one 16-byte LDS
//     read per MFMA operand.
//   * V is transposed into LDS (V^T[d][key]) while it is staged.
#include <algorithm>

#include "fm_common.hpp"
#include "fm_internal.h"
#include "fm_api.h"

namespace fm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BR = 128, BC = 64, HD = 128, NTH = 256;
constexpr int KS = HD + 8;  // K row stride in LDS (bf16 elements); 272 B
constexpr int VS = BC + 8;  // V^T row stride in LDS (bf16 elements); 144 B
constexpr float LN2 = 0.69314718055994530942f;

struct Smem {
    uint16_t k[BC * KS];
    uint16_t vt[HD * VS];
    int32_t mv[4][BC];
    int32_t next;
};

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline int swap_bits23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
__device__ inline uint32_t bf16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Index of split partial (sequence b, q tile qt, split s, head h).
__device__ inline int64_t partial_index(const AttnArgs& a, int b, int qt, int s, int h, int Tc) {
    const int MS = (a.S > 0 && Tc > 0) ? ceil_div(Tc, a.S) : 1;
    return ((int64_t)a.sl_off[b] + (int64_t)qt * MS + s) * a.H + h;
}

// Normalise and write one lane's query row (called only for valid rows).
__device__ inline void store_row(const AttnArgs& a, int64_t qrow, int h, int hh,
                                 const float* vals /*64, MFMA order*/, float inv) {
    uint16_t* op = (uint16_t*)a.out + qrow * ((int64_t)a.H * HD) + (int64_t)h * HD + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float* v = vals + dt * 16 + g * 4;
            u32x2 w;
            w.x = bf16_bits(v[0] * inv) | (bf16_bits(v[1] * inv) << 16);
            w.y = bf16_bits(v[2] * inv) | (bf16_bits(v[3] * inv) << 16);
            *(u32x2*)(op + 32 * dt + 8 * g) = w;
        }
    }
}

__global__ __launch_bounds__(NTH, 2) void fm_attn_bf16_kernel(AttnArgs a) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
    const int n_items = __builtin_amdgcn_readfirstlane(*a.n_items);
    const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
    const uint16_t* __restrict__ K = (const uint16_t*)a.k;
    const uint16_t* __restrict__ V = (const uint16_t*)a.v;
    const int64_t rs = (int64_t)a.H * HD;  // token row stride (elements)
    const float sl2 = a.scale_log2;
    const bool no_skip = (a.flags & FM_FLAG_NO_SKIP) != 0;

    for (;;) {
        if (tid == 0) {
            const int it = atomicAdd(a.sched_counter, 1);
            // the launch's last fetch: every workgroup has fetched its
            // terminating index, so the counter can be reset for the next call
            if (it == n_items + (int)gridDim.x - 1) atomicExch(a.sched_counter, 0);
            sm.next = it;
        }
        __syncthreads();
        const int it = __builtin_amdgcn_readfirstlane(sm.next);
        if (it >= n_items) break;
        const int32_t* rec = a.items + (int64_t)it * ITEM_WORDS;
        const int b = rec[0], h = rec[1], qt = rec[2];
        const int kbb = rec[3], kbe = rec[4], sidx = rec[5], nsp = rec[6];
        const int s_b = a.cu[b], e_b = a.cu[b + 1];
        const int Tc = ceil_div(e_b - s_b, BC);
        const int r0 = s_b + qt * BR, r1 = min(r0 + BR, e_b);
        const int32_t* __restrict__ xb = a.extrema + (int64_t)a.kb_off[b] * 8;
        const int qrow = r0 + 32 * w + n;
        const int64_t hoff = (int64_t)h * HD;

        // Q^T fragments (B operand): lane holds query n, channels 16s+8hh..+7
        bf16x8 qf[8];
        if (qrow < r1) {
            const uint16_t* qp = Q + (int64_t)qrow * rs + hoff + 8 * hh;
#pragma unroll
            for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*(const u32x4*)(qp + 16 * s));
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
        }
        float m_run = -INFINITY, l_run = 0.f;
        f32x16 o[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;

        const int kb_lo = no_skip ? 0 : kbb, kb_hi = no_skip ? Tc : kbe;
        for (int kb = kb_lo; kb < kb_hi; ++kb) {
            const int c0 = s_b + kb * BC, c1 = min(c0 + BC, e_b);
            int x[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] = xb[(int64_t)kb * 8 + t];
            const TileInfo ti = classify_tile(r0, r1, c0, c1, x, a.causal);
            if (ti.causal_full) continue;
            if (ti.cls == CLS_FULL && !no_skip) continue;
            const bool ragged = (c1 - c0) < BC;
            const bool use_mv = ti.need_lt || ti.need_ut;

            __syncthreads();  // previous tile's LDS reads are done
            // ---- stage K (rows permuted) ----
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int id = i * NTH + tid;
                const int key = id >> 4, dch = id & 15;
                u32x4 val = {0, 0, 0, 0};
                if (c0 + key < c1) val = *(const u32x4*)(K + (int64_t)(c0 + key) * rs + hoff + 8 * dch);
                const int row = (key & 32) | swap_bits23(key & 31);
                *(u32x4*)&sm.k[row * KS + 8 * dch] = val;
            }
            // ---- stage V transposed: thread = (8-channel chunk, 4 keys) ----
            {
                const int dch = tid & 15, kg = tid >> 4;
                u32x4 r[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 4 * kg + i;
                    r[i] = u32x4{0, 0, 0, 0};
                    if (c0 + key < c1) r[i] = *(const u32x4*)(V + (int64_t)(c0 + key) * rs + hoff + 8 * dch);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int sh = 16 * (j & 1);
                    u32x2 wv;
                    wv.x = ((r[0][j >> 1] >> sh) & 0xFFFFu) | (((r[1][j >> 1] >> sh) & 0xFFFFu) << 16);
                    wv.y = ((r[2][j >> 1] >> sh) & 0xFFFFu) | (((r[3][j >> 1] >> sh) & 0xFFFFu) << 16);
                    *(u32x2*)&sm.vt[(8 * dch + j) * VS + 4 * kg] = wv;
                }
            }
            if (use_mv && tid < BC) {
                const int64_t col = (int64_t)c0 + tid;
                Vec4 f;
                if (col < c1) f = fill_column(a.sv, a.n_vec, a.causal, a.N, col);
                else f = Vec4{INT_MIN, INT_MAX, INT_MIN, INT_MAX};
                sm.mv[0][tid] = f.lts; sm.mv[1][tid] = f.lte;
                sm.mv[2][tid] = f.uts; sm.mv[3][tid] = f.ute;
            }
            __syncthreads();

            // ---- S^T = K Q^T : two 32-key tiles x 8 k-steps ----
            f32x16 sacc[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[t][e] = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const bf16x8 ka = as_bf16x8(*(const u32x4*)&sm.k[(32 * t + n) * KS + 16 * s + 8 * hh]);
                    sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], sacc[t], 0, 0, 0);
                }
            }
            // register e of tile t holds key 32t + 16(e>>3) + 8hh + (e&7)
            if (ti.cls != CLS_UNMASKED || ragged) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int kl = 32 * t + 16 * (e >> 3) + 8 * hh + (e & 7);
                        const int j = c0 + kl;
                        bool msk = false;
                        if (ti.need_causal) msk |= j > qrow;
                        if (ragged) msk |= j >= c1;
                        if (ti.need_lt) msk |= (sm.mv[0][kl] <= qrow) & (qrow < sm.mv[1][kl]);
                        if (ti.need_ut) msk |= (sm.mv[2][kl] <= qrow) & (qrow < sm.mv[3][kl]);
                        if (msk) sacc[t][e] = -INFINITY;
                    }
                }
            }
            // ---- online softmax (base 2, scale folded) ----
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[t][e]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run, mx * sl2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            float rsum = 0.f;
            bf16x8 pb[2][2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][8 * c + e], sl2, -m_use));
                        rsum += p;
                        pb[t][c][e] = (__bf16)p;
                    }
                }
            }
            rsum += __shfl_xor(rsum, 32, 64);
            l_run = l_run * alpha + rsum;
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
            // ---- O^T += V^T P^T ----
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        const bf16x8 va = as_bf16x8(*(const u32x4*)&sm.vt[(32 * dt + n) * VS + 32 * t + 16 * c + 8 * hh]);
                        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[t][c], o[dt], 0, 0, 0);
                    }
                }
            }
        }

        // ---- epilogue ----
        if (nsp == 1) {
            if (qrow < r1) {
                float vals[64];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) vals[dt * 16 + e] = o[dt][e];
                const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
                store_row(a, qrow, h, hh, vals, inv);
                if (hh == 0)
                    a.lse[(int64_t)h * a.N + qrow] = l_run > 0.f ? (m_run + __log2f(l_run)) * LN2 : -INFINITY;
            }
        } else {
            float* po = a.partial + partial_index(a, b, qt, sidx, h, Tc) * (int64_t)(BR * HD + 2 * BR);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) po[(w * 64 + dt * 16 + e) * 64 + lane] = o[dt][e];
            if (hh == 0) {
                po[BR * HD + 32 * w + n] = m_run;
                po[BR * HD + BR + 32 * w + n] = l_run;
            }
        }
        __syncthreads();  // all threads have read sm.next and finished with LDS
    }
}

// N5: merge of split partials, in split order (deterministic).  The item
// with split_idx 0 of every split (q tile, head) owns the merge.
__global__ __launch_bounds__(NTH) void fm_merge_bf16_kernel(AttnArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
    const int n_items = *a.n_items;
    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        const int32_t* rec = a.items + (int64_t)it * ITEM_WORDS;
        const int nsp = rec[6];
        if (rec[5] != 0 || nsp <= 1) continue;
        const int b = rec[0], h = rec[1], qt = rec[2];
        const int s_b = a.cu[b], e_b = a.cu[b + 1];
        const int Tc = ceil_div(e_b - s_b, BC);
        const int r0 = s_b + qt * BR, r1 = min(r0 + BR, e_b);
        const int qrow = r0 + 32 * w + n;
        const int64_t P = (int64_t)(BR * HD + 2 * BR);
        const float* p0 = a.partial + partial_index(a, b, qt, 0, h, Tc) * P;
        // consecutive splits of one q tile occupy consecutive slots
        const int64_t step = (int64_t)a.H * P;
        float m_all = -INFINITY;
        for (int s = 0; s < nsp; ++s) m_all = fmaxf(m_all, p0[s * step + BR * HD + 32 * w + n]);
        const float m_use = (m_all == -INFINITY) ? 0.f : m_all;
        float l_all = 0.f;
        float acc[64];
#pragma unroll
        for (int r = 0; r < 64; ++r) acc[r] = 0.f;
        for (int s = 0; s < nsp; ++s) {
            const float* ps = p0 + s * step;
            const float wgt = __builtin_amdgcn_exp2f(ps[BR * HD + 32 * w + n] - m_use);
            l_all += wgt * ps[BR * HD + BR + 32 * w + n];
#pragma unroll
            for (int r = 0; r < 64; ++r) acc[r] += wgt * ps[(w * 64 + r) * 64 + lane];
        }
        if (qrow < r1) {
            const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
            store_row(a, qrow, h, hh, acc, inv);
            if (hh == 0)
                a.lse[(int64_t)h * a.N + qrow] = l_all > 0.f ? (m_all + __log2f(l_all)) * LN2 : -INFINITY;
        }
    }
}

hipError_t launch_attn_bf16(const AttnArgs& a, int n_cu, hipStream_t s) {
    static int occ = 0;
    if (occ == 0) {
        int o = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, fm_attn_bf16_kernel, NTH, 0) != hipSuccess || o < 1) o = 1;
        occ = o;
    }
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(a.items_cap, (int64_t)n_cu * occ));
    hipLaunchKernelGGL(fm_attn_bf16_kernel, dim3((unsigned)grid), dim3(NTH), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.S <= 0) return e;
    const int64_t mgrid = std::max<int64_t>(1, std::min<int64_t>(a.items_cap, (int64_t)n_cu * 4));
    hipLaunchKernelGGL(fm_merge_bf16_kernel, dim3((unsigned)mgrid), dim3(NTH), 0, s, a);
    return hipGetLastError();
}

}  // namespace fm
