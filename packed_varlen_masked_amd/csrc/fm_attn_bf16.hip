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
// Layout and schedule (this file's own):
//   * one workgroup = 8 waves = one 256-row q tile; wave w owns rows
//     32w..32w+31.  Every staged K/V tile feeds 256 query rows, which halves
//     the global->LDS traffic per MFMA against 128-row tiles.  The kernel is persistent: workgroups pull items from the
//     longest-first work list with one atomic counter.
//   * scores are computed transposed, S^T = K Q^T, so that in the MFMA
//     result each lane holds ONE query (lane & 31) and 16 keys per 32x32
//     tile.  Row max / row sum are per-lane reductions plus one exchange
//     with lane ^ 32, and O^T = V^T P^T keeps that ownership, so the
//     online-softmax rescale of O is a per-lane scalar.
//   * K and V tiles sit row-major in LDS ([key][channel], rows padded to
//     272 B).  The V^T operand is read with the gfx950 LDS transpose read
//     (ds_read_b64_tr_b16): each 16-lane group receives a 16-channel x
//     4-key block with one channel per lane.
//   * two LDS buffers: the global loads of the next visited tile are issued
//     before the current tile's MFMAs and written to the other buffer after
//     them, so HBM/L2 latency hides behind the matrix work.
//   * long rows are split over several items; each writes an fp32 partial
//     (O, m, l) and the last one to finish merges all partials in split
//     order (deterministic), then resets its counter.
#include <algorithm>

#include "fm_common.hpp"
#include "fm_internal.h"
#include "fm_api.h"

namespace fm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BR = 256, BC = 64, HD = 128;
constexpr int NW = 8, NTH = 64 * NW;    // 8 waves, 32 query rows each
constexpr float LN2 = 0.69314718055994530942f;
constexpr int PART = BR * HD + 2 * BR;  // floats per split partial: O row-major, then m, l
// Lazy rescale: the running row max used for the exponentials moves only when
// a new score exceeds it by more than 2^RESCALE_LOG2 (p then stays <= 2^8,
// exact in the final normalisation, and O is rescaled rarely).
constexpr float RESCALE_LOG2 = 8.0f;

// LDS tiles, rows padded so that every fragment address is one base register
// plus an immediate offset and reads are free of bank conflicts (64 banks):
//   K: 272-byte rows (17 chunks of 16 B): 16 consecutive rows of one chunk
//      fall in 16 distinct 4-bank groups;
//   V: 320-byte rows (20 chunks): the transpose read of 4 consecutive rows x
//      4 consecutive chunks per 32 lanes falls in 16 distinct 4-bank groups.
constexpr int KCH = 17, VCH = 20;                  // 16-byte chunks per row
constexpr int KBYTES = BC * KCH * 16;              // 17408
constexpr int VBYTES = BC * VCH * 16;              // 20480
constexpr int BUFBYTES = KBYTES + VBYTES;          // one K/V buffer
constexpr int KBLK = KBYTES / 1024, VBLK = VBYTES / 1024;   // 1 KB load blocks: 17, 20

// Asynchronous global -> LDS loads of one K/V tile into buffer `buf`.  A
// wave instruction writes 1 KB of LDS in lane order (16 B per lane); lane L of
// block blk fills chunk q = 64*blk + L of the tile, i.e. row q / CH, chunk
// q % CH.  Wave w issues blocks w, w+4, ...: q grows by 256 per block, so the
// lane's (row, chunk) advances by a fixed step and the address is a uniform
// tile base plus a 32-bit lane offset.  Padding
// chunks load chunk 0 of their row (never read).  Rows past the sequence end
// read its last valid key (finite data, masked out later), so every address
// stays inside the tensor.
__device__ __attribute__((always_inline)) inline void tile_issue(
    char* kdst, char* vdst, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, int64_t rs,
    int64_t hoff, int c0, int c1, int w, int lane) {
    const int last = c1 - 1 - c0;                       // last valid row of the tile
    const char* kt = (const char*)(K + (int64_t)c0 * rs + hoff);
    const char* vt = (const char*)(V + (int64_t)c0 * rs + hoff);
    const uint32_t rsb = (uint32_t)(rs * 2);            // row stride in bytes
    // wave w issues blocks w, w + NW, ...: the chunk index q grows by 64 * NW
    // per block, i.e. (row, chunk) advances by (KSTEP_R, KSTEP_C)
    constexpr int QS = 64 * NW;
    constexpr int KSTEP_R = QS / KCH, KSTEP_C = QS % KCH;
    constexpr int VSTEP_R = QS / VCH, VSTEP_C = QS % VCH;
    const int q = 64 * w + lane;
    int r = q / KCH, c = q - r * KCH;
#pragma unroll
    for (int i = 0; i < (KBLK + NW - 1) / NW; ++i) {
        if (NW * i + w < KBLK) {
            const uint32_t off = (uint32_t)min(r, last) * rsb + 16u * (uint32_t)(c < 16 ? c : 0);
            __builtin_amdgcn_global_load_lds((const void*)(kt + off), (lds_void*)(kdst + (NW * i + w) * 1024), 16, 0, 0);
        }
        c += KSTEP_C; r += KSTEP_R;
        if (c >= KCH) { c -= KCH; r += 1; }
    }
    r = q / VCH; c = q - r * VCH;
#pragma unroll
    for (int i = 0; i < (VBLK + NW - 1) / NW; ++i) {
        if (NW * i + w < VBLK) {
            const uint32_t off = (uint32_t)min(r, last) * rsb + 16u * (uint32_t)(c < 16 ? c : 0);
            __builtin_amdgcn_global_load_lds((const void*)(vt + off), (lds_void*)(vdst + (NW * i + w) * 1024), 16, 0, 0);
        }
        c += VSTEP_C; r += VSTEP_R;
        if (c >= VCH) { c -= VCH; r += 1; }
    }
}

__device__ __attribute__((always_inline)) inline void stage_mv(const AttnArgs& a, int32_t* mv, int c0, int c1,
                                                               int tid) {
    if (tid < BC) {
        const int64_t col = (int64_t)c0 + tid;
        const Vec4 f = col < c1 ? fill_column(a.sv, a.n_vec, a.causal, a.N, col)
                                : Vec4{INT_MIN, INT_MAX, INT_MIN, INT_MAX};
        mv[tid] = f.lts; mv[BC + tid] = f.lte; mv[2 * BC + tid] = f.uts; mv[3 * BC + tid] = f.ute;
    }
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Combine a per-lane value with the one of lane ^ 32 (the other half of the
// same query row) using the gfx950 lane swap: every lane receives both halves
// in the same order, so both copies of the row statistics stay identical.
__device__ inline float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline uint32_t bf16_bits(float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ inline int64_t partial_index(const AttnArgs& a, int b, int qt, int s, int h, int Tc) {
    const int MS = (a.S > 0 && Tc > 0) ? ceil_div(Tc, a.S) : 1;
    return ((int64_t)a.sl_off[b] + (int64_t)qt * MS + s) * a.H + h;
}

struct Item {
    int b, h, qt, kbb, kbe, sidx, nsp;
    int s_b, e_b, Tc, r0, r1, kb_hi;
    int64_t hoff;
    const int32_t* xb;
};

// Visit and interval bits of a window of up to 64 key blocks [base, base+64),
// one bit per block, from one vector load of the extrema per lane and two
// ballots (FlashMask article §3.2 rules): the KV loop does no lookups.
struct Win {
    int base;
    uint64_t visit, iv;
};

__device__ __attribute__((always_inline)) inline void load_window(Win& W, const AttnArgs& a, const Item& I,
                                                                  int base, bool no_skip, int lane) {
    const int kb = base + lane;
    bool v = false, iv = false;
    if (kb < I.kb_hi) {
        const u32x4 x0 = *(const u32x4*)(I.xb + (int64_t)kb * 8);
        const u32x4 x1 = *(const u32x4*)(I.xb + (int64_t)kb * 8 + 4);
        const int x[8] = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                          (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        const int c0 = I.s_b + kb * BC, c1 = min(c0 + BC, I.e_b);
        const TileInfo ti = classify_tile(I.r0, I.r1, c0, c1, x, a.causal);
        v = !ti.causal_full && (ti.cls != CLS_FULL || no_skip);
        iv = ti.need_lt || ti.need_ut;
    }
    W.base = base;
    W.visit = __ballot(v);
    W.iv = __ballot(iv);
}

// First visited key block at or after kb (loading windows as needed); *iv
// receives whether its interval vectors must be applied element-wise.
__device__ __attribute__((always_inline)) inline int next_visit(Win& W, const AttnArgs& a, const Item& I,
                                                                int kb, bool no_skip, int lane, bool* iv) {
    for (;;) {
        if (kb >= I.kb_hi) return I.kb_hi;
        if (kb >= W.base + 64) load_window(W, a, I, kb, no_skip, lane);
        const uint64_t m = W.visit >> (kb - W.base);
        if (m) {
            kb += __builtin_ctzll(m);
            *iv = (W.iv >> (kb - W.base)) & 1;
            return kb;
        }
        kb = W.base + 64;
    }
}

struct State {
    float m_run, l_run;
    f32x16 o[4];
};

// One key block, computed from `cur` while the next visited block streams
// into `nxt`.  Returns the next visited key block (*niv: its interval flag).
__device__ __attribute__((always_inline)) inline int kv_step(
    const AttnArgs& a, const Item& I, Win& W, int kb, bool iv, bool* niv, const char* kbase, const char* vbase,
    const int32_t* cmv, char* nk, char* nv, int32_t* nmv,
    const bf16x8 (&qf)[8], State& st, bool no_skip, int tid, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int64_t rs) {
    const int lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
    const int grp = lane >> 4, gi = lane & 15;
    const int c0 = I.s_b + kb * BC, c1 = min(c0 + BC, I.e_b);
    const bool ragged = (c1 - c0) < BC;
    const bool causal = a.causal && (c1 > I.r0 + 1);   // tile reaches above the diagonal
    const float sl2 = a.scale_log2;
    const int qrow = I.r0 + 32 * w + n;

    // ---- prefetch the next visited tile (asynchronous, straight to LDS) ----
    const int nkb = next_visit(W, a, I, kb + 1, no_skip, lane, niv);
    if (nkb < I.kb_hi) {
        const int nc0 = I.s_b + nkb * BC, nc1 = min(nc0 + BC, I.e_b);
        tile_issue(nk, nv, K, V, rs, I.hoff, nc0, nc1, w, lane);
        if (*niv) stage_mv(a, nmv, nc0, nc1, tid);
    }

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
            const bf16x8 ka = as_bf16x8(*(const u32x4*)(kbase + (32 * t + n) * (KCH * 16) + 32 * s + 16 * hh));
            sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], sacc[t], 0, 0, 0);
        }
    }
    // ---- element masks; register e of tile t holds key 32t + 8(e>>2) + 4hh + (e&3) ----
    if (causal || ragged || iv) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int kl0 = 32 * t + 8 * g + 4 * hh;
                int4 lts, lte, uts, ute;
                if (iv) {
                    lts = *(const int4*)&cmv[kl0];
                    lte = *(const int4*)&cmv[BC + kl0];
                    uts = *(const int4*)&cmv[2 * BC + kl0];
                    ute = *(const int4*)&cmv[3 * BC + kl0];
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = c0 + kl0 + q;
                    bool msk = (causal && j > qrow) || (ragged && j >= c1);
                    if (iv) {
                        const int s0 = q == 0 ? lts.x : q == 1 ? lts.y : q == 2 ? lts.z : lts.w;
                        const int e0 = q == 0 ? lte.x : q == 1 ? lte.y : q == 2 ? lte.z : lte.w;
                        const int s1 = q == 0 ? uts.x : q == 1 ? uts.y : q == 2 ? uts.z : uts.w;
                        const int e1 = q == 0 ? ute.x : q == 1 ? ute.y : q == 2 ? ute.z : ute.w;
                        msk |= ((s0 <= qrow) & (qrow < e0)) | ((s1 <= qrow) & (qrow < e1));
                    }
                    if (msk) sacc[t][4 * g + q] = -INFINITY;
                }
            }
        }
    }
    // ---- online softmax (base 2, scale folded, lazy rescale) ----
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[t][e]);
    mx = halves_max(mx) * sl2;
    if (__any(mx > st.m_run + RESCALE_LOG2)) {
        const float m_new = fmaxf(st.m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(st.m_run - (m_new == -INFINITY ? 0.f : m_new));
        st.l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.o[dt][e] *= alpha;
        st.m_run = m_new;
    }
    const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;
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
    st.l_run += halves_sum(rsum);
    // ---- O^T += V^T P^T ; V^T read with the LDS transpose read ----
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // lane part of the address: rows 4hh + gi/4, chunk 2(grp&1) + (gi&3)/2, half gi&1
            const char* vl = vbase + (4 * hh + (gi >> 2)) * (VCH * 16) +
                             16 * (2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const char* p = vl + (32 * t + 16 * c) * (VCH * 16) + 64 * dt;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(void*)p);
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(void*)(p + 8 * VCH * 16));
                const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[t][c], st.o[dt], 0, 0, 0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next tile's LDS writes have landed
    __syncthreads();
    return nkb;
}

__global__ __launch_bounds__(NTH, 2) void fm_attn_bf16_kernel(AttnArgs a) {
    static_assert(NTH / 64 == NW && BR == 32 * NW, "one wave per 32 query rows");
    // two K/V buffers as distinct LDS objects, so that the compiler can tell
    // the tile being read from the one being loaded asynchronously
    __shared__ __attribute__((aligned(1024))) char k0[KBYTES];
    __shared__ __attribute__((aligned(1024))) char v0[VBYTES];
    __shared__ __attribute__((aligned(1024))) char k1[KBYTES];
    __shared__ __attribute__((aligned(1024))) char v1[VBYTES];
    __shared__ __attribute__((aligned(16))) int32_t mv0[4 * BC];
    __shared__ __attribute__((aligned(16))) int32_t mv1[4 * BC];
    __shared__ __attribute__((aligned(16))) int32_t s_rec[ITEM_WORDS];
    __shared__ int32_t s_next;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
    const int n_items = __builtin_amdgcn_readfirstlane(*a.n_items);
    const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
    const uint16_t* __restrict__ K = (const uint16_t*)a.k;
    const uint16_t* __restrict__ V = (const uint16_t*)a.v;
    const int64_t rs = (int64_t)a.H * HD;
    const bool no_skip = (a.flags & FM_FLAG_NO_SKIP) != 0;

    // Work fetch: every fetch returns the next index; a workgroup stops at its
    // first index >= n_items.  The launch's last fetch (index
    // n_items + gridDim.x - 1) resets the counter for the next call.  The
    // next item's index and record are fetched while the current item's first
    // tile loads, and handed over through LDS when the item ends.
    const int last_fetch = n_items + (int)gridDim.x - 1;
    if (tid == 0) {
        const int v = atomicAdd(a.sched_counter, 1);
        if (v == last_fetch) atomicExch(a.sched_counter, 0);
        s_next = v;
    }
    __syncthreads();
    int it = __builtin_amdgcn_readfirstlane(s_next);
    if (it < n_items && tid < ITEM_WORDS) s_rec[tid] = a.items[(int64_t)it * ITEM_WORDS + tid];
    __syncthreads();
    while (it < n_items) {
        int nxt = 0;
        if (tid == 0) nxt = atomicAdd(a.sched_counter, 1);   // consumed below, after the tile loads issue
        Item I;
        I.b = s_rec[0]; I.h = s_rec[1]; I.qt = s_rec[2]; I.kbb = s_rec[3]; I.kbe = s_rec[4];
        I.sidx = s_rec[5]; I.nsp = s_rec[6];
        I.s_b = s_rec[8]; I.e_b = s_rec[9];
        const int kb_base = s_rec[10], slot0 = s_rec[11];
        I.Tc = ceil_div(I.e_b - I.s_b, BC);
        I.r0 = I.s_b + I.qt * BR; I.r1 = min(I.r0 + BR, I.e_b);
        I.xb = a.extrema + (int64_t)kb_base * 8;
        I.hoff = (int64_t)I.h * HD;
        I.kb_hi = no_skip ? I.Tc : I.kbe;
        const int qrow = I.r0 + 32 * w + n;

        // first tile (kb_begin is visited by construction of the work list),
        // Q fragments and the first flag window go out together
        Win W;
        W.base = INT_MIN / 2;
        W.visit = 0;
        W.iv = 0;
        bool iv = false, niv = false;
        int kb = no_skip ? I.kb_hi : I.kbb;
        if (no_skip) kb = next_visit(W, a, I, 0, no_skip, lane, &iv);
        if (kb < I.kb_hi) {
            const int c0 = I.s_b + kb * BC, c1 = min(c0 + BC, I.e_b);
            tile_issue(k0, v0, K, V, rs, I.hoff, c0, c1, w, lane);
        }
        // Q^T fragments (B operand): lane holds query n, channels 16s+8hh..+7
        bf16x8 qf[8];
        if (qrow < I.r1) {
            const uint16_t* qp = Q + (int64_t)qrow * rs + I.hoff + 8 * hh;
#pragma unroll
            for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*(const u32x4*)(qp + 16 * s));
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
        }
        // next item's record: waits only for the fetch issued first, not for
        // the tile and Q loads behind it
        int nrec = 0;
        if (w == 0) {
            nxt = __builtin_amdgcn_readfirstlane(nxt);
            if (nxt == last_fetch && lane == 0) atomicExch(a.sched_counter, 0);
            if (nxt < n_items && lane < ITEM_WORDS) nrec = a.items[(int64_t)nxt * ITEM_WORDS + lane];
        }
        if (kb < I.kb_hi) {
            if (!no_skip) {
                load_window(W, a, I, kb, no_skip, lane);
                iv = W.iv & 1;
            }
            if (iv) {
                const int c0 = I.s_b + kb * BC;
                stage_mv(a, mv0, c0, min(c0 + BC, I.e_b), tid);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        State st;
        st.m_run = -INFINITY; st.l_run = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.o[dt][e] = 0.f;
        while (kb < I.kb_hi) {
            kb = kv_step(a, I, W, kb, iv, &niv, k0, v0, mv0, k1, v1, mv1, qf, st, no_skip, tid, K, V, rs);
            if (kb >= I.kb_hi) break;
            kb = kv_step(a, I, W, kb, niv, &iv, k1, v1, mv1, k0, v0, mv0, qf, st, no_skip, tid, K, V, rs);
        }

        // ---- epilogue: normalised bf16 row, or the fp32 partial of a split row ----
        const int lr = 32 * w + n;
        if (I.nsp > 1) {
            float* po = a.partial + ((int64_t)(slot0 + I.sidx) * a.H + I.h) * PART;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *(float4*)(po + lr * HD + 32 * dt + 8 * g + 4 * hh) =
                        float4{st.o[dt][4 * g], st.o[dt][4 * g + 1], st.o[dt][4 * g + 2], st.o[dt][4 * g + 3]};
            if (hh == 0) { po[BR * HD + lr] = st.m_run; po[BR * HD + BR + lr] = st.l_run; }
        } else if (qrow < I.r1) {
            const float l = st.l_run;
            const float inv = l > 0.f ? 1.f / l : 0.f;
            uint16_t* op = (uint16_t*)a.out + (int64_t)qrow * rs + I.hoff + 4 * hh;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 wv;
                    wv.x = bf16_bits(st.o[dt][4 * g] * inv) | (bf16_bits(st.o[dt][4 * g + 1] * inv) << 16);
                    wv.y = bf16_bits(st.o[dt][4 * g + 2] * inv) | (bf16_bits(st.o[dt][4 * g + 3] * inv) << 16);
                    *(u32x2*)(op + 32 * dt + 8 * g) = wv;
                }
            if (hh == 0) a.lse[(int64_t)I.h * a.N + qrow] = l > 0.f ? (st.m_run + __log2f(l)) * LN2 : -INFINITY;
        }
        __syncthreads();  // every wave is done with s_rec and the LDS buffers
        if (w == 0) {
            if (lane < ITEM_WORDS) s_rec[lane] = nrec;
            if (lane == 0) s_next = nxt;
        }
        __syncthreads();
        it = __builtin_amdgcn_readfirstlane(s_next);
    }
}

// N5: merge of split partials in split order (deterministic).  Task =
// (split row group, 8-row slab); thread = (row of the slab, 4 channels).
constexpr int MNTH = 256, MROWS = MNTH / 32;

__global__ __launch_bounds__(MNTH) void fm_merge_bf16_kernel(AttnArgs a) {
    const int n_items = *a.n_items;
    const int tid = threadIdx.x, lr0 = tid >> 5, dq = (tid & 31) * 4;
    const int n_tasks = n_items * (BR / MROWS);
    for (int task = blockIdx.x; task < n_tasks; task += gridDim.x) {
        const int it = task / (BR / MROWS), slab = task % (BR / MROWS);
        const int32_t* rec = a.items + (int64_t)it * ITEM_WORDS;
        const int nsp = rec[6];
        if (rec[5] != 0 || nsp <= 1) continue;
        const int h = rec[1], qt = rec[2], s_b = rec[8], e_b = rec[9], slot0 = rec[11];
        const int lr = slab * MROWS + lr0;
        const int64_t qrow = (int64_t)s_b + qt * BR + lr;
        if (qrow >= e_b) continue;
        const float* p0 = a.partial + ((int64_t)slot0 * a.H + h) * PART;
        const int64_t step = (int64_t)a.H * PART;
        // all m first (independent loads), then one pass over the splits
        float m_all = -INFINITY;
#pragma unroll 4
        for (int s = 0; s < nsp; ++s) m_all = fmaxf(m_all, p0[s * step + BR * HD + lr]);
        const float m_use = (m_all == -INFINITY) ? 0.f : m_all;
        float l_all = 0.f;
        float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int s = 0; s < nsp; ++s) {
            const float* ps = p0 + s * step;
            const float ms = ps[BR * HD + lr], ls = ps[BR * HD + BR + lr];
            const float4 v = *(const float4*)(ps + lr * HD + dq);
            const float wgt = __builtin_amdgcn_exp2f(ms - m_use);
            l_all += wgt * ls;
            acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
        }
        const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
        uint16_t* op = (uint16_t*)a.out + qrow * ((int64_t)a.H * HD) + (int64_t)h * HD + dq;
        u32x2 wv;
        wv.x = bf16_bits(acc.x * inv) | (bf16_bits(acc.y * inv) << 16);
        wv.y = bf16_bits(acc.z * inv) | (bf16_bits(acc.w * inv) << 16);
        *(u32x2*)op = wv;
        if (dq == 0) a.lse[(int64_t)h * a.N + qrow] = l_all > 0.f ? (m_all + __log2f(l_all)) * LN2 : -INFINITY;
    }
}

hipError_t launch_attn_bf16(const AttnArgs& a, int n_cu, hipStream_t s) {
    static int occ = 0;
    if (occ == 0) {
        int o = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, fm_attn_bf16_kernel, NTH, 0) != hipSuccess || o < 1)
            o = 1;
        occ = o;
    }
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(a.items_cap, (int64_t)n_cu * occ));
    hipLaunchKernelGGL(fm_attn_bf16_kernel, dim3((unsigned)grid), dim3(NTH), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.S <= 0) return e;
    const int64_t mgrid = std::max<int64_t>(1, std::min<int64_t>(a.items_cap * (BR / MROWS), (int64_t)n_cu * 8));
    hipLaunchKernelGGL(fm_merge_bf16_kernel, dim3((unsigned)mgrid), dim3(MNTH), 0, s, a);
    return hipGetLastError();
}

}  // namespace fm
