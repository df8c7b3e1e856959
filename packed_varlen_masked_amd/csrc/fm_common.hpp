// Device helpers shared by the plan kernels and the attention kernels.
// Sources: PaddleNLP FlashMask article (m.nxbn.cn/news/70198) §2.2 (vectors
// and defaults), §3.1 (extrema), §3.2 (tile classes).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>
#include "fm_internal.h"
#include "fm_api.h"

namespace fm {

enum : int { CLS_FULL = 0, CLS_PARTIAL = 1, CLS_UNMASKED = 2 };

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// The four logical vectors of key column `col` ([FM] §2.2): LTS and UTS
// default to 0, LTE and UTE to the query length (N here, since indices are
// global); causal calls keep only the lower triangle (UT = [0, 0), empty).
struct Vec4 { int lts, lte, uts, ute; };

__device__ inline Vec4 fill_column(const int32_t* __restrict__ sv, int n_vec, int causal,
                                   int64_t N, int64_t col) {
    Vec4 r;
    r.lts = sv[col];
    const int n32 = (int)N;
    if (causal) {
        r.lte = (n_vec == 2) ? sv[N + col] : n32;
        r.uts = 0; r.ute = 0;
    } else if (n_vec == 2) {
        r.lte = n32; r.uts = 0; r.ute = sv[N + col];
    } else {
        r.lte = sv[N + col]; r.uts = sv[2 * N + col]; r.ute = sv[3 * N + col];
    }
    return r;
}

// Tile class from one key block's extrema ([FM] §3.2).  Rows [r0, r1) and
// columns [c0, c1) are already clipped to the sequence; r1 is exclusive.
// `need` reports which element tests a visited tile must apply.
struct TileInfo {
    int cls;
    bool need_causal;   // causal tile reaching above the diagonal
    bool need_lt;       // lower-triangle interval may touch the tile
    bool need_ut;       // upper-triangle interval may touch the tile
    bool causal_full;   // fully masked by the causal rule alone
};

__host__ __device__ inline TileInfo classify_tile(int r0, int r1, int c0, int c1,
                                                  const int* x, int causal) {
    TileInfo t;
    const int lts_min = x[0], lts_max = x[1], lte_min = x[2], lte_max = x[3];
    const int uts_min = x[4], uts_max = x[5], ute_min = x[6], ute_max = x[7];
    t.causal_full = causal && (c0 >= r1);
    t.need_causal = causal && (c1 > r0 + 1);
    const bool lt_full = (r0 >= lts_max) && (r1 <= lte_min);
    t.need_lt = (r0 < lte_max) && (r1 > lts_min);
    const bool ut_full = !causal && (r0 >= uts_max) && (r1 <= ute_min);
    t.need_ut = !causal && (r0 < ute_max) && (r1 > uts_min);
    if (t.causal_full || lt_full || ut_full) t.cls = CLS_FULL;
    else if (t.need_causal || t.need_lt || t.need_ut) t.cls = CLS_PARTIAL;
    else t.cls = CLS_UNMASKED;
    return t;
}

// ---- dropout bits -------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 32x32->64 products and
// xors with the key, the key advancing by the Weyl constants between
// rounds.  The dropout byte of a pair (query row i, key j of a sequence
// starting at s) for head h is byte (j - s) & 15 of the four words for
// counter (i, (j - s) >> 4, h, offset) and key (seed lo, seed hi).
// WIDE: each product as one 32 x 32 -> 64 multiply (one instruction instead
// of separate high and low products; the same bits).
template <bool WIDE = false>
__device__ __attribute__((always_inline)) inline void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                                                    uint32_t& c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint32_t hi0, lo0, hi1, lo1;
        if constexpr (WIDE) {
            const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
            hi0 = (uint32_t)(p0 >> 32); lo0 = (uint32_t)p0;
            hi1 = (uint32_t)(p1 >> 32); lo1 = (uint32_t)p1;
        } else {
            hi0 = __umulhi(0xD2511F53u, c0); lo0 = 0xD2511F53u * c0;
            hi1 = __umulhi(0xCD9E8D57u, c2); lo1 = 0xCD9E8D57u * c2;
        }
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
}

// Dropout words of a 64-key block kb of a sequence for the query row of a
// lane whose S^T registers hold one query (the forward, dQ): w[b][x] is
// word 2x + hh of 16-key block 4kb + b, the words whose bytes are this
// lane's keys (register 8c + e of S^T tile t is key 32t + 16c + 8(e>>2) +
// 4hh + (e&3): block 2t + c, byte 8(e>>2) + 4hh + (e&3)).  Lane half hh
// computes blocks 2hh, 2hh + 1 and the two halves swap the words the other
// one needs.
struct DropW { uint32_t w[4][2]; };
template <bool WIDE = false>
__device__ __attribute__((always_inline)) inline DropW drop_words(uint32_t seed_lo, uint32_t seed_hi, uint32_t offset,
                                                                  int row, int kb, int h, int hh) {
    uint32_t own[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        uint32_t c0 = (uint32_t)row, c1 = (uint32_t)(4 * kb + 2 * hh + u), c2 = (uint32_t)h, c3 = offset;
        philox4x32_10<WIDE>(c0, c1, c2, c3, seed_lo, seed_hi);
        own[u][0] = c0; own[u][1] = c1; own[u][2] = c2; own[u][3] = c3;
    }
    DropW d;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const uint32_t mine = hh ? own[u][2 * x + 1] : own[u][2 * x];
            const uint32_t send = hh ? own[u][2 * x] : own[u][2 * x + 1];
            const auto r = __builtin_amdgcn_permlane32_swap(send, send, false, false);
            const uint32_t recv = hh ? r[0] : r[1];
            d.w[u][x] = hh ? recv : mine;
            d.w[2 + u][x] = hh ? mine : recv;
        }
    return d;
}

// ---- wave helpers (wave64) --------------------------------------------
// min / max over the 64 lanes with DPP (no LDS traffic): quad swaps, the
// half-row and row mirrors leave every lane of a row with its row's value;
// the row broadcasts 15 and 31 carry rows 0-2 into row 3, whose lane 63
// then holds the result for the whole wave.
__device__ inline int wave_min(int v) {
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xf, 0xf, false));    // quad_perm [1,0,3,2]
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xf, 0xf, false));    // quad_perm [2,3,0,1]
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));   // row_half_mirror
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false));   // row_mirror
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false));   // row_bcast:15 into rows 1, 3
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false));   // row_bcast:31 into rows 2, 3
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ inline int wave_max(int v) {
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false));
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ inline long long wave_sum64(long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ inline uint64_t lanemask_lt() {
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Block-wide exclusive scan of one int64 per thread (blockDim.x <= 1024).
// `tmp` must hold blockDim.x / 64 + 1 values.  Returns the exclusive prefix;
// *total receives the block sum.  Contains __syncthreads.
__device__ inline long long block_exclusive_scan(long long v, long long* tmp, long long* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    long long x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        long long y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) tmp[wid] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        long long run = 0;
        for (int w = 0; w < nw; ++w) { long long t = tmp[w]; tmp[w] = run; run += t; }
        tmp[nw] = run;
    }
    __syncthreads();
    long long r = tmp[wid] + x - v;
    *total = tmp[nw];
    __syncthreads();
    return r;
}

}  // namespace fm
