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
