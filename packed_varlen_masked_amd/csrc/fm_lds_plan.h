// In-workgroup planner of the fused bf16 path: every workgroup of the
// attention launch rebuilds the whole plan of a small problem in LDS
// (block extrema, tile classes, visit lists, split chunks and their
// longest-first order) from cu_seqlens and the mask vectors, then runs its
// own items.  No launch and no global round trip separates planning from
// attention, and no workgroup waits for another.  One workgroup also writes
// the plan into the workspace in exactly the layout the separate planning
// kernels produce: the last one, which gets the shortest items of the
// longest-first order, or none.
//
// Method: PaddleNLP FlashMask article (m.nxbn.cn/news/70198) §3.1 (per-key-
// block min/max of LTS/LTE/UTS/UTE), §3.2 (FULL / PARTIAL / UNMASKED tile
// classes); work named by (sequence, head, q tile) as in the Varlen-Packing
// technical document (www.gsyq.cn/news/432802) §2, ordered longest first.
#pragma once
#include "fm_common.hpp"
#include "fm_internal.h"

namespace fm {

// Capacities (checked on the host before the fused path is chosen, and
// again here: a violation sets FM_STATUS_CAP and produces no items).
constexpr int LP_MAX_B = 255;          // sequences
constexpr int LP_MAX_SV = 16384;       // stored mask values (n_vec * N) staged in LDS
constexpr int LP_MAX_KB = 512;         // key blocks
constexpr int LP_MAX_ROWS = 512;       // q tiles
constexpr int LP_MAX_SLOTS = 1024;     // split chunks (work items per head)
constexpr int LP_MAX_TILES = 8192;     // tiles = visit-list capacity
constexpr int LP_MAX_MY = 16;          // items per workgroup

// Byte offsets of the planner's temporaries inside the (not yet used) K/V
// ring; everything is dead once the plan is built.
constexpr int LP_SEQ_INTS = 256;                                   // >= LP_MAX_B + 1
constexpr int LP_OFF_CU = 0;
constexpr int LP_OFF_KBOFF = LP_OFF_CU + 4 * LP_SEQ_INTS;
constexpr int LP_OFF_ROWOFF = LP_OFF_KBOFF + 4 * LP_SEQ_INTS;
constexpr int LP_OFF_TILEOFF = LP_OFF_ROWOFF + 4 * LP_SEQ_INTS;
constexpr int LP_OFF_SLOTBASE = LP_OFF_TILEOFF + 4 * LP_SEQ_INTS;
constexpr int LP_OFF_EXT = LP_OFF_SLOTBASE + 4 * LP_SEQ_INTS;     // int[LP_MAX_KB][8]
constexpr int LP_OFF_SLOTAT = LP_OFF_EXT + 32 * LP_MAX_KB;        // int[LP_MAX_SLOTS]: slot at each rank
constexpr int LP_OFF_KEY = LP_OFF_SLOTAT + 4 * LP_MAX_SLOTS;      // uint64[LP_MAX_SLOTS]: sort key per slot
constexpr int LP_OFF_SINFO = LP_OFF_KEY + 8 * LP_MAX_SLOTS;       // int4[LP_MAX_SLOTS]: chunk per slot
constexpr int LP_OFF_RANK = LP_OFF_SINFO + 16 * LP_MAX_SLOTS;     // int[LP_MAX_SLOTS]: rank per slot
constexpr int LP_OFF_SV = LP_OFF_RANK + 4 * LP_MAX_SLOTS;         // int[LP_MAX_SV]
constexpr int LP_TMP_BYTES = LP_OFF_SV + 4 * LP_MAX_SV;

struct LdsPlan {
    int status;   // 0, or FM_STATUS_* bits
    int n_items;
    int n_my;     // items of this workgroup, in s_myrec[0 .. n_my)
};

// Inclusive prefix sum across the 64 lanes of a wave with DPP row shifts
// and row broadcasts (no LDS traffic).
__device__ inline int wave_incl_scan(int v, int /*lane*/) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return v;
}

// min / max over aligned groups of 8 lanes (DPP quad permutes, then the
// half-row mirror): every lane of the group receives the result.
__device__ inline int min8(int x) {
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false));    // quad_perm [1,0,3,2]
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false));    // quad_perm [2,3,0,1]
    return min(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xf, 0xf, false));   // row_half_mirror
}
__device__ inline int max8(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false));
    return max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xf, 0xf, false));
}

// Index of the last entry <= x of an ascending int array of n + 1 entries
// (the owner of element x in a prefix-sum table); arr[0] <= x < arr[n].
__device__ inline int owner_of(const int* arr, int n, int x) {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (arr[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// Builds the plan of the call in LDS.  Tiles: Br query rows x Bc keys with
// Bc == 64 (one key block per wave of 64 lanes in the classification).
// `tmp` = LP_TMP_BYTES of LDS, `vis` = LP_MAX_TILES visit entries (key block
// | interval flag << 15, per q tile a run at the q tile's tile offset),
// `myrec` = LP_MAX_MY item records of this workgroup (word 12 = offset of
// the item's visits in `vis`).  Every thread of the workgroup must call it.
template <int Br, int Bc>
__device__ LdsPlan plan_in_lds(const AttnArgs& a, char* tmp, uint16_t* vis, int32_t (*myrec)[ITEM_WORDS]) {
    static_assert(Bc == 64, "one key block per wave");
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
    const int B = a.B, S = a.S, H = a.H;
    const int64_t N = a.N;
    int* t_cu = (int*)(tmp + LP_OFF_CU);
    int* t_kboff = (int*)(tmp + LP_OFF_KBOFF);
    int* t_rowoff = (int*)(tmp + LP_OFF_ROWOFF);
    int* t_tileoff = (int*)(tmp + LP_OFF_TILEOFF);
    int* t_slotbase = (int*)(tmp + LP_OFF_SLOTBASE);
    int* t_ext = (int*)(tmp + LP_OFF_EXT);
    int* t_slot_at = (int*)(tmp + LP_OFF_SLOTAT);
    uint64_t* t_key = (uint64_t*)(tmp + LP_OFF_KEY);
    int4* t_sinfo = (int4*)(tmp + LP_OFF_SINFO);
    int* t_rank = (int*)(tmp + LP_OFF_RANK);
    int* t_sv = (int*)(tmp + LP_OFF_SV);
    __shared__ int s_misc[8];   // status, FULL, PARTIAL, UNMASKED counts, split rows, filled slots
    __shared__ long long s_scan[17];
    int32_t* hdr = a.w_hdr;
    const bool writer = blockIdx.x == gridDim.x - 1;   // writes the plan to the workspace

    // ---- sequences: cu, validation, per-sequence prefix sums ----
    if (tid < 8) s_misc[tid] = 0;
    if (B > LP_MAX_B) {   // host bound violated
        if (writer && tid == 0) {
            hdr[HDR_STATUS] = FM_STATUS_CAP; hdr[HDR_NKB] = 0; hdr[HDR_NITEMS] = 0; hdr[HDR_SCHED] = 0;
            hdr[HDR_NSLOTS] = 0; hdr[HDR_NMERGE] = 0;
        }
        return LdsPlan{FM_STATUS_CAP, 0, 0};
    }
    // cu first, then the stored mask vectors (SoA [n_vec][N], contiguous)
    // into registers: the sequence prefix sums below run while the vector
    // loads are in flight (one memory round trip: LP_MAX_SV values are at
    // most 8 loads of 16 bytes per thread)
    constexpr int U = LP_MAX_SV / 4 / 512;
    static_assert(U * 4 * 512 == LP_MAX_SV, "one staging round covers the capacity");
    const int nsv = a.n_vec * (int)N;
    const bool sv_fits = nsv <= LP_MAX_SV && blockDim.x == 512;
    const bool sv16 = ((uintptr_t)a.sv & 15) == 0;
    const int n4 = sv16 ? (nsv >> 2) : 0;   // 16-byte loads; the rest one by one
    for (int i = tid; i <= B; i += blockDim.x) t_cu[i] = a.cu[i];
    int4 rv[U];
    int r1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { rv[u] = int4{0, 0, 0, 0}; r1[u] = 0; }
    if (sv_fits) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = u * 512 + tid;
            if (i < n4) rv[u] = ((const int4*)a.sv)[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = 4 * n4 + u * 512 + tid;
            if (i < nsv && i < 4 * n4 + U * 512) r1[u] = a.sv[i];
        }
    }
    __syncthreads();
    if (tid == 0) {
        const int bad = (t_cu[0] != 0 ? FM_STATUS_CU0 : 0) | (t_cu[B] != (int)N ? FM_STATUS_CUN : 0);
        if (bad) atomicOr(&s_misc[0], bad);
    }
    for (int b = tid; b < B; b += blockDim.x)
        if (t_cu[b + 1] < t_cu[b]) atomicOr(&s_misc[0], FM_STATUS_ORDER);
    if (wid == 0) {
        int ckb = 0, crow = 0, ctile = 0, cslot = 0;
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int b = b0 + lane;
            int tc = 0, tr = 0, ms = 0;
            if (b < B) {
                const int L = max(t_cu[b + 1] - t_cu[b], 0);
                tc = L ? ceil_div(L, Bc) : 0;
                tr = L ? ceil_div(L, Br) : 0;
                ms = (S > 0 && tc > 0) ? ceil_div(tc, S) : 1;
                // sizes beyond the capacities only matter once validated: clamp
                // so that the sums below cannot overflow
                tc = min(tc, LP_MAX_TILES); tr = min(tr, LP_MAX_TILES); ms = min(ms, LP_MAX_TILES);
            }
            const int i_kb = wave_incl_scan(tc, lane), i_row = wave_incl_scan(tr, lane);
            const int i_tile = wave_incl_scan(tr * tc, lane), i_slot = wave_incl_scan(tr * ms, lane);
            if (b < B) {
                t_kboff[b] = ckb + i_kb - tc; t_rowoff[b] = crow + i_row - tr;
                t_tileoff[b] = ctile + i_tile - tr * tc; t_slotbase[b] = cslot + i_slot - tr * ms;
            }
            ckb += __shfl(i_kb, 63, 64); crow += __shfl(i_row, 63, 64);
            ctile += __shfl(i_tile, 63, 64); cslot += __shfl(i_slot, 63, 64);
        }
        if (lane == 0) { t_kboff[B] = ckb; t_rowoff[B] = crow; t_tileoff[B] = ctile; t_slotbase[B] = cslot; }
    }
    if (sv_fits) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = u * 512 + tid;
            if (i < n4) ((int4*)t_sv)[i] = rv[u];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = 4 * n4 + u * 512 + tid;
            if (i < nsv && i < 4 * n4 + U * 512) t_sv[i] = r1[u];
        }
        // an unaligned vector array: the values past the first round
        for (int i = 4 * n4 + U * 512 + tid; i < nsv; i += 512) t_sv[i] = a.sv[i];
    }
    __syncthreads();
    const int n_kb = t_kboff[B], R = t_rowoff[B], n_tiles = t_tileoff[B], n_std = t_slotbase[B];
    int status = s_misc[0];
    if (!status && (!sv_fits || n_kb > LP_MAX_KB || R > LP_MAX_ROWS ||
                    n_tiles > LP_MAX_TILES || n_std > LP_MAX_SLOTS))
        status = FM_STATUS_CAP;
    if (writer && tid == 0) {
        hdr[HDR_STATUS] = status;
        hdr[HDR_NKB] = status ? 0 : n_kb;
        hdr[HDR_SCHED] = 0;
    }
    if (writer)
        for (int b = tid; b <= B; b += blockDim.x) a.w_kb_off[b] = status ? 0 : t_kboff[b];
    if (status) {
        if (writer && tid == 0) {
            hdr[HDR_NITEMS] = 0; hdr[HDR_NSLOTS] = 0; hdr[HDR_NMERGE] = 0;
            a.w_counts[0] = a.w_counts[1] = a.w_counts[2] = 0;
        }
        return LdsPlan{status, 0, 0};
    }

    // ---- block extrema (§3.1): 8 threads per key block, 8 columns each,
    // combined across the 8 lanes; the column order is rotated by the block
    // so that the lanes of a wave hit distinct banks.  Stored vector behind
    // each logical vector (LTS, LTE, UTS, UTE) for the accepted (n_vec,
    // causal) pairs; absent ones take their default (LTE: N; UTS, UTE: 0).
    // The sort keys and rank counters of the split slots are reset here too.
    const int n32 = (int)N;
    const int src[4] = {0, (a.n_vec == 4 || (a.causal && a.n_vec == 2)) ? 1 : -1, a.n_vec == 4 ? 2 : -1,
                        a.n_vec == 4 ? 3 : (!a.causal && a.n_vec == 2) ? 1 : -1};
    for (int i = tid; i < n_std; i += blockDim.x) { t_key[i] = ~0ull; t_rank[i] = 0; }
    for (int g0 = 0; g0 < n_kb; g0 += (int)blockDim.x / 8) {
        const int g = g0 + tid / 8, sl = tid & 7;
        const bool act = g < n_kb;
        int b = 0, c0 = 0, last = 0;
        if (act) {
            b = owner_of(t_kboff, B, g);
            c0 = t_cu[b] + (g - t_kboff[b]) * Bc;
            last = min(c0 + Bc, t_cu[b + 1]) - 1;
        }
        int mn[4], mx[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (src[t] < 0) {   // uniform
                mn[t] = mx[t] = t == 1 ? n32 : 0;
                continue;
            }
            int lo = INT_MAX, hi = INT_MIN;
            if (act) {
                const int* p = t_sv + src[t] * n32;
#pragma unroll
                for (int i = 0; i < 8; ++i) {   // columns past the block's last repeat it
                    const int x = p[min(c0 + 8 * sl + ((i + g) & 7), last)];
                    lo = min(lo, x); hi = max(hi, x);
                }
            }
            mn[t] = min8(lo); mx[t] = max8(hi);
        }
        if (act && sl == 0) {
            const int4 e0 = {mn[0], mx[0], mn[1], mx[1]}, e1 = {mn[2], mx[2], mn[3], mx[3]};
            ((int4*)t_ext)[2 * g] = e0;
            ((int4*)t_ext)[2 * g + 1] = e1;
            if (writer) {
                ((int4*)a.w_ext)[2 * (int64_t)g] = e0;
                ((int4*)a.w_ext)[2 * (int64_t)g + 1] = e1;
            }
        }
    }
    __syncthreads();

    // ---- tile classes and visit lists (§3.2): one q tile per wave, one key
    // block per lane; each q tile's split chunks go straight into its slots
    // (slot numbering as in the workspace plan: sequences in order, q tiles
    // in order, ceil(Tc / S) slots per q tile), keyed for the longest-first
    // order: (-chunk size, slot) ----
    auto n_split = [&](int cost) { return (S == 0 || cost <= S) ? 1 : ceil_div(cost, S); };
    int cnt[3] = {0, 0, 0}, nv = 0;
    for (int r = wid; r < R; r += nw) {
        const int b = owner_of(t_rowoff, B, r);
        const int qt = r - t_rowoff[b];
        const int s_b = t_cu[b], e_b = t_cu[b + 1];
        const int Tc = ceil_div(e_b - s_b, Bc);
        const int r0 = s_b + qt * Br, r1 = min(r0 + Br, e_b);
        const int vbase = t_tileoff[b] + qt * Tc;
        const int* xe = t_ext + t_kboff[b] * 8;
        int cost = 0;
        for (int kb0 = 0; kb0 < Tc; kb0 += 64) {
            const int kb = kb0 + lane;
            bool v = false, iv = false;
            if (kb < Tc) {
                const int4 x0 = ((const int4*)xe)[2 * kb], x1 = ((const int4*)xe)[2 * kb + 1];
                const int x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                const int c0 = s_b + kb * Bc, c1 = min(c0 + Bc, e_b);
                const TileInfo ti = classify_tile(r0, r1, c0, c1, x, a.causal);
                cnt[ti.cls] += 1;
                v = ti.cls != CLS_FULL;
                iv = ti.need_lt || ti.need_ut;
            }
            const uint64_t m = __ballot(v);
            if (v) vis[vbase + cost + __popcll(m & lanemask_lt())] = (uint16_t)(kb | ((int)iv << 15));
            cost += __popcll(m);
        }
        const int n = n_split(cost), q = cost / n, rem = cost % n;
        const int sb = t_slotbase[b] + qt * ((S > 0 && Tc > 0) ? ceil_div(Tc, S) : 1);
        for (int s = lane; s < n; s += 64) {
            const int size = q + (s < rem ? 1 : 0), start = s * q + min(s, rem);
            t_key[sb + s] = ((uint64_t)(FM_MAX_COST - size) << 32) | (uint64_t)(sb + s);
            t_sinfo[sb + s] = int4{(b << 16) | qt, s | (n << 16), start, size};
        }
        nv += n;
    }
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        int v = cnt[c];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0 && v) atomicAdd(&s_misc[1 + c], v);
    }
    if (lane == 0 && nv) atomicAdd(&s_misc[5], nv);
    __syncthreads();
    const int n_valid = s_misc[5];
    if (n_valid > LP_MAX_SLOTS || (long long)n_valid * H > (long long)LP_MAX_MY * gridDim.x) {
        if (writer && tid == 0) {
            hdr[HDR_STATUS] = FM_STATUS_CAP; hdr[HDR_NKB] = 0; hdr[HDR_NITEMS] = 0; hdr[HDR_NSLOTS] = 0; hdr[HDR_NMERGE] = 0;
            a.w_counts[0] = a.w_counts[1] = a.w_counts[2] = 0;
        }
        return LdsPlan{FM_STATUS_CAP, 0, 0};
    }
    // ---- one item per workgroup: when the writer has no item
    // (n_valid * H <= gridDim.x - 1), the longest-first order cannot change
    // the schedule (every item starts at once), so a workgroup takes the
    // (g / H)-th filled slot in slot order, head g % H, and skips the sort.
    // g is the item index with the 8 XCDs in mind: workgroups are dealt to
    // the XCDs in turn, so workgroup id runs item (id % 8) * c + id / 8,
    // c = ceil(items / 8): each XCD gets a run of c consecutive items (the
    // splits of a few q tiles, both heads), whose Q tiles and key ranges
    // then come from that XCD's own L2, and all 8 XCDs stay busy.  Every
    // item has one workgroup (id = 8 (g / c) ... < 8 c), and the writer,
    // G - 1, gets none while 8 c <= G - 1; otherwise workgroup id runs
    // item id.  The writer still sorts and writes the plan. ----
    if (!writer && (long long)n_valid * H <= (long long)gridDim.x - 1) {
        const int id = (int)blockIdx.x, n_it = n_valid * H, c = ceil_div(n_it, 8);
        const int g = 8 * c > (int)gridDim.x - 1 ? id : (id >> 3) < c ? (id & 7) * c + (id >> 3) : n_it;
        const int k = g / H, h = g - k * H;
        if (k >= n_valid) return LdsPlan{0, n_valid * H, 0};
        if (wid == 0) {
            int base = 0, slot = -1;
            for (int c0 = 0; c0 < n_std && slot < 0; c0 += 64) {
                const int i = c0 + lane;
                const bool f = i < n_std && t_key[i] != ~0ull;
                const uint64_t m = __ballot(f);
                const int r = base + __popcll(m & lanemask_lt());
                const uint64_t hit = __ballot(f && r == k);
                if (hit) slot = c0 + __builtin_ctzll(hit);
                base += __popcll(m);
            }
            if (lane < ITEM_WORDS) {
                const int4 si = t_sinfo[slot];
                const int b = si.x >> 16, qt = si.x & 0xffff, sp = si.y & 0xffff, n = si.y >> 16;
                const int start = si.z, size = si.w;
                const int s_b = t_cu[b], e_b = t_cu[b + 1];
                const int Tc = ceil_div(e_b - s_b, Bc);
                const int vb = t_tileoff[b] + qt * Tc + start;
                const int w = lane;
                myrec[0][w] = w == 0 ? b : w == 1 ? h : w == 2 ? qt
                            : w == 3 ? (size ? (int)(vis[vb] & 0x7fff) : 0)
                            : w == 4 ? (size ? (int)(vis[vb + size - 1] & 0x7fff) + 1 : 0)
                            : w == 5 ? sp : w == 6 ? n : w == 7 ? size : w == 8 ? s_b : w == 9 ? e_b
                            : w == 10 ? t_kboff[b]
                            : w == 11 ? t_slotbase[b] + qt * ((S > 0 && Tc > 0) ? ceil_div(Tc, S) : 1)
                            : w == 12 ? vb : 0;
            }
        }
        __syncthreads();
        return LdsPlan{0, n_valid * H, 1};
    }
    // ---- rank of every filled slot: the number of smaller keys, counted by
    // `parts` threads per slot over disjoint ranges ----
    {
        const int parts = max(1, min(8, (int)blockDim.x / max(n_std, 1)));
        const int chunk = ceil_div(n_std, parts);
        for (int t = tid; t < n_std * parts; t += blockDim.x) {
            const int i = t / parts, part = t - i * parts;
            const uint64_t key = t_key[i];
            if (key == ~0ull) continue;
            const int j0 = part * chunk, j1 = min(j0 + chunk, n_std);
            int rk = 0;
#pragma unroll 8
            for (int j = j0; j < j1; ++j) rk += t_key[j] < key ? 1 : 0;
            if (rk) atomicAdd(&t_rank[i], rk);
        }
    }
    __syncthreads();
    // invert: the slot at each rank
    for (int i = tid; i < n_std; i += blockDim.x)
        if (t_key[i] != ~0ull) t_slot_at[t_rank[i]] = i;
    __syncthreads();

    // ---- items: rank * H + head ----
    const int n_items = n_valid * H;
    auto record = [&](int it, int w) {   // word w of item `it`
        const int rk = it / H, h = it - rk * H;
        const int4 si = t_sinfo[t_slot_at[rk]];
        const int b = si.x >> 16, qt = si.x & 0xffff, s = si.y & 0xffff, n = si.y >> 16;
        const int start = si.z, size = si.w;
        const int s_b = t_cu[b], e_b = t_cu[b + 1];
        const int Tc = ceil_div(e_b - s_b, Bc);
        const int vb = t_tileoff[b] + qt * Tc + start;
        switch (w) {
            case 0: return b;
            case 1: return h;
            case 2: return qt;
            case 3: return size ? (int)(vis[vb] & 0x7fff) : 0;
            case 4: return size ? (int)(vis[vb + size - 1] & 0x7fff) + 1 : 0;
            case 5: return s;
            case 6: return n;
            case 7: return size;
            case 8: return s_b;
            case 9: return e_b;
            case 10: return t_kboff[b];
            case 11: return t_slotbase[b] + qt * ((S > 0 && Tc > 0) ? ceil_div(Tc, S) : 1);
            case 12: return vb;
            default: return 0;
        }
    };
    int n_my = 0;
    for (int k = 0; k < LP_MAX_MY; ++k) {
        const int it = blockIdx.x + k * gridDim.x;
        if (it >= n_items) break;
        if (tid < ITEM_WORDS) myrec[k][tid] = record(it, tid);
        ++n_my;
    }
    if (writer) {
        for (int idx = tid; idx < n_items * ITEM_WORDS; idx += blockDim.x) {
            const int it = idx / ITEM_WORDS, w = idx - it * ITEM_WORDS;
            a.w_items[idx] = w < 12 ? record(it, w) : 0;
        }
        // split rows: one merge entry per (split row, head), from its split 0
        if (a.w_merge)
            for (int it = tid; it < n_items; it += blockDim.x)
                if (record(it, 5) == 0 && record(it, 6) > 1) {
                    const int k = atomicAdd(&s_misc[4], 1);
                    int32_t* m = a.w_merge + (int64_t)k * MERGE_WORDS;
                    const int row0 = record(it, 8) + record(it, 2) * Br;
                    m[0] = record(it, 11); m[1] = record(it, 1); m[2] = row0;
                    m[3] = min(row0 + Br, record(it, 9)); m[4] = record(it, 6);
                    m[5] = m[6] = m[7] = 0;
                }
        __syncthreads();
        if (tid == 0) {
            hdr[HDR_NITEMS] = n_items;
            hdr[HDR_NSLOTS] = t_slotbase[B];
            hdr[HDR_NMERGE] = s_misc[4];
            a.w_counts[0] = s_misc[1]; a.w_counts[1] = s_misc[2]; a.w_counts[2] = s_misc[3];
        }
    }
    __syncthreads();   // the temporaries are dead from here on
    return LdsPlan{0, n_items, n_my};
}

}  // namespace fm
