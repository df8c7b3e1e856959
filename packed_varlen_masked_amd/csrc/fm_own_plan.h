// Per-workgroup planning of the fused bf16 path: every workgroup of the one
// attention launch derives its own work item(s) from cu_seqlens and the mask
// vectors of its own q-tile row only, instead of a planning launch (or a
// plan of the whole problem) ahead of the attention.
//
// Method: PaddleNLP FlashMask article (m.nxbn.cn/news/70198) §3.1 (per key
// block min/max of LTS/LTE/UTS/UTE), §3.2 (FULL / PARTIAL / UNMASKED tile
// classes); work named by (sequence, head, q tile) as in the Varlen-Packing
// technical document (www.gsyq.cn/news/432802) §2.
//
// Work items are the library's split chunks (the same chunks fm_build_worklist
// lists, so both paths give the same bits), numbered without knowing any
// tile class: q tile (b, qt) gets ceil(U / S) slots (one when S = 0 or
// U <= S), U = its key blocks not past the causal diagonal (all of them
// without the causal flag), an upper bound of its visit count.  A slot's
// workgroup classifies the row's U blocks, counts the visited ones (cost),
// cuts them into n = ceil(cost / S) chunks as the work list does and runs
// chunk s of its slot; slots s >= n (possible only when interval masks hide
// whole key blocks inside the causal range) have no work.
// Included by the attention source after its Item record is defined.
#pragma once
#include "fm_common.hpp"
#include "fm_internal.h"

namespace fm {

constexpr int OP_MAX_B = FUSED_MAX_B;       // sequences
constexpr int OP_MAX_ROWS = FUSED_MAX_ROWS; // q tiles over all sequences
constexpr int OP_MAX_MY = FUSED_MAX_MY;     // items per workgroup

// One of the workgroup's items: sequence, q tile (within the sequence and
// over all sequences), split slot within the q tile, head, and U.
struct MyItem { int b, qt, r, s, h, U; };

// Launch-wide tables, built by wave 0 of every workgroup in LDS.
struct OwnTables {
    int cu[OP_MAX_B + 1];        // cu_seqlens
    int rowoff[OP_MAX_B + 1];    // first q tile of each sequence (prefix of Tr_b)
    int qslot[OP_MAX_ROWS + 1];  // first slot of each q tile (prefix of its slot count)
    int qseq[OP_MAX_ROWS];       // sequence of each q tile
    MyItem my[OP_MAX_MY];        // this workgroup's items
    int misc[4];                 // status, R (q tiles), slots, items of this workgroup
};

// Inclusive prefix sum across the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS traffic).
__device__ __attribute__((always_inline)) inline int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return v;
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// words (the LDS serves one wave's instructions in order; this keeps the
// compiler from moving the reads up).
__device__ __attribute__((always_inline)) inline void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// Index of the last entry <= x of an ascending int array of n + 1 entries
// (the owner of element x in a prefix-sum table); arr[0] <= x < arr[n].
__device__ inline int owner_in(const int* arr, int n, int x) {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (arr[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// Key blocks of q tile qt of a sequence of length L that are not past the
// causal diagonal (every block without the causal flag).
template <int Br, int Bc>
__device__ __attribute__((always_inline)) inline int row_blocks(int L, int qt, int causal) {
    const int Tc = ceil_div(L, Bc);
    return causal ? min(Tc, ceil_div(min((qt + 1) * Br, L), Bc)) : Tc;
}

// Work item `k` of workgroup `id` of G among n_items: when every item has a
// workgroup of its own, workgroup id runs item (id mod 8) c + id / 8,
// c = ceil(n_items / 8) (workgroups go to the 8 XCDs in turn, so each XCD
// runs c consecutive items); otherwise items id, id + G, ...  Returns
// n_items when the workgroup has no k-th item.
__device__ __attribute__((always_inline)) inline int item_index(int id, int k, int G, int n_items) {
    const int c = ceil_div(n_items, 8);
    if (n_items <= G && 8 * c <= G) return (k == 0 && (id >> 3) < c) ? (id & 7) * c + (id >> 3) : n_items;
    const long long it = (long long)id + (long long)k * G;
    return it < n_items ? (int)it : n_items;
}

// Builds the tables and resolves this workgroup's items: wave 0 does the
// work (wave-wide DPP scans, no LDS round trip between lanes beyond the
// sequence lookups), then one barrier.  Every thread must call it.
// Returns the status (FM_STATUS_* bits of cu_seqlens, or FM_STATUS_CAP
// when the sizes exceed the tables; 0 = valid).
template <int Br, int Bc>
__device__ int own_setup(const AttnArgs& a, OwnTables& T) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int B = a.B, S = a.S, H = a.H;
    if (wid == 0) {
        int status = 0, R = 0, total = 0, n_my = 0;
        if (B > OP_MAX_B) {
            status = FM_STATUS_CAP;   // the host bound was violated
        } else {
            // sequences: lane b + 64 m holds cu[b], cu[b + 1] (all loads first)
            int lo[4], hi[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int b = lane + 64 * m;
                lo[m] = b < B ? a.cu[b] : 0;
                hi[m] = b < B ? a.cu[b + 1] : 0;
            }
            const int cu0 = a.cu[0], cuB = a.cu[B];
            bool bad = false;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int b = lane + 64 * m;
                if (64 * m >= B) break;
                bad |= b < B && hi[m] < lo[m];
                const int L = b < B ? max(hi[m] - lo[m], 0) : 0;
                const int tr = min(ceil_div(L, Br), OP_MAX_ROWS + 1);   // clamped: no overflow before validation
                const int incl = wave_incl_scan(tr);
                if (b < B) { T.cu[b] = lo[m]; T.rowoff[b] = R + incl - tr; }
                R += __builtin_amdgcn_readlane(incl, 63);
            }
            if (lane == 0) { T.cu[B] = cuB; T.rowoff[B] = R; }
            status = (__ballot(bad) ? FM_STATUS_ORDER : 0) | (cu0 != 0 ? FM_STATUS_CU0 : 0) |
                     (cuB != (int)a.N ? FM_STATUS_CUN : 0);
            if (!status && R > OP_MAX_ROWS) status = FM_STATUS_CAP;
        }
        wave_lds_order();
        if (!status) {
            // q tiles: lane r + 64 m, its sequence (binary search of rowoff),
            // its slot count ceil(U / S) (one when S = 0 or U <= S), prefix sums
#pragma unroll
            for (int m = 0; m < OP_MAX_ROWS / 64; ++m) {
                const int r = 64 * m + lane;
                int cnt = 0, b = 0;
                if (r < R) {
                    b = owner_in(T.rowoff, B, r);
                    const int U = row_blocks<Br, Bc>(T.cu[b + 1] - T.cu[b], r - T.rowoff[b], a.causal);
                    cnt = (S == 0 || U <= S) ? 1 : ceil_div(U, S);
                }
                if (64 * m < R) {
                    const int incl = wave_incl_scan(cnt);
                    if (r < R) { T.qslot[r] = total + incl - cnt; T.qseq[r] = b; }
                    total += __builtin_amdgcn_readlane(incl, 63);
                }
            }
            if (lane == 0) T.qslot[R] = total;
            wave_lds_order();
            // this workgroup's items: slot = item / H, head = item mod H (the
            // heads and splits of one q tile are neighbours, so one XCD reads
            // its Q tile); the slot's q tile is the last one whose first slot
            // is <= slot
            const int n_items = total * H;
            for (int k = 0; k < OP_MAX_MY; ++k) {
                const int it = item_index((int)blockIdx.x, k, (int)gridDim.x, n_items);
                if (it >= n_items) break;
                const int slot = it / H, h = it - slot * H;
                int below = 0;
#pragma unroll
                for (int m = 0; m < OP_MAX_ROWS / 64; ++m)
                    if (64 * m < R) below += __popcll(__ballot(64 * m + lane < R && T.qslot[64 * m + lane] <= slot));
                const int r = below - 1, b = T.qseq[r], qt = r - T.rowoff[b];
                if (lane == 0)
                    T.my[k] = MyItem{b, qt, r, slot - T.qslot[r], h,
                                     row_blocks<Br, Bc>(T.cu[b + 1] - T.cu[b], qt, a.causal)};
                ++n_my;
            }
        }
        if (lane == 0) { T.misc[0] = status; T.misc[1] = R; T.misc[2] = total; T.misc[3] = n_my; }
    }
    __syncthreads();
    return T.misc[0];
}

// Chunk m.s of the visit list of q tile m's row for head m.h.  Every thread
// must call it (one barrier).  The row's first U key blocks are reduced to
// their extrema straight from the mask vectors (8 lanes per block, 8 columns
// each; columns past a ragged block's end repeat its last one) and
// classified; lane 8i of wave w carries block 64j + 8w + i of pass j, and
// each wave writes its byte of the pass's 64-block masks.  After the barrier
// every wave compacts the masks into vis[0 .. cost) (ascending visited key
// blocks, key block | interval flag << 15; all waves write the same values)
// and derives the chunk.  Returns false when the slot has no chunk
// (s >= n); otherwise I is the item and vis_off its first entry, and split
// 0 writes the row's entry of the merge table.
template <int Br, int Bc, int HDim>
__device__ bool own_item(const AttnArgs& a, const OwnTables& T, const MyItem& m, Item& I, int& vis_off,
                         uint16_t* vis, uint64_t* wvis, uint64_t* wiv) {
    static_assert(Bc == 64, "eight lanes of eight columns per key block");
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int s_b = __builtin_amdgcn_readfirstlane(T.cu[m.b]), e_b = __builtin_amdgcn_readfirstlane(T.cu[m.b + 1]);
    const int r0 = s_b + m.qt * Br, r1 = min(r0 + Br, e_b);
    const int U = m.U;
    const int n_vec = a.n_vec;
    const int64_t N = a.N;
    const int n32 = (int)N;
    // stored vector behind each logical one (LTS, LTE, UTS, UTE); absent ones
    // take their default (LTE: N; UTS, UTE: 0)
    const int src[4] = {0, (n_vec == 4 || (a.causal && n_vec == 2)) ? 1 : -1, n_vec == 4 ? 2 : -1,
                        n_vec == 4 ? 3 : (!a.causal && n_vec == 2) ? 1 : -1};
    // window j = blocks 64 j .. 64 j + 63; wave w takes blocks 64 j + 8 w + 4 sp
    // + row (sub-pass sp = 0, 1; row = lane / 16), 16 lanes per block, 4
    // consecutive columns per lane (one 16-byte load per stored vector, so a
    // wave's loads of four blocks are 1 KB contiguous)
    const int nwin = ceil_div(U, 64);
    const int row = lane >> 4, li = lane & 15;
    for (int j = 0; j < nwin; ++j) {
        int lo[2][4], hi[2][4];
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const int kb = 64 * j + 8 * wid + 4 * sp + row;
            const int col = s_b + kb * Bc + 4 * li, cend = min(s_b + kb * Bc + Bc, e_b);
            const bool act = kb < U && col < cend;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                lo[sp][t] = INT_MAX; hi[sp][t] = INT_MIN;
                if (t >= n_vec || !act) continue;
                const int32_t* v = a.sv + (int64_t)t * N + col;
                int x[4];
                if (col + 3 < cend) {
                    int4 q4;
                    __builtin_memcpy(&q4, v, 16);
                    x[0] = q4.x; x[1] = q4.y; x[2] = q4.z; x[3] = q4.w;
                } else {   // the block's ragged end: columns past it repeat its last one
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = v[min(e, cend - 1 - col)];
                }
                lo[sp][t] = min(min(x[0], x[1]), min(x[2], x[3]));
                hi[sp][t] = max(max(x[0], x[1]), max(x[2], x[3]));
            }
        }
        uint32_t mv = 0, mi = 0;
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            int sm[4], sx[4];   // per stored vector: min / max over the 16 lanes of the block
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                int x = lo[sp][t], y = hi[sp][t];
                x = min(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false));    // quad_perm [1,0,3,2]
                x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false));    // quad_perm [2,3,0,1]
                x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xf, 0xf, false));   // row_half_mirror
                sm[t] = min(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xf, 0xf, false));   // row_mirror
                y = max(y, __builtin_amdgcn_update_dpp(y, y, 0xB1, 0xf, 0xf, false));
                y = max(y, __builtin_amdgcn_update_dpp(y, y, 0x4E, 0xf, 0xf, false));
                y = max(y, __builtin_amdgcn_update_dpp(y, y, 0x141, 0xf, 0xf, false));
                sx[t] = max(y, __builtin_amdgcn_update_dpp(y, y, 0x140, 0xf, 0xf, false));
            }
            const int kb = 64 * j + 8 * wid + 4 * sp + row;
            bool v = false, iv = false;
            if (kb < U) {
                const int c0 = s_b + kb * Bc;
                int x[8];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int d = t == 1 ? n32 : 0, i = src[t];   // i is uniform: selects, no indexing
                    x[2 * t] = i < 0 ? d : i == 0 ? sm[0] : i == 1 ? sm[1] : i == 2 ? sm[2] : sm[3];
                    x[2 * t + 1] = i < 0 ? d : i == 0 ? sx[0] : i == 1 ? sx[1] : i == 2 ? sx[2] : sx[3];
                }
                const TileInfo ti = classify_tile(r0, r1, c0, min(c0 + Bc, e_b), x, a.causal);
                v = ti.cls != CLS_FULL;
                iv = ti.need_lt || ti.need_ut;
            }
            // lanes 0, 16, 32, 48 carry blocks 4 sp + 0 .. 3 of this wave's byte
            const uint64_t bv = __ballot(v && li == 0), bi = __ballot(iv && li == 0);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                mv |= (uint32_t)((bv >> (16 * rr)) & 1ull) << (4 * sp + rr);
                mi |= (uint32_t)((bi >> (16 * rr)) & 1ull) << (4 * sp + rr);
            }
        }
        if (lane == 0) {
            ((uint8_t*)&wvis[j])[wid] = (uint8_t)mv;
            ((uint8_t*)&wiv[j])[wid] = (uint8_t)mi;
        }
    }
    __syncthreads();
    // every wave: visited blocks of each window, their running count, the list
    int cost = 0;
    for (int j0 = 0; j0 < nwin; j0 += 64) {
        const int j = j0 + lane;
        const int c = j < nwin ? __popcll(wvis[j]) : 0;
        const int incl = wave_incl_scan(c);
        const int n_here = min(64, nwin - j0);
        for (int jj = 0; jj < n_here; ++jj) {
            const uint64_t vm = wvis[j0 + jj], im = wiv[j0 + jj];
            const int base = cost + __builtin_amdgcn_readlane(incl, jj) - __popcll(vm);
            if ((vm >> lane) & 1ull)
                vis[base + __popcll(vm & lanemask_lt())] =
                    (uint16_t)((64 * (j0 + jj) + lane) | (int)(((im >> lane) & 1ull) << 15));
        }
        cost += __builtin_amdgcn_readlane(incl, 63);
    }
    wave_lds_order();
    const int S = a.S;
    const int n = (S == 0 || cost <= S) ? 1 : ceil_div(cost, S);
    if (m.s >= n) return false;
    const int q = cost / n, rem = cost % n;
    const int size = q + (m.s < rem ? 1 : 0), start = m.s * q + min(m.s, rem);
    const int slot0 = __builtin_amdgcn_readfirstlane(T.qslot[m.r]);
    I.b = m.b; I.h = m.h; I.qt = m.qt;
    I.kbb = size ? __builtin_amdgcn_readfirstlane((int)(vis[start] & 0x7fff)) : 0;
    I.kbe = size ? __builtin_amdgcn_readfirstlane((int)(vis[start + size - 1] & 0x7fff)) + 1 : 0;
    I.sidx = m.s; I.nsp = n; I.cost = size;
    I.s_b = s_b; I.e_b = e_b;
    I.slot0 = slot0;
    I.Tc = ceil_div(e_b - s_b, Bc);
    I.r0 = r0; I.r1 = r1;
    I.xb = a.extrema;   // block extrema are not read on this path
    I.hoff = (int64_t)m.h * HDim;
    vis_off = start;
    if (a.w_merge && m.s == 0 && wid == 0 && lane < MERGE_WORDS) {   // the row's merge-table entry
        const int w = lane;
        a.w_merge[((int64_t)m.r * a.H + m.h) * MERGE_WORDS + w] =
            w == 0 ? slot0 : w == 1 ? m.h : w == 2 ? r0 : w == 3 ? r1 : w == 4 ? n : 0;
    }
    return true;
}

// First key block of chunk s of a row of U blocks when every block is
// visited (the common case: the guess of the speculative first-tile copy);
// -1 when the chunk would not exist.
__device__ __attribute__((always_inline)) inline int guess_first_block(int U, int s, int S) {
    const int n = (S == 0 || U <= S) ? 1 : ceil_div(U, S);
    if (U == 0 || s >= n) return -1;
    const int q = U / n, rem = U % n;
    return s * q + min(s, rem);
}

}  // namespace fm
