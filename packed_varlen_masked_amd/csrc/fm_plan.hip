// Plan kernels: block extrema (preprocessing) and the tile classes / work
// list.  Sources: PaddleNLP FlashMask article (m.nxbn.cn/news/70198) §3.1
// (per-key-block min/max of LTS/LTE/UTS/UTE), §3.2 (three tile classes);
// Varlen-Packing technical document (www.gsyq.cn/news/432802) §2 (work named
// by (sequence, head, q tile)) and §1.2 (a fixed grid waits for its slowest
// block, hence compact items ordered longest first).
#include <algorithm>

#include "fm_common.hpp"
#include "fm_internal.h"

namespace fm {

// ------------------------------------------------------------------------
// Per-workgroup scan of the key-block counts of all sequences into LDS.
// Every workgroup of the extrema kernel repeats it (B is small next to N),
// which removes a launch and a grid-wide dependency.  Also validates cu.
// Returns the status bits (0 = valid) and leaves s_off[0..B] filled, and
// s_cu[0..B] = cu[0..B].
__device__ int scan_kblocks(const int32_t* __restrict__ cu, int B, int64_t N, int Bc,
                            int64_t cap, int32_t* s_off, int32_t* s_cu, long long* tmp) {
    __shared__ int s_bad;
    if (threadIdx.x == 0) s_bad = (cu[0] != 0 ? FM_STATUS_CU0 : 0) | (cu[B] != (int)N ? FM_STATUS_CUN : 0);
    __syncthreads();
    long long carry = 0;
    for (int base = 0; base < B; base += blockDim.x) {
        const int b = base + threadIdx.x;
        long long tc = 0;
        if (b < B) {
            const int c = cu[b];
            const int L = cu[b + 1] - c;
            if (L < 0) atomicOr(&s_bad, FM_STATUS_ORDER);
            tc = L > 0 ? ceil_div(L, Bc) : 0;
            s_cu[b] = c;
        }
        long long tot;
        const long long ex = block_exclusive_scan(tc, tmp, &tot);
        if (b < B) s_off[b] = (int32_t)min(carry + ex, (long long)INT_MAX);
        carry += tot;
    }
    if (threadIdx.x == 0) {
        s_cu[B] = cu[B];
        s_off[B] = (int32_t)min(carry, (long long)INT_MAX);
        if (carry > cap) atomicOr(&s_bad, FM_STATUS_CAP);
    }
    __syncthreads();
    return s_bad;
}

// min / max of the four filled vectors over columns [c0, c1), reduced across
// the wave; lane 2t returns the min and lane 2t+1 the max of vector t.
__device__ inline int block_extrema(const int32_t* __restrict__ sv, int n_vec, int causal, int64_t N,
                                    int64_t c0, int64_t c1, int lane) {
    int mn[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
    int mx[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
    for (int64_t col = c0 + lane; col < c1; col += 64) {
        const Vec4 f = fill_column(sv, n_vec, causal, N, col);
        mn[0] = min(mn[0], f.lts); mx[0] = max(mx[0], f.lts);
        mn[1] = min(mn[1], f.lte); mx[1] = max(mx[1], f.lte);
        mn[2] = min(mn[2], f.uts); mx[2] = max(mx[2], f.uts);
        mn[3] = min(mn[3], f.ute); mx[3] = max(mx[3], f.ute);
    }
    int outv = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int a = wave_min(mn[t]), z = wave_max(mx[t]);
        if (lane == 2 * t) outv = a;
        if (lane == 2 * t + 1) outv = z;
    }
    return outv;
}

// N2: grid-stride over the global key blocks.  For Bc <= 64 a wave takes
// four blocks at a time (16 lanes each, four columns per lane: coalesced,
// and the min / max reductions stay inside a row of 16 lanes); larger blocks
// take one wave each.
__global__ __launch_bounds__(256) void fm_extrema_kernel(
    const int32_t* __restrict__ sv, int n_vec, int causal, const int32_t* __restrict__ cu,
    int B, int64_t N, int Bc, int32_t* __restrict__ kb_off, int32_t* __restrict__ ext,
    int64_t ext_cap, int32_t* __restrict__ n_kblocks, int32_t* __restrict__ status) {
    extern __shared__ int32_t s_off[];  // [B+1] key-block offsets, then [B+1] cu
    int32_t* s_cu = s_off + B + 1;
    __shared__ long long tmp[17];
    const int bad = scan_kblocks(cu, B, N, Bc, ext_cap, s_off, s_cu, tmp);
    if (blockIdx.x == 0) {
        for (int b = threadIdx.x; b <= B; b += blockDim.x) kb_off[b] = bad ? 0 : s_off[b];
        if (threadIdx.x == 0) { *status = bad; *n_kblocks = bad ? 0 : s_off[B]; }
    }
    if (bad) return;
    const int total = s_off[B];
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int stride = gridDim.x * waves;
    // column range of global key block g: sequence = last b with s_off[b] <= g
    auto block_cols = [&](int g, int64_t& c0, int64_t& c1) {
        int lo = 0, hi = B;  // s_off[lo] <= g < s_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_off[mid] <= g) lo = mid; else hi = mid;
        }
        c0 = (int64_t)s_cu[lo] + (int64_t)(g - s_off[lo]) * Bc;
        c1 = min(c0 + Bc, (int64_t)s_cu[lo + 1]);
    };
    if (Bc <= 64) {
        // four blocks per wave: lanes 16r .. 16r+15 take block g0 + r, lane q
        // of the row its columns 4q .. 4q+3 (four loads of 4 B per vector, the
        // 16 lanes of a row together contiguous); min / max of the four columns
        // in the lane, then across the row with DPP (every lane of the row
        // gets the block's value)
        const int r = lane >> 4, q = lane & 15;
        auto row_min = [](int v) {
            v = min(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xf, 0xf, false));    // quad_perm [1,0,3,2]
            v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xf, 0xf, false));    // quad_perm [2,3,0,1]
            v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));   // row_half_mirror
            return min(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false)); // row_mirror
        };
        auto row_max = [](int v) {
            v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xf, 0xf, false));
            v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xf, 0xf, false));
            v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));
            return max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false));
        };
        const int nwaves = gridDim.x * waves;
        // 16-byte loads need 16-byte aligned vector rows
        const bool vec16 = ((uintptr_t)sv & 15) == 0 && (N & 3) == 0;
        for (int g0 = 4 * (blockIdx.x * waves + (threadIdx.x >> 6)); g0 < total; g0 += 4 * nwaves) {
            const int g = g0 + r;
            int64_t c0 = 0, c1 = 0;
            if (g < total) block_cols(g, c0, c1);
            int mn[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX}, mx[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
            Vec4 f[4];
            bool ok[4];
            const int64_t cq = c0 + 4 * q;   // first column of this lane
            if (vec16 && (c0 & 3) == 0 && 4 * q + 3 < Bc && cq + 3 < c1) {
                // the lane's four columns of each stored vector in one 16-byte load
                int4 x[4];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (v < n_vec) x[v] = *(const int4*)(sv + (int64_t)v * N + cq);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    auto at = [&](int v) { return k == 0 ? x[v].x : k == 1 ? x[v].y : k == 2 ? x[v].z : x[v].w; };
                    ok[k] = true;
                    f[k].lts = at(0);
                    if (causal) {
                        f[k].lte = n_vec == 2 ? at(1) : (int)N;
                        f[k].uts = 0; f[k].ute = 0;
                    } else if (n_vec == 2) {
                        f[k].lte = (int)N; f[k].uts = 0; f[k].ute = at(1);
                    } else {
                        f[k].lte = at(1); f[k].uts = at(2); f[k].ute = at(3);
                    }
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int64_t col = cq + k;
                    ok[k] = 4 * q + k < Bc && col < c1;
                    if (ok[k]) f[k] = fill_column(sv, n_vec, causal, N, col);
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (ok[k]) {
                    mn[0] = min(mn[0], f[k].lts); mx[0] = max(mx[0], f[k].lts);
                    mn[1] = min(mn[1], f[k].lte); mx[1] = max(mx[1], f[k].lte);
                    mn[2] = min(mn[2], f[k].uts); mx[2] = max(mx[2], f[k].uts);
                    mn[3] = min(mn[3], f[k].ute); mx[3] = max(mx[3], f[k].ute);
                }
            int outv = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int a = row_min(mn[t]), z = row_max(mx[t]);
                if (q == 2 * t) outv = a;
                if (q == 2 * t + 1) outv = z;
            }
            if (g < total && q < 8) ext[(int64_t)g * 8 + q] = outv;
        }
    } else {
        for (int g = blockIdx.x * waves + (threadIdx.x >> 6); g < total; g += stride) {
            int64_t c0, c1;
            block_cols(g, c0, c1);
            const int outv = block_extrema(sv, n_vec, causal, N, c0, c1, lane);
            if (lane < 8) ext[(int64_t)g * 8 + lane] = outv;
        }
    }
}

// ------------------------------------------------------------------------
// Sizes of sequence b that the worklist stage needs.
struct SeqDims { int s, e, L, Tr, Tc, MS; };

__device__ inline SeqDims seq_dims(const int32_t* __restrict__ cu, int b, int Br, int Bc, int S) {
    SeqDims d;
    d.s = cu[b]; d.e = cu[b + 1]; d.L = max(d.e - d.s, 0);
    d.Tr = d.L ? ceil_div(d.L, Br) : 0;
    d.Tc = d.L ? ceil_div(d.L, Bc) : 0;
    d.MS = (S > 0 && d.Tc > 0) ? ceil_div(d.Tc, S) : 1;
    return d;
}

// Tile classes of every q tile of sequence b (one wave per q tile, one key
// block per lane; FlashMask article §3.2), the class map, per-thread class
// counts, and the split slots of each q tile (cost = non-FULL blocks,
// chunks of at most S blocks whose sizes differ by at most one).
__device__ void classify_rows(const SeqDims& d, int b, int Br, int Bc, int S, int causal,
                              const int4* __restrict__ xs, int32_t* __restrict__ slots, long long slot_base,
                              int64_t slot_cap, long long map_base, uint8_t* __restrict__ tile_class,
                              int64_t tile_class_cap, long long (&my_cnt)[3], int group) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    // q tiles group * nw + wid, then every PLAN_RC * nw-th
    for (int qt = group * nw + wid; qt < d.Tr; qt += PLAN_RC * nw) {
        const int r0 = d.s + qt * Br, r1 = min(r0 + Br, d.e);
        int cost = 0, first = INT_MAX, last = -1;
        const int64_t map_row = map_base + (int64_t)qt * d.Tc;
        for (int kb0 = 0; kb0 < d.Tc; kb0 += 64) {
            const int kb = kb0 + lane;
            bool nonfull = false;
            if (kb < d.Tc) {
                const int4 a = xs[2 * kb], z = xs[2 * kb + 1];
                const int x[8] = {a.x, a.y, a.z, a.w, z.x, z.y, z.z, z.w};
                const int c0 = d.s + kb * Bc, c1 = min(c0 + Bc, d.e);
                const TileInfo ti = classify_tile(r0, r1, c0, c1, x, causal);
                my_cnt[0] += ti.cls == CLS_FULL;
                my_cnt[1] += ti.cls == CLS_PARTIAL;
                my_cnt[2] += ti.cls == CLS_UNMASKED;
                nonfull = ti.cls != CLS_FULL;
                if (tile_class && map_row + kb < tile_class_cap) tile_class[map_row + kb] = (uint8_t)ti.cls;
                if (nonfull) { first = min(first, kb); last = max(last, kb); }
            }
            cost += __popcll(__ballot(nonfull));
        }
        first = wave_min(first);
        last = wave_max(last);
        const int n = (S == 0 || cost <= S) ? 1 : ceil_div(cost, S);
        const int q = cost / n, r = cost % n;
        const int64_t sb = slot_base + (int64_t)qt * d.MS;
        if (sb + d.MS > slot_cap) continue;  // host bound violated: leave no slot
        // record fields other than the kb range, and empty slots past n
        for (int s = lane; s < d.MS; s += 64) {
            int32_t* rec = slots + (sb + s) * SLOT_WORDS;
            const int size = q + (s < r ? 1 : 0);
            rec[0] = b; rec[1] = qt; rec[2] = s; rec[3] = n;
            rec[6] = size; rec[7] = s < n ? 1 : 0;
            if (n == 1 && s == 0) {
                rec[4] = cost ? first : 0;
                rec[5] = cost ? last + 1 : 0;
            } else if (s >= n) {
                rec[4] = 0; rec[5] = 0;
            }
        }
        if (n > 1) {
            // second pass: kb range of each chunk from the rank of each
            // non-FULL block among the row's non-FULL blocks
            int rank0 = 0;
            const int big = r * (q + 1);
            for (int kb0 = 0; kb0 < d.Tc; kb0 += 64) {
                const int kb = kb0 + lane;
                bool nonfull = false;
                if (kb < d.Tc) {
                    const int4 a = xs[2 * kb], z = xs[2 * kb + 1];
                    const int x[8] = {a.x, a.y, a.z, a.w, z.x, z.y, z.z, z.w};
                    const int c0 = d.s + kb * Bc, c1 = min(c0 + Bc, d.e);
                    nonfull = classify_tile(r0, r1, c0, c1, x, causal).cls != CLS_FULL;
                }
                const uint64_t bal = __ballot(nonfull);
                if (nonfull) {
                    const int k = rank0 + __popcll(bal & lanemask_lt());
                    int s, off, size;
                    if (k < big) { s = k / (q + 1); off = k % (q + 1); size = q + 1; }
                    else { s = r + (k - big) / q; off = (k - big) % q; size = q; }
                    int32_t* rec = slots + (sb + s) * SLOT_WORDS;
                    if (off == 0) rec[4] = kb;
                    if (off == size - 1) rec[5] = kb + 1;
                }
                rank0 += __popcll(bal);
            }
        }
    }
}

// N3a: PLAN_RC workgroups per sequence (workgroup b * PLAN_RC + r takes
// q-tile group r of sequence b).  The sequence's extrema are staged in LDS
// once (one round of coalesced loads); each wave then classifies q tiles from
// LDS (one key block per lane), writes the class map, counts classes, and
// writes the split slots of its q tiles.
constexpr int TILES_NTH = 512;
constexpr int TILES_LDS_KB = 1024;   // key blocks staged in LDS (32 KB); longer rows read global memory

__global__ __launch_bounds__(TILES_NTH) void fm_tiles_kernel(
    const int32_t* __restrict__ cu, int B, int Br, int Bc, int S, int causal,
    const int32_t* __restrict__ kb_off, const int32_t* __restrict__ ext,
    const int32_t* __restrict__ status, int32_t* __restrict__ slots,
    long long* __restrict__ seq_counts, int32_t* __restrict__ sl_off,
    uint8_t* __restrict__ tile_class, int64_t tile_class_cap, int64_t slot_cap) {
    if (*status != 0) return;
    const int b = blockIdx.x / PLAN_RC, group = blockIdx.x % PLAN_RC;
    __shared__ long long tmp[17];
    __shared__ long long s_cnt[3];
    __shared__ int4 s_ext[2 * TILES_LDS_KB];
    const SeqDims d = seq_dims(cu, b, Br, Bc, S);
    long long* cnt_out = seq_counts + ((int64_t)b * PLAN_RC + group) * 3;
    if (group * (TILES_NTH / 64) >= d.Tr) {   // no q tile in this group
        if (threadIdx.x < 3) cnt_out[threadIdx.x] = 0;
        return;
    }
    // offsets of this sequence: slots (sum of Tr*MS) and class map (Tr*Tc)
    long long slot_base = 0, map_base = 0;
    for (int base = 0; base < b; base += blockDim.x) {
        const int bb = base + threadIdx.x;
        long long ns = 0, nm = 0;
        if (bb < b) {
            const SeqDims e = seq_dims(cu, bb, Br, Bc, S);
            ns = (long long)e.Tr * e.MS;
            nm = (long long)e.Tr * e.Tc;
        }
        long long t1, t2;
        block_exclusive_scan(ns, tmp, &t1);
        block_exclusive_scan(nm, tmp, &t2);
        slot_base += t1; map_base += t2;
    }
    const int4* __restrict__ xg = (const int4*)(ext + (int64_t)kb_off[b] * 8);
    const bool in_lds = d.Tc <= TILES_LDS_KB;
    if (in_lds)
        for (int i = threadIdx.x; i < 2 * d.Tc; i += blockDim.x) s_ext[i] = xg[i];
    if (threadIdx.x < 3) s_cnt[threadIdx.x] = 0;
    if (threadIdx.x == 0 && group == 0) sl_off[b] = (int32_t)slot_base;
    __syncthreads();
    const int4* xs = in_lds ? s_ext : xg;
    long long my_cnt[3] = {0, 0, 0};
    classify_rows(d, b, Br, Bc, S, causal, xs, slots, slot_base, slot_cap, map_base, tile_class,
                  tile_class_cap, my_cnt, group);
    const int lane = threadIdx.x & 63;
    // class counts of this group of q tiles
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const long long t = wave_sum64(my_cnt[c]);
        if (lane == 0) atomicAdd((unsigned long long*)&s_cnt[c], (unsigned long long)t);
    }
    __syncthreads();
    if (threadIdx.x < 3) cnt_out[threadIdx.x] = s_cnt[threadIdx.x];
}

// N3b: one workgroup.  Stable counting sort of the valid slots by
// descending cost (longest first), then one item per (slot, head).  Round
// trips are kept to two: the sizes (cu, class counts, status) are read
// together, then the slot records, which stay in LDS for the ranking and the
// scatter when they fit.
constexpr int SORT_LDS_INTS = 16384;            // 64 KB: slot records (<= 2048) or slot costs
constexpr int SORT_LDS_RECS = SORT_LDS_INTS / SLOT_WORDS;
constexpr int SORT_POS_LDS = 4096;              // 16 KB: rank of each slot

__global__ __launch_bounds__(1024) void fm_sort_kernel(
    const int32_t* __restrict__ cu, int B, int H, int Br, int Bc, int S, int cost_cap,
    const int32_t* __restrict__ kb_off,
    const int32_t* __restrict__ status, int32_t* __restrict__ status_rw,
    const int32_t* __restrict__ slots, int32_t* __restrict__ pos,
    const long long* __restrict__ seq_counts, int32_t* __restrict__ items, int64_t items_cap,
    int32_t* __restrict__ n_items, long long* __restrict__ class_counts,
    int32_t* __restrict__ sched_counter, int32_t* __restrict__ n_slots_out, int64_t slot_cap,
    int32_t* __restrict__ merge_list, int32_t* __restrict__ n_merge) {
    extern __shared__ int32_t hist[];  // [cost_cap + 1], SORT_LDS_INTS of slot data, SORT_POS_LDS ranks
    int32_t* s_slot = hist + ((cost_cap + 4) & ~3);
    int32_t* s_pos = s_slot + SORT_LDS_INTS;
    __shared__ long long tmp[17];
    __shared__ long long s_sum[4];
    __shared__ int s_nmerge;
    const int tid = threadIdx.x;
    if (tid == 0) s_nmerge = 0;
    const int st = *status;   // read together with the sizes below
    // total slots and class counts over sequences
    long long n_slots = 0;
    if (tid < 4) s_sum[tid] = 0;
    __syncthreads();
    for (int base = 0; base < B; base += blockDim.x) {
        const int b = base + tid;
        long long ns = 0;
        if (b < B) {
            const SeqDims d = seq_dims(cu, b, Br, Bc, S);
            ns = (long long)d.Tr * d.MS;
            for (int r = 0; r < PLAN_RC; ++r)
                for (int c = 0; c < 3; ++c)
                    atomicAdd((unsigned long long*)&s_sum[c],
                              (unsigned long long)seq_counts[((int64_t)b * PLAN_RC + r) * 3 + c]);
        }
        long long tot;
        block_exclusive_scan(ns, tmp, &tot);
        n_slots += tot;
    }
    if (st != 0) {
        if (tid == 0) {
            if (n_merge) *n_merge = 0;
            *n_items = 0;
            class_counts[0] = class_counts[1] = class_counts[2] = 0;
            if (sched_counter) *sched_counter = 0;
            if (n_slots_out) *n_slots_out = 0;
        }
        return;
    }
    if (n_slots > slot_cap) n_slots = 0;  // cannot happen with a valid plan; no items then
    const bool recs_in_lds = n_slots <= SORT_LDS_RECS;
    const bool cost_in_lds = !recs_in_lds && n_slots <= SORT_LDS_INTS;
    const bool pos_in_lds = n_slots <= SORT_POS_LDS;
    for (int c = tid; c <= cost_cap; c += blockDim.x) hist[c] = 0;
    if (recs_in_lds)
        for (long long i = tid; i < n_slots * (SLOT_WORDS / 4); i += blockDim.x)
            ((int4*)s_slot)[i] = ((const int4*)slots)[i];
    __syncthreads();
    auto slot_cost = [&](long long sl) {   // -1: empty slot
        const int32_t* rec = recs_in_lds ? s_slot + sl * SLOT_WORDS : slots + sl * SLOT_WORDS;
        return rec[7] ? min(rec[6], cost_cap) : -1;
    };
    for (long long sl = tid; sl < n_slots; sl += blockDim.x) {
        const int c = slot_cost(sl);
        if (c >= 0) atomicAdd(&hist[c], 1);
        if (cost_in_lds) s_slot[sl] = c;
    }
    __syncthreads();
    // descending exclusive scan: base[c] = number of valid slots with cost > c
    const int per = ceil_div(cost_cap + 1, (int)blockDim.x);
    long long local = 0;
    for (int t = 0; t < per; ++t) {
        const int rc = tid * per + t;  // reversed index
        if (rc <= cost_cap) local += hist[cost_cap - rc];
    }
    long long total_valid;
    long long run = block_exclusive_scan(local, tmp, &total_valid);
    for (int t = 0; t < per; ++t) {
        const int rc = tid * per + t;
        if (rc <= cost_cap) {
            const int c = cost_cap - rc;
            const int h = hist[c];
            hist[c] = (int32_t)run;
            run += h;
        }
    }
    __syncthreads();
    // stable rank inside each cost: one wave walks the slots in order
    const bool overflow = total_valid * H > items_cap;
    if (!overflow && tid < 64) {
        const int lane = tid;
        for (long long chunk = 0; chunk < n_slots; chunk += 64) {
            const long long sl = chunk + lane;
            int c = -1;
            if (sl < n_slots) c = cost_in_lds ? s_slot[sl] : slot_cost(sl);
            const bool valid = c >= 0;
            const int cost = valid ? c : 0;
            uint64_t eq = __ballot(valid);
            for (int bit = 0; bit < 15; ++bit) {
                const bool bb = (cost >> bit) & 1;
                const uint64_t m1 = __ballot(bb);
                eq &= bb ? m1 : ~m1;
            }
            if (valid) {
                const int before = __popcll(eq & lanemask_lt());
                const int rk = hist[cost] + before;
                if (pos_in_lds) s_pos[sl] = rk; else pos[sl] = rk;
                const bool leader = (eq >> lane) == 1ull;  // highest lane of its group
                __builtin_amdgcn_wave_barrier();
                if (leader) hist[cost] = rk + 1;
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();
    if (!overflow) {
        // every thread gathers the words of U items (ranks from LDS, sequence
        // bounds from global memory, all loads in flight together), then
        // writes them as 16-byte stores
        constexpr int U = 4;
        const long long total = n_slots * H;
        for (long long i0 = tid; i0 < total; i0 += (long long)U * blockDim.x) {
            int4 v0[U], v1[U], v2[U];
            int64_t dst[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const long long idx = i0 + (long long)u * blockDim.x;
                ok[u] = false;
                if (idx < total) {
                    const long long sl = idx / H;
                    const int h = (int)(idx - sl * H);
                    const int32_t* rec = recs_in_lds ? s_slot + sl * SLOT_WORDS : slots + sl * SLOT_WORDS;
                    if (rec[7]) {
                        ok[u] = true;
                        const int b = rec[0];
                        dst[u] = ((int64_t)(pos_in_lds ? s_pos[sl] : pos[sl]) * H + h) * ITEM_WORDS;
                        // seq, head, q tile, kb range, split index, splits, cost; then the
                        // derived words: sequence bounds, first extrema block, slot of split 0
                        v0[u] = int4{b, h, rec[1], rec[4]};
                        v1[u] = int4{rec[5], rec[2], rec[3], rec[6]};
                        v2[u] = int4{cu[b], cu[b + 1], kb_off[b], (int32_t)(sl - rec[2])};
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!ok[u]) continue;
                int4* it = (int4*)(items + dst[u]);
                it[0] = v0[u]; it[1] = v1[u]; it[2] = v2[u]; it[3] = int4{0, 0, 0, 0};
                if (merge_list && v1[u].y == 0 && v1[u].z > 1) {   // split 0 of a split row: one entry per head
                    const int k = atomicAdd(&s_nmerge, 1);
                    int32_t* m = merge_list + (int64_t)k * MERGE_WORDS;
                    const int row0 = v2[u].x + v0[u].z * Br;
                    m[0] = v2[u].w; m[1] = v0[u].y; m[2] = row0; m[3] = min(row0 + Br, v2[u].y); m[4] = v1[u].z;
                    m[5] = m[6] = m[7] = 0;
                }
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        *n_items = overflow ? 0 : (int32_t)(total_valid * H);
        if (overflow) atomicOr(status_rw, FM_STATUS_CAP);
        class_counts[0] = s_sum[0]; class_counts[1] = s_sum[1]; class_counts[2] = s_sum[2];
        if (sched_counter) *sched_counter = 0;
        if (n_slots_out) *n_slots_out = (int32_t)n_slots;
        if (n_merge) *n_merge = overflow ? 0 : s_nmerge;
    }
}

// ------------------------------------------------------------------------
hipError_t launch_extrema(const int32_t* sv, int n_vec, int causal, const int32_t* cu, int B,
                          int64_t N, int Bc, int32_t* kb_off, int32_t* extrema,
                          int64_t extrema_cap, int32_t* n_kblocks, int32_t* status,
                          int n_cu, hipStream_t s) {
    const int64_t kb_bound = (N + Bc - 1) / Bc + B;
    int64_t grid = (kb_bound + 3) / 4;
    grid = std::max<int64_t>(1, std::min<int64_t>(grid, (int64_t)n_cu * 8));
    const size_t lds = 2 * (size_t)(B + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(fm_extrema_kernel, dim3((unsigned)grid), dim3(256), lds, s, sv, n_vec,
                       causal, cu, B, N, Bc, kb_off, extrema, extrema_cap, n_kblocks, status);
    return hipGetLastError();
}

hipError_t launch_plan(const int32_t* sv, int n_vec, int32_t* ext, int64_t ext_cap, int32_t* n_kblocks,
                       int32_t* kb_off_out, const PlanPtrs& p, int n_cu, hipStream_t s) {
    const hipError_t e = launch_extrema(sv, n_vec, p.causal, p.cu, p.B, p.N, p.Bc, kb_off_out, ext, ext_cap,
                                        n_kblocks, p.status_rw, n_cu, s);
    return e != hipSuccess ? e : launch_worklist(p, s);
}

hipError_t launch_worklist(const PlanPtrs& p, hipStream_t s) {
    int32_t* slots = (int32_t*)(p.scratch + p.sl.off_slots);
    int32_t* pos = (int32_t*)(p.scratch + p.sl.off_pos);
    long long* seq_counts = (long long*)(p.scratch + p.sl.off_seq_counts);
    int32_t* sl_off = (int32_t*)(p.scratch + p.sl.off_sl_off);
    hipLaunchKernelGGL(fm_tiles_kernel, dim3((unsigned)p.B * PLAN_RC), dim3(TILES_NTH), 0, s, p.cu, p.B, p.Br, p.Bc, p.S,
                       p.causal, p.kb_off, p.extrema, p.status, slots, seq_counts, sl_off,
                       p.tile_class, p.tile_class_cap, p.sl.slot_cap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)(((p.cost_cap + 4) & ~3) + SORT_LDS_INTS + SORT_POS_LDS) * sizeof(int32_t);
    hipLaunchKernelGGL(fm_sort_kernel, dim3(1), dim3(1024), lds, s, p.cu, p.B, p.H, p.Br, p.Bc,
                       p.S, p.cost_cap, p.kb_off, p.status, p.status_rw, slots, pos, seq_counts, p.items,
                       p.items_cap, p.n_items, (long long*)p.class_counts, p.sched_counter,
                       p.n_slots, p.sl.slot_cap, p.merge_list, p.n_merge);
    return hipGetLastError();
}

}  // namespace fm
