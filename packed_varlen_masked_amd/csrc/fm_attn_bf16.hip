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
//     32w..32w+31.  Every staged K/V tile feeds 256 query rows.  The kernel
//     is persistent: workgroups pull items from the longest-first work list
//     with one atomic counter.
//   * scores are computed transposed, S^T = K Q^T, so that in the MFMA
//     result each lane holds ONE query (lane & 31) and 16 keys per 32x32
//     tile.  Row max / row sum are per-lane reductions plus one exchange
//     with lane ^ 32, and O^T = V^T P^T keeps that ownership, so the
//     online-softmax rescale of O is a per-lane scalar.
//   * K and V tiles sit row-major in LDS ([key][channel], rows padded); the
//     V^T operand is read with the gfx950 LDS transpose read
//     (ds_read_b64_tr_b16).
//   * two groups of four waves (one wave of each per SIMD) run the same
//     step in opposite phase: group 0 issues the MFMAs of S_j = K_j Q^T and
//     O += V_{j-1} P_{j-1}, then the softmax of tile j; group 1 the softmax
//     of tile j-1, then the same MFMAs.  While one wave of a SIMD feeds its
//     matrix unit the other keeps its vector unit busy.  All waves advance
//     together, one workgroup barrier per step.
//   * a 3-deep ring of K and V buffers filled by asynchronous global->LDS
//     copies (inline assembly, waited for explicitly): in step j waves 0-3
//     copy K_{j+2} and its mask vectors, waves 4-7 copy V_{j+1}; a step
//     ends by waiting for the copies of the step before.
//   * long rows are split over several items; each writes an fp32 partial
//     (O, m, l) that the merge kernel combines in split order.
//   * two entry kernels share the item code: the standard one reads the plan
//     from the workspace and pulls items from a counter; the fused one plans
//     a small problem in LDS in every workgroup and runs a static share.
#include <algorithm>

#include "fm_common.hpp"
#include "fm_internal.h"
#include "fm_api.h"
#include "fm_bf16_copies.h"

namespace fm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BR = 256, BC = 64, HD = 128;
constexpr int NW = 8, NTH = 64 * NW;    // 8 waves, 32 query rows each
constexpr int GW = NW / 2;              // waves per ping-pong group
constexpr float LN2 = 0.69314718055994530942f;
constexpr int PART = BR * HD / 2 + 3 * BR;  // 4-byte words per split partial: O as fp16, then m, l, e per row
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
constexpr int KBLK = KBYTES / 1024, VBLK = VBYTES / 1024;   // 1 KB copy blocks: 17, 20
constexpr int MVW = 4 * BC;                        // mask-vector words per tile
static_assert(KCH == bf16c::KCH && VCH == bf16c::VCH && BC == bf16c::BC && NW == 2 * bf16c::GW &&
              KBLK == bf16c::KBLK && VBLK == bf16c::VBLK, "copy table and kernel agree");

// The ring: three K slots, then three V slots, 20 KB each (a K tile fills 17
// KB, the rest of its slot takes the copies that keep every wave's count
// even), then the mask-vector slots.  Copies into the ring are issued with
// inline assembly, so the compiler does not track them: every wait for them
// is explicit (see the step below).
constexpr int SLOT_BYTES = bf16c::SLOT_BLK * 1024;
__shared__ __attribute__((aligned(1024))) char s_kv[6 * SLOT_BYTES];
__shared__ __attribute__((aligned(16))) int32_t s_mv[4 * MVW];   // mask vectors of tile t in slot t mod 4
__shared__ __attribute__((aligned(16))) int32_t s_sink[GW * BC];   // mask rows of absent vectors (never read)
__device__ __attribute__((always_inline)) inline char* kbuf(int i) { return s_kv + i * SLOT_BYTES; }
__device__ __attribute__((always_inline)) inline char* vbuf(int i) { return s_kv + (3 + i) * SLOT_BYTES; }

typedef __attribute__((address_space(3))) char lds_char;
__device__ __attribute__((always_inline)) inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_char*)p;
}
// Asynchronous copy instructions (global -> LDS): 64 lanes x 16 B through
// buffer resource `rs` (byte offset voff per lane; lanes past the resource's
// byte count write zeros), or 64 lanes x 4 B from base + voff, into LDS at
// dst + 16 * lane (4 * lane).  The leading s_nop covers the wait states
// between the scalar writes of the resource / base / M0 and their use.
__device__ __attribute__((always_inline)) inline void dmab16(void* dst, i32x4 rs, uint32_t voff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(voff), "s"(rs), "{m0}"(lds_addr(dst))
                 : "memory");
}
__device__ __attribute__((always_inline)) inline void dma4(void* dst, const void* base, uint32_t voff) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" :: "v"(voff), "s"(base), "{m0}"(lds_addr(dst))
                 : "memory");
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (s_waitcnt immediate; expcnt and lgkmcnt untouched).
template <int N>
__device__ __attribute__((always_inline)) inline void wait_vm() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

// Barrier between items: this wave's LDS operations are complete, its
// global stores may still be in flight (nothing after reads them).
__device__ __attribute__((always_inline)) inline void item_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier between phases.  No implied wait: every wave has already
// waited for the copies the next phase reads, and LDS reads of a phase are
// consumed (hence complete) inside it.  The memory clobber and scheduling
// barriers keep the compiler from moving work across phases.
__device__ __attribute__((always_inline)) inline void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
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

struct Item {
    int b, h, qt, kbb, kbe, sidx, nsp, cost;
    int s_b, e_b, Tc, r0, r1, slot0;
    int64_t hoff;
    const int32_t* xb;
};

struct State {
    float m_run, l_run;
    f32x16 o[4];
};

// Per-wave constants of the item loop.
struct Wave {
    int tid, lane, w, g, t, n, hh, qrow;   // t: wave index inside its group
    int mv_src;        // group 0: stored vector behind mask vector t (-1: absent)
    uint32_t rsb;      // row stride of q/k/v in bytes
    uint32_t vo[5];    // per-lane source byte offsets of the wave's copies in a tile of 64 rows
    bool no_skip;
    bool idle;         // the wave's 32 rows lie past the item's rows: it only copies
};

// MFMA phase, part 1: S^T = K Q^T, two 32-key tiles x 8 k-steps.  K
// fragments are read two k-steps ahead of the MFMAs that use them.
template <typename CP>
__device__ __attribute__((always_inline)) inline void s_part(const char* kl, const bf16x8 (&qf)[8],
                                                             f32x16 (&sacc)[2], int n, int hh, CP&& cp) {
    const char* kp = kl + n * (KCH * 16) + 16 * hh;
    auto kfrag = [&](int t, int s) { return as_bf16x8(*(const u32x4*)(kp + 32 * t * (KCH * 16) + 32 * s)); };
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[t][e] = 0.f;
    bf16x8 ka[3][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t) ka[s][t] = kfrag(t, s);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (s + 2 < 8) {
#pragma unroll
            for (int t = 0; t < 2; ++t) ka[(s + 2) % 3][t] = kfrag(t, s + 2);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
            sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s % 3][t], qf[s], sacc[t], 0, 0, 0);
        cp(s);
    }
    // keep the order: 4 reads, then (2 reads, 2 MFMAs) x 6, then 4 MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int s = 0; s < 6; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// MFMA phase, part 2: O^T += V^T P^T; V^T read with the LDS transpose read,
// one 16-key group ahead of the MFMAs that use it.
__device__ __attribute__((always_inline)) inline void pv_part(const char* vb, const bf16x8 (&pb)[2][2],
                                                              State& st, int lane) {
    const int hh = lane >> 5, grp = lane >> 4, gi = lane & 15;
    // lane part of the address: rows 4hh + gi/4, chunk 2(grp&1) + (gi&3)/2, half gi&1
    const char* vl = vb + (4 * hh + (gi >> 2)) * (VCH * 16) + 16 * (2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);
    auto vfrag = [&](int kg, int dt) {   // key group kg = 2t + c: keys 16kg..16kg+15
        const char* p = vl + 16 * kg * (VCH * 16) + 64 * dt;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(void*)p);
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(void*)(p + 8 * VCH * 16));
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    bf16x8 va[2][4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) va[0][dt] = vfrag(0, dt);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
        if (kg + 1 < 4) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) va[(kg + 1) & 1][dt] = vfrag(kg + 1, dt);
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kg & 1][dt], pb[kg >> 1][kg & 1], st.o[dt], 0, 0, 0);
    }
    // keep the order: 8 reads, then (8 reads, 4 MFMAs) x 3, then 4 MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int kg = 0; kg < 3; ++kg) {
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Rows [s, e) of a wave's 32 query rows as a bit mask (bit n = row n; s, e
// relative to the wave's first row, clamped; empty when e <= s).
__device__ __attribute__((always_inline)) inline uint32_t row_bits(int s, int e) {
    s = min(max(s, 0), 32);
    e = min(max(e, s), 32);
    const int w = e - s;   // s <= 31 whenever w > 0
    return w >= 32 ? 0xffffffffu : ((1u << w) - 1u) << (s & 31);
}
// Interval endpoint x (any int32 row index) relative to the wave's first row
// q0 >= 0, clamped below at 0 before the subtraction: max(x, q0) - q0 lies
// in [0, 2^31) and cannot wrap, where x - q0 would for x < INT32_MIN + q0.
__device__ __attribute__((always_inline)) inline int rel_row(int x, int q0) { return max(x, q0) - q0; }

// x, or y where the lane's bit of the 64-lane mask {lo: lanes 0-31, hi:
// lanes 32-63} is set (one v_cndmask with the mask in scalar registers).
__device__ __attribute__((always_inline)) inline float select_lanes(float x, float y, uint32_t lo, uint32_t hi) {
    const uint64_t m = ((uint64_t)hi << 32) | lo;
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "s"(m));
    return r;
}

// Element masks of a tile and the row maximum of its scaled scores.
// Register e of tile t holds key 32t + 8(e>>2) + 4hh + (e&3) for query row
// q0 + (lane & 31), q0 the wave's first row.  Where the tile needs element
// masks, lane L first builds the 32-row mask of key c0 + L: rows above the
// diagonal (causal: row < key), every row when the key lies past the
// sequence end, and the rows of the column intervals [LTS, LTE) and
// [UTS, UTE) (FlashMask article, §3: masked rows of a key column).  The
// masks of keys k and k + 4 read from lanes k and k + 4 are then exactly the
// 64-lane condition that selects -inf for register e.
__device__ __attribute__((always_inline)) inline float mask_max(f32x16 (&sacc)[2], bool causal, bool ragged, bool iv,
                                                                int c0, int c1, int q0, const int32_t* cmv,
                                                                float sl2, int lane) {
    if (causal || ragged || iv) {
        const int key = c0 + lane;
        uint32_t mk = causal ? row_bits(0, key - q0) : 0u;
        if (key >= c1) mk = 0xffffffffu;
        if (iv)
            mk |= row_bits(rel_row(cmv[lane], q0), rel_row(cmv[BC + lane], q0)) |
                  row_bits(rel_row(cmv[2 * BC + lane], q0), rel_row(cmv[3 * BC + lane], q0));
        const int mki = (int)mk;
        const float ninf = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int k0 = 32 * t + 8 * (e >> 2) + (e & 3);
                const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane(mki, k0);
                const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(mki, k0 + 4);
                sacc[t][e] = select_lanes(sacc[t][e], ninf, lo, hi);
            }
    }
    float mq[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) mq[e & 3] = fmaxf(mq[e & 3], sacc[t][e]);
    return halves_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]))) * sl2;
}

// Exponentials of a tile against the running max, after the lazy max
// update: the max used for the exponentials moves only when a score exceeds
// it by more than 2^RESCALE_LOG2 (p then stays <= 2^8).  Returns the factor
// alpha by which O and l must be rescaled (1 when the max did not move);
// the new row sum is added to l after that rescale by the caller.
template <bool DROP>
__device__ __attribute__((always_inline)) inline float exp_tile(const f32x16 (&sacc)[2], float mx, State& st,
                                                                bf16x8 (&pb)[2][2], float sl2, float& rsum,
                                                                const DropW& dw, int drop_t, float drop_ks) {
    float alpha = 1.f;
    if (__any(mx > st.m_run + RESCALE_LOG2)) {
        const float m_new = fmaxf(st.m_run, mx);
        alpha = __builtin_amdgcn_exp2f(st.m_run - (m_new == -INFINITY ? 0.f : m_new));
        st.m_run = m_new;
    }
    const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][8 * c + e], sl2, -m_use));
                rs[e & 3] += p;
                if constexpr (DROP) {   // the row sum keeps every p; O gets the kept ones, scaled
                    const uint32_t byte = (dw.w[2 * t + c][e >> 2] >> (8 * (e & 3))) & 0xffu;
                    pb[t][c][e] = (__bf16)(byte >= (uint32_t)drop_t ? p * drop_ks : 0.f);
                } else {
                    pb[t][c][e] = (__bf16)p;
                }
            }
        }
    }
    rsum = halves_sum((rs[0] + rs[1]) + (rs[2] + rs[3]));
    return alpha;
}

// ---- copies -----------------------------------------------------------
// Group 0 copies K tiles (and the mask vectors), group 1 copies V tiles: a
// tile is 20 blocks of 1 KB in its slot, wave t of the group fills blocks
// t, t+4, ..., t+16 with one copy instruction each (lane L of a block
// carries chunk 64*blk + L of the tile, i.e. row q / CH, chunk q % CH;
// chunks >= 16 are row padding).
constexpr int VIS_CAP = FM_MAX_COST + 1;   // visited key blocks per item
constexpr int WIN_CAP = VIS_CAP / 64;      // 64-block windows of the visit scan

// Tile geometry of key block kb of the item: first row, last valid row
// index inside the tile, and the byte offset of its first row from the
// item's head base.
struct Tile {
    int c0, last;
    size_t off;
};
__device__ __attribute__((always_inline)) inline Tile tile_at(const Item& I, const Wave& Wv, int kb) {
    Tile t;
    t.c0 = I.s_b + kb * BC;
    t.last = min(BC, I.e_b - t.c0) - 1;
    t.off = (size_t)t.c0 * Wv.rsb;
    return t;
}

// Buffer resource of the K or V rows of a tile that lie inside the
// sequence (rows 0..last from `src`): reads of rows past them return zeros,
// so the last tile of a sequence needs no clamped addresses.  Zero rows give
// scores that the tile's element mask sets to -inf and V rows that meet
// P = 0: they add exactly nothing.
__device__ __attribute__((always_inline)) inline i32x4 tile_rsrc(const Wave& Wv, const char* src, int last) {
    const uint64_t b = (uint64_t)(uintptr_t)src;
    i32x4 d;
    d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    d[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));   // stride 0
    d[2] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(last + 1) * Wv.rsb));
    d[3] = 0x00020000;   // raw 32-bit access
    return d;
}
// Block copy i (0..4) of this wave for the tile behind `rs` into the slot at
// `dst`.
__device__ __attribute__((always_inline)) inline void copy_one(const Wave& Wv, i32x4 rs, char* dst, int i) {
    dmab16(dst + 1024 * bf16c::copy_block(Wv.t, i), rs, Wv.vo[i]);
}
// This wave's five block copies of a tile.
__device__ __attribute__((always_inline)) inline void copy_tile(const Wave& Wv, i32x4 rs, char* dst) {
#pragma unroll
    for (int i = 0; i < 5; ++i) copy_one(Wv, rs, dst, i);
}

// Group 0: mask vector t of the tile (absent vectors go to the sink).
__device__ __attribute__((always_inline)) inline void copy_mask(const AttnArgs& a, const Wave& Wv, const Tile& tl,
                                                                int32_t* slot) {
    const bool own = Wv.mv_src >= 0;
    const int32_t* src = a.sv + (own ? (int64_t)Wv.mv_src * a.N : 0) + tl.c0;
    dma4(own ? slot + Wv.t * BC : s_sink + Wv.t * BC, src, 4u * (uint32_t)min(Wv.lane, tl.last));
}

// First tile of an item: group 0 copies its K and mask vectors into slot 0,
// group 1 its V into slot 0.
__device__ __attribute__((always_inline)) inline void copy_tile_pair(const AttnArgs& a, const Item& I, const Wave& Wv,
                                                                     const char* Kh, const char* Vh, int kb) {
    const Tile tl = tile_at(I, Wv, kb);
    if (Wv.g == 0) {
        copy_tile(Wv, tile_rsrc(Wv, Kh + tl.off, tl.last), kbuf(0));
        copy_mask(a, Wv, tl, s_mv);
    } else {
        copy_tile(Wv, tile_rsrc(Wv, Vh + tl.off, tl.last), vbuf(0));
    }
}
constexpr int BATCH_G0 = 6, BATCH_G1 = 5;   // copy instructions per wave per step (groups 0, 1)

// Visit queue: key blocks of the visited tiles j .. j+3 (indices past the
// item's last visited tile repeat it) and the interval flags of j .. j+3.
struct Queue {
    int kp, k0, k1, k2, k3;   // kp: tile j - 1
    uint32_t iv;   // bit i (i < 4): tile j + i needs the interval vectors; bit 4: tile j - 1
};

// Visit lists, entry = key block | interval flag << 15.  The standard kernel
// builds the list of its current item here from the block extrema; the fused
// kernel keeps the lists of every q tile of its plan here.
__shared__ uint16_t s_vis[VIS_CAP];
__shared__ uint64_t s_wvis[WIN_CAP], s_wiv[WIN_CAP];
__shared__ int32_t s_wcnt[WIN_CAP];

__device__ __attribute__((always_inline)) inline int vis_entry(const uint16_t* vis, int i) {
    return __builtin_amdgcn_readfirstlane((int)vis[i]);
}

// Ring slots of step j: K_j and V_j sit in slot u0 = j mod 3, K_{j+1} and
// V_{j+1} in u1, and u2 = (j+2) mod 3 = (j-1) mod 3 still holds V_{j-1}.
struct Slots {
    int u0, u1, u2;
    __device__ void next() { const int t = u0; u0 = u1; u1 = u2; u2 = t; }
};

// Softmax of one tile (all vector work): element masks where the tile
// needs them, the row max, the lazy max update, P in bf16 and its row sum.
// Returns alpha, the factor by which O and l (relative to the old max) must
// be rescaled; the caller applies it and adds the row sum to l.
template <bool DROP>
__device__ __attribute__((always_inline)) inline float softmax_tile(const AttnArgs& a, const Item& I, const Wave& Wv,
                                                                    f32x16 (&sacc)[2], int kb, bool iv,
                                                                    const int32_t* cmv, State& st, bf16x8 (&pb)[2][2],
                                                                    float& rsum) {
    const int c0 = I.s_b + kb * BC, c1 = min(c0 + BC, I.e_b);
    // the causal rule can mask a pair of this wave's rows only when the
    // tile's last key lies past the wave's first row
    const bool causal = a.causal && (c1 - 1 > Wv.qrow - Wv.n);
    const float mx = mask_max(sacc, causal, (c1 - c0) < BC, iv, c0, c1, Wv.qrow - Wv.n, cmv, a.scale_log2, Wv.lane);
    DropW dw;
    if constexpr (DROP) dw = drop_words<true>(a.seed_lo, a.seed_hi, a.offset, Wv.qrow, kb, I.h, Wv.hh);
    return exp_tile<DROP>(sacc, mx, st, pb, a.scale_log2, rsum, dw, a.drop_t, a.drop_ks);
}

// Step j of the KV loop, j = 0..T-1 (all waves in step).  Both groups
// compute S_j = K_j Q^T and O += V_{j-1} P_{j-1} on MFMA and the softmax
// of one tile in the step, in opposite orders so that the two waves of a
// SIMD (one per group) keep its matrix unit and its vector unit busy at the
// same time:
//   group 0: S_j and PV_{j-1} (MFMA), then the softmax of tile j (P_j);
//   group 1: the softmax of tile j-1 (S_{j-1}, kept from the step before),
//            then PV_{j-1} and S_j.
// O is rescaled by the softmax's alpha before the next PV adds to it.
// P_{-1} is zero and the V slot of step 0 holds zeros, so step 0 adds
// exactly nothing to O; the last tile's product (and, for group 1, its
// softmax) follows the loop.  Group 0 copies K_{j+2} into K slot u2 and its
// mask vectors into mask slot (j+2) mod 4, group 1 copies V_{j+1} into V
// slot u1, all last read in step j-1; the copy instructions sit between the
// MFMAs of S_j, so that the CU's load path takes them while the matrix unit
// works.  A step ends by waiting for the previous step's copies, then a
// barrier.
template <int G, bool DROP>
__device__ __attribute__((always_inline)) inline void kv_step(
    const AttnArgs& a, const Item& I, Queue& Qu, const Wave& Wv, Slots& sl, int j, int T, bool& rec_pending,
    int fv, int& nrec, int n_items, const bf16x8 (&qf)[8], f32x16 (&sacc)[2], bf16x8 (&pb)[2][2],
    State& st, const char* Kh, const char* Vh, const uint16_t* vis) {
    const int nk_raw = vis[min(j + 4, T - 1)];
    if (rec_pending) {   // wave 0: the next item's record, ahead of this step's copies
        const int nx = (int)gridDim.x + __builtin_amdgcn_readfirstlane(fv);   // fetch value -> item
        if (nx < n_items && Wv.lane < ITEM_WORDS) nrec = a.items[(int64_t)nx * ITEM_WORDS + Wv.lane];
        rec_pending = false;
    }
    if constexpr (G == 0) {
        const Tile tl = tile_at(I, Wv, Qu.k2);
        const i32x4 rs = tile_rsrc(Wv, Kh + tl.off, tl.last);
        char* kd = kbuf(sl.u2);
        int32_t* md = s_mv + ((j + 2) & 3) * MVW;
        s_part(kbuf(sl.u0), qf, sacc, Wv.n, Wv.hh, [&](int s) {
            if (s < 5) copy_one(Wv, rs, kd, s);
            else if (s == 5) copy_mask(a, Wv, tl, md);
        });
        pv_part(vbuf(sl.u2), pb, st, Wv.lane);
        float rsum;
        const float alpha =
            softmax_tile<DROP>(a, I, Wv, sacc, Qu.k0, (Qu.iv & 1u) != 0, s_mv + (j & 3) * MVW, st, pb, rsum);
        if (alpha != 1.f) {   // rare: the running max moved
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) st.o[dt][e] *= alpha;
        }
        st.l_run = st.l_run * alpha + rsum;
    } else {
        const Tile tl = tile_at(I, Wv, Qu.k1);
        const i32x4 rs = tile_rsrc(Wv, Vh + tl.off, tl.last);
        char* vd = vbuf(sl.u1);
        if (j > 0) {
            float rsum;
            const float alpha =
                softmax_tile<DROP>(a, I, Wv, sacc, Qu.kp, (Qu.iv & 16u) != 0, s_mv + ((j - 1) & 3) * MVW, st, pb, rsum);
            if (alpha != 1.f) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) st.o[dt][e] *= alpha;
            }
            st.l_run = st.l_run * alpha + rsum;
        }
        pv_part(vbuf(sl.u2), pb, st, Wv.lane);
        s_part(kbuf(sl.u0), qf, sacc, Wv.n, Wv.hh, [&](int s) {
            if (s < 5) copy_one(Wv, rs, vd, s);
        });
    }
    const int nk = __builtin_amdgcn_readfirstlane(nk_raw);
    Qu.kp = Qu.k0;
    Qu.k0 = Qu.k1; Qu.k1 = Qu.k2; Qu.k2 = Qu.k3; Qu.k3 = nk & 0x7fff;
    Qu.iv = ((Qu.iv >> 1) & 7u) | ((uint32_t)(nk >> 15) << 3) | ((Qu.iv & 1u) << 4);
    sl.next();
    if constexpr (G == 0) wait_vm<BATCH_G0>(); else wait_vm<BATCH_G1>();
    phase_barrier();
}

// Step j for a wave without rows: the same copies, queue, waits and
// barrier as kv_step, none of the products or the softmax.
template <int G>
__device__ __attribute__((always_inline)) inline void kv_step_idle(const AttnArgs& a, const Item& I, Queue& Qu,
                                                                   const Wave& Wv, Slots& sl, int j, int T,
                                                                   bool& rec_pending, int fv, int& nrec, int n_items,
                                                                   const char* Kh, const char* Vh, const uint16_t* vis) {
    const int nk_raw = vis[min(j + 4, T - 1)];
    if (rec_pending) {
        const int nx = (int)gridDim.x + __builtin_amdgcn_readfirstlane(fv);
        if (nx < n_items && Wv.lane < ITEM_WORDS) nrec = a.items[(int64_t)nx * ITEM_WORDS + Wv.lane];
        rec_pending = false;
    }
    if constexpr (G == 0) {
        const Tile tl = tile_at(I, Wv, Qu.k2);
        const i32x4 rs = tile_rsrc(Wv, Kh + tl.off, tl.last);
        char* kd = kbuf(sl.u2);
#pragma unroll
        for (int s = 0; s < 5; ++s) copy_one(Wv, rs, kd, s);
        copy_mask(a, Wv, tl, s_mv + ((j + 2) & 3) * MVW);
    } else {
        const Tile tl = tile_at(I, Wv, Qu.k1);
        const i32x4 rs = tile_rsrc(Wv, Vh + tl.off, tl.last);
        char* vd = vbuf(sl.u1);
#pragma unroll
        for (int s = 0; s < 5; ++s) copy_one(Wv, rs, vd, s);
    }
    const int nk = __builtin_amdgcn_readfirstlane(nk_raw);
    Qu.kp = Qu.k0;
    Qu.k0 = Qu.k1; Qu.k1 = Qu.k2; Qu.k2 = Qu.k3; Qu.k3 = nk & 0x7fff;
    Qu.iv = ((Qu.iv >> 1) & 7u) | ((uint32_t)(nk >> 15) << 3) | ((Qu.iv & 1u) << 4);
    sl.next();
    if constexpr (G == 0) wait_vm<BATCH_G0>(); else wait_vm<BATCH_G1>();
    phase_barrier();
}

// ---- per-launch and per-item set-up ----------------------------------
__device__ __attribute__((always_inline)) inline void wave_setup(const AttnArgs& a, Wave& Wv) {
    Wv.tid = threadIdx.x; Wv.lane = Wv.tid & 63; Wv.w = __builtin_amdgcn_readfirstlane(Wv.tid >> 6);
    Wv.g = Wv.w / GW; Wv.t = Wv.w % GW; Wv.n = Wv.lane & 31; Wv.hh = Wv.lane >> 5;
    Wv.no_skip = (a.flags & FM_FLAG_NO_SKIP) != 0;
    Wv.rsb = (uint32_t)(a.H * HD * 2);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const uint32_t cp = bf16c::copy_lane(Wv.g, Wv.t, i, Wv.lane);
        Wv.vo[i] = (cp & 0xffu) * Wv.rsb + (cp >> 8);
    }
    // Stored vector behind each logical mask vector (LTS, LTE, UTS, UTE) for
    // the accepted (n_vec, causal) pairs; wave t of group 0 stages vector t.
    // Absent ones take their default (LTE: N; UTS, UTE: 0), written into
    // every mask slot once.
    auto vsrc = [&](int t) {
        return t == 0 ? 0
             : t == 1 ? ((a.n_vec == 4 || (a.causal && a.n_vec == 2)) ? 1 : -1)
             : t == 2 ? (a.n_vec == 4 ? 2 : -1)
             : (a.n_vec == 4 ? 3 : (!a.causal && a.n_vec == 2) ? 1 : -1);
    };
    Wv.mv_src = Wv.g == 0 ? vsrc(Wv.t) : -1;
    for (int i = Wv.tid; i < 4 * MVW; i += NTH) {
        const int t = (i % MVW) / BC;
        if (vsrc(t) < 0) s_mv[i] = t == 1 ? (int)a.N : 0;
    }
}

// Item record (LDS, same for every lane) -> scalar fields.
__device__ __attribute__((always_inline)) inline Item item_of(const AttnArgs& a, const int32_t* rec) {
    auto r = [&](int i) { return __builtin_amdgcn_readfirstlane(rec[i]); };
    Item I;
    I.b = r(0); I.h = r(1); I.qt = r(2); I.kbb = r(3); I.kbe = r(4);
    I.sidx = r(5); I.nsp = r(6); I.cost = r(7);
    I.s_b = r(8); I.e_b = r(9);
    const int kb_base = r(10);
    I.slot0 = r(11);
    I.Tc = ceil_div(I.e_b - I.s_b, BC);
    I.r0 = I.s_b + I.qt * BR; I.r1 = min(I.r0 + BR, I.e_b);
    I.xb = a.extrema + (int64_t)kb_base * 8;
    I.hoff = (int64_t)I.h * HD;
    return I;
}

// ---- epilogue -----------------------------------------------------------
// bf16 row of out and its lse from an unnormalised O (per lane: query row
// `qrow`, channels 32dt + 8g + 4hh + 0..3 of o[dt][4g .. 4g+3]).
// Output rows of a finished item, through LDS: every wave writes its 32
// rows of O / l (bf16) into its own 8.5 KB of the free K/V ring (rows of
// 272 B: 16 bf16 groups of 8 B per lane land in distinct banks), then reads
// them back 16 B per lane and writes 4 whole rows per store instruction
// (1 KB, 256 B per row) instead of 16 scattered 8-byte pieces per lane.
// Waves 0-3 stage in K slots 1-2, waves 4-7 in V slots 1-2: K slot 0 and V
// slot 0 stay free for the next item's first tile, copied meanwhile.
constexpr int OST_ROW = 272, OST_WAVE = 32 * OST_ROW;
static_assert(GW * OST_WAVE <= 2 * SLOT_BYTES, "output staging fits in two ring slots");
__device__ __attribute__((always_inline)) inline void write_rows(const AttnArgs& a, const Wave& Wv, const Item& I,
                                                                 const State& st, float inv) {
    char* stg = (Wv.w < GW ? kbuf(1) : vbuf(1)) + (Wv.w % GW) * OST_WAVE;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 wv;
            wv.x = bf16_bits(st.o[dt][4 * g] * inv) | (bf16_bits(st.o[dt][4 * g + 1] * inv) << 16);
            wv.y = bf16_bits(st.o[dt][4 * g + 2] * inv) | (bf16_bits(st.o[dt][4 * g + 3] * inv) << 16);
            *(u32x2*)(stg + Wv.n * OST_ROW + 2 * (32 * dt + 8 * g + 4 * Wv.hh)) = wv;
        }
    const int64_t rs = (int64_t)a.H * HD;   // row stride of out (elements)
    const int q0 = I.r0 + 32 * Wv.w;       // the wave's first row
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (Wv.lane >> 4), c = Wv.lane & 15;   // row, 16-byte chunk
        const u32x4 v = *(const u32x4*)(stg + r * OST_ROW + 16 * c);
        if (q0 + r < I.r1) *(u32x4*)((uint16_t*)a.out + (int64_t)(q0 + r) * rs + I.hoff + 8 * c) = v;
    }
}
__device__ __attribute__((always_inline)) inline void write_lse(const AttnArgs& a, const Wave& Wv, const Item& I,
                                                                float m, float l) {
    if (Wv.hh == 0) a.lse[(int64_t)I.h * a.N + Wv.qrow] = l > 0.f ? (m + __log2f(l)) * LN2 : -INFINITY;
}

// Split rows: every split writes its partial, combined by
// fm_merge_bf16_kernel in split order after the attention launch.  Per row:
// O / l of the split as fp16, scaled by 2^-e with e chosen per row so that
// the row's largest magnitude lies below 2^15 (no overflow, 11 significant
// bits however large or small V is), then m, l and e as 4-byte words.
// Partial of split s, head h at ((slot0 + s) * H + h) * PART words; its O
// part is lane-major: the 8 values of channel groups (dt, 2gp) and
// (dt, 2gp + 1) of lane L of wave w are 16 bytes at word
// ((8 w + 2 dt + gp) * 64 + L) * 4, so every store instruction of a wave
// writes 1 KB contiguously.
__device__ __attribute__((always_inline)) inline int part_index(int w, int dt, int gp, int lane) {
    return ((8 * w + 2 * dt + gp) * 64 + lane) * 4;
}
__device__ inline uint32_t f16_pair(float x, float y) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y) << 16);
}

__device__ __attribute__((always_inline)) inline void epilogue(const AttnArgs& a, const Wave& Wv, const Item& I,
                                                               const State& st) {
    const float l = st.l_run, inv = l > 0.f ? 1.f / l : 0.f;
    if (I.nsp <= 1) {
        // every wave is past its last ring read and its copies are drained:
        // the ring is free for the output staging
        phase_barrier();
        write_rows(a, Wv, I, st, inv);
        if (Wv.qrow < I.r1) write_lse(a, Wv, I, st.m_run, l);
        return;
    }
    float mx = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(st.o[dt][j]));
    mx = halves_max(mx * inv);   // both lanes of the row take the same scale
    // mx < 2^(u + 1) with u its binary exponent: e = u - 14 puts it below 2^15
    const int u = (int)((__float_as_uint(mx) >> 23) & 0xff) - 127;
    const int e = mx > 0.f ? min(max(u - 14, -100), 113) : 0;
    const float sc = __uint_as_float((uint32_t)(127 - e) << 23) * inv;   // 2^-e / l
    uint32_t* po = (uint32_t*)a.partial + ((int64_t)(I.slot0 + I.sidx) * a.H + I.h) * PART;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            const int j = 8 * gp;
            // non-temporal: the partials are read once, by the merge launch;
            // streaming them out of the L2 keeps the end of this launch short
            __builtin_nontemporal_store(u32x4{f16_pair(st.o[dt][j] * sc, st.o[dt][j + 1] * sc),
                                              f16_pair(st.o[dt][j + 2] * sc, st.o[dt][j + 3] * sc),
                                              f16_pair(st.o[dt][j + 4] * sc, st.o[dt][j + 5] * sc),
                                              f16_pair(st.o[dt][j + 6] * sc, st.o[dt][j + 7] * sc)},
                                        (u32x4*)(po + part_index(Wv.w, dt, gp, Wv.lane)));
        }
    const int lr = 32 * Wv.w + Wv.n;
    if (Wv.hh == 0) {
        po[BR * HD / 2 + lr] = __float_as_uint(st.m_run);
        po[BR * HD / 2 + BR + lr] = __float_as_uint(l);
        po[BR * HD / 2 + 2 * BR + lr] = (uint32_t)e;
    }
}

// Q^T fragments (B operand) of the wave's 32 query rows: lane holds query
// qrow, channels 16s + 8hh .. +7 in qf[s]; rows at or past r1 are zero.
__device__ __attribute__((always_inline)) inline void load_q_row(const AttnArgs& a, int qrow, int hh, int r1,
                                                                 int64_t hoff, bf16x8 (&qf)[8]) {
    if (qrow < r1) {
        const uint16_t* qp = (const uint16_t*)a.q + (int64_t)qrow * ((int64_t)a.H * HD) + hoff + 8 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*(const u32x4*)(qp + 16 * s));
    } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
}
__device__ __attribute__((always_inline)) inline void load_q(const AttnArgs& a, const Wave& Wv, int r1, int64_t hoff,
                                                             bf16x8 (&qf)[8]) {
    load_q_row(a, Wv.qrow, Wv.hh, r1, hoff, qf);
}
// The block extrema of the wave's first visit window of an item (lane =
// key block lo + 64 w + lane, zero past hi).
__device__ __attribute__((always_inline)) inline void load_window0(const Item& I, const Wave& Wv, int lo, int hi,
                                                                   u32x4& x0, u32x4& x1) {
    x0 = u32x4{0, 0, 0, 0};
    x1 = u32x4{0, 0, 0, 0};
    const int kb = lo + 64 * Wv.w + Wv.lane;
    if (kb < hi) {
        x0 = *(const u32x4*)(I.xb + (int64_t)kb * 8);
        x1 = *(const u32x4*)(I.xb + (int64_t)kb * 8 + 4);
    }
}

// ---- one work item ----------------------------------------------------
// Q tile in registers, the first K/V tile on its way, the visit list, the KV
// loop, the epilogue.  STD: the visit list is built here from the block
// extrema in global memory (FlashMask article §3.2 rules) and the next
// item's record is prefetched during the loop; otherwise the list is ready
// in s_vis at `vis_off` (fused path).
// pre (standard kernel): the item's Q fragments, the extrema of its first
// visit window (pxw0, pxw1) and its first tile (pre_kb) were loaded by the
// item before it, during that item's output; `handover(T)` is called by
// every wave once the KV loop is done, to do the same for the next item.
template <bool STD, bool DROP, typename Handover>
__device__ __attribute__((always_inline)) inline void run_item(const AttnArgs& a, Wave& Wv, const Item& I,
                                                               int vis_off, bool& rec_pending, int fv, int& nrec,
                                                               int n_items, bf16x8 (&qf)[8], int pre_kb, bool pre,
                                                               const u32x4& pxw0, const u32x4& pxw1,
                                                               Handover&& handover) {
    const int tid = Wv.tid, lane = Wv.lane, w = Wv.w;
    const int64_t rs = (int64_t)a.H * HD;
    Wv.qrow = I.r0 + 32 * w + Wv.n;
    // a wave whose rows all lie past the q tile's end (short sequences) has
    // no products to compute: it runs the copy-only step below, and its O,
    // m and l stay empty (it writes no row)
    Wv.idle = I.r0 + 32 * w >= I.r1;
    const char* Kh = (const char*)a.k + I.hoff * 2;
    const char* Vh = (const char*)a.v + I.hoff * 2;
    const int lo = Wv.no_skip ? 0 : I.kbb, hi = Wv.no_skip ? I.Tc : I.kbe;

    // loads in the order they are needed (they complete in issue order): the
    // block extrema of the wave's first visit window, the first K/V tile
    // (kb_begin is visited by construction of the work list), then Q, which
    // the loop needs last
    const int nwin = (STD && lo < hi) ? ceil_div(hi - lo, 64) : 0;
    u32x4 xw0 = {0, 0, 0, 0}, xw1 = {0, 0, 0, 0};
    if constexpr (STD) {
        if (pre) {
            xw0 = pxw0;
            xw1 = pxw1;
        } else if (w < nwin) {
            load_window0(I, Wv, lo, hi, xw0, xw1);
        }
    }
    // (the fused kernel loaded Q before planning and may have copied the
    // first tile already, as may the standard kernel's previous item: pre_kb)
    if (!Wv.no_skip && lo < hi && lo != pre_kb) copy_tile_pair(a, I, Wv, Kh, Vh, lo);
    if constexpr (STD) {
        if (!pre) load_q(a, Wv, I.r1, I.hoff, qf);
    }

    int T;
    const uint16_t* vis;
    if constexpr (STD) {
        // windows of 64 key blocks, one extrema row per lane; wave w takes
        // windows w, w+8, ...
        for (int j = w; j < nwin; j += NW) {
            const int kb = lo + 64 * j + lane;
            bool v = false, iv = false;
            if (kb < hi) {
                const u32x4 x0 = j == w ? xw0 : *(const u32x4*)(I.xb + (int64_t)kb * 8);
                const u32x4 x1 = j == w ? xw1 : *(const u32x4*)(I.xb + (int64_t)kb * 8 + 4);
                const int x[8] = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                  (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
                const int c0 = I.s_b + kb * BC, c1 = min(c0 + BC, I.e_b);
                const TileInfo ti = classify_tile(I.r0, I.r1, c0, c1, x, a.causal);
                v = !ti.causal_full && (ti.cls != CLS_FULL || Wv.no_skip);
                iv = ti.need_lt || ti.need_ut;
            }
            const uint64_t vm = __ballot(v), im = __ballot(iv);
            if (lane == 0) { s_wvis[j] = vm; s_wiv[j] = im; s_wcnt[j] = __popcll(vm); }
        }
        __syncthreads();
        T = 0;
        for (int j0 = 0; j0 < nwin; j0 += 64) {   // total visited tiles
            const int j = j0 + lane;
            T += __reduce_add_sync(~0ull, j < nwin ? s_wcnt[j] : 0);
        }
        T = __builtin_amdgcn_readfirstlane(T);
        for (int j = w; j < nwin; j += NW) {
            int base = 0;
            for (int j0 = 0; j0 < j; j0 += 64) {
                const int jj = j0 + lane;
                base += __reduce_add_sync(~0ull, jj < j ? s_wcnt[jj] : 0);
            }
            const uint64_t vm = s_wvis[j], im = s_wiv[j];
            if ((vm >> lane) & 1ull) {
                const int pos = base + __popcll(vm & lanemask_lt());
                if (pos < VIS_CAP) s_vis[pos] = (uint16_t)((lo + 64 * j + lane) | (int)(((im >> lane) & 1ull) << 15));
            }
        }
        T = min(T, VIS_CAP);
        vis = s_vis;
        __syncthreads();
    } else {
        T = I.cost;
        vis = s_vis + vis_off;
    }

    State st;
    st.m_run = -INFINITY; st.l_run = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.o[dt][e] = 0.f;
    if (T > 0) {
        Queue Qu;
        const int e0 = vis_entry(vis, 0), e1 = vis_entry(vis, min(1, T - 1)), e2 = vis_entry(vis, min(2, T - 1)),
                  e3 = vis_entry(vis, min(3, T - 1));
        Qu.k0 = e0 & 0x7fff; Qu.k1 = e1 & 0x7fff; Qu.k2 = e2 & 0x7fff; Qu.k3 = e3 & 0x7fff;
        Qu.iv = (uint32_t)((e0 >> 15) | ((e1 >> 15) << 1) | ((e2 >> 15) << 2) | ((e3 >> 15) << 3));
        // prologue: the Q fragments, K_0 (with its mask vectors) and V_0
        // land before step 0; K_1 (and masks) is waited for at the end of
        // step 0.  The full wait also tells the compiler that the Q loads are
        // complete: it cannot see the copies, which share the hardware
        // counter, so any wait it placed for the Q loads inside the loop
        // would wait for the copies in flight.  V slot 2, read in step 0
        // against P = 0, is cleared.
        if (Wv.no_skip) copy_tile_pair(a, I, Wv, Kh, Vh, Qu.k0);
        wait_vm<0>();
        if (Wv.g == 0) {
            const Tile t1 = tile_at(I, Wv, Qu.k1);
            copy_tile(Wv, tile_rsrc(Wv, Kh + t1.off, t1.last), kbuf(1));
            copy_mask(a, Wv, t1, s_mv + MVW);
        }
        for (int i = tid; i < SLOT_BYTES / 16; i += NTH) ((u32x4*)vbuf(2))[i] = u32x4{0, 0, 0, 0};
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
        phase_barrier();
        f32x16 sacc[2];
        bf16x8 pb[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int c = 0; c < 2; ++c) pb[t][c] = as_bf16x8(u32x4{0, 0, 0, 0});   // P_{-1}
        Slots sl{0, 1, 2};
        Qu.kp = Qu.k0;
        if (Wv.idle) {
            if (Wv.g == 0)
                for (int j = 0; j < T; ++j)
                    kv_step_idle<0>(a, I, Qu, Wv, sl, j, T, rec_pending, fv, nrec, n_items, Kh, Vh, vis);
            else
                for (int j = 0; j < T; ++j)
                    kv_step_idle<1>(a, I, Qu, Wv, sl, j, T, rec_pending, fv, nrec, n_items, Kh, Vh, vis);
        } else if (Wv.g == 0)
            for (int j = 0; j < T; ++j)
                kv_step<0, DROP>(a, I, Qu, Wv, sl, j, T, rec_pending, fv, nrec, n_items, qf, sacc, pb, st, Kh, Vh, vis);
        else
            for (int j = 0; j < T; ++j)
                kv_step<1, DROP>(a, I, Qu, Wv, sl, j, T, rec_pending, fv, nrec, n_items, qf, sacc, pb, st, Kh, Vh, vis);
        // the last tile (V_{T-1} sits in slot u2 now): group 1 still owes its
        // softmax; then O += V_{T-1} P_{T-1}
        if (Wv.g == 1 && !Wv.idle) {
            float rsum;
            const float alpha = softmax_tile<DROP>(a, I, Wv, sacc, Qu.kp, (Qu.iv & 16u) != 0, s_mv + ((T - 1) & 3) * MVW,
                                             st, pb, rsum);
            if (alpha != 1.f) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) st.o[dt][e] *= alpha;
            }
            st.l_run = st.l_run * alpha + rsum;
        }
        if (!Wv.idle) pv_part(vbuf(sl.u2), pb, st, lane);
    }
    // copies past the item's last tile may still be in flight: drain them
    // here, before the output stores, so that the next item can refill the
    // ring without waiting for the stores to reach memory
    wait_vm<0>();
    handover(T);
    epilogue(a, Wv, I, st);
}

// ---- standard kernel: plan in the workspace ---------------------------
// Persistent grid.  Workgroup g starts with item g; further items come
// from the work counter: fetch value v means item gridDim.x + v.  Every
// workgroup that started an item fetches until it gets an index past the
// list, so the fetches number exactly n_items and the one returning
// n_items - 1 resets the counter for the next call.
template <bool DROP>
__global__ __launch_bounds__(NTH, 2) void fm_attn_bf16_kernel(AttnArgs a) {
    static_assert(NTH / 64 == NW && BR == 32 * NW && GW == 4, "one wave per 32 query rows, one per SIMD per group");
    __shared__ __attribute__((aligned(16))) int32_t s_rec[ITEM_WORDS];
    __shared__ int32_t s_next;

    Wave Wv;
    wave_setup(a, Wv);
    const int tid = Wv.tid, lane = Wv.lane, w = Wv.w;
    const int n_items = __builtin_amdgcn_readfirstlane(*a.n_items);
    const int G = (int)gridDim.x;
    const int last_fetch = n_items + G - 1;
    int it = blockIdx.x;
    if (it < n_items && tid < ITEM_WORDS) s_rec[tid] = a.items[(int64_t)it * ITEM_WORDS + tid];
    __syncthreads();
    // the next item's first loads, issued during this item's output (pre)
    bool pre = false;
    int pre_kb = -1;
    u32x4 nxw0 = {0, 0, 0, 0}, nxw1 = {0, 0, 0, 0};
    bf16x8 qf[8];
    while (it < n_items) {
        // the fetch value is only needed when the next record is read: no
        // arithmetic on it here, so nothing waits for the atomic's return
        int fv = 0, nrec = 0;
        if (tid == 0) fv = atomicAdd(a.sched_counter, 1);
        const Item I = item_of(a, s_rec);
        bool rec_pending = (w == 0);
        const bool pre_this = pre;
        const int pkb = pre_kb;
        const u32x4 pxw0 = nxw0, pxw1 = nxw1;
        bool handed = false;
        // An item that visited tiles read the next record in its first KV
        // step.  Once its loop is done and the ring drained: the record and
        // the next index to every wave, then the next item's Q, first extrema
        // window and first tile (K slot 0, V slot 0, which the output staging
        // leaves free) are issued before this item's output is written.
        // (the dropout kernel has no registers to spare for it)
        auto handover = [&](int T) {
            if (DROP || T == 0) return;
            handed = true;
            if (w == 0) {
                if (lane < ITEM_WORDS) s_rec[lane] = nrec;
                if (lane == 0) s_next = G + fv;
            }
            item_barrier();   // every wave is past its last ring and s_rec read
            pre = false;
            pre_kb = -1;
            if (__builtin_amdgcn_readfirstlane(s_next) < n_items) {
                const Item NI = item_of(a, s_rec);
                const int nlo = Wv.no_skip ? 0 : NI.kbb, nhi = Wv.no_skip ? NI.Tc : NI.kbe;
                if (64 * w < nhi - nlo) load_window0(NI, Wv, nlo, nhi, nxw0, nxw1);
                if (!Wv.no_skip && nlo < nhi) {
                    copy_tile_pair(a, NI, Wv, (const char*)a.k + NI.hoff * 2, (const char*)a.v + NI.hoff * 2, nlo);
                    pre_kb = nlo;
                }
                load_q_row(a, NI.r0 + 32 * w + Wv.n, Wv.hh, NI.r1, NI.hoff, qf);
                pre = true;
            }
        };
        run_item<true, DROP>(a, Wv, I, 0, rec_pending, fv, nrec, n_items, qf, pre_this ? pkb : -1, pre_this, pxw0,
                             pxw1, handover);
        int nxt = G + __builtin_amdgcn_readfirstlane(fv);
        if (w == 0) {
            nxt = __builtin_amdgcn_readfirstlane(nxt);
            if (nxt == last_fetch && lane == 0) atomicExch(a.sched_counter, 0);
        }
        if (!handed) {   // no tile visited: the record is read here
            pre = false;
            pre_kb = -1;
            if (rec_pending) {
                if (nxt < n_items && lane < ITEM_WORDS) nrec = a.items[(int64_t)nxt * ITEM_WORDS + lane];
            }
            // the ring copies were drained before the epilogue; the output
            // stores need no wait
            item_barrier();   // every wave is done with s_rec, the visit list and the LDS buffers
            if (w == 0) {
                if (lane < ITEM_WORDS) s_rec[lane] = nrec;
                if (lane == 0) s_next = nxt;
            }
            __syncthreads();
        }
        it = __builtin_amdgcn_readfirstlane(s_next);
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// ---- fused kernel: each workgroup plans its own items, then attends ------
// One launch for the whole forward of a small problem: wave 0 of every
// workgroup builds the launch-wide slot tables from cu_seqlens and resolves
// the workgroup's items (fm_own_plan.h); for each item the workgroup loads
// Q, copies the K/V tile its chunk most likely starts with (the chunk's
// start when every block of the row is visited) and, while those loads are
// in flight, derives the row's visit list from the mask vectors; then it
// runs its chunk.  No workgroup waits for another; split rows are combined
// by the merge launch that follows.
}  // namespace fm
#include "fm_own_plan.h"
namespace fm {
__shared__ OwnTables s_own;

__global__ __launch_bounds__(NTH, 2) void fm_fused_bf16_kernel(AttnArgs a) {
    static_assert(NW == 8 && NTH == 512, "the planner maps eight waves to the bytes of a 64-block window");
    Wave Wv;
    wave_setup(a, Wv);
    const int status = own_setup<BR, BC>(a, s_own);
    if (blockIdx.x == 0 && Wv.tid == 0) {
        // header: status, no plan in the workspace (no items and no split
        // rows listed, so a call with a ready plan on this workspace runs
        // nothing), the merge table of R q tiles x H heads
        a.w_hdr[HDR_STATUS] = status;
        a.w_hdr[HDR_NKB] = 0;
        a.w_hdr[HDR_NITEMS] = 0;
        a.w_hdr[HDR_SCHED] = 0;
        a.w_hdr[HDR_NSLOTS] = 0;
        a.w_hdr[HDR_NMERGE] = 0;
        a.w_hdr[HDR_NFUSED] = status ? 0 : s_own.misc[1] * a.H;
    }
    if (status != 0) return;
    const int n_my = __builtin_amdgcn_readfirstlane(s_own.misc[3]);
    const int n_items = __builtin_amdgcn_readfirstlane(s_own.misc[2]) * a.H;
    bool rec_pending = false;
    int nrec = 0;
    for (int k = 0; k < n_my; ++k) {
        auto u = [](int x) { return __builtin_amdgcn_readfirstlane(x); };   // wave-uniform copies
        const MyItem m = {u(s_own.my[k].b), u(s_own.my[k].qt), u(s_own.my[k].r), u(s_own.my[k].s),
                          u(s_own.my[k].h), u(s_own.my[k].U)};
        const int s_b = u(s_own.cu[m.b]), e_b = u(s_own.cu[m.b + 1]);
        const int r0 = s_b + m.qt * BR;
        Wv.qrow = r0 + 32 * Wv.w + Wv.n;
        bf16x8 qf[8];
        load_q(a, Wv, min(r0 + BR, e_b), (int64_t)m.h * HD, qf);   // in flight during the planning
        const int pre_kb = guess_first_block(m.U, m.s, a.S);
        if (pre_kb >= 0) {
            Item G;
            G.s_b = s_b; G.e_b = e_b;
            copy_tile_pair(a, G, Wv, (const char*)a.k + (int64_t)m.h * HD * 2, (const char*)a.v + (int64_t)m.h * HD * 2,
                           pre_kb);
        }
        Item I;
        int vis_off = 0;
        if (!own_item<BR, BC, HD>(a, s_own, m, I, vis_off, s_vis, s_wvis, s_wiv)) {
            __builtin_amdgcn_s_waitcnt(0);   // the guessed copy lands before the ring is reused
            __syncthreads();                 // every wave is done with the window masks
            continue;
        }
        run_item<false, false>(a, Wv, I, vis_off, rec_pending, 0, nrec, n_items, qf, pre_kb, false,
                               u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}, [](int) {});
        item_barrier();   // the ring, the visit list and the masks are free for the next item
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// ---- merge of split rows ----------------------------------------------
// Combines the partials of every split row in split order (deterministic,
// one pass with the running max): with m = max so far and O_s = the stored
// fp16 row times l_s 2^e_s,
//   m' = max(m, m_s),  l = l 2^(m - m') + l_s 2^(m_s - m'),
//   O = O 2^(m - m') + O_s 2^(m_s - m'),
// then out = O / l and lse = (m + log2 l) ln 2.  Work comes from the list of
// split rows the planner wrote (one entry per split row and head).  Task =
// (entry, wave slot w of the partial layout, channel group pair gp); thread
// = (lane of that wave, dt): every read instruction of a wave is 1 KB
// contiguous, and a thread issues the reads of up to MSPL splits before
// using any of them.
constexpr int MNTH = 256, MSPL = 16;

__global__ __launch_bounds__(MNTH) void fm_merge_bf16_kernel(AttnArgs a) {
    const int lane = threadIdx.x & 63, dt = threadIdx.x >> 6, n = lane & 31, hh = lane >> 5;
    // every entry below merge_cap lies inside the list, so a task's entry is
    // read together with the entry count (one memory round trip, not two)
    // and entries at or past the count are skipped
    const int n_merge = *a.n_merge;
    const int64_t n_tasks = a.merge_cap * NW * 2;
    for (int64_t task = blockIdx.x; task < n_tasks; task += gridDim.x) {
        const int64_t k = task / (NW * 2);
        const int w = (int)((task / 2) % NW), gp = (int)(task % 2);
        const int4 e0 = *(const int4*)(a.merge_list + k * MERGE_WORDS);
        const int nsp = a.merge_list[k * MERGE_WORDS + 4];
        if (k >= n_merge) break;                 // tasks only grow along the loop
        const int slot0 = e0.x, h = e0.y, lr = 32 * w + n;
        const int64_t qrow = (int64_t)e0.z + lr;
        if (qrow >= e0.w || nsp <= 1) continue;   // rows of one chunk wrote out themselves
        const uint32_t* p0 = (const uint32_t*)a.partial + ((int64_t)slot0 * a.H + h) * PART;
        const int64_t step = (int64_t)a.H * PART;
        const int oi = part_index(w, dt, gp, lane);
        float m = -INFINITY, l = 0.f;
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.f;
        for (int s0 = 0; s0 < nsp; s0 += MSPL) {
            float mv[MSPL], lv[MSPL];
            int ev[MSPL];
            u32x4 ov[MSPL];
#pragma unroll
            for (int u = 0; u < MSPL; ++u)
                if (s0 + u < nsp) {
                    const uint32_t* ps = p0 + (s0 + u) * step;
                    mv[u] = __uint_as_float(ps[BR * HD / 2 + lr]);
                    lv[u] = __uint_as_float(ps[BR * HD / 2 + BR + lr]);
                    ev[u] = (int)ps[BR * HD / 2 + 2 * BR + lr];
                    ov[u] = *(const u32x4*)(ps + oi);
                }
#pragma unroll
            for (int u = 0; u < MSPL; ++u)
                if (s0 + u < nsp) {
                    const float mn = fmaxf(m, mv[u]);
                    const float mu = mn == -INFINITY ? 0.f : mn;
                    const float ca = __builtin_amdgcn_exp2f(m - mu), cb = __builtin_amdgcn_exp2f(mv[u] - mu);
                    l = __builtin_fmaf(l, ca, lv[u] * cb);
                    const float f = __builtin_amdgcn_ldexpf(lv[u] * cb, ev[u]);
                    const uint32_t wd[4] = {ov[u].x, ov[u].y, ov[u].z, ov[u].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd[j] & 0xffff));
                        const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd[j] >> 16));
                        acc[2 * j] = __builtin_fmaf(acc[2 * j], ca, lo * f);
                        acc[2 * j + 1] = __builtin_fmaf(acc[2 * j + 1], ca, hi * f);
                    }
                    m = mn;
                }
        }
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* op = (uint16_t*)a.out + qrow * ((int64_t)a.H * HD) + (int64_t)h * HD + 32 * dt + 16 * gp + 4 * hh;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
            u32x2 wv;
            wv.x = bf16_bits(acc[4 * g2] * inv) | (bf16_bits(acc[4 * g2 + 1] * inv) << 16);
            wv.y = bf16_bits(acc[4 * g2 + 2] * inv) | (bf16_bits(acc[4 * g2 + 3] * inv) << 16);
            *(u32x2*)(op + 8 * g2) = wv;
        }
        if (dt == 0 && gp == 0 && hh == 0)
            a.lse[(int64_t)h * a.N + qrow] = l > 0.f ? (m + __log2f(l)) * LN2 : -INFINITY;
    }
}

namespace {
int occupancy(const void* fn) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, fn, NTH, 0) != hipSuccess || o < 1) o = 1;
    return o;
}

hipError_t launch_merge(const AttnArgs& a, int n_cu, hipStream_t s) {
    if (a.S <= 0) return hipSuccess;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(a.merge_cap * NW * 2, (int64_t)n_cu * 8));
    hipLaunchKernelGGL(fm_merge_bf16_kernel, dim3((unsigned)grid), dim3(MNTH), 0, s, a);
    return hipGetLastError();
}
}  // namespace

int fused_grid(int n_cu) {
    static const int occ = occupancy((const void*)fm_fused_bf16_kernel);
    return std::max(1, n_cu * occ);
}

hipError_t launch_attn_bf16(const AttnArgs& a, int n_cu, hipStream_t s) {
    static const int occ = occupancy((const void*)fm_attn_bf16_kernel<false>);
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(a.items_cap, (int64_t)n_cu * occ));
    if (a.drop_t > 0) hipLaunchKernelGGL(fm_attn_bf16_kernel<true>, dim3((unsigned)grid), dim3(NTH), 0, s, a);
    else hipLaunchKernelGGL(fm_attn_bf16_kernel<false>, dim3((unsigned)grid), dim3(NTH), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_merge(a, n_cu, s);
}

hipError_t launch_fused_bf16(const AttnArgs& a, int n_cu, hipStream_t s) {
    hipLaunchKernelGGL(fm_fused_bf16_kernel, dim3((unsigned)fused_grid(n_cu)), dim3(NTH), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_merge(a, n_cu, s);
}

}  // namespace fm
