// Backward of the FlashMask attention: dq, dk, dv from q, k, v, out, the
// output gradient dout and softmax_lse; bf16 in and out, fp32 accumulation,
// head_dim 128, on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Method (PaddleNLP FlashMask article, m.nxbn.cn/news/70198): §3.4 names the
// backward op (inputs q, k, v, the row intervals, out, softmax_lse and the
// output gradient; outputs the gradients of q, k and v); the block extrema
// and tile classes of §3.1/§3.2 decide which tiles are skipped, as in the
// forward; §4.2: the result does not depend on the order of floating-point
// accumulation (no atomics on dq).  The gradients are those of the
// forward's softmax attention, with P = exp(scale S - lse) on the allowed
// pairs:
//   dV = P^T dO,  dP = dO V^T,  Delta_i = <dO_i, O_i>,
//   dS = P o (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Layout and schedule (this file's own):
//   * delta kernel: Delta[h, i] = <dO_i, O_i> in fp32, 16 lanes per row.
//   * dK/dV kernel: one workgroup of 8 waves per (128-key tile, head);
//     wave 4g + t owns keys 32t..32t+31 (half of its key's K row in
//     registers, the rest of K and V in LDS) and query rows 32g..32g+31 of
//     each staged tile.  It walks the sequence's 64-row q tiles that are
//     not FULL against its key tile, stages Q, dO, lse and Delta of each in
//     an LDS ring with asynchronous copies, computes S = Q K^T and
//     dP = dO V^T with one key per lane (so the key's mask intervals are
//     lane constants), and accumulates dV^T = dO^T P and dK^T = Q^T dS
//     with the LDS transpose read; its two wave groups work in opposite
//     phase (in phase with dropout), and the two row halves are summed in
//     LDS.
//   * dQ kernel: one workgroup of 8 waves per (256-query tile, head); wave
//     w owns queries 32w..32w+31 with their Q and dO fragments, lse and
//     Delta in registers.  It walks the visited 64-key blocks, stages K and
//     V in an LDS ring with asynchronous copies, computes S^T = K Q^T and
//     dP^T = V dO^T with one query per lane (as the forward does), and
//     accumulates dQ^T = K^T dS^T; its two wave groups work in opposite
//     phase on 32-key half blocks, so that one wave of a SIMD issues
//     products while the other computes dS.
//   * small problems (fewer workgroups than compute units) cut each key
//     tile's q tiles and each query tile's key blocks into chunks that run
//     as separate workgroups and write fp32 partials; two reduce launches
//     sum them in chunk order.
//   * every output element is written by exactly one workgroup, and chunk
//     sums run in a fixed order: the same inputs give the same bits.

#include "fm_common.hpp"
#include "fm_internal.h"
#include "fm_api.h"

namespace fm {
namespace bwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int HD = 128;          // head_dim
constexpr int BLK = 64;          // key block of the extrema; q rows per dK/dV step; keys per dQ step
constexpr int NTH = 256;         // 4 waves
constexpr int ROW_R = 272;       // LDS row stride of tiles read by rows only
constexpr float LOG2E = 1.4426950408889634074f;

__device__ __attribute__((always_inline)) inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __attribute__((always_inline)) inline uint32_t bf16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __attribute__((always_inline)) inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A-operand fragments of the transpose of a row-major LDS tile (rows are
// the MFMA's k index, channels its m index) come from the gfx950 LDS
// transpose read: channel block dt (32 channels), k group kg (16 rows);
// within a group, lane half hh takes rows 4hh + {0..3, 8..11}, the order in
// which an MFMA result holds its rows (register e of a 32x32 result is row
// 8(e>>2) + 4hh + (e&3)), so the B operand can be packed straight from such
// a result.
// Tiles read both by rows (A operands of S, dP) and transposed (A operands
// of dV, dK, dQ) are stored with 256-byte rows, chunk c (16 bytes) of row r
// at chunk c ^ swz(r): 16 consecutive rows of one chunk, and the 4 rows x 4
// chunks of a transposed read, then fall in 16 distinct 4-bank groups
// (with padded rows only one of the two patterns can be conflict-free).
constexpr int ROW_S = 256;
__device__ __attribute__((always_inline)) inline int swz(int r) {
    r &= 15;
    return ((r & 3) << 2) | (r >> 2);
}
__device__ __attribute__((always_inline)) inline int soff(int r, int c) { return r * ROW_S + 16 * (c ^ swz(r)); }
// The transposed fragment (rows 16kg + 4hh + (gi>>2), +8; chunks
// 4dt + 2(grp&1) + ((gi&3)>>1); 8-byte half gi&1) of a swizzled tile.
__device__ __attribute__((always_inline)) inline bf16x8 tr_frag_s(const char* tile, int kg, int dt, int lane) {
    const int hh = lane >> 5, grp = lane >> 4, gi = lane & 15;
    const int r = 16 * kg + 4 * hh + (gi >> 2), c = 4 * dt + 2 * (grp & 1) + ((gi & 3) >> 1);
    const char* p0 = tile + soff(r, c) + 8 * (gi & 1);
    const char* p1 = tile + soff(r + 8, c) + 8 * (gi & 1);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(void*)p0);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(void*)p1);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Rows [s, e) of 32 as a bit mask (s, e relative, clamped; empty if e <= s).
__device__ __attribute__((always_inline)) inline uint32_t row_bits(int s, int e) {
    s = min(max(s, 0), 32);
    e = min(max(e, s), 32);
    const int w = e - s;
    return w >= 32 ? 0xffffffffu : ((1u << w) - 1u) << (s & 31);
}
// Interval endpoint x (any int32 row index) relative to the first row q0 >= 0
// of 32, clamped below at 0 first so that the subtraction cannot wrap.
__device__ __attribute__((always_inline)) inline int rel_row(int x, int q0) { return max(x, q0) - q0; }
// x, or y where the lane's bit of {lo: lanes 0-31, hi: lanes 32-63} is set.
__device__ __attribute__((always_inline)) inline float select_lanes(float x, float y, uint32_t lo, uint32_t hi) {
    const uint64_t m = ((uint64_t)hi << 32) | lo;
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "s"(m));
    return r;
}

// Sequence of global key block x (kb_off[0] <= x < kb_off[B]).
__device__ inline int seq_of_block(const int32_t* kb_off, int B, int x) {
    int lo = 0, hi = B;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (kb_off[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// The span of a workgroup: NB consecutive 64-row (or 64-key) blocks of one
// sequence starting at global block x (fewer at the sequence end).  Only
// workgroups whose local block index is a multiple of NB have a span.
struct Span {
    bool ok;
    int b, s_b, e_b, lo, hi, x;
    bool two;   // block x + 1 lies in the sequence
};
template <int NB>
__device__ inline Span span_of(const BwdArgs& a, int x) {
    Span sp;
    sp.ok = false;
    if (__builtin_amdgcn_readfirstlane(*a.status) != 0) return sp;
    const int n_kb = __builtin_amdgcn_readfirstlane(*a.n_kb);
    if (x >= n_kb) return sp;
    sp.b = seq_of_block(a.kb_off, a.B, x);
    const int kb0 = a.kb_off[sp.b], kb1 = a.kb_off[sp.b + 1];
    if ((x - kb0) % NB) return sp;
    sp.x = x;
    sp.two = x + 1 < kb1;
    sp.s_b = a.cu[sp.b];
    sp.e_b = a.cu[sp.b + 1];
    sp.lo = sp.s_b + (x - kb0) * BLK;
    sp.hi = min(sp.lo + NB * BLK, sp.e_b);
    sp.ok = true;
    return sp;
}

// Asynchronous copies of 64-row tiles (K and V in the dQ kernel, Q and dO in
// the dK/dV kernel) from global memory straight into swizzled LDS rows
// (buffer_load ... lds: 64 lanes x 16 bytes into 1 KB of LDS at M0 + 16
// lane; rows past the sequence read as zeros through the buffer's byte
// count).  Each lane's source is the chunk that the swizzled layout puts
// at its LDS position, so copy i of a tile fills rows 4i..4i+3 (16 copies
// per tensor, 2 per wave).  The copies are issued with inline assembly and
// waited for explicitly.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __attribute__((always_inline)) inline void dma_b16(void* dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
                 "{m0}"((uint32_t)(uintptr_t)(lds_char*)dst)
                 : "memory");
}
// Source offset (bytes from the block's first row) of this lane in copy i.
__device__ __attribute__((always_inline)) inline uint32_t stage_voff(int i, int lane, uint32_t rsb) {
    const int r = 4 * i + (lane >> 4);
    return (uint32_t)r * rsb + 16u * (uint32_t)((lane & 15) ^ swz(r));
}
// ---- Delta ---------------------------------------------------------------
// Delta[h, i] = sum_d dO[i, h, d] O[i, h, d]: 16 lanes per (row, head), 8
// channels each, summed over the 16 lanes with DPP (quad swaps, then the
// half-row and row mirrors leave the sum in every lane of the row).
__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <int CTRL>
__device__ inline float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

__global__ __launch_bounds__(NTH) void fm_bwd_delta_kernel(BwdArgs a) {
    const int64_t p = ((int64_t)blockIdx.x * NTH + threadIdx.x) >> 4;   // (row, head) = row * H + head
    const int sub = threadIdx.x & 15;
    const int64_t NH = a.N * a.H;
    float acc = 0.f;
    if (p < NH) {
        const u32x4 o = *(const u32x4*)((const char*)a.out + p * (2 * HD) + 16 * sub);
        const u32x4 g = *(const u32x4*)((const char*)a.dout + p * (2 * HD) + 16 * sub);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += bf_lo(o[i]) * bf_lo(g[i]) + bf_hi(o[i]) * bf_hi(g[i]);
    }
    acc = dpp_add<0xB1>(acc);    // quad_perm [1,0,3,2]
    acc = dpp_add<0x4E>(acc);    // quad_perm [2,3,0,1]
    acc = dpp_add<0x141>(acc);   // row_half_mirror
    acc = dpp_add<0x140>(acc);   // row_mirror
    if (p < NH && sub == 0) {
        const int64_t i = p / a.H;
        const int h = (int)(p - i * a.H);
        a.delta[(int64_t)h * a.N + i] = acc;
    }
}

// ---- dK / dV ---------------------------------------------------------------
// 8 waves: wave w = 4g + t owns keys 32t..32t+31 of the 128-key span (its
// key's K fragments in registers, the span's V rows in LDS) and query rows
// 32g..32g+31 of every staged 64-row q tile (two waves per SIMD).  The two
// groups work in opposite phase, as in the dQ kernel: in the step of q tile
// i, group 0 issues dV^T += dO_{i-1}^T P_{i-1}, dK^T += Q_{i-1}^T dS_{i-1}
// and S_i, dP_i, then turns S_i, dP_i into P_i, dS_i; group 1 first turns
// the S, dP it computed in the previous step into P, dS, then issues the
// same products.  Q, dO, lse and Delta of a tile sit in a 3-slot LDS ring
// filled by asynchronous copies (tile i + 1 into the slot tile i - 2 has
// left), one barrier per tile.  The groups' dK^T and dV^T are summed
// through LDS at the end.
constexpr int NTK = 512;
constexpr int KV_COMB = 4 * 64 * 16 * 16;   // bytes: one accumulator set of a group (16 x 16 B per lane)
constexpr int OFF_G = BLK * ROW_S, OFF_L2 = 2 * BLK * ROW_S, OFF_DL = OFF_L2 + 4 * BLK;
constexpr int QSLOT = OFF_DL + 4 * BLK;      // one ring slot: Q, dO (swizzled rows), lse (log2 units), Delta
constexpr int DKV_LDS = KV_COMB > 3 * QSLOT ? KV_COMB : 3 * QSLOT;
// the ring during the loop, the group sums after it
__shared__ __attribute__((aligned(16))) char s_dkv[DKV_LDS];
// the span's V rows (128 keys) and the upper half (channels 64..127) of its
// K rows, staged once (the lower half of a lane's K row stays in
// registers), and the mask intervals of each key
constexpr int KH_ROW = 144;   // bytes per row of the K half: 8 chunks + 1 of padding
__shared__ __attribute__((aligned(16))) char s_vt[2 * BLK * ROW_R];
__shared__ __attribute__((aligned(16))) char s_kh[2 * BLK * KH_ROW];
__shared__ __attribute__((aligned(16))) Vec4 s_kmv[2 * BLK];

// Copies of q tile rows [r0, r1) of Q and dO into ring slot `slot`.
__device__ __attribute__((always_inline)) inline void stage_qtile(const BwdArgs& a, int h, int r0, int r1, int slot,
                                                                  int w, int lane) {
    const uint32_t rsb = (uint32_t)a.H * 2 * HD;
    const uint32_t vo[2] = {stage_voff(2 * w, lane, rsb), stage_voff(2 * w + 1, lane, rsb)};
    const int64_t base = (int64_t)r0 * rsb + (int64_t)h * 2 * HD;
    const int nbytes = (r1 - r0 - 1) * (int)rsb + 2 * HD;   // through the tile's last row
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.q + base), (short)0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rg =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.dout + base), (short)0, nbytes, 0x00020000);
    char* sl = s_dkv + slot * QSLOT;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        dma_b16(sl + 1024 * (2 * w + x), rq, vo[x]);
        dma_b16(sl + OFF_G + 1024 * (2 * w + x), rg, vo[x]);
    }
}

// S = Q K^T and dP = dO V^T for rows 32g..32g+31 of a staged tile: register
// e is row 32g + 8(e>>2) + 4hh + (e&3), column = this lane's key.
// K fragments of k-steps 0..3 come from registers, 4..7 from the span's K
// half in LDS (kh_l: this lane's key row there).
__device__ __attribute__((always_inline)) inline void dkdv_sdp(const char* sl, const bf16x8 (&kf)[4], const char* kh_l,
                                                               const char* vb_l, f32x16& sc, f32x16& dp, int g, int n,
                                                               int hh) {
#pragma unroll
    for (int e = 0; e < 16; ++e) { sc[e] = 0.f; dp[e] = 0.f; }
    const int qrow = 32 * g + n;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int o = soff(qrow, 2 * s + hh);
        const bf16x8 kb = s < 4 ? kf[s & 3] : as_bf16x8(*(const u32x4*)(kh_l + 32 * (s - 4)));
        sc = mfma(as_bf16x8(*(const u32x4*)(sl + o)), kb, sc);
        dp = mfma(as_bf16x8(*(const u32x4*)(sl + OFF_G + o)), as_bf16x8(*(const u32x4*)(vb_l + 32 * s)), dp);
    }
}
// dV^T += dO^T P and dK^T += Q^T dS over the 16-row group 2g + c2.
__device__ __attribute__((always_inline)) inline void dkdv_acc_half(const char* sl, const bf16x8& pb, const bf16x8& db,
                                                                    f32x16 (&dv)[4], f32x16 (&dk)[4], int g, int c2,
                                                                    int lane) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        dv[dt] = mfma(tr_frag_s(sl + OFF_G, 2 * g + c2, dt, lane), pb, dv[dt]);
        dk[dt] = mfma(tr_frag_s(sl, 2 * g + c2, dt, lane), db, dk[dt]);
    }
}
__device__ __attribute__((always_inline)) inline void dkdv_acc(const char* sl, const bf16x8 (&pb)[2],
                                                               const bf16x8 (&db)[2], f32x16 (&dv)[4], f32x16 (&dk)[4],
                                                               int g, int lane) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) dkdv_acc_half(sl, pb[c2], db[c2], dv, dk, g, c2, lane);
}

// Dropout bytes of a wave's 32 rows x 32 keys (dK/dV): lane L writes the
// four words of (row L & 31, 16-key block L >> 5), u32 index
// ((row * 2 + block) * 4 + word).
__shared__ __attribute__((aligned(16))) uint32_t s_drop[8][256];

// This wave's dropout bytes for the tile at r0 (one Philox4x32-10 block per
// lane), written right after the wave has issued the tile's S and dP (its
// vector work then runs beside the products) and read by dkdv_pds.
__device__ __attribute__((always_inline)) inline void dkdv_dropw(const BwdArgs& a, int r0, int c0, int s_b, int h,
                                                                 int g, int t, int w, int lane) {
    uint32_t w0 = (uint32_t)(r0 + 32 * g + (lane & 31));
    uint32_t w1 = (uint32_t)(((c0 - s_b) >> 4) + 2 * t + (lane >> 5)), w2 = (uint32_t)h, w3 = a.offset;
    philox4x32_10(w0, w1, w2, w3, a.seed_lo, a.seed_hi);
    *(u32x4*)&s_drop[w][((lane & 31) * 2 + (lane >> 5)) * 4] = u32x4{w0, w1, w2, w3};
}

// P = exp2(S scale log2e - lse2), masked pairs 0; dS = P (dP - Delta); with
// dropout Z = keep * 256 / (256 - t): P Z for dV, dS = P (dP Z - Delta).
// Tile rows from r0, staged lse2 and Delta in slot sl; the B operands of
// dkdv_acc_half for the 16-row group 2g + c2.
template <bool DROP>
__device__ __attribute__((always_inline)) inline void dkdv_pds_half(const BwdArgs& a, const f32x16& sc,
                                                                    const f32x16& dp, bf16x8& pb, bf16x8& db,
                                                                    const char* sl, int r0, bool part, int kj,
                                                                    int g, int t, int w, int lane, int c2) {
    const int n = lane & 31, hh = lane >> 5;
    const float* s_l2 = (const float*)(sl + OFF_L2);
    const float* s_dl = (const float*)(sl + OFF_DL);
    const float sl2 = a.scale_log2;
    // the 8 probabilities of the half (register e = 8 c2 + k: row
    // 32g + 8(2c2 + (k>>2)) + 4hh + (k&3)), then the mask of a partial tile
    // in one pass (no branch per element), then P, dS
    float p[8], dl[8];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * c2 + jj;
        const float4 l4 = *(const float4*)(s_l2 + 32 * g + 8 * j + 4 * hh);
        const float4 d4 = *(const float4*)(s_dl + 32 * g + 8 * j + 4 * hh);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            p[4 * jj + c] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * j + c], sl2, -lv[c]));
            dl[4 * jj + c] = dv4[c];
        }
    }
    if (part) {
        const Vec4 mv = s_kmv[32 * t + n];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int row = r0 + 32 * g + 8 * (2 * c2 + (k >> 2)) + 4 * hh + (k & 3);
            const bool m = (a.causal && kj > row) || (mv.lts <= row && row < mv.lte) ||
                           (mv.uts <= row && row < mv.ute);
            p[k] = m ? 0.f : p[k];
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int e = 8 * c2 + k;
        float pz = p[k], dpz = dp[e];
        if constexpr (DROP) {
            const int rw = 8 * (2 * c2 + (k >> 2)) + 4 * hh + (k & 3);   // row within the wave's 32
            const uint32_t word = s_drop[w][(rw * 2 + (n >> 4)) * 4 + ((n & 15) >> 2)];
            const bool keep = ((word >> (8 * (n & 3))) & 0xffu) >= (uint32_t)a.drop_t;
            pz = keep ? p[k] * a.drop_ks : 0.f;
            dpz = keep ? dpz * a.drop_ks : 0.f;
        }
        pb[k] = (__bf16)pz;
        db[k] = (__bf16)(p[k] * (dpz - dl[k]));
    }
}
template <bool DROP>
__device__ __attribute__((always_inline)) inline void dkdv_pds(const BwdArgs& a, const f32x16& sc, const f32x16& dp,
                                                               bf16x8 (&pb)[2], bf16x8 (&db)[2], const char* sl,
                                                               int r0, bool part, int kj, int g, int t, int w,
                                                               int lane) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) dkdv_pds_half<DROP>(a, sc, dp, pb[c2], db[c2], sl, r0, part, kj, g, t, w, lane, c2);
}

// Group sums: group `from` writes its 4 accumulators, the other group adds
// them to its own (float addition commutes: the result does not depend on
// which group adds).  Lane L of wave slot t, accumulator dt, quad q at
// float4 ((4 dt + q) * 256 + 64 t + L).
__device__ __attribute__((always_inline)) inline void group_sum(f32x16 (&acc)[4], int g, int from, int t, int lane) {
    float4* buf = (float4*)s_dkv;
    __syncthreads();
    if (g == from) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                buf[(4 * dt + q) * 256 + 64 * t + lane] =
                    float4{acc[dt][4 * q], acc[dt][4 * q + 1], acc[dt][4 * q + 2], acc[dt][4 * q + 3]};
    }
    __syncthreads();
    if (g != from) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 o = buf[(4 * dt + q) * 256 + 64 * t + lane];
                acc[dt][4 * q] += o.x; acc[dt][4 * q + 1] += o.y;
                acc[dt][4 * q + 2] += o.z; acc[dt][4 * q + 3] += o.w;
            }
    }
}

// Chunk partials: 8 waves x 64 lanes x 4 accumulators of 16 floats
// (128 KB), float4 ((16 w + 4 dt + q) * 64 + lane): every store and load
// instruction of a wave covers 1 KB contiguously.
constexpr int PART_FLOATS = 8 * 64 * 64;
__device__ __attribute__((always_inline)) inline void store_acc(float* base, const f32x16 (&acc)[4], int w, int lane) {
    float4* p = (float4*)base;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            p[(16 * w + 4 * dt + q) * 64 + lane] = float4{acc[dt][4 * q], acc[dt][4 * q + 1], acc[dt][4 * q + 2],
                                                         acc[dt][4 * q + 3]};
}
// The reduce launches: RZ workgroups per tile, workgroup z summing the
// accumulator quads dt = z of every lane (4 float4 per thread per chunk).
// Per batch of CB chunks the flags are read first, then every written
// chunk's loads are issued before the sums, which run in chunk order.
constexpr int RZ = 4, CB = 8;   // chunks loaded per batch
__device__ __attribute__((always_inline)) inline void sum_chunks(const BwdArgs& a, const float* base,
                                                                 const int32_t* flags, int64_t slot0, int dt,
                                                                 float4 (&acc)[4], int w, int lane) {
    for (int c0 = 0; c0 < a.nc; c0 += CB) {
        bool wr[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) wr[c] = c0 + c < a.nc && flags[slot0 + c0 + c] == (int32_t)a.call_id;
        float4 v[CB][4];
#pragma unroll
        for (int c = 0; c < CB; ++c)
            if (wr[c]) {
                const float4* p = (const float4*)(base + (slot0 + c0 + c) * PART_FLOATS);
#pragma unroll
                for (int q = 0; q < 4; ++q) v[c][q] = p[(16 * w + 4 * dt + q) * 64 + lane];
            }
#pragma unroll
        for (int c = 0; c < CB; ++c)
            if (wr[c]) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[q].x += v[c][q].x; acc[q].y += v[c][q].y; acc[q].z += v[c][q].z; acc[q].w += v[c][q].w;
                }
            }
    }
}
// bf16 channels 32dt + 8q + 4hh + 0..3 (q = 0..3) of a row, times sc.
__device__ __attribute__((always_inline)) inline void store_quads_bf16(uint16_t* op, const float4 (&x)[4], float sc,
                                                                       int dt, int hh) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        u32x2 v2;
        v2.x = bf16_bits(x[q].x * sc) | (bf16_bits(x[q].y * sc) << 16);
        v2.y = bf16_bits(x[q].z * sc) | (bf16_bits(x[q].w * sc) << 16);
        *(u32x2*)(op + 32 * dt + 8 * q + 4 * hh) = v2;
    }
}
// bf16 row of 128 channels from a lane's 4 accumulators (channels
// 32dt + 8q + 4hh + 0..3), times sc.
__device__ __attribute__((always_inline)) inline void store_row_bf16(uint16_t* op, const f32x16 (&x)[4], float sc,
                                                                     int hh) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x2 v2;
            v2.x = bf16_bits(x[dt][4 * q] * sc) | (bf16_bits(x[dt][4 * q + 1] * sc) << 16);
            v2.y = bf16_bits(x[dt][4 * q + 2] * sc) | (bf16_bits(x[dt][4 * q + 3] * sc) << 16);
            *(u32x2*)(op + 32 * dt + 8 * q + 4 * hh) = v2;
        }
}

template <bool DROP>
__global__ __launch_bounds__(NTK, 1) void fm_bwd_dkdv_kernel(BwdArgs a) {
    const int h = blockIdx.y;
    const Span sp = span_of<2>(a, blockIdx.x);
    if (!sp.ok) return;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = w >> 2, t = w & 3;     // query-row half, key slot
    const int n = lane & 31, hh = lane >> 5;
    const int c0 = sp.lo, c1 = sp.hi;

    // extrema of the key tile: its one or two blocks combined
    int xe[8];
    {
        const int4 e0 = *(const int4*)(a.extrema + (int64_t)sp.x * 8);
        const int4 e1 = *(const int4*)(a.extrema + (int64_t)sp.x * 8 + 4);
        xe[0] = e0.x; xe[1] = e0.y; xe[2] = e0.z; xe[3] = e0.w;
        xe[4] = e1.x; xe[5] = e1.y; xe[6] = e1.z; xe[7] = e1.w;
        if (sp.two) {
            const int4 f0 = *(const int4*)(a.extrema + (int64_t)(sp.x + 1) * 8);
            const int4 f1 = *(const int4*)(a.extrema + (int64_t)(sp.x + 1) * 8 + 4);
            const int y[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) xe[i] = (i & 1) ? max(xe[i], y[i]) : min(xe[i], y[i]);
        }
    }

    // the span's V rows and the upper half of its K rows into LDS (rows
    // past the sequence: zeros), the keys' mask intervals; this lane's key
    // and the lower half of its K row (B operands: column n, channels
    // 16s + 8hh, s < 4)
#pragma unroll
    for (int u = 0; u < 2 * BLK * 16 / NTK; ++u) {
        const int c = tid + NTK * u, row = c >> 4, ch = c & 15;
        u32x4 vv = u32x4{0, 0, 0, 0}, kv = u32x4{0, 0, 0, 0};
        const int64_t off = ((int64_t)(c0 + row) * a.H + h) * 2 * HD + 16 * ch;
        if (c0 + row < c1) {
            vv = *(const u32x4*)((const char*)a.v + off);
            if (ch >= 8) kv = *(const u32x4*)((const char*)a.k + off);
        }
        *(u32x4*)(s_vt + row * ROW_R + 16 * ch) = vv;
        if (ch >= 8) *(u32x4*)(s_kh + row * KH_ROW + 16 * (ch - 8)) = kv;
    }
    if (tid < 2 * BLK) s_kmv[tid] = c0 + tid < c1 ? fill_column(a.sv, a.n_vec, a.causal, a.N, c0 + tid) : Vec4{0, 0, 0, 0};
    const int kj = c0 + 32 * t + n;
    const bool kvalid = kj < c1;
    bf16x8 kf[4];
    {
        const char* kp = (const char*)a.k + ((int64_t)kj * a.H + h) * 2 * HD + 16 * hh;
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[s] = as_bf16x8(kvalid ? *(const u32x4*)(kp + 32 * s) : u32x4{0, 0, 0, 0});
    }
    const char* vb_l = s_vt + (32 * t + n) * ROW_R + 16 * hh;
    const char* kh_l = s_kh + (32 * t + n) * KH_ROW + 16 * hh;

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) { dk[dt][e] = 0.f; dv[dt][e] = 0.f; }

    // q tiles of 64 rows from the sequence start; causal rows before c0 see
    // none of the tile's keys; with chunks, this workgroup's share only
    const int Tq_all = ceil_div(sp.e_b - sp.s_b, BLK);
    const int ch = blockIdx.z;
    const int Tq = a.nc > 1 ? min(Tq_all, (ch + 1) * a.qc) : Tq_all;
    const int i_first = max(a.causal ? (c0 - sp.s_b) / BLK : 0, a.nc > 1 ? ch * a.qc : 0);
    // next q tile at or after `from` whose class is not FULL (Tq if none);
    // the classes of a window of 64 q tiles from `wbase` (lane = tile) are
    // kept as ballots, so a step only scans bits
    int wbase = -1;
    uint64_t wv = 0, wp = 0;
    auto next_visit = [&](int from, bool& part) __attribute__((always_inline)) -> int {
        while (from < Tq) {
            if (wbase < 0 || from >= wbase + 64) {
                wbase = from;
                const int i = from + lane;
                bool v = false, p = false;
                if (i < Tq) {
                    const int r0 = sp.s_b + i * BLK, r1 = min(r0 + BLK, sp.e_b);
                    const TileInfo ti = classify_tile(r0, r1, c0, c1, xe, a.causal);
                    v = ti.cls != CLS_FULL;
                    p = ti.cls == CLS_PARTIAL;
                }
                wv = __ballot(v);
                wp = __ballot(p);
            }
            const int off = from - wbase;   // 0..63
            const uint64_t m = wv >> off;
            if (m) {
                const int bit = __builtin_ctzll(m);
                part = ((wp >> (off + bit)) & 1ull) != 0;
                return from + bit;
            }
            from = wbase + 64;
        }
        return Tq;
    };
    auto rstart = [&](int i) __attribute__((always_inline)) { return sp.s_b + i * BLK; };
    auto rend = [&](int i) __attribute__((always_inline)) { return min(sp.s_b + (i + 1) * BLK, sp.e_b); };

    // The pipeline: q tile i in slot i mod 3.  In step i every wave issues
    // its copies of tile i + 1 into the slot tile i - 2 has left, and wave 0
    // loads that tile's lse and Delta into registers; they are waited for
    // (and wave 0 stages lse in log2 units, +inf where no key is allowed or
    // past the sequence, so that P = 0 there) before the barrier that
    // publishes tile i + 1.
    float lsr = -INFINITY, dlr = 0.f;    // wave 0: lse, Delta of row `lane` of the tile in flight
    auto load_ld = [&](int i) __attribute__((always_inline)) {
        if (w == 0) {
            lsr = -INFINITY;
            dlr = 0.f;
            if (rstart(i) + lane < rend(i)) {
                lsr = a.lse[(int64_t)h * a.N + rstart(i) + lane];
                dlr = a.delta[(int64_t)h * a.N + rstart(i) + lane];
            }
        }
    };
    auto publish = [&](int slot) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0)
        asm volatile("" ::: "memory");
        if (w == 0) {
            ((float*)(s_dkv + slot * QSLOT + OFF_L2))[lane] = lsr == -INFINITY ? INFINITY : lsr * LOG2E;
            ((float*)(s_dkv + slot * QSLOT + OFF_DL))[lane] = dlr;
        }
        __syncthreads();
    };
    bool pc = false, pn = false;
    int ic = next_visit(i_first, pc);    // tile i
    const bool any = ic < Tq;
    if (a.nc > 1 && !any) return;   // empty chunk: no partial, its flag stays stale
    int in_ = Tq;                        // tile i + 1
    if (any) {
        stage_qtile(a, h, rstart(ic), rend(ic), 0, w, lane);
        load_ld(ic);
        in_ = next_visit(ic + 1, pn);
        publish(0);
    } else {
        __syncthreads();
    }
    auto advance = [&](int sn, int& in2, bool& pn2) __attribute__((always_inline)) {
        in2 = Tq;
        pn2 = false;
        if (in_ < Tq) {
            stage_qtile(a, h, rstart(in_), rend(in_), sn, w, lane);
            load_ld(in_);
            in2 = next_visit(in_ + 1, pn2);
        }
    };
    auto slot = [&](int k) __attribute__((always_inline)) { return (const char*)(s_dkv + k * QSLOT); };
    int sp_ = 2, sc_ = 0, sn_ = 1;   // slots of tiles i - 1, i, i + 1
    if constexpr (DROP) {
        // with dropout the vector work (the keep bytes and their tests)
        // outweighs the products, so a phase shift cannot hide it, and the
        // registers a shifted group carries across the barrier would spill:
        // both groups take each tile's steps in order, in phase
        f32x16 sc, dp;
        for (bool first = true; ic < Tq; first = false) {
            if (!first) publish(sc_);
            dkdv_sdp(slot(sc_), kf, kh_l, vb_l, sc, dp, g, n, hh);
            dkdv_dropw(a, rstart(ic), c0, sp.s_b, h, g, t, w, lane);
            int in2;
            bool pn2;
            advance(sn_, in2, pn2);
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {   // each half's P, dS straight into its products
                bf16x8 pb, db;
                dkdv_pds_half<DROP>(a, sc, dp, pb, db, slot(sc_), rstart(ic), pc, kj, g, t, w, lane, c2);
                dkdv_acc_half(slot(sc_), pb, db, dv, dk, g, c2, lane);
            }
            ic = in_; pc = pn; in_ = in2; pn = pn2;
            const int tt = sp_; sp_ = sc_; sc_ = sn_; sn_ = tt;
        }
    } else if (g == 0) {
        // group 0: products (the previous tile's dV, dK, then S, dP), then P, dS
        f32x16 sc, dp;
        bf16x8 pb[2], db[2];
        for (bool first = true; ic < Tq; first = false) {
            if (!first) {
                publish(sc_);
                dkdv_acc(slot(sp_), pb, db, dv, dk, g, lane);
            }
            dkdv_sdp(slot(sc_), kf, kh_l, vb_l, sc, dp, g, n, hh);
            int in2;
            bool pn2;
            advance(sn_, in2, pn2);
            dkdv_pds<DROP>(a, sc, dp, pb, db, slot(sc_), rstart(ic), pc, kj, g, t, w, lane);
            ic = in_; pc = pn; in_ = in2; pn = pn2;
            const int tt = sp_; sp_ = sc_; sc_ = sn_; sn_ = tt;
        }
        if (any) dkdv_acc(slot(sp_), pb, db, dv, dk, g, lane);   // the last tile's dV, dK
    } else {
        // group 1: P, dS of the previous tile, then the products
        f32x16 sc, dp;
        bf16x8 pb[2], db[2];
        int ip = Tq;
        bool pp = false;
        for (bool first = true; ic < Tq; first = false) {
            if (!first) {
                publish(sc_);
                dkdv_pds<DROP>(a, sc, dp, pb, db, slot(sp_), rstart(ip), pp, kj, g, t, w, lane);
            }
            int in2;
            bool pn2;
            advance(sn_, in2, pn2);
            if (!first) dkdv_acc(slot(sp_), pb, db, dv, dk, g, lane);
            dkdv_sdp(slot(sc_), kf, kh_l, vb_l, sc, dp, g, n, hh);
            ip = ic; pp = pc;
            ic = in_; pc = pn; in_ = in2; pn = pn2;
            const int tt = sp_; sp_ = sc_; sc_ = sn_; sn_ = tt;
        }
        if (ip < Tq) {   // the last tile: P, dS, then its dV, dK
            dkdv_pds<DROP>(a, sc, dp, pb, db, slot(sp_), rstart(ip), pp, kj, g, t, w, lane);
            dkdv_acc(slot(sp_), pb, db, dv, dk, g, lane);
        }
    }

    // dK summed into group 0, dV into group 1; then group 0 writes
    // dK = scale dK^T and group 1 dV = dV^T (lane = key kj, channels
    // 32dt + 8q + 4hh + 0..3)
    group_sum(dk, g, 1, t, lane);
    group_sum(dv, g, 0, t, lane);
    if (a.nc > 1) {   // this chunk's dK^T (group 0) and dV^T (group 1), unscaled
        const int64_t slot = ((int64_t)((sp.x + sp.b) >> 1) * a.H + h) * a.nc + ch;
        store_acc(a.part_kv + slot * PART_FLOATS, g == 0 ? dk : dv, w, lane);
        if (tid == 0) a.flag_kv[slot] = (int32_t)a.call_id;
        return;
    }
    if (kvalid)
        store_row_bf16((uint16_t*)(g == 0 ? a.dk : a.dv) + ((int64_t)kj * a.H + h) * HD, g == 0 ? dk : dv,
                       g == 0 ? a.scale : 1.f, hh);
}

// Sum of the dK/dV chunks of a key tile (chunk order), as the kernel above
// would have written it: wave 4g + t, lane = key 32t + n; group 0 dK, 1 dV.
__global__ __launch_bounds__(NTK) void fm_bwd_dkdv_reduce_kernel(BwdArgs a) {
    const int h = blockIdx.y, dt = blockIdx.z;
    const Span sp = span_of<2>(a, blockIdx.x);
    if (!sp.ok) return;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = w >> 2, t = w & 3, n = lane & 31, hh = lane >> 5;
    float4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const int64_t slot0 = ((int64_t)((sp.x + sp.b) >> 1) * a.H + h) * a.nc;
    sum_chunks(a, a.part_kv, a.flag_kv, slot0, dt, acc, w, lane);
    const int kj = sp.lo + 32 * t + n;
    if (kj < sp.hi)
        store_quads_bf16((uint16_t*)(g == 0 ? a.dk : a.dv) + ((int64_t)kj * a.H + h) * HD, acc,
                         g == 0 ? a.scale : 1.f, dt, hh);
}

// ---- dQ --------------------------------------------------------------------
// 8 waves, 256 queries (wave w: queries 32w..32w+31), two groups of four
// (one wave of each per SIMD) in opposite phase, as in the forward: in the
// step of key block j, group 0 issues dQ += dS_{j-1} K_{j-1} and S_j, dP_j,
// then turns S_j, dP_j into dS_j; group 1 first turns S_{j-1}, dP_{j-1}
// into dS_{j-1}, then issues the same products.  While one wave of a SIMD
// feeds its matrix unit, the other keeps its vector unit busy.  K, V and
// the mask intervals of a block sit in a 3-slot LDS ring: block j + 1 is
// stored (from registers loaded a step earlier) into the slot that block
// j - 2 has left, so one barrier per step suffices.
constexpr int NTQ = 512;         // dQ workgroup: 8 waves, 256 queries (two waves per SIMD)
constexpr int QBLK = NTQ / 128;  // 64-row blocks per dQ workgroup
constexpr int QSLOTS = 3;
__shared__ __attribute__((aligned(16))) char s_qk[QSLOTS][BLK * ROW_S];
__shared__ __attribute__((aligned(16))) char s_qv[QSLOTS][BLK * ROW_S];
__shared__ __attribute__((aligned(16))) Vec4 s_qmv[QSLOTS][BLK];

// Staging of a key block: K and V rows into their LDS slot with the
// asynchronous copies above (2 per wave per tensor); wave 0 also loads the
// mask intervals of key c0 + lane of a partial block into registers and
// stores them to the slot before the block is published.
__device__ __attribute__((always_inline)) inline void stage_block(const BwdArgs& a, int h, int c0, int c1, int slot,
                                                                  int w, const uint32_t (&vo)[2]) {
    const uint32_t rsb = (uint32_t)a.H * 2 * HD;
    const int64_t base = (int64_t)c0 * rsb + (int64_t)h * 2 * HD;
    const int nbytes = (c1 - c0 - 1) * (int)rsb + 2 * HD;   // through the block's last row
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.k + base), (short)0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.v + base), (short)0, nbytes, 0x00020000);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        dma_b16(s_qk[slot] + 1024 * (2 * w + x), rk, vo[x]);
        dma_b16(s_qv[slot] + 1024 * (2 * w + x), rv, vo[x]);
    }
}
// The stored vectors behind LTS, LTE, UTS, UTE of key c0 + lane (wave 0,
// partial blocks), defaults preset (as fill_column fills them).
__device__ __attribute__((always_inline)) inline Vec4 load_mv(const BwdArgs& a, int c0, int c1, bool part, int lane) {
    const int key = c0 + lane;
    const bool ld = part && key < c1;
    const int64_t N = a.N;
    const int s1 = (a.n_vec == 4 || (a.causal && a.n_vec == 2)) ? 1 : -1;
    const int s2 = a.n_vec == 4 ? 2 : -1;
    const int s3 = a.n_vec == 4 ? 3 : (!a.causal && a.n_vec == 2) ? 1 : -1;
    int m0 = 0, m1 = (int)N, m2 = 0, m3 = 0;
    if (ld) m0 = a.sv[key];
    if (ld && s1 >= 0) m1 = a.sv[s1 * N + key];
    if (ld && s2 >= 0) m2 = a.sv[s2 * N + key];
    if (ld && s3 >= 0) m3 = a.sv[s3 * N + key];
    return Vec4{m0, m1, m2, m3};
}

// The products of half u (keys 32u..32u+31) of a staged block: S^T = K Q^T
// and dP^T = V dO^T, register e = key 32u + 8(e>>2) + 4hh + (e&3), column =
// this lane's query.
// PF: the K and V fragments are read two k-steps ahead of the MFMAs that
// use them (an LDS read takes longer than one MFMA).  That pays with
// dropout, whose longer vector phase leaves a wave's products alone on the
// matrix unit; without dropout the partner wave covers the reads and the
// compiler's own order is 3 % faster.
template <bool PF>
__device__ __attribute__((always_inline)) inline void dq_sdp(int slot, int u, const bf16x8 (&qf)[8],
                                                             const bf16x8 (&gf)[8], f32x16& sc, f32x16& dp, int n,
                                                             int hh) {
#pragma unroll
    for (int e = 0; e < 16; ++e) { sc[e] = 0.f; dp[e] = 0.f; }
    const char* kt = s_qk[slot];
    const char* vt = s_qv[slot];
    auto frag = [&](const char* b, int s) __attribute__((always_inline)) {
        return as_bf16x8(*(const u32x4*)(b + soff(32 * u + n, 2 * s + hh)));
    };
    if constexpr (!PF) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            sc = mfma(frag(kt, s), qf[s], sc);
            dp = mfma(frag(vt, s), gf[s], dp);
        }
        return;
    }
    bf16x8 kr[3], vr[3];
#pragma unroll
    for (int s = 0; s < 2; ++s) { kr[s] = frag(kt, s); vr[s] = frag(vt, s); }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (s + 2 < 8) { kr[(s + 2) % 3] = frag(kt, s + 2); vr[(s + 2) % 3] = frag(vt, s + 2); }
        sc = mfma(kr[s % 3], qf[s], sc);
        dp = mfma(vr[s % 3], gf[s], dp);
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
// dQ^T += K^T dS^T over the 16-key groups 2u, 2u + 1 of a staged block;
// PF (as for dq_sdp): every transposed fragment is read before the MFMAs.
template <bool PF>
__device__ __attribute__((always_inline)) inline void dq_acc(int slot, int u, const bf16x8 (&db)[2], f32x16 (&dq)[4],
                                                             int lane) {
    if constexpr (!PF) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) dq[dt] = mfma(tr_frag_s(s_qk[slot], 2 * u + k, dt, lane), db[k], dq[dt]);
        return;
    }
    bf16x8 kt[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) kt[k][dt] = tr_frag_s(s_qk[slot], 2 * u + k, dt, lane);
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dq[dt] = mfma(kt[k][dt], db[k], dq[dt]);
    // keep the order: the 8 reads of group 2u, then those of 2u + 1 with
    // the first group's 4 MFMAs, then the last 4 MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}
// dS = P o (dP - Delta) of half u of a block as the B operand of dq_acc,
// with the element mask of a partial block (keys k and k + 4 of register e:
// the 32-row masks built by lanes k and k + 4 from the staged intervals).
template <bool DROP>
__device__ __attribute__((always_inline)) inline void dq_ds(const BwdArgs& a, f32x16& sc, const f32x16& dp,
                                                            bf16x8 (&db)[2], int slot, int u, bool part, int c0, int c1,
                                                            int kb, int q0, int qr, float l2, float dl, int h,
                                                            int lane, int hh) {
    if (part) {
        const int key = c0 + lane;
        const Vec4 mv = s_qmv[slot][lane];
        uint32_t mk = a.causal ? row_bits(0, key - q0) : 0u;
        if (key >= c1) mk = 0xffffffffu;
        mk |= row_bits(rel_row(mv.lts, q0), rel_row(mv.lte, q0)) | row_bits(rel_row(mv.uts, q0), rel_row(mv.ute, q0));
        const int mki = (int)mk;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int k0 = 32 * u + 8 * (e >> 2) + (e & 3);
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane(mki, k0);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(mki, k0 + 4);
            sc[e] = select_lanes(sc[e], -INFINITY, lo, hi);
        }
    }
    DropW dw;
    if constexpr (DROP) dw = drop_words(a.seed_lo, a.seed_hi, a.offset, qr, kb, h, hh);
    const float sl2 = a.scale_log2;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], sl2, -l2));
        float dpz = dp[e];
        if constexpr (DROP) {   // register e of half u: block 2u + (e >> 3), word 2((e >> 2) & 1) + hh
            const uint32_t byte = (dw.w[2 * u + (e >> 3)][(e >> 2) & 1] >> (8 * (e & 3))) & 0xffu;
            dpz = byte >= (uint32_t)a.drop_t ? dpz * a.drop_ks : 0.f;
        }
        db[e >> 3][e & 7] = (__bf16)(p * (dpz - dl));
    }
}

template <bool DROP>
__global__ __launch_bounds__(NTQ, 1) void fm_bwd_dq_kernel(BwdArgs a) {
    const int h = blockIdx.y;
    const Span sp = span_of<QBLK>(a, blockIdx.x);
    if (!sp.ok) return;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hh = lane >> 5, g = w >> 2;
    const int r0 = sp.lo, r1 = sp.hi;
    const int q0 = r0 + 32 * w;          // the wave's first row
    const int qr = q0 + n;               // this lane's query
    const bool qvalid = qr < r1;

    // Q and dO fragments (B operands: column = query n, channels 16s + 8hh),
    // lse in log2 units (+inf: no allowed key or no row, so P = 0) and Delta
    bf16x8 qf[8], gf[8];
    float l2 = INFINITY, dl = 0.f;
    {
        const int64_t off = ((int64_t)qr * a.H + h) * 2 * HD + 16 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            qf[s] = as_bf16x8(qvalid ? *(const u32x4*)((const char*)a.q + off + 32 * s) : u32x4{0, 0, 0, 0});
            gf[s] = as_bf16x8(qvalid ? *(const u32x4*)((const char*)a.dout + off + 32 * s) : u32x4{0, 0, 0, 0});
        }
        if (qvalid) {
            const float l = a.lse[(int64_t)h * a.N + qr];
            l2 = l == -INFINITY ? INFINITY : l * LOG2E;
            dl = a.delta[(int64_t)h * a.N + qr];
        }
    }
    f32x16 dq[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[dt][e] = 0.f;

    const int Tc = ceil_div(sp.e_b - sp.s_b, BLK);
    const int ch = blockIdx.z;
    const int kb_lim = a.causal ? min(Tc, (r1 - 1 - sp.s_b) / BLK + 1) : Tc;
    const int kb_end = a.nc > 1 ? min(kb_lim, (ch + 1) * a.kc) : kb_lim;
    const int kb_first = a.nc > 1 ? ch * a.kc : 0;
    const int32_t* xb = a.extrema + (int64_t)a.kb_off[sp.b] * 8;
    // Classes of a window of 64 key blocks from `wbase` (lane = block), kept
    // as ballots: the block extrema are read once per window, not once per
    // visited block.
    int wbase = -1;
    uint64_t wv = 0, wp = 0;
    auto next_visit = [&](int from, bool& part) __attribute__((always_inline)) -> int {
        while (from < kb_end) {
            if (wbase < 0 || from >= wbase + 64) {
                wbase = from;
                const int kb = from + lane;
                bool v = false, p = false;
                if (kb < kb_end) {
                    const int4 e0 = *(const int4*)(xb + (int64_t)kb * 8);
                    const int4 e1 = *(const int4*)(xb + (int64_t)kb * 8 + 4);
                    const int x[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
                    const int c0 = sp.s_b + kb * BLK, c1 = min(c0 + BLK, sp.e_b);
                    const TileInfo ti = classify_tile(r0, r1, c0, c1, x, a.causal);
                    v = ti.cls != CLS_FULL;
                    p = ti.cls == CLS_PARTIAL;
                }
                wv = __ballot(v);
                wp = __ballot(p);
            }
            const int off = from - wbase;   // 0..63
            const uint64_t m = wv >> off;
            if (m) {
                const int bit = __builtin_ctzll(m);
                part = ((wp >> (off + bit)) & 1ull) != 0;
                return from + bit;
            }
            from = wbase + 64;
        }
        return kb_end;
    };
    auto cstart = [&](int kb) __attribute__((always_inline)) { return sp.s_b + kb * BLK; };
    auto cend = [&](int kb) __attribute__((always_inline)) { return min(sp.s_b + (kb + 1) * BLK, sp.e_b); };

    // The pipeline, per visited block j (slot j mod 3) two half steps and one
    // barrier (nothing a block's second half reads changes inside the
    // block).  In the first half of block j every wave issues its
    // copies of block j + 1 into the slot block j - 2 has left; they (and
    // wave 0's mask intervals) are waited for at the end of block j, before
    // the barrier that publishes block j + 1.
    const uint32_t rsb = (uint32_t)a.H * 2 * HD;
    const uint32_t vo[2] = {stage_voff(2 * w, lane, rsb), stage_voff(2 * w + 1, lane, rsb)};
    Vec4 mvr = Vec4{0, 0, 0, 0};         // wave 0: mask intervals of the block in flight
    bool pc = false, pn = false;
    int kc = next_visit(kb_first, pc);   // block j
    if (a.nc > 1 && kc >= kb_end) return;   // empty chunk: no partial, its flag stays stale
    int kn = kb_end;                     // block j + 1
    // publish: wait for this wave's copies (and loads) of the block in
    // flight, put its mask intervals in place, barrier
    auto publish = [&](int slot, bool part) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0)
        asm volatile("" ::: "memory");
        if (w == 0 && part) s_qmv[slot][lane] = mvr;
        __syncthreads();
    };
    if (kc < kb_end) {
        stage_block(a, h, cstart(kc), cend(kc), 0, w, vo);
        if (w == 0 && pc) mvr = load_mv(a, cstart(kc), cend(kc), pc, lane);
        kn = next_visit(kc + 1, pn);
        publish(0, pc);
    } else {
        __syncthreads();
    }
    // issue block j + 1's copies into slot sn; returns block j + 2
    auto advance = [&](int sn, int& kn2, bool& pn2) __attribute__((always_inline)) {
        kn2 = kb_end;
        pn2 = false;
        if (kn < kb_end) {
            stage_block(a, h, cstart(kn), cend(kn), sn, w, vo);
            if (w == 0 && pn) mvr = load_mv(a, cstart(kn), cend(kn), pn, lane);
            kn2 = next_visit(kn + 1, pn2);
        }
    };
    int sp_ = 2, sc_ = 0, sn_ = 1;   // slots of blocks j - 1, j, j + 1
    if (q0 >= r1) {
        // a wave whose 32 queries all lie past the tile's end (short
        // sequences) only stages its share of each block and keeps the
        // barriers; its dQ stays zero
        for (bool first = true; kc < kb_end; first = false) {
            if (!first) publish(sc_, pc);
            int kn2;
            bool pn2;
            advance(sn_, kn2, pn2);
            kc = kn; pc = pn; kn = kn2; pn = pn2;
            const int t = sp_; sp_ = sc_; sc_ = sn_; sn_ = t;
        }
    } else if (g == 0) {
        // group 0: products of the half, then its dS
        f32x16 sc, dp;
        bf16x8 db[2];
        const bool any = kc < kb_end;
        for (bool first = true; kc < kb_end; first = false) {
            if (!first) {
                publish(sc_, pc);
                dq_acc<DROP>(sp_, 1, db, dq, lane);            // previous block, half 1
            }
            dq_sdp<DROP>(sc_, 0, qf, gf, sc, dp, n, hh);
            int kn2;
            bool pn2;
            advance(sn_, kn2, pn2);
            dq_ds<DROP>(a, sc, dp, db, sc_, 0, pc, cstart(kc), cend(kc), kc, q0, qr, l2, dl, h, lane, hh);
            dq_acc<DROP>(sc_, 0, db, dq, lane);
            dq_sdp<DROP>(sc_, 1, qf, gf, sc, dp, n, hh);
            dq_ds<DROP>(a, sc, dp, db, sc_, 1, pc, cstart(kc), cend(kc), kc, q0, qr, l2, dl, h, lane, hh);
            kc = kn; pc = pn; kn = kn2; pn = pn2;
            const int t = sp_; sp_ = sc_; sc_ = sn_; sn_ = t;
        }
        if (any) dq_acc<DROP>(sp_, 1, db, dq, lane);           // the last block, half 1
    } else {
        // group 1: dS of the previous half, then the products of this one
        f32x16 sc, dp;
        bf16x8 db[2];
        int kp = kb_end;
        bool pp = false;
        for (bool first = true; kc < kb_end; first = false) {
            if (!first) {
                publish(sc_, pc);
                dq_ds<DROP>(a, sc, dp, db, sp_, 1, pp, cstart(kp), cend(kp), kp, q0, qr, l2, dl, h, lane, hh);
            }
            int kn2;
            bool pn2;
            advance(sn_, kn2, pn2);
            if (!first) dq_acc<DROP>(sp_, 1, db, dq, lane);   // previous block, half 1
            dq_sdp<DROP>(sc_, 0, qf, gf, sc, dp, n, hh);
            dq_ds<DROP>(a, sc, dp, db, sc_, 0, pc, cstart(kc), cend(kc), kc, q0, qr, l2, dl, h, lane, hh);
            dq_acc<DROP>(sc_, 0, db, dq, lane);
            dq_sdp<DROP>(sc_, 1, qf, gf, sc, dp, n, hh);
            kp = kc; pp = pc;
            kc = kn; pc = pn; kn = kn2; pn = pn2;
            const int t = sp_; sp_ = sc_; sc_ = sn_; sn_ = t;
        }
        if (kp < kb_end) {   // the last block, half 1: dS, then its dQ
            dq_ds<DROP>(a, sc, dp, db, sp_, 1, pp, cstart(kp), cend(kp), kp, q0, qr, l2, dl, h, lane, hh);
            dq_acc<DROP>(sp_, 1, db, dq, lane);
        }
    }

    if (a.nc > 1) {   // this chunk's dQ^T, unscaled
        const int64_t slot = ((int64_t)((sp.x + (QBLK - 1) * sp.b) / QBLK) * a.H + h) * a.nc + ch;
        store_acc(a.part_q + slot * PART_FLOATS, dq, w, lane);
        if (tid == 0) a.flag_q[slot] = (int32_t)a.call_id;
        return;
    }
    // dQ = scale dQ^T: lane = query qr, channels 32dt + 8g + 4hh + 0..3
    if (qvalid) store_row_bf16((uint16_t*)a.dq + ((int64_t)qr * a.H + h) * HD, dq, a.scale, hh);
}

// Sum of the dQ chunks of a query tile (chunk order): wave w, lane = query
// 32w + n.
__global__ __launch_bounds__(NTQ) void fm_bwd_dq_reduce_kernel(BwdArgs a) {
    const int h = blockIdx.y, dt = blockIdx.z;
    const Span sp = span_of<QBLK>(a, blockIdx.x);
    if (!sp.ok) return;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hh = lane >> 5;
    float4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const int64_t slot0 = ((int64_t)((sp.x + (QBLK - 1) * sp.b) / QBLK) * a.H + h) * a.nc;
    sum_chunks(a, a.part_q, a.flag_q, slot0, dt, acc, w, lane);
    const int qr = sp.lo + 32 * w + n;
    if (qr < sp.hi) store_quads_bf16((uint16_t*)a.dq + ((int64_t)qr * a.H + h) * HD, acc, a.scale, dt, hh);
}

}  // namespace bwd

namespace {
hipError_t launch_dq_part(const BwdArgs& a, const dim3& grid, const dim3& rgrid, hipStream_t s) {
    if (a.drop_t > 0) hipLaunchKernelGGL(bwd::fm_bwd_dq_kernel<true>, grid, dim3(bwd::NTQ), 0, s, a);
    else hipLaunchKernelGGL(bwd::fm_bwd_dq_kernel<false>, grid, dim3(bwd::NTQ), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nc <= 1) return e;
    hipLaunchKernelGGL(bwd::fm_bwd_dq_reduce_kernel, rgrid, dim3(bwd::NTQ), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_dkdv_part(const BwdArgs& a, const dim3& grid, const dim3& rgrid, hipStream_t s) {
    if (a.drop_t > 0) hipLaunchKernelGGL(bwd::fm_bwd_dkdv_kernel<true>, grid, dim3(bwd::NTK), 0, s, a);
    else hipLaunchKernelGGL(bwd::fm_bwd_dkdv_kernel<false>, grid, dim3(bwd::NTK), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nc <= 1) return e;
    hipLaunchKernelGGL(bwd::fm_bwd_dkdv_reduce_kernel, rgrid, dim3(bwd::NTK), 0, s, a);
    return hipGetLastError();
}
}  // namespace

// Delta, then the dK/dV and dQ launches (and their reduces), which are
// independent of each other once Delta is written.  With a caller's second
// stream s_dq (and the caller's two events), the dQ launches are forked onto
// it after Delta and joined back into s, so that on problems where neither
// launch fills the chip the two run side by side; without one, everything
// runs on s, dK/dV first.
hipError_t launch_bwd_bf16(const BwdArgs& a, int64_t kb_cap, hipStream_t s, hipStream_t s_dq, hipEvent_t fork,
                           hipEvent_t join) {
    const int64_t nh = a.N * a.H;
    if (nh > 0) {
        const int64_t grid = (nh * 16 + bwd::NTH - 1) / bwd::NTH;
        hipLaunchKernelGGL(bwd::fm_bwd_delta_kernel, dim3((unsigned)grid), dim3(bwd::NTH), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (kb_cap <= 0 || a.N == 0) return hipSuccess;
    const dim3 grid((unsigned)kb_cap, (unsigned)a.H, (unsigned)a.nc);
    const dim3 rgrid((unsigned)kb_cap, (unsigned)a.H, (unsigned)bwd::RZ);
    hipError_t e;
    if (!s_dq) {
        if ((e = launch_dkdv_part(a, grid, rgrid, s)) != hipSuccess) return e;
        return launch_dq_part(a, grid, rgrid, s);
    }
    if ((e = hipEventRecord(fork, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(s_dq, fork, 0)) != hipSuccess) return e;
    if ((e = launch_dq_part(a, grid, rgrid, s_dq)) != hipSuccess) return e;
    if ((e = launch_dkdv_part(a, grid, rgrid, s)) != hipSuccess) return e;
    if ((e = hipEventRecord(join, s_dq)) != hipSuccess) return e;
    return hipStreamWaitEvent(s, join, 0);
}

}  // namespace fm
