// Host side of the C ABI declared in include/fm_api.h: argument checks,
// workspace layout, and the launch sequence (extrema -> tiles/sort ->
// attention [-> merge]) on the caller's stream.  No device allocation, no
// stream synchronisation (except the fm_read_status test helper).
#include "fm_api.h"
#include "fm_internal.h"
#include "fm_bf16_copies.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() { g_err.clear(); return FM_OK; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxBytes = (int64_t)1 << 46;  // 64 TiB: any layout above is rejected

// Number of compute units of the current device (cached per device).
int device_cus(int* n_cu) {
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FM_E_HIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
    if (cache[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            return fail(FM_E_HIP, "hipDeviceGetAttribute(multiprocessor count) failed");
        cache[dev] = v;
    }
    *n_cu = cache[dev];
    return FM_OK;
}

bool mask_form_ok(int n_vec, int causal) {
    if (causal) return n_vec == 1 || n_vec == 2;
    return n_vec == 2 || n_vec == 4;
}

// Upper bounds from host-known sizes only.
struct Caps { int64_t kb, qt, slot, item, map; int cost; };

bool compute_caps(int64_t N, int B, int H, int Br, int Bc, int S, Caps* c) {
    const double n = (double)N;
    c->kb = cdiv(N, Bc) + B;
    c->qt = cdiv(N, Br) + B;
    if (S == 0) {
        c->slot = c->qt;
    } else {
        // sum_b Tr_b * ceil(Tc_b / S) with Tr <= L/Br + 1, ceil(Tc/S) <= L/(Bc S) + 1/S + 1
        const double v = n * n / ((double)Br * Bc * S) + n * (1.0 + 1.0 / S) / Br + n / ((double)Bc * S) +
                         (double)B * (1.0 + 1.0 / S);
        if (v > 4e12) return false;
        c->slot = (int64_t)ceil(v) + 1;
    }
    const double m = n * n / ((double)Br * Bc) + n / Br + n / Bc + B;
    if (m > 4e12) return false;
    c->map = (int64_t)ceil(m) + 1;
    c->item = c->slot * H;
    c->cost = S > 0 ? S : (int)cdiv(N, Bc);
    return c->item < INT32_MAX;
}

fm::ScratchLayout scratch_layout(int B, const Caps& c) {
    fm::ScratchLayout s;
    size_t off = 0;
    s.off_slots = off; off = align256(off + (size_t)c.slot * fm::SLOT_WORDS * sizeof(int32_t));
    s.off_pos = off; off = align256(off + (size_t)c.slot * sizeof(int32_t));
    s.off_seq_counts = off; off = align256(off + (size_t)B * fm::PLAN_RC * 3 * sizeof(long long));
    s.off_sl_off = off; off = align256(off + (size_t)(B + 1) * sizeof(int32_t));
    s.bytes = off;
    s.slot_cap = c.slot;
    return s;
}

int check_sizes(int64_t N, int B, int H) {
    if (B < 1 || B > FM_MAX_SEQS) return fail(FM_E_INVAL, "B=%d outside [1, %d]", B, FM_MAX_SEQS);
    if (N < 0 || N >= INT32_MAX) return fail(FM_E_INVAL, "N=%lld outside [0, 2^31-1)", (long long)N);
    if (H < 1) return fail(FM_E_INVAL, "H=%d must be >= 1", H);
    return FM_OK;
}

int tile_config(int dtype, int D, int* bq, int* bk) {
    if (dtype == FM_BF16) {
        if (D != 128) return fail(FM_E_UNSUPPORTED, "bf16 path is built for head_dim 128 (got %d)", D);
        *bq = 256; *bk = 64;
        return FM_OK;
    }
    if (dtype == FM_F32) {
        if (D != 32 && D != 64 && D != 128)
            return fail(FM_E_UNSUPPORTED, "fp32 path is built for head_dim 32, 64, 128 (got %d)", D);
        *bq = 64; *bk = 32;
        return FM_OK;
    }
    return fail(FM_E_UNSUPPORTED, "unknown dtype %d", dtype);
}

int auto_split(int64_t N, int B, int H, int dtype) {
    if (dtype != FM_BF16) return 0;
    const int64_t est_items = (int64_t)H * (cdiv(N, 256) + B);
    return est_items >= 512 ? 0 : 6;
}

// The fused path (one launch in which every workgroup plans its own items)
// takes small problems: every bound of its tables holds for these sizes, and
// a workgroup runs at most a few items (each item pays its own planning, so
// larger problems are faster with the planning launches and the longest-first
// schedule of the planned path).
constexpr int64_t kFusedMaxTokens = 16384;

bool fused_eligible(int64_t N, int B, int H, int dtype, int D, int bq, int bk, int S, int n_vec,
                    unsigned flags, int n_cu) {
    (void)n_vec;
    if (dtype != FM_BF16 || D != 128 || bq != 256 || bk != 64 || N <= 0 || N > kFusedMaxTokens) return false;
    if (flags & (FM_FLAG_NO_SKIP | FM_FLAG_PLAN_READY)) return false;
    if (B > fm::FUSED_MAX_B) return false;
    Caps c;
    if (!compute_caps(N, B, H, bq, bk, S, &c)) return false;
    return c.qt <= fm::FUSED_MAX_ROWS && c.item <= (int64_t)fm::FUSED_MAX_MY * fm::fused_grid(n_cu);
}

// Entries of the merge table: the planners list split rows only (a split
// row has >= 2 slots, so slot_cap * H / 2 + 1 entries suffice); the fused
// path keeps one entry per (q tile, head).
int64_t merge_entries(const Caps& c, int H) { return std::max<int64_t>(c.slot * H / 2 + 1, c.qt * H); }

int layout_impl(int64_t N, int B, int H, int D, int Br, int Bc, int S, int want_map,
                fm_ws_layout* out) {
    int rc = check_sizes(N, B, H);
    if (rc) return rc;
    if (Br < 1 || Bc < 1) return fail(FM_E_INVAL, "block sizes must be >= 1 (got %d, %d)", Br, Bc);
    if (S < 0) return fail(FM_E_INVAL, "max_kb_per_item must be >= 0 here (got %d)", S);
    if (D < 1) return fail(FM_E_INVAL, "head_dim must be >= 1");
    Caps c;
    if (!compute_caps(N, B, H, Br, Bc, S, &c)) return fail(FM_E_INVAL, "problem too large for one plan");
    if (c.cost > FM_MAX_COST)
        return fail(FM_E_UNSUPPORTED, "a q tile may visit %d key blocks (> %d); raise block_k or split",
                    c.cost, FM_MAX_COST);
    if (cdiv(N, Bc) > 32767)   // visit-list entries hold the key block in 15 bits
        return fail(FM_E_UNSUPPORTED, "more than 32767 key blocks (N / block_k); raise block_k");
    const fm::ScratchLayout sl = scratch_layout(B, c);
    fm_ws_layout L;
    memset(&L, 0, sizeof(L));
    size_t off = 0;
    L.off_hdr = off; off = align256(off + 256);
    L.off_kb_off = off; off = align256(off + (size_t)(B + 1) * 4);
    L.off_extrema = off; off = align256(off + (size_t)c.kb * 32);
    L.off_items = off; off = align256(off + (size_t)c.item * fm::ITEM_WORDS * 4);
    L.off_tile_class = want_map ? off : 0; if (want_map) off = align256(off + (size_t)c.map);
    L.off_scratch = off; L.scratch_bytes = sl.bytes; off = align256(off + sl.bytes);
    // per (slot, head): Br x D fp16 values of O / l, then m, l and the scale exponent per row
    L.partial_bytes = S > 0 ? (size_t)c.slot * H * ((size_t)Br * D * 2 + 3 * (size_t)Br * 4) : 0;
    L.off_partial = S > 0 ? off : 0; off = align256(off + L.partial_bytes);
    // merge table (split rows)
    L.off_merge = S > 0 ? off : 0;
    if (S > 0) off = align256(off + (size_t)merge_entries(c, H) * fm::MERGE_WORDS * 4);
    if ((int64_t)off > kMaxBytes) return fail(FM_E_INVAL, "workspace would exceed 64 TiB");
    L.bytes = off;
    L.kb_cap = c.kb; L.item_cap = c.item; L.map_cap = want_map ? c.map : 0; L.slot_cap = c.slot;
    L.block_q = Br; L.block_k = Bc; L.max_kb_per_item = S; L.head_dim = D;
    *out = L;
    return FM_OK;
}

// Workspace of fm_attn_fwd_noalloc.  Each GPU the library runs on holds its
// own copy (loaded with the library's device code) until the process ends.
// On the host `scratch` names a stand-in, not device memory: host code uses
// only the device address hipGetSymbolAddress returns for it, looked up
// once per device with that device current.
static __device__ __align__(256) char scratch[FM_NOALLOC_SCRATCH_BYTES];

int noalloc_scratch(void** out) {
    static std::mutex mu;
    static std::vector<void*> addr;   // per device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(FM_E_HIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(FM_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return FM_OK;
}

// Flag value of one call that marks the partials it wrote: a process-wide
// counter, never 0, so flags need no clearing between calls.
uint32_t next_call_id() {
    static std::atomic<uint32_t> ctr{0};
    uint32_t v;
    do { v = ctr.fetch_add(1, std::memory_order_relaxed) + 1; } while (v == 0);
    return v;
}

int hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FM_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return FM_OK;
}

int preprocess_impl(const int32_t* sv, int n_vec, int causal, const int32_t* cu, int B, int64_t N,
                    int Bc, int32_t* kb_off, int32_t* ext, int64_t ext_cap, int32_t* nkb,
                    int32_t* status, hipStream_t s) {
    int rc = check_sizes(N, B, 1);
    if (rc) return rc;
    if (!mask_form_ok(n_vec, causal))
        return fail(FM_E_INVAL, "unsupported (n_vec=%d, causal=%d): causal takes 1 or 2 vectors, non-causal 2 or 4",
                    n_vec, causal);
    if (Bc < 1) return fail(FM_E_INVAL, "block_k must be >= 1");
    if (!cu || !kb_off || !ext || !nkb || !status || (N > 0 && !sv))
        return fail(FM_E_INVAL, "null pointer argument");
    if (ext_cap < cdiv(N, Bc) + B)
        return fail(FM_E_WORKSPACE, "extrema_cap %lld < ceil(N/block_k)+B = %lld", (long long)ext_cap,
                    (long long)(cdiv(N, Bc) + B));
    int n_cu = 0;
    if ((rc = device_cus(&n_cu))) return rc;
    return hip_check(fm::launch_extrema(sv, n_vec, causal ? 1 : 0, cu, B, N, Bc, kb_off, ext, ext_cap,
                                        nkb, status, n_cu, s), "extrema launch");
}

// Backward workspace: header, kb_off, extrema at block_k = 64, Delta, and
// for small problems the chunk partials and their flags.
struct BwdLayout {
    size_t off_hdr, off_kb_off, off_extrema, off_delta, off_part_kv, off_flag_kv, off_part_q, off_flag_q, bytes;
    int64_t kb_cap;
    int nc, qc, kc;
};

// Chunks of the backward, from the sizes only (so the bits do not depend
// on the device): when the dK/dV launch would have fewer than 256
// workgroups, each key tile's q tiles and each query tile's key blocks are
// cut into nc <= 8 chunks, about two workgroups per compute unit of a
// 256-CU device (16 chunks measured slower: more partial traffic, and the
// chunks' fixed start-up cost).
constexpr int kBwdChunkWgs = 256, kBwdMaxChunks = fm::BWD_MAX_CHUNKS;
constexpr size_t kBwdPartBytes = 8 * 64 * 64 * 4;   // one chunk partial: 8 waves x 64 lanes x 64 floats

int bwd_layout(int64_t N, int B, int H, BwdLayout* L) {
    const int bk = fm::bwd_block_k();
    L->kb_cap = cdiv(N, bk) + B;
    const int64_t wgs = (cdiv(N, 2 * bk) + B) * (int64_t)H;
    L->nc = wgs >= kBwdChunkWgs ? 1 : (int)std::min<int64_t>(kBwdMaxChunks, cdiv(2 * kBwdChunkWgs, std::max<int64_t>(wgs, 1)));
    L->qc = L->kc = (int)std::max<int64_t>(1, cdiv(cdiv(N, bk), L->nc));
    size_t off = 0;
    L->off_hdr = off; off = align256(off + 256);
    L->off_kb_off = off; off = align256(off + (size_t)(B + 1) * 4);
    L->off_extrema = off; off = align256(off + (size_t)L->kb_cap * 32);
    L->off_delta = off; off = align256(off + (size_t)H * (size_t)N * 4);
    L->off_part_kv = L->off_flag_kv = L->off_part_q = L->off_flag_q = 0;
    if (L->nc > 1) {
        const size_t skv = (size_t)((L->kb_cap + B) / 2 + 1) * H * L->nc;       // (x + b) / 2
        const size_t sq = (size_t)((L->kb_cap + 3 * (int64_t)B) / 4 + 1) * H * L->nc;   // (x + 3b) / 4
        L->off_part_kv = off; off = align256(off + skv * kBwdPartBytes);
        L->off_flag_kv = off; off = align256(off + skv * 4);
        L->off_part_q = off; off = align256(off + sq * kBwdPartBytes);
        L->off_flag_q = off; off = align256(off + sq * 4);
    }
    L->bytes = off;
    if ((int64_t)off > kMaxBytes) return fail(FM_E_INVAL, "problem too large");
    if (L->kb_cap > INT32_MAX / 2) return fail(FM_E_INVAL, "too many key blocks");
    return FM_OK;
}

int bwd_supported(int dtype, int D) {
    if (dtype != FM_BF16) return fail(FM_E_UNSUPPORTED, "the backward is built for bf16 only (dtype %d)", dtype);
    if (D != 128) return fail(FM_E_UNSUPPORTED, "the backward is built for head_dim 128 (got %d)", D);
    return FM_OK;
}

int worklist_impl(const int32_t* cu, int B, int64_t N, int H, int Br, int Bc, const int32_t* kb_off,
                  const int32_t* ext, const int32_t* status, int32_t* status_rw, int causal, int S,
                  int32_t* items, int64_t items_cap, int32_t* n_items, int64_t* counts,
                  uint8_t* map, int64_t map_cap, void* scratch, size_t scratch_bytes,
                  int32_t* sched, int32_t* n_slots, int32_t* merge, hipStream_t s) {
    int rc = check_sizes(N, B, H);
    if (rc) return rc;
    if (Br < 1 || Bc < 1) return fail(FM_E_INVAL, "block sizes must be >= 1");
    if (S < 0) return fail(FM_E_INVAL, "max_kb_per_item must be >= 0");
    if (!cu || !kb_off || !ext || !status || !items || !n_items || !counts || !scratch)
        return fail(FM_E_INVAL, "null pointer argument");
    Caps c;
    if (!compute_caps(N, B, H, Br, Bc, S, &c)) return fail(FM_E_INVAL, "problem too large for one plan");
    if (c.cost > FM_MAX_COST) return fail(FM_E_UNSUPPORTED, "cost bound %d > %d", c.cost, FM_MAX_COST);
    const fm::ScratchLayout sl = scratch_layout(B, c);
    if (scratch_bytes < sl.bytes)
        return fail(FM_E_WORKSPACE, "scratch %zu < %zu bytes", scratch_bytes, sl.bytes);
    if (items_cap < c.item)
        return fail(FM_E_WORKSPACE, "items_cap %lld < bound %lld", (long long)items_cap, (long long)c.item);
    if (map && map_cap < c.map)
        return fail(FM_E_WORKSPACE, "tile_class_cap %lld < bound %lld", (long long)map_cap, (long long)c.map);
    fm::PlanPtrs p;
    p.cu = cu; p.B = B; p.N = N; p.H = H; p.Br = Br; p.Bc = Bc; p.S = S; p.causal = causal ? 1 : 0;
    p.kb_off = kb_off; p.extrema = ext; p.status = status; p.status_rw = status_rw;
    p.items = items; p.items_cap = items_cap; p.n_items = n_items; p.class_counts = counts;
    p.sched_counter = sched; p.n_slots = n_slots; p.tile_class = map; p.tile_class_cap = map ? map_cap : 0;
    p.scratch = (char*)scratch; p.sl = sl; p.cost_cap = c.cost; p.merge_list = S > 0 ? merge : nullptr;
    p.n_merge = nullptr;
    return hip_check(fm::launch_worklist(p, s), "worklist launch");
}

struct Ws {
    char* base;
    fm_ws_layout L;
    int32_t* hdr() const { return (int32_t*)(base + L.off_hdr); }
    int64_t* counts() const { return (int64_t*)(base + L.off_hdr + fm::HDR_COUNTS_BYTE); }
};

int build_plan_impl(const Ws& w, const int32_t* cu, int B, int64_t N, int H, const int32_t* sv,
                    int n_vec, int causal, hipStream_t s) {
    const fm_ws_layout& L = w.L;
    int32_t* hdr = w.hdr();
    int rc = check_sizes(N, B, H);
    if (rc) return rc;
    if (!mask_form_ok(n_vec, causal))
        return fail(FM_E_INVAL, "unsupported (n_vec=%d, causal=%d): causal takes 1 or 2 vectors, non-causal 2 or 4",
                    n_vec, causal);
    if (!cu || (N > 0 && !sv)) return fail(FM_E_INVAL, "null pointer argument");
    Caps c;
    if (!compute_caps(N, B, H, L.block_q, L.block_k, L.max_kb_per_item, &c))
        return fail(FM_E_INVAL, "problem too large for one plan");
    fm::PlanPtrs p;
    p.cu = cu; p.B = B; p.N = N; p.H = H; p.Br = L.block_q; p.Bc = L.block_k; p.S = L.max_kb_per_item;
    p.causal = causal ? 1 : 0;
    p.kb_off = (const int32_t*)(w.base + L.off_kb_off);
    p.extrema = (const int32_t*)(w.base + L.off_extrema);
    p.status = hdr + fm::HDR_STATUS; p.status_rw = hdr + fm::HDR_STATUS;
    p.items = (int32_t*)(w.base + L.off_items); p.items_cap = L.item_cap;
    p.n_items = hdr + fm::HDR_NITEMS; p.class_counts = w.counts();
    p.sched_counter = hdr + fm::HDR_SCHED; p.n_slots = hdr + fm::HDR_NSLOTS;
    p.tile_class = L.off_tile_class ? (uint8_t*)(w.base + L.off_tile_class) : nullptr;
    p.tile_class_cap = L.off_tile_class ? L.map_cap : 0;
    p.scratch = w.base + L.off_scratch; p.sl = scratch_layout(B, c); p.cost_cap = c.cost;
    p.merge_list = L.off_merge ? (int32_t*)(w.base + L.off_merge) : nullptr;
    p.n_merge = L.off_merge ? hdr + fm::HDR_NMERGE : nullptr;
    int n_cu = 0;
    if ((rc = device_cus(&n_cu))) return rc;
    return hip_check(fm::launch_plan(sv, n_vec, (int32_t*)(w.base + L.off_extrema), L.kb_cap, hdr + fm::HDR_NKB,
                                     (int32_t*)(w.base + L.off_kb_off), p, n_cu, s),
                     "plan launch");
}

}  // namespace

extern "C" {

const char* fm_last_error(void) { return g_err.c_str(); }

int fm_version(void) { return 100; }

int fm_self_check(void) {
    using namespace fm::bf16c;
    for (int g = 0; g < 2; ++g) {
        const int nblk = g == 0 ? KBLK : VBLK, ch = g == 0 ? KCH : VCH;
        int seen[SLOT_BLK] = {0};
        for (int t = 0; t < GW; ++t)
            for (int i = 0; i < NCOPY; ++i) {
                const int blk = copy_block(t, i);
                if (blk < 0 || blk >= SLOT_BLK)
                    return fail(FM_E_INVAL, "copy table: group %d wave %d copy %d fills block %d", g, t, i, blk);
                seen[blk]++;
                for (int lane = 0; lane < 64; ++lane) {
                    const uint32_t cp = copy_lane(g, t, i, lane);
                    const int row = (int)(cp & 0xffu), byte = (int)(cp >> 8);
                    if (row >= BC || byte > 16 * 15 || byte % 16)
                        return fail(FM_E_INVAL, "copy table: group %d wave %d copy %d lane %d reads row %d byte %d",
                                    g, t, i, lane, row, byte);
                    // a data block must hold exactly the chunk the kernel reads there
                    if (blk < nblk) {
                        const int q = 64 * blk + lane;
                        if (row != q / ch || (q % ch < 16 && byte != 16 * (q % ch)))
                            return fail(FM_E_INVAL, "copy table: group %d block %d lane %d misplaced", g, blk, lane);
                    }
                }
            }
        for (int b = 0; b < SLOT_BLK; ++b)
            if (seen[b] != 1) return fail(FM_E_INVAL, "copy table: group %d block %d filled %d times", g, b, seen[b]);
    }
    return FM_OK;
}

int fm_get_tile_config(int dtype, int head_dim, int* block_q, int* block_k) {
    if (!block_q || !block_k) return fail(FM_E_INVAL, "null pointer argument");
    int rc = tile_config(dtype, head_dim, block_q, block_k);
    return rc ? rc : ok();
}

int fm_auto_split(int64_t N, int B, int H, int dtype, int head_dim) {
    int bq, bk;
    if (check_sizes(N, B, H) || tile_config(dtype, head_dim, &bq, &bk)) return -1;
    return auto_split(N, B, H, dtype);
}

int fm_workspace_layout(int64_t N, int B, int H, int head_dim, int block_q, int block_k,
                        int max_kb_per_item, int want_class_map, fm_ws_layout* out) {
    if (!out) return fail(FM_E_INVAL, "null pointer argument");
    int rc = layout_impl(N, B, H, head_dim, block_q, block_k, max_kb_per_item, want_class_map, out);
    return rc ? rc : ok();
}

size_t fm_workspace_size(int64_t N, int B, int H, int head_dim, int dtype, int max_kb_per_item) {
    int bq, bk;
    if (check_sizes(N, B, H) || tile_config(dtype, head_dim, &bq, &bk)) return 0;
    int S = max_kb_per_item < 0 ? auto_split(N, B, H, dtype) : max_kb_per_item;
    if (dtype == FM_F32) S = 0;
    fm_ws_layout L;
    if (layout_impl(N, B, H, head_dim, bq, bk, S, 0, &L)) return 0;
    return L.bytes;
}

size_t fm_worklist_scratch_size(int64_t N, int B, int H, int block_q, int block_k, int max_kb_per_item) {
    if (check_sizes(N, B, H) || block_q < 1 || block_k < 1 || max_kb_per_item < 0) return 0;
    Caps c;
    if (!compute_caps(N, B, H, block_q, block_k, max_kb_per_item, &c)) return 0;
    return scratch_layout(B, c).bytes;
}

int fm_preprocess_mask(const int32_t* startend, int n_vec, int causal, const int32_t* cu_seqlens, int B,
                       int64_t N, int block_k, int32_t* kb_off, int32_t* extrema, int64_t extrema_cap,
                       int32_t* n_kblocks, int32_t* status, hipStream_t stream) {
    int rc = preprocess_impl(startend, n_vec, causal, cu_seqlens, B, N, block_k, kb_off, extrema,
                             extrema_cap, n_kblocks, status, stream);
    return rc ? rc : ok();
}

int fm_build_worklist(const int32_t* cu_seqlens, int B, int64_t N, int H, int block_q, int block_k,
                      const int32_t* kb_off, const int32_t* extrema, const int32_t* status, int causal,
                      int max_kb_per_item, int32_t* items, int64_t items_cap, int32_t* n_items,
                      int64_t* class_counts, uint8_t* tile_class, int64_t tile_class_cap, void* scratch,
                      size_t scratch_bytes, hipStream_t stream) {
    int rc = worklist_impl(cu_seqlens, B, N, H, block_q, block_k, kb_off, extrema, status,
                           const_cast<int32_t*>(status), causal, max_kb_per_item, items, items_cap,
                           n_items, class_counts, tile_class, tile_class_cap, scratch, scratch_bytes,
                           nullptr, nullptr, nullptr, stream);
    return rc ? rc : ok();
}

int fm_build_plan(const int32_t* cu_seqlens, int B, int64_t N, int H, int head_dim, int dtype,
                  const int32_t* startend, int n_vec, int causal, int block_q, int block_k,
                  int max_kb_per_item, int want_class_map, void* workspace, size_t ws_bytes,
                  hipStream_t stream) {
    int bq = block_q, bk = block_k, rc;
    if (bq == 0 || bk == 0) {
        int dq, dk;
        if ((rc = tile_config(dtype, head_dim, &dq, &dk))) return rc;
        if (bq == 0) bq = dq;
        if (bk == 0) bk = dk;
    }
    int S = max_kb_per_item < 0 ? auto_split(N, B, H, dtype) : max_kb_per_item;
    if (dtype == FM_F32) S = 0;
    Ws w;
    if ((rc = layout_impl(N, B, H, head_dim, bq, bk, S, want_class_map, &w.L))) return rc;
    if (!workspace) return fail(FM_E_INVAL, "null workspace");
    if (ws_bytes < w.L.bytes) return fail(FM_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.L.bytes);
    w.base = (char*)workspace;
    rc = build_plan_impl(w, cu_seqlens, B, N, H, startend, n_vec, causal, stream);
    return rc ? rc : ok();
}

// Dropout probability -> byte threshold t = round(256 p) (0: no dropout) and
// the scale 256 / (256 - t) of kept values.
static int dropout_params(float p, int* t, float* ks) {
    if (!(p >= 0.f && p < 1.f)) return fail(FM_E_INVAL, "dropout probability must be in [0, 1) (got %g)", (double)p);
    *t = std::min(255, (int)floor((double)p * 256.0 + 0.5));
    *ks = (float)(256.0 / (256.0 - *t));
    return FM_OK;
}

static int attn_fwd_impl(const void* q, const void* k, const void* v, int dtype, int64_t N, int H, int D,
                  const int32_t* cu_seqlens, int B, const int32_t* startend, int n_vec, int causal,
                  float scale, void* out, float* softmax_lse, int block_q, int block_k,
                  int max_kb_per_item, void* workspace, size_t ws_bytes, unsigned flags,
                  float dropout_p, uint64_t seed, uint64_t offset, hipStream_t stream) {
    int rc = check_sizes(N, B, H);
    if (rc) return rc;
    int drop_t = 0;
    float drop_ks = 1.f;
    if ((rc = dropout_params(dropout_p, &drop_t, &drop_ks))) return rc;
    if (drop_t > 0 && (dtype != FM_BF16 || (flags & FM_FLAG_NO_SKIP)))
        return fail(FM_E_UNSUPPORTED, "dropout is built for the bf16 path without FM_FLAG_NO_SKIP");
    int dq, dk;
    if ((rc = tile_config(dtype, D, &dq, &dk))) return rc;
    const int bq = block_q ? block_q : dq, bk = block_k ? block_k : dk;
    if (dtype == FM_BF16 && (bq != 256 || bk != 64))
        return fail(FM_E_UNSUPPORTED, "bf16 path is built for block_q=256, block_k=64 (got %d, %d)", bq, bk);
    if (dtype == FM_F32 && (bq < 1 || bq > 64 || bk < 1 || bk > 64))
        return fail(FM_E_UNSUPPORTED, "fp32 path takes 1 <= block_q, block_k <= 64 (got %d, %d)", bq, bk);
    if (!mask_form_ok(n_vec, causal))
        return fail(FM_E_INVAL, "unsupported (n_vec=%d, causal=%d)", n_vec, causal);
    if (!(scale > 0.f) || !isfinite(scale)) return fail(FM_E_INVAL, "scale must be finite and > 0");
    if (flags & ~(FM_FLAG_NO_SKIP | FM_FLAG_PLAN_READY)) return fail(FM_E_INVAL, "unknown flags 0x%x", flags);
    int S = max_kb_per_item < 0 ? auto_split(N, B, H, dtype) : max_kb_per_item;
    if (dtype == FM_F32) {
        if (max_kb_per_item > 0) return fail(FM_E_UNSUPPORTED, "fp32 path does not split items");
        S = 0;
    }
    if ((flags & FM_FLAG_NO_SKIP) && S != 0)
        return fail(FM_E_INVAL, "FM_FLAG_NO_SKIP requires max_kb_per_item == 0");
    if (!cu_seqlens || !workspace) return fail(FM_E_INVAL, "null pointer argument");
    if (N > 0 && (!q || !k || !v || !out || !softmax_lse || !startend))
        return fail(FM_E_INVAL, "null pointer argument");
    Ws w;
    if ((rc = layout_impl(N, B, H, D, bq, bk, S, 0, &w.L))) return rc;
    if (ws_bytes < w.L.bytes) return fail(FM_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.L.bytes);
    w.base = (char*)workspace;
    int n_cu = 0;
    if ((rc = device_cus(&n_cu))) return rc;
    const bool fused = drop_t == 0 && fused_eligible(N, B, H, dtype, D, bq, bk, S, n_vec, flags, n_cu);
    if (!fused && !(flags & FM_FLAG_PLAN_READY)) {
        if ((rc = build_plan_impl(w, cu_seqlens, B, N, H, startend, n_vec, causal, stream))) return rc;
    }
    if (N == 0) return ok();
    fm::AttnArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = softmax_lse;
    a.N = N; a.H = H; a.D = D; a.B = B;
    a.cu = cu_seqlens; a.sv = startend; a.n_vec = n_vec; a.causal = causal ? 1 : 0;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    a.Br = bq; a.Bc = bk; a.S = S;
    a.kb_off = (const int32_t*)(w.base + w.L.off_kb_off);
    a.extrema = (const int32_t*)(w.base + w.L.off_extrema);
    a.items = (const int32_t*)(w.base + w.L.off_items);
    a.n_items = w.hdr() + fm::HDR_NITEMS;
    a.items_cap = w.L.item_cap;
    a.sched_counter = w.hdr() + fm::HDR_SCHED;
    const fm::ScratchLayout sl = [&] {
        Caps c;
        compute_caps(N, B, H, bq, bk, S, &c);
        return scratch_layout(B, c);
    }();
    a.sl_off = (const int32_t*)(w.base + w.L.off_scratch + sl.off_sl_off);
    a.partial = S > 0 ? (float*)(w.base + w.L.off_partial) : nullptr;
    a.merge_list = S > 0 ? (const int32_t*)(w.base + w.L.off_merge) : nullptr;
    a.n_merge = w.hdr() + fm::HDR_NMERGE;
    a.merge_cap = S > 0 ? [&] {
        Caps c;
        compute_caps(N, B, H, bq, bk, S, &c);
        return merge_entries(c, H);
    }() : 0;
    a.flags = flags;
    a.w_hdr = w.hdr();
    a.w_kb_off = (int32_t*)(w.base + w.L.off_kb_off);
    a.w_ext = (int32_t*)(w.base + w.L.off_extrema);
    a.w_items = (int32_t*)(w.base + w.L.off_items);
    a.w_counts = w.counts();
    a.w_merge = S > 0 ? (int32_t*)(w.base + w.L.off_merge) : nullptr;
    a.drop_t = drop_t; a.drop_ks = drop_ks;
    a.seed_lo = (uint32_t)seed; a.seed_hi = (uint32_t)(seed >> 32); a.offset = (uint32_t)offset;
    if (fused) {   // the fused path's merge table: one entry per (q tile, head)
        a.n_merge = w.hdr() + fm::HDR_NFUSED;
        if (S > 0) a.merge_cap = (cdiv(N, bq) + B) * (int64_t)H;
    }
    const hipError_t e = fused ? fm::launch_fused_bf16(a, n_cu, stream)
                       : dtype == FM_BF16 ? fm::launch_attn_bf16(a, n_cu, stream)
                                          : fm::launch_attn_f32(a, n_cu, stream);
    if ((rc = hip_check(e, "attention launch"))) return rc;
    return ok();
}

int fm_attn_fwd(const void* q, const void* k, const void* v, int dtype, int64_t N, int H, int D,
                const int32_t* cu_seqlens, int B, const int32_t* startend, int n_vec, int causal,
                float scale, void* out, float* softmax_lse, int block_q, int block_k,
                int max_kb_per_item, void* workspace, size_t ws_bytes, unsigned flags,
                hipStream_t stream) {
    return attn_fwd_impl(q, k, v, dtype, N, H, D, cu_seqlens, B, startend, n_vec, causal, scale, out, softmax_lse,
                         block_q, block_k, max_kb_per_item, workspace, ws_bytes, flags, 0.f, 0, 0, stream);
}

int fm_attn_fwd_dropout(const void* q, const void* k, const void* v, int dtype, int64_t N, int H, int D,
                        const int32_t* cu_seqlens, int B, const int32_t* startend, int n_vec, int causal,
                        float scale, void* out, float* softmax_lse, int block_q, int block_k,
                        int max_kb_per_item, void* workspace, size_t ws_bytes, unsigned flags,
                        float dropout_p, uint64_t seed, uint64_t offset, hipStream_t stream) {
    return attn_fwd_impl(q, k, v, dtype, N, H, D, cu_seqlens, B, startend, n_vec, causal, scale, out, softmax_lse,
                         block_q, block_k, max_kb_per_item, workspace, ws_bytes, flags, dropout_p, seed, offset,
                         stream);
}

int fm_attn_fwd_noalloc(const void* q, const void* k, const void* v, int dtype, int64_t N, int H, int D,
                        const int32_t* cu_seqlens, int B, const int32_t* startend, int n_vec, int causal,
                        float scale, void* out, float* softmax_lse, int block_q, int block_k,
                        int max_kb_per_item, unsigned flags, hipStream_t stream) {
    int rc = check_sizes(N, B, H);
    if (rc) return rc;
    if (flags & FM_FLAG_PLAN_READY)
        return fail(FM_E_INVAL, "FM_FLAG_PLAN_READY is not accepted: the allocation-free call builds its plan");
    // the layout fm_attn_fwd would need (its argument checks follow there)
    int dq, dk;
    if ((rc = tile_config(dtype, D, &dq, &dk))) return rc;
    const int bq = block_q ? block_q : dq, bk = block_k ? block_k : dk;
    const int S = dtype == FM_F32 ? 0 : max_kb_per_item < 0 ? auto_split(N, B, H, dtype) : max_kb_per_item;
    fm_ws_layout L;
    if ((rc = layout_impl(N, B, H, D, bq, bk, S, 0, &L))) return rc;
    if (L.bytes > FM_NOALLOC_SCRATCH_BYTES)
        return fail(FM_E_WORKSPACE,
                    "this problem needs a %zu-byte workspace, more than the %zu bytes of the allocation-free "
                    "entry point's array: call fm_attn_fwd with a workspace",
                    L.bytes, (size_t)FM_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((rc = noalloc_scratch(&ws))) return rc;
    rc = attn_fwd_impl(q, k, v, dtype, N, H, D, cu_seqlens, B, startend, n_vec, causal, scale, out, softmax_lse,
                       block_q, block_k, max_kb_per_item, ws, FM_NOALLOC_SCRATCH_BYTES, flags, 0.f, 0, 0, stream);
    return rc ? rc : ok();
}

int fm_fused_path(int64_t N, int B, int H, int head_dim, int dtype, int n_vec, int causal,
                  int max_kb_per_item, unsigned flags) {
    int bq, bk;
    if (check_sizes(N, B, H) || tile_config(dtype, head_dim, &bq, &bk) || !mask_form_ok(n_vec, causal)) return -1;
    const int S = max_kb_per_item < 0 ? auto_split(N, B, H, dtype) : max_kb_per_item;
    int n_cu = 0;
    if (device_cus(&n_cu)) return -1;
    return fused_eligible(N, B, H, dtype, head_dim, bq, bk, S, n_vec, flags, n_cu) ? 1 : 0;
}

size_t fm_bwd_workspace_size(int64_t N, int B, int H, int head_dim, int dtype) {
    BwdLayout L;
    if (check_sizes(N, B, H) || bwd_supported(dtype, head_dim) || bwd_layout(N, B, H, &L)) return 0;
    return L.bytes;
}

static int attn_bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* dout,
                  const float* softmax_lse, int dtype, int64_t N, int H, int D, const int32_t* cu_seqlens,
                  int B, const int32_t* startend, int n_vec, int causal, float scale, void* dq, void* dk,
                  void* dv, void* workspace, size_t ws_bytes, float dropout_p, uint64_t seed, uint64_t offset,
                  hipStream_t stream, hipStream_t dq_stream, hipEvent_t fork, hipEvent_t join) {
    int rc = check_sizes(N, B, H);
    if (dq_stream && (!fork || !join || dq_stream == stream))
        return fail(FM_E_INVAL, "a dQ stream needs two events and must differ from the stream");
    if (rc) return rc;
    int drop_t = 0;
    float drop_ks = 1.f;
    if ((rc = dropout_params(dropout_p, &drop_t, &drop_ks))) return rc;
    if ((rc = bwd_supported(dtype, D))) return rc;
    if (!mask_form_ok(n_vec, causal))
        return fail(FM_E_INVAL, "unsupported (n_vec=%d, causal=%d)", n_vec, causal);
    if (!(scale > 0.f) || !isfinite(scale)) return fail(FM_E_INVAL, "scale must be finite and > 0");
    if (!cu_seqlens || !workspace) return fail(FM_E_INVAL, "null pointer argument");
    if (N > 0 && (!q || !k || !v || !out || !dout || !softmax_lse || !startend || !dq || !dk || !dv))
        return fail(FM_E_INVAL, "null pointer argument");
    BwdLayout L;
    if ((rc = bwd_layout(N, B, H, &L))) return rc;
    if (ws_bytes < L.bytes) return fail(FM_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.bytes);
    char* base = (char*)workspace;
    int32_t* hdr = (int32_t*)(base + L.off_hdr);
    int32_t* kb_off = (int32_t*)(base + L.off_kb_off);
    int32_t* ext = (int32_t*)(base + L.off_extrema);
    if ((rc = preprocess_impl(startend, n_vec, causal, cu_seqlens, B, N, fm::bwd_block_k(), kb_off, ext,
                              L.kb_cap, hdr + fm::HDR_NKB, hdr + fm::HDR_STATUS, stream)))
        return rc;
    if (N == 0) return ok();
    fm::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = softmax_lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.delta = (float*)(base + L.off_delta);
    a.N = N; a.H = H; a.B = B;
    a.cu = cu_seqlens; a.sv = startend; a.n_vec = n_vec; a.causal = causal ? 1 : 0;
    a.scale = scale;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    a.kb_off = kb_off; a.extrema = ext; a.n_kb = hdr + fm::HDR_NKB; a.status = hdr + fm::HDR_STATUS;
    a.nc = L.nc; a.qc = L.qc; a.kc = L.kc;
    a.part_kv = L.nc > 1 ? (float*)(base + L.off_part_kv) : nullptr;
    a.flag_kv = L.nc > 1 ? (int32_t*)(base + L.off_flag_kv) : nullptr;
    a.part_q = L.nc > 1 ? (float*)(base + L.off_part_q) : nullptr;
    a.flag_q = L.nc > 1 ? (int32_t*)(base + L.off_flag_q) : nullptr;
    a.call_id = next_call_id();
    a.drop_t = drop_t; a.drop_ks = drop_ks;
    a.seed_lo = (uint32_t)seed; a.seed_hi = (uint32_t)(seed >> 32); a.offset = (uint32_t)offset;
    if ((rc = hip_check(fm::launch_bwd_bf16(a, L.kb_cap, stream, dq_stream, fork, join), "backward launch"))) return rc;
    return ok();
}

int fm_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                const float* softmax_lse, int dtype, int64_t N, int H, int D, const int32_t* cu_seqlens,
                int B, const int32_t* startend, int n_vec, int causal, float scale, void* dq, void* dk,
                void* dv, void* workspace, size_t ws_bytes, hipStream_t stream) {
    return attn_bwd_impl(q, k, v, out, dout, softmax_lse, dtype, N, H, D, cu_seqlens, B, startend, n_vec, causal,
                         scale, dq, dk, dv, workspace, ws_bytes, 0.f, 0, 0, stream, nullptr, nullptr, nullptr);
}

int fm_attn_bwd_streams(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* softmax_lse, int dtype, int64_t N, int H, int D, const int32_t* cu_seqlens,
                        int B, const int32_t* startend, int n_vec, int causal, float scale, void* dq, void* dk,
                        void* dv, void* workspace, size_t ws_bytes, hipStream_t stream, hipStream_t dq_stream,
                        hipEvent_t fork, hipEvent_t join) {
    if (!dq_stream) return fail(FM_E_INVAL, "null dQ stream (use fm_attn_bwd for one stream)");
    return attn_bwd_impl(q, k, v, out, dout, softmax_lse, dtype, N, H, D, cu_seqlens, B, startend, n_vec, causal,
                         scale, dq, dk, dv, workspace, ws_bytes, 0.f, 0, 0, stream, dq_stream, fork, join);
}

int fm_attn_bwd_dropout(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* softmax_lse, int dtype, int64_t N, int H, int D, const int32_t* cu_seqlens,
                        int B, const int32_t* startend, int n_vec, int causal, float scale, void* dq, void* dk,
                        void* dv, void* workspace, size_t ws_bytes, float dropout_p, uint64_t seed,
                        uint64_t offset, hipStream_t stream) {
    return attn_bwd_impl(q, k, v, out, dout, softmax_lse, dtype, N, H, D, cu_seqlens, B, startend, n_vec, causal,
                         scale, dq, dk, dv, workspace, ws_bytes, dropout_p, seed, offset, stream, nullptr, nullptr,
                         nullptr);
}

int fm_attn_bwd_dropout_streams(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* softmax_lse, int dtype, int64_t N, int H, int D,
                                const int32_t* cu_seqlens, int B, const int32_t* startend, int n_vec, int causal,
                                float scale, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                                float dropout_p, uint64_t seed, uint64_t offset, hipStream_t stream,
                                hipStream_t dq_stream, hipEvent_t fork, hipEvent_t join) {
    if (!dq_stream) return fail(FM_E_INVAL, "null dQ stream (use fm_attn_bwd_dropout for one stream)");
    return attn_bwd_impl(q, k, v, out, dout, softmax_lse, dtype, N, H, D, cu_seqlens, B, startend, n_vec, causal,
                         scale, dq, dk, dv, workspace, ws_bytes, dropout_p, seed, offset, stream, dq_stream, fork,
                         join);
}

int fm_rope_qk(void* q, void* k, int dtype, int64_t N, int Hq, int Hk, int head_dim, const int32_t* cu_seqlens,
               int B, const float* cos_table, const float* sin_table, int64_t max_pos, int inverse,
               int32_t* status, hipStream_t stream) {
    if (B < 1 || B > FM_MAX_SEQS) return fail(FM_E_INVAL, "B=%d outside [1, %d]", B, FM_MAX_SEQS);
    if (N < 0 || N >= INT32_MAX) return fail(FM_E_INVAL, "N=%lld outside [0, 2^31-1)", (long long)N);
    if (Hq < 0 || Hk < 0 || Hq + Hk < 1) return fail(FM_E_INVAL, "need Hq, Hk >= 0 and Hq + Hk >= 1");
    if (dtype != FM_BF16 && dtype != FM_F32) return fail(FM_E_UNSUPPORTED, "unknown dtype %d", dtype);
    const int mult = dtype == FM_BF16 ? 16 : 8;
    if (head_dim < mult || head_dim > 512 || head_dim % mult)
        return fail(FM_E_UNSUPPORTED, "head_dim %d: must be a multiple of %d in [%d, 512]", head_dim, mult, mult);
    if (max_pos < 1) return fail(FM_E_INVAL, "max_pos must be >= 1");
    if ((int64_t)N * (Hq + Hk) * (head_dim / 2) > ((int64_t)1 << 40)) return fail(FM_E_INVAL, "problem too large");
    if (!cu_seqlens) return fail(FM_E_INVAL, "null pointer argument");
    if (N > 0 && (!cos_table || !sin_table || (Hq > 0 && !q) || (Hk > 0 && !k)))
        return fail(FM_E_INVAL, "null pointer argument");
    auto misaligned = [](const void* p) { return p && ((uintptr_t)p & 15); };
    if (misaligned(q) || misaligned(k) || misaligned(cos_table) || misaligned(sin_table))
        return fail(FM_E_INVAL, "q, k and the tables must be 16-byte aligned");
    if (N == 0) return ok();
    fm::RopeArgs a;
    a.q = q; a.k = k; a.dtype = dtype; a.N = N; a.Hq = Hq; a.Hk = Hk; a.D = head_dim; a.B = B;
    a.cu = cu_seqlens; a.cos_t = cos_table; a.sin_t = sin_table; a.max_pos = max_pos;
    a.inverse = inverse ? 1 : 0; a.status = status;
    int rc = hip_check(fm::launch_rope(a, stream), "rope launch");
    return rc ? rc : ok();
}

int fm_read_status(const void* workspace, hipStream_t stream, int32_t* status) {
    if (!workspace || !status) return fail(FM_E_INVAL, "null pointer argument");
    int rc;
    if ((rc = hip_check(hipMemcpyAsync(status, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, stream),
                        "hipMemcpyAsync")))
        return rc;
    if ((rc = hip_check(hipStreamSynchronize(stream), "hipStreamSynchronize"))) return rc;
    return ok();
}

}  // extern "C"
