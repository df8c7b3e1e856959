// Internal interface between the host API (fm_api.cpp) and the HIP
// translation units.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace fm {

// Header words of the workspace (int32 index) and class counts (byte offset).
// HDR_NMERGE counts the planners' split-row list, HDR_NFUSED the fused
// path's merge table (one entry per q tile and head).
enum : int { HDR_STATUS = 0, HDR_NKB = 1, HDR_NITEMS = 2, HDR_SCHED = 3, HDR_NSLOTS = 4, HDR_NMERGE = 5,
             HDR_NFUSED = 6 };
// Split-row list entry (int32 x MERGE_WORDS): slot of split 0, head, first
// row, end row (exclusive), number of splits, three zero words.
constexpr int MERGE_WORDS = 8;
constexpr int HDR_COUNTS_BYTE = 64;
constexpr int ITEM_WORDS = 16;  // seq, head, q_tile, kb_begin, kb_end, split_idx, n_splits, cost,
                                // seq_start, seq_end, kb_base, split0_slot, 0, 0, 0, 0
constexpr int SLOT_WORDS = 8;   // seq, q_tile, split_idx, n_splits, kb_begin, kb_end, cost, valid
// Bounds of the fused path's per-workgroup planner (fm_own_plan.h): the host
// takes the fused path only when they hold.
constexpr int FUSED_MAX_B = 255;      // sequences
constexpr int FUSED_MAX_ROWS = 512;   // q tiles over all sequences
constexpr int FUSED_MAX_MY = 8;       // work items per workgroup
// Workgroups per sequence of the tile-class launch (each classifies every
// PLAN_RC-th group of q tiles); class counts are kept per (sequence, group).
constexpr int PLAN_RC = 16;

// Worklist scratch carved from one buffer (all offsets 256-aligned).
struct ScratchLayout {
    size_t off_slots, off_pos, off_seq_counts, off_sl_off, bytes;
    int64_t slot_cap;
};

struct PlanPtrs {
    const int32_t* cu;
    int B;
    int64_t N;
    int H, Br, Bc, S;
    int causal;
    const int32_t* kb_off;
    const int32_t* extrema;
    const int32_t* status;     // read
    int32_t* status_rw;        // written when capacities overflow (may equal status)
    int32_t* items;
    int64_t items_cap;
    int32_t* n_items;
    int64_t* class_counts;
    int32_t* sched_counter;    // nullable: zeroed when given
    int32_t* n_slots;          // nullable
    uint8_t* tile_class;       // nullable
    int64_t tile_class_cap;
    char* scratch;
    ScratchLayout sl;
    int cost_cap;              // largest cost a q tile can have (histogram size - 1)
    int32_t* merge_list;       // nullable: split-row list (S > 0), MERGE_WORDS per entry
    int32_t* n_merge;          // nullable: its entry count
};

hipError_t launch_extrema(const int32_t* sv, int n_vec, int causal, const int32_t* cu, int B,
                          int64_t N, int Bc, int32_t* kb_off, int32_t* extrema,
                          int64_t extrema_cap, int32_t* n_kblocks, int32_t* status,
                          int n_cu, hipStream_t s);

hipError_t launch_worklist(const PlanPtrs& p, hipStream_t s);

// Plan path: extrema, tile classes, sort (three launches).  Writes kb_off,
// extrema, n_kblocks and the status word too.
hipError_t launch_plan(const int32_t* sv, int n_vec, int32_t* ext, int64_t ext_cap, int32_t* n_kblocks,
                       int32_t* kb_off_out, const PlanPtrs& p, int n_cu, hipStream_t s);

// Attention launch arguments shared by the bf16 and fp32 paths.
struct AttnArgs {
    const void* q; const void* k; const void* v; void* out; float* lse;
    int64_t N; int H, D, B;
    const int32_t* cu; const int32_t* sv; int n_vec; int causal;
    float scale_log2;          // scale * log2(e)
    int Br, Bc, S;
    const int32_t* kb_off; const int32_t* extrema;
    const int32_t* items; const int32_t* n_items; int64_t items_cap;
    int32_t* sched_counter;
    const int32_t* sl_off;     // per-sequence first slot (split partial index)
    float* partial;            // split partials (S > 0)
    const int32_t* merge_list; // split-row list (S > 0)
    const int32_t* n_merge;
    int64_t merge_cap;         // entries the list can hold
    unsigned flags;
    // fused path only: where the in-kernel planner writes the plan
    int32_t* w_hdr; int32_t* w_kb_off; int32_t* w_ext; int32_t* w_items; int64_t* w_counts;
    int32_t* w_merge;          // split-row list (S > 0), else null
    // attention dropout (planned path): a pair is dropped when its byte is
    // below drop_t (0 = no dropout); kept values are scaled by drop_ks
    int drop_t; float drop_ks; uint32_t seed_lo, seed_hi, offset;
};

hipError_t launch_attn_bf16(const AttnArgs& a, int n_cu, hipStream_t s);
// One launch that plans in LDS and attends (small bf16 problems).
hipError_t launch_fused_bf16(const AttnArgs& a, int n_cu, hipStream_t s);
int fused_grid(int n_cu);
hipError_t launch_attn_f32(const AttnArgs& a, int n_cu, hipStream_t s);

// Backward launch arguments (bf16, head_dim 128).
struct BwdArgs {
    const void* q; const void* k; const void* v; const void* out; const void* dout; const float* lse;
    void* dq; void* dk; void* dv;
    float* delta;              // workspace: fp32 [H][N]
    int64_t N; int H, B;
    const int32_t* cu; const int32_t* sv; int n_vec; int causal;
    float scale, scale_log2;   // scale, scale * log2(e)
    const int32_t* kb_off; const int32_t* extrema; const int32_t* n_kb; const int32_t* status;
    // small problems: the q tiles of a key tile (dK/dV) and the key blocks of
    // a query tile (dQ) are cut into nc chunks of qc / kc that run as
    // separate workgroups writing fp32 partials; two reduce launches sum
    // them in chunk order.  nc == 1: no chunks, no partials.
    int nc, qc, kc;
    float* part_kv; int32_t* flag_kv;   // [slot_kv][nc] partials (128 KB each) and their flags
    float* part_q; int32_t* flag_q;     // [slot_q][nc]
    uint32_t call_id;                   // flag value of this call (never 0)
    int drop_t; float drop_ks; uint32_t seed_lo, seed_hi, offset;   // dropout, as in AttnArgs
};

// Rotary embedding of q and k rows in place (bf16 or fp32).
struct RopeArgs {
    void* q; void* k; int dtype;
    int64_t N; int Hq, Hk, D, B;
    const int32_t* cu; const float* cos_t; const float* sin_t; int64_t max_pos;
    int inverse; int32_t* status;
};
hipError_t launch_rope(const RopeArgs& a, hipStream_t s);

// Most chunks a backward tile is cut into (small problems).
constexpr int BWD_MAX_CHUNKS = 8;
// Key block (columns per extrema row) of the backward's plan.
constexpr int bwd_block_k() { return 64; }
// Delta, then dK/dV, then dQ; kb_cap bounds the number of 64-key blocks.
// s_dq, fork, join: a second stream and two events of the caller's for the
// dQ launches, or all null (everything on s).
hipError_t launch_bwd_bf16(const BwdArgs& a, int64_t kb_cap, hipStream_t s, hipStream_t s_dq, hipEvent_t fork,
                           hipEvent_t join);

}  // namespace fm
