/*
 * fm_api.h — C ABI of libflashmask_mi355.so: FlashMask-style attention
 * (forward and backward) over packed, variable-length sequences on MI355X
 * (gfx950).
 *
 * What is computed (sources cited by page title and section):
 *   [FM] PaddleNLP FlashMask article (m.nxbn.cn/news/70198)
 *   [VP] Varlen-Packing technical document (www.gsyq.cn/news/432802)
 *
 *   Sequences are concatenated without padding into one token axis of N
 *   rows; sequence b owns rows [cu_seqlens[b], cu_seqlens[b+1]) ([VP]
 *   background, §2).  Each key column j carries a column-wise sparse mask:
 *   query rows in [LTS_j, LTE_j) and [UTS_j, UTE_j) do not attend to it
 *   ([FM] §2.1, §2.2).  Endpoints are GLOBAL row indices into the packed
 *   axis ([FM] §6.7: a running offset is added per packed sample).  A
 *   causal call also hides keys after the query.  Pairs in different
 *   sequences never attend.  The forward returns `out` and `softmax_lse`,
 *   the outputs the backward op consumes ([FM] §3.4).
 *
 *   The kernels follow the two phases of [FM] §3: a preprocessing pass
 *   reduces the vectors to per-key-block min/max ("extrema", §3.1), and the
 *   attention loop classifies every Br x Bc tile as fully masked (skipped),
 *   partially masked (masked element by element) or unmasked (no mask work)
 *   (§3.2).  Work is a compact list of (sequence, head, q tile) items
 *   instead of the fixed seq_count x n_head x ceil(max_len/Br) grid of
 *   [VP] §2.
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device memory on the current device; the
 *     caller owns every buffer.  The library never allocates or frees
 *     device memory, never synchronises the stream (except fm_read_status,
 *     a test helper) and keeps no pointer after return.  All work is
 *     enqueued on `stream` (NULL = the legacy default stream).
 *   - Return value: FM_OK or an FM_E_* code; fm_last_error() then gives a
 *     thread-local message.  Arguments are checked on the host before any
 *     launch; nothing is enqueued when a call fails.
 *   - Errors in DEVICE data (cu_seqlens not starting at 0, decreasing, or
 *     not ending at N) cannot be seen on the host without a sync.  The
 *     preprocessing kernel detects them, writes a non-zero status word,
 *     and every later stage then produces no work items; `out` and
 *     `softmax_lse` are left unwritten.  fm_read_status() reports it.
 *   - Calls that share a workspace must be ordered on one stream.
 */
#ifndef FM_API_H
#define FM_API_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define FM_OK            0
#define FM_E_INVAL       1  /* bad shape, pointer, or argument combination */
#define FM_E_UNSUPPORTED 2  /* dtype / head_dim / size not built in        */
#define FM_E_WORKSPACE   3  /* workspace or output capacity too small       */
#define FM_E_HIP         4  /* a HIP runtime call or launch failed          */

/* ---- dtypes of q, k, v, out ------------------------------------------- */
#define FM_BF16 0           /* bf16 storage, fp32 accumulation (MFMA)       */
#define FM_F32  1           /* fp32 storage and arithmetic (reference path) */

/* ---- flags of fm_attn_fwd --------------------------------------------- */
/* Visit every tile that is fully masked by the interval vectors (but not
 * those fully masked by the causal rule) and mask it element by element
 * instead of skipping it.  Used to show that skipping changes no bit of
 * the result ([FM] §3.3).  Requires max_kb_per_item == 0.                 */
#define FM_FLAG_NO_SKIP    0x1u
/* The workspace already holds the plan built by fm_build_plan (or by
 * fm_preprocess_mask + fm_build_worklist at the workspace layout) for the
 * same cu_seqlens, startend, n_vec, causal, N, B, H, tiles and split: the
 * preprocessing and worklist launches are skipped.  This is the per-layer
 * call when every layer shares one mask.                                   */
#define FM_FLAG_PLAN_READY 0x2u

/* ---- limits ----------------------------------------------------------- */
#define FM_MAX_SEQS        16383  /* B: sequences per call                 */
#define FM_MAX_COST        8191   /* key blocks one work item may visit    */

/* Status word bits written by the preprocessing kernel. */
#define FM_STATUS_CU0      0x1    /* cu_seqlens[0] != 0                     */
#define FM_STATUS_ORDER    0x2    /* cu_seqlens decreases somewhere         */
#define FM_STATUS_CUN      0x4    /* cu_seqlens[B] != N                     */
#define FM_STATUS_CAP      0x8    /* more key blocks than extrema_cap       */
#define FM_STATUS_POS      0x10   /* fm_rope_qk: a position outside the tables */

/* Returns the message of the last failing call on this thread ("" if none). */
const char* fm_last_error(void);

/* Library version, e.g. 100 for 0.1.0. */
int fm_version(void);

/*
 * Host-only check of the fixed tables the kernels derive addresses from
 * (which wave copies which K/V block of a tile, and the row and byte each
 * lane reads): every block is copied exactly once and every lane stays
 * inside its tile.  Needs no GPU.  Returns FM_OK, or FM_E_INVAL with the
 * first violation in fm_last_error().
 */
int fm_self_check(void);

/*
 * Default tile sizes (Br query rows x Bc key columns) of fm_attn_fwd for a
 * (dtype, head_dim).  bf16 is built for head_dim 128 with Br = 256,
 * Bc = 64; fp32 is built for head_dim 32, 64 and 128 and accepts any
 * 1 <= Br <= 64, 1 <= Bc <= 64 (default 64 x 32).
 * Returns FM_E_UNSUPPORTED for other combinations.
 */
int fm_get_tile_config(int dtype, int head_dim, int* block_q, int* block_k);

/*
 * Split size S (max key blocks per work item) chosen when fm_attn_fwd
 * receives max_kb_per_item < 0.  Host-only arithmetic on the sizes: long
 * rows are cut (into chunks of at most 6 key blocks) only when fewer than
 * 512 items, H * (N / Br + B), would leave compute units idle.
 * Returns S >= 0, or -1 on bad arguments.
 */
int fm_auto_split(int64_t N, int B, int H, int dtype, int head_dim);

/*
 * Workspace layout.  All offsets are bytes from the workspace base and are
 * 256-byte aligned.  `*_cap` are host-side upper bounds computed from
 * (N, B, H, Br, Bc, S) only.
 *   hdr:        int32 status, n_kblocks, n_items, sched_counter, n_slots,
 *               n_merge, n_fused at byte 0..27; int64 class_counts[3] at
 *               byte 64.
 *   kb_off:     int32 [B+1]         first key block of each sequence
 *   extrema:    int32 [kb_cap][8]   per key block: min/max of LTS, LTE,
 *                                   UTS, UTE (in that order)
 *   items:      int32 [item_cap][16] work items (see fm_build_worklist)
 *   tile_class: uint8 [map_cap]     per-tile classes (only if requested)
 *   scratch:    worklist scratch (fm_worklist_scratch_size bytes)
 *   partial:    split partials (S > 0), per (slot, head) Br*D fp16 values of
 *               the split's O / l scaled by 2^-e (e per row), then Br each of
 *               fp32 m, fp32 l and int32 e: Br*D*2 + 3*Br*4 bytes
 *   merge:      int32 [max(slot_cap * H / 2 + 1, qt_cap * H)][8] (S > 0),
 *               entries of slot of split 0, head, first row, end row,
 *               number of splits, 3 zero words: the planners list the split
 *               rows (n_merge entries, one per split row and head); the
 *               fused path of fm_attn_fwd keeps one entry per (q tile,
 *               head), q tile r at r * H + head (n_fused entries; rows of
 *               one chunk say 1 split), qt_cap = ceil(N / block_q) + B.
 */
typedef struct fm_ws_layout {
    size_t  bytes;
    size_t  off_hdr, off_kb_off, off_extrema, off_items, off_tile_class;
    size_t  off_scratch, off_partial, off_merge;
    size_t  scratch_bytes, partial_bytes;
    int64_t kb_cap, item_cap, map_cap, slot_cap;
    int32_t block_q, block_k, max_kb_per_item, head_dim;
} fm_ws_layout;

/*
 * Fills *out for a problem; head_dim is needed only to size the split
 * partials (pass the attention head_dim; any value >= 1 when S == 0).
 * want_class_map != 0 reserves the per-tile class map.
 */
int fm_workspace_layout(int64_t N, int B, int H, int head_dim, int block_q, int block_k,
                        int max_kb_per_item, int want_class_map, fm_ws_layout* out);

/* Bytes of fm_workspace_layout(...).bytes for fm_attn_fwd's defaults:
 * tiles from fm_get_tile_config, split from max_kb_per_item (< 0 = auto),
 * no class map.  Returns 0 on bad arguments.                               */
size_t fm_workspace_size(int64_t N, int B, int H, int head_dim, int dtype, int max_kb_per_item);

/* Scratch bytes fm_build_worklist needs for these sizes (0 on bad args). */
size_t fm_worklist_scratch_size(int64_t N, int B, int H, int block_q, int block_k,
                                int max_kb_per_item);

/*
 * Preprocessing ([FM] §3.1).  Default-fills the stored vectors ([FM]
 * §2.2: LTS, UTS default to 0; LTE, UTE to the query length, here N) and
 * reduces them, per sequence and per key block of block_k columns starting
 * at the sequence's first column (the last block may be ragged), to
 *   extrema[g*8 + 0..7] = min LTS, max LTS, min LTE, max LTE,
 *                          min UTS, max UTS, min UTE, max UTE
 * for global key block g = kb_off[b] + kb.  In causal mode the UT slots
 * are 0.
 *
 * startend:  int32 [n_vec][N] device, structure-of-arrays.  Accepted
 *            (n_vec, causal): causal 1 = {LTS}, causal 2 = {LTS, LTE},
 *            non-causal 2 = {LTS, UTE}, non-causal 4 = {LTS, LTE, UTS, UTE};
 *            anything else -> FM_E_INVAL.  Any int32 value is accepted;
 *            start >= end is an empty interval.
 * cu_seqlens: int32 [B+1] device, 0 = cu[0] <= ... <= cu[B] = N
 *            (checked on the device, see the status word).
 * block_k:   >= 1.  kb_off: int32 [B+1] device (out).
 * extrema:   int32 [extrema_cap][8] device (out); extrema_cap must be at
 *            least ceil(N / block_k) + B (FM_E_WORKSPACE otherwise).
 * n_kblocks, status: int32 device scalars (out).
 */
int fm_preprocess_mask(const int32_t* startend, int n_vec, int causal,
                       const int32_t* cu_seqlens, int B, int64_t N, int block_k,
                       int32_t* kb_off, int32_t* extrema, int64_t extrema_cap,
                       int32_t* n_kblocks, int32_t* status, hipStream_t stream);

/*
 * Tile classification and work list ([FM] §3.2; [VP] §2 for the
 * (sequence, head, q tile) triple).  Inputs kb_off, extrema and status
 * come from fm_preprocess_mask with the same block_k.
 *
 * Tile (b, qt, kb): rows [r0, r1), columns [c0, c1), both clipped to the
 * sequence.  FULL when causal and c0 >= r1, or r0 >= LTS_max and
 * r1 <= LTE_min, or (non-causal) r0 >= UTS_max and r1 <= UTE_min; else
 * PARTIAL when a causal tile reaches above the diagonal (c1 > r0 + 1), or
 * r0 < LTE_max and r1 > LTS_min, or (non-causal) r0 < UTE_max and
 * r1 > UTS_min; else UNMASKED.  r1 is the exclusive row end.
 *
 * For every q tile, K = its non-FULL key blocks and cost = |K|.  With
 * S = max_kb_per_item: S == 0 or cost <= S gives one item over
 * [K_first, K_last + 1) ([0, 0) when K is empty); otherwise K is cut into
 * ceil(cost / S) consecutive chunks whose sizes differ by at most one,
 * larger chunks first.  One item per head.
 * Item record (int32 x 16): seq, head, q_tile, kb_begin, kb_end, split_idx,
 * n_splits, cost, then derived words for the attention kernel: seq_start
 * (cu_seqlens[seq]), seq_end, kb_base (kb_off[seq]), split0_slot (slot
 * index of split 0 of this q tile; its partials sit at (slot + s) * H +
 * head), and four zero words.  Order: ascending (-cost, seq, q_tile,
 * split_idx, head), i.e. longest first, deterministic.
 *
 * items: int32 [items_cap][16] device (out); n_items: int32 device (out).
 * class_counts: int64 [3] device (out): FULL, PARTIAL, UNMASKED tiles,
 *   counted once per (sequence, q tile, key block) for all heads.
 * tile_class: uint8 device (out, nullable): per sequence row-major
 *   [Tr_b][Tc_b], sequences concatenated; 0 FULL, 1 PARTIAL, 2 UNMASKED.
 * scratch: device, fm_worklist_scratch_size(...) bytes.
 */
int fm_build_worklist(const int32_t* cu_seqlens, int B, int64_t N, int H,
                      int block_q, int block_k, const int32_t* kb_off,
                      const int32_t* extrema, const int32_t* status, int causal,
                      int max_kb_per_item, int32_t* items, int64_t items_cap,
                      int32_t* n_items, int64_t* class_counts, uint8_t* tile_class,
                      int64_t tile_class_cap, void* scratch, size_t scratch_bytes,
                      hipStream_t stream);

/*
 * Both of the above into a workspace laid out by fm_workspace_layout(N,
 * B, H, head_dim, block_q, block_k, max_kb_per_item, want_class_map).
 * block_q / block_k = 0 take fm_get_tile_config(dtype, head_dim);
 * max_kb_per_item < 0 takes fm_auto_split.
 */
int fm_build_plan(const int32_t* cu_seqlens, int B, int64_t N, int H, int head_dim, int dtype,
                  const int32_t* startend, int n_vec, int causal, int block_q, int block_k,
                  int max_kb_per_item, int want_class_map, void* workspace, size_t ws_bytes,
                  hipStream_t stream);

/*
 * The forward ([FM] §3: FlashAttention-2 extended with the mask).
 *   out[i, h, :]     = sum_{j in A_i} softmax_j(scale * <q_i, k_j>) v_j
 *   softmax_lse[h, i] = ln sum_{j in A_i} exp(scale * <q_i, k_j>)
 * where A_i is the set of keys row i attends to (same sequence, not
 * masked).  A row with A_i empty gets out = 0 and lse = -inf.
 *
 * q, k, v, out: contiguous [N, H, D] of dtype (self-attention: one
 *   cu_seqlens for queries and keys; one mask for all heads).
 * softmax_lse: fp32 [H, N].  scale: finite, > 0.
 * block_q / block_k: 0 = defaults of fm_get_tile_config.
 * max_kb_per_item: < 0 auto (fm_auto_split), 0 = never split, else S.
 *   bf16 only; fp32 requires 0 or < 0 (treated as 0).
 * workspace: device, >= fm_workspace_layout(...).bytes for these sizes
 *   (class map not needed).  flags: FM_FLAG_*.
 * Without FM_FLAG_PLAN_READY the plan is built first.  Small bf16 problems
 * (see fm_fused_path) take the fused path: ONE attention launch in which
 * every workgroup derives its own work items (the chunks of the work list
 * above) from cu_seqlens and the mask vectors of its own q-tile row; no
 * plan is written to the workspace (its header then lists no items, so a
 * later FM_FLAG_PLAN_READY call on it runs nothing until fm_build_plan
 * fills it).  Split rows (S > 0) write partials that a second launch
 * combines in split order.  Results are deterministic: the same inputs
 * give the same bits, on either path.
 */
int fm_attn_fwd(const void* q, const void* k, const void* v, int dtype,
                int64_t N, int H, int D, const int32_t* cu_seqlens, int B,
                const int32_t* startend, int n_vec, int causal, float scale,
                void* out, float* softmax_lse, int block_q, int block_k,
                int max_kb_per_item, void* workspace, size_t ws_bytes,
                unsigned flags, hipStream_t stream);

/*
 * fm_attn_fwd with attention dropout on the probabilities ([FM] §3.4: the
 * op's dropout attribute and seed_offset input).  Pair (i, j) of head h in
 * a sequence starting at s is dropped when byte (j - s) & 15 of
 * Philox4x32-10 (Salmon et al., SC 2011) with key (seed mod 2^32,
 * seed >> 32) and counter (i, (j - s) >> 4, h, offset mod 2^32) is below
 * t = round(256 dropout_p) (little-endian bytes of the four words); kept
 * probabilities are scaled by 256 / (256 - t), so the effective dropout
 * probability is t / 256.  softmax_lse is the undropped normaliser.
 * 0 <= dropout_p < 1 (t = 0: no dropout, the same call as fm_attn_fwd);
 * bf16 only, not with FM_FLAG_NO_SKIP; always the planned path (never the
 * fused one).  The same (seed, offset) give the same mask in the backward.
 */
int fm_attn_fwd_dropout(const void* q, const void* k, const void* v, int dtype,
                        int64_t N, int H, int D, const int32_t* cu_seqlens, int B,
                        const int32_t* startend, int n_vec, int causal, float scale,
                        void* out, float* softmax_lse, int block_q, int block_k,
                        int max_kb_per_item, void* workspace, size_t ws_bytes,
                        unsigned flags, float dropout_p, uint64_t seed, uint64_t offset,
                        hipStream_t stream);

/* ---- allocation-free forward ------------------------------------------ */
/* Size of the library's own per-device array that fm_attn_fwd_noalloc uses
 * as its workspace: 64 MiB.                                                */
#define FM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * fm_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Its workspace is a fixed array
 * of FM_NOALLOC_SCRATCH_BYTES in the library's device code, one per GPU,
 * held until the process ends; the call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).  The caller still passes every
 * input and output.  Arguments, results and kernels are those of
 * fm_attn_fwd, except:
 *   - the problem's workspace, fm_workspace_layout(...).bytes for the tiles
 *     and split the call resolves to (fm_workspace_size for the defaults),
 *     must fit in FM_NOALLOC_SCRATCH_BYTES; larger problems are rejected
 *     with FM_E_WORKSPACE before anything is enqueued (the default calls of
 *     every workload up to 131072 tokens x 8 heads, and 32768 x 32, fit);
 *   - FM_FLAG_PLAN_READY is rejected (FM_E_INVAL): the array keeps only the
 *     last call's contents, so every call builds its own plan;
 *   - every call on one GPU shares that GPU's array: calls that can overlap
 *     on one GPU (unordered streams, several host threads) race on it and
 *     must be serialised by the caller.  Nothing in the array needs clearing
 *     between calls: each call writes every header word and plan entry it
 *     reads before reading it.
 * The array's device address is looked up (hipGetSymbolAddress) on the
 * first call made with a device current and kept per device.
 */
int fm_attn_fwd_noalloc(const void* q, const void* k, const void* v, int dtype,
                        int64_t N, int H, int D, const int32_t* cu_seqlens, int B,
                        const int32_t* startend, int n_vec, int causal, float scale,
                        void* out, float* softmax_lse, int block_q, int block_k,
                        int max_kb_per_item, unsigned flags, hipStream_t stream);

/*
 * 1 if fm_attn_fwd with these sizes and flags takes the fused one-launch
 * path (bf16, head_dim 128, default tiles, no FM_FLAG_NO_SKIP or
 * FM_FLAG_PLAN_READY, N <= 16384, B <= 255, at most 1024 q tiles and at
 * most 8 work items per workgroup of a launch with one workgroup per
 * compute unit, by the host's upper bounds); 0 if not; -1 on bad
 * arguments.  max_kb_per_item < 0 = auto.  Queries the current device's
 * CU count.
 */
int fm_fused_path(int64_t N, int B, int H, int head_dim, int dtype, int n_vec, int causal,
                  int max_kb_per_item, unsigned flags);

/*
 * Workspace bytes of fm_attn_bwd (0 on bad arguments): a status header,
 * kb_off [B+1] and extrema [ceil(N/64)+B][8] of the mask at block_k = 64,
 * Delta fp32 [H][N], and for small problems (fewer than 256 dK/dV
 * workgroups, (ceil(N/128) + B) * H < 256) fp32 partials of up to 8 chunks
 * per tile with their flags (any initial content; each call marks what it
 * writes with a fresh value).  Separate from the forward's workspace.
 */
size_t fm_bwd_workspace_size(int64_t N, int B, int H, int head_dim, int dtype);

/*
 * The backward ([FM] §3.4: the op takes q, k, v, the row intervals, out,
 * softmax_lse and the output gradient, and returns the gradients of q, k
 * and v; [FM] §4.2: exact, and deterministic because dq is not summed
 * with atomics).  With P_ij = exp(scale <q_i, k_j> - lse_i) on the allowed
 * pairs (0 elsewhere) and Delta_i = <dout_i, out_i>:
 *   dv_j = sum_i P_ij dout_i
 *   dS_ij = P_ij (<dout_i, v_j> - Delta_i)
 *   dq_i = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i
 * Fully masked tiles are skipped by the same block extrema and tile rules
 * as the forward (preprocessing runs inside this call).
 *
 * q, k, v, out, dout, dq, dk, dv: contiguous [N, H, D] bf16; D = 128 only
 *   (other dtypes / head_dims: FM_E_UNSUPPORTED).  out and softmax_lse
 *   (fp32 [H, N]) are the forward's outputs for the same inputs; rows with
 *   lse = -inf get dq = 0.  cu_seqlens, startend, n_vec, causal, scale as
 *   for fm_attn_fwd.  dq, dk, dv are written completely (zeros where no
 *   pair contributes) unless the device data is invalid (status word).
 * workspace: device, >= fm_bwd_workspace_size(...) bytes.
 * Launches: block extrema, Delta, dK/dV (one workgroup per 128-key tile
 * and head), dQ (one per 256-query tile and head); for small problems the
 * q tiles of a key tile and the key blocks of a query tile are cut into
 * chunks (separate workgroups, fp32 partials) and two more launches sum
 * them in chunk order.  The chunking depends on the sizes only: the same
 * inputs give the same bits on every run and device.  Everything runs on
 * `stream` (fm_attn_bwd_streams lets the dQ launches overlap the dK/dV ones
 * on a second stream of the caller's).
 */
int fm_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                const float* softmax_lse, int dtype, int64_t N, int H, int D,
                const int32_t* cu_seqlens, int B, const int32_t* startend, int n_vec, int causal,
                float scale, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                hipStream_t stream);

/*
 * fm_attn_bwd with the dQ launches on a second stream of the caller's
 * (same arguments and results, the same bits): after Delta the call
 * records `fork` on `stream`, makes `dq_stream` wait for it, enqueues the dQ
 * launches on `dq_stream` and the dK/dV launches on `stream`, then records
 * `join` on `dq_stream` and makes `stream` wait for it.  Everything the call
 * enqueues is thus ordered before whatever is enqueued on `stream`
 * afterwards, as with one stream, and on problems where neither launch
 * fills the chip the two run side by side.  The caller creates and owns
 * both streams and both events (hipEventDisableTiming is enough); calls that
 * share the events or dq_stream must be ordered by the caller.  dq_stream
 * must differ from `stream`; FM_E_INVAL otherwise or when an event is null.
 */
int fm_attn_bwd_streams(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* softmax_lse, int dtype, int64_t N, int H, int D,
                        const int32_t* cu_seqlens, int B, const int32_t* startend, int n_vec, int causal,
                        float scale, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                        hipStream_t stream, hipStream_t dq_stream, hipEvent_t fork, hipEvent_t join);

/*
 * fm_attn_bwd for a forward run with fm_attn_fwd_dropout: the same
 * (dropout_p, seed, offset) regenerate the forward's mask; with Z = keep *
 * 256 / (256 - t): dv = (P Z)^T dout, dS = P (Z (dout v^T) - Delta),
 * Delta_i = <dout_i, out_i>.
 */
int fm_attn_bwd_dropout(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* softmax_lse, int dtype, int64_t N, int H, int D,
                        const int32_t* cu_seqlens, int B, const int32_t* startend, int n_vec, int causal,
                        float scale, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                        float dropout_p, uint64_t seed, uint64_t offset, hipStream_t stream);

/*
 * fm_attn_bwd_dropout with the dQ launches on a second stream of the
 * caller's, exactly as fm_attn_bwd_streams does for fm_attn_bwd (same
 * arguments and results, the same bits; the same ordering, ownership and
 * FM_E_INVAL rules for dq_stream, fork and join).
 */
int fm_attn_bwd_dropout_streams(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* softmax_lse, int dtype, int64_t N, int H, int D,
                                const int32_t* cu_seqlens, int B, const int32_t* startend, int n_vec,
                                int causal, float scale, void* dq, void* dk, void* dv, void* workspace,
                                size_t ws_bytes, float dropout_p, uint64_t seed, uint64_t offset,
                                hipStream_t stream, hipStream_t dq_stream, hipEvent_t fork, hipEvent_t join);

/*
 * Rotary position embedding of packed q and k, in place, one launch for
 * both (Unsloth packing blog, fused QK RoPE section: one kernel for Q and
 * K, positions that restart in every packed sample, in place).  Row i of
 * sample b (cu_seqlens[b] <= i < cu_seqlens[b+1]) has position
 * p = i - cu_seqlens[b]; with x1 = x[:D/2], x2 = x[D/2:] of every head,
 *   x1 <- x1 cos[p] - x2 sin[p],   x2 <- x2 cos[p] + x1 sin[p]
 * i.e. x cos + rotate_half(x) sin; inverse != 0 negates sin (the
 * backward: the gradient rows go through the same call).
 *
 * q: [N, Hq, head_dim], k: [N, Hk, head_dim], contiguous, of dtype FM_BF16
 *   (fp32 arithmetic, rounded to bf16 once) or FM_F32; Hq or Hk may be 0
 *   (the pointer is then unused); base pointers 16-byte aligned.
 * head_dim: even, <= 512, and a multiple of 16 (bf16) or 8 (fp32).
 * cos_table, sin_table: fp32 [max_pos][head_dim / 2], 16-byte aligned.
 * cu_seqlens: int32 [B+1] device, valid as for fm_attn_fwd.
 * status: nullable int32 device word; rows whose position falls outside
 *   [0, max_pos) are left unchanged and FM_STATUS_POS is OR-ed into it.
 */
int fm_rope_qk(void* q, void* k, int dtype, int64_t N, int Hq, int Hk, int head_dim,
               const int32_t* cu_seqlens, int B, const float* cos_table, const float* sin_table,
               int64_t max_pos, int inverse, int32_t* status, hipStream_t stream);

/* Test helper: synchronises `stream` and copies the workspace's status
 * word to *status (0 = the device data was valid). */
int fm_read_status(const void* workspace, hipStream_t stream, int32_t* status);

#ifdef __cplusplus
}
#endif
#endif /* FM_API_H */
