// moe_internal.h -- internal declarations shared by the library's HIP sources.
// Not installed and not part of the C ABI (include/moe_mxfp4.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- tuning
constexpr int kWave = 64;
constexpr int kGemvThreads = 256;       // 4 waves
constexpr int kGemvLanesPerRow = 16;    // one DPP row of lanes shares a matrix row
constexpr int kGemvSlots = kGemvThreads / kGemvLanesPerRow;  // row slots per workgroup
constexpr int kGemvMaxTok = 4;          // tokens held per GEMV pass
constexpr int kGemvUnroll = 4;          // blocks per lane per loop step
// row units per work item: a unit is a (gate, up) row pair for gate_up and
// two adjacent rows for down
constexpr int kGateUpUnits = 32;
constexpr int kDownUnits = 64;
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;
constexpr int kRouteSlotBlock = 256;  // slots per block of the multi-block routing sort

// Counters that workgroups of a running kernel poll sit one per 128-byte
// line, kLineInts words apart: hundreds of pollers on one line keep one
// memory channel busy, and every workgroup's weight stream, which crosses
// all channels, then runs at that channel's pace (measured on the 9-token,
// 64-expert single launch: down units 9 -> 35 us once the first
// workgroups polled a shared counter).  The single launches' combine
// barrier: the unit that completes the queue raises kGoLines flags
// kGoStride words apart, and workgroup b polls flag b % kGoLines.
constexpr int kLineInts = 32;
constexpr int kGoLines = 64, kGoStride = 64;

// The self-routed single launch's counters (the int32 words at `flags`):
// list ready of expert e (index E unused) at e * kLineInts, gate_up units
// done of expert e (index E: the shared expert) at (E + 1 + e) * kLineInts,
// then one line of SelfFlags words, then the go flags.
enum SelfFlags : int {
    kSelfNext = 0,      // next unit to dequeue
    kSelfDone = 1,      // units run (the combine waits for all of them)
    kSelfExits = 2,     // workgroups done with the combine
    kSelfError = 3,     // a wait gave up (this launch)
    kSelfErrorOut = 4,  // ... as left by the last launch, for the caller
};
__host__ __device__ constexpr int64_t self_misc_word(int E) { return (int64_t)2 * (E + 1) * kLineInts; }
__host__ __device__ constexpr int64_t self_go_word(int E) { return self_misc_word(E) + kGoStride; }
__host__ __device__ constexpr int64_t self_flag_words(int E) {
    return self_go_word(E) + (int64_t)kGoLines * kGoStride;
}

// words of Workspace::queue (the single-launch expert layer of routed
// items): a line of these, then the go flags from kQueueGo
enum Queue : int {
    kQueueNext = 0,    // next unit to dequeue
    kQueueError = 1,   // nonzero: a wait gave up
    kQueueDone = 2,    // units run (the combine waits for all of them)
    kQueueHead = 4,
    kQueueGo = kGoStride,
    kQueueWords = kQueueGo + kGoLines * kGoStride,
};

// meta[] words in the workspace
enum Meta : int {
    kMetaNumGemv = 0,   // active experts on the GEMV path
    kMetaNumMfma = 1,   // active experts on the MFMA path
    kMetaNumMfmaItems = 2,  // (expert, token group) items of the MFMA path
    kMetaWords = 16,
};

// columns of the output covered by one down-projection tile of the GEMV
// path; also the width of its combine tile
constexpr int kColTile = 2 * kDownUnits;

// MFMA path: an item is one expert and up to kMfmaTok of its tokens; a
// gate_up tile is kMfmaRows gate rows with their up rows, a down tile is
// kMfmaDownRows output rows (also its combine tile width); the 4 waves of a
// workgroup split K.
constexpr int kMfmaTok = 16;      // tokens per MFMA column tile
constexpr int kMfmaItemTok = 64;  // tokens per wide item of the bf16 MFMA path
// The routed launch uses wide items (four quads per workgroup, the item's
// activations staged in LDS) when the layer averages at least this many
// tokens per expert (T * top_k >= kMfmaWideMeanTok * E)
constexpr int kMfmaWideMeanTok = 4;
// MXFP8 (prefill) path: items of up to kMx8Tok tokens (eight 16-token MFMA
// column tiles), weights in the same tile layout.
constexpr int kMx8Tok = 128;
// Self-routed layer (no routing pass): up to kSelfMaxTok tokens (one MFMA
// column tile per expert), whose logits [T, E] (T*E <= kSelfMaxPairs) the
// weight pass holds in LDS.
constexpr int kSelfMaxTok = 16;
constexpr int kSelfMaxPairs = 4096;
// ... and averaging fewer than kSelfMaxMeanTok tokens per expert
constexpr int kSelfMaxMeanTok = 8;
// Per-expert slot list of the self-routed layer: m, then the slots t*k + j
// of its m tokens in ascending token order (one 128-byte line per expert).
// Layers whose two GEMM grids hold at least kSelfListUnits workgroups
// (E * (I/32 + H/128)) write the lists in a pre-pass (one wave per expert)
// and the GEMM workgroups read them; smaller layers rank in every GEMM
// workgroup (no pre-pass launch).
constexpr int kSlotListInts = 32;
constexpr int kSelfListUnits = 2048;

// Bytes per row of h3s (h's four E8M0 scale bytes per 32-column block, the
// three terms' and a pad: I/8 bytes), rounded up to whole 128-byte cache
// lines.  In a single-launch layer one line of narrower rows would hold
// rows of items of different experts, finished at different times; a down
// unit's plain load of its own row would bring another row's unwritten
// bytes into its CU's and XCD's caches, where a later unit of that other
// expert could hit them.  With whole lines per row every line belongs to
// one item and is first read once that item's gate_up units are done.  (The
// code rows, 3I bytes with I a multiple of 128, are whole lines already.)
__host__ __device__ constexpr int h3s_stride(int I) { return (I / 8 + 127) / 128 * 128; }
// router GEMM: K is split (at most kRouterMaxSplit ways, over tiles of 16
// tokens x 16 experts) only for layers of fewer than kRouterWaves / 2 tiles
// of 16 tokens x 64 experts, so then T*E < kRouterWaves * 512 and there are
// fewer than kRouterWaves * 2 split tiles
constexpr int kRouterWaves = 256;
constexpr int kRouterMaxSplit = 16;
constexpr int kMfmaRows = 16;
constexpr int kMfmaDownRows = 32;
constexpr int kMfmaThreads = 256;

// One device's workspace, owned by the library.
struct Workspace {
    int device = -1;
    int64_t max_tokens = 0, E = 0, H = 0, I = 0;
    int kmax = 0;
    void* base = nullptr;       // single allocation holding everything below
    size_t bytes = 0;
    int32_t* ids = nullptr;     // [Tmax*kmax]
    float* wts = nullptr;       // [Tmax*kmax]
    int32_t* counts = nullptr;  // [E]
    int32_t* offsets = nullptr; // [E+1]
    int32_t* sorted = nullptr;  // [Tmax*kmax]
    int32_t* pos = nullptr;     // [Tmax*kmax]
    int32_t* gemv_list = nullptr;  // [E] active experts routed to the GEMV path
    int32_t* mfma_list = nullptr;  // [E] active experts routed to the MFMA path
    int4* mfma_items = nullptr;    // [E + Tmax*kmax/kMfmaTok] MFMA items: (expert, first sorted row, tokens, 0)
    int32_t* meta = nullptr;       // [kMetaWords]
    int32_t* tile_done = nullptr;  // [Tmax * H/kMfmaDownRows] finished down tiles per (token, column tile)
    int32_t* bhist = nullptr;      // [ceil(Tmax*kmax/kRouteSlotBlock) * E] per-block expert histograms
    int32_t* queue = nullptr;      // [kQueueWords] single-launch layer: Queue words, go flags
    int32_t* gu_done = nullptr;    // [max_items * kLineInts] finished gate_up units per MFMA item, one line each
    int32_t* slot_lists = nullptr; // [E * kSlotListInts] self-routed layer: per-expert slot lists
    int32_t* flags = nullptr;      // [self_flag_words(E)] the self-routed single launch (SelfFlags)
    float* logits = nullptr;       // [Tmax * E] logits computed from a router weight
    float* router_partial = nullptr;  // [kRouterMaxSplit * min(Tmax*E, kRouterWaves*512)] split-K partials
    int32_t* router_cnt = nullptr;    // [2 * kRouterWaves] finished splits per tile (split-K only)
    int max_items = 0;             // entries of mfma_items / gu_done
    int col_tiles = 0;             // H / kColTile
    // h and y: Tmax*kmax rows of the routed assignments (sorted order, or
    // slot order in a self-routed layer), then Tmax rows of the shared expert
    // h: the routed rows of the GEMV path as bf16 hi/lo pairs [rows, 2I];
    // h3q / h3s: h of the matrix-core paths (and of the shared expert on
    // every bf16 path) as three MXFP8 terms, codes [rows, 3I] and scales
    // [rows, h3s_stride(I)] (device_common.h, store_h3)
    uint16_t* h = nullptr;
    uint8_t* h3q = nullptr;
    uint8_t* h3s = nullptr;
    float* y = nullptr;         // [Tmax*(kmax+1), H] fp32
    uint8_t* x_codes = nullptr;   // [Tmax, H] E4M3 codes of x (MXFP8 path)
    uint8_t* x_scales = nullptr;  // [Tmax, H/32] E8M0
    uint8_t* h_codes = nullptr;   // [Tmax*(kmax+1), I] E4M3 codes of h, rows as h
    uint8_t* h_scales = nullptr;  // [Tmax*(kmax+1), I/32] E8M0
};

// Arguments common to the expert GEMM kernels.
struct GemmArgs {
    const uint16_t* x;          // [T, H] bf16
    const uint8_t* wgu;         // [E, 2I, H/2]
    const uint8_t* sgu;         // [E, 2I, H/32]
    const uint8_t* wdn;         // [E, H, I/2]
    const uint8_t* sdn;         // [E, H, I/32]
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* sorted;
    const int32_t* list;        // active experts for this path
    const int32_t* meta;
    int list_meta;              // which meta word holds the list length
    uint16_t* h;                // GEMV path's routed rows: [rows, 2I] bf16 hi/lo pairs (gemv.hip)
    uint8_t* h3q;               // matrix-core paths and the shared expert: [rows, 3I] codes of
    uint8_t* h3s;               // h's three MXFP8 terms, [rows, h3s_stride(I)] their scales (store_h3)
    float* y;
    int T, H, I, k;
    // combine state
    int32_t* tile_done;         // [T * tiles] experts done per (token, column tile)
    const int4* items;          // MFMA path: (expert, first sorted row, tokens, 0) per item
    // MXFP8 path
    const uint8_t* xq;          // [T, H] E4M3 codes of x
    const uint8_t* xs;          // [T, H/32] E8M0 scales of x
    uint8_t* hq;                // [T*k, I] E4M3 codes of h (sorted rows)
    uint8_t* hs;                // [T*k, I/32] E8M0 scales of h
    const float* wts;           // [T*k] routing weights
    const int32_t* pos;         // [T*k] slot -> row of y; null: row = slot (self-routed layer)
    uint16_t* out;              // [T, H] bf16
    int col_tiles;
    // single-launch layer (route, then one kernel for gate_up + down + combine)
    int32_t* queue;             // [kQueueWords], counters and go flags zeroed by the route
    int32_t* gu_done;           // [max items * kLineInts] finished gate_up units of item i at i * kLineInts, zeroed by the route
    // self-routed layer (no routing pass): each GEMM workgroup ranks its own
    // expert for every token from the router logits
    const float* logits;        // [T, E] fp32
    int E;
    int32_t* route_ids;         // [T*k] written by the weight pass (expert per slot)
    float* route_wts;           // [T*k] written by the weight pass (= wts)
    int32_t* slot_lists;        // [E * kSlotListInts] per-expert slot lists
    // optional shared expert: MXFP8 weights in the tile layout (null: none),
    // applied to every token; its h and y rows are sh_row0 + t (sh_row0 = T*k)
    const uint8_t* sh_wgu;      // [2I, H] as gate/up quads
    const uint8_t* sh_sgu;
    const uint8_t* sh_wdn;      // [H, I]
    const uint8_t* sh_sdn;
    int sh_row0;
};

// ---------------------------------------------------------------- launchers
// Workgroups of `kernel` (block threads, static LDS only) that fit on the
// current device at once: occupancy per CU x CUs.
hipError_t resident_grid(const void* kernel, int block, int* grid);

// Each returns the hipError_t of its launch.
// item_tok: tokens per MFMA item (kMfmaItemTok for bf16, kMx8Tok for MXFP8).
hipError_t launch_route(const float* logits, int T, int E, int k, const Workspace& ws,
                        int gemv_max_tokens, int path, int item_tok, hipStream_t stream);
// GEMV path: gate_up (+ SiLU * up -> h), then down (-> y) whose last
// finisher per (token, column tile) also combines that tile of the output.
// max_active bounds the number of routed experts (grids are sized by it).
hipError_t launch_gemv_gate_up(const GemmArgs& a, int max_active, hipStream_t stream);
hipError_t launch_gemv_down(const GemmArgs& a, int max_active, hipStream_t stream);
// MFMA path: items from the route's MFMA item list; max_items bounds their
// number.  Items of at most kMfmaTok tokens (split-K kernels) or, for the
// wide kernels, up to kMfmaItemTok tokens.  The down kernels only write y;
// launch_combine forms out.
hipError_t launch_mfma_gate_up(const GemmArgs& a, int max_items, hipStream_t stream);
hipError_t launch_mfma_down(const GemmArgs& a, int max_items, hipStream_t stream);
// Self-routed layer of at most kSelfMaxTok tokens (route_rank.h): no
// sorting pass.  gate_up runs one workgroup per (expert, row tile), each of
// which finds its expert's tokens (ranked from the logits, or from the slot
// lists; experts with none exit), plus one workgroup that writes the
// routing weights; down runs one per (expert, column tile pair).  h and y
// rows are indexed by slot t*k + j, so launch_combine runs with pos = null.
// lists: the GEMM workgroups read the slot lists written by
// launch_slot_lists instead of ranking their experts themselves.
// logits [T, E] fp32 = x [T, H] bf16 . wr [E, H]^T bf16 (router.hip)
hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* wr, int T, int E, int H,
                              const Workspace& ws, float* logits, hipStream_t stream);
hipError_t launch_slot_lists(const GemmArgs& a, hipStream_t stream);
hipError_t launch_self_gate_up(const GemmArgs& a, bool lists, hipStream_t stream);
hipError_t launch_self_down(const GemmArgs& a, bool lists, hipStream_t stream);
hipError_t launch_wide_gate_up(const GemmArgs& a, int max_items, hipStream_t stream);
hipError_t launch_wide_down(const GemmArgs& a, int max_items, hipStream_t stream);
// out = the weighted sum of the k per-assignment rows of y per token, in
// slot order (after a down kernel of the split launch); the row of slot s
// is pos[s], or s itself when pos is null.
hipError_t launch_combine(const GemmArgs& a, hipStream_t stream);
// The same two GEMMs (and the combine) in one persistent launch: workgroups
// dequeue gate_up units (item, row tile), then down units, each of which
// waits (bounded) until every gate_up unit of its item has published h.
// Needs the queue words and gu_done zeroed (the route does it).
hipError_t launch_mfma_fused(const GemmArgs& a, int max_items, hipStream_t stream);
// The whole self-routed layer (routing weights, slot lists, gate_up, down
// and the combine) in one persistent launch; a.slot_lists and the flags
// (zero at the first launch; the launch leaves them zero) from the
// workspace.
hipError_t launch_self_fused(const GemmArgs& a, int32_t* flags, hipStream_t stream);
hipError_t launch_wide_fused(const GemmArgs& a, int max_items, hipStream_t stream);
// The two GEMMs as one launch of one workgroup per unit (gate_up units,
// then down units that wait, bounded, for their item's gate_up units),
// each dequeued from queue[kQueueNext]; launch_combine forms out after it.
// Needs the queue words and gu_done zeroed (the route does it).
hipError_t launch_mfma_queue(const GemmArgs& a, int max_items, hipStream_t stream);
hipError_t launch_wide_queue(const GemmArgs& a, int max_items, hipStream_t stream);
// MXFP8 (prefill) path: encode x per token along H, then the scaled
// FP4 x FP8 matrix-core GEMMs (gate_up encodes h to MXFP8 in its epilogue;
// down writes y, launch_combine forms out).
hipError_t launch_quantize_x_mxfp8(const uint16_t* x, int T, int H, uint8_t* codes,
                                   uint8_t* scales, hipStream_t stream);
hipError_t launch_mx8_gate_up(const GemmArgs& a, int max_items, hipStream_t stream);
hipError_t launch_mx8_down(const GemmArgs& a, int max_items, hipStream_t stream);
hipError_t launch_quantize_mxfp4(const float* w, int64_t rows, int64_t cols, uint8_t* packed,
                                 uint8_t* scales, hipStream_t stream);
hipError_t launch_quantize_mxfp8(const float* w, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);
// The shared expert (MXFP8 weights) over all T tokens, on the bf16 matrix
// cores, as launches of its own (the VALU path and the single-launch layer;
// the other GEMM kernels run its blocks ahead of their routed ones when
// sh_wgu is set).  gate_up writes h rows sh_row0 + t, down writes y rows
// sh_row0 + t; the combine adds them with weight 1.
hipError_t launch_shared_gate_up(const GemmArgs& a, hipStream_t stream);
hipError_t launch_shared_down(const GemmArgs& a, hipStream_t stream);

}  // namespace moe
