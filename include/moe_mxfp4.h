/*
 * moe_mxfp4.h -- C ABI of the MI355X (gfx950) MXFP4 MoE expert layer.
 *
 * The operation (bjdmk.com.cn news page, section on the road to 1000
 * tokens/s; tilert.ai blog, section on the second leap; HyperAI transcript,
 * section on real-world case studies): the MoE expert layer of a
 * trillion-parameter model whose expert weights, and only those, are stored
 * as MXFP4 (4-bit E2M1 elements, one E8M0 power-of-two scale per 32
 * consecutive elements along the reduction dimension), run at the token
 * counts of a speculative-decode verify step (8 draft tokens + 1) or of a
 * prefill chunk.  Each token is routed to its top_k experts; each expert
 * computes SiLU(gate) * up and then the down projection; the expert outputs
 * are summed with the routing weights:
 *
 *   ids[t,:]  = the top_k experts by router logit (ties -> lower index),
 *               ordered by (logit desc, index asc)
 *   w[t,j]    = exp(l[t,ids[t,j]] - l[t,ids[t,0]]) / sum_i exp(l[t,ids[t,i]] - l[t,ids[t,0]])
 *   h         = SiLU(Wg[e] x_t) * (Wu[e] x_t),    SiLU(g) = g / (1 + exp(-g))
 *   out[t,:]  = sum_j w[t,j] * Wd[e_j] h_j
 *
 * The pages give no router or FFN formula; this is the standard softmax
 * top-k MoE with a SiLU-gated FFN, the plainest reading of "experts" they
 * describe.  Accumulation is fp32.  With bf16 activations the intermediate
 * h is carried to about 2^-12 relative (three MXFP8 terms on the matrix-core
 * paths, bf16 hi/lo pairs on the VALU path), so that the layer's error is
 * that of fp32 arithmetic between bf16 x and bf16 out; with MXFP8
 * activations (prefill) h is MXFP8.  out is bf16 rounded to nearest even.
 *
 * Data layout (all row-major, contiguous, caller-owned device memory):
 *   x              [T, H]        bf16 bit patterns
 *   router_logits  [T, E]        fp32 (any router bias already added)
 *   W_gate_up      [E, 2I, H/2]  uint8: two E2M1 codes per byte, element k of
 *                                a row in byte k/2, even k in the LOW nibble;
 *                                rows 0..I-1 are gate, rows I..2I-1 are up
 *   W_down         [E, H, I/2]   uint8, same packing
 *   scales->gate_up [E, 2I, H/32] uint8 E8M0 (value 2^(u-127), 0xFF = NaN)
 *   scales->down    [E, H, I/32]  uint8 E8M0
 *   out            [T, H]        bf16, fully overwritten
 * Every device pointer must be 16-byte aligned.  H and I must be multiples
 * of 128.
 *
 * Ownership: the caller owns every tensor and keeps it alive until the work
 * enqueued on `stream` has completed.  The library keeps no caller pointer.
 * It owns one workspace per device (routing arrays, h, per-assignment
 * outputs, the shared expert's rows, queue counters), allocated by
 * moe_mxfp4_init; the forward calls never allocate.
 *
 * Errors: arguments are validated synchronously before anything is
 * enqueued; a failed check returns a negative status, enqueues nothing and
 * leaves `out` untouched.  num_tokens == 0 is a valid no-op.  A failed HIP
 * call returns MOE_E_HIP; moe_mxfp4_status_string then also reports the
 * HIP error text.  Nothing aborts and no C++ exception crosses this ABI.
 * NaN inputs propagate and are not checked.
 *
 * Concurrency: one workspace per device, shared by every call on that
 * device; calls whose work overlaps on one device (e.g. on two streams)
 * race.  Calls on different devices are independent.  moe_mxfp4_init and
 * moe_mxfp4_finalize replace or free workspaces: no other host thread may
 * be inside a call of this library meanwhile (they synchronise the device
 * first, so work already enqueued is safe).
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_E_NULL (-1)      /* a required pointer is NULL */
#define MOE_E_SHAPE (-2)     /* a size is out of range or not a multiple it must be */
#define MOE_E_ALIGN (-3)     /* a device pointer is not 16-byte aligned */
#define MOE_E_TOPK (-4)      /* top_k outside 1..min(E, max_top_k) */
#define MOE_E_TOKENS (-5)    /* num_tokens above the max_tokens given to init */
#define MOE_E_NOT_INIT (-6)  /* moe_mxfp4_init was not called for the current device */
#define MOE_E_HIP (-7)       /* a HIP runtime call or kernel launch failed */
#define MOE_E_OPTION (-8)    /* an option value is not recognised */
#define MOE_E_LIMIT (-9)     /* a size exceeds the fixed limits of moe_mxfp4_forward_noalloc */
#define MOE_E_DTYPE (-10)    /* a tensor descriptor's element type is not the one required */

/* activation formats fed to the expert GEMMs */
#define MOE_ACT_BF16 0       /* x and h in bf16 (verify token counts) */
#define MOE_ACT_MXFP8 1      /* x and h encoded to MXFP8 E4M3 + E8M0 per 32 (prefill);
                                requires MOE_LAYOUT_TILES and runs on the scaled
                                FP4 x FP8 matrix cores (gemm_path AUTO or MFMA) */

/* GEMM path selection (moe_mxfp4_options.gemm_path) */
#define MOE_PATH_AUTO 0      /* the path that reads the given weight layout */
#define MOE_PATH_GEMV 1      /* VALU GEMV with DPP reductions (row-major weights) */
#define MOE_PATH_MFMA 2      /* bf16 matrix cores (weights in the MFMA tile layout) */

/* How the expert GEMMs are launched (moe_mxfp4_options.launch); the bf16
 * MFMA path only (the other paths always run split) */
#define MOE_LAUNCH_AUTO 0    /* the library's choice for the path */
#define MOE_LAUNCH_SPLIT 1   /* gate_up and down (+ combine) as two kernels */
#define MOE_LAUNCH_FUSED 2   /* one persistent kernel after the route: workgroups
                                dequeue gate_up units, then down units; a down unit
                                waits (bounded) for its item's gate_up units.  The
                                pages' persistent, gap-free execution (tilert.ai
                                blog, first leap; bjdmk.com.cn news page, road to
                                1000 tokens/s) applied to this layer */
#define MOE_LAUNCH_SELF_ROUTED 3 /* no routing pass: each GEMM workgroup ranks its
                                own expert for every token from router_logits,
                                and experts no token chose exit at once; h and
                                y rows are indexed by slot.  Layers of at most
                                16 tokens with T*E <= 4096 on the bf16 MFMA
                                path whose mean tokens per expert (T*top_k/E)
                                is below 8; other layers return MOE_E_OPTION.
                                AUTO takes it wherever it applies.  Same output
                                bits as SPLIT.  With NaN router logits the
                                result for that token is unspecified. */
#define MOE_LAUNCH_QUEUE 4   /* routed layers: after the route, the two GEMMs as
                                one launch of one workgroup per unit, each
                                dequeuing its unit from a counter (gate_up units,
                                then down units; a down unit waits, bounded, for
                                its item's gate_up units), then the combine.
                                Down units of finished items run beside the last
                                gate_up units, which the split launch's kernel
                                boundary leaves alone on a partly idle GPU.  Same
                                output bits as SPLIT.  AUTO takes it for layers
                                whose experts average at least 4 tokens
                                (T*top_k >= 4*E) and that have no shared expert;
                                with one, the shared expert's GEMMs run as kernels
                                of their own. */

/* Weight layouts (moe_mxfp4_options.weight_layout) */
#define MOE_LAYOUT_ROWS 0    /* row-major packed codes + scales, as described above */
#define MOE_LAYOUT_TILES 1   /* the MFMA tile layout written by moe_mxfp4_prepack */

/* The two E8M0 scale tensors (device pointers). */
typedef struct moe_mxfp4_scales {
    const uint8_t* gate_up; /* [E, 2I, H/32] */
    const uint8_t* down;    /* [E, H, I/32]  */
} moe_mxfp4_scales;

/* Element types of moe_tensor */
#define MOE_DT_BF16 1        /* bfloat16 bit patterns (2 bytes) */
#define MOE_DT_F32 2         /* float32 */
#define MOE_DT_U8 3          /* uint8 (packed codes, E8M0 scales) */
#define MOE_DT_I32 4         /* int32 */

/* A caller tensor as moe_mxfp4_forward_t sees it: device pointer, element
 * type (MOE_DT_*), rank 1..4 and extents; row-major and contiguous.  The
 * library reads the descriptor during the call only. */
typedef struct moe_tensor {
    void* data;
    int64_t shape[4];
    int32_t ndim;
    int32_t dtype;
} moe_tensor;

/* Options of moe_mxfp4_forward_ex.  Zero-initialised = moe_mxfp4_forward.
 * The optional outputs are device buffers the call fills (NULL to skip):
 * the routing result and, with MOE_ACT_MXFP8, the MXFP8 encoding of x. */
typedef struct moe_mxfp4_options {
    int32_t act_format;  /* MOE_ACT_BF16 or MOE_ACT_MXFP8 (E4M3 elements, ties to
                            even, saturating; scale 2^(floor(log2 amax) - 8) per 32
                            along K, the weights' rule with the E4M3 range: OCP MX
                            specification) */
    int32_t gemm_path;   /* MOE_PATH_* */
    int32_t* ids;        /* [T, top_k] expert per slot, slot order (logit desc, index asc) */
    float* weights;      /* [T, top_k] renormalised softmax weights */
    int32_t* counts;     /* [E] slots per expert */
    int32_t* offsets;    /* [E+1] exclusive prefix sum of counts */
    int32_t* sorted;     /* [T*top_k] slots t*top_k+j grouped by expert, ascending inside one */
    uint8_t* x_codes;    /* [T, H] E4M3 codes of x (MOE_ACT_MXFP8 only) */
    uint8_t* x_scales;   /* [T, H/32] E8M0 scales of x (MOE_ACT_MXFP8 only) */
    /* Optional hipEvent_t handles recorded on `stream` at the stage
     * boundaries: [0] before routing, [1] after routing (right after [0]
     * in a self-routed launch that returns no routing output; with
     * MOE_ACT_MXFP8, after the encoding of x), [2] after the
     * gate_up GEMM (after the single expert kernel in a fused launch),
     * [3] after the down GEMM and the combine.  Only the
     * first num_events (<= 4) are recorded; used to time the kernels. */
    void* const* events;
    int32_t num_events;
    /* MOE_LAYOUT_ROWS (0, the default) or MOE_LAYOUT_TILES: the layout of
     * W_gate_up, W_down and the scales.  ROWS runs the GEMV path, TILES the
     * MFMA path; asking for the other path returns MOE_E_OPTION. */
    int32_t weight_layout;
    /* MOE_LAUNCH_AUTO, _SPLIT, _FUSED, _SELF_ROUTED or _QUEUE (see above) */
    int32_t launch;
    /* Optional [1] int32 device output: nonzero if, in the fused or queue
     * launch, a down unit gave up waiting for its gate_up units (it then
     * went on, and out is not to be trusted).  The waits are bounded at
     * about four million polls; a correct launch never reaches that.  0 in
     * split launches. */
    int32_t* wait_error;
    /* Optional [E, H] bf16 router weight (device, row-major, 16-byte
     * aligned).  When set, the layer computes its router logits itself,
     * logits[t, e] = sum_h x[t, h] * W_router[e, h] -- bf16 products summed
     * in fp32 on the matrix cores, split over K for small T with the
     * partial sums added in a fixed order, so the same inputs give the same
     * bits -- and routes on them; router_logits is then ignored (it may be
     * NULL).  The pages keep routing at the model's original precision
     * (sandbot 1000-TPS post, technical-breakdown section). */
    const void* router_weight;
    /* Optional [T, E] fp32 device output: the logits the layer routed on
     * (the computed ones with router_weight, else a copy of router_logits). */
    float* logits_out;
    /* Optional shared expert, all four set or all NULL (else MOE_E_NULL),
     * each 16-byte aligned.  The pages store only the MoE experts in 4 bits
     * and keep the rest of the model at FP8 (bjdmk.com.cn news page,
     * co-design section; yifor-blog digest, selective FP4 quantisation); a
     * shared expert is read as one more SiLU-gated FFN of the routed
     * experts' shape (gate/up [2I, H], down [H, I]) whose weights are MXFP8
     * -- E4M3 codes, one E8M0 scale per 32 along K -- applied to every token
     * with weight 1:
     *   out[t,:] += Ws_down ( SiLU(Ws_gate x_t) * (Ws_up x_t) )
     * added in fp32 after the k routed terms, before the rounding to bf16.
     * Its h follows the activation format (bf16, or MXFP8 with
     * MOE_ACT_MXFP8).  The matrices are in the MXFP8 tile layout written by
     * moe_mxfp8_prepack: shared_gate_up / shared_gate_up_scales from
     * [2I, H] with gate_up_pairs = 1, shared_down / shared_down_scales from
     * [H, I] with gate_up_pairs = 0.  Works with every path and launch. */
    const uint8_t* shared_gate_up;
    const uint8_t* shared_gate_up_scales;
    const uint8_t* shared_down;
    const uint8_t* shared_down_scales;
    /* Optional copies of h on the MOE_ACT_MXFP8 path (NULL: not copied;
     * ignored on the other paths): h_codes [T*k, I] E4M3 codes and h_scales
     * [T*k, I/32] E8M0 scales of the routed assignments, row p holding the
     * assignment at position p of the expert-sorted order (`sorted`).  They
     * expose the encoding decision of h, taken on fp32 values, for tests. */
    uint8_t* h_codes;
    uint8_t* h_scales;
} moe_mxfp4_options;

/* Allocate the workspace on the current device for layers with at most
 * max_tokens tokens, exactly num_experts experts of hidden size `hidden`
 * and intermediate size `inter`, and top_k <= max_top_k.  Calling it again
 * on the same device replaces the previous workspace.  Sizes: max_tokens in
 * 1..2^20, num_experts in 1..1024, hidden and inter multiples of 128 in
 * 128..16384, max_top_k in 1..min(32, num_experts).
 * Returns MOE_OK, MOE_E_SHAPE, MOE_E_TOPK or MOE_E_HIP (allocation failed). */
int moe_mxfp4_init(int64_t max_tokens, int64_t num_experts, int64_t hidden,
                   int64_t inter, int32_t max_top_k);

/* Release the workspaces of every device (after synchronising them). */
void moe_mxfp4_finalize(void);

/* The layer with bf16 activations on row-major weights (the VALU GEMV
 * path), enqueued on `stream` (a hipStream_t; NULL = the null stream).
 * x, router_logits and out hold num_tokens rows.  Returns without
 * synchronising.  The matrix-core path, the faster one at every layer
 * size, reads the weights in the MFMA tile layout: rearrange them once at
 * weight load with moe_mxfp4_prepack (same bytes) and call
 * moe_mxfp4_forward_ex with weight_layout = MOE_LAYOUT_TILES (or
 * moe_mxfp4_forward_t). */
int moe_mxfp4_forward(const void* x, const float* router_logits, int64_t num_tokens,
                      int32_t top_k, const uint8_t* W_gate_up, const uint8_t* W_down,
                      const moe_mxfp4_scales* scales, void* out, void* stream);

/* moe_mxfp4_forward with options (activation format, path, debug outputs).
 * opt == NULL is the same as moe_mxfp4_forward. */
int moe_mxfp4_forward_ex(const void* x, const float* router_logits, int64_t num_tokens,
                         int32_t top_k, const uint8_t* W_gate_up, const uint8_t* W_down,
                         const moe_mxfp4_scales* scales, void* out, void* stream,
                         const moe_mxfp4_options* opt);

/* moe_mxfp4_forward_ex with every tensor described (element type, rank,
 * extents), for C callers that want the checks a framework binding makes.
 * Before anything else it requires, with T = x->shape[0] and H, E, I read
 * from the descriptors themselves:
 *   x              rank 2, BF16, [T, H]
 *   router_logits  rank 2, F32,  [T, E]   (NULL, or data NULL, when
 *                                          opt->router_weight is set)
 *   W_gate_up      rank 3, U8,   [E, 2I, H/2]
 *   W_down         rank 3, U8,   [E, H, I/2]
 *   scales[0]      rank 3, U8,   [E, 2I, H/32]
 *   scales[1]      rank 3, U8,   [E, H, I/32]
 *   out            rank 2, BF16, [T, H]
 * (the tile layout of opt->weight_layout = MOE_LAYOUT_TILES is stored in
 * tensors of the same shapes and byte counts), H even and I even, and, if
 * the current device has a workspace, E, H and I equal to those given to
 * moe_mxfp4_init.  A descriptor or data pointer that is NULL returns
 * MOE_E_NULL, a wrong element type MOE_E_DTYPE, a wrong rank or extent
 * MOE_E_SHAPE -- nothing is enqueued and out is untouched.  Then
 * it is moe_mxfp4_forward_ex on those pointers with num_tokens = T, whose
 * own checks (against the sizes given to moe_mxfp4_init, alignment,
 * options) follow.  scales points at two descriptors. */
int moe_mxfp4_forward_t(const moe_tensor* x, const moe_tensor* router_logits, int32_t top_k,
                        const moe_tensor* W_gate_up, const moe_tensor* W_down,
                        const moe_tensor* scales, const moe_tensor* out, void* stream,
                        const moe_mxfp4_options* opt);

/* Encode a float32 matrix w [rows, cols] to MXFP4 along cols (the block
 * rule of the weights: scale 2^(floor(log2 amax) - 2) with the exponent
 * clamped to [-127, 127], amax == 0 -> scale code 0, elements rounded to the
 * nearest E2M1 value with ties to the even code and saturating at 6; a block
 * with a non-finite element gets scale 0xFF and element codes 0).
 * packed [rows, cols/2], scales [rows, cols/32], all on the current device,
 * enqueued on `stream`.  cols must be a multiple of 32, w 16-byte aligned,
 * and packed 16-byte aligned when cols is a multiple of 32 (always). */
int moe_mxfp4_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* packed,
                       uint8_t* scales, void* stream);

/* Rearrange num_matrices MXFP4 matrices [rows, cols] (packed [.., rows,
 * cols/2], scales [.., rows, cols/32], row-major as above) into the MFMA
 * tile layout that forward_ex reads with weight_layout = MOE_LAYOUT_TILES.
 * Same byte counts: tiles holds rows*cols/2 and tile_scales rows*cols/32
 * bytes per matrix.  Layout: each 64-row quad (four 16-row groups) and
 * 128-column chunk (four MX blocks) becomes 4 KB of codes ordered
 * [group][lane][16 bytes] (lane = r + 16 g: block g of row r) followed, in
 * tile_scales, by 256 scale bytes ordered [lane][group].  gate_up_pairs != 0
 * (for W_gate_up, rows = 2I) makes quad q hold gate rows 32q..32q+31 as
 * groups 0, 1 and up rows I+32q..I+32q+31 as groups 2, 3; otherwise quad q
 * holds rows 64q..64q+63.  rows % 64 == 0, cols % 128 == 0; packed and tiles
 * 16-byte aligned, tile_scales 4-byte aligned.  A one-time step at weight
 * load (not part of a forward call).  Enqueued on `stream`. */
int moe_mxfp4_prepack(const uint8_t* packed, const uint8_t* scales, int64_t num_matrices,
                      int64_t rows, int64_t cols, int32_t gate_up_pairs, uint8_t* tiles,
                      uint8_t* tile_scales, void* stream);

/* Encode a float32 matrix w [rows, cols] to MXFP8 along cols (the 8-bit
 * weights beside the experts, e.g. the shared expert): E4M3 elements
 * (OCP "FN": no infinities, 0x7F/0xFF NaN), one E8M0 scale per 32, the
 * OCP MX block rule -- scale 2^(floor(log2 amax) - 8) with the exponent
 * clamped to [-127, 127], amax == 0 -> scale code 0, elements rounded to
 * the nearest E4M3 value with ties to the even code and saturating at 448;
 * a block with a non-finite element gets scale 0xFF and element codes 0.
 * codes [rows, cols] (one byte per element), scales [rows, cols/32], on the
 * current device, enqueued on `stream`.  cols % 32 == 0; w and codes
 * 16-byte aligned.  Returns MOE_OK, MOE_E_SHAPE, MOE_E_NULL, MOE_E_ALIGN or
 * MOE_E_HIP. */
int moe_mxfp8_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes,
                       uint8_t* scales, void* stream);

/* moe_mxfp4_prepack for MXFP8 matrices (codes [.., rows, cols], one byte
 * per element; scales [.., rows, cols/32]): the same quads, chunks, lanes,
 * gate/up pairing and scale order, with each 16-row group's codes split in
 * two halves -- [group][half h][lane][16 bytes], lane r + 16 g holding
 * bytes 16h..16h+15 of block g of row r -- so tiles holds rows*cols bytes
 * per matrix (8 KB per quad and chunk) and tile_scales rows*cols/32.  Same
 * constraints and status codes as moe_mxfp4_prepack. */
int moe_mxfp8_prepack(const uint8_t* codes, const uint8_t* scales, int64_t num_matrices,
                      int64_t rows, int64_t cols, int32_t gate_up_pairs, uint8_t* tiles,
                      uint8_t* tile_scales, void* stream);

/* The layer for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * needs no moe_mxfp4_init and calls no allocating routine: its working set
 * (per-expert slot lists, routing weights, h, the per-assignment outputs)
 * lives in one fixed device array of the library, about 5.6 MB, which each
 * device holds from its first call until the process ends.  It runs the
 * self-routed layer (the launches of moe_mxfp4_forward_ex with
 * MOE_LAUNCH_SELF_ROUTED, bf16 activations, weights in the MFMA tile layout
 * of moe_mxfp4_prepack, no shared expert), with the same output bits, for
 * layers of at most 16 tokens, 256 experts, top_k 8, hidden 8192 and inter
 * 4096 (multiples of 128) with num_tokens * num_experts <= 4096 and
 * num_tokens * top_k < 8 * num_experts; larger ones return MOE_E_LIMIT
 * (moe_mxfp4_status_string names the limits), bad pointers, sizes or
 * top_k the codes of moe_mxfp4_forward, all before anything is enqueued.
 * Arguments as moe_mxfp4_forward, plus the layer's num_experts, hidden and
 * inter sizes (which the workspace gives moe_mxfp4_forward); x,
 * router_logits and out hold num_tokens rows.  Nothing in the array needs
 * clearing between calls (every piece is written before it is read), but
 * all calls on one device share it: calls whose work overlaps on one device
 * (two streams, or two host threads) race.  The first call on a device
 * takes the array's device address (hipGetSymbolAddress) and may not be
 * captured into a graph; later calls may. */
int moe_mxfp4_forward_noalloc(const void* x, const float* router_logits, int64_t num_tokens,
                              int32_t top_k, int64_t num_experts, int64_t hidden, int64_t inter,
                              const uint8_t* W_gate_up, const uint8_t* W_down,
                              const moe_mxfp4_scales* scales, void* out, void* stream);

/* Static text of a status code; for MOE_E_HIP, the text of the last HIP
 * error seen by the calling thread. */
const char* moe_mxfp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
