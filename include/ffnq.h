/*
 * ffnq.h -- C ABI of libffnq: the quantized-weight gated FFN of a transformer
 * layer and the MoE routed half that reuses it, for AMD Instinct MI355X (gfx950).
 *
 * Source of the method (docs.rs pages of the `turbospark-runtime` crate):
 *   [gemma4/shared_expert.rs]  `encode_shared_expert_branch` and
 *                              `encode_shared_expert_branch_batched`
 *   [qwen/moe_batch.rs]        module doc and `encode_qwen_layer_moe_batched`
 *   [llama/dense.rs]           module doc (the FFN equation) and
 *                              `encode_llama_layer_dense`
 *
 * General conventions (every entry point):
 *   - Return value: FFNQ_OK (0) or a negative FFNQ_ERR_* code.  Every argument
 *     check runs on the host before anything is enqueued, so an INVALID,
 *     UNSUPPORTED, CAPACITY or WORKSPACE return enqueues nothing.  FFNQ_ERR_HIP
 *     means a launch failed; kernels of the same call enqueued before the
 *     failing one may already be on the stream.
 *   - Pointers named "device" are HIP device pointers; the ffnq_qmat / ffnq_ffn
 *     structs themselves live in host memory and are read during the call only.
 *   - Every device pointer must be 16-byte aligned (128-bit loads).  Tensors are
 *     contiguous and row-major, with no strides.
 *   - Ownership: the caller allocates every buffer.  The library allocates,
 *     frees and synchronises nothing and keeps no state between calls (two
 *     exceptions: ffnq_set_phase_events, a per-thread timing switch that never
 *     changes a result, and the per-GPU scratch array of ffnq_dense_noalloc,
 *     a static device array rather than an allocation).  Calls
 *     are asynchronous on `stream`; the caller keeps every buffer alive (and
 *     unmodified, for inputs) until the stream's work has completed -- the ABI
 *     form of the pages' rule that weight memory must outlive in-flight work
 *     ([gemma4/shared_expert.rs], doc of `encode_shared_expert_branch`).
 *   - Workspace: calls that take (ws, ws_bytes) write the bytes they need to
 *     *ws_bytes and return FFNQ_OK without enqueuing anything when ws == NULL.
 *     With ws != NULL, *ws_bytes is the workspace size the caller provides;
 *     FFNQ_ERR_WORKSPACE if it is smaller than required.  Its contents on entry
 *     do not matter.  Concurrent calls need distinct workspaces.
 *   - m == 0 (no tokens) is a no-op that returns FFNQ_OK after the checks.
 *   - bf16 is the 16-bit brain float (upper half of an IEEE binary32), passed as
 *     uint16_t storage.  Activations are bf16 at the ABI; every intermediate is
 *     fp32 and outputs are rounded to bf16 once, to nearest even.
 */
#ifndef FFNQ_H
#define FFNQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef FFNQ_API
#define FFNQ_API __attribute__((visibility("default")))
#endif

/* ---- status codes ------------------------------------------------------- */
#define FFNQ_OK                 0
#define FFNQ_ERR_INVALID       -1  /* NULL pointer, width <= 0, bad alignment, aliasing, K not a multiple of 64 */
#define FFNQ_ERR_UNSUPPORTED   -2  /* unknown fmt/act/tail, routed experts not INT4-affine, slot_cap > 32, ... */
#define FFNQ_ERR_CAPACITY      -3  /* slot_cap < top_k: not even one token fits a sub-batch */
#define FFNQ_ERR_WORKSPACE     -4  /* workspace or plan buffer too small */
#define FFNQ_ERR_HIP           -5  /* a kernel launch failed */

/* ---- weight formats ------------------------------------------------------
 * FFNQ_FMT_INT8_ROW: symmetric per-output-row INT8.
 *   q: int8  [n][k]      w[i][j] = s[i] * q[i][j]
 *   s: fp32  [n]
 *   z: NULL
 *   k must be a multiple of 64.
 * FFNQ_FMT_INT4_AFFINE_G64: affine INT4, groups of 64 consecutive inputs.
 *   q: uint8 [n][k/2]    code(i,j) = (q[i][j/2] >> (4*(j&1))) & 0xF
 *                        (even j in the low nibble)
 *   s: bf16  [n][k/64]   w[i][j] = s[i][j/64] * (code(i,j) - z[i][j/64])
 *   z: bf16  [n][k/64]
 *   k must be a multiple of 128 for the GPU kernels (64 defines the format;
 *   k % 128 == 64 is refused with FFNQ_ERR_UNSUPPORTED).
 * The pages name the routed blob layout "Affine" ([qwen/moe_batch.rs],
 * refusal of non-Affine layouts in `encode_qwen_layer_moe_batched`) and the
 * shared expert "INT8" ([gemma4/shared_expert.rs], branch doc); the exact bit
 * layouts above are this library's reading.
 */
#define FFNQ_FMT_INT8_ROW         1
#define FFNQ_FMT_INT4_AFFINE_G64  2

/* ---- tiled formats (the layout the GPU streams fastest) ---------------------
 * The same numbers as the two formats above, rearranged once by ffnq_pack so
 * that every load of the K loop reads 1 KB of contiguous memory and every
 * lane receives the codes its matrix-core step multiplies, in input order.
 * Each 16-row tile (rows >= n of the last tile are zero) is a run of 1 KB
 * steps; in a code step, the 16 bytes at [16*(16g + r), +16) belong to row r
 * (r = 0..15) and lane group g (g = 0..3), as four 32-bit words w[0..3]:
 *   FFNQ_FMT_INT8_ROW_TILED (k % 64 == 0): step b = code block b (inputs
 *     64b..64b+63); w[2d + h] holds the int8 codes of inputs
 *     64b + 32d + 8g + 4h + i (i = 0..3) in byte i (d, h = 0..1).  After all
 *     tiles: the fp32 row scales, padded to 16 per tile, then to a multiple
 *     of 256 bytes.
 *   FFNQ_FMT_INT4_AFFINE_G64_TILED (k % 128 == 0): code blocks of 128 inputs
 *     in groups of 8; group j is preceded by its scale/zero step (step 9j):
 *     block bi of the group, row r at bytes [128*bi + 8*r, +8) =
 *     {s[r][2b], s[r][2b+1]} then {z[r][2b], z[r][2b+1]} as bf16 pairs
 *     (b = 8j + bi; unused slots of a short last group are zero).  Code block
 *     b is step 9j + 1 + bi: w[d] holds the codes of inputs 128b + 32d + 8g + e
 *     (e = 0..7), code e = 2v in bits [4v, 4v+4) and e = 2v+1 in bits
 *     [16+4v, 20+4v) (v = 0..3).
 * A tiled ffnq_qmat has q = the packed buffer and s = z = NULL; stacked
 * experts follow each other ffnq_packed_bytes(fmt, n, k) bytes apart.  The
 * per-byte weight traffic is that of the row-major format (plus the zero
 * padding of a short last group or tile).
 */
#define FFNQ_FMT_INT8_ROW_TILED         3
#define FFNQ_FMT_INT4_AFFINE_G64_TILED  4

/* ---- gated activation, act = f(gate) * up  --------------------------------
 * The gate projection is the operand passed through f ([llama/dense.rs]: the
 * `encode_silu_mul` / `encode_gelu_mul` call takes ffn_gate first).
 *   SILU:      f(v) = v / (1 + exp(-v))
 *   GELU_TANH: f(v) = 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
 */
#define FFNQ_ACT_SILU       1
#define FFNQ_ACT_GELU_TANH  2

/* ---- tails (what happens to h = down(act)) -------------------------------- */
#define FFNQ_TAIL_NONE          0  /* h_out = bf16(h) */
#define FFNQ_TAIL_RESIDUAL      1  /* x_res = bf16(x_res + h)   [llama/dense.rs] residual add */
#define FFNQ_TAIL_RMSNORM       2  /* out = bf16(h / sqrt(mean(h^2) + eps) * w)   [gemma4/shared_expert.rs] */
#define FFNQ_TAIL_SIGMOID_GATE  3  /* h_out = bf16(h * sigmoid(<w_gate, x>))      [qwen/moe_batch.rs] shared expert */

/* Ceiling on expert slots per routed sub-batch: the pages' 32-pointer argument
 * buffer ([qwen/moe_batch.rs], module doc and the slot-count refusal). */
#define FFNQ_MAX_SLOTS 32
/* Largest expert count the router kernel holds per token. */
#define FFNQ_MAX_EXPERTS 1024

/* One quantized matrix of n output rows and k inputs.  For stacked expert
 * tensors the pointers address expert 0 and expert e starts at
 *   q + e*n*k (INT8) or q + e*n*k/2 (INT4) bytes,
 *   s + e*n   (INT8, fp32) or s + e*n*(k/64) (INT4, bf16) elements, z likewise;
 * for a tiled format at q + e*ffnq_packed_bytes(fmt, n, k) (s, z unused). */
typedef struct ffnq_qmat {
    int32_t fmt;      /* FFNQ_FMT_* */
    int32_t n;        /* output rows */
    int32_t k;        /* inputs (columns) */
    const void* q;    /* device: codes */
    const void* s;    /* device: scales */
    const void* z;    /* device: zero points (INT4) or NULL (INT8) */
} ffnq_qmat;

/* A gated FFN: gate and up are [inter][hidden], down is [hidden][inter]
 * ([gemma4/shared_expert.rs]: gate/up GEMVs take rows=inter, cols=hidden; the
 * down GEMV takes rows=hidden, cols=inter).  gate and up must share a format;
 * down may use another (per-tensor block type, [llama/dense.rs] module doc),
 * but either all three matrices are tiled or none is. */
typedef struct ffnq_ffn {
    ffnq_qmat gate, up, down;
} ffnq_ffn;

/* A device slot cache for routed experts streamed from host memory
 * ([qwen/moe_batch.rs] `encode_qwen_layer_moe_batched`: each sub-batch's
 * expert union is read into the expert cache's slots before its routed phases
 * run; the module doc: a sub-batch's union never exceeds the slot count).
 * The caller owns every field and keeps them between calls, so experts that
 * stay in their slots are not copied again. */
typedef struct ffnq_slot_cache {
    void* slots;          /* device: n_slots tiled gate matrices, then n_slots up, then n_slots down
                             (each at its ffnq_packed_bytes stride, as a stacked tiled expert tensor) */
    size_t slots_bytes;   /* bytes at slots: >= n_slots * (2 * packed(gate) + packed(down)) */
    int32_t n_slots;      /* 1 <= n_slots <= FFNQ_MAX_EXPERTS */
    int32_t* expert;      /* host [n_slots]: the expert each slot holds, -1 if none (in/out) */
    uint64_t* last_use;   /* host [n_slots]: the use stamp of each slot (in/out) */
    uint64_t clock;       /* the last stamp handed out (in/out) */
    uint64_t copied;      /* experts copied into slots, counted over calls (in/out) */
} ffnq_slot_cache;

/* ---- ffnq_dense ------------------------------------------------------------
 * Dense FFN half of a layer, for m token-major rows ([llama/dense.rs], the
 * module-doc equation and `encode_llama_layer_dense`):
 *     h = down( f(gate @ x_t) * (up @ x_t) )
 *   tail RESIDUAL: out[t] = bf16(out[t] + h)       (out is the residual stream, in/out)
 *   tail RMSNORM:  out[t] = bf16(rmsnorm(h) * norm_w)  (out is written only)
 * hidden, inter: the FFN widths (the dense width is intermediate_size; a width
 *   of 0 is refused, [llama/dense.rs] module doc).  Must match the ffn shapes.
 * x:      device bf16 [m][hidden]; must not overlap out.
 * out:    device bf16 [m][hidden].
 * norm_w: device bf16 [hidden] for RMSNORM, else ignored (may be NULL).
 * eps:    RMSNorm epsilon (>= 0), added to the mean of squares inside the sqrt.
 * ws:     device workspace (see conventions), or NULL to query *ws_bytes.
 */
FFNQ_API int ffnq_dense(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail,
               const uint16_t* x, uint16_t* out, const uint16_t* norm_w, float eps,
               void* ws, size_t* ws_bytes, hipStream_t stream);

/* ---- ffnq_dense_noalloc ------------------------------------------------------
 * ffnq_dense for callers that cannot allocate device memory (code recorded into
 * a HIP graph, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without (ws, ws_bytes), the same kernels and bit-identical results.
 * Its workspace is a device array inside the library, FFNQ_NOALLOC_SCRATCH_BYTES
 * per GPU, held from the first call on that GPU until the process ends; the
 * call allocates and frees nothing.  Every call on one GPU uses that GPU's
 * array, so calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller; a later call may start as soon as the
 * earlier one's kernels have completed on the stream (the array's contents on
 * entry do not matter).
 * Errors: those of ffnq_dense; FFNQ_ERR_WORKSPACE when the call needs more than
 * FFNQ_NOALLOC_SCRATCH_BYTES (the same query ffnq_dense answers with ws == NULL
 * gives the size; nothing is enqueued); FFNQ_ERR_HIP if the array's device
 * address cannot be obtained.
 */
#define FFNQ_NOALLOC_SCRATCH_BYTES (8u << 20)
FFNQ_API int ffnq_dense_noalloc(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail,
                                const uint16_t* x, uint16_t* out, const uint16_t* norm_w, float eps,
                                hipStream_t stream);

/* ---- ffnq_shared_expert ----------------------------------------------------
 * The shared (dense) expert branch: the same gated FFN with the shared
 * expert's tails, for m rows at once ([gemma4/shared_expert.rs]
 * `encode_shared_expert_branch_batched`; [qwen/moe_batch.rs] the gated shared
 * expert inside `encode_qwen_layer_moe_batched`):
 *   tail RMSNORM:      h_out[t] = bf16(rmsnorm(h) * aux)          aux = norm weight bf16 [hidden]
 *   tail SIGMOID_GATE: h_out[t] = bf16(h * sigmoid(<aux, x_t>))   aux = gate vector bf16 [hidden],
 *                      the logit is an fp32 dot product over hidden
 *   tail NONE:         h_out[t] = bf16(h)                          aux ignored
 * h_out:  device bf16 [m][hidden]; must not overlap x.  With SIGMOID_GATE this
 *         is the seed that ffnq_moe_routed_batched starts its accumulator at.
 */
FFNQ_API int ffnq_shared_expert(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail,
                       const uint16_t* x, uint16_t* h_out, const uint16_t* aux, float eps,
                       void* ws, size_t* ws_bytes, hipStream_t stream);

/* ---- ffnq_router_logits --------------------------------------------------------
 * The router GEMV in front of ffnq_moe_route ([qwen/moe_batch.rs]
 * `encode_qwen_layer_moe_batched`: the M router GEMVs run before the routed
 * half, which reads their fp32 logits back):
 *     logits[t][e] = sum_i w[e][i] * x[t][i]
 * with bf16 operands (exact in fp32) and fp32 products and sums; the order of
 * the sum is the library's own (results are within fp32 reassociation of the
 * exact dot product, not bit-equal to any particular order).
 * x:      device, bf16 [m][hidden], token-major (the rows ffnq_moe_layer reads).
 * w:      device, bf16 [n_experts][hidden], the router weight, row-major.
 * logits: device, fp32 [m][n_experts], written (the input of ffnq_moe_route).
 * All pointers 16-byte aligned; hidden a multiple of 8; logits must not
 * overlap x or w.  Asynchronous on `stream`; m == 0 is a no-op.
 * Errors: INVALID (NULL pointers, m < 0, hidden <= 0 or not a multiple of 8,
 * n_experts <= 0, misalignment, overlap, sizes past the library's limits),
 * HIP (launch failure). */
FFNQ_API int ffnq_router_logits(const uint16_t* x, const uint16_t* w, int m, int hidden, int n_experts,
                                float* logits, hipStream_t stream);

/* ---- ffnq_moe_route ----------------------------------------------------------
 * Router top-k and the expert-union plan, entirely on the device
 * ([qwen/moe_batch.rs]: the host top-k over read-back logits with
 * `router_topk_gemma4`, the cap min(slots, 32) and the sub-batch loop of
 * `encode_qwen_layer_moe_batched`; the module doc's union bound).
 *
 * logits:       device fp32 [m][n_experts].
 * expert_scale: device fp32 [n_experts] per-expert multiplier, or NULL (= ones).
 * top_k:        1 <= top_k <= n_experts; n_experts <= FFNQ_MAX_EXPERTS.
 * slot_cap:     expert slots per sub-batch; top_k <= slot_cap <= FFNQ_MAX_SLOTS.
 * topk_ids:     device int32 [m][top_k]: expert of pair p = t*top_k + r (pair
 *               order: token-major, rank within).
 * topk_w:       device fp32 [m][top_k]: route weights.
 * plan:         device int32 buffer of plan_bytes >= 4*FFNQ_PLAN_INTS(m, top_k).
 *
 * Selection: experts are ranked by logit, descending; equal logits go to the
 * lower index; NaN ranks as -inf.  Rank 0 is the largest logit.
 * Weights: w_r = exp(l_r - l_0) / sum_{r'<k} exp(l_r' - l_0) * scale[e_r]
 * (softmax over all experts renormalised over the selected ones; the full
 * denominator cancels).  A selected logit equal to l_0 contributes exp(0)=1
 * (this also fixes the all-(-inf) and +inf cases); NaN counts as -inf.
 *
 * Plan (all int32, fixed offsets sized for the worst case; S = sub-batches,
 * U = total union entries; unused entries are -1):
 *   [0]                               n_sub = S
 *   sub_tok_begin  [m+1]              token range of sub-batch b: [begin[b], begin[b+1])
 *   sub_union_begin[m+1]              its union entries: [ub[b], ub[b+1]) of union_expert
 *   union_expert   [m*k]              each sub-batch's union in first-appearance pair order;
 *                                     the slot of an expert is its index within its sub-batch
 *   pair_slot      [m*k]              slot (within its sub-batch) of pair p
 *   slot_pair_begin[m*k+1]            pairs of global union entry g: slot_pairs[spb[g] .. spb[g+1])
 *   slot_pairs     [m*k]              pair indices grouped by union entry, ascending within
 * Sub-batches are greedy and maximal: starting at token s, tokens are added
 * while the union of their experts stays <= slot_cap.
 */
#define FFNQ_PLAN_INTS(m, k) (1 + 2 * ((m) + 1) + 4 * (m) * (k) + 1)
#define FFNQ_PLAN_N_SUB(m, k)           0
#define FFNQ_PLAN_SUB_TOK_BEGIN(m, k)   1
#define FFNQ_PLAN_SUB_UNION_BEGIN(m, k) ((m) + 2)
#define FFNQ_PLAN_UNION_EXPERT(m, k)    (2 * (m) + 3)
#define FFNQ_PLAN_PAIR_SLOT(m, k)       (2 * (m) + 3 + (m) * (k))
#define FFNQ_PLAN_SLOT_PAIR_BEGIN(m, k) (2 * (m) + 3 + 2 * (m) * (k))
#define FFNQ_PLAN_SLOT_PAIRS(m, k)      (2 * (m) + 4 + 3 * (m) * (k))

FFNQ_API int ffnq_moe_route(const float* logits, const float* expert_scale, int m, int n_experts,
                   int top_k, int slot_cap, int32_t* topk_ids, float* topk_w,
                   int32_t* plan, size_t plan_bytes, hipStream_t stream);

/* ---- ffnq_moe_routed_batched -----------------------------------------------
 * The routed half for m tokens ([qwen/moe_batch.rs]: phase 1, the fused and
 * seeded phase 2 and the raw residual add of `encode_qwen_layer_moe_batched`):
 *   phase 1, per pair p = t*k + r with expert e = topk_ids[p]:
 *       act_p = f(gate_e @ x_t) * (up_e @ x_t)
 *   phase 2, per token t and output i, the fp32 accumulator is SEEDED:
 *       acc = seed[t][i]  (0 when seed == NULL)
 *       for r = 0..k-1:  acc += topk_w[t*k+r] * (down_e @ act_{t*k+r})[i]
 *   tail: resid[t][i] = bf16(resid[t][i] + acc)   (one raw residual add, no norm)
 * experts:   stacked [n_experts] INT4-affine gate/up [moe_inter][hidden] and
 *            down [hidden][moe_inter], all row-major or all tiled; other
 *            formats are refused (UNSUPPORTED), as the pages refuse non-Affine
 *            blobs for the batched pass.
 * x:         device bf16 [m][hidden]; must not overlap resid.
 * topk_ids, topk_w, plan: as written by ffnq_moe_route for the same m, k.
 * seed:      device bf16 [m][hidden] (the gated shared expert) or NULL.
 * resid:     device bf16 [m][hidden], in/out.
 * Expert ids outside [0, n_experts) and plan entries outside their ranges are
 * skipped on the device rather than dereferenced.  Contract: plan is the one
 * ffnq_moe_route wrote for these topk_ids; the call cannot check a device
 * plan on the host.  With any other plan the rows of tokens whose pairs it
 * does not list are unspecified (never a fault); ffnq_moe_routed_streamed,
 * which reads the plan back, refuses such a plan instead.
 */
FFNQ_API int ffnq_moe_routed_batched(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter,
                            int m, int top_k, int act, const uint16_t* x,
                            const int32_t* topk_ids, const float* topk_w, const int32_t* plan,
                            const uint16_t* seed, uint16_t* resid,
                            void* ws, size_t* ws_bytes, hipStream_t stream);

/* ---- ffnq_moe_layer --------------------------------------------------------
 * The whole MoE layer after routing in one call ([qwen/moe_batch.rs]
 * `encode_qwen_layer_moe_batched`: the sigmoid-gated shared expert seeds the
 * phase-2 accumulator, then the routed half and the raw residual add).  The
 * result is bit for bit that of
 *     ffnq_shared_expert(shared, hidden, shared_inter, m, act,
 *                        FFNQ_TAIL_SIGMOID_GATE, x, seed, shared_gate, ...)
 *     ffnq_moe_routed_batched(experts, ..., seed, resid, ...)
 * with seed an internal bf16 [m][hidden] (shared == NULL: no seed).  Fewer
 * launches: when both are tiled INT4 with matching launch shapes the shared
 * and routed gate/up run in one launch, and the routed reduction makes the
 * seed from the shared expert's fp32 partials instead of a separate tail.
 * experts, topk_ids, topk_w, plan, x, resid: as for ffnq_moe_routed_batched.
 * shared:       the shared expert's gate/up [shared_inter][hidden] and down
 *               [hidden][shared_inter] (any supported format), or NULL.
 * shared_gate:  device bf16 [hidden], the sigmoid gate vector (required with
 *               shared).
 * Errors and the workspace contract are those of the two calls it replaces.
 */
FFNQ_API int ffnq_moe_layer(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k,
                            int act, const ffnq_ffn* shared, int shared_inter, const uint16_t* shared_gate,
                            const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                            const int32_t* plan, uint16_t* resid, void* ws, size_t* ws_bytes,
                            hipStream_t stream);

/* ---- ffnq_moe_layer_logits -------------------------------------------------
 * ffnq_moe_route followed by ffnq_moe_layer in one call ([qwen/moe_batch.rs]
 * `encode_qwen_layer_moe_batched`: the router top-k over the batch's logits,
 * then the gated shared expert and the routed half), with the same results
 * bit for bit: topk_ids, topk_w and plan are written as ffnq_moe_route writes
 * them, and resid as ffnq_moe_layer leaves it.  For small batches (tiled INT4
 * experts, m <= 8, at most 64 pairs and m * n_experts <= 128 keys) the routing
 * runs inside the routed gate/up launch, every workgroup of which repeats it,
 * so the layer has no separate router launch; otherwise the router runs first
 * on the same stream.
 * Arguments: those of ffnq_moe_layer, plus logits / expert_scale / slot_cap /
 * plan_bytes as for ffnq_moe_route; topk_ids, topk_w and plan are outputs here.
 * Errors and the workspace contract: those of the two calls it replaces.
 */
FFNQ_API int ffnq_moe_layer_logits(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m,
                                   int top_k, int act, const ffnq_ffn* shared, int shared_inter,
                                   const uint16_t* shared_gate, const uint16_t* x, const float* logits,
                                   const float* expert_scale, int slot_cap, int32_t* topk_ids, float* topk_w,
                                   int32_t* plan, size_t plan_bytes, uint16_t* resid, void* ws, size_t* ws_bytes,
                                   hipStream_t stream);

/* ---- ffnq_moe_layer_sandwich -----------------------------------------------
 * The Gemma-style routed layer ([qwen/moe_batch.rs] module doc, first bullet:
 * Gemma's routed sum starts from nothing and its shared branch joins in the
 * sandwich tail after a norm; the router takes a learned per-expert scale;
 * [gemma4/shared_expert.rs] `encode_shared_expert_branch`: the shared branch's
 * down projection, then `post_feedforward_layernorm_1` into the bf16 row h1).
 * Per token t:
 *     route:   topk_ids, topk_w, plan as ffnq_moe_route(logits, expert_scale,
 *              ..., slot_cap) writes them;
 *     h1_t   = the shared expert with the RMSNorm tail (shared_norm_w, eps),
 *              bit for bit ffnq_shared_expert(..., FFNQ_TAIL_RMSNORM, ...);
 *     r_t    = bf16 of the routed sum started at +0.0 (no seed), bit for bit
 *              ffnq_moe_routed_batched(..., seed = NULL) on a zero row;
 *     z      = h1_t + r_t (exact), n = bf16(z / sqrt(mean(z^2) + eps) *
 *              post_norm_w), resid_t = bf16(resid_t + n).
 * The pages give no more of the sandwich tail than that the shared branch
 * joins after its own norm; the join, the second norm over it and the final
 * residual add are this library's reading of that sentence.
 * experts:        tiled or row-major INT4-affine g64 experts (UNSUPPORTED
 *                 otherwise), as for ffnq_moe_routed_batched.
 * shared:         the shared expert (any supported format; required).
 * shared_norm_w:  device bf16 [hidden], the shared branch's norm weight.
 * post_norm_w:    device bf16 [hidden], the tail norm's weight.
 * eps:            both norms' epsilon (finite, >= 0).
 * logits, expert_scale, slot_cap, topk_ids, topk_w, plan, plan_bytes: as for
 *                 ffnq_moe_route (outputs here).
 * x, resid:       as for ffnq_moe_routed_batched.
 * Workspace: h1 and r, the shared expert's workspace and the routed half's;
 * ws == NULL returns the size.  Errors: those of the calls it composes.
 */
FFNQ_API int ffnq_moe_layer_sandwich(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m,
                                     int top_k, int act, const ffnq_ffn* shared, int shared_inter,
                                     const uint16_t* shared_norm_w, const uint16_t* post_norm_w, float eps,
                                     const uint16_t* x, const float* logits, const float* expert_scale,
                                     int slot_cap, int32_t* topk_ids, float* topk_w, int32_t* plan,
                                     size_t plan_bytes, uint16_t* resid, void* ws, size_t* ws_bytes,
                                     hipStream_t stream);

/* ---- ffnq_moe_routed_streamed ----------------------------------------------
 * ffnq_moe_routed_batched for experts that live in host memory
 * ([qwen/moe_batch.rs] `encode_qwen_layer_moe_batched` with
 * `plan_and_stream_union`: the host plans each sub-batch from the routes, the
 * sub-batch's union experts are read into the cache slots after the previous
 * sub-batch is done, then its phase 1 and phase 2 run on those slots).  Per
 * sub-batch of the plan, in order, on `stream`: every union expert that no
 * slot holds is copied (host to device) into a slot that holds no expert of
 * this union -- an empty one first, else the least recently used; then the
 * routed phases run on the sub-batch's tokens with the slots as the experts.
 * The result is that of ffnq_moe_routed_batched on the same experts resident
 * (each token's arithmetic is the same; kernel shapes follow the sub-batch's
 * size, so the fp32 summation order may differ).
 * host_experts: tiled INT4 experts (FFNQ_FMT_INT4_AFFINE_G64_TILED, packed by
 *               ffnq_pack and copied out) whose q pointers address host
 *               memory, pinned (hipHostMalloc) for the copies to be
 *               asynchronous.  UNSUPPORTED for any other format.
 * x, topk_ids, topk_w, plan, seed, resid: as for ffnq_moe_routed_batched.
 * cache:        the slot cache; FFNQ_ERR_CAPACITY if a sub-batch's union has more
 *               experts than it has slots (the pages refuse rather than
 *               loop: plan with slot_cap <= n_slots).
 * host_staging: host int32 [FFNQ_PLAN_INTS(m, top_k) + m * top_k], pinned:
 *               the call copies the plan and the ids there and waits for the
 *               stream (the host's read-back of the routes), then checks
 *               them: a plan that is not one ffnq_moe_route could write for
 *               these ids (bounds, sub-batch ranges, union entries, pair
 *               lists) is refused with FFNQ_ERR_INVALID before any copy.
 * The call synchronises `stream` once (the read-back) and so cannot be
 * captured in a graph.  Workspace: the routed half's at m tokens and n_slots
 * experts, plus one sub-batch's ids and plan; ws == NULL returns the size.
 */
FFNQ_API int ffnq_moe_routed_streamed(const ffnq_ffn* host_experts, int n_experts, int hidden, int moe_inter,
                                      int m, int top_k, int act, const uint16_t* x, const int32_t* topk_ids,
                                      const float* topk_w, const int32_t* plan, const uint16_t* seed,
                                      uint16_t* resid, ffnq_slot_cache* cache, int32_t* host_staging,
                                      void* ws, size_t* ws_bytes, hipStream_t stream);

/* ---- ffnq_packed_bytes / ffnq_pack -----------------------------------------
 * Bytes of one n x k matrix (one expert) in a tiled format; fmt may name the
 * row-major format or its tiled form.  0 for an unknown format or shape.
 *
 * ffnq_pack rearranges `src` (row-major INT8_ROW or INT4_AFFINE_G64,
 * n_experts stacked as described at ffnq_qmat) into its tiled form at `dst`
 * (device, 16-byte aligned, at least n_experts * ffnq_packed_bytes(...)
 * bytes given in dst_bytes; must not overlap src).  Asynchronous on `stream`;
 * bit-exact rearrangement, no arithmetic.  Errors: INVALID (NULL pointers,
 * shapes, alignment, overlap), UNSUPPORTED (tiled or unknown src format,
 * INT4 with k % 128 != 0), WORKSPACE (dst_bytes too small). */
FFNQ_API size_t ffnq_packed_bytes(int fmt, int n, int k);
FFNQ_API int ffnq_pack(const ffnq_qmat* src, int n_experts, void* dst, size_t dst_bytes, hipStream_t stream);

/* Human-readable name of a status code (static string). */
FFNQ_API const char* ffnq_status_string(int status);

/* ---- per-kernel timing (profiling harnesses) ------------------------------
 * While `ev` is non-NULL on the calling thread, every ffnq_dense,
 * ffnq_shared_expert and ffnq_moe_routed_batched call made from that thread
 * launches its gate/up kernel with start/stop events ev[0]/ev[1] and its down
 * kernel with ev[2]/ev[3] (hipExtLaunchKernel: the timestamps are taken by
 * the kernel dispatch itself, so the elapsed time is the kernel's own
 * duration).  The four events belong to the caller (hipEventCreate, or a
 * framework's events, valid on the stream's device); the array must stay
 * valid until it is cleared.  NULL clears.  Returns FFNQ_OK.  Results never
 * depend on this switch. */
FFNQ_API int ffnq_set_phase_events(hipEvent_t* ev);

/* ---- practical read rate (measurement aid) --------------------------------
 * Not an operation of the method: a plain streaming read of `bytes` bytes of
 * device memory at `buf` (16-byte loads, a fixed grid of 256 workgroups of
 * 512 threads), so that a harness can set the weight-streaming kernels beside
 * the read rate this GPU reaches for the same number of bytes, next to the
 * published HBM peak.  `sink` (device, 4 bytes, 4-byte aligned) is almost
 * never written; its contents mean nothing.  With ffnq_set_phase_events set,
 * the launch takes ev[0]/ev[1].  Errors: INVALID (NULL pointers, buf not
 * 16-byte aligned, bytes not a multiple of 16), HIP.  bytes == 0 enqueues
 * nothing. */
FFNQ_API int ffnq_stream_read(const void* buf, size_t bytes, unsigned* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FFNQ_H */
