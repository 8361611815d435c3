/*
 * edge_moe.h - C ABI of the shared-matrix sparse-MoE expert layer for MI355X (gfx950).
 *
 * What the layer computes
 * -----------------------
 * A router picks, for every token, the top-k of E experts (10 of 512 in the
 * pages' model: the Chinese commentary page, section "145B 为什么不用同时装进显存";
 * byteiota "Edge0-145B: Run a 145B Open-Source Model on Your Laptop", Not
 * Compression - Architecture).  Each group of P = 64 consecutive experts shares
 * two large matrices and each expert keeps only a small set of parameters for
 * its differences (launch post "Edge0-145B: Frontier AI Capabilities on Your Own
 * Computer", Under the Hood, Architecture paragraph).  The base weights are
 * 4-bit integers and a LoRA branch runs in parallel with them (byteiota, The
 * Three Pillars, Recover-LoRA paragraph).
 *
 * The pages leave the form of the difference, the FFN shape and the numerics
 * open.  This library fixes them as follows (stated readings):
 *   up:    h  = S_up[g] x + B_up[e] R(A_up[e] x) + V_up[g] R(U_up[g] x)
 *   act:   a  = R(SiLU(h))
 *   down:  o  = S_dn[g] a + B_dn[e] R(A_dn[e] a) + V_dn[g] R(U_dn[g] a)
 *   out:   y_t = sum_{j=0..k-1} w_tj o_tj          (float32, slot order)
 * with g = e / P, R() = round to bf16 (nearest-even), every int4 weight equal
 * to q * s exactly, all other arithmetic in float32 (router: float64).  The
 * shared products are computed once per (token, group) however many of the
 * group's experts the token selected.
 *
 * Storage (every matrix N x K, out x in; "packed int4" = K/2 bytes per row,
 * element 2i in the low nibble of byte i, element 2i+1 in the high nibble,
 * two's complement; one IEEE fp16 scale per Gq_eff = min(quant_group, K)
 * consecutive elements of a row, scale array [N][K/Gq_eff]; bf16 and fp16
 * values are passed as uint16 bit patterns):
 *   s_up  [G][h][d]  int4    s_dn  [G][d][h]  int4         (G = E / P)
 *   a_up  [E][r][d]  int4    b_up  [E][h][r]  int4
 *   a_dn  [E][r][h]  int4    b_dn  [E][d][r]  int4
 *   lora_up_u [G][rL][d] bf16   lora_up_v [G][h][rL] bf16
 *   lora_dn_u [G][rL][h] bf16   lora_dn_v [G][d][rL] bf16
 *
 * Conventions for every call
 * --------------------------
 * - Pointers in the structs and arguments are DEVICE pointers unless stated;
 *   the dims / weights structs themselves are host memory read during the call.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 * - Calls are asynchronous on `stream`; the library never synchronises.  Inputs
 *   must stay valid and unmodified until the stream work completes.
 * - The caller owns every buffer.  The library allocates no device memory and
 *   keeps no pointer after a call returns; all scratch lives in the caller's
 *   workspace.  Outputs are overwritten, never accumulated into, and must not
 *   alias inputs or the workspace.
 * - Calls are thread-safe provided concurrent calls use distinct workspaces.
 * - Validation is synchronous and happens before anything is enqueued; a
 *   non-zero status means nothing was enqueued (except EDGE_MOE_EHIP, which is
 *   returned when a launch fails after earlier kernels were enqueued).
 *   Device-side faults surface at the caller's next synchronisation.
 * - No C++ exception crosses this interface.
 */
#ifndef EDGE_MOE_H
#define EDGE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EDGE_MOE_ABI_VERSION 5

/* Status codes. */
#define EDGE_MOE_OK           0
#define EDGE_MOE_EINVAL      -1  /* null / misaligned pointer, inconsistent dims        */
#define EDGE_MOE_EUNSUPPORTED -2 /* shape outside the kernels' limits, or not gfx950     */
#define EDGE_MOE_EWORKSPACE  -3  /* workspace null or smaller than edge_moe_workspace_bytes */
#define EDGE_MOE_EHIP        -4  /* a HIP call or kernel launch failed                  */

/* Layer shape.  Limits checked by every call:
 *   1 <= T <= 1<<20;  d, h multiples of 128 with 128 <= d, h <= 32768;
 *   n_experts a multiple of experts_per_group, n_experts <= 1024, groups <= 64;
 *   1 <= top_k <= min(n_experts, 32);
 *   delta_rank in [8, 256], a multiple of 8;  lora_rank in [2, 32], even;
 *   quant_group a power of two in [32, 4096]; for every matrix K is a multiple
 *   of Gq_eff = min(quant_group, K). */
typedef struct edge_moe_dims {
    int32_t T;                 /* tokens in the batch                     */
    int32_t d;                 /* model dimension                         */
    int32_t h;                 /* expert hidden dimension                 */
    int32_t n_experts;         /* E                                       */
    int32_t experts_per_group; /* P (64 in the pages' model)              */
    int32_t top_k;             /* k                                       */
    int32_t delta_rank;        /* r, rank of each expert's difference     */
    int32_t lora_rank;         /* rL, rank of the per-group LoRA branch   */
    int32_t quant_group;       /* Gq, int4 group size along K             */
} edge_moe_dims;

/* Weights of one layer (device pointers, layouts above; 16-byte aligned).
 * The last four members are optional stored copies of the int4 codes written
 * by edge_moe_tile_shared (the scales stay in the row-major arrays): s_up_t
 * and s_dn_t NULL or both set, a_up_t and a_dn_t each NULL or set.  When they
 * are set, batches of at most 16 tokens stream them instead of the row-major
 * codes (the row-major copies stay required: larger batches and the other
 * paths read them); both copies must hold the same values.  With all four
 * set, edge_moe_forward_persistent can run the layer as one persistent launch
 * (see there). */
typedef struct edge_moe_weights {
    const uint8_t*  s_up_q;  const uint16_t* s_up_scale;
    const uint8_t*  s_dn_q;  const uint16_t* s_dn_scale;
    const uint8_t*  a_up_q;  const uint16_t* a_up_scale;
    const uint8_t*  b_up_q;  const uint16_t* b_up_scale;
    const uint8_t*  a_dn_q;  const uint16_t* a_dn_scale;
    const uint8_t*  b_dn_q;  const uint16_t* b_dn_scale;
    const uint16_t* lora_up_u; const uint16_t* lora_up_v;
    const uint16_t* lora_dn_u; const uint16_t* lora_dn_v;
    const uint8_t*  s_up_t;    /* optional, tiled s_up codes */
    const uint8_t*  s_dn_t;    /* optional, tiled s_dn codes */
    const uint8_t*  a_up_t;    /* optional, tiled a_up codes */
    const uint8_t*  a_dn_t;    /* optional, column-blocked a_dn codes */
} edge_moe_weights;

/* Optional per-stage outputs of edge_moe_forward_traced (device pointers; any
 * member may be NULL).  "Rows" are the R = T * top_k (token, slot) pairs sorted
 * by expert, then token; "slot" s = t * top_k + j. */
typedef struct edge_moe_trace {
    int32_t*  expert_offsets;  /* [E+1]  first row of each expert                    */
    int32_t*  row_token;       /* [R]    token of each row                           */
    int32_t*  row_slot;        /* [R]    slot j of each row                          */
    uint16_t* act;             /* [R][h] bf16 activation a of each slot (slot order) */
    float*    expert_out;      /* [R][d] float32 expert output o of each slot (slot order) */
} edge_moe_trace;

/* Bytes of device workspace needed by edge_moe_route and edge_moe_forward for
 * these dims (the maximum of both).  Host-only; returns 0 for invalid dims. */
size_t edge_moe_workspace_bytes(const edge_moe_dims* dims);

/* Router (a1, a2 of the layer).
 *   x            [T][d] bf16, row-major, 16-byte aligned
 *   w_router     [E][d] bf16
 *   router_bias  [E] float32 or NULL
 *   topk_idx     [T][k] int32 out: selected experts, descending logit, ties to
 *                the lower index
 *   topk_w       [T][k] float32 out: softmax over the k selected logits
 *   logits_out   [T][E] float32 out or NULL: the logits, each the float64
 *                sum of the bf16 x bf16 products rounded once to float32,
 *                then the bias added in float32 and the sum rounded again
 *   ws, ws_bytes device workspace (>= edge_moe_workspace_bytes(dims))
 * Exactness.  Every bf16 x bf16 product is exact in float64.  The float64
 * sum is the exact dot product, and each logit the correctly rounded float32
 * of it, whenever the products of the dot are all multiples of 2^Q and the
 * sum of their magnitudes is below 2^(53+Q) (then every partial sum, in any
 * order, is an exact float64).  At d = 4096 it holds whenever the ratio of the
 * largest to the smallest nonzero magnitude of x's row, times the same ratio
 * for w_router's row, is below 2^25.  Outside it
 * the float64 accumulation may round, and a logit can differ from the
 * correctly rounded value by one float32 unit in the last place when the exact
 * sum lies within that rounding error of a float32 midpoint; this is not
 * detected.  The selection and weights follow the logits as computed.
 * Non-finite inputs are not supported (undefined results). */
int edge_moe_route(const edge_moe_dims* dims, const uint16_t* x, const uint16_t* w_router,
                   const float* router_bias, int32_t* topk_idx, float* topk_w,
                   float* logits_out, void* ws, size_t ws_bytes, void* stream);

/* Expert layer (a3-a11): permutation, shared and per-expert products, LoRA
 * branch, activation and weighted combine.
 *   x         [T][d] bf16 (the router's input)
 *   topk_idx  [T][k] int32 from edge_moe_route (or any selection with distinct
 *             in-range experts per token; not checked on the device)
 *   topk_w    [T][k] float32
 *   y         [T][d] float32 out
 * Results are bitwise reproducible for identical inputs and dims. */
int edge_moe_forward(const edge_moe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                     const float* topk_w, const edge_moe_weights* weights, float* y,
                     void* ws, size_t ws_bytes, void* stream);

/* The expert layer of a decode or verify batch as one persistent launch
 * (after a small one that clears its counters): one workgroup per compute
 * unit takes tasks from a queue in the workspace - the R1 / R2 inputs, the
 * shared up with the fused delta up, activation and R4 / R5 partial sums per
 * 128 columns, the R4 / R5 reductions, and the shared, LoRA and delta down per
 * 128 output columns, the last of which forms y.  The launch ramps between the
 * layer's phases are gone and phases overlap across groups (the pages: the
 * layer runs 48 deep and generation is bound by weight reads - byteiota, Not
 * Compression - Architecture; launch post, Under the Hood, Scheduling).
 * Same arguments, results and tolerances as edge_moe_forward (trace: as
 * edge_moe_forward_traced, NULL for none); requires T <= 8, T * top_k <= 128,
 * d = 4096, h a multiple of 1024 up to 16384, r = 128, rL = 8 or 16, quant
 * groups of 128, experts_per_group <= 64, and all four stored copies in
 * `weights` (edge_moe_tile_shared kinds 0-3); EDGE_MOE_EUNSUPPORTED otherwise. */
int edge_moe_forward_persistent(const edge_moe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                                const float* topk_w, const edge_moe_weights* weights, float* y, void* ws,
                                size_t ws_bytes, void* stream, const edge_moe_trace* trace);

/* edge_moe_forward that also copies per-stage intermediates into `trace`
 * (host struct of device pointers, NULL = none). */
int edge_moe_forward_traced(const edge_moe_dims* dims, const uint16_t* x,
                            const int32_t* topk_idx, const float* topk_w,
                            const edge_moe_weights* weights, float* y, void* ws,
                            size_t ws_bytes, void* stream, const edge_moe_trace* trace);

/* edge_moe_forward without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a 16 MiB array that the library holds on each GPU it runs on
 * until the process ends (its device address is looked up once per device, on
 * the first call there).  Every call on a GPU uses that GPU's one array, so
 * calls that overlap on one GPU (concurrent streams or threads) race and must
 * be serialised by the caller; each call overwrites what it reads.  Returns
 * EDGE_MOE_EWORKSPACE when edge_moe_workspace_bytes(dims) exceeds 16 MiB (at
 * d = 4096, h = 8192, 512 experts, top-10: up to 17 tokens); otherwise as
 * edge_moe_forward. */
int edge_moe_forward_noalloc(const edge_moe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                             const float* topk_w, const edge_moe_weights* weights, float* y, void* stream);

/* Next-layer prefetch (the prerouter idea: a light predictor names the next
 * layer's experts one step ahead so that their weights can be fetched while
 * the current layer computes; byteiota "Edge0-145B: Run a 145B Open-Source
 * Model on Your Laptop", The Three Pillars, Prerouter paragraph).  Reads the
 * shared matrices of the listed groups of one layer once, computing nothing,
 * so that a later layer call can find them in the GPU's memory-side cache.
 * Results of every other call are unchanged by it.
 *   groups   device int32[n_groups], the predicted groups (entries outside
 *            0..G-1 are skipped; duplicates are read twice)
 *   parts    bit 0: S_up (codes, or its decode-tiled copy when weights has
 *            one, and scales); bit 1: S_dn likewise
 *   ws       device scratch of at least edge_moe_prefetch_ws_bytes() bytes,
 *            written (no meaning) by the call
 * Meant to run on a second stream of default priority beside the layer;
 * asynchronous.  EDGE_MOE_EINVAL for bad pointers, n_groups < 0 or
 * n_groups > 4 G, parts outside 1..3. */
size_t edge_moe_prefetch_ws_bytes(void);
int edge_moe_prefetch(const edge_moe_dims* dims, const edge_moe_weights* weights, const int32_t* groups,
                      int32_t n_groups, int32_t parts, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- MX variant --
 * The expert layer with its six large matrices in MXFP4 instead of int4: the
 * microscaling format of the Open Compute Project's MX specification v1.0,
 * MI355X's native 4-bit floating format.  The pages ship 4-bit floating-point
 * builds of the model (byteiota "Edge0-145B: Run a 145B Open-Source Model on
 * Your Laptop", What You Need to Run It).
 *
 * Layouts: each matrix is stored N x K like the int4 one; codes [N][K/2] bytes,
 * two E2M1 codes per byte (element 2i in the low nibble: sign bit 3, exponent
 * bits 2..1 with bias 1, mantissa bit 0); scales [N][K/32] bytes, one E8M0
 * power of two 2^(X - 127) per 32 consecutive elements along K (X = 255 is
 * NaN: not allowed).  The weight is code value * 2^(X - 127) exactly.  LoRA
 * factors are bf16 as in edge_moe_weights.  16-byte aligned device pointers.
 *
 * Arithmetic: the int4 layer's, except that the inputs of the four large
 * MXFP4 products, x (for S_up, A_up) and a (for S_dn, A_dn), are first
 * quantised to MXFP8 along K, per block of 32: E8M0 byte
 * X = floor(log2(block max |v|)) - 8 + 127 limited to 0..254 (0 for an
 * all-zero block), each element v / 2^(X - 127) rounded to the nearest E4M3
 * value (ties to even, magnitudes past 448 saturated to 448).  The rank-r
 * inputs z1, z2 (bf16 after R1, R4) meet B_up, B_dn unquantised, and the
 * LoRA products take x and a unquantised; R1-R5 round to bf16 as in the int4
 * layer.  The large products run on the scaled FP4 x FP8 matrix cores, which
 * sum the 128 products of one instruction to about 2^-13.5 of their
 * magnitude sum, so results meet the layer's tolerance, not bit equality.
 * B_up and B_dn scale bytes must not exceed 252 (their weights are formed in
 * bf16).
 *
 * Shapes: delta_rank 128, d and h multiples of 512 (at least 512), lora_rank a
 * multiple of 8 from 8 to 32; any T.  quant_group is not used.  Other shapes:
 * EDGE_MOE_EUNSUPPORTED.  Every batch size runs the tiled large-batch kernels. */
typedef struct edge_moe_weights_mx {
    const uint8_t*  s_up_q;  const uint8_t* s_up_e;   /* [G][h][d/2], [G][h][d/32] */
    const uint8_t*  s_dn_q;  const uint8_t* s_dn_e;   /* [G][d][h/2], [G][d][h/32] */
    const uint8_t*  a_up_q;  const uint8_t* a_up_e;   /* [E][r][d/2], [E][r][d/32] */
    const uint8_t*  b_up_q;  const uint8_t* b_up_e;   /* [E][h][r/2], [E][h][r/32] */
    const uint8_t*  a_dn_q;  const uint8_t* a_dn_e;   /* [E][r][h/2], [E][r][h/32] */
    const uint8_t*  b_dn_q;  const uint8_t* b_dn_e;   /* [E][d][r/2], [E][d][r/32] */
    const uint16_t* lora_up_u; const uint16_t* lora_up_v;
    const uint16_t* lora_dn_u; const uint16_t* lora_dn_v;
} edge_moe_weights_mx;

/* Workspace bytes of edge_moe_forward_mx (0 for invalid or unsupported dims). */
size_t edge_moe_workspace_bytes_mx(const edge_moe_dims* dims);

/* The MX expert layer (a3-a11), arguments as edge_moe_forward_traced (trace may
 * be NULL); ws_bytes >= edge_moe_workspace_bytes_mx(dims).  The same status
 * codes; asynchronous on `stream`. */
int edge_moe_forward_mx(const edge_moe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                        const float* topk_w, const edge_moe_weights_mx* weights, float* y, void* ws,
                        size_t ws_bytes, void* stream, const edge_moe_trace* trace);

/* ------------------------------------------------ expert streaming from host --
 * The pages keep the expert library in host memory and bring the experts a
 * batch routes to into a small GPU memory, evicting the least recently used,
 * through fixed slots filled while other work runs (launch post "Edge0-145B:
 * Frontier AI Capabilities on Your Own Computer", Under the Hood, Loading
 * paragraph; byteiota "Edge0-145B: Run a 145B Open-Source Model on Your
 * Laptop", The Three Pillars, SSD expert streaming paragraph).  Here one
 * layer's per-expert tensors live in host memory (pinned, for the copies to
 * overlap) and HBM holds S slots per group: slot arrays shaped like the
 * layer's expert arrays with G * S experts in place of E.
 *
 * A batch runs unchanged kernels on a "slot layer": dims with
 * n_experts = G * S and experts_per_group = S, weights whose shared matrices
 * and LoRA factors are the resident layer's and whose expert tensors are the
 * slot arrays, and topk_idx renamed by edge_moe_cache_map (topk_w unchanged).
 * Slot g * S + s belongs to group g, so every (token, slot) pair computes what
 * it computes with all E experts resident: bitwise through edge_moe_forward;
 * through edge_moe_forward_persistent up to the order of fp32 additions (its
 * down tasks split a pass's distinct experts over two K halves by their rank,
 * so the numbering decides which partial sum a row's delta term joins).
 *
 * A cache is a host object: it keeps the pointers given to
 * edge_moe_cache_create until edge_moe_cache_destroy, the one exception to
 * the no-retained-pointer convention above.  One cache serves one layer and
 * is not thread-safe. */
typedef struct edge_moe_expert_tensors {
    /* per expert, in edge_moe_weights' layouts; the first eight required,
     * the two decode copies (edge_moe_tile_shared which = 2, 3) optional */
    void* a_up_q;  void* a_up_scale;   /* [E or G*S][r][d/2],  [..][r][d/Gq_eff] fp16  */
    void* b_up_q;  void* b_up_scale;   /* [..][h][r/2],        [..][h][r/Gq_eff]       */
    void* a_dn_q;  void* a_dn_scale;   /* [..][r][h/2],        [..][r][h/Gq_eff]       */
    void* b_dn_q;  void* b_dn_scale;   /* [..][d][r/2],        [..][d][r/Gq_eff]       */
    void* a_up_t;  void* a_dn_t;       /* [..][r * d / 2], [..][r * h / 2] (optional) */
} edge_moe_expert_tensors;

typedef struct edge_moe_cache_stats {
    int64_t hits;          /* distinct experts found resident            */
    int64_t misses;        /* distinct experts copied into a slot        */
    int64_t evictions;     /* misses that replaced a resident expert     */
    int64_t bytes_copied;  /* host -> HBM bytes issued                   */
} edge_moe_cache_stats;

typedef struct edge_moe_cache edge_moe_cache;

/* A cache of slots_per_group (1..P) slots per group.  host: the E experts'
 * tensors (host memory); slots: the G * S slots' tensors (device memory, set
 * exactly where host is set), or NULL for a cache that only plans (no copy is
 * issued; the policy and the statistics behave the same).  dims must pass
 * the layer's checks (T is not used otherwise); the per-expert sizes follow
 * from it, and the buffers must hold E (host) and G * S (slots) experts of
 * those sizes.  NULL for invalid arguments or no memory.  Slots start empty.
 * Copies go out as one gather kernel per call that reads the host memory
 * directly when every host tensor is device-addressable pinned memory
 * (hipHostMalloc) and 16-byte aligned, else as hipMemcpyAsync per tensor. */
edge_moe_cache* edge_moe_cache_create(const edge_moe_dims* dims, int32_t slots_per_group,
                                      const edge_moe_expert_tensors* host, const edge_moe_expert_tensors* slots);
void edge_moe_cache_destroy(edge_moe_cache* cache);

/* Make a batch's experts resident and rename them to slots.  topk_idx: HOST
 * int32[T][top_k] expert ids (as edge_moe_route wrote them); slot_idx: HOST
 * int32[T][top_k], receives each entry's slot.  Resident experts of the batch
 * are refreshed first; each missing one then takes a free slot of its group,
 * else the group's least recently used slot that the batch does not use, and
 * its tensors are copied there with hipMemcpyAsync on `stream`.  Work that
 * still reads a slot (an earlier batch's kernels) or writes one (an earlier
 * prefetch's copies on another stream) must be ordered before those copies
 * (same stream, or an event), and the layer call after them.
 * EDGE_MOE_EINVAL for a null cache or pointers or ids outside 0..E-1;
 * EDGE_MOE_EUNSUPPORTED when some group needs more distinct experts than it
 * has slots (nothing changes then); EDGE_MOE_EHIP when a copy could not be
 * enqueued (the placement was recorded, so the slots no longer match it:
 * destroy the cache).  stats (may be NULL) receives this call's counts. */
int edge_moe_cache_map(edge_moe_cache* cache, int32_t T, const int32_t* topk_idx, int32_t* slot_idx,
                       void* stream, edge_moe_cache_stats* stats);

/* Bring predicted experts in ahead of their batch (host int32[n] ids), e.g. on
 * a copy stream while the previous layer computes, so that the slots are
 * filled before edge_moe_cache_map needs them.  Same placement rule, except
 * that any slot not filled by this call may be replaced; experts past a
 * group's S in one call are skipped.  The same ordering duty and errors (ids
 * outside 0..E-1: EDGE_MOE_EINVAL). */
int edge_moe_cache_prefetch(edge_moe_cache* cache, int32_t n, const int32_t* experts, void* stream,
                            edge_moe_cache_stats* stats);

/* Counts summed over every map and prefetch call of the cache. */
int edge_moe_cache_totals(const edge_moe_cache* cache, edge_moe_cache_stats* stats);

/* The slot of a resident expert (0..G*S-1), -1 if not resident, -2 for a null
 * cache or an id outside 0..E-1. */
int edge_moe_cache_slot_of(const edge_moe_cache* cache, int32_t expert);

/* Residual between stacked layers (a12): x_out[t][i] = bf16(x[t][i] + y[t][i]),
 * the exact sum rounded once to the nearest bf16 (ties to even).  The layers
 * are stacked 48 deep in the pages' model (byteiota, Not Compression -
 * Architecture).  x, x_out: [T][d] bf16; y: [T][d] float32 (e.g. the output of
 * edge_moe_forward); x_out may equal x (in place).  16-byte aligned, d a
 * multiple of 8. */
int edge_moe_residual(int32_t T, int32_t d, const uint16_t* x, const float* y, uint16_t* x_out,
                      void* stream);

/* Plain device copy of `bytes` bytes (dst and src 16-byte aligned, bytes a
 * multiple of 16, non-overlapping), enqueued on `stream` as one kernel that
 * reads every source byte once and writes every destination byte once.  Not a
 * step of the layer: it is the reference workload of known size used to
 * calibrate the memory-traffic counters of a profiler against bytes. */
int edge_moe_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Matrix-core rate calibration (not a step of the layer): `blocks` workgroups
 * of four waves each run `iters` rounds of eight independent bf16 MFMA chains
 * (16 x 16 x 32, 16384 flops each), so one launch performs
 * blocks * 4 * iters * 8 * 16384 flops; out[blocks * 256] float receives a
 * fold of the accumulators.  Timed by the caller (events on `stream`), it
 * gives the measured dense bf16 rate to set beside the published peak.
 * EDGE_MOE_EINVAL for a null or misaligned out or non-positive counts. */
int edge_moe_mfma_peak(float* out, int32_t blocks, int32_t iters, void* stream);

/* Static description of a status code (never NULL). */
const char* edge_moe_status_string(int status);

/* Decode-tiled copy of the int4 codes of one matrix set (which = 0: s_up
 * [G][h][d], which = 1: s_dn [G][d][h], which = 2: a_up [E][r][d]; which = 3:
 * the column-blocked a_dn [E][r][h], defined at the end), written
 * from the row-major packed codes src_q into dst_q of the same size (M*N*K/2
 * bytes for M matrices of N x K).  A stored-format conversion done once per
 * layer, outside any step: the layer's values are unchanged, and the scales
 * keep their row-major arrays (each row's K/128 scales contiguous).
 *
 * Layout (N x K matrix g of the set; requires quant_group == 128, N a multiple
 * of 128, K a multiple of 1024): rows form tiles of 16 and tile groups of 8
 * tiles (128 rows); K forms blocks of 256 (two 128-element chunks).  For tile
 * group n, block b, tile t, chunk c and lane l = i + 16 j (i < 16, j < 4), the
 * 16 bytes at
 *     g*N*K/2 + n*64*K + b*16384 + t*2048 + c*1024 + l*16
 * hold elements [(2b + c)*128 + 32 j, +32) of row 128 n + 16 t + i, packed as
 * in the row-major layout.  So one 1 KB read of 64 lanes returns, per lane,
 * the 32 codes of one row that a 16 x 16 x 32 matrix-core operand needs, and
 * a workgroup that streams one tile group reads one contiguous region.
 *
 * Column-blocked a_dn (which = 3; requires r = 128 and h a multiple of 128):
 * for expert e and block cb of 128 elements of h, the 128 rows' 64-byte
 * segments follow each other: the 16 bytes at
 *     (e * h/128 + cb) * 8192 + n * 64 + 16 j
 * hold elements [128 cb + 32 j, +32) of row n of a_dn[e], packed as in the
 * row-major layout.  One block of all rows is then one contiguous 8 KB.
 *
 * Errors: EDGE_MOE_EINVAL for null or not 16-byte aligned pointers, or which
 * not 0..3; EDGE_MOE_EUNSUPPORTED when the shape is outside the layout
 * above.  src and dst must not overlap. */
int edge_moe_tile_shared(const edge_moe_dims* dims, int32_t which, const uint8_t* src_q, uint8_t* dst_q,
                         void* stream);

/* EDGE_MOE_ABI_VERSION of the built library. */
int edge_moe_abi_version(void);

/* Kernel timing for measurement: when enabled (on != 0) every kernel the
 * library enqueues is bracketed by HIP events recorded on the caller's stream,
 * and the per-kernel elapsed times are accumulated under the kernel's name.
 * edge_moe_prof_read fills up to `cap` entries (name, launches, total ms) after
 * synchronising the recorded events and returns the number of kernel names;
 * edge_moe_prof_reset clears the table.  Host-side bookkeeping for
 * measurement, guarded by one lock: calls from several threads are safe, and
 * while profiling is on every enqueue also records two events on its stream. */
int  edge_moe_prof_enable(int on);
int  edge_moe_prof_read(char (*names)[64], int64_t* launches, double* total_ms, int cap);
void edge_moe_prof_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* EDGE_MOE_H */
