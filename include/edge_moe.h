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

#define EDGE_MOE_ABI_VERSION 2

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
 * The last three members are optional decode-tiled copies of the int4 codes
 * written by edge_moe_tile_shared (the scales stay in the row-major arrays):
 * s_up_t and s_dn_t NULL or both set, a_up_t NULL or set.  When they are set,
 * batches of at most 16 tokens stream them instead of the row-major s_up_q /
 * s_dn_q / a_up_q (the row-major copies stay required: larger batches and the
 * other paths read them); both copies must hold the same values. */
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
 *   logits_out   [T][E] float32 out or NULL: the logits, each the correctly
 *                rounded float32 of the exact dot product (accumulated in
 *                float64), plus the bias added in float32
 *   ws, ws_bytes device workspace (>= edge_moe_workspace_bytes(dims))
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

/* edge_moe_forward that also copies per-stage intermediates into `trace`
 * (host struct of device pointers, NULL = none). */
int edge_moe_forward_traced(const edge_moe_dims* dims, const uint16_t* x,
                            const int32_t* topk_idx, const float* topk_w,
                            const edge_moe_weights* weights, float* y, void* ws,
                            size_t ws_bytes, void* stream, const edge_moe_trace* trace);

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

/* Static description of a status code (never NULL). */
const char* edge_moe_status_string(int status);

/* Decode-tiled copy of the int4 codes of one matrix set (which = 0: s_up
 * [G][h][d], which = 1: s_dn [G][d][h], which = 2: a_up [E][r][d]), written
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
 * Errors: EDGE_MOE_EINVAL for null or not 16-byte aligned pointers, or which
 * not 0, 1 or 2; EDGE_MOE_EUNSUPPORTED when the shape is outside the layout
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
 * edge_moe_prof_reset clears the table.  Host-side bookkeeping, not thread-safe. */
int  edge_moe_prof_enable(int on);
int  edge_moe_prof_read(char (*names)[64], int64_t* launches, double* total_ms, int cap);
void edge_moe_prof_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* EDGE_MOE_H */
