// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace em {

// kernel timing hooks (no-ops unless profiling is enabled)
void prof_begin(hipStream_t s);
void prof_end(hipStream_t s, const char* name);

// Permutation outputs and scratch (device pointers inside the workspace).
struct DispatchBufs {
    uint32_t* bm;       // [(E+G)][W] bitmaps: experts then groups
    uint32_t* pre;      // [(E+G)][W] exclusive prefix popcounts
    int32_t* total;     // [E+G] set bits per bitmap row
    int32_t* eoff;      // [E+1] first row of each expert
    int32_t* uoff;      // [G+1] first unique-token slot of each group
    int32_t* etile;     // [E+1] m-tile prefix over experts
    int32_t* etile_pf;  // [E+1] prefix of 128-row tiles over experts (tiled prefill GEMMs)
    int32_t* gtile_u;   // [G+1] m-tile prefix over groups' unique tokens
    int32_t* gtile_r;   // [G+1] m-tile prefix over groups' rows
    int32_t* row_tok;   // [R] token of each row
    int32_t* row_slot;  // [R] slot of each row
    int32_t* row_exp;   // [R] expert of each row
    int32_t* row_u;     // [R] unique-token slot (within the group list) of each row
    int32_t* slot_row;  // [T*k] row of each (token, slot)
    int32_t* ut_tok;    // [<= R] token of each unique-token slot
};

// Everything the expert-layer kernels read or write.
struct LayerArgs {
    int T, d, h, E, P, G, k, r, rL, gq;
    int mt;                     // rows per GEMM task (m-tile)
    const uint16_t* x;          // [T][d]
    const float* topk_w;        // [T][k]
    // weights
    const uint8_t* s_up; const uint16_t* s_up_s;
    const uint8_t* s_dn; const uint16_t* s_dn_s;
    const uint8_t* a_up; const uint16_t* a_up_s;
    const uint8_t* b_up; const uint16_t* b_up_s;
    const uint8_t* a_dn; const uint16_t* a_dn_s;
    const uint8_t* b_dn; const uint16_t* b_dn_s;
    const uint16_t* lu_u; const uint16_t* lu_v;
    const uint16_t* ld_u; const uint16_t* ld_v;
    // intermediates (workspace)
    uint16_t* xg;               // [Umax][d] bf16: x rows of each group's distinct tokens (prefill GEMMs)
    uint16_t* z1;               // [R][r]   bf16
    uint16_t* zl;               // [Umax][rL] bf16 (per unique token of a group)
    float* hs;                  // [Umax][h] shared-up + LoRA-up, fp32
    uint16_t* act;              // [R][h]   bf16
    uint16_t* z2;               // [R][r]   bf16
    uint16_t* zl2;              // [R][rL]  bf16
    float* o;                   // [R][d]   fp32
    float* y;                   // [T][d]   output
    DispatchBufs db;
    int max_etiles, max_gtiles_u, max_gtiles_r;   // grid bounds
    int pf;                     // shared up / down on the LDS-tiled prefill GEMMs (prefill_gemm_ok)
    int64_t umax, rmax;         // bounds on distinct (token, group) pairs and rows
    // microscaling variant: E8M0 block scales of the six MXFP4 matrices (the
    // codes are in s_up .. b_dn) and the MXFP8 copies of the product inputs
    const uint8_t* s_up_e; const uint8_t* s_dn_e;
    const uint8_t* a_up_e; const uint8_t* b_up_e;
    const uint8_t* a_dn_e; const uint8_t* b_dn_e;
    uint8_t* xq;  uint8_t* xs;  // [T][d] E4M3, [T][d/32] E8M0
    uint8_t* aq;  uint8_t* as;  // [R][h], [R][h/32]
};

// Small-batch expert layer (T <= 64, T*k <= 1024): three launches, every
// workgroup rebuilding its view of the routing from topk_idx in LDS.
struct DecodeArgs {
    int T, d, h, E, P, G, k, r, rL, rLp, gq, R;
    int S1;      // K slices of the R1 / R2 products (d / S1 is a multiple of 128)
    int cb2;     // columns per workgroup of the activation kernel (128, 256 or 512)
    int ncb2;    // h / cb2
    int npass;   // row passes of the down kernel (bound: every slot in one group)
    int nxmax;   // upper bound on distinct experts: min(E, R)
    int lds;     // LDS-streaming kernels (see decode_lds_ok)
    const uint16_t* x; const int32_t* idx; const float* topk_w;
    const uint8_t* s_up; const uint16_t* s_up_s;
    const uint8_t* s_dn; const uint16_t* s_dn_s;
    const uint8_t* a_up; const uint16_t* a_up_s;
    const uint8_t* b_up; const uint16_t* b_up_s;
    const uint8_t* a_dn; const uint16_t* a_dn_s;
    const uint8_t* b_dn; const uint16_t* b_dn_s;
    const uint16_t* lu_u; const uint16_t* lu_v;
    const uint16_t* ld_u; const uint16_t* ld_v;
    const uint8_t* s_up_t; const uint8_t* s_dn_t;     // decode-tiled codes of S_up, S_dn (or null)
    const uint8_t* a_up_t;                             // and of A_up (or null)
    float* hs;          // [T][G][h]      shared up, per (token, group)
    float* scratch;     // [64]           target of stores that have no output
    float* z1p;         // [S1][R][r]     partial sums of A_up x
    float* zlp;         // [4 S1][T][G][rLp] partial sums of U_up x
    uint16_t* act;      // [R][h]         bf16 activation per slot
    float* z2p;         // [ncb2][R][r + rL] partial sums of A_dn a, U_dn a
    uint16_t* z2;       // [R][r]
    uint16_t* zl2;      // [R][rLp]
    float* o;           // [R][d]         expert output per slot
    float* od;          // [R][d]         delta down of rows whose group hands it to another workgroup
    float* y;           // [T][d]
    uint32_t* cnt_e;    // [E]     arrivals per expert (activation kernel)
    uint32_t* cnt_c;    // [d/64]  arrivals per output column block (down kernel)
    // persistent single-launch layer (layer.hip)
    const uint8_t* a_dn_t;  // column-blocked A_dn codes [E][h/128][r][64 B] (or null)
    uint32_t* pl_ctr;   // [PL_C_COUNT] task queue head and arrival counters (zeroed per launch)
    float* pl_z1p;      // [4][R][r]     K-slice partial sums of A_up x
    float* pl_zlp;      // [4][T][G][16] K-slice partial sums of U_up x
    uint16_t* pl_z1b;   // [R][r]        z1 (R1), bf16
    uint16_t* pl_zlb;   // [T][G][16]    zl (R2), bf16
    float* pl_z2p;      // [h/128][R][PL_Z2W] per-column-block partial sums of A_dn a, U_dn a
    int pl_trace_o;     // store o + od back into o (per-slot outputs for a trace)
};

// Counter words of the persistent layer (uint32 at pl_ctr).
constexpr int PL_C_HEAD = 0;        // next task
constexpr int PL_C_ZREADY = 1;      // experts and groups whose z1 / zl are rounded
constexpr int PL_C_UP = 2;          // [64] up tasks done per group
constexpr int PL_C_Z2 = 66;         // [64] R4 / R5 reduction parts done per group
constexpr int PL_C_Z1E = 130;       // [1024] A_up x slices done per expert
constexpr int PL_C_ZLG = 1154;      // [64] U_up x slices done per group
constexpr int PL_C_DN = 1218;       // [256] down tasks done per 128-column block of d
constexpr int PL_C_ERR = 1474;      // set when a bounded wait gives up
constexpr int PL_C_COUNT = 1536;
constexpr int PL_Z2W = 160;         // floats per partial row (r + rL <= 144, five cache lines)
bool dec_layer_ok(const DecodeArgs& a);
hipError_t launch_dec_layer(const DecodeArgs& a, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
int decode_ns_down(int T);   // rows per down-kernel pass = 16 * decode_ns_down(T)
bool decode_lds_ok(int T, int d, int h, int r, int rL, int gq, int S1);

// Router launches.  `part` (nullable) is workspace for the K-split small-batch
// path (router_split_ok shapes: RK_NSL x T x E doubles); `logits` may then be
// null (no logits output), and must be given otherwise.
bool router_split_ok(int T, int d, int E);
size_t router_split_bytes(int T, int E);
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* bias,
                         float* logits, double* part, int32_t* idx, float* w, int T, int d, int E, int k,
                         hipStream_t stream);

hipError_t launch_dispatch(const int32_t* idx, const DispatchBufs& db, int T, int k, int E,
                           int P, int mt, hipStream_t stream);

hipError_t launch_expert_layer(const LayerArgs& a, hipStream_t stream);

hipError_t launch_gather_rows(const void* src, const int32_t* index, void* dst, int64_t rows,
                              int64_t row_bytes, hipStream_t stream);

// LDS-tiled shared-matrix GEMMs of large batches (prefill.hip)
enum PfMode { PF_HS = 0, PF_OUT = 1, PF_Z1 = 2, PF_Z2 = 3 };
constexpr int kPfSpareRows = 128;    // readable rows past the end of xg and act (one row tile)
constexpr int kPfTileRows = 128;     // rows per tile of the tiled prefill GEMMs
bool prefill_gemm_ok(int d, int h, int r, int rL, int gq);
hipError_t launch_prefill_gemm(const LayerArgs& a, int mode, int64_t max_rows, hipStream_t s);
hipError_t launch_gather_x(const LayerArgs& a, int64_t umax, hipStream_t s);
hipError_t launch_act(const LayerArgs& a, hipStream_t s);     // needs r == 128, h % 256 == 0
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
void launch_lora_in(const LayerArgs& a, int down, hipStream_t s);
constexpr int kPrefetchBlocks = 128;      // workgroups of the prefetch launch (sink: 256 words each)
hipError_t launch_prefetch(const uint8_t* const* bases, const size_t* group_bytes, int n_regions,
                           const int32_t* groups, int n_groups, int G, uint32_t* sink, int blocks, hipStream_t s);
hipError_t launch_combine(const LayerArgs& a, hipStream_t s);
bool mx_layer_ok(int d, int h, int r, int rL);
hipError_t launch_mx_layer(const LayerArgs& a, hipStream_t s);
hipError_t launch_mfma_peak(float* out, int blocks, int iters, hipStream_t stream);
hipError_t launch_tile_shared(const uint8_t* src_q, uint8_t* dst_q, int G, int N, int K, hipStream_t stream);
hipError_t launch_colblock(const uint8_t* src_q, uint8_t* dst_q, int M, int N, int K, hipStream_t stream);
hipError_t launch_residual(int T, int d, const uint16_t* x, const float* y, uint16_t* x_out,
                           hipStream_t stream);

}  // namespace em
