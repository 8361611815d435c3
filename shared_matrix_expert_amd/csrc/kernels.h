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
};

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* bias,
                         float* logits, int32_t* idx, float* w, int T, int d, int E, int k,
                         hipStream_t stream);

hipError_t launch_dispatch(const int32_t* idx, const DispatchBufs& db, int T, int k, int E,
                           int P, int mt, hipStream_t stream);

hipError_t launch_expert_layer(const LayerArgs& a, hipStream_t stream);

hipError_t launch_residual(int T, int d, const uint16_t* x, const float* y, uint16_t* x_out,
                           hipStream_t stream);

}  // namespace em
