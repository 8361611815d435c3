// Per-wave weight streaming for skinny int4 GEMMs (decode batches).
//
// A wave owns 16 weight rows and walks K in blocks of 256 elements (128 bytes
// per row).  Each global load covers the 128-byte lines of 8 whole rows (64
// lanes x 16 bytes, full cache lines); the loads run two to four blocks ahead
// in two alternating register sets.  A block passes through a wave-private
// LDS tile (16 rows x 144 bytes, padded against bank conflicts) into the MFMA
// operand layout.  Nothing synchronises the waves of a workgroup while they
// stream: the activation rows are already in LDS.
//
// Measured on a plain 134 MB stream of this shape (2 workgroups per CU): full
// line loads with the arithmetic reach ~4.3 TB/s, against ~3.3 TB/s for
// half-line MFMA-layout loads straight into registers.
#pragma once

#include "common.h"
#include "mfma_ops.h"

namespace em {

constexpr int WS_KB = 256;              // K elements per block
constexpr int WS_TP = 9;                // 16-byte slots per tile row (8 + 1 pad)
constexpr int WS_TILE = 16 * WS_TP;     // 16-byte slots per wave tile
typedef uint32_t ws_u4 __attribute__((ext_vector_type(4)));

// This lane's sources.  Load 0 of a block covers row l / 8 and load 1 row
// 8 + l / 8, bytes [16 (l % 8), +16) of the block's 128; the scale word is the
// fp16 pair of row l % 16 for the block's two 128-element chunks (quant groups
// of 128, so the pair is contiguous and 4-byte aligned).
struct WsSrc {
    const uint8_t* w;                   // row l / 8 at K = 0, plus 16 (l % 8)
    size_t w8;                          // bytes from row r to row r + 8
    const uint16_t* s;                  // scale row of row l % 16 at K = 0
};

EM_DEV void ws_src(WsSrc& p, const uint8_t* w_row0, size_t w_stride, const uint16_t* s_row0, size_t s_stride) {
    const int l = lane_id();
    p.w = w_row0 + (size_t)(l >> 3) * w_stride + 16 * (l & 7);
    p.w8 = 8 * w_stride;
    p.s = s_row0 + (size_t)(l & 15) * s_stride;
}

EM_DEV void ws_fetch(ws_u4& w0, ws_u4& w1, uint32_t& sp, const WsSrc& p, int b, int nb) {
    const int bb = min(b, nb - 1);                      // past the end: the last block again
    const uint8_t* q = p.w + (size_t)bb * (WS_KB / 2);
    w0 = *reinterpret_cast<const ws_u4*>(q);
    w1 = *reinterpret_cast<const ws_u4*>(q + p.w8);
    sp = *reinterpret_cast<const uint32_t*>(p.s + 2 * bb);
}

// Activation rows in LDS: row r of a stage at base + r * stride (elements), its
// 16-byte segments XOR-swizzled by r % 16 so that 16 lanes reading one segment
// of 16 rows hit distinct banks.
struct WsAct {
    const uint16_t* row[4];             // base of the row each lane supplies, per 16-row subtile
    int sw[4];                          // that row's swizzle (row % 16)
};

// Consume one block: transpose through the wave tile T, then the two chunks'
// MFMAs against the activation rows at stage offset k0.
template <int NS>
EM_DEV void ws_block(floatx4 (&acc)[NS], ws_u4 w0, ws_u4 w1, uint32_t spair, ws_u4* T, const WsAct& ar, int k0) {
    const int l = lane_id(), c = l >> 4, li = l & 15;
    T[(l >> 3) * WS_TP + (l & 7)] = w0;
    T[(8 + (l >> 3)) * WS_TP + (l & 7)] = w1;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const ws_u4 t = T[li * WS_TP + 4 * ch + c];
        const uint4 raw = make_uint4(t.x, t.y, t.z, t.w);
        uint4 af[NS][4];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int seg = (k0 >> 3) + (((16 * ch + 4 * c + s) ^ ar.sw[ms]) & 15) + ((16 * ch + 4 * c + s) & ~15);
                af[ms][s] = *reinterpret_cast<const uint4*>(ar.row[ms] + 8 * seg);
            }
        mac_fast<NS>(acc, af, raw, ch ? (spair >> 16) : (spair & 0xFFFFu));
    }
}

// acc[ms] += (this wave's 16 rows) . A over K in [kw, kw + K) of the weights and
// [0, K) of the staged activations; K a multiple of 512.
template <int NS>
EM_DEV void ws_gemm(floatx4 (&acc)[NS], const WsSrc& p0, int kw, ws_u4* T, const WsAct& ar, int K) {
    WsSrc p = p0;
    p.w += kw / 2;
    p.s += kw / 128;
    const int nb = K / WS_KB;
    ws_u4 a0, a1, a2, a3, b0, b1, b2, b3;      // set a: blocks b, b + 1; set b: b + 2, b + 3
    uint32_t as0, as1, bs0, bs1;
    ws_fetch(a0, a1, as0, p, 0, nb);
    ws_fetch(a2, a3, as1, p, 1, nb);
    int b = 0;
    for (; b + 4 <= nb; b += 4) {
        ws_fetch(b0, b1, bs0, p, b + 2, nb);
        ws_fetch(b2, b3, bs1, p, b + 3, nb);
        ws_block<NS>(acc, a0, a1, as0, T, ar, b * WS_KB);
        ws_block<NS>(acc, a2, a3, as1, T, ar, (b + 1) * WS_KB);
        ws_fetch(a0, a1, as0, p, b + 4, nb);
        ws_fetch(a2, a3, as1, p, b + 5, nb);
        ws_block<NS>(acc, b0, b1, bs0, T, ar, (b + 2) * WS_KB);
        ws_block<NS>(acc, b2, b3, bs1, T, ar, (b + 3) * WS_KB);
    }
    if (b < nb) {                       // two blocks left
        ws_block<NS>(acc, a0, a1, as0, T, ar, b * WS_KB);
        ws_block<NS>(acc, a2, a3, as1, T, ar, (b + 1) * WS_KB);
    }
}

}  // namespace em
