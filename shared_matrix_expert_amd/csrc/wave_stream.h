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

#include <type_traits>

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
// MFMAs against the activation rows at stage offset k0 (rows displaced by boff
// elements: the second of two stage buffers).
template <int NS>
EM_DEV void ws_block(floatx4 (&acc)[NS], ws_u4 w0, ws_u4 w1, uint32_t spair, ws_u4* T, const WsAct& ar, int k0,
                     int boff = 0) {
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
                af[ms][s] = *reinterpret_cast<const uint4*>(ar.row[ms] + boff + 8 * seg);
            }
        mac_fast<NS>(acc, af, raw, ch ? (spair >> 16) : (spair & 0xFFFFu));
    }
}

// Two 16-row tiles against the same activation fragments: one set of A reads
// serves both, and the two tiles' dequantisation and MFMA chains are
// independent work for the scheduler to interleave.
template <int NS>
EM_DEV void ws_block2(floatx4 (&acc0)[NS], floatx4 (&acc1)[NS], ws_u4 w00, ws_u4 w01, uint32_t sp0, ws_u4 w10,
                      ws_u4 w11, uint32_t sp1, ws_u4* T, const WsAct& ar, int k0) {
    const int l = lane_id(), c = l >> 4, li = l & 15;
    T[(l >> 3) * WS_TP + (l & 7)] = w00;
    T[(8 + (l >> 3)) * WS_TP + (l & 7)] = w01;
    T[WS_TILE + (l >> 3) * WS_TP + (l & 7)] = w10;
    T[WS_TILE + (8 + (l >> 3)) * WS_TP + (l & 7)] = w11;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const ws_u4 t0 = T[li * WS_TP + 4 * ch + c];
        const ws_u4 t1 = T[WS_TILE + li * WS_TP + 4 * ch + c];
        uint4 af[NS][4];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int seg = (k0 >> 3) + (((16 * ch + 4 * c + s) ^ ar.sw[ms]) & 15) + ((16 * ch + 4 * c + s) & ~15);
                af[ms][s] = *reinterpret_cast<const uint4*>(ar.row[ms] + 8 * seg);
            }
        mac_fast<NS>(acc0, af, make_uint4(t0.x, t0.y, t0.z, t0.w), ch ? (sp0 >> 16) : (sp0 & 0xFFFFu));
        mac_fast<NS>(acc1, af, make_uint4(t1.x, t1.y, t1.z, t1.w), ch ? (sp1 >> 16) : (sp1 & 0xFFFFu));
    }
}

// ws_gemm for two weight tiles at once (T holds two wave tiles).
template <int NS>
EM_DEV void ws_gemm2(floatx4 (&acc0)[NS], floatx4 (&acc1)[NS], const WsSrc& p0, const WsSrc& p1, int kw, ws_u4* T,
                     const WsAct& ar, int K) {
    WsSrc q0 = p0, q1 = p1;
    q0.w += kw / 2;
    q0.s += kw / 128;
    q1.w += kw / 2;
    q1.s += kw / 128;
    const int nb = K / WS_KB;
    ws_u4 a00, a01, a10, a11, b00, b01, b10, b11;   // set a: block b, set b: block b + 1 (tiles 0, 1)
    uint32_t as0, as1, bs0, bs1;
    ws_fetch(a00, a01, as0, q0, 0, nb);
    ws_fetch(a10, a11, as1, q1, 0, nb);
    ws_fetch(b00, b01, bs0, q0, 1, nb);
    ws_fetch(b10, b11, bs1, q1, 1, nb);
    for (int b = 0; b < nb; b += 2) {
        ws_block2<NS>(acc0, acc1, a00, a01, as0, a10, a11, as1, T, ar, b * WS_KB);
        ws_fetch(a00, a01, as0, q0, b + 2, nb);
        ws_fetch(a10, a11, as1, q1, b + 2, nb);
        ws_block2<NS>(acc0, acc1, b00, b01, bs0, b10, b11, bs1, T, ar, (b + 1) * WS_KB);
        ws_fetch(b00, b01, bs0, q0, b + 3, nb);
        ws_fetch(b10, b11, bs1, q1, b + 3, nb);
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

// ---- decode-tiled weights --------------------------------------------------------
// In the decode-tiled layout (defined in the public header) a 1 KB read of one
// 16-row tile returns to each lane the 32 codes its MFMA operand needs, and the
// tiles of a 128-row tile group follow each other block by block, so that the
// waves of a workgroup streaming one tile group read one contiguous region and
// no transposition through LDS is needed.  The loads are non-temporal: each
// weight byte is read once per step.
struct WsSrcT {
    const uint8_t* w;                   // this wave's tile at block 0, plus 16 lane
    const uint16_t* s;                  // scales of row lane % 16 of the tile (row-major, K / 128 per row)
};

// tg_q: the tile group's codes; tg_s: the scales of its row 0 (row-major, ks =
// K / 128 per row); t: the tile (0..7).
EM_DEV void ws_src_t(WsSrcT& p, const uint8_t* tg_q, const uint16_t* tg_s, int ks, int t) {
    const int l = lane_id();
    p.w = tg_q + (size_t)t * 2048 + 16 * l;
    p.s = tg_s + (size_t)(16 * t + (l & 15)) * ks;
}

// The codes of block b (clamped to nb - 1).
EM_DEV void ws_fetch_tq(ws_u4& w0, ws_u4& w1, const WsSrcT& p, int b, int nb) {
    const uint8_t* q = p.w + (size_t)min(b, nb - 1) * 16384;
    w0 = __builtin_nontemporal_load(reinterpret_cast<const ws_u4*>(q));
    w1 = __builtin_nontemporal_load(reinterpret_cast<const ws_u4*>(q + 1024));
}

// The codes and the scale pair of block b (clamped to nb - 1).
EM_DEV void ws_fetch_t(ws_u4& w0, ws_u4& w1, uint32_t& sp, const WsSrcT& p, int b, int nb) {
    const int bb = min(b, nb - 1);
    ws_fetch_tq(w0, w1, p, bb, nb);
    sp = *reinterpret_cast<const uint32_t*>(p.s + 2 * bb);
}

// The scale pairs of blocks [b0, b0 + 4) in one 16-byte load (b0 a multiple
// of 4; the row's scales 16-byte aligned).
EM_DEV ws_u4 ws_scales4_t(const WsSrcT& p, int b0) {
    return *reinterpret_cast<const ws_u4*>(p.s + 2 * b0);
}

// One block of a tiled tile: w0 / w1 are the MFMA operands of its two chunks.
template <int NS>
EM_DEV void ws_block_t(floatx4 (&acc)[NS], ws_u4 w0, ws_u4 w1, uint32_t spair, const WsAct& ar, int k0,
                       int boff = 0) {
    const int c = lane_id() >> 4;
    // both chunks' scales first: the register that held them is then free for
    // the load that refills this ring slot
    const float sc[2] = {16.0f * fp16_bits_to_f32((uint16_t)(spair & 0xFFFFu)),
                         16.0f * fp16_bits_to_f32((uint16_t)(spair >> 16))};
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const ws_u4 t = ch ? w1 : w0;
        uint4 af[NS][4];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int seg = (k0 >> 3) + (((16 * ch + 4 * c + s) ^ ar.sw[ms]) & 15) + ((16 * ch + 4 * c + s) & ~15);
                af[ms][s] = *reinterpret_cast<const uint4*>(ar.row[ms] + boff + 8 * seg);
            }
        mac_fast_f<NS>(acc, af, make_uint4(t.x, t.y, t.z, t.w), sc[ch]);
    }
}

// Two tiles of one wave against the same activation fragments (one set of A
// reads for both), over blocks [kw / 256, + K / 256) of the tiles and [0, K) of
// the staged activations; K a multiple of 512.
template <int NS>
EM_DEV void ws_block2_t(floatx4 (&acc0)[NS], floatx4 (&acc1)[NS], ws_u4 w00, ws_u4 w01, uint32_t sp0, ws_u4 w10,
                        ws_u4 w11, uint32_t sp1, const WsAct& ar, int k0) {
    const int c = lane_id() >> 4;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const ws_u4 t0 = ch ? w01 : w00;
        const ws_u4 t1 = ch ? w11 : w10;
        uint4 af[NS][4];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int seg = (k0 >> 3) + (((16 * ch + 4 * c + s) ^ ar.sw[ms]) & 15) + ((16 * ch + 4 * c + s) & ~15);
                af[ms][s] = *reinterpret_cast<const uint4*>(ar.row[ms] + 8 * seg);
            }
        mac_fast<NS>(acc0, af, make_uint4(t0.x, t0.y, t0.z, t0.w), ch ? (sp0 >> 16) : (sp0 & 0xFFFFu));
        mac_fast<NS>(acc1, af, make_uint4(t1.x, t1.y, t1.z, t1.w), ch ? (sp1 >> 16) : (sp1 & 0xFFFFu));
    }
}

template <int NS>
EM_DEV void ws_gemm2_t(floatx4 (&acc0)[NS], floatx4 (&acc1)[NS], const WsSrcT& p0, const WsSrcT& p1, int kw,
                       const WsAct& ar, int K) {
    const int b0 = kw / WS_KB, nb = b0 + K / WS_KB;
    ws_u4 a00, a01, a10, a11, c00, c01, c10, c11;      // set a: block b, set c: block b + 1 (tiles 0, 1)
    uint32_t as0, as1, cs0, cs1;
    ws_fetch_t(a00, a01, as0, p0, b0, nb);
    ws_fetch_t(a10, a11, as1, p1, b0, nb);
    ws_fetch_t(c00, c01, cs0, p0, b0 + 1, nb);
    ws_fetch_t(c10, c11, cs1, p1, b0 + 1, nb);
    for (int b = b0; b < nb; b += 2) {
        ws_block2_t<NS>(acc0, acc1, a00, a01, as0, a10, a11, as1, ar, (b - b0) * WS_KB);
        ws_fetch_t(a00, a01, as0, p0, b + 2, nb);
        ws_fetch_t(a10, a11, as1, p1, b + 2, nb);
        ws_block2_t<NS>(acc0, acc1, c00, c01, cs0, c10, c11, cs1, ar, (b + 1 - b0) * WS_KB);
        ws_fetch_t(c00, c01, cs0, p0, b + 3, nb);
        ws_fetch_t(c10, c11, cs1, p1, b + 3, nb);
    }
}

// ---- activation rows staged in pieces ------------------------------------------
// When the activation rows of a K range do not fit in LDS, the workgroup stages
// them in pieces (RP rows x SK elements, at most 32 KB, XOR-swizzled as above),
// two pieces resident: the one being read and the next, which is loaded into
// registers one piece ahead and written at the piece boundary.  The waves'
// weight streams run on across the boundary (a barrier with no memory fence:
// only this wave's LDS accesses are waited for), so a piece boundary costs one
// barrier, not a refill of the weight pipeline.
constexpr int WS_PIECE = 16384;          // elements per piece buffer (32 KB)

template <int RP, int NT>
struct WsPiece {
    // elements per row and piece: the largest power of two that fits, at most 1024
    static constexpr int SK = WS_PIECE / RP >= 1024 ? 1024 : (WS_PIECE / RP >= 512 ? 512 : 256);
    static constexpr int BPS = SK / WS_KB;              // weight blocks per piece
    static constexpr int NS = RP > 16 ? 2 : 1;          // 16-row MFMA subtiles
    static constexpr int U = RP * SK / 8 / NT;          // 16-byte loads per thread and piece
};

// This thread's share of a piece: global source at K = 0 and LDS offset.
template <int RP, int NT>
struct WsPieceSrc {
    const uint16_t* g[WsPiece<RP, NT>::U];
    int l[WsPiece<RP, NT>::U];
};

// rows[r] (r < RP): the activation row that staged row r holds.
template <int RP, int NT>
EM_DEV void ws_piece_src(WsPieceSrc<RP, NT>& q, const uint16_t* act, size_t stride, const int* rows) {
    using P = WsPiece<RP, NT>;
    constexpr int SPR = P::SK / 8;                      // 16-byte segments per staged row
#pragma unroll
    for (int u = 0; u < P::U; ++u) {
        const int i = (int)threadIdx.x + NT * u, r = i / SPR, sg = i % SPR;
        q.g[u] = act + (size_t)rows[r] * stride + 8 * sg;
        q.l[u] = r * P::SK + 8 * ((sg & ~15) | ((sg & 15) ^ (r & 15)));
    }
}

// Workgroup barrier that waits for this wave's LDS accesses only; the empty
// asm statements keep the compiler from moving memory accesses across it.
EM_DEV void ws_lds_barrier() {
    asm volatile("" ::: "memory");
    // vmcnt and expcnt left free, lgkmcnt = 0 (gfx9 encoding)
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// acc += (this wave's 16 weight rows) . A over K (a multiple of SK and of
// WS_RING blocks), with A's RP rows staged through xs (2 x WS_PIECE elements).  The
// weight loads run WS_RING blocks ahead in a ring of single-block register
// slots: a slot is refilled right after its block is consumed, and the loop
// body covers the whole ring, so no value moves between slots.  All NT
// threads of the workgroup call this with the same K.
constexpr int WS_RING = 4;

EM_DEV void ws_fetch_any(ws_u4& w0, ws_u4& w1, uint32_t& sp, const WsSrc& p, int b, int nb) {
    ws_fetch(w0, w1, sp, p, b, nb);
}
EM_DEV void ws_fetch_any(ws_u4& w0, ws_u4& w1, uint32_t& sp, const WsSrcT& p, int b, int nb) {
    ws_fetch_t(w0, w1, sp, p, b, nb);
}
template <int NS>
EM_DEV void ws_block_any(floatx4 (&acc)[NS], ws_u4 w0, ws_u4 w1, uint32_t sp, ws_u4* T, const WsAct& ar, int k0,
                         int boff, const WsSrc&) {
    ws_block<NS>(acc, w0, w1, sp, T, ar, k0, boff);
}
template <int NS>
EM_DEV void ws_block_any(floatx4 (&acc)[NS], ws_u4 w0, ws_u4 w1, uint32_t sp, ws_u4*, const WsAct& ar, int k0,
                         int boff, const WsSrcT&) {
    ws_block_t<NS>(acc, w0, w1, sp, ar, k0, boff);
}

template <int RP, int NT, int NS, class Src>
EM_DEV void ws_gemm_pieces(floatx4 (&acc)[NS], const Src& p, int K, const WsPieceSrc<RP, NT>& q, uint16_t* xs,
                           ws_u4* T) {
    using P = WsPiece<RP, NT>;
    static_assert(NS == P::NS, "subtiles of the staged rows");
    static_assert(WS_RING % P::BPS == 0, "piece boundaries fall on ring boundaries");
    const int li = lane_id() & 15;
    WsAct ar;
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) {
        const int r = min(ms * 16 + li, RP - 1);
        ar.row[ms] = xs + r * P::SK;
        ar.sw[ms] = r & 15;
    }
    const int nb = K / WS_KB, npc = K / P::SK;
    uint4 xa[P::U];
    auto piece_fetch = [&](int pc) {
        const int k = min(pc, npc - 1) * P::SK;         // past the end: the last piece again
#pragma unroll
        for (int u = 0; u < P::U; ++u) xa[u] = ld16(q.g[u] + k);
    };
    auto piece_store = [&](int buf) {
#pragma unroll
        for (int u = 0; u < P::U; ++u) *reinterpret_cast<uint4*>(xs + buf * WS_PIECE + q.l[u]) = xa[u];
    };
    piece_fetch(0);
    ws_u4 w0[WS_RING], w1[WS_RING];
    uint32_t sp[WS_RING];
    // tiled codes: the scale pairs of a ring turn (four blocks) in one load, a
    // turn ahead, issued before the turn's code refills (the same order in the
    // prologue, so that the loop's waits hold from the first turn on)
    constexpr bool TILED = std::is_same<Src, WsSrcT>::value;
    ws_u4 scc = {0u, 0u, 0u, 0u};
    if constexpr (TILED) {
        static_assert(WS_RING == 4, "four-block turns");
        scc = ws_scales4_t(p, 0);
        asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int j = 0; j < WS_RING; ++j) {
        if constexpr (TILED) {
            ws_fetch_tq(w0[j], w1[j], p, j, nb);
            asm volatile("" ::: "memory");
        } else {
            ws_fetch_any(w0[j], w1[j], sp[j], p, j, nb);
        }
    }
    piece_store(0);
    piece_fetch(1);
    ws_lds_barrier();
    for (int b = 0; b < nb; b += WS_RING) {
        ws_u4 scn = scc;
        if constexpr (TILED) {
            scn = ws_scales4_t(p, min(b + WS_RING, nb - WS_RING));
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int j = 0; j < WS_RING; ++j) {
            const int blk = b + j;
            const int buf = (blk / P::BPS) & 1;
            if constexpr (TILED) {
                const uint32_t spair = j == 0 ? scc.x : (j == 1 ? scc.y : (j == 2 ? scc.z : scc.w));
                ws_block_t<NS>(acc, w0[j], w1[j], spair, ar, (j % P::BPS) * WS_KB, buf * WS_PIECE);
                ws_fetch_tq(w0[j], w1[j], p, blk + WS_RING, nb);
            } else {
                ws_block_any<NS>(acc, w0[j], w1[j], sp[j], T, ar, (j % P::BPS) * WS_KB, buf * WS_PIECE, p);
                ws_fetch_any(w0[j], w1[j], sp[j], p, blk + WS_RING, nb);
            }
            if ((j + 1) % P::BPS == 0) {
                // piece boundary: the next piece goes into the other buffer
                // (read last in the piece before this one, which every wave has
                // left), then the one after it is fetched
                piece_store(buf ^ 1);
                ws_lds_barrier();
                piece_fetch(blk / P::BPS + 2);
            }
        }
        scc = scn;
    }
}

}  // namespace em
