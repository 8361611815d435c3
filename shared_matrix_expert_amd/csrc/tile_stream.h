// Workgroup-level weight streaming through LDS (gfx950).
//
// The cost of streaming int4 weights at decode batch sizes is set by how many
// cache lines each load instruction touches, not by the bytes: loading MFMA
// fragments straight from memory touches 16 half lines per kilobyte, and the
// activation and scale loads of every wave add several times more.  Here the
// 256 threads of a workgroup load a K-block of 64 weight rows as whole 256-byte
// row segments (full lines, coalesced), the block's scales in one 8-byte load
// per row and the activation rows once for the workgroup, store them in LDS in
// the MFMA operand layout, and each wave then reads its fragments from LDS.
// Two LDS buffers let the next block's global loads overlap this block's math.
#pragma once

#include "common.h"
#include "mfma_ops.h"

namespace em {

// KB: K elements per block (multiple of 128); NS: 16-row activation subtiles.
template <int NS, int KB>
struct StreamLds {
    static constexpr int NCH = KB / KC;                  // 128-element chunks per block
    static constexpr int AW = KB + 8;                    // padded activation row (elements)
    static constexpr int WP = NCH * 4 + 1;               // 16-byte slots per row, padded
    uint4 w[2][64][WP];                                  // [buf][row][chunk * 4 + lane group]
    uint16_t s[2][64][NCH];                              // one fp16 scale per row and chunk
    __attribute__((aligned(16))) uint16_t a[2][16 * NS][AW];
};

// Operands of one streamed product: 64 weight rows (rows past nw are not
// loaded and their results must not be stored) and up to 16*NS activation rows.
struct StreamArgs {
    const uint8_t* w;        // row 0 of the 64-row block, packed int4
    size_t w_stride;         // bytes between weight rows (K / 2)
    const uint16_t* s;       // scales of row 0
    size_t s_stride;         // elements between scale rows (K / gq)
    int nw;                  // valid weight rows (<= 64)
    int gq;                  // quant group (>= 128, a multiple of 128)
};

template <int NS, int KB>
struct StreamRegs {
    uint4 w[StreamLds<NS, KB>::NCH];                     // this thread's share of the weights
    uint2 s;                                             // scales (threads < 64)
    uint4 a[NS * KB / 128];                              // share of the activations
};

// Global -> registers for block [kb, kb + KB).  `arow` (LDS, 16*NS entries)
// holds the activation row pointers; rows past na are not loaded.
template <int NS, int KB>
EM_DEV void stream_fetch(StreamRegs<NS, KB>& r, const StreamArgs& sa, const uint16_t* const* arow, int na,
                         int kb) {
    constexpr int NCH = KB / KC;
    constexpr int SEG = KB / 32;                         // 16-byte segments per weight row
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int q = tid + 256 * i;
        const int row = q / SEG, seg = q % SEG;
        const int rr = row < sa.nw ? row : 0;
        r.w[i] = ld16(sa.w + rr * sa.w_stride + (kb >> 1) + 16 * seg);
    }
    if (tid < 64) {
        const int rr = tid < sa.nw ? tid : 0;
        const uint16_t* sp = sa.s + rr * sa.s_stride + kb / sa.gq;
        if (sa.gq == KC) {
            // NCH consecutive scales (NCH <= 4), 8-byte aligned when NCH == 4
            if constexpr (NCH == 4) {
                r.s = *reinterpret_cast<const uint2*>(sp);
            } else {
                uint32_t h[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < NCH; ++i) h[i] = sp[i];
                r.s = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
        } else {
            // one scale covers gq / 128 chunks
            uint32_t h[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < NCH; ++i) h[i] = sa.s[rr * sa.s_stride + (kb + i * KC) / sa.gq];
            r.s = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
    }
    constexpr int ASEG = KB / 8;                         // 16-byte segments per activation row
#pragma unroll
    for (int i = 0; i < NS * KB / 128; ++i) {
        const int q = tid + 256 * i;
        const int row = q / ASEG, seg = q % ASEG;
        const int rr = row < na ? row : 0;
        r.a[i] = ld16(arow[rr] + kb + 8 * seg);
    }
}

template <int NS, int KB>
EM_DEV void stream_store(StreamLds<NS, KB>& L, int buf, const StreamRegs<NS, KB>& r) {
    constexpr int NCH = KB / KC;
    constexpr int SEG = KB / 32;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int q = tid + 256 * i;
        const int row = q / SEG, seg = q % SEG;
        L.w[buf][row][seg] = r.w[i];
    }
    if (tid < 64) {
        const uint32_t h[4] = {r.s.x & 0xFFFFu, r.s.x >> 16, r.s.y & 0xFFFFu, r.s.y >> 16};
#pragma unroll
        for (int i = 0; i < NCH; ++i) L.s[buf][tid][i] = (uint16_t)h[i];
    }
    constexpr int ASEG = KB / 8;
#pragma unroll
    for (int i = 0; i < NS * KB / 128; ++i) {
        const int q = tid + 256 * i;
        const int row = q / ASEG, seg = q % ASEG;
        *reinterpret_cast<uint4*>(&L.a[buf][row][8 * seg]) = r.a[i];
    }
}

// This wave's 16 weight rows (16 wave + lane % 16) against the staged
// activation rows, for every chunk of the block in buffer `buf`.
template <int NS, int KB>
EM_DEV void stream_compute(floatx4 (&acc)[NS], const StreamLds<NS, KB>& L, int buf) {
    constexpr int NCH = KB / KC;
    const int lane = lane_id(), c = lane >> 4, li = lane & 15;
    const int row = wave_id() * 16 + li;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const uint4 raw = L.w[buf][row][ch * 4 + c];
        const uint32_t sb = L.s[buf][row][ch];
        uint4 af[NS][4];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                af[ms][s] = *reinterpret_cast<const uint4*>(&L.a[buf][ms * 16 + li][ch * KC + 32 * c + 8 * s]);
        mac_fast<NS>(acc, af, raw, sb);
    }
}

// acc += W[64 rows] . A over K range [k0, k1) (multiples of KB).  Every thread
// of the workgroup must call this; it synchronises the workgroup.
template <int NS, int KB>
EM_DEV void stream_gemm(floatx4 (&acc)[NS], StreamLds<NS, KB>& L, const StreamArgs& sa,
                        const uint16_t* const* arow, int na, int k0, int k1) {
    StreamRegs<NS, KB> r;
    stream_fetch<NS, KB>(r, sa, arow, na, k0);
    stream_store<NS, KB>(L, 0, r);
    __syncthreads();
    int buf = 0;
    for (int kb = k0; kb < k1; kb += KB) {
        const bool more = kb + KB < k1;
        if (more) stream_fetch<NS, KB>(r, sa, arow, na, kb + KB);
        stream_compute<NS, KB>(acc, L, buf);
        if (more) stream_store<NS, KB>(L, buf ^ 1, r);
        __syncthreads();
        buf ^= 1;
    }
}

}  // namespace em
