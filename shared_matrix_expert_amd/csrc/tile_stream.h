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
// loaded and their results must not be stored) and up to 16*NS activation rows
// a + arow[i] * a_stride (bf16).  The activation base is a plain global
// pointer and the row list holds indexes, so every load is a global load.
struct StreamArgs {
    const uint8_t* w;        // row 0 of the 64-row block, packed int4
    size_t w_stride;         // bytes between weight rows (K / 2)
    const uint16_t* s;       // scales of row 0
    size_t s_stride;         // elements between scale rows (K / gq)
    int nw;                  // valid weight rows (<= 64)
    int gq;                  // quant group (>= 128, a multiple of 128)
    const uint16_t* a;       // activation rows
    size_t a_stride;         // elements between activation rows
};

template <int NS, int KB>
struct StreamRegs {
    uint4 w[StreamLds<NS, KB>::NCH];                     // this thread's share of the weights
    uint32_t s;                                          // one scale
    uint4 a[NS * KB / 128];                              // share of the activations
};

// Per-thread sources, fixed for the whole K range: the weight row, the scale
// row and the activation rows this thread loads.  Rows past nw or na read a
// valid row again, so every load is unconditional: the loads of one block are
// a fixed sequence and the waits before the LDS stores count exactly the loads
// of the block still in flight behind them.
template <int NS, int KB>
struct StreamSrc {
    const uint8_t* w[StreamLds<NS, KB>::NCH];
    const uint16_t* s;
    const uint16_t* a[NS * KB / 128];
};

template <int NS, int KB>
EM_DEV void stream_src(StreamSrc<NS, KB>& p, const StreamArgs& sa, const int* arow, int na) {
    constexpr int NCH = KB / KC;
    constexpr int SEG = KB / 32;                         // 16-byte segments per weight row
    constexpr int ASEG = KB / 8;                         // 16-byte segments per activation row
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int q = tid + 256 * i;
        const int row = q / SEG, seg = q % SEG;
        p.w[i] = sa.w + (row < sa.nw ? row : 0) * sa.w_stride + 16 * seg;
    }
    const int srow = tid >> 2;
    p.s = sa.s + (srow < sa.nw ? srow : 0) * sa.s_stride;
#pragma unroll
    for (int i = 0; i < NS * KB / 128; ++i) {
        const int q = tid + 256 * i;
        const int row = q / ASEG, seg = q % ASEG;
        p.a[i] = sa.a + (size_t)arow[row < na ? row : 0] * sa.a_stride + 8 * seg;
    }
}

// Global -> registers for block [kb, kb + KB); the weight and scale rows are
// offset by woff bytes and soff elements (a later 64-row block).
template <int NS, int KB>
EM_DEV void stream_fetch(StreamRegs<NS, KB>& r, const StreamSrc<NS, KB>& p, int gq, int kb, size_t woff = 0,
                         size_t soff = 0) {
    constexpr int NCH = KB / KC;
#pragma unroll
    for (int i = 0; i < NCH; ++i) r.w[i] = ld16(p.w[i] + woff + (kb >> 1));
    // thread (row, chunk) = (tid / 4, tid % 4); chunks past NCH repeat the last
    const int ch = min((int)(threadIdx.x & 3), NCH - 1);
    r.s = p.s[soff + (kb + ch * KC) / gq];
#pragma unroll
    for (int i = 0; i < NS * KB / 128; ++i) r.a[i] = ld16(p.a[i] + kb);
}

// Activation rows past na hold copies of row 0: they only reach output rows
// that are never stored (an MFMA output row depends on its own A row alone).
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
    if ((tid & 3) < NCH) L.s[buf][tid >> 2][tid & 3] = (uint16_t)r.s;
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
// of the workgroup must call this; it synchronises the workgroup.  Global loads
// run two blocks ahead of the arithmetic (two register sets), so each block's
// load latency overlaps two blocks of work instead of one.
template <int NS, int KB>
EM_DEV void stream_gemm(floatx4 (&acc)[NS], StreamLds<NS, KB>& L, const StreamArgs& sa,
                        const int* arow, int na, int k0, int k1) {
    StreamSrc<NS, KB> p;
    stream_src<NS, KB>(p, sa, arow, na);
    StreamRegs<NS, KB> r0, r1;
    const int nb = (k1 - k0) / KB;
    // the second fetch is unconditional (a single block loads itself twice)
    stream_fetch<NS, KB>(r0, p, sa.gq, k0);
    stream_fetch<NS, KB>(r1, p, sa.gq, k0 + (nb > 1 ? KB : 0));
    stream_store<NS, KB>(L, 0, r0);
    __syncthreads();
    // Steady state: block b sits in LDS buffer 0, r1 holds block b + 1 and r0
    // receives block b + 2.  The loop only runs while blocks b + 2 and b + 3
    // exist, so its loads are unconditional and the waits exact.
    int b = 0;
    for (; b + 3 < nb; b += 2) {
        stream_fetch<NS, KB>(r0, p, sa.gq, k0 + (b + 2) * KB);
        stream_compute<NS, KB>(acc, L, 0);
        stream_store<NS, KB>(L, 1, r1);
        __syncthreads();
        stream_fetch<NS, KB>(r1, p, sa.gq, k0 + (b + 3) * KB);
        stream_compute<NS, KB>(acc, L, 1);
        stream_store<NS, KB>(L, 0, r0);
        __syncthreads();
    }
    // the last one, two or three blocks
    if (b + 2 < nb) {
        stream_fetch<NS, KB>(r0, p, sa.gq, k0 + (b + 2) * KB);
        stream_compute<NS, KB>(acc, L, 0);
        stream_store<NS, KB>(L, 1, r1);
        __syncthreads();
        stream_compute<NS, KB>(acc, L, 1);
        stream_store<NS, KB>(L, 0, r0);
        __syncthreads();
        stream_compute<NS, KB>(acc, L, 0);
    } else if (b + 1 < nb) {
        stream_compute<NS, KB>(acc, L, 0);
        stream_store<NS, KB>(L, 1, r1);
        __syncthreads();
        stream_compute<NS, KB>(acc, L, 1);
    } else {
        stream_compute<NS, KB>(acc, L, 0);
    }
    __syncthreads();
}

// Several 64-row weight blocks against the same activation rows: row block rb
// (0 <= rb < nrb) uses the weight rows sa.w + rb * rb_w (bytes) and scales
// sa.s + rb * rb_s (elements).  All (rb, K-block) steps run through one
// pipeline in (rb, kb) order, so the next row block's first loads overlap the
// current one's last blocks and the workgroup's start-up is paid once.
// epi(rb, acc) runs after row block rb's last step; acc is then reset.  Every
// thread of the workgroup must call this; it synchronises the workgroup.
template <int NS, int KB, class Epi>
EM_DEV void stream_gemm_rows(StreamLds<NS, KB>& L, const StreamArgs& sa, size_t rb_w, size_t rb_s, int nrb,
                             const int* arow, int na, int k0, int k1, Epi&& epi) {
    StreamSrc<NS, KB> p;
    stream_src<NS, KB>(p, sa, arow, na);
    const int nbk = (k1 - k0) / KB;
    const int nb = nrb * nbk;
    auto fetch = [&](StreamRegs<NS, KB>& r, int q) {
        const int rb = q / nbk, kb = q - rb * nbk;
        stream_fetch<NS, KB>(r, p, sa.gq, k0 + kb * KB, (size_t)rb * rb_w, (size_t)rb * rb_s);
    };
    floatx4 acc[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
    auto compute = [&](int buf, int q) {
        stream_compute<NS, KB>(acc, L, buf);
        const int rb = q / nbk;
        if (q - rb * nbk == nbk - 1) {
            epi(rb, acc);
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
        }
    };
    StreamRegs<NS, KB> r0, r1;
    fetch(r0, 0);
    fetch(r1, nb > 1 ? 1 : 0);
    stream_store<NS, KB>(L, 0, r0);
    __syncthreads();
    int b = 0;
    for (; b + 3 < nb; b += 2) {
        fetch(r0, b + 2);
        compute(0, b);
        stream_store<NS, KB>(L, 1, r1);
        __syncthreads();
        fetch(r1, b + 3);
        compute(1, b + 1);
        stream_store<NS, KB>(L, 0, r0);
        __syncthreads();
    }
    if (b + 2 < nb) {
        fetch(r0, b + 2);
        compute(0, b);
        stream_store<NS, KB>(L, 1, r1);
        __syncthreads();
        compute(1, b + 1);
        stream_store<NS, KB>(L, 0, r0);
        __syncthreads();
        compute(0, b + 2);
    } else if (b + 1 < nb) {
        compute(0, b);
        stream_store<NS, KB>(L, 1, r1);
        __syncthreads();
        compute(1, b + 1);
    } else {
        compute(0, b);
    }
    __syncthreads();
}

}  // namespace em
