// Wave-level operand loaders and int4 MAC steps shared by the GEMM kernels.
//
// K-slot mappings (both operands of an MFMA must use the same one):
//  * int4 chunk of 128: lane group c = lane/16 owns chunk elements
//    [32c, 32c+32) (one 16-byte load), MFMA s uses [32c + 8s, 32c + 8s + 8);
//  * bf16 step of 32: lane group c owns elements [8c, 8c+8).
#pragma once

#include "common.h"

namespace em {

constexpr int KC = 128;

EM_DEV uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// int4 weights: 32 elements [kk, kk+32) of one row (kk multiple of 32), as 4 dwords.
EM_DEV uint4 load_b_i4(const uint8_t* __restrict__ row, int kk, int K) {
    uint4 v = zero_u4();
    if (kk >= K) return v;
    if ((K & 31) == 0) return *reinterpret_cast<const uint4*>(row + (kk >> 1));
    const uint32_t* p = reinterpret_cast<const uint32_t*>(row + (kk >> 1));
    if (kk + 0 < K) v.x = p[0];
    if (kk + 8 < K) v.y = p[1];
    if (kk + 16 < K) v.z = p[2];
    if (kk + 24 < K) v.w = p[3];
    return v;
}

// bf16 weights: elements [kk, kk+8) of one row (K even), zero beyond K.
EM_DEV uint4 load_b_bf16(const uint16_t* __restrict__ row, int kk, int K) {
    uint4 v = zero_u4();
    const uint32_t* p = reinterpret_cast<const uint32_t*>(row + kk);
    if (kk + 0 < K) v.x = p[0];
    if (kk + 2 < K) v.y = p[1];
    if (kk + 4 < K) v.z = p[2];
    if (kk + 6 < K) v.w = p[3];
    return v;
}

// bf16 activations: elements [kk, kk+8) of a row whose storage is padded to a
// multiple of 8 elements; elements >= K read as zero.
EM_DEV uint4 load_a(const uint16_t* __restrict__ row, int kk, int K, bool valid) {
    uint4 v = zero_u4();
    if (!valid || kk >= K) return v;
    v = *reinterpret_cast<const uint4*>(row + kk);
    const int n = K - kk;                     // valid elements, > 0
    if (n < 8) {
        uint32_t* u = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (2 * i >= n) u[i] = 0u;
            else if (2 * i + 1 >= n) u[i] &= 0xFFFFu;
        }
    }
    return v;
}

EM_DEV void dequant_b(uint4 raw, uint4 b[4]) {
    uint32_t q[4][4];
    dequant8(raw.x, q[0]);
    dequant8(raw.y, q[1]);
    dequant8(raw.z, q[2]);
    dequant8(raw.w, q[3]);
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = make_uint4(q[s][0], q[s][1], q[s][2], q[s][3]);
}

// fp16 scale bits of the chunk at kk: one scale when the chunk lies in a single
// quant group (gq >= kvalid), else the kvalid/gq (<= 4) scales of the chunk.
EM_DEV uint2 load_scales(const uint16_t* __restrict__ srow, int kk, int gq, int kvalid, bool nvalid) {
    uint2 s = make_uint2(0u, 0u);
    if (!nvalid) return s;
    if (gq >= kvalid) {
        s.x = srow[kk / gq];
    } else {
        const int ng = kvalid / gq, i0 = kk / gq;
        uint32_t h[4] = {0u, 0u, 0u, 0u};
        for (int i = 0; i < ng; ++i) h[i] = srow[i0 + i];
        s.x = h[0] | (h[1] << 16);
        s.y = h[2] | (h[3] << 16);
    }
    return s;
}

EM_DEV float scale16(uint2 s, int i) {
    const uint32_t w = (i < 2) ? s.x : s.y;
    return 16.0f * fp16_bits_to_f32((uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

// One 128-wide int4 chunk: acc[ms] += scale * (A[ms] . W) for the active
// subtiles.  With quant groups narrower than the chunk (32 or 64) each group
// gets its own pass in which the A lanes of other groups are zero, so every
// partial sum carries a single scale.
template <int NS>
EM_DEV void mac_i4(floatx4 (&acc)[NS], const uint4 (&af)[NS][4], int nsub, uint4 raw, uint2 sbits,
                   int gq, int kvalid, int c) {
    uint4 b[4];
    dequant_b(raw, b);
    if (gq >= kvalid) {
        const float sc = scale16(sbits, 0);
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
            if (ms < nsub) {
                floatx4 t = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) t = mfma_bf16(af[ms][s], b[s], t);
                acc[ms] = fma4(sc, t, acc[ms]);
            }
        }
    } else {
        const int ng = kvalid / gq;
        const int lanes_per = gq / 32;
        const uint4 z = zero_u4();
        for (int gi = 0; gi < ng; ++gi) {
            const bool mine = (c / lanes_per) == gi;
            const float sc = scale16(sbits, gi);
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) {
                if (ms < nsub) {
                    floatx4 t = zero4();
#pragma unroll
                    for (int s = 0; s < 4; ++s) t = mfma_bf16(mine ? af[ms][s] : z, b[s], t);
                    acc[ms] = fma4(sc, t, acc[ms]);
                }
            }
        }
    }
}

// A fragments of one int4 chunk at kk for every active subtile.
template <int NS>
EM_DEV void load_afrag_i4(uint4 (&af)[NS][4], const uint16_t* const (&arow)[NS],
                          const bool (&av)[NS], int nsub, int kk, int K, int c) {
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            af[ms][s] = ms < nsub ? load_a(arow[ms], kk + 32 * c + 8 * s, K, av[ms]) : zero_u4();
}

// Stream 16 int4 weight rows (this lane: row `wrow`) over K range [kb, ke)
// against up to NS*16 activation rows, with DEPTH chunks of weights and
// scales in flight ahead of the math and the next chunk's activations
// prefetched.  kb and ke are multiples of 128 (ke may equal K < 128).
template <int NS, int DEPTH>
EM_DEV void stream_i4(floatx4 (&acc)[NS], const uint8_t* __restrict__ wrow,
                      const uint16_t* __restrict__ srow, bool nvalid, int kb, int ke, int K, int gq,
                      const uint16_t* const (&arow)[NS], const bool (&av)[NS], int nsub, int c) {
    uint4 ring[DEPTH];
    uint2 sring[DEPTH];
#pragma unroll
    for (int p = 0; p < DEPTH; ++p) {
        const int kk = kb + p * KC;
        const bool in = nvalid && kk < ke;
        ring[p] = in ? load_b_i4(wrow, kk + 32 * c, K) : zero_u4();
        sring[p] = in ? load_scales(srow, kk, gq, min(KC, K - kk), true) : make_uint2(0u, 0u);
    }
    uint4 af[NS][4];
    load_afrag_i4<NS>(af, arow, av, nsub, kb, K, c);
    for (int k0 = kb; k0 < ke; k0 += DEPTH * KC) {
#pragma unroll
        for (int p = 0; p < DEPTH; ++p) {
            const int kk = k0 + p * KC;
            if (kk < ke) {
                uint4 afn[NS][4];
                if (kk + KC < ke) load_afrag_i4<NS>(afn, arow, av, nsub, kk + KC, K, c);
                const uint4 cur = ring[p];
                const uint2 scur = sring[p];
                const int kn = kk + DEPTH * KC;
                const bool in = nvalid && kn < ke;
                ring[p] = in ? load_b_i4(wrow, kn + 32 * c, K) : zero_u4();
                sring[p] = in ? load_scales(srow, kn, gq, min(KC, K - kn), true) : make_uint2(0u, 0u);
                mac_i4<NS>(acc, af, nsub, cur, scur, gq, min(KC, K - kk), c);
                if (kk + KC < ke) {
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                        for (int s = 0; s < 4; ++s) af[ms][s] = afn[ms][s];
                }
            }
        }
    }
}

// ---------------------------------------------------------------- fast path ------
// Branch-free streaming for K a multiple of 128 and quant groups of >= 128
// elements (one scale per chunk).  Every load goes to a valid address (the
// caller points out-of-range rows or columns at row 0, whose results are never
// stored) so that the compiler keeps the loads in flight instead of waiting at
// the joins of divergent branches.

EM_DEV uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

template <int NS>
EM_DEV void mac_fast(floatx4 (&acc)[NS], const uint4 (&af)[NS][4], uint4 raw, uint32_t sbits) {
    uint4 b[4];
    dequant_b(raw, b);
    const float sc = 16.0f * fp16_bits_to_f32((uint16_t)sbits);
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) {
        floatx4 t = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) t = mfma_bf16(af[ms][s], b[s], t);
        acc[ms] = fma4(sc, t, acc[ms]);
    }
}

// mac_fast with the chunk's scale already converted (16 s as a float).
template <int NS>
EM_DEV void mac_fast_f(floatx4 (&acc)[NS], const uint4 (&af)[NS][4], uint4 raw, float sc16) {
    uint4 b[4];
    dequant_b(raw, b);
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) {
        floatx4 t = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) t = mfma_bf16(af[ms][s], b[s], t);
        acc[ms] = fma4(sc16, t, acc[ms]);
    }
}

template <int NS>
EM_DEV void load_afrag_fast(uint4 (&af)[NS][4], const uint16_t* const (&arow)[NS], int kk, int c) {
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s) af[ms][s] = ld16(arow[ms] + kk + 32 * c + 8 * s);
}

// acc += W[rows of this lane's column] . A over chunks [kb, ke); requires
// (ke - kb) / 128 to be a multiple of DEPTH and gq >= 128.
template <int NS, int DEPTH>
EM_DEV void stream_i4_fast(floatx4 (&acc)[NS], const uint8_t* __restrict__ wrow,
                           const uint16_t* __restrict__ srow, int kb, int ke, int gq,
                           const uint16_t* const (&arow)[NS], int c) {
    const int nch = (ke - kb) / KC;
    uint4 ring[DEPTH];
    uint32_t sring[DEPTH];
#pragma unroll
    for (int p = 0; p < DEPTH; ++p) {
        const int kk = kb + p * KC;
        ring[p] = ld16(wrow + ((kk + 32 * c) >> 1));
        sring[p] = srow[kk / gq];
    }
    uint4 af[NS][4];
    load_afrag_fast<NS>(af, arow, kb, c);
    for (int i = 0; i < nch; i += DEPTH) {
#pragma unroll
        for (int p = 0; p < DEPTH; ++p) {
            const int ch = i + p;
            const int kn = kb + min(ch + 1, nch - 1) * KC;      // next chunk (clamped)
            uint4 afn[NS][4];
            load_afrag_fast<NS>(afn, arow, kn, c);
            const uint4 cur = ring[p];
            const uint32_t scur = sring[p];
            const int kr = kb + min(ch + DEPTH, nch - 1) * KC;  // refill (clamped)
            ring[p] = ld16(wrow + ((kr + 32 * c) >> 1));
            sring[p] = srow[kr / gq];
            mac_fast<NS>(acc, af, cur, scur);
#pragma unroll
            for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                for (int s = 0; s < 4; ++s) af[ms][s] = afn[ms][s];
        }
    }
}

// Sum of n float32 values at p[0], p[stride], ... in index order, with the
// loads issued eight at a time ahead of the additions.
EM_DEV float ordered_sum(const float* __restrict__ p, int n, size_t stride) {
    float sum = 0.f;
    for (int s0 = 0; s0 < n; s0 += 8) {
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = p[(size_t)min(s0 + u, n - 1) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < n) sum += t[u];
    }
    return sum;
}

}  // namespace em
