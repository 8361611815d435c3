// Device pieces shared by the decode-batch kernels (decode.hip, layer.hip):
// routing views rebuilt in LDS from topk_idx, the cross-workgroup arrival and
// ordered-sum patterns, and the delta down over a pass of rows.
#pragma once

#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace em {

constexpr int DEC_RMAX = 1024;
constexpr int HS_RB = 2;          // 64-column blocks per shared-up workgroup (h / 64 a multiple)
constexpr int DEPTH = 4;

// ------------------------------------------------------------------ routing views --
struct RouteView {
    int16_t idx[DEC_RMAX];    // expert of each slot (E <= 1024)
    uint32_t ebits[32];
    unsigned long long tmask[64];
    int start[64];
    int16_t rows[DEC_RMAX];   // row -> slot (t*k + j)
    int8_t rtok[DEC_RMAX];    // row -> token (T <= 64)
    int nrows;
    int sel;
    uint32_t flag;
};

EM_DEV void rv_load(RouteView& v, const int32_t* __restrict__ idx, int R) {
    for (int i = threadIdx.x; i < R; i += blockDim.x) v.idx[i] = (int16_t)idx[i];
    __syncthreads();
}

// The xi-th smallest expert that any slot selected, or -1.
EM_DEV int rv_distinct_expert(RouteView& v, int R, int E, int xi) {
    const int nw = (E + 31) >> 5;
    if ((int)threadIdx.x < nw) v.ebits[threadIdx.x] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < R; i += blockDim.x) atomicOr(&v.ebits[v.idx[i] >> 5], 1u << (v.idx[i] & 31));
    __syncthreads();
    if (threadIdx.x == 0) {
        int sel = -1, acc = 0;
        for (int w = 0; w < nw; ++w) {
            const int pc = __popc(v.ebits[w]);
            if (xi < acc + pc) {
                uint32_t b = v.ebits[w];
                for (int r = xi - acc; r > 0; --r) b &= b - 1u;
                sel = w * 32 + __ffs(b) - 1;
                break;
            }
            acc += pc;
        }
        v.sel = sel;
    }
    __syncthreads();
    return v.sel;
}

// Number of distinct experts that any slot selected (builds v.ebits).
EM_DEV int rv_count_experts(RouteView& v, int R, int E) {
    const int nw = (E + 31) >> 5;
    if ((int)threadIdx.x < nw) v.ebits[threadIdx.x] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < R; i += blockDim.x) atomicOr(&v.ebits[v.idx[i] >> 5], 1u << (v.idx[i] & 31));
    __syncthreads();
    if (threadIdx.x == 0) {
        int n = 0;
        for (int w = 0; w < nw; ++w) n += __popc(v.ebits[w]);
        v.sel = n;
    }
    __syncthreads();
    const int n = v.sel;
    __syncthreads();
    return n;
}

// The xi-th smallest selected expert (v.ebits built by rv_count_experts).
EM_DEV int rv_nth_expert(RouteView& v, int E, int xi) {
    if (threadIdx.x == 0) {
        const int nw = (E + 31) >> 5;
        int sel = -1, acc = 0;
        for (int w = 0; w < nw; ++w) {
            const int pc = __popc(v.ebits[w]);
            if (xi < acc + pc) {
                uint32_t b = v.ebits[w];
                for (int r = xi - acc; r > 0; --r) b &= b - 1u;
                sel = w * 32 + __ffs(b) - 1;
                break;
            }
            acc += pc;
        }
        v.sel = sel;
    }
    __syncthreads();
    const int e = v.sel;
    __syncthreads();
    return e;
}

// Rows of expert e (one per token that chose it) in token order.
EM_DEV int rv_expert_rows(RouteView& v, int e, int T, int k) {
    if (threadIdx.x < 64) {
        const int t = threadIdx.x;
        int slot = -1;
        if (t < T)
            for (int j = 0; j < k; ++j)
                if (v.idx[t * k + j] == e) slot = t * k + j;
        const unsigned long long m = __ballot(slot >= 0);
        if (slot >= 0) {
            const int pos = __popcll(m & ((1ull << t) - 1ull));
            v.rows[pos] = slot;
            v.rtok[pos] = t;
        }
        if (t == 0) v.nrows = __popcll(m);
    }
    __syncthreads();
    return v.nrows;
}

// Distinct tokens of group g in token order (rows[] = rtok[] = token).
EM_DEV int rv_group_tokens(RouteView& v, int g, int T, int k, int P) {
    if (threadIdx.x < 64) {
        const int t = threadIdx.x;
        bool in = false;
        if (t < T)
            for (int j = 0; j < k; ++j) in |= (v.idx[t * k + j] / P) == g;
        const unsigned long long m = __ballot(in);
        if (in) {
            const int pos = __popcll(m & ((1ull << t) - 1ull));
            v.rows[pos] = t;
            v.rtok[pos] = t;
        }
        if (t == 0) v.nrows = __popcll(m);
    }
    __syncthreads();
    return v.nrows;
}

// Slots of group g sorted by (expert, token).
EM_DEV int rv_group_rows(RouteView& v, int g, int T, int k, int P, int R) {
    if (threadIdx.x < 64) v.tmask[threadIdx.x] = 0ull;
    __syncthreads();
    for (int i = threadIdx.x; i < R; i += blockDim.x) {
        const int e = v.idx[i];
        if (e / P == g) atomicOr(&v.tmask[e - g * P], 1ull << (i / k));
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int l = threadIdx.x;
        const int cnt = l < P ? __popcll(v.tmask[l]) : 0;
        int x = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (l >= off) x += y;
        }
        v.start[l] = x - cnt;
        if (l == 63) v.nrows = x;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < R; i += blockDim.x) {
        const int e = v.idx[i];
        if (e / P == g) {
            const int el = e - g * P, t = i / k;
            const int r = v.start[el] + __popcll(v.tmask[el] & ((1ull << t) - 1ull));
            v.rows[r] = i;
            v.rtok[r] = t;
        }
    }
    __syncthreads();
    return v.nrows;
}

// Whether any slot selected an expert of group g (cheap test before building rows).
EM_DEV bool rv_group_any(RouteView& v, int g, int P, int R) {
    int c = 0;
    for (int i = threadIdx.x; i < R; i += blockDim.x) c += (v.idx[i] / P) == g;
    return __syncthreads_count(c > 0) != 0;
}

// Cross-workgroup data of the arrival patterns below is written and read with
// agent-scope relaxed atomic accesses, which are coherent across the XCDs'
// L2s without an L2 write-back or invalidation (a release or acquire fence at
// agent scope would flush or invalidate the whole L2 of the XCD, and every
// workgroup would pay for it).
EM_DEV void st_agent(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
EM_DEV float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Count this workgroup's arrival at `counter` once its agent-scope stores have
// completed, and return (to every thread) whether it arrived last of `expected`.
EM_DEV bool arrive_last(RouteView& v, uint32_t* counter, uint32_t expected) {
    __builtin_amdgcn_s_waitcnt(0);        // this wave's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v.flag = (old == expected - 1u) ? 1u : 0u;
    }
    __syncthreads();
    return v.flag != 0u;
}

// Sum of n partials at p[0], p[stride], ... in index order, read with agent
// scope, loads issued eight at a time.
EM_DEV float ordered_sum_agent(const float* p, int n, size_t stride) {
    float sum = 0.f;
    for (int s0 = 0; s0 < n; s0 += 8) {
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = ld_agent(p + (size_t)min(s0 + u, n - 1) * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < n) sum += t[u];
    }
    return sum;
}


// Delta-down weights of four experts (this lane's 16 bytes and scale each).
struct DnRing {
    uint4 w[4];
    uint32_t s[4];
};

// Reorders the 8 bf16 of an A fragment to the K order (0,4,1,5,2,6,3,7) that
// dq_offset produces for the B side.
EM_DEV uint4 k_interleave(uint4 v) {
    return make_uint4((v.x & 0xFFFFu) | (v.z << 16), (v.x >> 16) | (v.z & 0xFFFF0000u),
                      (v.y & 0xFFFFu) | (v.w << 16), (v.y >> 16) | (v.w & 0xFFFF0000u));
}

// Eight two's-complement int4 codes q of one 32-bit word to four bf16 pairs
// holding 136 + q exactly: flipping each nibble's sign bit gives q + 8 in
// 0..15, which becomes the low mantissa bits below the exponent of 128.  The
// pairs come out in the K order (0,4,1,5,2,6,3,7).
// Each pair is one three-input bit operation, (v & M) ^ K: M = 0x000F000F keeps
// the two nibbles, and K = 0x43084308 is the exponent pattern 0x4300 of each
// half (which shares no bits with M, so ORing it in is an XOR) together with
// the sign-bit flip 0x0008.  The truth table of f(src0, src1, src2) is f
// evaluated on the bytes 0xF0, 0xCC, 0xAA: (0xF0 & 0xCC) ^ 0xAA = 0x6A.
EM_DEV uint4 dq_offset(uint32_t w) {
    constexpr uint32_t M = 0x000F000Fu, K = 0x43084308u;
    constexpr unsigned char AND_XOR = 0x6A;
    return make_uint4(__builtin_amdgcn_bitop3_b32(w, M, K, AND_XOR), __builtin_amdgcn_bitop3_b32(w >> 4, M, K, AND_XOR),
                      __builtin_amdgcn_bitop3_b32(w >> 8, M, K, AND_XOR), __builtin_amdgcn_bitop3_b32(w >> 12, M, K, AND_XOR));
}

// dq_offset with the pairs in natural K order: out[i] = (136 + q[2i]) |
// (136 + q[2i + 1]) << 16.  A byte permute puts byte i of w (low nibble
// q[2i]) at byte 0 and byte i of w >> 4 (low nibble q[2i + 1]) at byte 2; the
// same three-input operation as above then masks, flips and offsets both.
EM_DEV uint4 dq_offset_nat(uint32_t w) {
    constexpr uint32_t M = 0x000F000Fu, K = 0x43084308u;
    constexpr unsigned char AND_XOR = 0x6A;
    const uint32_t u = w >> 4;
    return make_uint4(__builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(u, w, 0x0C040C00u), M, K, AND_XOR),
                      __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(u, w, 0x0C050C01u), M, K, AND_XOR),
                      __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(u, w, 0x0C060C02u), M, K, AND_XOR),
                      __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(u, w, 0x0C070C03u), M, K, AND_XOR));
}

// Delta down for the rows of one pass (sorted by expert): acc[ms] (output rows
// ms*16 + 4c + q, this lane's column ncol) += B_dn[e(row)][ncol] . z2[row].
// Expert u of the pass (dexp[u], rows [dstart[u], dstart[u + 1])) owns the rows
// whose rank (expert starts at or before the row, less one) is u.  Each
// expert's product runs over the z2 rows of the 16-row subtiles that hold its
// rows, and only its own rows' outputs are kept.  The codes enter the MFMA as
// 136 + q (exact in bf16), so the product is corrected by 136 times the row
// sums of z2 (one product against a ones operand); both operands take the K
// order of dq_offset.  The B_dn rows of four experts are in flight while four are used.
template <int NS>
EM_DEV void delta_down_pass(floatx4 (&acc)[NS], const DecodeArgs& a, const int* dexp, const int* dstart,
                            uint64_t starts, int prow, const int (&slot_i)[NS], int ncol, int ub = 0,
                            int ue = DEC_RMAX) {
    const int nexp = __popcll(starts);
    ue = min(ue, nexp);
    if (ub >= ue) return;
    const int lane = lane_id(), c = lane >> 4;
    uint4 af[NS][4];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s) af[ms][s] = k_interleave(ld16(a.z2 + (size_t)slot_i[ms] * KC + 32 * c + 8 * s));
    // expert rank of each output row (-1 past the pass's rows)
    int rko[NS][4];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = ms * 16 + 4 * c + q;
            rko[ms][q] = i < prow ? __popcll(starts & ((2ull << i) - 1ull)) - 1 : -1;
        }
    floatx4 zc[NS];
    {
        const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
            floatx4 t = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) t = mfma_bf16(af[ms][s], ones, t);
#pragma unroll
            for (int q = 0; q < 4; ++q) zc[ms][q] = 136.0f * t[q];
        }
    }
    auto fetch = [&](DnRing& r, int u0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = dexp[min(u0 + q, ue - 1)];
            r.w[q] = ld16(a.b_dn + ((size_t)e * a.d + ncol) * (KC / 2) + 16 * c);
            r.s[q] = a.b_dn_s[(size_t)e * a.d + ncol];
        }
    };
    auto consume = [&](const DnRing& r, int u0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int u = u0 + q;
            if (u >= ue) break;
            const int r0 = dstart[u], r1 = u + 1 < nexp ? dstart[u + 1] : prow;
            uint4 b[4];
            b[0] = dq_offset(r.w[q].x);
            b[1] = dq_offset(r.w[q].y);
            b[2] = dq_offset(r.w[q].z);
            b[3] = dq_offset(r.w[q].w);
            const float sc = fp16_bits_to_f32((uint16_t)r.s[q]);
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) {
                if (r1 <= 16 * ms || r0 >= 16 * ms + 16) continue;
                floatx4 t = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) t = mfma_bf16(af[ms][s], b[s], t);
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    acc[ms][qq] = fmaf(rko[ms][qq] == u ? sc : 0.0f, t[qq] - zc[ms][qq], acc[ms][qq]);
            }
        }
    };
    DnRing d0, d1;
    fetch(d0, ub);
    int u0 = ub;
    for (; u0 + 8 <= ue; u0 += 8) {
        fetch(d1, u0 + 4);
        consume(d0, u0);
        fetch(d0, u0 + 8);
        consume(d1, u0 + 4);
    }
    if (u0 < ue) {
        fetch(d1, u0 + 4);
        consume(d0, u0);
        consume(d1, u0 + 4);
    }
}


}  // namespace em
