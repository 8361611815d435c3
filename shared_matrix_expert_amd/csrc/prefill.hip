// Shared-matrix products of large batches (steps a4 and a8-a10): LDS-tiled
// int4 x bf16 GEMMs on the matrix cores.
//
// Every group of 64 experts shares one up and one down matrix (launch post
// "Edge0-145B: Frontier AI Capabilities on Your Own Computer", Under the Hood,
// Architecture paragraph), so a prefill batch turns the shared part of the
// layer into one dense GEMM per group and matrix: the group's distinct tokens
// times S_up (up), the group's rows times S_dn (down).  At 16K tokens these
// two GEMMs are ~95 % of the layer's flops.
//
// Tile: 256 rows x 128 columns per workgroup of 4 waves (2 x 2, each wave 128
// rows x 64 columns = 8 x 4 MFMA 16x16 subtiles), K in steps of 128 = one
// quant group.  The activation tile (256 x 128 bf16 = 64 KB) moves from global
// memory straight into LDS (global_load_lds_dwordx4, no registers), double
// buffered, with the 16-byte slots of each row XOR-swizzled by the row so that
// the MFMA fragment reads are free of bank conflicts.  The int4 weights go
// into LDS the same way (128 columns x 64 bytes per step) and each wave converts
// its 64 columns exactly to bf16 in registers; every 128-element chunk is accumulated in
// a fresh fp32 tile and added to the result times 16 x its fp16 scale, so the
// weight values are exactly q x s.
//
// Workgroup order: blockIdx is remapped so that each XCD (blockIdx mod 8) runs
// a contiguous range of tiles, columns fastest: the workgroups that share an
// activation tile run together on one XCD and read it from that XCD's L2.
#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace em {

namespace {

constexpr int BM = 256, BN = 128, BK = 128;
constexpr int SLOTS = BK / 8;                    // 16-byte slots per activation row

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

struct PfTile {
    int g;          // group
    int r0, r1;     // rows [r0, r1) of the tile (r1 - r0 <= BM)
    int n0;         // first output column
};

// Tile b of the launch: row tiles of the groups in group order, columns fastest.
template <int MODE>
EM_DEV bool pf_tile(const LayerArgs& a, int b, int ntn, PfTile& t) {
    int m = b / ntn;
    t.n0 = (b % ntn) * BN;
    for (int g = 0; g < a.G; ++g) {
        const int r0 = MODE == PF_HS ? a.db.uoff[g] : a.db.eoff[g * a.P];
        const int r1 = MODE == PF_HS ? a.db.uoff[g + 1] : a.db.eoff[(g + 1) * a.P];
        const int nt = (r1 - r0 + BM - 1) / BM;
        if (m < nt) {
            t.g = g;
            t.r0 = r0 + m * BM;
            t.r1 = min(r1, t.r0 + BM);
            return true;
        }
        m -= nt;
    }
    return false;
}

// Activation tile for K step k0 into LDS: 256 rows x 16 slots.  Wave w, round
// i covers rows 16 i + 4 w .. + 3 (1 KB, lane-contiguous); lane l writes slot
// l % 16 of row 16 i + 4 w + l / 16 and fetches the row's global segment
// (l % 16) ^ (row % 16).  Rows past r1 repeat row r1 - 1.
EM_DEV void pf_fetch_a(uint4* As, const uint16_t* A, size_t lda, int r0, int r1, int k0) {
    const int w = wave_id(), l = lane_id();
    const int rsub = 4 * w + (l >> 4);
    const int seg = (l & 15) ^ (rsub & 15);
#pragma unroll
    for (int i = 0; i < BM / 16; ++i) {
        const int row = r0 + 16 * i + rsub;
        const uint16_t* src = A + (size_t)min(row, r1 - 1) * lda + k0 + 8 * seg;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(As + (16 * i + 4 * w) * SLOTS), 16, 0, 0);
    }
}

// Weight tile for K step k0 into LDS: 128 columns x 64 bytes (one int4 chunk
// per column), 4 slots of 16 bytes per column with slot = c ^ ((col / 4) % 4)
// holding the column's bytes [16c, 16c + 16), so that 16 lanes reading 16
// consecutive columns hit 16 distinct bank groups.  Wave w, round i covers
// columns 32 i + 16 w .. + 15 ... (two 1 KB rounds per wave).
EM_DEV void pf_fetch_b(uint4* Bs, const uint8_t* W, size_t wstride, int k0) {
    const int w = wave_id(), l = lane_id();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int col = 64 * i + 16 * w + (l >> 2);
        const int cseg = (l & 3) ^ ((col >> 2) & 3);
        const uint8_t* src = W + (size_t)col * wstride + (k0 >> 1) + 16 * cseg;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(Bs + (64 * i + 16 * w) * 4), 16, 0, 0);
    }
}

// acc[i][j] += (A rows of subtile i) x (16 x scale_j x dequant(B_j)) over one chunk.
EM_DEV void pf_compute(floatx4 (&acc)[8][4], const uint4* As, const uint4* Bs, const uint32_t (&sbits)[4],
                       int wm, int wn) {
    const int l = lane_id(), c = l >> 4, li = l & 15;
    uint4 bq[4][4];
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = 64 * wn + 16 * j + li;
        dequant_b(Bs[col * 4 + (c ^ ((col >> 2) & 3))], bq[j]);
        sc[j] = 16.0f * fp16_bits_to_f32((uint16_t)sbits[j]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 128 * wm + 16 * i + li;
        uint4 af[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) af[s] = As[row * SLOTS + ((4 * c + s) ^ li)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            floatx4 t = mfma_bf16(af[0], bq[j][0], zero4());
            t = mfma_bf16(af[1], bq[j][1], t);
            t = mfma_bf16(af[2], bq[j][2], t);
            t = mfma_bf16(af[3], bq[j][3], t);
            acc[i][j] = sc[j] * t + acc[i][j];
        }
    }
}

EM_DEV void pf_fetch_s(uint32_t (&sb)[4], const uint16_t* srow0, size_t sstride, int gq, int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) sb[j] = srow0[(size_t)(16 * j) * sstride + k0 / gq];
}

}  // namespace

template <int MODE>
__global__ void __launch_bounds__(256)
pf_gemm(LayerArgs a) {
    __shared__ uint4 As0[BM * SLOTS];
    __shared__ uint4 As1[BM * SLOTS];
    __shared__ uint4 Bs0[BN * 4];
    __shared__ uint4 Bs1[BN * 4];
    const int ntn = (MODE == PF_HS ? a.h : a.d) / BN;
    // XCD-aware order: XCD x = blockIdx % 8 takes tiles [x * per, (x + 1) * per)
    const int per = gridDim.x >> 3;
    const int b = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    PfTile t;
    if (!pf_tile<MODE>(a, b, ntn, t)) return;

    const int K = MODE == PF_HS ? a.d : a.h;
    const int N = MODE == PF_HS ? a.h : a.d;
    const int gq = min(a.gq, K);
    const uint16_t* A = MODE == PF_HS ? a.xg : a.act;
    const uint8_t* W = MODE == PF_HS ? a.s_up : a.s_dn;
    const uint16_t* S = MODE == PF_HS ? a.s_up_s : a.s_dn_s;
    const int l = lane_id(), wv = wave_id(), c = l >> 4, li = l & 15;
    const int wm = wv >> 1, wn = wv & 1;

    const uint8_t* Wt = W + ((size_t)t.g * N + t.n0) * (K / 2);          // the tile's 128 weight rows
    const uint16_t* srow0 = S + ((size_t)t.g * N + t.n0 + 64 * wn + li) * (K / gq);
    const size_t sstride = (size_t)(K / gq);

    floatx4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

    // ---- main loop: step k in buffers k % 2, the next step's loads in flight
    uint32_t s0[4], s1[4];
    pf_fetch_a(As0, A, (size_t)K, t.r0, t.r1, 0);
    pf_fetch_b(Bs0, Wt, (size_t)(K / 2), 0);
    pf_fetch_s(s0, srow0, sstride, gq, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int k0 = 0; k0 < K; k0 += 2 * BK) {
        // even step: buffers 0
        if (k0 + BK < K) {
            pf_fetch_a(As1, A, (size_t)K, t.r0, t.r1, k0 + BK);
            pf_fetch_b(Bs1, Wt, (size_t)(K / 2), k0 + BK);
            pf_fetch_s(s1, srow0, sstride, gq, k0 + BK);
        }
        pf_compute(acc, As0, Bs0, s0, wm, wn);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (k0 + BK >= K) break;
        // odd step: buffers 1
        if (k0 + 2 * BK < K) {
            pf_fetch_a(As0, A, (size_t)K, t.r0, t.r1, k0 + 2 * BK);
            pf_fetch_b(Bs0, Wt, (size_t)(K / 2), k0 + 2 * BK);
            pf_fetch_s(s0, srow0, sstride, gq, k0 + 2 * BK);
        }
        pf_compute(acc, As1, Bs1, s1, wm, wn);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- LoRA branch: V[g] (bf16 [N][rL]) x the rounded LoRA input rows (bf16 [rows][rLp])
    const int rLp = (a.rL + 7) & ~7;
    {
        const uint16_t* V = (MODE == PF_HS ? a.lu_v : a.ld_v) + (size_t)t.g * N * a.rL;
        const uint16_t* Z = MODE == PF_HS ? a.zl : a.zl2;
        for (int kb = 0; kb < a.rL; kb += 32) {
            const bool kv = kb + 8 * c < a.rL;
            uint4 bv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = t.n0 + 64 * wn + 16 * j + li;
                bv[j] = kv ? ld16(V + (size_t)n * a.rL + kb + 8 * c) : zero_u4();
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = min(t.r0 + 128 * wm + 16 * i + li, t.r1 - 1);
                const uint4 av = kv ? ld16(Z + (size_t)row * rLp + kb + 8 * c) : zero_u4();
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(av, bv[j], acc[i][j]);
            }
        }
    }

    // ---- per-expert delta down: B_dn[e] (int4 [d][r]) x R4 rows of expert e
    if constexpr (MODE == PF_OUT) {
        const int gq_r = min(a.gq, a.r);
        const int e_first = a.db.row_exp[t.r0], e_last = a.db.row_exp[t.r1 - 1];
        for (int e = e_first; e <= e_last; ++e) {
            const int p = max(a.db.eoff[e], t.r0) - t.r0;          // tile rows [p, q) are expert e's
            const int q = min(a.db.eoff[e + 1], t.r1) - t.r0;
            if (p >= q) continue;
            for (int k0 = 0; k0 < a.r; k0 += KC) {
                uint4 bq[4][4];
                float sc[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const size_t n = (size_t)e * a.d + t.n0 + 64 * wn + 16 * j + li;
                    dequant_b(ld16(a.b_dn + n * (a.r / 2) + (k0 >> 1) + 16 * c), bq[j]);
                    sc[j] = 16.0f * fp16_bits_to_f32(a.b_dn_s[n * (a.r / gq_r) + k0 / gq_r]);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int rl = 128 * wm + 16 * i;                  // subtile rows [rl, rl + 16)
                    if (rl + 16 <= p || rl >= q) continue;             // wave-uniform
                    const int row = rl + li;
                    const bool mine = row >= p && row < q;
                    const uint16_t* zr = a.z2 + (size_t)(t.r0 + (mine ? row : p)) * a.r + k0 + 32 * c;
                    uint4 af[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) af[s] = mine ? ld16(zr + 8 * s) : zero_u4();
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        floatx4 tt = mfma_bf16(af[0], bq[j][0], zero4());
                        tt = mfma_bf16(af[1], bq[j][1], tt);
                        tt = mfma_bf16(af[2], bq[j][2], tt);
                        tt = mfma_bf16(af[3], bq[j][3], tt);
                        acc[i][j] = sc[j] * tt + acc[i][j];
                    }
                }
            }
        }
    }

    // ---- store: lane holds rows 16 i + 4 c + v, column 16 j + li of its wave's block
    float* out = MODE == PF_HS ? a.hs : a.o;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = t.r0 + 128 * wm + 16 * i + 4 * c + v;
            if (row >= t.r1) continue;
            float* orow = out + (size_t)row * N + t.n0 + 64 * wn + li;
#pragma unroll
            for (int j = 0; j < 4; ++j) orow[16 * j] = acc[i][j][v];
        }
}

// xg[u] = x[ut_tok[u]]: the activation rows of every group's distinct tokens,
// contiguous per group, 16 bytes per thread.
__global__ void __launch_bounds__(256)
pf_gather_x(const uint16_t* __restrict__ x, const int32_t* __restrict__ ut_tok, const int32_t* __restrict__ n_u,
            uint16_t* __restrict__ xg, int d, int64_t umax) {
    const int segs = d / 8;
    const int64_t i = blockIdx.x * 256ll + threadIdx.x;
    if (i >= umax * segs) return;
    const int64_t u = i / segs;
    if (u >= *n_u) return;
    const int s = (int)(i % segs);
    reinterpret_cast<uint4*>(xg + u * d)[s] = reinterpret_cast<const uint4*>(x + (size_t)ut_tok[u] * d)[s];
}

bool prefill_gemm_ok(int d, int h, int r, int rL, int gq) {
    return gq % KC == 0 && r % KC == 0 && rL % 8 == 0 && rL <= 32 && d % BN == 0 && h % BN == 0 &&
           d % BK == 0 && h % BK == 0;
}

hipError_t launch_prefill_gemm(const LayerArgs& a, int mode, int64_t max_rows, hipStream_t s) {
    const int ntn = (mode == PF_HS ? a.h : a.d) / BN;
    const int64_t mt = max_rows / BM + a.G + 1;          // >= sum over groups of ceil(rows_g / BM)
    int64_t blocks = mt * ntn;
    blocks = (blocks + 7) & ~7ll;
    prof_begin(s);
    if (mode == PF_HS) {
        pf_gemm<PF_HS><<<(unsigned)blocks, 256, 0, s>>>(a);
        prof_end(s, "pf_shared_up");
    } else {
        pf_gemm<PF_OUT><<<(unsigned)blocks, 256, 0, s>>>(a);
        prof_end(s, "pf_down");
    }
    return hipGetLastError();
}

hipError_t launch_gather_x(const LayerArgs& a, int64_t umax, hipStream_t s) {
    const int64_t n = umax * (a.d / 8);
    prof_begin(s);
    pf_gather_x<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a.x, a.db.ut_tok, a.db.uoff + a.G, a.xg, a.d, umax);
    prof_end(s, "pf_gather_x");
    return hipGetLastError();
}

}  // namespace em
