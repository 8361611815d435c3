// Expert-layer products (steps a4-a11): int4 grouped GEMMs with the dequant
// fused into the MFMA operand path, the low-rank and LoRA branches, the
// activation epilogue and the weighted combine.
//
// Each group of 64 experts shares two large matrices and every expert keeps a
// small set of its own parameters (launch post "Edge0-145B: Frontier AI
// Capabilities on Your Own Computer", Under the Hood, Architecture paragraph);
// the difference is taken as a rank-r additive delta and the base as int4 with
// a parallel bf16 LoRA branch (byteiota "Edge0-145B: Run a 145B Open-Source
// Model on Your Laptop", The Three Pillars, Recover-LoRA paragraph).  The
// shared up product is computed once per (token, group) - over the group's
// distinct tokens - and every weight byte is streamed once per task.
//
// Work decomposition: a task is (segment, up to 64 rows, 64 output columns);
// each of the 4 waves of a workgroup owns 16 output columns and streams those
// 16 weight rows over K in 128-element chunks: one 16-byte load per lane,
// exact int4 -> bf16 conversion in registers, 4 MFMA 16x16x32 per 16-row
// subtile, one fp16 group scale applied to the chunk's fp32 partial sum.
#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace em {

enum Mode { M_Z1 = 0, M_HS = 1, M_ACT = 2, M_Z2 = 3, M_OUT = 4 };

constexpr int TASK_ROWS = 64;
constexpr int NSUB = TASK_ROWS / 16;

EM_DEV int find_seg(const int32_t* __restrict__ pre, int n, int b) {
    if (b >= pre[n]) return -1;
    int lo = 0, hi = n;                       // pre[lo] <= b < pre[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= b) lo = mid; else hi = mid;
    }
    return lo;
}

struct Task {
    int seg;        // expert or group
    int rbeg, rend; // rows [rbeg, rend) of this task (row or unique-slot indices)
};

// Map blockIdx.x onto (segment, 64-row slice).  kind 0: experts' rows, kind 1:
// groups' unique tokens, kind 2: groups' rows.
EM_DEV bool get_task(const LayerArgs& a, int kind, Task& tk) {
    const int b = blockIdx.x;
    const int32_t* tiles = kind == 0 ? a.db.etile : (kind == 1 ? a.db.gtile_u : a.db.gtile_r);
    const int nseg = kind == 0 ? a.E : a.G;
    const int s = find_seg(tiles, nseg, b);
    if (s < 0) return false;
    int r0, r1;
    if (kind == 0) { r0 = a.db.eoff[s]; r1 = a.db.eoff[s + 1]; }
    else if (kind == 1) { r0 = a.db.uoff[s]; r1 = a.db.uoff[s + 1]; }
    else { r0 = a.db.eoff[s * a.P]; r1 = a.db.eoff[(s + 1) * a.P]; }
    const int m = b - tiles[s];
    tk.seg = s;
    tk.rbeg = r0 + m * TASK_ROWS;
    tk.rend = min(r1, tk.rbeg + TASK_ROWS);
    return tk.rbeg < tk.rend;
}

template <int MODE>
__global__ void __launch_bounds__(256)
expert_gemm(LayerArgs a) {
    constexpr int kind = (MODE == M_Z1 || MODE == M_ACT || MODE == M_Z2) ? 0 : (MODE == M_HS ? 1 : 2);
    Task tk;
    if (!get_task(a, kind, tk)) return;
    const int lane = lane_id();
    const int c = lane >> 4;
    const int li = lane & 15;
    const int n0 = (blockIdx.y * 4 + wave_id()) * 16;

    // ---- per-mode operands
    int N, K, gq, lda;
    const uint8_t* W;
    const uint16_t* S;
    const uint16_t* A;
    if constexpr (MODE == M_Z1) {
        N = a.r; K = a.d; gq = min(a.gq, K); lda = a.d; A = a.x;
        W = a.a_up + (size_t)tk.seg * a.r * (a.d / 2);
        S = a.a_up_s + (size_t)tk.seg * a.r * (K / gq);
    } else if constexpr (MODE == M_HS) {
        N = a.h; K = a.d; gq = min(a.gq, K); lda = a.d; A = a.x;
        W = a.s_up + (size_t)tk.seg * a.h * (a.d / 2);
        S = a.s_up_s + (size_t)tk.seg * a.h * (K / gq);
    } else if constexpr (MODE == M_ACT) {
        N = a.h; K = a.r; gq = min(a.gq, K); lda = a.r; A = a.z1;
        W = a.b_up + (size_t)tk.seg * a.h * (a.r / 2);
        S = a.b_up_s + (size_t)tk.seg * a.h * (K / gq);
    } else if constexpr (MODE == M_Z2) {
        N = a.r; K = a.h; gq = min(a.gq, K); lda = a.h; A = a.act;
        W = a.a_dn + (size_t)tk.seg * a.r * (a.h / 2);
        S = a.a_dn_s + (size_t)tk.seg * a.r * (K / gq);
    } else {
        N = a.d; K = a.h; gq = min(a.gq, K); lda = a.h; A = a.act;
        W = a.s_dn + (size_t)tk.seg * a.d * (a.h / 2);
        S = a.s_dn_s + (size_t)tk.seg * a.d * (K / gq);
    }
    if (n0 >= N) return;
    const int ncol = n0 + li;
    const bool nvalid = ncol < N;
    const uint8_t* wrow = W + (size_t)(nvalid ? ncol : 0) * (K / 2);
    const uint16_t* srow = S + (size_t)(nvalid ? ncol : 0) * (K / gq);

    const int rows = tk.rend - tk.rbeg;
    const int nsub = (rows + 15) >> 4;
    const uint16_t* arow[NSUB];
    bool avalid[NSUB];
#pragma unroll
    for (int ms = 0; ms < NSUB; ++ms) {
        const int i = ms * 16 + li;
        avalid[ms] = i < rows;
        const int r = tk.rbeg + (avalid[ms] ? i : 0);
        int src;
        if constexpr (MODE == M_Z1) src = a.db.row_tok[r];
        else if constexpr (MODE == M_HS) src = a.db.ut_tok[r];
        else src = r;
        arow[ms] = A + (size_t)src * lda;
    }

    floatx4 acc[NSUB];
#pragma unroll
    for (int ms = 0; ms < NSUB; ++ms) acc[ms] = zero4();

    // ---- main K loop, one chunk of loads in flight ahead of the math
    uint4 raw = nvalid ? load_b_i4(wrow, 32 * c, K) : zero_u4();
    uint4 af[NSUB][4];
#pragma unroll
    for (int ms = 0; ms < NSUB; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            af[ms][s] = (ms < nsub) ? load_a(arow[ms], 32 * c + 8 * s, K, avalid[ms]) : make_uint4(0, 0, 0, 0);
    for (int k0 = 0; k0 < K; k0 += KC) {
        const int kn = k0 + KC;
        uint4 raw_n = make_uint4(0, 0, 0, 0);
        uint4 af_n[NSUB][4];
        if (kn < K) {
            raw_n = nvalid ? load_b_i4(wrow, kn + 32 * c, K) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int ms = 0; ms < NSUB; ++ms)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    af_n[ms][s] = (ms < nsub) ? load_a(arow[ms], kn + 32 * c + 8 * s, K, avalid[ms])
                                              : make_uint4(0, 0, 0, 0);
        }
        mac_i4<NSUB>(acc, af, nsub, raw, load_scales(srow, k0, gq, min(KC, K - k0), nvalid), gq,
                     min(KC, K - k0), c);
        raw = raw_n;
#pragma unroll
        for (int ms = 0; ms < NSUB; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s) af[ms][s] = af_n[ms][s];
    }

    // ---- K extensions
    if constexpr (MODE == M_HS || MODE == M_OUT) {
        // LoRA branch: V[g] (bf16 [N][rL]) times the rounded LoRA input (bf16 [rows][rL])
        const int rLp = (a.rL + 7) & ~7;
        const uint16_t* Vrow = (MODE == M_HS ? a.lu_v + (size_t)tk.seg * a.h * a.rL
                                             : a.ld_v + (size_t)tk.seg * a.d * a.rL) +
                               (size_t)(nvalid ? ncol : 0) * a.rL;
        const uint16_t* Z = MODE == M_HS ? a.zl : a.zl2;
        for (int kb = 0; kb < a.rL; kb += 32) {
            const uint4 bv = nvalid ? load_b_bf16(Vrow, kb + 8 * c, a.rL) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int ms = 0; ms < NSUB; ++ms) {
                if (ms < nsub) {
                    const int i = ms * 16 + li;
                    const uint4 av = load_a(Z + (size_t)(tk.rbeg + (i < rows ? i : 0)) * rLp,
                                            kb + 8 * c, a.rL, i < rows);
                    acc[ms] = mfma_bf16(av, bv, acc[ms]);
                }
            }
        }
    }
    if constexpr (MODE == M_OUT) {
        // per-expert delta: B_dn[e] (int4 [d][r]) times R(A_dn[e] a) (bf16 [rows][r]),
        // one pass per distinct expert among the task's rows (rows are expert-sorted)
        const int gq_r = min(a.gq, a.r);
        int my_e = -1, prev_e = -1;
        if (lane < rows) my_e = a.db.row_exp[tk.rbeg + lane];
        if (lane >= 1 && lane - 1 < rows) prev_e = a.db.row_exp[tk.rbeg + lane - 1];
        uint64_t starts = __ballot(lane < rows && (lane == 0 || my_e != prev_e));
        while (starts) {
            const int p = __ffsll((long long)starts) - 1;
            starts &= starts - 1;
            const int pend = starts ? __ffsll((long long)starts) - 1 : rows;
            const int e = __shfl(my_e, p, kWave);
            const uint8_t* w2 = a.b_dn + (size_t)e * a.d * (a.r / 2) + (size_t)(nvalid ? ncol : 0) * (a.r / 2);
            const uint16_t* s2 = a.b_dn_s + (size_t)e * a.d * (a.r / gq_r) + (size_t)(nvalid ? ncol : 0) * (a.r / gq_r);
            for (int k0 = 0; k0 < a.r; k0 += KC) {
                const uint4 raw2 = nvalid ? load_b_i4(w2, k0 + 32 * c, a.r) : make_uint4(0, 0, 0, 0);
                uint4 af2[NSUB][4];
#pragma unroll
                for (int ms = 0; ms < NSUB; ++ms) {
                    const int i = ms * 16 + li;
                    const bool v = i >= p && i < pend;
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        af2[ms][s] = (ms < nsub) ? load_a(a.z2 + (size_t)(tk.rbeg + (v ? i : 0)) * a.r,
                                                          k0 + 32 * c + 8 * s, a.r, v)
                                                 : make_uint4(0, 0, 0, 0);
                }
                mac_i4<NSUB>(acc, af2, nsub, raw2, load_scales(s2, k0, gq_r, min(KC, a.r - k0), nvalid),
                             gq_r, min(KC, a.r - k0), c);
            }
        }
    }

    // ---- epilogue: lane holds rows 16 ms + 4 c + v, column ncol
    if (!nvalid) return;
#pragma unroll
    for (int ms = 0; ms < NSUB; ++ms) {
        if (ms >= nsub) break;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = ms * 16 + 4 * c + v;
            if (i >= rows) continue;
            const int r = tk.rbeg + i;
            const float val = acc[ms][v];
            if constexpr (MODE == M_Z1) {
                a.z1[(size_t)r * a.r + ncol] = (uint16_t)f32_to_bf16_rne(val);
            } else if constexpr (MODE == M_Z2) {
                a.z2[(size_t)r * a.r + ncol] = (uint16_t)f32_to_bf16_rne(val);
            } else if constexpr (MODE == M_HS) {
                a.hs[(size_t)r * a.h + ncol] = val;
            } else if constexpr (MODE == M_ACT) {
                const float hv = val + a.hs[(size_t)a.db.row_u[r] * a.h + ncol];
                a.act[(size_t)r * a.h + ncol] = (uint16_t)f32_to_bf16_rne(silu(hv));
            } else {
                a.o[(size_t)r * a.d + ncol] = val;
            }
        }
    }
}

// ------------------------------------------------------------------ LoRA inputs ----
// zl[u] = R(U_up[g] x[t_u]) for the distinct tokens of each group and
// zl2[row] = R(U_dn[g] a[row]) for the rows of each group.  N = rL <= 32, so
// the 4 waves split K (chunks of 32, round robin) and their partial sums are
// added in wave order through LDS.
template <int DOWN>
__global__ void __launch_bounds__(256)
lora_in(LayerArgs a) {
    __shared__ float red[4][2][NSUB][64][4];
    Task tk;
    if (!get_task(a, DOWN ? 2 : 1, tk)) return;
    const int lane = lane_id(), wv = wave_id();
    const int c = lane >> 4, li = lane & 15;
    const int K = DOWN ? a.h : a.d;
    const uint16_t* U = DOWN ? a.ld_u + (size_t)tk.seg * a.rL * a.h
                             : a.lu_u + (size_t)tk.seg * a.rL * a.d;
    const uint16_t* A = DOWN ? a.act : a.x;
    const int rows = tk.rend - tk.rbeg;
    const int nsub = (rows + 15) >> 4;
    const uint16_t* arow[NSUB];
    bool avalid[NSUB];
#pragma unroll
    for (int ms = 0; ms < NSUB; ++ms) {
        const int i = ms * 16 + li;
        avalid[ms] = i < rows;
        const int r = tk.rbeg + (avalid[ms] ? i : 0);
        arow[ms] = A + (size_t)(DOWN ? r : a.db.ut_tok[r]) * K;
    }
    floatx4 acc[2][NSUB];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ms = 0; ms < NSUB; ++ms) acc[nt][ms] = zero4();
    for (int k0 = 32 * wv; k0 < K; k0 += 128) {
        uint4 af[NSUB];
#pragma unroll
        for (int ms = 0; ms < NSUB; ++ms)
            af[ms] = ms < nsub ? load_a(arow[ms], k0 + 8 * c, K, avalid[ms]) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int n = nt * 16 + li;
            if (nt * 16 >= a.rL) break;
            const uint4 bv = n < a.rL ? *reinterpret_cast<const uint4*>(U + (size_t)n * K + k0 + 8 * c)
                                      : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int ms = 0; ms < NSUB; ++ms)
                if (ms < nsub) acc[nt][ms] = mfma_bf16(af[ms], bv, acc[nt][ms]);
        }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ms = 0; ms < NSUB; ++ms)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wv][nt][ms][lane][v] = acc[nt][ms][v];
    __syncthreads();
    if (wv != 0) return;
    const int rLp = (a.rL + 7) & ~7;
    uint16_t* Z = DOWN ? a.zl2 : a.zl;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int n = nt * 16 + li;
        if (n >= a.rL) continue;
#pragma unroll
        for (int ms = 0; ms < NSUB; ++ms) {
            if (ms >= nsub) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = ms * 16 + 4 * c + v;
                if (i >= rows) continue;
                const float s = ((red[0][nt][ms][lane][v] + red[1][nt][ms][lane][v]) +
                                 red[2][nt][ms][lane][v]) + red[3][nt][ms][lane][v];
                Z[(size_t)(tk.rbeg + i) * rLp + n] = (uint16_t)f32_to_bf16_rne(s);
            }
        }
    }
}

// ------------------------------------------------------------------ combine --------
// y[t] = sum_j w[t, j] o[row(t, j)], j = 0..k-1 in order; a gather, no atomics.
__global__ void __launch_bounds__(256)
combine(const float* __restrict__ o, const float* __restrict__ w, const int32_t* __restrict__ slot_row,
        float* __restrict__ y, int T, int d, int k) {
    const int64_t i = blockIdx.x * 256ll + threadIdx.x;     // float4 index
    const int d4 = d >> 2;
    if (i >= (int64_t)T * d4) return;
    const int t = (int)(i / d4), n4 = (int)(i % d4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const float wj = w[(size_t)t * k + j];
        const float4 v = reinterpret_cast<const float4*>(o + (size_t)slot_row[(size_t)t * k + j] * d)[n4];
        acc.x = fmaf(wj, v.x, acc.x);
        acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z);
        acc.w = fmaf(wj, v.w, acc.w);
    }
    reinterpret_cast<float4*>(y + (size_t)t * d)[n4] = acc;
}

// ------------------------------------------------------------------ residual -------
// x_out = bf16(x + y) with a single rounding: x (bf16) and y (fp32) sum exactly
// in float64 for the layer's value ranges, and the float64 is rounded straight
// to bf16 (nearest-even on the bit pattern) instead of through fp32.
EM_DEV uint32_t f64_to_bf16_rne(double v) {
    if (v == 0.0) return (uint32_t)(__double_as_longlong(v) >> 48) & 0x8000u;
    int e;
    frexp(v, &e);                             // |v| = m 2^e, m in [0.5, 1)
    const double ulp = ldexp(1.0, e - 8);     // bf16 spacing in v's binade
    const double r = rint(v / ulp) * ulp;     // exact scaling; rint is half-to-even
    return f32_to_bf16_rne((float)r);         // r is a bf16 value: both conversions are exact
}

__global__ void __launch_bounds__(256)
residual_add(const uint16_t* __restrict__ x, const float* __restrict__ y, uint16_t* __restrict__ xo,
             int64_t n) {
    const int64_t i = blockIdx.x * 256ll + threadIdx.x;
    if (i >= n) return;
    const double s = (double)bf16_to_f32(x[i]) + (double)y[i];
    xo[i] = (uint16_t)f64_to_bf16_rne(s);
}

// Plain copy, 16 bytes per thread per step, grid-stride.
__global__ void __launch_bounds__(256)
copy_bytes(uint4* __restrict__ dst, const uint4* __restrict__ src, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        dst[i] = src[i];
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const size_t want = (n16 + 255) / 256, cap = 256 * 16;
    const size_t blocks = want < cap ? want : cap;
    prof_begin(stream);
    copy_bytes<<<(unsigned)blocks, 256, 0, stream>>>(static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16);
    prof_end(stream, "copy_bytes");
    return hipGetLastError();
}

// Decode-tiled copy of the codes of G matrices of N x K (layout in the public
// header): one thread per 16-byte unit of the destination.  Grid-stride, reads
// and writes in bounds by construction.
__global__ void __launch_bounds__(256)
tile_shared_q(uint4* __restrict__ dst, const uint8_t* __restrict__ src, int G, int N, int K) {
    const size_t units = (size_t)G * N * K / 32;          // 16-byte units
    const size_t per_tg = (size_t)K * 4;                   // units per tile group (64 K bytes)
    const size_t per_g = (size_t)N / 128 * per_tg;
    for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (size_t)gridDim.x * 256) {
        const size_t g = u / per_g, rg = u % per_g;
        const size_t n = rg / per_tg, rt = rg % per_tg;
        const size_t b = rt / 1024, rb = rt % 1024;        // 1024 units per block (16 KB)
        const size_t t = rb / 128, c = (rb / 64) % 2, l = rb % 64;
        const size_t row = 128 * n + 16 * t + (l & 15);
        const size_t off = (g * N + row) * (size_t)(K / 2) + (2 * b + c) * 64 + 16 * (l >> 4);
        dst[u] = *reinterpret_cast<const uint4*>(src + off);
    }
}

// Column-blocked copy of M matrices N x K (packed int4): for matrix m and
// block cb of 128 K elements, the N rows' 64-byte segments follow each other,
// so one block of all N rows is one contiguous N * 64 bytes.
__global__ void __launch_bounds__(256)
colblock_q(uint4* __restrict__ dst, const uint8_t* __restrict__ src, int M, int N, int K) {
    const size_t units = (size_t)M * N * K / 32;          // 16-byte units
    const size_t per_cb = (size_t)N * 4;
    const size_t per_m = (size_t)(K / 128) * per_cb;
    for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (size_t)gridDim.x * 256) {
        const size_t m = u / per_m, rm = u % per_m;
        const size_t cb = rm / per_cb, rc = rm % per_cb;
        const size_t n = rc / 4, j = rc % 4;
        dst[u] = *reinterpret_cast<const uint4*>(src + (m * N + n) * (size_t)(K / 2) + cb * 64 + 16 * j);
    }
}

hipError_t launch_colblock(const uint8_t* src_q, uint8_t* dst_q, int M, int N, int K, hipStream_t stream) {
    const size_t units = (size_t)M * N * K / 32;
    const size_t bq = (units + 255) / 256 < 8192 ? (units + 255) / 256 : 8192;
    prof_begin(stream);
    colblock_q<<<(unsigned)bq, 256, 0, stream>>>(reinterpret_cast<uint4*>(dst_q), src_q, M, N, K);
    prof_end(stream, "colblock");
    return hipGetLastError();
}

hipError_t launch_tile_shared(const uint8_t* src_q, uint8_t* dst_q, int G, int N, int K, hipStream_t stream) {
    const size_t units = (size_t)G * N * K / 32;
    const size_t bq = (units + 255) / 256 < 8192 ? (units + 255) / 256 : 8192;
    prof_begin(stream);
    tile_shared_q<<<(unsigned)bq, 256, 0, stream>>>(reinterpret_cast<uint4*>(dst_q), src_q, G, N, K);
    prof_end(stream, "tile_shared");
    return hipGetLastError();
}

hipError_t launch_residual(int T, int d, const uint16_t* x, const float* y, uint16_t* x_out,
                           hipStream_t s) {
    const int64_t n = (int64_t)T * d;
    prof_begin(s);
    residual_add<<<(int)((n + 255) / 256), 256, 0, s>>>(x, y, x_out, n);
    prof_end(s, "residual_add");
    return hipGetLastError();
}

// ------------------------------------------------------------------ trace copies ---
// dst[s] = src[index[s]] for rows of `width` 16-bit units (a row copy by index).
__global__ void __launch_bounds__(256)
gather_rows_u16(const uint16_t* __restrict__ src, const int32_t* __restrict__ index,
                uint16_t* __restrict__ dst, int64_t rows, int64_t width) {
    const int64_t i = blockIdx.x * 256ll + threadIdx.x;
    if (i >= rows * width) return;
    const int64_t r = i / width, c = i % width;
    dst[i] = src[(int64_t)index[r] * width + c];
}

hipError_t launch_gather_rows(const void* src, const int32_t* index, void* dst, int64_t rows,
                              int64_t row_bytes, hipStream_t s) {
    const int64_t width = row_bytes / 2;
    const int64_t n = rows * width;
    gather_rows_u16<<<(int)((n + 255) / 256), 256, 0, s>>>((const uint16_t*)src, index,
                                                           (uint16_t*)dst, rows, width);
    return hipGetLastError();
}

// ------------------------------------------------------------------ launcher -------
template <int MODE>
static void launch_gemm(const LayerArgs& a, int tiles, int N, hipStream_t s, const char* name) {
    dim3 grid(tiles, (N + 63) / 64);
    prof_begin(s);
    expert_gemm<MODE><<<grid, 256, 0, s>>>(a);
    prof_end(s, name);
}

hipError_t launch_expert_layer(const LayerArgs& a, hipStream_t s) {
    // a4-a6 inputs: R1 (per row) and R2 (per distinct token of a group)
    const bool pf_z = a.pf && a.r == KC;                 // rank-128 inputs on the tiled GEMM
    if (pf_z) {
        const hipError_t e = launch_prefill_gemm(a, PF_Z1, a.rmax, s);
        if (e != hipSuccess) return e;
    } else {
        launch_gemm<M_Z1>(a, a.max_etiles, a.r, s, "gemm_z1");
    }
    launch_lora_in(a, 0, s);
    // a4 + a6: shared up + LoRA up, once per (token, group)
    if (a.pf) {
        hipError_t e = launch_gather_x(a, a.umax, s);
        if (e == hipSuccess) e = launch_prefill_gemm(a, PF_HS, a.umax, s);
        if (e != hipSuccess) return e;
    } else {
        launch_gemm<M_HS>(a, a.max_gtiles_u, a.h, s, "gemm_shared_up");
    }
    // a5 + a7: delta up, sum, SiLU, R3
    if (a.pf && a.r == KC && a.h % 256 == 0) {
        const hipError_t e = launch_act(a, s);
        if (e != hipSuccess) return e;
    } else {
        launch_gemm<M_ACT>(a, a.max_etiles, a.h, s, "gemm_delta_up_act");
    }
    // a9 / a10 inputs: R4 (per row), R5 (per row)
    if (pf_z) {
        const hipError_t e = launch_prefill_gemm(a, PF_Z2, a.rmax, s);
        if (e != hipSuccess) return e;
    } else {
        launch_gemm<M_Z2>(a, a.max_etiles, a.r, s, "gemm_z2");
    }
    launch_lora_in(a, 1, s);
    // a8 - a10: shared down + delta down + LoRA down
    if (a.pf) {
        const hipError_t e = launch_prefill_gemm(a, PF_OUT, a.rmax, s);
        if (e != hipSuccess) return e;
    } else {
        launch_gemm<M_OUT>(a, a.max_gtiles_r, a.d, s, "gemm_down");
    }
    return launch_combine(a, s);   // a11
}

void launch_lora_in(const LayerArgs& a, int down, hipStream_t s) {
    prof_begin(s);
    if (down) {
        lora_in<1><<<a.max_gtiles_r, 256, 0, s>>>(a);
        prof_end(s, "lora_in_down");
    } else {
        lora_in<0><<<a.max_gtiles_u, 256, 0, s>>>(a);
        prof_end(s, "lora_in_up");
    }
}

hipError_t launch_combine(const LayerArgs& a, hipStream_t s) {
    const int64_t n4 = (int64_t)a.T * (a.d / 4);
    prof_begin(s);
    combine<<<(int)((n4 + 255) / 256), 256, 0, s>>>(a.o, a.topk_w, a.db.slot_row, a.y, a.T, a.d, a.k);
    prof_end(s, "combine");
    return hipGetLastError();
}

}  // namespace em
