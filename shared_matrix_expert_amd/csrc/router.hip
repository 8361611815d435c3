// Router: logits, top-k and renormalised softmax (steps a1, a2 of the layer).
//
// Each token activates the top 10 of 512 experts (the Chinese commentary page,
// section "145B 为什么不用同时装进显存"; byteiota "Edge0-145B: Run a 145B
// Open-Source Model on Your Laptop", Not Compression - Architecture).  The
// selection rule is a stated reading: fp32 logits equal to the correctly
// rounded exact dot product (bf16 x bf16 products are exact in float64 and the
// float64 accumulation is exact for the value ranges of these layers), plus an
// optional fp32 bias added in fp32; descending order, ties to the lower index;
// weights are the softmax over the selected k.
#include "common.h"
#include "kernels.h"

namespace em {

// -------------------------------------------------------------- small batches ----
// A workgroup of 4 waves takes 2 experts and up to 8 tokens: the tokens' rows
// are staged once in LDS, waves 2e and 2e + 1 stream the two halves of expert
// e's weight row (all loads issued before the arithmetic) and accumulate the
// exact bf16 products in float64.  Lane sums are reduced with a fixed
// butterfly and the two halves added through LDS, so the result is
// reproducible (and exact).  A verify batch reads the router weights once,
// spread over E/2 workgroups.
constexpr int RS_TOK = 8;
constexpr int RS_D = 4096;                // largest d of this path

__global__ void __launch_bounds__(256)
router_logits_small(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                    const float* __restrict__ bias, float* __restrict__ logits,
                    int T, int d, int E) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[RS_TOK][RS_D];
    __shared__ double part[2][RS_TOK];
    const int lane = lane_id(), wv = wave_id();
    const int ntg = (T + RS_TOK - 1) / RS_TOK;
    const int tg = blockIdx.x % ntg;
    const int e = (blockIdx.x / ntg) * 2 + (wv >> 1);
    const int half = wv & 1;
    const int t0 = tg * RS_TOK;
    const int nt = min(RS_TOK, T - t0);
    const int hd = d / 2;                          // elements per half (a multiple of 64)
    // every load is issued before the first LDS store (clamped addresses, zero
    // for rows past the batch), so the loads overlap
    constexpr int XV = RS_TOK * RS_D / (256 * 8);
    uint4 xv[XV];
#pragma unroll
    for (int u = 0; u < XV; ++u) {
        const int i = (threadIdx.x + 256 * u) * 8;
        const int t = min(i / d, nt - 1), kk = i % d;
        xv[u] = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + t) * d + kk);
    }
    const uint16_t* wrow = wr + (size_t)(e < E ? e : 0) * d + half * hd;
    uint4 wv8[RS_D / 2 / 512];
#pragma unroll
    for (int i = 0; i < RS_D / 2 / 512; ++i) {
        const int kk = (i * kWave + lane) * 8;
        const uint4 w = *reinterpret_cast<const uint4*>(wrow + min(kk, hd - 8));
        wv8[i] = (e < E && kk < hd) ? w : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < XV; ++u) {
        const int i = (threadIdx.x + 256 * u) * 8;
        if (i < RS_TOK * d) {
            const int t = i / d, kk = i % d;
            *reinterpret_cast<uint4*>(&xs[t][kk]) = t < nt ? xv[u] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __syncthreads();
    double acc[RS_TOK];
#pragma unroll
    for (int t = 0; t < RS_TOK; ++t) acc[t] = 0.0;
#pragma unroll
    for (int i = 0; i < RS_D / 2 / 512; ++i) {
        const int kk = (i * kWave + lane) * 8;
        if (kk >= hd) break;
        const uint32_t wu[4] = {wv8[i].x, wv8[i].y, wv8[i].z, wv8[i].w};
        double wd[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            wd[2 * q] = (double)bf16_to_f32(wu[q] & 0xFFFFu);
            wd[2 * q + 1] = (double)bf16_to_f32(wu[q] >> 16);
        }
#pragma unroll
        for (int t = 0; t < RS_TOK; ++t) {
            const uint4 xv = *reinterpret_cast<const uint4*>(&xs[t][half * hd + kk]);
            const uint32_t xu[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[t] = fma((double)bf16_to_f32(xu[q] & 0xFFFFu), wd[2 * q], acc[t]);
                acc[t] = fma((double)bf16_to_f32(xu[q] >> 16), wd[2 * q + 1], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < RS_TOK; ++t) {
        double v = acc[t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
        acc[t] = v;
    }
    if (half == 1 && lane < RS_TOK) {
        double v = acc[0];
#pragma unroll
        for (int t = 1; t < RS_TOK; ++t)
            if (t == lane) v = acc[t];
        part[wv >> 1][lane] = v;
    }
    __syncthreads();
    if (half == 0 && e < E && lane < nt) {
        double v = acc[0];
#pragma unroll
        for (int t = 1; t < RS_TOK; ++t)
            if (t == lane) v = acc[t];
        float l = (float)(v + part[wv >> 1][lane]);
        if (bias) l = l + bias[e];
        logits[(size_t)(t0 + lane) * E + e] = l;
    }
}

// ------------------------------------------------------- K-split small batches ----
// Up to 8 tokens, d = RK_NSL * 512.  A workgroup takes 8 experts and one K slice
// of 512: the slice of the tokens' rows and of the experts' rows is staged in
// LDS (16 KB instead of the whole x per workgroup), lane (t, e) of each wave
// forms the exact float64 dot product over a quarter of the slice, and the
// quarters are added in order.  The slice sums go to the workspace; the top-k
// kernel adds the slices in order and rounds once.  Every partial sum of exact
// bf16 products is exact in float64 here, as the whole sum is, so the logits
// are the same bits as the one-pass kernel's.
constexpr int RK_SLICE = 512;
constexpr int RK_NSL = 8;

__global__ void __launch_bounds__(256)
router_logits_split(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                    double* __restrict__ part, int T, int d, int E) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[8][RK_SLICE + 8];    // rows 1040 B apart
    __shared__ __attribute__((aligned(16))) uint16_t wsm[8][RK_SLICE + 8];
    __shared__ double red[3][kWave];
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    const int e0 = blockIdx.x * 8, k0 = blockIdx.y * RK_SLICE;
    uint4 xv[2], wv8[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = tid + 256 * u, r = q >> 6, seg = q & 63;
        xv[u] = *reinterpret_cast<const uint4*>(x + (size_t)min(r, T - 1) * d + k0 + 8 * seg);
        wv8[u] = *reinterpret_cast<const uint4*>(wr + (size_t)(e0 + r) * d + k0 + 8 * seg);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = tid + 256 * u, r = q >> 6, seg = q & 63;
        *reinterpret_cast<uint4*>(&xs[r][8 * seg]) = r < T ? xv[u] : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&wsm[r][8 * seg]) = wv8[u];
    }
    __syncthreads();
    const int t = lane & 7, e = lane >> 3;
    double acc = 0.0;
#pragma unroll 4
    for (int kk = wv * (RK_SLICE / 4); kk < (wv + 1) * (RK_SLICE / 4); kk += 8) {
        const uint4 a = *reinterpret_cast<const uint4*>(&xs[t][kk]);
        const uint4 b = *reinterpret_cast<const uint4*>(&wsm[e][kk]);
        const uint32_t au[4] = {a.x, a.y, a.z, a.w}, bu[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = fma((double)bf16_to_f32(au[q] & 0xFFFFu), (double)bf16_to_f32(bu[q] & 0xFFFFu), acc);
            acc = fma((double)bf16_to_f32(au[q] >> 16), (double)bf16_to_f32(bu[q] >> 16), acc);
        }
    }
    if (wv > 0) red[wv - 1][lane] = acc;
    __syncthreads();
    if (wv == 0 && t < T) {
        double sum = acc + red[0][lane];
        sum += red[1][lane];
        sum += red[2][lane];
        part[((size_t)blockIdx.y * T + t) * E + e0 + e] = sum;
    }
}

// -------------------------------------------------------------- large batches ----
// 128 tokens x 128 experts per workgroup, 8 x 8 float64 accumulators per thread,
// K staged through LDS in chunks of 16 as float64.  Thread (ty, tx) owns tokens
// ty + 16 i and experts tx + 16 j.
constexpr int RT_TILE = 128;
constexpr int RT_KC = 16;

__global__ void __launch_bounds__(256)
router_logits_tiled(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                    const float* __restrict__ bias, float* __restrict__ logits,
                    int T, int d, int E) {
    __shared__ double xs[RT_KC][RT_TILE];
    __shared__ double ws[RT_KC][RT_TILE];
    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
    const int t0 = blockIdx.x * RT_TILE, e0 = blockIdx.y * RT_TILE;
    double acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;

    // staging: 128 rows x 16 k = 2048 values per operand, 8 per thread
    const int srow = tid >> 1;            // 0..127
    const int skk = (tid & 1) * 8;        // 0 or 8
    for (int k0 = 0; k0 < d; k0 += RT_KC) {
        {
            const int t = t0 + srow;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < T) v = *reinterpret_cast<const uint4*>(x + (size_t)t * d + k0 + skk);
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xs[skk + 2 * i][srow] = (double)bf16_to_f32(u[i] & 0xFFFFu);
                xs[skk + 2 * i + 1][srow] = (double)bf16_to_f32(u[i] >> 16);
            }
            const int e = e0 + srow;
            uint4 w = make_uint4(0, 0, 0, 0);
            if (e < E) w = *reinterpret_cast<const uint4*>(wr + (size_t)e * d + k0 + skk);
            const uint32_t wu[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ws[skk + 2 * i][srow] = (double)bf16_to_f32(wu[i] & 0xFFFFu);
                ws[skk + 2 * i + 1][srow] = (double)bf16_to_f32(wu[i] >> 16);
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < RT_KC; ++kk) {
            double a[8], b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = xs[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = ws[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = t0 + ty + 16 * i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = e0 + tx + 16 * j;
            if (e >= E) continue;
            float l = (float)acc[i][j];
            if (bias) l = l + bias[e];
            logits[(size_t)t * E + e] = l;
        }
    }
}

// -------------------------------------------------------------- top-k -----------
// One wave per token.  A candidate is the 64-bit key (order-preserving bits of
// the logit, ~index): the larger key is the larger logit, or the equal logit
// with the lower index; 0 marks no candidate.  Each lane sorts its own keys
// (descending) once; a round takes the wave-wide maximum of the lanes' first
// keys with DPP row operations (no LDS), and the lane that held it shifts its
// list by one.  Then the softmax over the selected logits in float64.
EM_DEV uint64_t topk_key(float v, int i) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);     // order-preserving for non-NaN floats
    if (v == 0.0f) u = 0x80000000u;                      // +0 and -0 tie
    return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)i);
}

template <int CTRL, int ROW_MASK>
EM_DEV uint32_t dpp_max_u32(uint32_t x) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, ROW_MASK, 0xF, false);
    return o > x ? o : x;
}

// Maximum of an unsigned 32-bit value over the wave, the same value in every lane.
EM_DEV uint32_t wave_max_u32(uint32_t x) {
    x = dpp_max_u32<0xB1, 0xF>(x);       // quad_perm [1,0,3,2]
    x = dpp_max_u32<0x4E, 0xF>(x);       // quad_perm [2,3,0,1]
    x = dpp_max_u32<0x141, 0xF>(x);      // row_half_mirror
    x = dpp_max_u32<0x140, 0xF>(x);      // row_mirror
    x = dpp_max_u32<0x142, 0xA>(x);      // row_bcast:15
    x = dpp_max_u32<0x143, 0xC>(x);      // row_bcast:31: lane 63 holds the maximum
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Maximum key over the wave, the same value in every lane: the maximum of
// the upper halves (the logit bits), then, only when several lanes hold it,
// the maximum lower half (~index) among those lanes.
EM_DEV uint64_t wave_max_key(uint64_t x) {
    const uint32_t hi = (uint32_t)(x >> 32), lo = (uint32_t)x;
    const uint32_t mh = wave_max_u32(hi);
    const uint64_t tied = __ballot(hi == mh);
    uint32_t ml;
    if (__popcll(tied) == 1) ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, __ffsll((long long)tied) - 1);
    else ml = wave_max_u32(hi == mh ? lo : 0u);
    return ((uint64_t)mh << 32) | ml;
}

// Descending sort of N keys (N a power of two) with Batcher's odd-even merge
// network; every index is a compile-time constant, so the keys stay in registers.
template <int N>
EM_DEV void sort_desc(uint64_t (&k)[N]) {
#pragma unroll
    for (int p = 1; p < N; p <<= 1)
#pragma unroll
        for (int q = p; q >= 1; q >>= 1)
#pragma unroll
            for (int j = q % p; j + q < N; j += 2 * q)
#pragma unroll
                for (int i = 0; i < q; ++i)
                    if (i + j + q < N && (i + j) / (2 * p) == (i + j + q) / (2 * p)) {
                        const uint64_t a = k[i + j], b = k[i + j + q];
                        k[i + j] = a > b ? a : b;
                        k[i + j + q] = a > b ? b : a;
                    }
}

// b in the lanes set in `lanes`, a in the others: one v_cndmask per 32-bit
// half.  Written out so that the shift below stays a fixed set of selects
// (the compiler otherwise turns a select between neighbours into an indexed
// read, a compare chain per element).
EM_DEV uint64_t select_lanes(uint64_t a, uint64_t b, uint64_t lanes) {
    uint32_t lo, hi;
    asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(lo) : "v"((uint32_t)a), "v"((uint32_t)b), "s"(lanes));
    asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3"
                 : "=v"(hi) : "v"((uint32_t)(a >> 32)), "v"((uint32_t)(b >> 32)), "s"(lanes));
    return ((uint64_t)hi << 32) | lo;
}

// The selection of one token's top k from its logits (lane l holds experts
// l + 64 i), by one wave.
template <int MAXPER>
EM_DEV void topk_select(const float (&lv)[MAXPER], int t, int E, int k, int32_t* __restrict__ topk_idx,
                        float* __restrict__ topk_w) {
    const int lane = lane_id();
    uint64_t key[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        const int e = lane + kWave * i;
        key[i] = e < E ? topk_key(lv[i], e) : 0ull;
    }
    sort_desc<MAXPER>(key);
    float my_sel = 0.f, sel0 = 0.f;
    int my_idx = 0;
    for (int j = 0; j < k; ++j) {
        const uint64_t w = wave_max_key(key[0]);
        const int bi = (int)(~(uint32_t)w);
        const uint32_t hb = (uint32_t)(w >> 32);
        const float bv = __uint_as_float((hb & 0x80000000u) ? (hb & 0x7FFFFFFFu) : ~hb);
        if (j == 0) sel0 = bv;
        if (lane == j) { my_sel = bv; my_idx = bi; }
        const uint64_t won = __ballot(key[0] == w);      // keys are distinct: one lane
#pragma unroll
        for (int i = 0; i + 1 < MAXPER; ++i) key[i] = select_lanes(key[i], key[i + 1], won);
        key[MAXPER - 1] = select_lanes(key[MAXPER - 1], 0ull, won);
    }
    double u = (lane < k) ? exp((double)my_sel - (double)sel0) : 0.0;
    double s = u;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
    s = __shfl(s, 0, kWave);
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = my_idx;
        topk_w[(size_t)t * k + lane] = (float)(u / s);
    }
}

template <int MAXPER>
__global__ void __launch_bounds__(256)
router_topk(const float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
            int T, int E, int k) {
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T) return;
    const float* row = logits + (size_t)t * E;
    float lv[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) lv[i] = row[min(lane + kWave * i, E - 1)];
    topk_select<MAXPER>(lv, t, E, k, topk_idx, topk_w);
}

// One workgroup per token for the K-split logits: every thread adds the slice
// sums of two experts in slice order (all loads in flight), rounds once, adds
// the bias, and stores the logit (to LDS, and to `logits` when given); then
// one wave selects.
__global__ void __launch_bounds__(256)
router_topk_split(const double* __restrict__ part, const float* __restrict__ bias, float* __restrict__ logits,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int T, int E, int k) {
    __shared__ float lg[8 * kWave];
    const int t = blockIdx.x, tid = threadIdx.x;
    double pv[2][RK_NSL];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int sl = 0; sl < RK_NSL; ++sl)
            pv[h][sl] = part[((size_t)sl * T + t) * E + min(tid + 256 * h, E - 1)];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = tid + 256 * h;
        double sum = pv[h][0];
#pragma unroll
        for (int sl = 1; sl < RK_NSL; ++sl) sum += pv[h][sl];
        float l = (float)sum;
        if (e < E) {
            if (bias) l = l + bias[e];
            lg[e] = l;
            if (logits) logits[(size_t)t * E + e] = l;
        }
    }
    __syncthreads();
    if (wave_id() != 0) return;
    float lv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) lv[i] = lg[min(lane_id() + kWave * i, E - 1)];
    topk_select<8>(lv, t, E, k, topk_idx, topk_w);
}


// -------------------------------------------------------------- launchers -------
size_t router_split_bytes(int T, int E) { return (size_t)RK_NSL * T * E * sizeof(double); }

bool router_split_ok(int T, int d, int E) {
    return T <= 8 && d == RK_NSL * RK_SLICE && E % 8 == 0 && E <= 8 * kWave;
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* bias,
                         float* logits, double* part, int32_t* idx, float* w, int T, int d, int E, int k,
                         hipStream_t stream) {
    if (part && router_split_ok(T, d, E)) {
        prof_begin(stream);
        router_logits_split<<<dim3(E / 8, RK_NSL), 256, 0, stream>>>(x, wr, part, T, d, E);
        prof_end(stream, "router_logits_split");
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        prof_begin(stream);
        router_topk_split<<<T, 256, 0, stream>>>(part, bias, logits, idx, w, T, E, k);
        prof_end(stream, "router_topk");
        return hipGetLastError();
    }
    if (!logits) return hipErrorInvalidValue;
    if (T <= 2 * RS_TOK && d <= RS_D && d % 128 == 0) {
        const int ntg = (T + RS_TOK - 1) / RS_TOK;
        prof_begin(stream);
        router_logits_small<<<((E + 1) / 2) * ntg, 256, 0, stream>>>(x, wr, bias, logits, T, d, E);
        prof_end(stream, "router_logits_small");
    } else {
        dim3 grid((T + RT_TILE - 1) / RT_TILE, (E + RT_TILE - 1) / RT_TILE);
        prof_begin(stream);
        router_logits_tiled<<<grid, 256, 0, stream>>>(x, wr, bias, logits, T, d, E);
        prof_end(stream, "router_logits_tiled");
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    prof_begin(stream);
    if (E <= 8 * kWave) router_topk<8><<<(T + 3) / 4, 256, 0, stream>>>(logits, idx, w, T, E, k);
    else router_topk<16><<<(T + 3) / 4, 256, 0, stream>>>(logits, idx, w, T, E, k);
    prof_end(stream, "router_topk");
    return hipGetLastError();
}

}  // namespace em
