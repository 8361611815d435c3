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
// One wave per expert; every lane owns 8-element slices of the K axis, so the
// expert's weight row streams once through the wave (16 bytes per lane per
// step) and is applied to all T <= 16 tokens.  The T partial sums are reduced
// with a fixed butterfly, so results are reproducible.
template <int TMAX>
__global__ void __launch_bounds__(256)
router_logits_small(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                    const float* __restrict__ bias, float* __restrict__ logits,
                    int T, int d, int E) {
    const int lane = lane_id();
    const int e = blockIdx.x * 4 + wave_id();
    if (e >= E) return;
    double acc[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) acc[t] = 0.0;
    const uint16_t* wrow = wr + (size_t)e * d;
    for (int k0 = lane * 8; k0 < d; k0 += kWave * 8) {
        uint4 wv = *reinterpret_cast<const uint4*>(wrow + k0);
        double wd[8];
        const uint32_t wu[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wd[2 * i] = (double)bf16_to_f32(wu[i] & 0xFFFFu);
            wd[2 * i + 1] = (double)bf16_to_f32(wu[i] >> 16);
        }
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < T) {
                uint4 xv = *reinterpret_cast<const uint4*>(x + (size_t)t * d + k0);
                const uint32_t xu[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[t] = fma((double)bf16_to_f32(xu[i] & 0xFFFFu), wd[2 * i], acc[t]);
                    acc[t] = fma((double)bf16_to_f32(xu[i] >> 16), wd[2 * i + 1], acc[t]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        double v = acc[t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
        acc[t] = v;
    }
    if (lane < T) {
        double v = 0.0;
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
            if (t == lane) v = acc[t];
        float l = (float)v;
        if (bias) l = l + bias[e];
        logits[(size_t)lane * E + e] = l;
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
// One wave per token: k rounds of a wave-wide arg-max (larger logit, or equal
// logit and lower index), then the softmax over the selected logits in float64.
__global__ void __launch_bounds__(256)
router_topk(const float* __restrict__ logits, int32_t* __restrict__ topk_idx,
            float* __restrict__ topk_w, int T, int E, int k) {
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T) return;
    constexpr int MAXPER = 16;            // E <= 1024
    float v[MAXPER];
    const float* row = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        const int e = lane + kWave * i;
        v[i] = (e < E) ? row[e] : -INFINITY;
    }
    uint64_t taken = 0;                   // bit i: element lane + 64 i already selected
    float sel0 = 0.f, my_sel = 0.f;
    int my_idx = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < MAXPER; ++i) {
            const int e = lane + kWave * i;
            if (e < E && !((taken >> i) & 1ull)) {
                if (v[i] > bv || (v[i] == bv && e < bi)) { bv = v[i]; bi = e; }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oi = __shfl_xor(bi, off, kWave);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if ((bi & (kWave - 1)) == lane) taken |= 1ull << (bi / kWave);
        if (j == 0) sel0 = bv;
        if (lane == j) { my_sel = bv; my_idx = bi; }
    }
    double u = (lane < k) ? exp((double)my_sel - (double)sel0) : 0.0;
    double s = u;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
    // the butterfly gives every lane the same sum only up to rounding order;
    // take lane 0's value so that all weights share one denominator
    s = __shfl(s, 0, kWave);
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = my_idx;
        topk_w[(size_t)t * k + lane] = (float)(u / s);
    }
}

// -------------------------------------------------------------- launchers -------
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* bias,
                         float* logits, int32_t* idx, float* w, int T, int d, int E, int k,
                         hipStream_t stream) {
    if (T <= 4) {
        prof_begin(stream);
        router_logits_small<4><<<(E + 3) / 4, 256, 0, stream>>>(x, wr, bias, logits, T, d, E);
        prof_end(stream, "router_logits_small");
    } else if (T <= 16) {
        prof_begin(stream);
        router_logits_small<16><<<(E + 3) / 4, 256, 0, stream>>>(x, wr, bias, logits, T, d, E);
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
    router_topk<<<(T + 3) / 4, 256, 0, stream>>>(logits, idx, w, T, E, k);
    prof_end(stream, "router_topk");
    return hipGetLastError();
}

}  // namespace em
