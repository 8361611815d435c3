// C-ABI entry points: validation, workspace layout and launch sequencing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "edge_moe.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int check_dims(const edge_moe_dims* p) {
    if (!p) return EDGE_MOE_EINVAL;
    const edge_moe_dims& d = *p;
    if (d.T < 1 || d.d < 1 || d.h < 1 || d.n_experts < 1 || d.experts_per_group < 1 ||
        d.top_k < 1 || d.delta_rank < 1 || d.lora_rank < 1 || d.quant_group < 1)
        return EDGE_MOE_EINVAL;
    if (d.n_experts % d.experts_per_group != 0) return EDGE_MOE_EINVAL;
    if (d.top_k > d.n_experts) return EDGE_MOE_EINVAL;
    if ((d.d & 1) || (d.h & 1) || (d.delta_rank & 1)) return EDGE_MOE_EINVAL;
    const int Ks[3] = {d.d, d.h, d.delta_rank};
    for (int K : Ks) {
        const int g = d.quant_group < K ? d.quant_group : K;
        if (K % g != 0) return EDGE_MOE_EINVAL;
    }
    // limits of the kernels
    if (d.T > (1 << 20)) return EDGE_MOE_EUNSUPPORTED;
    if (d.d % 128 || d.h % 128 || d.d > 32768 || d.h > 32768) return EDGE_MOE_EUNSUPPORTED;
    if (d.n_experts > 1024 || d.n_experts / d.experts_per_group > 64) return EDGE_MOE_EUNSUPPORTED;
    if (d.top_k > 32) return EDGE_MOE_EUNSUPPORTED;
    if (d.delta_rank % 8 || d.delta_rank > 256) return EDGE_MOE_EUNSUPPORTED;
    if (d.lora_rank % 2 || d.lora_rank > 32) return EDGE_MOE_EUNSUPPORTED;
    if (!is_pow2(d.quant_group) || d.quant_group < 32 || d.quant_group > 4096) return EDGE_MOE_EUNSUPPORTED;
    return EDGE_MOE_OK;
}

struct Layout {
    size_t bm, pre, total, eoff, uoff, etile, etile_pf, gtile_u, gtile_r;
    size_t row_tok, row_slot, row_exp, row_u, slot_row, ut_tok;
    size_t xg, z1, zl, hs, act, z2, zl2, o;
    size_t logits;
    size_t fwd_bytes, route_bytes;
    int64_t R, Umax;
    int W, G, rLp;
};

Layout make_layout(const edge_moe_dims& d) {
    Layout L{};
    const int64_t T = d.T, E = d.n_experts, k = d.top_k;
    L.G = d.n_experts / d.experts_per_group;
    L.W = (int)((T + 31) / 32);
    L.R = T * k;
    L.Umax = L.R < T * L.G ? L.R : T * L.G;
    L.rLp = (d.lora_rank + 7) & ~7;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    const size_t nb = (size_t)(E + L.G) * L.W;
    L.bm = take(nb * 4);
    L.pre = take(nb * 4);
    L.total = take((E + L.G) * 4);
    L.eoff = take((E + 1) * 4);
    L.uoff = take((L.G + 1) * 4);
    L.etile = take((E + 1) * 4);
    L.etile_pf = take((E + 1) * 4);
    L.gtile_u = take((L.G + 1) * 4);
    L.gtile_r = take((L.G + 1) * 4);
    L.row_tok = take(L.R * 4);
    L.row_slot = take(L.R * 4);
    L.row_exp = take(L.R * 4);
    L.row_u = take(L.R * 4);
    L.slot_row = take(L.R * 4);
    L.ut_tok = take(L.Umax * 4);
    L.xg = take((size_t)(L.Umax + em::kPfSpareRows) * d.d * 2);   // + spare rows read by the last row tile
    L.z1 = take((size_t)L.R * d.delta_rank * 2);
    L.zl = take((size_t)L.Umax * L.rLp * 2);
    L.hs = take((size_t)L.Umax * d.h * 4);
    L.act = take((size_t)(L.R + em::kPfSpareRows) * d.h * 2);
    L.z2 = take((size_t)L.R * d.delta_rank * 2);
    L.zl2 = take((size_t)L.R * L.rLp * 2);
    L.o = take((size_t)L.R * d.d * 4);
    L.fwd_bytes = off;
    L.logits = 0;
    // fp32 logits, then (small batches) the router's K-slice sums
    L.route_bytes = align_up((size_t)T * E * 4);
    if (em::router_split_ok((int)T, d.d, (int)E)) L.route_bytes += align_up(em::router_split_bytes((int)T, (int)E));
    return L;
}

// Small-batch path: T <= 64 tokens and at most 1024 (token, slot) pairs.
bool use_decode(const edge_moe_dims& d) {
    return d.T <= 64 && (int64_t)d.T * d.top_k <= 1024 && d.experts_per_group <= 64;
}

struct DecLayout {
    size_t hs, z1p, zlp, act, z2p, z2, zl2, o, od, cnt_e, cnt_c, scratch, bytes;
    size_t pl_ctr, pl_z1p, pl_zlp, pl_z1b, pl_zlb, pl_z2p;   // persistent layer (T <= 8, r = 128)
    int S1, cb2, ncb2, N2;
    bool lds, pl;
};

DecLayout make_dec_layout(const edge_moe_dims& d) {
    DecLayout L{};
    const int64_t T = d.T, R = (int64_t)d.T * d.top_k, G = d.n_experts / d.experts_per_group;
    const int rLp = (d.lora_rank + 7) & ~7;
    L.S1 = d.d % 256 == 0 ? 2 : 1;            // K slices of the R1 / R2 products
    L.lds = em::decode_lds_ok(d.T, d.d, d.h, d.delta_rank, d.lora_rank, d.quant_group, L.S1);
    L.cb2 = L.lds ? 256 : (d.h % 512 == 0 ? 512 : (d.h % 256 == 0 ? 256 : 128));
    L.ncb2 = d.h / L.cb2;
    L.N2 = ((d.delta_rank + 15) & ~15) + ((d.lora_rank + 15) & ~15);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    L.hs = take((size_t)T * G * d.h * 4);
    L.z1p = take((size_t)L.S1 * R * d.delta_rank * 4);
    L.zlp = take((size_t)4 * L.S1 * T * G * rLp * 4);
    L.act = take((size_t)R * d.h * 2);
    L.z2p = take((size_t)L.ncb2 * R * L.N2 * 4);
    L.z2 = take((size_t)R * d.delta_rank * 2);
    L.zl2 = take((size_t)R * rLp * 2);
    L.o = take((size_t)R * d.d * 4);
    L.od = take((size_t)R * d.d * 4);
    L.cnt_e = take((size_t)d.n_experts * 4);
    L.cnt_c = take((size_t)(d.d / 64) * 4);
    L.scratch = take(64 * 4);
    // the persistent layer's buffers, for the shapes it can take
    L.pl = T <= 8 && R <= 128 && d.delta_rank == 128 && d.lora_rank <= 16;
    if (L.pl) {
        L.pl_ctr = take((size_t)em::PL_C_COUNT * 4);
        L.pl_z1p = take((size_t)4 * R * 128 * 4);
        L.pl_zlp = take((size_t)4 * T * G * 16 * 4);
        L.pl_z1b = take((size_t)R * 128 * 2);
        L.pl_zlb = take((size_t)T * G * 16 * 2);
        L.pl_z2p = take((size_t)(d.h / 128) * R * em::PL_Z2W * 4);
    }
    L.bytes = off;
    return L;
}

bool aligned(const void* p, size_t a) { return p && ((uintptr_t)p % a) == 0; }

// Shapes the decode-tiled codes take: quant groups of 128, d and h multiples
// of 1024 (whole tile groups of 128 rows, blocks of 256, and each row's scales
// a whole number of 16-byte pieces); for A_up also r a multiple of 128.
bool tile_shape_ok(const edge_moe_dims& d, int which = 0) {
    if (which == 3) return d.delta_rank == 128 && d.h % 128 == 0;
    return d.quant_group == 128 && d.d % 1024 == 0 && d.h % 1024 == 0 && (which != 2 || d.delta_rank % 128 == 0);
}

// gfx950 check, cached per device
int check_device() {
    static std::mutex mu;
    static std::unordered_map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return EDGE_MOE_EHIP;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return EDGE_MOE_EHIP;
    const std::string arch(prop.gcnArchName);
    const int st = arch.rfind("gfx950", 0) == 0 ? EDGE_MOE_OK : EDGE_MOE_EUNSUPPORTED;
    cache[dev] = st;
    return st;
}

// ----------------------------------------------------------------- profiling ----
// Measurement-only state (off unless edge_moe_prof_enable(1)).  One mutex
// guards the event pool and the table, so concurrent calls from several host
// threads may profile; the flag is read without the lock on the fast path.
struct ProfEntry { std::string name; hipEvent_t e0, e1; };
struct ProfState {
    std::atomic<bool> on{false};
    std::mutex mu;
    std::vector<ProfEntry> pending;
    std::vector<hipEvent_t> pool;
    std::unordered_map<hipStream_t, hipEvent_t> cur;     // open bracket per stream
    std::vector<std::string> order;
    std::unordered_map<std::string, std::pair<int64_t, double>> table;
};
ProfState& prof() { static ProfState s; return s; }

// caller holds p.mu
hipEvent_t prof_event(ProfState& p) {
    if (!p.pool.empty()) { hipEvent_t e = p.pool.back(); p.pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    hipEventCreate(&e);
    return e;
}

// caller holds p.mu
void prof_drain(ProfState& p) {
    for (auto& en : p.pending) {
        hipEventSynchronize(en.e1);
        float ms = 0.f;
        hipEventElapsedTime(&ms, en.e0, en.e1);
        auto it = p.table.find(en.name);
        if (it == p.table.end()) { p.order.push_back(en.name); p.table[en.name] = {1, ms}; }
        else { it->second.first += 1; it->second.second += ms; }
        p.pool.push_back(en.e0);
        p.pool.push_back(en.e1);
    }
    p.pending.clear();
}

// ------------------------------------------------------ allocation-free variant --
// The workspace of edge_moe_forward_noalloc: one file-scope device array, which
// each GPU holds its own copy of for the life of the process.  Host code only
// uses the array through the device address hipGetSymbolAddress returns for
// the current device (the array's own name on the host is not that address).
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of the current device's scratch (looked up once per device),
// or null if the lookup failed.
void* scratch_ptr() {
    static std::mutex mu;
    static void* ptrs[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

}  // namespace

namespace em {
// The layer's shape checks, for the host-side expert cache (cache.hip).
int layer_dims_status(const edge_moe_dims* d) { return check_dims(d); }

void prof_begin(hipStream_t s) {
    ProfState& p = prof();
    if (!p.on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(p.mu);
    hipEvent_t e = prof_event(p);
    hipEventRecord(e, s);
    p.cur[s] = e;
}
void prof_end(hipStream_t s, const char* name) {
    ProfState& p = prof();
    if (!p.on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(p.mu);
    auto it = p.cur.find(s);
    if (it == p.cur.end()) return;
    hipEvent_t e1 = prof_event(p);
    hipEventRecord(e1, s);
    p.pending.push_back({name, it->second, e1});
    p.cur.erase(it);
    if (p.pending.size() > 4096) prof_drain(p);
}
}  // namespace em

extern "C" {

size_t edge_moe_workspace_bytes(const edge_moe_dims* dims) {
    if (check_dims(dims) != EDGE_MOE_OK) return 0;
    const Layout L = make_layout(*dims);
    size_t n = L.fwd_bytes > L.route_bytes ? L.fwd_bytes : L.route_bytes;
    if (use_decode(*dims)) {
        const DecLayout D = make_dec_layout(*dims);
        n = n > D.bytes ? n : D.bytes;
    }
    return n;
}

int edge_moe_route(const edge_moe_dims* dims, const uint16_t* x, const uint16_t* w_router,
                   const float* router_bias, int32_t* topk_idx, float* topk_w,
                   float* logits_out, void* ws, size_t ws_bytes, void* stream) {
    int st = check_dims(dims);
    if (st != EDGE_MOE_OK) return st;
    if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return EDGE_MOE_EINVAL;
    if (router_bias && !aligned(router_bias, 4)) return EDGE_MOE_EINVAL;
    if (logits_out && !aligned(logits_out, 4)) return EDGE_MOE_EINVAL;
    const Layout L = make_layout(*dims);
    const edge_moe_dims& d = *dims;
    float* logits = logits_out;
    if (!logits) {
        if (!ws || !aligned(ws, kAlign)) return ws ? EDGE_MOE_EINVAL : EDGE_MOE_EWORKSPACE;
        if (ws_bytes < L.route_bytes) return EDGE_MOE_EWORKSPACE;
    }
    // small batches use the K-split logits when the workspace is there for
    // their slice sums (a caller that passes logits_out may pass no workspace)
    double* part = nullptr;
    if (em::router_split_ok(d.T, d.d, d.n_experts) && ws && aligned(ws, kAlign) && ws_bytes >= L.route_bytes)
        part = reinterpret_cast<double*>(static_cast<char*>(ws) + align_up((size_t)d.T * d.n_experts * 4));
    else if (!logits)
        logits = reinterpret_cast<float*>(ws);
    st = check_device();
    if (st != EDGE_MOE_OK) return st;
    hipError_t err = em::launch_router(x, w_router, router_bias, logits, part, topk_idx, topk_w, d.T, d.d,
                                       d.n_experts, d.top_k, (hipStream_t)stream);
    return err == hipSuccess ? EDGE_MOE_OK : EDGE_MOE_EHIP;
}

static em::DispatchBufs dispatch_bufs(const Layout& L, char* base) {
    em::DispatchBufs db{};
    db.bm = reinterpret_cast<uint32_t*>(base + L.bm);
    db.pre = reinterpret_cast<uint32_t*>(base + L.pre);
    db.total = reinterpret_cast<int32_t*>(base + L.total);
    db.eoff = reinterpret_cast<int32_t*>(base + L.eoff);
    db.uoff = reinterpret_cast<int32_t*>(base + L.uoff);
    db.etile = reinterpret_cast<int32_t*>(base + L.etile);
    db.etile_pf = reinterpret_cast<int32_t*>(base + L.etile_pf);
    db.gtile_u = reinterpret_cast<int32_t*>(base + L.gtile_u);
    db.gtile_r = reinterpret_cast<int32_t*>(base + L.gtile_r);
    db.row_tok = reinterpret_cast<int32_t*>(base + L.row_tok);
    db.row_slot = reinterpret_cast<int32_t*>(base + L.row_slot);
    db.row_exp = reinterpret_cast<int32_t*>(base + L.row_exp);
    db.row_u = reinterpret_cast<int32_t*>(base + L.row_u);
    db.slot_row = reinterpret_cast<int32_t*>(base + L.slot_row);
    db.ut_tok = reinterpret_cast<int32_t*>(base + L.ut_tok);
    return db;
}

static hipError_t copy_perm_trace(const edge_moe_trace* trace, const em::DispatchBufs& db,
                                  const edge_moe_dims& d, hipStream_t s) {
    const size_t R = (size_t)d.T * d.top_k;
    hipError_t err = hipSuccess;
    if (trace->expert_offsets)
        err = hipMemcpyAsync(trace->expert_offsets, db.eoff, (size_t)(d.n_experts + 1) * 4, hipMemcpyDeviceToDevice, s);
    if (err == hipSuccess && trace->row_token)
        err = hipMemcpyAsync(trace->row_token, db.row_tok, R * 4, hipMemcpyDeviceToDevice, s);
    if (err == hipSuccess && trace->row_slot)
        err = hipMemcpyAsync(trace->row_slot, db.row_slot, R * 4, hipMemcpyDeviceToDevice, s);
    return err;
}

static int forward_decode(const edge_moe_dims& d, const DecLayout& L, const uint16_t* x,
                          const int32_t* topk_idx, const float* topk_w, const edge_moe_weights* wt,
                          float* y, void* ws, void* stream, const edge_moe_trace* trace, bool persistent) {
    char* base = reinterpret_cast<char*>(ws);
    em::DecodeArgs a{};
    a.T = d.T; a.d = d.d; a.h = d.h; a.E = d.n_experts; a.P = d.experts_per_group;
    a.G = d.n_experts / d.experts_per_group; a.k = d.top_k; a.r = d.delta_rank; a.rL = d.lora_rank;
    a.rLp = (d.lora_rank + 7) & ~7; a.gq = d.quant_group; a.R = d.T * d.top_k;
    a.S1 = L.S1; a.cb2 = L.cb2; a.ncb2 = L.ncb2; a.lds = L.lds ? 1 : 0;
    const int rows_per_pass = 16 * em::decode_ns_down(d.T);
    a.npass = (a.R + rows_per_pass - 1) / rows_per_pass;
    a.nxmax = a.R < a.E ? a.R : a.E;
    a.x = x; a.idx = topk_idx; a.topk_w = topk_w;
    a.s_up = wt->s_up_q; a.s_up_s = wt->s_up_scale; a.s_dn = wt->s_dn_q; a.s_dn_s = wt->s_dn_scale;
    a.a_up = wt->a_up_q; a.a_up_s = wt->a_up_scale; a.b_up = wt->b_up_q; a.b_up_s = wt->b_up_scale;
    a.a_dn = wt->a_dn_q; a.a_dn_s = wt->a_dn_scale; a.b_dn = wt->b_dn_q; a.b_dn_s = wt->b_dn_scale;
    a.lu_u = wt->lora_up_u; a.lu_v = wt->lora_up_v; a.ld_u = wt->lora_dn_u; a.ld_v = wt->lora_dn_v;
    a.s_up_t = wt->s_up_t; a.s_dn_t = wt->s_dn_t; a.a_up_t = wt->a_up_t; a.a_dn_t = wt->a_dn_t;
    a.hs = reinterpret_cast<float*>(base + L.hs);
    a.z1p = reinterpret_cast<float*>(base + L.z1p);
    a.zlp = reinterpret_cast<float*>(base + L.zlp);
    a.act = reinterpret_cast<uint16_t*>(base + L.act);
    a.z2p = reinterpret_cast<float*>(base + L.z2p);
    a.z2 = reinterpret_cast<uint16_t*>(base + L.z2);
    a.zl2 = reinterpret_cast<uint16_t*>(base + L.zl2);
    a.o = reinterpret_cast<float*>(base + L.o);
    a.y = y;
    a.cnt_e = reinterpret_cast<uint32_t*>(base + L.cnt_e);
    a.cnt_c = reinterpret_cast<uint32_t*>(base + L.cnt_c);
    a.scratch = reinterpret_cast<float*>(base + L.scratch);
    a.od = reinterpret_cast<float*>(base + L.od);
    if (L.pl) {
        a.pl_ctr = reinterpret_cast<uint32_t*>(base + L.pl_ctr);
        a.pl_z1p = reinterpret_cast<float*>(base + L.pl_z1p);
        a.pl_zlp = reinterpret_cast<float*>(base + L.pl_zlp);
        a.pl_z1b = reinterpret_cast<uint16_t*>(base + L.pl_z1b);
        a.pl_zlb = reinterpret_cast<uint16_t*>(base + L.pl_zlb);
        a.pl_z2p = reinterpret_cast<float*>(base + L.pl_z2p);
    }
    a.pl_trace_o = trace && trace->expert_out ? 1 : 0;
    hipStream_t s = (hipStream_t)stream;
    hipError_t err = persistent ? em::launch_dec_layer(a, s) : em::launch_decode(a, s);
    if (err != hipSuccess) return EDGE_MOE_EHIP;
    if (trace) {
        // intermediates are stored per slot here; the permutation arrays come
        // from the general dispatch kernels, run after the copies (they reuse
        // the workspace)
        if (trace->act) err = hipMemcpyAsync(trace->act, a.act, (size_t)a.R * d.h * 2, hipMemcpyDeviceToDevice, s);
        if (err == hipSuccess && trace->expert_out)
            err = hipMemcpyAsync(trace->expert_out, a.o, (size_t)a.R * d.d * 4, hipMemcpyDeviceToDevice, s);
        if (err != hipSuccess) return EDGE_MOE_EHIP;
        if (trace->expert_offsets || trace->row_token || trace->row_slot) {
            const Layout GL = make_layout(d);
            em::DispatchBufs db = dispatch_bufs(GL, base);
            err = em::launch_dispatch(topk_idx, db, d.T, d.top_k, d.n_experts, d.experts_per_group, 64, s);
            if (err == hipSuccess) err = copy_perm_trace(trace, db, d, s);
            if (err != hipSuccess) return EDGE_MOE_EHIP;
        }
    }
    return EDGE_MOE_OK;
}

static int forward_impl(const edge_moe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                        const float* topk_w, const edge_moe_weights* wt, float* y, void* ws,
                        size_t ws_bytes, void* stream, const edge_moe_trace* trace, bool persistent = false) {
    int st = check_dims(dims);
    if (st != EDGE_MOE_OK) return st;
    if (!wt) return EDGE_MOE_EINVAL;
    if (!aligned(x, 16) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(y, 16))
        return EDGE_MOE_EINVAL;
    const void* wptrs[16] = {wt->s_up_q, wt->s_up_scale, wt->s_dn_q, wt->s_dn_scale,
                             wt->a_up_q, wt->a_up_scale, wt->b_up_q, wt->b_up_scale,
                             wt->a_dn_q, wt->a_dn_scale, wt->b_dn_q, wt->b_dn_scale,
                             wt->lora_up_u, wt->lora_up_v, wt->lora_dn_u, wt->lora_dn_v};
    for (const void* p : wptrs)
        if (!aligned(p, 16)) return EDGE_MOE_EINVAL;
    // the tiled copies: s_up / s_dn both or neither, a_up optional
    if ((wt->s_up_t != nullptr) != (wt->s_dn_t != nullptr)) return EDGE_MOE_EINVAL;
    if (wt->s_up_t) {
        if (!aligned(wt->s_up_t, 16) || !aligned(wt->s_dn_t, 16)) return EDGE_MOE_EINVAL;
        if (!tile_shape_ok(*dims)) return EDGE_MOE_EUNSUPPORTED;
    }
    if (wt->a_up_t) {
        if (!aligned(wt->a_up_t, 16)) return EDGE_MOE_EINVAL;
        if (!tile_shape_ok(*dims, 2)) return EDGE_MOE_EUNSUPPORTED;
    }
    if (wt->a_dn_t) {
        if (!aligned(wt->a_dn_t, 16)) return EDGE_MOE_EINVAL;
        if (!tile_shape_ok(*dims, 3)) return EDGE_MOE_EUNSUPPORTED;
    }
    if (!ws) return EDGE_MOE_EWORKSPACE;
    if (!aligned(ws, kAlign)) return EDGE_MOE_EINVAL;
    const Layout L = make_layout(*dims);
    const bool dec = use_decode(*dims);
    const DecLayout DL = dec ? make_dec_layout(*dims) : DecLayout{};
    if (ws_bytes < (dec ? DL.bytes : L.fwd_bytes)) return EDGE_MOE_EWORKSPACE;
    if (trace && ws_bytes < L.fwd_bytes) return EDGE_MOE_EWORKSPACE;
    st = check_device();
    if (st != EDGE_MOE_OK) return st;

    const edge_moe_dims& d = *dims;
    if (persistent) {
        // the persistent launch takes decode batches whose shapes it supports
        if (!dec || !DL.pl) return EDGE_MOE_EUNSUPPORTED;
        em::DecodeArgs probe{};
        probe.T = d.T; probe.d = d.d; probe.h = d.h; probe.E = d.n_experts; probe.P = d.experts_per_group;
        probe.G = d.n_experts / d.experts_per_group; probe.R = d.T * d.top_k; probe.r = d.delta_rank;
        probe.rL = d.lora_rank; probe.gq = d.quant_group;
        probe.s_up_t = wt->s_up_t; probe.s_dn_t = wt->s_dn_t; probe.a_up_t = wt->a_up_t; probe.a_dn_t = wt->a_dn_t;
        if (!em::dec_layer_ok(probe)) return EDGE_MOE_EUNSUPPORTED;
    }
    if (dec) return forward_decode(d, DL, x, topk_idx, topk_w, wt, y, ws, stream, trace, persistent);
    char* base = reinterpret_cast<char*>(ws);
    em::LayerArgs a{};
    a.T = d.T; a.d = d.d; a.h = d.h; a.E = d.n_experts; a.P = d.experts_per_group;
    a.G = L.G; a.k = d.top_k; a.r = d.delta_rank; a.rL = d.lora_rank; a.gq = d.quant_group;
    a.mt = 64;
    a.x = x; a.topk_w = topk_w;
    a.s_up = wt->s_up_q; a.s_up_s = wt->s_up_scale; a.s_dn = wt->s_dn_q; a.s_dn_s = wt->s_dn_scale;
    a.a_up = wt->a_up_q; a.a_up_s = wt->a_up_scale; a.b_up = wt->b_up_q; a.b_up_s = wt->b_up_scale;
    a.a_dn = wt->a_dn_q; a.a_dn_s = wt->a_dn_scale; a.b_dn = wt->b_dn_q; a.b_dn_s = wt->b_dn_scale;
    a.lu_u = wt->lora_up_u; a.lu_v = wt->lora_up_v; a.ld_u = wt->lora_dn_u; a.ld_v = wt->lora_dn_v;
    a.xg = reinterpret_cast<uint16_t*>(base + L.xg);
    a.z1 = reinterpret_cast<uint16_t*>(base + L.z1);
    a.zl = reinterpret_cast<uint16_t*>(base + L.zl);
    a.hs = reinterpret_cast<float*>(base + L.hs);
    a.act = reinterpret_cast<uint16_t*>(base + L.act);
    a.z2 = reinterpret_cast<uint16_t*>(base + L.z2);
    a.zl2 = reinterpret_cast<uint16_t*>(base + L.zl2);
    a.o = reinterpret_cast<float*>(base + L.o);
    a.y = y;
    a.db = dispatch_bufs(L, base);
    em::DispatchBufs& db = a.db;
    const int64_t R = L.R;
    const int64_t G = L.G;
    const int64_t E = d.n_experts;
    a.max_etiles = (int)((R + a.mt - 1) / a.mt + (E < R ? E : R));
    a.max_gtiles_u = (int)((L.Umax + a.mt - 1) / a.mt + G);
    a.max_gtiles_r = (int)((R + a.mt - 1) / a.mt + G);
    a.pf = em::prefill_gemm_ok(d.d, d.h, d.delta_rank, d.lora_rank, d.quant_group) ? 1 : 0;
    a.umax = L.Umax;
    a.rmax = R;

    hipStream_t s = (hipStream_t)stream;
    hipError_t err = em::launch_dispatch(topk_idx, db, d.T, d.top_k, d.n_experts, d.experts_per_group,
                                         a.mt, s);
    if (err != hipSuccess) return EDGE_MOE_EHIP;
    err = em::launch_expert_layer(a, s);
    if (err != hipSuccess) return EDGE_MOE_EHIP;
    if (trace) {
        err = copy_perm_trace(trace, db, d, s);
        if (err == hipSuccess && trace->act)
            err = em::launch_gather_rows(a.act, db.slot_row, trace->act, R, (int64_t)d.h * 2, s);
        if (err == hipSuccess && trace->expert_out)
            err = em::launch_gather_rows(a.o, db.slot_row, trace->expert_out, R, (int64_t)d.d * 4, s);
        if (err != hipSuccess) return EDGE_MOE_EHIP;
    }
    return EDGE_MOE_OK;
}

// ---------------------------------------------------------------- prefetch ----
size_t edge_moe_prefetch_ws_bytes(void) { return (size_t)em::kPrefetchBlocks * 256 * 4; }

int edge_moe_prefetch(const edge_moe_dims* dims, const edge_moe_weights* wt, const int32_t* groups,
                      int32_t n_groups, int32_t parts, void* ws, size_t ws_bytes, void* stream) {
    int st = check_dims(dims);
    if (st != EDGE_MOE_OK) return st;
    const edge_moe_dims& d = *dims;
    const int G = d.n_experts / d.experts_per_group;
    if (!wt || parts < 1 || parts > 3 || n_groups < 0 || n_groups > 4 * G) return EDGE_MOE_EINVAL;
    if (n_groups > 0 && !aligned(groups, 4)) return EDGE_MOE_EINVAL;
    if (!aligned(ws, 16)) return ws ? EDGE_MOE_EINVAL : EDGE_MOE_EWORKSPACE;
    if (ws_bytes < edge_moe_prefetch_ws_bytes()) return EDGE_MOE_EWORKSPACE;
    const uint8_t* up_q = wt->s_up_t ? wt->s_up_t : wt->s_up_q;
    const uint8_t* dn_q = wt->s_dn_t ? wt->s_dn_t : wt->s_dn_q;
    if (((parts & 1) && (!aligned(up_q, 16) || !aligned(wt->s_up_scale, 16))) ||
        ((parts & 2) && (!aligned(dn_q, 16) || !aligned(wt->s_dn_scale, 16))))
        return EDGE_MOE_EINVAL;
    if (n_groups == 0) return EDGE_MOE_OK;
    st = check_device();
    if (st != EDGE_MOE_OK) return st;
    const int gq_d = d.quant_group < d.d ? d.quant_group : d.d;
    const int gq_h = d.quant_group < d.h ? d.quant_group : d.h;
    const uint8_t* bases[4];
    size_t bytes[4];
    int n = 0;
    if (parts & 1) {
        bases[n] = up_q; bytes[n++] = (size_t)d.h * d.d / 2;
        bases[n] = reinterpret_cast<const uint8_t*>(wt->s_up_scale); bytes[n++] = (size_t)d.h * (d.d / gq_d) * 2;
    }
    if (parts & 2) {
        bases[n] = dn_q; bytes[n++] = (size_t)d.d * d.h / 2;
        bases[n] = reinterpret_cast<const uint8_t*>(wt->s_dn_scale); bytes[n++] = (size_t)d.d * (d.h / gq_h) * 2;
    }
    const hipError_t e = em::launch_prefetch(bases, bytes, n, groups, n_groups, G, static_cast<uint32_t*>(ws),
                                             em::kPrefetchBlocks, (hipStream_t)stream);
    return e == hipSuccess ? EDGE_MOE_OK : EDGE_MOE_EHIP;
}

// ---------------------------------------------------------------- MX variant --
// The general layout followed by the MXFP8 copies of the product inputs.
struct MxLayout {
    Layout L;
    size_t xq, xs, aq, as, bytes;
};

static MxLayout make_mx_layout(const edge_moe_dims& d) {
    MxLayout M{};
    M.L = make_layout(d);
    size_t off = M.L.fwd_bytes;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    const size_t T = (size_t)d.T, R = (size_t)M.L.R;
    M.xq = take(T * d.d);
    M.xs = take(T * d.d / 32);
    M.aq = take(R * d.h);
    M.as = take(R * d.h / 32);
    M.bytes = off;
    return M;
}

static bool mx_dims_ok(const edge_moe_dims& d) {
    return em::mx_layer_ok(d.d, d.h, d.delta_rank, d.lora_rank);
}

size_t edge_moe_workspace_bytes_mx(const edge_moe_dims* dims) {
    if (check_dims(dims) != EDGE_MOE_OK || !mx_dims_ok(*dims)) return 0;
    const MxLayout M = make_mx_layout(*dims);
    return M.bytes > M.L.route_bytes ? M.bytes : M.L.route_bytes;
}

int edge_moe_forward_mx(const edge_moe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                        const float* topk_w, const edge_moe_weights_mx* wt, float* y, void* ws,
                        size_t ws_bytes, void* stream, const edge_moe_trace* trace) {
    int st = check_dims(dims);
    if (st != EDGE_MOE_OK) return st;
    if (!wt) return EDGE_MOE_EINVAL;
    if (!aligned(x, 16) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(y, 16))
        return EDGE_MOE_EINVAL;
    const void* wptrs[16] = {wt->s_up_q, wt->s_up_e, wt->s_dn_q, wt->s_dn_e, wt->a_up_q, wt->a_up_e,
                             wt->b_up_q, wt->b_up_e, wt->a_dn_q, wt->a_dn_e, wt->b_dn_q, wt->b_dn_e,
                             wt->lora_up_u, wt->lora_up_v, wt->lora_dn_u, wt->lora_dn_v};
    for (const void* p : wptrs)
        if (!aligned(p, 16)) return EDGE_MOE_EINVAL;
    if (!mx_dims_ok(*dims)) return EDGE_MOE_EUNSUPPORTED;
    if (!ws) return EDGE_MOE_EWORKSPACE;
    if (!aligned(ws, kAlign)) return EDGE_MOE_EINVAL;
    const MxLayout M = make_mx_layout(*dims);
    if (ws_bytes < M.bytes) return EDGE_MOE_EWORKSPACE;
    st = check_device();
    if (st != EDGE_MOE_OK) return st;

    const edge_moe_dims& d = *dims;
    const Layout& L = M.L;
    char* base = reinterpret_cast<char*>(ws);
    em::LayerArgs a{};
    a.T = d.T; a.d = d.d; a.h = d.h; a.E = d.n_experts; a.P = d.experts_per_group;
    a.G = L.G; a.k = d.top_k; a.r = d.delta_rank; a.rL = d.lora_rank; a.gq = 32;
    a.mt = 64;
    a.x = x; a.topk_w = topk_w;
    a.s_up = wt->s_up_q; a.s_dn = wt->s_dn_q; a.a_up = wt->a_up_q; a.b_up = wt->b_up_q;
    a.a_dn = wt->a_dn_q; a.b_dn = wt->b_dn_q;
    a.s_up_e = wt->s_up_e; a.s_dn_e = wt->s_dn_e; a.a_up_e = wt->a_up_e; a.b_up_e = wt->b_up_e;
    a.a_dn_e = wt->a_dn_e; a.b_dn_e = wt->b_dn_e;
    a.lu_u = wt->lora_up_u; a.lu_v = wt->lora_up_v; a.ld_u = wt->lora_dn_u; a.ld_v = wt->lora_dn_v;
    a.z1 = reinterpret_cast<uint16_t*>(base + L.z1);
    a.zl = reinterpret_cast<uint16_t*>(base + L.zl);
    a.hs = reinterpret_cast<float*>(base + L.hs);
    a.act = reinterpret_cast<uint16_t*>(base + L.act);
    a.z2 = reinterpret_cast<uint16_t*>(base + L.z2);
    a.zl2 = reinterpret_cast<uint16_t*>(base + L.zl2);
    a.o = reinterpret_cast<float*>(base + L.o);
    a.xq = reinterpret_cast<uint8_t*>(base + M.xq);
    a.xs = reinterpret_cast<uint8_t*>(base + M.xs);
    a.aq = reinterpret_cast<uint8_t*>(base + M.aq);
    a.as = reinterpret_cast<uint8_t*>(base + M.as);
    a.y = y;
    a.db = dispatch_bufs(L, base);
    const int64_t R = L.R, G = L.G, E = d.n_experts;
    a.max_etiles = (int)((R + a.mt - 1) / a.mt + (E < R ? E : R));
    a.max_gtiles_u = (int)((L.Umax + a.mt - 1) / a.mt + G);
    a.max_gtiles_r = (int)((R + a.mt - 1) / a.mt + G);
    a.umax = L.Umax;
    a.rmax = R;
    hipStream_t s = (hipStream_t)stream;
    hipError_t err = em::launch_dispatch(topk_idx, a.db, d.T, d.top_k, d.n_experts, d.experts_per_group, a.mt, s);
    if (err == hipSuccess) err = em::launch_mx_layer(a, s);
    if (err != hipSuccess) return EDGE_MOE_EHIP;
    if (trace) {
        err = copy_perm_trace(trace, a.db, d, s);
        if (err == hipSuccess && trace->act)
            err = em::launch_gather_rows(a.act, a.db.slot_row, trace->act, R, (int64_t)d.h * 2, s);
        if (err == hipSuccess && trace->expert_out)
            err = em::launch_gather_rows(a.o, a.db.slot_row, trace->expert_out, R, (int64_t)d.d * 4, s);
        if (err != hipSuccess) return EDGE_MOE_EHIP;
    }
    return EDGE_MOE_OK;
}

int edge_moe_forward(const edge_moe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                     const float* topk_w, const edge_moe_weights* weights, float* y, void* ws,
                     size_t ws_bytes, void* stream) {
    return forward_impl(dims, x, topk_idx, topk_w, weights, y, ws, ws_bytes, stream, nullptr);
}

int edge_moe_forward_persistent(const edge_moe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                                const float* topk_w, const edge_moe_weights* weights, float* y, void* ws,
                                size_t ws_bytes, void* stream, const edge_moe_trace* trace) {
    return forward_impl(dims, x, topk_idx, topk_w, weights, y, ws, ws_bytes, stream, trace, true);
}

int edge_moe_forward_traced(const edge_moe_dims* dims, const uint16_t* x,
                            const int32_t* topk_idx, const float* topk_w,
                            const edge_moe_weights* weights, float* y, void* ws,
                            size_t ws_bytes, void* stream, const edge_moe_trace* trace) {
    return forward_impl(dims, x, topk_idx, topk_w, weights, y, ws, ws_bytes, stream, trace);
}

int edge_moe_forward_noalloc(const edge_moe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                             const float* topk_w, const edge_moe_weights* weights, float* y, void* stream) {
    const int st = check_dims(dims);
    if (st != EDGE_MOE_OK) return st;
    if (edge_moe_workspace_bytes(dims) > kScratchBytes) return EDGE_MOE_EWORKSPACE;
    const int dst = check_device();
    if (dst != EDGE_MOE_OK) return dst;
    void* ws = scratch_ptr();
    if (!ws) return EDGE_MOE_EHIP;
    return forward_impl(dims, x, topk_idx, topk_w, weights, y, ws, kScratchBytes, stream, nullptr);
}

int edge_moe_residual(int32_t T, int32_t d, const uint16_t* x, const float* y, uint16_t* x_out,
                      void* stream) {
    if (T < 1 || d < 8 || d % 8) return EDGE_MOE_EINVAL;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(x_out, 16)) return EDGE_MOE_EINVAL;
    const int st = check_device();
    if (st != EDGE_MOE_OK) return st;
    return em::launch_residual(T, d, x, y, x_out, (hipStream_t)stream) == hipSuccess ? EDGE_MOE_OK
                                                                                     : EDGE_MOE_EHIP;
}

int edge_moe_tile_shared(const edge_moe_dims* dims, int32_t which, const uint8_t* src_q, uint8_t* dst_q,
                         void* stream) {
    const int st = check_dims(dims);
    if (st != EDGE_MOE_OK) return st;
    if (which < 0 || which > 3) return EDGE_MOE_EINVAL;
    if (!aligned(src_q, 16) || !aligned(dst_q, 16)) return EDGE_MOE_EINVAL;
    if (!tile_shape_ok(*dims, which)) return EDGE_MOE_EUNSUPPORTED;
    const int G = which >= 2 ? dims->n_experts : dims->n_experts / dims->experts_per_group;
    const int N = which == 0 ? dims->h : (which == 1 ? dims->d : dims->delta_rank);
    const int K = (which == 1 || which == 3) ? dims->h : dims->d;
    const size_t qb = (size_t)G * N * K / 2;
    const char* s8 = reinterpret_cast<const char*>(src_q);
    const char* d8 = reinterpret_cast<const char*>(dst_q);
    if (d8 < s8 + qb && s8 < d8 + qb) return EDGE_MOE_EINVAL;
    const int dst_st = check_device();
    if (dst_st != EDGE_MOE_OK) return dst_st;
    const hipError_t err = which == 3 ? em::launch_colblock(src_q, dst_q, G, N, K, (hipStream_t)stream)
                                      : em::launch_tile_shared(src_q, dst_q, G, N, K, (hipStream_t)stream);
    return err == hipSuccess ? EDGE_MOE_OK : EDGE_MOE_EHIP;
}

int edge_moe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!dst || !src || bytes % 16 || !aligned(dst, 16) || !aligned(src, 16)) return EDGE_MOE_EINVAL;
    const char* d8 = static_cast<const char*>(dst);
    const char* s8 = static_cast<const char*>(src);
    if (d8 < s8 + bytes && s8 < d8 + bytes) return EDGE_MOE_EINVAL;
    const int st = check_device();
    if (st != EDGE_MOE_OK) return st;
    if (bytes == 0) return EDGE_MOE_OK;
    return em::launch_copy(dst, src, bytes, (hipStream_t)stream) == hipSuccess ? EDGE_MOE_OK : EDGE_MOE_EHIP;
}

int edge_moe_mfma_peak(float* out, int32_t blocks, int32_t iters, void* stream) {
    if (!aligned(out, 4) || blocks < 1 || iters < 1) return EDGE_MOE_EINVAL;
    const int st = check_device();
    if (st != EDGE_MOE_OK) return st;
    return em::launch_mfma_peak(out, blocks, iters, (hipStream_t)stream) == hipSuccess ? EDGE_MOE_OK : EDGE_MOE_EHIP;
}

const char* edge_moe_status_string(int status) {
    switch (status) {
        case EDGE_MOE_OK: return "ok";
        case EDGE_MOE_EINVAL: return "invalid argument (null or misaligned pointer, inconsistent dims)";
        case EDGE_MOE_EUNSUPPORTED: return "unsupported shape or device (needs gfx950)";
        case EDGE_MOE_EWORKSPACE: return "workspace missing or smaller than edge_moe_workspace_bytes()";
        case EDGE_MOE_EHIP: return "HIP runtime or kernel launch error";
        default: return "unknown status";
    }
}

int edge_moe_abi_version(void) { return EDGE_MOE_ABI_VERSION; }

int edge_moe_prof_enable(int on) {
    return prof().on.exchange(on != 0) ? 1 : 0;
}

int edge_moe_prof_read(char (*names)[64], int64_t* launches, double* total_ms, int cap) {
    ProfState& p = prof();
    std::lock_guard<std::mutex> lk(p.mu);
    prof_drain(p);
    int i = 0;
    for (const auto& n : p.order) {
        if (i < cap) {
            const auto& v = p.table[n];
            if (names) {
                size_t m = n.size() < 63 ? n.size() : 63;
                for (size_t j = 0; j < m; ++j) names[i][j] = n[j];
                names[i][m] = 0;
            }
            if (launches) launches[i] = v.first;
            if (total_ms) total_ms[i] = v.second;
        }
        ++i;
    }
    return i;
}

void edge_moe_prof_reset(void) {
    ProfState& p = prof();
    std::lock_guard<std::mutex> lk(p.mu);
    prof_drain(p);
    p.table.clear();
    p.order.clear();
}

}  // extern "C"
