// Expert streaming from host memory: an LRU cache of expert slots in HBM.
//
// The pages keep the expert library in host memory and stream the experts a
// token needs into a small GPU memory, least recently used ones leaving first,
// through fixed staging slots (launch post "Edge0-145B: Frontier AI
// Capabilities on Your Own Computer", Under the Hood, Loading paragraph;
// byteiota "Edge0-145B: Run a 145B Open-Source Model on Your Laptop", The
// Three Pillars, SSD expert streaming paragraph).  Here the per-expert delta
// tensors (A_up, B_up, A_dn, B_dn with their scales and optional decode-tiled
// copies) of a layer live in pinned host memory; HBM holds S slots per group.
//
// The layer kernels need no change: slot s of group g is expert g * S + s of
// a layer with G groups of S experts, and a batch's routed experts are
// renamed to their slots.  The shared matrices and LoRA factors (per group)
// stay resident and the group of every renamed expert is its own, so every
// row computes exactly what it computes with all experts resident.
//
// Planning (which experts hit, which slots their misses take) is host code.
// The copies of one call go out as one gather kernel on the caller's stream
// that reads the pinned host memory directly over the host link and writes
// the slots: a miss touches ten tensors of 8 KB to 512 KB, and one DMA copy per
// tensor would pay a per-copy cost larger than the transfer itself.  Host
// memory that the GPU cannot address (pageable) or that is not 16-byte
// aligned takes hipMemcpyAsync per tensor instead.  A cache created without
// device slot pointers only plans, which is how its replacement policy is
// tested without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "edge_moe.h"
#include "kernels.h"

namespace em {

int layer_dims_status(const edge_moe_dims* d);     // api.hip: the layer's shape checks

constexpr int kCacheTensors = 10;   // a_up, a_up_s, b_up, b_up_s, a_dn, a_dn_s, b_dn, b_dn_s, a_up_t, a_dn_t
constexpr int kMaxPairs = 256; // (expert, slot) pairs per gather launch
constexpr int GC_THREADS = 256;
constexpr int GC_UNROLL = 4;
constexpr uint32_t GC_CHUNK = GC_THREADS * 16 * GC_UNROLL;   // bytes per workgroup turn
constexpr int GC_MAX_BLOCKS = 64;   // enough reads in flight for the host link, few CUs taken

// Everything a gather launch needs travels in its kernel arguments (about 1.3
// KB), so a call needs no descriptor memory.
struct GatherArgs {
    const uint8_t* src[kCacheTensors];     // device addresses of the host tensors
    uint8_t* dst[kCacheTensors];           // slot tensors
    uint32_t bytes[kCacheTensors];         // per expert, multiples of 16 (0: tensor absent)
    uint32_t chunk_pre[kCacheTensors + 1]; // first chunk of each tensor within a pair
    int32_t n;                        // pairs
    uint16_t e[kMaxPairs];            // source expert of each pair
    uint16_t slot[kMaxPairs];         // destination slot of each pair
};

// Workgroups stride over (pair, chunk) items; a chunk is 16 KB of one tensor
// of one expert, each lane moving four 16-byte pieces with all four loads in
// flight before the first store.
__global__ void __launch_bounds__(GC_THREADS)
cache_gather(GatherArgs a) {
    const uint32_t per_pair = a.chunk_pre[kCacheTensors];
    const uint32_t total = (uint32_t)a.n * per_pair;
    for (uint32_t item = blockIdx.x; item < total; item += gridDim.x) {
        const uint32_t p = item / per_pair;
        uint32_t c = item % per_pair;
        int t = 0;
        while (t < kCacheTensors - 1 && c >= a.chunk_pre[t + 1]) ++t;
        c -= a.chunk_pre[t];
        const uint32_t nb = a.bytes[t];
        const uint8_t* src = a.src[t] + (size_t)a.e[p] * nb;
        uint8_t* dst = a.dst[t] + (size_t)a.slot[p] * nb;
        uint4 v[GC_UNROLL];
#pragma unroll
        for (int u = 0; u < GC_UNROLL; ++u) {
            const uint32_t off = c * GC_CHUNK + (uint32_t)(u * GC_THREADS + threadIdx.x) * 16u;
            if (off < nb) v[u] = *reinterpret_cast<const uint4*>(src + off);
        }
#pragma unroll
        for (int u = 0; u < GC_UNROLL; ++u) {
            const uint32_t off = c * GC_CHUNK + (uint32_t)(u * GC_THREADS + threadIdx.x) * 16u;
            if (off < nb) *reinterpret_cast<uint4*>(dst + off) = v[u];
        }
    }
}

}  // namespace em

namespace {

using em::GatherArgs;
using em::GC_CHUNK;
using em::GC_MAX_BLOCKS;
using em::GC_THREADS;
using em::kMaxPairs;

constexpr int kTensors = em::kCacheTensors;   // a_up, a_up_s, b_up, b_up_s, a_dn, a_dn_s, b_dn, b_dn_s, a_up_t, a_dn_t
struct Cache {
    edge_moe_dims dims;
    int G = 0, P = 0, S = 0;
    const uint8_t* host[kTensors] = {};
    const uint8_t* host_dev[kTensors] = {};   // device addresses of host[] (gather path)
    uint8_t* slot[kTensors] = {};
    size_t bytes[kTensors] = {};     // per expert
    bool dry = true;
    bool gather = false;             // copies by cache_gather, else hipMemcpyAsync
    std::vector<uint16_t> pend_e, pend_s;   // this call's misses, for the gather
    std::vector<int32_t> slot_expert;   // [G * S], -1 when free
    std::vector<int32_t> expert_slot;   // [E], -1 when not resident
    std::vector<uint64_t> last_use;     // [G * S]
    uint64_t tick = 0;
    edge_moe_cache_stats total{};
};

void per_expert_bytes(const edge_moe_dims& d, size_t out[kTensors]) {
    const size_t r = d.delta_rank, dd = d.d, h = d.h;
    const size_t gq_d = std::min<size_t>(d.quant_group, dd), gq_h = std::min<size_t>(d.quant_group, h);
    const size_t gq_r = std::min<size_t>(d.quant_group, r);
    out[0] = r * dd / 2;     out[1] = r * (dd / gq_d) * 2;     // A_up
    out[2] = h * r / 2;      out[3] = h * (r / gq_r) * 2;      // B_up
    out[4] = r * h / 2;      out[5] = r * (h / gq_h) * 2;      // A_dn
    out[6] = dd * r / 2;     out[7] = dd * (r / gq_r) * 2;     // B_dn
    out[8] = out[0];         out[9] = out[4];                  // tiled A_up, column-blocked A_dn
}

void tensor_ptrs(const edge_moe_expert_tensors* t, void* p[kTensors]) {
    void* src[kTensors] = {t->a_up_q, t->a_up_scale, t->b_up_q, t->b_up_scale, t->a_dn_q, t->a_dn_scale,
                           t->b_dn_q, t->b_dn_scale, t->a_up_t, t->a_dn_t};
    for (int i = 0; i < kTensors; ++i) p[i] = src[i];
}

// Bring expert e into a slot of its group.  A resident expert is refreshed
// (a hit); otherwise it takes the group's free slot, else its least recently
// used slot whose stamp is older than `pinned_from` (a miss), and its tensors
// are copied there.  Returns the slot, or -1 when every slot is pinned.
int place(Cache& c, int e, uint64_t pinned_from, hipStream_t s, edge_moe_cache_stats& st, hipError_t& err) {
    const int g = e / c.P;
    const int sl = c.expert_slot[e];
    if (sl >= 0) {
        c.last_use[sl] = c.tick;
        ++st.hits;
        return sl;
    }
    int best = -1;
    for (int i = g * c.S; i < (g + 1) * c.S; ++i) {
        if (c.slot_expert[i] < 0) { best = i; break; }
        if (c.last_use[i] >= pinned_from) continue;
        if (best < 0 || c.last_use[i] < c.last_use[best]) best = i;
    }
    if (best < 0) return -1;
    if (c.slot_expert[best] >= 0) {
        c.expert_slot[c.slot_expert[best]] = -1;
        ++st.evictions;
    }
    c.slot_expert[best] = e;
    c.expert_slot[e] = best;
    c.last_use[best] = c.tick;
    ++st.misses;
    for (int t = 0; t < kTensors; ++t) {
        if (!c.host[t]) continue;
        st.bytes_copied += (int64_t)c.bytes[t];
        if (!c.dry && !c.gather && err == hipSuccess)
            err = hipMemcpyAsync(c.slot[t] + (size_t)best * c.bytes[t], c.host[t] + (size_t)e * c.bytes[t],
                                 c.bytes[t], hipMemcpyHostToDevice, s);
    }
    if (!c.dry && c.gather) {
        c.pend_e.push_back((uint16_t)e);
        c.pend_s.push_back((uint16_t)best);
    }
    return best;
}

// The gather launches for the misses placed by one call.
hipError_t flush(Cache& c, hipStream_t s) {
    hipError_t err = hipSuccess;
    GatherArgs a{};
    uint32_t pre = 0;
    for (int t = 0; t < kTensors; ++t) {
        a.src[t] = c.host_dev[t];
        a.dst[t] = c.slot[t];
        a.bytes[t] = c.host[t] ? (uint32_t)c.bytes[t] : 0u;
        a.chunk_pre[t] = pre;
        pre += (a.bytes[t] + GC_CHUNK - 1) / GC_CHUNK;
    }
    a.chunk_pre[kTensors] = pre;
    for (size_t i0 = 0; i0 < c.pend_e.size() && err == hipSuccess; i0 += kMaxPairs) {
        const int n = (int)std::min<size_t>(kMaxPairs, c.pend_e.size() - i0);
        a.n = n;
        for (int i = 0; i < n; ++i) {
            a.e[i] = c.pend_e[i0 + i];
            a.slot[i] = c.pend_s[i0 + i];
        }
        const int blocks = (int)std::min<uint32_t>((uint32_t)n * pre, GC_MAX_BLOCKS);
        em::prof_begin(s);
        em::cache_gather<<<blocks, GC_THREADS, 0, s>>>(a);
        em::prof_end(s, "cache_gather");
        err = hipGetLastError();
    }
    c.pend_e.clear();
    c.pend_s.clear();
    return err;
}

void add(edge_moe_cache_stats& a, const edge_moe_cache_stats& b) {
    a.hits += b.hits; a.misses += b.misses; a.evictions += b.evictions; a.bytes_copied += b.bytes_copied;
}

}  // namespace

extern "C" {

edge_moe_cache* edge_moe_cache_create(const edge_moe_dims* dims, int32_t slots_per_group,
                                      const edge_moe_expert_tensors* host, const edge_moe_expert_tensors* slots) {
    // the layer's own shape rules, so that the per-expert sizes are those its
    // kernels address
    if (!host || em::layer_dims_status(dims) != EDGE_MOE_OK) return nullptr;
    if (slots_per_group < 1 || slots_per_group > dims->experts_per_group) return nullptr;
    Cache* c = new (std::nothrow) Cache();
    if (!c) return nullptr;
    c->dims = *dims;
    c->P = dims->experts_per_group;
    c->G = dims->n_experts / c->P;
    c->S = slots_per_group;
    per_expert_bytes(*dims, c->bytes);
    void* hp[kTensors];
    tensor_ptrs(host, hp);
    void* sp[kTensors] = {};
    if (slots) tensor_ptrs(slots, sp);
    c->dry = slots == nullptr;
    for (int t = 0; t < kTensors; ++t) {
        c->host[t] = static_cast<const uint8_t*>(hp[t]);
        c->slot[t] = static_cast<uint8_t*>(sp[t]);
        // the eight row-major tensors are required; the tiled ones optional, on both sides alike
        if (t < 8 && !c->host[t]) { delete c; return nullptr; }
        if (!c->dry && (c->host[t] != nullptr) != (c->slot[t] != nullptr)) { delete c; return nullptr; }
    }
    if (!c->dry) {
        // the gather path needs every host tensor addressable by the GPU
        // (pinned, hipHostMalloc) and 16-byte aligned on both sides
        bool ok = true;
        for (int t = 0; t < kTensors && ok; ++t) {
            if (!c->host[t]) continue;
            void* dp = nullptr;
            if (hipHostGetDevicePointer(&dp, const_cast<uint8_t*>(c->host[t]), 0) != hipSuccess || !dp) {
                (void)hipGetLastError();   // pageable memory: clear the error, copy by hipMemcpyAsync
                ok = false;
                break;
            }
            c->host_dev[t] = static_cast<const uint8_t*>(dp);
            ok = reinterpret_cast<uintptr_t>(dp) % 16 == 0 && reinterpret_cast<uintptr_t>(c->slot[t]) % 16 == 0 &&
                 c->bytes[t] % 16 == 0 && c->bytes[t] < (size_t(1) << 31);
        }
        c->gather = ok;
    }
    c->slot_expert.assign((size_t)c->G * c->S, -1);
    c->expert_slot.assign((size_t)dims->n_experts, -1);
    c->last_use.assign((size_t)c->G * c->S, 0);
    return reinterpret_cast<edge_moe_cache*>(c);
}

void edge_moe_cache_destroy(edge_moe_cache* cache) { delete reinterpret_cast<Cache*>(cache); }

int edge_moe_cache_map(edge_moe_cache* cache, int32_t T, const int32_t* topk_idx, int32_t* slot_idx,
                       void* stream, edge_moe_cache_stats* stats) {
    Cache* c = reinterpret_cast<Cache*>(cache);
    if (!c || T < 0 || (T > 0 && (!topk_idx || !slot_idx))) return EDGE_MOE_EINVAL;
    const int64_t n = (int64_t)T * c->dims.top_k;
    const int E = c->dims.n_experts;
    for (int64_t i = 0; i < n; ++i)
        if (topk_idx[i] < 0 || topk_idx[i] >= E) return EDGE_MOE_EINVAL;
    // feasibility first, so that a batch that cannot run changes nothing: no
    // group may need more distinct experts than it has slots
    std::vector<char> seen((size_t)E, 0);
    std::vector<int> per_group((size_t)c->G, 0);
    for (int64_t i = 0; i < n; ++i)
        if (!seen[topk_idx[i]]) {
            seen[topk_idx[i]] = 1;
            if (++per_group[topk_idx[i] / c->P] > c->S) return EDGE_MOE_EUNSUPPORTED;
        }
    edge_moe_cache_stats st{};
    const uint64_t batch = ++c->tick;
    // stamp the batch's resident experts before any miss is placed, so that no
    // miss evicts an expert this batch uses
    for (int64_t i = 0; i < n; ++i) {
        const int sl = c->expert_slot[topk_idx[i]];
        if (sl >= 0) c->last_use[sl] = batch;
    }
    hipError_t err = hipSuccess;
    for (int64_t i = 0; i < n; ++i) {
        const int e = topk_idx[i];
        if (seen[e] == 1) {                 // first occurrence: count and place once
            seen[e] = 2;
            place(*c, e, batch, (hipStream_t)stream, st, err);
        }
        slot_idx[i] = c->expert_slot[e];    // slot g * S + s is expert g * S + s of the slot layer
    }
    if (c->gather) {
        const hipError_t fe = flush(*c, (hipStream_t)stream);
        if (err == hipSuccess) err = fe;
    }
    add(c->total, st);
    if (stats) *stats = st;
    return err == hipSuccess ? EDGE_MOE_OK : EDGE_MOE_EHIP;
}

int edge_moe_cache_prefetch(edge_moe_cache* cache, int32_t n, const int32_t* experts, void* stream,
                            edge_moe_cache_stats* stats) {
    Cache* c = reinterpret_cast<Cache*>(cache);
    if (!c || n < 0 || (n > 0 && !experts)) return EDGE_MOE_EINVAL;
    for (int i = 0; i < n; ++i)
        if (experts[i] < 0 || experts[i] >= c->dims.n_experts) return EDGE_MOE_EINVAL;
    edge_moe_cache_stats st{};
    ++c->tick;
    hipError_t err = hipSuccess;
    // a prefetch may evict any slot but those it filled itself; listed experts
    // beyond a group's slots are skipped
    for (int i = 0; i < n; ++i) place(*c, experts[i], c->tick, (hipStream_t)stream, st, err);
    if (c->gather) {
        const hipError_t fe = flush(*c, (hipStream_t)stream);
        if (err == hipSuccess) err = fe;
    }
    add(c->total, st);
    if (stats) *stats = st;
    return err == hipSuccess ? EDGE_MOE_OK : EDGE_MOE_EHIP;
}

int edge_moe_cache_totals(const edge_moe_cache* cache, edge_moe_cache_stats* stats) {
    const Cache* c = reinterpret_cast<const Cache*>(cache);
    if (!c || !stats) return EDGE_MOE_EINVAL;
    *stats = c->total;
    return EDGE_MOE_OK;
}

int edge_moe_cache_slot_of(const edge_moe_cache* cache, int32_t expert) {
    const Cache* c = reinterpret_cast<const Cache*>(cache);
    if (!c || expert < 0 || expert >= c->dims.n_experts) return -2;
    return c->expert_slot[expert];
}

}  // extern "C"
