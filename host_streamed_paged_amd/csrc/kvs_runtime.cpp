// Host runtime of libkvs: configuration checks, arena carve, page tables,
// launch plans and the H2D ring pipeline. The C ABI is declared in
// include/kvs.h.
//
// The design follows the pages' statement of the problem: authoritative KV in
// pinned host memory, a bounded device region holding resident 256-token pages
// and one ring shared by all layers, with flash-attention consuming both
// (page 1, "Summary"; page 2, opening paragraph). The ring is filled by copy
// workgroups that ride inside the compute launches (or, for a prefetch, a
// copy-only launch on the pool's prefetch stream): each launch computes on
// the ring chunk the launch before it filled while its own copy workgroups
// pull a later chunk over the host link, so kernel boundaries on a stream
// order each copy before its reader and each reader before the slot's refill;
// HIP events order the pool's streams against each other.
#include "kvs.h"
#include "kvs_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

#define KVS_HIP(expr)                                                                      \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess) return fail(KVS_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

constexpr uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

constexpr int kMaxLanes = 3;   // compute lanes for ring chunks
constexpr int kWideCopyRounds = 7;   // 32 KB rounds per copy workgroup of a prefill-width launch
// automatic sizing (page 3, description of --kv-stream auto): a 2048-token
// floor, an 8192 MiB ceiling, and in the stage formula that reproduces its
// logs, 4 pages per layer above the resident ones
constexpr int64_t kAutoFloorTokens = 2048;
constexpr uint64_t kAutoStageExtraPages = 4;
constexpr uint64_t kAutoCeilingBytes = 8192ull << 20;

struct Layout {
    uint64_t page_bytes = 0;
    uint64_t ring_bytes = 0;
    uint64_t work_bytes = 0;
    uint64_t src_bytes = 0;    // per layer
    uint64_t seg_bytes = 0;    // per layer
    int32_t max_segs = 0;      // per layer
    int32_t max_groups = 0;
    uint64_t fixed = 0;        // ring + work + tables
};

int validate(const kvs_config* c) {
    if (!c) return fail(KVS_ERR_INVALID_ARG, "config is NULL");
    if (!kvs_type_pair_supported(c->type_k, c->type_v))
        return fail(KVS_ERR_UNSUPPORTED,
                    "K/V block types (%d, %d) have no attention kernel: only Q8_0 keys (%d) with Q4_0 (%d) or Q8_0 values are built",
                    c->type_k, c->type_v, KVS_TYPE_Q8_0, KVS_TYPE_Q4_0);
    if (c->head_dim != kvs::kHeadDim)
        return fail(KVS_ERR_UNSUPPORTED, "head_dim %d unsupported (kernels are built for %d)", c->head_dim, kvs::kHeadDim);
    if (c->page_tokens != kvs::kPageTokens)
        return fail(KVS_ERR_UNSUPPORTED, "page_tokens %d unsupported (pages hold %d tokens)", c->page_tokens, kvs::kPageTokens);
    if (c->n_layers < 1 || c->n_layers > 4096) return fail(KVS_ERR_INVALID_ARG, "n_layers %d out of range [1, 4096]", c->n_layers);
    if (c->n_kv_heads < 1 || c->n_kv_heads > 64) return fail(KVS_ERR_INVALID_ARG, "n_kv_heads %d out of range [1, 64]", c->n_kv_heads);
    if (c->n_q_heads < c->n_kv_heads || c->n_q_heads > 1024 || c->n_q_heads % c->n_kv_heads)
        return fail(KVS_ERR_INVALID_ARG, "n_q_heads %d must be a multiple of n_kv_heads %d (at most 1024)", c->n_q_heads, c->n_kv_heads);
    if (c->max_pages < 1 || c->max_pages > (1 << 22)) return fail(KVS_ERR_INVALID_ARG, "max_pages %d out of range [1, 2^22]", c->max_pages);
    if (c->max_q_tokens < 1 || c->max_q_tokens > 8192) return fail(KVS_ERR_INVALID_ARG, "max_q_tokens %d out of range [1, 8192]", c->max_q_tokens);
    if (c->ring_pages < 1 || c->ring_pages > 4096) return fail(KVS_ERR_INVALID_ARG, "ring_pages %d out of range [1, 4096]", c->ring_pages);
    if (c->chunk_pages < 1 || c->chunk_pages > kvs::kMaxCopyPages || c->ring_pages % c->chunk_pages)
        return fail(KVS_ERR_INVALID_ARG, "chunk_pages %d must be in [1, %d] and divide ring_pages %d", c->chunk_pages,
                    kvs::kMaxCopyPages, c->ring_pages);
    if (c->group_pages < 1) return fail(KVS_ERR_INVALID_ARG, "group_pages %d must be >= 1", c->group_pages);
    if (c->flags & ~uint32_t(KVS_FLAG_POISON_RING | KVS_FLAG_ZERO_COPY))
        return fail(KVS_ERR_INVALID_ARG, "unknown flag bits 0x%x", c->flags);
    return KVS_OK;
}

Layout layout_of(const kvs_config* c) {
    Layout L;
    L.page_bytes = (uint64_t)c->n_kv_heads * kvs::head_record_bytes(c->type_v == KVS_TYPE_Q8_0);
    L.ring_bytes = align256((uint64_t)c->ring_pages * L.page_bytes);
    L.max_groups = (c->max_pages + c->group_pages - 1) / c->group_pages;
    // partials: one record per (group, query token, query head)
    L.work_bytes = align256((uint64_t)L.max_groups * c->max_q_tokens * c->n_q_heads * kvs::kPartStride * sizeof(float));
    // segments: resident groups + (chunk windows add at most one split group each)
    L.max_segs = 2 * L.max_groups + c->max_pages + 1;
    L.src_bytes = align256((uint64_t)c->max_pages * sizeof(int32_t));
    L.seg_bytes = align256((uint64_t)L.max_segs * sizeof(kvs::Seg));
    L.fixed = L.ring_bytes + L.work_bytes + (uint64_t)c->n_layers * (L.src_bytes + L.seg_bytes);
    return L;
}

struct ChunkPlan {
    int32_t seg0 = 0, nseg = 0;   // segments of this chunk's launch
    int32_t rank0 = 0, npages = 0; // streamed ranks [rank0, rank0 + npages)
    std::vector<std::pair<int32_t, int32_t>> runs;  // (first logical page, count) of consecutive streamed pages
};

struct LayerState {
    const uint8_t* host = nullptr;
    int32_t host_pages = 0;
    bool host_new = true;            // records (re)registered since the last upload: upload every resident page
    int32_t pin_slots = 0;           // slots of the pinned region this layer owns (0: it takes general slots)
    std::vector<int32_t> pin_free;   // free slots of that region
    int32_t n_pages = -1;            // -1: page table not set
    std::vector<int32_t> src;        // per page: slot or -1 - rank
    std::vector<int32_t> slots_held;
    std::vector<kvs::Seg> segs;
    int32_t res_nseg = 0;            // segments [0, res_nseg) form the resident launch
    std::vector<ChunkPlan> chunks;
    bool whole_groups = true;        // no split-K group spans two chunk launches
    int32_t n_groups = 0;
    int32_t n_streamed = 0;
    int32_t* dev_src = nullptr;
    kvs::Seg* dev_segs = nullptr;
};

}  // namespace

struct kvs_pool {
    kvs_config cfg{};
    Layout L;
    int device = 0;
    uint8_t* arena = nullptr;
    uint64_t budget = 0;
    uint8_t* ring = nullptr;
    float* work = nullptr;
    uint8_t* slots = nullptr;
    int64_t n_slots = 0;
    std::vector<int32_t> slot_free;  // stack of free slot ids
    std::vector<LayerState> layers;
    hipStream_t pf_stream = nullptr; // prefetches (kvs_stream_enqueue) run here
    int64_t pin_top = 0;             // slots at the top of the slot range held by pinned regions
    int32_t n_cslots = 0;            // chunk slots in the ring
    hipEvent_t pf_done = nullptr;    // recorded on pf_stream after a prefetch
    hipEvent_t ring_free = nullptr;  // recorded on the compute stream after a layer's last ring read
    bool ring_used = false;          // ring_free has been recorded at least once
    hipEvent_t last_work = nullptr;  // recorded after every attend and probe
    bool worked = false;             // last_work has been recorded at least once
    hipEvent_t append_ev = nullptr;  // recorded after every kvs_append
    bool appended = false;           // append_ev has been recorded at least once
    // Compute lanes, used when a layer runs on more than one (otherwise its
    // launches go to the caller's stream). They are created back to back,
    // before any other stream of the pool: the runtime hands streams to its
    // hardware queues in turn, so consecutive streams land on distinct queues
    // and no two lanes serialize on a shared queue (the caller's stream, whose
    // queue is unknown, only forks, joins and combines).
    hipStream_t lanes[kMaxLanes] = {};
    hipEvent_t fork_ev = nullptr;
    hipEvent_t join_ev[kMaxLanes] = {};
    int32_t ring_next = 0;           // chunk slot that receives the next layer's chunk 0
    int32_t pf_layer = -1;           // layer whose chunk 0 was prefetched and not yet consumed
    bool broken = false;             // a HIP call failed mid-sequence
    float* scratch = nullptr;        // device address of the library's scratch array on this device
    kvs_status_info st{};
    // kernel timing (kvs_profile_*): per kind, event pairs in launch order
    bool profiling = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_ev[2];
    size_t prof_used[2] = {0, 0};
};

namespace {

constexpr size_t kMaxTimed = 65536;

bool stream_capturing(hipStream_t s);

// Launch fn() on stream, with a timing pair on its kernel's dispatch when
// profiling is on. Launches under graph capture go untimed: a replay would
// not refill the pair.
template <typename Fn>
hipError_t timed(kvs_pool* p, int kind, hipStream_t s, Fn fn) {
    if (!p->profiling || p->prof_used[kind] >= kMaxTimed || stream_capturing(s)) return fn();
    auto& v = p->prof_ev[kind];
    if (p->prof_used[kind] == v.size()) {
        hipEvent_t a, b;
        hipError_t e = hipEventCreate(&a);
        if (e != hipSuccess) return e;
        e = hipEventCreate(&b);
        if (e != hipSuccess) { (void)hipEventDestroy(a); return e; }
        v.push_back({a, b});
    }
    // the pair rides on the kernel's own dispatch (kvs::launch_kernel), so it
    // times the kernel's execution; a call that launched nothing leaves it
    auto& pr = v[p->prof_used[kind]];
    kvs::launch_timing() = kvs::LaunchTiming{pr.first, pr.second};
    hipError_t e = fn();
    const bool used = kvs::launch_timing().start == nullptr;
    kvs::launch_timing() = kvs::LaunchTiming{};
    if (e == hipSuccess && used) p->prof_used[kind]++;
    return e;
}

int check_device(const kvs_pool* p) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != p->device)
        return fail(KVS_ERR_INVALID_ARG, "pool belongs to device %d but device %d is current", p->device, dev);
    if (p->broken) return fail(KVS_ERR_HIP, "pool is unusable after an earlier HIP failure");
    return KVS_OK;
}

// Build segments and chunk plans for a layer from its residency.
int build_plan(const kvs_config& cfg, int32_t max_segs, LayerState& ls, int32_t n_pages, const uint8_t* resident) {
    const int32_t G = cfg.group_pages, C = cfg.chunk_pages;
    ls.src.assign(n_pages, 0);
    std::vector<int32_t> streamed;
    for (int32_t i = 0; i < n_pages; ++i)
        if (!resident[i]) { ls.src[i] = -1 - (int32_t)streamed.size(); streamed.push_back(i); }
    ls.n_streamed = (int32_t)streamed.size();
    ls.n_groups = (n_pages + G - 1) / G;
    std::vector<char> mixed(ls.n_groups, 0);
    for (int32_t pg : streamed) mixed[pg / G] = 1;
    ls.segs.clear();
    ls.chunks.clear();
    ls.whole_groups = true;
    for (int32_t g = 0; g < ls.n_groups; ++g)
        if (!mixed[g]) ls.segs.push_back({g, g * G, std::min(n_pages, (g + 1) * G) - g * G, kvs::kSegFresh});
    ls.res_nseg = (int32_t)ls.segs.size();
    // Chunks: runs of at most C streamed pages in ascending order. A chunk
    // boundary falls between split-K groups, so that each group is computed by
    // one launch, unless a group alone has more than C streamed pages: its
    // streamed pages then fill consecutive chunks and its running state is
    // carried from one launch to the next.
    std::vector<int32_t> gstream(ls.n_groups, 0);
    for (int32_t pg : streamed) gstream[pg / G]++;
    std::vector<std::pair<int32_t, int32_t>> spans;   // (rank0, npages)
    {
        int32_t rank0 = 0, cur = 0;
        for (int32_t g = 0; g < ls.n_groups; ++g) {
            int32_t sg = gstream[g];
            if (sg == 0) continue;
            if (cur > 0 && (cur + sg > C || sg > C)) { spans.push_back({rank0, cur}); rank0 += cur; cur = 0; }
            if (sg > C) {
                ls.whole_groups = false;
                for (; sg > 0; sg -= std::min(C, sg)) { spans.push_back({rank0, std::min(C, sg)}); rank0 += std::min(C, sg); }
                continue;
            }
            cur += sg;
        }
        if (cur > 0) spans.push_back({rank0, cur});
    }
    const int32_t n_chunks = (int32_t)spans.size();
    // page windows: chunk c owns [bound[c], bound[c + 1]); a bound is the start
    // of the group holding the chunk's first streamed page, or that page itself
    // where a group is split
    std::vector<int32_t> bound(n_chunks + 1, 0);
    bound[n_chunks] = n_pages;
    for (int32_t c = 1; c < n_chunks; ++c) {
        const int32_t first = streamed[spans[c].first], prev_last = streamed[spans[c].first - 1];
        bound[c] = (prev_last / G == first / G) ? first : (first / G) * G;
    }
    for (int32_t c = 0; c < n_chunks; ++c) {
        ChunkPlan cp;
        cp.rank0 = spans[c].first;
        cp.npages = spans[c].second;
        for (int32_t k = 0; k < cp.npages; ++k) {
            int32_t pg = streamed[cp.rank0 + k];
            if (!cp.runs.empty() && cp.runs.back().first + cp.runs.back().second == pg) cp.runs.back().second++;
            else cp.runs.push_back({pg, 1});
        }
        const int32_t w0 = bound[c], w1 = bound[c + 1];
        cp.seg0 = (int32_t)ls.segs.size();
        for (int32_t g = w0 / G; g * G < w1; ++g) {
            if (!mixed[g]) continue;
            int32_t a = std::max(w0, g * G), b = std::min(w1, std::min(n_pages, (g + 1) * G));
            if (a >= b) continue;
            ls.segs.push_back({g, a, b - a, a == g * G ? kvs::kSegFresh : 0});
        }
        cp.nseg = (int32_t)ls.segs.size() - cp.seg0;
        ls.chunks.push_back(std::move(cp));
    }
    // invariants the kernels rely on: every page appears in exactly one segment,
    // pages of a group appear in ascending order, a chunk launch only touches
    // streamed pages of its own chunk
    std::vector<int32_t> seen(n_pages, 0);
    std::vector<int32_t> next_in_group(ls.n_groups, -1);
    for (int32_t g = 0; g < ls.n_groups; ++g) next_in_group[g] = g * G;
    auto check_seg = [&](const kvs::Seg& s, int32_t rank_lo, int32_t rank_hi) -> bool {
        if (s.npages < 1 || s.page0 < 0 || s.page0 + s.npages > n_pages) return false;
        if (s.page0 != next_in_group[s.group]) return false;
        if (((s.flags & kvs::kSegFresh) != 0) != (s.page0 == s.group * G)) return false;
        for (int32_t q = s.page0; q < s.page0 + s.npages; ++q) {
            if (q / G != s.group || seen[q]++) return false;
            if (ls.src[q] < 0) {
                int32_t r = -1 - ls.src[q];
                if (r < rank_lo || r >= rank_hi) return false;
            }
        }
        next_in_group[s.group] = s.page0 + s.npages;
        return true;
    };
    for (int32_t i = 0; i < ls.res_nseg; ++i)
        if (!check_seg(ls.segs[i], 0, 0)) return fail(KVS_ERR_INVALID_ARG, "internal: resident plan check failed");
    for (const ChunkPlan& cp : ls.chunks)
        for (int32_t i = cp.seg0; i < cp.seg0 + cp.nseg; ++i)
            if (!check_seg(ls.segs[i], cp.rank0, cp.rank0 + cp.npages))
                return fail(KVS_ERR_INVALID_ARG, "internal: chunk plan check failed");
    for (int32_t q = 0; q < n_pages; ++q)
        if (seen[q] != 1) return fail(KVS_ERR_INVALID_ARG, "internal: page %d not covered once", q);
    if ((int32_t)ls.segs.size() > max_segs) return fail(KVS_ERR_INVALID_ARG, "internal: too many segments");
    return KVS_OK;
}

kvs::CopyJob make_copy(const kvs_pool* p, const LayerState& ls, int32_t c, int32_t cslot) {
    kvs::CopyJob cj{};
    const ChunkPlan& cp = ls.chunks[c];
    cj.host = ls.host;
    cj.ring_dst = p->ring + (uint64_t)cslot * p->cfg.chunk_pages * p->L.page_bytes;
    cj.page_bytes = (int64_t)p->L.page_bytes;
    cj.n_pages = cp.npages;
    cj.part_bytes = kvs::kCopyPartBytes;
    cj.parts_per_page = (int32_t)((p->L.page_bytes + kvs::kCopyPartBytes - 1) / kvs::kCopyPartBytes);
    int32_t k = 0;
    for (const auto& run : cp.runs)
        for (int32_t j = 0; j < run.second; ++j) cj.pages[k++] = run.first + j;
    return cj;
}

void count_copy(kvs_pool* p, const kvs::CopyJob& cj) {
    if (cj.n_pages <= 0) return;
    p->st.copies_issued++;
    p->st.pages_streamed += cj.n_pages;
    p->st.bytes_h2d += (int64_t)cj.n_pages * cj.page_bytes;
}

// Copy chunk 0 of `layer` into the ring on the pool's copy stream, after the
// previous ring reader is done.
bool stream_capturing(hipStream_t s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return cs != hipStreamCaptureStatusNone;
}

int prefetch(kvs_pool* p, int32_t layer) {
    const LayerState& ls = p->layers[layer];
    hipStream_t cs = p->pf_stream;
    if (p->ring_used) KVS_HIP(hipStreamWaitEvent(cs, p->ring_free, 0));
    if (p->appended) KVS_HIP(hipStreamWaitEvent(cs, p->append_ev, 0));   // host records it copies
    kvs::CopyJob cj = make_copy(p, ls, 0, p->ring_next);
    hipError_t e = kvs::launch_copy(cj, cs);
    if (e != hipSuccess) { p->broken = true; return fail(KVS_ERR_HIP, "prefetch copy launch failed: %s", hipGetErrorString(e)); }
    count_copy(p, cj);
    p->st.kernels_launched++;
    KVS_HIP(hipEventRecord(p->pf_done, cs));
    p->pf_layer = layer;
    return KVS_OK;
}

// Run the layer's launch plan. Ring chunks are moved by copy workgroups
// inside the compute launches; kernel boundaries on a stream order each copy
// before its reader and each reader before its slot is refilled.
//   n lanes (lanes_for: up to kMaxLanes = 3, n dividing the number of chunk
//   slots, which is at least 2 n; and every split-K group computed by a
//   single chunk launch, so that concurrent launches never share a group's
//   state): chunk c is computed on the pool's lane stream c mod n, and the
//   launch that computes chunk c copies chunk c + n, which belongs to the
//   same lane, into a slot last read by that lane (slot count a multiple of
//   n, at least 2 n). The lanes' copies overlap, so the host link stays busy.
//   They meet the caller's stream through one fork event and one join event
//   per lane per layer. Three lanes and the caller's stream fit the four
//   hardware queues a process gets by default: with a fourth lane two lanes
//   could share a queue, and the rate swung between 79 % and 87 % of the
//   link from one pool to the next in a process, against a steady 84-85 %
//   with three.
//   One lane (otherwise): every launch goes to the caller's stream; the
//   launch that computes chunk c copies chunk c + 1 (ring of >= 2 slots), or
//   copies and computes alternate (one slot).
// The resident groups are computed by the first launch of lane 0 (the
// caller's stream with one lane), which also copies chunk 0 unless it was
// prefetched.
// Compute lanes for a layer with n_ch ring chunks over R chunk slots: the
// most lanes n (up to kMaxLanes) with R a multiple of n and at least 2 n, so
// that a lane only ever refills slots it has read itself.
int lanes_for(int32_t R, int32_t n_ch, bool whole_groups) {
    if (n_ch < 2 || !whole_groups) return 1;
    for (int n = kMaxLanes; n >= 2; --n)
        if (n_ch >= n && R >= 2 * n && R % n == 0) return n;
    return 1;
}

template <typename LaunchFn>
int run_layer(kvs_pool* p, int32_t layer, hipStream_t stream, LaunchFn launch) {
    LayerState& ls = p->layers[layer];
    const int32_t n_ch = (int32_t)ls.chunks.size();
    const int32_t R = p->n_cslots;
    auto mark = [&](int r) { if (r) p->broken = true; return r; };
    int rc = KVS_OK;
    const int32_t slot0 = p->ring_next;
    bool prefetched = false;
    if (n_ch > 0 && p->pf_layer == layer) {
        if (hipStreamWaitEvent(stream, p->pf_done, 0) != hipSuccess) return mark(fail(KVS_ERR_HIP, "hipStreamWaitEvent(prefetch) failed"));
        prefetched = true;
    } else if (n_ch > 0 && p->ring_used) {
        if (hipStreamWaitEvent(stream, p->ring_free, 0) != hipSuccess) return mark(fail(KVS_ERR_HIP, "hipStreamWaitEvent(ring) failed"));
    }
    p->pf_layer = -1;
    // rows appended on another stream must be in the host records and slots
    // before this layer's launches read them (under graph capture an outside
    // event cannot be waited on; an append on the captured stream is ordered)
    if (p->appended && !stream_capturing(stream) && hipStreamWaitEvent(stream, p->append_ev, 0) != hipSuccess)
        return mark(fail(KVS_ERR_HIP, "hipStreamWaitEvent(append) failed"));
    if (p->cfg.flags & KVS_FLAG_ZERO_COPY) {
        // Zero-copy: streamed pages are read in place from the host records
        // (the launch's PageSource carries them), so there is no ring. With
        // whole groups every group has one segment, and a single launch takes
        // them all; otherwise each chunk's segments run in their own launch,
        // in order, so that a group's pages still fold in page order.
        const int32_t n_segs = (int32_t)ls.segs.size();
        if (n_segs == 0) return KVS_OK;
        auto run = [&](int32_t seg0, int32_t nseg) -> int {
            if (nseg == 0) return KVS_OK;
            int r = launch(stream, 0, seg0, nseg, nullptr, 0, kvs::CopyJob{});
            if (r) return mark(r);
            p->st.kernels_launched++;
            return KVS_OK;
        };
        if (n_ch == 0 || ls.whole_groups) return run(0, n_segs);
        int r = run(0, ls.res_nseg);
        for (int32_t c = 0; c < n_ch && !r; ++c) r = run(ls.chunks[c].seg0, ls.chunks[c].nseg);
        return r;
    }
    const int n_lanes = lanes_for(R, n_ch, ls.whole_groups);
    auto slot_of = [&](int32_t c) { return (slot0 + c) % R; };
    auto do_launch = [&](int lane, int32_t seg0, int32_t nseg, int32_t c_compute, int32_t c_copy) -> int {
        hipStream_t st = n_lanes > 1 ? p->lanes[lane] : stream;
        kvs::CopyJob cj{};
        if (c_copy >= 0) cj = make_copy(p, ls, c_copy, slot_of(c_copy));
        const uint8_t* ring_chunk = c_compute >= 0 ? p->ring + (uint64_t)slot_of(c_compute) * p->cfg.chunk_pages * p->L.page_bytes : nullptr;
        const int32_t rank0 = c_compute >= 0 ? ls.chunks[c_compute].rank0 : 0;
        int r = launch(st, lane, seg0, nseg, ring_chunk, rank0, cj);
        if (r) return mark(r);
        count_copy(p, cj);
        p->st.kernels_launched++;
        if (c_compute >= 0 && (p->cfg.flags & KVS_FLAG_POISON_RING)) {
            hipError_t e = kvs::launch_fill_u32(const_cast<uint8_t*>(ring_chunk), 0xA5A5A5A5u,
                                                (uint64_t)ls.chunks[c_compute].npages * p->L.page_bytes / 4, st);
            if (e != hipSuccess) return mark(fail(KVS_ERR_HIP, "ring poison fill failed: %s", hipGetErrorString(e)));
        }
        return KVS_OK;
    };
    if (n_lanes > 1) {
        // Lane k starts by copying chunk k into a slot of the ring, which
        // needs only the previous layer's ring reads done: the copy overlaps
        // that layer's combine and this layer's resident launch. Its compute
        // launches write the split-K partials, so they also wait for the
        // caller's stream up to here (the previous combine reads them).
        // Lane 0 takes the resident launch (and chunk 0's copy) after the
        // fork, like the caller's stream it stands in for.
        if (hipEventRecord(p->fork_ev, stream) != hipSuccess) return mark(fail(KVS_ERR_HIP, "lane fork failed"));
        for (int k = 1; k < n_lanes; ++k) {
            if (p->ring_used && hipStreamWaitEvent(p->lanes[k], p->ring_free, 0) != hipSuccess)
                return mark(fail(KVS_ERR_HIP, "lane ring wait failed"));
            if (p->appended && hipStreamWaitEvent(p->lanes[k], p->append_ev, 0) != hipSuccess)
                return mark(fail(KVS_ERR_HIP, "lane append wait failed"));
            if ((rc = do_launch(k, 0, 0, -1, k))) return rc;
            if (hipStreamWaitEvent(p->lanes[k], p->fork_ev, 0) != hipSuccess) return mark(fail(KVS_ERR_HIP, "lane fork failed"));
        }
        if (hipStreamWaitEvent(p->lanes[0], p->fork_ev, 0) != hipSuccess) return mark(fail(KVS_ERR_HIP, "lane fork failed"));
    }
    const int32_t c0 = (n_ch > 0 && !prefetched) ? 0 : -1;
    if (ls.res_nseg > 0 || c0 >= 0) {
        if ((rc = do_launch(0, 0, ls.res_nseg, -1, c0))) return rc;
    }
    if (n_lanes > 1) {
        for (int32_t c = 0; c < n_ch; ++c) {
            const ChunkPlan& cp = ls.chunks[c];
            const int32_t cc = (c + n_lanes < n_ch) ? c + n_lanes : -1;
            if ((rc = do_launch(c % n_lanes, cp.seg0, cp.nseg, c, cc))) return rc;
        }
        for (int k = 0; k < n_lanes; ++k)
            if (hipEventRecord(p->join_ev[k], p->lanes[k]) != hipSuccess || hipStreamWaitEvent(stream, p->join_ev[k], 0) != hipSuccess)
                return mark(fail(KVS_ERR_HIP, "lane join failed"));
    } else {
        for (int32_t c = 0; c < n_ch; ++c) {
            const ChunkPlan& cp = ls.chunks[c];
            if (R >= 2) {
                const int32_t cc = (c + 1 < n_ch) ? c + 1 : -1;
                if ((rc = do_launch(0, cp.seg0, cp.nseg, c, cc))) return rc;
            } else {
                if ((rc = do_launch(0, cp.seg0, cp.nseg, c, -1))) return rc;
                if (c + 1 < n_ch && (rc = do_launch(0, 0, 0, -1, c + 1))) return rc;
            }
        }
    }
    if (n_ch > 0) {
        p->ring_next = slot_of(n_ch);
        if (hipEventRecord(p->ring_free, stream) != hipSuccess) return mark(fail(KVS_ERR_HIP, "hipEventRecord(ring) failed"));
        p->ring_used = true;
    }
    return KVS_OK;
}

int check_layer_ready(const kvs_pool* p, int32_t layer) {
    if (layer < 0 || layer >= p->cfg.n_layers) return fail(KVS_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, p->cfg.n_layers);
    const LayerState& ls = p->layers[layer];
    if (!ls.host) return fail(KVS_ERR_NOT_READY, "layer %d has no host pages (call kvs_host_pages_set)", layer);
    if (ls.n_pages < 0) return fail(KVS_ERR_NOT_READY, "layer %d has no page table (call kvs_page_table_set)", layer);
    return KVS_OK;
}

// Ring chunks are ordered by events across the pool's copy streams; a graph
// captured from the compute stream cannot replay that exchange faithfully.
int check_capture(const kvs_pool* p, int32_t layer, hipStream_t s) {
    if (p->layers[layer].chunks.empty() || (p->cfg.flags & KVS_FLAG_ZERO_COPY)) return KVS_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return KVS_OK;
    }
    if (cs != hipStreamCaptureStatusNone)
        return fail(KVS_ERR_UNSUPPORTED, "layer %d streams pages through the ring, which cannot be captured in a graph", layer);
    return KVS_OK;
}

// Work of this pool issued on another stream (an earlier attend's combine
// still reading the split-K workspace, or a probe) must be done before a new
// call's launches reuse that memory: the call's stream
// waits for the pool's last recorded work. Under graph capture an outside
// event cannot be waited on; a captured sequence runs on the capture stream,
// which orders it.
int order_after_last_work(kvs_pool* p, hipStream_t s) {
    if (!p->worked || stream_capturing(s)) return KVS_OK;
    if (hipStreamWaitEvent(s, p->last_work, 0) != hipSuccess) {
        p->broken = true;
        return fail(KVS_ERR_HIP, "hipStreamWaitEvent(last work) failed");
    }
    return KVS_OK;
}

int record_last_work(kvs_pool* p, hipStream_t s) {
    if (hipEventRecord(p->last_work, s) != hipSuccess) {
        p->broken = true;
        return fail(KVS_ERR_HIP, "hipEventRecord failed");
    }
    p->worked = true;
    return KVS_OK;
}

int64_t pinned_free_count(const kvs_pool* p) {
    int64_t n = 0;
    for (const auto& ls : p->layers) n += (int64_t)ls.pin_free.size();
    return n;
}

int check_ring_free_for(const kvs_pool* p, int32_t layer) {
    const LayerState& ls = p->layers[layer];
    if (!ls.chunks.empty() && p->pf_layer >= 0 && p->pf_layer != layer)
        return fail(KVS_ERR_STATE, "ring holds an unconsumed prefetch of layer %d; attend it before layer %d", p->pf_layer, layer);
    return KVS_OK;
}

}  // namespace

extern "C" {

int kvs_type_pair_supported(int32_t type_k, int32_t type_v) {
    return type_k == KVS_TYPE_Q8_0 && (type_v == KVS_TYPE_Q4_0 || type_v == KVS_TYPE_Q8_0);
}

int kvs_config_validate(const kvs_config* cfg) { return validate(cfg); }

uint64_t kvs_page_bytes(const kvs_config* cfg) {
    if (validate(cfg)) return 0;
    return layout_of(cfg).page_bytes;
}

int kvs_min_budget_bytes(const kvs_config* cfg, uint64_t* out) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!out) return fail(KVS_ERR_INVALID_ARG, "out is NULL");
    *out = layout_of(cfg).fixed;
    return KVS_OK;
}

int kvs_plan_layer(const kvs_config* cfg, int32_t n_pages, const uint8_t* resident, kvs_plan_info* info,
                   int32_t* segs, int32_t seg_cap, int32_t* chunks, int32_t chunk_cap) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (n_pages < 0 || n_pages > cfg->max_pages)
        return fail(KVS_ERR_INVALID_ARG, "n_pages %d out of range [0, max_pages %d]", n_pages, cfg->max_pages);
    if ((n_pages > 0 && !resident) || !info) return fail(KVS_ERR_INVALID_ARG, "resident or info is NULL");
    LayerState ls;
    rc = build_plan(*cfg, layout_of(cfg).max_segs, ls, n_pages, resident);
    if (rc) return rc;
    info->n_groups = ls.n_groups;
    info->n_streamed = ls.n_streamed;
    info->n_segs = (int32_t)ls.segs.size();
    info->n_resident_segs = ls.res_nseg;
    info->n_chunks = (int32_t)ls.chunks.size();
    info->whole_groups = ls.whole_groups ? 1 : 0;
    if (segs) {
        if (seg_cap < info->n_segs) return fail(KVS_ERR_INVALID_ARG, "seg_cap %d < %d segments", seg_cap, info->n_segs);
        for (int32_t i = 0; i < info->n_segs; ++i) {
            segs[4 * i] = ls.segs[i].group;
            segs[4 * i + 1] = ls.segs[i].page0;
            segs[4 * i + 2] = ls.segs[i].npages;
            segs[4 * i + 3] = ls.segs[i].flags;
        }
    }
    if (chunks) {
        if (chunk_cap < info->n_chunks) return fail(KVS_ERR_INVALID_ARG, "chunk_cap %d < %d chunks", chunk_cap, info->n_chunks);
        for (int32_t c = 0; c < info->n_chunks; ++c) {
            chunks[4 * c] = ls.chunks[c].rank0;
            chunks[4 * c + 1] = ls.chunks[c].npages;
            chunks[4 * c + 2] = ls.chunks[c].seg0;
            chunks[4 * c + 3] = ls.chunks[c].nseg;
        }
    }
    return KVS_OK;
}

int64_t kvs_slots_for_budget(const kvs_config* cfg, uint64_t budget_bytes) {
    if (validate(cfg)) return 0;
    Layout L = layout_of(cfg);
    if (budget_bytes < L.fixed) return 0;
    return std::min<int64_t>((int64_t)((budget_bytes - L.fixed) / L.page_bytes), kvs::kMaxSlots);
}

int32_t kvs_auto_resident_pages(int64_t n_ctx) {
    if (n_ctx <= 0) return 0;
    const int64_t T = kvs::kPageTokens;
    const int64_t ctx_pages = (n_ctx + T - 1) / T;
    const int64_t tenth = (n_ctx + 9) / 10;                 // ceil(0.1 n_ctx) tokens
    int64_t pages = (tenth + T - 1) / T;                    // whole pages, rounded up
    pages = std::max<int64_t>(pages, (kAutoFloorTokens + T - 1) / T);
    pages = std::min(pages, ctx_pages);
    return (int32_t)std::min<int64_t>(pages, INT32_MAX);
}

uint64_t kvs_auto_stage_bytes(int32_t n_layers, int64_t n_ctx, uint64_t bytes_per_token) {
    if (n_layers <= 0 || n_ctx <= 0 || bytes_per_token == 0) return 0;
    const uint64_t pages = (uint64_t)kvs_auto_resident_pages(n_ctx) + kAutoStageExtraPages;
    const long double bytes = (long double)n_layers * pages * kvs::kPageTokens * bytes_per_token;
    return bytes >= (long double)kAutoCeilingBytes ? kAutoCeilingBytes : (uint64_t)bytes;
}

int kvs_auto_budget_bytes(const kvs_config* cfg, int64_t n_ctx, uint64_t* out) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!out) return fail(KVS_ERR_INVALID_ARG, "out is NULL");
    if (n_ctx < 0) return fail(KVS_ERR_INVALID_ARG, "n_ctx %lld < 0", (long long)n_ctx);
    const Layout L = layout_of(cfg);
    const long double want = (long double)L.fixed +
                             (long double)cfg->n_layers * kvs_auto_resident_pages(n_ctx) * L.page_bytes;
    uint64_t b = want >= (long double)kAutoCeilingBytes ? kAutoCeilingBytes : (uint64_t)want;
    *out = std::max<uint64_t>(b, L.fixed);
    return KVS_OK;
}

int kvs_residency_promote_newest(const uint8_t* cur, int32_t n_cur, int32_t n_new, int32_t max_resident, uint8_t* out) {
    if (n_cur < 0 || n_new < n_cur) return fail(KVS_ERR_INVALID_ARG, "page counts %d -> %d must not shrink", n_cur, n_new);
    if (max_resident < 0) return fail(KVS_ERR_INVALID_ARG, "max_resident %d < 0", max_resident);
    if ((n_cur > 0 && !cur) || (n_new > 0 && !out)) return fail(KVS_ERR_INVALID_ARG, "mask is NULL");
    std::vector<uint8_t> m(n_new, 0);
    for (int32_t i = 0; i < n_cur; ++i) m[i] = cur[i] ? 1 : 0;
    int64_t resident = 0;
    for (uint8_t v : m) resident += v;
    int32_t oldest = 0;                       // scan position for the oldest resident page
    for (int32_t i = n_cur; i < n_new; ++i) {
        if (max_resident == 0) break;
        m[i] = 1;
        ++resident;
        while (resident > max_resident) {
            while (oldest < i && !m[oldest]) ++oldest;
            m[oldest] = 0;                    // oldest < i: the new page itself is never evicted here
            --resident;
        }
    }
    for (int32_t i = 0; i < n_new; ++i) out[i] = m[i];
    return KVS_OK;
}

int kvs_pool_create(const kvs_config* cfg, void* dev_arena, uint64_t budget_bytes, kvs_pool** out_pool) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!out_pool) return fail(KVS_ERR_INVALID_ARG, "out_pool is NULL");
    if (!dev_arena) return fail(KVS_ERR_INVALID_ARG, "device arena is NULL");
    if ((uintptr_t)dev_arena & 255) return fail(KVS_ERR_INVALID_ARG, "device arena must be 256-byte aligned");
    Layout L = layout_of(cfg);
    if (budget_bytes < L.fixed)
        return fail(KVS_ERR_BUDGET, "budget %llu B is below the minimum %llu B (ring %llu + workspace %llu + tables)",
                    (unsigned long long)budget_bytes, (unsigned long long)L.fixed,
                    (unsigned long long)L.ring_bytes, (unsigned long long)L.work_bytes);
    kvs_pool* p = new kvs_pool();
    p->cfg = *cfg;
    p->L = L;
    p->arena = (uint8_t*)dev_arena;
    p->budget = budget_bytes;
    if (hipGetDevice(&p->device) != hipSuccess) { delete p; return fail(KVS_ERR_HIP, "hipGetDevice failed"); }
    uint8_t* cur = p->arena;
    p->ring = cur; cur += L.ring_bytes;
    p->work = (float*)cur; cur += L.work_bytes;
    p->layers.resize(cfg->n_layers);
    for (auto& ls : p->layers) {
        ls.dev_src = (int32_t*)cur; cur += L.src_bytes;
        ls.dev_segs = (kvs::Seg*)cur; cur += L.seg_bytes;
    }
    p->slots = cur;
    p->n_slots = std::min<int64_t>((int64_t)((budget_bytes - L.fixed) / L.page_bytes), kvs::kMaxSlots);
    for (int64_t s = p->n_slots - 1; s >= 0; --s) p->slot_free.push_back((int32_t)s);
    p->n_cslots = cfg->ring_pages / cfg->chunk_pages;
    auto cleanup = [&](const char* what, hipError_t e) {
        if (p->pf_stream) (void)hipStreamDestroy(p->pf_stream);
        for (auto s : p->lanes) if (s) (void)hipStreamDestroy(s);
        for (hipEvent_t ev : {p->pf_done, p->ring_free, p->last_work, p->fork_ev, p->append_ev}) if (ev) (void)hipEventDestroy(ev);
        for (hipEvent_t ev : p->join_ev) if (ev) (void)hipEventDestroy(ev);
        delete p;
        return fail(KVS_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
    };
    for (int k = 0; k < kMaxLanes; ++k) {   // first and back to back: one hardware queue each
        hipError_t e = hipStreamCreateWithFlags(&p->lanes[k], hipStreamNonBlocking);
        if (e != hipSuccess) return cleanup("hipStreamCreateWithFlags", e);
    }
    {
        hipError_t e = hipStreamCreateWithFlags(&p->pf_stream, hipStreamNonBlocking);
        if (e != hipSuccess) return cleanup("hipStreamCreateWithFlags", e);
    }
    for (hipEvent_t* ev : {&p->pf_done, &p->ring_free, &p->last_work, &p->fork_ev, &p->append_ev}) {
        hipError_t e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
        if (e != hipSuccess) return cleanup("hipEventCreateWithFlags", e);
    }
    for (int k = 0; k < kMaxLanes; ++k) {
        hipError_t e = hipEventCreateWithFlags(&p->join_ev[k], hipEventDisableTiming);
        if (e != hipSuccess) return cleanup("hipEventCreateWithFlags", e);
    }
    {
        // set-up of kvs_attend_noalloc: the scratch array's address on this device
        hipError_t e = kvs::scratch_region(&p->scratch);
        if (e != hipSuccess) return cleanup("hipGetSymbolAddress(scratch)", e);
    }
    p->st.page_bytes = (int64_t)L.page_bytes;
    p->st.slot_count = p->n_slots;
    p->st.ring_pages = cfg->ring_pages;
    p->st.workspace_bytes = (int64_t)L.work_bytes;
    if (getenv("KVS_LOG"))
        fprintf(stderr, "kvs: pool on device %d: budget %.2f MiB, minimum %.2f MiB, page %.4f MiB, %lld slots, ring %d pages, %d layers\n",
                p->device, budget_bytes / 1048576.0, L.fixed / 1048576.0, L.page_bytes / 1048576.0,
                (long long)p->n_slots, cfg->ring_pages, cfg->n_layers);
    *out_pool = p;
    return KVS_OK;
}

void kvs_pool_destroy(kvs_pool* p) {
    if (!p) return;
    if (p->pf_stream) (void)hipStreamSynchronize(p->pf_stream);
    if (p->last_work) (void)hipEventSynchronize(p->last_work);
    if (p->appended) (void)hipEventSynchronize(p->append_ev);
    for (auto s : p->lanes) if (s) (void)hipStreamSynchronize(s);
    if (p->pf_stream) (void)hipStreamDestroy(p->pf_stream);
    for (auto s : p->lanes) if (s) (void)hipStreamDestroy(s);
    for (hipEvent_t ev : {p->pf_done, p->ring_free, p->last_work, p->fork_ev, p->append_ev}) if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : p->join_ev) if (ev) (void)hipEventDestroy(ev);
    for (auto& v : p->prof_ev)
        for (auto& pr : v) { (void)hipEventDestroy(pr.first); (void)hipEventDestroy(pr.second); }
    delete p;
}

int kvs_host_pages_set(kvs_pool* p, int32_t layer, const void* pinned_records, int32_t n_pages) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    if (layer < 0 || layer >= p->cfg.n_layers) return fail(KVS_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, p->cfg.n_layers);
    if (!pinned_records || n_pages < 1) return fail(KVS_ERR_INVALID_ARG, "host records NULL or n_pages %d < 1", n_pages);
    if (p->pf_layer == layer) return fail(KVS_ERR_STATE, "layer %d has copies in flight from its prefetch", layer);
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, pinned_records) != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(KVS_ERR_UNSUPPORTED, "host records of layer %d are not pinned host memory", layer);
    }
    LayerState& ls = p->layers[layer];
    if (ls.n_pages > n_pages) return fail(KVS_ERR_INVALID_ARG, "layer %d's page table holds %d pages, more than %d host pages", layer, ls.n_pages, n_pages);
    ls.host = (const uint8_t*)pinned_records;
    ls.host_pages = n_pages;
    ls.host_new = true;   // resident slots no longer mirror the records: upload them all on the next table set
    return KVS_OK;
}

int kvs_page_table_set(kvs_pool* p, int32_t layer, int32_t n_pages, const uint8_t* resident, void* stream) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    if (layer < 0 || layer >= p->cfg.n_layers) return fail(KVS_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, p->cfg.n_layers);
    LayerState& ls = p->layers[layer];
    if (!ls.host) return fail(KVS_ERR_NOT_READY, "layer %d has no host pages (call kvs_host_pages_set first)", layer);
    if (n_pages < 0 || n_pages > p->cfg.max_pages || n_pages > ls.host_pages)
        return fail(KVS_ERR_INVALID_ARG, "n_pages %d out of range [0, min(max_pages %d, host pages %d)]", n_pages, p->cfg.max_pages, ls.host_pages);
    if (n_pages > 0 && !resident) return fail(KVS_ERR_INVALID_ARG, "resident mask is NULL");
    if (p->pf_layer == layer) return fail(KVS_ERR_STATE, "layer %d has an unconsumed prefetch", layer);
    // Pages that stay resident keep their slots (and their device copy, which
    // kvs_append keeps in step with the host record); only newly resident
    // pages are uploaded, unless the host records were registered again.
    const bool keep_ok = ls.n_pages >= 0 && !ls.host_new;
    std::vector<int32_t> keep(n_pages, -1);
    int64_t need = 0, kept = 0;
    for (int32_t i = 0; i < n_pages; ++i) {
        if (!resident[i]) continue;
        ++need;
        if (keep_ok && i < ls.n_pages && ls.src[i] >= 0) { keep[i] = ls.src[i]; ++kept; }
    }
    // slots this call can hand out: the layer's slots that are not kept, then
    // free ones (of the layer's pinned region for a pinned layer)
    std::vector<char> kept_slot;
    std::vector<int32_t> reuse;
    {
        std::vector<int32_t> kept_ids;
        for (int32_t i = 0; i < n_pages; ++i) if (keep[i] >= 0) kept_ids.push_back(keep[i]);
        std::sort(kept_ids.begin(), kept_ids.end());
        for (int32_t sl : ls.slots_held)
            if (!std::binary_search(kept_ids.begin(), kept_ids.end(), sl)) reuse.push_back(sl);
    }
    const std::vector<int32_t>& free_list = ls.pin_slots ? ls.pin_free : p->slot_free;
    const int64_t avail = (int64_t)reuse.size() + (int64_t)free_list.size();
    if (need - kept > avail)
        return fail(KVS_ERR_NO_SLOTS, "layer %d wants %lld resident pages but only %lld slots are free%s", layer, (long long)need,
                    (long long)(kept + avail), ls.pin_slots ? " in its pinned region" : "");
    LayerState trial;
    trial.host = ls.host;
    trial.host_pages = ls.host_pages;
    trial.host_new = false;
    trial.pin_slots = ls.pin_slots;
    trial.dev_src = ls.dev_src;
    trial.dev_segs = ls.dev_segs;
    rc = build_plan(p->cfg, p->L.max_segs, trial, n_pages, resident);
    if (rc) return rc;
    // assign slots (no pool state changes yet): kept ones, then the layer's
    // released ones, then free ones from the top of the free stack
    std::vector<int32_t> free_after(free_list);
    std::vector<std::pair<int32_t, int32_t>> uploads;   // (page, slot)
    size_t ri = 0;
    for (int32_t i = 0; i < n_pages; ++i) {
        if (!resident[i]) continue;
        int32_t sl = keep[i];
        if (sl < 0) {
            if (ri < reuse.size()) sl = reuse[ri++];
            else { sl = free_after.back(); free_after.pop_back(); }
            uploads.push_back({i, sl});
        }
        trial.src[i] = sl;
        trial.slots_held.push_back(sl);
    }
    for (; ri < reuse.size(); ++ri) free_after.push_back(reuse[ri]);
    // device work: the uploads go to slots nothing else reads once the pool's
    // earlier work is done. A HIP failure from here on leaves the device
    // tables in an unknown state, so it marks the pool unusable.
    hipStream_t s = (hipStream_t)stream;
    auto hip_fail = [&](const char* what, hipError_t e) {
        p->broken = true;
        return fail(KVS_ERR_HIP, "%s failed: %s (the pool is unusable)", what, hipGetErrorString(e));
    };
    hipError_t e = hipSuccess;
    if (p->worked && (e = hipStreamWaitEvent(s, p->last_work, 0)) != hipSuccess) return hip_fail("hipStreamWaitEvent", e);
    if (p->appended && (e = hipStreamWaitEvent(s, p->append_ev, 0)) != hipSuccess) return hip_fail("hipStreamWaitEvent", e);
    int64_t uploaded = 0;
    for (const auto& u : uploads) {
        e = hipMemcpyAsync(p->slots + (uint64_t)u.second * p->L.page_bytes, ls.host + (uint64_t)u.first * p->L.page_bytes,
                           p->L.page_bytes, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail("hipMemcpyAsync(resident page)", e);
        uploaded += (int64_t)p->L.page_bytes;
    }
    if (n_pages > 0 && (e = hipMemcpyAsync(trial.dev_src, trial.src.data(), n_pages * sizeof(int32_t), hipMemcpyHostToDevice, s)) != hipSuccess)
        return hip_fail("hipMemcpyAsync(page table)", e);
    // device copy of the segments: flags bits 8.. carry src[page0] (slot
    // indices below kMaxSlots, streamed ranks below max_pages <= 2^22)
    std::vector<kvs::Seg> dsegs(trial.segs);
    for (kvs::Seg& sg : dsegs)
        sg.flags = (sg.flags & kvs::kSegFlagMask) | (int32_t)((uint32_t)trial.src[sg.page0] << kvs::kSegSrcShift);
    if (!dsegs.empty() &&
        (e = hipMemcpyAsync(trial.dev_segs, dsegs.data(), dsegs.size() * sizeof(kvs::Seg), hipMemcpyHostToDevice, s)) != hipSuccess)
        return hip_fail("hipMemcpyAsync(segments)", e);
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail("hipStreamSynchronize", e);
    // commit
    if (ls.pin_slots) trial.pin_free = std::move(free_after);
    else p->slot_free = std::move(free_after);
    trial.n_pages = n_pages;
    ls = std::move(trial);
    p->st.resident_upload_bytes += uploaded;
    p->st.slots_used = p->n_slots - (int64_t)p->slot_free.size() - pinned_free_count(p);
    return KVS_OK;
}

int kvs_pool_pin_layer(kvs_pool* p, int32_t layer, int32_t n_slots) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    if (layer < 0 || layer >= p->cfg.n_layers) return fail(KVS_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, p->cfg.n_layers);
    if (n_slots < 1) return fail(KVS_ERR_INVALID_ARG, "n_slots %d < 1", n_slots);
    LayerState& ls = p->layers[layer];
    if (ls.pin_slots) return fail(KVS_ERR_STATE, "layer %d already has a pinned region", layer);
    if (!ls.slots_held.empty()) return fail(KVS_ERR_STATE, "layer %d holds resident slots; set an empty page table before pinning it", layer);
    if (p->pin_top + n_slots > p->n_slots)
        return fail(KVS_ERR_NO_SLOTS, "a pinned region of %d slots does not fit: %lld of %lld slots are pinned already", n_slots,
                    (long long)p->pin_top, (long long)p->n_slots);
    // bump allocation from the top: slots [top - n_slots, top) must be free
    const int64_t hi = p->n_slots - p->pin_top, lo = hi - n_slots;
    std::vector<char> is_free(p->n_slots, 0);
    for (int32_t sl : p->slot_free) is_free[sl] = 1;
    for (int64_t sl = lo; sl < hi; ++sl)
        if (!is_free[sl])
            return fail(KVS_ERR_NO_SLOTS, "slot %lld at the top of the pool is held by a resident page; release it before pinning %d slots",
                        (long long)sl, n_slots);
    std::vector<int32_t> rest;
    for (int32_t sl : p->slot_free) if (sl < lo || sl >= hi) rest.push_back(sl);
    p->slot_free = std::move(rest);
    ls.pin_free.clear();
    for (int64_t sl = hi - 1; sl >= lo; --sl) ls.pin_free.push_back((int32_t)sl);   // lowest handed out first
    ls.pin_slots = n_slots;
    p->pin_top += n_slots;
    p->st.pinned_slots = p->pin_top;
    return KVS_OK;
}

int kvs_pool_reset_pinned(kvs_pool* p) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    for (int32_t l = 0; l < p->cfg.n_layers; ++l)
        if (p->layers[l].pin_slots && !p->layers[l].slots_held.empty())
            return fail(KVS_ERR_STATE, "pinned layer %d still holds resident pages; set an empty page table first", l);
    for (auto& ls : p->layers) {
        if (!ls.pin_slots) continue;
        for (int32_t sl : ls.pin_free) p->slot_free.push_back(sl);
        ls.pin_free.clear();
        ls.pin_slots = 0;
    }
    p->pin_top = 0;
    p->st.pinned_slots = 0;
    return KVS_OK;
}

int kvs_stream_enqueue(kvs_pool* p, int32_t layer) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    if ((rc = check_layer_ready(p, layer))) return rc;
    if (p->pf_layer == layer) return KVS_OK;  // already prefetched
    if ((rc = check_ring_free_for(p, layer))) return rc;
    if (p->layers[layer].chunks.empty() || (p->cfg.flags & KVS_FLAG_ZERO_COPY)) return KVS_OK;
    return prefetch(p, layer);
}

}  // extern "C"

namespace {

// kvs_attend and kvs_attend_noalloc: the split-K partials go to the pool's
// workspace, or (noalloc) to the library's scratch array, and a noalloc call
// creates no timing events.
int attend_impl(kvs_pool* p, int32_t layer, const void* q, int32_t q_dtype, int32_t n_q, int64_t q_pos0, int64_t n_kv,
                float scale, int32_t causal, float* out, float* lse, void* stream, bool noalloc) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    if ((rc = check_layer_ready(p, layer))) return rc;
    const LayerState& ls = p->layers[layer];
    if (n_q < 1) return fail(KVS_ERR_INVALID_ARG, "n_q %d < 1", n_q);
    if (n_q > p->cfg.max_q_tokens)
        return fail(KVS_ERR_BATCH_TOO_WIDE, "query block of %d tokens is wider than max_q_tokens %d", n_q, p->cfg.max_q_tokens);
    if (!q || !out) return fail(KVS_ERR_INVALID_ARG, "q or out is NULL");
    if (q_dtype != KVS_Q_F32 && q_dtype != KVS_Q_F16) return fail(KVS_ERR_INVALID_ARG, "q_dtype %d unknown", q_dtype);
    if (!std::isfinite(scale)) return fail(KVS_ERR_INVALID_ARG, "scale is not finite");
    if (n_kv < 0 || (n_kv + kvs::kPageTokens - 1) / kvs::kPageTokens != ls.n_pages)
        return fail(KVS_ERR_INVALID_ARG, "n_kv %lld does not fill the layer's %d pages", (long long)n_kv, ls.n_pages);
    if (causal && (q_pos0 < 0 || q_pos0 + n_q > n_kv))
        return fail(KVS_ERR_INVALID_ARG, "causal queries at positions [%lld, %lld) must lie inside the cache of %lld tokens",
                    (long long)q_pos0, (long long)(q_pos0 + n_q), (long long)n_kv);
    if (noalloc) {
        const uint64_t need = (uint64_t)ls.n_groups * n_q * p->cfg.n_q_heads * kvs::kPartStride * sizeof(float);
        if (need > kvs::kScratchBytes)
            return fail(KVS_ERR_INVALID_ARG,
                        "kvs_attend_noalloc needs %llu bytes of split-K scratch (%d groups x %d query tokens x %d heads), "
                        "above its fixed %llu bytes; use kvs_attend or larger group_pages",
                        (unsigned long long)need, ls.n_groups, n_q, p->cfg.n_q_heads, (unsigned long long)kvs::kScratchBytes);
    }
    if ((rc = check_ring_free_for(p, layer))) return rc;
    hipStream_t s = (hipStream_t)stream;
    if ((rc = check_capture(p, layer, s))) return rc;
    if ((rc = order_after_last_work(p, s))) return rc;
    float* part = noalloc ? p->scratch : p->work;
    // a noalloc call creates no timing events
    auto timed_or_not = [&](int kind, hipStream_t st, auto fn) -> hipError_t {
        return noalloc ? fn() : timed(p, kind, st, fn);
    };

    kvs::AttendArgs a{};
    a.ps.slots = p->slots;
    a.ps.src = ls.dev_src;
    a.ps.host = (p->cfg.flags & KVS_FLAG_ZERO_COPY) ? ls.host : nullptr;
    a.ps.page_bytes = (int64_t)p->L.page_bytes;
    a.n_kv_heads = p->cfg.n_kv_heads;
    a.n_q_heads = p->cfg.n_q_heads;
    a.G = p->cfg.n_q_heads / p->cfg.n_kv_heads;
    a.q = q;
    a.q_f16 = q_dtype == KVS_Q_F16;
    a.v_q8 = p->cfg.type_v == KVS_TYPE_Q8_0;
    a.n_q = n_q;
    a.q_pos0 = q_pos0;
    a.n_kv = n_kv;
    a.scale_log2 = scale * 1.44269504088896340736f;
    a.causal = causal ? 1 : 0;
    a.part = part;
    a.spare = p->ring;
    const bool wide = kvs::prefill_rows(n_q * a.G);
    rc = run_layer(p, layer, s, [&](hipStream_t st, int /*lane*/, int32_t seg0, int32_t nseg, const uint8_t* ring_chunk,
                                    int32_t rank0, const kvs::CopyJob& cj) -> int {
        kvs::AttendArgs b = a;
        b.copy = cj;
        b.ps.ring_chunk = ring_chunk;
        b.ps.chunk_rank0 = rank0;
        if (nseg == 0) {   // a copy-only launch: the plain copy kernel, no compute footprint
            hipError_t e = kvs::launch_copy(cj, st);
            return e == hipSuccess ? KVS_OK : fail(KVS_ERR_HIP, "ring copy launch failed: %s", hipGetErrorString(e));
        }
        b.segs = ls.dev_segs + seg0;
        b.n_segs = nseg;
        // A prefill-width launch's workgroups hold most of a compute unit's
        // LDS, and so does each of its copy workgroups: a few copy workgroups
        // of whole pages keep the link as busy as many small ones and take
        // fewer compute units from the attention.
        if (wide && cj.n_pages > 0) b.copy = kvs::with_part_bytes(cj, (int64_t)kvs::kCopyPartBytes * kWideCopyRounds);
        hipError_t e = timed_or_not(0, st, [&] { return kvs::launch_attend(b, st); });
        return e == hipSuccess ? KVS_OK : fail(KVS_ERR_HIP, "attention kernel launch failed: %s", hipGetErrorString(e));
    });
    if (rc) return rc;
    hipError_t e = timed_or_not(1, s, [&] { return kvs::launch_combine(part, ls.n_groups, n_q, p->cfg.n_q_heads, out, lse, s); });
    if (e != hipSuccess) { p->broken = true; return fail(KVS_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e)); }
    p->st.kernels_launched++;
    return record_last_work(p, s);
}

}  // namespace

extern "C" {

int kvs_attend(kvs_pool* p, int32_t layer, const void* q, int32_t q_dtype, int32_t n_q, int64_t q_pos0, int64_t n_kv,
               float scale, int32_t causal, float* out, float* lse, void* stream) {
    return attend_impl(p, layer, q, q_dtype, n_q, q_pos0, n_kv, scale, causal, out, lse, stream, false);
}

int kvs_attend_noalloc(kvs_pool* p, int32_t layer, const void* q, int32_t q_dtype, int32_t n_q, int64_t q_pos0,
                       int64_t n_kv, float scale, int32_t causal, float* out, float* lse, void* stream) {
    return attend_impl(p, layer, q, q_dtype, n_q, q_pos0, n_kv, scale, causal, out, lse, stream, true);
}

int kvs_status(const kvs_pool* p, kvs_status_info* info) {
    if (!p || !info) return fail(KVS_ERR_INVALID_ARG, "pool or info is NULL");
    *info = p->st;
    return KVS_OK;
}

int kvs_debug_gather(kvs_pool* p, int32_t layer, int64_t tok0, int64_t n_tok, float* k_out, float* v_out, void* stream) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    if ((rc = check_layer_ready(p, layer))) return rc;
    const LayerState& ls = p->layers[layer];
    if (tok0 < 0 || n_tok < 0 || tok0 + n_tok > (int64_t)ls.n_pages * kvs::kPageTokens)
        return fail(KVS_ERR_INVALID_ARG, "tokens [%lld, %lld) outside the layer's %d pages", (long long)tok0, (long long)(tok0 + n_tok), ls.n_pages);
    if (n_tok > 0 && (!k_out || !v_out)) return fail(KVS_ERR_INVALID_ARG, "k_out or v_out is NULL");
    if ((rc = check_ring_free_for(p, layer))) return rc;
    hipStream_t s = (hipStream_t)stream;
    if ((rc = check_capture(p, layer, s))) return rc;
    if ((rc = order_after_last_work(p, s))) return rc;
    kvs::GatherArgs a{};
    a.ps.slots = p->slots;
    a.ps.src = ls.dev_src;
    a.ps.host = (p->cfg.flags & KVS_FLAG_ZERO_COPY) ? ls.host : nullptr;
    a.ps.page_bytes = (int64_t)p->L.page_bytes;
    a.n_kv_heads = p->cfg.n_kv_heads;
    a.tok0 = tok0;
    a.n_tok = n_tok;
    a.k_out = k_out;
    a.v_out = v_out;
    a.v_q8 = p->cfg.type_v == KVS_TYPE_Q8_0;
    rc = run_layer(p, layer, s, [&](hipStream_t st, int /*lane*/, int32_t seg0, int32_t nseg, const uint8_t* ring_chunk,
                                    int32_t rank0, const kvs::CopyJob& cj) -> int {
        kvs::GatherArgs b = a;
        b.copy = cj;
        b.ps.ring_chunk = ring_chunk;
        b.ps.chunk_rank0 = rank0;
        b.segs = ls.dev_segs + seg0;
        b.n_segs = nseg;
        hipError_t e = kvs::launch_gather(b, st);
        return e == hipSuccess ? KVS_OK : fail(KVS_ERR_HIP, "gather kernel launch failed: %s", hipGetErrorString(e));
    });
    if (rc) return rc;
    return record_last_work(p, s);
}

int kvs_debug_stage(kvs_pool* p, int32_t layer, int64_t n_kv, void* dst, void* stream) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    if ((rc = check_layer_ready(p, layer))) return rc;
    const LayerState& ls = p->layers[layer];
    if (n_kv < 0 || (n_kv + kvs::kPageTokens - 1) / kvs::kPageTokens != ls.n_pages)
        return fail(KVS_ERR_INVALID_ARG, "n_kv %lld does not fill the layer's %d pages", (long long)n_kv, ls.n_pages);
    if (ls.n_pages > 0 && !dst) return fail(KVS_ERR_INVALID_ARG, "dst is NULL");
    if ((uintptr_t)dst & 255) return fail(KVS_ERR_INVALID_ARG, "dst must be 256-byte aligned");
    if ((rc = check_ring_free_for(p, layer))) return rc;
    hipStream_t s = (hipStream_t)stream;
    if ((rc = check_capture(p, layer, s))) return rc;
    if ((rc = order_after_last_work(p, s))) return rc;
    kvs::StageArgs a{};
    a.ps.slots = p->slots;
    a.ps.src = ls.dev_src;
    a.ps.host = (p->cfg.flags & KVS_FLAG_ZERO_COPY) ? ls.host : nullptr;
    a.ps.page_bytes = (int64_t)p->L.page_bytes;
    a.n_kv_heads = p->cfg.n_kv_heads;
    a.n_kv = n_kv;
    a.staged = (uint8_t*)dst;
    a.v_q8 = p->cfg.type_v == KVS_TYPE_Q8_0;
    a.by_page = 1;
    rc = run_layer(p, layer, s, [&](hipStream_t st, int /*lane*/, int32_t seg0, int32_t nseg, const uint8_t* ring_chunk,
                                    int32_t rank0, const kvs::CopyJob& cj) -> int {
        kvs::StageArgs b = a;
        b.copy = cj;
        b.ps.ring_chunk = ring_chunk;
        b.ps.chunk_rank0 = rank0;
        b.segs = ls.dev_segs + seg0;
        b.n_segs = nseg;
        b.n_pages = 0;
        for (int32_t i = seg0; i < seg0 + nseg; ++i) b.n_pages += ls.segs[i].npages;
        hipError_t e = kvs::launch_stage(b, st);
        return e == hipSuccess ? KVS_OK : fail(KVS_ERR_HIP, "staging kernel launch failed: %s", hipGetErrorString(e));
    });
    if (rc) return rc;
    return record_last_work(p, s);
}

int kvs_debug_export_pages(kvs_pool* p, int32_t layer, void* dst, void* stream) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    if ((rc = check_layer_ready(p, layer))) return rc;
    const LayerState& ls = p->layers[layer];
    if (ls.n_pages > 0 && !dst) return fail(KVS_ERR_INVALID_ARG, "dst is NULL");
    if ((uintptr_t)dst & 15) return fail(KVS_ERR_INVALID_ARG, "dst must be 16-byte aligned");
    if ((rc = check_ring_free_for(p, layer))) return rc;
    hipStream_t s = (hipStream_t)stream;
    if ((rc = check_capture(p, layer, s))) return rc;
    if ((rc = order_after_last_work(p, s))) return rc;
    kvs::ExportArgs a{};
    a.ps.slots = p->slots;
    a.ps.src = ls.dev_src;
    a.ps.host = (p->cfg.flags & KVS_FLAG_ZERO_COPY) ? ls.host : nullptr;
    a.ps.page_bytes = (int64_t)p->L.page_bytes;
    a.dst = (uint8_t*)dst;
    rc = run_layer(p, layer, s, [&](hipStream_t st, int /*lane*/, int32_t seg0, int32_t nseg, const uint8_t* ring_chunk,
                                    int32_t rank0, const kvs::CopyJob& cj) -> int {
        kvs::ExportArgs b = a;
        b.copy = cj;
        b.ps.ring_chunk = ring_chunk;
        b.ps.chunk_rank0 = rank0;
        b.segs = ls.dev_segs + seg0;
        b.n_segs = nseg;
        hipError_t e = kvs::launch_export(b, st);
        return e == hipSuccess ? KVS_OK : fail(KVS_ERR_HIP, "export kernel launch failed: %s", hipGetErrorString(e));
    });
    if (rc) return rc;
    return record_last_work(p, s);
}

int kvs_append(kvs_pool* p, int32_t layer, const void* k_new, const void* v_new, int32_t dtype, int64_t pos0,
               int32_t n_tok, void* stream) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    if ((rc = check_layer_ready(p, layer))) return rc;
    const LayerState& ls = p->layers[layer];
    if (dtype != KVS_Q_F32 && dtype != KVS_Q_F16) return fail(KVS_ERR_INVALID_ARG, "dtype %d unknown", dtype);
    if (n_tok < 0 || pos0 < 0 || pos0 + n_tok > (int64_t)ls.n_pages * kvs::kPageTokens)
        return fail(KVS_ERR_INVALID_ARG, "tokens [%lld, %lld) outside the layer's %d pages", (long long)pos0,
                    (long long)(pos0 + n_tok), ls.n_pages);
    if (n_tok == 0) return KVS_OK;
    if (!k_new || !v_new) return fail(KVS_ERR_INVALID_ARG, "k_new or v_new is NULL");
    if ((((uintptr_t)k_new) | ((uintptr_t)v_new)) & 15) return fail(KVS_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
    if (p->pf_layer == layer) {
        for (int64_t pg = pos0 / kvs::kPageTokens; pg <= (pos0 + n_tok - 1) / kvs::kPageTokens; ++pg)
            if (ls.src[pg] < 0)
                return fail(KVS_ERR_STATE, "layer %d has a pending prefetch that may read streamed page %lld; append before kvs_stream_enqueue",
                            layer, (long long)pg);
    }
    hipStream_t s = (hipStream_t)stream;
    if ((rc = order_after_last_work(p, s))) return rc;   // no reader of the rows is still in flight
    kvs::AppendArgs a{};
    a.k = k_new;
    a.v = v_new;
    a.f16 = dtype == KVS_Q_F16 ? 1 : 0;
    a.pos0 = pos0;
    a.n_tok = n_tok;
    a.n_kv_heads = p->cfg.n_kv_heads;
    a.page_bytes = (int64_t)p->L.page_bytes;
    a.src = ls.dev_src;
    a.slots = p->slots;
    a.host = const_cast<uint8_t*>(ls.host);
    a.v_q8 = p->cfg.type_v == KVS_TYPE_Q8_0;
    hipError_t e = kvs::launch_append(a, s);
    if (e != hipSuccess) return fail(KVS_ERR_HIP, "append kernel launch failed: %s", hipGetErrorString(e));
    p->st.kernels_launched++;
    if (hipEventRecord(p->append_ev, s) != hipSuccess) { p->broken = true; return fail(KVS_ERR_HIP, "hipEventRecord failed"); }
    p->appended = true;
    return KVS_OK;
}

int kvs_debug_read_page(kvs_pool* p, int32_t layer, int32_t page, void* dst_host) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_device(p);
    if (rc) return rc;
    if ((rc = check_layer_ready(p, layer))) return rc;
    const LayerState& ls = p->layers[layer];
    if (page < 0 || page >= ls.n_pages) return fail(KVS_ERR_INVALID_ARG, "page %d out of range [0, %d)", page, ls.n_pages);
    if (!dst_host) return fail(KVS_ERR_INVALID_ARG, "dst_host is NULL");
    if (ls.src[page] < 0) return fail(KVS_ERR_NOT_RESIDENT, "page %d of layer %d is streamed, not resident", page, layer);
    if (p->worked) KVS_HIP(hipEventSynchronize(p->last_work));
    KVS_HIP(hipMemcpy(dst_host, p->slots + (uint64_t)ls.src[page] * p->L.page_bytes, p->L.page_bytes, hipMemcpyDeviceToHost));
    return KVS_OK;
}

int kvs_profile_enable(kvs_pool* p, int32_t enable) {
    if (!p) return fail(KVS_ERR_INVALID_ARG, "pool is NULL");
    p->profiling = enable != 0;
    return KVS_OK;
}

int kvs_profile_read(kvs_pool* p, int32_t kind, int64_t* launches, double* total_ms, int32_t reset) {
    if (!p || !launches || !total_ms) return fail(KVS_ERR_INVALID_ARG, "NULL argument");
    if (kind < 0 || kind > 1) return fail(KVS_ERR_INVALID_ARG, "kind %d unknown", kind);
    double ms = 0.0;
    for (size_t i = 0; i < p->prof_used[kind]; ++i) {
        auto& pr = p->prof_ev[kind][i];
        KVS_HIP(hipEventSynchronize(pr.second));
        float t = 0.f;
        KVS_HIP(hipEventElapsedTime(&t, pr.first, pr.second));
        ms += t;
    }
    *launches = (int64_t)p->prof_used[kind];
    *total_ms = ms;
    if (reset) p->prof_used[kind] = 0;
    return KVS_OK;
}

const char* kvs_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
