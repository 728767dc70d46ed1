// Kernels for streamed paged attention over Q8_0 K / Q4_0 V pages (gfx950):
// the split-K combine, the dequantizing gather probe, ring copies, and the
// dispatch of the attention kernels (kvs_decode.hip for up to 6 query rows per
// kv head, kvs_mfma.hip above).
//
// A page is 256 tokens of one layer (page 2, "Dynamic draft eject"); the
// device sees each page either in a resident slot or in the transfer ring
// (page 1, "Summary"), and the kernels read both through the same PageSource.
//
// Work split (split-K over pages, merged with log-sum-exp weights):
//   * one attention workgroup = one segment (consecutive pages of one logical
//     group) x one kv head x one tile of query rows (row = query token x head
//     in the GQA group);
//   * pages are folded into the group's running state in page order, so the
//     result does not depend on which pages are resident or how the ring
//     chunks them;
//   * the combine kernel merges the groups in ascending order.
// Scores are kept in log2 units (scale * log2 e folded into one multiplier) so
// the softmax uses exp2.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cmath>
#include <cstdlib>
#include <mutex>

#include "kvs_internal.h"
#include "kvs_device.h"

namespace kvs {
namespace {


// ---------------------------------------------------------------------------
// Split-K combine: one workgroup per (output row, CH-channel slice), so that
// a row's records are read by several compute units at once. Thread (gl, c) =
// (tid / CH, tid % CH) folds groups gl, gl + L, gl + 2 L, ... (L = THREADS /
// CH group lanes) of channel CH s + c into a running log-sum-exp state, BATCH
// groups per step so that BATCH record loads are in flight; the L group
// lanes of a channel are then merged in lane order. The order depends only
// on the number of groups, never on scheduling or residency.
// ---------------------------------------------------------------------------
template <int CH, int BATCH, int THREADS>
__global__ __launch_bounds__(THREADS) void combine_kernel(const float* __restrict__ part, int32_t n_groups,
                                                          int32_t rows, float* __restrict__ out,
                                                          float* __restrict__ lse) {
    constexpr int kLanes = THREADS / CH;   // group lanes per channel
    __shared__ float so[kLanes][CH];
    __shared__ float sm_[kLanes], sl_[kLanes];
    const int row = blockIdx.x, sl = blockIdx.y;
    const int gl = threadIdx.x / CH, c = threadIdx.x % CH;
    const int64_t gstride = (int64_t)rows * kPartStride;
    const float* p = part + (int64_t)row * kPartStride;
    const int ch = CH * sl + c;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int g0 = gl; g0 < n_groups; g0 += kLanes * BATCH) {
        float mg[BATCH], lg[BATCH], og[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int gi = g0 + k * kLanes;
            const bool ok = gi < n_groups;
            const float* q = p + (int64_t)(ok ? gi : 0) * gstride;
            const float2 ml = *(const float2*)(q + kHeadDim);
            mg[k] = ok ? ml.x : -INFINITY;
            lg[k] = ml.y;
            og[k] = q[ch];
        }
        float Mb = M;
#pragma unroll
        for (int k = 0; k < BATCH; ++k) Mb = fmaxf(Mb, mg[k]);
        if (Mb == -INFINITY) continue;
        const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
        L *= sc;
        O *= sc;
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const float w = (mg[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mg[k] - Mb);
            L = fmaf(lg[k], w, L);
            O = fmaf(og[k], w, O);
        }
        M = Mb;
    }
    so[gl][c] = O;
    if (c == 0) { sm_[gl] = M; sl_[gl] = L; }
    __syncthreads();
    if (gl == 0) {
        float Mt = sm_[0];
#pragma unroll
        for (int k = 1; k < kLanes; ++k) Mt = fmaxf(Mt, sm_[k]);
        float ot = 0.f, lt = 0.f;
        if (Mt != -INFINITY) {
#pragma unroll
            for (int k = 0; k < kLanes; ++k) {
                const float w = (sm_[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sm_[k] - Mt);
                ot = fmaf(so[k][c], w, ot);
                lt = fmaf(sl_[k], w, lt);
            }
        }
        const bool empty = Mt == -INFINITY;
        out[(int64_t)row * kHeadDim + ch] = empty ? 0.f : ot / lt;
        if (lse && sl == 0 && c == 0) lse[row] = empty ? -INFINITY : (Mt + log2f(lt)) * 0.69314718055994530942f;
    }
}
// Launches with many rows and many groups (a verify block over a long cache
// in single-page groups) take 32-channel slices with 512 threads: fewer
// workgroups read each record (such a launch is bound by the number of
// record reads), 16 group lanes per channel as before. With few rows the
// 16-channel slices keep more workgroups in flight.
constexpr int kCombWideGroups = 256;   // groups and rows from which a launch takes the wide shape
constexpr int kCombWideRows = 64;

// ---------------------------------------------------------------------------
// Split-K combine for blocks with many rows (a prefill ubatch): one wave per
// output row. Lane l holds channels 2 l and 2 l + 1 and folds the groups in
// ascending order, 8 records per step so that 8 coalesced 512-byte record
// loads are in flight; the row's m and l are uniform loads. The order depends
// only on the number of groups.
// ---------------------------------------------------------------------------
constexpr int kCombRowsMin = 512;   // rows from which a launch takes this kernel
constexpr int kCombBatch = 8;
__global__ __launch_bounds__(256) void combine_rows_kernel(const float* __restrict__ part, int32_t n_groups,
                                                           int32_t rows, float* __restrict__ out,
                                                           float* __restrict__ lse) {
    const int row = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + ((int)threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int64_t gstride = (int64_t)rows * kPartStride;
    const float* p = part + (int64_t)row * kPartStride;
    float M = -INFINITY, L = 0.f, O0 = 0.f, O1 = 0.f;
    for (int g0 = 0; g0 < n_groups; g0 += kCombBatch) {
        float2 ml[kCombBatch], og[kCombBatch];
#pragma unroll
        for (int k = 0; k < kCombBatch; ++k) {
            const int gi = g0 + k;
            const bool ok = gi < n_groups;   // uniform
            const float* q = p + (int64_t)(ok ? gi : 0) * gstride;
            ml[k] = *(const float2*)(q + kHeadDim);
            og[k] = *(const float2*)(q + 2 * lane);
            if (!ok) ml[k].x = -INFINITY;
        }
        float Mb = M;
#pragma unroll
        for (int k = 0; k < kCombBatch; ++k) Mb = fmaxf(Mb, ml[k].x);
        if (Mb == -INFINITY) continue;
        const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
        L *= sc;
        O0 *= sc;
        O1 *= sc;
#pragma unroll
        for (int k = 0; k < kCombBatch; ++k) {
            const float wk = (ml[k].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml[k].x - Mb);
            L = fmaf(ml[k].y, wk, L);
            O0 = fmaf(og[k].x, wk, O0);
            O1 = fmaf(og[k].y, wk, O1);
        }
        M = Mb;
    }
    const bool empty = M == -INFINITY;
    *(float2*)(out + (int64_t)row * kHeadDim + 2 * lane) = empty ? make_float2(0.f, 0.f) : make_float2(O0 / L, O1 / L);
    if (lse && lane == 0) lse[row] = empty ? -INFINITY : (M + log2f(L)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------------------
// Gather probe: dequantize tokens of the launch's pages into float32 through
// the block decoding the attention kernels use (kvs_device.h): each Q8_0 code
// and Q4_0 nibble becomes an exact f16 value, multiplied by the float32 block
// scale (exact: an 8-bit by 11-bit product). One workgroup per (segment, kv
// head); thread = token row of the page.
// ---------------------------------------------------------------------------
template <typename VT>
__global__ __launch_bounds__(kPageTokens) void gather_kernel(GatherArgs a) {
    if ((int)blockIdx.x >= a.n_segs) {   // ring refill workgroup
        copy_role(a.copy, ((int)blockIdx.x - a.n_segs) * (int)gridDim.y + (int)blockIdx.y);
        return;
    }
    const Seg seg = a.segs[blockIdx.x];
    const int g = blockIdx.y, t = threadIdx.x;
    const half2_t one = {(_Float16)1.f, (_Float16)1.f}, m1032 = {(_Float16)-1032.f, (_Float16)-1032.f};
    const half2_t m1152 = {(_Float16)-1152.f, (_Float16)-1152.f};
    for (int pi = 0; pi < seg.npages; ++pi) {
        const int page = seg.page0 + pi;
        const int64_t tok = (int64_t)page * kPageTokens + t;
        if (tok < a.tok0 || tok >= a.tok0 + a.n_tok) continue;
        const uint8_t* rec = page_ptr(a.ps, page);
        const uint8_t* kr = rec + (int64_t)g * kKTile + t * kKRow;
        const uint8_t* vr = rec + (int64_t)a.n_kv_heads * kKTile + (int64_t)g * VT::kTile + t * VT::kRow;
        float* ko = a.k_out + ((tok - a.tok0) * a.n_kv_heads + g) * kHeadDim;
        float* vo = a.v_out + ((tok - a.tok0) * a.n_kv_heads + g) * kHeadDim;
        for (int b = 0; b < kNB; ++b) {
            // blocks start on 2-byte boundaries: read 16-bit halves
            const uint16_t* kb = (const uint16_t*)(kr + b * kKBlock);
            const float dk = scale_f32(kb[0]);
            for (int j = 0; j < 4; ++j) {
                const uint32_t x0 = kb[1 + 4 * j] | ((uint32_t)kb[2 + 4 * j] << 16);
                const uint32_t x1 = kb[3 + 4 * j] | ((uint32_t)kb[4 + 4 * j] << 16);
                const half8_t c = q8_codes_f16(x0, x1);
                for (int e = 0; e < 8; ++e) ko[b * kQK + 8 * j + e] = (float)c[e] * dk;
            }
            const uint16_t* vb = (const uint16_t*)(vr + b * VT::kBlock);
            const float dv = scale_f32(vb[0]);
            if constexpr (VT::kQ8) {
                for (int j = 0; j < 16; ++j) {   // bytes 2 j, 2 j + 1: elements 2 j, 2 j + 1
                    const uint32_t w2 = vb[1 + j];
                    const half2_t c = q8_pair_f16((w2 & 0xFFu) | ((w2 >> 8) << 16), one, m1152);
                    vo[b * kQK + 2 * j] = (float)c[0] * dv;
                    vo[b * kQK + 2 * j + 1] = (float)c[1] * dv;
                }
                continue;
            }
            for (int j = 0; j < 8; ++j) {
                // bytes 2 j and 2 j + 1: elements 2 j, 2 j + 1 (low nibbles) and
                // 2 j + 16, 2 j + 17 (high nibbles)
                const uint32_t w2 = vb[1 + j];
                const uint32_t x = (w2 & 0xFFu) | ((w2 >> 8) << 16);
                const half2_t lo = q4_nibbles_f16((x & 0x000F000Fu) | 0x64006400u, one, m1032);
                const half2_t hi = q4_nibbles_f16(((x >> 4) & 0x000F000Fu) | 0x64006400u, one, m1032);
                vo[b * kQK + 2 * j] = (float)lo[0] * dv;
                vo[b * kQK + 2 * j + 1] = (float)lo[1] * dv;
                vo[b * kQK + 2 * j + 16] = (float)hi[0] * dv;
                vo[b * kQK + 2 * j + 17] = (float)hi[1] * dv;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Record export probe: the raw bytes of each page of the launch's segments,
// read from where the attention kernels read them (a resident slot, the ring
// chunk of this launch, or the pinned host record), copied to dst[page].
// One workgroup per (segment, 16 KB part of a page).
// ---------------------------------------------------------------------------
constexpr int kExportPart = 16384;
__global__ __launch_bounds__(256) void export_kernel(ExportArgs a) {
    if ((int)blockIdx.x >= a.n_segs) {   // ring refill workgroup
        copy_role(a.copy, ((int)blockIdx.x - a.n_segs) * (int)gridDim.y + (int)blockIdx.y);
        return;
    }
    const Seg seg = a.segs[blockIdx.x];
    const int64_t off = (int64_t)blockIdx.y * kExportPart;
    if (off >= a.ps.page_bytes) return;
    const int64_t n = a.ps.page_bytes - off < kExportPart ? a.ps.page_bytes - off : kExportPart;
    for (int pi = 0; pi < seg.npages; ++pi) {
        const int page = seg.page0 + pi;
        const uint4* src = (const uint4*)(page_ptr(a.ps, page) + off);
        uint4* dst = (uint4*)(a.dst + (int64_t)page * a.ps.page_bytes + off);
        for (int e = threadIdx.x; e < n / 16; e += 256) dst[e] = src[e];
    }
}

__global__ __launch_bounds__(256) void copy_kernel(CopyJob cj) { copy_role(cj, (int)blockIdx.x); }

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v, uint64_t n) {
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

}  // namespace

// Split-K partial records for kvs_attend_noalloc, for callers that cannot
// allocate: a fixed array in the library's own device memory (each GPU the
// library runs on holds one until the process ends). Host code never passes
// the array's name to a kernel: on the host it stands for the array, not for
// its device address, which scratch_region looks up once per device.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

hipError_t scratch_region(float** out) {
    static std::mutex mu;
    static float* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = (float*)p;
    }
    *out = addr[dev];
    return hipSuccess;
}

LaunchTiming& launch_timing() {
    static thread_local LaunchTiming t;
    return t;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    const int R = a.n_q * a.G;
    if (decode_supports(R)) return launch_decode(a, stream);
    return launch_mfma(a, stream);
}

hipError_t launch_combine(const float* part, int32_t n_groups, int32_t n_q, int32_t n_q_heads,
                          float* out, float* lse, hipStream_t stream) {
    const int rows = n_q * n_q_heads;
    if (rows <= 0) return hipSuccess;
    if (rows >= kCombRowsMin)
        return launch_kernel(combine_rows_kernel, dim3((rows + 3) / 4), dim3(256), stream, part, n_groups, rows, out, lse);
    if (n_groups >= kCombWideGroups && rows >= kCombWideRows) {
        return launch_kernel(combine_kernel<32, 8, 512>, dim3(rows, kHeadDim / 32), dim3(512), stream, part, n_groups,
                             rows, out, lse);
    }
    return launch_kernel(combine_kernel<16, 8, 256>, dim3(rows, kHeadDim / 16), dim3(256), stream, part, n_groups, rows,
                         out, lse);
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    const int cx = (copy_workgroups(a.copy) + a.n_kv_heads - 1) / a.n_kv_heads;
    if (a.v_q8) hipLaunchKernelGGL(gather_kernel<VQ8>, dim3(a.n_segs + cx, a.n_kv_heads), dim3(kPageTokens), 0, stream, a);
    else hipLaunchKernelGGL(gather_kernel<VQ4>, dim3(a.n_segs + cx, a.n_kv_heads), dim3(kPageTokens), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_export(const ExportArgs& a, hipStream_t stream) {
    const int parts = (int)((a.ps.page_bytes + kExportPart - 1) / kExportPart);
    const int cx = (copy_workgroups(a.copy) + parts - 1) / parts;
    if (a.n_segs <= 0 && cx == 0) return hipSuccess;
    hipLaunchKernelGGL(export_kernel, dim3(a.n_segs + cx, parts), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_copy(const CopyJob& cj, hipStream_t stream) {
    const int n = copy_workgroups(cj);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(copy_kernel, dim3(n), dim3(256), 0, stream, cj);
    return hipGetLastError();
}

hipError_t launch_fill_u32(void* dst, uint32_t value, uint64_t n_words, hipStream_t stream) {
    if (n_words == 0) return hipSuccess;
    uint64_t blocks = (n_words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t*)dst, value, n_words);
    return hipGetLastError();
}

}  // namespace kvs
