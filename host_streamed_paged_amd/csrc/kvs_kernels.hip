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

#include "kvs_internal.h"
#include "kvs_device.h"

namespace kvs {
namespace {

__device__ inline float f16_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits & 0xFFFFu));
}

// ---------------------------------------------------------------------------
// Split-K combine: one workgroup per output row (query token x head), 16
// waves. Wave s folds groups s, s + 16, s + 32, ... into a running
// log-sum-exp state, 8 groups per step so that 8 record loads are in flight;
// lane i owns channels 2i and 2i + 1 (one 8-byte load per record, so a wave
// reads a 512-byte record in one coalesced access). The 16 wave states are
// then merged in wave order. The order depends only on the number of groups,
// never on scheduling or residency.
// ---------------------------------------------------------------------------
constexpr int kCombWaves = 16;
constexpr int kCombBatch = 8;
__global__ __launch_bounds__(64 * kCombWaves) void combine_kernel(const float* __restrict__ part, int32_t n_groups,
                                                                  int32_t rows, float* __restrict__ out,
                                                                  float* __restrict__ lse) {
    __shared__ float2 so[kCombWaves][64];
    __shared__ float sm_[kCombWaves], sl_[kCombWaves];
    const int row = blockIdx.x;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t gstride = (int64_t)rows * kPartStride;
    const float* p = part + (int64_t)row * kPartStride;
    float M = -INFINITY, L = 0.f;
    float2 O = make_float2(0.f, 0.f);
    for (int g0 = wv; g0 < n_groups; g0 += kCombWaves * kCombBatch) {
        float mg[kCombBatch], lg[kCombBatch];
        float2 og[kCombBatch];
#pragma unroll
        for (int k = 0; k < kCombBatch; ++k) {
            const int gi = g0 + k * kCombWaves;
            const bool ok = gi < n_groups;
            const float* q = p + (int64_t)(ok ? gi : 0) * gstride;
            const float2 ml = *(const float2*)(q + kHeadDim);
            mg[k] = ok ? ml.x : -INFINITY;
            lg[k] = ml.y;
            og[k] = *(const float2*)(q + 2 * lane);
        }
        float Mb = M;
#pragma unroll
        for (int k = 0; k < kCombBatch; ++k) Mb = fmaxf(Mb, mg[k]);
        if (Mb == -INFINITY) continue;
        const float sc = (M == -INFINITY) ? 0.f : exp2f(M - Mb);
        L *= sc;
        O.x *= sc;
        O.y *= sc;
#pragma unroll
        for (int k = 0; k < kCombBatch; ++k) {
            const float w = (mg[k] == -INFINITY) ? 0.f : exp2f(mg[k] - Mb);
            L = fmaf(lg[k], w, L);
            O.x = fmaf(og[k].x, w, O.x);
            O.y = fmaf(og[k].y, w, O.y);
        }
        M = Mb;
    }
    so[wv][lane] = O;
    if (lane == 0) { sm_[wv] = M; sl_[wv] = L; }
    __syncthreads();
    if (wv == 0) {
        float Mt = sm_[0];
#pragma unroll
        for (int k = 1; k < kCombWaves; ++k) Mt = fmaxf(Mt, sm_[k]);
        float2 ot = make_float2(0.f, 0.f);
        float lt = 0.f;
        if (Mt != -INFINITY) {
#pragma unroll
            for (int k = 0; k < kCombWaves; ++k) {
                const float w = (sm_[k] == -INFINITY) ? 0.f : exp2f(sm_[k] - Mt);
                ot.x = fmaf(so[k][lane].x, w, ot.x);
                ot.y = fmaf(so[k][lane].y, w, ot.y);
                lt = fmaf(sl_[k], w, lt);
            }
        }
        const bool empty = Mt == -INFINITY;
        *(float2*)(out + (int64_t)row * kHeadDim + 2 * lane) = empty ? make_float2(0.f, 0.f)
                                                                      : make_float2(ot.x / lt, ot.y / lt);
        if (lse && lane == 0) lse[row] = empty ? -INFINITY : (Mt + log2f(lt)) * 0.69314718055994530942f;
    }
}

// ---------------------------------------------------------------------------
// Gather probe: dequantize tokens of the launch's pages into float32.
// One workgroup per (segment, kv head); thread = token row of the page.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPageTokens) void gather_kernel(GatherArgs a) {
    if ((int)blockIdx.x >= a.n_segs) {   // ring refill workgroup
        copy_role(a.copy, ((int)blockIdx.x - a.n_segs) * (int)gridDim.y + (int)blockIdx.y);
        return;
    }
    const Seg seg = a.segs[blockIdx.x];
    const int g = blockIdx.y, t = threadIdx.x;
    for (int pi = 0; pi < seg.npages; ++pi) {
        const int page = seg.page0 + pi;
        const int64_t tok = (int64_t)page * kPageTokens + t;
        if (tok < a.tok0 || tok >= a.tok0 + a.n_tok) continue;
        const uint8_t* rec = page_ptr(a.ps, page);
        const uint8_t* kr = rec + (int64_t)g * kKTile + t * kKRow;
        const uint8_t* vr = rec + (int64_t)a.n_kv_heads * kKTile + (int64_t)g * kVTile + t * kVRow;
        float* ko = a.k_out + ((tok - a.tok0) * a.n_kv_heads + g) * kHeadDim;
        float* vo = a.v_out + ((tok - a.tok0) * a.n_kv_heads + g) * kHeadDim;
        for (int b = 0; b < kNB; ++b) {
            const uint8_t* kb = kr + b * kKBlock;
            float dk = f16_bits_to_float((uint32_t)kb[0] | ((uint32_t)kb[1] << 8));
            for (int i = 0; i < kQK; ++i) ko[b * kQK + i] = dk * (float)(int8_t)kb[2 + i];
            const uint8_t* vb = vr + b * kVBlock;
            float dv = f16_bits_to_float((uint32_t)vb[0] | ((uint32_t)vb[1] << 8));
            for (int j = 0; j < 16; ++j) {
                uint32_t byte = vb[2 + j];
                vo[b * kQK + j] = dv * (float)((int)(byte & 15) - 8);
                vo[b * kQK + j + 16] = dv * (float)((int)(byte >> 4) - 8);
            }
        }
    }
}

__global__ __launch_bounds__(256) void copy_kernel(CopyJob cj) { copy_role(cj, (int)blockIdx.x); }

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v, uint64_t n) {
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

}  // namespace

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
    return launch_kernel(combine_kernel, dim3(rows), dim3(64 * kCombWaves), stream, part, n_groups, rows, out, lse);
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    const int cx = (copy_workgroups(a.copy) + a.n_kv_heads - 1) / a.n_kv_heads;
    hipLaunchKernelGGL(gather_kernel, dim3(a.n_segs + cx, a.n_kv_heads), dim3(kPageTokens), 0, stream, a);
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
