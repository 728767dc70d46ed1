// Kernels for streamed paged attention over Q8_0 K / Q4_0 V pages (gfx950).
//
// A page is 256 tokens of one layer (page 2, "Dynamic draft eject"); the
// device sees each page either in a resident slot or in the transfer ring
// (page 1, "Summary"), and the kernels read both through the same PageSource.
//
// Work split (split-K over pages, merged with log-sum-exp weights):
//   * one workgroup = one segment (consecutive pages of one logical group) x
//     one kv head x one tile of query rows (row = query token x head in the
//     GQA group);
//   * each page yields a self-contained partial (max, sum, weighted V) that is
//     merged into the group's running state in page order, so the result does
//     not depend on which pages are resident or how the ring chunks them;
//   * the combine kernel merges the groups in ascending order.
// Scores are kept in log2 units (scale * log2 e folded into one multiplier) so
// the softmax uses exp2.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cmath>
#include <cstdlib>

#include "kvs_internal.h"

namespace kvs {
namespace {

__device__ inline float f16_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits & 0xFFFFu));
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// ---------------------------------------------------------------------------
// Attention over a page range, generic in the number of query rows.
// 256 threads; each page's K and V tiles for the workgroup's kv head are staged
// in LDS, then: scores (thread = token), softmax statistics (wave = row), and
// P.V (thread = channel x 4 rows).
// ---------------------------------------------------------------------------
constexpr int kRT = 8;          // query rows per workgroup
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void attend_rows_kernel(AttendArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t k_s[kKTile];
    __shared__ __attribute__((aligned(16))) uint8_t v_s[kVTile];
    __shared__ float q_s[kRT][kHeadDim];
    __shared__ float p_s[kRT][kPageTokens];
    __shared__ float m_s[kRT], l_s[kRT];

    if ((int)blockIdx.x >= a.n_segs) {   // ring refill workgroup
        if (blockIdx.z == 0) copy_role(a.copy, ((int)blockIdx.x - a.n_segs) * (int)gridDim.y + (int)blockIdx.y);
        return;
    }
    const int tid = threadIdx.x;
    const Seg seg = a.segs[blockIdx.x];
    const int g = blockIdx.y;
    const int R = a.n_q * a.G;
    const int r0 = blockIdx.z * kRT;
    const int nr = min(kRT, R - r0);

    // query rows -> LDS (float)
    for (int e = tid; e < kRT * kHeadDim; e += kThreads) {
        int r = e / kHeadDim, c = e % kHeadDim;
        float v = 0.f;
        if (r < nr) {
            int rr = r0 + r, i = rr / a.G, h = g * a.G + rr % a.G;
            int64_t off = ((int64_t)i * a.n_q_heads + h) * kHeadDim + c;
            v = a.q_f16 ? (float)((const _Float16*)a.q)[off] : ((const float*)a.q)[off];
        }
        q_s[r][c] = v;
    }

    // this thread owns channel c of rows rsub, rsub+2, rsub+4, rsub+6
    const int c = tid & (kHeadDim - 1);
    const int rsub = tid >> 7;
    float acc[4], m_run[4], l_run[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) { acc[k] = 0.f; m_run[k] = -INFINITY; l_run[k] = 0.f; }
    if (!(seg.flags & kSegFresh)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int r = rsub + 2 * k;
            if (r < nr) {
                int rr = r0 + r, i = rr / a.G, h = g * a.G + rr % a.G;
                const float* pr = a.part + (((int64_t)seg.group * a.n_q + i) * a.n_q_heads + h) * kPartStride;
                acc[k] = pr[c];
                m_run[k] = pr[kHeadDim];
                l_run[k] = pr[kHeadDim + 1];
            }
        }
    }

    for (int pi = 0; pi < seg.npages; ++pi) {
        const int page = seg.page0 + pi;
        const uint8_t* rec = page_ptr(a.ps, page);
        const uint4* ksrc = (const uint4*)(rec + (int64_t)g * kKTile);
        const uint4* vsrc = (const uint4*)(rec + (int64_t)a.n_kv_heads * kKTile + (int64_t)g * kVTile);
        for (int e = tid; e < kKTile / 16; e += kThreads) ((uint4*)k_s)[e] = ksrc[e];
        for (int e = tid; e < kVTile / 16; e += kThreads) ((uint4*)v_s)[e] = vsrc[e];
        int64_t rem = a.n_kv - (int64_t)page * kPageTokens;
        const int valid = (int)(rem < 0 ? 0 : (rem > kPageTokens ? kPageTokens : rem));
        __syncthreads();

        // scores: thread = token
        {
            const int t = tid;
            float s[kRT];
#pragma unroll
            for (int r = 0; r < kRT; ++r) s[r] = 0.f;
            if (t < valid) {
                const uint8_t* row = k_s + t * kKRow;
                for (int b = 0; b < kNB; ++b) {
                    const uint8_t* blk = row + b * kKBlock;
                    float d = f16_bits_to_float((uint32_t)blk[0] | ((uint32_t)blk[1] << 8));
                    float dot[kRT];
#pragma unroll
                    for (int r = 0; r < kRT; ++r) dot[r] = 0.f;
                    for (int i = 0; i < kQK; ++i) {
                        float kv = (float)(int8_t)blk[2 + i];
#pragma unroll
                        for (int r = 0; r < kRT; ++r) dot[r] = fmaf(q_s[r][b * kQK + i], kv, dot[r]);
                    }
#pragma unroll
                    for (int r = 0; r < kRT; ++r) s[r] = fmaf(d, dot[r], s[r]);
                }
            }
            const int64_t kpos = (int64_t)page * kPageTokens + t;
#pragma unroll
            for (int r = 0; r < kRT; ++r) {
                bool ok = t < valid && r < nr;
                if (ok && a.causal) ok = kpos <= a.q_pos0 + (r0 + r) / a.G;
                p_s[r][t] = ok ? s[r] * a.scale_log2 : -INFINITY;
            }
        }
        __syncthreads();

        // softmax statistics of this page: wave w handles rows w and w + 4
        {
            const int w = tid >> 6, lane = tid & 63;
            for (int r = w; r < kRT; r += 4) {
                float x0 = p_s[r][lane], x1 = p_s[r][lane + 64], x2 = p_s[r][lane + 128], x3 = p_s[r][lane + 192];
                float m = wave_max(fmaxf(fmaxf(x0, x1), fmaxf(x2, x3)));
                float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
                if (m != -INFINITY) {
                    e0 = exp2f(x0 - m); e1 = exp2f(x1 - m); e2 = exp2f(x2 - m); e3 = exp2f(x3 - m);
                }
                p_s[r][lane] = e0; p_s[r][lane + 64] = e1; p_s[r][lane + 128] = e2; p_s[r][lane + 192] = e3;
                float l = wave_sum((e0 + e1) + (e2 + e3));
                if (lane == 0) { m_s[r] = m; l_s[r] = l; }
            }
        }
        __syncthreads();

        // P.V: thread = channel c for 4 rows; tokens past `valid` are never read
        {
            const int b = c >> 5, j = c & 31;
            const int byte_off = b * kVBlock + 2 + (j & 15);
            const int shift = (j < 16) ? 0 : 4;
            float ap[4] = {0.f, 0.f, 0.f, 0.f};
            for (int t = 0; t < valid; ++t) {
                const uint8_t* vr = v_s + t * kVRow;
                float d = f16_bits_to_float((uint32_t)vr[b * kVBlock] | ((uint32_t)vr[b * kVBlock + 1] << 8));
                float v = d * (float)((int)((vr[byte_off] >> shift) & 15) - 8);
#pragma unroll
                for (int k = 0; k < 4; ++k) ap[k] = fmaf(p_s[rsub + 2 * k][t], v, ap[k]);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                int r = rsub + 2 * k;
                float mp = m_s[r], lp = l_s[r];
                float M = fmaxf(m_run[k], mp);
                if (M != -INFINITY) {
                    float al = (m_run[k] == -INFINITY) ? 0.f : exp2f(m_run[k] - M);
                    float be = (mp == -INFINITY) ? 0.f : exp2f(mp - M);
                    acc[k] = acc[k] * al + ap[k] * be;
                    l_run[k] = l_run[k] * al + lp * be;
                    m_run[k] = M;
                }
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int r = rsub + 2 * k;
        if (r < nr) {
            int rr = r0 + r, i = rr / a.G, h = g * a.G + rr % a.G;
            float* pr = a.part + (((int64_t)seg.group * a.n_q + i) * a.n_q_heads + h) * kPartStride;
            pr[c] = acc[k];
            if (c == 0) { pr[kHeadDim] = m_run[k]; pr[kHeadDim + 1] = l_run[k]; }
        }
    }
}

// ---------------------------------------------------------------------------
// Split-K combine: one workgroup per (query token x head, 16-channel slice);
// 256 threads = 16 channels x 16 group slices. Each thread walks groups
// sl, sl + 16, ... in batches of 8 independent loads with an online
// log-sum-exp merge; the 16 slices are then merged in a fixed order. The order
// depends only on the number of groups, never on scheduling or residency.
// ---------------------------------------------------------------------------
constexpr int kCombSlices = 16;
constexpr int kCombCh = 16;
constexpr int kCombBatch = 8;
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part, int32_t n_groups,
                                                      int32_t rows, float* __restrict__ out,
                                                      float* __restrict__ lse) {
    __shared__ float so[kCombSlices][kCombCh + 1];
    __shared__ float sm_[kCombSlices], sl_[kCombSlices];
    const int row = blockIdx.x / (kHeadDim / kCombCh), slice = blockIdx.x % (kHeadDim / kCombCh);
    const int cl = threadIdx.x & (kCombCh - 1), sl = threadIdx.x / kCombCh;
    const int c = slice * kCombCh + cl;
    const int64_t gstride = (int64_t)rows * kPartStride;
    const float* p = part + (int64_t)row * kPartStride;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int g0 = sl; g0 < n_groups; g0 += kCombSlices * kCombBatch) {
        float mg[kCombBatch], lg[kCombBatch], og[kCombBatch];
#pragma unroll
        for (int k = 0; k < kCombBatch; ++k) {
            const int gi = g0 + k * kCombSlices;
            const bool ok = gi < n_groups;
            const float* q = p + (int64_t)(ok ? gi : 0) * gstride;
            mg[k] = ok ? q[kHeadDim] : -INFINITY;
            lg[k] = q[kHeadDim + 1];
            og[k] = q[c];
        }
        float Mb = M;
#pragma unroll
        for (int k = 0; k < kCombBatch; ++k) Mb = fmaxf(Mb, mg[k]);
        if (Mb == -INFINITY) continue;
        const float sc = (M == -INFINITY) ? 0.f : exp2f(M - Mb);
        L *= sc;
        O *= sc;
#pragma unroll
        for (int k = 0; k < kCombBatch; ++k) {
            const float w = (mg[k] == -INFINITY) ? 0.f : exp2f(mg[k] - Mb);
            L = fmaf(lg[k], w, L);
            O = fmaf(og[k], w, O);
        }
        M = Mb;
    }
    so[sl][cl] = O;
    if (cl == 0) { sm_[sl] = M; sl_[sl] = L; }
    __syncthreads();
    if (sl == 0) {
        float Mt = sm_[0];
#pragma unroll
        for (int k = 1; k < kCombSlices; ++k) Mt = fmaxf(Mt, sm_[k]);
        float ot = 0.f, lt = 0.f;
        if (Mt != -INFINITY) {
#pragma unroll
            for (int k = 0; k < kCombSlices; ++k) {
                const float w = (sm_[k] == -INFINITY) ? 0.f : exp2f(sm_[k] - Mt);
                ot = fmaf(so[k][cl], w, ot);
                lt = fmaf(sl_[k], w, lt);
            }
        }
        out[(int64_t)row * kHeadDim + c] = (Mt == -INFINITY) ? 0.f : ot / lt;
        if (lse && slice == 0 && cl == 0)
            lse[row] = (Mt == -INFINITY) ? -INFINITY : (Mt + log2f(lt)) * 0.69314718055994530942f;
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

hipError_t launch_attend(const AttendArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    const int R = a.n_q * a.G;
    if (decode_supports(R)) return launch_decode(a, stream);
    const int cx = (copy_workgroups(a.copy) + a.n_kv_heads - 1) / a.n_kv_heads;
    dim3 grid(a.n_segs + cx, a.n_kv_heads, (R + kRT - 1) / kRT);
    hipLaunchKernelGGL(attend_rows_kernel, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_combine(const float* part, int32_t n_groups, int32_t n_q, int32_t n_q_heads,
                          float* out, float* lse, hipStream_t stream) {
    const int rows = n_q * n_q_heads;
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3(rows * (kHeadDim / kCombCh)), dim3(256), 0, stream, part, n_groups, rows, out, lse);
    return hipGetLastError();
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
