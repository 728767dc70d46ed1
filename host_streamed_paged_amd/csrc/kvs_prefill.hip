// Prefill attention kernel: query blocks of more than 64 rows per kv head (a
// prefill ubatch, 256 tokens in page 2's "TLDR - recommended setup") on the
// staged matrix-core operands stage_kernel writes (kvs_mfma.hip), on CDNA4
// v_mfma_f32_16x16x32_f16.
//
// One workgroup = one segment (run of pages of one split-K group) x one kv
// head x a block of 256 query rows (row = query token x head of the GQA
// group); 8 waves, each owning 32 rows (two 16-row tiles) from scores to
// output, so no wave ever waits on another's results. The workgroup walks
// its pages in 64-token sub-blocks: the sub-block's staged operands (K
// fragments 16 KB, V^T fragments 16 KB, float32 K scales 1 KB) are brought
// into LDS once by LDS DMA, two sub-blocks ahead of their use (three
// buffers), and every wave reads them there, so each staged byte leaves L2
// once per workgroup instead of once per 16-row tile. Per sub-block and wave:
//   QK   A_b^T (16 tokens x 16 rows) = K_b . Q_b^T per 16-token tile and quant
//        block, with K_b the exact f16 codes and Q_b the query's exact f16
//        limbs (all products of a tile are issued before any is scaled); each
//        block's product times its float32 scale, summed in float32. The row
//        factor cq > 0 (scale * log2(e) over the query's scaling) turns them
//        into log2-unit scores inside the exponent.
//   softmax  the sub-block's row maxima (lanes n, n + 16, n + 32, n + 48 hold
//        a row's tokens), the running max m moving only when a sub-block's
//        max exceeds it by more than 8, p = exp2(cq s - m). The score tile's
//        register layout is the P^T operand of P.V, so P never leaves the
//        wave's registers.
//   PV   O^T (16 channels x 16 rows) += V^T (16 x 32 tokens) . P^T (32 x 16)
//        for the 8 channel tiles and 2 chunks of the sub-block, plus a ninth
//        tile of ones whose product is the row sum of the same f16 p that
//        weight V; a block whose page takes V divided by 8 keeps its
//        accumulator in units of 8 (an exact rescale when that changes).
// The running state (m, l, O) is updated in a fixed order of pages and
// sub-blocks from state and page data alone, so results do not depend on how
// pages are split into launches or which pages are resident.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cmath>

#include "kvs_internal.h"
#include "kvs_device.h"

namespace kvs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef KVS_PF_WAVES
#define KVS_PF_WAVES 8
#endif
#ifndef KVS_PF_RTW
#define KVS_PF_RTW 2
#endif
constexpr int kPWaves = KVS_PF_WAVES;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kRTW = KVS_PF_RTW;             // 16-row tiles per wave
constexpr int kRowsWG = 16 * kRTW * kPWaves; // rows per workgroup (256)
constexpr int kSub = 64;                     // tokens per sub-block
constexpr int kSubs = kPageTokens / kSub;    // sub-blocks per page
constexpr int kSubK = 4 * kNB * 64 * 16;     // K fragments of a sub-block (16 KB)
constexpr int kSubV = 2 * 8 * 64 * 16;       // V^T fragments of a sub-block (two 32-token chunks, 16 KB)
constexpr int kSubS = kSub * kNB * 4;        // float32 K scales of a sub-block (1 KB)
constexpr int kSubBytes = kSubK + kSubV + kSubS;
constexpr int kSubPieces = kSubBytes / 1024; // 1 KB LDS DMA pieces (one wave instruction each)
static_assert(kSubBytes % 1024 == 0, "sub-block is whole 1 KB pieces");
constexpr float kLazyMax = 8.f;
#ifndef KVS_PF_OCC
#define KVS_PF_OCC 1
#endif

// Three sub-block buffers (the one in use and two in flight), each its own
// LDS array: the compiler then orders a read of one buffer only after the
// DMA into that buffer, not after the DMAs still in flight into the others.

// Issue this wave's share of the LDS DMA of sub-block sb of a staged tile:
// piece p (1 KB) of [K | V^T | scales] goes to dst + 1024 p.
__device__ inline void dma_sub(const uint8_t* tile, int sb, uint8_t* dst, int w, int lane) {
#pragma unroll
    for (int k = 0; k < (kSubPieces + kPWaves - 1) / kPWaves; ++k) {
        const int p = w + kPWaves * k;
        if (p >= kSubPieces) break;
        const uint8_t* src;
        if (p < kSubK / 1024) src = tile + sb * kSubK + p * 1024;
        else if (p < (kSubK + kSubV) / 1024) src = tile + kStagedK + sb * kSubV + (p - kSubK / 1024) * 1024;
        else src = tile + kStagedOps + sb * kSubS + (p - (kSubK + kSubV) / 1024) * 1024;
        dma16(src + 16 * lane, dst + 1024 * p);
    }
}

template <int LIMBS>
__global__ __launch_bounds__(kPThreads, KVS_PF_OCC) void prefill_kernel(AttendArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t buf0[kSubBytes];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[kSubBytes];
    __shared__ __attribute__((aligned(16))) uint8_t buf2[kSubBytes];
    // 1-D grid: ring refill workgroups first, then one worker per (segment,
    // kv head, row block), row blocks of one (segment, kv head) consecutive.
    // Workgroups go to the 8 XCDs round-robin by linear index; workers are
    // permuted so that each XCD takes a contiguous range, and the row blocks
    // of one (segment, kv head), which read the same staged tiles, share an
    // XCD's L2.
    const int G = a.G, R = a.n_q * G;
    const int n_rb = (R + kRowsWG - 1) / kRowsWG;
    const int n_copy8 = (copy_workgroups(a.copy) + 7) & ~7;
    const int L = (int)blockIdx.x;
    if (L < n_copy8) {   // ring refill workgroup: its first 256 threads copy
        if (threadIdx.x < 256) copy_role(a.copy, L);
        return;
    }
    const int n_work = a.n_segs * a.n_kv_heads * n_rb;
    const int per_xcd = ((n_work + 7) & ~7) / 8;
    const int work = ((L - n_copy8) & 7) * per_xcd + ((L - n_copy8) >> 3);
    if (work >= n_work) return;
    const int seg_i = work / (n_rb * a.n_kv_heads);
    const int g = (work / n_rb) % a.n_kv_heads;
    const int rb = work % n_rb;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;
    const int r0 = rb * kRowsWG + 16 * kRTW * w;   // this wave's first row

    typedef int int4v __attribute__((ext_vector_type(4)));
    const int4v segv = scalar_load((const int4v*)(a.segs + seg_i));
    const Seg seg = {segv.x, segv.y, segv.z, segv.w};
    // staged tiles of the segment's first page for kv head g: pages of the
    // launch's segments are staged in order
    int first = 0;
    for (int i = 0; i < seg_i; ++i) first += scalar_load(&a.segs[i].npages);
    const int64_t tile_step = (int64_t)a.n_kv_heads * kStagedTile;
    const uint8_t* tile0 = a.staged + ((int64_t)first * a.n_kv_heads + g) * kStagedTile;
    const int n_steps = seg.npages * kSubs;
    dma_sub(tile0, 0, buf0, w, lane);
    if (n_steps > 1) dma_sub(tile0, 1, buf1, w, lane);

    // ---- this lane's query rows and their visible prefix
    half8_t qop[kRTW][LIMBS][kNB];
    float cq[kRTW];
    int64_t lim[kRTW];
    int qi_[kRTW], h_[kRTW];
#pragma unroll
    for (int rt = 0; rt < kRTW; ++rt) {
        const int r = r0 + 16 * rt + n;
        qi_[rt] = r / G;
        h_[rt] = g * G + r % G;
        lim[rt] = 0;
        if (r < R) {
            lim[rt] = a.n_kv;
            if (a.causal) {
                const int64_t c = a.q_pos0 + qi_[rt] + 1;
                lim[rt] = c < lim[rt] ? c : lim[rt];
            }
        }
        query_operands<LIMBS>(a, qi_[rt], h_[rt], r < R, gq, qop[rt], cq[rt]);
    }
    // smallest visible prefix of the wave's rows: sub-blocks below it need no mask
    int64_t lim_min = a.n_kv;
    if (a.causal) {
        const int64_t c = a.q_pos0 + r0 / G + 1;
        lim_min = c < lim_min ? c : lim_min;
    }

    // ---- running state: O^T tiles [ct][rt] hold channels 16 ct + 4 gq + i of
    // row 16 rt + n, block b's in units of 2^vsh_run[b]; lsum[rt] holds the
    // row sum (every value of it); m is replicated over the lanes of a row
    f32x4 o[8][kRTW], lsum[kRTW];
    float m_run[kRTW];
    int vsh_run[kNB] = {0, 0, 0, 0};
#pragma unroll
    for (int rt = 0; rt < kRTW; ++rt) {
        m_run[rt] = -INFINITY;
        lsum[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) o[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!(seg.flags & kSegFresh) && r0 + 16 * rt + n < R) {
            const float* pr = a.part + (((int64_t)seg.group * a.n_q + qi_[rt]) * a.n_q_heads + h_[rt]) * kPartStride;
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const float2* src = (const float2*)(pr + 16 * ct + 4 * gq);   // records are 8-byte aligned
                const float2 u = src[0], v = src[1];
                o[ct][rt] = f32x4{u.x, u.y, v.x, v.y};
            }
            m_run[rt] = pr[kHeadDim];
            const float l = pr[kHeadDim + 1];
            lsum[rt] = f32x4{l, l, l, l};
        }
    }
    half8_t ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (_Float16)1.f;

    // one step: compute sub-block `step` from B, the DMA of step + 2 goes to D
    auto do_step = [&](int step, const uint8_t* B, uint8_t* D) {
        const int pi = step / kSubs, sb = step % kSubs;
        const int page = seg.page0 + pi;
        const uint8_t* tile = tile0 + pi * tile_step;
        // this sub-block is in LDS for every wave (a wave has at most one later
        // sub-block's DMA in flight: 4 or 5 instructions), and every wave is
        // done with the buffer two sub-blocks ahead goes into
        // (the builtin, unlike inline asm, is known to the compiler's wait
        // tracking: it then needs no wait of its own before the reads)
        if (step + 1 < n_steps) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)
        lds_barrier();
        if (step + 2 < n_steps) {
            const int pn = (step + 2) / kSubs, sn = (step + 2) % kSubs;
            dma_sub(tile0 + pn * tile_step, sn, D, w, lane);
        }
        const int64_t base_tok = (int64_t)page * kPageTokens + kSub * sb;
        const bool mask_sub = base_tok + kSub > lim_min;   // wave-uniform

        // ---- QK (float32 products; cq * s is the log2-unit score)
        f32x4 s[4][kRTW];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4 acc[kRTW][kNB];
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                const half8_t kop = *(const half8_t*)(B + ((tt * kNB + b) * 64 + lane) * 16);
#pragma unroll
                for (int rt = 0; rt < kRTW; ++rt) {
                    acc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[rt][0][b], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if constexpr (LIMBS == 2)
                        acc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[rt][1][b], acc[rt][b], 0, 0, 0);
                }
            }
            // scales of the lane's four tokens 16 tt + 4 gq + i: [i][b] float32
            const f32x4* sc = (const f32x4*)(B + kSubK + kSubV + (16 * tt + 4 * gq) * kNB * 4);
            f32x4 d[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] = sc[i];
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma clang fp contract(off)
                    float t = acc[rt][0][i] * d[i][0];
                    t = __builtin_fmaf(acc[rt][1][i], d[i][1], t);
                    t = __builtin_fmaf(acc[rt][2][i], d[i][2], t);
                    s[tt][rt][i] = __builtin_fmaf(acc[rt][3][i], d[i][3], t);
                }
        }
        if (mask_sub) {
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt) {
                const int64_t x = lim[rt] - base_tok;
                const int lr = (int)(x < 0 ? 0 : (x > kSub ? kSub : x));
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[tt][rt][i] = 16 * tt + 4 * gq + i < lr ? s[tt][rt][i] : -INFINITY;
            }
        }

        // ---- softmax over the sub-block
        float alpha[kRTW], m_use[kRTW];
        bool rescale = false;
#pragma unroll
        for (int rt = 0; rt < kRTW; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tt][rt][i]);
            mx = max_xor16(mx);
            mx = max_xor32(mx) * cq[rt];
            // mx > -inf + 8 holds for any finite mx: the first visible sub-block sets m
            const bool grow = mx > m_run[rt] + kLazyMax;
            alpha[rt] = grow ? __builtin_amdgcn_exp2f(m_run[rt] - mx) : 1.f;   // 0 while the state is empty
            m_run[rt] = grow ? mx : m_run[rt];
            m_use[rt] = m_run[rt] == -INFINITY ? 0.f : m_run[rt];
            rescale |= grow;
        }
        // P^T operands: chunk c's slot j of lane group gq is token 32 c + 4 gq + j
        // (j < 4, tile 2 c) or 32 c + 12 + 4 gq + j (j >= 4, tile 2 c + 1)
        half8_t pop[2][kRTW];
#pragma unroll
        for (int rt = 0; rt < kRTW; ++rt)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pop[c][rt][j] = (_Float16)__builtin_amdgcn_exp2f(
                        __builtin_fmaf(s[2 * c + (j >> 2)][rt][j & 3], cq[rt], -m_use[rt]));
        if (__any(rescale)) {
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt) {
                lsum[rt] *= alpha[rt];
#pragma unroll
                for (int ct = 0; ct < 8; ++ct) o[ct][rt] *= alpha[rt];
            }
        }
        // ---- the page's V shifts (read at its first sub-block); an exact
        // rescale of a block's accumulators when its shift changes
        if (sb == 0) {
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                const int vsh = scalar_load((const int32_t*)(tile + kStagedShift) + b);
                if (vsh != vsh_run[b]) {
                    const float f = __builtin_amdgcn_ldexpf(1.f, vsh_run[b] - vsh);
#pragma unroll
                    for (int rt = 0; rt < kRTW; ++rt) {
                        o[2 * b][rt] *= f;
                        o[2 * b + 1][rt] *= f;
                    }
                    vsh_run[b] = vsh;
                }
            }
        }

        // ---- P.V, and the row sums on a tile of ones
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const half8_t vop = *(const half8_t*)(B + kSubK + ((c * 8 + ct) * 64 + lane) * 16);
#pragma unroll
                for (int rt = 0; rt < kRTW; ++rt)
                    o[ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[c][rt], o[ct][rt], 0, 0, 0);
            }
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt)
                lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pop[c][rt], lsum[rt], 0, 0, 0);
        }
    };
    // steps three at a time, so that each names its buffers statically
    for (int step = 0; step < n_steps; step += 3) {
        do_step(step, buf0, buf2);
        if (step + 1 < n_steps) do_step(step + 1, buf1, buf0);
        if (step + 2 < n_steps) do_step(step + 2, buf2, buf1);
    }

    // ---- group state -> partial records (O back in absolute units)
#pragma unroll
    for (int rt = 0; rt < kRTW; ++rt) {
        if (r0 + 16 * rt + n >= R) continue;
        float* pr = a.part + (((int64_t)seg.group * a.n_q + qi_[rt]) * a.n_q_heads + h_[rt]) * kPartStride;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const f32x4 ov = o[ct][rt] * __builtin_amdgcn_ldexpf(1.f, vsh_run[ct >> 1]);
            float2* dst = (float2*)(pr + 16 * ct + 4 * gq);   // records are 8-byte aligned
            dst[0] = make_float2(ov[0], ov[1]);
            dst[1] = make_float2(ov[2], ov[3]);
        }
        if (gq == 0) {
            pr[kHeadDim] = m_run[rt];
            pr[kHeadDim + 1] = lsum[rt][0];
        }
    }
}

template <int LIMBS>
hipError_t launch_limbs(const AttendArgs& a, hipStream_t stream) {
    const int R = a.n_q * a.G;
    const int64_t n_work = (int64_t)a.n_segs * a.n_kv_heads * ((R + kRowsWG - 1) / kRowsWG);
    const int64_t blocks = ((copy_workgroups(a.copy) + 7) & ~7) + ((n_work + 7) & ~7);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    return launch_kernel(prefill_kernel<LIMBS>, dim3((unsigned)blocks), dim3(kPThreads), stream, a);
}

}  // namespace

hipError_t launch_prefill(const AttendArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    return a.q_f16 ? launch_limbs<1>(a, stream) : launch_limbs<2>(a, stream);
}

}  // namespace kvs
