// Verify attention kernel: query blocks of 7 to 32 rows per kv head (a
// speculative verify batch of 1 + draft tokens times the heads of a GQA
// group; page 2, "Phase arena: speculative verify batches"), on CDNA4
// v_mfma_f32_16x16x32_f16.
//
// One workgroup of 8 waves = one kv head with all its rows (one or two
// 16-row tiles) x one slice of the launch's segments, walked in order, so
// each page's K and V are converted once for every row of the kv head. Two
// page buffers in LDS: the next page's K and V tiles (record layout) come in
// by LDS DMA while the current page is computed. Per page:
//   QK   wave w owns tokens [32 w, 32 w + 32) (two 16-token tiles) for every
//        row: A_b^T (16 tokens x 16 rows) = K_b . Q_b^T per tile, quant block
//        and row tile, with K_b the block's int8 codes as exact f16 and Q_b
//        the query's exact f16 limbs (one for f16 queries, two for f32). Each
//        block's product is multiplied by its float32 block scale and the
//        four are summed in float32, in block order.
//   softmax  page maxima per row across the 8 waves through LDS, the lazy
//        running max (it moves only when a page's max exceeds it by more
//        than 8 in log2 units), p = exp2(s - m). A wave's 32 tokens are
//        exactly one 32-token P.V chunk: the score registers are that
//        chunk's P^T operand, written to LDS once for the channel owners.
//   PV   wave w owns channels [16 w, 16 w + 16) (half of quant block w / 2):
//        O^T (16 channels x 16 rows) += V^T (16 x 32 tokens) . P^T (32 x 16)
//        over the 8 chunks, with V^T = d * (u - 8) (Q4_0) or d * code (Q8_0)
//        rounded once to f16, divided by 8 or 128 for a page whose block
//        could exceed the f16 range (the accumulator then kept in those
//        units).
// Barriers per page: one when the page's tiles have landed (which also
// frees the other buffer for the next page's DMA), one for the maxima, one
// for the P operands and row sums. The running state (m, l, O) is updated
// once per page in page order from state and page data alone, so results do
// not depend on how pages are split into launches or which are resident.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cmath>
#include <type_traits>

#include "kvs_internal.h"
#include "kvs_device.h"
#include "kvs_convert.h"

namespace kvs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kVW = 8;                        // waves
constexpr int kVThreads = 64 * kVW;
constexpr int kVTok = kPageTokens / kVW;      // tokens per wave in QK (32)
constexpr int kVChunks = kPageTokens / 32;    // 32-token P.V chunks per page
constexpr float kLazyMax = 8.f;

// This wave's share of the LDS DMA of one (page, kv head) K tile and V tile
// (1 KB pieces: wave w takes pieces w, w + 8, ...). A wave past the last
// piece copies the last piece again (the same bytes to the same place), so
// every wave issues the same number of DMA instructions and the code has no
// branch. The source addresses are returned so that the caller can keep
// their registers from being reused while the DMAs are in flight (the
// compiler would otherwise wait for the DMAs before reusing them).
template <typename VT>
struct PageDma {
    static constexpr int kKP = kKTile / 1024, kVP = VT::kTile / 1024;
    static constexpr int kKW = (kKP + kVW - 1) / kVW, kVWv = (kVP + kVW - 1) / kVW;
    const uint8_t* src[kKW + kVWv];
};
template <typename VT>
__device__ inline PageDma<VT> dma_page(const uint8_t* rec, int g, int n_kv_heads, uint8_t* k_lds, uint8_t* v_lds,
                                       int w, int lane) {
    using D = PageDma<VT>;
    static_assert(kKTile % 1024 == 0 && VT::kTile % 1024 == 0, "tiles in 1 KB pieces");
    const uint8_t* kt = rec + (int64_t)g * kKTile;
    const uint8_t* vt = rec + (int64_t)n_kv_heads * kKTile + (int64_t)g * VT::kTile;
    D ad;
#pragma unroll
    for (int k = 0; k < D::kKW; ++k) {
        const uint32_t p = (uint32_t)min(w + kVW * k, D::kKP - 1);
        ad.src[k] = kt + (p * 1024u + (uint32_t)lane * 16u);
        dma16(ad.src[k], k_lds + p * 1024);
    }
#pragma unroll
    for (int k = 0; k < D::kVWv; ++k) {
        const uint32_t p = (uint32_t)min(w + kVW * k, D::kVP - 1);
        ad.src[D::kKW + k] = vt + (p * 1024u + (uint32_t)lane * 16u);
        dma16(ad.src[D::kKW + k], v_lds + p * 1024);
    }
    return ad;
}
template <typename VT>
__device__ inline void keep(const PageDma<VT>& ad) {
#pragma unroll
    for (int k = 0; k < PageDma<VT>::kKW + PageDma<VT>::kVWv; ++k) asm volatile("" ::"v"(ad.src[k]));
}

// Block scales of this lane's four score tokens of a tile (token 4 gq + i of
// the tile), from the 16 binary16 values [i][b] in two 16-byte words (sa:
// i = 0, 1; sb: i = 2, 3), as float32 (exact).
__device__ inline void tile_scales(u32x4 sa, u32x4 sb, float (&d)[4][kNB]) {
    const uint32_t wd[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d[i][0] = scale_f32(wd[2 * i]);
        d[i][1] = scale_f32(wd[2 * i] >> 16);
        d[i][2] = scale_f32(wd[2 * i + 1]);
        d[i][3] = scale_f32(wd[2 * i + 1] >> 16);
    }
}

// s = sum over blocks of (block product x block scale) in float32, block 0
// first, each further block fused in, in block order.
__device__ inline void add_block(f32x4& s, const f32x4& acc, const float (&d)[4][kNB], int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma clang fp contract(off)
        s[i] = b == 0 ? acc[i] * d[i][0] : __builtin_fmaf(acc[i], d[i][b], s[i]);
    }
}

template <int RT, int LIMBS, typename VT>
__global__ __launch_bounds__(kVThreads) void verify_kernel(AttendArgs a) {
    // two page buffers as separate arrays: a read of one is ordered only
    // after the LDS DMAs into that one, not after the next page's DMA into
    // the other
    __shared__ __attribute__((aligned(16))) uint8_t k_lds0[kKTile];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds0[VT::kTile];
    __shared__ __attribute__((aligned(16))) uint8_t k_lds1[kKTile];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds1[VT::kTile];
    __shared__ __attribute__((aligned(16))) uint8_t p_lds[kVChunks * RT * 64 * 16];   // P^T operands [chunk][rt][lane]
    __shared__ __attribute__((aligned(16))) uint32_t ksc[kVW][kVTok * 2];               // K scales [token][block] f16
    __shared__ float red_m[kVW][16 * RT];
    __shared__ float red_l[kVW][16 * RT];
    __shared__ __attribute__((aligned(16))) uint16_t vsc[kNB][kPageTokens];   // the page's V scales, 0 past the cache
    // 1-D grid: the ring refill workgroups first, then the workers, permuted
    // so that each of the 8 XCDs takes a contiguous range of them.
    const int G = a.G, R = a.n_q * G;
    const int n_copy8 = (copy_workgroups(a.copy) + 7) & ~7;
    const int L = (int)blockIdx.x;
    if (L < n_copy8) {   // ring refill workgroup
        if (threadIdx.x < 256) copy_role(a.copy, L);
        return;
    }
    const int n_work = a.n_slices * a.n_kv_heads;
    const int per_xcd = ((n_work + 7) & ~7) / 8;
    const int work = ((L - n_copy8) & 7) * per_xcd + ((L - n_copy8) >> 3);
    if (work >= n_work) return;
    const int slice = work / a.n_kv_heads;
    const int g = work % a.n_kv_heads;
    if (slice >= a.n_segs) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;   // MFMA row/column index and lane group

    // ---- this lane's query rows (one per row tile) and their visible prefix
    half8_t qop[RT][LIMBS][kNB];
    float cq[RT];
    int qi_[RT], h_[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = 16 * rt + n;
        qi_[rt] = r / G;
        h_[rt] = g * G + r % G;
        query_operands<LIMBS>(a, qi_[rt], h_[rt], r < R, gq, qop[rt], cq[rt]);
    }
    // visible prefix: the smallest over the rows, lim_min (causal limits grow
    // with the query index; pages below it need no mask), and each row's
    // excess over it, in [0, n_q) (rows past R have zero queries and any
    // limit)
    int64_t lim_min = a.n_kv;
    if (a.causal) {
        const int64_t c = a.q_pos0 + 1;
        lim_min = c < lim_min ? c : lim_min;
    }
    int dlim[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        dlim[rt] = 0;
        if (a.causal) {
            const int64_t c = a.q_pos0 + qi_[rt] + 1;
            dlim[rt] = (int)((c < a.n_kv ? c : a.n_kv) - lim_min);
        }
    }
    const uint32_t magic = vconst(0x64006400u);
    const int vb = w >> 1, vh = w & 1;   // P.V: quant block and 16-channel half of this wave

    // ---- the walk: segments slice, slice + n_slices, ..., pages in order
    int seg_i = slice, pi = 0;
    int4v segv = scalar_load((const int4v*)(a.segs + seg_i));
    dma_page<VT>(page_record(a.ps, segv.y), g, a.n_kv_heads, k_lds0, v_lds0, w, lane);

    // running state: O^T tiles [rt] hold channels 16 w + 4 gq + i of row
    // 16 rt + n, in units of 2^vsh_run; m and l are replicated over the lanes
    // of a row
    f32x4 o[RT];
    float m_run[RT], l_run[RT];
    int vsh_run = 0;
    auto start_segment = [&]() {
        vsh_run = 0;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            m_run[rt] = -INFINITY;
            l_run[rt] = 0.f;
            o[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!(segv.w & kSegFresh) && 16 * rt + n < R) {
                const float* pr = a.part + (((int64_t)segv.x * a.n_q + qi_[rt]) * a.n_q_heads + h_[rt]) * kPartStride;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[rt][i] = pr[16 * w + 4 * gq + i];
                m_run[rt] = pr[kHeadDim];
                l_run[rt] = pr[kHeadDim + 1];
            }
        }
    };
    start_segment();

    // One page from buffer CUR; returns whether the walk has another page
    // (whose DMA into the other buffer it has issued). The last page of the
    // walk fetches the spare device record into the other buffer instead
    // (bytes that are not used), so that every page issues the same DMAs: a
    // DMA under a branch makes the compiler wait for it at every later LDS
    // read.
    auto step = [&](auto cur) -> bool {
        constexpr int CUR = decltype(cur)::value;
        uint8_t* const kc = CUR ? k_lds1 : k_lds0;
        uint8_t* const vc = CUR ? v_lds1 : v_lds0;
        uint8_t* const kn = CUR ? k_lds0 : k_lds1;
        uint8_t* const vn = CUR ? v_lds0 : v_lds1;
        const int npages = segv.z;
        const int page = segv.y + pi;
        const int64_t base_tok = (int64_t)page * kPageTokens;
        const bool mask_page = base_tok + kPageTokens > lim_min;   // uniform
        // lim_min - base_tok, clamped to a range where the row excesses
        // (below 2^24) cannot overflow
        const int64_t lx = lim_min - base_tok;
        const int lrel = (int)(lx < -kPageTokens ? -kPageTokens : (lx > kPageTokens ? kPageTokens : lx));
        const int64_t vx = a.n_kv - base_tok;
        const int valid = (int)(vx < 0 ? 0 : (vx > kPageTokens ? kPageTokens : vx));   // cached rows of the page
        // the next page of the walk
        int nseg_i = seg_i, npi = pi + 1;
        if (npi >= npages) {
            nseg_i += a.n_slices;
            npi = 0;
        }
        const bool has_next = nseg_i < a.n_segs;
        int4v nsegv = segv;
        if (has_next && npi == 0) nsegv = scalar_load((const int4v*)(a.segs + nseg_i));
        const uint8_t* const next_rec = has_next ? page_record(a.ps, nsegv.y + npi) : a.spare;

        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this page's DMAs (and any loaded state)
        lds_barrier();   // the page's tiles are in LDS; every wave is done with the other buffer
        // the page's V scales as a [block][token] table, read after the
        // barriers below: rows past the cache may hold any bytes (NaN
        // scales) and get 0, so that their V values are 0 (their scores are
        // masked). No LDS DMA is in flight yet.
#pragma unroll
        for (int k = 0; k < kNB * kPageTokens / kVThreads; ++k) {
            const int e = tid + kVThreads * k, t = e % kPageTokens, b = e / kPageTokens;
            const uint16_t bits = *(const uint16_t*)(vc + t * VT::kRow + b * VT::kBlock);
            vsc[b][t] = t < valid ? bits : (uint16_t)0;
        }
        const PageDma<VT> ad = dma_page<VT>(next_rec, g, a.n_kv_heads, kn, vn, w, lane);

        // ---- QK over this wave's 32 tokens (each tile's block scales are
        // published per token for the score lanes)
        f32x4 s[2][RT];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            KRaw kr[kNB];
#pragma unroll
            for (int b = 0; b < kNB; ++b) kr[b] = k_raw(kc, kVTok * w + 16 * tt + n, b, gq);
            // the four lanes of a token hold the same scales: all write them
            *(uint2*)&ksc[w][(16 * tt + n) * 2] = make_uint2(kr[0].db | (kr[1].db << 16), kr[2].db | (kr[3].db << 16));
            // written by this wave just above: the wave's own LDS operations
            // complete in order
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const u32x4* sp = (const u32x4*)&ksc[w][(16 * tt + 4 * gq) * 2];
            const u32x4 sa = sp[0], sb = sp[1];
            float dsc[4][kNB];
            tile_scales(sa, sb, dsc);
            // all products of the tile first, so that no scaling waits on the
            // matrix core's latency
            f32x4 acc[RT][kNB];
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                const half8_t kop = k_codes(kr[b], b);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    acc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[rt][0][b], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if constexpr (LIMBS == 2)
                        acc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[rt][1][b], acc[rt][b], 0, 0, 0);
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int b = 0; b < kNB; ++b) add_block(s[tt][rt], acc[rt][b], dsc, b);
        }

        // ---- mask, page maxima (lane value i of tile tt is token
        // 32 w + 16 tt + 4 gq + i); cq * s are the log2-unit scores (cq > 0)
        if (mask_page) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                // token 32 w + 16 tt + 4 gq + i is visible to the row when
                // 16 tt + i < its limit minus 32 w + 4 gq
                const int lr = lrel + dlim[rt] - kVTok * w - 4 * gq;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[tt][rt][i] = 16 * tt + i < lr ? s[tt][rt][i] : -INFINITY;
            }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tt][rt][i]);
            mx = max_xor16(mx);
            mx = max_xor32(mx);
            red_m[w][16 * rt + n] = mx * cq[rt];   // the same bits in the row's four lanes
        }
        lds_barrier();   // maxima published

        float m_use[RT], alpha[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float pm = red_m[0][16 * rt + n];
#pragma unroll
            for (int ww = 1; ww < kVW; ++ww) pm = fmaxf(pm, red_m[ww][16 * rt + n]);
            // pm > -inf + 8 holds for any finite pm: the first visible page sets m
            const bool grow = pm > m_run[rt] + kLazyMax;
            alpha[rt] = grow ? __builtin_amdgcn_exp2f(m_run[rt] - pm) : 1.f;   // 0 while the state is empty
            m_run[rt] = grow ? pm : m_run[rt];
            m_use[rt] = m_run[rt] == -INFINITY ? 0.f : m_run[rt];
        }
        // ---- probabilities -> this wave's chunk of P^T operands (slot
        // 8 gq + j is token 32 w + 4 gq + j for j < 4, 32 w + 12 + 4 gq + j
        // otherwise: tile j >> 2, value j & 3)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float ls = 0.f;
            half8_t pv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j >> 2][rt][j & 3], cq[rt], -m_use[rt]));
                ls += p;
                pv[j] = (_Float16)p;
            }
            *(half8_t*)(p_lds + ((w * RT + rt) * 64 + lane) * 16) = pv;
            ls = add_xor16(ls);
            ls = add_xor32(ls);
            red_l[w][16 * rt + n] = ls;   // the same bits in the row's four lanes
        }
        lds_barrier();   // P operands and row sums published

        bool rescale = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float lp = red_l[0][16 * rt + n];
#pragma unroll
            for (int ww = 1; ww < kVW; ++ww) lp += red_l[ww][16 * rt + n];
            l_run[rt] = l_run[rt] * alpha[rt] + lp;
            rescale |= alpha[rt] != 1.f;
        }
        if (__any(rescale)) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) o[rt] *= alpha[rt];
        }

        // ---- this page's V shift for block vb; the accumulator moves to its
        // units when it changes (an exact power-of-two rescale)
        const int vsh = v_shift_of<VT>(vc, vb, valid, lane);
        if (vsh != vsh_run) {
            const float f = __builtin_amdgcn_ldexpf(1.f, vsh_run - vsh);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) o[rt] *= f;
            vsh_run = vsh;
        }
        const VHalf hc = v_half<VT>(vh, vsh);

        // ---- P.V for channels 16 w .. 16 w + 15
        {
            // each chunk's LDS reads (V bytes, scales, P operands) are issued
            // two chunks ahead, after the current chunk's conversion (which
            // waits for its own reads), and scheduling barriers keep the
            // three parts of an iteration apart: a wait then never includes
            // reads issued after the ones it needs
            const VLane vl = v_lane<VT>(vb, gq, n, vh);
            VRaw1<VT> vr[3];
            half8_t pp[3][RT];
            auto read_chunk = [&](int c) {
                vr[c % 3] = v_raw1<VT>(vc, vl, vsc[vb], c, gq);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) pp[c % 3][rt] = *(const half8_t*)(p_lds + ((c * RT + rt) * 64 + lane) * 16);
            };
            read_chunk(0);
            read_chunk(1);
#pragma unroll
            for (int c = 0; c < kVChunks; ++c) {
                const half8_t vop = v_convert1<VT>(vr[c % 3], hc, magic);
                half8_t pc[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) pc[rt] = pp[c % 3][rt];
                asm volatile("" : "+v"(pc[0]));   // the P operands are waited for here too
                __builtin_amdgcn_sched_barrier(0);
                if (c + 2 < kVChunks) read_chunk(c + 2);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) o[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pc[rt], o[rt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- the segment's last page: group state -> partial record (O back
        // in absolute units)
        if (pi == npages - 1) {
            const float ounit = __builtin_amdgcn_ldexpf(1.f, vsh_run);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (16 * rt + n >= R) continue;
                float* pr = a.part + (((int64_t)segv.x * a.n_q + qi_[rt]) * a.n_q_heads + h_[rt]) * kPartStride;
                const f32x4 ov = o[rt] * ounit;
                float2* dst = (float2*)(pr + 16 * w + 4 * gq);
                dst[0] = make_float2(ov[0], ov[1]);
                dst[1] = make_float2(ov[2], ov[3]);
                if (w == 0 && gq == 0) {
                    pr[kHeadDim] = m_run[rt];
                    pr[kHeadDim + 1] = l_run[rt];
                }
            }
        }
        keep(ad);
        seg_i = nseg_i;
        pi = npi;
        if (has_next && npi == 0) {
            segv = nsegv;
            start_segment();
        }
        return has_next;
    };
    for (;;) {
        if (!step(std::integral_constant<int, 0>{})) break;
        if (!step(std::integral_constant<int, 1>{})) break;
    }
}

template <int RT, int LIMBS>
hipError_t launch_rt(const AttendArgs& a, hipStream_t stream) {
    // one worker per segment, unless the launch has many segments (a verify
    // block over a long cache): then one worker per compute unit, each
    // taking an even slice of its kv head's segments
    const int64_t units = a.n_kv_heads;
    const int64_t target = compute_units();
    int64_t slices = a.n_segs;
    if (units * a.n_segs > 2 * target && units * 8 <= target) slices = target / units;
    AttendArgs b = a;
    b.n_slices = (int32_t)slices;
    const int64_t n_work = slices * units;
    const int64_t blocks = ((copy_workgroups(a.copy) + 7) & ~7) + ((n_work + 7) & ~7);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (a.v_q8) return launch_kernel(verify_kernel<RT, LIMBS, VQ8>, dim3((unsigned)blocks), dim3(kVThreads), stream, b);
    return launch_kernel(verify_kernel<RT, LIMBS, VQ4>, dim3((unsigned)blocks), dim3(kVThreads), stream, b);
}

}  // namespace

bool verify_rows(int rows) { return rows > 6 && rows <= 32; }

hipError_t launch_verify(const AttendArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    if (!a.spare) return hipErrorInvalidValue;   // the walk's last DMA reads it
    const int R = a.n_q * a.G;
    if (R <= 16) return a.q_f16 ? launch_rt<1, 1>(a, stream) : launch_rt<1, 2>(a, stream);
    return a.q_f16 ? launch_rt<2, 1>(a, stream) : launch_rt<2, 2>(a, stream);
}

}  // namespace kvs
