// Matrix-core attention kernel for query blocks of 33 to 64 rows per kv head
// (a speculative verify batch of 1 + draft tokens with a long draft; page 2,
// "Phase arena: speculative verify batches"), on CDNA4
// v_mfma_f32_16x16x32_f16. Blocks of 7 to 32 rows take the verify kernel
// (kvs_verify.hip), which holds every row of a kv head in one workgroup.
//
// One workgroup = one segment (run of pages of one split-K group) x one kv
// head x a tile of 16 RT query rows (row = query token x head of the GQA
// group). 4 waves. Every page is staged whole in LDS by LDS DMA (K tile
// 34816 B, V tile 18432 B for Q4_0 V or 34816 B for Q8_0 V, record layout);
// the next page's K and V tiles are fetched once the wave's P.V reads are
// done. Then:
//   QK   wave w owns tokens [64 w, 64 w + 64) of the page:
//        A_b^T (16 tokens x 16 rows) = K_b (16 x 32) . Q_b^T (32 x 16) for each
//        32-wide quant block b, with K_b the block's int8 codes as exact f16
//        and Q_b the query as exact f16 limbs (one for f16 queries, a high and
//        a low limb for f32 ones, each row first scaled by a power of two).
//        Each block's product is multiplied by its float32 block scale and
//        the four are summed in float32, so no score is rounded to f16 and
//        no block scale can overflow an operand: the scores are float32 sums
//        of exact products, times scale * log2(e) (log2 units).
//   softmax  page maxima per row across the 4 waves through LDS; the running
//        max m, p = exp2(s - m). Each lane's scores sit exactly where the P.V
//        product wants its P operand, so P never leaves registers on the
//        producing wave; it is published to LDS for the channel owners.
//   PV   wave w owns channels [32 w, 32 w + 32) (= V quant block w):
//        O^T (16 channels x 16 rows) += V^T (16 x 32 tokens) . P^T (32 x 16).
//        The V operand is d * (u - 8) (Q4_0) or d * code (Q8_0) rounded once
//        to f16. A page whose block w holds a scale above 8188 (Q4_0) or
//        511.75 (Q8_0), where the product could exceed the f16 range, takes
//        it divided by 8 (Q4_0) or 128 (Q8_0) instead; the wave keeps its
//        accumulator in units of 2^shift and rescales it exactly when the
//        shift changes.
// The running state (m, l, O) is updated once per page in page order from
// state and page data alone, so results do not depend on how pages are split
// into launches or which pages are resident.
//
// Blocks of more than 64 rows per kv head (a prefill ubatch) go to the
// prefill kernel (kvs_prefill.hip), which converts each page once per
// 256-row block. The page conversion code of both is in kvs_convert.h.
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTokW = kPageTokens / kWaves;   // tokens per wave in QK (64)
constexpr int kChunks = kPageTokens / 32;     // 32-token MFMA chunks per page in PV
// The running max moves only when a page's max exceeds it by more than this
// (log2 units), so p <= 2^8 stays well inside f16 and O is rarely rescaled.
constexpr float kLazyMax = 8.f;

// LDS of the kernel (see mfma_kernel): one page's K tile and V tile in
// record layout, the P operands [chunk][row tile][lane] (16 bytes each) in a
// region of their own, so that the next page's K tile can be fetched into the
// K tile as soon as every wave is past QK, during the softmax and P.V of the
// current page, each wave's K block scales per token ([token][block] f16,
// the layout the score lanes read them in), and the row maxima and sums of
// the four waves. (Double-buffering the page tiles measured slower: the next
// page's LDS DMA then competes with the QK reads of the current one.)

// Stage one (page, kv head) tile of a page record into LDS by LDS DMA:
// wave-sized pieces of 1 KB, 34 for K and 18 (Q4_0) or 34 (Q8_0) for V.
__device__ inline void dma_k_tile(const uint8_t* rec, int g, uint8_t* k_lds, int w, int lane) {
    const uint8_t* kt = rec + (int64_t)g * kKTile;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int piece = w + 4 * k;
        if (piece < kKTile / 1024) dma16(kt + piece * 1024 + lane * 16, k_lds + piece * 1024);
    }
}
template <typename VT>
__device__ inline void dma_v_tile(const uint8_t* rec, int g, int n_kv_heads, uint8_t* v_lds, int w, int lane) {
    static_assert(VT::kTile % 1024 == 0, "V tile in 1 KB pieces");
    const uint8_t* vt = rec + (int64_t)n_kv_heads * kKTile + (int64_t)g * VT::kTile;
#pragma unroll
    for (int k = 0; k < (VT::kTile / 1024 + 3) / 4; ++k) {
        const int piece = w + 4 * k;
        if (piece < VT::kTile / 1024) dma16(vt + piece * 1024 + lane * 16, v_lds + piece * 1024);
    }
}


// Block scales of this lane's four score tokens of a tile (token 4 gq + i of
// the tile), from the 16 binary16 values [i][b] in two 16-byte words (sa:
// i = 0, 1; sb: i = 2, 3), as float32 (exact).
__device__ inline void tile_scales(u32x4 sa, u32x4 sb, float (&d)[4][kNB]) {
    const uint32_t w[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d[i][0] = scale_f32(w[2 * i]);
        d[i][1] = scale_f32(w[2 * i] >> 16);
        d[i][2] = scale_f32(w[2 * i + 1]);
        d[i][3] = scale_f32(w[2 * i + 1] >> 16);
    }
}

// Score accumulation over the quant blocks of a tile, in float32: block 0's
// product times its scale, then each further block's product fused in with
// its scale, in block order; the caller multiplies by the row factor last.
__device__ inline void add_block(f32x4& s, const f32x4& a, const float (&d)[4][kNB], int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma clang fp contract(off)
        s[i] = b == 0 ? a[i] * d[i][0] : __builtin_fmaf(a[i], d[i][b], s[i]);
    }
}


// Workgroups per CU the register budget is cut for.
#ifndef KVS_MFMA_OCC
#define KVS_MFMA_OCC 2
#endif
template <int RT, int LIMBS, typename VT>
__global__ __launch_bounds__(kThreads, KVS_MFMA_OCC)
void mfma_kernel(AttendArgs a) {
    // separate LDS arrays: a read of one is then ordered only after the LDS
    // DMA into that one, not after the next page's DMA into another
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[kKTile];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds[VT::kTile];
    __shared__ __attribute__((aligned(16))) uint8_t p_lds[kChunks * RT * 64 * 16];
    __shared__ __attribute__((aligned(16))) uint32_t ksc[kWaves][kTokW * 2];
    __shared__ float red_m[kWaves][16 * RT];
    __shared__ float red_l[kWaves][16 * RT];
    // 1-D grid: the ring refill workgroups first (so that they start at
    // once), then the workers. A worker owns one (kv head, row tile) and walks
    // the segments slice, slice + n_slices, ...: its query operands are built
    // once, and each segment's first page is fetched while the one before is
    // finished. Workgroups go to the 8 XCDs round-robin by linear index; the
    // workers are permuted so that each XCD takes a contiguous range, and the
    // row tiles of one kv head, which read the same pages, run together on one
    // XCD and share its L2.
    const int G = a.G, R = a.n_q * G;
    const int n_rt = (R + 16 * RT - 1) / (16 * RT);
    const int n_copy8 = (copy_workgroups(a.copy) + 7) & ~7;
    const int L = (int)blockIdx.x;
    if (L < n_copy8) {   // ring refill workgroup
        copy_role(a.copy, L);
        return;
    }
    const int n_work = a.n_slices * a.n_kv_heads * n_rt;
    const int per_xcd = ((n_work + 7) & ~7) / 8;
    const int work = ((L - n_copy8) & 7) * per_xcd + ((L - n_copy8) >> 3);
    if (work >= n_work) return;
    const int slice = work / (n_rt * a.n_kv_heads);
    const int g = (work / n_rt) % a.n_kv_heads;
    const int r0 = (work % n_rt) * 16 * RT;
    if (slice >= a.n_segs) return;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;   // MFMA row/column index and lane group
    typedef int int4v __attribute__((ext_vector_type(4)));

    {
        const uint8_t* rec = page_record(a.ps, scalar_load(&a.segs[slice].page0));
        dma_k_tile(rec, g, k_lds, w, lane);
        dma_v_tile<VT>(rec, g, a.n_kv_heads, v_lds, w, lane);
    }

    // ---- this lane's query rows (one per row tile) and their visible prefix
    half8_t qop[RT][LIMBS][kNB];
    float cq[RT];
    int qi_[RT], h_[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = r0 + 16 * rt + n;
        qi_[rt] = r / G;
        h_[rt] = g * G + r % G;
        query_operands<LIMBS>(a, qi_[rt], h_[rt], r < R, gq, qop[rt], cq[rt]);
    }

    const uint32_t m_nib = vconst(0x000F000Fu), magic = vconst(0x64006400u);

    // visible prefix: the smallest over the workgroup's rows, lim_min (causal
    // limits grow with the query index; pages below it need no mask), and
    // each row's excess over it, below 2^24 (rows past R have zero queries
    // and any limit)
    int64_t lim_min = a.n_kv;
    if (a.causal) {
        const int64_t c = a.q_pos0 + r0 / G + 1;
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

  for (int seg_i = slice; seg_i < a.n_segs; seg_i += a.n_slices) {
    const int4v segv = scalar_load((const int4v*)(a.segs + seg_i));
    const Seg seg = {segv.x, segv.y, segv.z, segv.w};

    // ---- running state: O^T tiles [ct][rt] hold channels 32 w + 16 ct + 4 gq + i
    // of row 16 rt + n, in units of 2^vsh_run; m and l are replicated over the
    // lanes of a row
    f32x4 o[2][RT];
    float m_run[RT], l_run[RT];
    int vsh_run = 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m_run[rt] = -INFINITY;
        l_run[rt] = 0.f;
        o[0][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        o[1][rt] = o[0][rt];
        if (!(seg.flags & kSegFresh) && r0 + 16 * rt + n < R) {
            const float* pr = a.part + (((int64_t)seg.group * a.n_q + qi_[rt]) * a.n_q_heads + h_[rt]) * kPartStride;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[ct][rt][i] = pr[32 * w + 16 * ct + 4 * gq + i];
            m_run[rt] = pr[kHeadDim];
            l_run[rt] = pr[kHeadDim + 1];
        }
    }
    // the stored state is in registers before any page's LDS DMA is issued
    // (a wait for it later would also wait for those DMAs): vmcnt(0), other
    // counters untouched
    __builtin_amdgcn_s_waitcnt(0x0F70);

    for (int pi = 0; pi < seg.npages; ++pi) {
        const int page = seg.page0 + pi;
        const int64_t base_tok = (int64_t)page * kPageTokens;
        const bool mask_page = base_tok + kPageTokens > lim_min;   // uniform
        const bool tail_page = base_tok + kPageTokens > a.n_kv;    // rows past the cache
        // lim_min - base_tok, clamped to a range where adding the row
        // excesses cannot overflow
        const int64_t lx = lim_min - base_tok;
        const int lrel = (int)(lx < -kPageTokens ? -kPageTokens : (lx > kPageTokens ? kPageTokens : lx));
        const int64_t vx = a.n_kv - base_tok;
        const int valid = (int)(vx < 0 ? 0 : (vx > kPageTokens ? kPageTokens : vx));   // cached rows of the page
        // the worker's next page (this segment's next, else the first of its
        // next segment), whose tiles are fetched while this page finishes
        const uint8_t* next_rec = nullptr;
        if (pi + 1 < seg.npages) next_rec = page_record(a.ps, page + 1);
        else if (seg_i + a.n_slices < a.n_segs) next_rec = page_record(a.ps, scalar_load(&a.segs[seg_i + a.n_slices].page0));

        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), known to the compiler's wait tracking
        lds_barrier();   // the page's tiles are in LDS for every wave
        if (tail_page) {
            // rows past the cache may hold any bytes (NaN scales): their V
            // scales are zeroed here, before the barriers that precede every
            // read of the V tile, so that their V values are 0 (their scores
            // are masked)
            for (int e = tid; e < (kPageTokens - valid) * kNB; e += kThreads)
                *(uint16_t*)(v_lds + (valid + e / kNB) * VT::kRow + (e % kNB) * VT::kBlock) = 0;
        }

        // ---- QK over this wave's 64 tokens, one product per quant block (the
        // conversion reads the next token tile's K bytes while converting the
        // current one, and publishes each tile's block scales per token for
        // the score lanes)
        f32x4 s[4][RT];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            KRaw kr[kNB];
#pragma unroll
            for (int b = 0; b < kNB; ++b) kr[b] = k_raw(k_lds, kTokW * w + 16 * tt + n, b, gq);
            if (gq == 0) {
                const KRaw* k = kr;
                *(uint2*)&ksc[w][(16 * tt + n) * 2] = make_uint2(k[0].db | (k[1].db << 16), k[2].db | (k[3].db << 16));
            }
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

        // ---- mask, page maxima (lane value i is token 64 w + 16 tt + 4 gq + i);
        // s holds the float32 products, cq * s the log2-unit scores (cq > 0)
        if (mask_page) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                // token 64 w + 16 tt + 4 gq + i is visible to the row when
                // 16 tt + i < its limit minus 64 w + 4 gq
                const int lr = lrel + dlim[rt] - kTokW * w - 4 * gq;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[tt][rt][i] = 16 * tt + i < lr ? s[tt][rt][i] : -INFINITY;
            }
        }
        float mx[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            mx[rt] = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx[rt] = fmaxf(mx[rt], s[tt][rt][i]);
            mx[rt] = max_xor16(mx[rt]);
            mx[rt] = max_xor32(mx[rt]);
            if (gq == 0) red_m[w][16 * rt + n] = mx[rt] * cq[rt];
        }
        lds_barrier();   // maxima published; every wave is done reading the K tile

        float m_use[RT], alpha[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float pm = red_m[0][16 * rt + n];
#pragma unroll
            for (int ww = 1; ww < kWaves; ++ww) pm = fmaxf(pm, red_m[ww][16 * rt + n]);
            // pm > -inf + 8 holds for any finite pm: the first visible page sets m
            const bool grow = pm > m_run[rt] + kLazyMax;
            alpha[rt] = grow ? __builtin_amdgcn_exp2f(m_run[rt] - pm) : 1.f;   // 0 while the state is empty
            m_run[rt] = grow ? pm : m_run[rt];
            m_use[rt] = m_run[rt] == -INFINITY ? 0.f : m_run[rt];
        }
        // ---- probabilities -> P operands in LDS (slot 8 gq + j of chunk c is
        // token 32 c + 4 gq + j for j < 4, 32 c + 12 + 4 gq + j otherwise)
        uint8_t* pbuf = p_lds;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float ls = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                half8_t pv;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * c2 + (j >> 2)][rt][j & 3], cq[rt], -m_use[rt]));
                    ls += p;
                    pv[j] = (_Float16)p;
                }
                *(half8_t*)(pbuf + (((2 * w + c2) * RT + rt) * 64 + lane) * 16) = pv;
            }
            ls = add_xor16(ls);
            ls = add_xor32(ls);
            if (gq == 0) red_l[w][16 * rt + n] = ls;
        }
        lds_barrier();   // P operands and row sums published

        bool rescale = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float lp = red_l[0][16 * rt + n];
#pragma unroll
            for (int ww = 1; ww < kWaves; ++ww) lp += red_l[ww][16 * rt + n];
            l_run[rt] = l_run[rt] * alpha[rt] + lp;
            rescale |= alpha[rt] != 1.f;
        }
        if (__any(rescale)) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) o[ct][rt] *= alpha[rt];
        }

        // ---- this page's V shift for block w; the accumulator moves to its
        // units when it changes (an exact power-of-two rescale)
        const int vsh = v_shift_of<VT>(v_lds, w, valid, lane);
        if (vsh != vsh_run) {
            const float f = __builtin_amdgcn_ldexpf(1.f, vsh_run - vsh);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) o[ct][rt] *= f;
            vsh_run = vsh;
        }

        // ---- P.V for channels 32 w .. 32 w + 31 (V quant block w)
        {
            const VLane vl = v_lane<VT>(w, gq, n, 0);
            VRaw<VT> vr[2];
            vr[0] = v_raw_o<VT>(v_lds, vl, 0);
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                half8_t vop[2];
                if (c + 1 < kChunks) vr[(c + 1) & 1] = v_raw_o<VT>(v_lds, vl, c + 1);
                v_convert<false, VT>(vr[c & 1], c, gq, valid, vsh, m_nib, magic, vop);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const half8_t pop = *(const half8_t*)(pbuf + ((c * RT + rt) * 64 + lane) * 16);
                    o[0][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[0], pop, o[0][rt], 0, 0, 0);
                    o[1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[1], pop, o[1][rt], 0, 0, 0);
                }
            }
        }
        // the next page's K tile (every wave is past QK) is fetched once this
        // wave's V reads are done: the compiler orders an LDS read after any
        // LDS DMA it cannot prove disjoint, so an earlier fetch would hold up
        // the reads of the V tile
        if (next_rec) dma_k_tile(next_rec, g, k_lds, w, lane);
        lds_barrier();   // every wave is done with this page's V tile and P operands
        if (next_rec) dma_v_tile<VT>(next_rec, g, a.n_kv_heads, v_lds, w, lane);
    }

    // ---- group state -> partial records (O back in absolute units)
    const float ounit = __builtin_amdgcn_ldexpf(1.f, vsh_run);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (r0 + 16 * rt + n >= R) continue;
        float* pr = a.part + (((int64_t)seg.group * a.n_q + qi_[rt]) * a.n_q_heads + h_[rt]) * kPartStride;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const f32x4 ov = o[ct][rt] * ounit;
            float2* dst = (float2*)(pr + 32 * w + 16 * ct + 4 * gq);
            dst[0] = make_float2(ov[0], ov[1]);
            dst[1] = make_float2(ov[2], ov[3]);
        }
        if (w == 0 && gq == 0) {
            pr[kHeadDim] = m_run[rt];
            pr[kHeadDim + 1] = l_run[rt];
        }
    }
  }
}

template <int RT, int LIMBS>
hipError_t launch_rt(const AttendArgs& a, hipStream_t stream) {
    const int R = a.n_q * a.G;
    const int64_t units = (int64_t)a.n_kv_heads * ((R + 16 * RT - 1) / (16 * RT));
    // workers: one per segment, unless the launch has few (kv head, row tile)
    // units and many segments (a verify block over a long cache): then about
    // as many workers as the compute units hold at once, each taking an even
    // slice of the segments
    const int64_t target = (int64_t)compute_units() * KVS_MFMA_OCC;
    int64_t slices = a.n_segs;
    if (units * a.n_segs > 2 * target && units * 8 <= target) slices = target / units;
    AttendArgs b = a;
    b.n_slices = (int32_t)slices;
    const int64_t n_work = slices * units;
    const int64_t blocks = ((copy_workgroups(a.copy) + 7) & ~7) + ((n_work + 7) & ~7);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (a.v_q8) return launch_kernel(mfma_kernel<RT, LIMBS, VQ8>, dim3((unsigned)blocks), dim3(kThreads), stream, b);
    return launch_kernel(mfma_kernel<RT, LIMBS, VQ4>, dim3((unsigned)blocks), dim3(kThreads), stream, b);
}

}  // namespace

// 16-row tiles (with two query limbs, wider tiles would not fit two
// workgroups' registers per compute unit), for 33 to 64 rows per kv head;
// blocks of up to 32 rows go to the verify kernel, blocks of more than 64 to
// the prefill kernel.
hipError_t launch_mfma(const AttendArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    if (prefill_rows(a.n_q * a.G)) return launch_prefill(a, stream);
    if (verify_rows(a.n_q * a.G)) return launch_verify(a, stream);
    return a.q_f16 ? launch_rt<1, 1>(a, stream) : launch_rt<1, 2>(a, stream);
}

bool prefill_rows(int rows) { return rows > 64; }


}  // namespace kvs
