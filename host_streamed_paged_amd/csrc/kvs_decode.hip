// Decode attention kernel for few query rows (R = query tokens x heads per kv
// head, R <= 6) on CDNA4, both products on the matrix cores. One workgroup
// per (page run of a split-K group, kv head); 256 threads = 4 waves, and each
// wave owns a 64-token slice of every page from load to weighted sum, so the
// waves never wait on each other until the per-page merge.
//
// Per 64-token slice (a page is 256 tokens of one layer; page 2, "Dynamic
// draft eject"), in 16x16x32 tiles where lane (n, kg) = (l & 15, l >> 4)
// holds operand slots 8 kg .. 8 kg + 7 of row or column n and output rows
// 4 kg .. 4 kg + 3 of column n:
//   QK  S = Q . K^T per (16-token tile, 32-wide block) on
//       v_mfma_i32_16x16x32_i8: exact integer products of the Q8_0 codes,
//       loaded straight from the page record into the lane of their token,
//       with the query held as 16-bit fixed point (per row scale, split into
//       int8 high and low bytes, one instruction each). Each block's
//       integer sum times its scale is accumulated in float32, block 0
//       first, in a fixed order.
//   softmax  lanes hold query rows of one token: slice maxima and row sums
//       are reductions over the 16 lanes of a DPP row; p = exp2(s - m) in
//       log2 units (the softmax scale is folded into the query scale).
//   PV  v_mfma_f32_16x16x32_f16: the slice's V rows are staged in the wave's
//       LDS region, p * d_v is rounded to f16 into a per-wave buffer, and
//       each V block forms two 16-channel tiles of V^T as exact f16 (a Q4_0
//       block's low and high nibbles, u - 8; a Q8_0 block's codes 0..15 and
//       16..31), multiplied against the rows' p * d_v over two 32-token
//       steps.
//   The 4 slice partials of a page are merged into one page partial in a
//   fixed order, and page partials are merged into the group state in page
//   order: results do not depend on how pages are split into launches or
//   which of them are resident.
// Loads are issued query first, then K codes and scales, then V rows, all as
// plain register loads, so each wait covers exactly what the next step reads.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cmath>
#include <type_traits>

#include "kvs_internal.h"
#include "kvs_device.h"

namespace kvs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlice = kPageTokens / kWaves;   // 64 tokens per wave
constexpr int kSlicePairs = kSlice / 2;        // 32 token pairs
constexpr int kPPStride = kSlicePairs * 8 + 8; // dwords per block row of pp (padded: no bank clash across blocks)
constexpr int kKW = 14;                        // K dwords per lane and 16-token tile


// lane i receives lane i +- 1 / 2 / 4 / 8 within its row of 16 (row rotate)
template <int N>
__device__ inline float dpp_ror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, true));
}
// max / sum over the 16 lanes of a DPP row (every lane gets the max; the sum's
// rounding may differ from lane to lane)
__device__ inline float max_over_row16(float v) {
    v = fmaxf(v, dpp_ror<1>(v));
    v = fmaxf(v, dpp_ror<2>(v));
    v = fmaxf(v, dpp_ror<4>(v));
    v = fmaxf(v, dpp_ror<8>(v));
    return v;
}
__device__ inline float sum_over_row16(float v) {
    v += dpp_ror<1>(v);
    v += dpp_ror<2>(v);
    v += dpp_ror<4>(v);
    v += dpp_ror<8>(v);
    return v;
}

__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Every array that is read or written 16 bytes at a time (LDS DMA targets,
// uint4 reads) sits on a 16-byte boundary; misaligned 128-bit LDS accesses
// are split and stall.
template <int R, typename VT>
struct DecodeSmem {
    alignas(16) uint8_t v[kWaves][kSlice * VT::kRow];         // each wave's V rows (record layout)
    alignas(16) uint32_t pp[kWaves][kNB][kPPStride];          // p * d_v as f16 pairs: [wave][block][pair * 8 + row]
    // slice partials (double-buffered by page parity); rows padded to 144
    // floats so that the rows' 16-byte stores fall on different LDS banks
    alignas(16) float sacc[2][kWaves][R][kHeadDim + 16];
    float sm_[2][kWaves][R], sl_[2][kWaves][R];
};

template <int R, typename VT>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(AttendArgs a) {
    __shared__ __attribute__((aligned(16))) DecodeSmem<R, VT> sm;
    if ((int)blockIdx.x >= a.n_segs) {   // ring refill workgroup
        copy_role(a.copy, ((int)blockIdx.x - a.n_segs) * (int)gridDim.y + (int)blockIdx.y);
        return;
    }
    const int tid = threadIdx.x;
    // the wave index is uniform: slice bounds and masks stay in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int g = blockIdx.y;
    const int G = a.G;

    // Matrix-core lane roles (16x16x32 tiles): lane (n, kg) = (l & 15, l >> 4)
    // holds operand slots 8 kg .. 8 kg + 7 of row or column n and output rows
    // 4 kg .. 4 kg + 3 of column n. Scores: token n of each 16-token tile,
    // channels 8 kg .. 8 kg + 7 of each 32-wide block.
    const int n = l & 15, kg = l >> 4;
    const int krow = (kSlice * w + n) * kKRow;   // this lane's token row in the K tile

    // K blocks and V rows are loaded into registers; the V rows are stored to
    // the wave's LDS region once the scores are done. Plain loads (no LDS DMA)
    // keep every load in flight of one kind, so that each score tile waits for
    // its own K codes only.
    uint8_t* vt = sm.v[w];
    auto page_rec = [&](int page) -> const uint8_t* { return page_record(a.ps, page); };
    // Per 16-token tile: this lane's 8 codes of blocks 0..3 (block b starts at
    // byte 34 b of the token row, its codes 2 bytes later: an even block's
    // 8-code window [34 b + 2 + 8 kg, +8) is covered by the 3 aligned dwords
    // from 34 b + 8 kg, an odd block's is itself 2 aligned dwords), then the 4
    // aligned dwords holding the block scales (bytes 0, 32, 68, 100; the scale
    // is the low half for an even block, the high half for an odd one).
    auto issue_k = [&](const uint8_t* rec, uint32_t (&kw)[4][kKW]) {
        const uint8_t* kt = rec + (int64_t)g * kKTile + krow;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint8_t* row = kt + t * 16 * kKRow;
            const uint32_t* b0 = (const uint32_t*)(row + 8 * kg);
            const uint32_t* b1 = (const uint32_t*)(row + kKBlock + 2 + 8 * kg);
            const uint32_t* b2 = (const uint32_t*)(row + 2 * kKBlock + 8 * kg);
            const uint32_t* b3 = (const uint32_t*)(row + 3 * kKBlock + 2 + 8 * kg);
            kw[t][0] = b0[0]; kw[t][1] = b0[1]; kw[t][2] = b0[2];
            kw[t][3] = b1[0]; kw[t][4] = b1[1];
            kw[t][5] = b2[0]; kw[t][6] = b2[1]; kw[t][7] = b2[2];
            kw[t][8] = b3[0]; kw[t][9] = b3[1];
            kw[t][10] = *(const uint32_t*)(row);
            kw[t][11] = *(const uint32_t*)(row + kKBlock - 2);
            kw[t][12] = *(const uint32_t*)(row + 2 * kKBlock);
            kw[t][13] = *(const uint32_t*)(row + 3 * kKBlock - 2);
        }
    };
    // V rows per slice, 4608 bytes (Q4_0) or 8704 (Q8_0): kVL coalesced
    // 16-byte loads and one 8-byte load per lane
    constexpr int kVL = kSlice * VT::kRow / 1024;
    static_assert(kSlice * VT::kRow == kVL * 1024 + 512, "V slice size");
    auto issue_v = [&](const uint8_t* rec, uint4 (&vr)[kVL], uint2& vr2) {
        const uint8_t* vsrc = rec + (int64_t)a.n_kv_heads * kKTile + (int64_t)g * VT::kTile + kSlice * w * VT::kRow;
#pragma unroll
        for (int k = 0; k < kVL; ++k) vr[k] = *(const uint4*)(vsrc + 1024 * k + 16 * l);
        vr2 = *(const uint2*)(vsrc + 1024 * kVL + 8 * l);
    };
    auto store_v = [&](const uint4 (&vr)[kVL], const uint2& vr2) {
#pragma unroll
        for (int k = 0; k < kVL; ++k) *(uint4*)(vt + 1024 * k + 16 * l) = vr[k];
        *(uint2*)(vt + 1024 * kVL + 8 * l) = vr2;
    };

    // ---- query rows -> 16-bit fixed point codes, built by every wave in the
    // layout of the score tiles' A operand: lane (n, kg) holds row n's
    // channels 32 b + 8 kg .. 32 b + 8 kg + 7 of each block b. The query loads
    // are issued first, before the segment is even known, and each wave
    // converts its own copy, so no wave waits for another's page loads to be
    // issued before its scores can start (vector memory counters retire in
    // order: the conversion waits for this wave's query loads only).
    uint4 qlo[kNB], qhi[kNB];   // raw query bits: elements 0..3 (all 8 for f16) and 4..7 of each window
    {
        const int qn = n < R ? n : 0;
        const int qi = qn / G, qhd = g * G + qn % G;
        const uint8_t* qrow = (const uint8_t*)a.q + ((int64_t)qi * a.n_q_heads + qhd) * kHeadDim * (a.q_f16 ? 2 : 4);
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk) {
            const int e0 = blk * kQK + 8 * kg;   // first element of this lane's window
            qlo[blk] = qhi[blk] = make_uint4(0u, 0u, 0u, 0u);
            if (n < R) {
                if (a.q_f16) {
                    qlo[blk] = *(const uint4*)(qrow + 2 * e0);
                } else {
                    qlo[blk] = ((const uint4*)(qrow + 4 * e0))[0];
                    qhi[blk] = ((const uint4*)(qrow + 4 * e0))[1];
                }
            }
        }
    }
    typedef int int4v __attribute__((ext_vector_type(4)));
    const int4v segv = scalar_load((const int4v*)(a.segs + blockIdx.x));
    const Seg seg = {segv.x, segv.y, segv.z, segv.w};
    // memory counters retire in order: query, then K codes, then V rows. The
    // segment carries its first page's source index, so the first record
    // address needs no read of the page table.
    const uint8_t* rec0 = page_record_of(a.ps, seg.page0, seg.flags >> kSegSrcShift);
    uint32_t kw[4][kKW];
    uint4 vr[kVL];
    uint2 vr2;
    issue_k(rec0, kw);
    issue_v(rec0, vr, vr2);
    // score operands: query row n (zero past R) as 16-bit fixed point with a
    // per-row scale, split into int8 high and low bytes
    long qa_hi[kNB], qa_lo[kNB];
    float qsv[4], kav[4];
    {
        float x[kNB][8];
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk) {
            const uint32_t wv[8] = {qlo[blk].x, qlo[blk].y, qlo[blk].z, qlo[blk].w,
                                    qhi[blk].x, qhi[blk].y, qhi[blk].z, qhi[blk].w};
            if (a.q_f16) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[blk][e] = scale_f32(wv[e >> 1] >> (16 * (e & 1)));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[blk][e] = __builtin_bit_cast(float, wv[e]);
            }
        }
        float amax = 0.f;
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[blk][e]));
        // over the row's 4 lanes (n, n + 16, n + 32, n + 48)
        amax = max_xor16(amax);
        amax = max_xor32(amax);
        // |code| <= 32639 keeps the high byte of (code + 128) >> 8 inside int8;
        // a negative softmax scale is folded into the codes' sign
        const float inv = amax > 0.f ? (a.scale_log2 < 0.f ? -32639.f : 32639.f) / amax : 0.f;
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk) {
            uint32_t hw[2] = {0u, 0u}, lw[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                int c = (int)rintf(x[blk][e] * inv);
                c = c > 32639 ? 32639 : (c < -32639 ? -32639 : c);
                const int hi = (c + 128) >> 8;
                const int lo = c - hi * 256;
                hw[e >> 2] |= (uint32_t)(hi & 0xFF) << (8 * (e & 3));
                lw[e >> 2] |= (uint32_t)(lo & 0xFF) << (8 * (e & 3));
            }
            qa_hi[blk] = (long)(((uint64_t)hw[1] << 32) | hw[0]);
            qa_lo[blk] = (long)(((uint64_t)lw[1] << 32) | lw[0]);
        }
        // code -> log2-unit score scale of row n, then of output rows 4 kg + i
        // (held by lanes 4 kg + i)
        const float qs_n = amax / 32639.f * fabsf(a.scale_log2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * kg + i;
            const float q = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * r, __builtin_bit_cast(int, qs_n)));
            qsv[i] = r < R ? q : 0.f;
            // a zero row scale is lifted to a tiny one so that 0 * -inf never arises
            kav[i] = fmaxf(qsv[i], 1e-30f);
        }
    }

    // group state, distributed for the per-page merge: thread owns channels
    // mc4 .. mc4 + 3 of row mr (threads of rows past R take no part), so each
    // thread's merge is one row deep
    static_assert(R * 32 <= kThreads, "one merge row per 32 threads");
    const int mr = tid >> 5, mc4 = 4 * (tid & 31);
    const bool mown = mr < R;
    const int mrr = mown ? mr : 0;
    float acc_run[4] = {0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    if (!(seg.flags & kSegFresh) && mown) {
        const int i = mrr / G, h = g * G + mrr % G;
        const float* pr = a.part + (((int64_t)seg.group * a.n_q + i) * a.n_q_heads + h) * kPartStride;
        const float2 a0 = *(const float2*)(pr + mc4), a1 = *(const float2*)(pr + mc4 + 2);   // records are 8-byte aligned
        acc_run[0] = a0.x; acc_run[1] = a0.y; acc_run[2] = a1.x; acc_run[3] = a1.y;
        m_run = pr[kHeadDim];
        l_run = pr[kHeadDim + 1];
    }

    uint32_t* ppw = sm.pp[w][0];
    // One page of the segment, its K blocks and V rows already in flight.
    // With PREFETCH (every page but the segment's last), the next page's K
    // blocks are loaded into the same registers as soon as the scores are
    // done, and its V rows as soon as this page's rows are in LDS, so that
    // they arrive while this page is still being computed. The last page is
    // peeled off the loop: every load site is then unconditional and each wait
    // covers exactly the loads it needs.
    auto page_body = [&](int pi, auto prefetch) {
        constexpr bool kPrefetch = decltype(prefetch)::value;
        const int page = seg.page0 + pi;
        const uint8_t* rec_next = kPrefetch ? page_rec(page + 1) : nullptr;
        const int par = pi & 1;
        const int64_t rem = a.n_kv - (int64_t)page * kPageTokens - kSlice * w;
        const int valid = (int)(rem < 0 ? 0 : (rem > kSlice ? kSlice : rem));   // valid rows of this slice

        // ---- scores. Slice row t is visible to query row r iff t <= lim[r].
        int lim[R];
        bool need_mask = false;   // wave-uniform: some row does not see the whole slice
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t l64 = (int64_t)valid - 1;
            if (a.causal) {
                const int64_t c = a.q_pos0 + r / G - (int64_t)page * kPageTokens - kSlice * w;
                l64 = c < l64 ? c : l64;
            }
            lim[r] = (int)(l64 < -1 ? -1 : l64);
            need_mask |= lim[r] < kSlice - 1;
        }
        // S = Q . K^T per (16-token tile, block) on v_mfma_i32_16x16x32_i8, once
        // for each byte of the query codes; s[t][i] is row 4 kg + i, token
        // 16 t + n, in units of the row scale
        float s[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int blk = 0; blk < kNB; ++blk) {
                const int o = blk == 0 ? 0 : blk == 1 ? 3 : blk == 2 ? 5 : 8;
                uint32_t c0, c1;
                if (blk & 1) {
                    c0 = kw[t][o];
                    c1 = kw[t][o + 1];
                } else {
                    c0 = __builtin_amdgcn_perm(kw[t][o + 1], kw[t][o], 0x05040302u);
                    c1 = __builtin_amdgcn_perm(kw[t][o + 2], kw[t][o + 1], 0x05040302u);
                }
                const long kb = (long)(((uint64_t)c1 << 32) | c0);
                const i32x4 zero = {0, 0, 0, 0};
                const i32x4 ih = __builtin_amdgcn_mfma_i32_16x16x32_i8(qa_hi[blk], kb, zero, 0, 0, 0);
                const i32x4 il = __builtin_amdgcn_mfma_i32_16x16x32_i8(qa_lo[blk], kb, zero, 0, 0, 0);
                const float d = scale_f32(kw[t][10 + blk] >> (16 * (blk & 1)));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma clang fp contract(off)
                    const float x = (float)(ih[i] * 256 + il[i]);
                    s[t][i] = blk == 0 ? x * d : __builtin_fmaf(x, d, s[t][i]);
                }
            }
        }
        if constexpr (kPrefetch) issue_k(rec_next, kw);   // the scores no longer need kw
        if (need_mask) {
            int limv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r0 = i, r1 = 4 + i;
                const int l0 = r0 < R ? lim[r0 < R ? r0 : 0] : -1;
                const int l1 = r1 < R ? lim[r1 < R ? r1 : 0] : -1;
                limv[i] = kg == 0 ? l0 : (kg == 1 ? l1 : -1);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[t][i] = 16 * t + n <= limv[i] ? s[t][i] : -INFINITY;
        }
        // ---- slice maxima, probabilities and row sums over the 16 lanes of
        // each output row. Masked scores are -inf and give exp2 = 0; a fully
        // masked slice uses 0 as its reference.
        float m_w[4], e[4][4], lsum[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m_w[i] = max_over_row16(fmaxf(fmaxf(s[0][i], s[1][i]), fmaxf(s[2][i], s[3][i])));
            const float mref = m_w[i] == -INFINITY ? 0.f : m_w[i];
            const float moff = -(kav[i] * mref);
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                e[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(kav[i], s[t][i], moff));
                acc += e[t][i];
            }
            lsum[i] = sum_over_row16(acc);
        }
        // The slice's V rows to LDS (read by other lanes of this wave only).
        // Maxima, exponentials and sums above need the scores alone, so they
        // run while the V rows (the last loads of the page) are still in
        // flight; the empty asm ties the rows to the row sums so that the
        // stores, and the wait for the V loads they imply, stay after them.
        {
            const float dep = lsum[0] + lsum[3];
#pragma unroll
            for (int k = 0; k < kVL; ++k)
                asm volatile("" : "+v"(vr[k].x), "+v"(vr[k].y), "+v"(vr[k].z), "+v"(vr[k].w) : "v"(dep));
            asm volatile("" : "+v"(vr2.x), "+v"(vr2.y) : "v"(dep));
        }
        store_v(vr, vr2);
        if constexpr (kPrefetch) issue_v(rec_next, vr, vr2);
        wave_lds_sync();
        // p * d_v as f16 pairs of tokens (t, t + 16), t = 32 q2 + n: the 4 rows
        // 4 kg .. 4 kg + 3 of a (pair, block) are one 16-byte store (rows past R
        // are zero; lanes of rows 8..15 hold none). Each block's scales are
        // first divided by a power of two 2^k_b that puts the slice's largest
        // magnitude in [0.5, 1), so that p * d_v (p <= 1) keeps its precision
        // in f16 whatever the scales' size; the slice partial of the block is
        // multiplied back by 2^k_b (exact).
        float vunit[kNB];
        {
            float dv[4][kNB];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int tok = 16 * t + n;
#pragma unroll
                for (int blk = 0; blk < kNB; ++blk) {
                    const float d = scale_f32(*(const uint16_t*)(vt + tok * VT::kRow + blk * VT::kBlock));
                    dv[t][blk] = tok < valid ? d : 0.f;   // rows past the cache may hold NaN scales
                }
            }
#pragma unroll
            for (int blk = 0; blk < kNB; ++blk) {
                // largest magnitude over the slice's 64 tokens (16 t + n over a DPP row)
                float mx = fmaxf(fmaxf(fabsf(dv[0][blk]), fabsf(dv[1][blk])), fmaxf(fabsf(dv[2][blk]), fabsf(dv[3][blk])));
                mx = max_over_row16(mx);
                const int kb = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) : 0;
                vunit[blk] = __builtin_amdgcn_ldexpf(1.f, kb);
                const float down = __builtin_amdgcn_ldexpf(1.f, -kb);
#pragma unroll
                for (int t = 0; t < 4; ++t) dv[t][blk] *= down;   // exact
            }
            if (kg < 2) {
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2) {
#pragma unroll
                    for (int blk = 0; blk < kNB; ++blk) {
                        uint32_t hv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const half2_t hp = {(_Float16)(e[2 * q2][i] * dv[2 * q2][blk]),
                                                (_Float16)(e[2 * q2 + 1][i] * dv[2 * q2 + 1][blk])};
                            hv[i] = 4 * kg + i < R ? __builtin_bit_cast(uint32_t, hp) : 0u;
                        }
                        *(uint4*)(ppw + blk * kPPStride + (16 * q2 + n) * 8 + 4 * kg) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
                    }
                }
            }
        }
        wave_lds_sync();

        // ---- P.V over the slice on the matrix cores: O^T = V^T . P' per V
        // block, two 16-channel tiles (Q4_0: the low nibbles and the high
        // ones; Q8_0: elements 0..15 and 16..31 of the block), in two 32-token
        // steps (v_mfma_f32_16x16x32_f16). Lane (n, kg) = (l & 15, l >> 4)
        // holds operand slots 8 kg .. 8 kg + 7; slots 8 kg + 2 i and
        // 8 kg + 2 i + 1 of step ks are tokens t = 32 ks + 4 kg + i and t + 16,
        // the pair one dword of the p * d_v buffer holds. A: channel n of the
        // tile as exact f16 (Q4_0: u - 8, high nibbles 16 (u - 8); Q8_0: the
        // code); B: query row n; C: channels 4 kg .. 4 kg + 3 of the tile, row
        // n. B columns of rows past R hold stale buffer words and only reach
        // output columns that are dropped.
        {
            const half2_t off_lo = {(_Float16)1032.f, (_Float16)1032.f};
            const half2_t off_hi = {(_Float16)1152.f, (_Float16)1152.f};
            const half2_t one = {(_Float16)1.f, (_Float16)1.f}, m1152 = {(_Float16)-1152.f, (_Float16)-1152.f};
            const uint32_t m_lo = vconst(0x000F000Fu), m_hi = vconst(0x00F000F0u), magic = vconst(0x64006400u);
#pragma unroll
            for (int vb = 0; vb < kNB; ++vb) {
                f32x4 clo = {0.f, 0.f, 0.f, 0.f}, chi = clo;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const uint8_t* vsrc = vt + (32 * ks + 4 * kg) * VT::kRow + vb * VT::kBlock + 2 + n;
                    const uint32_t* psrc = ppw + vb * kPPStride + (16 * ks + 4 * kg) * 8 + n;
                    u32x4 alo, ahi, bp;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (VT::kQ8) {
                            const uint32_t xl = __builtin_amdgcn_perm((uint32_t)vsrc[(i + 16) * VT::kRow], (uint32_t)vsrc[i * VT::kRow], 0x0c040c00u);
                            const uint32_t xh = __builtin_amdgcn_perm((uint32_t)vsrc[(i + 16) * VT::kRow + 16], (uint32_t)vsrc[i * VT::kRow + 16], 0x0c040c00u);
                            alo[i] = as_u(q8_pair_f16(xl, one, m1152));   // code, element n
                            ahi[i] = as_u(q8_pair_f16(xh, one, m1152));   // code, element 16 + n
                        } else {
                            const uint32_t x = __builtin_amdgcn_perm((uint32_t)vsrc[(i + 16) * VT::kRow], (uint32_t)vsrc[i * VT::kRow], 0x0c040c00u);
                            alo[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, (x & m_lo) | magic) - off_lo);  // u - 8
                            ahi[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, (x & m_hi) | magic) - off_hi);  // 16 (u - 8)
                        }
                        bp[i] = psrc[8 * i];
                    }
                    const half8_t pb = __builtin_bit_cast(half8_t, bp);
                    clo = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, alo), pb, clo, 0, 0, 0);
                    chi = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ahi), pb, chi, 0, 0, 0);
                }
                // slice partial -> LDS (the next page writes the other parity),
                // back in absolute units
                if (n < R) {
                    float* dst = &sm.sacc[par][w][n < R ? n : 0][32 * vb + 4 * kg];
                    *(f32x4*)dst = clo * vunit[vb];
                    // Q4_0 high nibbles carried 16 (u - 8)
                    *(f32x4*)(dst + 16) = chi * (VT::kQ8 ? vunit[vb] : vunit[vb] * 0.0625f);
                }
            }
        }
        if (n == 0 && kg < 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * kg + i;
                if (r < R) {
                    sm.sm_[par][w][r] = m_w[i] == -INFINITY ? -INFINITY : qsv[i] * m_w[i];
                    sm.sl_[par][w][r] = lsum[i];
                }
            }
        }
        lds_barrier();

        // ---- merge the 4 slices (fixed order), then the page into the group state
        if (mown) {
            float ms[kWaves], M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) { ms[ww] = sm.sm_[par][ww][mrr]; M = fmaxf(M, ms[ww]); }
            float pa[4] = {0.f, 0.f, 0.f, 0.f}, pl = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) {
                    const float f = __builtin_amdgcn_exp2f(ms[ww] - M);   // 0 for an empty slice
                    const f32x4 sv = *(const f32x4*)&sm.sacc[par][ww][mrr][mc4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) pa[c] = fmaf(sv[c], f, pa[c]);
                    pl = fmaf(sm.sl_[par][ww][mrr], f, pl);
                }
            }
            const float Mn = fmaxf(m_run, M);
            if (Mn != -INFINITY) {
                const float al = __builtin_amdgcn_exp2f(m_run - Mn);   // 0 from an empty state
                const float be = __builtin_amdgcn_exp2f(M - Mn);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc_run[c] = acc_run[c] * al + pa[c] * be;
                l_run = l_run * al + pl * be;
                m_run = Mn;
            }
        }
    };
    for (int pi = 0; pi + 1 < seg.npages; ++pi) page_body(pi, std::true_type{});
    page_body(seg.npages - 1, std::false_type{});

    if (mown) {
        const int i = mrr / G, h = g * G + mrr % G;
        float* pr = a.part + (((int64_t)seg.group * a.n_q + i) * a.n_q_heads + h) * kPartStride;
        *(float2*)(pr + mc4) = make_float2(acc_run[0], acc_run[1]);
        *(float2*)(pr + mc4 + 2) = make_float2(acc_run[2], acc_run[3]);
        if (mc4 == 0) { pr[kHeadDim] = m_run; pr[kHeadDim + 1] = l_run; }
    }
}

template <int R>
hipError_t launch_r(const AttendArgs& a, hipStream_t stream) {
    const int cx = (copy_workgroups(a.copy) + a.n_kv_heads - 1) / a.n_kv_heads;
    if (a.v_q8) return launch_kernel(decode_kernel<R, VQ8>, dim3(a.n_segs + cx, a.n_kv_heads), dim3(kThreads), stream, a);
    return launch_kernel(decode_kernel<R, VQ4>, dim3(a.n_segs + cx, a.n_kv_heads), dim3(kThreads), stream, a);
}

}  // namespace

// Up to 6 rows the query codes fit in registers (7 and 8 would spill).
bool decode_supports(int rows) { return rows >= 1 && rows <= 6; }

hipError_t launch_decode(const AttendArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    switch (a.n_q * a.G) {
        case 1: return launch_r<1>(a, stream);
        case 2: return launch_r<2>(a, stream);
        case 3: return launch_r<3>(a, stream);
        case 4: return launch_r<4>(a, stream);
        case 5: return launch_r<5>(a, stream);
        case 6: return launch_r<6>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvs
