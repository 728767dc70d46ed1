// Prefill attention kernel: query blocks of more than 64 rows per kv head (a
// prefill ubatch, 256 tokens in page 2's "TLDR - recommended setup"), on
// CDNA4 v_mfma_f32_16x16x32_f16, and the operand probe that writes out what
// it computes on.
//
// One workgroup = one segment (run of pages of one split-K group) x one kv
// head x a block of 256 query rows (row = query token x head of the GQA
// group); 8 waves, each owning 32 rows (two 16-row tiles) from scores to
// output. The workgroup walks its pages in 64-token sub-blocks, as a
// pipeline: the raw K and V rows of a sub-block (13 KB, or 17 KB with Q8_0
// V) are brought into LDS by LDS DMA three steps ahead (four raw buffers);
// in step st all 8 waves convert sub-block st + 1 into f16 matrix-core
// operands (K codes exact, K block scales as float32, V^T as d * (u - 8) or
// d * code rounded once to f16, divided by a power of two when the
// sub-block's scales could overflow; K operands in one of two K buffers, V^T
// in one of three V buffers), then compute the scores and probabilities of
// sub-block st and the P.V of sub-block st - 1. That P.V does not depend on
// st's scores, so its matrix instructions are issued in chunks between st's
// exponentials and run while the vector unit computes them; the state still
// sees every operation in the order of a sub-block-at-a-time walk, so the
// results are the same bits. Each page is converted once per row block,
// inside the workgroup: no staging launch, no staging memory. Per sub-block
// and wave:
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
//        weight V; a block whose sub-block takes V divided by 2^shift keeps
//        its accumulator in those units (an exact rescale when that changes).
// The running state (m, l, O) is updated in a fixed order of pages and
// sub-blocks from state and page data alone, so results do not depend on how
// pages are split into launches or which pages are resident.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cmath>

#include "kvs_internal.h"
#include "kvs_device.h"
#include "kvs_convert.h"

namespace kvs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kRTW = 2;                      // 16-row tiles per wave
constexpr int kRowsWG = 16 * kRTW * kPWaves; // rows per workgroup (256)
constexpr int kSub = 64;                     // tokens per sub-block
constexpr int kSubs = kPageTokens / kSub;    // sub-blocks per page
// Operands of a sub-block in LDS, in two buffers: the K buffer holds the K
// fragments [4 token tiles][4 blocks][64 lanes] x 16 B and then the K block
// scales [token][block] float32; the V buffer holds the V^T fragments
// [2 chunks][8 channel tiles][64 lanes] x 16 B and then the V shift of each
// block (16 B per block, the shift 4 times).
constexpr int kSubK = 4 * kNB * 64 * 16;       // 16 KB
constexpr int kSubV = 2 * 8 * 64 * 16;         // 16 KB
constexpr int kSubS = kSub * kNB * 4;          // 1 KB
constexpr int kKBytes = kSubK + kSubS;         // K buffer
constexpr int kVShiftOfs = kSubV;              // shifts in the V buffer
constexpr int kVBytes = kVShiftOfs + 16 * kNB; // V buffer
// A sub-block's raw rows for one kv head as the record holds them: 64 K rows
// (136 B each) then 64 V rows, moved by 1 KB LDS DMA pieces.
template <typename VT>
struct RawSub {
    static constexpr int kK = kSub * kKRow;                  // 8704 B
    static constexpr int kBytes = kK + kSub * VT::kRow;      // 13312 (Q4_0 V) / 17408 (Q8_0 V)
    static constexpr int kPieces = kBytes / 1024;
    static constexpr int kWavePieces = (kPieces + kPWaves - 1) / kPWaves;   // DMA instructions per wave
    static_assert(kBytes % 1024 == 0 && kK % 16 == 0, "raw sub-block is whole 1 KB pieces");
};
constexpr float kLazyMax = 8.f;

// s_waitcnt immediate: vmcnt(n) (6 bits, split over bits 3:0 and 15:14), the
// other counters not waited on
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Issue this wave's share of the LDS DMA of raw sub-block sb of kv head g of
// page record rec into dst: byte o of [K rows | V rows] comes from the K tile
// (o < 8704) or the V tile, in 16-byte lane pieces.
// Every wave issues exactly kWavePieces instructions (a wave past the last
// piece copies the last piece again, the same bytes to the same place), so
// the code has no branch and the count of DMAs in flight is fixed. The
// source addresses are returned so that the caller can keep their registers
// from being rewritten while the DMAs are in flight (the compiler would
// otherwise wait for the DMAs before reusing them).
template <typename VT>
struct DmaAddr {
    const uint8_t* src[RawSub<VT>::kWavePieces];
};
template <typename VT>
__device__ inline DmaAddr<VT> dma_raw(const uint8_t* rec, int g, int n_kv_heads, int sb, uint8_t* dst, int w, int lane) {
    const uint8_t* kt = rec + (int64_t)g * kKTile + sb * RawSub<VT>::kK;
    const uint8_t* vt = rec + (int64_t)n_kv_heads * kKTile + (int64_t)g * VT::kTile + sb * kSub * VT::kRow;
    DmaAddr<VT> ad;
#pragma unroll
    for (int k = 0; k < RawSub<VT>::kWavePieces; ++k) {
        const int p = min(w + kPWaves * k, RawSub<VT>::kPieces - 1);
        const int o = 1024 * p + 16 * lane;
        ad.src[k] = o < RawSub<VT>::kK ? kt + o : vt + (o - RawSub<VT>::kK);
        dma16(ad.src[k], dst + 1024 * p);
    }
    return ad;
}
template <typename VT>
__device__ inline void keep(const DmaAddr<VT>& ad) {
#pragma unroll
    for (int k = 0; k < RawSub<VT>::kWavePieces; ++k) asm volatile("" ::"v"(ad.src[k]));
}

// Convert a raw sub-block (LDS rw) into its operands (LDS kc, vc), with the
// conversion code of the other matrix-core paths (kvs_convert.h); `valid`
// rows of the sub-block are cached. Wave w converts K fragments (tile, block)
// = (w >> 2, w & 3) and (2 + (w >> 2), w & 3), their block scales, and V^T
// chunk w >> 2 of block w & 3. The code has no branch.
template <typename VT>
__device__ inline void convert_sub(const uint8_t* rw, uint8_t* kc, uint8_t* vc, int valid, int tid, int w, int lane,
                                   uint32_t m_nib, uint32_t magic) {
    const int n = lane & 15, gq = lane >> 4, b = w & 3, c = w >> 2;
    // The lane's 8 codes start at byte 34 b + 2 + 8 gq of its token's row:
    // three dwords from the dword holding that byte, shifted by 2 bytes for
    // an even block (the same codes k_codes takes; for the last block the
    // third dword lies past the row, inside the buffer, and is not used).
    // Lane offsets are made opaque so that the compiler forms each address
    // here instead of holding one per buffer across the caller's loop.
    const int kofs = kKBlock * b + 2 + 8 * gq, ksh = kofs & 3;
    // Scales: lane l of wave w takes the four block scales of token
    // 8 w + (l & 7) (eight lanes write the same 16 bytes, so the code has no
    // branch). Every LDS access here is a whole dword or wider.
    const int stok = 8 * w + (lane & 7);
    uint32_t ko = n * kKRow + (kofs - ksh), so = stok * kKRow, oo = lane * 16;
    const int vsh_b = (VT::kBlock * b) & 3;   // block b starts 0 or 2 bytes into a dword
    uint32_t vo = RawSub<VT>::kK + b * VT::kBlock - vsh_b + 4 * gq * VT::kRow, st16 = 16 * stok;
    uint32_t vdo = (c * 8 + 2 * b) * 1024 + lane * 16;   // the lane's two V^T fragment stores
    asm volatile("" : "+v"(ko), "+v"(so), "+v"(oo), "+v"(vo), "+v"(st16), "+v"(vdo));
    // Every LDS read of the conversion is issued first, so that one wait
    // covers them all (a read, its wait and its use per piece would make the
    // conversion a chain of LDS round trips). The K codes: three dwords per
    // fragment. The row's block scales: blocks 0, 1 in dword 0 and dword 8
    // (byte 34 = 32 + 2), blocks 2, 3 in dword 17 and dword 25 (byte 102).
    // Block b's V rows as whole dwords: an even block starts on a dword
    // boundary (its scale is the dword's low half), an odd one 2 bytes into
    // one (the high half); byte n of the codes follows 2 bytes after the
    // scale. The V shift of block b (v_shift_of over 64 rows, on the same
    // scale bits) takes the scale of row `lane`.
    uint32_t kx[2][3];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int f = w + 8 * k;   // (tile, block) = (f >> 2, b)
        const uint32_t* p = (const uint32_t*)(rw + 16 * (f >> 2) * kKRow + ko);
        kx[k][0] = p[0];
        kx[k][1] = p[1];
        kx[k][2] = p[2];
    }
    const uint32_t* rp = (const uint32_t*)(rw + so);
    const uint32_t d0 = rp[0], d1 = rp[8], d2 = rp[17], d3 = rp[25];
    uint32_t vs = RawSub<VT>::kK + lane * VT::kRow + VT::kBlock * b - vsh_b;
    asm volatile("" : "+v"(vs));
    const uint32_t w0 = *(const uint32_t*)(rw + vs);
    const uint32_t cb = (uint32_t)(2 + vsh_b + n);   // byte of code n from a row's first dword
    uint32_t rs[8], rb[8], rh[VT::kQ8 ? 8 : 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t* rd = (const uint32_t*)(rw + vo + (32 * c + (j < 4 ? j : 12 + j)) * VT::kRow);
        rs[j] = rd[0];
        rb[j] = rd[cb >> 2];
        if constexpr (VT::kQ8) rh[j] = rd[(cb + 16) >> 2];
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- the operands
#pragma unroll
    for (int k = 0; k < 2; ++k)
        *(half8_t*)(kc + (w + 8 * k) * 1024 + oo) = q8_codes_f16(__builtin_amdgcn_alignbyte(kx[k][1], kx[k][0], ksh),
                                                                  __builtin_amdgcn_alignbyte(kx[k][2], kx[k][1], ksh));
    *(f32x4*)(kc + kSubK + st16) = f32x4{scale_f32(d0), scale_f32(d1 >> 16), scale_f32(d2), scale_f32(d3 >> 16)};
    // every lane of the two waves of block b writes the shift
    const uint32_t sbits = (vsh_b ? w0 >> 16 : w0) & 0x7FFFu;
    const int vsh = __any(lane < valid && sbits > (VT::kQ8 ? kVBigBits8 : kVBigBits)) ? (VT::kQ8 ? kVShift8 : kVShift) : 0;
    *(int4v*)(vc + kVShiftOfs + 16 * b) = int4v{vsh, vsh, vsh, vsh};
    // the V rows as v_raw (kvs_convert.h) gives them
    VRaw<VT> vr;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        vr.d[j] = vsh_b ? rs[j] >> 16 : rs[j] & 0xFFFFu;
        vr.byte[j] = (rb[j] >> (8 * (cb & 3))) & 0xFFu;
        if constexpr (VT::kQ8) vr.hbyte[j] = (rh[j] >> (8 * ((cb + 16) & 3))) & 0xFFu;
    }
    half8_t vop[2];
    if (valid >= kSub)   // every row cached (all but the cache's last sub-block): no row mask
        v_convert<false, VT>(vr, c, gq, valid, vsh, m_nib, magic, vop);
    else
        v_convert<true, VT>(vr, c, gq, valid, vsh, m_nib, magic, vop);
    *(half8_t*)(vc + vdo) = vop[0];
    *(half8_t*)(vc + vdo + 1024) = vop[1];
}

template <int LIMBS, typename VT>
__global__ __launch_bounds__(kPThreads, 1) void prefill_kernel(AttendArgs a) {
    // Two K operand buffers (the sub-block whose scores are computed and the
    // next one being converted), three V operand buffers (those two and the
    // previous sub-block, whose P.V is computed in the same step) and four
    // raw buffers (the one being converted and DMAs in flight). Each raw
    // buffer is its own LDS array: the compiler then orders a read of one
    // array only after the DMA into that array, not after DMAs still in
    // flight into the others.
    __shared__ __attribute__((aligned(16))) uint8_t kc0[kKBytes];
    __shared__ __attribute__((aligned(16))) uint8_t kc1[kKBytes];
    __shared__ __attribute__((aligned(16))) uint8_t vcs[3 * kVBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rw0[RawSub<VT>::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rw1[RawSub<VT>::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rw2[RawSub<VT>::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rw3[RawSub<VT>::kBytes];
    // 1-D grid: ring refill workgroups first, then one worker per (segment,
    // kv head, row block), row blocks of one (segment, kv head) consecutive.
    // Workgroups go to the 8 XCDs round-robin by linear index; workers are
    // permuted so that each XCD takes a contiguous range, and the row blocks
    // of one (segment, kv head), which read the same pages, share an XCD's
    // L2.
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
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;
    const int r0 = rb * kRowsWG + 16 * kRTW * w;   // this wave's first row

    const int4v segv = scalar_load((const int4v*)(a.segs + seg_i));
    const Seg seg = {segv.x, segv.y, segv.z, segv.w};
    const int n_steps = seg.npages * kSubs;
    // the record of the segment's page pi, by selects (no branch)
    auto record = [&](int pi) {
        const int32_t page = seg.page0 + pi;
        const int32_t sv = scalar_load(a.ps.src + page);
        const uint8_t* res = a.ps.slots + (int64_t)sv * a.ps.page_bytes;
        const uint8_t* str = a.ps.host ? a.ps.host + (int64_t)page * a.ps.page_bytes
                                       : a.ps.ring_chunk + (int64_t)((-1 - sv) - a.ps.chunk_rank0) * a.ps.page_bytes;
        return sv >= 0 ? res : str;
    };
    auto dma_step = [&](int st, uint8_t* dst) {
        return dma_raw<VT>(record(st / kSubs), g, a.n_kv_heads, st % kSubs, dst, w, lane);
    };
    // cached rows of sub-block st
    auto valid_of = [&](int st) {
        const int64_t x = a.n_kv - ((int64_t)(seg.page0 + st / kSubs) * kPageTokens + kSub * (st % kSubs));
        return (int)(x < 0 ? 0 : (x > kSub ? kSub : x));
    };

    // ---- this lane's query rows and their visible prefix, counted from the
    // segment's first token (clamped to the segment)
    const int64_t seg_tok = (int64_t)seg.page0 * kPageTokens;
    const int seg_len = n_steps * kSub;
    auto rel = [&](int64_t t) { const int64_t x = t - seg_tok; return (int)(x < 0 ? 0 : (x > seg_len ? seg_len : x)); };
    half8_t qop[kRTW][LIMBS][kNB];
    float cq[kRTW];
    int lim[kRTW];
    int qi_[kRTW], h_[kRTW];
#pragma unroll
    for (int rt = 0; rt < kRTW; ++rt) {
        const int r = r0 + 16 * rt + n;
        qi_[rt] = r / G;
        h_[rt] = g * G + r % G;
        lim[rt] = 0;
        if (r < R) {
            int64_t l = a.n_kv;
            if (a.causal) {
                const int64_t c = a.q_pos0 + qi_[rt] + 1;
                l = c < l ? c : l;
            }
            lim[rt] = rel(l);
        }
        query_operands<LIMBS>(a, qi_[rt], h_[rt], r < R, gq, qop[rt], cq[rt]);
    }
    // smallest visible prefix of the wave's rows: sub-blocks below it need no mask
    int64_t lim_min = a.n_kv;
    if (a.causal) {
        const int64_t c = a.q_pos0 + r0 / G + 1;
        lim_min = c < lim_min ? c : lim_min;
    }
    const int lim_min_rel = rel(lim_min);

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
    const uint32_t m_nib = vconst(0x000F000Fu), magic = vconst(0x64006400u);
    // The first raw sub-blocks' DMAs go out after the query and state loads,
    // so that the wait for the first sub-block also covers every load into
    // registers (loads complete in order): no register of the loop below then
    // waits on a load.
    dma_step(0, rw0);
    dma_step(min(1, n_steps - 1), rw1);
    dma_step(min(2, n_steps - 1), rw2);

    // ---- scores of sub-block st from its K operands in KB, and from them
    // the P^T operands pp (relative to the running max after the sub-block)
    // and the factor alpha by which the state is to be rescaled when the
    // running max moved (rescale)
    auto scores = [&](int st, const uint8_t* KB, f32x4 (&s)[4][kRTW], float (&m_use)[kRTW], float (&alpha)[kRTW],
                      bool& rescale) {
        const int base_tok = kSub * st;                     // from the segment's first token
        const bool mask_sub = base_tok + kSub > lim_min_rel;   // wave-uniform

        // ---- QK (float32 products; cq * s is the log2-unit score)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4 acc[kRTW][kNB];
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                const half8_t kop = *(const half8_t*)(KB + ((tt * kNB + b) * 64 + lane) * 16);
#pragma unroll
                for (int rt = 0; rt < kRTW; ++rt) {
                    acc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[rt][0][b], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if constexpr (LIMBS == 2)
                        acc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[rt][1][b], acc[rt][b], 0, 0, 0);
                }
            }
            // scales of the lane's four tokens 16 tt + 4 gq + i: [i][b] float32
            const f32x4* sc = (const f32x4*)(KB + kSubK + (16 * tt + 4 * gq) * kNB * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 d = sc[i];
#pragma unroll
                for (int rt = 0; rt < kRTW; ++rt) {
#pragma clang fp contract(off)
                    float t = acc[rt][0][i] * d[0];
                    t = __builtin_fmaf(acc[rt][1][i], d[1], t);
                    t = __builtin_fmaf(acc[rt][2][i], d[2], t);
                    s[tt][rt][i] = __builtin_fmaf(acc[rt][3][i], d[3], t);
                }
            }
            // one token tile's products at a time (bounds the registers the
            // scheduler may spend on products in flight)
            __builtin_amdgcn_sched_barrier(0);
        }
        if (mask_sub) {
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt) {
                // token 16 tt + 4 gq + i is visible when 16 tt + i < lg
                // (compared with immediates: no per-token index registers)
                const int x = lim[rt] - base_tok;
                const int lg = (x < 0 ? 0 : (x > kSub ? kSub : x)) - 4 * gq;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[tt][rt][i] = 16 * tt + i < lg ? s[tt][rt][i] : -INFINITY;
            }
        }

        // ---- softmax over the sub-block
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
        __builtin_amdgcn_sched_barrier(0);
    };
    // P^T operands from the scores: chunk c's slot j of lane group gq is
    // token 32 c + 4 gq + j (j < 4, tile 2 c) or 32 c + 12 + 4 gq + j (j >= 4,
    // tile 2 c + 1); exps(k) gives slots 2 (k & 3) and 2 (k & 3) + 1 of chunk
    // (k >> 2) & 1 of row tile k >> 3
    // (the pair is pinned where it is computed: an empty volatile asm takes
    // it, so the compiler cannot sink the arithmetic to the pair's use)
    auto exps = [&](int k, const f32x4 (&s)[4][kRTW], const float (&m_use)[kRTW], half8_t (&pp)[2][kRTW]) {
        const int rt = k >> 3, c = (k >> 2) & 1, j0 = 2 * (k & 3);
        half2_t h;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            h[j] = (_Float16)__builtin_amdgcn_exp2f(
                __builtin_fmaf(s[2 * c + ((j0 + j) >> 2)][rt][(j0 + j) & 3], cq[rt], -m_use[rt]));
        asm volatile("" : "+v"(h));
        pp[c][rt][j0] = h[0];
        pp[c][rt][j0 + 1] = h[1];
    };
    // ---- the state rescaled when the running max moved
    auto apply_alpha = [&](const float (&alpha)[kRTW], bool rescale) {
        if (__any(rescale)) {
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt) {
                lsum[rt] *= alpha[rt];
#pragma unroll
                for (int ct = 0; ct < 8; ++ct) o[ct][rt] *= alpha[rt];
            }
        }
    };
    // ---- the V shifts of the sub-block in VB: an exact rescale of a
    // block's accumulators when its shift changes
    auto v_shifts = [&](const uint8_t* VB) {
        int vshs[kNB];   // all four reads before the first use
#pragma unroll
        for (int b = 0; b < kNB; ++b) vshs[b] = *(const int32_t*)(VB + kVShiftOfs + 16 * b);
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            const int vsh = __builtin_amdgcn_readfirstlane(vshs[b]);
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
    };
    // ---- P.V of the sub-block in VB with its P^T operands pp, and the row
    // sums on a tile of ones
    auto pv = [&](const uint8_t* VB, const half8_t (&pp)[2][kRTW]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const half8_t vop = *(const half8_t*)(VB + ((c * 8 + ct) * 64 + lane) * 16);
#pragma unroll
                for (int rt = 0; rt < kRTW; ++rt)
                    o[ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pp[c][rt], o[ct][rt], 0, 0, 0);
            }
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt)
                lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pp[c][rt], lsum[rt], 0, 0, 0);
        }
    };

    // ---- pipeline over sub-blocks. Step st: every wave converts sub-block
    // st + 1 (raw rows DMA'd two steps earlier), issues the DMA of st + 3,
    // computes the scores and probabilities of sub-block st and then the P.V
    // of sub-block st - 1, whose matrix instructions do not depend on the
    // scores and so can issue while they are computed. The state sees the
    // same operations in the same order as when each sub-block's P.V follows
    // its own scores: the rescale for st's max comes after st - 1's P.V, the
    // V shift rescale for st just before st's P.V. Past the last sub-block,
    // the DMA and the conversion repeat the last one into free buffers (no
    // branch, so the compiler counts the DMAs in flight exactly); nothing
    // reads them.
    constexpr int kWP = RawSub<VT>::kWavePieces;
    // The waits before the step barriers count this wave's DMAs still allowed
    // in flight. With two query limbs the kernel spills registers, and scratch
    // stores between the DMAs could retire ahead of them: then every vector
    // memory operation is waited for instead.
    constexpr int kWaitOne = LIMBS == 1 ? vm_wait(kWP) : vm_wait(0);
    constexpr int kWaitTwo = LIMBS == 1 ? vm_wait(2 * kWP) : vm_wait(0);
    auto vbuf = [&](int i) { return vcs + i * kVBytes; };   // V buffer of sub-block st: st % 3
    __builtin_amdgcn_s_waitcnt(kWaitTwo);   // raw 0 landed, 1 and 2 may be in flight
    lds_barrier();
    convert_sub<VT>(rw0, kc0, vbuf(0), valid_of(0), tid, w, lane, m_nib, magic);

    // the step's front: raw sub-block st + 1 is in LDS for every wave (a wave
    // may still have the DMA of st + 2 in flight), the operands of st are
    // published, and every wave is done with step st - 1, whose buffers take
    // st + 1 (K and V operands) and st + 3 (raw rows). The DMA of st + 3 is
    // issued after the conversion's LDS accesses: the compiler cannot tell
    // every one of them apart from the DMA's target and would wait for the
    // DMA there; after it, the step reads only operand buffers.
    auto front = [&](int st, int vi, uint8_t* KN, const uint8_t* Rn, uint8_t* D, bool prev) {
        __builtin_amdgcn_s_waitcnt(kWaitOne);
        lds_barrier();
        if (prev) v_shifts(vbuf(vi == 0 ? 2 : vi - 1));
        convert_sub<VT>(Rn, KN, vbuf(vi == 2 ? 0 : vi + 1), valid_of(min(st + 1, n_steps - 1)), tid, w, lane, m_nib, magic);
        const DmaAddr<VT> ad = dma_step(min(st + 3, n_steps - 1), D);
        __builtin_amdgcn_sched_barrier(0);
        return ad;
    };
    // P^T operands of the sub-blocks of even and of odd index: a step reads
    // the previous sub-block's from one and writes its own into the other
    // (the unrolled steps name them statically, so nothing is copied)
    half8_t pb0[2][kRTW], pb1[2][kRTW];
    // step 0: no previous sub-block
    {
        const DmaAddr<VT> ad = front(0, 0, kc1, rw1, rw3, false);
        f32x4 sc[4][kRTW];
        float m_use[kRTW], alpha[kRTW];
        bool rescale = false;
        scores(0, kc0, sc, m_use, alpha, rescale);
#pragma unroll
        for (int k = 0; k < 16; ++k) exps(k, sc, m_use, pb0);
        apply_alpha(alpha, rescale);
        keep<VT>(ad);
    }
    auto do_step = [&](int st, int vi, const uint8_t* KC, uint8_t* KN, const uint8_t* Rn, uint8_t* D,
                       const half8_t (&pprev)[2][kRTW], half8_t (&pc)[2][kRTW]) {
        const DmaAddr<VT> ad = front(st, vi, KN, Rn, D, true);
        f32x4 sc[4][kRTW];
        float m_use[kRTW], alpha[kRTW];
        bool rescale = false;
        scores(st, KC, sc, m_use, alpha, rescale);
        // P.V of sub-block st - 1 (independent of st's scores) in 16 chunks of
        // one channel tile, each followed by two of st's exponentials per row
        // tile, so that the vector unit works while the matrix products run;
        // the V operands are read two chunks ahead
        const uint8_t* VP = vbuf(vi == 0 ? 2 : vi - 1);
        auto vread = [&](int k) { return *(const half8_t*)(VP + (((k >> 3) * 8 + (k & 7)) * 64 + lane) * 16); };
        half8_t vq[3];
        vq[0] = vread(0);
        vq[1] = vread(1);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int c = k >> 3, ct = k & 7;
            if (k + 2 < 16) vq[(k + 2) % 3] = vread(k + 2);
#pragma unroll
            for (int rt = 0; rt < kRTW; ++rt)
                o[ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vq[k % 3], pprev[c][rt], o[ct][rt], 0, 0, 0);
            exps(k, sc, m_use, pc);
            if (ct == 7) {
#pragma unroll
                for (int rt = 0; rt < kRTW; ++rt)
                    lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pprev[c][rt], lsum[rt], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        apply_alpha(alpha, rescale);
        keep<VT>(ad);
    };
    // steps four at a time from step 1, so that each names its raw and K
    // buffers statically; the V buffer index st % 3 is carried along
    int vi = 1;
    auto nx = [](int i) { return i == 2 ? 0 : i + 1; };
    for (int st = 1; st < n_steps; st += 4) {
        do_step(st, vi, kc1, kc0, rw2, rw0, pb0, pb1);
        vi = nx(vi);
        if (st + 1 < n_steps) { do_step(st + 1, vi, kc0, kc1, rw3, rw1, pb1, pb0); vi = nx(vi); }
        if (st + 2 < n_steps) { do_step(st + 2, vi, kc1, kc0, rw0, rw2, pb0, pb1); vi = nx(vi); }
        if (st + 3 < n_steps) { do_step(st + 3, vi, kc0, kc1, rw1, rw3, pb1, pb0); vi = nx(vi); }
    }
    // the last sub-block's P.V (its operands were published before the last
    // step; its P^T operands are in the buffer of its index's parity)
    half8_t plast[2][kRTW];
    const bool last_odd = ((n_steps - 1) & 1) != 0;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rt = 0; rt < kRTW; ++rt) plast[c][rt] = last_odd ? pb1[c][rt] : pb0[c][rt];
    v_shifts(vbuf(vi == 0 ? 2 : vi - 1));
    pv(vbuf(vi == 0 ? 2 : vi - 1), plast);

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

// Operand probe: every (page, kv head) of a launch converted by convert_sub,
// sub-block by sub-block, and written out as one staged tile (the operands
// the prefill kernel computes on, in the layout kvs.h documents). Grid:
// (pages of the launch, kv heads); block x takes the x-th page of the
// launch's segments, in segment order, into tile x (with by_page, into tile
// `page`); blocks past the pages are ring refill workgroups.
template <typename VT>
__global__ __launch_bounds__(kPThreads) void stage_kernel(StageArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t kc[kKBytes];
    __shared__ __attribute__((aligned(16))) uint8_t vc[kVBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rw[RawSub<VT>::kBytes];
    if ((int)blockIdx.x >= a.n_pages) {   // ring refill workgroup: its first 256 threads copy
        if (threadIdx.x < 256) copy_role(a.copy, ((int)blockIdx.x - a.n_pages) * (int)gridDim.y + (int)blockIdx.y);
        return;
    }
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int slot = blockIdx.x, g = blockIdx.y;
    int rem = slot;
    int32_t page = -1;
    for (int si = 0; si < a.n_segs; ++si) {
        const int np = scalar_load(&a.segs[si].npages);
        if (rem < np) { page = scalar_load(&a.segs[si].page0) + rem; break; }
        rem -= np;
    }
    if (page < 0) return;   // past the launch's pages
    const uint8_t* rec = page_record(a.ps, page);
    uint8_t* tile = a.staged + ((int64_t)(a.by_page ? page : slot) * a.n_kv_heads + g) * kStagedTile;
    const uint32_t m_nib = vconst(0x000F000Fu), magic = vconst(0x64006400u);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    for (int sb = 0; sb < kSubs; ++sb) {
        dma_raw<VT>(rec, g, a.n_kv_heads, sb, rw, w, lane);
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
        lds_barrier();   // the raw rows are in LDS for every wave
        const int64_t x = a.n_kv - ((int64_t)page * kPageTokens + kSub * sb);
        convert_sub<VT>(rw, kc, vc, (int)(x < 0 ? 0 : (x > kSub ? kSub : x)), tid, w, lane, m_nib, magic);
        lds_barrier();   // the operands are in LDS for every wave
        for (int o = 16 * tid; o < kSubK; o += 16 * kPThreads) {
            *(u32x4*)(tile + sb * kSubK + o) = *(const u32x4*)(kc + o);
            *(u32x4*)(tile + kStagedK + sb * kSubV + o) = *(const u32x4*)(vc + o);
        }
        if (16 * tid < kSubS) *(u32x4*)(tile + kStagedOps + sb * kSubS + 16 * tid) = *(const u32x4*)(kc + kSubK + 16 * tid);
        if (tid < kNB) *(int32_t*)(tile + kStagedShift + 4 * (kNB * sb + tid)) = *(const int32_t*)(vc + kVShiftOfs + 16 * tid);
        lds_barrier();   // every wave is done with both buffers
    }
}

template <int LIMBS>
hipError_t launch_limbs(const AttendArgs& a, hipStream_t stream) {
    const int R = a.n_q * a.G;
    const int64_t n_work = (int64_t)a.n_segs * a.n_kv_heads * ((R + kRowsWG - 1) / kRowsWG);
    const int64_t blocks = ((copy_workgroups(a.copy) + 7) & ~7) + ((n_work + 7) & ~7);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (a.v_q8) return launch_kernel(prefill_kernel<LIMBS, VQ8>, dim3((unsigned)blocks), dim3(kPThreads), stream, a);
    return launch_kernel(prefill_kernel<LIMBS, VQ4>, dim3((unsigned)blocks), dim3(kPThreads), stream, a);
}

}  // namespace

hipError_t launch_prefill(const AttendArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    return a.q_f16 ? launch_limbs<1>(a, stream) : launch_limbs<2>(a, stream);
}

hipError_t launch_stage(const StageArgs& a, hipStream_t stream) {
    const int cx = (copy_workgroups(a.copy) + a.n_kv_heads - 1) / a.n_kv_heads;
    if (a.n_pages <= 0 && cx == 0) return hipSuccess;
    if (a.v_q8) return launch_kernel(stage_kernel<VQ8>, dim3(a.n_pages + cx, a.n_kv_heads), dim3(kPThreads), stream, a);
    return launch_kernel(stage_kernel<VQ4>, dim3(a.n_pages + cx, a.n_kv_heads), dim3(kPThreads), stream, a);
}

}  // namespace kvs
