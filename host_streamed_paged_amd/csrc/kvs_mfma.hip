// Matrix-core attention kernel for query blocks with more than a few rows:
// a speculative verify batch of 1 + draft tokens (page 2, "Phase arena:
// speculative verify batches") and a prefill ubatch (256 tokens in page 2's
// "TLDR - recommended setup"), on CDNA4 v_mfma_f32_16x16x32_f16.
//
// One workgroup = one segment (run of pages of one split-K group) x one kv
// head x a tile of 16 RT query rows (row = query token x head of the GQA
// group). 4 waves. Every page is staged whole in LDS by LDS DMA (K tile
// 34816 B, V tile 18432 B, record layout); the next page's K tile is fetched
// once every wave is past QK, its V tile once P.V is done. Then:
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
//        The V operand is d * (u - 8) rounded once to f16. A page whose block
//        w holds a scale above 8188 (where d * (u - 8) could exceed the f16
//        range) takes d * (u - 8) / 8 instead; the wave keeps its accumulator
//        in units of 2^shift and rescales it exactly when the shift changes.
// The running state (m, l, O) is updated once per page in page order from
// state and page data alone, so results do not depend on how pages are split
// into launches or which pages are resident.
//
// Staged mode, for blocks of more than 64 rows per kv head (a prefill
// ubatch): every row tile would otherwise decode the same page again, so
// stage_kernel first converts each (page, kv head) of the launch once into a
// tile of f16 matrix-core operands in fragment order (K: [token tile][block]
// [lane] x 16 B; V^T: [32-token chunk][channel tile][lane] x 16 B), the K
// block scales per token and the V shift of each block, with the same code;
// the attention kernel loads whole fragments from it. The operands, and so
// the results, are the same bits either way.
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTokW = kPageTokens / kWaves;   // tokens per wave in QK (64)
constexpr int kChunks = kPageTokens / 32;     // 32-token MFMA chunks per page in PV
// The running max moves only when a page's max exceeds it by more than this
// (log2 units), so p <= 2^8 stays well inside f16 and O is rarely rescaled.
constexpr float kLazyMax = 8.f;
// A V block scale of magnitude above 8188 (binary16 bits 0x6FFF) can make
// d * (u - 8) exceed the largest f16, 65504; such pages take the V operand
// divided by 2^kVShift.
constexpr uint32_t kVBigBits = 0x6FFFu;
constexpr int kVShift = 3;

// One page's tiles. (Double-buffering them measured slower: the next page's
// LDS DMA then competes with the QK reads of the current one.) The P
// operands [chunk][row tile][lane] (16 bytes each) have a region of their
// own, so that the next page's K tile can be fetched into `k` as soon as
// every wave is past QK, during the softmax and P.V of the current page.
// `ksc` holds each wave's K block scales per token ([token][block] f16), the
// layout the score lanes read them in.
template <int RT, bool STAGED>
struct MfmaSmem {
    alignas(16) uint8_t k[kKTile];   // K tile in record layout
    alignas(16) uint8_t v[kVTile];   // V tile in record layout
    alignas(16) uint8_t p[kChunks * RT * 64 * 16];
    alignas(16) uint32_t ksc[kWaves][kTokW * 2];
    float red_m[kWaves][16 * RT];
    float red_l[kWaves][16 * RT];
};
template <int RT>
struct MfmaSmem<RT, true> {
    alignas(16) uint8_t k[kChunks * RT * 64 * 16];   // P operands only
    float red_m[kWaves][16 * RT];
    float red_l[kWaves][16 * RT];
};

constexpr int kStagedK = kPageTokens * kHeadDim * 2;   // f16 K operands of one (page, kv head)
static_assert(2 * kStagedK == kStagedOps, "staged operands = K + V^T");
constexpr int kStagedShift = kStagedOps + kStagedScaleBytes;   // int32 V shift per block

template <int RT>
__device__ inline uint8_t* sm_p(MfmaSmem<RT, false>& sm) { return sm.p; }
template <int RT>
__device__ inline uint8_t* sm_p(MfmaSmem<RT, true>& sm) { return sm.k; }

// Stage one (page, kv head) tile of a page record into LDS by LDS DMA:
// wave-sized pieces of 1 KB, 34 for K and 18 for V.
__device__ inline void dma_k_tile(const uint8_t* rec, int g, uint8_t* k_lds, int w, int lane) {
    const uint8_t* kt = rec + (int64_t)g * kKTile;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int piece = w + 4 * k;
        if (piece < kKTile / 1024) dma16(kt + piece * 1024 + lane * 16, k_lds + piece * 1024);
    }
}
__device__ inline void dma_v_tile(const uint8_t* rec, int g, int n_kv_heads, uint8_t* v_lds, int w, int lane) {
    const uint8_t* vt = rec + (int64_t)n_kv_heads * kKTile + (int64_t)g * kVTile;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const int piece = w + 4 * k;
        if (piece < kVTile / 1024) dma16(vt + piece * 1024 + lane * 16, v_lds + piece * 1024);
    }
}

// K operand of v_mfma_f32_16x16x32_f16 for A_b^T = K_b . Q_b^T: this lane's 8
// codes [32 b + 8 gq, +8) of token `tok` of the K tile (record layout, in
// LDS) as exact f16, and the block's scale bits. Split into the LDS reads
// (k_raw) and the conversion (k_codes) so that a caller can read the next
// fragments while converting the current ones.
struct KRaw {
    uint32_t x0, x1, x2;   // 3 aligned dwords (even blocks) or 2 (odd blocks)
    uint32_t db;           // scale bits
};
__device__ inline KRaw k_raw(const uint8_t* k_lds, int tok, int b, int gq) {
    const uint8_t* blk = k_lds + tok * kKRow + b * kKBlock;
    KRaw r;
    if (b & 1) {   // codes start on a dword boundary
        const uint32_t* p = (const uint32_t*)(blk + 2 + 8 * gq);
        r.x0 = p[0];
        r.x1 = p[1];
        r.x2 = 0u;
    } else {       // codes start 2 bytes into a dword
        const uint32_t* p = (const uint32_t*)(blk + 8 * gq);
        r.x0 = p[0];
        r.x1 = p[1];
        r.x2 = p[2];
    }
    r.db = *(const uint16_t*)blk;
    return r;
}
__device__ inline half8_t k_codes(const KRaw& r, int b) {
    if (b & 1) return q8_codes_f16(r.x0, r.x1);
    return q8_codes_f16(__builtin_amdgcn_alignbyte(r.x1, r.x0, 2), __builtin_amdgcn_alignbyte(r.x2, r.x1, 2));
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

// V shift of quant block b of a page (V tile in LDS, record layout): kVShift
// if a cached row's scale magnitude exceeds 8188, else 0. Rows at or past
// `valid` are not cached and may hold any bytes. Wave-uniform.
__device__ inline int v_shift_of(const uint8_t* v_lds, int b, int valid, int lane) {
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = lane + 64 * j;
        const uint32_t bits = *(const uint16_t*)(v_lds + t * kVRow + b * kVBlock) & 0x7FFFu;
        mx = (t < valid && bits > mx) ? bits : mx;
    }
    return __any(mx > kVBigBits) ? kVShift : 0;
}

// V^T operands of O^T += V^T . P^T for chunk c (tokens [32 c, 32 c + 32)) and
// quant block b: vop[0] holds channel 32 b + n, vop[1] channel 32 b + 16 + n
// (low and high nibbles of byte n), for the lane's 8 token slots: slot j of
// lane group gq is token 32 c + 4 gq + j for j < 4, else 32 c + 12 + 4 gq + j.
// Each value is d * (u - 8) / 2^vshift rounded once to f16 ((u - 8) / 2^vshift
// is exact, and the product of two f16 values is rounded once). TAIL zeroes
// rows at or past `valid` (their scales may be NaN). Split into the LDS reads
// (v_raw) and the arithmetic (v_convert), like the K operand.
struct VRaw {
    uint32_t byte[8];   // nibble byte n of the slot's token
    uint32_t d[8];      // scale bits of the slot's token
};
__device__ inline VRaw v_raw(const uint8_t* v_lds, int b, int c, int gq, int n) {
    const uint8_t* vlane = v_lds + b * kVBlock + 4 * gq * kVRow;
    VRaw r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint8_t* row = vlane + (32 * c + (j < 4 ? j : 12 + j)) * kVRow;
        r.byte[j] = row[2 + n];
        r.d[j] = *(const uint16_t*)row;
    }
    return r;
}
template <bool TAIL>
__device__ inline void v_convert(const VRaw& r, int c, int gq, int valid, int vshift, uint32_t m_nib, uint32_t magic,
                                 half8_t (&vop)[2]) {
    const _Float16 cs = vshift ? (_Float16)0.125f : (_Float16)1.f;
    const half2_t cc = {cs, cs};
    const half2_t off = {(_Float16)-1032.f * cs, (_Float16)-1032.f * cs};
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) {
        const int j0 = 2 * jp, j1 = 2 * jp + 1;
        uint32_t d0 = r.d[j0], d1 = r.d[j1];
        if constexpr (TAIL) {
            const int o0 = 32 * c + (j0 < 4 ? j0 : 12 + j0), o1 = 32 * c + (j1 < 4 ? j1 : 12 + j1);
            d0 = o0 + 4 * gq < valid ? d0 : 0u;
            d1 = o1 + 4 * gq < valid ? d1 : 0u;
        }
        const half2_t dd = as_h2(d0 | (d1 << 16));
        const uint32_t x = __builtin_amdgcn_perm(r.byte[j1], r.byte[j0], 0x0c040c00u);
        const half2_t lo = q4_nibbles_f16((x & m_nib) | magic, cc, off) * dd;          // channel n
        const half2_t hi = q4_nibbles_f16(((x >> 4) & m_nib) | magic, cc, off) * dd;   // channel 16 + n
        vop[0][j0] = lo[0]; vop[0][j1] = lo[1];
        vop[1][j0] = hi[0]; vop[1][j1] = hi[1];
    }
}

// Offsets of the staged operands of one (page, kv head) tile.
__device__ inline int staged_k_offset(int tt16, int b, int lane) { return ((tt16 * kNB + b) * 64 + lane) * 16; }
__device__ inline int staged_v_offset(int c, int ct, int lane) { return kStagedK + ((c * 8 + ct) * 64 + lane) * 16; }
__device__ inline int staged_scale_offset(int tok) { return kStagedOps + tok * 8; }

// Position of this launch's segment `seg_i` in the staged tiles: pages of the
// launch's segments are staged in order.
__device__ inline int staged_first_tile(const Seg* segs, int seg_i) {
    int t = 0;
    for (int i = 0; i < seg_i; ++i) t += scalar_load(&segs[i].npages);
    return t;
}

// Workgroups per CU the register budget is cut for: up to 2 row tiles,
// KVS_MFMA_OCC_NARROW; staged launches keep one workgroup per CU.
#ifndef KVS_MFMA_OCC_NARROW
#define KVS_MFMA_OCC_NARROW 2
#endif
#ifndef KVS_MFMA_OCC_STAGED
#define KVS_MFMA_OCC_STAGED 1
#endif
template <int RT, bool STAGED, int LIMBS>
__global__ __launch_bounds__(kThreads, STAGED ? KVS_MFMA_OCC_STAGED : KVS_MFMA_OCC_NARROW)
void mfma_kernel(AttendArgs a) {
    static_assert(kChunks * RT * 64 * 16 <= kKTile, "P operands must fit in the K tile");
    __shared__ MfmaSmem<RT, STAGED> sm;
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

    auto issue_page = [&](int page) {
        if constexpr (!STAGED) {
            const uint8_t* rec = page_record(a.ps, page);
            dma_k_tile(rec, g, sm.k, w, lane);
            dma_v_tile(rec, g, a.n_kv_heads, sm.v, w, lane);
        }
    };
    issue_page(scalar_load(&a.segs[slice].page0));
    // staged operands of the current segment's first page, for kv head g
    const uint8_t* stile = nullptr;
    // staged operands are software-pipelined through registers: the K
    // fragments (and block scales) of page p + 1 are loaded while page p
    // computes P.V, and the V fragments of page p run a few 32-token chunks
    // ahead of their use
    const int64_t tile_step = (int64_t)a.n_kv_heads * kStagedTile;
    half8_t kf[STAGED ? 4 : 1][kNB], vf[STAGED ? kChunks : 1][2];
    u32x4 ks[STAGED ? 4 : 1][2];
    constexpr int kKAhead = 2;   // token tiles of the next page loaded during P.V
    auto load_k = [&](const uint8_t* pt, int tt0, int tt1) {
        if constexpr (STAGED) {
#pragma unroll
            for (int tt = tt0; tt < tt1; ++tt) {
#pragma unroll
                for (int b = 0; b < kNB; ++b) kf[tt][b] = *(const half8_t*)(pt + staged_k_offset(4 * w + tt, b, lane));
                const u32x4* sp = (const u32x4*)(pt + staged_scale_offset(kTokW * w + 16 * tt + 4 * gq));
                ks[tt][0] = sp[0];
                ks[tt][1] = sp[1];
            }
        }
    };
    constexpr int kVAhead = 4;   // V chunks in flight ahead of the one consumed
    auto load_v = [&](const uint8_t* pt, int c) {
        if constexpr (STAGED) {
            vf[c][0] = *(const half8_t*)(pt + staged_v_offset(c, 2 * w, lane));
            vf[c][1] = *(const half8_t*)(pt + staged_v_offset(c, 2 * w + 1, lane));
        }
    };

    // a staged worker takes one segment: fetch its first K fragments before
    // the query operands are built
    if constexpr (STAGED) {
        stile = a.staged + ((int64_t)staged_first_tile(a.segs, slice) * a.n_kv_heads + g) * kStagedTile;
        load_k(stile, 0, kKAhead);
    }

    // ---- this lane's query rows (one per row tile) and their visible prefix.
    // Each row is scaled by a power of two that puts its largest magnitude in
    // [2^14, 2^15), then split into f16 limbs: q' = hi + lo exactly enough
    // (hi = f16(q'), lo = f16(q' - hi)); f16 queries need only hi. The row's
    // score factor cq = scale * log2(e) / 2^shift undoes the scaling in f32.
    half8_t qop[RT][LIMBS][kNB];
    float cq[RT];
    int64_t lim[RT];
    int qi_[RT], h_[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = r0 + 16 * rt + n;
        qi_[rt] = r / G;
        h_[rt] = g * G + r % G;
        float x[kNB][8];
        lim[rt] = 0;
        if (r < R) {
            lim[rt] = a.n_kv;
            if (a.causal) {
                const int64_t c = a.q_pos0 + qi_[rt] + 1;
                lim[rt] = c < lim[rt] ? c : lim[rt];
            }
            const int64_t off = ((int64_t)qi_[rt] * a.n_q_heads + h_[rt]) * kHeadDim + 8 * gq;
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                if (a.q_f16) {
                    const u32x4 raw = *(const u32x4*)((const _Float16*)a.q + off + kQK * b);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const half2_t hv = as_h2(raw[e]);
                        x[b][2 * e] = (float)hv[0];
                        x[b][2 * e + 1] = (float)hv[1];
                    }
                } else {
                    const f32x4* qp = (const f32x4*)((const float*)a.q + off + kQK * b);
                    const f32x4 u0 = qp[0], u1 = qp[1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) { x[b][e] = u0[e]; x[b][4 + e] = u1[e]; }
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < kNB; ++b)
#pragma unroll
                for (int e = 0; e < 8; ++e) x[b][e] = 0.f;
        }
        float amax = 0.f;
#pragma unroll
        for (int b = 0; b < kNB; ++b)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[b][e]));
        amax = max_xor16(amax);   // over the row's four lanes n, n + 16, n + 32, n + 48
        amax = max_xor32(amax);
        const int ex = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 0;   // amax = m 2^ex, m in [0.5, 1)
        const float up = __builtin_amdgcn_ldexpf(1.f, 15 - ex);
        cq[rt] = a.scale_log2 * __builtin_amdgcn_ldexpf(1.f, ex - 15);
#pragma unroll
        for (int b = 0; b < kNB; ++b)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y = x[b][e] * up;   // exact
                const _Float16 hi = (_Float16)y;
                qop[rt][0][b][e] = hi;
                if constexpr (LIMBS == 2) qop[rt][LIMBS - 1][b][e] = (_Float16)(y - (float)hi);
            }
    }

    const uint32_t m_nib = vconst(0x000F000Fu), magic = vconst(0x64006400u);

    // smallest visible prefix over the workgroup's rows (causal limits grow
    // with the query index): pages below it need no mask
    int64_t lim_min = a.n_kv;
    if (a.causal) {
        const int64_t c = a.q_pos0 + r0 / G + 1;
        lim_min = c < lim_min ? c : lim_min;
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

    for (int pi = 0; pi < seg.npages; ++pi) {
        const int page = seg.page0 + pi;
        const int64_t base_tok = (int64_t)page * kPageTokens;
        const bool mask_page = base_tok + kPageTokens > lim_min;   // uniform
        const bool tail_page = base_tok + kPageTokens > a.n_kv;    // rows past the cache
        int limrel[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int64_t x = lim[rt] - base_tok;
            limrel[rt] = (int)(x < 0 ? 0 : (x > kPageTokens ? kPageTokens : x));
        }
        const int64_t vx = a.n_kv - base_tok;
        const int valid = (int)(vx < 0 ? 0 : (vx > kPageTokens ? kPageTokens : vx));   // cached rows of the page
        // the worker's next page (this segment's next, else the first of its
        // next segment), whose tiles are fetched while this page finishes
        const uint8_t* next_rec = nullptr;
        if constexpr (!STAGED) {
            if (pi + 1 < seg.npages) next_rec = page_record(a.ps, page + 1);
            else if (seg_i + a.n_slices < a.n_segs) next_rec = page_record(a.ps, scalar_load(&a.segs[seg_i + a.n_slices].page0));
        }

        if constexpr (!STAGED) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();   // the page's tiles are in LDS for every wave
        }
        if constexpr (STAGED) {
            load_k(stile + pi * tile_step, kKAhead, 4);
#pragma unroll
            for (int c = 0; c < kVAhead; ++c) load_v(stile + pi * tile_step, c);
        }

        // ---- QK over this wave's 64 tokens, one product per quant block (the
        // in-kernel conversion reads the next token tile's K bytes while
        // converting the current one, and publishes each tile's block scales
        // per token for the score lanes)
        f32x4 s[4][RT];
        KRaw kr[2][STAGED ? 1 : kNB];
        if constexpr (!STAGED) {
#pragma unroll
            for (int b = 0; b < kNB; ++b) kr[0][b] = k_raw(sm.k, kTokW * w + n, b, gq);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            u32x4 sa, sb;
            if constexpr (!STAGED) {
                if (gq == 0) {
                    const KRaw* k = kr[tt & 1];
                    *(uint2*)&sm.ksc[w][(16 * tt + n) * 2] =
                        make_uint2(k[0].db | (k[1].db << 16), k[2].db | (k[3].db << 16));
                }
                // written by this wave just above: the wave's own LDS
                // operations complete in order
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const u32x4* sp = (const u32x4*)&sm.ksc[w][(16 * tt + 4 * gq) * 2];
                sa = sp[0];
                sb = sp[1];
                if (tt + 1 < 4) {
#pragma unroll
                    for (int b = 0; b < kNB; ++b) kr[(tt + 1) & 1][b] = k_raw(sm.k, kTokW * w + 16 * (tt + 1) + n, b, gq);
                }
            } else {
                sa = ks[tt][0];
                sb = ks[tt][1];
            }
            float dsc[4][kNB];
            tile_scales(sa, sb, dsc);
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                half8_t kop;
                if constexpr (STAGED)
                    kop = kf[tt][b];
                else
                    kop = k_codes(kr[tt & 1][b], b);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[rt][0][b], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if constexpr (LIMBS == 2) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[rt][1][b], acc, 0, 0, 0);
                    add_block(s[tt][rt], acc, dsc, b);
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) s[tt][rt] *= cq[rt];
        }

        // ---- mask, page maxima (lane value i is token 64 w + 16 tt + 4 gq + i)
        if (mask_page) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tok = kTokW * w + 16 * tt + 4 * gq + i;
                        s[tt][rt][i] = tok < limrel[rt] ? s[tt][rt][i] : -INFINITY;
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
            if (gq == 0) sm.red_m[w][16 * rt + n] = mx[rt];
        }
        lds_barrier();   // maxima published; every wave is done reading the K tile
        if constexpr (!STAGED) {
            if (next_rec) dma_k_tile(next_rec, g, sm.k, w, lane);   // lands during softmax and P.V
        }

        float m_use[RT], alpha[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float pm = sm.red_m[0][16 * rt + n];
#pragma unroll
            for (int ww = 1; ww < kWaves; ++ww) pm = fmaxf(pm, sm.red_m[ww][16 * rt + n]);
            // pm > -inf + 8 holds for any finite pm: the first visible page sets m
            const bool grow = pm > m_run[rt] + kLazyMax;
            alpha[rt] = grow ? __builtin_amdgcn_exp2f(m_run[rt] - pm) : 1.f;   // 0 while the state is empty
            m_run[rt] = grow ? pm : m_run[rt];
            m_use[rt] = m_run[rt] == -INFINITY ? 0.f : m_run[rt];
        }
        // ---- probabilities -> P operands in LDS (slot 8 gq + j of chunk c is
        // token 32 c + 4 gq + j for j < 4, 32 c + 12 + 4 gq + j otherwise)
        uint8_t* pbuf = STAGED ? sm.k : sm_p(sm);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float ls = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                half8_t pv;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float p = __builtin_amdgcn_exp2f(s[2 * c2 + (j >> 2)][rt][j & 3] - m_use[rt]);
                    ls += p;
                    pv[j] = (_Float16)p;
                }
                *(half8_t*)(pbuf + (((2 * w + c2) * RT + rt) * 64 + lane) * 16) = pv;
            }
            ls = add_xor16(ls);
            ls = add_xor32(ls);
            if (gq == 0) sm.red_l[w][16 * rt + n] = ls;
        }
        lds_barrier();   // P operands and row sums published

        bool rescale = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float lp = sm.red_l[0][16 * rt + n];
#pragma unroll
            for (int ww = 1; ww < kWaves; ++ww) lp += sm.red_l[ww][16 * rt + n];
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
        int vsh;
        if constexpr (STAGED)
            vsh = scalar_load((const int32_t*)(stile + pi * tile_step + kStagedShift) + w);
        else
            vsh = v_shift_of(sm.v, w, valid, lane);
        if (vsh != vsh_run) {
            const float f = __builtin_amdgcn_ldexpf(1.f, vsh_run - vsh);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) o[ct][rt] *= f;
            vsh_run = vsh;
        }

        if constexpr (STAGED) {
            if (pi + 1 < seg.npages) load_k(stile + (pi + 1) * tile_step, 0, kKAhead);
        }

        // ---- P.V for channels 32 w .. 32 w + 31 (V quant block w)
        auto pv_page = [&](auto tail) {
            VRaw vr[2];
            if constexpr (!STAGED) vr[0] = v_raw(sm.v, w, 0, gq, n);
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                half8_t vop[2];
                if constexpr (STAGED) {
                    vop[0] = vf[c][0];
                    vop[1] = vf[c][1];
                    if (c + kVAhead < kChunks) load_v(stile + pi * tile_step, c + kVAhead);
                } else {
                    if (c + 1 < kChunks) vr[(c + 1) & 1] = v_raw(sm.v, w, c + 1, gq, n);
                    v_convert<decltype(tail)::value>(vr[c & 1], c, gq, valid, vsh, m_nib, magic, vop);
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const half8_t pop = *(const half8_t*)(pbuf + ((c * RT + rt) * 64 + lane) * 16);
                    o[0][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[0], pop, o[0][rt], 0, 0, 0);
                    o[1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[1], pop, o[1][rt], 0, 0, 0);
                }
            }
        };
        if (!STAGED && tail_page) pv_page(std::true_type{});
        else pv_page(std::false_type{});
        if constexpr (!STAGED) {
            lds_barrier();   // every wave is done with this page's V tile and P operands
            if (next_rec) dma_v_tile(next_rec, g, a.n_kv_heads, sm.v, w, lane);
        }
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
    if constexpr (STAGED) break;   // staged launches run one worker per segment
  }
}

// Converts each (page, kv head) of a launch once into f16 matrix-core
// operands, block scales and V shifts (the staged mode above). Grid: (pages
// of the launch, kv heads); block x stages the x-th page of the launch's
// segments, in segment order, into staged tile x (or, with by_page, into
// tile `page`); blocks past the pages are ring refill workgroups.
__global__ __launch_bounds__(kThreads) void stage_kernel(StageArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[kKTile];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds[kVTile];
    if ((int)blockIdx.x >= a.n_pages) {   // ring refill workgroup
        copy_role(a.copy, ((int)blockIdx.x - a.n_pages) * (int)gridDim.y + (int)blockIdx.y);
        return;
    }
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n = lane & 15, gq = lane >> 4;
    const int slot = blockIdx.x, g = blockIdx.y;
    int rem = slot;
    int32_t page = -1;
    for (int si = 0; si < a.n_segs; ++si) {
        const int np = scalar_load(&a.segs[si].npages);
        if (rem < np) { page = scalar_load(&a.segs[si].page0) + rem; break; }
        rem -= np;
    }
    if (page < 0) return;   // past the launch's pages
    {
        const uint8_t* rec = page_record(a.ps, page);
        dma_k_tile(rec, g, k_lds, w, lane);
        dma_v_tile(rec, g, a.n_kv_heads, v_lds, w, lane);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    uint8_t* tile = a.staged + ((int64_t)(a.by_page ? page : slot) * a.n_kv_heads + g) * kStagedTile;
    // K: wave w converts token tiles 4 w .. 4 w + 3, as the QK role does
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int b = 0; b < kNB; ++b)
            *(half8_t*)(tile + staged_k_offset(4 * w + tt, b, lane)) = k_codes(k_raw(k_lds, kTokW * w + 16 * tt + n, b, gq), b);
    // K block scales per token: thread t writes token t's four scales
    {
        const uint8_t* row = k_lds + tid * kKRow;
        const uint32_t d0 = *(const uint16_t*)row, d1 = *(const uint16_t*)(row + kKBlock);
        const uint32_t d2 = *(const uint16_t*)(row + 2 * kKBlock), d3 = *(const uint16_t*)(row + 3 * kKBlock);
        *(uint2*)(tile + staged_scale_offset(tid)) = make_uint2(d0 | (d1 << 16), d2 | (d3 << 16));
    }
    // V: wave w converts block w (channel tiles 2 w, 2 w + 1), as the PV role does
    const int64_t vx = a.n_kv - (int64_t)page * kPageTokens;
    const int valid = (int)(vx < 0 ? 0 : (vx > kPageTokens ? kPageTokens : vx));
    const int vsh = v_shift_of(v_lds, w, valid, lane);
    if (lane == 0) *((int32_t*)(tile + kStagedShift) + w) = vsh;
    const uint32_t m_nib = vconst(0x000F000Fu), magic = vconst(0x64006400u);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        half8_t vop[2];
        v_convert<true>(v_raw(v_lds, w, c, gq, n), c, gq, valid, vsh, m_nib, magic, vop);
        *(half8_t*)(tile + staged_v_offset(c, 2 * w, lane)) = vop[0];
        *(half8_t*)(tile + staged_v_offset(c, 2 * w + 1, lane)) = vop[1];
    }
}

int compute_units() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int RT, bool STAGED, int LIMBS>
hipError_t launch_rt(const AttendArgs& a, hipStream_t stream) {
    const int R = a.n_q * a.G;
    const int64_t units = (int64_t)a.n_kv_heads * ((R + 16 * RT - 1) / (16 * RT));
    // workers: one per segment, unless the launch is unstaged with few (kv
    // head, row tile) units and many segments (a verify block over a long
    // cache): then about as many workers as the compute units hold at once,
    // each taking an even slice of the segments
    const int64_t target = (int64_t)compute_units() * 2;
    int64_t slices = a.n_segs;
    if (!STAGED && units * a.n_segs > 2 * target && units * 8 <= target) slices = target / units;
    AttendArgs b = a;
    b.n_slices = (int32_t)slices;
    const int64_t n_work = slices * units;
    const int64_t blocks = ((copy_workgroups(a.copy) + 7) & ~7) + ((n_work + 7) & ~7);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    return launch_kernel(mfma_kernel<RT, STAGED, LIMBS>, dim3((unsigned)blocks), dim3(kThreads), stream, b);
}

template <int RT, bool STAGED>
hipError_t launch_limbs(const AttendArgs& a, hipStream_t stream) {
    return a.q_f16 ? launch_rt<RT, STAGED, 1>(a, stream) : launch_rt<RT, STAGED, 2>(a, stream);
}

}  // namespace

// Row tiles: in-kernel conversion takes 16-row tiles (with two query limbs,
// 32-row tiles would not fit two workgroups' registers per compute unit);
// staged launches take 32-row tiles.
hipError_t launch_mfma(const AttendArgs& a, hipStream_t stream) {
    if (a.n_segs <= 0 && copy_workgroups(a.copy) == 0) return hipSuccess;
    if (a.staged) return launch_limbs<2, true>(a, stream);
    return launch_limbs<1, false>(a, stream);
}

bool mfma_stages(int rows) { return rows > 64; }

hipError_t launch_stage(const StageArgs& a, hipStream_t stream) {
    const int cx = (copy_workgroups(a.copy) + a.n_kv_heads - 1) / a.n_kv_heads;
    if (a.n_pages <= 0 && cx == 0) return hipSuccess;
    return launch_kernel(stage_kernel, dim3(a.n_pages + cx, a.n_kv_heads), dim3(kThreads), stream, a);
}

}  // namespace kvs
