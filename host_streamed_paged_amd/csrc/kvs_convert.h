// Block conversion of page records into f16 matrix-core operands, shared by
// the matrix-core kernels (kvs_mfma.hip: the verify kernel, the staging
// probe) and the prefill kernel (kvs_prefill.hip), so that the probe of one
// checks the arithmetic of all. The K operand holds each Q8_0 code exactly;
// the V operand is d * (u - 8) (Q4_0) or d * code (Q8_0) rounded once to f16,
// divided by a power of two when the block's scales could overflow f16.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvs_internal.h"
#include "kvs_device.h"

namespace kvs {

// A V block scale of magnitude above 8188 (binary16 bits 0x6FFF) can make
// d * (u - 8) exceed the largest f16, 65504; such pages take the V operand
// divided by 2^kVShift.
constexpr uint32_t kVBigBits = 0x6FFFu;
constexpr int kVShift = 3;

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

// V shift of quant block b over the first NTOK rows of a V tile (a page, or
// a 64-token sub-block; V rows in LDS, record layout): for Q4_0, kVShift if a
// cached row's scale magnitude exceeds 8188, else 0; for Q8_0 (|code| <=
// 128), kVShift8 if one exceeds 511.75 (bits 0x5FFF), so that
// d * code / 2^shift stays within 65504. Rows at or past `valid` are not
// cached and may hold any bytes. Wave-uniform.
constexpr uint32_t kVBigBits8 = 0x5FFFu;
constexpr int kVShift8 = 7;
template <typename VT, int NTOK = kPageTokens>
__device__ inline int v_shift_of(const uint8_t* v_lds, int b, int valid, int lane) {
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < NTOK / 64; ++j) {
        const int t = lane + 64 * j;
        const uint32_t bits = *(const uint16_t*)(v_lds + t * VT::kRow + b * VT::kBlock) & 0x7FFFu;
        mx = (t < valid && bits > mx) ? bits : mx;
    }
    if constexpr (VT::kQ8) return __any(mx > kVBigBits8) ? kVShift8 : 0;
    return __any(mx > kVBigBits) ? kVShift : 0;
}

// V^T operands of O^T += V^T . P^T for chunk c (tokens [32 c, 32 c + 32)) and
// quant block b: vop[0] holds channel 32 b + n, vop[1] channel 32 b + 16 + n
// (Q4_0: low and high nibbles of byte n; Q8_0: codes n and 16 + n), for the
// lane's 8 token slots: slot j of lane group gq is token 32 c + 4 gq + j for
// j < 4, else 32 c + 12 + 4 gq + j. Each value is d * (u - 8) / 2^vshift or
// d * code / 2^vshift rounded once to f16 ((u - 8) / 2^vshift and
// code / 2^vshift are exact, and the product of two f16 values is rounded
// once). TAIL zeroes rows at or past `valid` (their scales may be NaN). Split
// into the LDS reads (v_raw) and the arithmetic (v_convert), like the K
// operand.
template <typename VT>
struct VRaw {
    uint32_t byte[8];                   // byte n of the slot's token (Q4_0 nibbles, Q8_0 code n)
    uint32_t hbyte[VT::kQ8 ? 8 : 1];    // Q8_0: code 16 + n
    uint32_t d[8];                      // scale bits of the slot's token
};
template <typename VT>
__device__ inline VRaw<VT> v_raw(const uint8_t* v_lds, int b, int c, int gq, int n) {
    const uint8_t* vlane = v_lds + b * VT::kBlock + 4 * gq * VT::kRow;
    VRaw<VT> r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint8_t* row = vlane + (32 * c + (j < 4 ? j : 12 + j)) * VT::kRow;
        r.byte[j] = row[2 + n];
        if constexpr (VT::kQ8) r.hbyte[j] = row[18 + n];
        r.d[j] = *(const uint16_t*)row;
    }
    return r;
}
template <bool TAIL, typename VT>
__device__ inline void v_convert(const VRaw<VT>& r, int c, int gq, int valid, int vshift, uint32_t m_nib, uint32_t magic,
                                 half8_t (&vop)[2]) {
    const _Float16 cs = vshift ? (VT::kQ8 ? (_Float16)0.0078125f : (_Float16)0.125f) : (_Float16)1.f;
    const half2_t cc = {cs, cs};
    const half2_t off = {(_Float16)-1032.f * cs, (_Float16)-1032.f * cs};
    const half2_t off8 = {(_Float16)-1152.f * cs, (_Float16)-1152.f * cs};
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
        half2_t lo, hi;
        if constexpr (VT::kQ8) {
            const uint32_t xh = __builtin_amdgcn_perm(r.hbyte[j1], r.hbyte[j0], 0x0c040c00u);
            lo = q8_pair_f16(x, cc, off8) * dd;                  // channel n
            hi = q8_pair_f16(xh, cc, off8) * dd;                 // channel 16 + n
        } else {
            lo = q4_nibbles_f16((x & m_nib) | magic, cc, off) * dd;          // channel n
            hi = q4_nibbles_f16(((x >> 4) & m_nib) | magic, cc, off) * dd;   // channel 16 + n
        }
        vop[0][j0] = lo[0]; vop[0][j1] = lo[1];
        vop[1][j0] = hi[0]; vop[1][j1] = hi[1];
    }
}

// One of the two V^T operands above, for a caller that owns one 16-channel
// half of block b: half h = 0 gives vop[0] (channel 32 b + n), h = 1 gives
// vop[1] (channel 32 b + 16 + n), with the same token slots and the same
// values. For Q4_0 the high nibble is taken in place: bits 0x6400 | (u << 4)
// are the f16 value 1024 + 16 u, and (1024 + 16 u) / 16 - 72 = u - 8 exactly.
template <typename VT>
struct VRaw1 {
    uint32_t byte[8];   // Q4_0: byte n of the slot's token; Q8_0: code 16 h + n
    uint32_t dd[4];     // scale bits of slots 2 i (low half) and 2 i + 1 (high half)
};
// The lane's byte offsets into the V tile for v_raw1: `ob` of its byte in
// token row 4 gq of block b (byte n, or code 16 h + n), `od` of that row's
// scale. Made opaque so that every read below is one constant offset from
// them (short address chains keep the reads attributable to their LDS array).
struct VLane {
    uint32_t ob, od;
};
template <typename VT>
__device__ inline VLane v_lane(int b, int gq, int n, int h) {
    VLane r;
    r.od = b * VT::kBlock + 4 * gq * VT::kRow;
    r.ob = r.od + 2 + (VT::kQ8 ? 16 * h : 0) + n;
    asm volatile("" : "+v"(r.ob), "+v"(r.od));
    return r;
}
// v_raw with the lane's offsets from v_lane (h = 0): every read one constant
// offset from them.
template <typename VT>
__device__ inline VRaw<VT> v_raw_o(const uint8_t* v_lds, const VLane& vl, int c) {
    VRaw<VT> r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int ro = (32 * c + (j < 4 ? j : 12 + j)) * VT::kRow;
        r.byte[j] = v_lds[vl.ob + ro];
        if constexpr (VT::kQ8) r.hbyte[j] = v_lds[vl.ob + 16 + ro];
        r.d[j] = *(const uint16_t*)(v_lds + (vl.od + ro));
    }
    return r;
}
// v_raw1's reads: the slots' bytes through the lane's offsets from v_lane,
// and their scales from a table of the tile's V scales, [block][token] as
// binary16 bits (vsc), with two 8-byte reads: slots 0..3 are tokens
// 32 c + 4 gq + 0..3, slots 4..7 tokens 32 c + 16 + 4 gq + 0..3.
template <typename VT>
__device__ inline VRaw1<VT> v_raw1(const uint8_t* v_lds, const VLane& vl, const uint16_t* vsc_b, int c, int gq) {
    VRaw1<VT> r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int ro = (32 * c + (j < 4 ? j : 12 + j)) * VT::kRow;
        r.byte[j] = v_lds[vl.ob + ro];
    }
    const uint2 lo = *(const uint2*)(vsc_b + 32 * c + 4 * gq);
    const uint2 hi = *(const uint2*)(vsc_b + 32 * c + 16 + 4 * gq);
    r.dd[0] = lo.x; r.dd[1] = lo.y; r.dd[2] = hi.x; r.dd[3] = hi.y;
    return r;
}
// Per-wave constants of v_convert1 for half h: the nibble mask and the f16
// factor and offset pairs (Q4_0), or the factor and offset (Q8_0).
struct VHalf {
    uint32_t mask;
    half2_t cc, off;
};
template <typename VT>
__device__ inline VHalf v_half(int h, int vshift) {
    const _Float16 cs = vshift ? (VT::kQ8 ? (_Float16)0.0078125f : (_Float16)0.125f) : (_Float16)1.f;
    VHalf r;
    if constexpr (VT::kQ8) {
        r.mask = 0u;
        r.cc = half2_t{cs, cs};
        r.off = half2_t{(_Float16)-1152.f * cs, (_Float16)-1152.f * cs};
    } else {
        const _Float16 c = h ? cs * (_Float16)0.0625f : cs;
        const _Float16 o = h ? (_Float16)-72.f * cs : (_Float16)-1032.f * cs;
        r.mask = h ? 0x00F000F0u : 0x000F000Fu;
        r.cc = half2_t{c, c};
        r.off = half2_t{o, o};
    }
    return r;
}
// The caller's scale table holds 0 for rows past the cache.
template <typename VT>
__device__ inline half8_t v_convert1(const VRaw1<VT>& r, const VHalf& vh, uint32_t magic) {
    half8_t vop;
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) {
        const int j0 = 2 * jp, j1 = 2 * jp + 1;
        const half2_t dd = as_h2(r.dd[jp]);
        const uint32_t x = __builtin_amdgcn_perm(r.byte[j1], r.byte[j0], 0x0c040c00u);
        half2_t v;
        if constexpr (VT::kQ8) v = q8_pair_f16(x, vh.cc, vh.off) * dd;
        else v = q4_nibbles_f16((x & vh.mask) | magic, vh.cc, vh.off) * dd;
        vop[j0] = v[0];
        vop[j1] = v[1];
    }
    return vop;
}

}  // namespace kvs
