// Small device helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <cstdint>

#include "kvs_internal.h"

namespace kvs {

// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not
// wait for outstanding global loads, so page data stays in flight across it.
// The wait is the builtin (lgkmcnt(0), the other counters untouched), not
// inline asm: the compiler's wait tracking then knows that every LDS and
// scalar load has completed here. A scalar load it still counts as pending
// would make each later wait for an LDS result a full lgkmcnt(0).
__device__ inline void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Uniform loads through the scalar cache (constant address space).
template <typename T>
__device__ inline T scalar_load(const T* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}

// A 32-bit constant held in a VGPR the compiler cannot see through, so
// three-operand VALU ops (v_and_or_b32) can take it: gfx9 VOP3 encodings have
// no literal field and read at most one scalar operand.
__device__ inline uint32_t vconst(uint32_t c) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
    return r;
}

// LDS DMA: each lane of the wave copies 16 bytes from global memory to
// lds_base + 16 * lane (lds_base must be the same for the whole wave).
__device__ inline void dma16(const void* gsrc, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// This lane's value combined with lane (i ^ 16) / (i ^ 32)'s by max or add.
// v_permlane16_swap / v_permlane32_swap hand every lane both values without an
// LDS round trip; max and add are commutative, so every lane of the pair gets
// the same bits.
__device__ inline float f_bits(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ inline uint32_t u_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ inline float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(u_bits(v), u_bits(v), false, false);
    return fmaxf(f_bits(r[0]), f_bits(r[1]));
}
__device__ inline float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(u_bits(v), u_bits(v), false, false);
    return fmaxf(f_bits(r[0]), f_bits(r[1]));
}
__device__ inline float add_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(u_bits(v), u_bits(v), false, false);
    return f_bits(r[0]) + f_bits(r[1]);
}
__device__ inline float add_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(u_bits(v), u_bits(v), false, false);
    return f_bits(r[0]) + f_bits(r[1]);
}

// ---- Block decoding, shared by every kernel that reads page records (the
// attention kernels, the staging kernel and the gather probe), so that a
// probe of one checks the arithmetic of all.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ inline half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ inline uint32_t as_u(half2_t x) { return __builtin_bit_cast(uint32_t, x); }

// A block scale: the binary16 in the low 16 bits of `bits`, as float32 (exact).
__device__ inline float scale_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits & 0xFFFFu));
}

// Eight Q8_0 codes, packed little-endian in two dwords, as exact binary16
// values: each code k is biased to u = k + 128 in [0, 255], 0x6400 | u is the
// binary16 value 1024 + u, and 1152 = 1024 + 128 is subtracted. Every step is
// exact, code -128 included.
__device__ inline half8_t q8_codes_f16(uint32_t x0, uint32_t x1) {
    const half2_t k_off = {(_Float16)1152.f, (_Float16)1152.f};
    const uint32_t c_hi64 = 0x64646464u;
    x0 ^= 0x80808080u;
    x1 ^= 0x80808080u;
    const half2_t e0 = as_h2(__builtin_amdgcn_perm(c_hi64, x0, 0x04010400u)) - k_off;
    const half2_t e1 = as_h2(__builtin_amdgcn_perm(c_hi64, x0, 0x04030402u)) - k_off;
    const half2_t e2 = as_h2(__builtin_amdgcn_perm(c_hi64, x1, 0x04010400u)) - k_off;
    const half2_t e3 = as_h2(__builtin_amdgcn_perm(c_hi64, x1, 0x04030402u)) - k_off;
    half8_t r;
    r[0] = e0[0]; r[1] = e0[1]; r[2] = e1[0]; r[3] = e1[1];
    r[4] = e2[0]; r[5] = e2[1]; r[6] = e3[0]; r[7] = e3[1];
    return r;
}

// Two Q4_0 nibbles u, held as the binary16 values 1024 + u (0x6400 | u in
// each half of `biased`), as the exact binary16 values (u - 8) * c for
// c = 1 or 1/8 passed as the pair {c, c} with minus_1032c = {-1032 c, -1032 c}:
// (1024 + u) c - 1032 c is one fused operation whose exact result is
// representable, so nothing is rounded.
__device__ inline half2_t q4_nibbles_f16(uint32_t biased, half2_t c, half2_t minus_1032c) {
    return __builtin_elementwise_fma(as_h2(biased), c, minus_1032c);
}

// Two Q8_0 codes, the bytes of the low and high halves of `pair` (bits 0..7
// and 16..23, the other bits zero), as the exact binary16 values code * c
// for c = 1 or 2^-7 passed as {c, c} with minus_1152c = {-1152 c, -1152 c}:
// the xor flips each code's sign bit (u = code + 128) and sets the 0x64
// exponent byte, giving 1024 + u, and (1024 + u) c - 1152 c = code * c is
// exact.
__device__ inline half2_t q8_pair_f16(uint32_t pair, half2_t c, half2_t minus_1152c) {
    return __builtin_elementwise_fma(as_h2(pair ^ 0x64806480u), c, minus_1152c);
}

// Query operands of the matrix-core kernels (16x16x32 f16 tiles, the query
// as the B operand): this lane's 8 elements [32 b + 8 gq, +8) of each block b
// of query row (token qi, head h), zero if !valid. The row is scaled by the
// power of two that puts its largest magnitude in [2^14, 2^15), and by the
// sign of the softmax scale (both exact), then split into f16 limbs:
// hi = f16(q'), and for LIMBS == 2 lo = f16(q' - hi), which holds an f32
// query to about 22 bits (an f16 query is exact in hi). cq = |scale| *
// log2(e) / 2^shift > 0 turns the float32 products into log2-unit scores
// (a zero scale gives zero operands and cq = 1: every score is 0). Every lane
// of the wave must call it (the row maximum is exchanged between lanes n,
// n + 16, n + 32, n + 48).
template <int LIMBS>
__device__ inline void query_operands(const AttendArgs& a, int qi, int h, bool valid, int gq,
                                      half8_t (&qop)[LIMBS][kNB], float& cq) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    float x[kNB][8];
    if (valid) {
        const int64_t off = ((int64_t)qi * a.n_q_heads + h) * kHeadDim + 8 * gq;
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            if (a.q_f16) {
                const u32x4_t raw = *(const u32x4_t*)((const _Float16*)a.q + off + kQK * b);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const half2_t hv = as_h2(raw[e]);
                    x[b][2 * e] = (float)hv[0];
                    x[b][2 * e + 1] = (float)hv[1];
                }
            } else {
                const f32x4_t* qp = (const f32x4_t*)((const float*)a.q + off + kQK * b);
                const f32x4_t u0 = qp[0], u1 = qp[1];
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
    amax = max_xor16(amax);   // over the row's four lanes
    amax = max_xor32(amax);
    const int ex = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 0;   // amax = m 2^ex, m in [0.5, 1)
    const float sgn = a.scale_log2 < 0.f ? -1.f : (a.scale_log2 > 0.f ? 1.f : 0.f);
    const float up = sgn * __builtin_amdgcn_ldexpf(1.f, 15 - ex);
    cq = a.scale_log2 == 0.f ? 1.f : fabsf(a.scale_log2) * __builtin_amdgcn_ldexpf(1.f, ex - 15);
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float y = x[b][e] * up;   // exact
            const _Float16 hi = (_Float16)y;
            qop[0][b][e] = hi;
            if constexpr (LIMBS == 2) qop[LIMBS - 1][b][e] = (_Float16)(y - (float)hi);
        }
}

// Page record of logical page `page` for this launch: a resident slot, a
// slot of the ring chunk the launch works on, or (zero-copy launches) the
// pinned host record itself.
// Record of page `page` whose source index src[page] is sv.
__device__ inline const uint8_t* page_record_of(const PageSource& ps, int32_t page, int32_t sv) {
    if (sv >= 0) return ps.slots + (int64_t)sv * ps.page_bytes;
    if (ps.host) return ps.host + (int64_t)page * ps.page_bytes;
    return ps.ring_chunk + (int64_t)((-1 - sv) - ps.chunk_rank0) * ps.page_bytes;
}
__device__ inline const uint8_t* page_record(const PageSource& ps, int32_t page) {
    return page_record_of(ps, page, scalar_load(ps.src + page));
}

// Compute units of the current device (cached per device).
inline int compute_units() {
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

// Launch a kernel; a pending timing pair (launch_timing) goes with it.
template <typename K, typename... Args>
inline hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
    LaunchTiming& t = launch_timing();
    if (t.start) {
        const LaunchTiming u = t;
        t = LaunchTiming{};
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, u.start, u.stop, 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
    }
    return hipGetLastError();
}

}  // namespace kvs
