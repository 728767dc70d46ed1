// KV append (gfx950): quantize a step's new K and V rows into the page
// records, the authoritative host record and, for a resident page, its device
// slot.
//
// The pages keep the whole KV history in pinned host memory and hold a
// working set on the device (page 1, "Summary"; page 2, opening paragraph):
// each new row is therefore written to the host record, and also to the
// device copy when its page is resident. The block rule is ggml's reference
// quantizer for Q8_0 and Q4_0 (the cache types named on page 1, "What it is
// useful for"; V is Q8_0 too in the q8_0-q8_0 pair of page 3, "1. Correctness
// - PPL parity"), in float32 with the scale stored as the nearest binary16:
//   Q8_0: d = max|x| / 127; code = round-half-away(x * (1 / d)), in [-127, 127];
//   Q4_0: d = (first element of largest magnitude) / -8;
//         nibble = min(15, trunc(x * (1 / d) + 8.5)).
// Divisions are IEEE float32 divisions, and every multiply and add rounds on
// its own as in the reference: the quantizers switch off floating-point
// contraction (a fused x * id + 8.5, or a scale converted through a fused
// multiply-add with a +0 addend, would change some codes and the sign of a
// zero scale).
//
// Work split: a workgroup of 256 threads takes 32 (token, kv head) rows;
// thread 8 j + b quantizes K block b (b < 4) or V block b - 4 of row j into
// LDS. The assembled rows (136 B of K, 72 B (Q4_0) or 136 B (Q8_0) of V per
// head) then leave LDS as 8-byte words: every row starts on an 8-byte
// boundary in the record.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cmath>

#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kRowsPerWG = 32;
constexpr int kKWords = kKRow / 8;           // 17

__device__ inline void load_block(const void* base, int f16, int64_t elem0, float (&x)[kQK]) {
    if (f16) {
        const uint4* p = (const uint4*)((const _Float16*)base + elem0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4 w = p[k];
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[8 * k + e] = (float)__builtin_bit_cast(_Float16, (unsigned short)(u[e >> 1] >> (16 * (e & 1))));
        }
    } else {
        const float4* p = (const float4*)((const float*)base + elem0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float4 w = p[k];
            x[4 * k] = w.x; x[4 * k + 1] = w.y; x[4 * k + 2] = w.z; x[4 * k + 3] = w.w;
        }
    }
}

__device__ inline uint32_t f16_bits(float d) {
    return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)d);
}

// one Q8_0 block into LDS (34 bytes at a 2-byte aligned offset)
__device__ inline void quant_q8_0(const float (&x)[kQK], uint8_t* dst) {
#pragma clang fp contract(off)
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kQK; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const float d = amax / 127.0f;
    const float id = d != 0.f ? 1.0f / d : 0.f;
    uint16_t* h = (uint16_t*)dst;
    h[0] = (uint16_t)f16_bits(d);
#pragma unroll
    for (int i = 0; i < kQK; i += 2) {
        int q[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float y = x[i + e] * id;
            float r = truncf(y);
            if (fabsf(y - r) >= 0.5f) r += copysignf(1.0f, y);   // half away from zero
            r = fminf(fmaxf(r, -127.f), 127.f);
            q[e] = (int)r;
        }
        h[1 + i / 2] = (uint16_t)((q[0] & 0xFF) | ((q[1] & 0xFF) << 8));
    }
}

// one Q4_0 block into LDS (18 bytes at a 2-byte aligned offset)
__device__ inline void quant_q4_0(const float (&x)[kQK], uint8_t* dst) {
#pragma clang fp contract(off)
    float amax = 0.f, m = 0.f;
#pragma unroll
    for (int i = 0; i < kQK; ++i) {
        const float a = fabsf(x[i]);
        if (a > amax) { amax = a; m = x[i]; }   // the first element of largest magnitude
    }
    float d = m / -8.0f;
    // d is a finished float32 value before its binary16 conversion: folding
    // the multiply into the conversion (v_fma_mix with a +0 addend) would turn
    // the -0 scale of an all-zero block into +0
    asm volatile("" : "+v"(d));
    const float id = d != 0.f ? 1.0f / d : 0.f;
    int nib[kQK];
#pragma unroll
    for (int i = 0; i < kQK; ++i) {
        const float y = x[i] * id + 8.5f;
        nib[i] = min(15, (int)truncf(y));
    }
    uint16_t* h = (uint16_t*)dst;
    h[0] = (uint16_t)f16_bits(d);
#pragma unroll
    for (int j = 0; j < 16; j += 2)
        h[1 + j / 2] = (uint16_t)((nib[j] | (nib[j + 16] << 4)) | ((nib[j + 1] | (nib[j + 17] << 4)) << 8));
}

template <typename VT>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    constexpr int kRowBytes = kKRow + VT::kRow;   // one head's K and V of one token (208 / 272 B)
    constexpr int kRowWords = kRowBytes / 8;
    static_assert(kRowBytes % 8 == 0, "rows leave LDS as 8-byte words");
    __shared__ __attribute__((aligned(16))) uint8_t rows[kRowsPerWG][kRowBytes];
    const int t = threadIdx.x;
    const int64_t n_rows = (int64_t)a.n_tok * a.n_kv_heads;
    const int64_t row0 = (int64_t)blockIdx.x * kRowsPerWG;
    {
        const int j = t >> 3, part = t & 7;
        const int64_t row = row0 + j;
        if (row < n_rows) {
            const int b = part & 3;
            float x[kQK];
            // inputs [n_tok, Hkv, 128]: row (token i, head g) = i * Hkv + g
            load_block(part < 4 ? a.k : a.v, a.f16, row * kHeadDim + b * kQK, x);
            if (part < 4)
                quant_q8_0(x, &rows[j][b * kKBlock]);
            else if constexpr (VT::kQ8)
                quant_q8_0(x, &rows[j][kKRow + b * VT::kBlock]);
            else
                quant_q4_0(x, &rows[j][kKRow + b * VT::kBlock]);
        }
    }
    __syncthreads();
    for (int i = t; i < kRowsPerWG * kRowWords; i += 256) {
        const int j = i / kRowWords, w = i - j * kRowWords;
        const int64_t row = row0 + j;
        if (row >= n_rows) continue;
        const int64_t tok = a.pos0 + row / a.n_kv_heads;
        const int g = (int)(row % a.n_kv_heads);
        const int64_t page = tok / kPageTokens;
        const int r = (int)(tok % kPageTokens);
        const int64_t off = w < kKWords ? (int64_t)g * kKTile + (int64_t)r * kKRow + 8 * w
                                        : (int64_t)a.n_kv_heads * kKTile + (int64_t)g * VT::kTile + (int64_t)r * VT::kRow +
                                              8 * (w - kKWords);
        const uint64_t val = *(const uint64_t*)&rows[j][8 * w];
        *(uint64_t*)(a.host + page * a.page_bytes + off) = val;
        const int32_t sv = a.src[page];
        if (sv >= 0) *(uint64_t*)(a.slots + (int64_t)sv * a.page_bytes + off) = val;
    }
    // the host record is read over the link by later ring copies and by the
    // CPU: make the writes visible beyond this device
    __threadfence_system();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
    const int64_t n_rows = (int64_t)a.n_tok * a.n_kv_heads;
    if (n_rows <= 0) return hipSuccess;
    const int64_t blocks = (n_rows + kRowsPerWG - 1) / kRowsPerWG;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (a.v_q8) hipLaunchKernelGGL(append_kernel<VQ8>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(append_kernel<VQ4>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvs
