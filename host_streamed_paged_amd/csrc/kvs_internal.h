// Internal interface between the host runtime (kvs_runtime.cpp) and the
// kernels (kvs_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvs.h"

namespace kvs {

constexpr int kPageTokens = 256;             // tokens per page
constexpr int kHeadDim = 128;                // d
constexpr int kQK = 32;                      // values per quant block
constexpr int kNB = kHeadDim / kQK;          // blocks per head row (4)
constexpr int kKBlock = 34;                  // Q8_0: f16 scale + 32 int8
constexpr int kKRow = kNB * kKBlock;         // 136 B: one head's K for one token
constexpr int kKTile = kPageTokens * kKRow;  // 34816 B: one head's K for one page
constexpr int kPartStride = kHeadDim + 2;    // partial record: acc[128], m (log2 units), l

// V block type of a page record. K is Q8_0 in both pairs the library builds:
// V is Q4_0 (f16 scale + 16 nibble bytes, the q8_0-q4_0 pair of page 2,
// "TLDR - recommended setup") or Q8_0 (the q8_0-q8_0 pair of page 3,
// "1. Correctness - PPL parity"). Kernels that read V are instantiated per
// type; the launch arguments carry the type as v_q8.
template <bool Q8>
struct VType {
    static constexpr bool kQ8 = Q8;
    static constexpr int kBlock = Q8 ? 34 : 18;              // bytes per 32-value block
    static constexpr int kRow = kNB * kBlock;                 // one head's V for one token (136 / 72 B)
    static constexpr int kTile = kPageTokens * kRow;          // one head's V for one page (34816 / 18432 B)
};
using VQ4 = VType<false>;
using VQ8 = VType<true>;
// Page record bytes per kv head.
__host__ __device__ constexpr int head_record_bytes(bool v_q8) { return kKTile + (v_q8 ? VQ8::kTile : VQ4::kTile); }
// Matrix-core operands of one (page, kv head) as the operand probe writes
// them (kvs_debug_stage): the f16 K and V^T operands in fragment order, the K
// block scales per token as float32, and the V scaling exponent of each
// (64-token sub-block, 32-channel block) (padded to keep tiles 256-byte
// aligned).
constexpr int kStagedK = kPageTokens * kHeadDim * 2;          // K operands [16 token tiles][4 blocks][64 lanes] x 16 B
constexpr int kStagedOps = 2 * kStagedK;                      // then V^T operands [8 chunks][8 channel tiles][64 lanes] x 16 B
constexpr int kStagedScaleBytes = kPageTokens * kNB * 4;      // K scales [token][block] float32
constexpr int kStagedShift = kStagedOps + kStagedScaleBytes;  // V shift per (sub-block, block), int32
constexpr int kStagedTile = kStagedShift + 256;
__host__ __device__ constexpr int staged_k_offset(int tt16, int b, int lane) { return ((tt16 * kNB + b) * 64 + lane) * 16; }
__host__ __device__ constexpr int staged_v_offset(int c, int ct, int lane) { return kStagedK + ((c * 8 + ct) * 64 + lane) * 16; }
__host__ __device__ constexpr int staged_scale_offset(int tok) { return kStagedOps + tok * kNB * 4; }
static_assert(kStagedTile == KVS_STAGED_TILE_BYTES, "staged tile size as documented in kvs.h");

// One run of consecutive logical pages of one split-K group, processed in
// page order by one workgroup. flags bit 0: page0 is the group's first page
// (start from an empty state instead of loading the stored one).
struct Seg {
    int32_t group;
    int32_t page0;
    int32_t npages;
    int32_t flags;
};
constexpr int32_t kSegFresh = 1;
// The device copy of a layer's segments carries src[page0] (see PageSource)
// in flags bits 8..31, so that a kernel finds its first page's record without
// a dependent read of the page table; bits 0..7 hold the flags proper. Slot
// indices and streamed ranks therefore stay within a signed 24-bit range.
constexpr int kSegSrcShift = 8;
constexpr int32_t kSegFlagMask = 0xFF;
constexpr int64_t kMaxSlots = (int64_t(1) << 23) - 1;

// Where page p's record lives: src[p] >= 0 is a resident slot index;
// src[p] < 0 means streamed with rank -1 - src[p], found in the ring chunk of
// the current launch at position rank - chunk_rank0, or, in a zero-copy
// launch (host set), read in place from the pinned host record of page p.
struct PageSource {
    const uint8_t* slots;       // base of the resident slots
    const uint8_t* ring_chunk;  // first ring slot of this launch's chunk (null if none)
    const int32_t* src;         // [n_pages] device table
    int32_t chunk_rank0;        // streamed rank of the chunk's first page
    int64_t page_bytes;
    const uint8_t* host;        // zero-copy launches: the layer's host records, else null
};

__host__ __device__ inline const uint8_t* page_ptr(const PageSource& ps, int32_t page) {
    int32_t s = ps.src[page];
    if (s >= 0) return ps.slots + (int64_t)s * ps.page_bytes;
    if (ps.host) return ps.host + (int64_t)page * ps.page_bytes;
    return ps.ring_chunk + (int64_t)((-1 - s) - ps.chunk_rank0) * ps.page_bytes;
}

// Ring refill carried by a launch: copy workgroups (blockIdx.x >= n_segs)
// copy n_pages page records from pinned host memory into consecutive ring
// slots at ring_dst, while the other workgroups compute on earlier slots.
constexpr int kMaxCopyPages = 16;
constexpr int kCopyPartBytes = 32768;   // bytes a copy workgroup moves per round
struct CopyJob {
    const uint8_t* host;                // the layer's host records (page-major)
    uint8_t* ring_dst;                  // first ring slot to fill
    int64_t page_bytes;
    int64_t part_bytes;                 // bytes per copy workgroup (a multiple of kCopyPartBytes)
    int32_t n_pages;                    // pages to copy (0: none)
    int32_t parts_per_page;             // copy workgroups per page
    int32_t pages[kMaxCopyPages];       // logical page of each copied slot
};

// Copy role of a workgroup (its first 256 threads): part `part` of the job's
// pages, in rounds of kCopyPartBytes. Each round's global loads are all
// issued before any of its stores, so that many host-memory reads are in
// flight over the link.
__device__ inline void copy_role(const CopyJob& cj, int part) {
    const int page_i = part / cj.parts_per_page, sub = part % cj.parts_per_page;
    if (page_i >= cj.n_pages) return;
    const int64_t off0 = (int64_t)sub * cj.part_bytes;
    const int64_t end = cj.page_bytes - off0 < cj.part_bytes ? cj.page_bytes : off0 + cj.part_bytes;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int kPer = kCopyPartBytes / 16 / 256;   // 8 x 16 bytes per thread
    for (int64_t off = off0; off < end; off += kCopyPartBytes) {
        const int64_t n = end - off < kCopyPartBytes ? end - off : kCopyPartBytes;
        const u32x4* src = (const u32x4*)(cj.host + (int64_t)cj.pages[page_i] * cj.page_bytes + off);
        u32x4* dst = (u32x4*)(cj.ring_dst + (int64_t)page_i * cj.page_bytes + off);
        const int n16 = (int)(n / 16);
        u32x4 v[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int e = threadIdx.x + 256 * k;
            if (e < n16) v[k] = __builtin_nontemporal_load(src + e);
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int e = threadIdx.x + 256 * k;
            if (e < n16) dst[e] = v[k];
        }
    }
}
// The same job cut into parts of part_bytes (a multiple of kCopyPartBytes):
// fewer, longer-running copy workgroups.
inline CopyJob with_part_bytes(const CopyJob& cj, int64_t part_bytes) {
    CopyJob r = cj;
    r.part_bytes = part_bytes;
    r.parts_per_page = (int32_t)((cj.page_bytes + part_bytes - 1) / part_bytes);
    return r;
}

__host__ __device__ inline int copy_workgroups(const CopyJob& cj) {
    return cj.n_pages * cj.parts_per_page;
}

struct AttendArgs {
    CopyJob copy;         // ring refill carried by this launch
    PageSource ps;
    const Seg* segs;      // this launch's segments
    int32_t n_segs;
    int32_t n_kv_heads;
    int32_t n_q_heads;
    int32_t G;            // query heads per kv head
    const void* q;        // [n_q, Hq, 128]
    int32_t q_f16;
    int32_t n_q;
    int64_t q_pos0;
    int64_t n_kv;
    float scale_log2;     // scale * log2(e): scores are kept in log2 units
    int32_t causal;
    float* part;          // [n_groups][n_q][Hq][kPartStride]
    int32_t n_slices;     // matrix-core kernel: segment slices per (kv head, row tile), set at launch
    int32_t v_q8;         // V blocks are Q8_0 (else Q4_0)
    const uint8_t* spare; // device memory of at least one page record (the ring's first slot) that a
                          // kernel may read and ignore
};

// Conversion of a launch's pages into staged operands (kvs_mfma.hip).
struct StageArgs {
    CopyJob copy;         // ring refill carried by this launch
    PageSource ps;
    const Seg* segs;      // the launch's segments; their pages are staged in order
    int32_t n_segs;
    int32_t n_kv_heads;
    int64_t n_kv;
    int32_t n_pages;      // pages of the launch's segments
    uint8_t* staged;      // [pages][n_kv_heads][kStagedTile]
    int32_t by_page;      // 1: page p goes to tile p (a probe of a whole layer), 0: the x-th page to tile x
    int32_t v_q8;         // V blocks are Q8_0 (else Q4_0)
};

struct GatherArgs {
    CopyJob copy;
    PageSource ps;
    const Seg* segs;
    int32_t n_segs;
    int32_t n_kv_heads;
    int64_t tok0;
    int64_t n_tok;
    float* k_out;         // [n_tok, Hkv, 128]
    float* v_out;
    int32_t v_q8;         // V blocks are Q8_0 (else Q4_0)
};

// Raw record export probe: the bytes of each page as the kernels read them.
struct ExportArgs {
    CopyJob copy;
    PageSource ps;
    const Seg* segs;
    int32_t n_segs;
    uint8_t* dst;         // [n_pages][page_bytes], device
};

// KV append: new K and V rows [n_tok, Hkv, 128] (f32 or f16) quantized into
// the page records of tokens pos0 .. pos0 + n_tok - 1.
struct AppendArgs {
    const void* k;
    const void* v;
    int32_t f16;              // 1: inputs are f16, 0: f32
    int64_t pos0;
    int32_t n_tok;
    int32_t n_kv_heads;
    int64_t page_bytes;
    const int32_t* src;       // the layer's device page table (slot >= 0 when resident)
    uint8_t* slots;           // resident slots
    uint8_t* host;            // the layer's host records (pinned, device-visible)
    int32_t v_q8;             // V blocks are Q8_0 (else Q4_0)
};

// Kernel timing: when the host sets a start/stop event pair here, the next
// kernel launched by this thread carries them on its dispatch
// (hipExtLaunchKernel), so their elapsed time spans the kernel's execution
// only, not the work of getting it onto the queue.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchTiming& launch_timing();   // this thread's pending pair (kvs_kernels.hip)

// The library's fixed scratch array of split-K partials (kvs_attend_noalloc):
// its size, and its device address on the current device, looked up once per
// device with hipGetSymbolAddress (kvs_kernels.hip, beside the array).
constexpr size_t kScratchBytes = size_t(KVS_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;
hipError_t scratch_region(float** out);

hipError_t launch_attend(const AttendArgs& a, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
// few-row decode kernel (kvs_decode.hip): rows = n_q * G in [1, 6]
bool decode_supports(int rows);
hipError_t launch_decode(const AttendArgs& a, hipStream_t stream);
// matrix-core kernels (kvs_mfma.hip) for more rows: routes to the verify
// kernel (kvs_verify.hip, 7 to 32 rows per kv head) and the prefill kernel
hipError_t launch_mfma(const AttendArgs& a, hipStream_t stream);
hipError_t launch_verify(const AttendArgs& a, hipStream_t stream);
bool verify_rows(int rows);    // rows per kv head that the verify kernel takes
// prefill kernel (kvs_prefill.hip), for blocks of more than 64 rows per kv head
hipError_t launch_prefill(const AttendArgs& a, hipStream_t stream);
bool prefill_rows(int rows);   // rows per kv head that the prefill kernel takes
// staging probe: each page's matrix-core operands written out (kvs_mfma.hip)
hipError_t launch_stage(const StageArgs& a, hipStream_t stream);
hipError_t launch_combine(const float* part, int32_t n_groups, int32_t n_q, int32_t n_q_heads,
                          float* out, float* lse, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);
hipError_t launch_export(const ExportArgs& a, hipStream_t stream);
hipError_t launch_fill_u32(void* dst, uint32_t value, uint64_t n_words, hipStream_t stream);
hipError_t launch_copy(const CopyJob& cj, hipStream_t stream);   // copy-only launch

}  // namespace kvs
