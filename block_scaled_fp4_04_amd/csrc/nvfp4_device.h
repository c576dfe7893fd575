// nvfp4_device.h -- device helpers shared by the gfx950 NVFP4 kernels:
// operand types, the exact E2M1 x E4M3 decode, the bfloat16 epilogue
// rounding, the split-K hand-off, wait counts and direct-to-LDS loads.
//
// Decode exactness: every a' = code * scale has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in fp16 (two FP4 codes per byte
// and one FP8 scale per 16 elements: "Peeling the Kernel Onion", section
// "The Benchmark Design").
#pragma once
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4v __attribute__((ext_vector_type(4)));

// Two E4M3 bytes of a 32-bit word -> two fp16 (exact: every finite E4M3
// value, subnormals included, is a normal fp16).
__device__ __forceinline__ h2 e4m3x2_lo(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}
__device__ __forceinline__ h2 e4m3x2_hi(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}

// Eight E2M1 codes (element 2j in bits 3:0 of byte j) times one fp16 scale.
// The four converts are kept apart from the four multiplies (the empty asm
// stops the scheduler from pairing each multiply right after its convert,
// which made every multiply wait on the result just produced).
__device__ __forceinline__ h8 decode8(uint32_t w, _Float16 s) {
    const h2 ss = {s, s};
    h2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    h2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    h2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    h2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
    asm("" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
    const h2 p0 = c0 * ss, p1 = c1 * ss, p2 = c2 * ss, p3 = c3 * ss;
    return h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// FP32 -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t to_bf16(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

// One accumulator element read out of the AGPR it lives in.  Done in asm so
// the accumulators stay in AGPRs until their block is stored (otherwise the
// compiler copies the whole accumulator file to VGPRs at once).  Only for
// accumulators that come straight from the MFMAs.
// 16-byte load with the non-temporal hint, for data read once per call
// (weights streamed from HBM): measured 9% faster for the grouped GEMM with
// its operands beyond the last-level cache.
__device__ __forceinline__ uint4 load_nt16(const uint8_t* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return uint4{t[0], t[1], t[2], t[3]};
}

__device__ __forceinline__ float acc_read(float x) {
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
    return r;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int s) {
    return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// Scale of MFMA sub-step s (0..3) from the pair (block of words 0-1, block of
// words 2-3).  Taken by value: selecting between two array elements by
// reference would keep the array in private memory.
__device__ __forceinline__ _Float16 scale_of(h2 pair, int s) {
    return s < 2 ? pair[0] : pair[1];
}
// ---------------------------------------------------------------------------
// Split-K hand-off between workgroups.
//
// Partial sums are written and read with relaxed device-scope atomic stores
// and loads (on gfx950 these are plain stores/loads with the device-coherence
// bit, so no cache-wide write-back or invalidate is needed); the writer waits
// for its stores to complete before it increments the tile's arrival counter,
// and the last arrival reads the partials only after its increment returned.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void publish(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Increments the counter once all earlier stores of the calling wave have
// completed; returns the counter's previous value.
__device__ __forceinline__ uint32_t arrive(uint32_t* counter) {
    __builtin_amdgcn_s_waitcnt(0);
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(uint32_t* counter) {
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Takes a ticket without waiting for this wave's earlier stores (for
// partials published with flags, which the reader checks itself).
__device__ __forceinline__ uint32_t take_ticket(uint32_t* counter) {
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Flagged partial sums: each FP32 value travels in one 64-bit word with a
// ready flag in its upper half, written by a single 64-bit store, so a
// reader that sees the flag also sees the value -- the writer need not wait
// for its stores before it takes its ticket.  The reader clears every word
// it consumed (flag 0) before the kernel ends, so the next call starts from
// cleared words.
constexpr uint64_t kReady = 1ull << 32;
__device__ __forceinline__ void publish_flagged(uint64_t* p, float v) {
    __hip_atomic_store(p, (uint64_t)__builtin_bit_cast(uint32_t, v) | kReady, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fetch_flagged(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void clear_flagged(uint64_t* p) {
    __hip_atomic_store(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float flagged_value(uint64_t w) {
    return __builtin_bit_cast(float, (uint32_t)w);
}

// Reads N flagged words at p[k * stride] (lane-relative) once they are all
// ready: polls at most `polls` times (each about 128 cycles apart); returns
// false, with whatever was read, if some word was still not ready then.
template <int N>
__device__ __forceinline__ bool gather_flagged(const uint64_t* p, int stride, uint32_t polls,
                                               float (&v)[N]) {
    uint64_t w[N];
    for (uint32_t it = 0;; ++it) {
#pragma unroll
        for (int k = 0; k < N; ++k) w[k] = fetch_flagged(p + k * stride);
        bool ok = true;
#pragma unroll
        for (int k = 0; k < N; ++k) ok = ok && (w[k] >> 32) != 0;
        if (__all(ok) || it + 1 >= polls) {
#pragma unroll
            for (int k = 0; k < N; ++k) v[k] = flagged_value(w[k]);
            return __all(ok);
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// Wait until at most N vector-memory instructions of this wave are in flight
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Wait until at most `steps` (0 .. 6, wave-uniform) groups of L vector-memory
// instructions are in flight.
template <int L>
__device__ __forceinline__ void wait_steps(int steps) {
    switch (steps) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<L>(); break;
        case 2: wait_vmcnt<(2 * L < 64 ? 2 * L : 0)>(); break;
        case 3: wait_vmcnt<(3 * L < 64 ? 3 * L : 0)>(); break;
        case 4: wait_vmcnt<(4 * L < 64 ? 4 * L : 0)>(); break;
        case 5: wait_vmcnt<(5 * L < 64 ? 5 * L : 0)>(); break;
        default: wait_vmcnt<(6 * L < 64 ? 6 * L : 0)>(); break;
    }
}

typedef __attribute__((address_space(3))) uint8_t* lds_u8;

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(lds_u8)(p);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16-byte buffer load into registers at voff + soff inside the buffer
// (bytes past its end read as zeros).
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return uint4{t[0], t[1], t[2], t[3]};
}

// Direct HBM -> LDS copies (buffer_load ... lds): every lane fetches 16 (or
// 4) bytes at voff + soff inside the buffer and the wave's 1024 (or 256)
// bytes land contiguously at LDS address `lds` (wave-uniform, through M0).
// Issued as inline assembly so that the compiler neither reorders LDS reads
// around them nor inserts its own conservative wait for every LDS read; the
// kernel waits for them explicitly with wait_vmcnt and orders LDS reuse with
// barriers.
// M0 is a reserved register to the compiler (hence its warning for the
// clobber); it never allocates it, and these kernels contain no instruction
// that reads it other than these loads, each of which sets it first.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                      uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                     uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
// Workgroup barrier that is also a compiler barrier for memory operations
// (it adds no wait for outstanding loads: those are waited for explicitly).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace
}  // namespace nvfp4
