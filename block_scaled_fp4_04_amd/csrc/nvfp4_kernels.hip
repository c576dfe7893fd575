// nvfp4_kernels.hip -- gfx950 (CDNA4) kernels of the NVFP4 block-scaled GEMM
//
//   C[m][n] = bf16_rne(alpha * sum_k a'[m][k] * b'[n][k]),
//   a'[m][k] = e2m1(A code) * e4m3(A scale of block k/16), likewise b'.
//
// Two FP4 codes per byte and one FP8 scale per 16 elements follow "Peeling
// the Kernel Onion", section "The Benchmark Design"; alpha and the output
// tensor follow the same page, section "The Chain of Reasoning".
//
// Exactness: every a' = code * scale has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in fp16; fp16 x fp16 products are exact in
// the FP32 accumulator of the fp16 MFMA.  The decode is therefore exact:
//   v_cvt_scalef32_pk_f16_fp4 (scale 1.0) turns two codes into two fp16,
//   v_pk_mul_f16 multiplies them by the block's fp16 scale (exact product).
// (The hardware scale operand of the FP4 converts only applies the scale's
// exponent, so it cannot carry an E4M3 scale by itself.)
//
// K-slot freedom: a dot product does not depend on the order of its terms,
// so the kernels feed MFMA K-slots with whatever elements make the loads
// contiguous, as long as A and B lanes agree and each 8-element group stays
// inside one 16-element scale block.
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
__device__ __forceinline__ h8 decode8(uint32_t w, _Float16 s) {
    const h2 ss = {s, s};
    const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    return h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// FP32 -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t to_bf16(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int s) {
    return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
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

// Wait until at most N vector-memory instructions of this wave are in flight
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

typedef __attribute__((address_space(3))) uint8_t* lds_u8;

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(lds_u8)(p);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Direct HBM -> LDS copies (buffer_load ... lds): every lane fetches 16 (or
// 4) bytes at voff + soff inside the buffer and the wave's 1024 (or 256)
// bytes land contiguously at LDS address `lds` (wave-uniform, through M0).
// Issued as inline assembly so that the compiler neither reorders LDS reads
// around them nor inserts its own conservative wait for every LDS read; the
// kernel waits for them explicitly with wait_vmcnt and orders LDS reuse with
// barriers.
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
// Workgroup barrier that is also a compiler barrier for memory operations
// (it adds no wait for outstanding loads: those are waited for explicitly).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Large-M tile kernel.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; workgroup tile BM x BN,
// wave tile (BM/2) x (BN/2) made of 32 x 32 MFMA blocks
// (v_mfma_f32_32x32x16_f16).  K advances in steps of two 64-element panels.
//
// HBM -> LDS: each step's packed codes (4 bits/element) and raw E4M3 scale
// bytes are copied with direct-to-LDS loads (16 and 4 bytes per lane) into a
// ring of NS stage buffers, NS-1 steps ahead of the step being multiplied, so
// several steps of loads are always in flight and no VGPRs are spent on
// staging.
//
// LDS code layout of one operand and panel: rows in groups of 32; within a
// group, first the low 16 bytes of the 32 rows, then the high 16 bytes
// (one 1 KB direct load per group):
//   offset(row, half) = (row / 32) * 1024 + half * 512 + (row % 32) * 16.
// MFMA lane l reads row l % 32, half l / 32 as one 16-byte read, so the lanes
// of each LDS phase touch consecutive bytes.  Scales: [panel][row][4 bytes].
//
// Decode and MFMA are software-pipelined: the operands of sub-step s+1 are
// decoded while the 16 MFMAs of sub-step s run, with the instruction
// scheduler told to alternate one MFMA and a few VALU instructions.
//
// Rows past the padded operand are clamped to its last row (their results
// are never stored).  The packed K is a whole number of steps (the packer
// pads with zeros), so every step holds two panels.
//
// Split-K (split_k > 1): the K steps are divided into split_k contiguous
// ranges; each workgroup publishes its FP32 tile to the workspace, and the
// last of a tile's workgroups to arrive adds the partial tiles in split order
// (deterministic) and runs the epilogue.
// ---------------------------------------------------------------------------
template <int BM, int BN, int NS, bool SPLIT>
__global__ void __launch_bounds__(256, 1) tile_kernel(GemmArgs a) {
    constexpr int MI = BM / 64;  // 32-row blocks per wave
    constexpr int NI = BN / 64;  // 32-column blocks per wave
    constexpr int A_CODE = 2 * BM * 32;
    constexpr int B_CODE = 2 * BN * 32;
    constexpr int A_SC = 2 * BM * 4;
    constexpr int B_SC = 2 * BN * 4;
    constexpr int OFF_B = A_CODE;
    constexpr int OFF_SA = A_CODE + B_CODE;
    constexpr int OFF_SB = OFF_SA + A_SC;
    constexpr int STAGE = OFF_SB + B_SC;
    constexpr int A_CCH = 2 * BM / 32;           // 1 KB code chunks of A per step
    constexpr int CCH = A_CCH + 2 * BN / 32;
    constexpr int A_SCH = 2 * BM / 64;           // 256 B scale chunks of A per step
    constexpr int SCH = A_SCH + 2 * BN / 64;
    static_assert(CCH % 4 == 0 && SCH % 4 == 0, "chunks must split evenly over 4 waves");
    constexpr int LPS = CCH / 4 + SCH / 4;       // direct loads per wave per step
    static_assert(NS >= 3 && NS <= 4 && (NS - 2) * LPS < 64, "pipeline depth");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane & 31, h = lane >> 5;

    // Workgroup -> (tile, split).  Consecutive workgroup ids are dealt to the
    // eight XCDs in turn; remap so that each XCD gets a contiguous range of
    // tiles, then walk tiles in groups of 8 along M for L2 reuse.
    int bid = blockIdx.x;
    const int total = gridDim.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int S = SPLIT ? a.split_k : 1;
    const int z = bid % S;
    const int t = bid / S;
    constexpr int GROUP_M = 8;
    const int in_group = GROUP_M * a.tiles_n;
    const int first_m = (t / in_group) * GROUP_M;
    const int gsize = min(a.tiles_m - first_m, GROUP_M);
    const int tm = first_m + (t % in_group) % gsize;
    const int tn = (t % in_group) / gsize;
    const int m0 = tm * BM, n0 = tn * BN;

    const int nst = a.P / 2;
    const int st0 = (int)((int64_t)z * nst / S);
    const int st1 = (int)((int64_t)(z + 1) * nst / S);

    const uint32_t lds0 = lds_addr(lds);

    // Direct-load plan of this wave (constant over K steps): for each of its
    // code and scale chunks, the lane's byte offset inside a panel and the
    // chunk's place in the stage buffer.
    const __amdgpu_buffer_rsrc_t rac = make_rsrc(a.a_codes, (uint32_t)a.P * a.Mp * 32u);
    const __amdgpu_buffer_rsrc_t rbc = make_rsrc(a.b_codes, (uint32_t)a.P * a.Np * 32u);
    const __amdgpu_buffer_rsrc_t ras = make_rsrc(a.a_scales, (uint32_t)a.P * a.Mp * 4u);
    const __amdgpu_buffer_rsrc_t rbs = make_rsrc(a.b_scales, (uint32_t)a.P * a.Np * 4u);
    uint32_t c_voff[CCH / 4], s_voff[SCH / 4];
#pragma unroll
    for (int i = 0; i < CCH / 4; ++i) {
        const int k = wave + 4 * i;
        const bool isA = k < A_CCH;
        const int R = isA ? BM : BN;
        const int grp = (isA ? k : k - A_CCH) % (R / 32);
        const int row = min((isA ? m0 : n0) + grp * 32 + q, (isA ? a.Mp : a.Np) - 1);
        c_voff[i] = (uint32_t)row * 32u + (uint32_t)h * 16u;
    }
#pragma unroll
    for (int i = 0; i < SCH / 4; ++i) {
        const int k = wave + 4 * i;
        const bool isA = k < A_SCH;
        const int R = isA ? BM : BN;
        const int c = (isA ? k : k - A_SCH) % (R / 64);
        const int row = min((isA ? m0 : n0) + c * 64 + lane, (isA ? a.Mp : a.Np) - 1);
        s_voff[i] = (uint32_t)row * 4u;
    }

    // Issue the direct loads of step st into stage buffer sb (LPS per wave).
    auto issue = [&](int st, int sb) {
        const uint32_t b = lds0 + (uint32_t)(sb * STAGE);
#pragma unroll
        for (int i = 0; i < CCH / 4; ++i) {
            const int k = wave + 4 * i;
            const bool isA = k < A_CCH;
            const int R = isA ? BM : BN;
            const int kk = isA ? k : k - A_CCH;
            const int pl = kk / (R / 32), grp = kk % (R / 32);
            const uint32_t panel = (uint32_t)(2 * st + pl);
            const uint32_t soff = panel * (uint32_t)(isA ? a.Mp : a.Np) * 32u;
            dma16(isA ? rac : rbc, c_voff[i], soff,
                  b + (uint32_t)((isA ? 0 : OFF_B) + (pl * (R / 32) + grp) * 1024));
        }
#pragma unroll
        for (int i = 0; i < SCH / 4; ++i) {
            const int k = wave + 4 * i;
            const bool isA = k < A_SCH;
            const int R = isA ? BM : BN;
            const int kk = isA ? k : k - A_SCH;
            const int pl = kk / (R / 64), c = kk % (R / 64);
            const uint32_t panel = (uint32_t)(2 * st + pl);
            const uint32_t soff = panel * (uint32_t)(isA ? a.Mp : a.Np) * 4u;
            dma4(isA ? ras : rbs, s_voff[i], soff,
                 b + (uint32_t)((isA ? OFF_SA : OFF_SB) + (pl * R + c * 64) * 4));
        }
    };

    f16v acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // Multiply one step (two panels) held in buffer b.
    auto compute = [&](const uint8_t* b) {
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
            uint4 ca[MI], cb[NI];
            h2 sa[MI], sb[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int g = wm * MI + i;
                ca[i] = *reinterpret_cast<const uint4*>(b + pl * BM * 32 + g * 1024 + h * 512 + q * 16);
                const uint32_t raw = *reinterpret_cast<const uint16_t*>(
                    b + OFF_SA + (pl * BM + g * 32 + q) * 4 + h * 2);
                sa[i] = e4m3x2_lo(raw);
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int g = wn * NI + j;
                cb[j] = *reinterpret_cast<const uint4*>(b + OFF_B + pl * BN * 32 + g * 1024 + h * 512 + q * 16);
                const uint32_t raw = *reinterpret_cast<const uint16_t*>(
                    b + OFF_SB + (pl * BN + g * 32 + q) * 4 + h * 2);
                sb[j] = e4m3x2_lo(raw);
            }
            h8 av[2][MI], bv[2][NI];
#pragma unroll
            for (int i = 0; i < MI; ++i) av[0][i] = decode8(word_of(ca[i], 0), sa[i][0]);
#pragma unroll
            for (int j = 0; j < NI; ++j) bv[0][j] = decode8(word_of(cb[j], 0), sb[j][0]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int cur = s & 1, nxt = cur ^ 1;
                if (s < 3) {
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        av[nxt][i] = decode8(word_of(ca[i], s + 1), (s + 1) < 2 ? sa[i][0] : sa[i][1]);
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        bv[nxt][j] = decode8(word_of(cb[j], s + 1), (s + 1) < 2 ? sb[j][0] : sb[j][1]);
                }
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[cur][i], bv[cur][j],
                                                                           acc[i][j], 0, 0, 0);
                if (s < 3) {
#pragma unroll
                    for (int m = 0; m < MI * NI; ++m) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, (8 * (MI + NI) + MI * NI - 1) / (MI * NI), 0);
                    }
                }
            }
        }
    };

    // Prologue: NS-1 steps in flight.
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
        if (st0 + u < st1) issue(st0 + u, u);

    int sb = 0;  // stage buffer of step st
    for (int st = st0; st < st1; ++st) {
        // Loads issued after step st's: steps st+1 .. min(st+NS-2, st1-1).
        const int later = min(NS - 2, st1 - 1 - st);
        if (later >= 2) wait_vmcnt<2 * LPS>();
        else if (later == 1) wait_vmcnt<LPS>();
        else wait_vmcnt<0>();
        wg_barrier();  // step st is in LDS; step st-1's buffer is free
        if (st + NS - 1 < st1) issue(st + NS - 1, sb == 0 ? NS - 1 : sb - 1);
        compute(lds + sb * STAGE);
        sb = sb == NS - 1 ? 0 : sb + 1;
    }

    // Split-K: publish the partial tile; the last arrival reduces in split order.
    if (SPLIT) {
        float* mine = a.partials + ((int64_t)t * S + z) * (BM * BN);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    publish(mine + ((i * NI + j) * 16 + v) * 256 + tid, acc[i][j][v]);
        __shared__ int s_last;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = arrive(a.counters + t);
            s_last = (old == (uint32_t)(S - 1));
            if (s_last) reset_counter(a.counters + t);  // all splits arrived
        }
        __syncthreads();
        if (!s_last) return;
        const float* all = a.partials + (int64_t)t * S * (BM * BN);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
        for (int zz = 0; zz < S; ++zz) {
            const float* pz = all + (int64_t)zz * (BM * BN);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[i][j][v] += fetch(pz + ((i * NI + j) * 16 + v) * 256 + tid);
        }
    }

    // Epilogue: y = alpha * acc (FP32), bfloat16 round-to-nearest-even.
    // 32x32 MFMA result layout: lane l holds column l % 32 and rows
    // 8 * (v / 4) + 4 * (l / 32) + v % 4 of its block.
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            // one 32 x 32 block at a time keeps few accumulators in VGPRs
            __builtin_amdgcn_sched_barrier(0);
            const int col = n0 + wn * (BN / 2) + j * 32 + q;
            if (col < a.N) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (row < a.M) a.out[(int64_t)row * a.N + col] = to_bf16(a.alpha * acc[i][j][v]);
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Skinny-M kernel (M <= 16), for decode-sized GEMMs that are bound by
// streaming B from HBM and by latency.
//
// v_mfma_f32_16x16x32_f16 with the (zero-padded) 16 rows of A as the MFMA A
// operand and 16 rows of B as the B operand.  Work unit: 16 B rows x 128 K
// (two panels).  Lane l holds row l % 16 and, with g = l / 16, the 16-byte
// half (g % 2) of panel (g / 2): one 16-byte load of codes and one 2-byte
// load of scales per operand, straight from HBM (B is used once, so it does
// not pass through LDS).  Each MFMA sub-step s takes word s of every lane.
// Lanes whose A row is at or beyond M skip their A loads (zeros).
//
// Grid: (N / 16 row groups) x split_k workgroups of WAVES waves; a
// workgroup owns one row group and a contiguous range of work units, dealt
// to its waves in turn; each wave issues the loads of up to UNITS work units
// before it waits, so one memory round trip covers them.  The wave partials
// are added in LDS in wave order; with split_k > 1 the workgroup partials
// are added by the last arrival in split order (deterministic).
// ---------------------------------------------------------------------------
template <int WAVES>
__global__ void __launch_bounds__(WAVES * 64) skinny_kernel(GemmArgs a) {
    constexpr int UNITS = 4;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int S = a.split_k;
    const int g = blockIdx.x / S;
    const int z = blockIdx.x % S;
    const int C = a.P / 2;
    const int c0 = (int)((int64_t)z * C / S);
    const int c1 = (int)((int64_t)(z + 1) * C / S);
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int pl = grp >> 1, half = grp & 1;
    const int nrow = g * 16 + r16;
    const bool a_row = r16 < a.M;

    f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int base = c0 + wave; base < c1; base += WAVES * UNITS) {
        uint4 bw[UNITS], aw[UNITS];
        uint32_t bs[UNITS], as[UNITS];
#pragma unroll
        for (int u = 0; u < UNITS; ++u) {
            const int c = base + WAVES * u;
            const int panel = 2 * c + pl;
            bw[u] = uint4{0u, 0u, 0u, 0u};
            aw[u] = uint4{0u, 0u, 0u, 0u};
            bs[u] = 0u;
            as[u] = 0u;
            if (c < c1 && panel < a.P) {
                const int64_t bo = (int64_t)panel * a.Np + nrow;
                bw[u] = *reinterpret_cast<const uint4*>(a.b_codes + bo * 32 + half * 16);
                bs[u] = *reinterpret_cast<const uint16_t*>(a.b_scales + bo * 4 + half * 2);
                if (a_row) {
                    const int64_t ao = (int64_t)panel * a.Mp + r16;
                    aw[u] = *reinterpret_cast<const uint4*>(a.a_codes + ao * 32 + half * 16);
                    as[u] = *reinterpret_cast<const uint16_t*>(a.a_scales + ao * 4 + half * 2);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UNITS; ++u) {
            const h2 sbh = e4m3x2_lo(bs[u]);
            const h2 sah = e4m3x2_lo(as[u]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const h8 av = decode8(word_of(aw[u], s), s < 2 ? sah[0] : sah[1]);
                const h8 bv = decode8(word_of(bw[u], s), s < 2 ? sbh[0] : sbh[1]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
            }
        }
    }

    __shared__ f4v red[WAVES][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    f4v sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[w][lane];

    if (S > 1) {
        float* mine = a.partials + ((int64_t)g * S + z) * 256;
#pragma unroll
        for (int v = 0; v < 4; ++v) publish(mine + v * 64 + lane, sum[v]);
        uint32_t old = 0;
        if (lane == 0) old = arrive(a.counters + g);
        old = __shfl(old, 0);
        if (old != (uint32_t)(S - 1)) return;
        if (lane == 0) reset_counter(a.counters + g);  // all splits arrived
        const float* all = a.partials + (int64_t)g * S * 256;
        f4v t = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int zz = 0; zz < S; ++zz) {
            f4v p;
#pragma unroll
            for (int v = 0; v < 4; ++v) p[v] = fetch(all + zz * 256 + v * 64 + lane);
            t += p;
        }
        sum = t;
    }

    // 16x16 MFMA result layout: lane l holds column l % 16, rows 4 * (l / 16) + v.
    const int col = g * 16 + r16;
    if (col < a.N) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 4 * grp + v;
            if (row < a.M) a.out[(int64_t)row * a.N + col] = to_bf16(a.alpha * sum[v]);
        }
    }
}

}  // namespace

size_t tile_partial_floats(int cfg, const GemmArgs& a) {
    if (a.split_k <= 1) return 0;
    const TileShape s = tile_shape(cfg);
    return (size_t)a.tiles_m * a.tiles_n * a.split_k * s.bm * s.bn;
}
size_t tile_counters(int cfg, const GemmArgs& a) {
    (void)cfg;
    return a.split_k <= 1 ? 0 : (size_t)a.tiles_m * a.tiles_n;
}
size_t skinny_partial_floats(const GemmArgs& a) {
    return a.split_k <= 1 ? 0 : (size_t)(a.Np / 16) * a.split_k * 256;
}
size_t skinny_counters(const GemmArgs& a) {
    return a.split_k <= 1 ? 0 : (size_t)(a.Np / 16);
}

hipError_t launch_tile(int cfg, const GemmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n * a.split_k));
    const dim3 block(256);
    const bool split = a.split_k > 1;
    switch (cfg) {
        case TILE_256x256:
            if (split) hipLaunchKernelGGL((tile_kernel<256, 256, 4, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((tile_kernel<256, 256, 4, false>), grid, block, 0, stream, a);
            break;
        case TILE_128x128:
            if (split) hipLaunchKernelGGL((tile_kernel<128, 128, 4, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((tile_kernel<128, 128, 4, false>), grid, block, 0, stream, a);
            break;
        default:
            if (split) hipLaunchKernelGGL((tile_kernel<64, 64, 4, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((tile_kernel<64, 64, 4, false>), grid, block, 0, stream, a);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.Np / 16) * a.split_k));
    hipLaunchKernelGGL(skinny_kernel<kSkinnyWaves>, grid, dim3(kSkinnyWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4
