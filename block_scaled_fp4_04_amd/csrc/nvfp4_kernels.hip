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
// Large-M tile kernel.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; workgroup tile BM x BN,
// wave tile (BM/2) x (BN/2) made of 32 x 32 MFMA blocks
// (v_mfma_f32_32x32x16_f16).  K advances in steps of two 64-element panels.
// Each step's packed codes (4 bits/element) and scales are copied from HBM
// to LDS with 16-byte loads; the scales are widened to fp16 on the way.
// LDS holds two such steps (double buffer): the next step's loads are in
// flight while the current one is decoded and multiplied.
//
// LDS code layout of one operand and panel: rows in groups of 32; within a
// group, first the low 16 bytes of the 32 rows, then the high 16 bytes:
//   offset(row, half) = (row / 32) * 1024 + half * 512 + (row % 32) * 16.
// MFMA lane l reads row l % 32, half l / 32 as one 16-byte read, so the 16
// lanes of each LDS phase touch 256 consecutive bytes.
// LDS scale layout: fp16 [panel][row][4 blocks].
//
// Split-K (split_k > 1): the K steps are divided into split_k contiguous
// ranges; each workgroup stores its FP32 tile to the workspace, and the last
// of a tile's workgroups to arrive (atomic counter) adds the partial tiles in
// split order (deterministic) and runs the epilogue.
// ---------------------------------------------------------------------------
template <int BM, int BN>
__global__ void __launch_bounds__(256, 1) tile_kernel(GemmArgs a) {
    constexpr int MI = BM / 64;  // 32-row blocks per wave
    constexpr int NI = BN / 64;  // 32-column blocks per wave
    constexpr int A_CODE = 2 * BM * 32;
    constexpr int B_CODE = 2 * BN * 32;
    constexpr int A_SC = 2 * BM * 8;
    constexpr int B_SC = 2 * BN * 8;
    constexpr int BUF = A_CODE + B_CODE + A_SC + B_SC;
    constexpr int CODE_CHUNKS = 4 * (BM + BN);  // 16-byte chunks per step
    constexpr int CPT = CODE_CHUNKS / 256;      // per thread
    constexpr int A_CPT = (4 * BM) / 256;       // first A_CPT chunks are A
    constexpr int SC_CHUNKS = (BM + BN) / 2;    // 16-byte scale chunks per step
    static_assert(CODE_CHUNKS % 256 == 0 && SC_CHUNKS <= 256, "tile shape");

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane & 31, h = lane >> 5;

    // Workgroup -> (tile, split).  Consecutive workgroup ids are dealt to the
    // eight XCDs in turn; remap so that each XCD gets a contiguous range of
    // tiles, then walk tiles in groups of 8 along M for L2 reuse.
    int bid = blockIdx.x;
    const int total = gridDim.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int S = a.split_k;
    const int z = bid % S;
    const int t = bid / S;
    constexpr int GROUP_M = 8;
    const int in_group = GROUP_M * a.tiles_n;
    const int first_m = (t / in_group) * GROUP_M;
    const int gsize = min(a.tiles_m - first_m, GROUP_M);
    const int tm = first_m + (t % in_group) % gsize;
    const int tn = (t % in_group) / gsize;
    const int m0 = tm * BM, n0 = tn * BN;

    const int nst = (a.P + 1) / 2;
    const int st0 = (int)((int64_t)z * nst / S);
    const int st1 = (int)((int64_t)(z + 1) * nst / S);

    // Per-thread copy plan (constant over K steps).
    int c_row[CPT], c_half[CPT], c_pl[CPT], c_lds[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + 256 * j;
        const bool isA = j < A_CPT;
        const int R = isA ? BM : BN;
        const int cc = isA ? c : c - 4 * BM;
        c_pl[j] = cc / (2 * R);
        const int rem = cc % (2 * R);
        c_row[j] = rem >> 1;
        c_half[j] = rem & 1;
        c_lds[j] = (isA ? 0 : A_CODE) + c_pl[j] * R * 32 + (c_row[j] >> 5) * 1024 +
                   c_half[j] * 512 + (c_row[j] & 31) * 16;
    }
    const bool sc_active = tid < SC_CHUNKS;
    const bool sc_isA = tid < BM / 2;
    const int sc_c = sc_isA ? tid : tid - BM / 2;
    const int sc_R = sc_isA ? BM : BN;
    const int sc_pl = sc_c / (sc_R / 4);
    const int sc_row = 4 * (sc_c % (sc_R / 4));
    const int sc_lds = A_CODE + B_CODE + (sc_isA ? 0 : A_SC) + (sc_pl * sc_R + sc_row) * 8;

    uint4 pre[CPT];
    uint4 pre_sc = {0u, 0u, 0u, 0u};

    auto load_step = [&](int st) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const bool isA = j < A_CPT;
            const int panel = 2 * st + c_pl[j];
            const int row = (isA ? m0 : n0) + c_row[j];
            const int Rp = isA ? a.Mp : a.Np;
            const uint8_t* base = isA ? a.a_codes : a.b_codes;
            uint4 v = {0u, 0u, 0u, 0u};
            if (panel < a.P && row < Rp)
                v = *reinterpret_cast<const uint4*>(
                    base + ((int64_t)panel * Rp + row) * 32 + c_half[j] * 16);
            pre[j] = v;
        }
        if (sc_active) {
            const int panel = 2 * st + sc_pl;
            const int row = (sc_isA ? m0 : n0) + sc_row;
            const int Rp = sc_isA ? a.Mp : a.Np;
            const uint8_t* base = sc_isA ? a.a_scales : a.b_scales;
            uint4 v = {0u, 0u, 0u, 0u};
            if (panel < a.P && row < Rp)
                v = *reinterpret_cast<const uint4*>(base + ((int64_t)panel * Rp + row) * 4);
            pre_sc = v;
        }
    };
    auto store_step = [&](int buf) {
        uint8_t* b = lds + buf * BUF;
#pragma unroll
        for (int j = 0; j < CPT; ++j) *reinterpret_cast<uint4*>(b + c_lds[j]) = pre[j];
        if (sc_active) {
            h2 s[8];
            s[0] = e4m3x2_lo(pre_sc.x); s[1] = e4m3x2_hi(pre_sc.x);
            s[2] = e4m3x2_lo(pre_sc.y); s[3] = e4m3x2_hi(pre_sc.y);
            s[4] = e4m3x2_lo(pre_sc.z); s[5] = e4m3x2_hi(pre_sc.z);
            s[6] = e4m3x2_lo(pre_sc.w); s[7] = e4m3x2_hi(pre_sc.w);
            uint4 w0, w1;
            w0.x = __builtin_bit_cast(uint32_t, s[0]); w0.y = __builtin_bit_cast(uint32_t, s[1]);
            w0.z = __builtin_bit_cast(uint32_t, s[2]); w0.w = __builtin_bit_cast(uint32_t, s[3]);
            w1.x = __builtin_bit_cast(uint32_t, s[4]); w1.y = __builtin_bit_cast(uint32_t, s[5]);
            w1.z = __builtin_bit_cast(uint32_t, s[6]); w1.w = __builtin_bit_cast(uint32_t, s[7]);
            *reinterpret_cast<uint4*>(b + sc_lds) = w0;
            *reinterpret_cast<uint4*>(b + sc_lds + 16) = w1;
        }
    };

    f16v acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    if (st0 < st1) {
        load_step(st0);
        store_step(0);
        __syncthreads();
    }
    for (int st = st0; st < st1; ++st) {
        const int buf = (st - st0) & 1;
        const bool more = st + 1 < st1;
        if (more) load_step(st + 1);
        const uint8_t* b = lds + buf * BUF;
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
            uint4 ca[MI], cb[NI];
            h2 sa[MI], sb[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int g = wm * MI + i;
                ca[i] = *reinterpret_cast<const uint4*>(b + pl * BM * 32 + g * 1024 + h * 512 +
                                                        q * 16);
                sa[i] = *reinterpret_cast<const h2*>(b + A_CODE + B_CODE +
                                                     (pl * BM + g * 32 + q) * 8 + h * 4);
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int g = wn * NI + j;
                cb[j] = *reinterpret_cast<const uint4*>(b + A_CODE + pl * BN * 32 + g * 1024 +
                                                        h * 512 + q * 16);
                sb[j] = *reinterpret_cast<const h2*>(b + A_CODE + B_CODE + A_SC +
                                                     (pl * BN + g * 32 + q) * 8 + h * 4);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                h8 av[MI], bv[NI];
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    av[i] = decode8(word_of(ca[i], s), s < 2 ? sa[i][0] : sa[i][1]);
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    bv[j] = decode8(word_of(cb[j], s), s < 2 ? sb[j][0] : sb[j][1]);
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j],
                                                                           acc[i][j], 0, 0, 0);
            }
        }
        if (more) store_step(buf ^ 1);
        __syncthreads();
    }

    // Split-K: publish the partial tile; the last arrival reduces.
    if (S > 1) {
        float* mine = a.partials + ((int64_t)t * S + z) * (BM * BN);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) mine[((i * NI + j) * 16 + v) * 256 + tid] = acc[i][j][v];
        __threadfence();
        __syncthreads();
        __shared__ int s_last;
        if (tid == 0) {
            const uint32_t old = atomicAdd(a.counters + t, 1u);
            s_last = (old == (uint32_t)(S - 1));
            if (s_last) a.counters[t] = 0u;  // every split has arrived: reset for the next call
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        const float* all = a.partials + (int64_t)t * S * (BM * BN);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int idx = ((i * NI + j) * 16 + v) * 256 + tid;
                    float sum = 0.0f;
                    for (int zz = 0; zz < S; ++zz)
                        sum += (zz == z) ? acc[i][j][v] : all[(int64_t)zz * (BM * BN) + idx];
                    acc[i][j][v] = sum;
                }
    }

    // Epilogue: y = alpha * acc (FP32), bfloat16 round-to-nearest-even.
    // 32x32 MFMA result layout: lane l holds column l % 32 and rows
    // 8 * (v / 4) + 4 * (l / 32) + v % 4 of its block.
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = n0 + wn * (BN / 2) + j * 32 + q;
            if (col >= a.N) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                if (row < a.M) a.out[(int64_t)row * a.N + col] = to_bf16(a.alpha * acc[i][j][v]);
            }
        }
}

// ---------------------------------------------------------------------------
// Skinny-M kernel (M <= 16), for decode-sized GEMMs that are bound by
// streaming B from HBM.
//
// v_mfma_f32_16x16x32_f16 with the (zero-padded) 16 rows of A as the MFMA A
// operand and 16 rows of B as the B operand.  Work unit: 16 B rows x 128 K
// (two panels).  Lane l holds row l % 16 and, with g = l / 16, the 16-byte
// half (g % 2) of panel (g / 2): one 16-byte load of codes and one 2-byte
// load of scales per operand, straight from HBM (B is used once, so it does
// not pass through LDS).  Each MFMA sub-step s takes word s of every lane.
//
// Grid: (N / 16 row groups) x split_k workgroups of 4 waves; a workgroup
// owns one row group and a contiguous range of work units, dealt to its
// waves in turn.  The 4 wave partials are added in LDS (fixed order), then
// across workgroups through the workspace by the last arrival (fixed order).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) skinny_kernel(GemmArgs a) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int S = a.split_k;
    const int g = blockIdx.x / S;
    const int z = blockIdx.x % S;
    const int C = (a.P + 1) / 2;
    const int c0 = (int)((int64_t)z * C / S);
    const int c1 = (int)((int64_t)(z + 1) * C / S);
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int pl = grp >> 1, half = grp & 1;
    const int nrow = g * 16 + r16;

    f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = c0 + wave; c < c1; c += 4) {
        const int panel = 2 * c + pl;
        uint4 bw = {0u, 0u, 0u, 0u}, aw = {0u, 0u, 0u, 0u};
        uint32_t bs = 0u, as = 0u;
        if (panel < a.P) {
            const int64_t bo = (int64_t)panel * a.Np + nrow;
            const int64_t ao = (int64_t)panel * a.Mp + r16;
            bw = *reinterpret_cast<const uint4*>(a.b_codes + bo * 32 + half * 16);
            bs = *reinterpret_cast<const uint16_t*>(a.b_scales + bo * 4 + half * 2);
            aw = *reinterpret_cast<const uint4*>(a.a_codes + ao * 32 + half * 16);
            as = *reinterpret_cast<const uint16_t*>(a.a_scales + ao * 4 + half * 2);
        }
        const h2 sbh = e4m3x2_lo(bs);
        const h2 sah = e4m3x2_lo(as);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const h8 av = decode8(word_of(aw, s), s < 2 ? sah[0] : sah[1]);
            const h8 bv = decode8(word_of(bw, s), s < 2 ? sbh[0] : sbh[1]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
        }
    }

    __shared__ f4v red[4][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    f4v sum = red[0][lane];
    sum += red[1][lane];
    sum += red[2][lane];
    sum += red[3][lane];

    if (S > 1) {
        float* mine = a.partials + ((int64_t)g * S + z) * 256;
#pragma unroll
        for (int v = 0; v < 4; ++v) mine[v * 64 + lane] = sum[v];
        __threadfence();
        uint32_t old = 0;
        if (lane == 0) old = atomicAdd(a.counters + g, 1u);
        old = __shfl(old, 0);
        if (old != (uint32_t)(S - 1)) return;
        if (lane == 0) a.counters[g] = 0u;  // every split has arrived: reset for the next call
        __threadfence();
        const float* all = a.partials + (int64_t)g * S * 256;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float t = 0.0f;
            for (int zz = 0; zz < S; ++zz) t += (zz == z) ? sum[v] : all[zz * 256 + v * 64 + lane];
            sum[v] = t;
        }
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
    switch (cfg) {
        case TILE_256x256: hipLaunchKernelGGL((tile_kernel<256, 256>), grid, block, 0, stream, a); break;
        case TILE_128x128: hipLaunchKernelGGL((tile_kernel<128, 128>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((tile_kernel<64, 64>), grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.Np / 16) * a.split_k));
    hipLaunchKernelGGL(skinny_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4
