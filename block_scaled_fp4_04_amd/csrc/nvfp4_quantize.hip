// nvfp4_quantize.hip -- gfx950 kernel that quantises fp32 rows to NVFP4
// straight into the packed operand layout the GEMM kernels read.
//
// Per 16-element block of a row (the format of "Peeling the Kernel Onion",
// section "The Benchmark Design": E2M1 codes two per byte, one FP8 E4M3
// scale per 16 elements; the recipe is "scale = E4M3(amax / 6), codes =
// round-to-nearest-even E2M1"):
//   scale byte = E4M3 value nearest to fp32(amax / 6), ties to the even byte,
//                saturating at 448;
//   code       = E2M1 magnitude nearest to fp32(x / scale), ties to the even
//                code, saturating at 6, with the sign bit of x; a block whose
//                scale is 0 keeps only the sign bits.
// amax / 6 is a single correctly rounded fp32 division.  The codes need
// only the side of each rounding boundary on which fp32(|x| / scale) falls,
// which is decided exactly by comparing |x| with boundary * scale (see
// e2m1_code below), without dividing.
//
// The input is fp32 or bfloat16; a bfloat16 value is widened to the fp32
// value it equals (its bits shifted up by 16), so both quantise alike.
//
// Lanes: every lane reads 32 contiguous bytes of a row-panel (64 elements =
// 4 blocks): 8 fp32 values, two lanes per block, whose amax is combined
// across the pair; or 16 bfloat16 values, one lane per block.  A lane writes
// the code bytes of its elements and the first lane of a block its scale
// byte.  Consecutive lanes take consecutive blocks and rows of a panel
// (grid x), so the loads and stores of a wave are contiguous; each lane
// walks a strided set of panels (grid y), with the next panel's loads in
// flight while it quantises the current one.  Padding rows and panels are
// written as zeros.
#include "nvfp4_internal.h"
#include "nvfp4_quant_device.h"

#include <algorithm>

namespace nvfp4 {
namespace {

// Elements per lane: 32 bytes of input.
template <typename T>
constexpr int kQuantEpl = 32 / (int)sizeof(T);

// (Plain arguments, so that they are preloaded into scalar registers before
// the waves start.)  T: float or uint16_t (bfloat16 bits).
template <typename T>
__global__ void __launch_bounds__(256) quantize_kernel(const T* __restrict__ x, int64_t ld,
                                                       int rows, int K, int Rp, int P,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
    constexpr int EPL = kQuantEpl<T>;  // 8 (fp32) or 16 (bfloat16)
    constexpr int LPR = 64 / EPL;      // lanes per row-panel: 8 or 4
    constexpr int W = EPL / 8;         // code words (8 codes each) per lane
    // grid: x covers the padded rows of a panel (LPR lanes per row); the
    // lane walks panels blockIdx.y, + gridDim.y, ..., loading the next one
    // while it quantises the current one
    const int t = (int)blockIdx.x * 256 + (int)threadIdx.x;
    const int r = t / LPR;
    const int j = t % LPR;                          // lane within the row-panel
    const int blk = j * EPL / 16;
    const int half = EPL == 8 ? (j & 1) : 0;        // which 8 of the block (fp32)
    const bool live = r < Rp;                       // whole LPR-lane groups live or not
    const bool row_has = live && r < rows;
    // The loads are unconditional, clamped into the input (the row to the
    // last one, the lane's elements to end by K): values read for a padding
    // row or past K only feed blocks that are written as zeros.  Without a
    // branch around them the compiler waits for each panel's loads alone.
    // QD panels in flight per lane (the one being quantised included): 3 or
    // 4, and non-temporal loads, measured 2-13% slower (fp32).
    const T* xrow = x + (int64_t)min(r, rows - 1) * ld;
    auto load = [&](int p, float (&v)[EPL]) {
        const int k = min(min(p, P - 1) * 64 + j * EPL, K - EPL);
        const uint4* src = reinterpret_cast<const uint4*>(xrow + k);
        const uint4 q0 = src[0], q1 = src[1];
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        if constexpr (sizeof(T) == 2) {
            // element 2i in the low half of word i
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
                v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(float, w[i]);
        }
    };
    constexpr int QD = 2;
    float ring[QD][EPL];
    int p = (int)blockIdx.y;
#pragma unroll
    for (int d = 0; d < QD - 1; ++d) load(p + d * (int)gridDim.y, ring[d]);
    for (; p < P; p += (int)gridDim.y) {
        load(p + (QD - 1) * (int)gridDim.y, ring[QD - 1]);
        float cur[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) cur[i] = ring[0][i];
        const bool has = row_has && p * 64 + blk * 16 < K;
        // amax (v_max ignores a NaN operand, as the definition's comparison
        // does); with two lanes per block they are an aligned pair: exchange
        // within it (DPP quad permutation 1,0,3,2)
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(cur[i]));
        if constexpr (EPL == 8) {
            const float o = __builtin_bit_cast(
                float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false));
            amax = __builtin_fmaxf(amax, o);
        }
        const uint32_t sb = e4m3_nearest(amax / 6.0f);
        const float s = e4m3_value(sb);
        const E2m1Search q = e2m1_search(s);
        const uint32_t keep = s > 0.0f ? 7u : 0u;   // a block whose scale is 0 keeps only signs
        uint32_t w[W];
#pragma unroll
        for (int c = 0; c < W; ++c) {
            float v8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v8[i] = cur[8 * c + i];
            w[c] = has ? e2m1_word(v8, q, keep) : 0u;
        }
        if (live) {
            const int64_t slot = (int64_t)p * Rp + r;
            uint8_t* dst = codes + slot * 32 + blk * 8 + half * 4;
            if constexpr (W == 1)
                *reinterpret_cast<uint32_t*>(dst) = w[0];
            else
                *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
            if (half == 0) scales[slot * 4 + blk] = has ? (uint8_t)sb : (uint8_t)0;
        }
#pragma unroll
        for (int d = 0; d + 1 < QD; ++d)
#pragma unroll
            for (int i = 0; i < EPL; ++i) ring[d][i] = ring[d + 1][i];
    }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
    // enough workgroups to fill the GPU a few times over; each lane walks
    // P / grid.y panels
    const int lpr = 64 / (a.bf16 ? kQuantEpl<uint16_t> : kQuantEpl<float>);   // lanes per row-panel
    const int gx = (a.Rp * lpr + 255) / 256;
    const int gy = std::max(1, std::min(a.P, (4096 + gx - 1) / gx));
    const dim3 grid((unsigned)gx, (unsigned)gy);
    if (a.bf16)
        hipLaunchKernelGGL(quantize_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(a.x), a.ld, a.rows, a.K, a.Rp, a.P,
                           a.codes, a.scales);
    else
        hipLaunchKernelGGL(quantize_kernel<float>, grid, dim3(256), 0, stream,
                           static_cast<const float*>(a.x), a.ld, a.rows, a.K, a.Rp, a.P,
                           a.codes, a.scales);
    return hipGetLastError();
}

}  // namespace nvfp4
