// nvfp4_grouped.hip -- gfx950 kernel of the grouped NVFP4 GEMM (the experts
// of a mixture-of-experts layer in one launch); decode and epilogue as in
// the single-GEMM kernels (nvfp4_device.h).
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

// ---------------------------------------------------------------------------
// Grouped skinny kernel: the experts of a mixture-of-experts layer in one
// launch.  Group g multiplies rows [offsets[g], offsets[g+1]) of A (tokens
// routed to expert g, typically about 16) by its own weight operand B_g; all
// groups share N and K.  ("Peeling the Kernel Onion", sections "The Critical
// Connection to Real Inference": 256 experts, 8 per token, about 16 tokens
// per expert at 512 requests; "Knowledge Created and Its Impact": grouped
// GEMMs to amortise the per-call overhead.)
//
// Workgroup: NB 16-row blocks of B_g (16 * NB columns of C) over the whole K
// range, WAVES waves splitting the 128-element K units in turn, each with
// the loads of UNITS units in flight (straight from HBM: B is used once).
// A is taken in chunks of 16 rows; up to CH chunks share one pass over B.
// Each A chunk is decoded once per K unit and feeds the
// v_mfma_f32_16x16x32_f16 of all NB blocks (lane layout as in the skinny
// kernel), so the decode of A is shared by 16 * NB columns.  Wave partials
// are added in LDS in wave order.  The workgroups of one group are
// consecutive and are kept on one XCD, so its A rows come from that XCD's L2
// after the first read.  Offsets are clamped to [0, M] on the device, so a
// malformed table cannot make the kernel read or write outside the buffers.
// ---------------------------------------------------------------------------
template <int WAVES, int CH, int UNITS, int NB>
__global__ void __launch_bounds__(WAVES * 64) grouped_kernel(GroupedArgs a) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int bid = blockIdx.x;
    const int total = gridDim.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int blocks = a.Np / 16;                  // 16-row blocks of B per group
    const int wgs = (blocks + NB - 1) / NB;        // workgroups per group
    const int g = bid / wgs;
    const int cb0 = (bid % wgs) * NB;              // first block of this workgroup
    const int nb = min(NB, blocks - cb0);          // blocks of this workgroup
    const int r0 = min(max(a.offsets[g], 0), a.M);
    const int r1 = min(max(a.offsets[g + 1], r0), a.M);
    if (r0 >= r1) return;

    const int C = a.P / 2;  // 128-element K units
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int pl = grp >> 1, half = grp & 1;
    const uint8_t* bc = a.b_codes + (int64_t)g * a.P * a.Np * 32;
    const uint8_t* bsc = a.b_scales + (int64_t)g * a.P * a.Np * 4;

    __shared__ f4v red[WAVES][CH * NB][64];
    for (int m0 = r0; m0 < r1; m0 += 16 * CH) {
        const int nch = min(CH, (r1 - m0 + 15) / 16);
        f4v acc[CH][NB];
#pragma unroll
        for (int ch = 0; ch < CH; ++ch)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[ch][j] = f4v{0.0f, 0.0f, 0.0f, 0.0f};
        for (int base = wave; base < C; base += WAVES * UNITS) {
            uint4 bw[UNITS][NB], aw[UNITS][CH];
            uint32_t bs[UNITS][NB], as[UNITS][CH];
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                const int c = base + WAVES * u;
                const int64_t panel = 2 * (int64_t)c + pl;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    bw[u][j] = uint4{0u, 0u, 0u, 0u};
                    bs[u][j] = 0u;
                    if (c < C && j < nb) {
                        const int64_t bo = panel * a.Np + (cb0 + j) * 16 + r16;
                        // weights are read once per call: non-temporal loads
                        bw[u][j] = load_nt16(bc + bo * 32 + half * 16);
                        bs[u][j] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(bsc + bo * 4 + half * 2));
                    }
                }
#pragma unroll
                for (int ch = 0; ch < CH; ++ch) {
                    aw[u][ch] = uint4{0u, 0u, 0u, 0u};
                    as[u][ch] = 0u;
                    const int row = m0 + ch * 16 + r16;
                    if (c < C && ch < nch && row < r1) {
                        const int64_t ao = panel * a.Mp + row;
                        aw[u][ch] = *reinterpret_cast<const uint4*>(a.a_codes + ao * 32 + half * 16);
                        as[u][ch] = *reinterpret_cast<const uint16_t*>(a.a_scales + ao * 4 + half * 2);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                h2 sbh[NB], sah[CH];
#pragma unroll
                for (int j = 0; j < NB; ++j) sbh[j] = e4m3x2_lo(bs[u][j]);
#pragma unroll
                for (int ch = 0; ch < CH; ++ch) sah[ch] = e4m3x2_lo(as[u][ch]);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    h8 bv[NB];
#pragma unroll
                    for (int j = 0; j < NB; ++j) bv[j] = decode8(word_of(bw[u][j], s), scale_of(sbh[j], s));
#pragma unroll
                    for (int ch = 0; ch < CH; ++ch) {
                        if (ch < nch) {
                            const h8 av = decode8(word_of(aw[u][ch], s), scale_of(sah[ch], s));
#pragma unroll
                            for (int j = 0; j < NB; ++j)
                                acc[ch][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv[j], acc[ch][j], 0, 0, 0);
                        }
                    }
                }
            }
        }

        // Add the wave partials in wave order; wave w finishes the (chunk,
        // block) pairs w, w + WAVES, ...
        __syncthreads();  // the previous pass's reads of red are done
#pragma unroll
        for (int ch = 0; ch < CH; ++ch)
#pragma unroll
            for (int j = 0; j < NB; ++j) red[wave][ch * NB + j][lane] = acc[ch][j];
        __syncthreads();
        for (int idx = wave; idx < nch * NB; idx += WAVES) {
            const int ch = idx / NB, j = idx % NB;
            if (j >= nb) continue;
            f4v sum = red[0][idx][lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) sum += red[w][idx][lane];
            // 16x16 MFMA result layout: lane l holds column l % 16, rows 4 * (l / 16) + v.
            const int col = (cb0 + j) * 16 + r16;
            if (col < a.N) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = m0 + ch * 16 + 4 * grp + v;
                    if (row < r1) a.out[(int64_t)row * a.N + col] = to_bf16(a.alpha * sum[v]);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_grouped(const GroupedArgs& a, hipStream_t stream) {
    const int blocks = a.Np / 16;
    const dim3 grid((unsigned)((int64_t)a.G * ((blocks + kGroupedBlocks - 1) / kGroupedBlocks)));
    hipLaunchKernelGGL((grouped_kernel<kGroupedWaves, kGroupedChunks, kGroupedUnits, kGroupedBlocks>), grid, dim3(kGroupedWaves * 64), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4
