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

// ---------------------------------------------------------------------------
// Grouped mid-size kernel: groups of a few dozen to a few hundred rows (a
// prefill-sized batch spread over the experts), too many rows for the
// skinny kernel's decode of A per 16-column block and too few for 256-row
// tiles.  The output of every group is cut into 64 x 64 tiles, numbered row
// block by row block in group order (a group's row blocks start at its first
// row; the last one may run past the group's end, and those rows are not
// stored), and a persistent grid takes the tiles in turn.  In a tile the
// waves split K as in the mid-size single-GEMM kernel: each wave owns the
// whole tile over every WAVES-th 64-element panel, with its operands loaded
// straight into registers (buffer loads, the panel in the scalar offset,
// DEPTH panels in flight) and decoded once per tile; the wave tiles are then
// added in LDS in wave order.  Before its first tile the workgroup counts
// the row blocks of every group into an LDS table (a workgroup-wide prefix
// sum over the offsets table, clamped to [0, M] as in the grouped skinny
// kernel); a tile's group is then a binary search in that table.
// ---------------------------------------------------------------------------
template <int WAVES>
__global__ void __launch_bounds__(WAVES * 64) grouped_wsplit_kernel(GroupedArgs a, int tiles_n) {
    constexpr int BM = 64, BN = 64, MI = BM / 32, NI = BN / 32;
    constexpr int DEPTH = 2;                   // panels of loads in flight per wave
    constexpr int IDX = MI * NI * 16;          // accumulator slots per lane
    static_assert(IDX % WAVES == 0, "every wave adds the same number of slots");
    constexpr int PER = IDX / WAVES;
    __shared__ __attribute__((aligned(16))) float red[WAVES][IDX][64];
    __shared__ int cum[kGroupedWsplitMaxGroups + 1];  // row blocks of the groups before g
    __shared__ int wsum[WAVES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: scalar load offsets)
    const int q = lane & 31, h = lane >> 5;
    auto rows_of = [&](int g, int& r0, int& r1) {
        r0 = min(max(a.offsets[g], 0), a.M);
        r1 = min(max(a.offsets[g + 1], r0), a.M);
    };

    {   // cum[g] for g = 0 .. G: each thread counts a contiguous range of groups
        const int per = (a.G + WAVES * 64 - 1) / (WAVES * 64);
        const int g_lo = min(tid * per, a.G), g_hi = min(g_lo + per, a.G);
        int cnt = 0;
        for (int g = g_lo; g < g_hi; ++g) {
            int r0, r1;
            rows_of(g, r0, r1);
            cnt += (r1 - r0 + BM - 1) / BM;
        }
        int incl = cnt;  // inclusive prefix sum over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int run = incl - cnt;
        for (int w = 0; w < wave; ++w) run += wsum[w];
        for (int g = g_lo; g < g_hi; ++g) {
            int r0, r1;
            rows_of(g, r0, r1);
            cum[g] = run;
            run += (r1 - r0 + BM - 1) / BM;
        }
        if (g_lo < g_hi && g_hi == a.G) cum[a.G] = run;
        __syncthreads();
    }
    const int total = cum[a.G] * tiles_n;

    const int P = a.P;
    const int count = P > wave ? (P - wave + WAVES - 1) / WAVES : 0;  // this wave's panels
    const __amdgpu_buffer_rsrc_t rac = make_rsrc(a.a_codes, (uint32_t)P * a.Mp * 32u);
    const __amdgpu_buffer_rsrc_t ras = make_rsrc(a.a_scales, (uint32_t)P * a.Mp * 4u);

    struct Regs {
        uint4 ca[MI], cb[NI];
        uint32_t sa[MI], sb[NI];
    };

    // Tiles in turn; with a grid of whole XCD rounds (workgroup w runs on
    // XCD w % 8), XCD x takes the x-th eighth of the tile order, so the tiles
    // of one group, which share its A rows and its weights, meet in that
    // XCD's L2.
    int t_begin = blockIdx.x, t_step = gridDim.x, t_end = total;
    if ((gridDim.x & 7) == 0) {
        const int x = blockIdx.x & 7;
        t_begin = (int)((int64_t)total * x / 8) + (blockIdx.x >> 3);
        t_step = gridDim.x >> 3;
        t_end = (int)((int64_t)total * (x + 1) / 8);
    }
    // A tile's rows, group, and the lane offsets and weight descriptors of
    // its loads.
    struct Src {
        int m0, n0, r1;
        uint32_t a_code[MI], a_sc[MI], b_code[NI], b_sc[NI];
        __amdgpu_buffer_rsrc_t rbc, rbs;
    };
    auto src_of = [&](int t) {
        Src s;
        const int vm = t / tiles_n, tn = t - vm * tiles_n;
        int lo = 0, hi = a.G;  // the group of row block vm: cum[g] <= vm < cum[g + 1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cum[mid] <= vm) lo = mid;
            else hi = mid;
        }
        const int g = lo;
        int r0;
        rows_of(g, r0, s.r1);
        s.m0 = r0 + (vm - cum[g]) * BM;
        s.n0 = tn * BN;
        // rows clamped to the padded operands (rows past the group's end
        // belong to the next group or to the padding: computed, not stored)
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint32_t r = (uint32_t)min(s.m0 + i * 32 + q, a.Mp - 1);
            s.a_code[i] = r * 32u + (uint32_t)h * 16u;
            s.a_sc[i] = r * 4u + (uint32_t)h * 2u;
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const uint32_t r = (uint32_t)min(s.n0 + j * 32 + q, a.Np - 1);
            s.b_code[j] = r * 32u + (uint32_t)h * 16u;
            s.b_sc[j] = r * 4u + (uint32_t)h * 2u;
        }
        s.rbc = make_rsrc(a.b_codes + (int64_t)g * P * a.Np * 32, (uint32_t)P * a.Np * 32u);
        s.rbs = make_rsrc(a.b_scales + (int64_t)g * P * a.Np * 4, (uint32_t)P * a.Np * 4u);
        return s;
    };
    // k-th panel of this wave in tile s; past its last panel it re-reads
    // that one and compute() gives it zero scales (unconditional loads:
    // exact wait counts, as in the single-GEMM kernel)
    auto load = [&](const Src& s, int k, Regs& r) {
        const uint32_t pnl = (uint32_t)(wave + min(k, count - 1) * WAVES);
        const uint32_t sa_off = pnl * (uint32_t)a.Mp, sb_off = pnl * (uint32_t)a.Np;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            r.ca[i] = load16(rac, s.a_code[i], sa_off * 32u);
            r.sa[i] = __builtin_amdgcn_raw_buffer_load_b16(ras, s.a_sc[i], sa_off * 4u, 0);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            r.cb[j] = load16(s.rbc, s.b_code[j], sb_off * 32u);
            r.sb[j] = __builtin_amdgcn_raw_buffer_load_b16(s.rbs, s.b_sc[j], sb_off * 4u, 0);
        }
    };

    f16v acc[MI][NI];
    auto compute = [&](const Regs& r, bool live) {  // live: a panel of the wave (uniform)
        h2 sa[MI], sb[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i) sa[i] = e4m3x2_lo(live ? r.sa[i] : 0u);
#pragma unroll
        for (int j = 0; j < NI; ++j) sb[j] = e4m3x2_lo(live ? r.sb[j] : 0u);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            h8 av[MI], bv[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i) av[i] = decode8(word_of(r.ca[i], s), scale_of(sa[i], s));
#pragma unroll
            for (int j = 0; j < NI; ++j) bv[j] = decode8(word_of(r.cb[j], s), scale_of(sb[j], s));
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    };

    // A wave whose panels fill whole rounds of the ring loads the next
    // tile's first panels in its last round, instead of reading its last
    // panel again, so that they arrive while this tile is reduced and
    // stored; other waves start each tile with fresh loads.
    const bool ahead = count > 0 && count % DEPTH == 0;  // (wave-uniform)
    const int k_last = count > 0 ? (count - 1) / DEPTH * DEPTH : 0;  // first panel of the last round
    if (t_begin >= t_end) return;
    Regs ring[DEPTH];
    int t = t_begin;
    Src cur = src_of(t);
    bool loaded = false;  // ring holds the current tile's first panels
    for (;;) {
        const int t_next = t + t_step;
        const bool more = t_next < t_end;
        const Src nxt = src_of(more ? t_next : t);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
        if (count > 0) {
            if (!loaded) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) load(cur, d, ring[d]);
                // (the first panels are taken as they arrive, so that the
                // compiler does not merge these loads with the loop's own)
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        asm volatile("" : "+v"(ring[d].ca[i].x), "+v"(ring[d].ca[i].y), "+v"(ring[d].ca[i].z),
                                          "+v"(ring[d].ca[i].w), "+v"(ring[d].sa[i]));
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        asm volatile("" : "+v"(ring[d].cb[j].x), "+v"(ring[d].cb[j].y), "+v"(ring[d].cb[j].z),
                                          "+v"(ring[d].cb[j].w), "+v"(ring[d].sb[j]));
                }
            }
            for (int k = 0; k < k_last; k += DEPTH) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    compute(ring[d], true);
                    load(cur, k + d + DEPTH, ring[d]);
                    __builtin_amdgcn_sched_barrier(0);  // each slot's loads right after its MFMAs
                }
            }
            // the last round: its loads fetch the next tile's first panels
            // (or, without a next tile or whole rounds, re-read the last one)
            const bool go = ahead && more;  // (wave-uniform)
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                compute(ring[d], k_last + d < count);
                load(go ? nxt : cur, go ? d : k_last + d + DEPTH, ring[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
            loaded = go;
        }
        const int m0 = cur.m0, n0 = cur.n0, r1 = cur.r1;

        // Add the wave tiles in wave order.
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) red[wave][(i * NI + j) * 16 + v][lane] = acc[i][j][v];
        __syncthreads();
        float sum[PER];  // slots wave w adds: w, w + WAVES, ...
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            float x = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) x += red[w][wave + u * WAVES][lane];
            sum[u] = x;
        }
        // Slot idx = (i * NI + j) * 16 + v of lane l is row i*32 + 8*(v/4) +
        // 4*(l/32) + v%4 and column j*32 + l%32 of the tile.
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int idx = wave + u * WAVES;
            const int v = idx & 15, ij = idx >> 4;
            const int i = ij / NI, j = ij % NI;
            const int row = m0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            const int col = n0 + j * 32 + q;
            if (row < r1 && col < a.N) a.out[(int64_t)row * a.N + col] = to_bf16(a.alpha * sum[u]);
        }
        __syncthreads();  // every wave is done reading red before the next tile writes it
        if (!more) break;
        t = t_next;
        cur = nxt;
    }
}

}  // namespace

hipError_t launch_grouped_wsplit(const GroupedArgs& a, hipStream_t stream) {
    const int64_t tiles_n = (a.N + 63) / 64;
    // at most one workgroup per CU (the wave tiles take 128 KB of LDS), and
    // no more workgroups than the tiles could number (each group adds at
    // most one partial row block)
    const int64_t bound = ((int64_t)(a.M + 63) / 64 + a.G) * tiles_n;
    const int grid = (int)(bound < kCUs ? bound : kCUs);
    hipLaunchKernelGGL((grouped_wsplit_kernel<kGroupedWsplitWaves>), dim3((unsigned)grid),
                       dim3(kGroupedWsplitWaves * 64), 0, stream, a, (int)tiles_n);
    return hipGetLastError();
}

hipError_t launch_grouped(const GroupedArgs& a, hipStream_t stream) {
    const int blocks = a.Np / 16;
    const dim3 grid((unsigned)((int64_t)a.G * ((blocks + kGroupedBlocks - 1) / kGroupedBlocks)));
    hipLaunchKernelGGL((grouped_kernel<kGroupedWaves, kGroupedChunks, kGroupedUnits, kGroupedBlocks>), grid, dim3(kGroupedWaves * 64), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4
