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
#include "nvfp4_device.h"
#include "nvfp4_quant_device.h"

namespace nvfp4 {
namespace {

// Sticky error flags of this device's kernels (kFlag* bits), read and
// cleared by the host through take_device_flags.
__device__ uint32_t g_device_flags;

__device__ __forceinline__ void raise_flag(uint32_t bit) {
    (void)__hip_atomic_fetch_or(&g_device_flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Large-M tile kernel.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; workgroup tile BM x BN,
// wave tile (BM/2) x (BN/2) made of 32 x 32 MFMA blocks
// (v_mfma_f32_32x32x16_f16).  K advances one 64-element panel at a time.
//
// HBM -> LDS: each panel's packed codes (4 bits/element) and raw E4M3 scale
// bytes are copied with direct-to-LDS loads (16 and 4 bytes per lane) into a
// ring of NS stage buffers, NS-1 panels ahead of the panel being multiplied,
// so several panels of loads are always in flight and no VGPRs are spent on
// staging.
//
// LDS code layout of one operand and panel: rows in groups of 32; within a
// group, first the low 16 bytes of the 32 rows, then the high 16 bytes
// (one 1 KB direct load per group):
//   offset(row, half) = (row / 32) * 1024 + half * 512 + (row % 32) * 16.
// MFMA lane l reads row l % 32, half l / 32 as one 16-byte read, so the lanes
// of each LDS phase touch consecutive bytes.  Scales: the rows' 4-byte scale
// words in (half tile, row within a 32-row block, block) order, so that a
// lane gets the words of all its row blocks with one read.
//
// Decode and MFMA are software-pipelined: the operands of sub-step s+1 are
// decoded while the MFMAs of sub-step s run (the scheduler is told to
// alternate one MFMA and a few VALU instructions), and the next panel's LDS
// reads are issued a whole panel ahead, so a panel's first sub-step never
// waits for LDS.  One barrier per panel both publishes the next panel's
// loads and hands the previous panel's buffer back to the loads.
//
// Tile rows past the padded operand read whatever lies beyond it (the next
// panel's first rows, or zeros past the end of the buffer); their results are
// never stored.  The packed K is a whole number of 128-element steps
// (the packer pads with zeros), so every workgroup runs an even number of
// panels.
//
// Without split-K the grid is persistent (as many workgroups as fit on the
// GPU at once) and each workgroup walks several tiles; its load ring runs on
// across tile boundaries, so a tile's first panels arrive while the previous
// tile is still being multiplied and stored.
//
// Split-K (split_k > 1): the K steps are divided into split_k contiguous
// ranges; each workgroup publishes its FP32 tile to the workspace, and the
// last of a tile's workgroups to arrive adds the partial tiles in split order
// (deterministic) and runs the epilogue.  A persistent launch whose last
// round would be at most half full is issued as two launches (launch_tile):
// the full rounds, then the remaining tiles with their K range split.
//
// Epilogue: 256 x 256 tiles (with N % 8 == 0) pass the output through a
// per-wave LDS staging block so that every store writes whole 128-byte
// lines; the other configurations store 8-byte pieces straight from the
// accumulators.
//
// Grouped mode (GROUPED): the experts of a mixture-of-experts layer with
// large groups; each workgroup finds its group and row block from the
// device offsets table (see the code), multiplies that group's B, and
// stores only the group's rows.
// ---------------------------------------------------------------------------
template <int BM, int BN, int NS, bool SPLIT, bool GROUPED = false>
__global__ void __launch_bounds__(256, 1) tile_kernel(GemmArgs a) {
    constexpr int MI = BM / 64;  // 32-row blocks per wave
    constexpr int NI = BN / 64;  // 32-column blocks per wave
    constexpr int OFF_B = BM * 32;
    constexpr int OFF_SA = OFF_B + BN * 32;
    constexpr int OFF_SB = OFF_SA + BM * 4;
    constexpr int STAGE = OFF_SB + BN * 4;
    constexpr int A_CCH = BM / 32;               // 1 KB code chunks of A per panel
    constexpr int CCH = A_CCH + BN / 32;
    constexpr int A_SCH = BM / 64;               // 256 B scale chunks of A per panel
    constexpr int SCH = A_SCH + BN / 64;
    constexpr int CPW = (CCH + 3) / 4;           // code chunks per wave
    constexpr int SPW = (SCH + 3) / 4;           // scale chunks per wave
    constexpr int LPS = CPW + SPW;               // direct loads per wave per panel
    static_assert(NS >= 3 && NS <= 8 && (NS - 2) * LPS < 64, "pipeline depth");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];
    // 256 x 256 tiles: per wave, a 32 x 64 bf16 staging block for the
    // epilogue (the ring keeps loading the next tile meanwhile, so the
    // epilogue cannot borrow ring buffers; this brings the workgroup to the
    // 160 KB of LDS).
    constexpr bool STAGED_OUT = BM == 256 && BN == 256;
    // (also the grouped mode's scheduling scratch, before the main loop)
    __shared__ __attribute__((aligned(16))) uint8_t out_stage[STAGED_OUT ? 4 * 4096 : 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // (& 3: the compiler then knows which direct loads are A's and which B's)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane & 31, h = lane >> 5;

    // Work items.  Without split-K the grid is persistent: workgroup w takes
    // tiles w, w + G, w + 2G, ... (G = gridDim.x, a multiple of 8 whenever a
    // workgroup gets more than one tile).  With split-K, workgroup w takes
    // the single (tile, K range) pair w.  Consecutive ids are dealt to the
    // eight XCDs in turn; the id is remapped so that each XCD works on a
    // contiguous range of tiles, walked in groups of 8 along M for L2 reuse.
    const int T = a.tile_count;
    const int S = SPLIT ? a.split_k : 1;
    const int G = SPLIT ? 1 : (int)gridDim.x;
    const int n_items = (SPLIT || GROUPED) ? 1 : (T - (int)blockIdx.x + G - 1) / G;
    auto item_of = [&](int it, int& t, int& z) {
        int bid = (int)blockIdx.x + it * G;
        const int total = T * S;
        if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
        z = bid % S;
        t = bid / S;
    };
    auto origin_of = [&](int t, int& m0, int& n0) {  // t: tile of this launch's range
        constexpr int GROUP_M = 8;
        t += a.tile_begin;
        const int in_group = GROUP_M * a.tiles_n;
        const int first_m = (t / in_group) * GROUP_M;
        const int gsize = min(a.tiles_m - first_m, GROUP_M);
        m0 = (first_m + (t % in_group) % gsize) * BM;
        n0 = ((t % in_group) / gsize) * BN;
    };
    int t0, z0;
    item_of(0, t0, z0);

    // Grouped mode (a mixture-of-experts layer with large groups): group g
    // owns rows [offsets[g], offsets[g+1]) of A and C and its own B operand.
    // The row blocks of all groups are numbered in group order (group g has
    // ceil(rows_g / BM) of them); tile t0 is row block t0 / tiles_n, column
    // block t0 % tiles_n, and the grid is an upper bound on the tiles.  Each
    // thread counts the row blocks of a contiguous range of groups, a
    // workgroup-wide prefix sum places the ranges, and the thread whose range
    // holds the row block publishes (group, first row, end row); a workgroup
    // past the last row block exits.  Offsets are clamped to [0, M] as in the
    // grouped skinny kernel.  Scratch: the epilogue's staging block.
    int grp = 0, grp_row0 = 0, row_end = a.M;
    if constexpr (GROUPED) {
        int* sch = reinterpret_cast<int*>(out_stage);  // [0..3] wave totals, [4..7] result
        const int vm = t0 / a.tiles_n;
        const int per = (a.groups + 255) / 256;
        const int g_lo = min(tid * per, a.groups), g_hi = min(g_lo + per, a.groups);
        auto rows_of = [&](int g, int& r0, int& r1) {
            r0 = min(max(a.offsets[g], 0), a.M);
            r1 = min(max(a.offsets[g + 1], r0), a.M);
        };
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
        if (tid == 0) sch[7] = 0;
        if (lane == 63) sch[wave] = incl;
        __syncthreads();
        int excl = incl - cnt;
        for (int w = 0; w < wave; ++w) excl += sch[w];
        if (vm >= excl && vm < excl + cnt) {
            int v = vm - excl;
            for (int g = g_lo; g < g_hi; ++g) {
                int r0, r1;
                rows_of(g, r0, r1);
                const int c = (r1 - r0 + BM - 1) / BM;
                if (v < c) {
                    sch[4] = g;
                    sch[5] = r0 + v * BM;
                    sch[6] = r1;
                    sch[7] = 1;
                    break;
                }
                v -= c;
            }
        }
        __syncthreads();
        if (sch[7] == 0) return;  // no tile: the whole workgroup leaves
        grp = __builtin_amdgcn_readfirstlane(sch[4]);
        grp_row0 = __builtin_amdgcn_readfirstlane(sch[5]);
        row_end = __builtin_amdgcn_readfirstlane(sch[6]);
    }
    const int nst = a.P / 2;
    const int p0 = 2 * (int)((int64_t)z0 * nst / S);
    const int p1 = 2 * (int)((int64_t)(z0 + 1) * nst / S);

    const uint32_t lds0 = lds_addr(lds);

    // Direct-load plan (constant over the panels of one tile): for each of
    // the wave's code and scale chunks, the lane's byte offset inside a
    // panel.  When an operand has fewer chunks than there are waves, chunks
    // are issued twice (same bytes to the same place), so every wave issues
    // LPS loads per panel.
    // Direct-load plan.  Lane offsets inside a tile's panel are the same for
    // every tile: the panel's and the tile's first row go into the scalar
    // offset.  Past the bottom or right edge of an operand a lane reads the
    // following panel's first rows, or, past the end of the operand, zeros
    // (the buffer range check covers the scalar offset too).  Either way
    // those rows only feed results that are never stored.
    uint32_t c_lane[CPW], s_lane[SPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int k = (wave + 4 * i) % CCH;
        const int grp = k < A_CCH ? k : k - A_CCH;
        c_lane[i] = (uint32_t)(grp * 32 + q) * 32u + (uint32_t)h * 16u;
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int k = (wave + 4 * i) % SCH;
        const bool isA = k < A_SCH;
        const int R = isA ? BM : BN;
        const int G2 = isA ? MI : NI;  // 32-row blocks per wave along this operand
        const int c = isA ? k : k - A_SCH;
        // LDS slot c*64 + lane holds the scales of tile row r: slots are in
        // (half of the tile, row within its 32-row block, block) order.
        const int slot = c * 64 + lane;
        const int half = slot / (R / 2), sr = slot % (R / 2);
        s_lane[i] = (uint32_t)(half * (R / 2) + (sr % G2) * 32 + sr / G2) * 4u;
    }
    const __amdgpu_buffer_rsrc_t rac = make_rsrc(a.a_codes, (uint32_t)a.P * a.Mp * 32u);
    const int64_t b_rows = GROUPED ? (int64_t)grp * a.P * a.Np : 0;  // B rows of the groups before
    const __amdgpu_buffer_rsrc_t rbc = make_rsrc(a.b_codes + b_rows * 32, (uint32_t)a.P * a.Np * 32u);
    const __amdgpu_buffer_rsrc_t ras = make_rsrc(a.a_scales, (uint32_t)a.P * a.Mp * 4u);
    const __amdgpu_buffer_rsrc_t rbs = make_rsrc(a.b_scales + b_rows * 4, (uint32_t)a.P * a.Np * 4u);
    // Tile whose panels are being loaded: byte offsets of its first A and B
    // rows inside a code panel (inside a scale panel: / 8).
    uint32_t base_a = 0, base_b = 0;
    auto load_tile = [&](int m0, int n0) {
        base_a = (uint32_t)m0 * 32u;
        base_b = (uint32_t)n0 * 32u;
    };
    const uint32_t a_stride = (uint32_t)a.Mp * 32u, b_stride = (uint32_t)a.Np * 32u;
    // Issue direct load d (0 <= d < LPS) of the panel at code offsets
    // (pa, pb) of A and B into stage buffer sb.  Scale offsets are the code
    // offsets / 8 (4 scale bytes per 32 code bytes).
    auto issue_one = [&](int sb, int d, uint32_t pa, uint32_t pb) {
        const uint32_t b = lds0 + (uint32_t)(sb * STAGE);
        if (d < CPW) {
            const int k = (wave + 4 * d) % CCH;
            const bool isA = k < A_CCH;
            const int grp = isA ? k : k - A_CCH;
            dma16(isA ? rac : rbc, c_lane[d], isA ? pa + base_a : pb + base_b,
                  b + (uint32_t)((isA ? 0 : OFF_B) + grp * 1024));
        } else {
            const int i = d - CPW;
            const int k = (wave + 4 * i) % SCH;
            const bool isA = k < A_SCH;
            const int c = isA ? k : k - A_SCH;
            dma4(isA ? ras : rbs, s_lane[i], (isA ? pa + base_a : pb + base_b) >> 3,
                 b + (uint32_t)((isA ? OFF_SA : OFF_SB) + c * 256));
        }
    };

    // Accumulators; each tile's first MFMAs start from zero, so they carry
    // nothing from one tile to the next.
    f16v acc[MI][NI];

    // Operand registers of one panel: raw codes (one 16-byte LDS read per
    // 32-row block: words 0..3 feed the four MFMA sub-steps) and the two
    // block scales of the lane's half, widened to fp16.
    struct PanelRegs {
        uint4 ca[MI], cb[NI];
        // scale words of the lane's rows; the lane's two E4M3 block scales
        // are in bits 16h+15:16h until ready_scales moves them to bits 15:0
        uint32_t sa[MI], sb[NI];
    };
    auto read_words = [&](const uint8_t* p, uint32_t (&w)[4], int n) {
        if (n == 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(p);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else if (n == 2) {
            const uint2 v = *reinterpret_cast<const uint2*>(p);
            w[0] = v.x; w[1] = v.y;
        } else {
            w[0] = *reinterpret_cast<const uint32_t*>(p);
        }
    };
    auto read_panel = [&](const uint8_t* b, PanelRegs& r) {
        uint32_t wa[4], wb[4];
        read_words(b + OFF_SA + (wm * (BM / 2) + q * MI) * 4, wa, MI);
        read_words(b + OFF_SB + (wn * (BN / 2) + q * NI) * 4, wb, NI);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            r.ca[i] = *reinterpret_cast<const uint4*>(b + (wm * MI + i) * 1024 + h * 512 + q * 16);
            r.sa[i] = wa[i];
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            r.cb[j] = *reinterpret_cast<const uint4*>(b + OFF_B + (wn * NI + j) * 1024 + h * 512 + q * 16);
            r.sb[j] = wb[j];
        }
    };
    // Done where a panel is first decoded (not right after its LDS reads,
    // which would make the wave wait for them there).
    auto ready_scales = [&](PanelRegs& r) {
#pragma unroll
        for (int i = 0; i < MI; ++i) r.sa[i] >>= 16 * h;
#pragma unroll
        for (int j = 0; j < NI; ++j) r.sb[j] >>= 16 * h;
    };
    h8 av[2][MI], bv[2][NI];  // decoded operands of the current / next sub-step
    auto decode = [&](const PanelRegs& r, int s, h8 (&ao)[MI], h8 (&bo)[NI]) {
#pragma unroll
        for (int i = 0; i < MI; ++i) ao[i] = decode8(word_of(r.ca[i], s), scale_of(e4m3x2_lo(r.sa[i]), s));
#pragma unroll
        for (int j = 0; j < NI; ++j) bo[j] = decode8(word_of(r.cb[j], s), scale_of(e4m3x2_lo(r.sb[j]), s));
    };
    // The four sub-steps of panel `cur` (its sub-step 0 is already decoded
    // in av/bv[0]); the decode of each following sub-step -- the last one
    // being sub-step 0 of panel `nxt` -- runs under the MFMAs, and so do the
    // direct loads of the cursor's panel into buffer lsb (spread over the
    // sub-steps).  B is the MFMA's first operand, so each 32 x 32 result
    // block holds its part of C transposed (see the epilogue).
    auto run_panel = [&](const PanelRegs& cur, PanelRegs& nxt, int lsb, uint32_t pc,
                         bool first) {
        const uint32_t pa = pc * a_stride, pb = pc * b_stride;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = s & 1, n = c ^ 1;
#pragma unroll
            for (int d = s * LPS / 4; d < (s + 1) * LPS / 4; ++d) issue_one(lsb, d, pa, pb);
            if (s < 3) {
                decode(cur, s + 1, av[n], bv[n]);
            } else {
                ready_scales(nxt);
                decode(nxt, 0, av[n], bv[n]);
            }
            // (j outermost: consecutive MFMAs share their first operand)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        bv[c][j], av[c][i], (first && s == 0) ? f16v{} : acc[i][j], 0, 0, 0);
            // each MFMA followed by its share of the sub-step's VALU work: 8
            // decode instructions per fragment, its scale convert and, in
            // the last sub-step, its scale shift (with the decode alone
            // counted, the last 16-24 instructions of a panel ran after its
            // last MFMA: 256 x 256 tiles 0.5-1% slower; a share of six
            // instead of five per MFMA was 2-3% slower)
#pragma unroll
            for (int m = 0; m < MI * NI; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, (10 * (MI + NI) + MI * NI - 1) / (MI * NI), 0);
            }
        }
    };
    // Panels of the current item (relative index 0 .. np-1).  The panel
    // NS-1 ahead of relative panel r lies in the workgroup's next tile when
    // r + NS - 1 >= np (np >= NS - 1 whenever there is a next tile): at
    // r = np - (NS-1) the load offsets switch to that tile.  Without a next
    // tile the last panel is loaded again: those buffers are never read, and
    // every panel then carries exactly LPS loads per wave (the wait counts
    // rely on it).
    const int np = p1 - p0;
    int cur_it = 0;           // item being multiplied
    int next_m0 = 0, next_n0 = 0;  // origin of item cur_it + 1, if any
    auto load_panel = [&](int r) -> uint32_t {
        const int q = r + NS - 1;
        if (q < np) return (uint32_t)(p0 + q);
        return (uint32_t)(cur_it + 1 < n_items ? p0 + q - np : p1 - 1);
    };
    auto start_item = [&](int it, int& m0, int& n0) {
        int t, z;
        item_of(it, t, z);
        if constexpr (GROUPED) {
            m0 = grp_row0;
            n0 = (t % a.tiles_n) * BN;
        } else {
            origin_of(t, m0, n0);
        }
        cur_it = it;
        if (it + 1 < n_items) {
            item_of(it + 1, t, z);
            origin_of(t, next_m0, next_n0);
        }
    };
    // One panel (the g-th this workgroup multiplies, relative panel r of its
    // item): wait until panel g+1 is resident (loads of panels g+2 ..
    // g+NS-2 may still be in flight), barrier (everyone is past panel g-1,
    // whose buffer now takes panel g+NS-1), read panel g+1 (a stale buffer
    // after the last panel; those values go unused), multiply panel g while
    // the loads of panel g+NS-1 are issued.  `first`: relative panel 0,
    // whose first MFMAs start from zero.
    auto step = [&](int g, int r, const PanelRegs& cur, PanelRegs& nxt, bool first) {
        // (the scheduling barriers keep the previous panel's MFMAs before the
        // workgroup barrier, and the LDS reads here, a panel ahead of use)
        __builtin_amdgcn_sched_barrier(0);
        wait_steps<LPS>(NS - 3);
        wg_barrier();
        read_panel(lds + ((g + 1) % NS) * STAGE, nxt);
        __builtin_amdgcn_sched_barrier(0);
        if (r == np - (NS - 1) && cur_it + 1 < n_items) load_tile(next_m0, next_n0);
        run_panel(cur, nxt, (g + NS - 1) % NS, load_panel(r), first);
    };

    // Epilogue of one tile: y = alpha * acc (FP32), bfloat16 round-to-nearest
    // even.  The 32x32 MFMA result layout puts column l % 32 of a block and
    // rows 8 * (v / 4) + 4 * (l / 32) + v % 4 in lane l; the blocks hold C
    // transposed, so lane l has row l % 32 of C and, for each v / 4, four
    // consecutive columns, stored as one 8-byte write when N % 4 == 0.
    // One 32 x 32 block (i, j) of the wave's part of the tile; val(v) gives
    // the lane's v-th value of the block.  Lane coordinates are recomputed
    // here (cheap, and no VGPR has to stay live across the main loop for
    // them); the block is stored through a uniform base address plus a
    // 32-bit lane offset (32 * N * 2 bytes < 4 GiB: the packed-size limit
    // of this path keeps N below 2^25).
    auto store_block = [&](int m0, int n0, int i, int j, auto&& val) {
        const bool vec = (a.N & 3) == 0;
        const uint32_t ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int lq = (int)(ln & 31u), lh = (int)(ln >> 5);
        const uint32_t lane_off = (uint32_t)lq * (uint32_t)a.N * 2u + (uint32_t)lh * 8u;
        const int row0 = m0 + wm * (BM / 2) + i * 32;
        const int col0 = n0 + wn * (BN / 2) + j * 32;
        uint8_t* base = reinterpret_cast<uint8_t*>(a.out + (int64_t)row0 * a.N + col0);
        if (row0 + lq < row_end) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int col = col0 + 8 * u + 4 * lh;
                const uint16_t e0 = to_bf16(a.alpha * val(4 * u + 0));
                const uint16_t e1 = to_bf16(a.alpha * val(4 * u + 1));
                const uint16_t e2 = to_bf16(a.alpha * val(4 * u + 2));
                const uint16_t e3 = to_bf16(a.alpha * val(4 * u + 3));
                uint8_t* p = base + lane_off + 16u * u;
                if (vec) {
                    if (col < a.N)
                        *reinterpret_cast<uint2*>(p) =
                            uint2{(uint32_t)e0 | ((uint32_t)e1 << 16), (uint32_t)e2 | ((uint32_t)e3 << 16)};
                } else {
                    uint16_t* o = reinterpret_cast<uint16_t*>(p);
                    if (col + 0 < a.N) o[0] = e0;
                    if (col + 1 < a.N) o[1] = e1;
                    if (col + 2 < a.N) o[2] = e2;
                    if (col + 3 < a.N) o[3] = e3;
                }
            }
        }
    };
    // Epilogue through the wave's LDS staging block (256 x 256 tiles, N % 8
    // == 0): for each row of 32 x 32 blocks and each pair of blocks, the
    // lanes write their bf16 values (row l % 32, four columns per 8-byte
    // write) into a 32 x 128-byte block, then read it back 16 bytes per lane
    // along rows, so that every store instruction writes eight whole
    // 128-byte lines of C.  Partial lines (the direct form writes 16 bytes
    // of 32 rows per instruction) left L2 incomplete for tall, narrow C and
    // were written back to memory several times over.  The 16-byte column
    // chunks of a staged row are XOR-swizzled by the row (mod 8) to spread
    // the writes over the LDS banks.  The block is private to the wave and
    // LDS instructions of one wave complete in order, so no barrier is
    // needed between the writes and the reads.
    auto store_tile_staged = [&](int m0, int n0) {
        uint8_t* st = out_stage + wave * 4096;
        const uint32_t ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int lq = (int)(ln & 31u), lh = (int)(ln >> 5);
        const int wsw = (lq & 7) * 16;                 // swizzle of the row this lane writes
        const int rrow = (int)(ln >> 3), rch = (int)(ln & 7u);  // row / chunk this lane reads
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < NI / 2; ++jj) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jl = 0; jl < 2; ++jl)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const f16v& c = acc[i][2 * jj + jl];
                        const uint16_t e0 = to_bf16(a.alpha * acc_read(c[4 * u + 0]));
                        const uint16_t e1 = to_bf16(a.alpha * acc_read(c[4 * u + 1]));
                        const uint16_t e2 = to_bf16(a.alpha * acc_read(c[4 * u + 2]));
                        const uint16_t e3 = to_bf16(a.alpha * acc_read(c[4 * u + 3]));
                        const int cb = jl * 64 + u * 16 + lh * 8;  // byte column in the staged row
                        *reinterpret_cast<uint2*>(st + lq * 128 + (cb ^ wsw)) =
                            uint2{(uint32_t)e0 | ((uint32_t)e1 << 16), (uint32_t)e2 | ((uint32_t)e3 << 16)};
                    }
                const int col = n0 + wn * (BN / 2) + jj * 64 + rch * 8;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int r = k * 8 + rrow;
                    const uint4 v = *reinterpret_cast<const uint4*>(st + r * 128 + ((rch * 16) ^ ((r & 7) * 16)));
                    const int row = m0 + wm * (BM / 2) + i * 32 + r;
                    if (row < row_end && col < a.N)
                        *reinterpret_cast<uint4*>(a.out + (int64_t)row * a.N + col) = v;
                }
            }
    };
    // Epilogue of a tile without split-K, straight from the accumulators
    // (read one at a time from AGPRs), one block at a time so that few
    // values sit in VGPRs.
    auto store_tile = [&](int m0, int n0) {
        if constexpr (STAGED_OUT) {
            if ((a.N & 7) == 0) {
                store_tile_staged(m0, n0);
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                store_block(m0, n0, i, j, [&](int v) { return acc_read(acc[i][j][v]); });
            }
    };

    // Prologue: NS-1 panels in flight; wait for the first and decode its
    // first sub-step.
    int m0, n0;
    start_item(0, m0, n0);
    load_tile(m0, n0);
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
        const uint32_t pc = load_panel(u - (NS - 1));
#pragma unroll
        for (int d = 0; d < LPS; ++d) issue_one(u, d, pc * a_stride, pc * b_stride);
    }
    PanelRegs r0, r1;
    wait_steps<LPS>(NS - 2);
    wg_barrier();
    read_panel(lds, r0);
    ready_scales(r0);
    decode(r0, 0, av[0], bv[0]);

    if constexpr (!SPLIT) {
        // The tiles of this workgroup in turn; a tile's result is stored
        // right after its last panel, while the loads of the next tile's
        // first panels are in flight.
        int g = 0;
        for (int it = 0; it < n_items; ++it) {
            if (it > 0) start_item(it, m0, n0);
            step(g, 0, r0, r1, true);
            step(g + 1, 1, r1, r0, false);
            g += 2;
            for (int r = 2; r < np; r += 2) {  // np is even
                step(g, r, r0, r1, false);
                step(g + 1, r + 1, r1, r0, false);
                g += 2;
            }
            store_tile(m0, n0);
        }
    } else {
        step(0, 0, r0, r1, true);
        step(1, 1, r1, r0, false);
        for (int r = 2; r < np; r += 2) {  // np is even
            step(r, r, r0, r1, false);
            step(r + 1, r + 1, r1, r0, false);
        }
        wait_vmcnt<0>();  // drain the look-ahead loads before the LDS is released
        __shared__ int s_last;
        if (S == 2) {
            // Two K slices: the sum of two partial tiles does not depend on
            // their order, so only the workgroup that finishes first
            // publishes its tile; the second adds it to its own accumulators.
            // The tile's counter takes one increment per arrival and one
            // from the first workgroup once its tile is out, so the second
            // (ticket 1 or 2) waits until it reads 3.  The first workgroup
            // is already running and never waits, so the wait ends; it is
            // bounded all the same (a.handoff_polls).  A second workgroup
            // that runs out of polls takes the tile's three increments back
            // (the counter is zero again once the first one has finished, so
            // later calls stay in step), leaves the tile unwritten and raises
            // the device's hand-off flag for the host to read.
            __syncthreads();
            if (tid == 0) s_last = (int)arrive(a.counters + t0);
            __syncthreads();
            const int64_t slot = (int64_t)t0 * S * (BM * BN);
            if (s_last == 0) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NI; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            publish(a.partials + slot + ((i * NI + j) * 16 + v) * 256 + tid, acc[i][j][v]);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (tid == 0) (void)arrive(a.counters + t0);  // the partial tile is out
                return;
            }
            __shared__ int s_ready;
            if (tid == 0) {
                int ready = 0;
                for (uint32_t it = 0; it < a.handoff_polls; ++it) {
                    if (__hip_atomic_load(a.counters + t0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= 3u) {
                        ready = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                if (ready) {
                    reset_counter(a.counters + t0);
                } else {
                    (void)__hip_atomic_fetch_sub(a.counters + t0, 3u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    raise_flag(kFlagHandoff);
                }
                s_ready = ready;
            }
            __syncthreads();
            if (!s_ready) return;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const float* po = a.partials + slot + (i * NI) * 16 * 256 + tid;
                float sum[NI][16];
#pragma unroll
                for (int j = 0; j < NI; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) sum[j][v] = fetch(po + (j * 16 + v) * 256);
#pragma unroll
                for (int j = 0; j < NI; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) sum[j][v] += acc[i][j][v];
#pragma unroll
                for (int j = 0; j < NI; ++j) store_block(m0, n0, i, j, [&](int v) { return sum[j][v]; });
            }
            return;
        }
        // More slices: every workgroup publishes its partial tile; the last
        // arrival adds them in split order.
        float* mine = a.partials + ((int64_t)t0 * S + z0) * (BM * BN);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    publish(mine + ((i * NI + j) * 16 + v) * 256 + tid, acc[i][j][v]);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = arrive(a.counters + t0);
            s_last = (old == (uint32_t)(S - 1));
            if (s_last) reset_counter(a.counters + t0);  // all splits arrived
        }
        __syncthreads();
        if (!s_last) return;
        // Add the S partial tiles in split order, one row of 32 x 32 blocks
        // at a time: its NI * 16 values of every split are loaded together
        // (the accumulators are dead by now, so the registers are free; one
        // value at a time would wait a full memory round trip per value).
        const float* all = a.partials + (int64_t)t0 * S * (BM * BN);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            float sum[NI][16];
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) sum[j][v] = 0.0f;
            for (int zz = 0; zz < S; ++zz) {
                const float* pz = all + (int64_t)zz * (BM * BN) + (i * NI) * 16 * 256 + tid;
                float part[NI][16];
#pragma unroll
                for (int j = 0; j < NI; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) part[j][v] = fetch(pz + (j * 16 + v) * 256);
#pragma unroll
                for (int j = 0; j < NI; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) sum[j][v] += part[j][v];
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) store_block(m0, n0, i, j, [&](int v) { return sum[j][v]; });
        }
    }
    wait_vmcnt<0>();  // drain the look-ahead loads before the LDS is released
}

// ---------------------------------------------------------------------------
// Skinny-M kernel (M <= 64), for decode-sized GEMMs that are bound by
// streaming B from HBM and by latency.
//
// v_mfma_f32_16x16x32_f16 with a 16-row block of A (zero-padded) as the MFMA
// A operand and 16 rows of B as the B operand; MB = ceil(M / 16) blocks of A
// share each decoded B fragment.  Work unit: 16 B rows x 128 K (two
// panels).  Lane l holds row l % 16 and, with g = l / 16, the 16-byte half
// (g % 2) of panel (g / 2): one 16-byte load of codes and one 2-byte load of
// scales per operand block, straight from HBM (B is used once, so it does
// not pass through LDS).  Each MFMA sub-step s takes word s of every lane.
// Rows of A at or beyond M come from the packed operand's zero padding.
//
// Grid: (N / 16 row groups) x split_k workgroups of WAVES waves; a
// workgroup owns one row group and a contiguous range of work units, dealt
// to its waves in turn; each wave issues the loads of up to UNITS work units
// before it waits, so one memory round trip covers them.  The wave partials
// are added in LDS in wave order; with split_k > 1 the workgroup partials
// are added by the last arrival in split order (deterministic).
// ---------------------------------------------------------------------------
// With one row block and at most 3 units in flight the registers are held
// to 64 per lane, so two 16-wave workgroups share a CU and one's memory
// latency hides under the other's decode work: 16 x 6144 x 6144 7.8 -> 7.0
// us, 16 x 16384 x 6144 19.1 -> 14.8 us (4 units would spill at that size).
// (Plain arguments, operands and geometry first, so that those can be
// preloaded into scalar registers before the waves start.)
template <int WAVES, int MB, int UNITS>
__global__ void __launch_bounds__(WAVES * 64, (MB == 1 && UNITS <= 3) ? 2 * WAVES / 4 : 1)
    skinny_kernel(const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales,
                  const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
                  int Np, int Mp, int P, int split_k, uint16_t* __restrict__ out,
                  uint64_t* flagged, uint32_t* counters, float alpha, int M, int N,
                  uint32_t polls) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int S = split_k;
    const int g = blockIdx.x / S;
    const int z = blockIdx.x % S;
    const int C = P / 2;
    const int c0 = (int)((int64_t)z * C / S);
    const int c1 = (int)((int64_t)(z + 1) * C / S);
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int pl = grp >> 1, half = grp & 1;
    const int nrow = g * 16 + r16;

    f4v acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = f4v{0.0f, 0.0f, 0.0f, 0.0f};
    for (int base = c0 + wave; base < c1; base += WAVES * UNITS) {
        // The loads are unconditional: a unit past the range re-reads the
        // range's last unit and both its operands get zero scales, so it
        // adds exact zeros (never a NaN of the re-read scales),
        // and rows of A past M are the packed operand's zero padding (they
        // only feed rows of C that are not stored).  The compiler can then
        // wait for each unit's loads alone and decode it while the later
        // units arrive.
        uint4 bw[UNITS], aw[UNITS][MB];
        uint32_t bs[UNITS], as[UNITS][MB];
#pragma unroll
        for (int u = 0; u < UNITS; ++u) {
            const int c = min(base + WAVES * u, c1 - 1);
            const int panel = 2 * c + pl;
            const int64_t bo = (int64_t)panel * Np + nrow;
            bw[u] = *reinterpret_cast<const uint4*>(b_codes + bo * 32 + half * 16);
            bs[u] = *reinterpret_cast<const uint16_t*>(b_scales + bo * 4 + half * 2);
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const int64_t ao = (int64_t)panel * Mp + 16 * b + r16;
                aw[u][b] = *reinterpret_cast<const uint4*>(a_codes + ao * 32 + half * 16);
                as[u][b] = *reinterpret_cast<const uint16_t*>(a_scales + ao * 4 + half * 2);
            }
        }
        // (keeps every load ahead of the first unit's decode: the scheduler
        // would otherwise hold back later units' loads to save registers)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < UNITS; ++u) {
            const bool live = base + WAVES * u < c1;   // (wave-uniform)
            const h2 sbh = e4m3x2_lo(live ? bs[u] : 0u);
            h2 sah[MB];
#pragma unroll
            for (int b = 0; b < MB; ++b) sah[b] = e4m3x2_lo(live ? as[u][b] : 0u);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const h8 bv = decode8(word_of(bw[u], s), scale_of(sbh, s));
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    const h8 av = decode8(word_of(aw[u][b], s), scale_of(sah[b], s));
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[b], 0, 0, 0);
                }
            }
        }
    }

    __shared__ f4v red[WAVES][MB][64];
#pragma unroll
    for (int b = 0; b < MB; ++b) red[wave][b][lane] = acc[b];
    __syncthreads();
    // wave b < MB adds the wave partials of A block b (in wave order); every
    // wave stays until the split-K hand-off is decided (barriers below)
    const int blk = wave < MB ? wave : 0;
    const bool reducer = wave < MB;
    f4v part[WAVES];  // all reads issued before the first add
#pragma unroll
    for (int w = 0; w < WAVES; ++w) part[w] = red[w][blk][lane];
    f4v sum = part[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += part[w];

    if (S > 1) {
        // Split K across workgroups (S <= WAVES): every workgroup publishes
        // its blocks as flagged words and takes a ticket without waiting for
        // the stores.  In the last arrival, wave w fetches split w's blocks
        // (all in flight at once, waiting only for their flags: the stores
        // belong to workgroups that already took their tickets) into the
        // LDS partial buffer -- the reducer waves put their own sums in slot
        // z -- and then clears that split's words; the reducer waves add the
        // S slots in split order.  A wave whose fetch runs past `polls`
        // adds what it has and raises the device's hand-off flag.
        uint64_t* slots = flagged + (int64_t)g * S * MB * 256;
        if (reducer) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                publish_flagged(slots + ((int64_t)z * MB + blk) * 256 + v * 64 + lane, sum[v]);
        }
        __shared__ uint32_t s_old;
        if (tid == 0) s_old = take_ticket(counters + g);
        __syncthreads();  // (also: every wave is done reading red)
        if (s_old != (uint32_t)(S - 1)) return;       // (uniform in the workgroup)
        if (tid == 0) reset_counter(counters + g);  // all splits arrived
        if (wave < S) {
            uint64_t* mine = slots + (int64_t)wave * MB * 256 + lane;
            if (wave != z) {
                float p[4 * MB];
                if (!gather_flagged<4 * MB>(mine, 64, polls, p) && lane == 0) raise_flag(kFlagHandoff);
#pragma unroll
                for (int b = 0; b < MB; ++b) red[wave][b][lane] = f4v{p[4 * b], p[4 * b + 1], p[4 * b + 2], p[4 * b + 3]};
            }
#pragma unroll
            for (int k = 0; k < 4 * MB; ++k) clear_flagged(mine + k * 64);
        }
        if (reducer) red[z][blk][lane] = sum;
        __syncthreads();
        if (!reducer) return;
        f4v t = red[0][blk][lane];
        for (int zz = 1; zz < S; ++zz) t += red[zz][blk][lane];
        sum = t;
    }
    if (!reducer) return;

    // 16x16 MFMA result layout: lane l holds column l % 16, rows 4 * (l / 16) + v.
    const int col = g * 16 + r16;
    if (col < N) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 16 * blk + 4 * grp + v;
            if (row < M) out[(int64_t)row * N + col] = to_bf16(alpha * sum[v]);
        }
    }
}

// ---------------------------------------------------------------------------
// Mid-size kernel: the waves of a workgroup split K.
//
// For GEMMs with a few hundred rows the large-M kernel has too few tiles to
// fill the machine without splitting K across workgroups, and small wave
// tiles make every operand block be decoded by several waves.  Here each of
// the WAVES waves owns the whole BM x BN tile (BM/32 x BN/32 blocks of
// v_mfma_f32_32x32x16_f16) over every WAVES-th panel of the workgroup's K
// range, so each element is decoded exactly once per tile and the waves
// share nothing until the end: no LDS staging and no barriers in the main
// loop.  Lane l of a 32-row block reads row l % 32, half l / 32 of a panel
// (16 bytes of codes, 2 bytes of scales) straight from HBM into registers
// -- a wave's reads of one block are 1 KB contiguous -- with DEPTH panels of
// loads in flight; the panel's offset is the loads' scalar offset.  At the end the wave tiles are added in LDS in wave order, then
// (split_k > 1) across workgroups by the last arrival in split order.
// Tiles: 128 x 64 (four waves), 64 x 64, 64 x 32 and 32 x 32 (eight waves).
// The smaller tiles cost more decode work per multiply-add but give enough
// workgroups to fill the CUs without splitting K across workgroups, whose
// hand-off costs more than that work at these sizes; they also hold fewer
// registers (about 120 and 90 per lane against 177), so two or three of
// their workgroups share a CU.
// ---------------------------------------------------------------------------
// (Plain arguments, operands and geometry first, so that those can be
// preloaded into scalar registers before the waves start.)
template <int BM, int BN, int WAVES, bool SPLIT>
__global__ void __launch_bounds__(WAVES * 64) wsplit_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, int Mp, int Np,
    int P, int tiles_n, int split_k, uint16_t* __restrict__ out, float* partials,
    uint32_t* counters, float alpha, int M, int N) {
    constexpr int MI = BM / 32;
    constexpr int NI = BN / 32;
    // panels of loads in flight per wave (ring of DEPTH slots); 2 measured
    // 2-15% faster than 4 (fewer registers held by loads) at 32..4096 rows
    constexpr int DEPTH = 2;
    __shared__ __attribute__((aligned(16))) float red[WAVES][MI * NI * 16][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: scalar load offsets)
    const int q = lane & 31, h = lane >> 5;

    const int S = SPLIT ? split_k : 1;
    int bid = blockIdx.x;
    const int total = gridDim.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int z = bid % S;
    const int t = bid / S;
    const int tm = t / tiles_n, tn = t % tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    const int nst = P / 2;
    const int p0 = 2 * (int)((int64_t)z * nst / S);
    const int p1 = 2 * (int)((int64_t)(z + 1) * nst / S);
    // this wave's panels: p0 + wave, p0 + wave + WAVES, ...
    const int count = (p1 - p0 > wave) ? (p1 - p0 - wave + WAVES - 1) / WAVES : 0;

    // Lane byte offsets inside one panel: the lane's row (clamped to the
    // padded operand; results of clamped rows are not stored), half h of its
    // 32 code bytes and of its 4 scale bytes.  The panel's own offset is
    // wave-uniform and goes into the loads' scalar offset, so addresses cost
    // no vector instructions.
    uint32_t a_code[MI], a_sc[MI], b_code[NI], b_sc[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const uint32_t r = (uint32_t)min(m0 + i * 32 + q, Mp - 1);
        a_code[i] = r * 32u + (uint32_t)h * 16u;
        a_sc[i] = r * 4u + (uint32_t)h * 2u;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const uint32_t r = (uint32_t)min(n0 + j * 32 + q, Np - 1);
        b_code[j] = r * 32u + (uint32_t)h * 16u;
        b_sc[j] = r * 4u + (uint32_t)h * 2u;
    }
    const __amdgpu_buffer_rsrc_t rac = make_rsrc(a_codes, (uint32_t)P * Mp * 32u);
    const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_scales, (uint32_t)P * Mp * 4u);
    const __amdgpu_buffer_rsrc_t rbc = make_rsrc(b_codes, (uint32_t)P * Np * 32u);
    const __amdgpu_buffer_rsrc_t rbs = make_rsrc(b_scales, (uint32_t)P * Np * 4u);

    struct Regs {
        uint4 ca[MI], cb[NI];
        uint32_t sa[MI], sb[NI];
    };
    // k-th panel of this wave.  Unconditional (count > 0): past the wave's
    // last panel it reads that panel again, and compute() then gives the
    // slot zero scales, so the compiler's wait counts stay exact (a branch
    // around the loads made every ring slot wait for all of them).
    auto load = [&](int k, Regs& r) {
        const uint32_t pnl = (uint32_t)(p0 + wave + min(k, count - 1) * WAVES);
        const uint32_t sa_off = pnl * (uint32_t)Mp, sb_off = pnl * (uint32_t)Np;  // rows before
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            r.ca[i] = load16(rac, a_code[i], sa_off * 32u);
            r.sa[i] = __builtin_amdgcn_raw_buffer_load_b16(ras, a_sc[i], sa_off * 4u, 0);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            r.cb[j] = load16(rbc, b_code[j], sb_off * 32u);
            r.sb[j] = __builtin_amdgcn_raw_buffer_load_b16(rbs, b_sc[j], sb_off * 4u, 0);
        }
    };

    f16v acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto compute = [&](const Regs& r, bool live) {  // live: a panel of the wave (wave-uniform)
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

    if (count > 0) {
        Regs ring[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load(d, ring[d]);
        // The first panels are taken as they arrive, here; otherwise the
        // compiler merges these loads with the loop's own (same form, other
        // index) into one load at the top of each iteration, which waits
        // for the panel it just asked for instead of one issued a step ahead.
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
        // 64 x 64 and 64 x 32 tiles are software-pipelined: each sub-step's
        // MFMAs run while the next sub-step's operands are decoded -- across
        // panels too, so the next panel's scales and first sub-step are
        // decoded under this panel's last MFMAs -- and a slot's loads go out
        // as soon as its last sub-step is decoded.  Measured 3-5% faster
        // with 64 x 64 tiles (512 x 2048 x 6144 14.65 -> 14.2 us) and 2% with
        // 64 x 32 (512 x 768 x 6144), but 1.5-3% slower with 32 x 32 and
        // 128 x 64 tiles, which keep the plain loop.
        constexpr bool PIPE = WAVES == 8 && BM * BN >= 64 * 32;
        if constexpr (PIPE) {
            h2 sa[MI], sb[NI];
            h8 av[MI], bv[NI];
            auto scales = [&](const Regs& r, bool live) {
#pragma unroll
                for (int i = 0; i < MI; ++i) sa[i] = e4m3x2_lo(live ? r.sa[i] : 0u);
#pragma unroll
                for (int j = 0; j < NI; ++j) sb[j] = e4m3x2_lo(live ? r.sb[j] : 0u);
            };
            auto decode = [&](const Regs& r, int s, h8* an, h8* bn) {
#pragma unroll
                for (int i = 0; i < MI; ++i) an[i] = decode8(word_of(r.ca[i], s), scale_of(sa[i], s));
#pragma unroll
                for (int j = 0; j < NI; ++j) bn[j] = decode8(word_of(r.cb[j], s), scale_of(sb[j], s));
            };
            auto mfmas = [&]() {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
            };
            scales(ring[0], true);
            decode(ring[0], 0, av, bv);
            for (int k = 0; k < count; k += DEPTH) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    const int dn = (d + 1) % DEPTH;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        h8 an[MI], bn[NI];
                        if (s < 3) {
                            decode(ring[d], s + 1, an, bn);
                            if (s == 2) load(k + d + DEPTH, ring[d]);  // ring[d] fully decoded
                        } else {
                            scales(ring[dn], k + d + 1 < count);  // panel k + d + 1 (zeros past the end)
                            decode(ring[dn], 0, an, bn);
                        }
                        mfmas();
#pragma unroll
                        for (int i = 0; i < MI; ++i) av[i] = an[i];
#pragma unroll
                        for (int j = 0; j < NI; ++j) bv[j] = bn[j];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            for (int k = 0; k < count; k += DEPTH) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    compute(ring[d], k + d < count);  // panel k + d (zeros past the end)
                    load(k + d + DEPTH, ring[d]);
                    // (each slot's loads go out right after its MFMAs, not
                    // after the next slot's: the scheduler would sink them)
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    // Add the wave tiles in wave order.
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) red[wave][(i * NI + j) * 16 + v][lane] = acc[i][j][v];
    __syncthreads();
    constexpr int IDX = MI * NI * 16;  // accumulator slots per lane
    static_assert(IDX % WAVES == 0, "every wave adds the same number of slots");
    constexpr int PER = IDX / WAVES;   // slots wave w adds: w, w + WAVES, ...
    float sum[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int idx = wave + u * WAVES;
        float x = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) x += red[w][idx][lane];
        sum[u] = x;
    }

    if (SPLIT) {
        // publish this workgroup's tile (slot order idx * 64 + lane); the
        // last arrival adds the S partial tiles in split order
        float* mine = partials + ((int64_t)t * S + z) * (BM * BN);
#pragma unroll
        for (int u = 0; u < PER; ++u) publish(mine + (wave + u * WAVES) * 64 + lane, sum[u]);
        __shared__ int s_last;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = arrive(counters + t);
            s_last = (old == (uint32_t)(S - 1));
            if (s_last) reset_counter(counters + t);  // all splits arrived
        }
        __syncthreads();
        if (!s_last) return;
        const float* all = partials + (int64_t)t * S * (BM * BN);
#pragma unroll
        for (int u = 0; u < PER; ++u) sum[u] = 0.0f;
        for (int zz = 0; zz < S; ++zz) {  // one batch of independent loads per split
            float part[PER];
#pragma unroll
            for (int u = 0; u < PER; ++u)
                part[u] = fetch(all + (int64_t)zz * (BM * BN) + (wave + u * WAVES) * 64 + lane);
#pragma unroll
            for (int u = 0; u < PER; ++u) sum[u] += part[u];
        }
    }

    // Epilogue: slot idx = (i * NI + j) * 16 + v of lane l is row
    // i*32 + 8*(v/4) + 4*(l/32) + v%4, column j*32 + l%32 of the tile.
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int idx = wave + u * WAVES;
        const int v = idx & 15, ij = idx >> 4;
        const int i = ij / NI, j = ij % NI;
        const int row = m0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        const int col = n0 + j * 32 + q;
        if (row < M && col < N) out[(int64_t)row * N + col] = to_bf16(alpha * sum[u]);
    }
}

// ---------------------------------------------------------------------------
// Dot-product kernel for M <= MR (MR <= 4): decode-sized GEMMs with one to
// four rows of A, bound by streaming B and by memory latency.
//
// With so few rows an MFMA would spend most of its decode work on the
// padding rows of A, and one workgroup per 16 columns leaves most CUs idle.
// Here each wave owns one row n of B over the whole of K, so there is no
// cross-wave or cross-workgroup reduction, and nothing goes through LDS:
//   * lane l takes half-panels l, l+64, ... of row n of B and the same
//     half-panels of the MR rows of A (16 bytes of codes and 2 bytes of
//     scales each, A from the L2 after its first reader); every load of a
//     batch is issued before the first wait, so one memory round trip
//     covers K up to 8192, and each half-panel is worked on as soon as its
//     own loads are in;
//   * codes of both operands are widened to fp16 without their scales
//     (v_cvt_scalef32_pk_f16_fp4, scale 1.0) and dotted in pairs
//     (v_dot2_f32_f16); inside a 16-element block the code products are
//     multiples of 1/4 below 36, so the block sum is exact in FP32, and
//     one FMA applies the product of the two block scales (exact: at most
//     8 significant bits, and the scaled block sum at most 20) while adding
//     the block to the running sum -- the only rounding, as in an MFMA
//     accumulator;
//   * the 64 lane sums are added in a fixed order with DPP moves (within
//     rows of 16 lanes, then across rows), and lane 63 stores.
// ---------------------------------------------------------------------------

// Source operand of a DPP move with zero fill for lanes it does not cover.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_src(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, true));
}

// Sum of x over the 64 lanes of the wave, complete in lane 63: windows of
// 2, 4, 8 and 16 lanes inside each row of 16 (row_shr:1,2,4,8), then row 0
// into row 1 and row 2 into row 3 (row_bcast:15), then rows 0-1 into rows
// 2-3 (row_bcast:31).  The order of the additions is fixed.
__device__ __forceinline__ float wave_sum_lane63(float x) {
    x += dpp_src<0x111, 0xF>(x);
    x += dpp_src<0x112, 0xF>(x);
    x += dpp_src<0x114, 0xF>(x);
    x += dpp_src<0x118, 0xF>(x);
    x += dpp_src<0x142, 0xA>(x);
    x += dpp_src<0x143, 0xC>(x);
    return x;
}

// The dot products of one batch: lane `lane` holds half-panels base + lane,
// base + lane + 64, ... of B (codes bw, scale words bsc) and of the MR rows
// of A (aw, asc); a half-panel past hp_total is weighted by zero.
template <int MR, int HPL>
__device__ __forceinline__ void gemv_batch(const uint4 (&bw)[HPL], const uint32_t (&bsc)[HPL],
                                           const uint4 (&aw)[HPL][MR],
                                           const uint32_t (&asc)[HPL][MR], int base, int lane,
                                           int hp_total, float (&acc)[MR]) {
#pragma unroll
    for (int i = 0; i < HPL; ++i) {
        const bool live = base + lane + 64 * i < hp_total;
        const h2 sb = e4m3x2_lo(bsc[i]);       // B scales of the half-panel's two blocks
        h2 sa[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) sa[m] = e4m3x2_lo(asc[i][m]);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            float bs[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) bs[m] = 0.0f;
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
                const uint32_t w = word_of(bw[i], 2 * blk + wd);
                const h2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
                const h2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
                const h2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
                const h2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const uint32_t v = word_of(aw[i][m], 2 * blk + wd);
                    bs[m] = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 0), b0, bs[m], false);
                    bs[m] = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 1), b1, bs[m], false);
                    bs[m] = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 2), b2, bs[m], false);
                    bs[m] = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 3), b3, bs[m], false);
                }
            }
            const float sbf = live ? (float)sb[blk] : 0.0f;
#pragma unroll
            for (int m = 0; m < MR; ++m)
                acc[m] = __builtin_fmaf(bs[m], live ? (float)sa[m][blk] * sbf : 0.0f, acc[m]);
        }
    }
}

// Four waves (rows of B) per workgroup: 4 consecutive rows share every
// 128-byte line of a packed panel (32 bytes each), so each workgroup reads
// whole lines.  Workgroups are dealt to the 8 XCDs in turn; the workgroup
// index is remapped to give each XCD a contiguous range of rows, so that
// neighbouring workgroups share their XCD's L2 (1 x 768 x 6144: 2.84 ->
// 2.65 us warm, 3.80 -> 3.60 us with the operands beyond the last-level
// cache, and the HBM fetches fell from 1.85x to 1.07x of the algorithmic
// bytes).  Fewer waves per workgroup for small N (more workgroups) was
// faster on some boxes and up to 12% slower on others with the operands
// beyond the last-level cache, where a line is then split between
// workgroups.
constexpr int kGemvWaves = 4;

// Plain arguments rather than the launch structure, in the order the kernel
// needs them (the operands and their geometry first): the leading ones can
// then be preloaded into scalar registers before the waves start, instead
// of being fetched from memory after.
template <int MR, int HPL>
__global__ void __launch_bounds__(64 * kGemvWaves) gemv_kernel(
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales,
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int Np, int Mp,
    int P, int total, uint16_t* __restrict__ out, float alpha, int M, int N) {
    const int lane = threadIdx.x & 63;
    // XCD x = blockIdx % 8 takes ranks [x q + min(x, r), ...) of the
    // total = 8 q + r workgroups (the grid), one after the other (a bijection).
    const int q8 = total >> 3, r8 = total & 7;
    const int x = blockIdx.x & 7;
    const int bid = x * q8 + min(x, r8) + (int)(blockIdx.x >> 3);
    const int n = bid * kGemvWaves + (threadIdx.x >> 6);  // B row (< Np: the grid is Np / 4)
    const int hp_total = P * 2;               // 32-element half-panels along K

    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.0f;

    // Batches of HPL half-panels per lane.  The loads are unconditional (a
    // lane past the end reads the last half-panel again and its block sums
    // are weighted by zero), so the compiler can wait for each half-panel's
    // loads alone and work on the first while the later ones arrive.
    for (int base = 0; base < hp_total; base += 64 * HPL) {
        uint4 bw[HPL], aw[HPL][MR];
        uint32_t bsc[HPL], asc[HPL][MR];
#pragma unroll
        for (int i = 0; i < HPL; ++i) {
            const int hp = min(base + lane + 64 * i, hp_total - 1);
            const int64_t panel = hp >> 1;
            const int half = hp & 1;
            const int64_t brow = panel * Np + n;
            bw[i] = *reinterpret_cast<const uint4*>(b_codes + brow * 32 + half * 16);
            bsc[i] = *reinterpret_cast<const uint16_t*>(b_scales + brow * 4 + half * 2);
            // rows MR-1 < 16 <= Mp: padding rows of A are zeros in memory
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const int64_t arow = panel * Mp + m;
                aw[i][m] = *reinterpret_cast<const uint4*>(a_codes + arow * 32 + half * 16);
                asc[i][m] = *reinterpret_cast<const uint16_t*>(a_scales + arow * 4 + half * 2);
            }
        }
        // The epilogue's arguments (past the preloaded ones) are fetched
        // while the operand loads are in flight rather than after the dot
        // products, where their scalar load sat on the kernel's last steps:
        // 1-2 x 768 x 6144 2.79 -> 2.77 and 3.23 -> 3.15 us.
        asm volatile("" ::"s"(alpha), "s"(M), "s"(N), "s"(out));
        gemv_batch<MR, HPL>(bw, bsc, aw, asc, base, lane, hp_total, acc);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = wave_sum_lane63(acc[m]);
    if (lane == 63 && n < N) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
            if (m < M) out[(int64_t)m * N + n] = to_bf16(alpha * acc[m]);
    }
}

// The dot-product kernel with the quantisation of A folded in: A arrives as
// fp32 or bfloat16 rows (T: float or uint16_t), and the workgroup quantises
// them itself, with the quantiser's rule and functions, so that the result
// is bit for bit that of nvfp4_quantize followed by the dot-product kernel
// -- one launch instead of two for a decode step's GEMM.
//   * Every wave first issues the loads of its row of B (as above); while
//     they are in flight, the workgroup's lanes quantise the MR rows of A
//     (two lanes per 16-element block, the block's amax combined over the
//     pair by one DPP exchange) into LDS in the packed form the dot products
//     read: codes [panel][row][32 bytes], scales [panel][row][4 bytes], rows
//     M..MR-1 and the blocks past K as zeros;
//   * after one barrier each lane reads its half-panels of A from LDS and
//     the dot products run exactly as in gemv_kernel.
// Every workgroup quantises all of A (it needs all of it), so WAVES rows of
// B per workgroup trade the quantisation work per lane against the number
// of workgroups streaming B.
// Rows of B per workgroup.
constexpr int kGemvQuantWaves = 8;

template <int MR, int HPL, int WAVES, typename T>
__global__ void __launch_bounds__(64 * WAVES) gemv_quant_kernel(
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales,
    const T* __restrict__ x, int64_t ldx, int Np, int P, int total, int K,
    uint16_t* __restrict__ out, float alpha, int M, int N) {
    __shared__ __attribute__((aligned(16))) uint8_t qa_codes[kGemvQuantElems / 2];
    __shared__ __attribute__((aligned(16))) uint8_t qa_scales[kGemvQuantElems / 16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int q8 = total >> 3, r8 = total & 7;
    const int xcd = blockIdx.x & 7;
    const int bid = xcd * q8 + min(xcd, r8) + (int)(blockIdx.x >> 3);
    const int n = bid * WAVES + (tid >> 6);   // B row (< Np: the grid is Np / WAVES)
    const int hp_total = P * 2;

    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.0f;

    uint4 bw[HPL];
    uint32_t bsc[HPL];
    auto load_b = [&](int base) {
#pragma unroll
        for (int i = 0; i < HPL; ++i) {
            const int hp = min(base + lane + 64 * i, hp_total - 1);
            const int64_t brow = (int64_t)(hp >> 1) * Np + n;
            bw[i] = *reinterpret_cast<const uint4*>(b_codes + brow * 32 + (hp & 1) * 16);
            bsc[i] = *reinterpret_cast<const uint16_t*>(b_scales + brow * 4 + (hp & 1) * 2);
        }
    };
    auto batch = [&](int base) {
        uint4 aw[HPL][MR];
        uint32_t asc[HPL][MR];
#pragma unroll
        for (int i = 0; i < HPL; ++i) {
            const int hp = min(base + lane + 64 * i, hp_total - 1);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const int slot = (hp >> 1) * MR + m;
                aw[i][m] = *reinterpret_cast<const uint4*>(qa_codes + slot * 32 + (hp & 1) * 16);
                asc[i][m] = *reinterpret_cast<const uint16_t*>(qa_scales + slot * 4 + (hp & 1) * 2);
            }
        }
        gemv_batch<MR, HPL>(bw, bsc, aw, asc, base, lane, hp_total, acc);
    };

    // Quantise A: half-block j = (row m, 16-element block b of Kp, half h);
    // the two halves of a block are adjacent lanes, and the work is a whole
    // number of pairs, so both lanes of a pair take the same rounds.  Loads
    // are clamped into the input (row to M - 1, elements to end by K); what
    // they bring in for padding rows or past K is written as zero.  The
    // loads of the first QR rounds go out before B's (the wait for them
    // then does not include B's, which arrive in order behind them).
    const int items = MR * P * 8;
    auto load_x = [&](int j, float (&v)[8]) {
        const int m = j / (P * 8), b = (j >> 1) % (P * 4), h = j & 1;
        const T* src = x + (int64_t)min(m, M - 1) * ldx + min(b * 16 + h * 8, K - 8);
        if constexpr (sizeof(T) == 2) {
            const uint4 q = *reinterpret_cast<const uint4*>(src);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
                v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
            }
        } else {
            const uint4 q0 = reinterpret_cast<const uint4*>(src)[0];
            const uint4 q1 = reinterpret_cast<const uint4*>(src)[1];
            const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(float, w[i]);
        }
    };
    auto quantise = [&](int j, const float (&v)[8]) {
        const int m = j / (P * 8), b = (j >> 1) % (P * 4), h = j & 1;
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
        const float o = __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false));
        amax = __builtin_fmaxf(amax, o);
        const uint32_t sb = e4m3_nearest(amax / 6.0f);
        const float sv = e4m3_value(sb);
        const bool has = m < M && b * 16 < K;
        const uint32_t w = has ? e2m1_word(v, e2m1_search(sv), sv > 0.0f ? 7u : 0u) : 0u;
        const int slot = (b >> 2) * MR + m;
        *reinterpret_cast<uint32_t*>(qa_codes + slot * 32 + (b & 3) * 8 + h * 4) = w;
        if (h == 0) qa_scales[slot * 4 + (b & 3)] = has ? (uint8_t)sb : (uint8_t)0;
    };
    constexpr int QR = 4;
    constexpr int STRIDE = 64 * WAVES;
    float xv[QR][8];
#pragma unroll
    for (int r = 0; r < QR; ++r) load_x(min(tid + r * STRIDE, items - 1), xv[r]);  // (clamped: unused past items)
    __builtin_amdgcn_sched_barrier(0);  // (keeps these loads ahead of B's)
    load_b(0);
    __builtin_amdgcn_sched_barrier(0);
    // (every loaded value is taken here, after B's loads were issued: with
    // the values used only inside the branches below, the compiler would
    // move each load into its branch, behind B's)
#pragma unroll
    for (int r = 0; r < QR; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(xv[r][i]));
#pragma unroll
    for (int r = 0; r < QR; ++r)
        if (tid + r * STRIDE < items) quantise(tid + r * STRIDE, xv[r]);
    for (int j = tid + QR * STRIDE; j < items; j += STRIDE) {
        float v[8];
        load_x(j, v);
        quantise(j, v);
    }
    __syncthreads();

    batch(0);
    for (int base = 64 * HPL; base < hp_total; base += 64 * HPL) {
        load_b(base);
        batch(base);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = wave_sum_lane63(acc[m]);
    if (lane == 63 && n < N) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
            if (m < M) out[(int64_t)m * N + n] = to_bf16(alpha * acc[m]);
    }
}

}  // namespace

hipError_t take_device_flags(uint32_t* flags) {
    *flags = 0;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_device_flags), sizeof(uint32_t));
    if (e == hipSuccess && *flags) {
        const uint32_t zero = 0;
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_device_flags), &zero, sizeof(uint32_t));
    }
    return e;
}

size_t tile_partial_floats(int cfg, const GemmArgs& a) {
    const TileShape s = tile_shape(cfg);
    if (a.split_k > 1) return (size_t)a.tile_count * a.split_k * s.bm * s.bn;
    if (a.tail_tiles > 0) return (size_t)a.tail_tiles * a.tail_split * s.bm * s.bn;
    return 0;
}
size_t tile_counters(int cfg, const GemmArgs& a) {
    (void)cfg;
    if (a.split_k > 1) return (size_t)a.tile_count;
    if (a.tail_tiles > 0) return (size_t)a.tail_tiles;
    return 0;
}
size_t skinny_flagged_words(const GemmArgs& a) {
    const int mb = (a.M + 15) / 16;
    return a.split_k <= 1 ? 0 : (size_t)(a.Np / 16) * a.split_k * mb * 256;
}
size_t skinny_counters(const GemmArgs& a) {
    return a.split_k <= 1 ? 0 : (size_t)(a.Np / 16);
}

// Workgroups of a tile kernel that are resident on the device at once
// (CUs x workgroups per CU), cached per device and configuration.
int resident_tiles(int cfg, int device) {
    constexpr int kMaxDevices = 64;
    static int cache[kMaxDevices][3] = {};
    if (device < 0 || device >= kMaxDevices || cfg < 0 || cfg > 2) return 0;
    int& r = cache[device][cfg];
    if (r == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
            return 0;
        const void* k = cfg == TILE_256x256   ? (const void*)tile_kernel<256, 256, 8, false>
                        : cfg == TILE_128x128 ? (const void*)tile_kernel<128, 128, 8, false>
                                              : (const void*)tile_kernel<64, 64, 8, false>;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 256, 0) != hipSuccess)
            return 0;
        r = cus * per_cu;
    }
    return r;
}

namespace {
hipError_t launch_tile_range(int cfg, const GemmArgs& a, int device, hipStream_t stream);
}  // namespace

hipError_t launch_tile(int cfg, const GemmArgs& a, int device, hipStream_t stream) {
    if (a.split_k > 1 || a.tail_tiles <= 0) return launch_tile_range(cfg, a, device, stream);
    // Tail: the full rounds of tiles first (persistent, whole K range), then
    // the last tail_tiles tiles with K split tail_split ways, so that they
    // occupy the CUs a last partial round would leave idle.  The launches
    // are ordered on the stream; the second one's workgroups reduce their
    // partial tiles through the workspace as any split-K launch does.
    GemmArgs head = a;
    head.tile_count = a.tile_count - a.tail_tiles;
    head.tail_tiles = 0;
    const hipError_t e = launch_tile_range(cfg, head, device, stream);
    if (e != hipSuccess) return e;
    GemmArgs tail = a;
    tail.tile_begin = a.tile_begin + head.tile_count;
    tail.tile_count = a.tail_tiles;
    tail.split_k = a.tail_split;
    tail.tail_tiles = 0;
    return launch_tile_range(cfg, tail, device, stream);
}

namespace {
hipError_t launch_tile_range(int cfg, const GemmArgs& a, int device, hipStream_t stream) {
    const int tiles = a.tile_count;
    const bool split = a.split_k > 1;
    int blocks = tiles * a.split_k;
    if (!split && a.P >= 8) {
        // persistent grid: at most one workgroup per resident slot; when
        // workgroups take several tiles their count is a multiple of 8, so
        // that each keeps its XCD's tile range.  (The kernel's look-ahead of
        // 7 panels may reach into the next tile only, hence K >= 512.)
        const int r = resident_tiles(cfg, device);
        if (r <= 0) return hipErrorInvalidValue;
        if (tiles > r) blocks = r >= 8 ? r / 8 * 8 : r;
    }
    const dim3 grid((unsigned)blocks);
    const dim3 block(256);
    switch (cfg) {
        case TILE_256x256:
            if (split) hipLaunchKernelGGL((tile_kernel<256, 256, 8, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((tile_kernel<256, 256, 8, false>), grid, block, 0, stream, a);
            break;
        case TILE_128x128:
            if (split) hipLaunchKernelGGL((tile_kernel<128, 128, 8, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((tile_kernel<128, 128, 8, false>), grid, block, 0, stream, a);
            break;
        default:
            if (split) hipLaunchKernelGGL((tile_kernel<64, 64, 8, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((tile_kernel<64, 64, 8, false>), grid, block, 0, stream, a);
            break;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_grouped_tile(const GemmArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((tile_kernel<256, 256, 8, false, true>), dim3((unsigned)a.tile_count), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

size_t wsplit_partial_floats(int cfg, const GemmArgs& a) {
    if (a.split_k <= 1) return 0;
    const TileShape s = wsplit_shape(cfg);
    return (size_t)a.tiles_m * a.tiles_n * a.split_k * s.bm * s.bn;
}

hipError_t launch_wsplit(int cfg, const GemmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n * a.split_k));
    const bool split = a.split_k > 1;
#define NVFP4_WSPLIT(BM, BN, W, S, T)                                                            \
    hipLaunchKernelGGL((wsplit_kernel<BM, BN, W, S>), grid, dim3(T), 0, stream, a.a_codes,       \
                       a.a_scales, a.b_codes, a.b_scales, a.Mp, a.Np, a.P, a.tiles_n, a.split_k, \
                       a.out, a.partials, a.counters, a.alpha, a.M, a.N)
    switch (cfg) {
        case WSPLIT_64x64:
            if (split) NVFP4_WSPLIT(64, 64, 8, true, 512);
            else NVFP4_WSPLIT(64, 64, 8, false, 512);
            break;
        case WSPLIT_64x32:
            if (split) NVFP4_WSPLIT(64, 32, 8, true, 512);
            else NVFP4_WSPLIT(64, 32, 8, false, 512);
            break;
        case WSPLIT_32x32:
            if (split) NVFP4_WSPLIT(32, 32, 8, true, 512);
            else NVFP4_WSPLIT(32, 32, 8, false, 512);
            break;
        default:  // WSPLIT_128x64
            if (split) NVFP4_WSPLIT(128, 64, 4, true, 256);
            else NVFP4_WSPLIT(128, 64, 4, false, 256);
            break;
    }
#undef NVFP4_WSPLIT
    return hipGetLastError();
}

hipError_t launch_gemv(const GemmArgs& a, hipStream_t stream) {
    // Np is a multiple of 16, so whole workgroups cover it.  One batch of
    // loads covers K up to 8192 (256 half-panels); a shorter K takes as
    // few half-panels per lane as it needs.
    const dim3 grid((unsigned)(a.Np / kGemvWaves)), block(64 * kGemvWaves);
    const int hpl = (int)std::min<int64_t>(4, (2 * (int64_t)a.P + 63) / 64);
    const int mr = a.M <= 1 ? 1 : a.M <= 2 ? 2 : 4;
    switch (mr * 8 + hpl) {
#define NVFP4_GEMV_CASE(MR, HPL) \
        case MR * 8 + HPL: hipLaunchKernelGGL((gemv_kernel<MR, HPL>), grid, block, 0, stream, a.b_codes, \
                                               a.b_scales, a.a_codes, a.a_scales, a.Np, a.Mp, a.P,  \
                                               (int)grid.x, a.out, a.alpha, a.M, a.N); break;
        NVFP4_GEMV_CASE(1, 1) NVFP4_GEMV_CASE(1, 2) NVFP4_GEMV_CASE(1, 3) NVFP4_GEMV_CASE(1, 4)
        NVFP4_GEMV_CASE(2, 1) NVFP4_GEMV_CASE(2, 2) NVFP4_GEMV_CASE(2, 3) NVFP4_GEMV_CASE(2, 4)
        NVFP4_GEMV_CASE(4, 1) NVFP4_GEMV_CASE(4, 2) NVFP4_GEMV_CASE(4, 3) NVFP4_GEMV_CASE(4, 4)
#undef NVFP4_GEMV_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_quant(const GemvQuantArgs& a, hipStream_t stream) {
    constexpr int W = kGemvQuantWaves;
    const dim3 grid((unsigned)(a.Np / W)), block(64 * W);   // Np % 16 == 0
    const int hpl = std::min(4, (2 * a.P + 63) / 64);
    const int mr = gemv_rows(a.M);
    switch ((mr * 8 + hpl) * 2 + (a.bf16 ? 1 : 0)) {
#define NVFP4_GEMVQ_CASE(MR, HPL)                                                                  \
        case (MR * 8 + HPL) * 2:                                                                   \
            hipLaunchKernelGGL((gemv_quant_kernel<MR, HPL, W, float>), grid, block, 0, stream,     \
                               a.b_codes, a.b_scales, static_cast<const float*>(a.x), a.ldx, a.Np, \
                               a.P, (int)grid.x, a.K, a.out, a.alpha, a.M, a.N);                   \
            break;                                                                                 \
        case (MR * 8 + HPL) * 2 + 1:                                                               \
            hipLaunchKernelGGL((gemv_quant_kernel<MR, HPL, W, uint16_t>), grid, block, 0, stream,  \
                               a.b_codes, a.b_scales, static_cast<const uint16_t*>(a.x), a.ldx,    \
                               a.Np, a.P, (int)grid.x, a.K, a.out, a.alpha, a.M, a.N);             \
            break;
        NVFP4_GEMVQ_CASE(1, 1) NVFP4_GEMVQ_CASE(1, 2) NVFP4_GEMVQ_CASE(1, 3) NVFP4_GEMVQ_CASE(1, 4)
        NVFP4_GEMVQ_CASE(2, 1) NVFP4_GEMVQ_CASE(2, 2) NVFP4_GEMVQ_CASE(2, 3) NVFP4_GEMVQ_CASE(2, 4)
        NVFP4_GEMVQ_CASE(4, 1) NVFP4_GEMVQ_CASE(4, 2) NVFP4_GEMVQ_CASE(4, 3) NVFP4_GEMVQ_CASE(4, 4)
#undef NVFP4_GEMVQ_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.Np / 16) * a.split_k));
    const dim3 block(kSkinnyWaves * 64);
    const int mb = (a.M + 15) / 16;
    // Work units in flight per wave: as many as a wave's share of its split
    // needs, at most 4 (2 with more than two row blocks: 128 VGPRs at 16
    // waves), so that no unit is loaded and decoded only to be discarded.
    const int per_split = (a.P / 2 + a.split_k - 1) / a.split_k;
    const int need = (per_split + kSkinnyWaves - 1) / kSkinnyWaves;
    int units = std::max(1, std::min(need, mb <= 2 ? 4 : 2));
    if (mb == 2 && units == 3) units = 4;  // (3 units of two row blocks spill registers; 4 do not)
    switch (mb * 8 + units) {
#define NVFP4_SKINNY_CASE(MB, U) \
        case MB * 8 + U: hipLaunchKernelGGL((skinny_kernel<kSkinnyWaves, MB, U>), grid, block, 0, stream, \
                                            a.b_codes, a.b_scales, a.a_codes, a.a_scales, a.Np, a.Mp, \
                                            a.P, a.split_k, a.out, a.flagged, a.counters, a.alpha, a.M, \
                                            a.N, a.handoff_polls); break;
        NVFP4_SKINNY_CASE(1, 1) NVFP4_SKINNY_CASE(1, 2) NVFP4_SKINNY_CASE(1, 3) NVFP4_SKINNY_CASE(1, 4)
        NVFP4_SKINNY_CASE(2, 1) NVFP4_SKINNY_CASE(2, 2) NVFP4_SKINNY_CASE(2, 4)
        NVFP4_SKINNY_CASE(3, 1) NVFP4_SKINNY_CASE(3, 2)
        NVFP4_SKINNY_CASE(4, 1) NVFP4_SKINNY_CASE(4, 2)
#undef NVFP4_SKINNY_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}



}  // namespace nvfp4
