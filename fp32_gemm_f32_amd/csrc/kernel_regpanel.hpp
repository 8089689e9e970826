// kernel_regpanel.hpp -- the large-tile FP32 GEMM kernel: one wave per SIMD, each wave's
// operands for a whole K-panel held in registers.
//
// Same product and the same ladder of the pages as kernel_mfma.hpp ("Shared Memory
// Tiling", "The tiled kernel"; "SGEMM: 2D Register Tiling Visualizer", "Why 2D Register
// Tiling Dominates"), arranged for one wave per SIMD:
//
//  * A workgroup of 4 waves (2 x 2) owns a 256 x 256 tile of C; each wave owns 128 x 128
//    of it, 4 x 4 blocks of 32 x 32 accumulated by v_mfma_f32_32x32x2_f32, all 256
//    accumulator registers in AGPRs. Per 8 values of k a wave reads 4 A-values (one
//    ds_read_b128 per 32-row block) and 4 B-values (one ds_read_b128 per k-step covering
//    the 4 interleaved column blocks) per lane and issues 64 MFMAs: 8 reads per 64 outer
//    products of 32 x 32, the largest register tile the register file allows.
//  * LDS holds ONE panel (256 x 32 of A, 32 x 256 of B, 64 KiB). Global loads stage the
//    panel after next in registers (16 chunks of 16 bytes per thread) while the MFMAs run,
//    so a panel's loads have most of two panels' time to land. The whole panel's operands
//    are read from LDS into 128 registers per lane (32 ds_read_b128) ahead of use, which
//    frees LDS for the next panel early in the current one:
//        step t of a panel (16 steps of 16 MFMAs; group g = t / 4 of 8 k-values):
//        t 0        read group 3 of this panel
//        after t 1  barrier: every wave has read this panel
//        t 2, 3     write the staged next panel into LDS
//        t 4 .. 11  load the panel after it from global memory (2 chunks per step)
//        after t 7  barrier: the next panel is in LDS
//        t 8 .. 15  read groups 0, 1, 2 of the next panel (their registers are free)
//    Every memory instruction sits between MFMAs of the same wave; each barrier sits right
//    behind MFMAs that keep the matrix pipe busy while the four waves meet.
//  * No vector ALU work in the main loop. Measured on gfx950, each VALU instruction
//    placed among the MFMAs of a one-wave-per-SIMD kernel costs matrix-pipe time (about
//    4 % at 8192^3 for some 40 per panel), so every per-lane condition is resolved outside
//    the loop: offsets of rows past M and columns past N are set to kOob once; B rows past
//    the item's K range lie past its buffer resource's end and read as zero; a panel wholly
//    past the range gets an empty resource (a scalar choice). Only A values past the end of
//    the K range within the last, partial panel need zeroing; that panel is written in the
//    peeled second-to-last panel step (or the prologue), which applies the selects.
//  * Loads and stores use buffer resources, so out-of-range lanes read zeros and drop
//    stores, as in kernel_mfma.hpp. The LDS layouts are kernel_mfma.hpp's: A rows of 32
//    floats with the 16-byte chunk swizzle a_swizzle<8>, B rows of 256 floats as they are;
//    both read phases and both write phases are conflict-free.
//
// Items are kernel_mfma.hpp's: without SK, workgroup i computes tile i % tiles over split
// i / tiles of K (one split for the plain product; the plan gives this kernel whole tiles).
// With SK the grid is sk.tiles_dp workgroups of one whole tile each followed by sk.G
// stream-K workgroups, each walking the segments of its range of K-panel units
// (streamk.hpp): a segment that covers its whole tile stores it to C, any other stores its
// partial sums to the workgroup's workspace slot for k_streamk_fixup<256, 256> to add.
#pragma once

#include "kernel_mfma.hpp"

namespace sgemm {

namespace regpanel {
constexpr int BM = 256, BN = 256, BK = 32, WT = 128, THREADS = 256;
constexpr int A_TILE = BM * BK;                 // floats of A in LDS
constexpr int LDS_FLOATS = A_TILE + BK * BN;    // one panel, 64 KiB
constexpr int STEPS = 16;                       // k-steps of 2 per panel
constexpr int LOAD_STEPS = 8;                   // steps 4 .. 11 carry the global loads
static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS");


// Release/acquire of LDS only around the barrier: the wave waits for its own LDS accesses,
// not for the global loads it has in flight.
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
}  // namespace regpanel

// One item: the tile at (m0, n0) over K range [kb, ke), stored to C (at element offset
// c_off, the split's slice) or, for a partial stream-K tile (TO_WS), to workspace slot
// `slot`. Force-inlined into the kernels, so the plain kernel sees constant arguments and
// the stream-K kernel holds no accumulators or staging registers across its segments.
template <bool SK>
__device__ __forceinline__ void regpanel_item(const GemmArgs &p, float *lds, int m0, int n0,
                                              int kb, int ke, int64_t c_off, bool to_workspace,
                                              int slot)
{
    using namespace regpanel;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lo = lane & 31, h = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = p.M, N = p.N, lda = p.lda, ldb = p.ldb;
    // Resource sizes, in 32-bit scalar min/select chains (the panel loop must not need the
    // vector ALU, nor branch, for them). A panel's A resource starts at (m0, k0): when the
    // tile holds A's last row it ends at A's end, a_end - 4 k0 bytes on; otherwise a_end is
    // all ones and the size saturates to the full range (4 K < 2^31). A panel's B resource
    // starts at (k0, n0) and ends at the end of row ke - 1, so rows of later splits read as
    // zero; with more than BK rows left, BK + 1 rows cover every offset the loads use. The
    // host's offset check keeps these products below 2^31.
    const uint32_t a_end =
        M - m0 <= BM ? uint32_t((M - 1 - m0) * lda + p.K) * 4u : 0xffffffffu;

    // ---- staging: thread tid loads A rows a_r + 32 i (16-byte chunk a_q of the panel's
    // 32 columns) and B rows b_r + 4 i (chunk b_q of the tile's 256 columns), i < 8
    const int a_r = tid >> 3, a_q = tid & 7;
    const int b_r = tid >> 6, b_q = tid & 63;
    uint32_t a_v[8], b_v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a_v[i] = m0 + a_r + 32 * i < M ? uint32_t(a_r + 32 * i) * uint32_t(lda) * 4u + 16u * a_q
                                       : kOob;
        b_v[i] = n0 + 4 * b_q < N ? uint32_t(b_r + 4 * i) * uint32_t(ldb) * 4u + 16u * b_q
                                  : kOob;
    }
    static_assert(32 % a_swizzle_period<8>() == 0, "a thread's A rows share one swizzle");
    const int a_lds = a_r * BK + 4 * (a_q ^ a_swizzle<8>(a_r));
    const int b_lds = A_TILE + b_r * BN + 4 * b_q;
    f32x4 pa[8], pb[8];
    int kp = 0;   // first k of the staged panel
    __amdgpu_buffer_rsrc_t ra, rb;
    // loads [LO, HI) of the 16 staging chunks (A chunk j for j < 8, else B chunk j - 8) of
    // the panel at k0; LO == 0 also sets the panel's resources
    auto load = [&](int k0, int lo_j, int hi_j) {
        if (lo_j == 0) {
            kp = k0;
            const int64_t ea = int64_t(m0) * lda + k0, eb = int64_t(k0) * ldb + n0;
            const int rows = ke - k0;
            const uint32_t na = min(a_end - 4u * uint32_t(k0), kFullRange);
            const uint32_t nb =
                min(uint32_t((min(rows, BK + 1) - 1) * ldb + (N - n0)) * 4u, kFullRange);
            // a panel past the K range reads zeros (selects, not a branch: the panel loop
            // stays one block)
            ra = make_rsrc32(p.A + ea, rows > 0 ? na : 0u);
            rb = make_rsrc32(p.B + eb, rows > 0 ? nb : 0u);
        }
#pragma unroll
        for (int j = lo_j; j < hi_j; ++j) {
            if (j < 8) pa[j] = load_b128(ra, a_v[j]);
            else pb[j - 8] = load_b128(rb, b_v[j - 8]);
        }
    };
    // staged chunk j to LDS; TAIL zeroes the A elements at or past ke (the only panel that
    // can hold them is the last one, and only its write asks for this)
    auto write = [&](int j, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        if (j < 8) {
            f32x4 v = pa[j];
            if constexpr (TAIL) {
                const int kc = kp + 4 * a_q;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = kc + e < ke ? v[e] : 0.0f;
            }
            *reinterpret_cast<f32x4 *>(lds + a_lds + 32 * j * BK) = v;
        } else {
            *reinterpret_cast<f32x4 *>(lds + b_lds + 4 * (j - 8) * BN) = pb[j - 8];
        }
    };

    // ---- operands: group g of 8 k-values; oa[g][r] = A row block r (k 8 g + 4 h .. + 3 of
    // row 32 r + lo), ob[g][s] = B row 8 g + 4 h + s, columns 4 lo .. 4 lo + 3 of the wave
    const int a_row = (wm * WT + lo) * BK;
    const int a_sw = a_swizzle<8>(lo);
    const int b_col = A_TILE + wn * WT + 4 * lo;
    f32x4 oa[4][4], ob[4][4];
    auto read = [&](int g, int j) {   // j < 4: A row block j, else B step j - 4
        if (j < 4)
            oa[g][j] = *reinterpret_cast<const f32x4 *>(lds + a_row + 32 * j * BK +
                                                        4 * ((2 * g + h) ^ a_sw));
        else
            ob[g][j - 4] =
                *reinterpret_cast<const f32x4 *>(lds + b_col + (8 * g + 4 * h + (j - 4)) * BN);
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = f32x16{};

    // ---- prologue: panel 0 into LDS, panel 1 staged, groups 0..2 of panel 0 read (in the
    // order the loop expects: group 0 oldest)
    load(kb, 0, 16);
#pragma unroll
    for (int j = 0; j < 16; ++j) write(j, std::true_type{});
    lds_barrier();
#pragma unroll
    for (int g = 0; g < 3; ++g) {
#pragma unroll
        for (int j = 0; j < 8; ++j) read(g, j);
        __builtin_amdgcn_sched_barrier(0);
    }
    load(kb + BK, 0, 16);
    __builtin_amdgcn_sched_barrier(0);

    // One panel of 16 steps. NEXT: a later panel exists (write, load, barriers, reads of
    // the next panel); TAILW: the panel written here may be the partial last one.
    auto panel = [&](auto next_tag, auto tailw_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        static_for<0, STEPS>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            constexpr int g = t >> 2, s = t & 3;
            constexpr int nr = t == 0 ? 8 : !NEXT ? 0 : (t >= 8 && t < 12) ? 4 : t >= 12 ? 2 : 0;
            constexpr int nw = NEXT && (t == 2 || t == 3) ? 8 : 0;
            constexpr int nl = NEXT && t >= 4 && t < 4 + LOAD_STEPS ? 16 / LOAD_STEPS : 0;
            if constexpr (t == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) read(3, j);
            }
            if constexpr (nw > 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) write((t - 2) * 8 + j, tailw_tag);
            }
            if constexpr (nl > 0) load(t == 4 ? kp + BK : kp, (t - 4) * nl, (t - 3) * nl);
            if constexpr (NEXT && t >= 8 && t < 12) {
#pragma unroll
                for (int j = 0; j < 4; ++j) read((t - 8) >> 1, ((t - 8) & 1) * 4 + j);
            }
            if constexpr (NEXT && t >= 12) {
#pragma unroll
                for (int j = 0; j < 2; ++j) read(2, (t - 12) * 2 + j);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(oa[g][r][s], ob[g][s][c],
                                                                     acc[r][c], 0, 0, 0);
            // pin the step's order: one memory instruction after each of its first MFMAs
            constexpr int nm = nr + nw + nl;
            static_assert(nm <= 16, "one memory instruction per MFMA at most");
            if constexpr (nm == 0) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 16, 0);
            } else {
                static_for<0, 16>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    if constexpr (i < nr)
                        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
                    else if constexpr (i < nr + nw)
                        __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
                    else if constexpr (i < nm)
                        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
                });
            }
            if constexpr (NEXT && (t == 1 || t == 7)) lds_barrier();
        });
    };

    const int np = (ke - kb + BK - 1) / BK;
    for (int pnl = 0; pnl + 2 < np; ++pnl) panel(std::true_type{}, std::false_type{});
    if (np >= 2) panel(std::true_type{}, std::true_type{});
    panel(std::false_type{}, std::false_type{});

    // ---- epilogue: lane (lo, h) holds rows 8 (v / 4) + v % 4 + 4 h of row block r and
    // columns 4 lo .. 4 lo + 3 of the wave tile (element c from column block c). A partial
    // stream-K tile goes to its workspace slot as all BM x BN sums, packed rows of BN
    // floats (the wave's 128 x 128 quarter of it). One store sequence serves both
    // destinations (a second copy of it costs the stream-K form its registers), so partial
    // tiles carry the same non-temporal hint as C.
    const int col = 4 * lo;
    __amdgpu_buffer_rsrc_t rc;
    uint32_t ldc4;
    int rows_left, cols_left;
    if (!to_workspace) {
        const int row0 = m0 + wm * WT, col0 = n0 + wn * WT;
        const int64_t ec = c_off + int64_t(row0) * p.ldc + col0;
        rc = make_rsrc(p.C + ec, p.c_bytes - ec * 4);
        ldc4 = uint32_t(p.ldc) * 4u;
        rows_left = M - row0;
        cols_left = N - col0;
    } else {
        const int64_t ew = int64_t(slot) * BM * BN + int64_t(wm * WT) * BN + wn * WT;
        rc = make_rsrc(p.W + ew, (int64_t(BM) * BN - (int64_t(wm * WT) * BN + wn * WT)) * 4);
        ldc4 = uint32_t(BN) * 4u;
        rows_left = WT;
        cols_left = WT;
    }
    // The chunk that crosses N is stored element by element. The stream-K form stores it
    // right after each vector store, from the same registers: a second pass over the
    // accumulators (the plain form's, kept as its timings were taken) makes it spill.
    const bool crosses = col < cols_left && col + 4 > cols_left;
    auto store_partial = [&](int lr, int c, float x) {
        const bool keep = crosses && col + c < cols_left && lr < rows_left;
        store_vec<1, kStoreNonTemporal>(rc, keep ? uint32_t(lr) * ldc4 + 4u * (col + c) : kOob,
                                        0u, x);
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int lr = r * 32 + 8 * (v >> 2) + (v & 3) + 4 * h;
            const f32x4 out = {acc[r][0][v], acc[r][1][v], acc[r][2][v], acc[r][3][v]};
            const bool ok = lr < rows_left && col + 4 <= cols_left;
            store_vec<4, kStoreNonTemporal>(rc, ok ? uint32_t(lr) * ldc4 + 16u * lo : kOob, 0u,
                                            out);
            store_data_guard<SK>();
            if constexpr (SK) {
                if (cols_left < WT) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        store_partial(lr, c, out[c]);
                        store_data_guard<true>();
                    }
                }
            }
        }
    }
    if (!SK && cols_left < WT) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int lr = r * 32 + 8 * (v >> 2) + (v & 3) + 4 * h;
                const bool partial = lr < rows_left && col < cols_left && col + 4 > cols_left;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    store_vec<1, kStoreNonTemporal>(
                        rc, partial && col + c < cols_left ? uint32_t(lr) * ldc4 + 4u * (col + c)
                                                           : kOob,
                        0u, acc[r][c][v]);
            }
    }
}

template <bool SK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_sgemm_regpanel(GemmArgs p)
{
    using namespace regpanel;
    __shared__ __attribute__((aligned(16))) float lds[LDS_FLOATS];
    if constexpr (!SK) {
        // one item per workgroup: tile item % tiles over split item / tiles
        const int ntiles = p.tiles_m * p.tiles_n;
        const int item = blockIdx.x;
        const int ls = item / ntiles;
        int tm, tn;
        tile_coords(item - ls * ntiles, p.tiles_m, p.tiles_n, tm, tn);
        const int m0 = __builtin_amdgcn_readfirstlane(tm * BM);
        const int n0 = __builtin_amdgcn_readfirstlane(tn * BN);
        const int kb = __builtin_amdgcn_readfirstlane(ls * p.k_chunk);
        const int ke = __builtin_amdgcn_readfirstlane(min(p.K, kb + p.k_chunk));
        regpanel_item<false>(p, lds, m0, n0, kb, ke, ls * p.c_split_stride, false, 0);
    } else {
        // workgroups below tiles_dp own one whole tile; the others walk a stream-K range,
        // laid out contiguously per XCD so neighbouring segments share its L2. One call
        // site for both (one inlined copy of the item).
        const int bid = blockIdx.x;
        const bool dp = bid < p.sk.tiles_dp;
        const int g = dp ? 0
                         : __builtin_amdgcn_readfirstlane(
                               xcd_contiguous(bid - p.sk.tiles_dp, p.sk.G));
        const int first = dp ? 0 : sk_start(p.sk, g);
        const int end = dp ? 1 : sk_start(p.sk, g + 1);
        const int P = p.sk.panels;
        for (int i = first; i < end;) {
            int t, kbp, kep;
            if (dp) {
                t = xcd_contiguous(bid, p.sk.tiles_dp);
                kbp = 0;
                kep = P;
            } else {
                const int u = i / P;
                t = p.sk.tiles_dp + u;
                kbp = i - u * P;
                kep = min(P, kbp + (end - i));
            }
            int tm, tn;
            grouped_tile(t, p.tiles_m, p.tiles_n, tm, tn);
            // every wave is done with the previous segment's LDS before this one's prologue
            // overwrites it
            if (i != first) lds_barrier();
            regpanel_item<true>(p, lds, __builtin_amdgcn_readfirstlane(tm * BM),
                                __builtin_amdgcn_readfirstlane(tn * BN),
                                __builtin_amdgcn_readfirstlane(kbp * BK),
                                __builtin_amdgcn_readfirstlane(min(p.K, kep * BK)), 0,
                                kbp != 0 || kep != P, 2 * g + (i == first ? 0 : 1));
            i = dp ? end : i + (kep - kbp);
        }
    }
}

}  // namespace sgemm
