// kernel_persist.hpp -- the FP32 GEMM kernel for shapes whose C is large next to their K:
// persistent workgroups that write each tile of C among the MFMAs of the next one.
//
// Same product and the same ladder of the pages as kernel_mfma.hpp ("Shared Memory
// Tiling", "The tiled kernel"; "SGEMM: 2D Register Tiling Visualizer", "Why 2D Register
// Tiling Dominates"), arranged for a short K. At 16384^2 x 64 a 128 x 256 tile's 128 KiB of C
// take about as long to leave the CU as its MFMAs take to run. Stored at the end of each
// tile, with two workgroups per CU, they go out as one burst ahead of the other workgroup's
// loads in the CU's memory pipeline, and its MFMAs wait (measured on gfx950: the same
// kernel with its stores dropped by the hardware runs 15 % faster, without them 20 %).
//
//  * One workgroup per CU walks tiles pos, pos + G, ... (G workgroups, pos its place in an
//    order that keeps each XCD's workgroups contiguous, so the tiles in flight on one XCD are
//    neighbours in the grouped tile order and share A rows and B columns in its L2). WAVES
//    waves: eight (2 x 4, two per SIMD, 64 x 64 each: the planned form) or four (2 x 2,
//    one per SIMD, 64 x 128 each); a wave's part is 32 x 32 blocks accumulated by
//    v_mfma_f32_32x32x2_f32. The eight-wave form is the faster (16384^2 x 64: 291 against
//    323 us): with one wave per SIMD and 8 MFMAs per k-step the load and barrier latencies
//    show; a second wave per SIMD hides them.
//  * Two accumulator sets per lane (64 registers each with eight waves, in 238 registers
//    in all; 128 each in the 256 AGPRs with four): tile i accumulates in set i % 2 while
//    the previous tile's set is written, one 4-byte buffer store at a time between the
//    MFMAs, spread over the tile's first two K-panels. Measured in a one-wave-per-SIMD MFMA
//    stream writing 1 GiB, stores placed so cost the matrix pipe nothing, while assembling
//    16-byte chunks of a row first (register moves among the MFMAs) cost a fifth of its
//    time.
//  * Why 4-byte stores: in the 32 x 32 MFMA's result a lane holds 16 rows of one column, so
//    one register over the wave is 2 rows of 32 consecutive columns, two whole 128-byte
//    lines. That needs plain 32-column blocks (no column interleave), so each B operand read
//    must give a lane four consecutive k of ONE column: B is kept transposed in LDS, one row
//    of BK floats per column of the tile in A's layout and chunk swizzle. It is loaded with
//    4-byte loads along its rows (a half-wave reads 32 consecutive columns of a row) and
//    written as 16-byte chunks of four k. The A and B^T reads and writes are conflict-free.
//  * Each tile's first k-step takes a zero accumulator operand: no register clears.
//  * The panel pipeline is kernel_regpanel.hpp's: one LDS stage (48 KiB), the panel after
//    next staged in registers (with eight waves 2 A chunks and 16 B values per thread), a
//    whole panel's operands read ahead, two barriers per panel, every memory instruction
//    between MFMAs (pinned by scheduling barriers). The stream of panels runs on across tiles: a tile's
//    last panels load the next tile's first ones.
//  * Whole tiles only: M and N are multiples of 128 and 256 (the host computes any
//    remaining strip of C with the other kernels), so no store needs a per-lane condition.
//    A sequence that checked rows and columns per lane at a tile boundary, where the whole
//    pipeline's registers are live, ran the kernel out of registers.
//  * No vector-ALU work among the MFMAs: B rows past K read zeros through the B resource's
//    end. Only a K that is not a multiple of BK needs selects, clearing A values past K
//    (NaN row padding must not reach C): that is a kernel of its own (KT).
#pragma once

#include "kernel_regpanel.hpp"

namespace sgemm {

namespace persist {
constexpr int BM = 128, BN = 256, BK = 32;
constexpr int A_TILE = BM * BK;                 // A: BM rows of BK floats
constexpr int LDS_FLOATS = A_TILE + BN * BK;    // + B^T: BN rows of BK floats (48 KiB)
constexpr int STEPS = 16;                       // k-steps of 2 per panel
constexpr int kSchedVmemWrite = 0x040;
static_assert(LDS_FLOATS * 4 <= 64 * 1024, "LDS");

// The tile's split over WAVES waves (4: one per SIMD, 2 x 2 of 64 x 128; 8: two per SIMD,
// 2 x 4 of 64 x 64) and what each thread stages of a panel.
template <int WAVES>
struct Shape {
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WGN = WAVES / 2;               // waves along N (2 along M)
    static constexpr int WM = BM / 2, WN = BN / WGN;
    static constexpr int RB = WM / 32, CB = WN / 32;    // 32 x 32 blocks per wave
    static constexpr int ACH = BM * BK / 4 / THREADS;   // A chunks per thread
    static constexpr int ASTEP = THREADS / 8;           // rows between a thread's A chunks
    static constexpr int BCH = BN * BK / 4 / THREADS;   // B^T chunks per thread
    static constexpr int NL = ACH + 4 * BCH;            // a panel's loads per thread
    static constexpr int NW = ACH + BCH;                // its LDS writes
    static constexpr int NRG = RB + CB;                 // operand reads per group of 8 k
    static constexpr int NS = RB * CB * 16;             // C values per lane per tile
    static_assert(ASTEP % 16 == 0 && NW % 2 == 0, "staging layout");
};

// Panel schedule, per k-step t:
//   t 0        read group 3 of this panel
//   after t 1  barrier: every wave has read this panel
//   t 2, 3     write the staged next panel into LDS
//   t 4 .. 11  load the panel after next
//   after t 7  barrier: the next panel is in LDS
//   t 8 .. 15  read groups 0, 1, 2 of the next panel (a group's registers are free once its
//              four k-steps are done: groups 0 and 1 from t 8, group 2 from t 12)
//   any t      stores of the previous tile, weighted by kStoreW
constexpr int kStoreW[16] = {2, 6, 2, 2, 4, 4, 4, 4, 2, 2, 2, 2, 7, 7, 7, 7};

constexpr int prefix(const int *a, int n)
{
    int s = 0;
    for (int i = 0; i < n; ++i) s += a[i];
    return s;
}
// n items over `slots` steps, evenly: the first index of step t
constexpr int spread(int n, int slots, int t) { return t * n / slots; }

// Stores of the previous tile at step t of a panel that carries part PART of its ns stores
// (0: none, 1: the first half, 2: the second half, 3: all): first index and count.
constexpr int store_first(int part, int ns, int t)
{
    const int h = part == 3 ? ns : ns / 2;
    return (part == 2 ? ns / 2 : 0) + prefix(kStoreW, t) * h / 64;
}
constexpr int store_n(int part, int ns, int t)
{
    return part == 0 ? 0 : store_first(part, ns, t + 1) - store_first(part, ns, t);
}

// Of n operations spread over a step's m MFMAs (slot i holds [i n / m, (i + 1) n / m)), how
// many of those with index in [lo, hi) fall in slot i.
constexpr int slot_count(int i, int m, int lo, int hi, int n)
{
    const int a = i * n / m, b = (i + 1) * n / m;
    const int x = a > lo ? a : lo, y = b < hi ? b : hi;
    return y > x ? y - x : 0;
}
}  // namespace persist

__device__ inline float load_b32(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

// Every helper of the kernel below is inlined before the compiler's scalar-replacement
// pass: left to its late inlining, the lambdas' by-reference state stays in private memory,
// whose loads count as per-lane values and turn buffer resources into vector values.
#define SGEMM_INLINE __attribute__((always_inline))

// A K-panel of a tile: the tile's origin, whether it exists (int, not bool: a bool carried
// through selects can become a per-lane mask) and the panel's first k.
struct PanelAt {
    int m0, n0, v, k0;
};

// The panel after next of panel j of tile t0 (np >= 2 panels per tile): a panel of t0 or
// of the next tile t1. Arithmetic, not selects: a select between values computed apart
// can become a branch, which splits a panel's schedule in two.
__device__ SGEMM_INLINE inline PanelAt panel_after_next(int j, int np, PanelAt t0, PanelAt t1)
{
    const int jj = j + 2;
    const int d = int(unsigned(np - 1 - jj) >> 31);   // jj >= np
    return PanelAt{t0.m0 + d * (t1.m0 - t0.m0), t0.n0 + d * (t1.n0 - t0.n0),
                   t0.v + d * (t1.v - t0.v), (jj - d * np) * persist::BK};
}

// static_for without recursion (a fold over the index sequence), always inlined.
template <int BEGIN, typename F, int... I>
__device__ SGEMM_INLINE inline void sfor_impl(F &f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, BEGIN + I>{}), ...);
}
template <int BEGIN, int END, typename F>
__device__ SGEMM_INLINE inline void sfor(F &&f)
{
    if constexpr (END > BEGIN) sfor_impl<BEGIN>(f, std::make_integer_sequence<int, END - BEGIN>{});
}

template <int WAVES, bool KT>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void k_sgemm_persist(GemmArgs p)
{
    using namespace persist;
    using Sh = Shape<WAVES>;
    constexpr int WM = Sh::WM, WN = Sh::WN, RB = Sh::RB, CB = Sh::CB, NL = Sh::NL, NW = Sh::NW;
    constexpr int ACH = Sh::ACH, BCH = Sh::BCH, NRG = Sh::NRG, NS = Sh::NS;
    using regpanel::lds_barrier;
    __shared__ __attribute__((aligned(16))) float lds[LDS_FLOATS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lo = lane & 31, h = lane >> 5;
    const int wm = wave / Sh::WGN, wn = wave % Sh::WGN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    const int T = p.tiles_m * p.tiles_n;
    const int G = gridDim.x;                    // at most T (host)
    const int pos = __builtin_amdgcn_readfirstlane(xcd_contiguous(blockIdx.x, G));
    const int ntl = (T - pos + G - 1) / G;      // this workgroup's tiles, at least one
    const int np = (K + BK - 1) / BK;           // panels per tile, at least one
    const uint32_t ldc4 = uint32_t(ldc) * 4u;

    // Panel 0 of tile i of this workgroup; past its last tile v = 0 (and the last tile's
    // origin). No branches: the index is clamped.
    auto origin = [&](int i) SGEMM_INLINE {
        const int v = int(unsigned(i - ntl) >> 31);   // i < ntl
        int tm, tn;
        grouped_tile(min(i, ntl - 1) * G + pos, p.tiles_m, p.tiles_n, tm, tn);
        return PanelAt{__builtin_amdgcn_readfirstlane(tm * BM),
                       __builtin_amdgcn_readfirstlane(tn * BN), __builtin_amdgcn_readfirstlane(v),
                       0};
    };

    // ---- staging: thread tid loads A rows a_r + ASTEP j (16-byte chunk a_q of the panel's
    // 32 columns, j < ACH) and B values at rows 4 b_k + e (e < 4) of columns b_n + 32 j
    // (j < BCH); the four values of one column form the 16-byte chunk b_k of its B^T row.
    const int a_r = tid >> 3, a_q = tid & 7;
    const int b_c = tid & 31, b_k = (tid >> 5) & 7, b_n = b_c + 32 * BCH * (tid >> 8);
    uint32_t a_v[ACH], b_v[4];
#pragma unroll
    for (int j = 0; j < ACH; ++j)
        a_v[j] = uint32_t(a_r + Sh::ASTEP * j) * uint32_t(lda) * 4u + 16u * a_q;
#pragma unroll
    for (int e = 0; e < 4; ++e) b_v[e] = uint32_t(4 * b_k + e) * uint32_t(ldb) * 4u + 4u * b_n;
    static_assert(32 % a_swizzle_period<8>() == 0, "a thread's rows share one swizzle");
    const int a_lds = a_r * BK + 4 * (a_q ^ a_swizzle<8>(a_r));
    const int b_lds = A_TILE + b_n * BK + 4 * (b_k ^ a_swizzle<8>(b_c));
    f32x4 pa[ACH], pb[BCH];
    int kp = 0;   // first k of the staged panel
    __amdgpu_buffer_rsrc_t ra, rb;
    // Resources of the panel at k0 of the tile at (m0, n0): A's ends at the end of row
    // min(M - 1, m0 + BM)'s K values (so the last row's reads past K stay inside A), B's at
    // the end of row min(K - 1, k0 + BK)'s tile columns (rows past K read zero); a missing
    // tile gets empty ones. Multiplications by the 0/1 flag, not selects (no branches).
    auto load_set = [&](PanelAt at) SGEMM_INLINE {
        const int m0 = at.m0, n0 = at.n0, k0 = at.k0;
        kp = k0;
        const uint32_t na = uint32_t(min(M - 1 - m0, BM) * lda + K - k0) * 4u;
        const uint32_t nb = uint32_t(min(K - 1 - k0, BK) * ldb + (N - n0)) * 4u;
        ra = make_rsrc32(p.A + (int64_t(m0) * lda + k0),
                         __builtin_amdgcn_readfirstlane(uint32_t(at.v) * na));
        rb = make_rsrc32(p.B + (int64_t(k0) * ldb + n0),
                         __builtin_amdgcn_readfirstlane(uint32_t(at.v) * nb));
    };
    auto load_one = [&](auto jc) SGEMM_INLINE {
        constexpr int j = decltype(jc)::value;
        if constexpr (j < ACH) {
            pa[j] = load_b128(ra, a_v[j]);
        } else {
            constexpr int c = (j - ACH) >> 2, e = (j - ACH) & 3;
            pb[c][e] = load_b32(rb, b_v[e] + 128u * c);
        }
    };
    // Staged chunk j to LDS (A chunks 0 .. ACH - 1, then B^T chunks); with KT the A values at
    // or past K are cleared.
    auto write_one = [&](auto jc) SGEMM_INLINE {
        constexpr int j = decltype(jc)::value;
        if constexpr (j < ACH) {
            f32x4 v = pa[j];
            if constexpr (KT) {
                const int kc = kp + 4 * a_q;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = kc + e < K ? v[e] : 0.0f;
            }
            *reinterpret_cast<f32x4 *>(lds + a_lds + Sh::ASTEP * j * BK) = v;
        } else {
            *reinterpret_cast<f32x4 *>(lds + b_lds + 32 * (j - ACH) * BK) = pb[j - ACH];
        }
    };

    // ---- operands: group g of 8 k-values; oa[g][r] = k 8 g + 4 h .. + 3 of A row 32 r + lo of
    // the wave, ob[g][c] = the same k of B column 32 c + lo of the wave
    const int a_row = (wm * WM + lo) * BK;
    const int b_row = A_TILE + (wn * WN + lo) * BK;
    const int sw = a_swizzle<8>(lo);
    f32x4 oa[4][RB], ob[4][CB];
    // q = NRG g + j: j < RB an A block, else B block j - RB
    auto read_one = [&](auto qc) SGEMM_INLINE {
        constexpr int g = decltype(qc)::value / NRG, j = decltype(qc)::value % NRG;
        const int chunk = 4 * ((2 * g + h) ^ sw);
        if constexpr (j < RB)
            oa[g][j] = *reinterpret_cast<const f32x4 *>(lds + a_row + 32 * j * BK + chunk);
        else
            ob[g][j - RB] =
                *reinterpret_cast<const f32x4 *>(lds + b_row + 32 * (j - RB) * BK + chunk);
    };

    f32x16 acc[2][RB][CB];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int c = 0; c < CB; ++c) acc[s][r][c] = f32x16{};

    // ---- C: lane (lo, h) holds, in register v of block (r, c), row 32 r + 8 (v / 4) + v % 4
    // + 4 h and column 32 c + lo of the wave's WM x WN. Store q of a tile is register
    // v = (q / CB) % 16 of block (q / (16 CB), q % CB): CB consecutive stores fill 2 rows of
    // the wave's columns. Rows 32 r + 8 (v / 4) go in the scalar offset (8 values), rows v % 4 + 4 h and
    // the column in one of 4 lane offsets, 128 c bytes in the instruction's offset.
    __amdgpu_buffer_rsrc_t rc = make_rsrc32(p.C, 0u);   // the previous tile (or none)
    uint32_t lane_c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        lane_c[e] = (uint32_t(4 * h + e) * uint32_t(ldc) + uint32_t(lo)) * 4u;
    auto store_one = [&](auto oc, auto qc) SGEMM_INLINE {
        constexpr int O = decltype(oc)::value, q = decltype(qc)::value;
        constexpr int r = q / (16 * CB), v = (q / CB) % 16, c = q % CB;
        const uint32_t so = uint32_t(32 * r + 8 * (v >> 2)) * ldc4;
        // the element goes through a float first: __builtin_bit_cast applied to a vector
        // element lvalue reads the vector's first element instead
        const float x = acc[O][r][c][v];
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), rc,
                                              lane_c[v & 3] + 128u * c, so, kStoreNonTemporal);
    };
    // The wave's part of the tile at (m0, n0) of C; an empty resource (every store dropped)
    // when there is no such tile. The size is explicitly uniform: a vector-computed one
    // would put every store in a loop over distinct resources.
    auto c_rsrc = [&](int m0, int n0, int on) SGEMM_INLINE {
        const int64_t e = int64_t(m0 + wm * WM) * ldc + n0 + wn * WN;
        return make_rsrc32(p.C + e, __builtin_amdgcn_readfirstlane(uint32_t(on) * kFullRange));
    };
    // ---- one panel of set S: FIRST starts the set from zero; PART selects the previous
    // tile's stores it carries; `next2` is the panel after next, loaded during this one.
    auto panel = [&](auto sc, auto first_tag, auto part_tag, PanelAt next2) SGEMM_INLINE {
        constexpr int S = decltype(sc)::value, O = 1 - S;
        constexpr bool FIRST = decltype(first_tag)::value;
        constexpr int PART = decltype(part_tag)::value;
        // The global base offsets are opaque to the compiler from here on: otherwise it
        // hoists every base + constant of the loads and stores out of the loop into
        // registers of their own (and spills them) instead of using the instructions'
        // immediate offsets.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            asm volatile("" : "+v"(b_v[e]));
            asm volatile("" : "+v"(lane_c[e]));
        }
        sfor<0, STEPS>([&](auto tc) SGEMM_INLINE {
            constexpr int t = decltype(tc)::value;
            constexpr int g = t >> 2, s = t & 3;
            constexpr int r0 = t >= 8 ? spread(3 * NRG, 8, t - 8) : 0;
            constexpr int nr = t == 0 ? NRG : t >= 8 ? spread(3 * NRG, 8, t - 7) - r0 : 0;
            constexpr int nw = t == 2 || t == 3 ? NW / 2 : 0;
            constexpr int l0 = t >= 4 && t < 12 ? spread(NL, 8, t - 4) : 0;
            constexpr int nl = t >= 4 && t < 12 ? spread(NL, 8, t - 3) - l0 : 0;
            constexpr int ns = store_n(PART, NS, t);
            static_assert(t >= 12 || r0 + nr <= 2 * NRG, "group 2 is still in use");
            if constexpr (t == 0) sfor<3 * NRG, 4 * NRG>(read_one);
            if constexpr (t >= 8) sfor<r0, r0 + nr>(read_one);
            if constexpr (nw > 0) sfor<(t - 2) * (NW / 2), (t - 1) * (NW / 2)>(write_one);
            if constexpr (t == 4) load_set(next2);
            if constexpr (nl > 0) sfor<l0, l0 + nl>(load_one);
            if constexpr (ns > 0) {
                constexpr int s0 = store_first(PART, NS, t);
                sfor<s0, s0 + ns>([&](auto qc) SGEMM_INLINE { store_one(std::integral_constant<int, O>{}, qc); });
            }
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int c = 0; c < CB; ++c) {
                    if constexpr (FIRST && t == 0)
                        acc[S][r][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            oa[g][r][s], ob[g][c][s], f32x16{}, 0, 0, 0);
                    else
                        acc[S][r][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            oa[g][r][s], ob[g][c][s], acc[S][r][c], 0, 0, 0);
                }
            // pin the step's order: its memory instructions spread over its MFMAs
            constexpr int n = nr + nw + nl + ns, m = RB * CB;
            sfor<0, m>([&](auto ic) SGEMM_INLINE {
                constexpr int i = decltype(ic)::value;
                constexpr int cr = slot_count(i, m, 0, nr, n);
                constexpr int cw = slot_count(i, m, nr, nr + nw, n);
                constexpr int cl = slot_count(i, m, nr + nw, nr + nw + nl, n);
                constexpr int cs = slot_count(i, m, nr + nw + nl, n, n);
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                if constexpr (cr > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, cr, 0);
                if constexpr (cw > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, cw, 0);
                if constexpr (cl > 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, cl, 0);
                if constexpr (cs > 0)
                    __builtin_amdgcn_sched_group_barrier(kSchedVmemWrite, cs, 0);
            });
            if constexpr (t == 1 || t == 7) lds_barrier();
        });
    };

    // ---- prologue: the first panel into LDS, the stream's second panel staged, groups
    // 0 .. 2 of the first panel read (group 0 oldest, as the panels expect)
    {
        const PanelAt t0 = origin(0);
        load_set(t0);
        sfor<0, NL>(load_one);
        sfor<0, NW>(write_one);
        lds_barrier();
        sfor<0, NRG>(read_one);
        __builtin_amdgcn_sched_barrier(0);
        sfor<NRG, 2 * NRG>(read_one);
        __builtin_amdgcn_sched_barrier(0);
        sfor<2 * NRG, 3 * NRG>(read_one);
        __builtin_amdgcn_sched_barrier(0);
        PanelAt t1 = t0;
        t1.k0 = BK;
        load_set(t1);
        sfor<0, NL>(load_one);
        __builtin_amdgcn_sched_barrier(0);
    }

    using F = std::true_type;
    using NF = std::false_type;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    // Tile i into set S; the previous tile `prev` (set 1 - S, none when prev.v is 0) is
    // stored during its first panels. Returns tile i.
    auto tile = [&](auto sc, int i, PanelAt prev) SGEMM_INLINE {
        const PanelAt t0 = origin(i), t1 = origin(i + 1);
        rc = c_rsrc(prev.m0, prev.n0, prev.v);
        panel(sc, F{}, P1{}, panel_after_next(0, np, t0, t1));
        panel(sc, NF{}, P2{}, panel_after_next(1, np, t0, t1));
        for (int j = 2; j < np; ++j) panel(sc, NF{}, P0{}, panel_after_next(j, np, t0, t1));
        return t0;
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // Tiles in pairs, set 0 then set 1, in one straight loop body. With an odd count the last
    // pair's second tile is a dummy (v = 0: its loads read zeros, its own stores are
    // dropped) that still carries the stores of the real last tile. A peeled odd tile, or a
    // loop exit after either set, lets the compiler merge the two tile bodies into one and
    // swap the sets by copying 128 registers per tile.
    PanelAt prev{0, 0, 0, 0};
    for (int i = 0; i < ntl; i += 2) {
        prev = tile(S0{}, i, prev);
        prev = tile(S1{}, i + 1, prev);
    }
    rc = c_rsrc(prev.m0, prev.n0, prev.v);
    sfor<0, NS>([&](auto qc) SGEMM_INLINE { store_one(S1{}, qc); });
}

}  // namespace sgemm
