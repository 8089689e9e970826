// kernel_mfma.hpp -- the hot kernel: LDS-tiled, register-tiled FP32 GEMM on the gfx950
// matrix cores.
//
// What it computes is the row-by-column product of "Shared Memory Tiling", "The naive
// kernel". How it gets there follows the ladder of the pages, carried onto CDNA4:
//
//  * Block tiling ("SGEMM: Shared Memory Tiling Visualizer", code panel; "Shared Memory
//    Tiling", "The tiled kernel"): a workgroup owns a BM x BN tile of C and walks K in
//    panels of BK, staging a BM x BK panel of A and a BK x BN panel of B in LDS once and
//    reusing every staged element BN (resp. BM) times. Elements past M, N or K are
//    staged as zeros, so ragged shapes need no special cases in the inner loop.
//  * Register tiling ("SGEMM: 2D Register Tiling Visualizer", "Why 2D Register Tiling
//    Dominates"): each wavefront owns a WM x WN sub-tile and forms outer products of a
//    column of A-values and a row of B-values. On gfx950 the outer product is one
//    instruction: v_mfma_f32_32x32x2_f32 adds a 32 x 2 by 2 x 32 product into a 32 x 32
//    FP32 accumulator block spread over 16 registers per lane (v_mfma_f32_16x16x4_f32, a
//    16 x 4 by 4 x 16 product into 4 registers, for tiles of 16-row granularity; MB below
//    is the block size). A wave holds (WM/MB) x (WN/MB) such blocks; per k-step it reads
//    WM/MB A-values and WN/MB B-values from LDS and issues (WM/MB)(WN/MB) MFMAs, the
//    hardware form of the pages' (TM + TN) reads per TM * TN multiply-adds.
//  * Software pipelining ("Shared Memory Tiling", "What tiling does not fix"): two LDS
//    stages; the global loads of panel p+1 are in flight while the MFMAs consume panel
//    p, so each panel costs one barrier instead of two. NSTG = 3 makes a ring of three
//    stages, with the loads of panel p+2 in flight during panel p.
//
// gfx950 specifics:
//  * Loads use buffer resources. A lane whose element lies outside the matrix gets the
//    voffset kOob, past the resource's size, and the hardware returns zero without
//    touching memory: that is the zero-fill of the pages' masked loads, and it also
//    keeps the last rows of B from reading past the end of the allocation. Resources
//    are rebased per workgroup (A) and per panel (B), keeping offsets in 31 bits.
//  * Every lane loads 16 bytes (four consecutive floats of a row) per buffer load. gfx950
//    serves 16-byte buffer loads and stores at any 4-byte aligned address, so odd leading
//    dimensions need no narrower path. When K % 4 != 0 the last chunk of an A row is only
//    partly inside the matrix; its elements past K are replaced by zero (in registers on
//    the way to LDS, or in LDS after a direct load has landed).
//  * C is written through a buffer resource too: rows past M get the voffset kOob and the
//    hardware drops the store; a chunk of columns that crosses N is stored element by
//    element.
//  * MFMA operand layout (32x32x2): lane l supplies A[l % 32][l / 32] and
//    B[l / 32][l % 32]; accumulator register v of lane l holds
//    D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32]. For 16x16x4 see MfmaShape<16>.
//  * K permutation: lanes 0-31 read 4 consecutive k of a row of A with one ds_read_b128
//    and lanes 32-63 the next 4, so four MFMAs consume 8 k values; the B operand of step
//    s is read from LDS row 8 kb + s + 4 (l / 32), which pairs the same k on both sides
//    (four lane groups and 16 k values per four steps for 16x16x4).
//  * Column interleave: a lane reads CI consecutive columns of a B row with one LDS load
//    and feeds them to CI different MFMA blocks, so MFMA column c of block j is column
//    CI c + j of the wave tile. In the epilogue each lane then owns CI consecutive
//    columns of a row and writes them with one vector store.
//  * LDS layout: B rows are stored as they are (each read is a contiguous row segment,
//    conflict-free). A rows are BK words; a 16-byte chunk q of row r is stored at chunk
//    position q ^ swz(r), which spreads the 8 (or 16) rows read by one ds_read_b128
//    phase over distinct banks.
//  * Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2; the
//    tile order gives each XCD a contiguous range of tiles, walked in groups of
//    kGroupM tile rows, so concurrently running tiles share A and B panels in L2.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "streamk.hpp"

namespace sgemm {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int W> struct fvec;
template <> struct fvec<1> { typedef float type; };
template <> struct fvec<2> { typedef f32x2 type; };
template <> struct fvec<4> { typedef f32x4 type; };

// Word 3 of a raw buffer resource on the gfx9 family: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;
// A voffset beyond every resource size built below: loads from it return zero.
constexpr uint32_t kOob = 0x80000000u;
constexpr int kXcds = 8;
// Pipeline placement inside a panel (build-time tuning knobs): the next panel's global
// loads are spread over the first SGEMM_LOAD_STEPS k-steps and its LDS writes over the
// SGEMM_WRITE_STEPS steps before the last one.
#ifndef SGEMM_LOAD_STEPS
#define SGEMM_LOAD_STEPS 4
#endif
#ifndef SGEMM_WRITE_STEPS
#define SGEMM_WRITE_STEPS 3
#endif
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;
#ifndef SGEMM_GROUP_M
#define SGEMM_GROUP_M 8
#endif
constexpr int kGroupM = SGEMM_GROUP_M;

struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int64_t a_bytes;   // bytes from A to the end of its last row
    int64_t b_bytes;   // bytes from B to the end of its last row
    int M, N, K, lda, ldb, ldc;
    int tiles_m, tiles_n;
    // Split-K: item i of the tiles_m * tiles_n * splits work items is tile i % tiles over
    // k in [s * k_chunk, min(K, (s + 1) * k_chunk)) with s = i / tiles, written to
    // C + s * c_split_stride. splits = 1, k_chunk = K is the plain product.
    int splits, k_chunk;
    int64_t c_split_stride;
    int64_t c_bytes;   // bytes from C to the end of its last row
    // Stream-K (the SK kernels only): the partition of streamk.hpp and the workspace of
    // 2 * sk.G partial tiles of BM x BN floats.
    SkGeom sk;
    float *W;
    // Column strip (plain kernels only): when strip_cols > 0, the tiles cover columns
    // [0, strip_n0), and the strip_cols = N - strip_n0 (at most kStripCols) columns past
    // them are computed on the vector ALUs, by the tiles of each row: with strip_rows = r
    // > 0, tile column t computes rows [t r, (t + 1) r) of its tile row's strip; with 0,
    // the last tile column computes all of them.
    int strip_n0;
    int strip_cols;
    int strip_rows;
    // Row strip (plain kernels only; never with a column strip): when rstrip > 0, the tiles
    // cover rows [0, M - rstrip) (tiles_m whole tile rows), and the rstrip (at most
    // STRIP_COLS_MAX) rows past them are computed on the vector ALUs by the tiles of each
    // tile column: tile row t computes columns [t c, (t + 1) c) of its tile column's share
    // of them, c = strip_rows.
    int rstrip;
};

// Most columns a strip may hold: a remainder of N past the last whole tile column of up to
// four columns (a tile's own limit is MfmaTile::STRIP_COLS_MAX; past one column only the
// spread form computes it).
constexpr int kStripCols = 4;

// Strip columns (or rows) loaded per panel by the kernel's strip modes: 1 the last tile
// column's (one column); 2, 3 and 4 the spread column strip's one, two and four columns;
// 5, 6 and 7 the row strip's one, two and four rows; 0 none.
__host__ __device__ constexpr int strip_mode_cols(int smode)
{
    return smode == 3 || smode == 6 ? 2 : smode == 4 || smode == 7 ? 4 : smode >= 1 ? 1 : 0;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const float *base, int64_t bytes)
{
    int32_t n = 0;
    if (bytes > 0) n = bytes >= int64_t(kOob) ? int32_t(kOob - 64) : int32_t(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, n,
                                             kBufferWord3);
}

// Size of a buffer resource that reaches every offset a kernel's loads can use: the host
// keeps all of them below 2^31 - 64 (offsets_fit in plan.hpp).
constexpr uint32_t kFullRange = kOob - 64u;

// A buffer resource of `bytes` bytes from base, the size already clamped by the caller in
// 32-bit scalar arithmetic (no 64-bit compares on the vector ALU inside a panel loop).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc32(const float *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0,
                                             int32_t(bytes), kBufferWord3);
}

__device__ inline f32x4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// s_waitcnt vmcnt(N): all but the last N vector memory loads this wave issued have landed
// (the gfx9 family counts them done in issue order).
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait_vmcnt<N_FIRST> in the wave where `first` holds (wave-uniform), wait_vmcnt<N_OTHER> in
// the others
template <int N_FIRST, int N_OTHER>
__device__ inline void wait_vmcnt_split(bool first)
{
    if constexpr (N_FIRST == N_OTHER) {
        wait_vmcnt<N_OTHER>();
    } else {
        if (first) wait_vmcnt<N_FIRST>();
        else wait_vmcnt<N_OTHER>();
    }
}

// Calls f(std::integral_constant<int, I>) for I = BEGIN .. END-1, so I is a constant
// expression inside f (needed by the scheduling builtins).
template <int BEGIN, int END, typename F>
__device__ inline void static_for(F &&f)
{
    if constexpr (BEGIN < END) {
        f(std::integral_constant<int, BEGIN>{});
        static_for<BEGIN + 1, END>(f);
    }
}

// Buffer store of W consecutive floats at voff + soff (dropped by the hardware when voff is
// out of range; soff stays below 2^31, so kOob + soff cannot wrap into range). C is written
// once and not read again by the kernel, so the stores carry the non-temporal hint (cache
// policy bit 1 on gfx950), which measurably speeds up the store-heavy low-K shapes.
constexpr int kStoreNonTemporal = 2;
// Stream-K partial tiles are read back by the fixup kernel right after, so they are stored
// with the default policy.
#ifndef SGEMM_PARTIAL_STORE_POLICY
#define SGEMM_PARTIAL_STORE_POLICY 0
#endif
constexpr int kStorePartial = SGEMM_PARTIAL_STORE_POLICY;
template <int W, int POLICY = kStoreNonTemporal>
__device__ inline void store_vec(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                 typename fvec<W>::type v)
{
    if constexpr (W == 4) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff,
                                               POLICY);
    } else if constexpr (W == 2) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, soff,
                                              POLICY);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, voff, soff,
                                              POLICY);
    }
}

// A vector store wider than 64 bits reads its data registers after it issues; a VALU
// write to those registers right behind it corrupts lanes of the stored data on gfx950
// (measured: the last four lanes of each 16-lane quarter). The compiler's hazard model
// skips stores whose soffset is an SGPR, as every epilogue store here is, so every kernel
// whose epilogue stores 16 bytes at a time pins two wait states behind each such store
// (the register allocator reuses a store's data registers immediately in the stream-K
// forms, and in the plain forms of the 4-wide column-interleaved tiles).
template <bool GUARD>
__device__ inline void store_data_guard()
{
    if constexpr (GUARD) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 1");
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Physical 16-byte chunk slot of logical chunk q in A-tile row r (CPR chunks per row).
// The 4-chunk form (64-byte rows) was chosen by measurement on gfx950: of seven XOR
// swizzles, those whose low bit follows row bit 3 alone (((r >> 1) ^ (r >> 3)) & 3 and
// (r >> 1) & 3) cost 4 bank-conflict cycles per ds_read_b128 and r & 3 cost 12, while this
// one and three others cost none.
template <int CPR>
__host__ __device__ constexpr int a_swizzle(int r)
{
    static_assert(CPR == 16 || CPR == 8 || CPR == 4 || CPR == 2,
                  "A row must hold 2, 4, 8 or 16 chunks");
    return CPR == 16 ? (r & 15)
         : CPR == 8 ? ((r & 7) ^ ((r >> 3) & 1))
         : CPR == 4 ? (((r >> 1) ^ (r >> 2)) & 3)
                    : (((r >> 2) ^ (r >> 3)) & 1);
}

// Rows after which a_swizzle<CPR> repeats. The kernel relies on it twice: all A chunks one
// thread stages lie a multiple of it apart (one swizzle per thread), and the rows one lane
// reads lie 32 apart (so 32 must be a multiple of it).
template <int CPR>
__host__ __device__ constexpr int a_swizzle_period()
{
    return CPR == 4 ? 8 : 16;
}

// Physical 16-byte chunk slot of logical chunk q in B-tile row r. The 32-wide blocks read
// B rows whole and need none. With 16-wide blocks one read phase covers lane groups 0 and
// 1, which read rows r and r + 4 of the panel: BN-float rows put those 1 KiB (or 2 KiB)
// apart, on the same banks, so rows with bit 2 set are moved by half of a 64-bank line.
template <int MB>
__host__ __device__ constexpr int b_swizzle(int r)
{
    return MB == 16 ? ((r >> 2) & 1) << 3 : 0;
}

// Position in the tile order of workgroup bid out of `total`: workgroups are dispatched
// round-robin over the XCDs, so bid % kXcds is the XCD; each XCD gets a contiguous range.
__device__ inline int xcd_contiguous(int bid, int total)
{
    const int q = total / kXcds, r = total % kXcds;
    const int x = bid % kXcds, l = bid / kXcds;
    return x < r ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;
}

// Tile t of the tile order: groups of kGroupM tile rows, walked column by column, so
// tiles close in the order share A rows and B columns.
__device__ inline void grouped_tile(int t, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int per_group = kGroupM * tiles_n;
    const int g = t / per_group;
    const int first = g * kGroupM;
    const int rows = min(tiles_m - first, kGroupM);
    const int w = t - g * per_group;
    tm = first + w % rows;
    tn = w / rows;
}

// Tile coordinates of workgroup bid when every tile has its own workgroup.
__device__ inline void tile_coords(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    grouped_tile(xcd_contiguous(bid, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// The FP32 MFMA instruction a wave tile is built from: an MB x MB block of C gains an
// MB x KSTEP by KSTEP x MB outer product per instruction; both shapes have the same
// throughput (4096 FLOP in 16 passes, 2048 in 8). Lane l supplies A[l % MB][l / MB] and
// B[l / MB][l % MB]; accumulator register v of lane l holds column l % MB and row
//  * 32 x 32 x 2 (16 registers): 8 (v / 4) + v % 4 + 4 (l / 32);
//  * 16 x 16 x 4 (4 registers):  v + 4 (l / 16).
// H = 64 / MB lane groups each read 4 consecutive k of an A row with one ds_read_b128, so a
// k-group of 4 H values of k feeds 4 MFMA steps (step s uses element s of every group).
template <int MB> struct MfmaShape;
template <> struct MfmaShape<32> {
    static constexpr int H = 2, KSTEP = 2, ACC = 16;
    typedef f32x16 acc_t;
    __device__ static acc_t mfma(float a, float b, const acc_t &c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    // row of accumulator register v inside the block, for lane group 0
    static constexpr int row(int v) { return 8 * (v >> 2) + (v & 3); }
};
template <> struct MfmaShape<16> {
    static constexpr int H = 4, KSTEP = 4, ACC = 4;
    typedef f32x4 acc_t;
    __device__ static acc_t mfma(float a, float b, const acc_t &c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static constexpr int row(int v) { return v; }
};

template <int BM, int BN, int BK, int WGM, int WGN, int KACC = 1, int KG = 1, int MB = 32,
          int NSTG = 2>
struct MfmaTile {
    static constexpr int kGroupThreads = 64 * WGM * WGN;   // one K-group of waves
    static constexpr int kThreads = kGroupThreads * KG;
    static constexpr int WM = BM / WGM;          // wave tile rows
    static constexpr int WN = BN / WGN;          // wave tile columns
    static constexpr int RB = WM / MB;           // MB-row MFMA blocks per wave
    static constexpr int CI = WN >= 4 * MB ? 4 : WN / MB;   // column interleave
    static constexpr int CG = WN / (MB * CI);    // interleaved column groups
    static constexpr int NACC = RB * CI * CG;    // MB x MB accumulator blocks per wave
    static constexpr int ACC = MfmaShape<MB>::ACC;   // registers per accumulator block
    static constexpr int CPR = BK / 4;           // 16-byte chunks per A-tile row
    static constexpr int A_CH = BM * BK / 4 / kGroupThreads;  // A chunks per thread per panel
    static constexpr int B_CH = BK * BN / 4 / kGroupThreads;  // B chunks per thread per panel
    static constexpr int A_TILE = BM * BK;       // floats per A stage
    static constexpr int B_TILE = BK * BN;       // floats per B stage
    static constexpr int STAGE = A_TILE + B_TILE;
    // The tile's stores are shared by the K-groups: store unit (r, g, q), the quad q of
    // accumulator registers (4 rows) of row block r and column group g (CI blocks side by
    // side), belongs to K-group u KG / UNITS for unit index u = (r CG + g) ACC/4 + q. After
    // the last panel each group writes its partial sums of the other groups' units to LDS
    // (one f32x4 per block, quad and lane, in a slot per writing group), reusing the stages'
    // memory, and the owner of each unit adds them and its own in ascending group order.
    static constexpr int UNITS = RB * CG * (ACC / 4);
    static constexpr int RED = KG > 1 ? KG * kGroupThreads * NACC * ACC : 0;
    // Column strip (see the kernel): per stage, 64 floats of the strip's B column (one per
    // value of k of the panel), loaded with the panel; then a reduction area for the lanes'
    // partial sums: one row per K-group and MFMA lane group, STRIP_RS floats apart. The
    // row stride is 64 / H words past a multiple of 64, so the H lane groups of a wave,
    // which write the same rows' sums into H different rows, hit different banks.
    // A strip of sc columns holds sc such columns per stage and K-group, and the spread
    // form's reduction area one float per thread, K-group and column.
    static constexpr int STRIP_STAGE = 64;
    static constexpr int STRIP_RS = (BM + 63) / 64 * 64 + 64 / MfmaShape<MB>::H;
    static constexpr int strip_red_for(int sc)
    {
        return KG * MfmaShape<MB>::H * STRIP_RS > KG * kGroupThreads * sc
                   ? KG * MfmaShape<MB>::H * STRIP_RS
                   : KG * kGroupThreads * sc;
    }
    static constexpr int strip_floats_for(int sc)
    {
        return NSTG * KG * STRIP_STAGE * sc + strip_red_for(sc);
    }
    // NSTG LDS stages per K-group
    static constexpr int STAGES = NSTG * KG * STAGE;
    static constexpr int BASE_FLOATS = STAGES > RED ? STAGES : RED;
    static constexpr int lds_floats_for(int sc)
    {
        return STAGES + strip_floats_for(sc) > BASE_FLOATS ? STAGES + strip_floats_for(sc)
                                                           : BASE_FLOATS;
    }
    // workgroups per CU that the LDS allows
    static constexpr int lds_occupancy(int floats) { return 160 * 1024 / (floats * 4); }
    static constexpr bool STRIP_OK = BM <= kGroupThreads * KG && BK <= 64 && RED <= STAGES &&
                                     (STAGES + strip_floats_for(1)) * 4 <= 160 * 1024;
    // The widest strip the tile takes: four columns, or two, where the room for them in LDS
    // leaves as many workgroups per CU as one column does; else one.
    static constexpr bool strip_fits(int sc)
    {
        return (STAGES + strip_floats_for(sc)) * 4 <= 160 * 1024 &&
               lds_occupancy(lds_floats_for(sc)) == lds_occupancy(lds_floats_for(1));
    }
    static constexpr int STRIP_COLS_MAX = !STRIP_OK ? 0 : strip_fits(4) ? 4 : strip_fits(2) ? 2 : 1;
    static constexpr int STRIP_RED = strip_red_for(STRIP_COLS_MAX > 0 ? STRIP_COLS_MAX : 1);
    static constexpr int STRIP_FLOATS = strip_floats_for(STRIP_COLS_MAX > 0 ? STRIP_COLS_MAX : 1);
    static constexpr int LDS_FLOATS =
        STRIP_OK && STAGES + STRIP_FLOATS > BASE_FLOATS ? STAGES + STRIP_FLOATS : BASE_FLOATS;
    static constexpr int LDS_BYTES = LDS_FLOATS * 4;
    static_assert(WM % MB == 0 && WN % MB == 0, "wave tile is made of MB x MB blocks");
    static_assert(WN % (MB * CI) == 0, "column groups");
    static_assert(BK % (4 * MfmaShape<MB>::KSTEP) == 0, "panels hold whole k-groups");
    static_assert((BM * BK / 4) % kGroupThreads == 0 && (BK * BN / 4) % kGroupThreads == 0,
                  "panel chunks divide evenly over a K-group");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS holds 160 KiB per workgroup");
};

// KG > 1 splits K inside the workgroup: KG groups of WGM x WGN waves compute the same
// tile, group g taking K-panels g, g + KG, g + 2 KG, ..., each with its own LDS stages;
// at the end of a tile the groups pass their sums through LDS and each adds, in ascending
// group order (deterministic), and stores its share of the tile's store units
// (MfmaTile::UNITS). This puts KG waves on each SIMD for tiles too small to fill the GPU
// otherwise, and spreads the tile's final sums and stores over all of them.
//
// DL selects direct global -> LDS loads: each 16-byte buffer load writes its lane's chunk
// straight into LDS (lane l of a wave at the wave's base + 16 l), so the next panel needs
// no staging registers, no LDS write instructions and no wait in the middle of the panel;
// the wave waits for its loads once, just before the panel's barrier. A lane picks the
// global chunk that belongs at its LDS slot, which keeps the A swizzle. Out-of-range
// lanes write zeros, as register loads return them. An A chunk that crosses K cannot be
// cleaned on its way into LDS, so in the panel that holds the end of the K range each lane
// zeroes the elements past K of its own chunks once they have landed, before the barrier.
//
// Without SK one workgroup computes one item (a tile, or a tile's K range under split-K)
// and the grid has one workgroup per item. With SK the grid is sk.tiles_dp workgroups of
// one tile each followed by sk.G stream-K workgroups, each walking the segments of its
// range of K-panel units (streamk.hpp): whole tiles go to C, partial ones to its two
// workspace slots. FORM (a strip mode of strip_mode_cols) selects the strip the kernel
// computes: each strip form is a kernel of its own, so that no form's registers or code
// weigh on the others (the plain tiles' kernel, FORM 0, holds none).
template <int BM, int BN, int BK, int WGM, int WGN, int KACC, int KG, bool DL, bool SK = false,
          int MB = 32, int NSTG = 2, int FORM = 0>
__global__ __launch_bounds__(64 * WGM * WGN * KG) void k_sgemm_mfma(GemmArgs p)
{
    static_assert(NSTG == 2 || (NSTG == 3 && DL), "two LDS stages, or three with direct loads");
    using T = MfmaTile<BM, BN, BK, WGM, WGN, KACC, KG, MB, NSTG>;
    static_assert(FORM == 0 || (!SK && DL && T::STRIP_OK &&
                                strip_mode_cols(FORM) <= T::STRIP_COLS_MAX),
                  "a strip form the tile can hold");
    using S = MfmaShape<MB>;
    typedef typename S::acc_t acc_t;
    constexpr int NT = T::kGroupThreads, WM = T::WM, WN = T::WN, RB = T::RB, CI = T::CI,
                  CG = T::CG, CPR = T::CPR, A_CH = T::A_CH, B_CH = T::B_CH;
    typedef typename fvec<CI>::type bvec;

    __shared__ __attribute__((aligned(16))) float lds_all[T::LDS_FLOATS];

    // K-group of this wave: uniform across the wave (NT is a multiple of 64), which the
    // compiler must be told, or every buffer load's resource looks divergent
    const int kg = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(int(threadIdx.x) / NT);
    const int tid = threadIdx.x % NT;         // thread index inside the K-group
    const int lane = tid & 63;
    const int lo = lane % MB, hi = lane / MB;   // operand row / column, lane group
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    // this group's stages: stage s at smem + s * KG * STAGE
    float *const smem = lds_all + kg * T::STAGE;
    constexpr int SSTRIDE = KG * T::STAGE;
    float *const red = lds_all;   // K-group sums, written once every stage is read

    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int ntiles = p.tiles_m * p.tiles_n;

    // ---- per-thread load assignment ----
    // Thread tid stages A chunks c = tid + i*NT, i.e. rows a_r0 + i*A_RSTEP at the fixed
    // k-columns 4*a_q .. +3, and B chunks at panel rows b_k0 + i*B_KSTEP, fixed columns
    // b_c0 .. +3. Because A_RSTEP is a multiple of the swizzle's period, every A chunk of a
    // thread has the same swizzle, so all offsets are one base plus a compile-time stride.
    constexpr int A_RSTEP = NT / CPR;
    constexpr int B_KSTEP = NT / (BN / 4);
    static_assert(NT % CPR == 0 && A_RSTEP % a_swizzle_period<CPR>() == 0 &&
                      NT % (BN / 4) == 0,
                  "chunk assignment strides");
    static_assert(MB % a_swizzle_period<CPR>() == 0, "a lane's A rows share one swizzle");
    // A register-staged lane loads logical chunk tid % CPR of its row and stores it at the
    // swizzled slot; a direct-loading lane owns LDS slot tid % CPR and loads the logical
    // chunk that belongs there.
    const int a_r0 = tid / CPR;
    const int a_q = DL ? (tid % CPR) ^ a_swizzle<CPR>(a_r0) : tid % CPR;
    const uint32_t a_off0 = uint32_t(a_r0) * uint32_t(lda) * 4u + uint32_t(a_q) * 16u;
    const uint32_t a_stride = uint32_t(A_RSTEP) * uint32_t(lda) * 4u;
    const int a_lds0 = a_r0 * BK + 4 * (a_q ^ a_swizzle<CPR>(a_r0));
    // B: a register-staged lane loads logical chunk tid % (BN/4) of its row and stores it at
    // the swizzled slot; a direct-loading lane owns slot tid % (BN/4) and loads the logical
    // chunk that belongs there (the swizzle is one per thread: its rows lie B_KSTEP apart)
    const int b_k0 = tid / (BN / 4);
    const int b_q = DL ? (tid % (BN / 4)) ^ b_swizzle<MB>(b_k0) : tid % (BN / 4);
    const int b_c0 = 4 * b_q;
    static_assert(MB == 32 || (B_KSTEP % 8 == 0 && BN / 4 >= 16),
                  "a thread's B rows share one swizzle, which stays inside the row");
    const uint32_t b_off0 = uint32_t(b_k0) * uint32_t(ldb) * 4u + uint32_t(b_c0) * 4u;
    const uint32_t b_stride = uint32_t(B_KSTEP) * uint32_t(ldb) * 4u;
    const int b_lds0 = b_k0 * BN + (MB == 32 ? b_c0 : 4 * (b_q ^ b_swizzle<MB>(b_k0)));

    // This workgroup's item: split ls of tile item % tiles, i.e. tile origin (lm0, ln0) and
    // K range [lkb, lkb + lK). All wave-uniform: keep them (and the loops they bound) on
    // the scalar unit. Stream-K workgroups set them per segment (below).
    int lm0 = 0, ln0 = 0, lkb = 0, lK = 0, ls = 0;
    // stream-K: this workgroup's index g, its next unit and the end of its range
    int sk_g = 0, sk_i = 0, sk_end = 0;
    bool sk_mode = false;
    if constexpr (!SK) {
        int tm, tn;
        const int item = blockIdx.x;
        ls = item / ntiles;
        tile_coords(item - ls * ntiles, p.tiles_m, p.tiles_n, tm, tn);
        lm0 = __builtin_amdgcn_readfirstlane(tm * BM);
        ln0 = __builtin_amdgcn_readfirstlane(tn * BN);
        lkb = __builtin_amdgcn_readfirstlane(ls * p.k_chunk);
        lK = __builtin_amdgcn_readfirstlane(min(K - lkb, p.k_chunk));
        ls = __builtin_amdgcn_readfirstlane(ls);
    } else {
        const int bid = blockIdx.x;
        if (bid < p.sk.tiles_dp) {
            int tm, tn;
            grouped_tile(xcd_contiguous(bid, p.sk.tiles_dp), p.tiles_m, p.tiles_n, tm, tn);
            lm0 = __builtin_amdgcn_readfirstlane(tm * BM);
            ln0 = __builtin_amdgcn_readfirstlane(tn * BN);
            lK = K;
        } else {
            // consecutive ranges on one XCD, so neighbouring segments share its L2
            sk_mode = true;
            sk_g = __builtin_amdgcn_readfirstlane(xcd_contiguous(bid - p.sk.tiles_dp, p.sk.G));
            sk_i = sk_start(p.sk, sk_g);
            sk_end = sk_start(p.sk, sk_g + 1);
        }
    }
    // ---- per-item load offsets and resource bounds (per segment under stream-K). The panel
    // loop then needs no vector-ALU work for its loads, which measurably costs matrix-pipe
    // time on gfx950:
    //  * a chunk whose row lies past M, or whose columns start past N, gets kOob here, once;
    //  * the K range needs no per-load test: a panel wholly past it gets empty resources,
    //    B rows past it lie past the end of the panel's B resource (sized to end at the
    //    item's last K row), and A values past it, which the loads do fetch (from the row's
    //    padding or the next split), are zeroed before use (write_slot, fix_k_tail);
    //  * resource sizes come from 32-bit scalar min/select chains (the host bounds every
    //    product below 2^31): A's only ends before the full range when the tile holds A's
    //    last row (a_end is all ones otherwise), B's when the item's last K row is in the
    //    panel (BK + 1 rows cover every offset of a panel otherwise).
    uint32_t a_voff[A_CH], b_voff[B_CH];
    uint32_t a_end = 0u;
    auto set_item = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int l = 0; l < A_CH; ++l)
            a_voff[l] = lm0 + a_r0 + l * A_RSTEP < M ? a_off0 + uint32_t(l) * a_stride : kOob;
        // columns past N inside a chunk only reach accumulators that are never stored
        const bool b_col_ok = ln0 + b_c0 < N;
#pragma unroll
        for (int i = 0; i < B_CH; ++i) b_voff[i] = b_col_ok ? b_off0 + uint32_t(i) * b_stride : kOob;
        a_end = M - lm0 <= BM ? uint32_t((M - 1 - lm0) * lda + (K - lkb)) * 4u : 0xffffffffu;
    };

    // ---- global -> register staging of one panel ----
    f32x4 ra[A_CH], rb[B_CH];
    __amdgpu_buffer_rsrc_t rsa, rsb;   // resources rebased at the panel being staged
    int k_load = 0;

    auto set_panel = [&](int k0) __attribute__((always_inline)) {
        k_load = k0;
        const int64_t ea = int64_t(lm0) * lda + lkb + k0, eb = int64_t(lkb + k0) * ldb + ln0;
        const int rows = lK - k0;
        const uint32_t na = min(a_end - 4u * uint32_t(k0), kFullRange);
        const uint32_t nb =
            min(uint32_t((min(rows, BK + 1) - 1) * ldb + (N - ln0)) * 4u, kFullRange);
        rsa = make_rsrc32(p.A + ea, rows > 0 ? na : 0u);
        rsb = make_rsrc32(p.B + eb, rows > 0 ? nb : 0u);
    };
    // staging slot l < A_CH is A chunk l, otherwise B chunk l - A_CH
    // (offsets are read through locals: a subscript of the offset arrays written straight
    // into the load, in the branch that a constant l rules out, makes the compiler drop the
    // kernel's host stub without a diagnostic; the build checks the library for undefined
    // symbols)
    auto load_slot = [&](int l) __attribute__((always_inline)) {
        if (l < A_CH) {
            const uint32_t off = a_voff[l];
            ra[l] = load_b128(rsa, off);
        } else {
            const int i = l - A_CH;
            const uint32_t off = b_voff[i];
            rb[i] = load_b128(rsb, off);
        }
    };
    auto write_slot = [&](float *As, int l) __attribute__((always_inline)) {
        if (l < A_CH) {
            // elements past the K range belong to the row padding, the next row or the next
            // split; zero them (a select, so a NaN there cannot leak). Done here, where the
            // data is needed anyway, so the select does not wait on the load early.
            const int kc = k_load + 4 * a_q;
            f32x4 v = ra[l];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = kc + e < lK ? v[e] : 0.0f;
            *reinterpret_cast<f32x4 *>(As + a_lds0 + l * A_RSTEP * BK) = v;
        } else
            *reinterpret_cast<f32x4 *>(As + T::A_TILE + b_lds0 + (l - A_CH) * B_KSTEP * BN) =
                rb[l - A_CH];
    };
    // direct load of staging slot l into stage As: A chunk tid + l * NT sits at byte
    // 16 (tid + l * NT) of the A tile, B chunk tid + i * NT at byte 16 (tid + i * NT) of the
    // B tile, so a wave's 64 chunks are contiguous and the wave passes its first chunk's
    // address (uniform) as the LDS base
    typedef __attribute__((address_space(3))) void *lds_ptr;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // after the direct loads of a panel have landed: zero the elements past the K range in
    // this lane's A chunks (their LDS slots are 16 (tid + l NT) bytes into the A tile). The
    // branch is uniform and taken only in the panel that holds the end of the range; a
    // panel wholly past it (with K-groups) read zeros already, through its empty resource.
    // Each chunk is read and written whole: neighbouring lanes' chunks are neighbouring 16
    // bytes, so the accesses are free of bank conflicts (element stores, 16 bytes apart
    // across the lanes, are not).
    auto fix_k_tail = [&](float *As) __attribute__((always_inline)) {
        if (k_load < lK && k_load + BK > lK) {
            const int kc = k_load + 4 * a_q;
            if (kc + 4 > lK) {
#pragma unroll
                for (int l = 0; l < A_CH; ++l) {
                    f32x4 *chunk = reinterpret_cast<f32x4 *>(As + (tid + l * NT) * 4);
                    f32x4 v = *chunk;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = kc + e < lK ? v[e] : 0.0f;
                    *chunk = v;
                }
            }
        }
    };
    auto load_direct = [&](float *As, int l) __attribute__((always_inline)) {
        if (l < A_CH) {
            const uint32_t off = a_voff[l];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsa, (lds_ptr)(As + (wave_u * 64 + l * NT) * 4), 16, off, 0, 0, 0);
        } else {
            const int i = l - A_CH;
            const uint32_t off = b_voff[i];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsb, (lds_ptr)(As + T::A_TILE + (wave_u * 64 + i * NT) * 4), 16, off, 0, 0, 0);
        }
    };

    // KACC accumulator sets take the k-steps in turn (KACC > 1 gives a wave with few MFMA
    // blocks independent accumulation chains); they are summed before the epilogue.
    acc_t acc[KACC][RB][CI * CG];
#pragma unroll
    for (int h = 0; h < KACC; ++h)
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CI * CG; ++j) acc[h][i][j] = acc_t{};

    // A-operand LDS rows of this lane: row wm*WM + rb*32 + lo, whose swizzle depends on
    // lo only (wm*WM + rb*32 is a multiple of 32).
    const int a_sw = a_swizzle<CPR>(lo);
    const int a_row0 = (wm * WM + lo) * BK;
    const int b_col0 = wn * WN + CI * lo;

    auto read_a = [&](const float *As, int kb, f32x4 (&a)[RB]) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
            a[r] = *reinterpret_cast<const f32x4 *>(As + a_row0 + r * MB * BK +
                                                    4 * ((S::H * kb + hi) ^ a_sw));
    };
    auto read_b = [&](const float *Bs, int t, bvec (&b)[CG]) {
        if constexpr (MB == 32) {
            const float *brow = Bs + (4 * S::H * (t >> 2) + (t & 3) + 4 * hi) * BN + b_col0;
#pragma unroll
            for (int g = 0; g < CG; ++g)
                b[g] = *reinterpret_cast<const bvec *>(brow + g * MB * CI);
        } else {
            // the row's bit 2 is bit 0 of the lane group, so the swizzle is per lane
            const float *brow = Bs + (4 * S::H * (t >> 2) + (t & 3) + 4 * hi) * BN;
            const int sw = b_swizzle<MB>(4 * hi);
#pragma unroll
            for (int g = 0; g < CG; ++g) {
                const int col = b_col0 + g * MB * CI;
                b[g] = *reinterpret_cast<const bvec *>(brow + 4 * ((col >> 2) ^ sw) + (col & 3));
            }
        }
    };

    // Operand registers: a[kb & 1] holds the A values of k-group kb, b[t & 1] the B values
    // of k-step t.
    f32x4 a[2][RB];
    bvec b[2][CG];

    // One panel of BK/2 MFMA k-steps from LDS stage `cur`. Everything else the panel does
    // is placed in the shadow of its MFMAs (each 32x32x2 MFMA holds the matrix pipe for
    // 64 cycles and the wave issues in order, so an instruction placed between two MFMAs
    // costs nothing):
    //   steps 0..LS-1       issue the global loads of the next panel (NEXT only)
    //   every step t        read the operands of step t+1 from LDS
    //   steps STEPS-1-WS..  write the staged next panel into the other stage (NEXT only)
    //   last step           barrier, then read step 0 of the next panel from the other
    //                       stage; the MFMAs of the last step need only registers, so
    //                       they cover the latency of those reads.
    // One barrier per panel is enough: the other stage was last read before the previous
    // panel's barrier, and this panel's reads of `cur` all precede this barrier. With
    // direct loads there are no LDS write steps; the wave waits for its loads before the
    // barrier instead.
    constexpr int STEPS = BK / S::KSTEP;
    constexpr int NL = A_CH + B_CH;                     // staging slots per panel
    // PAIR unrolls the panel loop by two (constant LDS stages). It costs 30-80 registers; it
    // measured 1-4 % faster for direct-load tiles of BK >= 32 up to 128 x 128 with one or
    // two K-groups, and slower for the short-K 128 x 256 x 16 tile (whose epilogue
    // dominates), the 256 x 256 ones (which then spill) and four K-groups (few panels each).
    constexpr bool PAIR = DL && BK >= 32 && BM * BN <= 128 * 128 && KG <= 2;
    // the stage of the current panel is panel_parity % NSTG where the stage is not a constant
    int panel_parity = 0;
    constexpr int LS = SGEMM_LOAD_STEPS;
    constexpr int WS = SGEMM_WRITE_STEPS;
    constexpr int PER_LOAD = (NL + LS - 1) / LS;
    constexpr int PER_WRITE = (NL + WS - 1) / WS;
    static_assert(LS + WS < STEPS, "loads and LDS writes of a panel need separate steps");

    // ---- column strip: the tiles also compute the strip_cols (1 to STRIP_COLS_MAX)
    // columns of C past the last tile column, instead of a column of tiles that would hold
    // that many valid columns. The strip's B values of a panel (zeros past the K range and
    // past strip_cols) are loaded straight into LDS with the panel, column j of stage s of
    // group kg at strip_lds + ((s KG + kg) SCM + j) STRIP_STAGE, value k of the panel at
    // + k, by the group's first wave. Two forms:
    //  * spread (strip_rows > 0): each tile of a row computes strip_rows of the row's strip
    //    rows, from the A panel in LDS (below, set_spread_item), for one, two or four
    //    columns (three: four, the last one zero);
    //  * last column (strip_rows = 0, one column): the tiles of the last tile column compute
    //    all of them. The MFMA's A operands already hold, in each lane, four consecutive values of
    //    k of each of the lane's rows (k-group kb: 4 (H kb + hi) .. + 3); a lane multiplies
    //    them by the strip's four B values for those k (one 16-byte LDS read per k-group,
    //    the same address for all lanes of a lane group) into sacc, on the vector ALU
    //    between the MFMAs. Waves that differ only in wn hold the same rows, so only the
    //    wn = 0 waves' sums are used; after the last panel the lane groups and K-groups are
    //    added in a fixed order.
    // Vector and LDS work among the MFMAs costs the matrix pipe time on gfx950. The spread
    // form costs each tile two LDS reads and four FMAs per panel and wave, against four
    // reads and 4 RB FMAs per k-group in the last column, so the plan uses it wherever a
    // K-group's threads cover a tile's share of the rows and few rounds of tiles make
    // that cheaper than the last-column form (strip_form_rows).
    constexpr int SCM = T::STRIP_COLS_MAX > 0 ? T::STRIP_COLS_MAX : 1;   // columns per stage
    float *const strip_lds = lds_all + T::STAGES;
    float *const strip_red = strip_lds + NSTG * KG * SCM * T::STRIP_STAGE;
    __amdgpu_buffer_rsrc_t rss;
    uint32_t s_off = kOob;
    float sacc[RB];
    f32x4 sbv;   // the strip's B values of the current k-group
    auto set_strip_item = [&]() __attribute__((always_inline)) {
        s_off = lane < BK ? uint32_t(lane) * uint32_t(ldb) * 4u : kOob;
#pragma unroll
        for (int r = 0; r < RB; ++r) sacc[r] = 0.0f;
    };
    // the strip's B resource for the panel at k0 of the item: it ends with the strip's
    // columns of the last row of the K range (rows past it read zeros)
    auto set_strip_panel = [&](int k0) __attribute__((always_inline)) {
        const int rows = lK - k0;
        const int64_t es = int64_t(lkb + k0) * ldb + p.strip_n0;
        const uint32_t ns =
            rows > 0 ? uint32_t((min(rows, BK) - 1) * ldb + p.strip_cols) * 4u : 0u;
        rss = make_rsrc32(p.B + es, ns);
    };
    // sc loads, one per column; columns past strip_cols take the out-of-range offset (zeros)
    auto strip_load = [&](int stage, auto sc_tag) __attribute__((always_inline)) {
        constexpr int SC = decltype(sc_tag)::value;
        if (wave_u == 0) {
#pragma unroll
            for (int j = 0; j < SC; ++j) {
                const uint32_t off = j < p.strip_cols ? s_off + 4u * uint32_t(j) : kOob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rss, (lds_ptr)(strip_lds + ((stage * KG + kg) * SCM + j) * T::STRIP_STAGE),
                    4, off, 0, 0, 0);
            }
        }
    };
    // Row strip: the strip rows' A values of a panel go to the same LDS columns (row j of
    // stage s of group kg at strip_lds + ((s KG + kg) SCM + j) STRIP_STAGE, value k at + k),
    // one load per row by the group's first wave, lane k loading value k; values past the
    // K range and rows past rstrip read zeros. The resource spans the strip rows from the
    // panel's first k; lanes past the K range are masked by offset, since the range also
    // covers the next row's start.
    int r_kvalid = 0;
    auto set_rstrip_panel = [&](int k0) __attribute__((always_inline)) {
        r_kvalid = min(lK - k0, BK);
        const int64_t ea = int64_t(M - p.rstrip) * lda + lkb + k0;
        const uint32_t na =
            r_kvalid > 0 ? uint32_t((p.rstrip - 1) * lda + r_kvalid) * 4u : 0u;
        rss = make_rsrc32(p.A + ea, na);
    };
    auto rstrip_load = [&](int stage, auto sc_tag) __attribute__((always_inline)) {
        constexpr int SC = decltype(sc_tag)::value;
        if (wave_u == 0) {
#pragma unroll
            for (int j = 0; j < SC; ++j) {
                const uint32_t off = j < p.rstrip && lane < r_kvalid
                                         ? (uint32_t(j) * uint32_t(lda) + uint32_t(lane)) * 4u
                                         : kOob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rss, (lds_ptr)(strip_lds + ((stage * KG + kg) * SCM + j) * T::STRIP_STAGE),
                    4, off, 0, 0, 0);
            }
        }
    };
    // The empty asm after the products keeps them at this step: left alone, the compiler
    // gathers the products of a whole panel at its end, with all their operands live.
    auto strip_fma = [&](const f32x4 (&av)[RB]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc[r] += av[r][e] * sbv[e];
            asm volatile("" : "+v"(sacc[r]));
        }
    };
    // Spread strip (strip_rows > 0): every tile of the row computes strip_rows rows of the
    // strip. Thread tid of a K-group owns chunk tid % CPR (four values of k) of row slot
    // tid / CPR; per panel it reads that A chunk and each strip column's four B values for
    // it from LDS (16-byte reads) and adds their four products per column, in one step of
    // the panel. Slots past strip_rows, or rows past the tile, read row 0 and are never
    // stored.
    int sp_aoff = 0, sp_boff = 0;
    float sp_acc[SCM];
    f32x4 sp_a, sp_b[SCM];
    auto set_spread_item = [&]() __attribute__((always_inline)) {
        const int q = tid / CPR, c = tid % CPR;
        const int row = (ln0 / BN) * p.strip_rows + q;
        const int lr = q < p.strip_rows && row < BM ? row : 0;
        sp_aoff = lr * BK + 4 * (c ^ a_swizzle<CPR>(lr));
        sp_boff = 4 * c;
#pragma unroll
        for (int j = 0; j < SCM; ++j) sp_acc[j] = 0.0f;
    };
    // Row strip, mirrored: thread tid of a K-group owns chunk c = tid % CPR (four values of
    // k) of column slot tid / CPR of the tile's share; per panel it reads that column's four
    // B values from the B panel in LDS (four 4-byte reads, BN floats apart, the same chunk
    // swizzle for all four) and each strip row's four A values (16-byte reads), and adds
    // four products per row. Slots past the share, or columns past the tile, read column 0
    // and are never stored.
    auto set_rspread_item = [&]() __attribute__((always_inline)) {
        const int q = tid / CPR, c = tid % CPR;
        const int col = (lm0 / BM) * p.strip_rows + q;
        const int lc = q < p.strip_rows && col < BN ? col : 0;
        sp_aoff = 4 * c * BN + 4 * ((lc >> 2) ^ b_swizzle<MB>(4 * c)) + (lc & 3);
        sp_boff = 4 * c;
#pragma unroll
        for (int j = 0; j < SCM; ++j) sp_acc[j] = 0.0f;
    };

    // NEXT (next_tag 1 or 2): a next panel follows, whose step 0 this one reads after its
    // barrier; 2 (NextTail): that next panel is its group's last, which may hold the end of
    // the K range (fix_k_tail applies to it; no other panel's code carries the tail's
    // branch). LOADS: the panel issues the global loads of a later one, into the stage read
    // longest ago: with two stages the next panel (every NEXT panel), with three the panel
    // after next (next_tag 1 only: the last but one panel loads nothing), so that two
    // panels' loads are in flight and each has two panels' time to land.
    // NS: the k-steps of the panel that run. A group's last panel runs only the k-groups
    // (4 steps each) that hold values of k inside its range; every other panel runs all.
    // STRIP: the panel also loads the next panel's strip values and computes this one's.
    using NextTail = std::integral_constant<int, 2>;
    // The barrier after a panel, once the wave's loads of the next one have landed. With
    // three stages __syncthreads() would also wait for the loads still in flight (the
    // panel after next); only the LDS accesses need ordering there: each wave waits for its
    // own loads before it, and for its LDS reads and fix_k_tail's writes in it.
    auto stage_barrier = [&]() __attribute__((always_inline)) {
        if constexpr (NSTG == 2) __syncthreads();
        else asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    auto panel = [&](auto cur_tag, auto next_tag, auto ns_tag, auto strip_tag) __attribute__((always_inline)) {
        constexpr int SMODE = decltype(strip_tag)::value;
        constexpr bool STRIP = SMODE != 0;          // the panel loads strip values
        constexpr bool COLS = SMODE == 1;           // last tile column: the whole strip
        constexpr bool SPREAD = SMODE >= 2 && SMODE <= 4;   // a share of the strip's rows
        constexpr bool ROWS = SMODE >= 5;           // row strip: a share of its columns
        constexpr int SC = strip_mode_cols(SMODE);  // strip columns (rows) loaded per panel
        constexpr bool NEXT = decltype(next_tag)::value != 0;
        constexpr bool TAIL_NEXT = decltype(next_tag)::value == 2;
        constexpr bool LOADS = NSTG == 2 ? NEXT : decltype(next_tag)::value == 1;
        constexpr int cur = decltype(cur_tag)::value;   // -1: the stage known at run time
        constexpr int NS = decltype(ns_tag)::value;
        static_assert(NS % 4 == 0 && NS <= STEPS && (NS == STEPS || !NEXT), "steps of a panel");
        const int cur_stage = cur >= 0 ? cur : NSTG == 2 ? (panel_parity & 1) : panel_parity % 3;
        const float *As = smem + cur_stage * SSTRIDE;
        const float *Bs = As + T::A_TILE;
        // the stage read after the barrier (Anext), and the one the loads go to (load_stage,
        // Aload); with two stages both are the other stage
        float *Anext = smem + (NSTG == 2 ? cur_stage ^ 1 : cur_stage == 2 ? 0 : cur_stage + 1) * SSTRIDE;
        const int load_stage = NSTG == 2 ? cur_stage ^ 1 : cur_stage == 0 ? 2 : cur_stage - 1;
        float *Aload = NSTG == 2 ? Anext : smem + load_stage * SSTRIDE;
        const float *Ss = strip_lds + (cur_stage * KG + kg) * SCM * T::STRIP_STAGE;
        static_for<0, NS>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            constexpr int kb = t >> 2, s = t & 3;
            constexpr bool next_b = t + 1 < NS;
            constexpr bool next_a = s == 0 && 4 * (kb + 1) < NS;
            constexpr int w0 = t - (STEPS - 1 - WS);            // write group of this step
            constexpr int l_first = t * PER_LOAD;
            constexpr int n_load = (LOADS && t < LS)
                ? ((t + 1) * PER_LOAD < NL ? PER_LOAD : (NL - t * PER_LOAD > 0 ? NL - t * PER_LOAD : 0))
                : 0;
            constexpr int w_first = (w0 > 0 ? w0 : 0) * PER_WRITE;
            constexpr int n_write = (LOADS && !DL && w0 >= 0 && w0 < WS)
                ? ((w0 + 1) * PER_WRITE < NL ? PER_WRITE
                                             : (NL - w0 * PER_WRITE > 0 ? NL - w0 * PER_WRITE : 0))
                : 0;
            if constexpr (n_load > 0) {
#pragma unroll
                for (int l = l_first; l < l_first + n_load; ++l) {
                    if constexpr (DL) load_direct(Aload, l); else load_slot(l);
                }
            }
            // strip: the next panel's B values with the first loads; k-group kb's B values
            // read at its first step and its products added at its third
            constexpr int n_sload = (STRIP && LOADS && t == 0) ? SC : 0;
            constexpr bool s_rd = COLS && s == 0;
            constexpr bool s_fma = COLS && s == 2;
            constexpr int n_sprd = SPREAD && t == 0 ? 1 + SC : ROWS && t == 0 ? 4 + SC : 0;
            if constexpr (n_sload > 0) {
                if constexpr (ROWS)
                    rstrip_load(NSTG == 2 ? cur_stage ^ 1 : load_stage,
                                std::integral_constant<int, SC>{});
                else
                    strip_load(NSTG == 2 ? cur_stage ^ 1 : load_stage,
                               std::integral_constant<int, SC>{});
            }
            if constexpr (s_fma) strip_fma(a[kb & 1]);
            if constexpr (s_rd)
                sbv = *reinterpret_cast<const f32x4 *>(Ss + 4 * (S::H * kb + hi));
            if constexpr ((SPREAD || ROWS) && t == 3) {
#pragma unroll
                for (int j = 0; j < SC; ++j) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sp_acc[j] += sp_a[e] * sp_b[j][e];
                    asm volatile("" : "+v"(sp_acc[j]));
                }
            }
            if constexpr (n_sprd > 0) {
                if constexpr (ROWS) {
                    // sp_a: the column's four B values; sp_b[j]: strip row j's four A values
#pragma unroll
                    for (int e = 0; e < 4; ++e) sp_a[e] = Bs[sp_aoff + e * BN];
                } else {
                    sp_a = *reinterpret_cast<const f32x4 *>(As + sp_aoff);
                }
#pragma unroll
                for (int j = 0; j < SC; ++j)
                    sp_b[j] = *reinterpret_cast<const f32x4 *>(Ss + j * T::STRIP_STAGE + sp_boff);
            }
            if constexpr (n_write > 0) {
#pragma unroll
                for (int l = w_first; l < w_first + n_write; ++l) write_slot(Aload, l);
            }
            if constexpr (next_b) read_b(Bs, t + 1, b[(t + 1) & 1]);
            if constexpr (next_a) read_a(As, kb + 1, a[(kb + 1) & 1]);
            if constexpr (t == STEPS - 1 && NEXT) {
                // keep the previous steps' MFMAs above the barrier: they cover the
                // completion of this panel's LDS writes
                __builtin_amdgcn_sched_barrier(0);
                // direct loads land in LDS when vmcnt counts them done
                if constexpr (DL) {
                    if constexpr (NSTG == 3 && LOADS)
                        wait_vmcnt_split<NL + SC * STRIP, NL>(wave_u == 0);
                    else
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    if constexpr (TAIL_NEXT) fix_k_tail(Anext);
                }
                stage_barrier();
                read_a(Anext, 0, a[0]);
                read_b(Anext + T::A_TILE, 0, b[0]);
            }
            // pin the order: memory instructions of this step first, then its MFMAs
            if constexpr (n_load + n_sload > 0)
                __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, n_load + n_sload, 0);

            if constexpr (n_write > 0)
                __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, n_write, 0);
            if constexpr (next_b || next_a || n_sprd > 0)
                __builtin_amdgcn_sched_group_barrier(
                    kSchedDsRead, (next_b ? CG : 0) + (next_a ? RB : 0) + n_sprd, 0);
            if constexpr (t == STEPS - 1 && NEXT)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RB + CG, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, RB * CG * CI, 0);
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int g = 0; g < CG; ++g)
#pragma unroll
                    for (int j = 0; j < CI; ++j) {
                        float bj;
                        if constexpr (CI == 1) bj = b[t & 1][g]; else bj = b[t & 1][g][j];
                        constexpr int h = t % KACC;
                        acc[h][r][g * CI + j] =
                            S::mfma(a[kb & 1][r][s], bj, acc[h][r][g * CI + j]);
                    }
        });
    };

    static_assert(STEPS % KACC == 0 && 4 % KACC == 0,
                  "accumulator sets divide the k-steps of a k-group");

    // The last panel of this group: panel index kg + (rounds - 1) KG of the item. Only its
    // k-groups that reach into the K range run (none if the panel lies wholly past it, as
    // the last panel of a group can when the panel count is not a multiple of KG); the
    // values of k past the range in the k-groups that do run are zeros in LDS.
    // Tiles above 128 x 128 skip only a panel wholly past the range: shorter copies of the
    // panel next to their large accumulator sets made the compiler spill.
    constexpr int KGROUPS = STEPS / 4;
    constexpr bool TRIM = BM * BN <= 128 * 128;
    using AllSteps = std::integral_constant<int, STEPS>;
    auto last_panel = [&](auto cur_tag, int rounds, auto strip_tag) __attribute__((always_inline)) {
        const int valid = lK - (kg + (rounds - 1) * KG) * BK;
        const int nkg = valid <= 0 ? 0 : (valid + 4 * S::KSTEP - 1) / (4 * S::KSTEP);
        if (!TRIM) {
            if (nkg > 0) panel(cur_tag, std::false_type{}, AllSteps{}, strip_tag);
        } else if (nkg >= KGROUPS) {
            panel(cur_tag, std::false_type{}, AllSteps{}, strip_tag);
        } else {
            static_for<1, KGROUPS>([&](auto nc) {
                constexpr int n = decltype(nc)::value;
                if (nkg == n)
                    panel(cur_tag, std::false_type{}, std::integral_constant<int, 4 * n>{},
                          strip_tag);
            });
        }
    };

    // ---- epilogue of one tile: accumulators to C through a buffer resource ----
    const int ldc = p.ldc;
    // K-group owning store unit (r, g, q) (MfmaTile::UNITS), and the LDS slot (one f32x4 per
    // lane) of writing group w's partial sums of block (r, g CI + c), quad q
    auto unit_owner = [](int r, int g, int q) constexpr {
        return ((r * CG + g) * (T::ACC / 4) + q) * KG / T::UNITS;
    };
    auto red_slot = [&](int w, int r, int j, int q) __attribute__((always_inline)) {
        return reinterpret_cast<f32x4 *>(
            red + (((w * T::NACC + r * CI * CG + j) * (T::ACC / 4) + q) * NT + tid) * 4);
    };
    // Sum the accumulator sets into acc[0]; then (KG > 1) each group adds all groups' sums
    // of its own store units, in ascending group order, into its acc[0].
    auto finish = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int h = 1; h < KACC; ++h)
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CI * CG; ++j) acc[0][i][j] += acc[h][i][j];
        if constexpr (KG > 1) {
            // every group has read its stages for the last time before red overwrites them;
            // then each writes its sums of the units other groups own
            __syncthreads();
            static_for<0, RB>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                static_for<0, CG>([&](auto gc) {
                    constexpr int g = decltype(gc)::value;
                    static_for<0, T::ACC / 4>([&](auto qc) {
                        constexpr int q = decltype(qc)::value;
                        if (unit_owner(i, g, q) != kg) {
#pragma unroll
                            for (int c = 0; c < CI; ++c) {
                                const acc_t &x = acc[0][i][g * CI + c];
                                *red_slot(kg, i, g * CI + c, q) =
                                    f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
                            }
                        }
                    });
                });
            });
            __syncthreads();
            static_for<0, RB>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                static_for<0, CG>([&](auto gc) {
                    constexpr int g = decltype(gc)::value;
                    static_for<0, T::ACC / 4>([&](auto qc) {
                        constexpr int q = decltype(qc)::value;
                        if (unit_owner(i, g, q) == kg) {
                            // the owner's own slot is not written: its sums come from
                            // registers, and in its place the loop reads (and drops) the
                            // slot of another group, which is
                            const int alt = kg == 0 ? 1 : 0;
#pragma unroll
                            for (int c = 0; c < CI; ++c) {
                                acc_t &x = acc[0][i][g * CI + c];
                                const f32x4 own = {x[4 * q], x[4 * q + 1], x[4 * q + 2],
                                                   x[4 * q + 3]};
                                f32x4 sum;
#pragma unroll
                                for (int w = 0; w < KG; ++w) {
                                    const f32x4 part = *red_slot(w == kg ? alt : w, i,
                                                                 g * CI + c, q);
                                    const f32x4 v = w == kg ? own : part;
                                    sum = w == 0 ? v : sum + v;
                                }
#pragma unroll
                                for (int e = 0; e < 4; ++e) x[4 * q + e] = sum[e];
                            }
                        }
                    });
                });
            });
        }
    };

    // Stores the tile through resource rsc (its first element at offset 0, rows ldc4 bytes
    // apart), rows_left x cols_left of it inside the destination, with cache policy POLICY.
    auto epilogue = [&](__amdgpu_buffer_rsrc_t rsc, uint32_t ldc4, int rows_left,
                        int cols_left, auto policy_tag) __attribute__((always_inline)) {
        constexpr int POLICY = decltype(policy_tag)::value;
        // Lane (lo, hi) owns rows lrow + dr (dr = 8 (v / 4) + v % 4 for accumulator v) and
        // columns col .. col + CI - 1 of each of its blocks. The row step dr * ldc goes in
        // the scalar offset; rows past M and chunks that cross N get voffset kOob (the
        // hardware drops those stores), and only a tile on the N edge stores the partial
        // chunks element by element.
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int lrow = wm * WM + r * MB + 4 * hi;
#pragma unroll
            for (int g = 0; g < CG; ++g) {
                const int col = wn * WN + g * MB * CI + CI * lo;
                const uint32_t vbase = uint32_t(lrow) * ldc4 + uint32_t(col) * 4u;
                const bool col_full = col + CI <= cols_left;
#pragma unroll
                for (int v = 0; v < T::ACC; ++v) {
                    if (unit_owner(r, g, v / 4) != kg) continue;
                    const int dr = S::row(v);
                    bvec out;
#pragma unroll
                    for (int j = 0; j < CI; ++j) {
                        if constexpr (CI == 1) out = acc[0][r][g * CI + j][v];
                        else out[j] = acc[0][r][g * CI + j][v];
                    }
                    const bool ok = col_full && lrow + dr < rows_left;
                    store_vec<CI, POLICY>(rsc, ok ? vbase : kOob, uint32_t(dr) * ldc4, out);
                    store_data_guard<CI >= 4>();
                }
            }
        }
        if (cols_left < BN) {
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int lrow = wm * WM + r * MB + 4 * hi;
#pragma unroll
                for (int g = 0; g < CG; ++g) {
                    const int col = wn * WN + g * MB * CI + CI * lo;
                    const uint32_t vbase = uint32_t(lrow) * ldc4 + uint32_t(col) * 4u;
                    const bool partial = col < cols_left && col + CI > cols_left;
#pragma unroll
                    for (int v = 0; v < T::ACC; ++v) {
                        if (unit_owner(r, g, v / 4) != kg) continue;
                        const int dr = S::row(v);
                        const bool ok = partial && lrow + dr < rows_left;
#pragma unroll
                        for (int j = 0; j < CI; ++j)
                            store_vec<1, POLICY>(rsc,
                                                 ok && col + j < cols_left ? vbase + 4u * j : kOob,
                                                 uint32_t(dr) * ldc4, acc[0][r][g * CI + j][v]);
                    }
                }
            }
        }
    };

    // one pass per item: once, or once per segment of a stream-K range
    for (;;) {
        bool to_workspace = false;
        int slot = 0;
        if constexpr (SK) {
            if (sk_mode) {
                if (sk_i >= sk_end) break;
                const int P = p.sk.panels;
                const int t = sk_i / P;
                const int kb = sk_i - t * P;
                const int ke = min(P, kb + (sk_end - sk_i));
                to_workspace = kb != 0 || ke != P;
                slot = 2 * sk_g + (sk_i == sk_start(p.sk, sk_g) ? 0 : 1);
                int tm, tn;
                grouped_tile(p.sk.tiles_dp + t, p.tiles_m, p.tiles_n, tm, tn);
                lm0 = __builtin_amdgcn_readfirstlane(tm * BM);
                ln0 = __builtin_amdgcn_readfirstlane(tn * BN);
                lkb = __builtin_amdgcn_readfirstlane(kb * BK);
                lK = __builtin_amdgcn_readfirstlane(min(K, ke * BK) - kb * BK);
                sk_i += ke - kb;
#pragma unroll
                for (int h = 0; h < KACC; ++h)
#pragma unroll
                    for (int i = 0; i < RB; ++i)
#pragma unroll
                        for (int j = 0; j < CI * CG; ++j) acc[h][i][j] = acc_t{};
                // every wave is done with the previous segment's LDS (operands and K-group
                // sums) before this one's first loads overwrite it
                __syncthreads();
            }
        }

        // ---- the item: the K loop of group kg (panels kg, kg + KG, ...), the K-group sums
        // and the epilogue, into C or (a partial stream-K tile) into workspace slot `slot`;
        // with STRIP also the column strip's rows of this tile
        auto run_item = [&](auto strip_tag) __attribute__((always_inline)) {
            constexpr int SMODE = decltype(strip_tag)::value;
            constexpr bool STRIP = SMODE != 0;
            constexpr int SC = strip_mode_cols(SMODE);
            using ScTag = std::integral_constant<int, SC>;
            constexpr bool ROWS = SMODE >= 5;
            auto setp = [&](int k0) __attribute__((always_inline)) {
                set_panel(k0);
                if constexpr (ROWS) set_rstrip_panel(k0);
                else if constexpr (STRIP) set_strip_panel(k0);
            };
            // the first loads of a panel: the strip's with the operands'
            auto sload = [&](int stage) __attribute__((always_inline)) {
                if constexpr (ROWS) rstrip_load(stage, ScTag{});
                else if constexpr (STRIP) strip_load(stage, ScTag{});
            };
            set_item();
            if constexpr (STRIP && !ROWS) set_strip_item();
            if constexpr (SMODE >= 2 && !ROWS) set_spread_item();
            if constexpr (ROWS) set_rspread_item();
            // rounds of panels of this group; a group whose last panel lies past the K range
            // loads only zeros for it
            auto group_rounds = [&]() { return ((lK + BK - 1) / BK + KG - 1) / KG; };
            setp(kg * BK);
            if constexpr (DL) {
#pragma unroll
                for (int l = 0; l < NL; ++l) load_direct(smem, l);
                sload(0);
                if constexpr (NSTG == 3) {
                    if (group_rounds() > 1) {
                        // the second panel's loads too, left in flight (the first panel is
                        // not its group's last, so it holds no end of the K range)
                        setp((KG + kg) * BK);
#pragma unroll
                        for (int l = 0; l < NL; ++l) load_direct(smem + SSTRIDE, l);
                        sload(1);
                        wait_vmcnt_split<NL + SC, NL>(wave_u == 0);
                    } else {
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                        fix_k_tail(smem);
                    }
                } else {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    fix_k_tail(smem);
                }
            } else {
#pragma unroll
                for (int l = 0; l < NL; ++l) load_slot(l);
#pragma unroll
                for (int l = 0; l < NL; ++l) write_slot(smem, l);
            }
            stage_barrier();
            read_a(smem, 0, a[0]);
            read_b(smem + T::A_TILE, 0, b[0]);

            const int rounds = group_rounds();
            // The loops never stage the last round's panel: the last two rounds run after
            // them, with the LDS stage known at run time, so the tail's code (the panel that
            // reads the last round's panel first, and the trimmed copies of the last panel)
            // exists once and no loop iteration carries it. The last round stages nothing,
            // and with three stages neither does the one before it.
            using SR = std::integral_constant<int, -1>;
            int r = 0;
            if constexpr (NSTG == 3) {
                // panel r loads panel r + 2; unrolled by three (constant stages) as PAIR is
                // by two
                using S0 = std::integral_constant<int, 0>;
                using S1 = std::integral_constant<int, 1>;
                using S2 = std::integral_constant<int, 2>;
                if constexpr (PAIR) {
                    for (; r + 4 < rounds; r += 3) {
                        setp(((r + 2) * KG + kg) * BK);
                        panel(S0{}, std::true_type{}, AllSteps{}, strip_tag);
                        setp(((r + 3) * KG + kg) * BK);
                        panel(S1{}, std::true_type{}, AllSteps{}, strip_tag);
                        setp(((r + 4) * KG + kg) * BK);
                        panel(S2{}, std::true_type{}, AllSteps{}, strip_tag);
                    }
                    if (r + 2 < rounds) {
                        setp(((r + 2) * KG + kg) * BK);
                        panel(S0{}, std::true_type{}, AllSteps{}, strip_tag);
                        ++r;
                    }
                    if (r + 2 < rounds) {
                        setp(((r + 2) * KG + kg) * BK);
                        panel(S1{}, std::true_type{}, AllSteps{}, strip_tag);
                        ++r;
                    }
                } else {
                    for (; r + 2 < rounds; ++r) {
                        setp(((r + 2) * KG + kg) * BK);
                        panel_parity = r;
                        panel(SR{}, std::true_type{}, AllSteps{}, strip_tag);
                    }
                }
                // the last round's loads were issued two panels ago (or in the prologue)
                if (r + 1 < rounds) {
                    panel_parity = r;
                    panel(SR{}, NextTail{}, AllSteps{}, strip_tag);
                }
            } else if constexpr (PAIR) {
                // two panels per iteration, so each one's LDS stage is a constant and its
                // operand reads carry the stage in their immediate offsets (no address
                // arithmetic on the vector ALU between the MFMAs)
                using S0 = std::integral_constant<int, 0>;
                using S1 = std::integral_constant<int, 1>;
                for (; r + 3 < rounds; r += 2) {
                    setp(((r + 1) * KG + kg) * BK);
                    panel(S0{}, std::true_type{}, AllSteps{}, strip_tag);
                    setp(((r + 2) * KG + kg) * BK);
                    panel(S1{}, std::true_type{}, AllSteps{}, strip_tag);
                }
                if (r + 3 == rounds) {
                    setp(((r + 1) * KG + kg) * BK);
                    panel(S0{}, std::true_type{}, AllSteps{}, strip_tag);
                    ++r;
                }
            } else {
                for (; r + 2 < rounds; ++r) {
                    setp(((r + 1) * KG + kg) * BK);
                    panel_parity = r;
                    panel(SR{}, std::true_type{}, AllSteps{}, strip_tag);
                }
            }
            if constexpr (NSTG == 2) {
                if (r + 1 < rounds) {
                    setp(((r + 1) * KG + kg) * BK);
                    panel_parity = r;
                    panel(SR{}, NextTail{}, AllSteps{}, strip_tag);
                }
            }
            panel_parity = rounds - 1;
            last_panel(SR{}, rounds, strip_tag);
            // the spread strip's partial sums go to LDS before the K-group sums, whose
            // barriers (KG > 1) then order them before the reads below
            if constexpr (SMODE >= 2) {
#pragma unroll
                for (int j = 0; j < SC; ++j) strip_red[(j * KG + kg) * NT + tid] = sp_acc[j];
            }
            finish();
            if constexpr (ROWS) {
                // each column's chunk sums, K-group by K-group, in ascending order of both,
                // for each of the strip's rows
                if constexpr (KG == 1) __syncthreads();
                const int q = threadIdx.x;
                const int col = (lm0 / BM) * p.strip_rows + q;
                if (q < p.strip_rows && col < BN && ln0 + col < N) {
                    for (int j = 0; j < SC && j < p.rstrip; ++j) {
                        float v = 0.0f;
                        for (int g = 0; g < KG; ++g)
                            for (int c = 0; c < CPR; ++c)
                                v += strip_red[(j * KG + g) * NT + q * CPR + c];
                        p.C[int64_t(M - p.rstrip + j) * ldc + ln0 + col] = v;
                    }
                }
            }
            if constexpr (SMODE >= 2 && !ROWS) {
                // each row's chunk sums, K-group by K-group, in ascending order of both, for
                // each of the strip's columns
                if constexpr (KG == 1) __syncthreads();
                const int q = threadIdx.x;
                const int row = (ln0 / BN) * p.strip_rows + q;
                if (q < p.strip_rows && row < BM && lm0 + row < M) {
                    for (int j = 0; j < SC && j < p.strip_cols; ++j) {
                        float v = 0.0f;
                        for (int g = 0; g < KG; ++g)
                            for (int c = 0; c < CPR; ++c)
                                v += strip_red[(j * KG + g) * NT + q * CPR + c];
                        p.C[int64_t(lm0 + row) * ldc + p.strip_n0 + j] = v;
                    }
                }
            }
            if constexpr (SMODE == 1) {
                // the wn = 0 waves' partial sums of each (K-group, lane group) for each row,
                // then their sum in ascending order of both, stored to C (rows past M are not)
                if (wn == 0) {
#pragma unroll
                    for (int r = 0; r < RB; ++r)
                        strip_red[(kg * S::H + hi) * T::STRIP_RS + wm * WM + r * MB + lo] =
                            sacc[r];
                }
                __syncthreads();
                const int row = threadIdx.x;
                if (row < BM && lm0 + row < M) {
                    float v = 0.0f;
                    for (int g = 0; g < KG * S::H; ++g) v += strip_red[g * T::STRIP_RS + row];
                    p.C[int64_t(lm0 + row) * ldc + p.strip_n0] = v;
                }
            }
        };
        using NoStrip = std::integral_constant<int, 0>;
        // the host launches the kernel of the plan's strip form (strip_kernel_mode); in the
        // last-column form only the last tile column computes the strip
        if constexpr (FORM == 1) {
            if (ln0 + BN == p.strip_n0)
                run_item(std::integral_constant<int, 1>{});
            else
                run_item(NoStrip{});
        } else {
            run_item(std::integral_constant<int, FORM>{});
        }
        {   // every K-group stores its own units of the tile
            if (!to_workspace) {
                const int64_t ec = ls * p.c_split_stride + int64_t(lm0) * ldc + ln0;
                epilogue(make_rsrc(p.C + ec, p.c_bytes - ec * 4), uint32_t(ldc) * 4u, M - lm0,
                         N - ln0, std::integral_constant<int, kStoreNonTemporal>{});
            } else {
                // a partial tile: all BM x BN sums, packed rows of BN floats
                epilogue(make_rsrc(p.W + int64_t(slot) * BM * BN, int64_t(BM) * BN * 4),
                         uint32_t(BN) * 4u, BM, BN, std::integral_constant<int, kStorePartial>{});
            }
        }
        if (!SK || !sk_mode) break;
    }
}

// C[i][j] = sum over s of W[s * stride + i * N + j], in ascending s: the second pass of
// split-K (a fixed summation order, so repeated runs give identical bits). Each lane owns
// VW consecutive columns of one row (VW = 4 needs N % 4 == 0 and a 16-byte aligned W; the
// stores to C are 16-byte wide only when c_vec says C's rows allow it). The slices are
// loaded in batches of kReduceBatch, all in flight together, and then added in order, so
// a whole batch costs one memory latency rather than one per slice.
constexpr int kReduceBatch = 16;

template <int VW>
__global__ __launch_bounds__(64) void k_splitk_reduce(int M, int N, int splits,
                                                     const float *__restrict__ W, int64_t stride,
                                                     float *__restrict__ C, int ldc, int c_vec)
{
    using V = typename std::conditional<VW == 4, f32x4, float>::type;
    const int64_t groups = int64_t(M) * (N / VW);
    for (int64_t gi = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; gi < groups;
         gi += int64_t(gridDim.x) * blockDim.x) {
        const int64_t e = gi * VW;
        V acc = *reinterpret_cast<const V *>(W + e);
        for (int s0 = 1; s0 < splits; s0 += kReduceBatch) {
            V t[kReduceBatch];
#pragma unroll
            for (int u = 0; u < kReduceBatch; ++u)
                if (s0 + u < splits) t[u] = *reinterpret_cast<const V *>(W + (s0 + u) * stride + e);
#pragma unroll
            for (int u = 0; u < kReduceBatch; ++u)
                if (s0 + u < splits) acc += t[u];
        }
        const int64_t row = e / N;
        float *dst = C + row * ldc + (e - row * N);
        if constexpr (VW == 4) {
            if (c_vec) {
                *reinterpret_cast<f32x4 *>(dst) = acc;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[j] = acc[j];
            }
        } else {
            *dst = acc;
        }
    }
}

// Stream-K fixup: every shared tile (streamk.hpp) gets the sum of its workgroups' partial
// tiles, added in ascending workgroup order, i.e. ascending K, so repeated runs give
// identical bits. One workgroup of 256 threads per shared tile; a tile that one workgroup
// covered whole was written to C by it and is skipped. Each thread owns kFixupChunks
// 16-byte chunks per pass (fewer in a last, partial pass) and loads them from up to
// kFixupBatch contributors at once
// (the first batch includes the first contributor, so a tile shared by a few workgroups
// costs one memory latency), then adds them in order. W must be 16-byte aligned; C's rows
// are stored 16 bytes at a time when ldc and C allow it, else element by element.
constexpr int kFixupChunks = 4;

template <int BM, int BN>
__global__ __launch_bounds__(256) void k_streamk_fixup(GemmArgs p)
{
    const SkGeom s = p.sk;
    const int t = blockIdx.x;
    const int u0 = t * s.panels;
    const int g0 = sk_owner(s, u0), g1 = sk_owner(s, u0 + s.panels - 1);
    if (g0 == g1) return;
    int tm, tn;
    grouped_tile(s.tiles_dp + t, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool c_vec = (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0;
    constexpr int CH = BM * BN / 4;                 // chunks per tile
    static_assert(CH % 256 == 0, "chunks divide over the workgroup");
    constexpr int PASS = 256 * kFixupChunks;        // chunks per full pass
    const int tid = threadIdx.x;
    // one pass over chunks c0 + q 256 + tid, q < NQ
    auto pass = [&](int c0, auto nq_tag) {
        constexpr int NQ = decltype(nq_tag)::value;
        f32x4 acc[NQ];
        for (int g = g0; g <= g1; g += kFixupBatch) {
            f32x4 v[kFixupBatch][NQ];
#pragma unroll
            for (int u = 0; u < kFixupBatch; ++u) {
                if (g + u > g1) break;
                const float *w = p.W + int64_t(sk_fixup_slot(s, g + u, g0, t)) * (BM * BN);
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    v[u][q] = *reinterpret_cast<const f32x4 *>(w + 4 * (c0 + q * 256 + tid));
            }
#pragma unroll
            for (int u = 0; u < kFixupBatch; ++u) {
                if (g + u > g1) break;
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    acc[q] = (g + u == g0) ? v[u][q] : acc[q] + v[u][q];
            }
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int c = c0 + q * 256 + tid;
            const int r = c / (BN / 4), col = 4 * (c % (BN / 4));
            const int row = m0 + r, left = p.N - (n0 + col);
            if (row >= p.M || left <= 0) continue;
            float *dst = p.C + int64_t(row) * p.ldc + n0 + col;
            if (c_vec && left >= 4) {
                *reinterpret_cast<f32x4 *>(dst) = acc[q];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j < left) dst[j] = acc[q][j];
            }
        }
    };
    for (int c0 = 0; c0 + PASS <= CH; c0 += PASS)
        pass(c0, std::integral_constant<int, kFixupChunks>{});
    if constexpr (CH % PASS != 0)
        pass(CH - CH % PASS, std::integral_constant<int, (CH % PASS) / 256>{});
}

}  // namespace sgemm
