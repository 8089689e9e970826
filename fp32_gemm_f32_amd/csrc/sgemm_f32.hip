// sgemm_f32.hip -- the C ABI declared in include/sgemm_f32.h.
//
// Every entry point validates its arguments first (pure host code, sgemm_validate.hpp),
// then takes the quick returns, then launches on the caller's stream. Launches go through
// hipLaunchKernel so the runtime's own status is returned, not a stale error left by
// earlier calls on the thread.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <vector>

#include "sgemm_f32.h"
#include "sgemm_validate.hpp"
#include "kernels_simple.hpp"
#include "kernels_ladder.hpp"
#include "kernel_mfma.hpp"
#include "plan.hpp"

namespace sgemm {
namespace {

constexpr int kAbiVersion = 2;
// Hardware grid dimensions above 65535 workgroups in y are avoided; the simple kernels
// stride their rows over the grid instead.
constexpr unsigned kMaxGridY = 65535;

template <typename... KArgs, typename... Args>
int launch(void (*kern)(KArgs...), dim3 grid, dim3 block, void *stream, Args... args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    void *argv[] = {static_cast<void *>(&args)...};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kern), grid, block,
                                         argv, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SGEMM_OK : SGEMM_ELAUNCH;
}

int fill_zero(int M, int N, float *C, int ldc, void *stream)
{
    const int64_t total = int64_t(M) * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return launch(k_fill_zero, dim3(unsigned(blocks)), dim3(256), stream, M, N, C, ldc);
}

// ------------------------------------------------------------------ variants ----------

typedef void (*MfmaKernel)(GemmArgs);

}  // namespace
// k_sgemm_regpanel lives in sgemm_regpanel.hip (a translation unit built with other options)
MfmaKernel regpanel_kernel();
MfmaKernel regpanel_streamk_kernel();
// k_sgemm_persist lives in sgemm_persist.hip (same reason)
MfmaKernel persist_kernel(int waves);
MfmaKernel persist_ktail_kernel(int waves);
namespace {

struct VariantEntry {
    Variant v;
    MfmaKernel kern;
    MfmaKernel kern_sk;     // stream-K form (NULL for variants without one)
    MfmaKernel fixup;       // its fixup kernel
    int threads;
    int mb;                 // MFMA block size (32: 32x32x2, 16: 16x16x4)
    int kg;                 // K-groups
    const char *kernel;     // kernel family: "mfma" (kernel_mfma.hpp), "regpanel", "persist"
    bool persistent = false;       // one workgroup per CU walks the tiles (kernel_persist.hpp)
    MfmaKernel kern_ktail = nullptr;   // its form for a K that is not a multiple of BK
    int stages = 2;                    // LDS stages per K-group (the template kernel)
    // the plain kernel's strip forms, indexed by strip_kernel_mode (1-7; null where the
    // tile cannot hold the form)
    MfmaKernel kern_strip[8] = {};
};

// The strip form a plain launch computes (k_sgemm_mfma's SMODE): 0 none; 1 one column in
// the last tile column; 2-4 one, two or four (three) columns spread over the tile rows;
// 5-7 one, two or four (three) rows spread over the tile columns.
int strip_kernel_mode(const GemmArgs &p)
{
    if (p.rstrip > 0) return p.rstrip == 1 ? 5 : p.rstrip == 2 ? 6 : 7;
    if (p.strip_cols > 0)
        return p.strip_rows == 0 ? 1 : p.strip_cols == 1 ? 2 : p.strip_cols == 2 ? 3 : 4;
    return 0;
}

template <int BM, int BN, int BK, int WGM, int WGN, int KACC, int KG, bool DL, int MB, int NSTG,
          int SMODE>
constexpr MfmaKernel strip_kernel()
{
    using Tile = MfmaTile<BM, BN, BK, WGM, WGN, KACC, KG, MB, NSTG>;
    if constexpr (DL && Tile::STRIP_OK && strip_mode_cols(SMODE) <= Tile::STRIP_COLS_MAX)
        return &k_sgemm_mfma<BM, BN, BK, WGM, WGN, KACC, KG, DL, false, MB, NSTG, SMODE>;
    else
        return nullptr;
}

// PLANNED variants also get a stream-K form and its fixup kernel; the others are never
// planned and are instantiated in their plain form only.
template <int BM, int BN, int BK, int WGM, int WGN, int KACC, int KG, bool DL, bool PLANNED,
          int MB = 32, int NSTG = 2>
constexpr VariantEntry entry(const char *name, int wg_per_cu, double rate, double overhead,
                             double solo, double latency, double sk_price = kStreamkPrice)
{
    MfmaKernel sk = nullptr, fix = nullptr;
    if constexpr (PLANNED) {
        sk = &k_sgemm_mfma<BM, BN, BK, WGM, WGN, KACC, KG, DL, true, MB, NSTG>;
        fix = &k_streamk_fixup<BM, BN>;
    }
    VariantEntry e{
        Variant{name, BM, BN, BK, WGM, WGN, wg_per_cu, rate, overhead, solo, DL, PLANNED},
        &k_sgemm_mfma<BM, BN, BK, WGM, WGN, KACC, KG, DL, false, MB, NSTG>, sk, fix,
        64 * WGM * WGN * KG, MB, KG, "mfma"};
    // the kernel's column strip (kernel_mfma.hpp): direct loads and room in LDS
    using Tile = MfmaTile<BM, BN, BK, WGM, WGN, KACC, KG, MB, NSTG>;
    e.v.strip = DL && Tile::STRIP_OK;
    e.v.strip_cols_max = e.v.strip ? Tile::STRIP_COLS_MAX : 0;
    e.v.sk_price = sk_price;
    e.v.latency = latency;
    e.stages = NSTG;
    e.kern_strip[1] = strip_kernel<BM, BN, BK, WGM, WGN, KACC, KG, DL, MB, NSTG, 1>();
    e.kern_strip[2] = strip_kernel<BM, BN, BK, WGM, WGN, KACC, KG, DL, MB, NSTG, 2>();
    e.kern_strip[3] = strip_kernel<BM, BN, BK, WGM, WGN, KACC, KG, DL, MB, NSTG, 3>();
    e.kern_strip[4] = strip_kernel<BM, BN, BK, WGM, WGN, KACC, KG, DL, MB, NSTG, 4>();
    e.kern_strip[5] = strip_kernel<BM, BN, BK, WGM, WGN, KACC, KG, DL, MB, NSTG, 5>();
    e.kern_strip[6] = strip_kernel<BM, BN, BK, WGM, WGN, KACC, KG, DL, MB, NSTG, 6>();
    e.kern_strip[7] = strip_kernel<BM, BN, BK, WGM, WGN, KACC, KG, DL, MB, NSTG, 7>();
    return e;
}

// The one-wave-per-SIMD kernel (kernel_regpanel.hpp): 256 x 256 tiles of four 128 x 128
// waves, with a stream-K form. Split-K does not plan it: its shapes have few tiles, where
// the smaller tiles win.
VariantEntry regpanel_entry(const char *name, double rate, double overhead, double latency)
{
    VariantEntry e{
        Variant{name, 256, 256, 32, 2, 2, 1, rate, overhead, 1.0, false, true, false},
        regpanel_kernel(), regpanel_streamk_kernel(), &k_streamk_fixup<256, 256>, 256, 32, 1,
        "regpanel"};
    // its stream-K form runs about 2 % over its price (4500^2 x 8192, 3000^2 x 8192,
    // 2500^2 x 16384, measured at steady state), besides the plain model's drift
    e.v.sk_price = 1.06;
    e.v.latency = latency;
    return e;
}

// The persistent kernel (kernel_persist.hpp): 128 x 256 tiles of four 64 x 128 waves (one
// per SIMD) or eight 64 x 64 waves (two per SIMD), one workgroup per CU, each tile's C
// stored among the next tile's MFMAs. Whole tiles only, at least two K-panels (the edges of
// a ragged product run through the plan after it, run_persistent); no split-K or stream-K
// form.
VariantEntry persist_entry(const char *name, int waves, bool planned, double rate,
                           double overhead, double latency)
{
    VariantEntry e{Variant{name, 128, 256, 32, 2, waves / 2, 1, rate, overhead, 1.0, false, planned,
                           false},
                   persist_kernel(waves), nullptr, nullptr, 64 * waves, 32, 1, "persist"};
    e.v.whole_tiles = true;
    e.persistent = true;
    e.kern_ktail = persist_ktail_kernel(waves);
    e.v.latency = latency;
    return e;
}

// Rates (throughput relative to 140 TFLOP/s), per-tile overheads (in units of K), solo
// factors and launch latencies (microseconds) of the planned variants are fitted on MI355X
// to steady-state times of every planned variant, forced, on 154 shapes (bench.py
// --plan-sweep): 68 chosen ones (1024-class, ragged, mid-size, low K, one tile per CU and
// many, K up to 32768) and 86 drawn at random (M and N log-uniform in 256..16384, K in
// 32..8192, at most 2e11 multiply-adds). Each variant's four constants are fitted first to
// its own times (least squares on the logarithm), then moved, from there, to lower the
// plan's regret over those shapes while the picks for 1024^3, 1023 x 1025 x 1027, 8192^3,
// 16384^2 x 64 and 256^2 x 32768 stay the fastest variants measured there. The forced-only
// variants keep the constants of the earlier fit (19 shapes) and no latency: the plan never
// prices them. The template kernel's planned variants load their panels
// straight into LDS ("_dl"), which measured as fast as or faster than staging through
// registers on every one of those shapes.
//  * 256 x 256, one wave per SIMD ("_rp", kernel_regpanel.hpp): long K and many tiles
//    (8192^3, 4096^3, 8192^2 x 1024), and as stream-K large ragged tile counts.
//  * 256 x 256 (8 waves of 64 x 128): the same tile in the template kernel; "_rp" is faster
//    on every measured shape, so it is no longer planned (forced use only).
//  * 128 x 256 (4 waves, 48 KiB of LDS): two workgroups per CU, so one stores while the
//    other computes; best when K is short and C's stores weigh as much as the MFMAs.
//  * 128 x 128 (4 waves, two per CU): shapes with about one 256 x 256 tile per CU or fewer.
//  * 64 x 64 as four K-groups of two 32 x 64 waves (several waves per SIMD on one tile,
//    two MFMAs per k-step each): shapes that give every CU about one tile.
//  * 64 x 64 as two K-groups, two workgroups per CU: shapes with a few such tiles per CU,
//    and ragged ones whose tile count just exceeds the CU count.
// The last entry stages through registers; it is never planned and stays as the measured
// comparison for the direct loads (forced through sgemm_f32_variant).
const VariantEntry kVariants[] = {
    entry<256, 256, 32, 4, 2, 1, 1, true, false>("mfma_256x256x32_w4x2_dl", 1, 1.085, 40, 1.0, 0.0),
    entry<128, 256, 16, 2, 2, 1, 1, true, true>("mfma_128x256x16_w2x2_dl", 2, 1.099, 38, 0.972,
                                                 3.30),
    entry<128, 128, 32, 2, 2, 1, 1, true, true>("mfma_128x128x32_w2x2_dl", 2, 1.099, 46, 0.978,
                                                 2.30),
    entry<64, 64, 32, 2, 1, 2, 4, true, false>("mfma_64x64x32_w2x1_acc2_kg4_dl", 1, 0.880, 212, 1.0,
                                                0.0),
    // its stream-K form is not planned: at 1536^2 x 4096 it ran 25 % slower than the plain
    // plan that its price matched (it still runs when forced). With one tile per CU (one wave
    // per SIMD) it runs 0.3-3 % ahead of the 64 x 64 x 64 tile up to K = 1024, within 0.6 %
    // of it at K = 1536-2048 and behind it from K = 3072, and behind it with a column strip
    // (1024^2 x 512 .. 4096, 1000^3, 1023 x 1024 x 1027 against 1023 x 1025 x 1027, steady
    // state).
    entry<64, 64, 32, 2, 1, 1, 2, true, true>("mfma_64x64x32_w2x1_kg2_dl", 2, 1.039, 76, 0.993,
                                              2.80, 0.0),
    entry<256, 256, 32, 4, 2, 1, 1, false, false>("mfma_256x256x32_w4x2", 1, 1.045, 52, 1.0, 0.0),
    entry<80, 64, 32, 1, 2, 1, 4, true, true, 16>("mfma16_80x64x32_w1x2_kg4_dl", 1, 1.041, 168, 1.0,
                                                   2.00),
    entry<80, 64, 32, 1, 2, 1, 2, true, true, 16>("mfma16_80x64x32_w1x2_kg2_dl", 2, 1.063, 75, 0.960,
                                                   3.00),
    entry<48, 64, 32, 1, 2, 1, 4, true, true, 16>("mfma16_48x64x32_w1x2_kg4_dl", 1, 0.975, 218, 1.0,
                                                   1.80),
    entry<64, 64, 64, 2, 2, 1, 2, true, true, 16>("mfma16_64x64x64_w2x2_kg2_dl", 1, 1.041, 161, 1.0,
                                                   1.85),
    regpanel_entry("mfma_256x256x32_w2x2_rp", 1.114, 51, 3.60),
    persist_entry("mfma_128x256x32_w2x2_ps", 4, false, 1.05, 0, 0.0),
    persist_entry("mfma_128x256x32_w2x4_ps", 8, true, 1.110, 29, 2.65),
    // 64 x 64 in 16-row blocks, two K-groups of four 32 x 32 waves, 32-deep panels (forced
    // use only)
    entry<64, 64, 32, 2, 2, 1, 2, true, false, 16>("mfma16_64x64x32_w2x2_kg2_dl", 2, 1.0, 26,
                                                   0.887, 0.0),
    // the same tile and the 32 x 32 one of two K-groups with three LDS stages per K-group:
    // each panel's loads are issued two panels ahead (96 KiB of LDS, one workgroup per CU;
    // forced use only)
    entry<64, 64, 32, 2, 2, 1, 2, true, false, 16, 3>("mfma16_64x64x32_w2x2_kg2_s3_dl", 1, 1.0,
                                                      26, 1.0, 0.0),
    entry<64, 64, 32, 2, 1, 1, 2, true, false, 32, 3>("mfma_64x64x32_w2x1_kg2_s3_dl", 1, 1.0, 92,
                                                      1.0, 0.0),
    // Tiles of one 32 x 32 block per wave for products with few 64 x 64 tiles (under one per
    // CU): 32 x 32 as eight K-groups of one wave (two per SIMD) with three LDS stages, whose
    // 16-deep panels are too short for two stages to hide a load (the two-stage form stays as
    // the measured comparison, forced use only); and 32 x 64 as four K-groups of two waves.
    // Their stream-K forms are not planned (not calibrated).
    entry<32, 32, 16, 1, 1, 1, 8, true, true, 32, 3>("mfma_32x32x16_w1x1_kg8_s3_dl", 1, 0.787,
                                                     583, 1.0, 1.65, 0.0),
    entry<32, 32, 16, 1, 1, 1, 8, true, false>("mfma_32x32x16_w1x1_kg8_dl", 1, 0.8125, 1082, 1.0,
                                               0.0),
    entry<32, 64, 32, 1, 2, 1, 4, true, true>("mfma_32x64x32_w1x2_kg4_dl", 1, 0.895, 295, 1.0,
                                              1.75, 0.0),
};
constexpr int kNumVariants = int(sizeof(kVariants) / sizeof(kVariants[0]));

Variant g_table[kNumVariants];
struct TableInit {
    TableInit() { for (int i = 0; i < kNumVariants; ++i) g_table[i] = kVariants[i].v; }
} g_table_init;

Operands make_operands(int M, int N, int K, int lda, int ldb, int ldc)
{
    Operands o;
    o.M = M; o.N = N; o.K = K; o.lda = lda; o.ldb = ldb; o.ldc = ldc;
    return o;
}

std::atomic<int> g_cus[64];

int device_cus(int *out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SGEMM_ELAUNCH;
    if (dev >= 0 && dev < 64) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) { *out = c; return SGEMM_OK; }
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return SGEMM_ELAUNCH;
    if (dev >= 0 && dev < 64) g_cus[dev].store(n, std::memory_order_relaxed);
    *out = n;
    return SGEMM_OK;
}

static_assert(kStripCols == kStripColsMax, "strip width of the kernels and of the plan");

// Kernel arguments of the plain product with variant e; with `cus` > 0, a thin remainder of
// N goes to strip workgroups when the plan prices that lower (strip_cols).
GemmArgs plain_args(const VariantEntry &e, const Operands &o, const float *A, const float *B,
                    float *C, int cus = 0)
{
    GemmArgs p{};
    p.A = A; p.B = B; p.C = C;
    p.a_bytes = span_elems(o.M, o.K, o.lda) * 4;
    p.b_bytes = span_elems(o.K, o.N, o.ldb) * 4;
    p.c_bytes = span_elems(o.M, o.N, o.ldc) * 4;
    p.M = o.M; p.N = o.N; p.K = o.K; p.lda = o.lda; p.ldb = o.ldb; p.ldc = o.ldc;
    const int rr = cus > 0 ? rstrip_rows(e.v, o, cus) : 0;
    const int r = cus > 0 && rr == 0 ? strip_cols(e.v, o, cus) : 0;
    p.tiles_m = rr > 0 ? o.M / e.v.BM : (o.M + e.v.BM - 1) / e.v.BM;
    p.tiles_n = (o.N - r + e.v.BN - 1) / e.v.BN;
    p.splits = 1;
    p.k_chunk = o.K;
    p.c_split_stride = 0;
    p.strip_n0 = o.N - r;
    p.strip_cols = r;
    p.strip_rows = rr > 0 ? rstrip_share_cols(e.v, o) : r > 0 ? strip_form_rows(e.v, o, cus) : 0;
    p.rstrip = rr;
    return p;
}

size_t streamk_workspace_bytes(const Variant &v, const SkGeom &g)
{
    return g.tiles_sk > 0 ? size_t(2) * size_t(g.G) * size_t(v.BM) * size_t(v.BN) * 4u : 0;
}

// Stream-K with variant v: the partition for this shape, with G = CUs x the variant's
// resident workgroups per CU; of the two ways to pick the shared tiles (streamk.hpp), the
// one streamk_cost prices lower. *cost receives that price when non-null.
SkGeom streamk_geometry(const Variant &v, const Operands &o, int cus, double *cost = nullptr)
{
    const int64_t tiles = ((int64_t(o.M) + v.BM - 1) / v.BM) * ((int64_t(o.N) + v.BN - 1) / v.BN);
    const int panels = (o.K + v.BK - 1) / v.BK;
    SkGeom best = sk_geometry(tiles, panels, cus * v.wg_per_cu, false);
    double best_cost = best.tiles_sk ? streamk_cost(v, o, cus, best,
                                                    streamk_workspace_bytes(v, best)) : 0.0;
    const SkGeom alt = sk_geometry(tiles, panels, cus * v.wg_per_cu, true);
    if (alt.tiles_sk > 0 && alt.tiles_dp != best.tiles_dp) {
        const double c = streamk_cost(v, o, cus, alt, streamk_workspace_bytes(v, alt));
        if (c < best_cost) { best = alt; best_cost = c; }
    }
    if (cost) *cost = best_cost;
    return best;
}

// The stream-K entry's choice: the cheapest of every planned variant run plainly or as
// stream-K (streamk_cost in plan.hpp). Returns the variant index and sets *sk.
int choose_streamk(const Operands &o, int cus, bool *sk)
{
    int best = -1;
    double best_cost = 0.0;
    *sk = false;
    for (int i = 0; i < kNumVariants; ++i) {
        const Variant &v = g_table[i];
        if (!v.planned || !variant_allowed(v, o)) continue;
        const double c_dp = plan_cost(g_table, i, o, cus);
        if (best < 0 || c_dp < best_cost) { best = i; best_cost = c_dp; *sk = false; }
        if (!kVariants[i].kern_sk || v.sk_price <= 0.0) continue;
        double c_sk = 0.0;
        const SkGeom g = streamk_geometry(v, o, cus, &c_sk);
        if (g.tiles_sk == 0) continue;
        // With two workgroups per CU, stream-K paid off only where some tiles still ran
        // whole (measured at steady state: 4200^3, 6000^3 and 6000^2 x 4096, 0.6-2 % faster
        // than plain); with every tile shared it ran 12 % slower (2500^2 x 16384, 128 x 128)
        // and 25 % slower (1536^2 x 4096, 64 x 64 x 32) than the plain plans it was priced at.
        if (v.wg_per_cu > 1 && g.tiles_dp == 0) continue;
        if (c_sk < best_cost) { best = i; best_cost = c_sk; *sk = true; }
    }
    return best;
}

int run_variant(int vi, const Operands &o, const float *A, const float *B, float *C,
                void *stream);

// The plan's choice for o (which never picks a whole-tile variant for a shape it does not
// fit).
int run_auto(const Operands &o, const float *A, const float *B, float *C, void *stream)
{
    int cus = 0;
    const int qs = device_cus(&cus);
    if (qs != SGEMM_OK) return qs;
    const int vi = choose_variant(g_table, o, cus);
    return vi < 0 ? SGEMM_ETOO_LARGE : run_variant(vi, o, A, B, C, stream);
}

// The persistent variant: its kernel on the whole-tile part of C (G = min(tiles, CUs)
// workgroups), the right and bottom strips, if any, through the plan. A product without a
// whole tile or with a single K-panel goes to the plan entirely.
int run_persistent(const VariantEntry &e, const Operands &o, const float *A, const float *B,
                   float *C, void *stream)
{
    const int Mi = o.M / e.v.BM * e.v.BM, Ni = o.N / e.v.BN * e.v.BN;
    if (Mi == 0 || Ni == 0 || o.K <= e.v.BK) return run_auto(o, A, B, C, stream);
    Operands oi = o;
    oi.M = Mi;
    oi.N = Ni;
    const GemmArgs p = plain_args(e, oi, A, B, C);
    int cus = 0;
    int st = device_cus(&cus);
    if (st != SGEMM_OK) return st;
    const int64_t tiles = int64_t(p.tiles_m) * p.tiles_n;
    const int64_t grid = std::min<int64_t>(tiles, cus);
    st = launch(o.K % e.v.BK ? e.kern_ktail : e.kern, dim3(unsigned(grid)), dim3(e.threads),
                stream, p);
    if (st != SGEMM_OK) return st;
    if (Ni < o.N) {
        Operands r = o;
        r.N = o.N - Ni;
        st = run_auto(r, A, B + Ni, C + Ni, stream);
        if (st != SGEMM_OK) return st;
    }
    if (Mi < o.M) {
        Operands b = o;
        b.M = o.M - Mi;
        b.N = Ni;
        st = run_auto(b, A + int64_t(Mi) * o.lda, B, C + int64_t(Mi) * o.ldc, stream);
    }
    return st;
}

// One workgroup per tile (or the persistent variant's walk).
int run_variant(int vi, const Operands &o, const float *A, const float *B, float *C,
                void *stream)
{
    const VariantEntry &e = kVariants[vi];
    if (e.persistent) return run_persistent(e, o, A, B, C, stream);
    int cus = 0;
    const int qs = device_cus(&cus);
    if (qs != SGEMM_OK) return qs;
    const GemmArgs p = plain_args(e, o, A, B, C, cus);
    const int64_t grid = int64_t(p.tiles_m) * p.tiles_n;
    if (grid > INT32_MAX) return SGEMM_ETOO_LARGE;
    const int mode = strip_kernel_mode(p);
    const MfmaKernel kern = mode ? e.kern_strip[mode] : e.kern;
    if (!kern) return SGEMM_ELAUNCH;   // the plan gave a strip form the tile lacks
    return launch(kern, dim3(unsigned(grid)), dim3(e.threads), stream, p);
}

// Split-K geometry: K is cut into `splits` ranges of whole BK panels (the last may be
// shorter); returns the number of non-empty ranges and the range length.
void splitk_geometry(int K, int BK, int splits, int *eff, int *k_chunk)
{
    const int panels = (K + BK - 1) / BK;
    const int per = (panels + splits - 1) / splits;
    *k_chunk = per * BK;
    *eff = (K + *k_chunk - 1) / *k_chunk;
}

// Splits chosen automatically: the count the cost model prices lowest, each range at least
// four 64-deep panels long, at most kMaxSplits. A count's price is the hot kernel's (the
// busiest CU's time for the variant the plan takes with that many items per tile) plus
// the reduce's, which reads the partial slices and writes C. Measured at steady state on
// eight under-filled shapes from 128^2 x 65536 to 640^2 x 8192, the prices follow the
// times within a few per cent.
constexpr int kMaxSplits = 32;
constexpr double kReduceUs = 2.0;              // the reduce kernel's launch and latency
constexpr double kReduceBytesPerUs = 4e6;      // the rate at which it streams the slices
int auto_splits(const Operands &o, int cus)
{
    int64_t by_k = o.K / (4 * 64);
    if (by_k > kMaxSplits) by_k = kMaxSplits;
    int best = 1;
    double best_us = -1.0;
    for (int s = 1; s <= by_k || s == 1; ++s) {
        Operands q = o;
        q.splits = s;
        const int vi = choose_variant(g_table, q, cus);
        if (vi < 0) continue;
        double us = plan_cost(g_table, vi, q, cus) / kUnitsPerUs;
        if (s > 1) us += kReduceUs + double(s + 1) * double(o.M) * o.N * 4.0 / kReduceBytesPerUs;
        if (best_us < 0.0 || us < best_us) { best = s; best_us = us; }
    }
    return best;
}

int run_splitk(int splits, const Operands &o0, const float *A, const float *B, float *C,
               float *W, size_t w_bytes, void *stream, int cus)
{
    Operands o = o0;
    o.splits = splits;
    const int vi = choose_variant(g_table, o, cus);
    if (vi < 0) return SGEMM_ETOO_LARGE;
    const VariantEntry &e = kVariants[vi];
    int eff = 0, k_chunk = 0;
    splitk_geometry(o.K, e.v.BK, splits, &eff, &k_chunk);
    const int64_t mn = int64_t(o.M) * o.N;
    if (w_bytes < size_t(eff) * size_t(mn) * 4u) return SGEMM_EINVAL_ARG;
    GemmArgs p{};
    p.A = A; p.B = B; p.C = W;
    p.a_bytes = span_elems(o.M, o.K, o.lda) * 4;
    p.b_bytes = span_elems(o.K, o.N, o.ldb) * 4;
    p.c_bytes = int64_t(eff) * mn * 4;
    p.M = o.M; p.N = o.N; p.K = o.K; p.lda = o.lda; p.ldb = o.ldb; p.ldc = o.N;
    p.tiles_m = (o.M + e.v.BM - 1) / e.v.BM;
    p.tiles_n = (o.N + e.v.BN - 1) / e.v.BN;
    p.splits = eff;
    p.k_chunk = k_chunk;
    p.c_split_stride = mn;
    const int64_t items = int64_t(p.tiles_m) * p.tiles_n * eff;
    if (items > INT32_MAX) return SGEMM_ETOO_LARGE;
    int st = launch(e.kern, dim3(unsigned(items)), dim3(e.threads), stream, p);
    if (st != SGEMM_OK) return st;
    const bool w_vec = (o.N % 4 == 0) && (reinterpret_cast<uintptr_t>(W) % 16 == 0);
    const int c_vec = (o.ldc % 4 == 0) && (reinterpret_cast<uintptr_t>(C) % 16 == 0);
    const int64_t groups = w_vec ? mn / 4 : mn;
    int64_t blocks = (groups + 63) / 64;
    if (blocks > 65536) blocks = 65536;
    const float *Wc = W;
    return w_vec ? launch(k_splitk_reduce<4>, dim3(unsigned(blocks)), dim3(64), stream, o.M, o.N,
                          eff, Wc, mn, C, o.ldc, c_vec)
                 : launch(k_splitk_reduce<1>, dim3(unsigned(blocks)), dim3(64), stream, o.M, o.N,
                          eff, Wc, mn, C, o.ldc, c_vec);
}

// Stream-K with variant vi (the partition may leave nothing to share: then it is the plain
// launch). W holds 2 G partial tiles.
int run_streamk(int vi, const Operands &o, const float *A, const float *B, float *C, float *W,
                size_t w_bytes, void *stream, int cus)
{
    const VariantEntry &e = kVariants[vi];
    GemmArgs p = plain_args(e, o, A, B, C);
    p.sk = streamk_geometry(e.v, o, cus);
    if (p.sk.tiles_sk == 0) return run_variant(vi, o, A, B, C, stream);
    if (w_bytes < streamk_workspace_bytes(e.v, p.sk)) return SGEMM_EINVAL_ARG;
    p.W = W;
    const int64_t grid = int64_t(p.sk.tiles_dp) + p.sk.G;
    if (grid > INT32_MAX) return SGEMM_ETOO_LARGE;
    const int st = launch(e.kern_sk, dim3(unsigned(grid)), dim3(e.threads), stream, p);
    if (st != SGEMM_OK) return st;
    return launch(e.fixup, dim3(unsigned(p.sk.tiles_sk)), dim3(256), stream, p);
}

// The stream-K entry's plan: variant index (or a negative status) and whether it shares
// tiles. variant >= 0 forces stream-K with that variant.
int plan_streamk(int variant, const Operands &o, int cus, bool *sk)
{
    if (variant >= kNumVariants || (variant >= 0 && !kVariants[variant].kern_sk))
        return SGEMM_EINVAL_ARG;
    if (variant >= 0) {
        if (!offsets_fit(kVariants[variant].v, o)) return SGEMM_ETOO_LARGE;
        *sk = streamk_geometry(kVariants[variant].v, o, cus).tiles_sk > 0;
        return variant;
    }
    const int vi = choose_streamk(o, cus, sk);
    return vi < 0 ? SGEMM_ETOO_LARGE : vi;
}

int run_hot(int variant, int M, int N, int K, const float *A, int lda, const float *B, int ldb,
            float *C, int ldc, void *stream)
{
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_OK) return st;
    if (variant >= kNumVariants) return SGEMM_EINVAL_ARG;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (K == 0) return fill_zero(M, N, C, ldc, stream);
    const Operands o = make_operands(M, N, K, lda, ldb, ldc);
    if (variant >= 0 && !offsets_fit(kVariants[variant].v, o)) return SGEMM_ETOO_LARGE;
    int cus = 0;
    const int qs = device_cus(&cus);
    if (qs != SGEMM_OK) return qs;
    const int vi = variant >= 0 ? variant : choose_variant(g_table, o, cus);
    if (vi < 0) return SGEMM_ETOO_LARGE;
    return run_variant(vi, o, A, B, C, stream);
}

}  // namespace
}  // namespace sgemm

// ------------------------------------------------------------------ static scratch --------
// The partial tiles of sgemm_f32_streamk_noalloc live in this file-scope device array
// instead of a caller's workspace. Each GPU the library runs on holds its own copy, for as
// long as the process lives. In host code `scratch` names a host-side stand-in, not the
// device memory: host code takes the array's device address from hipGetSymbolAddress
// (device_scratch below) and passes that to the kernels.
namespace sgemm {
constexpr size_t kScratchBytes = size_t(64) << 20;
}
static __device__ __align__(256) float scratch[sgemm::kScratchBytes / 4];

namespace sgemm {
namespace {

std::mutex g_scratch_mutex;
std::atomic<float *> g_scratch[64];

// Device address of the current device's scratch array, looked up once per device (with
// that device current) and kept; devices past the table's end look it up on every call.
int device_scratch(float **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SGEMM_ELAUNCH;
    float *p = dev < 64 ? g_scratch[dev].load(std::memory_order_acquire) : nullptr;
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        if (dev < 64) p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void *addr = nullptr;
            if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
                return SGEMM_ELAUNCH;
            p = static_cast<float *>(addr);
            if (dev < 64) g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SGEMM_OK;
}

}  // namespace
}  // namespace sgemm

using namespace sgemm;

extern "C" int sgemm_f32(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                         float *C, int ldc, void *stream)
{
    return run_hot(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

extern "C" int sgemm_f32_variant(int variant, int M, int N, int K, const float *A, int lda,
                                 const float *B, int ldb, float *C, int ldc, void *stream)
{
    return run_hot(variant < 0 ? -1 : variant, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

extern "C" size_t sgemm_f32_splitk_workspace_size(int M, int N, int K, int splits)
{
    if (M <= 0 || N <= 0 || K <= 0 || splits < 0 || splits > kMaxSplits) return 0;
    if (splits == 0) {
        int cus = 0;
        if (device_cus(&cus) != SGEMM_OK) return 0;
        splits = auto_splits(make_operands(M, N, K, K, N, N), cus);
    }
    if (splits <= 1) return 0;
    return size_t(splits) * size_t(M) * size_t(N) * 4u;   // one M x N slice per range
}

extern "C" int sgemm_f32_splitk(int M, int N, int K, const float *A, int lda, const float *B,
                                int ldb, float *C, int ldc, int splits, float *workspace,
                                size_t workspace_bytes, void *stream)
{
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_OK) return st;
    if (splits < 0 || splits > kMaxSplits) return SGEMM_EINVAL_ARG;
    if (M == 0 || N == 0) return SGEMM_OK;
    const Operands o = make_operands(M, N, K, lda, ldb, ldc);
    int cus = 0;
    if (splits == 0 && K > 0) {
        const int qs = device_cus(&cus);
        if (qs != SGEMM_OK) return qs;
        splits = auto_splits(o, cus);
    }
    if (splits >= 2 && K > 0) {
        // workspace checks come before any HIP call when the split count is given
        const int64_t w_elems = int64_t(workspace_bytes / 4);
        if (bad_ptr(workspace, w_elems > 0 ? w_elems : 1)) return SGEMM_EINVAL_PTR;
        if (workspace_bytes < size_t(splits) * size_t(M) * size_t(N) * 4u) return SGEMM_EINVAL_ARG;
        if (overlap(workspace, w_elems, A, span_elems(M, K, lda)) ||
            overlap(workspace, w_elems, B, span_elems(K, N, ldb)) ||
            overlap(workspace, w_elems, C, span_elems(M, N, ldc)))
            return SGEMM_EALIAS;
    }
    if (K == 0) return fill_zero(M, N, C, ldc, stream);
    if (splits <= 1) return run_hot(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);
    if (cus == 0) {
        const int qs = device_cus(&cus);
        if (qs != SGEMM_OK) return qs;
    }
    return run_splitk(splits, o, A, B, C, workspace, workspace_bytes, stream, cus);
}

extern "C" size_t sgemm_f32_streamk_workspace_size(int M, int N, int K, int lda, int ldb,
                                                   int ldc, int variant)
{
    if (M <= 0 || N <= 0 || K <= 0 || validate_shape(M, N, K, lda, ldb, ldc) != SGEMM_OK)
        return 0;
    int cus = 0;
    if (device_cus(&cus) != SGEMM_OK) return 0;
    const Operands o = make_operands(M, N, K, lda, ldb, ldc);
    bool sk = false;
    const int vi = plan_streamk(variant < 0 ? -1 : variant, o, cus, &sk);
    if (vi < 0 || !sk) return 0;
    return streamk_workspace_bytes(kVariants[vi].v, streamk_geometry(kVariants[vi].v, o, cus));
}

extern "C" int sgemm_f32_streamk(int M, int N, int K, const float *A, int lda, const float *B,
                                 int ldb, float *C, int ldc, int variant, float *workspace,
                                 size_t workspace_bytes, void *stream)
{
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_OK) return st;
    if (variant >= kNumVariants || (variant >= 0 && !kVariants[variant].kern_sk))
        return SGEMM_EINVAL_ARG;
    // the workspace, when one is given, is checked before any HIP call
    const int64_t w_elems = int64_t(workspace_bytes / 4);
    if (workspace_bytes > 0) {
        if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
            return SGEMM_EINVAL_PTR;
        if (overlap(workspace, w_elems, A, span_elems(M, K, lda)) ||
            overlap(workspace, w_elems, B, span_elems(K, N, ldb)) ||
            overlap(workspace, w_elems, C, span_elems(M, N, ldc)))
            return SGEMM_EALIAS;
    }
    if (M == 0 || N == 0) return SGEMM_OK;
    if (K == 0) return fill_zero(M, N, C, ldc, stream);
    const Operands o = make_operands(M, N, K, lda, ldb, ldc);
    int cus = 0;
    const int qs = device_cus(&cus);
    if (qs != SGEMM_OK) return qs;
    bool sk = false;
    const int vi = plan_streamk(variant < 0 ? -1 : variant, o, cus, &sk);
    if (vi < 0) return vi;
    if (!sk) return run_variant(vi, o, A, B, C, stream);
    return run_streamk(vi, o, A, B, C, workspace, workspace_bytes, stream, cus);
}

extern "C" int sgemm_f32_streamk_noalloc(int M, int N, int K, const float *A, int lda,
                                         const float *B, int ldb, float *C, int ldc, int variant,
                                         void *stream)
{
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_OK) return st;
    if (variant >= kNumVariants || (variant >= 0 && !kVariants[variant].kern_sk))
        return SGEMM_EINVAL_ARG;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (K == 0) return fill_zero(M, N, C, ldc, stream);
    const Operands o = make_operands(M, N, K, lda, ldb, ldc);
    int cus = 0;
    const int qs = device_cus(&cus);
    if (qs != SGEMM_OK) return qs;
    bool sk = false;
    const int vi = plan_streamk(variant < 0 ? -1 : variant, o, cus, &sk);
    if (vi < 0) return vi;
    if (!sk) return run_variant(vi, o, A, B, C, stream);
    const Variant &v = kVariants[vi].v;
    if (streamk_workspace_bytes(v, streamk_geometry(v, o, cus)) > kScratchBytes)
        return SGEMM_ESCRATCH;
    float *W = nullptr;
    const int ss = device_scratch(&W);
    if (ss != SGEMM_OK) return ss;
    return run_streamk(vi, o, A, B, C, W, kScratchBytes, stream, cus);
}

extern "C" size_t sgemm_f32_streamk_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int sgemm_f32_streamk_describe(int M, int N, int K, int variant, int num_cus,
                                          char *buf, int buflen)
{
    if (!buf || buflen <= 0) return SGEMM_EINVAL_ARG;
    if (M < 0 || N < 0 || K < 0) return SGEMM_EINVAL_DIM;
    if (M == 0 || N == 0 || K == 0) return SGEMM_EINVAL_DIM;
    int cus = num_cus;
    if (cus <= 0) {
        const int qs = device_cus(&cus);
        if (qs != SGEMM_OK) return qs;
    }
    const Operands o = make_operands(M, N, K, K, N, N);
    bool sk = false;
    const int vi = plan_streamk(variant < 0 ? -1 : variant, o, cus, &sk);
    if (vi < 0) return vi;
    const Variant &v = kVariants[vi].v;
    double c_sk = 0.0;
    const SkGeom g = streamk_geometry(v, o, cus, &c_sk);
    // the plan's prices, in microseconds at the cost model's unit rate: the cheapest plain
    // plan, and this variant as stream-K (0 when it has no shared tiles)
    double c_plain = -1.0;
    for (int i = 0; i < kNumVariants; ++i) {
        const Variant &w = g_table[i];
        if (!w.planned || !variant_allowed(w, o)) continue;
        const double c = plan_cost(g_table, i, o, cus);
        if (c_plain < 0.0 || c < c_plain) c_plain = c;
    }
    // a plain plan may leave a thin remainder of N to the last tile column (strip_cols)
    const int strip = sk || kVariants[vi].persistent ? 0 : strip_cols(v, o, cus);
    const int rstrip = sk || kVariants[vi].persistent ? 0 : rstrip_rows(v, o, cus);
    // walk every stream-K range with the kernels' own functions: each unit must belong to
    // exactly one range, each shared tile's partial slots must be distinct and written by
    // the segment that the fixup reads them for
    int64_t shared = 0, max_contrib = 0, max_segments = 0;
    bool ok = true;
    if (sk) {
        int next = 0;
        std::vector<int> written(size_t(2) * g.G, -1);
        for (int wg = 0; wg < g.G && ok; ++wg) {
            const int a = sk_start(g, wg), b = sk_start(g, wg + 1);
            ok = a == next && b > a;
            next = b;
            int64_t segs = 0;
            for (int i = a; i < b && ok;) {
                const int t = i / g.panels;
                const int kb = i - t * g.panels;
                const int ke = std::min(g.panels, kb + (b - i));
                if (kb != 0 || ke != g.panels) {
                    const int slot = 2 * wg + (i == a ? 0 : 1);
                    ok = written[size_t(slot)] < 0 && sk_slot(g, wg, t) == slot &&
                         sk_owner(g, i) == wg;
                    written[size_t(slot)] = t;
                }
                i += ke - kb;
                ++segs;
            }
            max_segments = std::max(max_segments, segs);
        }
        ok = ok && next == g.iters;
        for (int t = 0; t < g.tiles_sk && ok; ++t) {
            const int u0 = t * g.panels;
            const int g0 = sk_owner(g, u0), g1 = sk_owner(g, u0 + g.panels - 1);
            if (g0 == g1) continue;
            ++shared;
            max_contrib = std::max<int64_t>(max_contrib, g1 - g0 + 1);
            for (int wg = g0; wg <= g1 && ok; ++wg)
                ok = written[size_t(sk_slot(g, wg, t))] == t &&
                     sk_fixup_slot(g, wg, g0, t) == sk_slot(g, wg, t);
        }
    }
    const int n = snprintf(buf, size_t(buflen),
                           "{\"variant\": %d, \"name\": \"%s\", \"streamk\": %s, "
                           "\"BM\": %d, \"BN\": %d, \"BK\": %d, \"cus\": %d, "
                           "\"G\": %d, \"tiles\": %lld, \"tiles_dp\": %d, "
                           "\"tiles_sk\": %d, \"panels\": %d, \"units\": %lld, "
                           "\"shared_tiles\": %lld, \"max_contributors\": %lld, "
                           "\"max_segments\": %lld, \"workspace_bytes\": %zu, "
                           "\"partition_ok\": %s, \"strip_cols\": %d, "
                           "\"plain_cost_us\": %.2f, \"streamk_cost_us\": %.2f}",
                           vi, v.name, sk ? "true" : "false", v.BM, v.BN, v.BK, cus, g.G,
                           (long long)(int64_t((M - rstrip + v.BM - 1) / v.BM) *
                                       ((N - strip + v.BN - 1) / v.BN)),
                           sk ? g.tiles_dp : 0, sk ? g.tiles_sk : 0, g.panels,
                           (long long)(sk ? g.iters : 0), (long long)shared,
                           (long long)max_contrib, (long long)max_segments,
                           sk ? streamk_workspace_bytes(v, g) : size_t(0), ok ? "true" : "false",
                           strip, c_plain / kUnitsPerUs, g.tiles_sk ? c_sk / kUnitsPerUs : 0.0);
    if (n < 0 || n >= buflen) return SGEMM_EINVAL_ARG;
    return vi;
}

extern "C" int sgemm_f32_naive(int M, int N, int K, const float *A, int lda, const float *B,
                               int ldb, float *C, int ldc, void *stream)
{
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_OK) return st;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (K == 0) return fill_zero(M, N, C, ldc, stream);
    const dim3 block(16, 16);
    const int64_t gy = (int64_t(M) + 15) / 16;
    const dim3 grid(unsigned((N + 15) / 16), unsigned(gy < kMaxGridY ? gy : kMaxGridY));
    return launch(k_sgemm_naive, grid, block, stream, M, N, K, A, lda, B, ldb, C, ldc);
}

extern "C" int sgemm_f32_tiled(int M, int N, int K, const float *A, int lda, const float *B,
                               int ldb, float *C, int ldc, int tile, int pad, void *stream)
{
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_OK) return st;
    if ((tile != 16 && tile != 32) || (pad != 0 && pad != 1)) return SGEMM_EINVAL_ARG;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (K == 0) return fill_zero(M, N, C, ldc, stream);
    const int64_t gy = (int64_t(M) + tile - 1) / tile;
    const dim3 grid(unsigned((N + tile - 1) / tile), unsigned(gy < kMaxGridY ? gy : kMaxGridY));
    const dim3 block(tile, tile);
    if (tile == 16)
        return pad ? launch(k_sgemm_lds_tiled<16, 1>, grid, block, stream, M, N, K, A, lda, B,
                            ldb, C, ldc)
                   : launch(k_sgemm_lds_tiled<16, 0>, grid, block, stream, M, N, K, A, lda, B,
                            ldb, C, ldc);
    return pad ? launch(k_sgemm_lds_tiled<32, 1>, grid, block, stream, M, N, K, A, lda, B, ldb,
                        C, ldc)
               : launch(k_sgemm_lds_tiled<32, 0>, grid, block, stream, M, N, K, A, lda, B, ldb,
                        C, ldc);
}

extern "C" int sgemm_f32_regtiled(int M, int N, int K, const float *A, int lda, const float *B,
                                  int ldb, float *C, int ldc, int tm, int tn, void *stream)
{
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_OK) return st;
    const bool t41 = tm == 4 && tn == 1, t44 = tm == 4 && tn == 4, t88 = tm == 8 && tn == 8;
    if (!t41 && !t44 && !t88) return SGEMM_EINVAL_ARG;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (K == 0) return fill_zero(M, N, C, ldc, stream);
    const int bm = t88 ? 128 : 64, bn = t88 ? 128 : 64;
    const int64_t gy = (int64_t(M) + bm - 1) / bm;
    if (gy > int64_t(kMaxGridY)) return SGEMM_ETOO_LARGE;
    const dim3 grid(unsigned((N + bn - 1) / bn), unsigned(gy));
    if (t41)
        return launch(k_sgemm_regtile<64, 64, 8, 4, 1>, grid, dim3(16 * 64), stream, M, N, K, A,
                      lda, B, ldb, C, ldc);
    if (t44)
        return launch(k_sgemm_regtile<64, 64, 8, 4, 4>, grid, dim3(16 * 16), stream, M, N, K, A,
                      lda, B, ldb, C, ldc);
    return launch(k_sgemm_regtile<128, 128, 8, 8, 8>, grid, dim3(16 * 16), stream, M, N, K, A,
                  lda, B, ldb, C, ldc);
}

extern "C" int sgemm_f32_lds_transpose(int rows, int cols, const float *in, int ldi, float *out,
                                       int ldo, int tile, int pad, void *stream)
{
    if (rows < 0 || cols < 0) return SGEMM_EINVAL_DIM;
    if (ldi < (cols > 1 ? cols : 1) || ldo < (rows > 1 ? rows : 1)) return SGEMM_EINVAL_LD;
    const int64_t si = span_elems(rows, cols, ldi), so = span_elems(cols, rows, ldo);
    if (bad_ptr(in, si) || bad_ptr(out, so)) return SGEMM_EINVAL_PTR;
    if (overlap(out, so, in, si)) return SGEMM_EALIAS;
    if ((tile != 32 && tile != 64) || (pad != 0 && pad != 1)) return SGEMM_EINVAL_ARG;
    if (rows == 0 || cols == 0) return SGEMM_OK;
    const int64_t gy = (int64_t(rows) + tile - 1) / tile;
    if (gy > int64_t(kMaxGridY)) return SGEMM_ETOO_LARGE;
    const dim3 grid(unsigned((cols + tile - 1) / tile), unsigned(gy));
    const dim3 block(tile * tile / 4);
    if (tile == 32)
        return pad ? launch(k_lds_transpose<32, 1>, grid, block, stream, rows, cols, in, ldi, out, ldo)
                   : launch(k_lds_transpose<32, 0>, grid, block, stream, rows, cols, in, ldi, out, ldo);
    return pad ? launch(k_lds_transpose<64, 1>, grid, block, stream, rows, cols, in, ldi, out, ldo)
               : launch(k_lds_transpose<64, 0>, grid, block, stream, rows, cols, in, ldi, out, ldo);
}

extern "C" int sgemm_f32_variant_count(void) { return kNumVariants; }

extern "C" const char *sgemm_f32_variant_name(int variant)
{
    return (variant >= 0 && variant < kNumVariants) ? kVariants[variant].v.name : nullptr;
}

extern "C" int sgemm_f32_variant_info(int variant, char *buf, int buflen)
{
    if (!buf || buflen <= 0 || variant < 0 || variant >= kNumVariants) return SGEMM_EINVAL_ARG;
    const VariantEntry &e = kVariants[variant];
    const Variant &v = e.v;
    const int n = snprintf(buf, size_t(buflen),
                           "{\"variant\": %d, \"name\": \"%s\", \"BM\": %d, \"BN\": %d, "
                           "\"BK\": %d, \"waves\": [%d, %d], \"k_groups\": %d, "
                           "\"threads\": %d, \"mfma\": \"%dx%dx%d\", \"wg_per_cu\": %d, "
                           "\"direct_loads\": %s, \"planned\": %s, \"streamk\": %s, "
                           "\"rate\": %.3f, \"overhead\": %.1f, \"solo\": %.3f, \"latency_us\": %.2f, "
                           "\"kernel\": \"%s\", \"splitk\": %s, \"persistent\": %s, "
                           "\"whole_tiles\": %s, \"strip\": %s, \"strip_cols_max\": %d, "
                           "\"lds_stages\": %d}",
                           variant, v.name, v.BM, v.BN, v.BK, v.wgm, v.wgn, e.kg, e.threads, e.mb,
                           e.mb, e.mb == 32 ? 2 : 4, v.wg_per_cu, v.direct ? "true" : "false",
                           v.planned ? "true" : "false", e.kern_sk ? "true" : "false", v.rate,
                           v.overhead, v.solo, v.latency, e.kernel, v.splitk ? "true" : "false",
                           e.persistent ? "true" : "false", v.whole_tiles ? "true" : "false",
                           v.strip ? "true" : "false", v.strip ? v.strip_cols_max : 0, e.stages);
    if (n < 0 || n >= buflen) return SGEMM_EINVAL_ARG;
    return SGEMM_OK;
}

extern "C" const char *sgemm_f32_status_string(int status)
{
    switch (status) {
    case SGEMM_OK: return "ok";
    case SGEMM_EINVAL_DIM: return "invalid dimension (M, N or K is negative)";
    case SGEMM_EINVAL_LD: return "invalid leading dimension (lda < K, ldb < N or ldc < N)";
    case SGEMM_EINVAL_PTR: return "invalid pointer (NULL or not 4-byte aligned)";
    case SGEMM_EALIAS: return "C overlaps A or B";
    case SGEMM_ELAUNCH: return "HIP runtime error (launch or device query)";
    case SGEMM_EINVAL_ARG: return "invalid option argument";
    case SGEMM_ETOO_LARGE: return "shape too large for the selected kernel";
    case SGEMM_ESCRATCH:
        return "the plan's partial tiles exceed the library's static scratch (64 MiB per GPU)";
    default: return "unknown status";
    }
}

namespace {
// The JSON plan description of variant vi run plainly on o with `cus` compute units (the
// variant's tiles, grid and column strip), for sgemm_f32_plan_describe and
// sgemm_f32_variant_describe. Returns vi, or SGEMM_EINVAL_ARG if buf is too small.
int describe_plan(int vi, const Operands &o, int cus, char *buf, int buflen)
{
    const int M = o.M, N = o.N, K = o.K;
    const Variant &v = kVariants[vi].v;
    const bool pers = kVariants[vi].persistent;
    const int strip = pers ? 0 : strip_cols(v, o, cus);
    const int rstrip = pers ? 0 : rstrip_rows(v, o, cus);
    const int rcols = rstrip ? rstrip_share_cols(v, o) : 0;
    // a whole-tile variant's kernel covers the whole tiles; the edges run as launches of
    // their own, planned for their shapes
    const Operands w = pers ? whole_part(v, o) : o;
    const int edges = pers ? int(w.M < M) + int(w.N < N) : 0;
    const int64_t tm = (int64_t(w.M) - rstrip + v.BM - 1) / v.BM,
                  tn = (int64_t(w.N) - strip + v.BN - 1) / v.BN;
    // workgroups computing rows of the strip: every tile column holding some of its rows
    // (spread), or the last tile column
    const int srows = strip ? strip_form_rows(v, o, cus) : 0;
    const int64_t strip_tiles =
        rstrip ? tn * std::min<int64_t>(tm, (v.BN + rcols - 1) / rcols)
        : !strip ? 0 : srows ? tm * std::min<int64_t>(tn, (v.BM + srows - 1) / srows) : tm;
    // one workgroup per tile, or for the persistent variant one per CU over its tiles
    const int64_t grid = pers ? std::min<int64_t>(tm * tn, cus) : tm * tn;
    // operand bytes the tiles request: every A row panel once per tile column and every
    // B column panel once per tile row (before any cache reuse)
    const int64_t tile_bytes = 4 * (int64_t(w.M) * K * tn + int64_t(K) * w.N * tm);
    const int n = snprintf(buf, size_t(buflen),
                           "{\"variant\": %d, \"name\": \"%s\", \"BM\": %d, \"BN\": %d, "
                           "\"BK\": %d, \"waves\": [%d, %d], \"threads\": %d, \"grid\": %lld, "
                           "\"tiles\": [%lld, %lld], \"cus\": %d, \"wg_per_cu\": %d, "
                           "\"direct_loads\": %s, \"tile_request_bytes\": %lld, "
                           "\"strip_cols\": %d, \"strip_rows\": %d, \"row_strip\": %d, "
                           "\"row_strip_cols\": %d, \"strip_tiles\": %lld, "
                           "\"edge_launches\": %d}",
                           vi, v.name, v.BM, v.BN, v.BK, v.wgm, v.wgn, kVariants[vi].threads,
                           (long long)grid, (long long)tm, (long long)tn, cus, v.wg_per_cu,
                           v.direct ? "true" : "false", (long long)tile_bytes, strip,
                           srows, rstrip, rcols, (long long)strip_tiles, edges);
    if (n < 0 || n >= buflen) return SGEMM_EINVAL_ARG;
    return vi;
}
}  // namespace

// The shape checks and CU count both describe entry points share.
static int describe_args(int M, int N, int K, int lda, int ldb, int ldc, int num_cus,
                         char *buf, int buflen, Operands *o, int *cus)
{
    if (!buf || buflen <= 0) return SGEMM_EINVAL_ARG;
    const int vs = validate_shape(M, N, K, lda, ldb, ldc);
    if (vs != SGEMM_OK) return vs;
    *o = make_operands(M, N, K, lda, ldb, ldc);
    *cus = num_cus;
    if (*cus <= 0) return device_cus(cus);
    return SGEMM_OK;
}

extern "C" int sgemm_f32_plan_describe(int M, int N, int K, const float *A, int lda,
                                       const float *B, int ldb, const float *C, int ldc,
                                       int num_cus, char *buf, int buflen)
{
    (void)A; (void)B; (void)C;
    Operands o{};
    int cus = 0;
    const int st = describe_args(M, N, K, lda, ldb, ldc, num_cus, buf, buflen, &o, &cus);
    if (st != SGEMM_OK) return st;
    const int vi = choose_variant(g_table, o, cus);
    if (vi < 0) return SGEMM_ETOO_LARGE;
    return describe_plan(vi, o, cus, buf, buflen);
}

extern "C" int sgemm_f32_variant_describe(int variant, int M, int N, int K, int lda, int ldb,
                                          int ldc, int num_cus, char *buf, int buflen)
{
    if (variant >= kNumVariants) return SGEMM_EINVAL_ARG;
    Operands o{};
    int cus = 0;
    const int st = describe_args(M, N, K, lda, ldb, ldc, num_cus, buf, buflen, &o, &cus);
    if (st != SGEMM_OK) return st;
    int vi = variant >= 0 ? variant : choose_variant(g_table, o, cus);
    if (vi < 0) return SGEMM_ETOO_LARGE;
    if (!offsets_fit(kVariants[vi].v, o)) return SGEMM_ETOO_LARGE;
    // as run_persistent: without a whole tile or a second K-panel the plan runs it all
    const Variant &fv = kVariants[vi].v;
    if (kVariants[vi].persistent && (M < fv.BM || N < fv.BN || K <= fv.BK)) {
        vi = choose_variant(g_table, o, cus);
        if (vi < 0) return SGEMM_ETOO_LARGE;
    }
    return describe_plan(vi, o, cus, buf, buflen);
}

extern "C" int sgemm_f32_abi_version(void) { return kAbiVersion; }
