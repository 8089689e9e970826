// plan.hpp -- the hot kernel's tile variants and the choice among them (host code).
//
// A larger tile reuses each staged element more often but gives fewer workgroups, and
// past some size the reuse no longer pays for the lost parallelism ("Shared Memory
// Tiling", "Choosing a tile size"; "Visual walkthrough - Memory hierarchy", Step 7). On
// gfx950 the parallelism to fill is 256 compute units of 4 SIMDs. The choice below
// estimates, for each variant the operands allow, the time of the busiest compute unit,
//     ceil(tiles / CUs) x (work of one tile / the variant's measured rate + per-tile overhead)
//     + the launch's latency,
// and takes the smallest. The overhead (per-tile work that does not scale with K: the
// K-group sums, the epilogue's stores as far as other tiles' MFMAs do not cover them)
// and the latency (once per launch: the first panels' loads, which nothing overlaps, and
// the last tiles' stores) depend on the variant. A variant with two resident workgroups
// per CU runs slightly slower when the busiest CU gets fewer tiles than it can hold at
// once; its rate is scaled by `solo` in that case.
#pragma once

#include <cstdint>
#include <cstdio>

#include "streamk.hpp"

namespace sgemm {

// The stream-K price's default multiplier. The rates above were fitted before the plain
// kernels gained 2-5 % (measured at steady state on eleven shapes from 512^2 x 8192 to 6000^3,
// against the prices the model gives); stream-K forms measured at their price.
constexpr double kStreamkPrice = 1.03;

struct Variant {
    const char *name;
    int BM, BN, BK;
    int wgm, wgn;           // waves along M and N
    int wg_per_cu;          // workgroups resident per CU (LDS / register bound)
    double rate;            // relative per-CU throughput, measured at 8192^3
    double overhead;        // per-tile cost that does not scale with K, in units of K
    double solo;            // rate factor when a CU holds fewer than wg_per_cu tiles
    bool direct;            // direct global -> LDS loads
    bool planned;           // candidate for the automatic choice (else forced use only)
    bool splitk = true;     // candidate for split-K items too
    // computes whole BM x BN tiles only, with more than one K-panel (the persistent
    // kernel): on other shapes it runs on their whole-tile part and the right and bottom
    // edges go to the plan, as launches of their own
    bool whole_tiles = false;
    // a remainder of N past the last whole tile column may be computed by the tiles beside
    // the MFMAs, on the vector ALUs (the kernel's column strip): one column in either form,
    // up to strip_cols_max columns spread over the tiles of each row
    bool strip = false;
    int strip_cols_max = 1;
    // multiplier on the stream-K price (streamk_cost) of this variant's stream-K form; 0: the
    // form is not planned (it still runs when forced)
    double sk_price = kStreamkPrice;
    // the launch's fixed time, in microseconds (see above)
    double latency = 0.0;
};

struct Operands {
    int M, N, K, lda, ldb, ldc;
    int splits = 1;         // split-K: each tile's K range is cut into this many items
};

// Buffer offsets inside one workgroup's rows of A and C and one panel of B must stay
// below 2^31 bytes.
inline bool offsets_fit(const Variant &v, const Operands &o)
{
    const int64_t lim = int64_t(1) << 31;
    return int64_t(v.BM) * o.lda * 4 + int64_t(o.K) * 4 + 64 < lim &&
           int64_t(v.BK) * o.ldb * 4 + int64_t(v.BN) * 4 + 64 < lim &&
           int64_t(v.BM) * o.ldc * 4 + int64_t(v.BN) * 4 + 64 < lim;
}

// Most columns a strip may hold (the kernels' kStripCols).
constexpr int kStripColsMax = 4;

// Rows of the strip each tile computes when the strip's rows are spread over the tiles of
// a row: ceil(BM / whole tile columns), if one K-group's threads hold a (row, 16-byte
// chunk of a panel row) pair each (64 wgm wgn threads, BK / 4 chunks per row); else 0,
// and the tiles of the last tile column compute the whole strip.
inline int strip_spread_rows(const Variant &v, const Operands &o)
{
    const int tn = o.N / v.BN;
    if (tn <= 0) return 0;
    const int rows = (v.BM + tn - 1) / tn;
    return rows * (v.BK / 4) <= 64 * v.wgm * v.wgn ? rows : 0;
}

// Columns variant v could leave to the strip for o: N mod BN when that is 1 to the
// variant's strip_cols_max (past one column only where the spread form can take the
// strip's rows) and N holds at least one whole tile column, else 0 (the strip's B values
// of a panel lie inside the panel's rows of B, so the offsets bound of offsets_fit covers
// them). Whether the plan uses the strip is a choice priced by variant_cost (strip_cols).
inline int strip_eligible(const Variant &v, const Operands &o)
{
    if (!v.strip || o.splits != 1 || o.N <= v.BN) return 0;
    const int r = o.N % v.BN;
    if (r < 1 || r > v.strip_cols_max || r > kStripColsMax) return 0;
    return r == 1 || strip_spread_rows(v, o) > 0 ? r : 0;
}

// Strip columns the kernel loads and multiplies per panel for a strip of r columns: one,
// two or four (three take four, the last one zero).
inline int strip_load_cols(int r) { return r <= 1 ? 1 : r == 2 ? 2 : 4; }

// A whole-tile variant (the persistent kernel) also needs rows of C that start on 32-byte
// boundaries (ldc a multiple of 8): it stores C as 4-byte lane stores from the
// accumulators, 128 bytes of a row per 32 lanes, and on rows off those boundaries they cost
// it far more than the other tiles' 16-byte stores. Measured at 16384^2 x 64 against the
// 128 x 256 x 16 tile (steady state): ldc = 16384 0.92x its time, 16392 0.97x, 16388 1.18x,
// 16385 1.48x; rows of A or B off 16-byte boundaries cost neither kernel (0.92-0.93x).
inline bool variant_allowed(const Variant &v, const Operands &o)
{
    if (v.whole_tiles &&
        (o.M < v.BM || o.N < v.BN || o.K <= v.BK || o.splits != 1 || o.ldc % 8 != 0))
        return false;
    return offsets_fit(v, o);
}

// The whole-tile part of o for a whole-tile variant: M and N rounded down to its tiles.
inline Operands whole_part(const Variant &v, const Operands &o)
{
    Operands w = o;
    w.M = o.M / v.BM * v.BM;
    w.N = o.N / v.BN * v.BN;
    return w;
}

// Cost units: one multiply-add on one CU at rate 1 (140 TFLOP/s over 256 CUs).
constexpr double kUnitsPerUs = 140e12 / 2 / 256 * 1e-6;
// The strip's products run on the vector ALUs between the MFMAs of the tiles that compute
// it. Spread over the tiles of each row, every tile runs about 1-5 % longer, in proportion
// to its panels (each loads the panel's strip values); in the last tile column alone, those
// tiles run 7-11 % longer and the others not at all (measured at steady state against the
// same shapes without the column: 1023 x 1025 x 1027 and 1024 x 1025 x 1024 with 64 x 64
// tiles of 64- and 32-deep panels, 2048 x 2049 x 2048, 4096 x 4097 x 4096 and
// 8192 x 8193 x 1024 with 128 x 128 tiles). So the spread form wins while each CU runs
// few tiles, the last-column form once the strip tiles are a small share of many rounds
// (8192 x 8193 x 1024: 64 strip tiles among 4096). kStripSpreadShare is the share with
// 64-deep panels; where two workgroups share each CU, the other one's MFMAs cover half of
// it (128 x 128 tiles: 3.3 % at 2048 x 2049 x 2048, one tile per CU; 0.7 % at
// 4096 x 4097 x 4096, four).
constexpr double kStripSpreadShare = 0.02;
constexpr double kStripColumnShare = 0.10;
inline double strip_spread_share(const Variant &v, const Operands &o, int cus)
{
    const int64_t tm = (int64_t(o.M) + v.BM - 1) / v.BM;
    const int64_t per_cu = (tm * (o.N / v.BN) + cus - 1) / cus;
    // each column adds a 16-byte read and four FMAs per thread and panel to the A chunk's
    // read (one column: two reads)
    const int sc = strip_load_cols(strip_eligible(v, o));
    const double share = kStripSpreadShare * 64.0 / v.BK * (1.0 + sc) / 2.0;
    return per_cu >= v.wg_per_cu ? share / v.wg_per_cu : share;
}

// Busiest-CU estimate for variant v with tn tile columns (and tm tile rows; by default
// every row of M in a tile), in multiply-adds at rate 1.
inline double tiles_cost(const Variant &v, const Operands &o, int cus, int64_t tn,
                         int64_t tm = -1)
{
    if (tm < 0) tm = (int64_t(o.M) + v.BM - 1) / v.BM;
    // the busiest CU runs ceil(tiles / CUs) tiles; each is BM*BN*K multiply-adds at the
    // variant's measured relative rate plus the variant's per-tile overhead
    int64_t per_cu = (tm * tn * o.splits + cus - 1) / cus;
    // the persistent kernel walks its tiles in pairs: an odd count ends on an empty tile
    if (v.whole_tiles) per_cu += per_cu & 1;
    const double k = o.K > 0 ? double(o.K) / o.splits : 1;
    const double rate = per_cu >= v.wg_per_cu ? v.rate : v.rate * v.solo;
    return double(per_cu) * double(v.BM) * v.BN * (k / rate + v.overhead);
}

// The busiest CU's share of the strip when the last tile column computes it: one heavier
// tile per round of strip tiles, over its per_cu tiles.
inline double strip_column_share(const Variant &v, const Operands &o, int cus)
{
    const int64_t tm = (int64_t(o.M) + v.BM - 1) / v.BM;
    const int64_t per_cu = (tm * (o.N / v.BN) + cus - 1) / cus;
    return kStripColumnShare * double((tm + cus - 1) / cus) / double(per_cu > 0 ? per_cu : 1);
}

// Rows per tile of the strip's form for o: strip_spread_rows where spreading the rows is
// priced below the last-column form or the strip holds more than one column, else 0 (the
// last tile column computes them).
inline int strip_form_rows(const Variant &v, const Operands &o, int cus)
{
    const int rows = strip_spread_rows(v, o);
    if (rows > 0 && strip_eligible(v, o) > 1) return rows;
    return rows > 0 && strip_spread_share(v, o, cus) < strip_column_share(v, o, cus) ? rows : 0;
}

// The same with a column strip of the last N mod BN columns (strip_eligible), in the form
// strip_form_rows picks.
inline double strip_cost(const Variant &v, const Operands &o, int cus)
{
    const double share = strip_form_rows(v, o, cus) > 0 ? strip_spread_share(v, o, cus)
                                                        : strip_column_share(v, o, cus);
    return tiles_cost(v, o, cus, o.N / v.BN) * (1.0 + share);
}

// Row strip, the column strip's spread form mirrored: the rows of M past the last whole
// tile row computed by the tiles of each tile column, tile row t taking columns
// [t c, (t + 1) c) of its tile column's share, c = ceil(BN / whole tile rows), if one
// K-group's threads hold a (column, 16-byte chunk of a panel row) pair each; else 0.
inline int rstrip_share_cols(const Variant &v, const Operands &o)
{
    const int tm = o.M / v.BM;
    if (tm <= 0) return 0;
    const int cols = (v.BN + tm - 1) / tm;
    return cols * (v.BK / 4) <= 64 * v.wgm * v.wgn ? cols : 0;
}

// Rows variant v could leave to a row strip for o: M mod BM when that is 1 to the
// variant's strip_cols_max and M holds at least one whole tile row, else 0.
inline int rstrip_eligible(const Variant &v, const Operands &o)
{
    if (!v.strip || o.splits != 1 || o.M <= v.BM) return 0;
    const int r = o.M % v.BM;
    if (r < 1 || r > v.strip_cols_max || r > kStripColsMax) return 0;
    return rstrip_share_cols(v, o) > 0 ? r : 0;
}

// The row strip's share of a tile's time. Per panel every thread reads four B values of
// one column, BN floats apart in LDS: with 64-float rows the lanes of one column hit one
// bank, so the reads serialise over the panel's BK / 4 chunks, and the share grows with BK
// rather than shrinking (measured at steady state against the same tiles without the rows:
// 1025 x 1024 x 1024, 64 x 64 x 64 tiles 11.8 %, 64 x 64 x 32 tiles 5.7 %; two rows 14.5 and
// 7.7 %, four 19.1 and 15.3 %). Halved where another workgroup's MFMAs cover it.
constexpr double kRowStripShare = 0.10;
inline double rstrip_cost(const Variant &v, const Operands &o, int cus)
{
    const int64_t tm = o.M / v.BM, tn = (int64_t(o.N) + v.BN - 1) / v.BN;
    const int64_t per_cu = (tm * tn + cus - 1) / cus;
    const int sc = strip_load_cols(rstrip_eligible(v, o));
    double share = kRowStripShare * v.BK / 64.0 * (3.0 + sc) / 4.0;
    if (per_cu >= v.wg_per_cu) share /= v.wg_per_cu;
    return tiles_cost(v, o, cus, tn, tm) * (1.0 + share);
}

// Rows variant v leaves to a row strip for o: those of rstrip_eligible when the strip is
// priced below a last row of masked tiles and below a column strip, else 0.
inline int rstrip_rows(const Variant &v, const Operands &o, int cus)
{
    const int r = rstrip_eligible(v, o);
    if (r == 0) return 0;
    const double c = rstrip_cost(v, o, cus);
    if (!(c < tiles_cost(v, o, cus, (int64_t(o.N) + v.BN - 1) / v.BN))) return 0;
    if (strip_eligible(v, o) > 0 && !(c < strip_cost(v, o, cus))) return 0;
    return r;
}

// Columns variant v leaves to the strip for o: those of strip_eligible when the strip is
// priced below a last column of masked tiles and the plan takes no row strip, else 0.
inline int strip_cols(const Variant &v, const Operands &o, int cus)
{
    const int r = strip_eligible(v, o);
    if (r == 0) return 0;
    const int64_t tn_all = (int64_t(o.N) + v.BN - 1) / v.BN;
    if (!(strip_cost(v, o, cus) < tiles_cost(v, o, cus, tn_all))) return 0;
    return rstrip_rows(v, o, cus) > 0 ? 0 : r;
}

inline double variant_cost(const Variant &v, const Operands &o, int cus)
{
    if (rstrip_rows(v, o, cus) > 0) return rstrip_cost(v, o, cus);
    if (strip_cols(v, o, cus) > 0) return strip_cost(v, o, cus);
    return tiles_cost(v, o, cus, (int64_t(o.N) + v.BN - 1) / v.BN);
}

// Stream-K's fixed price: the fixup kernel's launch and latency, in microseconds, the rate
// at which partial tiles are written and read back, in bytes per microsecond, and the
// latency of each batch of partial-tile loads the fixup waits for in turn.
constexpr double kFixupUs = 3.0;
constexpr double kPartialBytesPerUs = 4e6;
constexpr double kFixupBatchUs = 0.7;

// Busiest-CU estimate for variant v run as stream-K with partition g (streamk.hpp), in the
// units of variant_cost: every CU gets the same share of the K-panel units, plus its
// plain tiles, plus a per-segment overhead (each stream-K workgroup starts one segment
// more than the whole tiles its range holds), plus the fixup and the partial tiles'
// round trip through memory.
inline double streamk_cost(const Variant &v, const Operands &o, int cus, const SkGeom &g,
                           size_t ws_bytes)
{
    const double tile = double(v.BM) * v.BN;
    const double dp_tiles = double(g.tiles_dp) / cus;                 // per CU
    const double sk_k = double(g.iters) * v.BK / cus;                  // K per CU, summed
    const double segs = double(v.wg_per_cu) * (double(g.iters) / g.G / g.panels + 1.0);
    const double work = tile * ((dp_tiles * o.K + sk_k) / v.rate + (dp_tiles + segs) * v.overhead);
    // contributors of the most shared tile: its units over a range's length, plus one
    const double contrib = double(g.panels) * g.G / double(g.iters) + 2.0;
    const double batches = contrib / kFixupBatch + 1.0;
    return (work + (v.latency + kFixupUs + batches * kFixupBatchUs +
                    double(ws_bytes) / kPartialBytesPerUs) *
                       kUnitsPerUs) *
           (v.sk_price > 0.0 ? v.sk_price : 1.0);
}

// The launch and latency of one more kernel on the stream, in microseconds: a whole-tile
// variant runs a ragged product's right and bottom edges as kernels of their own after its
// own, in stream order.
constexpr double kEdgeLaunchUs = 4.0;

// Busiest-CU estimate of the cheapest plan for o among the planned variants that take any
// shape (the edges of a whole-tile variant's product), plus one launch.
template <int NV>
inline double edge_cost(const Variant (&table)[NV], const Operands &o, int cus)
{
    double best = -1.0;
    for (int i = 0; i < NV; ++i) {
        const Variant &v = table[i];
        if (!v.planned || v.whole_tiles || !variant_allowed(v, o)) continue;
        const double c = variant_cost(v, o, cus);
        if (best < 0.0 || c < best) best = c;
    }
    return (best < 0.0 ? 0.0 : best) + kEdgeLaunchUs * kUnitsPerUs;
}

// Price of running variant i of the table on o as the plain entry does: variant_cost, or for
// a whole-tile variant its whole-tile part plus the right edge (all rows, the columns past
// the last whole tile column) and the bottom edge (the rows past the last whole tile row,
// the whole tile columns), each priced as the plan would run it; plus the variant's latency.
template <int NV>
inline double plan_cost(const Variant (&table)[NV], int i, const Operands &o, int cus)
{
    const Variant &v = table[i];
    const double latency = v.latency * kUnitsPerUs;
    if (!v.whole_tiles) return variant_cost(v, o, cus) + latency;
    // its panels run whole: a K that is not a multiple of BK costs the last one in full
    // (16384^2 x 65: 1.05x the 128 x 256 x 16 tile's time, against 0.92x at K = 64)
    Operands w = whole_part(v, o);
    w.K = (o.K + v.BK - 1) / v.BK * v.BK;
    double c = variant_cost(v, w, cus);
    if (w.N < o.N) {
        Operands r = o;
        r.N = o.N - w.N;
        c += edge_cost(table, r, cus);
    }
    if (w.M < o.M) {
        Operands b = o;
        b.M = o.M - w.M;
        b.N = w.N;
        c += edge_cost(table, b, cus);
    }
    return c + latency;
}

template <int NV>
inline int choose_variant(const Variant (&table)[NV], const Operands &o, int cus)
{
    int best = -1;
    double best_cost = 0.0;
    for (int i = 0; i < NV; ++i) {
        const Variant &v = table[i];
        if (!v.planned || !variant_allowed(v, o) || (o.splits > 1 && !v.splitk)) continue;
        const double c = plan_cost(table, i, o, cus);
        if (best < 0 || c < best_cost) { best = i; best_cost = c; }
    }
    return best;
}

}  // namespace sgemm
