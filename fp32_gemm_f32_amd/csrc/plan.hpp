// plan.hpp -- the hot kernel's tile variants and the choice among them (host code).
//
// A larger tile reuses each staged element more often but gives fewer workgroups, and
// past some size the reuse no longer pays for the lost parallelism ("Shared Memory
// Tiling", "Choosing a tile size"; "Visual walkthrough - Memory hierarchy", Step 7). On
// gfx950 the parallelism to fill is 256 compute units of 4 SIMDs. The choice below
// estimates, for each variant the operands allow, the time of
//     ceil(tiles / (CUs * workgroups per CU)) rounds x (work of one tile / its rate)
// and takes the smallest.
#pragma once

#include <cstdint>
#include <cstdio>

namespace sgemm {

struct Variant {
    const char *name;
    int BM, BN, BK;
    int wgm, wgn;           // waves along M and N
    bool vec;               // 16-byte loads (needs aligned rows and K % 4 == 0)
    int wg_per_cu;          // workgroups resident per CU (LDS / register bound)
    double rate;            // relative per-CU throughput of one tile's inner loop
};

struct Operands {
    int M, N, K, lda, ldb, ldc;
    bool a16, b16, c16;     // base pointers 16-byte aligned
};

inline bool vec_ok(const Operands &o)
{
    return o.a16 && o.b16 && (o.lda % 4) == 0 && (o.ldb % 4) == 0 && (o.K % 4) == 0;
}

inline bool c_vec_ok(const Operands &o) { return o.c16 && (o.ldc % 4) == 0; }

// Offsets inside one workgroup's A rows and one panel of B must stay below 2^31 bytes.
inline bool offsets_fit(const Variant &v, const Operands &o)
{
    const int64_t lim = int64_t(1) << 31;
    return int64_t(v.BM) * o.lda * 4 + int64_t(o.K) * 4 + 64 < lim &&
           int64_t(v.BK) * o.ldb * 4 + int64_t(v.BN) * 4 + 64 < lim;
}

inline bool variant_allowed(const Variant &v, const Operands &o)
{
    return (!v.vec || vec_ok(o)) && offsets_fit(v, o);
}

inline double variant_cost(const Variant &v, const Operands &o, int cus)
{
    const int64_t tm = (int64_t(o.M) + v.BM - 1) / v.BM;
    const int64_t tn = (int64_t(o.N) + v.BN - 1) / v.BN;
    const int64_t slots = int64_t(cus) * v.wg_per_cu;
    const int64_t rounds = (tm * tn + slots - 1) / slots;
    // one tile's work, in units of BM*BN*K multiply-adds, at the variant's rate; a
    // resident workgroup shares its CU with wg_per_cu - 1 others
    const double tile = double(v.BM) * v.BN * (o.K > 0 ? o.K : 1) * v.wg_per_cu / v.rate;
    return double(rounds) * tile;
}

template <int NV>
inline int choose_variant(const Variant (&table)[NV], const Operands &o, int cus)
{
    int best = -1;
    double best_cost = 0.0;
    for (int i = 0; i < NV; ++i) {
        const Variant &v = table[i];
        if (!variant_allowed(v, o)) continue;
        const double c = variant_cost(v, o, cus) * (v.vec ? 1.0 : 1.15);
        if (best < 0 || c < best_cost) { best = i; best_cost = c; }
    }
    return best;
}

}  // namespace sgemm
