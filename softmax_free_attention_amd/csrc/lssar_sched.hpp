// lssar_sched.hpp -- dispatch order of the forward's query blocks on the
// eight XCDs of an MI355X.
//
// The causal work of query block qb of a head is qb + 1 key tiles, and
// every block of a head reads that head's K and V^T.  Workgroups are handed
// to the XCDs round-robin (workgroup w runs on XCD w % 8) and each XCD has
// its own L2, so the order decides both the load balance and how many heads
// each L2 has to hold:
//
//  * the blocks of a head form pairs {pi, nqb - 1 - pi} of equal work
//    (nqb + 1 tiles; with an odd count the middle block stands alone);
//  * the pairs, numbered head by head, are cut into 8 contiguous slices of
//    (almost) equal count, one per XCD: an XCD holds the K and V^T of about
//    BH / 8 heads instead of all of them;
//  * within its slice an XCD runs the blocks largest first (ties by head), so
//    freed slots take ever smaller blocks and its work ends together;
//  * dispatch index w = 8 l + x is local position l of XCD x; a slice with
//    fewer blocks than the largest leaves its last indices empty (those
//    workgroups exit at once), so the grid has 8 * max_x n_x workgroups.
//
// The functions are plain integer arithmetic.  The prep kernel writes the
// (head, block) of every dispatch index into the workspace (index_of, one
// per block, and the empty indices), so the attention kernel reads its work
// item with one scalar load; the host uses them for the grid size and the
// schedule query of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

namespace lssar {

constexpr int kSchedXcds = 8;

// All counts fit 32 bits: the host rejects shapes with B H (nqb + 1) + 16
// >= 2^31, so G < 2^30 (the kernels then run no 64-bit scalar division).
struct FwdSched {
    int nqb;          // query blocks per head
    int np;           // pairs per head, ceil(nqb / 2)
    int G;            // pairs in all, BH * np

    __host__ __device__ FwdSched(int BH, int nqb_) : nqb(nqb_), np((nqb_ + 1) / 2),
                                                     G(BH * ((nqb_ + 1) / 2)) {}

    // first pair of XCD x's slice: floor(G x / 8) without overflow
    __host__ __device__ int lo(int x) const { return (G >> 3) * x + (((G & 7) * x) >> 3); }

    // Blocks among pairs [a, b) of one head whose size (tiles, qb + 1) is at
    // least S: block pi has size pi + 1 and block nqb - 1 - pi size nqb - pi;
    // the middle block of an odd count belongs to the first side only.
    __host__ __device__ int count_pairs(int a, int b, int S) const
    {
        const int sa = a > S - 1 ? a : S - 1;
        int c = b > sa ? b - sa : 0;
        const int hb = b < nqb - S + 1 ? b : nqb - S + 1;
        c += hb > a ? hb - a : 0;
        if ((nqb & 1) && a <= np - 1 && np - 1 < hb)
            c -= 1;
        return c;
    }

    // The slice [g0, g1) as: first head h0 with pairs [a0, ...), last head
    // h1 with pairs [..., b1), and the whole heads between them.
    struct Span {
        int h0, h1, a0, b1;
    };
    // (a non-empty slice, g0 < g1)
    __host__ __device__ Span span(int g0, int g1) const
    {
        Span sp;
        sp.h0 = g0 / np;
        sp.h1 = (g1 - 1) / np;
        sp.a0 = g0 - sp.h0 * np;
        sp.b1 = g1 - sp.h1 * np;
        return sp;
    }

    // Blocks of the slice of size at least S.
    __host__ __device__ int count_ge(const Span& sp, int S) const
    {
        if (sp.h0 == sp.h1)
            return count_pairs(sp.a0, sp.b1, S);
        return count_pairs(sp.a0, np, S) + count_pairs(0, sp.b1, S) +
               (sp.h1 - sp.h0 - 1) * count_pairs(0, np, S);
    }

    // Blocks of XCD x's slice.
    __host__ __device__ int count(int x) const
    {
        const int g0 = lo(x), g1 = lo(x + 1);
        return g0 < g1 ? count_ge(span(g0, g1), 1) : 0;
    }

    // Workgroups to launch: 8 times the largest slice.
    __host__ __device__ long long grid() const
    {
        int m = 0;
        for (int x = 0; x < kSchedXcds; ++x) {
            const int n = count(x);
            m = n > m ? n : m;
        }
        return (long long)kSchedXcds * m;
    }

    // The dispatch index of block qb of head bh (the inverse of item).
    __host__ __device__ int index_of(int bh, int qb) const
    {
        const int pi = qb < nqb - 1 - qb ? qb : nqb - 1 - qb;   // its pair
        const int g = bh * np + pi;
        // the slice holding pair g: largest x with lo(x) <= g
        int x = (int)(((long long)g * kSchedXcds + kSchedXcds - 1) / G);
        while (x > 0 && lo(x) > g)
            --x;
        while (x + 1 < kSchedXcds && lo(x + 1) <= g)
            ++x;
        const Span sp = span(lo(x), lo(x + 1));
        const int S = qb + 1;
        // blocks of larger size, then the heads before bh holding size S
        int l = count_ge(sp, S + 1);
        if (bh != sp.h0) {
            const bool h0_holds = (S - 1 >= sp.a0 && S - 1 < np) || (nqb - S >= sp.a0 && nqb - S < np);
            l += (h0_holds ? 1 : 0) + (bh - sp.h0 - 1);
        }
        return l * kSchedXcds + x;
    }

    // The (head, block) of dispatch index w; false for an empty index.
    __host__ __device__ bool item(int w, int& bh, int& qb) const
    {
        const int x = w & (kSchedXcds - 1);
        const int l = w / kSchedXcds;
        const int g0 = lo(x), g1 = lo(x + 1);
        if (g0 >= g1)
            return false;
        const Span sp = span(g0, g1);
        if (l >= count_ge(sp, 1))
            return false;
        // largest S with count_ge(S) > l
        int s_lo = 1, s_hi = nqb + 1;
        while (s_hi - s_lo > 1) {
            const int mid = (s_lo + s_hi) / 2;
            if (count_ge(sp, mid) > l)
                s_lo = mid;
            else
                s_hi = mid;
        }
        const int S = s_lo;
        // the r-th head holding a block of size S: h0, the whole heads (each
        // holds every size once), then h1
        int r = l - count_ge(sp, S + 1);
        auto holds = [&](int a, int b) {
            return (S - 1 >= a && S - 1 < b) || (nqb - S >= a && nqb - S < b);
        };
        qb = S - 1;
        if (sp.h0 == sp.h1) {
            bh = sp.h0;
            return true;
        }
        if (holds(sp.a0, np)) {
            if (r == 0) {
                bh = sp.h0;
                return true;
            }
            --r;
        }
        if (r < sp.h1 - sp.h0 - 1) {
            bh = sp.h0 + 1 + r;
            return true;
        }
        bh = sp.h1;
        return true;
    }
};

}  // namespace lssar
