// Host-side check of the local kernel's work-item order (local_work_item in
// kernels.h): for many geometries, every workgroup index maps to exactly one
// work item, in natural and in longest-first order, and longest-first order
// keeps each XCD's share of items.  Built and run by tests/test_abi.py.
#include <cstdio>
#include <vector>

#include "kernels.h"

using namespace rehyat;

int main() {
    int bad = 0, cases = 0;
    for (int BH : {1, 2, 12, 24})
        for (int F : {1, 3, 7, 21, 25})
            for (int Tc : {1, 3, 7})
                for (int To : {0, 1, 4})
                    for (int T : {1, 3, 19})
                        for (int lpt : {0, 1}) {
                            LocalParams p{};
                            p.BH = BH; p.F = F; p.Tc = Tc; p.To = To; p.HW = 1560;
                            p.n_chunks = (F + Tc - 1) / Tc; p.tiles_per_chunk = T; p.lpt_order = lpt;
                            const int n = BH * p.n_chunks * T;
                            std::vector<int> seen(n, 0);
                            for (int b = 0; b < n; ++b) {
                                const int it = local_work_item(p, b, n, 128);
                                if (it < 0 || it >= n) { ++bad; continue; }
                                ++seen[it];
                                // same XCD share as the natural order
                                LocalParams q = p; q.lpt_order = 0;
                                const int per = n / 8, tail = n % 8, x = b % 8;
                                const int s = x < tail ? x * (per + 1) : tail * (per + 1) + (x - tail) * per;
                                const int e = s + per + (x < tail ? 1 : 0);
                                if (it < s || it >= e) ++bad;
                                (void)q;
                            }
                            for (int i = 0; i < n; ++i) bad += seen[i] != 1;
                            ++cases;
                        }
    printf("%d geometries, %d violations\n", cases, bad);
    return bad != 0;
}
