// Host check of the attention kernel's work order (work_order.h): for every
// shape given, the queue slots work_plan sizes decode (work_item) to each
// (query-block pair, query head) of the layer exactly once, with the head in
// its KV group and every index in range.  Built and run by test_work_order.py.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "work_order.h"

using namespace crisp;

static int check(int n, int hq, int hkv)
{
    const int nb = (n + kB - 1) / kB, G = hq / hkv, npairs = (nb + 1) / 2;
    const WorkPlan w = work_plan(n, hq, hkv);
    if (w.run < 1 || w.per_xcd < 0) return 1;
    if (w.pair_major != ((long long)n * kD * 4 <= kPairMajorKvBytes ? 1 : 0)) return 2;
    std::vector<int> seen((size_t)npairs * hq, 0);
    long long valid = 0;
    for (long long b = 0; b < 8LL * w.per_xcd; ++b) {
        WorkItem it;
        if (!work_item((int)b, nb, hkv, G, w.run, w.pair_major != 0, &it)) continue;
        if (it.pair < 0 || it.pair >= npairs || it.h < 0 || it.h >= hq) return 3;
        if (it.g < 0 || it.g >= hkv || it.h / G != it.g) return 4;
        if (seen[(size_t)it.pair * hq + it.h]++) return 5;
        ++valid;
    }
    if (valid != (long long)npairs * hq) return 6;
    return 0;
}

int main(int argc, char** argv)
{
    // argv: triples n hq hkv
    int failures = 0, shapes = 0;
    for (int i = 1; i + 2 < argc; i += 3) {
        const int n = atoi(argv[i]), hq = atoi(argv[i + 1]), hkv = atoi(argv[i + 2]);
        const int rc = check(n, hq, hkv);
        ++shapes;
        if (rc) {
            printf("FAIL n=%d hq=%d hkv=%d code=%d\n", n, hq, hkv, rc);
            ++failures;
        }
    }
    printf("%d shapes, %d failures\n", shapes, failures);
    return failures ? 1 : 0;
}
