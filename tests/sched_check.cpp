// Host check of the persistent kernel's work lists (attn_sched.h), built by test_item_schedule.py:
//   sched_check G BH num_qtiles
// prints "name value" lines: how often each work item is assigned (min and max over items), whether the
// head-major lists are in use, how many items of a head sit on another XCD than the head's, and the
// causal tile steps per workgroup (min and max over workgroups).
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "attn_sched.h"

int main(int argc, char **argv)
{
    if (argc != 4) return 2;
    const int G = atoi(argv[1]), BH = atoi(argv[2]), num_qtiles = atoi(argv[3]);
    const int num_items = BH * num_qtiles;
    const bool by_heads = tsd::qb2_heads_schedule(G, BH, num_qtiles);
    std::vector<int> seen(num_items, 0);
    std::vector<long long> steps(G, 0);
    long long off_xcd = 0, bad_index = 0;
    for (int w = 0; w < G; ++w) {
        for (int j = 0; j < num_items + 1; ++j) {  // a list never holds more than every item
            int bh, qt;
            if (by_heads) {
                if (!tsd::qb2_sched_heads(w, j, G, BH, num_qtiles, bh, qt)) break;
            } else {
                const int p = tsd::qb2_sched(w, j, G, num_items);
                if (p >= num_items) break;
                qt = p / BH;
                bh = p % BH;
            }
            if (bh < 0 || bh >= BH || qt < 0 || qt >= num_qtiles) {
                ++bad_index;
                continue;
            }
            ++seen[qt * BH + bh];
            if (by_heads && bh % 8 != w % 8) ++off_xcd;
            steps[w] += 4LL * (num_qtiles - qt);  // causal: block qt covers rows up to (num_qtiles - qt) * 256
        }
    }
    int smin = 1 << 30, smax = 0;
    for (int c : seen) {
        smin = c < smin ? c : smin;
        smax = c > smax ? c : smax;
    }
    long long tmin = 1LL << 60, tmax = 0;
    for (long long t : steps) {
        tmin = t < tmin ? t : tmin;
        tmax = t > tmax ? t : tmax;
    }
    printf("by_heads %d\nassigned_min %d\nassigned_max %d\nbad_index %lld\noff_xcd %lld\nsteps_min %lld\nsteps_max %lld\n",
           by_heads ? 1 : 0, smin, smax, bad_index, off_xcd, tmin, tmax);
    return 0;
}
