// Host driver for the router's threshold search (select_threshold in
// route_core.h, compiled here for the CPU). Reads cases from stdin, one per
// line: "k n key_0 ... key_{n-1}" (n > k >= 1, keys as unsigned integers),
// and prints the threshold T of each case on its own line. The test that
// runs it checks the set that T selects against a sort.
#include "route_core.h"

#include <cstdio>
#include <vector>

int main()
{
    int k, n;
    while (std::scanf("%d %d", &k, &n) == 2) {
        std::vector<uint32_t> keys(n);
        uint32_t mx = 0u, mn = 0xFFFFFFFFu;
        for (int i = 0; i < n; ++i) {
            unsigned v;
            if (std::scanf("%u", &v) != 1) return 2;
            keys[i] = v;
            mx = keys[i] > mx ? keys[i] : mx;
            mn = keys[i] < mn ? keys[i] : mn;
        }
        const uint32_t T = hga::select_threshold(mx, mn, k, [&](uint32_t cand) {
            int c = 0;
            for (uint32_t x : keys) c += x >= cand;
            return c;
        });
        std::printf("%u\n", T);
    }
    return 0;
}
