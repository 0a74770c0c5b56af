// Host check of the tiled gate/up kernel's work schedule (csrc/internal.h):
// sched_slot and sched_pos are inverse maps between the sorted items and
// the workgroups of the launch, every workgroup position past the last item
// is empty, the launch is large enough for any tile list of a plan, and the
// XCDs (workgroup % 8) differ by at most one last-round share.  Prints
// "ok <cases>" and returns 0, or reports the first failure and returns 1.
#include "../../mixture_experts_gemm_amd/csrc/internal.h"

#include <cstdio>

using namespace moe;

static int fail(const char *what, long a, long b, long c)
{
    std::printf("FAIL %s %ld %ld %ld\n", what, a, b, c);
    return 1;
}

int main()
{
    long cases = 0;
    for (int ntn = 1; ntn <= 64; ntn += 3)
        for (int nitems = 0; nitems < 9000; nitems += (nitems < 300 ? 1 : 97)) {
            const int run = 2 * ntn;
            const SchedShape q = sched_shape(run, nitems);
            const long grid = 8L * run * ((nitems + 8L * run - 1) / (8L * run));
            long per_x[8] = {0};
            for (int s = 0; s < nitems; ++s) {
                const int b = sched_slot(s, q);
                if (b < 0 || b >= grid) return fail("slot outside the launch", ntn, nitems, s);
                if (sched_pos(b, q) != s) return fail("pos(slot(s)) != s", ntn, nitems, s);
                ++per_x[b & 7];
            }
            long taken = 0;
            for (int b = 0; b < grid; ++b) taken += sched_pos(b, q) >= 0;
            if (taken != nitems) return fail("positions holding an item", ntn, nitems, taken);
            long mx = 0, mn = 1L << 40;
            for (int x = 0; x < 8; ++x) {
                mx = per_x[x] > mx ? per_x[x] : mx;
                mn = per_x[x] < mn ? per_x[x] : mn;
            }
            if (mx - mn > q.lr) return fail("XCD imbalance", ntn, nitems, mx - mn);
            ++cases;
        }
    // the launch and the workspace's schedule hold the largest tile list of
    // every plan (MXFP4 and the 16-block format)
    long short_cases = 0;
    const int Ts[] = {16, 64, 200, 753, 3012, 4096, 16384};
    const int ds[] = {256, 768, 2048, 8192};
    const int Fs[] = {128, 384, 1408, 2048, 4096};
    const int Es[] = {8, 32, 256, 1024};
    const int ks[] = {1, 2, 8};
    for (int T : Ts)
        for (int d : ds)
            for (int F : Fs)
                for (int E : Es)
                    for (int k : ks) {
                        if (k > E) continue;
                        Shape s{T, d, E, F, k, 1e-6f};
                        for (int nv = 0; nv < 2; ++nv) {
                            Plan p = make_plan(s);
                            if (nv) nv_plan(s, p);
                            if (!p.tiled) continue;
                            const long items = max_tiles(s, p.tile_rows) * p.ntn1;
                            if (p.grid1 < items || p.grid1 % (16 * p.ntn1))
                                return fail("launch smaller than the items", T, d, F);
                            if (sched_entries(s) < p.grid1) return fail("schedule entries", T, d, F);
                            if (p.tile_rows == 64) ++short_cases;
                            ++cases;
                        }
                    }
    // the sweep reaches the 64-row tiles of shapes with few rows per expert
    if (short_cases == 0) return fail("no 64-row plan in the sweep", 0, 0, 0);
    std::printf("ok %ld (%ld with 64-row tiles)\n", cases, short_cases);
    return 0;
}
