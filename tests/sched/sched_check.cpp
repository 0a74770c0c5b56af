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

    // few-token plans: the gate/up kernel routes in its prologue only on a
    // streaming plan with at most kFewSlots slots and 256 experts, reading
    // one score plane, never for the 16-block weights; whole tile columns
    // only with an even number of chunks per K half (the column kernel's
    // loads assume it); and the decode thresholds the kernels were measured
    // on (E = 256, k = 8, F = 2048, d = 8192: 16-feature items at T = 1,
    // whole columns from T = 2)
    long few_cases = 0, fused = 0;
    for (int T = 1; T <= 64; ++T)
        for (int d : {256, 2048, 4096, 6144, 8192})
            for (int E : {8, 16, 64, 200, 256, 512})
                for (int k : {1, 2, 4, 8, 16})
                    for (int F : {256, 384, 1408, 2048}) {
                        if (k > E) continue;
                        Shape s{T, d, E, F, k, 1e-6f};
                        Plan p = make_plan(s);
                        if (p.fuse_route) {
                            if (!p.stream || !p.small_route || s.S() > kFewSlots || E > 256)
                                return fail("prologue routing outside its limits", T, d, E);
                            if (router_splits(s) != 1) return fail("prologue routing on split scores", T, d, E);
                            ++fused;
                        }
                        Plan q = p;
                        nv_plan(s, q);
                        if (q.fuse_route) return fail("16-block plan routes in the prologue", T, d, E);
                        if (p.stream && stream_columns(s) && (d / 128 / 2) % 2 != 0)  // 128-wide K chunks
                            return fail("whole columns with an odd chunk count per K half", T, d, E);
                        ++few_cases;
                    }
    if (fused == 0) return fail("no prologue-routing plan in the sweep", 0, 0, 0);
    for (int T = 1; T <= 8; ++T) {
        Shape s{T, 8192, 256, 2048, 8, 1e-6f};
        if (stream_columns(s) != (T >= 2)) return fail("decode column threshold", T, 8192, 256);
        if (make_plan(s).fuse_route != (T * 8 <= kFewSlots)) return fail("decode prologue routing", T, 8192, 256);
    }
    std::printf("ok %ld (%ld with 64-row tiles; %ld few-token plans, %ld routing in the prologue)\n", cases,
                short_cases, few_cases, fused);
    return 0;
}
