// Host-thread model of the work protocol of the fused decode kernel
// (fused.hip): a ticket counter hands out scan items, then attention items; the
// last scan arrival of a unit selects and raises the unit's ready word; an
// attention item waits (bounded) for that word, attends, and the last attention
// arrival merges.  Workgroups are modelled as groups of threads ("waves") that
// share an item slot and meet at barriers, as the kernel's waves meet at
// __syncthreads.  Nothing here runs on a GPU; the model checks the protocol's
// logic under random timing:
//
//   * every wave of a workgroup works on the same item (an item slot reused
//     before every wave has read it would split a workgroup across two items);
//   * every run ends (barriers have a deadline; a missed one is reported as a
//     hang instead of hanging the test);
//   * an attention item never reads a selection of an earlier call;
//   * a unit's output is either exact or NaN (when one of its waits was abandoned);
//   * the control words are consistent after every call.
//
// Variants (argv[1]):
//   shipped     ticket prefetch, two barriers around the item slot, epoch flags
//   noprefetch  a ticket claimed at the top of each iteration, two barriers
//   onebarrier  a ticket claimed at the top, ONE barrier around the item slot
//   flags01     the shipped loop with 0/1 ready flags reset by the last split
// argv[2] = trials, argv[3] = seed, argv[4] = spin limit (polls) for the first
// call of each trial (the second call always uses a long limit).
// Output: one line "hang=H mismatch=M stale=S wrong=W nan_units=N timeouts=T".
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

namespace {

enum Variant { kShipped, kNoPrefetch, kOneBarrier, kFlags01 };

struct Barrier {  // reusable barrier with a deadline
    std::mutex m;
    std::condition_variable cv;
    int n, waiting = 0;
    long gen = 0;
    explicit Barrier(int n_) : n(n_) {}
    bool wait() {  // false on a missed deadline (a hang)
        std::unique_lock<std::mutex> lk(m);
        const long g = gen;
        if (++waiting == n) {
            waiting = 0;
            ++gen;
            cv.notify_all();
            return true;
        }
        return cv.wait_for(lk, std::chrono::milliseconds(400), [&] { return gen != g; });
    }
};

struct Call {
    int U, C, S, W, NW, spin_limit;
    std::vector<int> nch;  // scan chunks of each unit (<= C); items j >= nch are skipped
};

struct Shared {
    std::atomic<int> ctl[4];  // ticket, finished, abandoned, epoch
    std::vector<std::atomic<int>> scan_arrive, ready, att_arrive;
    std::vector<std::atomic<int>> sel;       // the "selection": the call number that wrote it
    std::vector<std::atomic<int>> part;      // per (unit, split): call number attended, or -1 (NaN)
    std::vector<std::atomic<int>> out;       // per unit: call number merged, or -1 (NaN)
    std::atomic<int> hang{0}, mismatch{0}, stale{0};
    explicit Shared(int U, int S)
        : scan_arrive(U), ready(U), att_arrive(U), sel(U), part((size_t)U * S), out(U) {
        for (auto& c : ctl) c = 0;
        for (int u = 0; u < U; ++u) scan_arrive[u] = ready[u] = att_arrive[u] = sel[u] = out[u] = 0;
        for (auto& p : part) p = 0;
    }
};

void jitter(std::mt19937& rng, int max_us) {
    const int us = std::uniform_int_distribution<int>(0, max_us)(rng);
    if (us > max_us / 2) std::this_thread::sleep_for(std::chrono::microseconds(us - max_us / 2));
}

// One workgroup: NW threads; thread 0 plays the kernel's tid 0.
void workgroup(Variant var, const Call& c, Shared& sh, int call_no, int wg, unsigned seed) {
    const int n_items = c.U * (c.C + c.S);
    Barrier bar(c.NW);
    int sh_item = -1, sh_last = 0;
    std::vector<int> seen(c.NW, -2);
    const int epoch = sh.ctl[3].load();
    const int raised = epoch + 1;
    auto wave = [&](int w) {
        std::mt19937 rng(seed * 7919u + wg * 131u + w);
        int next = 0;
        if (w == 0 && var == kShipped) next = sh.ctl[0].fetch_add(1);
        if (var == kFlags01 && w == 0) next = sh.ctl[0].fetch_add(1);
        for (;;) {
            if (w == 0) {
                sh_item = (var == kShipped || var == kFlags01) ? next : sh.ctl[0].fetch_add(1);
            }
            if (!bar.wait()) { sh.hang = 1; return; }
            jitter(rng, 40);
            const int item = sh_item;
            seen[w] = item;
            if (var != kOneBarrier) {
                if (!bar.wait()) { sh.hang = 1; return; }
            }
            if (item >= n_items) break;
            if (w == 0 && (var == kShipped || var == kFlags01)) next = sh.ctl[0].fetch_add(1);
            const int sc = c.U * c.C;
            const bool scan = item < sc;
            const int u = scan ? item / c.C : (item - sc) / c.S;
            const int j = scan ? item % c.C : (item - sc) % c.S;
            if (scan) {
                if (j >= c.nch[u]) continue;  // past the row: skipped before any barrier, as in the kernel
                jitter(rng, 60);               // the block scores
                if (!bar.wait()) { sh.hang = 1; return; }
                if (seen[w] != seen[0]) sh.mismatch = 1;
                if (w == 0) sh_last = sh.scan_arrive[u].fetch_add(1) == c.nch[u] - 1;
                if (!bar.wait()) { sh.hang = 1; return; }
                if (!sh_last) continue;
                if (w == 0) sh.scan_arrive[u] = 0;
                jitter(rng, 200);              // the selection
                if (w == 0) sh.sel[u] = call_no;
                if (!bar.wait()) { sh.hang = 1; return; }
                if (w == 0) sh.ready[u].store(var == kFlags01 ? 1 : raised, std::memory_order_release);
            } else {
                if (w == 0) {
                    int polls = 0;
                    bool ok = true;
                    const int want = var == kFlags01 ? 1 : raised;
                    while (sh.ready[u].load(std::memory_order_acquire) != want) {
                        std::this_thread::sleep_for(std::chrono::microseconds(2));
                        if (++polls >= c.spin_limit) {
                            sh.ctl[2].fetch_add(1);
                            ok = false;
                            break;
                        }
                    }
                    sh_last = ok;
                }
                if (!bar.wait()) { sh.hang = 1; return; }
                if (seen[w] != seen[0]) sh.mismatch = 1;
                const bool ok = sh_last;
                if (!bar.wait()) { sh.hang = 1; return; }
                if (w == 0) {
                    if (ok) {
                        // attend: reads the selection; it must be this call's
                        if (sh.sel[u].load() != call_no) sh.stale = 1;
                        sh.part[(size_t)u * c.S + j] = call_no;
                    } else {
                        sh.part[(size_t)u * c.S + j] = -1;  // NaN partial
                    }
                }
                jitter(rng, 60);
                if (!bar.wait()) { sh.hang = 1; return; }
                if (w == 0) sh_last = sh.att_arrive[u].fetch_add(1) == c.S - 1;
                if (!bar.wait()) { sh.hang = 1; return; }
                if (!sh_last) continue;
                if (w == 0) {
                    sh.att_arrive[u] = 0;
                    if (var == kFlags01) sh.ready[u] = 0;
                    bool nan = false;
                    for (int s = 0; s < c.S; ++s) nan |= sh.part[(size_t)u * c.S + s].load() < 0;
                    sh.out[u] = nan ? -1 : call_no;
                }
            }
        }
        if (w == 0 && sh.ctl[1].fetch_add(1) == c.W - 1) {
            sh.ctl[0] = 0;
            sh.ctl[1] = 0;
            if (var != kFlags01) sh.ctl[3] = raised;
        }
    };
    std::vector<std::thread> th;
    for (int w = 0; w < c.NW; ++w) th.emplace_back(wave, w);
    for (auto& t : th) t.join();
}

// One call: W workgroups over the items; returns false if it hung.
bool run_call(Variant var, const Call& c, Shared& sh, int call_no, unsigned seed) {
    std::vector<std::thread> wgs;
    for (int g = 0; g < c.W; ++g) wgs.emplace_back(workgroup, var, std::cref(c), std::ref(sh), call_no, g, seed + g);
    for (auto& t : wgs) t.join();
    return !sh.hang;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc < 5) {
        fprintf(stderr, "usage: %s shipped|noprefetch|onebarrier|flags01 trials seed spin_limit\n", argv[0]);
        return 2;
    }
    Variant var = kShipped;
    if (!strcmp(argv[1], "noprefetch")) var = kNoPrefetch;
    else if (!strcmp(argv[1], "onebarrier")) var = kOneBarrier;
    else if (!strcmp(argv[1], "flags01")) var = kFlags01;
    const int trials = atoi(argv[2]);
    const unsigned seed = (unsigned)atoi(argv[3]);
    const int first_limit = atoi(argv[4]);
    int hang = 0, mismatch = 0, stale = 0, wrong = 0, nan_units = 0, timeouts = 0;
    std::mt19937 rng(seed);
    for (int t = 0; t < trials; ++t) {
        Call c;
        c.U = std::uniform_int_distribution<int>(1, 5)(rng);
        c.C = std::uniform_int_distribution<int>(1, 4)(rng);
        c.S = std::uniform_int_distribution<int>(1, 3)(rng);
        c.W = std::uniform_int_distribution<int>(1, 4)(rng);
        c.NW = std::uniform_int_distribution<int>(2, 3)(rng);
        for (int u = 0; u < c.U; ++u) c.nch.push_back(std::uniform_int_distribution<int>(1, c.C)(rng));
        Shared sh(c.U, c.S);
        // two calls on one control area: the first with the given spin limit, the
        // second with a limit long enough never to be reached
        for (int call = 1; call <= 2; ++call) {
            c.spin_limit = call == 1 ? first_limit : 1 << 30;
            const int abandoned_before = sh.ctl[2].load();
            if (!run_call(var, c, sh, call, seed * 1000003u + t * 17u + call)) {
                ++hang;
                break;
            }
            const int abandoned = sh.ctl[2].load() - abandoned_before;
            timeouts += abandoned;
            int nan_here = 0;
            for (int u = 0; u < c.U; ++u) {
                const int o = sh.out[u].load();
                if (o == -1) ++nan_here;
                else if (o != call) ++wrong;  // not merged by this call
            }
            if (nan_here > abandoned || (nan_here > 0) != (abandoned > 0)) ++wrong;
            if (call == 2 && nan_here > 0) ++wrong;
            nan_units += nan_here;
            if (sh.ctl[0] != 0 || sh.ctl[1] != 0) ++wrong;
            if (var != kFlags01 && sh.ctl[3] != call) ++wrong;
            for (int u = 0; u < c.U; ++u)
                if (sh.scan_arrive[u] != 0 || sh.att_arrive[u] != 0) ++wrong;
        }
        mismatch += sh.mismatch.load();
        stale += sh.stale.load();
    }
    printf("hang=%d mismatch=%d stale=%d wrong=%d nan_units=%d timeouts=%d\n", hang, mismatch, stale, wrong,
           nan_units, timeouts);
    return 0;
}
