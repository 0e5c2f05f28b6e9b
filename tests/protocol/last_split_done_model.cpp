// CPU model of the decode kernel's fused last-split-done merge (test
// infrastructure; shares nothing with the GPU code).
//
// The split-K producer of the lmdeploy PR "use PDL for paged attention"
// (Changes) writes per-split scratch that a reducer reads; the decode kernel
// fuses the reducer into the producer launch instead of overlapping two
// launches: every split workgroup publishes its (m, l, acc) state, then
// counts itself in on an arrival counter of its (request, kv head) group; the
// one that sees S - 1 merges all S states in split order and resets the
// counter for the next call.  This program runs that protocol on threads:
//
//   * a "call" has G groups of S splits; each (group, split) is a task, and
//     the tasks of a call are taken by T threads in a random order with
//     random pauses, so arrival order and interleaving vary;
//   * some splits are empty (m = -inf, l = 0, acc = 0) and must still arrive;
//   * the counters persist across calls (graph replays reuse the workspace);
//   * publication = plain stores of the state, then fetch_add(acq_rel) on the
//     counter; the merger's acquire side is the same fetch_add.  On the GPU
//     the release is the write-through stores completed (vmcnt(0)) before the
//     memory-side atomic, and the acquire the merger's cache-bypassing loads.
//
// Checks after each call: every group merged exactly once, its output equal
// bit for bit to a sequential merge in split order, every counter back at 0.
// Built with -fsanitize=thread, a publication that is not ordered before the
// merger's reads is reported as a data race.
//
// Modes plant one mistake each (the model must then fail):
//   correct       the protocol as the kernel runs it
//   signal_early  count in before storing the state
//   no_reset      the merger leaves the counter at S
//   skip_empty    empty splits do not count in
//
// usage: last_split_done_model MODE SEED CALLS THREADS
// exit 0 = all checks passed; 1 = a check failed; 2 = bad usage.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>
#include <string>
#include <thread>
#include <vector>

namespace {

constexpr int kDim = 8;   // accumulator values per state
const float kNegInf = -std::numeric_limits<float>::infinity();

enum class Mode { kCorrect, kSignalEarly, kNoReset, kSkipEmpty };

struct State {
    float m, l, acc[kDim];
};

// log-sum-exp merge of S states in split order (the reducer's definition)
void merge(const State *st, int S, float *out) {
    float M = kNegInf;
    for (int j = 0; j < S; ++j) M = std::fmax(M, st[j].m);
    float l = 0.f, o[kDim] = {};
    for (int j = 0; j < S; ++j) {
        if (st[j].m == kNegInf) continue;
        const float w = std::exp(st[j].m - M);
        l = std::fma(w, st[j].l, l);
        for (int d = 0; d < kDim; ++d) o[d] = std::fma(w, st[j].acc[d], o[d]);
    }
    for (int d = 0; d < kDim; ++d) out[d] = l > 0.f ? o[d] / l : 0.f;
}

struct Shared {
    int G, S;
    std::vector<State> scratch;              // [G][S], plain memory
    std::vector<std::atomic<int>> counters;  // [G], persist across calls
    std::vector<std::atomic<int>> merges;    // [G], merges seen this call
    std::vector<float> out;                  // [G][kDim], written by the merger
    Shared(int g, int s)
        : G(g), S(s), scratch((size_t)g * s), counters(g), merges(g), out((size_t)g * kDim) {
        for (auto &c : counters) c.store(0);
    }
};

void spin(std::mt19937 &rng) {
    const int n = (int)(rng() % 64);
    for (volatile int i = 0; i < n; ++i) {
    }
    if (rng() % 8 == 0) std::this_thread::yield();
}

// One split workgroup: publish, arrive, and merge if last.
void split_task(Shared &sh, const State &mine, int g, int j, Mode mode, std::mt19937 &rng) {
    State *dst = &sh.scratch[(size_t)g * sh.S + j];
    const bool empty = mine.m == kNegInf;
    auto store_state = [&] {
        dst->m = mine.m;
        dst->l = mine.l;
        for (int d = 0; d < kDim; ++d) dst->acc[d] = mine.acc[d];
    };
    int old = -1;
    if (mode == Mode::kSignalEarly) {
        old = sh.counters[g].fetch_add(1, std::memory_order_acq_rel);
        spin(rng);
        store_state();
    } else {
        store_state();
        spin(rng);
        if (mode == Mode::kSkipEmpty && empty) return;
        old = sh.counters[g].fetch_add(1, std::memory_order_acq_rel);
    }
    if (old != sh.S - 1) return;
    merge(&sh.scratch[(size_t)g * sh.S], sh.S, &sh.out[(size_t)g * kDim]);
    sh.merges[g].fetch_add(1, std::memory_order_relaxed);
    if (mode != Mode::kNoReset) sh.counters[g].store(0, std::memory_order_relaxed);
}

}  // namespace

int main(int argc, char **argv) {
    if (argc != 5) {
        std::fprintf(stderr, "usage: %s MODE SEED CALLS THREADS\n", argv[0]);
        return 2;
    }
    const std::string ms = argv[1];
    Mode mode;
    if (ms == "correct") mode = Mode::kCorrect;
    else if (ms == "signal_early") mode = Mode::kSignalEarly;
    else if (ms == "no_reset") mode = Mode::kNoReset;
    else if (ms == "skip_empty") mode = Mode::kSkipEmpty;
    else return 2;
    const unsigned seed = (unsigned)std::strtoul(argv[2], nullptr, 10);
    const int calls = std::atoi(argv[3]), threads = std::atoi(argv[4]);
    if (calls < 1 || threads < 1) return 2;

    constexpr int G = 48, S = 16;
    Shared sh(G, S);
    std::mt19937 rng(seed);
    int failures = 0;
    for (int call = 0; call < calls; ++call) {
        // this call's split states: about one in four empty
        std::vector<State> states((size_t)G * S);
        std::uniform_real_distribution<float> um(-8.f, 8.f), ul(1.f, 64.f), ua(-30.f, 30.f);
        for (auto &st : states) {
            if (rng() % 4 == 0) {
                st.m = kNegInf;
                st.l = 0.f;
                for (float &a : st.acc) a = 0.f;
            } else {
                st.m = um(rng);
                st.l = ul(rng);
                for (float &a : st.acc) a = ua(rng);
            }
        }
        std::vector<int> order((size_t)G * S);
        for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
        std::shuffle(order.begin(), order.end(), rng);
        for (auto &mg : sh.merges) mg.store(0);
        std::fill(sh.out.begin(), sh.out.end(), std::nanf(""));

        std::atomic<size_t> cursor{0};
        std::vector<std::thread> pool;
        for (int t = 0; t < threads; ++t) {
            pool.emplace_back([&, t] {
                std::mt19937 trng(seed * 7919u + (unsigned)call * 131u + (unsigned)t);
                for (;;) {
                    const size_t i = cursor.fetch_add(1, std::memory_order_relaxed);
                    if (i >= order.size()) break;
                    const int task = order[i];
                    split_task(sh, states[task], task / S, task % S, mode, trng);
                }
            });
        }
        for (auto &th : pool) th.join();

        for (int g = 0; g < G; ++g) {
            float ref[kDim];
            merge(&states[(size_t)g * S], S, ref);
            const int n = sh.merges[g].load();
            const int c = sh.counters[g].load();
            bool same = n == 1;
            for (int d = 0; d < kDim && same; ++d)
                same = std::memcmp(&ref[d], &sh.out[(size_t)g * kDim + d], sizeof(float)) == 0;
            if (!same || c != 0) {
                if (failures < 5)
                    std::fprintf(stderr, "call %d group %d: merges %d, counter %d, output %s\n",
                                 call, g, n, c, same ? "equal" : "differs");
                ++failures;
            }
        }
    }
    std::printf("%s: %d calls x %d groups x %d splits on %d threads, %d failed group checks\n",
                ms.c_str(), calls, G, S, threads, failures);
    return failures == 0 ? 0 : 1;
}
