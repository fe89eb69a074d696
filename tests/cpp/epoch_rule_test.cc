// Host build of the call-epoch rule and of the arrival that ends a call (epoch.h), with
// std::atomic counters and threads standing in for workgroups.  Exit status 0 when every
// check holds; each failed check prints one line.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <random>
#include <thread>
#include <vector>

#include "epoch.h"

using namespace sv;

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            ++failures;                                    \
            std::printf("FAIL %s:%d ", __FILE__, __LINE__); \
            std::printf(__VA_ARGS__);                      \
            std::printf("\n");                             \
        }                                                  \
    } while (0)

constexpr int kSingle = 256, kSlots = 32, kStride = 32;

struct Counters {
    std::atomic<uint32_t> top{0};
    std::atomic<uint32_t> slot[kSlots * kStride];
    Counters() {
        for (auto &s : slot) s.store(0);
    }
};

static Arrival arrive_host(Counters &c, int64_t i, int64_t n, bool gave_up) {
    return arrive(
        i, n, gave_up, &c.top, [&](int s) { return &c.slot[s * kStride]; }, kSingle, kSlots,
        [](std::atomic<uint32_t> *p, uint32_t v) { return p->fetch_add(v, std::memory_order_relaxed); },
        [](std::atomic<uint32_t> *p, uint32_t v) { return p->fetch_or(v, std::memory_order_relaxed); },
        [](std::atomic<uint32_t> *p) { p->store(0, std::memory_order_relaxed); });
}

// n units arrive from `threads` threads in a shuffled order; gave[i] marks the units that
// gave up.  Exactly one arrival is the last, it reports a give-up exactly when one happened,
// and every counter is back at zero.
static void arrival_case(int64_t n, const std::vector<char> &gave, int threads, unsigned seed) {
    Counters c;
    std::vector<int64_t> order(n);
    for (int64_t i = 0; i < n; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), std::mt19937(seed));
    std::atomic<int> lasts{0}, last_gave{-1};
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t) {
        pool.emplace_back([&, t] {
            for (int64_t q = t; q < n; q += threads) {
                const int64_t i = order[q];
                const Arrival a = arrive_host(c, i, n, gave[i] != 0);
                if (a.last) {
                    lasts.fetch_add(1);
                    last_gave.store(a.gave_up ? 1 : 0);
                } else {
                    CHECK(!a.gave_up, "n=%lld: a unit that is not the last reports a give-up", (long long)n);
                }
            }
        });
    }
    for (auto &th : pool) th.join();
    bool any = false;
    for (char g : gave) any = any || g;
    CHECK(lasts.load() == 1, "n=%lld: %d last arrivals", (long long)n, lasts.load());
    CHECK(last_gave.load() == (any ? 1 : 0), "n=%lld: last arrival reports gave_up=%d, expected %d", (long long)n,
          last_gave.load(), any ? 1 : 0);
    CHECK(c.top.load() == 0, "n=%lld: second-level counter left at %u", (long long)n, c.top.load());
    for (int s = 0; s < kSlots; ++s)
        CHECK(c.slot[s * kStride].load() == 0, "n=%lld: slot %d left at %u", (long long)n, s, c.slot[s * kStride].load());
}

// A model of the workspace protocol: tagged words (payload, tag) of one slot, the epoch, and
// a call whose finalize reads the slot.  A late workgroup reads the epoch after the call
// ended; with poisoning its word must never be taken for the next call's.
struct Word {
    uint32_t payload = 0, tag = 0;
};

static void late_workgroup_case() {
    uint32_t epoch = 0;
    Word slot;
    // call 1: the member of the slot is late; the finalize's wait gives up, recomputes, and
    // arrives as the only unit with gave_up = true
    uint32_t tag1 = epoch_tag(epoch);
    CHECK(!epoch_poisoned(epoch), "fresh epoch poisoned");
    Counters c;
    Arrival a = arrive_host(c, 0, 1, true);
    CHECK(a.last && a.gave_up, "single arrival that gave up");
    epoch = epoch_after(tag1, a.gave_up);
    CHECK(epoch_poisoned(epoch), "a call whose wait gave up leaves the epoch unpoisoned");
    // the late member now reads the epoch: poisoned, so it writes nothing
    const uint32_t seen = epoch;
    if (!epoch_poisoned(seen)) slot = Word{1234u, epoch_tag(seen)};
    // call 2 (verification) on the poisoned workspace: nothing verified, epoch unchanged
    CHECK(epoch_poisoned(epoch), "poison lost");
    // without the poison bit the late word would carry call 2's tag: the model's hazard
    CHECK(epoch_tag(tag1) == epoch_tag(epoch & ~kEpochPoison), "model: tags");
    CHECK(slot.tag != epoch_tag(epoch) && slot.tag != epoch_tag(tag1), "a late word carries a live tag");
    // zero-fill: epoch 0 and every word absent; the next call's tag is 1, which no word holds
    epoch = 0;
    slot = Word{};
    CHECK(slot.tag != epoch_tag(epoch), "zero-filled word is present");
    // a healthy call advances the epoch to its tag, unpoisoned
    a = arrive_host(c, 0, 1, false);
    CHECK(a.last && !a.gave_up, "single healthy arrival");
    epoch = epoch_after(epoch_tag(epoch), a.gave_up);
    CHECK(epoch == 1u && !epoch_poisoned(epoch), "healthy advance gives %u", epoch);
}

int main() {
    // the epoch arithmetic
    CHECK(epoch_tag(0u) == 1u, "tag of epoch 0");
    CHECK(epoch_after(7u, false) == 7u, "healthy call");
    CHECK(epoch_after(7u, true) == (7u | kEpochPoison), "call that gave up");
    CHECK(epoch_poisoned(epoch_after(7u, true)), "poison bit");
    CHECK(!epoch_poisoned(epoch_after(kEpochPoison - 2u, false)), "last healthy tag");
    CHECK(epoch_poisoned(epoch_after(kEpochPoison - 1u, false)), "spent tags poison the epoch");
    CHECK(epoch_poisoned(epoch_after(epoch_tag(kEpochPoison | 5u), false)), "a poisoned epoch stays poisoned");

    // arrivals: single-counter and two-level, no / one / many / all give-ups
    const int64_t sizes[] = {1, 2, 63, 256, 257, 1000, 8191};
    unsigned seed = 1;
    for (int64_t n : sizes) {
        for (int pattern = 0; pattern < 5; ++pattern) {
            std::vector<char> gave(n, 0);
            std::mt19937 rng(seed);
            if (pattern == 1) gave[rng() % n] = 1;                                 // one unit
            if (pattern == 2) gave[n - 1] = 1;                                     // the last unit index
            if (pattern == 3) for (int64_t i = 0; i < n; ++i) gave[i] = 1;         // every unit
            if (pattern == 4) for (int64_t i = 0; i < n; i += kSlots) gave[i] = 1;  // all of slot 0
            for (int threads : {1, 4, 8}) arrival_case(n, gave, threads, seed++);
        }
    }
    late_workgroup_case();
    if (failures == 0) std::printf("ok\n");
    return failures == 0 ? 0 : 1;
}
