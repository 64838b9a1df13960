// lookback_model.hip -- a CPU model of librlscan's single-pass decoupled
// look-back (lookback.hpp), run by host threads; built host-only and run
// under ThreadSanitizer by tests/test_lookback_model.py.  No GPU is used.
//
// What is the library's own code here: the status words and their encoding
// (publish_aggregate / publish_inclusive: call tags, integers in one word
// when they fit 32 bits and in two words, written one after the other,
// otherwise; float64 values as two tagged halves over two entries per tile),
// read_status, status_of, poll_step (the decision a look-back wave takes
// from its ballots) and the step operations (compose, apply, cuts_chain).
// What the model replays: the 64-lane window walk of look_back, lane by
// lane as a wave would run it (narrow first poll of kNarrow predecessors,
// then the whole window, folding from the nearest terminal entry), and the
// per-call sequence of the host side (a new tag per call, and the clear of
// the status words before the tags repeat).
//
// Each call: K tiles over one status buffer shared by every call, as the
// library's scratch is; one thread per tile: publish the aggregate (or the
// inclusive value when already known), walk back, publish the inclusive
// value (some tiles after a long delay, so that walks fold aggregates over
// several windows).  The buffer starts each call holding words of other tags, of both
// integer forms (stale words of earlier calls, or of no call).  Every
// tile's entering value must equal the sequential fold of the aggregates
// before it, exactly: values are integers and a is 0 or 1 (float32 steps)
// or 0, 1 or -1 (float64 steps), so no composition order rounds.  Besides, deterministic checks of torn states:
// one word of a two-word value written and the other stale must never read
// as ready.
//
// Usage: lookback_model [--trials N] [--seed S] [--no-unit]; prints "ok ..."
// and exits 0, or prints the first mismatch and exits 1 (--no-unit: the
// concurrent trials alone, without the deterministic checks).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "lookback.hpp"

using namespace rlscan;

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);             \
            std::fprintf(stderr, "\n");                    \
            ++g_failures;                                  \
        }                                                  \
    } while (0)

// Polls of one window before the model gives up (host threads always make
// progress, so reaching it is a failure).
constexpr uint64_t kModelPolls = uint64_t(1) << 26;

template <class A> struct Value;
template <> struct Value<StepD> { using type = float; };
template <> struct Value<StepI> { using type = int64_t; };
template <> struct Value<StepW> { using type = double; };

// The look-back walk of one tile, lane by lane (lane 63: the nearest
// predecessor).
// Walks that folded more than one window (every entry of a 64-tile window
// an aggregate, none cutting the chain), over all trials.
std::atomic<long> g_deep_walks{0};

template <class A>
typename Value<A>::type walk(TileStatus* base, uint32_t tag, int64_t tile, bool& gave_up) {
    using V = typename Value<A>::type;
    A acc = identity_step(A{});
    int64_t top = tile - 1;
    for (int windows = 1;; ++windows) {
        A s[kWave];
        int width = kNarrow;
        PollStep step{};
        for (uint64_t polls = 0;; ++polls) {
            uint64_t term = 0, ready = 0;
            for (int lane = 0; lane < kWave; ++lane) {
                const int64_t q = top - (kWave - 1 - lane);
                s[lane] = identity_step(A{});
                int kind = q < 0 ? 3 : 0;
                if (q >= 0 && kWave - 1 - lane < width)
                    kind = read_status(status_of<A>(base, q), tag, s[lane]);
                if (kind == 2 || (kind == 1 && cuts_chain(s[lane]))) term |= uint64_t(1) << lane;
                if (kind != 0) ready |= uint64_t(1) << lane;
            }
            step = poll_step(term, ready, width);
            if (step.done) break;
            if (step.widen) {
                width = kWave;
                continue;
            }
            if (polls >= kModelPolls) {
                gave_up = true;
                return V(0);
            }
            std::this_thread::yield();
        }
        // lanes from the nearest terminal entry (or all) up to lane 63, the
        // farthest first, as the wave's inclusive scan composes them
        A total = identity_step(A{});
        for (int lane = step.stop >= 0 ? step.stop : 0; lane < kWave; ++lane)
            total = compose(s[lane], total);
        acc = compose(acc, total);
        if (step.stop >= 0) {
            if (windows > 1) g_deep_walks.fetch_add(1, std::memory_order_relaxed);
            return acc.b;
        }
        top -= kWave;
    }
}

// Random aggregates of one call.  p_cut: probability that a tile's
// aggregate cuts the chain (a = 0), which sets the walk lengths.
StepI random_step(std::mt19937_64& rng, double p_cut, StepI) {
    std::uniform_real_distribution<double> u(0.0, 1.0);
    StepI s;
    s.a = u(rng) < p_cut ? 0u : 1u;
    const double r = u(rng);
    if (r < 0.5) {
        s.b = static_cast<int64_t>(rng() % 2001) - 1000;  // one-word partial sums
    } else if (r < 0.7) {
        const int64_t edge[] = {INT32_MAX, INT32_MIN, int64_t(INT32_MAX) + 1,
                                int64_t(INT32_MIN) - 1, -1, 0};
        s.b = edge[rng() % 6];  // around the one-word / two-word boundary
    } else {
        s.b = static_cast<int64_t>(rng() % (uint64_t(1) << 44)) - (int64_t(1) << 43);
    }
    return s;
}
StepD random_step(std::mt19937_64& rng, double p_cut, StepD) {
    std::uniform_real_distribution<double> u(0.0, 1.0);
    StepD s;
    s.a = u(rng) < p_cut ? 0.0 : 1.0;
    s.b = static_cast<float>(static_cast<int>(rng() % 201) - 100);
    return s;
}
StepW random_step(std::mt19937_64& rng, double p_cut, StepW) {
    std::uniform_real_distribution<double> u(0.0, 1.0);
    StepW s;
    s.a = u(rng) < p_cut ? 0.0 : (rng() % 4 == 0 ? -1.0 : 1.0);
    s.b = static_cast<double>(static_cast<int>(rng() % 2001) - 1000);
    return s;
}

// Words of other tags in the tiles' entries: integer words in either form,
// with tags other than `tag` (and never the current tag's short form).
void fill_stale(TileStatus* st, int64_t entries, uint32_t tag, std::mt19937_64& rng) {
    for (int64_t i = 0; i < entries; ++i)
        for (int k = 0; k < 4; ++k) {
            uint32_t t = static_cast<uint32_t>(rng() % kLastTag) + 1;
            if (t == tag) t = t == 1 ? 2 : t - 1;
            if (rng() % 2) t |= kShortForm;
            if (rng() % 5 == 0) t = 0;  // a cleared word
            store_word(&st[i].w[k], tagged(t, static_cast<uint32_t>(rng())));
        }
}

// One call of K tiles.  Returns false on a mismatch.
template <class A>
bool run_call(TileStatus* status, int64_t capacity, uint32_t tag, int K, double p_cut,
              std::mt19937_64& rng) {
    using V = typename Value<A>::type;
    const int64_t entries = int64_t(K) * StatusEntries<A>::value;
    if (entries > capacity) return true;
    fill_stale(status, entries, tag, rng);
    std::vector<A> agg(K);
    for (auto& a : agg) a = random_step(rng, p_cut, A{});
    std::vector<V> want(K);
    V x = V(0);
    for (int k = 0; k < K; ++k) {  // entering value of tile k: the fold of 0..k-1
        want[k] = x;
        x = apply(agg[k], x);
    }
    std::vector<V> got(K, V(0));
    std::vector<char> gave_up(K, 0);
    // yields before a tile starts, and before it publishes its inclusive
    // value: late inclusive values make successors fold aggregates further
    // back, over several windows when K > 64 and no aggregate cuts
    std::vector<uint64_t> delay(K), late(K);
    for (auto& d : delay) d = rng() % 64;
    for (auto& d : late) d = rng() % 4 == 0 ? rng() % 2048 : 0;
    std::atomic<int> start{0};
    std::vector<std::thread> threads;
    threads.reserve(K);
    for (int k = 0; k < K; ++k)
        threads.emplace_back([&, k] {
            while (start.load(std::memory_order_acquire) == 0) std::this_thread::yield();
            for (uint64_t i = 0; i < delay[k]; ++i) std::this_thread::yield();
            TileStatus* st = status_of<A>(status, k);
            const bool known = k == 0 || cuts_chain(agg[k]);
            if (known)
                publish_inclusive(st, apply(agg[k], V(0)), tag);
            else
                publish_aggregate(st, agg[k], tag);
            V carry = V(0);
            bool gu = false;
            if (k > 0) carry = walk<A>(status, tag, k, gu);
            for (uint64_t i = 0; i < late[k]; ++i) std::this_thread::yield();
            if (!known) publish_inclusive(st, apply(agg[k], carry), tag);
            got[k] = carry;
            gave_up[k] = gu;
        });
    start.store(1, std::memory_order_release);
    for (auto& t : threads) t.join();
    bool ok = true;
    for (int k = 0; k < K; ++k) {
        // a tile whose own aggregate cuts the chain needs no entering value,
        // but the walk still returns the fold, so every tile is checked
        if (gave_up[k] || !(got[k] == want[k])) {
            std::fprintf(stderr, "mismatch: kind %d tag %u K %d tile %d gave_up %d got %.17g want %.17g\n",
                         int(sizeof(A)), tag, K, k, int(gave_up[k]), double(got[k]),
                         double(want[k]));
            ok = false;
            break;
        }
    }
    return ok;
}

// Deterministic torn states: a value is ready only when every word of it
// carries the call's tag.
void torn_state_checks() {
    TileStatus st[2];
    const uint32_t tag = 77, old = 76;
    auto clear = [&] {
        for (auto& e : st)
            for (auto& w : e.w) store_word(&w, 0);
    };
    // integer aggregate that needs two words: low word published, high stale
    clear();
    const int64_t big = (int64_t(5) << 40) + 3;
    store_word(&st[0].w[0], tagged(tag, static_cast<uint32_t>(big)));
    store_word(&st[0].w[1], tagged(old, static_cast<uint32_t>(uint64_t(big) >> 32)));
    StepI si{};
    CHECK(read_status(st, tag, si) == 0, "two-word aggregate with a stale high word read as ready");
    publish_aggregate(st, StepI{1u, big}, tag);
    CHECK(read_status(st, tag, si) == 1 && si.b == big && si.a == 1u, "two-word aggregate");
    // inclusive two-word value: low word only -> not ready, even with the
    // aggregate complete (the inclusive value is read first)
    store_word(&st[0].w[2], tagged(tag, 9u));
    store_word(&st[0].w[3], tagged(old, 1u));
    CHECK(read_status(st, tag, si) == 0, "two-word inclusive value with a stale high word");
    publish_inclusive(st, -big, tag);
    CHECK(read_status(st, tag, si) == 2 && si.b == -big && si.a == 0u, "two-word inclusive value");
    // one-word forms: the short form of another tag, or of the current tag
    // without its flag bit, is not a value of this call
    clear();
    store_word(&st[0].w[0], tagged(old | kShortForm, 5u));
    CHECK(read_status(st, tag, si) == 0, "short form of another tag");
    publish_aggregate(st, StepI{1u, -7}, tag);
    CHECK(read_status(st, tag, si) == 1 && si.b == -7, "short-form aggregate");
    CHECK(read_status(st, kNeverTag, si) == 0, "kNeverTag matched a word");
    publish_inclusive(st, int64_t(INT32_MIN), tag);
    CHECK(read_status(st, tag, si) == 2 && si.b == INT32_MIN, "short-form inclusive at INT32_MIN");
    // float: aggregate a published, b stale
    clear();
    StepD sd{};
    store_word(&st[0].w[0], tagged(tag, __builtin_bit_cast(uint32_t, 1.0f)));
    store_word(&st[0].w[1], tagged(old, 0u));
    CHECK(read_status(st, tag, sd) == 0, "float aggregate with a stale b");
    publish_aggregate(st, StepD{0.5, 3.0f}, tag);
    CHECK(read_status(st, tag, sd) == 1 && sd.a == 0.5 && sd.b == 3.0f, "float aggregate");
    // float64 values: every half must carry the tag
    clear();
    StepW sw{};
    publish_f64(&st[1].w[0], 2.5, tag);
    store_word(&st[1].w[1], tagged(old, 0u));
    CHECK(read_status(st, tag, sw) == 0, "float64 inclusive value with a stale half");
    publish_inclusive(st, 2.5, tag);
    CHECK(read_status(st, tag, sw) == 2 && sw.b == 2.5 && sw.a == 0.0, "float64 inclusive value");
    clear();
    publish_f64(&st[0].w[0], 2.0, tag);
    CHECK(read_status(st, tag, sw) == 0, "float64 aggregate without b");
    publish_aggregate(st, StepW{2.0, -1.5}, tag);
    CHECK(read_status(st, tag, sw) == 1 && sw.a == 2.0 && sw.b == -1.5, "float64 aggregate");
    // the poll decision: nearest terminal lane and what it needs
    PollStep p = poll_step(uint64_t(1) << 61, ~uint64_t(0) << 61, kNarrow);
    CHECK(p.done && p.stop == 61 && !p.widen, "poll: terminal lane 61, lanes 61..63 ready");
    p = poll_step(uint64_t(1) << 61, uint64_t(0xB) << 60, kNarrow);
    CHECK(!p.done && p.stop == 61, "poll: lane 62 not ready");
    p = poll_step(0, ~uint64_t(0) << (kWave - kNarrow), kNarrow);
    CHECK(!p.done && p.widen && p.stop == -1, "poll: narrow window ready, no terminal: widen");
    p = poll_step(0, ~uint64_t(0), kWave);
    CHECK(p.done && p.stop == -1, "poll: whole window ready, no terminal: fold it and move on");
}

}  // namespace

int main(int argc, char** argv) {
    int trials = 200;
    uint64_t seed = 1;
    bool unit = true;
    for (int i = 1; i < argc; ++i) {
        if (!std::strcmp(argv[i], "--no-unit")) unit = false;
        if (i + 1 < argc && !std::strcmp(argv[i], "--trials")) trials = std::atoi(argv[++i]);
        else if (i + 1 < argc && !std::strcmp(argv[i], "--seed"))
            seed = std::strtoull(argv[++i], nullptr, 10);
    }
    if (unit) torn_state_checks();
    std::mt19937_64 rng(seed);
    constexpr int64_t kCapacity = 2 * 160;  // entries: up to 160 float64 tiles
    std::vector<TileStatus> status(kCapacity);
    uint64_t epoch = 0;
    int calls = 0, wraps = 0;
    for (int trial = 0; trial < trials && g_failures == 0; ++trial) {
        // the host side's tag sequence: a new tag per call; before the tags
        // would repeat, every status word is cleared
        if (rng() % 16 == 0) epoch = kLastTag - 1 - rng() % 3;
        const int ncalls = 1 + static_cast<int>(rng() % 4);
        for (int c = 0; c < ncalls && g_failures == 0; ++c) {
            if (epoch >= kLastTag) {
                for (auto& e : status)
                    for (auto& w : e.w) store_word(&w, 0);
                epoch = 0;
                ++wraps;
            }
            const uint32_t tag = static_cast<uint32_t>(++epoch);
            const int sizes[] = {1, 2, 3, 5, 17, 63, 64, 65, 130, 160};
            const int K = sizes[rng() % 10];
            const double cuts[] = {0.0, 0.02, 0.3, 0.7};
            const double p_cut = cuts[rng() % 4];
            bool ok;
            switch (rng() % 3) {
                case 0: ok = run_call<StepI>(status.data(), kCapacity, tag, K, p_cut, rng); break;
                case 1: ok = run_call<StepD>(status.data(), kCapacity, tag, K, p_cut, rng); break;
                default: ok = run_call<StepW>(status.data(), kCapacity, tag, K, p_cut, rng); break;
            }
            if (!ok) ++g_failures;
            ++calls;
        }
    }
    if (g_failures) {
        std::printf("FAILED: %d failure(s)\n", g_failures);
        return 1;
    }
    std::printf("ok: %d trials, %d calls, %d tag wraps, %ld walks over several windows\n",
                trials, calls, wraps, g_deep_walks.load());
    return 0;
}
