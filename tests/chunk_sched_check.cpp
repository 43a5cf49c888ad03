// Host check of the persistent chunk solver's task order (kq_chunk_sched.hpp),
// built and run by tests/test_chunk_sched.py.  For every chunk that the
// solver's recursion makes on an Mt x Nt tile grid it checks that
//   * the tickets name the task of each tile of the chunk once;
//   * every tile output a task reads (the errors of (I, J') and the
//     row-propagated errors of (I', J) of every slice of the chunk before
//     (I, J) in its row and column, older ones first, then the two freshest)
//     is written by a task of the same chunk with a smaller ticket, so the
//     holder of the smallest unfinished ticket never waits, and a launch
//     finishes whatever number of workgroups is resident.
// Then it runs each chunk on worker threads that draw tickets from an atomic
// counter, poll per-tile "written" words with a bounded spin and sleep at
// random, and checks that every task ran, no wait hit its bound, and every read
// found its value written.
#include "kq_chunk_sched.hpp"

#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <thread>
#include <vector>

using namespace kq;

static int fails = 0;
#define CHECK(c, ...)                          \
    do {                                       \
        if (!(c)) {                            \
            if (fails < 20) {                  \
                std::printf("FAIL: " __VA_ARGS__); \
                std::printf("\n");             \
            }                                  \
            ++fails;                           \
        }                                      \
    } while (0)

static void chunks(int K0, int K1, std::vector<std::pair<int, int>>& out) {
    if (K1 - K0 <= CHUNK) {
        out.push_back({K0, K1});
        return;
    }
    const int n = (K1 - K0 + CHUNK - 1) / CHUNK;
    const int mid = K0 + CHUNK * (n / 2);
    chunks(K0, mid, out);
    chunks(mid, K1, out);
}

struct Grid {
    int Mt, Nt, c0, c1;
    // ticket of the task that writes tile w's outputs (w = I Nt + J), -1 if none in the chunk
    int writer(int w) const {
        const int I = w / Nt, J = w % Nt;
        const int K = I + J;
        if (w < 0 || I >= Mt || K < c0 || K >= c1) return -1;
        return chunk_ticket(K, I - diag_lo(K, Nt), c0, Mt, Nt);
    }
    // the tiles whose outputs a task reads: phase 0 the older slices, phase 1 the two freshest
    void reads(int ticket, int phase, std::vector<int>& out) const {
        out.clear();
        const ChunkTask tk = chunk_task(ticket, c0, c1, Mt, Nt);
        const int I = diag_lo(tk.Kt, Nt) + tk.idx, J = tk.Kt - I;
        const int jl = c0 - I > 0 ? c0 - I : 0, il = c0 - J > 0 ? c0 - J : 0;
        if (phase == 0) {
            for (int jp = jl; jp <= J - 2; ++jp) out.push_back(I * Nt + jp);
            for (int ip = il; ip <= I - 2; ++ip) out.push_back(ip * Nt + J);
        } else {
            if (J - 1 >= jl) out.push_back(I * Nt + J - 1);
            if (I - 1 >= il) out.push_back((I - 1) * Nt + J);
        }
    }
};

static void check_order(const Grid& g) {
    const int n = chunk_tasks(g.c0, g.c1, g.Mt, g.Nt);
    std::set<long> seen;
    std::vector<int> rv;
    for (int t = 0; t < n; ++t) {
        const ChunkTask tk = chunk_task(t, g.c0, g.c1, g.Mt, g.Nt);
        CHECK(tk.Kt >= 0, "ticket %d of chunk [%d,%d) has no task", t, g.c0, g.c1);
        const int I = diag_lo(tk.Kt, g.Nt) + tk.idx, J = tk.Kt - I;
        CHECK(I >= 0 && I < g.Mt && J >= 0 && J < g.Nt, "task %d names tile (%d,%d) off the grid", t, I, J);
        CHECK(tk.Kt >= g.c0 && tk.Kt < g.c1, "task %d outside its chunk", t);
        CHECK(chunk_ticket(tk.Kt, tk.idx, g.c0, g.Mt, g.Nt) == t, "ticket %d does not round-trip", t);
        CHECK(seen.insert(long(I) * g.Nt + J).second, "task %d named twice", t);
        for (int phase = 0; phase < 2; ++phase) {
            g.reads(t, phase, rv);
            for (int w : rv) {
                const int r = g.writer(w);
                CHECK(r >= 0, "task %d (tile %d,%d) reads tile %d that no task of the chunk writes", t, I, J, w);
                CHECK(r < t, "task %d (tile %d,%d) reads tile %d written by task %d, a larger ticket", t, I, J, w, r);
            }
        }
    }
    CHECK(chunk_task(n, g.c0, g.c1, g.Mt, g.Nt).Kt < 0, "ticket past the chunk names a task");
    CHECK(int(seen.size()) == n, "chunk [%d,%d): %zu tasks named, %d expected", g.c0, g.c1, seen.size(), n);
}

static void simulate(const Grid& g, int workers, unsigned seed) {
    const int n = chunk_tasks(g.c0, g.c1, g.Mt, g.Nt);
    std::vector<std::atomic<int>> written(g.Mt * g.Nt);
    for (auto& f : written) f.store(0);
    std::atomic<int> counter{0}, timeouts{0}, ran{0};
    auto work = [&](unsigned s) {
        std::mt19937 rng(s);
        std::vector<int> rv;
        for (;;) {
            const int t = counter.fetch_add(1);
            if (t >= n) return;
            for (int phase = 0; phase < 2; ++phase) {
                if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
                g.reads(t, phase, rv);
                for (int w : rv) {  // poll each value read until it is written
                    long it = 0;
                    while (written[w].load(std::memory_order_acquire) == 0) {
                        if (++it > 200000000L) {
                            timeouts.fetch_add(1);
                            break;
                        }
                        std::this_thread::yield();
                    }
                }
            }
            const ChunkTask tk = chunk_task(t, g.c0, g.c1, g.Mt, g.Nt);
            const int I = diag_lo(tk.Kt, g.Nt) + tk.idx, J = tk.Kt - I;
            if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
            written[I * g.Nt + J].store(1, std::memory_order_release);
            ran.fetch_add(1);
        }
    };
    std::vector<std::thread> th;
    for (int w = 0; w < workers; ++w) th.emplace_back(work, seed * 131u + unsigned(w));
    for (auto& x : th) x.join();
    CHECK(timeouts.load() == 0 && ran.load() == n,
          "simulation %dx%d chunk [%d,%d) with %d workers: %d timeouts, %d of %d tasks", g.Mt, g.Nt, g.c0, g.c1,
          workers, timeouts.load(), ran.load(), n);
}

int main(int argc, char** argv) {
    // tile grids: the configured shapes in 32-tiles and small, ragged and degenerate ones
    const int shapes[][2] = {{1, 1},   {1, 2},   {2, 1},   {2, 2},   {3, 5},   {8, 8},   {16, 16}, {17, 3},
                             {3, 40},  {32, 32}, {33, 65}, {64, 64}, {48, 16}, {128, 128}, {32, 128},
                             {448, 128}, {128, 448}};
    long nchunks = 0;
    for (auto& s : shapes) {
        std::vector<std::pair<int, int>> cs;
        chunks(0, s[0] + s[1] - 1, cs);
        for (auto& c : cs) {
            Grid g{s[0], s[1], c.first, c.second};
            check_order(g);
            ++nchunks;
        }
    }
    const bool sim = argc < 2 || std::atoi(argv[1]) != 0;
    if (sim) {
        const int sim_shapes[][2] = {{8, 8}, {17, 3}, {33, 65}, {64, 64}};
        unsigned seed = 1;
        for (auto& s : sim_shapes) {
            std::vector<std::pair<int, int>> cs;
            chunks(0, s[0] + s[1] - 1, cs);
            for (auto& c : cs)
                for (int workers : {1, 3, 16}) simulate(Grid{s[0], s[1], c.first, c.second}, workers, seed++);
        }
    }
    std::printf("%ld chunks checked, %d failures\n", nchunks, fails);
    return fails ? 1 : 0;
}
