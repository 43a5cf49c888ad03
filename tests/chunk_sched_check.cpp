// Host check of the persistent chunk solver's task order (kq_chunk_sched.hpp),
// built and run by tests/test_chunk_sched.py.  For every chunk that the
// solver's recursion makes on an Mt x Nt tile grid it checks that
//   * the tickets name the task of each tile of the chunk once;
//   * every flag a task waits on belongs to a task of the same chunk with a
//     smaller ticket (so the holder of the smallest unfinished ticket never
//     waits, and a launch finishes whatever number of workgroups is resident);
//   * what each task reads is final once the wait before it is over: the task
//     of tile (I, J) first reads the errors of (I, J') and the row-propagated
//     errors of (I', J) of every older slice in the chunk (J' <= J - 2,
//     I' <= I - 2), then those of (I, J - 1) and (I - 1, J).  "Final" is checked
//     by following the waits transitively.
// Then it runs each chunk on worker threads that draw tickets from an atomic
// counter, wait on atomic flags with a bounded spin and sleep at random, and
// checks that every task ran, no wait hit its bound, and every read found its
// source task finished.
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
    // ticket of the task that raises flag word w (the sweep of a tile), -1 if none in the chunk
    int raiser(int w) const {
        const int I = w / Nt, J = w % Nt;
        const int K = I + J;
        if (w < 0 || I >= Mt || K < c0 || K >= c1) return -1;
        return chunk_ticket(K, I - diag_lo(K, Nt), c0, Mt, Nt);
    }
    // the flags a task waits on before its older slices (phase 0) and before its freshest (phase 1)
    void deps(int ticket, int phase, std::vector<int>& out) const {
        out.clear();
        const ChunkDeps d = chunk_deps(chunk_task(ticket, c0, c1, Mt, Nt), c0, Nt);
        for (int w : phase == 0 ? std::vector<int>{d.o0, d.o1} : std::vector<int>{d.f0, d.f1})
            if (w >= 0) out.push_back(w);
    }
    // the tiles whose sweep results (errors D and row-propagated errors R) a
    // task reads in each phase: the older slices, then the two freshest
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
    std::vector<int> dv, rv;
    // done_before[t] = the tasks known finished once all of t's waits are over (transitively)
    std::vector<std::set<int>> done_before(n);
    for (int t = 0; t < n; ++t) {
        const ChunkTask tk = chunk_task(t, g.c0, g.c1, g.Mt, g.Nt);
        CHECK(tk.Kt >= 0, "ticket %d of chunk [%d,%d) has no task", t, g.c0, g.c1);
        const int I = diag_lo(tk.Kt, g.Nt) + tk.idx, J = tk.Kt - I;
        CHECK(I >= 0 && I < g.Mt && J >= 0 && J < g.Nt, "task %d names tile (%d,%d) off the grid", t, I, J);
        CHECK(tk.Kt >= g.c0 && tk.Kt < g.c1, "task %d outside its chunk", t);
        CHECK(chunk_ticket(tk.Kt, tk.idx, g.c0, g.Mt, g.Nt) == t, "ticket %d does not round-trip", t);
        CHECK(seen.insert(long(I) * g.Nt + J).second, "task %d named twice", t);
        std::set<int> known;
        for (int phase = 0; phase < 2; ++phase) {
            g.deps(t, phase, dv);
            for (int w : dv) {
                const int r = g.raiser(w);
                CHECK(r >= 0, "task %d waits on flag %d that no task of the chunk raises", t, w);
                CHECK(r < t, "task %d waits on task %d with a larger ticket", t, r);
                if (r >= 0 && r < t) {
                    known.insert(r);
                    known.insert(done_before[r].begin(), done_before[r].end());
                }
            }
            g.reads(t, phase, rv);
            for (int w : rv) {
                const int r = g.raiser(w);
                CHECK(r >= 0 && known.count(r), "task %d (tile %d,%d) reads tile %d in phase %d before it is final", t,
                      I, J, w, phase);
            }
        }
        done_before[t] = known;
    }
    CHECK(chunk_task(n, g.c0, g.c1, g.Mt, g.Nt).Kt < 0, "ticket past the chunk names a task");
    CHECK(int(seen.size()) == n, "chunk [%d,%d): %zu tasks named, %d expected", g.c0, g.c1, seen.size(), n);
}

static void simulate(const Grid& g, int workers, unsigned seed) {
    const int n = chunk_tasks(g.c0, g.c1, g.Mt, g.Nt);
    std::vector<std::atomic<int>> flags(g.Mt * g.Nt);
    for (auto& f : flags) f.store(0);
    std::atomic<int> counter{0}, timeouts{0}, bad_reads{0}, ran{0};
    auto work = [&](unsigned s) {
        std::mt19937 rng(s);
        std::vector<int> dv, rv;
        for (;;) {
            const int t = counter.fetch_add(1);
            if (t >= n) return;
            for (int phase = 0; phase < 2; ++phase) {
                if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
                g.deps(t, phase, dv);
                for (int w : dv) {
                    long it = 0;
                    while (flags[w].load(std::memory_order_acquire) == 0) {
                        if (++it > 200000000L) {
                            timeouts.fetch_add(1);
                            break;
                        }
                        std::this_thread::yield();
                    }
                }
                g.reads(t, phase, rv);
                for (int w : rv)
                    if (flags[w].load(std::memory_order_acquire) == 0) bad_reads.fetch_add(1);
            }
            const ChunkTask tk = chunk_task(t, g.c0, g.c1, g.Mt, g.Nt);
            const int I = diag_lo(tk.Kt, g.Nt) + tk.idx, J = tk.Kt - I;
            if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
            flags[I * g.Nt + J].store(1, std::memory_order_release);
            ran.fetch_add(1);
        }
    };
    std::vector<std::thread> th;
    for (int w = 0; w < workers; ++w) th.emplace_back(work, seed * 131u + unsigned(w));
    for (auto& x : th) x.join();
    CHECK(timeouts.load() == 0 && bad_reads.load() == 0 && ran.load() == n,
          "simulation %dx%d chunk [%d,%d) with %d workers: %d timeouts, %d early reads, %d of %d tasks", g.Mt, g.Nt,
          g.c0, g.c1, workers, timeouts.load(), bad_reads.load(), ran.load(), n);
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
