// Host check of the persistent chunk solver's task order (kq_chunk_sched.hpp),
// built and run by tests/test_chunk_sched.py.  For every chunk that the
// solver's recursion makes on an Mt x Nt tile grid it checks that
//   * the tickets name each sweep and precompute task of the chunk once;
//   * every flag a task waits on belongs to a task of the same chunk with a
//     smaller ticket (so the holder of the smallest unfinished ticket never
//     waits, and a launch finishes whatever number of workgroups is resident);
//   * what each task reads is final once its waits are over: a sweep reads the
//     errors of (I, J - 1) and the row-propagated errors of (I - 1, J) and its
//     tile's pre-accumulated products; a precompute task reads the errors of
//     (I, J') and the row-propagated errors of (I', J) for every older slice in
//     the chunk.  "Final" is checked by following the waits transitively.
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
    // ticket of the task that raises flag word w (sweep or precompute of a tile), -1 if none in the chunk
    int raiser(int w) const {
        const int kind = w >= Mt * Nt ? 1 : 0;
        const int tile = w - kind * Mt * Nt;
        const int I = tile / Nt, J = tile % Nt;
        const int K = I + J;
        if (K < c0 || K >= c1) return -1;
        if (kind == 1 && K == c0) return -1;
        return chunk_ticket(kind, K, I - diag_lo(K, Nt), c0, c1, Mt, Nt);
    }
    void deps(int ticket, std::vector<int>& out) const {
        out.clear();
        const ChunkDeps d = chunk_deps(chunk_task(ticket, c0, c1, Mt, Nt), c0, Mt, Nt);
        for (int w : {d.w0, d.w1, d.w2})
            if (w >= 0) out.push_back(w);
    }
    // the tiles (kind 0: sweep result, 1: precompute result) a task reads, within the chunk
    void reads(int ticket, std::vector<int>& out) const {
        out.clear();
        const ChunkTask tk = chunk_task(ticket, c0, c1, Mt, Nt);
        const int I = diag_lo(tk.Kt, Nt) + tk.idx, J = tk.Kt - I;
        const int jl = c0 - I > 0 ? c0 - I : 0, il = c0 - J > 0 ? c0 - J : 0;
        if (tk.kind == 0) {
            if (J - 1 >= jl) out.push_back(I * Nt + J - 1);
            if (I - 1 >= il) out.push_back((I - 1) * Nt + J);
            if (tk.Kt > c0) out.push_back(Mt * Nt + I * Nt + J);
        } else {
            for (int jp = jl; jp <= J - 2; ++jp) out.push_back(I * Nt + jp);
            for (int ip = il; ip <= I - 2; ++ip) out.push_back(ip * Nt + J);
        }
    }
};

static void check_order(const Grid& g) {
    const int n = chunk_tasks(g.c0, g.c1, g.Mt, g.Nt);
    std::set<long> seen;
    std::vector<int> dv, rv;
    // closure[t] = the tasks known finished once t's waits are over (transitively)
    std::vector<std::set<int>> done_before(n);
    for (int t = 0; t < n; ++t) {
        const ChunkTask tk = chunk_task(t, g.c0, g.c1, g.Mt, g.Nt);
        CHECK(tk.kind == 0 || tk.kind == 1, "ticket %d of chunk [%d,%d) has no task", t, g.c0, g.c1);
        const int I = diag_lo(tk.Kt, g.Nt) + tk.idx, J = tk.Kt - I;
        CHECK(I >= 0 && I < g.Mt && J >= 0 && J < g.Nt, "task %d names tile (%d,%d) off the grid", t, I, J);
        CHECK(tk.Kt >= g.c0 && tk.Kt < g.c1 && (tk.kind == 0 || tk.Kt > g.c0), "task %d outside its chunk", t);
        CHECK(chunk_ticket(tk.kind, tk.Kt, tk.idx, g.c0, g.c1, g.Mt, g.Nt) == t, "ticket %d does not round-trip", t);
        CHECK(seen.insert(long(tk.kind) * g.Mt * g.Nt + long(I) * g.Nt + J).second, "task %d named twice", t);
        g.deps(t, dv);
        std::set<int> known;
        for (int w : dv) {
            const int r = g.raiser(w);
            CHECK(r >= 0, "task %d waits on flag %d that no task of the chunk raises", t, w);
            CHECK(r < t, "task %d waits on task %d with a larger ticket", t, r);
            if (r >= 0 && r < t) {
                known.insert(r);
                known.insert(done_before[r].begin(), done_before[r].end());
            }
        }
        done_before[t] = known;
        g.reads(t, rv);
        for (int w : rv) {
            const int r = g.raiser(w);
            CHECK(r >= 0 && known.count(r), "task %d (kind %d, tile %d,%d) reads flag %d's data before it is final",
                  t, tk.kind, I, J, w);
        }
    }
    CHECK(chunk_task(n, g.c0, g.c1, g.Mt, g.Nt).kind < 0, "ticket past the chunk names a task");
    CHECK(int(seen.size()) == n, "chunk [%d,%d): %zu tasks named, %d expected", g.c0, g.c1, seen.size(), n);
}

static void simulate(const Grid& g, int workers, unsigned seed) {
    const int n = chunk_tasks(g.c0, g.c1, g.Mt, g.Nt);
    std::vector<std::atomic<int>> flags(2 * g.Mt * g.Nt);
    for (auto& f : flags) f.store(0);
    std::atomic<int> counter{0}, timeouts{0}, bad_reads{0}, ran{0};
    auto work = [&](unsigned s) {
        std::mt19937 rng(s);
        std::vector<int> dv, rv;
        for (;;) {
            const int t = counter.fetch_add(1);
            if (t >= n) return;
            if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
            g.deps(t, dv);
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
            g.reads(t, rv);
            for (int w : rv)
                if (flags[w].load(std::memory_order_acquire) == 0) bad_reads.fetch_add(1);
            const ChunkTask tk = chunk_task(t, g.c0, g.c1, g.Mt, g.Nt);
            const int I = diag_lo(tk.Kt, g.Nt) + tk.idx, J = tk.Kt - I;
            if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
            flags[tk.kind * g.Mt * g.Nt + I * g.Nt + J].store(1, std::memory_order_release);
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
