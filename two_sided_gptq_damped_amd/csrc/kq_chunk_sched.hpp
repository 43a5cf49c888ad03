// Task order of the persistent chunk solver (FastKron page, section 2.3: the
// tiles of one tile-diagonal are independent; section 2.5: a chunk of
// tile-diagonals is solved before the band products that follow it).
//
// One launch solves the tile-diagonals [c0, c1) of a chunk.  Its workgroups
// draw tickets from one counter and run the task each ticket names, in ticket
// order:
//   group g = 0 .. c1 - c0 - 1:  the precompute tasks of diagonal c0 + g + 1
//                                (when it is in the chunk), then the sweep tasks
//                                of diagonal c0 + g,
// each diagonal's tiles by increasing row I.  A sweep task rounds tile (I, J);
// the precompute task of tile (I, J) on diagonal Kt sums the tile's chunk
// products over every slice older than its two freshest ones.  The tasks wait
// on one another through per-tile flags:
//   sweep (I, J)       the sweeps of (I - 1, J) and (I, J - 1) (its freshest
//                      slices) and its own precompute task, when Kt > c0;
//   precompute (I, J)  the sweeps of (I, J - 2) and (I - 2, J) when those are in
//                      the chunk (each sweep waited for the tile before it in
//                      its row and column, so the older slices are final too).
// Every task waits only on tasks with smaller tickets, and a workgroup waits
// only on the task it drew last, so the holder of the smallest unfinished
// ticket never waits on an unfinished task: the launch finishes whatever
// number of its workgroups is resident (chunk_sched_check verifies the order
// on the host for every chunk of a shape).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kq {

constexpr int CHUNK = 16;  // tile-diagonals per recursion leaf (chunk)

// tiles (I, J) with I + J = k, 0 <= I < Mt, 0 <= J < Nt: rows [lo, hi]
__host__ __device__ inline int diag_lo(int k, int Nt) { return k - Nt + 1 > 0 ? k - Nt + 1 : 0; }
__host__ __device__ inline int diag_hi(int k, int Mt) { return k < Mt - 1 ? k : Mt - 1; }
__host__ __device__ inline int diag_tiles(int k, int Mt, int Nt) {
    const int c = diag_hi(k, Mt) - diag_lo(k, Nt) + 1;
    return c > 0 ? c : 0;
}

struct ChunkTask {
    int kind;  // 0: sweep, 1: precompute, -1: no task (the ticket is past the chunk)
    int Kt;    // the tile's diagonal
    int idx;   // position on the diagonal: I = diag_lo(Kt) + idx
};

// number of tasks of chunk [c0, c1)
__host__ __device__ inline int chunk_tasks(int c0, int c1, int Mt, int Nt) {
    int s = 0;
    for (int k = c0; k < c1; ++k) s += diag_tiles(k, Mt, Nt) * (k > c0 ? 2 : 1);
    return s;
}

__host__ __device__ inline ChunkTask chunk_task(int ticket, int c0, int c1, int Mt, int Nt) {
    int t = ticket;
    for (int g = 0; c0 + g < c1; ++g) {
        const int kp = c0 + g + 1;
        if (kp < c1) {
            const int np = diag_tiles(kp, Mt, Nt);
            if (t < np) return ChunkTask{1, kp, t};
            t -= np;
        }
        const int ns = diag_tiles(c0 + g, Mt, Nt);
        if (t < ns) return ChunkTask{0, c0 + g, t};
        t -= ns;
    }
    return ChunkTask{-1, 0, 0};
}

// the ticket of a task (the inverse of chunk_task)
__host__ __device__ inline int chunk_ticket(int kind, int Kt, int idx, int c0, int c1, int Mt, int Nt) {
    int t = 0;
    for (int g = 0; c0 + g < c1; ++g) {
        const int kp = c0 + g + 1;
        if (kp < c1) {
            if (kind == 1 && kp == Kt) return t + idx;
            t += diag_tiles(kp, Mt, Nt);
        }
        if (kind == 0 && c0 + g == Kt) return t + idx;
        t += diag_tiles(c0 + g, Mt, Nt);
    }
    return -1;
}

// The flags a task waits on, at fixed slots (so a kernel keeps them in
// registers): the flag word index (see below) or -1 where there is none.
// Slot 0 the tile before it in its row, slot 1 the one before it in its column
// (for a precompute task: two tiles before), slot 2 its own precompute task.
// Flag words: [0, Mt Nt) the sweep of tile (I, J) is done (word I Nt + J),
// [Mt Nt, 2 Mt Nt) its precompute task is done.
struct ChunkDeps {
    int w0, w1, w2;
};

__host__ __device__ inline ChunkDeps chunk_deps(const ChunkTask& tk, int c0, int Mt, int Nt) {
    const int I = diag_lo(tk.Kt, Nt) + tk.idx, J = tk.Kt - I;
    ChunkDeps d{-1, -1, -1};
    if (tk.kind == 0 && tk.Kt > c0) {
        d.w0 = J >= 1 ? I * Nt + J - 1 : -1;
        d.w1 = I >= 1 ? (I - 1) * Nt + J : -1;
        d.w2 = Mt * Nt + I * Nt + J;
    } else if (tk.kind == 1 && tk.Kt - 2 >= c0) {
        // older slices: row tiles (I, J') with I + J' in [c0, Kt - 2], column tiles likewise
        d.w0 = J >= 2 ? I * Nt + J - 2 : -1;
        d.w1 = I >= 2 ? (I - 2) * Nt + J : -1;
    }
    return d;
}

}  // namespace kq
