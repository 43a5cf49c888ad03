// Task order of the persistent chunk solver (FastKron page, section 2.3: the
// tiles of one tile-diagonal are independent; section 2.5: a chunk of
// tile-diagonals is solved before the band products that follow it).
//
// One launch solves the tile-diagonals [c0, c1) of a chunk.  Its workgroups
// draw tickets from one counter; ticket t names the sweep of a tile, in
// tile-diagonal order and, on a diagonal, by increasing row I.  The task of
// tile (I, J) on diagonal Kt first sums the tile's chunk products over every
// slice older than its two freshest ones, then the two freshest, then sweeps
// the tile.  It waits on per-tile flags, raised when a tile's sweep is done:
//   before the older slices  the tiles two before it in its row and column,
//                            (I, J - 2) and (I - 2, J), when they are in the chunk
//                            (each of those waited for the tile before it in its
//                            row and column, so every older slice is final too);
//   before the freshest      (I, J - 1) and (I - 1, J).
// Every task waits only on tasks with smaller tickets, and a workgroup waits
// only on the task it drew last, so the holder of the smallest unfinished
// ticket never waits on an unfinished task: the launch finishes whatever
// number of its workgroups is resident (tests/chunk_sched_check.cpp verifies
// the order on the host for every chunk of the configured shapes).
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
    int Kt;   // the tile's diagonal, or -1: no task (the ticket is past the chunk)
    int idx;  // position on the diagonal: I = diag_lo(Kt) + idx
};

// number of tasks of chunk [c0, c1)
__host__ __device__ inline int chunk_tasks(int c0, int c1, int Mt, int Nt) {
    int s = 0;
    for (int k = c0; k < c1; ++k) s += diag_tiles(k, Mt, Nt);
    return s;
}

__host__ __device__ inline ChunkTask chunk_task(int ticket, int c0, int c1, int Mt, int Nt) {
    int t = ticket;
    for (int k = c0; k < c1; ++k) {
        const int nk = diag_tiles(k, Mt, Nt);
        if (t < nk) return ChunkTask{k, t};
        t -= nk;
    }
    return ChunkTask{-1, 0};
}

// the ticket of the task of tile idx on diagonal Kt (the inverse of chunk_task)
__host__ __device__ inline int chunk_ticket(int Kt, int idx, int c0, int Mt, int Nt) {
    int t = 0;
    for (int k = c0; k < Kt; ++k) t += diag_tiles(k, Mt, Nt);
    return t + idx;
}

// The flags a task waits on, at fixed slots (so a kernel keeps them in
// registers): the flag word of a tile (word I Nt + J: the sweep of tile (I, J) is
// done), or -1 where there is none.  o0, o1 before the older slices; f0, f1
// before the freshest.
struct ChunkDeps {
    int o0, o1, f0, f1;
};

__host__ __device__ inline ChunkDeps chunk_deps(const ChunkTask& tk, int c0, int Nt) {
    const int I = diag_lo(tk.Kt, Nt) + tk.idx, J = tk.Kt - I;
    ChunkDeps d{-1, -1, -1, -1};
    if (tk.Kt - 2 >= c0) {  // older slices: row tiles (I, J') with I + J' in [c0, Kt - 2], column tiles likewise
        d.o0 = J >= 2 ? I * Nt + J - 2 : -1;
        d.o1 = I >= 2 ? (I - 2) * Nt + J : -1;
    }
    if (tk.Kt - 1 >= c0) {
        d.f0 = J >= 1 ? I * Nt + J - 1 : -1;
        d.f1 = I >= 1 ? (I - 1) * Nt + J : -1;
    }
    return d;
}

}  // namespace kq
