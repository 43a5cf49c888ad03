// Task order of the persistent chunk solver (FastKron page, section 2.3: the
// tiles of one tile-diagonal are independent; section 2.5: a chunk of
// tile-diagonals is solved before the band products that follow it).
//
// One launch solves the tile-diagonals [c0, c1) of a chunk.  Its workgroups
// draw tickets from one counter; ticket t names the task of one tile, in
// tile-diagonal order and, on a diagonal, by increasing row I.  The task of
// tile (I, J) on diagonal Kt sums the tile's chunk products, first over every
// slice older than its two freshest ones, then over the freshest two, and
// sweeps the tile.  A slice is a swept tile's output: the errors D of (I, J')
// (a row slice) or the row-propagated errors RF of (I', J) (a column slice),
// for the tiles of the chunk before (I, J) in its row and column.  The task
// polls each value it reads until it is written (the values start as a pattern
// no result has), so it waits exactly for the tasks that write what it reads:
// tiles on earlier tile-diagonals, which have smaller tickets.  A workgroup
// waits only on the task it drew last, so the holder of the smallest
// unfinished ticket never waits on an unfinished task: the launch finishes
// whatever number of its workgroups is resident (tests/chunk_sched_check.cpp
// verifies the order on the host for every chunk of the configured shapes).
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

}  // namespace kq
