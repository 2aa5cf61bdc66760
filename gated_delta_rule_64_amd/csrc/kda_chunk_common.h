// Chunk geometry shared by the chunked forward and backward kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int C = 64;   // chunk rows

// byte offset of the chunk table inside the schedule
inline size_t sched_table_offset(int N) { return ((size_t)(3 * (size_t)N + 1) * 4 + 15) / 16 * 16; }

// Chunk c as (first row in the [B*T] row space, rows). Dense mode (no offsets): chunk c
// is chunk c % NT of sequence c / NT, computed here; packed mode: the schedule's table.
__device__ __forceinline__ int2 chunk_pos(bool dense, int NT, int T, const int2* table, int c) {
    if (dense) {
        const int ci = c % NT;
        return make_int2((c / NT) * T + ci * C, T - ci * C < C ? T - ci * C : C);
    }
    return table[c];
}

__device__ __forceinline__ int xcd_remap(int b, int G) {
    // blocks are dealt round-robin to the 8 XCDs; give each XCD a contiguous run of
    // work items so neighbouring items (same chain, same chunk) share an L2
    if (G % 8 != 0) return b;
    return (b % 8) * (G / 8) + b / 8;
}

// Offset of the packed schedule's slot order (int32 [N], slots by descending chunk count)
// in the schedule region: after the chunk table.
inline size_t sched_order_offset(int N, int NCmax) { return sched_table_offset(N) + (size_t)NCmax * 8; }

// Work item of a serial scan block b (G = chains * NVT blocks, NVT column slices per
// chain): its column slice vt, value head hv and sequence n. Without an order (dense
// mode) items follow xcd_remap. With the packed schedule's order, chains are walked
// longest sequence first, their ranks dealt round-robin to the 8 XCDs (block b runs on
// XCD b % 8) and each chain's slices kept on one XCD: the blocks dispatched first hold
// the longest chains, so short ones fill in behind them instead of a long one starting
// last.
__device__ __forceinline__ void scan_item(int b, int G, int NVT, int HV, const int32_t* order, int& vt,
                                          int& hv, int& n) {
    int chain;
    if (order == nullptr) {
        const int item = xcd_remap(b, G);
        vt = item % NVT;
        chain = item / NVT;
    } else if (G % 8 == 0 && (G / 8) % NVT == 0) {
        const int j = b / 8;
        vt = j % NVT;
        chain = (j / NVT) * 8 + b % 8;
    } else {
        vt = b % NVT;
        chain = b / NVT;
    }
    hv = chain % HV;
    n = chain / HV;
    if (order != nullptr) n = order[n];
}

}  // namespace kda
