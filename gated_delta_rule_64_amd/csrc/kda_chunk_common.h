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

}  // namespace kda
