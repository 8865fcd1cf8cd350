// causal_map.h -- token positions of a causal share, shared by the forward and backward
// kernels (device code only).
//
// Causal mask (slowleelab "Ring Attention" page, 4.5 limitation 2: a query attends only
// to keys at or before its own position).  Member r's local token x sits at position
//   contiguous  r*l + x
//   striped     x*N + r                                   (4.8)
//   zigzag      r*h + x for x < h, (2N-1-r)*h + (x-h) after, h = l/2
// Positions grow with the local index inside each zigzag half, and a 64-key (or
// 64-query) tile never straddles a zigzag half-block (l % 128 == 0 is required).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

constexpr int32_t kLayoutContiguous = 0;
constexpr int32_t kLayoutStriped = 1;

struct CausalMap {
    int32_t layout, rank, N, l;

    __device__ __forceinline__ int32_t pos(int32_t member, int32_t x) const {
        if (layout == kLayoutContiguous) return member * l + x;
        if (layout == kLayoutStriped) return x * N + member;
        const int32_t hl = l >> 1;
        return x < hl ? member * hl + x : (2 * N - 1 - member) * hl + (x - hl);
    }
    __device__ __forceinline__ int32_t qpos(int32_t a) const { return pos(rank, a); }

    // Number of keys b0, b0+1, ... of block j that local query a may attend to (any sign;
    // callers clamp to the tile).  The keys of one tile are consecutive positions for the
    // contiguous and zigzag layouts; for the striped layout key x of block j sits at
    // x*N + j <= a*N + rank  <=>  x <= a - (j > rank).
    __device__ __forceinline__ int32_t allowed(int32_t a, int32_t j, int32_t b0) const {
        if (layout == kLayoutStriped) return a - (j > rank ? 1 : 0) - b0 + 1;
        return qpos(a) - pos(j, b0) + 1;
    }

    // Tiles of `tile` keys of block j that hold a key some query up to local index a_max may
    // attend to: always a prefix of the block.
    __device__ __forceinline__ int32_t active_tiles(int32_t j, int32_t a_max, int32_t tile,
                                                    int32_t tiles_per_blk) const {
        auto prefix = [tile](int32_t keys, int32_t cap) {  // tiles covering keys 0..keys-1
            return keys <= 0 ? 0 : min(cap, (keys + tile - 1) / tile);
        };
        if (layout == kLayoutStriped)
            return prefix(a_max - (j > rank ? 1 : 0) + 1, tiles_per_blk);
        const int32_t q = qpos(a_max);
        if (layout == kLayoutContiguous) return prefix(q - j * l + 1, tiles_per_blk);
        const int32_t hl = l >> 1, ht = hl / tile;
        return prefix(q - j * hl + 1, ht) + prefix(q - (2 * N - 1 - j) * hl + 1, ht);
    }

    // Smallest local query index whose position is at or after p (l if none).
    __device__ __forceinline__ int32_t first_query(int32_t p) const {
        if (layout == kLayoutContiguous) {
            const int32_t a = p - rank * l;
            return a < 0 ? 0 : (a > l ? l : a);
        }
        if (layout == kLayoutStriped) {
            const int32_t d = p - rank;
            if (d <= 0) return 0;
            const int32_t a = (d + N - 1) / N;
            return a > l ? l : a;
        }
        const int32_t hl = l >> 1;
        const int32_t lo0 = rank * hl, lo1 = (2 * N - 1 - rank) * hl;
        if (p <= lo0) return 0;
        if (p < lo0 + hl) return p - lo0;
        if (p <= lo1) return hl;
        if (p < lo1 + hl) return hl + (p - lo1);
        return l;
    }
};

}  // namespace ra
