// Device helpers shared by the attention-forward kernels (product path only).
#pragma once
#include "fa_params.h"

namespace miattn {

// Where a workgroup's tile lives.
struct TileCoord {
    int b, h, kvh;          // sequence, query head, kv head
    int t;                  // q-tile index inside the sequence
    int64_t q0, kv0;        // first packed row of the sequence (0 for dense batches)
    int len_q, len_kv;      // sequence lengths
    int r0, r1;             // query rows [r0, r1) of the tile
    bool live;
};

// Decode the linear workgroup id.
//
// Work items are ordered (level, b, kv head, member of the GQA group), where level 0 holds
// the LAST q tile of every sequence: under a causal mask later tiles see more keys, so the
// heaviest tiles are dispatched first.  Workgroups are handed to the 8 XCDs round-robin
// (id mod 8), so the `group` query heads that share one kv head are given ids congruent
// mod 8: they run on the same XCD, back to back, and re-read that head's K/V tiles from
// the XCD's own L2.
__device__ inline TileCoord decode_tile(const FaParams& p, int L, int tile_m)
{
    TileCoord c;
    const int G = p.group;
    const int xcd = L & 7;
    const int s = L >> 3;
    const int gi = (s / G) * 8 + xcd;
    const int g = s - (s / G) * G;
    c.kvh = gi % p.Nkv;
    const int rest = gi / p.Nkv;
    c.b = rest % p.B;
    const int level = rest / p.B;
    c.live = level < p.n_levels;
    c.h = c.kvh * G + g;
    c.t = p.n_levels - 1 - level;
    c.q0 = 0;
    c.kv0 = 0;
    c.len_q = p.Sq;
    c.len_kv = p.Skv;
    if (c.live && p.cu_q) {
        c.q0 = c.b ? p.cu_q[c.b - 1] : 0;
        c.kv0 = c.b ? p.cu_kv[c.b - 1] : 0;
        c.len_q = (int)(p.cu_q[c.b] - c.q0);
        c.len_kv = (int)(p.cu_kv[c.b] - c.kv0);
    }
    if (c.live && (int64_t)c.t * tile_m >= c.len_q) c.live = false;
    // Tiles end at the sequence end: the ragged tile is the first one (the rows that see the
    // fewest keys under a causal mask), and the heaviest tiles are full.
    const int pad = (tile_m - c.len_q % tile_m) % tile_m;
    c.r0 = max(0, c.t * tile_m - pad);
    c.r1 = min(c.len_q, (c.t + 1) * tile_m - pad);
    return c;
}

// The visible keys of one sequence: row i sees key j when -pre <= j - i <= next (the band,
// already shifted to the sequence's diagonal) or j < pfx (the prefix).  The prefix is only
// given with an unbounded pre, so every row's visible keys form one range
// [max(0, i - pre), min(len_kv, max(i + next, pfx - 1) + 1)).
struct Band {
    int64_t pre, next, pfx;
};

__device__ inline Band band_of(const FaParams& p, const TileCoord& tc)
{
    const int64_t off = p.align_br ? (int64_t)tc.len_kv - tc.len_q : 0;
    Band bd;
    bd.pre = p.pre - off;
    bd.next = p.next + off;
    bd.pfx = 0;
    if (p.prefix) {
        const int64_t x = p.prefix[tc.b];
        bd.pfx = x < 0 ? 0 : (x > tc.len_kv ? tc.len_kv : x);
    }
    return bd;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011): ten rounds of two 32x32->64-bit
// products by 0xD2511F53 and 0xCD9E8D57, the key bumped by 0x9E3779B9 / 0xBB67AE85 between
// rounds.  Dropout draws the byte of probability (i, j) of head h in sequence / batch entry
// b from counter (j / 16, i, h + 256 b, offset): byte j % 4 of output word (j % 16) / 4.
__device__ inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1)
{
    #pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        // three-input XORs as one v_bitop3_b32 each (truth table 0x96: odd parity)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], k1, 0x96);
        c[0] = n0;
        c[1] = (uint32_t)p1;
        c[2] = n2;
        c[3] = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// Visible key range [lo, hi) of query rows [r0, r1).
__device__ inline void key_range(const Band& bd, int r0, int r1, int len_kv, int& lo, int& hi)
{
    int64_t a = (int64_t)r0 - bd.pre;
    int64_t z = (int64_t)(r1 - 1) + bd.next;
    if (bd.pfx > 0) {
        a = a < 0 ? a : 0;
        z = z > bd.pfx - 1 ? z : bd.pfx - 1;
    }
    z += 1;
    lo = a < 0 ? 0 : (a > len_kv ? len_kv : (int)a);
    hi = z < 0 ? 0 : (z > len_kv ? len_kv : (int)z);
}

}  // namespace miattn
