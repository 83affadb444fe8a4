// sv_philox.hpp -- the counter-based generator behind every random draw of
// lossless verification: Philox4x32-10, the stream layout (which counter a
// draw uses) and the maps from a 32-bit word to a uniform on the 2^-24
// lattice.
#pragma once

#include "sv_common.hpp"

namespace sv {

// --------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies by fixed odd multipliers on counter words 0 and 2,
// with the products' high halves mixed into the other two words and the
// round key; the key advances by two Weyl constants after every round.
// --------------------------------------------------------------------------
struct PhiloxKey {
    uint32_t lo, hi;
};

__device__ __forceinline__ PhiloxKey philox_key(uint64_t seed) {
    return PhiloxKey{static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32)};
}

__device__ __forceinline__ uint4 philox10(uint4 c, PhiloxKey k) {
    uint32_t k0 = k.lo, k1 = k.hi;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t a = static_cast<uint64_t>(0xD2511F53u) * c.x;
        const uint64_t b = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
        // three-input XORs in one instruction each (truth table 0x96: odd parity)
        c = make_uint4(__builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(b >> 32), c.y, k0, 0x96),
                       static_cast<uint32_t>(b),
                       __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(a >> 32), c.w, k1, 0x96),
                       static_cast<uint32_t>(a));
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// Stream tags (fourth counter word).
constexpr uint32_t kTagAccept = 1u;
constexpr uint32_t kTagRace = 2u;
constexpr uint32_t kTagScreen = 3u;

__device__ __forceinline__ uint32_t pick_word(const uint4 &r, uint32_t w) {
    return w == 0 ? r.x : (w == 1 ? r.y : (w == 2 ? r.z : r.w));
}

// One draw for vocabulary id x at (position, sequence, tag).
__device__ __forceinline__ uint32_t draw_u32(PhiloxKey k, uint32_t x, uint32_t pos, uint32_t seq,
                                             uint32_t tag) {
    return pick_word(philox10(make_uint4(x >> 2, pos, seq, tag), k), x & 3u);
}

// The race's word for id x is made of two independent draws: its high 16
// bits come from the screening stream, whose block at counter
// (x>>3, pos, seq, kTagScreen) serves eight consecutive ids (half x&1 of word
// (x>>1)&3), its low 16 bits are the high half of the race stream's draw.
// A sampler can bound an id's largest key from the screening bits alone, one
// block per eight ids, and draw the race stream only for ids that could win.
__device__ __forceinline__ uint32_t screen_half(const uint4 &s, uint32_t x) {
    return (pick_word(s, (x >> 1) & 3u) >> (16u * (x & 1u))) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t race_word_of(uint32_t hi16, uint32_t race_draw) {
    return (hi16 << 16) | (race_draw >> 16);
}
__device__ __forceinline__ uint32_t race_word(PhiloxKey k, uint32_t x, uint32_t pos,
                                              uint32_t seq) {
    const uint4 s = philox10(make_uint4(x >> 3, pos, seq, kTagScreen), k);
    return race_word_of(screen_half(s, x), draw_u32(k, x, pos, seq, kTagRace));
}

// The 23 leading bits on the odd points of the 2^-24 grid: (2k+1) 2^-24,
// exact in float and double, never 0 or 1.
__device__ __forceinline__ float lattice_u32f(uint32_t r) {
    return fmaf(static_cast<float>(r >> 9), 0x1.0p-23f, 0x1.0p-24f);
}
__device__ __forceinline__ double lattice_u64(uint32_t r) {
    return (2.0 * static_cast<double>(r >> 9) + 1.0) * 0x1.0p-24;
}

// Leading one bits of a Philox word.  With u its lattice uniform
// (2k+1) 2^-24 and n = min(leading ones, 23): 1 - u >= 2^(-1-n), and since
// E = -ln u >= 1 - u, -log2(E / ln 2) <= 1 + n + log2(ln 2) < 0.472 + n.
// Counts at most 31 (the bound only needs min(., 23)): ~r | 1 is never 0.
__device__ __forceinline__ int leading_ones(uint32_t r) { return __builtin_clz(~r | 1u); }
// Leading one bits of id x's 16 screening bits (the high half of its race
// word) as a float: exact below 16, and 2^32 - 1 when all 16 are ones, i.e.
// above every count a whole word can have, so that a test "ones >= a" keeps
// each id whose screening bits alone cannot rule it out.  The field is moved
// to the top of a word with zeros below, whose leading zeros v_ffbh_u32
// counts (all ones for a zero word).
__device__ __forceinline__ float screen_ones(const uint4 &s, uint32_t x) {
    const uint32_t w = ~pick_word(s, (x >> 1) & 3u);
    const uint32_t y = (x & 1u) ? (w & 0xFFFF0000u) : (w << 16);
    uint32_t n;
    asm("v_ffbh_u32 %0, %1" : "=v"(n) : "v"(y));
    return static_cast<float>(n);
}

}  // namespace sv
