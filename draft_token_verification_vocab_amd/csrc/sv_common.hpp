// sv_common.hpp -- shared device helpers of the specverify HIP library:
// element traits for 16-byte row loads, the fast transcendental wrappers and
// the wave reductions (the Philox generator is in sv_philox.hpp).
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

namespace sv {

constexpr int kWave = 64;
constexpr double kLn2 = 0.69314718055994530942;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr float kLog2e = 1.44269504088896340736f;
// Finite stand-in for "no maximum yet"; |l * log2(e)/T| stays far below it
// for the supported temperature range.
constexpr float kNoMax = -1.0e30f;
// Terms 2^d with d below this are exactly zero in float; clamping d keeps the
// entropy accumulator free of 0 * (-inf) for masked (-inf) logits.
constexpr float kMinExp2 = -200.0f;
// Most ids a bonus-candidate list (the row pass's list of the ids a draw from
// p at a row could pick) holds; a row with more is raced in full.
constexpr int kMaxBonusCand = 64;

// 16-byte streaming load with the non-temporal hint: logits rows are read
// exactly once, and on gfx950 the hint lifts a one-pass stream from ~6.0 to
// ~7.0 TB/s.
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
    const v4u32 r = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(p));
    return make_uint4(r.x, r.y, r.z, r.w);
}
// The same load at a wave-uniform base plus a 32-bit per-lane byte offset,
// the form the hardware addresses with a scalar base register.
__device__ __forceinline__ uint4 load_stream_at(const void *base, uint32_t byte_off) {
    return load_stream(reinterpret_cast<const uint4 *>(static_cast<const char *>(base) + byte_off));
}

// Buffer-addressed streaming loads: a resource descriptor over `bytes` bytes
// at `base` (raw buffer, no stride; the third descriptor word is the gfx9
// family's data-format field), then 16-byte non-temporal loads at a per-lane
// byte offset `voff` plus a wave-uniform byte offset `soff`.  A loop that
// advances only `soff` keeps its addressing in scalar registers: no 64-bit
// vector address arithmetic per load.  Every load must lie inside the
// described range.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes),
                                             0x00020000);
}
constexpr int kCachePolicyNT = 2;  // the non-temporal bit of a buffer load's cache policy
__device__ __forceinline__ uint4 load_stream_buf(buf_rsrc r, uint32_t voff, uint32_t soff) {
    const v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                                          static_cast<int>(soff), kCachePolicyNT);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Maximum of three floats in one v_max3_f32.  Written as an instruction so
// that a chain of them stays a chain: the compiler neither inserts operand
// canonicalisations (logits enter as reinterpreted integer bits) nor reshapes
// the chain into a tree of two-input maxima.  Operands are not NaN.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// x * y rounded to float.  Device code is compiled with floating-point
// contraction on, which may fuse a product into a following add or subtract
// even when the product has other uses; where the rounded product itself is
// the operand (a log2-normaliser m*c whose rounding residue is tracked
// apart), it must stay a separate multiply.
__device__ __forceinline__ float mul_rn(float x, float y) {
#pragma clang fp contract(off)
    return x * y;
}

// Raw hardware transcendentals (v_exp_f32 / v_log_f32: base 2, ~1 ulp).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// --------------------------------------------------------------------------
// Element traits: one 16-byte vector holds 8 bfloat16 or 4 float logits.
// --------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bfloat16 bit patterns
    static constexpr int kPerVec = 8;
    // Padding past the row's end: -1.996e30 (bfloat16 0xF1C9), below every
    // logit the passes take as finite (they treat logits <= -1e30 as -inf)
    // yet finite, so 2^(pad*c - m*c) is 0 and its entropy term 0 * d is 0.
    static constexpr uint32_t kPadPair = 0xF1C9F1C9u;
    __device__ static __forceinline__ void unpack(const uint4 &v, float *x) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    __device__ static __forceinline__ float at(const uint16_t *row, int i) {
        return __uint_as_float(static_cast<uint32_t>(row[i]) << 16);
    }
    // Element k of a vector (k a constant after unrolling).
    __device__ static __forceinline__ float elem(const uint4 &v, int k) {
        const uint32_t w = k / 2 == 0 ? v.x : (k / 2 == 1 ? v.y : (k / 2 == 2 ? v.z : v.w));
        return __uint_as_float(k % 2 == 0 ? w << 16 : w & 0xFFFF0000u);
    }
    // Vector `vi` of a row whose last vector is only partly inside V.
    __device__ static __forceinline__ uint4 partial(const uint16_t *row, int vi, int V) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e0 = vi * 8 + 2 * i, e1 = e0 + 1;
            uint32_t lo = e0 < V ? row[e0] : 0xF1C9u;
            uint32_t hi = e1 < V ? row[e1] : 0xF1C9u;
            w[i] = lo | (hi << 16);
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
    static constexpr uint32_t pad_word() { return kPadPair; }
};

template <>
struct Elem<float> {
    static constexpr int kPerVec = 4;
    __device__ static __forceinline__ void unpack(const uint4 &v, float *x) {
        x[0] = __uint_as_float(v.x);
        x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z);
        x[3] = __uint_as_float(v.w);
    }
    __device__ static __forceinline__ float at(const float *row, int i) { return row[i]; }
    __device__ static __forceinline__ float elem(const uint4 &v, int k) {
        return __uint_as_float(k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w)));
    }
    __device__ static __forceinline__ uint4 partial(const float *row, int vi, int V) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e = vi * 4 + i;
            w[i] = e < V ? __float_as_uint(row[e]) : 0xF1C9F2CAu;  // -2e30, as above
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
    static constexpr uint32_t pad_word() { return 0xF1C9F2CAu; }
};

__device__ __forceinline__ int clamp_len(int L, int K) { return L < 0 ? 0 : (L > K ? K : L); }

// --------------------------------------------------------------------------
// Wave-wide reductions with DPP row shifts and row broadcasts (a
// Hillis-Steele scan inside each 16-lane row, then rows 0..3 folded with
// row_bcast15 / row_bcast31).  The total lands in lane 63 and is returned to
// every lane.  Lanes without a source read the identity (0 bits).
// --------------------------------------------------------------------------
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_pull(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, false));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_pull64(uint64_t v) {
    const uint32_t lo = dpp_pull<CTRL, ROWS>(static_cast<uint32_t>(v));
    const uint32_t hi = dpp_pull<CTRL, ROWS>(static_cast<uint32_t>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t lane63_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), 63);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), 63);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Maximum of an unsigned 32-bit value over the wave (lanes without a DPP
// source read 0, the identity).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    uint32_t o;
    o = dpp_pull<0x111, 0xF>(v); v = o > v ? o : v;  // row_shr:1
    o = dpp_pull<0x112, 0xF>(v); v = o > v ? o : v;  // row_shr:2
    o = dpp_pull<0x114, 0xF>(v); v = o > v ? o : v;  // row_shr:4
    o = dpp_pull<0x118, 0xF>(v); v = o > v ? o : v;  // row_shr:8
    o = dpp_pull<0x142, 0xA>(v); v = o > v ? o : v;  // row_bcast15
    o = dpp_pull<0x143, 0xC>(v); v = o > v ? o : v;  // row_bcast31
    return __builtin_amdgcn_readlane(v, 63);
}

// Maximum of an unsigned 64-bit key over the wave.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t o;
    o = dpp_pull64<0x111, 0xF>(v); v = o > v ? o : v;  // row_shr:1
    o = dpp_pull64<0x112, 0xF>(v); v = o > v ? o : v;  // row_shr:2
    o = dpp_pull64<0x114, 0xF>(v); v = o > v ? o : v;  // row_shr:4
    o = dpp_pull64<0x118, 0xF>(v); v = o > v ? o : v;  // row_shr:8
    o = dpp_pull64<0x142, 0xA>(v); v = o > v ? o : v;  // row_bcast15
    o = dpp_pull64<0x143, 0xC>(v); v = o > v ? o : v;  // row_bcast31
    return lane63_u64(v);
}

// Sum of an unsigned 64-bit integer over the wave (exact in any order).
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
    v += dpp_pull64<0x111, 0xF>(v);
    v += dpp_pull64<0x112, 0xF>(v);
    v += dpp_pull64<0x114, 0xF>(v);
    v += dpp_pull64<0x118, 0xF>(v);
    v += dpp_pull64<0x142, 0xA>(v);
    v += dpp_pull64<0x143, 0xC>(v);
    return lane63_u64(v);
}

// Adds v into sh[key] for every active lane, one LDS atomic per distinct key
// in the wave: lanes sharing a key are summed first (exact integer sums).
// Call from wave-uniform control flow.
__device__ __forceinline__ void wave_keyed_add(unsigned long long *sh, int key, uint64_t v,
                                               bool active) {
    uint64_t todo = __ballot(active);
    const int lane = threadIdx.x & (kWave - 1);
    while (todo) {
        const int leader = __ffsll(static_cast<long long>(todo)) - 1;
        const int q = __shfl(key, leader, kWave);
        const bool mine = active && key == q;
        const uint64_t grp = __ballot(mine);
        const uint64_t sum = wave_sum_u64(mine ? v : 0ull);
        if (lane == leader) atomicAdd(&sh[q], static_cast<unsigned long long>(sum));
        todo &= ~grp;
    }
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_pull_f(float v) {
    return __uint_as_float(dpp_pull<CTRL, ROWS>(__float_as_uint(v)));
}

// Sum of a float over the wave (each lane's value counts once).
__device__ __forceinline__ float wave_sum_f32(float x) {
    x += dpp_pull_f<0x111, 0xF>(x);  // row_shr:1
    x += dpp_pull_f<0x112, 0xF>(x);  // row_shr:2
    x += dpp_pull_f<0x114, 0xF>(x);  // row_shr:4
    x += dpp_pull_f<0x118, 0xF>(x);  // row_shr:8
    x += dpp_pull_f<0x142, 0xA>(x);  // row_bcast15
    x += dpp_pull_f<0x143, 0xC>(x);  // row_bcast31
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 63));
}

// Sums of two floats over the wave, step by step together, so that the two
// dependency chains interleave.
__device__ __forceinline__ void wave_sum2_f32(float &x, float &y) {
    x += dpp_pull_f<0x111, 0xF>(x);
    y += dpp_pull_f<0x111, 0xF>(y);
    x += dpp_pull_f<0x112, 0xF>(x);
    y += dpp_pull_f<0x112, 0xF>(y);
    x += dpp_pull_f<0x114, 0xF>(x);
    y += dpp_pull_f<0x114, 0xF>(y);
    x += dpp_pull_f<0x118, 0xF>(x);
    y += dpp_pull_f<0x118, 0xF>(y);
    x += dpp_pull_f<0x142, 0xA>(x);
    y += dpp_pull_f<0x142, 0xA>(y);
    x += dpp_pull_f<0x143, 0xC>(x);
    y += dpp_pull_f<0x143, 0xC>(y);
    x = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 63));
    y = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(y), 63));
}

// Maximum of a non-negative double over the wave (such doubles order like
// their bit patterns).
__device__ __forceinline__ double wave_max_f64_nonneg(double x) {
    return __longlong_as_double(static_cast<long long>(
        wave_max_u64(static_cast<uint64_t>(__double_as_longlong(x)))));
}

// Sum of a double over the wave, in a fixed order.
__device__ __forceinline__ double wave_sum_f64(double x) {
    uint64_t v = static_cast<uint64_t>(__double_as_longlong(x));
    auto add = [](uint64_t a, uint64_t b) {
        return static_cast<uint64_t>(__double_as_longlong(
            __longlong_as_double(static_cast<long long>(a)) +
            __longlong_as_double(static_cast<long long>(b))));
    };
    v = add(v, dpp_pull64<0x111, 0xF>(v));
    v = add(v, dpp_pull64<0x112, 0xF>(v));
    v = add(v, dpp_pull64<0x114, 0xF>(v));
    v = add(v, dpp_pull64<0x118, 0xF>(v));
    v = add(v, dpp_pull64<0x142, 0xA>(v));
    v = add(v, dpp_pull64<0x143, 0xC>(v));
    return __longlong_as_double(static_cast<long long>(lane63_u64(v)));
}

// Order-preserving map of a float onto unsigned integers.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

}  // namespace sv
