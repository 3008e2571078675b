// Device helpers shared by the draft and verify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

namespace specdec {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Per-(row, segment) summary written by the streaming passes: max logit m,
// sum of exp((l - m) / T) over the segment, and the argmax (lowest id on ties).
struct alignas(16) SegStat {
    float m;
    float s;
    int idx;
    int pad;
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Philox4x32 with ten rounds (Salmon, Moraes, Dror, Shaw, SC'11): the two
// multipliers act on counter words 0 and 2; the key advances by the Weyl
// increments after every round.  Only output word 0 is needed per draw.
__device__ __forceinline__ uint32_t philox10_word0(uint32_t x0, uint32_t x1, uint32_t x2,
                                                   uint32_t x3, uint32_t key0, uint32_t key1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint32_t a = 0xD2511F53u * x0;
        const uint32_t ah = __umulhi(0xD2511F53u, x0);
        const uint32_t b = 0xCD9E8D57u * x2;
        const uint32_t bh = __umulhi(0xCD9E8D57u, x2);
        x0 = bh ^ x1 ^ key0;
        x1 = b;
        x2 = ah ^ x3 ^ key1;
        x3 = a;
        key0 += 0x9E3779B9u;
        key1 += 0xBB67AE85u;
    }
    return x0;
}

// Uniform of request b, position k, stream (0 draft, 1 ratio test, 2 final):
// the top 24 bits of word 0 scaled by 2^-24, exact in fp32.
__device__ __forceinline__ float counter_uniform(uint64_t seed, uint32_t offset, uint32_t b,
                                                 uint32_t k, uint32_t stream) {
    const uint32_t w = philox10_word0(b, k, stream, offset, (uint32_t)seed,
                                      (uint32_t)(seed >> 32));
    return (float)(w >> 8) * 5.9604644775390625e-08f;
}

// (max, sum) pair merge for online softmax; sums are relative to their max.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2, float invT) {
    if (m2 > m) {
        s = s * __expf((m - m2) * invT) + s2;
        m = m2;
    } else if (m2 != -INFINITY) {
        s = s + s2 * __expf((m2 - m) * invT);
    }
}

// argmax merge with the lowest index on ties.
__device__ __forceinline__ void merge_arg(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// Full-wave reductions (wave64).
__device__ __forceinline__ void wave_reduce_stat(float& m, float& s, int& idx, float invT) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        float m2 = __shfl_xor(m, off);
        float s2 = __shfl_xor(s, off);
        int i2 = __shfl_xor(idx, off);
        float mv = m;
        int iv = idx;
        merge_arg(mv, iv, m2, i2);
        merge_ms(m, s, m2, s2, invT);
        idx = iv;
    }
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// A 64-bit value moved through a DPP lane pattern, both halves with the same
// control; lanes whose source is outside the pattern (or whose row is masked
// off) read 0.
template <int CTRL, int ROWM = 0xF, int BANKM = 0xF, bool BC = true>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWM, BANKM, BC);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWM, BANKM, BC);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143, kDppWaveShr1 = 0x138;

__device__ __forceinline__ double readlane_f64(double x, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum across the wave (lane order), Hillis-Steele on DPP:
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then the total of row
// 0 into rows 1 and 3 and the total of rows 0-1 into rows 2 and 3.
__device__ __forceinline__ double wave_inclusive_scan_f64(double x) {
    x += dpp_f64<kDppRowShr1>(x);
    x += dpp_f64<kDppRowShr2>(x);
    x += dpp_f64<kDppRowShr4>(x);
    x += dpp_f64<kDppRowShr8>(x);
    x += dpp_f64<kDppRowBcast15, 0xA, 0xF, false>(x);
    x += dpp_f64<kDppRowBcast31, 0xC, 0xF, false>(x);
    return x;
}

// Reductions across the 16 lanes of a DPP row (lanes 16i .. 16i+15): xor-1 and
// xor-2 quad permutes, then the half-row and row mirrors; every lane of the
// row ends with the result.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int x) {
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within each 16 lanes

__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_mov<kDppXor1>(x));
    x = fmaxf(x, dpp_mov<kDppXor2>(x));
    x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
    return fmaxf(x, dpp_mov<kDppMirror>(x));
}

__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    x += dpp_mov<kDppHalfMirror>(x);
    return x + dpp_mov<kDppMirror>(x);
}

__device__ __forceinline__ int row16_min(int x) {
    x = min(x, dpp_mov<kDppXor1>(x));
    x = min(x, dpp_mov<kDppXor2>(x));
    x = min(x, dpp_mov<kDppHalfMirror>(x));
    return min(x, dpp_mov<kDppMirror>(x));
}

// Sum over each group of 8 lanes (8i .. 8i + 7); every lane of the group ends
// with it.
__device__ __forceinline__ float row8_sum(float x) {
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    return x + dpp_mov<kDppHalfMirror>(x);
}

// Wave-wide max and (max, lowest index among the lanes holding it), uniform.
__device__ __forceinline__ float readlane_f32(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ float wave_max_f32_dpp(float x) {
    x = row16_max(x);
    return fmaxf(fmaxf(readlane_f32(x, 0), readlane_f32(x, 16)),
                 fmaxf(readlane_f32(x, 32), readlane_f32(x, 48)));
}
__device__ __forceinline__ void wave_argmax_dpp(float& m, int& idx) {
    const float M = wave_max_f32_dpp(m);
    int cand = m == M ? idx : INT_MAX;
    cand = row16_min(cand);
    const int c = min(min(__builtin_amdgcn_readlane(cand, 0), __builtin_amdgcn_readlane(cand, 16)),
                      min(__builtin_amdgcn_readlane(cand, 32), __builtin_amdgcn_readlane(cand, 48)));
    m = M;
    idx = c;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait until at most n vector-memory operations of this wave are outstanding
// (expcnt and lgkmcnt left at their "no wait" maxima).  Direct global->LDS
// loads count here too; loads complete in issue order.  The s_waitcnt
// immediate holds vmcnt bits 3:0 at 3:0 and bits 5:4 at 15:14.
#define SPECDEC_VMCNT_IMM(n) (0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
#define SPECDEC_VMCNT_CASE(n) \
    case n: __builtin_amdgcn_s_waitcnt(SPECDEC_VMCNT_IMM(n)); break;
__device__ __forceinline__ void wait_vmcnt_le(int n) {
    switch (n) {
        SPECDEC_VMCNT_CASE(1) SPECDEC_VMCNT_CASE(2) SPECDEC_VMCNT_CASE(3)
        SPECDEC_VMCNT_CASE(4) SPECDEC_VMCNT_CASE(5) SPECDEC_VMCNT_CASE(6)
        SPECDEC_VMCNT_CASE(7) SPECDEC_VMCNT_CASE(8) SPECDEC_VMCNT_CASE(9)
        SPECDEC_VMCNT_CASE(10) SPECDEC_VMCNT_CASE(11) SPECDEC_VMCNT_CASE(12)
        SPECDEC_VMCNT_CASE(13) SPECDEC_VMCNT_CASE(14) SPECDEC_VMCNT_CASE(15)
        SPECDEC_VMCNT_CASE(16) SPECDEC_VMCNT_CASE(17) SPECDEC_VMCNT_CASE(18)
        SPECDEC_VMCNT_CASE(19) SPECDEC_VMCNT_CASE(20) SPECDEC_VMCNT_CASE(21)
        SPECDEC_VMCNT_CASE(22) SPECDEC_VMCNT_CASE(23) SPECDEC_VMCNT_CASE(24)
        SPECDEC_VMCNT_CASE(25) SPECDEC_VMCNT_CASE(26) SPECDEC_VMCNT_CASE(27)
        SPECDEC_VMCNT_CASE(28) SPECDEC_VMCNT_CASE(29) SPECDEC_VMCNT_CASE(30)
        SPECDEC_VMCNT_CASE(31) SPECDEC_VMCNT_CASE(32)
    default: __builtin_amdgcn_s_waitcnt(SPECDEC_VMCNT_IMM(0)); break;   // waiting for all is always safe
    }
}
#undef SPECDEC_VMCNT_CASE

// The same wait with a compile-time count (no branch).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt(SPECDEC_VMCNT_IMM(N));
}

// Accesses to data that workgroups on other XCDs read or wrote in the same
// launch.  With COH they are agent-scope relaxed atomics, which bypass the
// per-XCD caches (write-through stores, coherent loads), so no cache
// write-back or invalidate is needed around a grid barrier; without it they
// are plain accesses.  Wider values move as 64-bit halves.
template <bool COH, typename T>
__device__ __forceinline__ T coh_load(const T* p) {
    if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}
template <bool COH, typename T>
__device__ __forceinline__ void coh_store(T* p, T v) {
    if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}
template <bool COH>
__device__ __forceinline__ float4 coh_load_f32x4(const float* p) {
    if constexpr (COH) {
        const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
        const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return make_float4(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                           __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
    } else {
        return *reinterpret_cast<const float4*>(p);
    }
}
template <bool COH>
__device__ __forceinline__ void coh_store_f32x2(float* p, float a, float b) {
    if constexpr (COH) {
        const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
        __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *reinterpret_cast<float2*>(p) = make_float2(a, b);
    }
}
template <bool COH>
__device__ __forceinline__ SegStat coh_load_seg(const SegStat* p) {
    if constexpr (COH) {
        const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
        const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        SegStat x;
        x.m = __uint_as_float((uint32_t)a);
        x.s = __uint_as_float((uint32_t)(a >> 32));
        x.idx = (int)(uint32_t)b;
        x.pad = (int)(uint32_t)(b >> 32);
        return x;
    } else {
        return *p;
    }
}
template <bool COH>
__device__ __forceinline__ void coh_store_seg(SegStat* p, const SegStat& x) {
    if constexpr (COH) {
        uint64_t* q = reinterpret_cast<uint64_t*>(p);
        __hip_atomic_store(q, (uint64_t)__float_as_uint(x.m) | ((uint64_t)__float_as_uint(x.s) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 1, (uint64_t)(uint32_t)x.idx | ((uint64_t)(uint32_t)x.pad << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *p = x;
    }
}

// Inverse CDF over one weight per lane (lanes in token order): the lane whose
// interval [excl, incl) holds thr and thr - excl; past the end (rounding) the
// last lane with weight and +inf.  Neighbouring intervals share end points.
__device__ __forceinline__ int wave_pick(double w, double thr, double& rem) {
    const double incl = wave_inclusive_scan_f64(w);
    const double excl = dpp_f64<kDppWaveShr1>(incl);   // lane 0 reads 0
    unsigned long long hit = __ballot(w > 0.0 && thr >= excl && thr < incl);
    if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        rem = thr - readlane_f64(excl, l);
        return l;
    }
    const unsigned long long pos = __ballot(w > 0.0);
    rem = INFINITY;
    return pos ? 63 - __clzll((long long)pos) : 0;
}

}  // namespace specdec
