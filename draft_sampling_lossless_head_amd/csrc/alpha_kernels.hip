// Acceptance rate and total variation of each drafted position ("Speculative
// Decoding Part 1", section "수락 규칙": a token drawn from q passes the ratio
// test with probability sum_v min(p(v), q(v)), which equals 1 - D_TV(p, q)).
//
// One workgroup per (request b, position k < L_b), two passes over the target
// row p_k and the draft row q_k:
//   1. per row the max of the logits and sum exp((l - max) / T) (greedy: the
//      argmax, lowest id on ties);
//   2. sum_v min(p(v), q(v)) with p = exp((l_p - m_p) / T) / Z_p and q
//      likewise, as one exponential of the smaller exponent per token; the
//      total variation is 1 - alpha.
// Per-thread sums are fp32 (a few hundred terms each), the workgroup sums
// fp64.  At T = 0 both distributions are one-hot at their argmax, so alpha is
// 1 when the two argmaxes agree and 0 otherwise.
#include <climits>

#include "device_common.hpp"
#include "launch.hpp"

namespace specdec {

constexpr int kAlphaThreads = 256;

template <bool BF16>
__device__ __forceinline__ float logit_at(const void* base, size_t i) {
    if constexpr (BF16) return bf16_bits_to_float(static_cast<const uint16_t*>(base)[i]);
    else return static_cast<const float*>(base)[i];
}

// Eight logits from element i on (i % 8 == 0, 16-byte aligned rows).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <bool BF16>
__device__ __forceinline__ void logits8(const void* base, size_t i, float (&x)[8]) {
    if constexpr (BF16) {
        const u32x4_t w = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + i));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(w[j] << 16);
            x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    } else {
        const f32x4_t* f = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + i);
        const f32x4_t a = __builtin_nontemporal_load(f), b = __builtin_nontemporal_load(f + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = a[j];
            x[4 + j] = b[j];
        }
    }
}

// Running (max, sum of 2^((x - max) sc)) and (max, lowest argmax) of one row.
struct RowRun {
    float m, s;
    int idx;
};

__device__ __forceinline__ void run_add(RowRun& r, const float (&x)[8], int v0, int n, float sc,
                                        bool greedy) {
    float cm = -INFINITY;
    int ci = INT_MAX;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < n && x[j] > cm) {   // strict: the lowest id among equal values
            cm = x[j];
            ci = v0 + j;
        }
    }
    if (cm > r.m || (cm == r.m && ci < r.idx)) r.idx = ci;
    if (greedy) {
        r.m = fmaxf(r.m, cm);
        return;
    }
    const float nm = fmaxf(r.m, cm);
    if (nm == -INFINITY) return;   // nothing finite yet
    float add = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < n) add += __builtin_amdgcn_exp2f((x[j] - nm) * sc);
    r.s = r.s * __builtin_amdgcn_exp2f((r.m - nm) * sc) + add;
    r.m = nm;
}

// Workgroup merge of one RowRun per thread: every thread gets the result.
__device__ __forceinline__ RowRun block_merge(RowRun r, float invT, float* lds_m, float* lds_s,
                                              int* lds_i) {
    wave_reduce_stat(r.m, r.s, r.idx, invT);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        lds_m[wave] = r.m;
        lds_s[wave] = r.s;
        lds_i[wave] = r.idx;
    }
    __syncthreads();
    // the waves' results merged in a fixed order: (max, sum), and (max, lowest argmax)
    float m = lds_m[0], s = lds_s[0], am = lds_m[0];
    int idx = lds_i[0];
    for (int w = 1; w < kAlphaThreads / 64; ++w) {
        merge_ms(m, s, lds_m[w], lds_s[w], invT);
        merge_arg(am, idx, lds_m[w], lds_i[w]);
    }
    __syncthreads();
    return RowRun{m, s, idx};
}

__device__ __forceinline__ double block_sum_f64(double x, double* lds) {
    x = wave_sum_f64(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) lds[wave] = x;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kAlphaThreads / 64; ++w) t += lds[w];
    __syncthreads();
    return t;
}

template <bool PB, bool QB, bool VEC>
__global__ __launch_bounds__(kAlphaThreads)
void acceptance_rate_rows(AlphaArgs A) {
    __shared__ float lds_m[kAlphaThreads / 64], lds_s[kAlphaThreads / 64];
    __shared__ int lds_i[kAlphaThreads / 64];
    __shared__ double lds_d[kAlphaThreads / 64];
    const int G = A.gamma_max, V = A.V;
    const int b = (int)(blockIdx.x / (unsigned)G), k = (int)(blockIdx.x % (unsigned)G);
    const int tid = threadIdx.x;
    const size_t oi = (size_t)b * G + k;
    const int L = A.lens ? A.lens[b] : G;
    if (L < 0 || L > G || k >= L) {   // no such position, or an invalid length
        if (tid == 0) {
            A.alpha[oi] = NAN;
            if (A.tv) A.tv[oi] = NAN;
        }
        return;
    }
    const size_t prow = (size_t)((A.p_row_off ? A.p_row_off[b] : (int64_t)b * (G + 1)) + k);
    const size_t qrow = (size_t)((A.q_row_off ? A.q_row_off[b] : (int64_t)b * G) + k);
    const size_t p0 = prow * (size_t)V, q0 = qrow * (size_t)V;
    const float invT = A.invT;
    const float sc = invT * 1.4426950408889634f;   // exp(y / T) = 2^(y sc)
    const bool greedy = A.greedy != 0;

    // 1. normalisers (or argmaxes) of both rows
    RowRun rp{-INFINITY, 0.0f, INT_MAX}, rq{-INFINITY, 0.0f, INT_MAX};
    float x[8], y[8];
    if constexpr (VEC) {
        for (int v = tid * 8; v < V; v += kAlphaThreads * 8) {
            logits8<PB>(A.P, p0 + v, x);
            logits8<QB>(A.Q, q0 + v, y);
            run_add(rp, x, v, 8, sc, greedy);
            run_add(rq, y, v, 8, sc, greedy);
        }
    } else {
        for (int v = tid * 8; v < V; v += kAlphaThreads * 8) {
            const int n = min(8, V - v);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                x[j] = j < n ? logit_at<PB>(A.P, p0 + v + j) : -INFINITY;
                y[j] = j < n ? logit_at<QB>(A.Q, q0 + v + j) : -INFINITY;
            }
            run_add(rp, x, v, n, sc, greedy);
            run_add(rq, y, v, n, sc, greedy);
        }
    }
    const RowRun P = block_merge(rp, invT, lds_m, lds_s, lds_i);
    const RowRun Q = block_merge(rq, invT, lds_m, lds_s, lds_i);
    if (P.m == -INFINITY || Q.m == -INFINITY) {   // a row without a finite logit
        if (tid == 0) {
            A.alpha[oi] = NAN;
            if (A.tv) A.tv[oi] = NAN;
        }
        return;
    }
    if (greedy) {
        if (tid == 0) {
            const float a = P.idx == Q.idx ? 1.0f : 0.0f;
            A.alpha[oi] = a;
            if (A.tv) A.tv[oi] = 1.0f - a;
        }
        return;
    }

    // 2. alpha = sum_v min(p(v), q(v)) with min(2^a, 2^b) = 2^min(a, b): one
    //    exponential per token, the exponents a = l_p sc - (m_p sc + log2 Z_p)
    //    with the offset as an fp32 (hi, lo) pair (the same rounded sc scales
    //    the logits and the row max, so its rounding cancels in l - m).  TV is
    //    1 - alpha (sum |p - q| = sum p + sum q - 2 sum min(p, q)).
    const double op = (double)P.m * (double)sc + log2((double)P.s);
    const double oq = (double)Q.m * (double)sc + log2((double)Q.s);
    const float op_hi = (float)op, op_lo = (float)(op - (double)op_hi);
    const float oq_hi = (float)oq, oq_lo = (float)(oq - (double)oq_hi);
    float amin = 0.0f;
    auto add8 = [&](int n) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < n) {
                const float ea = fmaf(x[j], sc, -op_hi) - op_lo;
                const float eb = fmaf(y[j], sc, -oq_hi) - oq_lo;
                amin += __builtin_amdgcn_exp2f(fminf(ea, eb));
            }
        }
    };
    if constexpr (VEC) {
        for (int v = tid * 8; v < V; v += kAlphaThreads * 8) {
            logits8<PB>(A.P, p0 + v, x);
            logits8<QB>(A.Q, q0 + v, y);
            add8(8);
        }
    } else {
        for (int v = tid * 8; v < V; v += kAlphaThreads * 8) {
            const int n = min(8, V - v);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                x[j] = j < n ? logit_at<PB>(A.P, p0 + v + j) : -INFINITY;
                y[j] = j < n ? logit_at<QB>(A.Q, q0 + v + j) : -INFINITY;
            }
            add8(n);
        }
    }
    const double smin = block_sum_f64((double)amin, lds_d);
    if (tid == 0) {
        A.alpha[oi] = (float)smin;
        if (A.tv) A.tv[oi] = (float)(1.0 - smin);
    }
}

template <bool PB, bool QB>
static void launch_alpha_t(const AlphaArgs& a, bool vec, hipStream_t s) {
    const unsigned grid = (unsigned)((size_t)a.B * a.gamma_max);
    if (vec) hipLaunchKernelGGL((acceptance_rate_rows<PB, QB, true>), dim3(grid), dim3(kAlphaThreads), 0, s, a);
    else hipLaunchKernelGGL((acceptance_rate_rows<PB, QB, false>), dim3(grid), dim3(kAlphaThreads), 0, s, a);
}

hipError_t acceptance_rate_launch(const AlphaArgs& a, hipStream_t s) {
    if ((size_t)a.B * a.gamma_max == 0) return hipSuccess;
    // 16-byte vectors: every row starts on a multiple of 8 elements and both
    // base pointers are 16-byte aligned
    const bool vec = (a.V % 8) == 0 && (reinterpret_cast<uintptr_t>(a.P) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.Q) & 15) == 0;
    if (a.p_bf16 && a.q_bf16) launch_alpha_t<true, true>(a, vec, s);
    else if (a.p_bf16) launch_alpha_t<true, false>(a, vec, s);
    else if (a.q_bf16) launch_alpha_t<false, true>(a, vec, s);
    else launch_alpha_t<false, false>(a, vec, s);
    return hipGetLastError();
}

}  // namespace specdec
