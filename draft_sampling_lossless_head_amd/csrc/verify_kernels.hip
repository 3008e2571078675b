// Lossless verification kernels (VESSL "Speculative Decoding Part 1",
// sections "알고리즘" and "수락 규칙").  Four launches on the caller's stream:
//
//   verify_rows (x2)      one workgroup per segment of each target row p_k
//                         (k <= L) and draft row q_k (k < L): one pass with
//                         16-byte loads -> max and sum exp((l - max)/T)
//                         (sampling) or max and argmax (greedy), plus the
//                         logit at the draft token.
//   verify_decide         one thread per request: merges the segments,
//                         normalisers, the ratio test
//                         u * q(x) < p(x) at every position, first rejection
//                         n, emitted draft tokens, diagnostics.
//   verify_final_partials one workgroup per (request, 4096-token chunk) of the
//                         row that feeds the final draw: sum of max(0, p_n - q_n)
//                         (correction) or of p_L (bonus).
//   verify_final_draw     one workgroup per request: inverse CDF over the chunk
//                         sums, then over the chosen chunk -> final token.
// The final-draw pair is skipped for T == 0 (argmax of p_n, set by decide).
#include <algorithm>
#include <cfloat>
#include <climits>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace specdec {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 4096;          // tokens per chunk of the final draw
constexpr int kPerThread = kChunk / 256;
static_assert(kPerThread == 16, "the final draw works on runs of 16 tokens per thread");

// Most segments a verified row is split into.
constexpr int kMaxRowSegs = 16;

// Cache policy of a streaming buffer load: non-temporal.
constexpr int kBufNontemporal = 2;

int verify_num_chunks(int V) { return (V + kChunk - 1) / kChunk; }

// Segments per verified row: enough workgroups to fill the chip once (2048
// resident workgroups of 256 threads), each segment at least 4096 tokens.
// Fewer, longer segments stream better: at 2176 rows of 151936 bf16 logits,
// whole rows take 102.8 us, two segments per row 104.0 us, four 106.7 us,
// eight 107.2 us (measured), although whole rows leave a short second wave.
int verify_row_segs(int B, int gamma_max, int V) {
    const int64_t rows = std::max<int64_t>(1, (int64_t)B * (gamma_max + 1));
    const int64_t want = (2048 + rows - 1) / rows;
    const int64_t cap = std::max(1, std::min(kMaxRowSegs, V / 4096));
    return (int)std::max<int64_t>(1, std::min(want, cap));
}

__device__ __forceinline__ int64_t p_row(const VerifyArgs& a, int b, int k) {
    return (a.p_row_off ? a.p_row_off[b] : (int64_t)b * (a.gamma_max + 1)) + k;
}

__device__ __forceinline__ int64_t q_row(const VerifyArgs& a, int b, int k) {
    if (a.q_single_row) return b;
    return (a.q_row_off ? a.q_row_off[b] : (int64_t)b * a.gamma_max) + k;
}

__device__ __forceinline__ int request_len(const VerifyArgs& a, int b) {
    return a.lens ? a.lens[b] : a.gamma_max;
}

// Greedy rows: online (max, argmax) over n consecutive values from v0.
template <int N>
__device__ __forceinline__ void absorb_arg(const float (&x)[N], int v0, float& m, int& idx) {
    float lm = x[0];
    int li = 0;
#pragma unroll
    for (int t = 1; t < N; ++t)
        if (x[t] > lm) {
            lm = x[t];
            li = t;
        }
    if (lm > m) {
        m = lm;
        idx = v0 + li;
    }
}

// Sampling rows: running max m, its scaled copy mc = max(m c, -FLT_MAX) with
// c = log2(e) / T, and two partial sums of 2^(x c - mc).  A run of N values
// costs one max tree (v_max3), one rescale, and per value one fma, one exp2
// and one add; no argmax is kept (sampling never reads it).  The clamp keeps
// an all -inf prefix NaN-free: its terms are 2^(-inf) = 0.
struct SampStat {
    float m, mc, s0, s1;
};

template <int N>
__device__ __forceinline__ void absorb_samp(const float (&x)[N], SampStat& st, float c) {
    float lm = st.m;
#pragma unroll
    for (int t = 0; t < N; ++t) lm = fmaxf(lm, x[t]);
    const float mc = fmaxf(lm * c, -FLT_MAX);
    const float r = __builtin_amdgcn_exp2f(st.mc - mc);
    st.s0 *= r;
    st.s1 *= r;
    st.m = lm;
    st.mc = mc;
#pragma unroll
    for (int t = 0; t < N; ++t) {
        const float e = __builtin_amdgcn_exp2f(fmaf(x[t], c, -mc));
        if (t & 1) st.s1 += e;
        else st.s0 += e;
    }
}

// sum exp((x - m) / T) against the exact m: the terms were taken against the
// rounded mc, off by the factor 2^(m c - mc), whose exponent fma gives exactly.
__device__ __forceinline__ float samp_sum(const SampStat& st, float c) {
    const float s = st.s0 + st.s1;
    return st.m == -INFINITY ? s : s * __builtin_amdgcn_exp2f(fmaf(-st.m, c, st.mc));
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4_t& w, float* x) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        x[2 * h] = __uint_as_float(w[h] << 16);
        x[2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
    }
}

// Range-checked view of nbytes at base (raw buffer, no stride): a 16-byte
// load at an offset at or past nbytes returns zeros and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int64_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                             (int)(nbytes > 0 ? nbytes : 0), 0x00020000);
}

template <typename Vec>
__device__ __forceinline__ Vec load16_nt(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(Vec, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNontemporal));
}

// Words that decode to -inf in every lane of a vector.
template <bool BF16>
__device__ __forceinline__ uint32_t neg_inf_word() {
    return BF16 ? 0xFF80FF80u : 0xFF800000u;
}

// Runs of four vectors at j, j + 256, j + 512, j + 768 of the segment's n
// vectors at rv, in two ping-pong buffers so one run's loads are in flight
// while the other is absorbed.  Vector u of a run goes through its own view
// starting 256 u vectors in, so one 32-bit offset serves the four loads and
// a load past the end reads zeros instead of memory; the last run, partial
// or not, has such vectors replaced by -inf (no weight, never the max).
// Every load of the loop is unconditional: a load under a branch, or one
// whose only use lies past a loop exit, would be waited for together with
// the current run.
template <bool BF16, typename Vec, typename F>
__device__ __forceinline__ void scan_runs(const Vec* rv, int n, int j, int vid0, F& f) {
    if (j >= n) return;
    __amdgpu_buffer_rsrc_t r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = range_rsrc(rv + u * 256, (int64_t)(n - u * 256) * 16);
    const int nr = (n - j + 1023) / 1024;   // runs, the last possibly partial
    Vec A[4], Bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) A[u] = load16_nt<Vec>(r[u], j * 16);
    int q = 0;
    for (; q + 2 < nr; q += 2) {
#pragma unroll
        for (int u = 0; u < 4; ++u) Bv[u] = load16_nt<Vec>(r[u], (j + 1024) * 16);
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the run
        f.template run<4>(A, vid0 + j);
#pragma unroll
        for (int u = 0; u < 4; ++u) A[u] = load16_nt<Vec>(r[u], (j + 2048) * 16);
        __builtin_amdgcn_sched_barrier(0);
        f.template run<4>(Bv, vid0 + j + 1024);
        j += 2048;
    }
    auto last = [&](Vec (&w)[4], int jj) {
        using W = uint32_t __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (jj + u * 256 >= n) {
                const uint32_t ni = neg_inf_word<BF16>();
                w[u] = __builtin_bit_cast(Vec, W{ni, ni, ni, ni});
            }
        }
        f.template run<4>(w, vid0 + jj);
    };
    if (nr - q == 2) {
#pragma unroll
        for (int u = 0; u < 4; ++u) Bv[u] = load16_nt<Vec>(r[u], (j + 1024) * 16);
        __builtin_amdgcn_sched_barrier(0);
        f.template run<4>(A, vid0 + j);
        last(Bv, j + 1024);
    } else {
        last(A, j);
    }
}

// One segment of one row: 16-byte vectors [vlo, vhi), or, when the row
// length is no multiple of the vector width, single values [slo, shi).
// Thread tid takes vectors vlo + tid, + 256, ...; f.run<U>(w, i) absorbs U
// vectors at ids i, i + 256, ..., f.one(x, v) a single value.
template <bool BF16, typename F>
__device__ __forceinline__ void scan_segment(const void* row, int vlo, int vhi, int slo, int shi,
                                             int tid, F& f) {
    using Vec = typename std::conditional<BF16, u32x4_t, f32x4_t>::type;
    scan_runs<BF16>(reinterpret_cast<const Vec*>(row) + vlo, vhi - vlo, tid, vlo, f);
    if constexpr (BF16) {
        const uint16_t* r = static_cast<const uint16_t*>(row);
        for (int v = slo + tid; v < shi; v += 256) f.one(__uint_as_float((uint32_t)r[v] << 16), v);
    } else {
        const float* r = static_cast<const float*>(row);
        for (int v = slo + tid; v < shi; v += 256) f.one(r[v], v);
    }
}

// Absorbers over runs of U vectors at vector ids i, i + 256, ...
template <bool BF16>
struct SampAbsorb {
    SampStat st;
    float c;
    template <int U, typename Vec>
    __device__ __forceinline__ void run(const Vec (&w)[U], int) {
        constexpr int VW = BF16 ? 8 : 4;
        float x[U * VW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (BF16) {
                bf16x8_to_f32(w[u], x + u * 8);
            } else {
#pragma unroll
                for (int h = 0; h < 4; ++h) x[u * 4 + h] = w[u][h];
            }
        }
        absorb_samp<U * VW>(x, st, c);
    }
    __device__ __forceinline__ void one(float v, int) {
        const float x[1] = {v};
        absorb_samp<1>(x, st, c);
    }
};

template <bool BF16>
struct ArgAbsorb {
    float m;
    int idx;
    template <int U, typename Vec>
    __device__ __forceinline__ void run(const Vec (&w)[U], int i) {
        constexpr int VW = BF16 ? 8 : 4;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VW];
            if constexpr (BF16) {
                bf16x8_to_f32(w[u], x);
            } else {
#pragma unroll
                for (int h = 0; h < 4; ++h) x[h] = w[u][h];
            }
            absorb_arg<VW>(x, (i + u * 256) * VW, m, idx);
        }
    }
    __device__ __forceinline__ void one(float v, int id) {
        const float x[1] = {v};
        absorb_arg<1>(x, id, m, idx);
    }
};

// One workgroup per (segment, row): the row's statistics over that segment,
// as one RowStat part; verify_decide merges the parts of a row.
template <bool BF16, bool GREEDY>
__global__ __launch_bounds__(256)
void verify_rows(VerifyArgs a, int is_q) {
    __shared__ float red_m[4], red_s[4];
    __shared__ int red_i[4];
    const int seg = blockIdx.x;
    const int k = blockIdx.y;
    const int b = blockIdx.z;
    const int S = a.row_segs;
    const int L = request_len(a, b);
    if (L < 0 || L > a.gamma_max) return;
    if (is_q ? (k >= L) : (k > L)) return;
    const int V = a.V;
    const int64_t row = is_q ? q_row(a, b, k) : p_row(a, b, k);
    const void* base = is_q ? a.Q : a.P;
    const void* rp = BF16 ? static_cast<const void*>(static_cast<const uint16_t*>(base) + row * (int64_t)V)
                          : static_cast<const void*>(static_cast<const float*>(base) + row * (int64_t)V);
    const int tid = threadIdx.x;
    constexpr int VW = BF16 ? 8 : 4;
    const int nvec = (V % VW == 0) ? V / VW : 0;
    const int vlo = (int)((int64_t)nvec * seg / S), vhi = (int)((int64_t)nvec * (seg + 1) / S);
    const int slo = nvec ? 0 : (int)((int64_t)V * seg / S);
    const int shi = nvec ? 0 : (int)((int64_t)V * (seg + 1) / S);
    const float invT = a.invT;
    // The logit at the draft token (segment 0 of a drafted position), loaded
    // ahead of the scan through a view that is empty when there is none, so
    // the load is unconditional and nothing waits for it before the end.
    int xg = -1;
    if (seg == 0 && k < L) xg = a.draft[(size_t)b * a.gamma_max + k];
    const bool gv = xg >= 0 && xg < V;
    const __amdgpu_buffer_rsrc_t grs = range_rsrc(rp, gv ? (int64_t)V * (BF16 ? 2 : 4) : 0);
    uint32_t gbits;
    if constexpr (BF16) gbits = __builtin_amdgcn_raw_buffer_load_b16(grs, gv ? xg * 2 : 0, 0, 0);
    else gbits = __builtin_amdgcn_raw_buffer_load_b32(grs, gv ? xg * 4 : 0, 0, 0);

    float m, s;
    int idx;
    if constexpr (GREEDY) {
        ArgAbsorb<BF16> f{-INFINITY, INT_MAX};
        scan_segment<BF16>(rp, vlo, vhi, slo, shi, tid, f);
        m = f.m;
        s = 0.0f;
        idx = f.idx;
    } else {
        const float c = invT * 1.44269504088896340736f;
        SampAbsorb<BF16> f{{-INFINITY, -FLT_MAX, 0.0f, 0.0f}, c};
        scan_segment<BF16>(rp, vlo, vhi, slo, shi, tid, f);
        m = f.st.m;
        s = samp_sum(f.st, c);
        idx = INT_MAX;
    }

    wave_reduce_stat(m, s, idx, invT);
    const int lane = tid & 63, wave = tid >> 6;
    if (lane == 0) {
        red_m[wave] = m;
        red_s[wave] = s;
        red_i[wave] = idx;
    }
    __syncthreads();
    if (tid == 0) {
        float M = red_m[0], Sm = red_s[0];
        int I = red_i[0];
        for (int w = 1; w < 4; ++w) {
            float mv = M;
            int iv = I;
            merge_arg(mv, iv, red_m[w], red_i[w]);
            merge_ms(M, Sm, red_m[w], red_s[w], invT);
            I = iv;
        }
        const float gathered = BF16 ? __uint_as_float(gbits << 16) : __uint_as_float(gbits);
        RowStat rs;
        rs.m = M;
        rs.s = Sm;
        rs.idx = I;
        rs.gathered = gathered;
        const size_t slot = (size_t)b * (2 * a.gamma_max + 1) + (is_q ? a.gamma_max + 1 + k : k);
        a.rows[slot * S + seg] = rs;
    }
}

// The statistics of a whole row from its per-segment parts: max and sum
// merged online, argmax by lowest id on ties, the gathered logit from part 0.
// Parts are loaded four at a time, all four issued at once (ids clamped to
// the last part); the copies past S act as the neutral part (-inf, 0,
// INT_MAX).
__device__ __forceinline__ RowStat merged_row(const RowStat* parts, int S, float invT) {
    RowStat r{-INFINITY, 0.0f, INT_MAX, parts[0].gathered};
    for (int g0 = 0; g0 < S; g0 += 4) {
        RowStat p[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) p[g] = parts[min(g0 + g, S - 1)];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const bool in = g0 + g < S;
            const float om = in ? p[g].m : -INFINITY;
            const float os = in ? p[g].s : 0.0f;
            const int oi = in ? p[g].idx : INT_MAX;
            float mv = r.m;
            int iv = r.idx;
            merge_arg(mv, iv, om, oi);
            merge_ms(r.m, r.s, om, os, invT);
            r.idx = iv;
        }
    }
    return r;
}

// One wave per request; lane k handles position k (in chunks of 64).  The
// first rejection is the lowest set bit of a ballot.  One pass merges each
// row once and writes the per-position outputs; a request found invalid on
// the way (a draft token out of range, a row with no finite logit) has them
// overwritten afterwards.
__global__ __launch_bounds__(256)
void verify_decide(VerifyArgs a) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const int G = a.gamma_max;
    const int L = request_len(a, b);
    int32_t* out = a.out_tokens + (size_t)b * (G + 1);
    const int32_t* dr = a.draft + (size_t)b * G;
    const int S = a.row_segs;
    const RowStat* rs = a.rows + (size_t)b * (2 * G + 1) * S;
    const float invTf = a.invT;
    const double invT = (double)a.invT;

    bool bad = L < 0 || L > G;
    int n = L, idx_n = -1, idx_L = -1;
    double lzp_n = 0.0, lzq_n = 0.0, lzp_L = 0.0;
    for (int c0 = 0; !bad && c0 <= G; c0 += kWave) {
        const int k = c0 + lane;
        double lzp = 0.0, lzq = 0.0, ap = 0.0;
        bool reject = false, bad_l = false;
        RowStat p{};
        if (k <= L) {
            p = merged_row(rs + (size_t)k * S, S, invTf);
            bad_l = p.m == -INFINITY;
            lzp = a.greedy ? (double)p.m : (double)p.m * invT + log((double)p.s);
        }
        if (k < L) {
            const int x = dr[k];
            bad_l = bad_l || x < 0 || x >= a.V;
            const RowStat q = a.qprob ? p : merged_row(rs + (size_t)(G + 1 + k) * S, S, invTf);
            if (!a.qprob) bad_l = bad_l || q.m == -INFINITY;
            if (a.greedy) {
                lzq = a.qlogz ? (double)a.qlogz[(size_t)b * G + k] : (double)q.m;
                reject = p.idx != x;
                ap = reject ? 0.0 : 1.0;
            } else {
                const double px = exp((double)p.gathered * invT - lzp);
                double qx;
                if (a.qprob) {   // the draft's own q(x_k) and normaliser
                    lzq = (double)a.qlogz[(size_t)b * G + k];
                    qx = (double)a.qprob[(size_t)b * G + k];
                } else {
                    lzq = (double)q.m * invT + log((double)q.s);
                    qx = exp((double)q.gathered * invT - lzq);
                }
                ap = qx > 0.0 ? fmin(1.0, px / qx) : (px > 0.0 ? 1.0 : 0.0);
                const float u = a.uniforms ? a.uniforms[(size_t)b * (G + 1) + k]
                                           : counter_uniform(a.seed, a.offset, b, k, 1);
                reject = !((double)u * qx < px);
            }
        }
        if (k <= G) {
            if (a.p_logZ) a.p_logZ[(size_t)b * (G + 1) + k] = (float)lzp;
            if (k < G && a.q_logZ) a.q_logZ[(size_t)b * G + k] = (float)lzq;
            if (k < G && a.accept_prob) a.accept_prob[(size_t)b * G + k] = (float)ap;
        }
        bad = __ballot(bad_l) != 0;
        const unsigned long long rej = __ballot(reject);
        if (n == L && rej) {
            n = c0 + __ffsll((long long)rej) - 1;
            lzp_n = __shfl(lzp, n - c0);
            lzq_n = __shfl(lzq, n - c0);
            idx_n = __shfl(p.idx, n - c0);
        }
        if (L >= c0 && L < c0 + kWave) {
            lzp_L = __shfl(lzp, L - c0);
            idx_L = __shfl(p.idx, L - c0);
        }
    }
    if (bad) {
        for (int j = lane; j <= G; j += kWave) {
            out[j] = -1;
            if (a.p_logZ) a.p_logZ[(size_t)b * (G + 1) + j] = 0.0f;
            if (j < G && a.q_logZ) a.q_logZ[(size_t)b * G + j] = 0.0f;
            if (j < G && a.accept_prob) a.accept_prob[(size_t)b * G + j] = 0.0f;
        }
        if (lane == 0) {
            a.accepted[b] = -1;
            if (a.row_pos) a.row_pos[b] = -1;
            FinalInfo f;
            f.logZp = 0.0;
            f.logZq = 0.0;
            f.n = -1;
            f.mode = 0;
            f.prev = -1;
            f.pad1 = 0;
            a.fin[b] = f;
        }
        return;
    }
    if (n == L) {
        lzp_n = lzp_L;
        idx_n = idx_L;
    }
    for (int j = lane; j <= G; j += kWave) out[j] = j < n ? dr[j] : -1;
    if (lane == 0) {
        if (a.greedy) out[n] = idx_n;
        a.accepted[b] = n;
        if (a.row_pos) a.row_pos[b] = (!a.greedy && n < L) ? n : -1;
        FinalInfo f;
        f.logZp = lzp_n;
        f.logZq = lzq_n;
        f.n = n;
        f.mode = a.greedy ? 0 : (n < L ? 1 : 2);
        f.prev = n > 0 ? dr[n - 1] : -1;
        f.pad1 = 0;
        a.fin[b] = f;
    }
}

// Weights of the final draw: max(0, p - q) (correction) or p (bonus), with
// p = exp(P/T - logZp) and q = exp(Q/T - logZq); the exponent subtracts the
// fp64 normaliser as a (hi, lo) float pair.
template <bool PB, bool QB>
struct FinalRow {
    const void* pr;
    const void* qr;
    float invT, lzp_hi, lzp_lo, lzq_hi, lzq_lo;
    int residual;

    template <bool BF>
    __device__ __forceinline__ static void load16(const void* base, int v0, int V, float x[16]) {
        if (BF) {
            const uint16_t* r = static_cast<const uint16_t*>(base);
            if ((V % 8) == 0 && v0 + 16 <= V) {
                const uint4 t0 = *reinterpret_cast<const uint4*>(r + v0);
                const uint4 t1 = *reinterpret_cast<const uint4*>(r + v0 + 8);
                const uint32_t w[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
                for (int h = 0; h < 8; ++h) {
                    x[2 * h] = bf16_bits_to_float(w[h] & 0xFFFFu);
                    x[2 * h + 1] = bf16_bits_to_float(w[h] >> 16);
                }
                return;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) x[t] = v0 + t < V ? bf16_bits_to_float(r[v0 + t]) : 0.0f;
        } else {
            const float* r = static_cast<const float*>(base);
            if ((V % 4) == 0 && v0 + 16 <= V) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float4 t = *reinterpret_cast<const float4*>(r + v0 + 4 * h);
                    x[4 * h] = t.x; x[4 * h + 1] = t.y; x[4 * h + 2] = t.z; x[4 * h + 3] = t.w;
                }
                return;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) x[t] = v0 + t < V ? r[v0 + t] : 0.0f;
        }
    }

    // the 16 weights of tokens v0 .. v0 + 15 (0 beyond V)
    __device__ __forceinline__ void weights16(int v0, int V, float w[16]) const {
        float lp[16];
        load16<PB>(pr, v0, V, lp);
#pragma unroll
        for (int t = 0; t < 16; ++t) w[t] = __expf(fmaf(lp[t], invT, -lzp_hi) - lzp_lo);
        if (residual) {
            float lq[16];
            load16<QB>(qr, v0, V, lq);
#pragma unroll
            for (int t = 0; t < 16; ++t)
                w[t] = fmaxf(w[t] - __expf(fmaf(lq[t], invT, -lzq_hi) - lzq_lo), 0.0f);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t)
            if (v0 + t >= V) w[t] = 0.0f;
    }
};

template <bool PB, bool QB>
__device__ __forceinline__ FinalRow<PB, QB> make_final_row(const VerifyArgs& a, int b,
                                                           const FinalInfo& f, int residual) {
    FinalRow<PB, QB> fr;
    const int64_t V = a.V;
    fr.pr = PB ? (const void*)(static_cast<const uint16_t*>(a.P) + p_row(a, b, f.n) * V)
               : (const void*)(static_cast<const float*>(a.P) + p_row(a, b, f.n) * V);
    fr.qr = nullptr;
    if (residual)
        fr.qr = QB ? (const void*)(static_cast<const uint16_t*>(a.Q) + q_row(a, b, f.n) * V)
                   : (const void*)(static_cast<const float*>(a.Q) + q_row(a, b, f.n) * V);
    fr.invT = a.invT;
    fr.lzp_hi = (float)f.logZp;
    fr.lzp_lo = (float)(f.logZp - (double)fr.lzp_hi);
    fr.lzq_hi = (float)f.logZq;
    fr.lzq_lo = (float)(f.logZq - (double)fr.lzq_hi);
    fr.residual = residual;
    return fr;
}

// fp64 sum of this thread's run of kPerThread consecutive tokens of chunk c.
template <bool PB, bool QB>
__device__ __forceinline__ double thread_chunk_sum(const FinalRow<PB, QB>& fr, int c, int V,
                                                   int tid) {
    float w[kPerThread];
    fr.weights16(c * kChunk + tid * kPerThread, V, w);
    double acc = 0.0;
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) acc += (double)w[t];
    return acc;
}

__device__ __forceinline__ double block_sum_f64(double x, double* sh) {
    x = wave_sum_f64(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) sh[wave] = x;
    __syncthreads();
    return sh[0] + sh[1] + sh[2] + sh[3];
}

template <bool PB, bool QB>
__global__ __launch_bounds__(256)
void verify_final_partials(VerifyArgs a) {
    __shared__ double sh[4];
    const int c = blockIdx.x;
    const int b = blockIdx.y;
    const FinalInfo f = a.fin[b];
    if (f.mode == 0) return;
    const FinalRow<PB, QB> fr = make_final_row<PB, QB>(a, b, f, f.mode == 1);
    const double tot = block_sum_f64(thread_chunk_sum(fr, c, a.V, threadIdx.x), sh);
    if (threadIdx.x == 0) a.chunk_sums[(size_t)b * gridDim.x + c] = tot;
}

// Block-wide exclusive scan of one fp64 value per thread (256 threads).
__device__ __forceinline__ void block_scan_f64(double x, double* scan, double& excl,
                                               double& incl, double& total) {
    const int tid = threadIdx.x;
    __syncthreads();
    scan[tid] = x;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const double add = tid >= off ? scan[tid - off] : 0.0;
        __syncthreads();
        scan[tid] += add;
        __syncthreads();
    }
    incl = scan[tid];
    excl = tid > 0 ? scan[tid - 1] : 0.0;
    total = scan[255];
}

template <bool PB, bool QB>
__global__ __launch_bounds__(256)
void verify_final_draw(VerifyArgs a, int nchunk) {
    __shared__ double scan[256];
    __shared__ int sh_pick, sh_last[4];
    __shared__ double sh_rem;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    FinalInfo f = a.fin[b];
    if (f.mode == 0) return;
    const int G = a.gamma_max;
    const int V = a.V;
    double* sums = a.chunk_sums + (size_t)b * nchunk;

    const float u = a.uniforms ? a.uniforms[(size_t)b * (G + 1) + G]
                               : counter_uniform(a.seed, a.offset, b, 0, 2);
    const int per = (nchunk + 255) / 256;
    const int c0 = min(nchunk, tid * per);
    const int c1 = min(nchunk, c0 + per);
    double tsum = 0.0;
    for (int c = c0; c < c1; ++c) tsum += sums[c];
    double excl, incl, R;
    block_scan_f64(tsum, scan, excl, incl, R);

    int residual = f.mode == 1;
    if (!(R > 0.0)) {
        // Residual without mass after rounding: draw from p_n instead.
        residual = 0;
        const FinalRow<PB, QB> fp = make_final_row<PB, QB>(a, b, f, 0);
        for (int c = 0; c < nchunk; ++c) {
            const double t = block_sum_f64(thread_chunk_sum(fp, c, V, tid), scan);
            if (tid == 0) sums[c] = t;
        }
        __syncthreads();
        tsum = 0.0;
        for (int c = c0; c < c1; ++c) tsum += sums[c];
        block_scan_f64(tsum, scan, excl, incl, R);
    }
    const FinalRow<PB, QB> fr = make_final_row<PB, QB>(a, b, f, residual);
    const double thr = (double)u * R;

    // chunk holding thr (clamped to the last chunk with mass)
    if (tid == 0) sh_pick = -1;
    __syncthreads();
    if (tsum > 0.0 && thr >= excl && thr < incl) {
        double run = excl;
        int found = -1, last = -1;
        double last_run = 0.0;
        for (int c = c0; c < c1; ++c) {
            const double w = sums[c];
            if (w > 0.0) {
                last = c;
                last_run = run;
                if (thr < run + w) {
                    found = c;
                    break;
                }
            }
            run += w;
        }
        sh_pick = found >= 0 ? found : last;
        sh_rem = found >= 0 ? thr - run : thr - last_run;
    }
    __syncthreads();
    if (sh_pick < 0) {
        int lastc = -1;
        for (int c = c0; c < c1; ++c)
            if (sums[c] > 0.0) lastc = c;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) lastc = max(lastc, __shfl_xor(lastc, off));
        if (lane == 0) sh_last[wave] = lastc;
        __syncthreads();
        if (tid == 0) {
            sh_pick = max(max(sh_last[0], sh_last[1]), max(sh_last[2], sh_last[3]));
            sh_rem = INFINITY;
        }
        __syncthreads();
    }
    const int cstar = sh_pick;
    const double rem = sh_rem;
    if (cstar < 0) {   // no mass anywhere (cannot happen for a finite target row)
        if (tid == 0) a.out_tokens[(size_t)b * (G + 1) + f.n] = -1;
        return;
    }

    // rescan the chunk: per-thread runs of kPerThread tokens, same sums as
    // verify_final_partials, then the owning thread walks its run.
    const double mine = thread_chunk_sum(fr, cstar, V, tid);
    double e2, i2, tot2;
    block_scan_f64(mine, scan, e2, i2, tot2);
    if (tid == 0) sh_pick = -1;
    __syncthreads();
    if (mine > 0.0 && rem >= e2 && rem < i2) {
        double run = e2;
        int pick = -1, last = -1;
        const int v0 = cstar * kChunk + tid * kPerThread;
        float wr[kPerThread];
        fr.weights16(v0, V, wr);
        for (int t = 0; t < kPerThread && v0 + t < V; ++t) {
            const double w = (double)wr[t];
            if (w > 0.0) {
                last = v0 + t;
                if (rem < run + w) {
                    pick = v0 + t;
                    break;
                }
            }
            run += w;
        }
        sh_pick = pick >= 0 ? pick : last;
    }
    __syncthreads();
    if (sh_pick < 0) {
        // rem beyond the rescanned total: last token of the chunk with weight
        int lastv = -1;
        const int v0 = cstar * kChunk + tid * kPerThread;
        float wr[kPerThread];
        fr.weights16(v0, V, wr);
        for (int t = 0; t < kPerThread && v0 + t < V; ++t)
            if (wr[t] > 0.0f) lastv = v0 + t;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) lastv = max(lastv, __shfl_xor(lastv, off));
        if (lane == 0) sh_last[wave] = lastv;
        __syncthreads();
        if (tid == 0) sh_pick = max(max(sh_last[0], sh_last[1]), max(sh_last[2], sh_last[3]));
        __syncthreads();
    }
    if (tid == 0) a.out_tokens[(size_t)b * (G + 1) + f.n] = sh_pick;
}

__global__ void philox_uniforms_kernel(uint64_t seed, uint32_t offset, uint32_t stream, int B,
                                       int K, float* out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)B * K) return;
    const int b = (int)(i / K), k = (int)(i % K);
    out[i] = counter_uniform(seed, offset, b, k, stream);
}

template <bool PB, bool QB>
static void launch_final(const VerifyArgs& a, hipStream_t s) {
    const int nc = verify_num_chunks(a.V);
    void* t = prof_begin("verify_final_partials", s);
    hipLaunchKernelGGL((verify_final_partials<PB, QB>), dim3(nc, a.B), dim3(256), 0, s, a);
    prof_end(t, s);
    t = prof_begin("verify_final_draw", s);
    hipLaunchKernelGGL((verify_final_draw<PB, QB>), dim3(a.B), dim3(256), 0, s, a, nc);
    prof_end(t, s);
}

template <bool BF16>
static void launch_rows(const VerifyArgs& a, int is_q, hipStream_t s) {
    const int nrow = is_q ? a.gamma_max : a.gamma_max + 1;
    if (nrow == 0) return;
    dim3 grid(a.row_segs, nrow, a.B);
    void* t = prof_begin(is_q ? "verify_rows_q" : "verify_rows_p", s);
    if (a.greedy)
        hipLaunchKernelGGL((verify_rows<BF16, true>), grid, dim3(256), 0, s, a, is_q);
    else
        hipLaunchKernelGGL((verify_rows<BF16, false>), grid, dim3(256), 0, s, a, is_q);
    prof_end(t, s);
}

hipError_t verify_rows_decide_launch(const VerifyArgs& a, hipStream_t s) {
    if (a.p_bf16) launch_rows<true>(a, 0, s);
    else launch_rows<false>(a, 0, s);
    if (!a.qprob) {
        if (a.q_bf16) launch_rows<true>(a, 1, s);
        else launch_rows<false>(a, 1, s);
    }
    void* t = prof_begin("verify_decide", s);
    hipLaunchKernelGGL(verify_decide, dim3((a.B + 3) / 4), dim3(256), 0, s, a);
    prof_end(t, s);
    return hipGetLastError();
}

hipError_t verify_final_launch(const VerifyArgs& a, hipStream_t s) {
    if (!a.greedy) {
        if (a.p_bf16 && a.q_bf16) launch_final<true, true>(a, s);
        else if (a.p_bf16) launch_final<true, false>(a, s);
        else if (a.q_bf16) launch_final<false, true>(a, s);
        else launch_final<false, false>(a, s);
    }
    return hipGetLastError();
}

hipError_t verify_launch(const VerifyArgs& a, hipStream_t s) {
    hipError_t e = verify_rows_decide_launch(a, s);
    if (e != hipSuccess) return e;
    return verify_final_launch(a, s);
}

hipError_t philox_uniforms_launch(uint64_t seed, uint32_t offset, uint32_t stream, int B, int K,
                                  float* out, hipStream_t s) {
    const int64_t n = (int64_t)B * K;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(philox_uniforms_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       seed, offset, stream, B, K, out);
    return hipGetLastError();
}

}  // namespace specdec
