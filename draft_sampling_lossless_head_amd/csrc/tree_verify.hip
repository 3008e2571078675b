// Verification of a tree draft ("Speculative Decoding Part 1", section on
// spending the draft budget on a tree instead of a chain: the branches of a
// tree of continuations are verified in one target pass; the acceptance rule
// of the section on the acceptance rule keeps the output lossless).
//
// Recursive rejection over siblings: the walk starts at the root with target
// law r = p; the children of the current node are tested in increasing index,
// child c (token x) passing iff u_c q(x) < r(x) with q the draft law the
// children were drawn from.  A pass emits x and moves the walk to c (r = p of
// c); a failure sets r <- normalize(max(0, r - q)) and tests the next child.
// When every child has failed the final token is drawn from r; a node without
// children draws a bonus token from its p.  T == 0: the first child holding
// the argmax of p passes; the final token is that argmax.
//
// After j failures the residual is r_j = max(0, p - c_j q) / W_j with c_0 = 0,
// W_0 = 1, c_{j+1} = c_j + W_j and W_{j+1} = sum_v max(0, p(v) - c_{j+1} q(v))
// (the same law as the repeated normalisation, one pass over the vocabulary per
// failure and no stored row).
//
// W workgroups of 512 threads per request (W = 1 when the batch fills the
// device, up to 8 when it does not).  Workgroup i of a request owns a
// contiguous range of 512-token segments of the vocabulary and every one of
// them runs the same walk: each pass over a row covers its range only, and
// each reduction (normalisers, residual mass, argmax, the final draw's range
// totals) is exchanged through tagged words in device memory and merged in
// workgroup order, so all W workgroups take the same decisions.  Every pass
// over a row reads it in 8-token vectors spread over the threads; sums are
// fp64 per lane, the normalisers' (max, sum) pairs fp32 per lane as in the
// chain's verification.  The final draw is a two-level inverse CDF: the
// range holding u * W from the exchanged range totals, then inside it the sums
// of its 512-token segments (one wave each), the segment by one wave, and the
// token inside it; the range's workgroup hands the token to workgroup 0, which
// alone writes the outputs.
#include <algorithm>
#include <atomic>
#include <cfloat>
#include <climits>

#include "device_common.hpp"
#include "launch.hpp"

namespace specdec {

namespace {

constexpr int kTvThreads = 512;
constexpr int kTvWaves = kTvThreads / 64;
constexpr int kTvSeg = 512;                        // tokens per segment of the final draw
constexpr int kTvMaxSegs = kTreeVerifyMaxV / kTvSeg;
constexpr int kTvSegBatch = 4;            // segments per wave whose loads go out together
constexpr int kTreeSplitMax = 8;          // workgroups per request at most
constexpr int kTreeXchgWgs = 1024;        // split workgroups of one launch at most
constexpr unsigned kTreePollLimit = 1u << 20;

// Eight consecutive logits v0 .. v0 + 7 of a row (fp32); -inf past V.
template <bool BF>
__device__ __forceinline__ void load8(const void* base, size_t row_off, int v0, int V, bool vec,
                                      float x[8]) {
    if (vec && v0 + 8 <= V) {
        if constexpr (BF) {
            const uint4 w = *reinterpret_cast<const uint4*>(
                static_cast<const uint16_t*>(base) + row_off + v0);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                x[2 * h] = __uint_as_float(ww[h] << 16);
                x[2 * h + 1] = __uint_as_float(ww[h] & 0xFFFF0000u);
            }
        } else {
            const float* p = static_cast<const float*>(base) + row_off + v0;
            const float4 a = *reinterpret_cast<const float4*>(p);
            const float4 b = *reinterpret_cast<const float4*>(p + 4);
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int v = v0 + e;
            if (v < V) {
                if constexpr (BF)
                    x[e] = __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[row_off + v] << 16);
                else
                    x[e] = static_cast<const float*>(base)[row_off + v];
            } else {
                x[e] = -INFINITY;
            }
        }
    }
}

// Eight logits of vector i (< nvec) of a row of a multiple of 8 tokens: one
// or two 16-byte loads, no branch.
template <bool BF>
__device__ __forceinline__ void load8v(const void* base, size_t row_off, int i, float x[8]) {
    if constexpr (BF) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row_off +
                                                        8 * (size_t)i);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            x[2 * h] = __uint_as_float(ww[h] << 16);
            x[2 * h + 1] = __uint_as_float(ww[h] & 0xFFFF0000u);
        }
    } else {
        const float* p = static_cast<const float*>(base) + row_off + 8 * (size_t)i;
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

// A pass over the row's vectors: f(i, xp, xq) for every vector i < nvec of
// this thread (xq only with Q).  Aligned rows go in batches of kTvBatch
// vectors per thread whose loads all issue before the first is used (a
// clamped index past the end re-reads the last vector, skipped); other rows
// one vector at a time with bounds checks.
constexpr int kTvBatch = 8;
template <bool PB, bool QB, bool WITHQ, typename F>
__device__ __forceinline__ void row_pass(const TreeVerifyArgs& a, size_t prow, size_t qrow,
                                         int vlo, int vhi, bool vec, F&& f) {
    const int tid = threadIdx.x;
    if (vec) {
        for (int i0 = vlo + tid; i0 < vhi; i0 += kTvThreads * kTvBatch) {
            float xp[kTvBatch][8], xq[kTvBatch][8];
#pragma unroll
            for (int j = 0; j < kTvBatch; ++j) {
                const int i = min(i0 + j * kTvThreads, vhi - 1);
                load8v<PB>(a.P, prow, i, xp[j]);
                if constexpr (WITHQ) load8v<QB>(a.Q, qrow, i, xq[j]);
            }
#pragma unroll
            for (int j = 0; j < kTvBatch; ++j)
                if (i0 + j * kTvThreads < vhi) f(i0 + j * kTvThreads, xp[j], xq[j]);
        }
    } else {
        for (int i = vlo + tid; i < vhi; i += kTvThreads) {
            float xp[8], xq[8];
            load8<PB>(a.P, prow, 8 * i, a.V, false, xp);
            if constexpr (WITHQ) load8<QB>(a.Q, qrow, 8 * i, a.V, false, xq);
            f(i, xp, xq);
        }
    }
}

template <bool BF>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
    if constexpr (BF) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[idx] << 16);
    else return static_cast<const float*>(base)[idx];
}

struct TvShared {
    int parent[kTreeVerifyMaxNodes];
    int tok[kTreeVerifyMaxNodes];
    double segsum[kTvMaxSegs];
    float red_m[2][kTvWaves];
    float red_s[2][kTvWaves];
    int red_i[kTvWaves];
    double red_d[kTvWaves];
    uint32_t xv[kTreeSplitMax][4];   // exchanged values, by workgroup
    int xok;
    int xlast;   // this workgroup finished the split call last
    float clp[kTvThreads], clq[kTvThreads], cu[kTvThreads];   // children's logits and uniforms
};

// exp(y - lz) with the fp64 normaliser lz carried as a (hi, lo) float pair.
__device__ __forceinline__ float exp_rel(float y, float hi, float lo) {
    return __expf((y - hi) - lo);
}

// Block-wide sum of one fp64 value per thread; every thread gets the total
// (the partials are merged in the same order in every thread).
__device__ __forceinline__ double block_sum(TvShared& sh, double x) {
    x = wave_sum_f64(x);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.red_d[wave] = x;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kTvWaves; ++w) t += sh.red_d[w];
    return t;
}

// Exchange words of the split walk: [workgroup][parity][4] 64-bit words
// (tag << 32 | value), and one abort word.  Zero at load, and zeroed again by
// the last workgroup of every split call (tv_release), so each call starts
// from zeros, whether it is launched directly or replayed from a captured
// graph.  A tag is (epoch << 12) | exchange number with epoch >= 1, so a
// cleared word never matches.  Exchange s of a workgroup uses parity s & 1:
// it can only write exchange s + 2 after every workgroup of its request wrote
// s + 1, which each does after reading all of exchange s.
__device__ uint64_t tv_xchg[kTreeXchgWgs * 2 * 4 + 1];
constexpr int kTvAbortWord = kTreeXchgWgs * 2 * 4;
// Workgroups of the running split call that are done with the area.
__device__ unsigned tv_done;

struct TvGroup {
    int W, i;          // workgroups of the request, this one's index
    uint32_t epoch;
    unsigned limit;
    uint64_t* slots;   // the request's first exchange word
    uint32_t seq;      // exchanges so far
};

// Publishes this workgroup's four values for the next exchange and leaves
// every workgroup's values in sh.xv[0 .. W); false when a wait gave up (past
// the poll limit, or another workgroup of the launch gave up: the abort word
// holds the epoch).
__device__ __forceinline__ bool tv_exchange(TvShared& sh, TvGroup& g, uint32_t v0, uint32_t v1,
                                              uint32_t v2, uint32_t v3) {
    const int tid = threadIdx.x;
    const uint32_t mine = tid == 0 ? v0 : (tid == 1 ? v1 : (tid == 2 ? v2 : v3));
    __syncthreads();   // the previous exchange's values are read
    if (g.W == 1) {
        if (tid < 4) sh.xv[0][tid] = mine;
        __syncthreads();
        ++g.seq;
        return true;
    }
    const uint32_t tag = (g.epoch << 12) | (g.seq & 0xFFFu);
    const int par = (int)(g.seq & 1u);
    if (tid < 4)
        coh_store<true>(g.slots + ((size_t)g.i * 2 + par) * 4 + tid, ((uint64_t)tag << 32) | mine);
    if (tid < 64) {
        const int j = tid >> 2, w = tid & 3;
        int ok = 1;
        for (unsigned polls = 0;; ++polls) {
            bool up = true;
            // the abort word is read with the exchange words: one round trip a poll
            const uint64_t word = j < g.W ? coh_load<true>(g.slots + ((size_t)j * 2 + par) * 4 + w) : 0;
            const uint64_t ab = coh_load<true>(tv_xchg + kTvAbortWord);
            if (j < g.W) up = (uint32_t)(word >> 32) == tag;
            if (__all(up)) {
                if (j < g.W) sh.xv[j][w] = (uint32_t)word;
                break;
            }
            if (ab == (uint64_t)g.epoch || polls > g.limit) {
                if (tid == 0) coh_store<true>(tv_xchg + kTvAbortWord, (uint64_t)g.epoch);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (tid == 0) sh.xok = ok;
    }
    __syncthreads();
    ++g.seq;
    return sh.xok != 0;
}

__device__ __forceinline__ uint32_t f32_bits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ double f64_of(uint32_t lo, uint32_t hi) {
    return __hiloint2double((int)hi, (int)lo);
}
__device__ __forceinline__ uint32_t f64_lo(double x) { return (uint32_t)__double2loint(x); }
__device__ __forceinline__ uint32_t f64_hi(double x) { return (uint32_t)__double2hiint(x); }

template <bool PB, bool QB>
__device__ __forceinline__ void tree_walk(const TreeVerifyArgs& a, TvShared& sh) {
    const int W = a.split;
    const int b = (int)blockIdx.x / W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = a.M, V = a.V;
    const float invT = a.invT;
    int32_t* out = a.out_tokens + (size_t)b * (M + 1);
    int32_t* path = a.path ? a.path + (size_t)b * M : nullptr;
    const int nn = a.n_nodes ? a.n_nodes[b] : M;
    TvGroup grp;
    grp.W = W;
    grp.i = (int)blockIdx.x % W;
    grp.epoch = a.epoch;
    grp.limit = a.poll_limit;
    grp.slots = W > 1 ? tv_xchg + (size_t)b * W * 2 * 4 : tv_xchg;   // unused when W == 1
    grp.seq = 0;
    const bool lead = grp.i == 0;   // the workgroup that writes the outputs

    // The tree into LDS, checked: parents first, tokens in range.
    bool bad = nn < 0 || nn > M;
    for (int v = tid; v < M && !bad; v += kTvThreads) {
        const int pa = a.parent[(size_t)b * M + v];
        const int tk = a.tokens[(size_t)b * M + v];
        sh.parent[v] = pa;
        sh.tok[v] = tk;
        if (v < nn && (pa < -1 || pa >= v || tk < 0 || tk >= V)) bad = true;
    }
    bad = __syncthreads_or(bad);

    const size_t rows_b = (size_t)b * (M + 1);
    // whole 8-token vectors, each 16-byte aligned (the rows start 16-byte
    // aligned and hold a multiple of 8 tokens)
    const bool pvec = V % 8 == 0;
    const bool qvec = pvec;
    const int nvec = (V + 7) / 8;
    // this workgroup's segments and vectors
    const int nseg = (V + kTvSeg - 1) / kTvSeg;
    const int seg_lo = (int)((long long)grp.i * nseg / W);
    const int seg_hi = (int)((long long)(grp.i + 1) * nseg / W);
    const int nls = seg_hi - seg_lo;
    const int vlo = seg_lo * (kTvSeg / 8);
    const int vhi = min(nvec, seg_hi * (kTvSeg / 8));

    int node = -1, n = 0, final_tok = -1;
    while (!bad) {
        const size_t prow = (rows_b + (size_t)(node + 1)) * V;
        const size_t qrow = prow;   // Q has the same [B, M + 1, V] layout
        bool has_child = false;
        for (int c = node + 1; c < nn; ++c)
            if (sh.parent[c] == node) { has_child = true; break; }

        if (a.greedy) {
            // argmax of the node's target row, lowest id on ties
            float m = -INFINITY;
            int idx = INT_MAX;
            row_pass<PB, QB, false>(a, prow, qrow, vlo, vhi, pvec, [&](int i, float* x, float*) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (8 * i + e < V) merge_arg(m, idx, x[e], 8 * i + e);
            });
            wave_argmax_dpp(m, idx);
            __syncthreads();
            if (lane == 0) { sh.red_m[0][wave] = m; sh.red_i[wave] = idx; }
            __syncthreads();
            m = sh.red_m[0][0];
            idx = sh.red_i[0];
            for (int w = 1; w < kTvWaves; ++w) merge_arg(m, idx, sh.red_m[0][w], sh.red_i[w]);
            if (!tv_exchange(sh, grp, f32_bits(m), (uint32_t)idx, 0u, 0u)) { bad = true; break; }
            m = __uint_as_float(sh.xv[0][0]);
            idx = (int)sh.xv[0][1];
            for (int j = 1; j < W; ++j) merge_arg(m, idx, __uint_as_float(sh.xv[j][0]), (int)sh.xv[j][1]);
            if (m == -INFINITY) { bad = true; break; }
            int acc = -1;
            for (int c = node + 1; c < nn; ++c)
                if (sh.parent[c] == node && sh.tok[c] == idx) { acc = c; break; }
            if (acc < 0) { final_tok = idx; break; }
            if (lead && tid == 0 && path) path[n] = acc;
            if (lead && tid == 0) out[n] = sh.tok[acc];
            ++n;
            node = acc;
            continue;
        }

        // The first kTvThreads candidate children's logits at their tokens and
        // their uniforms: loaded now, used by the ratio tests after the pass.
        float c_lp = 0.0f, c_lq = 0.0f, c_u = 0.0f;
        const int c_id = node + 1 + tid;
        if (has_child) {
            const int x = c_id < nn ? sh.tok[c_id] : 0;
            c_lp = load1<PB>(a.P, prow + x);
            c_lq = load1<QB>(a.Q, qrow + x);
            if (a.uniforms) c_u = a.uniforms[rows_b + min(c_id, M - 1)];
        }

        // Normalisers of the node's target row and, with children, draft row.
        float mp = -INFINITY, sp = 0.0f, mq = -INFINITY, sq = 0.0f;
        auto absorb = [&](const float* x, float& m, float& sm) {
            float m8 = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) m8 = fmaxf(m8, x[e] * invT);
            if (m8 != -INFINITY) {
                float s8 = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) s8 += __expf(x[e] * invT - m8);
                merge_ms(m, sm, m8, s8, 1.0f);
            }
        };
        if (has_child)
            row_pass<PB, QB, true>(a, prow, qrow, vlo, vhi, pvec && qvec, [&](int, float* xp, float* xq) {
                absorb(xp, mp, sp);
                absorb(xq, mq, sq);
            });
        else
            row_pass<PB, QB, false>(a, prow, qrow, vlo, vhi, pvec,
                                    [&](int, float* xp, float*) { absorb(xp, mp, sp); });
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            merge_ms(mp, sp, __shfl_xor(mp, off), __shfl_xor(sp, off), 1.0f);
            merge_ms(mq, sq, __shfl_xor(mq, off), __shfl_xor(sq, off), 1.0f);
        }
        __syncthreads();
        if (lane == 0) {
            sh.red_m[0][wave] = mp; sh.red_s[0][wave] = sp;
            sh.red_m[1][wave] = mq; sh.red_s[1][wave] = sq;
        }
        if (has_child) {
            sh.clp[tid] = c_lp;
            sh.clq[tid] = c_lq;
            sh.cu[tid] = c_u;
        }
        __syncthreads();
        mp = sh.red_m[0][0]; sp = sh.red_s[0][0];
        mq = sh.red_m[1][0]; sq = sh.red_s[1][0];
        for (int w = 1; w < kTvWaves; ++w) {
            merge_ms(mp, sp, sh.red_m[0][w], sh.red_s[0][w], 1.0f);
            merge_ms(mq, sq, sh.red_m[1][w], sh.red_s[1][w], 1.0f);
        }
        if (!tv_exchange(sh, grp, f32_bits(mp), f32_bits(sp), f32_bits(mq), f32_bits(sq))) {
            bad = true;
            break;
        }
        mp = __uint_as_float(sh.xv[0][0]); sp = __uint_as_float(sh.xv[0][1]);
        mq = __uint_as_float(sh.xv[0][2]); sq = __uint_as_float(sh.xv[0][3]);
        for (int j = 1; j < W; ++j) {
            merge_ms(mp, sp, __uint_as_float(sh.xv[j][0]), __uint_as_float(sh.xv[j][1]), 1.0f);
            merge_ms(mq, sq, __uint_as_float(sh.xv[j][2]), __uint_as_float(sh.xv[j][3]), 1.0f);
        }
        if (mp == -INFINITY || (has_child && mq == -INFINITY)) { bad = true; break; }
        const double lzp = (double)mp + log((double)sp);
        const double lzq = has_child ? (double)mq + log((double)sq) : 0.0;
        const float lzp_hi = (float)lzp, lzp_lo = (float)(lzp - (double)lzp_hi);
        const float lzq_hi = (float)lzq, lzq_lo = (float)(lzq - (double)lzq_hi);

        // Ratio tests of the children in index order against r = max(0, p - c q) / W.
        double cc = 0.0, Wm = 1.0;
        int acc = -1;
        bool fallback = false;
        for (int ch = node + 1; ch < nn && has_child && !bad; ++ch) {
            if (sh.parent[ch] != node) continue;
            const int x = sh.tok[ch];
            const int ci = ch - node - 1;
            const bool pre = ci < kTvThreads;
            const float lpx = pre ? sh.clp[ci] : load1<PB>(a.P, prow + x);
            const float lqx = pre ? sh.clq[ci] : load1<QB>(a.Q, qrow + x);
            const double px = exp((double)lpx * (double)invT - lzp);
            const double qx = exp((double)lqx * (double)invT - lzq);
            const double rx = fmax(0.0, px - cc * qx) / Wm;
            const float u = a.uniforms ? (pre ? sh.cu[ci] : a.uniforms[rows_b + ch])
                                       : counter_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)ch, 3);
            if ((double)u * qx < rx) { acc = ch; break; }
            // failure: the residual's next mass
            cc += Wm;
            const float cf = (float)cc;
            double part = 0.0;
            row_pass<PB, QB, true>(a, prow, qrow, vlo, vhi, pvec && qvec, [&](int i, float* xp, float* xq) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float d = exp_rel(xp[e] * invT, lzp_hi, lzp_lo) -
                                    cf * exp_rel(xq[e] * invT, lzq_hi, lzq_lo);
                    part += (d > 0.0f && 8 * i + e < V) ? (double)d : 0.0;
                }
            });
            part = block_sum(sh, part);
            if (!tv_exchange(sh, grp, f64_lo(part), f64_hi(part), 0u, 0u)) { bad = true; break; }
            Wm = 0.0;
            for (int j = 0; j < W; ++j) Wm += f64_of(sh.xv[j][0], sh.xv[j][1]);
            if (!(Wm > 0.0)) { fallback = true; break; }
        }
        if (bad) break;
        if (acc >= 0) {
            if (lead && tid == 0 && path) path[n] = acc;
            if (lead && tid == 0) out[n] = sh.tok[acc];
            ++n;
            node = acc;
            continue;
        }

        // Final draw: weights max(0, p - c q) (residual after failures) or p.
        const bool resid = has_child && !fallback && cc > 0.0;
        const float cf = resid ? (float)cc : 0.0f;
        const float uf = a.uniforms ? a.uniforms[rows_b + M]
                                    : counter_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)M, 3);
        auto weights8 = [&](int v0, float w[8]) {
            float xp[8], xq[8];
            load8<PB>(a.P, prow, v0, V, pvec, xp);
            if (resid) load8<QB>(a.Q, qrow, v0, V, qvec, xq);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float d = exp_rel(xp[e] * invT, lzp_hi, lzp_lo);
                if (resid) d -= cf * exp_rel(xq[e] * invT, lzq_hi, lzq_lo);
                w[e] = (v0 + e < V && d > 0.0f) ? d : 0.0f;
            }
        };
        // sums of this workgroup's segments (one wave each, the loads of
        // kTvSegBatch segments issued together), then its range total
        for (int sl0 = wave; sl0 < nls; sl0 += kTvWaves * kTvSegBatch) {
            float xp[kTvSegBatch][8], xq[kTvSegBatch][8];
#pragma unroll
            for (int j = 0; j < kTvSegBatch; ++j) {
                const int sl = min(sl0 + j * kTvWaves, nls - 1);
                const int v0 = (seg_lo + sl) * kTvSeg + 8 * lane;
                load8<PB>(a.P, prow, v0, V, pvec, xp[j]);
                if (resid) load8<QB>(a.Q, qrow, v0, V, qvec, xq[j]);
            }
#pragma unroll
            for (int j = 0; j < kTvSegBatch; ++j) {
                const int sl = sl0 + j * kTvWaves;
                if (sl >= nls) break;
                const int v0 = (seg_lo + sl) * kTvSeg + 8 * lane;
                double t = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float d = exp_rel(xp[j][e] * invT, lzp_hi, lzp_lo);
                    if (resid) d -= cf * exp_rel(xq[j][e] * invT, lzq_hi, lzq_lo);
                    t += (v0 + e < V && d > 0.0f) ? (double)d : 0.0;
                }
                t = wave_sum_f64(t);
                if (lane == 0) sh.segsum[sl] = t;
            }
        }
        __syncthreads();
        // segments per lane, contiguous: lane l holds segments l*per .. l*per + per - 1;
        // every wave forms the same lane sums and total
        const int per = (nls + 63) / 64;
        double ls = 0.0;
        for (int j = 0; j < per; ++j) {
            const int sl = lane * per + j;
            if (sl < nls) ls += sh.segsum[sl];
        }
        const double mytot = readlane_f64(wave_inclusive_scan_f64(ls), 63);
        if (!tv_exchange(sh, grp, f64_lo(mytot), f64_hi(mytot), 0u, 0u)) { bad = true; break; }
        // the range holding u * total: past the end (rounding) the last range
        // with weight and +inf, as inside a range
        double total = 0.0;
        for (int j = 0; j < W; ++j) total += f64_of(sh.xv[j][0], sh.xv[j][1]);
        const double thr = (double)uf * total;
        int owner = -1, lastj = 0;
        double before = 0.0, rem0 = INFINITY;
        for (int j = 0; j < W; ++j) {
            const double tj = f64_of(sh.xv[j][0], sh.xv[j][1]);
            if (tj > 0.0) {
                lastj = j;
                if (owner < 0 && thr < before + tj) {
                    owner = j;
                    rem0 = thr - before;
                }
            }
            before += tj;
        }
        if (owner < 0) owner = lastj;
        int tok_mine = -1;
        if (grp.i == owner && wave == 0) {
            double rem;
            const int L = wave_pick(ls, rem0, rem);
            // walk lane L's segments (uniform: every lane reads the same LDS words)
            int sel = -1, lastpos = -1;
            for (int j = 0; j < per; ++j) {
                const int sl = L * per + j;
                if (sl >= nls) break;
                const double sv = sh.segsum[sl];
                if (sv > 0.0) {
                    lastpos = sl;
                    if (rem < sv) { sel = sl; break; }
                    rem -= sv;
                }
            }
            if (sel < 0) { sel = lastpos < 0 ? 0 : lastpos; rem = INFINITY; }
            float w[8];
            weights8((seg_lo + sel) * kTvSeg + 8 * lane, w);
            double t = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) t += (double)w[e];
            double rem2;
            const int L2 = wave_pick(t, rem, rem2);
            // the 8 weights of lane L2, uniform
            int tok = -1, lastp = -1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double we = (double)readlane_f32(w[e], L2);
                if (we > 0.0) {
                    lastp = e;
                    if (tok < 0) {
                        if (rem2 < we) tok = e;
                        else rem2 -= we;
                    }
                }
            }
            if (tok < 0) tok = lastp < 0 ? 0 : lastp;
            if (lane == 0) sh.red_i[0] = min((seg_lo + sel) * kTvSeg + 8 * L2 + tok, V - 1);
        }
        __syncthreads();
        if (grp.i == owner) tok_mine = sh.red_i[0];
        // the owner hands the token to every workgroup of the request
        if (!tv_exchange(sh, grp, (uint32_t)tok_mine, 0u, 0u, 0u)) { bad = true; break; }
        final_tok = (int)sh.xv[owner][0];
        break;
    }

    if (!lead) return;
    if (bad) {
        for (int j = tid; j <= M; j += kTvThreads) out[j] = -1;
        if (path) for (int j = tid; j < M; j += kTvThreads) path[j] = -1;
        if (tid == 0) a.accepted[b] = -1;
        return;
    }
    __syncthreads();   // the path's writes by thread 0 precede the tail
    for (int j = n + 1 + tid; j <= M; j += kTvThreads) out[j] = -1;
    if (path) for (int j = n + tid; j < M; j += kTvThreads) path[j] = -1;
    if (tid == 0) {
        out[n] = final_tok;
        a.accepted[b] = n;
    }
}

// End of a split call, in every workgroup: the count of finished workgroups
// is an acquire-release add, so the last one to finish sees every other
// workgroup's accesses to the area completed; it zeroes the words the call
// used, the abort word and the count.
__device__ __forceinline__ void tv_release(TvShared& sh, const TreeVerifyArgs& a) {
    __syncthreads();   // every thread of this workgroup is done with the area
    if (threadIdx.x == 0) {
        const unsigned d = __hip_atomic_fetch_add(&tv_done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        sh.xlast = d == gridDim.x - 1 ? 1 : 0;
    }
    __syncthreads();
    if (sh.xlast) {
        const int nw = a.B * a.split * 2 * 4;
        for (int e = (int)threadIdx.x; e < nw; e += kTvThreads) coh_store<true>(tv_xchg + e, (uint64_t)0);
        if (threadIdx.x == 0) {
            coh_store<true>(tv_xchg + kTvAbortWord, (uint64_t)0);
            coh_store<true>(&tv_done, 0u);
        }
    }
}

template <bool PB, bool QB>
__global__ __launch_bounds__(kTvThreads) void verify_tree_kernel(TreeVerifyArgs a) {
    __shared__ TvShared sh;
    tree_walk<PB, QB>(a, sh);
    if (a.split > 1) tv_release(sh, a);
}

}  // namespace

// Workgroups per request: all of them must be resident at once (the split
// walk's workgroups wait for each other), so B * W stays within the device's
// CUs; one per request when B fills the device.  A segment per workgroup at
// least.
static int tree_split(int B, int V) {
    static std::atomic<int> cus_cache[64];
    int dev = 0;
    (void)hipGetDevice(&dev);
    int cus = 0;
    if (dev >= 0 && dev < 64) cus = cus_cache[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 1;
        if (dev >= 0 && dev < 64) cus_cache[dev].store(cus, std::memory_order_relaxed);
    }
    const int nseg = (V + kTvSeg - 1) / kTvSeg;
    int w = std::min(std::min(kTreeSplitMax, cus / std::max(B, 1)), nseg);
    if ((long long)B * w > kTreeXchgWgs) w = kTreeXchgWgs / B;
    return std::max(w, 1);
}

hipError_t verify_tree_launch(const TreeVerifyArgs& a, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    TreeVerifyArgs x = a;
    x.split = tree_split(a.B, a.V);
    // every split call starts from a zeroed area (the last workgroup of the
    // previous one cleared it), so one fixed nonzero epoch serves all calls
    x.epoch = 1u;
    if (x.poll_limit == 0) x.poll_limit = kTreePollLimit;
    const dim3 grid((unsigned)((size_t)a.B * x.split)), block(kTvThreads);
    if (a.p_bf16 && a.q_bf16) hipLaunchKernelGGL((verify_tree_kernel<true, true>), grid, block, 0, s, x);
    else if (a.p_bf16) hipLaunchKernelGGL((verify_tree_kernel<true, false>), grid, block, 0, s, x);
    else if (a.q_bf16) hipLaunchKernelGGL((verify_tree_kernel<false, true>), grid, block, 0, s, x);
    else hipLaunchKernelGGL((verify_tree_kernel<false, false>), grid, block, 0, s, x);
    return hipGetLastError();
}

}  // namespace specdec
