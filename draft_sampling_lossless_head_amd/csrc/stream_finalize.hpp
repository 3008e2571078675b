// Finalize of the streaming q-free draft, shared by the per-position kernel
// and the persistent draft ("[논문리뷰] DSpark ...", §1.2 Sequential stage:
// one draw per position from the softmax of the draft logits).
#pragma once

#include <climits>

#include "device_common.hpp"
#include "launch.hpp"

namespace specdec {

// ---------------------------------------------------------------------------
// Finalize of the streaming q-free draft.  One wave per request row (no
// workgroup barriers; the caller is one whole wave); the inverse-CDF descent takes three dependent reads:
//   1. the row's ws <= 256 share summaries, four per lane: max, normaliser and
//      the share holding u * Z (fp64 weights and scan);
//   2. the share's 32-token segments (max and 4 group sums), read together:
//      the segment, then the 8-token group;
//   3. the group's 8 logits rebuilt as U + W1[prev] . W2 (the W1 row slice is
//      fetched at entry), then the token.
// Scaling factors use fp32 exponentials (relative error ~1e-7); sums, scans
// and the threshold are fp64.
// ---------------------------------------------------------------------------
struct FinStreamArgs {
    const SegStat* sup;     // [ws][bpad] share summaries
    const float* segm;      // [segments][bpad] max of each 32-token segment
    const float* gsums;     // [segments][bpad][4] 8-token group sums relative to it
    // share j covers segments seg_mult * floor(j * nunit / ws) .. (the same
    // for j + 1), at most 64 of them
    int ws, nunit, seg_mult, bpad;
    const int32_t* x0;
    int32_t* tokens;
    float* q_logZ;
    float* q_tok;
    const float* uniforms;
    uint64_t seed;
    uint32_t offset;
    int gamma, V;
    float invT;
    int greedy;
    const void* U;          // [B, gamma, V], bf16 or (u_f32) fp32
    int u_f32;
    const uint16_t* W1;     // [V, r]
    const uint16_t* W2P;    // packed W2 image
    int r;
    // Optional (persistent draft): after the token of row b, the word
    // ((k + 1) << 32) | token is written here, last.
    uint64_t* tflag;
    // Persistent draft: abort word and poll limit of the bounded waits.
    unsigned* abort_word;
    unsigned poll_limit;
};


// COH: the summaries and earlier tokens were written in the same launch by
// workgroups on other XCDs (the persistent draft).  TAGGED: each share
// summary is two 64-bit words (m, k + 1) and (s or argmax, k + 1), written
// once the share's segment summaries are out; the wave polls its row's
// shares until every tag reads k + 1 (bounded; gives up through the abort
// word), so no grid barrier precedes the finalize.
// xprev_lds / e_lds (optional, row b < 128): the conditioning token of row b
// (-1 if invalid) and the rows W1[prev] of the 128-row block already in LDS,
// 16-byte chunk c of row m in slot c ^ (m & 7).
// Returns false only when a tagged wait gave up (abort word set).
template <bool COH, bool TAGGED = false>
__device__ __forceinline__ bool finalize_row_stream(const FinStreamArgs& A, int b, int k,
                                                    int lane, const int* xprev_lds = nullptr,
                                                    const uint16_t* e_lds = nullptr) {
    const size_t outi = (size_t)b * A.gamma + k;
    const int V = A.V;
    const float invT = A.invT;
    auto put_token = [&](int tok) {   // lane 0
        coh_store<COH>(A.tokens + outi, tok);
        if (A.tflag)
            coh_store<COH>(A.tflag + b, ((uint64_t)(k + 1) << 32) | (uint64_t)(uint32_t)tok);
    };

    const int prev = xprev_lds ? xprev_lds[b]
                               : (k == 0) ? A.x0[b] : coh_load<COH>(A.tokens + outi - 1);
    if (prev < 0 || prev >= V) {
        if (lane == 0) {
            if (A.q_logZ) A.q_logZ[outi] = NAN;
            if (A.q_tok) A.q_tok[outi] = NAN;
            put_token(-1);
        }
        return true;
    }
    const float u = A.uniforms ? A.uniforms[outi] : counter_uniform(A.seed, A.offset, b, k, 0);
    // this lane's W1 slice for the rebuild (lane = 8t + sl: rank slice sl)
    const int span = A.r / 8;   // <= 32 bf16: at most 4 chunks of 16 bytes
    uint4 w1c[4];
    if (e_lds && (span & 7) == 0) {
        const uint16_t* er = e_lds + (size_t)b * A.r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kc = (lane & 7) * (span >> 3) + q;
            w1c[q] = (q * 8 < span) ? *reinterpret_cast<const uint4*>(er + ((kc ^ (b & 7)) << 3))
                                    : make_uint4(0u, 0u, 0u, 0u);
        }
    } else {
        const uint16_t* w1 = A.W1 + (size_t)prev * A.r + (lane & 7) * span;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w1c[q] = (q * 8 < span) ? *reinterpret_cast<const uint4*>(w1 + q * 8)
                                    : make_uint4(0u, 0u, 0u, 0u);
    }

    // 1) share summaries, four per lane (shares 4 * lane + q).
    float sm[4], ss[4];
    int si[4];
    if constexpr (TAGGED) {
        const uint64_t* s64 = reinterpret_cast<const uint64_t*>(A.sup);
        const uint32_t tag = (uint32_t)(k + 1);
        for (unsigned polls = 0;; ++polls) {
            bool up = true;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = 4 * lane + q;
                if (j < A.ws) {
                    const size_t e = 2 * ((size_t)j * A.bpad + b);
                    const uint64_t w0 = coh_load<true>(s64 + e);
                    const uint64_t w1 = coh_load<true>(s64 + e + 1);
                    up = up && (uint32_t)(w0 >> 32) == tag && (uint32_t)(w1 >> 32) == tag;
                    sm[q] = __uint_as_float((uint32_t)w0);
                    ss[q] = __uint_as_float((uint32_t)w1);
                    si[q] = (int)(uint32_t)w1;
                } else {
                    sm[q] = -INFINITY;
                    ss[q] = 0.0f;
                    si[q] = INT_MAX;
                }
            }
            if (__all(up)) break;
            if (coh_load<true>(A.abort_word) != 0u || polls > A.poll_limit) {
                if (lane == 0) coh_store<true>(A.abort_word, 1u);
                return false;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = 4 * lane + q;
            if (j < A.ws) {
                const SegStat x = coh_load_seg<COH>(A.sup + (size_t)j * A.bpad + b);
                sm[q] = x.m;
                ss[q] = x.s;
                si[q] = x.idx;
            } else {
                sm[q] = -INFINITY;
                ss[q] = 0.0f;
                si[q] = INT_MAX;
            }
        }
    }
    float M = sm[0];
    int AM = si[0];
#pragma unroll
    for (int q = 1; q < 4; ++q) merge_arg(M, AM, sm[q], si[q]);
    if (A.greedy) wave_argmax_dpp(M, AM);   // uniform from here on
    else M = wave_max_f32_dpp(M);
    if (A.greedy || M == -INFINITY) {
        if (lane == 0) {
            if (A.q_logZ) A.q_logZ[outi] = M == -INFINITY ? NAN : M;
            if (A.q_tok) A.q_tok[outi] = M == -INFINITY ? NAN : 1.0f;
            put_token((M == -INFINITY) ? -1 : AM);
        }
        return true;
    }
    double w[4];
    double lsum = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        w[q] = sm[q] != -INFINITY ? (double)ss[q] * (double)__expf((sm[q] - M) * invT) : 0.0;
        lsum += w[q];
    }
    const double Z = readlane_f64(wave_inclusive_scan_f64(lsum), kWave - 1);
    const double thr = (double)u * Z;
    double rem;
    const int ol = wave_pick(lsum, thr, rem);
    // the owning lane walks its four shares
    int qsel = 3;
    double qrem = INFINITY;
    {
        double run = 0.0;
        int last = -1;
        double last_run = 0.0;
        int found = -1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (found < 0 && w[q] > 0.0) {
                last = q;
                last_run = run;
                if (rem < run + w[q]) {
                    found = q;
                    qrem = rem - run;
                }
            }
            run += w[q];
        }
        if (found < 0) {
            found = last < 0 ? 0 : last;
            qrem = rem == INFINITY ? INFINITY : rem - last_run;
        }
        qsel = found;
    }
    const int sh = 4 * ol + __builtin_amdgcn_readlane(qsel, ol);
    const double rem1 = readlane_f64(qrem, ol);

    // 2) the share's 32-token segments and their group sums, one read.
    const int s0 = A.seg_mult * (int)((long long)sh * A.nunit / A.ws);
    const int s1 = A.seg_mult * (int)((long long)(sh + 1) * A.nunit / A.ws);
    const int sg = s0 + lane;
    const bool have = sg < s1;   // at most 64 segments per share (launcher guarantee)
    float ym = -INFINITY;
    float4 g4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (have) {
        const size_t sx = (size_t)sg * A.bpad + b;
        ym = coh_load<COH>(A.segm + sx);
        g4 = coh_load_f32x4<COH>(A.gsums + sx * 4);
    }
    const double ysc = ym != -INFINITY ? (double)__expf((ym - M) * invT) : 0.0;
    const double ys = ((double)g4.x + (double)g4.y) + ((double)g4.z + (double)g4.w);
    double rem2;
    const int sl_seg = wave_pick(ys * ysc, rem1, rem2);
    const int seg = s0 + sl_seg;
    // the chosen segment's 4 group weights to lanes 0..3
    const double gscale = readlane_f64(ysc, sl_seg);
    const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
    float mine = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float v = readlane_f32(gv[g], sl_seg);
        if (lane == g) mine = v;
    }
    double grem;
    const int grp = wave_pick(lane < 4 ? (double)mine * gscale : 0.0, rem2, grem);

    // 3) rebuild the group's 8 logits: lane = 8t + sl.
    const int t = lane >> 3, sl = lane & 7;
    const int vt = seg * kStreamSeg + grp * 8 + t;
    float part = 0.0f;
    float ut = 0.0f;
    if (vt < V) {
        const int nswz = w2p_swizzle(vt & (kPackTile - 1), A.r >> 3);
        if ((span & 7) == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q * 8 < span) {
                    const int kc = sl * (span >> 3) + q;
                    const uint4 c = *reinterpret_cast<const uint4*>(
                        A.W2P + (size_t)vt * A.r + ((kc ^ nswz) << 3));
                    const uint32_t aw[4] = {w1c[q].x, w1c[q].y, w1c[q].z, w1c[q].w};
                    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        part = fmaf(bf16_bits_to_float(aw[h] & 0xFFFFu),
                                    bf16_bits_to_float(cw[h] & 0xFFFFu), part);
                        part = fmaf(bf16_bits_to_float(aw[h] >> 16),
                                    bf16_bits_to_float(cw[h] >> 16), part);
                    }
                }
            }
        } else {   // span < 8 (r < 64)
            const uint16_t* w1 = A.W1 + (size_t)prev * A.r;
            for (int j = sl * span; j < (sl + 1) * span; ++j)
                part = fmaf(bf16_bits_to_float(w1[j]),
                            bf16_bits_to_float(A.W2P[w2p_index(vt, j, A.r)]), part);
        }
        ut = A.u_f32 ? static_cast<const float*>(A.U)[outi * (size_t)V + vt]
                     : bf16_bits_to_float(static_cast<const uint16_t*>(A.U)[outi * (size_t)V + vt]);
    }
    part = row8_sum(part);
    const float lt = ut + part;
    const float wtk = vt < V ? __expf((lt - M) * invT) : 0.0f;
    // token t's weight and logit to lane t
    float w8 = 0.0f, l8 = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float wq = readlane_f32(wtk, 8 * q);
        const float lq = readlane_f32(lt, 8 * q);
        if (lane == q) {
            w8 = wq;
            l8 = lq;
        }
    }
    double trem;
    const int tsel = wave_pick(lane < 8 ? (double)w8 : 0.0, grem, trem);
    const float lsel = readlane_f32(l8, tsel);
    if (lane == 0) {
        if (A.q_logZ) A.q_logZ[outi] = (float)((double)M * (double)invT + (double)__logf((float)Z));
        if (A.q_tok) A.q_tok[outi] = (float)((double)__expf((lsel - M) * invT) / Z);
        put_token(min(seg * kStreamSeg + grp * 8 + tsel, V - 1));
    }
    return true;
}

}  // namespace specdec
