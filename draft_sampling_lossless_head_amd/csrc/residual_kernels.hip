// Final draw of q-free verification ("Speculative Decoding Part 1", section
// "수락 규칙": after the first rejection at position n the token comes from the
// residual normalize(max(0, p_n - q_n)); after L acceptances from p_L).  The
// draft row q_n = U_n + W1[x_{n-1}] . W2 is rebuilt on the fly, streamed as in
// the q-free draft, and never written out:
//
//   verify_resid_stream    one persistent workgroup per CU: per 64-token slice
//                          x 128 rows the weights w = max(0, p_n - q_n)
//                          (residual rows) or p_L (bonus rows), summed per
//                          8-token group and per (row, workgroup share);
//   verify_resid_finalize  one wave per row: inverse CDF over share sums ->
//                          32-token segment -> 8-token group -> the token, from
//                          8 rebuilt weights.  A residual without mass after
//                          rounding falls back to p_n (exact two-pass scan).
#include <algorithm>
#include <type_traits>
#include <mutex>
#include <climits>

#include "device_common.hpp"
#include "launch.hpp"

namespace specdec {

constexpr int kResidStages = 4;   // W2 ring: items i+1 .. i+3 stream in while item i is used
typedef float f32x4_t __attribute__((ext_vector_type(4)));


// What one request row contributes: mode 1 residual (n < L), 2 bonus (n = L),
// 0 nothing (greedy or invalid).
struct RowInfo {
    int mode, n;
    size_t prow, urow;                 // element offsets of P_n and U_n
    float lzp_hi, lzp_lo, lzq_hi, lzq_lo;
};

__device__ __forceinline__ RowInfo resid_row_of(const ResidArgs& A, int b, const FinalInfo& f) {
    RowInfo ri;
    ri.mode = 0;
    ri.n = 0;
    ri.prow = ri.urow = 0;
    ri.lzp_hi = ri.lzp_lo = ri.lzq_hi = ri.lzq_lo = 0.0f;
    if (b >= A.B) return ri;
    if (f.mode != 1 && f.mode != 2) return ri;
    ri.mode = f.mode;
    ri.n = f.n;
    ri.prow = (size_t)((A.p_row_off ? A.p_row_off[b] : (int64_t)b * (A.G + 1)) + f.n) * A.V;
    ri.urow = f.mode == 1 ? ((size_t)b * A.G + f.n) * A.V : 0;
    ri.lzp_hi = (float)f.logZp;
    ri.lzp_lo = (float)(f.logZp - (double)ri.lzp_hi);
    ri.lzq_hi = (float)f.logZq;
    ri.lzq_lo = (float)(f.logZq - (double)ri.lzq_hi);
    return ri;
}

__device__ __forceinline__ RowInfo resid_row(const ResidArgs& A, int b) {
    return resid_row_of(A, b, A.fin[min(b, A.B - 1)]);
}

// Weight of one token: p = exp(lp / T - logZp), q = exp(lq / T - logZq), the
// normalisers applied as fp32 (hi, lo) pairs.
__device__ __forceinline__ float resid_weight(const RowInfo& ri, float lp, float lq, float invT) {
    const float p = __expf(fmaf(lp, invT, -ri.lzp_hi) - ri.lzp_lo);
    if (ri.mode != 1) return ri.mode == 2 ? p : 0.0f;
    const float q = __expf(fmaf(lq, invT, -ri.lzq_hi) - ri.lzq_lo);
    return fmaxf(p - q, 0.0f);
}

// Normalisers of one row as exp2 offsets: p = 2^(lp a + cp), q = 2^(lq a + cq)
// with a = log2(e) / T and c = -logZ log2(e) as fp32 (hi, lo) pairs; q = 0
// (cq = -inf) for rows without a residual, so max(0, p - q) = p for bonus rows.
struct RowExp2 {
    float cp_hi, cp_lo, cq_hi, cq_lo;
};

__device__ __forceinline__ RowExp2 row_exp2(const FinalInfo& f, int mode) {
    RowExp2 x;
    x.cp_hi = x.cp_lo = 0.0f;
    x.cq_hi = -INFINITY;
    x.cq_lo = 0.0f;
    if (mode == 0) return x;
    const double l2e = 1.4426950408889634;
    const double cp = -f.logZp * l2e;
    x.cp_hi = (float)cp;
    x.cp_lo = (float)(cp - (double)x.cp_hi);
    if (mode == 1) {
        const double cq = -f.logZq * l2e;
        x.cq_hi = (float)cq;
        x.cq_lo = (float)(cq - (double)x.cq_hi);
    }
    return x;
}

// Weight of one token in both kernels, with the same operations in the same
// order, so that the rebuild of a group reproduces the streamed weights
// exactly when it reproduces the logits: max(0, p - q), p for bonus rows.
__device__ __forceinline__ float resid_w(float lp, float lq, float a2, const RowExp2& cz) {
    const float p = __builtin_amdgcn_exp2f(fmaf(lp, a2, cz.cp_hi) + cz.cp_lo);
    const float q = __builtin_amdgcn_exp2f(fmaf(lq, a2, cz.cq_hi) + cz.cq_lo);
    return fmaxf(p - q, 0.0f);
}

__device__ __forceinline__ float exp2_scale(float invT) { return invT * 1.4426950408889634f; }

// One persistent workgroup per (row block, share) of 64-token items x 128
// rows.  Wave w owns rows 16w .. 16w + 15 and all 64 tokens of an item on
// 16x16x32 MFMAs: A is the packed W2 slice from LDS (tile m, operand row i is
// token 32 (m >> 1) + 8 (i >> 2) + 4 (m & 1) + (i & 3)), B is the row's
// conditioning embedding from registers.  Lane (n, kq) = (lane & 15, lane >> 4)
// then holds, for row 16w + n, the 8-token groups kq of both 32-token
// segments of the item, in token order: the U_n and P_n values it needs are
// two 16-byte loads each, straight into registers (a wave's load covers 64
// contiguous bytes of 16 rows), its accumulators start at U_n, and its group
// sums need no exchange.  Only W2 goes through LDS, in a ring of four stages;
// item i+3's loads go out before item i is used, so three items (~190 KB per
// CU) are in flight.  Every load is issued for every item, with addresses
// clamped for items past the share, so the wait counts are fixed.
template <int NK>
__global__ __launch_bounds__(kStreamWaves * 64, 1)
void verify_resid_stream(ResidArgs A, int nitem_v, int nrb, int ws) {
    constexpr int R = NK * 32;
    constexpr int W2B = kStreamItem * R * 2;           // packed W2 slice of one item
    constexpr int W2P = W2B / 1024 / kStreamWaves;     // 1 KB direct-load pieces per wave
    constexpr int NCH = R / 8;
    constexpr int LD = W2P + 4;                        // loads per item and wave
    constexpr int NS = kResidStages;                   // stages = register sets = lookahead + 1
    static_assert(W2P >= 1 && kStreamWaves * 16 == kStreamRows && 2 * LD < 64, "piece split");
    static_assert(NS == 4, "the loop below is unrolled for four stages");
    extern __shared__ __align__(16) char smem_r[];
    const int V = A.V;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, kq = lane >> 4;
    const int rb0 = (int)blockIdx.x / ws;
    const int jw = (int)blockIdx.x % ws;
    const int lo = (int)((long long)jw * nitem_v / ws);
    const int hi = (int)((long long)(jw + 1) * nitem_v / ws);
    const int my_n = hi - lo;
    if (my_n <= 0) return;   // whole workgroup: no share (the launch keeps ws <= nitem_v)
    const size_t bpad = (size_t)nrb * kStreamRows;

    const int bl = 16 * wave + n16;
    const int b = rb0 * kStreamRows + bl;
    // The decision and the anchor token load together; the conditioning token
    // of q_n is the anchor (n = 0) or the draft token the decide pass recorded.
    const int bc = min(b, A.B - 1);
    const FinalInfo fi = A.fin[bc];
    const int x0b = A.x0[bc];
    const RowInfo me = resid_row_of(A, b, fi);
    const RowExp2 cz = row_exp2(fi, me.mode);
    const float a2 = exp2_scale(A.invT);
    // B operand: E = W1[x_{n-1}], k = 32 kk + 8 kq .. + 7 (row 0 of W1 for
    // rows without a residual, whose q is not used).  Issued before the first
    // items, so waiting for item 0 covers it.
    bf16x8_t e[NK];
    {
        int prev = me.n == 0 ? x0b : fi.prev;
        prev = (me.mode == 1 && prev >= 0 && prev < V) ? prev : 0;   // verify_decide has checked it
        const uint16_t* erow = A.W1 + (size_t)prev * R + 8 * kq;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) e[kk] = *reinterpret_cast<const bf16x8_t*>(erow + 32 * kk);
    }
    const bool uok = me.mode == 1, pok = me.mode != 0;
    const uint16_t* ubase = A.U + me.urow + 8 * kq;
    const uint16_t* pbase = A.P + me.prow + 8 * kq;

    // A operand rows of this lane: token tm[m] of the item; its chunk swizzle
    // depends on the token's place in its 128-token pack tile.
    int tm[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) tm[m] = 32 * (m >> 1) + 8 * (n16 >> 2) + 4 * (m & 1) + (n16 & 3);

    u32x4_t uv[NS][2], pv[NS][2];
    auto issue_w2 = [&](int i) {
        const int iv = lo + min(i, my_n - 1);
        char* st = smem_r + (i % NS) * W2B;
        const char* wsrc = reinterpret_cast<const char*>(A.W2P) + (size_t)iv * W2B;
#pragma unroll
        for (int q = 0; q < W2P; ++q) {
            const int pc = q * kStreamWaves + wave;
            __builtin_amdgcn_global_load_lds(wsrc + pc * 1024 + lane * 16,
                                             (lds_ptr_t)(st + pc * 1024), 16, 0, 0);
        }
    };
    auto issue_up = [&](auto S, int i) {
        constexpr int s_ = decltype(S)::value;
        const int t = (lo + min(i, my_n - 1)) * kStreamItem;
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            const bool in = t + 32 * sg + 8 * kq < V;
            const uint16_t* us = (uok && in) ? ubase + t + 32 * sg : A.U;
            uv[s_][sg] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(us));
        }
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            const bool in = t + 32 * sg + 8 * kq < V;
            const uint16_t* ps = (pok && in) ? pbase + t + 32 * sg : A.P;
            pv[s_][sg] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ps));
        }
    };

    float run = 0.0f;   // this lane's part of the share's weight for its row
    auto step = [&](auto S, int i) {
        constexpr int s_ = decltype(S)::value;
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<(NS - 2) * LD>();                  // item i: items i+1, i+2 may be pending
        asm volatile("s_barrier" ::: "memory");    // every wave's W2 pieces of item i; item
        issue_w2(i + NS - 1);                      // i-1's stage and registers are free
        __builtin_amdgcn_sched_barrier(0);
        issue_up(std::integral_constant<int, (s_ + NS - 1) % NS>{}, i + NS - 1);
        __builtin_amdgcn_sched_barrier(0);
        const int iv = lo + i;
        const uint16_t* w2s = reinterpret_cast<const uint16_t*>(smem_r + (i % NS) * W2B);
        // accumulators start at U_n: acc[2 sg + (j >> 2)][j & 3] is token
        // iv*64 + 32 sg + 8 kq + j
        f32x4_t acc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = 4 * (m & 1) + c;
                const uint32_t wu = uv[s_][m >> 1][j >> 1];
                acc[m][c] = (j & 1) ? __uint_as_float(wu & 0xFFFF0000u) : __uint_as_float(wu << 16);
            }
        // operand (m, kk): chunk 4 kk + kq of token row tm[m], slot (4 kk + kq) ^ sw
        int abase[4], c0[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            abase[m] = tm[m] * R;
            c0[m] = kq ^ w2p_swizzle((iv & 1) * kStreamItem + tm[m], NCH);
        }
        auto lda = [&](int m, int kk) {
            return *reinterpret_cast<const bf16x8_t*>(w2s + abase[m] + (((4 * kk) ^ c0[m]) << 3));
        };
        bf16x8_t a0[4], a1[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) a0[m] = lda(m, 0);
#pragma unroll
        for (int kk = 0; kk < NK; kk += 2) {
#pragma unroll
            for (int m = 0; m < 4; ++m) a1[m] = lda(m, kk + 1);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[m], e[kk], acc[m], 0, 0, 0);
            if (kk + 2 < NK) {
#pragma unroll
                for (int m = 0; m < 4; ++m) a0[m] = lda(m, kk + 2);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[m], e[kk + 1], acc[m], 0, 0, 0);
        }
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            float g = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t wp = pv[s_][sg][j >> 1];
                const float lp = (j & 1) ? __uint_as_float(wp & 0xFFFF0000u) : __uint_as_float(wp << 16);
                g += resid_w(lp, acc[2 * sg + (j >> 2)][j & 3], a2, cz);
            }
            g = iv * kStreamItem + 32 * sg + 8 * kq < V ? g : 0.0f;
            A.gsums[((2 * (size_t)iv + sg) * bpad + b) * 4 + kq] = g;
            run += g;
        }
    };

    // Issue order E, W2(0) UP(0) .. W2(2) UP(2), then per step W2(i+3) UP(i+3):
    // after item i's last load come exactly items i+1 and i+2 (stores aside).
    __builtin_amdgcn_sched_barrier(0);
    issue_w2(0);
    __builtin_amdgcn_sched_barrier(0);
    issue_up(std::integral_constant<int, 0>{}, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue_w2(1);
    __builtin_amdgcn_sched_barrier(0);
    issue_up(std::integral_constant<int, 1>{}, 1);
    __builtin_amdgcn_sched_barrier(0);
    issue_w2(2);
    __builtin_amdgcn_sched_barrier(0);
    issue_up(std::integral_constant<int, 2>{}, 2);
    // Whole rounds of four steps, then the last zero to three steps outside the
    // loop (an exit from inside a round would let the compiler merge
    // pending-load states at the loop head and drain every load there).
    int i = 0;
    for (; i + NS - 1 < my_n; i += NS) {
        step(std::integral_constant<int, 0>{}, i);
        step(std::integral_constant<int, 1>{}, i + 1);
        step(std::integral_constant<int, 2>{}, i + 2);
        step(std::integral_constant<int, 3>{}, i + 3);
    }
    if (i < my_n) step(std::integral_constant<int, 0>{}, i);
    if (i + 1 < my_n) step(std::integral_constant<int, 1>{}, i + 1);
    if (i + 2 < my_n) step(std::integral_constant<int, 2>{}, i + 2);
    wait_vm<0>();   // no direct load into LDS outlives the workgroup

    // Share sum of the row: the four lanes kq of row n.
    run += __shfl_xor(run, 16);
    run += __shfl_xor(run, 32);
    if (kq == 0 && me.mode != 0) A.sup[(size_t)jw * bpad + b] = run;
}

__global__ __launch_bounds__(64)
void verify_resid_finalize(ResidArgs A, int nitem, int ws, int bpad) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const RowInfo ri = resid_row(A, b);
    if (ri.mode == 0) return;
    const int V = A.V, G = A.G;
    const float invT = A.invT;
    const float u = A.uniforms ? A.uniforms[(size_t)b * (G + 1) + G]
                               : counter_uniform(A.seed, A.offset, b, 0, 2);
    int32_t* out = A.out_tokens + (size_t)b * (G + 1) + ri.n;
    // W1 slice of this lane for the rebuild (lane = 8t + sl: rank slice sl)
    const int span = A.r / 8;
    uint4 w1c[4];
    {
        int prev = 0;
        if (ri.mode == 1) {
            prev = ri.n == 0 ? A.x0[b] : A.draft[(size_t)b * G + ri.n - 1];
            prev = (prev >= 0 && prev < V) ? prev : 0;
        }
        const uint16_t* w1 = A.W1 + (size_t)prev * A.r + (lane & 7) * span;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w1c[q] = (ri.mode == 1 && q * 8 < span) ? *reinterpret_cast<const uint4*>(w1 + q * 8)
                                                      : make_uint4(0u, 0u, 0u, 0u);
    }

    // 1) share sums, four per lane.
    double w[4], lsum = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j = 4 * lane + q;
        w[q] = j < ws ? (double)A.sup[(size_t)j * bpad + b] : 0.0;
        lsum += w[q];
    }
    const double Rm = __shfl(wave_inclusive_scan_f64(lsum), kWave - 1);
    if (!(Rm > 0.0)) {
        // No residual mass after rounding: draw from p_n, an exact two-pass scan
        // (lane j sums a contiguous run of the row, then walks it).
        RowInfo rp = ri;
        rp.mode = 2;
        const int run = (V + kWave - 1) / kWave;
        const int v0 = min(V, lane * run), v1 = min(V, v0 + run);
        double s = 0.0;
        for (int v = v0; v < v1; ++v)
            s += (double)resid_weight(rp, bf16_bits_to_float(A.P[rp.prow + v]), 0.0f, invT);
        const double Z = __shfl(wave_inclusive_scan_f64(s), kWave - 1);
        double rem;
        const int ol = wave_pick(s, (double)u * Z, rem);
        int tok = -1, last = -1;
        if (lane == ol) {
            double acc = 0.0;
            for (int v = v0; v < v1; ++v) {
                const double wv =
                    (double)resid_weight(rp, bf16_bits_to_float(A.P[rp.prow + v]), 0.0f, invT);
                if (wv > 0.0) {
                    last = v;
                    if (rem < acc + wv) {
                        tok = v;
                        break;
                    }
                }
                acc += wv;
            }
            if (tok < 0) tok = last;
            *out = tok;
        }
        return;
    }
    double rem;
    const int ol = wave_pick(lsum, (double)u * Rm, rem);
    int qsel;
    double qrem;
    {
        double runw = 0.0, last_run = 0.0;
        int found = -1, last = -1;
        qrem = INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (found < 0 && w[q] > 0.0) {
                last = q;
                last_run = runw;
                if (rem < runw + w[q]) {
                    found = q;
                    qrem = rem - runw;
                }
            }
            runw += w[q];
        }
        if (found < 0) {
            found = last < 0 ? 0 : last;
            qrem = rem == INFINITY ? INFINITY : rem - last_run;
        }
        qsel = found;
    }
    const int sh = 4 * ol + __shfl(qsel, ol);
    const double rem1 = __shfl(qrem, ol);

    // 2) the share's 32-token segments and their group sums, one read.
    const int s0 = 2 * (int)((long long)sh * nitem / ws);
    const int s1 = 2 * (int)((long long)(sh + 1) * nitem / ws);
    const int sg = s0 + lane;
    float4 g4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (sg < s1) g4 = *reinterpret_cast<const float4*>(A.gsums + ((size_t)sg * bpad + b) * 4);
    const double ys = ((double)g4.x + (double)g4.y) + ((double)g4.z + (double)g4.w);
    double rem2;
    const int seg = s0 + wave_pick(ys, rem1, rem2);
    const int sl_seg = seg - s0;
    const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
    float mine = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float v = __shfl(gv[g], sl_seg);
        if (lane == g) mine = v;
    }
    double grem;
    const int grp = wave_pick(lane < 4 ? (double)mine : 0.0, rem2, grem);

    // 3) rebuild the group's 8 weights: lane = 8t + sl.
    const int t = lane >> 3, sl = lane & 7;
    const int vt = seg * kStreamSeg + grp * 8 + t;
    float part = 0.0f, lq = 0.0f, lp = 0.0f;
    if (vt < V) {
        if (ri.mode == 1) {
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
                        for (int hh = 0; hh < 4; ++hh) {
                            part = fmaf(bf16_bits_to_float(aw[hh] & 0xFFFFu),
                                        bf16_bits_to_float(cw[hh] & 0xFFFFu), part);
                            part = fmaf(bf16_bits_to_float(aw[hh] >> 16),
                                        bf16_bits_to_float(cw[hh] >> 16), part);
                        }
                    }
                }
            } else {   // span < 8 (r < 64)
                int prev = ri.n == 0 ? A.x0[b] : A.draft[(size_t)b * G + ri.n - 1];
                prev = (prev >= 0 && prev < V) ? prev : 0;
                const uint16_t* w1 = A.W1 + (size_t)prev * A.r;
                for (int j = sl * span; j < (sl + 1) * span; ++j)
                    part = fmaf(bf16_bits_to_float(w1[j]),
                                bf16_bits_to_float(A.W2P[w2p_index(vt, j, A.r)]), part);
            }
            lq = bf16_bits_to_float(A.U[ri.urow + vt]);
        }
        lp = bf16_bits_to_float(A.P[ri.prow + vt]);
    }
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
    part += __shfl_xor(part, 4);
    const float wt = vt < V ? resid_w(lp, lq + part, exp2_scale(invT), row_exp2(A.fin[b], ri.mode)) : 0.0f;
    const float w8 = __shfl(wt, (lane & 7) * 8);
    double trem;
    const int tsel = wave_pick(lane < 8 ? (double)w8 : 0.0, grem, trem);
    if (lane == 0) *out = min(seg * kStreamSeg + grp * 8 + tsel, V - 1);
}

bool resid_streams(int B, int V, int r) {
    if ((V % 8) != 0 || !(r == 64 || r == 128 || r == 256)) return false;
    const int nitem_v = (V + kStreamItem - 1) / kStreamItem;
    const int ws = stream_shares(B, V);
    return 2 * ((nitem_v + ws - 1) / ws) <= 64;
}

template <int NK>
static void launch_resid_stream(const ResidArgs& A, int nitem_v, int nrb, int ws, hipStream_t s) {
    constexpr int STAGE = kStreamItem * NK * 32 * 2;
    // raise the dynamic LDS limit once per process (thread-safe)
    static std::once_flag attr_once;
    std::call_once(attr_once, [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&verify_resid_stream<NK>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        (void)hipGetLastError();
    });
    hipLaunchKernelGGL((verify_resid_stream<NK>), dim3(nrb * ws), dim3(kStreamWaves * 64),
                       (size_t)kResidStages * STAGE, s, A, nitem_v, nrb, ws);
}

hipError_t verify_resid_launch(const ResidArgs& A, hipStream_t s) {
    // every work item streams a W2 slice and U rows: both must exist
    if (!A.W2P || !A.U || !A.P || A.G <= 0) return hipErrorInvalidValue;
    const int nitem_v = (A.V + kStreamItem - 1) / kStreamItem;
    const int nrb = (A.B + kStreamRows - 1) / kStreamRows;
    const int ws = stream_shares(A.B, A.V);
    if (A.r == 256) launch_resid_stream<8>(A, nitem_v, nrb, ws, s);
    else if (A.r == 128) launch_resid_stream<4>(A, nitem_v, nrb, ws, s);
    else launch_resid_stream<2>(A, nitem_v, nrb, ws, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(verify_resid_finalize, dim3(A.B), dim3(64), 0, s, A, nitem_v, ws,
                       nrb * kStreamRows);
    return hipGetLastError();
}

}  // namespace specdec
