// Draft sampling kernels: DSpark's sequential stage ("[논문리뷰] DSpark ...",
// §1.2 Sequential stage).  Position k of every request is produced by two
// launches on the caller's stream:
//
//   draft_tile_*   one workgroup per 128-token vocabulary tile and group of
//                  request rows: bias tile = E[B x r] * W2[r x 128] (Markov:
//                  E = W1[x_{k-1}], RNN: E = split tanh(W_o z_k)), adds U_k,
//                  stores the fp32 draft logits and writes a (max, sum-exp,
//                  argmax) summary per (row, segment).  No probability tensor
//                  is written.
//   draft_finalize one workgroup per request row: fp64 combine of the segment
//                  summaries into the normaliser, inverse-CDF location of the
//                  segment holding u * Z, rescan of that segment's logits ->
//                  x_k, log Z, q(x_k).  T == 0 takes the argmax.
//
// The RNN head adds rnn_hidden_proj (the h_k part of W_g, W_c, W_o for all
// positions at once, bf16 MFMA) and rnn_gates (per position: the s_{k-1} and
// W1[x_{k-1}] parts, the gated state update and o = tanh(W_o z_k)).
#include <climits>

#include "device_common.hpp"
#include "launch.hpp"

namespace specdec {

constexpr int kTileV = 128;   // vocabulary columns per tile workgroup
constexpr int kLdsPad = 8;    // bf16 elements of padding per transposed W2 row

// ---------------------------------------------------------------------------
// Epilogue helpers: 4 consecutive logits of one request row.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void load4(const void* base, size_t i, float out[4]) {
    if constexpr (BF16) {
        const uint2 t = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + i);
        out[0] = bf16_bits_to_float(t.x & 0xFFFFu);
        out[1] = bf16_bits_to_float(t.x >> 16);
        out[2] = bf16_bits_to_float(t.y & 0xFFFFu);
        out[3] = bf16_bits_to_float(t.y >> 16);
    } else {
        const float4 t = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
        out[0] = t.x; out[1] = t.y; out[2] = t.z; out[3] = t.w;
    }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t i) {
    if constexpr (BF16) return bf16_bits_to_float(static_cast<const uint16_t*>(base)[i]);
    else return static_cast<const float*>(base)[i];
}

// ---------------------------------------------------------------------------
// bf16 MFMA bias tile.
//
// Workgroup = 4 waves.  WB waves split the request rows (32 rows each), the
// other 4/WB split the 128 columns, so each wave owns MB = WB blocks of 32
// columns.  The MFMA computes C[v][b] = sum_j W2[j][v] * E[b][j]:
//   A operand (32 v x 16 j) from the transposed W2 tile in LDS,
//   B operand (16 j x 32 b) straight from the E rows held in registers.
// Lane l then owns request row b = l % 32 and, per 32-column block, the 16
// columns 8*(i/4) + 4*(l/32) + i%4 (i = 0..15), i.e. four runs of four
// consecutive tokens: the epilogue adds U and stores q with 16-byte accesses,
// and the per-row reduction over v is lane-local plus one exchange.
// ---------------------------------------------------------------------------
template <int WB, int MODE, bool U_BF16>
__global__ __launch_bounds__(256, 2)
void draft_tile_mfma(const void* __restrict__ U, const uint16_t* __restrict__ W1,
                     const uint16_t* __restrict__ W2, const uint16_t* __restrict__ Erows,
                     const int32_t* __restrict__ x0, const int32_t* __restrict__ tokens,
                     float* __restrict__ q_logits, SegStat* __restrict__ stats,
                     int B, int gamma, int V, int r, int k, float invT, int greedy) {
    constexpr int MB = WB;
    constexpr int WV = 4 / WB;
    constexpr int NS = (MODE == kHeadRnn) ? 3 : 1;
    extern __shared__ __align__(16) uint16_t w2t[];   // [kTileV][r + kLdsPad]
    const int ldr = r + kLdsPad;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wb = wave % WB;
    const int wv = wave / WB;
    const int v_tile = blockIdx.x * kTileV;
    const int b = blockIdx.y * (32 * WB) + wb * 32 + (lane & 31);
    const bool brow = b < B;
    const int kgrp = lane >> 5;

    // 1) W2[:, tile] -> LDS, transposed to [v][j] in 8x8 register blocks.
    {
        const int nblk = (r / 8) * (kTileV / 8);
        const bool vec_ok = (V % 8) == 0;
        for (int blk = tid; blk < nblk; blk += 256) {
            const int vb = blk % (kTileV / 8);
            const int jb = blk / (kTileV / 8);
            const int v0 = v_tile + vb * 8;
            const int j0 = jb * 8;
            uint32_t w[8][4];
            if (vec_ok && v0 + 8 <= V) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint4 t = *reinterpret_cast<const uint4*>(W2 + (size_t)(j0 + i) * V + v0);
                    w[i][0] = t.x; w[i][1] = t.y; w[i][2] = t.z; w[i][3] = t.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const int va = v0 + 2 * h;
                        const uint32_t lo = va < V ? W2[(size_t)(j0 + i) * V + va] : 0u;
                        const uint32_t hi = va + 1 < V ? W2[(size_t)(j0 + i) * V + va + 1] : 0u;
                        w[i][h] = lo | (hi << 16);
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t o[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t a = w[2 * p][e >> 1];
                    const uint32_t c = w[2 * p + 1][e >> 1];
                    o[p] = (e & 1) ? ((a >> 16) | (c & 0xFFFF0000u)) : ((a & 0xFFFFu) | (c << 16));
                }
                *reinterpret_cast<uint4*>(w2t + (vb * 8 + e) * ldr + j0) =
                    make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }

    // 2) conditioning rows and the contraction.
    int prev = 0;
    bool erow_ok = brow;
    if (MODE == kHeadMarkov && brow) {
        prev = (k == 0) ? x0[b] : tokens[(size_t)b * gamma + k - 1];
        erow_ok = prev >= 0 && prev < V;
    }
    f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
    __syncthreads();

    const int nks = r / 16;
#pragma unroll
    for (int split = 0; split < NS; ++split) {
        const uint16_t* erow = (MODE == kHeadMarkov)
                                   ? W1 + (size_t)prev * r
                                   : Erows + ((size_t)b * 3 + split) * r;
        bf16x8_t e[16];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            if (ks < nks) {
                if (erow_ok) {
                    e[ks] = *reinterpret_cast<const bf16x8_t*>(erow + ks * 16 + kgrp * 8);
                } else {
#pragma unroll
                    for (int t = 0; t < 8; ++t) e[ks][t] = (__bf16)0.0f;
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            if (ks < nks) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int vl = wv * (32 * MB) + mb * 32 + (lane & 31);
                    const bf16x8_t a =
                        *reinterpret_cast<const bf16x8_t*>(w2t + vl * ldr + ks * 16 + kgrp * 8);
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, e[ks], acc[mb], 0, 0, 0);
                }
            }
        }
    }

    // 3) l = U + bias, store q, per-lane max / argmax.
    const size_t rowoff = ((size_t)(brow ? b : 0) * gamma + k) * (size_t)V;
    const bool vec_io = (V % 4) == 0;
    float m = -INFINITY;
    int amax = INT_MAX;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int v4 = v_tile + wv * (32 * MB) + mb * 32 + g * 8 + kgrp * 4;
            float u4[4];
            if (brow && vec_io && v4 + 3 < V) {
                load4<U_BF16>(U, rowoff + v4, u4);
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[mb][4 * g + t] += u4[t];
                *reinterpret_cast<float4*>(q_logits + rowoff + v4) =
                    make_float4(acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2],
                                acc[mb][4 * g + 3]);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (brow && v4 + t < V) {
                        acc[mb][4 * g + t] += load1<U_BF16>(U, rowoff + v4 + t);
                        q_logits[rowoff + v4 + t] = acc[mb][4 * g + t];
                    } else {
                        acc[mb][4 * g + t] = -INFINITY;
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) merge_arg(m, amax, acc[mb][4 * g + t], v4 + t);
        }
    }
    float s = 0.0f;
    if (!greedy && m != -INFINITY) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s += __expf((acc[mb][i] - m) * invT);
    }
    {
        const float m2 = __shfl_xor(m, 32);
        const float s2 = __shfl_xor(s, 32);
        const int i2 = __shfl_xor(amax, 32);
        float mv = m;
        int iv = amax;
        merge_arg(mv, iv, m2, i2);
        merge_ms(m, s, m2, s2, invT);
        amax = iv;
    }
    if (brow && lane < 32) {
        const int nseg = gridDim.x * WV;
        SegStat st;
        st.m = m;
        st.s = s;
        st.idx = amax;
        st.pad = 0;
        stats[(size_t)b * nseg + blockIdx.x * WV + wv] = st;
    }
}

// ---------------------------------------------------------------------------
// fp32-weight variant on the vector ALUs (small ranks such as r = 16).
// Workgroup = one 128-column tile; each thread owns one column and loops over
// the request rows; the per-row summary is a block reduction.
// ---------------------------------------------------------------------------
template <bool U_BF16>
__global__ __launch_bounds__(128)
void draft_tile_valu_f32w(const void* __restrict__ U, const float* __restrict__ W1,
                          const float* __restrict__ W2, const int32_t* __restrict__ x0,
                          const int32_t* __restrict__ tokens, float* __restrict__ q_logits,
                          SegStat* __restrict__ stats, int B, int gamma, int V, int r, int k,
                          float invT, int greedy) {
    __shared__ float red_m[2], red_s[2];
    __shared__ int red_i[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int v = blockIdx.x * kTileV + tid;
    for (int b = 0; b < B; ++b) {
        const int prev = (k == 0) ? x0[b] : tokens[(size_t)b * gamma + k - 1];
        const bool ok = prev >= 0 && prev < V;
        float l = -INFINITY;
        if (v < V) {
            float bias = 0.0f;
            if (ok) {
                for (int j = 0; j < r; ++j)
                    bias = fmaf(W1[(size_t)prev * r + j], W2[(size_t)j * V + v], bias);
            }
            const size_t off = ((size_t)b * gamma + k) * (size_t)V + v;
            l = load1<U_BF16>(U, off) + bias;
            q_logits[off] = l;
        }
        float m = l, s = (v < V && !greedy) ? 1.0f : 0.0f;
        int idx = v < V ? v : INT_MAX;
        wave_reduce_stat(m, s, idx, invT);
        if (lane == 0) {
            red_m[wave] = m;
            red_s[wave] = s;
            red_i[wave] = idx;
        }
        __syncthreads();
        if (tid == 0) {
            float mm = red_m[0], ss = red_s[0];
            int ii = red_i[0];
            float mv = mm;
            int iv = ii;
            merge_arg(mv, iv, red_m[1], red_i[1]);
            merge_ms(mm, ss, red_m[1], red_s[1], invT);
            SegStat st;
            st.m = mm;
            st.s = ss;
            st.idx = iv;
            st.pad = 0;
            stats[(size_t)b * gridDim.x + blockIdx.x] = st;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Per-row finalize: normaliser, inverse-CDF draw, outputs of position k.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256)
void draft_finalize(const SegStat* __restrict__ stats, int nseg, int seg_len,
                    const float* __restrict__ q_logits, const int32_t* __restrict__ x0,
                    int32_t* __restrict__ tokens, float* __restrict__ q_logZ,
                    float* __restrict__ q_tok, const float* __restrict__ uniforms,
                    uint64_t seed, uint32_t offset, int gamma, int V, int k, float invT,
                    int greedy) {
    __shared__ double scan[256];
    __shared__ float red_m[4];
    __shared__ int red_i[4];
    __shared__ int sh_seg;
    __shared__ double sh_rem;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const size_t outi = (size_t)b * gamma + k;

    const int prev = (k == 0) ? x0[b] : tokens[outi - 1];
    if (prev < 0 || prev >= V) {
        if (tid == 0) {
            tokens[outi] = -1;
            if (q_logZ) q_logZ[outi] = NAN;
            if (q_tok) q_tok[outi] = NAN;
        }
        return;
    }
    const SegStat* st = stats + (size_t)b * nseg;

    // 1) row max and argmax over the segment summaries.
    float M = -INFINITY;
    int AM = INT_MAX;
    for (int j = tid; j < nseg; j += 256) {
        const SegStat t = st[j];
        merge_arg(M, AM, t.m, t.idx);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(M, off);
        const int i2 = __shfl_xor(AM, off);
        merge_arg(M, AM, m2, i2);
    }
    if (lane == 0) {
        red_m[wave] = M;
        red_i[wave] = AM;
    }
    __syncthreads();
    M = red_m[0];
    AM = red_i[0];
    for (int w = 1; w < 4; ++w) merge_arg(M, AM, red_m[w], red_i[w]);

    if (greedy || M == -INFINITY) {
        if (tid == 0) {
            tokens[outi] = (M == -INFINITY) ? -1 : AM;
            if (q_logZ) q_logZ[outi] = M == -INFINITY ? NAN : M;
            if (q_tok) q_tok[outi] = M == -INFINITY ? NAN : 1.0f;
        }
        return;
    }

    // 2) fp64 sums of the segment summaries, contiguous chunk per thread,
    //    then an exclusive scan across threads (segment order = token order).
    const int per = (nseg + 255) / 256;
    const int j0 = min(nseg, tid * per);
    const int j1 = min(nseg, j0 + per);
    const double Md = (double)M;
    double tsum = 0.0;
    for (int j = j0; j < j1; ++j) {
        const SegStat t = st[j];
        if (t.m != -INFINITY) tsum += (double)t.s * exp(((double)t.m - Md) * (double)invT);
    }
    scan[tid] = tsum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const double add = tid >= off ? scan[tid - off] : 0.0;
        __syncthreads();
        scan[tid] += add;
        __syncthreads();
    }
    const double incl = scan[tid];
    const double excl = tid > 0 ? scan[tid - 1] : 0.0;
    const double Z = scan[255];
    if (tid == 0) sh_seg = -1;
    __syncthreads();

    const float u = uniforms ? uniforms[outi] : counter_uniform(seed, offset, b, k, 0);
    const double thr = (double)u * Z;

    // 3) locate the segment holding thr.
    if (tsum > 0.0 && thr >= excl && thr < incl) {
        double run = excl;
        int found = -1, last = -1;
        double last_run = 0.0, last_w = 0.0;
        for (int j = j0; j < j1; ++j) {
            const SegStat t = st[j];
            const double w = t.m != -INFINITY ? (double)t.s * exp(((double)t.m - Md) * (double)invT) : 0.0;
            if (w > 0.0) {
                last = j;
                last_run = run;
                last_w = w;
                if (thr < run + w) {
                    found = j;
                    break;
                }
            }
            run += w;
        }
        if (found >= 0) {
            sh_seg = found;
            sh_rem = thr - run;
        } else {
            // rounding left thr past this chunk's own running sum: clamp
            // to the end of its last segment with weight.
            sh_seg = last;
            sh_rem = thr - last_run;
            (void)last_w;
        }
    }
    __syncthreads();
    if (sh_seg < 0) {
        // thr >= Z after rounding: clamp to the last segment with weight.
        int lastj = -1;
        for (int j = j0; j < j1; ++j)
            if (st[j].m != -INFINITY && st[j].s > 0.0f) lastj = j;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) lastj = max(lastj, __shfl_xor(lastj, off));
        if (lane == 0) red_i[wave] = lastj;
        __syncthreads();
        if (tid == 0) {
            sh_seg = max(max(red_i[0], red_i[1]), max(red_i[2], red_i[3]));
            sh_rem = INFINITY;
        }
        __syncthreads();
    }

    // 4) rescan the chosen segment with one wave (2 tokens per lane).
    if (wave == 0) {
        const int seg = sh_seg;
        const double rem = sh_rem;
        const int v0 = seg * seg_len;
        const int v1 = min(V, v0 + seg_len);
        const float* row = q_logits + outi * (size_t)V;
        const int va = v0 + 2 * lane;
        const int vb = va + 1;
        const double w0 = va < v1 ? exp(((double)row[va] - Md) * (double)invT) : 0.0;
        const double w1 = vb < v1 ? exp(((double)row[vb] - Md) * (double)invT) : 0.0;
        const double lsum = w0 + w1;
        const double inc = wave_inclusive_scan_f64(lsum);
        double exc = __shfl_up(inc, 1);
        if (lane == 0) exc = 0.0;
        const unsigned long long hit = __ballot(lsum > 0.0 && inc > rem);
        int pick;
        if (hit) {
            const int L0 = __ffsll((long long)hit) - 1;
            const int mine = (w0 > 0.0 && rem < exc + w0) ? va : vb;
            pick = __shfl(mine, L0);
        } else {
            const unsigned long long pos = __ballot(lsum > 0.0);
            const int L1 = 63 - __clzll((long long)pos);
            const int mine = w1 > 0.0 ? vb : va;
            pick = __shfl(mine, L1);
        }
        pick = max(v0, min(pick, v1 - 1));   // stays inside the rescanned segment
        if (lane == 0) {
            tokens[outi] = pick;
            if (q_logZ) q_logZ[outi] = (float)(Md * (double)invT + log(Z));
            if (q_tok) q_tok[outi] = (float)(exp(((double)row[pick] - Md) * (double)invT) / Z);
        }
    }
}

// ---------------------------------------------------------------------------
// RNN head.
// ---------------------------------------------------------------------------

// out[m][n] = sum_t h[m][t] * Wcat[n][2r + t], m < M = B * gamma, n < 3r,
// Wcat = [W_g; W_c; W_o].  One wave per 32 x 32 output block, operands read
// straight from global memory in 16-byte runs along t.
__global__ __launch_bounds__(256)
void rnn_hidden_proj(const uint16_t* __restrict__ h, const uint16_t* __restrict__ Wg,
                     const uint16_t* __restrict__ Wc, const uint16_t* __restrict__ Wo,
                     float* __restrict__ out, int M, int r, int d) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m0 = blockIdx.y * 64 + (wave >> 1) * 32;
    const int n0 = blockIdx.x * 64 + (wave & 1) * 32;
    const int ld = 2 * r + d;
    const int kgrp = lane >> 5;
    const int m = m0 + (lane & 31);
    const int n = n0 + (lane & 31);
    const bool mok = m < M;
    const bool nok = n < 3 * r;
    const uint16_t* arow = h + (size_t)(mok ? m : 0) * d + kgrp * 8;
    const uint16_t* wsel = n < r ? Wg : (n < 2 * r ? Wc : Wo);
    const uint16_t* brow = wsel + (size_t)(nok ? n % r : 0) * ld + 2 * r + kgrp * 8;
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    bf16x8_t zero;
#pragma unroll
    for (int t = 0; t < 8; ++t) zero[t] = (__bf16)0.0f;
    for (int t0 = 0; t0 < d; t0 += 64) {
        bf16x8_t a[4], bb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = t0 + 16 * u;
            const bool in = t + kgrp * 8 + 8 <= d;   // d % 8 == 0: whole 8-runs only
            a[u] = (mok && in) ? *reinterpret_cast<const bf16x8_t*>(arow + t) : zero;
            bb[u] = (nok && in) ? *reinterpret_cast<const bf16x8_t*>(brow + t) : zero;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], bb[u], acc, 0, 0, 0);
    }
    if (nok) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int mm = m0 + 8 * (i >> 2) + 4 * kgrp + (i & 3);
            if (mm < M) out[(size_t)mm * 3 * r + n] = acc[i];
        }
    }
}

// Per position k: pre-activations = hidden part + W[:, 0:r] s_{k-1} +
// W[:, r:2r] W1[x_{k-1}] for W = W_g, W_c, W_o; gated state update; o split
// into three bf16 terms (hi, mid, lo) whose sum equals o to ~2^-25.
__global__ __launch_bounds__(256)
void rnn_gates(const float* __restrict__ hproj, const uint16_t* __restrict__ Wg,
               const uint16_t* __restrict__ Wc, const uint16_t* __restrict__ Wo,
               const uint16_t* __restrict__ W1, const int32_t* __restrict__ x0,
               const int32_t* __restrict__ tokens, const float* __restrict__ s_in,
               float* __restrict__ s_out, uint16_t* __restrict__ Erows, int gamma, int V, int r,
               int d, int k) {
    extern __shared__ float z[];   // [2r]: s_{k-1}, then W1[x_{k-1}]
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int prev = (k == 0) ? x0[b] : tokens[(size_t)b * gamma + k - 1];
    const bool ok = prev >= 0 && prev < V;
    for (int t = tid; t < r; t += blockDim.x) {
        z[t] = (k == 0) ? 0.0f : s_in[(size_t)b * r + t];
        z[r + t] = ok ? bf16_bits_to_float(W1[(size_t)prev * r + t]) : 0.0f;
    }
    __syncthreads();
    const int ld = 2 * r + d;
    const float* hp = hproj + ((size_t)b * gamma + k) * 3 * r;
    for (int i = tid; i < r; i += blockDim.x) {
        float ag = hp[i], ac = hp[r + i], ao = hp[2 * r + i];
        const uint16_t* gr = Wg + (size_t)i * ld;
        const uint16_t* cr = Wc + (size_t)i * ld;
        const uint16_t* orow = Wo + (size_t)i * ld;
        for (int t = 0; t < 2 * r; t += 8) {
            const uint4 wg = *reinterpret_cast<const uint4*>(gr + t);
            const uint4 wc = *reinterpret_cast<const uint4*>(cr + t);
            const uint4 wo = *reinterpret_cast<const uint4*>(orow + t);
            const uint32_t g4[4] = {wg.x, wg.y, wg.z, wg.w};
            const uint32_t c4[4] = {wc.x, wc.y, wc.z, wc.w};
            const uint32_t o4[4] = {wo.x, wo.y, wo.z, wo.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float z0 = z[t + 2 * q], z1 = z[t + 2 * q + 1];
                ag = fmaf(bf16_bits_to_float(g4[q] & 0xFFFFu), z0, ag);
                ag = fmaf(bf16_bits_to_float(g4[q] >> 16), z1, ag);
                ac = fmaf(bf16_bits_to_float(c4[q] & 0xFFFFu), z0, ac);
                ac = fmaf(bf16_bits_to_float(c4[q] >> 16), z1, ac);
                ao = fmaf(bf16_bits_to_float(o4[q] & 0xFFFFu), z0, ao);
                ao = fmaf(bf16_bits_to_float(o4[q] >> 16), z1, ao);
            }
        }
        const float g = 1.0f / (1.0f + expf(-ag));
        const float c = tanhf(ac);
        const float o = tanhf(ao);
        s_out[(size_t)b * r + i] = g * z[i] + (1.0f - g) * c;
        const uint32_t hi = float_to_bf16_bits(o);
        const float r1 = o - bf16_bits_to_float(hi);
        const uint32_t mid = float_to_bf16_bits(r1);
        const float r2 = r1 - bf16_bits_to_float(mid);
        const uint32_t lo = float_to_bf16_bits(r2);
        uint16_t* er = Erows + (size_t)b * 3 * r;
        er[i] = (uint16_t)hi;
        er[r + i] = (uint16_t)mid;
        er[2 * r + i] = (uint16_t)lo;
    }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
static int pick_wb(int B) { return B <= 32 ? 1 : (B <= 64 ? 2 : 4); }

int draft_num_segments(int B, int V, int w_bf16) {
    const int nt = (V + kTileV - 1) / kTileV;
    if (!w_bf16) return nt;
    return nt * (4 / pick_wb(B));
}

int draft_segment_len(int B, int w_bf16) {
    if (!w_bf16) return kTileV;
    return kTileV / (4 / pick_wb(B));
}

template <int WB, int MODE>
static hipError_t launch_tile_wb(const DraftArgs& a, int k, hipStream_t s) {
    const int nt = (a.V + kTileV - 1) / kTileV;
    dim3 grid(nt, (a.B + 32 * WB - 1) / (32 * WB));
    const size_t lds = (size_t)kTileV * (a.r + kLdsPad) * sizeof(uint16_t);
    // r = 256 needs 66 KB of LDS per workgroup (gfx950 has 160 KB per CU)
    static bool attr_set = false;
    if (!attr_set) {
        hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_tile_mfma<WB, MODE, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_tile_mfma<WB, MODE, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        (void)hipGetLastError();
        attr_set = true;
    }
    if (a.u_bf16)
        hipLaunchKernelGGL((draft_tile_mfma<WB, MODE, true>), grid, dim3(256), lds, s, a.U,
                           (const uint16_t*)a.W1, (const uint16_t*)a.W2, a.Erows, a.x0, a.tokens,
                           a.q_logits, a.stats, a.B, a.gamma, a.V, a.r, k, a.invT, a.greedy);
    else
        hipLaunchKernelGGL((draft_tile_mfma<WB, MODE, false>), grid, dim3(256), lds, s, a.U,
                           (const uint16_t*)a.W1, (const uint16_t*)a.W2, a.Erows, a.x0, a.tokens,
                           a.q_logits, a.stats, a.B, a.gamma, a.V, a.r, k, a.invT, a.greedy);
    return hipGetLastError();
}

hipError_t draft_tile_launch(const DraftArgs& a, int k, hipStream_t s) {
    if (!a.w_bf16) {
        dim3 grid((a.V + kTileV - 1) / kTileV);
        if (a.u_bf16)
            hipLaunchKernelGGL((draft_tile_valu_f32w<true>), grid, dim3(128), 0, s, a.U,
                               (const float*)a.W1, (const float*)a.W2, a.x0, a.tokens, a.q_logits,
                               a.stats, a.B, a.gamma, a.V, a.r, k, a.invT, a.greedy);
        else
            hipLaunchKernelGGL((draft_tile_valu_f32w<false>), grid, dim3(128), 0, s, a.U,
                               (const float*)a.W1, (const float*)a.W2, a.x0, a.tokens, a.q_logits,
                               a.stats, a.B, a.gamma, a.V, a.r, k, a.invT, a.greedy);
        return hipGetLastError();
    }
    const int wb = pick_wb(a.B);
    if (a.head == kHeadMarkov) {
        if (wb == 1) return launch_tile_wb<1, kHeadMarkov>(a, k, s);
        if (wb == 2) return launch_tile_wb<2, kHeadMarkov>(a, k, s);
        return launch_tile_wb<4, kHeadMarkov>(a, k, s);
    }
    if (wb == 1) return launch_tile_wb<1, kHeadRnn>(a, k, s);
    if (wb == 2) return launch_tile_wb<2, kHeadRnn>(a, k, s);
    return launch_tile_wb<4, kHeadRnn>(a, k, s);
}

hipError_t draft_finalize_launch(const DraftArgs& a, int k, hipStream_t s) {
    const int nseg = draft_num_segments(a.B, a.V, a.w_bf16);
    const int seg = draft_segment_len(a.B, a.w_bf16);
    hipLaunchKernelGGL(draft_finalize, dim3(a.B), dim3(256), 0, s, a.stats, nseg, seg, a.q_logits,
                       a.x0, a.tokens, a.q_logZ, a.q_tok, a.uniforms, a.seed, a.offset, a.gamma,
                       a.V, k, a.invT, a.greedy);
    return hipGetLastError();
}

hipError_t rnn_hidden_proj_launch(const DraftArgs& a, hipStream_t s) {
    const int M = a.B * a.gamma;
    dim3 grid((3 * a.r + 63) / 64, (M + 63) / 64);
    hipLaunchKernelGGL(rnn_hidden_proj, grid, dim3(256), 0, s, (const uint16_t*)a.h,
                       (const uint16_t*)a.Wg, (const uint16_t*)a.Wc, (const uint16_t*)a.Wo,
                       a.hproj, M, a.r, a.d);
    return hipGetLastError();
}

hipError_t rnn_gates_launch(const DraftArgs& a, int k, hipStream_t s) {
    const float* s_in = a.state + (size_t)((k + 1) & 1) * a.B * a.r;
    float* s_out = a.state + (size_t)(k & 1) * a.B * a.r;
    hipLaunchKernelGGL(rnn_gates, dim3(a.B), dim3(256), 2 * a.r * sizeof(float), s, a.hproj,
                       (const uint16_t*)a.Wg, (const uint16_t*)a.Wc, (const uint16_t*)a.Wo,
                       (const uint16_t*)a.W1, a.x0, a.tokens, s_in, s_out, a.Erows, a.gamma, a.V,
                       a.r, a.d, k);
    return hipGetLastError();
}

}  // namespace specdec
