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
#include <mutex>
#include <climits>

#include "device_common.hpp"
#include "launch.hpp"

namespace specdec {

constexpr int kResidStages = 2;


// What one request row contributes: mode 1 residual (n < L), 2 bonus (n = L),
// 0 nothing (greedy or invalid).
struct RowInfo {
    int mode, n;
    size_t prow, urow;                 // element offsets of P_n and U_n
    float lzp_hi, lzp_lo, lzq_hi, lzq_lo;
};

__device__ __forceinline__ RowInfo resid_row(const ResidArgs& A, int b) {
    RowInfo ri;
    ri.mode = 0;
    ri.n = 0;
    ri.prow = ri.urow = 0;
    ri.lzp_hi = ri.lzp_lo = ri.lzq_hi = ri.lzq_lo = 0.0f;
    if (b >= A.B) return ri;
    const FinalInfo f = A.fin[b];
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

// Weight of one token: p = exp(lp / T - logZp), q = exp(lq / T - logZq), the
// normalisers applied as fp32 (hi, lo) pairs.
__device__ __forceinline__ float resid_weight(const RowInfo& ri, float lp, float lq, float invT) {
    const float p = __expf(fmaf(lp, invT, -ri.lzp_hi) - ri.lzp_lo);
    if (ri.mode != 1) return ri.mode == 2 ? p : 0.0f;
    const float q = __expf(fmaf(lq, invT, -ri.lzq_hi) - ri.lzq_lo);
    return fmaxf(p - q, 0.0f);
}

// Work split, stage layout and wave mapping as the streaming draft tile: a
// work item is a 64-token slice x 128 rows; each stage holds the packed W2
// slice, the U_n slice and the P_n slice (16-byte chunk c of row bl in slot
// bl*8 + (c ^ ((bl>>1)&7))); wave w owns rows 32 (w & 3) .. + 31 and tokens
// 32 (w >> 2) .. + 31 on 32x32x16 MFMAs.  Two stages: item i+1 streams in while
// item i is contracted.
template <int NKS>
__global__ __launch_bounds__(kStreamWaves * 64, 1)
void verify_resid_stream(ResidArgs A, int nitem_v, int nrb, int ws) {
    constexpr int R = NKS * 16;
    constexpr int W2B = kStreamItem * R * 2;
    constexpr int SB = kStreamRows * kStreamItem * 2;   // U or P slice bytes
    constexpr int STAGE = W2B + 2 * SB;
    constexpr int W2P = W2B / 1024 / kStreamWaves;
    constexpr int SP = SB / 1024 / kStreamWaves;
    constexpr int NCH = R / 8;
    static_assert(W2P >= 1 && SP == 2, "piece split");
    extern __shared__ __align__(16) char smem_r[];
    const int V = A.V;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int rg = wave & 3, th = wave >> 2;
    const int rb0 = (int)blockIdx.x / ws;
    const int jw = (int)blockIdx.x % ws;
    const int lo = (int)((long long)jw * nitem_v / ws);
    const int hi = (int)((long long)(jw + 1) * nitem_v / ws);
    const int my_n = hi - lo;
    const size_t bpad = (size_t)nrb * kStreamRows;
    const uint16_t* Ubase = A.U;   // any readable chunk, for rows without a residual

    // This lane's U and P pieces: row bl, chunk c of every slice.
    size_t uoff[SP], poff[SP];
    int uc8[SP];
    bool uok[SP], pok[SP];
#pragma unroll
    for (int q = 0; q < SP; ++q) {
        const int sl = (q * kStreamWaves + wave) * 64 + lane;
        const int bl = sl >> 3;
        const int c = (sl & 7) ^ ((bl >> 1) & 7);
        const RowInfo ri = resid_row(A, rb0 * kStreamRows + bl);
        uc8[q] = c * 8;
        uok[q] = ri.mode == 1;
        pok[q] = ri.mode != 0;
        uoff[q] = ri.urow + c * 8;
        poff[q] = ri.prow + c * 8;
    }
    auto issue = [&](int i) {
        const int iv = lo + i;
        char* st = smem_r + (i % kResidStages) * STAGE;
        const char* wsrc = reinterpret_cast<const char*>(A.W2P) + (size_t)iv * W2B;
#pragma unroll
        for (int q = 0; q < W2P; ++q) {
            const int pc = q * kStreamWaves + wave;
            __builtin_amdgcn_global_load_lds(wsrc + pc * 1024 + lane * 16,
                                             (lds_ptr_t)(st + pc * 1024), 16, 0, 0);
        }
        const int tok = iv * kStreamItem;
#pragma unroll
        for (int q = 0; q < SP; ++q) {
            const int pc = q * kStreamWaves + wave;
            const bool in = tok + uc8[q] < V;
            const uint16_t* us = (uok[q] && in) ? A.U + uoff[q] + tok : Ubase;
            const uint16_t* ps = (pok[q] && in) ? A.P + poff[q] + tok : A.P;
            __builtin_amdgcn_global_load_lds(us, (lds_ptr_t)(st + W2B + pc * 1024), 16, 0, kCpolNT);
            __builtin_amdgcn_global_load_lds(ps, (lds_ptr_t)(st + W2B + SB + pc * 1024), 16, 0,
                                             kCpolNT);
        }
    };

    // This lane's compute row: its decision and conditioning row E = W1[x_{n-1}].
    const int bl = 32 * rg + (lane & 31);
    const int b = rb0 * kStreamRows + bl;
    const RowInfo me = resid_row(A, b);
    bf16x8_t e[NKS];
    {
        int prev = 0;
        if (me.mode == 1) {
            prev = me.n == 0 ? A.x0[b] : A.draft[(size_t)b * A.G + me.n - 1];
            prev = (prev >= 0 && prev < V) ? prev : 0;   // verify_decide has checked it
        }
        const uint16_t* erow = A.W1 + (size_t)prev * R;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (me.mode == 1) {
                e[ks] = *reinterpret_cast<const bf16x8_t*>(erow + ks * 16 + h * 8);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) e[ks][t] = (__bf16)0.0f;
            }
        }
    }
    wait_vmcnt_le(0);   // nothing but direct loads may be pending in the loop
    issue(0);

    int atok, arow;
    {
        const int i = lane & 31;
        const int g = i >> 3, hh = (i >> 2) & 1, c = i & 3;
        atok = 32 * th + 16 * hh + 8 * (g & 1) + 4 * (g >> 1) + c;
        arow = atok * R;
    }
    int uslot[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) uslot[q] = bl * 8 + ((4 * th + 2 * h + q) ^ ((bl >> 1) & 7));

    float run = 0.0f;   // this wave's half of the share's weight for the lane's row
    for (int i = 0; i < my_n; ++i) {
        const int iv = lo + i;
        wait_vmcnt_le(0);                         // item i (and item i-1's stores)
        asm volatile("s_barrier" ::: "memory");   // every wave's pieces; stage (i+1)%2 is free
        if (i + 1 < my_n) issue(i + 1);

        const char* st = smem_r + (i % kResidStages) * STAGE;
        const uint16_t* w2s = reinterpret_cast<const uint16_t*>(st);
        const int sw = w2p_swizzle((iv & 1) * 64 + atok, NCH);
        bf16x8_t afr[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            afr[ks] = *reinterpret_cast<const bf16x8_t*>(w2s + arow + (((2 * ks + h) ^ sw) << 3));
        const u32x4_t* us = reinterpret_cast<const u32x4_t*>(st + W2B);
        const u32x4_t* ps = reinterpret_cast<const u32x4_t*>(st + W2B + SB);
        u32x4_t uf[2], pf[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uf[q] = us[uslot[q]];
            pf[q] = ps[uslot[q]];
        }
        f32x16_t acc;
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[ks], e[ks], acc, 0, 0, 0);

        // accumulator idx = 4g + c holds run position 8 (g & 1) + 4 (g >> 1) + c
        const int v0 = iv * kStreamItem + 32 * th + 16 * h;
        float g0 = 0.0f, g1 = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int pos = 8 * (g & 1) + 4 * (g >> 1) + c;
                const uint32_t wu = uf[pos >> 3][(pos & 7) >> 1];
                const uint32_t wp = pf[pos >> 3][(pos & 7) >> 1];
                const float lq = acc[4 * g + c] + ((pos & 1) ? __uint_as_float(wu & 0xFFFF0000u)
                                                             : __uint_as_float(wu << 16));
                const float lp = (pos & 1) ? __uint_as_float(wp & 0xFFFF0000u)
                                           : __uint_as_float(wp << 16);
                float w = resid_weight(me, lp, lq, A.invT);
                w = v0 + pos < V ? w : 0.0f;
                if (pos < 8) g0 += w;
                else g1 += w;
            }
        if (me.mode != 0) {
            const size_t si = (2 * (size_t)iv + th) * bpad + b;
            *reinterpret_cast<float2*>(A.gsums + si * 4 + 2 * h) = make_float2(g0, g1);
        }
        float tot = g0 + g1;
        tot += __shfl_xor(tot, 32);
        run += tot;
    }

    // Share sums: the token-half-1 waves hand theirs to the half-0 waves.
    float* xs = reinterpret_cast<float*>(smem_r);   // the stages are idle now
    wait_vmcnt_le(0);
    __syncthreads();
    if (th == 1 && h == 0) xs[bl] = run;
    __syncthreads();
    if (th == 0 && h == 0 && me.mode != 0) A.sup[(size_t)jw * bpad + b] = run + xs[bl];
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
    const float wt = vt < V ? resid_weight(ri, lp, lq + part, invT) : 0.0f;
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

template <int NKS>
static void launch_resid_stream(const ResidArgs& A, int nitem_v, int nrb, int ws, hipStream_t s) {
    constexpr int STAGE = kStreamItem * NKS * 16 * 2 + 2 * kStreamRows * kStreamItem * 2;
    // raise the dynamic LDS limit once per process (thread-safe)
    static std::once_flag attr_once;
    std::call_once(attr_once, [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&verify_resid_stream<NKS>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        (void)hipGetLastError();
    });
    hipLaunchKernelGGL((verify_resid_stream<NKS>), dim3(nrb * ws), dim3(kStreamWaves * 64),
                       (size_t)kResidStages * STAGE, s, A, nitem_v, nrb, ws);
}

hipError_t verify_resid_launch(const ResidArgs& A, hipStream_t s) {
    // every work item streams a W2 slice and U rows: both must exist
    if (!A.W2P || !A.U || !A.P || A.G <= 0) return hipErrorInvalidValue;
    const int nitem_v = (A.V + kStreamItem - 1) / kStreamItem;
    const int nrb = (A.B + kStreamRows - 1) / kStreamRows;
    const int ws = stream_shares(A.B, A.V);
    if (A.r == 256) launch_resid_stream<16>(A, nitem_v, nrb, ws, s);
    else if (A.r == 128) launch_resid_stream<8>(A, nitem_v, nrb, ws, s);
    else launch_resid_stream<4>(A, nitem_v, nrb, ws, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(verify_resid_finalize, dim3(A.B), dim3(64), 0, s, A, nitem_v, ws,
                       nrb * kStreamRows);
    return hipGetLastError();
}

}  // namespace specdec
