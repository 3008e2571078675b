// Persistent, weight-stationary q-free Markov draft ("[논문리뷰] DSpark ...",
// §1.2 Sequential stage, Markov-head equation): every position of every
// request in one launch of one workgroup per CU, all resident at once.
//
// The per-position kernels read all of the packed W2 image once per position.
// Here each unit workgroup owns a fixed contiguous range of 32-token blocks
// (its share of the vocabulary) for the whole call, and each of its four
// waves (one per SIMD, so 512 registers each) keeps the MFMA A operands of up
// to NB of those blocks in registers: W2 crosses HBM once per call, and only
// U_k streams per position.  The requests are taken in blocks of 64 rows;
// for position k and row block rb a unit workgroup runs
//
//   1. wait for the tokens x_{k-1} of the block's rows (token words written by
//      the finalize workgroups; the anchors x_0 at k = 0);
//   2. E = W1[x_{k-1}] of the 64 rows gathered into LDS (direct loads, chunk c
//      of row n stored in slot c ^ (n & 7): conflict-free B reads).  The
//      block's first units of U are already in flight: U does not depend on
//      the tokens, so each wave issues them as soon as the previous block's
//      summaries are out;
//   3. per wave, units (32 rows x one of its 32-token blocks): U_k of the unit
//      streams through a wave-private LDS ring (direct loads, D units ahead),
//      16 (r = 256) 32x32x16 MFMAs against the resident W2 operands, then the
//      reduction of the previous unit: the block's max and four 8-token group
//      sums relative to it (the same segment summaries as the per-position
//      streaming tile), and a running (max, sum) of the wave's blocks per row;
//   4. the four waves' running summaries merged into one summary per (row,
//      workgroup share), written with the tag k + 1.
//
// The last few workgroups only finalize: one wave per row polls the row's
// tagged share summaries, runs the shared finalize (shares -> segment ->
// group -> token, rebuilding 8 logits) -> x_k, log Z, q(x_k), and publishes
// the token word.  While they draw the tokens of one row block, the unit
// workgroups already compute the next block, so the draw is off the critical
// path whenever there are two or more row blocks (B > 64).
//
// MFMA row i = 8g + 4h + c of a block holds token 16h + 8 (g & 1) + 4 (g >> 1)
// + c, so a lane's 16 accumulators are 16 contiguous tokens of one row and its
// U values are two 16-byte chunks.  Every workgroup must be resident at once
// (one per CU: a cooperative launch guarantees it, a plain launch gets it on an
// otherwise idle device).  Every wait is a bounded poll: if a wait does not
// complete within the poll limit the workgroup sets an abort word and every
// other workgroup leaves at its next poll, so the launch always ends.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <climits>

#include "device_common.hpp"
#include "launch.hpp"
#include "stream_finalize.hpp"

namespace specdec {

constexpr int kPersistWaves = 4;             // one wave per SIMD
constexpr int kPersistRows = 64;             // request rows of one row block
constexpr int kPersistFinWgs = 16;           // workgroups that only finalize
constexpr int kPersistUnit = 2048;           // bf16 U bytes of one unit: 32 rows x 32 tokens
constexpr unsigned kBarrierPolls = 1u << 20; // polls (with s_sleep) before a wait gives up

// Both values of a lane pair (l, l ^ 32), one in each result: swapping the
// upper half of one copy with the lower half of the other leaves lane l with
// {x[l % 32], x[32 + l % 32]}.  Max and sum of the two are pair-symmetric.
__device__ __forceinline__ float pair_max32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair_argmax32(float& m, int& a) {
    const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const auto ra = __builtin_amdgcn_permlane32_swap((unsigned)a, (unsigned)a, false, false);
    float m0 = __uint_as_float(rm[0]);
    int a0 = (int)ra[0];
    merge_arg(m0, a0, __uint_as_float(rm[1]), (int)ra[1]);
    m = m0;
    a = a0;
}

// Chunk swizzle of a U ring slot (32 rows x 64 bytes): conflict-free reads of
// chunks 2h and 2h + 1 of row m by lane (m, h), in groups of 8 or 16 lanes.
__device__ __forceinline__ int uswz(int m) { return ((m >> 1) ^ (m >> 2)) & 3; }
// The same for fp32 U (32 rows x 128 bytes): chunks 4h .. 4h + 3 of row m.
__device__ __forceinline__ int uswz8(int m) { return m & 7; }

struct PersistArgs {
    FinStreamArgs fin;   // finalize inputs and outputs (tokens, q_logZ, q_tok, ...)
    float* segm;         // [nblk][bpad] max of each 32-token block
    float* gsums;        // [nblk][bpad][4] 8-token group sums relative to it
    SegStat* sup;        // [shares][bpad] per-(share, row) summaries
    unsigned* bar;       // barrier words (kBarWords, zero at launch except the -inf
                         // values that stand in for the U chunks of absent tokens)
    int B, gamma, V, nblk, bpad;
    int nu;              // unit workgroups 0 .. nu - 1; the others finalize
};

// Layout of the synchronisation words (unsigned, in the workspace): the abort
// word, eight bf16 -inf values and four fp32 -inf values.
constexpr int kBarAbort = 0;
constexpr int kBarNegInf = 4;     // [4, 8)
constexpr int kBarNegInfF = 8;    // [8, 12)
constexpr int kBarWords = 12;
static_assert(kBarWords * sizeof(unsigned) <= kPersistBarBytes, "barrier words");

// Launch preamble: clears the abort word, the token words [B] and the tagged
// share summaries [ns] (two 64-bit words each), sets the -inf chunk, and
// fills the output tokens [ntok] with -1, which is what a draw that never
// happens (a wait that gave up) leaves behind.
__global__ void persist_bar_reset(unsigned* bar, uint64_t* tflag, int B, uint64_t* sup64,
                                  size_t ns, int32_t* tokens, size_t ntok) {
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    if (t < (size_t)kBarWords)
        bar[t] = t >= (size_t)kBarNegInfF ? 0xFF800000u : (t >= (size_t)kBarNegInf ? 0xFF80FF80u : 0u);
    if (t < (size_t)B) tflag[t] = 0u;
    for (size_t i = t; i < 2 * ns; i += stride) sup64[i] = 0u;
    for (size_t i = t; i < ntok; i += stride) tokens[i] = -1;
}

// Wait until the token words of rows r0 .. r0 + rows - 1 (rows <= 64) carry
// position k - 1: the word of row b reads (k << 32) | token once the
// finalize of (b, k - 1) is done.  Wave 0 polls with coherent loads and
// leaves the tokens in xprev[0 .. 63] (-1 for an invalid or absent row).
// Bounded: past the poll limit, or when another wave set the abort word,
// the abort word is set and false returned.
__device__ __forceinline__ bool rows_tokens(unsigned* bar, const uint64_t* tflag, int r0, int rows,
                                            unsigned k, int V, unsigned limit, int* xprev,
                                            int* ok_s) {
    if (threadIdx.x < 64) {
        int lane = threadIdx.x;
        asm volatile("" : "+v"(lane));   // recomputed here, not kept live across the kernel
        int ok = 1;
        for (unsigned polls = 0;; ++polls) {
            bool up = true;
            int tok = -1;
            if (lane < rows) {
                const uint64_t w = coh_load<true>(tflag + r0 + lane);
                up = (uint32_t)(w >> 32) >= k;
                tok = (int)(uint32_t)w;
            }
            if (__all(up)) {
                xprev[lane] = (tok >= 0 && tok < V) ? tok : -1;
                break;
            }
            if (coh_load<true>(bar + kBarAbort) != 0u || polls > limit) {
                if (lane == 0) coh_store<true>(bar + kBarAbort, 1u);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) *ok_s = ok;
    }
    __syncthreads();
    return *ok_s != 0;
}

// Per U element type: value bytes, unit bytes, direct loads per unit and
// wave, 16-byte chunks per unit row.
template <bool UF> struct PersistU {
    static constexpr int ES = UF ? 4 : 2;
    static constexpr int UNIT = kPersistUnit * ES / 2;
    static constexpr int LU = UF ? 4 : 2;
    static constexpr int CPR = UF ? 8 : 4;
};

// The kernel's body, a device function so that the host pass, which only
// needs the kernel's entry stub, never instantiates it (its instantiation
// there silently failed once the body depended on UF).
template <int NKS, int NB, int NR, bool GREEDY, bool UF>
__device__ __forceinline__ void draft_persist_body(const PersistArgs& P) {
    constexpr int R = NKS * 16;
    constexpr int NCH = R / 8;                  // 16-byte chunks per rank row
    constexpr int D = NR - 2;                   // units in flight per wave
    constexpr int EB = kPersistRows * R * 2;    // E rows of one row block
    using UT = PersistU<UF>;
    static_assert(NCH >= 8 && NCH % 2 == 0, "rank");
    static_assert(UT::LU * D <= 32, "vmcnt waits");
    static_assert(NKS >= 4, "the U read follows the stages that use the previous unit's U");
    extern __shared__ __align__(16) char smem_p[];
    __shared__ int ok_s;
    char* e_lds = smem_p;
    char* ring = smem_p + EB;
    int* xprev = reinterpret_cast<int*>(ring + kPersistWaves * NR * UT::UNIT);
    float* xsum = reinterpret_cast<float*>(xprev + kPersistRows);  // [wave][row][3]

    const FinStreamArgs& F = P.fin;
    const int V = P.V, B = P.B, G = P.gamma;
    const int tid = threadIdx.x;
    const int lane0 = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NU = P.nu, g = blockIdx.x;
    const int nrb = (B + kPersistRows - 1) / kPersistRows;

    if (g >= NU) {
        // Finalize workgroups: wave fw draws rows fw, fw + nfw, ... of each row
        // block, positions in order; each draw waits for its row's shares.
        const int fw = (g - NU) * kPersistWaves + wave;
        const int nfw = ((int)gridDim.x - NU) * kPersistWaves;
        for (int k = 0; k < G; ++k) {
            for (int rb = 0; rb < nrb; ++rb) {
                const int r1 = min(B, (rb + 1) * kPersistRows);
                for (int b = rb * kPersistRows + fw; b < r1; b += nfw) {
                    int lane = lane0;
                    asm volatile("" : "+v"(lane));
                    if (!finalize_row_stream<true, true>(F, b, k, lane)) return;
                }
            }
        }
        return;
    }

    const int blo = (int)((long long)g * P.nblk / NU);
    const int bhi = (int)((long long)(g + 1) * P.nblk / NU);
    auto wave_blocks = [&](int w) { return min(NB, max(0, (bhi - blo - w + 3) / 4)); };
    const int nj = wave_blocks(wave);   // this wave's blocks: blo + wave + 4 j, j < nj
    const size_t bpad = (size_t)P.bpad;
    const float sc = F.invT * 1.4426950408889634f;   // exp(y / T) = 2^(y * sc)

    // Resident MFMA A operands: block j, rank step ks, MFMA row lane % 32.
    const int i32 = lane0 & 31;
    const int h0 = lane0 >> 5;
    const int ptok = 16 * ((i32 >> 2) & 1) + 8 * ((i32 >> 3) & 1) + 4 * (i32 >> 4) + (i32 & 3);
    bf16x8_t wf[NB][NKS];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const bool ok = j < nj;
        const int v = (ok ? blo + wave + 4 * j : 0) * kStreamSeg + ptok;
        const int swz = w2p_swizzle(v & (kPackTile - 1), NCH);
        const uint16_t* row = F.W2P + (size_t)v * R;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (ok) {
                wf[j][ks] = *reinterpret_cast<const bf16x8_t*>(row + (((2 * ks + h0) ^ swz) << 3));
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) wf[j][ks][t] = (__bf16)0.0f;
            }
        }
    }

    struct Red {
        float m, g0, g1;
        int am;
    };
    // Reduction of one finished unit (block t, this lane's row) in 16 stages,
    // so that the next unit's MFMAs can be interleaved with it: logits
    // x = accumulators + U (tokens past V carry U = -inf and W2 = 0), the
    // block max, then this lane's two 8-token group sums relative to it
    // (greedy: max and argmax).  Accumulator 4g + c holds run position
    // 8 (g & 1) + 4 (g >> 1) + c.
    struct Reducer {
        float x[16];
        float ma, mb, m, ms, g0, g1;
        int am;
    };
    // vb: the first of this lane's 16 tokens (greedy only).
    auto stage = [&](Reducer& R, const f32x16_t& ac, const auto& uf, int vb, int st) {
        if (st < 4) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int pos = 8 * (st & 1) + 4 * (st >> 1) + c;
                float uv;
                if constexpr (UF) {
                    uv = __uint_as_float(uf[pos >> 2][pos & 3]);
                } else {
                    const uint32_t w = uf[pos >> 3][(pos & 7) >> 1];
                    uv = (pos & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
                }
                R.x[pos] = ac[4 * st + c] + uv;
            }
        } else if (st == 4) {
            R.ma = fmaxf(fmaxf(fmaxf(R.x[0], R.x[1]), fmaxf(R.x[2], R.x[3])),
                         fmaxf(fmaxf(R.x[4], R.x[5]), fmaxf(R.x[6], R.x[7])));
        } else if (st == 5) {
            R.mb = fmaxf(fmaxf(fmaxf(R.x[8], R.x[9]), fmaxf(R.x[10], R.x[11])),
                         fmaxf(fmaxf(R.x[12], R.x[13]), fmaxf(R.x[14], R.x[15])));
        } else if (st == 6) {
            R.m = fmaxf(R.ma, R.mb);
            if constexpr (GREEDY) {
                R.am = INT_MAX;
            } else {
                R.m = pair_max32(R.m);
                R.ms = R.m == -INFINITY ? 0.0f : R.m * sc;   // all -inf: every weight 0
                R.g0 = 0.0f;
                R.g1 = 0.0f;
            }
        } else if (st < 15) {
            const int q = st - 7;
            if constexpr (GREEDY) {
                R.am = (R.x[15 - 2 * q] == R.m) ? vb + 15 - 2 * q : R.am;
                R.am = (R.x[14 - 2 * q] == R.m) ? vb + 14 - 2 * q : R.am;
                if (q == 7) pair_argmax32(R.m, R.am);
            } else {
                R.g0 += __builtin_amdgcn_exp2f(fmaf(R.x[q], sc, -R.ms));
                R.g1 += __builtin_amdgcn_exp2f(fmaf(R.x[8 + q], sc, -R.ms));
            }
        }
    };
    auto finish = [&](const Reducer& R) -> Red {
        Red o;
        o.m = R.m;
        o.g0 = GREEDY ? 0.0f : R.g0;
        o.g1 = GREEDY ? 0.0f : R.g1;
        o.am = GREEDY ? R.am : 0;
        return o;
    };
    auto reduce = [&](const f32x16_t& ac, const auto& uf, int vb) -> Red {
        Reducer R;
#pragma unroll
        for (int st = 0; st < 15; ++st) stage(R, ac, uf, vb, st);
        return finish(R);
    };

    const char* ninf = reinterpret_cast<const char*>(P.bar + (UF ? kBarNegInfF : kBarNegInf));
    const char* ubase = reinterpret_cast<const char*>(F.U);
    const char* usrc[4];   // the first UT::LU used
    int utok[4], urow[4];
    int rows_b = 0;
    const size_t rg_step = (size_t)32 * G * (size_t)V;
    int ci = 0, cj = 0, cs = 0;
    size_t coff = 0;
    // U cursor of row block rbb at position kk: row group, block, ring slot,
    // and the U offset of (ci, cj) from the lane's unit-0 address.
    auto setup_cursor = [&](int kk, int rbb) {
        int ln = lane0;
        asm volatile("" : "+v"(ln));
        const int rr0 = rbb * kPersistRows;
        rows_b = min(kPersistRows, B - rr0);
#pragma unroll
        for (int q = 0; q < UT::LU; ++q) {
            // load q covers rows (32 / UT::LU) q .. + 32 / UT::LU - 1, UT::CPR lanes per row
            const int m = (32 / UT::LU) * q + ln / UT::CPR;
            const int c = UF ? ((ln & 7) ^ uswz8(m)) : ((ln & 3) ^ uswz(m));
            urow[q] = m;
            utok[q] = kStreamSeg * (blo + wave) + (16 / UT::ES) * c;
            usrc[q] = ubase + (((size_t)(rr0 + m) * G + kk) * (size_t)V + utok[q]) * UT::ES;
        }
        ci = 0;
        cj = 0;
        cs = 0;
        coff = 0;
    };
    for (int k = 0; k < G; ++k) {
        for (int rb = 0; rb < nrb; ++rb) {
            // Per-lane values below are recomputed for every row block from an
            // opaque copy of the lane id: hoisted out of the position loop they
            // would stay live next to the resident W2 operands and be spilled.
            int lane = lane0;
            asm volatile("" : "+v"(lane));
            const int h = lane >> 5, n = lane & 31;
            const int r0 = rb * kPersistRows;
            const int rows = min(kPersistRows, B - r0);
            const int nrg = (rows + 31) / 32;
            // 1. conditioning tokens of the row block (-1: invalid or absent):
            // the anchors, then the tokens the finalize workgroups publish.
            if (k == 0) {
                if (tid < kPersistRows) {
                    const int prev = tid < rows ? F.x0[r0 + tid] : -1;
                    xprev[tid] = (prev >= 0 && prev < V) ? prev : -1;
                }
                __syncthreads();
            } else if (!rows_tokens(P.bar, F.tflag, r0, rows, (unsigned)k, V, F.poll_limit, xprev,
                                    &ok_s)) {
                return;
            }
            // 2. E rows into LDS.  The first D units of U were issued at the end of
            //    the previous row block (here only for the launch's first block).
#pragma unroll
            for (int q = 0; q < NCH / 4; ++q) {
                const int pc = q * kPersistWaves + wave;
                const int o = pc * 64 + lane;
                const int row = o / NCH, slot = o % NCH;
                const int p = max(xprev[row], 0);
                __builtin_amdgcn_global_load_lds(F.W1 + (size_t)p * R + ((slot ^ (row & 7)) << 3),
                                                 (lds_ptr_t)(e_lds + pc * 1024), 16, 0, 0);
            }
            // U of unit (rgi, j): rows 32 rgi .. + 31 of the row block, the 64
            // bytes of block blo + wave + 4 j in each, into a ring slot of 32
            // rows x 64 bytes with 16-byte chunk c of row m in slot
            // c ^ uswz(m): direct load q (of 2) covers rows 16 q .. + 15, four
            // lanes per row, so each load reads whole 64-byte row pieces.
            // Absent rows and tokens read the -inf chunk.  A cursor issues
            // units in order; past the last unit it issues the same two loads
            // of the -inf chunk into the slot just freed, so every wait allows
            // the same count.
            auto issue_next = [&]() {
                char* dst = ring + (wave * NR + cs) * UT::UNIT;
                const int rlim = rows_b - 32 * ci;   // rows of the group present (<= 0 past the last)
                const int vlim = V - 128 * cj;
#pragma unroll
                for (int q = 0; q < UT::LU; ++q) {
                    const bool ok = urow[q] < rlim && utok[q] < vlim;
                    __builtin_amdgcn_global_load_lds(ok ? usrc[q] + coff * UT::ES : ninf,
                                                     (lds_ptr_t)(dst + q * 1024), 16, 0, 0);
                }
                coff += 128;
                if (++cj == nj) {
                    cj = 0;
                    ++ci;
                    coff += rg_step - (size_t)128 * nj;
                }
                if (++cs == NR) cs = 0;
            };
            if (nj > 0 && k == 0 && rb == 0) {
                setup_cursor(k, rb);
#pragma unroll
                for (int u = 0; u < D; ++u) issue_next();
                wait_vm<UT::LU * D>();                     // this wave's E loads have landed
            } else {
                wait_vm<0>();                          // E (and the U issued before it)
            }
            asm volatile("s_barrier" ::: "memory");    // ... and every wave's

            // 3. units of this wave, row group major.
            auto flush_run = [&](int rgi, float m, float s, int a) {
                if (h == 0) {
                    float* xs = xsum + ((size_t)wave * kPersistRows + 32 * rgi + n) * 3;
                    xs[0] = m;
                    xs[1] = s;
                    xs[2] = __int_as_float(a);
                }
            };
            // summaries of unit (rgi, j) at offset 4 j bpad + 32 rgi from the lane's base
            float* segm_l = P.segm + (size_t)(blo + wave) * bpad + r0 + n;
            float* gs_l = P.gsums + ((size_t)(blo + wave) * bpad + r0 + n) * 4 + 2 * h;
            // Every lane stores: rows without a valid conditioning token or past
            // B hold values nothing reads, and both halves of a row hold the
            // same block max.
            auto store = [&](const Red& o, int off) {
                if constexpr (!GREEDY) coh_store_f32x2<true>(gs_l + (size_t)off * 4, o.g0, o.g1);
                coh_store<true>(segm_l + off, o.m);
            };
            float run_m = -INFINITY, run_s = 0.0f;
            int run_a = INT_MAX;
            auto absorb = [&](const Red& o) {
                if constexpr (GREEDY) {
                    run_a = (o.m > run_m || (o.m == run_m && o.am < run_a)) ? o.am : run_a;
                    run_m = fmaxf(run_m, o.m);
                } else {
                    const float tot = pair_sum32(o.g0 + o.g1);
                    const float nm = fmaxf(run_m, o.m);
                    const float a = run_m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((run_m - nm) * sc);
                    const float c = o.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((o.m - nm) * sc);
                    run_s = run_s * a + tot * c;
                    run_m = nm;
                }
            };
            auto flush_reset = [&](int rgi) {
                flush_run(rgi, run_m, run_s, run_a);
                run_m = -INFINITY;
                run_s = 0.0f;
                run_a = INT_MAX;
            };

            // The pipeline starts from a previous unit whose logits are all -inf
            // (U = -inf, zero accumulators): it reduces to an empty record (max
            // -inf, sums 0) that stores into the first unit's slots, overwritten
            // later, and leaves the running summary unchanged.
            f32x16_t accp;
#pragma unroll
            for (int q = 0; q < 16; ++q) accp[q] = 0.0f;
            const uint32_t ni = UF ? 0xFF800000u : 0xFF80FF80u;
            const u32x4_t ninf4 = u32x4_t{ni, ni, ni, ni};
            u32x4_t ufp[4];
#pragma unroll
            for (int q = 0; q < UT::LU; ++q) ufp[q] = ninf4;
            Red redh;
            redh.m = -INFINITY;
            redh.g0 = redh.g1 = 0.0f;
            redh.am = INT_MAX;
            int tp = 0, offp = 0, rgp = 0, offh = 0, rgh = 0;
            int done = 0;   // units consumed
            int cu = 0;     // ring slot of the next unit
            bf16x8_t e[NKS];
            for (int rgi = 0; rgi < nrg; ++rgi) {
                {   // B operand of row group rgi: row 32 rgi + n, chunk 2 ks + h
                    const uint16_t* er = reinterpret_cast<const uint16_t*>(e_lds) + (32 * rgi + n) * R;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        e[ks] = *reinterpret_cast<const bf16x8_t*>(er + (((2 * ks + h) ^ (n & 7)) << 3));
                }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if (j < nj) {
                        // This unit's MFMAs, each followed by a stage of the previous
                        // unit's reduction; the stores and the running-summary update
                        // of the unit before that, the next direct load and the read of
                        // this unit's U go between them.  The order is fixed by
                        // scheduling barriers.
                        f32x16_t acc;
#pragma unroll
                        for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
                        Reducer Rd;
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) {
                            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j][ks], e[ks], acc, 0, 0, 0);
#pragma unroll
                            for (int st = ks * 15 / NKS; st < (ks + 1) * 15 / NKS; ++st)
                                stage(Rd, accp, ufp, tp * kStreamSeg + 16 * h, st);
                            if (ks == 0) store(redh, offh);
                            if (ks == 1) issue_next();
                            if (ks == 2) {
                                absorb(redh);
                                // the unit after it opened a row group (j - 1 == 0): flush
                                if (j == 1 || nj == 1) flush_reset(rgh);
                            }
                            if (ks == 3 * NKS / 4) {
                                // U of this unit for the next reduction (the stages that
                                // read the previous unit's U are done): D newer units are
                                // in flight.
                                wait_vm<UT::LU * D>();
                                const u32x4_t* us = reinterpret_cast<const u32x4_t*>(
                                    ring + (wave * NR + cu) * UT::UNIT);
#pragma unroll
                                for (int q = 0; q < UT::LU; ++q)
                                    ufp[q] = UF ? us[UT::CPR * n + ((4 * h + q) ^ uswz8(n))]
                                                : us[UT::CPR * n + ((2 * h + q) ^ uswz(n))];
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        if (++cu == NR) cu = 0;
                        redh = finish(Rd);
                        offh = offp;
                        rgh = rgp;
                        accp = acc;
                        tp = blo + wave + 4 * j;
                        offp = 4 * j * (int)bpad + 32 * rgi;
                        rgp = rgi;
                        ++done;
                    }
                }
            }
            if (done >= 1) {
                store(redh, offh);
                absorb(redh);
                if (nj == 1 || done == 1) flush_reset(rgh);
                const Red red = reduce(accp, ufp, tp * kStreamSeg + 16 * h);
                absorb(red);
                store(red, offp);
                flush_reset(rgp);
            }
            wait_vm<0>();      // this wave's segment summaries are out (written through)
            // The next row block's first units: U does not depend on the tokens.
            // The barriers below wait for LDS only, so these loads stay in flight
            // while the share summaries go out and the next tokens are awaited.
            {
                const int rbn = rb + 1 < nrb ? rb + 1 : 0;
                const int kn = rb + 1 < nrb ? k : k + 1;
                if (nj > 0 && kn < G) {
                    setup_cursor(kn, rbn);
#pragma unroll
                    for (int u = 0; u < D; ++u) issue_next();
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // xsum written
            // 4. one summary per (share, row): merge the waves' runs, tagged with
            // k + 1 in both words (read by the finalize without a grid barrier).
            if (tid < rows && xprev[tid] >= 0) {
                float m = -INFINITY, s = 0.0f;
                int a = INT_MAX;
                for (int w = 0; w < kPersistWaves; ++w) {
                    if (wave_blocks(w) == 0) continue;
                    const float* xs = xsum + ((size_t)w * kPersistRows + tid) * 3;
                    const float m2 = xs[0], s2 = xs[1];
                    const int a2 = __float_as_int(xs[2]);
                    if constexpr (GREEDY) {
                        merge_arg(m, a, m2, a2);
                    } else {
                        const float nm = fmaxf(m, m2);
                        const float ca = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m - nm) * sc);
                        const float cb = m2 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m2 - nm) * sc);
                        s = s * ca + s2 * cb;
                        m = nm;
                    }
                }
                const uint64_t tag = (uint64_t)(k + 1) << 32;
                uint64_t* e64 = reinterpret_cast<uint64_t*>(P.sup) +
                                2 * ((size_t)g * bpad + r0 + tid);
                coh_store<true>(e64, tag | __float_as_uint(m));
                coh_store<true>(e64 + 1, tag | (GREEDY ? (uint32_t)a : __float_as_uint(s)));
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // LDS (E, xsum) is reused by the next row block
        }
    }
}

template <int NKS, int NB, int NR, bool GREEDY, bool UF>
__global__ __launch_bounds__(kPersistWaves * 64, 1)
void draft_persist(PersistArgs P) {
    draft_persist_body<NKS, NB, NR, GREEDY, UF>(P);
}

// Blocks per wave held in registers (320 VGPRs of W2 operands) and U ring
// slots per wave (LDS: E rows + rings + tokens + run summaries <= 160 KB).
// Shallow rings are faster (measured): the units' 64-byte row pieces stream
// worse the more of them the chip has in flight, and with each row block's
// first units issued at the end of the previous block, two (r = 256) or
// three (r = 128, 64) units ahead keep the loop fed.
template <int NKS> struct PersistShape;
template <> struct PersistShape<16> { static constexpr int NB = 5, NR = 4; };
template <> struct PersistShape<8> { static constexpr int NB = 10, NR = 5; };
template <> struct PersistShape<4> { static constexpr int NB = 20, NR = 5; };

template <int NKS, bool UF>
static size_t persist_lds() {
    return (size_t)kPersistRows * NKS * 16 * 2 +
           (size_t)kPersistWaves * PersistShape<NKS>::NR * kPersistUnit * (UF ? 2 : 1) +
           kPersistRows * sizeof(int) + (size_t)kPersistWaves * kPersistRows * 3 * sizeof(float);
}

static int persist_nks(int r) { return r == 256 ? 16 : (r == 128 ? 8 : (r == 64 ? 4 : 0)); }

static int persist_nb(int r) {
    switch (persist_nks(r)) {
    case 16: return PersistShape<16>::NB;
    case 8: return PersistShape<8>::NB;
    case 4: return PersistShape<4>::NB;
    default: return 0;
    }
}

// The two process-wide settings of the persistent draft (spec_draft_set_persistent,
// spec_draft_set_poll_limit).  Atomic: a call reads each once, when it
// launches, so a change made by another thread applies from the next call on.
// Engine: 0 per-position kernels; 1 persistent, plain launch; 2 persistent,
// cooperative launch.
static std::atomic<int> g_persist_mode{1};
static std::atomic<unsigned> g_poll_limit{kBarrierPolls};

unsigned persist_set_poll_limit(unsigned polls) {
    return g_poll_limit.exchange(polls == 0 ? kBarrierPolls : polls);
}

unsigned persist_poll_limit() { return g_poll_limit.load(); }

int persist_set_mode(int mode) {
    if (mode < 0 || mode > 2) return -1;
    return g_persist_mode.exchange(mode);
}

int persist_mode() { return g_persist_mode.load(); }

static int persist_device_ok() {
    // per-device cache: CUs if the device can run the persistent draft, -1 if
    // not, 0 unknown; concurrent first calls store the same value
    static std::atomic<int> ok[64];
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 0 || dev >= 64) return 0;
    int v = ok[dev].load(std::memory_order_relaxed);
    if (!v) {
        int coop = 0, cus = 0;
        if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess)
            coop = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        v = coop && cus > 0 ? cus : -1;
        ok[dev].store(v, std::memory_order_relaxed);
    }
    return v > 0 ? v : 0;
}

// Workgroups of the persistent draft, one per CU: kPersistFinWgs finalize
// workgroups (fewer on a small device) and nu unit workgroups, at most one per
// 32-token block and at most kMaxShares (the finalize reads four shares per
// lane).  Returns nu + nf, or 0 when the device cannot run it.
static int persist_grid(int V, int* nu_out) {
    const int cus = persist_device_ok();
    const int nblk = (V + kStreamSeg - 1) / kStreamSeg;
    const int nf = std::max(1, std::min(kPersistFinWgs, cus / 16));
    const int nu = std::min(std::min(cus - nf, nblk), kMaxShares);
    if (nu <= 0) return 0;
    if (nu_out) *nu_out = nu;
    return nu + nf;
}

bool draft_persists(const DraftArgs& a, int mode) {
    if (mode == 0) return false;
    if (!(a.head == kHeadMarkov && a.w_bf16 && !a.q_logits && (a.V % 8) == 0 &&
          persist_nks(a.r) != 0 && a.B > 0 && a.gamma > 0))
        return false;
    int nu = 0;
    if (persist_grid(a.V, &nu) <= 0) return false;
    const int nblk = (a.V + kStreamSeg - 1) / kStreamSeg;
    return (nblk + nu - 1) / nu <= kPersistWaves * persist_nb(a.r);   // <= 20 blocks per share
}

template <int NKS, bool UF>
static hipError_t launch_persist(const PersistArgs& p, int ng, bool greedy, bool coop,
                                 hipStream_t s) {
    constexpr int NB = PersistShape<NKS>::NB, NR = PersistShape<NKS>::NR;
    const void* fn = greedy ? reinterpret_cast<const void*>(&draft_persist<NKS, NB, NR, true, UF>)
                            : reinterpret_cast<const void*>(&draft_persist<NKS, NB, NR, false, UF>);
    const size_t lds = persist_lds<NKS, UF>();
    // raise the dynamic LDS limit once per process (thread-safe)
    static std::once_flag attr_once;
    std::call_once(attr_once, [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_persist<NKS, NB, NR, true, UF>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_persist<NKS, NB, NR, false, UF>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        (void)hipGetLastError();
    });
    PersistArgs arg = p;
    void* args[] = {&arg};
    // Every workgroup must be resident at once (one per CU, grid <= CUs).  A
    // cooperative launch guarantees it by running alone on the device, which
    // costs ~10 us of idle device on each side of the launch; a plain launch
    // gets it whenever no other kernel holds CUs meanwhile, and otherwise the
    // bounded waits give up (abort word set, tokens left at -1).
    if (coop)
        return hipLaunchCooperativeKernel(fn, dim3(ng), dim3(kPersistWaves * 64), args,
                                          (unsigned)lds, s);
    return hipLaunchKernel(fn, dim3(ng), dim3(kPersistWaves * 64), args, (unsigned)lds, s);
}

hipError_t persist_clear_abort(unsigned* bar, hipStream_t s) {
    hipLaunchKernelGGL(persist_bar_reset, dim3(1), dim3(64), 0, s, bar, nullptr, 0, nullptr,
                       (size_t)0, nullptr, (size_t)0);
    return hipGetLastError();
}

hipError_t draft_persist_launch(const DraftArgs& a, unsigned* bar, int mode, hipStream_t s) {
    int nu = 0;
    const int ng = persist_grid(a.V, &nu);
    if (ng <= 0 || !bar || !a.tflag || !a.W2T) return hipErrorInvalidValue;
    PersistArgs p{};
    FinStreamArgs& f = p.fin;
    const int nblk = (a.V + kStreamSeg - 1) / kStreamSeg;
    const int bpad = (a.B + kStreamRows - 1) / kStreamRows * kStreamRows;
    f.sup = a.sup;
    f.segm = reinterpret_cast<const float*>(a.stats);
    f.gsums = a.gsums;
    f.ws = nu;
    f.nunit = nblk;
    f.seg_mult = 1;
    f.bpad = bpad;
    f.x0 = a.x0;
    f.tokens = a.tokens;
    f.q_logZ = a.q_logZ;
    f.q_tok = a.q_tok;
    f.uniforms = a.uniforms;
    f.seed = a.seed;
    f.offset = a.offset;
    f.gamma = a.gamma;
    f.V = a.V;
    f.invT = a.invT;
    f.greedy = a.greedy;
    f.U = a.U;
    f.u_f32 = a.u_bf16 ? 0 : 1;
    f.W1 = static_cast<const uint16_t*>(a.W1);
    f.W2P = a.W2T;
    f.r = a.r;
    f.tflag = a.tflag;
    f.abort_word = bar + kBarAbort;
    f.poll_limit = g_poll_limit.load();
    p.segm = reinterpret_cast<float*>(a.stats);
    p.gsums = a.gsums;
    p.sup = a.sup;
    p.bar = bar;
    p.B = a.B;
    p.gamma = a.gamma;
    p.V = a.V;
    p.nblk = nblk;
    p.bpad = bpad;
    p.nu = nu;
    const size_t ns = (size_t)nu * bpad;
    const size_t ntok = (size_t)a.B * a.gamma;
    const size_t nreset = std::max<size_t>(std::max<size_t>(kBarWords, a.B), std::max(2 * ns, ntok));
    const unsigned nblk_reset = (unsigned)std::min<size_t>((nreset + 255) / 256, 1024);
    hipLaunchKernelGGL(persist_bar_reset, dim3(nblk_reset), dim3(256), 0, s, bar, a.tflag, a.B,
                       reinterpret_cast<uint64_t*>(a.sup), ns, a.tokens, ntok);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool g = a.greedy != 0, c = mode == 2;
    switch (persist_nks(a.r)) {
    case 16: return a.u_bf16 ? launch_persist<16, false>(p, ng, g, c, s) : launch_persist<16, true>(p, ng, g, c, s);
    case 8: return a.u_bf16 ? launch_persist<8, false>(p, ng, g, c, s) : launch_persist<8, true>(p, ng, g, c, s);
    case 4: return a.u_bf16 ? launch_persist<4, false>(p, ng, g, c, s) : launch_persist<4, true>(p, ng, g, c, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace specdec
