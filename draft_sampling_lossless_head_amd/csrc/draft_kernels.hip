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
#include <algorithm>
#include <atomic>
#include <mutex>
#include <climits>

#include "device_common.hpp"
#include "launch.hpp"
#include "stream_finalize.hpp"

namespace specdec {

constexpr int kTileV = 128;   // vocabulary columns per tile workgroup
static_assert(kTileV == kPackTile, "a bias tile is one tile of the packed W2 image");
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
// Workgroup = 4 waves on one 128-token tile and Rt = 32*WB request rows.  WB
// waves split the rows (32 each), the other 4/WB split the columns, so each
// wave owns MB = WB blocks of 32 columns.  The MFMA computes
// C[v][b] = sum_j W2[j][v] * E[b][j]:
//   A operand (32 v x 16 j) from the W2 tile transposed into LDS,
//   B operand (16 j x 32 b) from the E rows held in registers.
// The accumulators are then written back into the same LDS as an [Rt][128]
// fp32 tile, and the epilogue walks it row-contiguously: 16 lanes per request
// row, 8 tokens per lane, U prefetched at kernel start, q stored with
// nontemporal 16-byte stores, and the row summary reduced over the 16 lanes.
// Row-contiguous access matters: with the MFMA lane layout each store
// instruction would touch 32 request rows 16 bytes at a time.
// ---------------------------------------------------------------------------
constexpr int kOutLd = kTileV + 4;   // fp32 row stride of the staged output tile

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// W2 [r, V] -> packed image (bf16; layout at w2p_index): 64 x 64 blocks of
// (rank, token) through LDS with 16-byte global accesses on both sides; tokens
// from V up to the end of the last 128-token tile are written as zeros.
__global__ __launch_bounds__(256)
void w2_pack(const uint16_t* __restrict__ W2, uint16_t* __restrict__ W2P, int r, int V) {
    __shared__ __align__(16) uint16_t t[64][72];   // [j][v]
    const int v0 = blockIdx.x * 64;
    const int j0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    const bool vec = (V % 8) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + i * 256;
        const int jj = c / 8, vc = (c % 8) * 8;
        const int j = j0 + jj, v = v0 + vc;
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (j < r) {
            if (vec && v + 8 <= V) {
                val = *reinterpret_cast<const uint4*>(W2 + (size_t)j * V + v);
            } else {
                uint32_t w[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint32_t lo = v + 2 * h < V ? W2[(size_t)j * V + v + 2 * h] : 0u;
                    const uint32_t hi = v + 2 * h + 1 < V ? W2[(size_t)j * V + v + 2 * h + 1] : 0u;
                    w[h] = lo | (hi << 16);
                }
                val = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        *reinterpret_cast<uint4*>(&t[jj][vc]) = val;
    }
    __syncthreads();
    const int vpad = (V + kPackTile - 1) / kPackTile * kPackTile;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + i * 256;
        const int vv = c / 8, jc = (c % 8) * 8;
        const int v = v0 + vv, j = j0 + jc;
        if (v < vpad && j < r) {
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 4; ++h)
                w[h] = (uint32_t)t[jc + 2 * h][vv] | ((uint32_t)t[jc + 2 * h + 1][vv] << 16);
            *reinterpret_cast<uint4*>(W2P + w2p_index(v, j, r)) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// Workgroup = 4 waves on one 128-token tile and RT = 32*WB request rows.
// OUT selects what the tile produces (see kOutQ / kOutStats / kOutResidual).
template <int WB, int MODE, bool U_BF16, int OUT>
__global__ __launch_bounds__(256, 2)
void draft_tile_mfma(TileParams P) {
    constexpr int MB = WB;
    constexpr int NS = (MODE == kHeadRnn) ? 3 : 1;
    constexpr int RT = 32 * WB;            // request rows of the tile
    constexpr int ITEMS = RT * 16 / 256;   // (row, 8-token group) items per thread
    extern __shared__ __align__(16) uint16_t smem[];
    const int V = P.V, r = P.r, k = P.k, B = P.B, gamma = P.gamma;
    const int ldr = r + kLdsPad;
    uint16_t* w2t = smem;                                   // [kTileV][ldr] bf16
    float* otile = reinterpret_cast<float*>(smem);          // [RT][kOutLd] fp32 (reused)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wb = wave % WB;
    const int wv = wave / WB;
    const int v_tile = blockIdx.x * kTileV;
    const int row0 = blockIdx.y * RT;
    const int b = row0 + wb * 32 + (lane & 31);
    const int kgrp = lane >> 5;
    const int nks = r / 16;
    const bool vec_u = U_BF16 ? (V % 8) == 0 : (V % 4) == 0;

    // Position of request row br (kOutResidual: its own; -1 = inactive).
    auto row_position = [&](int br) -> int {
        if (br >= B) return -1;
        return OUT == kOutResidual ? P.row_pos[br] : k;
    };
    auto u_offset = [&](int br, int pos) -> size_t {
        return ((size_t)br * gamma + pos) * (size_t)V;
    };
    auto out_offset = [&](int br, int pos) -> size_t {
        return OUT == kOutResidual ? (size_t)br * V : ((size_t)br * gamma + pos) * (size_t)V;
    };

    // 1) the packed W2 tile: one contiguous block of kTileV rows of r bf16
    //    (zero past V), read in 16-byte chunks and un-swizzled into LDS.
    const int cpr = r / 8;                       // chunks per token row
    const int nchunk = kTileV * cpr;             // <= 4096
    const uint16_t* wtile = P.W2T + (size_t)v_tile * r;
    uint4 wch[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c = tid + i * 256;
        wch[i] = make_uint4(0u, 0u, 0u, 0u);
        if (c < nchunk) wch[i] = *reinterpret_cast<const uint4*>(wtile + (size_t)c * 8);
    }

    // 2) prefetch this thread's U items.  Item (row, j) covers the two runs of
    //    four tokens 4j .. 4j+3 and 64 + 4j .. 64 + 4j + 3 of the tile row, so
    //    the 16 lanes of a row read and write 256 contiguous bytes per access.
    u32x4_t ureg[ITEMS][2];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int item = tid + it * 256;
        const int br = row0 + item / 16;
        const int pos = row_position(br);
        const int va = v_tile + (item % 16) * 4;
        ureg[it][0] = u32x4_t{0u, 0u, 0u, 0u};
        ureg[it][1] = u32x4_t{0u, 0u, 0u, 0u};
        if (pos >= 0 && vec_u && va + 68 <= V) {
            const size_t off = u_offset(br, pos) + va;
            if constexpr (U_BF16) {
                const u32x2_t a0 = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(P.U) + off));
                const u32x2_t a1 = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(P.U) + off + 64));
                ureg[it][0] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
            } else {
                ureg[it][0] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t*>(static_cast<const float*>(P.U) + off));
                ureg[it][1] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t*>(static_cast<const float*>(P.U) + off + 64));
            }
        }
    }

    // 3) conditioning rows (Markov: W1[x_{pos-1}]; RNN: split o rows).
    const int bpos = row_position(b);
    int prev = 0;
    bool erow_ok = bpos >= 0;
    if (MODE == kHeadMarkov && bpos >= 0) {
        prev = (bpos == 0) ? P.x0[b] : P.tokens[(size_t)b * gamma + bpos - 1];
        erow_ok = prev >= 0 && prev < V;
    }
    auto load_e = [&](int split, bf16x8_t (&e)[16]) {
        const uint16_t* erow =
            (MODE == kHeadMarkov)
                ? P.W1 + (size_t)prev * r
                : P.Erows + (((size_t)(b < B ? b : 0) * gamma + (bpos > 0 ? bpos : 0)) * 3 + split) * r;
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
    };
    // With up to 64 rows per tile the registers hold two sets of B operands:
    // the first set is loaded here, in flight with the W2 tile and U, and each
    // later RNN term is loaded while the previous one is multiplied (with
    // 128 rows each set is loaded just before its MFMAs).
    constexpr bool EPRE = WB <= 2;
    bf16x8_t e0[16], e1[16];
    if constexpr (EPRE) load_e(0, e0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c = tid + i * 256;
        if (c < nchunk) {
            const int vr = c / cpr;
            const int kc = (c % cpr) ^ w2p_swizzle(vr, cpr);
            *reinterpret_cast<uint4*>(w2t + vr * ldr + kc * 8) = wch[i];
        }
    }
    f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
    __syncthreads();

    // 4) the contraction (RNN: three bf16 terms of o against the same tile).
    auto contract = [&](const bf16x8_t (&e)[16]) {
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
    };
    // term t uses set t % 2; with EPRE, term t + 1 goes into the other set first
    if constexpr (EPRE) {
        if constexpr (NS > 1) load_e(1, e1);
        contract(e0);
        if constexpr (NS > 1) {
            if constexpr (NS > 2) load_e(2, e0);
            contract(e1);
        }
        if constexpr (NS > 2) contract(e0);
    } else {
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) {
            load_e(sp, e0);
            contract(e0);
        }
    }

    // 5) accumulators -> LDS as an [RT][128] fp32 tile (row = request).
    __syncthreads();
    {
        const int rl = wb * 32 + (lane & 31);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = wv * (32 * MB) + mb * 32 + g * 8 + kgrp * 4;
                *reinterpret_cast<float4*>(otile + rl * kOutLd + c) =
                    make_float4(acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2],
                                acc[mb][4 * g + 3]);
            }
    }
    __syncthreads();

    // 6) row-contiguous epilogue: l = U + bias, store l (kOutQ, kOutResidual),
    //    and the row summary of the tile (max, sum exp((l - max)/T), lowest
    //    argmax) reduced over the row's 16 lanes with DPP moves.
    const int nseg = gridDim.x;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int item = tid + it * 256;
        const int rl = item / 16;
        const int br = row0 + rl;
        const int pos = row_position(br);
        const int ca = (item % 16) * 4;            // first run: tile columns ca .. ca+3
        const int va = v_tile + ca;                // second run: va + 64 ..
        const float4 b0 = *reinterpret_cast<const float4*>(otile + rl * kOutLd + ca);
        const float4 b1 = *reinterpret_cast<const float4*>(otile + rl * kOutLd + ca + 64);
        float x[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        int vi[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) vi[t] = va + (t & 3) + (t >> 2) * 64;
        const bool rowok = pos >= 0;
        const size_t uoff = u_offset(rowok ? br : 0, rowok ? pos : 0) + va;
        const size_t ooff = out_offset(rowok ? br : 0, rowok ? pos : 0) + va;
        if (rowok && vec_u && va + 68 <= V) {
            if constexpr (U_BF16) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    x[2 * h] += bf16_bits_to_float(ureg[it][0][h] & 0xFFFFu);
                    x[2 * h + 1] += bf16_bits_to_float(ureg[it][0][h] >> 16);
                }
            } else {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    x[h] += __uint_as_float(ureg[it][0][h]);
                    x[4 + h] += __uint_as_float(ureg[it][1][h]);
                }
            }
            if (OUT != kOutStats) {
                f32x4_t o0 = {x[0], x[1], x[2], x[3]};
                f32x4_t o1 = {x[4], x[5], x[6], x[7]};
                __builtin_nontemporal_store(o0, reinterpret_cast<f32x4_t*>(P.out + ooff));
                __builtin_nontemporal_store(o1, reinterpret_cast<f32x4_t*>(P.out + ooff + 64));
            }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const size_t d = (t & 3) + (t >> 2) * 64;
                if (rowok && vi[t] < V) {
                    x[t] += load1<U_BF16>(P.U, uoff + d);
                    if (OUT != kOutStats) P.out[ooff + d] = x[t];
                } else {
                    x[t] = -INFINITY;
                }
            }
        }
        if (OUT == kOutResidual) continue;   // the verify pass needs no summaries
        float m = x[0];
#pragma unroll
        for (int t = 1; t < 8; ++t) m = fmaxf(m, x[t]);
        m = row16_max(m);
        float sa = 0.0f, sb = 0.0f;
        if (!P.greedy && m != -INFINITY) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sa += __expf((x[t] - m) * P.invT);
                sb += __expf((x[t + 4] - m) * P.invT);
            }
        }
        const float sum = row16_sum(sa + sb);
        int amax = INT_MAX;
#pragma unroll
        for (int t = 7; t >= 0; --t)
            if (x[t] == m) amax = min(amax, vi[t]);
        amax = row16_min(amax);
        if (OUT == kOutStats) {
            // 8-token group sums: lanes 2i and 2i+1 of a row hold the two
            // halves of groups i (first runs) and 8 + i (second runs).
            const float ga = sa + dpp_mov<kDppXor1>(sa);
            const float gb = sb + dpp_mov<kDppXor1>(sb);
            const int j = item % 16;
            if (rowok) {
                const int grp = (j & 1) ? 8 + (j >> 1) : (j >> 1);
                P.gsums[((size_t)br * nseg + blockIdx.x) * 16 + grp] = (j & 1) ? gb : ga;
            }
        }
        if (rowok && (item % 16) == 0) {
            SegStat st;
            st.m = m;
            st.s = sum;
            st.idx = amax;
            st.pad = 0;
            P.stats[(size_t)br * nseg + blockIdx.x] = st;
        }
    }
}

// ---------------------------------------------------------------------------
// q-free bias tile: summaries only, straight from the MFMA accumulators.
//
// Same work split as draft_tile_mfma (WB waves along the request rows, 4/WB
// along the tile's tokens, MB = WB blocks of 32 tokens per wave), but:
//   * the packed W2 tile is copied into LDS by direct global->LDS loads (16
//     bytes per lane, no register round trip) and read back swizzled;
//   * the A operand's rows are assigned to tokens so that every lane ends with
//     one contiguous run of RUN = 16 * MB tokens of its request row: MFMA row
//     i = 8g + 4h + c of block mb is token  wv*32*MB + 16*MB*h + 16*mb + 4g + c,
//     and the accumulator element idx of lane (b, h) is token
//     wv*32*MB + 16*MB*h + 16*mb + idx;
//   * U is read as that run (16-byte loads), and the epilogue reduces each
//     lane's run in registers: no output staging, no q store.
// Outputs per (row, tile): the SegStat (max, sum exp((l - max)/T), argmax) and
// the 16 sums over 8-token groups relative to the same max.
// ---------------------------------------------------------------------------

template <int WB, bool U_BF16>
__global__ __launch_bounds__(256, 2)
void draft_tile_stats(TileParams P) {
    constexpr int MB = WB;
    constexpr int NWV = 4 / WB;           // waves along the tile's tokens
    constexpr int RT = 32 * WB;           // request rows of the tile
    constexpr int RUN = 16 * MB;          // contiguous tokens per lane
    constexpr int NG = RUN / 8;           // 8-token groups per lane
    constexpr int UV = U_BF16 ? RUN / 8 : RUN / 4;   // 16-byte U loads per lane
    extern __shared__ __align__(16) uint16_t smem[];   // packed W2 tile [128][r]
    __shared__ float x_m[NWV][RT];
    __shared__ float x_s[NWV][RT];
    __shared__ int x_i[NWV][RT];
    const int V = P.V, r = P.r, k = P.k, B = P.B, gamma = P.gamma;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wb = wave % WB;
    const int wv = wave / WB;
    const int tile = blockIdx.x;
    const int v_tile = tile * kTileV;
    const int rl = wb * 32 + (lane & 31);  // request row within the tile
    const int b = blockIdx.y * RT + rl;
    const int h = lane >> 5;
    const int kgrp = lane >> 5;
    const int nks = r / 16;
    const int nchunk = r / 8;
    const bool active = b < B;

    // 1) the packed W2 tile (256 * r bytes) into LDS: wave w copies the 1 KB
    //    pieces w, w + 4, ... with one direct load per piece.
    {
        const char* src = reinterpret_cast<const char*>(P.W2T) + (size_t)tile * 256 * r;
        char* dst = reinterpret_cast<char*>(smem);
        const int npiece = r / 4;
        for (int pc = wave; pc < npiece; pc += 4)
            __builtin_amdgcn_global_load_lds(src + pc * 1024 + lane * 16,
                                             (lds_ptr_t)(dst + pc * 1024), 16, 0, 0);
    }

    // 2) the conditioning row E = W1[x_{k-1}] (MFMA B operand) and the U run.
    int prev = 0;
    bool erow_ok = false;
    if (active) {
        prev = (k == 0) ? P.x0[b] : P.tokens[(size_t)b * gamma + k - 1];
        erow_ok = prev >= 0 && prev < V;
    }
    const uint16_t* erow = P.W1 + (size_t)prev * r;
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
    f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
    __syncthreads();                 // ... and every other wave's

    // The U run, issued now so that it arrives during the contraction.  Each
    // lane reads whole lines over its consecutive loads, so these are plain
    // (cached) loads: a streaming hint would drop a line between them.
    const int run0 = wv * 32 * MB + 16 * MB * h;     // first token of the lane's run (tile-local)
    const int v0 = v_tile + run0;
    const size_t urow = ((size_t)(active ? b : 0) * gamma + k) * (size_t)V;
    const bool vec_u = (U_BF16 ? (V % 8) == 0 : (V % 4) == 0) && v0 + RUN <= V && erow_ok;
    u32x4_t ureg[UV];
#pragma unroll
    for (int q = 0; q < UV; ++q) {
        ureg[q] = u32x4_t{0u, 0u, 0u, 0u};
        if (vec_u) {
            if constexpr (U_BF16)
                ureg[q] = *reinterpret_cast<const u32x4_t*>(
                    static_cast<const uint16_t*>(P.U) + urow + v0 + q * 8);
            else
                ureg[q] = *reinterpret_cast<const u32x4_t*>(
                    static_cast<const float*>(P.U) + urow + v0 + q * 4);
        }
    }

    // 3) the contraction.  Lane l supplies A row i = l % 32 of each block.
    int arow[MB];
    int aswz[MB];
    {
        const int i = lane & 31;
        const int hi = (i >> 2) & 1, g = i >> 3, c = i & 3;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int vl = wv * 32 * MB + 16 * MB * hi + 16 * mb + 4 * g + c;
            arow[mb] = vl * r;
            aswz[mb] = w2p_swizzle(vl, nchunk);
        }
    }
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
        if (ks < nks) {
            const int kc = 2 * ks + kgrp;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                    smem + arow[mb] + ((kc ^ aswz[mb]) << 3));
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, e[ks], acc[mb], 0, 0, 0);
            }
        }
    }

    // 4) logits of the run: l = bias + U (-inf past V or for an inactive row).
    float x[RUN];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[16 * mb + i] = acc[mb][i];
    if (vec_u) {
#pragma unroll
        for (int q = 0; q < UV; ++q) {
            if constexpr (U_BF16) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    x[8 * q + 2 * t] += bf16_bits_to_float(ureg[q][t] & 0xFFFFu);
                    x[8 * q + 2 * t + 1] += bf16_bits_to_float(ureg[q][t] >> 16);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) x[4 * q + t] += __uint_as_float(ureg[q][t]);
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < RUN; ++t) {
            const int v = v0 + t;
            if (erow_ok && v < V) x[t] += load1<U_BF16>(P.U, urow + v);
            else x[t] = -INFINITY;
        }
    }

    // 5) tile-row max and lowest argmax: the lane's run, its partner lane
    //    (l ^ 32 holds the row's other half), then the other token waves.
    float m = x[0];
#pragma unroll
    for (int t = 1; t < RUN; ++t) m = fmaxf(m, x[t]);
    int am = INT_MAX;
#pragma unroll
    for (int t = RUN - 1; t >= 0; --t)
        if (x[t] == m) am = v0 + t;
    {
        const float m2 = __shfl_xor(m, 32);
        const int a2 = __shfl_xor(am, 32);
        merge_arg(m, am, m2, a2);
    }
    if constexpr (NWV > 1) {
        if (h == 0) {
            x_m[wv][rl] = m;
            x_i[wv][rl] = am;
        }
        __syncthreads();
        m = x_m[0][rl];
        am = x_i[0][rl];
#pragma unroll
        for (int w = 1; w < NWV; ++w) merge_arg(m, am, x_m[w][rl], x_i[w][rl]);
    }
    if (am == INT_MAX) am = v_tile;   // all -inf: any in-tile id (weight 0)

    // 6) group sums and the tile sum, relative to the tile-row max.
    float gs[NG];
    float tot = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float sg = 0.0f;
        if (!P.greedy && m != -INFINITY) {
#pragma unroll
            for (int t = 0; t < 8; ++t) sg += __expf((x[8 * g + t] - m) * P.invT);
        }
        gs[g] = sg;
        tot += sg;
    }
    tot += __shfl_xor(tot, 32);
    const int nseg = gridDim.x;
    if (active && !P.greedy) {
        float* gdst = P.gsums + ((size_t)b * nseg + tile) * 16 + run0 / 8;
        if constexpr (NG % 4 == 0) {
#pragma unroll
            for (int q = 0; q < NG / 4; ++q)
                *reinterpret_cast<float4*>(gdst + 4 * q) =
                    make_float4(gs[4 * q], gs[4 * q + 1], gs[4 * q + 2], gs[4 * q + 3]);
        } else {
            *reinterpret_cast<float2*>(gdst) = make_float2(gs[0], gs[1]);
        }
    }
    if constexpr (NWV > 1) {
        if (h == 0) x_s[wv][rl] = tot;
        __syncthreads();
        tot = x_s[0][rl];
#pragma unroll
        for (int w = 1; w < NWV; ++w) tot += x_s[w][rl];
    }
    if (active && h == 0 && wv == 0) {
        SegStat st;
        st.m = m;
        st.s = tot;
        st.idx = am;
        st.pad = 0;
        P.stats[(size_t)b * nseg + tile] = st;
    }
}

// ---------------------------------------------------------------------------
// Streaming q-free bias tile: one persistent workgroup per CU.
//
// Work item = (64-token slice, block of 128 request rows).  Workgroup g takes
// row block g / ws and the j-th contiguous share of that block's slices
// (j = g % ws).  Every item's two inputs are copied into an LDS stage by direct
// global->LDS loads: the packed W2 slice (64 rows of r bf16, contiguous in the
// packed image) and the U slice (128 rows x 64 bf16, 16-byte chunk c of row bl
// stored in slot bl*8 + (c ^ ((bl>>1)&7))).  Three stages: item i+2 streams in
// while item i is contracted and item i-1 reduced.
//
// Eight waves, two per SIMD.  Wave w owns rows 32 (w & 3) .. + 31 and tokens
// 32 (w >> 2) .. + 31 of each item, on 32x32x16 MFMAs: A = W2 slice (tokens x
// rank) from LDS, B = E = W1[x_{k-1}] rows in registers.  MFMA row i = 8g + 4h
// + c is token 16h + p(g, c) of the wave's 32, p(g, c) = 8 (g & 1) + 4 (g >> 1)
// + c, so lane (row, h = lane / 32) ends with tokens 16h .. 16h + 15 of its row
// and the 16-byte operand reads stay conflict-free under the packed swizzle.
// A segment is the wave's 32 tokens of one row: its max and four 8-token group
// sums relative to it; a running merge gives one summary per (row, share).
//
// Only the bf16-U, V % 8 == 0 shape is streamed this way (chunks never straddle
// V); waits on the direct loads use explicit vmcnt counts and a bare s_barrier,
// since a fenced barrier would drain the prefetches as well.
// ---------------------------------------------------------------------------
constexpr int kStreamStages = 3;


template <int NKS, bool GREEDY>   // NKS = r / 16 rank steps of the 32x32x16 MFMA
__global__ __launch_bounds__(kStreamWaves * 64, 1)
void draft_tile_stream(TileParams P, int nitem_v, int nrb, int ws) {
    constexpr int R = NKS * 16;
    constexpr int W2B = kStreamItem * R * 2;             // packed W2 slice bytes
    constexpr int UB = kStreamRows * kStreamItem * 2;    // U slice bytes
    constexpr int STAGE = W2B + UB;
    constexpr int W2P = W2B / 1024 / kStreamWaves;       // 1 KB pieces per wave
    constexpr int UP = UB / 1024 / kStreamWaves;
    constexpr int LOADS = W2P + UP;                      // direct loads per wave per item
    constexpr int NCH = R / 8;
    static_assert(W2P >= 1 && UP == 2, "piece split");
    extern __shared__ __align__(16) char smem_s[];
    const int V = P.V, k = P.k, B = P.B, gamma = P.gamma;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar LDS addresses
    const int h = lane >> 5;
    const int rg = wave & 3;         // row group: rows 32 rg .. + 31 of the row block
    const int th = wave >> 2;        // token half: tokens 32 th .. + 31 of an item
    const int rb0 = (int)blockIdx.x / ws;
    const int jw = (int)blockIdx.x % ws;
    const int lo = (int)((long long)jw * nitem_v / ws);
    const int hi = (int)((long long)(jw + 1) * nitem_v / ws);
    const int my_n = hi - lo;        // >= 1: ws <= nitem_v
    const uint16_t* Ub = static_cast<const uint16_t*>(P.U);
    const size_t bpad = (size_t)nrb * kStreamRows;

    // This lane's U pieces: row bl and 16-byte chunk c of every item's slice,
    // as offsets from the row block's first row.
    size_t ubase[UP];
    int ubl[UP], uc8[UP];
#pragma unroll
    for (int q = 0; q < UP; ++q) {
        const int sl = (q * kStreamWaves + wave) * 64 + lane;
        const int bl = sl >> 3;
        const int c = (sl & 7) ^ ((bl >> 1) & 7);
        ubl[q] = bl;
        uc8[q] = c * 8;
        ubase[q] = ((size_t)bl * gamma + k) * (size_t)V + c * 8;
    }
    const size_t rb_stride = (size_t)kStreamRows * gamma * (size_t)V;

    auto issue = [&](int i) {
        const int iv = lo + i;
        char* st = smem_s + (i % kStreamStages) * STAGE;
        const char* wsrc = reinterpret_cast<const char*>(P.W2T) + (size_t)iv * W2B;
#pragma unroll
        for (int q = 0; q < W2P; ++q) {
            const int pc = q * kStreamWaves + wave;
            __builtin_amdgcn_global_load_lds(wsrc + pc * 1024 + lane * 16,
                                             (lds_ptr_t)(st + pc * 1024), 16, 0, 0);
        }
        const size_t item_off = (size_t)rb0 * rb_stride + (size_t)iv * kStreamItem;
#pragma unroll
        for (int q = 0; q < UP; ++q) {
            const int pc = q * kStreamWaves + wave;
            const bool ok = rb0 * kStreamRows + ubl[q] < B && iv * kStreamItem + uc8[q] < V;
            const size_t off = ok ? ubase[q] + item_off : (size_t)k * (size_t)V;   // any valid chunk
            __builtin_amdgcn_global_load_lds(Ub + off, (lds_ptr_t)(st + W2B + pc * 1024), 16, 0,
                                             kCpolNT);
        }
    };

    // Conditioning rows E = W1[x_{k-1}] of this lane's row (MFMA B operand).
    const int bl = 32 * rg + (lane & 31);
    const int b = rb0 * kStreamRows + bl;
    bool erow_ok = false;
    bf16x8_t e[NKS];
    {
        int prev = 0;
        if (b < B) {
            prev = (k == 0) ? P.x0[b] : P.tokens[(size_t)b * gamma + k - 1];
            erow_ok = prev >= 0 && prev < V;
        }
        const uint16_t* erow = P.W1 + (size_t)(erow_ok ? prev : 0) * R;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (erow_ok) {
                e[ks] = *reinterpret_cast<const bf16x8_t*>(erow + ks * 16 + h * 8);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) e[ks][t] = (__bf16)0.0f;
            }
        }
    }
    // E must be complete before any direct load is in flight: the compiler
    // treats plain and direct loads pending together as unordered and would
    // otherwise drain every prefetch before each contraction.
    wait_vmcnt_le(0);
    issue(0);
    if (my_n > 1) issue(1);

    // A-operand row of this lane: MFMA row i = lane % 32 = 8g + 4h' + c.
    int atok, arow;
    {
        const int i = lane & 31;
        const int g = i >> 3, hh = (i >> 2) & 1, c = i & 3;
        atok = 32 * th + 16 * hh + 8 * (g & 1) + 4 * (g >> 1) + c;
        arow = atok * R;
    }
    // U chunks of the lane's 16 tokens (chunks 4 th + 2 h and + 1 of row bl)
    int uslot[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) uslot[q] = bl * 8 + ((4 * th + 2 * h + q) ^ ((bl >> 1) & 7));
    const float sc = P.invT * 1.4426950408889634f;   // exp(y / T) = 2^(y * sc)

    // Reduction of one finished item for this lane's row: the segment max and
    // the sums of this lane's two 8-token groups relative to it.
    struct Red {
        float m, g0, g1;
        int am;
    };
    auto reduce = [&](const f32x16_t& ac, const u32x4_t (&uf)[2], int iv) -> Red {
        // accumulator idx = 4g + c holds run position 8 (g & 1) + 4 (g >> 1) + c
        float x[16];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int pos = 8 * (g & 1) + 4 * (g >> 1) + c;
                const uint32_t w = uf[pos >> 3][(pos & 7) >> 1];
                const float uv = (pos & 1) ? __uint_as_float(w & 0xFFFF0000u)
                                           : __uint_as_float(w << 16);
                x[pos] = ac[4 * g + c] + uv;
            }
        const int v0 = iv * kStreamItem + 32 * th + 16 * h;
        if (iv * kStreamItem + kStreamItem > V) {   // the last slice: tokens past V
#pragma unroll
            for (int t = 0; t < 16; ++t) x[t] = v0 + t < V ? x[t] : -INFINITY;
        }
        Red o;
        float m = x[0];
#pragma unroll
        for (int t = 1; t < 16; ++t) m = fmaxf(m, x[t]);
        o.am = 0;   // the argmax is only read by greedy decoding
        if constexpr (GREEDY) {
            int am = INT_MAX;
#pragma unroll
            for (int t = 15; t >= 0; --t) am = x[t] == m ? v0 + t : am;
            const float m2 = __shfl_xor(m, 32);
            const int a2 = __shfl_xor(am, 32);
            am = (m2 > m || (m2 == m && a2 < am)) ? a2 : am;
            m = fmaxf(m, m2);
            o.am = am;
            o.g0 = o.g1 = 0.0f;
        } else {
            m = fmaxf(m, __shfl_xor(m, 32));
            const float ms = m == -INFINITY ? 0.0f : m * sc;   // all -inf: every weight 0
            float g0 = 0.0f, g1 = 0.0f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                g0 += __builtin_amdgcn_exp2f(fmaf(x[t], sc, -ms));
                g1 += __builtin_amdgcn_exp2f(fmaf(x[8 + t], sc, -ms));
            }
            o.g0 = g0;
            o.g1 = g1;
        }
        o.m = m;
        return o;
    };
    // Segment-major outputs: the max [seg][bpad] and the four group sums
    // [seg][bpad][4]; one wave's stores for an item are contiguous runs.
    auto store = [&](const Red& o, int iv) {
        const size_t si = (2 * (size_t)iv + th) * bpad + b;
        if constexpr (!GREEDY)
            *reinterpret_cast<float2*>(P.gsums + si * 4 + 2 * h) = make_float2(o.g0, o.g1);
        if (h == 0) P.segm[si] = o.m;
    };

    // Running summary of this wave's half of the share for the lane's row.
    float run_m = -INFINITY, run_s = 0.0f;
    int run_a = INT_MAX;
    auto absorb_run = [&](const Red& o) {
        if constexpr (GREEDY) {
            run_a = (o.m > run_m || (o.m == run_m && o.am < run_a)) ? o.am : run_a;
            run_m = fmaxf(run_m, o.m);
        } else {
            float tot = o.g0 + o.g1;
            tot += __shfl_xor(tot, 32);
            const float nm = fmaxf(run_m, o.m);
            const float a = run_m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((run_m - nm) * sc);
            const float c = o.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((o.m - nm) * sc);
            run_s = run_s * a + tot * c;
            run_m = nm;
        }
    };

    f32x16_t accp;
#pragma unroll
    for (int t = 0; t < 16; ++t) accp[t] = 0.0f;
    u32x4_t ufrp[2] = {u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}};
    int ivp = 0;
    bool have_p = false;   // an item waiting to be reduced
    // Item i-2's outputs are stored at the top of iteration i, before the
    // prefetch: stores count in vmcnt too, and only loads may be newer than
    // the item a wait is for (stores and loads may retire out of order).
    Red redh{};
    int ivh = 0;
    bool have_h = false;
    const bool reduce_first = th != 0;   // the two waves of a SIMD alternate phases
    for (int i = 0; i < my_n; ++i) {
        const int iv = lo + i;
        wait_vmcnt_le(i + 1 < my_n ? LOADS : 0);   // item i's direct loads (this wave)
        asm volatile("s_barrier" ::: "memory");    // ... and every wave's; stage (i-1)%3 is free
        if (have_h && erow_ok) store(redh, ivh);
        if (i + 2 < my_n) issue(i + 2);

        Red red;
        if (reduce_first) red = reduce(accp, ufrp, ivp);

        const char* st = smem_s + (i % kStreamStages) * STAGE;
        const uint16_t* w2s = reinterpret_cast<const uint16_t*>(st);
        const int sw = w2p_swizzle((iv & 1) * 64 + atok, NCH);
        bf16x8_t afr[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            afr[ks] = *reinterpret_cast<const bf16x8_t*>(w2s + arow + (((2 * ks + h) ^ sw) << 3));
        const u32x4_t* us = reinterpret_cast<const u32x4_t*>(st + W2B);
        u32x4_t ufr[2];
        ufr[0] = us[uslot[0]];
        ufr[1] = us[uslot[1]];
        f32x16_t acc;
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[ks], e[ks], acc, 0, 0, 0);
        {   // schedule: LDS reads ahead, then one MFMA per further read
            constexpr int NR = NKS + 2;
            constexpr int kAhead = NR < 8 ? NR : 8;
            __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
            for (int j = 0; j < NR - kAhead; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NKS - (NR - kAhead), 0);
        }
        if (!reduce_first) red = reduce(accp, ufrp, ivp);

        if (have_p) absorb_run(red);
        redh = red;
        ivh = ivp;
        have_h = have_p;
        accp = acc;
        ufrp[0] = ufr[0];
        ufrp[1] = ufr[1];
        ivp = iv;
        have_p = true;
    }
    if (have_h && erow_ok) store(redh, ivh);
    const Red red = reduce(accp, ufrp, ivp);
    if (erow_ok) store(red, ivp);
    absorb_run(red);

    // Share summaries: the token-half-1 waves hand their running summary to
    // the half-0 waves of the same rows, which merge and store them.
    float* xm = reinterpret_cast<float*>(smem_s);   // the stages are idle now
    float* xs = xm + kStreamRows;
    int* xa = reinterpret_cast<int*>(xs + kStreamRows);
    __syncthreads();
    if (th == 1 && h == 0) {
        xm[bl] = run_m;
        xs[bl] = run_s;
        xa[bl] = run_a;
    }
    __syncthreads();
    if (th == 0 && h == 0 && erow_ok) {
        const float m2 = xm[bl], s2 = xs[bl];
        const int a2 = xa[bl];
        SegStat sst;
        if constexpr (GREEDY) {
            float m = run_m;
            int am = run_a;
            merge_arg(m, am, m2, a2);
            sst.m = m;
            sst.s = 0.0f;
            sst.idx = am;
        } else {
            const float nm = fmaxf(run_m, m2);
            const float a = run_m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((run_m - nm) * sc);
            const float c = m2 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m2 - nm) * sc);
            sst.m = nm;
            sst.s = run_s * a + s2 * c;
            sst.idx = 0;
        }
        sst.pad = 0;
        P.sup[(size_t)jw * bpad + b] = sst;
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
// One workgroup (4 waves) per request row.  Thread t owns a contiguous run of
// about nseg/256 segment summaries; the fp64 run weights are scanned in token
// order (wave scans, then the four wave totals), the thread whose run holds
// u * Z walks it to the segment, and wave 0 rescans that segment's logits.
// ---------------------------------------------------------------------------
constexpr int kFinRun = 16;  // max summaries per thread (nseg <= 4096)

// Inputs the q-free draft needs to rebuild 8 logits of one tile row.
struct RebuildArgs {
    const float* gsums;     // group sums relative to the segment max, gps per summary
    int gps;                // 8-token groups per segment
    int row_stride;         // summaries between rows b and b + 1 (stats and gsums)
    int seg_stride;         // summaries between segments j and j + 1 of one row
    const void* U;          // [B, gamma, V]
    int u_bf16;
    const uint16_t* W1;     // [V, r]
    const uint16_t* W2T;    // [V, r]
    int r;
    // RNN head: the conditioning rows [B, gamma, 3, r] (three bf16 terms of
    // o_k) stand in for W1[prev]; null for the Markov head
    const uint16_t* erows;
};

__global__ __launch_bounds__(256)
void draft_finalize(const SegStat* __restrict__ stats, int nseg, int seg_len,
                    const float* __restrict__ q_logits, const int32_t* __restrict__ x0,
                    int32_t* __restrict__ tokens, float* __restrict__ q_logZ,
                    float* __restrict__ q_tok, const float* __restrict__ uniforms,
                    uint64_t seed, uint32_t offset, int B, int gamma, int V, int k, float invT,
                    int greedy, RebuildArgs rb) {
    __shared__ float sh_m[4];
    __shared__ int sh_i[4];
    __shared__ double sh_tot[4];
    __shared__ int sh_seg, sh_owner_last;
    __shared__ double sh_rem;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const size_t outi = (size_t)b * gamma + k;
    (void)B;

    const int prev = (k == 0) ? x0[b] : tokens[outi - 1];
    if (prev < 0 || prev >= V) {
        if (tid == 0) {
            tokens[outi] = -1;
            if (q_logZ) q_logZ[outi] = NAN;
            if (q_tok) q_tok[outi] = NAN;
        }
        return;
    }
    const SegStat* st = stats + (size_t)b * rb.row_stride;   // segment j at st[j * seg_stride]
    const size_t sj = (size_t)rb.seg_stride;
    const int per = (nseg + 255) / 256;
    const int j0 = min(nseg, tid * per);
    const int n = min(nseg, j0 + per) - j0;
    float sm[kFinRun], ss[kFinRun];
    int si[kFinRun];
#pragma unroll
    for (int t = 0; t < kFinRun; ++t) {
        if (t < n) {
            const SegStat x = st[(size_t)(j0 + t) * sj];
            sm[t] = x.m;
            ss[t] = x.s;
            si[t] = x.idx;
        } else {
            sm[t] = -INFINITY;
            ss[t] = 0.0f;
            si[t] = INT_MAX;
        }
    }

    // 1) row max and argmax.
    float M = -INFINITY;
    int AM = INT_MAX;
#pragma unroll
    for (int t = 0; t < kFinRun; ++t) merge_arg(M, AM, sm[t], si[t]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(M, off);
        const int i2 = __shfl_xor(AM, off);
        merge_arg(M, AM, m2, i2);
    }
    if (lane == 0) {
        sh_m[wave] = M;
        sh_i[wave] = AM;
    }
    __syncthreads();
    M = sh_m[0];
    AM = sh_i[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge_arg(M, AM, sh_m[w], sh_i[w]);
    if (greedy || M == -INFINITY) {
        if (tid == 0) {
            tokens[outi] = (M == -INFINITY) ? -1 : AM;
            if (q_logZ) q_logZ[outi] = M == -INFINITY ? NAN : M;
            if (q_tok) q_tok[outi] = M == -INFINITY ? NAN : 1.0f;
        }
        return;
    }

    // 2) run weights (fp64) and their scan in token order.
    double wr[kFinRun];
    double tsum = 0.0;
#pragma unroll
    for (int t = 0; t < kFinRun; ++t) {
        wr[t] = sm[t] != -INFINITY ? (double)ss[t] * (double)expf((sm[t] - M) * invT) : 0.0;
        tsum += wr[t];
    }
    // Neighbouring intervals share exact end points (the previous lane's
    // inclusive value), so [excl, incl) tile [0, Z) without gaps.
    const double incl_w = wave_inclusive_scan_f64(tsum);
    double excl_w = __shfl_up(incl_w, 1);
    if (lane == 0) excl_w = 0.0;
    if (lane == kWave - 1) sh_tot[wave] = incl_w;
    if (tid == 0) {
        sh_seg = -1;
        sh_owner_last = -1;
    }
    __syncthreads();
    double base = 0.0;
    for (int w = 0; w < wave; ++w) base += sh_tot[w];
    double Z = 0.0;
    for (int w = 0; w < 4; ++w) Z += sh_tot[w];
    const double incl = base + incl_w;
    const double excl = base + excl_w;
    const float u = uniforms ? uniforms[outi] : counter_uniform(seed, offset, b, k, 0);
    const double thr = (double)u * Z;

    // 3) the owning thread walks its run.
    if (tsum > 0.0 && thr >= excl && thr < incl) {
        double run = excl;
        int seg = -1, last = -1;
        double rem = 0.0, last_run = 0.0;
#pragma unroll
        for (int t = 0; t < kFinRun; ++t) {
            if (seg < 0 && wr[t] > 0.0) {
                last = j0 + t;
                last_run = run;
                if (thr < run + wr[t]) {
                    seg = j0 + t;
                    rem = thr - run;
                }
            }
            run += wr[t];
        }
        if (seg < 0) {   // rounding: end of the last segment with weight
            seg = last;
            rem = thr - last_run;
        }
        sh_seg = seg;
        sh_rem = rem;
    }
    if (tsum > 0.0) atomicMax(&sh_owner_last, tid);
    __syncthreads();
    if (sh_seg < 0 && tid == sh_owner_last) {
        // thr >= Z after rounding: clamp to the last segment with weight
        int last = -1;
#pragma unroll
        for (int t = 0; t < kFinRun; ++t)
            if (wr[t] > 0.0) last = j0 + t;
        sh_seg = last;
        sh_rem = INFINITY;
    }
    __syncthreads();
    if (wave != 0) return;
    const int seg = max(0, sh_seg);   // a finite row max always gives one segment weight
    const double rem = sh_rem;
    const double Md = (double)M;

    if (q_logits == nullptr) {
        // q-free draft: locate the 8-token group from the tile's group sums,
        // then rebuild that group's logits l = U + e . W2[:, v], e = W1[prev]
        // (Markov) or the three bf16 terms of o_k (RNN).
        const float mseg = st[(size_t)seg * sj].m;
        const double scale = (double)expf((mseg - M) * invT);   // as the tile weight
        const double wg = lane < rb.gps
                              ? (double)rb.gsums[((size_t)b * rb.row_stride + (size_t)seg * sj) *
                                                         rb.gps + lane] * scale
                              : 0.0;
        const double ginc = wave_inclusive_scan_f64(wg);
        double gexc = __shfl_up(ginc, 1);
        if (lane == 0) gexc = 0.0;
        unsigned long long ghit = __ballot(wg > 0.0 && ginc > rem);
        const bool gclamp = ghit == 0;
        if (gclamp) {
            const unsigned long long pos = __ballot(wg > 0.0);
            ghit = pos ? 1ull << (63 - __clzll((long long)pos)) : 1ull;
        }
        const int grp = __ffsll((long long)ghit) - 1;
        const double grem = gclamp ? INFINITY : rem - __shfl(gexc, grp);
        // lane = 8 * t + sl: token t of the group, rank slice sl
        const int t = lane >> 3, sl = lane & 7;
        const int vt = seg * seg_len + grp * 8 + t;
        const int span = rb.r / 8;
        float part = 0.0f;
        const int nterm = rb.erows ? 3 : 1;
        for (int term = 0; term < nterm && vt < V; ++term) {
            const uint16_t* w1 = rb.erows ? rb.erows + (outi * 3 + term) * (size_t)rb.r
                                          : rb.W1 + (size_t)prev * rb.r;
            if ((span & 7) == 0) {   // whole 16-byte chunks: span / 8 <= 4 of them
                const int nswz = w2p_swizzle(vt & (kPackTile - 1), rb.r >> 3);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (q < (span >> 3)) {
                        const int kc = sl * (span >> 3) + q;
                        const uint4 a = *reinterpret_cast<const uint4*>(w1 + kc * 8);
                        const uint4 c = *reinterpret_cast<const uint4*>(
                            rb.W2T + (size_t)vt * rb.r + ((kc ^ nswz) << 3));
                        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
                        const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            part = fmaf(bf16_bits_to_float(aw[t] & 0xFFFFu),
                                        bf16_bits_to_float(cw[t] & 0xFFFFu), part);
                            part = fmaf(bf16_bits_to_float(aw[t] >> 16),
                                        bf16_bits_to_float(cw[t] >> 16), part);
                        }
                    }
                }
            } else {
                for (int j = sl * span; j < (sl + 1) * span; ++j)
                    part = fmaf(bf16_bits_to_float(w1[j]),
                                bf16_bits_to_float(rb.W2T[w2p_index(vt, j, rb.r)]), part);
            }
        }
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 4);
        double wt = 0.0;
        float lt = 0.0f;
        if (vt < V) {
            const size_t uo = outi * (size_t)V + vt;
            lt = (rb.u_bf16 ? bf16_bits_to_float(static_cast<const uint16_t*>(rb.U)[uo])
                            : static_cast<const float*>(rb.U)[uo]) + part;
            wt = exp(((double)lt - Md) * (double)invT);
        }
        // token t's weight and logit live in lane 8t; gather them to lanes 0..7
        const double w8 = __shfl(wt, (lane & 7) * 8);
        const float l8 = __shfl(lt, (lane & 7) * 8);
        const double wl = lane < 8 ? w8 : 0.0;
        const double tinc = wave_inclusive_scan_f64(wl);
        double texc = __shfl_up(tinc, 1);
        if (lane == 0) texc = 0.0;
        unsigned long long thit = __ballot(wl > 0.0 && tinc > grem);
        if (!thit) {
            const unsigned long long pos = __ballot(wl > 0.0);
            thit = pos ? 1ull << (63 - __clzll((long long)pos)) : 1ull;
        }
        const int tsel = __ffsll((long long)thit) - 1;
        const float lsel = __shfl(l8, tsel);
        (void)texc;
        if (lane == 0) {
            tokens[outi] = min(seg * seg_len + grp * 8 + tsel, V - 1);
            if (q_logZ) q_logZ[outi] = (float)(Md * (double)invT + log(Z));
            if (q_tok) q_tok[outi] = (float)(exp(((double)lsel - Md) * (double)invT) / Z);
        }
        return;
    }

    // 4) wave 0 rescans the segment (2 tokens per lane).
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
    const unsigned long long found = __ballot(lsum > 0.0 && inc > rem);
    int pick;
    if (found) {
        const int L0 = __ffsll((long long)found) - 1;
        const int mine = (w0 > 0.0 && rem < exc + w0) ? va : vb;
        pick = __shfl(mine, L0);
    } else {
        const unsigned long long pos = __ballot(lsum > 0.0);
        const int L1 = pos ? 63 - __clzll((long long)pos) : 0;
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

__global__ __launch_bounds__(64)
void draft_finalize_stream(FinStreamArgs A, int k) { finalize_row_stream<false>(A, blockIdx.x, k, threadIdx.x & (kWave - 1)); }

// ---------------------------------------------------------------------------
// RNN head.
// ---------------------------------------------------------------------------

// Hidden part of the pre-activations, split over kHprojSplit ranges of the
// hidden size: part[s][m][n] = sum_{t in range s} h[m][t] * Wcat[n][2r + t],
// m < M = B * gamma, n < 3r, Wcat = [W_g; W_c; W_o] (the gates kernel sums
// the kHprojSplit partials).  One wave per 32 x 32 output block and range,
// operands straight from global memory in 16-byte runs along t, the next
// 64-wide chunk loaded while the current one is multiplied.
__global__ __launch_bounds__(256)
void rnn_hidden_proj(const uint16_t* __restrict__ h, const uint16_t* __restrict__ Wg,
                     const uint16_t* __restrict__ Wc, const uint16_t* __restrict__ Wo,
                     float* __restrict__ part, int M, int r, int d) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m0 = blockIdx.y * 64 + (wave >> 1) * 32;
    const int n0 = blockIdx.x * 64 + (wave & 1) * 32;
    const int sp = blockIdx.z;
    const int ld = 2 * r + d;
    const int kgrp = lane >> 5;
    const int m = m0 + (lane & 31);
    const int n = n0 + (lane & 31);
    const bool mok = m < M;
    const bool nok = n < 3 * r;
    const int span = (d + kHprojSplit * 64 - 1) / (kHprojSplit * 64) * 64;
    const int t_lo = min(d, sp * span), t_hi = min(d, t_lo + span);
    const uint16_t* arow = h + (size_t)(mok ? m : 0) * d + kgrp * 8;
    const uint16_t* wsel = n < r ? Wg : (n < 2 * r ? Wc : Wo);
    const uint16_t* brow = wsel + (size_t)(nok ? n % r : 0) * ld + 2 * r + kgrp * 8;
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    bf16x8_t zero;
#pragma unroll
    for (int t = 0; t < 8; ++t) zero[t] = (__bf16)0.0f;
    bf16x8_t a[2][4], bb[2][4];
    // Branch-free loads: an address outside the operands is clamped to a valid
    // one and the value zeroed after the load.
    auto load = [&](int buf, int t0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = t0 + 16 * u;
            const bool in = t + kgrp * 8 + 8 <= t_hi;   // d % 8 == 0: whole 8-runs only
            const int tc = in ? t : t_lo - kgrp * 8;     // a valid run of this range
            a[buf][u] = *reinterpret_cast<const bf16x8_t*>(arow + tc);
            bb[buf][u] = *reinterpret_cast<const bf16x8_t*>(brow + tc);
            if (!(mok && in)) a[buf][u] = zero;
            if (!(nok && in)) bb[buf][u] = zero;
        }
    };
    auto mul = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[buf][u], bb[buf][u], acc, 0, 0, 0);
    };
    if (t_lo < t_hi) load(0, t_lo);
    for (int t0 = t_lo; t0 < t_hi; t0 += 128) {
        if (t0 + 64 < t_hi) load(1, t0 + 64);
        mul(0);
        if (t0 + 128 < t_hi) load(0, t0 + 128);
        if (t0 + 64 < t_hi) mul(1);
    }
    if (nok) {
        float* out = part + (size_t)sp * M * 3 * r;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int mm = m0 + 8 * (i >> 2) + 4 * kgrp + (i & 3);
            if (mm < M) out[(size_t)mm * 3 * r + n] = acc[i];
        }
    }
}

// Per position k: pre-activations = hidden part (the kHprojSplit partials) +
// W[:, 0:r] s_{k-1} + W[:, r:2r] W1[x_{k-1}] for W = W_g, W_c, W_o; gated
// state update; o split into three bf16 terms (hi, mid, lo) whose sum equals
// o to ~2^-25, stored as the conditioning rows of (b, k) in Erows
// [B, gamma, 3, r].
// One workgroup per 32 requests x 32 features; its four waves split the
// contraction: waves 0 and 1 take halves of the state columns W[:, 0:r] and
// multiply each weight operand by the hi, mid and lo bf16 terms of the fp32
// state (their sum is s to ~2^-25, so the products keep fp32 accuracy);
// waves 2 and 3 take halves of the embedding columns W[:, r:2r].  Every
// weight is loaded once per workgroup, all of a wave's loads go out before
// its first MFMA (32x32x16 bf16), the four partial accumulators meet in LDS,
// and each wave finishes a quarter of the outputs.
__global__ __launch_bounds__(256)
void rnn_gates(const float* __restrict__ hpart, const uint16_t* __restrict__ Wg,
               const uint16_t* __restrict__ Wc, const uint16_t* __restrict__ Wo,
               const uint16_t* __restrict__ W1, const int32_t* __restrict__ x0,
               const int32_t* __restrict__ tokens, const float* __restrict__ s_in,
               float* __restrict__ s_out, uint16_t* __restrict__ Erows, int B, int gamma, int V,
               int r, int d, int k) {
    __shared__ float red[4][3][16][64];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kgrp = lane >> 5;
    const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32;
    const int b = m0 + (lane & 31);
    const int n = n0 + (lane & 31);
    const bool bok = b < B, nok = n < r;
    const int bc = bok ? b : 0;
    const int ld = 2 * r + d;
    const int prev = (k == 0) ? x0[bc] : tokens[(size_t)bc * gamma + k - 1];
    const bool pok = bok && prev >= 0 && prev < V;
    const int pc = pok ? prev : 0;
    bf16x8_t zero;
#pragma unroll
    for (int t = 0; t < 8; ++t) zero[t] = (__bf16)0.0f;
    f32x16_t acc[3];
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[q][i] = 0.0f;
    const uint16_t* wr[3] = {Wg + (size_t)(nok ? n : 0) * ld, Wc + (size_t)(nok ? n : 0) * ld,
                             Wo + (size_t)(nok ? n : 0) * ld};
    // This wave's rank steps (16 columns each) of its half: state half for
    // waves 0-1, embedding half for waves 2-3; at most 8 steps (r <= 256).
    const int nsteps = r / 16;
    const int half = (nsteps + 1) / 2;
    const bool state = w < 2;
    const int s_lo = (w & 1) ? half : 0;
    const int s_n = (w & 1) ? nsteps - half : half;
    // No branches among the loads: addresses are clamped to valid memory and
    // the values zeroed afterwards.
    const char* abase = state ? reinterpret_cast<const char*>(s_in + (size_t)bc * r)
                              : reinterpret_cast<const char*>(W1 + (size_t)pc * r);
    const int astride = state ? 4 : 2;
    const int ahi = state ? 16 : 0;
    const bool azero = state ? (!bok || k == 0) : !pok;
    const int col0 = state ? 0 : r;
    const size_t M = (size_t)B * gamma;
    // wave w finishes accumulator elements 4w .. 4w + 3: requests m0 + 8w +
    // 4 * kgrp + 0..3 of feature n.  Their hidden parts and old states depend
    // on nothing in this kernel, so they are loaded first, together with the
    // operands, instead of one round trip after the contraction.
    const int nc = nok ? n : 0;
    float hpv[4][3][kHprojSplit], sold[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const int m = m0 + 8 * w + 4 * kgrp + ii;
        const size_t row = (size_t)(m < B ? m : 0) * gamma + k;
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
            for (int sp = 0; sp < kHprojSplit; ++sp)
                hpv[ii][q][sp] = hpart[((size_t)sp * M + row) * 3 * r + (size_t)q * r + nc];
        sold[ii] = (k == 0) ? 0.0f : s_in[(size_t)(m < B ? m : 0) * r + nc];
    }
    constexpr int KB = 8;
    uint4 ra[KB][2];
    bf16x8_t bq[KB][3];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        const int ks = min(s_lo + min(j, max(s_n - 1, 0)), nsteps - 1);   // inside the row
        const int t = ks * 16 + kgrp * 8;
        const char* ap = abase + (size_t)t * astride;
        ra[j][0] = *reinterpret_cast<const uint4*>(ap);
        ra[j][1] = *reinterpret_cast<const uint4*>(ap + ahi);
#pragma unroll
        for (int q = 0; q < 3; ++q)
            bq[j][q] = *reinterpret_cast<const bf16x8_t*>(wr[q] + col0 + t);
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        if (j >= s_n) break;
        bf16x8_t bv[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) bv[q] = nok ? bq[j][q] : zero;
        if (state) {
            const uint32_t raw[8] = {ra[j][0].x, ra[j][0].y, ra[j][0].z, ra[j][0].w,
                                     ra[j][1].x, ra[j][1].y, ra[j][1].z, ra[j][1].w};
            bf16x8_t th, tm, tl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float sv = azero ? 0.0f : __uint_as_float(raw[e]);
                const uint32_t hi = float_to_bf16_bits(sv);
                const float r1 = sv - bf16_bits_to_float(hi);
                const uint32_t mid = float_to_bf16_bits(r1);
                const uint32_t lo = float_to_bf16_bits(r1 - bf16_bits_to_float(mid));
                th[e] = __builtin_bit_cast(__bf16, (uint16_t)hi);
                tm[e] = __builtin_bit_cast(__bf16, (uint16_t)mid);
                tl[e] = __builtin_bit_cast(__bf16, (uint16_t)lo);
            }
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(th, bv[q], acc[q], 0, 0, 0);
                acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tm, bv[q], acc[q], 0, 0, 0);
                acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tl, bv[q], acc[q], 0, 0, 0);
            }
        } else {
            bf16x8_t a = __builtin_bit_cast(bf16x8_t, ra[j][0]);
            if (azero) a = zero;
#pragma unroll
            for (int q = 0; q < 3; ++q)
                acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv[q], acc[q], 0, 0, 0);
        }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[w][q][i][lane] = acc[q][i];
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const int i = 4 * w + ii;
        const int m = m0 + 8 * w + 4 * kgrp + ii;
        if (m >= B || !nok) continue;
        const size_t row = (size_t)m * gamma + k;
        float pre[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            float hp = 0.0f;
#pragma unroll
            for (int sp = 0; sp < kHprojSplit; ++sp) hp += hpv[ii][q][sp];
            pre[q] = hp + ((red[0][q][i][lane] + red[1][q][i][lane]) +
                           (red[2][q][i][lane] + red[3][q][i][lane]));
        }
        const float g = 1.0f / (1.0f + expf(-pre[0]));
        const float c = tanhf(pre[1]);
        const float o = tanhf(pre[2]);
        s_out[(size_t)m * r + n] = g * sold[ii] + (1.0f - g) * c;
        const uint32_t hi = float_to_bf16_bits(o);
        const float r1 = o - bf16_bits_to_float(hi);
        const uint32_t mid = float_to_bf16_bits(r1);
        const float r2 = r1 - bf16_bits_to_float(mid);
        const uint32_t lo = float_to_bf16_bits(r2);
        uint16_t* er = Erows + row * 3 * r;
        er[n] = (uint16_t)hi;
        er[r + n] = (uint16_t)mid;
        er[2 * r + n] = (uint16_t)lo;
    }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
static int pick_wb(int B) { return B <= 32 ? 1 : (B <= 64 ? 2 : 4); }

static int cu_count();

// Contiguous shares per row block of the streaming tile: one workgroup per CU
// in all, at most 256 shares, none empty.
int stream_shares(int B, int V) {
    const int nitem_v = (V + kStreamItem - 1) / kStreamItem;
    const int nrb = (B + kStreamRows - 1) / kStreamRows;
    int ws = std::max(1, cu_count() / nrb);
    ws = std::min(ws, kMaxShares);
    return std::min(ws, nitem_v);
}

// The streaming tile serves the q-free Markov draft for bf16 U, V % 8 == 0,
// more than 64 rows and r in {64, 128, 256}; its segments are 64 tokens, and
// its finalize reads at most 64 segments per share.
bool draft_streams(const DraftArgs& a) {
    if (!(a.head == kHeadMarkov && a.w_bf16 && !a.q_logits && a.u_bf16 && (a.V % 8) == 0 &&
          pick_wb(a.B) == 4 && (a.r == 64 || a.r == 128 || a.r == 256)))
        return false;
    const int nitem_v = (a.V + kStreamItem - 1) / kStreamItem;
    const int ws = stream_shares(a.B, a.V);
    return 2 * ((nitem_v + ws - 1) / ws) <= 64;   // 32-token segments per share
}

int draft_segment_len(const DraftArgs& a) { return draft_streams(a) ? kStreamItem : kTileV; }

int draft_num_segments(const DraftArgs& a) {
    const int len = draft_segment_len(a);
    return (a.V + len - 1) / len;
}

int draft_max_segments(int V) { return (V + kStreamItem - 1) / kStreamItem; }

static int cu_count() {
    // per-device cache; concurrent first calls store the same value
    static std::atomic<int> n[64];
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 0 || dev >= 64) dev = 0;
    int c = n[dev].load(std::memory_order_relaxed);
    if (!c) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        n[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

template <int NKS>
static hipError_t launch_stream(const TileParams& p, hipStream_t s) {
    constexpr int STAGE = kStreamItem * NKS * 16 * 2 + kStreamRows * kStreamItem * 2;
    const size_t lds = (size_t)kStreamStages * STAGE;
    // raise the dynamic LDS limit once per process (thread-safe)
    static std::once_flag attr_once;
    std::call_once(attr_once, [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_tile_stream<NKS, false>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_tile_stream<NKS, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        (void)hipGetLastError();
    });
    const int nitem_v = (p.V + kStreamItem - 1) / kStreamItem;
    const int nrb = (p.B + kStreamRows - 1) / kStreamRows;
    const int ws = stream_shares(p.B, p.V);
    const int grid = nrb * ws;
    if (p.greedy)
        hipLaunchKernelGGL((draft_tile_stream<NKS, true>), dim3(grid), dim3(kStreamWaves * 64), lds,
                           s, p, nitem_v, nrb, ws);
    else
        hipLaunchKernelGGL((draft_tile_stream<NKS, false>), dim3(grid), dim3(kStreamWaves * 64), lds,
                           s, p, nitem_v, nrb, ws);
    return hipGetLastError();
}

template <int WB, int MODE, int OUT>
static hipError_t launch_tile(const TileParams& p, bool u_bf16, hipStream_t s) {
    const int nt = (p.V + kTileV - 1) / kTileV;
    dim3 grid(nt, (p.B + 32 * WB - 1) / (32 * WB));
    const size_t lds = std::max((size_t)kTileV * (p.r + kLdsPad) * sizeof(uint16_t),
                                (size_t)32 * WB * kOutLd * sizeof(float));
    // r = 256 needs 66 KB of LDS per workgroup (gfx950 has 160 KB per CU)
    // raise the dynamic LDS limit once per process (thread-safe)
    static std::once_flag attr_once;
    std::call_once(attr_once, [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_tile_mfma<WB, MODE, true, OUT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_tile_mfma<WB, MODE, false, OUT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        (void)hipGetLastError();
    });
    if (u_bf16)
        hipLaunchKernelGGL((draft_tile_mfma<WB, MODE, true, OUT>), grid, dim3(256), lds, s, p);
    else
        hipLaunchKernelGGL((draft_tile_mfma<WB, MODE, false, OUT>), grid, dim3(256), lds, s, p);
    return hipGetLastError();
}

template <int WB>
static hipError_t launch_stats(const TileParams& p, bool u_bf16, hipStream_t s) {
    constexpr int RT = 32 * WB;
    dim3 grid((p.V + kTileV - 1) / kTileV, (p.B + RT - 1) / RT);
    const size_t lds = (size_t)256 * p.r;   // the packed W2 tile
    // raise the dynamic LDS limit once per process (thread-safe)
    static std::once_flag attr_once;
    std::call_once(attr_once, [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_tile_stats<WB, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_tile_stats<WB, false>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
        (void)hipGetLastError();
    });
    if (u_bf16)
        hipLaunchKernelGGL((draft_tile_stats<WB, true>), grid, dim3(256), lds, s, p);
    else
        hipLaunchKernelGGL((draft_tile_stats<WB, false>), grid, dim3(256), lds, s, p);
    return hipGetLastError();
}

template <int MODE, int OUT>
static hipError_t launch_tile_b(const TileParams& p, bool u_bf16, hipStream_t s) {
    const int wb = pick_wb(p.B);
    if (wb == 1) return launch_tile<1, MODE, OUT>(p, u_bf16, s);
    if (wb == 2) return launch_tile<2, MODE, OUT>(p, u_bf16, s);
    return launch_tile<4, MODE, OUT>(p, u_bf16, s);
}

static TileParams tile_params(const DraftArgs& a, int k) {
    TileParams p{};
    p.U = a.U;
    p.W1 = (const uint16_t*)a.W1;
    p.W2T = a.W2T;
    p.Erows = a.Erows;
    p.x0 = a.x0;
    p.tokens = a.tokens;
    p.row_pos = nullptr;
    p.out = a.q_logits;
    p.stats = a.stats;
    p.gsums = a.gsums;
    p.sup = a.sup;
    p.segm = reinterpret_cast<float*>(a.stats);   // the streaming tile's per-segment maxima
    p.B = a.B;
    p.gamma = a.gamma;
    p.V = a.V;
    p.r = a.r;
    p.k = k;
    p.invT = a.invT;
    p.greedy = a.greedy;
    return p;
}

hipError_t w2_pack_launch(const uint16_t* W2, uint16_t* W2P, int r, int V, hipStream_t s) {
    const int vpad = (V + kPackTile - 1) / kPackTile * kPackTile;
    dim3 grid(vpad / 64, (r + 63) / 64);
    hipLaunchKernelGGL(w2_pack, grid, dim3(256), 0, s, W2, W2P, r, V);
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
    const TileParams p = tile_params(a, k);
    if (a.head == kHeadMarkov) {
        if (a.q_logits) return launch_tile_b<kHeadMarkov, kOutQ>(p, a.u_bf16, s);
        if (draft_streams(a)) {
            if (a.r == 256) return launch_stream<16>(p, s);
            if (a.r == 128) return launch_stream<8>(p, s);
            return launch_stream<4>(p, s);
        }
        const int wb = pick_wb(a.B);
        if (wb == 1) return launch_stats<1>(p, a.u_bf16, s);
        if (wb == 2) return launch_stats<2>(p, a.u_bf16, s);
        return launch_stats<4>(p, a.u_bf16, s);
    }
    if (a.q_logits) return launch_tile_b<kHeadRnn, kOutQ>(p, a.u_bf16, s);
    return launch_tile_b<kHeadRnn, kOutStats>(p, a.u_bf16, s);
}

hipError_t residual_rows_launch(const TileParams& p, bool u_bf16, hipStream_t s) {
    if (p.Erows) return launch_tile_b<kHeadRnn, kOutResidual>(p, u_bf16, s);
    return launch_tile_b<kHeadMarkov, kOutResidual>(p, u_bf16, s);
}

hipError_t draft_finalize_launch(const DraftArgs& a, int k, hipStream_t s) {
    if (draft_streams(a)) {
        FinStreamArgs f;
        f.sup = a.sup;
        f.segm = reinterpret_cast<const float*>(a.stats);
        f.gsums = a.gsums;
        f.ws = stream_shares(a.B, a.V);
        f.nunit = (a.V + kStreamItem - 1) / kStreamItem;
        f.seg_mult = kStreamItem / kStreamSeg;
        f.bpad = (a.B + kStreamRows - 1) / kStreamRows * kStreamRows;
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
        f.u_f32 = 0;   // the streaming tile takes bf16 U only
        f.W1 = static_cast<const uint16_t*>(a.W1);
        f.W2P = a.W2T;
        f.r = a.r;
        f.tflag = nullptr;
        f.abort_word = nullptr;
        f.poll_limit = 0;
        hipLaunchKernelGGL(draft_finalize_stream, dim3(a.B), dim3(64), 0, s, f, k);
        return hipGetLastError();
    }
    const int nseg = draft_num_segments(a);
    const int seg = draft_segment_len(a);
    RebuildArgs rb;
    rb.gsums = a.gsums;
    rb.gps = seg / 8;
    if (draft_streams(a)) {   // segment-major summaries [nseg][rows padded to 128]
        rb.row_stride = 1;
        rb.seg_stride = (a.B + kStreamRows - 1) / kStreamRows * kStreamRows;
    } else {                  // row-major [B][nseg]
        rb.row_stride = nseg;
        rb.seg_stride = 1;
    }
    rb.U = a.U;
    rb.u_bf16 = a.u_bf16;
    rb.W1 = (const uint16_t*)a.W1;
    rb.W2T = a.W2T;
    rb.r = a.r;
    rb.erows = a.head == kHeadRnn ? a.Erows : nullptr;
    hipLaunchKernelGGL(draft_finalize, dim3(a.B), dim3(256), 0, s, a.stats, nseg, seg, a.q_logits,
                       a.x0, a.tokens, a.q_logZ, a.q_tok, a.uniforms, a.seed, a.offset, a.B,
                       a.gamma, a.V, k, a.invT, a.greedy, rb);
    return hipGetLastError();
}

hipError_t rnn_hidden_proj_launch(const DraftArgs& a, hipStream_t s) {
    const int M = a.B * a.gamma;
    dim3 grid((3 * a.r + 63) / 64, (M + 63) / 64, kHprojSplit);
    hipLaunchKernelGGL(rnn_hidden_proj, grid, dim3(256), 0, s, (const uint16_t*)a.h,
                       (const uint16_t*)a.Wg, (const uint16_t*)a.Wc, (const uint16_t*)a.Wo,
                       a.hproj, M, a.r, a.d);
    return hipGetLastError();
}

hipError_t rnn_gates_launch(const DraftArgs& a, int k, hipStream_t s) {
    const float* s_in = a.state + (size_t)((k + 1) & 1) * a.B * a.r;
    float* s_out = a.state + (size_t)(k & 1) * a.B * a.r;
    hipLaunchKernelGGL(rnn_gates, dim3((a.r + 31) / 32, (a.B + 31) / 32), dim3(256), 0, s,
                       a.hproj, (const uint16_t*)a.Wg, (const uint16_t*)a.Wc,
                       (const uint16_t*)a.Wo, (const uint16_t*)a.W1, a.x0, a.tokens, s_in, s_out,
                       a.Erows, a.B, a.gamma, a.V, a.r, a.d, k);
    return hipGetLastError();
}

}  // namespace specdec
