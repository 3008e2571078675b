// DSpark confidence head and hardware-aware prefix scheduler (DSpark review,
// §2.1 "Confidence Head" and §2.2 "Hardware-Aware Prefix Scheduler").
//
// confidence_rows: one wave per drafted position (request b, position k).
//   The head reads the backbone hidden state h_k and the Markov embedding of
//   the token before position k, W1[x_{k-1}], and returns
//   c = sigmoid(w_h . h_k + w_e . W1[x_{k-1}]).  HBM-bound on h (d values per
//   position); w is a few KB and stays in L2.
//
// prefix schedule: two launches.
//   1. survival a_{r,j} = c_{r,0} * ... * c_{r,j}: one thread per request,
//      float32 products left to right;
//   2. one key per candidate, ~bits(a): for a in [0, 1] ascending keys mean
//      descending a, ties kept in id order r * gamma + j (lower request,
//      then lower position).  Each request's keys already ascend, so a
//      candidate's rank is its position in its own run plus binary-search
//      counts in every other run; many workgroups rank slices of the
//      candidates and scatter them, sorted, into the workspace;
//   (then one workgroup of 1024 threads:)
//   3. q_t = a_t cut to a multiple of 2^-48 as an integer; inclusive integer
//      prefix sums S_t give tau_t = R + S_t 2^-48 exactly (no dependence on
//      the order of the sums); Theta_t = tau_t * SPS(R + t) in double for every
//      t at once; the admitted count is the last t before the first fall of
//      Theta (ties do not stop the search);
//   4. l_r = number of admitted candidates of request r.
#include <climits>

#include "device_common.hpp"
#include "launch.hpp"

namespace specdec {

// ---------------------------------------------------------------------------
// Confidence head
// ---------------------------------------------------------------------------

constexpr int kConfThreads = 256;

template <bool BF16>
__device__ __forceinline__ float elem_at(const void* base, size_t i) {
    if constexpr (BF16) return bf16_bits_to_float(static_cast<const uint16_t*>(base)[i]);
    else return static_cast<const float*>(base)[i];
}

// Partial dot product of one lane: sum over i = lane*8 + 512 n (+ 0..7) of
// x[i] w[i], with 16-byte loads of x (i % 8 == 0 rows, 16-byte aligned).
template <bool BF16>
__device__ __forceinline__ float lane_dot_vec(const void* x, size_t x0, const float* w, int n,
                                              int lane) {
    float acc = 0.0f;
#pragma unroll 4
    for (int i = lane * 8; i < n; i += kWave * 8) {   // four 16-byte loads in flight per lane
        float v[8];
        if constexpr (BF16) {
            const u32x4_t q = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(x) + x0 + i));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = __uint_as_float(q[j] << 16);
                v[2 * j + 1] = __uint_as_float(q[j] & 0xFFFF0000u);
            }
        } else {
            typedef float f32x4v __attribute__((ext_vector_type(4)));
            const f32x4v* p = reinterpret_cast<const f32x4v*>(static_cast<const float*>(x) + x0 + i);
            const f32x4v a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = a[j];
                v[4 + j] = b[j];
            }
        }
        const float4 wa = *reinterpret_cast<const float4*>(w + i);
        const float4 wb = *reinterpret_cast<const float4*>(w + i + 4);
        acc += v[0] * wa.x + v[1] * wa.y + v[2] * wa.z + v[3] * wa.w;
        acc += v[4] * wb.x + v[5] * wb.y + v[6] * wb.z + v[7] * wb.w;
    }
    return acc;
}

template <bool BF16>
__device__ __forceinline__ float lane_dot_any(const void* x, size_t x0, const float* w, int n,
                                              int lane) {
    float acc = 0.0f;
    for (int i = lane; i < n; i += kWave) acc += elem_at<BF16>(x, x0 + i) * w[i];
    return acc;
}

template <bool HB, bool WB, bool VEC>
__global__ __launch_bounds__(kConfThreads)
void confidence_rows(ConfArgs A) {
    const int lane = threadIdx.x & 63;
    const size_t row = (size_t)blockIdx.x * (kConfThreads / kWave) + (threadIdx.x >> 6);
    const size_t nrows = (size_t)A.R * A.gamma;
    if (row >= nrows) return;
    const int b = (int)(row / (unsigned)A.gamma), k = (int)(row % (unsigned)A.gamma);
    const int prev = k == 0 ? A.x0[b] : A.draft[(size_t)b * A.gamma + k - 1];
    if (prev < 0 || prev >= A.V) {   // no token before this position (undrawn)
        if (lane == 0) A.c[row] = 0.0f;
        return;
    }
    float acc;
    if constexpr (VEC) {
        acc = lane_dot_vec<HB>(A.h, row * (size_t)A.d, A.w, A.d, lane) +
              lane_dot_vec<WB>(A.W1, (size_t)prev * A.r, A.w + A.d, A.r, lane);
    } else {
        acc = lane_dot_any<HB>(A.h, row * (size_t)A.d, A.w, A.d, lane) +
              lane_dot_any<WB>(A.W1, (size_t)prev * A.r, A.w + A.d, A.r, lane);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) A.c[row] = 1.0f / (1.0f + expf(-acc));
}

template <bool HB, bool WB>
static void launch_conf_t(const ConfArgs& a, bool vec, hipStream_t s) {
    const size_t rows = (size_t)a.R * a.gamma;
    const unsigned grid = (unsigned)((rows + kConfThreads / kWave - 1) / (kConfThreads / kWave));
    if (vec) hipLaunchKernelGGL((confidence_rows<HB, WB, true>), dim3(grid), dim3(kConfThreads), 0, s, a);
    else hipLaunchKernelGGL((confidence_rows<HB, WB, false>), dim3(grid), dim3(kConfThreads), 0, s, a);
}

hipError_t confidence_launch(const ConfArgs& a, hipStream_t s) {
    if ((size_t)a.R * a.gamma == 0) return hipSuccess;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    // 16-byte vectors: both row lengths multiples of 8 and every base aligned
    const bool vec = a.d % 8 == 0 && a.r % 8 == 0 && al16(a.h) && al16(a.W1) && al16(a.w) &&
                     al16(a.w + a.d);
    if (a.h_bf16 && a.w_bf16) launch_conf_t<true, true>(a, vec, s);
    else if (a.h_bf16) launch_conf_t<true, false>(a, vec, s);
    else if (a.w_bf16) launch_conf_t<false, true>(a, vec, s);
    else launch_conf_t<false, false>(a, vec, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prefix scheduler
// ---------------------------------------------------------------------------

constexpr int kSchedThreads = 1024;
constexpr double kTwo48 = 281474976710656.0;

__device__ __forceinline__ int64_t shfl_up_i64(int64_t x, int d) {
    const int lo = __shfl_up((int)(uint32_t)(uint64_t)x, d);
    const int hi = __shfl_up((int)(uint32_t)((uint64_t)x >> 32), d);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Theta_t for the integer prefix S_t of t admitted candidates, given
// SPS(R + t) (0 past the end of the table).
__device__ __forceinline__ double sched_theta(int R, int64_t S, double sps_B) {
    const double tau = (double)((int64_t)R * (int64_t)kTwo48 + S) / kTwo48;
    return tau * sps_B;
}

// Survival keys of every candidate in LDS: one thread per request forms the
// float32 products left to right from the staged confidences (clamped into
// [0, 1], NaN to 0, so that every request's keys ascend).
__device__ __forceinline__ void survival_keys(const float* c, int R, int G, float* cl,
                                              uint32_t* val, int tid, int nthreads) {
    const int N = R * G;
#pragma unroll 8
    for (int i = tid; i < N; i += nthreads) cl[i] = fminf(fmaxf(c[i], 0.0f), 1.0f);
    __syncthreads();
    for (int r = tid; r < R; r += nthreads) {
        float a = 1.0f;
        for (int j = 0; j < G; ++j) {
            a = a * cl[r * G + j];
            const uint32_t bits = a > 0.0f ? __float_as_uint(a) : 0u;   // -0 keys as +0
            val[r * G + j] = ~bits;
        }
    }
    __syncthreads();
}

// Keys of the ascending run val[lo, lo + n) below x (or at or below x when
// le): a branch-free binary search, top = the highest power of two <= n.
__device__ __forceinline__ int run_count(const uint32_t* val, int lo, int n, int top, uint32_t x,
                                         bool le) {
    int pos = 0;
    for (int b = top; b > 0; b >>= 1) {
        const int probe = pos + b;
        if (probe <= n) {
            const uint32_t y = val[lo + probe - 1];
            if (y < x || (le && y == x)) pos = probe;
        }
    }
    return pos;
}

// 1-2. The rank of each candidate in the order (key ascending, then id): its
// position j in its own request's run, plus, over the other requests, the
// keys at or below its key (earlier requests) or below it (later ones).
// The searches total R * gamma * R * log2(gamma) steps, so they are spread
// wide: every workgroup forms all keys (cheap, and redundant by design), then
// its 256 threads rank 16 candidates, 16 threads per candidate splitting the
// requests.  The candidates land sorted in the workspace.
constexpr int kRankThreads = 256;
constexpr int kRankSplit = 16;
constexpr int kRankPerWg = kRankThreads / kRankSplit;

__global__ __launch_bounds__(kRankThreads)
void schedule_rank_kernel(SchedArgs A) {
    __shared__ uint32_t val[kSchedMax];
    __shared__ float cl[kSchedMax];
    const int tid = threadIdx.x;
    const int R = A.R, G = A.gamma, N = R * G;
    survival_keys(A.c, R, G, cl, val, tid, kRankThreads);
    const int cand = blockIdx.x * kRankPerWg + tid / kRankSplit, sub = tid % kRankSplit;
    int cnt = 0;
    uint32_t x = 0;
    if (cand < N) {
        x = val[cand];
        const int rc = cand / G;
        const int top = 1 << (31 - __builtin_clz(G));
#pragma unroll 2
        for (int r = sub; r < R; r += kRankSplit)
            if (r != rc) cnt += run_count(val, r * G, G, top, x, r < rc);
        if (sub == 0) cnt += cand - rc * G;   // j: the earlier positions of its own request
    }
#pragma unroll
    for (int off = 1; off < kRankSplit; off <<= 1) cnt += __shfl_xor(cnt, off);
    if (cand < N && sub == 0) {
        A.ws_val[cnt] = x;
        A.ws_id[cnt] = cand;
    }
}

// 3-4. One workgroup over the sorted candidates: thread t owns sorted
// positions t E .. t E + E - 1.
template <int E>
__global__ __launch_bounds__(kSchedThreads)
void schedule_scan_kernel(SchedArgs A) {
    __shared__ int cnt_r[kSchedMax];        // per-request admitted counts
    __shared__ int64_t wave_tot[kSchedThreads / kWave];
    __shared__ int stop_t;
    __shared__ int64_t S_stop;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = A.R, G = A.gamma, N = R * G;
    const int base = tid * E;
    double sp[E + 1];
#pragma unroll
    for (int e = 0; e <= E; ++e) {
        const int Bt = R + base + e;
        sp[e] = (base + e <= N && Bt < A.nsps) ? A.sps[Bt] : 0.0;
    }
    uint32_t kv[E];
    int kid[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        kv[e] = base + e < N ? A.ws_val[base + e] : ~0u;
        kid[e] = base + e < N ? A.ws_id[base + e] : 0;
    }
    for (int r = tid; r < R; r += kSchedThreads) cnt_r[r] = 0;
    if (tid == 0) stop_t = INT_MAX;

    // 3. integer prefix sums of the cut survival values over the sorted order
    int64_t q[E];
    int64_t mine = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        q[e] = 0;
        if (base + e < N) {
            const float a = __uint_as_float(~kv[e]);
            q[e] = (int64_t)((double)a * kTwo48);
            mine += q[e];
        }
    }
    // block-wide exclusive scan of the per-thread totals
    int64_t incl = mine;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int64_t o = shfl_up_i64(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int64_t excl = incl - mine;
#pragma unroll
    for (int w = 0; w < kSchedThreads / kWave; ++w)
        if (w < wave) excl += wave_tot[w];

    // first fall of Theta: the smallest t >= 1 with Theta_t < Theta_{t-1}
    if (base < N) {
        int64_t S = excl;
        double prev = sched_theta(R, S, sp[0]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (base + e < N) {
                S += q[e];
                const int t = base + e + 1;
                const double th = sched_theta(R, S, sp[e + 1]);
                if (th < prev) {
                    atomicMin(&stop_t, t);
                    break;
                }
                prev = th;
            }
        }
    }
    __syncthreads();
    const int admitted = stop_t == INT_MAX ? N : stop_t - 1;
    // S at the admitted count: owned by the thread whose range ends it
    {
        int64_t S = excl;
        if (admitted == 0 && tid == 0) S_stop = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (base + e < N) {
                S += q[e];
                if (base + e + 1 == admitted) S_stop = S;
            }
        }
    }
    // 4. per-request counts of the admitted candidates
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (base + e < admitted) atomicAdd(&cnt_r[min(kid[e] / G, R - 1)], 1);
    __syncthreads();
    for (int r = tid; r < R; r += kSchedThreads) A.lens[r] = cnt_r[r];
    if (tid == 0) {
        if (A.B_out) A.B_out[0] = R + admitted;
        if (A.tau_out) A.tau_out[0] = (double)((int64_t)R * (int64_t)kTwo48 + S_stop) / kTwo48;
    }
}

size_t prefix_schedule_ws_bytes(int R, int gamma) {
    const size_t n = (size_t)R * gamma;
    return 2 * ((n * 4 + 255) / 256 * 256);
}

hipError_t prefix_schedule_launch(const SchedArgs& a, hipStream_t s) {
    const int N = a.R * a.gamma;
    if (N > 0)
        hipLaunchKernelGGL(schedule_rank_kernel, dim3((N + kRankPerWg - 1) / kRankPerWg),
                           dim3(kRankThreads), 0, s, a);
    const dim3 g(1), b(kSchedThreads);
    if (N <= kSchedThreads) hipLaunchKernelGGL(schedule_scan_kernel<1>, g, b, 0, s, a);
    else if (N <= 2 * kSchedThreads) hipLaunchKernelGGL(schedule_scan_kernel<2>, g, b, 0, s, a);
    else if (N <= 4 * kSchedThreads) hipLaunchKernelGGL(schedule_scan_kernel<4>, g, b, 0, s, a);
    else hipLaunchKernelGGL(schedule_scan_kernel<8>, g, b, 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tree drafts: the n nodes of highest survival ("Speculative Decoding Part 1",
// section "γ 재배분: 체인 대신 트리")
// ---------------------------------------------------------------------------
//
// One workgroup per tree of M <= 4096 candidate nodes listed parents first.
//   1. survival a_v = c_v * a_parent (root 1, float32) and depth, level by
//      level: in round t a node whose parent was finished in an earlier round
//      takes its value and is stamped t, so no node reads a value written in
//      the same round;
//   2. key (~bits(a) << 32) | (depth << 16) | v: ascending keys are higher
//      survival first, then shallower, then lower id; bitonic sort (one key
//      per thread, shuffles within a wave, for up to 1024 nodes; in LDS for
//      larger trees);
//   3. the first n ids out (-1 past M) and the exact sum of their survival
//      cut to multiples of 2^-48.

constexpr int kTreeThreads = 1024;

// The tree's score: every thread's part (a_v cut to multiples of 2^-48, as
// integers) summed exactly over the workgroup.
__device__ __forceinline__ void tree_score(const TreeArgs& A, size_t t, int64_t sum, int64_t* part) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const int lo = __shfl_xor((int)(uint32_t)(uint64_t)sum, off);
        const int hi = __shfl_xor((int)(uint32_t)((uint64_t)sum >> 32), off);
        sum += (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    }
    if (lane == 0) part[wave] = sum;
    __syncthreads();
    if (threadIdx.x == 0 && A.score) {
        int64_t tot = 0;
        for (int w = 0; w < kTreeThreads / kWave; ++w) tot += part[w];
        A.score[t] = (double)tot / kTwo48;
    }
}

__global__ __launch_bounds__(kTreeThreads)
void tree_select_kernel(TreeArgs A) {
    __shared__ uint64_t keys[kTreeMax];   // first: parent ids and confidences
    __shared__ float av[kTreeMax];
    __shared__ int stamp[kTreeMax];       // round in which the node was finished (0: not yet)
    __shared__ int depth[kTreeMax];
    __shared__ int flag_bad;
    __shared__ int64_t part[kTreeThreads / kWave];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = A.M, n = A.n;
    const size_t t = blockIdx.x;
    int* par = reinterpret_cast<int*>(keys);
    float* cc = reinterpret_cast<float*>(keys) + kTreeMax;
    if (tid == 0) flag_bad = 0;
    __syncthreads();
    for (int v = tid; v < M; v += kTreeThreads) {
        const int p = A.parent[t * M + v];
        if (p < -1 || p >= v) flag_bad = 1;
        par[v] = p;
        cc[v] = fminf(fmaxf(A.c[t * M + v], 0.0f), 1.0f);   // NaN to 0
        stamp[v] = 0;
    }
    __syncthreads();
    if (flag_bad) {
        for (int i = tid; i < n; i += kTreeThreads) A.sel[t * n + i] = -1;
        if (tid == 0 && A.score) A.score[t] = NAN;
        return;
    }

    // 1. survival and depth, one level per round
    for (int round = 1;; ++round) {
        int left = 0;
        for (int v = tid; v < M; v += kTreeThreads) {
            if (stamp[v] != 0) continue;
            const int p = par[v];
            if (p < 0) {
                av[v] = cc[v];
                depth[v] = 1;
                stamp[v] = round;
            } else {
                const int sp = stamp[p];
                if (sp != 0 && sp < round) {
                    av[v] = av[p] * cc[v];
                    depth[v] = depth[p] + 1;
                    stamp[v] = round;
                } else {
                    left = 1;
                }
            }
        }
        if (!__syncthreads_or(left)) break;   // also the barrier between rounds
    }

    // 2. keys and the sort (parents and confidences are no longer needed)
    auto key_of = [&](int v) -> uint64_t {
        if (v >= M) return ~0ull;   // past the tree: after every node
        const uint32_t bits = av[v] > 0.0f ? __float_as_uint(av[v]) : 0u;   // -0 keys as +0
        return ((uint64_t)(~bits) << 32) | ((uint32_t)depth[v] << 16) | (uint32_t)v;
    };
    if (M <= kTreeThreads) {
        // One key per thread, a bitonic sort of kTreeThreads keys: a compare
        // step whose partner is in the same wave (distance j < 64) is a
        // shuffle; only the steps with j >= 64 go through LDS, into one of two
        // buffers in turn, so one barrier per such step keeps the reads of a
        // buffer ahead of its next write.
        uint64_t key = key_of(tid);
        uint64_t* xb = keys;   // [2][kTreeThreads], over the parents and confidences
        int nb = 0;
        for (int k = 2; k <= kTreeThreads; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                uint64_t other;
                if (j >= kWave) {
                    uint64_t* buf = xb + nb * kTreeThreads;
                    nb ^= 1;
                    buf[tid] = key;
                    __syncthreads();
                    other = buf[tid ^ j];
                } else {
                    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)key, j);
                    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(key >> 32), j);
                    other = ((uint64_t)hi << 32) | lo;
                }
                // ascending runs where bit k of the index is clear; the lower
                // index of a pair keeps the smaller key there, the larger one
                // in the descending runs
                const bool up = (tid & k) == 0, lower = (tid & j) == 0;
                const uint64_t mn = key < other ? key : other, mx = key < other ? other : key;
                key = (lower == up) ? mn : mx;
            }
        }
        // 3. the first n nodes (thread i holds the i-th key) and their summed survival
        int64_t sum = 0;
        for (int i = tid; i < n; i += kTreeThreads) {
            int v = -1;
            if (i < M) {
                v = (int)(key & 0xFFFFu);
                sum += (int64_t)((double)av[v] * kTwo48);
            }
            A.sel[t * n + i] = v;
        }
        tree_score(A, t, sum, part);
        return;
    }
    int P = 1;
    while (P < M) P <<= 1;
    for (int v = tid; v < P; v += kTreeThreads) keys[v] = key_of(v);
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < (P >> 1); i += kTreeThreads) {
                const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
                const int hi = lo | j;
                const uint64_t x = keys[lo], y = keys[hi];
                if ((x > y) == ((lo & k) == 0)) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }

    // 3. the first n nodes and their summed survival
    int64_t sum = 0;
    for (int i = tid; i < n; i += kTreeThreads) {
        int v = -1;
        if (i < M) {
            v = (int)(keys[i] & 0xFFFFu);
            sum += (int64_t)((double)av[v] * kTwo48);
        }
        A.sel[t * n + i] = v;
    }
    tree_score(A, t, sum, part);
}

hipError_t tree_select_launch(const TreeArgs& a, hipStream_t s) {
    if (a.R == 0) return hipSuccess;
    hipLaunchKernelGGL(tree_select_kernel, dim3(a.R), dim3(kTreeThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace specdec
