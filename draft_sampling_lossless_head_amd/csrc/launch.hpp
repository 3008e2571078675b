// Internal interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specdec {

struct SegStat;

enum { kHeadMarkov = 0, kHeadRnn = 1 };

// Packed W2 image (bf16).  W2 [r, V] is stored token-major in tiles of 128
// tokens: tile t holds tokens 128t .. 128t + 127 (zeros past V), token v as r
// contiguous bf16 split into r / 8 chunks of 16 bytes, and chunk kc of token
// v sits in slot kc ^ w2p_swizzle(v % 128, r / 8) of its row.  A tile is one
// contiguous block of 256 * r bytes that a workgroup copies into LDS as is.
// The XOR swizzle makes the 16-byte operand reads of a 16x16x32 MFMA block
// conflict-free: 16 lanes read tokens 16a + 4m + c (a, c = 0..3, block m
// fixed) at one chunk, and s = c | ((a ^ m) << 2) gives 16 distinct slots.
constexpr int kPackTile = 128;

__host__ __device__ inline int w2p_swizzle(int vl, int nchunk) {
    const int f = (vl & 3) | ((((vl >> 4) ^ (vl >> 2)) & 3) << 2);
    int F = nchunk & -nchunk;           // largest power of two dividing nchunk
    if (F > 16) F = 16;
    return f & (F - 1);
}

// bf16 element offset of W2[j][v] in the packed image.
__host__ __device__ inline size_t w2p_index(int v, int j, int r) {
    const int slot = (j >> 3) ^ w2p_swizzle(v & (kPackTile - 1), r >> 3);
    return (size_t)v * r + (size_t)slot * 8 + (j & 7);
}

// Streaming bias tiles (q-free draft and residual): a work item is a 64-token
// slice x 128 request rows; one wave covers 32 tokens x 32 rows of it, and a
// segment is those 32 tokens of one row.  Workgroups take contiguous shares of
// a row block's slices, at most kMaxShares per row.
constexpr int kStreamItem = 64;
constexpr int kStreamSeg = 32;
constexpr int kStreamRows = 128;
constexpr int kStreamWaves = 8;
constexpr int kMaxShares = 256;
constexpr int kCpolNT = 2;          // cache-policy bit "nt": streamed once, do not keep
int stream_shares(int B, int V);

inline size_t w2p_bytes(int r, int V) {
    return (size_t)((V + kPackTile - 1) / kPackTile) * kPackTile * (size_t)r * 2;
}

// Everything one draft call needs, resolved and validated by the C ABI layer.
struct DraftArgs {
    int head;            // kHeadMarkov or kHeadRnn
    const void* U;       // [B, gamma, V]
    int u_bf16;
    const int32_t* x0;   // [B]
    const void* W1;      // [V, r]
    const void* W2;      // [r, V]
    int w_bf16;
    const void* h;       // RNN: [B, gamma, d] bf16
    const void* Wg;      // RNN: [r, 2r + d] bf16
    const void* Wc;
    const void* Wo;
    int B, gamma, V, r, d;
    float invT;          // 1 / T (1 when greedy)
    int greedy;
    const float* uniforms;
    uint64_t seed;
    uint32_t offset;
    int32_t* tokens;     // [B, gamma]
    float* q_logits;     // [B, gamma, V]
    float* q_logZ;       // [B, gamma] or null
    float* q_tok;        // [B, gamma] or null
    // workspace carve-outs
    SegStat* stats;      // [B, nseg]
    float* hproj;        // RNN: [B * gamma, 3r]
    float* state;        // RNN: [2, B, r]
    uint16_t* Erows;     // RNN: [B, gamma, 3, r] conditioning rows of every position
    const uint16_t* W2T; // bf16 weights: packed W2 image
    uint16_t* W2T_ws;    // workspace for that image when the caller passes none
    float* gsums;        // q-free draft: [B, nseg, 16] 8-token group sums
    SegStat* sup;        // streaming q-free draft: [shares][rows] range summaries
    unsigned* bar;       // persistent draft: grid-barrier words (kPersistBarBytes)
    uint64_t* tflag;     // persistent draft: per-row token words [B]
};

// Output modes of the bias tile kernel.
enum {
    kOutQ = 0,        // draft: store q logits + tile summaries
    kOutStats = 1,    // q-free draft: tile summaries + 8-token group sums only
    kOutResidual = 2  // verify: logits of row b at its own position, into [B, V]
};

// Arguments of one bias-tile launch.
struct TileParams {
    const void* U;            // [B, gamma, V]
    const uint16_t* W1;       // [V, r]
    const uint16_t* W2T;      // packed W2 image
    const uint16_t* Erows;    // RNN: [B, gamma, 3, r]; residual rows: non-null selects the RNN head
    const int32_t* x0;        // [B]
    const int32_t* tokens;    // [B, gamma] conditioning tokens (draft outputs)
    const int32_t* row_pos;   // kOutResidual: position per row (-1: inactive)
    float* out;               // kOutQ: [B, gamma, V]; kOutResidual: [B, V]
    SegStat* stats;           // [B, nseg]
    float* gsums;             // [B, nseg, 16]
    SegStat* sup;             // streaming tile: per (workgroup share, row) summaries
    float* segm;              // streaming tile: per (32-token segment, row) max
    int B, gamma, V, r, k;
    float invT;
    int greedy;
};

// Segment = the token range one (row, tile) summary covers: 128 tokens, or 64
// for the streaming q-free tile.  Workspace is sized for the larger count.
int draft_num_segments(const DraftArgs& a);
int draft_segment_len(const DraftArgs& a);
int draft_max_segments(int V);
hipError_t draft_tile_launch(const DraftArgs& a, int k, hipStream_t s);
hipError_t draft_finalize_launch(const DraftArgs& a, int k, hipStream_t s);
constexpr size_t kPersistBarBytes = 2048;   // abort word and the -inf chunk (room to spare)
// Persistent q-free Markov draft.  mode: the engine setting read once per call
// (0 per-position, 1 persistent with a plain launch, 2 persistent with a
// cooperative launch).
bool draft_persists(const DraftArgs& a, int mode);
hipError_t draft_persist_launch(const DraftArgs& a, unsigned* bar, int mode, hipStream_t s);
// Clears the persistent draft's abort word (a call that runs another engine
// leaves it at 0, so spec_draft_status reads "complete").
hipError_t persist_clear_abort(unsigned* bar, hipStream_t s);
int persist_set_mode(int mode);
int persist_mode();
unsigned persist_set_poll_limit(unsigned polls);   // 0: the default
unsigned persist_poll_limit();                     // also the split tree walk's wait limit
// W2 [r, V] bf16 -> packed image of w2p_bytes(r, V) bytes.
hipError_t w2_pack_launch(const uint16_t* W2, uint16_t* W2P, int r, int V, hipStream_t s);
// Recompute the logits of row b at position row_pos[b] into out [B, V] with the
// materialised draft's tile kernel (draft_tile_mfma in residual mode).  They
// equal the logits a q-free draft engine sampled from to fp32 rounding (the
// engines sum the contraction in other orders).
hipError_t residual_rows_launch(const TileParams& p, bool u_bf16, hipStream_t s);
// Ranges of the hidden size the RNN head's hidden projection is split over
// (the gates kernel sums the partials).
constexpr int kHprojSplit = 8;
hipError_t rnn_hidden_proj_launch(const DraftArgs& a, hipStream_t s);
hipError_t rnn_gates_launch(const DraftArgs& a, int k, hipStream_t s);

// Per (request, row slot, segment) summary written by the verify streaming
// pass; s is 0 for greedy rows.
struct alignas(16) RowStat {
    float m;        // max logit of the row
    float s;        // sum exp((l - m) / T)
    int idx;        // argmax, lowest id on ties
    float gathered; // logit at the draft token of that position (or 0)
};

// Per-request decision carried from the decide pass to the final draw.
struct alignas(16) FinalInfo {
    double logZp;   // normaliser of the target row used by the final draw
    double logZq;   // normaliser of the draft row (residual mode)
    int n;          // accepted count, or -1 for an invalid request
    int mode;       // 0 none (greedy or invalid), 1 residual, 2 bonus
    int prev;       // draft token x_{n-1} that conditions q_n (n >= 1), else -1
    int pad1;
};

struct VerifyArgs {
    const void* P;
    int p_bf16;
    const void* Q;
    int q_bf16;
    const int32_t* draft;       // [B, gamma_max]
    const int32_t* lens;        // [B] or null
    const int64_t* p_row_off;   // [B] or null
    const int64_t* q_row_off;   // [B] or null
    int B, gamma_max, V;
    float invT;
    int greedy;
    const float* uniforms;      // [B, gamma_max + 1] or null
    uint64_t seed;
    uint32_t offset;
    int32_t* accepted;
    int32_t* out_tokens;
    float* p_logZ;
    float* q_logZ;
    float* accept_prob;
    // q-free verification (the draft's own q(x_k) and log Z_k; no q rows)
    const float* qprob;         // [B, gamma_max] or null
    const float* qlogz;         // [B, gamma_max] or null
    int32_t* row_pos;           // [B] rejected position per request (-1 none)
    int q_single_row;           // Q holds one row per request (row b)
    // workspace carve-outs
    RowStat* rows;              // [B, 2 * gamma_max + 1, row_segs]
    int row_segs;               // segments per row (verify_row_segs)
    FinalInfo* fin;             // [B]
    double* chunk_sums;         // [B, nchunk]
};

// Final draw of q-free verification, streamed (residual_kernels.hip).
struct ResidArgs {
    const uint16_t* P;          // bf16 target rows: dense [B, G + 1, V] or packed
    const int64_t* p_row_off;   // [B] first target row of each request, or null
    const uint16_t* U;          // bf16 [B, G, V] draft base logits (G > 0)
    const uint16_t* W1;         // [V, r]
    const uint16_t* W2P;        // packed W2 image
    const int32_t* x0;          // [B]
    const int32_t* draft;       // [B, G]
    const FinalInfo* fin;       // [B] decisions of verify_decide
    float* gsums;               // [2 nitem][bpad][4] weight sums per 8-token group
    float* sup;                 // [ws][bpad] weight sums per (share, row)
    int32_t* out_tokens;        // [B, G + 1]
    const float* uniforms;      // [B, G + 1] or null
    uint64_t seed;
    uint32_t offset;
    int B, G, V, r;
    float invT;
};

// bf16 P and U, V % 8 == 0, r in {64, 128, 256}, at most 64 segments per share.
bool resid_streams(int B, int V, int r);
hipError_t verify_resid_launch(const ResidArgs& A, hipStream_t s);

int verify_num_chunks(int V);
int verify_row_segs(int B, int gamma_max, int V);
hipError_t verify_launch(const VerifyArgs& a, hipStream_t s);
// The three phases, for callers that insert work between them.
hipError_t verify_rows_decide_launch(const VerifyArgs& a, hipStream_t s);
hipError_t verify_final_launch(const VerifyArgs& a, hipStream_t s);

// Acceptance rate and total variation per drafted position (alpha_kernels.hip).
struct AlphaArgs {
    const void* P;              // target rows: dense [B, G + 1, V] or packed
    int p_bf16;
    const void* Q;              // draft rows: dense [B, G, V] or packed
    int q_bf16;
    const int32_t* lens;        // [B] or null (every request has G positions)
    const int64_t* p_row_off;   // [B] or null
    const int64_t* q_row_off;   // [B] or null
    int B, gamma_max, V;
    float invT;                 // 1 / T (1 when greedy)
    int greedy;
    float* alpha;               // [B, G]
    float* tv;                  // [B, G] or null
};
hipError_t acceptance_rate_launch(const AlphaArgs& a, hipStream_t s);

// Confidence head: c[b, k] = sigmoid(w[:d] . h[b, k] + w[d:] . W1[prev]).
struct ConfArgs {
    const void* h;              // [R, gamma, d] hidden states
    int h_bf16;
    int d;
    const int32_t* x0;          // [R] anchors
    const int32_t* draft;       // [R, gamma] drafted tokens
    const void* W1;             // [V, r] Markov embedding
    int w_bf16;
    int r;
    const float* w;             // [d + r] head weights
    int R, gamma, V;
    float* c;                   // [R, gamma] out
};
hipError_t confidence_launch(const ConfArgs& a, hipStream_t s);

// Prefix scheduler over R * gamma <= kSchedMax candidates.
constexpr int kSchedMax = 8192;
struct SchedArgs {
    const float* c;             // [R, gamma] confidences in [0, 1]
    int R, gamma;
    const double* sps;          // [nsps] steps per second by batch size
    int nsps;
    int32_t* lens;              // [R] out
    int32_t* B_out;             // [1] out or null
    double* tau_out;            // [1] out or null
    uint32_t* ws_val;           // [R * gamma] workspace: keys in sorted order
    int32_t* ws_id;             // [R * gamma] workspace: their candidate ids
};
size_t prefix_schedule_ws_bytes(int R, int gamma);
hipError_t prefix_schedule_launch(const SchedArgs& a, hipStream_t s);

// Top-n nodes of R draft trees of M <= kTreeMax nodes each.
constexpr int kTreeMax = 4096;
struct TreeArgs {
    const int32_t* parent;      // [R, M] parent ids in [-1, v)
    const float* c;             // [R, M] confidences in [0, 1]
    int R, M, n;
    int32_t* sel;               // [R, n] out
    double* score;              // [R] out or null
};
hipError_t tree_select_launch(const TreeArgs& a, hipStream_t s);

// Verification of R tree drafts of M <= kTreeVerifyMaxNodes nodes over
// V <= kTreeVerifyMaxV tokens (tree_verify.hip).
constexpr int kTreeVerifyMaxNodes = 1024;
constexpr int kTreeVerifyMaxV = 1 << 20;
struct TreeVerifyArgs {
    const void* P;              // [B, M + 1, V] target logits (row 0 the root, 1 + v node v)
    const void* Q;              // [B, M + 1, V] draft logits of each node's children
    int p_bf16, q_bf16;
    const int32_t* parent;      // [B, M] parents first, -1 = a child of the root
    const int32_t* tokens;      // [B, M] draft token of each node
    const int32_t* n_nodes;     // [B] nodes in use (<= M), or null for M
    int B, M, V;
    float invT;
    int greedy;
    const float* uniforms;      // [B, M + 1] or null (Philox stream 3)
    uint64_t seed;
    uint32_t offset;
    int32_t* accepted;          // [B] out
    int32_t* out_tokens;        // [B, M + 1] out
    int32_t* path;              // [B, M] out or null
    int split;                  // workgroups per request (set by the launcher)
    uint32_t epoch;             // tag of this call's exchange words (set by the launcher)
    unsigned poll_limit;        // polls before an exchange wait gives up
};
hipError_t verify_tree_launch(const TreeVerifyArgs& a, hipStream_t s);

hipError_t philox_uniforms_launch(uint64_t seed, uint32_t offset, uint32_t stream, int B, int K,
                                  float* out, hipStream_t s);

}  // namespace specdec
