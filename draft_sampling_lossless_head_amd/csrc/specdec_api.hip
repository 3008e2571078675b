// C ABI of the library (declared in include/specdec.h): argument
// validation, workspace carving and kernel dispatch on the caller's stream.
#include <cmath>
#include <cstdint>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>

#include "device_common.hpp"
#include "launch.hpp"
#include "profile.hpp"
#include "specdec.h"

using namespace specdec;

namespace {

thread_local std::string g_err;

spec_status_t fail(spec_status_t st, const std::string& msg) {
    g_err = msg;
    return st;
}

spec_status_t hip_fail(hipError_t e, const char* where) {
    g_err = std::string(where) + ": " + hipGetErrorString(e);
    return SPEC_ERR_HIP;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }   // NULL passes

bool dtype_ok(int dt) { return dt == SPEC_F32 || dt == SPEC_BF16; }

constexpr int kMaxV = 1 << 28;
constexpr int kMaxDraftV = 4096 * 64;    // the finalize holds <= 16 segment summaries per thread

struct DraftLayout {
    size_t stats, gsums, sup, bar, tflag, w2t, hproj, state, erows, total;
};

DraftLayout draft_layout(bool rnn, int B, int gamma, int V, int r) {
    DraftLayout L{};
    size_t off = 0;
    const size_t nseg = (size_t)draft_max_segments(V);   // 64-token segments at most
    const size_t bpad = ((size_t)B + 127) / 128 * 128;     // streamed rows come in blocks of 128
    L.stats = off;
    off += align_up(bpad * nseg * sizeof(SegStat));
    // q-free draft: one sum per 8 tokens, per segment (16 per 128-token
    // segment, 8 per 64-token segment; the 128-token layout can be larger)
    const size_t ngs = std::max((size_t)((V + 127) / 128) * 16, nseg * 8);
    L.gsums = off;
    off += align_up(bpad * ngs * sizeof(float));
    L.sup = off;   // streaming q-free draft: share summaries [256][bpad]
    off += align_up((size_t)256 * bpad * sizeof(SegStat));
    L.bar = off;   // persistent draft: barrier words
    off += align_up(kPersistBarBytes);
    L.tflag = off;   // persistent draft: per-row token words
    off += align_up(bpad * sizeof(uint64_t));
    L.w2t = off;   // packed bf16 W2 when the caller passes none
    off += align_up(w2p_bytes(r, V));
    if (rnn) {
        L.hproj = off;   // hidden-part partials [kHprojSplit][B * gamma][3r]
        off += align_up((size_t)kHprojSplit * B * gamma * 3 * r * sizeof(float));
        L.state = off;
        off += align_up((size_t)2 * B * r * sizeof(float));
        L.erows = off;   // conditioning rows of every position [B, gamma, 3, r]
        off += align_up((size_t)B * gamma * 3 * r * sizeof(uint16_t));
    }
    L.total = off;
    return L;
}

struct VerifyLayout {
    size_t rows, fin, chunks, rowpos, lrows, w2t, rgs, rsup, total;
};

// markov_r > 0 adds the q-free verification buffers: the recomputed logits of
// one row per request and a transposed W2.
VerifyLayout verify_layout(int B, int gamma_max, int V, int markov_r = 0) {
    VerifyLayout L{};
    size_t off = 0;
    L.rows = off;
    off += align_up((size_t)B * (2 * gamma_max + 1) * verify_row_segs(B, gamma_max, V) * sizeof(RowStat));
    L.fin = off;
    off += align_up((size_t)B * sizeof(FinalInfo));
    L.chunks = off;
    off += align_up((size_t)B * verify_num_chunks(V) * sizeof(double));
    if (markov_r > 0) {
        L.rowpos = off;
        off += align_up((size_t)B * sizeof(int32_t));
        L.lrows = off;
        off += align_up((size_t)B * V * sizeof(float));
        L.w2t = off;
        off += align_up(w2p_bytes(markov_r, V));
        // streamed final draw: group sums [2 nitem][rows padded to 128][4] and
        // share sums [256][rows padded]
        const size_t bpad = ((size_t)B + 127) / 128 * 128;
        const size_t nitem = ((size_t)V + 63) / 64;
        L.rgs = off;
        off += align_up(2 * nitem * bpad * 4 * sizeof(float));
        L.rsup = off;
        off += align_up((size_t)kMaxShares * bpad * sizeof(float));
    }
    L.total = off;
    return L;
}

spec_status_t check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return SPEC_OK;
    if (!ws) return fail(SPEC_ERR_WORKSPACE, "workspace pointer is null");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(SPEC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
        return fail(SPEC_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                            " bytes, got " + std::to_string(ws_bytes));
    return SPEC_OK;
}

spec_status_t check_T(float T) {
    if (!(T >= 0.0f) || std::isinf(T)) return fail(SPEC_ERR_INVALID, "temperature must be finite and >= 0");
    return SPEC_OK;
}

// Shared validation of the draft entry points (both heads).
spec_status_t check_draft_common(const void* U, int U_dtype, const int32_t* x0, const void* W1,
                                 const void* W2, int w_dtype, int r, int B, int gamma, int V,
                                 float T, int32_t* tokens, float* q_logits, float* q_logZ,
                                 float* q_tok_prob, const void* W2T) {
    if (B < 0 || gamma < 0) return fail(SPEC_ERR_INVALID, "B and gamma must be >= 0");
    if (V <= 0 || V > kMaxV) return fail(SPEC_ERR_INVALID, "V must be in [1, 2^28]");
    if (r <= 0) return fail(SPEC_ERR_INVALID, "rank r must be > 0");
    if (V > kMaxDraftV)
        return fail(SPEC_ERR_UNSUPPORTED, "draft sampling supports V <= 262144 (2048 tiles of 128)");
    if (spec_status_t st = check_T(T)) return st;
    if (!dtype_ok(U_dtype) || !dtype_ok(w_dtype)) return fail(SPEC_ERR_UNSUPPORTED, "dtype must be SPEC_F32 or SPEC_BF16");
    if ((int64_t)B * gamma > INT32_MAX) return fail(SPEC_ERR_UNSUPPORTED, "B * gamma too large");
    if (B == 0 || gamma == 0) return SPEC_OK;
    if (!U || !x0 || !W1 || !(W2 || W2T) || !tokens)
        return fail(SPEC_ERR_INVALID, "null required pointer (U, x0, W1, W2 or W2T, tokens)");
    if (!q_logits && (!q_logZ || !q_tok_prob))
        return fail(SPEC_ERR_INVALID, "without q_logits, q_logZ and q_tok_prob are required");
    if (!q_logits && w_dtype != SPEC_BF16)
        return fail(SPEC_ERR_UNSUPPORTED, "the q-free draft (q_logits == NULL) needs bf16 weights");
    if (W2T && w_dtype != SPEC_BF16)
        return fail(SPEC_ERR_UNSUPPORTED, "a packed W2T is bf16 only");
    if (!W2 && w_dtype != SPEC_BF16)
        return fail(SPEC_ERR_INVALID, "fp32 weights need W2");
    if (!aligned16(U) || !aligned16(W1) || !aligned16(W2) || !aligned16(W2T) ||
        !aligned16(q_logits))
        return fail(SPEC_ERR_UNSUPPORTED, "U, W1, W2, W2T and q_logits must be 16-byte aligned");
    if (w_dtype == SPEC_BF16 && (r % 16 != 0 || r > 256))
        return fail(SPEC_ERR_UNSUPPORTED, "bf16 weights need r % 16 == 0 and r <= 256");
    return SPEC_OK;
}

spec_status_t run_draft(DraftArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    void* t;
    if (a.w_bf16 && !a.W2T) {
        t = prof_begin("w2_pack", s);
        e = w2_pack_launch((const uint16_t*)a.W2, a.W2T_ws, a.r, a.V, s);
        prof_end(t, s);
        if (e != hipSuccess) return hip_fail(e, "w2_pack");
        a.W2T = a.W2T_ws;
    }
    if (a.head == kHeadRnn) {
        t = prof_begin("rnn_hidden_proj", s);
        e = rnn_hidden_proj_launch(a, s);
        prof_end(t, s);
        if (e != hipSuccess) return hip_fail(e, "rnn_hidden_proj");
    }
    const int mode = persist_mode();
    if (draft_persists(a, mode)) {
        t = prof_begin("draft_persist", s);
        e = draft_persist_launch(a, a.bar, mode, s);
        prof_end(t, s);
        if (e != hipSuccess) return hip_fail(e, "draft_persist");
        return SPEC_OK;
    }
    if (a.bar) {
        e = persist_clear_abort(a.bar, s);
        if (e != hipSuccess) return hip_fail(e, "persist_clear_abort");
    }
    for (int k = 0; k < a.gamma; ++k) {
        if (a.head == kHeadRnn) {
            t = prof_begin("rnn_gates", s);
            e = rnn_gates_launch(a, k, s);
            prof_end(t, s);
            if (e != hipSuccess) return hip_fail(e, "rnn_gates");
        }
        t = prof_begin(a.q_logits ? "draft_tile" : "draft_tile_qfree", s);
        e = draft_tile_launch(a, k, s);
        prof_end(t, s);
        if (e != hipSuccess) return hip_fail(e, "draft_tile");
        t = prof_begin("draft_finalize", s);
        e = draft_finalize_launch(a, k, s);
        prof_end(t, s);
        if (e != hipSuccess) return hip_fail(e, "draft_finalize");
    }
    return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_version(void) { return 100; }

const char* spec_last_error(void) { return g_err.c_str(); }

int spec_draft_set_persistent(int mode) { return persist_set_mode(mode); }

unsigned spec_draft_set_poll_limit(unsigned polls) { return persist_set_poll_limit(polls); }

spec_status_t spec_draft_status(const void* ws, size_t ws_bytes, int B, int gamma, int V, int r,
                                int32_t* status, void* stream) {
    g_err.clear();
    if (!status) return fail(SPEC_ERR_INVALID, "status is null");
    if (B <= 0 || gamma <= 0 || V <= 0 || V > kMaxDraftV || r <= 0)
        return fail(SPEC_ERR_INVALID, "B, gamma, V and r must be those of a draft call");
    const DraftLayout L = draft_layout(false, B, gamma, V, r);   // same prefix for the RNN head
    if (spec_status_t st = check_ws(const_cast<void*>(ws), ws_bytes, L.bar + kPersistBarBytes))
        return st;
    const char* word = static_cast<const char*>(ws) + L.bar;   // the abort word leads the block
    hipError_t e = hipMemcpyAsync(status, word, sizeof(int32_t), hipMemcpyDeviceToDevice,
                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "spec_draft_status");
}

spec_status_t spec_philox_uniforms(uint64_t seed, uint32_t offset, uint32_t stream, int B, int K,
                                   float* out, void* stream_handle) {
    g_err.clear();
    if (B < 0 || K < 0) return fail(SPEC_ERR_INVALID, "B and K must be >= 0");
    if ((int64_t)B * K == 0) return SPEC_OK;
    if (!out) return fail(SPEC_ERR_INVALID, "out is null");
    hipError_t e = philox_uniforms_launch(seed, offset, stream, B, K, out,
                                          static_cast<hipStream_t>(stream_handle));
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "philox_uniforms");
}

size_t spec_draft_markov_workspace_size(int B, int gamma, int V, int r) {
    if (B <= 0 || gamma <= 0 || V <= 0 || r <= 0) return 0;
    return draft_layout(false, B, gamma, V, r).total;
}

spec_status_t spec_draft_sample_markov(const void* U, int U_dtype, const int32_t* x0,
                                       const void* W1, const void* W2, const void* W2T,
                                       int w_dtype, int r, int B, int gamma, int V, float T,
                                       const float* uniforms, uint64_t seed, uint32_t offset,
                                       int32_t* tokens, float* q_logits, float* q_logZ,
                                       float* q_tok_prob, void* ws, size_t ws_bytes,
                                       void* stream) {
    g_err.clear();
    if (spec_status_t st = check_draft_common(U, U_dtype, x0, W1, W2, w_dtype, r, B, gamma, V, T,
                                              tokens, q_logits, q_logZ, q_tok_prob, W2T))
        return st;
    if (B == 0 || gamma == 0) return SPEC_OK;
    const DraftLayout L = draft_layout(false, B, gamma, V, r);
    if (spec_status_t st = check_ws(ws, ws_bytes, L.total)) return st;
    char* w = static_cast<char*>(ws);
    DraftArgs a{};
    a.head = kHeadMarkov;
    a.U = U;
    a.u_bf16 = U_dtype == SPEC_BF16;
    a.x0 = x0;
    a.W1 = W1;
    a.W2 = W2;
    a.w_bf16 = w_dtype == SPEC_BF16;
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.r = r;
    a.greedy = T == 0.0f;
    a.invT = a.greedy ? 1.0f : 1.0f / T;
    a.uniforms = uniforms;
    a.seed = seed;
    a.offset = offset;
    a.tokens = tokens;
    a.q_logits = q_logits;
    a.q_logZ = q_logZ;
    a.q_tok = q_tok_prob;
    a.stats = reinterpret_cast<SegStat*>(w + L.stats);
    a.gsums = reinterpret_cast<float*>(w + L.gsums);
    a.sup = reinterpret_cast<SegStat*>(w + L.sup);
    a.bar = reinterpret_cast<unsigned*>(w + L.bar);
    a.tflag = reinterpret_cast<uint64_t*>(w + L.tflag);
    a.W2T = static_cast<const uint16_t*>(W2T);
    a.W2T_ws = reinterpret_cast<uint16_t*>(w + L.w2t);
    return run_draft(a, stream);
}

size_t spec_draft_rnn_workspace_size(int B, int gamma, int V, int r, int d) {
    if (B <= 0 || gamma <= 0 || V <= 0 || r <= 0 || d < 0) return 0;
    return draft_layout(true, B, gamma, V, r).total;
}

spec_status_t spec_draft_sample_rnn(const void* U, int U_dtype, const int32_t* x0, const void* h,
                                    int h_dtype, int d, const void* W1, const void* W2,
                                    const void* W2T, const void* Wg, const void* Wc,
                                    const void* Wo, int w_dtype, int r, int B, int gamma, int V,
                                    float T, const float* uniforms, uint64_t seed,
                                    uint32_t offset, int32_t* tokens, float* q_logits,
                                    float* q_logZ, float* q_tok_prob, void* ws, size_t ws_bytes,
                                    void* stream) {
    g_err.clear();
    if (spec_status_t st = check_draft_common(U, U_dtype, x0, W1, W2, w_dtype, r, B, gamma, V, T,
                                              tokens, q_logits, q_logZ, q_tok_prob, W2T))
        return st;
    if (d < 0) return fail(SPEC_ERR_INVALID, "hidden size d must be >= 0");
    if (!dtype_ok(h_dtype)) return fail(SPEC_ERR_UNSUPPORTED, "dtype must be SPEC_F32 or SPEC_BF16");
    if (B == 0 || gamma == 0) return SPEC_OK;
    if (!h || !Wg || !Wc || !Wo) return fail(SPEC_ERR_INVALID, "null required pointer (h, Wg, Wc, Wo)");
    if (w_dtype != SPEC_BF16 || h_dtype != SPEC_BF16)
        return fail(SPEC_ERR_UNSUPPORTED, "the RNN head needs bf16 weights and bf16 hidden states");
    if (d % 8 != 0) return fail(SPEC_ERR_UNSUPPORTED, "the RNN head needs d % 8 == 0");
    if (!aligned16(h) || !aligned16(Wg) || !aligned16(Wc) || !aligned16(Wo))
        return fail(SPEC_ERR_UNSUPPORTED, "h, Wg, Wc and Wo must be 16-byte aligned");
    const DraftLayout L = draft_layout(true, B, gamma, V, r);
    if (spec_status_t st = check_ws(ws, ws_bytes, L.total)) return st;
    char* w = static_cast<char*>(ws);
    DraftArgs a{};
    a.head = kHeadRnn;
    a.U = U;
    a.u_bf16 = U_dtype == SPEC_BF16;
    a.x0 = x0;
    a.W1 = W1;
    a.W2 = W2;
    a.w_bf16 = 1;
    a.h = h;
    a.Wg = Wg;
    a.Wc = Wc;
    a.Wo = Wo;
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.r = r;
    a.d = d;
    a.greedy = T == 0.0f;
    a.invT = a.greedy ? 1.0f : 1.0f / T;
    a.uniforms = uniforms;
    a.seed = seed;
    a.offset = offset;
    a.tokens = tokens;
    a.q_logits = q_logits;
    a.q_logZ = q_logZ;
    a.q_tok = q_tok_prob;
    a.stats = reinterpret_cast<SegStat*>(w + L.stats);
    a.hproj = reinterpret_cast<float*>(w + L.hproj);
    a.state = reinterpret_cast<float*>(w + L.state);
    a.Erows = reinterpret_cast<uint16_t*>(w + L.erows);
    a.gsums = reinterpret_cast<float*>(w + L.gsums);
    a.sup = reinterpret_cast<SegStat*>(w + L.sup);
    a.bar = reinterpret_cast<unsigned*>(w + L.bar);
    a.tflag = reinterpret_cast<uint64_t*>(w + L.tflag);
    a.W2T = static_cast<const uint16_t*>(W2T);
    a.W2T_ws = reinterpret_cast<uint16_t*>(w + L.w2t);
    return run_draft(a, stream);
}

size_t spec_verify_workspace_size(int B, int gamma_max, int V) {
    if (B <= 0 || gamma_max < 0 || V <= 0) return 0;
    return verify_layout(B, gamma_max, V).total;
}

// Scratch of spec_verify_noalloc: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in symbol);
// it passes the device address hipGetSymbolAddress returns for the current
// device, looked up once per device.
static constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kNoAllocMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kNoAllocMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address, or an error status.
spec_status_t noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kNoAllocMaxDevices) return fail(SPEC_ERR_UNSUPPORTED, "device ordinal beyond 63");
    void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            g_scratch_addr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return SPEC_OK;
}

// Argument checks shared by spec_verify and spec_verify_noalloc (everything
// but the workspace).
spec_status_t verify_check(const void* P, int p_dtype, const void* Q, int q_dtype,
                           const int32_t* draft, int B, int gamma_max, int V, float T,
                           const int32_t* accepted, const int32_t* out_tokens) {
    if (B < 0 || gamma_max < 0) return fail(SPEC_ERR_INVALID, "B and gamma_max must be >= 0");
    if (V <= 0 || V > kMaxV) return fail(SPEC_ERR_INVALID, "V must be in [1, 2^28]");
    if (spec_status_t st = check_T(T)) return st;
    if (!dtype_ok(p_dtype) || !dtype_ok(q_dtype)) return fail(SPEC_ERR_UNSUPPORTED, "dtype must be SPEC_F32 or SPEC_BF16");
    if (B == 0) return SPEC_OK;
    if (!P || !accepted || !out_tokens)
        return fail(SPEC_ERR_INVALID, "null required pointer (P, accepted, out_tokens)");
    if (gamma_max > 0 && (!Q || !draft))
        return fail(SPEC_ERR_INVALID, "null required pointer (Q, draft)");
    if (!aligned16(P) || (Q && !aligned16(Q)))
        return fail(SPEC_ERR_UNSUPPORTED, "P and Q must be 16-byte aligned");
    return SPEC_OK;
}

spec_status_t verify_run(const void* P, int p_dtype, const void* Q, int q_dtype,
                         const int32_t* draft, const int32_t* lens, const int64_t* p_row_off,
                         const int64_t* q_row_off, int B, int gamma_max, int V, float T,
                         const float* uniforms, uint64_t seed, uint32_t offset,
                         int32_t* accepted, int32_t* out_tokens, float* p_logZ, float* q_logZ,
                         float* accept_prob, void* ws, const VerifyLayout& L, void* stream) {
    char* w = static_cast<char*>(ws);
    VerifyArgs a{};
    a.P = P;
    a.p_bf16 = p_dtype == SPEC_BF16;
    a.Q = Q;
    a.q_bf16 = q_dtype == SPEC_BF16;
    a.draft = draft;
    a.lens = lens;
    a.p_row_off = p_row_off;
    a.q_row_off = q_row_off;
    a.B = B;
    a.gamma_max = gamma_max;
    a.V = V;
    a.greedy = T == 0.0f;
    a.invT = a.greedy ? 1.0f : 1.0f / T;
    a.uniforms = uniforms;
    a.seed = seed;
    a.offset = offset;
    a.accepted = accepted;
    a.out_tokens = out_tokens;
    a.p_logZ = p_logZ;
    a.q_logZ = q_logZ;
    a.accept_prob = accept_prob;
    a.rows = reinterpret_cast<RowStat*>(w + L.rows);
    a.row_segs = verify_row_segs(B, gamma_max, V);
    a.fin = reinterpret_cast<FinalInfo*>(w + L.fin);
    a.chunk_sums = reinterpret_cast<double*>(w + L.chunks);
    hipError_t e = verify_launch(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "verify");
}

}  // namespace

spec_status_t spec_verify(const void* P, int p_dtype, const void* Q, int q_dtype,
                          const int32_t* draft, const int32_t* lens, const int64_t* p_row_off,
                          const int64_t* q_row_off, int B, int gamma_max, int V, float T,
                          const float* uniforms, uint64_t seed, uint32_t offset,
                          int32_t* accepted, int32_t* out_tokens, float* p_logZ, float* q_logZ,
                          float* accept_prob, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (spec_status_t st = verify_check(P, p_dtype, Q, q_dtype, draft, B, gamma_max, V, T, accepted, out_tokens))
        return st;
    if (B == 0) return SPEC_OK;
    const VerifyLayout L = verify_layout(B, gamma_max, V);
    if (spec_status_t st = check_ws(ws, ws_bytes, L.total)) return st;
    return verify_run(P, p_dtype, Q, q_dtype, draft, lens, p_row_off, q_row_off, B, gamma_max, V, T,
                      uniforms, seed, offset, accepted, out_tokens, p_logZ, q_logZ, accept_prob, ws, L,
                      stream);
}

size_t spec_verify_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

spec_status_t spec_verify_noalloc(const void* P, int p_dtype, const void* Q, int q_dtype,
                                  const int32_t* draft, const int32_t* lens,
                                  const int64_t* p_row_off, const int64_t* q_row_off, int B,
                                  int gamma_max, int V, float T, const float* uniforms,
                                  uint64_t seed, uint32_t offset, int32_t* accepted,
                                  int32_t* out_tokens, float* p_logZ, float* q_logZ,
                                  float* accept_prob, void* stream) {
    g_err.clear();
    if (spec_status_t st = verify_check(P, p_dtype, Q, q_dtype, draft, B, gamma_max, V, T, accepted, out_tokens))
        return st;
    if (B == 0) return SPEC_OK;
    const VerifyLayout L = verify_layout(B, gamma_max, V);
    if (L.total > kNoAllocScratchBytes)
        return fail(SPEC_ERR_WORKSPACE, "spec_verify_noalloc: B, gamma_max and V need " + std::to_string(L.total) +
                                            " bytes of scratch, more than its fixed " +
                                            std::to_string(kNoAllocScratchBytes) + " (use spec_verify)");
    void* ws = nullptr;
    if (spec_status_t st = noalloc_scratch(&ws)) return st;
    return verify_run(P, p_dtype, Q, q_dtype, draft, lens, p_row_off, q_row_off, B, gamma_max, V, T,
                      uniforms, seed, offset, accepted, out_tokens, p_logZ, q_logZ, accept_prob, ws, L,
                      stream);
}


spec_status_t spec_verify_tree(const void* P, int p_dtype, const void* Q, int q_dtype,
                               const int32_t* parent, const int32_t* tokens, const int32_t* n_nodes,
                               int B, int M, int V, float T, const float* uniforms, uint64_t seed,
                               uint32_t offset, int32_t* accepted, int32_t* out_tokens,
                               int32_t* path, void* stream) {
    g_err.clear();
    if (B < 0 || M < 0) return fail(SPEC_ERR_INVALID, "B and M must be >= 0");
    if (V <= 0 || V > kTreeVerifyMaxV) return fail(SPEC_ERR_INVALID, "V must be in [1, 2^20]");
    if (M > kTreeVerifyMaxNodes) return fail(SPEC_ERR_UNSUPPORTED, "M must be <= 1024");
    if (spec_status_t st = check_T(T)) return st;
    if (!dtype_ok(p_dtype) || !dtype_ok(q_dtype)) return fail(SPEC_ERR_UNSUPPORTED, "dtype must be SPEC_F32 or SPEC_BF16");
    if (B == 0) return SPEC_OK;
    if (!P || !accepted || !out_tokens)
        return fail(SPEC_ERR_INVALID, "null required pointer (P, accepted, out_tokens)");
    if (M > 0 && (!Q || !parent || !tokens))
        return fail(SPEC_ERR_INVALID, "null required pointer (Q, parent, tokens)");
    if (!aligned16(P) || (Q && !aligned16(Q)))
        return fail(SPEC_ERR_UNSUPPORTED, "P and Q must be 16-byte aligned");
    TreeVerifyArgs a{};
    a.P = P;
    a.p_bf16 = p_dtype == SPEC_BF16;
    a.Q = Q;
    a.q_bf16 = q_dtype == SPEC_BF16;
    a.parent = parent;
    a.tokens = tokens;
    a.n_nodes = n_nodes;
    a.B = B;
    a.M = M;
    a.V = V;
    a.greedy = T == 0.0f;
    a.invT = a.greedy ? 1.0f : 1.0f / T;
    a.uniforms = uniforms;
    a.seed = seed;
    a.offset = offset;
    a.accepted = accepted;
    a.out_tokens = out_tokens;
    a.path = path;
    a.poll_limit = persist_poll_limit();
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* t = prof_begin("verify_tree", s);
    hipError_t e = verify_tree_launch(a, s);
    prof_end(t, s);
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "verify_tree");
}

spec_status_t spec_acceptance_rate(const void* P, int p_dtype, const void* Q, int q_dtype,
                                   const int32_t* lens, const int64_t* p_row_off,
                                   const int64_t* q_row_off, int B, int gamma_max, int V, float T,
                                   float* alpha, float* tv, void* stream) {
    g_err.clear();
    if (B < 0 || gamma_max < 0) return fail(SPEC_ERR_INVALID, "B and gamma_max must be >= 0");
    if (V <= 0 || V > kMaxV) return fail(SPEC_ERR_INVALID, "V must be in [1, 2^28]");
    if (spec_status_t st = check_T(T)) return st;
    if (!dtype_ok(p_dtype) || !dtype_ok(q_dtype)) return fail(SPEC_ERR_UNSUPPORTED, "dtype must be SPEC_F32 or SPEC_BF16");
    if ((int64_t)B * gamma_max > INT32_MAX) return fail(SPEC_ERR_UNSUPPORTED, "B * gamma_max too large");
    if (B == 0 || gamma_max == 0) return SPEC_OK;
    if (!P || !Q || !alpha) return fail(SPEC_ERR_INVALID, "null required pointer (P, Q, alpha)");
    AlphaArgs a{};
    a.P = P;
    a.p_bf16 = p_dtype == SPEC_BF16;
    a.Q = Q;
    a.q_bf16 = q_dtype == SPEC_BF16;
    a.lens = lens;
    a.p_row_off = p_row_off;
    a.q_row_off = q_row_off;
    a.B = B;
    a.gamma_max = gamma_max;
    a.V = V;
    a.greedy = T == 0.0f;
    a.invT = a.greedy ? 1.0f : 1.0f / T;
    a.alpha = alpha;
    a.tv = tv;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* t = prof_begin("acceptance_rate", s);
    hipError_t e = acceptance_rate_launch(a, s);
    prof_end(t, s);
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "acceptance_rate");
}

spec_status_t spec_confidence_head(const void* h, int h_dtype, int d, const int32_t* x0,
                                   const int32_t* draft, const void* W1, int w_dtype, int r,
                                   const float* w, int R, int gamma, int V, float* c,
                                   void* stream) {
    g_err.clear();
    if (R < 0 || gamma < 0) return fail(SPEC_ERR_INVALID, "R and gamma must be >= 0");
    if (d <= 0 || r <= 0 || V <= 0) return fail(SPEC_ERR_INVALID, "d, r and V must be > 0");
    if (!dtype_ok(h_dtype) || !dtype_ok(w_dtype)) return fail(SPEC_ERR_UNSUPPORTED, "dtype must be SPEC_F32 or SPEC_BF16");
    if ((int64_t)R * gamma > INT32_MAX) return fail(SPEC_ERR_UNSUPPORTED, "R * gamma too large");
    if (R == 0 || gamma == 0) return SPEC_OK;
    if (!h || !x0 || !draft || !W1 || !w || !c) return fail(SPEC_ERR_INVALID, "null pointer (h, x0, draft, W1, w, c)");
    ConfArgs a{};
    a.h = h;
    a.h_bf16 = h_dtype == SPEC_BF16;
    a.d = d;
    a.x0 = x0;
    a.draft = draft;
    a.W1 = W1;
    a.w_bf16 = w_dtype == SPEC_BF16;
    a.r = r;
    a.w = w;
    a.R = R;
    a.gamma = gamma;
    a.V = V;
    a.c = c;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* t = prof_begin("confidence_head", s);
    hipError_t e = confidence_launch(a, s);
    prof_end(t, s);
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "confidence_head");
}

size_t spec_prefix_schedule_workspace_size(int R, int gamma) {
    if (R < 0 || gamma < 0 || (int64_t)R * gamma > kSchedMax) return 0;
    return prefix_schedule_ws_bytes(R, gamma);
}

spec_status_t spec_prefix_schedule(const float* c, int R, int gamma, const double* sps, int nsps,
                                   int32_t* lens, int32_t* B_out, double* tau_out, void* ws,
                                   size_t ws_bytes, void* stream) {
    g_err.clear();
    if (R < 0 || gamma < 0 || nsps < 0) return fail(SPEC_ERR_INVALID, "R, gamma and nsps must be >= 0");
    if (nsps > 0 && !sps) return fail(SPEC_ERR_INVALID, "null sps with nsps > 0");
    if ((int64_t)R * gamma > kSchedMax || R > kSchedMax)
        return fail(SPEC_ERR_UNSUPPORTED, "R and R * gamma must be <= 8192");
    if (R > 0 && (!lens || (gamma > 0 && !c))) return fail(SPEC_ERR_INVALID, "null c or lens");
    const size_t need = prefix_schedule_ws_bytes(R, gamma);
    if ((int64_t)R * gamma > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(SPEC_ERR_WORKSPACE, "workspace missing, unaligned or smaller than spec_prefix_schedule_workspace_size");
    SchedArgs a{};
    a.ws_val = static_cast<uint32_t*>(ws);
    a.ws_id = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + need / 2);
    a.c = c;
    a.R = R;
    a.gamma = gamma;
    a.sps = sps;
    a.nsps = nsps;
    a.lens = lens;
    a.B_out = B_out;
    a.tau_out = tau_out;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* t = prof_begin("prefix_schedule", s);
    hipError_t e = prefix_schedule_launch(a, s);
    prof_end(t, s);
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "prefix_schedule");
}

spec_status_t spec_tree_select(const int32_t* parent, const float* c, int R, int M, int n,
                               int32_t* sel, double* score, void* stream) {
    g_err.clear();
    if (R < 0 || M < 0 || n < 0) return fail(SPEC_ERR_INVALID, "R, M and n must be >= 0");
    if (M > kTreeMax) return fail(SPEC_ERR_UNSUPPORTED, "M must be <= 4096");
    if ((int64_t)R * M > INT32_MAX || (int64_t)R * n > INT32_MAX) return fail(SPEC_ERR_UNSUPPORTED, "R * M or R * n too large");
    if (R == 0) return SPEC_OK;
    if ((M > 0 && (!parent || !c)) || (n > 0 && !sel)) return fail(SPEC_ERR_INVALID, "null parent, c or sel");
    TreeArgs a{};
    a.parent = parent;
    a.c = c;
    a.R = R;
    a.M = M;
    a.n = n;
    a.sel = sel;
    a.score = score;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* t = prof_begin("tree_select", s);
    hipError_t e = tree_select_launch(a, s);
    prof_end(t, s);
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "tree_select");
}

size_t spec_pack_w2_bytes(int r, int V) {
    if (r <= 0 || V <= 0 || V > kMaxV) return 0;
    return w2p_bytes(r, V);
}

spec_status_t spec_pack_w2(const void* W2, void* W2T, int r, int V, void* stream) {
    g_err.clear();
    if (r <= 0 || V <= 0 || V > kMaxV) return fail(SPEC_ERR_INVALID, "bad r or V");
    if (!W2 || !W2T) return fail(SPEC_ERR_INVALID, "null W2 or W2T");
    if (r % 16 != 0 || r > 256) return fail(SPEC_ERR_UNSUPPORTED, "packing needs r % 16 == 0 and r <= 256");
    if (!aligned16(W2T)) return fail(SPEC_ERR_UNSUPPORTED, "W2T must be 16-byte aligned");
    hipError_t e = w2_pack_launch(static_cast<const uint16_t*>(W2), static_cast<uint16_t*>(W2T),
                                  r, V, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "w2_pack");
}

size_t spec_verify_markov_workspace_size(int B, int gamma_max, int V, int r) {
    if (B <= 0 || gamma_max < 0 || V <= 0 || r <= 0) return 0;
    return verify_layout(B, gamma_max, V, r).total;
}

size_t spec_draft_rnn_cond_offset(int B, int gamma, int V, int r, int d) {
    (void)d;
    if (B <= 0 || gamma <= 0 || V <= 0 || V > kMaxDraftV || r <= 0) return 0;
    return draft_layout(true, B, gamma, V, r).erows;
}

size_t spec_verify_rnn_workspace_size(int B, int gamma_max, int V, int r) {
    return spec_verify_markov_workspace_size(B, gamma_max, V, r);
}

// Verification of a q-free draft: the Markov head (cond == NULL: rows
// rebuilt from W1[x_{n-1}]) or the RNN head (cond: the draft's conditioning
// rows [B, gamma, 3, r]).
static spec_status_t verify_qfree(const void* P, int p_dtype, const void* U, int U_dtype,
                                  const int32_t* x0, const void* W1, const uint16_t* cond,
                                  const void* W2, const void* W2T, int w_dtype, int r,
                                  const int32_t* draft, const float* q_logZ,
                                  const float* q_tok_prob, const int32_t* lens,
                                  const int64_t* p_row_off, int B, int gamma_max, int V, float T,
                                  const float* uniforms, uint64_t seed, uint32_t offset,
                                  int32_t* accepted, int32_t* out_tokens, float* p_logZ,
                                  float* accept_prob, void* ws, size_t ws_bytes, void* stream);

spec_status_t spec_verify_rnn(const void* P, int p_dtype, const void* U, int U_dtype,
                              const void* cond, const void* W2, const void* W2T, int r,
                              const int32_t* draft, const float* q_logZ, const float* q_tok_prob,
                              const int32_t* lens, const int64_t* p_row_off, int B, int gamma_max,
                              int V, float T, const float* uniforms, uint64_t seed,
                              uint32_t offset, int32_t* accepted, int32_t* out_tokens,
                              float* p_logZ, float* accept_prob, void* ws, size_t ws_bytes,
                              void* stream) {
    g_err.clear();
    if (B > 0 && gamma_max > 0 && !cond)
        return fail(SPEC_ERR_INVALID, "null required pointer (cond)");
    if (!aligned16(cond)) return fail(SPEC_ERR_UNSUPPORTED, "cond must be 16-byte aligned");
    return verify_qfree(P, p_dtype, U, U_dtype, nullptr, nullptr, static_cast<const uint16_t*>(cond),
                        W2, W2T, SPEC_BF16, r, draft, q_logZ, q_tok_prob, lens, p_row_off, B,
                        gamma_max, V, T, uniforms, seed, offset, accepted, out_tokens, p_logZ,
                        accept_prob, ws, ws_bytes, stream);
}

spec_status_t spec_verify_markov(const void* P, int p_dtype, const void* U, int U_dtype,
                                 const int32_t* x0, const void* W1, const void* W2,
                                 const void* W2T, int w_dtype, int r, const int32_t* draft,
                                 const float* q_logZ, const float* q_tok_prob,
                                 const int32_t* lens, const int64_t* p_row_off, int B,
                                 int gamma_max, int V, float T, const float* uniforms,
                                 uint64_t seed, uint32_t offset, int32_t* accepted,
                                 int32_t* out_tokens, float* p_logZ, float* accept_prob,
                                 void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (B > 0 && gamma_max > 0 && (!x0 || !W1))
        return fail(SPEC_ERR_INVALID, "null required pointer (x0, W1)");
    return verify_qfree(P, p_dtype, U, U_dtype, x0, W1, nullptr, W2, W2T, w_dtype, r, draft,
                        q_logZ, q_tok_prob, lens, p_row_off, B, gamma_max, V, T, uniforms, seed,
                        offset, accepted, out_tokens, p_logZ, accept_prob, ws, ws_bytes, stream);
}

}  // extern "C"

static spec_status_t verify_qfree(const void* P, int p_dtype, const void* U, int U_dtype,
                                  const int32_t* x0, const void* W1, const uint16_t* cond,
                                  const void* W2, const void* W2T, int w_dtype, int r,
                                  const int32_t* draft, const float* q_logZ,
                                  const float* q_tok_prob, const int32_t* lens,
                                  const int64_t* p_row_off, int B, int gamma_max, int V, float T,
                                  const float* uniforms, uint64_t seed, uint32_t offset,
                                  int32_t* accepted, int32_t* out_tokens, float* p_logZ,
                                  float* accept_prob, void* ws, size_t ws_bytes, void* stream) {
    if (B < 0 || gamma_max < 0) return fail(SPEC_ERR_INVALID, "B and gamma_max must be >= 0");
    if (V <= 0 || V > kMaxDraftV) return fail(SPEC_ERR_INVALID, "V must be in [1, 262144]");
    if (r <= 0) return fail(SPEC_ERR_INVALID, "rank r must be > 0");
    if (spec_status_t st = check_T(T)) return st;
    if (!dtype_ok(p_dtype) || !dtype_ok(U_dtype)) return fail(SPEC_ERR_UNSUPPORTED, "dtype must be SPEC_F32 or SPEC_BF16");
    if (w_dtype != SPEC_BF16 || r % 16 != 0 || r > 256)
        return fail(SPEC_ERR_UNSUPPORTED, "q-free verification needs bf16 weights, r % 16 == 0, r <= 256");
    if ((int64_t)B * gamma_max > INT32_MAX) return fail(SPEC_ERR_UNSUPPORTED, "B * gamma_max too large");
    if (B == 0) return SPEC_OK;
    if (!P || !accepted || !out_tokens) return fail(SPEC_ERR_INVALID, "null required pointer (P, accepted, out_tokens)");
    if (gamma_max > 0 && (!U || !(W2 || W2T) || !draft || !q_logZ || !q_tok_prob))
        return fail(SPEC_ERR_INVALID, "null required pointer (U, W2 or W2T, draft, q_logZ, q_tok_prob)");
    if (!aligned16(P) || !aligned16(U) || !aligned16(W1) || !aligned16(W2) || !aligned16(W2T))
        return fail(SPEC_ERR_UNSUPPORTED, "P, U, W1, W2 and W2T must be 16-byte aligned");
    const VerifyLayout L = verify_layout(B, gamma_max, V, r);
    if (spec_status_t st = check_ws(ws, ws_bytes, L.total)) return st;
    char* w = static_cast<char*>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    VerifyArgs a{};
    a.P = P;
    a.p_bf16 = p_dtype == SPEC_BF16;
    a.Q = w + L.lrows;             // recomputed logits, one row per request
    a.q_bf16 = 0;
    a.q_single_row = 1;
    a.draft = draft;
    a.lens = lens;
    a.p_row_off = p_row_off;
    a.q_row_off = nullptr;
    a.B = B;
    a.gamma_max = gamma_max;
    a.V = V;
    a.greedy = T == 0.0f;
    a.invT = a.greedy ? 1.0f : 1.0f / T;
    a.uniforms = uniforms;
    a.seed = seed;
    a.offset = offset;
    a.accepted = accepted;
    a.out_tokens = out_tokens;
    a.p_logZ = p_logZ;
    a.q_logZ = nullptr;
    a.accept_prob = accept_prob;
    a.qprob = q_tok_prob;
    a.qlogz = q_logZ;
    a.row_pos = reinterpret_cast<int32_t*>(w + L.rowpos);
    a.rows = reinterpret_cast<RowStat*>(w + L.rows);
    a.row_segs = verify_row_segs(B, gamma_max, V);
    a.fin = reinterpret_cast<FinalInfo*>(w + L.fin);
    a.chunk_sums = reinterpret_cast<double*>(w + L.chunks);
    hipError_t e = verify_rows_decide_launch(a, s);
    if (e != hipSuccess) return hip_fail(e, "verify");
    if (!cond && !a.greedy && gamma_max > 0 && p_dtype == SPEC_BF16 && U_dtype == SPEC_BF16 &&
        resid_streams(B, V, r)) {
        // streamed final draw: residual rows rebuilt in registers, never stored
        // (gamma_max == 0 has no residual: the bonus draw below serves it)
        const uint16_t* w2t = static_cast<const uint16_t*>(W2T);
        if (!w2t) {
            void* t = prof_begin("w2_pack", s);
            e = w2_pack_launch(static_cast<const uint16_t*>(W2),
                               reinterpret_cast<uint16_t*>(w + L.w2t), r, V, s);
            prof_end(t, s);
            if (e != hipSuccess) return hip_fail(e, "w2_pack");
            w2t = reinterpret_cast<const uint16_t*>(w + L.w2t);
        }
        ResidArgs ra{};
        ra.P = static_cast<const uint16_t*>(P);
        ra.p_row_off = p_row_off;
        ra.U = static_cast<const uint16_t*>(U);
        ra.W1 = static_cast<const uint16_t*>(W1);
        ra.W2P = w2t;
        ra.x0 = x0;
        ra.draft = draft;
        ra.fin = a.fin;
        ra.gsums = reinterpret_cast<float*>(w + L.rgs);
        ra.sup = reinterpret_cast<float*>(w + L.rsup);
        ra.out_tokens = out_tokens;
        ra.uniforms = uniforms;
        ra.seed = seed;
        ra.offset = offset;
        ra.B = B;
        ra.G = gamma_max;
        ra.V = V;
        ra.r = r;
        ra.invT = a.invT;
        void* t = prof_begin("verify_resid", s);
        e = verify_resid_launch(ra, s);
        prof_end(t, s);
        return e == hipSuccess ? SPEC_OK : hip_fail(e, "verify_resid");
    }
    if (!a.greedy && gamma_max > 0) {
        const uint16_t* w2t = static_cast<const uint16_t*>(W2T);
        if (!w2t) {
            void* t = prof_begin("w2_pack", s);
            e = w2_pack_launch(static_cast<const uint16_t*>(W2),
                                    reinterpret_cast<uint16_t*>(w + L.w2t), r, V, s);
            prof_end(t, s);
            if (e != hipSuccess) return hip_fail(e, "w2_pack");
            w2t = reinterpret_cast<const uint16_t*>(w + L.w2t);
        }
        TileParams tp{};
        tp.U = U;
        tp.W1 = static_cast<const uint16_t*>(W1);
        tp.Erows = cond;   // RNN head: the draft's conditioning rows
        tp.W2T = w2t;
        tp.x0 = x0;
        tp.tokens = draft;
        tp.row_pos = a.row_pos;
        tp.out = reinterpret_cast<float*>(w + L.lrows);
        tp.B = B;
        tp.gamma = gamma_max;
        tp.V = V;
        tp.r = r;
        tp.k = 0;
        tp.invT = a.invT;
        tp.greedy = 0;
        void* t = prof_begin("verify_residual_rows", s);
        e = residual_rows_launch(tp, U_dtype == SPEC_BF16, s);
        prof_end(t, s);
        if (e != hipSuccess) return hip_fail(e, "verify_residual_rows");
    }
    e = verify_final_launch(a, s);
    return e == hipSuccess ? SPEC_OK : hip_fail(e, "verify");
}
