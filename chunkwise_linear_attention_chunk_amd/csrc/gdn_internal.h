// Internal interface between the C-ABI host code and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kDefaultCUs = 256;   // MI355X compute units: the plan's assumption when no device answers
constexpr int GDN_GATE_CHANNEL_K = 1;  // gate kind of per-channel (KDA) gates, as in gdn.h

// Per (chunk, head) gate block written by the per-chunk kernel, read by the recurrence: fp32 rows
// of 64 tokens.  Scalar gate, with r_k and r_q the key and query rows' L2-norm factors of the
// in-kernel prologue (else 1) folded in so that the recurrence applies none of them itself:
//   BETA beta,  SC r_k gamma_C / gamma,  GAK r_k gamma,  GAQ r_q gamma,
//   GLQ log2 gamma + log2 r_q,  GLK log2 gamma - log2 r_k,  GC gamma_C (one float).
// Per-channel gate: BETA, the [D_k] chunk decay 2^G_C, and at GC the chunk's decay bound for
// warmup CP (the product over its tokens of each token's largest channel decay).  Tail tokens
// carry beta = 0 and g = 0.
enum GateBlock {
    GB_BETA = 0, GB_SC = 64, GB_GAK = 128, GB_GAQ = 192, GB_GLQ = 256, GB_GLK = 320, GB_GC = 384,
    GB_DEC = 64, GB_FLOATS = 512
};

// The in-kernel prologue (gdn_fwd_args): raw gate inputs, beta logits, q/k rows to normalise.
struct Prologue {
    int qk_l2norm;          // 1: q and k rows used as x / sqrt(sum x^2 + kL2Eps)
    int beta_sigmoid;       // 1: beta holds logits
    const float *A_log;     // nullable [H_v]: g holds raw gate inputs
    const float *dt_bias;   // nullable [H_v] (scalar gate) or [H_v][D_k] (per-channel gate)
    float lower_bound;      // 0: -exp(A_log) softplus(x + b); < 0: lower_bound sigmoid(exp(A_log) (x + b))
};
constexpr float kL2Eps = 1e-6f;
// log-gate of a raw input x (activation of the gate cumsum kernel on the KDA page, section 2)
__device__ __forceinline__ float gate_activation(const Prologue &pr, float x, float a_log, float bias) {
    const float y = x + bias;
    if (pr.lower_bound < 0.f) return pr.lower_bound / (1.f + expf(-expf(a_log) * y));
    const float softplus = fmaxf(y, 0.f) + log1pf(expf(-fabsf(y)));
    return -expf(a_log) * softplus;
}
__device__ __forceinline__ float beta_value(const Prologue &pr, float b) {
    return pr.beta_sigmoid ? 1.f / (1.f + expf(-b)) : b;
}

// Device-side plan tables (built by the plan kernel from cu_seqlens or the batch shape).
struct SeqInfo {            // one per sequence
    int tok0;               // first token (row of the [B*T] token axis)
    int len;                // tokens
    int chunk0;             // global index of its first chunk
    int nchunks;            // ceil(len / 64)
    int seg0;               // global index of its first segment
};
struct ChunkInfo {          // one per global chunk
    int tok0;               // first token of the chunk
    int nv;                 // valid tokens (1..64)
};
struct SegInfo {            // one per (sequence, segment of at most seg_chunks chunks)
    int n;                  // sequence
    int j;                  // segment index within the sequence
    int c0;                 // first chunk of the segment within the sequence
    int nchunks;            // chunks in the segment (0 only for an empty sequence)
    int last;               // 1 for the last segment of its sequence
};

struct PlanParams {
    const int32_t *cu;      // nullable: batched form uses n * T
    int N, T;
    int total_tokens;       // B * T: sequence spans are clamped to [0, total_tokens)
    int total_chunks;       // chunk count the host planned from its copy of cu_seqlens
    int seg_chunks;         // segment length in chunks
    int total_segs;         // segment count the host planned
    SeqInfo *seq;           // [N]
    ChunkInfo *chunks;      // [total chunks]
    SegInfo *segs;          // [total segments]
    int *order;             // [total segments] longest first (ties by index)
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Batched input: segment gs of sequences with nc chunks each, segments of sl chunks.
__device__ __forceinline__ SegInfo seg_info(const SegInfo *segs, int gs, int T, int sl) {
    if (segs) return segs[gs];
    const int nc = ceil_div(T, kChunk), ns = max(1, ceil_div(nc, sl));
    const int n = gs / ns, j = gs - n * ns, c0 = j * sl;
    return SegInfo{n, j, c0, min(sl, nc - c0), j == ns - 1 ? 1 : 0};
}

// Batched (not packed) input has no tables: sequence n covers tokens [n T, n T + T).
__device__ __forceinline__ SeqInfo seq_info(const SeqInfo *seq, int n, int T) {
    if (seq) return seq[n];
    const int nc = (T + kChunk - 1) / kChunk;
    return SeqInfo{n * T, T, n * nc, nc, 0};
}
__device__ __forceinline__ ChunkInfo chunk_info(const ChunkInfo *chunks, int ci, int T) {
    if (chunks) return chunks[ci];
    const int nc = (T + kChunk - 1) / kChunk, n = ci / nc, c = ci - n * nc;
    return ChunkInfo{n * T + c * kChunk, min(kChunk, T - c * kChunk)};
}

struct IntraParams {
    const void *q, *k, *g, *beta;
    const ChunkInfo *chunks;  // nullptr: batched input of T tokens per sequence
    int T;
    int n_chunks, H_qk, H_v;
    float scale;
    void *A;                // [n_chunks][H_v][64][64] in the input dtype
    void *P;                // unused with a scalar gate (the recurrence forms P)
    float *gates;           // [n_chunks][H_v][GB_FLOATS]
    Prologue pro;
    // batched input in pieces: chunks [piece_lo, piece_lo + piece_cnt) of each of the N
    // sequences (piece_cnt 0: every chunk)
    int N, piece_lo, piece_cnt;
};

struct IntraKdaParams {       // per-channel gates
    const void *q, *k, *g, *beta;  // g: [tokens][H_v][D_k] in the input dtype
    const ChunkInfo *chunks;
    int T;
    int n_chunks, H_qk, H_v;
    float scale;
    void *A;                // [n_chunks][H_v][64][64]
    void *P;                // [n_chunks][H_v][parts][64][64]: scale (Lower(2^(G_i - G_j)) (.) Q K^T), hi (+ lo)
    void *kg;               // [n_chunks][H_v][64][D_k]: K 2^G
    void *kd, *qg;          // [n_chunks][H_v][parts][64][D_k]: K 2^(G_C - G), Q 2^G, hi (+ lo)
    float *gates;           // [n_chunks][H_v][GB_FLOATS]: beta and the chunk decay 2^G_C
    Prologue pro;
    int N, piece_lo, piece_cnt;   // as in IntraParams
};

struct ChunkParams {
    const void *q, *k, *v, *g, *beta;
    const void *A;          // from the intra kernel
    const float *h0;        // nullable [N][H_v][D_k][D_v]
    void *o;
    float *final_state;     // nullable
    const SeqInfo *seq;     // nullptr: batched input of T tokens per sequence (order = identity)
    const SegInfo *segs;    // nullptr: batched input, segments derived from T and seg_chunks
    const int *order;       // segment order (packed input)
    int T;
    int N, H_qk, H_v, D_v, n_slices;
    int seg_chunks, total_segs;
    float scale;
    int o_f32;              // 1: o is fp32 (the unrounded result), 0: o has the input dtype
    // context parallelism (workspace, fp32, [total_segs][H_v][D_k][cols]):
    float *seg_sstar;       // pre-process output: S* of the segment (cols = D_v)
    float *seg_m;           // pre-process output: transition M of the segment (cols = D_k)
    const float *seg_start; // main pass input for segments j >= 1 (cols = D_v)
    // from the per-chunk kernel: P, the gate blocks, and the gated tiles of per-channel gates
    const void *kg, *kd, *qg, *P;
    const float *gates;
    const int *warm;        // warmup CP: [total_segs][H_v] warmup chunks of each segment (nullable)
    // pieces (batched input): seg_only = j + 1 runs segment j of every sequence only (0: all), from
    // seg_start; seg_next (nullable) receives a non-last segment's end state as the next one's start
    int seg_only;
    float *seg_next;
    int n_cus;              // compute units of the device the launch goes to
    // nullable (main pass without CP): receives the state entering every chunk, fp32
    // [global chunk][H_v][D_k][D_v] (the backward's recomputed chunk states); o may then be null
    float *chunk_states;
    // nullable (that build, scalar gate, bf16): receives scale P = scale Lower(Gamma) (.) Q K^T of
    // every chunk as a bf16 pair, [global chunk][H_v] x (hi [64][64], lo [64][64]) row-major; the
    // tiles above the diagonal that the backward's scan reads, (0, 1) and (2, 3), are zeros
    void *pmat;
};

// chunk ci of the per-chunk grid: every chunk, or the chunks of one piece of a batched input
__device__ __forceinline__ int piece_chunk(int ci, int T, int piece_lo, int piece_cnt) {
    if (!piece_cnt) return ci;
    const int nn = ci / piece_cnt;
    return nn * ((T + kChunk - 1) / kChunk) + piece_lo + (ci - nn * piece_cnt);
}

struct WarmParams {         // warmup CP gate statistics
    const SegInfo *segs;    // nullptr: batched input
    const SeqInfo *seq;
    const float *gates;     // gate blocks (GB_GC: the chunk's decay bound)
    int T, H_v, seg_chunks, total_segs;
    float log2_tol;         // -inf: never (whole prefix)
    int *warm;              // [total_segs][H_v]
};

struct FixParams {
    const SegInfo *segs;
    const SeqInfo *seq;
    int T, N, H_v, D_v, seg_chunks, total_segs;
    const float *h0;        // nullable
    const float *seg_sstar, *seg_m;
    float *seg_start;
};

struct RecurrentParams {     // token-by-token path (gdn_fwd_recurrent)
    const void *q, *k, *v, *g, *beta;
    const float *h0;            // nullable; may alias final_state
    float *final_state;         // nullable
    void *o;
    const int32_t *cu;          // nullable: batched input of T tokens per sequence
    int T, N, H_qk, H_v, D_v, total_tokens;
    float scale;
    int o_f32;                  // 1: o is fp32
    Prologue pro;
};

struct BwdParams {           // backward (gdn_bwd), scalar gate
    const void *q, *k, *v, *beta, *dout;   // input dtype
    const void *g;                         // fp32 [tokens][H_v] (scalar gate) or [tokens][H_v][D_k] (input dtype)
    const float *h0, *dht;                 // nullable
    const void *A;                         // (I + L)^-1 of every chunk, from the per-chunk kernel
    const void *P, *kg, *kd, *qg;          // per-channel gates: its scale P, K e^G, K e^{G_C - G}, Q e^G
    const float *gates;                    // its gate blocks (GB_*, no prologue factors)
    const SeqInfo *seq;                    // nullptr: batched input
    const ChunkInfo *chunks;
    int T, N, n_chunks, H_qk, H_v, D_v;
    int64_t T_total;                       // B * T
    float scale;
    float *states, *dsnext;                // [n_chunks][H_v][D_k][D_v]: S entering, dS leaving each chunk
    float *pmat;                           // [n_chunks][H_v][64][64]: scale Pt
    int channel;                           // 1: per-channel gates (g is [tokens][H_v][D_k] in the input dtype)
    float *vp, *dlmat;                     // per-channel gates: V' [n_chunks][H_v][64][D_v], dL [n_chunks][H_v][64][64]
    float *dq, *dk, *dv, *dg, *dbeta, *dh0;
    float *dq_v, *dk_v;                    // per value head when H_v > H_qk, else dq / dk
    int replayed;                          // 1: states already holds every chunk's entering state
};

// Timed forward: when set, the library's next kernel launch on this host thread carries `start`
// (recorded as the kernel begins) and `stop` (as it ends) in its own dispatch, so no separate
// event packets sit between the kernels; the launch clears the hook.
struct LaunchEvents {
    hipEvent_t start, stop;
};
LaunchEvents &launch_events();
// kernel<<<grid, block, 0, s>>>(args...), with the hook's events if set
template <typename... KArgs, typename... Args>
inline void launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, Args... args) {
    LaunchEvents &le = launch_events();
    const hipEvent_t a = le.start, b = le.stop;
    le = LaunchEvents{nullptr, nullptr};
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, a, b, 0, static_cast<KArgs>(args)...);
}

hipError_t launch_plan(const PlanParams &p, hipStream_t s);
hipError_t launch_intra(int dtype, int D_k, const IntraParams &p, hipStream_t s);
hipError_t launch_intra_kda(int dtype, int D_k, const IntraKdaParams &p, hipStream_t s);
hipError_t launch_chunk(int dtype, int D_k, int BV, int gate, const ChunkParams &p, hipStream_t s);
// mode 1: context-parallel pre-process (chain only over value and identity columns)
hipError_t launch_cp_pre(int dtype, int D_k, int BV, int gate, const ChunkParams &p, hipStream_t s);
// the same maps in the X/Y/Z form (scalar gate, bf16), M written as bf16 pairs in operand order,
// which launch_cp_fix_xyz reads; hipErrorInvalidValue for other head widths
hipError_t launch_cp_pre_xyz(int D_k, const ChunkParams &p, hipStream_t s);
hipError_t launch_cp_fix_xyz(int D_k, const FixParams &p, hipStream_t s);
hipError_t launch_cp_fix(int dtype, int D_k, const FixParams &p, hipStream_t s);
hipError_t launch_warm_stats(const WarmParams &p, hipStream_t s);
hipError_t launch_bwd(int dtype, int D_k, const BwdParams &p, hipStream_t s);
// the per-chunk gradients on the matrix cores (bf16 inputs, scalar gate)
hipError_t launch_bwd_chunk_mma(int D_k, const BwdParams &p, hipStream_t s);
// per-channel gates, bf16 inputs: every per-chunk gradient on the matrix cores (the work of the
// plain kernels (a) and (b))
hipError_t launch_bwd_chunk_kda_mma(int D_k, const BwdParams &p, hipStream_t s);
hipError_t launch_recurrent(int dtype, int D_k, int gate, const RecurrentParams &p, hipStream_t s);

}  // namespace gdn
