// Internal interface between the C-ABI host code and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;  // tokens per chunk

// Device-side plan tables (built by the plan kernel from cu_seqlens or the batch shape).
struct SeqInfo {            // one per sequence
    int tok0;               // first token (row of the [B*T] token axis)
    int len;                // tokens
    int chunk0;             // global index of its first chunk
    int nchunks;            // ceil(len / 64)
};
struct ChunkInfo {          // one per global chunk
    int tok0;               // first token of the chunk
    int nv;                 // valid tokens (1..64)
};

struct PlanParams {
    const int32_t *cu;      // nullable: batched form uses n * T
    int N, T;
    int total_tokens;       // B * T: sequence spans are clamped to [0, total_tokens)
    int total_chunks;       // chunk count the host planned from its copy of cu_seqlens
    SeqInfo *seq;           // [N]
    ChunkInfo *chunks;      // [total chunks]
    int *order;             // [N] sequences, longest first (ties by index)
};

// Batched (not packed) input has no tables: sequence n covers tokens [n T, n T + T).
__device__ __forceinline__ SeqInfo seq_info(const SeqInfo *seq, int n, int T) {
    if (seq) return seq[n];
    const int nc = (T + kChunk - 1) / kChunk;
    return SeqInfo{n * T, T, n * nc, nc};
}
__device__ __forceinline__ ChunkInfo chunk_info(const ChunkInfo *chunks, int ci, int T) {
    if (chunks) return chunks[ci];
    const int nc = (T + kChunk - 1) / kChunk, n = ci / nc, c = ci - n * nc;
    return ChunkInfo{n * T + c * kChunk, min(kChunk, T - c * kChunk)};
}

struct IntraParams {
    const void *k, *g, *beta;
    const ChunkInfo *chunks;  // nullptr: batched input of T tokens per sequence
    int T;
    int n_chunks, H_qk, H_v;
    void *A;                // [n_chunks][H_v][64][64] in the input dtype
};

struct ChunkParams {
    const void *q, *k, *v, *g, *beta;
    const void *A;          // from the intra kernel
    const float *h0;        // nullable [N][H_v][D_k][D_v]
    void *o;
    float *final_state;     // nullable
    const SeqInfo *seq;     // nullptr: batched input of T tokens per sequence (order = identity)
    const int *order;
    int T;
    int N, H_qk, H_v, D_v, n_slices;
    float scale;
    int o_f32;              // 1: o is fp32 (the unrounded result), 0: o has the input dtype
};

hipError_t launch_plan(const PlanParams &p, hipStream_t s);
hipError_t launch_intra(int dtype, int D_k, const IntraParams &p, hipStream_t s);
hipError_t launch_chunk(int dtype, int D_k, int BV, const ChunkParams &p, hipStream_t s);

}  // namespace gdn
