// C ABI of libgdn (declared in include/gdn.h): argument validation, planning, workspace
// carve-up and the launch sequence.  Host code only; the kernels live in gdn_intra.hip and
// gdn_chunk.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
gdn_status fail(gdn_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
    int N = 0;
    int64_t total_chunks = 0;
    int BV = 32;
    int n_slices = 0;
    size_t off_A = 0, off_seq = 0, off_chunks = 0, off_order = 0, bytes = 0;
};

int env_int(const char *name, int dflt) {
    const char *s = std::getenv(name);
    return (s && *s) ? std::atoi(s) : dflt;
}

gdn_status validate_and_plan(const gdn_fwd_args *a, Plan *pl) {
    g_last_error.clear();
    if (!a) return fail(GDN_ERR_INVALID_ARG, "args is NULL");
    if (a->B < 0 || a->T < 0) return fail(GDN_ERR_INVALID_ARG, "B=%d and T=%d must be >= 0", a->B, a->T);
    if (a->H_qk <= 0 || a->H_v <= 0) return fail(GDN_ERR_INVALID_ARG, "head counts must be positive");
    if (a->H_v % a->H_qk) return fail(GDN_ERR_INVALID_ARG, "H_v=%d is not a multiple of H_qk=%d", a->H_v, a->H_qk);
    if (a->D_k <= 0 || a->D_v <= 0) return fail(GDN_ERR_INVALID_ARG, "head dims must be positive");
    if (a->D_k > 256) return fail(GDN_ERR_UNSUPPORTED, "D_k=%d > 256: the delta rule keeps all of D_k on chip", a->D_k);
    if (!(a->D_k == 64 || a->D_k == 128)) return fail(GDN_ERR_UNSUPPORTED, "D_k=%d: supported 64, 128", a->D_k);
    if (!(a->D_v == 64 || a->D_v == 128)) return fail(GDN_ERR_UNSUPPORTED, "D_v=%d: supported 64, 128", a->D_v);
    if (a->chunk_size <= 0 || (a->chunk_size & (a->chunk_size - 1)))
        return fail(GDN_ERR_INVALID_ARG, "chunk_size=%d is not a power of two", a->chunk_size);
    if (a->chunk_size != gdn::kChunk) return fail(GDN_ERR_UNSUPPORTED, "chunk_size=%d: supported 64", a->chunk_size);
    if (a->dtype != GDN_DTYPE_F32 && a->dtype != GDN_DTYPE_BF16) return fail(GDN_ERR_INVALID_ARG, "bad dtype %d", a->dtype);
    if (a->gate_kind != GDN_GATE_SCALAR && a->gate_kind != GDN_GATE_CHANNEL)
        return fail(GDN_ERR_INVALID_ARG, "bad gate_kind %d", a->gate_kind);
    if (a->gate_kind == GDN_GATE_CHANNEL) return fail(GDN_ERR_UNSUPPORTED, "per-channel gates are not built yet");
    if (!std::isfinite(a->scale)) return fail(GDN_ERR_INVALID_ARG, "scale is not finite");
    if (a->o_dtype != a->dtype && a->o_dtype != GDN_DTYPE_F32)
        return fail(GDN_ERR_INVALID_ARG, "o_dtype %d must equal dtype %d or be fp32", a->o_dtype, a->dtype);
    if (a->cp_mode < GDN_CP_AUTO || a->cp_mode > GDN_CP_ON) return fail(GDN_ERR_INVALID_ARG, "bad cp_mode %d", a->cp_mode);
    if ((int64_t)a->B * a->T > INT32_MAX / 2) return fail(GDN_ERR_UNSUPPORTED, "too many tokens (%lld)", (long long)a->B * a->T);

    const bool packed = a->cu_seqlens_dev != nullptr;
    if (packed) {
        if (!a->cu_seqlens_host) return fail(GDN_ERR_INVALID_ARG, "cu_seqlens_dev given without cu_seqlens_host");
        if (a->B != 1) return fail(GDN_ERR_INVALID_ARG, "packed sequences need B == 1 (got B=%d)", a->B);
        if (a->N <= 0) return fail(GDN_ERR_INVALID_ARG, "packed sequences need N >= 1 (got %d)", a->N);
        const int32_t *cu = a->cu_seqlens_host;
        if (cu[0] != 0) return fail(GDN_ERR_INVALID_ARG, "cu_seqlens[0]=%d must be 0", cu[0]);
        for (int i = 0; i < a->N; ++i)
            if (cu[i + 1] < cu[i]) return fail(GDN_ERR_INVALID_ARG, "cu_seqlens decreases at %d", i);
        if (cu[a->N] != a->T) return fail(GDN_ERR_INVALID_ARG, "cu_seqlens[N]=%d != T=%d", cu[a->N], a->T);
    } else {
        if (a->cu_seqlens_host) return fail(GDN_ERR_INVALID_ARG, "cu_seqlens_host given without cu_seqlens_dev");
        if (a->N != a->B) return fail(GDN_ERR_INVALID_ARG, "N=%d must equal B=%d when not packed", a->N, a->B);
    }
    const int64_t tokens = (int64_t)a->B * a->T;
    if (tokens > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o))
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta and o are required");

    pl->N = a->N;
    int64_t nch = 0;
    if (packed) {
        for (int i = 0; i < a->N; ++i) nch += (a->cu_seqlens_host[i + 1] - a->cu_seqlens_host[i] + gdn::kChunk - 1) / gdn::kChunk;
    } else {
        nch = (int64_t)a->B * ((a->T + gdn::kChunk - 1) / gdn::kChunk);
    }
    pl->total_chunks = nch;
    if (nch * a->H_v > INT32_MAX) return fail(GDN_ERR_UNSUPPORTED, "too many chunk-heads");

    // value columns per recurrence workgroup (16 per chain/output wave pair); GDN_BV overrides
    // for experiments.  fp32 with D_k = 128 fits the LDS budget only with one pair.
    const int bv_env = env_int("GDN_BV", 0);
    pl->BV = (a->dtype == GDN_DTYPE_F32 && a->D_k == 128) ? 16 : (bv_env == 16 ? 16 : 32);
    pl->n_slices = a->D_v / pl->BV;

    const size_t esz = a->dtype == GDN_DTYPE_BF16 ? 2 : 4;
    size_t off = 0;
    pl->off_A = off;      off = align_up(off + (size_t)nch * a->H_v * 64 * 64 * esz);
    pl->off_seq = off;    off = align_up(off + (size_t)a->N * sizeof(gdn::SeqInfo));
    pl->off_chunks = off; off = align_up(off + (size_t)nch * sizeof(gdn::ChunkInfo));
    pl->off_order = off;  off = align_up(off + (size_t)a->N * sizeof(int));
    pl->bytes = off;
    return GDN_OK;
}

}  // namespace

extern "C" size_t gdn_fwd_workspace_bytes(const gdn_fwd_args *a) {
    Plan pl;
    if (validate_and_plan(a, &pl) != GDN_OK) return 0;
    return pl.bytes;
}

namespace {

gdn_status run_fwd(const gdn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream,
                   void *const *events, uint32_t *stages_run) {
    Plan pl;
    const gdn_status st = validate_and_plan(a, &pl);
    if (st != GDN_OK) return st;
    if (!workspace && pl.bytes) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", pl.bytes);
    if (workspace_bytes < pl.bytes)
        return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(GDN_ERR_WORKSPACE, "workspace is not %zu-byte aligned", kAlign);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t ran = 0;
    // records the boundary after `stage` (or the start when stage < 0)
    auto mark = [&](int stage) -> hipError_t {
        if (stage >= 0) ran |= 1u << stage;
        return events ? hipEventRecord(static_cast<hipEvent_t>(events[stage + 1]), s) : hipSuccess;
    };
    auto done = [&](gdn_status r) {
        if (stages_run) *stages_run = ran;
        return r;
    };
    hipError_t e = mark(-1);
    if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "event record: %s", hipGetErrorString(e)));
    if (a->N == 0) return done(GDN_OK);
    char *ws = static_cast<char *>(workspace);
    const bool packed = a->cu_seqlens_dev != nullptr;
    gdn::SeqInfo *seq = packed ? reinterpret_cast<gdn::SeqInfo *>(ws + pl.off_seq) : nullptr;
    gdn::ChunkInfo *chunks = packed ? reinterpret_cast<gdn::ChunkInfo *>(ws + pl.off_chunks) : nullptr;
    int *order = packed ? reinterpret_cast<int *>(ws + pl.off_order) : nullptr;

    if (packed) {
        gdn::PlanParams pp{a->cu_seqlens_dev, a->N, a->T, a->B * a->T, (int)pl.total_chunks, seq, chunks, order};
        e = gdn::launch_plan(pp, s);
        if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "plan launch: %s", hipGetErrorString(e)));
        if ((e = mark(GDN_STAGE_PLAN)) != hipSuccess) return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));
    }

    gdn::IntraParams ip{a->k, a->g, a->beta, chunks, a->T, (int)pl.total_chunks, a->H_qk, a->H_v, ws + pl.off_A};
    e = gdn::launch_intra(a->dtype, a->D_k, ip, s);
    if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "intra launch: %s", hipGetErrorString(e)));
    if ((e = mark(GDN_STAGE_INTRA)) != hipSuccess) return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));

    gdn::ChunkParams cp{a->q, a->k, a->v, a->g, a->beta, ws + pl.off_A, a->h0, a->o, a->final_state,
                        seq, order, a->T, a->N, a->H_qk, a->H_v, a->D_v, pl.n_slices, a->scale,
                        a->o_dtype == GDN_DTYPE_F32 ? 1 : 0};
    e = gdn::launch_chunk(a->dtype, a->D_k, pl.BV, cp, s);
    if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "chunk launch: %s", hipGetErrorString(e)));
    if ((e = mark(GDN_STAGE_CHUNK)) != hipSuccess) return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));
    return done(GDN_OK);
}

}  // namespace

extern "C" gdn_status gdn_fwd(const gdn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream) {
    return run_fwd(a, workspace, workspace_bytes, stream, nullptr, nullptr);
}

extern "C" gdn_status gdn_fwd_timed(const gdn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream,
                                    void *const *events, uint32_t *stages_run) {
    if (!events) return fail(GDN_ERR_INVALID_ARG, "events is NULL");
    return run_fwd(a, workspace, workspace_bytes, stream, events, stages_run);
}

extern "C" const char *gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
        case GDN_ERR_HIP: return "GDN_ERR_HIP";
    }
    return "GDN_UNKNOWN_STATUS";
}

extern "C" const char *gdn_last_error(void) { return g_last_error.c_str(); }
