// C ABI of libgdn (declared in include/gdn.h): argument validation, planning, workspace
// carve-up and the launch sequence.  Host code only; the kernels live in gdn_intra.hip and
// gdn_chunk.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

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
    bool cp = false;          // in-GPU context parallelism
    bool warm = false;        // its warmup form (no S*, M, fix-up)
    bool xyz = false;         // exact form: the X/Y/Z pre-process (else the chain form)
    int pieces = 1;           // batched input without CP: chunk-range pieces (per-chunk kernel of the
                              // next piece on a side stream while the recurrence runs this one)
    int seg_chunks = 0;       // segment length in chunks (one segment per sequence without CP)
    int64_t total_segs = 0;
    size_t off_A = 0, off_seq = 0, off_chunks = 0, off_segs = 0, off_order = 0;
    size_t off_sstar = 0, off_m = 0, off_start = 0, off_warm = 0;
    size_t off_P = 0, off_gates = 0;                              // intra-chunk output matrix, gate blocks
    size_t off_kg = 0, off_kd = 0, off_qg = 0;                    // per-channel gates
    size_t bytes = 0;
};

constexpr int kNoSegments = 1 << 28;  // segment length meaning "the whole sequence"
// Measured on the Qwen3-Next shape: 1 piece 0.212-0.216 ms, 2: 0.239, 4: 0.252, 8: 0.282 ms per
// step (the latency-bound recurrence slows from ~168 to ~217 us while per-chunk work shares its
// CUs, and each range adds a launch and a state hand-off), so pieces are off unless GDN_PIECES asks.
constexpr int kDefaultPieces = 1;

// One side stream per device (default priority), created on first use and kept for the process.
hipError_t side_stream(hipStream_t *out) {
    static std::mutex mu;
    static hipStream_t streams[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!streams[dev] && (e = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking)) != hipSuccess) return e;
    *out = streams[dev];
    return hipSuccess;
}

// Compute units of the current device, queried once per device; the MI355X count when no device
// answers (planning is host-only and also runs where no GPU is present).
int device_cus() {
    static std::mutex mu;
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return gdn::kDefaultCUs;
    std::lock_guard<std::mutex> lock(mu);
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return gdn::kDefaultCUs;
        cus[dev] = n;
    }
    return cus[dev];
}

int64_t count_segments(const gdn_fwd_args *a, int sl) {
    auto segs = [&](int64_t len) {
        const int64_t nc = (len + gdn::kChunk - 1) / gdn::kChunk;
        return std::max<int64_t>(1, (nc + sl - 1) / sl);
    };
    if (a->cu_seqlens_dev) {
        int64_t t = 0;
        for (int i = 0; i < a->N; ++i) t += segs(a->cu_seqlens_host[i + 1] - a->cu_seqlens_host[i]);
        return t;
    }
    return (int64_t)a->B * segs(a->T);
}

int env_int(const char *name, int dflt) {
    const char *s = std::getenv(name);
    return (s && *s) ? std::atoi(s) : dflt;
}

// Checks shared by the chunked and the token-by-token entry points (chunk: the chunk_size the
// entry point requires).
gdn_status validate_args(const gdn_fwd_args *a, int chunk) {
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
    if (a->chunk_size != chunk) return fail(GDN_ERR_UNSUPPORTED, "chunk_size=%d: this entry point takes %d", a->chunk_size, chunk);
    if (a->dtype != GDN_DTYPE_F32 && a->dtype != GDN_DTYPE_BF16) return fail(GDN_ERR_INVALID_ARG, "bad dtype %d", a->dtype);
    if (a->gate_kind != GDN_GATE_SCALAR && a->gate_kind != GDN_GATE_CHANNEL)
        return fail(GDN_ERR_INVALID_ARG, "bad gate_kind %d", a->gate_kind);
    if (!std::isfinite(a->scale)) return fail(GDN_ERR_INVALID_ARG, "scale is not finite");
    if (a->o_dtype != a->dtype && a->o_dtype != GDN_DTYPE_F32)
        return fail(GDN_ERR_INVALID_ARG, "o_dtype %d must equal dtype %d or be fp32", a->o_dtype, a->dtype);
    if (a->cp_mode < GDN_CP_AUTO || a->cp_mode > GDN_CP_WARMUP) return fail(GDN_ERR_INVALID_ARG, "bad cp_mode %d", a->cp_mode);
    if (a->cp_form < GDN_CP_FORM_AUTO || a->cp_form > GDN_CP_FORM_XYZ) return fail(GDN_ERR_INVALID_ARG, "bad cp_form %d", a->cp_form);
    if (a->cp_form == GDN_CP_FORM_XYZ && (a->dtype != GDN_DTYPE_BF16 || a->gate_kind != GDN_GATE_SCALAR))
        return fail(GDN_ERR_UNSUPPORTED, "cp_form XYZ takes bf16 inputs with a scalar gate");
    if (!(a->cp_warmup_tol >= 0.f && a->cp_warmup_tol < 1.f))
        return fail(GDN_ERR_INVALID_ARG, "cp_warmup_tol must be in [0, 1)");
    if ((a->qk_l2norm != 0 && a->qk_l2norm != 1) || (a->beta_sigmoid != 0 && a->beta_sigmoid != 1))
        return fail(GDN_ERR_INVALID_ARG, "qk_l2norm and beta_sigmoid must be 0 or 1");
    if (!a->A_log && (a->dt_bias || a->gate_lower_bound != 0.f))
        return fail(GDN_ERR_INVALID_ARG, "dt_bias and gate_lower_bound need A_log");
    if (!(a->gate_lower_bound <= 0.f) || !std::isfinite(a->gate_lower_bound))
        return fail(GDN_ERR_INVALID_ARG, "gate_lower_bound must be 0 or a finite negative bound");
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
    return GDN_OK;
}

gdn_status validate_and_plan(const gdn_fwd_args *a, Plan *pl, bool allow_pieces = true) {
    const gdn_status st = validate_args(a, gdn::kChunk);
    if (st != GDN_OK) return st;
    const bool packed = a->cu_seqlens_dev != nullptr;
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
    const bool channel = a->gate_kind == GDN_GATE_CHANNEL;
    if (a->dtype == GDN_DTYPE_F32) pl->BV = (a->D_k == 128 || channel) ? 16 : 32;
    else pl->BV = bv_env == 16 && !channel ? 16 : 32;
    pl->n_slices = a->D_v / pl->BV;

    // ---- in-GPU context parallelism: split sequences into segments when too few
    //      (sequence, head, slice) chains exist to fill the chip (FlashQLA page, auto-CP).
    int64_t max_nc = 0;
    if (packed) {
        for (int i = 0; i < a->N; ++i)
            max_nc = std::max<int64_t>(max_nc, (a->cu_seqlens_host[i + 1] - a->cu_seqlens_host[i] + 63) / 64);
    } else {
        max_nc = (a->T + 63) / 64;
    }
    const int64_t chains = (int64_t)a->N * a->H_v * pl->n_slices;
    const int seg_env = env_int("GDN_CP_SEG", 0);
    int sl = a->cp_segment_chunks > 0 ? a->cp_segment_chunks : seg_env;
    if (sl <= 0) {
        // segments so the main pass fills the CUs once (one recurrence workgroup per CU; the
        // pre-process, with no output waves, then also runs in one round): fewer segments leave
        // CUs idle, more add rounds to both passes and serial steps to the fix-up
        const int64_t want = std::max<int64_t>(2, device_cus() / std::max<int64_t>(chains, 1));
        sl = (int)std::max<int64_t>(4, (max_nc + want - 1) / want);
    }
    bool cp = false;
    if (a->cp_mode == GDN_CP_ON || a->cp_mode == GDN_CP_WARMUP) cp = true;
    else if (a->cp_mode == GDN_CP_AUTO) cp = chains < 128 && max_nc >= 2 * (int64_t)sl;
    pl->cp = cp;
    pl->warm = cp && a->cp_mode == GDN_CP_WARMUP;
    pl->seg_chunks = cp ? sl : kNoSegments;
    // pieces: a batched input without CP is cut into P ranges of chunks (segments run one after
    // another, each from the previous one's end state), so that the per-chunk kernel of range j + 1
    // overlaps the recurrence over range j; GDN_PIECES overrides P for experiments
    if (!packed && !cp && allow_pieces) {
        const int want = std::max(1, env_int("GDN_PIECES", kDefaultPieces));
        if (want > 1 && max_nc >= 2 * (int64_t)want) {
            pl->seg_chunks = (int)((max_nc + want - 1) / want);
            pl->pieces = (int)((max_nc + pl->seg_chunks - 1) / pl->seg_chunks);
        }
    }
    pl->total_segs = count_segments(a, pl->seg_chunks);
    // the X/Y/Z pre-process (one workgroup per segment and head, S* and M together) where there
    // are enough (segment, head) pairs to fill the chip; the chain form (a workgroup per 32
    // virtual columns) for fewer, longer segments, where it measured faster
    if (cp && !pl->warm) {
        const bool can = a->dtype == GDN_DTYPE_BF16 && a->gate_kind == GDN_GATE_SCALAR;
        pl->xyz = a->cp_form == GDN_CP_FORM_XYZ ||
                  (a->cp_form == GDN_CP_FORM_AUTO && can && pl->total_segs * a->H_v >= device_cus());
    }
    if (pl->total_segs * a->H_v > INT32_MAX / 64) return fail(GDN_ERR_UNSUPPORTED, "too many segments");

    const size_t esz = a->dtype == GDN_DTYPE_BF16 ? 2 : 4;
    const size_t seg_heads = (size_t)pl->total_segs * a->H_v;
    size_t off = 0;
    pl->off_A = off;      off = align_up(off + (size_t)nch * a->H_v * 64 * 64 * esz);
    pl->off_seq = off;    off = align_up(off + (size_t)a->N * sizeof(gdn::SeqInfo));
    pl->off_chunks = off; off = align_up(off + (size_t)nch * sizeof(gdn::ChunkInfo));
    pl->off_segs = off;   off = align_up(off + (size_t)pl->total_segs * sizeof(gdn::SegInfo));
    pl->off_order = off;  off = align_up(off + (size_t)pl->total_segs * sizeof(int));
    const size_t tiles = (size_t)nch * a->H_v;
    // P is formed by the recurrence kernel itself with a scalar gate; with per-channel gates the
    // intra kernel forms it (its exponent factors live inside the contraction).  The per-channel
    // operands (P, Kg, Kd, Qg, A) are one part each: fp16 for bf16 inputs, fp32 for fp32 inputs.
    pl->off_P = off;       if (channel) off = align_up(off + tiles * 64 * 64 * esz);
    pl->off_gates = off;   off = align_up(off + tiles * gdn::GB_FLOATS * sizeof(float));
    if (channel) {
        pl->off_kg = off;  off = align_up(off + tiles * 64 * a->D_k * esz);
        pl->off_kd = off;  off = align_up(off + tiles * 64 * a->D_k * esz);
        pl->off_qg = off;  off = align_up(off + tiles * 64 * a->D_k * esz);
    }
    if (pl->warm) {
        pl->off_warm = off;  off = align_up(off + seg_heads * sizeof(int));
    } else if (pl->pieces > 1) {
        pl->off_start = off; off = align_up(off + seg_heads * a->D_k * a->D_v * sizeof(float));
    } else if (cp) {
        pl->off_sstar = off; off = align_up(off + seg_heads * a->D_k * a->D_v * sizeof(float));
        pl->off_m = off;     off = align_up(off + seg_heads * a->D_k * a->D_k * sizeof(float));
        pl->off_start = off; off = align_up(off + seg_heads * a->D_k * a->D_v * sizeof(float));
    }
    pl->bytes = off;
    return GDN_OK;
}

}  // namespace

extern "C" size_t gdn_fwd_workspace_bytes(const gdn_fwd_args *a) {
    Plan pl;
    if (validate_and_plan(a, &pl) != GDN_OK) return 0;
    return pl.bytes;
}

extern "C" gdn_status gdn_fwd_plan(const gdn_fwd_args *a, gdn_plan_info *info) {
    if (!info) return fail(GDN_ERR_INVALID_ARG, "info is NULL");
    Plan pl;
    const gdn_status st = validate_and_plan(a, &pl);
    if (st != GDN_OK) return st;
    int64_t max_nc = 0;
    for (int i = 0; i < a->N; ++i) {
        const int64_t len = a->cu_seqlens_dev ? a->cu_seqlens_host[i + 1] - a->cu_seqlens_host[i] : a->T;
        max_nc = std::max<int64_t>(max_nc, (len + gdn::kChunk - 1) / gdn::kChunk);
    }
    info->cp = pl.cp ? 1 : 0;
    info->segment_chunks = pl.cp ? pl.seg_chunks : (int32_t)max_nc;
    info->total_segments = pl.total_segs;
    info->value_cols_per_group = pl.BV;
    info->pieces = pl.pieces;
    info->workspace_bytes = pl.bytes;
    info->cp_form = pl.cp && !pl.warm ? (pl.xyz ? GDN_CP_FORM_XYZ : GDN_CP_FORM_CHAIN) : 0;
    return GDN_OK;
}

namespace {

gdn_status run_fwd(const gdn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream,
                   void *const *events, uint32_t *stages_run, bool allow_pieces = true) {
    Plan pl;
    const gdn_status st = validate_and_plan(a, &pl, allow_pieces);
    if (st != GDN_OK) return st;
    if (!workspace && pl.bytes) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", pl.bytes);
    if (workspace_bytes < pl.bytes)
        return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(GDN_ERR_WORKSPACE, "workspace is not %zu-byte aligned", kAlign);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t ran = 0;
    // Timed: every stage's kernel carries the boundary events in its own dispatch — the call's
    // first kernel the start (events[0]), each stage's kernel its end (events[stage + 1]) — armed
    // just before the stage's launch; a stage that launched nothing records them as plain events.
    bool first = true;
    auto arm = [&](int stage) {
        if (events)
            gdn::launch_events() = {first ? static_cast<hipEvent_t>(events[0]) : nullptr,
                                    static_cast<hipEvent_t>(events[stage + 1])};
    };
    auto mark = [&](int stage) -> hipError_t {
        ran |= 1u << stage;
        if (!events) return hipSuccess;
        gdn::LaunchEvents &le = gdn::launch_events();
        hipError_t r = hipSuccess;
        if (le.start) r = hipEventRecord(le.start, s);
        if (r == hipSuccess && le.stop) r = hipEventRecord(le.stop, s);
        le = gdn::LaunchEvents{nullptr, nullptr};
        first = false;
        return r;
    };
    auto done = [&](gdn_status r) {
        if (stages_run) *stages_run = ran;
        gdn::launch_events() = gdn::LaunchEvents{nullptr, nullptr};
        return r;
    };
    hipError_t e = hipSuccess;
    if (a->N == 0) {
        if (events && events[0] && (e = hipEventRecord(static_cast<hipEvent_t>(events[0]), s)) != hipSuccess)
            return done(fail(GDN_ERR_HIP, "event record: %s", hipGetErrorString(e)));
        return done(GDN_OK);
    }
    char *ws = static_cast<char *>(workspace);
    const bool packed = a->cu_seqlens_dev != nullptr;
    gdn::SeqInfo *seq = packed ? reinterpret_cast<gdn::SeqInfo *>(ws + pl.off_seq) : nullptr;
    gdn::ChunkInfo *chunks = packed ? reinterpret_cast<gdn::ChunkInfo *>(ws + pl.off_chunks) : nullptr;
    gdn::SegInfo *segs = packed ? reinterpret_cast<gdn::SegInfo *>(ws + pl.off_segs) : nullptr;
    int *order = packed ? reinterpret_cast<int *>(ws + pl.off_order) : nullptr;

    if (packed) {
        gdn::PlanParams pp{a->cu_seqlens_dev, a->N, a->T, a->B * a->T, (int)pl.total_chunks, pl.seg_chunks,
                           (int)pl.total_segs, seq, chunks, segs, order};
        arm(GDN_STAGE_PLAN);
        e = gdn::launch_plan(pp, s);
        if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "plan launch: %s", hipGetErrorString(e)));
        if ((e = mark(GDN_STAGE_PLAN)) != hipSuccess) return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));
    }

    const bool channel = a->gate_kind == GDN_GATE_CHANNEL;
    const gdn::Prologue pro{a->qk_l2norm, a->beta_sigmoid, a->A_log, a->dt_bias, a->gate_lower_bound};
    // the per-chunk kernel over every chunk (cnt 0), or over chunks [lo, lo + cnt) of each sequence
    auto intra = [&](int lo, int cnt, hipStream_t st) -> hipError_t {
        if (channel) {
            gdn::IntraKdaParams ip{a->q, a->k, a->g, a->beta, chunks, a->T, (int)pl.total_chunks, a->H_qk, a->H_v,
                                   a->scale, ws + pl.off_A, ws + pl.off_P, ws + pl.off_kg, ws + pl.off_kd,
                                   ws + pl.off_qg, reinterpret_cast<float *>(ws + pl.off_gates), pro, a->N, lo, cnt};
            return gdn::launch_intra_kda(a->dtype, a->D_k, ip, st);
        }
        gdn::IntraParams ip{a->q, a->k, a->g, a->beta, chunks, a->T, (int)pl.total_chunks, a->H_qk, a->H_v,
                            a->scale, ws + pl.off_A, ws + pl.off_P, reinterpret_cast<float *>(ws + pl.off_gates), pro,
                            a->N, lo, cnt};
        return gdn::launch_intra(a->dtype, a->D_k, ip, st);
    };

    gdn::ChunkParams cp{};
    cp.q = a->q; cp.k = a->k; cp.v = a->v; cp.g = a->g; cp.beta = a->beta;
    cp.A = ws + pl.off_A; cp.h0 = a->h0; cp.o = a->o; cp.final_state = a->final_state;
    cp.seq = seq; cp.segs = segs; cp.order = order;
    cp.T = a->T; cp.N = a->N; cp.H_qk = a->H_qk; cp.H_v = a->H_v; cp.D_v = a->D_v;
    cp.seg_chunks = pl.seg_chunks; cp.total_segs = (int)pl.total_segs;
    cp.scale = a->scale; cp.o_f32 = a->o_dtype == GDN_DTYPE_F32 ? 1 : 0;
    cp.P = ws + pl.off_P;
    cp.gates = reinterpret_cast<const float *>(ws + pl.off_gates);
    if (channel) {
        cp.kg = ws + pl.off_kg; cp.kd = ws + pl.off_kd; cp.qg = ws + pl.off_qg;
    }
    cp.n_slices = pl.n_slices;
    cp.n_cus = device_cus();

    if (pl.pieces > 1) {
        // pieces: the per-chunk kernel of range j runs on a side stream, the recurrence over range
        // j on `stream` once that range is done (and after range j - 1, whose end state it starts
        // from).  Timed: the intra stage is range 0 (the part not overlapped), the chunk stage the
        // rest up to the last range's end.
        hipStream_t side;
        if ((e = side_stream(&side)) != hipSuccess) return done(fail(GDN_ERR_HIP, "side stream: %s", hipGetErrorString(e)));
        const int P = pl.pieces, L = pl.seg_chunks, nc = (a->T + gdn::kChunk - 1) / gdn::kChunk;
        std::vector<hipEvent_t> ev(P + 1, nullptr);
        auto release = [&]() {
            for (hipEvent_t x : ev)
                if (x) (void)hipEventDestroy(x);
        };
        for (auto &x : ev)
            if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) {
                release();
                return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));
            }
        auto check = [&](hipError_t r, const char *what) {
            if (r != hipSuccess) fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(r));
            return r == hipSuccess;
        };
        bool ok = check(hipEventRecord(ev[0], s), "event") && check(hipStreamWaitEvent(side, ev[0], 0), "stream wait");
        if (ok && events && first && events[0]) ok = check(hipEventRecord(static_cast<hipEvent_t>(events[0]), s), "event");
        for (int j = 0; ok && j < P; ++j) {
            ok = check(intra(j * L, std::min(L, nc - j * L), side), "intra launch");
            if (ok && j == 0) {
                if (events && events[GDN_STAGE_INTRA + 1])
                    ok = check(hipEventRecord(static_cast<hipEvent_t>(events[GDN_STAGE_INTRA + 1]), side), "event");
                ran |= 1u << GDN_STAGE_INTRA;
            }
            ok = ok && check(hipEventRecord(ev[j + 1], side), "event");
        }
        cp.seg_start = cp.seg_next = reinterpret_cast<float *>(ws + pl.off_start);
        for (int j = 0; ok && j < P; ++j) {
            cp.seg_only = j + 1;
            ok = check(hipStreamWaitEvent(s, ev[j + 1], 0), "stream wait") &&
                 check(gdn::launch_chunk(a->dtype, a->D_k, pl.BV, a->gate_kind, cp, s), "chunk launch");
        }
        release();
        if (!ok) return done(GDN_ERR_HIP);
        ran |= 1u << GDN_STAGE_CHUNK;
        if (events && events[GDN_STAGE_CHUNK + 1] &&
            (e = hipEventRecord(static_cast<hipEvent_t>(events[GDN_STAGE_CHUNK + 1]), s)) != hipSuccess)
            return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));
        return done(GDN_OK);
    }

    arm(GDN_STAGE_INTRA);
    e = intra(0, 0, s);
    if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "intra launch: %s", hipGetErrorString(e)));
    if ((e = mark(GDN_STAGE_INTRA)) != hipSuccess) return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));

    if (pl.warm) {
        // warmup CP: each segment's warmup length from the gate statistics, no pre-process maps
        const float tol = a->cp_warmup_tol > 0.f ? a->cp_warmup_tol : 0x1p-24f;
        gdn::WarmParams wp{segs, seq, cp.gates, a->T, a->H_v, pl.seg_chunks, (int)pl.total_segs, std::log2(tol),
                           reinterpret_cast<int *>(ws + pl.off_warm)};
        arm(GDN_STAGE_CP_PRE);
        e = gdn::launch_warm_stats(wp, s);
        if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "warmup statistics launch: %s", hipGetErrorString(e)));
        if ((e = mark(GDN_STAGE_CP_PRE)) != hipSuccess) return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));
        cp.warm = wp.warm;
    } else if (pl.cp) {
        cp.seg_sstar = reinterpret_cast<float *>(ws + pl.off_sstar);
        cp.seg_m = reinterpret_cast<float *>(ws + pl.off_m);
        cp.seg_start = reinterpret_cast<float *>(ws + pl.off_start);
        const bool xyz = pl.xyz;
        arm(GDN_STAGE_CP_PRE);
        if (xyz) {
            e = gdn::launch_cp_pre_xyz(a->D_k, cp, s);
        } else {
            gdn::ChunkParams pre = cp;
            pre.n_slices = (a->D_v + a->D_k) / pl.BV;
            e = gdn::launch_cp_pre(a->dtype, a->D_k, pl.BV, a->gate_kind, pre, s);
        }
        if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "cp pre-process launch: %s", hipGetErrorString(e)));
        if ((e = mark(GDN_STAGE_CP_PRE)) != hipSuccess) return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));
        gdn::FixParams fp{segs, seq, a->T, a->N, a->H_v, a->D_v, pl.seg_chunks, (int)pl.total_segs, a->h0, cp.seg_sstar, cp.seg_m,
                          reinterpret_cast<float *>(ws + pl.off_start)};
        arm(GDN_STAGE_CP_FIX);
        e = xyz ? gdn::launch_cp_fix_xyz(a->D_k, fp, s) : gdn::launch_cp_fix(a->dtype, a->D_k, fp, s);
        if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "cp fix-up launch: %s", hipGetErrorString(e)));
        if ((e = mark(GDN_STAGE_CP_FIX)) != hipSuccess) return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));
    }
    arm(GDN_STAGE_CHUNK);
    e = gdn::launch_chunk(a->dtype, a->D_k, pl.BV, a->gate_kind, cp, s);
    if (e != hipSuccess) return done(fail(GDN_ERR_HIP, "chunk launch: %s", hipGetErrorString(e)));
    if ((e = mark(GDN_STAGE_CHUNK)) != hipSuccess) return done(fail(GDN_ERR_HIP, "event: %s", hipGetErrorString(e)));
    return done(GDN_OK);
}

}  // namespace

namespace gdn {
LaunchEvents &launch_events() {
    static thread_local LaunchEvents le{nullptr, nullptr};
    return le;
}
}  // namespace gdn

extern "C" gdn_status gdn_fwd(const gdn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream) {
    return run_fwd(a, workspace, workspace_bytes, stream, nullptr, nullptr);
}

// ---- allocation-free entry point: the workspace is a static device array, one copy per GPU.
// Host code never passes the array's name to a kernel or a copy (on the host it names a host-side
// stand-in, not device memory): it uses the device address hipGetSymbolAddress returns, looked up
// once per device with that device current.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

hipError_t scratch_address(void **out) {
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" gdn_status gdn_fwd_noalloc(const gdn_fwd_args *a, void *stream) {
    Plan pl;
    const gdn_status st = validate_and_plan(a, &pl, /*allow_pieces=*/false);
    if (st != GDN_OK) return st;
    if (pl.bytes > GDN_NOALLOC_SCRATCH_BYTES)
        return fail(GDN_ERR_WORKSPACE, "these arguments need %zu bytes of workspace; the allocation-free entry point "
                    "holds %zu", pl.bytes, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    if (a->N == 0) return GDN_OK;
    void *ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
    return run_fwd(a, ws, GDN_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, /*allow_pieces=*/false);
}

extern "C" gdn_status gdn_fwd_timed(const gdn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream,
                                    void *const *events, uint32_t *stages_run) {
    if (!events) return fail(GDN_ERR_INVALID_ARG, "events is NULL");
    return run_fwd(a, workspace, workspace_bytes, stream, events, stages_run);
}

namespace {

// the forward arguments a backward call implies (for validation and the chunk tables)
gdn_fwd_args bwd_as_fwd(const gdn_bwd_args *b) {
    gdn_fwd_args f{};
    f.B = b->B; f.T = b->T; f.H_qk = b->H_qk; f.H_v = b->H_v; f.D_k = b->D_k; f.D_v = b->D_v;
    f.chunk_size = b->chunk_size; f.dtype = b->dtype; f.gate_kind = b->gate_kind; f.scale = b->scale;
    f.q = b->q; f.k = b->k; f.v = b->v; f.g = b->g; f.beta = b->beta; f.h0 = b->h0;
    f.cu_seqlens_dev = b->cu_seqlens_dev; f.cu_seqlens_host = b->cu_seqlens_host; f.N = b->N;
    f.o = const_cast<void *>(b->dout); f.cp_mode = GDN_CP_OFF; f.o_dtype = b->dtype;   // (only checked, never written)
    return f;
}

struct BwdPlan {
    Plan fwd;
    size_t off_states = 0, off_dsn = 0, off_pmat = 0, off_vp = 0, off_dl = 0, off_dqv = 0, off_dkv = 0, bytes = 0;
};

gdn_status validate_and_plan_bwd(const gdn_bwd_args *b, BwdPlan *bp) {
    if (!b) return fail(GDN_ERR_INVALID_ARG, "args is NULL");
    const gdn_fwd_args f = bwd_as_fwd(b);
    gdn_status st = validate_and_plan(&f, &bp->fwd);
    if (st != GDN_OK) return st;
    if ((int64_t)b->B * b->T > 0 && (!b->dq || !b->dk || !b->dv || !b->dg || !b->dbeta))
        return fail(GDN_ERR_INVALID_ARG, "dq, dk, dv, dg and dbeta are required");
    size_t off = align_up(bp->fwd.bytes);
    const size_t st_bytes = (size_t)bp->fwd.total_chunks * b->H_v * b->D_k * b->D_v * sizeof(float);
    bp->off_states = off; off = align_up(off + st_bytes);
    bp->off_dsn = off;    off = align_up(off + st_bytes);
    // scale Pt (scalar gate; per-channel gates with fp32 inputs: scale P), and with per-channel gates
    // and fp32 inputs V' and dL of every chunk, between the two gradient kernels (bf16 inputs take
    // P from the per-chunk kernel and form every gradient of a chunk in one kernel)
    const bool kda_plain = b->gate_kind == GDN_GATE_CHANNEL && b->dtype == GDN_DTYPE_F32;
    bp->off_pmat = off;
    if (b->gate_kind != GDN_GATE_CHANNEL || kda_plain) off = align_up(off + (size_t)bp->fwd.total_chunks * b->H_v * 4096 * sizeof(float));
    if (kda_plain) {
        bp->off_vp = off; off = align_up(off + (size_t)bp->fwd.total_chunks * b->H_v * 64 * b->D_v * sizeof(float));
        bp->off_dl = off; off = align_up(off + (size_t)bp->fwd.total_chunks * b->H_v * 4096 * sizeof(float));
    }
    if (b->H_v != b->H_qk) {
        const size_t g_bytes = (size_t)b->B * b->T * b->H_v * b->D_k * sizeof(float);
        bp->off_dqv = off; off = align_up(off + g_bytes);
        bp->off_dkv = off; off = align_up(off + g_bytes);
    }
    bp->bytes = off;
    return GDN_OK;
}

}  // namespace

extern "C" size_t gdn_bwd_workspace_bytes(const gdn_bwd_args *a) {
    BwdPlan bp;
    if (validate_and_plan_bwd(a, &bp) != GDN_OK) return 0;
    return bp.bytes;
}

extern "C" gdn_status gdn_bwd(const gdn_bwd_args *a, void *workspace, size_t workspace_bytes, void *stream) {
    BwdPlan bp;
    const gdn_status st = validate_and_plan_bwd(a, &bp);
    if (st != GDN_OK) return st;
    if (!workspace && bp.bytes) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", bp.bytes);
    if (workspace_bytes < bp.bytes)
        return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, bp.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(GDN_ERR_WORKSPACE, "workspace is not %zu-byte aligned", kAlign);
    if (a->N == 0) return GDN_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    const Plan &pl = bp.fwd;
    const bool packed = a->cu_seqlens_dev != nullptr;
    gdn::SeqInfo *seq = packed ? reinterpret_cast<gdn::SeqInfo *>(ws + pl.off_seq) : nullptr;
    gdn::ChunkInfo *chunks = packed ? reinterpret_cast<gdn::ChunkInfo *>(ws + pl.off_chunks) : nullptr;
    hipError_t e;
    if (packed) {
        gdn::PlanParams pp{a->cu_seqlens_dev, a->N, a->T, a->B * a->T, (int)pl.total_chunks, pl.seg_chunks,
                           (int)pl.total_segs, seq, chunks, reinterpret_cast<gdn::SegInfo *>(ws + pl.off_segs),
                           reinterpret_cast<int *>(ws + pl.off_order)};
        if ((e = gdn::launch_plan(pp, s)) != hipSuccess) return fail(GDN_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
    }
    // Step 1 of the notes: the chunks' (I + L)^-1, as the forward forms it
    const bool channel = a->gate_kind == GDN_GATE_CHANNEL;
    if (channel) {
        gdn::IntraKdaParams ip{a->q, a->k, a->g, a->beta, chunks, a->T, (int)pl.total_chunks, a->H_qk, a->H_v,
                               a->scale, ws + pl.off_A, ws + pl.off_P, ws + pl.off_kg, ws + pl.off_kd,
                               ws + pl.off_qg, reinterpret_cast<float *>(ws + pl.off_gates), gdn::Prologue{}};
        e = gdn::launch_intra_kda(a->dtype, a->D_k, ip, s);
    } else {
        gdn::IntraParams ip{a->q, a->k, a->g, a->beta, chunks, a->T, (int)pl.total_chunks, a->H_qk, a->H_v,
                            a->scale, ws + pl.off_A, ws + pl.off_P, reinterpret_cast<float *>(ws + pl.off_gates),
                            gdn::Prologue{}};
        e = gdn::launch_intra(a->dtype, a->D_k, ip, s);
    }
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "intra launch: %s", hipGetErrorString(e));
    gdn::BwdParams bw{};
    bw.q = a->q; bw.k = a->k; bw.v = a->v; bw.beta = a->beta; bw.dout = a->dout;
    bw.g = a->g; bw.h0 = a->h0; bw.dht = a->dht; bw.A = ws + pl.off_A;
    if (channel) {
        bw.P = ws + pl.off_P; bw.kg = ws + pl.off_kg; bw.kd = ws + pl.off_kd; bw.qg = ws + pl.off_qg;
    }
    bw.gates = reinterpret_cast<const float *>(ws + pl.off_gates);
    bw.seq = seq; bw.chunks = chunks;
    bw.T = a->T; bw.N = a->N; bw.n_chunks = (int)pl.total_chunks; bw.H_qk = a->H_qk; bw.H_v = a->H_v; bw.D_v = a->D_v;
    bw.T_total = (int64_t)a->B * a->T; bw.scale = a->scale;
    bw.states = reinterpret_cast<float *>(ws + bp.off_states);
    bw.dsnext = reinterpret_cast<float *>(ws + bp.off_dsn);
    bw.pmat = reinterpret_cast<float *>(ws + bp.off_pmat);
    bw.channel = channel ? 1 : 0;
    const bool kda_plain = channel && a->dtype == GDN_DTYPE_F32;
    bw.vp = kda_plain ? reinterpret_cast<float *>(ws + bp.off_vp) : nullptr;
    bw.dlmat = kda_plain ? reinterpret_cast<float *>(ws + bp.off_dl) : nullptr;
    bw.dq = a->dq; bw.dk = a->dk; bw.dv = a->dv; bw.dg = a->dg; bw.dbeta = a->dbeta; bw.dh0 = a->dh0;
    const bool grouped = a->H_v != a->H_qk;
    bw.dq_v = grouped ? reinterpret_cast<float *>(ws + bp.off_dqv) : a->dq;
    bw.dk_v = grouped ? reinterpret_cast<float *>(ws + bp.off_dkv) : a->dk;
    // Step 2 of the notes (the state entering every chunk): the forward's main pass, with its output
    // dropped and every chunk's entering state stored
    gdn::ChunkParams cp{};
    cp.q = a->q; cp.k = a->k; cp.v = a->v; cp.g = a->g; cp.beta = a->beta;
    cp.A = ws + pl.off_A; cp.h0 = a->h0; cp.o = nullptr; cp.final_state = nullptr;
    cp.seq = seq;
    cp.segs = packed ? reinterpret_cast<gdn::SegInfo *>(ws + pl.off_segs) : nullptr;
    cp.order = packed ? reinterpret_cast<int *>(ws + pl.off_order) : nullptr;
    cp.T = a->T; cp.N = a->N; cp.H_qk = a->H_qk; cp.H_v = a->H_v; cp.D_v = a->D_v;
    cp.seg_chunks = pl.seg_chunks; cp.total_segs = (int)pl.total_segs;
    cp.scale = a->scale;
    cp.P = ws + pl.off_P;
    cp.gates = reinterpret_cast<const float *>(ws + pl.off_gates);
    if (channel) {
        cp.kg = ws + pl.off_kg; cp.kd = ws + pl.off_kd; cp.qg = ws + pl.off_qg;
    }
    cp.n_slices = pl.n_slices;
    cp.n_cus = device_cus();
    cp.chunk_states = bw.states;
    cp.pmat = bw.pmat;   // the scalar-gate bf16 replay forms the scan's scale P on the way
    if ((e = gdn::launch_chunk(a->dtype, a->D_k, pl.BV, a->gate_kind, cp, s)) != hipSuccess)
        return fail(GDN_ERR_HIP, "state replay launch: %s", hipGetErrorString(e));
    bw.replayed = 1;
    if ((e = gdn::launch_bwd(a->dtype, a->D_k, bw, s)) != hipSuccess)
        return fail(GDN_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

extern "C" gdn_status gdn_fwd_recurrent(const gdn_fwd_args *a, void *stream) {
    const gdn_status st = validate_args(a, 1);
    if (st != GDN_OK) return st;
    if (a->N == 0) return GDN_OK;
    const int64_t blocks = (int64_t)a->N * a->H_v * (a->D_v / 32);
    if (blocks > INT32_MAX) return fail(GDN_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
    gdn::RecurrentParams rp{a->q, a->k, a->v, a->g, a->beta, a->h0, a->final_state, a->o, a->cu_seqlens_dev,
                            a->T, a->N, a->H_qk, a->H_v, a->D_v, a->B * a->T, a->scale,
                            a->o_dtype == GDN_DTYPE_F32 ? 1 : 0,
                            gdn::Prologue{a->qk_l2norm, a->beta_sigmoid, a->A_log, a->dt_bias, a->gate_lower_bound}};
    const hipError_t e = gdn::launch_recurrent(a->dtype, a->D_k, a->gate_kind, rp, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "recurrent launch: %s", hipGetErrorString(e));
    return GDN_OK;
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
