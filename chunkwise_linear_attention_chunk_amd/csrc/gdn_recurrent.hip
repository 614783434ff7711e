// Token-by-token forward of the gated delta rule (the fused recurrent form, chunk size 1): the
// decode path.  Flash Linear Attention page, section 8 (fused_recurrent): one token per step,
// the output fused into the same loop after the update, no intermediate state written, only the
// final one; parallel over (sequence, head, value-column block), serial over tokens.
//
// Per token t of a sequence (state S [D_k, D_v], fp32):
//   S <- alpha_t S            (scalar gate; per-channel gate: Diag(alpha_t) S, rows decayed)
//   u  = S^T k_t,  y = S^T q_t                      (both on the decayed state)
//   w  = beta_t (v_t - u)
//   S <- S + k_t w^T
//   o_t = scale S^T q_t = scale (y + w (k_t . q_t))
// which is S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = scale S_t^T q_t.
#include "gdn_internal.h"
#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int kRecCols = 32;   // value columns per workgroup

// Workgroup: 256 threads on one (sequence, value head, 32 value columns).  Thread t holds the state
// rows RPT * (t / 8) .. + RPT - 1 (RPT = D_k / 32) of columns 4 (t % 8) .. + 3 in registers.
// Wave 0 stages the next token's k, q, decay, beta and k.q in LDS while the workgroup works on
// the current one; one barrier per token (the staged token and the column sums travel through
// double-buffered LDS).
template <typename T, int DK, int GATE>
__global__ __launch_bounds__(256) void recurrent_kernel(RecurrentParams p) {
    constexpr int RPT = DK / 32;           // state rows per thread
    constexpr int KPL = DK / 64;           // staged elements per lane of wave 0
    constexpr int NA = GATE ? DK : 1;      // decay values per token
    __shared__ __attribute__((aligned(16))) float sk[2][DK], sq[2][DK], sa[2][NA];
    __shared__ float sx[2][4];             // beta, k.q
    __shared__ __attribute__((aligned(16))) float red[2][4][2 * kRecCols];   // per-wave partial u, y

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c4 = tid & 7, rg = tid >> 3;
    const int ncb = p.D_v / kRecCols;
    const int cb = blockIdx.x % ncb, nh = blockIdx.x / ncb, h = nh % p.H_v, n = nh / p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    int tok0, len;
    if (p.cu) {   // packed: clamp the span into the token axis
        tok0 = min(max(p.cu[n], 0), p.total_tokens);
        len = min(max(p.cu[n + 1], tok0), p.total_tokens) - tok0;
    } else {
        tok0 = n * p.T;
        len = p.T;
    }
    const T *q = static_cast<const T *>(p.q);
    const T *k = static_cast<const T *>(p.k);
    const T *v = static_cast<const T *>(p.v);
    const T *beta = static_cast<const T *>(p.beta);
    const int col = cb * kRecCols + 4 * c4;
    const int64_t sbase = ((int64_t)n * p.H_v + h) * DK * p.D_v;

    // ---- state: h0 or zero.  The state is read once and written once per call: its loads and
    //      stores carry the non-temporal hint (streamed past the caches' reuse).
    float s[RPT][4];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        if (p.h0) {
            const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p.h0 + sbase + (int64_t)(RPT * rg + r) * p.D_v + col));
            s[r][0] = x[0]; s[r][1] = x[1]; s[r][2] = x[2]; s[r][3] = x[3];
        } else {
            s[r][0] = s[r][1] = s[r][2] = s[r][3] = 0.f;
        }
    }

    // ---- wave 0's staging: raw values of one token in registers, processed into LDS buffer b
    float rk[KPL], rq[KPL], rg_[KPL], rb = 0.f;
    auto load_raw = [&](int t) __attribute__((always_inline)) {
        const int64_t tok = tok0 + t;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            const int i = lane + 64 * e;
            rk[e] = to_f32(k[(tok * p.H_qk + hq) * DK + i]);
            rq[e] = to_f32(q[(tok * p.H_qk + hq) * DK + i]);
            if constexpr (GATE) rg_[e] = to_f32(static_cast<const T *>(p.g)[(tok * p.H_v + h) * DK + i]);
        }
        if constexpr (!GATE) rg_[0] = static_cast<const float *>(p.g)[tok * p.H_v + h];
        rb = to_f32(beta[tok * p.H_v + h]);
    };
    auto wave_sum = [](float x) __attribute__((always_inline)) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
        return x;
    };
    auto stage = [&](int b) __attribute__((always_inline)) {
        if (p.pro.qk_l2norm) {   // prologue: unit q and k rows
            float ssk = 0.f, ssq = 0.f;
#pragma unroll
            for (int e = 0; e < KPL; ++e) { ssk += rk[e] * rk[e]; ssq += rq[e] * rq[e]; }
            const float fk = 1.f / sqrtf(wave_sum(ssk) + kL2Eps), fq = 1.f / sqrtf(wave_sum(ssq) + kL2Eps);
#pragma unroll
            for (int e = 0; e < KPL; ++e) { rk[e] *= fk; rq[e] *= fq; }
        }
        float kq = 0.f;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            const int i = lane + 64 * e;
            sk[b][i] = rk[e];
            sq[b][i] = rq[e];
            kq += rk[e] * rq[e];
            if constexpr (GATE) {
                float gv = rg_[e];
                if (p.pro.A_log) gv = gate_activation(p.pro, gv, p.pro.A_log[h], p.pro.dt_bias ? p.pro.dt_bias[h * DK + i] : 0.f);
                sa[b][i] = fast_exp2(gv * kLog2e);
            }
        }
        kq = wave_sum(kq);
        if (lane == 0) {
            if constexpr (!GATE) {
                float gv = rg_[0];
                if (p.pro.A_log) gv = gate_activation(p.pro, gv, p.pro.A_log[h], p.pro.dt_bias ? p.pro.dt_bias[h] : 0.f);
                sa[b][0] = fast_exp2(gv * kLog2e);
            }
            sx[b][0] = beta_value(p.pro, rb);
            sx[b][1] = kq;
        }
    };

    float4 vnext = make_float4(0.f, 0.f, 0.f, 0.f);
    auto load_v = [&](int t) __attribute__((always_inline)) {
        const T *vp = v + ((int64_t)(tok0 + t) * p.H_v + h) * p.D_v + col;
        if constexpr (sizeof(T) == 4) {
            vnext = *reinterpret_cast<const float4 *>(vp);
        } else {
            const bf16x4 x = *reinterpret_cast<const bf16x4 *>(vp);
            vnext = make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
        }
    };
    if (len > 0) {
        if (wave == 0) {
            load_raw(0);
            stage(0);
            if (len > 1) load_raw(1);
        }
        load_v(0);
    }
    __syncthreads();

    for (int t = 0; t < len; ++t) {
        const int b = t & 1;
        const float4 vc = vnext;
        if (t + 1 < len) load_v(t + 1);
        // this token's operands into registers (the buffer is restaged two tokens later)
        float kr[RPT], qr[RPT], ar[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            kr[r] = sk[b][RPT * rg + r];
            qr[r] = sq[b][RPT * rg + r];
            if constexpr (GATE) ar[r] = sa[b][RPT * rg + r];
            else ar[r] = sa[b][0];
        }
        const float bt = sx[b][0], kq = sx[b][1];
        // decay, then the partial column sums u = S^T k and y = S^T q over this thread's rows
        float pu[4] = {0.f, 0.f, 0.f, 0.f}, py[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                s[r][c] *= ar[r];
                pu[c] += kr[r] * s[r][c];
                py[c] += qr[r] * s[r][c];
            }
        // over the wave's eight row groups (lane bits 3..5), then over the four waves via LDS
#pragma unroll
        for (int off = 8; off < 64; off <<= 1)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pu[c] += __shfl_xor(pu[c], off, 64);
                py[c] += __shfl_xor(py[c], off, 64);
            }
        if (lane < 8) {
            *reinterpret_cast<float4 *>(&red[b][wave][4 * c4]) = make_float4(pu[0], pu[1], pu[2], pu[3]);
            *reinterpret_cast<float4 *>(&red[b][wave][kRecCols + 4 * c4]) = make_float4(py[0], py[1], py[2], py[3]);
        }
        // wave 0 stages the next token into the other buffer (read two barriers ago at the latest)
        if (wave == 0 && t + 1 < len) {
            stage(b ^ 1);
            if (t + 2 < len) load_raw(t + 2);
        }
        __syncthreads();
        float u[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float4 a = *reinterpret_cast<const float4 *>(&red[b][w][4 * c4]);
            const float4 c = *reinterpret_cast<const float4 *>(&red[b][w][kRecCols + 4 * c4]);
            u[0] += a.x; u[1] += a.y; u[2] += a.z; u[3] += a.w;
            y[0] += c.x; y[1] += c.y; y[2] += c.z; y[3] += c.w;
        }
        const float vv[4] = {vc.x, vc.y, vc.z, vc.w};
        float wv[4], ov[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            wv[c] = bt * (vv[c] - u[c]);
            ov[c] = p.scale * (y[c] + wv[c] * kq);
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) s[r][c] += kr[r] * wv[c];
        if (rg == 0) {
            const int64_t oo = ((int64_t)(tok0 + t) * p.H_v + h) * p.D_v + col;
            if (p.o_f32) st4(static_cast<float *>(p.o) + oo, ov[0], ov[1], ov[2], ov[3]);
            else st4(static_cast<T *>(p.o) + oo, ov[0], ov[1], ov[2], ov[3]);
        }
    }

    if (p.final_state) {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            __builtin_nontemporal_store(f32x4{s[r][0], s[r][1], s[r][2], s[r][3]},
                                        reinterpret_cast<f32x4 *>(p.final_state + sbase + (int64_t)(RPT * rg + r) * p.D_v + col));
    }
}

}  // namespace

hipError_t launch_recurrent(int dtype, int D_k, int gate, const RecurrentParams &p, hipStream_t s) {
    const int64_t blocks = (int64_t)p.N * p.H_v * (p.D_v / kRecCols);
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(256);
#define GDN_REC_CASE(T, DK, G) hipLaunchKernelGGL((recurrent_kernel<T, DK, G>), grid, block, 0, s, p)
    if (dtype == 1 && D_k == 128) { if (gate) GDN_REC_CASE(bf16, 128, 1); else GDN_REC_CASE(bf16, 128, 0); }
    else if (dtype == 1 && D_k == 64) { if (gate) GDN_REC_CASE(bf16, 64, 1); else GDN_REC_CASE(bf16, 64, 0); }
    else if (dtype == 0 && D_k == 128) { if (gate) GDN_REC_CASE(float, 128, 1); else GDN_REC_CASE(float, 128, 0); }
    else if (dtype == 0 && D_k == 64) { if (gate) GDN_REC_CASE(float, 64, 1); else GDN_REC_CASE(float, 64, 0); }
    else return hipErrorInvalidValue;
#undef GDN_REC_CASE
    return hipGetLastError();
}

}  // namespace gdn
