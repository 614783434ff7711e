"""fp64 warmup context parallelism (TEST INFRASTRUCTURE ONLY).

Source: FlashQLA announcement (Qwen), section "further optimisation through gate decay": with
per-token decays alpha < 1 the influence of a past state fades geometrically (a sliding-window
property), so a CP rank can start from S = 0 some W chunks before its first chunk instead of from
the exact start state, dropping the correction matrix M; the warmup chunks write nothing, and a
separate gate-statistics step picks each rank's W.

Readings (the page leaves these open):
  * the ranks are the segments of L chunks of the exact in-GPU CP; a sequence's first segment
    starts from h0 (or zero) as usual;
  * W of segment j >= 1 and value head h is the fewest whole chunks right before the segment
    whose decay bound multiplies to <= tol, where a chunk's decay bound is
      scalar gate:       gamma_C = exp(sum of the chunk's log-gates),
      per-channel gate:  exp(sum over the chunk's tokens of max over channels of the log-gate);
    when no such W exists the segment starts at the sequence start from h0, which is exact;
  * the last segment's end state is the final state.
Error bound (pinned in tests/test_oracle_warmup.py): for a unit key and 0 <= beta <= 2 the
erase I - beta k k^T has spectral norm 1, so one token's transition has norm <= alpha_t (scalar)
or <= max_d alpha_t,d (per channel); a warmed-up segment's start state is off by at most the
product of the chunk decay bounds over its warmup times ||S_exact(warmup start)||_2, and every
later state by no more.
"""
import numpy as np

from .recurrent import flatten_batch, gdn_recurrent


def chunk_log_decay_bounds(g_seq, C, gate):
    """Per chunk of one sequence and head: log of the chunk's decay bound (see the readings).

    g_seq: [T] (scalar) or [T, D_k] (per channel) log-gates of one head."""
    g_seq = np.asarray(g_seq, dtype=np.float64)
    per_token = g_seq if gate == "scalar" else g_seq.max(axis=-1)
    nc = -(-len(per_token) // C)
    return np.array([per_token[c * C:(c + 1) * C].sum() for c in range(nc)])


def warmup_length(log_bounds, c0, tol):
    """Fewest chunks W <= c0 right before chunk c0 whose bounds multiply to <= tol (c0 if none)."""
    acc, lt = 0.0, (np.log(tol) if tol > 0 else -np.inf)
    for W in range(1, c0 + 1):
        acc += log_bounds[c0 - W]
        if acc <= lt:
            return W
    return c0


def warmup_cp(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, gate="scalar", seg_chunks=4, tol=2.0 ** -24,
              C=64):
    """Forward with warmup CP.  Returns (o shaped like v, final [N, H_v, D_k, D_v], W, ends) where
    W[(n, j, h)] is the warmup length of segment j of sequence n, head h, and ends[(n, j, h)] the
    segment's end state."""
    qf, kf, vf, gf, bf, cu, bt = flatten_batch(q, k, v, g, beta, cu_seqlens)
    H_qk, H_v = qf.shape[1], vf.shape[1]
    G = H_v // H_qk
    N = len(cu) - 1
    o = np.zeros(vf.shape)
    fin = np.zeros((N, H_v, qf.shape[2], vf.shape[2]))
    Ws, ends = {}, {}
    for n in range(N):
        t0, T = int(cu[n]), int(cu[n + 1] - cu[n])
        nc = -(-T // C)
        nseg = max(1, -(-nc // seg_chunks))
        for h in range(H_v):
            hq = h // G
            lb = chunk_log_decay_bounds(gf[t0:t0 + T, h], C, gate)
            for j in range(nseg):
                c0 = j * seg_chunks
                W = 0 if j == 0 else warmup_length(lb, c0, tol)
                start = c0 - W
                a, e = t0 + start * C, t0 + min((c0 + seg_chunks) * C, T)
                s0 = None
                if start == 0 and h0 is not None:
                    s0 = np.asarray(h0, dtype=np.float64)[n:n + 1, h:h + 1]
                sl = lambda x, hh: x[a:e, hh:hh + 1]
                oo, ff = gdn_recurrent(sl(qf, hq), sl(kf, hq), sl(vf, h), gf[a:e, h:h + 1], bf[a:e, h:h + 1], scale,
                                       h0=s0, gate=gate, n_threads=1)
                keep = t0 + c0 * C - a                      # warmup tokens write nothing
                o[a + keep:e, h] = oo[keep:, 0]
                Ws[(n, j, h)] = W
                ends[(n, j, h)] = ff[0, 0]
                if j == nseg - 1:
                    fin[n, h] = ff[0, 0]
            if T == 0 and h0 is not None:
                fin[n, h] = np.asarray(h0, dtype=np.float64)[n, h]
    if bt is not None:
        o = o.reshape(bt + o.shape[1:])
    return o, fin, Ws, ends
