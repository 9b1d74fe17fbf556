// qknorm_rope.hip -- per-(token, head) RMSNorm of Q and K with learned scales,
// followed by NeoX (rotate-half) rotary embedding, in one HBM pass.
//
// Passages: memra-engine 0.130.0 src/forward.rs, `Model::forward`, QK-norm and
// RoPE blocks (the reference runs them as four launches with two extra HBM
// round trips; here one wavefront reads each row once and writes it once);
// needle-core v3/model.rs, `rope_at` / `rope` (frequency and angle).
//
// Layout of the work: one wavefront owns one token, or for short inputs one of
// `groups` consecutive runs of its n_head + n_head_kv head rows (Q heads first,
// then K heads), so that short inputs still have enough wavefronts in flight.
// Lane L holds dims L and L + 64 of a row (one dim for head_dim 64), so every
// load and store is a 256-byte coalesced segment, the sum of squares is a
// wavefront reduction, and the rotary cos/sin of the token are computed once per
// lane and reused by every head of the run.
//
// Rotary pair (j, j + n/2): with n == head_dim == 128 both dims of a pair sit
// in the same lane (no data movement); with n == 64 the partner is lane L ^ 32
// (one cross-half shuffle); any other even n uses a general two-shuffle path.
//
// Over a cached prefix (memra-engine 0.101.0 src/spec.rs, `full_attn_verify`:
// new rows are normalised and rotated at their own positions and appended to
// the cache) row t of sequence s sits at position base_s + t - off[s], and its
// K row -- with the V row, when v_out is given -- goes to key row t + koff[s+1] -
// off[s+1] of the cache (the last rows of the sequence's key range).  Plain
// prefill is the case koff = off.
#include <algorithm>

#include "pfa_device.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

// head rows loaded before the first is reduced: eight keep ~4 KB of loads in flight per
// wavefront (four measured 3% slower at 8192 and 16384 tokens; sixteen no faster)
constexpr int kRowsInFlight = 8;

template <int D, int MODE, bool Q8>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(
    const float* q_in, const float* k_in, float* q_out, float* k_out,
    const float* __restrict__ v_in, float* __restrict__ v_out,
    const float* __restrict__ wq, const float* __restrict__ wk, SeqTable seqs, int T, int H,
    int Hkv, int n, double base, float eps, int groups, Q8Rows q8) {
    constexpr int E = D / 64;  // dims per lane
    const int lane = threadIdx.x & 63;

    // Per-lane constants: which rotary pair each of this lane's dims belongs to, weights.
    const RopeLane<D> rl = rope_lane<D>(lane, n, base);
    float wqv[E], wkv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        wqv[e] = wq[lane + 64 * e];
        wkv[e] = wk[lane + 64 * e];
    }

    const int waves = gridDim.x * (blockDim.x >> 6);
    const int rows = H + Hkv, per = (rows + groups - 1) / groups;  // head rows per unit
    for (int u = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); u < T * groups; u += waves) {
        const int t = u / groups, r0 = (u % groups) * per, r1 = min(r0 + per, rows);
        const int s = find_seq(seqs.off, seqs.n_seqs, t);
        const int q_end = seqs.off[s + 1], k_end = seqs.koff[s + 1];
        const int pos = (k_end - seqs.koff[s]) - (q_end - t);  // base_s + t - off[s]
        const int krow = t + k_end - q_end;                    // the K / V row it fills
        float cs[E], sn[E];
        rope_lane_angles<D>(rl, pos, cs, sn);

        // a finished row: f32 out, or (Q8) codes and the row's scale
        auto store_row = [&](const float* o, float* out, int8_t* c8, float* s8) {
            if constexpr (Q8) {
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(o[e]));
                const float sc = quant8_scale(wave_max_dpp(m));
#pragma unroll
                for (int e = 0; e < E; ++e) c8[lane + 64 * e] = (int8_t)quant8(o[e], sc);
                if (lane == 0) *s8 = sc;
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) out[lane + 64 * e] = o[e];
            }
        };
        auto do_rows = [&](const float* in, float* out, int8_t* c8, float* s8, int nrows,
                           const float* wv) {
            for (int h0 = 0; h0 < nrows; h0 += kRowsInFlight) {
                float x[kRowsInFlight][E];
#pragma unroll
                for (int u = 0; u < kRowsInFlight; ++u) {
                    if (h0 + u < nrows) {
#pragma unroll
                        for (int e = 0; e < E; ++e) x[u][e] = in[(h0 + u) * D + lane + 64 * e];
                    }
                }
#pragma unroll
                for (int u = 0; u < kRowsInFlight; ++u) {
                    if (h0 + u >= nrows) break;
                    float o[E];
                    norm_rope_row<D, MODE>(x[u], wv, cs, sn, rl, eps, o);
                    store_row(o, Q8 ? nullptr : out + (h0 + u) * D,
                              Q8 ? c8 + (h0 + u) * D : nullptr, Q8 ? s8 + h0 + u : nullptr);
                }
            }
        };
        // rows [r0, r1) of (Q heads, then K heads)
        if (r0 < H) {
            const int64_t row = (int64_t)t * H + r0;
            if constexpr (Q8)
                do_rows(q_in + row * D, nullptr, q8.q + row * D, q8.qs + row, min(r1, H) - r0,
                        wqv);
            else
                do_rows(q_in + row * D, q_out + row * D, nullptr, nullptr, min(r1, H) - r0, wqv);
        }
        if (r1 > H) {
            const int k0 = max(r0, H) - H;
            const int64_t row = (int64_t)krow * Hkv + k0;
            if constexpr (Q8)
                do_rows(k_in + ((int64_t)t * Hkv + k0) * D, nullptr, q8.k + row * D, q8.ks + row,
                        r1 - H - k0, wkv);
            else
                do_rows(k_in + ((int64_t)t * Hkv + k0) * D, k_out + row * D, nullptr, nullptr,
                        r1 - H - k0, wkv);
            if (Q8 && q8.v) {
                // V rows: quantised as given (no norm, no rotation), kRowsInFlight
                // rows loaded before the first is reduced
                const int nv = r1 - H - k0;
                const float* vin = v_in + ((int64_t)t * Hkv + k0) * D;
                for (int h0 = 0; h0 < nv; h0 += kRowsInFlight) {
                    float x[kRowsInFlight][E];
#pragma unroll
                    for (int u = 0; u < kRowsInFlight; ++u) {
                        if (h0 + u < nv) {
#pragma unroll
                            for (int e = 0; e < E; ++e) x[u][e] = vin[(h0 + u) * D + lane + 64 * e];
                        }
                    }
#pragma unroll
                    for (int u = 0; u < kRowsInFlight; ++u) {
                        if (h0 + u >= nv) break;
                        store_row(x[u], nullptr, q8.v + (row + h0 + u) * D, q8.vs + row + h0 + u);
                    }
                }
            } else if (v_out) {
                const float* vs = v_in + ((int64_t)t * Hkv + k0) * D;
                float* vd = v_out + ((int64_t)krow * Hkv + k0) * D;
                for (int c = lane; c < (r1 - H - k0) * D; c += 64) vd[c] = vs[c];
            }
        }
    }
}

template <int D, int MODE, bool Q8>
hipError_t launch_mode(const float* q_in, const float* k_in, float* q_out, float* k_out,
                       const float* v_in, float* v_out, const float* wq, const float* wk,
                       const SeqTable& seqs, int T, int H, int Hkv, int n, float base,
                       float eps, const Q8Rows& q8, hipStream_t stream) {
    // Work units: tokens, or for short inputs runs of at least 4 head rows of a
    // token, so that ~8192 wavefronts (2048 workgroups of 4) have work.  Up to 4
    // units per wavefront so the per-lane rotary frequencies (f64 pow) are
    // amortised.
    const int rows = H + Hkv;
    int groups = (8192 + T - 1) / T;
    groups = std::max(1, std::min(groups, (rows + 3) / 4));
    const long long units = (long long)T * groups;
    int blocks = (int)std::min<long long>((units + 3) / 4, 2048);
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((qknorm_rope_kernel<D, MODE, Q8>), dim3(blocks), dim3(256), 0, stream,
                       q_in, k_in, q_out, k_out, v_in, v_out, wq, wk, seqs, T, H, Hkv, n,
                       (double)base, eps, groups, q8);
    return hipGetLastError();
}

template <bool Q8>
hipError_t launch_any(const float* q_in, const float* k_in, float* q_out, float* k_out,
                      const float* v_in, float* v_out, const float* wq, const float* wk,
                      const SeqTable& seqs, int T, int H, int Hkv, int D, int rope_dim,
                      float base, float eps, const Q8Rows& q8, hipStream_t stream) {
#define PFA_QKN(DD, MM)                                                                         \
    launch_mode<DD, MM, Q8>(q_in, k_in, q_out, k_out, v_in, v_out, wq, wk, seqs, T, H, Hkv,     \
                            rope_dim, base, eps, q8, stream)
    if (D == 128) {
        if (rope_dim == 128) return PFA_QKN(128, kPairInLane);
        if (rope_dim == 64) return PFA_QKN(128, kPairXor32);
        return PFA_QKN(128, kPairGeneral);
    }
    // D == 64: one dim per lane.
    if (rope_dim == 64) return PFA_QKN(64, kPairXor32);
    return PFA_QKN(64, kPairGeneral);
#undef PFA_QKN
}

}  // namespace

hipError_t launch_qknorm_rope(const float* q_in, const float* k_in, float* q_out, float* k_out,
                              const float* v_in, float* v_out, const float* wq, const float* wk,
                              const SeqTable& seqs, int T, int H, int Hkv, int D, int rope_dim,
                              float base, float eps, hipStream_t stream) {
    return launch_any<false>(q_in, k_in, q_out, k_out, v_in, v_out, wq, wk, seqs, T, H, Hkv, D,
                             rope_dim, base, eps, Q8Rows{}, stream);
}

hipError_t launch_qknorm_rope_q8(const float* q_in, const float* k_in, const float* v_in,
                                 const float* wq, const float* wk, const SeqTable& seqs, int T,
                                 int H, int Hkv, int D, int rope_dim, float base, float eps,
                                 const Q8Rows& out, hipStream_t stream) {
    return launch_any<true>(q_in, k_in, nullptr, nullptr, v_in, nullptr, wq, wk, seqs, T, H, Hkv,
                            D, rope_dim, base, eps, out, stream);
}

}  // namespace pfa
