// attn_f32.hip -- flash-style causal grouped-query attention on f32 MFMA.
//
// Passages: memra-engine 0.130.0 src/forward.rs, `Model::forward`, SDPA block
// (causal GQA, T_q = T_kv = T, scale 1/sqrt(head_dim)); memra-engine 0.101.0
// src/spec.rs, `full_attn_verify` per-row fallback (row r attends keys up to
// and including itself).  The reference prefill calls an untiled ("naive")
// kernel; this one is tiled for gfx950:
//
//  * A workgroup is four wavefronts sharing one K/V head: `hpw` query heads of
//    the group times `rb` blocks of 32 query rows (hpw * rb = 4).  Every K/V
//    tile is read from HBM/L2 once per workgroup and reused from LDS by all of
//    its wavefronts -- the GQA reuse.
//  * Each wavefront computes S^T = K Q^T for 32 keys x its 32 queries with
//    v_mfma_f32_32x32x2f32 (64 steps over head_dim 128).  Computing the
//    transpose leaves every lane holding 16 scores of ONE query, which is exactly
//    the B-operand layout the second product O^T += V^T P^T needs, so the
//    probabilities never leave registers; the contraction index of each step is
//    free to permute, and the V reads follow the score registers' key order.
//  * Online softmax in base 2: Q is pre-multiplied by scale * log2(e).  The
//    running max is lazy: the weights are taken against it at once and only a
//    tile whose scores pass it by more than 8 takes the row max (one cross-half
//    exchange), moves it and rescales O and the sum, so most tiles do no
//    reduction and no rescaling.  The row sum stays a per-lane partial until the
//    end.
//  * Causal tile skipping: a workgroup visits only key tiles up to its last
//    query row; a wavefront skips the tiles past its own diagonal, and only the
//    diagonal/last tile is masked.
//  * K/V tiles are double-buffered in LDS (global loads for tile t+1 are in
//    flight while tile t is multiplied); the output is transposed through LDS
//    so the stores are coalesced rows.
//  * Work items are scheduled longest first across all packed sequences, and
//    the K/V head is the fastest-varying block index, so consecutive
//    workgroups (which the dispatcher spreads over the 8 XCDs) walk the same
//    key tiles of one head together while each XCD's L2 keeps them.
//  * Paired items (AttnSched::paired; the host pairs one causal sequence without a
//    key split when the paired grid is a whole round over the CUs or whole rounds of
//    two per CU, or at most one workgroup per CU in place of a split into long
//    chunks): the workgroup of
//    slot j takes item j and then item n - 1 - j of the longest-first order, so
//    every workgroup visits the same number of key tiles.  A workgroup alone on a CU runs at ~92% of the rate two
//    co-resident ones reach together, so equal work per workgroup is what fills
//    the last part of a run; with one item each, the hardware's placement left
//    CUs with 228 to 292 tiles at T = 4096 (8B-like heads) and a 12% tail.
//
// PREP = true is the fused entry: raw Q rows are RMS-normalised and rotated once
// as the Q tile is staged.  K arrives already normalised and rotated (the entry
// point prepares it once, into the caller's k_rot_out or the workspace, before
// this kernel runs): preparing it per tile here would repeat the work in every
// workgroup that visits the tile.
#include "pfa_device.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

constexpr int kBN = 32;       // keys per tile
constexpr int kWaves = 4;     // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ floatx16 mfma32x32x2(float a, float b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Fused entry: RMS-normalise and rotate one head row held in registers by one
// wavefront.  Lane L holds dims L + 64e (e < D/64) of the row (x[e], in place).
// w: the lane's norm weights; cs/sn: cos/sin of the row's rotary angle for each of
// the lane's dims (ignored for dims >= n); n: rotated dims.  With n == D == 128
// both halves of a pair sit in one lane; with n == 64 the partner of dim L < 64
// is lane L ^ 32; any other n exchanges through two shuffles.
template <int D>
__device__ __forceinline__ void prep_row(float (&x)[D / 64], const float* w, const float* cs,
                                         const float* sn, int n, float eps, int lane) {
    constexpr int E = D / 64;
    const int half = n >> 1;
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += x[e] * x[e];
    ss = wave_sum_dpp(ss);
    const float rs = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    float y[E];
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = x[e] * rs * w[e];
    if (E == 2 && n == 128) {
        x[0] = y[0] * cs[0] - y[E - 1] * sn[0];
        x[E - 1] = y[E - 1] * cs[0] + y[0] * sn[0];
    } else if (n == 64) {
        const float pv = __shfl_xor(y[0], 32, 64);
        x[0] = lane < 32 ? y[0] * cs[0] - pv * sn[0] : y[0] * cs[0] + pv * sn[0];
#pragma unroll
        for (int e = 1; e < E; ++e) x[e] = y[e];
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            const int p = c < half ? c + half : c - half;
            float pv = 0.0f;
#pragma unroll
            for (int sl = 0; sl < E; ++sl) {
                const float cand = __shfl(y[sl], p & 63, 64);
                if ((p >> 6) == sl) pv = cand;
            }
            x[e] = c >= n ? y[e] : (c < half ? y[e] * cs[e] - pv * sn[e] : y[e] * cs[e] + pv * sn[e]);
        }
    }
}

template <int D, bool PREP, bool PAIRED, bool MERGE>
__global__ __launch_bounds__(kThreads, 2) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, AttnSched sched, AttnGeom geom, PrepParams prep, Partials part) {
    constexpr int KS = D + 4;          // K tile row stride in LDS (floats): b128 reads conflict-free
    // V tile: key 8j + 4h + i (h = bit 2 of the key) at row 4j + i of half h, rows of D
    // floats; half 1 starts 16 D + 32 floats in.  A lane of half h reads its 16 operands of
    // a column block from one base at offsets s * D (ds_read2st64_b32 pairs, no address
    // arithmetic), and the two lane halves fall in different banks.
    constexpr int VH = 16 * D + 32;
    constexpr int VT = 32 * D + 32;
    constexpr int NQ = D / 2;          // Q operand registers per lane = MFMA steps of K Q^T
    constexpr int NCB = D / 32;        // 32-wide column blocks of O^T
    constexpr int BUF = kBN * KS + VT;
    constexpr int F4_PER_ROW = D / 4;
    constexpr int LD_PER_THREAD = kBN * F4_PER_ROW / kThreads;  // float4 of K (and of V) per thread
    constexpr int QS = D + 4;          // staging stride of Q / O rows
    // two K/V buffers, or the Q / O staging of the four wavefronts where that is larger
    constexpr int SMEM = 2 * BUF > kWaves * 32 * QS ? 2 * BUF : kWaves * 32 * QS;
    __shared__ __attribute__((aligned(16))) float smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, hl = lane >> 5, ln = lane & 31;

    // ---- work items: one, or with paired items j and n - 1 - j (see above)
    // (a separate instantiation: the pass loop costs the single-item kernel registers)
    int n_pass = 1, bid2 = 0;
    if constexpr (PAIRED) {
        const int hk = geom.chunks * geom.Hkv, j = (int)blockIdx.x / hk;
        const int j2 = sched.seg_start[sched.n_segs] - 1 - j;
        n_pass = j2 > j ? 2 : 1;
        bid2 = j2 * hk + (int)blockIdx.x % hk;
    }
    // (the loop body, the whole item, keeps the indentation of the single-item kernel)
#pragma unroll 1
    for (int pass = 0; pass < n_pass; ++pass) {
    const int bid = pass == 0 ? (int)blockIdx.x : bid2;
    // the previous item's output staging is read before this one's tiles are stored
    if (pass > 0) __syncthreads();
    const WorkItem wi = decode_item(sched, geom, bid);
    const int kv = wi.kv, chunk = wi.chunk, s0 = wi.s0, s1 = wi.s1, q0 = wi.q0;
    // key rows of the sequence: [ks0, ks1); query row i sees keys <= i + dsh (over a
    // cached prefix its position is base + i - s0; plain prefill: ks0 = s0, dsh = 0)
    const int ks0 = wi.k0, ks1 = wi.k1, dsh = ks1 - s1;
    // (the lambdas below must not capture the kernel-argument structs: taking their
    // address copies them into scratch memory and makes every value read from them
    // look divergent; they use these locals instead)
    const int n_kv = geom.Hkv, n_q = geom.H;
    const float* const k_in = k;
    // key tiles of the item (with a sliding window it starts at its first row's first
    // visible key); with a key split this workgroup takes tiles [t_begin, t_end)
    const KeyRange kr = item_key_range(sched, geom, wi, kBN);
    if (wi.kc >= kr.n_chunks) return;  // (uniform: the whole workgroup leaves)
    const int nt_seq = kr.nt_seq, t_begin = kr.t_begin, t_end = kr.t_end;
    const int win = geom.causal ? geom.window : 0;
    const bool split = kr.n_chunks > 1;

    // ---- wavefront role
    const int hloc = wave % geom.hpw, rblk = wave / geom.hpw;
    const int h = kv * geom.g + chunk * geom.hpw + hloc;
    const int wq0 = q0 + rblk * 32;
    const bool active = wq0 < s1;
    // tiles holding a key some row of this wavefront may see
    const int wave_tiles =
        geom.causal ? min((min(wq0 + 31, s1 - 1) + dsh - ks0) / kBN + 1, nt_seq) : nt_seq;
    const int wave_first = win > 0 ? max(0, wq0 + dsh - win + 1 - ks0) / kBN : 0;
    // (with a window: the lowest key the wavefront's last row sees; below it, masks)
    const int wave_lo = wq0 + 31 + dsh - win + 1;
    const int qi = wq0 + ln;

    // Fused entry, per lane: Q norm weights and rotary frequency (turns per position)
    // of its dims L + 64e.
    constexpr int E = D / 64;
    double turns[E];
    float wqv[E];
    if constexpr (PREP) {
        const int half = prep.rope_dim >> 1;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            turns[e] = c < prep.rope_dim
                           ? rope_turns_per_pos(c < half ? c : c - half, prep.rope_dim, prep.base)
                           : 0.0;
            wqv[e] = prep.wq[c];
        }
    }

    // ---- Q tile -> MFMA B operand: lane (hl, ln) holds Q[qi][hl*NQ .. hl*NQ+NQ),
    // pre-multiplied by scale * log2(e).
    float qr[NQ];
    if constexpr (!PREP) {
        const bool ok = active && qi < s1;
        const float* src = q + ((int64_t)(ok ? qi : s0) * geom.H + h) * D + hl * NQ;
#pragma unroll
        for (int c4 = 0; c4 < NQ / 4; ++c4) {
            const floatx4 x = ok ? *reinterpret_cast<const floatx4*>(src + 4 * c4)
                                 : floatx4{0.f, 0.f, 0.f, 0.f};
            qr[4 * c4 + 0] = x[0] * geom.qscale;
            qr[4 * c4 + 1] = x[1] * geom.qscale;
            qr[4 * c4 + 2] = x[2] * geom.qscale;
            qr[4 * c4 + 3] = x[3] * geom.qscale;
        }
    } else {
        // Fused entry: each wavefront normalises and rotates its 32 raw Q rows in
        // registers (8 at a time, lane L holding dims L + 64e), parks them in LDS
        // and picks up the operand layout from there.
        float* qs = smem + wave * 32 * QS;
        if (active) {
#pragma unroll 1
            for (int r0 = 0; r0 < 32; r0 += 8) {
                float x[8][E];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int row = wq0 + r0 + r;
                    const float* src = q + ((int64_t)(row < s1 ? row : s0) * geom.H + h) * D;
#pragma unroll
                    for (int e = 0; e < E; ++e) x[r][e] = row < s1 ? src[lane + 64 * e] : 0.0f;
                }
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    float cs[E], sn[E];
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        rope_cos_sin(wq0 + r0 + r + dsh - ks0, turns[e], cs[e], sn[e]);
                    prep_row<D>(x[r], wqv, cs, sn, prep.rope_dim, prep.eps, lane);
                }
#pragma unroll
                for (int r = 0; r < 8; ++r)
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        qs[(r0 + r) * QS + lane + 64 * e] = wq0 + r0 + r < s1 ? x[r][e] : 0.0f;
            }
        }
        __syncthreads();
        const float* src = qs + ln * QS + hl * NQ;
#pragma unroll
        for (int c4 = 0; c4 < NQ / 4; ++c4) {
            const floatx4 x = *reinterpret_cast<const floatx4*>(src + 4 * c4);
            qr[4 * c4 + 0] = x[0] * geom.qscale;
            qr[4 * c4 + 1] = x[1] * geom.qscale;
            qr[4 * c4 + 2] = x[2] * geom.qscale;
            qr[4 * c4 + 3] = x[3] * geom.qscale;
        }
        __syncthreads();
    }

    // ---- K/V tile staging: global -> registers -> LDS, K and V separately so that
    // only one of them is held in registers at a time.  Each tile is read through a
    // buffer resource that ends after the tile's last row inside the sequence (for
    // this K/V head), so rows past the end of the sequence read as zeros without any
    // branch.  (Its 32-bit size covers at most one tile, never the rest of the
    // sequence, which can pass 4 GB.)
    // Thread tid moves float4 number tid + 256 i of the 32 x D tile: row f / (D/4),
    // column 4 (f % (D/4)); its byte offset inside a tile is fixed.
    const uint32_t row_bytes = (uint32_t)n_kv * D * 4;
    floatx4 kvreg[LD_PER_THREAD];
    uint32_t kv_off[LD_PER_THREAD];
#pragma unroll
    for (int i = 0; i < LD_PER_THREAD; ++i) {
        const int f = tid + kThreads * i;
        kv_off[i] = (f / F4_PER_ROW) * row_bytes + 16 * (f % F4_PER_ROW);
    }
    auto tile_rsrc = [&](const float* base, int t) {
        const int k0 = ks0 + t * kBN;
        const uint32_t bytes = (uint32_t)(min(ks1 - k0, kBN) - 1) * row_bytes + D * 4;
        return buffer_rsrc(base + ((int64_t)k0 * n_kv + kv) * D, bytes);
    };
    auto load_rows = [&](const float* base, int t) {
        const auto r = tile_rsrc(base, t);
#pragma unroll
        for (int i = 0; i < LD_PER_THREAD; ++i) kvreg[i] = buffer_load_f4(r, kv_off[i]);
    };
    auto store_rows = [&](float* dst, int stride) {
#pragma unroll
        for (int i = 0; i < LD_PER_THREAD; ++i) {
            const int f = tid + kThreads * i;
            const int row = f / F4_PER_ROW, c4 = f % F4_PER_ROW;
            *reinterpret_cast<floatx4*>(dst + row * stride + 4 * c4) = kvreg[i];
        }
    };
    auto store_v = [&](float* dst) {
#pragma unroll
        for (int i = 0; i < LD_PER_THREAD; ++i) {
            const int f = tid + kThreads * i;
            const int key = f / F4_PER_ROW, c4 = f % F4_PER_ROW;
            const int at = ((key >> 2) & 1) * VH + (4 * (key >> 3) + (key & 3)) * D + 4 * c4;
            *reinterpret_cast<floatx4*>(dst + at) = kvreg[i];
        }
    };

    // ---- accumulators
    floatx16 oacc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.0f;
    // The softmax denominator is carried in f64: in a row dominated by one key
    // each lane's per-tile sum of the other weights can fall below half an f32
    // ulp of the running sum and would be dropped every time, a systematic
    // underestimate (~1e-5 relative at T = 16k with x8 outlier keys).
    float m_run = -INFINITY;
    double l_run = 0.0;

    load_rows(k_in, t_begin);
    store_rows(smem, KS);
    load_rows(v, t_begin);
    store_v(smem + kBN * KS);
    __syncthreads();

    for (int t = t_begin; t < t_end; ++t) {
        const int cur = (t - t_begin) & 1;
        const bool more = t + 1 < t_end;
        float* kn = smem + (cur ^ 1) * BUF;
        if (more) load_rows(k_in, t + 1);
        if (active && t < wave_tiles && t >= wave_first) {
            const float* ks = smem + cur * BUF;
            const float* vs = ks + kBN * KS;
            // S^T[key][query] = sum_d K[key][d] Q[query][d]; step s contracts
            // d = hl * NQ + s (lanes 0-31 and 32-63 supply the two k-slices).
            // Two partial sums (even / odd 4-step chunks): the MFMA rounds after
            // every product, so halving each chain's length and magnitude halves
            // the rounding error of the scores.
            floatx16 sacc, sacc1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sacc[r] = 0.0f;
                sacc1[r] = 0.0f;
            }
            const float* kp = ks + ln * KS + hl * NQ;
            // Operands are read one 8-step chunk ahead of the MFMAs that use them;
            // the scheduling fence stops the compiler from hoisting every read to
            // the top (which would hold 64 extra registers).
            floatx4 ka = *reinterpret_cast<const floatx4*>(kp);
            floatx4 kb = *reinterpret_cast<const floatx4*>(kp + 4);
#pragma unroll
            for (int c4 = 0; c4 < NQ / 4; c4 += 2) {
                floatx4 na = ka, nb = kb;
                if (c4 + 2 < NQ / 4) {
                    na = *reinterpret_cast<const floatx4*>(kp + 4 * c4 + 8);
                    nb = *reinterpret_cast<const floatx4*>(kp + 4 * c4 + 12);
                }
                sacc = mfma32x32x2(ka[0], qr[4 * c4 + 0], sacc);
                sacc1 = mfma32x32x2(kb[0], qr[4 * c4 + 4], sacc1);
                sacc = mfma32x32x2(ka[1], qr[4 * c4 + 1], sacc);
                sacc1 = mfma32x32x2(kb[1], qr[4 * c4 + 5], sacc1);
                sacc = mfma32x32x2(ka[2], qr[4 * c4 + 2], sacc);
                sacc1 = mfma32x32x2(kb[2], qr[4 * c4 + 6], sacc1);
                sacc = mfma32x32x2(ka[3], qr[4 * c4 + 3], sacc);
                sacc1 = mfma32x32x2(kb[3], qr[4 * c4 + 7], sacc1);
                ka = na;
                kb = nb;
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] += sacc1[r];
            // Register r of lane (hl, ln) holds key k0 + 8(r/4) + 4hl + r%4 for query qi.
            const int k0 = ks0 + t * kBN;
            // tiles reaching past the first row's last visible key, past the
            // sequence's keys, or (window) below the last row's first one, are masked
            if ((geom.causal && k0 + kBN - 1 > wq0 + dsh) || k0 + kBN > ks1 ||
                (win > 0 && k0 < wave_lo)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 8 * (r >> 2) + 4 * hl + (r & 3);
                    if ((geom.causal && key > qi + dsh) || key >= ks1 ||
                        (win > 0 && key < qi + dsh - win + 1))
                        sacc[r] = -INFINITY;
                }
            }
            // Weights against the running max straight away; only when some score
            // passes it by more than kLazyMax is the row max taken, O and l rescaled
            // and the weights recomputed (m moves to the row max).  A row that has
            // seen no key yet keeps m = -inf; exponents against -1e30 then give 0.
            const float lmax = max16(sacc);
            float pw[16];
            {
                const float m_sub = fmaxf(m_run, -1e30f);
#pragma unroll
                for (int r = 0; r < 16; ++r) pw[r] = __builtin_amdgcn_exp2f(sacc[r] - m_sub);
            }
            if (__any(lmax > m_run + kLazyMax)) {
                const float mt = max_halves(lmax);
                const bool bump = mt > m_run + kLazyMax;
                float alpha = bump ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
                if (bump) m_run = mt;
                const float m_new = fmaxf(m_run, -1e30f);
#pragma unroll
                for (int r = 0; r < 16; ++r) pw[r] = __builtin_amdgcn_exp2f(sacc[r] - m_new);
                l_run *= (double)alpha;
                // alpha is 1 in rows without a bump; hidden from the optimiser, which
                // would otherwise make the multiplication unconditional
                asm volatile("" : "+v"(alpha));
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
            }
            float psum = pw[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) psum += pw[r];
            l_run += (double)psum;
            // O^T[d][query] += sum_key V[key][d] P[query][key].  Each tile's products go
            // into a fresh accumulator that is added to O once per element: O is rounded
            // once per tile instead of once per key, which keeps long rows dominated by
            // one key accurate.  Step s contracts key 8(s/4) + 4hl + s%4, i.e. score
            // register s of the lane.
            float vop[16], vnext[16];
            auto read_v = [&](int cb, float* dst) {
                const float* vb = vs + hl * VH + ln + 32 * cb;
#pragma unroll
                for (int s = 0; s < 16; ++s) dst[s] = vb[s * D];
            };
            // (the first block's operands are read before the next tile's K is staged)
            read_v(0, vop);
            if (more) {
                store_rows(kn, KS);
                load_rows(v, t + 1);
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (cb + 1 < NCB) read_v(cb + 1, vnext);
                floatx16 pv;
#pragma unroll
                for (int r = 0; r < 16; ++r) pv[r] = 0.0f;
#pragma unroll
                for (int s = 0; s < 16; ++s) pv = mfma32x32x2(vop[s], pw[s], pv);
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] += pv[r];
#pragma unroll
                for (int s = 0; s < 16; ++s) vop[s] = vnext[s];
                // keep the column-block chains apart (bounded live registers)
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if (more) {
            // this wavefront has no work on tile t but still stages tile t+1
            store_rows(kn, KS);
            load_rows(v, t + 1);
        }
        if (more) store_v(kn + kBN * KS);
        __syncthreads();
    }

    // ---- epilogue: 1/l, transpose through LDS, coalesced row stores (to the output,
    // or for a split item to this unit's partial-result slot)
    const double l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.0 ? (float)(1.0 / l_tot) : 0.0f;
    // (the slot is wavefront-uniform: its buffer resource lives in scalar registers)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const size_t slot = (size_t)bid * kWaves + wave_u;
    if (split && hl == 0) {
        part.ml[slot * 32 + ln] = float2{m_run, (float)l_tot};
    }
    float* os = smem + wave * 32 * QS;
    if (active) {
        // lane (hl, ln), register r of block cb holds O[qi][cb*32 + 8(r/4) + 4hl + r%4]
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                floatx4 x;
                x[0] = oacc[cb][4 * r4 + 0] * inv;
                x[1] = oacc[cb][4 * r4 + 1] * inv;
                x[2] = oacc[cb][4 * r4 + 2] * inv;
                x[3] = oacc[cb][4 * r4 + 3] * inv;
                *reinterpret_cast<floatx4*>(os + ln * QS + cb * 32 + 8 * r4 + 4 * hl) = x;
            }
    }
    __syncthreads();
    if (active) {
#pragma unroll
        for (int i = 0; i < 32 * F4_PER_ROW / 64; ++i) {
            const int f = lane + 64 * i;
            const int r = f / F4_PER_ROW, c4 = f % F4_PER_ROW;
            const int row = wq0 + r;
            const floatx4 x = *reinterpret_cast<const floatx4*>(os + r * QS + 4 * c4);
            if (split) {
                *reinterpret_cast<floatx4*>(part.o + (slot * 32 + r) * D + 4 * c4) = x;
            } else if (row < s1) {
                floatx4 y = x;
                if (geom.gate) y *= gate_factors(geom.gate, geom.gate_per_head, row, n_q, h,
                                                 D, 4 * c4);
                *reinterpret_cast<floatx4*>(out + ((int64_t)row * n_q + h) * D + 4 * c4) = y;
            }
        }
    }
    if constexpr (MERGE) {
        // the item's last unit to arrive merges every key chunk's partial result
        __shared__ int last_flag;
        const size_t item_slot = ((size_t)wi.item * geom.chunks + chunk) * n_kv + kv;
        if (split && arrive_last(part, item_slot, kr.n_chunks, &last_flag)) {
            const size_t kstride = (size_t)geom.chunks * n_kv * kWaves;
            const size_t slot0 =
                (((size_t)wi.item * sched.max_chunks * geom.chunks + chunk) * n_kv + kv) *
                    kWaves + wave_u;
            if (active)
                merge_slot<D>(part, slot0, kstride, kr.n_chunks, out, wq0, s1, n_q, h,
                              geom.gate, geom.gate_per_head, lane);
            if (tid == 0) reset_counter(part, item_slot);
        }
    }
    }  // pass
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* out,
                           const AttnSched& sched, const AttnGeom& geom, int D,
                           const PrepParams* prep, const Partials& part, int n_items,
                           hipStream_t stream) {
    // paired items: workgroup j takes items j and n_items - 1 - j
    const long long slots = sched.paired ? (n_items + 1) / 2 : (long long)n_items * sched.max_chunks;
    const dim3 grid((unsigned)(slots * geom.chunks * geom.Hkv)), block(kThreads);
    const PrepParams p = prep ? *prep : PrepParams{nullptr, nullptr, nullptr, 0, 0.0f, 0.0};
    // paired items are never split (the host pairs only without a key split)
    const bool merge = part.cnt != nullptr;
#define PFA_LAUNCH_F32(DD, PP)                                                                    \
    do {                                                                                          \
        if (sched.paired)                                                                         \
            hipLaunchKernelGGL((attn_f32_kernel<DD, PP, true, false>), grid, block, 0, stream,   \
                               q, k, v, out, sched, geom, p, part);                               \
        else if (merge)                                                                           \
            hipLaunchKernelGGL((attn_f32_kernel<DD, PP, false, true>), grid, block, 0, stream,   \
                               q, k, v, out, sched, geom, p, part);                               \
        else                                                                                      \
            hipLaunchKernelGGL((attn_f32_kernel<DD, PP, false, false>), grid, block, 0, stream,  \
                               q, k, v, out, sched, geom, p, part);                               \
    } while (0)
    if (D == 128) {
        if (prep) PFA_LAUNCH_F32(128, true);
        else PFA_LAUNCH_F32(128, false);
    } else {
        if (prep) PFA_LAUNCH_F32(64, true);
        else PFA_LAUNCH_F32(64, false);
    }
#undef PFA_LAUNCH_F32
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && sched.max_chunks > 1 && !merge)
        e = launch_attn_combine(part, out, sched, geom, D, kWaves, kBN, n_items, stream);
    return e;
}

}  // namespace pfa
