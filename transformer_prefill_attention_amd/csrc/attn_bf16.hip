// attn_bf16.hip -- causal grouped-query attention with bf16 MFMA inputs and f32
// accumulation (v_mfma_f32_32x32x16_bf16).
//
// Passages: as attn_f32.hip (memra-engine 0.130.0 src/forward.rs, SDPA block;
// memra-engine 0.101.0 src/spec.rs, `full_attn_verify` per-row fallback for the
// causal rule).  What is rounded to bf16 (round to nearest even): the scaled Q,
// K, V and the softmax weights P, each just before its product; the scores, the
// softmax, the accumulation and the output stay f32 (the denominator f64).
//
// Same work split as the f32 kernel (four wavefronts on one K/V head, LDS tiles
// shared by the query heads of a group, longest-first items, S^T = K Q^T so
// that P lands in the B-operand layout).  Differences:
//  * 64-key tiles: a bf16 MFMA step is 16x cheaper than the f32 one, so the
//    per-tile fixed costs (barrier, row max) are spread over twice the keys.
//  * K is staged row-major as bf16 (row stride d+8: ds_read_b128 conflict-free);
//    V is staged transposed, V^T[d][key] (stride 64+4 keys, 4-key chunks
//    XOR-swizzled), because each lane's A operand of P.V is 8 consecutive keys
//    of one column; each thread loads 4x4 blocks as float4 rows and writes them
//    back as one bf16x4 of 4 keys per column.
//  * O is accumulated by the MFMA directly and rescaled only when the running
//    max of some query of the wavefront moves.
//
// SPLIT = true is the PFA_PREC_BF16X3 mode: Q and K are each split into a bf16
// high part and a bf16 low part (x = hi + lo to ~2^-17) and the scores take the
// three products hi.hi + hi.lo + lo.hi, so score rounding no longer grows with
// |score| the way plain bf16 inputs do (keys with large norms); P and V stay
// plain bf16.  K's low parts double its LDS tile, so one workgroup per CU.
#include "pfa_device.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBN = 64;       // keys per tile
// Wavefronts per workgroup: 8 for head_dim 128 (two per SIMD, all sharing each
// K/V tile, which halves every wavefront's share of the staging and conversion
// work), 4 for head_dim 64.
template <int D>
constexpr int waves_for() { return D == 128 ? 8 : 4; }

__device__ __forceinline__ floatx16 mfma_bf16(bf16x8 a, bf16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(64 * waves_for<D>(), (SPLIT || D == 128) ? 1 : 2) void attn_bf16_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, AttnSched sched, AttnGeom geom) {
    constexpr int kWaves = waves_for<D>();
    constexpr int kThreads = 64 * kWaves;
    // K row in LDS: [high parts | low parts (SPLIT only)], padded so that
    // ds_read_b128 of 32 different rows is conflict-free
    constexpr int KS = (SPLIT ? 2 * D : D) + 8;  // K row stride in LDS (bf16 elements)
    constexpr int VTS = kBN + 4;          // V^T row stride (bf16 elements)
    constexpr int KBYTES = kBN * KS * 2;
    constexpr int VBYTES = D * VTS * 2;
    constexpr int BUF = KBYTES + VBYTES;  // bytes per stage
    constexpr int NQS = D / 16;           // MFMA steps of K Q^T (16 dims each)
    constexpr int NCB = D / 32;           // 32-wide column blocks of O^T
    constexpr int QS = D + 4;             // f32 staging stride of O rows (epilogue)
    // the epilogue stages O through LDS four wavefronts at a time
    static_assert(4 * 32 * QS * 4 <= 2 * BUF, "O staging must fit in the K/V buffers");
    static_assert(kBN * D % (16 * kThreads) == 0, "V staging moves whole 4x4 blocks");
    // K staging: thread tid moves float4 number tid + 256 i of the tile (row f/(D/4),
    // columns 4 (f % (D/4)) ..+3), converted to bf16.
    constexpr int KF4_ROW = D / 4;
    constexpr int K_PER_THREAD = kBN * KF4_ROW / kThreads;
    // V staging: thread tid owns columns 4 cg..4 cg+3 (cg = tid % (D/4)) and V_BLK
    // blocks of 4 consecutive keys (key 4 kg + KG_STRIDE i, kg = tid / (D/4)); it
    // loads them as 4 float4 rows per block and writes them transposed, one bf16x4
    // of 4 keys per column.  The 4-key chunk index inside a V^T row is XOR-swizzled
    // with ((column >> 4) & 3), which makes both these writes and the operand reads
    // below free of LDS bank conflicts.
    constexpr int V_CG = D / 4;                       // column groups
    constexpr int V_KG = kThreads / V_CG;             // key groups (8 for D=128)
    constexpr int V_BLK = kBN / (4 * V_KG);           // 4-key blocks per thread
    constexpr int KG_STRIDE = 4 * V_KG;               // keys between a thread's blocks
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, hl = lane >> 5, ln = lane & 31;

    const WorkItem wi = decode_item(sched, geom, blockIdx.x);
    const int kv = wi.kv, chunk = wi.chunk, s0 = wi.s0, s1 = wi.s1, q0 = wi.q0;
    const int nt_seq = (s1 - s0 + kBN - 1) / kBN;
    const int n_tiles =
        geom.causal ? (min(q0 + sched.rows_per_item, s1) - 1 - s0) / kBN + 1 : nt_seq;

    const int hloc = wave % geom.hpw, rblk = wave / geom.hpw;
    const int h = kv * geom.g + chunk * geom.hpw + hloc;
    const int wq0 = q0 + rblk * 32;
    const bool active = wq0 < s1;
    const int wave_last = geom.causal ? min((wq0 + 31 - s0) / kBN, nt_seq - 1) : nt_seq - 1;
    const int qi = wq0 + ln;

    // ---- Q operand (B of K Q^T): for step s (16 dims), lane (hl, ln) supplies
    // Q[qi][hl*D/2 + 8s + e], e = 0..7 -- the contraction order is free to permute.
    bf16x8 qop[NQS], qlo[SPLIT ? NQS : 1];
    {
        const bool ok = active && qi < s1;
        const float* src = q + ((int64_t)(ok ? qi : s0) * geom.H + h) * D + hl * (D / 2);
#pragma unroll
        for (int s = 0; s < NQS; ++s) {
            floatx4 a = ok ? *reinterpret_cast<const floatx4*>(src + 8 * s) : floatx4{0, 0, 0, 0};
            floatx4 b = ok ? *reinterpret_cast<const floatx4*>(src + 8 * s + 4)
                           : floatx4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = (e < 4 ? a[e] : b[e - 4]) * geom.qscale;
                qop[s][e] = (__bf16)x;
                // high part + low part = x to ~2^-17 relative
                if constexpr (SPLIT) qlo[s][e] = (__bf16)(x - (float)qop[s][e]);
            }
        }
    }

    // ---- staging helpers.  Each tile is read through a buffer resource that starts
    // at the tile's first row of this K/V head and ends after the sequence's last
    // row of it: rows past the end of the sequence read as zeros, with no branches.
    // Per-thread byte offsets inside a tile are fixed.
    floatx4 kreg[K_PER_THREAD];
    floatx4 vreg[4 * V_BLK];
    const int v_cg = tid % V_CG, v_kg = tid / V_CG;
    const uint32_t row_bytes = (uint32_t)geom.Hkv * D * 4;  // bytes between tokens
    uint32_t koff[K_PER_THREAD], voff[4 * V_BLK];
#pragma unroll
    for (int i = 0; i < K_PER_THREAD; ++i) {
        const int f = tid + kThreads * i;
        koff[i] = (f / KF4_ROW) * row_bytes + 16 * (f % KF4_ROW);
    }
#pragma unroll
    for (int b = 0; b < V_BLK; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            voff[4 * b + e] = (4 * v_kg + KG_STRIDE * b + e) * row_bytes + 16 * v_cg;
    auto tile_rsrc = [&](const float* base, int t) {
        const int k0 = s0 + t * kBN;
        const uint32_t bytes = (uint32_t)(s1 - k0 - 1) * row_bytes + D * 4;
        return buffer_rsrc(base + ((int64_t)k0 * geom.Hkv + kv) * D, bytes);
    };
    auto load_k = [&](int t) {
        const auto r = tile_rsrc(k, t);
#pragma unroll
        for (int i = 0; i < K_PER_THREAD; ++i) kreg[i] = buffer_load_f4(r, koff[i]);
    };
    auto store_k = [&](int buf) {
        __bf16* ks = reinterpret_cast<__bf16*>(smem + buf * BUF);
#pragma unroll
        for (int i = 0; i < K_PER_THREAD; ++i) {
            const int f = tid + kThreads * i;
            const int row = f / KF4_ROW, c4 = f % KF4_ROW;
            bf16x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (__bf16)kreg[i][e];
            *reinterpret_cast<bf16x4*>(ks + row * KS + 4 * c4) = x;
            if constexpr (SPLIT) {
                bf16x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (__bf16)(kreg[i][e] - (float)x[e]);
                *reinterpret_cast<bf16x4*>(ks + row * KS + D + 4 * c4) = y;
            }
        }
    };
    auto load_v = [&](int t) {
        const auto r = tile_rsrc(v, t);
#pragma unroll
        for (int i = 0; i < 4 * V_BLK; ++i) vreg[i] = buffer_load_f4(r, voff[i]);
    };
    auto store_v = [&](int buf) {
        __bf16* vt = reinterpret_cast<__bf16*>(smem + buf * BUF + KBYTES);
#pragma unroll
        for (int b = 0; b < V_BLK; ++b) {
            const int chunk = v_kg + V_KG * b;  // 4-key chunk index of this block
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int col = 4 * v_cg + c;
                bf16x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (__bf16)vreg[4 * b + e][c];
                *reinterpret_cast<bf16x4*>(vt + col * VTS + 4 * (chunk ^ ((col >> 4) & 3))) = x;
            }
        }
    };

    floatx16 oacc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.0f;
    float m_run = -INFINITY;
    double l_run = 0.0;

    load_k(0);
    store_k(0);
    load_v(0);
    store_v(0);
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < n_tiles;
        if (more) load_k(t + 1);
        const bool work = active && t <= wave_last;
        floatx16 sacc[2];
        if (work) {
            const __bf16* ks = reinterpret_cast<const __bf16*>(smem + cur * BUF);
            // S^T for keys kb*32 + (0..31): A = K rows, B = Q^T; step s contracts
            // dims hl*D/2 + 8s + (0..7) for lane half hl.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
                const __bf16* kp = ks + (kb * 32 + ln) * KS + hl * (D / 2);
#pragma unroll
                for (int s = 0; s < NQS; ++s) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kp + 8 * s);
                    if constexpr (SPLIT) {
                        // small cross terms first, then the high product
                        const bf16x8 kl = *reinterpret_cast<const bf16x8*>(kp + D + 8 * s);
                        sacc[kb] = mfma_bf16(kl, qop[s], sacc[kb]);
                        sacc[kb] = mfma_bf16(ka, qlo[s], sacc[kb]);
                    }
                    sacc[kb] = mfma_bf16(ka, qop[s], sacc[kb]);
                }
            }
        }
        if (work) {
            const int k0 = s0 + t * kBN;
            // register r of block kb: key k0 + 32kb + 8(r/4) + 4hl + r%4.  A key is
            // hidden when it lies past min(qi, s1-1) (causal) or past s1-1.
            if ((geom.causal && k0 + kBN - 1 > wq0) || k0 + kBN > s1) {
                const int lim = (geom.causal ? min(qi, s1 - 1) : s1 - 1) - (k0 + 4 * hl);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = -INFINITY;
            }
            float mt = sacc[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[1][r]);
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float m_new = fmaxf(m_run, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            float psum = 0.0f;
            bf16x8 pop[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(sacc[kb][r] - m_new);
                    psum += p;
                    pop[2 * kb + (r >> 3)][r & 7] = (__bf16)p;
                }
            l_run = l_run * (double)alpha + (double)psum;
            // rescale O only if the max moved for some query of this wavefront
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
            }
            if (more) {
                store_k(cur ^ 1);
                load_v(t + 1);
            }
            // O^T[d][query] += sum_key V^T[d][key] P^T[key][query]; step s contracts
            // keys 16s + 8(e/4) + 4hl + e%4 (e = 0..7), i.e. P registers 8(s%2)+e of
            // score block s/2.  The A operand is two 4-key runs of V^T row d (the
            // 4-key chunks of a row are XOR-swizzled with (d >> 4) & 3).
            const __bf16* vt = reinterpret_cast<const __bf16*>(smem + cur * BUF + KBYTES);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int col = cb * 32 + ln;
                const int sw = (col >> 4) & 3;  // the chunk swizzle of this V^T row
                const __bf16* vrow = vt + col * VTS;
                const int c_lo = hl ^ sw, c_hi = (2 + hl) ^ sw;  // chunks 4s+hl, 4s+2+hl
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + 16 * s + 4 * c_lo);
                    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 16 * s + 4 * c_hi);
                    const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    oacc[cb] = mfma_bf16(va, pop[s], oacc[cb]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if (more) {
            store_k(cur ^ 1);
            load_v(t + 1);
        }
        if (more) store_v(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: 1/l, transpose through LDS (four wavefronts at a time), coalesced rows
    const double l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = (float)(1.0 / l_tot);
#pragma unroll
    for (int round = 0; round < kWaves / 4; ++round) {
        const bool mine = (wave >> 2) == round;
        float* os = reinterpret_cast<float*>(smem) + (wave & 3) * 32 * QS;
        if (mine && active) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    floatx4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = oacc[cb][4 * r4 + e] * inv;
                    *reinterpret_cast<floatx4*>(os + ln * QS + cb * 32 + 8 * r4 + 4 * hl) = x;
                }
        }
        __syncthreads();
        if (mine && active) {
            constexpr int F4 = D / 4;
#pragma unroll
            for (int i = 0; i < 32 * F4 / 64; ++i) {
                const int f = lane + 64 * i;
                const int r = f / F4, c4 = f % F4;
                const int row = wq0 + r;
                if (row < s1)
                    *reinterpret_cast<floatx4*>(out + ((int64_t)row * geom.H + h) * D + 4 * c4) =
                        *reinterpret_cast<const floatx4*>(os + r * QS + 4 * c4);
            }
        }
        if (round + 1 < kWaves / 4) __syncthreads();
    }
}

}  // namespace

hipError_t launch_attn_bf16(const float* q, const float* k, const float* v, float* out,
                            const AttnSched& sched, const AttnGeom& geom, int D, bool split_qk,
                            int n_items, hipStream_t stream) {
    const dim3 grid((unsigned)n_items * geom.chunks * geom.Hkv), block(64 * (D == 128 ? 8 : 4));
#define PFA_LAUNCH_BF16(DD, SS)                                                                  \
    hipLaunchKernelGGL((attn_bf16_kernel<DD, SS>), grid, block, 0, stream, q, k, v, out, sched, \
                       geom)
    if (D == 128) {
        if (split_qk) PFA_LAUNCH_BF16(128, true);
        else PFA_LAUNCH_BF16(128, false);
    } else {
        if (split_qk) PFA_LAUNCH_BF16(64, true);
        else PFA_LAUNCH_BF16(64, false);
    }
#undef PFA_LAUNCH_BF16
    return hipGetLastError();
}

}  // namespace pfa
